// Helpers shared by the grouped expert GEMMs (bf16, block-FP8, NVFP4, MXFP4).
#pragma once

#include "moe_internal.h"

namespace moe {

template <typename T>
__device__ __forceinline__ const T* expert_mat(const T* routed, const T* shared, int e, int E,
                                               int64_t stride) {
  return e < E ? routed + int64_t(e) * stride : shared + int64_t(e - E) * stride;
}

// Row (M index) held by accumulator register r of a 32x32 MFMA block, for this lane.
__device__ __forceinline__ int acc_row(int r, int lane) { return 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3); }

// Work item of a grouped-GEMM workgroup.  Workgroup b runs on XCD b % 8; the
// n = ntiles * ncol real items (tile-major, column block fastest) are split into 8
// contiguous runs, one per XCD, so that the workgroups sharing an expert's weight
// slabs and a tile's activation rows share one L2.  The grid must hold at least
// 8 * ceil(n / 8) workgroups; the surplus returns false.
__device__ __forceinline__ bool xcd_item(int ntiles, int ncol, int& tile, int& ct) {
  const int n = ntiles * ncol;
  const int per = (n + 7) >> 3;
  const int slot = int(blockIdx.x >> 3);
  const int j = int(blockIdx.x & 7) * per + slot;
  if (slot >= per || j >= n) return false;
  tile = j / ncol;
  ct = j - tile * ncol;
  return true;
}

// Byte offset of column col (0..127) of row `row` in an LDS staging tile of 128-byte
// rows (the gate/up epilogues' E4M3 codes of h).  The 16-byte chunks of a row are
// permuted by (row >> 1) & 7: a wave stores one column of 32 consecutive rows at a
// time, which without the permutation would all fall on the same bank; the copy-out
// reads whole chunks.
__device__ __forceinline__ int stg128(int row, int col) {
  return row * 128 + ((((col >> 4) ^ (row >> 1)) & 7) << 4) + (col & 15);
}

// grid for xcd_item: max_items rounded up to a multiple of the 8 XCDs
static inline unsigned xcd_grid(int64_t max_items) { return unsigned((max_items + 7) / 8 * 8); }

}  // namespace moe
