// Host-side plan and kernel launchers of the MoE library (internal).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "moe.h"
#include "moe_device.h"

namespace moe {


// Everything a call needs to know about a config, computed on the host from
// host-known sizes only (never from routing results).
struct Plan {
  int64_t T;
  int H, I, E, G, Gk, k, S, act, wt;
  int64_t Rk;           // routed rows T*k
  int64_t R;            // all rows T*(k+S)
  int nblk;             // permutation blocks of 64 tokens
  bool skinny;          // skinny expert kernels (else matrix-core tiles)
  bool small_route;     // selection + permutation in one block
  bool fused_down;      // forward: down projection fused with the combine
  int64_t max_active;   // upper bound on experts with rows
  int bm;               // M rows per tile of the matrix-core expert kernels
  int64_t max_tiles;    // upper bound on M tiles
  // workspace carve (byte offsets)
  size_t o_logits, o_ids, o_w, o_blk, o_off, o_meta, o_active, o_tiles, o_rowtok, o_inv, o_roww,
      o_h, o_ypw, o_yp32, o_xq, o_sx, o_hq, o_shq, o_xn, total;
  // optional timing events bound to kernel dispatches: [0],[1] start/stop of the
  // gate/up expert kernel, [2],[3] of the down kernel (all null when not timed)
  hipEvent_t ev[4] = {nullptr, nullptr, nullptr, nullptr};
};

enum TimedKernel { kUntimed = -1, kTimeGateUp = 0, kTimeDown = 1 };

// Launch `kern`; when the plan carries events for `slot`, the start/stop events are
// attached to this dispatch itself (no extra packets between kernels).
template <typename... KA, typename... A>
inline void launch_kernel(const Plan& p, int slot, void (*kern)(KA...), dim3 grid, dim3 block,
                          size_t lds, hipStream_t st, A... args) {
  if (slot >= 0 && p.ev[2 * slot])
    hipExtLaunchKernelGGL(kern, grid, block, uint32_t(lds), st, p.ev[2 * slot],
                          p.ev[2 * slot + 1], 0u, args...);
  else
    hipLaunchKernelGGL(kern, grid, block, lds, st, args...);
}

#define MOE_TRY(expr)              \
  do {                             \
    const int rc_ = (expr);        \
    if (rc_ != MOE_OK) return rc_; \
  } while (0)

int make_plan(const moe_config* cfg, Plan* p);
int check_launch();
int record_hip_error(hipError_t err);

int launch_logits(const Plan& p, const void* x, const void* wr, const float* bias, float* logits,
                  hipStream_t st);
// decoder step: RMSNorm of the rows (batch), or fused in front of the few-token router
int launch_rmsnorm(const Plan& p, const void* x, const void* gamma, float eps, void* xn,
                   hipStream_t st);
int launch_logits_norm(const Plan& p, const void* x, const void* gamma, float eps, const void* wr,
                       const float* bias, float* logits, void* xn, hipStream_t st);
// The quantisation of x that the selection launch can carry in workgroups of its own
// (x's block-FP8 or MXFP8 codes are read only by the expert kernels that follow, so
// it runs beside the selection instead of as a launch of its own).
struct XQuant {
  const bf16_t* x = nullptr;   // null: nothing to quantise
  int64_t rows = 0;
  int K = 0;
  bool mx = false;             // MXFP8 (E8M0 scales per 32) instead of block-FP8 (fp32 per 128)
  uint8_t* codes = nullptr;
  void* scales = nullptr;
  int nsel = 0;                // set by the launcher: workgroups of the selection itself
};
// whether launch_select can carry an XQuant for this plan (the row-selection kernel)
int launch_select(const Plan& p, const float* logits, int32_t* ids, float* w, int32_t* blk,
                  hipStream_t st, XQuant xq = XQuant());
int launch_scan_scatter(const Plan& p, const int32_t* ids, const float* w, int32_t* blk,
                        const int32_t* blk2, int32_t* offsets, int32_t* active, int32_t* meta,
                        int2* tiles, int32_t* row_token, int32_t* inv, float* row_w, int BM,
                        hipStream_t st);
int launch_permute(const Plan& p, const int32_t* ids, const float* w, int32_t* blk,
                   int32_t* offsets, int32_t* active, int32_t* meta, int2* tiles,
                   int32_t* row_token, int32_t* inv, float* row_w, int BM, hipStream_t st);
int launch_schedule(const Plan& p, const int32_t* offsets, int32_t* active, int32_t* meta,
                    int2* tiles, int BM, hipStream_t st);
int launch_route_permute_small(const Plan& p, const float* logits, int32_t* ids, float* w,
                               int32_t* offsets, int32_t* active, int32_t* meta, int2* tiles,
                               int32_t* row_token, int32_t* inv, float* row_w, int BM,
                               hipStream_t st);
bool decode_ffn_ok(const Plan& p);
// the sixteen-lanes-per-token selection covers this shape
bool select_rows_ok(const Plan& p);
// M rows per tile the matrix-core expert kernels use for this plan
int gemm_tile_rows(const Plan& p);
// the NVFP4 matrix-core kernels cover this shape
bool nv4_mfma_ok(const Plan& p);
// Decode path: gate/up (with in-kernel routing) then down + combine.  xq / sxq receive
// x's MXFP8 codes and E8M0 scales when the experts are MXFP4 (unused otherwise).
int launch_decode_ffn(const Plan& p, const void* x, const float* logits, const moe_weights* w,
                      int32_t* ids, float* wts, int32_t* offsets, int32_t* row_token,
                      int32_t* inv, float* h, const void* res, void* y, uint8_t* xq,
                      uint8_t* sxq, hipStream_t st);
// NVFP4 experts beyond the decode kernels: expert-major gate/up (h fp32) and down
// (unweighted fp32 rows), reading the permutation from global memory
int launch_nv_gateup_batch(const Plan& p, const void* x, const int32_t* row_token,
                           const int32_t* offsets, const int32_t* active, const int32_t* meta,
                           const moe_weights* w, float* h, hipStream_t st);
int launch_nv_down_batch(const Plan& p, const float* h, const int32_t* offsets,
                         const int32_t* active, const int32_t* meta, const moe_weights* w,
                         float* y_perm, hipStream_t st);
int launch_gateup_skinny(const Plan& p, const void* x, const int32_t* row_token,
                         const int32_t* offsets, const int32_t* active, const int32_t* meta,
                         const moe_weights* w, float* h, hipStream_t st);
int launch_down_skinny(const Plan& p, const float* h, const int32_t* offsets,
                       const int32_t* active, const int32_t* meta, const moe_weights* w,
                       float* y_perm, hipStream_t st);
int launch_down_combine_skinny(const Plan& p, const float* h, const int32_t* ids, const float* wts,
                               const int32_t* inv, const moe_weights* w, const void* res, void* y,
                               hipStream_t st);
int launch_gateup_mfma(const Plan& p, const void* x, const int32_t* row_token,
                       const int32_t* offsets, const int2* tiles, const int32_t* meta,
                       const moe_weights* w, void* h, const uint8_t* xq, const float* sx,
                       uint8_t* hq, float* shq, hipStream_t st);
int launch_down_mfma(const Plan& p, const void* h, const int32_t* offsets, const int2* tiles,
                     const int32_t* meta, const moe_weights* w, const float* row_w, float* out32,
                     bf16_t* out16, const float* sh_scale, hipStream_t st);
int launch_quant(const Plan& p, const void* in, bool in_bf16, int64_t rows, int K, uint8_t* codes,
                 float* scales, hipStream_t st);
// `res`: residual added to y (decoder step), or null
int launch_combine(const Plan& p, const float* y_perm, const int32_t* offsets, const int32_t* inv,
                   const float* w, const void* res, void* y, hipStream_t st);
int launch_combine_preweighted(const Plan& p, const bf16_t* y_perm, const int32_t* offsets,
                               const int32_t* inv, const void* res, void* y, hipStream_t st);

// MXFP4 experts on the block-scaled matrix cores (ffn_mx.hip)
bool mx4_ok(const Plan& p);
int launch_quant_mx(const void* in, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                    hipStream_t st);
int launch_gateup_mx4(const Plan& p, const uint8_t* xq, const uint8_t* sx, const int32_t* row_token,
                      const int32_t* offsets, const int2* tiles, const int32_t* meta,
                      const moe_weights* w, uint8_t* hq, uint8_t* shq, hipStream_t st);
int launch_down_mx4(const Plan& p, const uint8_t* hq, const uint8_t* shq, const int32_t* offsets,
                    const int2* tiles, const int32_t* meta, const moe_weights* w,
                    const float* row_w, float* out32, bf16_t* out16, hipStream_t st);

// Expert paging (pager.hip): device state layout, planner and copy kernels.
struct PagerLayout {
  size_t o_counters, o_key_slot, o_slot_key, o_stamp, total;
};
PagerLayout pager_layout(int E, int N);
struct PagerCopyArgs {
  const void* src[3];   // device views of the store's gate, up, down arrays [E, ...]
  void* dst[3];         // arena arrays [N, ...]
  int64_t chunks[3];    // 16-byte chunks per expert matrix
};
int launch_pager_reset(int E, int N, void* state, hipStream_t st);
int launch_pager_plan(const int32_t* ids, int nslot, int E, int N, int64_t expert_bytes,
                      void* state, int32_t* ids_slot, int32_t* copies, hipStream_t st);
int launch_pager_copy(const int32_t* copies, const PagerCopyArgs& a, int max_copies,
                      hipStream_t st);

}  // namespace moe
