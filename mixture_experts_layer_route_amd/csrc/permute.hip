// Permutation: per-expert row lists, built on the device with no host sync.
//
// TensorFold issue #1247 "Ling-3.0-tiny on a Qualcomm board" (jschmied's comment,
// list "What it does not cover") runs each bf16 expert on just the rows that
// picked it, at the cost of a host synchronisation per layer.  Here the rows are
// grouped on the device: a per-block histogram, one exclusive scan into expert
// offsets (plus the schedule the expert kernels read), and a stable scatter.
// Rows of one expert are ordered by ascending (token, slot); shared experts own
// T rows each after the T*k routed rows.
#include "moe_internal.h"
#include "route_select.h"

namespace moe {

// Exclusive scan over a block of up to 1024 threads; `tmp` holds >= 16 ints.
__device__ int block_exclusive_scan(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nw = (blockDim.x + 63) >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wv] = x;
  __syncthreads();
  if (wv == 0) {
    int t = lane < nw ? tmp[lane] : 0;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(t, o, 64);
      if (lane >= o) t += y;
    }
    if (lane < nw) tmp[lane] = t;
  }
  __syncthreads();
  const int base = wv > 0 ? tmp[wv - 1] : 0;
  total = tmp[nw - 1];
  __syncthreads();
  return base + x - v;
}

// Offsets, active-expert list and M-tile table from per-expert row counts.
// Called by every thread of a 1024-thread block; thread e owns expert e < EE.
// meta[0] = number of experts with rows, meta[1] = number of tiles.
__device__ void build_schedule(int cnt, int EE, int BM, int32_t* offsets, int32_t* active,
                               int32_t* meta, int2* tiles, int* tmp) {
  const int e = threadIdx.x;
  int total;
  const int off = block_exclusive_scan(e < EE ? cnt : 0, tmp, total);
  if (e < EE) offsets[e] = off;
  if (e == 0) offsets[EE] = total;
  const int has = (e < EE && cnt > 0) ? 1 : 0;
  int n_active;
  const int pos = block_exclusive_scan(has, tmp, n_active);
  if (has) active[pos] = e;
  if (BM > 0) {
    const int nt = has ? (cnt + BM - 1) / BM : 0;
    int n_tiles;
    const int t0 = block_exclusive_scan(nt, tmp, n_tiles);
    for (int i = 0; i < nt; ++i) tiles[t0 + i] = make_int2(e, i * BM);
    if (e == 0) meta[1] = n_tiles;
  }
  if (e == 0) meta[0] = n_active;
}

// ---------------------------------------------------------------------------
// Histogram per permutation block of 64 tokens (one wave each, four per block).
// grid = ceil(T/256), block = 256, dynamic LDS = 4*E ints.
__global__ __launch_bounds__(256) void k_perm_count(const int32_t* __restrict__ ids, int64_t T,
                                                    int k, int E, int32_t* __restrict__ blk) {
  extern __shared__ int cnt_lds[];
  const int wv = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += 256) cnt_lds[i] = 0;
  __syncthreads();
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t < T)
    for (int j = 0; j < k; ++j) atomicAdd(&cnt_lds[wv * E + ids[t * k + j]], 1);
  __syncthreads();
  for (int i = threadIdx.x; i < 4 * E; i += 256) {
    const int64_t b = int64_t(blockIdx.x) * 4 + i / E;
    if (b * 64 < T) blk[b * E + (i % E)] = cnt_lds[i];
  }
}

// Totals, offsets, per-block bases (in place over the histogram) and schedule.
// One block of 1024 threads.  The [nblk][E] histogram is walked in chunks of
// CB blocks staged through LDS with coalesced loads; thread e owns expert e.
__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ blk, int nblk, int64_t T,
                                                    int E, int S, int BM,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ active,
                                                    int32_t* __restrict__ meta,
                                                    int2* __restrict__ tiles) {
  constexpr int CHUNK = 16384;                     // ints staged per pass (64 KB)
  __shared__ int tmp[32];
  __shared__ int offs[1025];
  __shared__ int stage[CHUNK];
  const int e = threadIdx.x;
  const int CB = max(1, CHUNK / E);                // blocks per pass
  int cnt = 0;
  for (int b0 = 0; b0 < nblk; b0 += CB) {
    const int nb = min(CB, nblk - b0);
    __syncthreads();
    for (int i = threadIdx.x; i < nb * E; i += 1024) stage[i] = blk[int64_t(b0) * E + i];
    __syncthreads();
    if (e < E)
      for (int b = 0; b < nb; ++b) cnt += stage[b * E + e];
  }
  if (e >= E && e < E + S) cnt = int(T);
  build_schedule(cnt, E + S, BM, offs, active, meta, tiles, tmp);
  __syncthreads();
  if (e <= E + S) offsets[e] = offs[e];
  int run = e < E ? offs[e] : 0;
  for (int b0 = 0; b0 < nblk; b0 += CB) {
    const int nb = min(CB, nblk - b0);
    __syncthreads();
    for (int i = threadIdx.x; i < nb * E; i += 1024) stage[i] = blk[int64_t(b0) * E + i];
    __syncthreads();
    if (e < E) {
      for (int b = 0; b < nb; ++b) {
        const int c = stage[b * E + e];
        stage[b * E + e] = run;
        run += c;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < nb * E; i += 1024) blk[int64_t(b0) * E + i] = stage[i];
  }
}

// Stable scatter, one wave per permutation block of 64 tokens.  The rank of
// (t, j) among its block's rows of expert e is the number of lower lanes whose
// token also chose e: a 64-bit lane mask per (wave, expert) built with LDS
// atomic ORs.  grid = ceil(T/256), block = 256, dynamic LDS = 4*E*8 bytes.
__global__ __launch_bounds__(256) void k_perm_scatter(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int64_t T, int k, int E, int S,
    const int32_t* __restrict__ blk_base, int32_t* __restrict__ row_token,
    int32_t* __restrict__ inv, float* __restrict__ row_w) {
  extern __shared__ unsigned long long bits[];  // [4][E]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += 256) bits[i] = 0ull;
  __syncthreads();
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const bool valid = t < T;
  if (valid)
    for (int j = 0; j < k; ++j) atomicOr(&bits[wv * E + ids[t * k + j]], 1ull << lane);
  __syncthreads();
  if (!valid) return;
  const unsigned long long lower = (1ull << lane) - 1ull;
  const int32_t* base = blk_base + (int64_t(blockIdx.x) * 4 + wv) * E;
  for (int j = 0; j < k; ++j) {
    const int e = ids[t * k + j];
    const int r = base[e] + __popcll(bits[wv * E + e] & lower);
    row_token[r] = int32_t(t);
    inv[t * k + j] = r;
    if (row_w) row_w[r] = w[t * k + j];
  }
  for (int s = 0; s < S; ++s) {
    const int64_t r = T * k + int64_t(s) * T + t;
    row_token[r] = int32_t(t);
    if (row_w) row_w[r] = 1.0f;
  }
}

// Schedule only (active list + tiles) from existing offsets.  One block of 1024.
__global__ __launch_bounds__(1024) void k_schedule_from_offsets(
    const int32_t* __restrict__ offsets_in, int EE, int BM, int32_t* __restrict__ active,
    int32_t* __restrict__ meta, int2* __restrict__ tiles) {
  __shared__ int tmp[32];
  __shared__ int offs[1025];
  const int e = threadIdx.x;
  const int cnt = e < EE ? offsets_in[e + 1] - offsets_in[e] : 0;
  build_schedule(cnt, EE, BM, offs, active, meta, tiles, tmp);
}

// ---------------------------------------------------------------------------
// Small batches (T*k <= 256, T <= 64): selection, histogram, scan and scatter
// in one block of 1024 threads.  Thread e walks the slots in (t, j) order, so
// the rows of expert e come out in ascending (token, slot) order.
template <int QMAX>
__global__ __launch_bounds__(1024) void k_route_permute_small(
    const float* __restrict__ logits, int T, int E, int G, int Gk, int k, int S, int BM,
    int32_t* __restrict__ ids_out, float* __restrict__ w_out, int32_t* __restrict__ offsets,
    int32_t* __restrict__ active, int32_t* __restrict__ meta, int2* __restrict__ tiles,
    int32_t* __restrict__ row_token, int32_t* __restrict__ inv, float* __restrict__ row_w) {
  __shared__ int32_t ids_lds[256];
  __shared__ float w_lds[256];
  __shared__ int tmp[32];
  __shared__ int offs[1025];
  const int wv = threadIdx.x >> 6;
  for (int t = wv; t < T; t += 16)
    select_token_wave<QMAX>(logits + int64_t(t) * E, E, G, Gk, k, ids_lds + t * k, w_lds + t * k);
  __syncthreads();
  const int nslot = T * k;
  for (int i = threadIdx.x; i < nslot; i += 1024) {
    ids_out[i] = ids_lds[i];
    w_out[i] = w_lds[i];
  }
  const int e = threadIdx.x;
  int cnt = 0;
  if (e < E) {
    for (int i = 0; i < nslot; ++i) cnt += ids_lds[i] == e;
  } else if (e < E + S) {
    cnt = T;
  }
  build_schedule(cnt, E + S, BM, offs, active, meta, tiles, tmp);
  __syncthreads();
  if (e <= E + S) offsets[e] = offs[e];
  if (e < E && cnt > 0) {
    int r = offs[e];
    for (int i = 0; i < nslot; ++i) {
      if (ids_lds[i] == e) {
        row_token[r] = i / k;
        inv[i] = r;
        row_w[r] = w_lds[i];
        ++r;
      }
    }
  } else if (e >= E && e < E + S) {
    const int r0 = offs[e];
    for (int t = 0; t < T; ++t) {
      row_token[r0 + t] = t;
      row_w[r0 + t] = 1.0f;
    }
  }
}

// ---------------------------------------------------------------------------
int launch_scan_scatter(const Plan& p, const int32_t* ids, const float* w, int32_t* blk,
                        int32_t* offsets, int32_t* active, int32_t* meta, int2* tiles,
                        int32_t* row_token, int32_t* inv, float* row_w, int BM, hipStream_t st) {
  const unsigned g4 = unsigned((p.T + 255) / 256);
  hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, st, blk, p.nblk, p.T, p.E, p.S, BM,
                     offsets, active, meta, tiles);
  hipLaunchKernelGGL(k_perm_scatter, dim3(g4), dim3(256), size_t(4) * p.E * 8, st, ids, w, p.T,
                     p.k, p.E, p.S, blk, row_token, inv, row_w);
  return check_launch();
}

int launch_permute(const Plan& p, const int32_t* ids, const float* w, int32_t* blk,
                   int32_t* offsets, int32_t* active, int32_t* meta, int2* tiles,
                   int32_t* row_token, int32_t* inv, float* row_w, int BM, hipStream_t st) {
  const unsigned g4 = unsigned((p.T + 255) / 256);
  hipLaunchKernelGGL(k_perm_count, dim3(g4), dim3(256), size_t(4) * p.E * sizeof(int), st, ids,
                     p.T, p.k, p.E, blk);
  return launch_scan_scatter(p, ids, w, blk, offsets, active, meta, tiles, row_token, inv, row_w,
                             BM, st);
}

int launch_schedule(const Plan& p, const int32_t* offsets, int32_t* active, int32_t* meta,
                    int2* tiles, int BM, hipStream_t st) {
  hipLaunchKernelGGL(k_schedule_from_offsets, dim3(1), dim3(1024), 0, st, offsets, p.E + p.S, BM,
                     active, meta, tiles);
  return check_launch();
}

int launch_route_permute_small(const Plan& p, const float* logits, int32_t* ids, float* w,
                               int32_t* offsets, int32_t* active, int32_t* meta, int2* tiles,
                               int32_t* row_token, int32_t* inv, float* row_w, int BM,
                               hipStream_t st) {
#define MOE_SMALL(Q)                                                                          \
  hipLaunchKernelGGL(k_route_permute_small<Q>, dim3(1), dim3(1024), 0, st, logits, int(p.T), p.E, \
                     p.G, p.Gk, p.k, p.S, BM, ids, w, offsets, active, meta, tiles, row_token,    \
                     inv, row_w)
  if (p.E <= 64) MOE_SMALL(1);
  else if (p.E <= 128) MOE_SMALL(2);
  else if (p.E <= 256) MOE_SMALL(4);
  else if (p.E <= 512) MOE_SMALL(8);
  else MOE_SMALL(16);
#undef MOE_SMALL
  return check_launch();
}

}  // namespace moe
