// Permutation: per-expert row lists, built on the device with no host sync.
//
// TensorFold issue #1247 "Ling-3.0-tiny on a Qualcomm board" (jschmied's comment,
// list "What it does not cover") computes each bf16 expert over the rows routed
// to it, paying a host synchronisation per layer for the grouping.  Here the rows are
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
  int id[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) id[j] = (t < T && j < k) ? ids[t * k + j] : 0;
#pragma unroll
  for (int j = 0; j < 16; ++j)
    if (t < T && j < k) atomicAdd(&cnt_lds[wv * E + id[j]], 1);
  __syncthreads();
  for (int i = threadIdx.x; i < 4 * E; i += 256) {
    const int64_t b = int64_t(blockIdx.x) * 4 + i / E;
    if (b * 64 < T) blk[b * E + (i % E)] = cnt_lds[i];
  }
}

// Totals, offsets, per-block bases (in place over the histogram) and schedule.
// The histogram is blk [nblk][E], plus blk2 [nblk][E] when the counts of each
// block come in two halves (the bases are written over blk).  One block of 1024 threads.  The [nblk][E] histogram is staged through LDS in
// chunks with coalesced loads; each expert gets P = 1024 / E' threads (E' = E
// rounded up to a power of two, P <= 64) that own contiguous runs of blocks, so
// the per-expert sums and running bases are short per thread and combine by
// segmented shuffles over the P lanes of the expert.
__global__ __launch_bounds__(1024) void k_perm_scan(int32_t* __restrict__ blk,
                                                    const int32_t* __restrict__ blk2, int nblk, int64_t T,
                                                    int E, int S, int BM,
                                                    int32_t* __restrict__ offsets,
                                                    int32_t* __restrict__ active,
                                                    int32_t* __restrict__ meta,
                                                    int2* __restrict__ tiles) {
  constexpr int CHUNK = 16384;                     // ints staged per pass (64 KB)
  __shared__ int tmp[32];
  __shared__ int offs[1025];
  __shared__ int tot[1024];
  __shared__ int stage[CHUNK];
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int P = min(64, max(1, 1024 / Ep));       // threads per expert
  const int tid = threadIdx.x;
  const int ge = tid / P, gj = tid % P;            // expert and part of this thread
  const bool mine = ge < E;
  const int CB = max(1, CHUNK / E);                // blocks per pass
  auto part_range = [&](int nb, int& lo, int& hi) {
    const int per = (nb + P - 1) / P;
    lo = min(nb, gj * per);
    hi = min(nb, lo + per);
  };
  auto seg_sum = [&](int v) {                      // sum over the P lanes of the expert
    for (int o = 1; o < P; o <<= 1) v += __shfl_xor(v, o, 64);
    return v;
  };
  // global -> LDS, every load of a thread issued before the first store
  auto load_chunk = [&](int b0, int nb) {
    constexpr int PER = CHUNK / 1024;
    const int n = nb * E;
    int v[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * 1024;
      v[u] = i < n ? blk[int64_t(b0) * E + i] : 0;
    }
    if (blk2) {
      int v2[PER];
#pragma unroll
      for (int u = 0; u < PER; ++u) {
        const int i = tid + u * 1024;
        v2[u] = i < n ? blk2[int64_t(b0) * E + i] : 0;
      }
#pragma unroll
      for (int u = 0; u < PER; ++u) v[u] += v2[u];
    }
#pragma unroll
    for (int u = 0; u < PER; ++u) {
      const int i = tid + u * 1024;
      if (i < n) stage[i] = v[u];
    }
  };
  const bool one_chunk = nblk <= CB;               // then the staged copy is kept for pass 2
  int part = 0;
  for (int b0 = 0; b0 < nblk; b0 += CB) {
    const int nb = min(CB, nblk - b0);
    __syncthreads();
    load_chunk(b0, nb);
    __syncthreads();
    if (mine) {
      int lo, hi;
      part_range(nb, lo, hi);
      for (int b = lo; b < hi; ++b) part += stage[b * E + ge];
    }
  }
  const int sum = seg_sum(part);
  if (mine && gj == 0) tot[ge] = sum;
  __syncthreads();
  const int e = tid;
  int cnt = e < E ? tot[e] : 0;
  if (e >= E && e < E + S) cnt = int(T);
  build_schedule(cnt, E + S, BM, offs, active, meta, tiles, tmp);
  __syncthreads();
  // E + S may be 1024: the total offsets[E + S] then lies beyond the last thread
  for (int i = threadIdx.x; i <= E + S; i += blockDim.x) offsets[i] = offs[i];
  int run = mine ? offs[ge] : 0;
  for (int b0 = 0; b0 < nblk; b0 += CB) {
    const int nb = min(CB, nblk - b0);
    __syncthreads();
    if (!one_chunk) load_chunk(b0, nb);
    __syncthreads();
    int lo = 0, hi = 0, s = 0;
    if (mine) {
      part_range(nb, lo, hi);
      for (int b = lo; b < hi; ++b) s += stage[b * E + ge];
    }
    // exclusive prefix of the parts over the expert's lanes
    int incl = s;
    for (int o = 1; o < P; o <<= 1) {
      const int y = __shfl_up(incl, o, P);
      if (gj >= o) incl += y;
    }
    const int chunk_total = seg_sum(s);
    if (mine) {
      int r = run + incl - s;
      for (int b = lo; b < hi; ++b) {
        const int c = stage[b * E + ge];
        stage[b * E + ge] = r;
        r += c;
      }
    }
    run += chunk_total;
    __syncthreads();
    for (int i = tid; i < nb * E; i += 1024) blk[int64_t(b0) * E + i] = stage[i];
  }
}

// Same result as k_perm_scan when every thread's run of blocks fits in registers
// (ceil(nblk / P) <= RPT, P = 1024 / E' parts per expert, E' = E rounded up to a
// power of two).  Thread (part gj, expert ge) with the expert index fastest across
// lanes: its run of histogram entries is loaded once (coalesced over experts),
// summed, and rewritten as running bases from the same registers; the parts of an
// expert meet once in LDS, where expert thread e turns them into an exclusive
// prefix and its total.
template <int RPT>
__global__ __launch_bounds__(1024) void k_perm_scan_reg(int32_t* __restrict__ blk,
                                                        const int32_t* __restrict__ blk2, int nblk,
                                                        int64_t T, int E, int S, int BM,
                                                        int32_t* __restrict__ offsets,
                                                        int32_t* __restrict__ active,
                                                        int32_t* __restrict__ meta,
                                                        int2* __restrict__ tiles) {
  __shared__ int tmp[32];
  __shared__ int offs[1025];
  __shared__ int psum[1024];                       // [part][E'] sums, then exclusive prefixes
  int Ep = 1;
  while (Ep < E) Ep <<= 1;
  const int P = 1024 / Ep;
  const int tid = threadIdx.x, ge = tid & (Ep - 1), gj = tid / Ep;
  const bool mine = ge < E;
  const int per = (nblk + P - 1) / P;
  const int b0 = gj * per;
  int v[RPT];
#pragma unroll
  for (int i = 0; i < RPT; ++i) {
    const int b = b0 + i;
    v[i] = (mine && i < per && b < nblk) ? blk[int64_t(b) * E + ge] : 0;
  }
  if (blk2) {                                      // uniform: every load issued before any add
    int v2[RPT];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int b = b0 + i;
      v2[i] = (mine && i < per && b < nblk) ? blk2[int64_t(b) * E + ge] : 0;
    }
#pragma unroll
    for (int i = 0; i < RPT; ++i) v[i] += v2[i];
  }
  int part = 0;
#pragma unroll
  for (int i = 0; i < RPT; ++i) part += v[i];
  psum[tid] = part;
  __syncthreads();
  int cnt = 0;
  if (tid < E) {
    int run = 0;
    for (int g = 0; g < P; ++g) {
      const int x = psum[g * Ep + tid];
      psum[g * Ep + tid] = run;
      run += x;
    }
    cnt = run;
  } else if (tid < E + S) {
    cnt = int(T);
  }
  build_schedule(cnt, E + S, BM, offs, active, meta, tiles, tmp);
  __syncthreads();
  // E + S may be 1024: the total offsets[E + S] then lies beyond the last thread
  for (int i = threadIdx.x; i <= E + S; i += blockDim.x) offsets[i] = offs[i];
  if (mine) {
    int r = offs[ge] + psum[tid];
#pragma unroll
    for (int i = 0; i < RPT; ++i) {
      const int b = b0 + i;
      if (i < per && b < nblk) blk[int64_t(b) * E + ge] = r;
      r += v[i];
    }
  }
}

// Stable scatter, one block of four waves per permutation block of 64 tokens:
// lane = token of the block, wave w takes the slots j = w, w + 4, ...  The rank of
// (t, j) among the block's rows of expert e is the number of lower tokens of the
// block that also chose e (a token chooses an expert at most once): a 64-bit token
// mask per expert built with LDS atomic ORs.  grid = nblk, block = 256, dynamic
// LDS = E*8 bytes.
__global__ __launch_bounds__(256) void k_perm_scatter(
    const int32_t* __restrict__ ids, const float* __restrict__ w, int64_t T, int k, int E, int S,
    const int32_t* __restrict__ blk_base, int32_t* __restrict__ row_token,
    int32_t* __restrict__ inv, float* __restrict__ row_w) {
  extern __shared__ unsigned long long bits[];  // [E]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < E; i += 256) bits[i] = 0ull;
  __syncthreads();
  const int64_t t = int64_t(blockIdx.x) * 64 + lane;
  const bool valid = t < T;
  // this wave's slots of the token (k <= 16: at most four), all loads issued first
  int id[4];
  float wt[4];
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = wv + 4 * q;
    id[q] = (valid && j < k) ? ids[t * k + j] : 0;
    wt[q] = (valid && j < k && row_w) ? w[t * k + j] : 0.f;
  }
#pragma unroll
  for (int q = 0; q < 4; ++q)
    if (valid && wv + 4 * q < k) atomicOr(&bits[id[q]], 1ull << lane);
  __syncthreads();
  if (!valid) return;
  const unsigned long long lower = (1ull << lane) - 1ull;
  const int32_t* base = blk_base + int64_t(blockIdx.x) * E;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int j = wv + 4 * q;
    if (j >= k) break;
    const int e = id[q];
    const int r = base[e] + __popcll(bits[e] & lower);
    row_token[r] = int32_t(t);
    inv[t * k + j] = r;
    if (row_w) row_w[r] = wt[q];
  }
  for (int s = wv; s < S; s += 4) {
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
  // E + S may be 1024: the total offsets[E + S] then lies beyond the last thread
  for (int i = threadIdx.x; i <= E + S; i += blockDim.x) offsets[i] = offs[i];
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
                        const int32_t* blk2, int32_t* offsets, int32_t* active, int32_t* meta,
                        int2* tiles, int32_t* row_token, int32_t* inv, float* row_w, int BM,
                        hipStream_t st) {
  int Ep = 1;
  while (Ep < p.E) Ep <<= 1;
  const int per = (p.nblk + 1024 / Ep - 1) / (1024 / Ep);    // histogram blocks per thread
  if (per <= 8)
    hipLaunchKernelGGL(k_perm_scan_reg<8>, dim3(1), dim3(1024), 0, st, blk, blk2, p.nblk, p.T, p.E, p.S,
                       BM, offsets, active, meta, tiles);
  else if (per <= 16)
    hipLaunchKernelGGL(k_perm_scan_reg<16>, dim3(1), dim3(1024), 0, st, blk, blk2, p.nblk, p.T, p.E, p.S,
                       BM, offsets, active, meta, tiles);
  else if (per <= 32)
    hipLaunchKernelGGL(k_perm_scan_reg<32>, dim3(1), dim3(1024), 0, st, blk, blk2, p.nblk, p.T, p.E, p.S,
                       BM, offsets, active, meta, tiles);
  else
    hipLaunchKernelGGL(k_perm_scan, dim3(1), dim3(1024), 0, st, blk, blk2, p.nblk, p.T, p.E, p.S, BM,
                       offsets, active, meta, tiles);
  hipLaunchKernelGGL(k_perm_scatter, dim3(unsigned(p.nblk)), dim3(256), size_t(p.E) * 8, st, ids,
                     w, p.T, p.k, p.E, p.S, blk, row_token, inv, row_w);
  return check_launch();
}

int launch_permute(const Plan& p, const int32_t* ids, const float* w, int32_t* blk,
                   int32_t* offsets, int32_t* active, int32_t* meta, int2* tiles,
                   int32_t* row_token, int32_t* inv, float* row_w, int BM, hipStream_t st) {
  const unsigned g4 = unsigned((p.T + 255) / 256);
  hipLaunchKernelGGL(k_perm_count, dim3(g4), dim3(256), size_t(4) * p.E * sizeof(int), st, ids,
                     p.T, p.k, p.E, blk);
  return launch_scan_scatter(p, ids, w, blk, nullptr, offsets, active, meta, tiles, row_token, inv, row_w,
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
