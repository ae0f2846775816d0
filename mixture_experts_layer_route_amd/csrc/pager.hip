// Expert paging: routed experts kept in host memory, an HBM arena of slots.
//
// The HelloSun/ling30tiny model card describes the idea in its introduction:
// experts that are not active stay off the compute device and a bounded arena holds
// the experts the router currently selects; its RAM-limit table (RAM 上限實測)
// reports the arena in slots and a hot rate.  Here the store is pinned host memory
// (read by the GPU over the host link), the arena is HBM, and every decision is
// taken on the device after the routing, so the host never waits for it:
//   k_pager_plan  (one block) looks the call's distinct experts up, picks victim
//                 slots for the misses (slots the call does not need, least
//                 recently used first, ties to the lower slot; misses in ascending
//                 expert order take them in that order), updates the tables and
//                 counters, writes the call's slot ids and the copy list;
//   k_pager_copy  copies the missed experts' gate/up/down matrices from the store
//                 into their slots (grid-stride over 16-byte chunks).
// State (device memory, laid out by pager_layout): counters int64[8] = calls,
// routed references, lookups, hits, misses, bytes copied; key_slot[E]; slot_key[N];
// stamp[N] (number of the last call that used the slot, 0 = never used).
#include "moe_internal.h"

namespace moe {

PagerLayout pager_layout(int E, int N) {
  auto a256 = [](size_t v) { return (v + 255) & ~size_t(255); };
  PagerLayout L{};
  L.o_counters = 0;
  L.o_key_slot = a256(8 * sizeof(int64_t));
  L.o_slot_key = L.o_key_slot + a256(size_t(E) * 4);
  L.o_stamp = L.o_slot_key + a256(size_t(N) * 4);
  L.total = L.o_stamp + a256(size_t(N) * 8);
  return L;
}

__global__ __launch_bounds__(1024) void k_pager_reset(int64_t* __restrict__ counters,
                                                      int32_t* __restrict__ key_slot,
                                                      int32_t* __restrict__ slot_key,
                                                      int64_t* __restrict__ stamp, int E, int N) {
  const int tid = threadIdx.x;
  if (tid < 8) counters[tid] = 0;
  for (int e = tid; e < E; e += 1024) key_slot[e] = -1;
  for (int s = tid; s < N; s += 1024) {
    slot_key[s] = -1;
    stamp[s] = 0;
  }
}

// Minimum of a 64-bit value over the block (1024 threads); `red` holds >= 16 values.
__device__ int64_t block_min_i64(int64_t v, int64_t* red) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const int lo = __shfl_xor(int(uint32_t(uint64_t(v))), o, 64);
    const int hi = __shfl_xor(int(uint32_t(uint64_t(v) >> 32)), o, 64);
    const int64_t w = int64_t((uint64_t(uint32_t(hi)) << 32) | uint32_t(lo));
    v = w < v ? w : v;
  }
  if (lane == 0) red[wv] = v;
  __syncthreads();
  int64_t m = red[0];
  for (int i = 1; i < int(blockDim.x >> 6); ++i) m = red[i] < m ? red[i] : m;
  __syncthreads();
  return m;
}

// Exclusive scan over the block (1024 threads) of 0/1 flags; `tmp` holds >= 16 ints.
__device__ int block_scan_flags(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const uint64_t mask = __ballot(v != 0);
  const int below = __popcll(mask & ((1ull << lane) - 1ull));
  if (lane == 0) tmp[wv] = __popcll(mask);
  __syncthreads();
  int base = 0, tot = 0;
  for (int i = 0; i < int(blockDim.x >> 6); ++i) {
    if (i < wv) base += tmp[i];
    tot += tmp[i];
  }
  __syncthreads();
  total = tot;
  return base + below;
}

// One block of 1024 threads; E <= 1024, N <= E.  Thread e owns expert e, thread s slot s.
__global__ __launch_bounds__(1024) void k_pager_plan(
    const int32_t* __restrict__ ids, int nslot, int E, int N, int64_t expert_bytes,
    int64_t* __restrict__ counters, int32_t* __restrict__ key_slot, int32_t* __restrict__ slot_key,
    int64_t* __restrict__ stamp, int32_t* __restrict__ ids_slot, int32_t* __restrict__ copies) {
  __shared__ int need[1024];
  __shared__ int ks[1024];       // slot of each expert (updated in place)
  __shared__ int held[1024];     // slot held by an expert this call needs
  __shared__ int owner[1024];    // miss expert that takes the slot, or -1
  __shared__ int victim[1024];   // victim slot of the m-th miss
  __shared__ int tmp[16];
  __shared__ int64_t red[16];
  const int tid = threadIdx.x;
  const int64_t clock = counters[0] + 1;
  const int e = tid, s = tid;
  victim[tid] = -1;
  if (e < E) {
    need[e] = 0;
    ks[e] = key_slot[e];
  }
  int old_key = -1;
  int64_t st = INT64_MAX;
  if (s < N) {
    held[s] = 0;
    owner[s] = -1;
    old_key = slot_key[s];
    st = stamp[s];
  }
  __syncthreads();
  for (int i = tid; i < nslot; i += 1024) need[ids[i]] = 1;
  __syncthreads();
  const bool needed = e < E && need[e] != 0;
  if (needed && ks[e] >= 0) held[ks[e]] = 1;
  const bool is_miss = needed && ks[e] < 0;
  int n_miss, n_need;
  const int miss_rank = block_scan_flags(is_miss, tmp, n_miss);
  block_scan_flags(needed, tmp, n_need);
  // victims: the n_miss smallest (stamp, slot) among slots no needed expert holds,
  // taken one stamp value at a time (in slot order within a value)
  bool cand = s < N && held[s] == 0;
  int assigned = 0;
  while (assigned < n_miss) {                      // block-uniform loop
    const int64_t mv = block_min_i64(cand ? st : INT64_MAX, red);
    const bool eq = cand && st == mv;
    int cnt;
    const int r = block_scan_flags(eq, tmp, cnt);
    if (cnt == 0) break;                           // cannot happen while N >= distinct needs
    const int take = min(n_miss - assigned, cnt);
    if (eq && r < take) {
      victim[assigned + r] = s;
      cand = false;
    }
    assigned += take;
    __syncthreads();
  }
  if (is_miss && victim[miss_rank] >= 0) {
    const int v = victim[miss_rank];
    owner[v] = e;
    copies[1 + 2 * miss_rank] = e;
    copies[2 + 2 * miss_rank] = v;
  }
  __syncthreads();
  if (s < N && owner[s] >= 0) {
    if (old_key >= 0) ks[old_key] = -1;            // the evicted expert is not needed
    slot_key[s] = owner[s];
  }
  if (is_miss) ks[e] = victim[miss_rank];
  __syncthreads();
  if (needed && ks[e] >= 0) stamp[ks[e]] = clock;
  if (e < E) key_slot[e] = ks[e];
  // (a slot id is never negative here while N >= the distinct needs; clamped anyway)
  for (int i = tid; i < nslot; i += 1024) ids_slot[i] = max(ks[ids[i]], 0);
  if (tid == 0) {
    copies[0] = assigned;
    counters[0] = clock;
    counters[1] += nslot;
    counters[2] += n_need;
    counters[3] += n_need - n_miss;
    counters[4] += n_miss;
    counters[5] += int64_t(n_miss) * expert_bytes;
  }
}

// Copy the listed experts' three matrices (mat_bytes[j] each, a multiple of 16) from
// the store into their slots.  Work unit: one 16-byte chunk of one copy.
__global__ __launch_bounds__(256) void k_pager_copy(const int32_t* __restrict__ copies,
                                                    PagerCopyArgs a) {
  const int n = copies[0];
  const int64_t per = a.chunks[0] + a.chunks[1] + a.chunks[2];
  const int64_t total = int64_t(n) * per;
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  for (int64_t u = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; u < total; u += stride) {
    const int m = int(u / per);
    int64_t c = u - int64_t(m) * per;
    int j = 0;
    while (j < 2 && c >= a.chunks[j]) c -= a.chunks[j++];
    const int64_t key = copies[1 + 2 * m], slot = copies[2 + 2 * m];
    const uint4* src = reinterpret_cast<const uint4*>(a.src[j]) + key * a.chunks[j] + c;
    uint4* dst = reinterpret_cast<uint4*>(a.dst[j]) + slot * a.chunks[j] + c;
    *dst = *src;
  }
}

int launch_pager_reset(int E, int N, void* state, hipStream_t st) {
  const PagerLayout L = pager_layout(E, N);
  char* b = static_cast<char*>(state);
  hipLaunchKernelGGL(k_pager_reset, dim3(1), dim3(1024), 0, st,
                     reinterpret_cast<int64_t*>(b + L.o_counters),
                     reinterpret_cast<int32_t*>(b + L.o_key_slot),
                     reinterpret_cast<int32_t*>(b + L.o_slot_key),
                     reinterpret_cast<int64_t*>(b + L.o_stamp), E, N);
  return check_launch();
}

int launch_pager_plan(const int32_t* ids, int nslot, int E, int N, int64_t expert_bytes,
                      void* state, int32_t* ids_slot, int32_t* copies, hipStream_t st) {
  const PagerLayout L = pager_layout(E, N);
  char* b = static_cast<char*>(state);
  hipLaunchKernelGGL(k_pager_plan, dim3(1), dim3(1024), 0, st, ids, nslot, E, N, expert_bytes,
                     reinterpret_cast<int64_t*>(b + L.o_counters),
                     reinterpret_cast<int32_t*>(b + L.o_key_slot),
                     reinterpret_cast<int32_t*>(b + L.o_slot_key),
                     reinterpret_cast<int64_t*>(b + L.o_stamp), ids_slot, copies);
  return check_launch();
}

int launch_pager_copy(const int32_t* copies, const PagerCopyArgs& a, int max_copies,
                      hipStream_t st) {
  const int64_t per = a.chunks[0] + a.chunks[1] + a.chunks[2];
  const int64_t most = int64_t(max_copies) * per;
  const unsigned grid = unsigned(std::max<int64_t>(1, std::min<int64_t>(2048, (most + 255) / 256)));
  hipLaunchKernelGGL(k_pager_copy, dim3(grid), dim3(256), 0, st, copies, a);
  return check_launch();
}

}  // namespace moe
