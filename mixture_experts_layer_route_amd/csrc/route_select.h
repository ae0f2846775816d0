// Wave-level group-limited top-k selection for one token (device inline).
//
// Group-limited routing: TensorFold issue #1247 "Ling-3.0-tiny on a Qualcomm
// board", list "What it does not cover"; groups and kept-group count from its
// config paragraph.  Ties go to the lower group / expert index; the weights are
// the softmax over the chosen logits, which equals the softmax scores of the
// chosen experts renormalised to sum 1.
#pragma once

#include "moe_device.h"

namespace moe {

// ---------------------------------------------------------------------------
// Selection for one token by one wave.  `l` points to the token's E logits
// (bias included).  Groups: lane g < G holds group g's score (G <= 64).
// Experts: lane holds experts lane + 64q, q < QMAX, as (score, index) keys.
// Each of the Gk (then k) rounds is one wave-wide arg-max over the keys.
__device__ __forceinline__ float key_score(uint64_t key) {
  uint32_t u = uint32_t(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

template <int QMAX>
__device__ void select_token(const float* __restrict__ l, int E, int G, int Gk, int k,
                             int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int n = E / G;
  uint64_t kept = ~0ull;
  if (G > 1) {
    uint64_t gkey = 0;
    if (lane < G) {
      float m = l[lane * n];
      for (int i = 1; i < n; ++i) m = fmaxf(m, l[lane * n + i]);
      gkey = rank_key(m, lane);
    }
    kept = 0;
    for (int r = 0; r < Gk; ++r) {
      const uint64_t win = wave_max_u64(gkey);
      const int gw = key_index(win);
      kept |= 1ull << gw;
      if (lane == gw) gkey = 0;
    }
  }
  uint64_t keys[QMAX];
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    const int e = lane + 64 * q;
    keys[q] = (e < E && ((kept >> (e / n)) & 1ull)) ? rank_key(l[e], e) : 0ull;
  }
  int idsel = 0;
  float lsel = 0.f, lmax = 0.f;
  for (int r = 0; r < k; ++r) {
    uint64_t best = keys[0];
#pragma unroll
    for (int q = 1; q < QMAX; ++q) best = keys[q] > best ? keys[q] : best;
    const uint64_t win = wave_max_u64(best);
#pragma unroll
    for (int q = 0; q < QMAX; ++q)
      if (keys[q] == win) keys[q] = 0ull;
    const float lw = key_score(win);
    if (r == 0) lmax = lw;
    if (lane == r) { idsel = key_index(win); lsel = lw; }
  }
  // weights: softmax over the chosen logits (= renormalised softmax scores)
  const float p = lane < k ? __expf(lsel - lmax) : 0.f;
  const float z = wave_sum(p);
  if (lane < k) {
    ids_out[lane] = idsel;
    w_out[lane] = p / z;
  }
}

}  // namespace moe
