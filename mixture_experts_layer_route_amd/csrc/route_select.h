// Group-limited top-k selection for one token (device inline).
//
// Group-limited routing: TensorFold issue #1247 "Ling-3.0-tiny on a Qualcomm
// board", list "What it does not cover"; groups and kept-group count from its
// config paragraph.  Ties go to the lower group / expert index; the weights are
// the softmax over the chosen logits, which equals the softmax scores of the
// chosen experts renormalised to sum 1.  Softmax is monotone, so ranking runs
// on the fp32 logits themselves with (score, index) keys: larger key wins.
#pragma once

#include "moe_device.h"

namespace moe {

__device__ __forceinline__ float key_score(uint64_t key) {
  uint32_t u = uint32_t(key >> 32);
  u = (u & 0x80000000u) ? (u & 0x7FFFFFFFu) : ~u;
  return __uint_as_float(u);
}

// ---------------------------------------------------------------------------
// One wave per token (low latency, for a handful of tokens).  `l` points to the
// token's E logits.  Lane g < G holds group g's score (G <= 64); each lane holds
// experts lane + 64q, q < QMAX, as keys; each of the Gk (then k) rounds is one
// wave-wide arg-max.  Must be called with the whole wave active.
template <int QMAX>
__device__ void select_token_wave(const float* __restrict__ l, int E, int G, int Gk, int k,
                                  int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int n = E / G;
  float lv[QMAX];
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    const int e = lane + 64 * q;
    lv[q] = e < E ? l[e] : -__builtin_huge_valf();
  }
  uint64_t kept = ~0ull;
  if (G > 1) {
    // group maxima from the logits already in registers: lane g ends up with group g's score
    float gm = -__builtin_huge_valf();
    if ((n & (n - 1)) == 0 && n <= 64) {
      // groups are aligned runs of n lanes inside one 64-expert slice: segmented
      // max by DPP inside rows of 16 (plus readlane across rows for n = 32, 64),
      // then lane g picks group g's value from lane (g*n) % 64 of slice g*n/64
#pragma unroll
      for (int q = 0; q < QMAX; ++q) {
        float v = lv[q];
        if (n >= 2) v = fmaxf(v, dppf<0xB1>(v));     // quad_perm [1,0,3,2]
        if (n >= 4) v = fmaxf(v, dppf<0x4E>(v));     // quad_perm [2,3,0,1]
        if (n >= 8) v = fmaxf(v, dppf<0x141>(v));    // row_half_mirror
        if (n >= 16) v = fmaxf(v, dppf<0x140>(v));   // row_mirror
        const float r0 = lanef(v, 0), r1 = lanef(v, 16), r2 = lanef(v, 32), r3 = lanef(v, 48);
        const int per = 64 / n;                      // groups in this slice
        const int g = lane - q * per;                // this lane's group inside slice q
        const float sh = __shfl(v, (g * n) & 63, 64);   // whole wave active here
        if (g >= 0 && g < per && lane < G) {
          if (n >= 64) gm = fmaxf(fmaxf(r0, r1), fmaxf(r2, r3));
          else if (n == 32) gm = g == 0 ? fmaxf(r0, r1) : fmaxf(r2, r3);
          else gm = sh;
        }
      }
    } else if (n % 64 == 0) {
      // a group is n/64 whole slices
#pragma unroll
      for (int q = 0; q < QMAX; ++q) {
        const float v = wave_max(lv[q]);
        if (lane == (64 * q) / n) gm = fmaxf(gm, v);
      }
    } else {
      if (lane < G) {
        float m = l[lane * n];
        for (int i = 1; i < n; ++i) m = fmaxf(m, l[lane * n + i]);
        gm = m;
      }
    }
    uint64_t gkey = lane < G ? rank_key(gm, lane) : 0ull;
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
    keys[q] = (e < E && ((kept >> (e / n)) & 1ull)) ? rank_key(lv[q], e) : 0ull;
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
  const float p = lane < k ? __expf(lsel - lmax) : 0.f;
  const float z = wave_sum(p);
  if (lane < k) {
    ids_out[lane] = idsel;
    w_out[lane] = p / z;
  }
}

// ---------------------------------------------------------------------------
// One thread per token (throughput, for many tokens).  The token's logits are at
// l[e * stride] (LDS or global).  `gscratch` holds G floats per thread at
// gscratch[g * gstride].  Keys of the K best experts are kept sorted in
// registers by insertion.  Returns the K ids and weights through the pointers.
template <int K>
__device__ void select_token_thread(const float* l, int stride, int E, int G, int Gk,
                                    float* gscratch, int gstride, int32_t* __restrict__ ids_out,
                                    float* __restrict__ w_out) {
  const int n = E / G;
  uint64_t kept = ~0ull;
  if (G > 1) {
    for (int g = 0; g < G; ++g) {
      float m = l[(g * n) * stride];
      for (int i = 1; i < n; ++i) m = fmaxf(m, l[(g * n + i) * stride]);
      gscratch[g * gstride] = m;
    }
    kept = 0;
    for (int r = 0; r < Gk; ++r) {
      uint64_t best = 0;
      for (int g = 0; g < G; ++g) {
        if ((kept >> g) & 1ull) continue;
        const uint64_t key = rank_key(gscratch[g * gstride], g);
        best = key > best ? key : best;
      }
      kept |= 1ull << key_index(best);
    }
  }
  uint64_t keys[K];
#pragma unroll
  for (int i = 0; i < K; ++i) keys[i] = 0ull;
  for (int g = 0; g < G; ++g) {
    if (!((kept >> g) & 1ull)) continue;
    for (int e = g * n; e < (g + 1) * n; ++e) {
      const uint64_t c = rank_key(l[e * stride], e);
      if (c <= keys[K - 1]) continue;
      // sorted (descending) insertion: keys[i] = max(keys[i], min(keys[i-1], c))
#pragma unroll
      for (int i = K - 1; i >= 1; --i) {
        const uint64_t lo = keys[i - 1] < c ? keys[i - 1] : c;
        keys[i] = keys[i] > lo ? keys[i] : lo;
      }
      keys[0] = keys[0] > c ? keys[0] : c;
    }
  }
  const float lmax = key_score(keys[0]);
  float p[K], z = 0.f;
#pragma unroll
  for (int i = 0; i < K; ++i) {
    p[i] = __expf(key_score(keys[i]) - lmax);
    z += p[i];
  }
#pragma unroll
  for (int i = 0; i < K; ++i) {
    ids_out[i] = key_index(keys[i]);
    w_out[i] = p[i] / z;
  }
}

}  // namespace moe
