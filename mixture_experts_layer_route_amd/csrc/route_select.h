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
// wave-wide arg-max.  Must be called with the whole wave active.  Returns, in
// lane j < k, the id of the j-th chosen expert.
template <int QMAX>
__device__ int select_token_wave(const float* __restrict__ l, int E, int G, int Gk, int k,
                                 int32_t* __restrict__ ids_out, float* __restrict__ w_out) {
  const int lane = threadIdx.x & 63;
  const int n = E / G;
  float lv[QMAX];
#pragma unroll
  for (int q = 0; q < QMAX; ++q) {
    const int e = lane + 64 * q;
    const float v = l[min(e, E - 1)];   // clamped load, then masked: no branch around it
    lv[q] = e < E ? v : -__builtin_huge_valf();
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
  return idsel;
}

// ---------------------------------------------------------------------------
// Sixteen lanes per token (a DPP row): four tokens per wave, every reduction stays
// inside the row.  Lane r of the row holds experts [V*r, V*r + V) (E = 16 V).
// Groups of n = E/G experts: either a group spans n/V whole lanes (n >= V, n/V a
// power of two), or a lane holds V/n whole groups (n < V); G <= 64.  Keys are
// (score, index) as in select_token_wave.  Returns, in row lane j < k, the j-th
// chosen expert and its weight through `id_out` / `w_out`.
__device__ __forceinline__ uint32_t row_max_u32(uint32_t v) {
  v = max(v, dpp32_mov<0xB1>(v));    // quad_perm [1,0,3,2]
  v = max(v, dpp32_mov<0x4E>(v));    // quad_perm [2,3,0,1]
  v = max(v, dpp32_mov<0x141>(v));   // row_half_mirror
  return max(v, dpp32_mov<0x140>(v));   // row_mirror
}
// Row maximum of 64-bit keys as two 32-bit maxima (the high words, then the low
// words of the lanes holding the highest high word): the same lexicographic
// maximum with 32-bit DPP steps the compiler can fold into the max instructions.
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
  const uint32_t hi = uint32_t(v >> 32), lo = uint32_t(v);
  const uint32_t mh = row_max_u32(hi);
  const uint32_t ml = row_max_u32(hi == mh ? lo : 0u);
  return (uint64_t(mh) << 32) | ml;
}
__device__ __forceinline__ float row_sum(float v) {
  v += dppf<0xB1>(v);
  v += dppf<0x4E>(v);
  v += dppf<0x141>(v);
  return v + dppf<0x140>(v);
}
__device__ __forceinline__ float row_segmax(float v, int span) {   // max over aligned runs of `span` lanes
  if (span >= 2) v = fmaxf(v, dppf<0xB1>(v));
  if (span >= 4) v = fmaxf(v, dppf<0x4E>(v));
  if (span >= 8) v = fmaxf(v, dppf<0x141>(v));
  if (span >= 16) v = fmaxf(v, dppf<0x140>(v));
  return v;
}

// Sorts a lane's V keys into descending order: Batcher's odd-even merge network in
// its iterative form (valid for any V; checked exhaustively on 0/1 inputs up to 16).
template <int V>
__device__ __forceinline__ void sort_keys_desc(uint64_t (&kv)[V]) {
#pragma unroll
  for (int p = 1; p < V; p <<= 1)
#pragma unroll
    for (int kk = p; kk >= 1; kk >>= 1)
#pragma unroll
      for (int j = kk % p; j + kk < V; j += 2 * kk)
#pragma unroll
        for (int i = 0; i < kk; ++i)
          if (i + j + kk < V && (i + j) / (2 * p) == (i + j + kk) / (2 * p)) {
            const uint64_t a = kv[i + j], b = kv[i + j + kk];
            kv[i + j] = a > b ? a : b;
            kv[i + j + kk] = a > b ? b : a;
          }
}

template <int V>
__device__ void select_token_row(const float (&lv)[V], int E, int G, int Gk, int k, int& id_out,
                                 float& w_out) {
  const int r16 = threadIdx.x & 15;
  const int n = E / G;
  uint64_t kept = ~0ull;
  if (G > 1) {
    if (n >= V) {
      // one group per lane, spanning n / V lanes
      float m = lv[0];
#pragma unroll
      for (int i = 1; i < V; ++i) m = fmaxf(m, lv[i]);
      m = row_segmax(m, n / V);
      const int g = (V * r16) / n;
      uint64_t gk = rank_key(m, g);
      kept = 0;
      for (int r = 0; r < Gk; ++r) {
        const uint64_t win = row_max_u64(gk);
        const int gw = key_index(win);
        kept |= 1ull << gw;
        if (g == gw) gk = 0;
      }
    } else {
      // V / n whole groups per lane
      constexpr int GPL_MAX = V;
      uint64_t gk[GPL_MAX];
      const int gpl = V / n;
#pragma unroll
      for (int j = 0; j < GPL_MAX; ++j) {
        float m = -__builtin_huge_valf();
        if (j < gpl)
          for (int i = 0; i < n; ++i) m = fmaxf(m, lv[j * n + i]);
        gk[j] = j < gpl ? rank_key(m, r16 * gpl + j) : 0ull;
      }
      kept = 0;
      for (int r = 0; r < Gk; ++r) {
        uint64_t best = gk[0];
#pragma unroll
        for (int j = 1; j < GPL_MAX; ++j) best = gk[j] > best ? gk[j] : best;
        const uint64_t win = row_max_u64(best);
        kept |= 1ull << key_index(win);
#pragma unroll
        for (int j = 0; j < GPL_MAX; ++j)
          if (gk[j] == win) gk[j] = 0ull;
      }
    }
  }
  uint64_t kv[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int e = V * r16 + i;
    kv[i] = ((kept >> (e / n)) & 1ull) ? rank_key(lv[i], e) : 0ull;
  }
  // Each lane's keys in descending order, so its largest remaining key is kv[0]: a
  // round is one row arg-max over the lanes' heads, and the lane that held the
  // winner (keys are distinct) moves its next key up.  Same winners, in the same
  // order, as an arg-max over every remaining key.
  sort_keys_desc<V>(kv);
  int idsel = 0;
  float lsel = 0.f, lmax = 0.f;
  for (int r = 0; r < k; ++r) {
    const uint64_t win = row_max_u64(kv[0]);
    if (kv[0] == win) {
#pragma unroll
      for (int i = 0; i + 1 < V; ++i) kv[i] = kv[i + 1];
      kv[V - 1] = 0ull;
    }
    const float lw = key_score(win);
    if (r == 0) lmax = lw;
    if (r16 == r) { idsel = key_index(win); lsel = lw; }
  }
  const float p = r16 < k ? __expf(lsel - lmax) : 0.f;
  const float z = row_sum(p);
  id_out = idsel;
  w_out = p / z;
}

}  // namespace moe
