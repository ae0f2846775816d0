// Decode-sized batches (a handful of tokens): the expert side of the layer in
// two persistent kernels after the router logits.
//
// With a few tokens the layer is a stream over the chosen experts' weights
// (TensorFold issue #1247 "Ling-3.0-tiny on a Qualcomm board", list "What it does
// not cover": experts computed over the rows routed to them), so both kernels
// are organised around that stream:
//   gate/up: every block first routes the T tokens itself from the logits into
//     LDS (sixteen lanes or a wave per token select; the rows of each expert are
//     placed in ascending (token, slot) order; block 0 publishes the routing),
//     while idle waves prefetch the experts the routing is certain to choose; then
//     each wave walks work items (active expert, NI weight rows) round-robin over
//     the grid with the next item's loads in flight while the current one is
//     multiplied; h (fp32) goes to the workspace;
//   down + combine: item = (token t, NR output columns),
//     y[t,n] = sum_j w[t,j] (h[row(t,j)] . Wd[id(t,j)][n]) + sum_s (h[shared row] . Wd_s[n]),
//     all slots of a batch loaded before any is used, the next item's weights in
//     flight while the current one is reduced.
// A single kernel with a device-wide barrier between the two halves measured
// slower on MI355X than the launch it saves (the cross-XCD arrival counting and
// cache write-back cost tens of microseconds), so the halves are two launches.
// NVFP4 experts have their own item loops here (decode, and the expert-major ones
// for batches the decode kernels do not take), and MXFP4 experts share the NVFP4
// decode layout with MX block scales and MXFP8 activations; the decoder step adds
// the residual in the down kernels.
#include <type_traits>

#include "moe_internal.h"

#ifndef MOE_DEC_PF
#define MOE_DEC_PF 8   // prefetch loads (1 KB each) per prefetching wave, 0 = none
#endif
#ifndef MOE_DEC_PF_TOPM
#define MOE_DEC_PF_TOPM 2   // experts per token the prefetch covers (certain while <= Gk)
#endif
#include "route_select.h"

namespace moe {

template <typename TW>
__device__ __forceinline__ const TW* dexpert(const TW* routed, const TW* shared, int e, int E,
                                             int64_t stride) {
  return e < E ? routed + int64_t(e) * stride : shared + int64_t(e - E) * stride;
}

// Tag type: expert weights stored as NVFP4 (packed E2M1 codes, e4m3 scale per 16
// inputs, fp32 scale per matrix).
struct nvfp4_t {};
// Tag type: expert weights stored as MXFP4 (packed E2M1 codes, an E8M0 scale per 32
// inputs, no matrix scale); x and h enter the products as MXFP8 (E4M3 elements with
// a shared power-of-two exponent per 32).
struct mxfp4_t {};

template <typename TB>
__device__ __forceinline__ const TB* nv_expert(const TB* routed, const TB* shared, int e, int E,
                                               int64_t stride) {
  return e < E ? routed + int64_t(e) * stride : shared + int64_t(e - E) * stride;
}

typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2_t;

// Dot of 16 consecutive E2M1 weights (two dwords of codes, element 2i in the low
// nibble of byte i) with 16 bf16 activations (eight dwords of bf16 pairs).  Each
// code byte becomes a bf16 pair exactly (every E2M1 value is a bf16 value), and
// each pair product is accumulated in fp32 by the packed bf16 dot.
__device__ __forceinline__ float dot16_fp4_bf16(uint32_t c0, uint32_t c1, const uint32_t* x) {
  auto w = [](uint32_t c, int sel) {
    switch (sel) {
      case 0: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 0);
      case 1: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 1);
      case 2: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 2);
      default: return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(c, 1.0f, 3);
    }
  };
  auto xb = [&](int i) { return __builtin_bit_cast(bf16x2_t, x[i]); };
  float d0 = 0.f, d1 = 0.f;
  d0 = __builtin_amdgcn_fdot2_f32_bf16(w(c0, 0), xb(0), d0, false);
  d1 = __builtin_amdgcn_fdot2_f32_bf16(w(c0, 1), xb(1), d1, false);
  d0 = __builtin_amdgcn_fdot2_f32_bf16(w(c0, 2), xb(2), d0, false);
  d1 = __builtin_amdgcn_fdot2_f32_bf16(w(c0, 3), xb(3), d1, false);
  d0 = __builtin_amdgcn_fdot2_f32_bf16(w(c1, 0), xb(4), d0, false);
  d1 = __builtin_amdgcn_fdot2_f32_bf16(w(c1, 1), xb(5), d1, false);
  d0 = __builtin_amdgcn_fdot2_f32_bf16(w(c1, 2), xb(6), d0, false);
  d1 = __builtin_amdgcn_fdot2_f32_bf16(w(c1, 3), xb(7), d1, false);
  return d0 + d1;
}

// Dot of 16 consecutive E2M1 weights with 16 fp32 values.
__device__ __forceinline__ float dot16_fp4_f32(uint32_t c0, uint32_t c1, const float* v) {
  auto w = [](uint32_t c, int sel) {
    switch (sel) {
      case 0: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 0);
      case 1: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 1);
      case 2: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 2);
      default: return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(c, 1.0f, 3);
    }
  };
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const auto p = w(c0, b), q = w(c1, b);
    d0 = fmaf(p[0], v[2 * b], d0);
    d1 = fmaf(p[1], v[2 * b + 1], d1);
    d0 = fmaf(q[0], v[8 + 2 * b], d0);
    d1 = fmaf(q[1], v[8 + 2 * b + 1], d1);
  }
  return d0 + d1;
}

struct DecodeArgs {
  const void* x;
  const float* logits;
  const void *wg, *wu, *wd, *shg, *shu, *shd;
  // NVFP4 experts only: e4m3 block scales (one per 16 inputs) and fp32 matrix scales
  const uint8_t *bg, *bu, *bd, *shbg, *shbu, *shbd;
  const float *gg, *gu, *gd, *shgg, *shgu, *shgd;
  int32_t* ids;        // [T, k] routing outputs (published by block 0)
  float* w;            // [T, k]
  int32_t* offsets;    // [E+S+1]
  int32_t* row_token;  // [R]
  int32_t* inv;        // [T, k]
  float* h;            // [R, I] fp32
  void* y;             // [T, H]
  const void* res;     // [T, H] residual added to y (the decoder step), or null
  uint8_t* xq;         // MXFP4 experts: x's E4M3 codes [T, H] and E8M0 scales [T, H/32],
  uint8_t* sxq;        //   written by block 0
  int T, H, I, E, S, G, Gk, k;
};

// Gate/up item loop for NVFP4 experts.  Item = (active expert, 4 consecutive rows
// of I); row q of the item is handled by the 16 lanes of DPP row q, lane cc taking
// 32-input chunks cc, cc+16, ... (16 bytes of codes and two e4m3 scales each), so a
// row's partial sums meet in one DPP row reduction.  The matrix scales multiply
// the reduced gate and up values.  The next item's loads are in flight while the
// current one is multiplied.
template <int NS>
__device__ __forceinline__ void decode_gateup_nv(const DecodeArgs& a, const bf16_t* xs,
                                                 const int32_t* off_l, const int32_t* act_l,
                                                 const int32_t* rt_l, int n_act, int lane) {
  struct Buf {
    uint4 g[NS], u[NS];
    uint32_t sg[NS], su[NS];
    float gg, gu;
  };
  const int H = a.H, I = a.I, E = a.E;
  const int H2 = H / 2, H16 = H / 16, HC = H / 32;
  const int q = lane >> 4, cc = lane & 15;
  const int ipe = I / 4;
  const int total = n_act * ipe;
  const int64_t cstr = int64_t(I) * H2, bstr = int64_t(I) * H16;
  const int gstride = gridDim.x * 4;
  const uint8_t* wg = static_cast<const uint8_t*>(a.wg);
  const uint8_t* wu = static_cast<const uint8_t*>(a.wu);
  const uint8_t* shg = static_cast<const uint8_t*>(a.shg);
  const uint8_t* shu = static_cast<const uint8_t*>(a.shu);
  auto load = [&](int item, Buf& b) {
    const int u = item / ipe, row = (item - u * ipe) * 4 + q;
    const int e = act_l[u];
    const uint8_t* gp = nv_expert(wg, shg, e, E, cstr) + int64_t(row) * H2;
    const uint8_t* up = nv_expert(wu, shu, e, E, cstr) + int64_t(row) * H2;
    const uint8_t* gs = nv_expert(a.bg, a.shbg, e, E, bstr) + int64_t(row) * H16;
    const uint8_t* us = nv_expert(a.bu, a.shbu, e, E, bstr) + int64_t(row) * H16;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = cc + 16 * s;
      if (c < HC) {
        b.g[s] = *reinterpret_cast<const uint4*>(gp + c * 16);
        b.u[s] = *reinterpret_cast<const uint4*>(up + c * 16);
        b.sg[s] = *reinterpret_cast<const uint16_t*>(gs + c * 2);
        b.su[s] = *reinterpret_cast<const uint16_t*>(us + c * 2);
      }
    }
    b.gg = e < E ? a.gg[e] : a.shgg[e - E];
    b.gu = e < E ? a.gu[e] : a.shgu[e - E];
  };
  auto compute = [&](int item, const Buf& b) {
    const int u = item / ipe, i0 = (item - u * ipe) * 4;
    const int e = act_l[u];
    float sg0[NS], sg1[NS], su0[NS], su1[NS];
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      e4m3_pair(b.sg[s], sg0[s], sg1[s]);
      e4m3_pair(b.su[s], su0[s], su1[s]);
    }
    for (int r = off_l[e]; r < off_l[e + 1]; ++r) {
      const bf16_t* xr = xs + int64_t(rt_l[r]) * H;
      float ag = 0.f, au = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = cc + 16 * s;
        if (c < HC) {
          uint32_t xv[16];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint4 t4 = *reinterpret_cast<const uint4*>(xr + c * 32 + v * 8);
            xv[4 * v] = t4.x; xv[4 * v + 1] = t4.y; xv[4 * v + 2] = t4.z; xv[4 * v + 3] = t4.w;
          }
          ag = fmaf(dot16_fp4_bf16(b.g[s].x, b.g[s].y, xv), sg0[s], ag);
          au = fmaf(dot16_fp4_bf16(b.u[s].x, b.u[s].y, xv), su0[s], au);
          ag = fmaf(dot16_fp4_bf16(b.g[s].z, b.g[s].w, xv + 8), sg1[s], ag);
          au = fmaf(dot16_fp4_bf16(b.u[s].z, b.u[s].w, xv + 8), su1[s], au);
        }
      }
      ag = row_sum(ag) * b.gg;
      au = row_sum(au) * b.gu;
      if (cc == 0) a.h[int64_t(r) * I + i0 + q] = silu(ag) * au;
    }
  };
  Buf ba, bb;
  int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item < total) load(item, ba);
  while (item < total) {
    int nxt = item + gstride;
    if (nxt < total) load(nxt, bb);
    compute(item, ba);
    item = nxt;
    if (item >= total) break;
    nxt = item + gstride;
    if (nxt < total) load(nxt, ba);
    compute(item, bb);
    item = nxt;
  }
}

// Gate/up item loop for MXFP4 experts, laid out as the NVFP4 loop (item = active
// expert and 4 rows of I, a 16-lane DPP row per weight row, lane cc taking the 32-input
// chunks cc, cc+16, ...).  A chunk is one MX block of the weight row and of the token
// row, so its partial dot (E2M1 values times the E4M3 values of x: exact products,
// fp32 sums) is scaled once, by 2 to the sum of the two shared exponents.  xs holds
// the token rows' E4M3 values (unscaled, as bf16) and sx_l their E8M0 codes.
template <int NS>
__device__ __forceinline__ void decode_gateup_mx(const DecodeArgs& a, const bf16_t* xs,
                                                 const uint8_t* sx_l, const int32_t* off_l,
                                                 const int32_t* act_l, const int32_t* rt_l,
                                                 int n_act, int lane) {
  struct Buf {
    uint4 g[NS], u[NS];
    int sg[NS], su[NS];
  };
  const int H = a.H, I = a.I, E = a.E;
  const int H2 = H / 2, HC = H / 32;
  const int q = lane >> 4, cc = lane & 15;
  const int ipe = I / 4;
  const int total = n_act * ipe;
  const int64_t cstr = int64_t(I) * H2, bstr = int64_t(I) * HC;
  const int gstride = gridDim.x * 4;
  const uint8_t* wg = static_cast<const uint8_t*>(a.wg);
  const uint8_t* wu = static_cast<const uint8_t*>(a.wu);
  const uint8_t* shg = static_cast<const uint8_t*>(a.shg);
  const uint8_t* shu = static_cast<const uint8_t*>(a.shu);
  auto load = [&](int item, Buf& b) {
    const int u = item / ipe, row = (item - u * ipe) * 4 + q;
    const int e = act_l[u];
    const uint8_t* gp = nv_expert(wg, shg, e, E, cstr) + int64_t(row) * H2;
    const uint8_t* up = nv_expert(wu, shu, e, E, cstr) + int64_t(row) * H2;
    const uint8_t* gs = nv_expert(a.bg, a.shbg, e, E, bstr) + int64_t(row) * HC;
    const uint8_t* us = nv_expert(a.bu, a.shbu, e, E, bstr) + int64_t(row) * HC;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int c = cc + 16 * s;
      if (c < HC) {
        b.g[s] = *reinterpret_cast<const uint4*>(gp + c * 16);
        b.u[s] = *reinterpret_cast<const uint4*>(up + c * 16);
        b.sg[s] = gs[c];
        b.su[s] = us[c];
      }
    }
  };
  auto compute = [&](int item, const Buf& b) {
    const int u = item / ipe, i0 = (item - u * ipe) * 4;
    const int e = act_l[u];
    for (int r = off_l[e]; r < off_l[e + 1]; ++r) {
      const int t = rt_l[r];
      const bf16_t* xr = xs + int64_t(t) * H;
      const uint8_t* sr = sx_l + t * HC;
      float ag = 0.f, au = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = cc + 16 * s;
        if (c < HC) {
          uint32_t xv[16];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const uint4 t4 = *reinterpret_cast<const uint4*>(xr + c * 32 + v * 8);
            xv[4 * v] = t4.x; xv[4 * v + 1] = t4.y; xv[4 * v + 2] = t4.z; xv[4 * v + 3] = t4.w;
          }
          const int xe = int(sr[c]) - 254;
          const float dg = dot16_fp4_bf16(b.g[s].x, b.g[s].y, xv) + dot16_fp4_bf16(b.g[s].z, b.g[s].w, xv + 8);
          const float du = dot16_fp4_bf16(b.u[s].x, b.u[s].y, xv) + dot16_fp4_bf16(b.u[s].z, b.u[s].w, xv + 8);
          ag += ldexpf(dg, b.sg[s] + xe);
          au += ldexpf(du, b.su[s] + xe);
        }
      }
      ag = row_sum(ag);
      au = row_sum(au);
      if (cc == 0) a.h[int64_t(r) * I + i0 + q] = silu(ag) * au;
    }
  };
  Buf ba, bb;
  int item = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (item < total) load(item, ba);
  while (item < total) {
    int nxt = item + gstride;
    if (nxt < total) load(nxt, bb);
    compute(item, ba);
    item = nxt;
    if (item >= total) break;
    nxt = item + gstride;
    if (nxt < total) load(nxt, ba);
    compute(item, bb);
    item = nxt;
  }
}

// The block's token rows (bf16 in LDS) -> MXFP8 in place: each 32-input block gets
// its shared exponent X (kept as the E8M0 code X + 127) and its elements become their
// E4M3 values, held unscaled as bf16 (exact: an E4M3 value has four significant bits
// and lies within bf16's range).  Four lanes (a DPP quad) hold one block, eight values
// each.  Block 0 also writes the codes and scales to global memory.
__device__ __forceinline__ void quantize_rows_mx(bf16_t* xs, uint8_t* sx_l, int n8,
                                                 uint8_t* xq, uint8_t* sxq, bool pub) {
  for (int i0 = 0; i0 < n8; i0 += 256) {        // same trip count in every lane: quads stay whole
    const int i = i0 + int(threadIdx.x);
    const bool live = i < n8;
    const uint4 raw = live ? *reinterpret_cast<const uint4*>(xs + int64_t(i) * 8) : make_uint4(0u, 0u, 0u, 0u);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    float v[8];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      v[2 * j] = __uint_as_float(w[j] << 16);
      v[2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
    }
    float m = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) m = fmaxf(m, fabsf(v[j]));
    m = fmaxf(m, dppf<0xB1>(m));    // quad_perm [1,0,3,2]
    m = fmaxf(m, dppf<0x4E>(m));    // quad_perm [2,3,0,1]
    const int X = mx_exponent(m);
    const float inv = mx_inv_scale(X);
    const uint32_t c0 = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
    const uint32_t c1 = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
    if (live) {
      auto bits = [](auto f) {
        return (__float_as_uint(f[0]) >> 16) | (__float_as_uint(f[1]) & 0xFFFF0000u);
      };
      *reinterpret_cast<uint4*>(xs + int64_t(i) * 8) =
          make_uint4(bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c0, 1.0f, false)),
                     bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c0, 1.0f, true)),
                     bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c1, 1.0f, false)),
                     bits(__builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c1, 1.0f, true)));
      if ((threadIdx.x & 3) == 0) sx_l[i >> 2] = uint8_t(X + 127);
      if (pub) {
        *reinterpret_cast<uint2*>(xq + int64_t(i) * 8) = make_uint2(c0, c1);
        if ((threadIdx.x & 3) == 0) sxq[i >> 2] = uint8_t(X + 127);
      }
    }
  }
}

// SEL > 0: a wave per token (select_token_wave<SEL>); SEL < 0: sixteen lanes per
// token, four tokens per wave (select_token_row<-SEL>)
template <typename TA, typename TW, int NS, int SEL>
__global__ __launch_bounds__(256) void k_decode_gateup(DecodeArgs a) {
  constexpr int NI = 2;            // gate/up weight rows per item
  extern __shared__ __align__(16) unsigned char lds_raw[];
  const int T = a.T, H = a.H, I = a.I, E = a.E, S = a.S, k = a.k;
  const int R = T * (k + S), nslot = T * k;
  TA* xs = reinterpret_cast<TA*>(lds_raw);
  int32_t* off_l = reinterpret_cast<int32_t*>(lds_raw + ((size_t(T) * H * sizeof(TA) + 15) & ~size_t(15)));
  int32_t* act_l = off_l + (E + S + 1);
  int32_t* rt_l = act_l + (E + S);
  int32_t* ids_l = rt_l + R;
  int32_t* inv_l = ids_l + nslot;
  float* w_l = reinterpret_cast<float*>(inv_l + nslot);
  __shared__ int tmp[8];
  __shared__ int n_act_l;
  // byte offsets from lds_raw keep the LDS address space visible to the compiler
  const size_t bits_off = (size_t(reinterpret_cast<unsigned char*>(w_l + nslot) - lds_raw) + 7) & ~size_t(7);
  unsigned long long* bits_l = reinterpret_cast<unsigned long long*>(lds_raw + bits_off);   // [4][E]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const TA* x = static_cast<const TA*>(a.x);
  const TW* wg = static_cast<const TW*>(a.wg);
  const TW* wu = static_cast<const TW*>(a.wu);
  const TW* wd = static_cast<const TW*>(a.wd);
  const TW* shg = static_cast<const TW*>(a.shg);
  const TW* shu = static_cast<const TW*>(a.shu);
  const TW* shd = static_cast<const TW*>(a.shd);

  // ---------------------------------------------------------------- 1. routing
  // slot i = t*k + j.  Wave w owns slots [64w, 64w+64): bit (i % 64) of
  // bits[w][e] says slot i chose expert e, so a slot's rank among its expert's
  // rows is a popcount of the lower bits (rows stay in ascending slot order).
  // With at most four tokens (sixteen lanes each, E + S <= 256, T*k <= 64) wave 0
  // selects every token and also builds the row tables by itself (one_wave), so the
  // other waves meet it at a single barrier.
  const bool one_wave = SEL < 0 && T <= 4 && nslot <= 64 && E + S <= 256;
  if (!one_wave)
    for (int i = threadIdx.x; i < 4 * E; i += 256) bits_l[i] = 0ull;
  // the token rows and the logits travel in one memory round trip: the row
  // chunks are loaded into registers, the selection's logits loads follow, and
  // the rows are written to LDS afterwards
  // the token rows go global -> LDS by direct loads issued first (1 KB per wave
  // instruction), so they travel together with the selection's logits loads
  constexpr int CH = 16 / sizeof(TA);
  const int nch = T * H / CH;
  for (int c0 = wv * 64; c0 < nch; c0 += 256)
    if (c0 + lane < nch) dma16(x + int64_t(c0 + lane) * CH, xs + int64_t(c0) * CH);
  if constexpr (SEL < 0) {
    constexpr int V = -SEL;
    const int t = wv * 4 + (lane >> 4), r16 = lane & 15;
    if (wv * 4 < T) {                                  // uniform over the wave
      const float* l = a.logits + int64_t(min(t, T - 1)) * E + V * r16;
      float lv[V];
      if constexpr (V % 4 == 0) {
#pragma unroll
        for (int i = 0; i < V; i += 4) {
          const float4 q = *reinterpret_cast<const float4*>(l + i);
          lv[i] = q.x; lv[i + 1] = q.y; lv[i + 2] = q.z; lv[i + 3] = q.w;
        }
      } else {
#pragma unroll
        for (int i = 0; i < V; ++i) lv[i] = l[i];
      }
      int id;
      float wt;
      select_token_row<V>(lv, E, a.G, a.Gk, k, id, wt);
      if (t < T && r16 < k) {
        ids_l[t * k + r16] = id;
        w_l[t * k + r16] = wt;
      }
    }
  } else {
    for (int t = wv; t < T; t += 4)
      select_token_wave<SEL>(a.logits + int64_t(t) * E, E, a.G, a.Gk, k, ids_l + t * k, w_l + t * k);
  }
  // Weight prefetch while the routing is still being decided.  A token's j highest raw
  // logits for j <= Gk are always selected (the j-th lies in a group of rank <= j, so
  // its group is kept, and it outranks everything else in the kept groups), so waves
  // with no selection work read the logits of tokens 0..3, find their top experts and
  // pull slices of those experts' gate/up rows through the caches with direct-to-LDS
  // loads into a scratch area that is never read (MOE_DEC_PF loads of 1 KB per wave;
  // they retire after everything the prologue waits for, so the wait below leaves
  // exactly them in flight).
  bool prefetcher = false;
#if MOE_DEC_PF > 0
  // (not for 4-bit weights: their stream is short and arithmetic-bound, measured neutral)
  if constexpr (SEL < 0 && !std::is_same<TW, nvfp4_t>::value && !std::is_same<TW, mxfp4_t>::value) {
    constexpr int V = -SEL;
    const int ngrp = (T + 3) / 4;
    if (wv >= ngrp) {                                  // uniform over the wave
      prefetcher = true;
      const int r16 = lane & 15, q = lane >> 4, Tq = min(T, 4);
      const float* l = a.logits + int64_t(min(q, Tq - 1)) * E + V * r16;
      // top-MOE_DEC_PF_TOPM experts of each row's token (all certain while <= Gk)
      uint64_t key[V];
#pragma unroll
      for (int i = 0; i < V; ++i) key[i] = rank_key(l[i], V * r16 + i);
      int ex[4 * MOE_DEC_PF_TOPM];
#pragma unroll
      for (int m = 0; m < MOE_DEC_PF_TOPM; ++m) {
        uint64_t best = 0ull;
#pragma unroll
        for (int i = 0; i < V; ++i) best = key[i] > best ? key[i] : best;
        const uint64_t win = row_max_u64(best);
#pragma unroll
        for (int i = 0; i < V; ++i) key[i] = key[i] == win ? 0ull : key[i];
        const int id = key_index(win);
#pragma unroll
        for (int qq = 0; qq < 4; ++qq) ex[qq * MOE_DEC_PF_TOPM + m] = __builtin_amdgcn_readlane(id, 16 * qq);
      }
      const int topm = min(MOE_DEC_PF_TOPM, min(a.Gk, k));
      constexpr bool NV = std::is_same<TW, nvfp4_t>::value;
      const int64_t mb = NV ? int64_t(I) * H / 2 : int64_t(I) * H * int64_t(sizeof(TW));
      const int64_t span = int64_t(Tq) * topm * 2 * mb;   // bytes of the prefetch set
      const int npw = 4 - ngrp;                         // prefetching waves per block
      const int pw = wv - ngrp;
      const unsigned char* gb = static_cast<const unsigned char*>(a.wg);
      const unsigned char* ub = static_cast<const unsigned char*>(a.wu);
      unsigned char* scratch = lds_raw + ((bits_off + size_t(4) * E * 8 + 15) & ~size_t(15)) + pw * 1024;
#pragma unroll
      for (int j = 0; j < MOE_DEC_PF; ++j) {
        int64_t o = ((int64_t(blockIdx.x) * npw + pw) * MOE_DEC_PF + j) * 1024 + lane * 16;
        o %= span;
        const int slot = int(o / (2 * mb));              // token tq's m-th expert: tq*topm + m
        const int64_t rem = o - int64_t(slot) * 2 * mb;
        const int tq = slot / topm, m = slot - tq * topm;
        int e = ex[0];
#pragma unroll
        for (int c = 1; c < 4 * MOE_DEC_PF_TOPM; ++c)
          if (c == tq * MOE_DEC_PF_TOPM + m) e = ex[c];
        const unsigned char* src = (rem < mb ? gb + rem : ub + (rem - mb)) + int64_t(e) * mb;
        dma16(src, scratch);
      }
    }
  }
#endif
  if (prefetcher) wait_vm_lgkm0<MOE_DEC_PF>(); else wait_vm_lgkm0<0>();
  const bool pub = blockIdx.x == 0;
  if (one_wave) {
    if (wv == 0) {
      // everything below is this wave's own LDS traffic, in program order: the slot
      // masks (one 64-bit mask per expert), counts, one wave-wide exclusive scan of
      // (rows | 1 << 16 if active) over four experts per lane, then the placement
      for (int e = lane; e < E; e += 64) bits_l[e] = 0ull;
      if (lane < nslot) atomicOr(&bits_l[ids_l[lane]], 1ull << lane);
      int v[4], sum = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = 4 * lane + q;
        const int c = e < E ? __popcll(bits_l[e]) : e < E + S ? T : 0;
        v[q] = c | (c > 0 ? 1 << 16 : 0);
        sum += v[q];
      }
      int incl = sum;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(incl, o, 64);
        if (lane >= o) incl += y;
      }
      int run = incl - sum;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = 4 * lane + q;
        if (e < E + S) {
          off_l[e] = run & 0xFFFF;
          if (v[q]) act_l[run >> 16] = e;
          if (e >= E)
            for (int t = 0; t < T; ++t) rt_l[(run & 0xFFFF) + t] = t;
        }
        run += v[q];
      }
      const int total = __shfl(incl, 63, 64);
      if (lane == 0) {
        off_l[E + S] = total & 0xFFFF;
        n_act_l = total >> 16;
      }
      if (lane < nslot) {
        const int e = ids_l[lane];
        const int r = off_l[e] + __popcll(bits_l[e] & ((1ull << lane) - 1ull));
        rt_l[r] = lane / k;
        inv_l[lane] = r;
      }
    }
    __syncthreads();
  } else {
  __syncthreads();
  if (threadIdx.x < nslot) atomicOr(&bits_l[wv * E + ids_l[threadIdx.x]], 1ull << lane);
  __syncthreads();
  int tot = 0, nact = 0;
  for (int e0 = 0; e0 < E + S; e0 += 256) {
    const int e = e0 + threadIdx.x;
    int cnt = 0;
    if (e < E)
      cnt = __popcll(bits_l[e]) + __popcll(bits_l[E + e]) + __popcll(bits_l[2 * E + e]) +
            __popcll(bits_l[3 * E + e]);
    else if (e < E + S)
      cnt = T;
    // one scan for both the row offsets (low 16 bits) and the active-list
    // positions (high bits): at most T*(k+S) <= 768 rows
    int sum;
    const int ex = block_exclusive_scan_256(cnt | (cnt > 0 ? 1 << 16 : 0), tmp, sum);
    const int off = tot + (ex & 0xFFFF), pos = nact + (ex >> 16);
    if (e < E + S) off_l[e] = off;
    if (cnt > 0) act_l[pos] = e;
    if (e >= E && e < E + S)
      for (int t = 0; t < T; ++t) rt_l[off + t] = t;
    tot += sum & 0xFFFF;
    nact += sum >> 16;
  }
  if (threadIdx.x == 0) {
    off_l[E + S] = tot;
    n_act_l = nact;
  }
  __syncthreads();
  if (threadIdx.x < nslot) {
    const int i = threadIdx.x, e = ids_l[i];
    int r = off_l[e] + __popcll(bits_l[wv * E + e] & ((1ull << lane) - 1ull));
    for (int v = 0; v < wv; ++v) r += __popcll(bits_l[v * E + e]);
    rt_l[r] = i / k;
    inv_l[i] = r;
  }
  __syncthreads();
  }
  if (pub) {
    for (int i = threadIdx.x; i < nslot; i += 256) {
      a.ids[i] = ids_l[i];
      a.w[i] = w_l[i];
      a.inv[i] = inv_l[i];
    }
    for (int i = threadIdx.x; i <= E + S; i += 256) a.offsets[i] = off_l[i];
    for (int i = threadIdx.x; i < R; i += 256) a.row_token[i] = rt_l[i];
  }

  // ---------------------------------------------------------------- 2. gate/up
  if constexpr (std::is_same<TW, nvfp4_t>::value) {
    decode_gateup_nv<NS>(a, xs, off_l, act_l, rt_l, n_act_l, lane);
  } else if constexpr (std::is_same<TW, mxfp4_t>::value) {
    // the E8M0 codes of the token rows sit where the prefetch scratch would be
    uint8_t* sx_l = lds_raw + ((bits_off + size_t(4) * E * 8 + 15) & ~size_t(15));
    quantize_rows_mx(reinterpret_cast<bf16_t*>(xs), sx_l, T * H / 8, a.xq, a.sxq, pub);
    __syncthreads();
    decode_gateup_mx<NS>(a, reinterpret_cast<const bf16_t*>(xs), sx_l, off_l, act_l, rt_l, n_act_l, lane);
  } else {
  const int ipe = I / NI;
  const int total = n_act_l * ipe;
  const int64_t mstride = int64_t(I) * H;
  const int gstride = gridDim.x * 4;
  auto load_gu = [&](int item, Chunk8<TW> (&cg)[NS][NI], Chunk8<TW> (&cu)[NS][NI]) {
    const int u = item / ipe, i0 = (item - u * ipe) * NI;
    const int e = act_l[u];
    const TW* gp = dexpert(wg, shg, e, E, mstride) + int64_t(i0) * H;
    const TW* up = dexpert(wu, shu, e, E, mstride) + int64_t(i0) * H;
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      const int h = s * 512 + lane * 8;
      if (h < H) {
#pragma unroll
        for (int ii = 0; ii < NI; ++ii) {
          cg[s][ii].load(gp + int64_t(ii) * H + h);
          cu[s][ii].load(up + int64_t(ii) * H + h);
        }
      }
    }
  };
  auto compute_gu = [&](int item, const Chunk8<TW> (&cg)[NS][NI], const Chunk8<TW> (&cu)[NS][NI]) {
    const int u = item / ipe, i0 = (item - u * ipe) * NI;
    const int e = act_l[u];
    for (int r = off_l[e]; r < off_l[e + 1]; ++r) {
      const TA* xr = xs + rt_l[r] * H;
      float ag[NI], au[NI];
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) ag[ii] = au[ii] = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int h = s * 512 + lane * 8;
        if (h < H) {
          float xv[8];
          load8(xr + h, xv);
#pragma unroll
          for (int ii = 0; ii < NI; ++ii) {
            float f[8];
            cg[s][ii].get(f);
            ag[ii] = dot8(f, xv, ag[ii]);
            cu[s][ii].get(f);
            au[ii] = dot8(f, xv, au[ii]);
          }
        }
      }
#pragma unroll
      for (int ii = 0; ii < NI; ++ii) {
        const float g = wave_sum(ag[ii]);
        const float v = wave_sum(au[ii]);
        if (lane == ii) a.h[int64_t(r) * I + i0 + ii] = silu(g) * v;
      }
    }
  };
  {
    Chunk8<TW> ga[NS][NI], ua[NS][NI], gb[NS][NI], ub[NS][NI];
    int item = blockIdx.x * 4 + wv;
    if (item < total) load_gu(item, ga, ua);
    while (item < total) {
      int nxt = item + gstride;
      if (nxt < total) load_gu(nxt, gb, ub);
      compute_gu(item, ga, ua);
      item = nxt;
      if (item >= total) break;
      nxt = item + gstride;
      if (nxt < total) load_gu(nxt, ga, ua);
      compute_gu(item, gb, ub);
      item = nxt;
    }
  }
  }
  wait_vm_lgkm0<0>();   // no direct-to-LDS load may land after the workgroup's LDS is released
}

template <typename TA, typename TW, int NSD>
__global__ __launch_bounds__(256) void k_decode_down(DecodeArgs a) {
  constexpr int NR = 2;            // output columns per item
  constexpr int JB = 8;            // slots per load batch
  const int T = a.T, H = a.H, I = a.I, E = a.E, S = a.S, k = a.k;
  const int nslot = T * k;
  __shared__ int32_t ids_l[256], inv_l[256];
  __shared__ float w_l[256];
  __shared__ int32_t offsh_l[32];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const TW* wd = static_cast<const TW*>(a.wd);
  const TW* shd = static_cast<const TW*>(a.shd);
  for (int i = threadIdx.x; i < nslot; i += 256) {
    ids_l[i] = a.ids[i];
    inv_l[i] = a.inv[i];
    w_l[i] = a.w[i];
  }
  for (int i = threadIdx.x; i < S; i += 256) offsh_l[i] = a.offsets[E + i];
  __syncthreads();

  const int nblk_n = (H + NR - 1) / NR;
  const int dtotal = T * nblk_n;
  const int nsl = k + S;
  const int64_t dstride = int64_t(H) * I;
  const int gstride = gridDim.x * 4;
  auto slot_of = [&](int t, int j, int& e, int& r, float& wt) {
    if (j < k) {
      e = ids_l[t * k + j];
      r = inv_l[t * k + j];
      wt = w_l[t * k + j];
    } else {
      e = E + (j - k);
      r = offsh_l[j - k] + t;
      wt = 1.f;
    }
  };
  auto load = [&](int item, int jb, Chunk8<TW> (&cw)[JB][NSD][NR], float (&hv)[JB][NSD][8],
                  float (&wt)[JB]) {
    const int t = item / nblk_n, n0 = (item - t * nblk_n) * NR;
#pragma unroll
    for (int jj = 0; jj < JB; ++jj) {
      const int j = jb + jj;
      wt[jj] = 0.f;
      if (j < nsl) {
        int e, r;
        slot_of(t, j, e, r, wt[jj]);
        const TW* dp = dexpert(wd, shd, e, E, dstride) + int64_t(n0) * I;
#pragma unroll
        for (int s = 0; s < NSD; ++s) {
          const int kk = s * 512 + lane * 8;
          if (kk < I) {
#pragma unroll
            for (int nn = 0; nn < NR; ++nn)
              if (n0 + nn < H) cw[jj][s][nn].load(dp + int64_t(nn) * I + kk);
            load8(a.h + int64_t(r) * I + kk, hv[jj][s]);
          }
        }
      }
    }
  };
  Chunk8<TW> cw[JB][NSD][NR];
  float hv[JB][NSD][8];
  float wt[JB];
  for (int item = blockIdx.x * 4 + wv; item < dtotal; item += gstride) {
    const int t = item / nblk_n, n0 = (item - t * nblk_n) * NR;
    float acc[NR];
#pragma unroll
    for (int nn = 0; nn < NR; ++nn) acc[nn] = 0.f;
    for (int jb = 0; jb < nsl; jb += JB) {
      load(item, jb, cw, hv, wt);
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        if (jb + jj < nsl) {
#pragma unroll
          for (int s = 0; s < NSD; ++s) {
            const int kk = s * 512 + lane * 8;
            if (kk < I) {
#pragma unroll
              for (int nn = 0; nn < NR; ++nn) {
                float f[8];
                cw[jj][s][nn].get(f);
                acc[nn] = fmaf(wt[jj], dot8(f, hv[jj][s], 0.f), acc[nn]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int nn = 0; nn < NR; ++nn) {
      float v = wave_sum(acc[nn]);
      if (lane == nn && n0 + nn < H) {
        const int64_t o = int64_t(t) * H + n0 + nn;
        if (a.res) v += to_f32<TA>(static_cast<const TA*>(a.res)[o]);
        static_cast<TA*>(a.y)[o] = from_f32<TA>(v);
      }
    }
  }
}

// One 32-value block -> MXFP8 in place: the values become their E4M3 values (unscaled,
// exact in fp32); returns the E8M0 code X + 127 of the shared exponent.
__device__ __forceinline__ int quantize_block_mx(float (&v)[32]) {
  float m = 0.f;
#pragma unroll
  for (int j = 0; j < 32; ++j) m = fmaxf(m, fabsf(v[j]));
  const int X = mx_exponent(m);
  const float inv = mx_inv_scale(X);
#pragma unroll
  for (int j = 0; j < 32; j += 4) {
    const uint32_t c = e4m3x4(v[j] * inv, v[j + 1] * inv, v[j + 2] * inv, v[j + 3] * inv);
    const auto lo = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, false);
    const auto hi = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(c, 1.0f, true);
    v[j] = lo[0]; v[j + 1] = lo[1]; v[j + 2] = hi[0]; v[j + 3] = hi[1];
  }
  return X + 127;
}

// Down + combine for NVFP4 experts.  Block item = (token t, 4*RG output columns);
// the four waves split the token's k + S slots (slot j to wave j % 4, SP slots per
// load batch), so each h row is fetched once per item and the weight rows of
// every slot stream in parallel.  Within a wave, DPP row q (16 lanes) holds
// output columns n0 + 4g + q (g < RG), lane cc the 32-input chunks cc, cc+16, ...
// of h and of the weight row.  The slot weight w[t,j] is folded with the matrix
// scale of the slot's expert.  Per-wave partial sums meet in LDS and are added in
// wave order, so the result does not depend on timing.
// MX: MXFP4 down weights (an E8M0 scale per 32 inputs, no matrix scale); a lane's
// 32-input chunk of h is one MX block, so the lane quantises it to MXFP8 by itself
// (quantize_block_mx) and scales the chunk's dot by 2 to the sum of the two exponents.
template <int NSD, int RG, int SP, bool MX>
__global__ __launch_bounds__(256) void k_decode_down_nv(DecodeArgs a) {
  constexpr int NRB = 4 * RG;
  const int T = a.T, H = a.H, I = a.I, E = a.E, S = a.S, k = a.k;
  const int nslot = T * k, nsl = k + S;
  const int I2 = I / 2, I16 = I / 16, IC = I / 32;
  const int SB = MX ? IC : I16;                    // scale bytes per weight row
  __shared__ int32_t ids_l[256], inv_l[256];
  __shared__ float w_l[256];
  __shared__ int32_t offsh_l[32];
  __shared__ float part_l[4][NRB];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int q = lane >> 4, cc = lane & 15;
  const uint8_t* wd = static_cast<const uint8_t*>(a.wd);
  const uint8_t* shd = static_cast<const uint8_t*>(a.shd);
  for (int i = threadIdx.x; i < nslot; i += 256) {
    ids_l[i] = a.ids[i];
    inv_l[i] = a.inv[i];
    w_l[i] = a.w[i];
  }
  for (int i = threadIdx.x; i < S; i += 256) offsh_l[i] = a.offsets[E + i];
  __syncthreads();

  const int nb = (H + NRB - 1) / NRB;
  const int items = T * nb;
  const int64_t cstr = int64_t(H) * I2, bstr = int64_t(H) * SB;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int t = item / nb, n0 = (item - t * nb) * NRB;
    float acc[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g] = 0.f;
    for (int j0 = wv; j0 < nsl; j0 += 4 * SP) {
      uint4 wc[SP][RG][NSD];
      uint32_t wsc[SP][RG][NSD];
      float hv[SP][NSD][32];
      float wt[SP];
#pragma unroll
      for (int m = 0; m < SP; ++m) {
        const int j = j0 + 4 * m;
        wt[m] = 0.f;
        if (j < nsl) {
          int e, r;
          if (j < k) {
            e = ids_l[t * k + j];
            r = inv_l[t * k + j];
            wt[m] = w_l[t * k + j];
          } else {
            e = E + (j - k);
            r = offsh_l[j - k] + t;
            wt[m] = 1.f;
          }
          if (!MX) wt[m] *= e < E ? a.gd[e] : a.shgd[e - E];
          const uint8_t* cp = nv_expert(wd, shd, e, E, cstr);
          const uint8_t* bp = nv_expert(a.bd, a.shbd, e, E, bstr);
#pragma unroll
          for (int s = 0; s < NSD; ++s) {
            const int c = cc + 16 * s;
            if (c < IC) {
              const float4* hp = reinterpret_cast<const float4*>(a.h + int64_t(r) * I + c * 32);
#pragma unroll
              for (int v = 0; v < 8; ++v) {
                const float4 f = hp[v];
                hv[m][s][4 * v] = f.x; hv[m][s][4 * v + 1] = f.y;
                hv[m][s][4 * v + 2] = f.z; hv[m][s][4 * v + 3] = f.w;
              }
#pragma unroll
              for (int g = 0; g < RG; ++g) {
                const int n = n0 + 4 * g + q;
                if (n < H) {
                  wc[m][g][s] = *reinterpret_cast<const uint4*>(cp + int64_t(n) * I2 + c * 16);
                  if (MX)
                    wsc[m][g][s] = bp[int64_t(n) * SB + c];
                  else
                    wsc[m][g][s] = *reinterpret_cast<const uint16_t*>(bp + int64_t(n) * SB + c * 2);
                }
              }
            }
          }
        }
      }
#pragma unroll
      for (int m = 0; m < SP; ++m) {
        if (j0 + 4 * m < nsl) {
          int hx[NSD];     // MX: h's E8M0 codes less both biases (added to the weight's code)
#pragma unroll
          for (int s = 0; s < NSD; ++s) {
            hx[s] = 0;
            if (MX && cc + 16 * s < IC) hx[s] = quantize_block_mx(hv[m][s]) - 254;
          }
#pragma unroll
          for (int g = 0; g < RG; ++g) {
            const int n = n0 + 4 * g + q;
            float d = 0.f;
#pragma unroll
            for (int s = 0; s < NSD; ++s) {
              const int c = cc + 16 * s;
              if (c < IC && n < H) {
                if (MX) {
                  const float p = dot16_fp4_f32(wc[m][g][s].x, wc[m][g][s].y, hv[m][s]) +
                                  dot16_fp4_f32(wc[m][g][s].z, wc[m][g][s].w, hv[m][s] + 16);
                  d += ldexpf(p, int(wsc[m][g][s]) + hx[s]);
                } else {
                  float s0, s1;
                  e4m3_pair(wsc[m][g][s], s0, s1);
                  d = fmaf(dot16_fp4_f32(wc[m][g][s].x, wc[m][g][s].y, hv[m][s]), s0, d);
                  d = fmaf(dot16_fp4_f32(wc[m][g][s].z, wc[m][g][s].w, hv[m][s] + 16), s1, d);
                }
              }
            }
            acc[g] = fmaf(wt[m], d, acc[g]);
          }
        }
      }
    }
#pragma unroll
    for (int g = 0; g < RG; ++g) {
      const float v = row_sum(acc[g]);
      if (cc == 0) part_l[wv][4 * g + q] = v;
    }
    __syncthreads();
    if (threadIdx.x < NRB) {
      const int n = n0 + threadIdx.x;
      if (n < H) {
        float v = (part_l[0][threadIdx.x] + part_l[1][threadIdx.x]) +
                  (part_l[2][threadIdx.x] + part_l[3][threadIdx.x]);
        const int64_t o = int64_t(t) * H + n;
        if (a.res) v += bf16_to_f32(static_cast<const bf16_t*>(a.res)[o]);
        static_cast<bf16_t*>(a.y)[o] = f32_to_bf16(v);
      }
    }
    __syncthreads();
  }
}

// ---------------------------------------------------------------------------
// NVFP4 experts for batches beyond the decode kernels (the permutation comes from
// global memory: offsets, the active-expert list and meta[0] = its length).
//
// Dot of 16 bf16 pairs held as dwords with 16 bf16 activation pairs (two chains).
__device__ __forceinline__ float dot8_bf16x2(const uint32_t* w, const uint32_t* x) {
  float d0 = 0.f, d1 = 0.f;
#pragma unroll
  for (int p = 0; p < 8; p += 2) {
    d0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[p]),
                                         __builtin_bit_cast(bf16x2_t, x[p]), d0, false);
    d1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[p + 1]),
                                         __builtin_bit_cast(bf16x2_t, x[p + 1]), d1, false);
  }
  return d0 + d1;
}

// 16 bytes of E2M1 codes -> 16 bf16 pairs (exact: every E2M1 value is a bf16 value).
__device__ __forceinline__ void fp4x32_to_bf16(const uint4& c, uint32_t (&o)[16]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[4 * i + 0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 0));
    o[4 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 1));
    o[4 * i + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 2));
    o[4 * i + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w[i], 1.0f, 3));
  }
}

// Gate/up: item = (active expert, 4 consecutive rows of I), one 16-lane DPP row per
// weight row as in the decode kernel.  The item's codes are converted once to bf16
// pairs in registers; the expert's token rows then stream through with the next row's
// activations in flight while the current one is multiplied.
template <int NS>
__global__ __launch_bounds__(256) void k_nv_gateup_batch(DecodeArgs a,
                                                         const int32_t* __restrict__ active,
                                                         const int32_t* __restrict__ meta) {
  const int H = a.H, I = a.I, E = a.E;
  const int H2 = H / 2, H16 = H / 16, HC = H / 32;
  const int lane = threadIdx.x & 63, q = lane >> 4, cc = lane & 15;
  const int ipe = I / 4;
  const int total = meta[0] * ipe;
  const int64_t cstr = int64_t(I) * H2, bstr = int64_t(I) * H16;
  const bf16_t* x = static_cast<const bf16_t*>(a.x);
  const uint8_t* wgp = static_cast<const uint8_t*>(a.wg);
  const uint8_t* wup = static_cast<const uint8_t*>(a.wu);
  const uint8_t* shg = static_cast<const uint8_t*>(a.shg);
  const uint8_t* shu = static_cast<const uint8_t*>(a.shu);
  for (int item = blockIdx.x * 4 + (threadIdx.x >> 6); item < total; item += gridDim.x * 4) {
    const int u = item / ipe, i0 = (item - u * ipe) * 4, row = i0 + q;
    const int e = active[u];
    uint32_t wg[NS][16], wu[NS][16];
    float sg[NS][2], su[NS][2];
    {
      const uint8_t* gp = nv_expert(wgp, shg, e, E, cstr) + int64_t(row) * H2;
      const uint8_t* up = nv_expert(wup, shu, e, E, cstr) + int64_t(row) * H2;
      const uint8_t* gs = nv_expert(a.bg, a.shbg, e, E, bstr) + int64_t(row) * H16;
      const uint8_t* us = nv_expert(a.bu, a.shbu, e, E, bstr) + int64_t(row) * H16;
      uint4 cg[NS], cu[NS];
      uint32_t bg2[NS], bu2[NS];
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = cc + 16 * s;
        cg[s] = cu[s] = make_uint4(0u, 0u, 0u, 0u);
        bg2[s] = bu2[s] = 0u;
        if (c < HC) {
          cg[s] = *reinterpret_cast<const uint4*>(gp + c * 16);
          cu[s] = *reinterpret_cast<const uint4*>(up + c * 16);
          bg2[s] = *reinterpret_cast<const uint16_t*>(gs + c * 2);
          bu2[s] = *reinterpret_cast<const uint16_t*>(us + c * 2);
        }
      }
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        fp4x32_to_bf16(cg[s], wg[s]);
        fp4x32_to_bf16(cu[s], wu[s]);
        e4m3_pair(bg2[s], sg[s][0], sg[s][1]);
        e4m3_pair(bu2[s], su[s][0], su[s][1]);
      }
    }
    const float ggs = e < E ? a.gg[e] : a.shgg[e - E];
    const float gus = e < E ? a.gu[e] : a.shgu[e - E];
    const int r0 = a.offsets[e], r1 = a.offsets[e + 1];
    auto loadx = [&](int r, uint4 (&xv)[NS][4]) {
      const bf16_t* xr = x + int64_t(a.row_token[r]) * H;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        const int c = cc + 16 * s;
        if (c < HC) {
#pragma unroll
          for (int v = 0; v < 4; ++v) xv[s][v] = *reinterpret_cast<const uint4*>(xr + c * 32 + v * 8);
        }
      }
    };
    auto dot = [&](int r, const uint4 (&xv)[NS][4]) {
      float ag = 0.f, au = 0.f;
#pragma unroll
      for (int s = 0; s < NS; ++s) {
        if (cc + 16 * s < HC) {
          uint32_t xw[16];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            xw[4 * v] = xv[s][v].x; xw[4 * v + 1] = xv[s][v].y;
            xw[4 * v + 2] = xv[s][v].z; xw[4 * v + 3] = xv[s][v].w;
          }
          ag = fmaf(dot8_bf16x2(wg[s], xw), sg[s][0], ag);
          au = fmaf(dot8_bf16x2(wu[s], xw), su[s][0], au);
          ag = fmaf(dot8_bf16x2(wg[s] + 8, xw + 8), sg[s][1], ag);
          au = fmaf(dot8_bf16x2(wu[s] + 8, xw + 8), su[s][1], au);
        }
      }
      ag = row_sum(ag) * ggs;
      au = row_sum(au) * gus;
      if (cc == 0) a.h[int64_t(r) * I + i0 + q] = silu(ag) * au;
    };
    uint4 xa[NS][4], xb[NS][4];
    if (r0 < r1) loadx(r0, xa);
    for (int r = r0; r < r1; r += 2) {
      if (r + 1 < r1) loadx(r + 1, xb);
      dot(r, xa);
      if (r + 1 >= r1) break;
      if (r + 2 < r1) loadx(r + 2, xa);
      dot(r + 1, xb);
    }
  }
}

// Down: item = (active expert, 4*RG output columns), expert-major into unweighted
// fp32 rows y_perm[r, n] = h[r] . Wd[e][n].  The item's codes become fp32 weights
// once (E2M1 value times its e4m3 block scale, exact in fp32; the matrix scale
// multiplies the reduced sum), then the expert's h rows stream through with the next
// row in flight.
template <int NSD, int RG>
__global__ __launch_bounds__(256) void k_nv_down_batch(DecodeArgs a,
                                                       const int32_t* __restrict__ active,
                                                       const int32_t* __restrict__ meta,
                                                       float* __restrict__ y_perm) {
  constexpr int NRB = 4 * RG;
  const int H = a.H, I = a.I, E = a.E;
  const int I2 = I / 2, I16 = I / 16, IC = I / 32;
  const int lane = threadIdx.x & 63, q = lane >> 4, cc = lane & 15;
  const int nb = (H + NRB - 1) / NRB;
  const int total = meta[0] * nb;
  const int64_t cstr = int64_t(H) * I2, bstr = int64_t(H) * I16;
  const uint8_t* wdp = static_cast<const uint8_t*>(a.wd);
  const uint8_t* shd = static_cast<const uint8_t*>(a.shd);
  for (int item = blockIdx.x * 4 + (threadIdx.x >> 6); item < total; item += gridDim.x * 4) {
    const int u = item / nb, n0 = (item - u * nb) * NRB;
    const int e = active[u];
    float wf[RG][NSD][32];
    {
      const uint8_t* cp = nv_expert(wdp, shd, e, E, cstr);
      const uint8_t* bp = nv_expert(a.bd, a.shbd, e, E, bstr);
      uint4 wc[RG][NSD];
      uint32_t ws2[RG][NSD];
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        const int n = n0 + 4 * g + q;
#pragma unroll
        for (int s = 0; s < NSD; ++s) {
          const int c = cc + 16 * s;
          wc[g][s] = make_uint4(0u, 0u, 0u, 0u);
          ws2[g][s] = 0u;
          if (n < H && c < IC) {
            wc[g][s] = *reinterpret_cast<const uint4*>(cp + int64_t(n) * I2 + c * 16);
            ws2[g][s] = *reinterpret_cast<const uint16_t*>(bp + int64_t(n) * I16 + c * 2);
          }
        }
      }
#pragma unroll
      for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int s = 0; s < NSD; ++s) {
          float s0, s1;
          e4m3_pair(ws2[g][s], s0, s1);
          const uint32_t w[4] = {wc[g][s].x, wc[g][s].y, wc[g][s].z, wc[g][s].w};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float sc = i < 2 ? s0 : s1;
            const auto p0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 0);
            const auto p1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 1);
            const auto p2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 2);
            const auto p3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[i], 1.0f, 3);
            wf[g][s][8 * i + 0] = p0[0] * sc; wf[g][s][8 * i + 1] = p0[1] * sc;
            wf[g][s][8 * i + 2] = p1[0] * sc; wf[g][s][8 * i + 3] = p1[1] * sc;
            wf[g][s][8 * i + 4] = p2[0] * sc; wf[g][s][8 * i + 5] = p2[1] * sc;
            wf[g][s][8 * i + 6] = p3[0] * sc; wf[g][s][8 * i + 7] = p3[1] * sc;
          }
        }
    }
    const float gd = e < E ? a.gd[e] : a.shgd[e - E];
    const int r0 = a.offsets[e], r1 = a.offsets[e + 1];
    auto loadh = [&](int r, float4 (&hv)[NSD][8]) {
#pragma unroll
      for (int s = 0; s < NSD; ++s) {
        const int c = cc + 16 * s;
        if (c < IC) {
          const float4* hp = reinterpret_cast<const float4*>(a.h + int64_t(r) * I + c * 32);
#pragma unroll
          for (int v = 0; v < 8; ++v) hv[s][v] = hp[v];
        }
      }
    };
    auto dot = [&](int r, const float4 (&hv)[NSD][8]) {
#pragma unroll
      for (int g = 0; g < RG; ++g) {
        float d0 = 0.f, d1 = 0.f;
#pragma unroll
        for (int s = 0; s < NSD; ++s) {
          if (cc + 16 * s < IC) {
#pragma unroll
            for (int v = 0; v < 8; ++v) {
              d0 = fmaf(wf[g][s][4 * v + 0], hv[s][v].x, d0);
              d1 = fmaf(wf[g][s][4 * v + 1], hv[s][v].y, d1);
              d0 = fmaf(wf[g][s][4 * v + 2], hv[s][v].z, d0);
              d1 = fmaf(wf[g][s][4 * v + 3], hv[s][v].w, d1);
            }
          }
        }
        const float d = row_sum(d0 + d1) * gd;
        const int n = n0 + 4 * g + q;
        if (cc == 0 && n < H) y_perm[int64_t(r) * H + n] = d;
      }
    };
    float4 ha[NSD][8], hb[NSD][8];
    if (r0 < r1) loadh(r0, ha);
    for (int r = r0; r < r1; r += 2) {
      if (r + 1 < r1) loadh(r + 1, hb);
      dot(r, ha);
      if (r + 1 >= r1) break;
      if (r + 2 < r1) loadh(r + 2, ha);
      dot(r + 1, hb);
    }
  }
}

// ---------------------------------------------------------------------------
static size_t decode_lds(const Plan& p) {
  const size_t tsize = p.act == MOE_F32 ? 4 : 2;
  // after the token rows, the tables and the slot masks: the prefetch scratch (1 KB per
  // wave) or, for MXFP4 experts, the E8M0 codes of the token rows; 16-byte aligned
  const size_t tail = p.wt == MOE_MXFP4 ? size_t(p.T) * (p.H / 32) + 16
                                        : MOE_DEC_PF > 0 ? 4096 + 16 : 0;
  return ((size_t(p.T) * p.H * tsize + 15) & ~size_t(15)) +
         size_t(2 * (p.E + p.S) + 1 + p.R + 3 * p.T * p.k + 1) * 4 + size_t(4) * p.E * 8 + 8 + tail;
}

bool decode_ffn_ok(const Plan& p) {
  return p.skinny && p.T <= 16 && p.T * p.k <= 256 && p.S <= 32 && p.H <= 2048 && p.I <= 1024 &&
         p.I % 2 == 0 && decode_lds(p) <= size_t(64) * 1024;
}

// Blocks of a persistent launch: every CU gets as many as fit, at most `cap`.
static int persistent_blocks(const void* kern, size_t lds, int* blocks, int cap = 2) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, 256, lds) != hipSuccess) {
    check_launch();
    return MOE_ERR_HIP;
  }
  *blocks = cus * std::max(1, std::min(per_cu, cap));
  return MOE_OK;
}

template <typename TA, typename TW, int NS, int NSD, int Q>
static int launch_decode_t(const Plan& p, const DecodeArgs& a, hipStream_t st) {
  const auto k1 = k_decode_gateup<TA, TW, NS, Q>;
  const auto k2 = k_decode_down<TA, TW, NSD>;
  const size_t lds = decode_lds(p);
  int b1 = 0, b2 = 0;
  MOE_TRY(persistent_blocks(reinterpret_cast<const void*>(k1), lds, &b1));
  // down: items of two output columns (T*H/2 of them, 3072 for 4 tokens) over three
  // blocks per CU put more weight rows in flight at once than items of four over two
  // (measured on the 4-token Ling layer: 11.5 -> 10.6 us)
  MOE_TRY(persistent_blocks(reinterpret_cast<const void*>(k2), 0, &b2, 3));
  launch_kernel(p, kTimeGateUp, k1, dim3(b1), dim3(256), lds, st, a);
  MOE_TRY(check_launch());
  launch_kernel(p, kTimeDown, k2, dim3(b2), dim3(256), 0, st, a);
  return check_launch();
}

template <typename TW, int NS, int NSD, int Q>
static int launch_decode_nv_t(const Plan& p, const DecodeArgs& a, hipStream_t st) {
  constexpr bool MX = std::is_same<TW, mxfp4_t>::value;
  const auto k1 = k_decode_gateup<bf16_t, TW, NS, Q>;
  const size_t lds = decode_lds(p);
  int b1 = 0, b2 = 0;
  // the 4-bit items end in conversion-heavy arithmetic once their data has arrived, so
  // a third resident block per CU (its VGPRs allow three waves per SIMD) keeps SIMDs
  // busy while other waves still wait for weights (measured: 17.2 -> 15.9 us per step)
  MOE_TRY(persistent_blocks(reinterpret_cast<const void*>(k1), lds, &b1, 3));
  // columns per down item: as many as keep at least 256 items in flight
  const int64_t T = p.T;
  auto items = [&](int rg) { return T * ((p.H + 4 * rg - 1) / (4 * rg)); };
  const int rg = items(4) >= 256 ? 4 : items(2) >= 256 ? 2 : 1;
  constexpr int SP = NSD == 1 ? 2 : 1;
  launch_kernel(p, kTimeGateUp, k1, dim3(b1), dim3(256), lds, st, a);
  MOE_TRY(check_launch());
  if (rg == 4) {
    const auto k2 = k_decode_down_nv<NSD, 4, SP, MX>;
    MOE_TRY(persistent_blocks(reinterpret_cast<const void*>(k2), 0, &b2));
    launch_kernel(p, kTimeDown, k2, dim3(int(std::min<int64_t>(b2, items(4)))), dim3(256), 0, st, a);
  } else if (rg == 2) {
    const auto k2 = k_decode_down_nv<NSD, 2, SP, MX>;
    MOE_TRY(persistent_blocks(reinterpret_cast<const void*>(k2), 0, &b2));
    launch_kernel(p, kTimeDown, k2, dim3(int(std::min<int64_t>(b2, items(2)))), dim3(256), 0, st, a);
  } else {
    const auto k2 = k_decode_down_nv<NSD, 1, SP, MX>;
    MOE_TRY(persistent_blocks(reinterpret_cast<const void*>(k2), 0, &b2));
    launch_kernel(p, kTimeDown, k2, dim3(int(std::min<int64_t>(b2, items(1)))), dim3(256), 0, st, a);
  }
  return check_launch();
}

static DecodeArgs nv_batch_args(const Plan& p, const void* x, const int32_t* row_token,
                                const int32_t* offsets, const moe_weights* w, float* h) {
  DecodeArgs a{};
  a.x = x;
  a.wg = w->w_gate; a.wu = w->w_up; a.wd = w->w_down;
  a.shg = w->sh_gate; a.shu = w->sh_up; a.shd = w->sh_down;
  a.bg = w->b_gate; a.bu = w->b_up; a.bd = w->b_down;
  a.shbg = w->sh_b_gate; a.shbu = w->sh_b_up; a.shbd = w->sh_b_down;
  a.gg = w->g_gate; a.gu = w->g_up; a.gd = w->g_down;
  a.shgg = w->sh_g_gate; a.shgu = w->sh_g_up; a.shgd = w->sh_g_down;
  a.offsets = const_cast<int32_t*>(offsets);
  a.row_token = const_cast<int32_t*>(row_token);
  a.h = h;
  a.T = int(std::min<int64_t>(p.T, INT32_MAX)); a.H = p.H; a.I = p.I; a.E = p.E; a.S = p.S;
  return a;
}

int launch_nv_gateup_batch(const Plan& p, const void* x, const int32_t* row_token,
                           const int32_t* offsets, const int32_t* active, const int32_t* meta,
                           const moe_weights* w, float* h, hipStream_t st) {
  const DecodeArgs a = nv_batch_args(p, x, row_token, offsets, w, h);
  const int ns = (p.H + 511) / 512;
  const int64_t items = p.max_active * (p.I / 4);
  auto go = [&](auto kern) {
    int b = 0;
    MOE_TRY(persistent_blocks(reinterpret_cast<const void*>(kern), 0, &b));
    const int grid = int(std::max<int64_t>(1, std::min<int64_t>(b, (items + 3) / 4)));
    launch_kernel(p, kTimeGateUp, kern, dim3(grid), dim3(256), 0, st, a, active, meta);
    return check_launch();
  };
  if (ns <= 1) return go(k_nv_gateup_batch<1>);
  if (ns == 2) return go(k_nv_gateup_batch<2>);
  if (ns == 3) return go(k_nv_gateup_batch<3>);
  return go(k_nv_gateup_batch<4>);
}

int launch_nv_down_batch(const Plan& p, const float* h, const int32_t* offsets,
                         const int32_t* active, const int32_t* meta, const moe_weights* w,
                         float* y_perm, hipStream_t st) {
  const DecodeArgs a = nv_batch_args(p, nullptr, nullptr, offsets, w, const_cast<float*>(h));
  auto go = [&](auto kern, int rg) {
    int b = 0;
    MOE_TRY(persistent_blocks(reinterpret_cast<const void*>(kern), 0, &b));
    const int64_t items = p.max_active * ((p.H + 4 * rg - 1) / (4 * rg));
    const int grid = int(std::max<int64_t>(1, std::min<int64_t>(b, (items + 3) / 4)));
    launch_kernel(p, kTimeDown, kern, dim3(grid), dim3(256), 0, st, a, active, meta, y_perm);
    return check_launch();
  };
  if (p.I <= 512) return go(k_nv_down_batch<1, 2>, 2);
  return go(k_nv_down_batch<2, 1>, 1);
}

int launch_decode_ffn(const Plan& p, const void* x, const float* logits, const moe_weights* w,
                      int32_t* ids, float* wts, int32_t* offsets, int32_t* row_token,
                      int32_t* inv, float* h, const void* res, void* y, uint8_t* xq,
                      uint8_t* sxq, hipStream_t st) {
  DecodeArgs a{};
  a.xq = xq; a.sxq = sxq;
  a.x = x; a.logits = logits;
  a.wg = w->w_gate; a.wu = w->w_up; a.wd = w->w_down;
  a.shg = w->sh_gate; a.shu = w->sh_up; a.shd = w->sh_down;
  a.ids = ids; a.w = wts; a.offsets = offsets; a.row_token = row_token; a.inv = inv;
  a.bg = w->b_gate; a.bu = w->b_up; a.bd = w->b_down;
  a.shbg = w->sh_b_gate; a.shbu = w->sh_b_up; a.shbd = w->sh_b_down;
  a.gg = w->g_gate; a.gu = w->g_up; a.gd = w->g_down;
  a.shgg = w->sh_g_gate; a.shgu = w->sh_g_up; a.shgd = w->sh_g_down;
  a.h = h; a.y = y; a.res = res;
  a.T = int(p.T); a.H = p.H; a.I = p.I; a.E = p.E; a.S = p.S; a.G = p.G; a.Gk = p.Gk; a.k = p.k;
  const int ns = (p.H + 511) / 512, nsd = (p.I + 511) / 512;
  const bool rows = select_rows_ok(p);
  // 4-bit experts (NVFP4 or MXFP4): bf16 activations, their own item loops
#define MOE_NQ(TW, NSV, NSDV)                                                    \
  {                                                                              \
    if (rows) {                                                                  \
      if (p.E == 128) return launch_decode_nv_t<TW, NSV, NSDV, -8>(p, a, st);    \
      if (p.E == 256) return launch_decode_nv_t<TW, NSV, NSDV, -16>(p, a, st);   \
      if (p.E == 64) return launch_decode_nv_t<TW, NSV, NSDV, -4>(p, a, st);     \
      if (p.E == 16) return launch_decode_nv_t<TW, NSV, NSDV, -1>(p, a, st);     \
    }                                                                            \
    if (p.E <= 64) return launch_decode_nv_t<TW, NSV, NSDV, 1>(p, a, st);        \
    if (p.E <= 128) return launch_decode_nv_t<TW, NSV, NSDV, 2>(p, a, st);       \
    if (p.E <= 256) return launch_decode_nv_t<TW, NSV, NSDV, 4>(p, a, st);       \
    if (p.E <= 512) return launch_decode_nv_t<TW, NSV, NSDV, 8>(p, a, st);       \
    return launch_decode_nv_t<TW, NSV, NSDV, 16>(p, a, st);                      \
  }
#define MOE_NNS(TW, NSDV)                 \
  {                                       \
    if (ns <= 1) MOE_NQ(TW, 1, NSDV)      \
    if (ns == 2) MOE_NQ(TW, 2, NSDV)      \
    if (ns == 3) MOE_NQ(TW, 3, NSDV)      \
    MOE_NQ(TW, 4, NSDV)                   \
  }
  if (p.wt == MOE_NVFP4) {
    if (nsd <= 1) MOE_NNS(nvfp4_t, 1)
    MOE_NNS(nvfp4_t, 2)
  }
  if (p.wt == MOE_MXFP4) {
    if (nsd <= 1) MOE_NNS(mxfp4_t, 1)
    MOE_NNS(mxfp4_t, 2)
  }
#undef MOE_NNS
#undef MOE_NQ
#define MOE_DQ(TA, TW, NSV, NSDV)                                            \
  {                                                                          \
    if (rows) {                                                              \
      if (p.E == 128) return launch_decode_t<TA, TW, NSV, NSDV, -8>(p, a, st);  \
      if (p.E == 256) return launch_decode_t<TA, TW, NSV, NSDV, -16>(p, a, st); \
      if (p.E == 64) return launch_decode_t<TA, TW, NSV, NSDV, -4>(p, a, st);   \
      if (p.E == 16) return launch_decode_t<TA, TW, NSV, NSDV, -1>(p, a, st);   \
    }                                                                        \
    if (p.E <= 64) return launch_decode_t<TA, TW, NSV, NSDV, 1>(p, a, st);   \
    if (p.E <= 128) return launch_decode_t<TA, TW, NSV, NSDV, 2>(p, a, st);  \
    if (p.E <= 256) return launch_decode_t<TA, TW, NSV, NSDV, 4>(p, a, st);  \
    if (p.E <= 512) return launch_decode_t<TA, TW, NSV, NSDV, 8>(p, a, st);  \
    return launch_decode_t<TA, TW, NSV, NSDV, 16>(p, a, st);                 \
  }
#define MOE_DNS(TA, TW, NSDV)                  \
  {                                            \
    if (ns <= 1) MOE_DQ(TA, TW, 1, NSDV)       \
    if (ns == 2) MOE_DQ(TA, TW, 2, NSDV)       \
    if (ns == 3) MOE_DQ(TA, TW, 3, NSDV)       \
    MOE_DQ(TA, TW, 4, NSDV)                    \
  }
  if (p.wt == MOE_F32) {
    if (nsd <= 1) MOE_DNS(float, float, 1)
    MOE_DNS(float, float, 2)
  }
  if (nsd <= 1) MOE_DNS(bf16_t, bf16_t, 1)
  MOE_DNS(bf16_t, bf16_t, 2)
#undef MOE_DNS
#undef MOE_DQ
}

}  // namespace moe
