// Device helpers shared by the MoE kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// Workgroup barrier that also keeps the compiler from moving memory operations
// across it (s_barrier alone is not a memory barrier to the compiler); it adds no
// wait of its own, the explicit waitcnt before it decides what has landed.
__device__ __forceinline__ void block_sync_nowait() {
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Direct global -> LDS load of 16 bytes per lane (global_load_lds_dwordx4): the
// wave's 64 lanes write 1 KB at `lds` (wave-uniform), lane L at lds + 16 L.
typedef __attribute__((address_space(3))) void lvoid_t;
// The load is written in asm so that the compiler does not add its own
// conservative vmcnt(0) before every later LDS read; completion is tracked by
// the explicit waits below (VMEM loads complete in issue order).  The address
// and M0 are consumed when the load issues; M0 is saved and restored around it
// and the only register output is that saved scalar copy.
__device__ __forceinline__ void dma16(const void* g, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>((lvoid_t*)lds)));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(g)
      : "memory");
}
// The same for 4 bytes per lane (global_load_lds_dword): lane L writes lds + 4 L.
__device__ __forceinline__ void dma4(const void* g, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>((lvoid_t*)lds)));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dword %2, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(g)
      : "memory");
}
// s_waitcnt vmcnt(N) lgkmcnt(0) (gfx9 encoding: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4]<<14)
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));
}

#ifndef MOE_SWZ_SHIFT
#define MOE_SWZ_SHIFT 1
#endif
// Matrix tiles in LDS are 128-byte rows of eight 16-byte chunks.  swz16 gives the
// LDS position (in 16-byte units) of chunk `chunk` of row `row`: chunks are XOR-
// swizzled by (row >> 1) & 7, so that 16 consecutive rows read at the same chunk
// (what one ds_read_b128 serves together) land on 16 distinct 16-byte slots of the
// 256-byte bank line.
__device__ __forceinline__ int swz16(int row, int chunk) {
  return row * 8 + (chunk ^ ((row >> MOE_SWZ_SHIFT) & 7));
}
// A wave's direct-to-LDS load of 64 x 16 bytes fills rows 8j .. 8j+7 in LDS order
// (lane L writes position L % 8 of row 8j + L / 8): the logical chunk lane L must
// fetch so that the tile ends up swizzled as swz16 reads it.
__device__ __forceinline__ int dma_chunk(int lane, int j) {
  return (lane & 7) ^ (((8 * j + (lane >> 3)) >> MOE_SWZ_SHIFT) & 7);
}

constexpr int kWave = 64;

typedef uint16_t bf16_t;  // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

// ----------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(bf16_t v) { return __uint_as_float(uint32_t(v) << 16); }

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
// fp32 -> bf16, round to nearest even: the conversion gfx950 does in one instruction
// (v_cvt_pk_bf16_f32; the same rounding as adding 0x7FFF plus the kept lsb to the
// fp32 bits for every finite value, and NaN stays NaN)
__device__ __forceinline__ bf16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

template <typename T> __device__ __forceinline__ float to_f32(T v);
template <> __device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v); }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16_t from_f32<bf16_t>(float v) { return f32_to_bf16(v); }

// Eight consecutive elements -> fp32 (one 16-byte load for bf16, two for fp32).
__device__ __forceinline__ void load8(const bf16_t* p, float (&o)[8]) {
  uint4 v = *reinterpret_cast<const uint4*>(p);
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ void load8(const float* p, float (&o)[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
  o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
}

// Eight weights as they sit in memory (16 bytes of bf16 or 32 bytes of fp32).
template <typename TW> struct Chunk8;
template <> struct Chunk8<bf16_t> {
  uint4 v;
  __device__ __forceinline__ void load(const bf16_t* p) { v = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ void store(bf16_t* p) const { *reinterpret_cast<uint4*>(p) = v; }
  // element i = round(a[i] * r * g[i]) (fp32 products, then round to nearest even)
  __device__ __forceinline__ void set(const float (&a)[8], float r, const float (&g)[8]) {
    uint32_t w[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      w[i] = uint32_t(f32_to_bf16(a[2 * i] * r * g[2 * i])) |
             (uint32_t(f32_to_bf16(a[2 * i + 1] * r * g[2 * i + 1])) << 16);
    v = make_uint4(w[0], w[1], w[2], w[3]);
  }
  __device__ __forceinline__ void get(float (&o)[8]) const {
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      o[2 * i] = __uint_as_float(w[i] << 16);
      o[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
  }
};
template <> struct Chunk8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ void store(float* p) const {
    *reinterpret_cast<float4*>(p) = a;
    *reinterpret_cast<float4*>(p + 4) = b;
  }
  __device__ __forceinline__ void set(const float (&x)[8], float r, const float (&g)[8]) {
    a = make_float4(x[0] * r * g[0], x[1] * r * g[1], x[2] * r * g[2], x[3] * r * g[3]);
    b = make_float4(x[4] * r * g[4], x[5] * r * g[5], x[6] * r * g[6], x[7] * r * g[7]);
  }
  __device__ __forceinline__ void get(float (&o)[8]) const {
    o[0] = a.x; o[1] = a.y; o[2] = a.z; o[3] = a.w;
    o[4] = b.x; o[5] = b.y; o[6] = b.z; o[7] = b.w;
  }
};

__device__ __forceinline__ float dot8(const float (&a)[8], const float (&b)[8], float acc) {
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = fmaf(a[i], b[i], acc);
  return acc;
}

// OCP e4m3 (bias 7, 3 mantissa bits, max 448, no infinities), round to nearest
// even, saturating.  Built from the format definition: normals are
// (8 + m) * 2^(e-10) for e = 1..15 (code e<<3 | m), subnormals m * 2^-9.
__device__ __forceinline__ uint32_t f32_to_e4m3_formula(float v) {
  uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                       // below 2^-6: subnormal grid of 2^-9
    code = uint32_t(rintf(a * 512.0f));      // 0..8 (8 is the smallest normal, code 0x08)
  } else {
    int ex = int((__float_as_uint(a) >> 23) & 0xFF) - 127;   // -6..8
    float m = rintf(ldexpf(a, 3 - ex));      // 8..16, exact scaling, RNE
    if (m >= 16.0f) { m = 8.0f; ++ex; }
    code = (uint32_t(ex + 7) << 3) | (uint32_t(m) - 8u);
    if (code > 0x7Eu) code = 0x7Eu;
  }
  return sign | code;
}
// Four values -> four codes (byte i = value i) with the gfx950 packed conversion, which
// rounds to nearest even; the values are clamped to +-448 first so that it saturates
// like the formula above.  The two agree on every non-NaN fp32 input: compared
// exhaustively on the device, all 2^32 bit patterns but NaN, with no difference.
__device__ __forceinline__ uint32_t e4m3x4(float a, float b, float c, float d) {
  auto cl = [](float v) { return fminf(fmaxf(v, -448.0f), 448.0f); };
  const int lo = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), lo, true));
}

// MXFP8 activations (OCP Microscaling, E4M3 elements): the E8M0 shared exponent X of
// a block whose largest magnitude is m (finite, >= 0; all-zero and subnormal blocks
// give the clamp -127), and the power of two 2^-X that maps the block onto the E4M3
// grid (exact multiplication; X <= 119 for finite m, so the result is a normal float).
__device__ __forceinline__ int mx_exponent(float m) {
  const int e = int((__float_as_uint(m) >> 23) & 0xFF) - 127 - 8;   // floor(log2 m) - 8
  return min(max(e, -127), 127);
}
__device__ __forceinline__ float mx_inv_scale(int X) { return __uint_as_float(uint32_t(127 - X) << 23); }

// ----------------------------------------------------------------- wave reductions
// DPP steps inside each row of 16 lanes (quad swaps, half-row and row mirrors),
// then the four row results combined through readlane in a fixed order, so the
// result is the same in every lane and bitwise reproducible.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
  return uint32_t(__builtin_amdgcn_update_dpp(int(v), int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ float dppf(float v) { return __uint_as_float(dpp32<CTRL>(__float_as_uint(v))); }
__device__ __forceinline__ float lanef(float v, int l) {
  return __uint_as_float(uint32_t(__builtin_amdgcn_readlane(int(__float_as_uint(v)), l)));
}

__device__ __forceinline__ float wave_sum(float v) {
  v += dppf<0xB1>(v);    // quad_perm [1,0,3,2]
  v += dppf<0x4E>(v);    // quad_perm [2,3,0,1]
  v += dppf<0x141>(v);   // row_half_mirror
  v += dppf<0x140>(v);   // row_mirror
  return (lanef(v, 0) + lanef(v, 16)) + (lanef(v, 32) + lanef(v, 48));
}
__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dppf<0xB1>(v));
  v = fmaxf(v, dppf<0x4E>(v));
  v = fmaxf(v, dppf<0x141>(v));
  v = fmaxf(v, dppf<0x140>(v));
  return fmaxf(fmaxf(lanef(v, 0), lanef(v, 16)), fmaxf(lanef(v, 32), lanef(v, 48)));
}

// ------------------------------------------------------- activation quantisation
// Shared by the standalone quantisation kernels and the routing launch that carries the
// quantisation of x in extra workgroups.
//
// Block-FP8: per row and 128-wide block, scale = amax / 448 (1 for an all-zero block)
// and codes = e4m3(v / scale), rounded to nearest even and saturated.  One block per
// DPP row of 16 lanes (8 consecutive values per lane, one 16-byte load), four blocks
// per wave; `wave` numbers the waves over the launch.  Blocks past the end load a
// clamped block and store nothing.
template <typename TI>
__device__ __forceinline__ void quant_e4m3_wave(const TI* __restrict__ in, int64_t rows, int K,
                                                uint8_t* __restrict__ codes,
                                                float* __restrict__ scales, int64_t wave) {
  const int lane = threadIdx.x & 63, r16 = lane & 15;
  const int nkb = K / 128;
  const int64_t nblk = rows * nkb;
  const int64_t idx = wave * 4 + (lane >> 4);
  const bool live = idx < nblk;
  const int64_t id = live ? idx : nblk - 1;
  const int64_t row = id / nkb;
  const int kb = int(id - row * nkb);
  const int64_t off = row * K + kb * 128 + r16 * 8;
  float v[8];
  load8(in + off, v);
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, dppf<0xB1>(m));    // quad_perm [1,0,3,2]
  m = fmaxf(m, dppf<0x4E>(m));    // quad_perm [2,3,0,1]
  m = fmaxf(m, dppf<0x141>(m));   // row_half_mirror
  m = fmaxf(m, dppf<0x140>(m));   // row_mirror
  const float scale = m > 0.f ? m / 448.0f : 1.0f;
  const uint32_t c[2] = {e4m3x4(v[0] / scale, v[1] / scale, v[2] / scale, v[3] / scale),
                         e4m3x4(v[4] / scale, v[5] / scale, v[6] / scale, v[7] / scale)};
  if (live) {
    *reinterpret_cast<uint2*>(codes + off) = make_uint2(c[0], c[1]);
    if (r16 == 0) scales[row * nkb + kb] = scale;
  }
}

// MXFP8: per row and 32-wide block, X = floor(log2(amax)) - 8 (clamped to the E8M0
// range; -127 for an all-zero block), codes = e4m3(v * 2^-X), rounded to nearest even
// and saturated.  Eight values per lane (one 16-byte load), a block per four lanes;
// `idx` numbers the lanes over the launch (a multiple of 4 starts each block).
// Positions past the end load a clamped group and store nothing.
__device__ __forceinline__ void quant_mx_lane(const bf16_t* __restrict__ in, int64_t rows, int K,
                                              uint8_t* __restrict__ codes,
                                              uint8_t* __restrict__ scales, int64_t idx) {
  const int64_t n8 = rows * (K / 8);
  const bool live = idx < n8;
  const int64_t off = (live ? idx : n8 - 1) * 8;
  float v[8];
  load8(in + off, v);
  float m = 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) m = fmaxf(m, fabsf(v[i]));
  m = fmaxf(m, dppf<0xB1>(m));    // quad_perm [1,0,3,2]
  m = fmaxf(m, dppf<0x4E>(m));    // quad_perm [2,3,0,1]
  const int X = mx_exponent(m);
  const float inv = mx_inv_scale(X);
  const uint32_t c0 = e4m3x4(v[0] * inv, v[1] * inv, v[2] * inv, v[3] * inv);
  const uint32_t c1 = e4m3x4(v[4] * inv, v[5] * inv, v[6] * inv, v[7] * inv);
  if (live) {
    *reinterpret_cast<uint2*>(codes + off) = make_uint2(c0, c1);
    if ((idx & 3) == 0) scales[off / 32] = uint8_t(X + 127);
  }
}

// DPP move whose disabled-lane value is left undefined (every pattern used here reads
// an enabled lane), so it compiles to one v_mov_b32_dpp without a copy of the source
template <int CTRL>
__device__ __forceinline__ uint32_t dpp32_mov(uint32_t v) {
  return uint32_t(__builtin_amdgcn_mov_dpp(int(v), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
  const uint32_t lo = dpp32_mov<CTRL>(uint32_t(v)), hi = dpp32_mov<CTRL>(uint32_t(v >> 32));
  const uint64_t w = (uint64_t(hi) << 32) | lo;
  return w > v ? w : v;
}
__device__ __forceinline__ uint64_t lane_u64(uint64_t v, int l) {
  const uint32_t lo = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v)), l));
  const uint32_t hi = uint32_t(__builtin_amdgcn_readlane(int(uint32_t(v >> 32)), l));
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_u64<0xB1>(v);
  v = dpp_max_u64<0x4E>(v);
  v = dpp_max_u64<0x141>(v);
  v = dpp_max_u64<0x140>(v);
  uint64_t a = lane_u64(v, 0), b = lane_u64(v, 16), c = lane_u64(v, 32), d = lane_u64(v, 48);
  a = a > b ? a : b;
  c = c > d ? c : d;
  return a > c ? a : c;
}

// Exclusive scan over a block of 256 threads; `tmp` holds >= 4 ints.  All threads call it.
__device__ __forceinline__ int block_exclusive_scan_256(int v, int* tmp, int& total) {
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  if (lane == 63) tmp[wv] = x;
  __syncthreads();
  int base = 0;
  for (int i = 0; i < wv; ++i) base += tmp[i];
  total = tmp[0] + tmp[1] + tmp[2] + tmp[3];
  __syncthreads();
  return base + x - v;
}

// Total order key for (score desc, index asc) arg-max: larger key wins.
// Scores are finite fp32; -0 is folded onto +0 so that the two compare equal.
__device__ __forceinline__ uint64_t rank_key(float s, int idx) {
  uint32_t u = __float_as_uint(s + 0.0f);
  u = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (uint64_t(u) << 32) | uint32_t(0xFFFFFFFFu - uint32_t(idx));
}
__device__ __forceinline__ int key_index(uint64_t k) { return int(0xFFFFFFFFu - uint32_t(k)); }


// Two OCP e4m3 codes (low byte first) -> two floats (the gfx950 packed conversion
// with a unit scale decodes all 256 codes exactly, subnormals included).
__device__ __forceinline__ void e4m3_pair(uint32_t two, float& s0, float& s1) {
  const auto f = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(two, 1.0f, false);
  s0 = f[0];
  s1 = f[1];
}

__device__ __forceinline__ float silu(float g) { return g / (1.0f + __expf(-g)); }
// SiLU with the hardware reciprocal (within about 1 ulp of the correctly rounded
// quotient) for outputs that are rounded to bf16 or e4m3 right after: the expert
// GEMM epilogues, where the division sequence was a large share of the epilogue's
// arithmetic.  The fp32 h of the decode and skinny kernels keeps the exact division.
__device__ __forceinline__ float silu_lp(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

}  // namespace moe
