// Grouped SwiGLU expert GEMMs on CDNA4 matrix cores (bf16, block-FP8, NVFP4).
//
// According to TensorFold issue #1247 "Ling-3.0-tiny on a Qualcomm board"
// (jschmied's comment, list "What it does not cover"), the bf16 expert path there
// lacks a grouped kernel, which a port should supply; the same list names block
// FP8 among the expert formats it reads.  These kernels are that grouped
// kernel: one launch covers every expert, each workgroup reads its (expert, row
// offset) from the device tile table the permutation built, so the host never
// learns the per-expert row counts.  Workgroups beyond the live tile count exit.
//
// The pipelined kernels (k_gemm_bf16_v2, k_gemm_nv4, k_gemm_fp8_v2) take 128-row
// tiles of 256 weight rows per workgroup of 8 waves, K moving global -> LDS by
// direct-to-LDS loads through a three-slot ring, the 16-byte chunks of each tile row
// XOR-swizzled so that a ds_read_b128 of 16 lanes hits distinct banks; work items
// are laid out XCD by XCD so the workgroups sharing weight slabs share an L2.  The
// register-staged kernels (k_gemm_bf16, k_gemm_fp8: 128 x 128 tiles of 4 waves,
// double-buffered) cover the shapes the pipelined tiles do not divide.  The gate/up
// kernels gather activation rows through row_token while loading (the permuted
// activations are never materialised) and apply SwiGLU in registers: a wave holds
// gate columns and the matching up columns, so g and u of one (row, i) sit in the
// same lane and register.
#include "moe_internal.h"
#include "gemm_common.h"

namespace moe {

constexpr int TM = 128;   // rows per tile (the schedule's BM)
constexpr int TN = 128;   // output columns (or weight rows) per tile


// ===========================================================================
// bf16: BK = 64 bf16 per slab (128 bytes per row = 8 chunks).
struct GemmBf16Args {
  const bf16_t* a;            // gate/up: x [T, H] (gathered); down: h [R, I]
  const int32_t* row_token;   // gate/up only
  const int32_t* offsets;
  const int2* tiles;
  const int32_t* meta;
  const bf16_t* w0;           // gate/up: w_gate; down: w_down
  const bf16_t* w1;           // gate/up: w_up
  const bf16_t* sh0;
  const bf16_t* sh1;
  const float* row_w;         // down, weighted bf16 output
  bf16_t* out16;              // gate/up: h [R, I]; down: weighted y_perm [R, H]
  float* out32;               // down: unweighted y_perm [R, H]
  int K, N, E;                // K: reduction length; N: output width (I for h, H for y)
  int ES;                     // routed + shared experts (offsets holds ES + 1 entries)
};

template <bool GATEUP>
__global__ __launch_bounds__(256) void k_gemm_bf16(GemmBf16Args p) {
  constexpr int BK = 64;
  const int ncol = GATEUP ? p.N / 64 : p.N / TN;   // gate/up tile = 64 h columns
  int tile, ct;
  if (!xcd_item(p.meta[1], ncol, tile, ct)) return;
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int base = p.offsets[e];
  const int cnt = p.offsets[e + 1] - base;

  __shared__ uint4 As[2][TM * 8];
  __shared__ uint4 Bs[2][TN * 8];

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv >> 1, wn = wv & 1;
  const int kc = tid & 7;
  const int64_t K = p.K;

  const bf16_t* ag[4];
  const bf16_t* bg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = (tid >> 3) + 32 * i;
    const int m = min(m0 + rr, cnt - 1);
    if (GATEUP) {
      ag[i] = p.a + int64_t(p.row_token[base + m]) * K + kc * 8;
      const int c0 = ct * 64;
      const int64_t st = int64_t(p.N) * K;
      bg[i] = rr < 64 ? expert_mat(p.w0, p.sh0, e, p.E, st) + int64_t(c0 + rr) * K + kc * 8
                      : expert_mat(p.w1, p.sh1, e, p.E, st) + int64_t(c0 + rr - 64) * K + kc * 8;
    } else {
      ag[i] = p.a + int64_t(base + m) * K + kc * 8;
      bg[i] = expert_mat(p.w0, p.sh0, e, p.E, int64_t(p.N) * K) + int64_t(ct * TN + rr) * K + kc * 8;
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int mi = 0; mi < 2; ++mi)
#pragma unroll
    for (int ni = 0; ni < 2; ++ni)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[mi][ni][r] = 0.f;

  uint4 ra[4], rb[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ra[i] = *reinterpret_cast<const uint4*>(ag[i]);
    rb[i] = *reinterpret_cast<const uint4*>(bg[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = (tid >> 3) + 32 * i;
    As[0][swz16(rr, kc)] = ra[i];
    Bs[0][swz16(rr, kc)] = rb[i];
  }
  __syncthreads();

  const int nk = int(K / BK);
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) {
      const int64_t ko = int64_t(kt + 1) * BK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        ra[i] = *reinterpret_cast<const uint4*>(ag[i] + ko);
        rb[i] = *reinterpret_cast<const uint4*>(bg[i] + ko);
      }
    }
#pragma unroll
    for (int ks = 0; ks < BK / 16; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      bf16x8 af[2], bfr[2];
#pragma unroll
      for (int mi = 0; mi < 2; ++mi) {
        const int row = wm * 64 + mi * 32 + (lane & 31);
        uint4 v = As[cur][swz16(row, chunk)];
        af[mi] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int ni = 0; ni < 2; ++ni) {
        const int row = GATEUP ? (ni * 64 + wn * 32 + (lane & 31)) : (wn * 64 + ni * 32 + (lane & 31));
        uint4 v = Bs[cur][swz16(row, chunk)];
        bfr[ni] = __builtin_bit_cast(bf16x8, v);
      }
#pragma unroll
      for (int mi = 0; mi < 2; ++mi)
#pragma unroll
        for (int ni = 0; ni < 2; ++ni)
          acc[mi][ni] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mi], bfr[ni], acc[mi][ni], 0, 0, 0);
    }
    if (kt + 1 < nk) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = (tid >> 3) + 32 * i;
        As[cur ^ 1][swz16(rr, kc)] = ra[i];
        Bs[cur ^ 1][swz16(rr, kc)] = rb[i];
      }
    }
    __syncthreads();
  }

  // epilogue
#pragma unroll
  for (int mi = 0; mi < 2; ++mi) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * 64 + mi * 32 + acc_row(r, lane);
      if (m0 + row >= cnt) continue;
      const int64_t grow = int64_t(base + m0 + row);
      if (GATEUP) {
        const int col = ct * 64 + wn * 32 + (lane & 31);
        const float g = acc[mi][0][r], u = acc[mi][1][r];
        p.out16[grow * p.N + col] = f32_to_bf16(silu_lp(g) * u);
      } else {
#pragma unroll
        for (int ni = 0; ni < 2; ++ni) {
          const int col = ct * TN + wn * 64 + ni * 32 + (lane & 31);
          if (p.out32)
            p.out32[grow * p.N + col] = acc[mi][ni][r];
          else
            p.out16[grow * p.N + col] = f32_to_bf16(acc[mi][ni][r] * p.row_w[grow]);
        }
      }
    }
  }
}

// ===========================================================================
// bf16, pipelined: 128 x 256 tiles, 4 waves (2 x 2) of 64 x 128, K slabs of 64
// moved global -> LDS by direct-to-LDS loads (global_load_lds_dwordx4) in a
// 3-stage ring, so two slabs are in flight while one is multiplied.  Each wave
// load instruction fills 8 tile rows (1 KB); lane L lands in row L/8, 16-byte
// slot L%8 and fetches the logical chunk (L%8) ^ (L/8), which is the XOR swizzle
// the fragment reads undo.  Waits are explicit (vmcnt for the slab about to be
// read, lgkmcnt(0) so no fragment read is in flight when a slot is refilled)
// followed by a bare s_barrier.

// Tile configuration of the pipelined bf16 kernel: BM x BN outputs per workgroup
// of W = WM x WN waves, each owning (BM / WM) x (BN / WN) outputs as MI x NI
// blocks of 32 x 32; K moves in slabs of BK through a 3-stage LDS ring.  Tile rows
// in LDS are BK * 2 bytes = CH chunks of 16 bytes, XOR-swizzled by
// (row >> SH) & (CH - 1) so that the 16 rows one ds_read_b128 serves together at
// one chunk fall on 16 distinct 16-byte slots of the 256-byte bank line.  One
// wave-wide direct-to-LDS load writes 1 KB = RPD consecutive tile rows.
template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct BfTile {
  static constexpr int BM = BM_, BN = BN_, BK = BK_, WM = WM_, WN = WN_, W = WM * WN, NT = 64 * W;
  // waves per SIMD the register budget is sized for: two workgroups per CU when
  // a workgroup is 4 waves (its LDS ring is then kept under half the CU's LDS)
  static constexpr int WPE = W == 4 ? 2 : 2;
  static constexpr int MI = BM / WM / 32, NI = BN / WN / 32;
  static constexpr int CH = BK / 8, SH = CH == 8 ? 1 : 2, RPD = 64 / CH;
  static constexpr int AJ = BM / (RPD * W), BJ = BN / (RPD * W), L = AJ + BJ;  // loads per lane per slab
  static constexpr int A_U4 = BM * CH, STAGE_U4 = (BM + BN) * CH;
  static constexpr int RING_U4 = 3 * STAGE_U4;
  static constexpr int LSG = BN / 2 + 8, LSD = BN + 8;   // epilogue staging row strides (bf16)
  static constexpr int STG_U4 = BM * LSD * 2 / 16;
  static constexpr int SMEM_U4 = RING_U4 > STG_U4 ? RING_U4 : STG_U4;
  static_assert(BK == 32 || BK == 64, "slab depth");
  static_assert(AJ * RPD * W == BM && BJ * RPD * W == BN, "load tiling");
  static_assert(MI >= 1 && NI >= 2 && NI % 2 == 0, "wave tiling");
  __device__ static __forceinline__ int pos(int row, int chunk) {
    return row * CH + (chunk ^ ((row >> SH) & (CH - 1)));
  }
  // logical chunk lane `lane` fetches when its wave's load fills rows RPD*j ..
  __device__ static __forceinline__ int dma_chunk(int lane, int j) {
    return (lane % CH) ^ (((RPD * j + lane / CH) >> SH) & (CH - 1));
  }
};

#ifndef MOE_BF_BM
#define MOE_BF_BM 128
#endif
#ifndef MOE_BF_BN
#define MOE_BF_BN 256
#endif
#ifndef MOE_BF_BK
#define MOE_BF_BK 64
#endif
#ifndef MOE_BF_WM
#define MOE_BF_WM 2
#endif
#ifndef MOE_BF_WN
#define MOE_BF_WN 4
#endif
using BfCfg = BfTile<MOE_BF_BM, MOE_BF_BN, MOE_BF_BK, MOE_BF_WM, MOE_BF_WN>;
// largest number of routed + shared experts a layer may have (the persistent bf16 down
// kernel keeps the expert row offsets in LDS)
#define MOE_MAX_ES 1024
#ifndef MOE_BF_GU_PERSIST
#define MOE_BF_GU_PERSIST 1
#endif
// the NVFP4 kernel's tile (its per-thread conversion layout is built for this shape)
using Nv4Cfg = BfTile<128, 256, 64, 2, 4>;

template <bool GATEUP, class C>
__global__ __launch_bounds__(C::NT) __attribute__((amdgpu_waves_per_eu(C::WPE)))
void k_gemm_bf16_v2(GemmBf16Args p) {
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, WM = C::WM, WN = C::WN, W = C::W;
  constexpr int MI = C::MI, NI = C::NI, CH = C::CH, RPD = C::RPD, AJ = C::AJ, BJ = C::BJ;
  constexpr int L = C::L, NT = C::NT;
  __shared__ uint4 smem[C::SMEM_U4];
  const int ncol = GATEUP ? p.N / (BN / 2) : p.N / BN;
  int tile, ct;
  if (!xcd_item(p.meta[1], ncol, tile, ct)) return;
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int base = p.offsets[e];
  const int cnt = p.offsets[e + 1] - base;

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / WN, wn = wv % WN;
  const int64_t K = p.K;

  const bf16_t* ag[AJ];
#pragma unroll
  for (int i = 0; i < AJ; ++i) {
    const int r = RPD * (wv + W * i) + lane / CH;
    const int m = min(m0 + r, cnt - 1);
    ag[i] = (GATEUP ? p.a + int64_t(p.row_token[base + m]) * K : p.a + int64_t(base + m) * K) +
            C::dma_chunk(lane, wv + W * i) * 8;
  }
  const bf16_t* bg[BJ];
  {
    const int64_t st = int64_t(p.N) * K;
#pragma unroll
    for (int i = 0; i < BJ; ++i) {
      const int r = RPD * (wv + W * i) + lane / CH;
      if (GATEUP) {
        const int c0 = ct * (BN / 2);
        bg[i] = (r < BN / 2 ? expert_mat(p.w0, p.sh0, e, p.E, st) + int64_t(c0 + r) * K
                            : expert_mat(p.w1, p.sh1, e, p.E, st) + int64_t(c0 + r - BN / 2) * K) +
                C::dma_chunk(lane, wv + W * i) * 8;
      } else {
        bg[i] = expert_mat(p.w0, p.sh0, e, p.E, st) + int64_t(ct * BN + r) * K +
                C::dma_chunk(lane, wv + W * i) * 8;
      }
    }
  }

  // slab kt into ring slot `slot`: A rows then B rows
  auto issue = [&](int kt, int slot) {
    const int64_t ko = int64_t(kt) * BK;
    uint4* sa = smem + slot * C::STAGE_U4;
    uint4* sb = sa + C::A_U4;
#pragma unroll
    for (int i = 0; i < AJ; ++i) dma16(ag[i] + ko, sa + (wv + W * i) * 64);
#pragma unroll
    for (int i = 0; i < BJ; ++i) dma16(bg[i] + ko, sb + (wv + W * i) * 64);
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int a = 0; a < MI; ++a)
#pragma unroll
    for (int b = 0; b < NI; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  // down, weighted output: this lane's row weights, loaded while the K loop runs
  float roww[GATEUP ? 1 : MI][GATEUP ? 1 : 16];
  if (!GATEUP) {
#pragma unroll
    for (int a = 0; a < (GATEUP ? 1 : MI); ++a)
#pragma unroll
      for (int r = 0; r < (GATEUP ? 1 : 16); ++r) {
        const int row = wm * (BM / WM) + a * 32 + acc_row(r, lane);
        roww[a][r] = (p.out32 || m0 + row >= cnt) ? 0.f : p.row_w[base + m0 + row];
      }
  }

  auto load_frags = [&](const uint4* sa, const uint4* sb, int ks, bf16x8 (&af)[MI], bf16x8 (&bfr)[NI]) {
    const int chunk = ks * 2 + (lane >> 5);
#pragma unroll
    for (int a = 0; a < MI; ++a)
      af[a] = __builtin_bit_cast(bf16x8, sa[C::pos(wm * (BM / WM) + a * 32 + (lane & 31), chunk)]);
#pragma unroll
    for (int b = 0; b < NI; ++b) {
      // gate/up: blocks 0..NI/2-1 are gate columns, NI/2.. the matching up columns
      const int row = GATEUP ? ((b < NI / 2 ? 0 : BN / 2) + wn * (BN / 2 / WN) + (b % (NI / 2)) * 32 + (lane & 31))
                             : (wn * (BN / WN) + b * 32 + (lane & 31));
      bfr[b] = __builtin_bit_cast(bf16x8, sb[C::pos(row, chunk)]);
    }
  };
  // multiply the slab in `slot`; fragments of sub-step ks+1 are read while the
  // MFMAs of ks run; `between` (the refill) is issued after the first reads
  auto compute = [&](int slot, auto&& between) {
    const uint4* sa = smem + slot * C::STAGE_U4;
    const uint4* sb = sa + C::A_U4;
    constexpr int KS = BK / 16;
    bf16x8 af[2][MI], bfr[2][NI];
    load_frags(sa, sb, 0, af[0], bfr[0]);
    __builtin_amdgcn_sched_barrier(0);
    between();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) load_frags(sa, sb, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < NI; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][a], bfr[ks & 1][b], acc[a][b], 0, 0, 0);
    }
  };

  const int nk = int(K / BK);
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  // step kt: wait for slab kt, barrier, refill the slot slab kt-1 used with kt+2, multiply kt
#define MOE_BF_STEP(KT, SLOT, NSLOT)                                      \
  {                                                                       \
    if ((KT) + 1 < nk) wait_vm_lgkm0<L>(); else wait_vm_lgkm0<0>();       \
    block_sync_nowait();                                                  \
    compute(SLOT, [&] { if ((KT) + 2 < nk) issue((KT) + 2, NSLOT); });    \
  }
  for (int kt = 0; kt < nk; kt += 3) {
    MOE_BF_STEP(kt, 0, 2)
    if (kt + 1 < nk) MOE_BF_STEP(kt + 1, 1, 0)
    if (kt + 2 < nk) MOE_BF_STEP(kt + 2, 2, 1)
  }
#undef MOE_BF_STEP

  // Epilogue.  bf16 outputs go through LDS (the ring is free: every slab has been
  // read and no load is in flight) so that each row leaves as whole 16-byte
  // pieces; the unweighted fp32 output is stored straight from the registers.
  if (GATEUP || !p.out32) {
    constexpr int OC = GATEUP ? BN / 2 : BN;   // output columns of the tile
    constexpr int LS = GATEUP ? C::LSG : C::LSD;
    bf16_t* stg = reinterpret_cast<bf16_t*>(smem);
    __syncthreads();
#pragma unroll
    for (int a = 0; a < MI; ++a) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * (BM / WM) + a * 32 + acc_row(r, lane);
        if (GATEUP) {
#pragma unroll
          for (int b = 0; b < NI / 2; ++b) {
            const float g = acc[a][b][r], u = acc[a][b + NI / 2][r];
            stg[row * LS + wn * (BN / 2 / WN) + b * 32 + (lane & 31)] = f32_to_bf16(silu_lp(g) * u);
          }
        } else {
          const float wr = roww[GATEUP ? 0 : a][GATEUP ? 0 : r];
#pragma unroll
          for (int b = 0; b < NI; ++b)
            stg[row * LS + wn * (BN / WN) + b * 32 + (lane & 31)] = f32_to_bf16(acc[a][b][r] * wr);
        }
      }
    }
    __syncthreads();
    constexpr int CPR = OC / 8;                // 16-byte pieces per row
    const int rows = min(BM, cnt - m0);
    const int col0 = ct * OC;
    for (int i = tid; i < rows * CPR; i += NT) {
      const int row = i / CPR, c = i - row * CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(stg + row * LS + c * 8);
      *reinterpret_cast<uint4*>(p.out16 + int64_t(base + m0 + row) * p.N + col0 + c * 8) = v;
    }
    return;
  }
#pragma unroll
  for (int a = 0; a < MI; ++a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * (BM / WM) + a * 32 + acc_row(r, lane);
      if (m0 + row >= cnt) continue;
      const int64_t grow = int64_t(base + m0 + row);
#pragma unroll
      for (int b = 0; b < NI; ++b)
        p.out32[grow * p.N + ct * BN + wn * (BN / WN) + b * 32 + (lane & 31)] = acc[a][b][r];
    }
  }
}

// ===========================================================================
// NVFP4 weights on the bf16 matrix cores (tile, waves and activation ring of the
// pipelined bf16 kernel).  The weight slab of a 64-deep K step arrives as E2M1 codes
// (32 bytes per weight row) and e4m3 block scales (4 per row) in registers: thread t
// owns half row t / 2 of the slab (32 codes, two scale blocks).  One step ahead, and
// interleaved with the current step's MFMAs, it writes them as bf16 into the tile's
// swizzled LDS layout: an E2M1 value times an e4m3 scale has at most 6 significant
// bits, so the bf16 is exact and is the high half of the fp32 product.  A three-slot
// ring of converted slabs keeps one barrier per step.  The per-expert matrix scales
// multiply the accumulators in the epilogue.
struct GemmNv4Args {
  const bf16_t* a;            // gate/up: x [T, H] (gathered); down: h [R, I]
  const int32_t* row_token;
  const int32_t* offsets;
  const int2* tiles;
  const int32_t* meta;
  const uint8_t *w0, *w1, *sh0, *sh1;   // packed codes (gate/up: gate, up; down: down)
  const uint8_t *b0, *b1, *shb0, *shb1; // e4m3 block scales
  const float *g0, *g1, *shg0, *shg1;   // fp32 matrix scales
  const float* row_w;
  bf16_t* out16;
  float* out32;
  int K, N, E;
};

__device__ __forceinline__ uint32_t bf16_pair_hi(float lo, float hi) {
  // one v_perm_b32: bytes 2, 3 of lo, then bytes 2, 3 of hi
  return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

template <bool GATEUP>
__global__ __launch_bounds__(Nv4Cfg::NT) __attribute__((amdgpu_waves_per_eu(Nv4Cfg::WPE)))
void k_gemm_nv4(GemmNv4Args p) {
  using C = Nv4Cfg;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, WM = C::WM, WN = C::WN, W = C::W;
  constexpr int MI = C::MI, NI = C::NI, CH = C::CH, RPD = C::RPD, AJ = C::AJ, NT = C::NT;
  static_assert(BK == 64 && BN * 2 == NT, "one thread per half row of a 64-deep weight slab");
  constexpr int A_U4 = BM * CH, B_U4 = BN * CH;
  constexpr int RING_U4 = 3 * A_U4 + 3 * B_U4;
  constexpr int STG_U4 = BM * C::LSD * 2 / 16;
  __shared__ uint4 smem[RING_U4 > STG_U4 ? RING_U4 : STG_U4];
  const int ncol = GATEUP ? p.N / (BN / 2) : p.N / BN;
  int tile, ct;
  if (!xcd_item(p.meta[1], ncol, tile, ct)) return;
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int base = p.offsets[e];
  const int cnt = p.offsets[e + 1] - base;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / WN, wn = wv % WN;
  const int64_t K = p.K;

  const bf16_t* ag[AJ];
#pragma unroll
  for (int i = 0; i < AJ; ++i) {
    const int r = RPD * (wv + W * i) + lane / CH;
    const int m = min(m0 + r, cnt - 1);
    ag[i] = (GATEUP ? p.a + int64_t(p.row_token[base + m]) * K : p.a + int64_t(base + m) * K) +
            C::dma_chunk(lane, wv + W * i) * 8;
  }
  // this thread's weight half row: slab row wr, K half hh
  const int wr = tid >> 1, hh = tid & 1;
  const uint8_t* wc;
  const uint8_t* wsc;
  float gsc0, gsc1 = 0.f;
  {
    const int64_t cst = int64_t(p.N) * (K / 2), sst = int64_t(p.N) * (K / 16);
    int64_t row;
    bool second = false;
    if (GATEUP) {
      second = wr >= BN / 2;
      row = int64_t(ct) * (BN / 2) + (second ? wr - BN / 2 : wr);
    } else {
      row = int64_t(ct) * BN + wr;
    }
    wc = expert_mat(second ? p.w1 : p.w0, second ? p.sh1 : p.sh0, e, p.E, cst) + row * (K / 2) + hh * 16;
    wsc = expert_mat(second ? p.b1 : p.b0, second ? p.shb1 : p.shb0, e, p.E, sst) + row * (K / 16) + hh * 2;
    gsc0 = e < p.E ? p.g0[e] : p.shg0[e - p.E];
    if (GATEUP) gsc1 = e < p.E ? p.g1[e] : p.shg1[e - p.E];
  }
  auto issue_a = [&](int kt, int slot) {
    const int64_t ko = int64_t(kt) * BK;
    uint4* sa = smem + slot * A_U4;
#pragma unroll
    for (int i = 0; i < AJ; ++i) dma16(ag[i] + ko, sa + (wv + W * i) * 64);
  };
  auto fetch_b = [&](int kt, uint4& c, uint32_t& sc) {
    c = *reinterpret_cast<const uint4*>(wc + int64_t(kt) * 32);
    sc = *reinterpret_cast<const uint16_t*>(wsc + int64_t(kt) * 4);
  };
  // chunk j (8 values) of this thread's 32 codes -> bf16 in slot `slot`
  auto convert_chunk = [&](const uint4& c, float s0, float s1, int slot, int j) {
    const uint32_t w = j == 0 ? c.x : j == 1 ? c.y : j == 2 ? c.z : c.w;
    const float sc = j < 2 ? s0 : s1;
    const auto f0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0);
    const auto f1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1);
    const auto f2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2);
    const auto f3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
    smem[3 * A_U4 + slot * B_U4 + C::pos(wr, hh * 4 + j)] =
        make_uint4(bf16_pair_hi(f0[0] * sc, f0[1] * sc), bf16_pair_hi(f1[0] * sc, f1[1] * sc),
                   bf16_pair_hi(f2[0] * sc, f2[1] * sc), bf16_pair_hi(f3[0] * sc, f3[1] * sc));
  };

  f32x16 acc[MI][NI];
#pragma unroll
  for (int a = 0; a < MI; ++a)
#pragma unroll
    for (int b = 0; b < NI; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  float roww[GATEUP ? 1 : MI][GATEUP ? 1 : 16];
  if (!GATEUP) {
#pragma unroll
    for (int a = 0; a < (GATEUP ? 1 : MI); ++a)
#pragma unroll
      for (int r = 0; r < (GATEUP ? 1 : 16); ++r) {
        const int row = wm * (BM / WM) + a * 32 + acc_row(r, lane);
        roww[a][r] = (p.out32 || m0 + row >= cnt) ? 0.f : p.row_w[base + m0 + row];
      }
  }
  auto load_frags = [&](const uint4* sa, const uint4* sb, int ks, bf16x8 (&af)[MI], bf16x8 (&bfr)[NI]) {
    const int chunk = ks * 2 + (lane >> 5);
#pragma unroll
    for (int a = 0; a < MI; ++a)
      af[a] = __builtin_bit_cast(bf16x8, sa[C::pos(wm * (BM / WM) + a * 32 + (lane & 31), chunk)]);
#pragma unroll
    for (int b = 0; b < NI; ++b) {
      const int row = GATEUP ? ((b < NI / 2 ? 0 : BN / 2) + wn * (BN / 2 / WN) + (b % (NI / 2)) * 32 + (lane & 31))
                             : (wn * (BN / WN) + b * 32 + (lane & 31));
      bfr[b] = __builtin_bit_cast(bf16x8, sb[C::pos(row, chunk)]);
    }
  };
  // MFMAs on slab `slot`; the next slab's conversion (chunk ks after sub-step ks) and
  // the refill loads run between them
  auto compute = [&](int slot, bool conv, const uint4& c, uint32_t sc2, int cslot, auto&& between) {
    const uint4* sa = smem + slot * A_U4;
    const uint4* sb = smem + 3 * A_U4 + slot * B_U4;
    float s0 = 0.f, s1 = 0.f;
    if (conv) e4m3_pair(sc2, s0, s1);
    bf16x8 af[2][MI], bfr[2][NI];
    load_frags(sa, sb, 0, af[0], bfr[0]);
    __builtin_amdgcn_sched_barrier(0);
    between();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      if (ks + 1 < 4) load_frags(sa, sb, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < NI; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][a], bfr[ks & 1][b], acc[a][b], 0, 0, 0);
      if (conv) convert_chunk(c, s0, s1, cslot, ks);
    }
  };

  const int nk = int(K / BK);
  // prologue: A0, B0, B1, A1 (weight registers before the activation DMAs, so that
  // waiting for slab kt's activations and slab kt+1's weights leaves only A(kt+1) out)
  uint4 cA, cB;
  uint32_t sA = 0u, sB = 0u;
  issue_a(0, 0);
  fetch_b(0, cA, sA);
  if (nk > 1) {
    fetch_b(1, cB, sB);
    issue_a(1, 1);
    wait_vm_lgkm0<AJ + 2>();
  } else {
    wait_vm_lgkm0<0>();
  }
  {
    float s0, s1;
    e4m3_pair(sA, s0, s1);
#pragma unroll
    for (int j = 0; j < 4; ++j) convert_chunk(cA, s0, s1, 0, j);
  }
  // step kt: wait for A(kt) and B(kt+1); barrier; fetch B(kt+2) into the register
  // slot B(kt) used, DMA A(kt+2); multiply slab kt while converting B(kt+1)
#define MOE_NV_STEP(KT, SLOT, NSLOT, CNEXT, SNEXT, CFREE, SFREE)                             \
  {                                                                                          \
    if ((KT) + 1 < nk) wait_vm_lgkm0<AJ>(); else wait_vm_lgkm0<0>();                         \
    block_sync_nowait();                                                                     \
    compute(SLOT, (KT) + 1 < nk, CNEXT, SNEXT, NSLOT, [&] {                                  \
      if ((KT) + 2 < nk) {                                                                   \
        fetch_b((KT) + 2, CFREE, SFREE);                                                     \
        issue_a((KT) + 2, ((KT) + 2) % 3);                                                   \
      }                                                                                      \
    });                                                                                      \
  }
  // weight register slots alternate: slab kt+1 sits in cB (kt even) or cA (kt odd)
  for (int kt = 0; kt < nk; kt += 6) {
    MOE_NV_STEP(kt, 0, 1, cB, sB, cA, sA)
    if (kt + 1 < nk) MOE_NV_STEP(kt + 1, 1, 2, cA, sA, cB, sB)
    if (kt + 2 < nk) MOE_NV_STEP(kt + 2, 2, 0, cB, sB, cA, sA)
    if (kt + 3 < nk) MOE_NV_STEP(kt + 3, 0, 1, cA, sA, cB, sB)
    if (kt + 4 < nk) MOE_NV_STEP(kt + 4, 1, 2, cB, sB, cA, sA)
    if (kt + 5 < nk) MOE_NV_STEP(kt + 5, 2, 0, cA, sA, cB, sB)
  }
#undef MOE_NV_STEP

  if (GATEUP || !p.out32) {
    constexpr int OC = GATEUP ? BN / 2 : BN;
    constexpr int LS = GATEUP ? C::LSG : C::LSD;
    bf16_t* stg = reinterpret_cast<bf16_t*>(smem);
    __syncthreads();
#pragma unroll
    for (int a = 0; a < MI; ++a) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * (BM / WM) + a * 32 + acc_row(r, lane);
        if (GATEUP) {
#pragma unroll
          for (int b = 0; b < NI / 2; ++b) {
            const float g = acc[a][b][r] * gsc0, u = acc[a][b + NI / 2][r] * gsc1;
            stg[row * LS + wn * (BN / 2 / WN) + b * 32 + (lane & 31)] = f32_to_bf16(silu_lp(g) * u);
          }
        } else {
          const float wr2 = roww[GATEUP ? 0 : a][GATEUP ? 0 : r] * gsc0;
#pragma unroll
          for (int b = 0; b < NI; ++b)
            stg[row * LS + wn * (BN / WN) + b * 32 + (lane & 31)] = f32_to_bf16(acc[a][b][r] * wr2);
        }
      }
    }
    __syncthreads();
    constexpr int CPR = OC / 8;
    const int rows = min(BM, cnt - m0);
    const int col0 = ct * OC;
    for (int i = tid; i < rows * CPR; i += NT) {
      const int row = i / CPR, c = i - row * CPR;
      const uint4 v = *reinterpret_cast<const uint4*>(stg + row * LS + c * 8);
      *reinterpret_cast<uint4*>(p.out16 + int64_t(base + m0 + row) * p.N + col0 + c * 8) = v;
    }
    return;
  }
#pragma unroll
  for (int a = 0; a < MI; ++a) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int row = wm * (BM / WM) + a * 32 + acc_row(r, lane);
      if (m0 + row >= cnt) continue;
      const int64_t grow = int64_t(base + m0 + row);
#pragma unroll
      for (int b = 0; b < NI; ++b)
        p.out32[grow * p.N + ct * BN + wn * (BN / WN) + b * 32 + (lane & 31)] = acc[a][b][r] * gsc0;
    }
  }
}

// shapes the NVFP4 matrix-core kernels cover
bool nv4_mfma_ok(const Plan& p) {
  return p.wt == MOE_NVFP4 && p.I % (Nv4Cfg::BN / 2) == 0 && p.H % Nv4Cfg::BN == 0 &&
         p.H % Nv4Cfg::BK == 0 && p.I % Nv4Cfg::BK == 0;
}

// shapes the pipelined bf16 kernel covers (else the register-staged one runs)
static bool bf_pipelined_ok(const Plan& p) {
  return p.wt == MOE_BF16 && p.I % (BfCfg::BN / 2) == 0 && p.H % BfCfg::BN == 0 &&
         p.H % BfCfg::BK == 0 && p.I % BfCfg::BK == 0;
}

int gemm_tile_rows(const Plan& p) {
  return bf_pipelined_ok(p) ? BfCfg::BM : nv4_mfma_ok(p) ? Nv4Cfg::BM : TM;
}

// Grid of the persistent down-projection kernels: one workgroup per CU, a multiple of
// the 8 XCDs.
static int persistent_grid(unsigned* grid) {
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    check_launch();
    return MOE_ERR_HIP;
  }
  *grid = unsigned(std::max(8, cus / 8 * 8));
  return MOE_OK;
}

// ---------------------------------------------------------------------------
// bf16 down projection, persistent: the tile, ring and MFMA steps of
// k_gemm_bf16_v2<false>, with one workgroup per CU walking an XCD-contiguous run of
// tiles as k_gemm_fp8_down_p does.  Each tile's ring starts at slot 0 (static slots);
// once every wave is past the K loop the next tile's first two slabs go into slots
// 0-1 and the epilogue stages its weighted rows through slot 2, in two 64-row halves,
// while they land.  The next tile's set-up loads run during the K loop and its row
// weights arrive in LDS with its first slab, so nothing after the K loop waits for
// memory, and the epilogue's barriers wait for LDS only, so nothing waits for the
// slabs in flight.
__global__ __launch_bounds__(BfCfg::NT) __attribute__((amdgpu_waves_per_eu(BfCfg::WPE)))
void k_gemm_bf16_down_p(GemmBf16Args p) {
  using C = BfCfg;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, WM = C::WM, WN = C::WN, W = C::W;
  constexpr int MI = C::MI, NI = C::NI, CH = C::CH, RPD = C::RPD, AJ = C::AJ, BJ = C::BJ;
  constexpr int L = C::L, NT = C::NT, KS = BK / 16;
  static_assert(KS % 2 == 0, "fragment double buffer");
  __shared__ uint4 smem[C::RING_U4];
  __shared__ __align__(16) float rw_l[BM];                   // the tile's row weights
  __shared__ int offs_l[MOE_MAX_ES + 1];  // expert row offsets
  const bool weighted = p.out32 == nullptr;
  const int ncol = p.N / BN;
  const int n = p.meta[1] * ncol;
  const int per = (n + 7) >> 3;
  const int run0 = int(blockIdx.x & 7) * per, q0 = int(blockIdx.x >> 3), P = int(gridDim.x >> 3);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar registers)
  const int wm = wv / WN, wn = wv % WN;
  const int64_t K = p.K;
  const int nk = int(K / BK);
  const int64_t mst = int64_t(p.N) * K;                      // elements of one expert matrix
  // workgroup barrier for LDS hand-offs: waits for this wave's LDS operations only
  auto lds_sync = [] {
    wait_vm_lgkm0<63>();
    block_sync_nowait();
  };
  auto item_of = [&](int tau, int& tile, int& ct) {
    const int q = q0 + P * tau, j = run0 + q;
    if (q >= per || j >= n) return false;
    tile = j / ncol;
    ct = j - tile * ncol;
    return true;
  };

  const bf16_t* ag[AJ];
  const bf16_t* wbase;                                       // the tile's expert matrix
  uint32_t boff[BJ];                                         // this lane's element offsets in it
  int src_m0, src_base, src_cnt;
  auto set_source = [&](int e, int m0, int base, int cnt, int ct) {
    src_m0 = m0;
    src_base = base;
    src_cnt = cnt;
#pragma unroll
    for (int i = 0; i < AJ; ++i) {
      const int r = RPD * (wv + W * i) + lane / CH;
      const int m = min(m0 + r, cnt - 1);
      ag[i] = p.a + int64_t(base + m) * K + C::dma_chunk(lane, wv + W * i) * 8;
    }
    wbase = expert_mat(p.w0, p.sh0, e, p.E, mst);
#pragma unroll
    for (int i = 0; i < BJ; ++i) {
      const int r = RPD * (wv + W * i) + lane / CH;
      boff[i] = uint32_t((ct * BN + r) * K + C::dma_chunk(lane, wv + W * i) * 8);
    }
  };
  auto issue = [&](int kt, int slot) {
    const int ko = kt * BK;
    uint4* sa = smem + slot * C::STAGE_U4;
    uint4* sb = sa + C::A_U4;
#pragma unroll
    for (int i = 0; i < AJ; ++i) dma16(ag[i] + ko, sa + (wv + W * i) * 64);
#pragma unroll
    for (int i = 0; i < BJ; ++i) dma16(wbase + (boff[i] + ko), sb + (wv + W * i) * 64);
  };
  // the row weights of the tile set_source chose, into rw_l by wave 0 (rows past the
  // expert's last read its last row; the epilogue zeroes them); issued between slab 0
  // and slab 1, so slab 0's wait covers them
  auto issue_roww = [&] {
    if (weighted && wv == 0) {
      const float* rw = p.row_w + src_base + src_m0;
      const int last = src_cnt - src_m0 - 1;
#pragma unroll
      for (int h = 0; h < BM / 64; ++h) dma4(rw + min(h * 64 + lane, last), rw_l + h * 64);
    }
  };

  f32x16 acc[MI][NI];
  auto load_frags = [&](const uint4* sa, const uint4* sb, int ks, bf16x8 (&af)[MI], bf16x8 (&bfr)[NI]) {
    const int chunk = ks * 2 + (lane >> 5);
#pragma unroll
    for (int a = 0; a < MI; ++a)
      af[a] = __builtin_bit_cast(bf16x8, sa[C::pos(wm * (BM / WM) + a * 32 + (lane & 31), chunk)]);
#pragma unroll
    for (int b = 0; b < NI; ++b)
      bfr[b] = __builtin_bit_cast(bf16x8, sb[C::pos(wn * (BN / WN) + b * 32 + (lane & 31), chunk)]);
  };
  auto compute = [&](int slot, auto&& between) {
    const uint4* sa = smem + slot * C::STAGE_U4;
    const uint4* sb = sa + C::A_U4;
    bf16x8 af[2][MI], bfr[2][NI];
    load_frags(sa, sb, 0, af[0], bfr[0]);
    __builtin_amdgcn_sched_barrier(0);
    between();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) load_frags(sa, sb, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < NI; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][a], bfr[ks & 1][b], acc[a][b], 0, 0, 0);
    }
  };

  int tile, ct;
  if (!item_of(0, tile, ct)) return;
  for (int i = tid; i <= p.ES; i += NT) offs_l[i] = p.offsets[i];
  __syncthreads();
  {
    const int2 te = p.tiles[tile];
    const int b = __builtin_amdgcn_readfirstlane(offs_l[te.x]);
    set_source(te.x, te.y, b, __builtin_amdgcn_readfirstlane(offs_l[te.x + 1]) - b, ct);
  }
  issue(0, 0);
  issue_roww();
  if (nk > 1) issue(1, 1);
  for (int tau = 0;; ++tau) {
    const int m0 = src_m0, base = src_base, cnt = src_cnt;
    // the next tile's table entry, loaded now (the first step's wait covers it); its
    // expert's row range comes from LDS, so none of the set-up waits for memory after
    // the K loop
    int tile_n = 0, ct_n = 0;
    const bool more = item_of(tau + 1, tile_n, ct_n);
    int2 te_n = make_int2(0, 0);
    if (more) te_n = p.tiles[tile_n];
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
      for (int b = 0; b < NI; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    // slab kt in slot kt % 3; after an epilogue its stores are in the count too, so a
    // tile's first step waits for everything
#define MOE_BFP_STEP(KT, SLOT, NSLOT)                                                      \
    {                                                                                      \
      if ((KT) + 1 < nk && !((KT) == 0 && tau > 0)) wait_vm_lgkm0<L>(); else wait_vm_lgkm0<0>(); \
      block_sync_nowait();                                                                 \
      compute(SLOT, [&] { if ((KT) + 2 < nk) issue((KT) + 2, NSLOT); });                   \
    }
    for (int kt = 0; kt < nk; kt += 3) {
      MOE_BFP_STEP(kt, 0, 2)
      if (kt + 1 < nk) MOE_BFP_STEP(kt + 1, 1, 0)
      if (kt + 2 < nk) MOE_BFP_STEP(kt + 2, 2, 1)
    }
#undef MOE_BFP_STEP
    const int cur_ct = ct;
    const int rows = min(BM, cnt - m0);
    // this lane's row weights (accumulator rows: four consecutive rows per 16-byte read)
    float roww[MI][16];
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row0 = wm * (BM / WM) + a * 32 + 8 * g + 4 * (lane >> 5);
        const float4 v = weighted ? *reinterpret_cast<const float4*>(rw_l + row0) : make_float4(0.f, 0.f, 0.f, 0.f);
        roww[a][4 * g + 0] = row0 + 0 < rows ? v.x : 0.f;
        roww[a][4 * g + 1] = row0 + 1 < rows ? v.y : 0.f;
        roww[a][4 * g + 2] = row0 + 2 < rows ? v.z : 0.f;
        roww[a][4 * g + 3] = row0 + 3 < rows ? v.w : 0.f;
      }
    if (more) {
      tile = tile_n;
      ct = ct_n;
      const int base_n = __builtin_amdgcn_readfirstlane(offs_l[te_n.x]);
      set_source(te_n.x, te_n.y, base_n, __builtin_amdgcn_readfirstlane(offs_l[te_n.x + 1]) - base_n, ct_n);
    }
    wait_vm_lgkm0<0>();
    lds_sync();                      // every wave is past the K loop and has its row weights
    if (more) {
      issue(0, 0);
      issue_roww();
      if (nk > 1) issue(1, 1);
    }
    if (p.out32) {
      // unweighted fp32 rows straight from the registers
#pragma unroll
      for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int row = wm * (BM / WM) + a * 32 + acc_row(r, lane);
          if (row >= rows) continue;
          const int64_t grow = int64_t(base + m0 + row);
#pragma unroll
          for (int b = 0; b < NI; ++b)
            p.out32[grow * p.N + cur_ct * BN + wn * (BN / WN) + b * 32 + (lane & 31)] = acc[a][b][r];
        }
    } else {
      // weighted bf16 rows through slot 2, one 64-row half of the tile at a time, so
      // that each row leaves as whole 16-byte pieces
      constexpr int LS = C::LSD;
      bf16_t* stg = reinterpret_cast<bf16_t*>(smem + 2 * C::STAGE_U4);
#pragma unroll
      for (int half = 0; half < WM; ++half) {
        if (wm == half) {
#pragma unroll
          for (int a = 0; a < MI; ++a)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int lrow = a * 32 + acc_row(r, lane);
#pragma unroll
              for (int b = 0; b < NI; ++b)
                stg[lrow * LS + wn * (BN / WN) + b * 32 + (lane & 31)] = f32_to_bf16(acc[a][b][r] * roww[a][r]);
            }
        }
        lds_sync();
        constexpr int CPR = BN / 8;                // 16-byte pieces per row
        const int hrows = min(BM / WM, rows - half * (BM / WM));
        for (int i = tid; i < hrows * CPR; i += NT) {
          const int lrow = i / CPR, c = i - lrow * CPR;
          *reinterpret_cast<uint4*>(p.out16 + int64_t(base + m0 + half * (BM / WM) + lrow) * p.N +
                                    cur_ct * BN + c * 8) =
              *reinterpret_cast<const uint4*>(stg + lrow * LS + c * 8);
        }
        if (half + 1 < WM) lds_sync();
      }
    }
    if (!more) break;
  }
}

// ---------------------------------------------------------------------------
// bf16 gate/up + SwiGLU, persistent: the tile, ring and MFMA steps of
// k_gemm_bf16_v2<true> with the item walk of k_gemm_bf16_down_p (one workgroup per
// CU over an XCD-contiguous run of items, static ring slots, the next item's first two
// slabs loaded during the epilogue).  The activation rows are gathered through
// row_token, so an item's set-up needs its 128 row tokens before its first slab can be
// issued: for the next item they are fetched into LDS during the current item's
// first step (4-byte direct-to-LDS loads by wave 0, issued ahead of slab 2, so the
// second step's wait covers them), its table entry is loaded before the K loop and its
// expert's row range comes from LDS, so nothing after the K loop waits for memory.
// The h tile (128 rows x 128 columns) is staged through slot 2 in one pass.
__global__ __launch_bounds__(BfCfg::NT) __attribute__((amdgpu_waves_per_eu(BfCfg::WPE)))
void k_gemm_bf16_gateup_p(GemmBf16Args p) {
  using C = BfCfg;
  constexpr int BM = C::BM, BN = C::BN, BK = C::BK, WM = C::WM, WN = C::WN, W = C::W;
  constexpr int MI = C::MI, NI = C::NI, CH = C::CH, RPD = C::RPD, AJ = C::AJ, BJ = C::BJ;
  constexpr int L = C::L, NT = C::NT, KS = BK / 16, OC = BN / 2;
  static_assert(KS % 2 == 0, "fragment double buffer");
  static_assert(BM * C::LSG * 2 <= C::STAGE_U4 * 16, "h tile staging fits one ring slot");
  __shared__ uint4 smem[C::RING_U4];
  __shared__ int rt_l[BM];                 // the next item's row tokens
  __shared__ int offs_l[MOE_MAX_ES + 1];   // expert row offsets
  const int ncol = p.N / OC;
  const int n = p.meta[1] * ncol;
  const int per = (n + 7) >> 3;
  const int run0 = int(blockIdx.x & 7) * per, q0 = int(blockIdx.x >> 3), P = int(gridDim.x >> 3);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar registers)
  const int wm = wv / WN, wn = wv % WN;
  const int64_t K = p.K;
  const int nk = int(K / BK);
  const int64_t mst = int64_t(p.N) * K;                      // elements of one expert matrix
  auto lds_sync = [] {
    wait_vm_lgkm0<63>();
    block_sync_nowait();
  };
  auto item_of = [&](int tau, int& tile, int& ct) {
    const int q = q0 + P * tau, j = run0 + q;
    if (q >= per || j >= n) return false;
    tile = j / ncol;
    ct = j - tile * ncol;
    return true;
  };

  const bf16_t* ag[AJ];
  const bf16_t* bbase[BJ];                                   // gate or up matrix (wave-uniform)
  uint32_t boff[BJ];                                         // this lane's element offsets in it
  int src_m0, src_base, src_cnt;
  // rtok(r): the row token of the item's row r (rows past the expert's last repeat it)
  auto set_source = [&](int e, int m0, int base, int cnt, int ct, auto&& rtok) {
    src_m0 = m0;
    src_base = base;
    src_cnt = cnt;
#pragma unroll
    for (int i = 0; i < AJ; ++i) {
      const int r = RPD * (wv + W * i) + lane / CH;
      ag[i] = p.a + int64_t(rtok(r)) * K + C::dma_chunk(lane, wv + W * i) * 8;
    }
    const bf16_t* wg = expert_mat(p.w0, p.sh0, e, p.E, mst);
    const bf16_t* wu = expert_mat(p.w1, p.sh1, e, p.E, mst);
#pragma unroll
    for (int i = 0; i < BJ; ++i) {
      const int r0 = RPD * (wv + W * i), r = r0 + lane / CH;   // a load's rows: r0 .. r0+RPD-1
      bbase[i] = r0 < OC ? wg : wu;
      boff[i] = uint32_t((ct * OC + (r0 < OC ? r : r - OC)) * K + C::dma_chunk(lane, wv + W * i) * 8);
    }
  };
  auto issue = [&](int kt, int slot) {
    const int ko = kt * BK;
    uint4* sa = smem + slot * C::STAGE_U4;
    uint4* sb = sa + C::A_U4;
#pragma unroll
    for (int i = 0; i < AJ; ++i) dma16(ag[i] + ko, sa + (wv + W * i) * 64);
#pragma unroll
    for (int i = 0; i < BJ; ++i) dma16(bbase[i] + (boff[i] + ko), sb + (wv + W * i) * 64);
  };

  f32x16 acc[MI][NI];
  auto load_frags = [&](const uint4* sa, const uint4* sb, int ks, bf16x8 (&af)[MI], bf16x8 (&bfr)[NI]) {
    const int chunk = ks * 2 + (lane >> 5);
#pragma unroll
    for (int a = 0; a < MI; ++a)
      af[a] = __builtin_bit_cast(bf16x8, sa[C::pos(wm * (BM / WM) + a * 32 + (lane & 31), chunk)]);
#pragma unroll
    for (int b = 0; b < NI; ++b) {
      // blocks 0..NI/2-1 are gate columns, NI/2.. the matching up columns
      const int row = (b < NI / 2 ? 0 : OC) + wn * (OC / WN) + (b % (NI / 2)) * 32 + (lane & 31);
      bfr[b] = __builtin_bit_cast(bf16x8, sb[C::pos(row, chunk)]);
    }
  };
  auto compute = [&](int slot, auto&& between) {
    const uint4* sa = smem + slot * C::STAGE_U4;
    const uint4* sb = sa + C::A_U4;
    bf16x8 af[2][MI], bfr[2][NI];
    load_frags(sa, sb, 0, af[0], bfr[0]);
    __builtin_amdgcn_sched_barrier(0);
    between();
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      if (ks + 1 < KS) load_frags(sa, sb, ks + 1, af[(ks + 1) & 1], bfr[(ks + 1) & 1]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int a = 0; a < MI; ++a)
#pragma unroll
        for (int b = 0; b < NI; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[ks & 1][a], bfr[ks & 1][b], acc[a][b], 0, 0, 0);
    }
  };

  int tile, ct;
  if (!item_of(0, tile, ct)) return;
  for (int i = tid; i <= p.ES; i += NT) offs_l[i] = p.offsets[i];
  __syncthreads();
  {
    const int2 te = p.tiles[tile];
    const int b = __builtin_amdgcn_readfirstlane(offs_l[te.x]);
    const int c = __builtin_amdgcn_readfirstlane(offs_l[te.x + 1]) - b;
    set_source(te.x, te.y, b, c, ct, [&](int r) { return p.row_token[b + min(te.y + r, c - 1)]; });
  }
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int tau = 0;; ++tau) {
    const int m0 = src_m0, base = src_base, cnt = src_cnt;
    // the next item's table entry, loaded now (the first step's wait covers it)
    int tile_n = 0, ct_n = 0;
    const bool more = item_of(tau + 1, tile_n, ct_n);
    int2 te_n = make_int2(0, 0);
    if (more) te_n = p.tiles[tile_n];
    int base_n = 0, cnt_n = 0;
    // the next item's row tokens into rt_l (wave 0), issued in the first step ahead of
    // slab 2, so that the second step's wait covers them
    auto issue_rt_next = [&] {
      base_n = __builtin_amdgcn_readfirstlane(offs_l[te_n.x]);
      cnt_n = __builtin_amdgcn_readfirstlane(offs_l[te_n.x + 1]) - base_n;
      if (wv == 0) {
        const int32_t* rt = p.row_token + base_n;
        const int last = cnt_n - 1;
#pragma unroll
        for (int h = 0; h < BM / 64; ++h) dma4(rt + min(te_n.y + h * 64 + lane, last), rt_l + h * 64);
      }
    };
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
      for (int b = 0; b < NI; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    // slab kt in slot kt % 3; after an epilogue its stores are in the count too, so an
    // item's first step waits for everything
#define MOE_BGP_STEP(KT, SLOT, NSLOT)                                                      \
    {                                                                                      \
      if ((KT) + 1 < nk && !((KT) == 0 && tau > 0)) wait_vm_lgkm0<L>(); else wait_vm_lgkm0<0>(); \
      block_sync_nowait();                                                                 \
      compute(SLOT, [&] {                                                                  \
        if ((KT) == 0 && more) issue_rt_next();                                            \
        if ((KT) + 2 < nk) issue((KT) + 2, NSLOT);                                         \
      });                                                                                  \
    }
    for (int kt = 0; kt < nk; kt += 3) {
      MOE_BGP_STEP(kt, 0, 2)
      if (kt + 1 < nk) MOE_BGP_STEP(kt + 1, 1, 0)
      if (kt + 2 < nk) MOE_BGP_STEP(kt + 2, 2, 1)
    }
#undef MOE_BGP_STEP
    const int cur_ct = ct;
    const int rows = min(BM, cnt - m0);
    wait_vm_lgkm0<0>();
    lds_sync();                      // every wave is past the K loop; the row tokens have landed
    if (more) {
      tile = tile_n;
      ct = ct_n;
      set_source(te_n.x, te_n.y, base_n, cnt_n, ct_n, [&](int r) { return rt_l[r]; });
      issue(0, 0);
      if (nk > 1) issue(1, 1);
    }
    // h = silu(gate) * up through slot 2, so that each row leaves as whole 16-byte pieces
    constexpr int LS = C::LSG;
    bf16_t* stg = reinterpret_cast<bf16_t*>(smem + 2 * C::STAGE_U4);
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = wm * (BM / WM) + a * 32 + acc_row(r, lane);
#pragma unroll
        for (int b = 0; b < NI / 2; ++b) {
          const float g = acc[a][b][r], u = acc[a][b + NI / 2][r];
          stg[row * LS + wn * (OC / WN) + b * 32 + (lane & 31)] = f32_to_bf16(silu_lp(g) * u);
        }
      }
    lds_sync();
    constexpr int CPR = OC / 8;                // 16-byte pieces per row
    for (int i = tid; i < rows * CPR; i += NT) {
      const int row = i / CPR, c = i - row * CPR;
      *reinterpret_cast<uint4*>(p.out16 + int64_t(base + m0 + row) * p.N + cur_ct * OC + c * 8) =
          *reinterpret_cast<const uint4*>(stg + row * LS + c * 8);
    }
    if (!more) break;
  }
}

// ===========================================================================
// Block FP8.  Weights e4m3 with one fp32 scale per 128x128 block; activations
// e4m3 with one fp32 scale per row per 128 along K.  One K slab = 128 = one
// scale block.  Here the weight rows are the MFMA's M operand and activation
// rows its N operand, so the activation scale of an output is per lane and the
// weight scale is uniform over a 32-row block: after each slab's two
// 32x32x64 MFMAs the slab result is added as acc += slab * (s_act * s_w).
struct GemmFp8Args {
  const uint8_t* a;           // gate/up: x codes [T, H] (gathered); down: h codes [R, I]
  const float* a_scale;       // [rows, K/128]
  const int32_t* row_token;   // gate/up only
  const int32_t* offsets;
  const int2* tiles;
  const int32_t* meta;
  const uint8_t* w0;          // gate/up: w_gate; down: w_down
  const uint8_t* w1;          // gate/up: w_up
  const uint8_t* sh0;
  const uint8_t* sh1;
  const float* s0;            // block scales of w0 / w1 / shared
  const float* s1;
  const float* shs0;
  const float* shs1;
  const float* row_w;         // down, weighted bf16 output
  float* hout;                // gate/up: h fp32 [R, I] (register-staged kernel)
  uint8_t* qout;              // gate/up: h e4m3 codes [R, I] (pipelined kernel)
  float* qscale;              // gate/up: h scales [R, I/128] (pipelined kernel)
  bf16_t* out16;              // down: weighted y_perm [R, H] (bf16)
  float* out32;               // down: unweighted y_perm [R, H]
  int K, N, E;
};

template <bool GATEUP>
__global__ __launch_bounds__(256) void k_gemm_fp8(GemmFp8Args p) {
  constexpr int BK = 128;
  const int ncol = GATEUP ? p.N / 64 : p.N / TN;
  int tile, ct;
  if (!xcd_item(p.meta[1], ncol, tile, ct)) return;
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int base = p.offsets[e];
  const int cnt = p.offsets[e + 1] - base;

  __shared__ uint4 Ws[2][TN * 8];     // weight rows (M operand), 128 bytes of K each
  __shared__ uint4 Xs[2][TM * 8];     // activation rows (N operand)

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int ww = wv >> 1, wr = wv & 1;
  const int kc = tid & 7;
  const int64_t K = p.K;
  const int nkb = int(K / BK);

  const uint8_t* xg[4];
  const uint8_t* wg[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = (tid >> 3) + 32 * i;
    const int m = min(m0 + rr, cnt - 1);
    const int64_t arow = GATEUP ? int64_t(p.row_token[base + m]) : int64_t(base + m);
    xg[i] = p.a + arow * K + kc * 16;
    if (GATEUP) {
      const int64_t st = int64_t(p.N) * K;
      wg[i] = rr < 64 ? expert_mat(p.w0, p.sh0, e, p.E, st) + int64_t(ct * 64 + rr) * K + kc * 16
                      : expert_mat(p.w1, p.sh1, e, p.E, st) + int64_t(ct * 64 + rr - 64) * K + kc * 16;
    } else {
      wg[i] = expert_mat(p.w0, p.sh0, e, p.E, int64_t(p.N) * K) + int64_t(ct * TN + rr) * K + kc * 16;
    }
  }
  // activation scale rows of this lane's two 32-row N blocks
  const float* asr[2];
#pragma unroll
  for (int ri = 0; ri < 2; ++ri) {
    const int m = min(m0 + wr * 64 + ri * 32 + (lane & 31), cnt - 1);
    const int64_t arow = GATEUP ? int64_t(p.row_token[base + m]) : int64_t(base + m);
    asr[ri] = p.a_scale + arow * nkb;
  }
  // weight scale rows: this wave's two 32-row M blocks (gate/up: gate block, up block)
  const float* wsr[2];
  {
    const int64_t sst = int64_t(p.N / 128) * nkb;
    if (GATEUP) {
      const int sb = (ct * 64) / 128;
      wsr[0] = expert_mat(p.s0, p.shs0, e, p.E, sst) + int64_t(sb) * nkb;
      wsr[1] = expert_mat(p.s1, p.shs1, e, p.E, sst) + int64_t(sb) * nkb;
    } else {
      const int sb = ct;   // TN == 128 rows of W_down = one scale block
      wsr[0] = wsr[1] = expert_mat(p.s0, p.shs0, e, p.E, sst) + int64_t(sb) * nkb;
    }
  }

  f32x16 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

  uint4 rx[4], rw[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    rx[i] = *reinterpret_cast<const uint4*>(xg[i]);
    rw[i] = *reinterpret_cast<const uint4*>(wg[i]);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int rr = (tid >> 3) + 32 * i;
    Xs[0][swz16(rr, kc)] = rx[i];
    Ws[0][swz16(rr, kc)] = rw[i];
  }
  __syncthreads();

  for (int kb = 0; kb < nkb; ++kb) {
    const int cur = kb & 1;
    if (kb + 1 < nkb) {
      const int64_t ko = int64_t(kb + 1) * BK;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        rx[i] = *reinterpret_cast<const uint4*>(xg[i] + ko);
        rw[i] = *reinterpret_cast<const uint4*>(wg[i] + ko);
      }
    }
    float sa[2], sw[2];
#pragma unroll
    for (int ri = 0; ri < 2; ++ri) sa[ri] = asr[ri][kb];
#pragma unroll
    for (int wi = 0; wi < 2; ++wi) sw[wi] = wsr[wi][kb];

    f32x16 sl[2][2];
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) sl[a][b][r] = 0.f;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c0 = ks * 4 + (lane >> 5) * 2;
      i32x8 wf[2], xf[2];
#pragma unroll
      for (int wi = 0; wi < 2; ++wi) {
        const int row = GATEUP ? (wi * 64 + ww * 32 + (lane & 31)) : (ww * 64 + wi * 32 + (lane & 31));
        const uint4 lo = Ws[cur][swz16(row, c0)], hi = Ws[cur][swz16(row, c0 + 1)];
        wf[wi] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      }
#pragma unroll
      for (int ri = 0; ri < 2; ++ri) {
        const int row = wr * 64 + ri * 32 + (lane & 31);
        const uint4 lo = Xs[cur][swz16(row, c0)], hi = Xs[cur][swz16(row, c0 + 1)];
        xf[ri] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      }
#pragma unroll
      for (int wi = 0; wi < 2; ++wi)
#pragma unroll
        for (int ri = 0; ri < 2; ++ri)
          sl[wi][ri] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              wf[wi], xf[ri], sl[wi][ri], 0, 0, 0, 127, 0, 127);
    }
#pragma unroll
    for (int wi = 0; wi < 2; ++wi)
#pragma unroll
      for (int ri = 0; ri < 2; ++ri) {
        const float s = sa[ri] * sw[wi];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[wi][ri][r] = fmaf(sl[wi][ri][r], s, acc[wi][ri][r]);
      }
    if (kb + 1 < nkb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int rr = (tid >> 3) + 32 * i;
        Xs[cur ^ 1][swz16(rr, kc)] = rx[i];
        Ws[cur ^ 1][swz16(rr, kc)] = rw[i];
      }
    }
    __syncthreads();
  }

  // epilogue: lane -> activation row, register -> weight row (output column).
  // Registers 4q..4q+3 hold four consecutive columns, stored as one vector.
#pragma unroll
  for (int ri = 0; ri < 2; ++ri) {
    const int row = wr * 64 + ri * 32 + (lane & 31);
    if (m0 + row >= cnt) continue;
    const int64_t grow = int64_t(base + m0 + row);
    if (GATEUP) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int col = ct * 64 + ww * 32 + 8 * q + 4 * (lane >> 5);
        float4 v;
        v.x = silu_lp(acc[0][ri][4 * q + 0]) * acc[1][ri][4 * q + 0];
        v.y = silu_lp(acc[0][ri][4 * q + 1]) * acc[1][ri][4 * q + 1];
        v.z = silu_lp(acc[0][ri][4 * q + 2]) * acc[1][ri][4 * q + 2];
        v.w = silu_lp(acc[0][ri][4 * q + 3]) * acc[1][ri][4 * q + 3];
        *reinterpret_cast<float4*>(p.hout + grow * p.N + col) = v;
      }
    } else {
      const float wrow = p.row_w ? p.row_w[grow] : 1.f;
#pragma unroll
      for (int wi = 0; wi < 2; ++wi)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int col = ct * TN + ww * 64 + wi * 32 + 8 * q + 4 * (lane >> 5);
          if (p.out32) {
            *reinterpret_cast<float4*>(p.out32 + grow * p.N + col) =
                make_float4(acc[wi][ri][4 * q], acc[wi][ri][4 * q + 1], acc[wi][ri][4 * q + 2],
                            acc[wi][ri][4 * q + 3]);
          } else {
            uint2 pk;
            pk.x = uint32_t(f32_to_bf16(acc[wi][ri][4 * q] * wrow)) |
                   (uint32_t(f32_to_bf16(acc[wi][ri][4 * q + 1] * wrow)) << 16);
            pk.y = uint32_t(f32_to_bf16(acc[wi][ri][4 * q + 2] * wrow)) |
                   (uint32_t(f32_to_bf16(acc[wi][ri][4 * q + 3] * wrow)) << 16);
            *reinterpret_cast<uint2*>(p.out16 + grow * p.N + col) = pk;
          }
        }
    }
  }
}

// ===========================================================================
// Activation quantisation to e4m3, one wave per (row, 128-column block):
// scale = amax / 448 (fp32 division; 1 for an all-zero block), code = RNE(v / scale).
// Optional gather: row r reads source row row_token[r].
// ===========================================================================
// Block FP8, pipelined.  The slab of one K scale block (128 e4m3 = 128 bytes per
// tile row) has the same LDS layout as a bf16 slab of 64, so the same ring of
// direct-to-LDS loads, swizzle and XCD-aware item order apply.  Tile: BM = 128
// activation rows x BN = 256 weight rows (gate/up: 128 gate + the matching 128 up
// rows), 8 waves of 64 x 64.  The weight rows are the MFMA's M operand, so a
// 32-row weight block has one scale per slab and an activation row (a lane) has
// one; each slab's two 32x32x64 MFMAs go into a fresh block that is folded as
// acc += slab * (s_act * s_w).  All scales of the tile are staged in LDS before
// the K loop.  The gate/up epilogue applies SwiGLU and quantises h at once: the
// tile's 128 h columns are exactly one 128-wide scale block of each row.
struct Fp8Tile {
  static constexpr int BM = 128, BN = 256, KB = 128, WM = 2, WN = 4, W = WM * WN, NT = 64 * W;
  static constexpr int MI = BM / WM / 32, NI = BN / WN / 32;          // 2 x 2 blocks per wave
  static constexpr int AJ = BM / (8 * W), BJ = BN / (8 * W), L = AJ + BJ;
  static constexpr int A_U4 = BM * 8, STAGE_U4 = (BM + BN) * 8, RING_U4 = 3 * STAGE_U4;
  static constexpr int SMAX = 16;                                     // K <= 2048
};

template <bool GATEUP>
__global__ __launch_bounds__(Fp8Tile::NT) __attribute__((amdgpu_waves_per_eu(2)))
void k_gemm_fp8_v2(GemmFp8Args p) {
  using C = Fp8Tile;
  constexpr int BM = C::BM, BN = C::BN, W = C::W, WM = C::WM, WN = C::WN, MI = C::MI, NI = C::NI;
  constexpr int AJ = C::AJ, BJ = C::BJ, L = C::L, NT = C::NT, SMAX = C::SMAX;
  __shared__ uint4 smem[C::RING_U4];
  constexpr int SST = SMAX + 1;          // row stride of sa_l: odd, so 32 rows hit 32 banks
  __shared__ float sa_l[BM * SST];       // activation scales [row][slab]
  __shared__ float sw_l[4 * SMAX];       // weight block scales [block][slab]
  const int ncol = GATEUP ? p.N / (BN / 2) : p.N / BN;
  int tile, ct;
  if (!xcd_item(p.meta[1], ncol, tile, ct)) return;
  const int2 te = p.tiles[tile];
  const int e = te.x, m0 = te.y;
  const int base = p.offsets[e];
  const int cnt = p.offsets[e + 1] - base;
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wm = wv / WN, wn = wv % WN;
  const int64_t K = p.K;
  const int nkb = int(K / C::KB);

  const uint8_t* ag[AJ];
#pragma unroll
  for (int i = 0; i < AJ; ++i) {
    const int r = 8 * (wv + W * i) + (lane >> 3);
    const int m = min(m0 + r, cnt - 1);
    const int64_t arow = GATEUP ? int64_t(p.row_token[base + m]) : int64_t(base + m);
    ag[i] = p.a + arow * K + dma_chunk(lane, wv + W * i) * 16;
  }
  const int64_t mst = int64_t(p.N) * K;             // bytes of one expert matrix
  const uint8_t* bg[BJ];
#pragma unroll
  for (int i = 0; i < BJ; ++i) {
    const int r = 8 * (wv + W * i) + (lane >> 3);
    const int c = dma_chunk(lane, wv + W * i) * 16;
    if (GATEUP) {
      const int c0 = ct * (BN / 2);
      bg[i] = (r < BN / 2 ? expert_mat(p.w0, p.sh0, e, p.E, mst) + int64_t(c0 + r) * K
                          : expert_mat(p.w1, p.sh1, e, p.E, mst) + int64_t(c0 + r - BN / 2) * K) + c;
    } else {
      bg[i] = expert_mat(p.w0, p.sh0, e, p.E, mst) + int64_t(ct * BN + r) * K + c;
    }
  }
  auto issue = [&](int kt, int slot) {
    const int64_t ko = int64_t(kt) * C::KB;
    uint4* sa = smem + slot * C::STAGE_U4;
    uint4* sb = sa + C::A_U4;
#pragma unroll
    for (int i = 0; i < AJ; ++i) dma16(ag[i] + ko, sa + (wv + W * i) * 64);
#pragma unroll
    for (int i = 0; i < BJ; ++i) dma16(bg[i] + ko, sb + (wv + W * i) * 64);
  };
  const int nk = nkb;
  issue(0, 0);
  if (nk > 1) issue(1, 1);

  // scales of the tile -> LDS (while the first slabs are in flight).  Weight
  // scale blocks: gate/up [0] gate, [1] up (the tile's 128 h columns = block ct);
  // down: the two 128-row blocks 2ct, 2ct+1 of the tile's 256 output columns.
  {
    const int64_t sst = int64_t(p.N / 128) * nkb;
    constexpr int SP = BM * SMAX / NT;              // staged scales per thread (4)
    float sv[SP];
#pragma unroll
    for (int u = 0; u < SP; ++u) {                  // clamped loads, all in flight together
      const int i = min(tid + u * NT, BM * nkb - 1);
      const int row = i / nkb, kb = i - row * nkb;
      const int m = min(m0 + row, cnt - 1);
      const int64_t arow = GATEUP ? int64_t(p.row_token[base + m]) : int64_t(base + m);
      sv[u] = p.a_scale[arow * nkb + kb];
    }
#pragma unroll
    for (int u = 0; u < SP; ++u) {
      const int i = tid + u * NT;
      if (i < BM * nkb) sa_l[(i / nkb) * SST + i % nkb] = sv[u];
    }
    if (tid < 2 * nkb) {
      const int blk = tid / nkb, kb = tid - blk * nkb;
      float v;
      if (GATEUP)
        v = (blk == 0 ? expert_mat(p.s0, p.shs0, e, p.E, sst) : expert_mat(p.s1, p.shs1, e, p.E, sst))
                [int64_t(ct) * nkb + kb];
      else
        v = expert_mat(p.s0, p.shs0, e, p.E, sst)[int64_t(2 * ct + blk) * nkb + kb];
      sw_l[blk * SMAX + kb] = v;
    }
  }

  f32x16 acc[MI][NI];
#pragma unroll
  for (int a = 0; a < MI; ++a)
#pragma unroll
    for (int b = 0; b < NI; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  // this wave's weight blocks: gate/up b = 0 gate, 1 up (same h columns);
  // down: output columns wn*64 + 32b
  auto wrow = [&](int b) {
    return GATEUP ? (b == 0 ? 0 : BN / 2) + wn * (BN / 2 / WN) + (lane & 31)
                  : wn * (BN / WN) + b * 32 + (lane & 31);
  };
  const int swb0 = GATEUP ? 0 : (wn * (BN / WN)) / 128;   // scale block of weight block b
  auto compute = [&](int slot, int kt, auto&& between) {
    const uint4* sa = smem + slot * C::STAGE_U4;
    const uint4* sb = sa + C::A_U4;
    i32x8 af[2][MI], bfr[2][NI];
    auto frags = [&](int ks, i32x8 (&xa)[MI], i32x8 (&xb)[NI]) {
      const int c0 = ks * 4 + (lane >> 5) * 2;
#pragma unroll
      for (int a = 0; a < MI; ++a) {
        const int row = wm * (BM / WM) + a * 32 + (lane & 31);
        const uint4 lo = sa[swz16(row, c0)], hi = sa[swz16(row, c0 + 1)];
        xa[a] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      }
#pragma unroll
      for (int b = 0; b < NI; ++b) {
        const int row = wrow(b);
        const uint4 lo = sb[swz16(row, c0)], hi = sb[swz16(row, c0 + 1)];
        xb[b] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      }
    };
    frags(0, af[0], bfr[0]);
    __builtin_amdgcn_sched_barrier(0);
    between();
    frags(1, af[1], bfr[1]);
    __builtin_amdgcn_sched_barrier(0);
    float sact[MI], swt[NI];
#pragma unroll
    for (int a = 0; a < MI; ++a) sact[a] = sa_l[(wm * (BM / WM) + a * 32 + (lane & 31)) * SST + kt];
#pragma unroll
    for (int b = 0; b < NI; ++b) swt[b] = sw_l[(GATEUP ? b : swb0) * SMAX + kt];
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
      for (int b = 0; b < NI; ++b) {
        f32x16 sl;
#pragma unroll
        for (int r = 0; r < 16; ++r) sl[r] = 0.f;
        sl = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[0][b], af[0][a], sl, 0, 0, 0, 127, 0, 127);
        sl = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[1][b], af[1][a], sl, 0, 0, 0, 127, 0, 127);
        const float s = sact[a] * swt[b];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = fmaf(sl[r], s, acc[a][b][r]);
      }
  };
  __syncthreads();   // scales staged
#define MOE_F8_STEP(KT, SLOT, NSLOT)                                        \
  {                                                                         \
    if ((KT) + 1 < nk) wait_vm_lgkm0<L>(); else wait_vm_lgkm0<0>();         \
    block_sync_nowait();                                                    \
    compute(SLOT, KT, [&] { if ((KT) + 2 < nk) issue((KT) + 2, NSLOT); });  \
  }
  for (int kt = 0; kt < nk; kt += 3) {
    MOE_F8_STEP(kt, 0, 2)
    if (kt + 1 < nk) MOE_F8_STEP(kt + 1, 1, 0)
    if (kt + 2 < nk) MOE_F8_STEP(kt + 2, 2, 1)
  }
#undef MOE_F8_STEP

  // Epilogue.  Accumulator register r of block (a, b) holds weight row (output
  // column) 8(r/4) + 4(lane/32) + r%4 of the block for activation row lane%32:
  // four consecutive columns per register group.
  __syncthreads();   // every wave is done with the ring; it becomes staging space
  const int rows = min(BM, cnt - m0);
  if (GATEUP) {
    // h = silu(g) * u, its row amax over the tile's 128 columns (registers, the
    // lane 32 apart, then the four waves of the row block through LDS), scale =
    // amax / 448 (1 for an all-zero block), codes = e4m3(h / scale)
    float* red = reinterpret_cast<float*>(smem + 2048);       // [WM][MI][32][WN]
    uint8_t* stg = reinterpret_cast<uint8_t*>(smem);          // [BM][128] codes
    float hv[MI][16];
    float am[MI];
#pragma unroll
    for (int a = 0; a < MI; ++a) {
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        hv[a][r] = silu_lp(acc[a][0][r]) * acc[a][1][r];
        m = fmaxf(m, fabsf(hv[a][r]));
      }
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      am[a] = m;
      if (lane < 32) red[((wm * MI + a) * 32 + lane) * WN + wn] = m;
    }
    __syncthreads();
#pragma unroll
    for (int a = 0; a < MI; ++a) {
      const float* rr = red + ((wm * MI + a) * 32 + (lane & 31)) * WN;
      float m = rr[0];
#pragma unroll
      for (int j = 1; j < WN; ++j) m = fmaxf(m, rr[j]);
      const float scale = m > 0.f ? m / 448.0f : 1.0f;
      const int row = wm * (BM / WM) + a * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t pk = e4m3x4(hv[a][4 * g] / scale, hv[a][4 * g + 1] / scale,
                                   hv[a][4 * g + 2] / scale, hv[a][4 * g + 3] / scale);
        const int col = wn * (BN / 2 / WN) + 8 * g + 4 * (lane >> 5);
        *reinterpret_cast<uint32_t*>(stg + stg128(row, col)) = pk;
      }
      if (wn == 0 && lane < 32 && row < rows)
        p.qscale[int64_t(base + m0 + row) * (p.N / 128) + ct] = scale;
    }
    (void)am;
    __syncthreads();
    for (int i = tid; i < rows * 8; i += NT) {
      const int row = i >> 3, c = i & 7;
      *reinterpret_cast<uint4*>(p.qout + int64_t(base + m0 + row) * p.N + ct * 128 + c * 16) =
          *reinterpret_cast<const uint4*>(stg + stg128(row, c * 16));
    }
    return;
  }
  if (p.out32) {
#pragma unroll
    for (int a = 0; a < MI; ++a) {
      const int row = wm * (BM / WM) + a * 32 + (lane & 31);
      if (row >= rows) continue;
#pragma unroll
      for (int b = 0; b < NI; ++b)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = ct * BN + wn * (BN / WN) + b * 32 + 8 * g + 4 * (lane >> 5);
          *reinterpret_cast<float4*>(p.out32 + int64_t(base + m0 + row) * p.N + col) =
              make_float4(acc[a][b][4 * g], acc[a][b][4 * g + 1], acc[a][b][4 * g + 2], acc[a][b][4 * g + 3]);
        }
    }
    return;
  }
  // weighted bf16 rows through LDS: each register group is 4 consecutive columns
  constexpr int LS = BN + 8;
  bf16_t* stg = reinterpret_cast<bf16_t*>(smem);
#pragma unroll
  for (int a = 0; a < MI; ++a) {
    const int row = wm * (BM / WM) + a * 32 + (lane & 31);
    const float wr = row < rows ? p.row_w[base + m0 + row] : 0.f;
#pragma unroll
    for (int b = 0; b < NI; ++b)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * (BN / WN) + b * 32 + 8 * g + 4 * (lane >> 5);
        uint2 pk;
        pk.x = uint32_t(f32_to_bf16(acc[a][b][4 * g] * wr)) | (uint32_t(f32_to_bf16(acc[a][b][4 * g + 1] * wr)) << 16);
        pk.y = uint32_t(f32_to_bf16(acc[a][b][4 * g + 2] * wr)) | (uint32_t(f32_to_bf16(acc[a][b][4 * g + 3] * wr)) << 16);
        *reinterpret_cast<uint2*>(stg + row * LS + col) = pk;
      }
  }
  __syncthreads();
  for (int i = tid; i < rows * (BN / 8); i += NT) {
    const int row = i / (BN / 8), c = i - row * (BN / 8);
    *reinterpret_cast<uint4*>(p.out16 + int64_t(base + m0 + row) * p.N + ct * BN + c * 8) =
        *reinterpret_cast<const uint4*>(stg + row * LS + c * 8);
  }
}

// ---------------------------------------------------------------------------
// Block FP8 down projection, persistent.  The same tile, ring, MFMA steps and
// epilogues as k_gemm_fp8_v2<false>, but one workgroup per CU walks a run of items, so
// that a tile's first two slabs are loaded while the previous tile's epilogue runs.
// Phase stamps of the one-tile-per-workgroup kernels put 23% of a gate/up tile's time
// in its prologue (the set-up loads, then the first slabs' latency) and 19% in its
// epilogue, with one workgroup per CU and nothing else to overlap them; with K = I
// (four 128-deep slabs per tile) the down tile is dominated by them (47.5 -> 43 us on
// the 2048-token layer), while the gate/up tile's twelve slabs leave the persistent
// form no gain (67.9 against 66.2 us), so gate/up keeps k_gemm_fp8_v2.
// Items: the n = tiles x column blocks of the launch (tile-major) are split into 8
// contiguous runs, one per XCD (workgroup b runs on XCD b % 8), and the P workgroups
// of an XCD take items q, q + P, q + 2P, ... of their run, so the items in flight on
// an XCD at any time are neighbours, as the hardware's in-order dispatch would have
// them.  The scales ride in the ring: with each slab, waves 0-1 load the 128 rows'
// activation scales and the other waves the slab's weight block scales (4-byte
// direct-to-LDS loads), so every wait counts the same L + 1 loads per slab.
__global__ __launch_bounds__(Fp8Tile::NT) __attribute__((amdgpu_waves_per_eu(2)))
void k_gemm_fp8_down_p(GemmFp8Args p) {
  using C = Fp8Tile;
  constexpr int BM = C::BM, BN = C::BN, W = C::W, WM = C::WM, WN = C::WN, MI = C::MI, NI = C::NI;
  constexpr int AJ = C::AJ, BJ = C::BJ, L = C::L + 1, NT = C::NT;
  __shared__ uint4 smem[C::RING_U4];
  __shared__ float sa_r[3][BM];          // activation scales of the slab in each ring slot
  __shared__ float sw_r[3][2];           // weight block scales of the slab in each ring slot
  const int ncol = p.N / BN;
  const int n = p.meta[1] * ncol;
  const int per = (n + 7) >> 3;
  const int run0 = int(blockIdx.x & 7) * per, q0 = int(blockIdx.x >> 3), P = int(gridDim.x >> 3);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (scalar registers)
  const int wm = wv / WN, wn = wv % WN;
  const int64_t K = p.K;
  const int nk = int(K / C::KB);
  const int64_t mst = int64_t(p.N) * K;                // bytes of one expert matrix
  const int64_t sst = int64_t(p.N / 128) * nk;         // block scales of one expert matrix
  // Workgroup barrier for LDS hand-offs: waits for this wave's LDS operations only, not
  // for its global loads (the next item's slabs stay in flight across the epilogue's
  // barriers) nor its stores.
  auto lds_sync = [] {
    wait_vm_lgkm0<63>();
    block_sync_nowait();
  };
  auto item_of = [&](int tau, int& tile, int& ct) {
    const int q = q0 + P * tau, j = run0 + q;
    if (q >= per || j >= n) return false;
    tile = j / ncol;
    ct = j - tile * ncol;
    return true;
  };

  // ------------------------------------------------------------- issue side
  const uint8_t* ag[AJ];
  const uint8_t* bbase[BJ];                             // weight matrix of each load (wave-uniform)
  uint32_t boff[BJ];                                    // this lane's byte offset in it
  const float* scs;                                     // this lane's scale source (+ kt)
  int src_m0, src_base, src_cnt;                        // the item's rows
  auto set_source = [&](int tile, int ct) {
    const int2 te = p.tiles[tile];
    const int e = te.x, m0 = te.y;
    const int base = p.offsets[e];
    const int cnt = p.offsets[e + 1] - base;
    src_m0 = m0;
    src_base = base;
    src_cnt = cnt;
    auto arow_of = [&](int r) {
      const int m = min(m0 + r, cnt - 1);
      return int64_t(base + m);
    };
#pragma unroll
    for (int i = 0; i < AJ; ++i) {
      const int r = 8 * (wv + W * i) + (lane >> 3);
      ag[i] = p.a + arow_of(r) * K + dma_chunk(lane, wv + W * i) * 16;
    }
#pragma unroll
    for (int i = 0; i < BJ; ++i) {
      const int r0 = 8 * (wv + W * i), r = r0 + (lane >> 3);   // a load's rows: r0 .. r0+7
      const int c = dma_chunk(lane, wv + W * i) * 16;
      bbase[i] = expert_mat(p.w0, p.sh0, e, p.E, mst);
      boff[i] = uint32_t((ct * BN + r) * K + c);
    }
    if (wv < 2) {
      scs = p.a_scale + arow_of(wv * 64 + lane) * nk;
    } else {
      // the two 128-row scale blocks 2ct, 2ct+1 of the tile's 256 output columns
      scs = expert_mat(p.s0, p.shs0, e, p.E, sst) + int64_t(2 * ct + (lane & 1)) * nk;
    }
  };
  auto issue = [&](int kt, int slot) {
    const int64_t ko = int64_t(kt) * C::KB;
    uint4* sa = smem + slot * C::STAGE_U4;
    uint4* sb = sa + C::A_U4;
#pragma unroll
    for (int i = 0; i < AJ; ++i) dma16(ag[i] + ko, sa + (wv + W * i) * 64);
#pragma unroll
    for (int i = 0; i < BJ; ++i) dma16(bbase[i] + (boff[i] + ko), sb + (wv + W * i) * 64);
    if (wv < 2) {
      dma4(scs + kt, &sa_r[slot][wv * 64]);
    } else if (lane < 2) {
      dma4(scs + kt, &sw_r[slot][0]);
    }
  };

  // ------------------------------------------------------------- compute side
  auto wrow = [&](int b) { return wn * (BN / WN) + b * 32 + (lane & 31); };
  const int swb0 = (wn * (BN / WN)) / 128;            // scale block of this wave's weight rows
  f32x16 acc[MI][NI];
  auto compute = [&](int slot, auto&& between) {
    const uint4* sa = smem + slot * C::STAGE_U4;
    const uint4* sb = sa + C::A_U4;
    i32x8 af[2][MI], bfr[2][NI];
    auto frags = [&](int ks, i32x8 (&xa)[MI], i32x8 (&xb)[NI]) {
      const int c0 = ks * 4 + (lane >> 5) * 2;
#pragma unroll
      for (int a = 0; a < MI; ++a) {
        const int row = wm * (BM / WM) + a * 32 + (lane & 31);
        const uint4 lo = sa[swz16(row, c0)], hi = sa[swz16(row, c0 + 1)];
        xa[a] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      }
#pragma unroll
      for (int b = 0; b < NI; ++b) {
        const int row = wrow(b);
        const uint4 lo = sb[swz16(row, c0)], hi = sb[swz16(row, c0 + 1)];
        xb[b] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      }
    };
    frags(0, af[0], bfr[0]);
    __builtin_amdgcn_sched_barrier(0);
    between();
    frags(1, af[1], bfr[1]);
    __builtin_amdgcn_sched_barrier(0);
    float sact[MI], swt[NI];
#pragma unroll
    for (int a = 0; a < MI; ++a) sact[a] = sa_r[slot][wm * (BM / WM) + a * 32 + (lane & 31)];
#pragma unroll
    for (int b = 0; b < NI; ++b) swt[b] = sw_r[slot][swb0];
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
      for (int b = 0; b < NI; ++b) {
        f32x16 sl;
#pragma unroll
        for (int r = 0; r < 16; ++r) sl[r] = 0.f;
        sl = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[0][b], af[0][a], sl, 0, 0, 0, 127, 0, 127);
        sl = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[1][b], af[1][a], sl, 0, 0, 0, 127, 0, 127);
        const float s = sact[a] * swt[b];
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = fmaf(sl[r], s, acc[a][b][r]);
      }
  };

  int tile, ct;
  if (!item_of(0, tile, ct)) return;
  set_source(tile, ct);
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int tau = 0;; ++tau) {
    const int m0 = src_m0, base = src_base, cnt = src_cnt;
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
      for (int b = 0; b < NI; ++b)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    // Every item runs its ring from slot 0 (slab kt in slot kt % 3, slots fixed at
    // compile time by the unrolled steps).  After an epilogue its stores are in the
    // count too, so an item's first step waits for everything.
#define MOE_F8P_STEP(KT, SLOT, NSLOT)                                                      \
    {                                                                                      \
      if ((KT) + 1 < nk && !((KT) == 0 && tau > 0)) wait_vm_lgkm0<L>(); else wait_vm_lgkm0<0>(); \
      block_sync_nowait();                                                                 \
      compute(SLOT, [&] { if ((KT) + 2 < nk) issue((KT) + 2, NSLOT); });                   \
    }
    for (int kt = 0; kt < nk; kt += 3) {
      MOE_F8P_STEP(kt, 0, 2)
      if (kt + 1 < nk) MOE_F8P_STEP(kt + 1, 1, 0)
      if (kt + 2 < nk) MOE_F8P_STEP(kt + 2, 2, 1)
    }
#undef MOE_F8P_STEP
    // The next item's set-up loads are waited for here, where no slab is in flight, by
    // each wave before the barrier; once every wave has passed it the whole ring is
    // free: the next item's first two slabs go into slots 0 and 1 and the epilogue
    // stages through slot 2 while they land.
    const int cur_ct = ct;
    // down, weighted output: this wave's row weights, loaded before the next item's
    // slabs are issued (a load waited for in the epilogue would wait for them too)
    float wrv[MI];
#pragma unroll
    for (int a = 0; a < MI; ++a) {
      const int row = wm * (BM / WM) + a * 32 + (lane & 31);
      wrv[a] = (p.out32 || row >= cnt - m0) ? 0.f : p.row_w[base + m0 + row];
    }
    const bool more = item_of(tau + 1, tile, ct);
    if (more) set_source(tile, ct);
    wait_vm_lgkm0<0>();   // those loads have landed before any slab load is issued behind them
    lds_sync();
    if (more) {
      issue(0, 0);
      if (nk > 1) issue(1, 1);
    }
    const int rows = min(BM, cnt - m0);
    unsigned char* stage = reinterpret_cast<unsigned char*>(smem + 2 * C::STAGE_U4);
    if (p.out32) {
#pragma unroll
      for (int a = 0; a < MI; ++a) {
        const int row = wm * (BM / WM) + a * 32 + (lane & 31);
        if (row >= rows) continue;
#pragma unroll
        for (int b = 0; b < NI; ++b)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int col = cur_ct * BN + wn * (BN / WN) + b * 32 + 8 * g4 + 4 * (lane >> 5);
            *reinterpret_cast<float4*>(p.out32 + int64_t(base + m0 + row) * p.N + col) =
                make_float4(acc[a][b][4 * g4], acc[a][b][4 * g4 + 1], acc[a][b][4 * g4 + 2],
                            acc[a][b][4 * g4 + 3]);
          }
      }
    } else {
      // weighted bf16 rows through LDS, one 64-row half of the tile at a time (the
      // staging slot holds 48 KB): each register group is 4 consecutive columns
      constexpr int LS = BN + 8;
      bf16_t* stg = reinterpret_cast<bf16_t*>(stage);
#pragma unroll
      for (int half = 0; half < WM; ++half) {
        if (wm == half) {
#pragma unroll
          for (int a = 0; a < MI; ++a) {
            const int lrow = a * 32 + (lane & 31);
            const float wr = wrv[a];
#pragma unroll
            for (int b = 0; b < NI; ++b)
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                const int col = wn * (BN / WN) + b * 32 + 8 * g4 + 4 * (lane >> 5);
                uint2 pk;
                pk.x = uint32_t(f32_to_bf16(acc[a][b][4 * g4] * wr)) |
                       (uint32_t(f32_to_bf16(acc[a][b][4 * g4 + 1] * wr)) << 16);
                pk.y = uint32_t(f32_to_bf16(acc[a][b][4 * g4 + 2] * wr)) |
                       (uint32_t(f32_to_bf16(acc[a][b][4 * g4 + 3] * wr)) << 16);
                *reinterpret_cast<uint2*>(stg + lrow * LS + col) = pk;
              }
          }
        }
        lds_sync();
        const int hrows = min(BM / WM, rows - half * (BM / WM));
        for (int i = tid; i < hrows * (BN / 8); i += NT) {
          const int lrow = i / (BN / 8), c = i - lrow * (BN / 8);
          *reinterpret_cast<uint4*>(p.out16 + int64_t(base + m0 + half * (BM / WM) + lrow) * p.N +
                                    cur_ct * BN + c * 8) =
              *reinterpret_cast<const uint4*>(stg + lrow * LS + c * 8);
        }
        if (half + 1 < WM) lds_sync();
      }
    }
    if (!more) break;
  }
}


// shapes the pipelined fp8 kernels cover
static bool fp8_pipelined_ok(const Plan& p) {
  return p.wt == MOE_E4M3_B128 && p.I % 128 == 0 && p.H % Fp8Tile::BN == 0 &&
         p.H / 128 <= Fp8Tile::SMAX && p.I / 128 <= Fp8Tile::SMAX;
}

// Block-FP8 activations (x, or h in the register-staged path): quant_e4m3_wave per
// wave, 16 blocks of 128 per workgroup of 256.
template <typename TI>
__global__ __launch_bounds__(256) void k_quant_e4m3(const TI* __restrict__ in, int64_t rows, int K,
                                                    uint8_t* __restrict__ codes,
                                                    float* __restrict__ scales) {
  quant_e4m3_wave(in, rows, K, codes, scales, int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6));
}

// ===========================================================================
int launch_gateup_mfma(const Plan& p, const void* x, const int32_t* row_token,
                       const int32_t* offsets, const int2* tiles, const int32_t* meta,
                       const moe_weights* w, void* h, const uint8_t* xq, const float* sx,
                       uint8_t* hq, float* shq, hipStream_t st) {
  const unsigned grid = xcd_grid(p.max_tiles * (p.I / 64));
  if (p.wt == MOE_BF16) {
    GemmBf16Args a{};
    a.a = (const bf16_t*)x; a.row_token = row_token; a.offsets = offsets; a.tiles = tiles;
    a.meta = meta; a.w0 = (const bf16_t*)w->w_gate; a.w1 = (const bf16_t*)w->w_up;
    a.sh0 = (const bf16_t*)w->sh_gate; a.sh1 = (const bf16_t*)w->sh_up;
    a.out16 = (bf16_t*)h; a.K = p.H; a.N = p.I; a.E = p.E; a.ES = p.E + p.S;
    if (bf_pipelined_ok(p) && MOE_BF_GU_PERSIST) {
      unsigned pg = 0;
      MOE_TRY(persistent_grid(&pg));
      launch_kernel(p, kTimeGateUp, k_gemm_bf16_gateup_p, dim3(pg), dim3(BfCfg::NT), 0, st, a);
    } else if (bf_pipelined_ok(p))
      launch_kernel(p, kTimeGateUp, k_gemm_bf16_v2<true, BfCfg>,
                    dim3(xcd_grid(p.max_tiles * (p.I / (BfCfg::BN / 2)))), dim3(BfCfg::NT), 0, st, a);
    else
      launch_kernel(p, kTimeGateUp, k_gemm_bf16<true>, dim3(grid), dim3(256), 0, st, a);
  } else if (p.wt == MOE_NVFP4) {
    GemmNv4Args a{};
    a.a = (const bf16_t*)x; a.row_token = row_token; a.offsets = offsets; a.tiles = tiles;
    a.meta = meta;
    a.w0 = (const uint8_t*)w->w_gate; a.w1 = (const uint8_t*)w->w_up;
    a.sh0 = (const uint8_t*)w->sh_gate; a.sh1 = (const uint8_t*)w->sh_up;
    a.b0 = w->b_gate; a.b1 = w->b_up; a.shb0 = w->sh_b_gate; a.shb1 = w->sh_b_up;
    a.g0 = w->g_gate; a.g1 = w->g_up; a.shg0 = w->sh_g_gate; a.shg1 = w->sh_g_up;
    a.out16 = (bf16_t*)h; a.K = p.H; a.N = p.I; a.E = p.E;
    launch_kernel(p, kTimeGateUp, k_gemm_nv4<true>,
                  dim3(xcd_grid(p.max_tiles * (p.I / (Nv4Cfg::BN / 2)))), dim3(Nv4Cfg::NT), 0, st, a);
  } else {
    GemmFp8Args a{};
    a.a = xq; a.a_scale = sx; a.row_token = row_token; a.offsets = offsets; a.tiles = tiles;
    a.meta = meta; a.w0 = (const uint8_t*)w->w_gate; a.w1 = (const uint8_t*)w->w_up;
    a.sh0 = (const uint8_t*)w->sh_gate; a.sh1 = (const uint8_t*)w->sh_up;
    a.s0 = w->s_gate; a.s1 = w->s_up; a.shs0 = w->sh_s_gate; a.shs1 = w->sh_s_up;
    a.hout = (float*)h; a.qout = hq; a.qscale = shq; a.K = p.H; a.N = p.I; a.E = p.E;
    if (fp8_pipelined_ok(p)) {
      launch_kernel(p, kTimeGateUp, k_gemm_fp8_v2<true>,
                    dim3(xcd_grid(p.max_tiles * (p.I / (Fp8Tile::BN / 2)))), dim3(Fp8Tile::NT), 0, st, a);
      return check_launch();
    }
    launch_kernel(p, kTimeGateUp, k_gemm_fp8<true>, dim3(grid), dim3(256), 0, st, a);
    MOE_TRY(check_launch());
    return launch_quant(p, h, false, p.R, p.I, hq, shq, st);
  }
  return check_launch();
}

int launch_down_mfma(const Plan& p, const void* h, const int32_t* offsets, const int2* tiles,
                     const int32_t* meta, const moe_weights* w, const float* row_w, float* out32,
                     bf16_t* out16, const float* sh_scale, hipStream_t st) {
  const unsigned grid = xcd_grid(p.max_tiles * (p.H / TN));
  if (p.wt == MOE_BF16) {
    GemmBf16Args a{};
    a.a = (const bf16_t*)h; a.offsets = offsets; a.tiles = tiles; a.meta = meta;
    a.w0 = (const bf16_t*)w->w_down; a.sh0 = (const bf16_t*)w->sh_down;
    a.row_w = row_w; a.out16 = out16; a.out32 = out32; a.K = p.I; a.N = p.H; a.E = p.E;
    a.ES = p.E + p.S;
    // (k_gemm_bf16_v2<false> is the same tile one per workgroup; the persistent form
    // measured 153.3 against 160.9 us on the Inkling-shaped layer, equal on prefill)
    if (bf_pipelined_ok(p)) {
      unsigned pg = 0;
      MOE_TRY(persistent_grid(&pg));
      launch_kernel(p, kTimeDown, k_gemm_bf16_down_p, dim3(pg), dim3(BfCfg::NT), 0, st, a);
    } else
      launch_kernel(p, kTimeDown, k_gemm_bf16<false>, dim3(grid), dim3(256), 0, st, a);
  } else if (p.wt == MOE_NVFP4) {
    GemmNv4Args a{};
    a.a = (const bf16_t*)h; a.offsets = offsets; a.tiles = tiles; a.meta = meta;
    a.w0 = (const uint8_t*)w->w_down; a.sh0 = (const uint8_t*)w->sh_down;
    a.b0 = w->b_down; a.shb0 = w->sh_b_down; a.g0 = w->g_down; a.shg0 = w->sh_g_down;
    a.row_w = row_w; a.out16 = out16; a.out32 = out32; a.K = p.I; a.N = p.H; a.E = p.E;
    launch_kernel(p, kTimeDown, k_gemm_nv4<false>,
                  dim3(xcd_grid(p.max_tiles * (p.H / Nv4Cfg::BN))), dim3(Nv4Cfg::NT), 0, st, a);
  } else {
    GemmFp8Args a{};
    a.a = (const uint8_t*)h; a.a_scale = sh_scale; a.offsets = offsets; a.tiles = tiles;
    a.meta = meta; a.w0 = (const uint8_t*)w->w_down; a.sh0 = (const uint8_t*)w->sh_down;
    a.s0 = w->s_down; a.shs0 = w->sh_s_down; a.row_w = row_w; a.out16 = out16; a.out32 = out32;
    a.K = p.I; a.N = p.H; a.E = p.E;
    if (fp8_pipelined_ok(p)) {
      unsigned pg = 0;
      MOE_TRY(persistent_grid(&pg));
      launch_kernel(p, kTimeDown, k_gemm_fp8_down_p, dim3(pg), dim3(Fp8Tile::NT), 0, st, a);
    } else {
      launch_kernel(p, kTimeDown, k_gemm_fp8<false>, dim3(grid), dim3(256), 0, st, a);
    }
  }
  return check_launch();
}

int launch_quant(const Plan& p, const void* in, bool in_bf16, int64_t rows, int K, uint8_t* codes,
                 float* scales, hipStream_t st) {
  const int64_t n = rows * (K / 128);
  if (n == 0) return MOE_OK;
  const unsigned grid = unsigned((n + 15) / 16);   // 16 blocks of 128 per workgroup
  if (in_bf16)
    hipLaunchKernelGGL(k_quant_e4m3<bf16_t>, dim3(grid), dim3(256), 0, st, (const bf16_t*)in, rows,
                       K, codes, scales);
  else
    hipLaunchKernelGGL(k_quant_e4m3<float>, dim3(grid), dim3(256), 0, st, (const float*)in, rows, K,
                       codes, scales);
  (void)p;
  return check_launch();
}

}  // namespace moe
