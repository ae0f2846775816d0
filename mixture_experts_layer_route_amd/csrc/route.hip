// Router: logits, group-limited top-k and renormalised weights.
//
// Group-limited routing is named in TensorFold issue #1247 "Ling-3.0-tiny on a
// Qualcomm board" (jschmied's comment, list "What it does not cover"); its config
// paragraph fixes 128 experts in 8 groups of 16 with 4 groups kept, and the
// HelloSun/ling30tiny routing table (模型與路由) fixes 8 experts per token.  The
// pages do not name the score function; the layer takes the softmax of the
// logits, a group's score is its best expert score, ties go to the lower index
// and the chosen weights are renormalised to sum 1.
//
// Two logits kernels: a vector-FMA one for few tokens or fp32 layers (activation
// rows staged in LDS, every weight load of a wave issued before any is used), and
// a matrix-core one for bf16 batches that also selects the experts of its 64
// tokens (one thread each) and counts them per 64-token block for the
// permutation.
#include <algorithm>

#include "moe_internal.h"
#include "route_select.h"

namespace moe {

// ---------------------------------------------------------------------------
// Vector-FMA logits.  grid = (ceil(E/4), ceil(T/RT)), block = 256, dynamic LDS =
// RT * H * sizeof(TA) (RT <= 16).  Wave w of block (bx, by) computes expert
// 4*bx + w for tokens [by*RT, by*RT + RT).
template <typename TA>
__global__ __launch_bounds__(256) void k_router_logits_fma(
    const TA* __restrict__ x, const TA* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int64_t T, int H, int E, int RT) {
  constexpr int RTMAX = 16, SMAX = 4;                 // H <= 2048 per pass
  extern __shared__ __align__(16) unsigned char lds_raw[];
  TA* xs = reinterpret_cast<TA*>(lds_raw);
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int64_t t0 = int64_t(blockIdx.y) * RT;
  const int nt = int(min<int64_t>(RT, T - t0));
  const bool live = e < E;
  const TA* wrow = wr + int64_t(live ? e : 0) * H;
  float acc[RTMAX];
#pragma unroll
  for (int q = 0; q < RTMAX; ++q) acc[q] = 0.f;
  for (int hb = 0; hb < H; hb += 512 * SMAX) {
    const int hw = min(H - hb, 512 * SMAX);
    float wv[SMAX][8];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int h = s * 512 + lane * 8;
      if (h < hw) load8(wrow + hb + h, wv[s]);
    }
    // stage this pass of the token rows (16-byte chunks)
    constexpr int CH = 16 / sizeof(TA);
    const int chunks = nt * hw / CH;
    for (int c = threadIdx.x; c < chunks; c += 256) {
      const int q = c / (hw / CH), h = (c - q * (hw / CH)) * CH;
      *reinterpret_cast<uint4*>(xs + q * hw + h) =
          *reinterpret_cast<const uint4*>(x + (t0 + q) * H + hb + h);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int h = s * 512 + lane * 8;
      if (h < hw) {
#pragma unroll
        for (int q = 0; q < RTMAX; ++q) {
          if (q < nt) {
            float xv[8];
            load8(xs + q * hw + h, xv);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[q] = fmaf(xv[i], wv[s][i], acc[q]);
          }
        }
      }
    }
    __syncthreads();
  }
  if (!live) return;
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int q = 0; q < RTMAX; ++q) {
    if (q < nt) {
      const float s = wave_sum(acc[q]);
      if (lane == 0) logits[(t0 + q) * E + e] = s + b;
    }
  }
}

// ---------------------------------------------------------------------------
// Thread-per-token selection over global logits, 256 tokens per block, plus the
// per-64-token-block expert counts used by the permutation (when blk != null).
// grid = ceil(T/256), block = 256, dynamic LDS = (4*E + 256*G) * 4 bytes.
template <int K>
__global__ __launch_bounds__(256) void k_router_select(
    const float* __restrict__ logits, int64_t T, int E, int G, int Gk, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ blk) {
  extern __shared__ int sel_lds[];
  int* cnt = sel_lds;                                        // [4][E]
  float* gs = reinterpret_cast<float*>(sel_lds + 4 * E);     // [G][256]
  const int wv = threadIdx.x >> 6;
  for (int i = threadIdx.x; i < 4 * E; i += 256) cnt[i] = 0;
  __syncthreads();
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (t < T) {
    int32_t id[K];
    float wt[K];
    select_token_thread<K>(logits + t * E, 1, E, G, Gk, gs + threadIdx.x, 256, id, wt);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      ids[t * K + j] = id[j];
      w[t * K + j] = wt[j];
      if (blk) atomicAdd(&cnt[wv * E + id[j]], 1);
    }
  }
  __syncthreads();
  if (!blk) return;
  for (int i = threadIdx.x; i < 4 * E; i += 256) {
    const int64_t b = int64_t(blockIdx.x) * 4 + i / E;
    if (b * 64 < T) blk[b * E + (i % E)] = cnt[i];
  }
}

// ---------------------------------------------------------------------------
// Matrix-core logits for bf16 batches, E = 128*NE experts, 64 tokens per block:
// l = X W_r^T with v_mfma_f32_32x32x16_bf16.  H moves global -> LDS in slabs of
// 64 through a 3-stage ring of direct-to-LDS loads (lane L of a load fills row
// L/8, slot L%8 with logical chunk (L%8)^(L/8)); wave w owns experts
// [32*NE*w, 32*NE*(w+1)).  The logits tile then overlays the ring in LDS, wave 0
// selects the experts of the 64 tokens (one thread each) and the block's expert
// counts are written for the permutation.  grid = ceil(T/64), block = 256.
typedef __attribute__((address_space(3))) void lvoid_t;
__device__ __forceinline__ void dma16_r(const void* g, void* lds) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(uint32_t(reinterpret_cast<uintptr_t>((lvoid_t*)lds)));
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tglobal_load_lds_dwordx4 %2, off\n\ts_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(g)
      : "memory");
}
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0_r() {
  __builtin_amdgcn_s_waitcnt((N & 0xF) | (0x7 << 4) | ((N >> 4) << 14));
}

template <int NE, int K>
__global__ __launch_bounds__(256) void k_router_mfma(
    const bf16_t* __restrict__ x, const bf16_t* __restrict__ wr, const float* __restrict__ bias,
    int64_t T, int H, int G, int Gk, float* __restrict__ logits_out, int32_t* __restrict__ ids,
    float* __restrict__ w, int32_t* __restrict__ blk) {
  constexpr int E = 128 * NE, BT = 64, LDL = E + 1;
  constexpr int XU4 = BT * 8, WU4 = E * 8, STU4 = XU4 + WU4;          // uint4 per stage
  constexpr int RING_BYTES = 3 * STU4 * 16;
  constexpr int LG_BYTES = BT * LDL * 4 + BT * 64 * 4 + E * 4;        // logits + group scratch + counts
  constexpr int LDS_BYTES = RING_BYTES > LG_BYTES ? RING_BYTES : LG_BYTES;
  constexpr int AJ = BT / 32, BJ = E / 32, L = AJ + BJ;                // loads per lane per slab
  __shared__ __align__(16) uint4 ring[LDS_BYTES / 16];
  float* lg = reinterpret_cast<float*>(ring);                          // after the K loop
  float* gs = lg + BT * LDL;
  int* cnt = reinterpret_cast<int*>(gs + BT * 64);

  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int64_t t0 = int64_t(blockIdx.x) * BT;
  const bf16_t* xg[AJ];
#pragma unroll
  for (int i = 0; i < AJ; ++i)
    xg[i] = x + min<int64_t>(t0 + 8 * (wv + 4 * i) + (lane >> 3), T - 1) * H +
            dma_chunk(lane, wv + 4 * i) * 8;
  const bf16_t* wg[BJ];
#pragma unroll
  for (int i = 0; i < BJ; ++i)
    wg[i] = wr + int64_t(8 * (wv + 4 * i) + (lane >> 3)) * H + dma_chunk(lane, wv + 4 * i) * 8;
  auto issue = [&](int kt, int stage) {
    uint4* st = ring + stage * STU4;
    const int ko = kt * 64;
#pragma unroll
    for (int i = 0; i < AJ; ++i) dma16_r(xg[i] + ko, st + (wv + 4 * i) * 64);
#pragma unroll
    for (int i = 0; i < BJ; ++i) dma16_r(wg[i] + ko, st + XU4 + (wv + 4 * i) * 64);
  };

  f32x16 acc[2][NE];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < NE; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  auto compute = [&](int stage) {
    const uint4* xc = ring + stage * STU4;
    const uint4* wc = xc + XU4;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int chunk = ks * 2 + (lane >> 5);
      bf16x8 af[2], bfr[NE];
#pragma unroll
      for (int a = 0; a < 2; ++a)
        af[a] = __builtin_bit_cast(bf16x8, xc[swz16(a * 32 + (lane & 31), chunk)]);
#pragma unroll
      for (int b = 0; b < NE; ++b)
        bfr[b] = __builtin_bit_cast(bf16x8, wc[swz16(wv * 32 * NE + b * 32 + (lane & 31), chunk)]);
#pragma unroll
      for (int a = 0; a < 2; ++a)
#pragma unroll
        for (int b = 0; b < NE; ++b)
          acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[a], bfr[b], acc[a][b], 0, 0, 0);
    }
  };
  const int nk = H / 64;
  issue(0, 0);
  if (nk > 1) issue(1, 1);
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + 1 < nk) wait_vm_lgkm0_r<L>(); else wait_vm_lgkm0_r<0>();
    block_sync_nowait();
    if (kt + 2 < nk) issue(kt + 2, (kt + 2) % 3);
    compute(kt % 3);
  }
  wait_vm_lgkm0_r<0>();
  block_sync_nowait();      // every wave is done with the ring before it is overlaid

  // logits tile -> LDS [token][expert] (stride E+1), bias added
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int b = 0; b < NE; ++b) {
      const int e = wv * 32 * NE + b * 32 + (lane & 31);
      const float be = bias ? bias[e] : 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int t = a * 32 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
        lg[t * LDL + e] = acc[a][b][r] + be;
      }
    }
  for (int i = tid; i < E; i += 256) cnt[i] = 0;
  __syncthreads();
  const int nt = int(min<int64_t>(BT, T - t0));
  if (logits_out)
    for (int i = tid; i < nt * E; i += 256) logits_out[t0 * E + i] = lg[(i / E) * LDL + i % E];
  if (wv == 0 && lane < nt) {
    const int64_t t = t0 + lane;
    int32_t id[K];
    float wt[K];
    select_token_thread<K>(lg + lane * LDL, 1, E, G, Gk, gs + lane, 64, id, wt);
#pragma unroll
    for (int j = 0; j < K; ++j) {
      ids[t * K + j] = id[j];
      w[t * K + j] = wt[j];
      atomicAdd(&cnt[id[j]], 1);
    }
  }
  __syncthreads();
  if (blk)
    for (int i = tid; i < E; i += 256) blk[int64_t(blockIdx.x) * E + i] = cnt[i];
}

// ---------------------------------------------------------------------------
bool router_mfma_ok(const Plan& p) {
  return p.act == MOE_BF16 && (p.E == 128 || p.E == 256) && p.H % 64 == 0 && p.G <= 64 &&
         p.T > 16;
}

int launch_logits(const Plan& p, const void* x, const void* wr, const float* bias, float* logits,
                  hipStream_t st) {
  const int tsize = p.act == MOE_F32 ? 4 : 2;
  const int hpass = std::min(p.H, 2048);
  const int RT = int(std::max<int64_t>(1, std::min<int64_t>(16, 32768 / (int64_t(hpass) * tsize))));
  const dim3 grid((p.E + 3) / 4, unsigned((p.T + RT - 1) / RT));
  const size_t lds = size_t(RT) * hpass * tsize;
  if (p.act == MOE_F32)
    hipLaunchKernelGGL(k_router_logits_fma<float>, grid, dim3(256), lds, st, (const float*)x,
                       (const float*)wr, bias, logits, p.T, p.H, p.E, RT);
  else
    hipLaunchKernelGGL(k_router_logits_fma<bf16_t>, grid, dim3(256), lds, st, (const bf16_t*)x,
                       (const bf16_t*)wr, bias, logits, p.T, p.H, p.E, RT);
  return check_launch();
}

#define MOE_K_SWITCH(K_VAL, MACRO) \
  switch (K_VAL) {                 \
    case 1: MACRO(1); break;       \
    case 2: MACRO(2); break;       \
    case 3: MACRO(3); break;       \
    case 4: MACRO(4); break;       \
    case 5: MACRO(5); break;       \
    case 6: MACRO(6); break;       \
    case 7: MACRO(7); break;       \
    case 8: MACRO(8); break;       \
    case 9: MACRO(9); break;       \
    case 10: MACRO(10); break;     \
    case 11: MACRO(11); break;     \
    case 12: MACRO(12); break;     \
    case 13: MACRO(13); break;     \
    case 14: MACRO(14); break;     \
    case 15: MACRO(15); break;     \
    default: MACRO(16); break;     \
  }

int launch_select(const Plan& p, const float* logits, int32_t* ids, float* w, int32_t* blk,
                  hipStream_t st) {
  const dim3 grid(unsigned((p.T + 255) / 256));
  const size_t lds = (size_t(4) * p.E + size_t(256) * p.G) * 4;
#define MOE_SEL(KK)                                                                        \
  hipLaunchKernelGGL(k_router_select<KK>, grid, dim3(256), lds, st, logits, p.T, p.E, p.G, \
                     p.Gk, ids, w, blk)
  MOE_K_SWITCH(p.k, MOE_SEL)
#undef MOE_SEL
  return check_launch();
}

int launch_router_mfma(const Plan& p, const void* x, const void* wr, const float* bias,
                       float* logits_out, int32_t* ids, float* w, int32_t* blk, hipStream_t st) {
  const dim3 grid(unsigned((p.T + 63) / 64));
#define MOE_RM(KK)                                                                            \
  if (p.E == 128)                                                                             \
    hipLaunchKernelGGL((k_router_mfma<1, KK>), grid, dim3(256), 0, st, (const bf16_t*)x,     \
                       (const bf16_t*)wr, bias, p.T, p.H, p.G, p.Gk, logits_out, ids, w, blk); \
  else                                                                                        \
    hipLaunchKernelGGL((k_router_mfma<2, KK>), grid, dim3(256), 0, st, (const bf16_t*)x,     \
                       (const bf16_t*)wr, bias, p.T, p.H, p.G, p.Gk, logits_out, ids, w, blk)
  MOE_K_SWITCH(p.k, MOE_RM)
#undef MOE_RM
  return check_launch();
}

}  // namespace moe
