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
// a matrix-core one for bf16 batches; then one selection kernel (a wave per
// token) that also counts the chosen experts per 64-token block for the
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
// Logits for a few tokens (T <= 16): one wave per expert, every load of the
// expert's row chunks and of the token rows issued from global memory before
// any is used (one memory round trip per TQ tokens and SMAX 512-wide chunks of
// the hidden units: 16 x 1, 8 x 2 or 4 x 4 by H), then a DPP reduction per token.
// The waves share nothing, so each is a workgroup of its own and the experts spread
// over E CUs (every wave loads all T token rows; four waves to a workgroup measured
// 0.1-0.3 us slower per decode step).  grid = ceil(E / MOE_LOGITS_FEW_WAVES),
// block = 64 MOE_LOGITS_FEW_WAVES.
#ifndef MOE_LOGITS_FEW_WAVES
#define MOE_LOGITS_FEW_WAVES 1
#endif
template <typename TA, int TQ, int SMAX>
__global__ __launch_bounds__(256) void k_logits_few(const TA* __restrict__ x,
                                                    const TA* __restrict__ wr,
                                                    const float* __restrict__ bias,
                                                    float* __restrict__ logits, int T, int H,
                                                    int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * MOE_LOGITS_FEW_WAVES + (threadIdx.x >> 6);
  if (e >= E) return;                    // uniform over the wave
  const TA* wrow = wr + int64_t(e) * H;
  float acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  for (int hb = 0; hb < H; hb += 512 * SMAX) {
    Chunk8<TA> wc[SMAX];
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int h = hb + s * 512 + lane * 8;
      if (h < H) wc[s].load(wrow + h);
    }
#pragma unroll
    for (int g = 0; g < 16; g += TQ) {
      if (g >= T) break;
      Chunk8<TA> xc[TQ][SMAX];
#pragma unroll
      for (int q = 0; q < TQ; ++q)
#pragma unroll
        for (int s = 0; s < SMAX; ++s) {
          const int h = hb + s * 512 + lane * 8;
          if (g + q < T && h < H) xc[q][s].load(x + int64_t(g + q) * H + h);
        }
#pragma unroll
      for (int s = 0; s < SMAX; ++s) {
        const int h = hb + s * 512 + lane * 8;
        if (h < H) {
          float wv[8];
          wc[s].get(wv);
#pragma unroll
          for (int q = 0; q < TQ; ++q) {
            if (g + q < T) {
              float xv[8];
              xc[q][s].get(xv);
              acc[g + q] = dot8(xv, wv, acc[g + q]);
            }
          }
        }
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if (q < T) {
      const float v = wave_sum(acc[q]);
      if (lane == 0) logits[int64_t(q) * E + e] = v + b;
    }
  }
}

// Router logits of a handful of tokens with the pre-layer RMSNorm fused in front:
// x_n = round(x / sqrt(mean(x^2) + eps) * gamma) per token, l = x_n W_r^T (+ bias).
// Each block normalises the T rows once into LDS (wave w takes tokens w, w+4, ...;
// the same lane order and reduction as k_rmsnorm, so both paths produce the same
// rows), then its four waves form one expert's dot products each from LDS.
// T <= 16, H <= 2048 (the decode kernels' range).  Block 0
// also stores x_n, which the expert kernels read, so router and experts see the same
// rows.  The expert's router row is in flight during the normalisation.
// grid = ceil(E/4), block = 256, dynamic LDS = T*H elements.
template <typename TA>
__global__ __launch_bounds__(256) void k_logits_few_norm(const TA* __restrict__ x,
                                                         const TA* __restrict__ gamma, float eps,
                                                         const TA* __restrict__ wr,
                                                         const float* __restrict__ bias,
                                                         float* __restrict__ logits,
                                                         TA* __restrict__ xn_out, int T, int H,
                                                         int E) {
  constexpr int SMAX = 4;
  extern __shared__ __align__(16) unsigned char xn_raw[];
  TA* xn_l = reinterpret_cast<TA*>(xn_raw);
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int e = blockIdx.x * 4 + wv;
  const TA* wrow = wr + int64_t(min(e, E - 1)) * H;
  // one memory round trip: the router row, gamma and this wave's token rows (H <= 2048,
  // T <= 16: at most four tokens of four 512-wide slabs per wave) load together
  Chunk8<TA> wc0[SMAX], gc[SMAX], xc[4][SMAX];
#pragma unroll
  for (int s = 0; s < SMAX; ++s) {
    const int h = s * 512 + lane * 8;
    if (h < H) {
      wc0[s].load(wrow + h);
      gc[s].load(gamma + h);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (wv + 4 * j < T) xc[j][s].load(x + int64_t(wv + 4 * j) * H + h);
    }
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = wv + 4 * j;
    if (q >= T) break;                   // uniform over the wave
    float ss = 0.f;
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      if (s * 512 + lane * 8 < H) {
        float v[8];
        xc[j][s].get(v);
#pragma unroll
        for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
      }
    }
    const float rinv = 1.0f / sqrtf(wave_sum(ss) / float(H) + eps);
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int h = s * 512 + lane * 8;
      if (h < H) {
        float v[8], gv[8];
        xc[j][s].get(v);
        gc[s].get(gv);
        Chunk8<TA> o;
        o.set(v, rinv, gv);
        o.store(xn_l + q * H + h);
        if (blockIdx.x == 0) o.store(xn_out + int64_t(q) * H + h);
      }
    }
  }
  __syncthreads();
  if (e >= E) return;                    // uniform over the wave
  float acc[16];
#pragma unroll
  for (int q = 0; q < 16; ++q) acc[q] = 0.f;
  for (int hb = 0; hb < H; hb += 512 * SMAX) {
#pragma unroll
    for (int s = 0; s < SMAX; ++s) {
      const int h = hb + s * 512 + lane * 8;
      if (h < H) {
        float wv8[8];
        if (hb == 0) wc0[s].get(wv8); else load8(wrow + h, wv8);
#pragma unroll
        for (int q = 0; q < 16; ++q) {
          if (q < T) {
            float v[8];
            load8(xn_l + q * H + h, v);
            acc[q] = dot8(v, wv8, acc[q]);
          }
        }
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int q = 0; q < 16; ++q) {
    if (q < T) {
      const float v = wave_sum(acc[q]);
      if (lane == 0) logits[int64_t(q) * E + e] = v + b;
    }
  }
}

// RMSNorm of a batch (one wave per token): x_n = round(x / sqrt(mean(x^2) + eps) * gamma).
// grid = ceil(T/4), block = 256.
template <typename TA>
__global__ __launch_bounds__(256) void k_rmsnorm(const TA* __restrict__ x,
                                                 const TA* __restrict__ gamma, float eps,
                                                 TA* __restrict__ xn, int64_t T, int H) {
  const int lane = threadIdx.x & 63;
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const TA* xr = x + t * H;
  float ss = 0.f;
  for (int h = lane * 8; h < H; h += 512) {
    float v[8];
    load8(xr + h, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) ss = fmaf(v[i], v[i], ss);
  }
  const float rinv = 1.0f / sqrtf(wave_sum(ss) / float(H) + eps);
  for (int h = lane * 8; h < H; h += 512) {
    float v[8], gv[8];
    load8(xr + h, v);
    load8(gamma + h, gv);
    Chunk8<TA> o;
    o.set(v, rinv, gv);
    o.store(xn + t * H + h);
  }
}

int launch_rmsnorm(const Plan& p, const void* x, const void* gamma, float eps, void* xn,
                   hipStream_t st) {
  const dim3 grid(unsigned((p.T + 3) / 4));
  if (p.act == MOE_F32)
    hipLaunchKernelGGL(k_rmsnorm<float>, grid, dim3(256), 0, st, (const float*)x,
                       (const float*)gamma, eps, (float*)xn, p.T, p.H);
  else
    hipLaunchKernelGGL(k_rmsnorm<bf16_t>, grid, dim3(256), 0, st, (const bf16_t*)x,
                       (const bf16_t*)gamma, eps, (bf16_t*)xn, p.T, p.H);
  return check_launch();
}

int launch_logits_norm(const Plan& p, const void* x, const void* gamma, float eps, const void* wr,
                       const float* bias, float* logits, void* xn, hipStream_t st) {
  if (p.T > 16 || p.H > 2048) return MOE_ERR_UNSUPPORTED;   // the decode path's range only
  const dim3 grid(unsigned((p.E + 3) / 4));
  const size_t lds = size_t(p.T) * p.H * (p.act == MOE_F32 ? 4 : 2);
  if (p.act == MOE_F32)
    hipLaunchKernelGGL(k_logits_few_norm<float>, grid, dim3(256), lds, st, (const float*)x,
                       (const float*)gamma, eps, (const float*)wr, bias, logits, (float*)xn,
                       int(p.T), p.H, p.E);
  else
    hipLaunchKernelGGL(k_logits_few_norm<bf16_t>, grid, dim3(256), lds, st, (const bf16_t*)x,
                       (const bf16_t*)gamma, eps, (const bf16_t*)wr, bias, logits, (bf16_t*)xn,
                       int(p.T), p.H, p.E);
  return check_launch();
}

// ---------------------------------------------------------------------------
// Matrix-core router logits for bf16 batches: l = X W_r^T (+ bias), fp32 [T, E].
// One workgroup per 64-token x 64-expert tile, so a batch spreads over many CUs:
// eight waves, four tile positions (2 x 2, each 32 tokens x 32 experts, one 32x32
// MFMA block) times two halves of every 64-deep K slab; the halves meet through
// LDS at the end.  H moves global -> LDS in slabs of 64 through a ring of NSTG
// stages of direct-to-LDS loads, one 1 KB load per wave per operand and slab (the
// K loop is bound by how fast the loads are issued and land, not by the matrix
// cores, so every wave issues them); the rows are swizzled as swz16 reads them.
// grid = (ceil(T/64), E/64), block = 512.
__global__ __launch_bounds__(512) void k_logits_mfma(const bf16_t* __restrict__ x,
                                                     const bf16_t* __restrict__ wr,
                                                     const float* __restrict__ bias, int64_t T,
                                                     int H, int E, float* __restrict__ logits) {
  constexpr int BT = 64, BE = 64, XU4 = BT * 8, STU4 = XU4 + BE * 8;   // uint4 per stage
  constexpr int L = 2;                                                  // loads per lane per slab
#ifndef MOE_LOGITS_NSTG
#define MOE_LOGITS_NSTG 6
#endif
  constexpr int NSTG = MOE_LOGITS_NSTG;
  __shared__ uint4 ring[NSTG * STU4];
  const int tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  const int wt = wv & 3, kh = wv >> 2;             // tile position, K half
  const int wm = wt >> 1, wn = wt & 1;
  const int64_t t0 = int64_t(blockIdx.x) * BT;
  const int e0 = blockIdx.y * BE;
  // wave wv loads rows 8 wv .. 8 wv + 7 of both operands (8 lanes of 16 bytes per row)
  const int r = 8 * wv + (lane >> 3);
  const int c = dma_chunk(lane, wv) * 8;
  const bf16_t* xg = x + min<int64_t>(t0 + r, T - 1) * H + c;
  const bf16_t* wg = wr + int64_t(e0 + r) * H + c;
  auto issue = [&](int kt, int stage) {
    uint4* st = ring + stage * STU4;
    const int ko = kt * 64;
    dma16(xg + ko, st + wv * 64);
    dma16(wg + ko, st + XU4 + wv * 64);
  };
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
  auto compute = [&](int stage) {
    const uint4* xc = ring + stage * STU4;
    const uint4* wc = xc + XU4;
#pragma unroll
    for (int kq = 0; kq < 2; ++kq) {
      const int chunk = (kh * 2 + kq) * 2 + (lane >> 5);
      const bf16x8 af = __builtin_bit_cast(bf16x8, xc[swz16(wm * 32 + (lane & 31), chunk)]);
      const bf16x8 bfr = __builtin_bit_cast(bf16x8, wc[swz16(wn * 32 + (lane & 31), chunk)]);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af, bfr, acc, 0, 0, 0);
    }
  };
  const int nk = H / 64;
  for (int s = 0; s < NSTG - 1 && s < nk; ++s) issue(s, s);
  // step kt: wait for slab kt (NSTG - 2 later slabs may stay in flight while none has
  // been held back at the tail), barrier, refill the stage slab kt-1 used, multiply kt
  for (int kt = 0; kt < nk; ++kt) {
    if (kt + NSTG - 1 <= nk) wait_vm_lgkm0<(NSTG - 2) * L>(); else wait_vm_lgkm0<0>();
    block_sync_nowait();
    if (kt + NSTG - 1 < nk) issue(kt + NSTG - 1, (kt + NSTG - 1) % NSTG);
    compute(kt % NSTG);
  }
  // the second K half's partial sums join the first's through the (drained) ring
  float* red = reinterpret_cast<float*>(ring);
  __syncthreads();
  if (kh == 1) {
#pragma unroll
    for (int i = 0; i < 16; ++i) red[(wt * 16 + i) * 64 + lane] = acc[i];
  }
  __syncthreads();
  if (kh == 1) return;
  const int e = e0 + wn * 32 + (lane & 31);
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int64_t t = t0 + wm * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
    if (t < T) logits[t * E + e] = (acc[i] + red[(wt * 16 + i) * 64 + lane]) + b;
  }
}

// ---------------------------------------------------------------------------
// Matrix-core router logits for bf16 batches too small to fill the chip with the 64 x 64
// tiles above (a few thousand tokens): one workgroup per 32-token x 32-expert tile, its
// eight waves splitting H into eighths.  An MFMA's sum over its 16 k positions does not
// depend on which inputs a lane's k slots hold as long as both operands hold the same
// ones, so lane (row, half) of wave w takes the contiguous inputs
// [w H/8 + half H/16, + H/16) of its token row and of its expert row: every load of the
// wave is issued before the first MFMA (one memory round trip per workgroup instead of
// a slab ring), and the eight partial tiles are added in wave order through LDS.
// grid = (E/32, ceil(T/32)), block = 512; S = H/128 MFMA steps per wave.
template <int S>
__global__ __launch_bounds__(512) void k_logits_mfma_small(const bf16_t* __restrict__ x,
                                                           const bf16_t* __restrict__ wr,
                                                           const float* __restrict__ bias,
                                                           int64_t T, int H, int E,
                                                           float* __restrict__ logits) {
  __shared__ float red[8][16][64];
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int r = lane & 31, half = lane >> 5;
  const int64_t t0 = int64_t(blockIdx.y) * 32;
  const int e0 = blockIdx.x * 32;
  const int kb = wv * (16 * S) + half * (8 * S);
  const bf16_t* xa = x + min<int64_t>(t0 + r, T - 1) * H + kb;
  const bf16_t* wb = wr + int64_t(e0 + r) * H + kb;
  bf16x8 a[S], b[S];
#pragma unroll
  for (int j = 0; j < S; ++j) {
    a[j] = *reinterpret_cast<const bf16x8*>(xa + 8 * j);
    b[j] = *reinterpret_cast<const bf16x8*>(wb + 8 * j);
  }
  __builtin_amdgcn_sched_barrier(0);   // keep every load ahead of the first MFMA
  f32x16 acc;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc[i] = 0.f;
#pragma unroll
  for (int j = 0; j < S; ++j) acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[j], b[j], acc, 0, 0, 0);
#pragma unroll
  for (int i = 0; i < 16; ++i) red[wv][i][lane] = acc[i];
  __syncthreads();
  // thread (i, l) for i = wv and wv + 8: element i of lane l, summed over the waves in order
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = wv + 8 * q;
    float v = red[0][i][lane];
#pragma unroll
    for (int w = 1; w < 8; ++w) v += red[w][i][lane];
    const int64_t t = t0 + 8 * (i >> 2) + 4 * half + (i & 3);
    const int e = e0 + r;
    if (t < T) logits[t * E + e] = v + (bias ? bias[e] : 0.f);
  }
}

// ---------------------------------------------------------------------------
// Group-limited top-k from fp32 logits, one wave per token (wave-wide arg-max
// rounds), 16 waves per 64-token block; each block writes its per-expert row
// counts for the permutation.  grid = ceil(T/64), block = 1024.
template <int QMAX>
__global__ __launch_bounds__(1024) void k_select_wave(const float* __restrict__ logits, int64_t T,
                                                      int E, int G, int Gk, int k,
                                                      int32_t* __restrict__ ids,
                                                      float* __restrict__ w,
                                                      int32_t* __restrict__ blk) {
  __shared__ int cnt[1024];
  for (int i = threadIdx.x; i < E; i += 1024) cnt[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  for (int i = 0; i < 4; ++i) {
    const int64_t t = int64_t(blockIdx.x) * 64 + wv + 16 * i;
    if (t >= T) break;   // uniform over the wave
    const int id = select_token_wave<QMAX>(logits + t * E, E, G, Gk, k, ids + t * k, w + t * k);
    if (lane < k) atomicAdd(&cnt[id], 1);
  }
  __syncthreads();
  if (blk)
    for (int i = threadIdx.x; i < E; i += 1024) blk[int64_t(blockIdx.x) * E + i] = cnt[i];
}

// ---------------------------------------------------------------------------
// Same selection with sixteen lanes per token (select_token_row), four tokens per
// wave, 32 tokens per block of 8 waves, so that a batch of a few thousand tokens
// covers every CU.  Block 2b + h handles half h of permutation block b (64 tokens)
// and writes its per-expert row counts to blk[h][b] ([2][nblk][E]; the scan adds
// the halves).  Workgroups from xq.nsel = 2 * nblk on quantise x instead (eight waves
// of quant_e4m3_wave, or 512 lanes of quant_mx_lane, each).
// grid = 2 * nblk (+ the quantisation's workgroups), block = 512.
template <int V>
__global__ __launch_bounds__(512) void k_select_rows(const float* __restrict__ logits, int64_t T,
                                                     int E, int G, int Gk, int k,
                                                     int32_t* __restrict__ ids,
                                                     float* __restrict__ w,
                                                     int32_t* __restrict__ blk, int nblk,
                                                     XQuant xq) {
  if (int(blockIdx.x) >= xq.nsel) {      // uniform over the workgroup, before any barrier
    const int64_t qb = int64_t(blockIdx.x) - xq.nsel;
    if (xq.mx)
      quant_mx_lane(xq.x, xq.rows, xq.K, xq.codes, static_cast<uint8_t*>(xq.scales),
                    qb * 512 + threadIdx.x);
    else
      quant_e4m3_wave(xq.x, xq.rows, xq.K, xq.codes, static_cast<float*>(xq.scales),
                      qb * 8 + (threadIdx.x >> 6));
    return;
  }
  __shared__ int cnt[256];
  for (int i = threadIdx.x; i < E; i += 512) cnt[i] = 0;
  __syncthreads();
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6, r16 = lane & 15;
  const int64_t t = int64_t(blockIdx.x) * 32 + wv * 4 + (lane >> 4);
  const bool live = t < T;
  const float* l = logits + (live ? t : T - 1) * E + V * r16;
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
  select_token_row<V>(lv, E, G, Gk, k, id, wt);
  if (live && r16 < k) {
    ids[t * k + r16] = id;
    w[t * k + r16] = wt;
    atomicAdd(&cnt[id], 1);
  }
  __syncthreads();
  if (blk) {
    int32_t* dst = blk + (int64_t(blockIdx.x & 1) * nblk + (blockIdx.x >> 1)) * E;
    for (int i = threadIdx.x; i < E; i += 512) dst[i] = cnt[i];
  }
}

// the row selection covers E = 16 V (V <= 16) with groups spanning a power-of-two
// number of lanes, or whole groups inside a lane
bool select_rows_ok(const Plan& p) {
  if (p.E % 16 || p.E > 256 || p.k > 16) return false;
  const int V = p.E / 16, n = p.E / p.G;
  if (p.G == 1) return true;
  if (n >= V) {
    const int span = n / V;
    return n % V == 0 && (span & (span - 1)) == 0 && span <= 16;
  }
  return V % n == 0;
}

// ---------------------------------------------------------------------------
bool logits_mfma_ok(const Plan& p) {
  return p.act == MOE_BF16 && p.E % 64 == 0 && p.H % 64 == 0 && p.T > 16;
}

// the 32 x 32 tiles where the 64 x 64 ones would leave CUs idle (fewer workgroups than
// MOE_LOGITS_SMALL_BELOW, 256 by default: one per CU)
#ifndef MOE_LOGITS_SMALL_BELOW
#define MOE_LOGITS_SMALL_BELOW 256
#endif
static bool logits_small_ok(const Plan& p) {
  const int S = p.H / 128;
  if (p.act != MOE_BF16 || p.T <= 16 || p.T > int64_t(65535) * 32 || p.E % 32 || p.H % 128 ||
      (S != 8 && S != 12 && S != 16))
    return false;
  return !logits_mfma_ok(p) || (p.T + 63) / 64 * (p.E / 64) < MOE_LOGITS_SMALL_BELOW;
}

int launch_logits(const Plan& p, const void* x, const void* wr, const float* bias, float* logits,
                  hipStream_t st) {
  if (p.T <= 16) {
    const dim3 grid(unsigned((p.E + MOE_LOGITS_FEW_WAVES - 1) / MOE_LOGITS_FEW_WAVES));
    const dim3 block(64 * MOE_LOGITS_FEW_WAVES);
#define MOE_LF(TQ, SM)                                                                          \
  {                                                                                             \
    if (p.act == MOE_F32)                                                                       \
      hipLaunchKernelGGL((k_logits_few<float, TQ, SM>), grid, block, 0, st, (const float*)x,   \
                         (const float*)wr, bias, logits, int(p.T), p.H, p.E);                  \
    else                                                                                        \
      hipLaunchKernelGGL((k_logits_few<bf16_t, TQ, SM>), grid, block, 0, st,                  \
                         (const bf16_t*)x, (const bf16_t*)wr, bias, logits, int(p.T), p.H, p.E); \
  }
    if (p.H <= 512) MOE_LF(16, 1)
    else if (p.H <= 1024) MOE_LF(8, 2)
    else MOE_LF(4, 4)
#undef MOE_LF
    return check_launch();
  }
  if (logits_small_ok(p)) {
    const dim3 grid(unsigned(p.E / 32), unsigned((p.T + 31) / 32));
#define MOE_LS(SS)                                                                              \
  hipLaunchKernelGGL(k_logits_mfma_small<SS>, grid, dim3(512), 0, st, (const bf16_t*)x,        \
                     (const bf16_t*)wr, bias, p.T, p.H, p.E, logits)
    const int S = p.H / 128;
    if (S == 8) MOE_LS(8);
    else if (S == 12) MOE_LS(12);
    else MOE_LS(16);
#undef MOE_LS
    return check_launch();
  }
  if (logits_mfma_ok(p)) {
    const dim3 grid(unsigned((p.T + 63) / 64), unsigned(p.E / 64));
    hipLaunchKernelGGL(k_logits_mfma, grid, dim3(512), 0, st, (const bf16_t*)x, (const bf16_t*)wr,
                       bias, p.T, p.H, p.E, logits);
    return check_launch();
  }
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


int launch_select(const Plan& p, const float* logits, int32_t* ids, float* w, int32_t* blk,
                  hipStream_t st, XQuant xq) {
  const dim3 grid(unsigned((p.T + 63) / 64));
  if (select_rows_ok(p)) {
    const int V = p.E / 16;
    xq.nsel = 2 * p.nblk;
    int64_t nq = 0;                      // workgroups of the carried quantisation
    if (xq.x && xq.rows > 0) {
      if (xq.mx ? (xq.K % 32 != 0) : (xq.K % 128 != 0)) return MOE_ERR_UNSUPPORTED;
      nq = xq.mx ? (xq.rows * (xq.K / 8) + 511) / 512 : (xq.rows * (xq.K / 128) + 31) / 32;
    }
    const dim3 grid2(unsigned(xq.nsel + nq));
#define MOE_SR(VV)                                                                              \
  hipLaunchKernelGGL(k_select_rows<VV>, grid2, dim3(512), 0, st, logits, p.T, p.E, p.G, p.Gk, \
                     p.k, ids, w, blk, p.nblk, xq)
    if (V == 1) MOE_SR(1);
    else if (V == 2) MOE_SR(2);
    else if (V == 4) MOE_SR(4);
    else if (V == 8) MOE_SR(8);
    else if (V == 16) MOE_SR(16);
    else if (V == 3) MOE_SR(3);
    else if (V == 5) MOE_SR(5);
    else if (V == 6) MOE_SR(6);
    else if (V == 7) MOE_SR(7);
    else if (V <= 12) {
      if (V == 9) MOE_SR(9); else if (V == 10) MOE_SR(10); else if (V == 11) MOE_SR(11); else MOE_SR(12);
    } else {
      if (V == 13) MOE_SR(13); else if (V == 14) MOE_SR(14); else MOE_SR(15);
    }
#undef MOE_SR
    return check_launch();
  }
  if (xq.x) return MOE_ERR_UNSUPPORTED;  // only the row selection carries the quantisation
  if (p.E <= 64)
    hipLaunchKernelGGL(k_select_wave<1>, grid, dim3(1024), 0, st, logits, p.T, p.E, p.G, p.Gk, p.k, ids, w, blk);
  else if (p.E <= 128)
    hipLaunchKernelGGL(k_select_wave<2>, grid, dim3(1024), 0, st, logits, p.T, p.E, p.G, p.Gk, p.k, ids, w, blk);
  else if (p.E <= 256)
    hipLaunchKernelGGL(k_select_wave<4>, grid, dim3(1024), 0, st, logits, p.T, p.E, p.G, p.Gk, p.k, ids, w, blk);
  else if (p.E <= 512)
    hipLaunchKernelGGL(k_select_wave<8>, grid, dim3(1024), 0, st, logits, p.T, p.E, p.G, p.Gk, p.k, ids, w, blk);
  else
    hipLaunchKernelGGL(k_select_wave<16>, grid, dim3(1024), 0, st, logits, p.T, p.E, p.G, p.Gk, p.k, ids, w, blk);
  return check_launch();
}

}  // namespace moe
