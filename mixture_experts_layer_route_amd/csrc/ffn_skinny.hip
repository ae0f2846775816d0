// Skinny-M expert kernels: few rows per expert (decode), and every fp32 layer.
//
// The SwiGLU expert (config paragraph of TensorFold issue #1247 "Ling-3.0-tiny on
// a Qualcomm board": SwiGLU experts, null limit lists, so no clamp):
//   h = silu(x Wg^T) * (x Wu^T),  y = h Wd^T.
// With a handful of rows per expert the work is a stream over each chosen
// expert's weights, so these kernels are organised around the weight stream:
// every wave owns a few weight rows, each lane reads 8 consecutive elements
// (16 bytes of bf16) per step, all of a wave's weight loads are issued before
// any is consumed, and the few activation rows come from L2.  fp32 accumulation;
// one wave reduction per (output, row).
#include <algorithm>

#include "moe_internal.h"

namespace moe {

template <typename TW>
__device__ __forceinline__ const TW* expert_base(const TW* routed, const TW* shared, int e, int E,
                                                 int64_t stride) {
  return e < E ? routed + int64_t(e) * stride : shared + int64_t(e - E) * stride;
}

constexpr int kSteps = 4;            // 4 steps x 64 lanes x 8 elements = 2048 per pass
constexpr int kPass = kSteps * 512;

// ---------------------------------------------------------------------------
// Gate/up + SwiGLU.  grid = (max active experts, ceil(I / (4*NI))), block = 256,
// dynamic LDS = RC * min(H, 2048) * sizeof(TA).  Wave w of block (u, y) computes
// h[:, i0..i0+NI) for i0 = (4y + w) * NI over the rows of the u-th active expert,
// RC rows per pass.  The pass's activation rows are loaded into LDS by the whole
// block with the same wait as the wave's weight loads, which are all issued
// first.  h is fp32 [R, I].
template <typename TA, typename TW, int NI, int RC>
__global__ __launch_bounds__(256) void k_gateup_skinny(
    const TA* __restrict__ x, const int32_t* __restrict__ row_token,
    const int32_t* __restrict__ offsets, const int32_t* __restrict__ active,
    const int32_t* __restrict__ meta, const TW* __restrict__ wg, const TW* __restrict__ wu,
    const TW* __restrict__ shg, const TW* __restrict__ shu, float* __restrict__ hout, int H, int I,
    int E) {
  constexpr int CH = 16 / sizeof(TA);                      // activation elements per 16 bytes
  constexpr int XMAX = RC * kPass / CH / 256;              // 16-byte chunks per thread and pass
  extern __shared__ __align__(16) unsigned char lds_raw[];
  TA* xs = reinterpret_cast<TA*>(lds_raw);
  const int u = blockIdx.x;
  if (u >= meta[0]) return;
  const int lane = threadIdx.x & 63;
  const int i0 = (blockIdx.y * 4 + (threadIdx.x >> 6)) * NI;
  const bool live = i0 < I;
  const int e = active[u];
  const int r0 = offsets[e], r1 = offsets[e + 1];
  const int64_t mstride = int64_t(I) * H;
  const TW* gp = expert_base(wg, shg, e, E, mstride) + int64_t(live ? i0 : 0) * H;
  const TW* up = expert_base(wu, shu, e, E, mstride) + int64_t(live ? i0 : 0) * H;

  for (int rc = r0; rc < r1; rc += RC) {
    const int nr = min(RC, r1 - rc);
    float ag[NI][RC], au[NI][RC];
#pragma unroll
    for (int ii = 0; ii < NI; ++ii)
#pragma unroll
      for (int q = 0; q < RC; ++q) ag[ii][q] = au[ii][q] = 0.f;

    for (int hb = 0; hb < H; hb += kPass) {
      const int hw = min(H - hb, kPass);
      const int cpr = hw / CH;                             // chunks per row in this pass
      uint4 xr[XMAX];
#pragma unroll
      for (int c = 0; c < XMAX; ++c) {
        const int idx = threadIdx.x + 256 * c;
        if (idx < nr * cpr) {
          const int q = idx / cpr, h = (idx - q * cpr) * CH;
          xr[c] = *reinterpret_cast<const uint4*>(x + int64_t(row_token[rc + q]) * H + hb + h);
        }
      }
      Chunk8<TW> cg[kSteps][NI], cu[kSteps][NI];
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int h = s * 512 + lane * 8;
        if (h < hw) {
#pragma unroll
          for (int ii = 0; ii < NI; ++ii) {
            cg[s][ii].load(gp + int64_t(ii) * H + hb + h);
            cu[s][ii].load(up + int64_t(ii) * H + hb + h);
          }
        }
      }
#pragma unroll
      for (int c = 0; c < XMAX; ++c) {
        const int idx = threadIdx.x + 256 * c;
        if (idx < nr * cpr) {
          const int q = idx / cpr, h = (idx - q * cpr) * CH;
          *reinterpret_cast<uint4*>(xs + q * hw + h) = xr[c];
        }
      }
      __syncthreads();
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int h = s * 512 + lane * 8;
        if (h < hw) {
#pragma unroll
          for (int q = 0; q < RC; ++q) {
            if (q < nr) {
              float xv[8];
              load8(xs + q * hw + h, xv);
#pragma unroll
              for (int ii = 0; ii < NI; ++ii) {
                float wv[8];
                cg[s][ii].get(wv);
                ag[ii][q] = dot8(wv, xv, ag[ii][q]);
                cu[s][ii].get(wv);
                au[ii][q] = dot8(wv, xv, au[ii][q]);
              }
            }
          }
        }
      }
      __syncthreads();
    }
    if (live) {
#pragma unroll
      for (int q = 0; q < RC; ++q) {
        if (q < nr) {
#pragma unroll
          for (int ii = 0; ii < NI; ++ii) {
            const float g = wave_sum(ag[ii][q]);
            const float v = wave_sum(au[ii][q]);
            if (lane == ii) hout[int64_t(rc + q) * I + i0 + ii] = silu(g) * v;
          }
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection, unweighted, per expert.  grid = (max active, ceil(H/(4*NR))).
// y_perm[r, n] = sum_i h[r, i] Wd[e][n, i]  (fp32 out).
template <typename TW, int NR, int RC>
__global__ __launch_bounds__(256) void k_down_skinny(
    const float* __restrict__ hin, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ active, const int32_t* __restrict__ meta,
    const TW* __restrict__ wd, const TW* __restrict__ shd, float* __restrict__ y_perm, int H, int I,
    int E) {
  const int u = blockIdx.x;
  if (u >= meta[0]) return;
  const int lane = threadIdx.x & 63;
  const int n0 = (blockIdx.y * 4 + (threadIdx.x >> 6)) * NR;
  if (n0 >= H) return;
  const int e = active[u];
  const int r0 = offsets[e], r1 = offsets[e + 1];
  const TW* dp = expert_base(wd, shd, e, E, int64_t(H) * I) + int64_t(n0) * I;

  for (int rc = r0; rc < r1; rc += RC) {
    const int nr = min(RC, r1 - rc);
    float acc[NR][RC];
#pragma unroll
    for (int nn = 0; nn < NR; ++nn)
#pragma unroll
      for (int q = 0; q < RC; ++q) acc[nn][q] = 0.f;
    for (int kb = 0; kb < I; kb += kPass) {
      Chunk8<TW> cw[kSteps][NR];
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int kk = kb + s * 512 + lane * 8;
        if (kk < I) {
#pragma unroll
          for (int nn = 0; nn < NR; ++nn) cw[s][nn].load(dp + int64_t(nn) * I + kk);
        }
      }
#pragma unroll
      for (int s = 0; s < kSteps; ++s) {
        const int kk = kb + s * 512 + lane * 8;
        if (kk < I) {
#pragma unroll
          for (int q = 0; q < RC; ++q) {
            if (q < nr) {
              float hv[8];
              load8(hin + int64_t(rc + q) * I + kk, hv);
#pragma unroll
              for (int nn = 0; nn < NR; ++nn) {
                float wv[8];
                cw[s][nn].get(wv);
                acc[nn][q] = dot8(wv, hv, acc[nn][q]);
              }
            }
          }
        }
      }
    }
#pragma unroll
    for (int q = 0; q < RC; ++q) {
      if (q < nr) {
#pragma unroll
        for (int nn = 0; nn < NR; ++nn) {
          const float v = wave_sum(acc[nn][q]);
          if (lane == nn) y_perm[int64_t(rc + q) * H + n0 + nn] = v;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Down projection fused with the weighted combine, for few tokens.
// grid = (ceil(H/NR), ceil(T/4)), block = 256.  Wave w of block (x, y) owns
// token t = 4y + w and output columns n0..n0+NR, n0 = NR*x:
//   y[t, n] = sum_j w[t,j] * (h[inv[t,j]] . Wd[ids[t,j]][n]) + sum_s (h[T*k+s*T+t] . Wd_s[n])
// Slots are taken JB at a time with every weight and h load of the batch issued
// before any is used.
template <typename TW, typename TY, int NR>
__global__ __launch_bounds__(256) void k_down_combine_skinny(
    const float* __restrict__ hin, const int32_t* __restrict__ ids, const float* __restrict__ w,
    const int32_t* __restrict__ inv, const TW* __restrict__ wd, const TW* __restrict__ shd,
    const TY* res, TY* y, int T, int H, int I, int E, int k, int S) {
  constexpr int JB = 8;
  const int lane = threadIdx.x & 63;
  const int n0 = blockIdx.x * NR;
  const int t = blockIdx.y * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  const int64_t estride = int64_t(H) * I;
  const int nslots = k + S;
  float acc[NR];
#pragma unroll
  for (int nn = 0; nn < NR; ++nn) acc[nn] = 0.f;
  for (int jb = 0; jb < nslots; jb += JB) {
    for (int kb = 0; kb < I; kb += 512) {
      const int kk = kb + lane * 8;
      const bool kin = kk < I;
      Chunk8<TW> cw[JB][NR];
      float hv[JB][8];
      float wt[JB];
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        const int j = jb + jj;
        wt[jj] = 0.f;
        if (j < nslots && kin) {
          int e, r;
          if (j < k) {
            e = ids[t * k + j];
            r = inv[t * k + j];
            wt[jj] = w[t * k + j];
          } else {
            e = E + (j - k);
            r = T * k + (j - k) * T + t;
            wt[jj] = 1.f;
          }
          const TW* dp = expert_base(wd, shd, e, E, estride) + int64_t(n0) * I + kk;
#pragma unroll
          for (int nn = 0; nn < NR; ++nn)
            if (n0 + nn < H) cw[jj][nn].load(dp + int64_t(nn) * I);
          load8(hin + int64_t(r) * I + kk, hv[jj]);
        }
      }
#pragma unroll
      for (int jj = 0; jj < JB; ++jj) {
        if (jb + jj < nslots && kin) {
#pragma unroll
          for (int nn = 0; nn < NR; ++nn) {
            if (n0 + nn < H) {
              float wv[8];
              cw[jj][nn].get(wv);
              acc[nn] = fmaf(wt[jj], dot8(wv, hv[jj], 0.f), acc[nn]);
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
      if (res) v += to_f32<TY>(res[o]);
      y[o] = from_f32<TY>(v);
    }
  }
}

// ---------------------------------------------------------------------------
template <typename TA, typename TW>
static void gateup(const Plan& p, const void* x, const int32_t* rt, const int32_t* off,
                   const int32_t* act, const int32_t* meta, const moe_weights* w, float* h,
                   hipStream_t st) {
  constexpr int NI = 2, RC = 4;
  dim3 grid(unsigned(p.max_active), unsigned((p.I + 4 * NI - 1) / (4 * NI)));
  const size_t lds = size_t(RC) * std::min(p.H, kPass) * sizeof(TA);
  launch_kernel(p, kTimeGateUp, k_gateup_skinny<TA, TW, NI, RC>, grid, dim3(256), lds, st,
                (const TA*)x, rt, off, act, meta, (const TW*)w->w_gate, (const TW*)w->w_up,
                     (const TW*)w->sh_gate, (const TW*)w->sh_up, h, p.H, p.I, p.E);
}

int launch_gateup_skinny(const Plan& p, const void* x, const int32_t* row_token,
                         const int32_t* offsets, const int32_t* active, const int32_t* meta,
                         const moe_weights* w, float* h, hipStream_t st) {
  if (p.wt == MOE_NVFP4)
    return launch_nv_gateup_batch(p, x, row_token, offsets, active, meta, w, h, st);
  if (p.wt == MOE_F32)
    gateup<float, float>(p, x, row_token, offsets, active, meta, w, h, st);
  else
    gateup<bf16_t, bf16_t>(p, x, row_token, offsets, active, meta, w, h, st);
  return check_launch();
}

int launch_down_skinny(const Plan& p, const float* h, const int32_t* offsets,
                       const int32_t* active, const int32_t* meta, const moe_weights* w,
                       float* y_perm, hipStream_t st) {
  if (p.wt == MOE_NVFP4) return launch_nv_down_batch(p, h, offsets, active, meta, w, y_perm, st);
  constexpr int NR = 2, RC = 4;
  dim3 grid(unsigned(p.max_active), unsigned((p.H + 4 * NR - 1) / (4 * NR)));
  if (p.wt == MOE_F32)
    launch_kernel(p, kTimeDown, k_down_skinny<float, NR, RC>, grid, dim3(256), 0, st, h, offsets, active,
                       meta, (const float*)w->w_down, (const float*)w->sh_down, y_perm, p.H, p.I,
                       p.E);
  else
    launch_kernel(p, kTimeDown, k_down_skinny<bf16_t, NR, RC>, grid, dim3(256), 0, st, h, offsets, active,
                       meta, (const bf16_t*)w->w_down, (const bf16_t*)w->sh_down, y_perm, p.H,
                       p.I, p.E);
  return check_launch();
}

int launch_down_combine_skinny(const Plan& p, const float* h, const int32_t* ids, const float* wts,
                               const int32_t* inv, const moe_weights* w, const void* res, void* y,
                               hipStream_t st) {
  constexpr int NR = 4;
  dim3 grid(unsigned((p.H + NR - 1) / NR), unsigned((p.T + 3) / 4));
  const int T = int(p.T);
  if (p.wt == MOE_F32)
    launch_kernel(p, kTimeDown, k_down_combine_skinny<float, float, NR>, grid, dim3(256), 0, st, h, ids,
                       wts, inv, (const float*)w->w_down, (const float*)w->sh_down, (const float*)res, (float*)y, T,
                       p.H, p.I, p.E, p.k, p.S);
  else
    launch_kernel(p, kTimeDown, k_down_combine_skinny<bf16_t, bf16_t, NR>, grid, dim3(256), 0, st, h,
                       ids, wts, inv, (const bf16_t*)w->w_down, (const bf16_t*)w->sh_down,
                       (const bf16_t*)res, (bf16_t*)y, T, p.H, p.I, p.E, p.k, p.S);
  return check_launch();
}

}  // namespace moe
