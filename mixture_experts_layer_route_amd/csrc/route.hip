// Router: logits, group-limited top-k and renormalised weights.
//
// Group-limited routing is named in TensorFold issue #1247 "Ling-3.0-tiny on a
// Qualcomm board" (jschmied's comment, list "What it does not cover"); its config
// paragraph fixes 128 experts in 8 groups of 16 with 4 groups kept, and the
// HelloSun/ling30tiny routing table (模型與路由) fixes 8 experts per token.  The
// pages do not name the score function; the layer takes the softmax of the
// logits, a group's score is its best expert score, ties go to the lower index
// and the chosen weights are renormalised to sum 1.  Softmax is monotone, so
// groups and experts are ranked on the fp32 logits themselves and the weights
// are the softmax over the chosen logits (the renormalised softmax equals it).
#include "moe_internal.h"
#include "route_select.h"

namespace moe {

// ---------------------------------------------------------------------------
// Logits with vector FMAs: one wave per expert row, RT tokens per pass.
// grid = (ceil(E/4), ceil(T/RT)), block = 256.  Each lane covers 8 consecutive
// elements of H per step, accumulating fp32; a wave reduction finishes the dot.
template <typename TA, int RT>
__global__ __launch_bounds__(256) void k_router_logits_fma(
    const TA* __restrict__ x, const TA* __restrict__ wr, const float* __restrict__ bias,
    float* __restrict__ logits, int64_t T, int H, int E) {
  const int lane = threadIdx.x & 63;
  const int e = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (e >= E) return;
  const int64_t t0 = int64_t(blockIdx.y) * RT;
  const int nt = int(min<int64_t>(RT, T - t0));
  const TA* wrow = wr + int64_t(e) * H;
  float acc[RT];
#pragma unroll
  for (int q = 0; q < RT; ++q) acc[q] = 0.f;
  for (int h = lane * 8; h < H; h += 64 * 8) {
    float wv[8];
    load8(wrow + h, wv);
#pragma unroll
    for (int q = 0; q < RT; ++q) {
      if (q < nt) {
        float xv[8];
        load8(x + (t0 + q) * H + h, xv);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[q] = fmaf(xv[i], wv[i], acc[q]);
      }
    }
  }
  const float b = bias ? bias[e] : 0.f;
#pragma unroll
  for (int q = 0; q < RT; ++q) {
    if (q < nt) {
      float s = wave_sum(acc[q]);
      if (lane == 0) logits[(t0 + q) * E + e] = s + b;
    }
  }
}

// One wave per token.  grid = ceil(T/4), block = 256.
template <int QMAX>
__global__ __launch_bounds__(256) void k_router_select(
    const float* __restrict__ logits, int64_t T, int E, int G, int Gk, int k,
    int32_t* __restrict__ ids, float* __restrict__ w) {
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  select_token<QMAX>(logits + t * E, E, G, Gk, k, ids + t * k, w + t * k);
}

// ---------------------------------------------------------------------------
int launch_logits(const Plan& p, const void* x, const void* wr, const float* bias, float* logits,
                  hipStream_t st) {
  constexpr int RT = 8;
  const dim3 grid((p.E + 3) / 4, unsigned((p.T + RT - 1) / RT));
  if (p.act == MOE_F32)
    hipLaunchKernelGGL((k_router_logits_fma<float, RT>), grid, dim3(256), 0, st, (const float*)x,
                       (const float*)wr, bias, logits, p.T, p.H, p.E);
  else
    hipLaunchKernelGGL((k_router_logits_fma<bf16_t, RT>), grid, dim3(256), 0, st,
                       (const bf16_t*)x, (const bf16_t*)wr, bias, logits, p.T, p.H, p.E);
  return check_launch();
}

int launch_select(const Plan& p, const float* logits, int32_t* ids, float* w, hipStream_t st) {
  const dim3 grid(unsigned((p.T + 3) / 4));
#define MOE_SELECT(Q)                                                                              \
  hipLaunchKernelGGL(k_router_select<Q>, grid, dim3(256), 0, st, logits, p.T, p.E, p.G, p.Gk, p.k, \
                     ids, w)
  if (p.E <= 64) MOE_SELECT(1);
  else if (p.E <= 128) MOE_SELECT(2);
  else if (p.E <= 256) MOE_SELECT(4);
  else if (p.E <= 512) MOE_SELECT(8);
  else MOE_SELECT(16);
#undef MOE_SELECT
  return check_launch();
}

}  // namespace moe
