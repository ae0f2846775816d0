// Weighted combine back to token order (the weighted layer of the HelloSun/ling30tiny
// model card's numeric-check summary 數值檢查摘要; shared-expert sum per the Inkling
// PR summary of llama.cpp "Add TML Inkling architecture"):
//   y[t] = sum_j w[t,j] * y_perm[inv[t,j]] + sum_s y_perm[offsets[E+s] + t] (+ res[t])
// in that fixed order, fp32, then stored in the activation type.  `res` is the
// decoder step's residual input (or null); y may alias it element for element.  No atomics,
// so the result is bitwise reproducible.
#include "moe_internal.h"

namespace moe {

// grid = (T, ceil(H / 2048)), block = 256; each thread owns 8 consecutive columns.
// TP: element type of y_perm.  WEIGHTED: y_perm rows already carry their weight.
template <typename TP, typename TY, bool PREWEIGHTED>
__global__ __launch_bounds__(256) void k_combine(const TP* __restrict__ y_perm,
                                                 const int32_t* __restrict__ offsets,
                                                 const int32_t* __restrict__ inv,
                                                 const float* __restrict__ w, const TY* res,
                                                 TY* y, int H, int E, int k, int S) {
  const int64_t t = blockIdx.x;
  const int c = (blockIdx.y * 256 + threadIdx.x) * 8;
  if (c >= H) return;
  float acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  for (int j = 0; j < k; ++j) {
    const int64_t r = inv[t * k + j];
    const float wj = PREWEIGHTED ? 1.f : w[t * k + j];
    float v[8];
    load8(y_perm + r * H + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
  }
  for (int s = 0; s < S; ++s) {
    const int64_t r = int64_t(offsets[E + s]) + t;
    float v[8];
    load8(y_perm + r * H + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  if (res) {
    float v[8];
    load8(res + t * H + c, v);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += v[i];
  }
  TY* out = y + t * H + c;
  if constexpr (sizeof(TY) == 2) {
    uint4 pk;
    pk.x = uint32_t(f32_to_bf16(acc[0])) | (uint32_t(f32_to_bf16(acc[1])) << 16);
    pk.y = uint32_t(f32_to_bf16(acc[2])) | (uint32_t(f32_to_bf16(acc[3])) << 16);
    pk.z = uint32_t(f32_to_bf16(acc[4])) | (uint32_t(f32_to_bf16(acc[5])) << 16);
    pk.w = uint32_t(f32_to_bf16(acc[6])) | (uint32_t(f32_to_bf16(acc[7])) << 16);
    *reinterpret_cast<uint4*>(out) = pk;
  } else {
    *reinterpret_cast<float4*>(out) = make_float4(acc[0], acc[1], acc[2], acc[3]);
    *reinterpret_cast<float4*>(out + 4) = make_float4(acc[4], acc[5], acc[6], acc[7]);
  }
}

int launch_combine(const Plan& p, const float* y_perm, const int32_t* offsets, const int32_t* inv,
                   const float* w, const void* res, void* y, hipStream_t st) {
  dim3 grid(unsigned(p.T), unsigned((p.H + 2047) / 2048));
  if (p.act == MOE_F32)
    hipLaunchKernelGGL((k_combine<float, float, false>), grid, dim3(256), 0, st, y_perm, offsets,
                       inv, w, (const float*)res, (float*)y, p.H, p.E, p.k, p.S);
  else
    hipLaunchKernelGGL((k_combine<float, bf16_t, false>), grid, dim3(256), 0, st, y_perm, offsets,
                       inv, w, (const bf16_t*)res, (bf16_t*)y, p.H, p.E, p.k, p.S);
  return check_launch();
}

// bf16 rows that already carry their routing weight (the fused down epilogue).
int launch_combine_preweighted(const Plan& p, const bf16_t* y_perm, const int32_t* offsets,
                               const int32_t* inv, const void* res, void* y, hipStream_t st) {
  dim3 grid(unsigned(p.T), unsigned((p.H + 2047) / 2048));
  hipLaunchKernelGGL((k_combine<bf16_t, bf16_t, true>), grid, dim3(256), 0, st, y_perm, offsets,
                     inv, (const float*)nullptr, (const bf16_t*)res, (bf16_t*)y, p.H, p.E, p.k,
                     p.S);
  return check_launch();
}

}  // namespace moe
