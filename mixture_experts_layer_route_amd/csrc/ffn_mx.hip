// MXFP4 experts on gfx950's block-scaled matrix cores.
//
// The pages name 4-bit experts (TensorFold issue #1247 "Ling-3.0-tiny on a Qualcomm
// board", list "What it does not cover"; the graysoft "Ling-3.0-tiny-base - ROCmFP4"
// page) without a layout; these kernels take the OCP Microscaling reading: weights are
// E2M1 codes (two per byte, element 2i in the low nibble) with one E8M0 scale per 32
// inputs, and the activations (x, and h before the down projection) are quantised per
// row per 32 to MXFP8 (E4M3 codes, E8M0 shared exponent floor(log2(amax)) - 8).  Both
// operands then go straight into v_mfma_scale_f32_32x32x64_f8f6f4 (A = fp4 weights,
// B = fp8 activations) with the block scales as its per-lane scale operands, so the
// kernel does no dequantisation at all.
//
// Lane layout of one 32x32x64 step, as measured on the device: lane l (row l % 32,
// half h = l / 32) passes, for the fp4 A operand, 16 contiguous bytes = inputs
// [32h, 32h + 32) of the 64-input window, and for the fp8 B operand inputs
// [16h, 16h + 16) and [32 + 16h, 32 + 16h + 16); the scale a lane passes covers block h
// (inputs [32h, 32h + 32)) of its row on both operands.  The scale operand's byte is
// chosen by op_sel: each lane passes the word of its row's four scales of a 128-input
// slab shifted by 8h bytes, and op_sel 0 / 2 selects the first / second 64-input step.
//
// Tiles: 128 activation rows x 256 weight rows per workgroup of 8 waves (2 x 4, 64 x 64
// each), 128-input slabs through a three-slot direct-to-LDS ring (activation rows 128 B,
// weight rows 64 B, both XOR-swizzled so that a ds_read_b128 of 16 lanes hits distinct
// banks), every scale of the tile staged in LDS before the K loop, XCD-aware items.
// The gate/up epilogue applies SwiGLU and quantises h to MXFP8: a wave holds 32 h
// columns of its rows, exactly one 32-block, so each row's scale is a two-lane
// reduction.
#include "moe_internal.h"
#include "gemm_common.h"

namespace moe {

struct GemmMx4Args {
  const uint8_t* a;           // gate/up: x codes [T, H] (gathered); down: h codes [R, I]
  const uint8_t* a_scale;     // E8M0 [rows, K/32]
  const int32_t* row_token;   // gate/up only
  const int32_t* offsets;
  const int2* tiles;
  const int32_t* meta;
  const uint8_t* w0;          // gate/up: w_gate; down: w_down (packed E2M1, [N, K/2] per expert)
  const uint8_t* w1;          // gate/up: w_up
  const uint8_t* sh0;
  const uint8_t* sh1;
  const uint8_t* s0;          // E8M0 scales of w0 / w1 / shared [N, K/32] per expert
  const uint8_t* s1;
  const uint8_t* shs0;
  const uint8_t* shs1;
  const float* row_w;         // down, weighted bf16 output
  uint8_t* qout;              // gate/up: h codes [R, I]
  uint8_t* qscale;            // gate/up: h scales [R, I/32]
  bf16_t* out16;              // down: weighted y_perm [R, H] (bf16)
  float* out32;               // down: unweighted y_perm [R, H]
  int K, N, E;
};

struct Mx4Tile {
  static constexpr int BM = 128, BN = 256, KB = 128, WM = 2, WN = 4, W = WM * WN, NT = 64 * W;
  static constexpr int MI = BM / WM / 32, NI = BN / WN / 32;          // 2 x 2 blocks per wave
  static constexpr int AJ = BM / (8 * W);     // activation DMAs per wave: 8 rows of 128 B each
  static constexpr int BJ = BN / (16 * W);    // weight DMAs per wave: 16 rows of 64 B each
  static constexpr int L = AJ + BJ;
  static constexpr int A_U4 = BM * 8, B_U4 = BN * 4, STAGE_U4 = A_U4 + B_U4, RING_U4 = 3 * STAGE_U4;
  static constexpr int SMAX = 17;             // scale words per row (K <= 2048, +1 pad)
};

// 64-byte tile rows of four 16-byte chunks: chunk c of row r sits at r * 4 + (c ^ ((r >> 2) & 3)),
// so that 16 consecutive rows read at one chunk fill 16 distinct slots of the bank line.
__device__ __forceinline__ int swz4(int row, int chunk) { return row * 4 + (chunk ^ ((row >> 2) & 3)); }
// A wave's direct-to-LDS load of 64 x 16 bytes fills rows 16j .. 16j+15 (lane L writes
// position L % 4 of row 16j + L / 4): the logical chunk lane L fetches.
__device__ __forceinline__ int dma_chunk4(int lane, int j) {
  return (lane & 3) ^ (((16 * j + (lane >> 2)) >> 2) & 3);
}

template <bool GATEUP>
__global__ __launch_bounds__(Mx4Tile::NT) __attribute__((amdgpu_waves_per_eu(2)))
void k_gemm_mx4(GemmMx4Args p) {
  using C = Mx4Tile;
  constexpr int BM = C::BM, BN = C::BN, W = C::W, WM = C::WM, WN = C::WN, MI = C::MI, NI = C::NI;
  constexpr int AJ = C::AJ, BJ = C::BJ, L = C::L, NT = C::NT, SMAX = C::SMAX;
  __shared__ uint4 smem[C::RING_U4];
  __shared__ uint32_t sa_l[BM * SMAX];     // activation scale words [row][slab]
  __shared__ uint32_t sw_l[BN * SMAX];     // weight scale words [row][slab]
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
  const int nk = int(K / C::KB);
  const int sww = nk + 1;                                 // padded scale words per row

  const uint8_t* ag[AJ];
#pragma unroll
  for (int i = 0; i < AJ; ++i) {
    const int r = 8 * (wv + W * i) + (lane >> 3);
    const int m = min(m0 + r, cnt - 1);
    const int64_t arow = GATEUP ? int64_t(p.row_token[base + m]) : int64_t(base + m);
    ag[i] = p.a + arow * K + dma_chunk(lane, wv + W * i) * 16;
  }
  const int64_t kb2 = K / 2;                               // bytes of one weight row
  const int64_t mst = int64_t(p.N) * kb2;                  // bytes of one expert matrix
  auto wmat = [&](int r) -> int64_t {                      // tile weight row -> matrix row
    return GATEUP ? int64_t(ct * (BN / 2) + (r < BN / 2 ? r : r - BN / 2)) : int64_t(ct * BN + r);
  };
  const uint8_t* bg[BJ];
#pragma unroll
  for (int i = 0; i < BJ; ++i) {
    const int r = 16 * (wv + W * i) + (lane >> 2);
    const uint8_t* mat = GATEUP && r >= BN / 2 ? expert_mat(p.w1, p.sh1, e, p.E, mst)
                                               : expert_mat(p.w0, p.sh0, e, p.E, mst);
    bg[i] = mat + wmat(r) * kb2 + dma_chunk4(lane, wv + W * i) * 16;
  }
  auto issue = [&](int kt, int slot) {
    uint4* sa = smem + slot * C::STAGE_U4;
    uint4* sb = sa + C::A_U4;
#pragma unroll
    for (int i = 0; i < AJ; ++i) dma16(ag[i] + int64_t(kt) * 128, sa + (wv + W * i) * 64);
#pragma unroll
    for (int i = 0; i < BJ; ++i) dma16(bg[i] + int64_t(kt) * 64, sb + (wv + W * i) * 64);
  };
  issue(0, 0);
  if (nk > 1) issue(1, 1);

  // scales of the tile -> LDS, one word (four 32-blocks = one slab) per load
  {
    const int64_t srow = K / 32;                          // scale bytes per row
    const int64_t sst = int64_t(p.N) * srow;              // scale bytes per expert matrix
    constexpr int SPW = BN * (SMAX - 1) / NT;             // weight words per thread (<= 8)
    constexpr int SPA = BM * (SMAX - 1) / NT;             // activation words per thread (<= 4)
    uint32_t wvv[SPW], avv[SPA];
#pragma unroll
    for (int u = 0; u < SPW; ++u) {                       // clamped loads, all in flight
      const int i = min(tid + u * NT, BN * nk - 1);
      const int r = i / nk, kt = i - r * nk;
      const uint8_t* sm = GATEUP && r >= BN / 2 ? expert_mat(p.s1, p.shs1, e, p.E, sst)
                                                : expert_mat(p.s0, p.shs0, e, p.E, sst);
      wvv[u] = *reinterpret_cast<const uint32_t*>(sm + wmat(r) * srow + 4 * kt);
    }
#pragma unroll
    for (int u = 0; u < SPA; ++u) {
      const int i = min(tid + u * NT, BM * nk - 1);
      const int r = i / nk, kt = i - r * nk;
      const int m = min(m0 + r, cnt - 1);
      const int64_t arow = GATEUP ? int64_t(p.row_token[base + m]) : int64_t(base + m);
      avv[u] = *reinterpret_cast<const uint32_t*>(p.a_scale + arow * srow + 4 * kt);
    }
#pragma unroll
    for (int u = 0; u < SPW; ++u) {
      const int i = tid + u * NT;
      if (i < BN * nk) sw_l[(i / nk) * sww + i % nk] = wvv[u];
    }
#pragma unroll
    for (int u = 0; u < SPA; ++u) {
      const int i = tid + u * NT;
      if (i < BM * nk) sa_l[(i / nk) * sww + i % nk] = avv[u];
    }
  }

  f32x16 acc[MI][NI];
#pragma unroll
  for (int a = 0; a < MI; ++a)
#pragma unroll
    for (int b = 0; b < NI; ++b)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
  // this wave's weight rows: gate/up b = 0 gate, 1 up (same h columns); down: output
  // columns wn*64 + 32b
  auto wrow = [&](int b) {
    return GATEUP ? (b == 0 ? 0 : BN / 2) + wn * (BN / 2 / WN) + (lane & 31)
                  : wn * (BN / WN) + b * 32 + (lane & 31);
  };
  const int hsel = lane >> 5;
  auto compute = [&](int slot, int kt, auto&& between) {
    const uint4* sa = smem + slot * C::STAGE_U4;
    const uint4* sb = sa + C::A_U4;
    i32x8 af[2][MI], bfr[2][NI];
    auto frags = [&](int ks, i32x8 (&xa)[MI], i32x8 (&xb)[NI]) {
#pragma unroll
      for (int a = 0; a < MI; ++a) {                      // fp8: inputs 16h.. and 32+16h..
        const int row = wm * (BM / WM) + a * 32 + (lane & 31);
        const uint4 lo = sa[swz16(row, 4 * ks + hsel)], hi = sa[swz16(row, 4 * ks + hsel + 2)];
        xa[a] = i32x8{int(lo.x), int(lo.y), int(lo.z), int(lo.w), int(hi.x), int(hi.y), int(hi.z), int(hi.w)};
      }
#pragma unroll
      for (int b = 0; b < NI; ++b) {                      // fp4: 16 contiguous bytes, inputs 32h..
        const uint4 q = sb[swz4(wrow(b), 2 * ks + hsel)];
        xb[b] = i32x8{int(q.x), int(q.y), int(q.z), int(q.w), 0, 0, 0, 0};
      }
    };
    frags(0, af[0], bfr[0]);
    __builtin_amdgcn_sched_barrier(0);
    between();
    frags(1, af[1], bfr[1]);
    __builtin_amdgcn_sched_barrier(0);
    int sac[MI], swc[NI];
#pragma unroll
    for (int a = 0; a < MI; ++a)
      sac[a] = int(sa_l[(wm * (BM / WM) + a * 32 + (lane & 31)) * sww + kt] >> (8 * hsel));
#pragma unroll
    for (int b = 0; b < NI; ++b) swc[b] = int(sw_l[wrow(b) * sww + kt] >> (8 * hsel));
#pragma unroll
    for (int a = 0; a < MI; ++a)
#pragma unroll
      for (int b = 0; b < NI; ++b) {
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[0][b], af[0][a], acc[a][b],
                                                                    4, 0, 0, swc[b], 0, sac[a]);
        acc[a][b] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bfr[1][b], af[1][a], acc[a][b],
                                                                    4, 0, 2, swc[b], 2, sac[a]);
      }
  };
  __syncthreads();   // scales staged
#define MOE_MX_STEP(KT, SLOT, NSLOT)                                        \
  {                                                                         \
    if ((KT) + 1 < nk) wait_vm_lgkm0<L>(); else wait_vm_lgkm0<0>();         \
    block_sync_nowait();                                                    \
    compute(SLOT, KT, [&] { if ((KT) + 2 < nk) issue((KT) + 2, NSLOT); });  \
  }
  for (int kt = 0; kt < nk; kt += 3) {
    MOE_MX_STEP(kt, 0, 2)
    if (kt + 1 < nk) MOE_MX_STEP(kt + 1, 1, 0)
    if (kt + 2 < nk) MOE_MX_STEP(kt + 2, 2, 1)
  }
#undef MOE_MX_STEP

  // Epilogue.  Accumulator register r of block (a, b) holds weight row (output
  // column) 8(r/4) + 4(lane/32) + r%4 of the block for activation row lane%32.
  __syncthreads();   // every wave is done with the ring; it becomes staging space
  const int rows = min(BM, cnt - m0);
  if (GATEUP) {
    // h = silu(g) * u; the wave's 32 h columns are one MXFP8 block of each of its rows
    uint8_t* stg = reinterpret_cast<uint8_t*>(smem);      // [BM][128] codes
#pragma unroll
    for (int a = 0; a < MI; ++a) {
      float hv[16];
      float m = 0.f;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        hv[r] = silu_lp(acc[a][0][r]) * acc[a][1][r];
        m = fmaxf(m, fabsf(hv[r]));
      }
      m = fmaxf(m, __shfl_xor(m, 32, 64));
      const int X = mx_exponent(m);
      const float inv = mx_inv_scale(X);
      const int row = wm * (BM / WM) + a * 32 + (lane & 31);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const uint32_t pk = e4m3x4(hv[4 * g] * inv, hv[4 * g + 1] * inv, hv[4 * g + 2] * inv,
                                   hv[4 * g + 3] * inv);
        const int col = wn * 32 + 8 * g + 4 * (lane >> 5);
        *reinterpret_cast<uint32_t*>(stg + stg128(row, col)) = pk;
      }
      if (lane < 32 && row < rows)
        p.qscale[int64_t(base + m0 + row) * (p.N / 32) + ct * 4 + wn] = uint8_t(X + 127);
    }
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

// MXFP8 activations of x: quant_mx_lane per lane, 2,048 values per workgroup of 256.
__global__ __launch_bounds__(256) void k_quant_mx(const bf16_t* __restrict__ in, int64_t rows, int K,
                                                  uint8_t* __restrict__ codes,
                                                  uint8_t* __restrict__ scales) {
  quant_mx_lane(in, rows, K, codes, scales, int64_t(blockIdx.x) * 256 + threadIdx.x);
}

bool mx4_ok(const Plan& p) {
  return p.act == MOE_BF16 && p.wt == MOE_MXFP4 && p.H % Mx4Tile::BN == 0 && p.I % 128 == 0 &&
         p.H <= 2048 && p.I <= 2048;
}

int launch_quant_mx(const void* in, int64_t rows, int K, uint8_t* codes, uint8_t* scales,
                    hipStream_t st) {
  const int64_t n8 = rows * (K / 8);
  if (n8 == 0) return MOE_OK;
  hipLaunchKernelGGL(k_quant_mx, dim3(unsigned((n8 + 255) / 256)), dim3(256), 0, st,
                     (const bf16_t*)in, rows, K, codes, scales);
  return check_launch();
}

int launch_gateup_mx4(const Plan& p, const uint8_t* xq, const uint8_t* sx, const int32_t* row_token,
                      const int32_t* offsets, const int2* tiles, const int32_t* meta,
                      const moe_weights* w, uint8_t* hq, uint8_t* shq, hipStream_t st) {
  GemmMx4Args a{};
  a.a = xq; a.a_scale = sx; a.row_token = row_token; a.offsets = offsets; a.tiles = tiles;
  a.meta = meta; a.w0 = (const uint8_t*)w->w_gate; a.w1 = (const uint8_t*)w->w_up;
  a.sh0 = (const uint8_t*)w->sh_gate; a.sh1 = (const uint8_t*)w->sh_up;
  a.s0 = w->b_gate; a.s1 = w->b_up; a.shs0 = w->sh_b_gate; a.shs1 = w->sh_b_up;
  a.qout = hq; a.qscale = shq; a.K = p.H; a.N = p.I; a.E = p.E;
  launch_kernel(p, kTimeGateUp, k_gemm_mx4<true>,
                dim3(xcd_grid(p.max_tiles * (p.I / (Mx4Tile::BN / 2)))), dim3(Mx4Tile::NT), 0, st, a);
  return check_launch();
}

int launch_down_mx4(const Plan& p, const uint8_t* hq, const uint8_t* shq, const int32_t* offsets,
                    const int2* tiles, const int32_t* meta, const moe_weights* w,
                    const float* row_w, float* out32, bf16_t* out16, hipStream_t st) {
  GemmMx4Args a{};
  a.a = hq; a.a_scale = shq; a.offsets = offsets; a.tiles = tiles; a.meta = meta;
  a.w0 = (const uint8_t*)w->w_down; a.sh0 = (const uint8_t*)w->sh_down;
  a.s0 = w->b_down; a.shs0 = w->sh_b_down; a.row_w = row_w; a.out16 = out16; a.out32 = out32;
  a.K = p.I; a.N = p.H; a.E = p.E;
  launch_kernel(p, kTimeDown, k_gemm_mx4<false>,
                dim3(xcd_grid(p.max_tiles * (p.H / Mx4Tile::BN))), dim3(Mx4Tile::NT), 0, st, a);
  return check_launch();
}

}  // namespace moe
