// C ABI of the MoE layer: validation, workspace carve and launch sequences.
// Every call validates its arguments before enqueuing anything, never
// synchronises, never copies device memory to the host and never allocates.
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>

#include "moe_internal.h"

// Scratch of moe_forward_noalloc: a fixed array in device memory, one copy per GPU,
// held until the process ends.  In host code `scratch` is only a stand-in for the
// symbol; its device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace moe {

constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's copy of `scratch` (looked up once per device).
static int noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return record_hip_error(err);
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return record_hip_error(err);
    if (!ptr) return MOE_ERR_HIP;
    g_scratch_ptr[dev] = ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

static thread_local char g_hip_error[256] = "no HIP error recorded";

int record_hip_error(hipError_t err) {
  snprintf(g_hip_error, sizeof(g_hip_error), "HIP error %d: %s", int(err), hipGetErrorString(err));
  return MOE_ERR_HIP;
}

int check_launch() {
  const hipError_t err = hipGetLastError();
  return err == hipSuccess ? MOE_OK : record_hip_error(err);
}

static size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int make_plan(const moe_config* c, Plan* p) {
  if (!c || !p) return MOE_ERR_ARG;
  if (c->num_tokens < 1 || c->hidden < 1 || c->intermediate < 1 || c->num_experts < 1 ||
      c->num_groups < 1 || c->topk_groups < 1 || c->topk < 1 || c->num_shared < 0)
    return MOE_ERR_ARG;
  const int64_t T = c->num_tokens;
  const int H = c->hidden, I = c->intermediate, E = c->num_experts, G = c->num_groups;
  const int Gk = c->topk_groups, k = c->topk, S = c->num_shared;
  const int act = c->act_dtype, wt = c->weight_dtype;
  const bool dense32 = act == MOE_F32 && wt == MOE_F32;
  const bool dense16 = act == MOE_BF16 && wt == MOE_BF16;
  const bool fp8 = act == MOE_BF16 && wt == MOE_E4M3_B128;
  const bool nv4 = act == MOE_BF16 && wt == MOE_NVFP4;
  const bool mx4 = act == MOE_BF16 && wt == MOE_MXFP4;
  if (!(dense32 || dense16 || fp8 || nv4 || mx4)) return MOE_ERR_UNSUPPORTED;
  if (H % 8 || I % 8) return MOE_ERR_UNSUPPORTED;
  if (fp8 && (H % 128 || I % 128)) return MOE_ERR_UNSUPPORTED;
  // NVFP4 experts: the decode kernels (a handful of tokens) or the expert-major ones
  if (nv4 && (H % 32 || I % 32 || H > 2048 || I > 1024 || k + S > 32)) return MOE_ERR_UNSUPPORTED;
  // MXFP4 experts: the decode kernels (a handful of tokens) or the block-scaled
  // matrix-core kernels
  if (mx4 && (H % 256 || I % 128 || H > 2048 || I > 2048)) return MOE_ERR_UNSUPPORTED;
  if (E % G || G > 64 || Gk > G) return MOE_ERR_UNSUPPORTED;
  if (int64_t(k) > int64_t(Gk) * (E / G) || k > 16) return MOE_ERR_UNSUPPORTED;
  if (E + S > 1024) return MOE_ERR_UNSUPPORTED;
  if (T * int64_t(k + S) >= (int64_t(1) << 31)) return MOE_ERR_UNSUPPORTED;

  Plan q{};
  q.T = T; q.H = H; q.I = I; q.E = E; q.G = G; q.Gk = Gk; q.k = k; q.S = S;
  q.act = act; q.wt = wt;
  q.Rk = T * k;
  q.R = T * int64_t(k + S);
  q.nblk = int((T + 63) / 64);
  const bool mfma_shape = H % 128 == 0 && I % 64 == 0;
  // Few rows per expert on average: the weight stream dominates, skinny kernels.
  q.skinny = dense32 || (dense16 && (q.Rk <= 8 * int64_t(E) || !mfma_shape));
  if (nv4) q.skinny = q.Rk <= 8 * int64_t(E) || !nv4_mfma_ok(q);
  q.small_route = T <= 64 && T * k <= 256;
  q.fused_down = q.skinny && T <= 16;
  // NVFP4 batches the decode kernels do not take run the expert-major kernels + combine
  if (nv4 && q.fused_down && !decode_ffn_ok(q)) q.fused_down = false;
  // MXFP4: the decode kernels where they apply, else the matrix-core kernels
  if (mx4) {
    q.skinny = q.fused_down = T <= 16 && q.Rk <= 8 * int64_t(E);
    if (q.skinny && !decode_ffn_ok(q)) q.skinny = q.fused_down = false;
  }
  q.max_active = std::min<int64_t>(E, q.Rk) + S;
  q.bm = gemm_tile_rows(q);
  q.max_tiles = q.Rk / q.bm + std::min<int64_t>(E, q.Rk) + int64_t(S) * ((T + q.bm - 1) / q.bm);

  size_t o = 0;
  auto take = [&](size_t bytes) { const size_t at = o; o = align256(o + bytes); return at; };
  q.o_logits = take(size_t(T) * E * 4);
  q.o_ids = take(size_t(q.Rk) * 4);
  q.o_w = take(size_t(q.Rk) * 4);
  q.o_blk = take(size_t(2) * q.nblk * E * 4);   // [2][nblk][E]: the row selection counts half blocks
  q.o_off = take(size_t(E + S + 1) * 4);
  q.o_meta = take(16);
  q.o_active = take(size_t(E + S) * 4);
  q.o_tiles = take(size_t(q.max_tiles) * 8);
  q.o_rowtok = take(size_t(q.R) * 4);
  q.o_inv = take(size_t(q.Rk) * 4);
  q.o_roww = take(size_t(q.R) * 4);
  q.o_h = take(size_t(q.R) * I * 4);
  q.o_ypw = take(q.skinny ? 0 : size_t(q.R) * H * 2);
  q.o_yp32 = take(q.skinny && !q.fused_down ? size_t(q.R) * H * 4 : 0);
  // activation codes and scales: fp32 per 128 (block FP8) or one E8M0 byte per 32 (MXFP4),
  // the same number of bytes
  q.o_xq = take(fp8 || mx4 ? size_t(T) * H : 0);
  q.o_sx = take(fp8 || mx4 ? size_t(T) * (H / 128) * 4 : 0);
  q.o_hq = take(fp8 || mx4 ? size_t(q.R) * I : 0);
  q.o_shq = take(fp8 || mx4 ? size_t(q.R) * (I / 128) * 4 : 0);
  q.o_xn = take(size_t(T) * H * (act == MOE_F32 ? 4 : 2));   // normalised rows (decoder step)
  q.total = o;
  *p = q;
  return MOE_OK;
}

template <typename T>
static T* at(void* ws, size_t off) {
  return reinterpret_cast<T*>(static_cast<char*>(ws) + off);
}

static int check_ws(const Plan& p, const void* ws, size_t ws_bytes) {
  if (!ws) return MOE_ERR_ARG;
  if ((reinterpret_cast<uintptr_t>(ws) & 255) != 0) return MOE_ERR_ARG;
  if (ws_bytes < p.total) return MOE_ERR_WORKSPACE;
  return MOE_OK;
}

static int check_experts(const Plan& p, const moe_weights* w) {
  if (!w || !w->w_gate || !w->w_up || !w->w_down) return MOE_ERR_ARG;
  if (p.S > 0 && (!w->sh_gate || !w->sh_up || !w->sh_down)) return MOE_ERR_ARG;
  if (p.wt == MOE_E4M3_B128) {
    if (!w->s_gate || !w->s_up || !w->s_down) return MOE_ERR_ARG;
    if (p.S > 0 && (!w->sh_s_gate || !w->sh_s_up || !w->sh_s_down)) return MOE_ERR_ARG;
  }
  if (p.wt == MOE_MXFP4) {
    if (!w->b_gate || !w->b_up || !w->b_down) return MOE_ERR_ARG;
    if (p.S > 0 && (!w->sh_b_gate || !w->sh_b_up || !w->sh_b_down)) return MOE_ERR_ARG;
  }
  if (p.wt == MOE_NVFP4) {
    if (!w->b_gate || !w->b_up || !w->b_down || !w->g_gate || !w->g_up || !w->g_down)
      return MOE_ERR_ARG;
    if (p.S > 0 && (!w->sh_b_gate || !w->sh_b_up || !w->sh_b_down || !w->sh_g_gate ||
                    !w->sh_g_up || !w->sh_g_down))
      return MOE_ERR_ARG;
  }
  return MOE_OK;
}

// Expert FFN on permuted rows (schedule already in the workspace).
static int run_experts(const Plan& p, const void* x, const int32_t* off, const int32_t* rowtok,
                       const moe_weights* w, void* ws, float* y_perm32, bf16_t* y_perm16,
                       const float* row_w, hipStream_t st) {
  int32_t* active = at<int32_t>(ws, p.o_active);
  int32_t* meta = at<int32_t>(ws, p.o_meta);
  int2* tiles = at<int2>(ws, p.o_tiles);
  // (MXFP4 experts have no skinny kernels: the matrix-core ones take every batch here)
  if (p.skinny && p.wt != MOE_MXFP4) {
    float* h = at<float>(ws, p.o_h);
    MOE_TRY(launch_gateup_skinny(p, x, rowtok, off, active, meta, w, h, st));
    return launch_down_skinny(p, h, off, active, meta, w, y_perm32, st);
  }
  if (p.wt == MOE_BF16 || p.wt == MOE_NVFP4) {
    bf16_t* h = at<bf16_t>(ws, p.o_h);
    MOE_TRY(launch_gateup_mfma(p, x, rowtok, off, tiles, meta, w, h, nullptr, nullptr, nullptr,
                               nullptr, st));
    return launch_down_mfma(p, h, off, tiles, meta, w, row_w, y_perm32, y_perm16, nullptr, st);
  }
  uint8_t* xq = at<uint8_t>(ws, p.o_xq);
  float* sx = at<float>(ws, p.o_sx);
  uint8_t* hq = at<uint8_t>(ws, p.o_hq);
  float* shq = at<float>(ws, p.o_shq);
  float* h = at<float>(ws, p.o_h);
  if (p.wt == MOE_MXFP4) {
    uint8_t* sx8 = at<uint8_t>(ws, p.o_sx);
    uint8_t* shq8 = at<uint8_t>(ws, p.o_shq);
    MOE_TRY(launch_quant_mx(x, p.T, p.H, xq, sx8, st));
    MOE_TRY(launch_gateup_mx4(p, xq, sx8, rowtok, off, tiles, meta, w, hq, shq8, st));
    return launch_down_mx4(p, hq, shq8, off, tiles, meta, w, row_w, y_perm32, y_perm16, st);
  }
  MOE_TRY(launch_quant(p, x, true, p.T, p.H, xq, sx, st));
  MOE_TRY(launch_gateup_mfma(p, x, rowtok, off, tiles, meta, w, h, xq, sx, hq, shq, st));
  return launch_down_mfma(p, hq, off, tiles, meta, w, row_w, y_perm32, y_perm16, shq, st);
}

// Paged layer: the routing plan (original experts) and the slot-space plan (the
// arena's N slots as the experts of the permutation and the expert kernels).
struct PagedPlan {
  Plan route, slots;
  int N;
  size_t o_slots, o_ids_slot, o_copies, o_yp, total;
  int64_t mat_bytes[3];
};

static int make_paged_plan(const moe_config* c, int32_t num_slots, PagedPlan* pp) {
  PagedPlan q{};
  MOE_TRY(make_plan(c, &q.route));
  const Plan& p = q.route;
  if (p.wt != MOE_F32 && p.wt != MOE_BF16) return MOE_ERR_UNSUPPORTED;
  // every expert one call can need fits, and no more slots than experts
  if (num_slots < std::min<int64_t>(p.E, p.Rk) || num_slots > p.E) return MOE_ERR_UNSUPPORTED;
  moe_config cs = *c;
  cs.num_experts = num_slots;
  cs.num_groups = 1;
  cs.topk_groups = 1;
  MOE_TRY(make_plan(&cs, &q.slots));
  q.N = num_slots;
  size_t o = align256(p.total);
  q.o_slots = o;
  o = align256(o + q.slots.total);
  q.o_ids_slot = o;
  o = align256(o + size_t(p.Rk) * 4);
  q.o_copies = o;
  o = align256(o + size_t(1 + 2 * std::min<int64_t>(num_slots, p.Rk)) * 4);
  q.o_yp = o;
  o = align256(o + size_t(p.R) * p.H * 4);
  q.total = o;
  const int64_t b = p.wt == MOE_F32 ? 4 : 2;
  q.mat_bytes[0] = q.mat_bytes[1] = q.mat_bytes[2] = int64_t(p.I) * p.H * b;
  *pp = q;
  return MOE_OK;
}

// Device address under which a kernel reads `p`: pinned host memory (hipHostMalloc,
// torch pin_memory) or device memory; MOE_ERR_ARG for memory HIP does not know.  For
// host memory the pointer attributes and hipHostGetDevicePointer must agree.
static int device_view(const void* p, const void** out) {
  hipPointerAttribute_t a;
  if (hipPointerGetAttributes(&a, p) != hipSuccess || !a.devicePointer) {
    (void)hipGetLastError();   // the failed query must not surface as a launch error later
    return MOE_ERR_ARG;
  }
  if (a.type == hipMemoryTypeDevice) {
    *out = p;
    return MOE_OK;
  }
  if (a.type != hipMemoryTypeHost) return MOE_ERR_ARG;
  const char* hp = static_cast<const char*>(a.hostPointer);
  const void* v = static_cast<const char*>(a.devicePointer) + (hp ? static_cast<const char*>(p) - hp : 0);
  void* d = nullptr;
  if (hipHostGetDevicePointer(&d, const_cast<void*>(p), 0) != hipSuccess || d != v) {
    (void)hipGetLastError();
    return MOE_ERR_ARG;
  }
  *out = v;
  return MOE_OK;
}

// device_view of a whole array of `bytes`: its first and last byte must both be known
// to HIP and map to one contiguous device range.
static int device_range(const void* p, int64_t bytes, const void** out) {
  const void* first = nullptr;
  const void* last = nullptr;
  MOE_TRY(device_view(p, &first));
  MOE_TRY(device_view(static_cast<const char*>(p) + bytes - 1, &last));
  if (static_cast<const char*>(last) != static_cast<const char*>(first) + bytes - 1) return MOE_ERR_ARG;
  *out = first;
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int moe_workspace_size(const moe_config* cfg, size_t* bytes) {
  if (!bytes) return MOE_ERR_ARG;
  Plan p;
  MOE_TRY(make_plan(cfg, &p));
  *bytes = p.total;
  return MOE_OK;
}

int moe_workspace_slot(const moe_config* cfg, int slot, size_t* offset, size_t* bytes) {
  if (!offset || !bytes) return MOE_ERR_ARG;
  Plan p;
  MOE_TRY(make_plan(cfg, &p));
  const bool fp8 = p.wt == MOE_E4M3_B128, mx4 = p.wt == MOE_MXFP4;
  switch (slot) {
    case MOE_WS_LOGITS: *offset = p.o_logits; *bytes = size_t(p.T) * p.E * 4; break;
    case MOE_WS_ACT_CODES: *offset = p.o_xq; *bytes = fp8 || mx4 ? size_t(p.T) * p.H : 0; break;
    case MOE_WS_ACT_SCALES:
      *offset = p.o_sx;
      *bytes = fp8 ? size_t(p.T) * (p.H / 128) * 4 : mx4 ? size_t(p.T) * (p.H / 32) : 0;
      break;
    case MOE_WS_NORM_ROWS:
      *offset = p.o_xn;
      *bytes = size_t(p.T) * p.H * (p.act == MOE_F32 ? 4 : 2);
      break;
    default: return MOE_ERR_ARG;
  }
  return MOE_OK;
}

int moe_route(const moe_config* cfg, const void* x, const void* w_router, const float* router_bias,
              int32_t* topk_ids, float* topk_w, float* logits, void* ws, size_t ws_bytes,
              hipStream_t stream) {
  Plan p;
  MOE_TRY(make_plan(cfg, &p));
  if (!x || !w_router || !topk_ids || !topk_w) return MOE_ERR_ARG;
  MOE_TRY(check_ws(p, ws, ws_bytes));
  float* lg = logits ? logits : at<float>(ws, p.o_logits);
  MOE_TRY(launch_logits(p, x, w_router, router_bias, lg, stream));
  return launch_select(p, lg, topk_ids, topk_w, nullptr, stream);
}

int moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t* expert_offsets,
                int32_t* row_token, int32_t* inv_rows, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  Plan p;
  MOE_TRY(make_plan(cfg, &p));
  if (!topk_ids || !expert_offsets || !row_token || !inv_rows) return MOE_ERR_ARG;
  MOE_TRY(check_ws(p, ws, ws_bytes));
  return launch_permute(p, topk_ids, nullptr, at<int32_t>(ws, p.o_blk), expert_offsets,
                        at<int32_t>(ws, p.o_active), at<int32_t>(ws, p.o_meta),
                        at<int2>(ws, p.o_tiles), row_token, inv_rows, nullptr, p.bm, stream);
}

int moe_expert_ffn(const moe_config* cfg, const void* x, const int32_t* expert_offsets,
                   const int32_t* row_token, const moe_weights* w, float* y_perm, void* ws,
                   size_t ws_bytes, hipStream_t stream) {
  Plan p;
  MOE_TRY(make_plan(cfg, &p));
  if (!x || !expert_offsets || !row_token || !y_perm) return MOE_ERR_ARG;
  MOE_TRY(check_experts(p, w));
  MOE_TRY(check_ws(p, ws, ws_bytes));
  MOE_TRY(launch_schedule(p, expert_offsets, at<int32_t>(ws, p.o_active),
                          at<int32_t>(ws, p.o_meta), at<int2>(ws, p.o_tiles), p.bm, stream));
  return run_experts(p, x, expert_offsets, row_token, w, ws, y_perm, nullptr, nullptr, stream);
}

int moe_combine(const moe_config* cfg, const float* y_perm, const int32_t* expert_offsets,
                const int32_t* inv_rows, const float* topk_w, void* y, hipStream_t stream) {
  Plan p;
  MOE_TRY(make_plan(cfg, &p));
  if (!y_perm || !expert_offsets || !inv_rows || !topk_w || !y) return MOE_ERR_ARG;
  return launch_combine(p, y_perm, expert_offsets, inv_rows, topk_w, nullptr, y, stream);
}

// The layer on x, or (gamma != null) the decoder step around it: x_n = RMSNorm(x) feeds
// the router and the experts and x (`res`) is added to the combined output.
static int forward_impl(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                        int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                        hipStream_t stream, hipEvent_t* ev, const void* gamma = nullptr,
                        float eps = 0.f) {
  Plan p;
  MOE_TRY(make_plan(cfg, &p));
  if (ev)
    for (int i = 0; i < MOE_TIMED_EVENTS; ++i) p.ev[i] = ev[i];
  if (!x || !y || !w || !w->w_router) return MOE_ERR_ARG;
  MOE_TRY(check_experts(p, w));
  MOE_TRY(check_ws(p, ws, ws_bytes));
  const void* res = gamma ? x : nullptr;
  void* xn = at<void>(ws, p.o_xn);
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, p.o_ids);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, p.o_w);
  float* logits = at<float>(ws, p.o_logits);
  int32_t* off = at<int32_t>(ws, p.o_off);
  int32_t* active = at<int32_t>(ws, p.o_active);
  int32_t* meta = at<int32_t>(ws, p.o_meta);
  int2* tiles = at<int2>(ws, p.o_tiles);
  int32_t* rowtok = at<int32_t>(ws, p.o_rowtok);
  int32_t* inv = at<int32_t>(ws, p.o_inv);
  float* row_w = at<float>(ws, p.o_roww);

  int32_t* blk = at<int32_t>(ws, p.o_blk);
  bool x_quantised = false;   // x's FP8 / MX codes already written by the selection launch
  if (p.fused_down && decode_ffn_ok(p)) {
    // decode: the logits (with the norm in front for the decoder step), then gate/up
    // (routing in every block) and down + combine (+ residual)
    if (gamma) {
      MOE_TRY(launch_logits_norm(p, x, gamma, eps, w->w_router, w->router_bias, logits, xn, stream));
      x = xn;
    } else {
      MOE_TRY(launch_logits(p, x, w->w_router, w->router_bias, logits, stream));
    }
    return launch_decode_ffn(p, x, logits, w, ids, wts, off, rowtok, inv, at<float>(ws, p.o_h),
                             res, y, at<uint8_t>(ws, p.o_xq), at<uint8_t>(ws, p.o_sx), stream);
  }
  if (gamma) {
    MOE_TRY(launch_rmsnorm(p, x, gamma, eps, xn, stream));
    x = xn;
  }
  if (p.small_route) {
    MOE_TRY(launch_logits(p, x, w->w_router, w->router_bias, logits, stream));
    MOE_TRY(launch_route_permute_small(p, logits, ids, wts, off, active, meta, tiles, rowtok, inv,
                                       row_w, p.bm, stream));
  } else {
    MOE_TRY(launch_logits(p, x, w->w_router, w->router_bias, logits, stream));
    // the matrix-core FP8 / MX expert kernels read x's codes: their quantisation rides
    // in the selection launch where the row selection runs
    XQuant xq;
    if (!p.skinny && select_rows_ok(p) && (p.wt == MOE_E4M3_B128 || p.wt == MOE_MXFP4)) {
      xq.x = static_cast<const bf16_t*>(x);
      xq.rows = p.T;
      xq.K = p.H;
      xq.mx = p.wt == MOE_MXFP4;
      xq.codes = at<uint8_t>(ws, p.o_xq);
      xq.scales = at<void>(ws, p.o_sx);
      x_quantised = true;
    }
    MOE_TRY(launch_select(p, logits, ids, wts, blk, stream, xq));
    const int32_t* blk2 = select_rows_ok(p) ? blk + size_t(p.nblk) * p.E : nullptr;
    MOE_TRY(launch_scan_scatter(p, ids, wts, blk, blk2, off, active, meta, tiles, rowtok, inv,
                                row_w, p.bm, stream));
  }
  if (p.skinny) {
    float* h = at<float>(ws, p.o_h);
    MOE_TRY(launch_gateup_skinny(p, x, rowtok, off, active, meta, w, h, stream));
    if (p.fused_down) return launch_down_combine_skinny(p, h, ids, wts, inv, w, res, y, stream);
    float* yp = at<float>(ws, p.o_yp32);
    MOE_TRY(launch_down_skinny(p, h, off, active, meta, w, yp, stream));
    return launch_combine(p, yp, off, inv, wts, res, y, stream);
  }
  bf16_t* ypw = at<bf16_t>(ws, p.o_ypw);
  if (p.wt == MOE_BF16 || p.wt == MOE_NVFP4) {
    bf16_t* h = at<bf16_t>(ws, p.o_h);
    MOE_TRY(launch_gateup_mfma(p, x, rowtok, off, tiles, meta, w, h, nullptr, nullptr, nullptr,
                               nullptr, stream));
    MOE_TRY(launch_down_mfma(p, h, off, tiles, meta, w, row_w, nullptr, ypw, nullptr, stream));
  } else if (p.wt == MOE_MXFP4) {
    uint8_t* xq = at<uint8_t>(ws, p.o_xq);
    uint8_t* sx8 = at<uint8_t>(ws, p.o_sx);
    uint8_t* hq = at<uint8_t>(ws, p.o_hq);
    uint8_t* shq8 = at<uint8_t>(ws, p.o_shq);
    if (!x_quantised) MOE_TRY(launch_quant_mx(x, p.T, p.H, xq, sx8, stream));
    MOE_TRY(launch_gateup_mx4(p, xq, sx8, rowtok, off, tiles, meta, w, hq, shq8, stream));
    MOE_TRY(launch_down_mx4(p, hq, shq8, off, tiles, meta, w, row_w, nullptr, ypw, stream));
  } else {
    uint8_t* xq = at<uint8_t>(ws, p.o_xq);
    float* sx = at<float>(ws, p.o_sx);
    uint8_t* hq = at<uint8_t>(ws, p.o_hq);
    float* shq = at<float>(ws, p.o_shq);
    float* h = at<float>(ws, p.o_h);
    if (!x_quantised) MOE_TRY(launch_quant(p, x, true, p.T, p.H, xq, sx, stream));
    MOE_TRY(launch_gateup_mfma(p, x, rowtok, off, tiles, meta, w, h, xq, sx, hq, shq, stream));
    MOE_TRY(launch_down_mfma(p, hq, off, tiles, meta, w, row_w, nullptr, ypw, shq, stream));
  }
  return launch_combine_preweighted(p, ypw, off, inv, res, y, stream);
}

int moe_forward(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                hipStream_t stream) {
  return forward_impl(cfg, x, w, y, topk_ids_out, topk_w_out, ws, ws_bytes, stream, nullptr);
}

int moe_forward_timed(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                      int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                      hipStream_t stream, hipEvent_t* kernel_events) {
  if (!kernel_events) return MOE_ERR_ARG;
  for (int i = 0; i < MOE_TIMED_EVENTS; ++i)
    if (!kernel_events[i]) return MOE_ERR_ARG;
  return forward_impl(cfg, x, w, y, topk_ids_out, topk_w_out, ws, ws_bytes, stream, kernel_events);
}

int moe_forward_noalloc(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                        int32_t* topk_ids_out, float* topk_w_out, hipStream_t stream) {
  Plan p;
  MOE_TRY(make_plan(cfg, &p));
  if (!x || !y || !w || !w->w_router) return MOE_ERR_ARG;
  MOE_TRY(check_experts(p, w));
  if (p.total > size_t(MOE_NOALLOC_SCRATCH_BYTES)) return MOE_ERR_SCRATCH;
  void* ws = nullptr;
  MOE_TRY(noalloc_scratch(&ws));
  return forward_impl(cfg, x, w, y, topk_ids_out, topk_w_out, ws, MOE_NOALLOC_SCRATCH_BYTES,
                      stream, nullptr);
}

int moe_pager_state_layout(const moe_config* cfg, int32_t num_slots, size_t* offsets,
                           size_t* bytes) {
  if (!bytes) return MOE_ERR_ARG;
  PagedPlan pp;
  MOE_TRY(make_paged_plan(cfg, num_slots, &pp));
  const PagerLayout L = pager_layout(pp.route.E, num_slots);
  if (offsets) {
    offsets[0] = L.o_counters;
    offsets[1] = L.o_key_slot;
    offsets[2] = L.o_slot_key;
    offsets[3] = L.o_stamp;
  }
  *bytes = L.total;
  return MOE_OK;
}

int moe_pager_reset(const moe_config* cfg, int32_t num_slots, void* state, hipStream_t stream) {
  PagedPlan pp;
  MOE_TRY(make_paged_plan(cfg, num_slots, &pp));
  if (!state) return MOE_ERR_ARG;
  return launch_pager_reset(pp.route.E, num_slots, state, stream);
}

int moe_paged_workspace_size(const moe_config* cfg, int32_t num_slots, size_t* bytes) {
  if (!bytes) return MOE_ERR_ARG;
  PagedPlan pp;
  MOE_TRY(make_paged_plan(cfg, num_slots, &pp));
  *bytes = pp.total;
  return MOE_OK;
}

int moe_forward_paged(const moe_config* cfg, const void* x, const moe_weights* host_experts,
                      const moe_weights* resident, int32_t num_slots, void* state, void* y,
                      int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                      hipStream_t stream) {
  PagedPlan pp;
  MOE_TRY(make_paged_plan(cfg, num_slots, &pp));
  const Plan& p = pp.route;
  const Plan& q = pp.slots;
  if (!x || !y || !state || !host_experts || !resident || !resident->w_router) return MOE_ERR_ARG;
  if (!host_experts->w_gate || !host_experts->w_up || !host_experts->w_down) return MOE_ERR_ARG;
  MOE_TRY(check_experts(q, resident));
  MOE_TRY(check_ws(p, ws, ws_bytes));
  if (ws_bytes < pp.total) return MOE_ERR_WORKSPACE;
  PagerCopyArgs ca{};
  MOE_TRY(device_range(host_experts->w_gate, p.E * pp.mat_bytes[0], &ca.src[0]));
  MOE_TRY(device_range(host_experts->w_up, p.E * pp.mat_bytes[1], &ca.src[1]));
  MOE_TRY(device_range(host_experts->w_down, p.E * pp.mat_bytes[2], &ca.src[2]));
  ca.dst[0] = const_cast<void*>(resident->w_gate);
  ca.dst[1] = const_cast<void*>(resident->w_up);
  ca.dst[2] = const_cast<void*>(resident->w_down);
  for (int j = 0; j < 3; ++j) ca.chunks[j] = pp.mat_bytes[j] / 16;

  // routing over the layer's experts
  float* logits = at<float>(ws, p.o_logits);
  int32_t* ids = topk_ids_out ? topk_ids_out : at<int32_t>(ws, p.o_ids);
  float* wts = topk_w_out ? topk_w_out : at<float>(ws, p.o_w);
  MOE_TRY(launch_logits(p, x, resident->w_router, resident->router_bias, logits, stream));
  MOE_TRY(launch_select(p, logits, ids, wts, nullptr, stream));
  // residency: plan on the device, copy the misses into their slots
  int32_t* ids_slot = at<int32_t>(ws, pp.o_ids_slot);
  int32_t* copies = at<int32_t>(ws, pp.o_copies);
  MOE_TRY(launch_pager_plan(ids, int(p.Rk), p.E, pp.N, 3 * pp.mat_bytes[0], state, ids_slot,
                            copies, stream));
  MOE_TRY(launch_pager_copy(copies, ca, int(std::min<int64_t>(pp.N, p.Rk)), stream));
  // the rest of the layer over the slots: permutation, experts, combine
  void* wq = static_cast<char*>(ws) + pp.o_slots;
  int32_t* off = at<int32_t>(wq, q.o_off);
  int32_t* rowtok = at<int32_t>(wq, q.o_rowtok);
  int32_t* inv = at<int32_t>(wq, q.o_inv);
  MOE_TRY(launch_permute(q, ids_slot, nullptr, at<int32_t>(wq, q.o_blk), off,
                         at<int32_t>(wq, q.o_active), at<int32_t>(wq, q.o_meta),
                         at<int2>(wq, q.o_tiles), rowtok, inv, nullptr, q.bm, stream));
  float* yp = at<float>(ws, pp.o_yp);
  MOE_TRY(run_experts(q, x, off, rowtok, resident, wq, yp, nullptr, nullptr, stream));
  return launch_combine(q, yp, off, inv, wts, nullptr, y, stream);
}

int moe_forward_residual(const moe_config* cfg, const void* x, const void* norm_weight,
                         float norm_eps, const moe_weights* w, void* x_out, int32_t* topk_ids_out,
                         float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!norm_weight || !(norm_eps >= 0.f)) return MOE_ERR_ARG;
  return forward_impl(cfg, x, w, x_out, topk_ids_out, topk_w_out, ws, ws_bytes, stream, nullptr,
                      norm_weight, norm_eps);
}

const char* moe_strerror(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_ARG: return "invalid argument (null pointer, non-positive size or misaligned workspace)";
    case MOE_ERR_UNSUPPORTED: return "unsupported configuration (shape or dtype combination)";
    case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_size()";
    case MOE_ERR_HIP: return g_hip_error;
    case MOE_ERR_SCRATCH:
      return "config needs more scratch than moe_forward_noalloc holds (MOE_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
