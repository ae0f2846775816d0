/*
 * moe.h - C ABI of the fine-grained MoE layer on MI355X (gfx950).
 *
 * The layer (route -> permute -> grouped SwiGLU experts -> weighted combine) is
 * the one the pages describe for Ling-3.0-tiny and Inkling:
 *   - TensorFold issue #1247 "Ling-3.0-tiny on a Qualcomm board", jschmied's
 *     comment, config paragraph: 128 experts in 8 groups of 16 with 4 groups
 *     kept, hidden 1536, SwiGLU experts whose limit lists are null (no clamp);
 *     list "What it does not cover": the router is group-limited, and the bf16
 *     experts are computed per expert over the rows routed to it, a grouping
 *     that costs a host synchronisation per layer there.
 *   - HelloSun/ling30tiny model card, routing table (模型與路由): 8 experts per
 *     token; numeric-check summary (數值檢查摘要): routing plus a weighted layer.
 *   - llama.cpp PR "Add TML Inkling architecture", PR summary: 256 experts,
 *     top-6, plus 2 shared experts; large MoEs need 64-bit index arithmetic.
 *
 * Conventions shared by every call
 *   - Every pointer argument except `cfg`/`w` structs is a DEVICE pointer
 *     (memory from hipMalloc or a torch CUDA tensor); the structs themselves
 *     live in host memory and are read during the call only.
 *   - Layouts are row-major.  Expert matrices are [out, in] per expert, experts
 *     stacked: gate/up [E, I, H], down [E, H, I].  Shared experts have their
 *     own arrays of the same form with S in place of E.
 *   - Work is enqueued asynchronously on `stream`.  No call synchronises, copies
 *     device memory to the host, or allocates: every call can be captured into
 *     a HIP graph.  The caller owns every buffer and must keep it alive until
 *     the stream has finished the work.  The library keeps no pointer after a
 *     call returns and holds no device state, so calls on different streams
 *     with distinct workspaces may run concurrently.
 *   - The workspace `ws` is scratch memory of at least moe_workspace_size()
 *     bytes for the same config, 256-byte aligned; its contents on entry are
 *     ignored and on exit are unspecified.
 *   - Errors: every call returns MOE_OK (0) or a negative MOE_ERR_* code.
 *     Arguments are validated before anything is enqueued, so a failing call
 *     enqueues nothing (except MOE_ERR_HIP, reported after a launch failed).
 *     No C++ exception crosses this interface.  Preconditions that are NOT
 *     checked (checking would need a device-to-host sync): caller-supplied
 *     expert ids lie in [0, E) and are distinct per token; offsets/rows passed
 *     to moe_expert_ffn / moe_combine are the ones moe_permute produced for
 *     the same config; inputs are finite.
 *   - Determinism: for a fixed config, inputs and device, outputs are bitwise
 *     identical from run to run (no floating-point atomics anywhere).
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Status codes. */
#define MOE_OK               0
#define MOE_ERR_ARG         -1   /* null required pointer, non-positive size */
#define MOE_ERR_UNSUPPORTED -2   /* shape/dtype combination outside the supported set */
#define MOE_ERR_WORKSPACE   -3   /* workspace smaller than moe_workspace_size() */
#define MOE_ERR_HIP         -4   /* a HIP launch failed; moe_strerror() has the HIP text */
#define MOE_ERR_SCRATCH     -5   /* moe_forward_noalloc: the config needs more scratch than
                                    MOE_NOALLOC_SCRATCH_BYTES */

/* Element types. */
typedef enum {
  MOE_F32 = 0,        /* IEEE fp32 */
  MOE_BF16 = 1,       /* bfloat16 */
  MOE_E4M3_B128 = 2,  /* expert weights only: OCP e4m3 codes (uint8) with one fp32
                         scale per 128x128 block, value = decode(code) * scale */
  MOE_NVFP4 = 3,      /* expert weights only: FP4 E2M1 codes, two per byte (element 2i
                         in the low nibble), one OCP e4m3 scale per 16 consecutive
                         inputs and one fp32 scale per expert matrix,
                         value = e2m1(code) * e4m3(block scale) * matrix scale.  The
                         4-bit expert format TensorFold issue #1247 "Ling-3.0-tiny on a
                         Qualcomm board" names in its list "What it does not cover";
                         its layout is not on the pages and this one is a reading. */
  MOE_MXFP4 = 4       /* expert weights only: OCP Microscaling FP4 - E2M1 codes, two per
                         byte (element 2i in the low nibble), one E8M0 scale code per 32
                         consecutive inputs, value = e2m1(code) * 2^(scale - 127).  The layer
                         then quantises its activations (x, and h before the down
                         projection) per row per 32 to MXFP8 (E4M3 codes, E8M0 shared
                         exponent floor(log2(amax)) - 8); batches beyond a handful of
                         tokens multiply both operands on the block-scaled matrix cores,
                         up to 16 tokens the decode kernels form the same E2M1 x E4M3
                         products on the vector units.  A reading of the 4-bit experts the
                         pages name (TensorFold #1247, list "What it does not cover"; the
                         graysoft ROCmFP4 page) with the format gfx950 takes natively. */
} moe_dtype;

/*
 * Layer configuration.  Supported element-type pairs (act_dtype, weight_dtype):
 *   (MOE_F32, MOE_F32), (MOE_BF16, MOE_BF16), (MOE_BF16, MOE_E4M3_B128),
 *   (MOE_BF16, MOE_NVFP4), (MOE_BF16, MOE_MXFP4).
 * Constraints: T >= 1; H, I >= 1 and multiples of 8 (of 128 for e4m3 experts, of
 * 32 for NVFP4 experts, which also need H <= 2048, I <= 1024 and k + S <= 32; MXFP4
 * experts need H % 256 == 0, I % 128 == 0, H <= 2048 and I <= 2048);
 * E >= 1; G >= 1 with E % G == 0; 1 <= Gk <= G; 1 <= k <= Gk * E / G;
 * k <= 16; E + S <= 1024; T * (k + S) < 2^31.
 */
typedef struct {
  int64_t num_tokens;     /* T: tokens in this call */
  int32_t hidden;         /* H */
  int32_t intermediate;   /* I: SwiGLU intermediate size of every expert */
  int32_t num_experts;    /* E: routed experts */
  int32_t num_groups;     /* G: expert groups (1 = ungrouped); group g = experts [g*E/G, (g+1)*E/G) */
  int32_t topk_groups;    /* Gk: groups kept per token */
  int32_t topk;           /* k: routed experts per token */
  int32_t num_shared;     /* S: always-on shared experts, weight 1 */
  int32_t act_dtype;      /* x, router weight, y: MOE_F32 | MOE_BF16 */
  int32_t weight_dtype;   /* experts: MOE_F32 | MOE_BF16 | MOE_E4M3_B128 | MOE_NVFP4 */
} moe_config;

/* Weights of one layer (device pointers).  s_* scales are used only for MOE_E4M3_B128,
 * b_* and g_* only for MOE_NVFP4 (whose w_* arrays then hold packed codes:
 * gate/up [E, I, H/2] bytes, down [E, H, I/2] bytes).  MOE_MXFP4 uses the same packed
 * w_* arrays and b_* as E8M0 scale codes, gate/up [E, I, H/32], down [E, H, I/32]. */
typedef struct {
  const void*  w_router;      /* [E, H] act_dtype */
  const float* router_bias;   /* [E] fp32, added to the logits before the softmax; NULL = none */
  const void*  w_gate;        /* [E, I, H] weight_dtype */
  const void*  w_up;          /* [E, I, H] */
  const void*  w_down;        /* [E, H, I] */
  const float* s_gate;        /* [E, I/128, H/128] fp32 block scales (e4m3 only) */
  const float* s_up;          /* [E, I/128, H/128] */
  const float* s_down;        /* [E, H/128, I/128] */
  const void*  sh_gate;       /* [S, I, H]; NULL when S == 0 */
  const void*  sh_up;         /* [S, I, H] */
  const void*  sh_down;       /* [S, H, I] */
  const float* sh_s_gate;     /* [S, I/128, H/128] (e4m3 only) */
  const float* sh_s_up;       /* [S, I/128, H/128] */
  const float* sh_s_down;     /* [S, H/128, I/128] */
  const uint8_t* b_gate;      /* [E, I, H/16] e4m3 block scales (NVFP4 only) */
  const uint8_t* b_up;        /* [E, I, H/16] */
  const uint8_t* b_down;      /* [E, H, I/16] */
  const float* g_gate;        /* [E] fp32 scale of each expert matrix (NVFP4 only) */
  const float* g_up;          /* [E] */
  const float* g_down;        /* [E] */
  const uint8_t* sh_b_gate;   /* [S, I, H/16] (NVFP4 only) */
  const uint8_t* sh_b_up;     /* [S, I, H/16] */
  const uint8_t* sh_b_down;   /* [S, H, I/16] */
  const float* sh_g_gate;     /* [S] */
  const float* sh_g_up;       /* [S] */
  const float* sh_g_down;     /* [S] */
} moe_weights;

/*
 * Bytes of workspace any call below needs for `cfg` (host only, no device work).
 * Returns MOE_OK and writes *bytes, or a validation error.
 */
int moe_workspace_size(const moe_config* cfg, size_t* bytes);

/*
 * Router (group-limited routing of TensorFold #1247, "What it does not cover"):
 *   l[t,e] = sum_h x[t,h] W_r[e,h] (+ bias[e]), fp32 accumulation;
 *   s = softmax over all E logits;  group score = max s in the group;
 *   keep the Gk best groups, then the k best experts inside them
 *   (ties: lower group / expert index wins);  w = s[ids] / sum s[ids].
 * x [T,H] act_dtype.  Outputs: topk_ids [T,k] int32 ordered by score
 * descending (ties by lower id); topk_w [T,k] fp32; logits [T,E] fp32 with the
 * bias included, or NULL to skip writing them.
 */
int moe_route(const moe_config* cfg, const void* x, const void* w_router, const float* router_bias,
              int32_t* topk_ids, float* topk_w, float* logits,
              void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Permutation: the slots grouped by expert (the rows-per-expert grouping of
 * TensorFold #1247, list "What it does not cover"), computed on the device
 * without a host sync.
 * R = T*k + T*S rows.  Rows of routed expert e are the slots (t,j) with
 * topk_ids[t,j] == e, in ascending (t, j) order; shared expert s owns rows
 * [T*k + s*T, T*k + (s+1)*T), one per token in order.
 * Outputs: expert_offsets [E+S+1] int32 (exclusive prefix sum of the row
 * counts, expert_offsets[E+S] == R); row_token [R] int32 (token of each row);
 * inv_rows [T,k] int32 (row of each routed slot).
 */
int moe_permute(const moe_config* cfg, const int32_t* topk_ids, int32_t* expert_offsets,
                int32_t* row_token, int32_t* inv_rows, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Grouped SwiGLU experts on the permuted rows (config paragraph of TensorFold
 * #1247: SwiGLU, no clamp).  For each row r of expert e (shared experts are
 * e = E..E+S-1):  h = silu(x[row_token[r]] Wg[e]^T) * (x[row_token[r]] Wu[e]^T),
 * y_perm[r] = h Wd[e]^T, fp32 accumulation, UNWEIGHTED.  With e4m3 experts the
 * activations (x and h) are first quantised per row per 128 along K to e4m3
 * with an fp32 scale amax/448.  x [T,H] act_dtype; y_perm [R,H] fp32.
 * Uses w->w_gate/up/down (+ scales, + shared arrays); the router fields are ignored.
 */
int moe_expert_ffn(const moe_config* cfg, const void* x, const int32_t* expert_offsets,
                   const int32_t* row_token, const moe_weights* w, float* y_perm,
                   void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * Weighted combine (the weighted layer of the HelloSun/ling30tiny numeric-check
 * summary; shared sum of the Inkling PR summary):
 *   y[t] = sum_{j=0..k-1} topk_w[t,j] * y_perm[inv_rows[t,j]]
 *        + sum_{s<S} y_perm[expert_offsets[E+s] + t],
 * summed in that fixed order in fp32, then stored as act_dtype.  y [T,H].
 */
int moe_combine(const moe_config* cfg, const float* y_perm, const int32_t* expert_offsets,
                const int32_t* inv_rows, const float* topk_w, void* y, hipStream_t stream);

/*
 * The whole layer: route, permute, experts, combine, all on the device, no host
 * sync.  Same semantics as the four calls above in sequence, within rounding:
 * it may fuse steps (routing weight applied in the down projection, expert
 * outputs kept in bf16 for bf16 layers).  y [T,H] act_dtype.  topk_ids_out
 * [T,k] int32 / topk_w_out [T,k] fp32 receive the routing if non-NULL.
 */
int moe_forward(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                int32_t* topk_ids_out, float* topk_w_out,
                void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_forward with kernel timing, for benchmarks: identical work and results;
 * the four caller-created events are attached to two kernel dispatches
 * themselves (hipExtLaunchKernel start/stop events, so no packet is added
 * between kernels): kernel_events[0], [1] start and stop of the gate/up expert
 * kernel (SwiGLU fused; for up to 16 tokens it also recomputes the routing),
 * [2], [3] start and stop of the down-projection kernel (fused with the
 * combine for up to 16 tokens).  hipEventElapsedTime(ev[0], ev[1]) is then
 * that kernel's duration.  MOE_ERR_ARG if any of the events is NULL.
 */
#define MOE_TIMED_EVENTS 4
int moe_forward_timed(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                      int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                      hipStream_t stream, hipEvent_t* kernel_events);

/*
 * One MoE block of a decoder layer with its neighbours fused: the pre-MoE RMSNorm
 * and the residual add.  The stack it belongs to is the one TensorFold issue #1247
 * "Ling-3.0-tiny on a Qualcomm board" describes in jschmied's config paragraph
 * (24 layers, a dense layer 0, so 23 MoE blocks per decode step); the pages give
 * no norm epsilon, 1e-6 is the usual choice.
 *   x_n   = round(x / sqrt(mean over H of x^2 + norm_eps) * norm_weight)
 *   x_out = round(x + y),  y = the MoE layer of moe_forward applied to x_n
 * round() is to act_dtype (bf16 round-to-nearest-even, or fp32); the mean, the
 * reciprocal square root and the sum are fp32.  norm_weight: [H] act_dtype, 16-byte
 * aligned.  x_out may be x itself (the residual stream updated in place) but must
 * not overlap it otherwise.  Decode batches (T <= 16) compute the norm inside the
 * router-logits kernel and add the residual in the down/combine kernel; larger
 * batches add one norm kernel and add the residual in the combine.  Other
 * arguments, the workspace and the errors are those of moe_forward; MOE_ERR_ARG
 * also for a null norm_weight or a negative or NaN norm_eps.
 */
int moe_forward_residual(const moe_config* cfg, const void* x, const void* norm_weight,
                         float norm_eps, const moe_weights* w, void* x_out, int32_t* topk_ids_out,
                         float* topk_w_out, void* ws, size_t ws_bytes, hipStream_t stream);

/*
 * moe_forward for callers that cannot allocate device memory or pass a workspace:
 * code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * Same arguments, work and results as moe_forward (bit for bit), but the scratch is a
 * fixed array of MOE_NOALLOC_SCRATCH_BYTES inside the library's device code, one copy
 * per GPU, held from the first call on that GPU until the process ends; no call
 * allocates or frees anything.  Enough for decode and small batches (moe_workspace_size
 * <= 16 MiB: up to ~256 tokens of the Ling-shaped layer); larger configs return
 * MOE_ERR_SCRATCH before enqueuing anything.  Every call on one GPU shares that GPU's
 * array: calls whose work overlaps on the device (other host threads, or other streams
 * not ordered with this one) RACE and must not be issued; calls on one stream, or on
 * streams ordered by events, are safe.  Nothing in the array needs to start at zero
 * (moe_forward ignores its workspace's contents on entry).  The first call on a device
 * looks the array's device address up (hipGetSymbolAddress) with that device current.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (16u << 20)
int moe_forward_noalloc(const moe_config* cfg, const void* x, const moe_weights* w, void* y,
                        int32_t* topk_ids_out, float* topk_w_out, hipStream_t stream);

/*
 * Expert paging: the routed experts of a layer live in host memory and an HBM arena of
 * N slots holds the ones recent calls routed to (the HelloSun/ling30tiny model card:
 * introduction, where inactive experts stay off the compute device and a bounded
 * arena holds the selected ones; its RAM-limit table reports the arena in slots and a
 * hot rate).  Every decision is taken on the device after the routing, so no call
 * waits for the host.  Policy: per call the distinct routed experts are looked up; a
 * resident one is a hit; misses are copied from the store into the slots this call
 * does not need, least recently used first (a slot's stamp is the number of the last
 * call that used it; never-used slots first), ties to the lower slot, misses taken in
 * ascending expert order.  Shared experts are not paged (every token uses them).
 * Supported: fp32 and bf16 experts; k <= N <= E and N >= min(E, T*k) (every expert one
 * call needs fits), else MOE_ERR_UNSUPPORTED.
 *
 * State: device memory of moe_pager_state_layout() bytes, owned by the caller, one per
 * (layer, arena); moe_pager_reset() initialises it (a kernel on `stream`: empty arena,
 * zero counters).  Layout, at the offsets the layout call writes (offsets[0..3]):
 *   int64 counters[8]: [0] calls, [1] routed (token, slot) references, [2] lookups
 *     (distinct experts needed, summed over calls), [3] hits, [4] misses, [5] bytes
 *     copied from the store; hot rate = hits / lookups;
 *   int32 key_slot[E] (slot of each expert or -1), int32 slot_key[N] (expert in each
 *   slot or -1), int64 stamp[N].
 * Calls that share a state must be ordered on the device (one stream).
 */
int moe_pager_state_layout(const moe_config* cfg, int32_t num_slots, size_t* offsets,
                           size_t* bytes);
int moe_pager_reset(const moe_config* cfg, int32_t num_slots, void* state, hipStream_t stream);
/* Workspace bytes of moe_forward_paged for `cfg` and `num_slots` (host only). */
int moe_paged_workspace_size(const moe_config* cfg, int32_t num_slots, size_t* bytes);
/*
 * moe_forward with the routed experts paged.  host_experts: w_gate, w_up [E, I, H] and
 * w_down [E, H, I] in pinned host memory (hipHostMalloc or a pinned torch tensor; device
 * memory is accepted too), read by the GPU over the host link; its other fields are
 * ignored.  resident: device memory - w_router, router_bias, the arena's w_gate, w_up
 * [N, I, H] and w_down [N, H, I], and the shared experts sh_* (S > 0).  The call routes
 * (moe_route's semantics), updates the arena on the device (k_pager_plan, then the copy
 * of the misses), then runs the permutation, experts and combine of moe_permute /
 * moe_expert_ffn / moe_combine over the slots: y equals, bit for bit, that sequence of
 * calls on the resident layer.  Errors as moe_forward; MOE_ERR_ARG also when HIP does
 * not know a store pointer (not pinned).
 */
int moe_forward_paged(const moe_config* cfg, const void* x, const moe_weights* host_experts,
                      const moe_weights* resident, int32_t num_slots, void* state, void* y,
                      int32_t* topk_ids_out, float* topk_w_out, void* ws, size_t ws_bytes,
                      hipStream_t stream);

/*
 * Where a call leaves inspectable intermediate results in the workspace, for tests
 * and debugging (host only, no device work).  After moe_forward / moe_forward_timed /
 * moe_forward_residual (and moe_route with logits == NULL) the workspace holds:
 *   MOE_WS_LOGITS      [T,E] fp32 router logits the routing was decided on (bias included);
 *   MOE_WS_ACT_CODES   [T,H] uint8 e4m3 codes of x (block-FP8 and MXFP4 experts only,
 *                      else 0 bytes);
 *   MOE_WS_ACT_SCALES  their scales: [T,H/128] fp32 (block-FP8), [T,H/32] uint8 E8M0 (MXFP4);
 *   MOE_WS_NORM_ROWS   [T,H] act_dtype normalised rows (moe_forward_residual only).
 * The contents stay valid until the next call that uses the same workspace.  Writes the
 * byte offset from the workspace start and the slot's size; MOE_ERR_ARG for an unknown
 * slot or a null output pointer, or a validation error of the config.
 */
#define MOE_WS_LOGITS      0
#define MOE_WS_ACT_CODES   1
#define MOE_WS_ACT_SCALES  2
#define MOE_WS_NORM_ROWS   3
int moe_workspace_slot(const moe_config* cfg, int slot, size_t* offset, size_t* bytes);

/* Static description of a status code (for MOE_ERR_HIP: the last HIP error text
   seen by this thread).  Never NULL. */
const char* moe_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
