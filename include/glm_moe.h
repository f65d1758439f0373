/*
 * glm_moe.h - C ABI of the GLM-5.2 mixture-of-experts feed-forward layer on
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (frontier-model-atlas "GLM-5.2 model anatomy", Feed-forward /
 * Mixture of Experts panel): a sigmoid router scores E routed experts; an
 * expert-score correction bias takes part in the top-k selection only; the
 * selected un-biased scores are renormalised and then scaled (2.5 for
 * GLM-5.2); the token's expert outputs are summed with those weights and with
 * one always-on shared expert.  Expert MLPs are SiLU-gated with the w1 (gate),
 * w3 (up) and w2 (down) roles named on the PocketLLM "GLM-5.2" page
 * (Implemented execution path).  GLM-5.2 sizes: hidden 6144, 256 routed
 * experts, top-8, expert width 2048, one shared expert (PocketLLM "GLM-5.2",
 * Model specification table).
 *
 * Conventions shared by every entry point:
 *   - Every tensor pointer is a DEVICE pointer on the current HIP device,
 *     allocated and owned by the caller; the library never allocates, frees
 *     or retains device memory in route/forward.  All tensors are row-major
 *     and contiguous, 16-byte aligned.
 *   - Work is enqueued on `stream` and the call returns without
 *     synchronising.  Errors in arguments are detected synchronously, before
 *     anything is enqueued; kernel faults surface at the caller's next
 *     synchronisation.
 *   - No exceptions cross the ABI.  On failure the function returns a
 *     negative glm_moe_status and glm_moe_last_error() describes the cause.
 *   - Calls sharing one workspace must be ordered on one stream; calls with
 *     distinct workspaces are independent.
 *   - Results are deterministic: the same inputs give bit-identical outputs
 *     (no floating-point atomics anywhere).
 */
#ifndef GLM_MOE_H
#define GLM_MOE_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#if defined(__GNUC__)
#define GLM_MOE_API __attribute__((visibility("default")))
#else
#define GLM_MOE_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GLM_MOE_OK = 0,
  GLM_MOE_EINVAL = -1,        /* bad argument: null pointer, bad size, misalignment */
  GLM_MOE_EUNSUPPORTED = -2,  /* valid but not implemented: E > 256, dtype mix, D or F not /64 */
  GLM_MOE_EWORKSPACE = -3,    /* workspace_bytes smaller than glm_moe_workspace_size() */
  GLM_MOE_EHIP = -4           /* a HIP runtime call or kernel launch failed */
} glm_moe_status;

typedef enum {
  GLM_MOE_F32 = 0,
  GLM_MOE_BF16 = 1,
  GLM_MOE_MXFP8 = 2  /* weights only: OCP MX FP8, see glm_moe_forward_mx */
} glm_moe_dtype;

/* Layer sizes.  T tokens, hidden D, E routed experts, routed expert width F,
 * shared expert width F_shared.  act_dtype is the dtype of x; weight_dtype is
 * the dtype of w1/w3/w2 and the shared expert.  Supported pairs: F32/F32 and
 * BF16/BF16 (glm_moe_forward*), BF16/MXFP8 (glm_moe_forward_mx).  router_w,
 * corr_bias, out and topk_w are always fp32. */
typedef struct {
  int32_t T, D, E, F, F_shared;
  int32_t act_dtype;
  int32_t weight_dtype;
} glm_moe_dims;

/* Workspace bytes needed by glm_moe_route / glm_moe_forward for `d` and
 * `top_k` (written to *bytes).  Host-only; enqueues nothing.
 * Returns GLM_MOE_OK, or EINVAL / EUNSUPPORTED for dims that route/forward
 * would reject.  T = 0 yields 0 bytes. */
GLM_MOE_API int glm_moe_workspace_size(const glm_moe_dims* d, int top_k, size_t* bytes);

/* The same size as a return value, the form of the boundary's plain
 * statement: bytes of workspace glm_moe_route / glm_moe_forward need for `d`
 * and `top_k`.  Host-only; enqueues nothing.  Returns 0 when T = 0 (no
 * workspace needed; glm_moe_last_error() is then empty) and 0 for dims that
 * route/forward would reject (glm_moe_last_error() names the cause; use
 * glm_moe_workspace_size for the status code).  Any valid call with T > 0
 * needs a non-zero workspace. */
GLM_MOE_API size_t glm_moe_workspace_bytes(const glm_moe_dims* d, int top_k);

/* Router only: steps "sigmoid router scores", "correction bias affects top-k
 * selection", "un-biased selected scores renormalised and scaled" of the layer
 * statement (GLM-5.2 anatomy page, Mixture of Experts panel).
 *   x          [T][D]   act_dtype     layer input (the normalised FFN input)
 *   router_w   [E][D]   fp32
 *   corr_bias  [E]      fp32          added to sigmoid scores for selection only
 *   top_k      1 <= top_k <= min(E, 32)
 *   scale      routed scaling factor (2.5 for GLM-5.2); any finite value
 *   topk_idx   [T][top_k] int32  out: selected experts, slots in descending
 *              biased score, equal scores ordered by lower expert index
 *   topk_w     [T][top_k] fp32   out: scale * sigma_j / sum of selected sigma
 *   workspace  device buffer of at least glm_moe_workspace_size() bytes,
 *              256-byte aligned; contents on entry are ignored.
 * Logits are fp32 (bf16 x is used exactly; products are exact and summed in
 * fp32).  T = 0 is a successful no-op. */
GLM_MOE_API int glm_moe_route(const glm_moe_dims* d, const void* x, const float* router_w,
                  const float* corr_bias, int top_k, float scale,
                  int32_t* topk_idx, float* topk_w,
                  void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The whole layer: routing as glm_moe_route, then every (token, slot)
 * assignment runs through its expert (dropless), and
 *   out[t] = sum_j topk_w[t][j] * MLP_{idx[t][j]}(x[t]) + MLP_shared(x[t]),
 *   MLP(v) = w2 (SiLU(w1 v) * (w3 v)).
 *   w1, w3     [E][F][D]        weight_dtype  (gate, up)
 *   w2         [E][D][F]        weight_dtype  (down)
 *   shared_w1, shared_w3  [F_shared][D]; shared_w2 [D][F_shared]
 *   out        [T][D] fp32, overwritten (the residual add is not included)
 *   topk_idx_out, topk_w_out   nullable; if given, receive the routing
 * The bf16 path computes expert products on bf16 MFMA with fp32 accumulation
 * and rounds the gated hidden activations to bf16; per-slot expert outputs
 * and the final sum are fp32: the shared expert's output, then the weighted
 * slot outputs added in slot order.
 * The fp32 path keeps every intermediate in fp32.  T = 0 is a no-op. */
GLM_MOE_API int glm_moe_forward(const glm_moe_dims* d, const void* x, const float* router_w,
                    const float* corr_bias,
                    const void* w1, const void* w3, const void* w2,
                    const void* shared_w1, const void* shared_w3, const void* shared_w2,
                    int top_k, float scale, float* out,
                    int32_t* topk_idx_out, float* topk_w_out,
                    void* workspace, size_t workspace_bytes, hipStream_t stream);

/* glm_moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments and results as glm_moe_forward without the workspace: the
 * call works in a fixed 64 MiB buffer that the library holds on each GPU it
 * runs on until the process ends (its address is looked up once per device,
 * with that device current).  The call itself allocates and frees nothing.
 * Sizes whose workspace (glm_moe_workspace_bytes) exceeds 64 MiB are rejected
 * with GLM_MOE_EWORKSPACE before anything is enqueued; at the GLM-5.2 shape
 * (hidden 6144, 256 experts, top-8, width 2048) that admits batches of up to
 * 235 tokens, e.g. decode steps.  Every call on one GPU uses that GPU's
 * buffer: calls that overlap on one GPU (on different streams or host
 * threads) race and give undefined results; calls ordered on one stream are
 * safe.  Options (groups, norm, residual) and traces are not available here. */
GLM_MOE_API int glm_moe_forward_noalloc(const glm_moe_dims* d, const void* x,
                                        const float* router_w, const float* corr_bias,
                                        const void* w1, const void* w3, const void* w2,
                                        const void* shared_w1, const void* shared_w3,
                                        const void* shared_w2, int top_k, float scale, float* out,
                                        int32_t* topk_idx_out, float* topk_w_out,
                                        hipStream_t stream);

/* Stages of one forward call, in launch order (used by the stage trace). */
enum {
  GLM_MOE_STAGE_NORM = 0,          /* pre-norm RMSNorm (empty unless requested) */
  GLM_MOE_STAGE_ROUTER_LOGITS = 1,
  GLM_MOE_STAGE_ROUTER_TOPK = 2,
  GLM_MOE_STAGE_SCAN = 3,
  GLM_MOE_STAGE_SCATTER = 4,
  GLM_MOE_STAGE_GATE_UP = 5,
  GLM_MOE_STAGE_DOWN = 6,
  GLM_MOE_STAGE_SHARED_COMBINE = 7, /* combine (+ residual add) */
  GLM_MOE_NUM_STAGES = 8
};

/* Optional per-stage timing with HIP events recorded on the call's stream.
 * A trace owns host-side event objects (created here, released by destroy);
 * it records up to `max_calls` forward calls, then ignores further ones until
 * reset.  Not thread-safe; one trace per stream. */
typedef struct glm_moe_trace glm_moe_trace;
GLM_MOE_API int glm_moe_trace_create(glm_moe_trace** trace, int max_calls);
GLM_MOE_API int glm_moe_trace_destroy(glm_moe_trace* trace);
GLM_MOE_API int glm_moe_trace_reset(glm_moe_trace* trace);
/* Waits for the recorded events, then writes the per-stage time summed over
 * the recorded calls (milliseconds, GLM_MOE_NUM_STAGES floats) and the number
 * of calls recorded. */
GLM_MOE_API int glm_moe_trace_read(glm_moe_trace* trace, float* stage_ms, int* calls);

/* glm_moe_forward that also records per-stage events into `trace` (nullable:
 * then identical to glm_moe_forward). */
GLM_MOE_API int glm_moe_forward_traced(const glm_moe_dims* d, const void* x, const float* router_w,
                           const float* corr_bias,
                           const void* w1, const void* w3, const void* w2,
                           const void* shared_w1, const void* shared_w3,
                           const void* shared_w2,
                           int top_k, float scale, float* out,
                           int32_t* topk_idx_out, float* topk_w_out,
                           void* workspace, size_t workspace_bytes, hipStream_t stream,
                           glm_moe_trace* trace);

/* Options around the layer (all optional; a null options pointer, or a
 * zeroed struct, gives the plain GLM-5.2 layer above).
 *   n_group, topk_group, group_topk: group-limited routing as GLM-4.5 uses
 *     it ("Full Forward" GLM-4.5 note, How it works: sigmoid group routing).
 *     The E experts form n_group consecutive groups (E % n_group == 0); a
 *     group's score is the sum of its group_topk largest biased scores; each
 *     token keeps its topk_group best groups (equal scores: lower group) and
 *     picks its top_k experts inside them.  n_group 0 or 1 disables grouping;
 *     group_topk 0 means min(2, E / n_group).  Requires topk_group * E / n_group >= top_k and
 *     n_group <= 64.
 *   norm_weight, norm_eps: when norm_weight ([D] fp32) is given, x is the
 *     pre-norm residual stream h of the block and the layer runs on
 *     RMSNorm(h) = h / sqrt(mean(h^2) + eps) * norm_weight, computed in fp32
 *     and held in act_dtype (the pre-norm block of the "Full Forward" note).
 *   add_residual: nonzero adds x (the residual stream) to the output:
 *     out = x + layer(...), the block's residual add, done in fp32 after the
 *     shared and routed terms. */
typedef struct {
  int32_t n_group;
  int32_t topk_group;
  int32_t group_topk;
  const float* norm_weight;
  float norm_eps;
  int32_t add_residual;
} glm_moe_options;

/* glm_moe_workspace_size / glm_moe_route / glm_moe_forward_traced with
 * options (`opts` nullable).  Same conventions and error codes; invalid
 * options return GLM_MOE_EINVAL (or EUNSUPPORTED for n_group > 64). */
GLM_MOE_API int glm_moe_workspace_size_ex(const glm_moe_dims* d, const glm_moe_options* opts,
                                          int top_k, size_t* bytes);
GLM_MOE_API int glm_moe_route_ex(const glm_moe_dims* d, const glm_moe_options* opts,
                                 const void* x, const float* router_w, const float* corr_bias,
                                 int top_k, float scale, int32_t* topk_idx, float* topk_w,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);
GLM_MOE_API int glm_moe_forward_ex(const glm_moe_dims* d, const glm_moe_options* opts,
                                   const void* x, const float* router_w, const float* corr_bias,
                                   const void* w1, const void* w3, const void* w2,
                                   const void* shared_w1, const void* shared_w3,
                                   const void* shared_w2, int top_k, float scale, float* out,
                                   int32_t* topk_idx_out, float* topk_w_out, void* workspace,
                                   size_t workspace_bytes, hipStream_t stream,
                                   glm_moe_trace* trace);

/* A dense SiLU-gated feed-forward layer, out = w2 (SiLU(w1 x) * (w3 x)): the
 * leading dense layers of the model (GLM-5.2 anatomy page, Token path: 3
 * dense FFN blocks before the MoE blocks), run on the same grouped kernels as
 * one group.  Uses d->T, d->D, d->F_shared (the dense width) and the dtypes;
 * E and F are ignored.  w1, w3 [F_shared][D]; w2 [D][F_shared]; out [T][D]
 * fp32.  opts may give norm_weight / norm_eps / add_residual (grouping
 * fields are ignored).  Workspace from glm_moe_dense_workspace_size.
 * `trace` (nullable) records the stages as for glm_moe_forward_traced; the
 * router and scatter stages are empty. */
GLM_MOE_API int glm_moe_dense_workspace_size(const glm_moe_dims* d, const glm_moe_options* opts,
                                             size_t* bytes);
GLM_MOE_API int glm_moe_dense_ffn(const glm_moe_dims* d, const glm_moe_options* opts,
                                  const void* x, const void* w1, const void* w3, const void* w2,
                                  float* out, void* workspace, size_t workspace_bytes,
                                  hipStream_t stream, glm_moe_trace* trace);

/* MXFP8 expert weights (OCP Microscaling v1.0 MXFP8): each tensor is E4M3
 * codes (1 byte; bias 7, max 448, no infinities) in the bf16 layout above, plus
 * one E8M0 scale byte (value 2^(s - 127)) per 32 consecutive elements along
 * its rows (the contraction dimension).
 *
 * Scale layout ("K-step-major"): for a matrix of N rows and contraction K,
 * the four scales of row n covering elements [128 kt, 128 kt + 128) form the
 * dword at byte (kt * N + n) * 4, i.e. the array is [K/128][N][4] rather than
 * the row-major [N][K/32]; glm_moe_mx_pack_scales converts.  Per tensor:
 *   w1, w3 [E][F][D] codes, w1_scale, w3_scale [E][D/128][F][4];
 *   w2 [E][D][F] codes, w2_scale [E][F/128][D][4];
 *   shared_w1, shared_w3 [F_shared][D], scales [D/128][F_shared][4];
 *   shared_w2 [D][F_shared], scale [F_shared/128][D][4].
 * The pages name BF16/FP8 GLM-5.2 artifacts ("Inside GLM" course page,
 * Release anatomy lesson) without their scaling; this block format is the
 * one gfx950 applies inside its FP8 MFMA. */
typedef struct {
  const void* w1; const void* w1_scale;
  const void* w3; const void* w3_scale;
  const void* w2; const void* w2_scale;
  const void* shared_w1; const void* shared_w1_scale;
  const void* shared_w3; const void* shared_w3_scale;
  const void* shared_w2; const void* shared_w2_scale;
} glm_moe_mx_weights;

/* The layer with MXFP8 expert weights.  d->act_dtype must be GLM_MOE_BF16 and
 * d->weight_dtype GLM_MOE_MXFP8; D, F and F_shared must be multiples of 128
 * (else EUNSUPPORTED).  Routing is that of glm_moe_forward on the bf16 input.
 * The expert products take the input quantised to MXFP8 per token (blocks of
 * 32 along D) and the gated hidden values quantised per row (blocks of 32
 * along F): block scale = the smallest power of two keeping every element
 * within +-448, elements rounded to nearest E4M3, ties to even.  Accumulation
 * is fp32; the routed weights, shared expert and combine are as in
 * glm_moe_forward.  Workspace from glm_moe_workspace_size_ex with the same
 * dims.  Every pointer of `w` must be non-null and 16-byte aligned.  Other
 * arguments, options and errors as glm_moe_forward_ex. */
GLM_MOE_API int glm_moe_forward_mx(const glm_moe_dims* d, const glm_moe_options* opts,
                                   const void* x, const float* router_w, const float* corr_bias,
                                   const glm_moe_mx_weights* w, int top_k, float scale,
                                   float* out, int32_t* topk_idx_out, float* topk_w_out,
                                   void* workspace, size_t workspace_bytes, hipStream_t stream,
                                   glm_moe_trace* trace);

/* Where a forward call leaves the gated hidden rows in its workspace, for
 * inspection (a test can read back the hidden values the kernels computed
 * and quantised).  Byte offsets into the workspace of a call with the same
 * dims, options and top_k; valid after that call has completed, until the
 * workspace is reused.  bf16 layers hold bf16 hidden values, MXFP8 layers
 * E4M3 codes with E8M0 scales (fp32 layers keep fp32 values):
 *   row_assign   int32 [T*top_k]: expert-sorted row r holds assignment
 *                row_assign[r] = t*top_k + j (token t, slot j)
 *   hidden       [T*top_k][F]   rows in expert-sorted order
 *   hidden_scale [F/128][T*top_k][4]  (MXFP8 only; else 0)
 *   shared_hidden       [T][F_shared]
 *   shared_hidden_scale [F_shared/128][T][4]  (MXFP8 only; else 0)
 * Host-only; enqueues nothing.  Errors as glm_moe_workspace_size_ex. */
typedef struct {
  size_t row_assign, hidden, hidden_scale, shared_hidden, shared_hidden_scale;
} glm_moe_hidden_layout;
GLM_MOE_API int glm_moe_hidden_layout_of(const glm_moe_dims* d, const glm_moe_options* opts,
                                         int top_k, glm_moe_hidden_layout* layout);

/* Reorder MX scales from row-major [n_mats][N][K/32] (src) to the
 * K-step-major layout [n_mats][K/128][N][4] (dst) that glm_moe_forward_mx
 * reads; a pure byte permutation, run on `stream`.  Both are device
 * pointers, 16-byte aligned, of n_mats * N * K / 32 bytes each, and must not
 * overlap.  K must be a positive multiple of 128 and N positive (EINVAL
 * otherwise); n_mats == 0 does nothing.  For expert tensors pass n_mats = E. */
GLM_MOE_API int glm_moe_mx_pack_scales(const void* src, void* dst, int64_t n_mats, int N, int K,
                                       hipStream_t stream);

/* Static text for a status code. */
GLM_MOE_API const char* glm_moe_status_string(int status);

/* Description of the last failure on the calling thread ("" if none). */
GLM_MOE_API const char* glm_moe_last_error(void);

/* Library version, as major * 10000 + minor * 100 + patch. */
GLM_MOE_API int glm_moe_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GLM_MOE_H */
