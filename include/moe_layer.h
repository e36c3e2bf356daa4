/*
 * moe_layer.h -- C ABI of the MI355X (gfx950) sparse mixture-of-experts FFN layer.
 *
 * The layer (sources: the five pages about Step-3.5-Flash):
 *   - a router over E experts (llm-atlas "Step-3.5-Flash", table "Champs bruts du
 *     config.json": moe_num_experts 288, need_fp32_gate, use_moe_router_bias,
 *     moe_router_activation, moe_router_scaling_factor);
 *   - top-k selection with renormalised weights (moe_top_k 8, norm_expert_weight);
 *   - SiLU-gated expert FFNs of width I (moe_intermediate_size 1280) and an
 *     always-on shared expert of width Is (share_expert_dim 1280);
 *   - hidden size H (hidden_size 4096), bf16 weights (torch_dtype bfloat16);
 *   - INT4 weight-only storage, group 32, for decode (nipponese.news article,
 *     local-deployment paragraph: INT4-quantised weights for llama.cpp).
 *
 * y[t] = shared(x[t]) + sum_j w[t,j] * expert_{idx[t,j]}(x[t]),
 *   expert(x) = W_down (silu(W_gate x) * (W_up x)),  silu(z) = z / (1 + exp(-z))
 *   (the two projections optionally clamped first: see the SwiGLU limits).
 * Router: l = x W_r^T (+ b), accumulated in fp32.  Experts are ranked by
 * descending l (ties: lower expert index).  softmax scoring:
 * p = softmax over all E; sigmoid scoring: p = 1/(1+exp(-l)).  With renormalize,
 * w_j = p_j / sum over the k selected; then w *= routed_scale.
 *
 * Conventions for every entry point:
 *   - All tensors are row-major; the last dimension is contiguous ("[N][K]" means
 *     N rows of K elements, the nn.Linear [out][in] order).
 *   - Device pointers must be 16-byte aligned.  The caller owns every device
 *     buffer (activations, router weights, packed weights, output, workspace);
 *     the library allocates no device memory, apart from the static scratch
 *     array of moe_layer_forward_noalloc (one per GPU, below).  A handle owns
 *     host state (and for some configurations one HIP stream, below).
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the default stream),
 *     which must belong to the handle's device (the call makes that device
 *     current while it enqueues and restores the caller's afterwards).
 *     Nothing synchronises the host, and a forward enqueues kernels only (no
 *     memset or copy nodes; with the second stream below, also the event
 *     records and waits that fork and join it), so it can be captured in a HIP
 *     graph.
 *   - Argument errors are detected before anything is enqueued and returned as
 *     a status; moe_last_error() then holds a message (per thread).  Launch
 *     failures return MOE_ERR_DEVICE.  Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - A handle is immutable after moe_layer_create: concurrent forwards on one
 *     handle are allowed when each uses its own workspace and output.
 *   - A handle whose configuration has bf16 weights and activations and
 *     max_tokens >= 256 owns a second stream (default priority, non-blocking)
 *     and two events that fork it from and join it to the caller's stream,
 *     all created with the handle and destroyed by moe_layer_destroy.
 *     Batches of 256 to 1024 tokens that take the streaming GEMMs put the hot
 *     experts' LDS-tiled GEMMs there (few, long-running workgroups; a
 *     load-imbalanced batch has them): forked from `stream` by an event after
 *     the dispatch and joined back before the combine, so they overlap the
 *     streaming GEMMs on `stream`.  The output is the same as with everything
 *     in order.
 *     Concurrent forwards on one handle share that stream (and serialise
 *     there); while a forward on a handle is being captured into a graph, the
 *     second stream is part of the capture, so no other forward on that handle
 *     may run until the capture ends.
 */
#ifndef MOE_LAYER_H
#define MOE_LAYER_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 3
#define MOE_PACK_VERSION 1

typedef struct moe_layer* moe_layer_t;

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = 1,        /* a required pointer is NULL */
  MOE_ERR_SHAPE = 2,       /* a size is out of range or not a supported multiple */
  MOE_ERR_DTYPE = 3,       /* unsupported dtype / scoring / mode value */
  MOE_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned */
  MOE_ERR_WORKSPACE = 5,   /* workspace smaller than moe_layer_workspace_bytes() */
  MOE_ERR_UNSUPPORTED = 6, /* a valid request the library does not implement */
  MOE_ERR_DEVICE = 7       /* no usable gfx950 device, or a HIP call failed */
} moe_status_t;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_INT4_G32 = 2 } moe_dtype_t;
typedef enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1 } moe_score_t;
/* Where the router bias enters: the logits used for both selection and weights
 * (MOE_BIAS_LOGIT), or the selection scores only (MOE_BIAS_SELECT). */
typedef enum { MOE_BIAS_LOGIT = 0, MOE_BIAS_SELECT = 1 } moe_bias_mode_t;

/* Layer shape and numerics.  Limits: 1 <= top_k <= min(num_experts, 16),
 * num_experts <= 512, hidden % 64 == 0, inter % 32 == 0, shared_inter % 32 == 0
 * (0 = no shared expert), max_tokens >= 1.  INT4 weights additionally need
 * hidden, inter and shared_inter to be multiples of 128.
 * SwiGLU limits (llm-atlas "Step-3.5-Flash", config fields swiglu_limits and
 * swiglu_limits_shared: 0 on all layers but the last ones, where the routed
 * experts take 7 and the shared expert 16): a limit L > 0 replaces the gate
 * projection g by min(g, L) and the up projection u by min(max(u, -L), L)
 * before silu(g) * u.  The pages give only the values; this clamp is the
 * reading taken.  Each limit must be finite and >= 0 (MOE_ERR_SHAPE). */
typedef struct {
  int32_t hidden;        /* H (hidden_size) */
  int32_t num_experts;   /* E (moe_num_experts) */
  int32_t top_k;         /* k (moe_top_k) */
  int32_t inter;         /* I (moe_intermediate_size) */
  int32_t shared_inter;  /* Is (share_expert_dim); 0 = no shared expert */
  int32_t max_tokens;    /* largest T a forward will be called with */
  int32_t score;         /* moe_score_t */
  int32_t renormalize;   /* nonzero: w_j = p_j / sum_sel p (norm_expert_weight) */
  float routed_scale;    /* multiplies the weights after renormalisation (1 = none) */
  int32_t bias_mode;     /* moe_bias_mode_t; used only when a router bias is passed */
  int32_t act_dtype;     /* MOE_BF16 or MOE_F32: dtype of x and of the output */
  int32_t weight_dtype;  /* MOE_BF16 or MOE_INT4_G32: routed and shared expert weights */
  float swiglu_limit;        /* routed experts' SwiGLU limit L (0 = none), see below */
  float swiglu_limit_shared; /* the shared expert's SwiGLU limit (0 = none) */
} moe_layer_config_t;

/* Canonical (unpacked) expert weights, device pointers, read by
 * moe_layer_pack_weights only.
 *   MOE_BF16:     w_gate, w_up [E][I][H]; w_down [E][H][I];
 *                 s_gate, s_up [Is][H];   s_down [H][Is]       (bf16)
 *   MOE_INT4_G32: same element order, one signed 4-bit value q in [-8, 7] per
 *                 weight stored as u = q + 8, element k of a row in byte k/2,
 *                 low nibble for even k (rows of K/2 bytes); plus fp16 scales
 *                 sc_* with shape [..][N][K/32]: weight = scale[n][k/32] * q.
 * The sc_* pointers are ignored for bf16; the s_* and sc_s_* pointers are
 * ignored when shared_inter == 0. */
typedef struct {
  const void *w_gate, *w_up, *w_down;
  const void *s_gate, *s_up, *s_down;
  const void *sc_gate, *sc_up, *sc_down;
  const void *sc_s_gate, *sc_s_up, *sc_s_down;
} moe_weights_t;

/* Routing views returned by moe_layer_forward: device pointers into the
 * caller's workspace, valid until the workspace is reused.  Pair p = t*k + j is
 * token t's j-th choice (j in descending order of selection score; equal
 * scores in ascending expert order).
 *   topk_idx [T][k] int32, topk_w [T][k] fp32, topk_gap [T] fp32 (k-th minus
 *   (k+1)-th selection score; +inf when k == E);
 *   expert_counts [E] int32; expert_offsets [E+1] int32 (exclusive prefix sum,
 *   expert_offsets[E] = T*k);
 *   perm [T*k] int32: pair id stored at each permuted row (rows grouped by
 *   expert, ascending token inside a group); inv [T*k] int32: row of each pair. */
typedef struct {
  int32_t* topk_idx;
  float* topk_w;
  float* topk_gap;
  int32_t* expert_counts;
  int32_t* expert_offsets;
  int32_t* perm;
  int32_t* inv;
  /* Libraries built with index checks (moe_debug_checks() == 1): two int32,
   * both 0 unless a kernel of this forward read an out-of-range index (an
   * expert id in the dispatch, a token id in a GEMM's row gather, a permuted
   * row in the combine, a tile-list entry); then [0] is its kind (1 expert,
   * 2 token, 3 row, 4 tile entry) and [1] the first offending value, and the
   * kernel went on with the index clamped or the tile skipped.  NULL in
   * release builds. */
  int32_t* debug_flag;
} moe_route_t;

/* Version of this header's ABI (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* 1 if this library was built with index checks (build option --debug:
 * moe_route_t.debug_flag), else 0. */
int moe_debug_checks(void);

/* Validates *cfg, checks that `device` is a gfx950 GPU and returns a handle.
 * Errors: MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_DTYPE, MOE_ERR_DEVICE. */
moe_status_t moe_layer_create(const moe_layer_config_t* cfg, int device, moe_layer_t* out);

/* Releases the handle: its host memory and, if it owns them, its second
 * stream (after that stream's pending work) and the two events that fork and
 * join it.  NULL is ignored. */
void moe_layer_destroy(moe_layer_t layer);

/* Bytes of the packed weight buffer (routed experts followed by the shared
 * expert) for this handle's shape and weight dtype; format MOE_PACK_VERSION. */
size_t moe_layer_packed_bytes(moe_layer_t layer);

/* Bytes of device workspace one forward over num_tokens tokens needs
 * (0 < num_tokens <= max_tokens; returns 0 otherwise). */
size_t moe_layer_workspace_bytes(moe_layer_t layer, int32_t num_tokens);

/* Rewrites the canonical weights into the packed layout the kernels stream
 * (16x32 MFMA fragments in lane order; gate and up interleaved per 16 rows;
 * INT4 nibbles reordered for in-register widening).  `packed` is a device
 * buffer of moe_layer_packed_bytes() bytes.  Enqueued on `stream`. */
moe_status_t moe_layer_pack_weights(moe_layer_t layer, const moe_weights_t* canonical,
                                    void* packed, hipStream_t stream);

/* One layer call over num_tokens tokens (T):
 *   x          [T][H]  act_dtype (bf16 or fp32)
 *   router_w   [E][H]  bf16
 *   router_bias [E]    fp32, or NULL for no bias
 *   packed     the buffer filled by moe_layer_pack_weights
 *   out        [T][H]  act_dtype; may not alias x
 *   workspace  device scratch of at least moe_layer_workspace_bytes(layer, T)
 *   route      NULL, or receives device views of the routing results.
 * T == 0 is a no-op returning MOE_OK.  Errors: MOE_ERR_NULL, MOE_ERR_SHAPE
 * (T > max_tokens or T < 0), MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_DEVICE. */
moe_status_t moe_layer_forward(moe_layer_t layer, int32_t num_tokens, const void* x,
                               const void* router_w, const float* router_bias,
                               const void* packed, void* out, void* workspace,
                               size_t workspace_bytes, moe_route_t* route, hipStream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * moe_layer_forward without a workspace argument.  Its scratch is one static
 * device array of MOE_NOALLOC_SCRATCH_BYTES inside the library, one copy per
 * GPU, taken when the first handle on that GPU is created and held until the
 * process ends; the call itself allocates nothing and runs the same kernels
 * as moe_layer_forward (same results bit for bit).
 *   - num_tokens must need at most MOE_NOALLOC_SCRATCH_BYTES of workspace
 *     (moe_layer_workspace_bytes); a larger batch returns MOE_ERR_WORKSPACE
 *     before anything is enqueued.  64 MiB holds a 256-token batch of the
 *     Step-3.5-Flash layer (H 4096, 288 experts, top-8, widths 1280).
 *   - Every call on one GPU shares that GPU's array: calls whose work
 *     overlaps on the device (other streams, other handles, other threads)
 *     race and give undefined results.  Serialise them (one stream, or events).
 *   - route views point into that array and stay valid until the next call
 *     on the same GPU.  Nothing in it needs to be zero at the start of a call
 *     (the one counter the kernels use is cleared by a kernel of the call).
 *   - Errors: those of moe_layer_forward, MOE_ERR_WORKSPACE as above, and
 *     MOE_ERR_DEVICE if the array's device address could not be taken. */
#define MOE_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
moe_status_t moe_layer_forward_noalloc(moe_layer_t layer, int32_t num_tokens, const void* x,
                                       const void* router_w, const float* router_bias,
                                       const void* packed, void* out, moe_route_t* route,
                                       hipStream_t stream);

/* Number of events moe_layer_forward_timed records. */
#define MOE_STAGE_EVENTS 6

/* moe_layer_forward, and on `stream` also records stage_events[0] before the
 * router and stage_events[1..5] after the router, dispatch, gate/up GEMM,
 * down GEMM and combine stages, so that
 * hipEventElapsedTime(stage_events[i], stage_events[i+1]) is the duration of
 * stage i.  Top-k selection runs in one launch with the dispatch for batches
 * of up to 1024 tokens (it is then timed in the dispatch stage) and with the
 * router logits above that.  Work on the handle's second stream is timed only
 * where `stream` waits for it, before the combine stage.  stage_events holds
 * MOE_STAGE_EVENTS events created by the caller
 * (hipEventCreate or hipEventCreateWithFlags; events made with
 * hipEventDisableSystemFence only time the stages and skip the cache write-back
 * a default event's record performs, about 2 us each on a decode batch); a
 * NULL entry leaves that boundary unrecorded (to time one stage, pass its two
 * events only).  The same errors as moe_layer_forward, plus MOE_ERR_NULL for
 * a NULL array. */
moe_status_t moe_layer_forward_timed(moe_layer_t layer, int32_t num_tokens, const void* x,
                                     const void* router_w, const float* router_bias,
                                     const void* packed, void* out, void* workspace,
                                     size_t workspace_bytes, moe_route_t* route,
                                     hipStream_t stream, hipEvent_t* stage_events);

/* Short constant name of a status code. */
const char* moe_status_str(moe_status_t status);

/* Message of the last error returned on the calling thread ("" if none). */
const char* moe_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* MOE_LAYER_H */
