/*
 * moe.h -- C ABI of the compressed-expert MoE FFN layer for AMD Instinct
 * MI355X (gfx950).
 *
 * The layer is the forward pass of one mixture-of-experts FFN whose E = G*K
 * experts are clustered into G groups of K.  Expert i of group g is stored as
 * a shared group base plus a rank-r residual,
 *
 *     W~_i = W_base^g + A_i B_i^T,   A_i in R^{d_in x r},  B_i in R^{d_out x r}
 *
 * ("Breaking the MoE LLM Trilemma: Dynamic Expert Clustering with Structured
 * Compression", papernotes.org note, key design 2), with the base in FP16
 * and the residual factors in FP16 or INT4 (key design 4).  A token is routed
 * in two levels, first to top_groups groups, then to top_experts experts
 * inside each chosen group (key design 3).  Flat top-k MoE is the case
 * G = E, K = 1, r = 0.  Row vectors throughout: y = x W.
 *
 * Per expert the FFN is SwiGLU, h = SiLU(x W~_gate) * (x W~_up), y = h W~_down,
 * or GELU (tanh form), y = GELU(x W~_1) W~_2, with no biases and no outer
 * activation (the FFN block of "混合专家模型的路由机制与工程落地",
 * jiusizaji.com, section 1.2).  The layer output is the gate-weighted sum
 * over the selected experts, y = sum_i G_i(x) E_i(x) (same page, same
 * section).
 *
 * Routing (key design 3; the per-expert additive routing bias of the same
 * MoE routing page, section 2.2; router in FP32 as in its section 3.1):
 *   group logit  s_g = x . W_grp[:, g] + group_bias[g]        (FP32)
 *   expert logit e_j = x . W_exp[g][:, j] + expert_bias[g*K+j] (FP32)
 *   keep the top_groups largest s, then inside each chosen group the
 *   top_experts largest e; order: descending score, ties to the lower index.
 *   gate weight of (g, j) = softmax over the chosen s (at g) times softmax
 *   over the chosen e of g (at j).  With K = 1 the in-group weight is 1.
 *
 * All functions return MOE_OK (0) or an error code; on error
 * moe_last_error() (thread-local) describes it.  No exception crosses this
 * boundary.  Functions that take a stream enqueue work on it (a hipStream_t
 * passed as void*, NULL = the null stream) and return without waiting;
 * kernel faults surface at the caller's next synchronisation.
 */
#ifndef CEFN_MOE_H
#define CEFN_MOE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = 1, /* null pointer, bad size, T > T_max, ... */
  MOE_ERR_UNSUPPORTED = 2, /* valid but not built: dtype mix, limits below */
  MOE_ERR_OOM = 3,         /* device allocation failed */
  MOE_ERR_HIP = 4          /* a HIP runtime call failed */
};

typedef enum { MOE_F32 = 0, MOE_F16 = 1, MOE_BF16 = 2 } moe_dtype;

/* Residual factor storage.  INT4_G32: symmetric 4-bit codes q in [-8, 7]
 * with one fp16 scale per 32 consecutive entries along the factor's first
 * axis (d_in for A, d_out for B) and per rank column:
 *   scale = fp16_round_nearest_even(amax / 7.0f)   (FP32 division)
 *   q     = clamp(round_half_even(v / (float)scale), -8, 7)   (FP32)
 *   value = (float)q * (float)scale                 (exact in FP32)
 * amax == 0, or a scale that rounds to zero, gives scale 0 and q 0. */
typedef enum {
  MOE_RESID_NONE = 0,
  MOE_RESID_F32 = 1,
  MOE_RESID_F16 = 2,
  MOE_RESID_INT4_G32 = 3
} moe_resid;

typedef enum { MOE_ACT_GELU_TANH = 0, MOE_ACT_SWIGLU = 1 } moe_act;

/* Layer shape.  Supported: 1 <= G <= 256, 1 <= K <= 256, G*K <= 1024, and
 * K <= 64 when r > 0; 1 <= top_groups <= min(G, 8); 1 <= top_experts <= K;
 * top_groups*top_experts <= 16; d and f multiples of 64; r in {0} or 1..16
 * (r = 0 iff resid == MOE_RESID_NONE);
 * dtype mixes (x, base): (F32, F32), (F16, F16), (BF16, BF16), (BF16, F16)
 * -- bf16 activations are converted to fp16 for an fp16 base; residual F32
 * needs an F32 base, F16 an F16 base, INT4_G32 an F16 or BF16 base. */
typedef struct {
  int32_t T_max;       /* largest T a later call may pass */
  int32_t d;           /* model width (input and output of the layer) */
  int32_t f;           /* expert hidden width */
  int32_t G;           /* groups */
  int32_t K;           /* experts per group; E = G*K */
  int32_t top_groups;  /* groups chosen per token (kg) */
  int32_t top_experts; /* experts chosen per chosen group (ke); k = kg*ke */
  int32_t r;           /* residual rank */
  int32_t act;         /* moe_act */
  int32_t x_dtype;     /* moe_dtype of X and Y */
  int32_t base_dtype;  /* moe_dtype of the base weights */
  int32_t resid;       /* moe_resid */
} moe_config;

/* Weights, row-major, read only during moe_create (the caller keeps
 * ownership).  on_device = 0: every pointer is a HOST pointer; on_device = 1:
 * every pointer is a DEVICE pointer on the current HIP device (moe_create
 * reads them back before packing, so they may be freed once it returns).
 * Projections in order (gate, up, down) for SwiGLU, (w1, w2) for GELU;
 * d_in x d_out is d x f for the input projections and f x d for the output
 * projection.
 *   W_grp       float32 [d][G]
 *   W_exp       float32 [G][d][K]     (ignored, may be NULL, when K == 1)
 *   group_bias  float32 [G]           (NULL = zeros)
 *   expert_bias float32 [E]           (NULL = zeros; ignored when K == 1)
 *   base[p]     base_dtype [G][d_in][d_out]   (bf16 as raw uint16 bits)
 *   A[p]        [E][d_in][r]    float32 for RESID_F32 and RESID_INT4_G32
 *   B[p]        [E][d_out][r]   (INT4 is quantised inside moe_create from
 *                               these float32 values), float16 for F16;
 *                               NULL when r == 0. */
typedef struct {
  const float* W_grp;
  const float* W_exp;
  const float* group_bias;
  const float* expert_bias;
  const void* base[3];
  const void* A[3];
  const void* B[3];
  int32_t on_device;
} moe_weights;

/* Routing outputs, caller-owned DEVICE buffers (any may be NULL to skip it):
 *   idx      int32 [T][k]   global expert ids g*K + j, group-rank major:
 *                           entry a*ke + b is the b-th expert of the a-th group
 *   w        float [T][k]   gate weights (sum to 1 per token)
 *   gidx     int32 [T][kg]  chosen groups, best first
 *   counts   int32 [E]      tokens per expert
 *   offsets  int32 [E+1]    exclusive scan of counts, offsets[E] = T*k
 *   perm     int32 [T*k]    token ids, expert by expert, ascending within one
 *   gcounts  int32 [G]      tokens per group
 *   goffsets int32 [G+1]    exclusive scan of gcounts
 *   gperm    int32 [T*kg]   token ids, group by group, ascending within one */
typedef struct {
  int32_t* idx;
  float* w;
  int32_t* gidx;
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* gcounts;
  int32_t* goffsets;
  int32_t* gperm;
} moe_route_out;

typedef struct {
  int64_t stored_params;      /* G*sum_p d_in*d_out + E*r*sum_p (d_in + d_out) */
  int64_t stored_bytes;       /* expert weights as stored on the device */
  int64_t dense_equiv_params; /* E*sum_p d_in*d_out */
} moe_stats_t;

typedef struct moe_handle moe_handle;

/* Validate cfg, copy, re-lay-out and (for INT4) quantise the weights into
 * library-owned device memory on the current HIP device, and allocate the
 * workspace for T_max tokens.  Synchronous.  *out receives the handle. */
int moe_create(const moe_config* cfg, const moe_weights* weights, void* stream,
               moe_handle** out);

/* Routing only: scores, two-level top-k and gate weights, then the
 * per-expert and per-group token lists (counting, prefix sum, stable
 * scatter).  X: device [T][d] in x_dtype.  0 <= T <= T_max.  Every non-NULL
 * field of *out is written.  Asynchronous on stream. */
int moe_route(moe_handle* h, const void* X, int32_t T, const moe_route_out* out,
              void* stream);

/* The whole layer: Y = sum over the selected experts of gate weight times
 * expert FFN.  X, Y: device [T][d] in x_dtype (may not alias).  routing may
 * be NULL; otherwise its non-NULL fields receive the routing as in
 * moe_route (T = 0 included: zero counts and offsets).  Enqueue only: no
 * allocation, no host synchronisation, and the counters a pass needs are
 * cleared by its own kernels (no memset), so a call may be captured into a
 * HIP graph and replayed; replays give the same Y bit for bit.  One handle
 * is not re-entrant: calls on it must be ordered (one stream); distinct
 * handles are independent. */
int moe_forward(moe_handle* h, const void* X, int32_t T, void* Y,
                const moe_route_out* routing, void* stream);

/* moe_forward for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same kernels and results, but the workspace is a static
 * device array of 96 MiB per device (held until the process ends) instead
 * of the handle's own, carved per call for this T.  It calls no hipMalloc,
 * hipFree or other allocating routine.  A T whose workspace exceeds 96 MiB
 * is rejected with MOE_ERR_INVALID_ARG (the message gives the bytes it
 * needs); for scale, a d = 1024, f = 2816, top-2 layer needs about 66 MiB
 * at T = 2048.  The handle's device must be current.  All calls on one
 * device share the array: calls that overlap in time on one device (two
 * streams, two threads, two handles) race and give wrong results; order
 * them.  The counters it needs zeroed are cleared at the start of every
 * call. */
int moe_forward_noalloc(moe_handle* h, const void* X, int32_t T, void* Y,
                        const moe_route_out* routing, void* stream);

/* Gradients of the layer, caller-owned DEVICE buffers, float32, row-major,
 * in the shapes of moe_weights (written, not accumulated). */
typedef struct {
  float* dW_grp;        /* [d][G] */
  float* dW_exp;        /* [G][d][K]; may be NULL (zeros when K == 1) */
  float* d_group_bias;  /* [G]; may be NULL */
  float* d_expert_bias; /* [E]; may be NULL (zeros when K == 1) */
  float* dbase[3];      /* [G][d_in][d_out] per projection */
  float* dA[3];         /* [E][d_in][r] per projection (r > 0) */
  float* dB[3];         /* [E][d_out][r] per projection (r > 0) */
} moe_grads;

/* Backward pass of moe_forward for one batch: the gradients of
 * L = sum(dY * Y) with respect to X (dX, device [T][d] in x_dtype) and
 * every stored weight, through the experts and through the gate (softmax
 * over the chosen logits at each level; the top-k choice itself is held
 * fixed).  The factored form is kept: the base terms run once per (token,
 * group) -- D = dY W_down,base^T, dX gets dZbar W_in,base^T, dW_base^g =
 * X_g^T dZbar_g and hbar_g^T dY_g -- and the residual factors get
 * dA = dW~ B, dB = dW~^T A evaluated through rank-r products
 * ("Breaking the MoE LLM Trilemma", papernotes.org note: key design 2 and
 * the loss function / training strategy section).  INT4 residuals are
 * differentiated at their dequantised values.  X and dY: device [T][d] in
 * x_dtype.  The first call allocates the backward layouts and workspace for
 * T_max tokens (synchronous); later calls only enqueue on stream.  Every sum
 * runs in a fixed order, so equal inputs give equal bits.  T = 0 writes
 * zeros to every gradient.  Errors: MOE_ERR_INVALID_ARG (T outside
 * [0, T_max], a null buffer the layer needs), MOE_ERR_UNSUPPORTED (the
 * handle's groups are offloaded), MOE_ERR_OOM (first call). */
int moe_backward(moe_handle* h, const void* X, int32_t T, const void* dY, void* dX,
                 const moe_grads* grads, void* stream);

/* ---- idle-group offload ---------------------------------------------------
 * Whole groups of experts (a group's base and its experts' residual factors:
 * the unit the grouping makes, "Breaking the MoE LLM Trilemma" key design 4)
 * move to pinned host memory, and `slots` device slots hold the groups in
 * use; a group is swapped in when a batch routes tokens to it, the least
 * recently used resident group making room ("混合专家模型的路由机制与工程落地",
 * jiusizaji.com, section 6.2: swap inactive experts out, swap them in on
 * use, prefetch from the current batch's routing what the next batch will
 * need).  moe_offload_enable converts a created handle (synchronous;
 * 1 <= slots <= G); afterwards only moe_forward_offload and moe_route run on
 * it (moe_forward, moe_forward_noalloc and moe_backward return
 * MOE_ERR_UNSUPPORTED). */
typedef struct {
  int64_t calls;        /* moe_forward_offload calls */
  int64_t group_loads;  /* groups copied in because a batch needed them */
  int64_t group_hits;   /* needed groups that were already resident */
  int64_t prefetched;   /* groups copied in ahead of use (by recent use) */
  int64_t bytes_h2d;    /* host-to-device bytes of group weights */
  int64_t passes;       /* GEMM passes (more than one when a batch needs more groups than slots) */
} moe_offload_stats_t;

int moe_offload_enable(moe_handle* h, int32_t slots);

/* The layer with offloaded groups: routing on the device, then the host reads
 * which groups the batch touches (one device-to-host copy of the group counts
 * and a synchronisation of stream), copies the missing groups into slots on a
 * copy stream, and runs the grouped GEMMs once the copies of their groups
 * are done.  A batch that needs more groups than slots runs in passes of
 * slots/2 groups, the next pass's copies overlapping the current pass's
 * GEMMs.  After the batch, groups used often recently are copied into slots
 * of groups used less (prefetch).  Results equal moe_forward's.  Arguments as
 * moe_forward; calls on one handle must use one stream. */
int moe_forward_offload(moe_handle* h, const void* X, int32_t T, void* Y,
                        const moe_route_out* routing, void* stream);

int moe_offload_stats(const moe_handle* h, moe_offload_stats_t* out);

/* Free everything the handle owns (synchronises the device first).  NULL is
 * a no-op. */
int moe_destroy(moe_handle* h);

/* Text of the last error on this thread ("" if none). */
const char* moe_last_error(void);

/* Stored parameter and byte counts for a configuration; touches no device.
 * The count follows the compressed-expert form: one base per group and
 * projection, rank-r factors per expert. */
int moe_config_stats(const moe_config* cfg, moe_stats_t* out);

/* The same counts for a created layer. */
int moe_stats(const moe_handle* h, moe_stats_t* out);

/* ---- test and measurement exports -------------------------------------- */

/* Dequantised values of one residual factor as the kernels use them:
 * projection p, which = 0 for A (d_in x r) or 1 for B (d_out x r), expert
 * i; host_out (host, [n][r] float32, n = d_in or d_out).  For INT4 each
 * value is float(q) * float(scale), exact in FP32, decoded on the device by
 * the routine the GEMM kernels call (the GEMMs round it once more to their
 * 16-bit MFMA type).  Synchronous. */
int moe_debug_dequant(moe_handle* h, int32_t proj, int32_t which, int32_t expert, float* host_out);

/* INT4 codes and scales of the same factor as stored: q (host int8 [n][r],
 * values in [-8, 7]) and scale_bits (host uint16 [n/32][r], fp16 bits); either
 * may be NULL.  MOE_ERR_INVALID_ARG for a layer whose residual is not INT4.
 * Synchronous. */
int moe_debug_q(moe_handle* h, int32_t proj, int32_t which, int32_t expert, int8_t* q,
                uint16_t* scale_bits);

/* Both of the above in one call: projection p,
 * which = 0 for A (d_in x r) or 1 for B (d_out x r), expert i.  values
 * (host, [n][r] float32) receives the value the kernels use, decoded on
 * the device by the same routine the GEMM kernels call.  For INT4, q (host
 * int8 [n][r]) and scale_bits (host uint16 [n/32][r], fp16 bits) receive
 * the stored codes and scales when non-NULL.  Synchronous. */
int moe_debug_residual(moe_handle* h, int32_t proj, int32_t which, int32_t expert,
                       float* values, int8_t* q, uint16_t* scale_bits);

/* Per-stage GPU timing: after moe_profile_begin, each moe_forward records
 * a pair of HIP events, on the stream it was given, around every kernel it
 * launches whose stage bit is set in stage_mask (bit s = stage s in the
 * order router, scatter, ugemm, gemm1, vreduce, gemm2, combine; -1 =
 * all), for at
 * most max_calls calls.  moe_profile_end synchronises, writes the summed
 * milliseconds per stage into stage_ms[n_stages_cap], the stage count into
 * *n_stages, the recorded calls into *n_calls and comma-separated stage
 * names into names[names_cap], then stops recording.  Not for use under
 * stream capture. */
int moe_profile_begin(moe_handle* h, int32_t max_calls, int32_t stage_mask);
int moe_profile_end(moe_handle* h, float* stage_ms, int32_t n_stages_cap,
                    int32_t* n_stages, int32_t* n_calls, char* names, int32_t names_cap);

#ifdef __cplusplus
}
#endif
#endif /* CEFN_MOE_H */
