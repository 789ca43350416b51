/*
 * moe_sparse.h -- C ABI of libmoesparse, a routed Mixture-of-Experts SwiGLU
 * expert FFN with intra-expert activation sparsity, for AMD MI355X (gfx950).
 *
 * The method is arXiv 2605.08575, "Uncovering Intra-expert Activation
 * Sparsity for Efficient Mixture-of-Expert Model Execution".  Citations below
 * name the gist.science explanation page of that paper ("Technical Summary",
 * its Methodology subsections and Results) or the arXiv abstract quoted on
 * the mlsanity.com page.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Every array pointer is a DEVICE pointer owned by the caller (for example
 *    a PyTorch tensor's data_ptr()).  The library never allocates, frees or
 *    retains caller memory and never synchronises the host: each call only
 *    validates its arguments and enqueues kernels on `hip_stream` (a
 *    hipStream_t; NULL means the default stream).  Calls are therefore
 *    capturable in a HIP graph.  Concurrent calls on different streams need
 *    separate workspaces.  The state kept between calls is a per-device
 *    cache of an occupancy query (how many down-projection workgroups a
 *    device holds at once), read and written atomically, and, for
 *    moe_sparse_expert_ffn_noalloc only, its fixed scratch array per device
 *    and that array's device address.
 *  - Errors that the host can detect are returned before any HIP call is
 *    made (so they are reported even on a machine without a GPU):
 *      MOE_ERR_INVALID_ARG  a NULL required pointer, a non-positive size,
 *                           K > E, q outside [0,1], an unknown enum value,
 *                           or a pointer that is not 16-byte aligned;
 *      MOE_ERR_UNSUPPORTED  a shape outside what the kernels implement (see
 *                           moe_shape);
 *      MOE_ERR_WORKSPACE    workspace smaller than the *_workspace_size value.
 *    MOE_ERR_HIP reports a failed kernel launch.  Faults inside a kernel are
 *    asynchronous and surface at the caller's next synchronisation.
 *  - No exception crosses the ABI and nothing is printed.
 *  - Weight matrices are NEURON-MAJOR: w[e][j][:] is row j (one neuron) of
 *    expert e with H contiguous elements.  This holds for the down
 *    projection too: w_down[e][j][:] holds neuron j's H output weights, i.e.
 *    the transpose of the usual [H, I] down matrix, so that a neuron that is
 *    skipped owns one contiguous row that is never read (the "Fused Up-Down
 *    Projection" of the Technical Summary gathers only active neurons'
 *    weights).
 */
#ifndef MOE_SPARSE_H
#define MOE_SPARSE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,
    MOE_ERR_UNSUPPORTED = 2,
    MOE_ERR_WORKSPACE = 3,
    MOE_ERR_HIP = 4
} moe_status;

/* Element type of the hidden states (x_dtype) and of the weight matrices
 * (w_dtype). */
typedef enum { MOE_F32 = 0, MOE_BF16 = 1 } moe_dtype;

/* MOE_SPARSE applies the threshold mask; MOE_DENSE computes the ordinary
 * dense SwiGLU MoE layer (every neuron active) and serves as the baseline the
 * sparse execution is compared with (Technical Summary, Results: layer
 * speedup over the dense pipeline).  MOE_TOPK is the alternative the
 * threshold pass is contrasted with (Technical Summary, Methodology,
 * Activation Masking: a top-k selection instead of one elementwise pass):
 * for every (token, slot) pair the neuron_budget neurons with the largest
 * |a_j| are active, whatever their values. */
typedef enum { MOE_SPARSE = 0, MOE_DENSE = 1, MOE_TOPK = 2 } moe_mode;

/*
 * Layer shape.
 *   T  tokens in the batch (T = 0 is a valid empty batch: calls return MOE_OK
 *      and enqueue nothing)
 *   H  hidden size; E routed experts; I intermediate size of a routed expert
 *   K  experts per token (top-K routing), 1 <= K <= E, K <= 32
 *   S  shared experts (always active, weight 1; may be 0); I_shared their
 *      intermediate size (ignored when S = 0)
 *   x_dtype      moe_dtype of the hidden states x
 *   w_dtype      moe_dtype of every weight matrix (routed and shared)
 *   renormalize  1: the K routing weights are divided by their sum;
 *                0: they are the softmax probabilities over all E experts
 * Supported by the kernels (else MOE_ERR_UNSUPPORTED):
 *   x_dtype == w_dtype (bf16 weights with bf16 hidden states, or fp32 with
 *   fp32); H = s * 64 * L with s in {1,2,4,8,16}, where L = 8 for bf16 and 4
 *   for f32 (so H in {512,1024,2048,4096,8192} for bf16); I and I_shared
 *   multiples of 32 and at most 16384; E + S <= 512.
 */
typedef struct {
    int32_t T, H, E, I, K, S, I_shared;
    int32_t x_dtype, w_dtype;
    int32_t renormalize;
} moe_shape;

/*
 * Top-K softmax routing (Technical Summary, Methodology: the router logic is
 * kept unchanged).
 *   logits  [T,E] fp32, row-major.
 *   out topk_ids [T,K] int32: the K experts with the largest logits (softmax
 *           is strictly increasing, so these are the K most probable), in
 *           descending order; equal logits are ranked by lower expert id; a NaN
 *           logit ranks as -infinity.
 *   out topk_w   [T,K] fp32: softmax probability of each chosen expert
 *           (computed over all E), divided by the sum of the K chosen ones
 *           when renormalize = 1.  A NaN or +infinity logit makes the
 *           token's softmax denominator NaN, and so all its K weights.
 * Requires T >= 0, E >= 1, 1 <= K <= min(E, 32), E <= 512.
 */
moe_status moe_route_topk(const float *logits, int32_t T, int32_t E, int32_t K,
                          int32_t renormalize, int32_t *topk_ids, float *topk_w,
                          void *hip_stream);

/* Arguments of moe_sparse_expert_ffn.  Shapes refer to moe_shape; W denotes
 * ceil(max(I, I_shared)/32) and Imax = max(I, I_shared). */
typedef struct {
    const void *x;              /* [T,H] x_dtype, 16-byte aligned */
    const float *router_logits; /* [T,E] fp32 */
    const void *w_gate;         /* [E,I,H] w_dtype, neuron-major, 16-byte aligned */
    const void *w_up;           /* [E,I,H] */
    const void *w_down;         /* [E,I,H] neuron-major (transpose of [H,I]) */
    const void *ws_gate;        /* [S,I_shared,H] or NULL when S = 0 */
    const void *ws_up;
    const void *ws_down;
    const float *tau;           /* [E+S] fp32 thresholds (routed experts then
                                   shared ones); required in MOE_SPARSE,
                                   ignored in MOE_DENSE */
    float *y;                   /* OUT [T,H] fp32 layer output */
    uint32_t *mask_bits;        /* OUT or NULL: [T,K+S,W]; bit j%32 of word j/32
                                   of row (t,slot) is 1 iff neuron j was active
                                   for token t in that slot; slots 0..K-1 follow
                                   topk_ids, slots K..K+S-1 are the shared
                                   experts; bits at and beyond the expert's
                                   row count are 0 */
    int32_t *union_idx;         /* OUT or NULL: [E+S,Imax]; row e starts with the
                                   union_cnt[e] neurons active for at least one
                                   pair of expert e, ascending; later entries
                                   are unspecified */
    int32_t *union_cnt;         /* OUT or NULL: [E+S]; 0 for experts no token
                                   was routed to */
    int32_t *topk_ids;          /* OUT or NULL: [T,K] as moe_route_topk */
    float *topk_w;              /* OUT or NULL: [T,K] as moe_route_topk */
    void *workspace;            /* device scratch, 256-byte aligned */
    size_t workspace_bytes;     /* >= moe_workspace_size(shape, mode) */
    int32_t neuron_budget;      /* MOE_TOPK only: active neurons per (token,
                                   slot) pair, >= 0; an expert with fewer rows
                                   keeps all of them.  The order is |a_j|
                                   descending, a NaN score first, equal scores
                                   by ascending j.  tau is not read. */
} moe_ffn_args;

/*
 * Workspace bytes that moe_sparse_expert_ffn needs for this shape and mode
 * (depends on the shape only, never on the data).  Returns MOE_OK and sets
 * *bytes, or the status that moe_sparse_expert_ffn would return for an
 * invalid / unsupported shape (so a caller learns which check failed).
 */
moe_status moe_workspace_size(const moe_shape *shape, int32_t mode, size_t *bytes);

/*
 * The layer (Technical Summary, Methodology: Gate Projection, Activation
 * Masking, Fused Up-Down Projection).  For each token t and slot k with
 * expert e (routed slots from top-K routing, then the shared experts with
 * weight 1):
 *   a_j = SiLU(x_t . w_gate[e][j])        for every neuron j (dense gate)
 *   m_j = NOT(|a_j| < tau[e])             (MOE_DENSE: m_j = 1)
 *   h_j = a_j * (x_t . w_up[e][j]) where m_j = 1, exactly 0 where m_j = 0
 *   o   = sum_j h_j * w_down[e][j]
 *   y_t = sum_{k<K} topk_w[t,k] * o_{t,k} + sum_{s<S} o_{t,K+s}
 * Rows of w_down that are inactive for every token routed to an expert are
 * not read; neither are such rows of w_up for an expert with fewer than 16
 * routed pairs.  An expert with more (the bf16 matrix-core path)
 * computes its up products for every row of each 64-row tile together with
 * the gate, which reads each token tile's hidden states once; its h, and so
 * y, are the same.  A NaN score counts as active and propagates into y.
 * Accumulation is fp32; the result is deterministic (no floating-point
 * atomics): the same inputs give bitwise-identical outputs.
 * Requires 16-byte aligned x and weights and a 256-byte aligned workspace.
 */
moe_status moe_sparse_expert_ffn(const moe_shape *shape, int32_t mode,
                                 const moe_ffn_args *args, void *hip_stream);

/*
 * moe_sparse_expert_ffn without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  args->workspace and
 * args->workspace_bytes are ignored: the call uses a fixed scratch array of
 * MOE_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it runs on
 * until the process ends, and it calls no allocating routine.  Shapes whose
 * moe_workspace_size(shape, mode) exceeds that size return
 * MOE_ERR_WORKSPACE before any HIP call (64 MiB holds the decode layers of
 * the workloads above up to 64 tokens; a prefill batch needs a workspace).
 * Every call on one GPU shares that GPU's array, which keeps the last call's
 * contents (the kernels clear what must start at zero): calls that overlap
 * on one GPU (on different streams, or from several host threads) race and
 * must be serialised by the caller.  Outputs, errors and determinism are
 * those of moe_sparse_expert_ffn.
 */
#define MOE_NOALLOC_SCRATCH_BYTES (64u << 20)
moe_status moe_sparse_expert_ffn_noalloc(const moe_shape *shape, int32_t mode,
                                         const moe_ffn_args *args, void *hip_stream);

/*
 * Workspace bytes for moe_calibrate_threshold with Tc calibration tokens.
 */
moe_status moe_calibrate_workspace_size(const moe_shape *shape, int32_t Tc, size_t *bytes);

/*
 * Threshold calibration to a target sparsity q (Technical Summary, Results:
 * sparsity cutoffs / target sparsity).  Runs the routing and the dense gate
 * on Tc calibration tokens and sets, on the device,
 *   tau_out[e] = v[floor(q*N)]   (0-indexed ascending order statistic)
 * where v are the N scores |SiLU(x_t . w_gate[e][j])| over every routed
 * (token, slot) pair and every neuron of the selected expert; the shared
 * experts form a separate population.  q = 0 gives 0; floor(q*N) = N gives
 * +infinity.  With per_expert = 1 each expert uses its own pairs, and a
 * routed expert with no calibration pair falls back to the routed
 * population's value.  floor(q*N) is evaluated in double precision on the
 * float q.  NaN scores order after +infinity.  With no ties among the scores,
 * exactly floor(q*N) of them are < tau.
 *   x_calib [Tc,H] x_dtype; logits_calib [Tc,E] fp32; w_gate / ws_gate as in
 *   moe_ffn_args; tau_out [E+S] fp32.  Tc >= 1; q in [0,1].
 */
moe_status moe_calibrate_threshold(const moe_shape *shape, const void *x_calib,
                                   const float *logits_calib, int32_t Tc,
                                   const void *w_gate, const void *ws_gate, float q,
                                   int32_t per_expert, float *tau_out, void *workspace,
                                   size_t workspace_bytes, void *hip_stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char *moe_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MOE_SPARSE_H */
