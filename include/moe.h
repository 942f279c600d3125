/*
 * moe.h — C-ABI of the MI355X (gfx950) sparse MoE FFN layer library
 * (libmoe_mi355x.so).
 *
 * The layer: top-k routing with softmax, sigmoid or sqrtsoftplus scores and
 * an fp32 selection bias, sorted-segment dispatch into contiguous per-expert
 * groups, a grouped SwiGLU expert GEMM over stacked [E, out, in] weights, a
 * routing-weighted combine, an optional (sigmoid-gated) shared expert, and
 * the matching backward.
 *
 * Conventions for every entry point
 *   - Every array pointer is a caller-owned DEVICE buffer unless stated
 *     otherwise; the library never allocates or frees device memory and keeps
 *     no data between calls (per device it caches kernel attributes, the CU
 *     count, and one side stream with two events, created on first use and
 *     kept until the process ends).  `shape` and `w` point to HOST structs.
 *   - All arrays are dense, row-major, contiguous.
 *   - Calls are asynchronous on `stream` (a hipStream_t passed as void*;
 *     NULL = the default stream) and never synchronise with the host.
 *     Outputs are valid once the stream reaches the call.  A forward whose
 *     routed GEMMs are weight streams (decode-sized batches) runs the shared
 *     expert's GEMMs on the side stream, forked from `stream` and joined back
 *     into it by events before the call returns; graph capture of `stream`
 *     takes the side stream's work in with it.
 *   - Return value: MOE_OK (0) or a negative status.  All argument checks
 *     run on the host before anything is launched, so a failing call has no
 *     effect on device memory.  MOE_ELAUNCH reports a launch error.
 *   - T == 0 is valid: pointers to [T]-sized ([T*k], [T,H], ...) arrays may
 *     then be NULL and are not read; per-expert outputs are still written
 *     (counts and offsets zero, score sums zero, weight gradients zero).
 *   - dtype MOE_DTYPE_BF16: x, weights, activations and outputs are
 *     bfloat16, all accumulation is fp32; weight gradients are fp32; expert
 *     outputs are stored in binary16 (see moe_saved).  MOE_DTYPE_FP32:
 *     everything fp32.  Routing weights, logits, gates, bias are always fp32;
 *     expert ids are int64; counts/offsets/perm/pos are int32.
 *   - Limits: 1 <= k <= E <= 256; H % 8 == 0, I % 8 == 0, Is % 8 == 0;
 *     T * k < 2^31.
 *
 * Citations name the page title and the section on it that defines each
 * operation.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_OK 0
#define MOE_EINVAL (-1)        /* bad size, k <= 0, k > E, NULL required pointer */
#define MOE_EUNSUPPORTED (-2)  /* E > 256, unsupported dtype/score, size not a multiple of 8 */
#define MOE_EWORKSPACE (-3)    /* workspace NULL or smaller than moe_workspace_bytes */
#define MOE_ELAUNCH (-4)       /* a kernel launch failed (hipGetLastError) */

#define MOE_SCORE_SOFTMAX 0
#define MOE_SCORE_SIGMOID 1
#define MOE_SCORE_SQRTSOFTPLUS 2

#define MOE_DTYPE_FP32 0
#define MOE_DTYPE_BF16 1

/* moe_route flags */
#define MOE_ROUTE_LOGITS_IN 1  /* read `logits` instead of computing x . w_router^T */

/* moe_workspace_bytes ops */
#define MOE_OP_DISPATCH 1
#define MOE_OP_FFN_FORWARD 2
#define MOE_OP_FFN_BACKWARD 3
#define MOE_OP_ROUTE 4         /* scratch of moe_route (score sums, split reduction) */
#define MOE_OP_FFN_PARTIAL 5   /* scratch of moe_ffn_forward_partial */
#define MOE_OP_BLOCK 6         /* scratch of moe_parallel_block_forward */
#define MOE_OP_ROUTE_DISPATCH 7 /* scratch of moe_route_dispatch */
#define MOE_OP_LAYER_FORWARD 8  /* scratch of moe_layer_forward */

typedef struct moe_shape {
  int64_t T;   /* tokens */
  int64_t H;   /* hidden size */
  int64_t E;   /* routed experts (<= 256) */
  int64_t k;   /* experts per token */
  int64_t I;   /* routed expert intermediate size (moe_intermediate_size) */
  int64_t Is;  /* shared expert intermediate size; 0 = no shared expert */
  int32_t score;        /* MOE_SCORE_* */
  int32_t renorm;       /* norm_topk_prob: divide selected scores by their sum */
  int32_t shared_gated; /* shared expert scaled by sigmoid(x . w_shared_gate) */
  int32_t dtype;        /* MOE_DTYPE_* */
} moe_shape;

/* Expert parameters in the fused checkpoint layout ("mstar.model.components.moe",
 * SparseMoeBlock: experts.gate_up_proj (E, 2I, H), experts.down_proj (E, H, I)).
 * Rows [0, I) of each gate_up slice are the gate projection, rows [I, 2I) the
 * up projection.  The shared expert uses the same layout with E = 1 and Is. */
typedef struct moe_weights {
  const void* w_gate_up;      /* [E, 2I, H] */
  const void* w_down;         /* [E, H, I] */
  const void* ws_gate_up;     /* [2Is, H] or NULL when Is == 0 */
  const void* ws_down;        /* [H, Is]  or NULL when Is == 0 */
  const void* w_shared_gate;  /* [H] or NULL (needed when shared_gated) */
} moe_weights;

/* Activations the forward keeps for the backward (device).  h and s_h (the
 * operands of the down projections) have the layer dtype; the pre-activations
 * gu, s_gu are fp32 (the SwiGLU backward reads exact g, u); the expert
 * outputs y, s_y are binary16 (IEEE half) in a bf16 layer and fp32 in an
 * fp32 layer: the combine sums them in fp32 before the single rounding of
 * `out`, and half storage keeps 11 significant bits (bf16: 8) at half the
 * bytes of fp32.  Expert outputs beyond the half range (|y| > 65504) become
 * inf and propagate to `out`. */
typedef struct moe_saved {
  void* gu;    /* [T*k, 2I]  fp32 routed pre-activations (gate | up), sorted rows */
  void* h;     /* [T*k, I]   silu(gate) * up, sorted rows (dtype) */
  void* y;     /* [T*k, H]   routed expert outputs before weighting, sorted rows (half / fp32) */
  void* s_gu;  /* [T, 2Is]   fp32 shared pre-activations (NULL when Is == 0) */
  void* s_h;   /* [T, Is]    dtype */
  void* s_y;   /* [T, H]     shared expert output before the gate (half / fp32) */
} moe_saved;

/* Gradient outputs of moe_ffn_backward (device).  dx has the layer dtype;
 * every weight gradient is fp32 (master-gradient precision: the weight
 * gradients are sums over many rows and heavy-tailed across experts). */
typedef struct moe_grads {
  void* dx;              /* [T, H] dtype */
  float* dw_router;      /* [E, H] fp32 */
  float* dw_gate_up;     /* [E, 2I, H] fp32 */
  float* dw_down;        /* [E, H, I] fp32 */
  float* dws_gate_up;    /* [2Is, H] fp32 or NULL */
  float* dws_down;       /* [H, Is] fp32 or NULL */
  float* dw_shared_gate; /* [H] fp32 or NULL */
  float* dlogits;        /* [T, E] fp32, optional (NULL: not returned) */
} moe_grads;

/*
 * moe_route — the router ("mstar.model.components.moe", Router contract and
 * TopKRouter; "Sparse MoE FFN for DFlash-family drafters", What's here:
 * MoEGate with the aux-loss-free balancing bias).
 *
 *   logits[t,e] = sum_h x[t,h] w_router[e,h]      (fp32 accumulation)
 *   score: softmax over all E, sigmoid, or sqrt(softplus)
 *   key   = logit            (no bias: every score is increasing in the logit)
 *         = fl32(score + sel_bias[e])   (bias: fixed fp32 score recipe)
 *   ids[t, 0..k-1]: the k largest keys, descending, ties to the lower index
 *   weights[t,j] = score[t, ids[t,j]] (unbiased), / sum_j when renorm
 *   gate[t] = sigmoid(x[t] . w_shared_gate) when w_shared_gate != NULL
 *
 * x [T,H] dtype; w_router [E,H] dtype; w_shared_gate [H] dtype or NULL;
 * sel_bias [E] fp32 or NULL (used for selection only, never in the weights);
 * logits [T,E] fp32: output if non-NULL, or input when flags has
 * MOE_ROUTE_LOGITS_IN (then x and w_router are not read and gate must be
 * NULL); weights [T,k] fp32 out; ids [T,k] int64 out; gate [T] fp32 out or
 * NULL.
 *
 * score_sums [E] fp32 out or NULL: sum over the T tokens of each expert's
 * unbiased score (the fp32 scores the weights come from), the input of the
 * load-balancing aux loss ("feat: Phase 43", aux loss computed in the gating
 * step before dispatch).  The router kernel writes per-tile column sums into
 * ws, a second kernel adds them in a fixed order, so two calls give
 * identical bits.  T == 0 writes zeros.
 *
 * ws: scratch of at least moe_workspace_bytes(shape, MOE_OP_ROUTE) bytes,
 * 16-byte aligned, contents scratch; required with score_sums, optional
 * otherwise.  When given, a bf16 router whose token tiles are too few to
 * fill the GPU (short batches, e.g. decode) splits its reduction over H
 * across workgroups and adds the partial logit tiles in a fixed order: the
 * logits may then differ from a call without ws in the last bits (both
 * within fp32 accumulation error), and two calls with ws give identical
 * bits.
 *
 * Errors: MOE_EINVAL (NULL x/w_router/weights/ids, k out of range, gate
 * requested without w_shared_gate), MOE_EUNSUPPORTED (E > 256),
 * MOE_EWORKSPACE (score_sums without ws, or a ws that is too small or
 * misaligned).
 */
int moe_route(const moe_shape* shape, const void* x, const void* w_router,
              const void* w_shared_gate, const float* sel_bias, float* logits,
              float* weights, int64_t* ids, float* gate, float* score_sums,
              void* ws, size_t ws_bytes, int flags, void* stream);

/*
 * moe_aux_loss — the load-balancing auxiliary loss and its score gradient
 * ("feat: Phase 43", load balancing aux loss in the gating step, independent
 * of the dispatch kind).  The pages give no formula; this is the Switch-style
 * reading
 *
 *   loss    = alpha * E * sum_e f_e * P_e,  f_e = counts[e] / (T*k),
 *                                           P_e = score_sums[e] / T
 *   coef[e] = d loss / d score[t,e] = alpha * E * counts[e] / (T*k*T)
 *             (the same for every token t; counts carry no gradient)
 *
 * score_sums [E] fp32 from moe_route; counts [E] int32 from moe_dispatch or
 * moe_balance_counts; loss [1] fp32 out or NULL; coef [E] fp32 out or NULL
 * (pass it to moe_ffn_backward as aux_coef to add alpha * aux to the loss
 * being differentiated).  Accumulation in fp64, fixed order.  Errors:
 * MOE_EINVAL (NULL score_sums/counts, both outputs NULL, T == 0).
 */
int moe_aux_loss(const moe_shape* shape, const float* score_sums, const int32_t* counts,
                 float alpha, float* loss, float* coef, void* stream);

/*
 * moe_dispatch — sorted-segment dispatch ("Sparse MoE FFN for DFlash-family
 * drafters", What's here, SparseMoE: one argsort into contiguous per-expert
 * segments; "feat: Phase 43 — Sparse/Grouped MoE Dispatch", arg_sort then
 * index_select).  A counting sort, stable in the flat index i = t*k + j:
 *
 *   counts[e]  = #{i : ids[i] == e}
 *   offsets[e] = sum_{e' < e} counts[e'], offsets[E] = T*k
 *   pos[i]     = offsets[ids[i]] + #{i' < i : ids[i'] == ids[i]}
 *   perm[pos[i]] = i
 *   x_sorted[pos[t*k+j]] = x[t]            (only when x_sorted != NULL)
 *
 * ids [T,k] int64 (values must lie in [0,E)); x [T,H] dtype (may be NULL
 * when x_sorted is NULL); counts [E], offsets [E+1], perm [T*k], pos [T*k]
 * int32 out; x_sorted [T*k, H] dtype out or NULL.  ws: device workspace of
 * at least moe_workspace_bytes(shape, MOE_OP_DISPATCH) bytes.
 */
int moe_dispatch(const moe_shape* shape, const int64_t* ids, const void* x,
                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                 void* x_sorted, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_route_dispatch — moe_route followed by moe_dispatch (without the row
 * gather) in two launches: the router counts, per tile of tokens, how many
 * selections each expert received as it makes them ("Sparse MoE FFN for
 * DFlash-family drafters", What's here, SparseMoE: one sort of the
 * (token, slot) pairs into expert segments), and one kernel turns those
 * counts into counts, offsets, perm and pos.  Arguments and outputs as the two
 * calls' (weights, ids, logits, gate, score_sums as moe_route; counts,
 * offsets, perm, pos as moe_dispatch), all bit for bit equal to them.
 * ws: at least moe_workspace_bytes(shape, MOE_OP_ROUTE_DISPATCH) bytes
 * (the router's scratch, then the per-tile loads); required.
 * Errors: those of moe_route and moe_dispatch.
 */
int moe_route_dispatch(const moe_shape* shape, const void* x, const void* w_router,
                       const void* w_shared_gate, const float* sel_bias, float* logits,
                       float* weights, int64_t* ids, float* gate, float* score_sums,
                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* pos,
                       void* ws, size_t ws_bytes, int flags, void* stream);

/*
 * moe_ffn_forward — grouped SwiGLU experts, combine and shared expert
 * ("mstar.model.components.moe", SparseMoeBlock fused layout and
 * SparseMoeBlockWithSharedExpert: out = routed(x) + sigmoid(shared_gate(x)) *
 * shared_expert(x); "feat: Phase 43", index_select -> expert -> index_add).
 *
 *   for each expert e with counts[e] > 0, sorted rows r in its segment:
 *     [g | u] = x_sorted[r] . w_gate_up[e]^T;  h = silu(g) * u
 *     y[r]    = h . w_down[e]^T
 *   out[t] = sum_{j=0..k-1} weights[t,j] * y[pos[t*k+j]]   (fp32, this order)
 *          + gate[t] * S(x[t])     (gate = 1 when ungated; S = shared SwiGLU)
 *
 * y and S are stored (workspace or saved) in binary16 for a bf16 layer and in
 * fp32 for an fp32 layer, and widened to fp32 for the sum (see moe_saved).
 * Empty experts launch no work and their weights are never read.
 * x [T,H]; x_sorted [T*k,H] or NULL (then rows are read from x through
 * perm[r] / k); offsets/perm/pos from moe_dispatch; weights [T,k] fp32;
 * gate [T] fp32 (required when shared_gated); out [T,H] dtype.
 * saved: NULL for inference, else every non-NULL buffer in it receives the
 * activations the backward needs (gu and h and y required; s_* when Is > 0).
 * An inference call of a bf16 layer whose expert GEMMs are weight streams
 * (decode-sized batches: segments of a few rows) keeps h as a pair of bf16
 * tensors, hi = bf16(h) and lo = bf16(h - hi), which the down projection
 * multiplies both (its operand then has about 16 significant bits); the
 * workspace holds the lo parts.  Calls with saved activations use bf16 h,
 * the operand the backward differentiates.
 * ws: at least moe_workspace_bytes(shape, MOE_OP_FFN_FORWARD) bytes.
 */
int moe_ffn_forward(const moe_shape* shape, const moe_weights* w, const void* x,
                    const void* x_sorted, const int32_t* offsets, const int32_t* perm,
                    const int32_t* pos, const float* weights, const float* gate,
                    void* out, const moe_saved* saved, void* ws, size_t ws_bytes,
                    void* stream);

/*
 * moe_layer_forward — the whole inference forward of the layer in one call:
 * moe_route_dispatch (no logits, no score sums, flags 0) followed by
 * moe_ffn_forward (rows read from x through perm, no saved activations), the
 * sequence of "mstar.model.components.moe", Router contract and
 * SparseMoeBlockWithSharedExpert (route, run the experts on their segments,
 * add the gated shared expert).  Arguments as those two calls' (weights, ids,
 * gate, counts, offsets, perm, pos are outputs, as there), and every output
 * bit for bit equal to theirs.  The one call lets the library order the
 * work: for a decode-sized bf16 layer with a shared expert (routed GEMMs
 * that are weight streams, T * k <= 8 E) the shared expert's GEMMs, which need only x, are
 * queued on the library's side stream before the routing and joined back
 * before the combine, so its weight stream overlaps the routing's small
 * kernels; with a stage profile running everything stays on `stream`.
 * ws: at least moe_workspace_bytes(shape, MOE_OP_LAYER_FORWARD) bytes (the
 * routing's scratch, then the forward's); required.
 * Errors: those of moe_route_dispatch and moe_ffn_forward; every argument is
 * checked before the first launch.
 */
int moe_layer_forward(const moe_shape* shape, const moe_weights* w, const void* x,
                      const void* w_router, const void* w_shared_gate, const float* sel_bias,
                      float* weights, int64_t* ids, float* gate, int32_t* counts,
                      int32_t* offsets, int32_t* perm, int32_t* pos, void* out, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * moe_ffn_forward_noalloc — moe_ffn_forward for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation): an inference call (no saved
 * activations) that takes no workspace.  Its scratch is a 64 MiB device
 * array inside the library, one per GPU, held until the process ends; no
 * call allocates or frees memory, or creates a stream or an event (the
 * shared expert always runs on `stream`).  Same arguments and results as
 * moe_ffn_forward with saved == NULL; the outputs equal that call's bit for
 * bit.
 *   Limit: MOE_EWORKSPACE when moe_workspace_bytes(shape,
 *   MOE_OP_FFN_FORWARD) exceeds 64 MiB (on a 256-CU device e.g. the
 *   Qwen2-MoE-like layer, H 2048, 60 experts top-4, shared 5632, up to about
 *   540 tokens; larger batches take moe_ffn_forward).
 *   Every call on a GPU uses that GPU's one array: calls that overlap on one
 *   GPU (two streams, two host threads) race and must be ordered by the
 *   caller.  Nothing in the array is read before the call writes it, so no
 *   clearing is needed between calls.
 * Errors: those of moe_ffn_forward; MOE_ELAUNCH also when the array's
 * device address cannot be obtained.
 */
int moe_ffn_forward_noalloc(const moe_shape* shape, const moe_weights* w, const void* x,
                            const void* x_sorted, const int32_t* offsets, const int32_t* perm,
                            const int32_t* pos, const float* weights, const float* gate,
                            void* out, void* stream);

/*
 * moe_ffn_forward_partial — one tensor-parallel share of the expert MLPs
 * ("mstar.model.components.moe", ParallelSparseMoeBlock: with more than one
 * rank the expert weights are split along the intermediate dimension and the
 * partial down-projection outputs are all-reduced before the top-k weighted
 * sum; ParallelSparseMoeBlockWithSharedExpert: the shared MLP is split the
 * same way).  shape->I and shape->Is are this share's slice sizes; w holds
 * the share's slices in the usual layouts: w_gate_up [E, 2I, H] with rows
 * [0, I) a slice of the gate rows and [I, 2I) the same slice of the up rows,
 * w_down [E, H, I] the matching columns; ws_gate_up [2Is, H], ws_down [H, Is]
 * likewise.  Routing (offsets, perm) is the full layer's: every share routes
 * identically.
 *
 *   y_part[r] = w_down[e] . (silu(g) * u)   for sorted row r of expert e,
 *   s_part[t] = ws_down . (silu(gs) * us)   (before the shared gate)
 *
 * y_part [T*k, H] fp32 out (sorted rows, the rows of moe_ffn_forward's saved y);
 * s_part [T, H] fp32 out (required when Is > 0, else ignored).  Summing the
 * shares' y_part and s_part element-wise (the all-reduce of a TP group) and
 * passing the sums to moe_combine gives the layer output.  saved (or NULL):
 * its gu, h, s_gu, s_h (each optional) receive this share's activations; its
 * y and s_y are ignored.  ws: at least moe_workspace_bytes(shape,
 * MOE_OP_FFN_PARTIAL) bytes.  Errors as moe_ffn_forward.
 */
int moe_ffn_forward_partial(const moe_shape* shape, const moe_weights* w, const void* x,
                            const void* x_sorted, const int32_t* offsets, const int32_t* perm,
                            float* y_part, float* s_part, const moe_saved* saved, void* ws,
                            size_t ws_bytes, void* stream);

/*
 * moe_combine — the top-k weighted sum and the shared term
 * ("mstar.model.components.moe", SparseMoeBlockWithSharedExpert: routed
 * output plus the sigmoid-gated shared expert output):
 *
 *   out[t] = sum_{j < k} weights[t,j] * y[pos[t*k+j]]  (+ gate[t] * s_y[t])
 *
 * in fp32, j in increasing order, rounded once to the layer dtype.  y [T*k, H]
 * fp32 sorted rows; pos [T*k] from moe_dispatch; weights [T,k] fp32; s_y
 * [T,H] fp32 or NULL (no shared term); gate [T] fp32 or NULL (ungated
 * shared term; needs s_y); out [T,H] dtype.  Errors: MOE_EINVAL (NULL or
 * misaligned required pointer, gate without s_y).
 */
int moe_combine(const moe_shape* shape, const float* y, const int32_t* pos, const float* weights,
                const float* gate, const float* s_y, void* out, void* stream);

/* Norms of the parallel dense + MoE block (moe_parallel_block_forward).  Each
 * scale is [H] in the layer dtype and is applied as given (a checkpoint that
 * stores w with an implied 1 + w passes 1 + w). */
typedef struct moe_block_norms {
  const void* g_pre_moe;     /* norm of the residual that feeds the experts */
  const void* g_post_dense;  /* norm of the dense MLP output */
  const void* g_post_moe;    /* norm of the MoE output */
  const void* g_post;        /* norm of their sum */
  float eps;                 /* added to mean(v^2) in every norm */
  float layer_scalar;        /* multiplies residual + block output */
} moe_block_norms;

/*
 * moe_parallel_block_forward — a dense MLP and the MoE side by side
 * (the DeepSpec issue "Feat: Compatible with Gamme4 MoE structure", Decoder
 * layer forward pass): the router reads the residual (moe_route on
 * `residual`, then moe_dispatch), the experts read its RMS-normalised copy,
 * and
 *
 *   N(v; g)  = v / sqrt(mean(v^2) + eps) * g            (per token, over H)
 *   x_moe    = N(residual; g_pre_moe)                    (layer dtype)
 *   moe[t]   = sum_j weights[t,j] * expert_{ids[t,j]}(x_moe[t])
 *   dense[t] = ws_down . (silu(gate) * up)(x_dense[t])   (the shared-expert
 *                                                        slots of w, width Is)
 *   out      = (residual + N(N(dense; g_post_dense) + N(moe; g_post_moe);
 *               g_post)) * layer_scalar
 *
 * shape: Is = dense MLP width (> 0), shared_gated = 0, k <= 8, H <= 8192.
 * residual, x_dense, out [T,H] dtype; offsets/perm/pos/weights from
 * moe_route(residual) and moe_dispatch.  Expert outputs are stored as in
 * moe_ffn_forward; every norm sums squares in fp32 (fp64 in an fp32 layer)
 * in a fixed order.  ws: at least moe_workspace_bytes(shape, MOE_OP_BLOCK)
 * bytes.  Errors: MOE_EINVAL (NULL or misaligned pointers, Is == 0, a gated
 * shared expert), MOE_EUNSUPPORTED (k > 8, H > 8192), MOE_EWORKSPACE.
 */
int moe_parallel_block_forward(const moe_shape* shape, const moe_weights* w,
                               const moe_block_norms* norms, const void* residual,
                               const void* x_dense, const int32_t* offsets, const int32_t* perm,
                               const int32_t* pos, const float* weights, void* out, void* ws,
                               size_t ws_bytes, void* stream);

/*
 * moe_ffn_backward — gradients of the layer ("feat: Phase 43", sparse
 * dispatch backward reaches router logits, expert parameters and input
 * activations; "Sparse MoE FFN for DFlash-family drafters", Tests: grouped
 * vs sorted-loop parity of outputs and grads).  For fixed ids:
 *
 *   dy[pos[t,j]]  = weights[t,j] * dout[t];  dweights[t,j] = dout[t] . y[pos[t,j]]
 *   dh = dy . w_down[e];  dg = dh * u * silu'(g);  du = dh * silu(g)
 *   dw_down[e] = sum_r dy[r]^T h[r];  dw_gate_up[e] = sum_r [dg|du][r]^T x[r]
 *   dx[t] = sum_j ([dg|du] . w_gate_up[e])[pos[t,j]]  + shared + router terms
 *   dscores from dweights (through renorm), dlogits through the score
 *   function (softmax couples all E), dw_router = dlogits^T x,
 *   dx += dlogits . w_router.  The bias and the permutation get no gradient.
 *
 * Weight gradients are written (not accumulated); experts with no rows get
 * exact zeros.  Every reduction runs in a fixed order without float atomics,
 * so two calls give identical bits.  logits [T,E] fp32 from moe_route;
 * ids, weights, gate, offsets, perm, pos and saved as produced by the
 * forward; x_sorted may be NULL (rows read from x through perm).
 * aux_coef [E] fp32 or NULL: moe_aux_loss's coef; when given, it is added to
 * every token's score gradient before the score-function backward, so
 * dlogits, dw_router and dx are those of sum(out * dout) + aux loss.
 * In a bf16 layer the per-slot data gradients (the rows of [dg|du] . w_gate_up
 * and the shared expert's) are kept in binary16 until their fp32 sum into dx:
 * one beyond the half range (65504) makes dx inf.
 * ws: at least moe_workspace_bytes(shape, MOE_OP_FFN_BACKWARD) bytes.
 * Errors: MOE_EINVAL (a NULL required pointer: w and its routed weights, x,
 * w_router, logits, ids, weights, offsets, perm, pos, saved and its routed
 * buffers, dout, grads and dx and the weight gradients, the shared ones when
 * Is > 0 and gate, w_shared_gate, dw_shared_gate when gated; or a tensor
 * not 16-byte aligned), MOE_EUNSUPPORTED (k > 8: the combine backward keeps
 * a token's k slot rows in registers), MOE_EWORKSPACE.
 */
int moe_ffn_backward(const moe_shape* shape, const moe_weights* w, const void* x,
                     const void* w_router, const float* logits, const int64_t* ids,
                     const float* weights, const float* gate, const int32_t* offsets,
                     const int32_t* perm, const int32_t* pos, const void* x_sorted,
                     const moe_saved* saved, const void* dout, const float* aux_coef,
                     const moe_grads* grads, void* ws, size_t ws_bytes, void* stream);

/*
 * moe_balance_counts — expert loads and the aux-loss-free bias controller
 * ("Sparse MoE FFN for DFlash-family drafters", What's here, MoEGate and the
 * deferred balance updates): an fp32 per-expert bias moved only by the
 * loads, by the sign of each expert's distance from the mean load, with no
 * gradient; a training forward's loads are applied when the next one
 * starts (the caller keeps them and calls this with ids == NULL).
 *
 *   counts[e] = #{(t,j) : ids[t,j] == e}
 *   if bias != NULL:  bias[e] += rate * sign(T*k/E - counts[e])  (sign(0)=0)
 *
 * ids [T,k] int64; counts [E] int32 out; bias [E] fp32 in/out or NULL.
 * When ids == NULL, counts is an INPUT (e.g. stashed from an earlier
 * forward) and only the bias update runs; the mean load then uses T*k.
 */
int moe_balance_counts(const moe_shape* shape, const int64_t* ids, int32_t* counts,
                       float* bias, float rate, void* stream);

/*
 * moe_score_f32 — the fixed fp32 score recipe the router uses for the biased
 * selection key, applied elementwise: s[i] = sigmoid32(l[i]) (score 1),
 * sqrtsoftplus32(l[i]) (score 2) or exp32(l[i]) (score 0: the softmax
 * numerator).  The recipe is stated in the router source; it exists so the
 * key computation can be checked exhaustively over every fp32 input.
 * l, s: n fp32 device values.  Errors: MOE_EINVAL (n < 0, NULL pointers),
 * MOE_EUNSUPPORTED (unknown score).
 */
int moe_score_f32(int score, const float* l, float* s, int64_t n, void* stream);

/*
 * moe_bandwidth_probe — measurement aid: a plain HBM stream of `bytes` bytes
 * (a multiple of 16; the remainder is ignored) by kernels of this library,
 * the ceiling the layer's memory-bound kernels are read against.
 *   kind 0: read src (dst receives one 4-byte word per launched thread:
 *           wgs * 256 * 4 bytes, a fold of what was read, so the loads stay);
 *   kind 1: write dst (non-temporal stores);
 *   kind 2: copy src -> dst (plain loads, non-temporal stores).
 * Each workgroup of 256 threads moves 32 KB blocks (8 independent 16-byte
 * accesses per thread, a wave's access one contiguous KB), walking the blocks
 * grid-stride; wgs workgroups (wgs <= 0: 8 per compute unit).  src and dst:
 * device buffers, 16-byte aligned.  Errors: MOE_EINVAL (unknown kind, NULL
 * or misaligned pointer, negative size).
 */
int moe_bandwidth_probe(int kind, const void* src, void* dst, int64_t bytes, int wgs, void* stream);

/*
 * Stage timing (profiling aid; the per-stage attribution of layer time).
 * moe_profile_begin(max_calls) makes the next max_calls calls of
 * moe_ffn_forward / moe_ffn_backward record HIP events on their own stream
 * at every stage boundary; moe_profile_end waits for the last event and
 * writes, for each stage s < n_stages, the milliseconds summed over the
 * recorded calls (stage_ms[s]) and the number of recorded calls of each kind
 * (n_calls[0] forward, n_calls[1] backward).  Stages:
 *   0 routed gate_up + SwiGLU GEMM   1 routed down GEMM
 *   2 shared gate_up + SwiGLU GEMM   3 shared down GEMM    4 combine
 *   5 combine backward   6 routed dh GEMM + SwiGLU backward
 *   7 routed down weight gradient    8 routed gate_up weight gradient
 *   9 routed dx GEMM    10 shared expert backward   11 router backward
 *  12 dx sum
 * Process-wide state, not thread-safe; returns MOE_EINVAL on bad arguments
 * and MOE_ELAUNCH if a HIP event call fails.
 */
#define MOE_N_STAGES 13
int moe_profile_begin(int max_calls);
int moe_profile_end(float* stage_ms, int n_stages, int* n_calls);

/* Device workspace bytes needed by op (MOE_OP_*) for this shape; 0 when the
 * shape is invalid. */
size_t moe_workspace_bytes(const moe_shape* shape, int op);

/* Static description of a status code. */
const char* moe_status_str(int status);

#ifdef __cplusplus
}
#endif
#endif /* MOE_MI355X_H */
