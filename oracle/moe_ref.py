"""Plain, slow CPU oracle of the sparse MoE FFN layer (NumPy, float64).

TEST INFRASTRUCTURE: only tests, the smoke check and the bench's CPU-baseline
leg may import this package.  It shares no code with the HIP path.

What it computes is the plain definition of the layer: the dense-masked MoE,
where every expert runs on every token and the routing mask picks the
outputs ("feat: Phase 43 — Sparse/Grouped MoE Dispatch", Summary and the
DispatchKind::DenseMasked reference: the sparse path is numerically the
dense-masked result with the masked-away matmuls skipped).  The per-expert
loop ("mstar.model.components.moe", dispatch_experts_fused) is kept beside it
as a cross-check, and is what the large-shape tests call on sampled tokens.

Two readings of a bf16 layer are available.  By default nothing is rounded:
the exact float64 result of the definition.  With bf16=True the oracle is
the operand-rounding model of a layer computed "in bf16 with fp32
accumulation": every matrix-product operand the layer holds as a bf16 tensor
(the expert activation h in the forward; the weighted output gradient
w * dout and the SwiGLU gradient dg | du in the backward; the same for the
shared expert) is rounded to bf16 once, from its exact value, and nothing
else is rounded.

Conventions (all arrays row-major):
  x [T,H]; w_router [E,H]; w_gate_up [E,2I,H] (rows [0,I) gate, [I,2I) up);
  w_down [E,H,I]; ws_gate_up [2Is,H]; ws_down [H,Is]; w_shared_gate [H];
  sel_bias [E] fp32; ids [T,k] int64; weights [T,k].
Inputs arrive already rounded to their storage dtype (bf16 or fp32) and are
upcast to float64 here.
"""
from __future__ import annotations

import itertools
from typing import Dict, Optional, Tuple

import numpy as np

from . import score_f32

SOFTMAX, SIGMOID, SQRTSOFTPLUS = 0, 1, 2


# ----------------------------------------------------------------------------
# Router ("mstar.model.components.moe", Router contract and TopKRouter;
# "Sparse MoE FFN for DFlash-family drafters", What's here: MoEGate)
# ----------------------------------------------------------------------------

def router_logits(x: np.ndarray, w_router: np.ndarray) -> np.ndarray:
    """logits[t,e] = sum_h x[t,h] w_router[e,h], float64 (TopKRouter's gate
    projection; the layer keeps them as fp32)."""
    return np.asarray(x, np.float64) @ np.asarray(w_router, np.float64).T


def scores_f64(logits: np.ndarray, score: int) -> np.ndarray:
    """Router scores in float64.  softmax over all E (TopKRouter: softmax
    top-k router), sigmoid, or sqrtsoftplus = sqrt(log(1+e^l)) (MoEGate)."""
    l = np.asarray(logits, np.float64)
    if score == SOFTMAX:
        z = np.exp(l - l.max(axis=-1, keepdims=True))
        return z / z.sum(axis=-1, keepdims=True)
    if score == SIGMOID:
        return 1.0 / (1.0 + np.exp(-l))
    if score == SQRTSOFTPLUS:
        return np.sqrt(np.maximum(l, 0.0) + np.log1p(np.exp(-np.abs(l))))
    raise ValueError(score)


def selection_keys(logits32: np.ndarray, score: int,
                   sel_bias: Optional[np.ndarray]) -> np.ndarray:
    """The fp32 values the top-k compares.

    Without a bias every score function is strictly increasing in the logit,
    so the top-k by score is the top-k by logit: the key is the fp32 logit.
    With the aux-loss-free bias (used for selection only) the key is
    fl32(score32(logit) + bias) with the fixed fp32 recipe of score_f32."""
    l32 = np.asarray(logits32, np.float32)
    if sel_bias is None:
        key = l32.copy()
    else:
        s32 = score_f32.scores32(l32, score)
        key = (s32 + np.asarray(sel_bias, np.float32)[None, :]).astype(np.float32)
    key[key == 0] = np.float32(0.0)   # -0.0 and +0.0 are the same key
    return key


def topk_select(keys: np.ndarray, k: int) -> np.ndarray:
    """ids[t, 0..k-1]: the k largest keys of each row in descending order;
    equal keys go to the lower expert index first."""
    keys = np.asarray(keys)
    order = np.argsort(-keys.astype(np.float64), axis=-1, kind="stable")
    return order[:, :k].astype(np.int64)


def topk_bruteforce(keys: np.ndarray, k: int) -> np.ndarray:
    """Same selection by exhaustive search over all C(E,k) subsets: the winner
    is the subset whose keys, listed in (key desc, index asc) order, are
    lexicographically largest, compared element by element as
    (key, -index)."""
    T, E = keys.shape
    out = np.zeros((T, k), np.int64)
    for t in range(T):
        best = None
        best_ids = None
        for sub in itertools.combinations(range(E), k):
            ranked = sorted(sub, key=lambda e: (-float(keys[t, e]), e))
            vec = [(float(keys[t, e]), -e) for e in ranked]
            if best is None or vec > best:
                best, best_ids = vec, ranked
        out[t] = best_ids
    return out


def routing_weights(scores: np.ndarray, ids: np.ndarray, renorm: bool) -> np.ndarray:
    """Selected unbiased scores; with norm_topk_prob each token's k selected
    scores are divided by their own total, so its weights add up to one
    ("mstar.model.components.moe", TopKRouter, the norm_topk_prob parameter).
    The bias never enters the weights."""
    w = np.take_along_axis(np.asarray(scores, np.float64), ids, axis=-1)
    if renorm:
        s = w.sum(axis=-1, keepdims=True)
        w = np.where(s > 0, w / np.where(s > 0, s, 1.0), 0.0)
    return w


def route(logits32: np.ndarray, k: int, score: int, renorm: bool,
          sel_bias: Optional[np.ndarray] = None) -> Tuple[np.ndarray, np.ndarray]:
    """Router contract: (tokens, hidden) in -> routing weights (tokens, k)
    and int64 expert ids (tokens, k).  Selection from fp32 logits, weights
    from float64 scores of those logits."""
    keys = selection_keys(logits32, score, sel_bias)
    ids = topk_select(keys, k)
    s = scores_f64(np.asarray(logits32, np.float64), score)
    return routing_weights(s, ids, renorm), ids


# ----------------------------------------------------------------------------
# bf16 operands.  A bf16 layer computes "in bf16 with fp32 accumulation": every
# GEMM operand is a bf16 tensor.  The expert activation h = silu(g)*u is the
# operand of the down projection, so in a bf16 layer it is rounded to bf16
# (round to nearest, ties to even) once, from its exact value.
# ----------------------------------------------------------------------------

def round_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (8 significant bits),
    ties to even, directly from float64 (a single rounding).  Normal range
    only; zeros, infinities and NaN pass through."""
    a = np.asarray(a, np.float64)
    m, e = np.frexp(a)                      # a = m * 2^e, 0.5 <= |m| < 1
    r = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    return np.where(np.isfinite(a) & (a != 0), r, a)


# ----------------------------------------------------------------------------
# Experts: SwiGLU over the fused layout ("mstar.model.components.moe",
# SparseMoeBlock: gate_up_proj (E, 2I, H), down_proj (E, H, I);
# dispatch_experts_fused runs SwiGLU per expert)
# ----------------------------------------------------------------------------

def silu(z):
    return z / (1.0 + np.exp(-z))


def swiglu_mlp(x: np.ndarray, w_gate_up: np.ndarray, w_down: np.ndarray, bf16: bool = False) -> np.ndarray:
    """down · (silu(gate · x) * (up · x)); gate = rows [0,I) of w_gate_up,
    up = rows [I,2I).  bf16=True: the down projection's operand h is a bf16
    tensor (rounded once)."""
    x = np.asarray(x, np.float64)
    wgu = np.asarray(w_gate_up, np.float64)
    I = wgu.shape[0] // 2
    g = x @ wgu[:I].T
    u = x @ wgu[I:].T
    h = silu(g) * u
    if bf16:
        h = round_bf16(h)
    return h @ np.asarray(w_down, np.float64).T


def routing_mask(ids: np.ndarray, weights: np.ndarray, E: int) -> np.ndarray:
    """M[t,e] = weight of e for token t if selected, else 0."""
    T, k = ids.shape
    M = np.zeros((T, E), np.float64)
    for j in range(k):
        M[np.arange(T), ids[:, j]] += weights[:, j]
    return M


def shared_gate(x: np.ndarray, w_shared_gate: Optional[np.ndarray]) -> np.ndarray:
    """sigmoid(shared_gate(x)) per token, or 1 for an ungated shared expert
    ("mstar.model.components.moe", SparseMoeBlockWithSharedExpert)."""
    if w_shared_gate is None:
        return np.ones(np.asarray(x).shape[0])
    z = np.asarray(x, np.float64) @ np.asarray(w_shared_gate, np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def shared_term(x, ws_gate_up, ws_down, w_shared_gate, bf16: bool = False):
    if ws_gate_up is None:
        return np.zeros(np.asarray(x).shape, np.float64)
    return shared_gate(x, w_shared_gate)[:, None] * swiglu_mlp(x, ws_gate_up, ws_down, bf16)


def dense_masked_forward(x, ids, weights, w_gate_up, w_down, ws_gate_up=None,
                         ws_down=None, w_shared_gate=None, bf16: bool = False) -> np.ndarray:
    """out[t] = sum_e M[t,e] y_e(x_t) + g_t S(x_t): every expert on every
    token, masked by the routing ("feat: Phase 43", DenseMasked reference;
    shared term per SparseMoeBlockWithSharedExpert's stated output)."""
    x = np.asarray(x, np.float64)
    E = np.asarray(w_gate_up).shape[0]
    M = routing_mask(ids, weights, E)
    out = np.zeros(x.shape, np.float64)
    for e in range(E):
        out += M[:, e:e + 1] * swiglu_mlp(x, w_gate_up[e], w_down[e], bf16)
    return out + shared_term(x, ws_gate_up, ws_down, w_shared_gate, bf16)


def per_expert_loop_forward(x, ids, weights, w_gate_up, w_down, ws_gate_up=None,
                            ws_down=None, w_shared_gate=None, bf16: bool = False) -> np.ndarray:
    """Loop over the experts that received tokens and run SwiGLU on exactly
    those rows ("mstar.model.components.moe", dispatch_experts_fused;
    "feat: Phase 43", index_select -> expert -> index_add)."""
    x = np.asarray(x, np.float64)
    T, k = ids.shape
    out = np.zeros(x.shape, np.float64)
    for e in np.unique(ids):
        t_idx, j_idx = np.nonzero(ids == e)
        y = swiglu_mlp(x[t_idx], w_gate_up[e], w_down[e], bf16)
        np.add.at(out, t_idx, weights[t_idx, j_idx][:, None] * y)
    return out + shared_term(x, ws_gate_up, ws_down, w_shared_gate, bf16)


# ----------------------------------------------------------------------------
# Sorted-segment dispatch ("Sparse MoE FFN for DFlash-family drafters",
# What's here, SparseMoE: one argsort -> contiguous per-expert segments;
# "feat: Phase 43", sparse_grouped_dispatch: arg_sort permutation)
# ----------------------------------------------------------------------------

# ----------------------------------------------------------------------------
# Parallel dense + MoE block (the DeepSpec issue "Feat: Compatible with Gamme4 MoE structure":
# Decoder layer forward pass).  The dense MLP and the MoE branch run side by side: the router reads
# the residual stream, the experts read its RMS-normalised copy, each branch's output is normalised,
# the sum normalised again, added to the residual and scaled by the layer scalar.
# ----------------------------------------------------------------------------

def rms_norm(v: np.ndarray, g: np.ndarray, eps: float) -> np.ndarray:
    """v / sqrt(mean(v^2 over the hidden axis) + eps) * g, float64.  g is the
    per-channel scale as applied (a checkpoint that stores w with an implied
    1 + w passes g = 1 + w)."""
    v = np.asarray(v, np.float64)
    ms = np.mean(v * v, axis=-1, keepdims=True)
    return v / np.sqrt(ms + eps) * np.asarray(g, np.float64)[None, :]


def parallel_block_forward(residual, x_dense, ids, weights, w_gate_up, w_down, wd_gate_up, wd_down,
                           g_pre_moe, g_post_dense, g_post_moe, g_post, eps: float, layer_scalar: float,
                           bf16: bool = False) -> np.ndarray:
    """out = (residual + N_post(N_post_dense(MLP(x_dense)) + N_post_moe(MoE(N_pre_moe(residual)))))
    * layer_scalar, with the MoE routed by (ids, weights) from the residual.
    x_dense is the dense branch's input as the caller gives it.  bf16=True:
    the experts' input N_pre_moe(residual) is a bf16 tensor (rounded once)
    and the MLPs round h as in the rest of the layer."""
    r = np.asarray(residual, np.float64)
    x_moe = rms_norm(r, g_pre_moe, eps)
    if bf16:
        x_moe = round_bf16(x_moe)
    h1 = swiglu_mlp(x_dense, wd_gate_up, wd_down, bf16)
    h2 = dense_masked_forward(x_moe, ids, weights, w_gate_up, w_down, bf16=bf16)
    h = rms_norm(h1, g_post_dense, eps) + rms_norm(h2, g_post_moe, eps)
    return (r + rms_norm(h, g_post, eps)) * float(layer_scalar)


def dispatch(ids: np.ndarray, E: int) -> Dict[str, np.ndarray]:
    """counts[e]; offsets = exclusive prefix of counts (offsets[E] = T*k);
    perm = stable argsort of the flattened ids (flat index t*k + j), so
    segment e holds its (t,j) pairs in increasing flat index; pos = the
    inverse permutation (pos[t*k+j] = row of that pair in sorted order)."""
    flat = np.asarray(ids, np.int64).ravel()
    counts = np.bincount(flat, minlength=E).astype(np.int64)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int64)
    perm = np.argsort(flat, kind="stable").astype(np.int64)
    pos = np.empty_like(perm)
    pos[perm] = np.arange(perm.size)
    return {"counts": counts, "offsets": offsets, "perm": perm, "pos": pos}


# ----------------------------------------------------------------------------
# Aux-loss-free balance ("Sparse MoE FFN for DFlash-family drafters",
# What's here, MoEGate and the deferred balance updates): an fp32 per-expert
# bias that only the expert loads move, by the sign of their distance from
# the mean load, and that no gradient reaches; the loads of one training
# forward are kept aside and folded into the bias when the next forward
# starts.
# ----------------------------------------------------------------------------

def balance_update(bias: np.ndarray, counts: np.ndarray, rate: float,
                   tokens_times_k: int) -> np.ndarray:
    """b <- b + rate * sign(mean_load - load_e), mean_load = T*k/E, sign(0)=0,
    in fp32.  Under-loaded experts move up, over-loaded experts move down."""
    E = counts.shape[0]
    mean = np.float64(tokens_times_k) / E
    step = np.sign(mean - np.asarray(counts, np.float64)).astype(np.float32)
    return (np.asarray(bias, np.float32) + np.float32(rate) * step).astype(np.float32)


class BalanceState:
    """Deferred apply: a training forward stashes its counts, the next
    forward applies them before routing and clears the stash; an eval
    forward stashes nothing; applying with nothing stashed is a no-op."""

    def __init__(self, bias: np.ndarray, rate: float):
        self.bias = np.asarray(bias, np.float32).copy()
        self.rate = float(rate)
        self.pending: Optional[Tuple[np.ndarray, int]] = None

    def apply_pending(self) -> bool:
        if self.pending is None:
            return False
        counts, tk = self.pending
        self.bias = balance_update(self.bias, counts, self.rate, tk)
        self.pending = None
        return True

    def after_forward(self, counts: np.ndarray, tokens_times_k: int, training: bool):
        if training:
            self.pending = (np.asarray(counts).copy(), int(tokens_times_k))


def aux_loss(scores: np.ndarray, ids: np.ndarray, E: int, alpha: float = 1.0) -> float:
    """Switch-style load-balancing loss alpha * E * sum_e f_e P_e with f_e the
    share of (token, slot) pairs routed to e and P_e the mean score of e over
    the tokens.  It reads only router outputs, computed before dispatch
    ("feat: Phase 43", load balancing auxiliary loss computed in top_k_gating
    before dispatch).  The pages give no formula: this is the plainest
    standard reading, with the coefficient alpha = 1 unless stated."""
    Tk = ids.size
    f = np.bincount(np.asarray(ids).ravel(), minlength=E) / Tk
    P = np.asarray(scores, np.float64).mean(axis=0)
    return float(alpha * E * np.sum(f * P))


def aux_dscores(ids: np.ndarray, T: int, E: int, alpha: float = 1.0) -> np.ndarray:
    """Gradient of aux_loss with respect to every score s[t,e].  The loads f
    come from the discrete selection and carry no gradient, and P_e is a plain
    mean over the T tokens, so d aux / d s[t,e] = alpha * E * f_e / T for
    every token t: one coefficient per expert, [E]."""
    f = np.bincount(np.asarray(ids).ravel(), minlength=E) / np.asarray(ids).size
    return alpha * E * f / T


# ----------------------------------------------------------------------------
# Backward, analytic in float64 ("feat: Phase 43", sparse dispatch backward
# reaches router logits, expert parameters and input activations;
# "Sparse MoE FFN for DFlash-family drafters", Tests: parity of grads).
# The bias and the permutation carry no gradient.
# ----------------------------------------------------------------------------

def _mlp_parts(x, wgu, wd, bf16=False):
    """g, u, sigmoid(g), h, y; in a bf16 layer h is a bf16 tensor."""
    I = wgu.shape[0] // 2
    g = x @ wgu[:I].T
    u = x @ wgu[I:].T
    sg = 1.0 / (1.0 + np.exp(-g))
    h = g * sg * u
    if bf16:
        h = round_bf16(h)
    return g, u, sg, h, h @ wd.T


def _swiglu_grad(x, wgu, wd, dy, bf16=False):
    """h (bf16 in a bf16 layer) and the SwiGLU gradient (dg | du) before any
    rounding: dh = dy wd, dg = dh u silu'(g), du = dh silu(g)."""
    g, u, sg, h, _ = _mlp_parts(x, wgu, wd, bf16)
    dh = dy @ wd
    dsilu = sg * (1.0 + g * (1.0 - sg))
    return h, np.concatenate([dh * u * dsilu, dh * g * sg], axis=1)


def _mlp_backward(x, wgu, wd, dy, bf16=False):
    """Gradients of y = wd (silu(g) u), g = wg x, u = wu x, given dy.  In a
    bf16 layer the operands of the gradient GEMMs are bf16 tensors: dy (the
    caller rounds it), h, and (dg | du)."""
    h, dgu = _swiglu_grad(x, wgu, wd, dy, bf16)
    if bf16:
        dgu = round_bf16(dgu)
    return {"dx": dgu @ wgu, "dw_gate_up": dgu.T @ x, "dw_down": dy.T @ h}


def mlp_operands_before_rounding(x, wgu, wd, dy):
    """The values the operand-rounding model of a bf16 layer rounds, for one
    expert's rows: dy (the weighted output gradient w * dout, as given), h
    and (dg | du), the last formed from the rounded dy as in the model.  For
    a check's tolerance (which roundings are near a tie), not a result."""
    h = _mlp_parts(x, wgu, wd, False)[3]
    _, dgu = _swiglu_grad(x, wgu, wd, round_bf16(dy), True)
    return {"dy": np.asarray(dy, np.float64), "h": h, "dgu": dgu}


def score_backward(logits: np.ndarray, score: int, dscores: np.ndarray) -> np.ndarray:
    """dlogits from dscores for each score function (softmax couples all E)."""
    l = np.asarray(logits, np.float64)
    s = scores_f64(l, score)
    if score == SOFTMAX:
        return s * (dscores - np.sum(s * dscores, axis=-1, keepdims=True))
    if score == SIGMOID:
        return dscores * s * (1.0 - s)
    if score == SQRTSOFTPLUS:
        return dscores * (1.0 / (1.0 + np.exp(-l))) / (2.0 * s)
    raise ValueError(score)


def layer_backward(x, w_router, ids, logits, score, renorm, w_gate_up, w_down,
                   dout, ws_gate_up=None, ws_down=None, w_shared_gate=None,
                   loop: bool = False, bf16: bool = False,
                   aux_alpha: float = 0.0) -> Dict[str, np.ndarray]:
    """Gradients of the full layer output w.r.t. x, w_router, the stacked
    expert weights and the shared expert, for a fixed selection ids.
    loop=False: dense-masked (every expert on every token, masked);
    loop=True: the per-expert loop over selected rows only.
    bf16=True: a bf16 layer, whose matrix-product operands are bf16 tensors:
    h (forward), the weighted output gradient dy = w * dout, the SwiGLU
    gradient (dg | du), and the same three for the shared expert.
    aux_alpha != 0: the gradient of sum(out * dout) + aux_loss(scores, ids,
    E, aux_alpha), i.e. aux_dscores added to every token's score gradient."""
    rb = round_bf16 if bf16 else (lambda a: a)
    x = np.asarray(x, np.float64)
    dout = np.asarray(dout, np.float64)
    T, H = x.shape
    E = w_gate_up.shape[0]
    k = ids.shape[1]
    s = scores_f64(logits, score)
    w = routing_weights(s, ids, renorm)
    dw = np.zeros((T, k))
    dx = np.zeros_like(x)
    dWgu = np.zeros(w_gate_up.shape)
    dWd = np.zeros(w_down.shape)
    for e in range(E):
        wgu = np.asarray(w_gate_up[e], np.float64)
        wd = np.asarray(w_down[e], np.float64)
        if loop:
            t_idx, j_idx = np.nonzero(ids == e)
            if t_idx.size == 0:
                continue
            xe = x[t_idx]
            ye = _mlp_parts(xe, wgu, wd, bf16)[4]
            dw[t_idx, j_idx] = np.sum(dout[t_idx] * ye, axis=1)
            gr = _mlp_backward(xe, wgu, wd, rb(w[t_idx, j_idx][:, None] * dout[t_idx]), bf16)
            np.add.at(dx, t_idx, gr["dx"])
        else:
            M = np.zeros(T)
            sel = np.zeros(T, bool)
            for j in range(k):
                hit = ids[:, j] == e
                M[hit] += w[hit, j]
                sel |= hit
            ye = _mlp_parts(x, wgu, wd, bf16)[4]
            for j in range(k):
                hit = ids[:, j] == e
                dw[hit, j] = np.sum(dout[hit] * ye[hit], axis=1)
            gr = _mlp_backward(x, wgu, wd, rb(M[:, None] * dout), bf16)
            dx += gr["dx"]
        dWgu[e] = gr["dw_gate_up"]
        dWd[e] = gr["dw_down"]
    # routing weights -> selected scores (renorm) -> all scores -> logits
    s_sel = np.take_along_axis(s, ids, axis=-1)
    if renorm:
        den = s_sel.sum(axis=-1, keepdims=True)
        ds_sel = (dw - np.sum(w * dw, axis=-1, keepdims=True)) / den
    else:
        ds_sel = dw
    dscores = np.zeros((T, E))
    for j in range(k):
        dscores[np.arange(T), ids[:, j]] += ds_sel[:, j]
    if aux_alpha != 0.0:
        dscores += aux_dscores(ids, T, E, aux_alpha)[None, :]
    dlogits = score_backward(logits, score, dscores)
    wr = np.asarray(w_router, np.float64)
    dx += dlogits @ wr
    out = {"dx": dx, "dw_router": dlogits.T @ x, "dw_gate_up": dWgu,
           "dw_down": dWd, "dlogits": dlogits, "dweights": dw}
    if ws_gate_up is not None:
        wsgu = np.asarray(ws_gate_up, np.float64)
        wsd = np.asarray(ws_down, np.float64)
        S = _mlp_parts(x, wsgu, wsd, bf16)[4]
        gsh = shared_gate(x, w_shared_gate)
        gr = _mlp_backward(x, wsgu, wsd, rb(gsh[:, None] * dout), bf16)
        dx += gr["dx"]
        out["dws_gate_up"] = gr["dw_gate_up"]
        out["dws_down"] = gr["dw_down"]
        if w_shared_gate is not None:
            dz = np.sum(dout * S, axis=1) * gsh * (1.0 - gsh)
            out["dw_shared_gate"] = dz @ x
            dx += dz[:, None] * np.asarray(w_shared_gate, np.float64)[None, :]
    return out


def layer_forward(x, w_router, k, score, renorm, w_gate_up, w_down, ws_gate_up=None,
                  ws_down=None, w_shared_gate=None, sel_bias=None, ids=None,
                  loop: bool = False) -> Dict[str, np.ndarray]:
    """Whole layer: route from fp32 logits, then dense-masked (or loop)
    experts plus the shared term.  ``ids`` may be given to fix the
    selection (used for finite differences)."""
    logits = router_logits(x, w_router)
    logits32 = logits.astype(np.float32)
    if ids is None:
        weights, ids = route(logits32, k, score, renorm, sel_bias)
    s = scores_f64(logits, score)
    weights = routing_weights(s, ids, renorm)
    fwd = per_expert_loop_forward if loop else dense_masked_forward
    out = fwd(x, ids, weights, w_gate_up, w_down, ws_gate_up, ws_down, w_shared_gate)
    return {"out": out, "logits": logits, "ids": ids, "weights": weights}
