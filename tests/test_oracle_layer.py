"""Pins for the oracle's expert path, shared expert, balance and backward
(CPU only).

Pins: the per-expert loop equals the dense-masked definition; E=1, k=1
reduces to a textbook SwiGLU MLP computed with torch's own silu; identical
experts give (sum of weights) * MLP; the shared term sums separately; empty
experts are skipped; the aux loss is a function of router outputs only,
its score gradient is the derivative of its value;
balance semantics; central finite differences of the analytic backward.
Planted mistakes (gate/up swapped, shared gate dropped) must fail.
"""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from workloads import WORKLOADS, make_inputs, exact_dyadic_inputs


def _np(t):
    return t.detach().to(torch.float64).cpu().numpy()


def _tiny(seed=0, Is=0, gated=False, T=64, H=32, E=8, I=24):
    rng = np.random.default_rng(seed)
    d = {"x": rng.normal(0, 1, (T, H)),
         "w_router": rng.normal(0, H ** -0.5, (E, H)),
         "w_gate_up": rng.normal(0, H ** -0.5, (E, 2 * I, H)),
         "w_down": rng.normal(0, I ** -0.5, (E, H, I))}
    if Is:
        d["ws_gate_up"] = rng.normal(0, H ** -0.5, (2 * Is, H))
        d["ws_down"] = rng.normal(0, Is ** -0.5, (H, Is))
        if gated:
            d["w_shared_gate"] = rng.normal(0, H ** -0.5, (H,))
    return d


def _shared_args(d):
    return d.get("ws_gate_up"), d.get("ws_down"), d.get("w_shared_gate")


@pytest.mark.parametrize("score,renorm,k", [(0, True, 2), (0, False, 4), (1, True, 3), (2, True, 6)])
def test_loop_equals_dense_masked(score, renorm, k):
    d = _tiny(seed=score + k, Is=16, gated=True)
    l32 = R.router_logits(d["x"], d["w_router"]).astype(np.float32)
    w, ids = R.route(l32, k, score, renorm)
    a = R.dense_masked_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"], *_shared_args(d))
    b = R.per_expert_loop_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"], *_shared_args(d))
    assert np.max(np.abs(a - b)) < 1e-12


def test_tiny_workload_loop_equals_dense_masked():
    wl = WORKLOADS["tiny_fp32"]
    inp = {k: _np(v) for k, v in make_inputs(wl).items()}
    l32 = R.router_logits(inp["x"], inp["w_router"]).astype(np.float32)
    w, ids = R.route(l32, wl.k, wl.score, wl.renorm)
    a = R.dense_masked_forward(inp["x"], ids, w, inp["w_gate_up"], inp["w_down"])
    b = R.per_expert_loop_forward(inp["x"], ids, w, inp["w_gate_up"], inp["w_down"])
    assert np.max(np.abs(a - b)) < 1e-12


def test_single_expert_is_textbook_swiglu():
    """E=1, k=1, renorm: the layer is a dense SwiGLU MLP; compare with
    torch.nn.functional.silu in float64."""
    d = _tiny(seed=3, E=1)
    out = R.layer_forward(d["x"], d["w_router"], 1, 0, True, d["w_gate_up"], d["w_down"])["out"]
    x = torch.tensor(d["x"])
    wgu = torch.tensor(d["w_gate_up"][0])
    wd = torch.tensor(d["w_down"][0])
    I = wgu.shape[0] // 2
    ref = (torch.nn.functional.silu(x @ wgu[:I].T) * (x @ wgu[I:].T)) @ wd.T
    assert np.max(np.abs(out - ref.numpy())) < 1e-12


def test_gate_up_swap_is_caught():
    d = _tiny(seed=4, E=1)
    wgu = d["w_gate_up"].copy()
    I = wgu.shape[1] // 2
    swapped = np.concatenate([wgu[:, I:], wgu[:, :I]], axis=1)   # planted mistake
    good = R.swiglu_mlp(d["x"], wgu[0], d["w_down"][0])
    bad = R.swiglu_mlp(d["x"], swapped[0], d["w_down"][0])
    x = torch.tensor(d["x"])
    ref = ((torch.nn.functional.silu(x @ torch.tensor(wgu[0, :I]).T) * (x @ torch.tensor(wgu[0, I:]).T))
           @ torch.tensor(d["w_down"][0]).T).numpy()
    assert np.max(np.abs(good - ref)) < 1e-12 and np.max(np.abs(bad - ref)) > 1e-3


def test_identical_experts_invariant():
    d = _tiny(seed=5)
    d["w_gate_up"][:] = d["w_gate_up"][0]
    d["w_down"][:] = d["w_down"][0]
    l32 = R.router_logits(d["x"], d["w_router"]).astype(np.float32)
    for renorm in (True, False):
        w, ids = R.route(l32, 3, 0, renorm)
        out = R.dense_masked_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"])
        mlp = R.swiglu_mlp(d["x"], d["w_gate_up"][0], d["w_down"][0])
        assert np.max(np.abs(out - w.sum(-1, keepdims=True) * mlp)) < 1e-12


@pytest.mark.parametrize("gated", [False, True])
def test_shared_expert_sums_separately(gated):
    d = _tiny(seed=6, Is=40, gated=gated)
    l32 = R.router_logits(d["x"], d["w_router"]).astype(np.float32)
    w, ids = R.route(l32, 2, 0, False)
    with_s = R.dense_masked_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"], *_shared_args(d))
    without = R.dense_masked_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"])
    S = R.swiglu_mlp(d["x"], d["ws_gate_up"], d["ws_down"])
    g = R.shared_gate(d["x"], d.get("w_shared_gate"))
    if gated:
        # the gate is interior: no sigmoid saturates to exactly 0 or 1 in fp32
        g32 = g.astype(np.float32)
        assert np.all((g32 > 0) & (g32 < 1))
        ref_gate = 1.0 / (1.0 + np.exp(-(d["x"] @ d["w_shared_gate"])))
        assert np.max(np.abs(g - ref_gate)) < 1e-15
        # planted mistake: dropping the gate multiply must fail this pin
        assert np.max(np.abs((with_s - without) - S)) > 1e-3
    assert np.max(np.abs((with_s - without) - g[:, None] * S)) < 1e-12


def test_workload_gates_do_not_saturate():
    wl = WORKLOADS["qwen2moe"]
    inp = make_inputs(wl, T=256)
    z = _np(inp["x"]) @ _np(inp["w_shared_gate"])
    g = (1.0 / (1.0 + np.exp(-z))).astype(np.float32)
    assert np.all((g > 0) & (g < 1))


def test_empty_expert_is_skipped():
    d = _tiny(seed=8)
    l32 = R.router_logits(d["x"], d["w_router"]).astype(np.float32)
    l32[:, 5] = -50.0                      # expert 5 never chosen
    w, ids = R.route(l32, 2, 0, True)
    assert not np.any(ids == 5)
    ref = R.per_expert_loop_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"])
    d["w_gate_up"][5] = np.nan
    d["w_down"][5] = np.nan
    out = R.per_expert_loop_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"])
    assert np.all(np.isfinite(out)) and np.array_equal(out, ref)
    gr = R.layer_backward(d["x"], d["w_router"], ids, l32.astype(np.float64), 0, True,
                          d["w_gate_up"], d["w_down"], np.ones_like(d["x"]), loop=True)
    assert np.all(gr["dw_gate_up"][5] == 0) and np.all(gr["dw_down"][5] == 0)


def test_aux_loss_closed_form_and_dispatch_independence():
    E, T, k = 8, 64, 2
    # uniform scores and perfectly balanced loads: E * sum (1/E)(1/E) = 1
    ids = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)])
    s = np.full((T, E), 1.0 / E)
    assert abs(R.aux_loss(s, ids, E) - 1.0) < 1e-15
    # all load on one expert with score 1 there: E * 1 * 1 = E
    s1 = np.zeros((T, E))
    s1[:, 0] = 1.0
    assert abs(R.aux_loss(s1, np.zeros((T, 1), np.int64), E) - E) < 1e-12
    # the aux loss reads router outputs only: running either dispatch
    # leaves its inputs, hence its bits, unchanged
    d = _tiny(seed=9)
    l32 = R.router_logits(d["x"], d["w_router"]).astype(np.float32)
    w, ids = R.route(l32, 2, 0, True)
    sc = R.scores_f64(l32.astype(np.float64), 0)
    before = R.aux_loss(sc, ids, E)
    R.dense_masked_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"])
    a = R.aux_loss(sc, ids, E)
    R.per_expert_loop_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"])
    b = R.aux_loss(sc, ids, E)
    assert before == a == b


def test_aux_dscores_is_the_gradient_of_the_aux_value():
    """aux_loss is linear in the scores, so a one-sided difference of the
    value in each s[t,e] is its exact derivative (up to rounding); every
    token gets the same per-expert coefficient E * f_e / T."""
    rng = np.random.default_rng(4)
    T, E, k, alpha = 7, 5, 2, 0.3
    s = rng.uniform(0, 1, (T, E))
    ids = np.array([rng.choice(E, k, replace=False) for _ in range(T)])
    c = R.aux_dscores(ids, T, E, alpha)
    base = R.aux_loss(s, ids, E, alpha)
    for t in range(T):
        for e in range(E):
            s2 = s.copy()
            s2[t, e] += 0.5
            assert abs((R.aux_loss(s2, ids, E, alpha) - base) / 0.5 - c[e]) < 1e-13
    # loads counted by hand: expert e's share of the T*k pairs
    for e in range(E):
        share = sum(int(ids[t, j] == e) for t in range(T) for j in range(k)) / (T * k)
        assert abs(c[e] - alpha * E * share / T) < 1e-15


def test_aux_gradient_vanishes_for_softmax_at_balanced_load():
    """With every expert at the mean load the coefficient is the same for all
    e, and softmax scores sum to one, so the aux term has no logit gradient;
    sigmoid scores do not sum to a constant, so it does not vanish there."""
    T, E, k = 16, 8, 2
    ids = np.array([[(2 * t) % E, (2 * t + 1) % E] for t in range(T)])
    rng = np.random.default_rng(5)
    logits = rng.normal(0, 1, (T, E))
    c = np.broadcast_to(R.aux_dscores(ids, T, E, 1.0), (T, E))
    assert np.max(np.abs(R.score_backward(logits, 0, c))) < 1e-16
    assert np.max(np.abs(R.score_backward(logits, 1, c))) > 1e-3


@pytest.mark.parametrize("score,renorm", [(0, True), (1, False), (2, True)])
def test_aux_backward_finite_differences(score, renorm):
    """d/d(x, w_router) of sum(out * dout) + aux_loss(scores, ids, E, alpha)
    by central differences, selection held fixed."""
    d = _tiny(seed=20 + score, T=12, H=10, E=6, I=8)
    k, alpha = 2, 0.7
    logits = R.router_logits(d["x"], d["w_router"])
    ids = R.topk_select(R.selection_keys(logits.astype(np.float32), score, None), k)
    rng = np.random.default_rng(98)
    dout = rng.normal(0, 1, d["x"].shape)
    g = R.layer_backward(d["x"], d["w_router"], ids, logits, score, renorm, d["w_gate_up"],
                         d["w_down"], dout, aux_alpha=alpha)
    g0 = R.layer_backward(d["x"], d["w_router"], ids, logits, score, renorm, d["w_gate_up"],
                          d["w_down"], dout)
    assert np.max(np.abs(g["dlogits"] - g0["dlogits"])) > 1e-4   # the term is really there
    for key in ("dw_gate_up", "dw_down"):                          # and reaches nothing else
        assert np.array_equal(g[key], g0[key])

    def total(dd):
        lg = R.router_logits(dd["x"], dd["w_router"])
        return _loss(dd, ids, score, renorm, dout, False) + R.aux_loss(R.scores_f64(lg, score), ids, 6, alpha)
    h = 1e-6
    for pname, gname in (("x", "dx"), ("w_router", "dw_router")):
        flat = d[pname].reshape(-1)
        for idx in rng.choice(flat.size, size=12, replace=False):
            old = flat[idx]
            flat[idx] = old + h
            lp = total(d)
            flat[idx] = old - h
            lm = total(d)
            flat[idx] = old
            fd = (lp - lm) / (2 * h)
            an = g[gname].reshape(-1)[idx]
            assert abs(fd - an) < 1e-6 * max(1.0, abs(fd)), (pname, idx, fd, an)


def test_balance_semantics():
    E, T, k = 8, 16, 2
    bias = np.zeros(E, np.float32)
    counts = np.array([8, 4, 4, 4, 4, 4, 2, 2])   # mean 4
    nb = R.balance_update(bias, counts, 1e-3, T * k)
    assert nb.dtype == np.float32
    assert np.array_equal(np.sign(nb), [-1, 0, 0, 0, 0, 0, 1, 1])
    # equal loads leave the bias unchanged
    assert np.array_equal(R.balance_update(nb, np.full(E, 4), 1e-3, T * k), nb)
    st = R.BalanceState(bias, 1e-3)
    assert not st.apply_pending()                 # nothing stashed: no-op
    st.after_forward(counts, T * k, training=False)
    assert st.pending is None                     # eval does not stash
    st.after_forward(counts, T * k, training=True)
    assert st.apply_pending()
    b1 = st.bias.copy()
    assert not st.apply_pending()                 # second apply is a no-op
    assert np.array_equal(st.bias, b1) and np.array_equal(b1, nb)


def test_exact_dyadic_logits_are_exact_in_fp32():
    inp = exact_dyadic_inputs(32, 7168, 16, 8, seed=1)
    x = inp["x"].to(torch.float32)
    w = inp["w_router"].to(torch.float32)
    l64 = R.router_logits(_np(inp["x"]), _np(inp["w_router"]))
    # any fp32 summation order gives the exact value
    l32_fwd = (x @ w.T).numpy()
    l32_rev = (x.flip(1) @ w.flip(1).T).numpy()
    assert np.array_equal(l64.astype(np.float32).astype(np.float64), l64)
    assert np.array_equal(l32_fwd, l64.astype(np.float32))
    assert np.array_equal(l32_rev, l64.astype(np.float32))


# ----------------------------------------------------------------------------
# backward: central finite differences (float64), selection held fixed
# ----------------------------------------------------------------------------

def _loss(d, ids, score, renorm, dout, shared):
    logits = R.router_logits(d["x"], d["w_router"])
    s = R.scores_f64(logits, score)
    w = R.routing_weights(s, ids, renorm)
    out = R.dense_masked_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"],
                                 *(_shared_args(d) if shared else (None, None, None)))
    return float(np.sum(out * dout))


@pytest.mark.parametrize("score,renorm,shared", [(0, True, False), (0, False, True), (1, True, True),
                                                 (2, True, False), (2, False, True)])
def test_backward_finite_differences(score, renorm, shared):
    d = _tiny(seed=10 + score, Is=12 if shared else 0, gated=shared, T=12, H=10, E=6, I=8)
    k = 3
    logits = R.router_logits(d["x"], d["w_router"])
    ids = R.topk_select(R.selection_keys(logits.astype(np.float32), score, None), k)
    rng = np.random.default_rng(99)
    dout = rng.normal(0, 1, d["x"].shape)
    sa = _shared_args(d) if shared else (None, None, None)
    g = R.layer_backward(d["x"], d["w_router"], ids, logits, score, renorm, d["w_gate_up"],
                         d["w_down"], dout, *sa)
    g_loop = R.layer_backward(d["x"], d["w_router"], ids, logits, score, renorm, d["w_gate_up"],
                              d["w_down"], dout, *sa, loop=True)
    for key in g:
        assert np.max(np.abs(g[key] - g_loop[key])) < 1e-11, key
    names = [("x", "dx"), ("w_router", "dw_router"), ("w_gate_up", "dw_gate_up"), ("w_down", "dw_down")]
    if shared:
        names += [("ws_gate_up", "dws_gate_up"), ("ws_down", "dws_down"),
                  ("w_shared_gate", "dw_shared_gate")]
    h = 1e-6
    for pname, gname in names:
        p = d[pname]
        flat = p.reshape(-1)
        for idx in rng.choice(flat.size, size=min(12, flat.size), replace=False):
            old = flat[idx]
            flat[idx] = old + h
            lp = _loss(d, ids, score, renorm, dout, shared)
            flat[idx] = old - h
            lm = _loss(d, ids, score, renorm, dout, shared)
            flat[idx] = old
            fd = (lp - lm) / (2 * h)
            an = g[gname].reshape(-1)[idx]
            assert abs(fd - an) < 1e-6 * max(1.0, abs(fd)), (pname, idx, fd, an)


def test_round_bf16_matches_library_conversion():
    """The oracle's float64 -> bf16 rounding equals torch's fp32 -> bf16
    conversion on fp32-representable values, and rounds exact float64
    halfway cases to even."""
    rng = np.random.default_rng(21)
    a32 = np.concatenate([rng.normal(0, 3, 200000), rng.normal(0, 1e-3, 1000), [1.0, -2.5, 3.0e30]])
    a32 = a32.astype(np.float32)
    want = torch.tensor(a32).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(R.round_bf16(a32.astype(np.float64)), want)
    # halfway between 1 and 1 + 2^-7: ties to the even neighbour (1.0);
    # just above the halfway point rounds up
    assert R.round_bf16(1.0 + 2.0 ** -8) == 1.0
    assert R.round_bf16(1.0 + 3 * 2.0 ** -8) == 1.0 + 2.0 ** -6
    assert R.round_bf16(1.0 + 2.0 ** -8 + 2.0 ** -40) == 1.0 + 2.0 ** -7
    assert R.round_bf16(0.0) == 0.0 and np.isnan(R.round_bf16(np.nan))


def test_bf16_layer_rounds_only_the_down_operand():
    d = _tiny(seed=22, Is=16)
    l32 = R.router_logits(d["x"], d["w_router"]).astype(np.float32)
    w, ids = R.route(l32, 2, 0, True)
    a = R.dense_masked_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"], d["ws_gate_up"], d["ws_down"], bf16=True)
    b = R.per_expert_loop_forward(d["x"], ids, w, d["w_gate_up"], d["w_down"], d["ws_gate_up"], d["ws_down"],
                                  bf16=True)
    assert np.max(np.abs(a - b)) < 1e-12
    # written out by hand for one token and its first expert
    t, e = 3, ids[3, 0]
    I = d["w_gate_up"].shape[1] // 2
    g = d["w_gate_up"][e, :I] @ d["x"][t]
    u = d["w_gate_up"][e, I:] @ d["x"][t]
    h = torch.tensor(g / (1 + np.exp(-g)) * u, dtype=torch.float64)
    # single rounding float64 -> bf16 (via float32 with round-to-odd-free path:
    # values here are far from bf16 halfway points, so double rounding agrees)
    hb = h.to(torch.float32).to(torch.bfloat16).to(torch.float64).numpy()
    y = d["w_down"][e] @ hb
    assert np.max(np.abs(R.swiglu_mlp(d["x"][t:t + 1], d["w_gate_up"][e], d["w_down"][e], True)[0] - y)) < 1e-12


def test_bf16_backward_loop_equals_dense_and_hand_check():
    """bf16 mode of the backward: the loop and dense-masked forms agree, and
    one expert's weight gradient written out by hand matches."""
    d = _tiny(seed=23, Is=16, gated=True, T=20, H=16, E=5, I=8)
    k = 2
    logits = R.router_logits(d["x"], d["w_router"])
    ids = R.topk_select(R.selection_keys(logits.astype(np.float32), 0, None), k)
    dout = np.random.default_rng(5).normal(0, 1, d["x"].shape)
    sa = _shared_args(d)
    a = R.layer_backward(d["x"], d["w_router"], ids, logits, 0, True, d["w_gate_up"], d["w_down"], dout, *sa,
                         bf16=True)
    b = R.layer_backward(d["x"], d["w_router"], ids, logits, 0, True, d["w_gate_up"], d["w_down"], dout, *sa,
                         loop=True, bf16=True)
    for key in a:
        assert np.max(np.abs(a[key] - b[key])) < 1e-11, key
    # dw_down[e] = sum over routed rows of bf16(w * dout)^T bf16(h)
    e = int(ids[0, 0])
    w = R.routing_weights(R.scores_f64(logits, 0), ids, True)
    I = d["w_gate_up"].shape[1] // 2
    acc = np.zeros_like(d["w_down"][e])
    for t in range(d["x"].shape[0]):
        for j in range(k):
            if ids[t, j] != e:
                continue
            g = d["w_gate_up"][e, :I] @ d["x"][t]
            u = d["w_gate_up"][e, I:] @ d["x"][t]
            h = torch.tensor(g / (1 + np.exp(-g)) * u).to(torch.float32).to(torch.bfloat16).double().numpy()
            dy = torch.tensor(w[t, j] * dout[t]).to(torch.float32).to(torch.bfloat16).double().numpy()
            acc += np.outer(dy, h)
    assert np.max(np.abs(acc - a["dw_down"][e])) < 1e-12
    # the exact (non-bf16) mode differs: the reading is not vacuous
    ex = R.layer_backward(d["x"], d["w_router"], ids, logits, 0, True, d["w_gate_up"], d["w_down"], dout, *sa)
    assert np.max(np.abs(ex["dx"] - a["dx"])) > 1e-6


@pytest.mark.parametrize("gated", [False, True])
@pytest.mark.parametrize("bf16", [False, True])
def test_fused_n_shared_equals_sum_of_shared_experts(gated, bf16):
    """n_shared = 2 shared experts fused into one MLP of twice the width (the
    gate rows of both, then the up rows of both; the down columns side by
    side) give the sum of the two experts' outputs: each intermediate column
    is computed and rounded on its own, so only the summation order of the
    down projection differs ("Phase 43" shared-expert tests: n_shared fused
    width replays one MLP)."""
    rng = np.random.default_rng(12)
    T, H, Ie = 9, 16, 6
    x = rng.normal(0, 1, (T, H))
    g = [rng.normal(0, H ** -0.5, (Ie, H)) for _ in range(2)]
    u = [rng.normal(0, H ** -0.5, (Ie, H)) for _ in range(2)]
    d = [rng.normal(0, Ie ** -0.5, (H, Ie)) for _ in range(2)]
    wsg = rng.normal(0, H ** -0.5, (H,)) if gated else None
    fused = R.shared_term(x, np.concatenate(g + u), np.concatenate(d, axis=1), wsg, bf16=bf16)
    parts = sum(R.shared_term(x, np.concatenate([g[i], u[i]]), d[i], wsg, bf16=bf16) for i in range(2))
    assert np.max(np.abs(fused - parts)) < 1e-12
    # pairing a gate slice with the wrong up slice is caught
    wrong = R.shared_term(x, np.concatenate(g + u[::-1]), np.concatenate(d, axis=1), wsg, bf16=bf16)
    assert np.max(np.abs(wrong - parts)) > 1e-3
