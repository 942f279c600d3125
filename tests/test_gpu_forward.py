"""GPU parity of the full forward (route -> dispatch -> grouped SwiGLU GEMMs
-> combine + shared expert) against the float64 dense-masked oracle.

fp32 layer: max-abs <= 1e-5 against the exact oracle.  bf16 layer: max-abs
<= 2e-2 * RMS(reference) against the oracle's operand-rounding model (the
down projections' operand h is a bf16 tensor), with half a bf16 ulp allowed
only on elements where that alone exceeds the bound (gpu_helpers.gate_bf16);
the error against the exact oracle is logged beside it.  The oracle routes
from the GPU's fp32 logits after the ids were checked bit-exact.
"""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from workloads import WORKLOADS, Workload, exact_dyadic_inputs, make_inputs

from gpu_helpers import (assert_close, bf16_half_ulp, bf16_tol, gate_out_exact, make_layer, need_gpu, np64,
                         oracle_selection, report_exact, say)

pytestmark = pytest.mark.gpu

SMALL = [
    # name, T, H, E, k, I, Is, score, renorm, gated, bias
    ("softmax_renorm", 300, 256, 8, 2, 192, 0, 0, True, False, 0.0),
    ("softmax_shared_gated", 257, 320, 12, 3, 136, 320, 0, False, True, 0.0),
    ("sigmoid_shared", 129, 256, 16, 4, 256, 192, 1, True, False, 0.0),
    ("sqrtsoftplus_bias", 333, 384, 32, 6, 128, 128, 2, True, False, 0.5),
    ("e256_k8", 200, 256, 256, 8, 64, 64, 0, True, False, 0.0),
    # 40 tokens, shared intermediate 1024: the shared down projection splits K
    ("shared_splitk", 40, 256, 8, 2, 128, 1024, 1, True, True, 0.0),
    # 40 tokens, H 1024: the shared gate_up + SwiGLU splits K as well
    ("shared_splitk_gu", 40, 1024, 8, 2, 128, 512, 0, True, True, 0.0),
    # 300 tokens, Is 1024: the shared down projection runs on the 256x256
    # kernel with 4 tiles, split in two along K
    ("shared_q64_splitk", 300, 512, 8, 2, 128, 1024, 0, True, True, 0.0),
    # 256 tokens, small shared expert: its GEMMs stream with 64-row tiles
    ("shared_stream_bm64", 256, 256, 8, 2, 64, 256, 1, True, True, 0.0),
    # top-12 of 32: the combine's generic path for k > 8 (the forward only;
    # the backward takes k <= 8)
    ("k12", 60, 256, 32, 12, 64, 0, 0, True, False, 0.0),
]


def _wl(name, T, H, E, k, I, Is, score, renorm, gated, bias, dtype="bf16"):
    return Workload(name, T=T, H=H, E=E, k=k, I=I, Is=Is, score=score, renorm=renorm,
                    shared_gated=gated, bias_var=bias, dtype=dtype, seed=T + E)


def _run_and_check(w: Workload, inp, fuse_gather=False):
    layer = make_layer(w, inp, fuse_gather=fuse_gather)
    out = layer.forward(inp["x"], save=True)
    torch.cuda.synchronize()
    s = layer.last
    l32 = s["logits"].cpu().numpy()
    ids = s["ids"].cpu().numpy()
    assert np.array_equal(ids, oracle_selection(l32, w, inp.get("sel_bias")))
    wts = R.routing_weights(R.scores_f64(l32.astype(np.float64), w.score), ids, w.renorm)
    f = {k: np64(v) for k, v in inp.items() if k not in ("dout",)}
    args = (f["x"], ids, wts, f["w_gate_up"], f["w_down"], f.get("ws_gate_up"), f.get("ws_down"),
            f.get("w_shared_gate") if w.shared_gated else None)
    ref = R.dense_masked_forward(*args, bf16=w.dtype == "bf16")
    got = np64(out)
    assert_close(got, ref, w.dtype, w.name)
    if w.dtype == "bf16":
        report_exact(got, R.dense_masked_forward(*args), w.name)
    return layer, out, ref


def test_tiny_fp32_workload_full_parity():
    """The tiny fp32 layer (T64 H128 E8 top-2 I256, softmax renorm): every
    token against the dense-masked oracle at max-abs 1e-5."""
    need_gpu()
    w = WORKLOADS["tiny_fp32"]
    inp = make_inputs(w, device="cuda")
    _run_and_check(w, inp)


@pytest.mark.parametrize("case", SMALL, ids=[c[0] for c in SMALL])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_small_layers(case, dtype):
    need_gpu()
    w = _wl(*case, dtype=dtype)
    inp = make_inputs(w, device="cuda")
    _run_and_check(w, inp)


SPLIT_CASES = [
    # inference forwards whose expert GEMMs are weight streams: h travels as
    # a bf16 pair (hi + lo) into the down projections
    ("split_routed_shared_splitk", 40, 1024, 8, 2, 128, 512, 0, True, True, 0.0),
    ("split_shared_bm64", 256, 256, 8, 2, 64, 256, 1, True, True, 0.0),
    ("split_e60_k4", 16, 1024, 60, 4, 256, 1024, 0, False, True, 0.0),
]


@pytest.mark.parametrize("case", SPLIT_CASES, ids=[c[0] for c in SPLIT_CASES])
def test_inference_split_activation_against_exact(case):
    """An inference forward (no saved activations) of a bf16 layer whose
    expert GEMMs are weight streams: every token against the exact
    (unrounded) oracle at max-abs <= 2e-2 * RMS, and more of its elements
    are the correct bf16 rounding of the exact value than in the same
    layer's forward with saved activations (bf16 h)."""
    need_gpu()
    w = _wl(*case)
    inp = make_inputs(w, device="cuda")
    layer = make_layer(w, inp)
    out = np64(layer.forward(inp["x"], save=False))
    saved = np64(make_layer(w, inp).forward(inp["x"], save=True))
    torch.cuda.synchronize()
    s = layer.last
    l32 = layer._route(inp["x"], want_logits=True)["logits"].cpu().numpy()
    ids = s["ids"].cpu().numpy()
    assert np.array_equal(ids, oracle_selection(l32, w, None))
    wts = R.routing_weights(R.scores_f64(l32.astype(np.float64), w.score), ids, w.renorm)
    f = {k: np64(v) for k, v in inp.items() if k not in ("dout",)}
    exact = R.dense_masked_forward(f["x"], ids, wts, f["w_gate_up"], f["w_down"], f.get("ws_gate_up"),
                                   f.get("ws_down"), f.get("w_shared_gate") if w.shared_gated else None)
    gate_out_exact(out, exact, w.name)
    rounded = R.round_bf16(exact)
    c_split, c_saved = float(np.mean(out == rounded)), float(np.mean(saved == rounded))
    say(f"{w.name}: correctly rounded elements {c_split:.4f} (split h) vs {c_saved:.4f} (bf16 h); max-abs against "
        f"the exact oracle {np.max(np.abs(out - exact)):.3e} vs {np.max(np.abs(saved - exact)):.3e}")
    assert c_split > c_saved


LAYER_CASES = [
    # name, T, H, E, k, I, Is, score, renorm, gated, bias
    # decode-sized with a shared expert: its GEMMs are queued before the routing
    ("decode_qwen2moe_T16", 16, 2048, 60, 4, 1408, 5632, 0, False, True, 0.0),
    ("decode_small_bias", 24, 256, 8, 2, 128, 256, 2, True, False, 0.5),
    # prefill-sized: everything on the caller's stream
    ("prefill_gated", 300, 256, 8, 2, 192, 256, 1, True, True, 0.0),
    # no shared expert
    ("decode_no_shared", 16, 256, 16, 4, 128, 0, 0, True, False, 0.0),
]


@pytest.mark.parametrize("case", LAYER_CASES, ids=[c[0] for c in LAYER_CASES])
@pytest.mark.parametrize("profiled", [False, True], ids=["plain", "stage_profile"])
def test_layer_forward_equals_route_dispatch_then_ffn_forward(case, profiled):
    """moe_layer_forward (the layer's inference forward) against its
    definition, moe_route_dispatch followed by moe_ffn_forward: every routing
    output and the layer output bit for bit, with and without a stage
    profile (which keeps all of it on the caller's stream)."""
    need_gpu()
    from sparse_mixture_experts_route_amd import _lib as L
    w = _wl(*case)
    inp = make_inputs(w, device="cuda")
    layer = make_layer(w, inp)
    x = inp["x"]
    if profiled:
        L.moe_profile_begin(4)
    out = layer.forward(x)
    if profiled:
        L.moe_profile_end()
    torch.cuda.synchronize()
    whole = dict(layer.last)
    sh = layer._shape_T(w.T)
    r = layer._route(x, dispatch=True)
    ref = torch.empty_like(x)
    L.moe_ffn_forward(sh, layer.weights, x, None, r["offsets"], r["perm"], r["pos"], r["weights"], r["gate"], ref,
                      None, layer._workspace(sh, L.OP_FFN_FORWARD, x.device))
    torch.cuda.synchronize()
    for name in ("weights", "ids", "counts", "offsets", "perm", "pos"):
        assert torch.equal(whole[name], r[name]), name
    if w.shared_gated:
        assert torch.equal(whole["gate"], r["gate"])
    assert torch.equal(out, ref)
    say(f"{w.name}: moe_layer_forward equals the two calls bit for bit ({'profiled' if profiled else 'plain'})")


def test_layer_forward_no_tokens():
    """A batch of no tokens: moe_layer_forward writes what the two calls write
    (zero counts and offsets) and launches nothing else."""
    need_gpu()
    from sparse_mixture_experts_route_amd import _lib as L
    w = _wl(*LAYER_CASES[0])
    inp = make_inputs(w.with_(T=8), device="cuda")
    layer = make_layer(w, inp)
    sh = layer._shape_T(0)
    dev = inp["x"].device
    x = inp["x"][:0]
    outs = []
    for call in ("whole", "two"):
        counts = torch.full((w.E,), -1, dtype=torch.int32, device=dev)
        offsets = torch.full((w.E + 1,), -1, dtype=torch.int32, device=dev)
        e32 = torch.empty((0,), dtype=torch.int32, device=dev)
        wts = torch.empty((0, w.k), dtype=torch.float32, device=dev)
        ids = torch.empty((0, w.k), dtype=torch.int64, device=dev)
        gate = torch.empty((0,), dtype=torch.float32, device=dev)
        out = torch.empty_like(x)
        if call == "whole":
            L.moe_layer_forward(sh, layer.weights, x, layer.p["w_router"], layer.p["w_shared_gate"], None, wts, ids,
                                gate, counts, offsets, e32, e32, out, layer._workspace(sh, L.OP_LAYER_FORWARD, dev))
        else:
            L.moe_route_dispatch(sh, x, layer.p["w_router"], layer.p["w_shared_gate"], None, None, wts, ids, gate,
                                 counts, offsets, e32, e32, layer._workspace(sh, L.OP_ROUTE_DISPATCH, dev))
            L.moe_ffn_forward(sh, layer.weights, x, None, offsets, e32, e32, wts, gate, out, None,
                              layer._workspace(sh, L.OP_FFN_FORWARD, dev))
        torch.cuda.synchronize()
        outs.append((counts.clone(), offsets.clone()))
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])


PREFILL_CASES = [
    # name, T, H, E, k, I, Is, score, renorm, gated, bias: every GEMM of these
    # on the 256x256 kernel (no split activation), a ragged last m-tile and a
    # ragged last n-tile
    ("gated_ragged_T", 4200, 4096, 16, 2, 256, 512, 0, False, True, 0.0),
    ("ungated_ragged_H", 4096, 4104, 16, 3, 128, 256, 2, True, False, 0.5),
]


@pytest.mark.parametrize("case", PREFILL_CASES, ids=[c[0] for c in PREFILL_CASES])
def test_inference_forward_equals_saving_forward(case):
    """At prefill sizes the inference forward (moe_layer_forward) and the
    forward that saves its activations (routing and moe_ffn_forward with the
    saved g, u, h, y, S) give the same output bit for bit: the epilogues that
    also store the saved rows change nothing of what they compute.  A sample
    of tokens, the last m-tile's included, against the exact oracle."""
    need_gpu()
    w = _wl(*case)
    inp = make_inputs(w, device="cuda")
    layer = make_layer(w, inp)
    out = layer.forward(inp["x"], save=False)
    saving = make_layer(w, inp).forward(inp["x"], save=True)
    torch.cuda.synchronize()
    assert torch.equal(out, saving)
    s = layer.last
    l32 = layer._route(inp["x"], want_logits=True)["logits"].cpu().numpy()
    ids = s["ids"].cpu().numpy()
    assert np.array_equal(ids, oracle_selection(l32, w, inp.get("sel_bias")))
    wts = R.routing_weights(R.scores_f64(l32.astype(np.float64), w.score), ids, w.renorm)
    toks = np.concatenate([np.arange(4), np.arange(w.T - 4, w.T), np.arange(256, w.T, 997)])
    f = {k: np64(v) for k, v in inp.items() if k not in ("dout",)}
    exact = R.dense_masked_forward(f["x"][toks], ids[toks], wts[toks], f["w_gate_up"], f["w_down"], f["ws_gate_up"],
                                   f["ws_down"], f.get("w_shared_gate") if w.shared_gated else None)
    gate_out_exact(np64(out[torch.as_tensor(toks, device=out.device)]), exact, f"{w.name}: {len(toks)} tokens")


def test_fused_gather_matches_sorted_copy():
    need_gpu()
    w = _wl(*SMALL[1])
    inp = make_inputs(w, device="cuda")
    a = make_layer(w, inp, fuse_gather=False).forward(inp["x"])
    b = make_layer(w, inp, fuse_gather=True).forward(inp["x"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_exact_dyadic_preactivations_bitwise():
    """Exact-dyadic inputs make every fp32 accumulation exact, so the saved
    fp32 pre-activations g, u equal the exact products bit for bit."""
    need_gpu()
    T, H, E, k, I, Is = 160, 512, 8, 2, 128, 64
    w = Workload("dyadic", T=T, H=H, E=E, k=k, I=I, Is=Is, score=0, renorm=True)
    inp = exact_dyadic_inputs(T, H, E, I, Is, seed=5, device="cuda")
    layer = make_layer(w, inp)
    layer.forward(inp["x"], save=True)
    torch.cuda.synchronize()
    s = layer.last
    perm = s["perm"].cpu().numpy()
    x = np64(inp["x"])
    ids = s["ids"].cpu().numpy()
    e_of_row = ids.reshape(-1)[perm]
    gu_ref = np.zeros((T * k, 2 * I))
    for e in range(E):
        rows = np.nonzero(e_of_row == e)[0]
        gu_ref[rows] = x[perm[rows] // k] @ np64(inp["w_gate_up"][e]).T
    # the saved fp32 pre-activations are exact
    assert torch.equal(s["gu"].cpu(), torch.tensor(gu_ref, dtype=torch.float32))
    sgu = torch.tensor(x @ np64(inp["ws_gate_up"]).T, dtype=torch.float32)
    assert torch.equal(s["s_gu"].cpu(), sgu)


def test_empty_experts_are_skipped_with_nan_weights():
    """Experts that receive no token are never read: poisoning their weights
    with NaN leaves the output bit-identical."""
    need_gpu()
    w = _wl("empties", 300, 256, 16, 2, 128, 0, 0, True, False, 0.0)
    inp = make_inputs(w, device="cuda")
    inp["x"][:, 0] = 1.0
    inp["w_router"][:5] = 0.0
    inp["w_router"][:5, 0] = -30.0      # experts 0..4 lose every token
    layer = make_layer(w, inp)
    ref = layer.forward(inp["x"]).clone()
    counts = layer.last["counts"].cpu().numpy()
    empty = np.nonzero(counts == 0)[0]
    assert len(empty) >= 1
    for e in empty:
        inp["w_gate_up"][int(e)] = float("nan")
        inp["w_down"][int(e)] = float("nan")
    out = make_layer(w, inp).forward(inp["x"])
    torch.cuda.synchronize()
    assert torch.isfinite(out).all()
    assert torch.equal(out, ref)


def test_shared_expert_sums_separately():
    need_gpu()
    w = _wl(*SMALL[1])
    inp = make_inputs(w, device="cuda")
    with_s = np64(make_layer(w, inp).forward(inp["x"]))
    w0 = w.with_(Is=0, shared_gated=False)
    inp0 = {k: v for k, v in inp.items() if k not in ("ws_gate_up", "ws_down", "w_shared_gate")}
    without = np64(make_layer(w0, inp0).forward(inp["x"]))
    f = {k: np64(v) for k, v in inp.items()}
    gS = R.shared_term(f["x"], f["ws_gate_up"], f["ws_down"], f["w_shared_gate"], bf16=True)
    # the difference of two bf16 outputs carries the rounding of each of them
    # (at the magnitude of routed + shared, not of the shared term), so that
    # is what is allowed beyond the 2e-2 * RMS bound
    slack = bf16_half_ulp(with_s) + bf16_half_ulp(without)
    raw = float(np.max(np.abs((with_s - without) - gS)))
    err = float(np.max(np.maximum(np.abs((with_s - without) - gS) - slack, 0.0)))
    say(f"shared term: {err:.3e} beyond the two outputs' rounding (raw {raw:.3e}, tol {bf16_tol(gS):.3e})")
    assert err <= bf16_tol(gS), f"shared term: {err:.3e} > {bf16_tol(gS):.3e}"


def test_forward_deterministic():
    need_gpu()
    w = _wl(*SMALL[3])
    inp = make_inputs(w, device="cuda")
    a = make_layer(w, inp).forward(inp["x"]).clone()
    b = make_layer(w, inp).forward(inp["x"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_router_contract_and_deferred_balance():
    """route(x) -> (weights (T,k) fp32, ids (T,k) int64, state): None for a
    stateless router, the bias for one with a selection bias; a training
    forward stashes counts and the next forward applies them first; eval does
    not stash; a second apply is a no-op; the bias stays fp32."""
    need_gpu()
    w0 = _wl(*SMALL[0])
    inp0 = make_inputs(w0, device="cuda")
    weights, ids, state = make_layer(w0, inp0).route(inp0["x"])
    assert weights.dtype == torch.float32 and ids.dtype == torch.int64 and state is None
    w = _wl(*SMALL[3])
    inp = make_inputs(w, device="cuda")
    layer = make_layer(w, inp, rate=1e-2)
    weights, ids, state = layer.route(inp["x"])
    assert weights.dtype == torch.float32 and ids.dtype == torch.int64
    assert torch.equal(state.bias, layer.balance.bias) and state.counts is None
    assert tuple(ids.shape) == (w.T, w.k)
    b0 = layer.balance.bias.clone()
    layer.forward(inp["x"], training=False)
    assert not layer.balance.pending
    layer.forward(inp["x"], training=True)
    assert layer.balance.pending
    assert torch.equal(layer.balance.bias, b0)        # not mutated before the next forward
    counts = layer.last["counts"].cpu().numpy()
    assert layer.balance.apply_pending(layer.shape)
    torch.cuda.synchronize()
    b1 = layer.balance.bias.clone()
    want = R.balance_update(b0.cpu().numpy(), counts, 1e-2, w.T * w.k)
    assert np.array_equal(b1.cpu().numpy(), want)
    assert not layer.balance.apply_pending(layer.shape)   # second apply: no-op
    assert torch.equal(layer.balance.bias, b1)
    assert layer.balance.bias.dtype == torch.float32


@pytest.mark.parametrize("gated", [False, True])
def test_n_shared_2_fused_shared_expert(gated):
    """Two shared experts of width 96 fused into one of width 192 (gate rows
    of both, up rows of both, down columns side by side): the layer output
    equals the routed term plus the sum of the two experts computed
    separately by the oracle."""
    need_gpu()
    Ie = 96
    w = _wl("n_shared_2", 200, 256, 16, 4, 128, 2 * Ie, 0, True, gated, 0.0)
    inp = make_inputs(w, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(77)
    parts = [{"gu": (torch.randn((2 * Ie, w.H), generator=g, device="cuda") / w.H ** 0.5).to(torch.bfloat16),
              "d": (torch.randn((w.H, Ie), generator=g, device="cuda") / Ie ** 0.5).to(torch.bfloat16)}
             for _ in range(2)]
    inp["ws_gate_up"] = torch.cat([parts[0]["gu"][:Ie], parts[1]["gu"][:Ie], parts[0]["gu"][Ie:],
                                   parts[1]["gu"][Ie:]]).contiguous()
    inp["ws_down"] = torch.cat([parts[0]["d"], parts[1]["d"]], dim=1).contiguous()
    layer = make_layer(w, inp)
    out = layer.forward(inp["x"], save=True)
    torch.cuda.synchronize()
    s = layer.last
    l32 = s["logits"].cpu().numpy()
    ids = s["ids"].cpu().numpy()
    wts = R.routing_weights(R.scores_f64(l32.astype(np.float64), w.score), ids, w.renorm)
    f = {k: np64(v) for k, v in inp.items() if k not in ("dout",)}
    wsg = f["w_shared_gate"] if gated else None

    def oracle(bf16):
        ref = R.dense_masked_forward(f["x"], ids, wts, f["w_gate_up"], f["w_down"], bf16=bf16)
        for p in parts:
            ref = ref + R.shared_term(f["x"], np64(p["gu"]), np64(p["d"]), wsg, bf16=bf16)
        return ref
    assert_close(np64(out), oracle(True), "bf16", f"n_shared=2 fused (gated={gated})")
    report_exact(np64(out), oracle(False), f"n_shared=2 fused (gated={gated})")


def test_router_states_threaded_through_the_block():
    """Stateful router ("mstar.model.components.moe", Router contract: a
    stateful router reads router_states and returns the next state; the
    block returns it when asked): threading the state explicitly through
    three training forwards selects exactly what the layer's own deferred
    balance selects, leaves the layer's own state and every earlier state
    untouched, and the bias it carries follows the oracle's controller."""
    need_gpu()
    from sparse_mixture_experts_route_amd.layer import RouterState
    w = _wl(*SMALL[3])
    inp = make_inputs(w, device="cuda")
    own = make_layer(w, inp, rate=1e-2)
    ext = make_layer(w, inp, rate=1e-2)
    b0 = ext.balance.bias.clone()
    st = RouterState(b0.clone())
    seen = [st]
    oracle = R.BalanceState(b0.cpu().numpy(), 1e-2)
    for i in range(3):
        x = make_inputs(w.with_(seed=50 + i), device="cuda")["x"]
        own.forward(x, training=True)
        out, st = ext.forward(x, training=True, router_states=st, return_router_states=True)
        torch.cuda.synchronize()
        oracle.apply_pending()
        assert np.array_equal(st.bias.cpu().numpy(), oracle.bias), f"step {i}: bias"
        assert torch.equal(own.last["ids"], ext.last["ids"]), f"step {i}: ids"
        assert torch.equal(st.counts, ext.last["counts"]) and st.tokens_k == w.T * w.k
        oracle.after_forward(st.counts.cpu().numpy(), w.T * w.k, training=True)
        seen.append(st)
    assert torch.equal(ext.balance.bias, b0) and not ext.balance.pending   # own state untouched
    assert torch.equal(seen[0].bias, b0)                                  # inputs not mutated
    # eval forward: the state passes through with nothing pending
    _, st2 = ext.forward(x, training=False, router_states=st, return_router_states=True)
    assert st2.counts is None
    # a stateless router ignores router_states and returns None
    w0 = _wl(*SMALL[0])
    inp0 = make_inputs(w0, device="cuda")
    out0, none = make_layer(w0, inp0).forward(inp0["x"], router_states=st, return_router_states=True)
    assert none is None
