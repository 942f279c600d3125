"""GPU parity of the full forward (route -> dispatch -> grouped SwiGLU GEMMs
-> combine + shared expert) against the dense-masked oracle.

fp32: max-abs <= 1e-5; bf16: max-abs <= 2e-2 * RMS(reference).  The oracle
routes from the GPU's fp32 logits after the ids were checked bit-exact.
"""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from workloads import WORKLOADS, Workload, exact_dyadic_inputs, make_inputs

from gpu_helpers import assert_close, bf16_half_ulp, bf16_tol, make_layer, need_gpu, np64, oracle_selection, say

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
    ref = R.dense_masked_forward(f["x"], ids, wts, f["w_gate_up"], f["w_down"], f.get("ws_gate_up"),
                                 f.get("ws_down"), f.get("w_shared_gate") if w.shared_gated else None,
                                 bf16=w.dtype == "bf16")
    err, tol = assert_close(np64(out), ref, w.dtype, w.name)
    say(f"{w.name}: max-abs {err:.3e} (tol {tol:.3e})")
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


def test_fused_gather_matches_sorted_copy():
    need_gpu()
    w = _wl(*SMALL[1])
    inp = make_inputs(w, device="cuda")
    a = make_layer(w, inp).forward(inp["x"])
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
    # (at the magnitude of routed + shared), so that is what is allowed
    # beyond the 2e-2 * RMS bound
    slack = bf16_half_ulp(with_s) + bf16_half_ulp(without)
    err = float(np.max(np.maximum(np.abs((with_s - without) - gS) - slack, 0.0)))
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
    """route(x) -> (weights (T,k) fp32, ids (T,k) int64, None); a training
    forward stashes counts and the next forward applies them first; eval does
    not stash; a second apply is a no-op; the bias stays fp32."""
    need_gpu()
    w = _wl(*SMALL[3])
    inp = make_inputs(w, device="cuda")
    layer = make_layer(w, inp, rate=1e-2)
    weights, ids, state = layer.route(inp["x"])
    assert weights.dtype == torch.float32 and ids.dtype == torch.int64 and state is None
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
