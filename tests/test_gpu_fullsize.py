"""Full-size parity of the layer in the launch configuration bench.py times
(layers built by bench.build_layer: fused row gather, fp32 selection bias
where the workload has one), at the sizes of the five layer configurations.

Checked exactly (integer work): the top-k ids against the oracle's selection
on the GPU's own fp32 logits, every token; expert counts, segment offsets,
the stable permutation and its inverse.  Checked against the float64 oracle
(per-expert loop, bf16-operand reading): sampled tokens of the output
(max-abs beyond bf16 rounding <= 2e-2 * RMS of the sampled reference), every
token for the decode-sized forwards; for the training shape, the data
gradient and the router-logit gradient of sampled tokens and both weight
gradients of one whole expert; for one share of an 8-way tensor-parallel
split, sampled partial rows.
"""
import numpy as np
import pytest
import torch

import bench
from oracle import moe_ref as R
from workloads import WORKLOADS, decode_workload

from gpu_helpers import (bf16_err, bf16_tol, need_gpu, np64, oracle_partial_rows, oracle_selection,
                         oracle_tokens_forward, sample_tokens, say)
from sparse_mixture_experts_route_amd.layer import forward_partial, tp_share_params

pytestmark = pytest.mark.gpu


def _check_dispatch(w, s):
    ids = s["ids"].cpu().numpy()
    counts = s["counts"].cpu().numpy()
    offsets = s["offsets"].cpu().numpy()
    perm = s["perm"].cpu().numpy()
    pos = s["pos"].cpu().numpy()
    flat = ids.reshape(-1)
    assert np.array_equal(counts, np.bincount(flat, minlength=w.E))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(counts)]))
    assert np.array_equal(perm, np.argsort(flat, kind="stable"))
    assert np.array_equal(pos[perm], np.arange(flat.size))
    return ids, counts


def _forward_and_route(w):
    layer, inp = bench.build_layer(w)
    out = layer.forward(inp["x"], training=False, save=False)
    torch.cuda.synchronize()
    s = dict(layer.last)
    # the same router call with the fp32 logits written out
    r = layer._route(inp["x"], want_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(r["ids"], s["ids"]) and torch.equal(r["weights"], s["weights"])
    l32 = r["logits"].cpu().numpy()
    assert np.array_equal(s["ids"].cpu().numpy(), oracle_selection(l32, w, inp.get("sel_bias")))
    return layer, inp, out, s, l32


def _check_tokens(w, inp, out, s, l32, toks):
    ids = s["ids"].cpu().numpy()
    wts = R.routing_weights(R.scores_f64(l32.astype(np.float64), w.score), ids, w.renorm)
    got = np64(out[torch.as_tensor(toks, device=out.device)])
    ref = oracle_tokens_forward(w, inp, ids, wts, toks)
    err, tol = bf16_err(got, ref), bf16_tol(ref)
    say(f"{w.name}: {len(toks)} tokens, max-abs beyond rounding {err:.3e} (tol {tol:.3e})")
    assert err <= tol


FORWARD = [("dsv4flash", 24), ("qwen2moe", 24), ("deepseekv3", 8)]


@pytest.mark.parametrize("name,n", FORWARD, ids=[f[0] for f in FORWARD])
def test_fullsize_forward(name, n):
    need_gpu()
    w = WORKLOADS[name]
    say(f"full-size forward {name}: T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} Is={w.Is}")
    layer, inp, out, s, l32 = _forward_and_route(w)
    ids, counts = _check_dispatch(w, s)
    toks = sample_tokens(ids, counts, n, seed=1)
    _check_tokens(w, inp, out, s, l32, toks)


@pytest.mark.parametrize("T", [16, 64, 256])
def test_fullsize_decode_every_token(T):
    need_gpu()
    w = decode_workload(T)
    say(f"decode forward T={T}")
    layer, inp, out, s, l32 = _forward_and_route(w)
    _check_dispatch(w, s)
    _check_tokens(w, inp, out, s, l32, np.arange(T))


def test_fullsize_training_backward():
    """Qwen2-MoE-like shape at T=8192, forward + backward as the bench runs it."""
    need_gpu()
    w = WORKLOADS["qwen2moe_train"]
    say(f"full-size training T={w.T} H={w.H} E={w.E} k={w.k} I={w.I} Is={w.Is}")
    layer, inp = bench.build_layer(w)
    layer.forward(inp["x"], training=False, save=True)
    g = layer.backward(inp["dout"], want_dlogits=True)
    torch.cuda.synchronize()
    s = layer.last
    ids, counts = _check_dispatch(w, s)
    l32 = s["logits"].cpu().numpy()
    assert np.array_equal(ids, oracle_selection(l32, w, inp.get("sel_bias")))
    f = {k: np64(inp[k]) for k in ("w_router", "w_gate_up", "w_down")}
    # data and router-logit gradients of sampled tokens (each token's own path)
    toks = sample_tokens(ids, counts, 8, seed=2)
    tt = torch.as_tensor(toks, device="cuda")
    ref = R.layer_backward(np64(inp["x"][tt]), f["w_router"], ids[toks], l32[toks].astype(np.float64), w.score,
                           w.renorm, f["w_gate_up"], f["w_down"], np64(inp["dout"][tt]), np64(inp["ws_gate_up"]),
                           np64(inp["ws_down"]), np64(inp["w_shared_gate"]) if w.shared_gated else None,
                           loop=True, bf16=True)
    err = bf16_err(np64(g["dx"][tt]), ref["dx"])
    say(f"dx on {len(toks)} tokens: {err:.3e} (tol {bf16_tol(ref['dx']):.3e})")
    assert err <= bf16_tol(ref["dx"])
    dl = np64(g["dlogits"][tt])
    err = float(np.max(np.abs(dl - ref["dlogits"])))
    say(f"dlogits on {len(toks)} tokens: {err:.3e} (tol {bf16_tol(ref['dlogits']):.3e})")
    assert err <= bf16_tol(ref["dlogits"])
    # both weight gradients of the least-loaded non-empty expert, from all its rows
    used = np.nonzero(counts > 0)[0]
    e = int(used[np.argmin(counts[used])])
    te = np.nonzero((ids == e).any(axis=1))[0]
    et = torch.as_tensor(te, device="cuda")
    ref = R.layer_backward(np64(inp["x"][et]), f["w_router"], ids[te], l32[te].astype(np.float64), w.score,
                           w.renorm, f["w_gate_up"], f["w_down"], np64(inp["dout"][et]), loop=True, bf16=True)
    for name in ("dw_gate_up", "dw_down"):
        got = np64(g[name][e])
        want = ref[name][e]
        err, tol = float(np.max(np.abs(got - want))), bf16_tol(want)
        say(f"{name}[{e}] ({len(te)} tokens): {err:.3e} (tol {tol:.3e})")
        assert err <= tol


def test_fullsize_tp8_share_rows():
    """One share of an 8-way tensor-parallel split of the DSV4-shaped layer
    (slices I/8 = 256, Is/8 = 256) as bench.py times it: sampled partial rows
    and shared rows against the float64 oracle MLP on that share's slices."""
    need_gpu()
    w = WORKLOADS["dsv4flash"]
    layer, inp = bench.build_layer(w)
    layer.forward(inp["x"], training=False, save=False)
    s = layer.last
    sw = tp_share_params(layer.p, 8, 5)
    y, sy = forward_partial(layer.shape, sw, 8, inp["x"], s["offsets"], s["perm"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(3)
    P = w.T * w.k
    rows = np.unique(np.concatenate([[0, P - 1], rng.choice(P, 30, replace=False)]))
    ref = oracle_partial_rows(w, inp, sw, s, rows)
    got = np64(y[torch.as_tensor(rows, device="cuda")])
    err = float(np.max(np.abs(got - ref)))
    say(f"tp8 share 5: {len(rows)} partial rows, max-abs {err:.3e} (tol {bf16_tol(ref):.3e})")
    assert err <= bf16_tol(ref)
    toks = rng.choice(w.T, 8, replace=False)
    refs = R.swiglu_mlp(np64(inp["x"][torch.as_tensor(toks, device="cuda")]), np64(sw["ws_gate_up"]),
                        np64(sw["ws_down"]), True)
    err = float(np.max(np.abs(np64(sy[torch.as_tensor(toks, device="cuda")]) - refs)))
    say(f"tp8 share 5: 8 shared rows, max-abs {err:.3e} (tol {bf16_tol(refs):.3e})")
    assert err <= bf16_tol(refs)
