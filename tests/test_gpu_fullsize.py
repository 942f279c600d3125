"""Full-size parity of the layer in the launch configuration bench.py times
(layers built by bench.build_layer: fused row gather, fp32 selection bias
where the workload has one), at the sizes of the five layer configurations.

Checked exactly (integer work): the top-k ids against the oracle's selection
on the GPU's own fp32 logits, every token; expert counts, segment offsets,
the stable permutation and its inverse.  Checked against the float64 oracle
(per-expert loop): sampled tokens of the output, every token for the
decode-sized forwards, against the exact (unrounded) oracle (max-abs <= 2e-2
* RMS of the sampled reference; half a bf16 ulp allowed only where that alone
exceeds the bound), the operand-rounding model's distance logged beside (an
inference forward whose expert GEMMs are weight streams carries h as a bf16
pair, so its down projections see an exact operand); for the training
shape, every gradient tensor over all 8192 tokens (dx, dlogits, the
router-weight gradient, both weight gradients of every expert including the
most loaded one, the shared expert's and its gate's) against the
operand-rounding model, the exact oracle's error logged beside; for one share
of an 8-way tensor-parallel split, sampled partial rows against both.
"""
import numpy as np
import pytest
import torch

import bench
from oracle import moe_ref as R
from workloads import WORKLOADS, decode_workload

from gpu_helpers import (GRADS, STACKED, assert_close, check_grads, gate_out_exact, gate_with_ties, need_gpu, np64,
                         oracle_partial_rows, oracle_selection, oracle_tokens_forward, report_exact, report_model,
                         sample_tokens, say, tie_ulp)
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
    exact = oracle_tokens_forward(w, inp, ids, wts, toks)
    gate_out_exact(got, exact, f"{w.name}: {len(toks)} tokens")
    report_model(got, oracle_tokens_forward(w, inp, ids, wts, toks, bf16=True), f"{w.name}: {len(toks)} tokens")


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
    """Qwen2-MoE-like shape at T=8192, forward + backward as the bench runs
    it, against the oracle's per-expert-loop backward on every token."""
    import time
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
    say(f"expert loads: max {counts.max()} (expert {int(np.argmax(counts))}), min {counts.min()}")
    g = {k: v for k, v in g.items() if v is not None}
    t0 = time.time()
    f = {k: np64(inp[k]) for k in ("x", "w_router", "w_gate_up", "w_down", "dout", "ws_gate_up", "ws_down",
                                   "w_shared_gate")}
    args = (f["x"], f["w_router"], ids, l32.astype(np.float64), w.score, w.renorm, f["w_gate_up"], f["w_down"],
            f["dout"], f["ws_gate_up"], f["ws_down"], f["w_shared_gate"] if w.shared_gated else None)
    ref = R.layer_backward(*args, loop=True, bf16=True)
    exact = R.layer_backward(*args, loop=True)
    say(f"oracle backward on all {w.T} tokens (operand model and exact): {time.time() - t0:.1f} s")
    check_grads(w, g, ref, "training shape", exact=exact, names=[n for n, _ in GRADS if n not in STACKED])
    # the stacked weight gradients: 350 M / 170 M elements summing up to 636
    # rows each, where one tie-broken operand rounding on a dominant term can
    # move an element by ~0.4 % of itself; such roundings are allowed for
    wts = R.routing_weights(R.scores_f64(l32.astype(np.float64), w.score), ids, w.renorm)
    a_gu = np.zeros(ref["dw_gate_up"].shape)
    a_d = np.zeros(ref["dw_down"].shape)
    for e in range(w.E):
        t_idx, j_idx = np.nonzero(ids == e)
        if t_idx.size == 0:
            continue
        dy = wts[t_idx, j_idx][:, None] * f["dout"][t_idx]
        ops = R.mlp_operands_before_rounding(f["x"][t_idx], f["w_gate_up"][e], f["w_down"][e], dy)
        a_gu[e] = tie_ulp(ops["dgu"]).T @ np.abs(f["x"][t_idx])
        a_d[e] = tie_ulp(ops["dy"]).T @ np.abs(R.round_bf16(ops["h"])) + \
            np.abs(R.round_bf16(ops["dy"])).T @ tie_ulp(ops["h"])
    gate_with_ties(np64(g["dw_gate_up"]), ref["dw_gate_up"], a_gu, "training shape dw_gate_up")
    gate_with_ties(np64(g["dw_down"]), ref["dw_down"], a_d, "training shape dw_down")
    for name in STACKED:
        report_exact(np64(g[name]), exact[name], f"training shape {name}")
    # the heaviest segment's weight gradients on their own (the longest K of
    # the weight-gradient GEMM), against that expert's RMS
    e = int(np.argmax(counts))
    for name, a in (("dw_gate_up", a_gu), ("dw_down", a_d)):
        gate_with_ties(np64(g[name][e]), ref[name][e], a[e], f"{name}[{e}] ({counts[e]} rows, most loaded)")


def test_backward_saved_rows_past_2gib():
    """A layer whose saved fp32 pre-activations pass 2 GiB (T=16384, k=4,
    I=4608: 65536 sorted rows of 36 KB, the last ~7300 past byte 2^31), so
    the SwiGLU-backward GEMM reads the saved g, u and writes dg | du past the
    32-bit offsets of a descriptor based at the buffer (its descriptors are
    based at each tile's first row).  The last expert owns the rows at the end
    of the sorted order; the oracle runs on the tokens routed to it, which
    gives that expert's weight gradients whole and dx, dlogits of those
    tokens (each depends on its own token only)."""
    need_gpu()
    w = WORKLOADS["qwen2moe_train"].with_(name="rows_past_2gib", T=16384, H=64, E=8, k=4, I=4608, Is=0,
                                          shared_gated=False, renorm=True, seed=6)
    P = w.T * w.k
    row_bytes = 2 * w.I * 4
    first_past = (2 ** 31 + row_bytes - 1) // row_bytes
    assert P * row_bytes > 2 ** 31 and first_past < P
    say(f"saved rows: {P} x {row_bytes} bytes = {P * row_bytes / 2 ** 30:.2f} GiB; rows from {first_past} past 2^31")
    layer, inp = bench.build_layer(w)
    layer.forward(inp["x"], training=False, save=True)
    g = layer.backward(inp["dout"], want_dlogits=True)
    torch.cuda.synchronize()
    s = layer.last
    ids, counts = _check_dispatch(w, s)
    offsets = s["offsets"].cpu().numpy()
    e = w.E - 1
    say(f"expert {e}: rows {offsets[e]} .. {P - 1}, {P - max(offsets[e], first_past)} of them past 2^31")
    assert offsets[e] < first_past
    l32 = s["logits"].cpu().numpy()
    assert np.array_equal(ids, oracle_selection(l32, w, inp.get("sel_bias")))
    sub = np.nonzero((ids == e).any(axis=1))[0]
    f = {k: np64(inp[k]) for k in ("x", "w_router", "w_gate_up", "w_down", "dout")}
    ref = R.layer_backward(f["x"][sub], f["w_router"], ids[sub], l32[sub].astype(np.float64), w.score, w.renorm,
                           f["w_gate_up"], f["w_down"], f["dout"][sub], loop=True, bf16=True)
    got = {"dx": g["dx"][torch.from_numpy(sub).to(g["dx"].device)],
           "dlogits": g["dlogits"][torch.from_numpy(sub).to(g["dlogits"].device)]}
    check_grads(w, got, ref, f"tokens of expert {e}", names=["dx", "dlogits"])
    wts = R.routing_weights(R.scores_f64(l32.astype(np.float64), w.score), ids, w.renorm)
    t_idx, j_idx = np.nonzero(ids == e)
    dy = wts[t_idx, j_idx][:, None] * f["dout"][t_idx]
    ops = R.mlp_operands_before_rounding(f["x"][t_idx], f["w_gate_up"][e], f["w_down"][e], dy)
    a_gu = tie_ulp(ops["dgu"]).T @ np.abs(f["x"][t_idx])
    a_d = tie_ulp(ops["dy"]).T @ np.abs(R.round_bf16(ops["h"])) + np.abs(R.round_bf16(ops["dy"])).T @ tie_ulp(ops["h"])
    gate_with_ties(np64(g["dw_gate_up"][e]), ref["dw_gate_up"][e], a_gu, f"dw_gate_up[{e}] ({counts[e]} rows)")
    gate_with_ties(np64(g["dw_down"][e]), ref["dw_down"][e], a_d, f"dw_down[{e}] ({counts[e]} rows)")


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
    got = np64(y[torch.as_tensor(rows, device="cuda")])
    toks = rng.choice(w.T, 8, replace=False)
    xs = np64(inp["x"][torch.as_tensor(toks, device="cuda")])
    gots = np64(sy[torch.as_tensor(toks, device="cuda")])
    for bf, tag in ((True, "operand model"), (False, "exact oracle")):
        assert_close(got, oracle_partial_rows(w, inp, sw, s, rows, bf), "fp32-acc",
                     f"tp8 share 5: {len(rows)} partial rows [{tag}]")
        refs = R.swiglu_mlp(xs, np64(sw["ws_gate_up"]), np64(sw["ws_down"]), bf)
        assert_close(gots, refs, "fp32-acc", f"tp8 share 5: 8 shared rows [{tag}]")


def test_fullsize_parallel_block_tokens():
    """The parallel dense + MoE block at the Qwen2-MoE-like shape with a
    5632-wide dense MLP (the block bench.py times): sampled tokens of the
    output against the exact oracle (its operand-rounding model logged)."""
    from sparse_mixture_experts_route_amd.layer import ParallelDenseMoEBlock
    need_gpu()
    w = WORKLOADS["qwen2moe"].with_(Is=0, shared_gated=False)
    Id = WORKLOADS["qwen2moe"].Is
    layer, inp = bench.build_layer(w)
    g = torch.Generator(device="cuda").manual_seed(12)
    dt = inp["x"].dtype
    dense = {"w_gate_up": (torch.randn((2 * Id, w.H), generator=g, device="cuda") * w.H ** -0.5).to(dt),
             "w_down": (torch.randn((w.H, Id), generator=g, device="cuda") * Id ** -0.5).to(dt)}
    norms = {n: (1.0 + 0.3 * torch.randn((w.H,), generator=g, device="cuda")).to(dt)
             for n in ("g_pre_moe", "g_post_dense", "g_post_moe", "g_post")}
    residual = (inp["x"].float() * 2.5).to(dt)
    x_dense = torch.randn(inp["x"].shape, generator=g, device="cuda").to(dt)
    blk = ParallelDenseMoEBlock(layer, dense, norms, eps=1e-6, layer_scalar=0.8)
    out = blk.forward(residual, x_dense)
    r = layer._route(residual, want_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(r["ids"], layer.last["ids"])
    ids, counts = _check_dispatch(w, layer.last)
    l32 = r["logits"].cpu().numpy()
    assert np.array_equal(ids, oracle_selection(l32, w, None))
    toks = sample_tokens(ids, counts, 16, seed=4)
    tt = torch.as_tensor(toks, device="cuda")
    wts = R.routing_weights(R.scores_f64(l32[toks].astype(np.float64), w.score), ids[toks], w.renorm)
    f = {k: np64(v) for k, v in dense.items()}
    args = (np64(residual[tt]), np64(x_dense[tt]), ids[toks], wts, np64(inp["w_gate_up"]), np64(inp["w_down"]),
            f["w_gate_up"], f["w_down"], *[np64(norms[n]) for n in ("g_pre_moe", "g_post_dense", "g_post_moe",
                                                                    "g_post")], 1e-6, 0.8)
    got = np64(out[tt])
    gate_out_exact(got, R.parallel_block_forward(*args), f"parallel block: {len(toks)} tokens")
    report_model(got, R.parallel_block_forward(*args, bf16=True), f"parallel block: {len(toks)} tokens")
