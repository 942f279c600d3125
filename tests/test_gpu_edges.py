"""Edge cases of the whole layer on the GPU against the oracle: one token,
zero tokens, every expert selected (k = E), k = 1, a single expert, hidden sizes that take
the other GEMM engines (K not a multiple of 64 or of 32), and intermediate
sizes that leave ragged 256-wide output tiles.  Forward and backward, with
the bounds of test_gpu_forward and test_gpu_backward."""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from workloads import Workload, make_inputs

from gpu_helpers import assert_close, check_grads, make_layer, need_gpu, np64, oracle_selection, report_exact

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, H, E, k, I, Is, score, renorm, gated
    ("one_token", 1, 256, 8, 2, 128, 64, 0, True, True),
    ("k_equals_E", 70, 256, 8, 8, 64, 0, 0, True, False),
    ("k_one", 90, 256, 16, 1, 128, 64, 1, False, False),
    ("h288_dma_path", 120, 288, 8, 2, 96, 96, 2, True, True),     # K % 64 = 32
    ("h264_generic_path", 77, 264, 12, 3, 72, 40, 0, False, True),  # K % 32 = 8
    ("ragged_tiles", 300, 256, 4, 2, 328, 264, 0, True, False),     # N not a multiple of 256
    ("single_expert", 100, 256, 1, 1, 128, 64, 0, True, True),      # E = 1: every token, weight 1
]


def _layer(case, dtype):
    name, T, H, E, k, I, Is, score, renorm, gated = case
    w = Workload(name, T=T, H=H, E=E, k=k, I=I, Is=Is, score=score, renorm=renorm, shared_gated=gated,
                 dtype=dtype, seed=T * 7 + H, backward=True)
    inp = make_inputs(w, device="cuda")
    return w, inp, make_layer(w, inp)


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_edge_forward_backward(case, dtype):
    need_gpu()
    w, inp, layer = _layer(case, dtype)
    out = layer.forward(inp["x"], save=True)
    g = layer.backward(inp["dout"], want_dlogits=True)
    torch.cuda.synchronize()
    s = layer.last
    l32 = s["logits"].cpu().numpy()
    ids = s["ids"].cpu().numpy()
    assert np.array_equal(ids, oracle_selection(l32, w, inp.get("sel_bias")))
    if w.k == w.E:
        assert np.array_equal(np.sort(ids, axis=1), np.tile(np.arange(w.E), (w.T, 1)))
    wts = R.routing_weights(R.scores_f64(l32.astype(np.float64), w.score), ids, w.renorm)
    f = {kk: np64(v) for kk, v in inp.items()}
    wsg = f.get("w_shared_gate") if w.shared_gated else None
    bf = dtype == "bf16"
    fargs = (f["x"], ids, wts, f["w_gate_up"], f["w_down"], f.get("ws_gate_up"), f.get("ws_down"), wsg)
    assert_close(np64(out), R.dense_masked_forward(*fargs, bf16=bf), dtype, f"{w.name} {dtype} out")
    if bf:
        report_exact(np64(out), R.dense_masked_forward(*fargs), f"{w.name} {dtype} out")
    bargs = (f["x"], f["w_router"], ids, l32.astype(np.float64), w.score, w.renorm, f["w_gate_up"], f["w_down"],
             f["dout"], f.get("ws_gate_up"), f.get("ws_down"), wsg)
    check_grads(w, g, R.layer_backward(*bargs, bf16=bf), f"{w.name} {dtype}",
                exact=R.layer_backward(*bargs) if bf else None)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_zero_tokens(dtype):
    """T = 0 with a gated shared expert and the aux loss on: the forward and
    backward run, return empty outputs and zero weight gradients."""
    need_gpu()
    w = Workload("zero", T=8, H=256, E=8, k=2, I=128, Is=64, score=0, renorm=True, shared_gated=True, dtype=dtype,
                 seed=3, backward=True)
    inp = make_inputs(w, device="cuda")
    layer = make_layer(w, inp)
    layer.aux_alpha = 0.0      # the aux loss of no tokens is undefined; forward without it
    x0 = inp["x"][:0]
    out = layer.forward(x0, training=True, save=True)
    g = layer.backward(inp["dout"][:0], want_dlogits=True)
    torch.cuda.synchronize()
    assert tuple(out.shape) == (0, w.H)
    assert torch.equal(layer.last["counts"].cpu(), torch.zeros(w.E, dtype=torch.int32))
    for name in ("dw_router", "dw_gate_up", "dw_down", "dws_gate_up", "dws_down", "dw_shared_gate"):
        assert torch.count_nonzero(g[name]).item() == 0, name
