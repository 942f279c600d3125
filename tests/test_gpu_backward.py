"""GPU parity of the backward (moe_ffn_backward) against the oracle's
analytic float64 gradients (themselves pinned by finite differences).

fp32 layer: max-abs <= 1e-5 per gradient tensor against the exact oracle
(the named exceptions of gpu_helpers.FP32_EXCEPTIONS aside); bf16 layer:
max-abs <= 2e-2 * RMS(reference) per gradient tensor against the oracle's
operand-rounding model (h, dy = w * dout and dg | du are bf16 tensors; dx is
stored in bf16: half a bf16 ulp is allowed only on its elements where that
alone exceeds the bound), the exact oracle's error logged beside.  Also: two
runs give identical bits, experts with no rows get exact-zero weight
gradients.
"""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from workloads import WORKLOADS, Workload, make_inputs

from gpu_helpers import check_grads, make_layer, need_gpu, np64

pytestmark = pytest.mark.gpu

def _fwd_bwd(w, inp):
    layer = make_layer(w, inp)
    layer.forward(inp["x"], save=True)
    g = layer.backward(inp["dout"], want_dlogits=True)
    torch.cuda.synchronize()
    return layer, g


def _check(w, inp, layer, g):
    s = layer.last
    l32 = s["logits"].cpu().numpy()
    ids = s["ids"].cpu().numpy()
    f = {k: np64(v) for k, v in inp.items()}
    args = (f["x"], f["w_router"], ids, l32.astype(np.float64), w.score, w.renorm, f["w_gate_up"], f["w_down"],
            f["dout"], f.get("ws_gate_up"), f.get("ws_down"), f.get("w_shared_gate") if w.shared_gated else None)
    bf = w.dtype == "bf16"
    ref = R.layer_backward(*args, bf16=bf)
    check_grads(w, g, ref, f"{w.name} {w.dtype}", exact=R.layer_backward(*args) if bf else None)


def test_tiny_fp32_backward_parity():
    need_gpu()
    w = WORKLOADS["tiny_fp32"].with_(backward=True)
    inp = make_inputs(w, device="cuda")
    layer, g = _fwd_bwd(w, inp)
    _check(w, inp, layer, g)


CASES = [
    Workload("bwd_softmax_gated", T=257, H=256, E=12, k=4, I=136, Is=192, score=0, renorm=False,
             shared_gated=True, seed=11, backward=True),
    Workload("bwd_sqrtsoftplus_bias", T=200, H=320, E=16, k=6, I=128, Is=128, score=2, renorm=True,
             bias_var=0.5, seed=12, backward=True),
    Workload("bwd_sigmoid", T=150, H=256, E=8, k=2, I=256, Is=0, score=1, renorm=True, seed=13, backward=True),
    # 40 tokens: both shared-expert GEMMs of the forward split K (the saved
    # gate | up pre-activations come from the split reduction)
    Workload("bwd_shared_splitk", T=40, H=1024, E=8, k=2, I=128, Is=512, score=1, renorm=True,
             shared_gated=True, seed=14, backward=True),
    # whole 64-row slices of tokens for the shared weight gradients' reduction
    Workload("bwd_shared_t320", T=320, H=256, E=8, k=2, I=128, Is=192, score=0, renorm=True,
             shared_gated=True, seed=15, backward=True),
]


@pytest.mark.parametrize("w", CASES, ids=[c.name for c in CASES])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_small_backward_parity(w, dtype):
    need_gpu()
    w = w.with_(dtype=dtype)
    inp = make_inputs(w, device="cuda")
    layer, g = _fwd_bwd(w, inp)
    _check(w, inp, layer, g)


def test_backward_deterministic_and_empty_experts_zero():
    need_gpu()
    w = CASES[0]
    inp = make_inputs(w, device="cuda")
    inp["x"][:, 0] = 1.0
    inp["w_router"][:3] = 0.0
    inp["w_router"][:3, 0] = -30.0       # experts 0..2 receive no rows
    l1, g1 = _fwd_bwd(w, inp)
    g1 = {k: v.clone() for k, v in g1.items()}
    _, g2 = _fwd_bwd(w, inp)
    for k in g1:
        assert torch.equal(g1[k], g2[k]), k
    counts = l1.last["counts"].cpu().numpy()
    empty = np.nonzero(counts == 0)[0]
    assert len(empty) >= 3
    for e in empty:
        assert not g1["dw_gate_up"][int(e)].any()
        assert not g1["dw_down"][int(e)].any()
