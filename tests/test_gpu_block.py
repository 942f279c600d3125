"""GPU parity of the parallel dense + MoE block (moe_parallel_block_forward;
the DeepSpec issue "Feat: Compatible with Gamme4 MoE structure", Decoder layer
forward pass) against the oracle's parallel_block_forward: the router on the
residual (ids bit-exact on the GPU's own fp32 logits), the experts on its
RMS-normalised copy, the dense MLP beside them, three output norms, the
residual and the layer scalar.  bf16: max-abs <= 2e-2 * RMS against the
oracle's operand-rounding model (half a bf16 ulp allowed only on elements
where that alone exceeds the bound), the exact oracle's error logged beside;
fp32: 1e-5 against the exact oracle."""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from sparse_mixture_experts_route_amd.layer import ParallelDenseMoEBlock
from workloads import Workload, make_inputs

from gpu_helpers import assert_close, make_layer, need_gpu, np64, oracle_selection, report_exact

pytestmark = pytest.mark.gpu

CASES = [
    # name, T, H, E, k, I, Id (dense width), score, renorm, bias
    ("softmax", 150, 256, 8, 2, 128, 192, 0, True, 0.0),
    ("sqrtsoftplus_bias", 257, 384, 16, 4, 64, 256, 2, True, 0.5),
    ("sigmoid_ragged_h", 100, 264, 12, 3, 96, 136, 1, False, 0.0),
]


def _block(case, dtype):
    name, T, H, E, k, I, Id, score, renorm, bias = case
    w = Workload(name, T=T, H=H, E=E, k=k, I=I, Is=0, score=score, renorm=renorm, bias_var=bias, dtype=dtype,
                 seed=T + Id)
    inp = make_inputs(w, device="cuda")
    dt = inp["x"].dtype
    g = torch.Generator(device="cuda").manual_seed(T * 3 + H)
    rnd = lambda *shape, scale=1.0: (torch.randn(shape, generator=g, device="cuda") * scale).to(dt)
    dense = {"w_gate_up": rnd(2 * Id, H, scale=H ** -0.5), "w_down": rnd(H, Id, scale=Id ** -0.5)}
    norms = {n: (1.0 + 0.3 * torch.randn((H,), generator=g, device="cuda")).to(dt)
             for n in ("g_pre_moe", "g_post_dense", "g_post_moe", "g_post")}
    x_dense = rnd(T, H)
    residual = (inp["x"].float() * 2.5).to(dt)        # a residual stream of larger scale than unit
    blk = ParallelDenseMoEBlock(make_layer(w, inp), dense, norms, eps=1e-6, layer_scalar=0.8)
    return w, inp, blk, dense, norms, x_dense, residual


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_parallel_block_parity(case, dtype):
    need_gpu()
    w, inp, blk, dense, norms, x_dense, residual = _block(case, dtype)
    out = blk.forward(residual, x_dense)
    torch.cuda.synchronize()
    # the router read the residual: same call with the fp32 logits written out
    r = blk.moe._route(residual, want_logits=True)
    torch.cuda.synchronize()
    assert torch.equal(r["ids"], blk.moe.last["ids"])
    l32 = r["logits"].cpu().numpy()
    ids = r["ids"].cpu().numpy()
    assert np.array_equal(ids, oracle_selection(l32, w, inp.get("sel_bias")))
    wts = R.routing_weights(R.scores_f64(l32.astype(np.float64), w.score), ids, w.renorm)
    bargs = (np64(residual), np64(x_dense), ids, wts, np64(inp["w_gate_up"]), np64(inp["w_down"]),
             np64(dense["w_gate_up"]), np64(dense["w_down"]), np64(norms["g_pre_moe"]), np64(norms["g_post_dense"]),
             np64(norms["g_post_moe"]), np64(norms["g_post"]), 1e-6, 0.8)
    assert_close(np64(out), R.parallel_block_forward(*bargs, bf16=dtype == "bf16"), dtype, f"block {w.name} {dtype}")
    if dtype == "bf16":
        report_exact(np64(out), R.parallel_block_forward(*bargs), f"block {w.name} {dtype}")


def test_parallel_block_deterministic_and_scalar_linear():
    need_gpu()
    w, inp, blk, dense, norms, x_dense, residual = _block(CASES[0], "bf16")
    a = blk.forward(residual, x_dense).clone()
    b = blk.forward(residual, x_dense).clone()
    blk.layer_scalar = 1.6
    c = blk.forward(residual, x_dense)
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    # 1.6 = 2 * 0.8: the fp32 result before rounding doubles exactly
    assert torch.equal(c.float(), (2.0 * a.float()).to(c.dtype).float())
