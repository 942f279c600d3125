"""Pins for the oracle's parallel dense + MoE block (the DeepSpec issue
"Feat: Compatible with Gamme4 MoE structure", Decoder layer forward pass) and
its RMSNorm (CPU only).

RMSNorm: equals torch's own rms_norm; unit RMS and scale invariance with
eps = 0.  Block: zero final norm scale leaves residual * scalar; linear in the
layer scalar; the MoE branch sees only the normalised residual, so scaling
the residual by c > 0 moves the output by exactly c * residual * scalar
(a planted mistake that feeds the raw residual to the experts breaks it);
with a zero expert down projection the block reduces to torch rms_norm of the
dense MLP.
"""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R


def _block_inputs(seed=0, T=10, H=24, E=6, k=2, I=8, Id=16):
    rng = np.random.default_rng(seed)
    d = {"residual": rng.normal(0, 1.5, (T, H)), "x_dense": rng.normal(0, 1, (T, H)),
         "w_gate_up": rng.normal(0, H ** -0.5, (E, 2 * I, H)), "w_down": rng.normal(0, I ** -0.5, (E, H, I)),
         "wd_gate_up": rng.normal(0, H ** -0.5, (2 * Id, H)), "wd_down": rng.normal(0, Id ** -0.5, (H, Id)),
         "g_pre_moe": rng.uniform(0.5, 1.5, H), "g_post_dense": rng.uniform(0.5, 1.5, H),
         "g_post_moe": rng.uniform(0.5, 1.5, H), "g_post": rng.uniform(0.5, 1.5, H)}
    ids = np.array([rng.choice(E, k, replace=False) for _ in range(T)])
    w = rng.uniform(0.1, 1.0, (T, k))
    return d, ids, w / w.sum(axis=1, keepdims=True)


def _run(d, ids, w, eps=1e-6, scalar=0.75, residual=None, **kw):
    r = d["residual"] if residual is None else residual
    return R.parallel_block_forward(r, d["x_dense"], ids, w, d["w_gate_up"], d["w_down"], d["wd_gate_up"],
                                    d["wd_down"], d["g_pre_moe"], d["g_post_dense"], d["g_post_moe"],
                                    kw.get("g_post", d["g_post"]), eps, scalar, bf16=kw.get("bf16", False))


def test_rms_norm_equals_torch_and_closed_forms():
    rng = np.random.default_rng(1)
    v = rng.normal(0, 3, (7, 40))
    g = rng.uniform(0.5, 2.0, 40)
    got = R.rms_norm(v, g, 1e-5)
    ref = torch.nn.functional.rms_norm(torch.tensor(v), (40,), torch.tensor(g), 1e-5).numpy()
    assert np.max(np.abs(got - ref)) < 1e-12
    unit = R.rms_norm(v, np.ones(40), 0.0)
    assert np.max(np.abs(np.sqrt(np.mean(unit ** 2, axis=1)) - 1.0)) < 1e-14
    assert np.max(np.abs(R.rms_norm(3.5 * v, g, 0.0) - R.rms_norm(v, g, 0.0))) < 1e-13
    assert np.max(np.abs(R.rms_norm(-2.0 * v, g, 0.0) + R.rms_norm(v, g, 0.0))) < 1e-13
    # a constant row c gives c / sqrt(c^2 + eps) in every channel
    c = np.full((1, 40), 0.3)
    assert np.allclose(R.rms_norm(c, np.ones(40), 0.01), 0.3 / np.sqrt(0.09 + 0.01), rtol=0, atol=1e-15)


def test_block_identities():
    d, ids, w = _block_inputs()
    out = _run(d, ids, w)
    # zero final scale: only the residual is left
    assert np.array_equal(_run(d, ids, w, g_post=np.zeros(24)), d["residual"] * 0.75)
    # linear in the layer scalar (times 2 is exact in binary floating point)
    assert np.array_equal(_run(d, ids, w, scalar=1.5), 2.0 * out)
    assert not np.allclose(out, d["residual"] * 0.75)


@pytest.mark.parametrize("bf16", [False, True])
def test_moe_branch_sees_only_the_normalised_residual(bf16):
    """The router's ids and weights are held fixed; the experts read
    rms_norm(residual) (eps = 0), so scaling the residual by c > 0 changes
    the output by exactly c * residual * scalar up to rounding."""
    d, ids, w = _block_inputs(seed=3)
    c = 2.0   # a power of two keeps the bf16 rounding of the normalised input identical
    a = _run(d, ids, w, eps=0.0, bf16=bf16)
    b = _run(d, ids, w, eps=0.0, bf16=bf16, residual=c * d["residual"])
    assert np.max(np.abs((b - a) - (c - 1.0) * d["residual"] * 0.75)) < 1e-12
    # planted mistake: the first norm of the block (the experts' input) left
    # out, so the experts read the raw residual; the invariance breaks
    orig = R.rms_norm

    def skip_first(v, g, eps, calls=[0]):
        calls[0] += 1
        return np.asarray(v, np.float64) if calls[0] % 4 == 1 else orig(v, g, eps)
    R.rms_norm = skip_first
    try:
        bad_a = _run(d, ids, w, eps=0.0)
        bad_b = _run(d, ids, w, eps=0.0, residual=c * d["residual"])
    finally:
        R.rms_norm = orig
    assert np.max(np.abs((bad_b - bad_a) - (c - 1.0) * d["residual"] * 0.75)) > 1e-3


def test_block_with_silent_experts_is_the_normed_dense_mlp():
    d, ids, w = _block_inputs(seed=5)
    d["w_down"] = np.zeros_like(d["w_down"])
    out = _run(d, ids, w, eps=1e-6, scalar=1.0)
    t = lambda a: torch.tensor(np.asarray(a, np.float64))
    h1 = t(R.swiglu_mlp(d["x_dense"], d["wd_gate_up"], d["wd_down"]))
    F = torch.nn.functional
    ref = t(d["residual"]) + F.rms_norm(F.rms_norm(h1, (24,), t(d["g_post_dense"]), 1e-6), (24,),
                                          t(d["g_post"]), 1e-6)
    assert np.max(np.abs(out - ref.numpy())) < 1e-12
