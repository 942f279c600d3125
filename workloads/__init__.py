"""Seeded synthetic workloads for the sparse MoE FFN layer.

This module is shared by the oracle-side tests and the HIP-side tests and
bench.  It holds shapes and random draws only: none of the layer's
arithmetic (routing, dispatch, expert MLPs, combine) lives here.

Workload shapes follow the five layer configurations the pages name:
  * the router contract and the fused checkpoint layout
    ``gate_up_proj (E, 2I, H)`` / ``down_proj (E, H, I)`` of
    "mstar.model.components.moe" (Router contract; SparseMoeBlock);
  * the routing shapes listed in "MoE: shared experts, parameterized V_TOPK
    routing, explicit stage attribution" (section 1, C_SET_TOPK_REG):
    Qwen2-MoE 60/top-4, DeepSeek-V2-Lite 64/top-6, DeepSeek-V3 256/top-8;
  * the DSV4-Flash MoE draft fields of "Sparse MoE FFN for DFlash-family
    drafters" (What's here: 64 routed + 1 shared, top-6,
    moe_intermediate_size 2048).

Draw recipe (per tensor, in this order, from one ``torch.Generator`` seeded
with the workload's seed): x, w_router, w_gate_up, w_down, shared gate_up,
shared down, shared gate, selection bias, dout.  Normal draws are made in
fp32 and rounded to the layer dtype (round-to-nearest-even for bf16).
Weights are N(0, 1/fan_in) (the second argument is a variance).  Large
stacked weights are drawn one expert at a time so the fp32 temporary stays
small.  Values drawn on a CUDA device differ from values drawn on the CPU
for the same seed; every parity test copies the device draw to the host.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import torch

SCORE_SOFTMAX = 0
SCORE_SIGMOID = 1
SCORE_SQRTSOFTPLUS = 2
SCORE_NAMES = {SCORE_SOFTMAX: "softmax", SCORE_SIGMOID: "sigmoid",
               SCORE_SQRTSOFTPLUS: "sqrtsoftplus"}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    T: int                # tokens
    H: int                # hidden size
    E: int                # routed experts
    k: int                # experts per token (top-k)
    I: int                # moe_intermediate_size
    Is: int = 0           # shared expert intermediate (0: no shared expert)
    score: int = SCORE_SOFTMAX
    renorm: bool = True   # norm_topk_prob
    shared_gated: bool = False
    dtype: str = "bf16"   # "bf16" or "fp32": x, weights, outputs
    bias_var: float = 0.0  # selection-bias variance (0: no bias)
    zipf: float = 0.0     # >0: Zipf(zipf) expert popularity via a constant feature
    seed: int = 0
    backward: bool = False

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)

    @property
    def torch_dtype(self) -> torch.dtype:
        return torch.bfloat16 if self.dtype == "bf16" else torch.float32

    @property
    def has_bias(self) -> bool:
        return self.bias_var > 0.0

    def fwd_flops(self) -> float:
        """Algorithmic forward GEMM flops: router (+gate logit), routed
        SwiGLU experts on the T*k selected rows, shared expert."""
        T, H, E, k, I, Is = self.T, self.H, self.E, self.k, self.I, self.Is
        gated = 1 if (Is and self.shared_gated) else 0
        return 2.0 * T * H * (E + gated) + 2.0 * T * k * 3 * H * I + 2.0 * T * 3 * H * Is


# The five layer configurations (tiny fp32, Qwen2-MoE-like, DSV4-Flash-draft-
# like, DeepSeek-V3-shaped, training of the Qwen2-MoE-like shape).
WORKLOADS: Dict[str, Workload] = {
    "tiny_fp32": Workload("tiny_fp32", T=64, H=128, E=8, k=2, I=256, Is=0,
                          score=SCORE_SOFTMAX, renorm=True, dtype="fp32", seed=0),
    "qwen2moe": Workload("qwen2moe", T=4096, H=2048, E=60, k=4, I=1408, Is=5632,
                         score=SCORE_SOFTMAX, renorm=False, shared_gated=True, seed=1),
    "dsv4flash": Workload("dsv4flash", T=8192, H=4096, E=64, k=6, I=2048, Is=2048,
                          score=SCORE_SQRTSOFTPLUS, renorm=True, bias_var=0.5, seed=2),
    "deepseekv3": Workload("deepseekv3", T=16384, H=7168, E=256, k=8, I=2048, Is=2048,
                           score=SCORE_SOFTMAX, renorm=True, zipf=1.1, seed=3),
    "qwen2moe_train": Workload("qwen2moe_train", T=8192, H=2048, E=60, k=4, I=1408,
                               Is=5632, score=SCORE_SOFTMAX, renorm=False,
                               shared_gated=True, seed=4, backward=True),
}
DECODE_TOKENS = (16, 64, 256)


def decode_workload(T: int) -> Workload:
    """Decode-shaped forward of the training shape at T tokens."""
    return WORKLOADS["qwen2moe_train"].with_(name=f"qwen2moe_decode_T{T}", T=T,
                                             backward=False, seed=5)


def _normal(g: torch.Generator, shape, std: float, dtype, device) -> torch.Tensor:
    t = torch.randn(shape, generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _stacked(g, E, rows, cols, std, dtype, device) -> torch.Tensor:
    out = torch.empty((E, rows, cols), dtype=dtype, device=device)
    for e in range(E):
        out[e].copy_(_normal(g, (rows, cols), std, dtype, device))
    return out


def zipf_log_popularity(E: int, s: float, g: torch.Generator) -> torch.Tensor:
    """log p_e for Zipf(s) popularity over a seeded permutation of ranks."""
    ranks = torch.randperm(E, generator=g, device=g.device).to(torch.float64) + 1.0
    logp = -s * torch.log(ranks)
    logp = logp - torch.logsumexp(logp, 0)
    return logp


def make_inputs(w: Workload, device="cpu", T: Optional[int] = None,
                seed: Optional[int] = None) -> Dict[str, torch.Tensor]:
    """Draw every input of one layer call.  Keys: x, w_router, w_gate_up,
    w_down, ws_gate_up, ws_down, w_shared_gate, sel_bias, dout (absent keys
    mean the feature is off)."""
    T = w.T if T is None else T
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(w.seed if seed is None else seed)
    dt = w.torch_dtype
    H, E, I, Is = w.H, w.E, w.I, w.Is
    out: Dict[str, torch.Tensor] = {}
    x = _normal(g, (T, H), 1.0, dt, device)
    w_router = _normal(g, (E, H), 1.0 / math.sqrt(H), dt, device)
    if w.zipf > 0.0:
        # A constant feature carries a per-expert log-popularity into every
        # logit, so expert loads follow Zipf(s) and some experts get none.
        x[:, 0] = 1.0
        logp = zipf_log_popularity(E, w.zipf, g)
        w_router[:, 0] = logp.to(device=device, dtype=torch.float32).to(dt)
    out["x"] = x
    out["w_router"] = w_router
    out["w_gate_up"] = _stacked(g, E, 2 * I, H, 1.0 / math.sqrt(H), dt, device)
    out["w_down"] = _stacked(g, E, H, I, 1.0 / math.sqrt(I), dt, device)
    if Is:
        out["ws_gate_up"] = _normal(g, (2 * Is, H), 1.0 / math.sqrt(H), dt, device)
        out["ws_down"] = _normal(g, (H, Is), 1.0 / math.sqrt(Is), dt, device)
        if w.shared_gated:
            out["w_shared_gate"] = _normal(g, (H,), 1.0 / math.sqrt(H), dt, device)
    if w.has_bias:
        out["sel_bias"] = _normal(g, (E,), math.sqrt(w.bias_var), torch.float32, device)
    if w.backward:
        out["dout"] = _normal(g, (T, H), 1.0, dt, device)
    return out


def exact_dyadic_inputs(T: int, H: int, E: int, I: int, Is: int = 0, seed: int = 0,
                        dtype=torch.bfloat16, device="cpu", gated: bool = False
                        ) -> Dict[str, torch.Tensor]:
    """Inputs on a coarse dyadic grid: x in {-4..4}/4, weights in {-4..4}/64.
    Every product is a multiple of 2^-8 and partial sums of up to 2^15 terms
    stay inside 24 significant bits, so an fp32 accumulation of x.W is exact
    in any order."""
    device = torch.device(device)
    g = torch.Generator(device=device)
    g.manual_seed(seed)

    def grid(shape, denom):
        v = torch.randint(-4, 5, shape, generator=g, device=device)
        return (v.to(torch.float32) / denom).to(dtype)

    out = {"x": grid((T, H), 4.0), "w_router": grid((E, H), 64.0),
           "w_gate_up": grid((E, 2 * I, H), 64.0), "w_down": grid((E, H, I), 64.0)}
    if Is:
        out["ws_gate_up"] = grid((2 * Is, H), 64.0)
        out["ws_down"] = grid((H, Is), 64.0)
        if gated:
            out["w_shared_gate"] = grid((H,), 64.0)
    return out
