"""Shared helpers of the GPU parity tests (imported by tests only)."""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from sparse_mixture_experts_route_amd import _lib as L
from sparse_mixture_experts_route_amd.layer import MoEFFN
from workloads import Workload

DTYPE_CODE = {"bf16": L.DTYPE_BF16, "fp32": L.DTYPE_FP32}


def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no HIP device")
    L.load()  # fail loudly when the library is missing


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def np64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def shape_of(w: Workload, T=None) -> L.MoeShape:
    return L.make_shape(w.T if T is None else T, w.H, w.E, w.k, w.I, w.Is, w.score, w.renorm,
                        w.shared_gated, DTYPE_CODE[w.dtype])


def make_layer(w: Workload, inp, T=None, fuse_gather=False, rate=1e-3) -> MoEFFN:
    params = {k: v for k, v in inp.items() if k not in ("x", "dout", "sel_bias")}
    bias = inp.get("sel_bias")
    return MoEFFN(shape_of(w, T), params, sel_bias=None if bias is None else bias.clone(), rate=rate,
                  fuse_gather=fuse_gather)


def bf16_tol(ref: np.ndarray) -> float:
    return 2e-2 * float(np.sqrt(np.mean(ref ** 2)))


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at each reference value: the error of storing the
    exact value itself in bf16 (8 significant bits)."""
    _, e = np.frexp(np.asarray(ref, np.float64))   # |ref| in [2^(e-1), 2^e)
    return np.where(ref != 0, np.ldexp(1.0, e - 9), 0.0)


def bf16_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max-abs error of a bf16 output beyond the correct rounding of the
    reference value to bf16."""
    return float(np.max(np.maximum(np.abs(got - ref) - bf16_half_ulp(ref), 0.0))) if ref.size else 0.0


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = ""):
    """fp32: max-abs <= 1e-5.  bf16 output: max-abs <= 2e-2 * RMS(ref),
    counting only the error beyond the bf16 rounding of each reference
    element (a correctly rounded result passes even where rounding an
    outlier alone exceeds the bound).  Pass dtype="fp32-acc" for an fp32
    tensor of a bf16 layer (bound 2e-2 * RMS, no rounding allowance)."""
    raw = float(np.max(np.abs(got - ref))) if ref.size else 0.0
    if dtype == "fp32":
        err, tol = raw, 1e-5
    elif dtype == "fp32-acc":
        err, tol = raw, bf16_tol(ref)
    else:
        err, tol = bf16_err(got, ref), bf16_tol(ref)
    assert err <= tol, f"{what}: max-abs {err:.3e} (raw {raw:.3e}) > tol {tol:.3e}"
    return err, tol


def oracle_selection(logits32: np.ndarray, w: Workload, bias):
    keys = R.selection_keys(logits32, w.score, None if bias is None else np64(bias).astype(np.float32))
    return R.topk_select(keys, w.k)


def sample_tokens(ids: np.ndarray, counts: np.ndarray, n: int, seed: int = 0) -> np.ndarray:
    """Seeded token subset that always holds the first and last token routed
    to the most loaded expert and tokens routed to the rarest used experts."""
    rng = np.random.default_rng(seed)
    T = ids.shape[0]
    picks = set(rng.choice(T, size=min(n, T), replace=False).tolist())
    e_max = int(np.argmax(counts))
    rows = np.nonzero((ids == e_max).any(axis=1))[0]
    if rows.size:
        picks.update([int(rows[0]), int(rows[-1])])
    used = np.nonzero(counts > 0)[0]
    rare = used[np.argsort(counts[used], kind="stable")[:4]]
    for e in rare:
        r = np.nonzero((ids == e).any(axis=1))[0]
        if r.size:
            picks.add(int(r[0]))
    return np.array(sorted(picks))


def oracle_tokens_forward(w: Workload, inp, ids, weights_f64, toks) -> np.ndarray:
    """Per-expert loop oracle on a token subset; weights fetched per expert."""
    x = np64(inp["x"][toks])
    out = np.zeros_like(x)
    sub_ids = ids[toks]
    for e in np.unique(sub_ids):
        t_idx, j_idx = np.nonzero(sub_ids == e)
        wgu = np64(inp["w_gate_up"][int(e)])
        wd = np64(inp["w_down"][int(e)])
        y = R.swiglu_mlp(x[t_idx], wgu, wd, w.dtype == "bf16")
        np.add.at(out, t_idx, weights_f64[toks][t_idx, j_idx][:, None] * y)
    if w.Is:
        wsg = np64(inp["w_shared_gate"]) if w.shared_gated else None
        out += R.shared_term(x, np64(inp["ws_gate_up"]), np64(inp["ws_down"]), wsg, w.dtype == "bf16")
    return out


def oracle_partial_rows(w, inp, sw, s, rows):
    """The share's MLP output for sorted rows `rows` (float64 oracle)."""
    offsets = s["offsets"].cpu().numpy()
    perm = s["perm"].cpu().numpy()
    x = np64(inp["x"])
    out = np.zeros((len(rows), w.H))
    e_of = np.searchsorted(offsets, rows, side="right") - 1
    for e in np.unique(e_of):
        sel = np.nonzero(e_of == e)[0]
        toks = perm[rows[sel]] // w.k
        out[sel] = R.swiglu_mlp(x[toks], np64(sw["w_gate_up"][int(e)]), np64(sw["w_down"][int(e)]),
                                w.dtype == "bf16")
    return out
