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


def make_layer(w: Workload, inp, T=None, fuse_gather=True, rate=1e-3) -> MoEFFN:
    params = {k: v for k, v in inp.items() if k not in ("x", "dout", "sel_bias")}
    bias = inp.get("sel_bias")
    return MoEFFN(shape_of(w, T), params, sel_bias=None if bias is None else bias.clone(), rate=rate,
                  fuse_gather=fuse_gather)


def rms(a: np.ndarray) -> float:
    return float(np.sqrt(np.mean(np.asarray(a, np.float64) ** 2))) if np.size(a) else 0.0


def bf16_tol(ref: np.ndarray) -> float:
    """The bf16 bound: 2e-2 times the RMS of the reference tensor."""
    return 2e-2 * rms(ref)


def bf16_half_ulp(ref: np.ndarray) -> np.ndarray:
    """Half a bf16 ulp at each reference value: the largest error of storing
    a value of that binade in bf16 (8 significant bits)."""
    _, e = np.frexp(np.asarray(ref, np.float64))   # |ref| in [2^(e-1), 2^e)
    return np.where(ref != 0, np.ldexp(1.0, e - 9), 0.0)


def _at_max(d, ref, tol):
    """Where the largest error sits: the reference value there in units of
    the bound's RMS, and half a bf16 ulp of it in units of the bound."""
    i = int(np.argmax(d))
    r = float(np.asarray(ref).ravel()[i])
    if not tol:
        return f"at ref {r:+.3e}"
    return f"at ref {r / (tol / 2e-2):+.2f} rms (half bf16 ulp there {bf16_half_ulp(np.array(r)) / tol:.2f} tol)"


def gate_bf16(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """A tensor the layer stores in bf16: max-abs <= 2e-2 * RMS(ref).  One
    exception, confined to the elements it concerns: where half a bf16 ulp of
    the reference value exceeds the bound, no bf16 number need lie within the
    bound of it, so for those elements (counted and printed) the error beyond
    half an ulp is bounded instead.  Returns (error, tol, raw max-abs, number
    of such elements)."""
    tol = bf16_tol(ref)
    if not ref.size:
        return 0.0, tol, 0.0, 0
    d = np.abs(np.asarray(got, np.float64) - ref)
    half = bf16_half_ulp(ref)
    out = half > tol
    n_out = int(out.sum())
    e_in = float(d[~out].max()) if n_out < ref.size else 0.0
    e_out = float((d[out] - half[out]).max()) if n_out else 0.0
    raw = float(d.max())
    err = max(e_in, e_out)
    say(f"{what}: max-abs {raw:.3e} (tol {tol:.3e}, {raw / tol if tol else 0:.3f} of it) {_at_max(d, ref, tol)}; {n_out} of "
        f"{ref.size} elements where half a bf16 ulp exceeds the bound, error past half an ulp there {e_out:.3e}")
    assert err <= tol, f"{what}: max-abs {err:.3e} > tol {tol:.3e} (raw {raw:.3e}, {n_out} beyond bf16 reach)"
    return err, tol, raw, n_out


def gate_acc(got: np.ndarray, ref: np.ndarray, what: str = ""):
    """An fp32 tensor of a bf16 layer (weight gradients, logit gradients,
    partial rows): max-abs <= 2e-2 * RMS."""
    tol = bf16_tol(ref)
    err = float(np.max(np.abs(np.asarray(got, np.float64) - ref))) if ref.size else 0.0
    say(f"{what}: max-abs {err:.3e} (tol {tol:.3e}, {err / tol if tol else 0:.3f} of it)")
    assert err <= tol, f"{what}: max-abs {err:.3e} > tol {tol:.3e}"
    return err, tol


FP32_TOL = 1e-5
# fp32 tensors held to a stated larger bound (each measured; see the design
# notes' tolerance reading): the score column sums add T fp32 scores of the
# fixed fp32 recipe (a few ulp each, not unbiased); the router-weight and
# shared-gate weight gradients sum over T tokens a logit gradient or gate
# derivative formed from fp32 scores and gates.
FP32_EXCEPTIONS = {"score sums": 3e-5, "dw_router": 2e-5, "dw_shared_gate": 3e-5}


def gate_fp32(got: np.ndarray, ref: np.ndarray, what: str = "", tol: float = FP32_TOL):
    """A tensor of an fp32 layer against the exact float64 oracle: max-abs <=
    tol (1e-5).  Elements where half an fp32 ulp of the reference value alone
    exceeds tol (|ref| >= 256) are held to it beyond half an ulp."""
    if not ref.size:
        return 0.0, tol
    ref = np.asarray(ref, np.float64)
    d = np.abs(np.asarray(got, np.float64) - ref)
    _, e = np.frexp(ref)
    half = np.where(ref != 0, np.ldexp(1.0, e - 25), 0.0)
    out = half > tol
    err = float(np.max(np.where(out, d - half, d)))
    say(f"{what}: max-abs {float(d.max()):.3e} (tol {tol:.3e}, rms {rms(ref):.3e}, {int(out.sum())} elements past "
        f"fp32 reach)")
    assert err <= tol, f"{what}: max-abs {err:.3e} > tol {tol:.3e}"
    return err, tol


def assert_close(got: np.ndarray, ref: np.ndarray, dtype: str, what: str = "", tol: float = FP32_TOL):
    """The parity gate for one tensor.  dtype "fp32": a tensor of an fp32
    layer against the exact oracle (gate_fp32); "bf16": a tensor stored in
    bf16 (gate_bf16); "fp32-acc": an fp32 tensor of a bf16 layer (max-abs <=
    2e-2 * RMS).  Returns (error, tol)."""
    if dtype == "fp32":
        return gate_fp32(got, ref, what, tol)
    if dtype == "fp32-acc":
        return gate_acc(got, ref, what)
    return gate_bf16(got, ref, what)[:2]


def gate_tensor(got_t: torch.Tensor, ref: np.ndarray, layer_dtype: str, what: str = "", tol: float = FP32_TOL):
    """assert_close with the kind taken from the stored tensor's dtype."""
    got = np64(got_t)
    if layer_dtype == "fp32":
        return gate_fp32(got, ref, what, tol)
    if got_t.dtype == torch.bfloat16:
        return gate_bf16(got, ref, what)[:2]
    return gate_acc(got, ref, what)


def report_exact(got: np.ndarray, exact: np.ndarray, what: str = ""):
    """For the log: a bf16 layer's tensor against the exact (unrounded)
    oracle, in units of the 2e-2 * RMS bound."""
    if not exact.size:
        return
    tol = bf16_tol(exact)
    d = np.abs(np.asarray(got, np.float64) - exact)
    say(f"{what}: against the exact oracle max-abs {float(d.max()):.3e} = "
        f"{float(d.max()) / tol if tol else 0.0:.3f} of 2e-2 * RMS; {int((d > tol).sum())} of {d.size} elements above it")


def report_model(got: np.ndarray, model: np.ndarray, what: str = ""):
    """For the log: distance from the oracle's operand-rounding model, in
    units of the 2e-2 * RMS bound."""
    if not model.size:
        return
    tol = bf16_tol(model)
    d = float(np.max(np.abs(np.asarray(got, np.float64) - model)))
    say(f"{what}: against the operand-rounding model max-abs {d:.3e} = {d / tol if tol else 0.0:.3f} of 2e-2 * RMS")


def gate_out_exact(got: np.ndarray, exact: np.ndarray, what: str = ""):
    """A bf16 layer's output against the exact (unrounded) float64 oracle:
    max-abs <= 2e-2 * RMS, half a bf16 ulp allowed only on elements where
    that alone exceeds the bound."""
    return gate_bf16(got, exact, what + " [exact oracle]")


GRADS = [("dx", "dx"), ("dw_router", "dw_router"), ("dw_gate_up", "dw_gate_up"), ("dw_down", "dw_down"),
         ("dws_gate_up", "dws_gate_up"), ("dws_down", "dws_down"), ("dw_shared_gate", "dw_shared_gate"),
         ("dlogits", "dlogits")]


STACKED = ("dw_gate_up", "dw_down")


TIE_REL = 2.0 ** -16


def tie_ulp(v: np.ndarray) -> np.ndarray:
    """One bf16 ulp where v lies within TIE_REL (relative) of a bf16 rounding
    midpoint, else 0.  A GPU that rounds such an operand from its own fp32
    value (a few fp32 ulp from the exact one) may correctly land on either
    neighbour, one bf16 ulp apart."""
    v = np.asarray(v, np.float64)
    _, e = np.frexp(v)
    ulp = np.ldexp(1.0, e - 8)               # 8 significant bits
    q = np.abs(v) / ulp
    dist = np.abs(q - np.floor(q) - 0.5) * ulp
    return np.where((v != 0) & (dist <= TIE_REL * np.abs(v)), ulp, 0.0)


def gate_with_ties(got: np.ndarray, ref: np.ndarray, allow: np.ndarray, what: str = ""):
    """fp32 weight gradients of a bf16 layer against the operand-rounding
    model: |got - ref| <= 2e-2 * RMS(ref) + allow elementwise, where allow
    propagates one bf16 ulp of every operand the model rounds from within
    TIE_REL of a midpoint (see tie_ulp).  Logs how many elements needed it."""
    tol = bf16_tol(ref)
    d = np.abs(got - ref)
    over = d > tol
    excess = float(np.max(d - allow)) if ref.size else 0.0
    say(f"{what}: max-abs {float(d.max()):.3e} = {float(d.max()) / tol:.3f} of 2e-2 * RMS; {int(over.sum())} of "
        f"{d.size} elements above it, all within the tie allowance: {bool(np.all(d <= tol + allow))} "
        f"(largest error past the allowance {excess / tol:.3f} of the bound)")
    assert np.all(d <= tol + allow), f"{what}: {int((d > tol + allow).sum())} elements beyond 2e-2 * RMS + ties"


def check_grads(w, g, ref, tag, names=None, exact=None):
    """Every gradient tensor against the oracle's (for a bf16 layer: its
    operand-rounding model); all failures are collected and reported
    together.  exact: the unrounded oracle's gradients, reported beside."""
    fails = []
    for gk, rk in GRADS:
        if (names is not None and gk not in names) or gk not in g or rk not in ref:
            continue
        try:
            gate_tensor(g[gk], ref[rk], w.dtype, f"{tag} {gk}", tol=FP32_EXCEPTIONS.get(gk, FP32_TOL))
        except AssertionError as e:
            fails.append(str(e))
        if exact is not None and w.dtype == "bf16" and rk in exact:
            report_exact(np64(g[gk]), exact[rk], f"{tag} {gk}")
    assert not fails, "; ".join(fails)


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


def oracle_tokens_forward(w: Workload, inp, ids, weights_f64, toks, bf16: bool = False) -> np.ndarray:
    """Per-expert loop oracle on a token subset; weights fetched per expert.
    bf16=True: the operand-rounding model of a bf16 layer."""
    x = np64(inp["x"][toks])
    out = np.zeros_like(x)
    sub_ids = ids[toks]
    for e in np.unique(sub_ids):
        t_idx, j_idx = np.nonzero(sub_ids == e)
        wgu = np64(inp["w_gate_up"][int(e)])
        wd = np64(inp["w_down"][int(e)])
        y = R.swiglu_mlp(x[t_idx], wgu, wd, bf16)
        np.add.at(out, t_idx, weights_f64[toks][t_idx, j_idx][:, None] * y)
    if w.Is:
        wsg = np64(inp["w_shared_gate"]) if w.shared_gated else None
        out += R.shared_term(x, np64(inp["ws_gate_up"]), np64(inp["ws_down"]), wsg, bf16)
    return out


def oracle_partial_rows(w, inp, sw, s, rows, bf16: bool = False):
    """The share's MLP output for sorted rows `rows` (float64 oracle;
    bf16=True: the operand-rounding model)."""
    offsets = s["offsets"].cpu().numpy()
    perm = s["perm"].cpu().numpy()
    x = np64(inp["x"])
    out = np.zeros((len(rows), w.H))
    e_of = np.searchsorted(offsets, rows, side="right") - 1
    for e in np.unique(e_of):
        sel = np.nonzero(e_of == e)[0]
        toks = perm[rows[sel]] // w.k
        out[sel] = R.swiglu_mlp(x[toks], np64(sw["w_gate_up"][int(e)]), np64(sw["w_down"][int(e)]), bf16)
    return out
