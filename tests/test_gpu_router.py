"""GPU parity of the router (moe_route) and of the fixed fp32 score recipe.

ids must equal the oracle's selection bit for bit given the GPU's own fp32
logits; logits within fp32 accumulation error (bitwise for exact-dyadic
inputs); weights and gate within fp32 rounding.
"""
import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from oracle import score_f32 as SF
from sparse_mixture_experts_route_amd import _lib as L
from workloads import exact_dyadic_inputs

from gpu_helpers import need_gpu, np64, say

pytestmark = pytest.mark.gpu

ROUTING_SHAPES = [(8, 2), (16, 1), (32, 4), (60, 4), (64, 6), (128, 8), (256, 8)]


def _route(T, H, E, k, score, renorm, dtype, x, wr, bias=None, wg=None, logits_in=None, scratch=False):
    dev = torch.device("cuda")
    sh = L.make_shape(T, H, E, k, 64, 64 if wg is not None else 0, score, renorm, wg is not None,
                      L.DTYPE_BF16 if dtype == torch.bfloat16 else L.DTYPE_FP32)
    weights = torch.empty((T, k), dtype=torch.float32, device=dev)
    ids = torch.empty((T, k), dtype=torch.int64, device=dev)
    gate = torch.empty((T,), dtype=torch.float32, device=dev) if wg is not None else None
    if logits_in is not None:
        L.moe_route(sh, None, None, None, bias, logits_in, weights, ids, None, flags=L.ROUTE_LOGITS_IN)
        logits = logits_in
    else:
        logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        ws = None
        if scratch:
            ws = torch.empty((max(L.workspace_bytes(sh, L.OP_ROUTE), 256),), dtype=torch.uint8, device=dev)
        L.moe_route(sh, x, wr, wg, bias, logits, weights, ids, gate, ws=ws)
    torch.cuda.synchronize()
    return logits, weights, ids, gate


@pytest.mark.parametrize("E,k", ROUTING_SHAPES)
@pytest.mark.parametrize("score", [0, 1, 2])
@pytest.mark.parametrize("with_bias", [False, True])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("H", [264, 320])
def test_router_parity(E, k, score, with_bias, dtype, H):
    need_gpu()
    # T ragged against the 16- and 32-token tiles; H = 264 takes the register-
    # staged bf16 kernel (K not a multiple of 64), H = 320 the LDS-ring one
    T = 100
    g = torch.Generator(device="cuda").manual_seed(E * 7 + k + score)
    x = torch.randn((T, H), generator=g, device="cuda").to(dtype)
    wr = (torch.randn((E, H), generator=g, device="cuda") / H ** 0.5).to(dtype)
    bias = (torch.randn((E,), generator=g, device="cuda") * 0.7) if with_bias else None
    for renorm in (False, True):
        logits, weights, ids, _ = _route(T, H, E, k, score, renorm, dtype, x, wr, bias)
        l_gpu = logits.cpu().numpy()
        # logits within fp32 accumulation error of the float64 product
        xr, wrr = np64(x), np64(wr)
        ref = R.router_logits(xr, wrr)
        bound = 2.0 * H * 2.0 ** -24 * (np.abs(xr) @ np.abs(wrr).T) + 1e-30
        assert np.all(np.abs(l_gpu - ref) <= bound)
        # ids bit-exact given the GPU's fp32 logits
        b32 = None if bias is None else bias.cpu().numpy()
        want = R.topk_select(R.selection_keys(l_gpu, score, b32), k)
        got = ids.cpu().numpy()
        assert np.array_equal(got, want), f"{np.argwhere(got != want)[:5]}"
        wref = R.routing_weights(R.scores_f64(l_gpu.astype(np.float64), score), want, renorm)
        assert np.max(np.abs(weights.cpu().numpy() - wref)) < 2e-6
    if with_bias:
        # the bias is not vacuous: it changes the selection of some tokens
        nobias = R.topk_select(R.selection_keys(l_gpu, score, None), k)
        if k < E:
            assert not np.array_equal(nobias, want)


def test_router_exact_dyadic_logits_bitwise():
    need_gpu()
    for E, k in ((64, 6), (256, 8)):
        inp = exact_dyadic_inputs(96, 2048, E, 8, seed=E, device="cuda")
        logits, _, ids, _ = _route(96, 2048, E, k, 0, True, torch.bfloat16, inp["x"], inp["w_router"])
        ref = R.router_logits(np64(inp["x"]), np64(inp["w_router"])).astype(np.float32)
        assert np.array_equal(logits.cpu().numpy(), ref)
        assert np.array_equal(ids.cpu().numpy(), R.topk_select(ref, k))


@pytest.mark.parametrize("E,k", ROUTING_SHAPES)
def test_router_logits_in_ties_and_last_expert(E, k):
    """Tie-heavy integer logits: ties go to the lower index; forcing expert
    E-1 selects it (256 experts select expert 255)."""
    need_gpu()
    rng = np.random.default_rng(E + k)
    T = 70
    l = rng.integers(-1, 2, (T, E)).astype(np.float32)
    l[5, E - 1] = 9.0
    l[6] = -0.0
    l[6, ::2] = 0.0
    lt = torch.tensor(l, device="cuda")
    for score in (0, 1, 2):
        _, weights, ids, _ = _route(T, 64, E, k, score, True, torch.bfloat16, None, None, logits_in=lt)
        got = ids.cpu().numpy()
        want = R.topk_select(R.selection_keys(l, score, None), k)
        assert np.array_equal(got, want)
        assert got[5, 0] == E - 1
        assert list(got[6]) == list(range(k))  # all keys equal (+0 and -0): lowest indices
        if E <= 16:
            assert np.array_equal(got, R.topk_bruteforce(l, k))
        assert np.allclose(weights.cpu().numpy().sum(-1), 1.0, atol=1e-6)


@pytest.mark.parametrize("E,k,H", [(60, 4, 512), (64, 6, 512), (256, 8, 512), (140, 4, 264)])
def test_router_shared_gate(E, k, H):
    need_gpu()
    T = 77
    g = torch.Generator(device="cuda").manual_seed(3)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    wr = (torch.randn((E, H), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16)
    wg = (torch.randn((H,), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16)
    logits, weights, ids, gate = _route(T, H, E, k, 0, False, torch.bfloat16, x, wr, wg=wg)
    ref = R.shared_gate(np64(x), np64(wg))
    gv = gate.cpu().numpy()
    assert np.max(np.abs(gv - ref)) < 2e-6
    assert np.all((gv > 0) & (gv < 1))        # interior: the gate is exercised
    # the extra gate column does not disturb routing
    want = R.topk_select(R.selection_keys(logits.cpu().numpy(), 0, None), k)
    assert np.array_equal(ids.cpu().numpy(), want)


@pytest.mark.parametrize("T", [1, 16, 37, 256, 1000])
@pytest.mark.parametrize("E,k,gated", [(60, 4, True), (64, 6, False), (140, 4, True), (256, 8, False)])
def test_router_split_reduction(T, E, k, gated):
    """With scratch, short batches split the reduction over H across
    workgroups and add the partial tiles in split order (T = 1000 still splits
    in two: 63 tiles of 16 tokens).  Same contract as the one-pass router:
    logits within fp32 accumulation error, ids exact given the GPU's logits,
    weights and gate within fp32 rounding, identical bits on a second call."""
    need_gpu()
    H = 2048
    g = torch.Generator(device="cuda").manual_seed(T * 3 + E)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    wr = (torch.randn((E, H), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16)
    wg = (torch.randn((H,), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16) if gated else None
    bias = torch.randn((E,), generator=g, device="cuda") * 0.5
    xr, wrr = np64(x), np64(wr)
    ref = R.router_logits(xr, wrr)
    bound = 2.0 * H * 2.0 ** -24 * (np.abs(xr) @ np.abs(wrr).T) + 1e-30
    runs = [_route(T, H, E, k, 2, True, torch.bfloat16, x, wr, bias, wg, scratch=s) for s in (True, False, True)]
    for logits, weights, ids, gate in runs[:2]:
        l_gpu = logits.cpu().numpy()
        assert np.all(np.abs(l_gpu - ref) <= bound)
        want = R.topk_select(R.selection_keys(l_gpu, 2, bias.cpu().numpy()), k)
        assert np.array_equal(ids.cpu().numpy(), want)
        wref = R.routing_weights(R.scores_f64(l_gpu.astype(np.float64), 2), want, True)
        assert np.max(np.abs(weights.cpu().numpy() - wref)) < 2e-6
        if gated:
            assert np.max(np.abs(gate.cpu().numpy() - R.shared_gate(xr, np64(wg)))) < 2e-6
    for a, b in zip(runs[0], runs[2]):
        if a is not None:
            assert torch.equal(a, b)


@pytest.mark.parametrize("T,H,E,k,gated,score", [
    (2048, 1024, 96, 6, False, 2),     # 8 m-tiles, the reduction over H split in two
    (2085, 2048, 100, 4, True, 0),     # ragged; gate row and filler rows copied; split in four
    (4133, 4096, 256, 8, False, 1),    # 256 experts read in place, 32-token selection tiles, split in eight
    (2048, 512, 140, 4, True, 2),      # 144 columns, no split
    (2050, 1024, 256, 8, True, 0),     # 257 columns: two column tiles
])
def test_router_gemm_form(T, H, E, k, gated, score):
    """Batches of 2048 tokens and more with more than 80 columns (bf16, H %
    64 == 0, with scratch) take the logits as a GEMM on the 256x256 engine,
    its reduction over H split
    into fp32 partials that the selection adds in split order.  Same contract
    as the other forms: logits within fp32 accumulation error, ids exact given
    the GPU's logits, weights and gate within fp32 rounding, identical bits on
    a second call."""
    _check_prefill_router(T, H, E, k, gated, score)


@pytest.mark.parametrize("T,H,E,k,gated,score", [
    (2048, 1024, 64, 6, False, 2),     # 128 tiles of 16 tokens
    (2085, 2048, 60, 4, True, 0),      # ragged last tile; 61 columns with the gate row
    (4133, 512, 48, 4, False, 1),      # 48 columns
    (4096, 2048, 60, 4, True, 1),      # the Qwen2-MoE layer's router
    (8192, 4096, 64, 6, False, 2),     # the DSV4-Flash layer's router
])
def test_router_prefill_narrow(T, H, E, k, gated, score):
    """Prefill batches with at most 64 columns (bf16, H % 64 == 0): the
    LDS-ring kernel, each wave selecting four tokens at once.  Same contract
    as the other forms, with and without scratch."""
    _check_prefill_router(T, H, E, k, gated, score)
    _check_prefill_router(T, H, E, k, gated, score, scratch=False)


def _check_prefill_router(T, H, E, k, gated, score, scratch=True):
    need_gpu()
    g = torch.Generator(device="cuda").manual_seed(T + 5 * E)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    wr = (torch.randn((E, H), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16)
    wg = (torch.randn((H,), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16) if gated else None
    bias = torch.randn((E,), generator=g, device="cuda") * 0.5
    xr, wrr = np64(x), np64(wr)
    ref = R.router_logits(xr, wrr)
    bound = 2.0 * H * 2.0 ** -24 * (np.abs(xr) @ np.abs(wrr).T) + 1e-30
    runs = [_route(T, H, E, k, score, True, torch.bfloat16, x, wr, bias, wg, scratch=scratch) for _ in range(2)]
    logits, weights, ids, gate = runs[0]
    l_gpu = logits.cpu().numpy()
    assert np.all(np.abs(l_gpu - ref) <= bound)
    want = R.topk_select(R.selection_keys(l_gpu, score, bias.cpu().numpy()), k)
    assert np.array_equal(ids.cpu().numpy(), want)
    wref = R.routing_weights(R.scores_f64(l_gpu.astype(np.float64), score), want, True)
    assert np.max(np.abs(weights.cpu().numpy() - wref)) < 2e-6
    if gated:
        assert np.max(np.abs(gate.cpu().numpy() - R.shared_gate(xr, np64(wg)))) < 2e-6
    for a, b in zip(runs[0], runs[1]):
        if a is not None:
            assert torch.equal(a, b)


def test_router_deterministic():
    need_gpu()
    T, H, E, k = 1000, 1024, 64, 6
    g = torch.Generator(device="cuda").manual_seed(9)
    x = torch.randn((T, H), generator=g, device="cuda").to(torch.bfloat16)
    wr = (torch.randn((E, H), generator=g, device="cuda") / H ** 0.5).to(torch.bfloat16)
    b = torch.randn((E,), generator=g, device="cuda")
    a = _route(T, H, E, k, 2, True, torch.bfloat16, x, wr, b)
    c = _route(T, H, E, k, 2, True, torch.bfloat16, x, wr, b)
    for u, v in zip(a[:3], c[:3]):
        assert torch.equal(u, v)


def _oracle_chunk(score, lo, n):
    bits = np.arange(lo, lo + n, dtype=np.uint64).astype(np.uint32)
    v = bits.view(np.float32)
    if score == 0:
        return SF.exp32(v)
    if score == 1:
        return SF.sigmoid32(v)
    return SF.sqrtsoftplus32(v)


def _sweep(score, chunk_ids):
    chunk = 1 << 24
    workers = min(16, len(os.sched_getaffinity(0)))
    bad = 0
    done = 0
    with ThreadPoolExecutor(max_workers=workers) as ex:
        for b0 in range(0, len(chunk_ids), workers):
            starts = [c * chunk for c in chunk_ids[b0:b0 + workers]]
            futs = [ex.submit(_oracle_chunk, score, s0, chunk) for s0 in starts]
            for s0, f in zip(starts, futs):
                want = f.result()
                host = np.arange(s0, s0 + chunk, dtype=np.uint64).astype(np.uint32).view(np.float32)
                lv = torch.from_numpy(host).to("cuda")
                out = torch.empty_like(lv)
                L.moe_score_f32(score, lv, out)
                got = out.cpu().numpy()
                same = (got.view(np.uint32) == want.view(np.uint32)) | (np.isnan(got) & np.isnan(want))
                bad += int((~same).sum())
                done += 1
            say(f"score {score}: {done}/{len(chunk_ids)} chunks of 2^24 bit patterns checked, mismatches {bad}")
    return bad


@pytest.mark.parametrize("quarter", [0, 1, 2, 3])
@pytest.mark.parametrize("score", [1, 2, 0])
def test_score_recipe_matches_oracle_on_every_fp32(score, quarter):
    """The kernel's fp32 score recipe equals the oracle's bit for bit on every
    fp32 bit pattern: each test covers one quarter of the 2^32 patterns (64
    blocks of 2^24 consecutive ones), so the four quarters of a score cover
    all of them (positive and negative, normal, subnormal, inf, NaN)."""
    need_gpu()
    assert _sweep(score, list(range(64 * quarter, 64 * (quarter + 1)))) == 0
