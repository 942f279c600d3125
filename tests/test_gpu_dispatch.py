"""GPU parity of the counting-sort dispatch (moe_dispatch) and of the
balance counts (moe_balance_counts): bit-exact against the oracle."""
import numpy as np
import pytest
import torch

from oracle import moe_ref as R
from sparse_mixture_experts_route_amd import _lib as L

from gpu_helpers import need_gpu

pytestmark = pytest.mark.gpu


def _ids(kind, T, E, k, rng):
    if T == 0:
        return np.zeros((0, k), np.int64)
    if kind == "uniform":
        return np.array([rng.permutation(E)[:k] for _ in range(T)], np.int64).reshape(T, k)
    if kind == "zipf":
        p = 1.0 / np.arange(1, E + 1) ** 1.1
        p /= p.sum()
        out = np.zeros((T, k), np.int64)
        for t in range(T):
            out[t] = rng.choice(E, size=k, replace=False, p=p)
        return out
    if kind == "one_expert_heavy":   # many empty experts, one huge segment
        out = np.array([rng.permutation(min(E, k + 2))[:k] for _ in range(T)], np.int64).reshape(T, k)
        return out
    raise ValueError(kind)


# up to 512 pairs the one-launch path runs; (128, 60, 4) and (64, 256, 8) are
# its largest case, (129, 60, 4) the smallest of the three-kernel path
@pytest.mark.parametrize("T,E,k", [(0, 8, 2), (1, 8, 2), (7, 60, 4), (1000, 64, 6), (3000, 256, 8),
                                   (171, 16, 1), (2048, 60, 4), (4097, 64, 6), (128, 60, 4), (129, 60, 4),
                                   (64, 256, 8)])
@pytest.mark.parametrize("kind", ["uniform", "zipf", "one_expert_heavy"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_dispatch_bit_exact(T, E, k, kind, dtype):
    need_gpu()
    rng = np.random.default_rng(T * 31 + E + k)
    ids = _ids(kind, T, E, k, rng)
    H = 136
    dev = torch.device("cuda")
    sh = L.make_shape(T, H, E, k, 64, 0, 0, True, False, L.DTYPE_BF16 if dtype == torch.bfloat16 else L.DTYPE_FP32)
    x = torch.randn((max(T, 1), H), device=dev).to(dtype)[:T]
    ids_t = torch.tensor(ids, device=dev)
    P = T * k
    counts = torch.full((E,), -7, dtype=torch.int32, device=dev)
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device=dev)
    perm = torch.full((max(P, 1),), -7, dtype=torch.int32, device=dev)
    pos = torch.full((max(P, 1),), -7, dtype=torch.int32, device=dev)
    xs = torch.empty((max(P, 1), H), dtype=dtype, device=dev)
    ws = torch.empty(L.workspace_bytes(sh, L.OP_DISPATCH), dtype=torch.uint8, device=dev)
    L.moe_dispatch(sh, ids_t if T else None, x, counts, offsets, perm, pos, xs, ws)
    torch.cuda.synchronize()
    ref = R.dispatch(ids, E)
    assert np.array_equal(counts.cpu().numpy(), ref["counts"])
    assert np.array_equal(offsets.cpu().numpy(), ref["offsets"])
    if P:
        assert np.array_equal(perm.cpu().numpy()[:P], ref["perm"])
        assert np.array_equal(pos.cpu().numpy()[:P], ref["pos"])
        tok = torch.tensor(ref["perm"] // k, device=dev)
        assert torch.equal(xs[:P], x[tok])        # the gather is an exact copy
    # balance counts give the same histogram; the bias moves by sign(mean - c)
    c2 = torch.zeros((E,), dtype=torch.int32, device=dev)
    bias = torch.linspace(-1, 1, E, device=dev)
    b0 = bias.cpu().numpy().copy()
    L.moe_balance_counts(sh, ids_t if T else None, c2, bias, 1e-3)
    torch.cuda.synchronize()
    assert np.array_equal(c2.cpu().numpy(), ref["counts"])
    assert np.array_equal(bias.cpu().numpy(), R.balance_update(b0, ref["counts"], 1e-3, P))


def test_balance_from_stashed_counts():
    need_gpu()
    E, T, k = 8, 16, 2
    dev = torch.device("cuda")
    sh = L.make_shape(T, 64, E, k, 64)
    counts = torch.tensor([8, 4, 4, 4, 4, 4, 2, 2], dtype=torch.int32, device=dev)
    bias = torch.zeros(E, device=dev)
    L.moe_balance_counts(sh, None, counts, bias, 1e-3)
    torch.cuda.synchronize()
    want = R.balance_update(np.zeros(E, np.float32), counts.cpu().numpy(), 1e-3, T * k)
    assert np.array_equal(bias.cpu().numpy(), want)
    # equal loads leave the bias unchanged
    L.moe_balance_counts(sh, None, torch.full((E,), 4, dtype=torch.int32, device=dev), bias, 1e-3)
    torch.cuda.synchronize()
    assert np.array_equal(bias.cpu().numpy(), want)


def test_dispatch_deterministic():
    need_gpu()
    rng = np.random.default_rng(1)
    T, E, k = 20000, 64, 6
    ids = torch.tensor(_ids("uniform", T, E, k, rng), device="cuda")
    sh = L.make_shape(T, 64, E, k, 64)
    ws = torch.empty(L.workspace_bytes(sh, L.OP_DISPATCH), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(2):
        o = [torch.empty(n, dtype=torch.int32, device="cuda") for n in (E, E + 1, T * k, T * k)]
        L.moe_dispatch(sh, ids, None, *o, None, ws)
        outs.append(o)
    torch.cuda.synchronize()
    for a, b in zip(*outs):
        assert torch.equal(a, b)


ROUTE_DISPATCH = [
    # T, H, E, k, gated, dtype, score, with_bias
    (0, 256, 8, 2, False, torch.bfloat16, 0, False),
    (1, 256, 8, 2, True, torch.bfloat16, 0, False),
    (16, 2048, 60, 4, True, torch.bfloat16, 0, False),       # split reduction over H; one tile: the router sorts
    (12, 2048, 64, 6, False, torch.bfloat16, 2, True),       # one tile, ragged
    (32, 1024, 256, 8, False, torch.bfloat16, 0, False),     # one 32-token tile of 256 experts: 256 pairs
    (24, 512, 140, 4, True, torch.bfloat16, 1, False),       # two tiles: the sort kernel
    (300, 320, 12, 3, False, torch.bfloat16, 1, False),
    (2048, 1024, 64, 6, False, torch.bfloat16, 2, True),     # multi-tile batches from here
    (4097, 512, 60, 4, True, torch.bfloat16, 0, False),      # ragged last tile
    (8192, 512, 64, 6, False, torch.bfloat16, 2, True),
    (8192, 4096, 64, 6, False, torch.bfloat16, 2, True),     # the DSV4-Flash layer's router
    (3000, 256, 256, 8, False, torch.bfloat16, 0, False),    # router as a GEMM (more than 80 columns)
    (2500, 2048, 120, 4, True, torch.bfloat16, 1, True),     # the same with a gate row and a split over H
    (1000, 264, 80, 4, True, torch.bfloat16, 0, False),      # register-staged router (H % 64 != 0)
    (777, 128, 32, 4, False, torch.float32, 1, False),
]


@pytest.mark.parametrize("case", ROUTE_DISPATCH, ids=[f"T{c[0]}_E{c[2]}_k{c[3]}" for c in ROUTE_DISPATCH])
@pytest.mark.parametrize("logits_in", [False, True])
def test_route_dispatch_equals_route_then_dispatch(case, logits_in):
    """moe_route_dispatch (router tiles count their selections; one kernel
    sorts from those counts) writes exactly what moe_route followed by
    moe_dispatch writes: weights, ids, logits, gate, score sums, counts,
    offsets, perm and pos, bit for bit; and the permutation is the oracle's
    stable sort."""
    need_gpu()
    T, H, E, k, gated, dtype, score, with_bias = case
    if logits_in and gated:
        pytest.skip("the gate needs x")
    dev = torch.device("cuda")
    g = torch.Generator(device="cuda").manual_seed(T * 7 + E)
    x = torch.randn((max(T, 1), H), generator=g, device="cuda").to(dtype)[:T]
    wr = (torch.randn((E, H), generator=g, device="cuda") / H ** 0.5).to(dtype)
    wg = (torch.randn((H,), generator=g, device="cuda") / H ** 0.5).to(dtype) if gated else None
    bias = torch.randn((E,), generator=g, device="cuda") * 0.5 if with_bias else None
    lin = torch.randn((max(T, 1), E), generator=g, device="cuda")[:T].contiguous() if logits_in else None
    sh = L.make_shape(T, H, E, k, 64, 64 if gated else 0, score, True, gated,
                      L.DTYPE_BF16 if dtype == torch.bfloat16 else L.DTYPE_FP32)
    P = T * k
    flags = L.ROUTE_LOGITS_IN if logits_in else 0

    def bufs():
        return {"logits": lin if logits_in else torch.full((max(T, 1), E), 7.0, device=dev)[:T],
                "weights": torch.full((max(T, 1), k), 7.0, device=dev)[:T],
                "ids": torch.full((max(T, 1), k), -7, dtype=torch.int64, device=dev)[:T],
                "gate": torch.full((max(T, 1),), 7.0, device=dev)[:T] if gated else None,
                "sums": torch.full((E,), 7.0, device=dev),
                "counts": torch.full((E,), -7, dtype=torch.int32, device=dev),
                "offsets": torch.full((E + 1,), -7, dtype=torch.int32, device=dev),
                "perm": torch.full((max(P, 1),), -7, dtype=torch.int32, device=dev),
                "pos": torch.full((max(P, 1),), -7, dtype=torch.int32, device=dev)}
    a, b = bufs(), bufs()
    xx, ww = (None, None) if logits_in else (x, wr)
    rws = torch.empty((max(L.workspace_bytes(sh, L.OP_ROUTE), 256),), dtype=torch.uint8, device=dev)
    L.moe_route(sh, xx, ww, wg, bias, a["logits"], a["weights"], a["ids"], a["gate"], flags=flags,
                score_sums=a["sums"], ws=rws)
    dws = torch.empty((L.workspace_bytes(sh, L.OP_DISPATCH),), dtype=torch.uint8, device=dev)
    L.moe_dispatch(sh, a["ids"] if T else None, None, a["counts"], a["offsets"], a["perm"], a["pos"], None, dws)
    fws = torch.empty((L.workspace_bytes(sh, L.OP_ROUTE_DISPATCH),), dtype=torch.uint8, device=dev)
    L.moe_route_dispatch(sh, xx, ww, wg, bias, b["logits"], b["weights"], b["ids"], b["gate"], b["counts"],
                         b["offsets"], b["perm"], b["pos"], fws, flags=flags, score_sums=b["sums"])
    torch.cuda.synchronize()
    for key in a:
        if a[key] is not None:
            assert torch.equal(a[key], b[key]), key
    ref = R.dispatch(a["ids"].cpu().numpy(), E)
    assert np.array_equal(b["counts"].cpu().numpy(), ref["counts"])
    assert np.array_equal(b["perm"].cpu().numpy()[:P], ref["perm"])
