"""Pins for the oracle's fixed fp32 score recipe (CPU only).

The recipe is pinned against float64 library functions (accuracy within a
few ulp over dense samples of the fp32 line), special values and closed
forms; the summation order of the softmax denominator is pinned by a
hand-derived case where the order changes the rounded result.
"""
import math

import numpy as np
import pytest

from oracle import score_f32 as sf

F32 = np.float32


def _ulp_dist(a, b):
    """Distance in units in the last place between fp32 arrays (finite)."""
    ai = a.astype(np.float32).view(np.int32).astype(np.int64)
    bi = b.astype(np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def _float_range(lo, hi, stride):
    """Every stride-th fp32 value in [lo, hi] by bit pattern."""
    lo, hi = F32(lo), F32(hi)
    vals = []
    for a, b in ((lo, min(hi, F32(-0.0))), (max(lo, F32(0.0)), hi)):
        if a > b:
            continue
        ia = np.array([abs(a)], np.float32).view(np.uint32)[0]
        ib = np.array([abs(b)], np.float32).view(np.uint32)[0]
        lo_i, hi_i = min(ia, ib), max(ia, ib)
        bits = np.arange(lo_i, hi_i + 1, stride, dtype=np.uint64).astype(np.uint32)
        v = bits.view(np.float32)
        vals.append(-v if a < 0 else v)
    return np.concatenate(vals)


def test_constants_split_ln2():
    # C1 has at most 16 significant bits so n*C1 is exact for |n| < 256,
    # and C1 + C2 reproduces ln 2 to far better than fp32 precision.
    c1 = float(sf.C1)
    assert c1 * 65536.0 == math.floor(c1 * 65536.0)
    assert abs((c1 + float(sf.C2)) - math.log(2.0)) < 1e-12
    assert sf.LOG2E == F32(1.0 / math.log(2.0))


def test_exp32_accuracy_dense_sample():
    x = np.concatenate([_float_range(-87.0, 88.0, 97), np.linspace(-20, 20, 100001, dtype=np.float32)])
    got = sf.exp32(x)
    ref = np.exp(x.astype(np.float64)).astype(np.float32)
    d = _ulp_dist(got, ref)
    assert d.max() <= 2, (x[d.argmax()], got[d.argmax()], ref[d.argmax()])


def test_exp32_special_values():
    x = np.array([0.0, -0.0, 1.0, np.inf, -np.inf, 200.0, -200.0, 89.5, -104.5, np.nan], np.float32)
    got = sf.exp32(x)
    assert got[0] == 1.0 and got[1] == 1.0
    assert _ulp_dist(got[2:3], np.array([math.e], np.float32))[0] <= 1
    assert np.isposinf(got[3]) and got[4] == 0.0
    assert np.isposinf(got[5]) and got[6] == 0.0 and np.isposinf(got[7]) and got[8] == 0.0
    assert np.isnan(got[9])
    # exact powers of two come out exact (r = 0 for x = n ln2 rounded)
    # and the subnormal tail decays monotonically to zero
    tail = sf.exp32(np.linspace(-103.9, -87.5, 4001, dtype=np.float32))
    assert np.all(np.diff(tail.astype(np.float64)) >= 0)
    assert tail[0] > 0


def test_log1p32_accuracy():
    y = np.concatenate([_float_range(0.0, 1.0, 61), np.array([0.0, 1.0, 1e-30, 1e-7], np.float32)])
    got = sf.log1p32(y)
    ref = np.log1p(y.astype(np.float64)).astype(np.float32)
    d = _ulp_dist(got, ref)
    assert d.max() <= 3, (y[d.argmax()], got[d.argmax()], ref[d.argmax()])
    assert sf.log1p32(np.float32(0.0)) == 0.0


@pytest.mark.parametrize("fn,ref,maxulp", [
    (sf.sigmoid32, lambda l: 1.0 / (1.0 + np.exp(-l)), 3),
    (sf.softplus32, lambda l: np.log1p(np.exp(-np.abs(l))) + np.maximum(l, 0.0), 4),
    (sf.sqrtsoftplus32, lambda l: np.sqrt(np.log1p(np.exp(-np.abs(l))) + np.maximum(l, 0.0)), 3),
])
def test_score_accuracy(fn, ref, maxulp):
    l = np.concatenate([_float_range(-80.0, 80.0, 211), np.linspace(-16, 16, 200001, dtype=np.float32)])
    got = fn(l)
    want = ref(l.astype(np.float64)).astype(np.float32)
    d = _ulp_dist(got, want)
    assert d.max() <= maxulp, (l[d.argmax()], got[d.argmax()], want[d.argmax()])


def test_score_closed_forms():
    assert sf.sigmoid32(np.float32(0.0)) == F32(0.5)
    # softplus(0) = ln 2, sqrtsoftplus(0) = sqrt(ln 2)
    assert _ulp_dist(sf.softplus32(np.array([0.0], np.float32)), np.array([math.log(2)], np.float32))[0] <= 1
    assert _ulp_dist(sf.sqrtsoftplus32(np.array([0.0], np.float32)),
                     np.array([math.sqrt(math.log(2))], np.float32))[0] <= 1
    # large positive logit: softplus(l) = l exactly in fp32
    assert sf.softplus32(np.float32(40.0)) == F32(40.0)
    assert sf.sqrtsoftplus32(np.float32(100.0)) == F32(10.0)
    # sigmoid symmetry s(l) + s(-l) = 1 within rounding
    l = np.linspace(-10, 10, 1001, dtype=np.float32)
    assert np.max(np.abs(sf.sigmoid32(l).astype(np.float64) + sf.sigmoid32(-l) - 1.0)) < 2e-7


def test_scores_are_monotone():
    l = np.sort(np.random.default_rng(0).normal(0, 6, 200000).astype(np.float32))
    for s in (sf.sigmoid32(l), sf.sqrtsoftplus32(l)):
        assert np.all(np.diff(s.astype(np.float64)) >= 0)


def test_tree_sum_order_pinned():
    # 2^24 + 1 + 1 summed left to right rounds back to 2^24 twice; the fixed
    # lane tree adds lanes 1 and 3 first (d=2), then lane 0 (d=1): 2^24 + 2.
    v = np.zeros(8, np.float32)
    v[0] = 2.0 ** 24
    v[1] = 1.0
    v[3] = 1.0
    assert sf.tree_sum64(v) == F32(2.0 ** 24 + 2.0)
    # strided lane partials: entries 0, 64, 128 share lane 0 and are added
    # left to right before the tree: (2^24 + 1) + 1 = 2^24.
    w = np.zeros(256, np.float32)
    w[0] = 2.0 ** 24
    w[64] = 1.0
    w[128] = 1.0
    assert sf.tree_sum64(w) == F32(2.0 ** 24)


def test_tree_sum_accuracy_and_softmax():
    rng = np.random.default_rng(1)
    for E in (8, 60, 64, 100, 256):
        v = rng.random((50, E)).astype(np.float32)
        s = sf.tree_sum64(v)
        exact = np.array([math.fsum(map(float, r)) for r in v])
        assert np.max(np.abs(s - exact) / exact) < E * 6e-8
        l = rng.normal(0, 3, (50, E)).astype(np.float32)
        p = sf.softmax32(l)
        ref = np.exp(l - l.max(-1, keepdims=True).astype(np.float64))
        ref /= ref.sum(-1, keepdims=True)
        assert np.max(np.abs(p - ref)) < 1e-6
        assert np.all(np.argmax(p, -1) == np.argmax(l, -1))
