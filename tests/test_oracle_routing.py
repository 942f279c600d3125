"""Pins for the oracle's router and dispatch (CPU only).

Top-k is pinned by brute force over all C(E,k) subsets on tiny inputs and by
NumPy's stable argsort; weights by their closed forms; dispatch by a Python
counting loop written from the definition and by permutation invariants.
Planted mistakes (tie-break flipped, unstable sort, bias leaking into the
weights) must each fail the matching pin.
"""
import numpy as np
import pytest

from oracle import moe_ref as R
from oracle import score_f32 as sf


def _keys(rng, T, E, tie_heavy):
    if tie_heavy:
        return rng.integers(-1, 2, (T, E)).astype(np.float32)
    return rng.normal(0, 1, (T, E)).astype(np.float32)


@pytest.mark.parametrize("E,k", [(8, 2), (8, 8), (16, 1), (6, 3), (5, 5), (10, 4)])
@pytest.mark.parametrize("tie_heavy", [False, True])
def test_topk_matches_bruteforce(E, k, tie_heavy):
    rng = np.random.default_rng(E * 100 + k + tie_heavy)
    keys = _keys(rng, 40, E, tie_heavy)
    assert np.array_equal(R.topk_select(keys, k), R.topk_bruteforce(keys, k))


def test_topk_signed_zero_is_one_key():
    logits = np.array([[-0.0, 0.0, -1.0, 0.0]], np.float32)
    keys = R.selection_keys(logits, 1, None)
    assert list(R.topk_select(keys, 3)[0]) == [0, 1, 3]


def test_topk_negative_tiebreak_flip_is_caught():
    rng = np.random.default_rng(7)
    keys = _keys(rng, 40, 8, True)

    def flipped(keys, k):  # planted mistake: ties to the higher index
        E = keys.shape[1]
        o = np.argsort(-keys[:, ::-1].astype(np.float64), axis=-1, kind="stable")
        return (E - 1 - o)[:, :k]
    assert not np.array_equal(flipped(keys, 2), R.topk_bruteforce(keys, 2))


@pytest.mark.parametrize("E,k", [(16, 1), (32, 4), (60, 4), (64, 6), (128, 8), (256, 8)])
def test_routing_shape_matrix_invariants(E, k):
    """Production routing shapes (16/1, 32/4, 60/4, 64/6, 128/8, 256/8):
    every selected key >= every unselected key, descending order, ties to the
    lower index; expert E-1 is reachable."""
    rng = np.random.default_rng(E)
    keys = rng.normal(0, 1, (64, E)).astype(np.float32)
    keys[:8] = np.round(keys[:8])            # some rows full of ties
    keys[8, E - 1] = 10.0                     # force the last expert
    ids = R.topk_select(keys, k)
    assert ids[8, 0] == E - 1
    for t in range(keys.shape[0]):
        sel = ids[t]
        assert len(set(sel)) == k
        ks = keys[t, sel]
        assert np.all(ks[:-1] >= ks[1:])
        for a, b in zip(sel[:-1], sel[1:]):
            if keys[t, a] == keys[t, b]:
                assert a < b
        rest = np.setdiff1d(np.arange(E), sel)
        if rest.size:
            assert keys[t, rest].max() <= ks.min()
            # a tie across the cut goes to the lower index
            tied = rest[keys[t, rest] == ks.min()]
            assert np.all(tied > sel[ks == ks.min()].max())


@pytest.mark.parametrize("score", [0, 1, 2])
def test_selection_without_bias_equals_exact_score_topk(score):
    """No bias: selecting on the fp32 logit gives the same experts as
    selecting on the exact (float64) scores, because every score function is
    strictly increasing in the logit."""
    rng = np.random.default_rng(score)
    l32 = rng.normal(0, 2, (200, 60)).astype(np.float32)
    ids = R.topk_select(R.selection_keys(l32, score, None), 4)
    s64 = R.scores_f64(l32.astype(np.float64), score)
    ids64 = np.argsort(-s64, axis=-1, kind="stable")[:, :4]
    assert np.array_equal(ids, ids64)


def test_selection_with_bias_uses_recipe():
    rng = np.random.default_rng(3)
    l32 = rng.normal(0, 1, (100, 64)).astype(np.float32)
    b = rng.normal(0, 0.7, 64).astype(np.float32)
    keys = R.selection_keys(l32, 2, b)
    assert keys.dtype == np.float32
    assert np.array_equal(keys, (sf.sqrtsoftplus32(l32) + b).astype(np.float32))
    # the bias changes the selection for some rows (it is not vacuous)
    assert not np.array_equal(R.topk_select(keys, 6), R.topk_select(R.selection_keys(l32, 2, None), 6))


def test_weights_closed_forms():
    rng = np.random.default_rng(4)
    l32 = rng.normal(0, 2, (50, 16)).astype(np.float32)
    # softmax, k = E, no renorm: weights are the full softmax in ranked order
    w, ids = R.route(l32, 16, 0, False)
    p = np.exp(l32 - l32.max(-1, keepdims=True).astype(np.float64))
    p /= p.sum(-1, keepdims=True)
    assert np.allclose(np.take_along_axis(p, ids, -1), w, atol=1e-15)
    assert np.allclose(w.sum(-1), 1.0, atol=1e-12)
    # renorm: sums to one; no renorm: raw selected probabilities
    for score in (0, 1, 2):
        w, ids = R.route(l32, 4, score, True)
        assert np.allclose(w.sum(-1), 1.0, atol=1e-12)
        w2, ids2 = R.route(l32, 4, score, False)
        s = R.scores_f64(l32.astype(np.float64), score)
        assert np.array_equal(ids, ids2)
        assert np.allclose(w2, np.take_along_axis(s, ids, -1), atol=0)


def test_bias_never_enters_weights():
    rng = np.random.default_rng(5)
    l32 = rng.normal(0, 1, (80, 32)).astype(np.float32)
    b = rng.normal(0, 1, 32).astype(np.float32)
    w, ids = R.route(l32, 4, 2, True, b)
    s = R.scores_f64(l32.astype(np.float64), 2)
    sel = np.take_along_axis(s, ids, -1)
    assert np.allclose(w, sel / sel.sum(-1, keepdims=True), atol=1e-15)
    # planted mistake: weights from biased keys must not pass this pin
    bad = sel + b[ids]
    bad = bad / bad.sum(-1, keepdims=True)
    assert not np.allclose(w, bad, atol=1e-6)


def _dispatch_by_loop(ids, E):
    """Counting sort written as plain loops from the definition."""
    flat = list(np.asarray(ids).ravel())
    counts = [0] * E
    for e in flat:
        counts[e] += 1
    offsets = [0]
    for c in counts:
        offsets.append(offsets[-1] + c)
    fill = list(offsets[:-1])
    pos = [0] * len(flat)
    perm = [0] * len(flat)
    for i, e in enumerate(flat):
        pos[i] = fill[e]
        perm[fill[e]] = i
        fill[e] += 1
    return counts, offsets, perm, pos


@pytest.mark.parametrize("T,E,k", [(64, 8, 2), (100, 60, 4), (33, 256, 8), (1, 4, 4), (0, 8, 2)])
def test_dispatch_matches_counting_loop(T, E, k):
    rng = np.random.default_rng(T + E)
    ids = np.array([rng.permutation(E)[:k] for _ in range(T)], np.int64).reshape(T, k)
    d = R.dispatch(ids, E)
    c, o, p, q = _dispatch_by_loop(ids, E)
    assert list(d["counts"]) == c and list(d["offsets"]) == o
    assert list(d["perm"]) == p and list(d["pos"]) == q
    flat = ids.ravel()
    assert d["counts"].sum() == T * k
    assert np.all(np.diff(d["offsets"]) >= 0)
    assert np.array_equal(np.sort(d["perm"]), np.arange(T * k))
    assert np.all(np.diff(flat[d["perm"]]) >= 0)
    for e in range(E):
        seg = d["perm"][d["offsets"][e]:d["offsets"][e + 1]]
        assert np.all(np.diff(seg) > 0)        # stable: flat index increases


def test_dispatch_unstable_sort_is_caught():
    rng = np.random.default_rng(11)
    ids = rng.integers(0, 8, (64, 2)).astype(np.int64)
    good = R.dispatch(ids, 8)["perm"]
    # swap two entries inside the largest segment: a planted instability
    bad = good.copy()
    bad[0], bad[1] = bad[1], bad[0]
    _, _, p, _ = _dispatch_by_loop(ids, 8)
    assert list(good) == p and list(bad) != p
