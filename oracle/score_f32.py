"""Fixed fp32 score recipe used to take the expert-selection decision.

TEST INFRASTRUCTURE: this package is the CPU oracle.  Only tests, the smoke
check and the bench's CPU-baseline leg may import it; the product path never
does.

Why a fixed recipe: with a selection bias the top-k compares
``score(logit) + bias`` ("Sparse MoE FFN for DFlash-family drafters",
What's here, MoEGate: sqrtsoftplus routing with an aux-loss-free balancing
bias).  The pages fix neither precision nor method for the score, so the
decision is taken in fp32 with the recipe below, written out step by step.
The HIP router implements the same recipe independently; since every step is
a single IEEE-754 binary32 operation (add, subtract, multiply, divide, square
root, round-to-integer, max) evaluated in a fixed order without fused
multiply-add, two implementations that follow it agree bit for bit.

Recipe (all operations binary32, round-to-nearest-even):
  exp32(x):
    x != x -> NaN; x > 89 -> +inf; x < -104 -> +0
    n  = rint(x * LOG2E)                       (rint: ties to even)
    r  = (x - n*C1) - n*C2                     (Cody & Waite range reduction,
                                                C1 = ln2 truncated to 16 bits,
                                                C2 = fl32(ln2 - C1))
    p  = Horner of sum_{i=0..7} r^i / i!       (Taylor series of exp on
                                                |r| <= ln2/2; highest term first)
    n1 = floor(n/2), n2 = n - n1
    result = (p * 2^n1) * 2^n2                 (2^n1, 2^n2 built exactly)
  log1p32(y), 0 <= y <= 1:
    s = y / (2 + y);  z = s*s                  (log1p(y) = 2 atanh(y/(2+y)))
    q = Horner of sum_{i=0..8} z^i / (2i+1)
    result = (2*s) * q
  sigmoid32(l)      = 1 / (1 + exp32(-l))
  softplus32(l)     = max(l, 0) + log1p32(exp32(-|l|))
  sqrtsoftplus32(l) = sqrt(softplus32(l))
  softmax32(l[0..E-1]) = exp32(l_e - m) / S, m = max_e l_e, with S summed in
    this fixed order: lane L (0..63) first adds v[L], v[L+64], v[L+128],
    v[L+192] left to right (absent entries are 0), then for d = 32,16,8,4,2,1
    every lane replaces its partial a[L] by a[L] + a[L xor d].

References for the method: W. J. Cody and W. Waite, "Software Manual for the
Elementary Functions" (1980), additive range reduction with a split ln 2;
J.-M. Muller, "Elementary Functions: Algorithms and Implementation",
polynomial evaluation on the reduced range; log1p via the atanh series.
"""
from __future__ import annotations

import numpy as np

F32 = np.float32

LOG2E = F32(1.4426950408889634)
_LN2 = 0.6931471805599453094172321
C1 = F32(np.floor(_LN2 * 65536.0) / 65536.0)      # ln 2 truncated to 16 bits
C2 = F32(_LN2 - float(C1))
EXP_TAYLOR = [F32(1.0 / f) for f in (5040.0, 720.0, 120.0, 24.0, 6.0, 2.0, 1.0, 1.0)]
ATANH_COEF = [F32(1.0 / d) for d in (17.0, 15.0, 13.0, 11.0, 9.0, 7.0, 5.0, 3.0, 1.0)]


def _pow2(n: np.ndarray) -> np.ndarray:
    """2^n exactly, for integer n in [-126, 127], built from its bits."""
    bits = ((n.astype(np.int64) + 127) << 23).astype(np.uint32)
    return bits.view(np.float32)


def exp32(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    with np.errstate(over="ignore", under="ignore", invalid="ignore"):
        xc = np.clip(x, F32(-104.0), F32(89.0))
        n = np.rint(xc * LOG2E)
        r = (xc - n * C1) - n * C2
        p = EXP_TAYLOR[0]
        for c in EXP_TAYLOR[1:]:
            p = p * r + c
        n_i = n.astype(np.int64)
        n1 = np.floor_divide(n_i, 2)
        n2 = n_i - n1
        res = (p * _pow2(n1)) * _pow2(n2)
        res = np.where(x > F32(89.0), F32(np.inf), res)
        res = np.where(x < F32(-104.0), F32(0.0), res)
        res = np.where(np.isnan(x), F32(np.nan), res)
    return res.astype(np.float32)


def log1p32(y) -> np.ndarray:
    """log(1+y) for 0 <= y <= 1."""
    y = np.asarray(y, dtype=np.float32)
    s = y / (F32(2.0) + y)
    z = s * s
    q = ATANH_COEF[0]
    for c in ATANH_COEF[1:]:
        q = q * z + c
    return ((F32(2.0) * s) * q).astype(np.float32)


def sigmoid32(l) -> np.ndarray:
    l = np.asarray(l, dtype=np.float32)
    with np.errstate(over="ignore"):
        return (F32(1.0) / (F32(1.0) + exp32(-l))).astype(np.float32)


def softplus32(l) -> np.ndarray:
    l = np.asarray(l, dtype=np.float32)
    return (np.maximum(l, F32(0.0)) + log1p32(exp32(-np.abs(l)))).astype(np.float32)


def sqrtsoftplus32(l) -> np.ndarray:
    return np.sqrt(softplus32(l)).astype(np.float32)


def tree_sum64(v: np.ndarray) -> np.ndarray:
    """Fixed-order sum over the last axis (length <= 256) as stated above."""
    v = np.asarray(v, dtype=np.float32)
    n = v.shape[-1]
    assert n <= 256
    pad = np.zeros(v.shape[:-1] + (256,), dtype=np.float32)
    pad[..., :n] = v
    a = pad[..., 0:64]
    for i in range(1, 4):
        a = a + pad[..., 64 * i:64 * (i + 1)]
    lanes = np.arange(64)
    for d in (32, 16, 8, 4, 2, 1):
        a = a + a[..., lanes ^ d]
    return a[..., 0]


def softmax32(l) -> np.ndarray:
    l = np.asarray(l, dtype=np.float32)
    m = l.max(axis=-1, keepdims=True)
    v = exp32(l - m)
    S = tree_sum64(v)[..., None]
    return (v / S).astype(np.float32)


def scores32(logits32: np.ndarray, score: int) -> np.ndarray:
    """Row-wise fp32 scores of fp32 logits [T, E] (0 softmax, 1 sigmoid,
    2 sqrtsoftplus)."""
    if score == 0:
        return softmax32(logits32)
    if score == 1:
        return sigmoid32(logits32)
    if score == 2:
        return sqrtsoftplus32(logits32)
    raise ValueError(f"unknown score function {score}")
