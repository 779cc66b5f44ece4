"""Textbook (unquantised, untiled) attention in fp64, and exact fp32 rounding of
rationals: independent yardsticks for pinning the oracle."""
from fractions import Fraction

import numpy as np


def attention_fp64(q, k, v, causal=False, sm_scale=None):
    """softmax(q k^T * sm_scale) v per head, fp64, whole score matrix at once."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    N, d = q.shape[-2], q.shape[-1]
    if sm_scale is None:
        sm_scale = 1.0 / np.sqrt(d)
    s = np.einsum("...id,...jd->...ij", q, k) * sm_scale
    if causal:
        mask = np.triu(np.ones((N, N), bool), 1)
        s = np.where(mask, -np.inf, s)
    s = s - s.max(axis=-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=-1, keepdims=True)
    return np.einsum("...ij,...jd->...id", p, v)


def rn32(x: Fraction) -> np.float32:
    """Round a rational to the nearest binary32 (ties to even), by integer arithmetic."""
    if x == 0:
        return np.float32(0.0)
    sign = -1 if x < 0 else 1
    a = abs(x)
    # find e with 2^23 <= a * 2^-e < 2^24 (normal numbers)
    e = a.numerator.bit_length() - a.denominator.bit_length() - 23
    while a / Fraction(2) ** e >= 2 ** 24:
        e += 1
    while a / Fraction(2) ** e < 2 ** 23:
        e -= 1
    e = max(e, -149)  # subnormal quantum 2^-149
    m = a / Fraction(2) ** e
    lo = m.numerator // m.denominator
    rem = m - lo
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and lo % 2 == 1):
        lo += 1
    return np.float32(sign * float(lo * Fraction(2) ** e))


def cos_sim(a, b):
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


def rel_l1(a, b):
    """sum |a - b| / sum |b| (b is the reference)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.abs(a - b).sum() / np.abs(b).sum())


def rmse(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.sqrt(np.mean((a - b) ** 2)))
