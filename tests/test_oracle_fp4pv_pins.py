"""Pins of the oracle's MXFP4 P~V variant (variant 3) against things other than itself.

Page: [SA3] "SageAttention3: Microscaling FP4 Attention for Inference and an Exploration
of 8-Bit Training" (abstract, under the NeurIPS Conference 2025 heading of the author
page): attention with FP4 operands.  The pages fix no block format; the oracle reads
both operands of P~V as MXFP4 blocks of 32 along the keys (E8M0 scale, E2M1 elements):
V per channel with the OCP exponent rule, P~ per row with the smallest power-of-two
scale that holds the block max without saturating.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads
from tests.ref64 import cos_sim
from tests.test_oracle_pins import E2M1_TABLE, _e2m1_by_thresholds


def _e8m0(code: int) -> float:
    """E8M0 scale value, decoded by torch's float8_e8m0fnu."""
    return torch.tensor([int(code)], dtype=torch.uint8).view(torch.float8_e8m0fnu).float().item()


# --------------------------------------------------------------------------
# the P~ block rule
# --------------------------------------------------------------------------

def test_p_block_scale_is_the_smallest_that_does_not_saturate(orc):
    """For every block: the scale 2^E is the smallest power of two with max/2^E <= 6 (the
    largest E2M1 magnitude), checked with exact rationals, and every element is the E2M1
    code of P~/2^E by the rounding thresholds.  An all-zero block gets code 0."""
    rng = np.random.default_rng(7)
    blocks = [rng.uniform(0, 1, 32) * 2.0 ** rng.integers(-30, 1) for _ in range(300)]
    blocks += [rng.uniform(0, 1, 32) ** 8 for _ in range(50)]          # spread-out weights
    edge = [1.0, np.nextafter(np.float32(1.0), np.float32(0)), 0.75, np.nextafter(np.float32(0.75), np.float32(1)),
            0.375, 2.0 ** -20, 1.5 * 2.0 ** -40]
    for a in edge:
        b = rng.uniform(0, 1, 32) * a
        b[5] = a
        blocks.append(b)
    blocks.append(np.zeros(32))
    p = np.array(blocks, np.float32)
    codes, e8 = orc.p_block_fp4(p)
    for blk, cs, e in zip(p, codes, e8):
        a = Fraction(float(blk.max()))
        if a == 0:
            assert e == 0 and not cs.any()
            continue
        assert 0 < e < 254
        X = Fraction(_e8m0(e))
        assert a / X <= 6 and a / (X / 2) > 6, (float(a), int(e))
        assert [int(c) for c in cs] == [_e2m1_by_thresholds(float(Fraction(float(x)) / X)) for x in blk]


def test_p_block_keeps_a_weight_just_below_a_power_of_two(orc):
    """The reason for the rule: 1 - 2^-24 and 1 get the same value (1), where the OCP
    exponent (floor(log2 max) - 2) would map 1 - 2^-24 to 7.99.. and clip it to 6/8."""
    one_minus = np.nextafter(np.float32(1.0), np.float32(0))
    p = np.zeros((2, 32), np.float32)
    p[0, 0], p[1, 0] = 1.0, one_minus
    codes, e8 = orc.p_block_fp4(p)
    vals = [orc.e2m1_decode(codes[i, :1])[0] * _e8m0(e8[i]) for i in range(2)]
    assert vals == [1.0, 1.0]


# --------------------------------------------------------------------------
# V in MXFP4 (per channel, blocks of 32 tokens)
# --------------------------------------------------------------------------

def test_v_mx_blocks_run_along_the_tokens(orc):
    """quant_v_mx: for channel c and token block b, the OCP rule (E8M0 code =
    floor(log2 max|V|) - 2 + 127, elements E2M1(V / 2^(code - 127))) over V[32b:32b+32, c];
    tokens past N are zeros (ragged N), and the codes run along the tokens."""
    rng = np.random.default_rng(8)
    N, d = 77, 32
    v = rng.standard_normal((1, 1, N, d)) * 2.0 ** rng.integers(-10, 8, (1, 1, 1, d))
    v[0, 0, 32:64, 3] = 0.0            # an all-zero block
    v[0, 0, 40, 4] = 8.0               # max a power of two: element 4
    v = v.astype(np.float16)
    r = orc.quant_v_mx(v, smooth_v=0)
    codes, e8 = r["v_codes"][0, 0], r["v_e8"][0, 0]
    Np = codes.shape[1]
    assert Np == 128 and e8.shape == (d, 4)
    for c in range(d):
        col = np.zeros(Np, np.float32)
        col[:N] = v[0, 0, :, c].astype(np.float32)
        for b in range(Np // 32):
            blk = col[32 * b:32 * b + 32]
            a = float(np.abs(blk).max())
            want_e8 = 0 if a == 0 else math.frexp(a)[1] - 1 - 2 + 127
            assert e8[c, b] == want_e8, (c, b)
            X = _e8m0(e8[c, b])
            want = [(_e2m1_by_thresholds(float(x) / X) if a else 0) for x in blk]
            want = [w if a else (8 if math.copysign(1.0, float(x)) < 0 else 0) for w, x in zip(want, blk)]
            assert [int(q) for q in codes[c, 32 * b:32 * b + 32]] == want, (c, b)
    assert codes[4, 40] == 6
    assert not codes[:, N:].any()


def test_v_mx_smoothing_subtracts_the_exact_token_mean(orc):
    """smooth_v: each channel loses its exact token mean (rational sum of the fp16 values,
    rounded once to fp32) before the block rule."""
    rng = np.random.default_rng(9)
    N, d = 50, 32
    v = (rng.standard_normal((1, 1, N, d)) + 3.0).astype(np.float16)
    r = orc.quant_v_mx(v, smooth_v=1)
    for c in range(d):
        mean = sum((Fraction(float(x)) for x in v[0, 0, :, c]), Fraction(0)) / N
        assert r["v_mean"][0, 0, c] == np.float32(float(mean))
    # the codes are those of V - mean
    shifted = (v[0, 0].astype(np.float32) - r["v_mean"][0, 0][None, :])
    blk = shifted[:32, 0]
    X = _e8m0(r["v_e8"][0, 0, 0, 0])
    assert [int(q) for q in r["v_codes"][0, 0, 0, :32]] == [_e2m1_by_thresholds(float(x) / X) for x in blk]


# --------------------------------------------------------------------------
# attention
# --------------------------------------------------------------------------

def _lossless_v(N, d, rng):
    """V exactly representable in MXFP4 along the tokens: entries in {0, +-1, +-2, +-4}
    times 2^(b - 2) in token block b, with a 4 * 2^(b - 2) in every (channel, block)."""
    v = rng.choice([0.0, 1.0, -1.0, 2.0, -2.0, 4.0, -4.0], (N, d))
    for b0 in range(0, N, 32):
        v[b0, :] = 4.0
        v[b0:b0 + 32] *= 2.0 ** (b0 // 32 - 2)
    return v


@pytest.mark.parametrize("causal", [0, 1])
def test_q_zero_gives_the_mean_of_the_visible_v(orc, causal):
    """Q = 0: every visible P~ is 1, exact in the P~ rule (scale 2^-2, element 4), so
    O_i is the plain mean of the visible V rows; V is exact in MXFP4 with a different
    scale in every token block, so O equals the fp64 mean (pins the V block index and
    scale, the P~ shift without 448, and the masking)."""
    rng = np.random.default_rng(10)
    N, d = 150, 64
    v = _lossless_v(N, d, rng)
    q = np.zeros((1, 1, N, d), np.float16)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float16)
    o = orc.attn(q, k, v.astype(np.float16)[None, None], causal=causal, variant=3, bkv=64)
    if causal:
        ref = np.cumsum(v, 0) / np.arange(1, N + 1)[:, None]
    else:
        ref = np.broadcast_to(v.mean(0), (N, d))
    assert np.max(np.abs(o[0, 0] - ref)) < 1e-12


def _fp4_lossless_case(N=160, d=64, seed=12):
    """Q, K entries in {0, 1} (exact in MXFP4: a block max of 1 gives scale 2^-2 and
    element 4); every q row has three ones, so the scores are integers in [0, 3].  With
    sm_scale = ln 2 the weights are 2^(S - m), i.e. 1, 1/2, 1/4 or 1/8 of the running max:
    exact in the P~ rule (block scale 2^-2 or finer, elements >= 1/2)."""
    rng = np.random.default_rng(seed)
    q = np.zeros((N, d))
    for i in range(N):
        q[i, rng.choice(d, 3, replace=False)] = 1.0
    k = (rng.uniform(size=(N, d)) < 0.3).astype(np.float64)
    # the first keys miss the ones of later rows, so running maxima move in later tiles
    k[:40, :] = 0.0
    k[:40, 0] = 1.0
    return q, k, _lossless_v(N, d, rng)


@pytest.mark.parametrize("causal", [0, 1])
def test_lossless_inputs_match_base2_softmax_attention(orc, causal):
    """Inputs on which every FP4 step is exact: O equals fp64 attention with weights
    2^(S - max S) (pins the scores, the per-tile rescale and the block codes of P~ and V)."""
    q, k, v = _fp4_lossless_case()
    f = lambda a: a.astype(np.float16)[None, None]
    o = orc.attn(f(q), f(k), f(v), causal=causal, variant=3, smooth_k=0, bkv=64, sm_scale=math.log(2.0))
    S = q @ k.T
    if causal:
        S = np.where(np.tril(np.ones(S.shape, bool)), S, -np.inf)
    w = np.exp2(S - S.max(1, keepdims=True))
    ref = (w @ v) / w.sum(1, keepdims=True)
    # kscale = fl32(ln 2) * fl32(log2 e) is 1 up to an ulp, so the weights are exact up to
    # a relative 2^-23 * |S - m| (<= 3)
    assert np.max(np.abs(o[0, 0] - ref)) < 1e-5
    # some row's running max does move after its first tile (the rescale is exercised)
    assert (S[:, :64].max(1) < S.max(1)).any()


def _p_rule_bruteforce(p):
    """The P~ rule for one block, by search: the smallest E with max/2^E <= 6, then the
    nearest E2M1 magnitude of each p/2^E (a tie to the even code).  Also returns the
    smallest relative distance of a scaled weight to a rounding midpoint."""
    a = max(p)
    if a == 0:
        return [0.0] * len(p), math.inf
    E = math.frexp(a)[1] - 5          # max / 2^E >= 8: a lower bound of the answer
    while a / 2.0 ** E > 6:
        E += 1
    X = 2.0 ** E
    out, gap = [], math.inf
    for x in p:
        y = x / X
        best = min(range(8), key=lambda c: (abs(E2M1_TABLE[c] - y), c % 2))
        out.append(E2M1_TABLE[best] * X)
        if y:
            gap = min(gap, min(abs(y - mid) / y for mid in (0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0)))
    return out, gap


@pytest.mark.parametrize("causal", [0, 1])
def test_l_sums_the_unrounded_p(orc, causal):
    """R-11 in the FP4 path: with V constant 4 (exact), O_i = 4 * sum_j Pdec_ij / sum_j P~_ij,
    Pdec the MXFP4 value of P~ in its 32-key block (found here by search), P~ =
    2^(1.5 (S - m)) against the running max of the 64-key tiles; so O differs from 4,
    which a sum of the rounded weights would give."""
    q, k, _ = _fp4_lossless_case(N=130, seed=13)
    N, d = q.shape
    v = np.full((1, 1, N, d), 4.0, np.float16)
    f = lambda a: a.astype(np.float16)[None, None]
    o = orc.attn(f(q), f(k), v, causal=causal, variant=3, smooth_k=0, bkv=64, sm_scale=1.5 * math.log(2.0))
    S = q @ k.T
    ref = np.zeros(N)
    for i in range(N):
        jmax = i + 1 if causal else N
        m = -np.inf
        num = den = 0.0
        for j0 in range(0, jmax, 64):
            j1 = min(j0 + 64, jmax)
            mnew = max(m, S[i, j0:j1].max())
            a = 2.0 ** (1.5 * (m - mnew)) if np.isfinite(m) else 0.0
            p = [float(np.float32(2.0 ** (1.5 * (s - mnew)))) for s in S[i, j0:j1]]
            p += [0.0] * (64 - len(p))
            (d0, g0), (d1, g1) = _p_rule_bruteforce(p[:32]), _p_rule_bruteforce(p[32:])
            dec = d0 + d1
            # away from the rounding midpoints, where fp32 and fp64 weights could decide apart
            assert min(g0, g1) > 1e-6
            num = a * num + sum(dec)
            den = a * den + sum(p)
            m = mnew
        ref[i] = 4.0 * num / den
    assert np.max(np.abs(o[0, 0] - ref[:, None])) < 1e-5
    assert np.max(np.abs(ref - 4.0)) > 1e-2


@pytest.mark.parametrize("causal", [0, 1])
def test_v_smoothing_returns_a_constant_v_exactly(orc, causal):
    """smooth_v with V constant per channel: V - mean = 0, so every V code is 0 and O is the
    mean, i.e. V itself."""
    rng = np.random.default_rng(14)
    N, d = 100, 32
    q = rng.standard_normal((1, 1, N, d)).astype(np.float16)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float16)
    row = rng.standard_normal(d).astype(np.float16)
    v = np.broadcast_to(row, (1, 1, N, d)).copy()
    o = orc.attn(q, k, v, causal=causal, variant=3, smooth_v=1)
    assert np.array_equal(o[0, 0], np.broadcast_to(row.astype(np.float32).astype(np.float64), (N, d)))


def test_power_of_two_scaling_of_v_scales_o(orc):
    """Scaling V by 2^k shifts every V block exponent by k and leaves the elements alone, so O
    scales by exactly 2^k."""
    x = workloads.make_inputs(1, N=200, B=1, H=1)
    o1 = orc.attn(x["q"], x["k"], x["v"], variant=3)
    o2 = orc.attn(x["q"], x["k"], (x["v"].astype(np.float32) * 8).astype(np.float16), variant=3)
    assert np.array_equal(o2, 8 * o1)


def test_fp4_attention_tracks_fp64_attention_config1(orc):
    """Accuracy on workload 1's recipe against unquantised fp64 attention: MXFP4 on both
    products is coarse (cosine 0.967 measured, against 0.986 with FP8 P~V), but far from a
    wrong computation (a dropped scale or a misplaced block gives well below 0.9)."""
    x = workloads.make_inputs(1)
    exact = orc.attn(x["q"], x["k"], x["v"], exact=1)
    o3 = orc.attn(x["q"], x["k"], x["v"], variant=3)
    assert cos_sim(o3, exact) > 0.96
