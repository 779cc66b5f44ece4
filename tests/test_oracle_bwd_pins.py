"""Pins of the backward oracle (dQ, dK, dV of the 8-bit forward), CPU only.

The backward follows the SageAttention3 abstract (author page, "NeurIPS Conference 2025"
heading: 8-bit attention for both forward and backward propagation) and
FlashAttention-2's backward order (P = exp(s - L), D = rowsum(dO * O),
dS = P * (dP - D)).  Its readings are listed in oracle.c; these tests tie it to things
other than itself: fp64 autograd with quantisation off, closed forms, exact
invariances of the quantised path, and the quality of the quantised gradients
against exact ones.
"""
import math

import numpy as np
import pytest
import torch

import workloads
from tests.ref64 import cos_sim


def _autograd(q, k, v, dout, causal, sm_scale=None):
    """fp64 textbook attention backward by torch autograd (CPU)."""
    t = [torch.from_numpy(np.asarray(a, np.float64)).requires_grad_(i < 3) for i, a in enumerate((q, k, v, dout))]
    qq, kk, vv, gg = t
    d = q.shape[-1]
    sc = 1.0 / math.sqrt(d) if sm_scale is None else sm_scale
    s = (qq @ kk.transpose(-1, -2)) * sc
    if causal:
        N = q.shape[-2]
        s = s.masked_fill(torch.triu(torch.ones(N, N, dtype=torch.bool), 1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vv
    o.backward(gg)
    return dict(dq=qq.grad.numpy(), dk=kk.grad.numpy(), dv=vv.grad.numpy(), o=o.detach().numpy())


def _case(N, d, seed, B=1, H=2, k_sigma=2.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, H, N, d))
    k = rng.standard_normal((B, H, N, d)) + k_sigma * rng.standard_normal((B, H, 1, d))
    v = rng.standard_normal((B, H, N, d))
    dout = rng.standard_normal((B, H, N, d))
    f = lambda a: a.astype(np.float16)
    return f(q), f(k), f(v), f(dout)


@pytest.mark.parametrize("N,d,causal", [(37, 32, 0), (37, 32, 1), (130, 64, 1), (1, 16, 0)])
def test_exact_mode_equals_autograd(orc, N, d, causal):
    q, k, v, dout = _case(N, d, seed=N + causal)
    ref = _autograd(q, k, v, dout, causal)
    o = ref["o"].astype(np.float16)
    g = orc.attn_bwd(q, k, v, o, dout, causal=causal, exact=1)
    # exact mode takes D from the given (fp16-rounded) O; autograd's D uses the exact O.  The
    # difference is sum_j P_ij (D_exact - D_16) K_j: compare with D computed the same way.
    ref16 = _autograd_with_d(q, k, v, dout, o, causal)
    for n in ("dq", "dk", "dv"):
        assert np.max(np.abs(g[n] - ref16[n])) < 1e-10, n
    assert np.max(np.abs(g["dv"] - ref["dv"])) < 1e-10  # dV does not depend on D
    for n in ("dq", "dk"):
        if np.abs(ref[n]).max() < 1e-12:  # one token: the scores do not matter
            assert np.abs(g[n]).max() < 1e-10, n
        else:
            assert cos_sim(g[n], ref[n]) > 0.999999, n


def _autograd_with_d(q, k, v, dout, o16, causal):
    """The textbook backward with D = rowsum(dO * O16) for a given O16 (closed form in fp64)."""
    qf, kf, vf, gf = (np.asarray(a, np.float64) for a in (q, k, v, dout))
    d = q.shape[-1]
    s = qf @ np.swapaxes(kf, -1, -2) / math.sqrt(d)
    if causal:
        N = q.shape[-2]
        s = np.where(np.triu(np.ones((N, N), bool), 1), -np.inf, s)
    s = s - s.max(-1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(-1, keepdims=True)
    dp = gf @ np.swapaxes(vf, -1, -2)
    D = (gf * o16.astype(np.float64)).sum(-1, keepdims=True)
    ds = p * (dp - D)
    return dict(dq=ds @ kf / math.sqrt(d), dk=np.swapaxes(ds, -1, -2) @ qf / math.sqrt(d),
                dv=np.swapaxes(p, -1, -2) @ gf)


def test_closed_form_form_of_exact_mode(orc):
    """The closed form used above is itself autograd when O is exact (no fp16 rounding of O)."""
    q, k, v, dout = _case(20, 8, seed=3)
    ref = _autograd(q, k, v, dout, 1)
    cf = _autograd_with_d(q, k, v, dout, ref["o"], 1)
    for n in ("dq", "dk", "dv"):
        assert np.max(np.abs(cf[n] - ref[n])) < 1e-12, n


@pytest.mark.parametrize("causal", [0, 1])
def test_quantised_gradients_track_exact_ones(orc, causal):
    """The 8-bit backward on workload 1's recipe (K with channel offsets) stays close to the
    exact fp64 gradients: cosine >= 0.9995 for dQ, dK and dV (measured: 0.99989 or better).
    dQ uses the smoothed K: with K itself the channel offsets multiply the rounding of the
    row sums of dS (cosine 0.997)."""
    x = workloads.make_inputs(1)
    q, k, v = x["q"], x["k"], x["v"]
    rng = np.random.default_rng(7)
    dout = rng.standard_normal(q.shape).astype(np.float16)
    ref = _autograd(q, k, v, dout, causal)
    o = ref["o"].astype(np.float16)
    g = orc.attn_bwd(q, k, v, o, dout, causal=causal, blk_q=64, blk_k=64)
    c = {n: cos_sim(g[n], ref[n]) for n in ("dq", "dk", "dv")}
    assert min(c.values()) >= 0.9995, c


def test_zero_output_gradient_gives_zero(orc):
    q, k, v, _ = _case(50, 16, seed=4)
    dout = np.zeros_like(q)
    o = _autograd(q, k, v, dout, 0)["o"].astype(np.float16)
    for exact in (0, 1):
        g = orc.attn_bwd(q, k, v, o, dout, exact=exact, blk_q=32, blk_k=16)
        for n in ("dq", "dk", "dv"):
            assert not g[n].any(), (n, exact)


def test_single_token(orc):
    """N = 1: P = 1, so dV = dO exactly (2^8 * 1 is exact in fp16), and with V smoothed V' = 0
    and O = V make dP = 0 and D = 0, so dQ = dK = 0 exactly."""
    q, k, v, dout = _case(1, 32, seed=5, H=3)
    g = orc.attn_bwd(q, k, v, v, dout, blk_q=32, blk_k=16)
    assert np.array_equal(g["dv"], dout.astype(np.float64))
    assert not g["dq"].any() and not g["dk"].any()


@pytest.mark.parametrize("causal", [0, 1])
def test_constant_v_gives_zero_score_gradients(orc, causal):
    """V equal for every token: the output is V whatever the scores, so dQ = dK = 0; in the
    8-bit path V' = 0 after smoothing, dP = 0 and D = dO . (O - vmean) = 0 exactly."""
    q, k, _, dout = _case(70, 32, seed=6)
    rng = np.random.default_rng(8)
    row = rng.standard_normal((1, 2, 1, 32)).astype(np.float16)
    v = np.repeat(row, 70, axis=2)
    g = orc.attn_bwd(q, k, v, v, dout, causal=causal, blk_q=32, blk_k=16)
    assert not g["dq"].any() and not g["dk"].any()
    ref = _autograd(q, k, v, dout, causal)
    assert cos_sim(g["dv"], ref["dv"]) > 0.9999


def test_v_offset_does_not_change_the_8bit_gradients(orc):
    """V smoothing: adding a per-channel offset to V (and hence to O) leaves V', its INT8 codes,
    dP and D unchanged, so dQ, dK, dV are bit-identical.  (Without the shift of D by
    dO . vmean, dS would move by P * dO . offset.)"""
    q, k, v, dout = _case(90, 32, seed=9)
    rng = np.random.default_rng(10)
    off = rng.integers(-4, 5, (1, 2, 1, 32)).astype(np.float64)
    # tokens in +- pairs: every channel mean is exactly 0 (and exactly off after the
    # offset), and values stay exact in fp16 after the offset
    w = np.round(v[:, :, :45].astype(np.float64) * 64) / 64
    v = np.concatenate([w, -w], axis=2)
    o = np.round(_autograd(q, k, v, dout, 1)["o"] * 64) / 64
    g0 = orc.attn_bwd(q, k, v.astype(np.float16), o.astype(np.float16), dout, causal=1, blk_q=32, blk_k=16)
    g1 = orc.attn_bwd(q, k, (v + off).astype(np.float16), (o + off).astype(np.float16), dout, causal=1,
                      blk_q=32, blk_k=16)
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(g0[n], g1[n]), n


def test_power_of_two_scaling_of_dout(orc):
    """dO * 2^10: every quantity the backward forms from dO scales by 2^10 exactly (INT8 codes
    unchanged, sigma divided by 2^10), so the gradients scale exactly."""
    q, k, v, dout = _case(60, 32, seed=11)
    o = _autograd(q, k, v, dout, 0)["o"].astype(np.float16)
    g0 = orc.attn_bwd(q, k, v, o, dout, blk_q=32, blk_k=16)
    g1 = orc.attn_bwd(q, k, v, o, (dout.astype(np.float64) * 1024).astype(np.float16), blk_q=32, blk_k=16)
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(g1[n], g0[n] * 1024), n


def test_smoothing_k_is_invisible_in_exact_mode_and_small_in_8bit(orc):
    """K smoothing only changes the forward's INT8 codes: exact mode ignores it, and the 8-bit
    gradients with and without it are both close to the exact ones."""
    q, k, v, dout = _case(64, 32, seed=12, k_sigma=6.0)
    ref = _autograd(q, k, v, dout, 0)
    o = ref["o"].astype(np.float16)
    ga = orc.attn_bwd(q, k, v, o, dout, exact=1, smooth_k=0)
    gb = orc.attn_bwd(q, k, v, o, dout, exact=1, smooth_k=1)
    for n in ("dq", "dk", "dv"):
        assert np.array_equal(ga[n], gb[n])
    c = {s: cos_sim(orc.attn_bwd(q, k, v, o, dout, smooth_k=s, blk_q=32, blk_k=16)["dq"], ref["dq"]) for s in (0, 1)}
    assert c[1] > c[0], c  # smoothing helps the INT8 scores, as in the forward
