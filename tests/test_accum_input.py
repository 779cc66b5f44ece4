"""The P~V accumulator stress input separates fp32 accumulation from narrower forms.

The FP8 P~V variant follows the SageAttention2 abstract ("two-level accumulation
strategy for P~V to enhance the accuracy of FP8 P~V"): the P~V sums must not live in
an accumulator narrower than fp32.  On gfx950 the FP8 matrix instruction accumulates
in fp32, and the kernel lets it accumulate every key tile straight into O.  The GPU
test `test_fp8_pv_accumulator_is_fp32` runs workloads.make_accum_stress through the
kernel; this CPU test shows that its input would expose a narrower accumulator.

Model: O = sum over key tiles of the tile's exact sum of P~8 * V8 products (64 keys),
added to an accumulator that rounds to w significand bits after every addition.  The
codes and scales are the oracle's.  fp32 (24 bits, round to nearest even) must stay
well inside the O bar; an accumulator of 20 bits, or a 22-bit one that truncates,
must exceed it.
"""
import numpy as np

import workloads

TOL_MAX_ABS = 2e-3


def _round_bits(x, w, mode):
    m, e = np.frexp(x)
    s = 2.0 ** w
    m = np.round(m * s) / s if mode == "rne" else np.trunc(m * s) / s
    return np.ldexp(m, e)


def _o_error(codes, v_scale, N, w, mode):
    prod = 448.0 * codes  # P~ * 448 = 448 for every key (Q = 0)
    parts = prod.reshape(N // 64, 64, -1).sum(axis=1)
    acc = np.zeros(parts.shape[1])
    for t in range(parts.shape[0]):
        acc = _round_bits(acc + parts[t], w, mode)
    scale = v_scale.astype(np.float64) / (448.0 * N)  # l = N: every P~ is 1
    return float(np.abs((acc - prod.sum(axis=0)) * scale).max()), float(np.abs(prod.sum(axis=0) * scale).max())


def test_accum_stress_input_separates_accumulator_widths(orc):
    c = workloads.make_accum_stress()
    N, d = c["N"], c["d"]
    r = orc.quant(c["q"], c["k"], c["v"], with_v=True)
    codes = orc.e4m3_decode(r["v_f8"][0, 0, :, :N]).T  # [N, d]
    vs = r["v_scale"][0, 0]
    assert np.all(np.abs(codes).max(axis=0) == 448.0)
    err = {(w, m): _o_error(codes, vs, N, w, m)[0] for w, m in ((24, "rne"), (20, "rne"), (22, "rz"), (16, "rne"))}
    omax = _o_error(codes, vs, N, 53, "rne")[1]
    assert 0.05 < omax < 0.25  # a small result after the cancellation: fp16 keeps it to 2^-13
    assert err[(24, "rne")] < TOL_MAX_ABS / 5, err
    assert err[(20, "rne")] > TOL_MAX_ABS, err
    assert err[(22, "rz")] > 2 * TOL_MAX_ABS, err
    assert err[(16, "rne")] > 10 * TOL_MAX_ABS, err
