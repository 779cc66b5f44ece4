"""Seeded synthetic workloads for the 8-bit attention forward.

This module only draws inputs; it holds none of the attention method's
arithmetic.  Both the oracle side and the GPU side are fed the same fp16 bytes
from here.

The pages measure on real Q/K/V activations of language, image and video
models (SageAttention summary page, "Key points"); those tensors are not
available, so these recipes stand in for them.  Each keeps the property the
pages say matters: K carries a per-channel offset shared by all tokens
(the channel-wise outlier that K smoothing removes, SageAttention summary page,
"Summary" and "Interesting ideas" I1).

Recipe (per config): Q, V ~ N(0, 1); K = N(0, 1) + off[b, h, c] with
off ~ N(0, sigma) drawn once per (b, h, channel); config 3 additionally
multiplies exactly ceil(0.01 * B * H * d) (b, h, channel) columns of K by 20.
Values are drawn in fp64, rounded to fp32, then to fp16 (nearest even).
Sub-streams of the seed: Q = 0, K = 1, V = 2, offsets = 3, outlier choice = 4,
Q offsets (only for the Q-smoothing stress input) = 5, V offsets (only for the
V-smoothing stress input) = 6.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gen.c")
_LIB = os.path.join(_HERE, "libgen.so")

# Shapes, masks and quantisation blocks of the five workloads.
CONFIGS = {
    1: dict(name="tiny-noncausal", B=1, H=2, N=256, d=64, causal=0, variant=0,
            blk_q=64, blk_k=64, k_sigma=5.0),
    2: dict(name="llm-prefill-causal", B=4, H=32, N=4096, d=128, causal=1, variant=0,
            blk_q=128, blk_k=64, k_sigma=5.0),
    3: dict(name="image-gen-noncausal", B=2, H=24, N=8192, d=64, causal=0, variant=0,
            blk_q=128, blk_k=64, k_sigma=3.0, outlier_frac=0.01, outlier_mult=20.0),
    4: dict(name="video-dit-long-noncausal", B=1, H=48, N=17776, d=64, causal=0, variant=0,
            blk_q=128, blk_k=64, k_sigma=5.0),
    5: dict(name="sa2-style-causal-fp8pv", B=2, H=32, N=32768, d=128, causal=1, variant=1,
            blk_q=128, blk_k=64, k_sigma=5.0),
}


def build(force: bool = False) -> str:
    """Compile gen.c into libgen.so (gcc, OpenMP)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _get():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        u64, i64, p = ctypes.c_uint64, ctypes.c_int64, ctypes.c_void_p
        lib.gen_uniform.argtypes = [u64, u64, u64, u64, p]
        lib.gen_normal.argtypes = [u64, u64, u64, u64, p]
        lib.gen_tensor.argtypes = [u64, u64, i64, i64, i64, p, p, p]
        _lib = lib
    return _lib


def uniform(seed: int, sid: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        _get().gen_uniform(seed, sid, start, n, out.ctypes.data)
    return out


def normal(seed: int, sid: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.float64)
    if n:
        _get().gen_normal(seed, sid, start, n, out.ctypes.data)
    return out


def tensor_f16(seed: int, sid: int, G: int, N: int, d: int,
               shift: np.ndarray | None = None, scale: np.ndarray | None = None) -> np.ndarray:
    """[G, N, d] fp16 tensor: fp16(fp32((z + shift[g, c]) * scale[g, c]))."""
    out32 = np.empty((G, N, d), dtype=np.float32)
    sh = None if shift is None else np.ascontiguousarray(shift, dtype=np.float64).reshape(G * d)
    sc = None if scale is None else np.ascontiguousarray(scale, dtype=np.float64).reshape(G * d)
    if out32.size:
        _get().gen_tensor(seed, sid, G, N, d,
                          None if sh is None else sh.ctypes.data,
                          None if sc is None else sc.ctypes.data, out32.ctypes.data)
    return out32.astype(np.float16)


def config(cfg) -> dict:
    return dict(CONFIGS[cfg]) if isinstance(cfg, int) else dict(cfg)


def make_inputs(cfg, seed: int | None = None, N: int | None = None, B: int | None = None,
                H: int | None = None, q_sigma: float = 0.0, v_sigma: float = 0.0,
                v_spread: float = 1.0) -> dict:
    """Draw Q, K, V (fp16, [B, H, N, d]) for a config.

    N, B, H override the config's shape (same recipe, other size).  q_sigma > 0
    adds a per-channel offset ~ N(0, q_sigma) to Q as well (stress input for Q
    smoothing); v_sigma > 0 does the same for V (stress input for V smoothing), and
    v_spread scales V's token noise: V = v_spread * z + off, off ~ N(0, v_sigma).
    """
    c = config(cfg)
    cid = cfg if isinstance(cfg, int) else 0
    if seed is None:
        seed = 1000 + cid
    if N is not None:
        c["N"] = N
    if B is not None:
        c["B"] = B
    if H is not None:
        c["H"] = H
    Bv, Hv, Nv, d = c["B"], c["H"], c["N"], c["d"]
    G = Bv * Hv
    off = normal(seed, 3, G * d).reshape(G, d) * c.get("k_sigma", 0.0)
    mult = None
    frac = c.get("outlier_frac", 0.0)
    if frac > 0:
        n_out = math.ceil(frac * G * d)
        # choose n_out (head, channel) columns without replacement: the indices
        # of the n_out smallest uniforms of stream 4
        idx = np.argsort(uniform(seed, 4, G * d), kind="stable")[:n_out]
        mult = np.ones(G * d)
        mult[idx] = c["outlier_mult"]
        mult = mult.reshape(G, d)
        c["outlier_columns"] = np.sort(idx)
    q_shift = None
    if q_sigma > 0:
        q_shift = normal(seed, 5, G * d).reshape(G, d) * q_sigma
    v_shift = v_mult = None
    if v_sigma > 0:
        v_shift = normal(seed, 6, G * d).reshape(G, d) * (v_sigma / v_spread)
    if v_spread != 1.0:
        v_mult = np.full((G, d), v_spread)
    q = tensor_f16(seed, 0, G, Nv, d, shift=q_shift)
    k = tensor_f16(seed, 1, G, Nv, d, shift=off, scale=mult)
    v = tensor_f16(seed, 2, G, Nv, d, shift=v_shift, scale=v_mult)
    shp = (Bv, Hv, Nv, d)
    c.update(seed=seed, q=q.reshape(shp), k=k.reshape(shp), v=v.reshape(shp))
    return c


def make_accum_stress(N: int = 16384, d: int = 128, big: float = 640.0, seed: int = 11) -> dict:
    """Input that separates an fp32 P~V accumulator from narrower ones (FP8 P~V variant).

    Q = 0, so every score is 0 and every P~ * 448 is exactly 448.  K follows workload 5's
    recipe (it does not matter).  In each V channel the first half of the tokens is +big
    and the second half -big (the sign chosen per channel), except exactly N/16 random
    tokens of each half, which hold U(0, 2): the running sum of P~ V climbs to about
    N/2 * 448^2 and cancels back to a small result (|O| about 0.125), so the rounding of
    every tile's addition at the peak magnitude shows in O.  Token 0 keeps +-big, so
    every channel's absmax is big.  Drawn with numpy's PCG64 (seed).
    """
    rng = np.random.default_rng(seed)
    sign = np.where(rng.random(d) < 0.5, 1.0, -1.0)
    v = np.empty((N, d), np.float64)
    v[: N // 2] = big * sign
    v[N // 2:] = -big * sign
    k_small = N // 16
    for c in range(d):
        for lo in (1, N // 2):
            idx = lo + rng.choice(N // 2 - 1, k_small, replace=False)
            v[idx, c] = rng.uniform(0.0, 2.0, k_small)
    kin = make_inputs(5, B=1, H=1, N=N)
    return dict(name="accum-stress", B=1, H=1, N=N, d=d, causal=0, variant=1, blk_q=128, blk_k=64,
                smooth_q=0, q=np.zeros((1, 1, N, d), np.float16), k=kin["k"][..., :d].copy(),
                v=v.astype(np.float16).reshape(1, 1, N, d))


def attention_ops(B: int, H: int, N: int, d: int, causal: int) -> float:
    """Operation count the throughput metric uses: 4*B*H*N^2*d, halved for causal."""
    ops = 4.0 * B * H * N * N * d
    return ops / 2 if causal else ops
