"""CPU oracle of the SageAttention 8-bit attention forward (ctypes over oracle.c).

TEST INFRASTRUCTURE ONLY: tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package; the GPU product path never does.

Every function works on numpy arrays.  Tensors are [B, H, N, d] fp16 (numpy
float16), as the GPU path takes them.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
CFLAGS = ["-O2", "-ffp-contract=off", "-fno-fast-math", "-std=c11", "-fPIC", "-shared", "-pthread"]


def build(force: bool = False, src: str = _SRC, out: str = _LIB) -> str:
    """Compile oracle.c with gcc (no fast-math, no contraction)."""
    if force or not os.path.exists(out) or os.path.getmtime(out) < os.path.getmtime(src):
        tmp = out + ".tmp"
        subprocess.check_call(["gcc", *CFLAGS, src, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


def load(path: str | None = None):
    """Load an oracle library (the default build, or another path for tests)."""
    if path is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        path = _LIB
    lib = ctypes.CDLL(path)
    p, i, d, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_double, ctypes.c_size_t
    lib.oracle_attn_rows.argtypes = [p, p, p, i, i, i, i, i, d, i, i, i, i, i, i, i, i, i, p, p, i, p, i, p]
    lib.oracle_attn_rows.restype = i
    lib.oracle_quant.argtypes = [p, p, p, i, i, i, i, i, i, i, i, i, i, p, p, p, p, p, p, p, p, p]
    lib.oracle_quant.restype = i
    lib.oracle_quant_mx.argtypes = [p, p, i, i, i, i, i, p, p, p, p, p]
    lib.oracle_quant_mx.restype = i
    lib.oracle_quant_v_mx.argtypes = [p, i, i, i, i, i, p, p, p]
    lib.oracle_quant_v_mx.restype = i
    lib.oracle_p_block_fp4.argtypes = [p, i, p, p]
    lib.oracle_p_block_fp4.restype = None
    lib.oracle_qk_int32.argtypes = [p, p, i, i, i, i, i, i, p]
    lib.oracle_qk_int32.restype = i
    lib.oracle_attn_bwd.argtypes = [p, p, p, p, p, i, i, i, i, i, d, i, i, i, i, i, p, p, p, i]
    lib.oracle_attn_bwd.restype = i
    lib.oracle_qsmooth_terms.argtypes = [p, i, p, i, ctypes.c_float, p, p]
    lib.oracle_qsmooth_terms.restype = None
    lib.oracle_pad_len.argtypes = [i]
    lib.oracle_pad_len.restype = i
    for name in ("oracle_f16_decode_n", "oracle_f16_encode_n", "oracle_e4m3_decode_n",
                 "oracle_e4m3_encode_n", "oracle_e2m1_decode_n", "oracle_e2m1_encode_n"):
        getattr(lib, name).argtypes = [p, sz, p]
        getattr(lib, name).restype = None
    return lib


class Oracle:
    """Thin numpy front end of one oracle library."""

    def __init__(self, path: str | None = None):
        self.lib = load(path)

    # ---- number formats
    def f16_decode(self, codes: np.ndarray) -> np.ndarray:
        c = np.ascontiguousarray(codes, dtype=np.uint16)
        out = np.empty(c.shape, dtype=np.float64)
        self.lib.oracle_f16_decode_n(c.ctypes.data, c.size, out.ctypes.data)
        return out

    def f16_encode(self, x: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint16)
        self.lib.oracle_f16_encode_n(a.ctypes.data, a.size, out.ctypes.data)
        return out

    def e4m3_decode(self, codes: np.ndarray) -> np.ndarray:
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(c.shape, dtype=np.float64)
        self.lib.oracle_e4m3_decode_n(c.ctypes.data, c.size, out.ctypes.data)
        return out

    def e2m1_decode(self, codes: np.ndarray) -> np.ndarray:
        c = np.ascontiguousarray(codes, dtype=np.uint8)
        out = np.empty(c.shape, dtype=np.float64)
        self.lib.oracle_e2m1_decode_n(c.ctypes.data, c.size, out.ctypes.data)
        return out

    def e2m1_encode(self, x: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint8)
        self.lib.oracle_e2m1_encode_n(a.ctypes.data, a.size, out.ctypes.data)
        return out

    def e4m3_encode(self, x: np.ndarray) -> np.ndarray:
        a = np.ascontiguousarray(x, dtype=np.float64)
        out = np.empty(a.shape, dtype=np.uint8)
        self.lib.oracle_e4m3_encode_n(a.ctypes.data, a.size, out.ctypes.data)
        return out

    def qsmooth_terms(self, qmean, khat, kscale, dk) -> np.ndarray:
        """FP8 path: the Q-smoothing terms (fp32) of the keys khat [n, d] (int8) with scales
        dk [n] for one Q-block mean qmean [d] (fp32), kscale = sm_scale * log2(e) (fp32)."""
        qm = np.ascontiguousarray(qmean, dtype=np.float32)
        kh = np.ascontiguousarray(khat, dtype=np.int8)
        dkv = np.ascontiguousarray(dk, dtype=np.float32)
        n, d = kh.shape
        out = np.empty(n, np.float32)
        self.lib.oracle_qsmooth_terms(qm.ctypes.data, d, kh.ctypes.data, n, float(kscale), dkv.ctypes.data,
                                      out.ctypes.data)
        return out

    def pad_len(self, N: int) -> int:
        return self.lib.oracle_pad_len(N)

    # ---- steps 1-3
    def quant(self, q, k, v=None, blk_q=128, blk_k=64, smooth_k=1, smooth_q=0, with_v=False, smooth_v=0,
              q_group=None) -> dict:
        """q_group: rows per Q scale (divides blk_q; default blk_q)."""
        q = _f16(q)
        k = _f16(k)
        B, H, N, d = q.shape
        G, Np = B * H, self.pad_len(N)
        if q_group is None:
            q_group = blk_q
        nqb, nkb, nqg = -(-N // blk_q), -(-N // blk_k), -(-N // q_group)
        r = dict(q_i8=np.empty((B, H, Np, d), np.int8), k_i8=np.empty((B, H, Np, d), np.int8),
                 q_scale=np.empty((B, H, nqg), np.float32), k_scale=np.empty((B, H, nkb), np.float32),
                 k_mean=np.empty((B, H, d), np.float32), q_mean=np.empty((B, H, nqb, d), np.float32))
        vp = 0
        if with_v:
            v = _f16(v)
            r["v_f8"] = np.empty((B, H, d, Np), np.uint8)
            r["v_scale"] = np.empty((B, H, d), np.float32)
            r["v_mean"] = np.empty((B, H, d), np.float32)
            vp = v.ctypes.data
        rc = self.lib.oracle_quant(
            q.ctypes.data, k.ctypes.data, vp, B, H, N, d, blk_q, blk_k, q_group, smooth_k, smooth_q, smooth_v,
            r["q_i8"].ctypes.data, r["k_i8"].ctypes.data, r["q_scale"].ctypes.data,
            r["k_scale"].ctypes.data, r["k_mean"].ctypes.data, r["q_mean"].ctypes.data,
            r["v_f8"].ctypes.data if with_v else None, r["v_scale"].ctypes.data if with_v else None,
            r["v_mean"].ctypes.data if with_v else None)
        if rc:
            raise ValueError("oracle_quant: bad arguments")
        return r

    def quant_mx(self, q, k, smooth_k=1) -> dict:
        """Variant 2 (MXFP4) tensors: E2M1 codes one per byte [B, H, Np, d], E8M0 block
        scales [B, H, Np, d/32], k_mean [B, H, d]."""
        q = _f16(q)
        k = _f16(k)
        B, H, N, d = q.shape
        Np = self.pad_len(N)
        r = dict(q_codes=np.empty((B, H, Np, d), np.uint8), k_codes=np.empty((B, H, Np, d), np.uint8),
                 q_e8=np.empty((B, H, Np, d // 32), np.uint8), k_e8=np.empty((B, H, Np, d // 32), np.uint8),
                 k_mean=np.empty((B, H, d), np.float32))
        rc = self.lib.oracle_quant_mx(q.ctypes.data, k.ctypes.data, B, H, N, d, smooth_k, r["q_codes"].ctypes.data,
                                      r["k_codes"].ctypes.data, r["q_e8"].ctypes.data, r["k_e8"].ctypes.data,
                                      r["k_mean"].ctypes.data)
        if rc:
            raise ValueError("oracle_quant_mx: bad arguments")
        return r

    def quant_v_mx(self, v, smooth_v=0) -> dict:
        """Variant 3's V: E2M1 codes one per byte [B, H, d, Np] (tokens along the last axis),
        E8M0 scales [B, H, d, Np/32] (one per channel and block of 32 tokens), v_mean [B, H, d]."""
        v = _f16(v)
        B, H, N, d = v.shape
        Np = self.pad_len(N)
        r = dict(v_codes=np.empty((B, H, d, Np), np.uint8), v_e8=np.empty((B, H, d, Np // 32), np.uint8),
                 v_mean=np.empty((B, H, d), np.float32))
        rc = self.lib.oracle_quant_v_mx(v.ctypes.data, B, H, N, d, int(smooth_v), r["v_codes"].ctypes.data,
                                        r["v_e8"].ctypes.data, r["v_mean"].ctypes.data)
        if rc:
            raise ValueError("oracle_quant_v_mx: bad arguments")
        return r

    def p_block_fp4(self, p) -> tuple:
        """Variant 3's MXFP4 rule for attention weights: p [n, 32] fp32 -> (codes [n, 32], e8 [n])."""
        a = np.ascontiguousarray(p, dtype=np.float32).reshape(-1, 32)
        codes = np.empty(a.shape, np.uint8)
        e8 = np.empty(a.shape[0], np.uint8)
        self.lib.oracle_p_block_fp4(a.ctypes.data, a.shape[0], codes.ctypes.data, e8.ctypes.data)
        return codes, e8

    # ---- step 4
    def qk_int32(self, q_i8_head, k_i8_head, r0, nr, c0, nc) -> np.ndarray:
        a = np.ascontiguousarray(q_i8_head, dtype=np.int8)
        b = np.ascontiguousarray(k_i8_head, dtype=np.int8)
        Np, d = a.shape
        out = np.empty((nr, nc), np.int32)
        if self.lib.oracle_qk_int32(a.ctypes.data, b.ctypes.data, Np, d, r0, nr, c0, nc, out.ctypes.data):
            raise ValueError("oracle_qk_int32: bad arguments")
        return out

    # ---- steps 1-9 for chosen rows
    def attn_rows(self, q, k, v, heads, rows, causal=0, sm_scale=None, variant=0, blk_q=128,
                  blk_k=64, bkv=64, smooth_k=1, smooth_q=None, smooth_v=0, exact=0, nthreads=0, q_group=None):
        """O (fp64, before the fp16 rounding) for rows[i] of flat head heads[i].
        q_group: rows per Q scale (divides blk_q; default blk_q)."""
        q, k, v = _f16(q), _f16(k), _f16(v)
        B, H, N, d = q.shape
        if sm_scale is None:
            sm_scale = 1.0 / np.sqrt(d)
        if smooth_q is None:
            smooth_q = 1 if variant == 1 else 0
        if q_group is None:
            q_group = blk_q
        heads = np.ascontiguousarray(heads, dtype=np.int32)
        rows = np.ascontiguousarray(rows, dtype=np.int32)
        out = np.empty((heads.size, d), np.float64)
        used = ctypes.c_int(0)
        rc = self.lib.oracle_attn_rows(
            q.ctypes.data, k.ctypes.data, v.ctypes.data, B, H, N, d, causal, float(sm_scale), variant,
            blk_q, blk_k, bkv, q_group, smooth_k, smooth_q, smooth_v, exact, heads.ctypes.data, rows.ctypes.data,
            heads.size, out.ctypes.data, nthreads, ctypes.byref(used))
        if rc:
            raise ValueError("oracle_attn_rows: bad arguments")
        self.threads_used = used.value
        return out

    def attn_bwd(self, q, k, v, o, dout, causal=0, sm_scale=None, blk_q=128, blk_k=64, smooth_k=1, smooth_v=1,
                 exact=0, nthreads=0) -> dict:
        """dq, dk, dv ([B, H, N, d] fp64) of the 8-bit forward (variant-0 scores) given its output
        o and the output gradient dout (fp16 arrays).  exact=1: no quantisation or rounding."""
        q, k, v, o, dout = _f16(q), _f16(k), _f16(v), _f16(o), _f16(dout)
        B, H, N, d = q.shape
        for t in (k, v, o, dout):
            if t.shape != q.shape:
                raise ValueError("q, k, v, o, dout must share one shape")
        if sm_scale is None:
            sm_scale = 1.0 / np.sqrt(d)
        r = {n: np.empty((B, H, N, d), np.float64) for n in ("dq", "dk", "dv")}
        rc = self.lib.oracle_attn_bwd(q.ctypes.data, k.ctypes.data, v.ctypes.data, o.ctypes.data, dout.ctypes.data,
                                      B, H, N, d, int(causal), float(sm_scale), blk_q, blk_k, int(smooth_k),
                                      int(smooth_v), int(exact), r["dq"].ctypes.data, r["dk"].ctypes.data,
                                      r["dv"].ctypes.data, nthreads)
        if rc:
            raise ValueError("oracle_attn_bwd: bad arguments")
        return r

    def attn(self, q, k, v, **kw) -> np.ndarray:
        """O for every row, [B, H, N, d] fp64."""
        B, H, N, d = q.shape
        heads = np.repeat(np.arange(B * H, dtype=np.int32), N)
        rows = np.tile(np.arange(N, dtype=np.int32), B * H)
        return self.attn_rows(q, k, v, heads, rows, **kw).reshape(B, H, N, d)


def _f16(x) -> np.ndarray:
    a = np.ascontiguousarray(x)
    if a.dtype != np.float16:
        raise TypeError(f"expected float16, got {a.dtype}")
    return a
