"""SageAttention-style 8-bit attention forward for the MI355X (gfx950).

Thin Python binding over the C ABI of libsage.so (include/sage.h): it checks
dtypes, shapes and devices, allocates outputs and the workspace with torch, and
passes raw device pointers and the current HIP stream.  Every step of the
computation runs in the HIP kernels of libsage.so; there is no other path.

Method (pages): "SageAttention: Accurate 8-Bit Attention for Plug-and-play
Inference Acceleration" (summary page, "Summary", "Interesting ideas" I1/I3) and
"SageAttention2 ..." (abstract: Q smoothing, FP8 P~/V, two-level accumulation) and
"SageAttention3 ..." (abstract: FP4 attention; variants 2 and 3 in MXFP4).
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

__all__ = ["attn", "attn_noalloc", "attn_fwd_train", "attn_bwd", "quant_qk", "quant_v", "attn_prequant", "attn_qf16",
           "attn_qf16_fp8",
           "quant_qk_mx", "attn_prequant_mx", "attn_qf16_mx", "quant_v_mx", "attn_qf16_fp4",
           "debug_qk_int32", "workspace_bytes",
           "kv_tile", "pad_len", "SageError", "library_path", "VARIANT_FP16PV", "VARIANT_FP8PV", "VARIANT_MXFP4",
           "VARIANT_FP4PV"]

VARIANT_FP16PV = 0
VARIANT_FP8PV = 1
VARIANT_MXFP4 = 2
VARIANT_FP4PV = 3

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libsage.so")
_lib = None


class SageError(RuntimeError):
    pass


class _Params(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_int), ("blk_q", ctypes.c_int), ("blk_k", ctypes.c_int),
                ("smooth_k", ctypes.c_int), ("smooth_q", ctypes.c_int), ("smooth_v", ctypes.c_int),
                ("q_group", ctypes.c_int)]


def library_path() -> str:
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise SageError(f"{_LIB_PATH} is missing: build it first "
                        "(python -c 'import __graft_entry__ as g; g.build()')")
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, F, S = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
    PP = ctypes.POINTER(_Params)
    sig = {
        "sage_version": ([], I),
        "sage_pad_len": ([I], I),
        "sage_kv_tile": ([I, I], I),
        "sage_workspace_bytes": ([I, I, I, I, I, PP], S),
        "sage_quant_qk": ([P, P, I, I, I, I, PP, P, P, P, P, P, P, P, S, P], I),
        "sage_quant_v": ([P, I, I, I, I, P, P, P, S, P], I),
        "sage_quant_v_ex": ([P, I, I, I, I, I, P, P, P, P, S, P], I),
        "sage_attn_fwd": ([P, P, P, P, I, I, I, I, I, F, I, P, S, P], I),
        "sage_attn_fwd_ex": ([P, P, P, P, I, I, I, I, I, F, I, PP, P, S, P], I),
        "sage_attn_fwd_prequant": ([P, P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, I, PP, P], I),
        "sage_attn_fwd_qf16": ([P, P, P, P, P, I, I, I, I, I, F, PP, P], I),
        "sage_attn_fwd_qf16_fp8": ([P, P, P, P, P, P, P, I, I, I, I, I, F, PP, P], I),
        "sage_quant_qk_mx": ([P, P, I, I, I, I, I, P, P, P, P, P, P, S, P], I),
        "sage_attn_fwd_prequant_mx": ([P, P, P, P, P, P, P, P, I, I, I, I, I, F, PP, P], I),
        "sage_attn_fwd_qf16_mx": ([P, P, P, P, P, P, P, I, I, I, I, I, F, PP, P], I),
        "sage_quant_v_mx": ([P, I, I, I, I, I, P, P, P, P, S, P], I),
        "sage_attn_fwd_qf16_fp4": ([P, P, P, P, P, P, P, I, I, I, I, I, F, PP, P], I),
        "sage_debug_qk_int32": ([P, P, I, I, I, I, P, I, P, P], I),
        "sage_attn_fwd_noalloc": ([P, P, P, P, I, I, I, I, I, F, I, PP, P], I),
        "sage_attn_fwd_train": ([P, P, P, P, P, I, I, I, I, I, F, PP, P, S, P], I),
        "sage_attn_bwd_workspace_bytes": ([I, I, I, I, PP], S),
        "sage_attn_bwd": ([P, P, P, P, P, P, P, P, P, I, I, I, I, I, F, PP, P, S, P], I),
        "sage_last_error": ([], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    _lib = lib
    return lib


def _check(rc: int, what: str):
    if rc != 0:
        msg = _load().sage_last_error().decode()
        raise SageError(f"{what} failed ({rc}): {msg}")


def _params(blk_q=128, blk_k=64, smooth_k=True, smooth_q=False, smooth_v=False, q_group=0) -> _Params:
    return _Params(ctypes.sizeof(_Params), int(blk_q), int(blk_k), int(bool(smooth_k)), int(bool(smooth_q)),
                   int(bool(smooth_v)), int(q_group))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _check_qkv(*ts):
    ref = ts[0]
    for t in ts:
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float16:
            raise TypeError("q, k, v must be float16 tensors")
        if not t.is_cuda:
            raise ValueError("q, k, v must be on a GPU")
        if t.dim() != 4 or t.shape != ref.shape or t.device != ref.device:
            raise ValueError("q, k, v must share one [B, H, N, d] shape and device")
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    return ref.shape


def _check_out(out, shape, device):
    """A caller-supplied output must be a contiguous fp16 [B, H, N, d] tensor on the inputs' GPU;
    None allocates one."""
    if out is None:
        return torch.empty(shape, dtype=torch.float16, device=device)
    if not isinstance(out, torch.Tensor) or out.dtype != torch.float16:
        raise TypeError("out must be a float16 tensor")
    if tuple(out.shape) != tuple(shape):
        raise ValueError(f"out must have shape {tuple(shape)}, got {tuple(out.shape)}")
    if out.device != device:
        raise ValueError("out must be on the same device as the inputs")
    if not out.is_contiguous():
        raise ValueError("out must be contiguous")
    return out


def _check_tensor(t, name, shape, dtype, device):
    """A pre-quantised operand: a contiguous tensor of exactly this shape and dtype on `device`."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != device:
        raise ValueError(f"{name} must be on {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _check_n(N, Np):
    """N of a pre-quantised call must be the length the padded tensors were made for."""
    N = int(N)
    if N < 1 or pad_len(N) != Np:
        raise ValueError(f"N = {N} does not match the padded length {Np} of the quantised tensors")
    return N


def pad_len(N: int) -> int:
    return _load().sage_pad_len(N)


def kv_tile(variant: int, d: int) -> int:
    return _load().sage_kv_tile(variant, d)


def workspace_bytes(B, H, N, d, variant=0, blk_q=128, blk_k=64, smooth_k=True, smooth_q=None,
                    smooth_v=False, q_group=0) -> int:
    if smooth_q is None:
        smooth_q = variant == VARIANT_FP8PV
    p = _params(blk_q, blk_k, smooth_k, smooth_q, smooth_v, q_group)
    return _load().sage_workspace_bytes(B, H, N, d, variant, ctypes.byref(p))


def _workspace(nbytes, device, workspace):
    if workspace is not None:
        if not isinstance(workspace, torch.Tensor) or workspace.device != device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the inputs' device")
        if workspace.numel() * workspace.element_size() < nbytes:
            raise ValueError("workspace too small")
        return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def attn(q, k, v, causal=False, sm_scale=None, variant=VARIANT_FP16PV, blk_q=128, blk_k=64,
         smooth_k=True, smooth_q=None, smooth_v=False, q_group=0, out=None, workspace=None):
    """o = SageAttention(q, k, v) for [B, H, N, d] fp16 tensors on the GPU.

    An empty input (B, H or N zero) returns the empty output without a launch.

    smooth_v (variants 1-3) subtracts V's token mean before FP8 / MXFP4 and adds it to O.
    q_group: rows per Q scale (0 = blk_q; 1 = per token)."""
    B, H, N, d = _check_qkv(q, k, v)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if smooth_q is None:
        smooth_q = variant == VARIANT_FP8PV
    out = _check_out(out, q.shape, q.device)
    if q.numel() == 0:  # no heads or no tokens: nothing to compute (the C ABI wants B, H, N >= 1)
        return out
    p = _params(blk_q, blk_k, smooth_k, smooth_q, smooth_v, q_group)
    lib = _load()
    nbytes = lib.sage_workspace_bytes(B, H, N, d, variant, ctypes.byref(p))
    if nbytes == 0:
        _check(-1, "sage_workspace_bytes")
    ws = _workspace(nbytes, q.device, workspace)
    rc = lib.sage_attn_fwd_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, int(bool(causal)),
                              float(sm_scale), int(variant), ctypes.byref(p), _ptr(ws),
                              ws.numel() * ws.element_size(), _stream(q.device))
    _check(rc, "sage_attn_fwd_ex")
    return out


# Workspace of attn_noalloc: the library's own array per GPU (SAGE_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 128 * 1024 * 1024


def attn_noalloc(q, k, v, out, causal=False, sm_scale=None, variant=VARIANT_FP16PV, blk_q=128, blk_k=64,
                 smooth_k=True, smooth_q=None, smooth_v=False, q_group=0):
    """attn() without any device allocation: the caller passes `out` (a contiguous fp16
    [B, H, N, d] tensor), and the library uses its own per-GPU workspace array
    (sage_attn_fwd_noalloc).  Shapes whose workspace exceeds NOALLOC_SCRATCH_BYTES raise
    SageError.  Calls that overlap in time on one GPU share that array and race."""
    B, H, N, d = _check_qkv(q, k, v)
    if out is None:
        raise ValueError("attn_noalloc needs a caller-allocated out")
    out = _check_out(out, q.shape, q.device)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if smooth_q is None:
        smooth_q = variant == VARIANT_FP8PV
    if q.numel() == 0:
        return out
    p = _params(blk_q, blk_k, smooth_k, smooth_q, smooth_v, q_group)
    rc = _load().sage_attn_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(out), B, H, N, d, int(bool(causal)),
                                       float(sm_scale), int(variant), ctypes.byref(p), _stream(q.device))
    _check(rc, "sage_attn_fwd_noalloc")
    return out


def attn_fwd_train(q, k, v, causal=False, sm_scale=None, blk_q=128, blk_k=64, smooth_k=True, out=None, lse=None,
                   workspace=None):
    """The variant-0 forward for training: returns (o, lse), lse [B, H, N] fp32 the natural-log
    row log-sum-exp of the dequantised scores, which attn_bwd takes.  blk_q must be 64 or 128."""
    B, H, N, d = _check_qkv(q, k, v)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    out = _check_out(out, q.shape, q.device)
    if lse is None:
        lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    _check_tensor(lse, "lse", (B, H, N), torch.float32, q.device)
    if q.numel() == 0:
        return out, lse
    p = _params(blk_q, blk_k, smooth_k, False, False, 0)
    lib = _load()
    nbytes = lib.sage_workspace_bytes(B, H, N, d, VARIANT_FP16PV, ctypes.byref(p))
    if nbytes == 0:
        _check(-1, "sage_workspace_bytes")
    ws = _workspace(nbytes, q.device, workspace)
    rc = lib.sage_attn_fwd_train(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(lse), B, H, N, d, int(bool(causal)),
                                 float(sm_scale), ctypes.byref(p), _ptr(ws), ws.numel() * ws.element_size(),
                                 _stream(q.device))
    _check(rc, "sage_attn_fwd_train")
    return out, lse


def attn_bwd(q, k, v, o, dout, lse, causal=False, sm_scale=None, blk_q=128, blk_k=64, smooth_k=True,
             workspace=None) -> dict:
    """dq, dk, dv ([B, H, N, d] fp32) of the 8-bit forward at q, k, v given its output o, the
    output gradient dout (fp16 like q) and the lse of attn_fwd_train (same options)."""
    B, H, N, d = _check_qkv(q, k, v, o, dout)
    _check_tensor(lse, "lse", (B, H, N), torch.float32, q.device)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    r = {n: torch.empty((B, H, N, d), dtype=torch.float32, device=q.device) for n in ("dq", "dk", "dv")}
    if q.numel() == 0:
        return r
    p = _params(blk_q, blk_k, smooth_k, False, False, 0)
    lib = _load()
    nbytes = lib.sage_attn_bwd_workspace_bytes(B, H, N, d, ctypes.byref(p))
    if nbytes == 0:
        _check(-1, "sage_attn_bwd_workspace_bytes")
    ws = _workspace(nbytes, q.device, workspace)
    rc = lib.sage_attn_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(r["dq"]), _ptr(r["dk"]),
                           _ptr(r["dv"]), B, H, N, d, int(bool(causal)), float(sm_scale), ctypes.byref(p), _ptr(ws),
                           ws.numel() * ws.element_size(), _stream(q.device))
    _check(rc, "sage_attn_bwd")
    return r


def quant_qk(q, k, blk_q=128, blk_k=64, smooth_k=True, smooth_q=False, q_group=0) -> dict:
    """Smoothing + per-block INT8 of Q and K.  Returns the int8 tensors, scales and means."""
    B, H, N, d = _check_qkv(q, k)
    dev = q.device
    Np = pad_len(N)
    nqb, nkb, nqg = -(-N // blk_q), -(-N // blk_k), -(-N // (q_group or blk_q))
    r = dict(q_i8=torch.empty((B, H, Np, d), dtype=torch.int8, device=dev),
             k_i8=torch.empty((B, H, Np, d), dtype=torch.int8, device=dev),
             q_scale=torch.empty((B, H, nqg), dtype=torch.float32, device=dev),
             k_scale=torch.empty((B, H, nkb), dtype=torch.float32, device=dev),
             k_mean=torch.zeros((B, H, d), dtype=torch.float32, device=dev),
             q_mean=torch.zeros((B, H, nqb, d), dtype=torch.float32, device=dev))
    p = _params(blk_q, blk_k, smooth_k, smooth_q, False, q_group)
    lib = _load()
    ws = _workspace(lib.sage_workspace_bytes(B, H, N, d, 0, ctypes.byref(p)), dev, None)
    rc = lib.sage_quant_qk(_ptr(q), _ptr(k), B, H, N, d, ctypes.byref(p), _ptr(r["q_i8"]), _ptr(r["k_i8"]),
                           _ptr(r["q_scale"]), _ptr(r["k_scale"]), _ptr(r["k_mean"]),
                           _ptr(r["q_mean"]) if smooth_q else None, _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "sage_quant_qk")
    return r


def quant_v(v, smooth_v=False) -> dict:
    """FP8 E4M3 V with per-channel scales: v_f8 [B, H, d, Np] (uint8 codes), v_scale [B, H, d],
    v_mean [B, H, d] (the token mean taken out with smooth_v, else zeros)."""
    B, H, N, d = _check_qkv(v)
    dev = v.device
    Np = pad_len(N)
    r = dict(v_f8=torch.empty((B, H, d, Np), dtype=torch.uint8, device=dev),
             v_scale=torch.empty((B, H, d), dtype=torch.float32, device=dev),
             v_mean=torch.zeros((B, H, d), dtype=torch.float32, device=dev))
    lib = _load()
    ws = _workspace(lib.sage_workspace_bytes(B, H, N, d, 1, None), dev, None)
    rc = lib.sage_quant_v_ex(_ptr(v), B, H, N, d, int(bool(smooth_v)), _ptr(r["v_f8"]), _ptr(r["v_scale"]),
                             _ptr(r["v_mean"]), _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "sage_quant_v_ex")
    return r


def attn_prequant(qk: dict, v, N, causal=False, sm_scale=None, variant=VARIANT_FP16PV, vq: dict | None = None,
                  blk_q=128, blk_k=64, smooth_q=None, smooth_v=False, q_group=0, out=None):
    """The attention kernel alone, on quant_qk() / quant_v() outputs (quant_v(smooth_v=True) with
    smooth_v)."""
    if variant not in (VARIANT_FP16PV, VARIANT_FP8PV):
        raise ValueError("attn_prequant takes variant 0 or 1 (the MXFP4 variant: attn_prequant_mx)")
    B, H, Np, d = qk["q_i8"].shape
    dev = qk["q_i8"].device
    N = _check_n(N, Np)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    if smooth_q is None:
        smooth_q = variant == VARIANT_FP8PV
    nqb, nkb, nqg = -(-N // blk_q), -(-N // blk_k), -(-N // (q_group or blk_q))
    _check_tensor(qk["q_i8"], "q_i8", (B, H, Np, d), torch.int8, dev)
    _check_tensor(qk["k_i8"], "k_i8", (B, H, Np, d), torch.int8, dev)
    _check_tensor(qk["q_scale"], "q_scale", (B, H, nqg), torch.float32, dev)
    _check_tensor(qk["k_scale"], "k_scale", (B, H, nkb), torch.float32, dev)
    if smooth_q:
        _check_tensor(qk["q_mean"], "q_mean", (B, H, nqb, d), torch.float32, dev)
    if variant == VARIANT_FP16PV:
        _check_tensor(v, "v", (B, H, N, d), torch.float16, dev)
    else:
        if vq is None:
            raise ValueError("variant 1 needs the FP8 V of quant_v()")
        _check_tensor(vq["v_f8"], "v_f8", (B, H, d, Np), torch.uint8, dev)
        _check_tensor(vq["v_scale"], "v_scale", (B, H, d), torch.float32, dev)
        if smooth_v:
            _check_tensor(vq["v_mean"], "v_mean", (B, H, d), torch.float32, dev)
    out = _check_out(out, (B, H, N, d), dev)
    p = _params(blk_q, blk_k, True, smooth_q, smooth_v, q_group)
    rc = _load().sage_attn_fwd_prequant(
        _ptr(qk["q_i8"]), _ptr(qk["k_i8"]), _ptr(qk["q_scale"]), _ptr(qk["k_scale"]),
        _ptr(qk["q_mean"]) if smooth_q else None, _ptr(v) if variant == 0 else None,
        _ptr(vq["v_f8"]) if variant == 1 else None, _ptr(vq["v_scale"]) if variant == 1 else None,
        _ptr(vq["v_mean"]) if smooth_v else None, _ptr(out), B, H, N, d, int(bool(causal)), float(sm_scale), int(variant), ctypes.byref(p), _stream(dev))
    _check(rc, "sage_attn_fwd_prequant")
    return out


def attn_qf16(q, qk: dict, v, causal=False, sm_scale=None, blk_q=128, blk_k=64, q_group=0, smooth_q=False,
              out=None):
    """Variant 0 attention on fp16 q (quantised inside the kernel, with Q smoothing if asked) and
    the K of quant_qk()."""
    B, H, N, d = _check_qkv(q, v)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    Np = pad_len(N)
    _check_tensor(qk["k_i8"], "k_i8", (B, H, Np, d), torch.int8, q.device)
    _check_tensor(qk["k_scale"], "k_scale", (B, H, -(-N // blk_k)), torch.float32, q.device)
    out = _check_out(out, q.shape, q.device)
    p = _params(blk_q, blk_k, True, smooth_q, False, q_group)
    rc = _load().sage_attn_fwd_qf16(_ptr(q), _ptr(qk["k_i8"]), _ptr(qk["k_scale"]), _ptr(v), _ptr(out), B, H, N, d,
                                    int(bool(causal)), float(sm_scale), ctypes.byref(p), _stream(q.device))
    _check(rc, "sage_attn_fwd_qf16")
    return out


def attn_qf16_fp8(q, qk: dict, vq: dict, causal=False, sm_scale=None, blk_q=128, blk_k=64, smooth_q=True,
                  smooth_v=False, q_group=0, out=None):
    """Variant 1 attention on fp16 q (quantised, with Q smoothing by default, inside the kernel),
    the K of quant_qk() and the V of quant_v()."""
    B, H, N, d = _check_qkv(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    Np = pad_len(N)
    _check_tensor(qk["k_i8"], "k_i8", (B, H, Np, d), torch.int8, q.device)
    _check_tensor(qk["k_scale"], "k_scale", (B, H, -(-N // blk_k)), torch.float32, q.device)
    _check_tensor(vq["v_f8"], "v_f8", (B, H, d, Np), torch.uint8, q.device)
    _check_tensor(vq["v_scale"], "v_scale", (B, H, d), torch.float32, q.device)
    if smooth_v:
        _check_tensor(vq["v_mean"], "v_mean", (B, H, d), torch.float32, q.device)
    out = _check_out(out, q.shape, q.device)
    p = _params(blk_q, blk_k, True, smooth_q, smooth_v, q_group)
    rc = _load().sage_attn_fwd_qf16_fp8(
        _ptr(q), _ptr(qk["k_i8"]), _ptr(qk["k_scale"]), _ptr(vq["v_f8"]), _ptr(vq["v_scale"]),
        _ptr(vq["v_mean"]) if smooth_v else None, _ptr(out), B, H, N, d, int(bool(causal)), float(sm_scale),
        ctypes.byref(p), _stream(q.device))
    _check(rc, "sage_attn_fwd_qf16_fp8")
    return out


def quant_qk_mx(q, k, smooth_k=True) -> dict:
    """Per-token MXFP4 of Q and K' (variant 2): q_f4 / k_f4 [B, H, Np, d/2] (two E2M1 codes per
    byte), q_e8 / k_e8 [B, H, Np, d/32] (E8M0 block scales), k_mean [B, H, d]."""
    B, H, N, d = _check_qkv(q, k)
    dev = q.device
    Np = pad_len(N)
    r = dict(q_f4=torch.empty((B, H, Np, d // 2), dtype=torch.uint8, device=dev),
             k_f4=torch.empty((B, H, Np, d // 2), dtype=torch.uint8, device=dev),
             q_e8=torch.empty((B, H, Np, d // 32), dtype=torch.uint8, device=dev),
             k_e8=torch.empty((B, H, Np, d // 32), dtype=torch.uint8, device=dev),
             k_mean=torch.zeros((B, H, d), dtype=torch.float32, device=dev))
    lib = _load()
    ws = _workspace(lib.sage_workspace_bytes(B, H, N, d, VARIANT_MXFP4, None), dev, None)
    rc = lib.sage_quant_qk_mx(_ptr(q), _ptr(k), B, H, N, d, int(bool(smooth_k)), _ptr(r["q_f4"]), _ptr(r["k_f4"]),
                              _ptr(r["q_e8"]), _ptr(r["k_e8"]), _ptr(r["k_mean"]), _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "sage_quant_qk_mx")
    return r


def attn_prequant_mx(qk: dict, vq: dict, N, causal=False, sm_scale=None, smooth_v=False, out=None):
    """The variant-2 attention kernel alone, on quant_qk_mx() and quant_v() outputs."""
    B, H, Np, dh = qk["q_f4"].shape
    d = 2 * dh
    dev = qk["q_f4"].device
    N = _check_n(N, Np)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    _check_mx_operands(qk, vq, B, H, N, d, dev, smooth_v, with_q=True)
    out = _check_out(out, (B, H, N, d), dev)
    p = _params(128, 64, True, False, smooth_v)
    rc = _load().sage_attn_fwd_prequant_mx(
        _ptr(qk["q_f4"]), _ptr(qk["k_f4"]), _ptr(qk["q_e8"]), _ptr(qk["k_e8"]), _ptr(vq["v_f8"]), _ptr(vq["v_scale"]),
        _ptr(vq["v_mean"]) if smooth_v else None, _ptr(out), B, H, N, d, int(bool(causal)), float(sm_scale),
        ctypes.byref(p), _stream(dev))
    _check(rc, "sage_attn_fwd_prequant_mx")
    return out


def attn_qf16_mx(q, qk: dict, vq: dict, causal=False, sm_scale=None, smooth_v=False, out=None):
    """Variant-2 attention on fp16 q (quantised to MXFP4 inside the kernel) and the K of quant_qk_mx()."""
    B, H, N, d = _check_qkv(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    _check_mx_operands(qk, vq, B, H, N, d, q.device, smooth_v, with_q=False)
    out = _check_out(out, q.shape, q.device)
    p = _params(128, 64, True, False, smooth_v)
    rc = _load().sage_attn_fwd_qf16_mx(
        _ptr(q), _ptr(qk["k_f4"]), _ptr(qk["k_e8"]), _ptr(vq["v_f8"]), _ptr(vq["v_scale"]),
        _ptr(vq["v_mean"]) if smooth_v else None, _ptr(out), B, H, N, d, int(bool(causal)), float(sm_scale),
        ctypes.byref(p), _stream(q.device))
    _check(rc, "sage_attn_fwd_qf16_mx")
    return out


def _check_mx_operands(qk, vq, B, H, N, d, dev, smooth_v, with_q):
    Np = pad_len(N)
    names = (("q", "k") if with_q else ("k",))
    for n in names:
        _check_tensor(qk[f"{n}_f4"], f"{n}_f4", (B, H, Np, d // 2), torch.uint8, dev)
        _check_tensor(qk[f"{n}_e8"], f"{n}_e8", (B, H, Np, d // 32), torch.uint8, dev)
    _check_tensor(vq["v_f8"], "v_f8", (B, H, d, Np), torch.uint8, dev)
    _check_tensor(vq["v_scale"], "v_scale", (B, H, d), torch.float32, dev)
    if smooth_v:
        _check_tensor(vq["v_mean"], "v_mean", (B, H, d), torch.float32, dev)


def quant_v_mx(v, smooth_v=False) -> dict:
    """Variant 3's V in MXFP4 along the tokens: v_f4 [B, H, d, Np/2] (two E2M1 codes per byte, the
    lower token in the low nibble), v_e8 [B, H, Np/32, d] (E8M0, channel c at (c % 32) * (d/32) +
    c / 32), v_mean [B, H, d] (the token mean taken out with smooth_v, else zeros)."""
    B, H, N, d = _check_qkv(v)
    dev = v.device
    Np = pad_len(N)
    r = dict(v_f4=torch.empty((B, H, d, Np // 2), dtype=torch.uint8, device=dev),
             v_e8=torch.empty((B, H, Np // 32, d), dtype=torch.uint8, device=dev),
             v_mean=torch.zeros((B, H, d), dtype=torch.float32, device=dev))
    lib = _load()
    ws = _workspace(lib.sage_workspace_bytes(B, H, N, d, VARIANT_FP8PV, None), dev, None)
    rc = lib.sage_quant_v_mx(_ptr(v), B, H, N, d, int(bool(smooth_v)), _ptr(r["v_f4"]), _ptr(r["v_e8"]),
                             _ptr(r["v_mean"]), _ptr(ws), ws.numel(), _stream(dev))
    _check(rc, "sage_quant_v_mx")
    return r


def attn_qf16_fp4(q, qk: dict, vq: dict, causal=False, sm_scale=None, smooth_v=False, out=None):
    """Variant-3 attention (MXFP4 scores and MXFP4 P~V) on fp16 q (quantised inside the kernel),
    the K of quant_qk_mx() and the V of quant_v_mx()."""
    B, H, N, d = _check_qkv(q)
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(d)
    Np = pad_len(N)
    _check_tensor(qk["k_f4"], "k_f4", (B, H, Np, d // 2), torch.uint8, q.device)
    _check_tensor(qk["k_e8"], "k_e8", (B, H, Np, d // 32), torch.uint8, q.device)
    _check_tensor(vq["v_f4"], "v_f4", (B, H, d, Np // 2), torch.uint8, q.device)
    _check_tensor(vq["v_e8"], "v_e8", (B, H, Np // 32, d), torch.uint8, q.device)
    if smooth_v:
        _check_tensor(vq["v_mean"], "v_mean", (B, H, d), torch.float32, q.device)
    out = _check_out(out, q.shape, q.device)
    p = _params(128, 64, True, False, smooth_v)
    rc = _load().sage_attn_fwd_qf16_fp4(
        _ptr(q), _ptr(qk["k_f4"]), _ptr(qk["k_e8"]), _ptr(vq["v_f4"]), _ptr(vq["v_e8"]),
        _ptr(vq["v_mean"]) if smooth_v else None, _ptr(out), B, H, N, d, int(bool(causal)), float(sm_scale),
        ctypes.byref(p), _stream(q.device))
    _check(rc, "sage_attn_fwd_qf16_fp4")
    return out


def debug_qk_int32(q_i8, k_i8, N, tiles) -> torch.Tensor:
    """int32 S = Qhat Khat^T tiles (128 queries x 64 keys) as the attention kernel forms them.
    tiles: list of (flat head, query tile, key tile)."""
    B, H, Np, d = q_i8.shape
    dev = q_i8.device
    N = _check_n(N, Np)
    _check_tensor(q_i8, "q_i8", (B, H, Np, d), torch.int8, dev)
    _check_tensor(k_i8, "k_i8", (B, H, Np, d), torch.int8, dev)
    t = torch.tensor(list(tiles), dtype=torch.int32, device=dev).reshape(-1, 3).contiguous()
    out = torch.empty((t.shape[0], 128, 64), dtype=torch.int32, device=dev)
    rc = _load().sage_debug_qk_int32(_ptr(q_i8), _ptr(k_i8), B, H, N, d, _ptr(t), t.shape[0], _ptr(out),
                                     _stream(dev))
    _check(rc, "sage_debug_qk_int32")
    return out
