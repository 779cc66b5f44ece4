"""Host-only checks of the C ABI (no GPU needed, no kernel launched).

The library must load, export every function include/sage.h declares, and reject
bad arguments with the documented status before touching the HIP runtime.
"""
import ctypes
import os
import re

import pytest

import quantized_bit_attention_amd as sage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sage.h")
P = ctypes.c_void_p
A = P(0x10000)          # aligned, never dereferenced: every call below fails validation first
MIS = P(0x10002)        # misaligned


def header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(sage.library_path()):
        pytest.skip("libsage.so not built")
    return sage._load()


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), n


def test_status_codes_match_header():
    src = open(HEADER).read()
    codes = dict(re.findall(r"(SAGE_\w+)\s*=\s*(-?\d+)", src))
    assert codes["SAGE_OK"] == "0" and codes["SAGE_ERR_INVALID_ARG"] == "-1"
    assert codes["SAGE_ERR_UNSUPPORTED"] == "-2" and codes["SAGE_ERR_WORKSPACE"] == "-3"
    assert codes["SAGE_ERR_HIP"] == "-4"


def test_pure_helpers(lib):
    assert lib.sage_pad_len(1) == 128 and lib.sage_pad_len(128) == 128 and lib.sage_pad_len(17776) == 17792
    assert lib.sage_pad_len(0) == -1
    assert lib.sage_kv_tile(0, 64) == 64 and lib.sage_kv_tile(1, 128) == 64
    assert lib.sage_kv_tile(2, 64) == 64 and lib.sage_kv_tile(3, 128) == 64
    assert lib.sage_kv_tile(4, 64) < 0 and lib.sage_kv_tile(0, 96) < 0
    assert lib.sage_version() >= 100


def test_workspace_size(lib):
    # variant 0, config-2 shape: int64 partial sums (one per 256 tokens) + int8 K + K scales + k_mean
    # (each piece 256-aligned); the attention kernel quantises Q itself, so there is no int8 Q
    B, H, N, d = 4, 32, 4096, 128
    G, Np = B * H, 4096
    up = lambda x: (x + 255) // 256 * 256
    expect = up(G * 16 * d * 8) + up(G * Np * d) + up(G * 64 * 4) + up(G * d * 4)
    assert sage.workspace_bytes(B, H, N, d, 0) == expect
    # with Q smoothing the attention kernel also takes the block means itself
    assert sage.workspace_bytes(B, H, N, d, 0, smooth_q=True) == expect
    v1 = sage.workspace_bytes(B, H, N, d, 1)
    assert v1 > expect   # V in FP8 + q means
    # V smoothing adds the [G, d] fp32 means; it has no meaning for the fp16 P~V variant
    assert sage.workspace_bytes(B, H, N, d, 1, smooth_v=True) == v1 + up(G * d * 4)
    assert sage.workspace_bytes(B, H, N, d, 0, smooth_v=True) == 0
    # per-token Q scales: formed in the kernel as well
    assert sage.workspace_bytes(B, H, N, d, 0, smooth_q=True, q_group=1) == expect
    assert sage.workspace_bytes(B, H, N, d, 0, q_group=3) == 0
    # MXFP4 variant: K and V statistics, packed E2M1 K (d/2 bytes per row), its E8M0 scales
    # (d/32 per row), k_mean, FP8 V and its scales; the attention kernel quantises Q itself
    ns = N // 256
    v2 = (up(G * ns * d * 8) * 2 + up(G * ns * d * 4) * 2 + up(G * Np * d // 2) + up(G * d * 4)
          + up(G * d * Np) + up(G * d * 4) + up(G * Np * d // 32))
    assert sage.workspace_bytes(B, H, N, d, 2) == v2
    # MXFP4 P~V variant: as variant 2, but V in packed E2M1 (Np/2 bytes per channel) with one
    # E8M0 scale per channel and 32 tokens, and no per-channel FP8 scales
    v3 = (up(G * ns * d * 8) * 2 + up(G * ns * d * 4) * 2 + up(G * Np * d // 2) + up(G * d * 4)
          + up(G * d * Np // 2) + up(G * Np * d // 32) + up(G * (Np // 32) * d))
    assert sage.workspace_bytes(B, H, N, d, 3) == v3
    assert sage.workspace_bytes(B, H, N, d, 3, smooth_v=True) == v3 + up(G * d * 4)
    assert sage.workspace_bytes(B, H, N, d, 3, smooth_q=True) == 0
    assert sage.workspace_bytes(1, 1, 0, 64, 0) == 0
    assert sage.workspace_bytes(1, 1, 64, 80, 0) == 0


def attn(lib, q=A, k=A, v=A, o=A, B=1, H=1, N=64, d=64, causal=0, sm=0.125, variant=0, ws=A, wsb=1 << 30,
         params=None):
    if params is None:
        return lib.sage_attn_fwd(q, k, v, o, B, H, N, d, causal, sm, variant, ws, wsb, None)
    return lib.sage_attn_fwd_ex(q, k, v, o, B, H, N, d, causal, sm, variant, ctypes.byref(params), ws, wsb, None)


@pytest.mark.parametrize("kw,code,msg", [
    (dict(d=96), -2, "head dim"),
    (dict(d=32), -2, "head dim"),
    (dict(N=0), -1, "N must be"),
    (dict(B=0), -1, "B, H, N"),
    (dict(B=1 << 12, H=1 << 8, N=1 << 10, d=128), -1, "2^31"),
    (dict(causal=2), -1, "causal"),
    (dict(variant=4), -1, "variant"),
    (dict(variant=-1), -1, "variant"),
    (dict(sm=0.0), -1, "sm_scale"),
    (dict(sm=float("nan")), -1, "sm_scale"),
    (dict(sm=float("inf")), -1, "sm_scale"),
    (dict(q=None), -1, "q is NULL"),
    (dict(v=MIS), -1, "aligned"),
    (dict(o=None), -1, "o is NULL"),
    (dict(ws=None), -3, "workspace"),
    (dict(wsb=16), -3, "too small"),
    (dict(ws=P(0x10010)), -3, "256-byte"),
])
def test_attn_rejects(lib, kw, code, msg):
    assert attn(lib, **kw) == code
    assert msg in lib.sage_last_error().decode()


def test_params_rejected(lib):
    p = sage._params(blk_q=48)
    assert attn(lib, params=p) == -2 and b"blk_q" in lib.sage_last_error()
    p = sage._params(blk_k=8)
    assert attn(lib, params=p) == -2 and b"blk_k" in lib.sage_last_error()
    p = sage._params()
    p.struct_size = 4
    assert attn(lib, params=p) == -1 and b"struct_size" in lib.sage_last_error()
    p = sage._params()
    p.smooth_k = 3
    assert attn(lib, params=p) == -1
    p = sage._params(smooth_v=True)
    p.smooth_v = 2
    assert attn(lib, params=p, variant=1) == -1 and b"smooth_v" in lib.sage_last_error()
    p = sage._params(smooth_v=True)
    assert attn(lib, params=p, variant=0) == -2 and b"smooth_v" in lib.sage_last_error()


def test_older_params_layouts_are_accepted(lib):
    # the five- and six-int sage_params of libraries 0.1 and 0.2 still parse: the call
    # gets past the parameters and fails on the NULL q instead
    for n in (5, 6):
        p = sage._params(smooth_v=True, q_group=3)  # fields past struct_size are not read
        p.struct_size = n * ctypes.sizeof(ctypes.c_int)
        assert attn(lib, params=p, q=None, variant=1) == -1 and b"q is NULL" in lib.sage_last_error()
    assert lib.sage_version() >= 300


@pytest.mark.parametrize("blk_q,q_group,code", [(128, 0, -1), (128, 1, -1), (64, 16, -1), (32, 32, -1),
                                                (128, 3, -2), (64, 128, -2), (128, -1, -2)])
def test_q_group_validation(lib, blk_q, q_group, code):
    # accepted values fail later, on the NULL q; rejected ones name q_group
    p = sage._params(blk_q=blk_q, q_group=q_group)
    assert attn(lib, params=p, q=None) == code
    assert (b"q_group" in lib.sage_last_error()) == (code == -2)


def test_other_entry_points_reject(lib):
    I = ctypes.c_int
    # quant_qk: q_mean required when smooth_q is on
    p = sage._params(smooth_q=True)
    rc = lib.sage_quant_qk(A, A, 1, 1, 64, 64, ctypes.byref(p), A, A, A, A, A, None, A, 1 << 20, None)
    assert rc == -1 and b"q_mean" in lib.sage_last_error()
    rc = lib.sage_quant_qk(A, A, 1, 1, 64, 64, None, A, A, A, A, A, None, None, 1 << 20, None)
    assert rc == -3
    rc = lib.sage_quant_v(A, 1, 1, 64, 64, A, MIS, A, 1 << 20, None)
    assert rc == -1
    # V smoothing needs somewhere to put the means, and 0 / 1 only
    rc = lib.sage_quant_v_ex(A, 1, 1, 64, 64, 1, A, A, None, A, 1 << 20, None)
    assert rc == -1 and b"v_mean" in lib.sage_last_error()
    rc = lib.sage_quant_v_ex(A, 1, 1, 64, 64, 2, A, A, A, A, 1 << 20, None)
    assert rc == -1 and b"smooth_v" in lib.sage_last_error()
    rc = lib.sage_quant_v_ex(A, 1, 1, 64, 64, 1, A, A, A, A, 16, None)
    assert rc == -3
    rc = lib.sage_attn_fwd_prequant(A, A, A, A, None, None, A, A, None, A, 1, 1, 64, 64, 0, 0.125, 1, None, None)
    assert rc == -1 and b"q_mean" in lib.sage_last_error()       # variant 1 smooths Q by default
    rc = lib.sage_attn_fwd_prequant(A, A, A, A, None, None, A, A, None, A, 1, 1, 64, 64, 0, 0.125, 0, None, None)
    assert rc == -1 and b"v is NULL" in lib.sage_last_error()
    p = sage._params(smooth_q=True, smooth_v=True)
    rc = lib.sage_attn_fwd_prequant(A, A, A, A, A, None, A, A, None, A, 1, 1, 64, 64, 0, 0.125, 1,
                                    ctypes.byref(p), None)
    assert rc == -1 and b"v_mean" in lib.sage_last_error()
    rc = lib.sage_debug_qk_int32(A, A, 1, 1, 64, 64, A, 0, A, None)
    assert rc == -1 and b"n_tiles" in lib.sage_last_error()
    # the fused-Q kernels check their operands before any launch
    rc = lib.sage_attn_fwd_qf16_fp8(A, A, A, None, A, None, A, 1, 1, 64, 64, 0, 0.125, None, None)
    assert rc == -1 and b"v_f8 is NULL" in lib.sage_last_error()
    rc = lib.sage_attn_fwd_qf16_fp8(A, A, A, A, A, None, A, 1, 1, 64, 64, 0, 0.125,
                                    ctypes.byref(sage._params(smooth_v=True)), None)
    assert rc == -1 and b"v_mean" in lib.sage_last_error()
    rc = lib.sage_quant_v_mx(A, 1, 1, 64, 64, 1, A, A, None, A, 1 << 20, None)
    assert rc == -1 and b"v_mean" in lib.sage_last_error()
    rc = lib.sage_quant_v_mx(A, 1, 1, 64, 64, 1, A, A, A, A, 16, None)
    assert rc == -3 and b"too small" in lib.sage_last_error()
    rc = lib.sage_attn_fwd_qf16_fp4(A, A, A, A, None, None, A, 1, 1, 64, 64, 0, 0.125, None, None)
    assert rc == -1 and b"v_e8 is NULL" in lib.sage_last_error()
    rc = lib.sage_attn_fwd_qf16_fp4(A, A, A, A, A, None, A, 1, 1, 64, 64, 0, 0.125,
                                    ctypes.byref(sage._params(smooth_q=True)), None)
    assert rc == -2 and b"smooth_q" in lib.sage_last_error()
    rc = lib.sage_attn_fwd_qf16(A, None, A, A, A, 1, 1, 64, 64, 0, 0.125, None, None)
    assert rc == -1 and b"k_i8 is NULL" in lib.sage_last_error()
    rc = lib.sage_attn_fwd_qf16(A, A, A, A, A, 1, 1, 64, 96, 0, 0.125, None, None)
    assert rc == -2


def test_mxfp4_entry_points_reject(lib):
    # Q smoothing is not part of the MXFP4 variant
    p = sage._params(smooth_q=True)
    assert attn(lib, params=p, variant=2) == -2 and b"smooth_q" in lib.sage_last_error()
    rc = lib.sage_attn_fwd_prequant_mx(A, A, A, A, A, A, None, A, 1, 1, 64, 64, 0, 0.125, ctypes.byref(p), None)
    assert rc == -2
    rc = lib.sage_attn_fwd_prequant_mx(A, A, A, None, A, A, None, A, 1, 1, 64, 64, 0, 0.125, None, None)
    assert rc == -1 and b"k_e8 is NULL" in lib.sage_last_error()
    p = sage._params(smooth_v=True)
    rc = lib.sage_attn_fwd_prequant_mx(A, A, A, A, A, A, None, A, 1, 1, 64, 64, 0, 0.125, ctypes.byref(p), None)
    assert rc == -1 and b"v_mean" in lib.sage_last_error()
    rc = lib.sage_quant_qk_mx(A, A, 1, 1, 64, 64, 2, A, A, A, A, None, A, 1 << 20, None)
    assert rc == -1 and b"smooth_k" in lib.sage_last_error()
    rc = lib.sage_quant_qk_mx(A, A, 1, 1, 64, 96, 1, A, A, A, A, None, A, 1 << 20, None)
    assert rc == -2
    rc = lib.sage_quant_qk_mx(A, A, 1, 1, 64, 64, 1, A, A, A, A, None, None, 0, None)
    assert rc == -3
    # the pre-quantised int8 entry point points MXFP4 callers to their own
    rc = lib.sage_attn_fwd_prequant(A, A, A, A, None, None, A, A, None, A, 1, 1, 64, 64, 0, 0.125, 2, None, None)
    assert rc == -1 and b"prequant_mx" in lib.sage_last_error()
    rc = lib.sage_attn_fwd_qf16_mx(A, A, None, A, A, None, A, 1, 1, 64, 64, 0, 0.125, None, None)
    assert rc == -1 and b"k_e8 is NULL" in lib.sage_last_error()
    rc = lib.sage_attn_fwd_qf16_mx(A, A, A, A, A, None, A, 1, 1, 64, 64, 0, 0.125,
                                   ctypes.byref(sage._params(smooth_q=True)), None)
    assert rc == -2


def test_binding_fails_loudly_without_gpu_tensors():
    torch = pytest.importorskip("torch")
    x = torch.zeros((1, 1, 8, 64), dtype=torch.float16)
    with pytest.raises(ValueError, match="GPU"):
        sage.attn(x, x, x)
    with pytest.raises(TypeError):
        sage.attn(x.float(), x, x)


def test_bench_refuses_several_gpus():
    # one GPU only: the multi-GPU request ends before anything touches a device
    import subprocess
    import sys
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=300)
    assert res.returncode == 2
    assert "one GPU" in res.stdout + res.stderr
    assert not res.stdout.lstrip().startswith("{")
