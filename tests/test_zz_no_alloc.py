"""sage_attn_fwd_noalloc: the whole forward with the library's own per-GPU workspace array.

For callers that cannot allocate device memory.  Through the C ABI it must give the
bits of sage_attn_fwd_ex with a caller workspace (same kernels), on two calls in a
row with the second smaller (the array keeps the first call's contents), and reject
shapes whose workspace exceeds the array before launching anything.
"""
import ctypes
import sys

import numpy as np
import pytest

import quantized_bit_attention_amd as sage
import workloads

torch = pytest.importorskip("torch")

P = ctypes.c_void_p
A = P(0x10000)  # aligned, never dereferenced: the calls below are rejected first


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def test_noalloc_rejects_oversized_shapes_before_any_launch():
    lib = sage._load()
    # workload 5 (64 heads of N = 32768, d = 128, variant 1) needs about 0.8 GB of workspace
    assert sage.workspace_bytes(2, 32, 32768, 128, 1) > sage.NOALLOC_SCRATCH_BYTES
    rc = lib.sage_attn_fwd_noalloc(A, A, A, A, 2, 32, 32768, 128, 1, 0.088, 1, None, None)
    assert rc == -3
    msg = lib.sage_last_error().decode()
    assert "workspace" in msg and str(sage.NOALLOC_SCRATCH_BYTES) in msg
    # the LLM-prefill shape fits
    assert sage.workspace_bytes(4, 32, 4096, 128, 0) <= sage.NOALLOC_SCRATCH_BYTES
    # argument errors still come before any HIP call
    assert lib.sage_attn_fwd_noalloc(None, A, A, A, 1, 1, 64, 64, 0, 0.125, 0, None, None) == -1
    assert lib.sage_attn_fwd_noalloc(A, A, A, A, 1, 1, 64, 96, 0, 0.125, 0, None, None) == -2


CASES = [
    # (variant, options, first (larger) shape, second (smaller) shape)
    (0, dict(causal=True), (2, 8, 2048, 128), (1, 3, 333, 128)),
    (0, dict(causal=False, blk_q=64, blk_k=32), (1, 4, 1500, 64), (1, 2, 129, 64)),
    (1, dict(causal=True, smooth_v=True), (1, 6, 2048, 128), (1, 2, 200, 128)),
    (2, dict(causal=False), (2, 3, 1024, 64), (1, 1, 65, 64)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("variant,opts,big,small", CASES)
def test_noalloc_matches_workspace_call(variant, opts, big, small):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    for shape in (big, small):
        B, H, N, d = shape
        cfg = 5 if d == 128 else 1
        x = workloads.make_inputs(cfg, B=B, H=H, N=N)
        assert x["q"].shape[-1] == d
        q, k, v = (torch.from_numpy(x[n]).cuda() for n in ("q", "k", "v"))
        say(f"noalloc variant {variant} {shape} {opts}")
        ref = sage.attn(q, k, v, variant=variant, **opts)
        out = torch.empty_like(q)
        got = sage.attn_noalloc(q, k, v, out, variant=variant, **opts)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.isfinite(got.float()).all()
        assert torch.equal(got, ref)


@pytest.mark.gpu
def test_noalloc_rejects_oversized_shape_on_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # 64 heads of N = 32768 need more than the array: rejected, nothing launched, out untouched
    x = torch.zeros((1, 64, 32768, 128), dtype=torch.float16, device="cuda")
    out = torch.full_like(x, 7.0)
    with pytest.raises(sage.SageError, match="workspace"):
        sage.attn_noalloc(x, x, x, out, variant=1, causal=True)
    torch.cuda.synchronize()
    assert bool((out == 7.0).all())
