"""GPU parity of the 8-bit attention backward (dQ, dK, dV) against the CPU oracle.

The backward follows the SageAttention3 abstract (author page, "NeurIPS Conference
2025" heading: 8-bit attention for forward and backward propagation); readings in
oracle.c.  Every case feeds the same fp16 q, k, v, dout and the same o (the oracle's
forward output rounded to fp16) to both sides; the GPU also takes the row
log-sum-exp from its own training forward (attn_fwd_train).

Bar, per gradient tensor: max |gpu - oracle| <= 2e-3 * max |oracle| and cosine >=
0.9999.  The two sides share every INT8 code (same rules, same fp32 decisions); they
differ by fp32 against fp64 arithmetic in the sums and in P = 2^(s - L), and by the
fp16 rounding of 2^8 P and sigma dS where those fp32 and fp64 values straddle a
rounding midpoint (one fp16 step, 2^-11 of one term of a sum).
"""
import sys

import numpy as np
import pytest

import workloads
from tests.ref64 import cos_sim

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

REL_MAX = 2e-3
TOL_COS = 0.9999


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_bit_attention_amd as s
    s._load()
    return s


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def run_case(sage, orc, cfg, shape, causal, blk_q, blk_k, seed=0):
    x = workloads.make_inputs(cfg, **shape)
    q, k, v = x["q"], x["k"], x["v"]
    rng = np.random.default_rng(100 + seed)
    dout = rng.standard_normal(q.shape).astype(np.float16)
    o16 = orc.attn(q, k, v, causal=causal, variant=0, blk_q=blk_q, blk_k=blk_k, bkv=64).astype(np.float16)
    qd, kd, vd = dev(q), dev(k), dev(v)
    _, lse = sage.attn_fwd_train(qd, kd, vd, causal=bool(causal), blk_q=blk_q, blk_k=blk_k)
    g = sage.attn_bwd(qd, kd, vd, dev(o16), dev(dout), lse, causal=bool(causal), blk_q=blk_q, blk_k=blk_k)
    torch.cuda.synchronize()
    g = {n: t.cpu().numpy().astype(np.float64) for n, t in g.items()}
    r = orc.attn_bwd(q, k, v, o16, dout, causal=causal, blk_q=blk_q, blk_k=blk_k, smooth_k=1, smooth_v=1)
    return g, r


def check(name, g, r):
    for n in ("dq", "dk", "dv"):
        assert np.isfinite(g[n]).all(), (name, n)
        if not r[n].any():  # one token: the scores carry no gradient (dQ = dK = 0 exactly)
            say(f"  [{name}] {n}: oracle 0, max|gpu| = {np.abs(g[n]).max():.3e}")
            assert np.abs(g[n]).max() <= 1e-6, (name, n)
            continue
        rel = float(np.abs(g[n] - r[n]).max() / np.abs(r[n]).max())
        c = cos_sim(g[n], r[n])
        say(f"  [{name}] {n}: max|diff|/max|ref| = {rel:.3e}  cos = {c:.9f}")
        assert rel <= REL_MAX, (name, n)
        assert c >= TOL_COS, (name, n)


CASES = [
    # name, recipe cfg, shape, causal, blk_q, blk_k
    ("cfg1_noncausal", 1, dict(), 0, 64, 64),
    ("n333_causal_d128", 2, dict(N=333, B=1, H=2), 1, 128, 64),
    ("n200_d64_blk16", 3, dict(N=200, B=1, H=3), 0, 64, 16),
    ("n65_causal_d64", 1, dict(N=65, B=1, H=2), 1, 64, 32),
    ("n1000_causal_d128", 5, dict(N=1000, B=1, H=2), 1, 128, 64),
    ("n1_d128", 2, dict(N=1, B=1, H=2), 0, 128, 64),
    ("n777_d64_blk128", 4, dict(N=777, B=2, H=1), 0, 128, 128),
    # causal blocks go longest first across pairs of heads; the third head goes alone
    ("odd_heads_causal_d128", 2, dict(N=1000, B=1, H=3), 1, 128, 64),
]


@pytest.mark.parametrize("name,cfg,shape,causal,blk_q,blk_k", CASES, ids=[c[0] for c in CASES])
def test_bwd_matches_oracle(sage, orc, name, cfg, shape, causal, blk_q, blk_k):
    say(f"bwd {name} cfg{cfg} {shape} causal={causal} blk {blk_q}/{blk_k}")
    g, r = run_case(sage, orc, cfg, shape, causal, blk_q, blk_k)
    check(name, g, r)


FULL = [
    # recipe cfg (its full shape), heads compared (every element), causal
    (2, [0, 17, 34, 51, 68, 85, 102, 127], 1),   # LLM prefill: B=4 H=32 N=4096 d=128
    (3, [0, 23, 47], 0),                          # image generation: B=2 H=24 N=8192 d=64
]


@pytest.mark.slow
@pytest.mark.parametrize("cfg,heads,causal", FULL, ids=[f"cfg{c[0]}" for c in FULL])
def test_bwd_full_size(sage, orc, cfg, heads, causal):
    """A workload's full shape: the GPU backward over all heads; every element of the listed
    heads (including the first and the last) against the oracle."""
    x = workloads.make_inputs(cfg)
    B, H, N, d = x["q"].shape
    assert heads[-1] == B * H - 1
    rng = np.random.default_rng(12)
    dout = rng.standard_normal(x["q"].shape).astype(np.float16)
    say(f"bwd full size cfg{cfg} {x['q'].shape} causal={causal}: oracle forward of heads {heads}")
    sel = lambda a: np.ascontiguousarray(a.reshape(B * H, N, d)[heads].reshape(1, len(heads), N, d))
    qs, ks, vs, gs = sel(x["q"]), sel(x["k"]), sel(x["v"]), sel(dout)
    o16 = orc.attn(qs, ks, vs, causal=causal, variant=0, blk_q=128, blk_k=64, bkv=64).astype(np.float16)
    # the GPU runs every head; o of the other heads comes from the GPU forward (their
    # gradients are not compared)
    qd, kd, vd = dev(x["q"]), dev(x["k"]), dev(x["v"])
    o, lse = sage.attn_fwd_train(qd, kd, vd, causal=bool(causal))
    o.view(B * H, N, d)[heads] = dev(o16.reshape(len(heads), N, d))
    g = sage.attn_bwd(qd, kd, vd, o, dev(dout), lse, causal=bool(causal))
    torch.cuda.synchronize()
    g = {n: t.view(B * H, N, d)[heads].cpu().numpy().astype(np.float64).reshape(1, len(heads), N, d)
         for n, t in g.items()}
    say(f"  oracle backward of heads {heads}")
    r = orc.attn_bwd(qs, ks, vs, o16, gs, causal=causal, blk_q=128, blk_k=64, smooth_k=1, smooth_v=1)
    check(f"cfg{cfg} full size", g, r)


def test_bwd_is_deterministic(sage):
    x = workloads.make_inputs(2, N=700, B=1, H=2)
    rng = np.random.default_rng(3)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    dout = dev(rng.standard_normal(x["q"].shape).astype(np.float16))
    o, lse = sage.attn_fwd_train(q, k, v, causal=True)
    a = sage.attn_bwd(q, k, v, o, dout, lse, causal=True)
    b = sage.attn_bwd(q, k, v, o, dout, lse, causal=True)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv"):
        assert torch.equal(a[n], b[n]), n


def test_train_forward_output_and_lse(sage, orc):
    """attn_fwd_train's output is attn's up to the divisor (the sum of the unrounded weights
    instead of the fp16 ones: each fp16 weight is within 2^-11 of its value relative, so the
    divisors differ by at most 2^-11 relative; the fp16 outputs then differ by that plus at most
    one fp16 step, 2^-10 relative),
    and its lse is the log-sum-exp of the oracle's scores."""
    x = workloads.make_inputs(2, N=300, B=1, H=2)
    q, k, v = dev(x["q"]), dev(x["k"]), dev(x["v"])
    o, lse = sage.attn_fwd_train(q, k, v, causal=True)
    o2 = sage.attn(q, k, v, causal=True)
    torch.cuda.synchronize()
    a, b = o.float(), o2.float()
    assert float((a - b).abs().max()) <= 3 * 2.0 ** -11 * float(b.abs().max())
    # lse against the oracle: the textbook log-sum-exp of the dequantised INT8 scores
    r = orc.quant(x["q"], x["k"], blk_q=128, blk_k=64, smooth_k=1)
    qi = r["q_i8"][0, :, :300].astype(np.int64)
    ki = r["k_i8"][0, :, :300].astype(np.int64)
    qs = np.repeat(r["q_scale"][0], 128, axis=1)[:, :300].astype(np.float64)
    ks = np.repeat(r["k_scale"][0], 64, axis=1)[:, :300].astype(np.float64)
    s = np.einsum("hic,hjc->hij", qi, ki) * qs[:, :, None] * ks[:, None, :] / np.sqrt(128)
    s = np.where(np.tril(np.ones((300, 300), bool)), s, -np.inf)
    m = s.max(-1, keepdims=True)
    ref = (m + np.log(np.exp(s - m).sum(-1, keepdims=True)))[..., 0]
    got = lse.cpu().numpy()[0].astype(np.float64)
    assert np.max(np.abs(got - ref)) < 1e-4


def test_bwd_rejects_unsupported_options(sage):
    x = torch.zeros((1, 1, 64, 64), dtype=torch.float16, device="cuda")
    lse = torch.zeros((1, 1, 64), dtype=torch.float32, device="cuda")
    with pytest.raises(sage.SageError, match="blk_q"):
        sage.attn_bwd(x, x, x, x, x, lse, blk_q=32)
    with pytest.raises(ValueError, match="lse"):
        sage.attn_bwd(x, x, x, x, x, lse[..., :32])
