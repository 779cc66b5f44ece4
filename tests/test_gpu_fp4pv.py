"""GPU parity of the MXFP4 P~V variant (variant 3: SageAttention3 abstract, FP4 attention):
MXFP4 V bit-exact against the oracle, O against the oracle's fp64 O within the bar of the
other variants (max-abs 2e-3, cosine >= 0.9999), the fused kernel equal to the whole call,
and determinism at full size.
"""
import numpy as np
import pytest

import workloads
from tests.test_gpu_parity import check_o, dev, host, inputs, oracle_kw, say

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def sage():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import quantized_bit_attention_amd as s
    s._load()
    return s


def unpack_v(g, d):
    """The library's V layout -> the oracle's: codes [.., d, Np/2] two per byte (low nibble
    first) -> [.., d, Np]; scales [.., Np/32, d] with channel c at (c % 32) * (d/32) + c / 32
    -> [.., d, Np/32]."""
    f4 = g["v_f4"]
    codes = np.stack([f4 & 15, f4 >> 4], axis=-1).reshape(*f4.shape[:-1], 2 * f4.shape[-1])
    e8 = g["v_e8"]
    c = np.arange(d)
    e8 = e8[..., (c % 32) * (d // 32) + c // 32]          # [.., Np/32, d] in channel order
    return codes, np.swapaxes(e8, -1, -2)


V_CASES = [
    # recipe cfg, shape overrides, smooth_v, special
    (5, dict(N=1000, B=1, H=2), 0, None),
    (5, dict(N=1000, B=1, H=2), 1, None),
    (1, dict(N=77, B=2, H=1), 0, None),
    (3, dict(N=300, B=1, H=3), 1, None),
    (1, dict(N=200, B=1, H=1), 0, "ties"),
    (2, dict(N=129, B=1, H=1), 1, "const_channels"),
]


@pytest.mark.parametrize("cfg,shape,smooth_v,special", V_CASES)
def test_quant_v_mx_bitexact(sage, orc, cfg, shape, smooth_v, special):
    c = workloads.make_inputs(cfg, **shape)
    v = c["v"].copy()
    if special == "ties":
        # E2M1 midpoints and saturation at the block scale 2^0 (block max 4): 0.25, 0.75, ..
        mids = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 4.0], np.float16)
        v[0, 0, :, :] = np.resize(mids, v.shape[2])[:, None]
    if special == "const_channels":
        v[0, 0, :, :5] = np.float16(1.5)
    say(f"quant_v_mx {v.shape} smooth_v={smooth_v} {special or ''}")
    g = {k: host(t) for k, t in sage.quant_v_mx(dev(v), smooth_v=bool(smooth_v)).items()}
    r = orc.quant_v_mx(v, smooth_v=smooth_v)
    d = v.shape[-1]
    codes, e8 = unpack_v(g, d)
    assert np.array_equal(codes, r["v_codes"])
    assert np.array_equal(e8, r["v_e8"])
    if smooth_v:
        assert np.array_equal(g["v_mean"].view(np.uint32), r["v_mean"].view(np.uint32))


EDGE4 = [
    ("n1_causal", 5, dict(N=1, B=1, H=1), dict(causal=1)),
    ("n17_d64", 1, dict(N=17, B=1, H=2), dict(causal=0)),
    ("n64_d64", 3, dict(N=64, B=1, H=2), dict(causal=1)),
    ("n129_causal_d128", 2, dict(N=129, B=2, H=1), dict(causal=1)),
    ("n333_causal_d128", 5, dict(N=333, B=1, H=2), dict(causal=1)),
    ("n200_d64", 3, dict(N=200, B=1, H=2), dict(causal=0)),
    ("n520_d128", 2, dict(N=520, B=1, H=2), dict(causal=0)),
    ("nosmoothk", 1, dict(N=256, B=1, H=2), dict(causal=1, smooth_k=0)),
    ("smoothv_d128", 5, dict(N=300, B=1, H=2), dict(causal=0, smooth_v=1)),
    ("smoothv_causal_d64", 4, dict(N=333, B=1, H=2), dict(causal=1, smooth_v=1)),
]


def run_fp4(sage, c):
    return host(sage.attn(dev(c["q"]), dev(c["k"]), dev(c["v"]), causal=bool(c["causal"]), variant=3,
                          smooth_k=bool(c.get("smooth_k", 1)), smooth_q=False, smooth_v=bool(c.get("smooth_v", 0))))


@pytest.mark.parametrize("name,cfg,shape,opt", EDGE4, ids=[e[0] for e in EDGE4])
def test_attn_fp4pv_edge_cases_all_rows(sage, orc, name, cfg, shape, opt):
    c = dict(workloads.config(cfg))
    c.update(workloads.make_inputs(cfg, **shape))
    c.update(opt, variant=3, smooth_q=0)
    say(f"attn fp4pv edge {name} {c['q'].shape} {opt}")
    g = run_fp4(sage, c)
    o = orc.attn(c["q"], c["k"], c["v"], **oracle_kw(c))
    check_o(f"fp4pv {name}", g, o)


def test_attn_fp4pv_tiny_weights(sage, orc):
    """Keys whose weights fall below 2^-124 of the row maximum: their 32-key blocks take E8M0
    code 0 (scale 2^-127), which the kernel converts by an exact 2^127 scaling.  Scores
    from K rows 32 e1 (key 0 of every block of 32) and 16 e1 (the rest), Q rows 32 e1, and
    sm_scale chosen so the rest sit 126.5 below the maximum in base 2."""
    N, d = 256, 64
    q = np.zeros((1, 1, N, d), np.float16)
    k = np.zeros((1, 1, N, d), np.float16)
    q[..., 0] = 32.0
    k[..., 0] = 16.0
    k[0, 0, ::64, 0] = 32.0                 # one strong key per 64-key tile
    v = workloads.make_inputs(1, N=N, B=1, H=1)["v"]
    sm = 126.5 / 512.0 / 1.4426950408889634
    say("attn fp4pv tiny weights")
    g = host(sage.attn(dev(q), dev(k), dev(v), variant=3, smooth_k=False, smooth_q=False, sm_scale=sm))
    o = orc.attn(q, k, v, variant=3, smooth_k=0, sm_scale=sm)
    check_o("fp4pv tiny weights", g, o)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_attn_full_size_fp4pv_sampled_rows(sage, orc, cfg):
    """Variant 3 on each workload's full shape, every row of two heads (the first and the last)."""
    c = dict(inputs(cfg))
    c.update(variant=3, smooth_q=0)
    B, H, N, d = c["q"].shape
    say(f"attn fp4pv cfg{cfg} full size {c['q'].shape} causal={c['causal']}")
    g = run_fp4(sage, c)
    rng = np.random.default_rng(cfg)
    rows = np.sort(rng.choice(N, 256 if N <= 8192 else 64, replace=False))
    for gh in (0, B * H - 1):
        b, h = divmod(gh, H)
        o = orc.attn_rows(c["q"], c["k"], c["v"], np.full(rows.size, gh), rows, **oracle_kw(c))
        check_o(f"fp4pv cfg{cfg} head {gh} {rows.size} rows", g[b, h, rows], o)


@pytest.mark.parametrize("cfg,shape,causal,smooth_v", [(2, dict(N=333, B=1, H=2), 1, 0),
                                                        (3, dict(N=200, B=1, H=3), 0, 1),
                                                        (5, dict(N=1000, B=1, H=2), 1, 1)])
def test_fused_fp4pv_matches_whole_call(sage, cfg, shape, causal, smooth_v):
    """The whole call and the attention kernel alone on quant_qk_mx / quant_v_mx outputs give
    the same bits."""
    c = workloads.make_inputs(cfg, **shape)
    qd, kd, vd = dev(c["q"]), dev(c["k"]), dev(c["v"])
    say(f"fp4pv fused vs whole {c['q'].shape} causal={causal} smooth_v={smooth_v}")
    whole = sage.attn(qd, kd, vd, causal=bool(causal), variant=3, smooth_q=False, smooth_v=bool(smooth_v))
    qk = sage.quant_qk_mx(qd, kd)
    vq = sage.quant_v_mx(vd, smooth_v=bool(smooth_v))
    fused = sage.attn_qf16_fp4(qd, qk, vq, causal=bool(causal), smooth_v=bool(smooth_v))
    torch.cuda.synchronize()
    assert torch.isfinite(whole.float()).all()
    assert torch.equal(whole, fused)


def test_full_size_fp4pv_deterministic(sage):
    c = dict(inputs(2))
    say(f"determinism fp4pv cfg2 {c['q'].shape}")
    q, k, v = dev(c["q"]), dev(c["k"]), dev(c["v"])
    a = sage.attn(q, k, v, causal=True, variant=3, smooth_q=False)
    b = sage.attn(q, k, v, causal=True, variant=3, smooth_q=False)
    torch.cuda.synchronize()
    assert torch.isfinite(a.float()).all()
    assert torch.equal(a, b)


@pytest.mark.parametrize("shape", [(1, 1, 0, 64), (0, 2, 16, 128)])
def test_attn_fp4pv_empty_inputs(sage, shape):
    q = torch.zeros(shape, dtype=torch.float16, device="cuda")
    o = sage.attn(q, q, q, variant=3, smooth_q=False)
    assert o.shape == q.shape


def test_fp4pv_rejects_q_smoothing_and_bad_operands(sage):
    q = torch.zeros((1, 1, 100, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(sage.SageError, match="smooth_q"):
        sage.attn(q, q, q, variant=3, smooth_q=True)
    qk = sage.quant_qk_mx(q, q)
    vq = sage.quant_v_mx(q)
    with pytest.raises(ValueError, match="v_e8"):
        sage.attn_qf16_fp4(q, qk, dict(vq, v_e8=vq["v_e8"][:, :, :2]))
    with pytest.raises(ValueError, match="v_mean"):
        sage.attn_qf16_fp4(q, qk, dict(vq, v_mean=vq["v_mean"][..., :8]), smooth_v=True)
