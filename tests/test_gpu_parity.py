"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar (stated for this path): int8 Q/K codes, their scales and means, FP8 V codes and
scales, and int32 Q K^T tiles bit-exact; O within max-abs 2e-3 and cosine >= 0.9999
of the oracle's fp64 O.  Shapes: the five workloads at full size (O on every row of
chosen heads; options of the method on sampled rows), plus small and ragged cases
compared on every row.
"""
import functools
import math
import sys

import numpy as np
import pytest

import workloads
from tests.ref64 import cos_sim

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

TOL_MAX_ABS = 2e-3
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


@functools.lru_cache(maxsize=2)
def inputs(cfg, **kw):
    return workloads.make_inputs(cfg, **kw)


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


def cfg_kw(c):
    return dict(causal=c["causal"], variant=c["variant"], blk_q=c["blk_q"], blk_k=c["blk_k"],
                smooth_v=bool(c.get("smooth_v", 0)), q_group=c.get("q_group", 0))


def oracle_kw(c):
    """Oracle options for the GPU call's options.  The online-softmax tile comes from the
    library (sage_kv_tile): FP8 codes of P~ depend on the running max at each tile."""
    import quantized_bit_attention_amd as s
    bkv = s.kv_tile(c["variant"], c["q"].shape[-1])
    assert bkv > 0
    return dict(causal=c["causal"], variant=c["variant"], blk_q=c["blk_q"], blk_k=c["blk_k"], bkv=bkv,
                smooth_k=c.get("smooth_k", 1), smooth_q=c.get("smooth_q", 1 if c["variant"] == 1 else 0),
                smooth_v=c.get("smooth_v", 0), q_group=c.get("q_group", 0) or None)


def check_o(name, g16, o64):
    g = g16.astype(np.float64)
    err = np.abs(g - o64)
    mx = float(err.max())
    c = cos_sim(g, o64)
    say(f"  [{name}] O max_abs={mx:.3e} cos={c:.9f} n={o64.size}")
    assert np.isfinite(g).all()
    assert mx <= TOL_MAX_ABS, name
    assert c >= TOL_COS, name


def sample_rows(N, causal, rng, n_rand=24):
    rows = {0, 1, min(2, N - 1), N - 1, max(0, N - 2)}
    for r in (31, 32, 63, 64, 65, 127, 128, 129, 255, 256):
        if r < N:
            rows.add(r)
    last_tile = (N - 1) // 128 * 128
    rows.update(range(last_tile, min(N, last_tile + 4)))
    rows.update(int(r) for r in rng.integers(0, N, n_rand))
    return sorted(rows)


# --------------------------------------------------------------------------
# quantisation: bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_quant_qk_bitexact(sage, orc, cfg):
    c = inputs(cfg)
    sq = 1 if c["variant"] == 1 else 0
    say(f"quant_qk cfg{cfg} {c['q'].shape}")
    g = sage.quant_qk(dev(c["q"]), dev(c["k"]), blk_q=c["blk_q"], blk_k=c["blk_k"], smooth_k=True, smooth_q=bool(sq))
    g = {k: host(v) for k, v in g.items()}
    r = orc.quant(c["q"], c["k"], blk_q=c["blk_q"], blk_k=c["blk_k"], smooth_k=1, smooth_q=sq)
    for key in ("q_i8", "k_i8", "q_scale", "k_scale", "k_mean") + (("q_mean",) if sq else ()):
        same = np.array_equal(g[key].view(np.uint8) if g[key].dtype == np.int8 else g[key].view(np.uint32),
                              r[key].view(np.uint8) if r[key].dtype == np.int8 else r[key].view(np.uint32))
        if not same:
            diff = np.nonzero(g[key] != r[key])
            say(f"  {key}: {len(diff[0])} mismatches, first at {[d[0] for d in diff]}")
        assert same, key


QGROUP_QUANT = [
    # recipe cfg, shape overrides, blk_q, blk_k, q_group, smooth_q
    (1, dict(N=333, B=1, H=2), 64, 64, 1, 0),
    (2, dict(N=1000, B=1, H=2), 128, 64, 16, 1),
    (3, dict(N=200, B=1, H=3), 32, 16, 4, 0),
    (5, dict(N=4096, B=1, H=2), 128, 64, 1, 1),
    (2, dict(N=129, B=2, H=1), 64, 32, 2, 1),
]


@pytest.mark.parametrize("cfg,shape,blk_q,blk_k,q_group,sq", QGROUP_QUANT)
def test_quant_qk_q_group_bitexact(sage, orc, cfg, shape, blk_q, blk_k, q_group, sq):
    """Q scales per group of q_group rows inside the smoothing block: codes, scales and
    means bit-exact.  One row is all zeros, so with per-token scales its scale is 0."""
    c = workloads.make_inputs(cfg, **shape)
    q = c["q"].copy()
    q[0, 0, 5] = 0
    say(f"quant_qk q_group={q_group} {q.shape} blk_q={blk_q} smooth_q={sq}")
    g = sage.quant_qk(dev(q), dev(c["k"]), blk_q=blk_q, blk_k=blk_k, smooth_q=bool(sq), q_group=q_group)
    g = {k: host(v) for k, v in g.items()}
    r = orc.quant(q, c["k"], blk_q=blk_q, blk_k=blk_k, smooth_k=1, smooth_q=sq, q_group=q_group)
    assert g["q_scale"].shape == r["q_scale"].shape
    for key in ("q_i8", "k_i8", "q_scale", "k_scale", "k_mean") + (("q_mean",) if sq else ()):
        view = np.uint8 if g[key].dtype == np.int8 else np.uint32
        same = np.array_equal(g[key].view(view), r[key].view(view))
        if not same:
            diff = np.nonzero(g[key] != r[key])
            say(f"  {key}: {len(diff[0])} mismatches, first at {[d[0] for d in diff]}")
        assert same, key


def pack_e2m1(codes):
    """Two codes per byte, the lower channel in the low nibble (the GPU layout)."""
    c = codes.astype(np.uint8)
    return c[..., 0::2] | (c[..., 1::2] << 4)


MX_QUANT = [
    # recipe cfg, shape overrides, smooth_k
    (5, dict(N=1000, B=1, H=2), 1),
    (1, dict(N=333, B=1, H=3), 1),
    (3, dict(N=200, B=1, H=2), 1),     # outlier K channels
    (2, dict(N=129, B=2, H=1), 0),
]


@pytest.mark.parametrize("cfg,shape,smooth_k", MX_QUANT)
def test_quant_mx_bitexact(sage, orc, cfg, shape, smooth_k):
    """Per-token MXFP4 of Q and K': E2M1 codes, E8M0 scales and k_mean bit-exact.  Q carries
    an all-zero block, a power-of-two maximum and values that saturate at 6."""
    c = workloads.make_inputs(cfg, **shape)
    q = c["q"].copy()
    q[0, 0, 3, :32] = 0
    q[0, 0, 4, 7] = 8.0
    q[0, 0, 5, 0] = -7.99
    q[0, 0, 6, :] = -0.0
    say(f"quant_mx {q.shape} smooth_k={smooth_k}")
    g = sage.quant_qk_mx(dev(q), dev(c["k"]), smooth_k=bool(smooth_k))
    g = {k: host(v) for k, v in g.items()}
    r = orc.quant_mx(q, c["k"], smooth_k=smooth_k)
    for name in ("q", "k"):
        want_f4 = pack_e2m1(r[f"{name}_codes"])
        for key, want in ((f"{name}_f4", want_f4), (f"{name}_e8", r[f"{name}_e8"])):
            same = np.array_equal(g[key], want)
            if not same:
                bad = np.nonzero(g[key] != want)
                say(f"  {key}: {len(bad[0])} mismatches, first at {[b[0] for b in bad]}")
            assert same, key
    assert np.array_equal(g["k_mean"].view(np.uint32), r["k_mean"].view(np.uint32))


@pytest.mark.parametrize("smooth_v", [0, 1])
@pytest.mark.parametrize("case", ["cfg5", "ragged_d64", "ties", "offset", "const_channels"])
def test_quant_v_bitexact(sage, orc, case, smooth_v):
    if case == "cfg5":
        v = inputs(5)["v"]
    elif case == "ragged_d64":
        v = workloads.make_inputs(1, N=333, B=1, H=3)["v"]
    elif case == "offset":
        v = workloads.make_inputs(5, N=777, B=1, H=2, v_sigma=1.0)["v"]
    elif case == "const_channels":
        # constant channels: zero, positive, negative; with V smoothing all become 0
        # (scale 0, codes 0) and the mean carries the whole channel
        v = workloads.make_inputs(1, N=300, B=1, H=2)["v"].copy()
        v[0, 0, :, 0] = 0
        v[0, 0, :, 1] = 1.5
        v[0, 1, :, 5] = -0.2
        v[0, 1, :, 63] = 65504
    else:
        # every channel's absmax is 448, so the scale is 1 and the codes are E4M3(V):
        # the values are all E4M3 ties, their fp16 neighbours and the codes themselves
        codes = orc.e4m3_decode(np.arange(256, dtype=np.uint8))
        pos = np.unique(codes[np.isfinite(codes) & (codes >= 0)])
        mids = 0.5 * (pos[1:] + pos[:-1])
        vals = np.concatenate([pos, mids, -mids])
        vals16 = vals.astype(np.float16)
        up = np.nextafter(vals16, np.float16(np.inf))
        dn = np.nextafter(vals16, np.float16(-np.inf))
        allv = np.concatenate([vals16, up, dn, -vals16])
        allv = allv[np.abs(allv.astype(np.float64)) <= 448]
        n = -(-allv.size // 64) * 64
        col = np.zeros(n, np.float16)
        col[:allv.size] = allv
        col[0] = 448
        v = np.tile(col[:, None], (1, 64))[None, None].copy()
        v[0, 0, :, 1::2] *= np.float16(-1)
        v = v.astype(np.float16)
    say(f"quant_v {case} {v.shape} smooth_v={smooth_v}")
    g = sage.quant_v(dev(v), smooth_v=bool(smooth_v))
    r = orc.quant(v, v, v, with_v=True, smooth_v=smooth_v)
    assert np.array_equal(host(g["v_scale"]).view(np.uint32), r["v_scale"].view(np.uint32))
    assert np.array_equal(host(g["v_mean"]).view(np.uint32), r["v_mean"].view(np.uint32))
    gv = host(g["v_f8"])
    if not np.array_equal(gv, r["v_f8"]):
        bad = np.nonzero(gv != r["v_f8"])
        say(f"  v_f8 mismatches: {len(bad[0])} first {[b[0] for b in bad]}")
    assert np.array_equal(gv, r["v_f8"])


# --------------------------------------------------------------------------
# int32 Q K^T tiles: bit-exact
# --------------------------------------------------------------------------

@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_qk_int32_tiles(sage, orc, cfg):
    c = inputs(cfg)
    B, H, N, d = c["q"].shape
    r = orc.quant(c["q"], c["k"], blk_q=c["blk_q"], blk_k=c["blk_k"], smooth_k=1,
                  smooth_q=1 if c["variant"] == 1 else 0)
    Np = r["q_i8"].shape[2]
    nqt, nkt = Np // 128, Np // 64
    if cfg == 1:
        tiles = [(g, qt, kt) for g in range(B * H) for qt in range(nqt) for kt in range(nkt)]
    else:
        tiles = []
        for g in (0, B * H - 1):
            tiles += [(g, 0, 0), (g, nqt - 1, nkt - 1), (g, nqt - 1, 0), (g, 0, nkt - 1),
                      (g, nqt // 2, nkt // 2), (g, nqt // 2, nkt // 2 + 1)]
    say(f"qk_int32 cfg{cfg} {len(tiles)} tiles")
    qi, ki = r["q_i8"].reshape(B * H, Np, d), r["k_i8"].reshape(B * H, Np, d)
    got = host(sage.debug_qk_int32(dev(r["q_i8"]), dev(r["k_i8"]), N, tiles))
    for n, (g, qt, kt) in enumerate(tiles):
        ref = orc.qk_int32(qi[g], ki[g], qt * 128, 128, kt * 64, 64)
        assert np.array_equal(got[n], ref), (g, qt, kt)
    # an entry outside the tensors gives zeros instead of reading past them
    got = host(sage.debug_qk_int32(dev(r["q_i8"]), dev(r["k_i8"]), N, [(B * H, 0, 0), (0, nqt, 0)]))
    assert not got.any()


# --------------------------------------------------------------------------
# O: within tolerance
# --------------------------------------------------------------------------

def run_gpu(sage, c, **over):
    kw = cfg_kw(c)
    kw.update(over)
    o = sage.attn(dev(c["q"]), dev(c["k"]), dev(c["v"]), **kw)
    return host(o)


def test_attn_config1_all_rows(sage, orc):
    c = inputs(1)
    say("attn cfg1 all rows")
    g = run_gpu(sage, c)
    o = orc.attn(c["q"], c["k"], c["v"], **oracle_kw(c))
    check_o("cfg1", g, o)


# Whole heads at full size: every row of these heads is compared with the oracle.
# Workload 2 (128 heads) in four chunks of 32, eight heads of workloads 3 and 4, four of
# workload 5 (including the last), and rows 0-511 of every workload-5 head (the early
# causal rows see few keys, so one FP8 code of P~ weighs the most there).
WHOLE_HEADS = (
    [(2, tuple(range(32 * i, 32 * i + 32)), None) for i in range(4)]
    + [(3, (0, 5, 11, 17, 23, 29, 41, 47), None)]
    + [(4, (hd,), None) for hd in (0, 6, 13, 20, 27, 34, 41, 47)]
    + [(5, (hd,), None) for hd in (0, 21, 42, 63)]
    + [(5, tuple(range(64)), 512)]
)

# GPU output of each full-size workload, one call per workload per session; and the
# per-case O margins, printed at the end of the module.
_FULL_O = {}
MARGINS = []


def full_size_gpu(sage, cfg):
    if cfg not in _FULL_O:
        _FULL_O.clear()  # one workload's output at a time (workload 5's O is 512 MiB)
        c = inputs(cfg)
        B, H, N, d = c["q"].shape
        say(f"attn cfg{cfg} full size {c['q'].shape} causal={c['causal']} variant={c['variant']} "
            f"kv_tile={sage.kv_tile(c['variant'], d)}")
        _FULL_O[cfg] = run_gpu(sage, c).reshape(B * H, N, d)
    return _FULL_O[cfg]


@pytest.fixture(scope="module", autouse=True)
def margin_report():
    yield
    if MARGINS:
        say("O margins against the oracle (bar: max_abs <= 2e-3, cos >= 0.9999):")
        for name, mx, c, n in MARGINS:
            say(f"  {name:40s} max_abs={mx:.3e} ({100 * mx / TOL_MAX_ABS:5.1f}% of bar) cos={c:.9f} n={n}")


@pytest.mark.slow
@pytest.mark.parametrize("cfg,heads,nrows", WHOLE_HEADS,
                         ids=[f"cfg{c}-h{h[0]}-{h[-1]}" + (f"-rows{r}" if r else "") for c, h, r in WHOLE_HEADS])
def test_attn_full_size_whole_heads(sage, orc, cfg, heads, nrows):
    c = inputs(cfg)
    B, H, N, d = c["q"].shape
    g = full_size_gpu(sage, cfg)
    nr = N if nrows is None else min(nrows, N)
    hs = np.repeat(np.asarray(heads, np.int32), nr)
    rs = np.tile(np.arange(nr, dtype=np.int32), len(heads))
    say(f"  oracle: cfg{cfg} heads {heads[0]}..{heads[-1]} ({len(heads)}), rows 0..{nr - 1}")
    o = orc.attn_rows(c["q"], c["k"], c["v"], hs, rs, **oracle_kw(c))
    name = f"cfg{cfg} heads {heads[0]}-{heads[-1]} rows<{nr}"
    got = g[hs, rs].astype(np.float64)
    MARGINS.append((name, float(np.abs(got - o).max()), cos_sim(got, o), o.size))
    check_o(name, g[hs, rs], o)


EDGE = [
    # name, recipe cfg, overrides of shape, attention options
    ("n1_v0", 1, dict(N=1, B=1, H=1), dict(causal=0, variant=0)),
    ("n1_v1_causal", 5, dict(N=1, B=1, H=1), dict(causal=1, variant=1)),
    ("n17_causal_d64", 1, dict(N=17, B=1, H=2), dict(causal=1, variant=0)),
    ("n65_d128", 2, dict(N=65, B=1, H=2), dict(causal=0, variant=0)),
    ("n129_causal_d128", 2, dict(N=129, B=2, H=1), dict(causal=1, variant=0)),
    ("n200_v1_d64", 1, dict(N=200, B=1, H=2), dict(causal=0, variant=1)),
    ("n300_v1_causal_d64", 3, dict(N=300, B=1, H=2), dict(causal=1, variant=1)),
    ("n520_v1_causal_d64_smoothv", 4, dict(N=520, B=1, H=2), dict(causal=1, variant=1, smooth_v=1)),
    ("n333_v1_causal", 5, dict(N=333, B=1, H=2), dict(causal=1, variant=1)),
    ("blk32_16", 2, dict(N=300, B=1, H=2), dict(causal=1, variant=0, blk_q=32, blk_k=16)),
    ("blk64_128", 3, dict(N=520, B=1, H=2), dict(causal=0, variant=0, blk_q=64, blk_k=128)),
    ("blk32_v1_smoothq", 5, dict(N=400, B=1, H=2), dict(causal=0, variant=1, blk_q=32, blk_k=32)),
    ("nosmooth", 1, dict(N=256, B=1, H=2), dict(causal=0, variant=0, smooth_k=0)),
    ("v0_smoothq", 2, dict(N=256, B=1, H=2), dict(causal=1, variant=0, smooth_q=1)),
    ("v1_no_smoothq", 5, dict(N=256, B=1, H=2), dict(causal=1, variant=1, smooth_q=0)),
    # V smoothing (variant 1): N = 1 leaves V' = 0, so O is the mean, i.e. V itself
    ("n1_v1_smoothv", 5, dict(N=1, B=1, H=1), dict(causal=1, variant=1, smooth_v=1)),
    ("n200_v1_d64_smoothv", 1, dict(N=200, B=1, H=2), dict(causal=0, variant=1, smooth_v=1)),
    ("n333_v1_causal_smoothv", 5, dict(N=333, B=1, H=2), dict(causal=1, variant=1, smooth_v=1)),
    ("blk32_v1_smoothqv", 5, dict(N=400, B=1, H=2), dict(causal=0, variant=1, blk_q=32, blk_k=32, smooth_v=1)),
    ("v1_smoothv_no_smoothq", 5, dict(N=256, B=1, H=2), dict(causal=1, variant=1, smooth_q=0, smooth_v=1)),
    # Q scales finer than the block (q_group rows per scale; 1 = per token)
    ("qg1_v0_d64", 1, dict(N=200, B=1, H=2), dict(causal=0, variant=0, blk_q=64, q_group=1)),
    ("qg4_causal_d128", 2, dict(N=300, B=1, H=2), dict(causal=1, variant=0, q_group=4)),
    ("qg16_blk64_d64", 3, dict(N=520, B=1, H=2), dict(causal=0, variant=0, blk_q=64, blk_k=16, q_group=16)),
    ("qg1_v1_smoothq", 5, dict(N=333, B=1, H=2), dict(causal=1, variant=1, q_group=1)),
    ("qg2_v0_smoothq", 2, dict(N=256, B=1, H=2), dict(causal=1, variant=0, smooth_q=1, q_group=2)),
    ("qg8_v1_smoothqv_d64", 1, dict(N=257, B=1, H=2), dict(causal=0, variant=1, blk_q=32, q_group=8,
                                                           smooth_v=1)),
    # rows dominated by one key (workload 3's x20 outlier K channels): the fp16 rounding of
    # the dominant weight must cancel between P~ V and l (2.06e-3 before l summed the fp16
    # weights, at N = 2100 with the default seed)
    ("peaked_n2100_d64", 3, dict(N=2100, B=1, H=2), dict(causal=0, variant=0)),
    ("peaked_n2100_d64_seed2", 3, dict(N=2100, B=1, H=2, seed=2), dict(causal=0, variant=0)),
    ("peaked_n3000_causal_d64", 3, dict(N=3000, B=1, H=2, seed=1), dict(causal=1, variant=0)),
    # causal query tiles go longest first across pairs of heads; an odd head count leaves
    # the last head alone (24 workgroups: also through the XCD remap; 27: without it)
    ("odd_heads_causal_d128", 2, dict(N=1000, B=1, H=3), dict(causal=1, variant=0)),
    ("odd_heads_causal_d64_v1", 3, dict(N=1100, B=1, H=3), dict(causal=1, variant=1)),
    # MXFP4 scores (variant 2)
    ("mx_n1_causal", 5, dict(N=1, B=1, H=1), dict(causal=1, variant=2, smooth_q=0)),
    ("mx_n17_d64", 1, dict(N=17, B=1, H=2), dict(causal=0, variant=2, smooth_q=0)),
    ("mx_n129_causal_d128", 2, dict(N=129, B=2, H=1), dict(causal=1, variant=2, smooth_q=0)),
    ("mx_n333_causal_d128", 5, dict(N=333, B=1, H=2), dict(causal=1, variant=2, smooth_q=0)),
    ("mx_n200_d64", 3, dict(N=200, B=1, H=2), dict(causal=0, variant=2, smooth_q=0)),
    ("mx_nosmoothk", 1, dict(N=256, B=1, H=2), dict(causal=1, variant=2, smooth_q=0, smooth_k=0)),
    ("mx_smoothv", 5, dict(N=300, B=1, H=2), dict(causal=0, variant=2, smooth_q=0, smooth_v=1)),
]


@pytest.mark.parametrize("name,cfg,shape,opt", EDGE, ids=[e[0] for e in EDGE])
def test_attn_edge_cases_all_rows(sage, orc, name, cfg, shape, opt):
    c = dict(workloads.config(cfg))
    c.update(workloads.make_inputs(cfg, **shape))
    c.update(opt)
    say(f"attn edge {name} {c['q'].shape} {opt}")
    kw = cfg_kw(c)
    kw["smooth_k"] = bool(c.get("smooth_k", 1))
    kw["smooth_q"] = bool(c.get("smooth_q", 1 if c["variant"] == 1 else 0))
    g = host(sage.attn(dev(c["q"]), dev(c["k"]), dev(c["v"]), **kw))
    o = orc.attn(c["q"], c["k"], c["v"], **oracle_kw(c))
    if name.startswith("peaked"):
        MARGINS.append((name, float(np.abs(g.astype(np.float64) - o).max()), cos_sim(g.astype(np.float64), o), o.size))
    check_o(name, g, o)


def test_fp8_pv_accumulator_is_fp32(sage, orc):
    """FP8 P~V accumulates every key tile straight into the fp32 O of the matrix instruction
    (the outer level of two-level accumulation, SageAttention2 abstract).  On this input
    (workloads.make_accum_stress: Q = 0, V sums that climb to ~1e9 and cancel) an
    accumulator of 20 or fewer significand bits, or a truncating 22-bit one, misses the O
    bar (tests/test_accum_input.py); fp32 keeps a tenth of it."""
    c = workloads.make_accum_stress()
    say(f"attn fp8 accumulator stress {c['q'].shape}")
    g = run_gpu(sage, c, smooth_q=False)
    o = orc.attn(c["q"], c["k"], c["v"], **oracle_kw(c))
    check_o("fp8 accumulator stress", g, o)
    MARGINS.append(("fp8 accumulator stress", float(np.abs(g.astype(np.float64) - o).max()),
                    cos_sim(g.astype(np.float64), o), o.size))


def test_attn_q_offset_stress_variant1(sage, orc):
    """Q with a large per-channel offset: the Q-smoothing term carries real weight."""
    c = dict(workloads.config(5))
    c.update(workloads.make_inputs(5, N=2048, B=1, H=2, q_sigma=4.0))
    say("attn v1 q-offset stress N=2048")
    g = run_gpu(sage, c)
    o = orc.attn(c["q"], c["k"], c["v"], **oracle_kw(c))
    check_o("q_offset_v1", g, o)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_attn_full_size_mxfp4_sampled_rows(sage, orc, cfg):
    """The MXFP4 variant on each workload's full shape (sampled rows)."""
    c = dict(inputs(cfg))
    c.update(variant=2, smooth_q=0)
    B, H, N, d = c["q"].shape
    G = B * H
    say(f"attn mxfp4 cfg{cfg} full size {c['q'].shape} causal={c['causal']}")
    g = run_gpu(sage, c).reshape(G, N, d)
    rng = np.random.default_rng(300 + cfg)
    heads, rows = [], []
    for hd in (0, G // 2 + 1, G - 1):
        for r in sample_rows(N, c["causal"], rng):
            heads.append(hd)
            rows.append(r)
    o = orc.attn_rows(c["q"], c["k"], c["v"], heads, rows, **oracle_kw(c))
    check_o(f"mxfp4 cfg{cfg} sampled {len(rows)} rows", g[heads, rows], o)


def test_prequant_mx_matches_whole_call(sage):
    c = workloads.make_inputs(5, N=1000, B=1, H=2, v_sigma=1.0)
    say("prequant_mx vs whole call, with V smoothing")
    q, k, v = dev(c["q"]), dev(c["k"]), dev(c["v"])
    N = c["q"].shape[2]
    whole = sage.attn(q, k, v, causal=True, variant=2, smooth_q=False, smooth_v=True)
    qk = sage.quant_qk_mx(q, k)
    vq = sage.quant_v(v, smooth_v=True)
    pre = sage.attn_prequant_mx(qk, vq, N, causal=True, smooth_v=True)
    fused = sage.attn_qf16_mx(q, qk, vq, causal=True, smooth_v=True)
    torch.cuda.synchronize()
    assert torch.isfinite(whole.float()).all()
    # the whole call quantises Q in the attention kernel: same codes, same bits
    assert torch.equal(whole, pre)
    assert torch.equal(whole, fused)


@pytest.mark.parametrize("cfg,shape,causal", [(2, dict(N=333, B=1, H=2), 1), (3, dict(N=200, B=1, H=3), 0),
                                              (1, dict(N=65, B=1, H=1), 0)])
def test_fused_mx_q_matches_quant_pass(sage, cfg, shape, causal):
    """Variant 2's in-kernel MXFP4 Q equals quant_qk_mx's: fused and pre-quantised kernels give
    the same bits.  Q carries an all-zero block, a negative zero row and saturating values."""
    c = workloads.make_inputs(cfg, **shape)
    q = c["q"].copy()
    q[0, 0, 2, :32] = 0
    q[0, 0, 3, :] = -0.0
    q[0, 0, 4, 1] = -7.99
    say(f"fused MX Q {q.shape} causal={causal}")
    qd, kd, vd = dev(q), dev(c["k"]), dev(c["v"])
    qk = sage.quant_qk_mx(qd, kd)
    vq = sage.quant_v(vd)
    fused = sage.attn_qf16_mx(qd, qk, vq, causal=bool(causal))
    pre = sage.attn_prequant_mx(qk, vq, q.shape[2], causal=bool(causal))
    torch.cuda.synchronize()
    assert torch.equal(fused, pre)


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_attn_full_size_per_token_q_sampled_rows(sage, orc, cfg):
    """Per-token Q scales (q_group = 1) on each workload's full shape (sampled rows)."""
    c = dict(inputs(cfg))
    c.update(q_group=1)
    B, H, N, d = c["q"].shape
    G = B * H
    say(f"attn q_group=1 cfg{cfg} full size {c['q'].shape} causal={c['causal']} variant={c['variant']}")
    g = run_gpu(sage, c).reshape(G, N, d)
    rng = np.random.default_rng(200 + cfg)
    heads, rows = [], []
    for hd in (0, G // 2, G - 1):
        for r in sample_rows(N, c["causal"], rng):
            heads.append(hd)
            rows.append(r)
    o = orc.attn_rows(c["q"], c["k"], c["v"], heads, rows, **oracle_kw(c))
    check_o(f"q_group=1 cfg{cfg} sampled {len(rows)} rows", g[heads, rows], o)


def test_attn_per_token_q_mixed_row_magnitudes(sage, orc):
    """One Q row in eight 64x larger: parity per block and per token, and the per-token
    GPU output is the closer one to exact attention on the ordinary rows."""
    rng = np.random.default_rng(9)
    N, d = 512, 128
    q = rng.standard_normal((1, 2, N, d))
    q[:, :, ::8] *= 64.0
    q = q.astype(np.float16)
    k = rng.standard_normal((1, 2, N, d)).astype(np.float16)
    v = rng.standard_normal((1, 2, N, d)).astype(np.float16)
    exact = orc.attn(q, k, v, exact=1)
    ordinary = np.ones(N, bool)
    ordinary[::8] = False
    err = {}
    for qg in (0, 1):
        say(f"attn mixed-magnitude Q rows q_group={qg}")
        g = host(sage.attn(dev(q), dev(k), dev(v), q_group=qg))
        o = orc.attn(q, k, v, q_group=qg or None)
        check_o(f"mixed rows q_group={qg}", g, o)
        err[qg] = float(np.abs(g.astype(np.float64) - exact)[:, :, ordinary].mean())
    say(f"  mean |O - exact| on ordinary rows: per block {err[0]:.3e}, per token {err[1]:.3e}")
    assert err[1] < err[0] / 4


@pytest.mark.parametrize("cfg", [2, 3, 4, 5])
def test_attn_full_size_smooth_v_sampled_rows(sage, orc, cfg):
    """Variant 1 with Q and V smoothing on each workload's full shape (sampled rows)."""
    c = dict(inputs(cfg))
    c.update(variant=1, smooth_q=1, smooth_v=1)
    B, H, N, d = c["q"].shape
    G = B * H
    say(f"attn smooth_v cfg{cfg} full size {c['q'].shape} causal={c['causal']}")
    g = run_gpu(sage, c).reshape(G, N, d)
    rng = np.random.default_rng(100 + cfg)
    heads, rows = [], []
    for hd in (0, G // 3, G - 1):
        for r in sample_rows(N, c["causal"], rng):
            heads.append(hd)
            rows.append(r)
    o = orc.attn_rows(c["q"], c["k"], c["v"], heads, rows, **oracle_kw(c))
    check_o(f"smooth_v cfg{cfg} sampled {len(rows)} rows", g[heads, rows], o)


def test_attn_v_offset_stress_smooth_v(sage, orc):
    """V = 0.25 z + a per-channel offset ~ N(0, 1): parity with and without V smoothing, and
    the smoothed GPU output is the closer one to exact attention (the point of smoothing V;
    the oracle gives mean errors of about 2.0e-3 and 0.54e-3 here)."""
    c = dict(workloads.config(5))
    c.update(workloads.make_inputs(5, N=2048, B=1, H=2, v_sigma=1.0, v_spread=0.25))
    exact = orc.attn(c["q"], c["k"], c["v"], causal=1, exact=1)
    err = {}
    for sv in (0, 1):
        c["smooth_v"] = sv
        say(f"attn v1 v-offset stress N=2048 smooth_v={sv}")
        g = run_gpu(sage, c)
        o = orc.attn(c["q"], c["k"], c["v"], **oracle_kw(c))
        check_o(f"v_offset smooth_v={sv}", g, o)
        err[sv] = float(np.abs(g.astype(np.float64) - exact).mean())
    say(f"  mean |O - exact|: plain {err[0]:.3e}, smoothed {err[1]:.3e}")
    assert err[1] < 0.5 * err[0]


def test_prequant_smooth_v_matches_whole_call(sage):
    c = workloads.make_inputs(5, N=1000, B=1, H=2, v_sigma=1.0)
    say("prequant vs whole call, variant 1 with Q and V smoothing")
    q, k, v = dev(c["q"]), dev(c["k"]), dev(c["v"])
    N = c["q"].shape[2]
    whole = sage.attn(q, k, v, causal=True, variant=1, smooth_v=True)
    qk = sage.quant_qk(q, k, smooth_q=True)
    vq = sage.quant_v(v, smooth_v=True)
    pre = sage.attn_prequant(qk, None, N, causal=True, variant=1, vq=vq, smooth_v=True)
    torch.cuda.synchronize()
    assert torch.isfinite(whole.float()).all()
    assert torch.equal(whole, pre)


@pytest.mark.parametrize("variant", [0, 1])
def test_attn_degenerate_inputs(sage, orc, variant):
    """Q = 0 (uniform attention) and constant K (zero codes after smoothing)."""
    rng = np.random.default_rng(5)
    N, d = 150, 64
    v = rng.standard_normal((1, 1, N, d)).astype(np.float16)
    k = rng.standard_normal((1, 1, N, d)).astype(np.float16)
    q = rng.standard_normal((1, 1, N, d)).astype(np.float16)
    for name, (qq, kk) in {"q_zero": (np.zeros_like(q), k), "k_const": (q, np.full_like(k, 1.5))}.items():
        for causal in (0, 1):
            say(f"attn degenerate {name} variant={variant} causal={causal}")
            g = host(sage.attn(dev(qq), dev(kk), dev(v), causal=bool(causal), variant=variant))
            o = orc.attn(qq, kk, v, causal=causal, variant=variant)
            check_o(f"{name} v{variant} c{causal}", g, o)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [0, 1])
def test_attn_rising_scores_interior_tiles(sage, orc, d, causal):
    """Variant 0's interior tiles form P~ against the row's running reference and fall back
    to the tile maximum when a lane's 32 weights sum past 2^10.  Keys along one direction
    with an oscillating, rising weight f(j) put the scores of later tiles up to ~20 (base 2)
    above the reference or far below it, so along every row some interior tiles are kept
    with large P~ and others are recomputed; rows differ in scale and (causal) in prefix."""
    rng = np.random.default_rng(17)
    N = 1000
    sm = 1.0 / np.sqrt(d)
    a = np.sqrt(20.0 / (sm * 1.4426950408889634))  # |u|^2 sm log2(e) = 20
    u = rng.standard_normal(d)
    u *= a / np.linalg.norm(u)
    j = np.arange(N)
    f = 0.6 * np.sin(j / 37.0) + 0.4 * j / N
    q = np.empty((1, 2, N, d), np.float16)
    k = np.empty((1, 2, N, d), np.float16)
    for hh in range(2):
        q[0, hh] = (u[None, :] * (0.5 + j / N)[:, None] + 0.05 * rng.standard_normal((N, d))).astype(np.float16)
        k[0, hh] = (u[None, :] * f[:, None] + 0.05 * rng.standard_normal((N, d))).astype(np.float16)
    v = rng.standard_normal((1, 2, N, d)).astype(np.float16)
    say(f"attn rising scores d={d} causal={causal}")
    g = host(sage.attn(dev(q), dev(k), dev(v), causal=bool(causal), variant=0))
    o = orc.attn(q, k, v, causal=causal, variant=0, bkv=sage.kv_tile(0, d))
    check_o(f"rising d{d} c{causal}", g, o)


@pytest.mark.parametrize("d,sigma,causal", [(128, 74.0, 0), (128, 251.0, 1), (64, 74.0, 1), (64, 251.0, 0)])
def test_attn_large_logit_scale(sage, orc, d, sigma, causal):
    """Logit scales far past the workloads': Q and K with standard deviation 74 or 251 give
    c = dQ dK sm_scale log2(e) of about 0.9 to 15 per unit of the INT8 score, row maxima
    of about 3e4 and 4e5 (base 2) and a softmax that is close to a hard maximum.  Every
    fp32 step of the exponent (c S - m) has to hold here, since differences of a few
    units decide the weights; variant 0 against the oracle on every element."""
    rng = np.random.default_rng(31)
    N = 700
    q = (sigma * rng.standard_normal((1, 2, N, d))).astype(np.float16)
    k = (sigma * rng.standard_normal((1, 2, N, d))).astype(np.float16)
    v = rng.standard_normal((1, 2, N, d)).astype(np.float16)
    say(f"attn large logit scale d={d} sigma={sigma} causal={causal}")
    g = host(sage.attn(dev(q), dev(k), dev(v), causal=bool(causal), variant=0))
    o = orc.attn(q, k, v, causal=causal, variant=0, bkv=sage.kv_tile(0, d))
    check_o(f"large logits d{d} s{sigma:g} c{causal}", g, o)


@pytest.mark.parametrize("shape", [(1, 1, 0, 64), (0, 2, 16, 128), (2, 0, 8, 64)])
@pytest.mark.parametrize("variant", [0, 1, 2])
def test_attn_empty_inputs(sage, shape, variant):
    """No heads or no tokens: the output is empty, nothing is launched."""
    say(f"attn empty shape={shape} variant={variant}")
    import torch
    x = torch.zeros(shape, dtype=torch.float16, device="cuda")
    o = sage.attn(x, x, x, causal=True, variant=variant)
    assert o.shape == x.shape and o.numel() == 0


@pytest.mark.parametrize("cfg,variant", [(5, 1), (2, 2), (5, 2)])
def test_full_size_deterministic(sage, cfg, variant):
    """Two whole calls on the same full-size input give the same bits (no races between the
    waves that share a tile, and no order-dependent reductions)."""
    c = dict(inputs(cfg))
    c["variant"] = variant
    say(f"determinism cfg{cfg} variant {variant} {c['q'].shape}")
    q, k, v = dev(c["q"]), dev(c["k"]), dev(c["v"])
    kw = cfg_kw(c)
    kw["smooth_q"] = variant == 1
    a = sage.attn(q, k, v, **kw)
    b = sage.attn(q, k, v, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(a.float()).all()
    assert torch.equal(a, b)


def test_prequant_matches_whole_call_and_is_deterministic(sage):
    c = inputs(2)
    say("prequant vs whole call, determinism (cfg2)")
    q, k, v = dev(c["q"]), dev(c["k"]), dev(c["v"])
    a = sage.attn(q, k, v, **cfg_kw(c))
    b = sage.attn(q, k, v, **cfg_kw(c))
    qk = sage.quant_qk(q, k, blk_q=c["blk_q"], blk_k=c["blk_k"])
    p = sage.attn_prequant(qk, v, c["q"].shape[2], causal=True, variant=0, blk_q=c["blk_q"], blk_k=c["blk_k"])
    torch.cuda.synchronize()
    assert torch.equal(a, b)
    assert torch.equal(a, p)


FUSED = [
    # recipe cfg, shape overrides, blk_q, blk_k, causal, q_group
    (2, dict(N=333, B=1, H=3), 128, 64, 1, 0),
    (2, dict(N=1000, B=2, H=1), 64, 16, 0, 0),
    (3, dict(N=200, B=1, H=2), 32, 64, 1, 0),
    (3, dict(N=4096, B=1, H=2), 128, 128, 0, 0),
    (1, dict(N=65, B=1, H=1), 32, 32, 0, 0),
    (2, dict(N=333, B=1, H=2), 128, 64, 1, 1),
    (3, dict(N=300, B=1, H=2), 64, 64, 0, 2),
    (2, dict(N=257, B=1, H=2), 128, 16, 1, 8),
    (3, dict(N=129, B=1, H=1), 32, 32, 0, 16),
    (2, dict(N=500, B=1, H=2), 128, 64, 0, 64),
]


@pytest.mark.parametrize("cfg,shape,blk_q,blk_k,causal,q_group", FUSED)
def test_fused_q_quantisation_matches_quant_pass(sage, cfg, shape, blk_q, blk_k, causal, q_group):
    """Variant 0 quantises Q inside the attention kernel: the whole call, the fused kernel
    alone and the quantisation pass + pre-quantised kernel give the same bits.  One Q block
    is all zeros (scale 0, codes 0)."""
    c = workloads.make_inputs(cfg, **shape)
    q = c["q"].copy()
    q[0, 0, :blk_q] = 0
    say(f"fused Q {q.shape} blk_q={blk_q} blk_k={blk_k} causal={causal} q_group={q_group}")
    qd, kd, vd = dev(q), dev(c["k"]), dev(c["v"])
    N = q.shape[2]
    kw = dict(causal=bool(causal), blk_q=blk_q, blk_k=blk_k, q_group=q_group)
    whole = sage.attn(qd, kd, vd, variant=0, **kw)
    qk = sage.quant_qk(qd, kd, blk_q=blk_q, blk_k=blk_k, q_group=q_group)
    fused = sage.attn_qf16(qd, qk, vd, **kw)
    pre = sage.attn_prequant(qk, vd, N, variant=0, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(whole.float()).all()
    assert torch.equal(whole, fused)
    assert torch.equal(whole, pre)


FUSED_SMOOTH = [
    # variant, recipe cfg, shape overrides, blk_q, blk_k, causal, q_group, smooth_v
    (1, 5, dict(N=333, B=1, H=2), 128, 64, 1, 0, 0),
    (1, 5, dict(N=1000, B=1, H=2), 64, 32, 0, 0, 1),
    (1, 1, dict(N=200, B=1, H=2), 32, 64, 1, 0, 0),
    (1, 3, dict(N=300, B=1, H=2), 128, 16, 0, 1, 0),
    (1, 2, dict(N=257, B=1, H=2), 64, 64, 1, 8, 1),
    (1, 4, dict(N=129, B=2, H=1), 128, 64, 0, 32, 0),
    (0, 2, dict(N=333, B=1, H=2), 128, 64, 1, 0, 0),
    (0, 3, dict(N=200, B=1, H=2), 32, 32, 0, 4, 0),
]


@pytest.mark.parametrize("variant,cfg,shape,blk_q,blk_k,causal,q_group,smooth_v", FUSED_SMOOTH)
def test_fused_smoothed_q_matches_quant_pass(sage, variant, cfg, shape, blk_q, blk_k, causal, q_group, smooth_v):
    """With Q smoothing the attention kernel takes each Q block's exact mean and quantises the
    smoothed rows itself: the whole call, the fused kernel alone and the quantisation pass +
    pre-quantised kernel give the same bits.  One Q block is all zeros; one has an offset
    larger than its spread."""
    c = workloads.make_inputs(cfg, **shape)
    q = c["q"].copy()
    q[0, 0, :blk_q] = 0
    q[0, -1, blk_q:2 * blk_q] += np.float16(6.0)
    say(f"fused smoothed Q v{variant} {q.shape} blk_q={blk_q} blk_k={blk_k} causal={causal} q_group={q_group} "
        f"smooth_v={smooth_v}")
    qd, kd, vd = dev(q), dev(c["k"]), dev(c["v"])
    N = q.shape[2]
    kw = dict(causal=bool(causal), blk_q=blk_q, blk_k=blk_k, q_group=q_group, smooth_q=True)
    qk = sage.quant_qk(qd, kd, blk_q=blk_q, blk_k=blk_k, smooth_q=True, q_group=q_group)
    if variant == 1:
        whole = sage.attn(qd, kd, vd, variant=1, smooth_v=bool(smooth_v), **kw)
        vq = sage.quant_v(vd, smooth_v=bool(smooth_v))
        fused = sage.attn_qf16_fp8(qd, qk, vq, smooth_v=bool(smooth_v), **kw)
        pre = sage.attn_prequant(qk, vd, N, variant=1, vq=vq, smooth_v=bool(smooth_v), **kw)
    else:
        whole = sage.attn(qd, kd, vd, variant=0, **kw)
        fused = sage.attn_qf16(qd, qk, vd, **kw)
        pre = sage.attn_prequant(qk, vd, N, variant=0, **kw)
    torch.cuda.synchronize()
    assert torch.isfinite(whole.float()).all()
    assert torch.equal(whole, fused)
    assert torch.equal(whole, pre)


@pytest.mark.parametrize("variant", [0, 1, 2])
def test_attn_maximum_size_sampled_heads(sage, orc, variant):
    """B*H*pad_len(N)*d one tile short of 2^31 (131071 heads of N = 100, d = 128): offsets
    near the limit of the contract.  Inputs come from torch's seeded generator on the
    GPU; the sampled heads are copied back for the oracle."""
    H, N, d = 131071, 100, 128
    assert H * 128 * d < 2 ** 31 <= (H + 1) * 128 * d
    gen = torch.Generator(device="cuda").manual_seed(77 + variant)
    shape = (1, H, N, d)
    q = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).half()
    k = (torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32)
         + 3.0 * torch.randn((1, H, 1, d), generator=gen, device="cuda", dtype=torch.float32)).half()
    v = torch.randn(shape, generator=gen, device="cuda", dtype=torch.float32).half()
    say(f"attn maximum size {shape} variant={variant}")
    o = sage.attn(q, k, v, causal=True, variant=variant)
    heads = [0, 1, H // 2, H - 2, H - 1]
    sel = torch.tensor(heads, device="cuda")
    qs, ks, vs = (host(t.index_select(1, sel)) for t in (q, k, v))
    g = host(o.index_select(1, sel)).astype(np.float64)
    del q, k, v, o
    torch.cuda.empty_cache()
    ref = orc.attn(qs, ks, vs, causal=1, variant=variant)
    check_o(f"max size v{variant}", g, ref)


def test_api_rejects_bad_arguments_on_gpu(sage):
    q = torch.zeros((1, 1, 64, 96), dtype=torch.float16, device="cuda")
    with pytest.raises(sage.SageError, match="head dim"):
        sage.attn(q, q, q)
    q = torch.zeros((1, 1, 64, 64), dtype=torch.float16, device="cuda")
    with pytest.raises(sage.SageError, match="sm_scale"):
        sage.attn(q, q, q, sm_scale=-1.0)
    with pytest.raises(sage.SageError, match="blk_q"):
        sage.attn(q, q, q, blk_q=48)


def test_binding_rejects_bad_outputs_and_operands(sage):
    """The binding checks caller-supplied outputs and pre-quantised operands before any
    launch: a wrong shape, dtype, layout or length would make the kernels read or write
    past the buffers."""
    B, H, N, d = 1, 2, 200, 64
    q = torch.zeros((B, H, N, d), dtype=torch.float16, device="cuda")
    bad_outs = [torch.zeros((B, H, N + 1, d), dtype=torch.float16, device="cuda"),
                torch.zeros((B, H, N, d), dtype=torch.float32, device="cuda"),
                torch.zeros((B, H, d, N), dtype=torch.float16, device="cuda").transpose(2, 3)]
    for out in bad_outs:
        with pytest.raises((ValueError, TypeError)):
            sage.attn(q, q, q, out=out)
    with pytest.raises(ValueError):
        sage.attn(q, q, q, workspace=torch.zeros(16, dtype=torch.uint8))
    qk = sage.quant_qk(q, q)
    vq = sage.quant_v(q)
    # N must give the padded length the quantised tensors have
    with pytest.raises(ValueError, match="padded length"):
        sage.attn_prequant(qk, q, 300)
    with pytest.raises(ValueError):
        sage.attn_prequant(qk, q, N, out=bad_outs[0])
    # scales of another block size
    with pytest.raises(ValueError, match="k_scale"):
        sage.attn_prequant(qk, q, N, blk_k=32)
    with pytest.raises(TypeError, match="v_f8"):
        sage.attn_prequant(sage.quant_qk(q, q, smooth_q=True), None, N, variant=1,
                           vq=dict(vq, v_f8=vq["v_f8"].to(torch.int8)))
    with pytest.raises(ValueError, match="k_i8"):
        sage.attn_qf16(torch.zeros((B, H, 100, d), dtype=torch.float16, device="cuda"), qk,
                       torch.zeros((B, H, 100, d), dtype=torch.float16, device="cuda"))
    mx = sage.quant_qk_mx(q, q)
    with pytest.raises(ValueError, match="padded length"):
        sage.attn_prequant_mx(mx, vq, 100)
    with pytest.raises(ValueError, match="v_mean"):
        sage.attn_qf16_mx(q, mx, dict(vq, v_mean=vq["v_mean"][..., :8]), smooth_v=True)
    with pytest.raises(ValueError):
        sage.debug_qk_int32(qk["q_i8"], qk["k_i8"], 1000, [(0, 0, 0)])
    torch.cuda.synchronize()
