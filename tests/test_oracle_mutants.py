"""The pins catch plausible mistakes in the oracle.

Each case copies oracle.c, plants one mistake by text substitution (a dropped
term, a wrong sign, index or constant, a transposed operand), builds the copy on
the CPU, and runs the pin battery against it: at least one pin must fail.
The real oracle is never modified.
"""
import os
import shutil
import subprocess

import pytest

import oracle as oracle_pkg
from oracle import Oracle
from tests import test_oracle_bwd_pins as bw
from tests import test_oracle_fp4pv_pins as fp4
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle_pkg.__file__), "oracle.c")

MUTANTS = {
    "v0 rescale dropped": ("o[c] = alpha * o[c] + acc;", "o[c] = o[c] + acc;"),
    "v1 outer rescale dropped": ("o[c] = alpha * o[c] + inner[c];", "o[c] = o[c] + inner[c];"),
    "l rescale dropped": ("l = alpha * l + psum;", "l = l + psum;"),
    "mean divisor off by one": ("((double)(r1 - r0) * 16777216.0)", "((double)(r1 - r0 + 1) * 16777216.0)"),
    "smoothing not applied": ("mean_mode ? v - mean[c] : v", "v"),
    "q-smoothing term sign": ("sj += P->sm_scale * dk * ds;", "sj -= P->sm_scale * dk * ds;"),
    "int8 range 128": ("float r = 127.0f / a;", "float r = 128.0f / a;"),
    "truncation instead of rne": ("float t = rintf(xs[i] * r);", "float t = truncf(xs[i] * r);"),
    "scale not divided": ("return a / 127.0f;", "return a / 128.0f;"),
    "causal includes diagonal wrongly": ("if (P->causal && j > i) {", "if (P->causal && j >= i + 1 && j != i + 1) {"),
    "k scale indexed by q block": ("h->ks[j / P->blk_k]", "h->ks[j / P->blk_q]"),
    "q block index from k blocks": ("const int qb = i / P->blk_q;", "const int qb = i / P->blk_k;"),
    "v fp8 operand transposed": ("acc += p[j - j0] * oracle_e4m3_decode(vrow[j]);",
                                 "acc += p[j - j0] * oracle_e4m3_decode(h->vt[(size_t)j * d + c % d]);"),
    "fp8 epilogue 448 dropped": ("o[c] * (double)h->vs[c] / (448.0 * l)", "o[c] * (double)h->vs[c] / l"),
    "e4m3 rounding floors": ("double q = nearbyint(ldexp(a, 3 - E));", "double q = floor(ldexp(a, 3 - E));"),
    "f16 encode exponent bias": ("((E + 15) << 10)", "((E + 14) << 10)"),
    "dequant drops q scale": ("sj = P->sm_scale * (double)h->qs[i / P->q_group] * dk * (double)S;",
                              "sj = P->sm_scale * dk * (double)S;"),
    "q scale indexed by smoothing block": ("h->qs[i / P->q_group]", "h->qs[i / P->blk_q]"),
    "q groups span the smoothing block": ("int r0 = gi * grp, r1 = r0 + grp < N ? r0 + grp : N;",
                                          "int r0 = gi * grp, r1 = (r0 / blk + 1) * blk < N ? (r0 / blk + 1) * blk : N;"),
    "p~ fp8 scale dropped": ("const float shift = kLog2_448f - mnew;", "const float shift = 0.0f - mnew;"),
    "fp8 q-smoothing term sign": ("t[j - j0] = fmaf(S, c, term);", "t[j - j0] = fmaf(S, c, -term);"),
    "fp8 shift from the tile max": ("const float shift = kLog2_448f - mnew;", "const float shift = kLog2_448f - tmax;"),
    "fp8 mean fixed point truncates": ("(int64_t)rintf(ldexpf(qm[c], 27 - e))", "(int64_t)truncf(ldexpf(qm[c], 27 - e))"),
    "fp8 term scale exponent": ("f->s3 = ldexpf(1.0f, e - 27);", "f->s3 = ldexpf(1.0f, e - 26);"),
    "fp8 l sums the fp8 value": ("psum += (double)p448 / 448.0;", "psum += oracle_e4m3_decode(oracle_e4m3_encode((double)p448)) / 448.0;"),
    "v mean not added back": ("/ (448.0 * l) + (double)h->vm[c];", "/ (448.0 * l);"),
    "v mean subtracted twice": ("      if (smooth_v) x = x - mean;\n      float y = x * r;",
                                "      if (smooth_v) x = x - mean - mean;\n      float y = x * r;"),
    "mx exponent off by one": ("code = (e - 1) - 2 + 127;", "code = (e - 1) - 1 + 127;"),
    "e2m1 ties to odd": ("(dc == db && (c & 1) == 0)", "(dc == db && (c & 1) == 1)"),
    "mx score drops the k block scale": ("(int)h->qe[(size_t)i * nb + b] + (int)h->ke[(size_t)j * nb + b] - 254",
                                         "(int)h->qe[(size_t)i * nb + b] + (int)h->ke[(size_t)j * nb] - 254"),
    "mx k not smoothed": ("quant_head_mx(k, N, Np, d, P->smooth_k ? 1 : 0,", "quant_head_mx(k, N, Np, d, 0,"),
    "v absmax before smoothing": ("      if (smooth_v) x = x - mean;\n      a = fmaxf(a, fabsf(x));",
                                  "      a = fmaxf(a, fabsf(x));"),
    # MXFP4 P~V (variant 3)
    "fp4 p rule saturates": ("code = (e - 1) - 2 + (f > 1.5 ? 1 : 0) + 127;", "code = (e - 1) - 2 + 127;"),
    "fp4 p blocks of 64 keys": ("for (int b0 = 0; b0 < bkv; b0 += 32) {\n      const uint8_t e = p_block_fp4(pf + b0, 32, pc + b0);\n"
                                "      for (int u = b0; u < b0 + 32; ++u)",
                                "for (int b0 = 0; b0 < bkv; b0 += 64) {\n      const uint8_t e = p_block_fp4(pf + b0, 64, pc + b0);\n"
                                "      for (int u = b0; u < b0 + 64; ++u)"),
    "fp4 l sums the decoded p": ("l = alpha * l + wsum;",
                                 "{ double s2 = 0.0; for (int u = 0; u < bkv; ++u) s2 += pdec[u]; l = alpha * l + s2; }"),
    "fp4 rescale dropped": ("o[cc] = alpha * o[cc] + inner[cc];", "o[cc] = o[cc] + inner[cc];"),
    "fp4 v scale of the wrong block": ("(int)erow[j / 32] - 127", "(int)erow[j / 64] - 127"),
    "fp4 v mean not added back": ("o[cc] = o[cc] / l + (double)h->vm[cc];", "o[cc] = o[cc] / l;"),
    "fp4 p shift keeps 448": ("pf[j - j0] = (float)exp2((double)fmaf(Sf[j - j0], c, -mnew));",
                              "pf[j - j0] = (float)exp2((double)fmaf(Sf[j - j0], c, kLog2_448f - mnew));"),
    "fp4 v tokens shifted": ("const int t = 32 * b + u;", "const int t = 32 * b + u + 1;"),
    "fp4 v smoothing skipped": ("x[u] = smooth_v ? y - mean : y;", "x[u] = y;"),
    # backward
    "bwd D without the V-mean shift": ("if (!P->exact && P->smooth_v) D -= g * (double)vmean[c];", ""),
    "bwd dS sign": ("const double dsv = p * (dp - D);", "const double dsv = p * (D - dp);"),
    "bwd dK uses K": ("dk[(size_t)j * d + c] += P->sm_scale * ds[j] * qv;",
                      "dk[(size_t)j * d + c] += P->sm_scale * ds[j] * kv;"),
    "bwd dQ without sm_scale": ("dq[(size_t)i * d + c] += P->sm_scale * ds[j] * kv;",
                                "dq[(size_t)i * d + c] += ds[j] * kv;"),
    "bwd P not normalised": ("const double L = m + log(lsum);", "const double L = m;"),
    "bwd dP scale of V dropped": ("dp = (double)gs[i] * (double)vs[j] * (double)S;", "dp = (double)gs[i] * (double)S;"),
    "bwd sigma not undone": ("ds[j] = oracle_f16_decode(oracle_f16_encode(sigma * dsv)) / sigma;",
                             "ds[j] = oracle_f16_decode(oracle_f16_encode(sigma * dsv));"),
    "bwd sigma from V only": ("const double bound = 2.0 * gmax * vmax;", "const double bound = 2.0 * vmax;"),
    "bwd dV uses the row of dO of the key": ("dv[(size_t)j * d + c] += pr[j] * gv;",
                                             "dv[(size_t)j * d + c] += pr[j] * gf[(size_t)j * d + c];"),
    "bwd causal mask dropped": ("const int jend = P->causal ? i + 1 : N;", "const int jend = N;"),
    "bwd dQ uses unsmoothed K": ("const float x = (float)oracle_f16_decode(k[(size_t)t * d + c]) - kmean[c];",
                                 "const float x = (float)oracle_f16_decode(k[(size_t)t * d + c]);"),
}


def _battery(orc):
    """The pins, as (name, thunk) pairs."""
    yield "f16 decode", lambda: pins.test_f16_decode_all_codes_match_numpy(orc)
    yield "f16 encode", lambda: pins.test_f16_encode_matches_numpy_rne(orc)
    yield "e4m3 decode", lambda: pins.test_e4m3_decode_all_codes_match_torch(orc)
    yield "e4m3 encode", lambda: pins.test_e4m3_encode_rne_and_saturation(orc)
    for a in [(7, 3, 4, 3, 4), (10, 5, 10, 4, 10), (5, 8, 2, 5, 2), (10, 5, 10, 4, 5), (7, 3, 4, 3, 1)]:
        yield f"fraction quant {a}", lambda a=a: pins.test_quant_matches_fraction_bruteforce(orc, *a)
    yield "per-token scale", lambda: pins.test_per_token_q_scale_is_the_row_absmax(orc)
    yield "per-token mixed rows", lambda: pins.test_per_token_q_helps_rows_of_mixed_magnitude(orc)
    yield "roundtrip", lambda: pins.test_quant_roundtrip_bound_and_absmax(orc)
    yield "smoothing shift", lambda: pins.test_smoothing_subtracts_exact_token_mean(orc)
    yield "qk int32", lambda: pins.test_qk_int32_matches_numpy_int64(orc)
    for a in [(37, 0, 16), (37, 1, 16)]:
        yield f"online {a}", lambda a=a: pins.test_online_softmax_equals_textbook(orc, *a)
    for var in (0, 1):
        yield f"q zero v{var}", lambda var=var: pins.test_closed_form_q_zero_gives_mean_of_visible_v(orc, var)
        for causal in (0, 1):
            yield f"lossless v{var} c{causal}", (
                lambda var=var, causal=causal: pins.test_lossless_inputs_match_exact_attention(orc, var, causal))
    yield "single token", lambda: pins.test_closed_form_single_token_and_causal_row0(orc)
    for var in (0, 1):
        yield f"q smoothing term v{var}", lambda var=var: pins.test_q_smoothing_term_restores_scores(orc, var)
    for causal in (0, 1):
        yield f"fp8 l unrounded c{causal}", lambda causal=causal: pins.test_fp8_l_sums_the_unrounded_p(orc, causal)
    for seed in (0, 1, 2):
        yield f"fp8 q smoothing term {seed}", lambda seed=seed: pins.test_fp8_q_smoothing_term_bruteforce(orc, seed)
    yield "vs fp64 cfg1", lambda: pins.test_oracle_vs_fp64_attention_config1(orc)
    yield "v smoothing quant", lambda: pins.test_v_smoothing_quant_matches_fraction_bruteforce(orc)
    for causal in (0, 1):
        yield f"v smoothing constant c{causal}", (
            lambda causal=causal: pins.test_v_smoothing_constant_v_is_returned_exactly(orc, causal))
    yield "v smoothing offset", lambda: pins.test_v_smoothing_removes_the_channel_offset_error(orc)
    yield "e2m1 decode", lambda: pins.test_e2m1_decode_matches_the_ocp_table(orc)
    yield "e2m1 encode", lambda: pins.test_e2m1_encode_rne_and_saturation(orc)
    yield "mx block", lambda: pins.test_mx_block_matches_bruteforce(orc)
    for causal in (0, 1):
        yield f"mx lossless c{causal}", lambda causal=causal: pins.test_mx_lossless_inputs_match_exact_attention(orc, causal)
    yield "mx k smoothing", lambda: pins.test_mx_k_smoothing_removes_the_channel_offset_error(orc)
    yield "fp4 p rule", lambda: fp4.test_p_block_scale_is_the_smallest_that_does_not_saturate(orc)
    yield "fp4 p below a power of two", lambda: fp4.test_p_block_keeps_a_weight_just_below_a_power_of_two(orc)
    yield "fp4 v blocks", lambda: fp4.test_v_mx_blocks_run_along_the_tokens(orc)
    yield "fp4 v smoothing", lambda: fp4.test_v_mx_smoothing_subtracts_the_exact_token_mean(orc)
    for causal in (0, 1):
        yield f"fp4 q zero c{causal}", lambda causal=causal: fp4.test_q_zero_gives_the_mean_of_the_visible_v(orc, causal)
        yield f"fp4 lossless c{causal}", (
            lambda causal=causal: fp4.test_lossless_inputs_match_base2_softmax_attention(orc, causal))
        yield f"fp4 l unrounded c{causal}", lambda causal=causal: fp4.test_l_sums_the_unrounded_p(orc, causal)
        yield f"fp4 const v c{causal}", lambda causal=causal: fp4.test_v_smoothing_returns_a_constant_v_exactly(orc, causal)
    yield "fp4 v scaling", lambda: fp4.test_power_of_two_scaling_of_v_scales_o(orc)
    yield "fp4 vs fp64", lambda: fp4.test_fp4_attention_tracks_fp64_attention_config1(orc)
    for a in [(37, 32, 0), (37, 32, 1)]:
        yield f"bwd exact {a}", lambda a=a: bw.test_exact_mode_equals_autograd(orc, *a)
    for causal in (0, 1):
        yield f"bwd quality c{causal}", lambda causal=causal: bw.test_quantised_gradients_track_exact_ones(orc, causal)
        yield f"bwd const v c{causal}", lambda causal=causal: bw.test_constant_v_gives_zero_score_gradients(orc, causal)
    yield "bwd single token", lambda: bw.test_single_token(orc)
    yield "bwd v offset", lambda: bw.test_v_offset_does_not_change_the_8bit_gradients(orc)
    yield "bwd dout scaling", lambda: bw.test_power_of_two_scaling_of_dout(orc)


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


def test_battery_passes_on_real_oracle():
    orc = Oracle()
    for name, fn in _battery(orc):
        fn()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, mutant_dir):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation site not found: {old}"
    mut_src = os.path.join(mutant_dir, f"m_{abs(hash(name))}.c")
    with open(mut_src, "w") as f:
        f.write(src.replace(old, new))
    so = mut_src[:-2] + ".so"
    subprocess.check_call(["gcc", *oracle_pkg.CFLAGS, mut_src, "-o", so, "-lm"])
    orc = Oracle(so)
    caught = []
    for pin, fn in _battery(orc):
        try:
            fn()
        except (AssertionError, ValueError, FloatingPointError):
            caught.append(pin)
            break
    assert caught, f"no pin caught mutant '{name}'"
