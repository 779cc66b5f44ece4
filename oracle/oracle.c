/*
 * oracle.c -- plain, slow CPU oracle of the SageAttention 8-bit attention forward.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
 * cpu_baseline leg of bench.py may load or call this library.  The GPU product
 * path never links, imports or calls it, and shares no code with it.
 *
 * Sources (titles of the pages this follows):
 *  [SA-sum]  "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
 *            Acceleration" (research summary page): sections "Summary",
 *            "Key points", "Interesting ideas" I1-I5.
 *  [SA2]     "SageAttention2: Efficient Attention with Thorough Outlier Smoothing
 *            and Per-thread INT4 Quantization" (ICML 2025 abstract), and the
 *            arXiv 2411.10958 abstract of SageAttention2.
 *  [SA2-v]   the arXiv 2502.01776 abstract of SageAttention2 ("smooth Q and V").
 *  [SA2-g]   the same abstracts on the granularity of the Q/K scales: "thread-level"
 *            (ICML 2025, arXiv 2411.10958) and "warp-level" (arXiv 2502.01776); the
 *            [SA-sum] "Key points" speak of per-token quantisation.
 *  [SA3]     the SageAttention3 abstract (author page, "NeurIPS Conference 2025"): FP4 attention on matrix
 *            units with microscaling.  The pages give no block format; variant 2 reads
 *            it as OCP MXFP4 (Microscaling Formats v1.0): E2M1 elements, one E8M0
 *            scale per 32 consecutive values.
 *  [FA]      FlashAttention / FlashAttention-2 and "Online normalizer calculation
 *            for softmax", entries of the reference list on the [SA-sum] page.
 *
 * What it computes, per (batch b, head h), in the order of the method:
 *   1. k_mean[c] = mean over the N tokens of K[:, c]          ([SA-sum] I1)
 *   2. K' = K - k_mean (fp32); Q' = Q - q_mean(block) when Q smoothing is on ([SA2])
 *   3. symmetric INT8 quantisation of Q', K' with one fp32 scale per group of rows:
 *      K per block of blk_k keys; Q per group of q_group rows, which may be finer
 *      than the Q-smoothing block of blk_q rows ([SA2-g]; q_group divides blk_q,
 *      q_group = 1 is per-token)
 *   4. S = Qhat Khat^T with exact integer accumulation
 *   5. s = sm_scale * dQ * dK * S  (+ sm_scale * dK * (q_mean . Khat_j) with Q smoothing)
 *   6. causal / sequence-end mask
 *   7. online softmax over key tiles of `bkv` keys in ascending order ([FA])
 *   8. P~ V: P~ rounded to fp16 (variant 0) or P~*448 to FP8 E4M3 with V in
 *      per-channel-scaled FP8 and a fresh accumulator per tile (variant 1, [SA2]
 *      "two-level accumulation"); with V smoothing ([SA2-v]) the FP8 V is of
 *      V' = V - v_mean (token mean per channel)
 *   9. O / l (variant 1 also * dV / 448, plus v_mean with V smoothing: the rows
 *      of P~ / l sum to one, so the mean comes back out unchanged)
 * The backward (oracle_attn_bwd, [SA3]: 8-bit attention for the backward too) returns
 * dQ, dK, dV of the variant-0 forward in FlashAttention-2's order, with dP = dO V^T in
 * INT8 (per-token scales, V smoothed) and the products with P and dS on fp16 operands;
 * its readings are listed where it is defined.
 * Variant 2 ([SA3]) replaces steps 3-5: Q and K' are quantised per token to MXFP4
 * (blocks of 32 channels), S = sum over blocks of 2^(eq + ek) * (E2M1 dot product),
 * s = sm_scale * S (no Q smoothing); steps 6-9 are those of variant 1.
 * Variant 3 ([SA3]: FP4 attention) takes variant 2's scores and also runs P~ V in MXFP4:
 * P~ per row in blocks of 32 keys (p_block_fp4) and V per channel in blocks of 32 tokens
 * (quant_v_head_mx); attn_row_fp4 states the fp32 sequence that decides the P~ codes.
 *
 * Readings where the pages are silent (each also listed in the design notes):
 *  - means are exact: fp16 inputs are integer multiples of 2^-24, so the token
 *    sum is an exact int64; the mean is (float)((double)sum / (N * 2^24)).
 *  - scale = absmax / 127 (fp32), codes = rint(x' * (127 / absmax)) clamped to
 *    [-127, 127] (round half to even); an all-zero block gets scale 0 and codes 0.
 *  - sm_scale is applied at dequantisation, never folded into Q before quantising.
 *  - the Q-smoothing term is dK_j * (q_mean . Khat_j), i.e. it uses the
 *    dequantised smoothed K.
 *  - l sums the unrounded P~ (fp64 here).
 *  - P~ in FP8 uses the static scale 448 (P~ <= 1 after max subtraction).
 *  - V in FP8: per channel, scale = absmax_t |V[t, c]| / 448, codes =
 *    E4M3FN(V * (448 / absmax)) rounded to nearest even after clamping to +-448.
 *  - V smoothing (variant 1, optional): v_mean is the exact token mean like
 *    k_mean, V' = V - v_mean in fp32, and V' takes V's place in the rule above.
 *
 * Floating-point decisions that produce integer codes (int8 Q/K codes, fp8 V
 * codes) are taken in fp32, the precision the GPU kernels use.  Everything else
 * (scores, exponentials, sums, O) is fp64.
 *
 * Build: gcc -O2 -ffp-contract=off -std=c11 -fPIC -shared -pthread (no fast-math).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <unistd.h>

/* ------------------------------------------------------------------------ */
/* Number formats                                                           */
/* ------------------------------------------------------------------------ */

/* IEEE binary16 -> double (exact). */
double oracle_f16_decode(uint16_t h) {
  int s = h >> 15, e = (h >> 10) & 31, m = h & 1023;
  double v;
  if (e == 0)
    v = ldexp((double)m, -24);
  else if (e == 31)
    v = m ? NAN : INFINITY;
  else
    v = ldexp((double)(1024 + m), e - 25);
  return s ? -v : v;
}

/* double -> IEEE binary16, round to nearest, ties to even. */
uint16_t oracle_f16_encode(double x) {
  uint16_t s = signbit(x) ? 0x8000 : 0;
  if (isnan(x)) return (uint16_t)(s | 0x7e00);
  double a = fabs(x);
  if (a >= 65520.0) return (uint16_t)(s | 0x7c00); /* rounds to infinity */
  if (a < 0x1.0p-14) {                              /* subnormal range, quantum 2^-24 */
    double q = nearbyint(ldexp(a, 24));             /* 0..1024; 1024 encodes 2^-14 */
    return (uint16_t)(s | (uint16_t)q);
  }
  int e;
  frexp(a, &e);                                     /* a in [2^(e-1), 2^e) */
  int E = e - 1;
  double q = nearbyint(ldexp(a, 10 - E));           /* 1024..2048 */
  if (q == 2048.0) { q = 1024.0; E += 1; }
  if (E > 15) return (uint16_t)(s | 0x7c00);
  return (uint16_t)(s | ((E + 15) << 10) | ((int)q - 1024));
}

/* OCP FP8 E4M3FN: bias 7, no infinities, S.1111.111 is NaN, max 448. */
double oracle_e4m3_decode(uint8_t c) {
  int s = c >> 7, e = (c >> 3) & 15, m = c & 7;
  if (e == 15 && m == 7) return NAN;
  double v = (e == 0) ? ldexp((double)m, -9) : ldexp((double)(8 + m), e - 10);
  return s ? -v : v;
}

/* double -> E4M3FN, round to nearest even, saturating at +-448, sign of zero kept. */
uint8_t oracle_e4m3_encode(double x) {
  uint8_t s = signbit(x) ? 0x80 : 0;
  if (isnan(x)) return (uint8_t)(s | 0x7f);
  double a = fabs(x);
  if (a >= 448.0) return (uint8_t)(s | 0x7e);
  if (a < 0x1.0p-6) {                 /* subnormals: quantum 2^-9 */
    double q = nearbyint(ldexp(a, 9)); /* 0..8; 8 encodes 2^-6 */
    return (uint8_t)(s | (uint8_t)q);
  }
  int e;
  frexp(a, &e);
  int E = e - 1;                      /* a in [2^E, 2^(E+1)), -6 <= E <= 8 */
  double q = nearbyint(ldexp(a, 3 - E)); /* 8..16 */
  if (q == 16.0) { q = 8.0; E += 1; }
  /* a < 448 keeps the result at or below 448 = code 0x7e */
  return (uint8_t)(s | ((E + 7) << 3) | ((int)q - 8));
}

/* OCP FP4 E2M1 (the MX element format): sign, 2 exponent bits (bias 1), 1 mantissa
 * bit; exponent 0 is subnormal (m * 0.5).  Magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6. */
double oracle_e2m1_decode(uint8_t c) {
  int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
  double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
  return s ? -v : v;
}

/* double -> E2M1: the nearest of the eight magnitudes, a tie going to the even code,
 * saturating at 6; the sign is kept (also of zero). */
uint8_t oracle_e2m1_encode(double x) {
  uint8_t s = signbit(x) ? 8 : 0;
  double a = fabs(x);
  if (a >= 6.0) return (uint8_t)(s | 7); /* saturate (distances to huge values all round alike) */
  int best = 0;
  for (int c = 1; c < 8; ++c) {
    double dc = fabs(oracle_e2m1_decode((uint8_t)c) - a), db = fabs(oracle_e2m1_decode((uint8_t)best) - a);
    if (dc < db || (dc == db && (c & 1) == 0)) best = c;
  }
  return (uint8_t)(s | best);
}

/* One MX block of n values (MXFP4): shared exponent E = floor(log2(max |x|)) - 2 (2 is
 * the largest exponent of E2M1), E8M0 code E + 127 clamped to [0, 254], elements
 * E2M1(x / 2^(code - 127)).  An all-zero block gets code 0 and zero elements.
 * Returns the E8M0 code. */
static uint8_t mx_block(const float* x, int n, uint8_t* codes) {
  float a = 0.0f;
  for (int i = 0; i < n; ++i) a = fmaxf(a, fabsf(x[i]));
  int code = 0;
  if (a > 0.0f) {
    int e;
    frexp((double)a, &e); /* a in [2^(e-1), 2^e) */
    code = (e - 1) - 2 + 127;
    if (code < 0) code = 0;
    if (code > 254) code = 254;
  }
  for (int i = 0; i < n; ++i) codes[i] = oracle_e2m1_encode(ldexp((double)x[i], 127 - code));
  return (uint8_t)code;
}

/* MXFP4 of one block of n attention weights P~ (variant 3; P~ in [0, 1]).  The pages give
 * no format for P~.  The block is read as MXFP4 with the smallest shared exponent that
 * holds the block's largest weight a without saturating, E = ceil(log2(a / 6)), instead
 * of the OCP rule's floor(log2 a) - 2 (which maps a to [4, 8) and clips [6, 8) to 6):
 *   E8M0 code = E + 127, clamped to [0, 254] (0 for an all-zero block); with
 *   a = f * 2^e, f in [1, 2): E = e - 2, or e - 1 when f > 1.5;
 *   elements E2M1(P~ / 2^(code - 127)), nearest even (the largest lies in (3, 6]).
 * So a weight just below a power of two (1 - 2^-24, say) keeps its value up to the
 * element grid, where the OCP rule would clip it to 6/8 of itself.
 * Returns the E8M0 code. */
static uint8_t p_block_fp4(const float* p, int n, uint8_t* codes) {
  float a = 0.0f;
  for (int i = 0; i < n; ++i) a = fmaxf(a, p[i]);
  int code = 0;
  if (a > 0.0f) {
    int e;
    const double f = 2.0 * frexp((double)a, &e); /* a = f * 2^(e-1), f in [1, 2) */
    code = (e - 1) - 2 + (f > 1.5 ? 1 : 0) + 127;
    if (code < 0) code = 0;
    if (code > 254) code = 254;
  }
  for (int i = 0; i < n; ++i) codes[i] = oracle_e2m1_encode(ldexp((double)p[i], 127 - code));
  return (uint8_t)code;
}

/* ------------------------------------------------------------------------ */
/* Step 1-3: means, smoothing, per-block INT8 quantisation                  */
/* ------------------------------------------------------------------------ */

/* Exact mean over rows [r0, r1) of channel c of one head x[N][d] (fp16 bits).
 * Every fp16 value times 2^24 is an integer, so the int64 sum is exact and
 * independent of order; one rounding to double, one to float. */
static float exact_mean(const uint16_t* x, int d, int r0, int r1, int c) {
  int64_t acc = 0;
  for (int t = r0; t < r1; ++t) acc += (int64_t)ldexp(oracle_f16_decode(x[(size_t)t * d + c]), 24);
  return (float)((double)acc / ((double)(r1 - r0) * 16777216.0));
}

/* Symmetric INT8 quantisation of one block of n fp32 values (the values are
 * already smoothed).  Returns the scale; writes codes. */
static float quant_block_i8(const float* xs, size_t n, int8_t* out) {
  float a = 0.0f;
  for (size_t i = 0; i < n; ++i) a = fmaxf(a, fabsf(xs[i]));
  if (a == 0.0f) {
    memset(out, 0, n);
    return 0.0f;
  }
  float r = 127.0f / a;
  for (size_t i = 0; i < n; ++i) {
    float t = rintf(xs[i] * r);
    if (t > 127.0f) t = 127.0f;
    if (t < -127.0f) t = -127.0f;
    out[i] = (int8_t)t;
  }
  return a / 127.0f;
}

/* Quantise one head's [N][d] tensor.
 *  mean_mode 0: no smoothing; 1: subtract the mean over all N tokens
 *  (k_mean[d] written); 2: subtract the mean of each block of `blk` rows
 *  (blk_mean[nblk][d] written).  The smoothed rows are then quantised with one
 *  scale per group of `grp` rows (grp divides blk): scale[ceil(N / grp)].
 *  out is [Np][d] with rows >= N zero. */
static void quant_head(const uint16_t* x, int N, int Np, int d, int blk, int grp, int mean_mode,
                       int8_t* out, float* scale, float* k_mean, float* blk_mean) {
  int nblk = (N + blk - 1) / blk, ngrp = (N + grp - 1) / grp;
  float* mean = (float*)malloc(sizeof(float) * (size_t)d);
  float* buf = (float*)malloc(sizeof(float) * (size_t)N * d); /* the smoothed tensor */
  if (mean_mode == 1) {
    for (int c = 0; c < d; ++c) mean[c] = exact_mean(x, d, 0, N, c);
    if (k_mean) memcpy(k_mean, mean, sizeof(float) * (size_t)d);
  }
  for (int b = 0; b < nblk; ++b) {
    int r0 = b * blk, r1 = r0 + blk < N ? r0 + blk : N;
    if (mean_mode == 2) {
      for (int c = 0; c < d; ++c) mean[c] = exact_mean(x, d, r0, r1, c);
      if (blk_mean) memcpy(blk_mean + (size_t)b * d, mean, sizeof(float) * (size_t)d);
    }
    for (int t = r0; t < r1; ++t)
      for (int c = 0; c < d; ++c) {
        float v = (float)oracle_f16_decode(x[(size_t)t * d + c]);
        buf[(size_t)t * d + c] = mean_mode ? v - mean[c] : v;
      }
  }
  for (int gi = 0; gi < ngrp; ++gi) {
    int r0 = gi * grp, r1 = r0 + grp < N ? r0 + grp : N;
    scale[gi] = quant_block_i8(buf + (size_t)r0 * d, (size_t)(r1 - r0) * d, out + (size_t)r0 * d);
  }
  memset(out + (size_t)N * d, 0, (size_t)(Np - N) * d);
  free(mean);
  free(buf);
}

/* Variant 2: one head's [N][d] tensor to MXFP4 per token (d / 32 blocks of 32
 * channels), after subtracting the token mean when mean_mode == 1 (k_mean[d]
 * written).  codes [Np][d] (one E2M1 code per byte), e8 [Np][d/32]; rows >= N zero. */
static void quant_head_mx(const uint16_t* x, int N, int Np, int d, int mean_mode, uint8_t* codes, uint8_t* e8,
                          float* k_mean) {
  float* mean = (float*)calloc((size_t)d, sizeof(float));
  float* row = (float*)malloc(sizeof(float) * (size_t)d);
  if (mean_mode == 1) {
    for (int c = 0; c < d; ++c) mean[c] = exact_mean(x, d, 0, N, c);
    if (k_mean) memcpy(k_mean, mean, sizeof(float) * (size_t)d);
  }
  for (int t = 0; t < N; ++t) {
    for (int c = 0; c < d; ++c) {
      float v = (float)oracle_f16_decode(x[(size_t)t * d + c]);
      row[c] = mean_mode ? v - mean[c] : v;
    }
    for (int b = 0; b < d / 32; ++b)
      e8[(size_t)t * (d / 32) + b] = mx_block(row + 32 * b, 32, codes + (size_t)t * d + 32 * b);
  }
  memset(codes + (size_t)N * d, 0, (size_t)(Np - N) * d);
  memset(e8 + (size_t)N * (d / 32), 0, (size_t)(Np - N) * (d / 32));
  free(mean);
  free(row);
}

/* V in FP8 for one head: per-channel scale absmax / 448, codes transposed to
 * vt[d][Np] (columns >= N zero).  With smooth_v, each channel first loses its
 * exact token mean (written to vmean[d]); otherwise vmean (when non-NULL) is 0. */
static void quant_v_head(const uint16_t* v, int N, int Np, int d, int smooth_v, uint8_t* vt, float* vscale,
                         float* vmean) {
  for (int c = 0; c < d; ++c) {
    const float mean = smooth_v ? exact_mean(v, d, 0, N, c) : 0.0f;
    if (vmean) vmean[c] = mean;
    float a = 0.0f;
    for (int t = 0; t < N; ++t) {
      float x = (float)oracle_f16_decode(v[(size_t)t * d + c]);
      if (smooth_v) x = x - mean;
      a = fmaxf(a, fabsf(x));
    }
    uint8_t* row = vt + (size_t)c * Np;
    memset(row, 0, (size_t)Np);
    if (a == 0.0f) {
      vscale[c] = 0.0f;
      continue;
    }
    float r = 448.0f / a;
    for (int t = 0; t < N; ++t) {
      float x = (float)oracle_f16_decode(v[(size_t)t * d + c]);
      if (smooth_v) x = x - mean;
      float y = x * r;
      if (y > 448.0f) y = 448.0f;
      if (y < -448.0f) y = -448.0f;
      row[t] = oracle_e4m3_encode((double)y);
    }
    vscale[c] = a / 448.0f;
  }
}

/* V in MXFP4 for one head (variant 3): per channel, blocks of 32 consecutive tokens
 * (the contraction dimension of P~ V), the OCP rule of mx_block; tokens >= N are zeros.
 * codes vt[d][Np] (one E2M1 code per byte), e8 [d][Np/32].  With smooth_v each channel
 * first loses its exact token mean (vmean[d]; zeros otherwise). */
static void quant_v_head_mx(const uint16_t* v, int N, int Np, int d, int smooth_v, uint8_t* vt, uint8_t* e8,
                            float* vmean) {
  float x[32];
  for (int c = 0; c < d; ++c) {
    const float mean = smooth_v ? exact_mean(v, d, 0, N, c) : 0.0f;
    if (vmean) vmean[c] = mean;
    for (int b = 0; b < Np / 32; ++b) {
      for (int u = 0; u < 32; ++u) {
        const int t = 32 * b + u;
        if (t < N) {
          const float y = (float)oracle_f16_decode(v[(size_t)t * d + c]);
          x[u] = smooth_v ? y - mean : y;
        } else {
          x[u] = 0.0f;
        }
      }
      e8[(size_t)c * (Np / 32) + b] = mx_block(x, 32, vt + (size_t)c * Np + 32 * b);
    }
  }
}

/* ------------------------------------------------------------------------ */
/* Parameters and per-head preparation                                      */
/* ------------------------------------------------------------------------ */

typedef struct {
  int B, H, N, d, causal, variant;
  int blk_q, blk_k, bkv;
  int q_group;    /* rows per Q scale; divides blk_q */
  int smooth_k, smooth_q, smooth_v;
  int exact;      /* 1: no quantisation at all, fp64 everywhere (pins the online softmax) */
  double sm_scale;
} params_t;

int oracle_pad_len(int N) { return (N + 127) / 128 * 128; }

typedef struct {
  int8_t *qi, *ki;   /* [Np][d] */
  float *qs, *ks;    /* per Q group, per K block */
  float *kmean;      /* [d] */
  float *qmean;      /* [nqb][d] (only with smooth_q) */
  uint8_t* vt;       /* [d][Np] (variant 1) */
  float* vs;         /* [d] (variant 1) */
  float* vm;         /* [d] (variant 1): v_mean, zeros without V smoothing */
  uint8_t *qc, *kc;  /* [Np][d] E2M1 codes (variant 2) */
  uint8_t *qe, *ke;  /* [Np][d/32] E8M0 block scales (variants 2, 3) */
  uint8_t* ve;       /* [d][Np/32] E8M0 scales of V (variant 3; vt holds E2M1 codes then) */
} prep_t;

static void prep_head(const params_t* P, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                      prep_t* h) {
  int N = P->N, d = P->d, Np = oracle_pad_len(N);
  int nqb = (N + P->blk_q - 1) / P->blk_q, nkb = (N + P->blk_k - 1) / P->blk_k;
  int nqg = (N + P->q_group - 1) / P->q_group;
  memset(h, 0, sizeof(*h));
  if (P->exact) return;
  if (P->variant >= 2) {
    h->qc = (uint8_t*)malloc((size_t)Np * d);
    h->kc = (uint8_t*)malloc((size_t)Np * d);
    h->qe = (uint8_t*)malloc((size_t)Np * (d / 32));
    h->ke = (uint8_t*)malloc((size_t)Np * (d / 32));
    h->kmean = (float*)calloc((size_t)d, sizeof(float));
    quant_head_mx(k, N, Np, d, P->smooth_k ? 1 : 0, h->kc, h->ke, h->kmean);
    quant_head_mx(q, N, Np, d, 0, h->qc, h->qe, NULL);
  } else {
    h->qi = (int8_t*)malloc((size_t)Np * d);
    h->ki = (int8_t*)malloc((size_t)Np * d);
    h->qs = (float*)malloc(sizeof(float) * (size_t)nqg);
    h->ks = (float*)malloc(sizeof(float) * (size_t)nkb);
    h->kmean = (float*)calloc((size_t)d, sizeof(float));
    h->qmean = (float*)calloc((size_t)nqb * d, sizeof(float));
    quant_head(k, N, Np, d, P->blk_k, P->blk_k, P->smooth_k ? 1 : 0, h->ki, h->ks, h->kmean, NULL);
    quant_head(q, N, Np, d, P->blk_q, P->q_group, P->smooth_q ? 2 : 0, h->qi, h->qs, NULL, h->qmean);
  }
  if (P->variant == 1 || P->variant == 2) {
    h->vt = (uint8_t*)malloc((size_t)d * Np);
    h->vs = (float*)malloc(sizeof(float) * (size_t)d);
    h->vm = (float*)malloc(sizeof(float) * (size_t)d);
    quant_v_head(v, N, Np, d, P->smooth_v, h->vt, h->vs, h->vm);
  } else if (P->variant == 3) {
    h->vt = (uint8_t*)malloc((size_t)d * Np);
    h->ve = (uint8_t*)malloc((size_t)d * (Np / 32));
    h->vm = (float*)malloc(sizeof(float) * (size_t)d);
    quant_v_head_mx(v, N, Np, d, P->smooth_v, h->vt, h->ve, h->vm);
  }
}

static void free_prep(prep_t* h) {
  free(h->qi); free(h->ki); free(h->qs); free(h->ks); free(h->kmean); free(h->qmean);
  free(h->vt); free(h->vs); free(h->vm);
  free(h->qc); free(h->kc); free(h->qe); free(h->ke); free(h->ve);
}

/* ------------------------------------------------------------------------ */
/* Steps 4-9 for one query row                                               */
/* ------------------------------------------------------------------------ */

/* Exact integer dot product of two int8 rows. */
static int32_t dot_i8(const int8_t* a, const int8_t* b, int d) {
  int32_t s = 0;
  for (int c = 0; c < d; ++c) s += (int32_t)a[c] * (int32_t)b[c];
  return s;
}

/* ------------------------------------------------------------------------ */
/* Variants 1 and 2: P~ in FP8, decided in fp32                              */
/* ------------------------------------------------------------------------ */

/* log2(448) rounded to fp32: P~ * 448 = 2^(x - m + log2 448). */
static const float kLog2_448f = 8.807354922057604f;

/* The Q-smoothing term of key j for a Q block with mean qm[d] ([SA2]: the term q_mean . K_j
 * added back to the scores).  It enters the fp32 decision of P~'s FP8 code, so it is
 * formed as a reproducible fp32 number:
 *   qm in fixed point with 28 bits under the block's largest |qm| < 2^e (e >= -100):
 *   Qbar_c = rint(qm_c * 2^(27 - e));
 *   B_j = sum_c Qbar_c * Khat_jc, an exact integer; b = B_j rounded once to fp32;
 *   term = ((kscale * dK_j) * 2^(e - 27)) * b in fp32.
 * Qbar is the mean itself up to 2^-28 of the block's largest |qm|. */
typedef struct {
  int64_t qbar[256];
  float s3; /* 2^(e - 27) */
} qmfix_t;

static void qmean_fixed(const float* qm, int d, qmfix_t* f) {
  float am = 0.0f;
  for (int c = 0; c < d; ++c) am = fmaxf(am, fabsf(qm[c]));
  int e = 0;
  frexpf(am, &e); /* am in [2^(e-1), 2^e); e = 0 for am = 0 */
  if (e < -100) e = -100;
  for (int c = 0; c < d; ++c) f->qbar[c] = (int64_t)rintf(ldexpf(qm[c], 27 - e));
  f->s3 = ldexpf(1.0f, e - 27);
}

static float qsmooth_term(const qmfix_t* f, const int8_t* khat, int d, float kscale, float dk) {
  int64_t B = 0;
  for (int c = 0; c < d; ++c) B += f->qbar[c] * (int64_t)khat[c];
  const float b = (float)(double)B;
  const float w = kscale * dk;
  const float w3 = w * f->s3;
  return w3 * b;
}

/* MXFP4 score of query i and key j (variants 2 and 3): per 32-channel block the exact
 * E2M1 dot product times both block scales, summed exactly (fp64 holds every partial
 * sum), then rounded once to fp32. */
static float mx_score(const prep_t* h, int d, int i, int j) {
  const int nb = d / 32;
  double acc = 0.0;
  for (int b = 0; b < nb; ++b) {
    double blk = 0.0;
    for (int cc = 32 * b; cc < 32 * b + 32; ++cc)
      blk += oracle_e2m1_decode(h->qc[(size_t)i * d + cc]) * oracle_e2m1_decode(h->kc[(size_t)j * d + cc]);
    acc += ldexp(blk, (int)h->qe[(size_t)i * nb + b] + (int)h->ke[(size_t)j * nb + b] - 254);
  }
  return (float)acc;
}

/* O row i of one head for variants 1 and 2 (fp64, before the final fp16 rounding).
 *
 * The FP8 code of P~ * 448 is an integer that floating point decides, so it is decided
 * in the precision the GPU kernels use, fp32, by this sequence of correctly rounded fp32
 * operations (fmaf: one rounding):
 *   kscale = sm_scale * log2(e)              (sm_scale as the fp32 number the C ABI takes)
 *   variant 1: c_j = (dQ_i * kscale) * dK_j, S_ij the exact int32 product;
 *              with Q smoothing t_j = fmaf(S_ij, c_j, term_j), else t_j = c_j * S_ij
 *   variant 2: c_j = kscale, S_ij the exact MX score rounded to fp32, t_j = c_j * S_ij
 *   m = running max of t over the visible keys of the tiles so far (base-2 units)
 *   shift = log2(448) - m
 *   z_j = t_j + shift with Q smoothing, else fmaf(S_ij, c_j, shift)
 *   P~_j * 448 = 2^(z_j) rounded to fp32;  code_j = E4M3(P~_j * 448), nearest even.
 * The rest is fp64: alpha = 2^(m_old - m_new), l sums P~ (the unrounded fp32 value, R-11),
 * O = alpha * O + sum_j code_j * Vhat_j per tile (two-level: a fresh sum per tile), and
 * the epilogue O * dV / (448 l) (+ v_mean). */
static void attn_row_fp8(const params_t* P, const prep_t* h, int i, double* o, double* work) {
  const int N = P->N, d = P->d, bkv = P->bkv, Np = oracle_pad_len(N);
  float* t = (float*)work;          /* t_j of the tile (fp32) */
  double* p = work + bkv;           /* P~ * 448 of the tile, then its FP8 value */
  double* inner = work + 2 * bkv;   /* the per-tile accumulator, d entries */
  const float kscale = (float)P->sm_scale * 1.4426950408889634f;
  const int qb = i / P->blk_q;
  const int with_term = P->variant == 1 && P->smooth_q;
  static __thread qmfix_t qf;
  if (with_term) qmean_fixed(h->qmean + (size_t)qb * d, d, &qf);
  float m = -INFINITY;
  double l = 0.0;
  for (int c = 0; c < d; ++c) o[c] = 0.0;

  for (int j0 = 0; j0 < N; j0 += bkv) {
    if (P->causal && j0 > i) break; /* every key of this and later tiles is masked */
    int j1 = j0 + bkv < N ? j0 + bkv : N;
    if (P->causal && j1 > i + 1) j1 = i + 1; /* keys > i are masked: left out of the tile */
    float tmax = -INFINITY;
    float Sf[256], cj[256];
    for (int j = j0; j < j1; ++j) {
      float S, c;
      if (P->variant == 2) {
        S = mx_score(h, d, i, j);
        c = kscale;
      } else {
        S = (float)dot_i8(h->qi + (size_t)i * d, h->ki + (size_t)j * d, d);
        const float dk = h->ks[j / P->blk_k];
        c = (h->qs[i / P->q_group] * kscale) * dk;
      }
      Sf[j - j0] = S;
      cj[j - j0] = c;
      if (with_term) {
        const float term = qsmooth_term(&qf, h->ki + (size_t)j * d, d, kscale, h->ks[j / P->blk_k]);
        t[j - j0] = fmaf(S, c, term);
      } else {
        t[j - j0] = c * S;
      }
      if (t[j - j0] > tmax) tmax = t[j - j0];
    }
    /* key 0 is visible to every row, so tmax is finite and m is finite after tile 0 */
    const float mnew = tmax > m ? tmax : m;
    const double alpha = exp2((double)m - (double)mnew); /* m = -inf gives 0 */
    const float shift = kLog2_448f - mnew;
    double psum = 0.0;
    for (int j = j0; j < j1; ++j) {
      const float z = with_term ? t[j - j0] + shift : fmaf(Sf[j - j0], cj[j - j0], shift);
      const float p448 = (float)exp2((double)z);
      psum += (double)p448 / 448.0;
      p[j - j0] = oracle_e4m3_decode(oracle_e4m3_encode((double)p448));
    }
    l = alpha * l + psum;
    for (int c = 0; c < d; ++c) {
      double acc = 0.0;
      const uint8_t* vrow = h->vt + (size_t)c * Np;
      for (int j = j0; j < j1; ++j) acc += p[j - j0] * oracle_e4m3_decode(vrow[j]);
      inner[c] = acc;
    }
    for (int c = 0; c < d; ++c) o[c] = alpha * o[c] + inner[c];
    m = mnew;
  }
  for (int c = 0; c < d; ++c) o[c] = o[c] * (double)h->vs[c] / (448.0 * l) + (double)h->vm[c];
}

/* O row i of one head for variant 3 (fp64, before the final fp16 rounding): the scores
 * of variant 2, and P~ V with both operands in MXFP4 ([SA3]: FP4 attention).
 *
 * P~ is decided in fp32 like the FP8 codes of variants 1 and 2, with the shift of P~
 * itself (no 448):
 *   c = kscale = sm_scale * log2(e);  t_j = c * S_ij;  m = running max of t over the
 *   visible keys of the tiles so far;  z_j = fmaf(S_ij, c, -m);  P~_j = 2^(z_j) rounded
 *   to fp32 (P~ <= 1, and P~ = 1 exactly at the running max).
 * Each aligned block of 32 keys (bkv is a multiple of 32) is one MX block of the row,
 * coded by p_block_fp4 with masked keys as zeros.  V is MXFP4 per channel over blocks of
 * 32 tokens (quant_v_head_mx), so both operands of P~ V share the same key blocks.
 * fp64 from there: alpha = 2^(m_old - m_new), l sums the unrounded fp32 P~ (R-11),
 * O = alpha * O + sum_j Pdec_j * Vdec_j per tile (a fresh sum per tile), and the
 * epilogue O / l (+ v_mean). */
static void attn_row_fp4(const params_t* P, const prep_t* h, int i, double* o, double* work) {
  const int N = P->N, d = P->d, bkv = P->bkv, Np = oracle_pad_len(N);
  double* inner = work + 2 * bkv; /* the per-tile accumulator, d entries */
  const float c = (float)P->sm_scale * 1.4426950408889634f;
  float m = -INFINITY;
  double l = 0.0;
  for (int cc = 0; cc < d; ++cc) o[cc] = 0.0;
  float Sf[256], pf[256];
  uint8_t pc[256];
  double pdec[256];

  for (int j0 = 0; j0 < N; j0 += bkv) {
    if (P->causal && j0 > i) break;
    int j1 = j0 + bkv < N ? j0 + bkv : N;
    if (P->causal && j1 > i + 1) j1 = i + 1;
    float tmax = -INFINITY;
    for (int j = j0; j < j1; ++j) {
      Sf[j - j0] = mx_score(h, d, i, j);
      const float t = c * Sf[j - j0];
      if (t > tmax) tmax = t;
    }
    const float mnew = tmax > m ? tmax : m;
    const double alpha = exp2((double)m - (double)mnew);
    double wsum = 0.0;
    for (int u = 0; u < bkv; ++u) pf[u] = 0.0f; /* masked keys and keys >= N: P~ = 0 */
    for (int j = j0; j < j1; ++j) {
      pf[j - j0] = (float)exp2((double)fmaf(Sf[j - j0], c, -mnew));
      wsum += (double)pf[j - j0];
    }
    /* MX blocks of 32 keys: codes and their values */
    for (int b0 = 0; b0 < bkv; b0 += 32) {
      const uint8_t e = p_block_fp4(pf + b0, 32, pc + b0);
      for (int u = b0; u < b0 + 32; ++u) pdec[u] = ldexp(oracle_e2m1_decode(pc[u]), (int)e - 127);
    }
    l = alpha * l + wsum;
    for (int cc = 0; cc < d; ++cc) {
      double acc = 0.0;
      const uint8_t* vrow = h->vt + (size_t)cc * Np;
      const uint8_t* erow = h->ve + (size_t)cc * (Np / 32);
      for (int j = j0; j < j1; ++j)
        acc += pdec[j - j0] * ldexp(oracle_e2m1_decode(vrow[j]), (int)erow[j / 32] - 127);
      inner[cc] = acc;
    }
    for (int cc = 0; cc < d; ++cc) o[cc] = alpha * o[cc] + inner[cc];
    m = mnew;
  }
  for (int cc = 0; cc < d; ++cc) o[cc] = o[cc] / l + (double)h->vm[cc];
}

/* O row i of one head (fp64, before the final fp16 rounding).
 * work: 2 * bkv + d doubles of scratch. */
static void attn_row(const params_t* P, const prep_t* h, const uint16_t* q, const uint16_t* k,
                     const uint16_t* v, int i, double* o, double* work) {
  if (P->variant == 3 && !P->exact) {
    attn_row_fp4(P, h, i, o, work);
    return;
  }
  if (P->variant >= 1 && !P->exact) {
    attn_row_fp8(P, h, i, o, work);
    return;
  }
  const int N = P->N, d = P->d, bkv = P->bkv;
  double* s = work;            /* scores of the tile */
  double* p = work + bkv;      /* P~ of the tile */
  const int qb = i / P->blk_q;
  double m = -INFINITY, l = 0.0;
  for (int c = 0; c < d; ++c) o[c] = 0.0;

  /* Q-smoothing term depends on the key only (per query block). */
  const float* qm = (P->smooth_q && !P->exact) ? h->qmean + (size_t)qb * d : NULL;

  for (int j0 = 0; j0 < N; j0 += bkv) {
    if (P->causal && j0 > i) break; /* every key of this and later tiles is masked */
    int j1 = j0 + bkv < N ? j0 + bkv : N;
    double tmax = -INFINITY;
    for (int j = j0; j < j1; ++j) {
      double sj;
      if (P->causal && j > i) {
        sj = -INFINITY;
      } else if (P->exact) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
          acc += oracle_f16_decode(q[(size_t)i * d + c]) * oracle_f16_decode(k[(size_t)j * d + c]);
        sj = P->sm_scale * acc;
      } else {
        int32_t S = dot_i8(h->qi + (size_t)i * d, h->ki + (size_t)j * d, d);
        double dk = (double)h->ks[j / P->blk_k];
        sj = P->sm_scale * (double)h->qs[i / P->q_group] * dk * (double)S;
        if (qm) {
          double ds = 0.0;
          for (int c = 0; c < d; ++c) ds += (double)qm[c] * (double)h->ki[(size_t)j * d + c];
          sj += P->sm_scale * dk * ds;
        }
      }
      s[j - j0] = sj;
      if (sj > tmax) tmax = sj;
    }
    double mnew = m > tmax ? m : tmax;
    double alpha;
    if (mnew == -INFINITY) {
      alpha = 1.0;
      for (int j = j0; j < j1; ++j) p[j - j0] = 0.0;
    } else {
      alpha = exp(m - mnew); /* m = -inf gives 0 */
      for (int j = j0; j < j1; ++j) p[j - j0] = exp(s[j - j0] - mnew);
    }
    double psum = 0.0;
    for (int j = j0; j < j1; ++j) psum += p[j - j0];
    l = alpha * l + psum;

    if (P->exact) {
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = j0; j < j1; ++j) acc += p[j - j0] * oracle_f16_decode(v[(size_t)j * d + c]);
        o[c] = alpha * o[c] + acc;
      }
    } else {
      /* P~ rounded to fp16, V in fp16, wide accumulation */
      for (int j = j0; j < j1; ++j) p[j - j0] = oracle_f16_decode(oracle_f16_encode(p[j - j0]));
      for (int c = 0; c < d; ++c) {
        double acc = 0.0;
        for (int j = j0; j < j1; ++j) acc += p[j - j0] * oracle_f16_decode(v[(size_t)j * d + c]);
        o[c] = alpha * o[c] + acc;
      }
    }
    m = mnew;
  }
  for (int c = 0; c < d; ++c) o[c] = o[c] / l;
}

/* ------------------------------------------------------------------------ */
/* Threading over work items                                                */
/* ------------------------------------------------------------------------ */

typedef struct {
  const params_t* P;
  const uint16_t *q, *k, *v;
  prep_t* preps;        /* one per head slot */
  const int* head_slot; /* item -> prep index */
  const int* heads;     /* item -> b*H+h */
  const int* rows;      /* item -> row */
  int n_items;
  double* out;          /* [n_items][d] */
  int next;
  pthread_mutex_t mu;
} job_t;

static void* worker(void* arg) {
  job_t* J = (job_t*)arg;
  const params_t* P = J->P;
  size_t hs = (size_t)P->N * P->d;
  double* work = (double*)malloc(sizeof(double) * (size_t)(2 * P->bkv + P->d));
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int it = J->next;
    J->next += 16;
    pthread_mutex_unlock(&J->mu);
    if (it >= J->n_items) break;
    int end = it + 16 < J->n_items ? it + 16 : J->n_items;
    for (; it < end; ++it) {
      size_t g = (size_t)J->heads[it];
      attn_row(P, &J->preps[J->head_slot[it]], J->q + g * hs, J->k + g * hs, J->v + g * hs,
               J->rows[it], J->out + (size_t)it * P->d, work);
    }
  }
  free(work);
  return NULL;
}

typedef struct {
  const params_t* P;
  const uint16_t *q, *k, *v;
  prep_t* preps;
  const int* uheads;
  int n;
  int next;
  pthread_mutex_t mu;
} prepjob_t;

static void* prep_worker(void* arg) {
  prepjob_t* J = (prepjob_t*)arg;
  size_t hs = (size_t)J->P->N * J->P->d;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int it = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (it >= J->n) break;
    size_t g = (size_t)J->uheads[it];
    prep_head(J->P, J->q + g * hs, J->k + g * hs, J->v + g * hs, &J->preps[it]);
  }
  return NULL;
}

static int pick_threads(int want) {
  if (want > 0) return want;
  long n = sysconf(_SC_NPROCESSORS_ONLN);
  return n > 0 ? (int)n : 1;
}

static int check_params(const params_t* P) {
  if (P->B < 1 || P->H < 1 || P->N < 1 || P->d < 1) return -1;
  if (P->blk_q < 1 || P->blk_k < 1 || P->bkv < 1) return -1;
  if (P->bkv > 256 || P->d > 256) return -1; /* the row functions keep one tile and one row on the stack */
  if (P->q_group < 1 || P->blk_q % P->q_group) return -1;
  if (P->causal != 0 && P->causal != 1) return -1;
  if (P->variant < 0 || P->variant > 3) return -1;
  if (P->variant >= 2 && (P->d % 32 || P->smooth_q)) return -1; /* MX blocks of 32; no Q smoothing */
  if (P->variant == 3 && P->bkv % 32) return -1;                 /* tiles of whole P~ blocks */
  if (P->smooth_v != 0 && P->smooth_v != 1) return -1;
  if (!(P->sm_scale > 0.0) || !isfinite(P->sm_scale)) return -1;
  if ((int64_t)P->d * 127 * 127 > 2147483647LL) return -1; /* int32 bound of S */
  return 0;
}

/*
 * O for a list of (head, row) items.
 *  q, k, v: [B*H][N][d] fp16 bits.  heads[i] in [0, B*H), rows[i] in [0, N).
 *  out: [n_items][d] fp64 (before rounding to fp16).
 *  Returns 0, or -1 on bad arguments.  nthreads <= 0 uses every online core;
 *  the count actually used is written to *threads_used when non-NULL.
 */
int oracle_attn_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int H, int N,
                     int d, int causal, double sm_scale, int variant, int blk_q, int blk_k, int bkv,
                     int q_group, int smooth_k, int smooth_q, int smooth_v, int exact, const int* heads,
                     const int* rows, int n_items, double* out, int nthreads, int* threads_used) {
  params_t P = {B, H, N, d, causal, variant, blk_q, blk_k, bkv, q_group, smooth_k, smooth_q, smooth_v, exact,
                sm_scale};
  if (check_params(&P)) return -1;
  for (int i = 0; i < n_items; ++i)
    if (heads[i] < 0 || heads[i] >= B * H || rows[i] < 0 || rows[i] >= N) return -1;
  /* unique heads, in order of first appearance */
  int G = B * H;
  int* slot_of = (int*)malloc(sizeof(int) * (size_t)G);
  int* uheads = (int*)malloc(sizeof(int) * (size_t)(n_items > 0 ? n_items : 1));
  int* head_slot = (int*)malloc(sizeof(int) * (size_t)(n_items > 0 ? n_items : 1));
  for (int g = 0; g < G; ++g) slot_of[g] = -1;
  int nu = 0;
  for (int i = 0; i < n_items; ++i) {
    if (slot_of[heads[i]] < 0) { slot_of[heads[i]] = nu; uheads[nu++] = heads[i]; }
    head_slot[i] = slot_of[heads[i]];
  }
  prep_t* preps = (prep_t*)calloc((size_t)(nu > 0 ? nu : 1), sizeof(prep_t));
  int nt = pick_threads(nthreads);
  if (threads_used) *threads_used = nt;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);

  prepjob_t PJ = {&P, q, k, v, preps, uheads, nu, 0, PTHREAD_MUTEX_INITIALIZER};
  for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, prep_worker, &PJ);
  for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);

  job_t J = {&P, q, k, v, preps, head_slot, heads, rows, n_items, out, 0, PTHREAD_MUTEX_INITIALIZER};
  for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, worker, &J);
  for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);

  for (int u = 0; u < nu; ++u) free_prep(&preps[u]);
  free(preps); free(th); free(slot_of); free(uheads); free(head_slot);
  return 0;
}

/*
 * Quantised tensors of steps 1-3 (and the FP8 V of variant 1) for all heads.
 *  q_i8, k_i8: [G][Np][d];  q_scale [G][ceil(N/q_group)], k_scale [G][nkb];  k_mean [G][d];
 *  q_mean [G][nqb][d] (zeros unless smooth_q);  v_f8 [G][d][Np], v_scale [G][d],
 *  v_mean [G][d] (zeros unless smooth_v; may be NULL) (only when v_f8 != NULL).  Np = oracle_pad_len(N).  Heads run on a thread pool;
 *  each head is computed sequentially, so the result does not depend on threading.
 */
typedef struct {
  const uint16_t *q, *k, *v;
  int N, d, Np, blk_q, blk_k, q_group, smooth_k, smooth_q, smooth_v, nqb, nkb, nqg;
  int8_t *q_i8, *k_i8;
  float *q_scale, *k_scale, *k_mean, *q_mean, *v_scale, *v_mean;
  uint8_t* v_f8;
  int G, next;
  pthread_mutex_t mu;
} quantjob_t;

static void* quant_worker(void* arg) {
  quantjob_t* J = (quantjob_t*)arg;
  size_t hs = (size_t)J->N * J->d, hp = (size_t)J->Np * J->d;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int g = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (g >= J->G) break;
    int d = J->d;
    if (J->k_mean) memset(J->k_mean + (size_t)g * d, 0, sizeof(float) * (size_t)d);
    if (J->q_mean) memset(J->q_mean + (size_t)g * J->nqb * d, 0, sizeof(float) * (size_t)J->nqb * d);
    quant_head(J->k + g * hs, J->N, J->Np, d, J->blk_k, J->blk_k, J->smooth_k ? 1 : 0, J->k_i8 + g * hp,
               J->k_scale + (size_t)g * J->nkb, J->k_mean ? J->k_mean + (size_t)g * d : NULL, NULL);
    quant_head(J->q + g * hs, J->N, J->Np, d, J->blk_q, J->q_group, J->smooth_q ? 2 : 0, J->q_i8 + g * hp,
               J->q_scale + (size_t)g * J->nqg, NULL, J->q_mean ? J->q_mean + (size_t)g * J->nqb * d : NULL);
    if (J->v_f8)
      quant_v_head(J->v + g * hs, J->N, J->Np, d, J->smooth_v, J->v_f8 + g * hp, J->v_scale + (size_t)g * d,
                   J->v_mean ? J->v_mean + (size_t)g * d : NULL);
  }
  return NULL;
}

int oracle_quant(const uint16_t* q, const uint16_t* k, const uint16_t* v, int B, int H, int N, int d,
                 int blk_q, int blk_k, int q_group, int smooth_k, int smooth_q, int smooth_v, int8_t* q_i8,
                 int8_t* k_i8, float* q_scale, float* k_scale, float* k_mean, float* q_mean, uint8_t* v_f8,
                 float* v_scale, float* v_mean) {
  if (B < 1 || H < 1 || N < 1 || d < 1 || blk_q < 1 || blk_k < 1) return -1;
  if (q_group < 1 || blk_q % q_group) return -1;
  if (smooth_v != 0 && smooth_v != 1) return -1;
  quantjob_t J = {q, k, v, N, d, oracle_pad_len(N), blk_q, blk_k, q_group, smooth_k, smooth_q, smooth_v,
                  (N + blk_q - 1) / blk_q, (N + blk_k - 1) / blk_k, (N + q_group - 1) / q_group, q_i8, k_i8,
                  q_scale, k_scale,
                  k_mean, q_mean, v_scale, v_mean, v_f8, B * H, 0, PTHREAD_MUTEX_INITIALIZER};
  int nt = pick_threads(0);
  if (nt > J.G) nt = J.G;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
  for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, quant_worker, &J);
  for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
  free(th);
  return 0;
}

/*
 * S = Qhat Khat^T for one head, rows [r0, r0+nr) x keys [c0, c0+nc), exact int32.
 *  q_i8, k_i8: [Np][d] of that head.  out: [nr][nc].
 */
int oracle_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int Np, int d, int r0, int nr, int c0,
                    int nc, int32_t* out) {
  if (r0 < 0 || c0 < 0 || r0 + nr > Np || c0 + nc > Np) return -1;
  for (int i = 0; i < nr; ++i)
    for (int j = 0; j < nc; ++j)
      out[(size_t)i * nc + j] = dot_i8(q_i8 + (size_t)(r0 + i) * d, k_i8 + (size_t)(c0 + j) * d, d);
  return 0;
}

/*
 * Variant 2 tensors for all heads: q_codes, k_codes [G][Np][d] (one E2M1 code per
 * byte), q_e8, k_e8 [G][Np][d/32] E8M0, k_mean [G][d] (zeros unless smooth_k).
 */
int oracle_quant_mx(const uint16_t* q, const uint16_t* k, int B, int H, int N, int d, int smooth_k,
                    uint8_t* q_codes, uint8_t* k_codes, uint8_t* q_e8, uint8_t* k_e8, float* k_mean) {
  if (B < 1 || H < 1 || N < 1 || d < 32 || d % 32) return -1;
  const int Np = oracle_pad_len(N), G = B * H;
  const size_t hs = (size_t)N * d, hp = (size_t)Np * d, he = (size_t)Np * (d / 32);
  for (int g = 0; g < G; ++g) {
    memset(k_mean + (size_t)g * d, 0, sizeof(float) * (size_t)d);
    quant_head_mx(k + g * hs, N, Np, d, smooth_k ? 1 : 0, k_codes + g * hp, k_e8 + g * he, k_mean + (size_t)g * d);
    quant_head_mx(q + g * hs, N, Np, d, 0, q_codes + g * hp, q_e8 + g * he, NULL);
  }
  return 0;
}

/*
 * Variant 3's V for all heads: v_codes [G][d][Np] (one E2M1 code per byte),
 * v_e8 [G][d][Np/32] E8M0, v_mean [G][d] (zeros unless smooth_v).
 */
int oracle_quant_v_mx(const uint16_t* v, int B, int H, int N, int d, int smooth_v, uint8_t* v_codes,
                      uint8_t* v_e8, float* v_mean) {
  if (B < 1 || H < 1 || N < 1 || d < 1 || (smooth_v != 0 && smooth_v != 1)) return -1;
  const int Np = oracle_pad_len(N), G = B * H;
  const size_t hs = (size_t)N * d;
  for (int g = 0; g < G; ++g)
    quant_v_head_mx(v + g * hs, N, Np, d, smooth_v, v_codes + (size_t)g * d * Np,
                    v_e8 + (size_t)g * d * (Np / 32), v_mean + (size_t)g * d);
  return 0;
}

/* The MXFP4 rule of P~ (p_block_fp4) on n_blocks blocks of 32 fp32 weights. */
void oracle_p_block_fp4(const float* p, int n_blocks, uint8_t* codes, uint8_t* e8) {
  for (int b = 0; b < n_blocks; ++b) e8[b] = p_block_fp4(p + 32 * b, 32, codes + 32 * b);
}

/* Array forms of the codecs (for tests). */
/* ------------------------------------------------------------------------ */
/* Backward: dQ, dK, dV of the 8-bit forward ([SA3]: 8-bit attention for      */
/* both forward and backward propagation)                                    */
/* ------------------------------------------------------------------------ */

/*
 * The pages say only that the backward is 8-bit as well.  Readings (each also in the
 * design notes):
 *  - The backward differentiates O = softmax(s) V at the forward's scores s: the variant-0
 *    scores (smoothed K, per-block INT8 Q and K, exact int32 S, dequantised); the
 *    quantisers pass gradients straight through (dS/dQ uses Q itself, dS/dK uses K).
 *  - FlashAttention-2's backward order ([FA]): P = exp(s - L) with L the row log-sum-exp,
 *    D_i = sum_c dO_ic O_ic with O the forward output, dS = P * (dP - D).
 *  - 8-bit where SageAttention puts 8 bits, on the score-shaped product: dP = dO V^T
 *    (a dot product over the head dimension, like Q K^T) takes dO and V in INT8 with one
 *    scale per token (absmax / 127, nearest even, the forward's rule) and exact int32
 *    sums.  V is smoothed first (its exact token mean per channel is subtracted, the K
 *    rule): that shifts every dP_ij of row i by dO_i . vmean, and D_i is shifted by the
 *    same amount, so dS does not change in exact arithmetic.
 *  - dQ uses the smoothed K' = K - kmean (the forward's K smoothing, fp32, rounded to fp16
 *    as the operand): in exact arithmetic every row of dS sums to zero, so dS K' = dS K,
 *    and K' keeps a channel offset of K from multiplying the rounding of dS.
 *  - The products with P or dS (dV = P^T dO, dK = dS^T Q, dQ = dS K') keep FP16 operands
 *    and fp32 accumulation, as SageAttention keeps P~ V in FP16: P is rounded to fp16 as
 *    2^8 P, and dS as sigma dS with sigma = 2^(14 - e), where 2^e is the first power of
 *    two above B = 2 max_i |dO_i| max_j |V'_j| (Euclidean norms of the rows), which bounds
 *    |dS| (|dS_ij| <= |dP_ij - D_i| <= max_j dP_ij - min_j dP_ij): the scaled operands stay
 *    in fp16's normal range; both scales are undone after the sums.
 *  - Gradients are returned unrounded (fp64 here, fp32 on the GPU).
 * exact = 1 turns every quantisation and rounding off (fp64 throughout): the textbook
 * attention backward, which the pins compare with autograd.
 */
typedef struct {
  int B, H, N, d, causal, blk_q, blk_k, smooth_k, smooth_v, exact;
  double sm_scale;
} bwdparams_t;

static void bwd_head(const bwdparams_t* P, const uint16_t* q, const uint16_t* k, const uint16_t* v,
                     const uint16_t* o, const uint16_t* dout, double* dq, double* dk, double* dv) {
  const int N = P->N, d = P->d, Np = oracle_pad_len(N);
  const int nqb = (N + P->blk_q - 1) / P->blk_q, nkb = (N + P->blk_k - 1) / P->blk_k;
  int8_t *qi = NULL, *ki = NULL, *vi = NULL, *gi = NULL;
  float *qs = NULL, *ks = NULL, *vs = NULL, *gs = NULL, *vmean = NULL, *vsm = NULL, *kmean = NULL;
  double* ksm = NULL; /* K' rounded to fp16 */
  double* s = (double*)malloc(sizeof(double) * (size_t)N);
  double* pr = (double*)malloc(sizeof(double) * (size_t)N);
  double* ds = (double*)malloc(sizeof(double) * (size_t)N);
  /* the fp16 inputs as doubles (exact) */
  double* qf = (double*)malloc(sizeof(double) * (size_t)N * d);
  double* kf = (double*)malloc(sizeof(double) * (size_t)N * d);
  double* gf = (double*)malloc(sizeof(double) * (size_t)N * d);
  for (size_t e = 0; e < (size_t)N * d; ++e) {
    qf[e] = oracle_f16_decode(q[e]);
    kf[e] = oracle_f16_decode(k[e]);
    gf[e] = oracle_f16_decode(dout[e]);
    dq[e] = dk[e] = dv[e] = 0.0;
  }

  if (!P->exact) {
    /* forward's Q and K codes (variant 0: K smoothed over all tokens, Q not smoothed) */
    qi = (int8_t*)malloc((size_t)Np * d);
    ki = (int8_t*)malloc((size_t)Np * d);
    qs = (float*)malloc(sizeof(float) * (size_t)nqb);
    ks = (float*)malloc(sizeof(float) * (size_t)nkb);
    kmean = (float*)calloc((size_t)d, sizeof(float));
    quant_head(k, N, Np, d, P->blk_k, P->blk_k, P->smooth_k ? 1 : 0, ki, ks, P->smooth_k ? kmean : NULL, NULL);
    /* K' in fp16, the operand of dQ */
    ksm = (double*)malloc(sizeof(double) * (size_t)N * d);
    for (int t = 0; t < N; ++t)
      for (int c = 0; c < d; ++c) {
        const float x = (float)oracle_f16_decode(k[(size_t)t * d + c]) - kmean[c];
        ksm[(size_t)t * d + c] = oracle_f16_decode(oracle_f16_encode((double)x));
      }
    quant_head(q, N, Np, d, P->blk_q, P->blk_q, 0, qi, qs, NULL, NULL);
    /* V' = V - vmean (fp32), then V' and dO in INT8 per token */
    vmean = (float*)calloc((size_t)d, sizeof(float));
    vsm = (float*)malloc(sizeof(float) * (size_t)N * d);
    if (P->smooth_v)
      for (int c = 0; c < d; ++c) vmean[c] = exact_mean(v, d, 0, N, c);
    for (int t = 0; t < N; ++t)
      for (int c = 0; c < d; ++c) {
        const float x = (float)oracle_f16_decode(v[(size_t)t * d + c]);
        vsm[(size_t)t * d + c] = P->smooth_v ? x - vmean[c] : x;
      }
    vi = (int8_t*)malloc((size_t)N * d);
    gi = (int8_t*)malloc((size_t)N * d);
    vs = (float*)malloc(sizeof(float) * (size_t)N);
    gs = (float*)malloc(sizeof(float) * (size_t)N);
    float* row = (float*)malloc(sizeof(float) * (size_t)d);
    for (int t = 0; t < N; ++t) {
      vs[t] = quant_block_i8(vsm + (size_t)t * d, (size_t)d, vi + (size_t)t * d);
      for (int c = 0; c < d; ++c) row[c] = (float)oracle_f16_decode(dout[(size_t)t * d + c]);
      gs[t] = quant_block_i8(row, (size_t)d, gi + (size_t)t * d);
    }
    free(row);
  }

  /* the fp16 operand scales: 2^8 for P; sigma = 2^(14 - e) for dS */
  double sigma = 1.0;
  const double pscale = 256.0;
  if (!P->exact) {
    double gmax = 0.0, vmax = 0.0;
    for (int t = 0; t < N; ++t) {
      double a = 0.0, b = 0.0;
      for (int c = 0; c < d; ++c) {
        const double g = oracle_f16_decode(dout[(size_t)t * d + c]);
        const double w = (double)vsm[(size_t)t * d + c];
        a += g * g;
        b += w * w;
      }
      if (sqrt(a) > gmax) gmax = sqrt(a);
      if (sqrt(b) > vmax) vmax = sqrt(b);
    }
    const double bound = 2.0 * gmax * vmax;
    if (bound > 0.0) {
      int e;
      frexp(bound, &e); /* bound in [2^(e-1), 2^e) */
      sigma = ldexp(1.0, 14 - e);
    }
  }

  for (int i = 0; i < N; ++i) {
    const int jend = P->causal ? i + 1 : N;
    /* scores, their log-sum-exp, P */
    double m = -INFINITY;
    for (int j = 0; j < jend; ++j) {
      double sj;
      if (P->exact) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
          acc += oracle_f16_decode(q[(size_t)i * d + c]) * oracle_f16_decode(k[(size_t)j * d + c]);
        sj = P->sm_scale * acc;
      } else {
        const int32_t S = dot_i8(qi + (size_t)i * d, ki + (size_t)j * d, d);
        sj = P->sm_scale * (double)qs[i / P->blk_q] * (double)ks[j / P->blk_k] * (double)S;
      }
      s[j] = sj;
      if (sj > m) m = sj;
    }
    double lsum = 0.0;
    for (int j = 0; j < jend; ++j) lsum += exp(s[j] - m);
    const double L = m + log(lsum);
    /* D_i (with V smoothed, the same shift dO_i . vmean as every dP_ij of the row) */
    double D = 0.0;
    for (int c = 0; c < d; ++c) {
      const double g = oracle_f16_decode(dout[(size_t)i * d + c]);
      D += g * oracle_f16_decode(o[(size_t)i * d + c]);
      if (!P->exact && P->smooth_v) D -= g * (double)vmean[c];
    }
    for (int j = 0; j < jend; ++j) {
      const double p = exp(s[j] - L);
      double dp;
      if (P->exact) {
        double acc = 0.0;
        for (int c = 0; c < d; ++c)
          acc += oracle_f16_decode(dout[(size_t)i * d + c]) * oracle_f16_decode(v[(size_t)j * d + c]);
        dp = acc;
      } else {
        const int32_t S = dot_i8(gi + (size_t)i * d, vi + (size_t)j * d, d);
        dp = (double)gs[i] * (double)vs[j] * (double)S;
      }
      const double dsv = p * (dp - D);
      if (P->exact) {
        pr[j] = p;
        ds[j] = dsv;
      } else {
        pr[j] = oracle_f16_decode(oracle_f16_encode(pscale * p)) / pscale;
        ds[j] = oracle_f16_decode(oracle_f16_encode(sigma * dsv)) / sigma;
      }
    }
    /* dQ_i = sm_scale sum_j dS_ij K'_j;  dK_j += sm_scale dS_ij Q_i;  dV_j += P_ij dO_i */
    for (int j = 0; j < jend; ++j)
      for (int c = 0; c < d; ++c) {
        const double kv = P->exact ? kf[(size_t)j * d + c] : ksm[(size_t)j * d + c];
        const double qv = qf[(size_t)i * d + c];
        const double gv = gf[(size_t)i * d + c];
        dq[(size_t)i * d + c] += P->sm_scale * ds[j] * kv;
        dk[(size_t)j * d + c] += P->sm_scale * ds[j] * qv;
        dv[(size_t)j * d + c] += pr[j] * gv;
      }
  }
  free(s); free(pr); free(ds); free(qf); free(kf); free(gf);
  free(qi); free(ki); free(vi); free(gi); free(qs); free(ks); free(vs); free(gs); free(vmean); free(vsm);
  free(kmean); free(ksm);
}

typedef struct {
  const bwdparams_t* P;
  const uint16_t *q, *k, *v, *o, *dout;
  double *dq, *dk, *dv;
  int G, next;
  pthread_mutex_t mu;
} bwdjob_t;

static void* bwd_worker(void* arg) {
  bwdjob_t* J = (bwdjob_t*)arg;
  const size_t hs = (size_t)J->P->N * J->P->d;
  for (;;) {
    pthread_mutex_lock(&J->mu);
    int g = J->next++;
    pthread_mutex_unlock(&J->mu);
    if (g >= J->G) break;
    bwd_head(J->P, J->q + g * hs, J->k + g * hs, J->v + g * hs, J->o + g * hs, J->dout + g * hs, J->dq + g * hs,
             J->dk + g * hs, J->dv + g * hs);
  }
  return NULL;
}

/*
 * dQ, dK, dV ([B][H][N][d] fp64 each) of the forward at q, k, v given its output o and
 * the output gradient dout (all [B][H][N][d] fp16 bits).  Heads run on a thread pool;
 * each head is computed sequentially, so the result does not depend on threading.
 * Returns 0, or -1 on bad arguments.
 */
int oracle_attn_bwd(const uint16_t* q, const uint16_t* k, const uint16_t* v, const uint16_t* o,
                    const uint16_t* dout, int B, int H, int N, int d, int causal, double sm_scale, int blk_q,
                    int blk_k, int smooth_k, int smooth_v, int exact, double* dq, double* dk, double* dv,
                    int nthreads) {
  if (B < 1 || H < 1 || N < 1 || d < 1 || d > 256 || blk_q < 1 || blk_k < 1) return -1;
  if ((causal != 0 && causal != 1) || (smooth_k != 0 && smooth_k != 1) || (smooth_v != 0 && smooth_v != 1) ||
      (exact != 0 && exact != 1))
    return -1;
  if (!(sm_scale > 0.0) || !isfinite(sm_scale)) return -1;
  bwdparams_t P = {B, H, N, d, causal, blk_q, blk_k, smooth_k, smooth_v, exact, sm_scale};
  bwdjob_t J = {&P, q, k, v, o, dout, dq, dk, dv, B * H, 0, PTHREAD_MUTEX_INITIALIZER};
  int nt = pick_threads(nthreads);
  if (nt > J.G) nt = J.G;
  pthread_t* th = (pthread_t*)malloc(sizeof(pthread_t) * (size_t)nt);
  for (int t = 0; t < nt; ++t) pthread_create(&th[t], NULL, bwd_worker, &J);
  for (int t = 0; t < nt; ++t) pthread_join(th[t], NULL);
  free(th);
  return 0;
}

/* The Q-smoothing terms of n keys (khat [n][d]) for one Q-block mean qm[d], as the FP8
 * path forms them (qsmooth_term): out[j] in fp32. */
void oracle_qsmooth_terms(const float* qm, int d, const int8_t* khat, int n, float kscale, const float* dk,
                          float* out) {
  qmfix_t f;
  if (d < 1 || d > 256) return;
  qmean_fixed(qm, d, &f);
  for (int j = 0; j < n; ++j) out[j] = qsmooth_term(&f, khat + (size_t)j * d, d, kscale, dk[j]);
}

void oracle_e2m1_decode_n(const uint8_t* c, size_t n, double* out) {
  for (size_t i = 0; i < n; ++i) out[i] = oracle_e2m1_decode(c[i]);
}
void oracle_e2m1_encode_n(const double* x, size_t n, uint8_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = oracle_e2m1_encode(x[i]);
}
void oracle_f16_decode_n(const uint16_t* h, size_t n, double* out) {
  for (size_t i = 0; i < n; ++i) out[i] = oracle_f16_decode(h[i]);
}
void oracle_f16_encode_n(const double* x, size_t n, uint16_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = oracle_f16_encode(x[i]);
}
void oracle_e4m3_decode_n(const uint8_t* c, size_t n, double* out) {
  for (size_t i = 0; i < n; ++i) out[i] = oracle_e4m3_decode(c[i]);
}
void oracle_e4m3_encode_n(const double* x, size_t n, uint8_t* out) {
  for (size_t i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(x[i]);
}
