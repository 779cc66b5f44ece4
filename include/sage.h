/*
 * sage.h -- C ABI of the MI355X (gfx950) 8-bit attention forward.
 *
 * The operation is SageAttention's plug-and-play quantised attention forward:
 *   "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
 *    Acceleration" (research summary page, sections "Summary" and
 *    "Interesting ideas" I1, I3): K is smoothed by subtracting its mean over
 *    tokens, Q and K are quantised to INT8, Q K^T runs on 8-bit matrix units,
 *    the online (FlashAttention-style) softmax follows, P~ V stays in FP16;
 *   "SageAttention2: Efficient Attention with Thorough Outlier Smoothing and
 *    Per-thread INT4 Quantization" (abstract): Q is smoothed as well, P~ and V
 *    are quantised to FP8, and P~ V uses two-level accumulation.  Here Q/K stay
 *    INT8 in variants 0 and 1 (one fp32 scale per block of tokens, or per group
 *    of rows).  The FP8 matrix instruction accumulates in fp32; the kernel lets it
 *    add each key tile's products straight into O, which is the fp32 outer buffer of
 *    the two-level scheme (a stress input on which a 22-bit truncating or a 20-bit
 *    accumulator would miss the O tolerance pins this).  The FP8 code of P~ * 448 is
 *    decided in fp32 by a fixed sequence of operations (scores, running max, exp2),
 *    so the codes are reproducible;
 *   "SageAttention3: Microscaling FP4 Attention for Inference and An Exploration
 *    of 8-Bit Training" (abstract): FP4 attention on matrix units, taken here as
 *    variant 2 (MXFP4 Q K^T on the scaled FP4 MFMA, P~ V as variant 1) and variant 3
 *    (P~ V in MXFP4 as well, both operands in blocks of 32 keys).
 *
 * Conventions for every entry point:
 *  - All tensor pointers are DEVICE pointers, allocated and owned by the caller.
 *    The library never allocates, frees or keeps caller memory, and keeps no
 *    state between calls.
 *  - q, k, v, o are [B, H, N, d] contiguous IEEE fp16, 16-byte aligned.
 *  - d must be 64 or 128 (SAGE_ERR_UNSUPPORTED otherwise); N >= 1;
 *    B*H*pad_len(N)*d < 2^31.
 *  - Quantised Q/K tensors are [B, H, Np, d] int8 with Np = sage_pad_len(N);
 *    rows >= N are zero.  Q scales are [B, H, ceil(N / q_group)] fp32 (q_group =
 *    blk_q unless sage_params sets it), K scales [B, H, ceil(N / blk_k)] fp32.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work and returns without waiting.
 *  - Arguments are checked before anything is launched; a bad argument returns a
 *    negative status and launches nothing.  No exception crosses the ABI.
 *    sage_last_error() gives a message for the calling thread's last failure.
 *  - Calls that share a workspace must not overlap in time.
 */
#ifndef SAGE_H_
#define SAGE_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  SAGE_OK = 0,
  SAGE_ERR_INVALID_ARG = -1, /* null/misaligned pointer, bad size or flag */
  SAGE_ERR_UNSUPPORTED = -2, /* head dim other than 64/128, bad block sizes */
  SAGE_ERR_WORKSPACE = -3,   /* workspace missing or smaller than required */
  SAGE_ERR_HIP = -4          /* a HIP launch failed (message in sage_last_error) */
};

enum {
  SAGE_VARIANT_INT8QK_FP16PV = 0, /* SageAttention: INT8 Q K^T, FP16 P~ V (fp32 accumulation) */
  SAGE_VARIANT_INT8QK_FP8PV = 1,  /* SageAttention2-style: + Q smoothing, FP8 P~ and V; each key tile's
                                     P~ V products summed by the matrix unit into the fp32 O */
  SAGE_VARIANT_MXFP4QK_FP8PV = 2, /* SageAttention3-style FP4 scores: per-token MXFP4 Q and K' (OCP
                                     microscaling, blocks of 32 channels), P~ V as variant 1; no Q
                                     smoothing */
  SAGE_VARIANT_MXFP4QK_FP4PV = 3  /* SageAttention3-style FP4 attention: the scores of variant 2, and
                                     P~ V on the scaled FP4 MFMA with P~ and V in MXFP4 over blocks
                                     of 32 keys (see sage_quant_v_mx for V, sage_attn_fwd_qf16_fp4
                                     for P~) */
};

/* Optional knobs.  Pass NULL for the defaults; set struct_size = sizeof(sage_params). */
typedef struct {
  int struct_size;
  int blk_q;    /* tokens per Q scale block: 32, 64 or 128 (default 128) */
  int blk_k;    /* tokens per K scale block: 16, 32, 64 or 128 (default 64) */
  int smooth_k; /* subtract the token mean of K (default 1) */
  int smooth_q; /* subtract the block mean of Q and add its term back (default: variant == 1) */
  int smooth_v; /* variants 1-3: subtract the token mean of V before FP8 / MXFP4, add it to O
                   (SageAttention2 abstract, "smooth Q and V"; default 0) */
  int q_group;  /* rows per Q scale: 0 (= blk_q, default) or a power of two <= blk_q.
                   The SageAttention2 abstracts quantise Q and K at thread- / warp-level
                   granularity; here each lane of the attention kernel owns one query,
                   so per-token Q scales (q_group = 1) cost nothing in the kernel.  Q
                   smoothing keeps its mean per block of blk_q rows.  K's finest scale
                   block, blk_k = 16, is the 16 keys a lane holds. */
} sage_params;
/* The older layouts (struct_size 20: no smooth_v, no q_group; 24: no q_group) are
 * still accepted; the missing fields take their defaults. */

/* Library version, major * 10000 + minor * 100 + patch. */
int sage_version(void);

/* Rows of the padded int8 / fp8 tensors: N rounded up to a multiple of 128. */
int sage_pad_len(int N);

/* Keys per online-softmax tile (the tile over which the running max advances; the
 * FP8 codes of P~ in variants 1 and 2 depend on the max at each tile).  Ascending
 * tiles of this size define the exact schedule of the softmax.  Returns < 0 for bad
 * arguments. */
int sage_kv_tile(int variant, int d);

/* Bytes of device workspace sage_attn_fwd / sage_attn_fwd_ex / sage_quant_qk /
 * sage_quant_v need for this shape (0 for bad arguments).  p may be NULL. */
size_t sage_workspace_bytes(int B, int H, int N, int d, int variant, const sage_params* p);

/*
 * Smoothing and per-block INT8 quantisation of Q and K ([SA summary page]
 * "Summary", I1; Q smoothing from the SageAttention2 abstract).
 *   k_mean[B,H,d] = exact mean of K over the N tokens (fp32; exact integer sum of the
 *     fp16 values, one rounding to fp64 by the division, one to fp32);
 *   K' = K - k_mean (fp32); per block of blk_k tokens: scale = max|K'| / 127,
 *     code = rint(K' * (127 / max|K'|)) in [-127, 127] (ties to even); a block of
 *     zeros gets scale 0 and codes 0;
 *   Q: the same per group of q_group tokens (q_group divides blk_q); with smooth_q,
 *     the exact mean of each block of blk_q tokens is subtracted first and written
 *     to q_mean[B,H,ceil(N/blk_q),d].
 * q_mean may be NULL unless smooth_q is on; k_mean may be NULL.
 */
int sage_quant_qk(const void* q, const void* k, int B, int H, int N, int d, const sage_params* p,
                  int8_t* q_i8, int8_t* k_i8, float* q_scale, float* k_scale, float* k_mean,
                  float* q_mean, void* ws, size_t ws_bytes, void* stream);

/*
 * FP8 E4M3 (OCP E4M3FN: bias 7, max 448) quantisation of V with one scale per
 * channel (SageAttention2 abstract: P~ and V in FP8):
 *   v_scale[B,H,d] = max_t |V[t,c]| / 448;
 *   v_f8[B,H,d,Np] = E4M3(clamp(V[t,c] * (448 / max_t|V[t,c]|), +-448)), round to
 *   nearest even, stored transposed (keys contiguous); columns >= N are 0; a
 *   channel of zeros gets scale 0 and codes 0.
 */
int sage_quant_v(const void* v, int B, int H, int N, int d, uint8_t* v_f8, float* v_scale,
                 void* ws, size_t ws_bytes, void* stream);

/*
 * sage_quant_v with optional V smoothing (SageAttention2 abstract: Q and V are
 * smoothed).  smooth_v = 1: v_mean[B,H,d] = exact token mean of V per channel (the
 * k_mean rule of sage_quant_qk), V' = V - v_mean in fp32, and the rule above applies
 * to V' (v_scale = max|V'| / 448).  The attention output adds v_mean back: each row
 * of the normalised P~ sums to one.  v_mean (16-byte aligned) is required with
 * smooth_v and ignored without it; smooth_v = 0 is sage_quant_v.
 */
int sage_quant_v_ex(const void* v, int B, int H, int N, int d, int smooth_v, uint8_t* v_f8,
                    float* v_scale, float* v_mean, void* ws, size_t ws_bytes, void* stream);

/*
 * o = SageAttention(q, k, v): the whole plug-and-play forward (quantisation kernels
 * plus the attention kernel; the attention kernel quantises Q itself, see
 * sage_attn_fwd_qf16, sage_attn_fwd_qf16_fp8, sage_attn_fwd_qf16_mx and
 * sage_attn_fwd_qf16_fp4).  causal: key j is visible to query i iff j <= i.
 * sm_scale: softmax scale (finite, > 0; normally 1/sqrt(d)), applied when the int32
 * scores are dequantised.  variant: SAGE_VARIANT_*.  ws: device workspace of at
 * least sage_workspace_bytes(...) bytes.
 */
int sage_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                  int causal, float sm_scale, int variant, void* ws, size_t ws_bytes, void* stream);

/* sage_attn_fwd with explicit sage_params (block sizes, smoothing switches). */
int sage_attn_fwd_ex(const void* q, const void* k, const void* v, void* o, int B, int H, int N,
                     int d, int causal, float sm_scale, int variant, const sage_params* p, void* ws,
                     size_t ws_bytes, void* stream);

/*
 * sage_attn_fwd_ex for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments, same
 * kernels and the same result as sage_attn_fwd_ex with a workspace, but the workspace is
 * the library's own array of SAGE_NOALLOC_SCRATCH_BYTES (128 MiB) per GPU, which each GPU
 * the library runs on holds until the process ends.  Nothing is allocated or freed per
 * call.  Shapes whose workspace (sage_workspace_bytes) exceeds the array return
 * SAGE_ERR_WORKSPACE before any launch (e.g. B*H = 128 heads of N = 4096, d = 128, variant
 * 0 fit; B*H = 64 heads of N = 32768, d = 128, variant 1 do not).  All calls on one GPU
 * share its array: calls that overlap in time on one GPU (other streams, other host
 * threads) race and give wrong results; calls in order on one stream are safe.  The
 * array keeps the last call's contents; no pass reads workspace it has not written in
 * the same call.  The first call on a device looks the array's address up (no
 * allocation).
 */
#define SAGE_NOALLOC_SCRATCH_BYTES (128u * 1024u * 1024u)
int sage_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int d,
                          int causal, float sm_scale, int variant, const sage_params* p, void* stream);

/*
 * The attention kernel alone, on tensors sage_quant_qk / sage_quant_v(_ex) produced
 * (same p).  Variant 0 reads v (fp16); variant 1 reads v_f8 / v_scale, with
 * smooth_q q_mean, and with smooth_v v_mean (16-byte aligned, [B,H,d]).  Pointers a
 * call does not read may be NULL.  Used to time the attention kernel by itself.
 * (Library 0.2 added v_mean after v_scale.)
 */
int sage_attn_fwd_prequant(const int8_t* q_i8, const int8_t* k_i8, const float* q_scale,
                           const float* k_scale, const float* q_mean, const void* v,
                           const uint8_t* v_f8, const float* v_scale, const float* v_mean, void* o,
                           int B, int H, int N, int d, int causal, float sm_scale, int variant,
                           const sage_params* p, void* stream);

/*
 * The attention kernel that sage_attn_fwd runs for variant 1: Q is fp16 and each
 * workgroup quantises its own rows in its prologue with the rule of sage_quant_qk (same
 * codes and scales; with p->smooth_q (the default for this variant) the exact mean of each
 * Q block of blk_q rows is taken out first and its term added back to the scores); K
 * comes from sage_quant_qk (same p), V from sage_quant_v(_ex) (same smooth_v).  Used to
 * time the fused kernel by itself.
 */
int sage_attn_fwd_qf16_fp8(const void* q, const int8_t* k_i8, const float* k_scale, const uint8_t* v_f8,
                           const float* v_scale, const float* v_mean, void* o, int B, int H, int N, int d,
                           int causal, float sm_scale, const sage_params* p, void* stream);

/*
 * Per-token MXFP4 of Q and K for the MXFP4 variant (SageAttention3 abstract: FP4
 * attention; the block format is read as OCP Microscaling MXFP4):
 *   K' = K - k_mean with smooth_k (the sage_quant_qk rule for k_mean), Q unsmoothed;
 *   each token's d channels form d/32 blocks of 32; per block the E8M0 scale code
 *   s = floor(log2(max |x|)) - 2 + 127 clamped to [0, 254] (0 for an all-zero block)
 *   and E2M1 elements E2M1(x / 2^(s - 127)): round to nearest, ties to the even code,
 *   saturating at 6, sign kept.
 *   q_f4, k_f4 [B,H,Np,d/2]: two codes per byte, the lower channel in the low nibble;
 *   q_e8, k_e8 [B,H,Np,d/32]: the scale codes; rows >= N zero.
 * ws: sage_workspace_bytes(..., 2, NULL) bytes suffice (only the K sums are used).
 */
int sage_quant_qk_mx(const void* q, const void* k, int B, int H, int N, int d, int smooth_k,
                     uint8_t* q_f4, uint8_t* k_f4, uint8_t* q_e8, uint8_t* k_e8, float* k_mean,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * The MXFP4 variant's attention kernel alone, on sage_quant_qk_mx and
 * sage_quant_v(_ex) outputs: S = sum over blocks of 2^(sq + sk - 254) times the E2M1
 * dot product (fp32 matrix-unit accumulation), then the online softmax and FP8 P~ V
 * of variant 1.  v_mean is read only with p->smooth_v (16-byte aligned).
 */
int sage_attn_fwd_prequant_mx(const uint8_t* q_f4, const uint8_t* k_f4, const uint8_t* q_e8,
                              const uint8_t* k_e8, const uint8_t* v_f8, const float* v_scale,
                              const float* v_mean, void* o, int B, int H, int N, int d, int causal,
                              float sm_scale, const sage_params* p, void* stream);

/*
 * The attention kernel that sage_attn_fwd runs for the MXFP4 variant: Q is fp16 and
 * each workgroup quantises its rows to MXFP4 in its prologue (the sage_quant_qk_mx rule,
 * same codes and scales); K comes from sage_quant_qk_mx, V from sage_quant_v(_ex).
 * Used to time the fused kernel by itself.
 */
int sage_attn_fwd_qf16_mx(const void* q, const uint8_t* k_f4, const uint8_t* k_e8, const uint8_t* v_f8,
                          const float* v_scale, const float* v_mean, void* o, int B, int H, int N, int d,
                          int causal, float sm_scale, const sage_params* p, void* stream);

/*
 * The attention kernel that sage_attn_fwd runs for variant 0: Q is fp16 and each
 * workgroup quantises its own rows per group of q_group rows (default blk_q; the
 * sage_quant_qk rule above, same codes and scales, with p->smooth_q the block means
 * taken out first and their term added back); K comes pre-quantised from sage_quant_qk
 * (k_i8, k_scale, same p); v is fp16.  Used to time the fused kernel by itself, and for
 * callers that keep K quantised across calls.
 */
int sage_attn_fwd_qf16(const void* q, const int8_t* k_i8, const float* k_scale, const void* v,
                       void* o, int B, int H, int N, int d, int causal, float sm_scale,
                       const sage_params* p, void* stream);

/*
 * Training forward of the 8-bit backward (SageAttention3 abstract: 8-bit attention for
 * training; FlashAttention-2 "Backward pass": the backward recomputes P from the row
 * log-sum-exp).  sage_attn_fwd_ex with variant SAGE_VARIANT_INT8QK_FP16PV (same passes,
 * same scores and fp16 weights), except that o is divided by the row sum of the unrounded
 * weights, the sum lse is defined on, where sage_attn_fwd_ex divides by the sum of the fp16
 * weights P~ V multiplies; the two o differ in their last fp16 bits.  Additionally
 *   lse[B,H,N] fp32 (16-byte aligned, device) = ln of the row sum of exp(sm_scale * S)
 *   over the visible keys, S the dequantised INT8 scores of the smoothed K (the shift by
 *   K's mean drops out of the softmax), i.e. ln(l) + the running maximum, per row.
 * p must satisfy the backward's rules: blk_q 64 or 128, smooth_q 0, q_group 0 (one Q
 * scale per block); otherwise SAGE_ERR_UNSUPPORTED.  ws: sage_workspace_bytes(..., 0, p).
 */
int sage_attn_fwd_train(const void* q, const void* k, const void* v, void* o, float* lse, int B, int H, int N,
                        int d, int causal, float sm_scale, const sage_params* p, void* ws, size_t ws_bytes,
                        void* stream);

/* Device workspace bytes sage_attn_bwd needs for this shape (0 for bad arguments or a p
 * the backward does not support). */
size_t sage_attn_bwd_workspace_bytes(int B, int H, int N, int d, const sage_params* p);

/*
 * 8-bit attention backward (SageAttention3 abstract: 8-bit attention for training; the
 * gradient order of FlashAttention-2 "Backward pass"), differentiating the variant-0
 * forward of the same q, k, v, causal, sm_scale and p:
 *   q, k, v, o, dout: fp16 [B,H,N,d]; lse: sage_attn_fwd_train's output for o;
 *   dq, dk, dv: fp32 [B,H,N,d] (device, 16-byte aligned), fully overwritten.
 * The quantisers are straight-through: dQ, dK, dV are the gradients of attention with
 * the forward's dequantised Q and K (K smoothed when p->smooth_k).  Inside:
 *   P recomputed from the INT8 scores and lse; dV = P^T dO with P as fp16(2^8 P);
 *   dP = dO V^T with dO and V - mean_t(V) in per-token INT8 (the mean's term drops out
 *   of dS, as it shifts every row's dP and D by the same amount);
 *   D = rowsum(dO * O) - dO . mean_t(V); dS = P * (dP - D);
 *   dQ = sm_scale dS K' (K' = K - mean_t(K) in fp16), dK = sm_scale dS^T Qdeq, both
 *   with dS as fp16 of a power-of-two multiple of dS chosen per call from bounds of
 *   |dO| and |V| so that it cannot overflow.
 * p: blk_q 64 or 128, smooth_q 0, q_group 0; otherwise SAGE_ERR_UNSUPPORTED.
 * ws: at least sage_attn_bwd_workspace_bytes(...) bytes.  d 64 or 128.
 */
int sage_attn_bwd(const void* q, const void* k, const void* v, const void* o, const void* dout, const float* lse,
                  float* dq, float* dk, float* dv, int B, int H, int N, int d, int causal, float sm_scale,
                  const sage_params* p, void* ws, size_t ws_bytes, void* stream);

/*
 * V of variant 3 in MXFP4 along the tokens (SageAttention3 abstract: FP4 attention; the
 * block format is read as OCP MXFP4, as for Q and K): for each channel c, every block of
 * 32 consecutive tokens gets the E8M0 code floor(log2 max|x|) - 2 + 127 clamped to
 * [0, 254] (0 for an all-zero block) and E2M1 elements of x / 2^(code - 127), nearest
 * even, saturating at 6; x = V (or V - v_mean with smooth_v, v_mean the exact token mean
 * of sage_quant_v_ex); tokens >= N are zeros.
 *   v_f4 [B,H,d,Np/2] bytes: two codes per byte along the tokens, the lower in the low
 *     nibble (16-byte aligned);
 *   v_e8 [B,H,Np/32,d] E8M0 codes, the scale of channel c at position
 *     (c % 32) * (d/32) + c / 32 (4-byte aligned);
 *   v_mean [B,H,d] fp32, written with smooth_v (may be NULL otherwise).
 * ws: with smooth_v, sage_workspace_bytes(B, H, N, d, 3, p) bytes with p->smooth_v = 1
 * suffice (only the token sums are used); may be NULL without it.
 */
int sage_quant_v_mx(const void* v, int B, int H, int N, int d, int smooth_v, uint8_t* v_f4, uint8_t* v_e8,
                    float* v_mean, void* ws, size_t ws_bytes, void* stream);

/*
 * The attention kernel that sage_attn_fwd runs for variant 3: Q is fp16 and quantised in
 * the kernel to MXFP4 (the sage_quant_qk_mx rule); K from sage_quant_qk_mx; V from
 * sage_quant_v_mx (same smooth_v as p).  Scores as variant 2; then, per query row and
 * 64-key tile, with c = sm_scale * log2(e) and m the running maximum of c * S over the
 * visible keys so far: P~_j = 2^fma(S_j, c, -m) in fp32 (<= 1), and each block of 32 keys
 * becomes MXFP4 with the smallest power-of-two scale 2^E that holds its largest weight a
 * without saturation (E8M0 code = E + 127, E = ceil(log2(a / 6)); 0 for a block of zeros;
 * elements E2M1(P~ / 2^E), nearest even).  O accumulates the E2M1 x E2M1 products with
 * both scales in fp32, rescaled when m moves; l sums the unrounded P~; O / l (+ v_mean).
 */
int sage_attn_fwd_qf16_fp4(const void* q, const uint8_t* k_f4, const uint8_t* k_e8, const uint8_t* v_f4,
                           const uint8_t* v_e8, const float* v_mean, void* o, int B, int H, int N, int d,
                           int causal, float sm_scale, const sage_params* p, void* stream);

/*
 * Test surface: the int32 products S = Qhat Khat^T that the attention kernel forms,
 * for chosen 128 x 64 tiles.  tiles[3*i + 0..2] = (flat head b*H+h, query tile, key
 * tile) with query rows [128*qt, 128*qt+128) and keys [64*kt, 64*kt+64) of the padded
 * tensors; tiles is a device array.  s_out: device [n_tiles][128][64] int32.
 * A tile outside the tensors yields zeros.
 */
int sage_debug_qk_int32(const int8_t* q_i8, const int8_t* k_i8, int B, int H, int N, int d,
                        const int* tiles, int n_tiles, int32_t* s_out, void* stream);

/* Message for the calling thread's last non-OK status ("" if none). */
const char* sage_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H_ */
