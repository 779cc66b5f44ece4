// sage_attn.hip -- fused 8-bit attention forward for gfx950 (CDNA4).
//
// Method: "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
// Acceleration" (summary page: "Summary", "Interesting ideas" I3): INT8 Q K^T,
// FlashAttention-style tiling with an online softmax, P~ V in FP16.
// "SageAttention2 ..." (abstract): FP8 P~ and V with two-level accumulation, and the
// Q-smoothing term added back to the scores.
// "SageAttention3 ..." (abstract): FP4 attention on matrix units; variant 2 reads it as
// OCP MXFP4 scores (E2M1 with an E8M0 scale per 32 channels) before the FP8 P~ V.
// Online softmax: "Online normalizer calculation for softmax" and FlashAttention(-2),
// entries of the summary page's reference list.
//
// Mapping onto CDNA4:
//  - A workgroup is 4 waves and owns 128 query rows of one head; each wave owns 32
//    rows.  Key/value tiles of 64 keys go through LDS once per workgroup.
//  - Scores are formed transposed, S^T = Khat Qhat^T, with v_mfma_i32_32x32x32_i8:
//    every lane then holds one query (column l%32) and 16 consecutive keys, so a
//    row max or sum needs only its own registers plus one v_permlane32_swap.
//    The K rows are loaded into the A operand in the order perm(r) so that
//    accumulator register i of lane half h is key 16h + i.
//  - Variant 2 forms the same S^T with v_mfma_scale_f32_32x32x64_f8f6f4 on packed E2M1
//    codes (the INT8 tile layouts with D/2 byte columns) and per-lane E8M0 scales.
//  - O is kept transposed, O^T = V^T P^T: P~ (converted in registers) is the B
//    operand as it stands; V^T comes from row-major LDS through ds_read_b64_tr_b16
//    (variant 0, fp16, v_mfma_f32_32x32x16_f16) or from the key-contiguous FP8 V^T
//    (variants 1 and 2, v_mfma_f32_32x32x64_f8f6f4), accumulated in fp32 in O.
//  - Causal: tiles past a wave's last row are skipped; workgroups run
//    longest-first and consecutive workgroups of one head stay on one XCD.
#include <type_traits>

#include "sage_device.h"
#include "sage_internal.h"
#include "sage_tiles.h"

namespace sage {

constexpr int kAttnWaves = 4;                     // waves per attention workgroup
constexpr int kAttnThreads = 64 * kAttnWaves;
constexpr int kAttnRows = 32 * kAttnWaves;        // query rows per attention workgroup
constexpr int kDbgWaves = 4;
                      // the int32 test kernel: 128 x 64 tiles

// (tile layouts, copies and the INT8 score product: sage_tiles.h)

// S^T tile with MXFP4 operands (variant 2).  The K and Q tiles hold two E2M1 codes
// per byte in the int8 layout of D/2 byte columns, so the operand reads are those of
// qk_tile; the 32 codes a lane brings to a 64-channel k-step are one MX block.  Byte ks
// of ksw[st] is the E8M0 scale of that block of the lane's key, byte ks of qsw the one
// of its query (v_mfma_scale_f32_32x32x64_f8f6f4, formats E2M1 x E2M1, fp32 result).
template <int D>
__device__ __forceinline__ void qk_tile_mx(const int8_t* sK, const int8_t* sQw, int lane, const uint32_t* ksw,
                                           uint32_t qsw, f32x16* s) {
  constexpr int CPR = D / 32;  // 16-byte chunks per row of D/2 bytes
  const int8_t* kbase = sK + 16 * lane;
  const int8_t* qbase = sQw + 16 * lane;
  f32x16 acc[2] = {f32x16{}, f32x16{}};
  auto step = [&](auto ksc) {
    constexpr int ks = decltype(ksc)::value;
    const i32x4 q4 = *reinterpret_cast<const i32x4*>(qbase + ks * 1024);
    const i32x8 qop = __builtin_shufflevector(q4, q4, 0, 1, 2, 3, -1, -1, -1, -1);  // FP4 uses 4 registers
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const i32x4 k4 = *reinterpret_cast<const i32x4*>(kbase + (st * CPR + 2 * ks) * 512);
      const i32x8 kop = __builtin_shufflevector(k4, k4, 0, 1, 2, 3, -1, -1, -1, -1);
      acc[st] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(kop, qop, acc[st], 4, 4, ks, (int)ksw[st], ks,
                                                               (int)qsw);
    }
  };
  step(std::integral_constant<int, 0>{});
  if constexpr (D == 128) step(std::integral_constant<int, 1>{});
  s[0] = acc[0];
  s[1] = acc[1];
}

// The MX scale bytes a lane brings to its k-steps, from a token's D/32 scale bytes
// (byte ks = block 2*ks + h).
template <int D>
__device__ __forceinline__ uint32_t mx_lane_scales(const uint8_t* e8_row, int h) {
  if constexpr (D == 128) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(e8_row);
    return __builtin_amdgcn_perm(w, w, h ? 0x0c0c0301u : 0x0c0c0200u);
  } else {
    return (uint32_t)e8_row[h];
  }
}

// 16 bytes of key `key`, chunk `chunk16`, of the K tile.
template <int D>
__device__ __forceinline__ const int8_t* k_lds_chunk(const int8_t* sK, int key, int chunk16) {
  return sK + 16 * k_slot<D>(key, chunk16);
}

// Rescaling of the running O is skipped while the row max grows by at most 2^8
// (variant 0 only): P~ is then computed against the older max and may reach 256,
// which fp16 and the fp32 sums hold exactly as well.
constexpr float kLazyLog2 = 8.0f;

// Online-softmax update for one 64-key tile of one lane (one query, 32 keys:
// s[st][i] is key kl + 32*st + i).  Works in the exp2 domain: x = S * c (+ bias),
// c = dQ * dK * sm_scale * log2(e).  Updates the reference max m and the lane's
// partial sum l (the lane pair l, l^32 shares m; l is summed over the pair at the
// end) and writes P~ already packed as the B operand of the P~V product:
//  variant 0: pk[st*8 + u*4 + q] = fp16 pair (P~ of keys 8u+2q, 8u+2q+1 of block st);
//  variant 1: pk[st*4 + w] = four E4M3 codes of P~ * 448 (keys 4w..4w+3 of block st);
//  variant 3: pk[w] = eight E2M1 codes of the lane's 32 keys (s[st][i] is key kl + 16*st + i
//  there), their MX block of P~, and pscale = its E8M0 scale code.
// alpha is the factor the running O must be scaled by (rescale is false for the whole
// wave when no lane needs it).
// MASK: keys >= N, and keys > qi when causal, get P~ = 0 and stay out of the max.
// DEFER0 (variant 3, unmasked interior tiles): leave the packed weights of a P~ block with
// scale code 0 for fp4_code0_fix after the interleaved block, so that block stays one
// basic block.
// RSUM (variant 0): l sums the fp16 weights the P~ V product uses, so the fp16 rounding of a
// dominant weight cancels in O / l; without it (training forward) l sums the unrounded P~,
// the sum the row log-sum-exp is defined on.
template <int VARIANT, bool CAUSAL, bool SMOOTHQ, bool MASK, bool DEFER0 = false, bool RSUM = true, typename SV>
__device__ __forceinline__ void softmax_tile(const SV* s, const float* c, const float* bias, int kl, int N,
                                             int qi, float& m, float& l, uint32_t* pk, float& alpha,
                                             bool& rescale, float lazy = kLazyLog2, uint32_t* pscale = nullptr) {
  // key kl + j is visible iff j <= jmax (keys < N, and <= qi when causal): one compare
  // against a constant per score
  const int jmax = (CAUSAL ? min(qi, N - 1) : N - 1) - kl;
  constexpr int KST = VARIANT == 3 ? 16 : 32;  // key step between the two products
  auto keep = [&](int st, int i) { return !MASK || KST * st + i <= jmax; };
  float x[2][16];
  float mt;
  if (SMOOTHQ) {
    mt = -INFINITY;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        x[st][i] = fmaf((float)s[st][i], c[st], bias[32 * st + i]);
        mt = keep(st, i) ? fmaxf(mt, x[st][i]) : mt;
      }
  } else if constexpr (VARIANT >= 2) {
    // fp32 scores (MXFP4); c > 0, so max_j fl(c * S_j) = fl(c * max_j S_j)
    float mf[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      mf[st] = -INFINITY;
#pragma unroll
      for (int i = 0; i < 16; ++i) mf[st] = keep(st, i) ? fmaxf(mf[st], s[st][i]) : mf[st];
    }
    mt = fmaxf(c[0] * mf[0], c[1] * mf[1]);
  } else {
    // c >= 0, so max_j fl(c * S_j) = fl(c * max_j S_j): the max is taken on the integers
    int mi[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      mi[st] = INT_MIN;
#pragma unroll
      for (int i = 0; i < 16; ++i) mi[st] = max(mi[st], keep(st, i) ? s[st][i] : INT_MIN);
    }
    const float m0 = (MASK && mi[0] == INT_MIN) ? -INFINITY : c[0] * (float)mi[0];
    const float m1 = (MASK && mi[1] == INT_MIN) ? -INFINITY : c[1] * (float)mi[1];
    mt = fmaxf(m0, m1);
  }
  mt = pair_max(mt);
  // m is finite after the first tile: key 0 is visible to every row
  // variant 1: P~ * 448 must stay <= 448 for FP8, so the max moves as soon as a row's
  // does (a wave whose rows all keep their max has alpha = 1 exactly and skips the
  // rescale)
  rescale = __builtin_amdgcn_ballot_w64(mt > m + (VARIANT == 0 ? lazy : 0.0f)) != 0;
  // branch-free so the caller's fast path stays one basic block
  const float mnew = rescale ? fmaxf(m, mt) : m;
  alpha = rescale ? __builtin_amdgcn_exp2f(m - mnew) : 1.0f;  // exp2(-inf) = 0 on the first tile
  m = mnew;
  l *= alpha;
  const float shift = VARIANT == 0 || VARIANT == 3 ? -m : kLog2_448 - m;
  float psum[2] = {0.0f, 0.0f};
  if constexpr (VARIANT == 3) {
    // P~ = 2^fma(S, c, -m) <= 1; the lane's 32 keys are one MX block: its scale is the
    // smallest power of two 2^E with max/2^E <= 6 (E8M0 code = biased exponent of the max
    // - 2, + 1 when its mantissa exceeds 1.5), the elements E2M1(P~ / 2^E)
    float pf[2][16];
    float pm = 0.0f;
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float pv = __builtin_amdgcn_exp2f(fmaf(s[st][i], c[st], shift));
        if (MASK) pv = keep(st, i) ? pv : 0.0f;
        pf[st][i] = pv;
        psum[st] += pv;
        pm = fmaxf(pm, pv);
      }
    const uint32_t pb = __float_as_uint(pm);
    const int code = max((int)(pb >> 23) - 2 + ((pb & 0x7fffffu) > 0x400000u ? 1 : 0), 0);
    const float sc = __uint_as_float((uint32_t)max(code, 1) << 23);  // 2^(code - 127)
    // the conversion divides by the scale (a power of two: exact) and rounds to nearest
    // even, saturating at 6; pk[w] holds keys 8w .. 8w+7, the lower key in the low nibble
    auto convert = [&](float scale, float mul, uint32_t* out) {
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        const float* q8 = &pf[w >> 1][8 * (w & 1)];
        uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q8[0] * mul, q8[1] * mul, scale, 0);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q8[2] * mul, q8[3] * mul, scale, 1);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q8[4] * mul, q8[5] * mul, scale, 2);
        word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q8[6] * mul, q8[7] * mul, scale, 3);
        out[w] = word;
      }
    };
    convert(sc, 1.0f, pk);
    if (!DEFER0 && __builtin_amdgcn_ballot_w64(code == 0) != 0) {
      // a block of zeros, or a largest weight below 2^-124 (scale code 0, 2^-127): such
      // lanes scale by 2^127 by hand (exact) and convert with a unit scale.  Only the
      // packed words are redone, so the common path keeps the weights where they are.
      uint32_t pk0[4];
      convert(1.0f, 0x1.0p127f, pk0);
#pragma unroll
      for (int w = 0; w < 4; ++w) pk[w] = code == 0 ? pk0[w] : pk[w];
    }
    *pscale = (uint32_t)code;
    l += psum[0] + psum[1];
    return;
  }
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      float pv[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float e = SMOOTHQ ? x[st][i + j] + shift : fmaf((float)s[st][i + j], c[st], shift);
        pv[j] = __builtin_amdgcn_exp2f(e);
        if (MASK) pv[j] = keep(st, i + j) ? pv[j] : 0.0f;
      }
      if constexpr (VARIANT == 0) {
        pk[st * 8 + i / 2] = pack_f16x2(pv[0], pv[1]);
        pk[st * 8 + i / 2 + 1] = pack_f16x2(pv[2], pv[3]);
        // an empty use keeps each pack next to its exps: left alone, the compiler sinks
        // the packs past the end of the interleaved block, so all 32 fp32 P~ of the lane
        // stay live across it (about 30 VGPRs, the third wave per SIMD at d = 64)
        asm volatile("" ::"v"(pk[st * 8 + i / 2]), "v"(pk[st * 8 + i / 2 + 1]));
      } else {
        pk[st * 4 + i / 4] = cvt_pk_fp8(pv[2], pv[3], cvt_pk_fp8(pv[0], pv[1], 0u, false), true);
      }
      if (VARIANT == 0 && RSUM) {
        psum[st] = sum_f16x2(pk[st * 8 + i / 2], psum[st]);
        psum[st] = sum_f16x2(pk[st * 8 + i / 2 + 1], psum[st]);
      } else {
        psum[st] += (pv[0] + pv[1]) + (pv[2] + pv[3]);
      }
    }
  l += psum[0] + psum[1];
}


// Variant 3, unmasked tile whose softmax deferred the rare scale code 0 (a P~ block whose
// largest weight is below 2^-124, or all zero): the lanes with that code redo their P~
// from S exactly as softmax_tile formed it (2^fma(S, c, -m) with the updated m), scale it
// by 2^127 by hand (exact) and convert with a unit scale.
__device__ __forceinline__ void fp4_code0_fix(const f32x16* s, const float* c, float m, uint32_t code,
                                              uint32_t* pk) {
  float pf[2][16];
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; ++i) pf[st][i] = __builtin_amdgcn_exp2f(fmaf(s[st][i], c[st], -m)) * 0x1.0p127f;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const float* q8 = &pf[w >> 1][8 * (w & 1)];
    uint32_t word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, q8[0], q8[1], 1.0f, 0);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q8[2], q8[3], 1.0f, 1);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q8[4], q8[5], 1.0f, 2);
    word = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q8[6], q8[7], 1.0f, 3);
    pk[w] = code == 0u ? word : pk[w];
  }
}

// Variant 0, unmasked tile: P~ against the row's current reference m, without the
// tile's maximum.  The reference only has to keep P~ within fp16 and the sums
// finite, so a tile whose P~ stay small keeps it: when every lane's 32 P~ sum to at
// most kFastSum = 2^10, l gains that sum and pk holds the tile, and the function
// returns false.  Otherwise (a key far above m, or m = -inf on a row's first tile) it
// returns true for the whole wave, leaves m and l untouched, and the caller recomputes
// the tile with softmax_tile, which moves m to the running maximum.
// RSUM: as in softmax_tile.
constexpr float kFastSum = 1024.0f;  // 2^10
template <bool RSUM = true>
__device__ __forceinline__ bool softmax_tile_fast(const i32x16* s, const float* c, float m, float& l,
                                                  uint32_t* pk) {
  const float shift = -m;
  float psum[2] = {0.0f, 0.0f};
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; i += 4) {
      float p[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) p[j] = __builtin_amdgcn_exp2f(fmaf((float)s[st][i + j], c[st], shift));
      pk[st * 8 + i / 2] = pack_f16x2(p[0], p[1]);
      pk[st * 8 + i / 2 + 1] = pack_f16x2(p[2], p[3]);
      asm volatile("" ::"v"(pk[st * 8 + i / 2]), "v"(pk[st * 8 + i / 2 + 1]));  // as in softmax_tile
      if (RSUM) {
        psum[st] = sum_f16x2(pk[st * 8 + i / 2], psum[st]);
        psum[st] = sum_f16x2(pk[st * 8 + i / 2 + 1], psum[st]);
      } else {
        psum[st] += (p[0] + p[1]) + (p[2] + p[3]);
      }
    }
  const float t = psum[0] + psum[1];
  // also true for inf and NaN sums
  const bool slow = __builtin_amdgcn_ballot_w64(!(t <= kFastSum)) != 0;
  l = slow ? l : l + t;
  return slow;
}

// Q smoothing: the term sm_scale*log2(e) * dK_j * (qmean_sb . Khat_j) of every key j of a
// tile, for each Q block sb of the workgroup (up to 4), runs on the matrix unit.  The
// prologue splits each block mean into four int8 limbs (split_qmean), so qmean . Khat
// is four exact int32 dot products; limb k of block sb is column 4*sb + k of a
// 16-column int8 matrix in LDS.
//
// Limbs of one block mean (wave sb, D/64 channels per lane): with |qmean| < 2^e and
// s0 = 2^(e-6), l0 = rint(qmean / s0), then each next limb is the rounded residual in
// units 128 times smaller: l_k = rint(r_k / (s0 * 2^-7k)), r_(k+1) = r_k - l_k*s0*2^-7k.
// Each residual is exact in fp32 and every limb lies in [-64, 64]:
// qmean = s3 * (2^21*l0 + 2^14*l1 + 2^7*l2 + l3) up to s3/2 per channel, s3 = s0 * 2^-21
// (2^-27 of the block's largest mean), below the fp32 rounding of the bias itself.  Only
// the last limb rounds a non-integer residual, and 128 * (higher limbs) is even, so the
// limbs compose exactly rint(qmean * 2^(27-e)), ties to even: the fixed-point mean that
// defines the term.
template <int D>
__device__ __forceinline__ void split_qmean(const float* qmean, bool valid, int8_t* sQl, float* sScale, int sb) {
  const int lane = threadIdx.x & 63;
  float x[D / 64];
  float am = 0.0f;
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    x[j] = valid ? qmean[lane + 64 * j] : 0.0f;
    am = fmaxf(am, fabsf(x[j]));
  }
  am = wave_max(am);
  // am < 2^e; tiny means share the exponent of 2^-100 so that 1/s0 stays finite
  const int e = max(__builtin_amdgcn_frexp_expf(am), -100);
#pragma unroll
  for (int j = 0; j < D / 64; ++j) {
    float v = x[j];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const float lk = rintf(v * __builtin_amdgcn_ldexpf(1.0f, 6 - e + 7 * k));
      v = v - lk * __builtin_amdgcn_ldexpf(1.0f, e - 6 - 7 * k);  // exact
      sQl[(4 * sb + k) * D + lane + 64 * j] = (int8_t)(int)lk;
    }
  }
  if (lane == 0) sScale[sb] = __builtin_amdgcn_ldexpf(1.0f, e - 27);  // s3
}

// The bias of keys 16*wave .. 16*wave + 15 of the K tile in sK for every Q block, one
// 16x16x64 INT8 MFMA per 64 channels: A = the limb matrix (row = lane%16 = 4*block +
// limb), B = those keys (column = lane%16), the same 16 channels per lane for both.  Lane
// l then holds key 16*wave + l%16 in column l%16 and rows 4*(l/16) + 0..3, i.e. the four
// limbs of Q block l/16: it combines them in its own registers and writes one bias.
// wk = sm_scale * log2(e) * dK of those 16 keys (one K block: blk_k >= 16).
template <int D>
__device__ __forceinline__ void smooth_q_bias(const int8_t* sK, const int8_t* sQl, const float* sScale, float wk,
                                              float* sBias) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = lane & 15, grp = lane >> 4;
  i32x4 acc = {0, 0, 0, 0};
#pragma unroll
  for (int kk = 0; kk < D / 64; ++kk) {
    const i32x4 ka = *reinterpret_cast<const i32x4*>(k_lds_chunk<D>(sK, 16 * wave + n, 4 * kk + grp));
    const i32x4 qa = *reinterpret_cast<const i32x4*>(sQl + n * D + 64 * kk + 16 * grp);
    acc = __builtin_amdgcn_mfma_i32_16x16x64_i8(qa, ka, acc, 0, 0, 0);
  }
  // The dot product of the fixed-point mean with the key, B = 2^21 L0 + 2^14 L1 + 2^7 L2 + L3,
  // is formed exactly and rounded once to fp32, so the term is a reproducible fp32 number
  // (it decides FP8 codes of P~): |l_k . Khat| <= 64*127*D < 2^21, so 128*L0 + L1 and
  // 128*L2 + L3 fit in int32, and the fp64 fma is exact (|B| < 2^43).
  const float b = (float)__builtin_fma((double)(acc[0] * 128 + acc[1]), 16384.0, (double)(acc[2] * 128 + acc[3]));
  sBias[grp * kTileKV + 16 * wave + n] = wk * sScale[grp] * b;
}

// Instruction order of the interior-tile block: after a few operand reads, each MFMA
// is followed by the LDS reads for the next one and a share of the softmax's VALU
// instructions, which execute while the MFMA occupies the matrix unit.  (Written as
// loops without conditionals: a guarded sched_group_barrier is not honoured.)
template <int D, int VARIANT, bool SMOOTHQ>
__device__ __forceinline__ void interleave_schedule() {
  // every MFMA takes two LDS operand reads (K and Q, two V transposes, or two V^T
  // halves); they are issued LEAD MFMAs ahead of their use, so the LDS latency (about
  // 200 cycles) overlaps the MFMAs and VALU work in between
  constexpr int LEAD = 2;
  constexpr int MFMA = (VARIANT >= 2 ? 2 * (D / 64) : 2 * (D / 32)) + (VARIANT == 0 ? 4 * (D / 32) : D / 32);
  constexpr int VALU_PER = VARIANT == 0 ? (D == 128 ? 5 : 12)
                           : VARIANT == 1 ? (D == 128 ? 8 : 14)
                           : VARIANT == 3 ? (D == 128 ? 22 : 40)
                                          : (D == 128 ? 20 : 16);
  // with Q smoothing the softmax first reads its 32 biases (8 reads of 16 bytes)
  __builtin_amdgcn_sched_group_barrier(0x100, 2 * LEAD + (SMOOTHQ ? 8 : 0), 0);
#pragma unroll
  for (int i = 0; i < MFMA; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
    __builtin_amdgcn_sched_group_barrier(0x002, VALU_PER, 0);
  }
}

// FUSEQ: Q arrives as fp16 and each workgroup quantises its own rows into the LDS
// operand tile, with the rule of the quantisation pass: INT8 per group of q_group =
// 1 .. 128 rows (the workgroup's 128 rows are whole groups; with Q smoothing the exact
// mean of each Q block of blk_q rows is taken out first), or MXFP4 per 32-channel block
// (one lane's operand per block).
// Two workgroups per CU; at d = 64 the 8-bit P~V variants are held to 168 VGPRs, which
// gives a third (their LDS is small): variant 3 and variant 1 with causal Q smoothing sat
// at 169-171 VGPRs and run 10-14 % faster with the third wave (a spill or two).
// TRAIN (training forward, variant 0): l sums the unrounded P~ (RSUM off), so the row
// log-sum-exp is that of the weights themselves; O can then differ from the inference
// forward's in its last fp16 bits.
// KT (blk_k >= 64): one K block covers each key tile, so a tile has one K scale and every
// lane the same K factor of c (a scalar operand), instead of one scale per 16-key quarter.
template <int D, int VARIANT, bool CAUSAL, bool SMOOTHQ, bool FUSEQ, bool TRAIN = false, bool KT = false>
__global__ __launch_bounds__(kAttnThreads, D == 64 && VARIANT >= 1 ? 3 : 2) void attn_kernel(AttnArgs a) {
  static_assert(!TRAIN || (VARIANT == 0 && !SMOOTHQ), "training forward: variant 0 without Q smoothing");
  static_assert(!KT || VARIANT <= 1, "one K scale per tile: INT8 scores");
  static_assert(!FUSEQ || VARIANT <= 1 || !SMOOTHQ, "in-kernel Q quantisation with Q smoothing: INT8 Q only");
  static_assert(VARIANT < 2 || !SMOOTHQ, "MXFP4 scores: no Q smoothing");
  using L = Lds<D, VARIANT>;
  constexpr int KD = qk_row_bytes<D, VARIANT>();  // bytes per Q / K row
  constexpr int NCT = D / 32;                       // 32-channel output tiles
  constexpr int NSUB = SMOOTHQ ? kAttnRows / 32 : 1;  // Q blocks a workgroup can span (blk_q >= 32)
  // Two slots per tile kind, as separate LDS objects: the loop body is instantiated
  // per slot parity, so the compiler can tell the slot being filled by an in-flight
  // copy from the slot being read and does not wait for the copy.
  __shared__ __attribute__((aligned(16))) int8_t sK0[L::K_BYTES];
  __shared__ __attribute__((aligned(16))) int8_t sK1[L::K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sV0[L::V_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sV1[L::V_BYTES];
  __shared__ __attribute__((aligned(16))) int8_t sQ[kAttnRows * KD];
  __shared__ __attribute__((aligned(16))) int8_t sQl[SMOOTHQ ? 16 * D : 1];  // limbs of the Q block means
  __shared__ float sQs[SMOOTHQ ? NSUB : 1];                                   // their scales
  __shared__ __attribute__((aligned(16))) float sBias0[SMOOTHQ ? NSUB * kTileKV : 1];
  __shared__ __attribute__((aligned(16))) float sBias1[SMOOTHQ ? NSUB * kTileKV : 1];
  __shared__ float sAmax[kAttnWaves];  // FUSEQ: |Q| max of each wave's rows
  __shared__ float sQmean[FUSEQ && SMOOTHQ ? NSUB * D : 1];    // FUSEQ with Q smoothing: the block means
  __shared__ double sQsum[FUSEQ && SMOOTHQ ? kAttnWaves * D : 1];  //  and each wave's column sums

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, ql = lane & 31;
  const int N = a.N;

  // workgroup -> (head, query tile).  Consecutive workgroup ids go round-robin over the
  // 8 XCDs; remap so each XCD walks a contiguous range of (head, tile) pairs, heads
  // one after another.  Causal query tiles differ in length (tile qt sees qt + 1 key
  // blocks), so they go longest first across each pair of heads: walking one head's
  // tiles after another's would start the last head's longest tiles late and leave the
  // XCD's other workgroup slots idle at the end (about a tenth of the kernel at
  // B=4 H=32 N=4096).  Two heads at a time keep the K/V working set of an XCD small.
  const int nqt = (a.Np + kAttnRows - 1) / kAttnRows;
  const int total = a.G * nqt;
  int vid = blockIdx.x;
  if ((total & 7) == 0) vid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  int g, qt;
  if constexpr (CAUSAL) {
    const int pair = vid / (2 * nqt), r = vid - pair * 2 * nqt;
    if (2 * pair + 1 < a.G) {
      g = 2 * pair + (r & 1);
      qt = nqt - 1 - (r >> 1);
    } else {  // odd head count: the last head alone
      g = 2 * pair;
      qt = nqt - 1 - r;
    }
  } else {
    g = vid / nqt;
    qt = vid % nqt;
  }
  const int q0 = qt * kAttnRows;
  const int qw = q0 + 32 * wave;  // first row of this wave
  const int qi = qw + ql;         // this lane's query row
  const bool wave_active = qw < N;

  const int8_t* __restrict__ qh = FUSEQ ? nullptr : a.q_i8 + (size_t)g * a.Np * KD;
  const int8_t* __restrict__ kh = a.k_i8 + (size_t)g * a.Np * KD;
  const float* __restrict__ ksc = VARIANT >= 2 ? nullptr : a.k_scale + (size_t)g * a.nkb;

  const int ntiles_all = (N + kTileKV - 1) / kTileKV;
  const int wg_last_row = min(q0 + kAttnRows - 1, N - 1);
  const int T = CAUSAL ? min(ntiles_all, wg_last_row / kTileKV + 1) : ntiles_all;
  const int wave_last = CAUSAL ? min(ntiles_all - 1, min(qw + 31, N - 1) / kTileKV) : ntiles_all - 1;

  int8_t* const sQw = sQ + wave * (KD / 32) * 1024;
  // FUSEQ: lane l holds fp16 Q of row qw + l%32, the channels its operand reads take:
  // variant 0: 32*ks + 16*h .. +15 in qraw[2ks], qraw[2ks+1]; variant 2: the MX block
  // 64*ks + 32*h .. +31 in qraw[4ks .. 4ks+3].  Rows >= N are zeros.
  uint4 qraw[FUSEQ ? D / 16 : 1];
  if constexpr (FUSEQ) {
    constexpr int PER = VARIANT >= 2 ? 4 : 2;  // 16-byte loads per k-step
    const bool row_ok = wave_active && qi < N;
    const uint16_t* qsrc = a.q + ((size_t)g * N + (row_ok ? qi : 0)) * D + 8 * PER * h;
#pragma unroll
    for (int ks = 0; ks < D / (16 * PER); ++ks)
#pragma unroll
      for (int j = 0; j < PER; ++j)
        qraw[PER * ks + j] =
            row_ok ? *reinterpret_cast<const uint4*>(qsrc + 16 * PER * ks + 8 * j) : make_uint4(0u, 0u, 0u, 0u);
  } else {
    // qw < N <= Np, and Np is a multiple of 32: an active wave's rows lie in the tensor
    if (wave_active) load_q_tile<KD>(make_rsrc(qh, (size_t)a.Np * KD), qw, sQw);
  }
  // block and group sizes are powers of two
  const int kshift = __builtin_ctz(a.blk_k), qshift = __builtin_ctz(a.blk_q);
  // Q scale of this lane's row: one per group of q_group rows, so uniform over the wave
  // for groups of 32 rows or more (FUSEQ: set once the group's |Q| max is known)
  float dq = (!FUSEQ && VARIANT < 2 && wave_active)
                 ? a.q_scale[(size_t)g * a.nqg + (min(qi, N - 1) >> __builtin_ctz(a.q_group))]
                 : 0.0f;
  // variant 2: the MX scale bytes of this lane's query (rows >= N hold zeros)
  uint32_t qsw = 0;
  if constexpr (VARIANT >= 2 && !FUSEQ) {
    if (wave_active) qsw = mx_lane_scales<D>(a.q_e8 + ((size_t)g * a.Np + qi) * (D / 32), h);
  }

  f32x16 o[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o[ct] = f32x16{};
  float m = -INFINITY, l = 0.0f;

  // Software pipeline over key tiles.  Iteration t (t = 0..T) issues the MFMA work
  // S(t+1) = K(t+1) Q^T and O += P~(t-1) V(t-1), and the VALU work softmax(t); neither
  // depends on the other, so the wave keeps both units busy.  O is rescaled for tile t
  // after P~(t-1) V(t-1) has been added, P~(t) waits in registers for the next
  // iteration.  LDS: K(t+2) is copied into the slot of K(t) at the start of iteration t;
  // V(t+1) into the slot of V(t-1) right after the barrier that ends iteration t; the
  // barrier also waits for the copies started before it.
  const TileCopy<D, VARIANT, kAttnWaves> copy(a.Np);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kh, (size_t)a.Np * KD);
  const __amdgpu_buffer_rsrc_t vrs =
      VARIANT == 0   ? make_rsrc(a.v + (size_t)g * N * D, (size_t)N * D * 2)
      : VARIANT == 3 ? make_rsrc(a.v_f8 + (size_t)g * D * (a.Np / 2), (size_t)D * (a.Np / 2))
                     : make_rsrc(a.v_f8 + (size_t)g * D * a.Np, (size_t)D * a.Np);

  copy.k_tile(krs, 0, sK0);
  copy.v_tile(vrs, 0, a.Np, sV0);
  if (T > 1) copy.k_tile(krs, 1, sK1);
  // iteration 0 multiplies P~(-1) = 0 by the V slot it reads, which is filled only after
  // it; clear that slot (0 times a stale NaN pattern would not be 0)
  for (int e = tid; e < L::V_BYTES / 16; e += kAttnThreads)
    reinterpret_cast<uint4*>(sV1)[e] = make_uint4(0u, 0u, 0u, 0u);
  if constexpr (FUSEQ && SMOOTHQ) {
    // The exact means of the workgroup's Q blocks, by the quantisation pass's rule: the
    // sum of the fp16 values is exact in fp64 (they are multiples of 2^-24 below 2^16, so
    // a sum of up to 128 needs 47 bits), and sum / count rounds once to fp64, then to
    // fp32.  Each wave sums its 32 rows: it stages half of its channels at a time in its
    // own part of the Q operand tile (written with codes only later) and lane l adds
    // channel l of the half down the rows.
    uint16_t* const stage = reinterpret_cast<uint16_t*>(sQw);  // 32 rows x D/2 fp16
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      // lane (ql, h) holds channels 32*(i/2) + 16h + 8*(i%2) .. +7 in qraw[i]: this half
      // covers channels [half*D/2, half*D/2 + D/2)
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        const int c0 = 32 * (i >> 1) + 16 * h + 8 * (i & 1);
        if (c0 / (D / 2) == half)
          *reinterpret_cast<uint4*>(stage + ql * (D / 2) + c0 - half * (D / 2)) = qraw[i];
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the wave's LDS writes are done
      __builtin_amdgcn_wave_barrier();
      if (lane < D / 2) {
        double sum = 0.0;
#pragma unroll 8
        for (int r = 0; r < 32; ++r) sum += (double)(float)__builtin_bit_cast(_Float16, stage[r * (D / 2) + lane]);
        sQsum[wave * D + half * (D / 2) + lane] = sum;
      }
      __builtin_amdgcn_s_waitcnt(0xc07f);
      __builtin_amdgcn_wave_barrier();
    }
    __syncthreads();
    if (tid < D) {
      for (int sb = 0; sb < (kAttnRows >> qshift); ++sb) {
        const int r0 = sb << qshift, r1 = min(r0 + a.blk_q, N - q0);
        double sum = 0.0;
        for (int w = r0 >> 5; w < (r0 + a.blk_q) >> 5; ++w) sum += sQsum[w * D + tid];
        sQmean[sb * D + tid] = r1 > r0 ? (float)(sum / (double)(r1 - r0)) : 0.0f;
      }
    }
    __syncthreads();
  }

  if constexpr (SMOOTHQ) {
    // wave sb splits the mean of the workgroup's Q block sb (up to 4 blocks; the others
    // get zero limbs)
    static_assert(NSUB == kAttnWaves, "one wave per Q block of the workgroup");
    const int sb = wave, qb = (q0 >> qshift) + sb;
    const float* qm = FUSEQ ? sQmean + sb * D : a.q_mean + ((size_t)g * a.nqb + qb) * D;
    split_qmean<D>(qm, sb * a.blk_q < kAttnRows && qb < a.nqb, sQl, sQs, sb);
  }

  // FUSEQ with Q smoothing: the smoothed fp32 values of this lane's fp16 Q, xs[8i + j] =
  // channel 32*(i/2) + 16h + 8*(i%2) + j minus its block mean; rows >= N are zero, as in
  // the quantisation pass
  float xs[FUSEQ && SMOOTHQ ? D / 2 : 1];
  if constexpr (FUSEQ && SMOOTHQ) {
    const bool row_ok = wave_active && qi < N;
    const float* mrow = sQmean + ((32 * wave + ql) >> qshift) * D;
#pragma unroll
    for (int i = 0; i < D / 16; ++i) {
      const int c0 = 32 * (i >> 1) + 16 * h + 8 * (i & 1);
      const float4 m0 = *reinterpret_cast<const float4*>(mrow + c0);
      const float4 m1 = *reinterpret_cast<const float4*>(mrow + c0 + 4);
      const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
      const uint32_t w[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const f16x2 hv = __builtin_bit_cast(f16x2, w[u]);
        xs[8 * i + 2 * u] = row_ok ? (float)hv[0] - mv[2 * u] : 0.0f;
        xs[8 * i + 2 * u + 1] = row_ok ? (float)hv[1] - mv[2 * u + 1] : 0.0f;
      }
    }
  }
  if constexpr (FUSEQ && VARIANT <= 1) {
    float lm;  // this lane's half of row qi: its |Q| max
    if constexpr (SMOOTHQ) {
      lm = 0.0f;
#pragma unroll
      for (int j = 0; j < D / 2; ++j) lm = fmaxf(lm, fabsf(xs[j]));
    } else {
      // with the sign bits cleared, fp16 bit patterns order like the values, so a packed
      // 16-bit integer max finds the |Q| max exactly
      typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
      u16x2 mx = {0, 0};
#pragma unroll
      for (int i = 0; i < D / 16; ++i) {
        const uint32_t w[4] = {qraw[i].x, qraw[i].y, qraw[i].z, qraw[i].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) mx = __builtin_elementwise_max(mx, __builtin_bit_cast(u16x2, w[j] & 0x7fff7fffu));
      }
      const u16x2 mb = {__builtin_elementwise_max(mx[0], mx[1]), 0};
      lm = (float)__builtin_bit_cast(f16x2, mb)[0];
    }
    const float am = wave_max(lm);
    if (lane == 0) sAmax[wave] = am;
    if (a.q_group < 32) {
      // groups inside the wave: the row's max over the lane pair, then over the group's
      // q_group consecutive rows (lanes)
      float gm = pair_max(lm);
      for (int off = 1; off < a.q_group; off <<= 1) gm = fmaxf(gm, __shfl_xor(gm, off));
      dq = gm;  // the group's |Q| max until the scale is formed below
    }
  }
  wait_copies();
  __syncthreads();
  if constexpr (FUSEQ && VARIANT >= 2) {
    // each k-step's 32 channels of this lane are one MX block
#pragma unroll
    for (int ks = 0; ks < D / 64; ++ks) {
      float v[32];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t w[4] = {qraw[4 * ks + j].x, qraw[4 * ks + j].y, qraw[4 * ks + j].z, qraw[4 * ks + j].w};
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const f16x2 hv = __builtin_bit_cast(f16x2, w[u]);
          v[8 * j + 2 * u] = (float)hv[0];
          v[8 * j + 2 * u + 1] = (float)hv[1];
        }
      }
      uint4 packed;
      qsw |= mx_block_fp4(v, packed) << (8 * ks);
      *reinterpret_cast<uint4*>(sQw + ks * 1024 + 16 * lane) = packed;
    }
  }
  if constexpr (FUSEQ && VARIANT <= 1) {
    // a group of 32 rows or more spans waves w0 .. w0 + q_group/32 - 1
    float amax = dq;
    if (a.q_group >= 32) {
      const int wpb = a.q_group >> 5, w0 = wave & ~(wpb - 1);
      amax = sAmax[w0];
      for (int w = 1; w < wpb; ++w) amax = fmaxf(amax, sAmax[w0 + w]);
    }
    dq = i8_scale(amax);
    const float r = i8_factor(amax);
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      uint32_t pk4[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = 2 * ks + u / 2, j0 = 2 * (u & 1);  // qraw[i], words j0 and j0 + 1
        const uint4 src = qraw[i];
        const uint32_t w0v = (u & 1) ? src.z : src.x, w1v = (u & 1) ? src.w : src.y;
        const f16x2 h0 = __builtin_bit_cast(f16x2, w0v), h1 = __builtin_bit_cast(f16x2, w1v);
        float x[4] = {(float)h0[0], (float)h0[1], (float)h1[0], (float)h1[1]};
        if constexpr (SMOOTHQ) {
          x[0] = xs[8 * i + 2 * j0];
          x[1] = xs[8 * i + 2 * j0 + 1];
          x[2] = xs[8 * i + 2 * j0 + 2];
          x[3] = xs[8 * i + 2 * j0 + 3];
        }
        pk4[u] = pack_bytes4(i8_code_int(x[0], r), i8_code_int(x[1], r), i8_code_int(x[2], r), i8_code_int(x[3], r));
      }
      *reinterpret_cast<uint4*>(sQw + ks * 1024 + 16 * lane) = make_uint4(pk4[0], pk4[1], pk4[2], pk4[3]);
    }
  }
  // scale factors c = dQ * dK * sm_scale * log2(e); the raw K scales of a tile are
  // loaded one iteration before they are needed.  S, c and packed P~ alternate
  // between two register sets by tile parity.
  // (variant 2: S is fp32 from the scaled MFMA, c = sm_scale * log2(e), and kw holds
  // the MX scale bytes of this lane's key in each 32-key block of tile t+1)
  constexpr int NPK = VARIANT == 0 ? 16 : VARIANT == 3 ? 4 : 8;
  using SAcc = std::conditional_t<VARIANT >= 2, f32x16, i32x16>;
  SAcc sA[2], sB[2];
  float cA[2], cB[2], kq[4];  // kq: raw K scales of tile t+1 (see tile_kscales)
  uint32_t kw[2];
  const unsigned last_key = (unsigned)(N - 1);
  uint32_t pkA[NPK], pkB[NPK];
#pragma unroll
  for (int i = 0; i < NPK; ++i) pkB[i] = 0u;  // P~(-1)
  // variant 3: E8M0 scale codes of the P~ blocks (by tile parity) and of this lane's V
  // channels (byte ct: channel 32*ct + l%32) for the V tiles in the two LDS slots; the
  // zero P~(-1) and V slot of iteration 0 get unit scales (code 127)
  uint32_t pscA = 127u, pscB = 127u;
  bool fp4_fix_pending = false;  // variant 3: P~ of the last tile needs fp4_code0_fix
  uint32_t vsc[2] = {0x7f7f7f7fu, 0x7f7f7f7fu};
  auto v_scales = [&](int t) -> uint32_t {
    const uint8_t* e = a.v_e8 + ((size_t)g * (a.Np / 32) + 2 * t + h) * D + ql * (D / 32);
    if constexpr (D == 128) return *reinterpret_cast<const uint32_t*>(e);
    else return (uint32_t)*reinterpret_cast<const uint16_t*>(e);
  };
  const float dqs = dq * a.kscale;
  // MX scale bytes of the keys this lane's A-operand rows hold in tile t (clamped into
  // the padded tensor; the pad rows carry zeros)
  auto mx_kscales = [&](int t, uint32_t* w) {
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int key = min(t * kTileKV + k_row_key<VARIANT>(st, ql), a.Np - 1);
      w[st] = mx_lane_scales<D>(a.k_e8 + ((size_t)g * a.Np + key) * (D / 32), h);
    }
  };
  // S(t) for the K tile in sKt
  auto score_tile = [&](const int8_t* sKt, SAcc* out) {
    if constexpr (VARIANT >= 2)
      qk_tile_mx<D>(sKt, sQw, lane, kw, qsw, out);
    else
      qk_tile<D>(sKt, sQw, lane, out);
  };
  if constexpr (VARIANT >= 2) {
    mx_kscales(0, kw);
    if (wave_active) score_tile(sK0, sA);  // tile 0 is visible to every row
    cA[0] = cA[1] = a.kscale;
    mx_kscales(1, kw);
    if constexpr (VARIANT == 3) vsc[0] = v_scales(0);
  } else {
    if (wave_active) score_tile(sK0, sA);  // tile 0 is visible to every row
    tile_kscales_for<KT>(ksc, 0, last_key, kshift, kq);
    cA[0] = dqs * (KT ? kq[0] : kscale_of(kq, 0, h));
    cA[1] = dqs * (KT ? kq[0] : kscale_of(kq, 1, h));
    if (SMOOTHQ)
      smooth_q_bias<D>(sK0, sQl, sQs, a.kscale * kscale_quarter(ksc, 0, wave_id(), last_key, kshift), sBias0);
    tile_kscales_for<KT>(ksc, 1, last_key, kshift, kq);
  }
  __syncthreads();
  // V(1) is copied by iteration 0, after its barrier.  Nothing is in flight when the
  // loop starts, so the compiler sees no pending copy into a slot the loop reads.

  // transpose-read base of this lane in a V tile (variant 0)
  const int vbase_off = pv_lane_offset<D>(lane);

  // O += P~(t-1) V(t-1) from the V tile in slot sVp with P~ packed in pkp (variant 3:
  // with the scale code psp of the P~ block and the V scale bytes vs).
  auto pv_tile = [&](const uint8_t* sVp, const uint32_t* pkp, uint32_t psp = 0u, uint32_t vs = 0u) {
    if constexpr (VARIANT == 0) {
      // A operand V^T: a transpose read of 4 keys x 16 channels (one 128-byte block)
      // gives lane j of a 16-lane group channel C0 + j for 4 keys.
      pv_tile_f16<D>(sVp + vbase_off, pkp, o);
    } else if constexpr (VARIANT == 3) {
      // E2M1 x E2M1 with both MX scales: lane half h brings keys 32h .. 32h + 31 of the
      // tile for its query (B) and for its channel (A, 16 bytes of the V^T slot)
      const i32x4 p4 = {(int)pkp[0], (int)pkp[1], (int)pkp[2], (int)pkp[3]};
      const i32x8 pb = __builtin_shufflevector(p4, p4, 0, 1, 2, 3, -1, -1, -1, -1);  // FP4 uses 4 registers
      auto tile_ct = [&](auto ctc) {  // the scale byte select must be a constant
        constexpr int ct = decltype(ctc)::value;
        const i32x4 v4 = *reinterpret_cast<const i32x4*>(sVp + 16 * lane + ct * 1024);
        const i32x8 va = __builtin_shufflevector(v4, v4, 0, 1, 2, 3, -1, -1, -1, -1);
        o[ct] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(va, pb, o[ct], 4, 4, ct, (int)vs, 0, (int)psp);
      };
      tile_ct(std::integral_constant<int, 0>{});
      tile_ct(std::integral_constant<int, 1>{});
      if constexpr (NCT == 4) {
        tile_ct(std::integral_constant<int, 2>{});
        tile_ct(std::integral_constant<int, 3>{});
      }
    } else {
      // the FP8 MFMA accumulates in fp32, straight into O: the fp32 outer accumulator of
      // two-level accumulation, already rescaled for this tile at the end of the last
      // iteration
      i32x8 pb;
#pragma unroll
      for (int w = 0; w < 8; ++w) pb[w] = (int)pkp[w];
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const i32x4 v0 = *reinterpret_cast<const i32x4*>(sVp + 16 * lane + (4 * ct) * 512);
        const i32x4 v1 = *reinterpret_cast<const i32x4*>(sVp + 16 * lane + (4 * ct + 2) * 512);
        const i32x4 vv[2] = {v0, v1};
        o[ct] = mfma_f8(__builtin_bit_cast(i32x8, vv), pb, o[ct]);
      }
    }
  };

  auto iteration = [&](int t, auto parity) {
    constexpr int cur = decltype(parity)::value;
    int8_t* const sKc = cur == 0 ? sK0 : sK1;         // K(t), refilled with K(t+2)
    const int8_t* const sKn = cur == 0 ? sK1 : sK0;   // K(t+1)
    uint8_t* const sVp = cur == 0 ? sV1 : sV0;        // V(t-1), refilled with V(t+1)
    const float* const sBc = cur == 0 ? sBias0 : sBias1;
    float* const sBn = cur == 0 ? sBias1 : sBias0;
    SAcc* const s = cur == 0 ? sA : sB;               // S(t)
    SAcc* const sn = cur == 0 ? sB : sA;              // S(t+1)
    float* const c = cur == 0 ? cA : cB;
    float* const cn = cur == 0 ? cB : cA;
    uint32_t* const pk = cur == 0 ? pkA : pkB;        // P~(t)
    uint32_t* const pkp = cur == 0 ? pkB : pkA;       // P~(t-1)
    uint32_t* const psc = cur == 0 ? &pscA : &pscB;   // variant 3: block scale of P~(t)
    const uint32_t psp = cur == 0 ? pscB : pscA;      //  and of P~(t-1)

    if constexpr (VARIANT == 3) {
      // P~(t-1) of an interior tile that took scale code 0 (its S, c and the row's m are
      // still those of tile t-1 here)
      if (fp4_fix_pending) {
        fp4_code0_fix(sn, cn, m, psp, pkp);
        fp4_fix_pending = false;
      }
    }
    const bool compute = wave_active && t < T && t <= wave_last;
    const bool compute_next = wave_active && t + 1 <= wave_last && t + 1 < T;
    // P~(-1) and the V slot read at t = 0 are zeros, so iteration 0 may run the
    // interleaved block too: its P~V adds nothing
    const bool pv_prev = wave_active && t - 1 <= wave_last;
    const bool full = (t + 1) * kTileKV <= N && (!CAUSAL || t * kTileKV + kTileKV - 1 <= qw);

    if constexpr (VARIANT >= 2) {
      cn[0] = cn[1] = a.kscale;
    } else {
      cn[0] = dqs * (KT ? kq[0] : kscale_of(kq, 0, h));  // tile t+1
      cn[1] = dqs * (KT ? kq[0] : kscale_of(kq, 1, h));
    }
    if (t + 2 < T) copy.k_tile(krs, t + 2, sKc);
    if (SMOOTHQ && t + 1 < T)
      smooth_q_bias<D>(sKn, sQl, sQs, a.kscale * kscale_quarter(ksc, t + 1, wave_id(), last_key, kshift), sBn);

    float alpha = 1.0f;
    bool rescale = false;
    const float* bias = SMOOTHQ ? sBc + ((qw - q0) >> qshift) * kTileKV + 16 * h : nullptr;
    const int kl = t * kTileKV + (VARIANT == 3 ? 32 : 16) * h;  // key of register 0 of this lane
    if (compute && compute_next && pv_prev && full) {
      // Interior tile: one basic block, MFMA work (S(t+1), P~(t-1) V(t-1)) interleaved
      // with the softmax of tile t so the matrix and vector units run together.
      // variant 0: a wave inside its interleaved block gets issue priority over the other
      // wave of the SIMD while that one copies tiles or waits at a barrier (1-2 % at
      // d = 128, neutral at d = 64; variant 1 measured slower with it)
      if constexpr (VARIANT == 0) __builtin_amdgcn_s_setprio(3);
      if constexpr (VARIANT != 0) {
        pv_tile(sVp, pkp, psp, vsc[cur ^ 1]);
        score_tile(sKn, sn);
        softmax_tile<VARIANT, CAUSAL, SMOOTHQ, false, VARIANT == 3>(s, c, bias, kl, N, qi, m, l, pk, alpha, rescale,
                                                                     kLazyLog2, psc);
        interleave_schedule<D, VARIANT, SMOOTHQ>();
        // variant 3: a P~ block with scale code 0 is repaired at the start of the next
        // iteration, ahead of its interleaved block (a branch here would split this one)
        if constexpr (VARIANT == 3) fp4_fix_pending = __builtin_amdgcn_ballot_w64(*psc == 0u) != 0;
      } else if constexpr (!SMOOTHQ) {
        // (at d = 64 this holds the kernel to two waves per SIMD, 197 VGPRs: 3-5 % faster
        // than the general softmax at three waves, which would spill under a 168 cap)
        score_tile(sKn, sn);
        pv_tile(sVp, pkp);
        const bool slow = softmax_tile_fast<!TRAIN>(s, c, m, l, pk);
        interleave_schedule<D, VARIANT, SMOOTHQ>();
        __builtin_amdgcn_s_setprio(0);
        // the reference moves to the row maximum (rare after a row's first tiles)
        if (slow)
          softmax_tile<VARIANT, CAUSAL, SMOOTHQ, false, false, !TRAIN>(s, c, bias, kl, N, qi, m, l, pk, alpha, rescale,
                                                                      0.0f);
      } else {
        score_tile(sKn, sn);
        pv_tile(sVp, pkp);
        softmax_tile<VARIANT, CAUSAL, SMOOTHQ, false>(s, c, bias, kl, N, qi, m, l, pk, alpha, rescale);
        interleave_schedule<D, VARIANT, SMOOTHQ>();
        __builtin_amdgcn_s_setprio(0);
      }
    } else {
      if (compute_next) score_tile(sKn, sn);
      if (pv_prev) pv_tile(sVp, pkp, psp, vsc[cur ^ 1]);
      if (compute) {
        if (full)
          softmax_tile<VARIANT, CAUSAL, SMOOTHQ, false, false, !TRAIN>(s, c, bias, kl, N, qi, m, l, pk, alpha,
                                                                       rescale, kLazyLog2, psc);
        else
          softmax_tile<VARIANT, CAUSAL, SMOOTHQ, true, false, !TRAIN>(s, c, bias, kl, N, qi, m, l, pk, alpha,
                                                                      rescale, kLazyLog2, psc);
      }
    }
    if (rescale) {  // O already holds P~(t-1) V(t-1)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) o[ct] *= alpha;
    }

    // K scales of tile t+2 for the next iteration: issued here, their latency overlaps
    // the barrier
    if constexpr (VARIANT >= 2)
      mx_kscales(t + 2, kw);
    else
      tile_kscales_for<KT>(ksc, t + 2, last_key, kshift, kq);
    if (t < T) {
      wait_copies();
      __syncthreads();
      if (t + 1 < T) {
        copy.v_tile(vrs, t + 1, a.Np, sVp);
        if constexpr (VARIANT == 3) vsc[cur ^ 1] = v_scales(t + 1);  // read with V(t+1) at iteration t+2
      }
    }
  };

  for (int t = 0; t <= T; t += 2) {
    iteration(t, std::integral_constant<int, 0>{});
    if (t + 1 <= T) iteration(t + 1, std::integral_constant<int, 1>{});
  }

  if (!wave_active) return;
  l = pair_sum(l);
  const float inv = 1.0f / l;
  if (qi >= N) return;
  // training: the row log-sum-exp, log(sum_j e^(s_ij)) = ln2 * (m + log2 l) (m and l are in
  // base-2 units; variants 1 and 2 count P~ * 448)
  if (a.lse && h == 0)
    a.lse[(size_t)g * N + qi] =
        0.6931471805599453f * (m + __builtin_amdgcn_logf(l) - (VARIANT == 1 || VARIANT == 2 ? kLog2_448 : 0.0f));
  uint16_t* orow = a.o + ((size_t)g * N + qi) * D;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int c0 = ct * 32 + 8 * a4 + 4 * h;
      float y[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) y[b] = o[ct][4 * a4 + b] * inv;
      if (VARIANT == 1 || VARIANT == 2) {  // variant 3's V scales sit inside the product
        const float4 dv = *reinterpret_cast<const float4*>(a.v_scale + (size_t)g * D + c0);
        y[0] *= dv.x; y[1] *= dv.y; y[2] *= dv.z; y[3] *= dv.w;
      }
      if (VARIANT != 0) {
        if (a.v_mean) {  // V smoothing: every row of P~ sums to one after the division by l
          const float4 vm = *reinterpret_cast<const float4*>(a.v_mean + (size_t)g * D + c0);
          y[0] += vm.x; y[1] += vm.y; y[2] += vm.z; y[3] += vm.w;
        }
      }
      *reinterpret_cast<uint2*>(orow + c0) = make_uint2(pack_f16x2(y[0], y[1]), pack_f16x2(y[2], y[3]));
    }
}

// The int32 score tiles the attention kernel forms (test surface): same loads, same
// qk_tile.  tiles[3i..3i+2] = (head, query tile of 128, key tile of 64).
// A tile entry outside the tensors yields a tile of zeros.
template <int D>
__global__ __launch_bounds__(64 * kDbgWaves) void debug_qk_kernel(const int8_t* __restrict__ q_i8,
                                                            const int8_t* __restrict__ k_i8, int G, int Np,
                                                            const int* __restrict__ tiles,
                                                            int32_t* __restrict__ s_out) {
  __shared__ __attribute__((aligned(16))) int8_t sK[Lds<D, 0>::K_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, ql = lane & 31;
  const int g = tiles[3 * blockIdx.x], qt = tiles[3 * blockIdx.x + 1], kt = tiles[3 * blockIdx.x + 2];
  if (g < 0 || g >= G || qt < 0 || qt >= Np / kBlockQ || kt < 0 || kt >= Np / kTileKV) {
    int32_t* out = s_out + (size_t)blockIdx.x * kBlockQ * kTileKV;
    for (int e = tid; e < kBlockQ * kTileKV; e += 64 * kDbgWaves) out[e] = 0;
    return;
  }
  const int8_t* qh = q_i8 + (size_t)g * Np * D;
  const int8_t* kh = k_i8 + (size_t)g * Np * D;
  __shared__ __attribute__((aligned(16))) int8_t sQ[64 * kDbgWaves / 2 * D];
  const TileCopy<D, 0, kDbgWaves> copy(Np);
  copy.k_tile(make_rsrc(kh, (size_t)Np * D), kt, sK);
  int8_t* const sQw = sQ + wave * (D / 32) * 1024;
  load_q_tile<D>(make_rsrc(qh, (size_t)Np * D), qt * kBlockQ + 32 * wave, sQw);
  wait_copies();
  __syncthreads();
  i32x16 s[2];
  qk_tile<D>(sK, sQw, lane, s);
  int32_t* out = s_out + (size_t)blockIdx.x * kBlockQ * kTileKV + (size_t)(32 * wave + ql) * kTileKV;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      *reinterpret_cast<int4*>(out + 32 * st + 16 * h + i) = make_int4(s[st][i], s[st][i + 1], s[st][i + 2], s[st][i + 3]);
}

// ---------------------------------------------------------------------------
// launchers

template <int D, int VARIANT, bool CAUSAL, bool SMOOTHQ, bool FUSEQ = false, bool TRAIN = false>
static hipError_t launch_one(const AttnArgs& a, hipStream_t st) {
  const int grid = a.G * ((a.Np + kAttnRows - 1) / kAttnRows);
  if constexpr (VARIANT <= 1 && FUSEQ) {
    if (a.blk_k >= kTileKV) {
      attn_kernel<D, VARIANT, CAUSAL, SMOOTHQ, FUSEQ, TRAIN, true><<<grid, kAttnThreads, 0, st>>>(a);
      return hipGetLastError();
    }
  }
  attn_kernel<D, VARIANT, CAUSAL, SMOOTHQ, FUSEQ, TRAIN><<<grid, kAttnThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int VARIANT>
static hipError_t launch_dv(int causal, int smooth_q, const AttnArgs& a, hipStream_t st) {
  if (causal)
    return smooth_q ? launch_one<D, VARIANT, true, true>(a, st) : launch_one<D, VARIANT, true, false>(a, st);
  return smooth_q ? launch_one<D, VARIANT, false, true>(a, st) : launch_one<D, VARIANT, false, false>(a, st);
}

hipError_t launch_attn(int d, int variant, int causal, int smooth_q, const AttnArgs& a, hipStream_t st) {
  if (a.q) {  // fp16 Q, quantised in the kernel (variants 0 and 1 with or without Q smoothing, 2, 3)
    if (variant <= 1) {
      auto one = [&](auto dc, auto vc) -> hipError_t {
        constexpr int DD = decltype(dc)::value, VV = decltype(vc)::value;
        if constexpr (VV == 0) {
          if (a.lse && !smooth_q)  // the training forward
            return causal ? launch_one<DD, 0, true, false, true, true>(a, st)
                          : launch_one<DD, 0, false, false, true, true>(a, st);
        }
        if (causal)
          return smooth_q ? launch_one<DD, VV, true, true, true>(a, st) : launch_one<DD, VV, true, false, true>(a, st);
        return smooth_q ? launch_one<DD, VV, false, true, true>(a, st) : launch_one<DD, VV, false, false, true>(a, st);
      };
      if (d == 64)
        return variant == 0 ? one(std::integral_constant<int, 64>{}, std::integral_constant<int, 0>{})
                            : one(std::integral_constant<int, 64>{}, std::integral_constant<int, 1>{});
      return variant == 0 ? one(std::integral_constant<int, 128>{}, std::integral_constant<int, 0>{})
                          : one(std::integral_constant<int, 128>{}, std::integral_constant<int, 1>{});
    }
    if (smooth_q) return hipErrorInvalidValue;
    if (variant == 3) {
      if (d == 64) return causal ? launch_one<64, 3, true, false, true>(a, st) : launch_one<64, 3, false, false, true>(a, st);
      return causal ? launch_one<128, 3, true, false, true>(a, st) : launch_one<128, 3, false, false, true>(a, st);
    }
    if (variant == 2) {
      if (d == 64) return causal ? launch_one<64, 2, true, false, true>(a, st) : launch_one<64, 2, false, false, true>(a, st);
      return causal ? launch_one<128, 2, true, false, true>(a, st) : launch_one<128, 2, false, false, true>(a, st);
    }
    return hipErrorInvalidValue;
  }
  if (variant == 3) return hipErrorInvalidValue;  // variant 3 always quantises Q in the kernel
  if (variant == 2) {  // MXFP4 scores, never with Q smoothing
    if (smooth_q) return hipErrorInvalidValue;
    if (d == 64) return causal ? launch_one<64, 2, true, false>(a, st) : launch_one<64, 2, false, false>(a, st);
    return causal ? launch_one<128, 2, true, false>(a, st) : launch_one<128, 2, false, false>(a, st);
  }
  if (d == 64)
    return variant == 0 ? launch_dv<64, 0>(causal, smooth_q, a, st) : launch_dv<64, 1>(causal, smooth_q, a, st);
  return variant == 0 ? launch_dv<128, 0>(causal, smooth_q, a, st) : launch_dv<128, 1>(causal, smooth_q, a, st);
}

hipError_t launch_debug_qk(int d, const int8_t* q_i8, const int8_t* k_i8, int G, int Np, const int* tiles,
                           int n_tiles, int32_t* s_out, hipStream_t st) {
  if (d == 64)
    debug_qk_kernel<64><<<n_tiles, 64 * kDbgWaves, 0, st>>>(q_i8, k_i8, G, Np, tiles, s_out);
  else
    debug_qk_kernel<128><<<n_tiles, 64 * kDbgWaves, 0, st>>>(q_i8, k_i8, G, Np, tiles, s_out);
  return hipGetLastError();
}

}  // namespace sage
