// sage_internal.h -- launcher interface between the C ABI (sage_api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

struct QuantArgs {
  const uint16_t* q;  // [G][N][D] fp16
  const uint16_t* k;
  int8_t* q_i8;       // [G][Np][D]
  int8_t* k_i8;
  float* q_scale;     // [G][nqg]
  float* k_scale;     // [G][nkb]
  float* k_mean;      // [G][D] or null
  float* q_mean;      // [G][nqb][D] or null
  const long long* ksum_part;  // [G][nsplit][D] from the statistics pass
  int G, N, Np, blk_q, blk_k, nqb, nkb, nsplit, smooth_k, smooth_q;
  int q_group, nqg;   // rows per Q scale (divides blk_q) and Q scales per head
  int with_q;         // 0: quantise only K
};

struct AttnArgs {
  const uint16_t* q;      // [G][N][D] fp16 (Q quantised in the kernel) or null
  const int8_t* q_i8;     // [G][Np][D] (pre-quantised Q)
  const int8_t* k_i8;     // [G][Np][D]
  const float* q_scale;   // [G][nqg]
  const float* k_scale;   // [G][nkb]
  const float* q_mean;    // [G][nqb][D] (variant 1 with Q smoothing)
  const uint16_t* v;      // [G][N][D] fp16 (variant 0)
  const uint8_t* v_f8;    // [G][D][Np] (variants 1, 2); variant 3: [G][D][Np/2] E2M1 pairs
  const uint8_t* v_e8;    // [G][Np/32][D] MX scales of V (variant 3)
  const float* v_scale;   // [G][D] (variant 1)
  const float* v_mean;    // [G][D] (variants 1, 2 with V smoothing) or null
  const uint8_t* q_e8;    // [G][Np][D/32] MX block scales (variant 2; q_i8 / k_i8 then
  const uint8_t* k_e8;    //  hold [G][Np][D/2] bytes of two E2M1 codes each)
  uint16_t* o;            // [G][N][D] fp16
  float* lse;             // [G][N] row log-sum-exp of the dequantised scores (natural log), or null
  int G, N, Np, blk_q, blk_k, nqb, nkb;
  int q_group, nqg;       // rows per Q scale (a power of two dividing blk_q), scales per head
  float kscale;           // sm_scale * log2(e)
};

// token rows per workgroup of the statistics pass; the workspace holds one partial
// sum per (head, split of kStatRows tokens, channel)
constexpr int kStatRows = 256;
int stat_splits(int N);
// Statistics pass outputs, [G][nsplit][D] each, folded into split 0 by the pass; the V
// max and min are only written when V is given, the V sums only with v_sums.
struct StatsOut {
  long long* ksum;  // exact sums of K in units of 2^-24
  long long* vsum;  // the same for V
  float* vmax;      // max of V per channel
  float* vmin;      // min of V per channel
};
hipError_t launch_stats(int d, const void* k, const void* v, bool v_sums, int G, int N, const StatsOut& out,
                        hipStream_t st);
hipError_t launch_quant(int d, const QuantArgs& a, hipStream_t st);
hipError_t launch_quant_v(int d, const void* v, int G, int N, int Np, const StatsOut& stats, int smooth_v,
                          uint8_t* v_f8, float* v_scale, float* v_mean, hipStream_t st);
// Variant 2: per-token MXFP4 of x (Q, or K with smooth = 1 and the statistics pass's
// sums): codes [G][Np][D/2] (two E2M1 per byte), e8 [G][Np][D/32]; rows >= N zero.
hipError_t launch_quant_mx(int d, const void* x, int G, int N, int Np, const long long* ksum_part, int smooth,
                           uint8_t* codes, uint8_t* e8, float* k_mean, hipStream_t st);
// Variant 3: V to MXFP4 along the tokens, v_f4 [G][D][Np/2] (two E2M1 per byte),
// v_e8 [G][Np/32][D] (channel c at (c % 32) * (D/32) + c / 32); vsum_part from the
// statistics pass (used with smooth_v).
hipError_t launch_quant_v_mx(int d, const void* v, int G, int N, int Np, const long long* vsum_part, int smooth_v,
                             uint8_t* v_f4, uint8_t* v_e8, float* v_mean, hipStream_t st);
hipError_t launch_attn(int d, int variant, int causal, int smooth_q, const AttnArgs& a, hipStream_t st);
// Backward (sage_bwd.hip).  Inputs [G][N][D] fp16 unless noted; the workspace pieces are
// filled by the statistics pass (ksum, vsum), the quantisation pass (q_i8, k_i8 and their
// scales, variant-0 rules) and the preparation kernel (the rest).
struct BwdArgs {
  const uint16_t *q, *k, *v, *o, *dout;
  const float* lse;            // [G][N] natural-log row log-sum-exp of the forward
  const int8_t *q_i8, *k_i8;   // [G][Np][D] forward codes
  const float *q_scale, *k_scale;
  const long long *ksum, *vsum;  // [G][nsplit][D], split 0 = the head's exact sums
  int8_t *v_i8, *do_i8;        // [G][Np][D] per-token INT8 of V' and dO
  float *v_scale, *do_scale;   // [G][Np]
  float *dvec, *lse2;          // [G][Np]: D' per row; log2-sum-exp (+inf on pad rows)
  float* nrm;                  // [G][Np/64][2]: max |dO_i|, max |V'_j| per 64 rows
  uint16_t* kp;                // [G][Np][D] K' = K - kmean in fp16, pad rows zero
  float *dq, *dk, *dv;         // [G][N][D] fp32 outputs
  int G, N, Np, blk_q, blk_k, nqb, nkb, nsplit, smooth_k;
  float kscale, sm_scale;      // sm_scale * log2(e), sm_scale
};
hipError_t launch_bwd(int d, int causal, const BwdArgs& a, hipStream_t st);

hipError_t launch_debug_qk(int d, const int8_t* q_i8, const int8_t* k_i8, int G, int Np, const int* tiles,
                           int n_tiles, int32_t* s_out, hipStream_t st);

}  // namespace sage
