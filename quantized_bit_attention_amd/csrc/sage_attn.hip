// sage_attn.hip -- fused 8-bit attention forward for gfx950 (CDNA4).
//
// Method: "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
// Acceleration" (summary page: "Summary", "Interesting ideas" I3): INT8 Q K^T,
// FlashAttention-style tiling with an online softmax, P~ V in FP16.
// "SageAttention2 ..." (abstract): FP8 P~ and V with two-level accumulation, and the
// Q-smoothing term added back to the scores.
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
//  - O is kept transposed, O^T = V^T P^T: P~ (converted in registers) is the B
//    operand as it stands; V^T comes from row-major LDS through ds_read_b64_tr_b16
//    (variant 0, fp16, v_mfma_f32_32x32x16_f16) or from the key-contiguous FP8 V^T
//    (variant 1, v_mfma_f32_32x32x64_f8f6f4).
//  - Causal: tiles past a wave's last row are skipped; workgroups run
//    longest-first and consecutive workgroups of one head stay on one XCD.
#include "sage_device.h"
#include "sage_internal.h"

namespace sage {

template <int D, int VARIANT>
struct Lds {
  static constexpr int KROW = D + 16;            // bytes per K row (padding breaks bank conflicts)
  static constexpr int VROW = D + 16;            // halves per V row (variant 0)
  static constexpr int VTROW = kTileKV + 16;     // bytes per V^T row (variant 1)
  static constexpr int K_BYTES = kTileKV * KROW;
  static constexpr int V_BYTES = VARIANT == 0 ? kTileKV * VROW * 2 : D * VTROW;
  static constexpr int K_CHUNKS = kTileKV * D / 16 / kThreads;                          // 16 B per thread
  static constexpr int V_CHUNKS = (VARIANT == 0 ? kTileKV * D * 2 : D * kTileKV) / 16 / kThreads;
};

// Row of the K tile that feeds A-operand row r: accumulator register i of lane half h
// then holds key 16h + i of the 32-key block.
__device__ __forceinline__ int k_perm(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

template <int D, int VARIANT>
__device__ __forceinline__ void load_k_tile(const int8_t* __restrict__ kh, int t, i32x4* reg) {
  using L = Lds<D, VARIANT>;
#pragma unroll
  for (int i = 0; i < L::K_CHUNKS; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int row = c / (D / 16), col = (c % (D / 16)) * 16;
    reg[i] = *reinterpret_cast<const i32x4*>(kh + (size_t)(t * kTileKV + row) * D + col);
  }
}
template <int D, int VARIANT>
__device__ __forceinline__ void store_k_tile(int8_t* sK, const i32x4* reg) {
  using L = Lds<D, VARIANT>;
#pragma unroll
  for (int i = 0; i < L::K_CHUNKS; ++i) {
    const int c = threadIdx.x + kThreads * i;
    const int row = c / (D / 16), col = (c % (D / 16)) * 16;
    *reinterpret_cast<i32x4*>(sK + row * L::KROW + col) = reg[i];
  }
}

// V tile t into registers.  Variant 0: fp16 rows [key][D] of the caller's V, keys >= N
// read as zero.  Variant 1: FP8 V^T rows [channel][64 keys] of the padded tensor.
template <int D, int VARIANT>
__device__ __forceinline__ void load_v_tile(const void* __restrict__ vh, int t, int N, int Np, i32x4* reg) {
  using L = Lds<D, VARIANT>;
#pragma unroll
  for (int i = 0; i < L::V_CHUNKS; ++i) {
    const int c = threadIdx.x + kThreads * i;
    if (VARIANT == 0) {
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      const int key = t * kTileKV + row;
      reg[i] = key < N ? *reinterpret_cast<const i32x4*>((const uint16_t*)vh + (size_t)key * D + col)
                       : i32x4{0, 0, 0, 0};
    } else {
      const int row = c / 4, col = (c % 4) * 16;
      reg[i] = *reinterpret_cast<const i32x4*>((const uint8_t*)vh + (size_t)row * Np + t * kTileKV + col);
    }
  }
}
template <int D, int VARIANT>
__device__ __forceinline__ void store_v_tile(uint8_t* sV, const i32x4* reg) {
  using L = Lds<D, VARIANT>;
#pragma unroll
  for (int i = 0; i < L::V_CHUNKS; ++i) {
    const int c = threadIdx.x + kThreads * i;
    if (VARIANT == 0) {
      const int row = c / (D / 8), col = (c % (D / 8)) * 8;
      *reinterpret_cast<i32x4*>(sV + (row * L::VROW + col) * 2) = reg[i];
    } else {
      const int row = c / 4, col = (c % 4) * 16;
      *reinterpret_cast<i32x4*>(sV + row * L::VTROW + col) = reg[i];
    }
  }
}

// Q operand (B of S^T = K Q^T) for this lane's query row: D/32 k-steps of 16 bytes.
template <int D>
__device__ __forceinline__ void load_q_operand(const int8_t* __restrict__ qh, int row, int h, i32x4* qop) {
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    qop[ks] = *reinterpret_cast<const i32x4*>(qh + (size_t)row * D + 32 * ks + 16 * h);
}

// S^T for the 64-key tile in LDS: s[st][i] = Qhat[query l%32] . Khat[key 32*st + 16h + i]
// (exact int32).
template <int D, int VARIANT>
__device__ __forceinline__ void qk_tile(const int8_t* sK, const i32x4* qop, int lane, i32x16* s) {
  using L = Lds<D, VARIANT>;
  const int ql = lane & 31, h = lane >> 5;
  const int pr = k_perm(ql);
#pragma unroll
  for (int st = 0; st < 2; ++st) {
    i32x16 acc = {};
    const int8_t* kr = sK + (32 * st + pr) * L::KROW + 16 * h;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
      acc = mfma_i8(*reinterpret_cast<const i32x4*>(kr + 32 * ks), qop[ks], acc);
    s[st] = acc;
  }
}

// Online-softmax update for one 64-key tile of one lane (one query, 32 keys:
// s[st][i] is key kl + 32*st + i).  Works in the exp2 domain: x = S * c (+ bias),
// c = dQ * dK * sm_scale * log2(e).  Updates the running max m and the lane's partial
// sum l (the lane pair l, l^32 shares m; l is summed over the pair at the end), writes
// P~ (variant 0) or P~ * 448 (variant 1, ready for FP8) and the rescale factor alpha.
// MASK: keys >= N, and keys > qi when causal, get P~ = 0 and stay out of the max.
template <int VARIANT, bool CAUSAL, bool SMOOTHQ, bool MASK>
__device__ __forceinline__ void softmax_tile(const i32x16* s, const float* c, const float* bias, int kl, int N,
                                             int qi, float& m, float& l, float (&p)[2][16], float& alpha) {
  auto keep = [&](int st, int i) {
    const int key = kl + 32 * st + i;
    return !MASK || (key < N && (!CAUSAL || key <= qi));
  };
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
  } else {
    // c >= 0, so max_j fl(c * S_j) = fl(c * max_j S_j): the max is taken on the integers
    int mi[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      mi[st] = INT_MIN;
#pragma unroll
      for (int i = 0; i < 16; ++i) mi[st] = keep(st, i) ? max(mi[st], s[st][i]) : mi[st];
    }
    const float m0 = (MASK && mi[0] == INT_MIN) ? -INFINITY : c[0] * (float)mi[0];
    const float m1 = (MASK && mi[1] == INT_MIN) ? -INFINITY : c[1] * (float)mi[1];
    mt = fmaxf(m0, m1);
  }
  mt = pair_max(mt);
  const float mnew = fmaxf(m, mt);  // finite: key 0 (tile 0) is visible to every row
  alpha = exp2f(m - mnew);
  m = mnew;
  const float shift = VARIANT == 0 ? -mnew : kLog2_448 - mnew;
  float psum = 0.0f;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float e = SMOOTHQ ? x[st][i] + shift : fmaf((float)s[st][i], c[st], shift);
      float pv = __builtin_amdgcn_exp2f(e);
      if (MASK) pv = keep(st, i) ? pv : 0.0f;
      p[st][i] = pv;
      psum += pv;
    }
  l = alpha * l + psum;
}

template <int D, int VARIANT, bool CAUSAL, bool SMOOTHQ>
__global__ __launch_bounds__(kThreads, 2) void attn_kernel(AttnArgs a) {
  using L = Lds<D, VARIANT>;
  constexpr int NCT = D / 32;                       // 32-channel output tiles
  constexpr int NSUB = SMOOTHQ ? 4 : 1;             // Q blocks a workgroup can span (blk_q >= 32)
  __shared__ __attribute__((aligned(16))) int8_t sK[L::K_BYTES];
  __shared__ __attribute__((aligned(16))) uint8_t sV[L::V_BYTES];
  __shared__ __attribute__((aligned(16))) float sQm[SMOOTHQ ? NSUB * D : 1];
  __shared__ float sBias[SMOOTHQ ? NSUB * kTileKV : 1];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, ql = lane & 31;
  const int N = a.N;

  // workgroup -> (head, query tile).  Consecutive workgroup ids go round-robin over the
  // 8 XCDs; remap so each XCD walks a contiguous range of (head, tile) pairs, heads
  // one after another, and for causal the longest tiles of a head first.
  const int nqt = a.Np / kBlockQ;
  const int total = a.G * nqt;
  int vid = blockIdx.x;
  if ((total & 7) == 0) vid = (blockIdx.x & 7) * (total >> 3) + (blockIdx.x >> 3);
  const int g = vid / nqt;
  const int qt = CAUSAL ? nqt - 1 - vid % nqt : vid % nqt;
  const int q0 = qt * kBlockQ;
  const int qw = q0 + 32 * wave;  // first row of this wave
  const int qi = qw + ql;         // this lane's query row
  const bool wave_active = qw < N;

  const int8_t* __restrict__ qh = a.q_i8 + (size_t)g * a.Np * D;
  const int8_t* __restrict__ kh = a.k_i8 + (size_t)g * a.Np * D;
  const void* vh = VARIANT == 0 ? (const void*)(a.v + (size_t)g * N * D)
                                : (const void*)(a.v_f8 + (size_t)g * D * a.Np);
  const float* __restrict__ ksc = a.k_scale + (size_t)g * a.nkb;

  const int ntiles_all = (N + kTileKV - 1) / kTileKV;
  const int wg_last_row = min(q0 + kBlockQ - 1, N - 1);
  const int ntiles = CAUSAL ? min(ntiles_all, wg_last_row / kTileKV + 1) : ntiles_all;
  const int wave_last_tile = CAUSAL ? min(ntiles_all - 1, min(qw + 31, N - 1) / kTileKV) : ntiles_all - 1;

  i32x4 qop[D / 32];
  load_q_operand<D>(qh, qi, h, qop);
  const float dq = wave_active ? a.q_scale[(size_t)g * a.nqb + qw / a.blk_q] : 0.0f;

  if (SMOOTHQ) {
    // block means of the (up to 4) Q blocks this workgroup's rows belong to
    for (int e = tid; e < NSUB * D; e += kThreads) {
      const int sb = e / D, c = e % D;
      const int qb = (q0 + sb * a.blk_q) / a.blk_q;
      sQm[e] = (sb * a.blk_q < kBlockQ && qb < a.nqb) ? a.q_mean[((size_t)g * a.nqb + qb) * D + c] : 0.0f;
    }
  }

  f32x16 o[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) o[ct] = f32x16{};
  float m = -INFINITY, l = 0.0f;

  i32x4 kreg[L::K_CHUNKS], vreg[L::V_CHUNKS];
  load_k_tile<D, VARIANT>(kh, 0, kreg);
  load_v_tile<D, VARIANT>(vh, 0, N, a.Np, vreg);

  for (int t = 0; t < ntiles; ++t) {
    __syncthreads();  // every wave is done with the previous tile in LDS
    store_k_tile<D, VARIANT>(sK, kreg);
    store_v_tile<D, VARIANT>(sV, vreg);
    __syncthreads();
    if (t + 1 < ntiles) {  // next tile's global loads overlap this tile's math
      load_k_tile<D, VARIANT>(kh, t + 1, kreg);
      load_v_tile<D, VARIANT>(vh, t + 1, N, a.Np, vreg);
    }

    if (SMOOTHQ) {
      // Q-smoothing term of every key of the tile for each Q block of the workgroup:
      // bias[sb][j] = sm_scale*log2(e) * dK_j * (qmean_sb . Khat_j), in fp32.
      constexpr int CH = D / 32;  // 32-channel chunks per key, summed across adjacent lanes
      const int nsub = kBlockQ / a.blk_q;
      for (int item = tid; item < nsub * kTileKV * CH; item += kThreads) {
        const int chunk = item % CH, key = (item / CH) % kTileKV, sb = item / (CH * kTileKV);
        const int8_t* kr = sK + key * L::KROW + chunk * 32;
        const float* qm = sQm + sb * D + chunk * 32;
        float acc = 0.0f;
#pragma unroll
        for (int c = 0; c < 32; ++c) acc = fmaf(qm[c], (float)kr[c], acc);
        for (int off = 1; off < CH; off <<= 1) acc += __shfl_xor(acc, off);
        if (chunk == 0) {
          const int kj = min(t * kTileKV + key, N - 1);
          sBias[sb * kTileKV + key] = a.kscale * ksc[kj / a.blk_k] * acc;
        }
      }
      __syncthreads();
    }

    if (!wave_active || t > wave_last_tile) continue;

    i32x16 s[2];
    qk_tile<D, VARIANT>(sK, qop, lane, s);

    const bool full = (t + 1) * kTileKV <= N && (!CAUSAL || t * kTileKV + kTileKV - 1 <= qw);
    float c[2];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int kb = min(t * kTileKV + 32 * st + 16 * h, N - 1) / a.blk_k;
      c[st] = dq * ksc[kb] * a.kscale;
    }

    float p[2][16];
    float alpha;
    const float* bias = SMOOTHQ ? sBias + ((qw - q0) / a.blk_q) * kTileKV + 16 * h : nullptr;
    const int kl = t * kTileKV + 16 * h;  // key of register 0 of this lane
    if (full)
      softmax_tile<VARIANT, CAUSAL, SMOOTHQ, false>(s, c, bias, kl, N, qi, m, l, p, alpha);
    else
      softmax_tile<VARIANT, CAUSAL, SMOOTHQ, true>(s, c, bias, kl, N, qi, m, l, p, alpha);

    if (VARIANT == 0) {
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) o[ct] *= alpha;
      const _Float16* sVh = reinterpret_cast<const _Float16*>(sV);
      const int G16 = lane >> 4, j16 = lane & 15;
#pragma unroll
      for (int st = 0; st < 2; ++st)
#pragma unroll
        for (int u = 0; u < 2; ++u) {
          uint32_t pk[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) pk[q] = pack_f16x2(p[st][8 * u + 2 * q], p[st][8 * u + 2 * q + 1]);
          const f16x8 pb = __builtin_bit_cast(f16x8, pk);
          const int row = 32 * st + 16 * (G16 >> 1) + 8 * u + (j16 >> 2);
#pragma unroll
          for (int ct = 0; ct < NCT; ++ct) {
            const int col = ct * 32 + 16 * (G16 & 1) + 4 * (j16 & 3);
            const i16x4 a0 = lds_read_tr16(sVh + row * L::VROW + col);
            const i16x4 a1 = lds_read_tr16(sVh + (row + 4) * L::VROW + col);
            const i16x4 a01[2] = {a0, a1};
            o[ct] = mfma_f16(__builtin_bit_cast(f16x8, a01), pb, o[ct]);
          }
        }
    } else {
      uint32_t pk[8];
#pragma unroll
      for (int w = 0; w < 8; ++w) {
        const int st = w / 4, b = 4 * (w % 4);
        const uint32_t lo = cvt_pk_fp8(p[st][b], p[st][b + 1], 0u, false);
        pk[w] = cvt_pk_fp8(p[st][b + 2], p[st][b + 3], lo, true);
      }
      const i32x8 pb = __builtin_bit_cast(i32x8, pk);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const uint8_t* vr = sV + (ct * 32 + ql) * L::VTROW + 16 * h;
        const i32x4 v0 = *reinterpret_cast<const i32x4*>(vr);
        const i32x4 v1 = *reinterpret_cast<const i32x4*>(vr + 32);
        const i32x4 vv[2] = {v0, v1};
        const f32x16 inner = mfma_f8(__builtin_bit_cast(i32x8, vv), pb, f32x16{});  // fresh per tile
#pragma unroll
        for (int i = 0; i < 16; ++i) o[ct][i] = fmaf(alpha, o[ct][i], inner[i]);
      }
    }
  }

  if (!wave_active) return;
  l = pair_sum(l);
  const float inv = 1.0f / l;
  if (qi >= N) return;
  uint16_t* orow = a.o + ((size_t)g * N + qi) * D;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int c0 = ct * 32 + 8 * a4 + 4 * h;
      float y[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) y[b] = o[ct][4 * a4 + b] * inv;
      if (VARIANT == 1) {
        const float4 dv = *reinterpret_cast<const float4*>(a.v_scale + (size_t)g * D + c0);
        y[0] *= dv.x; y[1] *= dv.y; y[2] *= dv.z; y[3] *= dv.w;
      }
      *reinterpret_cast<uint2*>(orow + c0) = make_uint2(pack_f16x2(y[0], y[1]), pack_f16x2(y[2], y[3]));
    }
}

// The int32 score tiles the attention kernel forms (test surface): same loads, same
// qk_tile.  tiles[3i..3i+2] = (head, query tile of 128, key tile of 64).
// A tile entry outside the tensors yields a tile of zeros.
template <int D>
__global__ __launch_bounds__(kThreads) void debug_qk_kernel(const int8_t* __restrict__ q_i8,
                                                            const int8_t* __restrict__ k_i8, int G, int Np,
                                                            const int* __restrict__ tiles,
                                                            int32_t* __restrict__ s_out) {
  using L = Lds<D, 0>;
  __shared__ __attribute__((aligned(16))) int8_t sK[L::K_BYTES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, ql = lane & 31;
  const int g = tiles[3 * blockIdx.x], qt = tiles[3 * blockIdx.x + 1], kt = tiles[3 * blockIdx.x + 2];
  if (g < 0 || g >= G || qt < 0 || qt >= Np / kBlockQ || kt < 0 || kt >= Np / kTileKV) {
    int32_t* out = s_out + (size_t)blockIdx.x * kBlockQ * kTileKV;
    for (int e = tid; e < kBlockQ * kTileKV; e += kThreads) out[e] = 0;
    return;
  }
  const int8_t* qh = q_i8 + (size_t)g * Np * D;
  const int8_t* kh = k_i8 + (size_t)g * Np * D;
  i32x4 kreg[L::K_CHUNKS];
  load_k_tile<D, 0>(kh, kt, kreg);
  store_k_tile<D, 0>(sK, kreg);
  __syncthreads();
  i32x4 qop[D / 32];
  load_q_operand<D>(qh, qt * kBlockQ + 32 * wave + ql, h, qop);
  i32x16 s[2];
  qk_tile<D, 0>(sK, qop, lane, s);
  int32_t* out = s_out + (size_t)blockIdx.x * kBlockQ * kTileKV + (size_t)(32 * wave + ql) * kTileKV;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int i = 0; i < 16; i += 4)
      *reinterpret_cast<int4*>(out + 32 * st + 16 * h + i) = make_int4(s[st][i], s[st][i + 1], s[st][i + 2], s[st][i + 3]);
}

// ---------------------------------------------------------------------------
// launchers

template <int D, int VARIANT, bool CAUSAL, bool SMOOTHQ>
static hipError_t launch_one(const AttnArgs& a, hipStream_t st) {
  const int grid = a.G * (a.Np / kBlockQ);
  attn_kernel<D, VARIANT, CAUSAL, SMOOTHQ><<<grid, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

template <int D, int VARIANT>
static hipError_t launch_dv(int causal, int smooth_q, const AttnArgs& a, hipStream_t st) {
  if (causal)
    return smooth_q ? launch_one<D, VARIANT, true, true>(a, st) : launch_one<D, VARIANT, true, false>(a, st);
  return smooth_q ? launch_one<D, VARIANT, false, true>(a, st) : launch_one<D, VARIANT, false, false>(a, st);
}

hipError_t launch_attn(int d, int variant, int causal, int smooth_q, const AttnArgs& a, hipStream_t st) {
  if (d == 64)
    return variant == 0 ? launch_dv<64, 0>(causal, smooth_q, a, st) : launch_dv<64, 1>(causal, smooth_q, a, st);
  return variant == 0 ? launch_dv<128, 0>(causal, smooth_q, a, st) : launch_dv<128, 1>(causal, smooth_q, a, st);
}

hipError_t launch_debug_qk(int d, const int8_t* q_i8, const int8_t* k_i8, int G, int Np, const int* tiles,
                           int n_tiles, int32_t* s_out, hipStream_t st) {
  if (d == 64)
    debug_qk_kernel<64><<<n_tiles, kThreads, 0, st>>>(q_i8, k_i8, G, Np, tiles, s_out);
  else
    debug_qk_kernel<128><<<n_tiles, kThreads, 0, st>>>(q_i8, k_i8, G, Np, tiles, s_out);
  return hipGetLastError();
}

}  // namespace sage
