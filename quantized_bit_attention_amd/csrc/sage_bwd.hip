// sage_bwd.hip -- 8-bit attention backward for gfx950 (CDNA4): dQ, dK, dV.
//
// Method: "SageAttention3: Microscaling FP4 Attention for Inference and An Exploration of
// 8-Bit Training" (abstract on the author page, "NeurIPS Conference 2025"): an 8-bit
// attention for the backward pass as well as the forward.  The backward follows
// FlashAttention-2 (an entry of the SageAttention summary page's reference list): it
// recomputes P = exp(s - L) from the forward's scores and the row log-sum-exp L, forms
// D_i = sum_c dO_ic O_ic, dP = dO V^T, dS = P (dP - D), and accumulates dV = P^T dO,
// dK = dS^T Q, dQ = dS K.
//
// 8-bit products: the recomputed scores use the forward's INT8 codes (K smoothed, per-block
// Q and K scales, exact int32); dP = dO V^T runs on per-token INT8 dO and V' (V minus its
// token mean, which shifts dP_ij and D_i by the same dO_i . vmean, so dS does not move),
// also with exact int32 sums.  The products with P and dS keep fp16 operands and fp32
// accumulation, as SageAttention keeps P~ V in FP16: P enters as fp16(2^8 P) and dS as
// fp16(sigma dS), sigma = 2^(14 - e) with 2^e the first power of two above
// 2 max|dO_i| max|V'_j| (a bound of |dS|), and dQ uses the smoothed K' in fp16.
//
// Kernels (all on [G = B*H heads][N][D] tensors):
//  - bwd_prep_kernel: per token, INT8 V' and dO with their scales, D', the log-sum-exp in
//    base 2, K' in fp16, and per 64-row block the largest |dO_i| and |V'_j| (for sigma);
//  - bwd_dkdv_kernel: a workgroup owns 32 keys per wave (8 waves at d = 128, 4 at d = 64)
//    and walks 64-row query tiles through two LDS slots.  S = Qhat Khat^T and dP = dOhat V'hat^T come out of v_mfma_i32_32x32x32_i8
//    with the query tile as the A operand (rows in the k_perm order of the forward's K
//    tile), so each lane holds one key and 16 consecutive rows of each 32-row block; P
//    and dS are then packed as fp16 pairs in exactly the layout of the forward's P~, and
//    dV^T = dO^T P and dK^T = Q^T dS run as the forward's P~ V product with the dO and Q
//    fp16 tiles in place of V;
//  - bwd_dq_kernel: the forward's layout (a workgroup owns 128 query rows, their Qhat and
//    dOhat rows held as register operands): S^T and dP^T per 64-key tile through two LDS
//    slots, dS packed as the forward's P~, and dQ^T = K'^T dS^T as its P~ V product with
//    the K' fp16 tile in place of V.
// Both number their workgroups so that each XCD walks a contiguous range of heads.
// No atomics: dK and dV are written by the key blocks' owners, dQ by the query blocks'
// owners, so the results are deterministic.
#include "sage_device.h"
#include "sage_internal.h"
#include "sage_tiles.h"

namespace sage {

constexpr int kBwdWaves = 4;
constexpr int kBwdThreads = 64 * kBwdWaves;
constexpr int kBwdRows = 32 * kBwdWaves;  // keys (dK/dV) or query rows (dQ) per workgroup
constexpr float kPScale = 256.0f;         // P enters the fp16 products as 2^8 P
constexpr float kLog2PScale = 8.0f;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}
__device__ __forceinline__ double wave_sum_f64(double x) {
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) x += __shfl_xor(x, off);
  return x;
}

// Workgroup ids are dealt round-robin over the 8 XCDs, each with its own L2; renumber
// them so each XCD walks a contiguous range of (head, block) pairs and the tiles of a
// head stay in one L2 while its blocks run.
__device__ __forceinline__ int xcd_block(int total) {
  const int b = blockIdx.x;
  return (total & 7) == 0 ? (b & 7) * (total >> 3) + (b >> 3) : b;
}

// Head g and length rank of this workgroup among the nb blocks of a head (rank 0: the
// block with the most work).  Causal blocks differ in length, so they go longest first
// across each pair of heads: one head's blocks after another's would start the last
// head's longest blocks late and leave the XCD's other workgroup slots idle at the end.
// Without the mask every block is as long as the others and heads go one after another.
template <bool CAUSAL>
__device__ __forceinline__ void head_rank(int G, int nb, int& g, int& rank) {
  const int vid = xcd_block(G * nb);
  if (CAUSAL) {
    const int pair = vid / (2 * nb), r = vid - pair * 2 * nb;
    if (2 * pair + 1 < G) {
      g = 2 * pair + (r & 1);
      rank = r >> 1;
    } else {  // odd head count: the last head alone
      g = 2 * pair;
      rank = r;
    }
  } else {
    g = vid / nb;
    rank = vid % nb;
  }
}

// sigma = 2^(14 - e), 2^e the first power of two above 2 max|dO_i| max|V'_j| (1 when the bound is 0),
// from the per-block maxima the preparation pass wrote ([nblk][2]).  Every thread of the
// workgroup gets the same value.
__device__ __forceinline__ float bwd_sigma(const float* nrm, int nblk, float* sRed) {
  const int tid = threadIdx.x;
  float gm = 0.0f, vm = 0.0f;
  for (int b = tid; b < nblk; b += blockDim.x) {
    gm = fmaxf(gm, nrm[2 * b]);
    vm = fmaxf(vm, nrm[2 * b + 1]);
  }
  gm = wave_max(gm);
  vm = wave_max(vm);
  if ((tid & 63) == 0) {
    sRed[2 * (tid >> 6)] = gm;
    sRed[2 * (tid >> 6) + 1] = vm;
  }
  __syncthreads();
  gm = 0.0f;
  vm = 0.0f;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) {
    gm = fmaxf(gm, sRed[2 * w]);
    vm = fmaxf(vm, sRed[2 * w + 1]);
  }
  __syncthreads();
  const float bound = 2.0f * gm * vm;
  return bound > 0.0f ? __builtin_amdgcn_ldexpf(1.0f, 14 - __builtin_amdgcn_frexp_expf(bound)) : 1.0f;
}

// ---------------------------------------------------------------------------
// preparation: one workgroup per (head, 64 tokens); wave w takes tokens 16w .. 16w+15,
// a token D/8 lanes with 8 consecutive channels each (16-byte loads), so a wave works on
// 512/D tokens at a time.  Pad tokens run the same arithmetic on zeros, which gives zero
// codes, scales and D'.
template <int D>
__global__ __launch_bounds__(256) void bwd_prep_kernel(BwdArgs a) {
  constexpr int LPR = D / 8;       // lanes per token
  constexpr int RPP = 64 / LPR;    // tokens per pass of a wave
  const int nblk = a.Np / 64;
  const int g = blockIdx.x / nblk, blk = blockIdx.x % nblk;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane / LPR, c0 = 8 * (lane % LPR);  // token of the pass, first channel
  __shared__ float sRed[8];
  // exact token means of K and V (split 0 of the statistics pass holds the head's sums)
  float kmean[8], vmean[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    kmean[j] = a.smooth_k ? fixed24_mean(a.ksum[(size_t)g * a.nsplit * D + c0 + j], a.N) : 0.0f;
    vmean[j] = fixed24_mean(a.vsum[(size_t)g * a.nsplit * D + c0 + j], a.N);
  }
  // reductions over the LPR lanes of a token (aligned groups of consecutive lanes)
  auto gmax = [](float x) {
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) x = fmaxf(x, __shfl_xor(x, off));
    return x;
  };
  auto gsum = [](float x) {
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) x += __shfl_xor(x, off);
    return x;
  };
  auto gsum64 = [](double x) {
#pragma unroll
    for (int off = 1; off < LPR; off <<= 1) x += __shfl_xor(x, off);
    return x;
  };
  float gmx = 0.0f, vmx = 0.0f;
#pragma unroll
  for (int pass = 0; pass < 16 / RPP; ++pass) {
    const int t = blk * 64 + 16 * wave + pass * RPP + sub;
    const bool ok = t < a.N;
    const size_t row = (size_t)g * a.Np + t;
    const size_t src = ((size_t)g * a.N + (ok ? t : 0)) * D + c0;
    const uint4 z = make_uint4(0u, 0u, 0u, 0u);
    const uint4 vraw = ok ? *reinterpret_cast<const uint4*>(a.v + src) : z;
    const uint4 graw = ok ? *reinterpret_cast<const uint4*>(a.dout + src) : z;
    const uint4 oraw = ok ? *reinterpret_cast<const uint4*>(a.o + src) : z;
    const uint4 kraw = ok ? *reinterpret_cast<const uint4*>(a.k + src) : z;
    const f16x8 v8 = __builtin_bit_cast(f16x8, vraw), g8 = __builtin_bit_cast(f16x8, graw);
    const f16x8 o8 = __builtin_bit_cast(f16x8, oraw), k8 = __builtin_bit_cast(f16x8, kraw);
    float vv[8], gg[8];
    uint32_t kp[4];
    float va = 0.0f, ga = 0.0f, vn = 0.0f, gn = 0.0f;
    double dsum = 0.0;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float vx = ok ? (float)v8[j] - vmean[j] : 0.0f;
      const float gx = (float)g8[j], ox = (float)o8[j];
      const float kx = ok ? (float)k8[j] - kmean[j] : 0.0f;
      if (j & 1) kp[j >> 1] |= (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)kx) << 16;
      else kp[j >> 1] = __builtin_bit_cast(uint16_t, (_Float16)kx);
      vv[j] = vx;
      gg[j] = gx;
      va = fmaxf(va, fabsf(vx));
      ga = fmaxf(ga, fabsf(gx));
      vn = fmaf(vx, vx, vn);
      gn = fmaf(gx, gx, gn);
      // exact products of fp16 values; the fp64 sum of the row is exact for ordinary data
      dsum += (double)gx * (double)ox - (double)gx * (double)vmean[j];
    }
    va = gmax(va);
    ga = gmax(ga);
    vn = gsum(vn);
    gn = gsum(gn);
    dsum = gsum64(dsum);
    const float vr = i8_factor(va), gr = i8_factor(ga);
    *reinterpret_cast<uint4*>(a.kp + row * D + c0) = make_uint4(kp[0], kp[1], kp[2], kp[3]);
    *reinterpret_cast<uint2*>(a.v_i8 + row * D + c0) =
        make_uint2(pack_bytes4(i8_code_int(vv[0], vr), i8_code_int(vv[1], vr), i8_code_int(vv[2], vr), i8_code_int(vv[3], vr)),
                   pack_bytes4(i8_code_int(vv[4], vr), i8_code_int(vv[5], vr), i8_code_int(vv[6], vr), i8_code_int(vv[7], vr)));
    *reinterpret_cast<uint2*>(a.do_i8 + row * D + c0) =
        make_uint2(pack_bytes4(i8_code_int(gg[0], gr), i8_code_int(gg[1], gr), i8_code_int(gg[2], gr), i8_code_int(gg[3], gr)),
                   pack_bytes4(i8_code_int(gg[4], gr), i8_code_int(gg[5], gr), i8_code_int(gg[6], gr), i8_code_int(gg[7], gr)));
    if (c0 == 0) {
      a.v_scale[row] = i8_scale(va);
      a.do_scale[row] = i8_scale(ga);
      a.dvec[row] = (float)dsum;
      // pad rows: +inf, which gives them P = 0
      a.lse2[row] = ok ? a.lse[(size_t)g * a.N + t] * 1.4426950408889634f : INFINITY;
    }
    gmx = fmaxf(gmx, __builtin_sqrtf(gn));
    vmx = fmaxf(vmx, __builtin_sqrtf(vn));
  }
  const float gmax_w = wave_max(gmx), vmax_w = wave_max(vmx);
  if (lane == 0) {
    sRed[2 * wave] = gmax_w;
    sRed[2 * wave + 1] = vmax_w;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    float gm = 0.0f, vm = 0.0f;
    for (int w = 0; w < 4; ++w) {
      gm = fmaxf(gm, sRed[2 * w]);
      vm = fmaxf(vm, sRed[2 * w + 1]);
    }
    a.nrm[((size_t)g * nblk + blk) * 2] = gm;
    a.nrm[((size_t)g * nblk + blk) * 2 + 1] = vm;
  }
}

// The INT8 product of one 32-row block st of an A tile in the k_tile layout with a B
// operand held in registers (b[ks]: the lane's 16 bytes of k-step ks): acc[i] = row
// 32*st + 16*h + i of the tile . column l%32.
template <int D>
__device__ __forceinline__ i32x16 i8_block_regb(const int8_t* sA, int st, const i32x4* b, int lane) {
  constexpr int CPR = D / 16;
  const int8_t* abase = sA + 16 * lane;
  i32x16 acc = {};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks)
    acc = mfma_i8(*reinterpret_cast<const i32x4*>(abase + (st * CPR + 2 * ks) * 512), b[ks], acc);
  return acc;
}

// The fp16 product of one 32-row block st of a [64 rows][D] fp16 tile (v_tile layout,
// vbase = tile + pv_lane_offset) with 8 packed weights of the lane's 16 rows of block st.
template <int D>
__device__ __forceinline__ void f16_block(const uint8_t* vbase, const uint32_t* pk, int st, f32x16* o) {
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const uint32_t pq[4] = {pk[u * 4], pk[u * 4 + 1], pk[u * 4 + 2], pk[u * 4 + 3]};
    const f16x8 pb = __builtin_bit_cast(f16x8, pq);
#pragma unroll
    for (int ct = 0; ct < D / 32; ++ct) {
      const i16x4 a0 = lds_read_tr16(vbase + 128 * ((8 * st + 2 * u) * (D / 16) + 2 * ct));
      const i16x4 a1 = lds_read_tr16(vbase + 128 * ((8 * st + 2 * u + 1) * (D / 16) + 2 * ct));
      const i16x4 a01[2] = {a0, a1};
      o[ct] = mfma_f16(__builtin_bit_cast(f16x8, a01), pb, o[ct]);
    }
  }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 32 keys per wave of one head (wave w: keys 32w .. 32w+31), 64-row
// query tiles through two LDS slots: the copies of tile t+1 (the INT8 and fp16 Q and dO
// tiles and the tile's row values) run while tile t is worked on.  8 waves at d = 128
// (96 KB of LDS, one workgroup per CU, two waves per SIMD); 4 at d = 64, whose registers
// leave room for three waves per SIMD (three workgroups per CU).  Np is a multiple of
// 128, so the last workgroup of a head may have waves past the padded tensor: they take
// part in the copies and barriers only.
template <int D> constexpr int kv_waves() { return D == 128 ? 8 : 4; }
template <int D> constexpr int kv_keys() { return 32 * kv_waves<D>(); }

// 64 consecutive floats (one per lane) from a [Np] float array of the head into LDS.
__device__ __forceinline__ void copy_row_values(__amdgpu_buffer_rsrc_t rs, int t, float* dst) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)dst, 4, 4u * (threadIdx.x & 63),
                                           (uint32_t)(t * kTileKV * 4), 0, 0);
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(64 * kv_waves<D>(), D == 128 ? 1 : 3) void bwd_dkdv_kernel(BwdArgs a) {
  constexpr int kKvWaves = kv_waves<D>(), kKvKeys = kv_keys<D>();
  constexpr int NCT = D / 32;
  // two slots per tile kind, as separate LDS objects (the step is instantiated per slot
  // parity, so the compiler can tell the slot being filled from the slot being read)
  __shared__ __attribute__((aligned(16))) int8_t sQ0[kTileKV * D];      // Qhat tile (k_tile layout)
  __shared__ __attribute__((aligned(16))) int8_t sQ1[kTileKV * D];
  __shared__ __attribute__((aligned(16))) int8_t sG0[kTileKV * D];      // dOhat tile (k_tile layout)
  __shared__ __attribute__((aligned(16))) int8_t sG1[kTileKV * D];
  __shared__ __attribute__((aligned(16))) uint8_t sQf0[kTileKV * D * 2];  // Q fp16 tile (v_tile layout)
  __shared__ __attribute__((aligned(16))) uint8_t sQf1[kTileKV * D * 2];
  __shared__ __attribute__((aligned(16))) uint8_t sGf0[kTileKV * D * 2];  // dO fp16 tile (v_tile layout)
  __shared__ __attribute__((aligned(16))) uint8_t sGf1[kTileKV * D * 2];
  __shared__ __attribute__((aligned(16))) float sL0[kTileKV];  // 8 - log2-sum-exp of the rows
  __shared__ __attribute__((aligned(16))) float sL1[kTileKV];
  __shared__ __attribute__((aligned(16))) float sD0[kTileKV];  // sigma 2^-8 D' of the rows
  __shared__ __attribute__((aligned(16))) float sD1[kTileKV];
  __shared__ __attribute__((aligned(16))) float sGs0[kTileKV];  // INT8 scales of the dO rows
  __shared__ __attribute__((aligned(16))) float sGs1[kTileKV];
  __shared__ float sRed[2 * kKvWaves];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5;
  const int nkb = (a.Np + kKvKeys - 1) / kKvKeys;
  int g, kb;  // causal: key block kb meets the queries from kb on, so rank order is kb order
  head_rank<CAUSAL>(a.G, nkb, g, kb);
  const int k0 = kb * kKvKeys, kw = k0 + 32 * wave, key = kw + (lane & 31);
  const int N = a.N, Np = a.Np;
  const bool has_keys = kw < Np;  // kw and Np are multiples of 32

  const float sigma = bwd_sigma(a.nrm + (size_t)g * (Np / 64) * 2, Np / 64, sRed);

  // B operands of this wave: Khat and V'hat rows of its 32 keys (pad rows are zero)
  i32x4 kb_op[D / 32], vb_op[D / 32];
  {
    const int8_t* kr = a.k_i8 + ((size_t)g * Np + (has_keys ? key : 0)) * D + 16 * h;
    const int8_t* vr = a.v_i8 + ((size_t)g * Np + (has_keys ? key : 0)) * D + 16 * h;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      kb_op[ks] = *reinterpret_cast<const i32x4*>(kr + 32 * ks);
      vb_op[ks] = *reinterpret_cast<const i32x4*>(vr + 32 * ks);
    }
  }
  // the key's K scale times sm_scale * log2(e), and its V' scale.  The loop forms
  // 2^8 P = 2^(s c + 8 - L) and sigma dS = (2^8 P) x with x = sigma 2^-8 (dP - D), so the
  // scales 2^8 and sigma 2^-8 (powers of two) ride on the per-row L and D and on this
  // key's V' scale.
  const float ck = a.kscale * a.k_scale[(size_t)g * a.nkb + min(key, N - 1) / a.blk_k];
  const float sig8 = sigma * (1.0f / kPScale);
  const float dvs = a.v_scale[(size_t)g * Np + min(key, Np - 1)] * sig8;

  f32x16 dv[NCT], dk[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) dv[ct] = dk[ct] = f32x16{};

  const TileCopy<D, 0, kKvWaves> copy(Np);
  const __amdgpu_buffer_rsrc_t qrs = make_rsrc(a.q_i8 + (size_t)g * Np * D, (size_t)Np * D);
  const __amdgpu_buffer_rsrc_t grs = make_rsrc(a.do_i8 + (size_t)g * Np * D, (size_t)Np * D);
  const __amdgpu_buffer_rsrc_t qfrs = make_rsrc(a.q + (size_t)g * N * D, (size_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t gfrs = make_rsrc(a.dout + (size_t)g * N * D, (size_t)N * D * 2);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(a.lse2 + (size_t)g * Np, (size_t)Np * 4);
  const __amdgpu_buffer_rsrc_t drs = make_rsrc(a.dvec + (size_t)g * Np, (size_t)Np * 4);
  const __amdgpu_buffer_rsrc_t gsrs = make_rsrc(a.do_scale + (size_t)g * Np, (size_t)Np * 4);
  const int vb = pv_lane_offset<D>(lane);

  // causal: rows below the workgroup's first key see none of its keys (t0 is even)
  const int t0 = CAUSAL ? k0 / kTileKV : 0;
  const int T = (N + kTileKV - 1) / kTileKV;

  // copies of tile t into one slot; wave 0 also brings the tile's 64 row values
  auto issue = [&](int t, int8_t* q, int8_t* gq, uint8_t* qf, uint8_t* gf, float* L, float* Dv, float* Gs) {
    copy.k_tile(qrs, t, q);
    copy.k_tile(grs, t, gq);
    copy.v_tile(qfrs, t, Np, qf);
    copy.v_tile(gfrs, t, Np, gf);
    if (wave == 0) {
      copy_row_values(lrs, t, L);
      copy_row_values(drs, t, Dv);
      copy_row_values(gsrs, t, Gs);
    }
  };
  // wave 0, once its copies have landed: the row values become 8 - L (pad rows: L = +inf,
  // so 2^8 P = 0) and sigma 2^-8 D'; no other wave reads the slot before the next barrier
  auto fix_rows = [&](float* L, float* Dv) {
    if (wave == 0) {
      wait_copies();
      L[lane] = kLog2PScale - L[lane];
      Dv[lane] *= sig8;
    }
  };

  auto step = [&](int t, auto parity) __attribute__((always_inline)) {
    constexpr int cur = decltype(parity)::value;
    const int8_t* const cQ = cur ? sQ1 : sQ0;
    const int8_t* const cG = cur ? sG1 : sG0;
    const uint8_t* const cQf = cur ? sQf1 : sQf0;
    const uint8_t* const cGf = cur ? sGf1 : sGf0;
    const float* const cL = cur ? sL1 : sL0;
    const float* const cD = cur ? sD1 : sD0;
    const float* const cGs = cur ? sGs1 : sGs0;
    // tile t is in place; every wave is done with tile t-1, whose slot takes tile t+1
    wait_copies();
    __syncthreads();
    if (t + 1 < T) {
      if (cur) issue(t + 1, sQ0, sG0, sQf0, sGf0, sL0, sD0, sGs0);
      else issue(t + 1, sQ1, sG1, sQf1, sGf1, sL1, sD1, sGs1);
    }
    const int r0 = t * kTileKV;
    // this wave's keys are all beyond the tile's last row: nothing to add
    const bool active = has_keys && (!CAUSAL || r0 + kTileKV - 1 >= kw);
    // causal: only a tile with a row before one of the wave's keys needs the mask
    const bool diag = CAUSAL && r0 < kw + 31;
    auto block = [&](int st) {
      const float c = a.q_scale[(size_t)g * a.nqb + min(r0, N - 1) / a.blk_q] * ck;
      const i32x16 s = i8_block_regb<D>(cQ, st, kb_op, lane);
      const i32x16 dp = i8_block_regb<D>(cG, st, vb_op, lane);
      // rows 32*st + 16*h + i of the tile
      const float4* pl = reinterpret_cast<const float4*>(cL + 32 * st + 16 * h);
      const float4* pd = reinterpret_cast<const float4*>(cD + 32 * st + 16 * h);
      const float4* pg = reinterpret_cast<const float4*>(cGs + 32 * st + 16 * h);
      uint32_t pkp[8], pks[8];
      // row r0 + 32 st + 16 h + i sees the key iff i >= thr
      const int thr = diag ? key - (r0 + 32 * st + 16 * h) : -1;
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 L4 = pl[q4], D4 = pd[q4], G4 = pg[q4];
        const float Lr[4] = {L4.x, L4.y, L4.z, L4.w}, Dr[4] = {D4.x, D4.y, D4.z, D4.w};
        const float Gr[4] = {G4.x, G4.y, G4.z, G4.w};
        float p[4], ds[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * q4 + b;
          float pv = __builtin_amdgcn_exp2f(fmaf((float)s[i], c, Lr[b]));  // 2^8 P
          if (CAUSAL) pv = i >= thr ? pv : 0.0f;
          p[b] = pv;
          ds[b] = pv * fmaf((float)dp[i], Gr[b] * dvs, -Dr[b]);          // sigma dS
        }
        pkp[2 * q4] = pack_f16x2(p[0], p[1]);
        pkp[2 * q4 + 1] = pack_f16x2(p[2], p[3]);
        pks[2 * q4] = pack_f16x2(ds[0], ds[1]);
        pks[2 * q4 + 1] = pack_f16x2(ds[2], ds[3]);
      }
      f16_block<D>(cGf + vb, pkp, st, dv);
      f16_block<D>(cQf + vb, pks, st, dk);
    };
    if (active) {
      block(0);
      block(1);
    }
    if (t + 1 < T) {
      if (cur) fix_rows(sL0, sD0);
      else fix_rows(sL1, sD1);
    }
  };

  if (t0 < T) {
    issue(t0, sQ0, sG0, sQf0, sGf0, sL0, sD0, sGs0);
    fix_rows(sL0, sD0);
  }
  for (int t = t0; t < T; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < T) step(t + 1, std::integral_constant<int, 1>{});
  }

  if (key >= N) return;
  const float sv = 1.0f / kPScale, sk = a.sm_scale / sigma;
  float* dvr = a.dv + ((size_t)g * N + key) * D;
  float* dkr = a.dk + ((size_t)g * N + key) * D;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int c0 = ct * 32 + 8 * a4 + 4 * h;
      *reinterpret_cast<float4*>(dvr + c0) = make_float4(dv[ct][4 * a4] * sv, dv[ct][4 * a4 + 1] * sv,
                                                         dv[ct][4 * a4 + 2] * sv, dv[ct][4 * a4 + 3] * sv);
      *reinterpret_cast<float4*>(dkr + c0) = make_float4(dk[ct][4 * a4] * sk, dk[ct][4 * a4 + 1] * sk,
                                                         dk[ct][4 * a4 + 2] * sk, dk[ct][4 * a4 + 3] * sk);
    }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 128 query rows of one head (wave w: rows 32w .. 32w+31), 64-key tiles.
// The wave's Qhat and dOhat rows are the B operands, held in registers; the K, V' and K'
// tiles go through two LDS slots, tile t+1 copied while tile t is worked on.
template <int D, bool CAUSAL>
__global__ __launch_bounds__(kBwdThreads, 2) void bwd_dq_kernel(BwdArgs a) {
  constexpr int NCT = D / 32;
  // two slots per tile kind, as separate LDS objects: the loop body is instantiated per
  // slot parity, so the compiler can tell the slot being filled from the slot being read
  __shared__ __attribute__((aligned(16))) int8_t sK0[kTileKV * D];       // Khat tile (k_tile layout)
  __shared__ __attribute__((aligned(16))) int8_t sK1[kTileKV * D];
  __shared__ __attribute__((aligned(16))) int8_t sV0[kTileKV * D];       // V'hat tile (k_tile layout)
  __shared__ __attribute__((aligned(16))) int8_t sV1[kTileKV * D];
  __shared__ __attribute__((aligned(16))) uint8_t sKf0[kTileKV * D * 2];  // K' fp16 tile (v_tile layout)
  __shared__ __attribute__((aligned(16))) uint8_t sKf1[kTileKV * D * 2];
  __shared__ __attribute__((aligned(16))) float sVs0[kTileKV];  // INT8 scales of the tile's V' rows
  __shared__ __attribute__((aligned(16))) float sVs1[kTileKV];
  __shared__ float sRed[8];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, h = lane >> 5, ql = lane & 31;
  const int nqt = a.Np / kBwdRows;
  int g, qt;  // causal: query tile qt meets the keys up to its own, so the longest is the last
  head_rank<CAUSAL>(a.G, nqt, g, qt);
  if (CAUSAL) qt = nqt - 1 - qt;
  const int q0 = qt * kBwdRows, qw = q0 + 32 * wave, qi = qw + ql;
  const int N = a.N, Np = a.Np;

  const float sigma = bwd_sigma(a.nrm + (size_t)g * (Np / 64) * 2, Np / 64, sRed);

  // B operands: bytes 32 ks + 16 h .. +15 of this lane's Qhat and dOhat row for k-step ks
  // (qi < Np; pad rows are zero)
  i32x4 qb[D / 32], gb[D / 32];
  {
    const int8_t* qr = a.q_i8 + ((size_t)g * Np + qi) * D + 16 * h;
    const int8_t* gr = a.do_i8 + ((size_t)g * Np + qi) * D + 16 * h;
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks) {
      qb[ks] = *reinterpret_cast<const i32x4*>(qr + 32 * ks);
      gb[ks] = *reinterpret_cast<const i32x4*>(gr + 32 * ks);
    }
  }
  const size_t rq = (size_t)g * Np + qi;
  // sigma dS = P x with x = sigma (dP - D): sigma (a power of two) rides on the row's D
  // and dO scale
  const float l2 = a.lse2[rq], drs = a.dvec[rq] * sigma, gss = a.do_scale[rq] * sigma;
  const float cq = a.kscale * a.q_scale[(size_t)g * a.nqb + min(qi, N - 1) / a.blk_q];

  f32x16 dq[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) dq[ct] = f32x16{};

  const TileCopy<D, 0, kBwdWaves> copy(Np);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k_i8 + (size_t)g * Np * D, (size_t)Np * D);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v_i8 + (size_t)g * Np * D, (size_t)Np * D);
  // K' is padded to Np rows of zeros: the copy of the last tile stays inside
  const __amdgpu_buffer_rsrc_t kfrs = make_rsrc(a.kp + (size_t)g * Np * D, (size_t)Np * D * 2);
  const int vb = pv_lane_offset<D>(lane);
  const int ntiles = (N + kTileKV - 1) / kTileKV;
  const int T = CAUSAL ? min(ntiles, (min(q0 + kBwdRows, N) - 1) / kTileKV + 1) : ntiles;
  const int wave_last = CAUSAL ? min(ntiles - 1, min(qw + 31, N - 1) / kTileKV) : ntiles - 1;
  const unsigned last_key = (unsigned)(N - 1);
  const int kshift = __builtin_ctz(a.blk_k);
  const float* const vsc = a.v_scale + (size_t)g * Np;  // Np >= 64 * ntiles

  // S^T and dP^T of tile t (Khat, V'hat in sK, sV), dS packed as P~, dQ^T += K'^T dS^T
  auto tile = [&](int t, const int8_t* sK, const int8_t* sV, const uint8_t* sKf, const float* sVs, bool full) {
    float kq[4];
    tile_kscales(a.k_scale + (size_t)g * a.nkb, t, last_key, kshift, kq);
    constexpr int CPR = D / 16;
    const int8_t* kbase = sK + 16 * lane;
    const int8_t* vbase = sV + 16 * lane;
    i32x16 s[2] = {i32x16{}, i32x16{}}, dp[2] = {i32x16{}, i32x16{}};
#pragma unroll
    for (int ks = 0; ks < D / 32; ++ks)
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        s[st] = mfma_i8(*reinterpret_cast<const i32x4*>(kbase + (st * CPR + 2 * ks) * 512), qb[ks], s[st]);
        dp[st] = mfma_i8(*reinterpret_cast<const i32x4*>(vbase + (st * CPR + 2 * ks) * 512), gb[ks], dp[st]);
      }
    uint32_t pk[16];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const float c = cq * kscale_of(kq, st, h);
      const float4* pv4 = reinterpret_cast<const float4*>(sVs + 32 * st + 16 * h);
      // key t*64 + 32 st + 16 h + i carries weight iff i <= thr: keys past N, and past
      // the row when causal, carry none
      const int thr = full ? 15 : (CAUSAL ? min(N - 1, qi) : N - 1) - (t * kTileKV + 32 * st + 16 * h);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const float4 V4 = pv4[q4];
        const float Vr[4] = {V4.x, V4.y, V4.z, V4.w};
        float ds[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) {
          const int i = 4 * q4 + b;
          float pv = __builtin_amdgcn_exp2f(fmaf((float)s[st][i], c, -l2));
          pv = i <= thr ? pv : 0.0f;
          ds[b] = pv * fmaf((float)dp[st][i], gss * Vr[b], -drs);  // sigma dS
        }
        pk[st * 8 + 2 * q4] = pack_f16x2(ds[0], ds[1]);
        pk[st * 8 + 2 * q4 + 1] = pack_f16x2(ds[2], ds[3]);
      }
    }
    pv_tile_f16<D>(sKf + vb, pk, dq);
  };

  // step t: tile t sits in slot t % 2; the barrier also ends every wave's reads of
  // slot (t + 1) % 2 (tile t - 1), which then takes tile t + 1
  auto step = [&](int t, auto parity) __attribute__((always_inline)) {
    constexpr int cur = decltype(parity)::value;
    const int8_t* const cK = cur ? sK1 : sK0;
    const int8_t* const cV = cur ? sV1 : sV0;
    const uint8_t* const cKf = cur ? sKf1 : sKf0;
    const float* const cVs = cur ? sVs1 : sVs0;
    int8_t* const nK = cur ? sK0 : sK1;
    int8_t* const nV = cur ? sV0 : sV1;
    uint8_t* const nKf = cur ? sKf0 : sKf1;
    float* const nVs = cur ? sVs0 : sVs1;
    wait_copies();
    __syncthreads();
    float vnext = 0.0f;
    if (t + 1 < T) {
      copy.k_tile(krs, t + 1, nK);
      copy.k_tile(vrs, t + 1, nV);
      copy.v_tile(kfrs, t + 1, Np, nKf);
      if (tid < kTileKV) vnext = vsc[(t + 1) * kTileKV + tid];
    }
    // only the tail tile and, causal, tiles with a key after the wave's first row mask
    if (qw < N && t <= wave_last)
      tile(t, cK, cV, cKf, cVs, (t + 1) * kTileKV <= N && (!CAUSAL || t * kTileKV + kTileKV - 1 <= qw));
    if (t + 1 < T && tid < kTileKV) nVs[tid] = vnext;
  };

  copy.k_tile(krs, 0, sK0);
  copy.k_tile(vrs, 0, sV0);
  copy.v_tile(kfrs, 0, Np, sKf0);
  if (tid < kTileKV) sVs0[tid] = vsc[tid];
  for (int t = 0; t < T; t += 2) {
    step(t, std::integral_constant<int, 0>{});
    if (t + 1 < T) step(t + 1, std::integral_constant<int, 1>{});
  }

  if (qi >= N) return;
  const float sq = a.sm_scale / sigma;
  float* dqr = a.dq + ((size_t)g * N + qi) * D;
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int a4 = 0; a4 < 4; ++a4) {
      const int c0 = ct * 32 + 8 * a4 + 4 * h;
      *reinterpret_cast<float4*>(dqr + c0) = make_float4(dq[ct][4 * a4] * sq, dq[ct][4 * a4 + 1] * sq,
                                                         dq[ct][4 * a4 + 2] * sq, dq[ct][4 * a4 + 3] * sq);
    }
}

// ---------------------------------------------------------------------------

template <int D>
static hipError_t launch_bwd_d(int causal, const BwdArgs& a, hipStream_t st) {
  const int G = a.G;
  bwd_prep_kernel<D><<<G * (a.Np / 64), 256, 0, st>>>(a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int grid_kv = G * ((a.Np + kv_keys<D>() - 1) / kv_keys<D>()), grid_q = G * (a.Np / kBwdRows);
  if (causal) {
    bwd_dkdv_kernel<D, true><<<grid_kv, 64 * kv_waves<D>(), 0, st>>>(a);
    bwd_dq_kernel<D, true><<<grid_q, kBwdThreads, 0, st>>>(a);
  } else {
    bwd_dkdv_kernel<D, false><<<grid_kv, 64 * kv_waves<D>(), 0, st>>>(a);
    bwd_dq_kernel<D, false><<<grid_q, kBwdThreads, 0, st>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_bwd(int d, int causal, const BwdArgs& a, hipStream_t st) {
  return d == 64 ? launch_bwd_d<64>(causal, a, st) : launch_bwd_d<128>(causal, a, st);
}

}  // namespace sage
