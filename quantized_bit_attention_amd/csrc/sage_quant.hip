// sage_quant.hip -- smoothing and quantisation kernels (gfx950).
//
// Method: "SageAttention: Accurate 8-Bit Attention for Plug-and-play Inference
// Acceleration" (summary page, "Summary" and "Interesting ideas" I1): K loses its
// token mean, then Q and K become INT8 with one fp32 scale per block of tokens.
// "SageAttention2 ..." (abstracts): Q loses its block mean; V becomes FP8 with one
// scale per channel, optionally after losing its token mean ("smooth Q and V").
// "SageAttention3 ..." (abstract): FP4 attention, read as per-token OCP MXFP4 of Q and
// K' (variant 2).
//
// All passes are bound by HBM bandwidth: they read fp16 rows with 16-byte loads and
// write int8 / fp8 / packed fp4 codes.
//
// Exactness: token sums are exact int64 sums of the fp16 values in units of 2^-24,
// so means do not depend on summation order; every fp32 step (subtract, multiply by
// the reciprocal, divide) is a single IEEE operation, with contraction off.
#include "sage_device.h"
#include "sage_internal.h"

#pragma clang fp contract(off)

namespace sage {

// Pass 1: per (head, split of kStatRows tokens) partial sums of K (exact, int64) and,
// for WITH_V, the partial max and min of V per channel (packed fp16, exact) and, for
// V_SUMS (V smoothing), the sums of V.
//   ksum_part, vsum_part [G][nsplit][D] int64; vmax_part, vmin_part [G][nsplit][D] fp32.
// A thread accumulates its at most kStatRows / RPI values per channel in fp64, which is
// exact: every fp16 value is an integer multiple of 2^-24 below 2^16 in magnitude, so
// up to 2^13 of them sum exactly within fp64's 53-bit significand.  The thread totals
// are then converted to int64 units of 2^-24 and summed exactly.  A thread issues all
// its row loads at once (8 at a time when it also reads V).
template <int D, bool WITH_V, bool V_SUMS>
__global__ __launch_bounds__(kThreads) void stats_kernel(const uint16_t* __restrict__ k,
                                                         const uint16_t* __restrict__ v, int N,
                                                         int nsplit, long long* __restrict__ ksum_part,
                                                         long long* __restrict__ vsum_part,
                                                         float* __restrict__ vmax_part,
                                                         float* __restrict__ vmin_part) {
  constexpr int TPR = D / 8;            // threads per row
  constexpr int RPI = kThreads / TPR;   // rows per iteration
  constexpr int NIT = kStatRows / RPI;  // rows per thread
  constexpr int BATCH = WITH_V ? 8 : NIT;
  static_assert(NIT % BATCH == 0 && NIT <= 8192, "row batches; exact fp64 thread sums");
  const int split = blockIdx.x % nsplit, g = blockIdx.x / nsplit;  // 1-D grid: G may exceed 65535
  const int tid = threadIdx.x, cg = tid % TPR, r0 = tid / TPR;
  const size_t head = (size_t)g * N * D;
  const int t0 = split * kStatRows, t1 = min(N, t0 + kStatRows);

  static_assert(WITH_V || !V_SUMS, "V sums need V");
  double acc[8], vacc[8];
  f16x2 vmx[4], vmn[4];
  const f16x2 ninf = __builtin_bit_cast(f16x2, 0xFC00FC00u), pinf = __builtin_bit_cast(f16x2, 0x7C007C00u);
#pragma unroll
  for (int j = 0; j < 8; ++j) { acc[j] = 0.0; vacc[j] = 0.0; }
#pragma unroll
  for (int j = 0; j < 4; ++j) { vmx[j] = ninf; vmn[j] = pinf; }

#pragma unroll 1
  for (int base = 0; base < NIT; base += BATCH) {
    uint4 kk[BATCH], vv[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int t = t0 + r0 + RPI * (base + b);
      kk[b] = t < t1 ? *reinterpret_cast<const uint4*>(k + head + (size_t)t * D + cg * 8) : make_uint4(0, 0, 0, 0);
      vv[b] = (WITH_V && t < t1) ? *reinterpret_cast<const uint4*>(v + head + (size_t)t * D + cg * 8)
                                 : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const uint32_t w[4] = {kk[b].x, kk[b].y, kk[b].z, kk[b].w};
      const uint32_t u[4] = {vv[b].x, vv[b].y, vv[b].z, vv[b].w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2 hk = __builtin_bit_cast(f16x2, w[j]);
        acc[2 * j] += (double)(float)hk[0];
        acc[2 * j + 1] += (double)(float)hk[1];
        if (WITH_V) {
          // rows past N hold zeros: they stay out of the max and min (and add 0 to the sums)
          const f16x2 hv = __builtin_bit_cast(f16x2, u[j]);
          const bool in = t0 + r0 + RPI * (base + b) < t1;
          if (V_SUMS) {
            vacc[2 * j] += (double)(float)hv[0];
            vacc[2 * j + 1] += (double)(float)hv[1];
          }
          vmx[j] = __builtin_elementwise_max(vmx[j], in ? hv : ninf);
          vmn[j] = __builtin_elementwise_min(vmn[j], in ? hv : pinf);
        }
      }
    }
  }

  float vm[8], vn[8];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    vm[2 * j] = (float)vmx[j][0];
    vm[2 * j + 1] = (float)vmx[j][1];
    vn[2 * j] = (float)vmn[j][0];
    vn[2 * j + 1] = (float)vmn[j][1];
  }
  // two rounds through LDS: (K sums, V max), then (V sums, V min)
  __shared__ long long s_sum[kThreads][8];
  __shared__ float s_max[kThreads][8];
  const size_t o = ((size_t)g * nsplit + split) * D + tid;
#pragma unroll
  for (int round = 0; round < (WITH_V ? 2 : 1); ++round) {
    if (round) __syncthreads();  // the first round's reads are done
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      s_sum[tid][j] = (long long)((round ? vacc[j] : acc[j]) * 16777216.0);  // exact: an integer below 2^53
      s_max[tid][j] = round ? vn[j] : vm[j];
    }
    __syncthreads();
    if (tid < D) {
      const int cgc = tid / 8, jj = tid % 8;
      long long sm = 0;
      float m = round ? INFINITY : -INFINITY;
      for (int r = 0; r < RPI; ++r) {
        sm += s_sum[r * TPR + cgc][jj];
        m = round ? fminf(m, s_max[r * TPR + cgc][jj]) : fmaxf(m, s_max[r * TPR + cgc][jj]);
      }
      if (round == 0) {
        ksum_part[o] = sm;
        if (WITH_V) vmax_part[o] = m;
      } else {
        if (V_SUMS) vsum_part[o] = sm;
        vmin_part[o] = m;
      }
    }
  }
}

// Pass 1b: fold the per-split partials of each head into split 0 (exact int64 sums of
// K and V, max and min of V), so the later passes read D values per head instead of
// nsplit * D.  Four threads per channel take every fourth split, then combine
// through LDS.  The V arrays are null when only K was summed.
template <int D>
__global__ __launch_bounds__(4 * D) void stats_finalize_kernel(int nsplit, long long* __restrict__ ksum_part,
                                                               long long* __restrict__ vsum_part,
                                                               float* __restrict__ vmax_part,
                                                               float* __restrict__ vmin_part) {
  __shared__ long long s_sum[4][D], s_vsum[4][D];
  __shared__ float s_max[4][D], s_min[4][D];
  const int g = blockIdx.x, c = threadIdx.x % D, j = threadIdx.x / D;
  const size_t base = (size_t)g * nsplit * D + c;
  const bool with_v = vmax_part != nullptr, with_vsum = vsum_part != nullptr;
  long long s = 0, vs = 0;
  float mx = -INFINITY, mn = INFINITY;
#pragma unroll 4
  for (int sp = j; sp < nsplit; sp += 4) {
    const size_t o = base + (size_t)sp * D;
    s += ksum_part[o];
    if (with_vsum) vs += vsum_part[o];
    if (with_v) {
      mx = fmaxf(mx, vmax_part[o]);
      mn = fminf(mn, vmin_part[o]);
    }
  }
  s_sum[j][c] = s;
  s_vsum[j][c] = vs;
  s_max[j][c] = mx;
  s_min[j][c] = mn;
  __syncthreads();  // every thread has read its splits before split 0 is overwritten
  if (j == 0) {
    ksum_part[base] = s_sum[0][c] + s_sum[1][c] + s_sum[2][c] + s_sum[3][c];
    if (with_vsum) vsum_part[base] = s_vsum[0][c] + s_vsum[1][c] + s_vsum[2][c] + s_vsum[3][c];
    if (with_v) {
      vmax_part[base] = fmaxf(fmaxf(s_max[0][c], s_max[1][c]), fmaxf(s_max[2][c], s_max[3][c]));
      vmin_part[base] = fminf(fminf(s_min[0][c], s_min[1][c]), fminf(s_min[2][c], s_min[3][c]));
    }
  }
}

// Block reduction of a non-negative float max over the workgroup.
__device__ __forceinline__ float block_max(float x, float* red) {
  for (int off = 32; off > 0; off >>= 1) x = fmaxf(x, __shfl_xor(x, off));
  const int wave = threadIdx.x / 64;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
}

// Pass 2: smooth + quantise one block of rows (a K block or a Q block) per workgroup.
//   blockIdx.x < G * nkb: K block (mean from the pass-1 partial sums when smooth_k);
//   otherwise a Q block (its own exact block mean when smooth_q).  With with_q = 0 the
//   grid holds only the K blocks (the attention kernel then quantises Q itself).
//   K has one scale per block; Q one per group of q_group rows (q_group divides blk_q).
// MAXR: rows per block rounded up to a multiple of kThreads / (D/8).
template <int D, int MAXR>
__global__ __launch_bounds__(kThreads) void quant_kernel(QuantArgs a) {
  constexpr int TPR = D / 8;
  constexpr int RPI = kThreads / TPR;
  constexpr int NIT = MAXR / RPI;
  __shared__ float s_mean[D];
  __shared__ long long s_sum[kThreads][8];
  __shared__ float s_red[4];
  __shared__ float s_row[MAXR], s_grp[MAXR];  // Q groups finer than the block

  const int tid = threadIdx.x, cg = tid % TPR, r0 = tid / TPR;
  const int nk_blocks = a.G * a.nkb;
  const bool is_k = (int)blockIdx.x < nk_blocks;
  const int idx = is_k ? (int)blockIdx.x : (int)blockIdx.x - nk_blocks;
  const int nb = is_k ? a.nkb : a.nqb;
  const int blk = is_k ? a.blk_k : a.blk_q;
  const int g = idx / nb, b = idx % nb;
  const int t0 = b * blk, t1 = min(a.N, t0 + blk), rows = t1 - t0;
  const uint16_t* __restrict__ src = (is_k ? a.k : a.q) + (size_t)g * a.N * D;
  int8_t* __restrict__ dst = (is_k ? a.k_i8 : a.q_i8) + (size_t)g * a.Np * D;
  const bool smooth = is_k ? a.smooth_k : a.smooth_q;

  // load the block's rows: thread holds rows r0 + RPI*it, channels cg*8 .. cg*8+7
  uint4 raw[NIT];
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int r = r0 + RPI * it;
    raw[it] = r < rows ? *reinterpret_cast<const uint4*>(src + (size_t)(t0 + r) * D + cg * 8)
                       : make_uint4(0, 0, 0, 0);
  }

  if (smooth) {
    if (is_k) {
      if (tid < D) {
        const long long s = a.ksum_part[(size_t)g * a.nsplit * D + tid];  // folded into split 0
        const float m = fixed24_mean(s, a.N);
        s_mean[tid] = m;
        if (b == 0 && a.k_mean) a.k_mean[(size_t)g * D + tid] = m;
      }
    } else {
      long long acc[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) acc[j] = 0;
#pragma unroll
      for (int it = 0; it < NIT; ++it) {
        const uint32_t w[4] = {raw[it].x, raw[it].y, raw[it].z, raw[it].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          acc[2 * j] += f16_bits_to_fixed24(w[j] & 0xffffu);
          acc[2 * j + 1] += f16_bits_to_fixed24(w[j] >> 16);
        }
      }
#pragma unroll
      for (int j = 0; j < 8; ++j) s_sum[tid][j] = acc[j];
      __syncthreads();
      if (tid < D) {
        long long s = 0;
        for (int r = 0; r < RPI; ++r) s += s_sum[r * TPR + tid / 8][tid % 8];
        const float m = fixed24_mean(s, rows);
        s_mean[tid] = m;
        if (a.q_mean) a.q_mean[((size_t)g * a.nqb + b) * D + tid] = m;
      }
    }
  } else if (tid < D) {
    s_mean[tid] = 0.0f;
  }
  __syncthreads();

  float mean[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) mean[j] = s_mean[cg * 8 + j];

  // smoothed values and their absmax (per row, over this thread's 8 channels)
  float x[NIT][8];
  float ramax[NIT];
  float amax = 0.0f;
#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const uint32_t w[4] = {raw[it].x, raw[it].y, raw[it].z, raw[it].w};
    const bool valid = r0 + RPI * it < rows;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x2 h = __builtin_bit_cast(f16x2, w[j]);
      float x0 = (float)h[0], x1 = (float)h[1];
      if (smooth) { x0 = x0 - mean[2 * j]; x1 = x1 - mean[2 * j + 1]; }
      x[it][2 * j] = valid ? x0 : 0.0f;
      x[it][2 * j + 1] = valid ? x1 : 0.0f;
    }
    ramax[it] = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j) ramax[it] = fmaxf(ramax[it], fabsf(x[it][j]));
    amax = fmaxf(amax, ramax[it]);
  }
  const int grp = is_k ? blk : a.q_group;
  float* const scale = is_k ? a.k_scale + (size_t)g * a.nkb : a.q_scale + (size_t)g * a.nqg;
  float r[NIT];
  if (grp >= blk) {  // one scale for the block
    amax = block_max(amax, s_red);
#pragma unroll
    for (int it = 0; it < NIT; ++it) r[it] = i8_factor(amax);
    if (tid == 0) scale[b] = i8_scale(amax);
  } else {
    // each row's absmax over the TPR threads that hold it, then each group's over its rows
#pragma unroll
    for (int it = 0; it < NIT; ++it) {
      float v = ramax[it];
      for (int off = 1; off < TPR; off <<= 1) v = fmaxf(v, __shfl_xor(v, off));
      if (cg == 0) s_row[r0 + RPI * it] = v;
    }
    __syncthreads();
    const int ngr = (rows + grp - 1) / grp;
    if (tid < ngr) {
      float m = 0.0f;
      for (int i = tid * grp; i < min(rows, (tid + 1) * grp); ++i) m = fmaxf(m, s_row[i]);
      s_grp[tid] = m;
      scale[t0 / grp + tid] = i8_scale(m);
    }
    __syncthreads();
#pragma unroll
    for (int it = 0; it < NIT; ++it) r[it] = i8_factor(s_grp[min((r0 + RPI * it) / grp, MAXR - 1)]);
  }

#pragma unroll
  for (int it = 0; it < NIT; ++it) {
    const int row = r0 + RPI * it;
    if (row < rows) {
      uint32_t packed[2] = {0u, 0u};
#pragma unroll
      for (int j = 0; j < 8; ++j) packed[j / 4] |= i8_code(x[it][j], r[it]) << (8 * (j % 4));
      *reinterpret_cast<uint2*>(dst + (size_t)(t0 + row) * D + cg * 8) = make_uint2(packed[0], packed[1]);
    }
  }
  // the last block of a head zeroes the pad rows [N, Np)
  if (b == nb - 1) {
    const int npad = a.Np - a.N;
    for (int e = tid; e < npad * (D / 8); e += kThreads) {
      const int row = a.N + e / (D / 8), c8 = e % (D / 8);
      *reinterpret_cast<uint2*>(dst + (size_t)row * D + c8 * 8) = make_uint2(0u, 0u);
    }
  }
}

// Pass 3 (variant 1): V -> FP8 E4M3 with per-channel scales, transposed to [G][D][Np].
// With V smoothing each channel first loses its exact token mean (v_mean, from the
// pass-1 sums); the absmax of V - v_mean is max(fl(max - v_mean), fl(v_mean - min))
// because rounding is monotonic, so no second pass over V is needed.
// One workgroup per (64-token tile, head); the tile goes through LDS so both the fp16
// reads and the fp8 writes are contiguous.
template <int D>
__global__ __launch_bounds__(kThreads) void quant_v_kernel(const uint16_t* __restrict__ v, int N, int Np,
                                                           int nsplit, const long long* __restrict__ vsum_part,
                                                           const float* __restrict__ vmax_part,
                                                           const float* __restrict__ vmin_part, int smooth_v,
                                                           uint8_t* __restrict__ v_f8,
                                                           float* __restrict__ v_scale,
                                                           float* __restrict__ v_mean) {
  constexpr int TPR = D / 8;
  constexpr int RPI = kThreads / TPR;
  constexpr int TT = 64;  // tokens per tile
  __shared__ float s_r[D], s_mean[D];
  __shared__ uint8_t s_t[D][TT + 4];
  const int ntiles = Np / 64;  // 1-D grid over (head, 64-token tile)
  const int tile = blockIdx.x % ntiles, g = blockIdx.x / ntiles, tid = threadIdx.x;
  if (tid < D) {
    const size_t o = (size_t)g * nsplit * D + tid;  // folded into split 0
    const float mean = smooth_v ? fixed24_mean(vsum_part[o], N) : 0.0f;
    const float hi = vmax_part[o] - mean, lo = mean - vmin_part[o];
    const float m = fmaxf(hi, lo) > 0.0f ? fmaxf(hi, lo) : 0.0f;  // +0 for a constant channel
    s_r[tid] = m > 0.0f ? 448.0f / m : 0.0f;
    s_mean[tid] = mean;
    if (tile == 0) {
      v_scale[(size_t)g * D + tid] = m / 448.0f;
      if (v_mean) v_mean[(size_t)g * D + tid] = mean;
    }
  }
  __syncthreads();
  const int cg = tid % TPR, r0 = tid / TPR;
  const size_t head = (size_t)g * N * D;
  for (int rr = r0; rr < TT; rr += RPI) {
    const int t = tile * TT + rr;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (t < N) raw = *reinterpret_cast<const uint4*>(v + head + (size_t)t * D + cg * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    const bool centre = smooth_v && t < N;  // padding columns stay code 0
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      f16x2 h = __builtin_bit_cast(f16x2, w[j]);
      const int c = cg * 8 + 2 * j;
      const float x0 = centre ? (float)h[0] - s_mean[c] : (float)h[0];
      const float x1 = centre ? (float)h[1] - s_mean[c + 1] : (float)h[1];
      float y0 = fminf(fmaxf(x0 * s_r[c], -448.0f), 448.0f);
      float y1 = fminf(fmaxf(x1 * s_r[c + 1], -448.0f), 448.0f);
      const uint32_t p = cvt_pk_fp8(y0, y1, 0u, false);
      s_t[c][rr] = (uint8_t)(p & 0xffu);
      s_t[c + 1][rr] = (uint8_t)((p >> 8) & 0xffu);
    }
  }
  __syncthreads();
  // write D rows of 64 bytes: 4 threads per row, 16 bytes each
  uint8_t* out = v_f8 + (size_t)g * D * Np + (size_t)tile * TT;
  for (int e = tid; e < D * 4; e += kThreads) {
    const int c = e / 4, part = e % 4;
    uint32_t wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      wv[q] = (uint32_t)s_t[c][part * 16 + 4 * q] | ((uint32_t)s_t[c][part * 16 + 4 * q + 1] << 8) |
              ((uint32_t)s_t[c][part * 16 + 4 * q + 2] << 16) | ((uint32_t)s_t[c][part * 16 + 4 * q + 3] << 24);
    *reinterpret_cast<uint4*>(out + (size_t)c * Np + part * 16) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
  }
}

// ---------------------------------------------------------------------------
// launchers

int stat_splits(int N) { return (N + kStatRows - 1) / kStatRows; }

template <int D>
static void launch_stats_d(const void* k, const void* v, bool v_sums, int G, int N, const StatsOut& out,
                           hipStream_t st) {
  const int ns = stat_splits(N);
  const int grid = ns * G;
  const uint16_t* kk = (const uint16_t*)k;
  const uint16_t* vv = (const uint16_t*)v;
  if (v && v_sums)
    stats_kernel<D, true, true><<<grid, kThreads, 0, st>>>(kk, vv, N, ns, out.ksum, out.vsum, out.vmax, out.vmin);
  else if (v)
    stats_kernel<D, true, false><<<grid, kThreads, 0, st>>>(kk, vv, N, ns, out.ksum, nullptr, out.vmax, out.vmin);
  else
    stats_kernel<D, false, false><<<grid, kThreads, 0, st>>>(kk, nullptr, N, ns, out.ksum, nullptr, nullptr, nullptr);
  stats_finalize_kernel<D><<<G, 4 * D, 0, st>>>(ns, out.ksum, v && v_sums ? out.vsum : nullptr,
                                                v ? out.vmax : nullptr, v ? out.vmin : nullptr);
}

hipError_t launch_stats(int d, const void* k, const void* v, bool v_sums, int G, int N, const StatsOut& out,
                        hipStream_t st) {
  if (d == 64)
    launch_stats_d<64>(k, v, v_sums, G, N, out, st);
  else
    launch_stats_d<128>(k, v, v_sums, G, N, out, st);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_quant_d(const QuantArgs& a, hipStream_t st) {
  const int maxblk = (a.with_q && a.blk_q > a.blk_k) ? a.blk_q : a.blk_k;
  const int grid = a.G * (a.nkb + (a.with_q ? a.nqb : 0));
  constexpr int RPI = kThreads / (D / 8);
  if (maxblk <= 32 && 32 % RPI == 0)
    quant_kernel<D, (32 > RPI ? 32 : RPI)><<<grid, kThreads, 0, st>>>(a);
  else if (maxblk <= 64)
    quant_kernel<D, 64><<<grid, kThreads, 0, st>>>(a);
  else
    quant_kernel<D, 128><<<grid, kThreads, 0, st>>>(a);
  return hipGetLastError();
}

hipError_t launch_quant(int d, const QuantArgs& a, hipStream_t st) {
  return d == 64 ? launch_quant_d<64>(a, st) : launch_quant_d<128>(a, st);
}

// ---------------------------------------------------------------------------
// Variant 2: Q and K' to MXFP4 per token (OCP microscaling: blocks of 32 channels,
// one E8M0 scale each, E2M1 elements).  One thread per (token, block): it reads the
// block's 32 fp16 values, subtracts K's token mean (smooth_k), and writes 16 bytes of
// codes (two per byte, the lower channel in the low nibble) and one scale byte.

template <int D>
__global__ __launch_bounds__(kThreads) void quant_mx_kernel(const uint16_t* __restrict__ x, int N, int Np,
                                                            int nsplit, const long long* __restrict__ ksum_part,
                                                            int smooth, uint8_t* __restrict__ codes,
                                                            uint8_t* __restrict__ e8, float* __restrict__ k_mean) {
  constexpr int BPT = D / 32;             // blocks per token
  constexpr int TOK = kThreads / BPT;     // tokens per workgroup
  __shared__ float s_mean[D];
  const int ntiles = Np / TOK;  // 1-D grid over (head, tile of TOK tokens)
  const int tb = blockIdx.x % ntiles, g = blockIdx.x / ntiles, tid = threadIdx.x;
  if (tid < D) {
    float m = 0.0f;
    if (smooth) {
      m = fixed24_mean(ksum_part[(size_t)g * nsplit * D + tid], N);  // folded into split 0
      if (tb == 0 && k_mean) k_mean[(size_t)g * D + tid] = m;
    }
    s_mean[tid] = m;
  }
  __syncthreads();
  const int t = tb * TOK + tid / BPT, b = tid % BPT;
  if (t >= Np) return;
  uint4 packed = make_uint4(0u, 0u, 0u, 0u);
  uint32_t scode = 0;
  if (t < N) {
    const uint16_t* src = x + ((size_t)g * N + t) * D + 32 * b;
    float v[32];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint4 raw = *reinterpret_cast<const uint4*>(src + 8 * i);
      const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f16x2 hv = __builtin_bit_cast(f16x2, w[j]);
        v[8 * i + 2 * j] = (float)hv[0] - s_mean[32 * b + 8 * i + 2 * j];
        v[8 * i + 2 * j + 1] = (float)hv[1] - s_mean[32 * b + 8 * i + 2 * j + 1];
      }
    }
    scode = mx_block_fp4(v, packed);
  }
  *reinterpret_cast<uint4*>(codes + ((size_t)g * Np + t) * (D / 2) + 16 * b) = packed;
  e8[((size_t)g * Np + t) * BPT + b] = (uint8_t)scode;
}

hipError_t launch_quant_mx(int d, const void* x, int G, int N, int Np, const long long* ksum_part, int smooth,
                           uint8_t* codes, uint8_t* e8, float* k_mean, hipStream_t st) {
  const int ns = stat_splits(N);
  if (d == 64) {
    const int grid = Np / (kThreads / 2) * G;
    quant_mx_kernel<64><<<grid, kThreads, 0, st>>>((const uint16_t*)x, N, Np, ns, ksum_part, smooth, codes, e8, k_mean);
  } else {
    const int grid = Np / (kThreads / 4) * G;
    quant_mx_kernel<128><<<grid, kThreads, 0, st>>>((const uint16_t*)x, N, Np, ns, ksum_part, smooth, codes, e8, k_mean);
  }
  return hipGetLastError();
}

// Variant 3: V -> MXFP4 along the tokens (the contraction dimension of P~ V): for each
// channel, blocks of 32 consecutive tokens get one E8M0 scale and 32 E2M1 codes (the
// OCP rule of mx_block_fp4), after the exact token mean with V smoothing.  Tokens >= N
// are zeros.  One workgroup per (64-token tile, head): the tile goes through LDS as
// fp32 so the fp16 reads run along the channels and each thread then codes one
// (channel, 32-token block).
//   v_f4 [G][D][Np/2]: two codes per byte, the lower token in the low nibble;
//   v_e8 [G][Np/32][D]: the scale of channel c sits at (c % 32) * (D/32) + c / 32, so the
//        D/32 scales one lane of the P~ V product needs (channels r, r+32, ..) are adjacent.
template <int D>
__global__ __launch_bounds__(kThreads) void quant_v_mx_kernel(const uint16_t* __restrict__ v, int N, int Np,
                                                              int nsplit, const long long* __restrict__ vsum_part,
                                                              int smooth_v, uint8_t* __restrict__ v_f4,
                                                              uint8_t* __restrict__ v_e8,
                                                              float* __restrict__ v_mean) {
  constexpr int TPR = D / 8;
  constexpr int RPI = kThreads / TPR;
  constexpr int TT = 64;  // tokens per tile
  __shared__ float s_mean[D];
  __shared__ float s_t[D][TT + 1];
  const int ntiles = Np / TT;  // 1-D grid over (head, 64-token tile)
  const int tile = blockIdx.x % ntiles, g = blockIdx.x / ntiles, tid = threadIdx.x;
  if (tid < D) {
    const float mean = smooth_v ? fixed24_mean(vsum_part[(size_t)g * nsplit * D + tid], N) : 0.0f;
    s_mean[tid] = mean;
    if (tile == 0 && v_mean) v_mean[(size_t)g * D + tid] = mean;
  }
  __syncthreads();
  const int cg = tid % TPR, r0 = tid / TPR;
  const size_t head = (size_t)g * N * D;
  for (int rr = r0; rr < TT; rr += RPI) {
    const int t = tile * TT + rr;
    uint4 raw = make_uint4(0, 0, 0, 0);
    if (t < N) raw = *reinterpret_cast<const uint4*>(v + head + (size_t)t * D + cg * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
    const bool centre = smooth_v && t < N;  // padding tokens stay zero
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const f16x2 h = __builtin_bit_cast(f16x2, w[j]);
      const int c = cg * 8 + 2 * j;
      s_t[c][rr] = centre ? (float)h[0] - s_mean[c] : (float)h[0];
      s_t[c + 1][rr] = centre ? (float)h[1] - s_mean[c + 1] : (float)h[1];
    }
  }
  __syncthreads();
  if (tid < 2 * D) {
    const int c = tid % D, b = tid / D;  // channel, 32-token block of the tile
    float x[32];
#pragma unroll
    for (int u = 0; u < 32; ++u) x[u] = s_t[c][32 * b + u];
    uint4 packed;
    const uint32_t code = mx_block_fp4(x, packed);
    *reinterpret_cast<uint4*>(v_f4 + ((size_t)g * D + c) * (Np / 2) + tile * (TT / 2) + 16 * b) = packed;
    v_e8[((size_t)g * (Np / 32) + 2 * tile + b) * D + (c % 32) * (D / 32) + c / 32] = (uint8_t)code;
  }
}

hipError_t launch_quant_v_mx(int d, const void* v, int G, int N, int Np, const long long* vsum_part, int smooth_v,
                             uint8_t* v_f4, uint8_t* v_e8, float* v_mean, hipStream_t st) {
  const int grid = Np / 64 * G;
  const int ns = stat_splits(N);
  if (d == 64)
    quant_v_mx_kernel<64><<<grid, kThreads, 0, st>>>((const uint16_t*)v, N, Np, ns, vsum_part, smooth_v, v_f4, v_e8,
                                                     v_mean);
  else
    quant_v_mx_kernel<128><<<grid, kThreads, 0, st>>>((const uint16_t*)v, N, Np, ns, vsum_part, smooth_v, v_f4, v_e8,
                                                      v_mean);
  return hipGetLastError();
}

hipError_t launch_quant_v(int d, const void* v, int G, int N, int Np, const StatsOut& stats, int smooth_v,
                          uint8_t* v_f8, float* v_scale, float* v_mean, hipStream_t st) {
  const int grid = Np / 64 * G;
  const int ns = stat_splits(N);
  if (d == 64)
    quant_v_kernel<64><<<grid, kThreads, 0, st>>>((const uint16_t*)v, N, Np, ns, stats.vsum, stats.vmax, stats.vmin,
                                                  smooth_v, v_f8, v_scale, v_mean);
  else
    quant_v_kernel<128><<<grid, kThreads, 0, st>>>((const uint16_t*)v, N, Np, ns, stats.vsum, stats.vmax,
                                                   stats.vmin, smooth_v, v_f8, v_scale, v_mean);
  return hipGetLastError();
}

}  // namespace sage
