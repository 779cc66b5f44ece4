// sage_device.h -- gfx950 device helpers shared by the quantisation and attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sage {

typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x16 __attribute__((ext_vector_type(16)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;   // 4 waves of 64
constexpr int kBlockQ = 128;    // query rows per attention workgroup (32 per wave)
constexpr int kTileKV = 64;     // keys per online-softmax tile
constexpr int kPad = 128;       // the int8 / fp8 tensors are padded to a multiple of this
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLog2_448 = 8.807354922057604f;  // log2(448): P~ * 448 is exp2(x + log2 448)

// ---- MFMA (gfx950).  32x32 output tile: lane l, register i holds row
// 8*(i/4) + 4*(l/32) + i%4, column l%32.  Operand A: lane l holds row l%32 and the
// k-slots of half l/32; operand B: column l%32, the same k-slots.
__device__ __forceinline__ i32x16 mfma_i8(i32x4 a, i32x4 b, i32x16 c) {
  return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// FP8 E4M3 (OCP) x FP8 E4M3, fp32 accumulation; unit scales select the plain instruction.
__device__ __forceinline__ f32x16 mfma_f8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

// Value of the same register in lane l ^ 32.  v_permlane32_swap exchanges the upper
// half of the first operand with the lower half of the second; with both equal to x,
// result[0] = (x[0..31], x[0..31]) and result[1] = (x[32..63], x[32..63]).
__device__ __forceinline__ float pair_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float pair_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LDS transpose read of 16-bit data: inside each group of 16 lanes, lane i receives
// element i%4 of the 4-element rows addressed by lanes 4e + i/4 (e = 0..3).
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_ptr) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
}

// fp16 bits -> value * 2^24 as an exact integer (every fp16 is a multiple of 2^-24).
__device__ __forceinline__ long long f16_bits_to_fixed24(uint32_t h) {
  uint32_t e = (h >> 10) & 31u, m = h & 1023u;
  long long mag = e ? ((long long)(1024u + m) << (e - 1)) : (long long)m;
  return (h & 0x8000u) ? -mag : mag;
}

// Exact fixed-point sum (units of 2^-24) divided by count: one correctly rounded fp64
// division, then round to fp32.
__device__ __forceinline__ float fixed24_mean(long long sum, int count) {
  return (float)((double)sum / ((double)count * 16777216.0));
}

// Round to nearest even and pack two floats as OCP E4M3 into the low (hi = false) or
// high half of `old`.  Inputs must already lie in [-448, 448].
__device__ __forceinline__ uint32_t cvt_pk_fp8(float a, float b, uint32_t old, bool hi) {
  return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
            : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

// Per-block INT8 quantisation of Q and K: scale = absmax / 127, code = x * (127 / absmax)
// rounded to nearest even and saturated at +-127 (an all-zero block gets factor 0).
// Every kernel that quantises goes through these, so their codes and scales agree bit
// for bit.
// (x * r is formed as fma(x, r, +0): the same fp32 value, except that -0 becomes +0,
// which gives the same code.)
__device__ __forceinline__ float i8_scale(float amax) { return amax / 127.0f; }
__device__ __forceinline__ float i8_factor(float amax) { return amax > 0.0f ? 127.0f / amax : 0.0f; }
__device__ __forceinline__ int i8_code_int(float x, float r) {
  float t = rintf(__builtin_fmaf(x, r, 0.0f));
  t = fminf(fmaxf(t, -127.0f), 127.0f);
  return (int)t;
}
__device__ __forceinline__ uint32_t i8_code(float x, float r) { return (uint32_t)i8_code_int(x, r) & 0xffu; }
// Low bytes of four ints packed as bytes 0..3.
__device__ __forceinline__ uint32_t pack_bytes4(int c0, int c1, int c2, int c3) {
  const uint32_t lo = __builtin_amdgcn_perm((uint32_t)c1, (uint32_t)c0, 0x0c0c0400u);
  const uint32_t hi = __builtin_amdgcn_perm((uint32_t)c3, (uint32_t)c2, 0x0c0c0400u);
  return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

// Maximum of x over the 64 lanes of the wave (rows of 16 lanes by DPP, then the row
// pairs and the two halves by permlane swaps).
__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false)));  // quad [1,0,3,2]
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false)));  // quad [2,3,0,1]
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x124, 0xF, 0xF, false))); // row_ror 4
  x = fmaxf(x, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x128, 0xF, 0xF, false))); // row_ror 8
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  auto r2 = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r2[0]), __uint_as_float(r2[1]));
}

// MXFP4 (OCP microscaling) of one block of 32 values: the E8M0 scale code
// floor(log2 max|v|) - 2 + 127 clamped to [0, 254] (0 for an all-zero block) and the 32
// E2M1 codes of v / 2^(code - 127), two per byte with the lower index in the low nibble.
// The quantisation pass and the attention kernel's fused prologue both use this.
// E2M1 rounding: to nearest with ties to the even code (0.25 -> 0, 0.75 -> 1,
// 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4), saturating at 6, sign kept (also of
// zero).
__device__ __forceinline__ uint32_t e2m1_code(float v) {
  const float a = fabsf(v);
  const uint32_t m = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
                     (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) + (uint32_t)(a > 5.0f);
  return m | ((__float_as_uint(v) >> 28) & 8u);
}
__device__ __forceinline__ uint32_t mx_block_fp4(const float* v, uint4& packed) {
  float am = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) am = fmaxf(am, fabsf(v[i]));
  // frexp_exp(am) = floor(log2 am) + 1
  const uint32_t code = am > 0.0f ? (uint32_t)min(max(__builtin_amdgcn_frexp_expf(am) - 1 - 2 + 127, 0), 254) : 0u;
  const int sh = 127 - (int)code;  // elements are v * 2^sh, exact
  uint32_t word[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 32; i += 2) {
    // v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds exactly like e2m1_code (checked on
    // MI355X over the ties, the saturation range, signed zeros and 50k random values);
    // the first value lands in the low nibble
    const uint32_t pair = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, __builtin_amdgcn_ldexpf(v[i], sh),
                                                                   __builtin_amdgcn_ldexpf(v[i + 1], sh), 1.0f, 0);
    word[i / 8] |= (pair & 0xffu) << (4 * (i % 8));
  }
  packed = make_uint4(word[0], word[1], word[2], word[3]);
  return code;
}

// acc + the two fp16 values of a packed word (v_dot2_f32_f16 against ones: the products are
// exact, the sum is in fp32).
__device__ __forceinline__ float sum_f16x2(uint32_t packed, float acc) {
  const f16x2 ones = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, packed), ones, acc, false);
}
__device__ __forceinline__ uint32_t pack_f16x2(float a, float b) {
  f32x2 v = {a, b};
  f16x2 h = __builtin_convertvector(v, f16x2);  // v_cvt_pk_f16_f32, round to nearest even
  return __builtin_bit_cast(uint32_t, h);
}

}  // namespace sage
