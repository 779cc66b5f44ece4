// sage_tiles.h -- LDS tile layouts, global->LDS tile copies and the INT8 score product on
// the gfx950 matrix unit, shared by the attention forward and backward kernels.
#pragma once

#include "sage_device.h"

namespace sage {

// LDS tiles are written straight from memory (global_load_lds_dwordx4 /
// buffer_load_dwordx4 ... lds: lane l of a wave writes 16 bytes at base + 16*l), so a
// tile is an array of 16-byte slots whose order the copy chooses freely.  Each tile
// is stored in the order the MFMA operand reads consume it: every read pass of a wave
// (8 lanes of ds_read_b128, 16 lanes of ds_read_b64_tr_b16) covers one contiguous
// 128-byte run, which is free of bank conflicts, and every operand address is the
// lane's base plus a compile-time offset.
// Bytes per Q / K row: D int8 codes, or D/2 bytes of two E2M1 codes (variants 2, 3).
template <int D, int VARIANT>
constexpr int qk_row_bytes() { return VARIANT >= 2 ? D / 2 : D; }

template <int D, int VARIANT>
struct Lds {
  static constexpr int K_BYTES = kTileKV * qk_row_bytes<D, VARIANT>();  // 64 keys
  static constexpr int V_BYTES = VARIANT == 0   ? kTileKV * D * 2     // 64 keys x D fp16
                                 : VARIANT == 3 ? D * kTileKV / 2     // D channels x 64 keys E2M1
                                                : D * kTileKV;        // D channels x 64 keys fp8
};

// Row of the K tile that feeds A-operand row r: accumulator register i of lane half h
// then holds key 16h + i of the 32-key block.
__device__ __forceinline__ int k_perm(int r) { return 16 * ((r >> 2) & 1) + 4 * (r >> 3) + (r & 3); }

// Key (within the 64-key tile) of A-operand row r of the S^T product of 32-key block st.
// Variants 0-2: key 32*st + k_perm(r), so register i of lane half h is key 32*st + 16h + i.
// Variant 3 interleaves the two products so that lane half h holds the 32 consecutive
// keys 32h .. 32h + 31 (register i of product st is key 32h + 16*st + i): one MX block of
// P~ per lane, the k-slots of its half of the FP4 P~ V operand.
template <int VARIANT>
__device__ __forceinline__ int k_row_key(int st, int r) {
  return VARIANT == 3 ? 32 * ((r >> 2) & 1) + 16 * st + 4 * (r >> 3) + (r & 3) : 32 * st + k_perm(r);
}

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* gbl_ptr_t;

__device__ __forceinline__ void wait_copies() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Index of this wave in the workgroup as a scalar, so LDS destinations of the tile
// copies (M0) are formed with scalar instructions.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }

// K tile: slot (st*CPR + c)*32 + x holds bytes 16c..16c+15 of key 32*st + k_perm(x),
// x = A-operand row.  Lane l of the operand read for 32-key block st, k-step ks, is
// at 16*l + (st*CPR + 2*ks)*512.
template <int D>
__device__ __forceinline__ int k_slot(int key, int chunk) {
  constexpr int CPR = D / 16;
  return ((key >> 5) * CPR + chunk) * 32 + 8 * ((key >> 2) & 3) + 4 * ((key >> 4) & 1) + (key & 3);
}

__device__ __forceinline__ void copy16_to_lds(__amdgpu_buffer_rsrc_t rs, uint32_t voff, uint32_t soff,
                                              void* lds_wave_base) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_ptr_t)lds_wave_base, 16, voff, soff, 0, 0);
}

// Source offsets of the tile copies.  The waves of the workgroup split a tile's 1 KB
// copy instructions round-robin; copy i of a wave starts (i * NWAVES) KB after its
// first one in LDS and a fixed number of bytes after it in memory, so each lane keeps
// one base offset per tensor, and tile t adds a uniform t * (bytes per tile).
template <int D, int VARIANT, int NWAVES>
struct TileCopy {
  static constexpr int KD = qk_row_bytes<D, VARIANT>();  // bytes per K row
  static constexpr int CPR = KD / 16;
  static constexpr int K_COPIES = kTileKV * CPR / 64;                                      // 1 KB each
  static constexpr int V_COPIES = Lds<D, VARIANT>::V_BYTES / 16 / 64;
  static constexpr int K_PER_WAVE = (K_COPIES + NWAVES - 1) / NWAVES;
  static constexpr int V_PER_WAVE = (V_COPIES + NWAVES - 1) / NWAVES;
  // memory distance between copy c and copy c + NWAVES of a lane (see the layouts above)
  static constexpr uint32_t K_STEP = (uint32_t)((NWAVES * 2) / CPR) * 32 * KD;
  static constexpr uint32_t V_STEP = VARIANT == 0 ? (uint32_t)(NWAVES * 8 / (D / 16)) * 4 * 2 * D
                                                  : (uint32_t)(NWAVES * 2 / 4) * 32;  // channels (x Np)
  uint32_t koff, voff;

  __device__ __forceinline__ TileCopy(int Np) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    {
      const int s = (wave % K_COPIES) * 64 + lane;
      const int x = s & 31, rest = s >> 5;
      koff = (uint32_t)k_row_key<VARIANT>(rest / CPR, x) * KD + (rest % CPR) * 16;
    }
    {
      const int s = (wave % V_COPIES) * 64 + lane;
      if (VARIANT == 0) {
        constexpr int BPR = D / 16;
        const int w = s & 7, blk = s >> 3;
        voff = (uint32_t)(4 * (blk / BPR) + (w >> 1)) * (2 * D) + 2 * (16 * (blk % BPR) + 8 * (w & 1));
      } else if (VARIANT == 3) {
        // copy c: channels 32c .. 32c + 31; lane l takes channel 32c + l%32, keys 32h .. 32h + 31
        // of the tile (h = l/32), the 16 bytes its P~ V operand reads
        voff = (uint32_t)(32 * (s >> 6) + (lane & 31)) * (uint32_t)(Np / 2) + 16 * (lane >> 5);
      } else {
        const int y = s & 31, rest = s >> 5;
        voff = (uint32_t)(32 * (rest >> 2) + y) * Np + 16 * (rest & 3);
      }
    }
    static_assert((NWAVES * 2) % CPR == 0, "K copies of one wave must step by whole 32-key blocks");
    static_assert(VARIANT != 3 || (K_PER_WAVE == 1 && V_PER_WAVE == 1), "variant 3: one K and one V copy per wave");
    static_assert(VARIANT != 0 || (NWAVES * 8) % (D / 16) == 0, "V copies must step by whole key rows");
    static_assert(VARIANT == 0 || (NWAVES * 2) % 4 == 0, "V^T copies must step by whole channel rows");
  }

  // K tile t of the padded int8 / packed-E2M1 tensor (resource over this head); the
  // tile and copy steps go in the scalar offset.
  __device__ __forceinline__ void k_tile(__amdgpu_buffer_rsrc_t krs, int t, int8_t* sK) const {
    const int wave = wave_id();
#pragma unroll
    for (int i = 0; i < K_PER_WAVE; ++i) {
      const int c = i * NWAVES + wave;
      if (K_COPIES % NWAVES == 0 || c < K_COPIES)
        copy16_to_lds(krs, koff, (uint32_t)(t * kTileKV * KD) + i * K_STEP, sK + c * 1024);
    }
  }
  // V tile t.  Variant 0 puts the whole offset in the lane offset so keys >= N fall
  // outside the resource and land as zeros.
  __device__ __forceinline__ void v_tile(__amdgpu_buffer_rsrc_t vrs, int t, int Np, uint8_t* sV) const {
    const int wave = wave_id();
#pragma unroll
    for (int i = 0; i < V_PER_WAVE; ++i) {
      const int c = i * NWAVES + wave;
      if (V_COPIES % NWAVES == 0 || c < V_COPIES) {
        if (VARIANT == 0)
          copy16_to_lds(vrs, voff + i * V_STEP + (uint32_t)(t * kTileKV * 2 * D), 0u, sV + c * 1024);
        else if (VARIANT == 3)
          copy16_to_lds(vrs, voff, (uint32_t)(t * kTileKV / 2), sV + c * 1024);
        else
          copy16_to_lds(vrs, voff + i * V_STEP * (uint32_t)Np, (uint32_t)(t * kTileKV), sV + c * 1024);
      }
    }
  }
};

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, size_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (uint32_t)bytes, 0x00020000);
}

// Q operand (B of S^T = K Q^T): each wave copies its 32 query rows into LDS once, as
// D/32 runs of 64 lanes x 16 bytes (lane l: row l%32, bytes 32*ks + 16*(l/32)), so the
// operand read of k-step ks is at wave base + ks*1024 + 16*l.
template <int D>
__device__ __forceinline__ void load_q_tile(__amdgpu_buffer_rsrc_t qrs, int row0, int8_t* sQw) {
  const int lane = threadIdx.x & 63;
  const uint32_t off = (uint32_t)(row0 + (lane & 31)) * D + 16 * (lane >> 5);
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) copy16_to_lds(qrs, off + 32 * ks, 0u, sQw + ks * 1024);
}

// S^T for the 64-key tile in LDS: s[st][i] = Qhat[query l%32] . Khat[key 32*st + 16h + i]
// (exact int32).
template <int D>
__device__ __forceinline__ void qk_tile(const int8_t* sK, const int8_t* sQw, int lane, i32x16* s) {
  constexpr int CPR = D / 16;
  const int8_t* kbase = sK + 16 * lane;
  const int8_t* qbase = sQw + 16 * lane;
  // the two 32-key accumulation chains alternate, so consecutive MFMAs are independent
  i32x16 acc[2] = {i32x16{}, i32x16{}};
#pragma unroll
  for (int ks = 0; ks < D / 32; ++ks) {
    const i32x4 qop = *reinterpret_cast<const i32x4*>(qbase + ks * 1024);
#pragma unroll
    for (int st = 0; st < 2; ++st)
      acc[st] = mfma_i8(*reinterpret_cast<const i32x4*>(kbase + (st * CPR + 2 * ks) * 512), qop, acc[st]);
  }
  s[0] = acc[0];
  s[1] = acc[1];
}

// K scales of the four 16-key quarters of tile t (blk_k = 2^kshift, keys clamped to
// the last one, so any t reads inside the array).  A quarter's block is the same for the
// whole wave, so these are scalar loads (off the vector-memory path of the tile copies);
// lane half h of 32-key block st then takes quarter 2*st + h (kscale_of).
__device__ __forceinline__ void tile_kscales(const float* ksc, int t, unsigned last_key, int kshift,
                                             float* kq) {
  // the scales are read-only while the kernel runs: read them through the constant
  // address space, which allows scalar loads
  typedef const __attribute__((address_space(4))) float* const_ptr;
  const const_ptr kc = (const_ptr)ksc;
  if (kshift >= 6) {  // blocks of 64 keys or more: one K block covers the tile (one load)
    const float v = kc[min((unsigned)(t * kTileKV), last_key) >> kshift];
    kq[0] = kq[1] = kq[2] = kq[3] = v;
    return;
  }
#pragma unroll
  for (int j = 0; j < 4; ++j) kq[j] = kc[min((unsigned)(t * kTileKV + 16 * j), last_key) >> kshift];
}
__device__ __forceinline__ float kscale_of(const float* kq, int st, int h) { return h ? kq[2 * st + 1] : kq[2 * st]; }
// KT (blk_k >= 64, known at compile time): the tile's one K scale, in kq[0] only.
template <bool KT>
__device__ __forceinline__ void tile_kscales_for(const float* ksc, int t, unsigned last_key, int kshift, float* kq) {
  if constexpr (KT) {
    typedef const __attribute__((address_space(4))) float* const_ptr;
    kq[0] = ((const_ptr)ksc)[min((unsigned)(t * kTileKV), last_key) >> kshift];
  } else {
    tile_kscales(ksc, t, last_key, kshift, kq);
  }
}
// K scale of the 16 keys 16*w .. of tile t (w uniform: a scalar load).
__device__ __forceinline__ float kscale_quarter(const float* ksc, int t, int w, unsigned last_key, int kshift) {
  typedef const __attribute__((address_space(4))) float* const_ptr;
  return ((const_ptr)ksc)[min((unsigned)(t * kTileKV + 16 * w), last_key) >> kshift];
}

// O^T += V^T P~^T for one 64-key tile with fp16 operands (v_mfma_f32_32x32x16_f16): the
// V tile is [64 keys][D channels] fp16 in the layout TileCopy::v_tile writes (read with
// the LDS transpose read, so lane j of a 16-lane group gets channel C0 + j of 4 keys); pk
// holds P~ as fp16 pairs in the layout of the S^T accumulator (pk[st*8 + u*4 + q]: keys
// 8u + 2q, 8u + 2q + 1 of the lane's 16 keys in 32-key block st).  The same product
// serves any pair (tile of rows x D fp16, packed fp16 weights of those rows).
// vbase = the tile + pv_lane_offset<D>(lane).
template <int D>
__device__ __forceinline__ int pv_lane_offset(int lane) {
  const int G16 = lane >> 4, j16 = lane & 15;
  return 128 * (4 * (G16 >> 1) * (D / 16) + (G16 & 1)) + 8 * j16;
}
template <int D>
__device__ __forceinline__ void pv_tile_f16(const uint8_t* vbase, const uint32_t* pk, f32x16* o) {
  constexpr int NCT = D / 32;
#pragma unroll
  for (int st = 0; st < 2; ++st)
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const uint32_t pq[4] = {pk[st * 8 + u * 4], pk[st * 8 + u * 4 + 1], pk[st * 8 + u * 4 + 2], pk[st * 8 + u * 4 + 3]};
      const f16x8 pb = __builtin_bit_cast(f16x8, pq);
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const i16x4 a0 = lds_read_tr16(vbase + 128 * ((8 * st + 2 * u) * (D / 16) + 2 * ct));
        const i16x4 a1 = lds_read_tr16(vbase + 128 * ((8 * st + 2 * u + 1) * (D / 16) + 2 * ct));
        const i16x4 a01[2] = {a0, a1};
        o[ct] = mfma_f16(__builtin_bit_cast(f16x8, a01), pb, o[ct]);
      }
    }
}

}  // namespace sage
