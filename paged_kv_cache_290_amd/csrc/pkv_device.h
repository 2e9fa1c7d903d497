// Device-side helpers for the gfx950 kernels of libpagedkv (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkv {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef short v4i16_t __attribute__((ext_vector_type(4)));

// bf16 is carried as raw 16-bit storage.  Widening is exact: the 16 bits are the top
// half of a float32.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 with round-to-nearest-even (gfx950 lowers this to v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}
// Two floats -> packed bf16 pair (lo in bits 0-15), RNE, one v_cvt_pk_bf16_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{lo, hi}, bf16x2_t));
}

// Sum of a*b over the two bf16 lanes of each operand, accumulated into c in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), c, false);
}

// Cross-lane moves.  DPP controls (GFX9 encoding): quad_perm is an 8-bit lane map
// inside each group of 4 lanes; 0x120 + n rotates right by n inside each row of 16.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}
constexpr int kQuadSwap1 = 0xB1;  // lanes (1,0,3,2)
constexpr int kQuadSwap2 = 0x4E;  // lanes (2,3,0,1)
constexpr int kRowRor4 = 0x124;
constexpr int kRowRor8 = 0x128;
constexpr int kRowMirror = 0x140;      // lane i <- lane 15-i inside each row of 16
constexpr int kRowHalfMirror = 0x141;  // lane i <- lane 7-i inside each half row of 8

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  return __shfl_xor(x, mask, 64);
}

// Max over the 16 lanes that share (lane & 3): the 4-lane quads hold equal values.
__device__ __forceinline__ float wave_max_over_quads(float x) {
  x = fmaxf(x, dpp<kRowRor4>(x));
  x = fmaxf(x, dpp<kRowRor8>(x));
  x = fmaxf(x, shfl_xor(x, 16));
  x = fmaxf(x, shfl_xor(x, 32));
  return x;
}

// Transposing 8-byte LDS read of 16-bit elements (ds_read_b64_tr_b16).  Within each
// 16-lane group, lane i receives element i % 4 of the 8-byte rows addressed by lanes
// 4j + i / 4 of the group, j = 0..3 (element j of the result from row j).
__device__ __forceinline__ v4i16_t lds_read_tr16(const void *p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) v4i16_t *)(p));
}

__device__ __forceinline__ bool wave_any(bool p) {
  return __builtin_amdgcn_ballot_w64(p) != 0;
}

__device__ __forceinline__ int readlane(int x, int lane) {
  return __builtin_amdgcn_readlane(x, lane);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer access.  A descriptor covers `bytes` from `base` (stride 0); a load at an
// offset outside that range fetches nothing from memory and returns zeros.
typedef __amdgpu_buffer_rsrc_t buffer_rsrc_t;
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family data format word (32-bit elements)

__device__ __forceinline__ buffer_rsrc_t make_rsrc(const void *base, int bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes,
                                           kRsrcWord3);
}
__device__ __forceinline__ uint4 buffer_load16(buffer_rsrc_t r, int offset) {
  const u32x4_t x = __builtin_amdgcn_raw_buffer_load_b128(r, offset, 0, 0);
  return uint4{x.x, x.y, x.z, x.w};
}

// Workgroups are dispatched round-robin over the 8 XCDs (each with its own L2): XCD x
// receives workgroups x, x+8, x+16, ...  This maps the hardware index to a virtual one
// so that each XCD receives one contiguous range of virtual work, keeping work items
// that share data on one L2.  It is a bijection of [0, grid) for every grid size: XCD
// x holds grid/8 workgroups, plus one when x < grid%8.
__device__ __forceinline__ int xcd_remap(int wg, int grid) {
  const int x = wg & 7;
  return x * (grid >> 3) + min(x, grid & 7) + (wg >> 3);
}

// Sequence owning global query row `row`: the last s with qsl[s] <= row.
__device__ __forceinline__ int find_seq(const int32_t *qsl, int num_seqs, int row) {
  int lo = 0, hi = num_seqs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (qsl[mid] <= row) lo = mid; else hi = mid - 1;
  }
  return lo;
}

}  // namespace pkv
