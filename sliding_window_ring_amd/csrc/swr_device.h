// swr_device.h -- device-side building blocks for gfx950 (CDNA4) kernels:
// vector types, bf16 / OCP-fp8 conversion, the bf16 MFMA wrapper, bounded
// buffer loads and wave-level reductions.  Written for gfx950 only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

// Third word of a raw buffer resource on gfx9-family parts (gfx950 included):
// 32-bit data format, no swizzle.  Reads past num_records return zero and
// writes past it are dropped, so every region access is bounded in hardware.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           kBufferWord3);
}

__device__ __forceinline__ u32x4 load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// Streaming read: the non-temporal cache policy (bit 1 of the aux operand on
// gfx94x/gfx950) marks lines read once, so K/V streams do not evict reused data.
__device__ __forceinline__ u32x4 load16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 2);
}

__device__ __forceinline__ u32x2 load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
}

__device__ __forceinline__ void store16(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, off, 0, 0);
}

__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, uint32_t off, u32x2 v) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, off, 0, 0);
}

__device__ __forceinline__ void store2(__amdgpu_buffer_rsrc_t r, uint32_t off, uint16_t v) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, off, 0, 0);
}

__device__ __forceinline__ void store1(__amdgpu_buffer_rsrc_t r, uint32_t off, uint8_t v) {
  __builtin_amdgcn_raw_buffer_store_b8(v, r, off, 0, 0);
}

// 8 OCP e4m3 codes (two dwords, code i in byte i) -> 8 bf16, exact
// (every e4m3 value is a bf16 value).  Uses the gfx950 conversion with a unit
// scale; the per-tensor scale is applied by the caller outside the MFMA.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(u32x2 c) {
  bf16x2 a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, false);
  bf16x2 b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[0], 1.0f, true);
  bf16x2 e = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, false);
  bf16x2 f = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c[1], 1.0f, true);
  return bf16x8{a[0], a[1], b[0], b[1], e[0], e[1], f[0], f[1]};
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) { return __builtin_bit_cast(bf16x8, v); }

// Region layout (one request's K or V for one layer).  Per KV head a region
// stores S = cap rounded up to 32 slots.
//   K: tiles of 32 slots.  Slot 32t + k sits in half h = (k/4)%2, row
//      r = 4*(k/8) + k%4 of tile t -- row r of half h is exactly MFMA A row r
//      of the score sub-tile h (keys 8*(r/4) + 4h + r%4), whose C fragment
//      is the P^T fragment of the value product.  Each half holds its 16
//      rows granule-major: D/R granules of 16 rows x 16 bytes (R = 8 bf16 or
//      16 fp8 dims), so one lane group's operand load (4 granules x 16 rows)
//      is 1 KB of contiguous memory.
//        byte offset = ((g*S + 32t)*D + h*16*D)*esize + (d/R)*256 + r*16 + (d%R)*esize
//   V: blocks of 8 slots, ((g*(S/8) + slot/8)*D + d)*8 + slot%8 elements:
//      one 16-byte load is 8 consecutive keys of one dim (the V^T operand).
// (stored_slots: swr_internal.h)

// Byte offset of K granule (slot-half base, granule q, row r): the start of
// the half is ((g*S + 32t)*D + h*16*D)*esize.
__device__ __forceinline__ uint32_t k_half_base(int g, int S, int tile_slot0, int half, int D, int esize) {
  return ((uint32_t)(g * S + tile_slot0) * (uint32_t)D + (uint32_t)(half * 16 * D)) * (uint32_t)esize;
}

// D = A(16x32) * B(32x16) + C with bf16 inputs and fp32 accumulation.
// Lane l supplies row (l % 16) of A and column (l % 16) of B, each as 8
// k-values of lane group l / 16; lane l receives C rows 4*(l/16) .. +3 of
// column l % 16.  A and B use the same k assignment per (lane group, element),
// so any fixed permutation of the k axis applied to both leaves D unchanged.
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Reductions over the four lanes l, l^16, l^32, l^48 (the lanes that hold
// one C column of a 16x16 MFMA tile).
__device__ __forceinline__ float max4lanes(float v) {
  v = fmaxf(v, __shfl_xor(v, 16));
  v = fmaxf(v, __shfl_xor(v, 32));
  return v;
}

__device__ __forceinline__ float sum4lanes(float v) {
  v += __shfl_xor(v, 16);
  v += __shfl_xor(v, 32);
  return v;
}

// Reductions over the 16 lanes of a DPP row (lanes 16k .. 16k+15), every
// lane receiving the result: swaps within quads, then the half-row mirror
// (quad 0 <-> 1, 2 <-> 3) and the row mirror (half 0 <-> 1).  Each step pairs
// lanes symmetrically, so all 16 lanes end with the same value.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
constexpr int kDppQuadSwap1 = 0xB1;   // quad_perm [1,0,3,2]
constexpr int kDppQuadSwap2 = 0x4E;   // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

__device__ __forceinline__ float max16lanes(float v) {
  v = fmaxf(v, dpp_move<kDppQuadSwap1>(v));
  v = fmaxf(v, dpp_move<kDppQuadSwap2>(v));
  v = fmaxf(v, dpp_move<kDppRowHalfMirror>(v));
  v = fmaxf(v, dpp_move<kDppRowMirror>(v));
  return v;
}

__device__ __forceinline__ float sum16lanes(float v) {
  v += dpp_move<kDppQuadSwap1>(v);
  v += dpp_move<kDppQuadSwap2>(v);
  v += dpp_move<kDppRowHalfMirror>(v);
  v += dpp_move<kDppRowMirror>(v);
  return v;
}

__device__ __forceinline__ uint16_t bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (__bf16)x);
}

}  // namespace swr
