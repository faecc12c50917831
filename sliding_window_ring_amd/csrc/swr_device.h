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

// A 16-byte load from global memory through a pointer the compiler is told
// is global.  Where its address-space inference loses track of a pointer
// taken from the kernel's arguments it emits a flat load instead, which also
// counts on the LDS counter: the next LDS access then waits for every load
// in flight, not just this one (measured 0.2 us on a verify call).
__device__ __forceinline__ u32x4 load16_global(const void* ptr) {
  return *(const __attribute__((address_space(1))) u32x4*)ptr;
}

// A value the caller knows is the same in every lane of the wave (a load
// whose address depends only on the workgroup), moved to scalar registers.
// Without it a buffer resource built from a vector load's result lives in
// vector registers, and the compiler wraps each buffer access in a loop over
// the distinct resources of the wave -- one pass, but a dozen extra
// instructions per access.  Wrong if the lanes differ: only for values
// uniform by construction.
__device__ __forceinline__ int wave_uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t wave_uniform(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
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
//      is the P^T fragment of the value product.  A granule is 16 bytes of
//      one row (R = 8 bf16 or 16 fp8 dims); each half holds its 16 rows in
//      1 KB blocks of four granules, row-major in the block: one lane
//      group's operand load (4 granules x 16 rows) is one contiguous block,
//      and a row's four granules are 64 contiguous bytes (a token written
//      alone touches half as many lines, a quarter as many as granule-major).
//        byte offset = ((g*S + 32t)*D + h*16*D)*esize + (q/4)*1024 + r*64 + (q%4)*16 + (d%R)*esize,
//        q = d/R
//   V: blocks of 8 slots, ((g*(S/8) + slot/8)*D + d)*8 + slot%8 elements:
//      one 16-byte load is 8 consecutive keys of one dim (the V^T operand).
// (stored_slots: swr_internal.h)

// Byte offset of the start of a K tile half: ((g*S + 32t)*D + h*16*D)*esize.
__device__ __forceinline__ uint32_t k_half_base(int g, int S, int tile_slot0, int half, int D, int esize) {
  return ((uint32_t)(g * S + tile_slot0) * (uint32_t)D + (uint32_t)(half * 16 * D)) * (uint32_t)esize;
}

// Byte offset, within a K tile half, of granule q of row r.
__device__ __forceinline__ uint32_t k_granule_offset(int q, int r) {
  return (uint32_t)((q >> 2) * 1024 + r * 64 + (q & 3) * 16);
}

// OCP E4M3FN code of value/scale: the quotient is formed in binary64 with
// correct rounding (value is bf16, scale fp32, so the binary64 quotient sits
// on the same side of every E4M3 rounding midpoint as the exact one), then
// rounded to nearest, ties to even, on the E4M3 grid (quantum 2^-9 below
// 2^-6, 2^(e-3) in binade e above), saturating at +-448.
__device__ __forceinline__ uint8_t e4m3_encode(float value, float scale) {
  const double v = __ddiv_rn((double)value, (double)scale);
  const uint8_t sign = __builtin_signbit(v) ? 0x80 : 0x00;
  const double a = __builtin_fabs(v);
  if (__builtin_isnan(a)) return sign | 0x7F;
  if (a >= 448.0) return sign | 0x7E;
  if (a < 0x1p-6) {
    // subnormal range: code = round(a / 2^-9); 8 lands on the smallest normal 0x08
    return sign | (uint8_t)__builtin_rint(a * 512.0);
  }
  // binade e (-6 .. 8) from the binary64 exponent field; a * 2^(3-e) is exact
  int e = (int)((__builtin_bit_cast(uint64_t, a) >> 52) & 0x7FF) - 1023;
  const double pow2 = __builtin_bit_cast(double, (uint64_t)(1023 + 3 - e) << 52);
  int m = (int)__builtin_rint(a * pow2);  // 8 .. 16
  if (m == 16) {
    m = 8;
    ++e;
  }
  return sign | (uint8_t)(((e + 7) << 3) | (m - 8));
}

// Writes head dims 8*d8 .. 8*d8+7 of one token's K and V (bf16 bits, two
// per word) into slot `slot` of KV head g of a region storing S slots per
// head: one K granule store (16 bytes bf16, 8 bytes fp8) and eight V element
// stores into the slot's 8-slot V blocks.  fp8 regions take the E4M3 codes
// of value/scale.  The buffer resources bound the stores to the region.
template <bool FP8>
__device__ __forceinline__ void store_token_piece(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int slot,
                                                  int g, int S, int D, int d8, u32x4 kbits, u32x4 vbits,
                                                  float k_scale, float v_scale) {
  constexpr int ESZ = FP8 ? 1 : 2;
  const int k32 = slot & 31;
  const uint32_t koff = k_half_base(g, S, slot & ~31, (k32 >> 2) & 1, D, ESZ) +
                        k_granule_offset(FP8 ? d8 >> 1 : d8, 4 * (k32 >> 3) + (k32 & 3)) +
                        (uint32_t)(FP8 ? (d8 & 1) * 8 : 0);
  // V element (slot, g, d) at ((g*(S/8) + slot/8)*D + d)*8 + slot%8
  const uint32_t vrow = (uint32_t)((((size_t)g * (S >> 3) + (size_t)(slot >> 3)) * D + (size_t)d8 * 8) * 8 +
                                   (size_t)(slot & 7));
  if (!FP8) {
    store16(rk, koff, kbits);
#pragma unroll
    for (int e = 0; e < 8; ++e) store2(rv, (vrow + 8 * e) * 2, (uint16_t)(vbits[e >> 1] >> (16 * (e & 1))));
  } else {
    uint32_t kc[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t kb16 = (kbits[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      const uint32_t vb16 = (vbits[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      kc[e >> 2] |= (uint32_t)e4m3_encode(__builtin_bit_cast(float, kb16 << 16), k_scale) << (8 * (e & 3));
      store1(rv, vrow + 8 * e, e4m3_encode(__builtin_bit_cast(float, vb16 << 16), v_scale));
    }
    store8(rk, koff, u32x2{kc[0], kc[1]});
  }
}

// Writes the E4M3 codes of head dims 8*d8 .. 8*d8+7 of one token's K (if
// !is_v) or V (bf16 bits, two per word) into slot `slot` of KV head g of an
// fp8 region storing S slots per head, where store_token_piece puts them:
// half of that call's encodes, so that two lanes can share a piece.
__device__ __forceinline__ void store_token_half_fp8(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int slot,
                                                     int g, int S, int D, int d8, bool is_v, u32x4 bits,
                                                     float scale) {
  uint32_t c[2] = {0u, 0u};
#pragma unroll
  for (int e = 0; e < 8; ++e)
    c[e >> 2] |= (uint32_t)e4m3_encode(__builtin_bit_cast(float, ((bits[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16),
                                       scale)
                 << (8 * (e & 3));
  if (!is_v) {
    const int k32 = slot & 31;
    store8(rk, k_half_base(g, S, slot & ~31, (k32 >> 2) & 1, D, 1) + k_granule_offset(d8 >> 1, 4 * (k32 >> 3) + (k32 & 3)) +
                   (uint32_t)((d8 & 1) * 8),
           u32x2{c[0], c[1]});
  } else {
    const uint32_t vrow = (uint32_t)((((size_t)g * (S >> 3) + (size_t)(slot >> 3)) * D + (size_t)d8 * 8) * 8 +
                                     (size_t)(slot & 7));
#pragma unroll
    for (int e = 0; e < 8; ++e) store1(rv, vrow + 8 * e, (uint8_t)(c[e >> 2] >> (8 * (e & 3))));
  }
}

// Writes the E4M3 code of one head dim d of one token (K if !is_v, else V)
// into slot `slot` of KV head g of an fp8 region storing S slots per head:
// one byte, at the place store_token_piece puts it.
__device__ __forceinline__ void store_token_code(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, int slot,
                                                 int g, int S, int D, int d, bool is_v, uint8_t code) {
  if (!is_v) {
    const int k32 = slot & 31;
    store1(rk, k_half_base(g, S, slot & ~31, (k32 >> 2) & 1, D, 1) + k_granule_offset(d >> 4, 4 * (k32 >> 3) + (k32 & 3)) +
                   (uint32_t)(d & 15), code);
  } else {
    store1(rv, (uint32_t)((((size_t)g * (S >> 3) + (size_t)(slot >> 3)) * D + (size_t)d) * 8 + (size_t)(slot & 7)), code);
  }
}

// The bf16 values an fp8 region holds for four bf16 values (bits, two per
// word) after a store: the E4M3 codes of x/scale, decoded (in units of
// scale).
__device__ __forceinline__ u32x2 fp8_stored_values4(u32x2 x, float scale) {
  uint32_t c = 0u;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    c |= (uint32_t)e4m3_encode(__builtin_bit_cast(float, ((x[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16), scale)
         << (8 * e);
  const u32x4 v = __builtin_bit_cast(u32x4, fp8x8_to_bf16x8(u32x2{c, 0u}));
  return u32x2{v[0], v[1]};
}

// Waits until every vector memory access the wave has issued is complete,
// stores included (on gfx9-family parts the vector memory counter covers
// loads and stores), so that a later load by the wave sees what it stored.
// The memory clobber keeps the compiler from moving accesses across it.
__device__ __forceinline__ void wait_vm_all() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

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
