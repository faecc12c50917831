// append.hip -- writing new tokens' K and V into per-request regions, and
// zero-filling device ranges, on gfx950.
//
// "Announcing Carat" (ring buffer section): a token's slot is its absolute
// position modulo the window, and the new token simply overwrites the oldest
// slot.  "Improving Decode Throughput on Intel Gaudi 3" (Our approach): K and
// V of a token are written together to the same slot, so the two rings keep
// one rotation.  Global regions use slot = position.
//
// One thread moves 8 consecutive head dims of one (request, token, KV head):
// one 16-byte read of K and of V, one 16-byte (bf16) or 8-byte (fp8) store
// into the slot's K granule, and eight 2-byte / 1-byte V stores into the
// 8-slot V blocks (region layout: swr_device.h).
// Stores go through bounded buffer resources: a slot outside the region is
// dropped by the hardware instead of written.
#include "swr_device.h"
#include "swr_internal.h"

namespace swr {

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

template <bool FP8>
__global__ void __launch_bounds__(256) append_kernel(const AppendParams p) {
  const int d8n = p.D / 8;
  const long total = (long)p.B * p.T * p.Hkv * d8n;
  const long idx = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int d8 = (int)(idx % d8n);
  long rest = idx / d8n;
  const int g = (int)(rest % p.Hkv);
  rest /= p.Hkv;
  const int t = (int)(rest % p.T);
  const int b = (int)(rest / p.T);

  const int n = p.n_new ? p.n_new[b] : p.T;
  if (t >= n) return;
  // slots of this request's region (global regions may carry their own)
  const int cap = (!p.wrap && p.cap_b) ? max(min(p.cap_b[b], p.cap), 0) : p.cap;
  if (p.wrap && t < n - cap) return;  // a later token of this call owns the slot
  const long pos = (long)p.pos0[b] + t;
  if (pos < 0) return;
  long slot;
  if (p.wrap) {
    slot = pos % cap;
  } else {
    if (pos >= cap) return;
    slot = pos;
  }

  const size_t src = (((size_t)b * p.T + t) * p.Hkv + g) * p.D + (size_t)d8 * 8;
  const u32x4 kbits = *reinterpret_cast<const u32x4*>(p.k_new + src);
  const u32x4 vbits = *reinterpret_cast<const u32x4*>(p.v_new + src);
  constexpr int ESZ = FP8 ? 1 : 2;
  const int S = stored_slots(cap);
  const uint32_t region_bytes = (uint32_t)S * (uint32_t)(p.Hkv * p.D * ESZ);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_base + p.k_off[b], region_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_base + p.v_off[b], region_bytes);
  // K: this thread's 8 dims are one bf16 granule, or half an fp8 granule
  const int k32 = (int)(slot & 31);
  const uint32_t koff = k_half_base(g, S, (int)(slot & ~31L), (k32 >> 2) & 1, p.D, ESZ) +
                        (uint32_t)((FP8 ? d8 >> 1 : d8) * 256 + (4 * (k32 >> 3) + (k32 & 3)) * 16 +
                                   (FP8 ? (d8 & 1) * 8 : 0));
  // V element (slot, g, d) at ((g*(S/8) + slot/8)*D + d)*8 + slot%8
  const uint32_t vrow = (uint32_t)((((size_t)g * (S >> 3) + (size_t)(slot >> 3)) * p.D + (size_t)d8 * 8) * 8 +
                                   (size_t)(slot & 7));
  if (!FP8) {
    store16(rk, koff, kbits);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint16_t bits = (uint16_t)(vbits[e >> 1] >> (16 * (e & 1)));
      store2(rv, (vrow + 8 * e) * 2, bits);
    }
  } else {
    uint32_t kc[2] = {0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t kb16 = (kbits[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      const uint32_t vb16 = (vbits[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      const float kv = __builtin_bit_cast(float, kb16 << 16);
      const float vv = __builtin_bit_cast(float, vb16 << 16);
      kc[e >> 2] |= (uint32_t)e4m3_encode(kv, p.k_scale) << (8 * (e & 3));
      store1(rv, vrow + 8 * e, e4m3_encode(vv, p.v_scale));
    }
    store8(rk, koff, u32x2{kc[0], kc[1]});
  }
}

__global__ void __launch_bounds__(256) zero16_kernel(u32x4* dst, size_t n16) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    dst[i] = u32x4{0u, 0u, 0u, 0u};
}

__global__ void __launch_bounds__(256) zero1_kernel(uint8_t* dst, size_t n) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) dst[i] = 0;
}

hipError_t launch_append(const AppendParams& p, int fp8, hipStream_t s) {
  const long total = (long)p.B * p.T * p.Hkv * (p.D / 8);
  if (total == 0) return hipSuccess;
  const int blocks = (int)((total + 255) / 256);
  if (fp8)
    hipLaunchKernelGGL(append_kernel<true>, dim3(blocks), dim3(256), 0, s, p);
  else
    hipLaunchKernelGGL(append_kernel<false>, dim3(blocks), dim3(256), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_zero_fill(void* ptr, size_t bytes, hipStream_t s) {
  if (bytes == 0) return hipSuccess;
  uint8_t* p8 = static_cast<uint8_t*>(ptr);
  const size_t head = (16 - (reinterpret_cast<uintptr_t>(p8) & 15)) & 15;
  const size_t pre = head < bytes ? head : bytes;
  const size_t n16 = (bytes - pre) / 16;
  const size_t post = bytes - pre - n16 * 16;
  if (pre) hipLaunchKernelGGL(zero1_kernel, dim3(1), dim3(256), 0, s, p8, pre);
  if (n16) {
    size_t blocks = (n16 + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(zero16_kernel, dim3((unsigned)blocks), dim3(256), 0, s,
                       reinterpret_cast<u32x4*>(p8 + pre), n16);
  }
  if (post) hipLaunchKernelGGL(zero1_kernel, dim3(1), dim3(256), 0, s, p8 + pre + n16 * 16, post);
  return hipGetLastError();
}

}  // namespace swr
