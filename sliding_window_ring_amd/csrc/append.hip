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
  store_token_piece<FP8>(rk, rv, (int)slot, g, S, p.D, d8, kbits, vbits, p.k_scale, p.v_scale);
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
