// read_ceiling.hip -- a plain streaming read of a device range, the yardstick
// the attention kernels' HBM rates are compared with on this chip.
//
// Each thread keeps eight 16-byte non-temporal loads in flight and folds the
// words into one xor.  A thread stores its
// fold only when it equals one fixed value: the loads stay live with next to
// no writes.  The sink takes at most 256 words.
#include "swr_device.h"
#include "swr_internal.h"

namespace swr {

constexpr int kReadUnroll = 8;
constexpr int kReadThreads = 256;

// pattern 0: word i of the range goes to thread i mod (grid * 256), so the
// whole grid sweeps the range front to back together.  pattern 1: workgroup
// w streams its own contiguous span of the range (as an attention workgroup
// streams its unit's region), 32 KB per step.
template <int PATTERN>
__global__ void __launch_bounds__(kReadThreads) read_ceiling_kernel(const u32x4* __restrict__ src, size_t n16,
                                                                    size_t span16, uint32_t* sink) {
  uint32_t acc = 0;
  size_t i, end, stride;
  if (PATTERN == 0) {
    i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
    end = n16;
    stride = (size_t)gridDim.x * kReadThreads;
  } else {
    i = (size_t)blockIdx.x * span16 + threadIdx.x;
    end = min(n16, (size_t)(blockIdx.x + 1) * span16);
    stride = kReadThreads;
  }
  for (; i < end; i += stride * kReadUnroll) {
    u32x4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const size_t j = i + (size_t)u * stride;
      v[u] = j < end ? __builtin_nontemporal_load(src + j) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u][0] ^ v[u][1] ^ v[u][2] ^ v[u][3];
  }
  if (acc == 0x5EEDF00Du) sink[threadIdx.x] = acc;
}

hipError_t launch_read_ceiling(const void* src, size_t n16, uint32_t* sink, int grid, int pattern,
                               hipStream_t s) {
  const u32x4* p = reinterpret_cast<const u32x4*>(src);
  // spans of whole 32 KB steps
  constexpr size_t step16 = (size_t)kReadThreads * kReadUnroll;
  const size_t span16 = (n16 + (size_t)grid * step16 - 1) / ((size_t)grid * step16) * step16;
  if (pattern == 0)
    hipLaunchKernelGGL(read_ceiling_kernel<0>, dim3((unsigned)grid), dim3(kReadThreads), 0, s, p, n16, span16,
                       sink);
  else
    hipLaunchKernelGGL(read_ceiling_kernel<1>, dim3((unsigned)grid), dim3(kReadThreads), 0, s, p, n16, span16,
                       sink);
  return hipGetLastError();
}

}  // namespace swr
