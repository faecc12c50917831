// gather.hip -- the paged-cache baseline on gfx950: copies each request's
// sliding window out of a paged KV cache into a ring region, so that the
// ring decode kernel can read it.
//
// "Improving Decode Throughput on Intel Gaudi 3" (Expensive KV gathers): a
// paged cache keeps a request's tokens in scattered fixed-size pages, and a
// sliding-window layer that reads them must first gather the window's pages
// into a contiguous buffer every step, which moves the window's bytes three
// times (read, write, read again) where the ring reads them once.  This
// kernel is that gather, written for the same region layout the ring uses
// (swr_device.h), so the attention after it is the very same kernel.
//
// One workgroup takes one 32-slot tile of one (request, KV head) ring: it
// loads the tile's tokens from their page rows (consecutive threads read
// consecutive 16-byte pieces of a row), parks them in LDS, and writes the
// tile back in the ring's own order -- consecutive threads write
// consecutive 16 bytes, for K's granules and for V's 8-slot blocks alike --
// so both the reads and the writes stream.
#include "gather.h"
#include "swr_device.h"
#include "swr_internal.h"

namespace swr {

template <int D>
__global__ void __launch_bounds__(256) paged_gather_kernel(const GatherArgs a) {
  constexpr int D8 = D / 8;
  __shared__ __attribute__((aligned(16))) uint16_t tk[32][D], tv[32][D];
  __shared__ int slot_ok[32];
  const int tiles = (a.W + 31) / 32;
  const int t = blockIdx.x % tiles;
  const int g = (blockIdx.x / tiles) % a.Hkv;
  const int b = blockIdx.x / (tiles * a.Hkv);
  const int P = a.pos[b];
  if (P < 0) return;  // uniform over the workgroup
  const int tid = threadIdx.x;

  // slot 32t + i holds the window position P - ((P - slot) mod W), if that
  // is >= 0, the slot is a slot of the ring and the position's page is a
  // page of the pool
  auto page_of = [&](int i, int& row) -> int64_t {
    const int slot = 32 * t + i;
    if (slot >= a.W) return -1;
    int back = (P - slot) % a.W;
    if (back < 0) back += a.W;
    const int p = P - back;
    if (p < 0) return -1;
    const int pi = p / a.page_tokens;
    if (pi >= a.max_pages) return -1;
    const int64_t page = a.block_table[(size_t)b * a.max_pages + pi];
    row = p - pi * a.page_tokens;
    return (page >= 0 && page < a.n_pages) ? page : -1;
  };
  if (tid < 32) {
    int row = 0;
    slot_ok[tid] = page_of(tid, row) >= 0;
  }
  // loads: piece k = (token i, dims 8*d8 ..) of the tile, into LDS
#pragma unroll
  for (int m = 0; m < (32 * D8 + 255) / 256; ++m) {
    const int k = tid + 256 * m;
    if (k < 32 * D8) {
      const int i = k / D8, d8 = k - (k / D8) * D8;
      int row = 0;
      const int64_t page = page_of(i, row);
      u32x4 kb = {0u, 0u, 0u, 0u}, vb = {0u, 0u, 0u, 0u};
      if (page >= 0) {
        const size_t src = (((size_t)page * a.page_tokens + (size_t)row) * a.Hkv + g) * D + (size_t)d8 * 8;
        kb = *reinterpret_cast<const u32x4*>(a.k_pages + src);
        vb = *reinterpret_cast<const u32x4*>(a.v_pages + src);
      }
      *reinterpret_cast<u32x4*>(&tk[i][8 * d8]) = kb;
      *reinterpret_cast<u32x4*>(&tv[i][8 * d8]) = vb;
    }
  }
  __syncthreads();

  const int S = stored_slots(a.W);
  const uint32_t region_bytes = (uint32_t)S * (uint32_t)(a.Hkv * D * 2);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(a.k_base + a.k_off[b], region_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(a.v_base + a.v_off[b], region_bytes);
  // K: granule u of the tile in storage order (half, 1 KB block, row,
  // granule): byte u*16 from the tile's start
  const uint32_t kt = k_half_base(g, S, 32 * t, 0, D, 2);
#pragma unroll
  for (int m = 0; m < (4 * D + 255) / 256; ++m) {
    const int u = tid + 256 * m;
    if (u < 4 * D) {
      const int h = u / (2 * D), rem = u - h * (2 * D);
      const int qb = rem / 64, r = (rem / 4) & 15, q4 = rem & 3;
      const int i = 8 * (r >> 2) + 4 * h + (r & 3);  // the row's slot in the tile
      if (slot_ok[i]) store16(rk, kt + (uint32_t)u * 16, *reinterpret_cast<const u32x4*>(&tk[i][8 * (4 * qb + q4)]));
    }
  }
  // V: block blk (slots 8*blk ..) of the tile, dim d: 16 bytes at
  // ((g*(S/8) + 4t + blk)*D + d)*16
  const uint32_t vt = (uint32_t)(((size_t)g * (S >> 3) + (size_t)(4 * t)) * D) * 16;
#pragma unroll
  for (int m = 0; m < (4 * D + 255) / 256; ++m) {
    const int u = tid + 256 * m;
    if (u < 4 * D) {
      const int blk = u / D, d = u - blk * D;
      uint32_t w[4];
      bool all = true;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        w[e / 2] = (uint32_t)tv[8 * blk + e][d] | (uint32_t)tv[8 * blk + e + 1][d] << 16;
        all = all && slot_ok[8 * blk + e] && slot_ok[8 * blk + e + 1];
      }
      if (all) {
        store16(rv, vt + (uint32_t)u * 16, u32x4{w[0], w[1], w[2], w[3]});
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (slot_ok[8 * blk + e]) store2(rv, vt + (uint32_t)u * 16 + 2 * e, tv[8 * blk + e][d]);
      }
    }
  }
}

hipError_t launch_paged_gather(const GatherArgs& a, hipStream_t s) {
  const long blocks = (long)a.B * a.Hkv * ((a.W + 31) / 32);
  if (blocks == 0) return hipSuccess;
  const dim3 grid((unsigned)blocks), block(256);
  switch (a.D) {
    case 64: hipLaunchKernelGGL(paged_gather_kernel<64>, grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL(paged_gather_kernel<128>, grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL(paged_gather_kernel<256>, grid, block, 0, s, a); break;
    case 512: hipLaunchKernelGGL(paged_gather_kernel<512>, grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace swr
