// global.hip -- global-layer grouped attention on gfx950, in two passes.
//
// "Announcing Carat" (More FLOPs can be faster; Doing it all in one kernel
// can be slower): for a global layer the G query heads that share a KV head,
// times the S proposed positions, form one group of rows; scores over the
// key_count = context + proposals keys, a causal softmax by query position
// and a weighted sum of values, with the key axis padded to a multiple of 64
// and the tail masked.  The page computes scores, softmax and the value
// product as separate matrix operations and stores the scores in between.
//
// On MI355X a single request's global layer (24.6 MB of K/V at 6005 keys)
// must be spread over all 256 CUs to stream at HBM speed, and a plain
// split over keys would leave a 32 x D fp32 partial per key chunk -- as many
// bytes as the chunk's K/V.  So the work is split the way the page splits
// it, keeping the intermediate small:
//   pass 1 (score_kernel): one workgroup per (request, KV head, two 32-key
//     tiles, all loads issued up front) computes the tiles' scores over the
//     full head dim with bf16 MFMA
//     (waves split the head dim and add their partial scores through LDS),
//     applies the causal mask and the scale, and stores fp32 scores:
//     rows x 4 bytes per key, 6% of the key's K/V bytes at 32 rows.
//   pass 2 (pv_kernel): one workgroup per (request, KV head, 512-key chunk,
//     slice of dsl value dims) runs the online softmax over its chunk's
//     scores and multiplies by its V slice with bf16 MFMA.  Its partial is
//     rows x dsl floats; a request whose keys fit one chunk writes its bf16
//     output directly.
//   pass 3 (merge_kernel): for requests with several chunks, merges the
//     chunk partials in chunk order into the bf16 output.  (A merge done by
//     the last-finishing workgroup of pass 2 would need a device-scope
//     release fence per workgroup, which writes back the XCD's L2 and costs
//     far more than a kernel boundary on this chip.)
// The sibling slices of one chunk read the same scores; they are placed on
// the same XCD (workgroup j runs on XCD j % 8) so those reads hit its L2.
#include <algorithm>

#include "swr_device.h"
#include "swr_internal.h"

namespace swr {

namespace {

__device__ __forceinline__ int region_slots(const AttnParams& p, int b) {
  return p.cap_b ? max(min(p.cap_b[b], p.cap), 0) : p.cap;
}

__device__ __forceinline__ int unit_keys(const AttnParams& p, int b) {
  return max(min(p.key_count[b], region_slots(p, b)), 0);
}

}  // namespace

// ------------------------------------------------------------------ pass 1

constexpr int kScoreTiles = 2;  // 32-key tiles per score workgroup

template <int D, int DS, int NCT, bool FP8>
__global__ void __launch_bounds__(64 * (D / DS)) score_kernel(const AttnParams p) {
  constexpr int DSPLIT = D / DS;
  constexpr int NCH = DS / 32;
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int RED = 2 * NCT * 4;
  constexpr int T = kScoreTiles;
  __shared__ float red[DSPLIT > 1 ? T * DSPLIT * RED * 64 : 1];

  const int lane = threadIdx.x & 63;
  const int ds = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int tgroups = (p.max_tiles + T - 1) / T;
  const int unit = blockIdx.x / tgroups;
  const int t0 = (blockIdx.x - unit * tgroups) * T;

  const int Hkv = p.Hkv, G = p.G, S = p.S;
  const int b = unit / Hkv;
  const int g = unit - b * Hkv;
  const int cap_r = region_slots(p, b);
  const int d_base = ds * DS;

  // Every load is issued before the key count is known: tiles past the keys
  // read zeros or slots of the region that are never stored as scores.
  const uint32_t region_bytes = (uint32_t)cap_r * (uint32_t)(Hkv * D * ESZ);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_base + p.k_off[b], region_bytes);
  bf16x8 kop[T][2][NCH];
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      // A row lr of sub-tile `sub` is key 8*(lr/4) + 4*sub + lr%4: lane group
      // lq receives the scores of keys 8*lq + 4*sub + 0..3.
      const int e = 8 * (lr >> 2) + 4 * sub + (lr & 3);
      const uint32_t base = ((uint32_t)(g * cap_r + (t0 + u) * 32 + e) * D + d_base) * ESZ;
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t off = base + (uint32_t)((4 * c + lq) * 8 * ESZ);
        kop[u][sub][c] = FP8 ? fp8x8_to_bf16x8(load8(rk, off)) : as_bf16x8(load16_stream(rk, off));
      }
    }
  // Q rows: loaded unconditionally from a valid row (no divergent branch
  // between the loads), rows past G*S zeroed by select.
  bool row_ok[NCT];
  int row_i[NCT];
  bf16x8 qop[NCT][NCH];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int row = ct * 16 + lr;
    row_ok[ct] = row < p.rows;
    const int rr = row_ok[ct] ? row : 0;
    const int i = rr / G;
    const int h = rr - i * G;
    row_i[ct] = i;
    const uint16_t* qrow = p.q + ((size_t)(b * S + i) * p.Hq + g * G + h) * D + d_base;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const u32x4 bits = *reinterpret_cast<const u32x4*>(qrow + (4 * c + lq) * 8);
      qop[ct][c] = as_bf16x8(row_ok[ct] ? bits : u32x4{0u, 0u, 0u, 0u});
    }
  }
  const int n_keys = unit_keys(p, b);
  if (t0 >= ((n_keys + 31) >> 5)) return;
  int row_lim[NCT];  // last key the row may see
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) row_lim[ct] = min(p.pos[b * S + row_i[ct]], n_keys - 1);
  f32x4 sc[T][2][NCT];
#pragma unroll
  for (int u = 0; u < T; ++u)
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) acc = mfma16x16x32(kop[u][sub][c], qop[ct][c], acc);
        sc[u][sub][ct] = acc;
      }

  if (DSPLIT > 1) {  // add the head-dim slices in slice order; wave 0 stores
#pragma unroll
    for (int u = 0; u < T; ++u)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r)
            red[((u * DSPLIT + ds) * RED + (sub * NCT + ct) * 4 + r) * 64 + lane] = sc[u][sub][ct][r];
    __syncthreads();
    if (ds != 0) return;
#pragma unroll
    for (int u = 0; u < T; ++u)
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float a = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < DSPLIT; ++s2)
              a += red[((u * DSPLIT + s2) * RED + (sub * NCT + ct) * 4 + r) * 64 + lane];
            sc[u][sub][ct][r] = a;
          }
  }

#pragma unroll
  for (int u = 0; u < T; ++u) {
    const int kb = (t0 + u) * 32;
    if (kb >= n_keys) break;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int row = ct * 16 + lr;
      if (!row_ok[ct]) continue;
      float* dst = p.ws_scores + ((size_t)unit * p.rows + row) * p.kpad + kb + 8 * lq;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        f32x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int key = kb + 8 * lq + 4 * sub + r;
          v[r] = key <= row_lim[ct] ? sc[u][sub][ct][r] * p.qk_scale : -INFINITY;
        }
        *reinterpret_cast<f32x4*>(dst + 4 * sub) = v;
      }
    }
  }
}

// ------------------------------------------------------------------ pass 2

constexpr int kPvWaves = 4;        // waves per workgroup, each takes every 4th tile
constexpr int kPvTilesPerWave = 4;
constexpr int kChunkTiles = kPvWaves * kPvTilesPerWave;  // 16 tiles = 512 keys

template <int DSL, int NCT, bool FP8>
__global__ void __launch_bounds__(64 * kPvWaves) pv_kernel(const AttnParams p, int D) {
  constexpr int KW = kPvWaves, TPW = kPvTilesPerWave, CT = kChunkTiles;
  constexpr int NDT = DSL / 16;
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int RS = DSL + 4;
  __shared__ float cml[KW][32][2];
  __shared__ float co[KW][32][RS];

  const int lane = threadIdx.x & 63;
  const int kw = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int lq = lane >> 4;

  // workgroup -> (chunk group, value slice): siblings share an XCD
  const int j = blockIdx.x;
  const int xcd = j & 7;
  const int slot = j >> 3;
  const int group = (slot / p.nds) * 8 + xcd;
  const int ds = slot - (slot / p.nds) * p.nds;
  const int units = p.B * p.Hkv;
  if (group >= units * p.nchunk) return;
  const int unit = group / p.nchunk;
  const int chunk = group - unit * p.nchunk;
  const int Hkv = p.Hkv, G = p.G, S = p.S;
  const int b = unit / Hkv;
  const int g = unit - b * Hkv;
  const int cap_r = region_slots(p, b);
  const int d0 = ds * DSL;

  // ---- every load of this wave up front, before the key count is known
  // (scores past the keys are read but never used; the score buffer is
  // padded to whole chunks, so the reads stay inside the workspace)
  f32x4 sv[TPW][NCT][2];
  bf16x8 vv[TPW][NDT];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = chunk * CT + kw + i * KW;
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int row = min(ct * 16 + lr, p.rows - 1);
      const float* src = p.ws_scores + ((size_t)unit * p.rows + row) * p.kpad + t * 32 + 8 * lq;
      sv[i][ct][0] = *reinterpret_cast<const f32x4*>(src);
      sv[i][ct][1] = *reinterpret_cast<const f32x4*>(src + 4);
    }
  }
  const uint32_t region_bytes = (uint32_t)cap_r * (uint32_t)(Hkv * D * ESZ);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_base + p.v_off[b], region_bytes);
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = chunk * CT + kw + i * KW;
    const uint32_t vbase = ((uint32_t)((g * (cap_r >> 3) + t * 4 + lq) * D + d0 + lr)) * 8 * ESZ;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) {
      const uint32_t off = vbase + (uint32_t)(dt * 16 * 8 * ESZ);
      vv[i][dt] = FP8 ? fp8x8_to_bf16x8(load8(rv, off)) : as_bf16x8(load16_stream(rv, off));
    }
  }
  const int n_keys = unit_keys(p, b);
  const int nt = (n_keys + 31) >> 5;
  const int nvalid = (nt + CT - 1) / CT;
  if (chunk >= nvalid) return;

  // ---- online softmax over the chunk and O^T += V^T . P^T
  f32x4 o[NCT][NDT];
  float m_run[NCT], l_run[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = chunk * CT + kw + i * KW;
    if (t >= nt) continue;
    const int kb = t * 32;
    bf16x8 pop[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const bool ok = ct * 16 + lr < p.rows;
      float s[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) s[e] = ok ? sv[i][ct][e >> 2][e & 3] : -INFINITY;
      float tmax = s[0];
#pragma unroll
      for (int e = 1; e < 8; ++e) tmax = fmaxf(tmax, s[e]);
      tmax = max4lanes(tmax);
      const float m_new = fmaxf(m_run[ct], tmax);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run[ct] - m_use);
      float psum = 0.f;
      bf16x8 pv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const __bf16 pb = (__bf16)fast_exp2(s[e] - m_use);
        pv[e] = pb;
        psum += (float)pb;
      }
      pop[ct] = pv;
      l_run[ct] = l_run[ct] * alpha + psum;
      m_run[ct] = m_new;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[ct][dt] *= alpha;
    }
    if (kb + 32 > n_keys) {  // zero the values of keys past key_count
      u32x4 keep;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int k0 = kb + 8 * lq + 2 * q;
        keep[q] = (k0 < n_keys ? 0x0000FFFFu : 0u) | (k0 + 1 < n_keys ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        vv[i][dt] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vv[i][dt]) & keep);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[ct][dt] = mfma16x16x32(vv[i][dt], pop[ct], o[ct][dt]);
  }
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) l_run[ct] = sum4lanes(l_run[ct]);

  // ---- merge the waves (in wave order) through LDS
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int row = ct * 16 + lr;
    if (row >= p.rows) continue;
    if (lq == 0) {
      cml[kw][row][0] = m_run[ct];
      cml[kw][row][1] = l_run[ct];
    }
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) *reinterpret_cast<f32x4*>(&co[kw][row][16 * dt + 4 * lq]) = o[ct][dt];
  }
  __syncthreads();

  const int items = p.rows * (DSL / 4);
  const size_t slice = (size_t)unit * p.nds + ds;  // unit * nds + ds
  for (int it = threadIdx.x; it < items; it += blockDim.x) {
    const int row = it / (DSL / 4);
    const int d4 = (it - row * (DSL / 4)) * 4;
    float M = -INFINITY;
#pragma unroll
    for (int k = 0; k < KW; ++k) M = fmaxf(M, cml[k][row][0]);
    const float M_use = (M == -INFINITY) ? 0.f : M;
    float L = 0.f;
    f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < KW; ++k) {
      const float w = fast_exp2(cml[k][row][0] - M_use);
      L += cml[k][row][1] * w;
      O += *reinterpret_cast<const f32x4*>(&co[k][row][d4]) * w;
    }
    if (nvalid == 1) {
      const float inv = L > 0.f ? p.v_scale / L : 0.f;
      const int i = row / G, h = row - (row / G) * G;
      bf16x4 w = {(__bf16)(O[0] * inv), (__bf16)(O[1] * inv), (__bf16)(O[2] * inv), (__bf16)(O[3] * inv)};
      *reinterpret_cast<bf16x4*>(p.out + ((size_t)(b * S + i) * p.Hq + g * G + h) * D + d0 + d4) = w;
    } else {
      const size_t part = (slice * p.nchunk + chunk) * p.rows + row;
      *reinterpret_cast<f32x4*>(p.ws_part + part * DSL + d4) = O;
      if (d4 == 0) {
        p.ws_pml[part * 2 + 0] = M;
        p.ws_pml[part * 2 + 1] = L;
      }
    }
  }
}

// ------------------------------------------------------------------ pass 3

// One thread per (request, KV head, value slice, row, 4 dims); merges the
// chunk partials in chunk order.  Requests with a single chunk were written
// by pass 2.
__global__ void __launch_bounds__(256) merge_kernel(const AttnParams p, int D) {
  const int per_slice = p.rows * (p.dsl / 4);
  const int units = p.B * p.Hkv;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= units * p.nds * per_slice) return;
  const int slice = idx / per_slice;  // unit * nds + ds
  const int rem = idx - slice * per_slice;
  const int row = rem / (p.dsl / 4);
  const int d4 = (rem - row * (p.dsl / 4)) * 4;
  const int unit = slice / p.nds;
  const int ds = slice - unit * p.nds;
  const int b = unit / p.Hkv;
  const int g = unit - b * p.Hkv;
  const size_t base = (size_t)slice * p.nchunk * p.rows + row;
  // Chunks are merged 16 at a time, every load of a group in flight together
  // and issued before the key count is known (addresses are clamped to the
  // launch's chunk count; chunks past this request's keys are dropped by
  // select, never multiplied, so whatever they hold cannot leak in).  The
  // running (M, L, O) is rescaled between groups; sums run in chunk order.
  constexpr int GRP = 16;
  float M = -INFINITY, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  int nvalid = -1;
  for (int c0 = 0; c0 < p.nchunk; c0 += GRP) {
    float m[GRP], l[GRP];
    f32x4 o[GRP];
#pragma unroll
    for (int k = 0; k < GRP; ++k) {
      const size_t part = base + (size_t)min(c0 + k, p.nchunk - 1) * p.rows;
      m[k] = p.ws_pml[part * 2];
      l[k] = p.ws_pml[part * 2 + 1];
      o[k] = *reinterpret_cast<const f32x4*>(p.ws_part + part * p.dsl + d4);
    }
    if (nvalid < 0) {
      const int nt = (unit_keys(p, b) + 31) >> 5;
      nvalid = (nt + kChunkTiles - 1) / kChunkTiles;
      if (nvalid <= 1) return;  // pass 2 wrote this request's output
    }
    if (c0 >= nvalid) break;
    float Mg = M;
#pragma unroll
    for (int k = 0; k < GRP; ++k) Mg = fmaxf(Mg, c0 + k < nvalid ? m[k] : -INFINITY);
    const float M_use = (Mg == -INFINITY) ? 0.f : Mg;
    const float a = fast_exp2(M - M_use);
    L *= a;
    O *= a;
#pragma unroll
    for (int k = 0; k < GRP; ++k) {
      const bool ok = c0 + k < nvalid;
      const float w = fast_exp2(m[k] - M_use);
      L += ok ? l[k] * w : 0.f;
      const f32x4 t = o[k] * w;
      O[0] += ok ? t[0] : 0.f;
      O[1] += ok ? t[1] : 0.f;
      O[2] += ok ? t[2] : 0.f;
      O[3] += ok ? t[3] : 0.f;
    }
    M = Mg;
  }
  const float inv = L > 0.f ? p.v_scale / L : 0.f;
  const int i = row / p.G, h = row - (row / p.G) * p.G;
  bf16x4 w = {(__bf16)(O[0] * inv), (__bf16)(O[1] * inv), (__bf16)(O[2] * inv), (__bf16)(O[3] * inv)};
  *reinterpret_cast<bf16x4*>(p.out + ((size_t)(b * p.S + i) * p.Hq + g * p.G + h) * D + ds * p.dsl + d4) = w;
}

// ------------------------------------------------------------------ host

namespace {

int cdiv(long a, long b) { return (int)((a + b - 1) / b); }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

// head dims per wave in the score pass
int score_ds(int D, int nct) {
  if (D <= 128) return D;
  return nct == 2 ? 128 : 256;
}

template <int D, int DS, int NCT>
hipError_t launch_scores(const AttnPlan& pl, const AttnParams& p, hipStream_t s) {
  const int grid = pl.units * cdiv(pl.max_tiles, kScoreTiles);
  if (pl.fp8)
    hipLaunchKernelGGL((score_kernel<D, DS, NCT, true>), dim3(grid), dim3(64 * (D / DS)), 0, s, p);
  else
    hipLaunchKernelGGL((score_kernel<D, DS, NCT, false>), dim3(grid), dim3(64 * (D / DS)), 0, s, p);
  return hipGetLastError();
}

hipError_t launch_scores_any(const AttnPlan& pl, const AttnParams& p, hipStream_t s) {
  const bool two = pl.nct == 2;
  switch (pl.D) {
    case 64: return two ? launch_scores<64, 64, 2>(pl, p, s) : launch_scores<64, 64, 1>(pl, p, s);
    case 128: return two ? launch_scores<128, 128, 2>(pl, p, s) : launch_scores<128, 128, 1>(pl, p, s);
    case 256: return two ? launch_scores<256, 128, 2>(pl, p, s) : launch_scores<256, 256, 1>(pl, p, s);
    case 512: return two ? launch_scores<512, 128, 2>(pl, p, s) : launch_scores<512, 256, 1>(pl, p, s);
  }
  return hipErrorInvalidValue;
}

template <int DSL, int NCT>
hipError_t launch_pv(const AttnPlan& pl, const AttnParams& p, hipStream_t s) {
  if (pl.fp8)
    hipLaunchKernelGGL((pv_kernel<DSL, NCT, true>), dim3(pl.grid2), dim3(64 * kPvWaves), 0, s, p, pl.D);
  else
    hipLaunchKernelGGL((pv_kernel<DSL, NCT, false>), dim3(pl.grid2), dim3(64 * kPvWaves), 0, s, p, pl.D);
  return hipGetLastError();
}

}  // namespace

bool plan_global(int B, int S, int Hq, int Hkv, int D, int max_keys, AttnPlan* pl) {
  if (B < 0 || S < 1 || S > 8 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || max_keys < 1) return false;
  if (D != 64 && D != 128 && D != 256 && D != 512) return false;
  const int rows = (Hq / Hkv) * S;
  if (rows > 32) return false;
  pl->mode = MODE_GLOBAL;
  pl->D = D;
  pl->nct = rows > 16 ? 2 : 1;
  pl->rows = rows;
  pl->units = B * Hkv;
  pl->g_ds = score_ds(D, pl->nct);
  pl->threads = 64 * (D / pl->g_ds);
  pl->max_tiles = cdiv(max_keys, 32);
  pl->kw = kPvWaves;
  pl->nsplit = 1;
  pl->tiles_per_split = pl->max_tiles;
  // value slices: narrow when the job is small (more workgroups to fill the
  // chip), wider when it is large (fewer passes over the scores)
  pl->dsl = ((long)pl->units * pl->max_tiles <= 4096 || D < 64) ? 32 : 64;
  pl->nds = D / pl->dsl;
  pl->nchunk = cdiv(pl->max_tiles, kChunkTiles);
  pl->grid2 = cdiv((long)pl->units * pl->nchunk, 8) * 8 * pl->nds;
  const size_t kpad = (size_t)pl->nchunk * kChunkTiles * 32;  // whole chunks
  size_t off = 0;
  pl->off_scores = off;
  off = align256(off + (size_t)pl->units * rows * kpad * sizeof(float));
  pl->off_part = off;
  off = align256(off + (size_t)pl->units * pl->nds * pl->nchunk * rows * pl->dsl * sizeof(float));
  pl->off_pml = off;
  off = align256(off + (size_t)pl->units * pl->nds * pl->nchunk * rows * 2 * sizeof(float));
  pl->off_count = off;
  pl->ws_bytes = pl->units > 0 ? off : 0;
  pl->lds_bytes = 0;
  return true;
}

hipError_t launch_global(const AttnPlan& pl, const AttnParams& p0, hipStream_t s) {
  if (pl.units == 0) return hipSuccess;
  AttnParams p = p0;
  p.max_tiles = pl.max_tiles;
  p.kpad = pl.nchunk * kChunkTiles * 32;
  p.nchunk = pl.nchunk;
  p.nds = pl.nds;
  p.dsl = pl.dsl;
  hipError_t e = launch_scores_any(pl, p, s);
  if (e != hipSuccess) return e;
  if (pl.dsl == 32)
    e = pl.nct == 2 ? launch_pv<32, 2>(pl, p, s) : launch_pv<32, 1>(pl, p, s);
  else
    e = pl.nct == 2 ? launch_pv<64, 2>(pl, p, s) : launch_pv<64, 1>(pl, p, s);
  if (e != hipSuccess || pl.nchunk <= 1) return e;
  const long items = (long)pl.units * pl.nds * pl.rows * (pl.dsl / 4);
  hipLaunchKernelGGL(merge_kernel, dim3(cdiv(items, 256)), dim3(256), 0, s, p, pl.D);
  return hipGetLastError();
}

}  // namespace swr
