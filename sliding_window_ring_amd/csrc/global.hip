// global.hip -- global-layer grouped attention on gfx950, chunked form.
//
// "Announcing Carat" (More FLOPs can be faster; Doing it all in one kernel
// can be slower): for a global layer the G query heads that share a KV head,
// times the S proposed positions, form one group of rows; scores over the
// key_count = context + proposals keys, a causal softmax by query position
// and a weighted sum of values, with the key axis padded to a multiple of 64
// and the tail masked.  The page computes scores, softmax and the value
// product as separate matrix operations and stores the scores in between.
//
// On MI355X a single request's global layer (24.6 MB of K/V at 6005 keys,
// two KV heads) must be spread over many CUs to stream at HBM speed, and each
// workgroup must put all of its loads in flight at once: a chain of
// dependent round trips per workgroup, not bandwidth, is what bounds a job
// this small.  So a block of keys (two of the page's 64-key pads) becomes
// the unit of work:
//   pass 1 (chunk_kernel): one workgroup per (request, KV head, 128 keys)
//     issues every K, V and Q load on entry, then runs the three products of
//     the page on its chunk -- scores (bf16 MFMA, fp32), the masked softmax
//     over the chunk, and P x V (bf16 MFMA, fp32) -- with Q, the scores and
//     P kept in LDS, and writes the chunk's unnormalised rows with their
//     (max, sum).
//   pass 2 (chunk_merge_kernel): one workgroup per (request, KV head, row,
//     quarter of the head dims) merges the chunks: weights 2^(m_c - M), sums
//     in a fixed order, division by the weighted row sum.
// The chunk length trades workgroups (CUs pulling K/V) against partial
// bytes (rows x D fp32 per chunk, written and read back): at 128 keys and
// 32 rows the partials are a quarter of the K/V bytes.  A merge done by the
// last-finishing workgroup of pass 1 instead would need a device-scope
// release fence per workgroup, which writes back the XCD's L2 and costs far
// more than the kernel boundary on this chip.
#include <algorithm>

#include "swr_device.h"
#include "swr_internal.h"

namespace swr {

namespace {

// Slots of request b's region.  The per-request capacity is read without a
// branch (a null cap_b reads an in-bounds word of k_off instead, then
// ignored), so the loads of k_off[b], v_off[b] and the capacity go out
// together rather than one after another.
__device__ __forceinline__ int region_slots(const AttnParams& p, int b) {
  const int32_t* cb = p.cap_b ? p.cap_b : reinterpret_cast<const int32_t*>(p.k_off);
  const int raw = cb[b];
  return p.cap_b ? max(min(raw, p.cap), 0) : p.cap;
}

__device__ __forceinline__ int unit_keys(const AttnParams& p, int b) {
  return max(min(p.key_count[b], region_slots(p, b)), 0);
}

}  // namespace

// ------------------------------------------------------------------ pass 1

constexpr int kChunkKeys = 128;                 // keys per workgroup of pass 1
constexpr int kChunkWaves = kChunkKeys / 8;     // 16 waves: two per 16-key subtile

// One workgroup per (request, KV head, 128-key chunk), sixteen waves.  Every
// K, V and Q load of the workgroup is issued on entry (256 KB of K/V at
// D = 512; Q goes to LDS once), before the key count is read: addresses past
// the region are bounded by the buffer resource, and a chunk past the
// request's keys only leaves without using what it loaded.
//   scores   wave (kq, dh) = (w % 8, w / 8): keys 16*kq .. +15 over head-dim
//            half dh, bf16 MFMA into fp32; the two halves meet in LDS and
//            are added in half order
//   softmax  16 lanes per row, eight keys per lane (rows spread over the
//            waves); masked (key count, causal by query position), max and
//            sum over the chunk by DPP within the lanes' row, P rounded to
//            bf16 into LDS; the row's (max, sum) go to the workspace
//   values   waves w < PVW: O^T(dims w*DPW .. +DPW, rows) = V^T . P^T over
//            the chunk, bf16 MFMA into fp32; the unnormalised rows go to the
//            workspace for pass 2 with streaming stores.
template <int D, int NCT, bool FP8>
__global__ void __launch_bounds__(64 * kChunkWaves) chunk_kernel(const AttnParams p) {
  constexpr int CK = kChunkKeys;
  constexpr int NW = kChunkWaves;
  constexpr int KQ = CK / 16;                        // 16-key subtiles (score waves per half)
  constexpr int ROWS = 16 * NCT;
  constexpr int DH = D / 2;                          // head dims per score wave
  constexpr int NCH = DH / 32;                       // 32-dim k chunks per score wave
  constexpr int PVW = D / 16 < NW ? D / 16 : NW;     // value waves
  constexpr int DPW = D / PVW;                       // value dims per value wave
  constexpr int NDT = DPW / 16;                      // 16-dim value tiles per value wave
  constexpr int KS = CK / 32;                        // 32-key k steps of the value product
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr bool KPAIR = FP8 && NCH % 2 == 0;        // 16-byte fp8 K loads (two k chunks)
  constexpr bool VPAIR = FP8 && NDT % 2 == 0;        // 16-byte fp8 V loads (two adjacent dims)
  constexpr int SLOTS = 4 * NW;                      // softmax rows in flight (16 lanes each)
  constexpr int KPL = CK / 16;                       // keys per softmax lane
  constexpr int SRS = CK + 4;                        // LDS row strides (floats / bf16)
  constexpr int PRS = CK + 8;
  constexpr int QRS = D + 8;
  static_assert(ROWS <= SLOTS, "one softmax pass covers the rows");
  __shared__ float sbuf[2][ROWS][SRS];
  __shared__ __attribute__((aligned(16))) __bf16 pbuf[ROWS][PRS];
  __shared__ __attribute__((aligned(16))) __bf16 qbuf[ROWS][QRS];

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int unit = blockIdx.x / p.nchunk;
  const int chunk = blockIdx.x - unit * p.nchunk;
  const int Hkv = p.Hkv, G = p.G, S = p.S;
  const int b = unit / Hkv;
  const int g = unit - b * Hkv;
  const int k0 = chunk * CK;
  const int64_t k_off = p.k_off[b], v_off = p.v_off[b];
  const int cap_r = region_slots(p, b);
  const uint32_t region_bytes = (uint32_t)cap_r * (uint32_t)(Hkv * D * ESZ);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_base + k_off, region_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_base + v_off, region_bytes);

  // Head dim (within the wave's half) of k element 8*lq + j of chunk c; with
  // paired fp8 loads a lane's 16 bytes cover two chunks (a fixed permutation
  // of the k axis, applied to Q as well).
  auto kdim = [&](int c) { return KPAIR ? 64 * (c >> 1) + 16 * lq + 8 * (c & 1) : (4 * c + lq) * 8; };
  // Head dim of A row lr of value tile dt (paired fp8: tiles 2t, 2t+1 take
  // the even and odd dims of one 32-dim block).
  const int vw = wave < PVW ? wave : 0;
  auto vdim = [&](int dt) {
    return vw * DPW + (VPAIR ? 32 * (dt >> 1) + 2 * lr + (dt & 1) : 16 * dt + lr);
  };

  // ---------------------------------------------------------- loads
  const int kq = wave % KQ, dh = wave / KQ;
  bf16x8 kop[NCH];
  {
    const uint32_t base = ((uint32_t)(g * cap_r + k0 + 16 * kq + lr) * D + dh * DH) * ESZ;
    if (KPAIR) {
#pragma unroll
      for (int c = 0; c < NCH; c += 2) {
        const u32x4 w = load16_stream(rk, base + (uint32_t)kdim(c));
        kop[c] = fp8x8_to_bf16x8(u32x2{w[0], w[1]});
        kop[c + 1] = fp8x8_to_bf16x8(u32x2{w[2], w[3]});
      }
    } else {
#pragma unroll
      for (int c = 0; c < NCH; ++c) {
        const uint32_t off = base + (uint32_t)(kdim(c) * ESZ);
        kop[c] = FP8 ? fp8x8_to_bf16x8(load8(rk, off)) : as_bf16x8(load16_stream(rk, off));
      }
    }
  }
  bf16x8 vop[KS][NDT];
  if (wave < PVW) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t vblock = (uint32_t)(g * (cap_r >> 3) + ((k0 + 32 * ks) >> 3) + lq) * D;
      if (VPAIR) {
#pragma unroll
        for (int dt = 0; dt < NDT; dt += 2) {
          const u32x4 w = load16_stream(rv, (vblock + (uint32_t)vdim(dt)) * 8);
          vop[ks][dt] = fp8x8_to_bf16x8(u32x2{w[0], w[1]});
          vop[ks][dt + 1] = fp8x8_to_bf16x8(u32x2{w[2], w[3]});
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint32_t off = (vblock + (uint32_t)vdim(dt)) * 8 * ESZ;
          vop[ks][dt] = FP8 ? fp8x8_to_bf16x8(load8(rv, off)) : as_bf16x8(load16_stream(rv, off));
        }
      }
    }
  }
  // Q of the group's rows, once per workgroup, into LDS (rows past p.rows
  // load row 0 and store zeros)
  constexpr int QPIECES = ROWS * D / 8;
#pragma unroll
  for (int k = 0; k < (QPIECES + 64 * NW - 1) / (64 * NW); ++k) {
    const int idx = threadIdx.x + k * 64 * NW;
    if (idx < QPIECES) {
      const int row = idx / (D / 8), d8 = (idx - row * (D / 8)) * 8;
      const bool ok = row < p.rows;
      const int rr = ok ? row : 0;
      const int i = rr / G, h = rr - (rr / G) * G;
      const bf16x8 v = *reinterpret_cast<const bf16x8*>(p.q + ((size_t)(b * S + i) * p.Hq + g * G + h) * D + d8);
      *reinterpret_cast<bf16x8*>(&qbuf[row][d8]) = ok ? v : bf16x8{};
    }
  }
  // softmax role: slot wave*4 + lane/16 takes row `srow` (slots past the
  // rows idle), keys k0 + KPL*(lane%16) ..; its query position is fetched
  // with the loads
  const int srow = wave * 4 + lq;
  const bool srow_ok = srow < p.rows;
  const int qp = p.pos[b * S + (srow_ok ? srow : 0) / G];

  const int n_keys = unit_keys(p, b);
  if (k0 >= n_keys) return;  // past this request's keys (uniform over the workgroup)

  // ---------------------------------------------------------- scores
  __syncthreads();  // Q in LDS
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      acc = mfma16x16x32(kop[c], *reinterpret_cast<const bf16x8*>(&qbuf[ct * 16 + lr][dh * DH + kdim(c)]), acc);
    *reinterpret_cast<f32x4*>(&sbuf[dh][ct * 16 + lr][16 * kq + 4 * lq]) = acc;
  }
  __syncthreads();

  // ---------------------------------------------------------- softmax
  const size_t slot = ((size_t)unit * p.nchunk + chunk) * p.rows;
  if (srow < ROWS) {
    const int kk = KPL * lr;
    float sv[KPL];
    float mx = -INFINITY;
#pragma unroll
    for (int e4 = 0; e4 < KPL; e4 += 4) {
      const f32x4 s0 = *reinterpret_cast<const f32x4*>(&sbuf[0][srow][kk + e4]);
      const f32x4 s1 = *reinterpret_cast<const f32x4*>(&sbuf[1][srow][kk + e4]);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int key = k0 + kk + e4 + e;
        const bool vis = srow_ok && key < n_keys && key <= qp;
        sv[e4 + e] = vis ? (s0[e] + s1[e]) * p.qk_scale : -INFINITY;
        mx = fmaxf(mx, sv[e4 + e]);
      }
    }
    const float m = max16lanes(mx);
    const float m_use = (m == -INFINITY) ? 0.f : m;
    float ps = 0.f;
#pragma unroll
    for (int e4 = 0; e4 < KPL; e4 += 4) {
      bf16x4 pb;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pb[e] = (__bf16)fast_exp2(sv[e4 + e] - m_use);
        ps += (float)pb[e];
      }
      *reinterpret_cast<bf16x4*>(&pbuf[srow][kk + e4]) = pb;
    }
    const float l = sum16lanes(ps);
    if (lr == 0 && srow_ok) {
      p.ws_pml[(slot + srow) * 2 + 0] = m;
      p.ws_pml[(slot + srow) * 2 + 1] = l;
    }
  }
  __syncthreads();
  if (wave >= PVW) return;

  // ---------------------------------------------------------- values
  if (k0 + CK > n_keys) {  // last chunk: zero values of keys past the count
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      u32x4 keep;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int kk = k0 + 32 * ks + 8 * lq + 2 * j;
        keep[j] = (kk < n_keys ? 0x0000FFFFu : 0u) | (kk + 1 < n_keys ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        vop[ks][dt] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vop[ks][dt]) & keep);
    }
  }
  f32x4 o[NCT][NDT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const bf16x8 pt = *reinterpret_cast<const bf16x8*>(&pbuf[ct * 16 + lr][32 * ks + 8 * lq]);
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[ct][dt] = mfma16x16x32(vop[ks][dt], pt, o[ct][dt]);
    }
  }
  // Lane (lr, lq) holds rows ct*16 + lr; group q of four consecutive dims
  // starts at qdim(q).
  auto qdim = [&](int q) { return vw * DPW + (VPAIR ? 32 * (q >> 1) + 8 * lq + 4 * (q & 1) : 16 * q + 4 * lq); };
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int row = ct * 16 + lr;
    if (row >= p.rows) continue;
    float* dst = p.ws_part + (slot + row) * D;
#pragma unroll
    for (int q = 0; q < NDT; ++q) {
      f32x4 v;
      if (VPAIR) {
        const int t = q & ~1, hh = 2 * (q & 1);
        v = f32x4{o[ct][t][hh], o[ct][t + 1][hh], o[ct][t][hh + 1], o[ct][t + 1][hh + 1]};
      } else {
        v = o[ct][q];
      }
      __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(dst + qdim(q)));
    }
  }
}

// ------------------------------------------------------------------ pass 2

// One workgroup per (request, KV head, row, quarter of the head dims).  Thread
// group k of NG takes chunks k, k+NG, ... for its four dims; every chunk's
// (max, sum, row) loads of a batch are issued together, with indices clamped
// to the launch's chunk count and issued before the request's chunk count
// is known (chunks past it are dropped by select, never multiplied, so
// whatever they hold cannot leak in).  Each group keeps a running
// (M, L, O) rescaled between batches; the groups are then merged in group
// order through LDS.  out = v_scale * sum_c 2^(m_c - M) acc_c /
// sum_c 2^(m_c - M) l_c.
constexpr int kMergeThreads = 256;
constexpr int kMaxChunks = 512;  // 65536 keys
constexpr int kMergeBatch = 16;

template <int D>
__global__ void __launch_bounds__(kMergeThreads) chunk_merge_kernel(const AttnParams p) {
  constexpr int PART = D / 4;                  // dims per workgroup
  constexpr int TPG = PART / 4;                // threads per group (4 dims each)
  constexpr int NG = kMergeThreads / TPG;      // chunk groups
  __shared__ float gml[NG][2];
  __shared__ __attribute__((aligned(16))) float obuf[NG][PART];

  const int tid = threadIdx.x;
  const int quarter = blockIdx.x & 3;
  const int ur = blockIdx.x >> 2;              // unit * rows + row
  const int unit = ur / p.rows;
  const int row = ur - unit * p.rows;
  const int b = unit / p.Hkv, g = unit - (unit / p.Hkv) * p.Hkv;
  const int grp = tid / TPG;
  const int d4 = (tid - grp * TPG) * 4;
  const size_t slot0 = (size_t)unit * p.nchunk * p.rows + row;  // + c * rows

  float M = -INFINITY, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  int nvalid = p.nchunk;
  for (int c0 = grp; c0 < nvalid; c0 += kMergeBatch * NG) {
    float m[kMergeBatch], l[kMergeBatch];
    f32x4 a[kMergeBatch];
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const size_t at = slot0 + (size_t)min(c0 + j * NG, p.nchunk - 1) * p.rows;
      m[j] = p.ws_pml[at * 2];
      l[j] = p.ws_pml[at * 2 + 1];
      a[j] = *reinterpret_cast<const f32x4*>(p.ws_part + at * D + quarter * PART + d4);
    }
    if (c0 == grp) nvalid = min((unit_keys(p, b) + kChunkKeys - 1) / kChunkKeys, p.nchunk);
    float mb = M;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) mb = (c0 + j * NG < nvalid) ? fmaxf(mb, m[j]) : mb;
    const float m_use = (mb == -INFINITY) ? 0.f : mb;
    const float alpha = fast_exp2(M - m_use);  // 0 while nothing was merged
    L *= alpha;
    O *= alpha;
#pragma unroll
    for (int j = 0; j < kMergeBatch; ++j) {
      const bool ok = c0 + j * NG < nvalid;
      const float w = fast_exp2(m[j] - m_use);
      L += ok ? l[j] * w : 0.f;
      O += ok ? a[j] * w : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    M = mb;
  }
  if (d4 == 0) {
    gml[grp][0] = M;
    gml[grp][1] = L;
  }
  *reinterpret_cast<f32x4*>(&obuf[grp][d4]) = O;
  __syncthreads();
  if (grp != 0) return;
  float Mt = gml[0][0];
#pragma unroll
  for (int k = 1; k < NG; ++k) Mt = fmaxf(Mt, gml[k][0]);
  const float mt_use = (Mt == -INFINITY) ? 0.f : Mt;
  float Lt = 0.f;
  f32x4 Ot = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < NG; ++k) {
    const float w = fast_exp2(gml[k][0] - mt_use);
    Lt += gml[k][1] * w;
    Ot += *reinterpret_cast<const f32x4*>(&obuf[k][d4]) * w;
  }
  const float inv = Lt > 0.f ? p.v_scale / Lt : 0.f;
  const int i = row / p.G, h = row - (row / p.G) * p.G;
  bf16x4 w = {(__bf16)(Ot[0] * inv), (__bf16)(Ot[1] * inv), (__bf16)(Ot[2] * inv), (__bf16)(Ot[3] * inv)};
  *reinterpret_cast<bf16x4*>(p.out + ((size_t)(b * p.S + i) * p.Hq + g * p.G + h) * D + quarter * PART + d4) = w;
}

// ------------------------------------------------------------------ host

namespace {

int cdiv(long a, long b) { return (int)((a + b - 1) / b); }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

template <int D, int NCT>
hipError_t launch_chunks(const AttnPlan& pl, const AttnParams& p, hipStream_t s) {
  const dim3 grid(pl.units * pl.nchunk), block(64 * kChunkWaves);
  if (pl.fp8)
    hipLaunchKernelGGL((chunk_kernel<D, NCT, true>), grid, block, 0, s, p);
  else
    hipLaunchKernelGGL((chunk_kernel<D, NCT, false>), grid, block, 0, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_merge_kernel<D>), dim3(pl.units * pl.rows * 4), dim3(kMergeThreads), 0, s, p);
  return hipGetLastError();
}

}  // namespace

bool plan_global(int B, int S, int Hq, int Hkv, int D, int max_keys, AttnPlan* pl) {
  if (B < 0 || S < 1 || S > 8 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || max_keys < 1) return false;
  if (D != 64 && D != 128 && D != 256 && D != 512) return false;
  const int rows = (Hq / Hkv) * S;
  if (rows > 32) return false;
  const int nchunk = cdiv(max_keys, kChunkKeys);
  if (nchunk > kMaxChunks) return false;
  pl->mode = MODE_GLOBAL;
  pl->D = D;
  pl->nct = rows > 16 ? 2 : 1;
  pl->rows = rows;
  pl->units = B * Hkv;
  pl->threads = 64 * kChunkWaves;
  pl->max_tiles = cdiv(max_keys, 32);
  pl->kw = 1;
  pl->nsplit = 1;
  pl->tiles_per_split = pl->max_tiles;
  pl->nchunk = nchunk;
  size_t off = 0;
  pl->off_part = off;
  off = align256(off + (size_t)pl->units * nchunk * rows * D * sizeof(float));
  pl->off_pml = off;
  off = align256(off + (size_t)pl->units * nchunk * rows * 2 * sizeof(float));
  pl->ws_bytes = pl->units > 0 ? off : 0;
  pl->lds_bytes = 0;
  return true;
}

hipError_t launch_global(const AttnPlan& pl, const AttnParams& p0, hipStream_t s) {
  if (pl.units == 0) return hipSuccess;
  AttnParams p = p0;
  p.nchunk = pl.nchunk;
  const bool two = pl.nct == 2;
  switch (pl.D) {
    case 64: return two ? launch_chunks<64, 2>(pl, p, s) : launch_chunks<64, 1>(pl, p, s);
    case 128: return two ? launch_chunks<128, 2>(pl, p, s) : launch_chunks<128, 1>(pl, p, s);
    case 256: return two ? launch_chunks<256, 2>(pl, p, s) : launch_chunks<256, 1>(pl, p, s);
    case 512: return two ? launch_chunks<512, 2>(pl, p, s) : launch_chunks<512, 1>(pl, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace swr
