// attn.hip -- grouped-query attention over per-request sliding-window rings
// on gfx950 (global layers and small-batch verify in chunked form: chunked.hip).
//
// One kernel template serves the two ring entry points and long global calls:
//   decode  : one query token per request over its sliding-window ring
//             ("Announcing Carat", ring buffer section; "Improving Decode
//             Throughput on Intel Gaudi 3", Our approach: the ring is read in
//             place, in storage order, with no gather and no un-rotation);
//             with the append, the same launch first writes the new token
//             into its slot (the token replaces the oldest one);
//   verify  : G heads x S proposals per KV head over the ring plus the
//             proposals ("Announcing Carat", Doing it all in one kernel can be
//             slower: the grouped rows share one K/V stream);
//   gstream : a global layer over contiguous regions (keys 0 .. key_count-1,
//             causal by query position) when the regions are long enough that
//             one streaming pass with a split-K merge beats the chunked form
//             of chunked.hip.
//
// Work unit: one (request, KV head).  A workgroup takes a range of 32-key
// tiles of one unit (split-K across workgroups when the batch is small); its
// waves split the tiles (kw) and/or the head dimension (ds).  Per tile, per
// wave:
//   scores  = K(32 keys x ds) . Q^T(ds x rows)    bf16 MFMA 16x16x32, fp32
//   (waves sharing a tile add their ds-partial scores through LDS)
//   online softmax in the base-2 domain, per row, in fp32
//   O^T    += V^T(ds x 32 keys) . P^T(32 keys x rows)   bf16 MFMA, fp32
// Keys are laid out on the MFMA k axis so that the score fragment a lane
// holds (row l%16, keys 8*(l/16)+0..7) is exactly the P^T fragment it must
// supply, and the V^T fragment is one 16-byte load from the 8-slot V blocks
// of the region layout.  No shuffles sit between the two contractions.  K
// is stored in that same key order (swr_device.h), so each K operand load of
// a lane group is 1 KB of contiguous memory.
//
// fp8 K/V are read 16 bytes per lane like bf16 (not 8): a K load covers two
// 8-dim k chunks, which is a fixed permutation of the head-dim (k) axis that
// Q takes too; a V load covers the 8 keys of two adjacent dims, which feed
// two consecutive value tiles (even and odd dims), and the output stores
// interleave them back.
#include <algorithm>

#include "swr_device.h"
#include "swr_internal.h"

namespace swr {

// An empty instruction that reads v: what computes v is placed before it
// (and v's own load, if any, waited for), and with the memory clobber no load
// or store moves across it.
__device__ __forceinline__ void pin(u32x4 v) { asm volatile("" ::"v"(v) : "memory"); }
// The same as a read-write of v: what uses v afterwards stays after it.
__device__ __forceinline__ void hold(u32x4& v) { asm volatile("" : "+v"(v)::"memory"); }

// Slots of request b's region (global regions may carry a capacity each).
__device__ __forceinline__ int region_cap(const AttnParams& p, int b) {
  return p.cap_b ? max(min(p.cap_b[b], p.cap), 0) : p.cap;
}

template <int D, int DS, int NCT, int KW, bool FP8, int MODE, int WPE>
__global__ void __launch_bounds__(64 * (D / DS) * KW) __attribute__((amdgpu_waves_per_eu(WPE)))
attn_kernel(const AttnParams p) {
  constexpr int DSPLIT = D / DS;
  constexpr int NCH = DS / 32;  // QK k-chunks of 32 dims
  constexpr int NDT = DS / 16;  // PV tiles of 16 dims
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr int RED = 2 * NCT * 4;  // score floats per lane per tile
  constexpr int RS = D + 4;         // padded LDS row stride (floats)
  constexpr bool DEC = MODE == MODE_DECODE || MODE == MODE_DECODE_APPEND;
  constexpr bool GS = MODE == MODE_GSTREAM || MODE == MODE_GSTREAM_APPEND;
  constexpr bool APP = MODE == MODE_DECODE_APPEND || MODE == MODE_GSTREAM_APPEND;
  static_assert(!(APP && FP8) || DS <= 256, "an fp8 append writes a slice's K and V from one wave's lanes");
  extern __shared__ float smem[];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform: scalar registers
  const int ds = wave % DSPLIT;
  const int kw = wave / DSPLIT;
  const int lr = lane & 15;  // row within a 16-row column tile; also key row of the K operand
  const int lq = lane >> 4;  // lane group: which 8 keys / 8 dims of the k axis

  // gstream: the split balanced from the requests' key counts (split tiles
  // [st_lo, st_hi)); the workgroups past the last split exit here
  int unit, split, st_lo = 0, st_hi = 0;
  if constexpr (GS) {
    const StreamSplit x = stream_split(p, blockIdx.x);
    if (x.unit < 0) return;
    unit = x.unit;
    split = x.split;
    st_lo = (int)((long)x.split * x.tiles / x.n);
    st_hi = (int)((long)(x.split + 1) * x.tiles / x.n);
  } else {
    unit = blockIdx.x / p.nsplit;
    split = blockIdx.x - unit * p.nsplit;
  }
  const int Hkv = p.Hkv, G = p.G, S = p.S;
  const int b = unit / Hkv;
  const int g = unit - b * Hkv;
  const int d_base = ds * DS;
  // Head dim of k element 8*lq + j of QK chunk c (relative to d_base), and
  // head dim of A row lr of value tile dt (absolute).
  auto kdim = [&](int c) { return FP8 ? 64 * (c >> 1) + 16 * lq + 8 * (c & 1) : (4 * c + lq) * 8; };
  auto vdim = [&](int dt) { return FP8 ? d_base + 32 * (dt >> 1) + 2 * lr + (dt & 1) : d_base + 16 * dt + lr; };

  // ---------------------------------------------------------------- keys
  const int cap_r = region_cap(p, b);
  int n_keys;         // ring slots ever written; global: keys of the request
  int ring_head = 0;  // verify: slot of the newest committed position
  if (DEC) {
    n_keys = min(p.pos[b] + 1, p.cap);
  } else if (MODE == MODE_VERIFY) {
    const int p0 = p.pos[b];
    n_keys = min(p0, p.cap);
    ring_head = p0 > 0 ? (p0 - 1) % p.cap : 0;
  } else {
    n_keys = min(key_count_of(p, b), cap_r);
  }
  n_keys = max(n_keys, 0);
  const int nt_region = (n_keys + 31) >> 5;
  const int nt_total = nt_region + (MODE == MODE_VERIFY ? 1 : 0);
  const int t_begin = GS ? st_lo : split * p.tiles_per_split;
  const int t_end = min(nt_total, GS ? st_hi : t_begin + p.tiles_per_split);
  if (t_begin >= t_end) return;  // empty split: the combine step skips it
  const int n_it = (t_end - t_begin + KW - 1) / KW;

  // ---------------------------------------------------------------- rows
  // Row r = i*G + h: proposal i, head h of the group (query head g*G + h).
  bool row_ok[NCT];
  int row_i[NCT];
  int row_lim[NCT];  // verify: largest slot age still in the window; global: last visible key
  bf16x8 qop[NCT][NCH];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    const int row = ct * 16 + lr;
    row_ok[ct] = row < p.rows;
    const int i = row_ok[ct] ? row / G : 0;
    const int h = row_ok[ct] ? row - i * G : 0;
    row_i[ct] = i;
    row_lim[ct] = GS ? min(qpos_of(p, b, i), n_keys - 1) : p.cap - 2 - i;
    const uint16_t* qrow = p.q + ((size_t)(b * S + i) * p.Hq + g * G + h) * D + d_base;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      if (row_ok[ct])
        qop[ct][c] = *reinterpret_cast<const bf16x8*>(qrow + kdim(c));
      else
        qop[ct][c] = bf16x8{};
    }
  }

  const int S_r = stored_slots(cap_r);  // slots stored per KV head (region layout: swr_device.h)
  const uint32_t region_bytes = (uint32_t)S_r * (uint32_t)(Hkv * D * ESZ);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_base + p.k_off[b], region_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_base + p.v_off[b], region_bytes);

  f32x4 o[NCT][NDT];
  float m_run[NCT], l_run[NCT];
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) {
    m_run[ct] = -INFINITY;
    l_run[ct] = 0.f;
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // K and V operand registers.  The loads for tile t+KW are issued as soon as
  // tile t has consumed the registers (K after the score product, V after the
  // value product), so every wave keeps a tile's worth of loads in flight
  // while it computes.  fp8 outside verify (RAW): the loads land as codes
  // (kraw, vraw) and are converted to bf16 operands only where the tile is
  // used, since a conversion next to its load makes the wave wait for the
  // tile there and then; the next tile's loads then go out as soon as this
  // tile's codes are converted.  (fp8 verify converts at the load: the raw
  // registers would cost its larger row tiles occupancy.)
  constexpr bool RAW = FP8 && MODE != MODE_VERIFY;
  bf16x8 kop[2][NCH];
  bf16x8 vop[NDT];
  u32x4 kraw[2][RAW ? NCH / 2 : 1];
  u32x4 vraw[RAW ? NDT / 2 : 1];

  // RAW: a wave with no next tile still issues its next-tile loads, through
  // a resource of zero bytes (they return zeros and read nothing), so that
  // the loop has no branch around its loads and every wait can count exactly
  // the loads ahead of the ones it needs.
  const __amdgpu_buffer_rsrc_t rnull = make_rsrc(p.k_base, 0);
  auto load_k = [&](int t, bool live = true) {
    const int kb = t * 32;
    const bool prop_tile = (MODE == MODE_VERIFY) && (t == nt_region);
#pragma unroll
    for (int sub = 0; sub < 2; ++sub) {
      // A row lr of sub-tile `sub` holds key 8*(lr/4) + 4*sub + lr%4, so the
      // C rows lane group lq receives are keys 8*lq + 4*sub + 0..3.  In the
      // region that key is row lr of half `sub` of the tile: the lane reads
      // 16 bytes of granule (d_base + kdim(c)) / R of that row.
      const int e = 8 * (lr >> 2) + 4 * sub + (lr & 3);
      if (!prop_tile) {
        constexpr int R = FP8 ? 16 : 8;  // dims per 16-byte granule
        const uint32_t hb = k_half_base(g, S_r, kb, sub, D, ESZ);
        if (RAW) {
#pragma unroll
          for (int c = 0; c < NCH; c += 2)
            kraw[sub][c / 2] = load16_stream(live ? rk : rnull, hb + k_granule_offset((d_base + kdim(c)) / R, lr));
        } else if (FP8) {
#pragma unroll
          for (int c = 0; c < NCH; c += 2) {
            const u32x4 w = load16_stream(rk, hb + k_granule_offset((d_base + kdim(c)) / R, lr));
            kop[sub][c] = fp8x8_to_bf16x8(u32x2{w[0], w[1]});
            kop[sub][c + 1] = fp8x8_to_bf16x8(u32x2{w[2], w[3]});
          }
        } else {
#pragma unroll
          for (int c = 0; c < NCH; ++c)
            kop[sub][c] = as_bf16x8(load16_stream(rk, hb + k_granule_offset((d_base + kdim(c)) / R, lr)));
        }
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) kop[sub][c] = bf16x8{};
        if (e < S) {
          const uint16_t* src = p.k_prop + ((size_t)(b * S + e) * Hkv + g) * D + d_base;
#pragma unroll
          for (int c = 0; c < NCH; ++c) kop[sub][c] = *reinterpret_cast<const bf16x8*>(src + kdim(c));
        }
      }
    }
  };

  // Proposal values (bf16, outside the ring) as the V^T operand of tile dt.
  // Over an fp8 ring the accumulator holds values in units of v_scale, so a
  // proposal enters as v / v_scale, split into a bf16 head and (second
  // pass, lo = true) the bf16 remainder: the pair carries it to ~2^-16.
  auto prop_v = [&](int dt, bool lo) -> bf16x8 {
    const int d = vdim(dt);
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pi = 8 * lq + e;
      uint16_t bits = 0;
      if (pi < S) bits = p.v_prop[((size_t)(b * S + pi) * Hkv + g) * D + d];
      if (FP8) {
        const float x = __builtin_bit_cast(float, (uint32_t)bits << 16) * p.inv_v_scale;
        const __bf16 hi = (__bf16)x;
        v[e] = lo ? (__bf16)(x - (float)hi) : hi;
      } else {
        v[e] = __builtin_bit_cast(__bf16, bits);
      }
    }
    return v;
  };

  auto load_v = [&](int t, bool live = true) {
    const int kb = t * 32;
    const bool prop_tile = (MODE == MODE_VERIFY) && (t == nt_region);
    if (!prop_tile) {
      const uint32_t vblock = (uint32_t)(g * (S_r >> 3) + (kb >> 3) + lq) * D;
      if (RAW) {
#pragma unroll
        for (int dt = 0; dt < NDT; dt += 2)
          vraw[dt / 2] = load16_stream(live ? rv : rnull, (vblock + (uint32_t)vdim(dt)) * 8);
      } else if (FP8) {
#pragma unroll
        for (int dt = 0; dt < NDT; dt += 2) {
          const u32x4 w = load16_stream(rv, (vblock + (uint32_t)vdim(dt)) * 8);
          vop[dt] = fp8x8_to_bf16x8(u32x2{w[0], w[1]});
          vop[dt + 1] = fp8x8_to_bf16x8(u32x2{w[2], w[3]});
        }
      } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) vop[dt] = as_bf16x8(load16_stream(rv, (vblock + (uint32_t)vdim(dt)) * 16));
      }
    } else {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) vop[dt] = prop_v(dt, false);
    }
  };

  // RAW: the codes of a tile as bf16 operands
  auto cvt_k = [&]() {
    if constexpr (RAW) {
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int c = 0; c < NCH; c += 2) {
          kop[sub][c] = fp8x8_to_bf16x8(u32x2{kraw[sub][c / 2][0], kraw[sub][c / 2][1]});
          kop[sub][c + 1] = fp8x8_to_bf16x8(u32x2{kraw[sub][c / 2][2], kraw[sub][c / 2][3]});
        }
    }
  };
  auto cvt_v = [&]() {
    if constexpr (RAW) {
      // held behind the next tile's K loads: converted ahead of them, the
      // codes would have to arrive before those loads could go out
#pragma unroll
      for (int j = 0; j < NDT / 2; ++j) hold(vraw[j]);
#pragma unroll
      for (int dt = 0; dt < NDT; dt += 2) {
        vop[dt] = fp8x8_to_bf16x8(u32x2{vraw[dt / 2][0], vraw[dt / 2][1]});
        vop[dt + 1] = fp8x8_to_bf16x8(u32x2{vraw[dt / 2][2], vraw[dt / 2][3]});
      }
    }
  };

  // Fused append (decode; a streamed global call of one token per request):
  // the new token, position pos in slot pos % W (global: slot pos), is
  // written by the waves that read its tile, each its own head-dim slice; no
  // other workgroup reads the tile.
  //  bf16: the wave loads the tile as it is (the slot still holds the token
  //   it evicts), puts the new token into its operand registers, and stores
  //   back every cache line of the tile that holds a byte of the slot, whole
  //   (a line left partly written costs its next reader a merge with memory,
  //   which over a batch measured about as much as a separate append launch).
  //   The stores go out after the tile's score product: ahead of it they
  //   would sit in front of the loads that the product waits for, and that
  //   wait (the load counter counts stores as well) would hold the wave until
  //   they were acknowledged.  The tiles are walked in storage order, as the
  //   decode walks them: rotating each split to end on the token's tile
  //   measured 1-3 us slower at B=56 over rings carved from one pool (74.2 -
  //   74.5 us against 75.3 - 77.6 us for three sets of positions).
  //  fp8 (the registers hold decoded values, not the stored codes): the
  //   stores go out with the first loads and the wave waits for them once,
  //   before the token tile's loads; the split walks its tiles in rotated
  //   order, starting after the token's tile, so that the wait falls at the
  //   end of the wave's read stream.
  constexpr bool SUBST = APP && !FP8;
  constexpr bool FIRST = APP && FP8;
  const int nt = t_end - t_begin;
  int rot = 0;  // local tile index lam is tile t_begin + (lam + rot) mod nt
  bool writer = false;
  int t_new = -1, slot_new = 0;
  if (APP) {
    // a ring slot is the position mod W; a global region's slot is the
    // position itself, stored only below the request's capacity
    slot_new = DEC ? p.pos[b] % p.cap : p.pos[b];
    t_new = slot_new >> 5;
    if (t_new >= t_begin && t_new < t_end && (DEC || slot_new < cap_r)) {
      if (FIRST) {
        rot = t_new - t_begin + 1;
        if (rot == nt) rot = 0;
        writer = kw == (nt - 1) % KW;
      } else {
        writer = kw == (t_new - t_begin) % KW;  // the wave whose tile it is
      }
    }
  }
  auto tile_at = [&](int lam) {
    int x = lam + rot;
    if (x >= nt) x -= nt;
    return t_begin + x;
  };
  // fp8: lane l < DS/8 encodes K dims 8*(d_base/8 + l) .. +7 and lane
  // DS/8 + l the same dims of V, which halves the chain of encodes a lane runs
  auto write_new = [&]() {
    if (FIRST && lane < DS / 4) {
      const bool is_v = lane >= DS / 8;
      const int d8 = d_base / 8 + lane - (is_v ? DS / 8 : 0);
      const size_t src = ((size_t)b * Hkv + g) * D + (size_t)d8 * 8;
      const u32x4 bits = *reinterpret_cast<const u32x4*>((is_v ? p.v_prop : p.k_prop) + src);
      store_token_half_fp8(rk, rv, slot_new, g, S_r, D, d8, is_v, bits, is_v ? p.v_scale_store : p.k_scale_store);
    }
  };

  // bf16: the wave's slice of the new token, staged in LDS until its tile
  // comes round (K granules and V values by head dim)
  __shared__ __attribute__((aligned(16))) __bf16 stage_k[SUBST ? D : 8], stage_v[SUBST ? D : 8];
  const int k32_new = slot_new & 31;
  const int h_new = (k32_new >> 2) & 1, r_new = 4 * (k32_new >> 3) + (k32_new & 3);

  if (kw < nt) {
    const int t0 = tile_at(kw);
    if (FIRST && writer && t0 == t_new) {  // the wave's only tile: store, wait, then load
      write_new();
      wait_vm_all();
    }
    load_k(t0);
    load_v(t0);
    if (FIRST && writer && t0 != t_new) write_new();
    if (SUBST && writer && lane < DS / 8) {
      const size_t src = ((size_t)b * Hkv + g) * D + d_base + (size_t)lane * 8;
      *reinterpret_cast<u32x4*>(&stage_k[d_base + lane * 8]) = *reinterpret_cast<const u32x4*>(p.k_prop + src);
      *reinterpret_cast<u32x4*>(&stage_v[d_base + lane * 8]) = *reinterpret_cast<const u32x4*>(p.v_prop + src);
    }
  }

  if (RAW) {
    // Q's loads, issued before the first tile's, are waited for here, behind
    // them: left pending into the loop they would make the loop's first
    // product wait for every load in flight
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int c = 0; c < NCH; ++c) pin(__builtin_bit_cast(u32x4, qop[ct][c]));
  }

  for (int it = 0; it < n_it; ++it) {
    const int lam = kw + it * KW;
    if (lam >= nt) {  // wave-uniform; keeps the barrier count equal across waves
      if (DSPLIT > 1) __syncthreads();
      continue;
    }
    const int t = tile_at(lam);
    const bool has_next = lam + KW < nt;
    const int t_next = has_next ? tile_at(lam + KW) : 0;
    const bool prop_tile = (MODE == MODE_VERIFY) && (t == nt_region);
    const int kb = t * 32;
    const bool subst = SUBST && writer && t == t_new;  // wave-uniform
    // RAW: the next tile's loads go out as soon as this tile's codes are
    // converted; the other forms load straight into the operand registers,
    // after this tile's product has read them
    const int t_load = has_next ? t_next : t;
    auto next_k = [&]() {
      if (FIRST && writer && has_next && t_next == t_new) wait_vm_all();
      load_k(t_load, has_next);
    };

    if (subst) {
      // K: row r_new of half h_new is the new token
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (sub != h_new) continue;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          if (lr == r_new) kop[sub][c] = *reinterpret_cast<const bf16x8*>(&stage_k[d_base + kdim(c)]);
      }
      // V: lane group k32/8 holds the slot's 8-key blocks; element k32%8 of
      // each is the new token
      if (lq == (k32_new >> 3)) {
        const int e = k32_new & 7;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          u32x4 w = __builtin_bit_cast(u32x4, vop[dt]);
          const uint32_t nv = __builtin_bit_cast(uint16_t, stage_v[vdim(dt)]);
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j == (e >> 1)) w[j] = (e & 1) ? ((w[j] & 0x0000FFFFu) | (nv << 16)) : ((w[j] & 0xFFFF0000u) | nv);
          }
          vop[dt] = __builtin_bit_cast(bf16x8, w);
        }
      }
    }

    // ------------------------------------------------ scores = K . Q^T
    if (RAW) cvt_k();
    if (RAW) {  // the conversions first, so that the loads reuse their registers
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int c = 0; c < NCH; ++c) pin(__builtin_bit_cast(u32x4, kop[sub][c]));
      next_k();
    }
    f32x4 sc[2][NCT];
#pragma unroll
    for (int sub = 0; sub < 2; ++sub)
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NCH; ++c) acc = mfma16x16x32(kop[sub][c], qop[ct][c], acc);
        sc[sub][ct] = acc;
      }
    if (subst) {
      // the slot's lines, whole, now that the score product has read the
      // operands: K, the lanes of the two rows sharing the token row's lines
      // (one 128-byte line per chunk); V, the 16 lanes of the token's lane
      // group (256 bytes per tile of 16 dims), before the value product's
      // mask of keys past the count touches the registers
      const uint32_t hb = k_half_base(g, S_r, kb, h_new, D, ESZ);
#pragma unroll
      for (int sub = 0; sub < 2; ++sub) {
        if (sub != h_new) continue;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
          if ((lr >> 1) == (r_new >> 1))
            store16(rk, hb + k_granule_offset((d_base + kdim(c)) / 8, lr), __builtin_bit_cast(u32x4, kop[sub][c]));
      }
      if (lq == (k32_new >> 3)) {
        const uint32_t vblock = (uint32_t)(g * (S_r >> 3) + (kb >> 3) + lq) * D;
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt)
          store16(rv, (vblock + (uint32_t)vdim(dt)) * 16, __builtin_bit_cast(u32x4, vop[dt]));
      }
    }
    if (!RAW && has_next) next_k();

    if (DSPLIT > 1) {  // add the head-dim slices of the scores, in slice order
      float* buf = smem + (size_t)((it & 1) * KW + kw) * DSPLIT * RED * 64;
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) buf[(ds * RED + (sub * NCT + ct) * 4 + r) * 64 + lane] = sc[sub][ct][r];
      __syncthreads();
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            float a = 0.f;
#pragma unroll
            for (int s2 = 0; s2 < DSPLIT; ++s2) a += buf[(s2 * RED + (sub * NCT + ct) * 4 + r) * 64 + lane];
            sc[sub][ct][r] = a;
          }
    }

    // ------------------------------------------------ masked online softmax
    // (proposal keys are bf16 values: no k_scale folded into their scores)
    const float qs = (FP8 && prop_tile) ? p.qk_scale_prop : p.qk_scale;
    bf16x8 pop[NCT];
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      float s[8];
#pragma unroll
      for (int sub = 0; sub < 2; ++sub)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int e = 4 * sub + r;     // element of the P^T fragment
          const int key = kb + 8 * lq + e;
          bool vis;
          if (DEC) {
            vis = key < n_keys;
          } else if (GS) {
            vis = key <= row_lim[ct];
          } else if (prop_tile) {
            const int pi = 8 * lq + e;  // proposal index
            vis = pi < S && pi <= row_i[ct];
          } else {
            int age = ring_head - key;  // positions back from the newest committed one
            if (age < 0) age += p.cap;
            vis = key < n_keys && age <= row_lim[ct];
          }
          vis = vis && row_ok[ct];
          s[e] = vis ? sc[sub][ct][r] * qs : -INFINITY;
        }
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
        psum += (float)pb;  // the weights the PV product actually uses
      }
      pop[ct] = pv;
      l_run[ct] = l_run[ct] * alpha + psum;
      m_run[ct] = m_new;
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[ct][dt] *= alpha;
    }

    // ------------------------------------------------ O^T += V^T . P^T
    if (RAW) cvt_v();
    if (RAW) {
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) pin(__builtin_bit_cast(u32x4, vop[dt]));
      load_v(t_load, has_next);
    }
    if (!prop_tile && kb + 32 > n_keys) {  // last region tile: zero values of keys past the valid range
      u32x4 keep;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int k0 = kb + 8 * lq + 2 * j;
        keep[j] = (k0 < n_keys ? 0x0000FFFFu : 0u) | (k0 + 1 < n_keys ? 0xFFFF0000u : 0u);
      }
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt)
        vop[dt] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vop[dt]) & keep);
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) o[ct][dt] = mfma16x16x32(vop[dt], pop[ct], o[ct][dt]);
    if (FP8 && prop_tile) {  // remainder of the scaled proposal values
#pragma unroll
      for (int dt = 0; dt < NDT; ++dt) {
        const bf16x8 vlo = prop_v(dt, true);
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct) o[ct][dt] = mfma16x16x32(vlo, pop[ct], o[ct][dt]);
      }
    }
    if (!RAW && has_next) load_v(t_next);
  }

#pragma unroll
  for (int ct = 0; ct < NCT; ++ct) l_run[ct] = sum4lanes(l_run[ct]);

  // The lane's outputs of row tile ct as NDT groups of four consecutive head
  // dims: group q starts at dim d_base + qdim(q).  bf16 K/V: group dt is tile
  // dt (dims 16*dt + 4*lq + r).  fp8: tiles 2t and 2t+1 hold the even and
  // odd dims of 32*t + 8*lq + 0..7; groups 2t and 2t+1 are its two halves.
  auto qdim = [&](int q) { return FP8 ? 32 * (q >> 1) + 8 * lq + 4 * (q & 1) : 16 * q + 4 * lq; };
  auto qval = [&](int ct, int q) -> f32x4 {
    if (!FP8) return o[ct][q];
    const int t = q & ~1, h = 2 * (q & 1);
    return f32x4{o[ct][t][h], o[ct][t + 1][h], o[ct][t][h + 1], o[ct][t + 1][h + 1]};
  };

  // partial slot: gstream, the split's number (the workgroup); else by unit
  const size_t part = GS ? (size_t)blockIdx.x : (size_t)unit * p.nsplit + split;
  if (KW == 1) {
    // This wave holds rows ct*16+lr, dims d_base + 16*dt + 4*lq + 0..3.
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int row = ct * 16 + lr;
      if (!row_ok[ct]) continue;
      const int i = row / G, h = row - (row / G) * G;
      if (p.nsplit == 1) {
        const float inv = l_run[ct] > 0.f ? p.v_scale / l_run[ct] : 0.f;
        uint16_t* dst = p.out + ((size_t)(b * S + i) * p.Hq + g * G + h) * D + d_base;
#pragma unroll
        for (int q = 0; q < NDT; ++q) {
          const f32x4 v = qval(ct, q);
          bf16x4 w = {(__bf16)(v[0] * inv), (__bf16)(v[1] * inv), (__bf16)(v[2] * inv), (__bf16)(v[3] * inv)};
          *reinterpret_cast<bf16x4*>(dst + qdim(q)) = w;
        }
      } else {
        float* dst = p.ws_acc + (part * p.rows + row) * D + d_base;
#pragma unroll
        for (int q = 0; q < NDT; ++q) *reinterpret_cast<f32x4*>(dst + qdim(q)) = qval(ct, q);
        if (ds == 0 && lq == 0) {
          p.ws_ml[(part * p.rows + row) * 2 + 0] = m_run[ct];
          p.ws_ml[(part * p.rows + row) * 2 + 1] = l_run[ct];
        }
      }
    }
  } else {
    // Merge the KW key-split waves through LDS, in wave order.
    if (DSPLIT > 1) __syncthreads();  // the score buffer aliases this space
    float* cml = smem;                         // [KW][rows][2]
    float* co = smem + KW * p.rows * 2;        // [KW][rows][RS]
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      const int row = ct * 16 + lr;
      if (!row_ok[ct]) continue;
      if (ds == 0 && lq == 0) {
        cml[(kw * p.rows + row) * 2 + 0] = m_run[ct];
        cml[(kw * p.rows + row) * 2 + 1] = l_run[ct];
      }
#pragma unroll
      for (int q = 0; q < NDT; ++q)
        *reinterpret_cast<f32x4*>(co + (size_t)(kw * p.rows + row) * RS + d_base + qdim(q)) = qval(ct, q);
    }
    __syncthreads();
    const int nchunk = p.rows * (D / 4);
    for (int idx = threadIdx.x; idx < nchunk; idx += blockDim.x) {
      const int row = idx / (D / 4);
      const int d4 = (idx - row * (D / 4)) * 4;
      float M = -INFINITY;
#pragma unroll
      for (int k = 0; k < KW; ++k) M = fmaxf(M, cml[(k * p.rows + row) * 2]);
      const float M_use = (M == -INFINITY) ? 0.f : M;
      float L = 0.f;
      f32x4 O = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KW; ++k) {
        const float w = fast_exp2(cml[(k * p.rows + row) * 2] - M_use);
        L += cml[(k * p.rows + row) * 2 + 1] * w;
        O += *reinterpret_cast<const f32x4*>(co + (size_t)(k * p.rows + row) * RS + d4) * w;
      }
      const int i = row / G, h = row - (row / G) * G;
      if (p.nsplit == 1) {
        const float inv = L > 0.f ? p.v_scale / L : 0.f;
        bf16x4 w = {(__bf16)(O[0] * inv), (__bf16)(O[1] * inv), (__bf16)(O[2] * inv), (__bf16)(O[3] * inv)};
        *reinterpret_cast<bf16x4*>(p.out + ((size_t)(b * S + i) * p.Hq + g * G + h) * D + d4) = w;
      } else {
        *reinterpret_cast<f32x4*>(p.ws_acc + (part * p.rows + row) * D + d4) = O;
        if (d4 == 0) {
          p.ws_ml[(part * p.rows + row) * 2 + 0] = M;
          p.ws_ml[(part * p.rows + row) * 2 + 1] = L;
        }
      }
    }
  }
}

// Split-K merge: out = v_scale * sum_s 2^(m_s - M) acc_s / sum_s 2^(m_s - M) l_s
// over the non-empty splits of each (request, KV head).  One thread per four
// output dims of one row.  Partials are read sixteen splits at a time, all
// loads issued before any is used (indices past the last split are clamped
// to it and their values dropped by selects), so a thread waits for one
// round trip per sixteen splits instead of one per split.
constexpr int kCombineBatch = 16;

template <int MODE>
__global__ void __launch_bounds__(256) combine_kernel(const AttnParams p, int D, int units) {
  const int per_row = D / 4;
  const int per_unit = p.rows * per_row;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= units * per_unit) return;
  const int unit = idx / per_unit;
  const int rem = idx - unit * per_unit;
  const int row = rem / per_row;
  const int d4 = (rem - row * per_row) * 4;
  const int b = unit / p.Hkv, g = unit - (unit / p.Hkv) * p.Hkv;

  static_assert(MODE == MODE_DECODE || MODE == MODE_VERIFY, "a streamed call's splits go to merge_grouped");
  int n_keys = MODE == MODE_VERIFY ? min(p.pos[b], p.cap) : min(p.pos[b] + 1, p.cap);
  n_keys = max(n_keys, 0);
  const int nt_total = ((n_keys + 31) >> 5) + (MODE == MODE_VERIFY ? 1 : 0);
  const int nvalid = min(p.nsplit, (nt_total + p.tiles_per_split - 1) / p.tiles_per_split);

  const size_t base = (size_t)unit * p.nsplit;
  float M = -INFINITY, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = 0; s0 < nvalid; s0 += kCombineBatch) {
    float m[kCombineBatch], l[kCombineBatch];
    f32x4 a[kCombineBatch];
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const size_t at = (base + min(s0 + j, p.nsplit - 1)) * p.rows + row;
      m[j] = p.ws_ml[at * 2];
      l[j] = p.ws_ml[at * 2 + 1];
      a[j] = *reinterpret_cast<const f32x4*>(p.ws_acc + at * D + d4);
    }
    float mb = -INFINITY;
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) mb = (s0 + j < nvalid) ? fmaxf(mb, m[j]) : mb;
    const float M_new = fmaxf(M, mb);
    const float M_use = (M_new == -INFINITY) ? 0.f : M_new;
    const float alpha = fast_exp2(M - M_use);  // 0 while nothing was merged yet
    L *= alpha;
    O *= alpha;
#pragma unroll
    for (int j = 0; j < kCombineBatch; ++j) {
      const bool ok = s0 + j < nvalid;
      const float w = fast_exp2(m[j] - M_use);
      L += ok ? l[j] * w : 0.f;
      O += ok ? a[j] * w : f32x4{0.f, 0.f, 0.f, 0.f};
    }
    M = M_new;
  }
  const float inv = L > 0.f ? p.v_scale / L : 0.f;
  const int i = row / p.G, h = row - (row / p.G) * p.G;
  bf16x4 w = {(__bf16)(O[0] * inv), (__bf16)(O[1] * inv), (__bf16)(O[2] * inv), (__bf16)(O[3] * inv)};
  *reinterpret_cast<bf16x4*>(p.out + ((size_t)(b * p.S + i) * p.Hq + g * p.G + h) * D + d4) = w;
}

// ------------------------------------------------------------------ host

namespace {

struct Shape {
  int ds, kw;
};

// Waves per workgroup: D/ds share each key tile, kw split the tiles.  A
// global layer streamed in one pass takes the decode shapes for up to 16 rows
// and the grouped verify shapes above that.  At 512 dims four 128-dim
// slices share each tile at two waves per SIMD: measured on the 16-request
// mixed step, 225 us (bf16) and 130 us (fp8) against 241 and 187 us for two
// 256-dim slices x two key-split waves at one wave per SIMD.
Shape pick_shape(int mode, int D, int nct) {
  if (mode == MODE_DECODE || mode == MODE_DECODE_APPEND ||
      ((mode == MODE_GSTREAM || mode == MODE_GSTREAM_APPEND) && nct == 1)) {
    switch (D) {
      case 64: return {64, 4};
      case 128: return {128, 4};
      case 256: return {256, 4};
      case 512: return {128, 1};
    }
  } else if (nct == 1) {
    switch (D) {
      case 64: return {64, 1};
      case 128: return {128, 1};
      case 256: return {256, 1};
      case 512: return {256, 1};
    }
  } else {
    switch (D) {
      case 64: return {64, 1};
      case 128: return {128, 1};
      case 256: return {128, 1};
      case 512: return {128, 1};
    }
  }
  return {0, 0};
}

constexpr int kNumCU = 256;

int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }

// Two waves stay resident per SIMD, so that one computes while the other's
// loads are in flight, wherever the kernel then fits the 256 registers of a
// lane without spilling (per the compiler's resource report): the decode
// shapes up to 256 dims (128 for a streamed global call, which holds a
// little more per row) and the 512-dim one (four 128-dim slices per tile),
// and the grouped shapes with 128-dim slices except the verify above 128
// dims (bf16) or 64 dims (fp8).  Everything else keeps one wave and all the
// registers.
template <int D, int DS, int NCT, int KW, bool FP8, int MODE>
constexpr int waves_per_simd() {
  constexpr bool DEC = MODE == MODE_DECODE || MODE == MODE_DECODE_APPEND;
  if (NCT == 1) return ((KW > 1 && (D <= 128 || (D == 256 && DEC))) || (D == 512 && DS <= 128)) ? 2 : 1;
  if (MODE == MODE_VERIFY) return (D <= 64 || (D <= 128 && !FP8)) ? 2 : 1;
  return DS <= 128 ? 2 : 1;
}

template <int D, int DS, int NCT, int KW, int MODE>
hipError_t launch_fixed(const AttnPlan& pl, const AttnParams& p, hipStream_t s) {
  constexpr int W8 = waves_per_simd<D, DS, NCT, KW, true, MODE>();
  constexpr int W16 = waves_per_simd<D, DS, NCT, KW, false, MODE>();
  if (pl.fp8)
    hipLaunchKernelGGL((attn_kernel<D, DS, NCT, KW, true, MODE, W8>), dim3(pl.units * pl.nsplit),
                       dim3(pl.threads), pl.lds_bytes, s, p);
  else
    hipLaunchKernelGGL((attn_kernel<D, DS, NCT, KW, false, MODE, W16>), dim3(pl.units * pl.nsplit),
                       dim3(pl.threads), pl.lds_bytes, s, p);
  return hipGetLastError();
}

// Decode takes the single-row-tile shapes with key-split waves; verify takes
// one wave group per tile; a streamed global call takes the decode shapes for
// up to 16 rows and the grouped shapes above.
template <int MODE>
hipError_t launch_mode(const AttnPlan& pl, const AttnParams& p, hipStream_t s) {
  const bool decode_shape = MODE == MODE_DECODE || MODE == MODE_DECODE_APPEND ||
                            ((MODE == MODE_GSTREAM || MODE == MODE_GSTREAM_APPEND) && pl.nct == 1);
  if constexpr (MODE != MODE_VERIFY) {
    if (decode_shape) {
      switch (pl.D) {
        case 64: return launch_fixed<64, 64, 1, 4, MODE>(pl, p, s);
        case 128: return launch_fixed<128, 128, 1, 4, MODE>(pl, p, s);
        case 256: return launch_fixed<256, 256, 1, 4, MODE>(pl, p, s);
        case 512: return launch_fixed<512, 128, 1, 1, MODE>(pl, p, s);
      }
      return hipErrorInvalidValue;
    }
  }
  if constexpr (MODE == MODE_VERIFY) {
    if (pl.nct == 1) {
      switch (pl.D) {
        case 64: return launch_fixed<64, 64, 1, 1, MODE>(pl, p, s);
        case 128: return launch_fixed<128, 128, 1, 1, MODE>(pl, p, s);
        case 256: return launch_fixed<256, 256, 1, 1, MODE>(pl, p, s);
        case 512: return launch_fixed<512, 256, 1, 1, MODE>(pl, p, s);
      }
      return hipErrorInvalidValue;
    }
  }
  if constexpr (MODE != MODE_DECODE && MODE != MODE_DECODE_APPEND) {
    switch (pl.D) {
      case 64: return launch_fixed<64, 64, 2, 1, MODE>(pl, p, s);
      case 128: return launch_fixed<128, 128, 2, 1, MODE>(pl, p, s);
      case 256: return launch_fixed<256, 128, 2, 1, MODE>(pl, p, s);
      case 512: return launch_fixed<512, 128, 2, 1, MODE>(pl, p, s);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace

// A global call streams in one pass when the K/V of all its units spans at
// least this many 32-key tiles: the split-K partials are then a small
// fraction of the bytes read, and there are enough splits to fill the chip.
constexpr long kStreamTiles = 2048;
// Workgroups of a streamed global call's split pass (at least): two
// resident per CU, so that its splits, balanced from the requests' key
// counts on the device (stream_split), run in one round.  Against fixed
// splits of up to 32 tiles (spread over about four per CU if every unit had
// the longest one's tiles), same box: the 16-request mixed step's global
// layer (contexts log-uniform in 512 .. 65536, 2 KV heads x 512) 213 ->
// 201 us, a B=56 layer with contexts U[1024, 4096] 120.5 -> 104.3 us; 768,
// 1024 and 1536 workgroups (smaller splits, more rounds) were slower on both.
constexpr long kStreamWorkgroups = 2 * kNumCU;

bool plan_attention(int mode, int B, int S, int Hq, int Hkv, int D, int fp8, int cap_or_max_keys,
                    AttnPlan* pl) {
  if (mode == MODE_GLOBAL) {
    if (B < 0 || Hkv < 1 || cap_or_max_keys < 1) return false;
    if ((long)B * Hkv * ceil_div(cap_or_max_keys, 32) < kStreamTiles) {
      if (!plan_chunked(MODE_GLOBAL, B, S, Hq, Hkv, D, cap_or_max_keys, pl)) return false;
      pl->fp8 = fp8 ? 1 : 0;
      return true;
    }
    mode = MODE_GSTREAM;
  }
  // A verify runs in chunked form (every chunk's loads in flight at once,
  // sixteen waves per 256 keys) unless its (request, KV head) units fill
  // the chip twice over with bf16 K/V: this kernel gives a verify's 32 rows
  // two waves per unit, one per 128-dim slice, each walking the unit's tiles
  // alone, and over fp8 it converts each load as it lands.  W=1024, 8 KV
  // heads x 256, S=4, this kernel against the chunked form: B=32 bf16 93 vs
  // 77 us, fp8 136 vs 60; B=64 bf16 107-117 vs 143, fp8 146 vs 115; B=128
  // bf16 203 vs 275, fp8 285 vs 218.  The chunked form's partials take
  // about 132 KB of workspace per unit.
  if (mode == MODE_VERIFY && B >= 0 && Hkv >= 1 && (fp8 || (long)B * Hkv < 2L * kNumCU)) {
    if (!plan_chunked(MODE_VERIFY, B, S, Hq, Hkv, D, cap_or_max_keys, pl)) return false;
    pl->fp8 = fp8 ? 1 : 0;
    return true;
  }
  if (B < 0 || S < 1 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || cap_or_max_keys < 1) return false;
  if (D != 64 && D != 128 && D != 256 && D != 512) return false;
  const int G = Hq / Hkv;
  const int rows = G * S;
  const bool dec = mode == MODE_DECODE || mode == MODE_DECODE_APPEND;
  if (dec) {
    if (S != 1 || G > 16) return false;
  } else {
    if (S > 8 || rows > 32) return false;
  }
  const int nct = rows > 16 ? 2 : 1;
  const Shape sh = pick_shape(mode, D, nct);
  if (sh.ds == 0) return false;
  pl->mode = mode;
  pl->chunked = 0;
  pl->D = D;
  pl->fp8 = fp8 ? 1 : 0;
  pl->ds = sh.ds;
  pl->nct = nct;
  pl->kw = sh.kw;
  pl->units = B * Hkv;
  pl->rows = rows;
  pl->threads = 64 * (D / sh.ds) * sh.kw;
  pl->max_tiles = ceil_div(cap_or_max_keys, 32) + (mode == MODE_VERIFY ? 1 : 0);

  // Split-K across workgroups only when the units alone do not fill the chip.
  int tps = pl->max_tiles;
  if (mode == MODE_GSTREAM) {
    // the split sizes come from the key counts, on the device (stream_split);
    // here only the grid: units * nsplit workgroups, nsplit >= 2
    tps = 1;
  } else if (pl->units > 0 && pl->units < kNumCU) {
    if (dec) {
      // The split count that puts the fewest tiles on the busiest CU: with
      // the splits spread evenly over the CUs, ceil(units * nsplit / CUs)
      // splits of ceil(max_tiles / nsplit) tiles; ties go to fewer splits
      // (less to combine), and a split keeps at least two tiles per wave.
      // Against a fixed target of two splits per CU, at W=1024 (32 tiles),
      // 8 KV heads x 256: B=12 24.8 -> 23.1 us, B=16 29.2 -> 28.7, B=20 39.0
      // -> 35.5, B=24 43.5 -> 41.2, B=28 47.4 -> 38.4 (unsplit: at 224 units
      // one round of whole units beats three splits per unit).  Counting two
      // workgroups per CU in this model, or letting a split go down to one
      // tile per wave, measured slower: B=12 23.1 -> 24.9 us, B=28 38.3 ->
      // 44.3, 56 units of one KV head 17.7 -> 18.3.
      long best = -1;
      for (int ns = 1; ns <= pl->max_tiles; ++ns) {
        const int t = ceil_div(pl->max_tiles, ns);
        if (ns > 1 && t < 2 * sh.kw) break;
        const long load = (long)ceil_div((long)pl->units * ceil_div(pl->max_tiles, t), kNumCU) * t;
        if (best < 0 || load < best) {
          best = load;
          tps = t;
        }
      }
    } else {
      tps = std::max(4, ceil_div((long)pl->max_tiles * pl->units, 4 * kNumCU));
    }
    tps = std::min(tps, pl->max_tiles);
  }
  pl->tiles_per_split = std::max(tps, 1);
  pl->nsplit = ceil_div(pl->max_tiles, pl->tiles_per_split);
  if (mode == MODE_GSTREAM)
    pl->nsplit = pl->units > 0 ? (int)ceil_div(std::max(kStreamWorkgroups, 2L * pl->units), pl->units) : 1;
  pl->ws_bytes =
      pl->nsplit > 1 ? (size_t)pl->units * pl->nsplit * rows * (size_t)(D + 2) * sizeof(float) + 256 : 0;

  size_t red = (D / sh.ds) > 1 ? (size_t)2 * sh.kw * (D / sh.ds) * (2 * nct * 4) * 64 * sizeof(float) : 0;
  size_t comb = sh.kw > 1 ? (size_t)sh.kw * rows * (2 + D + 4) * sizeof(float) : 0;
  pl->lds_bytes = std::max(red, comb);
  return true;
}

bool plan_global_append(int B, int S, int Hq, int Hkv, int D, int fp8, int max_keys, AttnPlan* pl) {
  if (B < 0 || S < 1 || Hkv < 1 || max_keys < S) return false;
  if ((long)B * Hkv * ceil_div(max_keys, 32) < kStreamTiles) {
    // the global chunked form: the chunk holding the tokens' slots takes them
    // from their buffers (over fp8, as the values of the codes to be stored)
    // and the merge stores them
    if (!plan_chunked(MODE_GLOBAL, B, S, Hq, Hkv, D, max_keys, pl)) return false;
    pl->fp8 = fp8 ? 1 : 0;
    return true;
  }
  return plan_attention(MODE_GLOBAL, B, S, Hq, Hkv, D, fp8, max_keys, pl);
}

hipError_t launch_attention(const AttnPlan& pl, const AttnParams& p, hipStream_t s) {
  if (pl.units == 0) return hipSuccess;
  if (pl.chunked) return launch_chunked(pl, p, s);
  hipError_t e;
  switch (pl.mode) {
    case MODE_DECODE: e = launch_mode<MODE_DECODE>(pl, p, s); break;
    case MODE_DECODE_APPEND: e = launch_mode<MODE_DECODE_APPEND>(pl, p, s); break;
    case MODE_VERIFY: e = launch_mode<MODE_VERIFY>(pl, p, s); break;
    case MODE_GSTREAM: e = launch_mode<MODE_GSTREAM>(pl, p, s); break;
    case MODE_GSTREAM_APPEND: e = launch_mode<MODE_GSTREAM_APPEND>(pl, p, s); break;
    default: return hipErrorInvalidValue;
  }
  if (e != hipSuccess || pl.nsplit == 1) return e;
  // a streamed global call: its splits, numbered from the key counts, merged
  // with each row's splits spread over thread groups
  if (pl.mode == MODE_GSTREAM || pl.mode == MODE_GSTREAM_APPEND) return launch_split_merge(pl, p, s);
  const long total = (long)pl.units * pl.rows * (pl.D / 4);
  const int blocks = ceil_div(total, 256);
  if (pl.mode == MODE_DECODE || pl.mode == MODE_DECODE_APPEND)
    hipLaunchKernelGGL(combine_kernel<MODE_DECODE>, dim3(blocks), dim3(256), 0, s, p, pl.D, pl.units);
  else
    hipLaunchKernelGGL(combine_kernel<MODE_VERIFY>, dim3(blocks), dim3(256), 0, s, p, pl.D, pl.units);
  return hipGetLastError();
}

}  // namespace swr
