// chunked.hip -- grouped attention in chunked form on gfx950: global layers,
// and sliding-layer verify when the batch is small.
//
// "Announcing Carat" (More FLOPs can be faster; Doing it all in one kernel
// can be slower): the G query heads that share a KV head, times the S
// proposed positions, form one group of rows; scores over the keys, a masked
// softmax and a weighted sum of values.  For a global layer the keys are the
// key_count = context + proposals keys of a contiguous region, the mask is
// causal by query position, and the key axis is padded to a multiple of 64
// with the tail masked; the page computes scores, softmax and the value
// product as separate matrix operations and stores the scores in between.
// For a sliding layer the keys are the ring's committed slots (in storage
// order, "Announcing Carat", ring buffer section) plus the S proposals, and
// the mask is the window by slot age.
//
// On MI355X a job of a few tens of MB (24.6 MB of K/V for a 6005-key global
// verify, 67 MB for a B=8 sliding verify) must be spread over most of the
// 256 CUs to stream at HBM speed, and each workgroup must put all of its
// loads in flight at once: a chain of dependent round trips per workgroup,
// not bandwidth, is what bounds a job this small.  So a block of keys (two
// of the page's 64-key pads) becomes the unit of work:
//   pass 1 (chunk_kernel): one workgroup per (request, KV head, 128 keys)
//     issues its K and Q loads on entry and its V loads as soon as the
//     scores are computed, and runs the three products of
//     the page on its chunk -- scores (bf16 MFMA, fp32), the masked softmax
//     over the chunk, and P x V (bf16 MFMA, fp32) -- with Q, the scores and
//     P kept in LDS, and writes the chunk's unnormalised rows with their
//     (max, sum).  In a verify call ring chunk 0 of each (request, KV head)
//     also takes the S proposals (read from their own buffers) as a step
//     of their own (up to 256 head dims ahead of its ring halves, while
//     their loads are in flight): a separate proposal workgroup would start
//     only when a ring chunk leaves its CU, a second round at the end of the
//     pass.
//   pass 2: merges the chunk partials, weights 2^(m_c - M), sums in a fixed
//     order, division by the weighted row sum.  With many chunks per row
//     (global) one workgroup per (request, KV head, row, quarter of the
//     head dims) splits the chunks over thread groups (merge_grouped); with
//     few (verify) one thread per four output dims takes every chunk
//     (merge_flat).
// The chunk length trades workgroups (CUs pulling K/V) against partial
// bytes (rows x D fp32 per chunk, written and read back): at 128 keys and
// 32 rows the partials are a quarter of the K/V bytes.  A merge done by the
// last-finishing workgroup of pass 1 instead would need a device-scope
// release fence per workgroup, which writes back the XCD's L2 and costs about
// as much as the kernel boundary it would save on this chip.
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

// Region keys a (request, KV head) attends to: the global key count, or the
// slots holding committed positions (verify: positions < pos0; a ring has
// W slots, a global region its own capacity and never wraps).
template <int MODE>
__device__ __forceinline__ int region_keys(const AttnParams& p, int b) {
  if (MODE == MODE_VERIFY) return max(min(p.pos[b], region_slots(p, b)), 0);
  return max(min(key_count_of(p, b), region_slots(p, b)), 0);
}

}  // namespace

// ------------------------------------------------------------------ pass 1

constexpr int kChunkKeys = 128;                 // keys per workgroup of pass 1 (global)
constexpr int kChunkWaves = kChunkKeys / 8;     // 16 waves: two per 16-key subtile
constexpr int kVerifyChunkKeys = 2 * kChunkKeys;  // verify ring chunks: two halves in turn

// Chunks of one (request, KV head) that pass 1 filled, a prefix of the
// launch's chunks: the region chunks up to the key count (verify: the ring
// chunks, chunk 0 holding the proposals).  A streamed global call (attn.hip)
// fills one partial per split, numbered by stream_split; merge_grouped
// finds a unit's run of them there.
template <int MODE>
__device__ __forceinline__ int valid_chunks(const AttnParams& p, int b) {
  const int ck = MODE == MODE_VERIFY ? kVerifyChunkKeys : kChunkKeys;
  const int n = (region_keys<MODE>(p, b) + ck - 1) / ck;
  return min(MODE == MODE_VERIFY ? max(n, 1) : n, p.nchunk);  // verify: chunk 0 holds the proposals
}

// One workgroup per (request, KV head, chunk), sixteen waves.  Every K and
// Q load of the workgroup is issued on entry (Q goes to LDS once), the V
// loads right after the score products (256 KB of K/V in all at D = 512),
// the K loads before the key count is read: addresses past the region are
// bounded by the buffer resource, and a chunk past the request's keys only
// leaves without using what it loaded.
//   scores   wave (kq, dh) = (w % 8, w / 8): the 16 keys of half kq%2 of
//            the chunk's 32-slot tile kq/2 (row r = key 8*(r/4) + 4*(kq%2)
//            + r%4 of the tile, as stored) over head-dim half dh, bf16 MFMA
//            into fp32; the two halves meet in LDS (in key order) and are
//            added in half order
//   softmax  16 lanes per row, eight keys per lane (rows spread over the
//            waves); masked, max and sum over the chunk by DPP within the
//            lanes' row, P rounded to bf16 into LDS; the row's (max, sum) go
//            to the workspace
//   values   waves w < PVW: O^T(dims w*DPW .. +DPW, rows) = V^T . P^T over
//            the chunk, bf16 MFMA into fp32; the unnormalised rows go to the
//            workspace for pass 2 with streaming stores.
// A verify ring chunk is 256 keys taken as two 128-key halves in turn (Q,
// then K of both on entry, V of both after the first half's scores), the softmax
// lanes carrying each row's running (max, sum) from one half to the next
// and the value waves rescaling their rows by the factor the softmax lanes
// leave in LDS: one partial per 256 keys, so pass 1 writes and pass 2 reads
// half as many.
// Masks: global -- key < key_count and key <= q_pos of the row's position;
// verify ring chunk -- a committed slot no older than W-2-i positions before
// pos0-1 for proposal i (position pos0+i sees positions >= pos0+i-W+1);
// verify proposal step -- proposal j <= i.  Over an fp8 ring the proposals
// are bf16 values: their scores take scale * log2(e) without k_scale, and
// their value product is multiplied by 1/v_scale in fp32, since pass 2
// multiplies every chunk by v_scale.
// Fused append (a global call storing its own S tokens at pos0 .. pos0+S-1):
// the chunk holding their slots takes them in place of the slots' old
// contents, and the merge pass stores them (below).
template <int D, int NCT>
struct ChunkSmem {
  float sbuf[2][16 * NCT][kChunkKeys + 4];
  __attribute__((aligned(16))) __bf16 pbuf[16 * NCT][kChunkKeys + 8];
  __attribute__((aligned(16))) __bf16 qbuf[16 * NCT][D + 8];
  float alpha[16 * NCT];  // verify: each row's rescale from one half to the next
};

// The call's own tokens, staged by the global chunk that holds their slots
// when a global call appends them itself (over an fp8 region the values its
// stored codes decode to, in units of the scale): dynamic LDS of [S][D] bf16
// for K, then V in the region's 8-slot block form, [2][D][8] bf16 -- the
// block holding key pos0 and the next, a token at slot (pos0 + j) % 8 of
// block (pos0 + j) / 8 - pos0 / 8 (S <= 8 tokens span at most two), so that
// a lane takes a key group's tokens with one 16-byte read per value tile.  A
// verify call stages its proposals as [2][S][D] bf16 (K, then V).  Sized at
// launch; none for the other calls.
extern __shared__ __attribute__((aligned(16))) __bf16 chunk_tokens[];
constexpr int kTokenBlocks = 2;  // 8-slot V blocks a global call's S <= 8 tokens span

// Piece t of a global call's tokens over an fp8 region: values 4t .. 4t+3
// of K's S*D values then V's ((token j, head dim d) at j*D + d), as bf16
// bits.
__device__ __forceinline__ u32x4 load_token_piece4(const AttnParams& p, int b, int g, int D, int t) {
  const int n = p.S * D, v = 4 * t;
  const bool is_v = v >= n;
  const int r = v - (is_v ? n : 0), j = r / D, d = r - j * D;
  const size_t src = ((size_t)(b * p.S + j) * p.Hkv + g) * D + (size_t)d;
  const u32x2 w = *reinterpret_cast<const u32x2*>((is_v ? p.v_prop : p.k_prop) + src);
  return u32x4{w[0], w[1], 0u, 0u};
}

// Writes piece t's values, as the region will hold them, to the staged
// tokens: K's token-major, V's into the 8-slot blocks.
__device__ __forceinline__ void stage_token_piece4(const AttnParams& p, __bf16* tok, int S, int D, int pos0, int t,
                                                   u32x4 bits) {
  const bool is_v = 4 * t >= S * D;
  const u32x2 vals = fp8_stored_values4(u32x2{bits[0], bits[1]}, is_v ? p.v_scale_store : p.k_scale_store);
  if (!is_v) {
    *reinterpret_cast<u32x2*>(&tok[4 * t]) = vals;
    return;
  }
  const int r = 4 * t - S * D, j = r / D, d = r - j * D;
  const int key = pos0 + j, bi = (key >> 3) - (pos0 >> 3), slot = key & 7;
  uint16_t* vb = reinterpret_cast<uint16_t*>(tok + S * D);
#pragma unroll
  for (int i = 0; i < 4; ++i) vb[(bi * D + d + i) * 8 + slot] = (uint16_t)(vals[i >> 1] >> (16 * (i & 1)));
}
// One chunk of one (request, KV head); every wave of the workgroup calls it
// with the same arguments.  Returns early (all waves alike) for a chunk past
// the request's keys; waves without value work return after the softmax.
// TOK (global calls that append their own tokens): the chunk holding the
// tokens' slots stages them; a kernel of its own, since the staging code,
// present but switched off, measured about 0.5 us slower on the calls that
// append nothing.
template <int D, int NCT, bool FP8, int MODE, bool TOK>
__device__ __forceinline__ void chunk_item(const AttnParams& p, ChunkSmem<D, NCT>& sm, int unit, int chunk) {
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
  constexpr int NH = MODE == MODE_VERIFY ? 2 : 1;    // 128-key halves per ring chunk (verify: 256 keys)
  constexpr int NS = MODE == MODE_VERIFY ? NH + 1 : NH;  // steps: the halves (verify: then the proposals)
  constexpr int ESZ = FP8 ? 1 : 2;
  constexpr bool KPAIR = FP8 && NCH % 2 == 0;        // 16-byte fp8 K loads (two k chunks)
  constexpr bool VPAIR = FP8 && NDT % 2 == 0;        // 16-byte fp8 V loads (two adjacent dims)
  constexpr int KPL = CK / 16;                       // keys per softmax lane
  static_assert(ROWS <= 4 * NW, "one softmax pass covers the rows");
  auto& sbuf = sm.sbuf;
  auto& pbuf = sm.pbuf;
  auto& qbuf = sm.qbuf;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int lr = lane & 15;
  const int lq = lane >> 4;
  const int Hkv = p.Hkv, G = p.G, S = p.S;
  const int b = unit / Hkv;
  const int g = unit - b * Hkv;
  // verify: ring chunk 0 of each (request, KV head) also takes the S
  // proposals, as a step of their own before its ring halves
  const bool with_prop = MODE == MODE_VERIFY && chunk == 0;
  const int k0 = chunk * CK * NH;  // region slot of key 0
  // one request per workgroup: its region offsets and slot count are
  // workgroup-uniform
  const int64_t k_off = wave_uniform(p.k_off[b]), v_off = wave_uniform(p.v_off[b]);
  const int cap_r = wave_uniform(region_slots(p, b));
  const int S_r = stored_slots(cap_r);  // slots stored per KV head (region layout: swr_device.h)
  const uint32_t region_bytes = (uint32_t)S_r * (uint32_t)(Hkv * D * ESZ);
  const __amdgpu_buffer_rsrc_t rk = make_rsrc(p.k_base + k_off, region_bytes);
  const __amdgpu_buffer_rsrc_t rv = make_rsrc(p.v_base + v_off, region_bytes);

  // Head dim (within the wave's half) of k element 8*lq + j of chunk c; with
  // paired fp8 loads a lane's 16 bytes cover two chunks (a fixed permutation
  // of the k axis, applied to Q and to bf16 proposal keys as well).
  auto kdim = [&](int c) { return KPAIR ? 64 * (c >> 1) + 16 * lq + 8 * (c & 1) : (4 * c + lq) * 8; };
  // Head dim of A row lr of value tile dt (paired fp8: tiles 2t, 2t+1 take
  // the even and odd dims of one 32-dim block).
  const int vw = wave < PVW ? wave : 0;
  auto vdim = [&](int dt) {
    return vw * DPW + (VPAIR ? 32 * (dt >> 1) + 2 * lr + (dt & 1) : 16 * dt + lr);
  };

  // ---------------------------------------------------------- loads
  // fp8 region codes land in kraw / vraw and become bf16 operands only where
  // the product needs them: a conversion next to its load would make the
  // wave wait for each load in turn (the compiler places it right there),
  // where the bf16 operands let all of them fly at once.
  const int kq = wave % KQ, dh = wave / KQ;
  // Operands of half h (keys k0 + 128h ..) of the chunk.
  bf16x8 kop[NS][NCH];
  bf16x8 vop[NS][KS][NDT];
  u32x4 kraw[NH][FP8 ? NCH : 1];  // paired: entries 0 .. NCH/2-1; else the low halves
  u32x4 vraw[NH][KS][FP8 ? NDT : 1];
  auto load_v = [&](int h) {
    if (wave >= PVW) return;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const uint32_t vblock = (uint32_t)(g * (S_r >> 3) + ((k0 + CK * h + 32 * ks) >> 3) + lq) * D;
      if (VPAIR) {
#pragma unroll
        for (int dt = 0; dt < NDT; dt += 2)
          vraw[h][ks][dt / 2] = load16_stream(rv, (vblock + (uint32_t)vdim(dt)) * 8);
      } else {
#pragma unroll
        for (int dt = 0; dt < NDT; ++dt) {
          const uint32_t off = (vblock + (uint32_t)vdim(dt)) * 8 * ESZ;
          if (FP8) {
            const u32x2 w = load8(rv, off);
            vraw[h][ks][dt] = u32x4{w[0], w[1], 0u, 0u};
          } else {
            vop[h][ks][dt] = as_bf16x8(load16_stream(rv, off));
          }
        }
      }
    }
  };
  auto cvt_v = [&](int h) {
    if constexpr (FP8) {
      if (wave >= PVW) return;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        if (VPAIR) {
#pragma unroll
          for (int dt = 0; dt < NDT; dt += 2) {
            vop[h][ks][dt] = fp8x8_to_bf16x8(u32x2{vraw[h][ks][dt / 2][0], vraw[h][ks][dt / 2][1]});
            vop[h][ks][dt + 1] = fp8x8_to_bf16x8(u32x2{vraw[h][ks][dt / 2][2], vraw[h][ks][dt / 2][3]});
          }
        } else {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            vop[h][ks][dt] = fp8x8_to_bf16x8(u32x2{vraw[h][ks][dt][0], vraw[h][ks][dt][1]});
        }
      }
    }
  };
  auto cvt_k = [&](int h) {
    if constexpr (FP8) {
      if (KPAIR) {
#pragma unroll
        for (int c = 0; c < NCH; c += 2) {
          kop[h][c] = fp8x8_to_bf16x8(u32x2{kraw[h][c / 2][0], kraw[h][c / 2][1]});
          kop[h][c + 1] = fp8x8_to_bf16x8(u32x2{kraw[h][c / 2][2], kraw[h][c / 2][3]});
        }
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) kop[h][c] = fp8x8_to_bf16x8(u32x2{kraw[h][c][0], kraw[h][c][1]});
      }
    }
  };
  // Q of the group's rows, once per workgroup, into LDS.  Rows past p.rows
  // take row 0's values: their scores are masked and their outputs never
  // stored, so any finite values do, and no select on the loaded data
  // (which the compiler places right after the load, holding every later
  // load of the wave behind a full round trip) is needed.  Q goes out ahead
  // of K (it does not wait for the region offsets): loads return in issue
  // order, so Q, and the staged tokens of a call that appends, reach LDS
  // while K is still in flight.  Verify: the first half's scores then wait
  // for that half's keys alone.  Global: issued after K, Q had made the LDS
  // writes wait for every K load (a 6005-key call that appends, in a graph:
  // 17.0 -> 16.5 us; the attention alone unchanged).
  constexpr int QPIECES = ROWS * D / 8;
  constexpr int QPT = (QPIECES + 64 * NW - 1) / (64 * NW);  // Q pieces per thread
  bf16x8 qv[QPT];
  auto load_q = [&] {
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int idx = threadIdx.x + k * 64 * NW;
      const int row = min(idx, QPIECES - 1) / (D / 8), d8 = (min(idx, QPIECES - 1) - row * (D / 8)) * 8;
      const int rr = row < p.rows ? row : 0;
      const int i = rr / G, hq = rr - (rr / G) * G;
      qv[k] = as_bf16x8(load16_global(p.q + ((size_t)(b * S + i) * p.Hq + g * G + hq) * D + d8));
    }
  };
  auto store_q = [&] {
#pragma unroll
    for (int k = 0; k < QPT; ++k) {
      const int idx = threadIdx.x + k * 64 * NW;
      if (idx < QPIECES) {
        const int row = idx / (D / 8), d8 = (idx - row * (D / 8)) * 8;
        *reinterpret_cast<bf16x8*>(&qbuf[row][d8]) = qv[k];
      }
    }
  };
  load_q();
  // global call that appends its own S tokens (keys pos0 .. pos0+S-1):
  // the chunk holding any of their slots stages them in LDS (bf16: one
  // 16-byte piece of K and of V per thread, S*D/8 <= 512 pieces; fp8: one
  // 4-value piece of K or V per thread, each value encoded and decoded, so
  // that the encodes spread over every wave of the workgroup), loaded after
  // Q and ahead of the region's loads (the load counter drains in order: the
  // staging then waits for Q and the tokens, not for K; the tokens wait for
  // their position, and Q issued behind them had waited too: 16.4 -> 16.2 us
  // for the 6005-key call in a graph) and written to LDS after the region's
  // loads have gone out; the Q barrier covers the writes.
  // V goes into the 8-slot block form (chunk_tokens), so that the value
  // operands take a key group's tokens with one 16-byte read and a mask per
  // tile: taken element by element, the 2-byte reads and their waits ran in
  // turn and cost the call about 1 us.  The operands take the tokens in
  // place of the slots' old contents, and the regions receive them from the
  // merge pass, after every chunk has read.  Over an fp8 region the staged
  // values are those of the codes the merge will store, exactly as a later
  // call reads them.
  // Verify: the proposal-carrying chunk stages the S proposals' K and V the
  // same way (bf16, as they arrive, also over an fp8 ring), and its
  // proposal step takes its operands from there.
  constexpr bool SUBP = MODE == MODE_GLOBAL && TOK;
  __bf16* const tok_k = chunk_tokens;
  __bf16* const tok_v = chunk_tokens + S * D;
  int pos0 = 0;
  bool tok_chunk = false, tok_piece = false;
  u32x4 tok_kbits = {0u, 0u, 0u, 0u}, tok_vbits = {0u, 0u, 0u, 0u};
  if constexpr (SUBP) {
    if (p.append) {
      pos0 = p.pos[b];
      tok_chunk = pos0 < k0 + CK && pos0 + S > k0;  // uniform over the workgroup
      if (FP8) {
        tok_piece = tok_chunk && (int)threadIdx.x < 2 * S * (D / 4);
        if (tok_piece) tok_kbits = load_token_piece4(p, b, g, D, threadIdx.x);
      } else {
        tok_piece = tok_chunk && (int)threadIdx.x < S * (D / 8);
        if (tok_piece) {
          const int j = threadIdx.x / (D / 8), d8 = threadIdx.x - j * (D / 8);
          const size_t src = ((size_t)(b * S + j) * Hkv + g) * D + (size_t)d8 * 8;
          tok_kbits = load16_global(p.k_prop + src);
          tok_vbits = load16_global(p.v_prop + src);
        }
      }
    }
  }
  if constexpr (MODE == MODE_VERIFY) {
    tok_piece = with_prop && (int)threadIdx.x < S * (D / 8);
    if (tok_piece) {
      const int j = threadIdx.x / (D / 8), d8 = threadIdx.x - j * (D / 8);
      const size_t src = ((size_t)(b * S + j) * Hkv + g) * D + (size_t)d8 * 8;
      tok_kbits = load16_global(p.k_prop + src);
      tok_vbits = load16_global(p.v_prop + src);
    }
  }
  {  // K of every half
#pragma unroll
    for (int h = 0; h < NH; ++h) {
      // row lr of half kq%2 of tile kq/2; granule (dh*DH + kdim(c)) / R of it
      constexpr int R = FP8 ? 16 : 8;
      const uint32_t hb = k_half_base(g, S_r, k0 + CK * h + 32 * (kq >> 1), kq & 1, D, ESZ);
      if (KPAIR) {
#pragma unroll
        for (int c = 0; c < NCH; c += 2)
          kraw[h][c / 2] = load16_stream(rk, hb + k_granule_offset((dh * DH + kdim(c)) / R, lr));
      } else {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
          const int dim = dh * DH + kdim(c);
          const uint32_t off = hb + k_granule_offset(dim / R, lr) + (uint32_t)((dim % R) * ESZ);
          if (FP8) {
            const u32x2 w = load8(rk, off);
            kraw[h][c] = u32x4{w[0], w[1], 0u, 0u};
          } else {
            kop[h][c] = as_bf16x8(load16_stream(rk, off));
          }
        }
      }
    }
  }
  store_q();
  if constexpr (SUBP) {
    if (FP8) {
      // piece t: values 4t .. 4t+3 of K's S*D then V's (token j = 4t/D of
      // K or V); a K piece lands at tok_k[4t], a V piece in the V blocks
      if (tok_piece) stage_token_piece4(p, chunk_tokens, S, D, pos0, threadIdx.x, tok_kbits);
      for (int t = threadIdx.x + 64 * NW; tok_chunk && t < 2 * S * (D / 4); t += 64 * NW)
        stage_token_piece4(p, chunk_tokens, S, D, pos0, t, load_token_piece4(p, b, g, D, t));
    } else if (tok_piece) {  // the thread's piece: token j, head dims 8*d8 .. +7
      *reinterpret_cast<u32x4*>(&tok_k[threadIdx.x * 8]) = tok_kbits;
      const int j = threadIdx.x / (D / 8), d8 = threadIdx.x - j * (D / 8);
      const int key = pos0 + j, bi = (key >> 3) - (pos0 >> 3), slot = key & 7;
      uint16_t* vb = reinterpret_cast<uint16_t*>(tok_v);
#pragma unroll
      for (int i = 0; i < 8; ++i)
        vb[(bi * D + d8 * 8 + i) * 8 + slot] = (uint16_t)(tok_vbits[i >> 1] >> (16 * (i & 1)));
    }
  }
  if constexpr (MODE == MODE_VERIFY) {
    if (tok_piece) {  // proposal j, head dims 8*d8 .. +7
      *reinterpret_cast<u32x4*>(&tok_k[threadIdx.x * 8]) = tok_kbits;
      *reinterpret_cast<u32x4*>(&tok_v[threadIdx.x * 8]) = tok_vbits;
    }
  }
  // softmax role: slot wave*4 + lane/16 takes row `srow` (slots past the
  // rows idle), keys KPL*(lane%16) .. of the chunk; a global row's query
  // position is fetched with the loads
  const int srow = wave * 4 + lq;
  const bool srow_ok = srow < p.rows;
  const int si = (srow_ok ? srow : 0) / G;  // proposal index of the row
  const int qp = MODE == MODE_GLOBAL ? qpos_of(p, b, si) : 0;

  const int n_keys = region_keys<MODE>(p, b);
  if (!with_prop && k0 >= n_keys) return;  // past this request's keys (uniform over the workgroup)

  // ---------------------------------------------------------- scores
  __syncthreads();  // Q (and the staged proposals) in LDS
  const size_t slot = ((size_t)unit * p.nchunk + chunk) * p.rows;
  // verify: slot age of the newest committed position, and the oldest age
  // row i still sees
  const int ring_head = (MODE == MODE_VERIFY && p.pos[b] > 0) ? (p.pos[b] - 1) % p.cap : 0;
  const int age_lim = p.cap - 2 - si;
  // halves this chunk computes: a half wholly past the key count adds
  // nothing (uniform over the workgroup; verify's proposal-carrying chunk
  // can have none)
  const int nh = k0 >= n_keys ? 0 : (k0 + CK >= n_keys ? 1 : NH);
  float m_run = -INFINITY, l_run = 0.f;  // softmax lanes: the row's running (max, sum)
  f32x4 o[NCT][NDT];                     // value lanes: rows ct*16 + lr, unnormalised
#pragma unroll
  for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
    for (int dt = 0; dt < NDT; ++dt) o[ct][dt] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Verify: the proposals' step (h = NH), keys 0 .. S-1 of the step, bf16
  // values over any ring (over an fp8 ring their scores take scale *
  // log2(e) without k_scale, and their value product is multiplied by
  // 1/v_scale in fp32, since the merge multiplies by v_scale).  Up to 256
  // head dims it comes first: its operands are in LDS already, so it needs
  // no K of the ring's and runs while the last waves' K loads are still in
  // flight.  At 512 dims the ring's K registers in flight leave it no room,
  // and it comes after the ring halves.
  constexpr bool PROP_FIRST = MODE == MODE_VERIFY && D <= 256;
#pragma unroll
  for (int step = 0; step < NS; ++step) {
    const int h = PROP_FIRST ? (step == 0 ? NH : step - 1) : step;
    const bool ph = MODE == MODE_VERIFY && h == NH;
    if (ph ? !with_prop : h >= nh) continue;
    const int kh = k0 + CK * h;  // region slot of the half's key 0
    const float qs = (FP8 && ph) ? p.qk_scale_prop : p.qk_scale;
    if (ph) {
      // row lr of subtile kq is key 32*(kq/2) + 8*(lr/4) + 4*(kq%2) + lr%4
      // (so proposals j < 8 land in subtiles 0 and 1); rows past S are zero
      const int pj = 32 * (kq >> 1) + 8 * (lr >> 2) + 4 * (kq & 1) + (lr & 3);
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        kop[h][c] = pj < S ? *reinterpret_cast<const bf16x8*>(&tok_k[pj * D + dh * DH + kdim(c)]) : bf16x8{};
    } else {
      cvt_k(h);
    }
    if constexpr (SUBP) {
      if (tok_chunk) {  // this lane's K row is token j of the call
        const int j = kh + 32 * (kq >> 1) + 8 * (lr >> 2) + 4 * (kq & 1) + (lr & 3) - pos0;
        if (j >= 0 && j < S) {
#pragma unroll
          for (int c = 0; c < NCH; ++c)
            kop[h][c] = *reinterpret_cast<const bf16x8*>(&tok_k[j * D + dh * DH + kdim(c)]);
        }
      }
    }
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct) {
      // the proposals (S <= 8) are keys of subtiles 0 and 1 only: the other
      // waves' scores would be masked, and their part of sbuf is not read
      // unmasked, so they skip the product
      if (ph && kq >= 2) continue;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int c = 0; c < NCH; ++c)
        acc = mfma16x16x32(kop[h][c], *reinterpret_cast<const bf16x8*>(&qbuf[ct * 16 + lr][dh * DH + kdim(c)]), acc);
      // C rows 4*lq + r are keys 8*lq + 4*(kq%2) + r of tile kq/2
      *reinterpret_cast<f32x4*>(&sbuf[dh][ct * 16 + lr][32 * (kq >> 1) + 8 * lq + 4 * (kq & 1)]) = acc;
    }
    // V loads (every half's) go out once the first half's scores are
    // computed rather than on entry: a smaller first burst of requests
    // across all workgroups streams faster, and the value loads still
    // overlap the softmax.
    if (h == 0) {
#pragma unroll
      for (int hh = 0; hh < NH; ++hh)
        if (hh < nh) load_v(hh);
    }
    __syncthreads();

    // -------------------------------------------------------- softmax
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
          const int j = kk + e4 + e;  // key of the half
          bool vis;
          if (MODE == MODE_GLOBAL) {
            vis = kh + j < n_keys && kh + j <= qp;
          } else if (ph) {
            vis = j < S && j <= si;
          } else {
            int age = ring_head - (kh + j);
            if (age < 0) age += p.cap;
            vis = kh + j < n_keys && age <= age_lim;
          }
          vis = vis && srow_ok;
          sv[e4 + e] = vis ? (s0[e] + s1[e]) * qs : -INFINITY;
          mx = fmaxf(mx, sv[e4 + e]);
        }
      }
      const float m_new = fmaxf(m_run, max16lanes(mx));
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = fast_exp2(m_run - m_use);  // 0 on the first half
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
      l_run = l_run * alpha + sum16lanes(ps);
      m_run = m_new;
      if (NS > 1 && lr == 0) sm.alpha[srow] = alpha;
    }
    __syncthreads();

    // --------------------------------------------------------- values
    if (wave < PVW) {
      if (ph) {
        // k step 0, lane group 0 holds keys 0..7: proposal j at element j
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) vop[h][ks][dt] = bf16x8{};
        if (lq == 0) {
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) {
            bf16x8 v;
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = j < S ? tok_v[j * D + vdim(dt)] : (__bf16)0.f;
            vop[h][0][dt] = v;
          }
        }
      } else {
        cvt_v(h);
      }
      if constexpr (SUBP) {
        if (tok_chunk) {  // values of the call's own tokens
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            // lane group lq's keys are the 8-slot block starting at `base`;
            // m: its slots that hold the call's tokens
            const int base = kh + 32 * ks + 8 * lq;
            u32x4 m;
#pragma unroll
            for (int e2 = 0; e2 < 4; ++e2) {
              const unsigned j0 = (unsigned)(base + 2 * e2 - pos0);
              m[e2] = (j0 < (unsigned)S ? 0x0000FFFFu : 0u) | (j0 + 1u < (unsigned)S ? 0xFFFF0000u : 0u);
            }
            if ((m[0] | m[1] | m[2] | m[3]) != 0u) {
              const int bi = (base >> 3) - (pos0 >> 3);
#pragma unroll
              for (int dt = 0; dt < NDT; ++dt) {
                const u32x4 w = *reinterpret_cast<const u32x4*>(&tok_v[(bi * D + vdim(dt)) * 8]);
                vop[h][ks][dt] = __builtin_bit_cast(bf16x8, (__builtin_bit_cast(u32x4, vop[h][ks][dt]) & ~m) | (w & m));
              }
            }
          }
        }
      }
      if (!ph && kh + CK > n_keys) {  // last half: zero values of keys past the count
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          u32x4 keep;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int kk = kh + 32 * ks + 8 * lq + 2 * j;
            keep[j] = (kk < n_keys ? 0x0000FFFFu : 0u) | (kk + 1 < n_keys ? 0xFFFF0000u : 0u);
          }
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            vop[h][ks][dt] = __builtin_bit_cast(bf16x8, __builtin_bit_cast(u32x4, vop[h][ks][dt]) & keep);
        }
      }
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        if (NS > 1 && step > 0) {  // rescale to the running maximum of the row
          const float a = sm.alpha[ct * 16 + lr];
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[ct][dt] *= a;
        }
        if (FP8 && ph) {
          // over an fp8 ring the rows hold values in units of v_scale: the
          // proposals' product (bf16 values, P as for any key; zero past
          // key 31) is taken on its own and scaled by 1/v_scale in fp32, so
          // that a row seeing one proposal alone returns its value exactly
          const bf16x8 pt = *reinterpret_cast<const bf16x8*>(&pbuf[ct * 16 + lr][8 * lq]);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt)
            o[ct][dt] += mfma16x16x32(vop[h][0][dt], pt, f32x4{0.f, 0.f, 0.f, 0.f}) * p.inv_v_scale;
          continue;
        }
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (ph && ks > 0) continue;  // the proposals' P is zero past key 31
          const bf16x8 pt = *reinterpret_cast<const bf16x8*>(&pbuf[ct * 16 + lr][32 * ks + 8 * lq]);
#pragma unroll
          for (int dt = 0; dt < NDT; ++dt) o[ct][dt] = mfma16x16x32(vop[h][ks][dt], pt, o[ct][dt]);
        }
      }
    }
  }

  // ----------------------------------------------------------- partials
  if (srow < ROWS && lr == 0 && srow_ok) {
    p.ws_pml[(slot + srow) * 2 + 0] = m_run;
    p.ws_pml[(slot + srow) * 2 + 1] = l_run;
  }
  if (wave >= PVW) return;
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

// Global: workgroup j takes chunk j % nchunk of unit j / nchunk.  Verify:
// when the units are a multiple of the 8 XCDs (workgroup j runs on XCD
// j % 8), all ring chunks of a unit go to one XCD, whose L2 then serves the
// unit's Q to all of them after one read.
// Up to 256 head dims two global workgroups stay resident per CU (eight
// waves per SIMD, 64 registers a lane); 512 dims, and verify with its two
// halves' operands, need more registers and keep one.
template <int D, int NCT, bool FP8, int MODE, bool TOK>
__global__ void __launch_bounds__(64 * kChunkWaves)
__attribute__((amdgpu_waves_per_eu(D <= 256 && MODE != MODE_VERIFY ? 8 : 4))) chunk_kernel(const AttnParams p) {
  __shared__ ChunkSmem<D, NCT> sm;
  if (MODE == MODE_VERIFY) {
    const int nring = p.nchunk;
    int unit, rc;
    if ((p.B * p.Hkv) % 8 == 0) {
      const int x = blockIdx.x & 7, sl = blockIdx.x >> 3;
      unit = x + 8 * (sl / nring);
      rc = sl - (sl / nring) * nring;
    } else {
      unit = blockIdx.x / nring;
      rc = blockIdx.x - unit * nring;
    }
    chunk_item<D, NCT, FP8, MODE, TOK>(p, sm, unit, rc);
  } else {
    const int unit = blockIdx.x / p.nchunk;
    chunk_item<D, NCT, FP8, MODE, TOK>(p, sm, unit, blockIdx.x - unit * p.nchunk);
  }
}

// ------------------------------------------------------------------ pass 2

// Both merges read every chunk's (max, sum, row) loads of a batch together,
// issued before the request's chunk count is known (chunks past it but
// inside the launch's chunk count are dropped by select, never multiplied,
// so whatever they hold cannot leak in), and keep a running (M, L, O)
// rescaled between batches.
// out = v_scale * sum_c 2^(m_c - M) acc_c / sum_c 2^(m_c - M) l_c.
constexpr int kMergeThreads = 256;
constexpr int kMergeBatch = 16;
constexpr int kMaxChunks = 513;  // 65536 region keys (+ a proposal chunk)

// A global call that appended its own tokens: token j goes into slot
// pos0 + j of its region (dropped past the region, as by the append call).
// Done by the merge pass, once every chunk has read: the token's bits are
// loaded before the merge's own loads and stored after them, so the stores
// add no round trip of their own.  bf16 regions take 8-dim pieces
// (CallToken); fp8 regions one E4M3 code per thread (CallTokenCode).
struct CallToken {
  u32x4 k, v;
  int j = -1, d8 = 0;
};

__device__ __forceinline__ CallToken load_call_token(const AttnParams& p, int D, int b, int g, int j, int d8) {
  CallToken t;
  const size_t src = ((size_t)(b * p.S + j) * p.Hkv + g) * D + (size_t)d8 * 8;
  t.k = *reinterpret_cast<const u32x4*>(p.k_prop + src);
  t.v = *reinterpret_cast<const u32x4*>(p.v_prop + src);
  t.j = j;
  t.d8 = d8;
  return t;
}

// Region of request b for a token store.  UNIFORM: b is the same in every
// lane of the wave (merge_grouped: one request per workgroup), so the
// resource goes to scalar registers; merge_flat's waves can span two
// requests and keep the compiler's per-resource loop.
template <bool UNIFORM>
struct TokenRegion {
  __amdgpu_buffer_rsrc_t rk, rv;
  int cap_r, S_r;
  __device__ __forceinline__ TokenRegion(const AttnParams& p, int D, int b, int esize) {
    int64_t ko = p.k_off[b], vo = p.v_off[b];
    cap_r = region_slots(p, b);
    if (UNIFORM) {
      ko = wave_uniform(ko);
      vo = wave_uniform(vo);
      cap_r = wave_uniform(cap_r);
    }
    S_r = stored_slots(cap_r);
    const uint32_t region_bytes = (uint32_t)S_r * (uint32_t)(p.Hkv * D * esize);
    rk = make_rsrc(p.k_base + ko, region_bytes);
    rv = make_rsrc(p.v_base + vo, region_bytes);
  }
};

template <bool UNIFORM>
__device__ __forceinline__ void store_call_token(const AttnParams& p, int D, int b, int g, const CallToken& t) {
  const TokenRegion<UNIFORM> r(p, D, b, 2);
  const int slot = p.pos[b] + t.j;
  if (t.j < 0 || slot < 0 || slot >= r.cap_r) return;
  const int S_r = r.S_r;
  const __amdgpu_buffer_rsrc_t rk = r.rk, rv = r.rv;
  store_token_piece<false>(rk, rv, slot, g, S_r, D, t.d8, t.k, t.v, p.k_scale_store, p.v_scale_store);
}

// fp8 regions: the call's token values are encoded one per thread, spread
// over the unit's row workgroups of each quarter (2*S*PART values of the
// quarter's dims, `per` to a row); an encode is too long a chain to leave
// all of them to the row-0 threads.
struct CallTokenCode {
  uint16_t bits = 0;
  int j = -1, d = 0;
  bool is_v = false;
};

__device__ __forceinline__ CallTokenCode load_call_token_code(const AttnParams& p, int D, int part, int quarter, int b,
                                                              int g, int v) {
  CallTokenCode t;
  const int n = p.S * part;  // values of one of K, V in the quarter
  t.is_v = v >= n;
  const int r = v - (t.is_v ? n : 0);
  t.j = r / part;
  t.d = quarter * part + (r - t.j * part);
  const size_t src = ((size_t)(b * p.S + t.j) * p.Hkv + g) * D + (size_t)t.d;
  t.bits = (t.is_v ? p.v_prop : p.k_prop)[src];
  return t;
}

template <bool UNIFORM>
__device__ __forceinline__ void store_call_token_code(const AttnParams& p, int D, int b, int g, const CallTokenCode& t) {
  const TokenRegion<UNIFORM> r(p, D, b, 1);
  const int slot = p.pos[b] + t.j;
  if (t.j < 0 || slot < 0 || slot >= r.cap_r) return;
  const int S_r = r.S_r;
  const __amdgpu_buffer_rsrc_t rk = r.rk, rv = r.rv;
  const uint8_t code = e4m3_encode(__builtin_bit_cast(float, (uint32_t)t.bits << 16),
                                   t.is_v ? p.v_scale_store : p.k_scale_store);
  store_token_code(rk, rv, slot, g, S_r, D, t.d, t.is_v, code);
}

struct RunningRow {
  float M = -INFINITY, L = 0.f;
  f32x4 O = {0.f, 0.f, 0.f, 0.f};
};

// Adds chunks c = c0 + j*step (j < kMergeBatch, c < nvalid) of the row at
// `slot0` (+ c*rows), four dims at `d`; `navail` (>= 1) partials are stored
// for the row.  On the first batch the request's chunk count is read (the
// chunked form; a streamed call's count is known), and `issued` runs, after
// the batch's loads are issued: work that waits only for earlier loads then
// overlaps them.  CLAMP: indices past the stored partials read the last one
// again (their values dropped by the selects below), so the batch's loads go
// out with no branch between them; with a branch per partial the compiler
// copied a loaded register inside one and waited there for the loads so far,
// a round trip in the middle of the batch (6005-key global verify 15.5 ->
// 15.3 us).  Where a row has only a few partials (the sliding verify's four)
// the repeated loads cost more than that (21.4 -> 22.3 us) and each partial
// keeps its branch.
template <int MODE, bool CLAMP, typename F>
__device__ __forceinline__ void merge_batch(const AttnParams& p, int D, int b, size_t slot0, int d, int c0,
                                            int step, int navail, bool first, int& nvalid, RunningRow& r,
                                            F&& issued) {
  float m[kMergeBatch], l[kMergeBatch];
  f32x4 a[kMergeBatch];
#pragma unroll
  for (int j = 0; j < kMergeBatch; ++j) {
    if (CLAMP) {
      const size_t at = slot0 + (size_t)min(c0 + j * step, navail - 1) * p.rows;
      m[j] = p.ws_pml[at * 2];
      l[j] = p.ws_pml[at * 2 + 1];
      a[j] = *reinterpret_cast<const f32x4*>(p.ws_part + at * D + d);
    } else {
      m[j] = -INFINITY;
      l[j] = 0.f;
      a[j] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (c0 + j * step < navail) {  // past the stored partials: no load at all
        const size_t at = slot0 + (size_t)(c0 + j * step) * p.rows;
        m[j] = p.ws_pml[at * 2];
        l[j] = p.ws_pml[at * 2 + 1];
        a[j] = *reinterpret_cast<const f32x4*>(p.ws_part + at * D + d);
      }
    }
  }
  if (first) {
    if (MODE != MODE_GSTREAM) nvalid = valid_chunks<MODE>(p, b);
    issued();
  }
  float mb = r.M;
#pragma unroll
  for (int j = 0; j < kMergeBatch; ++j) mb = (c0 + j * step < nvalid) ? fmaxf(mb, m[j]) : mb;
  const float m_use = (mb == -INFINITY) ? 0.f : mb;
  const float alpha = fast_exp2(r.M - m_use);  // 0 while nothing was merged
  r.L *= alpha;
  r.O *= alpha;
#pragma unroll
  for (int j = 0; j < kMergeBatch; ++j) {
    const bool ok = c0 + j * step < nvalid;
    const float w = fast_exp2(m[j] - m_use);
    r.L += ok ? l[j] * w : 0.f;
    r.O += ok ? a[j] * w : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  r.M = mb;
}

__device__ __forceinline__ void store_row4(const AttnParams& p, int D, int b, int g, int row, int d, float L,
                                           f32x4 O) {
  const float inv = L > 0.f ? p.v_scale / L : 0.f;
  const int i = row / p.G, h = row - (row / p.G) * p.G;
  bf16x4 w = {(__bf16)(O[0] * inv), (__bf16)(O[1] * inv), (__bf16)(O[2] * inv), (__bf16)(O[3] * inv)};
  *reinterpret_cast<bf16x4*>(p.out + ((size_t)(b * p.S + i) * p.Hq + g * p.G + h) * D + d) = w;
}

// Many chunks per row: one workgroup per (request, KV head, row, quarter of
// the head dims); thread group k of NG takes chunks k, k+NG, ... for its
// four dims, and the groups are merged in group order through LDS.
// FP8: the call's tokens (if it appended them) go into fp8 regions.
template <int D, int MODE, bool FP8 = false>
__global__ void __launch_bounds__(kMergeThreads) merge_grouped(const AttnParams p) {
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
  const int d = quarter * PART + (tid - grp * TPG) * 4;
  // the row's partials: the chunked form stores nchunk per unit; a streamed
  // call's unit has n splits from its first one on (stream_split)
  size_t slot0 = (size_t)unit * p.nchunk * p.rows + row;
  int navail = p.nchunk;
  if constexpr (MODE == MODE_GSTREAM) {
    const StreamSplit x = stream_split(p, 0, unit);
    slot0 = (size_t)x.first * p.rows + row;
    navail = x.n;
  }

  // the call's tokens, this quarter's dims: bf16 as 8-dim pieces in the
  // row-0 workgroup; fp8 one value per thread, `per` values to a row
  CallToken tok;
  CallTokenCode tcode;
  const int tok_values = 2 * p.S * PART;
  const int per = (tok_values + p.rows - 1) / p.rows;
  if (MODE == MODE_GLOBAL && p.append) {
    if constexpr (FP8) {
      if (tid < per && row * per + tid < tok_values) tcode = load_call_token_code(p, D, PART, quarter, b, g, row * per + tid);
    } else if (row == 0 && tid < p.S * (PART / 8)) {
      tok = load_call_token(p, D, b, g, tid / (PART / 8), quarter * (PART / 8) + tid % (PART / 8));
    }
  }
  bool tokens_stored = false;
  auto store_tokens = [&] {
    if (MODE == MODE_GLOBAL && p.append && !tokens_stored) {
      if constexpr (FP8)
        store_call_token_code<true>(p, D, b, g, tcode);
      else
        store_call_token<true>(p, D, b, g, tok);
    }
    tokens_stored = true;
  };
  RunningRow r;
  int nvalid = navail;
  for (int c0 = grp; c0 < nvalid; c0 += kMergeBatch * NG) {
    // the tokens' stores go out once the first batch's loads are in flight
    merge_batch<MODE, true>(p, D, b, slot0, d, c0, NG, navail, c0 == grp, nvalid, r, [&] { store_tokens(); });
  }
  store_tokens();  // a group with no chunk to merge
  if constexpr (FP8) {  // rows * kMergeThreads < tok_values: the rest in turn
    if (MODE == MODE_GLOBAL && p.append)
      for (int k = tid + kMergeThreads; k < per; k += kMergeThreads)
        if (row * per + k < tok_values)
          store_call_token_code<true>(p, D, b, g, load_call_token_code(p, D, PART, quarter, b, g, row * per + k));
  }
  if (tid - grp * TPG == 0) {
    gml[grp][0] = r.M;
    gml[grp][1] = r.L;
  }
  *reinterpret_cast<f32x4*>(&obuf[grp][d - quarter * PART]) = r.O;
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
    Ot += *reinterpret_cast<const f32x4*>(&obuf[k][d - quarter * PART]) * w;
  }
  store_row4(p, D, b, g, row, d, Lt, Ot);
}

// Few chunks per row: one thread per (request, KV head, row, four dims)
// takes every chunk in order.
template <int MODE, bool FP8 = false>
__global__ void __launch_bounds__(kMergeThreads) merge_flat(const AttnParams p, int D) {
  const int per_row = D / 4;
  const int per_unit = p.rows * per_row;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= p.B * p.Hkv * per_unit) return;
  const int unit = idx / per_unit;
  const int rem = idx - unit * per_unit;
  const int row = rem / per_row;
  const int d = (rem - row * per_row) * 4;
  const int b = unit / p.Hkv, g = unit - (unit / p.Hkv) * p.Hkv;
  const size_t slot0 = (size_t)unit * p.nchunk * p.rows + row;

  // the call's tokens: bf16, thread d/8 of row 0 (of each unit) takes head
  // dims d .. d+7 of every token, one token per loop; fp8, the unit's
  // threads take the 2*S*D values in turn, one per thread at a time
  RunningRow r;
  int nvalid = p.nchunk;
  for (int c0 = 0; c0 < nvalid; c0 += kMergeBatch) {
    merge_batch<MODE, false>(p, D, b, slot0, d, c0, 1, p.nchunk, c0 == 0, nvalid, r, [] {});
  }
  if (MODE == MODE_GLOBAL && p.append) {
    if constexpr (FP8) {
      for (int v = rem; v < 2 * p.S * D; v += per_unit)
        store_call_token_code<false>(p, D, b, g, load_call_token_code(p, D, D, 0, b, g, v));
    } else if (row == 0 && d % 8 == 0) {
      for (int j = 0; j < p.S; ++j) store_call_token<false>(p, D, b, g, load_call_token(p, D, b, g, j, d / 8));
    }
  }
  store_row4(p, D, b, g, row, d, r.L, r.O);
}

// A streamed global call with few splits per unit: one thread per four
// output dims of one row takes every split of its unit in order (kMergeBatch
// loads at a time), one unit per workgroup (`chunks` workgroups each), so
// that the split numbering (stream_split) is workgroup-uniform.
__global__ void __launch_bounds__(kMergeThreads) merge_stream_flat(const AttnParams p, int D, int chunks) {
  const int unit = blockIdx.x / chunks;
  const int local = (blockIdx.x - unit * chunks) * kMergeThreads + threadIdx.x;
  const StreamSplit x = stream_split(p, 0, unit);  // every lane takes part
  const int per_row = D / 4;
  if (local >= p.rows * per_row) return;
  const int row = local / per_row;
  const int d = (local - row * per_row) * 4;
  const int b = unit / p.Hkv, g = unit - (unit / p.Hkv) * p.Hkv;
  const size_t slot0 = (size_t)x.first * p.rows + row;
  RunningRow r;
  int nvalid = x.n;
  for (int c0 = 0; c0 < nvalid; c0 += kMergeBatch)
    merge_batch<MODE_GSTREAM, true>(p, D, b, slot0, d, c0, 1, x.n, c0 == 0, nvalid, r, [] {});
  store_row4(p, D, b, g, row, d, r.L, r.O);
}

// ------------------------------------------------------------------ host

namespace {

int cdiv(long a, long b) { return (int)((a + b - 1) / b); }
size_t align256(size_t x) { return (x + 255) / 256 * 256; }

template <int D, int NCT, bool FP8, int MODE>
void launch_chunk_kernel(bool tok, dim3 grid, dim3 block, size_t lds, hipStream_t s, const AttnParams& p) {
  if constexpr (MODE == MODE_GLOBAL) {
    if (tok) {
      hipLaunchKernelGGL((chunk_kernel<D, NCT, FP8, MODE, true>), grid, block, lds, s, p);
      return;
    }
  }
  hipLaunchKernelGGL((chunk_kernel<D, NCT, FP8, MODE, false>), grid, block, lds, s, p);
}

template <int D, int NCT, int MODE>
hipError_t launch_chunks(const AttnPlan& pl, const AttnParams& p, hipStream_t s) {
  const dim3 grid(pl.units * pl.nchunk), block(64 * kChunkWaves);
  const size_t tok_bytes = MODE == MODE_VERIFY ? (size_t)2 * p.S * D * sizeof(uint16_t)
                           : (MODE == MODE_GLOBAL && p.append)
                               ? ((size_t)p.S * D + (size_t)kTokenBlocks * D * 8) * sizeof(uint16_t)
                               : 0;
  const bool tok = MODE == MODE_GLOBAL && p.append;
  if (pl.fp8)
    launch_chunk_kernel<D, NCT, true, MODE>(tok, grid, block, tok_bytes, s, p);
  else
    launch_chunk_kernel<D, NCT, false, MODE>(tok, grid, block, tok_bytes, s, p);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const bool fp8_tokens = MODE == MODE_GLOBAL && p.append && pl.fp8;  // the merge stores codes
  const dim3 mgrid(pl.units * pl.rows * 4), fgrid(cdiv((long)pl.units * pl.rows * (D / 4), kMergeThreads));
  if (pl.nchunk > kMergeBatch) {
    if (fp8_tokens)
      hipLaunchKernelGGL((merge_grouped<D, MODE, true>), mgrid, dim3(kMergeThreads), 0, s, p);
    else
      hipLaunchKernelGGL((merge_grouped<D, MODE>), mgrid, dim3(kMergeThreads), 0, s, p);
  } else {
    if (fp8_tokens)
      hipLaunchKernelGGL((merge_flat<MODE, true>), fgrid, dim3(kMergeThreads), 0, s, p, D);
    else
      hipLaunchKernelGGL((merge_flat<MODE>), fgrid, dim3(kMergeThreads), 0, s, p, D);
  }
  return hipGetLastError();
}

template <int MODE>
hipError_t launch_chunks_mode(const AttnPlan& pl, const AttnParams& p, hipStream_t s) {
  const bool two = pl.nct == 2;
  switch (pl.D) {
    case 64: return two ? launch_chunks<64, 2, MODE>(pl, p, s) : launch_chunks<64, 1, MODE>(pl, p, s);
    case 128: return two ? launch_chunks<128, 2, MODE>(pl, p, s) : launch_chunks<128, 1, MODE>(pl, p, s);
    case 256: return two ? launch_chunks<256, 2, MODE>(pl, p, s) : launch_chunks<256, 1, MODE>(pl, p, s);
    case 512: return two ? launch_chunks<512, 2, MODE>(pl, p, s) : launch_chunks<512, 1, MODE>(pl, p, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_split_merge(const AttnPlan& pl, const AttnParams& p0, hipStream_t s) {
  AttnParams p = p0;
  p.ws_part = p0.ws_acc;
  p.ws_pml = p0.ws_ml;
  p.nchunk = pl.nsplit;  // unused by the streamed merges: each unit's splits come from stream_split
  if (pl.nsplit <= 16) {
    // few splits per unit on average: a thread per four dims walks them
    // (at B=56 x 2 KV heads x 512, about 5 per unit: 6.6 us, against 32 us
    // for the grouped merge's 3584 mostly idle workgroups)
    const int chunks = cdiv((long)pl.rows * (pl.D / 4), kMergeThreads);
    hipLaunchKernelGGL(merge_stream_flat, dim3(pl.units * chunks), dim3(kMergeThreads), 0, s, p, pl.D, chunks);
    return hipGetLastError();
  }
  const dim3 grid(pl.units * pl.rows * 4), block(kMergeThreads);
  switch (pl.D) {
    case 64: hipLaunchKernelGGL((merge_grouped<64, MODE_GSTREAM>), grid, block, 0, s, p); break;
    case 128: hipLaunchKernelGGL((merge_grouped<128, MODE_GSTREAM>), grid, block, 0, s, p); break;
    case 256: hipLaunchKernelGGL((merge_grouped<256, MODE_GSTREAM>), grid, block, 0, s, p); break;
    case 512: hipLaunchKernelGGL((merge_grouped<512, MODE_GSTREAM>), grid, block, 0, s, p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool plan_chunked(int mode, int B, int S, int Hq, int Hkv, int D, int keys, AttnPlan* pl) {
  if (mode != MODE_GLOBAL && mode != MODE_VERIFY) return false;
  if (B < 0 || S < 1 || S > 8 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || keys < 1) return false;
  if (D != 64 && D != 128 && D != 256 && D != 512) return false;
  const int rows = (Hq / Hkv) * S;
  if (rows > 32) return false;
  const int nchunk = mode == MODE_VERIFY ? cdiv(keys, kVerifyChunkKeys) : cdiv(keys, kChunkKeys);
  if (nchunk > kMaxChunks) return false;
  pl->mode = mode;
  pl->chunked = 1;
  pl->D = D;
  pl->nct = rows > 16 ? 2 : 1;
  pl->rows = rows;
  pl->units = B * Hkv;
  pl->threads = 64 * kChunkWaves;
  pl->max_tiles = cdiv(keys, 32);
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

hipError_t launch_chunked(const AttnPlan& pl, const AttnParams& p0, hipStream_t s) {
  if (pl.units == 0) return hipSuccess;
  AttnParams p = p0;
  p.nchunk = pl.nchunk;
  return pl.mode == MODE_VERIFY ? launch_chunks_mode<MODE_VERIFY>(pl, p, s)
                                : launch_chunks_mode<MODE_GLOBAL>(pl, p, s);
}

}  // namespace swr
