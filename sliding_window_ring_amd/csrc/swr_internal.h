// swr_internal.h -- host-side launch plans and kernel entry declarations
// shared by the C-ABI layer (swr_api.cpp) and the kernel sources.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace swr {

// MODE_GLOBAL is what a global-layer call asks for; the planner runs it either
// in chunked form (chunked.hip) or, for long regions, as MODE_GSTREAM: the
// single-pass split-K kernel of the ring calls over a contiguous region.
// MODE_VERIFY runs in chunked form when the batch is small.
// MODE_DECODE_APPEND is a decode that first writes the new token into its
// ring slot (the fused append + decode call); MODE_GSTREAM_APPEND the same
// for a streamed global call of one token per request (slot = position).
enum Mode {
  MODE_DECODE = 0,
  MODE_VERIFY = 1,
  MODE_GLOBAL = 2,
  MODE_GSTREAM = 3,
  MODE_DECODE_APPEND = 4,
  MODE_GSTREAM_APPEND = 5
};

// Slots a region stores per KV head: its capacity rounded up to whole
// 32-slot K tiles (region layout: swr_device.h).
__host__ __device__ constexpr int stored_slots(int cap) { return (cap + 31) & ~31; }

// Everything an attention launch reads, by value.
struct AttnParams {
  const uint8_t* k_base;
  const uint8_t* v_base;
  const int64_t* k_off;
  const int64_t* v_off;
  const int32_t* cap_b;    // per-request slots (global regions) or null: every region has cap
  int cap;                 // slots per region (ring: W)
  float qk_scale;          // scale * k_scale * log2(e): scores in the base-2 domain
  float v_scale;           // applied to the normalised output
  float qk_scale_prop;     // verify: scale * log2(e) for the bf16 proposal keys (no k_scale)
  float inv_v_scale;       // verify: 1 / v_scale, applied to the bf16 proposals' value product
  const uint16_t* q;       // bf16 [B][S][Hq][D]
  uint16_t* out;           // bf16 [B][S][Hq][D]
  const int32_t* pos;      // decode: pos[B]; verify: pos0[B]; global (both forms): q_pos[B][S]
  const int32_t* key_count;  // global: [B]
  const uint16_t* k_prop;  // verify: proposals; fused append: the tokens to store.  bf16 [B][S][Hkv][D]
  const uint16_t* v_prop;
  int append;              // chunked global call storing its own S tokens at pos0 + j (by the merge)
  int qpos_from_pos0;      // streamed global: pos is pos0[B]; q_pos[b][i] = pos0[b] + i, key_count = pos0[b] + S
  float k_scale_store;     // fp8 regions: the scales a stored token's K and V are divided by
  float v_scale_store;
  float* ws_acc;           // split partials: [units][nsplit][rows][D]
  float* ws_ml;            // split partials: [units][nsplit][rows][2] (max, sum)
  int B, S, Hq, Hkv, G, rows;
  int nsplit;              // workgroups per (request, KV head)
  int tiles_per_split;     // 32-key tiles each split covers
  // chunked form (a chunk of keys per workgroup, then a merge)
  float* ws_part;          // [units][nchunk][rows][D] unnormalised chunk outputs
  float* ws_pml;           // [units][nchunk][rows][2] (max, sum) of each chunk
  int nchunk;              // chunks per unit (of the longest request; verify: + the proposals')
};

// Global calls: the key count of request b and the position of its query i,
// from the arrays, or derived from pos0 when the call appended its S tokens
// at pos0 .. pos0+S-1 itself.
__device__ __forceinline__ int key_count_of(const AttnParams& p, int b) {
  return p.qpos_from_pos0 ? p.pos[b] + p.S : p.key_count[b];
}
__device__ __forceinline__ int qpos_of(const AttnParams& p, int b, int i) {
  return p.qpos_from_pos0 ? p.pos[b] + i : p.pos[b * p.S + i];
}

// Streamed global calls: the splits, balanced over the grid from the
// requests' key counts.  Request b has stream_tiles(b) tiles of 32 keys (its
// keys up to its region's capacity); T is the tiles of all (request, KV head)
// units and P = units * nsplit the grid's workgroups.  A split takes at most
// R = ceil(T / (P - units)) tiles, unit u takes n_u = ceil(tiles_u / R)
// splits (so that sum n_u <= T / R + units <= P), split s the tiles
// [s * tiles_u / n_u, (s + 1) * tiles_u / n_u), and the splits are numbered
// request by request, KV head by KV head: workgroup w computes split w (the
// rest exit), and the merge finds unit u's partials at first_u .. first_u +
// n_u - 1.  The split pass and the merge compute the numbering alike.
__device__ __forceinline__ int stream_tiles(const AttnParams& p, int b) {
  const int cap = p.cap_b ? max(min(p.cap_b[b], p.cap), 0) : p.cap;
  return (max(min(key_count_of(p, b), cap), 0) + 31) >> 5;
}
// Inclusive prefix sum over the wave's 64 lanes.
__device__ __forceinline__ int wave_prefix_sum(int x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(x, o, 64);
    if (lane >= o) x += y;
  }
  return x;
}
struct StreamSplit {
  int unit = -1;  // -1: past the last split
  int split = 0, first = 0, n = 0, tiles = 0;
};
// The split numbered w (unit < 0), or unit's first split and split count
// (w ignored).  Every lane of the wave takes part (64 requests at a time, one
// per lane: the key counts load together, and wave scans number the splits);
// the result is wave-uniform.
__device__ __forceinline__ StreamSplit stream_split(const AttnParams& p, int w, int unit = -1) {
  const int lane = threadIdx.x & 63;
  long t = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    const int tb = b < p.B ? stream_tiles(p, b) : 0;
    t += __builtin_amdgcn_readlane(wave_prefix_sum(tb), 63);
  }
  t *= p.Hkv;
  const long room = (long)p.B * p.Hkv * (p.nsplit - 1);  // P - units > 0: nsplit >= 2
  const int r = (int)max(1L, (t + room - 1) / room);
  StreamSplit x;
  int first = 0;
  for (int b0 = 0; b0 < p.B; b0 += 64) {
    const int b = b0 + lane;
    const int tb = b < p.B ? stream_tiles(p, b) : 0;
    const int n = (tb + r - 1) / r;
    const int cnt = p.Hkv * n;
    const int incl = first + wave_prefix_sum(cnt);
    const int excl = incl - cnt;
    const bool here = b < p.B && (unit >= 0 ? b == unit / p.Hkv : (w >= excl && w < incl));
    const unsigned long long m = __ballot(here);
    if (m) {
      const int src = __ffsll(m) - 1;
      const int nb = __builtin_amdgcn_readlane(n, src);
      const int eb = __builtin_amdgcn_readlane(excl, src);
      const int bb = b0 + src;
      const int g = unit >= 0 ? unit - bb * p.Hkv : (w - eb) / nb;
      x.unit = bb * p.Hkv + g;
      x.first = eb + g * nb;
      x.n = nb;
      x.tiles = __builtin_amdgcn_readlane(tb, src);
      x.split = unit >= 0 ? 0 : w - x.first;
      return x;
    }
    first = __builtin_amdgcn_readlane(incl, 63);
  }
  return x;
}

// Launch geometry chosen on the host for one attention call.
struct AttnPlan {
  int mode, D, fp8;
  int ds;        // head dims per wave (D / ds waves share a key tile)
  int nct;       // 16-row column tiles (rows = G*S <= 16*nct)
  int kw;        // waves splitting the keys inside a workgroup
  int units;     // B * Hkv
  int rows;      // G * S
  int max_tiles; // 32-key tiles of the longest unit
  int nsplit;
  int tiles_per_split;
  size_t ws_bytes;  // 0 when nsplit == 1 (decode, verify)
  size_t lds_bytes;
  int threads;
  // chunked form
  int chunked;     // 1: chunk_kernel + merge (chunked.hip)
  int nchunk;      // chunks per unit
  size_t off_part, off_pml;  // workspace offsets
};

// Chunked form (chunked.hip): per-chunk attention, then a merge.  mode is
// MODE_GLOBAL (keys = max_key_count) or MODE_VERIFY (keys = ring window W).
bool plan_chunked(int mode, int B, int S, int Hq, int Hkv, int D, int keys, AttnPlan* plan);
hipError_t launch_chunked(const AttnPlan& plan, const AttnParams& p, hipStream_t stream);
// Merge of the split partials of a streamed global call (many splits per
// row), by the chunked form's grouped merge.
hipError_t launch_split_merge(const AttnPlan& plan, const AttnParams& p, hipStream_t stream);

// Fills *plan; returns false for shapes outside the compiled set.
bool plan_attention(int mode, int B, int S, int Hq, int Hkv, int D, int fp8, int cap_or_max_keys,
                    AttnPlan* plan);

hipError_t launch_attention(const AttnPlan& plan, const AttnParams& p, hipStream_t stream);

// Plan of a global call that appends its S tokens itself (max_keys bounds
// pos0 + S): in chunked form (tokens read from their buffers by the chunk
// holding their slots, stored by the merge), or for long calls the streamed
// global pass (run after the append kernel), positions derived from pos0.
bool plan_global_append(int B, int S, int Hq, int Hkv, int D, int fp8, int max_keys, AttnPlan* plan);

struct AppendParams {
  uint8_t* k_base;
  uint8_t* v_base;
  const int64_t* k_off;
  const int64_t* v_off;
  const int32_t* cap_b;
  int cap;
  int wrap;
  float k_scale, v_scale;
  const uint16_t* k_new;  // bf16 [B][T][Hkv][D]
  const uint16_t* v_new;
  const int32_t* pos0;
  const int32_t* n_new;   // may be null
  int B, T, Hkv, D;
};

hipError_t launch_append(const AppendParams& p, int fp8, hipStream_t stream);
hipError_t launch_zero_fill(void* ptr, size_t bytes, hipStream_t stream);

}  // namespace swr

#include "swr.h"

namespace swr {

// Validation, planning and launch shared by the attention entry points
// (swr_api.cpp): mode is MODE_DECODE, MODE_VERIFY or MODE_GLOBAL as asked
// for; append fuses the append of the tokens in k_prop / v_prop.
swr_status attend(int mode, int append, const swr_kv* kv, const void* q, void* out, const int32_t* pos,
                  const int32_t* key_count, const void* k_prop, const void* v_prop, int cap_or_max_keys, int B,
                  int S, int Hq, int Hkv, int D, float scale, void* ws, size_t ws_bytes, hipStream_t stream);

}  // namespace swr
