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
// ring slot (the fused append + decode call).
enum Mode { MODE_DECODE = 0, MODE_VERIFY = 1, MODE_GLOBAL = 2, MODE_GSTREAM = 3, MODE_DECODE_APPEND = 4 };

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
  float inv_v_scale;       // verify: 1 / v_scale, applied to the bf16 proposal values
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
