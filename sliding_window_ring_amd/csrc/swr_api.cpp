// swr_api.cpp -- the C ABI declared in include/swr.h: host-side argument
// validation, launch planning, and the host bookkeeping of the shared KV pool.
// Every check runs before any HIP call, so an invalid call never touches
// device memory.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <map>
#include <mutex>
#include <new>

#include "gather.h"
#include "swr.h"
#include "swr_internal.h"

using swr::AttnParams;
using swr::AttnPlan;

namespace {

constexpr double kLog2e = 1.4426950408889634;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_d(int D) { return D == 64 || D == 128 || D == 256 || D == 512; }

int elem_size(int dtype) { return dtype == SWR_KV_FP8_E4M3 ? 1 : 2; }

// Slots a region stores (whole 32-slot tiles), without the int overflow of
// the device-side helper for capacities near INT32_MAX.
int64_t stored_slots64(int cap) { return ((int64_t)cap + 31) / 32 * 32; }

// Checks the fields of a KV view that every call shares.
swr_status check_kv(const swr_kv* kv, int Hkv, int D) {
  if (!kv || !kv->k_base || !kv->v_base || !kv->k_off || !kv->v_off) return SWR_ERR_INVALID;
  if (!aligned16(kv->k_base) || !aligned16(kv->v_base)) return SWR_ERR_INVALID;
  if (kv->cap <= 0 || kv->cap % 8 != 0) return SWR_ERR_INVALID;
  if (kv->dtype != SWR_KV_BF16 && kv->dtype != SWR_KV_FP8_E4M3) return SWR_ERR_INVALID;
  if (kv->dtype == SWR_KV_FP8_E4M3) {
    if (!(kv->k_scale > 0.f) || !std::isfinite(kv->k_scale)) return SWR_ERR_INVALID;
    if (!(kv->v_scale > 0.f) || !std::isfinite(kv->v_scale)) return SWR_ERR_INVALID;
  }
  const double bytes = (double)stored_slots64(kv->cap) * Hkv * D * elem_size(kv->dtype);
  if (bytes > 4294967295.0) return SWR_ERR_UNSUPPORTED;  // regions are addressed with 32-bit offsets
  return SWR_OK;
}

swr_status to_status(hipError_t e) { return e == hipSuccess ? SWR_OK : SWR_ERR_LAUNCH; }

// Launch of the append kernel for an already validated call.
swr_status append_tokens(const swr_kv* kv, const void* k_new, const void* v_new, const int32_t* pos0,
                         const int32_t* n_new, int B, int T, int Hkv, int D, int wrap, hipStream_t stream) {
  swr::AppendParams p{};
  p.k_base = static_cast<uint8_t*>(kv->k_base);
  p.v_base = static_cast<uint8_t*>(kv->v_base);
  p.k_off = kv->k_off;
  p.v_off = kv->v_off;
  p.cap_b = kv->cap_b;
  p.cap = kv->cap;
  p.wrap = wrap ? 1 : 0;
  p.k_scale = kv->k_scale;
  p.v_scale = kv->v_scale;
  p.k_new = static_cast<const uint16_t*>(k_new);
  p.v_new = static_cast<const uint16_t*>(v_new);
  p.pos0 = pos0;
  p.n_new = n_new;
  p.B = B;
  p.T = T;
  p.Hkv = Hkv;
  p.D = D;
  return to_status(swr::launch_append(p, kv->dtype == SWR_KV_FP8_E4M3, stream));
}

}  // namespace

namespace swr {

// Shared validation and launch of the attention calls.  mode is what the
// caller asked for (decode, verify, global); `append` fuses the append of the
// tokens in k_prop / v_prop (decode: the new token at pos; global: S tokens
// at pos0 .. pos0+S-1).
swr_status attend(int mode, int append, const swr_kv* kv, const void* q, void* out,
                  const int32_t* pos, const int32_t* key_count, const void* k_prop,
                  const void* v_prop, int cap_or_max_keys, int B, int S, int Hq, int Hkv, int D,
                  float scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (B < 0 || S < 1 || Hq < 1 || Hkv < 1 || D < 1) return SWR_ERR_INVALID;
  if (Hq % Hkv != 0) return SWR_ERR_INVALID;
  if (!std::isfinite(scale)) return SWR_ERR_INVALID;
  if (!supported_d(D)) return SWR_ERR_UNSUPPORTED;
  swr_status st = check_kv(kv, Hkv, D);
  if (st != SWR_OK) return st;
  if (!q || !out || !pos || !aligned16(q) || !aligned16(out)) return SWR_ERR_INVALID;
  if (mode != swr::MODE_GLOBAL && kv->cap_b) return SWR_ERR_INVALID;  // rings share one window
  if ((mode == swr::MODE_VERIFY || append) &&
      (!k_prop || !v_prop || !aligned16(k_prop) || !aligned16(v_prop)))
    return SWR_ERR_INVALID;
  if (mode == swr::MODE_GLOBAL) {
    if ((!append && !key_count) || cap_or_max_keys < 1) return SWR_ERR_INVALID;
    if (append && cap_or_max_keys < S) return SWR_ERR_INVALID;
    // the padded contraction reads pad64(key_count) slots of every region
    if (((int64_t)cap_or_max_keys + 63) / 64 * 64 > kv->cap) return SWR_ERR_INVALID;
  }
  const int fp8 = kv->dtype == SWR_KV_FP8_E4M3;
  AttnPlan pl;
  bool planned;
  if (mode == swr::MODE_GLOBAL && append)
    planned = swr::plan_global_append(B, S, Hq, Hkv, D, fp8, cap_or_max_keys, &pl);
  else
    planned = swr::plan_attention(append ? swr::MODE_DECODE_APPEND : mode, B, S, Hq, Hkv, D, fp8,
                                  cap_or_max_keys, &pl);
  if (!planned) return SWR_ERR_UNSUPPORTED;
  if (pl.ws_bytes > 0 && (!ws || ws_bytes < pl.ws_bytes || !aligned16(ws))) return SWR_ERR_WORKSPACE;
  if (B == 0) return SWR_OK;

  AttnParams p{};
  p.k_base = static_cast<const uint8_t*>(kv->k_base);
  p.v_base = static_cast<const uint8_t*>(kv->v_base);
  p.k_off = kv->k_off;
  p.v_off = kv->v_off;
  p.cap_b = kv->cap_b;
  p.cap = kv->cap;
  const double ks = kv->dtype == SWR_KV_FP8_E4M3 ? (double)kv->k_scale : 1.0;
  p.qk_scale = (float)((double)scale * ks * kLog2e);
  p.v_scale = kv->dtype == SWR_KV_FP8_E4M3 ? kv->v_scale : 1.0f;
  p.qk_scale_prop = (float)((double)scale * kLog2e);
  p.inv_v_scale = (float)(1.0 / (double)p.v_scale);
  p.q = static_cast<const uint16_t*>(q);
  p.out = static_cast<uint16_t*>(out);
  p.pos = pos;
  p.key_count = key_count;
  p.k_prop = static_cast<const uint16_t*>(k_prop);
  p.v_prop = static_cast<const uint16_t*>(v_prop);
  p.k_scale_store = kv->k_scale;
  p.v_scale_store = kv->v_scale;
  if (mode == swr::MODE_GLOBAL && append) {
    if (pl.chunked) {
      p.append = 1;  // taken by the chunk holding the slots, stored by the merge
    } else if (S == 1) {
      // long call of one token per request: the split holding the token's
      // tile takes it in place of the slot's old contents and stores it, as
      // the fused decode does
      pl.mode = swr::MODE_GSTREAM_APPEND;
    } else {
      // long call of several tokens: the append kernel first, then the
      // streamed pass
      const swr_status st2 = append_tokens(kv, k_prop, v_prop, pos, nullptr, B, S, Hkv, D, 0, stream);
      if (st2 != SWR_OK) return st2;
    }
    p.qpos_from_pos0 = 1;  // positions and key counts derived from pos0
  }
  if (pl.chunked) {
    uint8_t* w = static_cast<uint8_t*>(ws);
    p.ws_part = reinterpret_cast<float*>(w + pl.off_part);
    p.ws_pml = reinterpret_cast<float*>(w + pl.off_pml);
  } else if (pl.ws_bytes > 0) {
    float* w = static_cast<float*>(ws);
    p.ws_acc = w;
    p.ws_ml = w + (size_t)pl.units * pl.nsplit * pl.rows * D;
  }
  p.B = B;
  p.S = S;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.G = Hq / Hkv;
  p.rows = pl.rows;
  p.nsplit = pl.nsplit;
  p.tiles_per_split = pl.tiles_per_split;
  return to_status(swr::launch_attention(pl, p, stream));
}

}  // namespace swr

namespace {
using swr::attend;
}  // namespace

namespace swr {
hipError_t launch_read_ceiling(const void* src, size_t n16, uint32_t* sink, int grid, int pattern,
                               hipStream_t stream);
}  // namespace swr

extern "C" {

swr_status swr_ring_kv_append(const swr_kv* kv, const void* k_new, const void* v_new,
                              const int32_t* pos0, const int32_t* n_new, int B, int T, int Hkv,
                              int D, int wrap, hipStream_t stream) {
  if (B < 0 || T < 1 || Hkv < 1 || D < 1) return SWR_ERR_INVALID;
  if (!supported_d(D)) return SWR_ERR_UNSUPPORTED;
  swr_status st = check_kv(kv, Hkv, D);
  if (st != SWR_OK) return st;
  if (!k_new || !v_new || !pos0 || !aligned16(k_new) || !aligned16(v_new)) return SWR_ERR_INVALID;
  if (wrap && kv->cap_b) return SWR_ERR_INVALID;  // rings share one window
  if (B == 0) return SWR_OK;
  return append_tokens(kv, k_new, v_new, pos0, n_new, B, T, Hkv, D, wrap, stream);
}

swr_status swr_swa_decode(const swr_kv* ring, const void* q, void* out, const int32_t* pos, int B,
                          int Hq, int Hkv, int D, float scale, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  if (!ring) return SWR_ERR_INVALID;
  return attend(swr::MODE_DECODE, 0, ring, q, out, pos, nullptr, nullptr, nullptr, ring->cap, B, 1,
                Hq, Hkv, D, scale, ws, ws_bytes, stream);
}

swr_status swr_swa_append_decode(const swr_kv* ring, const void* k_new, const void* v_new,
                                 const void* q, void* out, const int32_t* pos, int B, int Hq,
                                 int Hkv, int D, float scale, void* ws, size_t ws_bytes,
                                 hipStream_t stream) {
  if (!ring) return SWR_ERR_INVALID;
  return attend(swr::MODE_DECODE, 1, ring, q, out, pos, nullptr, k_new, v_new, ring->cap, B, 1, Hq,
                Hkv, D, scale, ws, ws_bytes, stream);
}

swr_status swr_gqa_verify(const swr_kv* ring, const void* k_prop, const void* v_prop,
                          const void* q, void* out, const int32_t* pos0, int B, int S, int Hq,
                          int Hkv, int D, float scale, void* ws, size_t ws_bytes,
                          hipStream_t stream) {
  if (!ring) return SWR_ERR_INVALID;
  return attend(swr::MODE_VERIFY, 0, ring, q, out, pos0, nullptr, k_prop, v_prop, ring->cap, B, S,
                Hq, Hkv, D, scale, ws, ws_bytes, stream);
}

swr_status swr_global_attend(const swr_kv* kv, const void* q, void* out, const int32_t* q_pos,
                             const int32_t* key_count, int max_key_count, int B, int S, int Hq,
                             int Hkv, int D, float scale, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  return attend(swr::MODE_GLOBAL, 0, kv, q, out, q_pos, key_count, nullptr, nullptr, max_key_count,
                B, S, Hq, Hkv, D, scale, ws, ws_bytes, stream);
}

swr_status swr_global_append_attend(const swr_kv* kv, const void* k_new, const void* v_new,
                                    const void* q, void* out, const int32_t* pos0,
                                    int max_key_count, int B, int S, int Hq, int Hkv, int D,
                                    float scale, void* ws, size_t ws_bytes, hipStream_t stream) {
  return attend(swr::MODE_GLOBAL, 1, kv, q, out, pos0, nullptr, k_new, v_new, max_key_count, B, S,
                Hq, Hkv, D, scale, ws, ws_bytes, stream);
}

size_t swr_workspace_bytes(int op, int B, int S, int Hq, int Hkv, int D, int cap_or_max_keys) {
  int mode;
  switch (op) {
    case SWR_OP_SWA_DECODE: mode = swr::MODE_DECODE; S = 1; break;
    case SWR_OP_GQA_VERIFY: mode = swr::MODE_VERIFY; break;
    case SWR_OP_GLOBAL_ATTEND: mode = swr::MODE_GLOBAL; break;
    case SWR_OP_SWA_APPEND_DECODE: mode = swr::MODE_DECODE_APPEND; S = 1; break;
    case SWR_OP_GLOBAL_APPEND_ATTEND: {  // the larger of the bf16 and fp8 plans
      AttnPlan p16, p8;
      if (!swr::plan_global_append(B, S, Hq, Hkv, D, 0, cap_or_max_keys, &p16)) return 0;
      if (!swr::plan_global_append(B, S, Hq, Hkv, D, 1, cap_or_max_keys, &p8)) return 0;
      return std::max(p16.ws_bytes, p8.ws_bytes);
    }
    default: return 0;
  }
  // the larger of the bf16 and fp8 plans: the element type can pick the
  // launch form (a verify over fp8 runs chunked at every batch)
  AttnPlan p16, p8;
  if (!swr::plan_attention(mode, B, S, Hq, Hkv, D, 0, cap_or_max_keys, &p16)) return 0;
  if (!swr::plan_attention(mode, B, S, Hq, Hkv, D, 1, cap_or_max_keys, &p8)) return 0;
  return std::max(p16.ws_bytes, p8.ws_bytes);
}

int64_t swr_kv_region_bytes(int cap, int Hkv, int D, int dtype) {
  if (cap <= 0 || cap % 8 != 0 || Hkv <= 0 || D <= 0) return -1;
  if (dtype != SWR_KV_BF16 && dtype != SWR_KV_FP8_E4M3) return -1;
  return stored_slots64(cap) * Hkv * D * elem_size(dtype);
}

swr_status swr_zero_fill(void* ptr, size_t bytes, hipStream_t stream) {
  if (bytes == 0) return SWR_OK;
  if (!ptr) return SWR_ERR_INVALID;
  return to_status(swr::launch_zero_fill(ptr, bytes, stream));
}

swr_status swr_paged_gather_window(const void* k_pages, const void* v_pages, int64_t n_pages, int page_tokens,
                                   const int32_t* block_table, int max_pages, const int32_t* pos,
                                   const swr_kv* ring, int B, int Hkv, int D, hipStream_t stream) {
  if (B < 0 || Hkv < 1 || D < 1 || n_pages < 1 || page_tokens < 1 || max_pages < 1) return SWR_ERR_INVALID;
  if (!supported_d(D)) return SWR_ERR_UNSUPPORTED;
  swr_status st = check_kv(ring, Hkv, D);
  if (st != SWR_OK) return st;
  if (ring->cap_b) return SWR_ERR_INVALID;                  // rings share one window
  if (ring->dtype != SWR_KV_BF16) return SWR_ERR_UNSUPPORTED;
  if (!k_pages || !v_pages || !block_table || !pos || !aligned16(k_pages) || !aligned16(v_pages))
    return SWR_ERR_INVALID;
  if ((int64_t)B * max_pages > INT32_MAX) return SWR_ERR_UNSUPPORTED;
  const int64_t threads = (int64_t)B * Hkv * (ring->cap / 8) * (D / 8);
  if ((threads + 255) / 256 > INT32_MAX) return SWR_ERR_UNSUPPORTED;
  if (B == 0) return SWR_OK;
  swr::GatherArgs a{};
  a.k_pages = static_cast<const uint16_t*>(k_pages);
  a.v_pages = static_cast<const uint16_t*>(v_pages);
  a.block_table = block_table;
  a.pos = pos;
  a.k_base = static_cast<uint8_t*>(ring->k_base);
  a.v_base = static_cast<uint8_t*>(ring->v_base);
  a.k_off = ring->k_off;
  a.v_off = ring->v_off;
  a.n_pages = n_pages;
  a.page_tokens = page_tokens;
  a.max_pages = max_pages;
  a.B = B;
  a.Hkv = Hkv;
  a.D = D;
  a.W = ring->cap;
  return to_status(swr::launch_paged_gather(a, stream));
}

swr_status swr_read_ceiling(const void* src, size_t bytes, void* sink, int grid, int pattern,
                            hipStream_t stream) {
  // read_ceiling.hip; a measurement aid, kept out of the attention kernels' shared header
  if (bytes == 0) return SWR_OK;
  if (!src || !sink || (reinterpret_cast<uintptr_t>(src) & 15) || (bytes & 15) || bytes > (size_t(1) << 40) ||
      grid < 1 || grid > 65536 || (pattern != 0 && pattern != 1))
    return SWR_ERR_INVALID;
  return to_status(
      swr::launch_read_ceiling(src, bytes / 16, static_cast<uint32_t*>(sink), grid, pattern, stream));
}

const char* swr_status_string(swr_status s) {
  switch (s) {
    case SWR_OK: return "ok";
    case SWR_ERR_INVALID: return "invalid argument";
    case SWR_ERR_UNSUPPORTED: return "unsupported shape";
    case SWR_ERR_WORKSPACE: return "workspace missing or too small";
    case SWR_ERR_LAUNCH: return "HIP launch error";
    case SWR_ERR_NOMEM: return "pool exhausted";
  }
  return "unknown status";
}

}  // extern "C"

// ------------------------------------------------------------------ pool

struct swr_pool {
  uint8_t* base;                   // device buffer (null: bookkeeping only)
  size_t size;
  std::map<int64_t, size_t> used;  // offset -> bytes (sorted by offset)
  size_t used_bytes = 0;
  mutable std::mutex mu;
};

namespace {
constexpr int64_t kPoolAlign = 256;
int64_t align_up(int64_t x) { return (x + kPoolAlign - 1) / kPoolAlign * kPoolAlign; }

// Carves a K and a V region of `tokens` slots rounded up to `mult` (8 for a
// ring, 64 for a global region) and, when the pool has a device buffer,
// zero-fills both on the stream; on any failure the pool is as before.
swr_status carve_kv(swr_pool* pool, int tokens, int mult, int Hkv, int D, int dtype, hipStream_t stream,
                    int64_t* k_offset, int64_t* v_offset, int32_t* cap) {
  if (!pool || !k_offset || !v_offset || !cap || tokens <= 0 || Hkv <= 0 || D <= 0) return SWR_ERR_INVALID;
  const int64_t c = ((int64_t)tokens + mult - 1) / mult * mult;
  if (c > INT32_MAX) return SWR_ERR_INVALID;
  const int64_t rb = swr_kv_region_bytes((int)c, Hkv, D, dtype);
  if (rb <= 0) return SWR_ERR_INVALID;
  int64_t ko, vo;
  swr_status st = swr_pool_alloc(pool, (size_t)rb, &ko);
  if (st != SWR_OK) return st;
  st = swr_pool_alloc(pool, (size_t)rb, &vo);
  if (st == SWR_OK && pool->base) {
    st = to_status(swr::launch_zero_fill(pool->base + ko, (size_t)rb, stream));
    if (st == SWR_OK) st = to_status(swr::launch_zero_fill(pool->base + vo, (size_t)rb, stream));
    if (st != SWR_OK) swr_pool_free(pool, vo);
  }
  if (st != SWR_OK) {
    swr_pool_free(pool, ko);
    return st;
  }
  *k_offset = ko;
  *v_offset = vo;
  *cap = (int32_t)c;
  return SWR_OK;
}
}  // namespace

extern "C" {

swr_status swr_pool_create(void* base, size_t bytes, swr_pool** pool) {
  if (!pool || bytes == 0 || (reinterpret_cast<uintptr_t>(base) % kPoolAlign) != 0) return SWR_ERR_INVALID;
  swr_pool* p = new (std::nothrow) swr_pool();
  if (!p) return SWR_ERR_NOMEM;
  p->base = static_cast<uint8_t*>(base);
  p->size = bytes;
  *pool = p;
  return SWR_OK;
}

void swr_pool_destroy(swr_pool* pool) { delete pool; }

swr_status swr_pool_alloc(swr_pool* pool, size_t bytes, int64_t* offset) {
  if (!pool || !offset || bytes == 0 || bytes > (size_t)INT64_MAX / 2) return SWR_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  // first fit: walk the used ranges in address order, try each gap
  int64_t cursor = 0;
  for (const auto& kv : pool->used) {
    const int64_t start = align_up(cursor);
    if (start + (int64_t)bytes <= kv.first) {
      pool->used.emplace(start, bytes);
      pool->used_bytes += bytes;
      *offset = start;
      return SWR_OK;
    }
    cursor = kv.first + (int64_t)kv.second;
  }
  const int64_t start = align_up(cursor);
  if (start + (int64_t)bytes > (int64_t)pool->size) return SWR_ERR_NOMEM;
  pool->used.emplace(start, bytes);
  pool->used_bytes += bytes;
  *offset = start;
  return SWR_OK;
}

swr_status swr_pool_free(swr_pool* pool, int64_t offset) {
  if (!pool) return SWR_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  auto it = pool->used.find(offset);
  if (it == pool->used.end()) return SWR_ERR_INVALID;
  pool->used_bytes -= it->second;
  pool->used.erase(it);
  return SWR_OK;
}

swr_status swr_pool_alloc_ring(swr_pool* pool, int W, int Hkv, int D, int dtype, hipStream_t stream,
                               int64_t* k_off, int64_t* v_off, int32_t* cap) {
  return carve_kv(pool, W, 8, Hkv, D, dtype, stream, k_off, v_off, cap);
}

swr_status swr_pool_alloc_global(swr_pool* pool, int tokens, int Hkv, int D, int dtype, hipStream_t stream,
                                 int64_t* k_off, int64_t* v_off, int32_t* cap) {
  return carve_kv(pool, tokens, 64, Hkv, D, dtype, stream, k_off, v_off, cap);
}

int64_t swr_request_kv_bytes(int n_sliding, int W, int Hkv_s, int D_s, int n_global, int context, int Hkv_g,
                             int D_g, int dtype, int full_context) {
  if (n_sliding < 0 || n_global < 0 || context < 1 || (n_sliding > 0 && W < 1)) return -1;
  const int64_t ring_slots = full_context ? (int64_t)context : (int64_t)W;
  const int64_t ring_cap = (ring_slots + 7) / 8 * 8, glob_cap = ((int64_t)context + 63) / 64 * 64;
  if (ring_cap > INT32_MAX || glob_cap > INT32_MAX) return -1;
  int64_t total = 0;
  if (n_sliding > 0) {
    const int64_t rb = swr_kv_region_bytes((int)ring_cap, Hkv_s, D_s, dtype);
    if (rb <= 0) return -1;
    total += 2 * rb * n_sliding;
  }
  if (n_global > 0) {
    const int64_t gb = swr_kv_region_bytes((int)glob_cap, Hkv_g, D_g, dtype);
    if (gb <= 0) return -1;
    total += 2 * gb * n_global;
  }
  return total;
}

swr_status swr_pool_release(swr_pool* pool, int n, const int64_t* k_off, const int64_t* v_off) {
  if (!pool || n < 0 || (n > 0 && (!k_off || !v_off))) return SWR_ERR_INVALID;
  swr_status st = SWR_OK;
  for (int i = 0; i < n; ++i) {
    if (swr_pool_free(pool, k_off[i]) != SWR_OK) st = SWR_ERR_INVALID;
    if (swr_pool_free(pool, v_off[i]) != SWR_OK) st = SWR_ERR_INVALID;
  }
  return st;
}

swr_status swr_pool_admit(swr_pool* pool, int n_sliding, int W, int Hkv_s, int D_s, int n_global, int context,
                          int Hkv_g, int D_g, int dtype, hipStream_t stream, int64_t* k_off, int64_t* v_off,
                          int32_t* global_cap) {
  if (!pool || n_sliding < 0 || n_global < 0 || n_sliding + n_global < 1 || context < 1) return SWR_ERR_INVALID;
  if (!k_off || !v_off || (n_global > 0 && !global_cap)) return SWR_ERR_INVALID;
  if (swr_request_kv_bytes(n_sliding, W, Hkv_s, D_s, n_global, context, Hkv_g, D_g, dtype, 0) < 0)
    return SWR_ERR_INVALID;
  int done = 0;
  swr_status st = SWR_OK;
  int32_t cap = 0;
  for (; done < n_sliding + n_global; ++done) {
    const bool glob = done >= n_sliding;
    st = glob ? carve_kv(pool, context, 64, Hkv_g, D_g, dtype, stream, &k_off[done], &v_off[done], &cap)
              : carve_kv(pool, W, 8, Hkv_s, D_s, dtype, stream, &k_off[done], &v_off[done], &cap);
    if (st != SWR_OK) break;
    if (glob) *global_cap = cap;
  }
  if (st != SWR_OK) {  // all or nothing
    swr_pool_release(pool, done, k_off, v_off);
    return st;
  }
  return SWR_OK;
}

swr_status swr_pool_stats(const swr_pool* pool, size_t* used, size_t* largest_free) {
  if (!pool) return SWR_ERR_INVALID;
  std::lock_guard<std::mutex> lk(pool->mu);
  size_t largest = 0;
  int64_t cursor = 0;
  for (const auto& kv : pool->used) {
    const int64_t start = align_up(cursor);
    if (kv.first > start) largest = std::max(largest, (size_t)(kv.first - start));
    cursor = kv.first + (int64_t)kv.second;
  }
  const int64_t start = align_up(cursor);
  if ((int64_t)pool->size > start) largest = std::max(largest, (size_t)((int64_t)pool->size - start));
  if (used) *used = pool->used_bytes;
  if (largest_free) *largest_free = largest;
  return SWR_OK;
}

}  // extern "C"
