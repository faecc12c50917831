/*
 * swr.h -- C ABI of libswr.so: sliding-window ring and grouped-verify
 * attention for Gemma-4-style decode and speculative verification on AMD
 * Instinct MI355X (gfx950).
 *
 * Pages this interface follows:
 *   [Carat] "Announcing Carat: An inference engine designed for Gemma 4"
 *           - "Replacing page lookups with a ring buffer": each request owns a
 *             fixed ring; a token's slot is its absolute position modulo the
 *             window; a new token reuses the oldest slot without moving data.
 *           - "More FLOPs can be faster": global layers, key_count = context +
 *             proposals, scores over the keys, causal softmax by query
 *             position, weighted sum of values; the key dimension padded up
 *             to a multiple of 64 with a zero-initialised, masked tail.
 *           - "Doing it all in one kernel can be slower": the query heads that
 *             share a KV head times the proposed positions form one group of
 *             rows (8 x 4 = 32) against the same keys and values.
 *   [Gaudi] "Improving Decode Throughput on Intel Gaudi 3"
 *           - "Patching sliding window KV allocation": sliding layers keep
 *             only the last 1024 tokens.
 *           - "Our approach": rings are carved from the same HBM pool as the
 *             global-layer KV; K and V are written in lockstep, so the rings
 *             share one rotation and attention reads them in place.
 *   [Thor]  "gemma-cuda-hybrid" README, "Features": grouped-query attention
 *           reading KV once per KV head; FP8 (e4m3) KV cache.
 *
 * Conventions for every call below
 *   - All pointers marked "device" point to GPU memory the caller owns; the
 *     library allocates no device memory and keeps no state between calls
 *     (the pool functions keep host-side bookkeeping of a caller-owned
 *     device buffer).
 *   - Calls are asynchronous on `stream`; the caller keeps every buffer alive
 *     until the stream has passed the call.
 *   - Every call validates its host-side arguments first and, on failure,
 *     returns an error without touching device memory or launching.  Kernel
 *     launch failures are reported as SWR_ERR_LAUNCH.  Nothing throws.
 *   - bf16 means the 16-bit bfloat16 format; fp32 sums; outputs are rounded to
 *     bf16 with round-to-nearest-even.
 *   - Values that live in device memory (positions, key counts, region
 *     offsets) cannot be checked on the host; the preconditions stated for
 *     them are the caller's.  Every region read and write goes through a
 *     buffer resource whose base is k_base + k_off[b] (v_base + v_off[b])
 *     and whose extent is the region's size, so a position or key count out
 *     of range gives wrong numbers, not an access outside the region -- but
 *     only while k_off[b] and v_off[b] point at regions of the stated
 *     capacity inside allocated memory: a wrong offset moves the base itself
 *     and can fault.  Queries, outputs, new tokens and workspaces are plain
 *     arrays of the sizes stated for each call.
 *
 * KV region layout (one request, one layer; K and V regions separate; a
 * region has `cap` slots, cap a multiple of 8, and stores S = cap rounded up
 * to a multiple of 32 slots per KV head)
 *   slot s in [0, cap), KV head g in [0, Hkv), dim d in [0, D); element size
 *   e = 2 bytes (SWR_KV_BF16) or 1 byte (SWR_KV_FP8_E4M3); a granule is 16
 *   bytes = R dims of one slot (R = 8 bf16, 16 fp8):
 *     K: slot s = 32t + k lies in tile t, half h = (k/4)%2, row
 *       r = 4*(k/8) + k%4; each half holds its 16 rows in 1 KB blocks of
 *       four granules per row (granule q = d/R).  Byte offset of (s, g, d):
 *         ((g*S + 32t)*D + h*16*D)*e + (q/4)*1024 + r*64 + (q%4)*16 + (d%R)*e
 *       i.e. K is [Hkv][S/32][2][D/(4R)][16][4][R]; D is a multiple of 4R
 *     V element (s, g, d) at element index ((g*(S/8) + s/8)*D + d)*8 + (s%8)
 *       i.e. V is [Hkv][S/8][D][8]: blocks of 8 slots
 *   Each (request, KV head) reads one contiguous K stream and one contiguous
 *   V stream, which is what HBM streams best.  The K row order inside a tile
 *   is the key order of the gfx950 bf16 matrix instruction's operand in the
 *   kernels; a lane group's operand load (16 rows x 4 granules) is one
 *   contiguous 1 KB block, and a row's four granules are 64 contiguous
 *   bytes, so a token written on its own touches few cache lines.  V is
 *   kept in blocks of 8 slots so that the values of one dim for 8
 *   consecutive slots are contiguous: the operand shape along the key axis.
 *   A region is S*Hkv*D*e bytes (swr_kv_region_bytes).
 *   Ring regions: cap = W for every request, slot = position mod W.
 *   Global regions: slot = position; each region holds >= pad64(key_count)
 *   slots, those beyond key_count holding finite values (the pool's zero
 *   fill provides this); regions may differ in capacity (swr_kv.cap_b).
 */
#ifndef SWR_H
#define SWR_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h> /* hipStream_t */

#ifdef __cplusplus
extern "C" {
#endif

typedef enum swr_status {
  SWR_OK = 0,
  SWR_ERR_INVALID = 1,     /* a null pointer, a negative size, an inconsistent shape */
  SWR_ERR_UNSUPPORTED = 2, /* a shape outside the compiled set (see each call) */
  SWR_ERR_WORKSPACE = 3,   /* workspace missing or smaller than swr_workspace_bytes() */
  SWR_ERR_LAUNCH = 4,      /* the HIP runtime reported an error */
  SWR_ERR_NOMEM = 5        /* the pool has no free range large enough */
} swr_status;

typedef enum swr_kv_dtype {
  SWR_KV_BF16 = 0,     /* elements are bf16 */
  SWR_KV_FP8_E4M3 = 1  /* elements are OCP E4M3FN codes; value = decode(code) * scale */
} swr_kv_dtype;

typedef enum swr_op {
  SWR_OP_SWA_DECODE = 0,
  SWR_OP_GQA_VERIFY = 1,
  SWR_OP_GLOBAL_ATTEND = 2,
  SWR_OP_SWA_APPEND_DECODE = 3,
  SWR_OP_GLOBAL_APPEND_ATTEND = 4
} swr_op;

/* One layer's view of per-request K/V regions inside one or two device
 * buffers (usually the shared pool: [Gaudi] "Our approach"). */
typedef struct swr_kv {
  void* k_base;          /* device: base of the buffer holding K regions */
  void* v_base;          /* device: base of the buffer holding V regions (may equal k_base) */
  const int64_t* k_off;  /* device [B]: byte offset of request b's K region from k_base (16-B aligned) */
  const int64_t* v_off;  /* device [B]: same for V */
  const int32_t* cap_b;  /* device [B] per-request slot counts of global regions (multiples of 8,
                            each <= cap), or NULL when every region has `cap` slots.  Must be
                            NULL for rings. */
  int32_t cap;           /* slots per region: the window W for rings; for global regions the
                            capacity (the largest one when cap_b is given) */
  int32_t dtype;         /* swr_kv_dtype */
  float k_scale;         /* fp8 only: per-tensor scale of K (> 0, finite) */
  float v_scale;         /* fp8 only: per-tensor scale of V (> 0, finite) */
} swr_kv;

/* ------------------------------------------------------------------ append */

/* Write new tokens' K and V into each request's region ([Carat] ring section:
 * a token's slot is its position modulo the window; [Gaudi] "Our approach":
 * K and V of a token go to the same slot).  The same call writes contiguous
 * global regions (wrap == 0).
 *   k_new, v_new : device bf16 [B][T][Hkv][D] (row-major, 16-B aligned)
 *   pos0         : device int32 [B], position of token 0 of request b (>= 0)
 *   n_new        : device int32 [B] tokens to write for request b (0..T), or
 *                  NULL for T each
 *   wrap != 0    : ring, slot = position mod cap.  When n_new > cap only the
 *                  last cap tokens are written, which is what writing them one
 *                  after another leaves behind.
 *   wrap == 0    : global region, slot = position (position < the region's
 *                  capacity; larger positions are dropped).
 *   kv->cap_b must be NULL when wrap != 0.
 *   fp8 regions store the code nearest to value/scale (exact quotient,
 *   ties to even, saturating at +-448; NaN -> 0x7F with its sign).
 * Supported: D in {64, 128, 256, 512}; T >= 1; B >= 0 (B == 0 is a no-op). */
swr_status swr_ring_kv_append(const swr_kv* kv, const void* k_new, const void* v_new,
                              const int32_t* pos0, const int32_t* n_new, int B, int T, int Hkv,
                              int D, int wrap, hipStream_t stream);

/* -------------------------------------------------------- sliding decode */

/* Sliding-window GQA decode, one query token per request ([Carat] ring
 * section; [Gaudi] "Our approach": the ring is read in place, no gather, no
 * un-rotation).  The query at pos[b] sees the keys at positions
 * max(0, pos-W+1) .. pos, all of which are in the ring (its own token was
 * appended first), i.e. ring slots 0 .. min(pos+1, W)-1 in any rotation.
 *   ring  : ring regions, ring->cap = W
 *   q     : device bf16 [B][Hq][D]; query head h reads KV head h / (Hq/Hkv)
 *   out   : device bf16 [B][Hq][D]
 *   pos   : device int32 [B], >= 0
 *   scale : multiplies q.k before the softmax (e.g. 1/sqrt(D))
 *   ws    : device workspace of ws_bytes >= swr_workspace_bytes(SWR_OP_SWA_DECODE, B, 1, Hq,
 *           Hkv, D, W) (may be NULL when that is 0)
 * Supported: D in {64, 128, 256, 512}; Hq/Hkv in 1..16. */
swr_status swr_swa_decode(const swr_kv* ring, const void* q, void* out, const int32_t* pos, int B,
                          int Hq, int Hkv, int D, float scale, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* Append + sliding decode in one call ([Carat] ring section: a decode step
 * writes the new token into the slot of the oldest one and attends over the
 * window; [Gaudi] "Our approach": K and V go to the same slot).  Equivalent
 * to swr_ring_kv_append(ring, k_new, v_new, pos, NULL, B, 1, Hkv, D, 1) followed
 * by swr_swa_decode(ring, q, out, pos, ...): the ring holds the same bytes
 * afterwards and the output is the same attention, from one launch (plus
 * the split merge when B*Hkv is small) instead of two.
 *   k_new, v_new : device bf16 [B][Hkv][D], the token at position pos[b]
 *   ring, q, out, pos, scale : as for swr_swa_decode
 *   ws : >= swr_workspace_bytes(SWR_OP_SWA_APPEND_DECODE, B, 1, Hq, Hkv, D, W)
 * Supported: as swr_swa_decode. */
swr_status swr_swa_append_decode(const swr_kv* ring, const void* k_new, const void* v_new,
                                 const void* q, void* out, const int32_t* pos, int B, int Hq,
                                 int Hkv, int D, float scale, void* ws, size_t ws_bytes,
                                 hipStream_t stream);

/* ------------------------------------------------------- sliding verify */

/* Speculative verification on a sliding layer ([Carat] "Doing it all in one
 * kernel can be slower": G query heads x S proposed positions per KV head).
 * The ring holds committed positions < pos0[b]; the S proposals are passed
 * separately so that none of the keys the first rows still need is evicted.
 * Row (i, h) at position pos0+i sees ring keys with position >= pos0+i-W+1
 * and proposals 0..i.  After acceptance the caller appends the accepted
 * prefix with swr_ring_kv_append.
 *   k_prop, v_prop : device bf16 [B][S][Hkv][D]
 *   q, out         : device bf16 [B][S][Hq][D]
 *   pos0           : device int32 [B], >= 0
 *   ws             : >= swr_workspace_bytes(SWR_OP_GQA_VERIFY, B, S, Hq, Hkv, D, W)
 * Supported: D in {64, 128, 256, 512}; 1 <= S <= 8; (Hq/Hkv)*S <= 32. */
swr_status swr_gqa_verify(const swr_kv* ring, const void* k_prop, const void* v_prop,
                          const void* q, void* out, const int32_t* pos0, int B, int S, int Hq,
                          int Hkv, int D, float scale, void* ws, size_t ws_bytes,
                          hipStream_t stream);

/* ------------------------------------------------------- global layers */

/* Global-layer grouped attention over contiguous regions ([Carat] "More FLOPs
 * can be faster" and "Doing it all in one kernel can be slower").  Keys
 * 0 .. key_count[b]-1 are in the region (proposals appended first, so
 * key_count = context + proposals); the contraction runs over
 * pad64(key_count) keys whose tail is masked; row (i, h) sees keys
 * j <= q_pos[b][i] (and j < key_count[b]).
 *   kv            : global regions; each holds >= pad64(key_count[b]) slots
 *   q, out        : device bf16 [B][S][Hq][D]
 *   q_pos         : device int32 [B][S]
 *   key_count     : device int32 [B], 1 <= key_count[b] <= max_key_count
 *   max_key_count : host bound on key_count, sizes the launch and workspace
 *   ws            : >= swr_workspace_bytes(SWR_OP_GLOBAL_ATTEND, B, S, Hq, Hkv, D, max_key_count)
 * Supported: D in {64, 128, 256, 512}; 1 <= S <= 8; (Hq/Hkv)*S <= 32. */
swr_status swr_global_attend(const swr_kv* kv, const void* q, void* out, const int32_t* q_pos,
                             const int32_t* key_count, int max_key_count, int B, int S, int Hq,
                             int Hkv, int D, float scale, void* ws, size_t ws_bytes,
                             hipStream_t stream);

/* Append + global-layer attention in one call ([Carat] "More FLOPs can be
 * faster": the proposals join the global KV, key_count = context +
 * proposals, then the grouped attention).  Writes the S tokens of request b
 * at positions pos0[b] .. pos0[b]+S-1 (slot = position) and computes the rows
 * of swr_global_attend with q_pos[b][i] = pos0[b] + i and key_count[b] =
 * pos0[b] + S.  Equivalent to swr_ring_kv_append(kv, k_new, v_new, pos0, NULL, B,
 * S, Hkv, D, 0) followed by swr_global_attend: same region bytes, same
 * attention.  When the K/V of all (request, KV head) pairs spans fewer than
 * 2048 tiles of 32 keys the call is one chunked pass plus its merge: the
 * chunk holding the tokens' slots takes them from k_new/v_new (over fp8, as
 * the values of the codes that will be stored) and the merge stores them
 * once every chunk has read.  Longer calls stream in one split-K pass; with
 * one token per request (S = 1) the split that reads the token's tile takes
 * it in place of the slot's old contents and stores it (over fp8, its
 * codes), with more the append runs first.
 *   k_new, v_new  : device bf16 [B][S][Hkv][D]
 *   q, out        : device bf16 [B][S][Hq][D]
 *   pos0          : device int32 [B], pos0[b] >= 0, pos0[b] + S <= max_key_count and
 *                   <= the region's capacity
 *   max_key_count : host bound on pos0[b] + S, sizes the launch and workspace
 *   ws : >= swr_workspace_bytes(SWR_OP_GLOBAL_APPEND_ATTEND, B, S, Hq, Hkv, D, max_key_count)
 * Supported: as swr_global_attend. */
swr_status swr_global_append_attend(const swr_kv* kv, const void* k_new, const void* v_new,
                                    const void* q, void* out, const int32_t* pos0,
                                    int max_key_count, int B, int S, int Hq, int Hkv, int D,
                                    float scale, void* ws, size_t ws_bytes, hipStream_t stream);

/* swr_global_append_attend without a caller workspace, for callers that
 * cannot allocate device memory (code under graph capture, serving loops
 * that forbid allocation).  Same arguments, semantics and results as
 * swr_global_append_attend minus ws / ws_bytes: the workspace is a static
 * device array of the library, 16 MiB per device, held from module load
 * until the process ends (its device address is looked up once per device,
 * with that device current).  Allocates nothing.  SWR_ERR_WORKSPACE when
 * the call needs more than 16 MiB (swr_workspace_bytes(
 * SWR_OP_GLOBAL_APPEND_ATTEND, ...) > 16 MiB), checked before any launch.
 * All calls on one device share the array and each call's partials are
 * left in it: calls that may overlap on one device (other streams, other
 * host threads) race and must not be issued. */
swr_status swr_global_append_attend_noalloc(const swr_kv* kv, const void* k_new, const void* v_new,
                                            const void* q, void* out, const int32_t* pos0,
                                            int max_key_count, int B, int S, int Hq, int Hkv, int D,
                                            float scale, hipStream_t stream);

/* Workspace bytes an attention call needs (0 when it needs none), for
 * either element type: the larger of the bf16 and fp8 calls' needs, since
 * the type can pick the launch form.  For decode and verify
 * `cap_or_max_keys` is the window W; for global attention it is
 * max_key_count.  Returns 0 for unsupported shapes as well (the call then
 * reports the shape error).  The workspace holds per-split partial results
 * (running maximum, weight sum and unnormalised output rows, fp32). */
size_t swr_workspace_bytes(int op, int B, int S, int Hq, int Hkv, int D, int cap_or_max_keys);

/* ------------------------------------------------------------ the pool */

/* Host-side carve of one device buffer into K/V regions ([Gaudi] "Our
 * approach": rings and global KV share one HBM pool).  The pool keeps byte
 * ranges on the host (first fit, 256-byte aligned ranges, thread-safe); the
 * region carves below also zero-fill what they hand out, on the caller's
 * stream, with the zero-fill kernel (no memset node, so the fill may be
 * captured into a graph): a fresh ring holds zeros, and a global region's
 * tail past the key count holds the zeros the padded contraction multiplies
 * ([Carat] "More FLOPs can be faster": the key axis is padded to a multiple
 * of 64 with a zero-initialised tail). */
typedef struct swr_pool swr_pool;

/* Bytes of one K (or V) region of `cap` slots: (cap rounded up to 32) *
 * Hkv * D * element size (-1 if the shape is invalid). */
int64_t swr_kv_region_bytes(int cap, int Hkv, int D, int dtype);

/* A pool over `bytes` bytes of the device buffer at `base` (256-byte
 * aligned; the caller owns it and keeps it alive while the pool is used).
 * base == NULL makes a bookkeeping-only pool: it carves the same ranges but
 * fills nothing and launches nothing (the caller then zero fills).
 * SWR_ERR_INVALID for a null `pool`, bytes == 0 or a misaligned base. */
swr_status swr_pool_create(void* base, size_t bytes, swr_pool** pool);
void swr_pool_destroy(swr_pool* pool);
/* Reserve `bytes` (> 0); *offset receives its 256-B aligned start (bytes
 * from base).  Nothing is filled. */
swr_status swr_pool_alloc(swr_pool* pool, size_t bytes, int64_t* offset);
/* Release a range returned by any of the carves (SWR_ERR_INVALID if unknown). */
swr_status swr_pool_free(swr_pool* pool, int64_t offset);
/* A ring for one request of one sliding layer ([Carat] ring section: each
 * request owns a fixed ring of W slots): a K region and a V region of
 * cap = W rounded up to a multiple of 8 slots (Hkv x D, element type dtype),
 * both zero-filled on `stream`.  *k_off, *v_off: the regions' offsets from
 * base; *cap: the slots (the ring's W in swr_kv.cap).  SWR_ERR_NOMEM when
 * the pool has no room (the pool is then as before the call); SWR_ERR_LAUNCH
 * when the fill could not be launched (the ranges are released again). */
swr_status swr_pool_alloc_ring(swr_pool* pool, int W, int Hkv, int D, int dtype, hipStream_t stream,
                               int64_t* k_off, int64_t* v_off, int32_t* cap);
/* A contiguous global-layer region for `tokens` keys of one request
 * ([Carat] "More FLOPs can be faster"): K and V regions of cap = tokens
 * rounded up to a multiple of 64 slots, both zero-filled on `stream`, so the
 * padded tail of every key count up to `tokens` holds zeros.  Outputs and
 * errors as for swr_pool_alloc_ring. */
swr_status swr_pool_alloc_global(swr_pool* pool, int tokens, int Hkv, int D, int dtype, hipStream_t stream,
                                 int64_t* k_off, int64_t* v_off, int32_t* cap);
/* Bytes in use and the largest free range. */
swr_status swr_pool_stats(const swr_pool* pool, size_t* used, size_t* largest_free);

/* Admission of one request ([Gaudi] "Patching sliding window KV
 * allocation": a sliding layer only ever reads its last W tokens, so it
 * keeps W slots however long the request grows, and only the global layers
 * take KV in proportion to the context).  Carves, all or nothing, the K and
 * V regions of n_sliding rings (as swr_pool_alloc_ring, shape Hkv_s x D_s)
 * and of n_global global regions of `context` tokens (as
 * swr_pool_alloc_global, shape Hkv_g x D_g), all of element type dtype, and
 * zero-fills every one of them on `stream`.
 *   k_off, v_off : host int64 [n_sliding + n_global] (out), sliding layers
 *                  first, in layer order
 *   global_cap   : host int32 (out): the global regions' cap (may be NULL
 *                  when n_global == 0)
 * SWR_ERR_NOMEM when the request does not fit, SWR_ERR_LAUNCH when a fill
 * could not be launched; the pool is then as before the call.
 * SWR_ERR_INVALID for a null pool or output, negative layer counts, no layer
 * at all, context < 1 or an invalid shape. */
swr_status swr_pool_admit(swr_pool* pool, int n_sliding, int W, int Hkv_s, int D_s, int n_global,
                          int context, int Hkv_g, int D_g, int dtype, hipStream_t stream, int64_t* k_off,
                          int64_t* v_off, int32_t* global_cap);
/* Releases the n K and n V ranges of a request (as filled by
 * swr_pool_admit); SWR_ERR_INVALID if any offset was not allocated (the
 * others are still released). */
swr_status swr_pool_release(swr_pool* pool, int n, const int64_t* k_off, const int64_t* v_off);
/* Region bytes (K and V of every layer, before the pool's 256-byte
 * alignment) that swr_pool_admit carves for one request, or, with
 * full_context != 0, what a cache that keeps the full context in every
 * layer (sliding ones included) would carve: the two admission policies the
 * page compares.  -1 for an invalid shape. */
int64_t swr_request_kv_bytes(int n_sliding, int W, int Hkv_s, int D_s, int n_global, int context,
                             int Hkv_g, int D_g, int dtype, int full_context);

/* Zero `bytes` of device memory at `ptr` with a kernel on `stream` (no
 * memset node, so it may be captured into a graph). */
swr_status swr_zero_fill(void* ptr, size_t bytes, hipStream_t stream);

/* ------------------------------------------------------ paged baseline */

/* The paged-cache path the ring replaces ([Gaudi] "Expensive KV gathers":
 * a sliding-window layer over a paged cache first gathers the window's
 * pages into a contiguous buffer each step).  Copies request b's window --
 * the positions max(0, pos[b]-W+1) .. pos[b] -- from its pages into ring
 * slot position mod W of `ring`, the layout swr_swa_decode reads, so that
 * a gather followed by swr_swa_decode computes what the ring computes after
 * swr_ring_kv_append.  Slots that hold no window position (pos[b] < W-1) and
 * slots whose page is missing keep what they held.
 *   k_pages, v_pages : device bf16 [n_pages][page_tokens][Hkv][D] (16-B
 *                      aligned): the token at position p of request b is row
 *                      p mod page_tokens of page block_table[b][p / page_tokens]
 *   block_table      : device int32 [B][max_pages]; an entry outside
 *                      0 .. n_pages-1, or a page index >= max_pages, is a
 *                      missing page (its slots are skipped, nothing is read)
 *   pos              : device int32 [B] (a negative entry skips the request)
 *   ring             : bf16 ring regions (ring->cap = W, cap_b NULL)
 * Errors: SWR_ERR_INVALID for null or misaligned pointers, B < 0, Hkv < 1,
 * n_pages, page_tokens or max_pages < 1, or cap_b set; SWR_ERR_UNSUPPORTED
 * for an fp8 ring or D outside {64, 128, 256, 512}.  B == 0 is a no-op. */
swr_status swr_paged_gather_window(const void* k_pages, const void* v_pages, int64_t n_pages,
                                   int page_tokens, const int32_t* block_table, int max_pages,
                                   const int32_t* pos, const swr_kv* ring, int B, int Hkv, int D,
                                   hipStream_t stream);

/* Measurement aid, outside the attention path: one streaming read of `bytes`
 * (a multiple of 16, at most 2^40) of device memory at `src` (16-byte
 * aligned) by `grid` workgroups (1 .. 65536) of 256 threads on `stream`.
 * pattern 0: the grid sweeps the range together (16-byte word i to thread
 * i mod (grid * 256)); pattern 1: each workgroup streams one contiguous span
 * of about bytes / grid.  Timing it over a range well beyond the chip's
 * caches gives the HBM read rate the attention kernels are compared with.
 * `sink`: caller-owned device memory of at least 1024 bytes that the kernel
 * may write (its contents mean nothing).  SWR_ERR_INVALID for a null
 * pointer, a misaligned `src`, a size that is not a multiple of 16 or too
 * large, a grid out of range or another pattern; SWR_OK with no launch for
 * bytes == 0. */
swr_status swr_read_ceiling(const void* src, size_t bytes, void* sink, int grid, int pattern,
                            hipStream_t stream);

/* Text for a status code (static storage). */
const char* swr_status_string(swr_status status);

#ifdef __cplusplus
}
#endif

#endif /* SWR_H */
