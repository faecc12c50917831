/*
 * swr_layout.c -- the device byte layout of a K/V region, as a codec between
 * that layout and the logical [slot][Hkv][D] arrays the oracle computes on.
 *
 * TEST INFRASTRUCTURE ONLY (as swr_oracle.c): only the test suite, the smoke
 * check and the CPU-baseline leg of the benchmark may load it.  It shares no
 * source with the GPU library: the layout below is restated from the one the
 * library's header declares, and it holds no attention arithmetic, so a
 * change of the device layout touches this file alone.
 *
 * The pages fix no layout.  What they fix, and what the oracle's arithmetic
 * relies on, is the logical content of a region: slot s of a ring holds the
 * token whose position is s modulo the window ("Announcing Carat", ring
 * buffer section), K and V of a token share the slot ("Improving Decode
 * Throughput on Intel Gaudi 3", Our approach).  The logical region of `cap`
 * slots is element (s, g, d) at index (s*Hkv + g)*D + d, an element being a
 * bf16 bit pattern (2 bytes) or an E4M3 code (1 byte).
 *
 * Device layout of one region (per KV head, S = cap rounded up to 32 slots
 * are stored; a granule is 16 bytes, R = 8 bf16 or 16 fp8 dims):
 *   K: [Hkv][S/32][2][D/(4R)][16][4][R] -- slot 32t + k sits in tile t, half
 *      (k/4)%2, row 4*(k/8) + k%4; granule q = d/R of that row is in block
 *      q/4, position q%4 of the row's four granules.
 *   V: [Hkv][S/8][D][8] -- blocks of 8 slots, element (s, g, d) at
 *      ((g*(S/8) + s/8)*D + d)*8 + s%8.
 * Slots cap .. S-1 of a region hold no token; pack leaves them as they are.
 */
#include <stdint.h>
#include <string.h>

static int esize_of(int dtype) { return dtype == 1 ? 1 : 2; }

static int64_t stored_slots(int64_t cap) { return (cap + 31) / 32 * 32; }

/* K rows are blocks of four granules: D must hold a whole number of them. */
static int shape_ok(int cap, int Hkv, int D, int dtype) {
  const int R = 16 / esize_of(dtype);
  return cap > 0 && cap % 8 == 0 && Hkv > 0 && D > 0 && D % (4 * R) == 0 && (dtype == 0 || dtype == 1);
}

/* Element index (units of the element size) of (s, g, d) in a K region. */
static int64_t k_elem(int64_t s, int g, int d, int64_t cap, int D, int dtype) {
  const int64_t S = stored_slots(cap);
  const int64_t R = 16 / esize_of(dtype);
  const int64_t t = s / 32, k = s % 32;
  const int64_t half = (k / 4) % 2, row = 4 * (k / 8) + k % 4;
  const int64_t q = d / R;
  return ((int64_t)g * S + 32 * t) * D + half * 16 * D + (q / 4) * 64 * R + row * 4 * R + (q % 4) * R + d % R;
}

/* Element index of (s, g, d) in a V region. */
static int64_t v_elem(int64_t s, int g, int d, int64_t cap, int D) {
  const int64_t S = stored_slots(cap);
  return (((int64_t)g * (S / 8) + s / 8) * D + d) * 8 + s % 8;
}

/* Bytes of one K (or V) region of `cap` slots in the device layout, or -1. */
int64_t orc_region_bytes(int cap, int Hkv, int D, int dtype) {
  if (!shape_ok(cap, Hkv, D, dtype)) return -1;
  return stored_slots(cap) * Hkv * D * esize_of(dtype);
}

/* Copies the logical region `logical` ([cap][Hkv][D] elements) into the
 * device-layout region `region` (is_v: V layout, else K).  Returns 0, or -1
 * for an invalid shape. */
int orc_layout_pack(const uint8_t* logical, uint8_t* region, int cap, int Hkv, int D, int dtype, int is_v) {
  if (!shape_ok(cap, Hkv, D, dtype)) return -1;
  const int e = esize_of(dtype);
  for (int64_t s = 0; s < cap; ++s)
    for (int g = 0; g < Hkv; ++g)
      for (int d = 0; d < D; ++d) {
        const int64_t src = (s * Hkv + g) * D + d;
        const int64_t dst = is_v ? v_elem(s, g, d, cap, D) : k_elem(s, g, d, cap, D, dtype);
        memcpy(region + dst * e, logical + src * e, (size_t)e);
      }
  return 0;
}

/* The inverse: the device-layout region `region` into the logical region
 * `logical` ([cap][Hkv][D] elements).  Returns 0, or -1 for an invalid shape. */
int orc_layout_unpack(const uint8_t* region, uint8_t* logical, int cap, int Hkv, int D, int dtype, int is_v) {
  if (!shape_ok(cap, Hkv, D, dtype)) return -1;
  const int e = esize_of(dtype);
  for (int64_t s = 0; s < cap; ++s)
    for (int g = 0; g < Hkv; ++g)
      for (int d = 0; d < D; ++d) {
        const int64_t dst = (s * Hkv + g) * D + d;
        const int64_t src = is_v ? v_elem(s, g, d, cap, D) : k_elem(s, g, d, cap, D, dtype);
        memcpy(logical + dst * e, region + src * e, (size_t)e);
      }
  return 0;
}
