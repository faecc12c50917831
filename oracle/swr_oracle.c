/*
 * swr_oracle.c -- plain, slow CPU oracle for the sliding-window ring and
 * grouped-verify attention path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * CPU-baseline leg of the benchmark may load this code.  The GPU library
 * never links it, includes it or calls it, and this file shares no source
 * with the GPU library: every format and formula below is written out again
 * from the pages it cites.
 *
 * Sources (the web pages this method comes from):
 *   [Carat]  "Announcing Carat: An inference engine designed for Gemma 4"
 *            sections "Replacing page lookups with a ring buffer",
 *            "More FLOPs can be faster" (the qk_matmul / causal_softmax /
 *            pv_matmul code block), "Doing it all in one kernel can be slower".
 *   [Gaudi]  "Improving Decode Throughput on Intel Gaudi 3"
 *            sections "Patching sliding window KV allocation", "Our approach".
 *   [Thor]   "gemma-cuda-hybrid" README, section "Features" (GQA shapes,
 *            FP8 e4m3 KV cache).
 *
 * Arithmetic is IEEE binary64 throughout (compile with -ffp-contract=off and
 * without -ffast-math so that the result does not depend on the host).
 * Every sum runs in a fixed, stated order.
 *
 * Readings of points the pages leave open (each also listed in the design
 * notes of the repository):
 *   R1 window: a query at position p sees keys at positions p-W+1 .. p
 *      (W keys including itself) [Gaudi "Patching..."; Carat ring section].
 *   R2 GQA map: query head h reads KV head h / G (contiguous groups of G)
 *      [Carat "Doing it all..."; Thor "Features"].
 *   R3 softmax: exact softmax, no soft-capping, no sinks; masked keys get
 *      weight exactly 0 [Carat code block, causal_softmax].
 *   R4 global padding: the contraction runs over pad64(key_count) keys; the
 *      tail is masked, so it adds exact zeros when it holds finite values
 *      [Carat "More FLOPs can be faster"].
 *   R5 sliding verify: the ring holds committed positions < p0; the S
 *      proposals come in a separate buffer; row i (position p0+i) sees ring
 *      keys with position >= p0+i-W+1 and proposals 0..i.
 *   R6 fp8: OCP E4M3FN (bias 7, no infinities, S.1111.111 is NaN, max 448);
 *      a stored code is round-to-nearest-even of the exact quotient x/scale,
 *      saturating to +-448; element value = decode(code) * scale
 *      [Thor "Features": FP8 (e4m3) KV cache].
 *
 * Regions.  The oracle computes on logical regions: request b's K (or V)
 * region of `cap` slots is element (s, g, d) at element index
 * (s*Hkv + g)*D + d from its byte offset, an element being a bf16 bit
 * pattern (2 bytes) or an E4M3 code (1 byte).  Nothing here knows how the
 * GPU library lays a region out in device memory: that byte layout is a
 * separate codec (swr_layout.c), used only to move regions between the two
 * forms.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_BF16 0
#define ORC_FP8 1

#define ORC_OK 0
#define ORC_EINVAL (-1)
#define ORC_ENOMEM (-2)

/* ------------------------------------------------------------------ */
/* Scalar formats                                                      */
/* ------------------------------------------------------------------ */

/* bf16 is the upper 16 bits of an IEEE binary32: widening is exact. */
double orc_bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP E4M3FN decode (R6): sign | 4-bit exponent (bias 7) | 3-bit mantissa.
 * Exponent field 0 encodes subnormals m * 2^-9; 0x7F / 0xFF are NaN. */
double orc_e4m3_value(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double mag;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    mag = ldexp((double)m, -9);
  else
    mag = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -mag : mag;
}

/* Encode one bf16 value with a per-tensor scale (R6).
 * v = |x| / scale is formed in binary64.  x has 8 significant bits and the
 * scale 24, so x/scale cannot sit within 2^-37 (relative) of an E4M3
 * rounding midpoint without equalling it: the binary64 quotient rounds to
 * the same code as the exact quotient.
 * The nearest code is found by searching the ordered table of the 127
 * non-negative finite codes (0x00..0x7E increase in value); ties go to the
 * even code (even mantissa).  NaN keeps its sign and becomes 0x7F. */
uint8_t orc_e4m3_encode(uint16_t x_bits, float scale) {
  double x = orc_bf16_value(x_bits);
  uint8_t sign = signbit(x) ? 0x80 : 0x00;
  if (isnan(x)) return (uint8_t)(sign | 0x7F);
  double v = fabs(x) / (double)scale;
  if (v >= 448.0) return (uint8_t)(sign | 0x7E); /* saturate */
  int lo = 0, hi = 0x7E; /* largest code whose value is <= v */
  while (lo < hi) {
    int mid = (lo + hi + 1) / 2;
    if (orc_e4m3_value((uint8_t)mid) <= v)
      lo = mid;
    else
      hi = mid - 1;
  }
  double a = orc_e4m3_value((uint8_t)lo);
  double b = orc_e4m3_value((uint8_t)(lo + 1)); /* lo < 0x7E here */
  double da = v - a, db = b - v;                 /* both exact (Sterbenz) */
  int code;
  if (da < db)
    code = lo;
  else if (db < da)
    code = lo + 1;
  else
    code = (lo % 2 == 0) ? lo : lo + 1;
  return (uint8_t)(sign | code);
}

/* ------------------------------------------------------------------ */
/* Logical regions                                                     */
/* ------------------------------------------------------------------ */

static int elem_size(int dtype) { return dtype == ORC_FP8 ? 1 : 2; }

/* Element index of (slot s, KV head g, dim d) in a logical region. */
static size_t elem_index(int64_t s, int g, int d, int Hkv, int D) {
  return (size_t)((s * Hkv + g) * D + d);
}

/* Bytes of one logical K (or V) region of `cap` slots. */
int64_t orc_logical_region_bytes(int cap, int Hkv, int D, int dtype) {
  if (cap <= 0 || Hkv <= 0 || D <= 0 || (dtype != ORC_BF16 && dtype != ORC_FP8)) return -1;
  return (int64_t)cap * Hkv * D * elem_size(dtype);
}

static double read_elem(const uint8_t* region, size_t idx, int dtype, double scale) {
  if (dtype == ORC_FP8) return orc_e4m3_value(region[idx]) * scale;
  uint16_t b;
  memcpy(&b, region + 2 * idx, 2);
  return orc_bf16_value(b);
}

static void write_elem(uint8_t* region, size_t idx, int dtype, float scale, uint16_t x) {
  if (dtype == ORC_FP8)
    region[idx] = orc_e4m3_encode(x, scale);
  else
    memcpy(region + 2 * idx, &x, 2);
}

/* ------------------------------------------------------------------ */
/* Append (a token's K and V go to the same slot)                      */
/* ------------------------------------------------------------------ */

/* Slots of request b's region: caps[b] when a per-request array is given
 * (global regions), else cap. */
static int64_t region_cap(int cap, const int32_t* caps, int b) { return caps ? caps[b] : cap; }

/* Appends tokens t = 0 .. n_new[b]-1 of request b (n_new == NULL: T) at
 * positions pos0[b] + t, one after another.  wrap != 0: slot = pos mod cap
 * (ring [Carat ring section; Gaudi "Our approach"]); wrap == 0: slot = pos,
 * which must be < the region's capacity (contiguous global region).  A later
 * token that maps to the same slot overwrites an earlier one, as sequential
 * appends would.  caps (global regions only, may be NULL): per-request
 * capacities.  k_new / v_new: bf16 bits [B][T][Hkv][D]. */
int orc_kv_append(uint8_t* k_base, uint8_t* v_base, const int64_t* k_off, const int64_t* v_off,
                  int cap, const int32_t* caps, int dtype, float k_scale, float v_scale,
                  const uint16_t* k_new, const uint16_t* v_new, const int32_t* pos0,
                  const int32_t* n_new, int B, int T, int Hkv, int D, int wrap) {
  if (cap <= 0 || B < 0 || T < 0 || Hkv <= 0 || D <= 0) return ORC_EINVAL;
  if (wrap && caps) return ORC_EINVAL;
  for (int b = 0; b < B; ++b) {
    int n = n_new ? n_new[b] : T;
    int64_t cb = region_cap(cap, caps, b);
    if (n < 0 || n > T || pos0[b] < 0 || cb <= 0) return ORC_EINVAL;
    if (!wrap && (int64_t)pos0[b] + n > cb) return ORC_EINVAL;
  }
  for (int b = 0; b < B; ++b) {
    int n = n_new ? n_new[b] : T;
    int64_t cb = region_cap(cap, caps, b);
    uint8_t* kr = k_base + k_off[b];
    uint8_t* vr = v_base + v_off[b];
    for (int t = 0; t < n; ++t) {
      int64_t p = (int64_t)pos0[b] + t;
      int64_t s = wrap ? p % cb : p;
      for (int g = 0; g < Hkv; ++g)
        for (int d = 0; d < D; ++d) {
          size_t src = (((size_t)b * T + t) * Hkv + g) * D + d;
          write_elem(kr, elem_index(s, g, d, Hkv, D), dtype, k_scale, k_new[src]);
          write_elem(vr, elem_index(s, g, d, Hkv, D), dtype, v_scale, v_new[src]);
        }
    }
  }
  return ORC_OK;
}

/* ------------------------------------------------------------------ */
/* Attention over one (request, KV head) unit                          */
/* ------------------------------------------------------------------ */

/* A key the unit may read: either a slot of the region or one of the
 * separately passed proposal rows. */
typedef struct {
  int64_t slot;  /* >= 0: region slot; < 0: proposal index -(slot+1) */
  int64_t pos;   /* absolute position of the key */
} key_ref;

typedef struct {
  const uint8_t* kr;
  const uint8_t* vr;
  int dtype;
  double k_scale, v_scale;
  const uint16_t* k_prop; /* [S][Hkv][D] for this request, or NULL */
  const uint16_t* v_prop;
  int g, Hkv, D;
} unit_src;

static void load_key(const unit_src* u, key_ref kr, double* kd, double* vd) {
  for (int d = 0; d < u->D; ++d) {
    if (kr.slot >= 0) {
      kd[d] = read_elem(u->kr, elem_index(kr.slot, u->g, d, u->Hkv, u->D), u->dtype, u->k_scale);
      vd[d] = read_elem(u->vr, elem_index(kr.slot, u->g, d, u->Hkv, u->D), u->dtype, u->v_scale);
    } else {
      int64_t i = -(kr.slot + 1);
      size_t idx = ((size_t)i * u->Hkv + u->g) * u->D + d;
      kd[d] = orc_bf16_value(u->k_prop[idx]);
      vd[d] = orc_bf16_value(u->v_prop[idx]);
    }
  }
}

/* rows: number of query rows; q: [rows][D] (binary64); lo/hi: per row, the
 * visible key positions are lo[r] <= pos <= hi[r].  Keys are visited in the
 * given order for every sum.  Softmax is the two-pass definition: the row
 * maximum first, then weights exp(s - max) (exactly 0 for masked keys), the
 * weight sum l, and out = (sum_k w_k v_k) / l. */
static int attend_unit(const unit_src* u, const key_ref* keys, int nk, int rows, const double* q,
                       const int64_t* lo, const int64_t* hi, double scale, double* out) {
  int D = u->D;
  double* s = (double*)malloc(sizeof(double) * (size_t)rows * (nk > 0 ? nk : 1));
  double* kd = (double*)malloc(sizeof(double) * D);
  double* vd = (double*)malloc(sizeof(double) * D);
  double* acc = (double*)calloc((size_t)rows * D, sizeof(double));
  double* m = (double*)malloc(sizeof(double) * rows);
  double* l = (double*)calloc(rows, sizeof(double));
  if (!s || !kd || !vd || !acc || !m || !l) {
    free(s); free(kd); free(vd); free(acc); free(m); free(l);
    return ORC_ENOMEM;
  }
  /* scores: s = scale * (q . k), dot product in ascending d */
  for (int k = 0; k < nk; ++k) {
    load_key(u, keys[k], kd, vd);
    for (int r = 0; r < rows; ++r) {
      int vis = keys[k].pos >= lo[r] && keys[k].pos <= hi[r];
      if (!vis) {
        s[(size_t)r * nk + k] = -INFINITY;
        continue;
      }
      double dot = 0.0;
      for (int d = 0; d < D; ++d) dot += q[(size_t)r * D + d] * kd[d];
      s[(size_t)r * nk + k] = scale * dot;
    }
  }
  for (int r = 0; r < rows; ++r) {
    m[r] = -INFINITY;
    for (int k = 0; k < nk; ++k)
      if (s[(size_t)r * nk + k] > m[r]) m[r] = s[(size_t)r * nk + k];
  }
  /* weights, their sum, and the weighted sum of values, in key order */
  for (int k = 0; k < nk; ++k) {
    load_key(u, keys[k], kd, vd);
    for (int r = 0; r < rows; ++r) {
      double sc = s[(size_t)r * nk + k];
      double w = (sc == -INFINITY) ? 0.0 : exp(sc - m[r]);
      l[r] += w;
      for (int d = 0; d < D; ++d) acc[(size_t)r * D + d] += w * vd[d];
    }
  }
  for (int r = 0; r < rows; ++r)
    for (int d = 0; d < D; ++d)
      out[(size_t)r * D + d] = (l[r] > 0.0) ? acc[(size_t)r * D + d] / l[r] : 0.0;
  free(s); free(kd); free(vd); free(acc); free(m); free(l);
  return ORC_OK;
}

/* Query rows of a unit: row r = i*G + h (proposal i, head h of the group),
 * query head g*G + h.  q: bf16 bits [B][S][Hq][D]. */
static void gather_q(const uint16_t* q, int b, int g, int S, int Hq, int G, int D, double* qd) {
  for (int i = 0; i < S; ++i)
    for (int h = 0; h < G; ++h)
      for (int d = 0; d < D; ++d)
        qd[((size_t)i * G + h) * D + d] =
            orc_bf16_value(q[(((size_t)b * S + i) * Hq + (size_t)g * G + h) * D + d]);
}

static void scatter_out(double* out, const double* od, int b, int g, int S, int Hq, int G, int D) {
  for (int i = 0; i < S; ++i)
    for (int h = 0; h < G; ++h)
      for (int d = 0; d < D; ++d)
        out[(((size_t)b * S + i) * Hq + (size_t)g * G + h) * D + d] =
            od[((size_t)i * G + h) * D + d];
}

/* Position held by ring slot s when the newest committed position is
 * `last` (slot = pos mod W): the largest p <= last with p = s (mod W). */
static int64_t ring_slot_pos(int64_t s, int64_t last, int W) {
  return last - (((last - s) % W) + W) % W;
}

static int check_common(int B, int S, int Hq, int Hkv, int D) {
  if (B < 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || D <= 0 || Hq % Hkv != 0) return ORC_EINVAL;
  return ORC_OK;
}

/* Sliding-window decode (one query token per request) [Carat ring section;
 * Gaudi "Our approach"]: the token at pos[b] is already in the ring.  The
 * ring is read in storage order (slot 0 first) with no un-rotation. */
int orc_swa_decode(const uint8_t* k_base, const uint8_t* v_base, const int64_t* k_off,
                   const int64_t* v_off, int W, int dtype, double k_scale, double v_scale,
                   const uint16_t* q, const int32_t* pos, int B, int Hq, int Hkv, int D,
                   double scale, double* out) {
  if (check_common(B, 1, Hq, Hkv, D) || W <= 0) return ORC_EINVAL;
  for (int b = 0; b < B; ++b)
    if (pos[b] < 0) return ORC_EINVAL;
  int G = Hq / Hkv, rc = ORC_OK;
#pragma omp parallel for schedule(dynamic)
  for (int un = 0; un < B * Hkv; ++un) {
    int b = un / Hkv, g = un % Hkv;
    int64_t p = pos[b];
    int nk = (int)(p + 1 < W ? p + 1 : W); /* slots ever written */
    unit_src u = {k_base + k_off[b], v_base + v_off[b], dtype, k_scale, v_scale, NULL, NULL, g, Hkv, D};
    key_ref* keys = (key_ref*)malloc(sizeof(key_ref) * nk);
    double* qd = (double*)malloc(sizeof(double) * (size_t)G * D);
    double* od = (double*)malloc(sizeof(double) * (size_t)G * D);
    int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * G);
    int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * G);
    int r = ORC_ENOMEM;
    if (keys && qd && od && lo && hi) {
      for (int s = 0; s < nk; ++s) keys[s] = (key_ref){s, ring_slot_pos(s, p, W)};
      for (int h = 0; h < G; ++h) {
        lo[h] = p - W + 1 > 0 ? p - W + 1 : 0; /* R1 */
        hi[h] = p;
      }
      gather_q(q, b, g, 1, Hq, G, D, qd);
      r = attend_unit(&u, keys, nk, G, qd, lo, hi, scale, od);
      if (r == ORC_OK) scatter_out(out, od, b, g, 1, Hq, G, D);
    }
    if (r != ORC_OK) {
#pragma omp atomic write
      rc = r;
    }
    free(keys); free(qd); free(od); free(lo); free(hi);
  }
  return rc;
}

/* Speculative verify on a sliding layer (R5) [Carat "Doing it all in one
 * kernel can be slower": the G query heads of a KV head times the S proposed
 * positions form G*S rows against the same keys].  The ring holds positions
 * < pos0[b]; proposals i = 0..S-1 sit at positions pos0[b]+i in k_prop/v_prop
 * (bf16 bits [B][S][Hkv][D]).  Keys are visited ring slots first (storage
 * order), then proposals 0..S-1. */
int orc_gqa_verify(const uint8_t* k_base, const uint8_t* v_base, const int64_t* k_off,
                   const int64_t* v_off, int W, int dtype, double k_scale, double v_scale,
                   const uint16_t* k_prop, const uint16_t* v_prop, const uint16_t* q,
                   const int32_t* pos0, int B, int S, int Hq, int Hkv, int D, double scale,
                   double* out) {
  if (check_common(B, S, Hq, Hkv, D) || W <= 0) return ORC_EINVAL;
  for (int b = 0; b < B; ++b)
    if (pos0[b] < 0) return ORC_EINVAL;
  int G = Hq / Hkv, rows = G * S, rc = ORC_OK;
#pragma omp parallel for schedule(dynamic)
  for (int un = 0; un < B * Hkv; ++un) {
    int b = un / Hkv, g = un % Hkv;
    int64_t p0 = pos0[b];
    int nr = (int)(p0 < W ? p0 : W); /* committed ring slots */
    int nk = nr + S;
    unit_src u = {k_base + k_off[b], v_base + v_off[b], dtype, k_scale, v_scale,
                  k_prop + (size_t)b * S * Hkv * D, v_prop + (size_t)b * S * Hkv * D, g, Hkv, D};
    key_ref* keys = (key_ref*)malloc(sizeof(key_ref) * nk);
    double* qd = (double*)malloc(sizeof(double) * (size_t)rows * D);
    double* od = (double*)malloc(sizeof(double) * (size_t)rows * D);
    int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * rows);
    int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * rows);
    int r = ORC_ENOMEM;
    if (keys && qd && od && lo && hi) {
      for (int s = 0; s < nr; ++s) keys[s] = (key_ref){s, ring_slot_pos(s, p0 - 1, W)};
      for (int i = 0; i < S; ++i) keys[nr + i] = (key_ref){-(int64_t)i - 1, p0 + i};
      for (int i = 0; i < S; ++i)
        for (int h = 0; h < G; ++h) {
          int64_t qp = p0 + i;
          lo[i * G + h] = qp - W + 1 > 0 ? qp - W + 1 : 0; /* R1 per row */
          hi[i * G + h] = qp;                              /* causal among proposals */
        }
      gather_q(q, b, g, S, Hq, G, D, qd);
      r = attend_unit(&u, keys, nk, rows, qd, lo, hi, scale, od);
      if (r == ORC_OK) scatter_out(out, od, b, g, S, Hq, G, D);
    }
    if (r != ORC_OK) {
#pragma omp atomic write
      rc = r;
    }
    free(keys); free(qd); free(od); free(lo); free(hi);
  }
  return rc;
}

/* Global-layer attention over a contiguous region [Carat "More FLOPs can be
 * faster": key_count = context + proposals; qk_matmul, causal_softmax with
 * the query positions, pv_matmul].  Key j sits in slot j.  Row (i, h) with
 * query position q_pos[b][i] sees keys j <= q_pos[b][i], j < key_count[b].
 * padded != 0 (the pages' form, R4): keys are visited over
 * 0 .. pad64(key_count)-1, the tail contributing zero-weight terms;
 * padded == 0: keys 0 .. key_count-1 only.  caps (may be NULL): per-request
 * region capacities, else every region has `cap` slots. */
int orc_global_attend(const uint8_t* k_base, const uint8_t* v_base, const int64_t* k_off,
                      const int64_t* v_off, int cap, const int32_t* caps, int dtype,
                      double k_scale, double v_scale, const uint16_t* q, const int32_t* q_pos,
                      const int32_t* key_count, int padded, int B, int S, int Hq, int Hkv, int D,
                      double scale, double* out) {
  if (check_common(B, S, Hq, Hkv, D) || cap <= 0) return ORC_EINVAL;
  for (int b = 0; b < B; ++b) {
    int64_t kc = key_count[b], kp = padded ? (kc + 63) / 64 * 64 : kc;
    int64_t cb = region_cap(cap, caps, b);
    if (kc <= 0 || kp > cb) return ORC_EINVAL;
    for (int i = 0; i < S; ++i)
      if (q_pos[b * S + i] < 0) return ORC_EINVAL;
  }
  int G = Hq / Hkv, rows = G * S, rc = ORC_OK;
#pragma omp parallel for schedule(dynamic)
  for (int un = 0; un < B * Hkv; ++un) {
    int b = un / Hkv, g = un % Hkv;
    int64_t kc = key_count[b];
    int nk = (int)(padded ? (kc + 63) / 64 * 64 : kc);
    unit_src u = {k_base + k_off[b], v_base + v_off[b], dtype, k_scale, v_scale, NULL, NULL, g, Hkv, D};
    key_ref* keys = (key_ref*)malloc(sizeof(key_ref) * nk);
    double* qd = (double*)malloc(sizeof(double) * (size_t)rows * D);
    double* od = (double*)malloc(sizeof(double) * (size_t)rows * D);
    int64_t* lo = (int64_t*)malloc(sizeof(int64_t) * rows);
    int64_t* hi = (int64_t*)malloc(sizeof(int64_t) * rows);
    int r = ORC_ENOMEM;
    if (keys && qd && od && lo && hi) {
      for (int j = 0; j < nk; ++j) keys[j] = (key_ref){j, j};
      for (int i = 0; i < S; ++i)
        for (int h = 0; h < G; ++h) {
          int64_t qp = q_pos[b * S + i];
          lo[i * G + h] = 0;
          hi[i * G + h] = qp < kc - 1 ? qp : kc - 1;
        }
      gather_q(q, b, g, S, Hq, G, D, qd);
      r = attend_unit(&u, keys, nk, rows, qd, lo, hi, scale, od);
      if (r == ORC_OK) scatter_out(out, od, b, g, S, Hq, G, D);
    }
    if (r != ORC_OK) {
#pragma omp atomic write
      rc = r;
    }
    free(keys); free(qd); free(od); free(lo); free(hi);
  }
  return rc;
}

/* Threads the parallel loops above will use. */
int orc_num_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

/* Sets the threads of the parallel loops (n >= 1, for timing on fewer
 * cores); returns the previous count.  Results do not depend on it: every
 * unit is computed by one thread in a fixed order. */
int orc_set_threads(int n) {
#ifdef _OPENMP
  const int prev = omp_get_max_threads();
  if (n >= 1) omp_set_num_threads(n);
  return prev;
#else
  (void)n;
  return 1;
#endif
}

/* Array forms of the scalar codecs, for the test suite. */
void orc_bf16_value_n(const uint16_t* x, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_value(x[i]);
}

void orc_e4m3_value_n(const uint8_t* x, int64_t n, double* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_value(x[i]);
}

void orc_e4m3_encode_n(const uint16_t* x, int64_t n, float scale, uint8_t* out) {
  for (int64_t i = 0; i < n; ++i) out[i] = orc_e4m3_encode(x[i], scale);
}
