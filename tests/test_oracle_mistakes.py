"""Planted mistakes: each case edits one plausible mistake into a copy of the
oracle source, builds it, and checks that at least one pin fails against it.
This is the evidence that the pins constrain the oracle (a pin that passes
for a broken oracle would prove nothing).  Runs on the CPU only.
"""
import os

import pytest

import oracle
import test_oracle_attention as att
import test_oracle_formats as fmt
import test_oracle_ring as ring

ORACLE_DIR = os.path.dirname(oracle.__file__)
SRC = {f: open(os.path.join(ORACLE_DIR, f)).read() for f in oracle.SOURCES}
ARITH, LAYOUT = "swr_oracle.c", "swr_layout.c"

# (name, source file, original snippet, planted mistake)
MISTAKES = [
    ("e4m3 exponent bias 8", ARITH, "ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    ("e4m3 subnormal scale", ARITH, "mag = ldexp((double)m, -9);", "mag = ldexp((double)m, -10);"),
    ("e4m3 ties away from zero", ARITH, "code = (lo % 2 == 0) ? lo : lo + 1;", "code = lo + 1;"),
    ("e4m3 ties truncate", ARITH, "code = (lo % 2 == 0) ? lo : lo + 1;", "code = lo;"),
    ("encode divides by scale twice", ARITH, "double v = fabs(x) / (double)scale;",
     "double v = fabs(x) / (double)scale / (double)scale;"),
    ("logical index drops the KV head", ARITH, "return (size_t)((s * Hkv + g) * D + d);",
     "return (size_t)(s * D + d);"),
    ("V region not blocked", LAYOUT, "return (((int64_t)g * (S / 8) + s / 8) * D + d) * 8 + s % 8;",
     "return ((int64_t)g * S + s) * D + d;"),
    ("K tile rows in slot order", LAYOUT, "const int64_t half = (k / 4) % 2, row = 4 * (k / 8) + k % 4;",
     "const int64_t half = k / 16, row = k % 16;"),
    ("K granule ignores the element size", LAYOUT, "const int64_t R = 16 / esize_of(dtype);",
     "const int64_t R = 8;"),
    ("K granules not grouped by row", LAYOUT, "(q / 4) * 64 * R + row * 4 * R + (q % 4) * R + d % R",
     "q * 16 * R + row * R + d % R"),
    ("K head stride ignores the tile padding", LAYOUT, "return ((int64_t)g * S + 32 * t) * D + half * 16 * D",
     "return ((int64_t)g * cap + 32 * t) * D + half * 16 * D"),
    ("V packed in the K layout", LAYOUT,
     "const int64_t dst = is_v ? v_elem(s, g, d, cap, D) : k_elem(s, g, d, cap, D, dtype);",
     "const int64_t dst = k_elem(s, g, d, cap, D, dtype);"),
    ("append slot off by one", ARITH, "int64_t s = wrap ? p % cb : p;", "int64_t s = wrap ? (p + 1) % cb : p;"),
    ("dot product drops the last dim", ARITH, "for (int d = 0; d < D; ++d) dot += q[(size_t)r * D + d] * kd[d];",
     "for (int d = 0; d < D - 1; ++d) dot += q[(size_t)r * D + d] * kd[d];"),
    ("score scale missing", ARITH, "s[(size_t)r * nk + k] = scale * dot;", "s[(size_t)r * nk + k] = dot;"),
    ("weight sum counts keys", ARITH, "l[r] += w;", "l[r] += (w > 0.0) ? 1.0 : 0.0;"),
    ("GQA heads interleaved", ARITH,
     "orc_bf16_value(q[(((size_t)b * S + i) * Hq + (size_t)g * G + h) * D + d]);",
     "orc_bf16_value(q[(((size_t)b * S + i) * Hq + (size_t)h * (Hq / G) + g) * D + d]);"),
    ("verify window one key too wide", ARITH, "lo[i * G + h] = qp - W + 1 > 0 ? qp - W + 1 : 0; /* R1 per row */",
     "lo[i * G + h] = qp - W > 0 ? qp - W : 0;"),
    ("verify not causal among proposals", ARITH, "hi[i * G + h] = qp;                              /* causal among proposals */",
     "hi[i * G + h] = p0 + S - 1;"),
    ("proposal positions shifted", ARITH, "keys[nr + i] = (key_ref){-(int64_t)i - 1, p0 + i};",
     "keys[nr + i] = (key_ref){-(int64_t)i - 1, p0 + i + 1};"),
    ("ring slot position ignores wrap", ARITH, "return last - (((last - s) % W) + W) % W;",
     "return s + (last / W) * W;"),
    ("global mask not causal", ARITH, "hi[i * G + h] = qp < kc - 1 ? qp : kc - 1;", "hi[i * G + h] = kc - 1;"),
    ("global mask one key late", ARITH, "hi[i * G + h] = qp < kc - 1 ? qp : kc - 1;",
     "hi[i * G + h] = qp + 1 < kc - 1 ? qp + 1 : kc - 1;"),
    ("decode reads one slot short", ARITH, "int nk = (int)(p + 1 < W ? p + 1 : W); /* slots ever written */",
     "int nk = (int)(p < W ? p : W);"),
]

CHECKS = [
    fmt.test_e4m3_decode_matches_torch_all_codes,
    fmt.test_e4m3_landmarks,
    lambda: fmt.test_e4m3_encode_matches_torch_power_of_two_scales(2.0 ** -4),
    fmt.test_e4m3_encode_exact_rational_brute_force,
    fmt.test_e4m3_encode_ties_to_even,
    fmt.test_e4m3_round_trip_all_finite_codes,
    ring.test_slot_is_position_mod_window_one_by_one,
    ring.test_fp8_append_stores_encoded_codes,
    *[lambda a=a: ring.test_codec_unpack_matches_layout_views(*a) for a in ring.CODEC_SHAPES],
    *[lambda a=a: ring.test_codec_round_trips(*a) for a in ring.CODEC_SHAPES],
    *att.ALL_CHECKS,
]


def test_every_mistake_snippet_is_present_once():
    for name, f, orig, _ in MISTAKES:
        assert SRC[f].count(orig) == 1, name


def test_unmodified_source_passes_all_checks():
    for c in CHECKS:
        c()


def test_arithmetic_holds_no_layout():
    # the device byte layout lives in the codec alone: the attention
    # arithmetic reads logical [slot][Hkv][D] regions
    for word in ("S / 8", "/ 32", "granule", "half", "1024"):
        assert word not in SRC[ARITH].split("#include")[1], word


@pytest.mark.parametrize("name,f,orig,bad", MISTAKES, ids=[m[0] for m in MISTAKES])
def test_planted_mistake_is_caught(name, f, orig, bad, tmp_path):
    path = oracle.build_variant(f, SRC[f].replace(orig, bad), str(tmp_path))
    caught = None
    with oracle.use_library(path):
        for c in CHECKS:
            try:
                c()
            except (AssertionError, ValueError) as e:  # a pin failed
                caught = (getattr(c, "__name__", "check"), e)
                break
    assert caught is not None, f"no pin catches: {name}"
