"""CPU tests of the C ABI: the library loads, exports every function the
header declares, and rejects invalid arguments before touching the GPU.

No call here reaches a HIP runtime function: each one fails host-side
validation first (the header promises validation precedes any launch), so
these run without a GPU.
"""
import ctypes
import os
import re

import pytest

import sliding_window_ring_amd as swr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = open(os.path.join(ROOT, "include", "swr.h")).read()

OK, INVALID, UNSUPPORTED, WORKSPACE, LAUNCH, NOMEM = range(6)
FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def declared_functions():
    body = re.sub(r"/\*.*?\*/", "", HEADER, flags=re.S)
    return sorted(set(re.findall(r"\b(swr_[a-z0-9_]+)\s*\(", body)))


# The boundary's calls by the names the hot path's step list gives them
# (ring append, sliding decode, grouped verify, global attention, workspace
# sizing, status text) and the shared pool's carves, plus the two fused calls.
BOUNDARY = ["swr_ring_kv_append", "swr_swa_decode", "swr_gqa_verify", "swr_global_attend",
            "swr_workspace_bytes", "swr_status_string", "swr_pool_create", "swr_pool_alloc_ring",
            "swr_pool_alloc_global", "swr_pool_free", "swr_pool_destroy",
            "swr_swa_append_decode", "swr_global_append_attend"]


def test_header_declares_the_boundary_calls():
    names = declared_functions()
    for n in BOUNDARY:
        assert n in names, n


def test_library_exports_the_boundary_calls():
    lib = ctypes.CDLL(swr.LIB_PATH)
    for n in BOUNDARY:
        assert hasattr(lib, n), n


def test_library_exports_every_declared_function():
    lib = ctypes.CDLL(swr.LIB_PATH)
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing
    assert sorted(swr.EXPORTS) == declared_functions()


def test_status_strings():
    for s in range(6):
        assert swr.lib.swr_status_string(s).decode() == swr.STATUS[s]


def kv(cap=1024, dtype=0, k_scale=1.0, v_scale=1.0, base=FAKE):
    return swr.SwrKV(base, base, FAKE, FAKE, None, cap, dtype, k_scale, v_scale)


def decode(k=None, q=FAKE, out=FAKE, pos=FAKE, B=56, Hq=64, Hkv=8, D=256, scale=0.0625, ws=None, wsb=0):
    r = kv() if k is None else k
    return swr.lib.swr_swa_decode(ctypes.byref(r), q, out, pos, B, Hq, Hkv, D, scale, ws, wsb, None)


def test_decode_validation():
    assert decode(q=None) == INVALID
    assert decode(out=None) == INVALID
    assert decode(pos=None) == INVALID
    assert decode(q=FAKE + 2) == INVALID           # misaligned
    assert decode(Hq=60) == INVALID                # not a multiple of Hkv
    assert decode(B=-1) == INVALID
    assert decode(D=96) == UNSUPPORTED
    assert decode(Hq=8 * 32) == UNSUPPORTED        # 32 query heads per KV head
    assert decode(k=kv(cap=1004)) == INVALID       # cap not a multiple of 8
    assert decode(k=kv(cap=0)) == INVALID
    assert decode(k=kv(dtype=7)) == INVALID
    assert decode(k=kv(dtype=1, k_scale=0.0)) == INVALID
    assert decode(k=kv(dtype=1, v_scale=float("nan"))) == INVALID
    assert decode(k=kv(base=FAKE + 8)) == INVALID
    assert decode(scale=float("inf")) == INVALID
    assert swr.lib.swr_swa_decode(None, FAKE, FAKE, FAKE, 1, 8, 1, 64, 1.0, None, 0, None) == INVALID
    assert decode(k=kv(cap=1 << 22)) == UNSUPPORTED  # region beyond 32-bit offsets
    withcaps = kv()
    withcaps.cap_b = FAKE
    assert decode(k=withcaps) == INVALID           # rings share one window


def test_decode_small_batch_needs_workspace():
    # 16 requests x 8 KV heads fill half the chip: split-K needs a workspace
    need = swr.workspace_bytes(swr.SWR_OP_SWA_DECODE, 16, 1, 64, 8, 256, 1024)
    assert need > 0
    assert decode(B=16) == WORKSPACE
    assert decode(B=16, ws=FAKE, wsb=need - 1) == WORKSPACE
    assert swr.workspace_bytes(swr.SWR_OP_SWA_DECODE, 56, 1, 64, 8, 256, 1024) == 0


def test_verify_and_global_validation():
    r = kv()
    f = swr.lib.swr_gqa_verify
    assert f(ctypes.byref(r), None, FAKE, FAKE, FAKE, FAKE, 8, 4, 64, 8, 256, 0.06, None, 0, None) == INVALID
    assert f(ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, FAKE, 8, 9, 64, 8, 256, 0.06, None, 0, None) == UNSUPPORTED
    assert f(ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, FAKE, 8, 4, 128, 8, 256, 0.06, None, 0, None) == UNSUPPORTED
    assert f(ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, FAKE, 8, 4, 64, 8, 256, 0.06, None, 0, None) == WORKSPACE
    g = swr.lib.swr_global_attend
    rg = kv(cap=6016)
    assert g(ctypes.byref(rg), FAKE, FAKE, FAKE, None, 6005, 1, 4, 16, 2, 512, 0.04, None, 0, None) == INVALID
    assert g(ctypes.byref(rg), FAKE, FAKE, FAKE, FAKE, 6017, 1, 4, 16, 2, 512, 0.04, None, 0, None) == INVALID
    assert g(ctypes.byref(rg), FAKE, FAKE, FAKE, FAKE, 0, 1, 4, 16, 2, 512, 0.04, None, 0, None) == INVALID
    assert g(ctypes.byref(rg), FAKE, FAKE, FAKE, FAKE, 6005, 1, 4, 16, 2, 512, 0.04, None, 0, None) == WORKSPACE
    # a key bound near INT32_MAX is past the region, not an overflow
    assert g(ctypes.byref(rg), FAKE, FAKE, FAKE, FAKE, 2**31 - 1, 1, 4, 16, 2, 512, 0.04, None, 0, None) == INVALID


def test_regions_past_32_bit_offsets_are_unsupported():
    # capacities whose regions pass 4 GiB (the kernels address a region with
    # 32-bit offsets), up to INT32_MAX with no overflow on the way
    g = swr.lib.swr_global_attend
    for cap in (2_097_152, 2**31 - 8):
        r = kv(cap=cap)
        assert g(ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, 6005, 1, 4, 16, 2, 512, 0.04, None, 0, None) == UNSUPPORTED
    r = kv(cap=2_097_120)  # just under 4 GiB at 2 KV heads x 512 bf16
    assert g(ctypes.byref(r), FAKE, FAKE, FAKE, FAKE, 6005, 1, 4, 16, 2, 512, 0.04, None, 0, None) == WORKSPACE


def test_fused_append_decode_validation():
    f = swr.lib.swr_swa_append_decode

    def call(k=None, kn=FAKE, vn=FAKE, q=FAKE, out=FAKE, pos=FAKE, B=56, Hq=64, Hkv=8, D=256, ws=None, wsb=0):
        r = kv() if k is None else k
        return f(ctypes.byref(r), kn, vn, q, out, pos, B, Hq, Hkv, D, 0.0625, ws, wsb, None)

    assert call(kn=None) == INVALID
    assert call(vn=None) == INVALID
    assert call(vn=FAKE + 2) == INVALID            # misaligned
    assert call(pos=None) == INVALID
    assert call(D=96) == UNSUPPORTED
    withcaps = kv()
    withcaps.cap_b = FAKE
    assert call(k=withcaps) == INVALID             # rings share one window
    need = swr.workspace_bytes(swr.SWR_OP_SWA_APPEND_DECODE, 16, 1, 64, 8, 256, 1024)
    assert need == swr.workspace_bytes(swr.SWR_OP_SWA_DECODE, 16, 1, 64, 8, 256, 1024) > 0
    assert call(B=16) == WORKSPACE
    assert call(B=0) == OK


def test_fused_global_append_validation():
    g = swr.lib.swr_global_append_attend
    rg = kv(cap=6016)

    def call(kn=FAKE, vn=FAKE, pos0=FAKE, mk=6005, S=4, Hq=16, ws=None, wsb=0):
        return g(ctypes.byref(rg), kn, vn, FAKE, FAKE, pos0, mk, 1, S, Hq, 2, 512, 0.04, ws, wsb, None)

    assert call(kn=None) == INVALID
    assert call(vn=FAKE + 8) == INVALID
    assert call(pos0=None) == INVALID
    assert call(mk=3) == INVALID                   # fewer keys than the tokens it appends
    assert call(mk=6017) == INVALID                # padded contraction past the capacity
    assert call(S=9) == UNSUPPORTED
    need = swr.workspace_bytes(swr.SWR_OP_GLOBAL_APPEND_ATTEND, 1, 4, 16, 2, 512, 6005)
    assert need > 0
    assert call() == WORKSPACE
    # the size covers both element types; the fp8 form needs all of it
    r8 = kv(cap=6016, dtype=1, k_scale=0.01, v_scale=0.01)
    assert g(ctypes.byref(r8), FAKE, FAKE, FAKE, FAKE, FAKE, 6005, 1, 4, 16, 2, 512, 0.04, FAKE, need - 1,
             None) == WORKSPACE


def test_append_validation():
    r = kv()
    f = swr.lib.swr_ring_kv_append
    assert f(ctypes.byref(r), FAKE, FAKE, FAKE, None, 56, 0, 8, 256, 1, None) == INVALID   # T == 0
    assert f(ctypes.byref(r), None, FAKE, FAKE, None, 56, 1, 8, 256, 1, None) == INVALID
    assert f(ctypes.byref(r), FAKE, FAKE, None, None, 56, 1, 8, 256, 1, None) == INVALID
    assert f(ctypes.byref(r), FAKE, FAKE, FAKE, None, 56, 1, 8, 200, 1, None) == UNSUPPORTED
    assert f(None, FAKE, FAKE, FAKE, None, 56, 1, 8, 256, 1, None) == INVALID
    # B == 0 is a valid no-op that launches nothing
    assert f(ctypes.byref(r), FAKE, FAKE, FAKE, None, 0, 1, 8, 256, 1, None) == OK


def test_read_ceiling_validation():
    f = swr.lib.swr_read_ceiling
    assert f(FAKE, 1 << 20, FAKE, 0, 0, None) == INVALID       # grid out of range
    assert f(FAKE, 1 << 20, FAKE, 65537, 1, None) == INVALID
    assert f(FAKE, 1 << 20, FAKE, 256, 2, None) == INVALID     # no such pattern
    assert f(FAKE, (1 << 20) + 8, FAKE, 256, 0, None) == INVALID  # not whole 16-byte words
    assert f(FAKE + 8, 1 << 20, FAKE, 256, 0, None) == INVALID  # misaligned
    assert f(None, 1 << 20, FAKE, 256, 0, None) == INVALID
    assert f(FAKE, 1 << 20, None, 256, 0, None) == INVALID
    assert f(FAKE, 0, FAKE, 256, 0, None) == OK                 # nothing to read, no launch


def gather(ring=None, kp=FAKE, vp=FAKE, n_pages=4096, pt=16, bt=FAKE, max_pages=257, pos=FAKE, B=56, Hkv=8,
           D=256):
    r = kv() if ring is None else ring
    return swr.lib.swr_paged_gather_window(kp, vp, n_pages, pt, bt, max_pages, pos, ctypes.byref(r), B, Hkv, D,
                                           None)


def test_paged_gather_validation():
    for bad in (dict(kp=None), dict(vp=None), dict(bt=None), dict(pos=None), dict(kp=FAKE + 8),
                dict(vp=FAKE + 2), dict(n_pages=0), dict(pt=0), dict(max_pages=0), dict(B=-1), dict(Hkv=0)):
        assert gather(**bad) == INVALID, bad
    assert gather(D=96) == UNSUPPORTED
    assert gather(ring=kv(dtype=1)) == UNSUPPORTED         # bf16 rings only
    assert gather(ring=kv(cap=1020)) == INVALID            # window not a multiple of 8
    r = kv()
    r.cap_b = FAKE
    assert gather(ring=r) == INVALID                       # rings share one window
    assert swr.lib.swr_paged_gather_window(FAKE, FAKE, 4096, 16, FAKE, 257, FAKE, None, 56, 8, 256,
                                           None) == INVALID
    assert gather(B=0) == OK                               # nothing to gather, no launch


def test_zero_batch_attention_is_a_no_op():
    assert decode(B=0) == OK


def test_verify_workspace_is_one_partial_per_256_ring_keys():
    # B=8 x 8 KV heads, W=1024: 4 ring chunks of 256 keys per unit (the
    # first also takes the proposals), 32 rows of 256 fp32 dims each, plus a
    # (max, sum) per row
    units, chunks, rows, d = 8 * 8, 1024 // 256, 8 * 4, 256
    want = units * chunks * rows * d * 4 + units * chunks * rows * 2 * 4
    assert swr.workspace_bytes(swr.SWR_OP_GQA_VERIFY, 8, 4, 64, 8, 256, 1024) == want


def test_verify_workspace_covers_either_element_type():
    # B=64 x 8 KV heads = 512 units: with bf16 K/V the verify runs unsplit in
    # the ring kernel (no workspace), over fp8 in chunked form; the query has
    # no element type, so it reports the chunked form's partials
    units, chunks, rows, d = 64 * 8, 1024 // 256, 8 * 4, 256
    want = units * chunks * rows * d * 4 + units * chunks * rows * 2 * 4
    assert swr.workspace_bytes(swr.SWR_OP_GQA_VERIFY, 64, 4, 64, 8, 256, 1024) == want


def test_workspace_bytes_unsupported_is_zero():
    assert swr.workspace_bytes(swr.SWR_OP_GQA_VERIFY, 8, 9, 64, 8, 256, 1024) == 0
    assert swr.workspace_bytes(99, 8, 4, 64, 8, 256, 1024) == 0


def test_region_bytes():
    assert swr.region_bytes(1024, 8, 256) == 1024 * 8 * 256 * 2
    assert swr.region_bytes(2**31 - 8, 1, 64) == 2**31 * 64 * 2  # 64-bit count, slots rounded to 32
    assert swr.region_bytes(1024, 8, 256, swr.SWR_KV_FP8_E4M3) == 1024 * 8 * 256
    with pytest.raises(ValueError):
        swr.region_bytes(1001, 8, 256)
