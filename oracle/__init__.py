"""CPU oracle for the sliding-window ring / grouped-verify attention path.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The GPU library
(``sliding_window_ring_amd``) never imports it and shares no code with it.

The arithmetic lives in ``swr_oracle.c`` (plain C, IEEE binary64, fixed
summation order) and works on logical regions ([slot][Hkv][D] elements);
``swr_layout.c`` is the codec between those and the device byte layout the
GPU library declares.  This module only builds them with gcc and marshals
numpy arrays through ctypes.  The functions that take pools take them in the
device layout (the form the GPU tests compare byte for byte) and go through
the codec; the ``*_logical`` ones take logical regions directly.  Each function below names the passage of the pages it
follows; the C file states the readings taken where the pages are silent.

Pages:
  * "Announcing Carat: An inference engine designed for Gemma 4" (ring buffer
    section; "More FLOPs can be faster"; "Doing it all in one kernel can be
    slower").
  * "Improving Decode Throughput on Intel Gaudi 3" ("Patching sliding window KV
    allocation"; "Our approach").
  * "gemma-cuda-hybrid" README ("Features": GQA shapes, FP8 e4m3 KV cache).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
# swr_oracle.c: formats, append and attention on logical [slot][Hkv][D]
# regions; swr_layout.c: the codec between those and the device byte layout
SOURCES = ("swr_oracle.c", "swr_layout.c")
_LIB = os.path.join(_HERE, "liboracle.so")

BF16 = 0
FP8 = 1

_CFLAGS = ["-O2", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]


def _compile(srcs, out):
    tmp = out + ".tmp%d" % os.getpid()
    subprocess.check_call(["gcc", *_CFLAGS, *srcs, "-o", tmp, "-lm"])
    os.replace(tmp, out)


def build(force: bool = False) -> str:
    """Compile the oracle sources with gcc into liboracle.so next to them."""
    srcs = [os.path.join(_HERE, f) for f in SOURCES]
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(map(os.path.getmtime, srcs)):
        _compile(srcs, _LIB)
    return _LIB


_SAN_LIB = os.path.join(_HERE, "_build_san", "liboracle_san.so")
_SAN_FLAGS = ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined", "-fno-omit-frame-pointer", "-g"]


def build_sanitized(force: bool = False) -> str:
    """The oracle under AddressSanitizer and UndefinedBehaviorSanitizer
    (gcc), for the sanitized run of the pins (tests/test_sanitizers.py);
    loading it needs gcc's libasan preloaded (sanitizer_runtime())."""
    srcs = [os.path.join(_HERE, f) for f in SOURCES]
    if force or not os.path.exists(_SAN_LIB) or os.path.getmtime(_SAN_LIB) < max(map(os.path.getmtime, srcs)):
        os.makedirs(os.path.dirname(_SAN_LIB), exist_ok=True)
        tmp = _SAN_LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *_CFLAGS, *_SAN_FLAGS, *srcs, "-o", tmp, "-lm"])
        os.replace(tmp, _SAN_LIB)
    return _SAN_LIB


def sanitizer_runtime() -> str:
    """gcc's ASan runtime, for LD_PRELOAD into an uninstrumented Python."""
    out = subprocess.run(["gcc", "-print-file-name=libasan.so"], stdout=subprocess.PIPE, text=True,
                         check=True).stdout.strip()
    if not os.path.isabs(out) or not os.path.exists(out):
        raise FileNotFoundError("gcc's libasan not found")
    return out


_lib = None


def _bind(h):
    """Declare the C signatures on a loaded oracle library."""
    P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
    F, D = ctypes.c_float, ctypes.c_double
    h.orc_bf16_value_n.argtypes = [P, I64, P]
    h.orc_e4m3_value_n.argtypes = [P, I64, P]
    h.orc_e4m3_encode_n.argtypes = [P, I64, F, P]
    h.orc_region_bytes.argtypes = [I, I, I, I]
    h.orc_region_bytes.restype = I64
    h.orc_logical_region_bytes.argtypes = [I, I, I, I]
    h.orc_logical_region_bytes.restype = I64
    h.orc_layout_pack.argtypes = [P, P, I, I, I, I, I]
    h.orc_layout_unpack.argtypes = [P, P, I, I, I, I, I]
    h.orc_kv_append.argtypes = [P, P, P, P, I, P, I, F, F, P, P, P, P, I, I, I, I, I]
    h.orc_swa_decode.argtypes = [P, P, P, P, I, I, D, D, P, P, I, I, I, I, D, P]
    h.orc_gqa_verify.argtypes = [P, P, P, P, I, I, D, D, P, P, P, P, I, I, I, I, I, D, P]
    h.orc_global_attend.argtypes = [P, P, P, P, I, P, I, D, D, P, P, P, I, I, I, I, I, I, D, P]
    h.orc_num_threads.restype = I
    h.orc_set_threads.argtypes = [I]
    h.orc_set_threads.restype = I
    return h


def lib():
    global _lib
    if _lib is None:
        _lib = _bind(ctypes.CDLL(build()))
    return _lib


def build_variant(name: str, src_text: str, out_dir: str) -> str:
    """Compile the oracle with source file `name` replaced by `src_text`
    (tests use this to plant a mistake and check that the pins catch it).
    Returns the library path."""
    srcs = []
    for f in SOURCES:
        if f == name:
            path = os.path.join(out_dir, "variant_" + f)
            with open(path, "w") as fh:
                fh.write(src_text)
            srcs.append(path)
        else:
            srcs.append(os.path.join(_HERE, f))
    so = os.path.join(out_dir, "liboracle_variant.so")
    _compile(srcs, so)
    return so


class use_library:
    """Context manager: route this module's functions to another build of the
    oracle (a planted-mistake variant) for the duration of the block."""

    def __init__(self, path: str):
        self.handle = _bind(ctypes.CDLL(path))

    def __enter__(self):
        global _lib
        lib()
        self.saved, _lib = _lib, self.handle
        return self

    def __exit__(self, *exc):
        global _lib
        _lib = self.saved
        return False


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


def num_threads() -> int:
    """OpenMP threads the oracle's parallel loops use."""
    return lib().orc_num_threads()


def set_threads(n: int) -> int:
    """Set the oracle's OpenMP threads (for timing on fewer cores); returns
    the previous count.  Results are the same for any count."""
    return lib().orc_set_threads(int(n))


# ---------------------------------------------------------------- formats

def bf16_value(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (upper half of an IEEE binary32)."""
    x = _c(bits, np.uint16)
    out = np.empty(x.shape, np.float64)
    lib().orc_bf16_value_n(_p(x), x.size, _p(out))
    return out


def e4m3_value(codes) -> np.ndarray:
    """OCP E4M3FN decode ("gemma-cuda-hybrid", Features: FP8 e4m3 KV)."""
    x = _c(codes, np.uint8)
    out = np.empty(x.shape, np.float64)
    lib().orc_e4m3_value_n(_p(x), x.size, _p(out))
    return out


def e4m3_encode(bits, scale: float) -> np.ndarray:
    """E4M3FN code of bf16 values divided by a per-tensor scale: nearest code
    to the exact quotient, ties to even, saturating at +-448."""
    x = _c(bits, np.uint16)
    out = np.empty(x.shape, np.uint8)
    lib().orc_e4m3_encode_n(_p(x), x.size, ctypes.c_float(scale), _p(out))
    return out


def region_bytes(cap: int, hkv: int, d: int, dtype: int) -> int:
    """Bytes of one K (or V) region of `cap` slots in the device layout
    (cap a multiple of 8)."""
    n = lib().orc_region_bytes(cap, hkv, d, dtype)
    if n < 0:
        raise ValueError("invalid region shape")
    return int(n)


def logical_region_bytes(cap: int, hkv: int, d: int, dtype: int) -> int:
    """Bytes of one logical region: [cap][Hkv][D] elements."""
    n = lib().orc_logical_region_bytes(cap, hkv, d, dtype)
    if n < 0:
        raise ValueError("invalid region shape")
    return int(n)


def unpack_region(region, cap: int, hkv: int, d: int, dtype: int, is_v: bool) -> np.ndarray:
    """The logical content ([cap][Hkv][D] elements, as bytes) of a region in
    the device layout."""
    r = _c(region, np.uint8)
    if r.size < region_bytes(cap, hkv, d, dtype):
        raise ValueError("region too small")
    out = np.empty(logical_region_bytes(cap, hkv, d, dtype), np.uint8)
    _check_rc(lib().orc_layout_unpack(_p(r), _p(out), cap, hkv, d, dtype, 1 if is_v else 0), "layout_unpack")
    return out


def pack_region(logical, region, cap: int, hkv: int, d: int, dtype: int, is_v: bool) -> None:
    """Writes a logical region ([cap][Hkv][D] elements, as bytes) into
    `region` (a writable uint8 array of the device layout), in place."""
    lg = _c(logical, np.uint8)
    assert region.dtype == np.uint8 and region.flags.c_contiguous
    if lg.size < logical_region_bytes(cap, hkv, d, dtype) or region.size < region_bytes(cap, hkv, d, dtype):
        raise ValueError("region too small")
    _check_rc(lib().orc_layout_pack(_p(lg), _p(region), cap, hkv, d, dtype, 1 if is_v else 0), "layout_pack")


def _caps_of(cap, caps, B):
    return [int(cap)] * B if caps is None else [int(c) for c in np.asarray(caps).ravel()[:B]]


def to_logical(k_pool, v_pool, k_off, v_off, caps, hkv, d, dtype):
    """Logical copies of B regions of device-layout pools: returns
    (k_log, v_log, offsets) with request b's [caps[b]][Hkv][D] elements at
    byte offset offsets[b] of k_log and of v_log."""
    lens = [logical_region_bytes(c, hkv, d, dtype) for c in caps]
    offs = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64) if lens else np.zeros(0, np.int64)
    total = int(sum(lens))
    k_log = np.zeros(max(total, 1), np.uint8)
    v_log = np.zeros(max(total, 1), np.uint8)
    for b, c in enumerate(caps):
        rb = region_bytes(c, hkv, d, dtype)
        ko, vo, lo = int(k_off[b]), int(v_off[b]), int(offs[b])
        k_log[lo:lo + lens[b]] = unpack_region(k_pool[ko:ko + rb], c, hkv, d, dtype, False)
        v_log[lo:lo + lens[b]] = unpack_region(v_pool[vo:vo + rb], c, hkv, d, dtype, True)
    return k_log, v_log, offs


def from_logical(k_log, v_log, offs, k_pool, v_pool, k_off, v_off, caps, hkv, d, dtype):
    """Writes logical regions (as returned by to_logical) back into the
    device-layout pools, in place."""
    for b, c in enumerate(caps):
        rb = region_bytes(c, hkv, d, dtype)
        ko, vo, lo = int(k_off[b]), int(v_off[b]), int(offs[b])
        n = logical_region_bytes(c, hkv, d, dtype)
        pack_region(k_log[lo:lo + n], k_pool[ko:ko + rb], c, hkv, d, dtype, False)
        pack_region(v_log[lo:lo + n], v_pool[vo:vo + rb], c, hkv, d, dtype, True)


# ---------------------------------------------------------------- operations

def _check_rc(rc, what):
    if rc != 0:
        raise ValueError(f"oracle {what} rejected its arguments (rc={rc})")


def kv_append_logical(k_log, v_log, offs, cap, dtype, k_scale, v_scale, k_new, v_new, pos0, n_new=None,
                      wrap=True, caps=None):
    """The append of kv_append on logical regions (request b's
    [cap][Hkv][D] elements at byte offset offs[b] of k_log / v_log), in
    place."""
    k_new = _c(k_new, np.uint16)
    v_new = _c(v_new, np.uint16)
    B, T, hkv, d = k_new.shape
    offs = _c(offs, np.int64)
    pos0 = _c(pos0, np.int32)
    nn = None if n_new is None else _c(n_new, np.int32)
    assert k_log.dtype == np.uint8 and v_log.dtype == np.uint8
    cp = None if caps is None else _c(caps, np.int32)
    rc = lib().orc_kv_append(_p(k_log), _p(v_log), _p(offs), _p(offs), cap, _p(cp), dtype,
                             ctypes.c_float(k_scale), ctypes.c_float(v_scale), _p(k_new), _p(v_new),
                             _p(pos0), _p(nn), B, T, hkv, d, 1 if wrap else 0)
    _check_rc(rc, "kv_append")


def kv_append(k_pool, v_pool, k_off, v_off, cap, dtype, k_scale, v_scale, k_new, v_new, pos0,
              n_new=None, wrap=True, caps=None):
    """Append tokens to each request's region of device-layout pools, in
    place.

    Ring mode (wrap=True): slot = position mod cap ("Announcing Carat", ring
    buffer section; "Improving Decode Throughput on Intel Gaudi 3", "Our
    approach": K and V of a token go to the same slot).  Global mode
    (wrap=False): slot = position; caps optionally gives each request's
    region capacity.  k_new, v_new: bf16 bits [B][T][Hkv][D].  The regions
    are read into logical form, appended to, and written back through the
    layout codec.
    """
    k_new = np.asarray(k_new)
    B, _, hkv, d = k_new.shape
    assert k_pool.dtype == np.uint8 and v_pool.dtype == np.uint8
    cl = _caps_of(cap, caps, B)
    k_log, v_log, offs = to_logical(k_pool, v_pool, k_off, v_off, cl, hkv, d, dtype)
    kv_append_logical(k_log, v_log, offs, cap, dtype, k_scale, v_scale, k_new, v_new, pos0, n_new, wrap,
                      None if caps is None else cl)
    from_logical(k_log, v_log, offs, k_pool, v_pool, k_off, v_off, cl, hkv, d, dtype)


def paged_gather_window(k_pool, v_pool, k_off, v_off, W, k_pages, v_pages, block_table, pos):
    """The paged-cache gather that a sliding-window layer needs when its KV
    lives in scattered pages ("Improving Decode Throughput on Intel Gaudi 3",
    "Expensive KV gathers"), into bf16 ring regions, in place.

    Request b's window is the positions max(0, pos[b]-W+1) .. pos[b]; the
    token at position p is row p mod page_tokens of page
    block_table[b][p // page_tokens] of k_pages / v_pages (bf16 bits
    [n_pages][page_tokens][Hkv][D]).  Each is appended at ring slot p mod W;
    a position whose page index is past the table or whose entry is not a
    page of the pool is skipped, as is a request with pos < 0.
    """
    k_pages = np.asarray(k_pages, np.uint16)
    v_pages = np.asarray(v_pages, np.uint16)
    n_pages, pt, hkv, d = k_pages.shape
    bt = np.asarray(block_table, np.int64)
    pos = np.asarray(pos, np.int64)
    B = pos.shape[0]
    k_log, v_log, offs = to_logical(k_pool, v_pool, k_off, v_off, [W] * B, hkv, d, BF16)
    for b in range(B):
        P = int(pos[b])
        if P < 0:
            continue
        for p in range(max(0, P - W + 1), P + 1):
            i = p // pt
            if i >= bt.shape[1] or not 0 <= bt[b, i] < n_pages:
                continue
            page, row = int(bt[b, i]), p % pt
            kv_append_logical(k_log, v_log, offs[b:b + 1], W, BF16, 1.0, 1.0, k_pages[page, row][None, None],
                              v_pages[page, row][None, None], np.array([p], np.int32))
    from_logical(k_log, v_log, offs, k_pool, v_pool, k_off, v_off, [W] * B, hkv, d, BF16)


def swa_decode_logical(k_log, v_log, offs, W, dtype, k_scale, v_scale, q, pos, hkv, scale):
    """swa_decode on logical ring regions (request b's [W][Hkv][D] elements
    at byte offset offs[b])."""
    q = _c(q, np.uint16)
    B, hq, d = q.shape
    out = np.empty((B, hq, d), np.float64)
    offs = _c(offs, np.int64)
    rc = lib().orc_swa_decode(_p(k_log), _p(v_log), _p(offs), _p(offs), W, dtype, k_scale, v_scale, _p(q),
                              _p(_c(pos, np.int32)), B, hq, hkv, d, scale, _p(out))
    _check_rc(rc, "swa_decode")
    return out


def swa_decode(k_pool, v_pool, k_off, v_off, W, dtype, k_scale, v_scale, q, pos, hkv, scale):
    """Sliding-window decode over each request's ring, read in storage order.

    q: bf16 bits [B][Hq][D]; pos[b]: the query's position, its token already in
    the ring.  Rings in device-layout pools.  Returns float64 [B][Hq][D].
    """
    B, _, d = np.asarray(q).shape
    k_log, v_log, offs = to_logical(k_pool, v_pool, k_off, v_off, [W] * B, hkv, d, dtype)
    return swa_decode_logical(k_log, v_log, offs, W, dtype, k_scale, v_scale, q, pos, hkv, scale)


def gqa_verify_logical(k_log, v_log, offs, W, dtype, k_scale, v_scale, k_prop, v_prop, q, pos0, hkv, scale):
    """gqa_verify on logical ring regions."""
    q = _c(q, np.uint16)
    B, S, hq, d = q.shape
    out = np.empty((B, S, hq, d), np.float64)
    offs = _c(offs, np.int64)
    rc = lib().orc_gqa_verify(_p(k_log), _p(v_log), _p(offs), _p(offs), W, dtype, k_scale, v_scale,
                              _p(_c(k_prop, np.uint16)), _p(_c(v_prop, np.uint16)), _p(q),
                              _p(_c(pos0, np.int32)), B, S, hq, hkv, d, scale, _p(out))
    _check_rc(rc, "gqa_verify")
    return out


def gqa_verify(k_pool, v_pool, k_off, v_off, W, dtype, k_scale, v_scale, k_prop, v_prop, q, pos0,
               hkv, scale):
    """Speculative verify on a sliding layer: G heads x S proposals per KV head.

    q: bf16 bits [B][S][Hq][D]; k_prop, v_prop: bf16 bits [B][S][Hkv][D];
    the ring holds positions < pos0[b].  Rings in device-layout pools.
    Returns float64 [B][S][Hq][D].
    """
    B, _, _, d = np.asarray(q).shape
    k_log, v_log, offs = to_logical(k_pool, v_pool, k_off, v_off, [W] * B, hkv, d, dtype)
    return gqa_verify_logical(k_log, v_log, offs, W, dtype, k_scale, v_scale, k_prop, v_prop, q, pos0, hkv, scale)


def global_attend_logical(k_log, v_log, offs, cap, dtype, k_scale, v_scale, q, q_pos, key_count, hkv, scale,
                          padded=True, caps=None):
    """global_attend on logical regions."""
    q = _c(q, np.uint16)
    B, S, hq, d = q.shape
    out = np.empty((B, S, hq, d), np.float64)
    offs = _c(offs, np.int64)
    cp = None if caps is None else _c(caps, np.int32)
    rc = lib().orc_global_attend(_p(k_log), _p(v_log), _p(offs), _p(offs), cap, _p(cp), dtype, k_scale, v_scale,
                                 _p(q), _p(_c(q_pos, np.int32)), _p(_c(key_count, np.int32)),
                                 1 if padded else 0, B, S, hq, hkv, d, scale, _p(out))
    _check_rc(rc, "global_attend")
    return out


def global_attend(k_pool, v_pool, k_off, v_off, cap, dtype, k_scale, v_scale, q, q_pos, key_count,
                  hkv, scale, padded=True, caps=None):
    """Global-layer attention over contiguous regions ("Announcing Carat",
    "More FLOPs can be faster": scores over key_count keys, causal softmax by
    query position, weighted sum of values; padded=True contracts over the
    64-padded key range with a masked tail).

    q: bf16 bits [B][S][Hq][D]; q_pos: [B][S]; key_count: [B].
    caps: optional per-request region capacities.  Regions in device-layout
    pools.  Returns float64 [B][S][Hq][D].
    """
    B, _, _, d = np.asarray(q).shape
    cl = _caps_of(cap, caps, B)
    k_log, v_log, offs = to_logical(k_pool, v_pool, k_off, v_off, cl, hkv, d, dtype)
    return global_attend_logical(k_log, v_log, offs, cap, dtype, k_scale, v_scale, q, q_pos, key_count, hkv, scale,
                                 padded, None if caps is None else cl)
