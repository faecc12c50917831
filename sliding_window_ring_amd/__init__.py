"""Python binding of libswr.so (include/swr.h): sliding-window ring and
grouped-verify attention on MI355X (gfx950).

This module only marshals arguments: torch tensors supply device memory and
the current HIP stream; every step of the computation runs in the library's
HIP kernels.  If libswr.so has not been built, importing this package raises
ImportError (there is no fallback path).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass, field
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswr.so")

SWR_KV_BF16 = 0
SWR_KV_FP8_E4M3 = 1
SWR_OP_SWA_DECODE = 0
SWR_OP_GQA_VERIFY = 1
SWR_OP_GLOBAL_ATTEND = 2
SWR_OP_SWA_APPEND_DECODE = 3
SWR_OP_GLOBAL_APPEND_ATTEND = 4

STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported shape", 3: "workspace missing or too small",
          4: "HIP launch error", 5: "pool exhausted"}

EXPORTS = [
    "swr_ring_kv_append", "swr_swa_decode", "swr_swa_append_decode", "swr_gqa_verify", "swr_global_attend",
    "swr_global_append_attend", "swr_global_append_attend_noalloc", "swr_workspace_bytes",
    "swr_kv_region_bytes", "swr_pool_create", "swr_pool_destroy", "swr_pool_alloc", "swr_pool_free",
    "swr_pool_alloc_ring", "swr_pool_alloc_global", "swr_pool_stats", "swr_pool_admit", "swr_pool_release", "swr_request_kv_bytes",
    "swr_zero_fill", "swr_paged_gather_window", "swr_read_ceiling",
    "swr_status_string",
]


class SwrKV(ctypes.Structure):
    """Mirror of `swr_kv` in include/swr.h."""
    _fields_ = [
        ("k_base", ctypes.c_void_p), ("v_base", ctypes.c_void_p),
        ("k_off", ctypes.c_void_p), ("v_off", ctypes.c_void_p), ("cap_b", ctypes.c_void_p),
        ("cap", ctypes.c_int32), ("dtype", ctypes.c_int32),
        ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float),
    ]


class SwrError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn}: {STATUS.get(status, status)} (status {status})")
        self.status = status


def _load(path: str = LIB_PATH) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with "
                          "`python sliding_window_ring_amd/build.py` (hipcc, gfx950)")
    lib = ctypes.CDLL(path)
    P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    KV = ctypes.POINTER(SwrKV)
    sig = {
        "swr_ring_kv_append": ([KV, P, P, P, P, I, I, I, I, I, P], I),
        "swr_swa_decode": ([KV, P, P, P, I, I, I, I, F, P, SZ, P], I),
        "swr_swa_append_decode": ([KV, P, P, P, P, P, I, I, I, I, F, P, SZ, P], I),
        "swr_gqa_verify": ([KV, P, P, P, P, P, I, I, I, I, I, F, P, SZ, P], I),
        "swr_global_attend": ([KV, P, P, P, P, I, I, I, I, I, I, F, P, SZ, P], I),
        "swr_global_append_attend": ([KV, P, P, P, P, P, I, I, I, I, I, I, F, P, SZ, P], I),
        "swr_global_append_attend_noalloc": ([KV, P, P, P, P, P, I, I, I, I, I, I, F, P], I),
        "swr_workspace_bytes": ([I, I, I, I, I, I, I], SZ),
        "swr_kv_region_bytes": ([I, I, I, I], I64),
        "swr_pool_create": ([P, SZ, ctypes.POINTER(P)], I),
        "swr_pool_destroy": ([P], None),
        "swr_pool_alloc": ([P, SZ, ctypes.POINTER(I64)], I),
        "swr_pool_free": ([P, I64], I),
        "swr_pool_alloc_ring": ([P, I, I, I, I, P, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                 ctypes.POINTER(ctypes.c_int32)], I),
        "swr_pool_alloc_global": ([P, I, I, I, I, P, ctypes.POINTER(I64), ctypes.POINTER(I64),
                                   ctypes.POINTER(ctypes.c_int32)], I),
        "swr_pool_stats": ([P, ctypes.POINTER(SZ), ctypes.POINTER(SZ)], I),
        "swr_pool_admit": ([P, I, I, I, I, I, I, I, I, I, P, P, P, ctypes.POINTER(ctypes.c_int32)], I),
        "swr_pool_release": ([P, I, P, P], I),
        "swr_request_kv_bytes": ([I, I, I, I, I, I, I, I, I, I], I64),
        "swr_zero_fill": ([P, SZ, P], I),
        "swr_paged_gather_window": ([P, P, I64, I, P, I, P, KV, I, I, I, P], I),
        "swr_read_ceiling": ([P, SZ, P, I, I, P], I),
        "swr_status_string": ([I], ctypes.c_char_p),
    }
    for name, (args, res) in sig.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = res
    return lib


lib = _load()


def _check(fn: str, status: int):
    if status != 0:
        raise SwrError(fn, status)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _dev(t: torch.Tensor, name: str, dtype=None):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t


@dataclass
class KVLayer:
    """One layer's K/V regions: per-request byte offsets into base buffers
    (usually one shared pool tensor).  Mirrors `swr_kv`."""
    k_base: torch.Tensor          # device uint8 buffer holding the K regions
    v_base: torch.Tensor          # device uint8 buffer holding the V regions
    k_off: torch.Tensor           # device int64 [B]
    v_off: torch.Tensor           # device int64 [B]
    cap: int                      # slots per region (ring: W; global: the largest capacity)
    dtype: int = SWR_KV_BF16
    k_scale: float = 1.0
    v_scale: float = 1.0
    cap_b: Optional[torch.Tensor] = None  # device int32 [B] per-request capacities (global regions)
    _c: SwrKV = field(default=None, repr=False)

    def c(self) -> SwrKV:
        _dev(self.k_off, "k_off", torch.int64)
        _dev(self.v_off, "v_off", torch.int64)
        if self.cap_b is not None:
            _dev(self.cap_b, "cap_b", torch.int32)
        self._c = SwrKV(self.k_base.data_ptr(), self.v_base.data_ptr(), self.k_off.data_ptr(),
                        self.v_off.data_ptr(), None if self.cap_b is None else self.cap_b.data_ptr(),
                        self.cap, self.dtype, self.k_scale, self.v_scale)
        return self._c


def region_bytes(cap: int, hkv: int, d: int, dtype: int = SWR_KV_BF16) -> int:
    n = lib.swr_kv_region_bytes(cap, hkv, d, dtype)
    if n < 0:
        raise ValueError("invalid region shape")
    return int(n)


def workspace_bytes(op: int, B: int, S: int, Hq: int, Hkv: int, D: int, cap_or_max_keys: int) -> int:
    return int(lib.swr_workspace_bytes(op, B, S, Hq, Hkv, D, cap_or_max_keys))


def _workspace(op, B, S, Hq, Hkv, D, n, ws, device):
    need = workspace_bytes(op, B, S, Hq, Hkv, D, n)
    if ws is None and need > 0:
        ws = torch.empty(need, dtype=torch.uint8, device=device)
    return ws, (0 if ws is None else ws.numel() * ws.element_size())


def ring_kv_append(kv: KVLayer, k_new: torch.Tensor, v_new: torch.Tensor, pos0: torch.Tensor,
                   n_new: Optional[torch.Tensor] = None, wrap: bool = True, stream=None) -> None:
    """swr_ring_kv_append: k_new, v_new bf16 [B][T][Hkv][D]; pos0 (and n_new)
    int32 [B]; wrap=False writes contiguous global regions (slot = position)."""
    _dev(k_new, "k_new", torch.bfloat16)
    _dev(v_new, "v_new", torch.bfloat16)
    _dev(pos0, "pos0", torch.int32)
    if n_new is not None:
        _dev(n_new, "n_new", torch.int32)
    B, T, hkv, d = k_new.shape
    _check("swr_ring_kv_append", lib.swr_ring_kv_append(ctypes.byref(kv.c()), _ptr(k_new), _ptr(v_new), _ptr(pos0),
                                                        _ptr(n_new), B, T, hkv, d, 1 if wrap else 0,
                                                        _stream(stream)))


def paged_gather_window(k_pages: torch.Tensor, v_pages: torch.Tensor, block_table: torch.Tensor,
                        pos: torch.Tensor, ring: KVLayer, stream=None) -> None:
    """swr_paged_gather_window: k_pages, v_pages bf16 [n_pages][page_tokens][Hkv][D];
    block_table int32 [B][max_pages]; pos int32 [B]."""
    _dev(k_pages, "k_pages", torch.bfloat16)
    _dev(v_pages, "v_pages", torch.bfloat16)
    _dev(block_table, "block_table", torch.int32)
    _dev(pos, "pos", torch.int32)
    if k_pages.dim() != 4 or v_pages.shape != k_pages.shape:
        raise ValueError("k_pages and v_pages must both be [n_pages][page_tokens][Hkv][D]")
    if block_table.dim() != 2 or pos.shape != (block_table.shape[0],):
        raise ValueError("block_table must be [B][max_pages] and pos [B]")
    n_pages, page_tokens, hkv, d = k_pages.shape
    B, max_pages = block_table.shape
    _check("swr_paged_gather_window",
           lib.swr_paged_gather_window(_ptr(k_pages), _ptr(v_pages), n_pages, page_tokens, _ptr(block_table),
                                       max_pages, _ptr(pos), ctypes.byref(ring.c()), B, hkv, d,
                                       _stream(stream)))


def swa_decode(ring: KVLayer, q: torch.Tensor, pos: torch.Tensor, hkv: int, scale: float,
               out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
               stream=None) -> torch.Tensor:
    """swr_swa_decode: q bf16 [B][Hq][D]; pos int32 [B] -> out bf16 [B][Hq][D]."""
    _dev(q, "q", torch.bfloat16)
    _dev(pos, "pos", torch.int32)
    B, hq, d = q.shape
    out = torch.empty_like(q) if out is None else _dev(out, "out", torch.bfloat16)
    ws, wsb = _workspace(SWR_OP_SWA_DECODE, B, 1, hq, hkv, d, ring.cap, ws, q.device)
    _check("swr_swa_decode", lib.swr_swa_decode(ctypes.byref(ring.c()), _ptr(q), _ptr(out), _ptr(pos), B,
                                                hq, hkv, d, scale, _ptr(ws), wsb, _stream(stream)))
    return out


def swa_append_decode(ring: KVLayer, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                      pos: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
                      ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """swr_swa_append_decode: k_new, v_new bf16 [B][Hkv][D] (or [B][1][Hkv][D]),
    q bf16 [B][Hq][D], pos int32 [B] -> out bf16 [B][Hq][D]."""
    _dev(k_new, "k_new", torch.bfloat16)
    _dev(v_new, "v_new", torch.bfloat16)
    _dev(q, "q", torch.bfloat16)
    _dev(pos, "pos", torch.int32)
    B, hq, d = q.shape
    hkv = k_new.shape[-2]
    out = torch.empty_like(q) if out is None else _dev(out, "out", torch.bfloat16)
    ws, wsb = _workspace(SWR_OP_SWA_APPEND_DECODE, B, 1, hq, hkv, d, ring.cap, ws, q.device)
    _check("swr_swa_append_decode",
           lib.swr_swa_append_decode(ctypes.byref(ring.c()), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                     _ptr(pos), B, hq, hkv, d, scale, _ptr(ws), wsb, _stream(stream)))
    return out


def gqa_verify(ring: KVLayer, k_prop: torch.Tensor, v_prop: torch.Tensor, q: torch.Tensor,
               pos0: torch.Tensor, scale: float, out: Optional[torch.Tensor] = None,
               ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """swr_gqa_verify: q bf16 [B][S][Hq][D], k_prop/v_prop bf16 [B][S][Hkv][D],
    pos0 int32 [B] -> out bf16 [B][S][Hq][D]."""
    _dev(q, "q", torch.bfloat16)
    _dev(k_prop, "k_prop", torch.bfloat16)
    _dev(v_prop, "v_prop", torch.bfloat16)
    _dev(pos0, "pos0", torch.int32)
    B, S, hq, d = q.shape
    hkv = k_prop.shape[2]
    out = torch.empty_like(q) if out is None else _dev(out, "out", torch.bfloat16)
    ws, wsb = _workspace(SWR_OP_GQA_VERIFY, B, S, hq, hkv, d, ring.cap, ws, q.device)
    _check("swr_gqa_verify", lib.swr_gqa_verify(ctypes.byref(ring.c()), _ptr(k_prop), _ptr(v_prop), _ptr(q),
                                                _ptr(out), _ptr(pos0), B, S, hq, hkv, d, scale, _ptr(ws),
                                                wsb, _stream(stream)))
    return out


def global_attend(kv: KVLayer, q: torch.Tensor, q_pos: torch.Tensor, key_count: torch.Tensor,
                  max_key_count: int, hkv: int, scale: float, out: Optional[torch.Tensor] = None,
                  ws: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """swr_global_attend: q bf16 [B][S][Hq][D], q_pos int32 [B][S], key_count
    int32 [B] -> out bf16 [B][S][Hq][D]."""
    _dev(q, "q", torch.bfloat16)
    _dev(q_pos, "q_pos", torch.int32)
    _dev(key_count, "key_count", torch.int32)
    B, S, hq, d = q.shape
    out = torch.empty_like(q) if out is None else _dev(out, "out", torch.bfloat16)
    ws, wsb = _workspace(SWR_OP_GLOBAL_ATTEND, B, S, hq, hkv, d, max_key_count, ws, q.device)
    _check("swr_global_attend", lib.swr_global_attend(ctypes.byref(kv.c()), _ptr(q), _ptr(out), _ptr(q_pos),
                                                      _ptr(key_count), max_key_count, B, S, hq, hkv, d, scale,
                                                      _ptr(ws), wsb, _stream(stream)))
    return out


def global_append_attend(kv: KVLayer, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                         pos0: torch.Tensor, max_key_count: int, scale: float,
                         out: Optional[torch.Tensor] = None, ws: Optional[torch.Tensor] = None,
                         stream=None) -> torch.Tensor:
    """swr_global_append_attend: k_new, v_new bf16 [B][S][Hkv][D], q bf16
    [B][S][Hq][D], pos0 int32 [B] -> out bf16 [B][S][Hq][D]."""
    _dev(k_new, "k_new", torch.bfloat16)
    _dev(v_new, "v_new", torch.bfloat16)
    _dev(q, "q", torch.bfloat16)
    _dev(pos0, "pos0", torch.int32)
    B, S, hq, d = q.shape
    hkv = k_new.shape[2]
    out = torch.empty_like(q) if out is None else _dev(out, "out", torch.bfloat16)
    ws, wsb = _workspace(SWR_OP_GLOBAL_APPEND_ATTEND, B, S, hq, hkv, d, max_key_count, ws, q.device)
    _check("swr_global_append_attend",
           lib.swr_global_append_attend(ctypes.byref(kv.c()), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                        _ptr(pos0), max_key_count, B, S, hq, hkv, d, scale, _ptr(ws), wsb,
                                        _stream(stream)))
    return out


def global_append_attend_noalloc(kv: KVLayer, k_new: torch.Tensor, v_new: torch.Tensor, q: torch.Tensor,
                                 pos0: torch.Tensor, max_key_count: int, scale: float,
                                 out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """swr_global_append_attend_noalloc: global_append_attend with the
    library's static device scratch as workspace (no allocation by the
    library; `out` given by the caller allocates nothing here either)."""
    _dev(k_new, "k_new", torch.bfloat16)
    _dev(v_new, "v_new", torch.bfloat16)
    _dev(q, "q", torch.bfloat16)
    _dev(pos0, "pos0", torch.int32)
    B, S, hq, d = q.shape
    hkv = k_new.shape[2]
    out = torch.empty_like(q) if out is None else _dev(out, "out", torch.bfloat16)
    _check("swr_global_append_attend_noalloc",
           lib.swr_global_append_attend_noalloc(ctypes.byref(kv.c()), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                                _ptr(pos0), max_key_count, B, S, hq, hkv, d, scale, _stream(stream)))
    return out


def zero_fill(t: torch.Tensor, offset: int = 0, nbytes: Optional[int] = None, stream=None) -> None:
    """swr_zero_fill over bytes [offset, offset+nbytes) of a device tensor."""
    _dev(t, "t")
    total = t.numel() * t.element_size()
    nbytes = total - offset if nbytes is None else nbytes
    if offset < 0 or offset + nbytes > total:
        raise ValueError("range outside the tensor")
    _check("swr_zero_fill", lib.swr_zero_fill(ctypes.c_void_p(t.data_ptr() + offset), nbytes, _stream(stream)))


def read_ceiling(src: torch.Tensor, sink: torch.Tensor, grid: int, pattern: int = 0, stream=None) -> None:
    """swr_read_ceiling: one streaming read of the whole device tensor `src`
    (a measurement aid); sink: a device tensor of at least 1024 bytes."""
    _dev(src, "src")
    _dev(sink, "sink")
    if sink.numel() * sink.element_size() < 1024:
        raise ValueError("sink needs at least 1024 bytes")
    _check("swr_read_ceiling", lib.swr_read_ceiling(ctypes.c_void_p(src.data_ptr()),
                                                    src.numel() * src.element_size(),
                                                    ctypes.c_void_p(sink.data_ptr()), grid, pattern,
                                                    _stream(stream)))


def request_kv_bytes(n_sliding: int, W: int, hkv_s: int, d_s: int, n_global: int, context: int, hkv_g: int,
                     d_g: int, dtype: int = SWR_KV_BF16, full_context: bool = False) -> int:
    """swr_request_kv_bytes: one request's region bytes under ring admission,
    or with every layer at full context."""
    return int(lib.swr_request_kv_bytes(n_sliding, W, hkv_s, d_s, n_global, context, hkv_g, d_g, dtype,
                                        1 if full_context else 0))


class Pool:
    """A device byte buffer shared by ring and global regions ("Improving
    Decode Throughput on Intel Gaudi 3", Our approach), carved by the
    library's host bookkeeping (swr_pool_*); the carves zero-fill what they
    hand out on the stream."""

    def __init__(self, nbytes: int, device="cuda"):
        self.buffer = torch.empty(nbytes, dtype=torch.uint8, device=device)
        h = ctypes.c_void_p()
        _check("swr_pool_create", lib.swr_pool_create(ctypes.c_void_p(self.buffer.data_ptr()), nbytes,
                                                      ctypes.byref(h)))
        self._h = h

    def alloc(self, nbytes: int) -> int:
        off = ctypes.c_int64()
        _check("swr_pool_alloc", lib.swr_pool_alloc(self._h, nbytes, ctypes.byref(off)))
        return off.value

    def free(self, offset: int) -> None:
        _check("swr_pool_free", lib.swr_pool_free(self._h, offset))

    def alloc_ring(self, W: int, hkv: int, d: int, dtype: int = SWR_KV_BF16, stream=None):
        """swr_pool_alloc_ring: a zero-filled ring (K and V) of W slots
        (rounded up to 8).  Returns (k_offset, v_offset, cap)."""
        ko, vo, cap = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check("swr_pool_alloc_ring", lib.swr_pool_alloc_ring(self._h, W, hkv, d, dtype, _stream(stream),
                                                              ctypes.byref(ko), ctypes.byref(vo), ctypes.byref(cap)))
        return ko.value, vo.value, cap.value

    def alloc_global(self, tokens: int, hkv: int, d: int, dtype: int = SWR_KV_BF16, stream=None):
        """swr_pool_alloc_global: a zero-filled global region (K and V) of
        `tokens` slots rounded up to 64.  Returns (k_offset, v_offset, cap)."""
        ko, vo, cap = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
        _check("swr_pool_alloc_global", lib.swr_pool_alloc_global(self._h, tokens, hkv, d, dtype, _stream(stream),
                                                                  ctypes.byref(ko), ctypes.byref(vo),
                                                                  ctypes.byref(cap)))
        return ko.value, vo.value, cap.value

    def admit(self, n_sliding: int, W: int, hkv_s: int, d_s: int, n_global: int, context: int, hkv_g: int,
              d_g: int, dtype: int = SWR_KV_BF16, stream=None):
        """swr_pool_admit: one request's rings and global regions, all or
        nothing, zero-filled on the stream.  Returns (k_offsets, v_offsets,
        global_cap), sliding layers first."""
        n = n_sliding + n_global
        ko, vo, gcap = (ctypes.c_int64 * max(n, 1))(), (ctypes.c_int64 * max(n, 1))(), ctypes.c_int32(0)
        _check("swr_pool_admit", lib.swr_pool_admit(self._h, n_sliding, W, hkv_s, d_s, n_global, context, hkv_g,
                                                    d_g, dtype, _stream(stream), ko, vo, ctypes.byref(gcap)))
        return list(ko[:n]), list(vo[:n]), gcap.value

    def release(self, k_offsets, v_offsets) -> None:
        """swr_pool_release: the ranges of a request admitted by admit()."""
        n = len(k_offsets)
        _check("swr_pool_release", lib.swr_pool_release(self._h, n, (ctypes.c_int64 * max(n, 1))(*k_offsets),
                                                        (ctypes.c_int64 * max(n, 1))(*v_offsets)))

    def stats(self):
        used, largest = ctypes.c_size_t(), ctypes.c_size_t()
        _check("swr_pool_stats", lib.swr_pool_stats(self._h, ctypes.byref(used), ctypes.byref(largest)))
        return used.value, largest.value

    def close(self):
        if self._h:
            lib.swr_pool_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass
