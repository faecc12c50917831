"""Seeded synthetic inputs shared by the oracle side and the GPU side.

This module holds random draws and shape bookkeeping only: no attention, no
slot arithmetic, no quantisation.  Both the oracle and the GPU library receive
exactly these arrays (bf16 as uint16 bit patterns) and each does its own
arithmetic on them.

Workloads (shapes from "gemma-cuda-hybrid" Features: sliding layers 8 KV heads
x head_dim 256, global layers 2 KV heads x head_dim 512; window 1024 from
"Improving Decode Throughput on Intel Gaudi 3" and "Announcing Carat"; 8 query
heads per KV head and 4 proposed positions from "Announcing Carat", "Doing it
all in one kernel can be slower"; batch 56 from the Gaudi page's trace; key
count 6005 from "Announcing Carat", "More FLOPs can be faster").
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED_BASE = 1000  # workload n uses seed SEED_BASE + n


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def bf16_bits(x) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    # u + 0x7FFF + lsb cannot pass 2^32 for non-NaN inputs; NaNs are fixed below
    r = ((u + ((u >> 16) & 1) + np.uint32(0x7FFF)) >> 16).astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        r[nan] = ((u[nan] >> 16) | 0x40).astype(np.uint16)  # keep NaN quiet
    return r


def bf16_to_f32(bits) -> np.ndarray:
    """bf16 bit patterns to float32 (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def normal_bf16(g: np.random.Generator, shape) -> np.ndarray:
    """Standard-normal draws rounded to bf16 (bits)."""
    return bf16_bits(g.standard_normal(shape, dtype=np.float32))


def uniform_int(g: np.random.Generator, lo: int, hi: int, n: int) -> np.ndarray:
    """n integers uniform on the inclusive range [lo, hi]."""
    return g.integers(lo, hi + 1, size=n, dtype=np.int64).astype(np.int32)


def log_uniform_int(g: np.random.Generator, lo: int, hi: int, n: int) -> np.ndarray:
    """n integers round(exp(U[ln lo, ln hi]))."""
    return np.rint(np.exp(g.uniform(np.log(lo), np.log(hi), size=n))).astype(np.int32)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hkv: int
    G: int
    D: int
    W: int = 0          # ring window (sliding layers), 0 for global layers
    S: int = 1          # query positions per request (proposals)
    pos_lo: int = 0     # position / context draw range
    pos_hi: int = 0
    key_count: int = 0  # fixed global key count, if any
    steps: int = 0      # tiny workload: tokens appended one by one

    @property
    def Hq(self) -> int:
        return self.Hkv * self.G


# The five workloads.  Numbers are the workloads' own; see the module docstring
# for where each shape comes from.
TINY = Workload("tiny ring decode", B=1, Hkv=1, G=2, D=64, W=16, steps=40)
SWA_DECODE = Workload("sliding decode", B=56, Hkv=8, G=8, D=256, W=1024, pos_lo=1024, pos_hi=4096)
SWA_VERIFY = Workload("sliding verify", B=8, Hkv=8, G=8, D=256, W=1024, S=4, pos_lo=1024,
                      pos_hi=8192)
GLOBAL_VERIFY = Workload("global verify", B=1, Hkv=2, G=8, D=512, S=4, key_count=6005)
MIXED_SLIDING = Workload("mixed step, sliding layer", B=16, Hkv=8, G=8, D=256, W=1024,
                         pos_lo=512, pos_hi=65536)
MIXED_GLOBAL = Workload("mixed step, global layer", B=16, Hkv=2, G=8, D=512, S=1, pos_lo=512,
                        pos_hi=65536)

GLOBAL_SWEEP = (4000, 8192)  # key counts swept in steps of 1


def tiny_sequence(seed: int = SEED_BASE + 1):
    """40 tokens for the tiny workload: per step q [Hq][D], k and v [Hkv][D]."""
    w = TINY
    g = rng(seed)
    q = normal_bf16(g, (w.steps, w.Hq, w.D))
    k = normal_bf16(g, (w.steps, w.Hkv, w.D))
    v = normal_bf16(g, (w.steps, w.Hkv, w.D))
    return q, k, v


def sliding_decode(w: Workload = SWA_DECODE, seed: int = SEED_BASE + 2, positions=None):
    """Decode batch for a sliding layer.

    Returns dict with
      pos     [B]            query positions (the query token is the newest key)
      start   [B]            first position still inside the window
      n       [B]            number of tokens in the window (<= W)
      k, v    [B][W][Hkv][D] window tokens in position order (first n valid)
      q       [B][Hq][D]
    Window = the W positions ending at pos ("Improving Decode Throughput on
    Intel Gaudi 3": sliding layers keep only the last 1024 tokens).
    """
    g = rng(seed)
    pos = uniform_int(g, w.pos_lo, w.pos_hi, w.B) if positions is None else \
        np.asarray(positions, np.int32)
    n = np.minimum(pos.astype(np.int64) + 1, w.W).astype(np.int32)
    start = (pos - n + 1).astype(np.int32)
    k = normal_bf16(g, (w.B, w.W, w.Hkv, w.D))
    v = normal_bf16(g, (w.B, w.W, w.Hkv, w.D))
    q = normal_bf16(g, (w.B, w.Hq, w.D))
    return dict(pos=pos, start=start, n=n, k=k, v=v, q=q)


def sliding_verify(w: Workload = SWA_VERIFY, seed: int = SEED_BASE + 3, positions=None):
    """Verify batch for a sliding layer: committed history before p0, S proposals.

    Returns dict with p0 [B], start [B], n [B] (committed window tokens,
    positions start .. p0-1), k, v [B][W][Hkv][D] (history in position order),
    k_prop, v_prop [B][S][Hkv][D], q [B][S][Hq][D].
    """
    g = rng(seed)
    p0 = uniform_int(g, w.pos_lo, w.pos_hi, w.B) if positions is None else \
        np.asarray(positions, np.int32)
    n = np.minimum(p0.astype(np.int64), w.W).astype(np.int32)
    start = (p0 - n).astype(np.int32)
    k = normal_bf16(g, (w.B, w.W, w.Hkv, w.D))
    v = normal_bf16(g, (w.B, w.W, w.Hkv, w.D))
    k_prop = normal_bf16(g, (w.B, w.S, w.Hkv, w.D))
    v_prop = normal_bf16(g, (w.B, w.S, w.Hkv, w.D))
    q = normal_bf16(g, (w.B, w.S, w.Hq, w.D))
    return dict(p0=p0, start=start, n=n, k=k, v=v, k_prop=k_prop, v_prop=v_prop, q=q)


def global_verify(w: Workload = GLOBAL_VERIFY, seed: int = SEED_BASE + 4, key_count=None):
    """Global-layer verify: key_count keys (context plus the S proposals,
    "Announcing Carat", "More FLOPs can be faster"), queries at the last S
    positions.  Returns dict with key_count [B], q_pos [B][S],
    k, v [B][key_count_max][Hkv][D], q [B][S][Hq][D]."""
    g = rng(seed)
    kc = np.full(w.B, w.key_count if key_count is None else key_count, np.int32)
    kmax = int(kc.max())
    q_pos = (kc[:, None] - w.S + np.arange(w.S, dtype=np.int32)[None, :]).astype(np.int32)
    k = normal_bf16(g, (w.B, kmax, w.Hkv, w.D))
    v = normal_bf16(g, (w.B, kmax, w.Hkv, w.D))
    q = normal_bf16(g, (w.B, w.S, w.Hq, w.D))
    return dict(key_count=kc, q_pos=q_pos, k=k, v=v, q=q)


def mixed_contexts(seed: int = SEED_BASE + 5, B: int = MIXED_GLOBAL.B):
    """Context lengths of the mixed step, log-uniform on [512, 65536]."""
    return log_uniform_int(rng(seed), MIXED_GLOBAL.pos_lo, MIXED_GLOBAL.pos_hi, B)


def request_tokens(seed: int, b: int, n: int, hkv: int, d: int):
    """K and V (bf16 bits [n][Hkv][D]) for one request, drawn from a stream of
    its own so that large workloads can be produced one request at a time."""
    g = rng(seed * 100003 + b)
    return normal_bf16(g, (n, hkv, d)), normal_bf16(g, (n, hkv, d))
