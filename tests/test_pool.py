"""CPU tests of the pool carve (host bookkeeping only; no device memory).

"Improving Decode Throughput on Intel Gaudi 3" (Our approach): ring buffers
are carved from the same HBM pool as global-layer KV, so their balance follows
the request mix.  The pool here is first fit over byte ranges with 256-byte
alignment; global regions are rounded up to 64 slots ("Announcing Carat",
More FLOPs can be faster: the padded tail).  The reference model below is a
plain list-based first-fit allocator, written independently of the C++ one.
"""
import ctypes
import random

import pytest

import sliding_window_ring_amd as swr

ALIGN = 256


class Pool:
    def __init__(self, size):
        self.h = ctypes.c_void_p()
        assert swr.lib.swr_pool_create(size, ctypes.byref(self.h)) == 0

    def alloc(self, n):
        off = ctypes.c_int64(-1)
        st = swr.lib.swr_pool_alloc(self.h, n, ctypes.byref(off))
        return st, off.value

    def free(self, off):
        return swr.lib.swr_pool_free(self.h, off)

    def stats(self):
        u, l = ctypes.c_size_t(), ctypes.c_size_t()
        assert swr.lib.swr_pool_stats(self.h, ctypes.byref(u), ctypes.byref(l)) == 0
        return u.value, l.value

    def __del__(self):
        swr.lib.swr_pool_destroy(self.h)


class ModelPool:
    """First fit over a sorted list of (start, size) ranges."""

    def __init__(self, size):
        self.size = size
        self.ranges = []

    def alloc(self, n):
        cursor = 0
        for i, (s, z) in enumerate(self.ranges):
            start = -(-cursor // ALIGN) * ALIGN
            if start + n <= s:
                self.ranges.insert(i, (start, n))
                return start
            cursor = s + z
        start = -(-cursor // ALIGN) * ALIGN
        if start + n > self.size:
            return None
        self.ranges.append((start, n))
        return start

    def free(self, off):
        for i, (s, _) in enumerate(self.ranges):
            if s == off:
                del self.ranges[i]
                return True
        return False


def test_random_alloc_free_matches_first_fit_model():
    rnd = random.Random(7)
    size = 1 << 24
    p, m = Pool(size), ModelPool(size)
    live = []
    for _ in range(3000):
        if live and rnd.random() < 0.45:
            off = live.pop(rnd.randrange(len(live)))
            assert p.free(off) == 0 and m.free(off)
        else:
            n = rnd.choice([1, 255, 256, 4096, 100000, 1 << 20, rnd.randrange(1, 300000)])
            st, off = p.alloc(n)
            want = m.alloc(n)
            if want is None:
                assert st == 5  # SWR_ERR_NOMEM
            else:
                assert st == 0 and off == want
                live.append(off)
        # invariants: aligned, inside the pool, disjoint
        rs = sorted(m.ranges)
        for (s, z), (s2, _) in zip(rs, rs[1:]):
            assert s + z <= s2
        assert all(s % ALIGN == 0 and s + z <= size for s, z in rs)
    used, _ = p.stats()
    assert used == sum(z for _, z in m.ranges)


def test_free_unknown_offset_is_rejected():
    p = Pool(1 << 20)
    st, off = p.alloc(1000)
    assert st == 0
    assert p.free(off + 256) == 1
    assert p.free(off) == 0
    assert p.free(off) == 1


def test_exhaustion_and_reuse():
    p = Pool(4096)
    st, a = p.alloc(4096)
    assert st == 0 and a == 0
    assert p.alloc(1)[0] == 5
    assert p.free(a) == 0
    assert p.alloc(4096) == (0, 0)


@pytest.mark.parametrize("tokens,global_layer,cap", [(1024, 0, 1024), (1000, 0, 1000), (1001, 0, 1008),
                                                     (6005, 1, 6016), (6016, 1, 6016), (1, 1, 64)])
def test_alloc_kv_rounds_capacity(tokens, global_layer, cap):
    p = Pool(1 << 28)
    ko, vo, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    assert swr.lib.swr_pool_alloc_kv(p.h, tokens, 2, 512, 0, global_layer, ctypes.byref(ko), ctypes.byref(vo),
                                     ctypes.byref(c)) == 0
    assert c.value == cap
    rb = swr.region_bytes(cap, 2, 512)
    assert vo.value >= ko.value + rb and ko.value % ALIGN == 0 and vo.value % ALIGN == 0
    assert p.stats()[0] == 2 * rb


def test_alloc_kv_failure_releases_the_first_region():
    rb = swr.region_bytes(1024, 8, 256)
    p = Pool(rb + rb // 2)
    ko, vo, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
    assert swr.lib.swr_pool_alloc_kv(p.h, 1024, 8, 256, 0, 0, ctypes.byref(ko), ctypes.byref(vo),
                                     ctypes.byref(c)) == 5
    assert p.stats()[0] == 0


def test_mixed_rings_and_global_regions_share_one_pool():
    # 16 requests: one ring (1024 slots) and one global region each, as in the
    # mixed serving step; every range is disjoint and inside the pool.
    ctx = [512, 700, 1500, 3000, 5000, 9000, 12000, 20000, 30000, 40000, 50000, 60000, 65536, 800, 2048, 4096]
    p = Pool(1 << 31)
    ranges = []
    for n in ctx:
        for tokens, hkv, d, g in ((1024, 8, 256, 0), (n + 1, 2, 512, 1)):
            ko, vo, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
            assert swr.lib.swr_pool_alloc_kv(p.h, tokens, hkv, d, 0, g, ctypes.byref(ko), ctypes.byref(vo),
                                             ctypes.byref(c)) == 0
            rb = swr.region_bytes(c.value, hkv, d)
            ranges += [(ko.value, rb), (vo.value, rb)]
            if g:
                assert c.value % 64 == 0 and c.value >= n + 1
    ranges.sort()
    for (s, z), (s2, _) in zip(ranges, ranges[1:]):
        assert s + z <= s2
