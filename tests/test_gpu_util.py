"""The library's utility kernels on the GPU: zero fill over ragged ranges (the
pool zero-fills every region it hands out) and the streaming-read
measurement kernel.  Neither may touch a byte outside its range."""
import numpy as np
import pytest
import torch

import sliding_window_ring_amd as swr

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("offset,nbytes", [(0, 0), (0, 16), (3, 1), (5, 29), (16, 4096), (7, (1 << 20) + 9),
                                           (0, 1 << 22)])
def test_zero_fill_exact_range(offset, nbytes):
    t = torch.full(((1 << 22) + 64,), 0xA5, dtype=torch.uint8, device="cuda")
    swr.zero_fill(t, offset, nbytes)
    torch.cuda.synchronize()
    h = t.cpu().numpy()
    assert np.all(h[offset:offset + nbytes] == 0)
    assert np.all(h[:offset] == 0xA5) and np.all(h[offset + nbytes:] == 0xA5)


@pytest.mark.parametrize("pattern", [0, 1])
@pytest.mark.parametrize("grid", [1, 7, 256, 65536])
def test_read_ceiling_reads_and_leaves_memory_alone(grid, pattern):
    src = torch.arange((1 << 20) + 48, dtype=torch.int32, device="cuda").view(torch.uint8)
    before = src.clone()
    guard = torch.full((3 * 1024,), 0x3C, dtype=torch.uint8, device="cuda")
    swr.read_ceiling(src, guard[1024:2048], grid, pattern)
    torch.cuda.synchronize()
    assert torch.equal(src, before)
    g = guard.cpu().numpy()
    assert np.all(g[:1024] == 0x3C) and np.all(g[2048:] == 0x3C)


def test_pool_admit_zero_fills_each_region_and_nothing_else():
    # one request of a small Gemma-like mix: 5 rings of 64 slots (2 x 64) and
    # 2 global regions of a 300-token context (1 x 128) -> cap 320
    pool = swr.Pool(8 << 20)
    pool.buffer.fill_(0xA5)
    ko, vo, cap = pool.admit(5, 64, 2, 64, 2, 300, 1, 128)
    torch.cuda.synchronize()
    assert cap == 320
    h = pool.buffer.cpu().numpy()
    mask = np.zeros(h.size, bool)
    for i, (k, v) in enumerate(zip(ko, vo)):
        rb = swr.region_bytes(64, 2, 64) if i < 5 else swr.region_bytes(320, 1, 128)
        mask[k:k + rb] = True
        mask[v:v + rb] = True
    assert np.all(h[mask] == 0) and np.all(h[~mask] == 0xA5)
    pool.release(ko, vo)
    assert pool.stats()[0] == 0


@pytest.mark.gpu
def test_ring_and_global_carves_zero_fill_their_regions_and_nothing_else():
    # a ring of 1001 slots (rounded to 1008) and a global region of 6005
    # tokens (rounded to 6016, the padded tail included) carved from a pool
    # whose bytes start non-zero
    pool = swr.Pool(32 << 20)
    pool.buffer.fill_(0x5A)
    rk, rv, rcap = pool.alloc_ring(1001, 2, 64)
    gk, gv, gcap = pool.alloc_global(6005, 2, 512)
    torch.cuda.synchronize()
    assert (rcap, gcap) == (1008, 6016)
    h = pool.buffer.cpu().numpy()
    mask = np.zeros(h.size, bool)
    for o, n in ((rk, swr.region_bytes(1008, 2, 64)), (rv, swr.region_bytes(1008, 2, 64)),
                 (gk, swr.region_bytes(6016, 2, 512)), (gv, swr.region_bytes(6016, 2, 512))):
        mask[o:o + n] = True
    assert np.all(h[mask] == 0) and np.all(h[~mask] == 0x5A)
    for o in (rk, rv, gk, gv):
        pool.free(o)
    assert pool.stats()[0] == 0
