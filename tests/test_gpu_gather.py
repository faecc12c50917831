"""GPU parity of swr_paged_gather_window, the paged-cache baseline
("Improving Decode Throughput on Intel Gaudi 3", Expensive KV gathers): the
ring bytes it leaves must be those of the oracle's gather, bit for bit, on
rings that start from random bytes (so untouched slots are checked too), and
a gather followed by the ring decode must attend as the oracle does over the
same window."""
import numpy as np
import pytest
import torch

import oracle
import sliding_window_ring_amd as swr
import synthetic
from gpu_common import dev_bf16, dev_i32, host_f64, layer, pool_bytes
from helpers import assert_parity

pytestmark = pytest.mark.gpu


def paged_case(seed, pos, W, hkv, d, pt, spare=5):
    """Request b's window tokens (positions lo_b = max(0, pos_b-W+1) .. pos_b,
    [B][W][Hkv][D], the first pos_b-lo_b+1 valid) laid out in pages of pt
    tokens whose ids are shuffled over a pool with `spare` unused pages.
    Only the pages holding window positions exist (earlier table entries are
    -1); their other rows hold noise."""
    g = synthetic.rng(seed)
    B = pos.size
    lo = np.maximum(pos - W + 1, 0)
    wk = synthetic.normal_bf16(g, (B, W, hkv, d))
    wv = synthetic.normal_bf16(g, (B, W, hkv, d))
    first, last = lo // pt, pos // pt
    n_used = int((last - first + 1).sum())
    ids = np.random.default_rng(seed).permutation(n_used + spare)
    bt = np.full((B, int(last.max()) + 1), -1, np.int32)
    kp = synthetic.normal_bf16(g, (n_used + spare, pt, hkv, d))
    vp = synthetic.normal_bf16(g, (n_used + spare, pt, hkv, d))
    k = 0
    for b in range(B):
        for i in range(int(first[b]), int(last[b]) + 1):
            bt[b, i] = ids[k]
            k += 1
            p0, p1 = max(i * pt, int(lo[b])), min(i * pt + pt - 1, int(pos[b]))
            kp[bt[b, i], p0 - i * pt:p1 - i * pt + 1] = wk[b, p0 - lo[b]:p1 - lo[b] + 1]
            vp[bt[b, i], p0 - i * pt:p1 - i * pt + 1] = wv[b, p0 - lo[b]:p1 - lo[b] + 1]
    return wk, wv, kp, vp, bt


def run_gather(W, d, hkv, pt, pos, seed, bt_edit=None):
    pos = np.asarray(pos, np.int32)
    B = pos.size
    wk, wv, kp, vp, bt = paged_case(seed, pos, W, hkv, d, pt)
    if bt_edit is not None:
        bt = bt_edit(bt, kp.shape[0])
    rb = oracle.region_bytes(W, hkv, d, oracle.BF16)
    g = synthetic.rng(seed + 1)
    k0 = g.integers(0, 256, B * rb, dtype=np.uint8)
    v0 = g.integers(0, 256, B * rb, dtype=np.uint8)
    off = np.arange(B, dtype=np.int64) * rb
    L = layer(k0.copy(), v0.copy(), off, off, W)
    swr.paged_gather_window(dev_bf16(kp), dev_bf16(vp), dev_i32(np.ascontiguousarray(bt)), dev_i32(pos), L)
    torch.cuda.synchronize()
    oracle.paged_gather_window(k0, v0, off, off, W, kp, vp, bt, pos)
    assert np.array_equal(pool_bytes(L.k_base), k0), "K ring bytes"
    assert np.array_equal(pool_bytes(L.v_base), v0), "V ring bytes"
    return L, wk, wv, pos


@pytest.mark.parametrize("D", [64, 128, 256, 512])
@pytest.mark.parametrize("W,pt", [(64, 16), (1024, 16), (96, 8), (256, 32), (40, 16)])
def test_gather_bytes_bit_exact(W, pt, D):
    # windows partly filled (pos < W - 1, partial 8-slot blocks), exactly
    # full, wrapped once and several times
    pos = [0, 5, W - 2, W - 1, W, W + 37, 3 * W + 13]
    run_gather(W, D, 2, pt, pos, seed=80 + D)


def test_gather_missing_pages_leave_slots_alone():
    def edit(bt, n_pages):
        bt = bt.copy()
        bt[0, 1] = -1
        bt[1, 0] = n_pages + 7
        bt[2, 3] = n_pages
        return bt[:, :-1]  # the last page of the longest request is past the table
    run_gather(64, 128, 2, 16, [40, 63, 200, 150], seed=91, bt_edit=edit)


def test_gather_decode_b56_shape():
    # the benchmark's decode shape (B=56, W=1024, 8 KV heads x 256), positions
    # U[1024, 4096]: gather, then the ring decode, against the oracle's decode
    # over the window appended in order
    W, hkv, d, G = 1024, 8, 256, 8
    pos = synthetic.uniform_int(synthetic.rng(92), 1024, 4096, 56)
    L, wk, wv, pos = run_gather(W, d, hkv, 16, pos, seed=93)
    q = synthetic.normal_bf16(synthetic.rng(94), (pos.size, hkv * G, d))
    scale = d ** -0.5
    out = swr.swa_decode(L, dev_bf16(q), dev_i32(pos), hkv, scale)
    torch.cuda.synchronize()
    rb = oracle.region_bytes(W, hkv, d, oracle.BF16)
    kp = np.zeros(pos.size * rb, np.uint8)
    vp = np.zeros(pos.size * rb, np.uint8)
    off = np.arange(pos.size, dtype=np.int64) * rb
    lo = np.maximum(pos - W + 1, 0).astype(np.int32)
    oracle.kv_append(kp, vp, off, off, W, oracle.BF16, 1.0, 1.0, wk, wv, lo, (pos - lo + 1).astype(np.int32))
    ref = oracle.swa_decode(kp, vp, off, off, W, oracle.BF16, 1.0, 1.0, q, pos, hkv, scale)
    assert_parity(host_f64(out), ref, "paged gather + ring decode, B=56")
