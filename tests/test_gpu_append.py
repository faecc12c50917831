"""GPU parity of swr_kv_append against the oracle: the appended region bytes
must be identical (bf16 copies and fp8 codes alike), on rings and on global
regions ("Announcing Carat", ring buffer section: slot = position mod window;
"Improving Decode Throughput on Intel Gaudi 3", Our approach: K and V go to
the same slot)."""
import numpy as np
import pytest
import torch

import oracle
import synthetic
from gpu_common import dev_bf16, dev_i32, layer, pool_bytes

pytestmark = pytest.mark.gpu


def fitting(pos0, n_new, T, cap):
    """(pos0, counts) of the tokens of each request that land below a global
    region's capacity: what the library's dropping of positions past it
    leaves written.  The oracle refuses such positions rather than dropping
    them; a request none of whose tokens fit starts at the capacity with
    none to write."""
    p = np.asarray(pos0, np.int64)
    n = np.full(len(p), T, np.int64) if n_new is None else np.asarray(n_new, np.int64)
    fit = np.clip(np.minimum(n, cap - p), 0, None)
    return np.minimum(p, cap).astype(np.int32), fit.astype(np.int32)


def run_both(B, T, hkv, d, cap, dtype, ks, vs, pos0, n_new, wrap, seed, special=False, oracle_tokens=None):
    """The library's append and the oracle's on the same starting bytes;
    oracle_tokens: the oracle's (pos0, counts) where they differ (global
    positions past the capacity, see fitting)."""
    g = synthetic.rng(seed)
    rb = oracle.region_bytes(cap, hkv, d, dtype)
    # start from the same random bytes on both sides so untouched slots are checked too
    k_pool = g.integers(0, 256, B * rb + 512, dtype=np.uint8)
    v_pool = g.integers(0, 256, B * rb + 512, dtype=np.uint8)
    k_off = np.arange(B, dtype=np.int64) * rb + 256
    v_off = k_off.copy()
    k_new = synthetic.normal_bf16(g, (B, T, hkv, d))
    v_new = synthetic.normal_bf16(g, (B, T, hkv, d))
    if special:
        # saturation, subnormals, exact E4M3 midpoints (at scale 1), signed zeros, infinities
        vals = np.array([448.0, 465.0, 1e5, -1e5, 2.0 ** -10, 3 * 2.0 ** -10, 2.0 ** -12, 1.0625, 1.1875,
                         -0.0, 0.0, np.inf, -np.inf, 0.017578125, 240.0, -232.0], np.float32)
        flat = k_new.reshape(-1)
        flat[:vals.size] = synthetic.bf16_bits(vals)
        flat = v_new.reshape(-1)
        flat[-vals.size:] = synthetic.bf16_bits(vals[::-1].copy())
    L = layer(k_pool, v_pool, k_off, v_off, cap, dtype, ks, vs)
    import sliding_window_ring_amd as swr
    swr.ring_kv_append(L, dev_bf16(k_new), dev_bf16(v_new), dev_i32(pos0),
                  None if n_new is None else dev_i32(n_new), wrap=wrap)
    torch.cuda.synchronize()
    op0, on = (pos0, n_new) if oracle_tokens is None else oracle_tokens
    oracle.kv_append(k_pool, v_pool, k_off, v_off, cap, dtype, ks, vs, k_new, v_new, op0, on, wrap=wrap)
    gk, gv = pool_bytes(L.k_base), pool_bytes(L.v_base)
    nk = int(np.count_nonzero(gk != k_pool))
    nv = int(np.count_nonzero(gv != v_pool))
    assert nk == 0 and nv == 0, f"{nk} K bytes and {nv} V bytes differ"


def test_ring_decode_batch_one_token():
    # the B=56 decode shape: one new token per request, rings already wrapped
    pos = synthetic.uniform_int(synthetic.rng(1), 1024, 4096, 56)
    run_both(56, 1, 8, 256, 1024, oracle.BF16, 1, 1, pos, None, True, seed=2)


def test_ring_many_tokens_wraps_and_ragged_counts():
    # more tokens than slots: only the last W of each request survive
    run_both(3, 40, 2, 64, 16, oracle.BF16, 1, 1, np.array([0, 7, 1000], np.int32),
             np.array([40, 17, 3], np.int32), True, seed=3)


def test_ring_every_head_dim():
    for d in (64, 128, 512):
        run_both(2, 5, 3, d, 32, oracle.BF16, 1, 1, np.array([30, 3], np.int32), None, True, seed=4 + d)


def test_global_region_slots_are_positions():
    run_both(2, 4, 2, 512, 6016, oracle.BF16, 1, 1, np.array([6001, 0], np.int32), None, False, seed=5)


def test_global_positions_past_capacity_are_dropped():
    # the library drops positions past the capacity: tokens 4..7 of request 0
    # and all of request 1 fall past it, request 2 fits exactly; every byte
    # equals the oracle's append of the tokens that fit
    pos0 = np.array([60, 64, 56], np.int32)
    run_both(3, 8, 1, 64, 64, oracle.BF16, 1, 1, pos0, None, False, seed=6, oracle_tokens=fitting(pos0, None, 8, 64))


@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (0.0123, 0.0456), (2.0 ** -4, 3.0), (1e-3, 7.5)])
def test_fp8_codes_bit_exact(ks, vs):
    run_both(4, 9, 2, 256, 64, oracle.FP8, ks, vs, np.array([0, 60, 2000, 5], np.int32),
             np.array([9, 9, 4, 0], np.int32), True, seed=7, special=True)


def test_fp8_decode_batch_shape():
    pos = synthetic.uniform_int(synthetic.rng(8), 1024, 4096, 56)
    run_both(56, 1, 8, 256, 1024, oracle.FP8, 0.0107, 0.0093, pos, None, True, seed=9, special=True)


def test_fp8_every_bf16_value():
    # all 65536 bf16 patterns except NaNs through the device encoder, at scale
    # 1, arbitrary scales, the smallest positive fp32 (a subnormal scale) and
    # scales near both ends of the fp32 range: 256 tokens x 256 dims of one
    # request
    allb = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    allb = allb[~np.isnan(synthetic.bf16_to_f32(allb))]
    n = allb.size
    pad = (-n) % 256
    vals = np.concatenate([allb, np.zeros(pad, np.uint16)]).reshape(1, -1, 1, 256)
    T = vals.shape[1]
    for s in (1.0, 0.37, 0.0123, 2.0 ** -149, 1e-30, 3e37, 3.4028235e38):
        rb = oracle.region_bytes(256, 1, 256, oracle.FP8)
        kp = np.zeros(rb, np.uint8)
        vp = np.zeros(rb, np.uint8)
        off = np.zeros(1, np.int64)
        L = layer(kp, vp, off, off, 256, oracle.FP8, s, s)
        import sliding_window_ring_amd as swr
        swr.ring_kv_append(L, dev_bf16(vals), dev_bf16(vals), dev_i32([0]), wrap=False)
        torch.cuda.synchronize()
        oracle.kv_append(kp, vp, off, off, 256, oracle.FP8, s, s, vals, vals, np.array([0], np.int32), wrap=False)
        assert np.array_equal(pool_bytes(L.k_base), kp)
        assert np.array_equal(pool_bytes(L.v_base), vp)
        assert T == 256
