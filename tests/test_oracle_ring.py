"""Pins for the oracle's append / slot mapping.

"Announcing Carat" (Replacing page lookups with a ring buffer): a token's slot
is its absolute position modulo the window, and a new token reuses the oldest
slot without moving the rest.  "Improving Decode Throughput on Intel Gaudi 3"
(Our approach): K and V of a token are written together, so both rings carry
the same rotation.  The region layout read back here uses numpy reshapes of
the declared layout, not the oracle's own index arithmetic: S = cap rounded
up to 32 slots per KV head; K [Hkv][S/32][2][D/R][16][R] with R the dims of
a 16-byte granule and slot 32t + k in half (k/4)%2, row 4*(k/8) + k%4 of
tile t; V in 8-slot blocks [Hkv][S/8][D][8].
"""
import numpy as np
import pytest

import oracle
import synthetic
from helpers import f64


def stored(cap):
    return -(-cap // 32) * 32


def k_view(pool, off, cap, hkv, d, esize=2):
    """[slot][Hkv][D] view of a K region: tiles of 32 slots, each two halves
    of 16 rows; a half holds blocks of four 16-byte granules, row-major within
    the block ([Hkv][S/32][2][D/(4R)][16][4][R])."""
    S, R = stored(cap), 16 // esize
    a = pool[off:off + S * hkv * d * esize].view(np.uint16 if esize == 2 else np.uint8)
    a = a.reshape(hkv, S // 32, 2, d // (4 * R), 16, 4, R)
    slot = np.arange(cap)
    t, k = slot // 32, slot % 32
    half, row = (k // 4) % 2, 4 * (k // 8) + k % 4
    return a[:, t, half, :, row, :, :].reshape(cap, hkv, d)


def v_view(pool, off, cap, hkv, d, esize=2):
    """[slot][Hkv][D] view of a V region laid out [Hkv][S/8][D][8]."""
    S = stored(cap)
    v = pool[off:off + S * hkv * d * esize].view(np.uint16 if esize == 2 else np.uint8).reshape(hkv, S // 8, d, 8)
    return v.transpose(1, 3, 0, 2).reshape(S, hkv, d)[:cap]


def position_tokens(n, hkv, d, base=0):
    """Token t carries value (base + t) in every element (exact in bf16 for
    small integers), and its V carries -(base + t)."""
    vals = np.arange(base, base + n, dtype=np.float32)
    k = np.broadcast_to(vals[:, None, None], (n, hkv, d))
    return synthetic.bf16_bits(k), synthetic.bf16_bits(-k)


def test_slot_is_position_mod_window_one_by_one():
    W, hkv, d = 16, 2, 32
    rb = oracle.region_bytes(W, hkv, d, oracle.BF16)
    kp = np.zeros(rb, np.uint8)
    vp = np.zeros(rb, np.uint8)
    off = np.zeros(1, np.int64)
    k, v = position_tokens(40, hkv, d, base=1)  # value = position + 1 (0 = empty)
    for t in range(40):
        oracle.kv_append(kp, vp, off, off, W, oracle.BF16, 1.0, 1.0, k[None, t:t + 1], v[None, t:t + 1],
                         np.array([t], np.int32))
        K = f64(k_view(kp, 0, W, hkv, d))
        V = f64(v_view(vp, 0, W, hkv, d))
        for s in range(W):
            # newest position j <= t with j = s (mod W), or empty
            cands = [j for j in range(t + 1) if j % W == s]
            want = (max(cands) + 1) if cands else 0
            assert np.all(K[s] == want), (t, s)
            assert np.all(V[s] == -want), (t, s)


def test_batched_append_equals_sequential_appends():
    W, hkv, d, T = 16, 1, 32, 37
    g = synthetic.rng(5)
    k = synthetic.normal_bf16(g, (3, T, hkv, d))
    v = synthetic.normal_bf16(g, (3, T, hkv, d))
    pos0 = np.array([0, 5, 1000], np.int32)
    n_new = np.array([37, 20, 3], np.int32)
    rb = oracle.region_bytes(W, hkv, d, oracle.BF16)
    off = np.arange(3, dtype=np.int64) * rb
    kp1, vp1 = np.zeros(3 * rb, np.uint8), np.zeros(3 * rb, np.uint8)
    oracle.kv_append(kp1, vp1, off, off, W, oracle.BF16, 1, 1, k, v, pos0, n_new)
    kp2, vp2 = np.zeros(3 * rb, np.uint8), np.zeros(3 * rb, np.uint8)
    for b in range(3):
        for t in range(n_new[b]):
            oracle.kv_append(kp2, vp2, off[b:b + 1], off[b:b + 1], W, oracle.BF16, 1, 1,
                             k[b:b + 1, t:t + 1], v[b:b + 1, t:t + 1], np.array([pos0[b] + t], np.int32))
    assert np.array_equal(kp1, kp2) and np.array_equal(vp1, vp2)


def test_global_mode_slot_is_position_and_bounds():
    cap, hkv, d = 64, 2, 32
    rb = oracle.region_bytes(cap, hkv, d, oracle.BF16)
    kp, vp = np.zeros(rb, np.uint8), np.zeros(rb, np.uint8)
    off = np.zeros(1, np.int64)
    k, v = position_tokens(10, hkv, d, base=50)
    oracle.kv_append(kp, vp, off, off, cap, oracle.BF16, 1, 1, k[None], v[None], np.array([50], np.int32),
                     wrap=False)
    K = f64(k_view(kp, 0, cap, hkv, d))
    for s in range(cap):
        assert np.all(K[s] == (s if 50 <= s < 60 else 0))
    with pytest.raises(ValueError):  # position 64 would be outside the region
        oracle.kv_append(kp, vp, off, off, cap, oracle.BF16, 1, 1, k[None], v[None],
                         np.array([55], np.int32), wrap=False)


def test_fp8_append_stores_encoded_codes():
    W, hkv, d = 16, 2, 64
    g = synthetic.rng(9)
    k = synthetic.normal_bf16(g, (1, 5, hkv, d))
    v = synthetic.normal_bf16(g, (1, 5, hkv, d))
    ks, vs = 0.0123, 0.0456
    rb = oracle.region_bytes(W, hkv, d, oracle.FP8)
    kp, vp = np.zeros(rb, np.uint8), np.zeros(rb, np.uint8)
    off = np.zeros(1, np.int64)
    oracle.kv_append(kp, vp, off, off, W, oracle.FP8, ks, vs, k, v, np.array([14], np.int32))
    K = k_view(kp, 0, W, hkv, d, esize=1)
    V = v_view(vp, 0, W, hkv, d, esize=1)
    for t in range(5):
        s = (14 + t) % W
        assert np.array_equal(K[s], oracle.e4m3_encode(k[0, t], ks))
        assert np.array_equal(V[s], oracle.e4m3_encode(v[0, t], vs))


def scatter_to_pages(tokens_k, tokens_v, pt, rng, spare=3):
    """Lays out each request's token sequence ([B][n][Hkv][D] bits) in pages of
    pt tokens whose ids are shuffled over the pool (with `spare` unused
    pages): page block_table[b][i] holds positions pt*i .. pt*i+pt-1."""
    B, n, hkv, d = tokens_k.shape
    per = -(-n // pt)
    ids = rng.permutation(B * per + spare)
    bt = ids[:B * per].reshape(B, per).astype(np.int32)
    kp = np.zeros((B * per + spare, pt, hkv, d), np.uint16)
    vp = np.zeros_like(kp)
    for b in range(B):
        for p in range(n):
            kp[bt[b, p // pt], p % pt] = tokens_k[b, p]
            vp[bt[b, p // pt], p % pt] = tokens_v[b, p]
    return kp, vp, bt


@pytest.mark.parametrize("W,pt,pos", [(16, 4, [3, 15, 16, 37]), (32, 16, [0, 31, 45, 100]), (64, 16, [63, 64, 65, 130])])
def test_paged_gather_puts_each_window_position_in_its_slot(W, pt, pos):
    # "Improving Decode Throughput on Intel Gaudi 3" (Expensive KV gathers):
    # the window of the query at pos, read from pages, lands where the ring
    # keeps it; the slots read back through the layout views above
    hkv, d, B = 2, 32, len(pos)
    n = max(pos) + 1
    # position p of request b carries (p + 1) * 2^b: exact in bf16, distinct per request
    vals = np.arange(1, n + 1, dtype=np.float32)[None, :, None, None] * 2.0 ** np.arange(B)[:, None, None, None]
    tk = synthetic.bf16_bits(np.broadcast_to(vals, (B, n, hkv, d)))
    tv = synthetic.bf16_bits(-np.broadcast_to(vals, (B, n, hkv, d)))
    kp, vp, bt = scatter_to_pages(tk, tv, pt, np.random.default_rng(5))
    rb = oracle.region_bytes(W, hkv, d, oracle.BF16)
    kpool = np.zeros(B * rb, np.uint8)
    vpool = np.zeros(B * rb, np.uint8)
    off = np.arange(B, dtype=np.int64) * rb
    oracle.paged_gather_window(kpool, vpool, off, off, W, kp, vp, bt, np.array(pos, np.int32))
    for b, P in enumerate(pos):
        kv = f64(k_view(kpool, int(off[b]), W, hkv, d))
        vv = f64(v_view(vpool, int(off[b]), W, hkv, d))
        for s in range(W):
            p = P - ((P - s) % W)
            want = (p + 1) * 2.0 ** b if p >= 0 else 0.0
            assert np.all(kv[s] == want), (b, s)
            assert np.all(vv[s] == -want if p >= 0 else vv[s] == 0.0), (b, s)


def test_paged_gather_equals_appending_the_window():
    # the same rings as appending each request's last W tokens in order
    W, pt, hkv, d = 32, 16, 2, 64
    g = synthetic.rng(41)
    pos = np.array([5, 40, 95], np.int32)
    B, n = pos.size, int(pos.max()) + 1
    tk = synthetic.normal_bf16(g, (B, n, hkv, d))
    tv = synthetic.normal_bf16(g, (B, n, hkv, d))
    kp, vp, bt = scatter_to_pages(tk, tv, pt, np.random.default_rng(6))
    rb = oracle.region_bytes(W, hkv, d, oracle.BF16)
    off = np.arange(B, dtype=np.int64) * rb
    got_k, got_v = np.zeros(B * rb, np.uint8), np.zeros(B * rb, np.uint8)
    oracle.paged_gather_window(got_k, got_v, off, off, W, kp, vp, bt, pos)
    want_k, want_v = np.zeros(B * rb, np.uint8), np.zeros(B * rb, np.uint8)
    for b in range(B):
        lo = max(0, int(pos[b]) - W + 1)
        oracle.kv_append(want_k, want_v, off[b:b + 1], off[b:b + 1], W, oracle.BF16, 1.0, 1.0,
                         tk[b:b + 1, lo:pos[b] + 1], tv[b:b + 1, lo:pos[b] + 1], np.array([lo], np.int32))
    assert np.array_equal(got_k, want_k) and np.array_equal(got_v, want_v)


def test_paged_gather_skips_missing_pages():
    W, pt, hkv, d = 16, 4, 1, 32
    n = 20
    vals = np.arange(1, n + 1, dtype=np.float32)[None, :, None, None]
    tk = synthetic.bf16_bits(np.broadcast_to(vals, (1, n, hkv, d)))
    kp, vp, bt = scatter_to_pages(tk, tk, pt, np.random.default_rng(7), spare=0)
    bt = bt.copy()
    bt[0, 2] = -1               # positions 8..11
    bt[0, 3] = kp.shape[0] + 4  # positions 12..15: not a page of the pool
    rb = oracle.region_bytes(W, hkv, d, oracle.BF16)
    kpool = np.full(rb, 0x11, np.uint8)
    vpool = np.full(rb, 0x11, np.uint8)
    off = np.zeros(1, np.int64)
    oracle.paged_gather_window(kpool, vpool, off, off, W, kp, vp, bt[:, :4], np.array([19], np.int32))
    kv = k_view(kpool, 0, W, hkv, d)
    for p in range(4, 20):
        s = p % W
        if 8 <= p < 20:  # pages 2, 3 missing; page 4 is past the table's 4 columns
            assert np.all(kv[s] == 0x1111), p
        else:
            assert np.all(f64(kv[s]) == p + 1), p


# --- the layout codec: the device byte layout against the numpy views above
# (written from the declared layout, independently of the codec's index
# arithmetic), on random bytes, ragged capacities and both element types

CODEC_SHAPES = [(16, 1, 64, oracle.BF16), (40, 2, 32, oracle.BF16), (1024, 2, 256, oracle.BF16),
                (40, 2, 64, oracle.FP8), (1000, 1, 512, oracle.FP8)]


@pytest.mark.parametrize("cap,hkv,d,dtype", CODEC_SHAPES)
def test_codec_unpack_matches_layout_views(cap, hkv, d, dtype):
    g = synthetic.rng(cap + 7 * d + dtype)
    esize = 2 if dtype == oracle.BF16 else 1
    rb = oracle.region_bytes(cap, hkv, d, dtype)
    assert rb == stored(cap) * hkv * d * esize
    region = g.integers(0, 256, rb, dtype=np.uint8)
    et = np.uint16 if esize == 2 else np.uint8
    for is_v, view in ((False, k_view), (True, v_view)):
        got = oracle.unpack_region(region, cap, hkv, d, dtype, is_v).view(et).reshape(cap, hkv, d)
        assert np.array_equal(got, view(region, 0, cap, hkv, d, esize)), is_v


@pytest.mark.parametrize("cap,hkv,d,dtype", CODEC_SHAPES)
def test_codec_round_trips(cap, hkv, d, dtype):
    g = synthetic.rng(3 * cap + d + dtype)
    rb = oracle.region_bytes(cap, hkv, d, dtype)
    lb = oracle.logical_region_bytes(cap, hkv, d, dtype)
    assert lb == cap * hkv * d * (2 if dtype == oracle.BF16 else 1)
    for is_v in (False, True):
        logical = g.integers(0, 256, lb, dtype=np.uint8)
        region = np.zeros(rb, np.uint8)
        oracle.pack_region(logical, region, cap, hkv, d, dtype, is_v)
        assert np.array_equal(oracle.unpack_region(region, cap, hkv, d, dtype, is_v), logical)
        # every logical byte lands somewhere, and only the padding slots stay zero
        assert np.count_nonzero(region) == np.count_nonzero(logical)
        region2 = g.integers(0, 256, rb, dtype=np.uint8)
        back = region2.copy()
        oracle.pack_region(oracle.unpack_region(region2, cap, hkv, d, dtype, is_v), back, cap, hkv, d, dtype,
                           is_v)
        assert np.array_equal(back, region2)
