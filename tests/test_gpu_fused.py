"""GPU parity of the fused append + attention calls against the oracle.

swr_swa_append_decode must leave the ring with the bytes the oracle's append
of the new token leaves (bit-exact), and return the oracle's decode over that
ring; swr_global_append_attend likewise for the S proposals written into a
global region at pos0 .. pos0+S-1 and the oracle's global attention with
key_count = pos0 + S and queries at pos0 + i ("Announcing Carat", ring buffer
section and "More FLOPs can be faster").  Before each call the slots being
written hold stale tokens (the one a ring slot evicts, rejected proposals in a
global region), so a missing or misplaced store shows in the bytes and in the
output.  Outputs are held to max-abs <= 1e-2 and relative L2 <= 5e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import sliding_window_ring_amd as swr
import synthetic
from gpu_common import dev_bf16, dev_i32, host_bits, host_f64, layer
from helpers import assert_parity, global_pools, ring_pools

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------ sliding decode

def fused_decode_case(w, x, dtype=oracle.BF16, ks=1.0, vs=1.0, seed=61):
    """The ring holds the window's tokens older than pos and, in the new
    token's slot, the token it evicts (position pos - W) where there is one.
    Returns (gpu out, oracle out, gpu K bytes, gpu V bytes, oracle K, oracle V)."""
    B, W = w.B, w.W
    scale = 1.0 / np.sqrt(w.D)
    n, pos = x["n"], x["pos"]
    kp, vp, ko, vo = ring_pools(x["k"], x["v"], x["start"], n - 1, W, dtype, ks, vs)
    g = synthetic.rng(seed)
    stale_k = synthetic.normal_bf16(g, (B, 1, w.Hkv, w.D))
    stale_v = synthetic.normal_bf16(g, (B, 1, w.Hkv, w.D))
    oracle.kv_append(kp, vp, ko, vo, W, dtype, ks, vs, stale_k, stale_v, np.maximum(pos - W, 0).astype(np.int32),
                     (pos >= W).astype(np.int32), wrap=True)
    kn = np.ascontiguousarray(x["k"][np.arange(B), n - 1])  # [B][Hkv][D], the token at pos
    vn = np.ascontiguousarray(x["v"][np.arange(B), n - 1])
    L = layer(kp, vp, ko, vo, W, dtype, ks, vs)
    out = swr.swa_append_decode(L, dev_bf16(kn), dev_bf16(vn), dev_bf16(x["q"]), dev_i32(pos), scale)
    torch.cuda.synchronize()
    oracle.kv_append(kp, vp, ko, vo, W, dtype, ks, vs, kn[:, None], vn[:, None], pos, wrap=True)
    ref = oracle.swa_decode(kp, vp, ko, vo, W, dtype, ks, vs, x["q"], pos, w.Hkv, scale)
    return out, ref, L.k_base.cpu().numpy(), L.v_base.cpu().numpy(), kp, vp


def check_decode(w, x, what, dtype=oracle.BF16, ks=1.0, vs=1.0):
    out, ref, gk, gv, kp, vp = fused_decode_case(w, x, dtype, ks, vs)
    assert np.array_equal(gk, kp), f"{what}: K ring bytes"
    assert np.array_equal(gv, vp), f"{what}: V ring bytes"
    return assert_parity(host_f64(out), ref, what)


def test_fused_decode_tiny_sequence_step_by_step():
    """Workload 1 through the fused call: 40 tokens, one call per step; the
    ring bytes equal the oracle's after every step and step 0 (one visible
    key) returns that key's value bits exactly."""
    w = synthetic.TINY
    q, k, v = synthetic.tiny_sequence()
    rb = oracle.region_bytes(w.W, w.Hkv, w.D, oracle.BF16)
    kp = np.zeros(rb, np.uint8)
    vp = np.zeros(rb, np.uint8)
    off = np.zeros(1, np.int64)
    L = layer(kp, vp, off, off, w.W)
    scale = 1.0 / np.sqrt(w.D)
    for t in range(w.steps):
        pos = np.array([t], np.int32)
        out = swr.swa_append_decode(L, dev_bf16(k[None, t]), dev_bf16(v[None, t]), dev_bf16(q[None, t]),
                                    dev_i32(pos), scale)
        torch.cuda.synchronize()
        oracle.kv_append(kp, vp, off, off, w.W, oracle.BF16, 1, 1, k[None, t:t + 1], v[None, t:t + 1], pos)
        assert np.array_equal(L.k_base.cpu().numpy(), kp), t
        assert np.array_equal(L.v_base.cpu().numpy(), vp), t
        ref = oracle.swa_decode(kp, vp, off, off, w.W, oracle.BF16, 1, 1, q[None, t], pos, w.Hkv, scale)
        assert_parity(host_f64(out), ref, f"step {t}")
        if t == 0:
            assert np.array_equal(host_bits(out)[0], np.repeat(v[0], w.G, axis=0))


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_fused_decode_b56_full_workload(dtype):
    w = synthetic.SWA_DECODE
    ks, vs = (0.0107, 0.0093) if dtype == oracle.FP8 else (1.0, 1.0)
    e = check_decode(w, synthetic.sliding_decode(w), "fused B=56 decode", dtype, ks, vs)
    print("fused B=56 decode max-abs %.3e rel-L2 %.3e" % e)


@pytest.mark.parametrize("positions", [
    (0, 1, 2, 15, 16, 31, 32, 33),          # partial rings: the new token's tile is the last one
    (1022, 1023, 1024, 1025, 2047, 5000, 100000, 63),
    (1024, 1056, 1088, 1119, 1151, 1183, 1215, 1247),  # the new slot at the start/end of tiles
])
def test_fused_decode_edges(positions):
    # 8 requests x 8 KV heads: split-K, so the split holding the new slot varies
    w = synthetic.Workload("t", B=len(positions), Hkv=8, G=8, D=256, W=1024)
    x = synthetic.sliding_decode(w, seed=62, positions=positions)
    check_decode(w, x, f"fused decode {positions}")


@pytest.mark.parametrize("D,G,Hkv,W", [(64, 1, 4, 64), (128, 4, 2, 256), (512, 2, 2, 128), (256, 16, 1, 96),
                                       (64, 2, 1, 16), (512, 8, 2, 1024)])
def test_fused_decode_shapes(D, G, Hkv, W):
    w = synthetic.Workload("t", B=5, Hkv=Hkv, G=G, D=D, W=W)
    x = synthetic.sliding_decode(w, seed=63, positions=(0, W // 2 + 3, W - 1, W, 3 * W + 5))
    check_decode(w, x, f"fused decode D={D} G={G}")


@pytest.mark.parametrize("D,G", [(64, 2), (128, 16), (256, 8), (512, 8)])
def test_fused_decode_fp8(D, G):
    w = synthetic.Workload("t", B=5, Hkv=2, G=G, D=D, W=128)
    x = synthetic.sliding_decode(w, seed=64, positions=(0, 31, 127, 128, 900))
    check_decode(w, x, f"fused fp8 decode D={D}", oracle.FP8, 0.011, 0.0097)


def test_fused_decode_many_requests_no_split():
    # 40 requests x 8 KV heads = 320 units: one workgroup per unit
    w = synthetic.Workload("t", B=40, Hkv=8, G=8, D=256, W=1024, pos_lo=0, pos_hi=3000)
    assert swr.workspace_bytes(swr.SWR_OP_SWA_APPEND_DECODE, w.B, 1, w.Hq, w.Hkv, w.D, w.W) == 0
    check_decode(w, synthetic.sliding_decode(w, seed=65), "fused decode B=40")


@pytest.mark.parametrize("B", [12, 20, 28])
def test_fused_decode_split_counts(B):
    # two, three (the last one ragged) and no splits per (request, KV head):
    # the new token's tile falls in any split
    w = synthetic.Workload("t", B=B, Hkv=8, G=8, D=256, W=1024, pos_lo=0, pos_hi=4096)
    check_decode(w, synthetic.sliding_decode(w, seed=67 + B), f"fused decode B={B}")


def test_fused_decode_small_batch_split_k():
    w = synthetic.MIXED_SLIDING
    assert swr.workspace_bytes(swr.SWR_OP_SWA_APPEND_DECODE, w.B, 1, w.Hq, w.Hkv, w.D, w.W) > 0
    check_decode(w, synthetic.sliding_decode(w, seed=66, positions=synthetic.mixed_contexts()),
                 "fused B=16 split-K decode")


# ------------------------------------------------------------ global layers

def fused_global_case(x, S, cap, dtype=oracle.BF16, ks=1.0, vs=1.0, caps=None, seed=71):
    """x from synthetic.global_verify (or alike): keys 0 .. key_count-1, the
    last S of them the proposals.  The regions hold keys 0 .. pos0-1 and stale
    tokens in the proposals' slots; the call writes the proposals and attends.
    caps: optional per-request capacities (regions laid out back to back)."""
    kc = x["key_count"].astype(np.int32)
    B, _, hkv, D = x["k"].shape
    pos0 = (kc - S).astype(np.int32)
    scale = 1.0 / np.sqrt(D)
    g = synthetic.rng(seed)
    k_stale, v_stale = x["k"].copy(), x["v"].copy()
    for b in range(B):
        k_stale[b, pos0[b]:kc[b]] = synthetic.normal_bf16(g, (S, hkv, D))
        v_stale[b, pos0[b]:kc[b]] = synthetic.normal_bf16(g, (S, hkv, D))
    if caps is None:
        kp, vp, ko, vo = global_pools(k_stale, v_stale, kc, cap, dtype, ks, vs)
    else:
        rbs = [oracle.region_bytes(int(c), hkv, D, dtype) for c in caps]
        ko = np.concatenate([[0], np.cumsum(rbs)[:-1]]).astype(np.int64)
        vo = ko.copy()
        kp = np.zeros(int(sum(rbs)), np.uint8)
        vp = np.zeros(int(sum(rbs)), np.uint8)
        oracle.kv_append(kp, vp, ko, vo, cap, dtype, ks, vs, k_stale, v_stale, np.zeros(B, np.int32), kc,
                         wrap=False, caps=caps)
    kn = np.ascontiguousarray(np.stack([x["k"][b, pos0[b]:kc[b]] for b in range(B)]))
    vn = np.ascontiguousarray(np.stack([x["v"][b, pos0[b]:kc[b]] for b in range(B)]))
    L = layer(kp, vp, ko, vo, cap, dtype, ks, vs)
    if caps is not None:
        L.cap_b = dev_i32(caps)
    out = swr.global_append_attend(L, dev_bf16(kn), dev_bf16(vn), dev_bf16(x["q"]), dev_i32(pos0), int(kc.max()),
                                   scale)
    torch.cuda.synchronize()
    oracle.kv_append(kp, vp, ko, vo, cap, dtype, ks, vs, kn, vn, pos0, wrap=False, caps=caps)
    q_pos = (pos0[:, None] + np.arange(S, dtype=np.int32)[None, :]).astype(np.int32)
    ref = oracle.global_attend(kp, vp, ko, vo, cap, dtype, ks, vs, x["q"], q_pos, kc, hkv, scale, caps=caps)
    assert np.array_equal(L.k_base.cpu().numpy(), kp), "K region bytes"
    assert np.array_equal(L.v_base.cpu().numpy(), vp), "V region bytes"
    return out, ref


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_fused_global_verify_6005_keys(dtype):
    w = synthetic.GLOBAL_VERIFY
    ks, vs = (0.0099, 0.0108) if dtype == oracle.FP8 else (1.0, 1.0)
    out, ref = fused_global_case(synthetic.global_verify(w, seed=72), w.S, 6016, dtype, ks, vs)
    e = assert_parity(host_f64(out), ref, "fused global verify 6005")
    print("fused global verify max-abs %.3e rel-L2 %.3e" % e)


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
@pytest.mark.parametrize("S,G,D", [(4, 8, 512), (1, 8, 512), (2, 4, 64), (3, 4, 256), (1, 16, 128), (8, 4, 128)])
def test_fused_global_shapes(S, G, D, dtype):
    # key counts: no context (proposals only), proposals across a 128-key
    # chunk boundary and a 32-key tile boundary, chunk-aligned context, and
    # proposals from pos0 = 6, 317 (across an 8-slot value block inside a
    # chunk: the staged tokens fill two blocks) and 254 (across a chunk
    # boundary from an uneven slot).  Over fp8 the value codes load in pairs
    # of dims only at D=512, so the smaller head dims take the unpaired
    # substitution of the call's tokens.
    kc = np.array([S, 126 + S, 128 + S, 131, 700, 2000, 6 + S, 317 + S, 254 + S], np.int32)
    kc = np.maximum(kc, S)
    B = kc.size
    g = synthetic.rng(73)
    x = dict(key_count=kc, k=synthetic.normal_bf16(g, (B, 2048, 2, D)),
             v=synthetic.normal_bf16(g, (B, 2048, 2, D)), q=synthetic.normal_bf16(g, (B, S, 2 * G, D)))
    ks, vs = (4.2 / 448, 5.2 / 448) if dtype == oracle.FP8 else (1.0, 1.0)
    out, ref = fused_global_case(x, S, 2048, dtype, ks, vs)
    assert_parity(host_f64(out), ref, f"fused global S={S} G={G} D={D}")


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
@pytest.mark.parametrize("S,G,D", [(1, 16, 128), (8, 4, 128), (3, 4, 256), (2, 4, 64)])
def test_fused_global_many_chunks(S, G, D, dtype):
    # more than 16 chunks of 128 keys: the merge pass that groups chunks per
    # row, which also stores the call's tokens (over fp8, one value per
    # thread across the row workgroups)
    kc = np.array([S, 2100, 2300 + S], np.int32)
    B = kc.size
    g = synthetic.rng(76)
    x = dict(key_count=kc, k=synthetic.normal_bf16(g, (B, 2560, 2, D)),
             v=synthetic.normal_bf16(g, (B, 2560, 2, D)), q=synthetic.normal_bf16(g, (B, S, 2 * G, D)))
    ks, vs = (3.1 / 448, 3.6 / 448) if dtype == oracle.FP8 else (1.0, 1.0)
    out, ref = fused_global_case(x, S, 2560, dtype, ks, vs)
    assert_parity(host_f64(out), ref, f"fused global, many chunks, S={S} G={G} D={D}")


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_fused_global_per_request_capacities(dtype):
    S, G, D = 4, 8, 512
    kc = np.array([4, 67, 640, 1500], np.int32)
    caps = np.array([64, 128, 704, 1536], np.int32)
    g = synthetic.rng(74)
    B = kc.size
    x = dict(key_count=kc, k=synthetic.normal_bf16(g, (B, 1536, 2, D)),
             v=synthetic.normal_bf16(g, (B, 1536, 2, D)), q=synthetic.normal_bf16(g, (B, S, 2 * G, D)))
    ks, vs = (0.012, 0.0116) if dtype == oracle.FP8 else (1.0, 1.0)
    out, ref = fused_global_case(x, S, int(caps.max()), dtype, ks, vs, caps=caps)
    assert_parity(host_f64(out), ref, "fused global, per-request capacities")


@pytest.mark.parametrize("dtype,S", [(oracle.BF16, 4), (oracle.FP8, 4), (oracle.BF16, 1), (oracle.FP8, 1)],
                         ids=["bf16", "fp8", "S1", "fp8S1"])
def test_fused_global_streamed(dtype, S):
    # units x tiles >= 2048: the streamed pass with positions derived from
    # pos0; S > 1 runs the append kernel first, S = 1 takes the token in the
    # split that reads its tile
    kc = np.array([S, 63, 64, 65, 700, 2000, 4099, 5000], np.int32)
    assert kc.size * 2 * -(-int(kc.max()) // 32) >= 2048
    G, D = 8, 512
    g = synthetic.rng(75)
    B = kc.size
    x = dict(key_count=kc, k=synthetic.normal_bf16(g, (B, 5000, 2, D)),
             v=synthetic.normal_bf16(g, (B, 5000, 2, D)), q=synthetic.normal_bf16(g, (B, S, 2 * G, D)))
    ks, vs = (4.2 / 448, 5.2 / 448) if dtype == oracle.FP8 else (1.0, 1.0)
    out, ref = fused_global_case(x, S, 5056, dtype, ks, vs)
    assert_parity(host_f64(out), ref, "fused streamed global")


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
@pytest.mark.parametrize("G,D", [(8, 512), (16, 128), (4, 256), (8, 64), (32, 128)])
def test_fused_global_streamed_one_token(G, D, dtype):
    # one token per request in a streamed call: the split holding the token's
    # tile substitutes it and stores it.  Tokens at slot 0 (the only key), at
    # the last and first slots of a 32-key tile, at the last slot of a
    # request's capacity, and deep in long regions; the decode shapes (up to
    # 16 rows) and, at G = 32, the 32-row shapes
    kc = np.array([1, 32, 33, 64, 96, 191, 700, 2047, 4000, 4093, 4096], np.int32)
    caps = np.array([64, 64, 64, 64, 128, 192, 704, 2048, 4032, 4096, 4096], np.int32)  # each >= pad64(count)
    B = kc.size
    assert B * 2 * -(-int(kc.max()) // 32) >= 2048
    g = synthetic.rng(77)
    x = dict(key_count=kc, k=synthetic.normal_bf16(g, (B, 4096, 2, D)),
             v=synthetic.normal_bf16(g, (B, 4096, 2, D)), q=synthetic.normal_bf16(g, (B, 1, 2 * G, D)))
    ks, vs = (3.9 / 448, 4.7 / 448) if dtype == oracle.FP8 else (1.0, 1.0)
    out, ref = fused_global_case(x, 1, int(caps.max()), dtype, ks, vs, caps=caps)
    assert_parity(host_f64(out), ref, f"fused streamed global, one token, G={G} D={D}")
    if dtype == oracle.BF16:  # the request whose only key is its own token returns its value bits
        assert np.array_equal(host_bits(out)[0, 0], np.repeat(x["v"][0, 0], G, axis=0))


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_fused_global_streamed_stack_layer(dtype):
    # a global layer of the B=56 decode step at its full size (2 KV heads x
    # 512, 8 query heads each, contexts U[1024, 4096], one new token per
    # request, per-request capacities): the streamed pass that takes each
    # token in the split reading its tile, as the 60-layer stack runs it
    B, D, G = 56, 512, 8
    g = synthetic.rng(78)
    kc = (synthetic.uniform_int(g, 1024, 4096, B) + 1).astype(np.int32)
    caps = ((kc + 63) // 64 * 64).astype(np.int32)
    x = dict(key_count=kc, k=synthetic.normal_bf16(g, (B, int(kc.max()), 2, D)),
             v=synthetic.normal_bf16(g, (B, int(kc.max()), 2, D)), q=synthetic.normal_bf16(g, (B, 1, 2 * G, D)))
    ks, vs = (4.4 / 448, 4.6 / 448) if dtype == oracle.FP8 else (1.0, 1.0)
    out, ref = fused_global_case(x, 1, int(caps.max()), dtype, ks, vs, caps=caps)
    e = assert_parity(host_f64(out), ref, "fused streamed global, B=56 stack layer")
    print("fused streamed global B=56 max-abs %.3e rel-L2 %.3e" % e)
