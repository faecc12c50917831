"""GPU parity of the attention calls against the oracle.

Every case feeds the same seeded inputs (rings and regions built by the
oracle's append, copied to the device) to swr_swa_decode / swr_gqa_verify /
swr_global_attend and to the float64 oracle, and holds the bf16 outputs to
max-abs <= 1e-2 and relative L2 <= 5e-3.  Cases span several 32-key tiles
and ragged tails, the full workload sizes (B=56 sliding decode, B=8 sliding
verify, the 6005-key global verify), the split-K path, every head dim, and
the degenerate cases (a single visible key, a ring that has not wrapped,
proposals at position 0).
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


# ------------------------------------------------------------------ decode

def decode_case(w, x, dtype=oracle.BF16, ks=1.0, vs=1.0):
    scale = 1.0 / np.sqrt(w.D)
    kp, vp, ko, vo = ring_pools(x["k"], x["v"], x["start"], x["n"], w.W, dtype, ks, vs)
    ref = oracle.swa_decode(kp, vp, ko, vo, w.W, dtype, ks, vs, x["q"], x["pos"], w.Hkv, scale)
    L = layer(kp, vp, ko, vo, w.W, dtype, ks, vs)
    out = swr.swa_decode(L, dev_bf16(x["q"]), dev_i32(x["pos"]), w.Hkv, scale)
    torch.cuda.synchronize()
    return out, ref


def test_decode_tiny_sequence_step_by_step():
    """Workload 1: W=16, 2 query heads on 1 KV head, D=64; 40 tokens appended
    one at a time on the GPU, decode after each; ring bytes bit-exact with the
    oracle's after every append, outputs within tolerance, and step 0 (one
    visible key) returns that key's value bits exactly."""
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
        swr.ring_kv_append(L, dev_bf16(k[None, t:t + 1]), dev_bf16(v[None, t:t + 1]), dev_i32(pos))
        out = swr.swa_decode(L, dev_bf16(q[None, t]), dev_i32(pos), w.Hkv, scale)
        torch.cuda.synchronize()
        oracle.kv_append(kp, vp, off, off, w.W, oracle.BF16, 1, 1, k[None, t:t + 1], v[None, t:t + 1], pos)
        assert np.array_equal(L.k_base.cpu().numpy(), kp), t
        assert np.array_equal(L.v_base.cpu().numpy(), vp), t
        ref = oracle.swa_decode(kp, vp, off, off, w.W, oracle.BF16, 1, 1, q[None, t], pos, w.Hkv, scale)
        assert_parity(host_f64(out), ref, f"step {t}")
        if t == 0:
            assert np.array_equal(host_bits(out)[0], np.repeat(v[0], w.G, axis=0))


def test_decode_b56_full_workload():
    w = synthetic.SWA_DECODE
    out, ref = decode_case(w, synthetic.sliding_decode(w))
    e = assert_parity(host_f64(out), ref, "B=56 decode")
    print("B=56 decode max-abs %.3e rel-L2 %.3e" % e)


@pytest.mark.parametrize("positions", [
    (0, 1, 2, 15, 16, 31, 32, 33),          # partial rings, ragged last tiles
    (1022, 1023, 1024, 1025, 2047, 5000, 100000, 63),
])
def test_decode_edges(positions):
    w = synthetic.Workload("t", B=len(positions), Hkv=8, G=8, D=256, W=1024)
    out, ref = decode_case(w, synthetic.sliding_decode(w, seed=21, positions=positions))
    assert_parity(host_f64(out), ref, f"decode {positions}")
    if positions[0] == 0:  # a single visible key: output = that value, exactly
        x = synthetic.sliding_decode(w, seed=21, positions=positions)
        assert np.array_equal(host_bits(out)[0], np.repeat(x["v"][0, 0], w.G, axis=0))


@pytest.mark.parametrize("D,G,Hkv,W", [(64, 1, 4, 64), (128, 4, 2, 256), (512, 2, 2, 128), (256, 16, 1, 96),
                                       (64, 2, 1, 16)])
def test_decode_shapes(D, G, Hkv, W):
    w = synthetic.Workload("t", B=5, Hkv=Hkv, G=G, D=D, W=W)
    out, ref = decode_case(w, synthetic.sliding_decode(w, seed=22, positions=(0, W // 2 + 3, W - 1, W, 3 * W + 5)))
    assert_parity(host_f64(out), ref, f"decode D={D} G={G}")


def test_decode_small_batch_uses_split_k():
    # 16 requests x 8 KV heads: fewer units than CUs, so the keys are split
    # across workgroups and merged by the combine step
    w = synthetic.MIXED_SLIDING
    ctx = synthetic.mixed_contexts()
    assert swr.workspace_bytes(swr.SWR_OP_SWA_DECODE, w.B, 1, w.Hq, w.Hkv, w.D, w.W) > 0
    out, ref = decode_case(w, synthetic.sliding_decode(w, seed=23, positions=ctx))
    assert_parity(host_f64(out), ref, "B=16 split-K decode")


@pytest.mark.parametrize("B", [12, 20, 28])
def test_decode_split_counts(B):
    # the split count minimises the busiest CU's tiles: B=12 two splits of
    # 16 tiles, B=20 three splits (11, 11 and a ragged 10), B=28 none (224
    # units in one round); positions include partial windows
    w = synthetic.Workload("t", B=B, Hkv=8, G=8, D=256, W=1024)
    g = synthetic.rng(24)
    positions = synthetic.uniform_int(g, 0, 4096, B)
    positions[:3] = (0, 300, 1023)
    out, ref = decode_case(w, synthetic.sliding_decode(w, seed=24 + B, positions=positions))
    assert_parity(host_f64(out), ref, f"B={B} decode")


@pytest.mark.parametrize("ks,vs", [(2.0 ** -6, 2.0 ** -6), (0.00917, 0.01033)])
def test_decode_fp8_ring(ks, vs):
    w = synthetic.Workload("t", B=12, Hkv=8, G=8, D=256, W=1024)
    x = synthetic.sliding_decode(w, seed=24, positions=(0, 5, 100, 1023, 1024, 1500, 2000, 3000, 4000, 5000,
                                                       6000, 7000))
    out, ref = decode_case(w, x, oracle.FP8, ks, vs)
    assert_parity(host_f64(out), ref, "fp8 decode")


@pytest.mark.parametrize("D,G", [(64, 2), (128, 16), (512, 8)])
def test_decode_fp8_head_dims(D, G):
    w = synthetic.Workload("t", B=5, Hkv=2, G=G, D=D, W=128)
    x = synthetic.sliding_decode(w, seed=25, positions=(0, 31, 127, 128, 900))
    out, ref = decode_case(w, x, oracle.FP8, 0.011, 0.0097)
    assert_parity(host_f64(out), ref, f"fp8 decode D={D}")


# ------------------------------------------------------------------ verify

def verify_case(w, x, dtype=oracle.BF16, ks=1.0, vs=1.0):
    scale = 1.0 / np.sqrt(w.D)
    kp, vp, ko, vo = ring_pools(x["k"], x["v"], x["start"], x["n"], w.W, dtype, ks, vs)
    ref = oracle.gqa_verify(kp, vp, ko, vo, w.W, dtype, ks, vs, x["k_prop"], x["v_prop"], x["q"], x["p0"],
                            w.Hkv, scale)
    L = layer(kp, vp, ko, vo, w.W, dtype, ks, vs)
    out = swr.gqa_verify(L, dev_bf16(x["k_prop"]), dev_bf16(x["v_prop"]), dev_bf16(x["q"]), dev_i32(x["p0"]),
                         scale)
    torch.cuda.synchronize()
    return out, ref


def assert_lone_proposal_exact(out, x, w):
    """Request 0 starts at position 0: its ring holds nothing yet, so the
    rows of its first proposal see that proposal alone and return its value
    bits exactly (over an fp8 ring too: the proposals are bf16)."""
    assert int(x["p0"][0]) == 0
    assert np.array_equal(host_bits(out)[0, 0], np.repeat(x["v_prop"][0, 0], w.G, axis=0))


def test_verify_b8_full_workload():
    w = synthetic.SWA_VERIFY
    out, ref = verify_case(w, synthetic.sliding_verify(w))
    e = assert_parity(host_f64(out), ref, "B=8 verify")
    print("B=8 verify max-abs %.3e rel-L2 %.3e" % e)


@pytest.mark.parametrize("S,G", [(1, 8), (2, 8), (3, 8), (4, 8), (8, 4), (4, 2), (5, 1)])
def test_verify_proposal_counts(S, G):
    w = synthetic.Workload("t", B=8, Hkv=2, G=G, D=256, W=128, S=S)
    x = synthetic.sliding_verify(w, seed=31, positions=(0, 1, 5, 126, 127, 128, 129, 1000))
    out, ref = verify_case(w, x)
    assert_parity(host_f64(out), ref, f"verify S={S} G={G}")
    assert_lone_proposal_exact(out, x, w)


@pytest.mark.parametrize("D", [256, 512])
@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_verify_ring_chunk_halves(dtype, D):
    # A ring chunk of the chunked form covers 256 slots as two 128-key
    # halves: committed counts that end inside the first half, exactly at
    # and just past the half boundary, inside the second half, at a chunk
    # boundary and past the window (wrapped rings)
    positions = (0, 1, 127, 128, 129, 200, 255, 256, 257, 300, 511, 512, 700, 1023, 1024, 1500)
    w = synthetic.Workload("t", B=len(positions), Hkv=2, G=8, D=D, W=1024, S=4)
    x = synthetic.sliding_verify(w, seed=42, positions=positions)
    ks, vs = (4.2 / 448, 4.4 / 448) if dtype == oracle.FP8 else (1.0, 1.0)
    out, ref = verify_case(w, x, dtype, ks, vs)
    assert_parity(host_f64(out), ref, "verify ring chunk halves")
    assert_lone_proposal_exact(out, x, w)


@pytest.mark.parametrize("D", [64, 128, 512])
def test_verify_head_dims(D):
    w = synthetic.Workload("t", B=3, Hkv=2, G=8, D=D, W=64, S=4)
    out, ref = verify_case(w, synthetic.sliding_verify(w, seed=32, positions=(3, 64, 300)))
    assert_parity(host_f64(out), ref, f"verify D={D}")


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
@pytest.mark.parametrize("B", [32, 64])
def test_verify_large_batch(dtype, B):
    """Batches that fill the chip: 256 units run in chunked form, 512 units
    with bf16 K/V in the ring kernel without splitting (over fp8 every batch
    runs chunked)."""
    w = synthetic.Workload("t", B=B, Hkv=8, G=8, D=64, W=96, S=4)
    x = synthetic.sliding_verify(w, seed=40, positions=synthetic.uniform_int(synthetic.rng(41), 0, 400, B))
    out, ref = verify_case(w, x, dtype, *((0.0105, 0.0094) if dtype else (1.0, 1.0)))
    assert_parity(host_f64(out), ref, "large-batch verify")


@pytest.mark.parametrize("D,S,G", [(64, 4, 8), (256, 4, 8), (512, 4, 8), (256, 2, 4)])
def test_verify_fp8_ring(D, S, G):
    """fp8 ring history with bf16 proposals (the proposals are not yet in the
    ring, so they keep the precision they arrive in)."""
    w = synthetic.Workload("t", B=4, Hkv=2, G=G, D=D, W=256, S=S)
    x = synthetic.sliding_verify(w, seed=38, positions=(0, 5, 256, 1000))
    out, ref = verify_case(w, x, oracle.FP8, 0.0102, 0.0089)
    assert_parity(host_f64(out), ref, f"fp8 verify D={D} S={S} G={G}")
    assert_lone_proposal_exact(out, x, w)


# ------------------------------------------------------------------ global

def global_case(w, x, cap, dtype=oracle.BF16, ks=1.0, vs=1.0):
    scale = 1.0 / np.sqrt(w.D)
    kp, vp, ko, vo = global_pools(x["k"], x["v"], x["key_count"], cap, dtype, ks, vs)
    ref = oracle.global_attend(kp, vp, ko, vo, cap, dtype, ks, vs, x["q"], x["q_pos"], x["key_count"],
                               w.Hkv, scale)
    L = layer(kp, vp, ko, vo, cap, dtype, ks, vs)
    out = swr.global_attend(L, dev_bf16(x["q"]), dev_i32(x["q_pos"]), dev_i32(x["key_count"]),
                            int(x["key_count"].max()), w.Hkv, scale)
    torch.cuda.synchronize()
    return out, ref


def test_global_verify_6005_keys():
    w = synthetic.GLOBAL_VERIFY
    out, ref = global_case(w, synthetic.global_verify(w), 6016)
    e = assert_parity(host_f64(out), ref, "global verify 6005")
    print("global verify max-abs %.3e rel-L2 %.3e" % e)


def test_global_verify_6005_keys_fp8():
    w = synthetic.GLOBAL_VERIFY
    out, ref = global_case(w, synthetic.global_verify(w, seed=39), 6016, oracle.FP8, 0.0099, 0.0108)
    assert_parity(host_f64(out), ref, "global verify 6005 fp8")


def test_global_sweep_subset():
    """Key counts from the 4000..8192 sweep: 6000..6080, multiples of 64 +-1,
    the endpoints and random counts; batched as separate requests that share
    one key history."""
    g = synthetic.rng(33)
    counts = sorted(set(list(range(6000, 6081, 4)) + [4000, 8192, 4095, 4096, 4097, 6015, 6016, 6017, 8127,
                                                      8128, 8129, 5000, 7777] +
                        list(g.integers(4000, 8193, 8))))
    w = synthetic.GLOBAL_VERIFY
    hist = synthetic.global_verify(synthetic.Workload("t", B=1, Hkv=2, G=8, D=512, S=4, key_count=8192), seed=34)
    for chunk in (counts[:len(counts) // 2], counts[len(counts) // 2:]):
        B = len(chunk)
        kc = np.array(chunk, np.int32)
        x = dict(key_count=kc, q_pos=(kc[:, None] - 4 + np.arange(4, dtype=np.int32)[None, :]).astype(np.int32),
                 k=np.repeat(hist["k"], B, axis=0), v=np.repeat(hist["v"], B, axis=0),
                 q=synthetic.normal_bf16(g, (B, 4, 16, 512)))
        ww = synthetic.Workload("t", B=B, Hkv=2, G=8, D=512, S=4)
        out, ref = global_case(ww, x, 8192)
        for b in range(B):
            assert_parity(host_f64(out)[b], ref[b], f"key_count {chunk[b]}")
    assert w.key_count == 6005


def sweep_counts():
    """The checked counts of the 4000..8192 key-count sweep: every count in
    6000..6080, each multiple of 64 in range with its neighbours, the
    endpoints, and 64 seeded random counts."""
    mult = [m + d for m in range(4032, 8193, 64) for d in (-1, 0, 1)]
    rnd = synthetic.rng(35).integers(4000, 8193, 64)
    return sorted({c for c in list(range(6000, 6081)) + mult + [4000, 8192] + [int(r) for r in rnd]
                   if 4000 <= c <= 8192})


SWEEP_GROUPS = 6


@pytest.mark.parametrize("group", range(SWEEP_GROUPS))
def test_global_sweep_each_count_as_launched(group):
    """Each checked count of the sweep as its own B=1 call, launched as the
    benchmark times it (max_key_count = the count), over one region of 8192
    keys whose keys past the count are other (finite, masked) tokens."""
    counts = sweep_counts()[group::SWEEP_GROUPS]
    hist = synthetic.global_verify(synthetic.Workload("t", B=1, Hkv=2, G=8, D=512, S=4, key_count=8192), seed=36)
    kp, vp, ko, vo = global_pools(hist["k"], hist["v"], np.array([8192], np.int32), 8192)
    L = layer(kp, vp, ko, vo, 8192)
    q = synthetic.normal_bf16(synthetic.rng(37 + group), (1, 4, 16, 512))
    qd = dev_bf16(q)
    scale = 512 ** -0.5
    ws = torch.zeros(swr.workspace_bytes(swr.SWR_OP_GLOBAL_ATTEND, 1, 4, 16, 2, 512, 8192), dtype=torch.uint8,
                     device="cuda")
    outs = []
    for kc in counts:
        qp = np.arange(kc - 4, kc, dtype=np.int32)[None, :]
        outs.append(swr.global_attend(L, qd, dev_i32(qp), dev_i32([kc]), kc, 2, scale, ws=ws).clone())
    torch.cuda.synchronize()
    for kc, out in zip(counts, outs):
        qp = np.arange(kc - 4, kc, dtype=np.int32)[None, :]
        ref = oracle.global_attend(kp, vp, ko, vo, 8192, oracle.BF16, 1.0, 1.0, q, qp, np.array([kc], np.int32), 2,
                                   scale)
        assert_parity(host_f64(out), ref, f"key_count {kc}")


def test_sweep_counts_cover_the_stated_set():
    c = sweep_counts()
    assert set(range(6000, 6081)) <= set(c)
    assert {4000, 8192, 4095, 4096, 4097, 8191} <= set(c)
    assert len(c) >= 81 + 3 * 65


@pytest.mark.parametrize("S,G,D", [(1, 8, 512), (2, 8, 512), (4, 2, 64), (3, 4, 256), (1, 16, 128)])
def test_global_shapes(S, G, D):
    kc = np.array([1, 63, 64, 65, 700, 2000], np.int32)
    w = synthetic.Workload("t", B=kc.size, Hkv=2, G=G, D=D, S=S)
    g = synthetic.rng(35)
    x = dict(key_count=kc,
             q_pos=np.maximum(kc[:, None] - S + np.arange(S, dtype=np.int32)[None, :], 0).astype(np.int32),
             k=synthetic.normal_bf16(g, (kc.size, 2048, 2, D)), v=synthetic.normal_bf16(g, (kc.size, 2048, 2, D)),
             q=synthetic.normal_bf16(g, (kc.size, S, w.Hq, D)))
    out, ref = global_case(w, x, 2048)
    assert_parity(host_f64(out), ref, f"global S={S} G={G} D={D}")


# A global call whose units span at least 2048 tiles of 32 keys in all
# (B * Hkv * ceil(max_key_count / 32)) runs as one streaming split-K pass
# instead of the three-pass form; these cases sit above that bound, with
# ragged key counts and query positions that stop short of the last key.
STREAM_COUNTS = np.array([1, 63, 64, 65, 700, 2000, 4099, 5000], np.int32)


def streamed_inputs(S, G, D, seed):
    kc = STREAM_COUNTS
    g = synthetic.rng(seed)
    base = kc[:, None] - S + np.arange(S, dtype=np.int32)[None, :]
    early = base // 2 + np.arange(kc.size, dtype=np.int32)[:, None] % 3  # causal cut well inside the keys
    q_pos = np.where((np.arange(kc.size) % 2 == 1)[:, None], early, base)
    q_pos = np.clip(q_pos, 0, kc[:, None] - 1).astype(np.int32)
    kmax = int(kc.max())
    return dict(key_count=kc, q_pos=q_pos, k=synthetic.normal_bf16(g, (kc.size, kmax, 2, D)),
                v=synthetic.normal_bf16(g, (kc.size, kmax, 2, D)), q=synthetic.normal_bf16(g, (kc.size, S, 2 * G, D)))


@pytest.mark.parametrize("S,G,D", [(4, 8, 512), (1, 8, 512), (1, 8, 256), (4, 2, 64), (3, 4, 128)])
def test_global_streamed_shapes(S, G, D):
    x = streamed_inputs(S, G, D, seed=36)
    assert x["key_count"].size * 2 * -(-int(x["key_count"].max()) // 32) >= 2048
    w = synthetic.Workload("t", B=x["key_count"].size, Hkv=2, G=G, D=D, S=S)
    out, ref = global_case(w, x, 5056)
    assert_parity(host_f64(out), ref, f"streamed global S={S} G={G} D={D}")


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_global_streamed_many_requests(dtype):
    # 70 requests (the split numbering reads the key counts 64 at a time, one
    # per lane), some with a single key or a single tile, each region with a
    # capacity of its own; streamed: units x tiles >= 2048
    S, G, D, hkv = 1, 8, 128, 2
    g = synthetic.rng(38)
    B = 70
    kc = synthetic.uniform_int(g, 1, 2000, B)
    kc[:5] = (1, 1, 31, 2000, 33)
    caps = np.maximum((kc + 63) // 64 * 64, 64).astype(np.int32)
    assert B * hkv * -(-int(kc.max()) // 32) >= 2048
    cap = int(caps.max())
    k = synthetic.normal_bf16(g, (B, cap, hkv, D))
    v = synthetic.normal_bf16(g, (B, cap, hkv, D))
    q = synthetic.normal_bf16(g, (B, S, hkv * G, D))
    q_pos = np.maximum(kc - 1, 0).astype(np.int32).reshape(B, S)
    ks, vs = (4.4 / 448, 4.1 / 448) if dtype == oracle.FP8 else (1.0, 1.0)
    rbs = [oracle.region_bytes(int(c), hkv, D, dtype) for c in caps]
    ko = np.concatenate([[0], np.cumsum(rbs)[:-1]]).astype(np.int64)
    vo = ko.copy()
    kp = np.zeros(int(sum(rbs)), np.uint8)
    vp = np.zeros(int(sum(rbs)), np.uint8)
    oracle.kv_append(kp, vp, ko, vo, cap, dtype, ks, vs, k, v, np.zeros(B, np.int32), kc, wrap=False, caps=caps)
    scale = 1.0 / np.sqrt(D)
    ref = oracle.global_attend(kp, vp, ko, vo, cap, dtype, ks, vs, q, q_pos, kc, hkv, scale, caps=caps)
    L = layer(kp, vp, ko, vo, cap, dtype, ks, vs)
    L.cap_b = dev_i32(caps)
    out = swr.global_attend(L, dev_bf16(q), dev_i32(q_pos), dev_i32(kc), int(kc.max()), hkv, scale)
    torch.cuda.synchronize()
    assert_parity(host_f64(out), ref, "streamed global, 70 requests")


def test_global_streamed_fp8():
    S, G, D = 4, 8, 512
    x = streamed_inputs(S, G, D, seed=37)
    w = synthetic.Workload("t", B=x["key_count"].size, Hkv=2, G=G, D=D, S=S)
    out, ref = global_case(w, x, 5056, oracle.FP8, 4.2 / 448, 3.9 / 448)
    assert_parity(host_f64(out), ref, "streamed global fp8")
