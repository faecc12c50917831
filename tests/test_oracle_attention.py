"""Pins for the oracle's attention: decode over a ring, sliding verify,
global attention with a padded tail.

Each pin ties the oracle to something other than itself:
  * torch scaled_dot_product_attention on the CPU in float64 (a library
    routine) over the keys in plain position order, with the visibility rule
    written as a boolean mask over positions;
  * closed forms (one key -> its value exactly; all-zero keys -> mean of the
    visible values);
  * invariances the pages state: the output does not depend on the ring's
    rotation ("Improving Decode Throughput on Intel Gaudi 3", Our approach),
    and a zero, masked tail leaves it unchanged ("Announcing Carat", More
    FLOPs can be faster);
  * special cases that reduce to another operation (verify with S=1 is a
    decode; a ring larger than the context is a global layer).
The check_* functions are also run against planted-mistake builds of the
oracle (test_oracle_mistakes.py).
"""
import numpy as np

import oracle
import synthetic
from helpers import f64, global_pools, ring_pools, sdpa

TOL = 1e-11  # float64 oracle vs float64 library attention


# ------------------------------------------------------------------ decode

def check_tiny_sequence():
    """Workload 1: W=16 ring, 40 tokens appended one by one, decode after
    each; every step against SDPA over the window in position order."""
    w = synthetic.TINY
    q, k, v = synthetic.tiny_sequence()
    rb = oracle.region_bytes(w.W, w.Hkv, w.D, oracle.BF16)
    kp, vp = np.zeros(rb, np.uint8), np.zeros(rb, np.uint8)
    off = np.zeros(1, np.int64)
    scale = 1.0 / np.sqrt(w.D)
    for t in range(w.steps):
        oracle.kv_append(kp, vp, off, off, w.W, oracle.BF16, 1, 1, k[None, t:t + 1], v[None, t:t + 1],
                         np.array([t], np.int32))
        out = oracle.swa_decode(kp, vp, off, off, w.W, oracle.BF16, 1, 1, q[None, t],
                                np.array([t], np.int32), w.Hkv, scale)[0]
        lo = max(0, t - w.W + 1)
        for h in range(w.Hq):
            g = h // w.G
            ref = sdpa(f64(q[t, h])[None], f64(k[lo:t + 1, g]), f64(v[lo:t + 1, g]),
                       np.ones((1, t + 1 - lo), bool), scale)[0]
            assert np.max(np.abs(out[h] - ref)) < TOL, (t, h)
        if t == 0:  # a single visible key: the output is that key's value, exactly
            for h in range(w.Hq):
                assert np.array_equal(out[h], f64(v[0, h // w.G]))


def check_decode_batch(B=5, W=64, Hkv=2, G=4, D=32, positions=(0, 10, 63, 64, 200)):
    w = synthetic.Workload("t", B=B, Hkv=Hkv, G=G, D=D, W=W)
    x = synthetic.sliding_decode(w, seed=11, positions=positions)
    kp, vp, ko, vo = ring_pools(x["k"], x["v"], x["start"], x["n"], W)
    scale = 1.0 / np.sqrt(D)
    out = oracle.swa_decode(kp, vp, ko, vo, W, oracle.BF16, 1, 1, x["q"], x["pos"], Hkv, scale)
    for b in range(B):
        n = x["n"][b]
        for h in range(w.Hq):
            g = h // G
            ref = sdpa(f64(x["q"][b, h])[None], f64(x["k"][b, :n, g]), f64(x["v"][b, :n, g]),
                       np.ones((1, n), bool), scale)[0]
            assert np.max(np.abs(out[b, h] - ref)) < TOL, (b, h)
    return out


def check_rotation_invariance():
    """The same window stored at a different rotation gives the same output."""
    W, Hkv, G, D = 32, 1, 2, 32
    w = synthetic.Workload("t", B=1, Hkv=Hkv, G=G, D=D, W=W)
    x = synthetic.sliding_decode(w, seed=12, positions=[100])
    outs = []
    for shift in (0, 5, 17):
        kp, vp, ko, vo = ring_pools(x["k"], x["v"], x["start"] + shift, x["n"], W)
        outs.append(oracle.swa_decode(kp, vp, ko, vo, W, oracle.BF16, 1, 1, x["q"], x["pos"] + shift,
                                      Hkv, 0.25))
    # storage order changes the summation order only
    assert np.max(np.abs(outs[0] - outs[1])) < 1e-13
    assert np.max(np.abs(outs[0] - outs[2])) < 1e-13
    assert not np.array_equal(ring_pools(x["k"], x["v"], x["start"], x["n"], W)[0],
                              ring_pools(x["k"], x["v"], x["start"] + 5, x["n"], W)[0])


def check_zero_keys_give_mean_of_values():
    W, Hkv, G, D = 32, 2, 2, 32
    w = synthetic.Workload("t", B=2, Hkv=Hkv, G=G, D=D, W=W)
    x = synthetic.sliding_decode(w, seed=13, positions=[20, 77])
    k0 = np.zeros_like(x["k"])
    kp, vp, ko, vo = ring_pools(k0, x["v"], x["start"], x["n"], W)
    out = oracle.swa_decode(kp, vp, ko, vo, W, oracle.BF16, 1, 1, x["q"], x["pos"], Hkv, 0.3)
    for b in range(2):
        n = x["n"][b]
        for h in range(w.Hq):
            mean = f64(x["v"][b, :n, h // G]).mean(axis=0)
            assert np.max(np.abs(out[b, h] - mean)) < 1e-13


def check_identical_queries_identical_outputs():
    W, Hkv, G, D = 32, 2, 4, 32
    w = synthetic.Workload("t", B=1, Hkv=Hkv, G=G, D=D, W=W)
    x = synthetic.sliding_decode(w, seed=14, positions=[50])
    q = x["q"].copy()
    q[0, 5] = q[0, 6]  # two heads of KV head 1
    kp, vp, ko, vo = ring_pools(x["k"], x["v"], x["start"], x["n"], W)
    out = oracle.swa_decode(kp, vp, ko, vo, W, oracle.BF16, 1, 1, q, x["pos"], Hkv, 0.25)
    assert np.array_equal(out[0, 5], out[0, 6])
    assert not np.array_equal(out[0, 4], out[0, 5])


# ------------------------------------------------------------------ verify

def verify_reference(x, W, G, scale):
    """SDPA over [window history, proposals] in position order with the
    per-row window edge and causal rule written as a position mask."""
    B, S, Hq, D = x["q"].shape
    out = np.empty((B, S, Hq, D))
    for b in range(B):
        n, p0 = x["n"][b], x["p0"][b]
        kpos = np.concatenate([np.arange(p0 - n, p0), p0 + np.arange(S)])
        qpos = p0 + np.arange(S)
        mask = (kpos[None, :] >= qpos[:, None] - W + 1) & (kpos[None, :] <= qpos[:, None])
        for h in range(Hq):
            g = h // G
            kk = np.concatenate([f64(x["k"][b, :n, g]), f64(x["k_prop"][b, :, g])])
            vv = np.concatenate([f64(x["v"][b, :n, g]), f64(x["v_prop"][b, :, g])])
            out[b, :, h] = sdpa(f64(x["q"][b, :, h]), kk, vv, mask, scale)
    return out


def run_verify(x, W, Hkv, scale, k=None, v=None, k_prop=None, v_prop=None):
    kp, vp, ko, vo = ring_pools(x["k"] if k is None else k, x["v"] if v is None else v, x["start"],
                                x["n"], W)
    return oracle.gqa_verify(kp, vp, ko, vo, W, oracle.BF16, 1, 1,
                             x["k_prop"] if k_prop is None else k_prop,
                             x["v_prop"] if v_prop is None else v_prop, x["q"], x["p0"], Hkv, scale)


def check_verify_matches_sdpa():
    W, Hkv, G, D, S = 64, 2, 4, 32, 4
    w = synthetic.Workload("t", B=4, Hkv=Hkv, G=G, D=D, W=W, S=S)
    x = synthetic.sliding_verify(w, seed=21, positions=[1, 30, 64, 300])
    out = run_verify(x, W, Hkv, 0.2)
    ref = verify_reference(x, W, G, 0.2)
    assert np.max(np.abs(out - ref)) < TOL


def check_verify_masks():
    """Row i ignores proposals after i and the i+1 oldest ring keys, and does
    depend on the oldest key it should see."""
    W, Hkv, G, D, S = 32, 1, 2, 32, 4
    w = synthetic.Workload("t", B=1, Hkv=Hkv, G=G, D=D, W=W, S=S)
    x = synthetic.sliding_verify(w, seed=22, positions=[90])  # full ring, p0 >= W
    base = run_verify(x, W, Hkv, 0.25)
    g = synthetic.rng(23)
    for i in range(S):
        kp2 = x["k_prop"].copy()
        vp2 = x["v_prop"].copy()
        kp2[:, i + 1:] = synthetic.normal_bf16(g, kp2[:, i + 1:].shape)
        vp2[:, i + 1:] = synthetic.normal_bf16(g, vp2[:, i + 1:].shape)
        out = run_verify(x, W, Hkv, 0.25, k_prop=kp2, v_prop=vp2)
        assert np.array_equal(out[:, :i + 1], base[:, :i + 1]), i
        if i + 1 < S:
            assert not np.array_equal(out[:, i + 1:], base[:, i + 1:])
        # history index j holds position p0 - W + j; row i sees j >= i + 1
        k2, v2 = x["k"].copy(), x["v"].copy()
        k2[:, :i + 1] = synthetic.normal_bf16(g, k2[:, :i + 1].shape)
        v2[:, :i + 1] = synthetic.normal_bf16(g, v2[:, :i + 1].shape)
        out = run_verify(x, W, Hkv, 0.25, k=k2, v=v2)
        assert np.array_equal(out[:, i], base[:, i]), i
        k3, v3 = x["k"].copy(), x["v"].copy()
        k3[:, i + 1] = synthetic.normal_bf16(g, k3[:, i + 1].shape)
        v3[:, i + 1] = synthetic.normal_bf16(g, v3[:, i + 1].shape)
        out = run_verify(x, W, Hkv, 0.25, k=k3, v=v3)
        assert not np.array_equal(out[:, i], base[:, i]), i


def check_verify_single_proposal_is_decode():
    W, Hkv, G, D = 32, 2, 2, 32
    w = synthetic.Workload("t", B=3, Hkv=Hkv, G=G, D=D, W=W, S=1)
    x = synthetic.sliding_verify(w, seed=24, positions=[5, 32, 77])
    ver = run_verify(x, W, Hkv, 0.25)
    kp, vp, ko, vo = ring_pools(x["k"], x["v"], x["start"], x["n"], W)
    oracle.kv_append(kp, vp, ko, vo, W, oracle.BF16, 1, 1, x["k_prop"], x["v_prop"], x["p0"])
    dec = oracle.swa_decode(kp, vp, ko, vo, W, oracle.BF16, 1, 1, x["q"][:, 0], x["p0"], Hkv, 0.25)
    assert np.max(np.abs(ver[:, 0] - dec)) < 1e-13


# ------------------------------------------------------------------ global

def global_reference(x, G, scale):
    B, S, Hq, D = x["q"].shape
    out = np.empty((B, S, Hq, D))
    for b in range(B):
        kc = x["key_count"][b]
        mask = np.arange(kc)[None, :] <= x["q_pos"][b][:, None]
        for h in range(Hq):
            out[b, :, h] = sdpa(f64(x["q"][b, :, h]), f64(x["k"][b, :kc, h // G]),
                                f64(x["v"][b, :kc, h // G]), mask, scale)
    return out


def check_global_matches_sdpa(key_count=300, Hkv=2, G=8, D=64, S=4):
    w = synthetic.Workload("t", B=1, Hkv=Hkv, G=G, D=D, S=S, key_count=key_count)
    x = synthetic.global_verify(w, seed=31)
    cap = (key_count + 63) // 64 * 64
    kp, vp, ko, vo = global_pools(x["k"], x["v"], x["key_count"], cap)
    scale = 1.0 / np.sqrt(D)
    out = oracle.global_attend(kp, vp, ko, vo, cap, oracle.BF16, 1, 1, x["q"], x["q_pos"],
                               x["key_count"], Hkv, scale)
    ref = global_reference(x, G, scale)
    assert np.max(np.abs(out - ref)) < TOL
    return x, (kp, vp, ko, vo, cap), out


def check_padded_tail_leaves_output_unchanged():
    """6005 keys: contracting over 6016 (zero, masked tail) or over exactly
    6005 gives bit-identical output ("Announcing Carat", More FLOPs)."""
    w = synthetic.GLOBAL_VERIFY
    x = synthetic.global_verify(w, seed=32)
    cap = 6016
    kp, vp, ko, vo = global_pools(x["k"][:, :, :, :64], x["v"][:, :, :, :64], x["key_count"], cap)
    q = x["q"][:, :, :, :64].copy()
    padded = oracle.global_attend(kp, vp, ko, vo, cap, oracle.BF16, 1, 1, q, x["q_pos"],
                                  x["key_count"], w.Hkv, 0.125, padded=True)
    exact = oracle.global_attend(kp, vp, ko, vo, cap, oracle.BF16, 1, 1, q, x["q_pos"],
                                 x["key_count"], w.Hkv, 0.125, padded=False)
    assert np.array_equal(padded, exact)
    return x, (kp, vp, ko, vo, cap), q, padded


def check_global_equals_sliding_when_window_covers_context():
    kc, Hkv, G, D = 40, 2, 2, 32
    w = synthetic.Workload("t", B=1, Hkv=Hkv, G=G, D=D, S=1, key_count=kc)
    x = synthetic.global_verify(w, seed=33)
    kp, vp, ko, vo = global_pools(x["k"], x["v"], x["key_count"], 64)
    glob = oracle.global_attend(kp, vp, ko, vo, 64, oracle.BF16, 1, 1, x["q"], x["q_pos"],
                                x["key_count"], Hkv, 0.25)
    ring = oracle.swa_decode(kp, vp, ko, vo, 64, oracle.BF16, 1, 1, x["q"][:, 0], x["q_pos"][:, 0],
                             Hkv, 0.25)
    assert np.array_equal(glob[:, 0], ring)


def check_fp8_power_of_two_scales_equal_dequantised_bf16():
    W, Hkv, G, D = 32, 2, 2, 64
    w = synthetic.Workload("t", B=2, Hkv=Hkv, G=G, D=D, W=W)
    x = synthetic.sliding_decode(w, seed=41, positions=[20, 90])
    ks, vs = 2.0 ** -3, 2.0 ** -4
    kp8, vp8, ko, vo = ring_pools(x["k"], x["v"], x["start"], x["n"], W, oracle.FP8, ks, vs)
    out8 = oracle.swa_decode(kp8, vp8, ko, vo, W, oracle.FP8, ks, vs, x["q"], x["pos"], Hkv, 0.2)
    kdq = synthetic.bf16_bits((oracle.e4m3_value(oracle.e4m3_encode(x["k"], ks)) * ks).astype(np.float32))
    vdq = synthetic.bf16_bits((oracle.e4m3_value(oracle.e4m3_encode(x["v"], vs)) * vs).astype(np.float32))
    kpb, vpb, ko2, vo2 = ring_pools(kdq, vdq, x["start"], x["n"], W)
    outb = oracle.swa_decode(kpb, vpb, ko2, vo2, W, oracle.BF16, 1, 1, x["q"], x["pos"], Hkv, 0.2)
    assert np.array_equal(out8, outb)


ALL_CHECKS = [
    check_tiny_sequence, check_decode_batch, check_rotation_invariance,
    check_zero_keys_give_mean_of_values, check_identical_queries_identical_outputs,
    check_verify_matches_sdpa, check_verify_masks, check_verify_single_proposal_is_decode,
    check_global_matches_sdpa, check_padded_tail_leaves_output_unchanged,
    check_global_equals_sliding_when_window_covers_context,
    check_fp8_power_of_two_scales_equal_dequantised_bf16,
]


def test_tiny_sequence():
    check_tiny_sequence()


def test_decode_batch_with_partial_and_wrapped_rings():
    check_decode_batch()


def test_decode_gemma_sliding_shape():
    # the sliding-layer head shape (8 KV heads x 256, 8 q heads each), 3 requests
    check_decode_batch(B=3, W=1024, Hkv=8, G=8, D=256, positions=(1024, 2500, 4096))


def test_rotation_invariance():
    check_rotation_invariance()


def test_zero_keys_give_mean_of_values():
    check_zero_keys_give_mean_of_values()


def test_identical_queries_identical_outputs():
    check_identical_queries_identical_outputs()


def test_verify_matches_sdpa():
    check_verify_matches_sdpa()


def test_verify_masks():
    check_verify_masks()


def test_verify_single_proposal_is_decode():
    check_verify_single_proposal_is_decode()


def test_global_matches_sdpa():
    check_global_matches_sdpa()


def test_global_matches_sdpa_gemma_global_shape():
    check_global_matches_sdpa(key_count=1000, Hkv=2, G=8, D=512, S=4)


def test_padded_tail_leaves_output_unchanged():
    check_padded_tail_leaves_output_unchanged()


def test_nonfinite_tail_shows_why_the_tail_is_zeroed():
    # With NaN in the padded tail, the masked terms are 0 * NaN: the padded
    # contraction needs a zero-initialised tail, the exact one does not.
    x, (kp, vp, ko, vo, cap), q, _ = check_padded_tail_leaves_output_unchanged()
    vp = vp.copy()
    kc = int(x["key_count"][0])
    vv = vp.view(np.uint16).reshape(2, cap // 8, 64, 8)  # [Hkv][cap/8][D][8]
    for s in range(kc, cap):
        vv[:, s // 8, :, s % 8] = 0x7FC0
    padded = oracle.global_attend(kp, vp, ko, vo, cap, oracle.BF16, 1, 1, q, x["q_pos"],
                                  x["key_count"], 2, 0.125, padded=True)
    exact = oracle.global_attend(kp, vp, ko, vo, cap, oracle.BF16, 1, 1, q, x["q_pos"],
                                 x["key_count"], 2, 0.125, padded=False)
    assert np.all(np.isnan(padded)) and np.all(np.isfinite(exact))


def test_global_equals_sliding_when_window_covers_context():
    check_global_equals_sliding_when_window_covers_context()


def test_fp8_power_of_two_scales_equal_dequantised_bf16():
    check_fp8_power_of_two_scales_equal_dequantised_bf16()
