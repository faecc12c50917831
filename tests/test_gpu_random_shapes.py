"""Seeded random configurations of every attention entry point against the
oracle.

The other GPU tests pick their shapes by hand, one axis at a time; here each
case draws a whole configuration inside the documented envelope (include/
swr.h): head dim, KV heads, query heads per KV head, proposals, window or
capacity, positions or key counts (partial and wrapped rings, counts on and
off tile and chunk edges), element type and scales, and per-request global
capacities.  The append call draws its token counts too
(none, a few, more than a ring holds), positions past a global region's
capacity (dropped) and special values (saturation, subnormals, signed
zeros, infinities); the paged gather (the baseline the ring replaces)
draws its page size and window.  The draws fall on both sides of the
launch-form thresholds:
split-K or whole-unit decode, chunked or ring-kernel verify, chunked or
streamed global calls (with one token per request or several for the fused
call).  Outputs are held to the parity bar; the fused calls' region bytes
must equal the oracle's append bit for bit.
"""
import numpy as np
import pytest

import oracle
import synthetic
from gpu_common import host_f64
from helpers import assert_parity
from test_gpu_append import fitting, run_both
from test_gpu_attention import decode_case, global_case, verify_case
from test_gpu_fused import fused_decode_case, fused_global_case
from test_gpu_gather import run_gather

pytestmark = pytest.mark.gpu

N_CASES = 40
DIMS = (64, 128, 256, 512)


def draw_dtype(g):
    if g.random() < 0.5:
        return oracle.BF16, 1.0, 1.0
    return oracle.FP8, float(g.uniform(2.5, 6.5) / 448), float(g.uniform(2.5, 6.5) / 448)


def draw_positions(g, B, W, floor=0):
    """Per request: inside a partial ring, at its last slot or the wrap, or
    wrapped far past it."""
    out = []
    for _ in range(B):
        kind = g.integers(0, 4)
        if kind == 0:
            p = int(g.integers(floor, max(floor + 1, W)))
        elif kind == 1:
            p = int(g.choice([W - 2, W - 1, W, W + 1]))
        elif kind == 2:
            p = int(g.integers(W, 4 * W))
        else:
            p = int(32 * g.integers(1, 4 * W // 32 + 1) + g.choice([-1, 0, 1]))
        out.append(max(p, floor))
    return np.array(out, np.int32)


def sliding_workload(g, verify):
    D = int(g.choice(DIMS))
    if verify:
        S = int(g.integers(1, 9))
        G = int(g.choice([gg for gg in (1, 2, 4, 8, 16) if gg * S <= 32]))
    else:
        S, G = 1, int(g.choice((1, 2, 4, 8, 16)))
    big = g.random() < 0.2  # enough (request, KV head) units to fill the chip
    if big:
        # (a verify with bf16 K/V leaves the chunked form at 512 units)
        Hkv, B, D = 8, int(g.integers(64 if verify else 32, 81)), int(g.choice((64, 128)))
        W = int(8 * g.integers(2, 17))
    else:
        Hkv = int(g.choice((1, 2, 4, 8)))
        B = int(g.integers(1, 9))
        W = int(8 * g.integers(2, (1024 if D <= 256 else 512) // 8 + 1))
    return synthetic.Workload("random", B=B, Hkv=Hkv, G=G, D=D, W=W, S=S)


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_decode(case):
    g = synthetic.rng(5000 + case)
    w = sliding_workload(g, verify=False)
    dtype, ks, vs = draw_dtype(g)
    x = synthetic.sliding_decode(w, seed=5100 + case, positions=draw_positions(g, w.B, w.W))
    out, ref = decode_case(w, x, dtype, ks, vs)
    assert_parity(host_f64(out), ref, f"random decode {w} dtype={dtype}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_fused_decode(case):
    g = synthetic.rng(5200 + case)
    w = sliding_workload(g, verify=False)
    dtype, ks, vs = draw_dtype(g)
    x = synthetic.sliding_decode(w, seed=5300 + case, positions=draw_positions(g, w.B, w.W))
    out, ref, gk, gv, kp, vp = fused_decode_case(w, x, dtype, ks, vs)
    assert np.array_equal(gk, kp), f"random fused decode {w}: K ring bytes"
    assert np.array_equal(gv, vp), f"random fused decode {w}: V ring bytes"
    assert_parity(host_f64(out), ref, f"random fused decode {w} dtype={dtype}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_verify(case):
    g = synthetic.rng(5400 + case)
    w = sliding_workload(g, verify=True)
    dtype, ks, vs = draw_dtype(g)
    x = synthetic.sliding_verify(w, seed=5500 + case, positions=draw_positions(g, w.B, w.W))
    out, ref = verify_case(w, x, dtype, ks, vs)
    assert_parity(host_f64(out), ref, f"random verify {w} dtype={dtype}")


def global_draw(g):
    D = int(g.choice(DIMS))
    S = int(g.integers(1, 9)) if g.random() < 0.6 else 1
    G = int(g.choice([gg for gg in (1, 2, 4, 8, 16) if gg * S <= 32]))
    Hkv = int(g.choice((1, 2, 4)))
    B = int(g.integers(1, 7))
    long_call = g.random() < 0.4  # the streamed form (>= 2048 tiles over all units)
    hi = 6000 if long_call else 1500
    kc = np.array([int(g.choice([g.integers(S, hi), 64 * g.integers(1, hi // 64) + g.integers(-1, 2)]))
                   for _ in range(B)], np.int32)
    kc = np.maximum(kc, S)
    if long_call:  # make sure the units span the streamed form's 2048 tiles
        need = -(-2048 // (B * Hkv)) * 32
        kc[int(g.integers(0, B))] = max(int(kc.max()), need)
    per_request = g.random() < 0.4
    caps = ((kc + 63) // 64 * 64 + 64 * g.integers(0, 3, size=B)).astype(np.int32) if per_request else None
    cap = int(caps.max()) if per_request else int(-(-int(kc.max()) // 64) * 64)
    return D, S, G, Hkv, B, kc, caps, cap


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_global(case):
    g = synthetic.rng(5600 + case)
    D, S, G, Hkv, B, kc, caps, cap = global_draw(g)
    dtype, ks, vs = draw_dtype(g)
    w = synthetic.Workload("random", B=B, Hkv=Hkv, G=G, D=D, S=S)
    x = synthetic.global_verify(w, seed=5700 + case, key_count=kc)
    # query positions anywhere in the context, ascending (causal rows that
    # see from one key up to all of them)
    qp = np.sort(np.stack([synthetic.uniform_int(g, 0, int(k) - 1, S) for k in kc]), axis=1).astype(np.int32)
    x["q_pos"] = qp
    out, ref = global_case(w, x, cap, dtype, ks, vs)
    assert_parity(host_f64(out), ref, f"random global B={B} Hkv={Hkv} G={G} D={D} S={S} dtype={dtype}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_fused_global(case):
    g = synthetic.rng(5800 + case)
    D, S, G, Hkv, B, kc, caps, cap = global_draw(g)
    dtype, ks, vs = draw_dtype(g)
    kmax = int(kc.max())
    x = dict(key_count=kc, k=synthetic.normal_bf16(g, (B, kmax, Hkv, D)),
             v=synthetic.normal_bf16(g, (B, kmax, Hkv, D)), q=synthetic.normal_bf16(g, (B, S, Hkv * G, D)))
    out, ref = fused_global_case(x, S, cap, dtype, ks, vs, caps=caps, seed=5900 + case)
    assert_parity(host_f64(out), ref, f"random fused global B={B} Hkv={Hkv} G={G} D={D} S={S} dtype={dtype}")


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_append(case):
    g = synthetic.rng(6000 + case)
    D = int(g.choice(DIMS))
    hkv = int(g.choice((1, 2, 4, 8)))
    B = int(g.integers(1, 9))
    T = int(g.integers(1, 33))
    wrap = bool(g.random() < 0.6)
    dtype, ks, vs = draw_dtype(g)
    cap = int(8 * g.integers(2, (512 if D == 512 else 2048) // 8 + 1))
    pos0 = (g.integers(0, 4 * cap, B) if wrap else g.integers(0, cap + 8, B)).astype(np.int32)
    n_new = None if g.random() < 0.4 else g.integers(0, T + 1, B).astype(np.int32)
    run_both(B, T, hkv, D, cap, dtype, ks, vs, pos0, n_new, wrap, seed=6100 + case, special=bool(g.random() < 0.3),
             oracle_tokens=None if wrap else fitting(pos0, n_new, T, cap))


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_paged_gather(case):
    g = synthetic.rng(6200 + case)
    D = int(g.choice(DIMS))
    hkv = int(g.choice((1, 2, 4, 8)))
    W = int(8 * g.integers(2, (512 if D == 512 else 1024) // 8 + 1))
    pt = int(g.choice((1, 3, 8, 16, 32, 64)))
    B = int(g.integers(1, 9))
    run_gather(W, D, hkv, pt, draw_positions(g, B, W), seed=6300 + case)
