"""The attention calls captured in a HIP graph and replayed.

A serving loop issues these short launches from a graph.  Each case runs the
call eagerly on one copy of the inputs, checks that eager result against the
oracle (output at the parity bar, region bytes bit for bit), captures the
call on a second copy, and replays the graph three times with other work and
synchronisations in between; every replay must give the eager output bit for
bit and leave the same region bytes (the library launches kernels only -- no
memset or copy nodes -- and its workspace is the caller's, reused by every
replay).  A multi-layer step in one graph is checked against the oracle in
test_gpu_stack.py.
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


def replay_and_check(run, outs_and_regions, other):
    """run() issues the call(s); outs_and_regions() returns the tensors to
    compare.  Eager results come from a first run on the same inputs."""
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    for rep in range(3):
        other()  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        yield rep, [t.clone() for t in outs_and_regions()]


def copies(kp, vp, ko, vo, cap, dtype=oracle.BF16, ks=1.0, vs=1.0):
    return layer(kp.copy(), vp.copy(), ko, vo, cap, dtype, ks, vs), layer(kp.copy(), vp.copy(), ko, vo, cap, dtype,
                                                                          ks, vs)


def busy_work():
    a = torch.randn(1 << 20, device="cuda")
    return lambda: a.mul_(1.0001).add_(0.5)


def test_fused_decode_in_graph_split_k():
    # 16 requests x 8 KV heads: split-K with its combine, and a workspace
    w = synthetic.Workload("t", B=16, Hkv=8, G=8, D=256, W=1024)
    x = synthetic.sliding_decode(w, seed=81, positions=synthetic.mixed_contexts())
    kp, vp, ko, vo = ring_pools(x["k"], x["v"], x["start"], x["n"] - 1, w.W)
    kn = dev_bf16(np.ascontiguousarray(x["k"][np.arange(w.B), x["n"] - 1]))
    vn = dev_bf16(np.ascontiguousarray(x["v"][np.arange(w.B), x["n"] - 1]))
    q, pos = dev_bf16(x["q"]), dev_i32(x["pos"])
    ws = torch.zeros(swr.workspace_bytes(swr.SWR_OP_SWA_APPEND_DECODE, w.B, 1, w.Hq, w.Hkv, w.D, w.W),
                     dtype=torch.uint8, device="cuda")
    assert ws.numel() > 0
    Le, Lg = copies(kp, vp, ko, vo, w.W)
    out_e = swr.swa_append_decode(Le, kn, vn, q, pos, 0.0625, ws=ws)
    torch.cuda.synchronize()
    want = (host_bits(out_e), Le.k_base.cpu().numpy(), Le.v_base.cpu().numpy())
    rk, rv = kp.copy(), vp.copy()
    oracle.kv_append(rk, rv, ko, vo, w.W, oracle.BF16, 1.0, 1.0, kn.view(torch.int16).cpu().numpy().view(np.uint16)[:, None],
                     vn.view(torch.int16).cpu().numpy().view(np.uint16)[:, None], x["pos"])
    assert np.array_equal(want[1], rk) and np.array_equal(want[2], rv)
    assert_parity(host_f64(out_e), oracle.swa_decode(rk, rv, ko, vo, w.W, oracle.BF16, 1.0, 1.0, x["q"], x["pos"],
                                                      w.Hkv, 0.0625), "eager split-K fused decode")
    out_g = torch.empty_like(out_e)
    for rep, (o, kb, vb) in replay_and_check(
            lambda: swr.swa_append_decode(Lg, kn, vn, q, pos, 0.0625, out=out_g, ws=ws),
            lambda: (out_g, Lg.k_base, Lg.v_base), busy_work()):
        assert np.array_equal(host_bits(o), want[0]), rep
        assert np.array_equal(kb.cpu().numpy(), want[1]) and np.array_equal(vb.cpu().numpy(), want[2]), rep


def fused_global_in_graph(x, S, cap, dtype, ks, vs):
    """Regions hold keys 0 .. pos0-1; the call stores the S tokens at pos0 and
    attends over key_count = pos0 + S."""
    kc = x["key_count"].astype(np.int32)
    B, _, hkv, D = x["k"].shape
    pos0 = (kc - S).astype(np.int32)
    kp, vp, ko, vo = global_pools(x["k"], x["v"], pos0, cap, dtype, ks, vs)
    kn = dev_bf16(np.stack([x["k"][b, pos0[b]:kc[b]] for b in range(B)]))
    vn = dev_bf16(np.stack([x["v"][b, pos0[b]:kc[b]] for b in range(B)]))
    q, p0 = dev_bf16(x["q"]), dev_i32(pos0)
    Hq = x["q"].shape[2]
    ws = torch.zeros(swr.workspace_bytes(swr.SWR_OP_GLOBAL_APPEND_ATTEND, B, S, Hq, hkv, D, int(kc.max())),
                     dtype=torch.uint8, device="cuda")
    Le, Lg = copies(kp, vp, ko, vo, cap, dtype, ks, vs)
    scale = D ** -0.5
    out_e = swr.global_append_attend(Le, kn, vn, q, p0, int(kc.max()), scale, ws=ws)
    torch.cuda.synchronize()
    want = (host_bits(out_e), Le.k_base.cpu().numpy(), Le.v_base.cpu().numpy())
    rk, rv = kp.copy(), vp.copy()
    kn_h = np.stack([x["k"][b, pos0[b]:kc[b]] for b in range(B)])
    vn_h = np.stack([x["v"][b, pos0[b]:kc[b]] for b in range(B)])
    oracle.kv_append(rk, rv, ko, vo, cap, dtype, ks, vs, kn_h, vn_h, pos0, wrap=False)
    assert np.array_equal(want[1], rk) and np.array_equal(want[2], rv)
    q_pos = (pos0[:, None] + np.arange(S, dtype=np.int32)[None, :]).astype(np.int32)
    ref = oracle.global_attend(rk, rv, ko, vo, cap, dtype, ks, vs, x["q"], q_pos, kc, hkv, scale)
    assert_parity(host_f64(out_e), ref, "eager fused global")
    out_g = torch.empty_like(out_e)
    for rep, (o, kb, vb) in replay_and_check(
            lambda: swr.global_append_attend(Lg, kn, vn, q, p0, int(kc.max()), scale, out=out_g, ws=ws),
            lambda: (out_g, Lg.k_base, Lg.v_base), busy_work()):
        assert np.array_equal(host_bits(o), want[0]), rep
        assert np.array_equal(kb.cpu().numpy(), want[1]) and np.array_equal(vb.cpu().numpy(), want[2]), rep


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_fused_global_verify_in_graph(dtype):
    # one request, 6005 keys: the chunked form
    w = synthetic.GLOBAL_VERIFY
    ks, vs = (0.0099, 0.0108) if dtype == oracle.FP8 else (1.0, 1.0)
    fused_global_in_graph(synthetic.global_verify(w, seed=82), w.S, 6016, dtype, ks, vs)


def test_fused_global_streamed_in_graph():
    # 8 requests up to 5000 keys: the append kernel, the streamed pass and its merge
    kc = np.array([1, 63, 64, 65, 700, 2000, 4099, 5000], np.int32)
    g = synthetic.rng(84)
    B = kc.size
    x = dict(key_count=kc, k=synthetic.normal_bf16(g, (B, 5000, 2, 512)),
             v=synthetic.normal_bf16(g, (B, 5000, 2, 512)), q=synthetic.normal_bf16(g, (B, 1, 16, 512)))
    fused_global_in_graph(x, 1, 5056, oracle.BF16, 1.0, 1.0)


def test_global_attend_in_graph():
    w = synthetic.GLOBAL_VERIFY
    x = synthetic.global_verify(w, seed=83)
    kp, vp, ko, vo = global_pools(x["k"], x["v"], x["key_count"], 6016)
    L = layer(kp, vp, ko, vo, 6016)
    q, qp, kcs = dev_bf16(x["q"]), dev_i32(x["q_pos"]), dev_i32(x["key_count"])
    ws = torch.zeros(swr.workspace_bytes(swr.SWR_OP_GLOBAL_ATTEND, 1, w.S, w.Hq, w.Hkv, w.D, w.key_count),
                     dtype=torch.uint8, device="cuda")
    out_e = swr.global_attend(L, q, qp, kcs, w.key_count, w.Hkv, w.D ** -0.5, ws=ws)
    torch.cuda.synchronize()
    want = host_bits(out_e)
    ref = oracle.global_attend(kp, vp, ko, vo, 6016, oracle.BF16, 1, 1, x["q"], x["q_pos"], x["key_count"], w.Hkv,
                               w.D ** -0.5)
    assert_parity(host_f64(out_e), ref, "eager global")
    out_g = torch.empty_like(out_e)
    for rep, (o,) in replay_and_check(
            lambda: swr.global_attend(L, q, qp, kcs, w.key_count, w.Hkv, w.D ** -0.5, out=out_g, ws=ws),
            lambda: (out_g,), busy_work()):
        assert np.array_equal(host_bits(o), want), rep


def test_paged_gather_then_decode_in_graph():
    # the paged-cache baseline's two launches (gather, then the ring decode)
    # captured together; the ring workspace starts from random bytes
    W, hkv, d, G, pt = 256, 2, 128, 4, 16
    pos = np.array([3, 255, 256, 700, 1000], np.int32)
    B = pos.size
    g = synthetic.rng(97)
    n_pages = int((pos // pt + 1).sum()) + 3
    kpages = dev_bf16(synthetic.normal_bf16(g, (n_pages, pt, hkv, d)))
    vpages = dev_bf16(synthetic.normal_bf16(g, (n_pages, pt, hkv, d)))
    per = int(pos.max()) // pt + 1
    ids = np.random.default_rng(97).permutation(n_pages)
    bt = np.full((B, per), -1, np.int32)
    k = 0
    for b in range(B):
        n = int(pos[b]) // pt + 1
        bt[b, :n] = ids[k:k + n]
        k += n
    bt, pos_d = dev_i32(bt), dev_i32(pos)
    q = dev_bf16(synthetic.normal_bf16(g, (B, hkv * G, d)))
    rb = oracle.region_bytes(W, hkv, d, oracle.BF16)
    start = g.integers(0, 256, B * rb, dtype=np.uint8)
    off = np.arange(B, dtype=np.int64) * rb
    Le, Lg = copies(start, start, off, off, W)
    ws = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_SWA_DECODE, B, 1, hkv * G, hkv, d, W)),
                     dtype=torch.uint8, device="cuda")  # 10 units: split-K with its combine
    swr.paged_gather_window(kpages, vpages, bt, pos_d, Le)
    out_e = swr.swa_decode(Le, q, pos_d, hkv, d ** -0.5, ws=ws)
    torch.cuda.synchronize()
    want = (host_bits(out_e), Le.k_base.cpu().numpy(), Le.v_base.cpu().numpy())
    out_g = torch.empty_like(out_e)

    def run():
        swr.paged_gather_window(kpages, vpages, bt, pos_d, Lg)
        swr.swa_decode(Lg, q, pos_d, hkv, d ** -0.5, out=out_g, ws=ws)

    for rep, (o, kb, vb) in replay_and_check(run, lambda: (out_g, Lg.k_base, Lg.v_base), busy_work()):
        assert np.array_equal(host_bits(o), want[0]), rep
        assert np.array_equal(kb.cpu().numpy(), want[1]) and np.array_equal(vb.cpu().numpy(), want[2]), rep
