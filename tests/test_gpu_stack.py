"""A decode step through a multi-layer attention stack, captured in one HIP
graph and replayed, against the oracle.

"Improving Decode Throughput on Intel Gaudi 3" (Patching sliding window KV
allocation) describes Gemma 4's mix: sliding-window layers with a global
layer after every five.  "gemma-cuda-hybrid" (Features) captures the step in a
graph.  Here the step is two groups of five sliding layers and one global
layer; every layer owns its K/V regions and its query, and appends its own new
token (swr_swa_append_decode; swr_global_append_attend with one token) before
attending.  The twelve calls are captured once; each replay is a new decode
step: the positions advance by one and new tokens and queries are copied in
between replays (eager work outside the graph).  After every replay each
layer's output is compared with the oracle at the parity bar and every
region's bytes with the oracle's appends, bit for bit.  Requests sit at
positions before, at and past the ring's wrap, and both the decode's split
combine and the global layer's chunked form run (12 (request, KV head) units).
"""
import numpy as np
import pytest
import torch

import oracle
import sliding_window_ring_amd as swr
import synthetic
from gpu_common import dev_bf16, dev_i32, host_f64, layer
from helpers import assert_parity, global_pools, ring_pools

pytestmark = pytest.mark.gpu

B = 6
W, SHKV, SD = 512, 2, 256          # sliding layers (16 tiles: the decode splits each ring in two)
GHKV, GD = 2, 512                  # global layers
G = 8
GROUPS, PER_GROUP = 2, 5
STEPS = 3
POS0 = np.array([0, 5, 510, 511, 900, 3000], np.int32)  # position of step 0's token


def layer_kinds():
    return [("s", i) for i in range(GROUPS * PER_GROUP)] + [("g", i) for i in range(GROUPS)]


def order():
    """Call order: five sliding layers, then a global one, per group."""
    seq = []
    for grp in range(GROUPS):
        seq += [("s", grp * PER_GROUP + j) for j in range(PER_GROUP)] + [("g", grp)]
    return seq


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_decode_stack_in_one_graph_matches_oracle(dtype):
    g = synthetic.rng(synthetic.SEED_BASE + 90 + dtype)
    cap_g = -(-(int(POS0.max()) + STEPS) // 64) * 64
    fp8 = dtype == oracle.FP8
    ks = vs = (4.5 / 448 if fp8 else 1.0)
    host, dev = {}, {}
    # sliding layers: the W - 1 positions before step 0's token, as far as
    # they exist; global layers: every position before it
    for kind, i in layer_kinds():
        if kind == "s":
            n = np.minimum(POS0, W - 1).astype(np.int32)
            k = synthetic.normal_bf16(g, (B, W, SHKV, SD))
            v = synthetic.normal_bf16(g, (B, W, SHKV, SD))
            kp, vp, ko, vo = ring_pools(k, v, (POS0 - n).astype(np.int32), n, W, dtype, ks, vs)
            cap = W
        else:
            k = synthetic.normal_bf16(g, (B, int(POS0.max()) + 1, GHKV, GD))
            v = synthetic.normal_bf16(g, (B, int(POS0.max()) + 1, GHKV, GD))
            kp, vp, ko, vo = global_pools(k, v, POS0, cap_g, dtype, ks, vs)
            cap = cap_g
        host[kind, i] = [kp, vp, ko, vo, cap]
        dev[kind, i] = layer(kp, vp, ko, vo, cap, dtype, ks, vs)

    # per-layer device inputs the graph reads (refilled between replays)
    hq_s, hq_g = SHKV * G, GHKV * G
    tok = {}
    for kind, i in layer_kinds():
        if kind == "s":
            tok[kind, i] = dict(k=torch.empty(B, SHKV, SD, dtype=torch.bfloat16, device="cuda"),
                                v=torch.empty(B, SHKV, SD, dtype=torch.bfloat16, device="cuda"),
                                q=torch.empty(B, hq_s, SD, dtype=torch.bfloat16, device="cuda"),
                                out=torch.empty(B, hq_s, SD, dtype=torch.bfloat16, device="cuda"))
        else:
            tok[kind, i] = dict(k=torch.empty(B, 1, GHKV, GD, dtype=torch.bfloat16, device="cuda"),
                                v=torch.empty(B, 1, GHKV, GD, dtype=torch.bfloat16, device="cuda"),
                                q=torch.empty(B, 1, hq_g, GD, dtype=torch.bfloat16, device="cuda"),
                                out=torch.empty(B, 1, hq_g, GD, dtype=torch.bfloat16, device="cuda"))
    pos = dev_i32(POS0)
    ws_s = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_SWA_APPEND_DECODE, B, 1, hq_s, SHKV, SD, W)),
                       dtype=torch.uint8, device="cuda")
    ws_g = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_GLOBAL_APPEND_ATTEND, B, 1, hq_g, GHKV, GD, cap_g)),
                       dtype=torch.uint8, device="cuda")
    assert swr.workspace_bytes(swr.SWR_OP_SWA_APPEND_DECODE, B, 1, hq_s, SHKV, SD, W) > 0  # split combine runs

    def step():
        for kind, i in order():
            t = tok[kind, i]
            if kind == "s":
                swr.swa_append_decode(dev[kind, i], t["k"], t["v"], t["q"], pos, SD ** -0.5, out=t["out"], ws=ws_s)
            else:
                swr.global_append_attend(dev[kind, i], t["k"], t["v"], t["q"], pos, cap_g, GD ** -0.5,
                                         out=t["out"], ws=ws_g)

    def new_inputs():
        x = {}
        for kind, i in layer_kinds():
            hkv, d, hq = (SHKV, SD, hq_s) if kind == "s" else (GHKV, GD, hq_g)
            x[kind, i] = (synthetic.normal_bf16(g, (B, hkv, d)), synthetic.normal_bf16(g, (B, hkv, d)),
                          synthetic.normal_bf16(g, (B, hq, d)))
        return x

    # capture with the step-0 inputs in place (capture runs nothing)
    x = new_inputs()
    for key, (k, v, q) in x.items():
        t = tok[key]
        t["k"].copy_(dev_bf16(k).view(t["k"].shape))
        t["v"].copy_(dev_bf16(v).view(t["v"].shape))
        t["q"].copy_(dev_bf16(q).view(t["q"].shape))
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    busy = torch.randn(1 << 20, device="cuda")

    for s in range(STEPS):
        p = (POS0 + s).astype(np.int32)
        if s > 0:
            x = new_inputs()
            for key, (k, v, q) in x.items():
                t = tok[key]
                t["k"].copy_(dev_bf16(k).view(t["k"].shape))
                t["v"].copy_(dev_bf16(v).view(t["v"].shape))
                t["q"].copy_(dev_bf16(q).view(t["q"].shape))
            pos.copy_(dev_i32(p))
        busy.mul_(1.0001).add_(0.5)  # unrelated eager work before the replay
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for kind, i in order():
            kp, vp, ko, vo, cap = host[kind, i]
            k, v, q = x[kind, i]
            what = f"step {s} layer {kind}{i} ({'fp8' if fp8 else 'bf16'})"
            if kind == "s":
                oracle.kv_append(kp, vp, ko, vo, W, dtype, ks, vs, k[:, None], v[:, None], p)
                ref = oracle.swa_decode(kp, vp, ko, vo, W, dtype, ks, vs, q, p, SHKV, SD ** -0.5)
            else:
                oracle.kv_append(kp, vp, ko, vo, cap, dtype, ks, vs, k[:, None], v[:, None], p, wrap=False)
                ref = oracle.global_attend(kp, vp, ko, vo, cap, dtype, ks, vs, q[:, None], p[:, None], p + 1,
                                           GHKV, GD ** -0.5)
            L = dev[kind, i]
            assert np.array_equal(L.k_base.cpu().numpy(), kp), what + ": K region bytes"
            assert np.array_equal(L.v_base.cpu().numpy(), vp), what + ": V region bytes"
            assert_parity(host_f64(tok[kind, i]["out"]), ref, what)
