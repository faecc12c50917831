"""The mixed serving step: 16 requests, contexts log-uniform on [512, 65536],
a sliding layer (W=1024 rings, 8 KV heads x 256) and a global layer
(contiguous regions, 2 KV heads x 512, one query position each) carved from
one pool ("Improving Decode Throughput on Intel Gaudi 3", Our approach: rings
come from the same HBM pool as global-layer KV).  Run with bf16 K/V and with
fp8 e4m3 K/V holding per-tensor scales ("gemma-cuda-hybrid", Features: FP8
(e4m3) KV cache).

The pool image is written on the host by the oracle's append at offsets from
an independent first-fit model (which must agree with the library's pool
carve), copied to the device, and both sides attend over it.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sliding_window_ring_amd as swr
import synthetic
from gpu_common import dev_bf16, dev_i32, dev_i64, host_f64
from helpers import assert_parity

pytestmark = pytest.mark.gpu

W, SHKV, SD, GHKV, GD, G = 1024, 8, 256, 2, 512, 8
ALIGN = 256


def carve(ctx, dtype):
    """Offsets of each request's ring K/V and global K/V, first fit with no
    frees (consecutive 256-byte aligned ranges); global capacity pad64(ctx+1)."""
    off, lay = 0, []
    for c in ctx:
        entry = {}
        for name, cap, hkv, d in (("ring", W, SHKV, SD), ("glob", -(-(int(c) + 1) // 64) * 64, GHKV, GD)):
            rb = oracle.region_bytes(cap, hkv, d, dtype)
            ko = off
            off = -(-(off + rb) // ALIGN) * ALIGN
            vo = off
            off = -(-(off + rb) // ALIGN) * ALIGN
            entry[name] = (ko, vo, cap)
        lay.append(entry)
    return lay, off


def library_carve(ctx, dtype, total):
    h = ctypes.c_void_p()
    assert swr.lib.swr_pool_create(None, total, ctypes.byref(h)) == 0  # bookkeeping only
    out = []
    for c in ctx:
        entry = {}
        for name, tokens, hkv, d, gl in (("ring", W, SHKV, SD, 0), ("glob", int(c) + 1, GHKV, GD, 1)):
            ko, vo, cap = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int32()
            carve = swr.lib.swr_pool_alloc_global if gl else swr.lib.swr_pool_alloc_ring
            assert carve(h, tokens, hkv, d, dtype, None, ctypes.byref(ko), ctypes.byref(vo), ctypes.byref(cap)) == 0
            entry[name] = (ko.value, vo.value, cap.value)
        out.append(entry)
    swr.lib.swr_pool_destroy(h)
    return out


@pytest.fixture(scope="module")
def step_inputs():
    ctx = synthetic.mixed_contexts()
    seed = synthetic.SEED_BASE + 5
    ring_k, ring_v, glob_k, glob_v = [], [], [], []
    for b, c in enumerate(ctx):
        n = min(int(c) + 1, W)
        k, v = synthetic.request_tokens(seed, 2 * b, n, SHKV, SD)
        ring_k.append(k)
        ring_v.append(v)
        k, v = synthetic.request_tokens(seed, 2 * b + 1, int(c) + 1, GHKV, GD)
        glob_k.append(k)
        glob_v.append(v)
    g = synthetic.rng(seed)
    qs = synthetic.normal_bf16(g, (len(ctx), SHKV * G, SD))
    qg = synthetic.normal_bf16(g, (len(ctx), 1, GHKV * G, GD))
    return ctx, ring_k, ring_v, glob_k, glob_v, qs, qg


def amax_scale(arrays):
    return float(max(np.abs(synthetic.bf16_to_f32(a)).max() for a in arrays)) / 448.0


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_mixed_step_shared_pool(step_inputs, dtype):
    ctx, ring_k, ring_v, glob_k, glob_v, qs, qg = step_inputs
    B = len(ctx)
    lay, total = carve(ctx, dtype)
    assert library_carve(ctx, dtype, total) == lay  # the library's carve is the model's first fit
    if dtype == oracle.FP8:
        sks, svs = amax_scale(ring_k), amax_scale(ring_v)
        gks, gvs = amax_scale(glob_k), amax_scale(glob_v)
    else:
        sks = svs = gks = gvs = 1.0
    pool = np.zeros(total, np.uint8)
    for b, c in enumerate(ctx):
        n = ring_k[b].shape[0]
        ko, vo, cap = lay[b]["ring"]
        oracle.kv_append(pool, pool, [ko], [vo], cap, dtype, sks, svs, ring_k[b][None], ring_v[b][None],
                         [int(c) - n + 1])
        ko, vo, cap = lay[b]["glob"]
        oracle.kv_append(pool, pool, [ko], [vo], cap, dtype, gks, gvs, glob_k[b][None], glob_v[b][None], [0],
                         wrap=False, caps=[cap])
    pos = np.asarray(ctx, np.int32)
    rk = np.array([lay[b]["ring"][0] for b in range(B)], np.int64)
    rv = np.array([lay[b]["ring"][1] for b in range(B)], np.int64)
    gk = np.array([lay[b]["glob"][0] for b in range(B)], np.int64)
    gv = np.array([lay[b]["glob"][1] for b in range(B)], np.int64)
    caps = np.array([lay[b]["glob"][2] for b in range(B)], np.int32)
    kc = (pos + 1).astype(np.int32)

    ref_s = oracle.swa_decode(pool, pool, rk, rv, W, dtype, sks, svs, qs, pos, SHKV, SD ** -0.5)
    ref_g = oracle.global_attend(pool, pool, gk, gv, int(caps.max()), dtype, gks, gvs, qg, pos[:, None], kc,
                                 GHKV, GD ** -0.5, caps=caps)

    dpool = torch.from_numpy(pool).cuda()
    sliding = swr.KVLayer(dpool, dpool, dev_i64(rk), dev_i64(rv), W, dtype, sks, svs)
    glob = swr.KVLayer(dpool, dpool, dev_i64(gk), dev_i64(gv), int(caps.max()), dtype, gks, gvs,
                       cap_b=dev_i32(caps))
    out_s = swr.swa_decode(sliding, dev_bf16(qs), dev_i32(pos), SHKV, SD ** -0.5)
    out_g = swr.global_attend(glob, dev_bf16(qg), dev_i32(pos[:, None]), dev_i32(kc), int(kc.max()), GHKV,
                              GD ** -0.5)
    torch.cuda.synchronize()
    e1 = assert_parity(host_f64(out_s), ref_s, "mixed sliding layer")
    e2 = assert_parity(host_f64(out_g), ref_g, "mixed global layer")
    print(f"mixed {'fp8' if dtype else 'bf16'}: sliding max-abs {e1[0]:.2e} rel {e1[1]:.2e}; "
          f"global max-abs {e2[0]:.2e} rel {e2[1]:.2e}")


def test_global_back_to_back_calls_share_a_workspace():
    """The merge counters live in the workspace: two calls in a row with
    different inputs and one workspace both match the oracle."""
    kc = 3000
    w = synthetic.Workload("t", B=2, Hkv=2, G=8, D=512, S=4, key_count=kc)
    ws = torch.zeros(swr.workspace_bytes(swr.SWR_OP_GLOBAL_ATTEND, 2, 4, 16, 2, 512, kc), dtype=torch.uint8,
                     device="cuda")
    for seed in (51, 52, 53):
        x = synthetic.global_verify(w, seed=seed)
        cap = 3008
        from helpers import global_pools
        kp, vp, ko, vo = global_pools(x["k"], x["v"], x["key_count"], cap)
        ref = oracle.global_attend(kp, vp, ko, vo, cap, oracle.BF16, 1, 1, x["q"], x["q_pos"], x["key_count"], 2,
                                   512 ** -0.5)
        L = swr.KVLayer(torch.from_numpy(kp).cuda(), torch.from_numpy(vp).cuda(), dev_i64(ko), dev_i64(vo), cap)
        out = swr.global_attend(L, dev_bf16(x["q"]), dev_i32(x["q_pos"]), dev_i32(x["key_count"]), kc, 2,
                                512 ** -0.5, ws=ws)
        torch.cuda.synchronize()
        assert_parity(host_f64(out), ref, f"global call seed {seed}")
