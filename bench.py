#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one sliding-window layer of the B=56 decode batch (append the new
token into each request's 1024-slot ring, then GQA decode over the ring) plus
one global layer of the 6005-key speculative verify (append the 4 proposals,
then the grouped 32-row attention over the 64-padded region).  Every step
uses the K/V of a different layer (3 sliding layers x 470 MB, 24 global
layers x 24.6 MB, all carved from one pool), so the K/V stream comes from
HBM and not from the 256 MB Infinity Cache.

Prints one JSON line: aggregate algorithmic K/V GB/s of the step, us/layer of
each layer type, the roofline of the dominant kernel (the sliding decode),
and the oracle's rate on the host cores as a CPU baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s

# workload constants (see synthetic/__init__.py for their sources)
B, HKV, G, D, W = 56, 8, 8, 256, 1024          # sliding decode layer
GB_, GHKV, GG, GD, GS, KC = 1, 2, 8, 512, 4, 6005  # global verify layer
N_SLIDING_SETS, N_GLOBAL_SETS = 3, 24

PMC_SUMMARY = os.path.join(ROOT, "profiles", "swa_decode_b56_hbm_traffic.json")
KERNEL_SOURCES = [os.path.join(ROOT, "sliding_window_ring_amd", "csrc", f)
                  for f in ("attn.hip", "swr_device.h", "swr_internal.h")]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        with open(f, "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(bytes_per_launch_algo):
    """HBM bytes per decode launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel source; else None."""
    try:
        with open(PMC_SUMMARY) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_hash") != kernel_source_hash():
        return None
    return s.get("hbm_bytes_per_launch")


def build_layers(swr, torch, pool):
    """Carve and fill all layer sets from one pool."""
    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1002)
    sliding = []
    for _ in range(N_SLIDING_SETS):
        ko, vo = [], []
        for _b in range(B):
            k_off, v_off, cap = pool.alloc_kv(W, HKV, D)
            ko.append(k_off)
            vo.append(v_off)
        L = swr.KVLayer(pool.buffer, pool.buffer, torch.tensor(ko, device=dev), torch.tensor(vo, device=dev), W)
        pos = torch.randint(1024, 4097, (B,), device=dev, dtype=torch.int32, generator=gen)
        # history: the W-1 tokens before pos, written through the library's own append
        for half in range(2):
            k = torch.randn(B, W // 2, HKV, D, device=dev, generator=gen).to(torch.bfloat16)
            v = torch.randn(B, W // 2, HKV, D, device=dev, generator=gen).to(torch.bfloat16)
            swr.kv_append(L, k, v, (pos - W + half * (W // 2)).to(torch.int32))
        k_new = torch.randn(B, 1, HKV, D, device=dev, generator=gen).to(torch.bfloat16)
        v_new = torch.randn(B, 1, HKV, D, device=dev, generator=gen).to(torch.bfloat16)
        q = torch.randn(B, HKV * G, D, device=dev, generator=gen).to(torch.bfloat16)
        sliding.append(dict(L=L, pos=pos, k_new=k_new, v_new=v_new, q=q, out=torch.empty_like(q)))
    glob = []
    for _ in range(N_GLOBAL_SETS):
        k_off, v_off, cap = pool.alloc_kv(KC, GHKV, GD, global_layer=True)
        L = swr.KVLayer(pool.buffer, pool.buffer, torch.tensor([k_off], device=dev),
                        torch.tensor([v_off], device=dev), cap)
        ctx = KC - GS
        k = torch.randn(1, ctx, GHKV, GD, device=dev, generator=gen).to(torch.bfloat16)
        v = torch.randn(1, ctx, GHKV, GD, device=dev, generator=gen).to(torch.bfloat16)
        swr.kv_append(L, k, v, torch.zeros(1, device=dev, dtype=torch.int32), wrap=False)
        k_prop = torch.randn(1, GS, GHKV, GD, device=dev, generator=gen).to(torch.bfloat16)
        v_prop = torch.randn(1, GS, GHKV, GD, device=dev, generator=gen).to(torch.bfloat16)
        q = torch.randn(1, GS, GHKV * GG, GD, device=dev, generator=gen).to(torch.bfloat16)
        glob.append(dict(L=L, ctx=torch.tensor([ctx], device=dev, dtype=torch.int32),
                         q_pos=torch.arange(ctx, KC, device=dev, dtype=torch.int32).view(1, GS),
                         kc=torch.tensor([KC], device=dev, dtype=torch.int32), k_prop=k_prop, v_prop=v_prop,
                         q=q, out=torch.empty_like(q)))
    torch.cuda.synchronize()
    return sliding, glob


def algorithmic_bytes():
    """Bytes each operation must move (K/V read at the exact key count, new
    tokens read and written, queries read, outputs written)."""
    decode = B * HKV * W * D * 2 * 2 + 2 * B * HKV * G * D * 2
    append_s = B * HKV * D * 2 * 2 * 2
    glob = KC * GHKV * GD * 2 * 2 + 2 * GS * GHKV * GG * GD * 2
    append_g = GS * GHKV * GD * 2 * 2 * 2
    return decode, append_s, glob, append_g


def cpu_baseline(seconds: float = 12.0):
    """The oracle on a bounded sample of the same workload: 16 of the 56
    decode requests plus the global verify, repeated for about `seconds`."""
    import numpy as np

    import oracle
    import synthetic

    sys.path.insert(0, os.path.join(ROOT, "tests"))
    from helpers import global_pools, ring_pools

    nb = 16
    w = synthetic.Workload("sample", B=nb, Hkv=HKV, G=G, D=D, W=W, pos_lo=1024, pos_hi=4096)
    x = synthetic.sliding_decode(w, seed=synthetic.SEED_BASE + 2)
    kp, vp, ko, vo = ring_pools(x["k"], x["v"], x["start"], x["n"], W)
    gx = synthetic.global_verify()
    gk, gv, gko, gvo = global_pools(gx["k"], gx["v"], gx["key_count"], 6016)
    per_rep = nb * HKV * W * D * 4 + 2 * nb * HKV * G * D * 2 + algorithmic_bytes()[2]
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.swa_decode(kp, vp, ko, vo, W, oracle.BF16, 1, 1, x["q"], x["pos"], HKV, 1 / 16)
        oracle.global_attend(gk, gv, gko, gvo, 6016, oracle.BF16, 1, 1, gx["q"], gx["q_pos"], gx["key_count"],
                             GHKV, GD ** -0.5)
        reps += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    return {"value": round(per_rep * reps / el / 1e9, 4), "unit": "GB/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{reps} repetitions of: sliding decode for 16 of the 56 requests (full 1024-key windows, "
                      f"8 KV heads x 256) + the 6005-key global verify; binary64 C oracle, {el:.1f} s"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for --gpus {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import sliding_window_ring_amd as swr

    torch.cuda.set_device(0)
    if args.copy_calibration:
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_launch": {"read": 1 << 30, "write": 1 << 30}}))
        return
    per_layer_pool = B * 2 * swr.region_bytes(W, HKV, D) * N_SLIDING_SETS + \
        N_GLOBAL_SETS * 2 * swr.region_bytes(6016, GHKV, GD) + (1 << 20)
    pool = swr.Pool(per_layer_pool)
    sliding, glob = build_layers(swr, torch, pool)
    gws = torch.empty(max(swr.workspace_bytes(swr.SWR_OP_GLOBAL_ATTEND, 1, GS, GHKV * GG, GHKV, GD, KC), 16),
                      dtype=torch.uint8, device="cuda")
    dws = torch.empty(max(swr.workspace_bytes(swr.SWR_OP_SWA_DECODE, B, 1, HKV * G, HKV, D, W), 16),
                      dtype=torch.uint8, device="cuda")
    scale_s, scale_g = D ** -0.5, GD ** -0.5

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]

    def global_layer(g):
        swr.kv_append(g["L"], g["k_prop"], g["v_prop"], g["ctx"], wrap=False)
        swr.global_attend(g["L"], g["q"], g["q_pos"], g["kc"], KC, GHKV, scale_g, out=g["out"], ws=gws)

    def step(i, events=None):
        s = sliding[i % N_SLIDING_SETS]
        g = glob[i % N_GLOBAL_SETS]
        if events:
            events[0].record()
        swr.kv_append(s["L"], s["k_new"], s["v_new"], s["pos"])
        if events:
            events[1].record()
        swr.swa_decode(s["L"], s["q"], s["pos"], HKV, scale_s, out=s["out"], ws=dws)
        if events:
            events[2].record()
        global_layer(g)
        if events:
            events[3].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(i, ev[i])
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    append_s = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps * 1e3
    decode_us = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps * 1e3
    global_us = sum(e[2].elapsed_time(e[3]) for e in ev) / args.steps * 1e3

    # The global layer's launches are short: also time them the way a serving
    # loop issues them, captured in one HIP graph holding all 24 global layers.
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for g in glob:
            global_layer(g)
    graph.replay()
    torch.cuda.synchronize()
    g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    g0.record()
    for _ in range(reps):
        graph.replay()
    g1.record()
    torch.cuda.synchronize()
    global_graph_us = g0.elapsed_time(g1) / (reps * N_GLOBAL_SETS) * 1e3
    b_dec, b_app_s, b_glob, b_app_g = algorithmic_bytes()
    step_bytes = b_dec + b_app_s + b_glob + b_app_g
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = b_dec / (decode_us * 1e-6) / 1e9
    traffic = measured_traffic(b_dec)

    result = {
        "metric": "attention KV GB/s & % HBM peak; us/layer, sliding decode B=56 + global verify",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "one sliding-window decode layer (B=56, ring W=1024, 8 KV heads x 256, 8 q heads per KV "
                        "head, positions U[1024,4096]) + one global verify layer (B=1, 2 KV heads x 512, 8 q heads "
                        "per KV head x 4 proposals = 32 rows, 6005 keys padded to 6016); K/V bf16",
            "sliding_layer_sets": N_SLIDING_SETS, "global_layer_sets": N_GLOBAL_SETS,
            "algorithmic_bytes_per_step": step_bytes,
        },
        "hbm_peak_frac": round(value / HBM_PEAK_GBS, 4),
        "us_per_layer": {
            "sliding_decode_b56_attention": round(decode_us, 2),
            "sliding_decode_b56_append": round(append_s, 2),
            "global_verify_6005_append_and_attention": round(global_us, 2),
            "global_verify_6005_in_layer_graph": round(global_graph_us, 2),
        },
        "layer_gbs": {
            "sliding_decode_b56_attention": round(achieved, 1),
            "global_verify_6005": round((b_glob + b_app_g) / (global_us * 1e-6) / 1e9, 1),
            "global_verify_6005_in_layer_graph": round((b_glob + b_app_g) / (global_graph_us * 1e-6) / 1e9, 1),
        },
        "roofline": {
            "kernel": "attn_kernel<256,256,1,4,bf16,decode> (swr_swa_decode, B=56)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": b_dec,
        },
        "host_wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline()
    print(json.dumps(result))


if __name__ == "__main__":
    main()
