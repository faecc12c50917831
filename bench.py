#!/usr/bin/env python3
"""Benchmark of the attention hot path on one MI355X.

One step = one sliding-window layer of the B=56 decode batch (append the new
token into each request's 1024-slot ring, then GQA decode over the ring) plus
one global layer of the 6005-key speculative verify (append the 4 proposals,
then the grouped 32-row attention over the 64-padded region).  Each layer is
one library call that does both (swr_swa_append_decode,
swr_global_append_attend); the separate append and attention calls are timed
beside it.  Every step uses the K/V of a different layer (3 sliding layers x
470 MB, 24 global layers x 24.6 MB, all carved from one pool), so the K/V
stream comes from HBM and not from the 256 MB Infinity Cache.

Prints one JSON line: aggregate algorithmic K/V GB/s of the step, us/layer of
each layer type, the roofline of the dominant kernel (the sliding decode),
the chip's measured streaming-read ceiling, the other workloads (sliding
verify, fp8 decode, the paged-cache baseline of the decode, the mixed step,
a 60-layer decode stack, the global key-count sweep) and the oracle's rate
on the host cores as a CPU baseline.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
                    [--no-extra] [--no-sweep]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E peak, GB/s

# workload constants (see synthetic/__init__.py for their sources)
B, HKV, G, D, W = 56, 8, 8, 256, 1024          # sliding decode layer
GB_, GHKV, GG, GD, GS, KC = 1, 2, 8, 512, 4, 6005  # global verify layer
N_SLIDING_SETS, N_GLOBAL_SETS = 3, 24

# Counter summaries (rocprofv3 FETCH_SIZE / WRITE_SIZE, scaled by a 1 GiB
# copy) of the kernels each roofline entry covers, and the sources those
# kernels are built from: a summary is reported only while the sources still
# hash to the value recorded in it.
CSRC = os.path.join(ROOT, "sliding_window_ring_amd", "csrc")
TRAFFIC = {
    "decode": (os.path.join(ROOT, "profiles", "swa_decode_b56_hbm_traffic.json"),
               [os.path.join(CSRC, f) for f in ("attn.hip", "swr_device.h", "swr_internal.h")]),
    "global": (os.path.join(ROOT, "profiles", "global_verify_6005_hbm_traffic.json"),
               [os.path.join(CSRC, f) for f in ("chunked.hip", "swr_device.h", "swr_internal.h")]),
    "verify": (os.path.join(ROOT, "profiles", "sliding_verify_b8_hbm_traffic.json"),
               [os.path.join(CSRC, f) for f in ("chunked.hip", "swr_device.h", "swr_internal.h")]),
}


def code_only(text: str) -> str:
    """C++ source without its comments, trailing blanks and empty lines: a
    change to a comment leaves the kernel, and its counters, as they were.
    (The kernel sources hold no string literal with a comment marker.)"""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return "\n".join(line.rstrip() for line in text.splitlines() if line.strip())


def kernel_source_hash(sources) -> str:
    h = hashlib.sha256()
    for f in sources:
        with open(f, encoding="utf-8") as fh:
            h.update(code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def measured_traffic(which):
    """HBM bytes per launch (per layer for the two-launch forms) from the
    committed counter summary, if it was taken on the current kernel
    sources; else None."""
    path, sources = TRAFFIC[which]
    try:
        with open(path) as f:
            s = json.load(f)
    except (OSError, ValueError):
        return None
    if s.get("kernel_source_hash") != kernel_source_hash(sources):
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
            k_off, v_off, cap = pool.alloc_ring(W, HKV, D)
            ko.append(k_off)
            vo.append(v_off)
        L = swr.KVLayer(pool.buffer, pool.buffer, torch.tensor(ko, device=dev), torch.tensor(vo, device=dev), W)
        pos = torch.randint(1024, 4097, (B,), device=dev, dtype=torch.int32, generator=gen)
        # history: the W-1 tokens before pos, written through the library's own append
        for half in range(2):
            k = torch.randn(B, W // 2, HKV, D, device=dev, generator=gen).to(torch.bfloat16)
            v = torch.randn(B, W // 2, HKV, D, device=dev, generator=gen).to(torch.bfloat16)
            swr.ring_kv_append(L, k, v, (pos - W + half * (W // 2)).to(torch.int32))
        k_new = torch.randn(B, 1, HKV, D, device=dev, generator=gen).to(torch.bfloat16)
        v_new = torch.randn(B, 1, HKV, D, device=dev, generator=gen).to(torch.bfloat16)
        q = torch.randn(B, HKV * G, D, device=dev, generator=gen).to(torch.bfloat16)
        sliding.append(dict(L=L, pos=pos, k_new=k_new, v_new=v_new, q=q, out=torch.empty_like(q)))
    glob = []
    for _ in range(N_GLOBAL_SETS):
        k_off, v_off, cap = pool.alloc_global(KC, GHKV, GD)
        L = swr.KVLayer(pool.buffer, pool.buffer, torch.tensor([k_off], device=dev),
                        torch.tensor([v_off], device=dev), cap)
        ctx = KC - GS
        k = torch.randn(1, ctx, GHKV, GD, device=dev, generator=gen).to(torch.bfloat16)
        v = torch.randn(1, ctx, GHKV, GD, device=dev, generator=gen).to(torch.bfloat16)
        swr.ring_kv_append(L, k, v, torch.zeros(1, device=dev, dtype=torch.int32), wrap=False)
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
    tokens read and written, queries read, outputs written), the same for the
    fused calls as for the separate ones: the fused sliding call moves decode
    + append_s, the fused global call glob + append_g."""
    decode = B * HKV * W * D * 2 * 2 + 2 * B * HKV * G * D * 2
    append_s = B * HKV * D * 2 * 2 * 2
    glob = KC * GHKV * GD * 2 * 2 + 2 * GS * GHKV * GG * GD * 2
    append_g = GS * GHKV * GD * 2 * 2 * 2
    return decode, append_s, glob, append_g


def cpu_baseline():
    """The oracle as it stands (binary64 C, OpenMP over (request, KV head)
    units) on the host's cores, per workload: the median of 3 runs with all
    threads and of 3 with one thread, in us per layer, on the same synthetic
    inputs the tests use.  The large layers are timed on stated samples and
    scaled by the keys they hold (the oracle's time is linear in units x
    keys); the regions are built in the oracle's own logical form.  `value`
    is the headline step's rate on this baseline: the B=56 decode layer plus
    the 6005-key verify layer."""
    import statistics

    import numpy as np

    import oracle
    import synthetic

    oracle.build()
    threads = oracle.num_threads()

    def med3(fn):
        ts = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            ts.append(time.perf_counter() - t0)
        return statistics.median(ts) * 1e6

    def both(fn):
        t_all = med3(fn)
        prev = oracle.set_threads(1)
        t_one = med3(fn)
        oracle.set_threads(prev)
        return t_all, t_one

    def ring_logical(k, v, start, n, w, dtype=oracle.BF16, ks=1.0, vs=1.0):
        B = k.shape[0]
        lrb = oracle.logical_region_bytes(w, k.shape[2], k.shape[3], dtype)
        kl, vl = np.zeros(B * lrb, np.uint8), np.zeros(B * lrb, np.uint8)
        offs = np.arange(B, dtype=np.int64) * lrb
        oracle.kv_append_logical(kl, vl, offs, w, dtype, ks, vs, k, v, start, n, wrap=True)
        return kl, vl, offs

    res = {}
    # sliding decode B=56 (W=1024, 8 x 256): 8 of the 56 requests, x 7
    ws2 = synthetic.Workload("sample", B=8, Hkv=HKV, G=G, D=D, W=W, pos_lo=1024, pos_hi=4096)
    x = synthetic.sliding_decode(ws2, seed=synthetic.SEED_BASE + 2)
    kl, vl, offs = ring_logical(x["k"], x["v"], x["start"], x["n"], W)
    t_all, t_one = both(lambda: oracle.swa_decode_logical(kl, vl, offs, W, oracle.BF16, 1, 1, x["q"], x["pos"],
                                                          HKV, D ** -0.5))
    res["sliding_decode_b56"] = {"oracle_us_per_layer": round(t_all * 7, 1), "oracle_us_per_layer_1_thread":
                                 round(t_one * 7, 1), "threads": min(threads, 8 * HKV),
                                 "sample": "8 of the 56 requests (full windows), time x 7"}
    # sliding verify B=8 (S=4, 32 rows per KV head): whole
    wv = synthetic.SWA_VERIFY
    x = synthetic.sliding_verify()
    kl, vl, offs = ring_logical(x["k"], x["v"], x["start"], x["n"], wv.W)
    t_all, t_one = both(lambda: oracle.gqa_verify_logical(kl, vl, offs, wv.W, oracle.BF16, 1, 1, x["k_prop"],
                                                          x["v_prop"], x["q"], x["p0"], wv.Hkv, wv.D ** -0.5))
    res["sliding_verify_b8"] = {"oracle_us_per_layer": round(t_all, 1), "oracle_us_per_layer_1_thread": round(t_one, 1),
                                "threads": min(threads, wv.B * wv.Hkv), "sample": "whole layer"}
    # global verify, 6005 keys (padded contraction over 6016): whole
    gx = synthetic.global_verify()
    lrb = oracle.logical_region_bytes(6016, GHKV, GD, oracle.BF16)
    gk, gv, goff = np.zeros(lrb, np.uint8), np.zeros(lrb, np.uint8), np.zeros(1, np.int64)
    oracle.kv_append_logical(gk, gv, goff, 6016, oracle.BF16, 1, 1, gx["k"], gx["v"], np.zeros(1, np.int32),
                             gx["key_count"], wrap=False)
    t_all, t_one = both(lambda: oracle.global_attend_logical(gk, gv, goff, 6016, oracle.BF16, 1, 1, gx["q"],
                                                             gx["q_pos"], gx["key_count"], GHKV, GD ** -0.5))
    res["global_verify_6005"] = {"oracle_us_per_layer": round(t_all, 1), "oracle_us_per_layer_1_thread":
                                 round(t_one, 1), "threads": min(threads, GHKV), "sample": "whole layer"}
    # mixed step (16 requests, contexts log-uniform [512, 65536]): the sliding
    # layer whole, the global layer on every eighth request, scaled by keys
    ctx = [int(c) for c in synthetic.mixed_contexts()]
    seed = synthetic.SEED_BASE + 5
    msw, mgw = synthetic.MIXED_SLIDING, synthetic.MIXED_GLOBAL
    sample = list(range(0, len(ctx), 8))
    key_scale = sum(c + 1 for c in ctx) / sum(ctx[b] + 1 for b in sample)
    g = synthetic.rng(seed)
    qs = synthetic.normal_bf16(g, (len(ctx), msw.Hq, msw.D))
    qg = synthetic.normal_bf16(g, (len(sample), 1, mgw.Hq, mgw.D))
    ring = [synthetic.request_tokens(seed, 2 * b, min(c + 1, msw.W), msw.Hkv, msw.D) for b, c in enumerate(ctx)]
    glob = [synthetic.request_tokens(seed, 2 * b + 1, ctx[b] + 1, mgw.Hkv, mgw.D) for b in sample]
    for dtype, name in ((oracle.BF16, "mixed_step_bf16"), (oracle.FP8, "mixed_step_fp8")):
        amax = lambda arrs: float(max(np.abs(synthetic.bf16_to_f32(a)).max() for a in arrs)) / 448.0
        sks, svs = (amax([r[0] for r in ring]), amax([r[1] for r in ring])) if dtype else (1.0, 1.0)
        gks, gvs = (amax([r[0] for r in glob]), amax([r[1] for r in glob])) if dtype else (1.0, 1.0)
        lrb = oracle.logical_region_bytes(msw.W, msw.Hkv, msw.D, dtype)
        skl, svl = np.zeros(len(ctx) * lrb, np.uint8), np.zeros(len(ctx) * lrb, np.uint8)
        soff = np.arange(len(ctx), dtype=np.int64) * lrb
        for b, c in enumerate(ctx):
            n = ring[b][0].shape[0]
            oracle.kv_append_logical(skl, svl, soff[b:b + 1], msw.W, dtype, sks, svs, ring[b][0][None],
                                     ring[b][1][None], [c - n + 1])
        caps = [-(-(ctx[b] + 1) // 64) * 64 for b in sample]
        glr = [oracle.logical_region_bytes(cp, mgw.Hkv, mgw.D, dtype) for cp in caps]
        goffs = np.concatenate([[0], np.cumsum(glr)[:-1]]).astype(np.int64)
        gkl, gvl = np.zeros(int(sum(glr)), np.uint8), np.zeros(int(sum(glr)), np.uint8)
        for i, b in enumerate(sample):
            oracle.kv_append_logical(gkl, gvl, goffs[i:i + 1], caps[i], dtype, gks, gvs, glob[i][0][None],
                                     glob[i][1][None], [0], wrap=False, caps=[caps[i]])
        pos = np.asarray(ctx, np.int32)
        gpos = np.asarray([ctx[b] for b in sample], np.int32)
        ts_all, ts_one = both(lambda: oracle.swa_decode_logical(skl, svl, soff, msw.W, dtype, sks, svs, qs, pos,
                                                                msw.Hkv, msw.D ** -0.5))
        tg_all, tg_one = both(lambda: oracle.global_attend_logical(gkl, gvl, goffs, max(caps), dtype, gks, gvs, qg,
                                                                   gpos[:, None], gpos + 1, mgw.Hkv, mgw.D ** -0.5,
                                                                   caps=caps))
        res[name] = {"oracle_us_per_layer": round(ts_all + tg_all * key_scale, 1),
                     "oracle_us_per_layer_1_thread": round(ts_one + tg_one * key_scale, 1),
                     "threads": {"sliding": min(threads, len(ctx) * msw.Hkv),
                                 "global_sample": min(threads, len(sample) * mgw.Hkv)},
                     "sample": f"one sliding layer (16 requests) + one global layer timed on requests {sample} "
                               f"({len(sample) * mgw.Hkv} units, so at most that many threads) and scaled by keys "
                               f"(x {key_scale:.2f})"}
    b_dec, b_app_s, b_glob, b_app_g = algorithmic_bytes()
    step_us = res["sliding_decode_b56"]["oracle_us_per_layer"] + res["global_verify_6005"]["oracle_us_per_layer"]
    step_us1 = res["sliding_decode_b56"]["oracle_us_per_layer_1_thread"] + \
        res["global_verify_6005"]["oracle_us_per_layer_1_thread"]
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next(line.split(":", 1)[1].strip() for line in f if line.startswith("model name"))
    except (OSError, StopIteration):
        pass
    return {"value": round((b_dec + b_glob) / (step_us * 1e-6) / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": "the step's two layers: sliding decode B=56 (timed on 8 of the 56 requests, x 7) + the "
                      "6005-key global verify; binary64 C oracle, median of 3 runs",
            "value_1_thread": round((b_dec + b_glob) / (step_us1 * 1e-6) / 1e9, 4),
            "per_config": res,
            "host": {"cpu": cpu, "logical_cpus": os.cpu_count(), "oracle_threads": threads}}


def _graph_timed(torch, fn, calls, replays):
    """Average us per call of fn(i), i = 0 .. calls-1, captured once in a HIP
    graph and replayed `replays` times: for calls short enough that launching
    them one by one from Python would time the host's issue rate.  The graph
    must hold enough work that a replay outlasts its own launch from the host
    (tens of microseconds): a few short calls per graph time the launch."""
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(calls):
            fn(i)
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * calls) * 1e3


def _timed(torch, fn, reps, sets):
    """Average us per call of fn(i) over `reps` calls cycling through `sets`,
    with events on the current stream around the whole loop."""
    for i in range(2):
        fn(i % sets)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(reps):
        fn(i % sets)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps * 1e3


def paged_baseline(swr, torch, randn, gen, dev, page_tokens=16):
    """The B=56 decode over a paged cache: per step, swr_paged_gather_window
    copies each request's window out of its pages (ids shuffled over the
    pool) into a ring-layout workspace, and swr_swa_decode reads it.  Only the
    pages that hold window positions are allocated."""
    import numpy as np
    import synthetic
    w = synthetic.SWA_DECODE
    sets = []
    for _ in range(2):
        pos = torch.randint(w.pos_lo, w.pos_hi + 1, (w.B,), device=dev, dtype=torch.int32, generator=gen)
        ph = pos.cpu().numpy().astype(np.int64)
        first, last = np.maximum(ph - w.W + 1, 0) // page_tokens, ph // page_tokens
        n_pages = int((last - first + 1).sum())
        ids = torch.randperm(n_pages, generator=torch.Generator().manual_seed(int(ph.sum()))).numpy()
        bt = np.full((w.B, int(last.max()) + 1), -1, np.int32)
        k = 0
        for b in range(w.B):
            n = int(last[b] - first[b] + 1)
            bt[b, first[b]:last[b] + 1] = ids[k:k + n]
            k += n
        kp = randn(n_pages, page_tokens, w.Hkv, w.D)
        vp = randn(n_pages, page_tokens, w.Hkv, w.D)
        rb = swr.region_bytes(w.W, w.Hkv, w.D)
        kb = torch.zeros(w.B * rb, dtype=torch.uint8, device=dev)
        vb = torch.zeros_like(kb)
        off = torch.arange(w.B, device=dev, dtype=torch.int64) * rb
        L = swr.KVLayer(kb, vb, off, off.clone(), w.W)
        q = randn(w.B, w.Hq, w.D)
        sets.append((kp, vp, torch.from_numpy(bt).to(dev), pos, L, q, torch.empty_like(q)))
    ws = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_SWA_DECODE, w.B, 1, w.Hq, w.Hkv, w.D, w.W)),
                     dtype=torch.uint8, device=dev)

    def gather(i):
        s = sets[i]
        swr.paged_gather_window(s[0], s[1], s[2], s[3], s[4])

    def decode(i):
        s = sets[i]
        swr.swa_decode(s[4], s[5], s[3], w.Hkv, w.D ** -0.5, out=s[6], ws=ws)

    def both(i):
        gather(i)
        decode(i)

    # reference for the gather's rate: torch's device copy of as many bytes
    src = torch.empty(w.B * w.Hkv * w.W * w.D * 2, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)

    def copy(i):
        dst.copy_(src)

    us_g = _timed(torch, gather, 60, len(sets))
    us_d = _timed(torch, decode, 60, len(sets))
    us = _timed(torch, both, 60, len(sets))
    us_c = _timed(torch, copy, 30, 1)
    kv = w.B * w.Hkv * w.W * w.D * 2 * 2
    nbytes = kv + 2 * w.B * w.Hq * w.D * 2
    return {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1), "algorithmic_bytes": nbytes,
            "hbm_peak_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
            "gather_us": round(us_g, 2), "gather_GB/s_moved": round(2 * kv / us_g / 1e3, 1),
            "torch_copy_same_bytes_GB/s_moved": round(2 * kv / (2 * us_c) / 1e3, 1),
            "decode_on_gathered_ring_us": round(us_d, 2), "page_tokens": page_tokens,
            "note": "the same decode kernel after a gather of each window's pages (read and written once more); "
                    "GB/s and hbm_peak_frac count the decode's algorithmic bytes over gather + decode"}


def read_ceiling(swr, torch):
    """Achievable HBM read rate on this chip: the library's plain streaming
    read (swr_read_ceiling) over 2 GiB, alternating two buffers so that no
    launch finds its range in the 256 MB last-level cache; the best of a
    grid sweep, each grid timed over 10 launches."""
    nb = 2 << 30
    bufs = [torch.ones(nb, dtype=torch.uint8, device="cuda") for _ in range(2)]
    sink = torch.zeros(1024, dtype=torch.uint8, device="cuda")
    best = (0.0, 0, 0)
    sweep = {}
    for pattern in (0, 1):
        for grid in (128, 192, 256, 320, 384, 448, 512, 768, 1024, 2048, 4096, 8192, 16384):
            us = _timed(torch, lambda i: swr.read_ceiling(bufs[i], sink, grid, pattern), 10, 2)
            gbs = nb / (us * 1e-6) / 1e9
            sweep[f"{('sweep', 'span')[pattern]}_{grid}"] = round(gbs, 1)
            best = max(best, (gbs, grid, pattern))
    del bufs
    torch.cuda.empty_cache()
    # One-shot reads of the sizes of the chunked calls' K/V: what the chip
    # gives a job that is one burst, not a stream.  12 rotating buffers
    # (more than the last-level cache), four launches each, captured in one
    # HIP graph: launched from the host one by one, these short reads would
    # be timed at the rate the host issues them.
    one_shot = {}
    for label, nbytes, grids in (("sliding_verify_b8_kv_64MiB", 64 << 20, (256, 512)),
                                 ("global_verify_6005_kv_24.6MB", KC * GHKV * GD * 2 * 2, (94, 188, 256))):
        bufs = [torch.ones(nbytes, dtype=torch.uint8, device="cuda") for _ in range(12)]
        for grid in grids:
            for pattern in (0, 1):
                us = _graph_timed(torch, lambda i: swr.read_ceiling(bufs[i % len(bufs)], sink, grid, pattern),
                                  4 * len(bufs), 4)
                one_shot[f"{label}_{('sweep', 'span')[pattern]}_{grid}"] = {
                    "us": round(us, 2), "GB/s": round(nbytes / (us * 1e-6) / 1e9, 1)}
        del bufs
        torch.cuda.empty_cache()
    return {"GB/s": round(best[0], 1), "bytes_per_launch": nb, "grid": best[1],
            "pattern": ("grid-wide sweep", "contiguous span per workgroup")[best[2]],
            "kernel": "read_ceiling_kernel (swr_read_ceiling), 256 threads, 16-byte non-temporal loads",
            "GB/s_by_pattern_and_grid": sweep, "one_shot_reads": one_shot}


def decode_stack(swr, torch, randn, dev):
    """One decode step's attention through a Gemma-4-31B-shaped stack: 50
    sliding layers and 10 global layers ("Improving Decode Throughput on
    Intel Gaudi 3", Patching sliding window KV allocation), five sliding to
    one global, at B=56 with contexts U[1024, 4096].  Every layer appends its
    token and attends (swr_swa_append_decode, swr_global_append_attend with
    S=1) over rings and regions of its own, 30 GB in all, so nothing is read
    from the caches; all of them are carved from one pool by the library
    (swr_pool_alloc_ring / swr_pool_alloc_global, layer by layer, request by
    request), as a server holds them.  The 60 calls are one HIP graph, timed
    over 5 replays."""
    gen = torch.Generator(device=dev)
    gen.manual_seed(1006)
    pos = torch.randint(1024, 4097, (B,), device=dev, dtype=torch.int32, generator=gen)
    ctx = [int(c) for c in pos.tolist()]
    caps = [(c + 1 + 63) // 64 * 64 for c in ctx]
    # one random source for every layer's history (the layers differ in where they live)
    hk, hv = randn(B, W, HKV, D), randn(B, W, HKV, D)
    gkh, gvh = randn(B, max(ctx) + 1, GHKV, GD), randn(B, max(ctx) + 1, GHKV, GD)
    rb = swr.region_bytes(W, HKV, D)
    grb = [swr.region_bytes(c, GHKV, GD) for c in caps]
    pool = swr.Pool(50 * B * 2 * rb + 10 * 2 * sum(grb) + (64 << 20))
    sliding, glob = [], []
    for _ in range(50):
        ko, vo = [], []
        for _b in range(B):
            k_off, v_off, _cap = pool.alloc_ring(W, HKV, D)
            ko.append(k_off)
            vo.append(v_off)
        L = swr.KVLayer(pool.buffer, pool.buffer, torch.tensor(ko, device=dev), torch.tensor(vo, device=dev), W)
        swr.ring_kv_append(L, hk, hv, (pos - W).to(torch.int32))
        sliding.append(L)
    for _ in range(10):
        ko, vo, cb = [], [], []
        for c in ctx:
            k_off, v_off, cap = pool.alloc_global(c + 1, GHKV, GD)
            ko.append(k_off)
            vo.append(v_off)
            cb.append(cap)
        assert cb == caps
        L = swr.KVLayer(pool.buffer, pool.buffer, torch.tensor(ko, device=dev), torch.tensor(vo, device=dev),
                        max(caps), cap_b=torch.tensor(caps, device=dev, dtype=torch.int32))
        swr.ring_kv_append(L, gkh, gvh, torch.zeros(B, device=dev, dtype=torch.int32), n_new=pos, wrap=False)
        glob.append(L)
    q_s, q_g = randn(B, HKV * G, D), randn(B, 1, GHKV * GG, GD)
    kn_s, vn_s = randn(B, HKV, D), randn(B, HKV, D)
    kn_g, vn_g = randn(B, 1, GHKV, GD), randn(B, 1, GHKV, GD)
    out_s, out_g = torch.empty_like(q_s), torch.empty_like(q_g)
    dws = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_SWA_APPEND_DECODE, B, 1, HKV * G, HKV, D, W)),
                      dtype=torch.uint8, device=dev)
    gws = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_GLOBAL_APPEND_ATTEND, B, 1, GHKV * GG, GHKV, GD,
                                                  max(ctx) + 1)), dtype=torch.uint8, device=dev)

    def step():
        for i in range(10):
            for j in range(5):
                swr.swa_append_decode(sliding[5 * i + j], kn_s, vn_s, q_s, pos, D ** -0.5, out=out_s, ws=dws)
            swr.global_append_attend(glob[i], kn_g, vn_g, q_g, pos, max(ctx) + 1, GD ** -0.5, out=out_g, ws=gws)

    step()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    graph.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 5
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / reps * 1e3
    n_win = sum(min(c + 1, W) for c in ctx)
    sliding_bytes = n_win * HKV * D * 2 * 2 + 2 * B * HKV * G * D * 2 + B * HKV * D * 2 * 2 * 2
    global_bytes = sum(c + 1 for c in ctx) * GHKV * GD * 2 * 2 + 2 * B * GHKV * GG * GD * 2 + \
        B * GHKV * GD * 2 * 2 * 2
    nbytes = 50 * sliding_bytes + 10 * global_bytes
    del sliding, glob, pool, hk, hv, gkh, gvh
    torch.cuda.empty_cache()
    return {"us": round(us, 1), "GB/s": round(nbytes / us / 1e3, 1), "algorithmic_bytes": nbytes,
            "layers": "50 sliding (W=1024, 8 KV heads x 256) + 10 global (2 KV heads x 512), five sliding to one global",
            "batch": B, "contexts": "U[1024, 4096], seed 1006",
            "note": "one HIP graph of the 60 fused append + attention calls; every layer on K/V of its own, "
                    "carved from one pool"}


def global_verify_fp8(swr, torch, randn, dev, n_layers=48):
    """The 6005-key global verify layer over fp8 e4m3 regions: 48 layers of
    12.3 MB (590 MB, more than twice the last-level cache), each captured in
    one HIP graph as the bf16 layers are; the attention call alone and the
    call that appends its 4 proposals first (bf16 tokens in, codes stored)."""
    fp8 = swr.SWR_KV_FP8_E4M3
    sc = 4.5 / 448
    pool = swr.Pool(n_layers * 2 * swr.region_bytes(6016, GHKV, GD, fp8) + (1 << 20))
    layers = []
    for _ in range(n_layers):
        k_off, v_off, cap = pool.alloc_global(KC, GHKV, GD, fp8)
        L = swr.KVLayer(pool.buffer, pool.buffer, torch.tensor([k_off], device=dev), torch.tensor([v_off], device=dev),
                        cap, fp8, sc, sc)
        ctx = KC - GS
        swr.ring_kv_append(L, randn(1, ctx, GHKV, GD), randn(1, ctx, GHKV, GD),
                           torch.zeros(1, device=dev, dtype=torch.int32), wrap=False)
        q = randn(1, GS, GHKV * GG, GD)
        layers.append(dict(L=L, ctx=torch.tensor([ctx], device=dev, dtype=torch.int32),
                           q_pos=torch.arange(ctx, KC, device=dev, dtype=torch.int32).view(1, GS),
                           kc=torch.tensor([KC], device=dev, dtype=torch.int32), k_prop=randn(1, GS, GHKV, GD),
                           v_prop=randn(1, GS, GHKV, GD), q=q, out=torch.empty_like(q)))
    ws = torch.zeros(max(swr.workspace_bytes(swr.SWR_OP_GLOBAL_ATTEND, 1, GS, GHKV * GG, GHKV, GD, KC),
                         swr.workspace_bytes(swr.SWR_OP_GLOBAL_APPEND_ATTEND, 1, GS, GHKV * GG, GHKV, GD, KC), 16),
                     dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def graph_us(layer_fn):
        return _graph_timed(torch, lambda i: layer_fn(layers[i]), len(layers), 10)

    us_attn = graph_us(lambda g: swr.global_attend(g["L"], g["q"], g["q_pos"], g["kc"], KC, GHKV, GD ** -0.5,
                                                   out=g["out"], ws=ws))
    us_fused = graph_us(lambda g: swr.global_append_attend(g["L"], g["k_prop"], g["v_prop"], g["q"], g["ctx"], KC,
                                                           GD ** -0.5, out=g["out"], ws=ws))
    attn_bytes = KC * GHKV * GD * 2 + 2 * GS * GHKV * GG * GD * 2
    fused_bytes = attn_bytes + GS * GHKV * GD * (2 + 1) * 2
    del layers, pool
    torch.cuda.empty_cache()
    return ({"us": round(us_attn, 2), "GB/s": round(attn_bytes / us_attn / 1e3, 1), "algorithmic_bytes": attn_bytes,
             "layers_in_graph": n_layers},
            {"us": round(us_fused, 2), "GB/s": round(fused_bytes / us_fused / 1e3, 1), "algorithmic_bytes": fused_bytes,
             "layers_in_graph": n_layers})


def other_workloads(swr, torch, sweep=True):
    """The remaining workloads, each timed on its own (us per call, GB/s of
    algorithmic bytes): sliding verify B=8, fp8 sliding decode B=56, the B=56
    decode over a paged cache (gather, then the decode), the mixed 16-request
    step (bf16 and fp8, rings and global regions in one pool), and the global
    verify over every key count 4000..8192."""
    import synthetic

    dev = torch.device("cuda", 0)
    gen = torch.Generator(device=dev)
    gen.manual_seed(1003)
    res = {}

    def randn(*shape):
        return torch.randn(*shape, device=dev, generator=gen).to(torch.bfloat16)

    # --- sliding verify: B=8, W=1024, S=4 proposals, 32 rows per KV head
    w = synthetic.SWA_VERIFY
    sets = []
    for _ in range(8):
        rb = swr.region_bytes(w.W, w.Hkv, w.D)
        kb = torch.empty(w.B * rb, dtype=torch.uint8, device=dev)
        vb = torch.empty_like(kb)
        off = torch.arange(w.B, device=dev, dtype=torch.int64) * rb
        L = swr.KVLayer(kb, vb, off, off.clone(), w.W)
        p0 = torch.randint(w.pos_lo, w.pos_hi + 1, (w.B,), device=dev, dtype=torch.int32, generator=gen)
        swr.ring_kv_append(L, randn(w.B, w.W, w.Hkv, w.D), randn(w.B, w.W, w.Hkv, w.D), (p0 - w.W).to(torch.int32))
        q = randn(w.B, w.S, w.Hq, w.D)
        sets.append((L, randn(w.B, w.S, w.Hkv, w.D), randn(w.B, w.S, w.Hkv, w.D), q, p0, torch.empty_like(q)))
    ws = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_GQA_VERIFY, w.B, w.S, w.Hq, w.Hkv, w.D, w.W)),
                     dtype=torch.uint8, device=dev)
    us = _timed(torch, lambda i: swr.gqa_verify(sets[i][0], sets[i][1], sets[i][2], sets[i][3], sets[i][4],
                                                w.D ** -0.5, out=sets[i][5], ws=ws), 100, len(sets))
    nbytes = w.B * w.Hkv * (w.W - 1) * w.D * 4 + 2 * w.B * w.S * w.Hkv * w.D * 2 + 2 * w.B * w.S * w.Hq * w.D * 2
    res["sliding_verify_b8"] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                                "algorithmic_bytes": nbytes, "sets": len(sets)}
    del sets

    # --- the same verify over fp8 rings (16 sets of 33.6 MB: twice the last-level cache)
    sets = []
    for _ in range(16):
        rb = swr.region_bytes(w.W, w.Hkv, w.D, swr.SWR_KV_FP8_E4M3)
        kb = torch.empty(w.B * rb, dtype=torch.uint8, device=dev)
        vb = torch.empty_like(kb)
        off = torch.arange(w.B, device=dev, dtype=torch.int64) * rb
        L = swr.KVLayer(kb, vb, off, off.clone(), w.W, swr.SWR_KV_FP8_E4M3, 4.5 / 448, 4.5 / 448)
        p0 = torch.randint(w.pos_lo, w.pos_hi + 1, (w.B,), device=dev, dtype=torch.int32, generator=gen)
        swr.ring_kv_append(L, randn(w.B, w.W, w.Hkv, w.D), randn(w.B, w.W, w.Hkv, w.D), (p0 - w.W).to(torch.int32))
        q = randn(w.B, w.S, w.Hq, w.D)
        sets.append((L, randn(w.B, w.S, w.Hkv, w.D), randn(w.B, w.S, w.Hkv, w.D), q, p0, torch.empty_like(q)))
    us = _timed(torch, lambda i: swr.gqa_verify(sets[i][0], sets[i][1], sets[i][2], sets[i][3], sets[i][4],
                                                w.D ** -0.5, out=sets[i][5], ws=ws), 100, len(sets))
    nbytes = w.B * w.Hkv * (w.W - 1) * w.D * 2 + 2 * w.B * w.S * w.Hkv * w.D * 2 + 2 * w.B * w.S * w.Hq * w.D * 2
    res["sliding_verify_b8_fp8"] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                                    "algorithmic_bytes": nbytes, "sets": len(sets)}
    del sets, ws

    # --- the same verify at B=32 (256 units: the batch fills the chip), bf16 (3 sets of 269 MB)
    # and fp8 (4 sets of 135 MB)
    w = synthetic.Workload("sliding verify B=32", B=32, Hkv=8, G=8, D=256, W=1024, S=4, pos_lo=1024, pos_hi=8192)
    for dt, n_sets, name in ((swr.SWR_KV_BF16, 3, "sliding_verify_b32"), (swr.SWR_KV_FP8_E4M3, 4, "sliding_verify_b32_fp8")):
        fp8 = dt == swr.SWR_KV_FP8_E4M3
        sets = []
        for _ in range(n_sets):
            rb = swr.region_bytes(w.W, w.Hkv, w.D, dt)
            kb = torch.empty(w.B * rb, dtype=torch.uint8, device=dev)
            vb = torch.empty_like(kb)
            off = torch.arange(w.B, device=dev, dtype=torch.int64) * rb
            L = swr.KVLayer(kb, vb, off, off.clone(), w.W, *((dt, 4.5 / 448, 4.5 / 448) if fp8 else ()))
            p0 = torch.randint(w.pos_lo, w.pos_hi + 1, (w.B,), device=dev, dtype=torch.int32, generator=gen)
            swr.ring_kv_append(L, randn(w.B, w.W, w.Hkv, w.D), randn(w.B, w.W, w.Hkv, w.D), (p0 - w.W).to(torch.int32))
            q = randn(w.B, w.S, w.Hq, w.D)
            sets.append((L, randn(w.B, w.S, w.Hkv, w.D), randn(w.B, w.S, w.Hkv, w.D), q, p0, torch.empty_like(q)))
        ws = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_GQA_VERIFY, w.B, w.S, w.Hq, w.Hkv, w.D, w.W)),
                         dtype=torch.uint8, device=dev)
        us = _timed(torch, lambda i: swr.gqa_verify(sets[i][0], sets[i][1], sets[i][2], sets[i][3], sets[i][4],
                                                    w.D ** -0.5, out=sets[i][5], ws=ws), 40, len(sets))
        nbytes = w.B * w.Hkv * (w.W - 1) * w.D * 2 * (1 if fp8 else 2) + 2 * w.B * w.S * w.Hkv * w.D * 2 + \
            2 * w.B * w.S * w.Hq * w.D * 2
        res[name] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1), "algorithmic_bytes": nbytes,
                     "sets": len(sets)}
        del sets, ws

    # --- one GPU's share of the B=56 decode under KV-head sharding (8 GPUs, one KV head each):
    # 10 sets of 58.7 MB, more than twice the 256 MB last-level cache
    w = synthetic.SWA_DECODE
    sets = []
    for _ in range(10):
        rb = swr.region_bytes(w.W, 1, w.D)
        kb = torch.empty(w.B * rb, dtype=torch.uint8, device=dev)
        vb = torch.empty_like(kb)
        off = torch.arange(w.B, device=dev, dtype=torch.int64) * rb
        L = swr.KVLayer(kb, vb, off, off.clone(), w.W)
        pos = torch.randint(w.pos_lo, w.pos_hi + 1, (w.B,), device=dev, dtype=torch.int32, generator=gen)
        swr.ring_kv_append(L, randn(w.B, w.W, 1, w.D), randn(w.B, w.W, 1, w.D), (pos - w.W + 1).to(torch.int32))
        q = randn(w.B, w.G, w.D)
        sets.append((L, q, pos, torch.empty_like(q)))
    hws = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_SWA_DECODE, w.B, 1, w.G, 1, w.D, w.W)),
                      dtype=torch.uint8, device=dev)
    us = _timed(torch, lambda i: swr.swa_decode(sets[i][0], sets[i][1], sets[i][2], 1, w.D ** -0.5, out=sets[i][3],
                                                ws=hws), 60, len(sets))
    nbytes = w.B * w.W * w.D * 4 + 2 * w.B * w.G * w.D * 2
    res["sliding_decode_b56_one_kv_head_share"] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                                                   "algorithmic_bytes": nbytes, "sets": len(sets)}
    del sets, hws

    # --- fp8 sliding decode, B=56
    w = synthetic.SWA_DECODE
    sets = []
    for _ in range(3):
        rb = swr.region_bytes(w.W, w.Hkv, w.D, swr.SWR_KV_FP8_E4M3)
        kb = torch.empty(w.B * rb, dtype=torch.uint8, device=dev)
        vb = torch.empty_like(kb)
        off = torch.arange(w.B, device=dev, dtype=torch.int64) * rb
        L = swr.KVLayer(kb, vb, off, off.clone(), w.W, swr.SWR_KV_FP8_E4M3, 4.5 / 448, 4.5 / 448)
        pos = torch.randint(w.pos_lo, w.pos_hi + 1, (w.B,), device=dev, dtype=torch.int32, generator=gen)
        for half in range(2):
            swr.ring_kv_append(L, randn(w.B, w.W // 2, w.Hkv, w.D), randn(w.B, w.W // 2, w.Hkv, w.D),
                          (pos - w.W + 1 + half * (w.W // 2)).to(torch.int32))
        q = randn(w.B, w.Hq, w.D)
        sets.append((L, q, pos, torch.empty_like(q), randn(w.B, w.Hkv, w.D), randn(w.B, w.Hkv, w.D)))
    us = _timed(torch, lambda i: swr.swa_decode(sets[i][0], sets[i][1], sets[i][2], w.Hkv, w.D ** -0.5,
                                                out=sets[i][3]), 60, len(sets))
    nbytes = w.B * w.Hkv * w.W * w.D * 2 + 2 * w.B * w.Hq * w.D * 2
    res["sliding_decode_b56_fp8"] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                                     "algorithmic_bytes": nbytes}
    # the same layer with its append (bf16 tokens in, fp8 codes stored)
    us = _timed(torch, lambda i: swr.swa_append_decode(sets[i][0], sets[i][4], sets[i][5], sets[i][1], sets[i][2],
                                                       w.D ** -0.5, out=sets[i][3]), 60, len(sets))
    nbytes += w.B * w.Hkv * w.D * (2 + 1) * 2
    res["sliding_decode_b56_fp8_append_and_attention"] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                                                          "algorithmic_bytes": nbytes}
    del sets

    # --- the paged-cache baseline of the same B=56 decode: each request's
    # window in 16-token pages scattered over a page pool, gathered into a
    # ring-layout workspace every step, then the same decode kernel
    res["sliding_decode_b56_paged_gather_baseline"] = paged_baseline(swr, torch, randn, gen, dev)

    # --- the global verify layer over fp8 regions, in a layer graph
    res["global_verify_6005_fp8_attention_only_in_graph"], res["global_verify_6005_fp8_in_layer_graph"] = \
        global_verify_fp8(swr, torch, randn, dev)

    # --- mixed step: 16 requests, contexts log-uniform [512, 65536], one pool
    ctx = [int(c) for c in synthetic.mixed_contexts()]
    B = len(ctx)
    ws_s, ws_g = synthetic.MIXED_SLIDING, synthetic.MIXED_GLOBAL
    for dtype, name in ((swr.SWR_KV_BF16, "mixed_step_bf16"), (swr.SWR_KV_FP8_E4M3, "mixed_step_fp8")):
        esz = 2 if dtype == swr.SWR_KV_BF16 else 1
        rb_s = swr.region_bytes(ws_s.W, ws_s.Hkv, ws_s.D, dtype)
        caps = [(c + 1 + 63) // 64 * 64 for c in ctx]
        total = 2 * B * rb_s + 2 * sum(swr.region_bytes(c, ws_g.Hkv, ws_g.D, dtype) for c in caps) + (1 << 24)
        pool = swr.Pool(total)
        rk, rv, gk, gv, gc = [], [], [], [], []
        for c in ctx:
            k_off, v_off, _ = pool.alloc_ring(ws_s.W, ws_s.Hkv, ws_s.D, dtype)
            rk.append(k_off)
            rv.append(v_off)
            k_off, v_off, cap = pool.alloc_global(c + 1, ws_g.Hkv, ws_g.D, dtype)
            gk.append(k_off)
            gv.append(v_off)
            gc.append(cap)
        sc = 4.5 / 448 if dtype else 1.0
        sl = swr.KVLayer(pool.buffer, pool.buffer, torch.tensor(rk, device=dev), torch.tensor(rv, device=dev), ws_s.W,
                         dtype, sc, sc)
        gl = swr.KVLayer(pool.buffer, pool.buffer, torch.tensor(gk, device=dev), torch.tensor(gv, device=dev),
                         max(gc), dtype, sc, sc, cap_b=torch.tensor(gc, device=dev, dtype=torch.int32))
        pos = torch.tensor(ctx, device=dev, dtype=torch.int32)
        n_ring = min(ws_s.W, min(ctx) + 1)
        for b, c in enumerate(ctx):
            one = torch.tensor([b], device=dev)
            n = min(c + 1, ws_s.W)
            ring = swr.KVLayer(pool.buffer, pool.buffer, sl.k_off[one], sl.v_off[one], ws_s.W, dtype, sc, sc)
            swr.ring_kv_append(ring, randn(1, n, ws_s.Hkv, ws_s.D), randn(1, n, ws_s.Hkv, ws_s.D),
                          torch.tensor([c - n + 1], device=dev, dtype=torch.int32))
            glob1 = swr.KVLayer(pool.buffer, pool.buffer, gl.k_off[one], gl.v_off[one], gc[b], dtype, sc, sc)
            for s0 in range(0, c + 1, 8192):
                n2 = min(8192, c + 1 - s0)
                swr.ring_kv_append(glob1, randn(1, n2, ws_g.Hkv, ws_g.D), randn(1, n2, ws_g.Hkv, ws_g.D),
                              torch.tensor([s0], device=dev, dtype=torch.int32), wrap=False)
        qs = randn(B, ws_s.Hq, ws_s.D)
        qg = randn(B, 1, ws_g.Hq, ws_g.D)
        kc = pos + 1
        dws = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_SWA_DECODE, B, 1, ws_s.Hq, ws_s.Hkv, ws_s.D,
                                                      ws_s.W)), dtype=torch.uint8, device=dev)
        gws = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_GLOBAL_ATTEND, B, 1, ws_g.Hq, ws_g.Hkv, ws_g.D,
                                                      max(ctx) + 1)), dtype=torch.uint8, device=dev)
        outs, outg = torch.empty_like(qs), torch.empty_like(qg)
        torch.cuda.synchronize()

        def mixed(_i):
            swr.swa_decode(sl, qs, pos, ws_s.Hkv, ws_s.D ** -0.5, out=outs, ws=dws)
            swr.global_attend(gl, qg, pos.view(B, 1), kc, max(ctx) + 1, ws_g.Hkv, ws_g.D ** -0.5, out=outg, ws=gws)

        us = _timed(torch, mixed, 30, 1)
        nbytes = sum(min(c + 1, ws_s.W) for c in ctx) * ws_s.Hkv * ws_s.D * esz * 2 + \
            sum(c + 1 for c in ctx) * ws_g.Hkv * ws_g.D * esz * 2 + \
            2 * B * (ws_s.Hq * ws_s.D + ws_g.Hq * ws_g.D) * 2
        res[name] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1), "algorithmic_bytes": nbytes,
                     "contexts": ctx}

        # the same step with each layer appending its token first (the token
        # at position ctx, already in the regions above, is written again)
        kn_s, vn_s = randn(B, ws_s.Hkv, ws_s.D), randn(B, ws_s.Hkv, ws_s.D)
        kn_g, vn_g = randn(B, 1, ws_g.Hkv, ws_g.D), randn(B, 1, ws_g.Hkv, ws_g.D)
        fws = torch.zeros(max(16, swr.workspace_bytes(swr.SWR_OP_GLOBAL_APPEND_ATTEND, B, 1, ws_g.Hq, ws_g.Hkv,
                                                      ws_g.D, max(ctx) + 1)), dtype=torch.uint8, device=dev)

        def mixed_fused(_i):
            swr.swa_append_decode(sl, kn_s, vn_s, qs, pos, ws_s.D ** -0.5, out=outs, ws=dws)
            swr.global_append_attend(gl, kn_g, vn_g, qg, pos, max(ctx) + 1, ws_g.D ** -0.5, out=outg, ws=fws)

        us = _timed(torch, mixed_fused, 30, 1)
        nbytes += B * (ws_s.Hkv * ws_s.D + ws_g.Hkv * ws_g.D) * (2 + esz) * 2
        res[name + "_append_and_attention"] = {"us": round(us, 2), "GB/s": round(nbytes / us / 1e3, 1),
                                               "algorithmic_bytes": nbytes}
        del pool, sl, gl, dws, gws, fws
        torch.cuda.synchronize()

    res["decode_step_b56_gemma4_31b_attention_stack"] = decode_stack(swr, torch, randn, dev)

    if not sweep:
        return res
    # --- global verify over every key count 4000..8192 (one region of 8192 slots)
    lo, hi = synthetic.GLOBAL_SWEEP
    cap = 8192
    rb = swr.region_bytes(cap, GHKV, GD)
    kb = torch.zeros(rb, dtype=torch.uint8, device=dev)
    vb = torch.zeros_like(kb)
    off = torch.zeros(1, device=dev, dtype=torch.int64)
    L = swr.KVLayer(kb, vb, off, off.clone(), cap)
    swr.ring_kv_append(L, randn(1, hi, GHKV, GD), randn(1, hi, GHKV, GD), torch.zeros(1, device=dev, dtype=torch.int32),
                  wrap=False)
    counts = torch.arange(lo, hi + 1, device=dev, dtype=torch.int32)
    qpos = (counts.view(-1, 1) - GS + torch.arange(GS, device=dev, dtype=torch.int32).view(1, -1)).contiguous()
    q = randn(1, GS, GHKV * GG, GD)
    out = torch.empty_like(q)
    ws = torch.zeros(swr.workspace_bytes(swr.SWR_OP_GLOBAL_ATTEND, 1, GS, GHKV * GG, GHKV, GD, hi), dtype=torch.uint8,
                     device=dev)
    n = counts.numel()
    # three launches back to back per key count, each between its own events;
    # the fastest of the three is the count's time (a single eager launch can
    # include a wait for the host to issue it)
    rep3 = 3
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n * rep3 + 1)]
    for i in range(3):
        swr.global_attend(L, q, qpos[i:i + 1], counts[i:i + 1], hi, GHKV, GD ** -0.5, out=out, ws=ws)
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n):
        for r in range(rep3):
            swr.global_attend(L, q, qpos[i:i + 1], counts[i:i + 1], lo + i, GHKV, GD ** -0.5, out=out, ws=ws)
            ev[i * rep3 + r + 1].record()
    torch.cuda.synchronize()
    t = [min(ev[i * rep3 + r].elapsed_time(ev[i * rep3 + r + 1]) for r in range(rep3)) * 1e3 for i in range(n)]
    ts = sorted(t)
    at64 = [t[i] for i in range(n) if (lo + i) % 64 == 0]
    off64 = [t[i] for i in range(n) if (lo + i) % 64 != 0]
    res["global_verify_sweep_4000_8192"] = {
        "counts": n, "us_min": round(ts[0], 2), "us_median": round(ts[n // 2], 2), "us_p99": round(ts[int(n * 0.99)], 2),
        "us_max": round(ts[-1], 2), "us_mean_at_multiples_of_64": round(sum(at64) / len(at64), 2),
        "us_mean_elsewhere": round(sum(off64) / len(off64), 2),
        "note": "one region reused (warm in cache), eager launches, fastest of 3 per count: shows the shape is flat "
                "in the key count"}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true", help="skip the other workloads")
    ap.add_argument("--no-sweep", action="store_true", help="skip the global key-count sweep of the other workloads")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy 5 times (reference for the HBM byte counters)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library has no multi-GPU path (asked for --gpus {args.gpus}).",
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
    gws = torch.zeros(max(swr.workspace_bytes(swr.SWR_OP_GLOBAL_ATTEND, 1, GS, GHKV * GG, GHKV, GD, KC),
                          swr.workspace_bytes(swr.SWR_OP_GLOBAL_APPEND_ATTEND, 1, GS, GHKV * GG, GHKV, GD, KC), 16),
                      dtype=torch.uint8, device="cuda")
    dws = torch.zeros(max(swr.workspace_bytes(swr.SWR_OP_SWA_APPEND_DECODE, B, 1, HKV * G, HKV, D, W), 16),
                      dtype=torch.uint8, device="cuda")
    scale_s, scale_g = D ** -0.5, GD ** -0.5

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]

    def sliding_layer(s):  # append the token at pos into the ring, then decode
        swr.swa_append_decode(s["L"], s["k_new"], s["v_new"], s["q"], s["pos"], scale_s, out=s["out"], ws=dws)

    def global_layer(g):  # append the 4 proposals at ctx .. ctx+3, then the grouped verify
        swr.global_append_attend(g["L"], g["k_prop"], g["v_prop"], g["q"], g["ctx"], KC, scale_g, out=g["out"],
                                 ws=gws)

    def global_separate(g):
        swr.ring_kv_append(g["L"], g["k_prop"], g["v_prop"], g["ctx"], wrap=False)
        swr.global_attend(g["L"], g["q"], g["q_pos"], g["kc"], KC, GHKV, scale_g, out=g["out"], ws=gws)

    def step(i, events=None):
        s = sliding[i % N_SLIDING_SETS]
        g = glob[i % N_GLOBAL_SETS]
        if events:
            events[0].record()
        sliding_layer(s)
        if events:
            events[1].record()
        global_layer(g)
        if events:
            events[2].record()

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t_start.record()
    for i in range(args.steps):
        step(i)
    t_end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step = t_start.elapsed_time(t_end) / args.steps

    # Per-layer times within the step: the same K steps again with events
    # between the launches (each event adds a few microseconds of its own,
    # which is why the timed steps above carry none).
    for i in range(args.steps):
        step(i, ev[i])
    torch.cuda.synchronize()
    sliding_us = sum(e[0].elapsed_time(e[1]) for e in ev) / args.steps * 1e3
    global_us = sum(e[1].elapsed_time(e[2]) for e in ev) / args.steps * 1e3
    # The roofline kernel (the fused sliding layer) alone: launches back to
    # back over the 3 layer sets, events around the loop.
    sliding_b2b_us = _timed(torch, lambda i: sliding_layer(sliding[i]), 60, N_SLIDING_SETS)

    # The separate calls, each timed over the same layer sets: the decode
    # without its append, back to back, and the append alone, a launch of a
    # few microseconds, from a captured graph.
    decode_only_us = _timed(torch, lambda i: swr.swa_decode(sliding[i]["L"], sliding[i]["q"], sliding[i]["pos"], HKV,
                                                            scale_s, out=sliding[i]["out"], ws=dws),
                            30, N_SLIDING_SETS)
    def append_only(i):
        s = sliding[i % N_SLIDING_SETS]
        swr.ring_kv_append(s["L"], s["k_new"], s["v_new"], s["pos"])

    append_only_us = _graph_timed(torch, append_only, 8 * N_SLIDING_SETS, 10)

    # The global layer's launches are short: also time them the way a serving
    # loop issues them, captured in one HIP graph holding all 24 global layers
    # -- the fused call, the separate append + attention, and the attention
    # call alone.
    def graph_us(layer_fn):
        return _graph_timed(torch, lambda i: layer_fn(glob[i]), N_GLOBAL_SETS, 10)

    global_graph_us = graph_us(global_layer)
    global_sep_graph_us = graph_us(global_separate)
    global_attn_graph_us = graph_us(lambda g: swr.global_attend(g["L"], g["q"], g["q_pos"], g["kc"], KC, GHKV,
                                                                scale_g, out=g["out"], ws=gws))
    b_dec, b_app_s, b_glob, b_app_g = algorithmic_bytes()
    step_bytes = b_dec + b_app_s + b_glob + b_app_g
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    achieved = (b_dec + b_app_s) / (sliding_b2b_us * 1e-6) / 1e9
    glob_achieved = (b_glob + b_app_g) / (global_graph_us * 1e-6) / 1e9
    traffic = measured_traffic("decode")
    ceiling = read_ceiling(swr, torch)

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
        "hbm_read_ceiling": ceiling,
        "read_ceiling_frac": round(value / ceiling["GB/s"], 4),
        "us_per_layer": {
            "sliding_decode_b56_append_and_attention": round(sliding_b2b_us, 2),
            "sliding_decode_b56_append_and_attention_events_in_step": round(sliding_us, 2),
            "sliding_decode_b56_attention_only": round(decode_only_us, 2),
            "sliding_decode_b56_separate_append": round(append_only_us, 2),
            "global_verify_6005_append_and_attention_events_in_step": round(global_us, 2),
            "global_verify_6005_in_layer_graph": round(global_graph_us, 2),
            "global_verify_6005_separate_append_and_attention_in_graph": round(global_sep_graph_us, 2),
            "global_verify_6005_attention_only_in_graph": round(global_attn_graph_us, 2),
        },
        "layer_gbs": {
            "sliding_decode_b56_append_and_attention": round(achieved, 1),
            "sliding_decode_b56_attention_only": round(b_dec / (decode_only_us * 1e-6) / 1e9, 1),
            "global_verify_6005_events_in_step": round((b_glob + b_app_g) / (global_us * 1e-6) / 1e9, 1),
            "global_verify_6005_in_layer_graph": round((b_glob + b_app_g) / (global_graph_us * 1e-6) / 1e9, 1),
        },
        "roofline": {
            "kernel": "attn_kernel<256,256,1,4,bf16,decode+append> (swr_swa_append_decode, B=56)",
            "bound": "hbm",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "traffic": traffic,
            "algorithmic_bytes_per_launch": b_dec + b_app_s,
            "frac_of_read_ceiling": round(achieved / ceiling["GB/s"], 4),
        },
        # the other target: the global verify layer (chunk pass + merge, with
        # its append), its own algorithmic bytes over its time per layer in a
        # 24-layer graph
        "roofline_global_verify": {
            "kernel": "chunk_kernel<512,2,bf16,global> + merge_grouped<512> (swr_global_append_attend, 6005 keys, "
                      "per layer of a 24-layer graph)",
            "bound": "hbm",
            "achieved": round(glob_achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(glob_achieved / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("global"),
            "algorithmic_bytes_per_launch": b_glob + b_app_g,
            "us_per_layer": round(global_graph_us, 2),
            "floor_us": round((b_glob + b_app_g) / HBM_PEAK_GBS / 1e3, 2),
        },
        "host_wall_s": round(wall, 3),
    }
    if not args.no_extra:
        result["other_workloads"] = ow = other_workloads(swr, torch, sweep=not args.no_sweep)
        v = ow["sliding_verify_b8"]
        result["roofline_sliding_verify"] = {
            "kernel": "chunk_kernel<256,2,bf16,verify> + merge_flat (swr_gqa_verify, B=8, W=1024, S=4)",
            "bound": "hbm",
            "achieved": v["GB/s"],
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(v["GB/s"] / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("verify"),
            "algorithmic_bytes_per_launch": v["algorithmic_bytes"],
            "us_per_layer": v["us"],
            "floor_us": round(v["algorithmic_bytes"] / HBM_PEAK_GBS / 1e3, 2),
        }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cb = cpu_baseline()
        pc = cb["per_config"]
        pc["sliding_decode_b56"]["gpu_us_per_layer"] = round(decode_only_us, 2)
        pc["global_verify_6005"]["gpu_us_per_layer"] = round(global_attn_graph_us, 2)
        if not args.no_extra:
            ow = result["other_workloads"]
            pc["sliding_verify_b8"]["gpu_us_per_layer"] = ow["sliding_verify_b8"]["us"]
            pc["mixed_step_bf16"]["gpu_us_per_layer"] = ow["mixed_step_bf16"]["us"]
            pc["mixed_step_fp8"]["gpu_us_per_layer"] = ow["mixed_step_fp8"]["us"]
    print(json.dumps(result))


if __name__ == "__main__":
    main()
