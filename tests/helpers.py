"""Shared test helpers: host-side pools built with the oracle, a library
attention routine (torch SDPA on the CPU in float64) used to pin the oracle,
and the error metrics of the parity bar."""
from __future__ import annotations

import json
import os

import numpy as np
import torch

import oracle

# Parity bar for bf16 attention outputs against the float64 oracle: relative
# L2 error over the whole output <= 5e-3, and per element |got - ref| <=
# max(1e-2, one bf16 ulp of |ref|).  The element bound is the 1e-2 max-abs
# bar wherever bf16 can meet it; an output of magnitude >= 2 (a row that sees
# one to a few keys returns about a value itself) is spaced 2^-6 or more in
# bf16, so rounding the softmax weights and the output to bf16 (up to 2^-8
# relative each; the weight of a row's largest score, 1, is exact) can pass
# 1e-2 alone -- there the bound is one ulp of the output's binade, the size
# of those two roundings together.
MAX_ABS_TOL = 1e-2
REL_L2_TOL = 5e-3


def bf16_ulp(x):
    """Spacing of bf16 numbers at |x| (8 significant bits); 2^-133 at 0."""
    a = np.abs(np.asarray(x, np.float64))
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -126)))
    return np.exp2(e - 7)


def errors(got, ref):
    """(max-abs error, relative L2 error) of got against ref, in float64."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    diff = got - ref
    max_abs = float(np.max(np.abs(diff))) if diff.size else 0.0
    den = float(np.linalg.norm(ref.ravel()))
    rel = float(np.linalg.norm(diff.ravel())) / den if den > 0 else float(np.linalg.norm(diff))
    return max_abs, rel


def assert_parity(got, ref, what=""):
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    max_abs, rel = errors(got, ref)
    bound = np.maximum(MAX_ABS_TOL, bf16_ulp(ref))
    over = np.abs(got - ref) > bound
    log = os.environ.get("SWR_PARITY_LOG")
    if log:  # headroom of each check: worst element error / its bound, rel-L2 / its bound
        elem = float(np.max(np.abs(got - ref) / bound)) if got.size else 0.0
        with open(log, "a") as f:
            f.write(json.dumps({"test": os.environ.get("PYTEST_CURRENT_TEST", "").split(" ")[0], "what": what,
                                "n": int(got.size), "max_abs": max_abs, "rel_l2": rel,
                                "elem_frac": elem, "rel_frac": rel / REL_L2_TOL}) + "\n")
    assert not over.any() and rel <= REL_L2_TOL, (
        f"{what}: {int(over.sum())} elements past max(1e-2, 1 bf16 ulp) (max-abs {max_abs:.3e}), "
        f"rel-L2 {rel:.3e} (tol {REL_L2_TOL})")
    return max_abs, rel


def ring_pools(hist_k, hist_v, start, n, W, dtype=oracle.BF16, k_scale=1.0, v_scale=1.0):
    """One ring of W slots per request, filled by the oracle's append of each
    request's window tokens (hist_* [B][W][Hkv][D] in position order, the first
    n[b] valid, starting at position start[b]).  Returns k_pool, v_pool,
    k_off, v_off (host uint8 pools and byte offsets)."""
    B, _, hkv, d = hist_k.shape
    rb = oracle.region_bytes(W, hkv, d, dtype)
    k_pool = np.zeros(B * rb, np.uint8)
    v_pool = np.zeros(B * rb, np.uint8)
    off = np.arange(B, dtype=np.int64) * rb
    oracle.kv_append(k_pool, v_pool, off, off, W, dtype, k_scale, v_scale, hist_k, hist_v, start, n,
                     wrap=True)
    return k_pool, v_pool, off, off.copy()


def global_pools(k, v, key_count, cap, dtype=oracle.BF16, k_scale=1.0, v_scale=1.0):
    """One contiguous region of `cap` slots per request holding keys
    0..key_count[b]-1 (the rest zero), written by the oracle's append."""
    B, _, hkv, d = k.shape
    rb = oracle.region_bytes(cap, hkv, d, dtype)
    k_pool = np.zeros(B * rb, np.uint8)
    v_pool = np.zeros(B * rb, np.uint8)
    off = np.arange(B, dtype=np.int64) * rb
    oracle.kv_append(k_pool, v_pool, off, off, cap, dtype, k_scale, v_scale, k, v,
                     np.zeros(B, np.int32), np.asarray(key_count, np.int32), wrap=False)
    return k_pool, v_pool, off, off.copy()


def f64(bits):
    """bf16 bits to float64 via torch (a library conversion, independent of
    the oracle's own widening)."""
    t = torch.from_numpy(np.ascontiguousarray(bits, np.uint16).view(np.int16))
    return t.view(torch.bfloat16).to(torch.float64).numpy()


def sdpa(q, k, v, mask, scale):
    """torch scaled_dot_product_attention on the CPU in float64.
    q [R][D], k/v [N][D], mask [R][N] bool (True = visible)."""
    qt = torch.as_tensor(q, dtype=torch.float64)[None, None]
    kt = torch.as_tensor(k, dtype=torch.float64)[None, None]
    vt = torch.as_tensor(v, dtype=torch.float64)[None, None]
    mt = torch.as_tensor(mask, dtype=torch.bool)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mt, scale=scale)
    return out[0, 0].numpy()
