"""The fused global-layer call without caller workspace
(swr_global_append_attend_noalloc, static device scratch) against the same
call with a workspace (swr_global_append_attend), both through the C ABI.

Two calls in a row share the scratch array; the second is smaller than the
first, so stale partials of the first are in the array when the second runs.
Outputs must meet the parity bar against the workspace call's (they run the
same kernels, so they are compared bit for bit as well), and the region
bytes each call leaves must be identical.
"""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import sliding_window_ring_amd as swr
import synthetic
from gpu_common import dev_bf16, dev_i32, host_bits, host_f64, layer
from helpers import assert_parity, global_pools

pytestmark = pytest.mark.gpu

noalloc = swr.lib.swr_global_append_attend_noalloc  # the C entry point, signature set by the binding


def case(seed, kc, S, G, D, hkv, cap, dtype):
    """Regions holding keys 0 .. kc-S-1 (two device copies), the S new tokens,
    queries and positions."""
    g = synthetic.rng(seed)
    kc = np.asarray(kc, np.int32)
    B = kc.size
    k = synthetic.normal_bf16(g, (B, int(kc.max()), hkv, D))
    v = synthetic.normal_bf16(g, (B, int(kc.max()), hkv, D))
    q = synthetic.normal_bf16(g, (B, S, hkv * G, D))
    pos0 = (kc - S).astype(np.int32)
    ks, vs = (4.6 / 448, 4.4 / 448) if dtype == oracle.FP8 else (1.0, 1.0)
    kp, vp, ko, vo = global_pools(k, v, pos0, cap, dtype, ks, vs)
    kn = np.ascontiguousarray(np.stack([k[b, pos0[b]:kc[b]] for b in range(B)]))
    vn = np.ascontiguousarray(np.stack([v[b, pos0[b]:kc[b]] for b in range(B)]))
    return dict(L1=layer(kp, vp, ko, vo, cap, dtype, ks, vs), L2=layer(kp, vp, ko, vo, cap, dtype, ks, vs),
                kn=dev_bf16(kn), vn=dev_bf16(vn), q=dev_bf16(q), pos0=dev_i32(pos0), mk=int(kc.max()),
                B=B, S=S, Hq=hkv * G, hkv=hkv, D=D)


def run_both(c):
    scale = c["D"] ** -0.5
    out_ws = swr.global_append_attend(c["L1"], c["kn"], c["vn"], c["q"], c["pos0"], c["mk"], scale)
    out_na = torch.empty_like(out_ws)
    st = noalloc(ctypes.byref(c["L2"].c()), ctypes.c_void_p(c["kn"].data_ptr()), ctypes.c_void_p(c["vn"].data_ptr()),
                 ctypes.c_void_p(c["q"].data_ptr()), ctypes.c_void_p(out_na.data_ptr()),
                 ctypes.c_void_p(c["pos0"].data_ptr()), c["mk"], c["B"], c["S"], c["Hq"], c["hkv"], c["D"], scale,
                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, swr.STATUS.get(st, st)
    torch.cuda.synchronize()
    assert_parity(host_f64(out_na), host_f64(out_ws), "no-allocation call against the workspace call")
    assert np.array_equal(host_bits(out_na), host_bits(out_ws))
    assert torch.equal(c["L1"].k_base, c["L2"].k_base) and torch.equal(c["L1"].v_base, c["L2"].v_base)


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_noalloc_matches_workspace_call_twice_second_smaller(dtype):
    # first: the 6005-key verify layer (2 KV heads x 512, 32 rows)
    run_both(case(501, [6005], 4, 8, 512, 2, 6016, dtype))
    # second, smaller: two requests of a few hundred keys, 16 rows
    run_both(case(502, [300, 77], 2, 8, 512, 2, 320, dtype))


@pytest.mark.parametrize("dtype", [oracle.BF16, oracle.FP8], ids=["bf16", "fp8"])
def test_noalloc_streamed_one_token_twice_second_smaller(dtype):
    # streamed calls (the units span >= 2048 tiles of 32 keys) of one token
    # per request, whose split pass takes each token itself; at 64 head dims
    # their partials (at least 512 slots) fit the scratch
    kc1 = [4100, 4500, 4093, 5000, 4200, 4800, 4300, 4097]
    assert len(kc1) * 2 * -(-max(kc1) // 32) >= 2048
    run_both(case(503, kc1, 1, 8, 64, 2, 5056, dtype))
    kc2 = [8300, 8200, 8192, 8257]
    assert len(kc2) * 2 * -(-max(kc2) // 32) >= 2048
    run_both(case(504, kc2, 1, 8, 64, 2, 8320, dtype))


def test_noalloc_rejects_a_call_past_the_scratch():
    # 16 MiB of scratch: 16 requests of 8,000 keys need more
    need = swr.workspace_bytes(swr.SWR_OP_GLOBAL_APPEND_ATTEND, 16, 4, 16, 2, 512, 8000)
    assert need > (16 << 20)
    fake = swr.SwrKV(0x10000, 0x10000, 0x10000, 0x10000, None, 8000 + 64 - 8000 % 64, 0, 1.0, 1.0)
    st = noalloc(ctypes.byref(fake), 0x10000, 0x10000, 0x10000, 0x10000, 0x10000, 8000, 16, 4, 16, 2, 512, 0.04,
                 None)
    assert st == 3  # SWR_ERR_WORKSPACE, before anything is launched
