"""Helpers for the GPU parity tests: moving host pools and bf16 bit arrays to
the device and back, and building the library's KV views."""
from __future__ import annotations

import numpy as np
import torch

import sliding_window_ring_amd as swr


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(bits, np.uint16)
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host_f64(t: torch.Tensor) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def dev_i32(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int32)).cuda()


def dev_i64(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.int64)).cuda()


def dev_u8(a) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, np.uint8)).cuda()


def layer(k_pool, v_pool, k_off, v_off, cap, dtype=0, k_scale=1.0, v_scale=1.0) -> swr.KVLayer:
    """Device copies of host pools (numpy uint8) as a KV view."""
    return swr.KVLayer(dev_u8(k_pool), dev_u8(v_pool), dev_i64(k_off), dev_i64(v_off), cap, dtype,
                       float(k_scale), float(v_scale))


def pool_bytes(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()
