"""Helpers for the GPU parity tests: host <-> device copies and comparisons."""
import sys

import numpy as np
import pytest


def require_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import combine_balancing_amd as cba
    cba.lib()  # raises if the HIP library is missing: no fallback exists
    return torch


def dev(a):
    """numpy -> device tensor (uint16 bf16 patterns travel as int16)."""
    import torch
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).cuda()


def host(t, dtype=None):
    a = t.detach().cpu()
    if a.dtype.is_floating_point and a.element_size() == 2:
        a = a.view(__import__("torch").int16)
    a = a.numpy()
    if a.dtype == np.int16:
        a = a.view(np.uint16)
    return a if dtype is None else a.astype(dtype)


def note(msg):
    """Name the case on stdout before a GPU step (survives a crash)."""
    print(f"[gpu-case] {msg}", flush=True)
    sys.stdout.flush()


def bf16_ulp_diff(a, b):
    """|a - b| in bf16 ulps, via the ordered integer view of the patterns."""
    def ordered(x):
        x = x.astype(np.int32)
        return np.where(x & 0x8000, 0x8000 - (x & 0x7FFF), 0x8000 + x)
    return np.abs(ordered(a) - ordered(b))


def f32(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32)
