"""Helpers for the GPU parity tests: device set-up and row extraction."""
from __future__ import annotations

import sys

import numpy as np
import pytest


def log(*a):
    print("[gpu-test]", *a, file=sys.stderr, flush=True)


def device():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import kv_cache_quantization_quantize_amd as kvq
    kvq.lib()       # raises (fails the test) when the HIP library is missing
    return torch.device("cuda:0")


def bits(t) -> np.ndarray:
    """fp16 / int16 tensor -> numpy uint16 bit patterns (on the host)."""
    import torch
    if t.dtype == torch.float16:
        t = t.view(torch.int16)
    return t.cpu().numpy().view(np.uint16)


def rows(t, idx) -> np.ndarray:
    """t [L, T, H, R] -> [n, R] at the (l, t, h) triples idx [n, 3]."""
    import torch
    i = torch.as_tensor(idx, device=t.device)
    r = t[i[:, 0], i[:, 1], i[:, 2]]
    if r.dtype in (torch.float16, torch.int16):
        return bits(r)
    return r.cpu().numpy()


def lam_rows(lam, idx) -> np.ndarray:
    import torch
    i = torch.as_tensor(idx, device=lam.device)
    return lam[i[:, 0], i[:, 2]].cpu().numpy().astype(np.float32)


def all_idx(L, T, H) -> np.ndarray:
    l, t, h = np.meshgrid(np.arange(L), np.arange(T), np.arange(H), indexing="ij")
    return np.stack([l.ravel(), t.ravel(), h.ravel()], axis=1)
