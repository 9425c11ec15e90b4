"""Helpers for the GPU tests: device upload/download and the GEMM tolerance check."""
from __future__ import annotations

import sys

import numpy as np


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def torch_cuda():
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a ROCm GPU")
    return torch


def dev(a: np.ndarray):
    """Host array -> device tensor with the same bytes (uint16 is carried as int16)."""
    torch = torch_cuda()
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    elif a.dtype == np.uint32:
        a = a.view(np.int32)
    return torch.from_numpy(a).to("cuda")


def host(t, dtype=None) -> np.ndarray:
    a = t.detach().cpu().numpy()
    if dtype is not None:
        a = a.view(dtype)
    return a


def empty_u8(n):
    torch = torch_cuda()
    return torch.empty(int(n), dtype=torch.uint8, device="cuda")


def empty_u16(n):
    torch = torch_cuda()
    return torch.empty(int(n), dtype=torch.int16, device="cuda")


def empty_f32(*shape):
    torch = torch_cuda()
    return torch.empty(*shape, dtype=torch.float32, device="cuda")


def zeros_u32(n=1):
    torch = torch_cuda()
    return torch.zeros(int(n), dtype=torch.int32, device="cuda")


def check_gemm(y_gpu: np.ndarray, y_ref: np.ndarray, a_ref: np.ndarray, what: str, rel: float = 1e-3):
    """|Y_gpu - Y| <= rel * sum_k |x_k w_k| elementwise (Y, A from the fp64 oracle)."""
    err = np.abs(y_gpu.astype(np.float64) - y_ref)
    bound = rel * a_ref
    bad = err > bound
    if bad.any():
        i = int(np.argmax(err - bound))
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} outside 1e-3*sum|xw|; worst flat index {i}: "
            f"gpu {y_gpu.reshape(-1)[i]!r} ref {y_ref.reshape(-1)[i]!r} bound {bound.reshape(-1)[i]!r}")
