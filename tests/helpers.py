"""Shared test helpers (comparison metrics, tensor -> array conversion)."""
from __future__ import annotations

import sys

import numpy as np
import torch


def say(*a):
    """Print and flush, so a GPU run names its case before each step."""
    print(*a, flush=True)
    sys.stdout.flush()


def np32(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float32).numpy()


def npu8(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().view(torch.uint8).numpy()


def row_rel_err(got, ref) -> float:
    """max over rows of max|got - ref| / max|ref| of that row; all-zero reference rows count absolutely."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    scale = np.abs(ref).max(axis=-1, keepdims=True)
    scale = np.where(scale == 0, 1.0, scale)
    return float((np.abs(got - ref) / scale).max())


class HostExperts:
    """Per-expert host copies of packed GPU weights, fetched on first use (for ExpertWeights)."""

    def __init__(self, t: torch.Tensor):
        self.t = t
        self.shape = tuple(t.shape)
        self.fp8 = t.dtype == torch.float8_e4m3fn

    def __getitem__(self, e):
        x = self.t[e].detach().cpu()
        return x.view(torch.uint8).numpy() if self.fp8 else x.to(torch.float32).numpy()


TOL = {"f32": 1e-4, "bf16": 1e-2, "fp8": 2e-2}
