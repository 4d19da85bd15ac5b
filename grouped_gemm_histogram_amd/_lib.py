"""ctypes loader for ``libmoe.so`` (the C ABI declared in ``include/moe.h``).

``load()`` opens the library once and returns a frozen dataclass of its entry
points, following the loader pattern of the transformers PR #45621 write-up
(section 1: a cached loader returning a frozen dataclass of kernels, and an
ImportError naming whatever is missing).  A failure is remembered and raised
again on every later call; loading is never retried.
"""

from __future__ import annotations

import ctypes
import functools
import os
from dataclasses import dataclass
from typing import Callable, Optional

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_OK, MOE_ERR_INVALID_ARG, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_LAUNCH = range(5)
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_EPI_NONE, MOE_EPI_SILU_MUL = 0, 1

P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
SZ = ctypes.c_size_t


class MoeAux(ctypes.Structure):
    _fields_ = [("topk_ids", P), ("topk_weights", P), ("offsets", P),
                ("sorted_rows", P), ("row_pos", P), ("stage_events", ctypes.POINTER(P))]


# stage 3: nothing for f32/bf16 layers (the gate/up GEMM gathers token rows); per-token
# quantisation for fp8
FORWARD_STAGES = ("route", "offsets", "act_staging", "gemm_gate_up", "gemm_down", "combine")


# name -> (restype, argtypes); mirrors include/moe.h
SIGNATURES: dict[str, tuple] = {
    "moe_route_topk": (I32, [P, I64, I32, I32, I64, I32, P, P, P]),
    "moe_build_offsets_workspace": (SZ, [I64, I32]),
    "moe_build_offsets": (I32, [P, I64, I32, P, P, P, P, SZ, P]),
    "moe_build_offsets_noalloc": (I32, [P, I64, I32, P, P, P, P]),
    "moe_permute": (I32, [P, I32, I64, I64, I32, P, P, I32, I64, P, I32, P, P]),
    "moe_grouped_gemm": (I32, [P, P, P, P, I32, P, I32, I64, I64, I64, I32, P, I32, P, P]),
    "moe_grouped_gemm_gather": (I32, [P, P, I64, P, I32, P, P, I32, P, I32, I64, I64, I64, I32, P, I32, P,
                                      P]),
    "moe_quantize_rows": (I32, [P, I64, I64, P, P, P]),
    "moe_grouped_gemm_tile_shape": (I32, [I32, I32, I32, I64, I32, ctypes.POINTER(I32), ctypes.POINTER(I32),
                                          ctypes.POINTER(I32)]),
    "moe_unpermute_combine": (I32, [P, I32, P, P, P, I32, I64, I64, I32, P, I32, P]),
    "moe_forward_workspace": (SZ, [I64, I64, I64, I32, I32, I32]),
    "moe_forward": (I32, [P, I32, P, P, P, P, P, I32, I64, I64, I64, I32, I32, I64, I32, P, I32,
                          ctypes.POINTER(MoeAux), P, SZ, P]),
    "moe_backward_workspace": (SZ, [I64, I64, I64, I32, I32, I32]),
    "moe_backward": (I32, [P, P, P, P, P, I32, I64, I64, I64, I32, I32, P, P, P, P, P, P, P, P, I32, P, P,
                           SZ, P]),
    "moe_status_string": (ctypes.c_char_p, [I32]),
    "moe_last_error": (ctypes.c_char_p, []),
    "moe_abi_version": (I32, []),
}


@dataclass(frozen=True)
class MoeKernels:
    route_topk: Callable
    build_offsets_workspace: Callable
    build_offsets: Callable
    build_offsets_noalloc: Callable
    permute: Callable
    grouped_gemm: Callable
    grouped_gemm_gather: Callable
    quantize_rows: Callable
    grouped_gemm_tile_shape: Callable
    unpermute_combine: Callable
    forward_workspace: Callable
    forward: Callable
    backward_workspace: Callable
    backward: Callable
    status_string: Callable
    last_error: Callable
    abi_version: Callable
    path: str


_failure: Optional[ImportError] = None


@functools.cache
def _load_once() -> MoeKernels:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built (run grouped_gemm_histogram_amd.build.build())")
    try:
        lib = ctypes.CDLL(LIB_PATH)
    except OSError as exc:
        raise ImportError(f"cannot load {LIB_PATH}: {exc}") from exc
    fns = {}
    missing = []
    for name, (res, args) in SIGNATURES.items():
        try:
            f = getattr(lib, name)
        except AttributeError:
            missing.append(name)
            continue
        f.restype, f.argtypes = res, args
        fns[name[len("moe_"):]] = f
    if missing:
        raise ImportError(f"{LIB_PATH} lacks entry points: {', '.join(missing)}")
    return MoeKernels(path=LIB_PATH, **fns)


def load() -> MoeKernels:
    """The library's entry points (cached).  Raises ImportError, every time, if it cannot load."""
    global _failure
    if _failure is not None:
        raise _failure
    try:
        return _load_once()
    except ImportError as exc:
        _failure = exc
        raise
