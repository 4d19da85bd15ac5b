"""Torch-tensor wrappers over the C ABI: argument marshalling only.

Every function checks devices, dtypes, shapes and contiguity, allocates its
outputs with torch (device memory and the current stream are torch's), and
calls the HIP library; a non-OK status raises RuntimeError with the
library's message.  There is no fallback: without the built library on a
GPU, ``load()`` raises ImportError.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional

import torch

from . import _lib
from ._lib import MoeAux, load

_DT = {torch.float32: _lib.MOE_F32, torch.bfloat16: _lib.MOE_BF16,
       torch.float8_e4m3fn: _lib.MOE_FP8_E4M3}
_EPI = {"none": _lib.MOE_EPI_NONE, "silu_mul": _lib.MOE_EPI_SILU_MUL}


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _check(status: int) -> None:
    if status != _lib.MOE_OK:
        lib = load()
        raise RuntimeError(f"{lib.status_string(status).decode()}: {lib.last_error().decode()}")


def _need(t: torch.Tensor, name: str, dtype=None, shape=None, device=None) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def route_topk(logits: torch.Tensor, k: int, num_valid_rows: int = -1, renormalize: bool = True):
    """logits f32 [T, E] -> (topk_ids int32 [T, k], topk_weights f32 [T, k])."""
    _need(logits, "logits", torch.float32)
    T, E = logits.shape
    ids = torch.empty(T, k, dtype=torch.int32, device=logits.device)
    w = torch.empty(T, k, dtype=torch.float32, device=logits.device)
    _check(load().route_topk(_p(logits), T, E, k, num_valid_rows, int(bool(renormalize)),
                             _p(ids), _p(w), _stream(logits)))
    return ids, w


def build_offsets(topk_ids: torch.Tensor, E: int):
    """flat ids int32 [R] -> (offsets int32 [E+1], sorted_rows int32 [R], row_pos int32 [R])."""
    _need(topk_ids, "topk_ids", torch.int32)
    ids = topk_ids.reshape(-1)
    R = ids.numel()
    dev = ids.device
    lib = load()
    ws = torch.empty(max(1, lib.build_offsets_workspace(R, E)), dtype=torch.uint8, device=dev)
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev)
    sorted_rows = torch.empty(R, dtype=torch.int32, device=dev)
    row_pos = torch.empty(R, dtype=torch.int32, device=dev)
    _check(lib.build_offsets(_p(ids), R, E, _p(offsets), _p(sorted_rows), _p(row_pos), _p(ws),
                             ws.numel(), _stream(ids)))
    return offsets, sorted_rows, row_pos


def build_offsets_noalloc(topk_ids: torch.Tensor, E: int, offsets: torch.Tensor, sorted_rows: torch.Tensor,
                          row_pos: torch.Tensor):
    """build_offsets into caller-provided outputs, with no workspace (the library's static scratch):
    flat ids int32 [R] -> offsets int32 [E+1], sorted_rows int32 [R], row_pos int32 [R]."""
    _need(topk_ids, "topk_ids", torch.int32)
    ids = topk_ids.reshape(-1)
    R = ids.numel()
    dev = ids.device
    _need(offsets, "offsets", torch.int32, (E + 1,), dev)
    _need(sorted_rows, "sorted_rows", torch.int32, (R,), dev)
    _need(row_pos, "row_pos", torch.int32, (R,), dev)
    _check(load().build_offsets_noalloc(_p(ids), R, E, _p(offsets), _p(sorted_rows), _p(row_pos), _stream(ids)))
    return offsets, sorted_rows, row_pos


def permute(x: torch.Tensor, sorted_rows: torch.Tensor, offsets: torch.Tensor, k: int,
            out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
            out_scales: Optional[torch.Tensor] = None):
    """x [T, H] -> x_perm [R, H] (rows >= offsets[E] untouched); fp8 also returns scales [H/128, R]."""
    _need(x, "x", (torch.float32, torch.bfloat16))
    T, H = x.shape
    R = sorted_rows.numel()
    E = offsets.numel() - 1
    out_dtype = out_dtype or x.dtype
    _need(sorted_rows, "sorted_rows", torch.int32, device=x.device)
    _need(offsets, "offsets", torch.int32, device=x.device)
    if out is None:
        out = torch.empty(R, H, dtype=out_dtype, device=x.device)
    _need(out, "out", out_dtype, (R, H), x.device)
    fp8 = out_dtype == torch.float8_e4m3fn
    if fp8 and out_scales is None:
        out_scales = torch.empty(H // 128, R, dtype=torch.float32, device=x.device)
    _check(load().permute(_p(x), _DT[x.dtype], T, H, k, _p(sorted_rows), _p(offsets), E, R,
                          _p(out), _DT[out_dtype], _p(out_scales) if fp8 else None, _stream(x)))
    return (out, out_scales) if fp8 else out


def _gemm(a, b, offsets, epilogue, a_scales, b_scales, out_dtype, out, out_scales, gather):
    _need(a, "a", tuple(_DT))
    A_rows, K = a.shape
    E, N, K2 = b.shape
    if K2 != K:
        raise ValueError(f"K mismatch: a has {K}, b has {K2}")
    _need(b, "b", a.dtype, device=a.device)
    _need(offsets, "offsets", torch.int32, (E + 1,), a.device)
    if gather is not None:
        rows, div = gather
        _need(rows, "gather_rows", torch.int32, device=a.device)
        M = rows.numel()
    else:
        M = A_rows
    fp8 = a.dtype == torch.float8_e4m3fn
    if fp8:
        _need(a_scales, "a_scales", torch.float32, (K // 128, A_rows), a.device)
        _need(b_scales, "b_scales", torch.float32, (E, N // 128, K // 128), a.device)
    n_out = N // 2 if epilogue == "silu_mul" else N
    out_dtype = out_dtype or (torch.bfloat16 if fp8 else a.dtype)
    if out is None:
        out = torch.empty(M, n_out, dtype=out_dtype, device=a.device)
    _need(out, "out", out_dtype, (M, n_out), a.device)
    fp8_out = out_dtype == torch.float8_e4m3fn
    if fp8_out and out_scales is None:
        out_scales = torch.empty(n_out // 128, M, dtype=torch.float32, device=a.device)
    common = (_p(b), _p(b_scales) if fp8 else None, _DT[a.dtype], _p(offsets), E, M, N, K, _EPI[epilogue],
              _p(out), _DT[out_dtype], _p(out_scales) if fp8_out else None, _stream(a))
    if gather is None:
        _check(load().grouped_gemm(_p(a), _p(a_scales) if fp8 else None, *common))
    else:
        _check(load().grouped_gemm_gather(_p(a), _p(a_scales) if fp8 else None, A_rows, _p(rows), int(div),
                                          *common))
    return (out, out_scales) if fp8_out else out


def grouped_gemm(a: torch.Tensor, b: torch.Tensor, offsets: torch.Tensor, epilogue: str = "none",
                 a_scales: Optional[torch.Tensor] = None, b_scales: Optional[torch.Tensor] = None,
                 out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
                 out_scales: Optional[torch.Tensor] = None):
    """a [M, K] x b [E, N, K] over segments of offsets -> c [M, N or N/2] (+ scales for fp8 out).

    fp8 activation scales (a_scales, and the returned scales) are block-major:
    [K/128, M] and [N_out/128, M].
    """
    return _gemm(a, b, offsets, epilogue, a_scales, b_scales, out_dtype, out, out_scales, None)


def grouped_gemm_gather(a: torch.Tensor, b: torch.Tensor, offsets: torch.Tensor, gather_rows: torch.Tensor,
                        gather_div: int, epilogue: str = "none", a_scales: Optional[torch.Tensor] = None,
                        b_scales: Optional[torch.Tensor] = None, out_dtype: Optional[torch.dtype] = None,
                        out: Optional[torch.Tensor] = None, out_scales: Optional[torch.Tensor] = None):
    """grouped_gemm with product row p reading a[gather_rows[p] // gather_div]; c has gather_rows.numel() rows.

    a [A_rows, K] holds token rows (a_scales [K/128, A_rows] for fp8); gather_rows is
    sorted_rows of build_offsets and gather_div is k.
    """
    return _gemm(a, b, offsets, epilogue, a_scales, b_scales, out_dtype, out, out_scales,
                 (gather_rows, gather_div))


def quantize_rows(x: torch.Tensor):
    """bf16 x [T, H] -> (e4m3 codes [T, H], f32 scales [H/128, T]), per row and 128 channels."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    xq = torch.empty(T, H, dtype=torch.float8_e4m3fn, device=x.device)
    xs = torch.empty(H // 128, T, dtype=torch.float32, device=x.device)
    _check(load().quantize_rows(_p(x), T, H, _p(xq), _p(xs), _stream(x)))
    return xq, xs


def grouped_gemm_tile_shape(dtype: torch.dtype, epilogue: str, M_rows: int, E: int,
                            out_dtype: Optional[torch.dtype] = None):
    """(tile rows, tile weight rows, K elements per slice) of moe_grouped_gemm for a dtype, epilogue,
    launch size (M_rows product rows over E experts) and output dtype (default: bf16 for fp8
    operands, else the operand dtype)."""
    out_dtype = out_dtype or (torch.bfloat16 if dtype == torch.float8_e4m3fn else dtype)
    m, n, k = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(load().grouped_gemm_tile_shape(_DT[dtype], _EPI[epilogue], _DT[out_dtype], M_rows, E,
                                          ctypes.byref(m), ctypes.byref(n), ctypes.byref(k)))
    return m.value, n.value, k.value


def unpermute_combine(y: torch.Tensor, row_pos: torch.Tensor, topk_weights: torch.Tensor,
                      offsets: torch.Tensor, k: int, out_dtype: Optional[torch.dtype] = None,
                      out: Optional[torch.Tensor] = None):
    """y [R, H] -> out [T, H] = weighted sum of each token's valid rows."""
    _need(y, "y", (torch.float32, torch.bfloat16))
    R, H = y.shape
    T = R // k
    E = offsets.numel() - 1
    _need(row_pos, "row_pos", torch.int32, device=y.device)
    _need(topk_weights, "topk_weights", torch.float32, device=y.device)
    _need(offsets, "offsets", torch.int32, device=y.device)
    out_dtype = out_dtype or y.dtype
    if out is None:
        out = torch.empty(T, H, dtype=out_dtype, device=y.device)
    _need(out, "out", out_dtype, (T, H), y.device)
    _check(load().unpermute_combine(_p(y), _DT[y.dtype], _p(row_pos), _p(topk_weights), _p(offsets),
                                    E, T, H, k, _p(out), _DT[out_dtype], _stream(y)))
    return out


@dataclass
class ForwardAux:
    topk_ids: torch.Tensor
    topk_weights: torch.Tensor
    offsets: torch.Tensor
    sorted_rows: torch.Tensor
    row_pos: torch.Tensor


def forward_workspace_bytes(T: int, H: int, I: int, E: int, k: int, w_dtype: torch.dtype) -> int:
    return load().forward_workspace(T, H, I, E, k, _DT[w_dtype])


def forward(x: torch.Tensor, logits: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, k: int,
            num_valid_rows: int = -1, renormalize: bool = True,
            w13_scale: Optional[torch.Tensor] = None, w2_scale: Optional[torch.Tensor] = None,
            out_dtype: Optional[torch.dtype] = None, out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, return_aux: bool = False,
            stage_events=None):
    """The whole layer: x [T, H], logits f32 [T, E], w13 [E, 2I, H], w2 [E, H, I] -> out [T, H].

    ``stage_events``: optional sequence of 7 hipEvent_t handles (ints) that the
    library records before the first stage and after each of the six stages.
    """
    _need(x, "x", (torch.float32, torch.bfloat16))
    T, H = x.shape
    E, I2, H2 = w13.shape
    I = I2 // 2
    dev = x.device
    _need(logits, "logits", torch.float32, (T, E), dev)
    _need(w13, "w13", tuple(_DT), (E, 2 * I, H), dev)
    _need(w2, "w2", w13.dtype, (E, H, I), dev)
    fp8 = w13.dtype == torch.float8_e4m3fn
    if fp8:
        _need(w13_scale, "w13_scale", torch.float32, (E, 2 * I // 128, H // 128), dev)
        _need(w2_scale, "w2_scale", torch.float32, (E, H // 128, I // 128), dev)
    out_dtype = out_dtype or (torch.float32 if w13.dtype == torch.float32 else torch.bfloat16)
    if out is None:
        out = torch.empty(T, H, dtype=out_dtype, device=dev)
    _need(out, "out", out_dtype, (T, H), dev)
    lib = load()
    need = lib.forward_workspace(T, H, I, E, k, _DT[w13.dtype])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, device=dev)
    aux_t = None
    aux_c = None
    ev_arr = None
    if stage_events is not None:
        if len(stage_events) != len(_lib.FORWARD_STAGES) + 1:
            raise ValueError("stage_events needs one event per stage boundary (7)")
        ev_arr = (ctypes.c_void_p * len(stage_events))(*stage_events)
        aux_c = MoeAux()
        aux_c.stage_events = ctypes.cast(ev_arr, ctypes.POINTER(ctypes.c_void_p))
    if return_aux:
        R = T * k
        aux_t = ForwardAux(torch.empty(T, k, dtype=torch.int32, device=dev),
                           torch.empty(T, k, dtype=torch.float32, device=dev),
                           torch.empty(E + 1, dtype=torch.int32, device=dev),
                           torch.empty(R, dtype=torch.int32, device=dev),
                           torch.empty(R, dtype=torch.int32, device=dev))
        aux_c = aux_c or MoeAux()
        aux_c.topk_ids = aux_t.topk_ids.data_ptr()
        aux_c.topk_weights = aux_t.topk_weights.data_ptr()
        aux_c.offsets = aux_t.offsets.data_ptr()
        aux_c.sorted_rows = aux_t.sorted_rows.data_ptr()
        aux_c.row_pos = aux_t.row_pos.data_ptr()
    _check(lib.forward(_p(x), _DT[x.dtype], _p(logits), _p(w13), _p(w13_scale) if fp8 else None,
                       _p(w2), _p(w2_scale) if fp8 else None, _DT[w13.dtype], T, H, I, E, k,
                       num_valid_rows, int(bool(renormalize)), _p(out), _DT[out_dtype],
                       ctypes.byref(aux_c) if aux_c is not None else None, _p(workspace),
                       workspace.numel(), _stream(x)))
    return (out, aux_t) if return_aux else out


@dataclass
class Gradients:
    dx: torch.Tensor              # [T, H]
    dw13: torch.Tensor            # [E, 2I, H]
    dw2: torch.Tensor             # [E, H, I]
    dtopk_weights: torch.Tensor   # f32 [T, k]


def backward_workspace_bytes(T: int, H: int, I: int, E: int, k: int, w_dtype: torch.dtype = torch.bfloat16) -> int:
    return load().backward_workspace(T, H, I, E, k, _DT[w_dtype])


def backward(x: torch.Tensor, w13: torch.Tensor, w2: torch.Tensor, dout: torch.Tensor,
             topk_weights: torch.Tensor, offsets: torch.Tensor, sorted_rows: torch.Tensor,
             row_pos: torch.Tensor, grad_dtype: torch.dtype = torch.float32,
             workspace: Optional[torch.Tensor] = None, w13_scale: Optional[torch.Tensor] = None,
             w2_scale: Optional[torch.Tensor] = None) -> Gradients:
    """Gradients of the layer for the routing ``forward`` chose (its aux outputs):
    x, dout bf16 [T, H]; w13 [E, 2I, H]; w2 [E, H, I] (bf16, or e4m3 with block scales
    w13_scale [E, 2I/128, H/128] and w2_scale [E, H/128, I/128]) -> dx, dw13, dw2
    (grad_dtype), dtopk_weights (f32)."""
    _need(x, "x", torch.bfloat16)
    T, H = x.shape
    E, I2, _ = w13.shape
    I = I2 // 2
    k = topk_weights.shape[1] if topk_weights.dim() == 2 else 1
    dev = x.device
    _need(w13, "w13", (torch.bfloat16, torch.float8_e4m3fn), (E, 2 * I, H), dev)
    _need(w2, "w2", w13.dtype, (E, H, I), dev)
    fp8 = w13.dtype == torch.float8_e4m3fn
    if fp8:
        _need(w13_scale, "w13_scale", torch.float32, (E, 2 * I // 128, H // 128), dev)
        _need(w2_scale, "w2_scale", torch.float32, (E, H // 128, I // 128), dev)
    _need(dout, "dout", torch.bfloat16, (T, H), dev)
    _need(topk_weights, "topk_weights", torch.float32, (T, k), dev)
    _need(offsets, "offsets", torch.int32, (E + 1,), dev)
    _need(sorted_rows, "sorted_rows", torch.int32, device=dev)
    _need(row_pos, "row_pos", torch.int32, device=dev)
    if sorted_rows.numel() != T * k or row_pos.numel() != T * k:
        raise ValueError("sorted_rows and row_pos need T*k entries")
    g = Gradients(torch.empty(T, H, dtype=grad_dtype, device=dev),
                  torch.empty(E, 2 * I, H, dtype=grad_dtype, device=dev),
                  torch.empty(E, H, I, dtype=grad_dtype, device=dev),
                  torch.empty(T, k, dtype=torch.float32, device=dev))
    lib = load()
    need = lib.backward_workspace(T, H, I, E, k, _DT[w13.dtype])
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _need(workspace, "workspace", torch.uint8, device=dev)
    _check(lib.backward(_p(x), _p(w13), _p(w13_scale) if fp8 else None, _p(w2), _p(w2_scale) if fp8 else None,
                        _DT[w13.dtype], T, H, I, E, k, _p(topk_weights), _p(offsets), _p(sorted_rows), _p(row_pos),
                        _p(dout), _p(g.dx), _p(g.dw13), _p(g.dw2), _DT[grad_dtype], _p(g.dtopk_weights),
                        _p(workspace), workspace.numel(), _stream(x)))
    return g
