"""Brute-force dense evaluation of the MoE layer: a pin for the per-expert oracle.

Test infrastructure only (see ``oracle/__init__``).

Deliberately built differently from ``oracle.layer`` and sharing none of its
code: routing by a full sort of each token's logits (``np.lexsort``), no
histogram, no offsets and no permutation; every token goes through every
expert densely and the expert outputs are gated by a [T, E] matrix holding the
routing weight of each (token, expert) pair (zero when not routed).  For the
fp8 variant the quantisation uses torch's e4m3 cast instead of the oracle's
own encoder.  Meant for tiny shapes only (T * E expert evaluations).
"""

from __future__ import annotations

import numpy as np


def route_by_sort(logits, k: int, renormalize: bool = True):
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    ids = np.empty((T, k), dtype=np.int64)
    w = np.empty((T, k), dtype=np.float32)
    for t in range(T):
        # primary key: descending logit; secondary key: ascending expert id
        order = np.lexsort((np.arange(E), -lg[t].astype(np.float64)))
        sel = order[:k]
        ids[t] = sel
        vals = lg[t, sel].astype(np.float64)
        if renormalize:
            z = np.exp(vals - vals.max())
            w[t] = (z / z.sum()).astype(np.float32)
        else:
            allv = lg[t].astype(np.float64)
            z = np.exp(allv - allv.max())
            w[t] = (z[sel] / z.sum()).astype(np.float32)
    return ids, w


def _fp8_roundtrip_rows(v32: np.ndarray) -> np.ndarray:
    """Per-128-group quantise/dequantise with torch's e4m3 cast (float64 result)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(v32, dtype=np.float32))
    g = t.reshape(*t.shape[:-1], t.shape[-1] // 128, 128)
    amax = g.abs().amax(dim=-1, keepdim=True)
    s = torch.where(amax == 0, torch.ones_like(amax), amax / 448.0)
    q = (g / s).clamp(-448.0, 448.0).to(torch.float8_e4m3fn)
    return (q.to(torch.float64) * s.to(torch.float64)).reshape(t.shape).numpy()


def _fp8_dequant_blocks(codes_u8: np.ndarray, scales: np.ndarray) -> np.ndarray:
    import torch
    vals = torch.from_numpy(np.ascontiguousarray(codes_u8)).view(torch.float8_e4m3fn).to(
        torch.float64).numpy()
    N, K = vals.shape
    s = np.kron(np.asarray(scales, dtype=np.float64), np.ones((128, 128)))[:N, :K]
    return vals * s


def dense_forward(x, logits, w13, w2, k: int, num_valid_rows: int = -1, renormalize: bool = True,
                  w13_scale=None, w2_scale=None) -> np.ndarray:
    """out [T, H] float64; every token through every expert, gated by routing weight."""
    x = np.asarray(x, dtype=np.float32)
    T, H = x.shape
    E = w13.shape[0]
    I = w2.shape[2]
    fp8 = w13_scale is not None
    ids, w = route_by_sort(logits, k, renormalize)
    V = T * k if num_valid_rows < 0 else num_valid_rows
    gate = np.zeros((T, E), dtype=np.float64)
    for t in range(T):
        for j in range(k):
            if t * k + j < V:
                gate[t, ids[t, j]] += float(w[t, j])
    xv = _fp8_roundtrip_rows(x) if fp8 else x.astype(np.float64)
    out = np.zeros((T, H), dtype=np.float64)
    for e in range(E):
        if fp8:
            a = _fp8_dequant_blocks(w13[e], w13_scale[e])
            b = _fp8_dequant_blocks(w2[e], w2_scale[e])
        else:
            a = np.asarray(w13[e], dtype=np.float64)
            b = np.asarray(w2[e], dtype=np.float64)
        for t in range(T):
            g = a[:I] @ xv[t]
            u = a[I:] @ xv[t]
            hrow = g * u / (1.0 + np.exp(-g))
            if fp8:
                hrow = _fp8_roundtrip_rows(hrow.astype(np.float32)[None, :])[0]
            out[t] += gate[t, e] * (b @ hrow)
    return out
