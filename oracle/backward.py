"""Gradients of the MoE expert layer (the backward of ``oracle.layer``), float64.

Test infrastructure only (see ``oracle/__init__``).

The pages trace a training-time NaN to sentinel rows whose outputs a kernel
left uninitialised (the transformers PR #45621 write-up, section 3), and
credit the fused kernels with their training speed-up (the LlamaFactory
PR #10481 write-up, "why it is better"): the layer has a backward.  It is the
derivative of the forward in ``oracle.layer`` with the routing (expert ids and
routing weights) given, written here as the same per-expert loop over the
expert-contiguous segments:

  forward, per valid routed row p = row_pos[r] of token t = r // k, expert e:
    gu_p = W13[e] x_t            g = gu_p[:I], u = gu_p[I:]
    h_p  = silu(g) * u           y_p = W2[e] h_p
    out[t] += w[r] * y_p
  backward, given dout [T, H]:
    dy_p   = w[r] * dout[t]                      (routing weight applied in the combine)
    dw[r]  = dout[t] . y_p                       (gradient of the routing weight)
    dh_p   = W2[e]^T dy_p
    dg     = dh_p * u * silu'(g),  du = dh_p * silu(g),  dgu_p = [dg, du]
    dx_t  += W13[e]^T dgu_p                      (summed over the token's slots)
    dW2[e]  += dy_p h_p^T,   dW13[e] += dgu_p x_t^T

with silu'(g) = s (1 + g (1 - s)), s = sigmoid(g).  Sentinel rows (permuted
positions >= offsets[E]) contribute nothing: their dx share, dW terms and
routing-weight gradient are exactly zero.  bf16/f32 layers only.
"""

from __future__ import annotations

import numpy as np

from .layer import ExpertWeights, permute_rows, silu
from .routing import build_offsets


def dsilu(g: np.ndarray) -> np.ndarray:
    """Derivative of silu(g) = g * sigmoid(g)."""
    with np.errstate(over="ignore"):
        s = 1.0 / (1.0 + np.exp(-g))
    return s * (1.0 + g * (1.0 - s))


def backward(x, ids, w, W: ExpertWeights, dout) -> dict:
    """All gradients of the layer for fixed routing ``ids`` [T, k], ``w`` [T, k].

    ``x`` [T, H] and the weights hold the stored values (f32, or bf16 values as
    floats); ``dout`` [T, H].  Returns float64 ``dx`` [T, H], ``dw13`` [E, 2I, H],
    ``dw2`` [E, H, I], ``dw`` [T, k], and the permuted intermediates ``gu``
    [V, 2I], ``h`` [V, I], ``y`` [V, H], ``dy`` [V, H], ``dgu`` [V, 2I],
    ``dx_perm`` [V, H], with the routing arrays ``offsets``, ``sorted_rows``,
    ``row_pos``.
    """
    assert not W.fp8, "the backward covers bf16/f32 layers"
    x = np.asarray(x, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    ids = np.asarray(ids)
    T, H = x.shape
    k = ids.shape[1]
    E, I = W.E, W.I
    flat_ids = ids.reshape(-1)
    flat_w = np.asarray(w, dtype=np.float64).reshape(-1)
    offsets, sorted_rows, row_pos = build_offsets(flat_ids, E)
    V = int(offsets[-1])
    rows = np.asarray(sorted_rows[:V], dtype=np.int64)   # flat slot r of permuted row p
    tok = rows // k

    xp = permute_rows(x, sorted_rows, offsets, k)        # [V, H]
    dy = flat_w[rows][:, None] * dout[tok]               # [V, H]
    gu = np.zeros((V, 2 * I))
    h = np.zeros((V, I))
    y = np.zeros((V, H))
    dgu = np.zeros((V, 2 * I))
    dxp = np.zeros((V, H))
    dw13 = np.zeros((E, 2 * I, H))
    dw2 = np.zeros((E, H, I))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        w13, w2 = W.gate_up(e), W.down(e)
        gu_e = xp[a:b] @ w13.T
        g, u = gu_e[:, :I], gu_e[:, I:]
        h_e = silu(g) * u
        gu[a:b], h[a:b] = gu_e, h_e
        y[a:b] = h_e @ w2.T
        dh = dy[a:b] @ w2
        dgu[a:b, :I] = dh * u * dsilu(g)
        dgu[a:b, I:] = dh * silu(g)
        dxp[a:b] = dgu[a:b] @ w13
        dw2[e] = dy[a:b].T @ h_e
        dw13[e] = dgu[a:b].T @ xp[a:b]

    dx = np.zeros((T, H))
    dw = np.zeros(T * k)
    for j in range(k):                                   # slot order, as the forward's combine
        r = np.arange(T) * k + j
        p = np.asarray(row_pos)[r]
        valid = (flat_ids[r] >= 0) & (flat_ids[r] < E) & (p < V)
        pv = np.where(valid, p, 0)
        dx += np.where(valid[:, None], dxp[pv], 0.0)
        dw[r] = np.where(valid, np.einsum("th,th->t", dout, y[pv]), 0.0)
    return dict(dx=dx, dw13=dw13, dw2=dw2, dw=dw.reshape(T, k), gu=gu, h=h, y=y, dy=dy, dgu=dgu,
                dx_perm=dxp, offsets=offsets, sorted_rows=sorted_rows, row_pos=row_pos)
