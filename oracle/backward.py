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
routing-weight gradient are exactly zero.

The fp8 layer (``backward_fp8``): its forward quantises the token rows and h per
row and 128 channels and uses dequantised block-scaled weights (``oracle.layer``).
The pages trace a training NaN to that path's backward (the transformers PR
#45621 write-up, section 3) without fixing its arithmetic; the reading taken is
the straight-through one used for training through fake quantisation: each
quantise-then-dequantise step passes gradients unchanged, the weight gradients
are those of the dequantised weight values, and everything else is the chain
rule of the forward as it ran, so y and dW2 use the quantised h (h-hat):

    x-hat = dq(q(x)),  gu_p = W13-hat[e] x-hat_t,  h_p = silu(g) * u,  h-hat_p = dq(q(h_p))
    y_p = W2-hat[e] h-hat_p,   dw[r] = dout[t] . y_p,   dy_p = w[r] dout[t]
    dh_p = W2-hat[e]^T dy_p (straight through h-hat),   dgu_p as above
    dx_t = sum over slots of W13-hat[e]^T dgu_p (straight through x-hat)
    dW2[e] = sum dy_p h-hat_p^T,   dW13[e] = sum dgu_p x-hat_t^T
"""

from __future__ import annotations

import numpy as np

from .layer import ExpertWeights, dequant128, permute_rows, quant128, silu
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
    assert not W.fp8, "backward covers bf16/f32 layers; backward_fp8 the fp8 layer"
    return _backward(np.asarray(x, dtype=np.float64), ids, w, W, dout, None)


def backward_fp8(x, ids, w, W: ExpertWeights, dout) -> dict:
    """Gradients of the fp8 layer (``W.fp8``: e4m3 codes with 128x128 block scales) for
    fixed routing, straight through the quantisation of x and h (see the module doc).

    ``x`` [T, H] holds the token rows as given to the forward (bf16 values as floats);
    they are quantised per row and 128 channels here, as the forward does.  ``dw13`` and
    ``dw2`` are gradients of the dequantised weight values.  Returns the keys of
    ``backward`` plus ``x_hat`` [T, H] and ``h_hat`` [V, I]; ``h`` is the unquantised h.
    """
    assert W.fp8, "backward_fp8 needs block-scaled e4m3 weights"
    q, s = quant128(np.asarray(x, dtype=np.float32))
    x_hat = dequant128(q, s)

    def h_round(h):
        hq, hs = quant128(h.astype(np.float32))   # the forward quantises h from float32
        return dequant128(hq, hs)

    res = _backward(x_hat, ids, w, W, dout, h_round)
    res["x_hat"] = x_hat
    return res


def _backward(x, ids, w, W: ExpertWeights, dout, h_round) -> dict:
    """The chain rule through the per-expert loop; ``h_round`` (or None) maps h to the
    h the down projection consumes, with the gradient passed straight through it."""
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
    h_hat = np.zeros((V, I))
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
        hh_e = h_e if h_round is None else h_round(h_e)
        gu[a:b], h[a:b], h_hat[a:b] = gu_e, h_e, hh_e
        y[a:b] = hh_e @ w2.T
        dh = dy[a:b] @ w2
        dgu[a:b, :I] = dh * u * dsilu(g)
        dgu[a:b, I:] = dh * silu(g)
        dxp[a:b] = dgu[a:b] @ w13
        dw2[e] = dy[a:b].T @ hh_e
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
    return dict(dx=dx, dw13=dw13, dw2=dw2, dw=dw.reshape(T, k), gu=gu, h=h, h_hat=h_hat, y=y, dy=dy, dgu=dgu,
                dx_perm=dxp, offsets=offsets, sorted_rows=sorted_rows, row_pos=row_pos)
