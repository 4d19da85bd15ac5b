"""The MoE expert layer as a plain per-expert loop, in float64.

Test infrastructure only (see ``oracle/__init__``).

This is the "before" structure of the LlamaFactory PR #10481 write-up
(section 1: a Python loop over experts) and the ``eager`` backend of the
"트랜스포머에서 전문가 혼합 (MoEs)" write-up (expert backends section), run
over the expert-contiguous segments that the grouped path uses, so that every
intermediate (permuted rows, h, per-row expert outputs) can be compared.

Conventions:

* gate/up weights ``w13[e]`` are [2I, H]: rows [0, I) gate, rows [I, 2I) up;
  ``h = silu(gate) * up`` (the SiLU(fc1_1) * fc1_2 step of the LlamaFactory
  write-up, section 1); down weights ``w2[e]`` are [H, I].
* the routing weight is applied in the combine, after the down projection.
* sentinel rows (permuted positions >= offsets[E]) are zero in h and in the
  expert outputs: the transformers PR #45621 write-up, section 3, traces a
  NaN to sentinel outputs that a kernel left uninitialised.

fp8 variant (block-scaled e4m3): activations are quantised per token and per
128-channel group before permuting, weights carry one fp32 scale per 128x128
block, h is quantised per row and per 128-channel group straight from its
float32 value; each GEMM is the product of the dequantised operands.
"""

from __future__ import annotations

import numpy as np

from . import e4m3
from .routing import build_offsets, route_topk

GROUP = 128


def silu(g: np.ndarray) -> np.ndarray:
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


# ----------------------------------------------------------------------------- fp8 helpers

def quant128(v) -> tuple[np.ndarray, np.ndarray]:
    """Per-128-group quantisation of float32 rows (last dim a multiple of 128).

    For each group: amax = max |v|; scale s = amax / 448 as a correctly rounded
    float32 division (s = 1 when amax == 0); code = e4m3 RNE of the float32
    quotient v / s.  Returns (uint8 codes, float32 scales [..., n/128]).
    """
    v = np.asarray(v, dtype=np.float32)
    n = v.shape[-1]
    if n % GROUP:
        raise ValueError("last dimension must be a multiple of 128")
    g = v.reshape(v.shape[:-1] + (n // GROUP, GROUP))
    amax = np.abs(g).max(axis=-1)
    s = np.where(amax == 0, np.float32(1.0), amax / np.float32(e4m3.MAX)).astype(np.float32)
    q = e4m3.encode((g / s[..., None]).astype(np.float32))
    return q.reshape(v.shape), s


def dequant128(codes, scales) -> np.ndarray:
    """Inverse of quant128 in float64: decode(code) * scale of its group."""
    c = np.asarray(codes)
    n = c.shape[-1]
    d = e4m3.decode(c).reshape(c.shape[:-1] + (n // GROUP, GROUP))
    return (d * np.asarray(scales, dtype=np.float64)[..., None]).reshape(c.shape)


def dequant_blocks(codes, scales) -> np.ndarray:
    """[N, K] e4m3 codes with [ceil(N/128), ceil(K/128)] fp32 block scales -> float64."""
    c = np.asarray(codes)
    N, K = c.shape
    s = np.asarray(scales, dtype=np.float64)
    full = np.repeat(np.repeat(s, GROUP, axis=0), GROUP, axis=1)[:N, :K]
    return e4m3.decode(c) * full


# ----------------------------------------------------------------------------- weights

class ExpertWeights:
    """Per-expert float64 view of packed weights (f32/bf16 values, or fp8 codes + scales)."""

    def __init__(self, w13, w2, w13_scale=None, w2_scale=None):
        self.w13, self.w2 = w13, w2
        self.s13, self.s2 = w13_scale, w2_scale
        self.fp8 = w13_scale is not None
        self.E = w13.shape[0]
        self.I = w2.shape[2]
        self.H = w2.shape[1]

    def gate_up(self, e: int) -> np.ndarray:
        if self.fp8:
            return dequant_blocks(self.w13[e], self.s13[e])
        return np.asarray(self.w13[e], dtype=np.float64)

    def down(self, e: int) -> np.ndarray:
        if self.fp8:
            return dequant_blocks(self.w2[e], self.s2[e])
        return np.asarray(self.w2[e], dtype=np.float64)


def expert_h(xe: np.ndarray, w13e: np.ndarray, I: int) -> np.ndarray:
    """h = SiLU(x Wg^T) * (x Wu^T) in float64."""
    gate = xe @ w13e[:I].T
    up = xe @ w13e[I:].T
    return silu(gate) * up


# ----------------------------------------------------------------------------- the layer

def permute_rows(x, sorted_rows, offsets, k: int):
    """Permuted position p < offsets[E] holds token row sorted_rows[p] // k."""
    V = int(offsets[-1])
    return np.asarray(x)[np.asarray(sorted_rows[:V], dtype=np.int64) // k]


def grouped_ffn(xp, offsets, W: ExpertWeights, R: int):
    """Per-expert loop over segments [offsets[e], offsets[e+1]) of the permuted rows.

    ``xp`` is float64 [V, H] (fp8: the dequantised permuted activations).
    Returns h [R, I] and y [R, H] in float64 (fp8: h is the dequantised
    quantised h, and also returned as codes + scales), with rows >= V zero.
    """
    E, H, I = W.E, W.H, W.I
    V = int(offsets[-1])
    h = np.zeros((R, I), dtype=np.float64)
    y = np.zeros((R, H), dtype=np.float64)
    hq = np.zeros((R, I), dtype=np.uint8) if W.fp8 else None
    hs = np.ones((R, I // GROUP), dtype=np.float32) if W.fp8 else None
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a == b:
            continue
        he = expert_h(xp[a:b], W.gate_up(e), I)
        if W.fp8:
            q, s = quant128(he.astype(np.float32))
            hq[a:b], hs[a:b] = q, s
            he = dequant128(q, s)
        h[a:b] = he
        y[a:b] = he @ W.down(e).T
    assert V <= R
    return h, y, hq, hs


def combine(y, row_pos, flat_ids, flat_w, T: int, k: int, E: int):
    """out[t] = sum over slots j (ascending) with a valid row of w[t,j] * y[row_pos[t*k+j]]."""
    H = y.shape[1]
    out = np.zeros((T, H), dtype=np.float64)
    for j in range(k):
        r = np.arange(T) * k + j
        valid = (flat_ids[r] >= 0) & (flat_ids[r] < E)
        contrib = flat_w[r].astype(np.float64)[:, None] * y[row_pos[r]]
        out += np.where(valid[:, None], contrib, 0.0)
    return out


def forward(x, logits, W: ExpertWeights, k: int, num_valid_rows: int = -1,
            renormalize: bool = True) -> dict:
    """The whole layer.  ``x`` [T, H] holds the stored input values (f32, or bf16 values as floats)."""
    x = np.asarray(x, dtype=np.float32)
    T, H = x.shape
    E = W.E
    R = T * k
    ids, w = route_topk(logits, k, num_valid_rows, renormalize)
    flat_ids, flat_w = ids.reshape(-1), w.reshape(-1)
    offsets, sorted_rows, row_pos = build_offsets(flat_ids, E)
    res = dict(ids=ids, w=w, offsets=offsets, sorted_rows=sorted_rows, row_pos=row_pos)
    if W.fp8:
        xq, xs = quant128(x)                     # per token, before permuting
        xq_p = permute_rows(xq, sorted_rows, offsets, k)
        xs_p = permute_rows(xs, sorted_rows, offsets, k)
        xp = dequant128(xq_p, xs_p)
        res.update(xq=xq, xs=xs, xq_perm=xq_p, xs_perm=xs_p)
    else:
        xp = permute_rows(x, sorted_rows, offsets, k).astype(np.float64)
        res.update(x_perm=xp)
    h, y, hq, hs = grouped_ffn(xp, offsets, W, R)
    res.update(h=h, y=y, hq=hq, hs=hs)
    res["out"] = combine(y, row_pos, flat_ids, flat_w, T, k, E)
    return res


# ----------------------------------------------------------------------------- one token at a time

def token_output(x_t, ids_t, w_t, W: ExpertWeights, weight_cache: dict | None = None) -> np.ndarray:
    """Output of one token from its routed slots (sentinel slots skipped).

    Same definition as ``forward`` evaluated for a single token; used to check
    sampled tokens of layers too large to run whole.
    """
    E, I = W.E, W.I
    x_t = np.asarray(x_t, dtype=np.float32)
    if W.fp8:
        q, s = quant128(x_t[None, :])
        xv = dequant128(q, s)[0]
    else:
        xv = x_t.astype(np.float64)
    out = np.zeros(W.H, dtype=np.float64)
    for e, wt in zip(ids_t, w_t):
        e = int(e)
        if not (0 <= e < E):
            continue
        if weight_cache is not None and e in weight_cache:
            w13e, w2e = weight_cache[e]
        else:
            w13e, w2e = W.gate_up(e), W.down(e)
            if weight_cache is not None:
                weight_cache[e] = (w13e, w2e)
        h = expert_h(xv[None, :], w13e, I)
        if W.fp8:
            hq, hs = quant128(h.astype(np.float32))
            h = dequant128(hq, hs)
        out += float(wt) * (h @ w2e.T)[0]
    return out


def sampled_outputs(x_rows, ids_rows, w_rows, W: ExpertWeights) -> np.ndarray:
    """Outputs of a few tokens (rows of x with their routed ids and weights).

    The same definition as ``token_output``, organised by expert so that each
    expert's weights are converted once: for every expert used by the sample,
    h and the expert output are computed for the sample rows routed to it;
    each token then sums its slots in ascending order.
    """
    x_rows = np.asarray(x_rows, dtype=np.float32)
    S, H = x_rows.shape
    k = np.asarray(ids_rows).shape[1]
    E, I = W.E, W.I
    if W.fp8:
        q, s = quant128(x_rows)
        xv = dequant128(q, s)
    else:
        xv = x_rows.astype(np.float64)
    y = np.zeros((S, k, H), dtype=np.float64)
    ids_rows = np.asarray(ids_rows)
    for e in sorted(set(int(v) for v in ids_rows.reshape(-1) if 0 <= v < E)):
        sel = np.argwhere(ids_rows == e)              # (sample, slot) pairs routed to e
        h = expert_h(xv[sel[:, 0]], W.gate_up(e), I)
        if W.fp8:
            hq, hs = quant128(h.astype(np.float32))
            h = dequant128(hq, hs)
        y[sel[:, 0], sel[:, 1]] = h @ W.down(e).T
    out = np.zeros((S, H), dtype=np.float64)
    for j in range(k):
        valid = (ids_rows[:, j] >= 0) & (ids_rows[:, j] < E)
        out += np.where(valid[:, None], np.asarray(w_rows, np.float64)[:, j:j + 1] * y[:, j], 0.0)
    return out


def layer_forward_dense_inputs(inputs) -> dict:
    """Convenience: run ``forward`` on a workloads.LayerInputs (tensors on the CPU)."""
    import torch  # plain tensor-to-array conversion only
    cfg = inputs.cfg

    def f32(t):
        return t.detach().to("cpu", torch.float32).numpy()

    if cfg.dtype == "fp8":
        W = ExpertWeights(inputs.w13.cpu().view(torch.uint8).numpy(),
                          inputs.w2.cpu().view(torch.uint8).numpy(),
                          inputs.w13_scale.cpu().numpy(), inputs.w2_scale.cpu().numpy())
    else:
        W = ExpertWeights(f32(inputs.w13), f32(inputs.w2))
    return forward(f32(inputs.x), f32(inputs.logits), W, cfg.k, cfg.num_valid_rows,
                   cfg.renormalize)
