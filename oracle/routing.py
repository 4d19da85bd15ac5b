"""Routing, per-expert histogram, offsets and the stable permutation.

Test infrastructure only (see ``oracle/__init__``).

Layout conventions: flat routed row ``r = t*k + j`` for token t and slot j;
expert id ``E`` marks a sentinel row (unrouted or padding).
"""

from __future__ import annotations

import numpy as np


def route_topk(logits, k: int, num_valid_rows: int = -1, renormalize: bool = True):
    """Top-k routing of each token.

    The router picks a small subset of experts per token ("트랜스포머에서 전문가
    혼합 (MoEs)" write-up, MoE basics section).  Selection: k passes, each
    taking the largest logit not yet taken; equal logits go to the lower
    expert id (numpy's argmax returns the first maximum; -0.0 == +0.0).
    Slot j holds the j-th selection.

    Weights: softmax over the k selected logits when ``renormalize`` (else the
    softmax over all E logits, read at the selected experts), computed in
    float64 and rounded once to float32.

    Flat rows ``r >= num_valid_rows`` (when it is >= 0) become sentinel:
    id = E, weight = 0.

    Returns ``ids`` int32 [T, k] and ``w`` float32 [T, k].
    """
    lg = np.asarray(logits, dtype=np.float32)
    T, E = lg.shape
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    taken = np.zeros((T, E), dtype=bool)
    ids = np.empty((T, k), dtype=np.int64)
    rows = np.arange(T)
    for j in range(k):
        masked = np.where(taken, -np.inf, lg)
        best = np.argmax(masked, axis=1)
        ids[:, j] = best
        taken[rows, best] = True

    sel = np.take_along_axis(lg, ids, axis=1).astype(np.float64)
    if renormalize:
        z = np.exp(sel - sel[:, :1])
        w = z / z.sum(axis=1, keepdims=True)
    else:
        full = lg.astype(np.float64)
        z = np.exp(full - full.max(axis=1, keepdims=True))
        p = z / z.sum(axis=1, keepdims=True)
        w = np.take_along_axis(p, ids, axis=1)

    ids = ids.astype(np.int32)
    w = w.astype(np.float32)
    if num_valid_rows >= 0:
        flat_ids = ids.reshape(-1)
        flat_w = w.reshape(-1)
        flat_ids[num_valid_rows:] = E
        flat_w[num_valid_rows:] = 0.0
    return ids, w


def build_offsets(flat_ids, E: int):
    """Histogram with the sentinel bin left out, exclusive scan, stable permutation.

    The transformers PR #45621 write-up, section 2: sentinel rows are not
    computed; they are left out of the histogram, or sorted as the largest key
    so that they fall to the end, and ``offsets[-1]`` equals the valid-row
    count.  Here both hold at once: ids outside [0, E) count as the sentinel
    key E, ``cnt[e]`` counts only e < E, ``offsets`` = [0, cumsum(cnt)], and
    the permutation is a stable sort by key (rows of one expert keep
    ascending flat order; sentinel rows form the tail, also ascending).

    Returns ``offsets`` int32 [E+1], ``sorted_rows`` int32 [R] (flat row at
    each permuted position) and ``row_pos`` int32 [R] (its inverse).
    """
    ids = np.asarray(flat_ids).astype(np.int64).reshape(-1)
    R = ids.shape[0]
    key = np.where((ids >= 0) & (ids < E), ids, E)
    cnt = np.bincount(key, minlength=E + 1)[:E]
    offsets = np.zeros(E + 1, dtype=np.int64)
    offsets[1:] = np.cumsum(cnt)
    sorted_rows = np.argsort(key, kind="stable")
    row_pos = np.empty(R, dtype=np.int64)
    row_pos[sorted_rows] = np.arange(R)
    return offsets.astype(np.int32), sorted_rows.astype(np.int32), row_pos.astype(np.int32)
