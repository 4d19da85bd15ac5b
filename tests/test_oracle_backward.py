"""Pins of the backward oracle (CPU only).

The backward is pinned to the forward oracle (itself pinned elsewhere) by
central finite differences: for random directions d, the directional
derivative of L = sum(out * dout) computed from two forward evaluations must
equal <gradient, d>.  Any dropped term, wrong sign, transposed operand or
misrouted row in the backward breaks one of these.  Plus exact invariants:
sentinel slots contribute nothing.
"""

import numpy as np
import pytest

from oracle import backward as ob
from oracle import layer as ol
from oracle import routing as orr


def _problem(seed, T=7, H=8, I=4, E=3, k=2, nv=-1):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H))
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = orr.route_topk(logits, k, nv)
    w13 = rng.standard_normal((E, 2 * I, H)) * 0.5
    w2 = rng.standard_normal((E, H, I)) * 0.5
    dout = rng.standard_normal((T, H))
    return x, ids, w.astype(np.float64), w13, w2, dout


def _loss(x, ids, w, w13, w2, dout):
    """sum(out * dout) of the forward oracle with the routing held fixed."""
    T, H = x.shape
    k = ids.shape[1]
    W = ol.ExpertWeights(w13, w2)
    flat_ids = ids.reshape(-1)
    offsets, sorted_rows, row_pos = orr.build_offsets(flat_ids, W.E)
    xp = ol.permute_rows(x, sorted_rows, offsets, k).astype(np.float64)
    _, y, _, _ = ol.grouped_ffn(xp, offsets, W, T * k)
    out = ol.combine(y, row_pos, flat_ids, w.reshape(-1), T, k, W.E)
    return float(np.sum(out * dout))


@pytest.mark.parametrize("seed,nv", [(0, -1), (1, 9), (2, 4)])
def test_backward_matches_finite_differences(seed, nv):
    x, ids, w, w13, w2, dout = _problem(seed, nv=nv)
    g = ob.backward(x, ids, w, ol.ExpertWeights(w13, w2), dout)
    rng = np.random.default_rng(100 + seed)
    eps = 1e-5
    args = dict(x=x, w=w, w13=w13, w2=w2)
    grads = dict(x=g["dx"], w=g["dw"], w13=g["dw13"], w2=g["dw2"])
    for name in args:
        for _ in range(3):
            d = rng.standard_normal(args[name].shape)
            plus = dict(args, **{name: args[name] + eps * d})
            minus = dict(args, **{name: args[name] - eps * d})
            fd = (_loss(plus["x"], ids, plus["w"], plus["w13"], plus["w2"], dout) -
                  _loss(minus["x"], ids, minus["w"], minus["w13"], minus["w2"], dout)) / (2 * eps)
            an = float(np.sum(grads[name] * d))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def test_backward_sentinels_contribute_nothing():
    # nv = 5 of 14 routed rows valid: the rest are sentinel (id = E)
    x, ids, w, w13, w2, dout = _problem(3, T=7, E=4, k=2, nv=5)
    g = ob.backward(x, ids, w, ol.ExpertWeights(w13, w2), dout)
    E = w13.shape[0]
    sentinel = ids >= E
    assert sentinel.any() and (~sentinel).any()
    assert np.all(g["dw"][sentinel] == 0.0)
    dead_tokens = sentinel.all(axis=1)
    assert dead_tokens.any()
    assert np.all(g["dx"][dead_tokens] == 0.0)
    counts = np.bincount(ids[~sentinel], minlength=E)
    for e in np.flatnonzero(counts == 0):
        assert np.all(g["dw13"][e] == 0.0) and np.all(g["dw2"][e] == 0.0)
    # poisoning the inputs of all-sentinel tokens changes nothing
    x2 = x.copy()
    x2[dead_tokens] = np.nan
    g2 = ob.backward(x2, ids, w, ol.ExpertWeights(w13, w2), dout)
    for key in ("dx", "dw13", "dw2", "dw"):
        a, b = g[key], g2[key]
        if key == "dx":
            a, b = a[~dead_tokens], b[~dead_tokens]
        assert np.array_equal(a, b), key


def test_dsilu_is_the_derivative_of_silu():
    gv = np.linspace(-12, 12, 97)
    eps = 1e-6
    fd = (ol.silu(gv + eps) - ol.silu(gv - eps)) / (2 * eps)
    assert np.max(np.abs(fd - ob.dsilu(gv))) < 1e-8
    assert ob.dsilu(np.array([0.0]))[0] == 0.5          # silu'(0) = sigmoid(0) = 1/2


# ----------------------------------------------------------------------------- fp8 layer

def _fp8_problem(seed, T=7, H=128, I=128, E=3, k=2, nv=-1):
    """Small fp8 layer: e4m3 weight codes with one fp32 scale per 128x128 block."""
    from oracle import e4m3
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    ids, w = orr.route_topk(logits, k, nv)
    q13 = e4m3.encode((rng.standard_normal((E, 2 * I, H)) * 3).astype(np.float32))
    q2 = e4m3.encode((rng.standard_normal((E, H, I)) * 3).astype(np.float32))
    s13 = (rng.random((E, 2 * I // 128, H // 128)) * 0.02 + 0.01).astype(np.float32)
    s2 = (rng.random((E, H // 128, I // 128)) * 0.02 + 0.01).astype(np.float32)
    dout = rng.standard_normal((T, H))
    return x, ids, w.astype(np.float64), ol.ExpertWeights(q13, q2, s13, s2), dout


def _frozen_loss(x, w, w13, w2, ids, dout, cx, ch):
    """sum(out * dout) of the fp8 forward with its quantisation errors frozen: x-hat = x + cx,
    h-hat = h + ch (cx, ch taken at the evaluation point), weights given as dequantised values.
    At the evaluation point this is the fp8 forward; its exact gradient is the
    straight-through gradient."""
    T, H = x.shape
    k = ids.shape[1]
    E, I = w13.shape[0], w2.shape[2]
    flat_ids = ids.reshape(-1)
    offsets, sorted_rows, row_pos = orr.build_offsets(flat_ids, E)
    xp = ol.permute_rows(x + cx, sorted_rows, offsets, k)
    y = np.zeros((T * k, H))
    hs = np.zeros((int(offsets[-1]), I))
    for e in range(E):
        a, b = int(offsets[e]), int(offsets[e + 1])
        if a < b:
            h = ol.expert_h(xp[a:b], w13[e], I)
            hs[a:b] = h
            y[a:b] = (h + (0.0 if ch is None else ch[a:b])) @ w2[e].T
    out = ol.combine(y, row_pos, flat_ids, w.reshape(-1), T, k, E)
    return float(np.sum(out * dout)), hs


@pytest.mark.parametrize("seed,nv", [(0, -1), (1, 9)])
def test_backward_fp8_matches_frozen_error_finite_differences(seed, nv):
    x, ids, w, W, dout = _fp8_problem(seed, nv=nv)
    g = ob.backward_fp8(x, ids, w, W, dout)
    w13 = np.stack([W.gate_up(e) for e in range(W.E)])
    w2 = np.stack([W.down(e) for e in range(W.E)])
    # the quantisation errors at the evaluation point, from the forward's own quantisers
    xq, xs = ol.quant128(x)
    cx = ol.dequant128(xq, xs) - x.astype(np.float64)
    _, h0 = _frozen_loss(x.astype(np.float64), w, w13, w2, ids, dout, cx, None)
    hq, hs = ol.quant128(h0.astype(np.float32))
    ch = ol.dequant128(hq, hs) - h0
    assert np.any(cx != 0) and np.any(ch != 0)          # both quantisers are lossy here
    rng = np.random.default_rng(200 + seed)
    eps = 1e-6
    args = dict(x=x.astype(np.float64), w=w, w13=w13, w2=w2)
    grads = dict(x=g["dx"], w=g["dw"], w13=g["dw13"], w2=g["dw2"])
    for name in args:
        for _ in range(3):
            d = rng.standard_normal(args[name].shape)
            plus = dict(args, **{name: args[name] + eps * d})
            minus = dict(args, **{name: args[name] - eps * d})
            lp, _ = _frozen_loss(plus["x"], plus["w"], plus["w13"], plus["w2"], ids, dout, cx, ch)
            lm, _ = _frozen_loss(minus["x"], minus["w"], minus["w13"], minus["w2"], ids, dout, cx, ch)
            fd = (lp - lm) / (2 * eps)
            an = float(np.sum(grads[name] * d))
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, fd, an)


def test_backward_fp8_forward_intermediates_match_the_forward_oracle():
    """The fp8 backward's x-hat, h-hat and y are the fp8 forward oracle's."""
    x, ids, w, W, dout = _fp8_problem(4)
    g = ob.backward_fp8(x, ids, w, W, dout)
    # the forward oracle routes from logits; here the routing is given, so run its loop directly
    T, k = ids.shape
    flat_ids = ids.reshape(-1)
    off, sr, rp = orr.build_offsets(flat_ids, W.E)
    xq, xs = ol.quant128(x)
    xp = ol.dequant128(ol.permute_rows(xq, sr, off, k), ol.permute_rows(xs, sr, off, k))
    h, y, hq, hs = ol.grouped_ffn(xp, off, W, T * k)
    V = int(off[-1])
    assert np.array_equal(g["h_hat"], h[:V])
    np.testing.assert_allclose(g["y"], y[:V], rtol=1e-12, atol=1e-12)


def test_backward_fp8_sentinels_contribute_nothing():
    x, ids, w, W, dout = _fp8_problem(3, T=7, E=4, k=2, nv=5)
    g = ob.backward_fp8(x, ids, w, W, dout)
    sentinel = ids >= W.E
    assert sentinel.any() and (~sentinel).any()
    assert np.all(g["dw"][sentinel] == 0.0)
    dead_tokens = sentinel.all(axis=1)
    assert dead_tokens.any()
    assert np.all(g["dx"][dead_tokens] == 0.0)
    counts = np.bincount(ids[~sentinel], minlength=W.E)
    for e in np.flatnonzero(counts == 0):
        assert np.all(g["dw13"][e] == 0.0) and np.all(g["dw2"][e] == 0.0)
    x2 = x.copy()
    x2[dead_tokens] = np.nan
    g2 = ob.backward_fp8(x2, ids, w, W, dout)
    for key in ("dx", "dw13", "dw2", "dw"):
        a, b = g[key], g2[key]
        if key == "dx":
            a, b = a[~dead_tokens], b[~dead_tokens]
        assert np.array_equal(a, b), key
