"""Pins for the oracle's layer: brute force, closed forms, textbook SwiGLU, invariants."""
import json
import os

import numpy as np
import pytest
import torch

from oracle import brute, layer, routing
from oracle.layer import ExpertWeights
from workloads import generate, get_config

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def rel_err(got, ref):
    """max over tokens of max|got-ref| / max|ref| of that token (rows of zeros compare absolutely)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    scale = np.abs(ref).max(axis=1, keepdims=True)
    scale = np.where(scale == 0, 1.0, scale)
    return float((np.abs(got - ref) / scale).max()) if got.size else 0.0


def _rand_layer(rng, T, H, I, E, fp8=False):
    x = rng.standard_normal((T, H)).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    w13 = (rng.standard_normal((E, 2 * I, H)) * 0.1).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * 0.1).astype(np.float32)
    if not fp8:
        return x, lg, w13, w2, None, None
    from workloads import quantize_weight_blocks
    q13, s13, q2, s2 = [], [], [], []
    for e in range(E):
        a, b = quantize_weight_blocks(torch.from_numpy(w13[e]))
        q13.append(a.view(torch.uint8).numpy()); s13.append(b.numpy())
        a, b = quantize_weight_blocks(torch.from_numpy(w2[e]))
        q2.append(a.view(torch.uint8).numpy()); s2.append(b.numpy())
    return x, lg, np.stack(q13), np.stack(q2), np.stack(s13), np.stack(s2)


def test_golden_tiny_layer():
    d = json.load(open(os.path.join(GOLDEN, "layer_tiny.json")))
    W = ExpertWeights(np.array(d["w13"], np.float32), np.array(d["w2"], np.float32))
    for c in d["cases"]:
        res = layer.forward(np.array(d["x"], np.float32), np.array(d["logits"], np.float32), W,
                            c["k"], c["num_valid_rows"])
        np.testing.assert_allclose(res["out"], np.array(c["out"]), rtol=1e-6, atol=1e-7)


def test_tiny_workload_matches_brute_force():
    cfg = get_config("tiny_f32")
    inp = generate(cfg, "cpu")
    x, lg = inp.x.numpy(), inp.logits.numpy()
    w13, w2 = inp.w13.numpy(), inp.w2.numpy()
    res = layer.forward(x, lg, ExpertWeights(w13, w2), cfg.k)
    ref = brute.dense_forward(x, lg, w13, w2, cfg.k)
    assert rel_err(res["out"], ref) < 1e-12


@pytest.mark.parametrize("seed", range(6))
def test_random_shapes_match_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    E = [1, 2, 3, 8, 5, 4][seed]
    k = int(rng.integers(1, E + 1))
    T = int(rng.integers(1, 20)) * 2 + 1
    H, I = [(16, 32), (24, 8), (64, 48), (32, 256), (128, 16), (40, 40)][seed]
    x, lg, w13, w2, _, _ = _rand_layer(rng, T, H, I, E)
    for nv in (-1, 0, (T * k) // 2, T * k - 1):
        for renorm in (True, False):
            res = layer.forward(x, lg, ExpertWeights(w13, w2), k, nv, renorm)
            ref = brute.dense_forward(x, lg, w13, w2, k, nv, renorm)
            assert rel_err(res["out"], ref) < 1e-12, (nv, renorm)


@pytest.mark.parametrize("E,k,T", [(3, 2, 9), (1, 1, 5), (4, 4, 3)])
def test_fp8_matches_brute_force(E, k, T):
    rng = np.random.default_rng(E * 10 + k)
    x, lg, q13, q2, s13, s2 = _rand_layer(rng, T, 256, 128, E, fp8=True)
    for nv in (-1, T * k // 2):
        res = layer.forward(x, lg, ExpertWeights(q13, q2, s13, s2), k, nv)
        ref = brute.dense_forward(x, lg, q13, q2, k, nv, True, s13, s2)
        assert rel_err(res["out"], ref) < 1e-9


def test_top1_unit_weight_is_per_expert_ffn():
    rng = np.random.default_rng(7)
    T, H, I, E = 23, 32, 48, 5
    x, lg, w13, w2, _, _ = _rand_layer(rng, T, H, I, E)
    res = layer.forward(x, lg, ExpertWeights(w13, w2), 1)
    assert np.all(res["w"] == 1.0)
    xt = torch.from_numpy(x).double()
    for t in range(T):
        e = int(np.argmax(lg[t]))
        wg = torch.from_numpy(w13[e, :I]).double()
        wu = torch.from_numpy(w13[e, I:]).double()
        wd = torch.from_numpy(w2[e]).double()
        ffn = (torch.nn.functional.silu(xt[t] @ wg.T) * (xt[t] @ wu.T)) @ wd.T
        np.testing.assert_allclose(res["out"][t], ffn.numpy(), rtol=1e-12, atol=1e-14)


def test_single_expert_is_textbook_swiglu():
    rng = np.random.default_rng(8)
    T, H, I = 31, 64, 96
    x, lg, w13, w2, _, _ = _rand_layer(rng, T, H, I, 1)
    res = layer.forward(x, lg, ExpertWeights(w13, w2), 1)
    xt = torch.from_numpy(x).double()
    gate = torch.nn.Linear(H, I, bias=False).double()
    up = torch.nn.Linear(H, I, bias=False).double()
    down = torch.nn.Linear(I, H, bias=False).double()
    with torch.no_grad():
        gate.weight.copy_(torch.from_numpy(w13[0, :I]))
        up.weight.copy_(torch.from_numpy(w13[0, I:]))
        down.weight.copy_(torch.from_numpy(w2[0]))
        ref = down(torch.nn.functional.silu(gate(xt)) * up(xt)).numpy()
    np.testing.assert_allclose(res["out"], ref, rtol=1e-12, atol=1e-14)
    assert res["offsets"].tolist() == [0, T]


def test_sentinels_contribute_exactly_zero():
    rng = np.random.default_rng(9)
    T, H, I, E, k = 12, 16, 32, 4, 2
    x, lg, w13, w2, _, _ = _rand_layer(rng, T, H, I, E)
    W = ExpertWeights(w13, w2)
    res0 = layer.forward(x, lg, W, k, 0)
    assert np.all(res0["out"] == 0) and res0["offsets"].tolist() == [0] * (E + 1)
    nv = 9
    res = layer.forward(x, lg, W, k, nv)
    assert np.all(res["h"][nv:] == 0) and np.all(res["y"][nv:] == 0)
    # tokens whose rows are all sentinel: exact zeros; NaN in their inputs changes nothing
    x_nan = x.copy()
    x_nan[(nv + k - 1) // k:] = np.nan
    res_nan = layer.forward(x_nan, lg, W, k, nv)
    full_dead = np.arange(T) * k >= nv
    assert np.all(res_nan["out"][full_dead] == 0)
    assert np.array_equal(res_nan["out"][~full_dead][:-1], res["out"][~full_dead][:-1])


def test_down_weight_scaling_is_exact():
    rng = np.random.default_rng(10)
    x, lg, w13, w2, _, _ = _rand_layer(rng, 15, 32, 16, 3)
    a = layer.forward(x, lg, ExpertWeights(w13, w2), 2)["out"]
    b = layer.forward(x, lg, ExpertWeights(w13, 2 * w2), 2)["out"]
    assert np.array_equal(2 * a, b)


def test_token_permutation_equivariance():
    rng = np.random.default_rng(11)
    x, lg, w13, w2, _, _ = _rand_layer(rng, 21, 32, 16, 4)
    W = ExpertWeights(w13, w2)
    a = layer.forward(x, lg, W, 2)["out"]
    p = rng.permutation(21)
    b = layer.forward(x[p], lg[p], W, 2)["out"]
    assert rel_err(b, a[p]) < 1e-13


def test_token_output_matches_forward():
    rng = np.random.default_rng(12)
    x, lg, q13, q2, s13, s2 = _rand_layer(rng, 7, 128, 256, 3, fp8=True)
    for W in (ExpertWeights(q13, q2, s13, s2),):
        res = layer.forward(x, lg, W, 2, 11)
        ids = res["ids"]
        for t in range(7):
            o = layer.token_output(x[t], ids[t], res["w"][t], W)
            assert rel_err(o[None], res["out"][t][None]) < 1e-12
    x, lg, w13, w2, _, _ = _rand_layer(rng, 7, 32, 16, 3)
    W = ExpertWeights(w13, w2)
    res = layer.forward(x, lg, W, 3)
    for t in range(7):
        o = layer.token_output(x[t], res["ids"][t], res["w"][t], W)
        assert rel_err(o[None], res["out"][t][None]) < 1e-12


def test_quant128_properties():
    rng = np.random.default_rng(13)
    v = (rng.standard_normal((5, 384)) * 3).astype(np.float32)
    v[2, 128:256] = 0
    q, s = layer.quant128(v)
    assert s.shape == (5, 3) and s[2, 1] == 1.0 and np.all(q[2, 128:256] == 0)
    g = v.reshape(5, 3, 128)
    amax = np.abs(g).max(-1)
    nz = amax > 0
    assert np.array_equal(s[nz], (amax / np.float32(448))[nz])
    # the group maximum lands on +-448 (code 0x7E / 0xFE)
    d = layer.dequant128(q, s)
    rel = np.abs(d - v) / np.repeat(s, 128, axis=1)
    assert rel.max() <= 16.0          # half an e4m3 ulp at the top binade (32) in scale units
    np.testing.assert_allclose(np.abs(d).reshape(5, 3, 128).max(-1)[nz], amax[nz], rtol=1e-6)


def test_sampled_outputs_match_forward():
    rng = np.random.default_rng(14)
    for fp8 in (False, True):
        x, lg, a, b, sa, sb = _rand_layer(rng, 9, 128, 128, 4, fp8=fp8)
        W = ExpertWeights(a, b, sa, sb)
        res = layer.forward(x, lg, W, 3, 20)
        pick = np.array([0, 4, 8, 6])
        o = layer.sampled_outputs(x[pick], res["ids"][pick], res["w"][pick], W)
        assert rel_err(o, res["out"][pick]) < 1e-12
