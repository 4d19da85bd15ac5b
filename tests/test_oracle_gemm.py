"""Pins for the oracle's stand-alone grouped GEMM."""
import numpy as np
import torch

from oracle import gemm, layer, routing
from oracle.layer import ExpertWeights


def test_single_group_is_plain_product_and_textbook_swiglu():
    rng = np.random.default_rng(0)
    A = rng.standard_normal((9, 20))
    B = rng.standard_normal((1, 12, 20))
    off = np.array([0, 9])
    C = gemm.grouped_gemm(A, B, off)
    # explicit triple loop on a tiny case
    ref = np.zeros((9, 12))
    for i in range(9):
        for j in range(12):
            s = 0.0
            for k in range(20):
                s += A[i, k] * B[0, j, k]
            ref[i, j] = s
    np.testing.assert_allclose(C, ref, rtol=1e-13, atol=1e-13)
    S = gemm.grouped_gemm(A, B, off, "silu_mul")
    t = torch.from_numpy(A) @ torch.from_numpy(B[0]).T
    np.testing.assert_allclose(S, (torch.nn.functional.silu(t[:, :6]) * t[:, 6:]).numpy(),
                               rtol=1e-13, atol=1e-13)


def test_segments_and_sentinel_rows():
    rng = np.random.default_rng(1)
    A = rng.standard_normal((10, 8))
    B = rng.standard_normal((3, 4, 8))
    off = np.array([0, 3, 3, 7])       # expert 1 empty, rows 7..9 sentinel
    C = gemm.grouped_gemm(A, B, off)
    assert np.all(C[7:] == 0)
    np.testing.assert_allclose(C[0:3], A[0:3] @ B[0].T, rtol=1e-14)
    np.testing.assert_allclose(C[3:7], A[3:7] @ B[2].T, rtol=1e-14)


def test_composition_matches_layer_ffn():
    # gate/up GEMM with SiLU*up, then down GEMM == the layer oracle's per-expert loop
    rng = np.random.default_rng(2)
    T, H, I, E, k = 13, 32, 24, 4, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    w13 = (rng.standard_normal((E, 2 * I, H)) * 0.1).astype(np.float32)
    w2 = (rng.standard_normal((E, H, I)) * 0.1).astype(np.float32)
    res = layer.forward(x, lg, ExpertWeights(w13, w2), k, num_valid_rows=20)
    R = T * k
    xp = np.zeros((R, H))
    xp[:20] = res["x_perm"]
    h = gemm.grouped_gemm(xp, w13, res["offsets"], "silu_mul")
    y = gemm.grouped_gemm(h, w2, res["offsets"])
    np.testing.assert_allclose(h, res["h"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(y, res["y"], rtol=1e-13, atol=1e-15)


def test_fp8_composition_matches_layer_ffn():
    from workloads import quantize_weight_blocks
    rng = np.random.default_rng(3)
    T, H, I, E, k = 6, 256, 128, 3, 2
    x = rng.standard_normal((T, H)).astype(np.float32)
    lg = rng.standard_normal((T, E)).astype(np.float32)
    q13, s13, q2, s2 = [], [], [], []
    for e in range(E):
        a, b = quantize_weight_blocks(torch.randn(2 * I, H, generator=torch.Generator().manual_seed(e)) * 0.05)
        q13.append(a.view(torch.uint8).numpy()); s13.append(b.numpy())
        a, b = quantize_weight_blocks(torch.randn(H, I, generator=torch.Generator().manual_seed(9 + e)) * 0.05)
        q2.append(a.view(torch.uint8).numpy()); s2.append(b.numpy())
    q13, s13, q2, s2 = map(np.stack, (q13, s13, q2, s2))
    res = layer.forward(x, lg, ExpertWeights(q13, q2, s13, s2), k)
    hd, hq, hs = gemm.grouped_gemm(res["xq_perm"], q13, res["offsets"], "silu_mul",
                                   res["xs_perm"], s13, out_fp8=True)
    assert np.array_equal(hq, res["hq"]) and np.array_equal(hs, res["hs"])
    y = gemm.grouped_gemm(hq, q2, res["offsets"], "none", hs, s2)
    np.testing.assert_allclose(y, res["y"], rtol=1e-12, atol=1e-14)
