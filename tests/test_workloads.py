"""The seeded generators: determinism, shapes, distributions."""
import numpy as np
import pytest
import torch

from workloads import CONFIGS, generate, get_config, small_variant, quantize_weight_blocks


def test_configs_present():
    assert {"tiny_f32", "gptoss20b_bf16", "sweep_bf16_v16384", "sweep_bf16_v8192",
            "sweep_bf16_v2048", "mixtral8x7b_bf16", "deepseekv3_fp8"} <= set(CONFIGS)
    c = get_config("gptoss20b_bf16")
    assert (c.T, c.H, c.I, c.E, c.k) == (4096, 2880, 2880, 32, 4)
    assert abs(c.gemm_flops() - 815.4e9) / 815.4e9 < 1e-3


def test_tiny_deterministic_and_shaped():
    cfg = get_config("tiny_f32")
    a, b = generate(cfg, "cpu"), generate(cfg, "cpu")
    for n in ("x", "logits", "w13", "w2"):
        assert torch.equal(getattr(a, n), getattr(b, n))
    assert a.x.shape == (64, 128) and a.w13.shape == (8, 512, 128) and a.w2.shape == (8, 128, 256)
    assert abs(a.w13.std().item() - 0.02) < 1e-3
    c = generate(cfg, "cpu", seed=1)
    assert not torch.equal(a.x, c.x)


def test_small_bf16_and_bias():
    cfg = small_variant(get_config("mixtral8x7b_bf16"), 64).replace(H=256, I=128)
    a = generate(cfg, "cpu")
    assert a.x.dtype == torch.bfloat16 and a.w13.dtype == torch.bfloat16
    assert a.logits.dtype == torch.float32


def test_fp8_weight_blocks():
    torch.manual_seed(0)
    w = torch.randn(300, 260) * 0.02
    q, s = quantize_weight_blocks(w)
    assert q.dtype == torch.float8_e4m3fn and s.shape == (3, 3)
    deq = q.float() * s.repeat_interleave(128, 0).repeat_interleave(128, 1)[:300, :260]
    assert (deq - w).abs().max() <= 16 * s.max()   # half an e4m3 ulp at 256..448 is 16
    assert torch.isfinite(deq).all()


def test_sweep_valid_rows_scale():
    c = small_variant(get_config("sweep_bf16_v2048"), 256)
    assert c.R == 2048 and c.V == 256
