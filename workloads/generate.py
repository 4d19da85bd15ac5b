"""Seeded generation of a layer's input tensors.

Every tensor is drawn from its own ``torch.Generator`` seeded with
``(seed << 8) | tensor_id`` (1 hidden states, 2 router logits, 3 per-expert
logit bias, 4 gate/up weights, 5 down weights), so each tensor can be
regenerated on its own.  Draws are fp32 standard normals; weights are scaled
by 0.02.  bf16 tensors are rounded to nearest-even by torch's cast.

fp8 weights (the DeepSeek-V3-shaped workload) are prepared here once, as
input preparation: each 128x128 block of an expert's fp32 weights gets the
scale ``amax/448`` (1 for an all-zero block) and its values are cast to OCP
e4m3 by torch after clamping to the format's range.  The layer itself (both
the HIP path and the oracle) consumes these codes and scales as given.

Values depend on the device the generator runs on (torch's CPU and GPU
generators differ); a test or benchmark draws once and hands the same tensors
to both sides.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import Optional

import torch

from .configs import LayerConfig

FP8_MAX = 448.0
BLOCK = 128

TID_HIDDEN, TID_LOGITS, TID_BIAS, TID_W13, TID_W2 = 1, 2, 3, 4, 5


@dataclass
class LayerInputs:
    cfg: LayerConfig
    x: torch.Tensor                 # [T, H]  f32 or bf16
    logits: torch.Tensor            # [T, E]  f32
    w13: torch.Tensor               # [E, 2I, H]  f32 / bf16 / float8_e4m3fn
    w2: torch.Tensor                # [E, H, I]
    w13_scale: Optional[torch.Tensor] = None   # [E, 2I/128, H/128] f32 (fp8 only)
    w2_scale: Optional[torch.Tensor] = None    # [E, H/128, I/128]  f32 (fp8 only)

    def to(self, device) -> "LayerInputs":
        mv = lambda t: None if t is None else t.to(device)
        return LayerInputs(self.cfg, mv(self.x), mv(self.logits), mv(self.w13), mv(self.w2),
                           mv(self.w13_scale), mv(self.w2_scale))


def _gen(device, seed: int, tid: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((int(seed) << 8) | int(tid))
    return g


def _act_dtype(cfg: LayerConfig) -> torch.dtype:
    return torch.float32 if cfg.dtype == "f32" else torch.bfloat16


def quantize_weight_blocks(w: torch.Tensor):
    """fp32 [N, K] -> (e4m3 codes [N, K], fp32 scales [ceil(N/128), ceil(K/128)])."""
    N, K = w.shape
    nb, kb = -(-N // BLOCK), -(-K // BLOCK)
    wp = torch.zeros(nb * BLOCK, kb * BLOCK, dtype=torch.float32, device=w.device)
    wp[:N, :K] = w
    blk = wp.view(nb, BLOCK, kb, BLOCK)
    amax = blk.abs().amax(dim=(1, 3))
    s = torch.where(amax > 0, amax / FP8_MAX, torch.ones_like(amax))
    q = (blk / s[:, None, :, None]).clamp_(-FP8_MAX, FP8_MAX)
    q = q.view(nb * BLOCK, kb * BLOCK)[:N, :K].to(torch.float8_e4m3fn)
    return q.contiguous(), s.contiguous()


def generate(cfg: LayerConfig, device="cpu", seed: Optional[int] = None) -> LayerInputs:
    seed = cfg.seed if seed is None else seed
    T, H, I, E = cfg.T, cfg.H, cfg.I, cfg.E
    adt = _act_dtype(cfg)

    x = torch.randn(T, H, generator=_gen(device, seed, TID_HIDDEN), device=device,
                    dtype=torch.float32).to(adt)
    logits = torch.randn(T, E, generator=_gen(device, seed, TID_LOGITS), device=device,
                         dtype=torch.float32)
    if cfg.logit_bias:
        bias = torch.randn(E, generator=_gen(device, seed, TID_BIAS), device=device,
                           dtype=torch.float32)
        logits = logits + bias[None, :]

    g13 = _gen(device, seed, TID_W13)
    g2 = _gen(device, seed, TID_W2)
    if cfg.dtype == "fp8":
        if H % BLOCK or I % BLOCK:
            raise ValueError("fp8 workloads need H and I to be multiples of 128")
        w13 = torch.empty(E, 2 * I, H, dtype=torch.float8_e4m3fn, device=device)
        w2 = torch.empty(E, H, I, dtype=torch.float8_e4m3fn, device=device)
        s13 = torch.empty(E, 2 * I // BLOCK, H // BLOCK, dtype=torch.float32, device=device)
        s2 = torch.empty(E, H // BLOCK, I // BLOCK, dtype=torch.float32, device=device)
        for e in range(E):
            a = torch.randn(2 * I, H, generator=g13, device=device, dtype=torch.float32) * 0.02
            w13[e], s13[e] = quantize_weight_blocks(a)
            b = torch.randn(H, I, generator=g2, device=device, dtype=torch.float32) * 0.02
            w2[e], s2[e] = quantize_weight_blocks(b)
        return LayerInputs(cfg, x, logits, w13, w2, s13, s2)

    wdt = adt
    w13 = torch.empty(E, 2 * I, H, dtype=wdt, device=device)
    w2 = torch.empty(E, H, I, dtype=wdt, device=device)
    for e in range(E):
        w13[e] = (torch.randn(2 * I, H, generator=g13, device=device, dtype=torch.float32)
                  * 0.02).to(wdt)
        w2[e] = (torch.randn(H, I, generator=g2, device=device, dtype=torch.float32)
                 * 0.02).to(wdt)
    return LayerInputs(cfg, x, logits, w13, w2)
