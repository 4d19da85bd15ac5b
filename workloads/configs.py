"""The MoE layer workloads.

Each workload is one expert layer: T tokens of width H, E experts with SwiGLU
FFNs of intermediate width I, top-k routing.  Packed weights follow the
stacked-experts layout the MoE write-up ("트랜스포머에서 전문가 혼합 (MoEs)",
section on WeightConverter / MergeModulelist) describes: one contiguous
tensor per projection, expert-major:

* ``w13``  [E, 2I, H]  rows [0, I) are gate, rows [I, 2I) are up;
* ``w2``   [E, H, I].

Shapes borrow real models (gpt-oss-20b uses 4 of 32 experts per token, per
the same write-up's section on active vs total parameters); values are
synthetic: hidden states and router logits ~ N(0, 1), weights ~ N(0, 0.02).
"""

from __future__ import annotations

import dataclasses
from dataclasses import dataclass


@dataclass(frozen=True)
class LayerConfig:
    name: str
    T: int            # tokens
    H: int            # hidden width (K of gate/up, N of down)
    I: int            # intermediate width (N/2 of gate/up, K of down)
    E: int            # experts; expert id E is the sentinel
    k: int            # experts per token
    dtype: str        # "f32" | "bf16" | "fp8"  (fp8: e4m3 weights + block scales, bf16 activations)
    num_valid_rows: int = -1   # <0: all T*k flat rows valid; else rows r >= V are sentinel
    logit_bias: bool = False   # add a per-expert N(0,1) bias to skew expert loads
    renormalize: bool = True   # softmax over the k selected logits
    seed: int = 0
    description: str = ""

    @property
    def R(self) -> int:
        return self.T * self.k

    @property
    def V(self) -> int:
        return self.R if self.num_valid_rows < 0 else min(self.num_valid_rows, self.R)

    def gemm_flops(self, valid_rows: int | None = None) -> float:
        """Algorithmic flops of both grouped GEMMs: 4*V*H*I (gate/up) + 2*V*H*I (down)."""
        v = self.V if valid_rows is None else valid_rows
        return 6.0 * v * self.H * self.I

    def replace(self, **kw) -> "LayerConfig":
        return dataclasses.replace(self, **kw)


CONFIGS: dict[str, LayerConfig] = {}


def _add(cfg: LayerConfig) -> None:
    CONFIGS[cfg.name] = cfg


_add(LayerConfig(
    "tiny_f32", T=64, H=128, I=256, E=8, k=2, dtype="f32",
    description="tiny fp32 layer, top-2 softmax routing, no sentinels"))
_add(LayerConfig(
    "gptoss20b_bf16", T=4096, H=2880, I=2880, E=32, k=4, dtype="bf16",
    description="gpt-oss-20b-shaped bf16 layer, top-4 of 32, softmax over the selected 4"))
for _v in (16384, 8192, 2048):
    _add(LayerConfig(
        f"sweep_bf16_v{_v}", T=2048, H=2048, I=768, E=128, k=8, dtype="bf16",
        num_valid_rows=_v,
        description=f"sentinel sweep: 16384 routed rows, {_v} valid, rest sentinel (id = E)"))
_add(LayerConfig(
    "mixtral8x7b_bf16", T=8192, H=4096, I=14336, E=8, k=2, dtype="bf16", logit_bias=True,
    description="Mixtral-8x7B-shaped bf16 layer, top-2 of 8, skewed logits (per-expert bias)"))
_add(LayerConfig(
    "deepseekv3_fp8", T=8192, H=7168, I=2048, E=256, k=8, dtype="fp8",
    description="DeepSeek-V3-shaped fp8 layer: e4m3 weights with 128x128 block scales, "
                "activations quantised per token per 128 channels, bf16 output"))


def get_config(name: str) -> LayerConfig:
    return CONFIGS[name]


def small_variant(cfg: LayerConfig, T: int, name_suffix: str = "_small") -> LayerConfig:
    """Same layer with fewer tokens (parity at sizes the oracle finishes quickly).

    For a sentinel workload the valid fraction is kept: V scales with T.
    """
    nv = cfg.num_valid_rows
    if nv >= 0:
        nv = (nv * T) // cfg.T
    return cfg.replace(name=cfg.name + name_suffix, T=T, num_valid_rows=nv)
