"""Whole-layer parity (moe_forward through the C ABI) against the oracle.

Small variants of every workload and every workload at its full size (in the
launch configuration the benchmark times) run whole through the oracle and are
compared element by element: routing, offsets and permutation bit-exact over
all rows, outputs within the dtype's row-normalised tolerance, sentinel-only
tokens exactly zero.
"""
import numpy as np
import pytest
import torch

from helpers import TOL, HostExperts, np32, row_rel_err, say
from oracle import layer as olayer
from oracle.layer import ExpertWeights
from workloads import generate, get_config, small_variant

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# Reduced-width variants: same E, k, routing structure and dtype; widths keep
# ragged tails for the 64/128-column tiles and the 128-byte K slices.
SMALL = {
    "tiny_f32": dict(T=64),
    "gptoss20b_bf16": dict(T=512, H=712, I=456),
    "sweep_bf16_v16384": dict(T=256, H=512, I=192),
    "sweep_bf16_v8192": dict(T=256, H=512, I=192),
    "sweep_bf16_v2048": dict(T=256, H=512, I=192),
    "mixtral8x7b_bf16": dict(T=512, H=384, I=1408),
    "deepseekv3_fp8": dict(T=256, H=512, I=256, E=32),
}


def _small_cfg(name):
    base = get_config(name)
    kw = dict(SMALL[name])
    cfg = small_variant(base, kw.pop("T"))
    return cfg.replace(**kw)


def _weights_host(inp):
    if inp.cfg.dtype == "fp8":
        return ExpertWeights(HostExperts(inp.w13), HostExperts(inp.w2),
                             inp.w13_scale.cpu().numpy(), inp.w2_scale.cpu().numpy())
    return ExpertWeights(HostExperts(inp.w13), HostExperts(inp.w2))


def _run(inp, **kw):
    import grouped_gemm_histogram_amd as g
    cfg = inp.cfg
    out, aux = g.forward(inp.x, inp.logits, inp.w13, inp.w2, cfg.k, cfg.num_valid_rows,
                         cfg.renormalize, inp.w13_scale, inp.w2_scale, return_aux=True, **kw)
    torch.cuda.synchronize()
    return out, aux


def _check_routing(aux, ref):
    assert np.array_equal(aux.topk_ids.cpu().numpy(), ref["ids"])
    np.testing.assert_allclose(aux.topk_weights.cpu().numpy(), ref["w"], rtol=1e-5, atol=1e-7)
    assert np.array_equal(aux.offsets.cpu().numpy(), ref["offsets"])
    assert np.array_equal(aux.sorted_rows.cpu().numpy(), ref["sorted_rows"])
    assert np.array_equal(aux.row_pos.cpu().numpy(), ref["row_pos"])


@pytest.mark.parametrize("name", list(SMALL))
def test_layer_small(name):
    cfg = _small_cfg(name)
    say(f"layer small {cfg}")
    inp = generate(cfg, "cpu")
    dev = inp.to(DEV)
    out, aux = _run(dev)
    ref = olayer.forward(np32(inp.x), inp.logits.numpy(), _weights_host(inp), cfg.k,
                         cfg.num_valid_rows, cfg.renormalize)
    _check_routing(aux, ref)
    got = np32(out)
    dead = np.all(ref["out"] == 0, axis=1)
    assert np.all(got[dead] == 0)
    err = row_rel_err(got[~dead], ref["out"][~dead])
    say(f"  max row-relative error {err:.3e} (tolerance {TOL[cfg.dtype]})")
    assert err <= TOL[cfg.dtype]
    # determinism: a second run is bitwise identical
    out2, _ = _run(dev)
    assert torch.equal(out.cpu().view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32),
                       out2.cpu().view(torch.int16 if out.dtype == torch.bfloat16 else torch.int32))


def test_layer_sentinel_poison():
    """NaN in the inputs of all-sentinel tokens and in every output/workspace byte changes nothing."""
    cfg = _small_cfg("sweep_bf16_v2048")
    say(f"layer poison {cfg}")
    inp = generate(cfg, "cpu").to(DEV)
    import grouped_gemm_histogram_amd as g
    base, _ = _run(inp)
    V = cfg.V
    x = inp.x.clone()
    x[(V + cfg.k - 1) // cfg.k:] = float("nan")
    need = g.forward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, inp.w13.dtype)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    out = torch.full_like(base, float("nan"))
    g.forward(x, inp.logits, inp.w13, inp.w2, cfg.k, cfg.num_valid_rows, out=out, workspace=ws)
    torch.cuda.synchronize()
    dead = torch.arange(cfg.T, device=DEV) * cfg.k >= V
    assert (out[dead] == 0).all()
    assert torch.equal(out[~dead].view(torch.int16), base[~dead].view(torch.int16))


@pytest.mark.parametrize("T,nv", [(512, 3001), (512, -1), (511, 2999)])
def test_layer_fp8_scale_copies(T, nv):
    """fp8 token scales reach the routed positions by the gather pass (R = T*k >= 4096) or
    by the quantising kernel's per-slot stores (below): both compared whole, with sentinel
    rows and a workspace filled with NaN bytes beforehand."""
    import grouped_gemm_histogram_amd as g
    cfg = small_variant(get_config("deepseekv3_fp8"), T).replace(H=512, I=256, E=32, num_valid_rows=nv)
    say(f"layer fp8 scale copies {cfg}: R={cfg.T * cfg.k}")
    inp = generate(cfg, "cpu")
    dev = inp.to(DEV)
    need = g.forward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, dev.w13.dtype)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)
    out, aux = g.forward(dev.x, dev.logits, dev.w13, dev.w2, cfg.k, cfg.num_valid_rows, cfg.renormalize,
                         dev.w13_scale, dev.w2_scale, workspace=ws, return_aux=True)
    torch.cuda.synchronize()
    ref = olayer.forward(np32(inp.x), inp.logits.numpy(), _weights_host(inp), cfg.k,
                         cfg.num_valid_rows, cfg.renormalize)
    _check_routing(aux, ref)
    got = np32(out)
    dead = np.all(ref["out"] == 0, axis=1)
    assert np.all(got[dead] == 0)
    err = row_rel_err(got[~dead], ref["out"][~dead])
    say(f"  max row-relative error {err:.3e} (tolerance {TOL[cfg.dtype]})")
    assert err <= TOL[cfg.dtype]


# Routing shapes of the layer path above decode sizes (routing and per-chunk histograms in one
# launch, chunks of 16 tokens): token counts off the chunk size, one expert, 1024 experts,
# k = 16 (256-row chunks), odd k (ragged 64-row steps), tied logits, partial and empty
# valid-row prefixes, and more chunks than one pass of the per-bin scan covers; narrow
# widths keep the GEMMs cheap.
ROUTING_SHAPES = [
    # T, E, k, num_valid_rows, tied logits
    (17, 1, 1, -1, False),
    (1000, 1024, 16, -1, True),
    (333, 65, 3, 500, False),
    (4100, 8, 2, -1, True),
    (20, 256, 16, 0, False),
    (77, 40, 5, 301, True),
    (130, 300, 9, -1, False),
    # more than 1024 chunks of 16 tokens: the per-bin scan runs several passes with a carry
    (20000, 64, 2, -1, False),
    (40000, 1024, 16, 300000, True),
]


@pytest.mark.parametrize("T,E,k,nv,ties", ROUTING_SHAPES)
def test_layer_routing_shapes(T, E, k, nv, ties):
    cfg = small_variant(get_config("gptoss20b_bf16"), T, "_route").replace(
        H=128, I=128, E=E, k=k, num_valid_rows=nv)
    say(f"layer routing shapes T={T} E={E} k={k} nv={nv} ties={ties}")
    inp = generate(cfg, "cpu")
    if ties:
        lg = torch.round(inp.logits * 2) / 2
        zero = lg == 0
        lg[zero] = torch.where(torch.rand(int(zero.sum()), generator=torch.Generator().manual_seed(T)) < 0.5,
                               -0.0, 0.0)
        inp.logits = lg.contiguous()
    dev = inp.to(DEV)
    out, aux = _run(dev)
    ref = olayer.forward(np32(inp.x), inp.logits.numpy(), _weights_host(inp), cfg.k,
                         cfg.num_valid_rows, cfg.renormalize)
    _check_routing(aux, ref)
    got = np32(out)
    dead = np.all(ref["out"] == 0, axis=1)
    assert np.all(got[dead] == 0)
    if (~dead).any():
        assert row_rel_err(got[~dead], ref["out"][~dead]) <= TOL[cfg.dtype]


def test_layer_no_valid_rows():
    cfg = _small_cfg("gptoss20b_bf16").replace(num_valid_rows=0)
    inp = generate(cfg, "cpu").to(DEV)
    out, aux = _run(inp)
    assert (out == 0).all()
    assert aux.offsets.cpu().tolist() == [0] * (cfg.E + 1)


def test_layer_top1_unit_weight_is_expert_ffn():
    cfg = _small_cfg("mixtral8x7b_bf16").replace(k=1)
    say(f"layer top-1 {cfg}")
    inp = generate(cfg, "cpu")
    out, aux = _run(inp.to(DEV))
    assert (aux.topk_weights == 1.0).all()
    W = _weights_host(inp)
    ids = aux.topk_ids.cpu().numpy()
    x = np32(inp.x)
    ref = np.zeros((cfg.T, cfg.H))
    for e in range(cfg.E):
        rows = np.nonzero(ids[:, 0] == e)[0]
        if rows.size:
            ref[rows] = olayer.expert_h(x[rows].astype(np.float64), W.gate_up(e), cfg.I) @ W.down(e).T
    assert row_rel_err(np32(out), ref) <= TOL["bf16"]


# ------------------------------------------------------------------------------ decode sizes

DECODE = [
    # workload, T, width overrides; at most 8 routed rows per expert -> 16-row decode tiles
    ("gptoss20b_bf16", 1, {}), ("gptoss20b_bf16", 3, {}), ("gptoss20b_bf16", 16, {}),
    ("gptoss20b_bf16", 64, {}),
    # skewed loads (per-expert logit bias): one expert spans several 16-row tiles
    ("mixtral8x7b_bf16", 32, dict(H=384, I=1408)),
    # fp8: decode tiles with f32 h quantised in a second pass
    ("deepseekv3_fp8", 4, dict(H=512, I=256, E=32)),
    ("deepseekv3_fp8", 1, {}),
    # sentinel rows in the one-launch routing + offsets path: a valid prefix ending inside a
    # token's slots, and no valid row at all
    ("gptoss20b_bf16", 8, dict(num_valid_rows=13)),
    ("deepseekv3_fp8", 4, dict(H=512, I=256, E=32, num_valid_rows=0)),
]


@pytest.mark.parametrize("name,T,kw", DECODE)
def test_layer_decode_sizes(name, T, kw):
    import grouped_gemm_histogram_amd as g
    cfg = small_variant(get_config(name), T, "_decode").replace(**kw)
    say(f"layer decode {cfg.name}: T={T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}")
    inp = generate(cfg, DEV)
    assert g.grouped_gemm_tile_shape(inp.w13.dtype, "silu_mul", cfg.R, cfg.E, torch.float32)[0] == 16
    out, aux = _run(inp)
    ref = olayer.forward(np32(inp.x), inp.logits.cpu().numpy(), _weights_host(inp), cfg.k,
                         cfg.num_valid_rows, cfg.renormalize)
    _check_routing(aux, ref)
    if name.startswith("mixtral"):
        assert np.diff(ref["offsets"]).max() > 16          # the skew case covers several m-tiles
    dead = np.all(ref["out"] == 0, axis=1)                 # tokens with no valid row: exact zeros
    assert np.all(np32(out)[dead] == 0)
    err = row_rel_err(np32(out), ref["out"])
    say(f"  max row-relative error {err:.3e}")
    assert err <= TOL[cfg.dtype]


# ------------------------------------------------------------------------------ full size

FULL = ["gptoss20b_bf16", "sweep_bf16_v16384", "sweep_bf16_v8192", "sweep_bf16_v2048",
        "mixtral8x7b_bf16", "deepseekv3_fp8"]


@pytest.mark.parametrize("name", FULL)
def test_layer_full_size(name):
    """Every workload at its full size, in the launch configuration the benchmark times,
    compared whole: routing, offsets and permutation bit-exact over all rows, and every
    token's output against the oracle's per-expert loop (weights fetched one expert at a
    time), sentinel-only tokens exactly zero."""
    cfg = get_config(name)
    say(f"layer full {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} V={cfg.V}")
    inp = generate(cfg, DEV)
    out, aux = _run(inp)
    got = np32(out)
    x_host = np32(inp.x)
    del out
    ref = olayer.forward(x_host, inp.logits.cpu().numpy(), _weights_host(inp), cfg.k,
                         cfg.num_valid_rows, cfg.renormalize)
    _check_routing(aux, ref)
    assert int(ref["offsets"][-1]) == cfg.V
    dead = (np.arange(cfg.T) * cfg.k) >= cfg.V
    assert np.all(got[dead] == 0)
    assert np.all(ref["out"][dead] == 0)
    err = row_rel_err(got[~dead], ref["out"][~dead])
    say(f"  all {int((~dead).sum())} tokens with valid rows: max row-relative error {err:.3e} "
        f"(tolerance {TOL[cfg.dtype]})")
    assert err <= TOL[cfg.dtype]
