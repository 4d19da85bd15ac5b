"""Backward parity (moe_backward through the C ABI) against the backward oracle.

The routing is the oracle's (computed on the host from the same logits) and is
handed to the GPU, so the oracle never takes an input from the HIP path.
Small bf16 layers and the full-size gpt-oss-20b-shaped layer are compared
whole, element by element.

Tolerance, derived from the arithmetic.  The GPU feeds bf16 operands (dy, h,
dgu and x, each rounded once: relative error <= 2^-9 of the element) to fp32
MFMA accumulation.  An element of a product then errs by about 2^-9 times the
magnitudes summed into it, not times its own value: dh[p, j] = sum_h dy[p, h]
W2[h, j] can nearly cancel, and an element built from it (dgu, and a dW13 row
of an expert with one routed row, which is dgu[p, j] x[p]) then carries that
absolute error on a tiny value.  So every gradient is compared against the
scale of its natural unit: dx per token row (the forward's convention), dW13
and dW2 per expert matrix, the routing-weight gradients over all slots; each
within 2e-2, a few 2^-9 with margin.
"""
import numpy as np
import pytest
import torch

from helpers import HostExperts, np32, row_rel_err, say
from oracle import backward as obwd, routing as orouting
from oracle.layer import ExpertWeights
from workloads import generate, get_config, small_variant

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = 2e-2

SMALL = {
    "gptoss20b_bf16": dict(T=384, H=712, I=456),
    "sweep_bf16_v2048": dict(T=256, H=512, I=192),
    "mixtral8x7b_bf16": dict(T=384, H=384, I=1408),
}


def _cfg(name):
    base = get_config(name)
    kw = dict(SMALL[name])
    return small_variant(base, kw.pop("T")).replace(**kw)


def _dout(T, H, seed):
    g = torch.Generator().manual_seed(seed)
    return torch.randn(T, H, generator=g).to(torch.bfloat16)


def _routing(inp):
    cfg = inp.cfg
    ids, w = orouting.route_topk(inp.logits.cpu().numpy(), cfg.k, cfg.num_valid_rows, cfg.renormalize)
    off, sr, rp = orouting.build_offsets(ids.reshape(-1), cfg.E)
    return ids, w, off, sr, rp


def _nan_workspace(cfg, w_dtype):
    """A backward workspace whose every byte is 0xFF (NaN in any float view)."""
    import grouped_gemm_histogram_amd as g
    need = g.backward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, w_dtype)
    return torch.full((need,), 0xFF, dtype=torch.uint8, device=DEV)


def _gpu_backward(inp, w, off, sr, rp, dout, grad_dtype=torch.float32, workspace=None):
    import grouped_gemm_histogram_amd as g
    T = inp.cfg.T
    gr = g.backward(inp.x, inp.w13, inp.w2, dout.to(DEV),
                    torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).reshape(T, -1).to(DEV),
                    torch.from_numpy(off).to(DEV), torch.from_numpy(sr).to(DEV), torch.from_numpy(rp).to(DEV),
                    grad_dtype=grad_dtype, workspace=workspace)
    torch.cuda.synchronize()
    return gr


def _per_expert(got, ref):
    """max over experts of max|got - ref| / max|ref| over the expert's whole gradient matrix."""
    E = ref.shape[0]
    return row_rel_err(got.reshape(E, -1), ref.reshape(E, -1))


def _weights(inp):
    return ExpertWeights(HostExperts(inp.w13), HostExperts(inp.w2))


@pytest.mark.parametrize("name", list(SMALL))
def test_backward_small_layers(name):
    cfg = _cfg(name)
    say(f"backward {cfg.name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} nv={cfg.num_valid_rows}")
    inp = generate(cfg, DEV)
    ids, w, off, sr, rp = _routing(inp)
    dout = _dout(cfg.T, cfg.H, 21)
    gr = _gpu_backward(inp, w, off, sr, rp, dout)
    ref = obwd.backward(inp.x.float().cpu().numpy(), ids, w, _weights(inp), dout.float().numpy())
    errs = {"dx": row_rel_err(np32(gr.dx), ref["dx"]),
            "dw13": _per_expert(np32(gr.dw13), ref["dw13"]),
            "dw2": _per_expert(np32(gr.dw2), ref["dw2"]),
            "dw": row_rel_err(np32(gr.dtopk_weights).reshape(1, -1), ref["dw"].reshape(1, -1))}
    say(f"  errors {errs}")
    for key, err in errs.items():
        assert err <= TOL, (key, err)
    # sentinel slots: zero routing-weight gradient; tokens with no valid slot: zero dx
    sentinel = ids >= cfg.E
    assert np.all(np32(gr.dtopk_weights)[sentinel] == 0)
    dead = sentinel.all(axis=1)
    assert np.all(np32(gr.dx)[dead] == 0)
    # experts with no rows: exactly zero weight gradients
    empty = np.flatnonzero(np.diff(off) == 0)
    for e in empty:
        assert np.all(np32(gr.dw13)[e] == 0) and np.all(np32(gr.dw2)[e] == 0)


def test_backward_decode_size():
    """A few tokens (at most 8 routed rows per expert): the M-grouped GEMMs take the decode tiles."""
    cfg = small_variant(get_config("gptoss20b_bf16"), 6).replace(H=712, I=456)
    say(f"backward decode-size T={cfg.T} R={cfg.R}")
    inp = generate(cfg, DEV)
    ids, w, off, sr, rp = _routing(inp)
    dout = _dout(cfg.T, cfg.H, 27)
    gr = _gpu_backward(inp, w, off, sr, rp, dout)
    ref = obwd.backward(inp.x.float().cpu().numpy(), ids, w, _weights(inp), dout.float().numpy())
    errs = {"dx": row_rel_err(np32(gr.dx), ref["dx"]),
            "dw13": _per_expert(np32(gr.dw13), ref["dw13"]),
            "dw2": _per_expert(np32(gr.dw2), ref["dw2"]),
            "dw": row_rel_err(np32(gr.dtopk_weights).reshape(1, -1), ref["dw"].reshape(1, -1))}
    say(f"  errors {errs}")
    for key, err in errs.items():
        assert err <= TOL, (key, err)
    for e in np.flatnonzero(np.diff(off) == 0):
        assert np.all(np32(gr.dw13)[e] == 0) and np.all(np32(gr.dw2)[e] == 0)


def test_backward_bf16_grads_and_determinism():
    cfg = _cfg("gptoss20b_bf16")
    inp = generate(cfg, DEV)
    ids, w, off, sr, rp = _routing(inp)
    dout = _dout(cfg.T, cfg.H, 22)
    a = _gpu_backward(inp, w, off, sr, rp, dout, torch.bfloat16)
    b = _gpu_backward(inp, w, off, sr, rp, dout, torch.bfloat16)
    for f in ("dx", "dw13", "dw2", "dtopk_weights"):
        assert torch.equal(getattr(a, f), getattr(b, f)), f
    ref = obwd.backward(inp.x.float().cpu().numpy(), ids, w, _weights(inp), dout.float().numpy())
    assert row_rel_err(np32(a.dx), ref["dx"]) <= TOL
    assert _per_expert(np32(a.dw2), ref["dw2"]) <= TOL
    assert _per_expert(np32(a.dw13), ref["dw13"]) <= TOL


def test_backward_sentinel_rows_are_poison_proof():
    """NaN in the inputs of tokens whose slots are all sentinel, and a workspace of NaN bytes,
    reach no gradient."""
    cfg = _cfg("sweep_bf16_v2048")
    inp = generate(cfg, DEV)
    ids, w, off, sr, rp = _routing(inp)
    dead = (ids >= cfg.E).all(axis=1)
    assert dead.any()
    dout = _dout(cfg.T, cfg.H, 23)
    clean = _gpu_backward(inp, w, off, sr, rp, dout)
    x_p = inp.x.clone()
    x_p[torch.from_numpy(dead).to(DEV)] = float("nan")
    d_p = dout.clone()
    d_p[torch.from_numpy(dead)] = float("nan")
    poisoned = _gpu_backward(inp.__class__(inp.cfg, x_p, inp.logits, inp.w13, inp.w2), w, off, sr, rp, d_p,
                             workspace=_nan_workspace(cfg, torch.bfloat16))
    for f in ("dx", "dw13", "dw2", "dtopk_weights"):
        assert torch.equal(getattr(clean, f), getattr(poisoned, f)), f


def test_backward_no_valid_rows():
    cfg = _cfg("sweep_bf16_v2048").replace(num_valid_rows=0)
    inp = generate(cfg, DEV)
    ids, w, off, sr, rp = _routing(inp)
    assert off[-1] == 0
    gr = _gpu_backward(inp, w, off, sr, rp, _dout(cfg.T, cfg.H, 24))
    for f in ("dx", "dw13", "dw2", "dtopk_weights"):
        assert torch.count_nonzero(getattr(gr, f)).item() == 0, f


def test_backward_full_size():
    """The gpt-oss-20b-shaped layer at full size, every gradient compared whole."""
    cfg = get_config("gptoss20b_bf16")
    say(f"backward full size {cfg.name}")
    inp = generate(cfg, DEV)
    ids, w, off, sr, rp = _routing(inp)
    dout = _dout(cfg.T, cfg.H, 25)
    gr = _gpu_backward(inp, w, off, sr, rp, dout)
    got = {"dx": np32(gr.dx), "dw13": np32(gr.dw13), "dw2": np32(gr.dw2), "dw": np32(gr.dtopk_weights)}
    del gr
    ref = obwd.backward(inp.x.float().cpu().numpy(), ids, w, _weights(inp), dout.float().numpy())
    errs = {"dx": row_rel_err(got["dx"], ref["dx"]),
            "dw13": _per_expert(got["dw13"], ref["dw13"]),
            "dw2": _per_expert(got["dw2"], ref["dw2"]),
            "dw": row_rel_err(got["dw"].reshape(1, -1), ref["dw"].reshape(1, -1))}
    say(f"  errors {errs}")
    for key, err in errs.items():
        assert err <= TOL, (key, err)


# ----------------------------------------------------------------------------- fp8 layer

FP8_SMALL = [
    # the DeepSeek-V3-shaped fp8 layer at reduced width, all rows valid and a third valid
    dict(T=256, H=512, I=256, E=32, nv=-1),
    dict(T=192, H=384, I=384, E=16, nv=192 * 8 // 3),
    # decode size: at most 8 routed rows per expert
    dict(T=6, H=512, I=256, E=32, nv=-1),
]


def _fp8_cfg(T, H, I, E, nv):
    base = get_config("deepseekv3_fp8")
    cfg = small_variant(base, T, "_bwd").replace(H=H, I=I, E=E)
    return cfg.replace(num_valid_rows=nv)


def _fp8_weights(inp):
    return ExpertWeights(HostExperts(inp.w13), HostExperts(inp.w2), inp.w13_scale.cpu().numpy(),
                         inp.w2_scale.cpu().numpy())


def _gpu_backward_fp8(inp, w, off, sr, rp, dout, grad_dtype=torch.float32, x=None, workspace=None):
    import grouped_gemm_histogram_amd as g
    T = inp.cfg.T
    gr = g.backward(inp.x if x is None else x, inp.w13, inp.w2, dout.to(DEV),
                    torch.from_numpy(np.ascontiguousarray(w, dtype=np.float32)).reshape(T, -1).to(DEV),
                    torch.from_numpy(off).to(DEV), torch.from_numpy(sr).to(DEV), torch.from_numpy(rp).to(DEV),
                    grad_dtype=grad_dtype, w13_scale=inp.w13_scale, w2_scale=inp.w2_scale, workspace=workspace)
    torch.cuda.synchronize()
    return gr


@pytest.mark.parametrize("case", FP8_SMALL, ids=lambda c: f"T{c['T']}-H{c['H']}-I{c['I']}-E{c['E']}-nv{c['nv']}")
def test_backward_fp8_layers(case):
    cfg = _fp8_cfg(**case)
    say(f"backward fp8 {cfg.name} T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k} nv={cfg.num_valid_rows}")
    inp = generate(cfg, DEV)
    ids, w, off, sr, rp = _routing(inp)
    dout = _dout(cfg.T, cfg.H, 41)
    gr = _gpu_backward_fp8(inp, w, off, sr, rp, dout)
    ref = obwd.backward_fp8(inp.x.float().cpu().numpy(), ids, w, _fp8_weights(inp), dout.float().numpy())
    errs = {"dx": row_rel_err(np32(gr.dx), ref["dx"]),
            "dw13": _per_expert(np32(gr.dw13), ref["dw13"]),
            "dw2": _per_expert(np32(gr.dw2), ref["dw2"]),
            "dw": row_rel_err(np32(gr.dtopk_weights).reshape(1, -1), ref["dw"].reshape(1, -1))}
    say(f"  errors {errs}")
    for key, err in errs.items():
        assert err <= TOL, (key, err)
    sentinel = ids >= cfg.E
    assert np.all(np32(gr.dtopk_weights)[sentinel] == 0)
    assert np.all(np32(gr.dx)[sentinel.all(axis=1)] == 0)
    for e in np.flatnonzero(np.diff(off) == 0):
        assert np.all(np32(gr.dw13)[e] == 0) and np.all(np32(gr.dw2)[e] == 0)


def test_backward_fp8_poison_and_determinism():
    """NaN in the inputs of all-sentinel tokens and a workspace of NaN bytes reach no gradient;
    reruns are bitwise equal."""
    cfg = _fp8_cfg(T=192, H=384, I=384, E=16, nv=192 * 8 // 3)
    inp = generate(cfg, DEV)
    ids, w, off, sr, rp = _routing(inp)
    dead = (ids >= cfg.E).all(axis=1)
    assert dead.any()
    dout = _dout(cfg.T, cfg.H, 42)
    clean = _gpu_backward_fp8(inp, w, off, sr, rp, dout, torch.bfloat16)
    again = _gpu_backward_fp8(inp, w, off, sr, rp, dout, torch.bfloat16)
    x_p = inp.x.clone()
    x_p[torch.from_numpy(dead).to(DEV)] = float("nan")
    d_p = dout.clone()
    d_p[torch.from_numpy(dead)] = float("nan")
    poisoned = _gpu_backward_fp8(inp, w, off, sr, rp, d_p, torch.bfloat16, x=x_p,
                                 workspace=_nan_workspace(cfg, torch.float8_e4m3fn))
    for f in ("dx", "dw13", "dw2", "dtopk_weights"):
        assert torch.equal(getattr(clean, f), getattr(again, f)), f
        assert torch.equal(getattr(clean, f), getattr(poisoned, f)), f
