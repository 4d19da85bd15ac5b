"""moe_forward captured in a HIP graph (torch.cuda.CUDAGraph) and replayed.

The layer enqueues only kernels on the caller's stream (no allocation, no memset, no
host synchronisation), so a serving loop can capture it once and replay it.  Each
replay is compared bitwise with an eager call on the same inputs, with eager work and
synchronisations between the replays, and again after new inputs are copied into the
captured buffers.
"""
import pytest
import torch

from helpers import say
from workloads import generate, get_config, small_variant

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

CASES = [
    ("gptoss20b_bf16", 1, {}),
    ("gptoss20b_bf16", 64, {}),
    ("gptoss20b_bf16", 512, dict(H=712, I=456)),
    ("deepseekv3_fp8", 4, dict(H=512, I=256, E=32)),
    ("deepseekv3_fp8", 600, dict(H=512, I=256, E=32)),
]


def _bits(t):
    return t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32)


@pytest.mark.parametrize("name,T,kw", CASES)
def test_forward_graph_replay(name, T, kw):
    import grouped_gemm_histogram_amd as g
    cfg = small_variant(get_config(name), T, "_graph").replace(**kw)
    say(f"graph replay {cfg.name}: T={cfg.T} H={cfg.H} I={cfg.I} E={cfg.E} k={cfg.k}")
    inp = generate(cfg, DEV)
    x, logits = inp.x.clone(), inp.logits.clone()       # the captured input buffers

    def eager(xx, ll):
        out = g.forward(xx, ll, inp.w13, inp.w2, cfg.k, cfg.num_valid_rows, cfg.renormalize,
                        inp.w13_scale, inp.w2_scale)
        torch.cuda.synchronize()
        return out

    need = g.forward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, inp.w13.dtype)
    ws = torch.empty(need, dtype=torch.uint8, device=DEV)
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=DEV)

    def step():
        g.forward(x, logits, inp.w13, inp.w2, cfg.k, cfg.num_valid_rows, cfg.renormalize,
                  inp.w13_scale, inp.w2_scale, out=out, workspace=ws)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()                                          # warm-up outside the capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()

    ref = eager(x, logits)
    for i in range(3):
        out.fill_(float("nan"))
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(ref)), f"replay {i}"
        eager(x * 0.5, logits)                          # the program's own work in between

    gen = torch.Generator(device=DEV).manual_seed(7)
    x.copy_(torch.randn(x.shape, generator=gen, device=DEV).to(x.dtype))
    logits.copy_(torch.randn(logits.shape, generator=gen, device=DEV))
    ref2 = eager(x, logits)
    graph.replay()
    torch.cuda.synchronize()
    assert torch.equal(_bits(out), _bits(ref2))
    assert not torch.equal(_bits(ref2), _bits(ref))
