#!/usr/bin/env python3
"""Benchmark of the MoE expert layer (route -> offsets -> gate/up GEMM + SiLU*up
reading token rows through the permutation -> down GEMM -> combine; the fp8
layer quantises token rows first) on one MI355X.

One step = one moe_forward call over the whole synthetic batch, inputs already
resident in HBM.  Prints one JSON line: layer tokens/s (value, from the timed steps,
which record no events), per-stage device times from HIP events recorded by the
library between its stages in a second pass of as many steps, the
grouped GEMMs' MFMA TFLOP/s against the dense peak, the roofline of the
dominant kernel (the gate/up GEMM), and the CPU oracle timed on a bounded
sample of the same workload.

Warm-up (untimed) is at least --warmup steps and at least --warmup-seconds of
work, so the timed steps run at the GPU's steady clock; the JSON "warmup" field
is the number of warm-up steps made.

    python bench.py [--gpus 1] [--steps 20] [--warmup 5] [--workload gptoss20b_bf16]
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks
PEAK_TFLOPS = {"bf16": 2500.0, "fp8": 5000.0, "f32": 157.3}
HBM_PEAK_GBS = 8000.0
METRIC = "MoE layer tokens/s + grouped-GEMM MFMA TFLOP/s (% peak), gpt-oss-20b shape"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gemm_gate_up.json")
GEMM_SRC = os.path.join(ROOT, "grouped_gemm_histogram_amd", "csrc", "gemm.hip")


class HipEvents:
    """A block of hipEvent_t handles (the library records them on its stream)."""

    def __init__(self, n: int):
        self.hip = ctypes.CDLL("libamdhip64.so")
        self.hip.hipEventCreate.argtypes = [ctypes.POINTER(ctypes.c_void_p)]
        self.hip.hipEventElapsedTime.argtypes = [ctypes.POINTER(ctypes.c_float), ctypes.c_void_p,
                                                 ctypes.c_void_p]
        self.hip.hipEventDestroy.argtypes = [ctypes.c_void_p]
        self.ev = []
        for _ in range(n):
            h = ctypes.c_void_p()
            if self.hip.hipEventCreate(ctypes.byref(h)) != 0:
                raise RuntimeError("hipEventCreate failed")
            self.ev.append(h.value)

    def record(self, i: int, stream: int) -> None:
        """Record event i on a HIP stream handle (the stream the library's work is queued on)."""
        self.hip.hipEventRecord.argtypes = [ctypes.c_void_p, ctypes.c_void_p]
        if self.hip.hipEventRecord(self.ev[i], ctypes.c_void_p(stream)) != 0:
            raise RuntimeError("hipEventRecord failed")

    def ms(self, a: int, b: int) -> float:
        out = ctypes.c_float()
        if self.hip.hipEventElapsedTime(ctypes.byref(out), self.ev[a], self.ev[b]) != 0:
            raise RuntimeError("hipEventElapsedTime failed")
        return out.value

    def close(self):
        for h in self.ev:
            self.hip.hipEventDestroy(h)


def source_sha() -> str:
    return hashlib.sha256(open(GEMM_SRC, "rb").read()).hexdigest()[:16]


def load_traffic(workload: str):
    """HBM bytes per gate/up GEMM launch from committed rocprofv3 counter runs, if still current."""
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    entry = d.get(workload)
    if not entry or entry.get("gemm_source_sha") != source_sha():
        return None
    return entry.get("traffic_bytes")


def tokens_with_rows(cfg) -> int:
    """Tokens with at least one valid routed row (valid rows are a prefix of the flat rows)."""
    return min(cfg.T, -(-cfg.V // cfg.k))


def gate_up_bytes(cfg, offsets) -> float:
    """Algorithmic HBM bytes of one gate/up launch: each touched expert's W13 (and its
    block scales) read once, each token row it gathers read once, h written once."""
    H, I, V = cfg.H, cfg.I, cfg.V
    tv = tokens_with_rows(cfg)
    touched = sum(1 for e in range(cfg.E) if offsets[e + 1] > offsets[e])
    if cfg.dtype == "fp8":
        w = touched * (2 * I * H + (2 * I // 128) * (H // 128) * 4)
        return w + tv * H + tv * (H // 128) * 4 + V * I + V * (I // 128) * 4
    esz = 4 if cfg.dtype == "f32" else 2
    return touched * 2 * I * H * esz + tv * H * esz + V * I * esz


def predicted_mfma_flops(offsets, M_rows: int, n_out_total: int, K: int, tile) -> float:
    """MFMA flops the grouped GEMM executes for these offsets: every expert segment is covered by
    ceil(M_e / tile_m) tiles in M, each computing 16*ceil(rows/16) rows, by ceil(N_out / n_out)
    tiles of tile_n weight rows, over ceil(K / k_slice) slices."""
    tile_m, tile_n, k_slice = tile
    n_tiles = -(-n_out_total // tile_n)
    kt = -(-K // k_slice)
    rows = 0
    off = [min(max(int(v), 0), M_rows) for v in offsets]
    for e in range(len(off) - 1):
        m = off[e + 1] - off[e]
        while m > 0:
            r = min(tile_m, m)
            rows += 16 * (-(-r // 16))
            m -= r
    return 2.0 * rows * n_tiles * tile_n * kt * k_slice


def clamp_ab(g, cfg, inp, steps: int) -> dict:
    """Sentinel rows excluded (this layer) vs clamped onto the last expert (the behaviour the
    transformers PR #45621 write-up, section 2, removes): same output, more GEMM rows."""
    import torch
    k, E = cfg.k, cfg.E
    def staged(clamp: bool):
        ids, w = g.route_topk(inp.logits, k, cfg.num_valid_rows, cfg.renormalize)
        if clamp:
            ids = torch.where(ids >= E, torch.full_like(ids, E - 1), ids)
        off, sr, rp = g.build_offsets(ids, E)
        h = g.grouped_gemm_gather(inp.x, inp.w13, off, sr, k, "silu_mul")
        y = g.grouped_gemm(h, inp.w2, off, "none")
        return g.unpermute_combine(y, rp, w, off, k)
    out = {}
    for clamp in (False, True):
        for _ in range(2):
            o = staged(clamp)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            o = staged(clamp)
        e1.record()
        torch.cuda.synchronize()
        out["clamped_ms" if clamp else "excluded_ms"] = e0.elapsed_time(e1) / steps
        out["out_clamped" if clamp else "out_excluded"] = o
    same = torch.equal(out.pop("out_clamped").view(torch.int16), out.pop("out_excluded").view(torch.int16))
    out["outputs_identical"] = bool(same)
    return out


def cpu_baseline(cfg, inp, sample_tokens: int, min_seconds: float = 10.0) -> dict:
    """The oracle as it stands, on the first ``sample_tokens`` tokens with the full weights,
    repeated in whole passes until at least ``min_seconds`` of wall time have passed."""
    import numpy as np
    import torch
    from oracle import layer as olayer
    from oracle.layer import ExpertWeights

    S = min(sample_tokens, cfg.T)
    f32 = lambda t: t.detach().to("cpu", torch.float32).numpy()
    if cfg.dtype == "fp8":
        W = ExpertWeights(inp.w13.cpu().view(torch.uint8).numpy(), inp.w2.cpu().view(torch.uint8).numpy(),
                          inp.w13_scale.cpu().numpy(), inp.w2_scale.cpu().numpy())
    else:
        W = ExpertWeights(f32(inp.w13), f32(inp.w2))
    x = f32(inp.x[:S])
    lg = inp.logits[:S].cpu().numpy()
    nv = cfg.num_valid_rows if cfg.num_valid_rows < 0 else min(cfg.num_valid_rows, S * cfg.k)
    threads, blas = None, None
    try:
        from threadpoolctl import threadpool_info
        libs = [i for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max((i.get("num_threads", 0) for i in libs), default=None)
        blas = ", ".join(sorted({f"{i.get('internal_api')} {i.get('version')}" for i in libs})) or None
    except Exception:
        pass
    passes = 0
    t0 = time.perf_counter()
    while passes == 0 or time.perf_counter() - t0 < min_seconds:
        olayer.forward(x, lg, W, cfg.k, nv, cfg.renormalize)
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": S * passes / dt, "unit": "tokens/s", "cores": threads or os.cpu_count(),
            "kind": "oracle", "seconds": dt, "passes": passes,
            "sample": f"first {S} of {cfg.T} tokens, full weights (float64 per-expert loop), "
                      f"{passes} pass{'es' if passes > 1 else ''}",
            "host_cpus": len(os.sched_getaffinity(0)), "blas": blas, "cpu_model": cpu_model()}


def cpu_model() -> str | None:
    """The host CPU's model name (from /proc/cpuinfo)."""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def warm(torch, call, at_least: int, seconds: float) -> int:
    """Untimed warm-up: at least `at_least` calls and at least `seconds` of wall time, so that
    the timed region starts at the GPU's steady clock (a cold MI355X runs the first few hundred
    milliseconds of work measurably slower).  Returns the number of calls made."""
    n = 0
    t0 = time.perf_counter()
    while n < at_least or time.perf_counter() - t0 < seconds:
        call()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    return n


def time_events(torch, call, n: int, scrub=None) -> float:
    """Mean device time (us) of call() over n calls, timed with HIP events on the stream the
    library runs on.  Without scrub: one event pair around n back-to-back calls.  With scrub:
    before every call (outside its event pair) the 512 MB buffer is read through once, so the
    call's inputs are no longer in L2 or the 256 MB MALL and no dirty lines are left to flush."""
    stream = torch.cuda.current_stream().cuda_stream
    if scrub is None:
        ev = HipEvents(2)
        ev.record(0, stream)
        for _ in range(n):
            call()
        ev.record(1, stream)
        torch.cuda.synchronize()
        us = ev.ms(0, 1) / n * 1e3
        ev.close()
        return us
    ev = HipEvents(2 * n)
    for i in range(n):
        scrub.sum()
        ev.record(2 * i, stream)
        call()
        ev.record(2 * i + 1, stream)
    torch.cuda.synchronize()
    us = sum(ev.ms(2 * i, 2 * i + 1) for i in range(n)) / n * 1e3
    ev.close()
    return us


def time_permute(g, torch, cfg, inp, aux, steps: int, scrub) -> dict:
    """moe_permute on its own (the scatter step; the layer's gate/up GEMM reads token rows
    through the permutation instead): V rows read and written.  `us` back to back (the token
    rows stay in the MALL from call to call), `cold_us` with a 512 MB read between calls."""
    fp8 = cfg.dtype == "fp8"
    out_dt = torch.float8_e4m3fn if fp8 else inp.x.dtype
    xp = torch.empty(cfg.R, cfg.H, dtype=out_dt, device=inp.x.device)
    xs = torch.empty(cfg.H // 128, cfg.R, dtype=torch.float32, device=inp.x.device) if fp8 else None

    def call():
        g.permute(inp.x, aux.sorted_rows, aux.offsets, cfg.k, out_dtype=out_dt, out=xp, out_scales=xs)
    warm(torch, call, 5, 0.2)
    n = max(steps, 20)
    us = time_events(torch, call, n)
    cold = time_events(torch, call, n, scrub)
    esz = inp.x.element_size()
    V = cfg.V
    moved = V * cfg.H * esz + (V * cfg.H + V * (cfg.H // 128) * 4 if fp8 else V * cfg.H * esz)
    return {"us": us, "bytes": moved, "gbs": moved / (us * 1e-6) / 1e9,
            "cold_us": cold, "cold_gbs": moved / (cold * 1e-6) / 1e9}


def time_combine(g, torch, cfg, inp, aux, steps: int, scrub) -> dict:
    """moe_unpermute_combine on its own over bf16 rows y [R, H] (values from the seeded hidden
    states; only the access pattern matters): V rows + T output rows + 8 B per slot, back to
    back and with a 512 MB read between calls."""
    y = inp.x.repeat_interleave(cfg.k, dim=0)[: cfg.R].to(torch.bfloat16).contiguous()
    out = torch.empty(cfg.T, cfg.H, dtype=torch.bfloat16, device=inp.x.device)

    def call():
        g.unpermute_combine(y, aux.row_pos, aux.topk_weights, aux.offsets, cfg.k, out=out)
    warm(torch, call, 5, 0.2)
    n = max(steps, 20)
    us = time_events(torch, call, n)
    cold = time_events(torch, call, n, scrub)
    moved = cfg.V * cfg.H * 2 + cfg.T * cfg.H * 2 + 8 * cfg.T * cfg.k
    return {"us": us, "bytes": moved, "gbs": moved / (us * 1e-6) / 1e9,
            "cold_us": cold, "cold_gbs": moved / (cold * 1e-6) / 1e9}


def time_decode(g, torch, cfg, inp, steps: int, tokens=(1, 8, 64)) -> list:
    """The layer at decode sizes on the same weights: the first T tokens of the batch.  These
    launches take the 16-row decode tiles; the bound is streaming each touched expert's weights
    once, so the rate reported is touched-weight bytes per layer time against 8 TB/s."""
    res = []
    esz = {"f32": 4, "bf16": 2, "fp8": 1}[cfg.dtype]
    for T in tokens:
        c = cfg.replace(T=T)
        x, lg = inp.x[:T].contiguous(), inp.logits[:T].contiguous()
        ws = torch.empty(g.forward_workspace_bytes(T, c.H, c.I, c.E, c.k, inp.w13.dtype), dtype=torch.uint8,
                         device=x.device)
        out = torch.empty(T, c.H, dtype=inp.x.dtype, device=x.device)
        _, aux = g.forward(x, lg, inp.w13, inp.w2, c.k, -1, c.renormalize, inp.w13_scale, inp.w2_scale, out=out,
                           workspace=ws, return_aux=True)
        off = aux.offsets.cpu().tolist()
        touched = sum(1 for e in range(c.E) if off[e + 1] > off[e])

        def call():
            g.forward(x, lg, inp.w13, inp.w2, c.k, -1, c.renormalize, inp.w13_scale, inp.w2_scale, out=out,
                      workspace=ws)
        warm(torch, call, 5, 0.3)
        ev = HipEvents(2)
        stream = torch.cuda.current_stream().cuda_stream
        n = max(steps, 50)
        ev.record(0, stream)
        for _ in range(n):
            call()
        ev.record(1, stream)
        torch.cuda.synchronize()
        us = ev.ms(0, 1) / n * 1e3
        ev.close()
        wbytes = touched * 3 * c.I * c.H * esz
        res.append({"T": T, "experts_touched": touched, "us_per_layer": us,
                    "weight_gbs": wbytes / (us * 1e-6) / 1e9, "frac_hbm": wbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS})
    return res


def time_backward(g, torch, cfg, inp, aux, warmup: int, steps: int, warm_s: float) -> dict:
    """moe_backward for the forward's routing, timed with HIP events on its stream, with f32
    gradients and again with bf16 gradients (the weight gradients then store half the bytes).

    GEMM work: 16*V*H*I flops, of which 4*V*H*I recompute the forward's SiLU*up product
    and 12*V*H*I are the data- and weight-gradient products (fp8 layers: the recompute runs
    on the fp8 codes, the gradient products on the dequantised bf16 values)."""
    dout = torch.randn(cfg.T, cfg.H, generator=torch.Generator(device="cuda:0").manual_seed(7),
                       device="cuda:0").to(torch.bfloat16)
    ws = torch.empty(g.backward_workspace_bytes(cfg.T, cfg.H, cfg.I, cfg.E, cfg.k, inp.w13.dtype),
                     dtype=torch.uint8, device="cuda:0")
    V, H, I = cfg.V, cfg.H, cfg.I
    res = {}
    for name, gdt in (("f32", torch.float32), ("bf16", torch.bfloat16)):
        def call():
            return g.backward(inp.x, inp.w13, inp.w2, dout, aux.topk_weights, aux.offsets, aux.sorted_rows,
                              aux.row_pos, grad_dtype=gdt, workspace=ws, w13_scale=inp.w13_scale,
                              w2_scale=inp.w2_scale)
        n_warm = warm(torch, call, max(1, warmup), warm_s)
        ev = HipEvents(2)
        stream = torch.cuda.current_stream().cuda_stream   # the stream the wrappers queue on
        ev.record(0, stream)
        for _ in range(steps):
            call()
        ev.record(1, stream)
        torch.cuda.synchronize()
        ms = ev.ms(0, 1) / steps
        ev.close()
        res[name] = {"ms": ms, "warmup": n_warm,
                     "gemm_tflops_with_recompute": 16.0 * V * H * I / (ms * 1e-3) / 1e12,
                     "gemm_tflops_gradients_only": 12.0 * V * H * I / (ms * 1e-3) / 1e12}
    return {"ms": res["f32"]["ms"], "steps": steps, "grad_dtype": "f32", "workspace_bytes": ws.numel(),
            "gemm_tflops_with_recompute": res["f32"]["gemm_tflops_with_recompute"],
            "gemm_tflops_gradients_only": res["f32"]["gemm_tflops_gradients_only"],
            "by_grad_dtype": res}


def main() -> int:
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps before timing (at least)")
    ap.add_argument("--warmup-seconds", type=float, default=2.0,
                    help="warm-up also lasts at least this long (GPU clock ramp); 0 disables")
    ap.add_argument("--workload", default="gptoss20b_bf16")
    ap.add_argument("--cpu-sample", type=int, default=4096,
                    help="tokens for the CPU oracle baseline (default: the whole layer)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="the CPU oracle baseline repeats whole passes over its sample for at least this long")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--clamp-ab", action="store_true",
                    help="also time the staged layer with sentinel rows clamped onto the last expert")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-size layer timings")
    ap.add_argument("--decode-only", type=int, default=0, metavar="T",
                    help="time only the layer on the first T tokens (decode size) and print that line")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip timing moe_backward (bf16 and fp8 workloads time it by default)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="after timing, run one plain 1 GiB device copy (counter calibration)")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for {args.gpus}); the library has no "
              f"multi-GPU path. Run with --gpus 1.", file=sys.stderr)
        return 2

    import torch

    import grouped_gemm_histogram_amd as g
    from workloads import generate, get_config

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    g.load()
    cfg = get_config(args.workload)
    dev = "cuda:0"
    inp = generate(cfg, dev)
    T, H, I, E, k = cfg.T, cfg.H, cfg.I, cfg.E, cfg.k
    if args.decode_only:
        a = torch.randn(4096, 4096, device=dev).to(torch.bfloat16)
        warm(torch, lambda: torch.matmul(a, a), 1, args.warmup_seconds)
        dec = time_decode(g, torch, cfg, inp, args.steps, tokens=(args.decode_only,))[0]
        print(json.dumps({"metric": "MoE layer time at decode size", "workload": cfg.name, "dtype": cfg.dtype,
                          "steps": max(args.steps, 50), **dec}))
        return 0
    need = g.forward_workspace_bytes(T, H, I, E, k, inp.w13.dtype)
    ws = torch.empty(need, dtype=torch.uint8, device=dev)
    out = torch.empty(T, H, dtype=torch.float32 if cfg.dtype == "f32" else torch.bfloat16, device=dev)

    def step(events=None):
        g.forward(inp.x, inp.logits, inp.w13, inp.w2, k, cfg.num_valid_rows, cfg.renormalize,
                  inp.w13_scale, inp.w2_scale, out=out, workspace=ws, stage_events=events)

    # offsets of this routing, for the predicted MFMA work (outside the timed region)
    _, aux = g.forward(inp.x, inp.logits, inp.w13, inp.w2, k, cfg.num_valid_rows, cfg.renormalize,
                       inp.w13_scale, inp.w2_scale, out=out, workspace=ws, return_aux=True)
    torch.cuda.synchronize()
    offsets_host = aux.offsets.cpu().tolist()

    n_warm = warm(torch, step, args.warmup, args.warmup_seconds)

    # the timed steps: plain layer calls, no instrumentation
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps

    # the same number of steps again with HIP events between the library's stages (per-stage
    # device times, the gate/up kernel's duration for the roofline); recording events adds a
    # few microseconds per stage, so this pass is not the one timed above
    nst = len(g._lib.FORWARD_STAGES)
    ev = HipEvents(args.steps * (nst + 1))
    for i in range(args.steps):
        step(ev.ev[i * (nst + 1):(i + 1) * (nst + 1)])
    torch.cuda.synchronize()
    stage_ms = {}
    for s, name in enumerate(g._lib.FORWARD_STAGES):
        stage_ms[name] = sum(ev.ms(i * (nst + 1) + s, i * (nst + 1) + s + 1)
                             for i in range(args.steps)) / args.steps
    device_ms = sum(ev.ms(i * (nst + 1), i * (nst + 1) + nst) for i in range(args.steps)) / args.steps
    ev.close()

    scrub = torch.ones(64 << 20, dtype=torch.int64, device=dev)   # 512 MB, read to evict caches
    permute = time_permute(g, torch, cfg, inp, aux, args.steps, scrub)
    combine = time_combine(g, torch, cfg, inp, aux, args.steps, scrub)
    del scrub

    decode = None
    if cfg.dtype == "bf16" and not args.no_decode:
        decode = time_decode(g, torch, cfg, inp, args.steps)

    backward = None
    if cfg.dtype in ("bf16", "fp8") and not args.no_backward:
        backward = time_backward(g, torch, cfg, inp, aux, args.warmup, args.steps, args.warmup_seconds)

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        b.copy_(a)
        torch.cuda.synchronize()

    V = cfg.V
    esz = 4 if cfg.dtype == "f32" else 2
    f_gu, f_dn = 4.0 * V * H * I, 2.0 * V * H * I
    peak = PEAK_TFLOPS[cfg.dtype]
    gu_tf = f_gu / (stage_ms["gemm_gate_up"] * 1e-3) / 1e12
    dn_tf = f_dn / (stage_ms["gemm_down"] * 1e-3) / 1e12
    gemm_tf = (f_gu + f_dn) / ((stage_ms["gemm_gate_up"] + stage_ms["gemm_down"]) * 1e-3) / 1e12
    tokens_valid = tokens_with_rows(cfg)
    combine_bytes = V * H * esz + T * H * esz + 8 * T * k
    traffic = load_traffic(cfg.name)
    R = cfg.R
    # moe_forward picks bf16 tiles for the rows that can be valid (V), other dtypes for R
    tr = V if cfg.dtype == "bf16" else R
    pred_dn = predicted_mfma_flops(offsets_host, R, H, I, g.grouped_gemm_tile_shape(inp.w13.dtype, "none", max(tr, 1), E))
    # SiLU*up tiles hold tile_n/2 output columns: count them against N_out = I
    # the fp8 layer's gate/up writes e4m3 h (f32 h at decode sizes, quantised after)
    h_dt = torch.float8_e4m3fn if cfg.dtype == "fp8" and R > 8 * E else None
    tm, tn, ks = g.grouped_gemm_tile_shape(inp.w13.dtype, "silu_mul", max(tr, 1), E, h_dt)
    pred_gu = predicted_mfma_flops(offsets_host, R, I, H, (tm, tn // 2, ks)) * 2

    # The dominant kernel's bound: the larger of its MFMA time and its HBM time at peak.
    gu_bytes = gate_up_bytes(cfg, offsets_host)
    gu_s = stage_ms["gemm_gate_up"] * 1e-3
    t_mfma, t_hbm = f_gu / (peak * 1e12), gu_bytes / (HBM_PEAK_GBS * 1e9)
    if t_mfma >= t_hbm:
        roofline = {"kernel": "grouped_gemm gate/up + SiLU*up", "bound": "mfma", "achieved": gu_tf,
                    "peak": peak, "unit": "TFLOP/s", "frac": gu_tf / peak, "traffic": traffic}
    else:
        gbs = gu_bytes / gu_s / 1e9
        roofline = {"kernel": "grouped_gemm gate/up + SiLU*up", "bound": "hbm", "achieved": gbs,
                    "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS, "traffic": traffic}
    roofline["algorithmic_bytes"] = gu_bytes
    roofline["algorithmic_flops"] = f_gu

    rec = {
        "metric": METRIC,
        "value": T / (ms_per_step * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": n_warm,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) hidden states and logits, N(0,0.02) weights)",
        "config": {"workload": cfg.name, "T": T, "H": H, "I": I, "E": E, "k": k,
                   "valid_rows": V, "routed_rows": cfg.R},
        "gemm_tflops": gemm_tf,
        "gemm_frac_peak": gemm_tf / peak,
        "gemm_gate_up_tflops": gu_tf,
        "gemm_down_tflops": dn_tf,
        "stage_ms": stage_ms,
        "device_ms_per_step": device_ms,
        "combine_gbs": combine_bytes / (stage_ms["combine"] * 1e-3) / 1e9,
        "permute_standalone": permute,
        "combine_standalone": combine,
        "valid_rows_offsets_last": offsets_host[-1],
        "predicted_mfma_flops": {"gemm_gate_up": pred_gu, "gemm_down": pred_dn},
        "roofline": roofline,
    }
    if cfg.dtype == "fp8":
        # per-token quantisation: bf16 rows read, e4m3 codes and f32 scales written
        q_bytes = T * H * 2 + T * H + T * (H // 128) * 4
        rec["quantize_gbs"] = q_bytes / (stage_ms["act_staging"] * 1e-3) / 1e9
    if decode is not None:
        rec["decode"] = decode
    if backward is not None:
        rec["backward"] = backward
    if args.clamp_ab:
        rec["clamp_ab"] = clamp_ab(g, cfg, inp, max(3, args.steps // 2))
    if not args.no_cpu_baseline:
        rec["cpu_baseline"] = cpu_baseline(cfg, inp, args.cpu_sample, args.cpu_seconds)
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
