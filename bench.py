"""Throughput of the MoE expert layer (forward + backward) on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload longseq]
                    [--unfused] [--no-plain] [--no-cpu-baseline] [--cpu-tokens N]

One step = one pass of the whole layer over one batch of synthetic, seeded
inputs already resident in HBM: route (top-k, histogram, slot map) ->
dispatch -> grouped SwiGLU GEMM -> down GEMM -> combine, then combine backward
-> FFN input gradients -> FFN weight gradients -> dispatch backward -> gate
backward.  Prints one JSON line.  Default workload: the long-sequence slice
(T=131072 tokens, H=2048, E=32, top-4, I=1408, bf16, forward + backward), the
largest of the layer sizes that fits one GPU (the 128k-token workload of the
UniEP article's evaluation).  The headline times the fused calls
(dispatch+up, down+combine, the one-launch backward); the same run then times
the plain calls over the same number of steps ("plain_path"), so fused and
plain are compared on one GPU in one process.  After the timed steps the
library's bounded-wait record is checked (moe_sync_status): a step in which
a wait gave up is an error, not a result.

Each library call inside the timed steps is bracketed by HIP events recorded
on the stream the call launches on, so per-call device times are measured on
the very steps that are timed.  The roofline entry is computed for the call
with the largest total time from its algorithmic flop (or byte) count.
After the timed steps one more step runs with a 512 MiB buffer written before
every HBM-bound call, so that those calls read their inputs from HBM rather
than from L2 or the 256 MiB Infinity Cache where the step leaves them;
"hbm_flushed" reports their rates (the per-call figures are the unflushed
ones).  The CPU baseline times the oracle (plain fp64 numpy) on a bounded
sample of the same layer: the first --cpu-tokens tokens, full expert weights.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "MoE layer fwd+bwd tokens/sec on 1 MI355X; % MFMA peak (GEMM), % HBM BW"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 dense bf16 flop/clk/CU
PEAK_F32_TFLOPS = 157.3
PEAK_HBM_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="longseq")
    ap.add_argument("--unfused", action="store_true",
                    help="time the plain calls instead of the fused persistent kernels "
                         "(dispatch+up, down+combine, and the one-launch backward)")
    ap.add_argument("--no-plain", action="store_true",
                    help="do not time the plain calls after the fused ones")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=0,
                    help="tokens of the CPU-baseline sample (default: about 6e12 flop of oracle work)")
    ap.add_argument("--fwd-only", action="store_true")
    ap.add_argument("--no-hbm-flush", action="store_true",
                    help="skip the extra step that times the HBM-bound calls with the caches flushed")
    ap.add_argument("--route-ranks", type=int, default=0, metavar="G",
                    help="instead of the layer, time Algorithm 1 with G explicit ranks "
                         "(moe_route_ranks) on the workload's routing, beside the oracle")
    ap.add_argument("--tune-sweep", action="store_true",
                    help="instead of the headline, time the fused step for every candidate value "
                         "of each schedule knob (one knob at a time) beside the band model's "
                         "prediction, and print one JSON line")
    ap.add_argument("--copy-reference", action="store_true",
                    help="only run a plain 256 MiB device copy three times (the reference that "
                         "calibrates the FETCH_SIZE / WRITE_SIZE counters)")
    return ap.parse_args()


def copy_reference():
    import torch
    n = 256 * 1024 * 1024
    a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(f"copied {n} bytes x3", flush=True)


def algorithmic_work(d, b):
    """Algorithmic flop / byte counts per call (b = bytes per element).  Kinds:
    "mfma" (flop), "hbm" (bytes; also timed with caches flushed), "latency"
    (bytes, but a few small dependent launches: reported, not flushed)."""
    T, H, E, K, I, Ns, R = d.T, d.H, d.E, d.K, d.I, d.n_shared, d.R
    RA = R + Ns * T
    gemm = lambda rows, m: 2.0 * rows * H * I * m
    return {
        "route": ("latency", 4.0 * T * E + 8.0 * T * K + 4.0 * E + 8.0 * R),
        "dispatch": ("hbm", b * T * H + b * R * H + 4.0 * R),
        "ffn_up": ("mfma", gemm(RA, 2)),
        "ffn_down": ("mfma", gemm(RA, 1)),
        "dispatch_ffn": ("mfma", gemm(RA, 2)),
        "ffn_combine": ("mfma", gemm(RA, 1)),
        "combine": ("hbm", b * R * H + b * Ns * T * H + b * T * H + 8.0 * R),
        "combine_bwd": ("hbm", b * T * H + 2 * b * R * H + 12.0 * R),
        "ffn_bwd_act": ("mfma", gemm(RA, 1)),
        "ffn_bwd_input": ("mfma", gemm(RA, 2)),
        "ffn_bwd_wgrad_gate_up": ("mfma", gemm(RA, 2)),
        "ffn_bwd_wgrad_down": ("mfma", gemm(RA, 1)),
        "ffn_bwd": ("mfma", gemm(RA, 6)),
        "dispatch_bwd": ("hbm", b * RA * H + b * T * H + 4.0 * R),
        "route_bwd": ("latency", 12.0 * T * K + 4.0 * T * E),
    }


def main():
    args = parse()
    if args.copy_reference:
        copy_reference()
        return
    if args.gpus != 1:
        print(f"bench.py: the layer runs on one GPU; --gpus {args.gpus} is not supported "
              "(across GPUs it would shard by expert, which is not implemented)",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    import combine_moe_route_histogram_amd as M
    from combine_moe_route_histogram_amd import layer as L

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    M.moe_init(0)
    cfg = synth.config(args.workload)
    if args.route_ranks:
        bench_route_ranks(args, cfg)
        return
    if args.tune_sweep:
        tune_sweep(args, cfg)
        return
    backward = ("bwd" in cfg.passes) and not args.fwd_only
    t_gen = time.time()
    inp = synth.make_inputs(cfg, with_grad=backward)
    p = {k: synth.to_torch(v, "cuda") for k, v in inp.items()}
    gen_s = time.time() - t_gen
    d = L.make_dims(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.n_shared, cfg.dtype)
    b = L.Buffers(d, backward=backward)
    stream = torch.cuda.current_stream()

    calls = []  # (name, start_event, end_event)
    bpe = 2 if cfg.dtype == "bf16" else 4
    work = algorithmic_work(d, bpe)
    flush = {"buf": None}   # set: write it before every HBM-bound call (evicts L2 and MALL)

    def timed(name, fn, *a):
        if flush["buf"] is not None and work[name][0] == "hbm":
            flush["buf"].fill_(1)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn(*a)
        e1.record(stream)
        calls.append((name, e0, e1))

    def step(fused):
        timed("route", L.route, b, p)
        if fused:
            timed("dispatch_ffn", M.moe_dispatch_ffn, d, p["x"], b.slot_src, b.slot, b.offsets, p["w1"],
                  p["w3"], p.get("ws1"), p.get("ws3"), b.x_perm, b.ab, b.h, b.ws)
            timed("ffn_combine", M.moe_ffn_combine, d, b.h, b.offsets, p["w2"], p.get("ws2"),
                  b.slot, b.topk_w, b.y, b.out, b.ws)
        else:
            timed("dispatch", M.moe_dispatch, d, p["x"], b.slot, b.x_perm)
            timed("ffn_up", M.moe_expert_ffn_up, d, b.x_perm, p["x"], b.offsets, p["w1"], p["w3"],
                  p.get("ws1"), p.get("ws3"), b.ab, b.h, b.ws)
            timed("ffn_down", M.moe_expert_ffn_down, d, b.h, b.offsets, p["w2"], p.get("ws2"),
                  b.y, b.ws)
            timed("combine", M.moe_combine, d, b.y, b.slot, b.topk_w, b.out)
        if backward:
            timed("combine_bwd", M.moe_combine_bwd, d, p["dout"], b.y, b.slot, b.topk_w, b.dy,
                  b.dtopk_w)
            if fused:   # B and W in one launch, W tiles in the gaps of B
                timed("ffn_bwd", M.moe_expert_ffn_bwd, d, b.dy, p.get("dout"), b.offsets, p["w1"],
                      p["w3"], p["w2"], p.get("ws1"), p.get("ws3"), p.get("ws2"), b.ab, b.x_perm,
                      p["x"], b.h, b.dab, b.dx_rows, b.dw1, b.dw3, b.dw2, b.dws1, b.dws3, b.dws2,
                      b.ws)
            else:
                timed("ffn_bwd_act", M.moe_expert_ffn_bwd_act, d, b.dy, p.get("dout"), b.offsets,
                      p["w2"], p.get("ws2"), b.ab, b.dab, b.ws)
                timed("ffn_bwd_input", M.moe_expert_ffn_bwd_input, d, b.dab, b.offsets, p["w1"],
                      p["w3"], p.get("ws1"), p.get("ws3"), b.dx_rows, b.ws)
                timed("ffn_bwd_wgrad_gate_up", M.moe_expert_ffn_bwd_weight_gate_up, d, b.x_perm,
                      p["x"], b.dab, b.offsets, b.dw1, b.dw3, b.dws1, b.dws3, b.ws)
                timed("ffn_bwd_wgrad_down", M.moe_expert_ffn_bwd_weight_down, d, b.h, b.dy,
                      p.get("dout"), b.offsets, b.dw2, b.dws2, b.ws)
            timed("dispatch_bwd", M.moe_dispatch_bwd, d, b.dx_rows, b.slot, b.dx)
            timed("route_bwd", M.moe_route_bwd, d, b.dtopk_w, b.topk_w, b.topk_idx, b.dlogits)

    def run(fused):
        """W untimed steps, then exactly K timed steps between two device
        synchronisations; returns (ms per step, mean device ms per call)."""
        for _ in range(args.warmup):
            step(fused)
        torch.cuda.synchronize()
        calls.clear()
        t0 = time.perf_counter()
        for _ in range(args.steps):
            step(fused)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        # a bounded wait that gave up inside the timed steps makes them invalid
        M.moe_sync_status()
        per = {}
        for name, e0, e1 in calls:
            per.setdefault(name, []).append(e0.elapsed_time(e1))
        calls.clear()
        return wall * 1e3 / args.steps, {k: float(np.mean(v)) for k, v in per.items()}

    fused = not args.unfused
    ms_per_step, per_call_ms = run(fused)
    tokens_per_s = cfg.T / (ms_per_step * 1e-3)

    # one more step, untimed as a whole: a 512 MiB buffer is written before
    # each HBM-bound call, so its inputs come from HBM rather than from the
    # 256 MiB Infinity Cache (MALL) or L2, where the step leaves them
    hbm_flushed = {}
    if not args.no_hbm_flush:
        flush["buf"] = torch.empty(512 << 20, dtype=torch.uint8, device="cuda")
        flush["buf"].fill_(1)   # first touch of the new buffer outside any timed call
        torch.cuda.synchronize()
        step(fused)
        torch.cuda.synchronize()
        M.moe_sync_status()
        flush["buf"] = None
    for name, e0, e1 in calls:
        kind, amount = work[name]
        if kind == "hbm":
            ms = e0.elapsed_time(e1)
            rate = amount / (ms * 1e-3) / 1e9
            hbm_flushed[name] = {"ms": round(ms, 4), "GB/s": round(rate, 1),
                                 "frac": round(rate / PEAK_HBM_GBS, 4)}
    calls.clear()

    peak_mfma = PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_F32_TFLOPS

    def breakdown(per):
        out = {}
        for k, ms in per.items():
            kind, amount = work[k]
            if kind == "mfma":
                rate = amount / (ms * 1e-3) / 1e12
                out[k] = {"ms": round(ms, 4), "TFLOP/s": round(rate, 1), "frac": round(rate / peak_mfma, 4)}
            else:
                rate = amount / (ms * 1e-3) / 1e9
                out[k] = {"ms": round(ms, 4), "GB/s": round(rate, 1), "frac": round(rate / PEAK_HBM_GBS, 4)}
        return out

    # the same number of steps of the other path, in the same process on the
    # same buffers (fused vs plain on one GPU)
    other = None
    if not args.no_plain:
        o_ms, o_per = run(not fused)
        other = {"path": "unfused" if fused else "fused", "ms_per_step": round(o_ms, 4),
                 "value": round(cfg.T / (o_ms * 1e-3), 1), "per_call": breakdown(o_per)}

    dom = max(per_call_ms, key=per_call_ms.get)
    kind, amount = work[dom]
    # HBM bytes per launch of the dominant kernel from the committed counter
    # summary, only if it was taken on the kernel sources being run
    from combine_moe_route_histogram_amd.profsum import traffic_bytes
    traffic = traffic_bytes(dom, cfg.name)
    if kind == "mfma":
        ach = amount / (per_call_ms[dom] * 1e-3) / 1e12
        roofline = {"bound": "mfma", "kernel": dom, "achieved": round(ach, 1), "peak": peak_mfma,
                    "unit": "TFLOP/s", "frac": round(ach / peak_mfma, 4), "traffic": traffic,
                    "traffic_unit": "bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                    "work_per_launch": amount}
    else:
        ach = amount / (per_call_ms[dom] * 1e-3) / 1e9
        roofline = {"bound": "hbm", "kernel": dom, "achieved": round(ach, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(ach / PEAK_HBM_GBS, 4), "traffic": traffic,
                    "traffic_unit": "bytes per launch (FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                    "work_per_launch": amount}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg, inp, args.cpu_tokens, backward)

    line = {
        "metric": METRIC, "value": round(tokens_per_s, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": cfg.dtype,
        "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={cfg.T} H={cfg.H} E={cfg.E} top-{cfg.K} I={cfg.I}"
                               f" shared={cfg.n_shared} {cfg.dtype} {'fwd+bwd' if backward else 'fwd'}",
                   "T": cfg.T, "H": cfg.H, "E": cfg.E, "K": cfg.K, "I": cfg.I,
                   "n_shared": cfg.n_shared, "passes": "fwd+bwd" if backward else "fwd",
                   "path": "fused" if fused else "unfused"},
        "roofline": roofline,
        "cpu_baseline": cpu,
        "per_call": breakdown(per_call_ms),
        "plain_path" if fused else "fused_path": other,
        "hbm_flushed": hbm_flushed,
        "input_gen_s": round(gen_s, 1),
    }
    print(json.dumps(line), flush=True)


TUNE_CANDIDATES = {
    "band_up": (2, 4, 8, 16),
    "band_act": (2, 4, 8, 16),
    "small_group": (2, 4, 5, 8, 12, 16),
    "band_wgrad_up": (2, 4, 8, 16),
    "band_wgrad_down": (2, 4, 8, 16),
    "combine_tokens": (8, 16, 32, 64),
    "copy_tokens": (16, 32, 64, 128),
    "copy_in_tiles": (0, 1),
}
# the calls whose time each knob changes
TUNE_CALLS = {
    "band_up": ("dispatch_ffn",), "band_act": ("ffn_bwd",), "small_group": ("dispatch_ffn", "ffn_bwd"),
    "band_wgrad_up": ("ffn_bwd",), "band_wgrad_down": ("ffn_bwd",), "combine_tokens": ("ffn_combine",),
    "copy_tokens": ("dispatch_ffn",), "copy_in_tiles": ("dispatch_ffn",),
}


def tune_sweep(args, cfg):
    """Every candidate of every schedule knob (one at a time, the others at
    the library's choice), timed on the fused step; the band model's
    prediction beside the measured time of the call the knob schedules."""
    import numpy as np
    import torch
    import synth
    import combine_moe_route_histogram_amd as M
    from combine_moe_route_histogram_amd import layer as L

    backward = "bwd" in cfg.passes
    inp = synth.make_inputs(cfg, with_grad=backward)
    p = {k: synth.to_torch(v, "cuda") for k, v in inp.items()}
    d = L.make_dims(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.n_shared, cfg.dtype)
    b = L.Buffers(d, backward=backward)
    stream = torch.cuda.current_stream()
    chosen = M.moe_get_tuning(d).as_dict()
    calls = []

    def timed(name, fn, *a):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        fn(*a)
        e1.record(stream)
        calls.append((name, e0, e1))

    def step():
        L.route(b, p)
        timed("dispatch_ffn", M.moe_dispatch_ffn, d, p["x"], b.slot_src, b.slot, b.offsets, p["w1"],
              p["w3"], p.get("ws1"), p.get("ws3"), b.x_perm, b.ab, b.h, b.ws)
        timed("ffn_combine", M.moe_ffn_combine, d, b.h, b.offsets, p["w2"], p.get("ws2"), b.slot,
              b.topk_w, b.y, b.out, b.ws)
        if backward:
            M.moe_combine_bwd(d, p["dout"], b.y, b.slot, b.topk_w, b.dy, b.dtopk_w)
            timed("ffn_bwd", M.moe_expert_ffn_bwd, d, b.dy, p.get("dout"), b.offsets, p["w1"], p["w3"],
                  p["w2"], p.get("ws1"), p.get("ws3"), p.get("ws2"), b.ab, b.x_perm, p["x"], b.h,
                  b.dab, b.dx_rows, b.dw1, b.dw3, b.dw2, b.dws1, b.dws3, b.dws2, b.ws)

    def measure(tune):
        if tune:
            os.environ["MOE_TUNE"] = tune
        else:
            os.environ.pop("MOE_TUNE", None)
        M.moe_init(0)
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        calls.clear()
        for _ in range(args.steps):
            step()
        M.moe_sync_status()
        per = {}
        for name, e0, e1 in calls:
            per.setdefault(name, []).append(e0.elapsed_time(e1))
        return {k: round(float(np.median(v)), 4) for k, v in per.items()}

    base = measure(None)
    sweep = {}
    for knob, values in TUNE_CANDIDATES.items():
        rows = []
        for v in values:
            ms = measure(f"{knob}={v}")
            key = [c for c in TUNE_CALLS[knob] if c in ms]
            pred = M.moe_tuning_predict(d, knob, v)
            rows.append({"value": v, "chosen": v == chosen[knob],
                         "ms": round(sum(ms[c] for c in key), 4),
                         "predicted_bytes_per_flop": round(pred, 7) if pred >= 0 else None})
            print(f"# {cfg.name} {knob}={v}: {rows[-1]}", file=sys.stderr, flush=True)
        best = min(rows, key=lambda r: r["ms"])
        sweep[knob] = {"calls": TUNE_CALLS[knob], "chosen": chosen[knob], "measured_best": best["value"],
                       "candidates": rows}
    measure(None)
    print(json.dumps({"workload": cfg.name, "steps": args.steps, "warmup": args.warmup,
                      "chosen": chosen, "baseline_ms": base, "sweep": sweep}), flush=True)


def bench_route_ranks(args, cfg):
    """Algorithm 1 with G ranks: moe_route_ranks on the workload's routing."""
    import numpy as np
    import torch
    import synth
    import combine_moe_route_histogram_amd as M
    from combine_moe_route_histogram_amd import layer as L

    G = args.route_ranks
    inp = synth.make_inputs(cfg, with_grad=False)
    d = L.make_dims(cfg.T, cfg.H, cfg.E, cfg.K, cfg.I, cfg.n_shared, cfg.dtype)
    b = L.Buffers(d, backward=False)
    p = {"logits": synth.to_torch(inp["logits"], "cuda")}
    L.route(b, p)
    i32 = lambda n: torch.empty(n, dtype=torch.int32, device="cuda")
    T, E, K = cfg.T, cfg.E, cfg.K
    rc, rb, cnt, off, slot, src = i32(G * E), i32(G * E), i32(E), i32(E + 1), i32(T * K), i32(T * K)
    ws = torch.empty(M.moe_route_ranks_workspace_bytes(d, G), dtype=torch.uint8, device="cuda")
    call = lambda: M.moe_route_ranks(d, b.topk_idx, G, rc, rb, cnt, off, slot, src, ws)
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        call()
    torch.cuda.synchronize()
    times = []
    for _ in range(args.steps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        times.append((e0, e1))
    torch.cuda.synchronize()
    us = float(np.mean([a.elapsed_time(c) for a, c in times])) * 1e3
    assert torch.equal(slot, b.slot.reshape(-1)) and torch.equal(src, b.slot_src.reshape(-1))  # one-rank map
    nbytes = 3.0 * T * K * 4 + 2.0 * G * E * 4 + 4.0 * (2 * E + 1)
    gbs = nbytes / (us * 1e-6) / 1e9
    import oracle as O
    idx = b.topk_idx.cpu().numpy()
    t0 = time.perf_counter()
    reps = 0
    while time.perf_counter() - t0 < 10.0:
        O.slot_map_ranks(idx, E, G)
        reps += 1
    cpu_s = (time.perf_counter() - t0) / reps
    print(json.dumps({
        "metric": f"moe_route_ranks latency (Algorithm 1, G={G} ranks)", "value": round(us, 2),
        "unit": "us", "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "higher_is_better": False, "dtype": "int32", "data": "synthetic",
        "config": {"workload": f"{cfg.name}: T={T} E={E} top-{K}, G={G}"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": round(gbs / PEAK_HBM_GBS, 5), "traffic": None,
                     "note": "latency-bound: 5 small dependent launches"},
        "cpu_baseline": {"value": round(cpu_s * 1e6, 1), "unit": "us", "cores": 1, "kind": "oracle",
                         "sample": f"oracle slot_map_ranks on the same routing, {reps} runs"},
    }), flush=True)


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def cpu_baseline(cfg, inp, n_tokens, backward):
    """The oracle as it stands, on the first n_tokens tokens with full weights
    (default: about 6e12 flop of fp64 GEMM work, 10-30 s on a server CPU)."""
    import numpy as np
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:
        threads = os.cpu_count() or 1
    if n_tokens <= 0:
        per_token = 2.0 * (cfg.K * cfg.I + cfg.n_shared * cfg.I_shared) * cfg.H * 3 * (3 if backward else 1)
        n_tokens = int(6e12 / per_token)
    n = max(1, min(n_tokens, cfg.T))
    sub = dict(inp)
    for k in ("logits", "x", "dout"):
        if k in sub:
            sub[k] = np.ascontiguousarray(inp[k][:n])
    t0 = time.perf_counter()
    f = O.forward(sub, cfg.K, cfg.dtype)
    if backward:
        O.backward(sub, f, cfg.dtype)
    sec = time.perf_counter() - t0
    return {"value": round(n / sec, 2), "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"first {n} of {cfg.T} tokens, full expert weights, "
                      f"{'fwd+bwd' if backward else 'fwd'}, fp64 numpy; {sec:.1f} s",
            "cpu": cpu_model(), "nproc": os.cpu_count()}


if __name__ == "__main__":
    main()
