"""Text summaries of rocprofv3 output, and the HBM-traffic lookup bench.py uses.

    python -m combine_moe_route_histogram_amd.profsum stats DIR --title T --command C > OUT.md
    python -m combine_moe_route_histogram_amd.profsum traffic --fetch D1 --write D2 \\
        --copy-fetch D3 --copy-write D4 --workload W --command-fetch C1 --command-write C2 \\
        --command-copy-fetch C3 --command-copy-write C4 --out BASE
    python -m combine_moe_route_histogram_amd.profsum counters --mfma D1 --l2 D2 --title T \\
        --command-mfma C1 --command-l2 C2 [--skip N] > OUT.md

`stats` reads DIR/*kernel_stats.csv (rocprofv3 --kernel-trace --stats
--output-format csv) and prints a Markdown table.  `traffic` reads the
FETCH_SIZE and WRITE_SIZE counter collections of a run of the layer and of
the copy reference (bench.py --copy-reference: a 256 MiB device copy), derives
the counter scale factors from the copy, and writes BASE.md (table) and
BASE.json (per-kernel bytes per dispatch, plus a fingerprint of the kernel
sources and build flags).  bench.py reports a kernel's traffic only while that
fingerprint matches the sources it runs, so a kernel changed since its
counters were taken reports none.  `counters` reads a pass with
GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES and SQ_INSTS_VALU_MFMA_MOPS_BF16
and a pass with TCC_HIT_sum and TCC_MISS_sum, and prints per kernel the
running clock, the MFMA busy share, the bf16 rate and the L2 hit rate.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import re
import sys
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")

COPY_BYTES = 256 * 1024 * 1024

# bench.py call -> the kernel that does its work (regex on the short kernel name)
CALL_KERNEL = {
    "dispatch_ffn": r"^dispatch_ffn_kernel",
    "ffn_combine": r"^ffn_combine_kernel",
    "ffn_bwd": r"^ffn_bwd_kernel",
    "ffn_up": r"^gemm_bf16_kernel<BfCfg<0,",
    "ffn_down": r"^gemm_bf16_kernel<BfCfg<1,",
    "ffn_bwd_act": r"^gemm_bf16_kernel<BfCfg<2,",
    "ffn_bwd_input": r"^gemm_bf16_kernel<BfCfg<3,",
    "ffn_bwd_wgrad_gate_up": r"^gemm_bf16_kernel<BfCfg<4,",
    "ffn_bwd_wgrad_down": r"^gemm_bf16_kernel<BfCfg<5,",
    "dispatch": r"^dispatch_kernel",
    "combine": r"^combine_kernel",
    "combine_bwd": r"^combine_bwd_kernel",
    "dispatch_bwd": r"^dispatch_bwd_kernel",
}


def _code_only(text: str) -> str:
    """C/C++ source without comments and blank space (a comment edit does not
    change the kernels)."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def source_fingerprint() -> str:
    """sha256 over the code of the kernel sources and the public header
    (comments and blank space left out) and the build flags."""
    from . import build as B
    h = hashlib.sha256()
    files = sorted(glob.glob(os.path.join(PKG, "csrc", "*.hip")) +
                   glob.glob(os.path.join(PKG, "csrc", "*.hpp")) +
                   glob.glob(os.path.join(ROOT, "include", "*.h")))
    for f in files:
        h.update(os.path.basename(f).encode())
        with open(f, encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    h.update(" ".join(B.COMMON_FLAGS[1:]).replace(ROOT, "").encode())
    return h.hexdigest()[:16]


def short_name(name: str) -> str:
    name = re.sub(r"^void ", "", name)
    name = name.replace("moe::", "")
    return re.sub(r"\((.*)\)$", "", name).strip()


def _one_csv(d: str, suffix: str) -> str:
    hits = sorted(glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True))
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_stats(d: str):
    rows = []
    with open(_one_csv(d, "kernel_stats.csv")) as fh:
        for r in csv.DictReader(fh):
            rows.append((short_name(r["Name"]), int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                         float(r["TotalDurationNs"]) / 1e6, float(r["Percentage"])))
    rows.sort(key=lambda x: -x[3])
    return rows


def timed_means(d: str, skip: int):
    """Per kernel: mean duration (us) of its dispatches after the first `skip`
    (the warm-up steps), from the kernel trace; None where the trace is absent."""
    try:
        path = _one_csv(d, "kernel_trace.csv")
    except FileNotFoundError:
        return None
    runs = defaultdict(list)
    with open(path) as fh:
        for r in csv.DictReader(fh):
            runs[short_name(r["Kernel_Name"])].append(
                (int(r["Start_Timestamp"]), int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for k, v in runs.items():
        v.sort()
        tail = [x[1] for x in v[skip:]] or [x[1] for x in v]
        out[k] = sum(tail) / len(tail) / 1e3
    return out


def counter_means(d: str, counter: str):
    """Per kernel: mean counter value per dispatch (KiB for FETCH_SIZE / WRITE_SIZE)."""
    vals = defaultdict(list)
    with open(_one_csv(d, "counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            if r["Counter_Name"] == counter:
                vals[short_name(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}


def copy_scale(d: str, counter: str) -> float:
    """COPY_BYTES divided by what the counter reads for the copy kernel."""
    means = counter_means(d, counter)
    cands = {k: v for k, v in means.items() if "copy" in k.lower()}
    if not cands:
        raise RuntimeError(f"no copy kernel in {d}")
    kib = max(v[0] for v in cands.values())
    return (COPY_BYTES / 1024.0) / kib


def cmd_stats(a):
    rows = kernel_stats(a.dir)
    out = [f"# {a.title}", "", "Command (from the repository root on an MI355X):", "",
           f"    {a.command}", ""]
    if a.note:
        out += [a.note, ""]
    timed = timed_means(a.dir, a.skip) if a.skip else None
    if timed is None:
        out += ["| kernel | calls | avg us | total ms | % |", "|---|---:|---:|---:|---:|"]
        for n, c, avg, tot, pct in rows:
            out.append(f"| {n} | {c} | {avg:.1f} | {tot:.2f} | {pct:.2f} |")
    else:
        out += [f"avg us: all dispatches; timed avg us: without the first {a.skip} dispatches of "
                "each kernel (the warm-up steps), the figure to set beside bench.py's per-call "
                "event times.", ""]
        out += ["| kernel | calls | avg us | timed avg us | total ms | % |",
                "|---|---:|---:|---:|---:|---:|"]
        for n, c, avg, tot, pct in rows:
            out.append(f"| {n} | {c} | {avg:.1f} | {timed.get(n, avg):.1f} | {tot:.2f} | {pct:.2f} |")
    print("\n".join(out))


def cmd_traffic(a):
    fs = copy_scale(a.copy_fetch, "FETCH_SIZE")
    ws = copy_scale(a.copy_write, "WRITE_SIZE")
    fetch = counter_means(a.fetch, "FETCH_SIZE")
    write = counter_means(a.write, "WRITE_SIZE")
    kernels = {}
    for k in sorted(set(fetch) | set(write), key=lambda k: -fetch.get(k, (0, 0))[0]):
        if k.startswith("at::") or "copyBuffer" in k or "elementwise" in k:
            continue
        f, nf = fetch.get(k, (0.0, 0))
        w, nw = write.get(k, (0.0, 0))
        kernels[k] = {"fetch_kib_raw": round(f, 1), "write_kib_raw": round(w, 1),
                      "bytes_read": int(f * 1024 * fs), "bytes_written": int(w * 1024 * ws),
                      "dispatches": max(nf, nw)}
    data = {"workload": a.workload, "fingerprint": source_fingerprint(),
            "fetch_scale": round(fs, 4), "write_scale": round(ws, 4), "kernels": kernels}
    with open(a.out + ".json", "w") as fh:
        json.dump(data, fh, indent=1)
        fh.write("\n")
    md = [f"# HBM-side traffic per dispatch: {a.workload} layer", "",
          "Commands (from the repository root on an MI355X; one counter per run):", "",
          f"    {a.command_fetch}", f"    {a.command_write}", "",
          f"Calibration: a plain {COPY_BYTES >> 20} MiB device-to-device copy; the counters read "
          f"x{fs:.2f} (FETCH_SIZE) and x{ws:.2f} (WRITE_SIZE) below the bytes it moves, so the "
          "raw values are scaled by those factors.  Calibration commands:", "",
          f"    {a.command_copy_fetch}", f"    {a.command_copy_write}", "",
          f"Source fingerprint {data['fingerprint']} (kernel sources and build flags).", "",
          "| kernel | FETCH_SIZE KiB (raw) | read MiB (scaled) | WRITE_SIZE KiB (raw) | written MiB (scaled) |",
          "|---|---:|---:|---:|---:|"]
    for k, v in kernels.items():
        md.append(f"| {k} | {v['fetch_kib_raw']:.0f} | {v['bytes_read'] / 2**20:.1f} | "
                  f"{v['write_kib_raw']:.0f} | {v['bytes_written'] / 2**20:.1f} |")
    with open(a.out + ".md", "w") as fh:
        fh.write("\n".join(md) + "\n")
    print(f"wrote {a.out}.json and {a.out}.md")


# MI355X: GRBM_GUI_ACTIVE is collected per XCD and summed over the 8 XCDs;
# SQ_VALU_MFMA_BUSY_CYCLES is counted per SIMD and summed over 256 CUs x 4
# SIMDs.
XCDS = 8
SIMDS = 256 * 4


def counter_runs(d: str, skip: int):
    """Per kernel and counter: values of the dispatches after the first `skip`
    (in dispatch order), and per kernel the dispatch durations in ns."""
    vals = defaultdict(lambda: defaultdict(list))
    with open(_one_csv(d, "counter_collection.csv")) as fh:
        for r in csv.DictReader(fh):
            k = short_name(r["Kernel_Name"])
            vals[k][r["Counter_Name"]].append(
                (int(r["Dispatch_Id"]), float(r["Counter_Value"]),
                 int(r["End_Timestamp"]) - int(r["Start_Timestamp"])))
    out = {}
    for k, per in vals.items():
        out[k] = {}
        for c, v in per.items():
            v.sort()
            tail = v[skip:] or v
            out[k][c] = ([x[1] for x in tail], [x[2] for x in tail])
    return out


def cmd_counters(a):
    """MFMA utilisation at the running clock, the clock itself and the L2 hit
    rate per kernel, from a pass with GRBM_GUI_ACTIVE, SQ_VALU_MFMA_BUSY_CYCLES
    and SQ_INSTS_VALU_MFMA_MOPS_BF16 and a pass with TCC_HIT_sum and
    TCC_MISS_sum."""
    m = counter_runs(a.mfma, a.skip)
    l2 = counter_runs(a.l2, a.skip)
    mean = lambda xs: sum(xs) / len(xs)
    rows = []
    for k, c in m.items():
        if "GRBM_GUI_ACTIVE" not in c or k.startswith("at::") or "elementwise" in k:
            continue
        gui, durs = c["GRBM_GUI_ACTIVE"]
        ns = mean(durs)
        cycles = mean(gui) / XCDS
        busy = mean(c.get("SQ_VALU_MFMA_BUSY_CYCLES", ([0.0], []))[0])
        mops = mean(c.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", ([0.0], []))[0])
        hit = miss = None
        if k in l2 and "TCC_HIT_sum" in l2[k]:
            hit, miss = mean(l2[k]["TCC_HIT_sum"][0]), mean(l2[k]["TCC_MISS_sum"][0])
        rows.append((ns, k, len(durs), cycles / ns, busy / (SIMDS * cycles) if cycles else 0.0,
                     mops * 512 / ns / 1e3, None if hit is None or hit + miss == 0 else hit / (hit + miss)))
    rows.sort(reverse=True)
    out = [f"# {a.title}", "", "Commands (from the repository root on an MI355X; one pass each):", "",
           f"    {a.command_mfma}", f"    {a.command_l2}", ""]
    if a.note:
        out += [a.note, ""]
    out += [f"Averages over the dispatches after the first {a.skip} of each kernel.  clock = "
            f"GRBM_GUI_ACTIVE / {XCDS} (summed over the XCDs) / dispatch time; MFMA busy = "
            f"SQ_VALU_MFMA_BUSY_CYCLES / ({SIMDS} SIMDs x clock cycles), the share of the matrix "
            "cores' time at the running clock; bf16 TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 / "
            "dispatch time (it counts the MFMAs issued, so rows of a partial 32-row block count "
            "in full); L2 hit = TCC_HIT / (TCC_HIT + TCC_MISS).  Dispatch times are under the "
            "profiler; the clock is left out for dispatches under 100 us, whose busy window is "
            "wider than their timestamps.", "",
            "| kernel | dispatches | us | clock GHz | MFMA busy % | bf16 TFLOP/s | L2 hit % |",
            "|---|---:|---:|---:|---:|---:|---:|"]
    for ns, k, n, ghz, util, tf, l2h in rows:
        l2s = "" if l2h is None else f"{100 * l2h:.1f}"
        ghzs = f"{ghz:.2f}" if ns >= 100e3 else ""   # short dispatches: the busy window is wider
        mf = (f"{100 * util:.1f}", f"{tf:.0f}") if tf > 0 else ("", "")
        out.append(f"| {k} | {n} | {ns / 1e3:.1f} | {ghzs} | {mf[0]} | {mf[1]} | {l2s} |")
    print("\n".join(out))


def traffic_bytes(call: str, workload: str):
    """HBM bytes (read + written) per dispatch of the kernel behind `call`, from
    profiles/<workload>_hbm_traffic.json, or None if absent or taken on other
    kernel sources."""
    path = os.path.join(PROFILES, f"{workload}_hbm_traffic.json")
    pat = CALL_KERNEL.get(call)
    if not pat or not os.path.exists(path):
        return None
    with open(path) as fh:
        data = json.load(fh)
    if data.get("fingerprint") != source_fingerprint():
        return None
    for k, v in data["kernels"].items():
        if re.match(pat, k):
            return v["bytes_read"] + v["bytes_written"]
    return None


def main(argv=None):
    ap = argparse.ArgumentParser()
    sp = ap.add_subparsers(dest="cmd", required=True)
    s = sp.add_parser("stats")
    s.add_argument("dir")
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--note", default="")
    s.add_argument("--skip", type=int, default=0, help="warm-up dispatches per kernel to leave out")
    t = sp.add_parser("traffic")
    for n in ("fetch", "write", "copy-fetch", "copy-write", "workload", "out", "command-fetch",
              "command-write", "command-copy-fetch", "command-copy-write"):
        t.add_argument("--" + n, required=True)
    c = sp.add_parser("counters")
    for n in ("mfma", "l2", "title", "command-mfma", "command-l2"):
        c.add_argument("--" + n, required=True)
    c.add_argument("--note", default="")
    c.add_argument("--skip", type=int, default=0, help="warm-up dispatches per kernel to leave out")
    a = ap.parse_args(argv)
    {"stats": cmd_stats, "traffic": cmd_traffic, "counters": cmd_counters}[a.cmd](a)


if __name__ == "__main__":
    main()
