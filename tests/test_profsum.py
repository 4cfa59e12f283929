"""Host-side checks of the rocprofv3 summary tool (no GPU): the kernel-time
table with and without warm-up dispatches, the copy-calibrated traffic
scaling, and the fingerprint that ties a traffic file to the kernel code."""
import csv
import json
import os

from combine_moe_route_histogram_amd import profsum as P


def _write(path, header, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


def test_stats_table_leaves_out_warmup(tmp_path, capsys):
    d = tmp_path / "prof"
    d.mkdir()
    _write(d / "run_kernel_stats.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage"],
           [["void moe::k_a(int)", 3, 600000, 200000, 75.0], ["void moe::k_b(int)", 3, 200000, 66666, 25.0]])
    trace = []
    for i, (name, dur) in enumerate([("void moe::k_a(int)", 400000), ("void moe::k_b(int)", 100000),
                                     ("void moe::k_a(int)", 100000), ("void moe::k_b(int)", 50000),
                                     ("void moe::k_a(int)", 100000), ("void moe::k_b(int)", 50000)]):
        trace.append([name, 1000 * i, 1000 * i + dur])
    _write(d / "run_kernel_trace.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp"], trace)
    P.main(["stats", str(d), "--title", "T", "--command", "C", "--skip", "1"])
    out = capsys.readouterr().out
    row_a = [l for l in out.splitlines() if l.startswith("| k_a ")][0]
    cells = [c.strip() for c in row_a.strip("|").split("|")]
    assert cells[1] == "3" and cells[2] == "200.0" and cells[3] == "100.0"   # timed avg: last two


def test_traffic_scaling_and_fingerprint(tmp_path):
    def pmc(dirname, counter, rows):
        d = tmp_path / dirname
        d.mkdir()
        _write(d / "p_counter_collection.csv", ["Kernel_Name", "Counter_Name", "Counter_Value"],
               [[k, counter, v] for k, v in rows])
        return str(d)
    copy_kib = P.COPY_BYTES / 1024.0
    f = pmc("fetch", "FETCH_SIZE", [("void moe::gemm(int)", 1000.0), ("void moe::gemm(int)", 3000.0)])
    w = pmc("write", "WRITE_SIZE", [("void moe::gemm(int)", 500.0)])
    cf = pmc("copy_fetch", "FETCH_SIZE", [("void copyBuffer(int)", copy_kib / 2)])
    cw = pmc("copy_write", "WRITE_SIZE", [("void copyBuffer(int)", copy_kib)])
    out = str(tmp_path / "traffic")
    P.main(["traffic", "--fetch", f, "--write", w, "--copy-fetch", cf, "--copy-write", cw,
            "--workload", "x", "--out", out, "--command-fetch", "a", "--command-write", "b",
            "--command-copy-fetch", "c", "--command-copy-write", "d"])
    data = json.load(open(out + ".json"))
    k = data["kernels"]["gemm"]
    assert data["fetch_scale"] == 2.0 and data["write_scale"] == 1.0
    assert k["bytes_read"] == 2000 * 1024 * 2 and k["bytes_written"] == 500 * 1024
    assert data["fingerprint"] == P.source_fingerprint()


def test_fingerprint_ignores_comments():
    a = "int f(int x) { return x + 1; }  // one\n/* two */"
    b = "int f(int x) {\n  return x + 1;\n}\n"
    assert P._code_only(a) == P._code_only(b)
    assert P._code_only(a) != P._code_only(a.replace("+ 1", "+ 2"))


def test_counters_clock_mfma_busy_and_l2_hit(tmp_path, capsys):
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    ns = 1_000_000                                   # 1 ms per dispatch
    cycles = 1_600_000                               # 1.6 GHz per XCD
    busy = 0.5 * P.SIMDS * cycles                    # matrix cores busy half the time
    mfma, l2 = tmp_path / "mfma", tmp_path / "l2"
    mfma.mkdir()
    l2.mkdir()
    rows = []
    for i, scale in ((1, 3.0), (2, 1.0), (3, 1.0)):  # dispatch 1: warm-up, left out
        for c, v in (("GRBM_GUI_ACTIVE", cycles * P.XCDS * scale), ("SQ_VALU_MFMA_BUSY_CYCLES", busy),
                     ("SQ_INSTS_VALU_MFMA_MOPS_BF16", 1e12 / 512)):
            rows.append([i, "void moe::gemm(int)", c, v, 0, ns])
    _write(mfma / "p_counter_collection.csv", hdr, rows)
    _write(l2 / "p_counter_collection.csv", hdr,
           [[i, "void moe::gemm(int)", c, v, 0, ns] for i in (1, 2, 3)
            for c, v in (("TCC_HIT_sum", 300.0), ("TCC_MISS_sum", 100.0))])
    P.main(["counters", "--mfma", str(mfma), "--l2", str(l2), "--title", "T", "--command-mfma", "a",
            "--command-l2", "b", "--skip", "1"])
    row = [l for l in capsys.readouterr().out.splitlines() if l.startswith("| gemm ")][0]
    cells = [c.strip() for c in row.strip("|").split("|")]
    assert cells[1:] == ["2", "1000.0", "1.60", "50.0", "1000", "75.0"]
