"""Short text / JSON summaries of rocprofv3 output for the library's kernels.

    kt       --dir D --title T --command C [--bench-json F] --out profiles/<name>.txt
             per-kernel calls and durations from `rocprofv3 --kernel-trace --stats`
    traffic  --fetch-dir D1 --write-dir D2 --workload W --copy-bytes B --command-fetch C1
             --command-write C2 --out profiles/traffic_<W>.json
             FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel role, with the counters of
             the plain device copy of B bytes that bench.py --copy-calibration B runs last
    mfma     --dir D --workload W --command C [--append] --out profiles/<name>.txt
             MFMA busy share, executed FP8 flops and clock per GEMM kernel from
             SQ_VALU_MFMA_BUSY_CYCLES, SQ_INSTS_VALU_MFMA_MOPS_F8, SQ_BUSY_CU_CYCLES, GRBM_GUI_ACTIVE
    mem      --dir D --workload W --command C [--append] --out profiles/<name>.txt
             L2-miss reads per GEMM / combine kernel: count, mean latency and mean number in
             flight (TCC_EA0_RDREQ, TCC_EA0_RDREQ_LEVEL) and the share of cycles the read
             interface stalled for DRAM or GMI credits, against GRBM_GUI_ACTIVE

Kernel roles come from the demangled names: bs_gemm_kernel<Cfg<mode, BM, B rows, waves, wave
rows, stages>, ...> and big_gemm_kernel<mode, ...> with mode 0 dense, 1 gate/up, 2 down.
Pure host code over CSV files.
"""
import argparse
import csv
import glob
import hashlib
import json
import os
import re

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
CSRC = os.path.join(ROOT, "fp8_block_scaled_grouped_amd", "csrc")
MODES = {0: "dense", 1: "g1u1", 2: "down"}


def source_hash():
    """Hash of every kernel source and compiled-in table (bench.py checks it before using counters)."""
    h = hashlib.sha256()
    for f in sorted(os.listdir(CSRC)):
        if f.endswith((".hip", ".h", ".cpp")):
            h.update(f.encode())
            with open(os.path.join(CSRC, f), "rb") as fh:
                h.update(fh.read())
    return h.hexdigest()[:16]


def role(name):
    """(role, readable label) of a kernel name, role None for kernels outside the library."""
    m = re.search(r"bs_gemm_kernel<[^<]*Cfg<(\d+), (\d+), (\d+), (\d+), (\d+), (\d+)>", name)
    if m:
        mode, bm, bnb, nw, _, st = (int(x) for x in m.groups())
        return MODES[mode], "%s (BM %d, B rows %d, %d waves, %d stages)" % (MODES[mode], bm, bnb, nw, st)
    m = re.search(r"dense_small_kernel<(\d+), (true|false)>", name)
    if m:
        return "dense", "dense small-M (%d row tiles, 8 waves, %s B)" % (
            int(m.group(1)), "pre-shuffled" if m.group(2) == "true" else "plain")
    m = re.search(r"big_gemm_kernel<(\d+)", name)
    if m:
        mode = int(m.group(1))
        return MODES[mode], "%s (BM 256, B rows 256, 8 waves)" % MODES[mode]
    for key in ("fused_moe_kernel", "splitk_reduce_kernel", "combine_kernel", "quant_1x128_kernel",
                "sort_count_kernel", "sort_scan_kernel", "sort_scatter_kernel", "sort_small_kernel",
                "grouped_topk_reg_kernel", "grouped_topk_kernel", "shuffle_128x128_kernel"):
        if key in name:
            return key.replace("_kernel", ""), key
    if "copyBuffer" in name:
        return "copy", "__amd_rocclr_copyBuffer"
    return None, name


def find(d, suffix):
    fs = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not fs:
        raise SystemExit("no *%s under %s" % (suffix, d))
    return fs


def rows(path):
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def cmd_kt(a):
    stats = []
    for f in find(a.dir, "kernel_stats.csv"):
        stats += rows(f)
    lines = ["rocprofv3 kernel trace: %s" % a.title, "", "command (<repo> = the repository root, <out> = any output directory):",
             "  " + a.command, "", "libmoe355 kernels (input generation, weight copies and the oracle's host copies are "
             "torch / runtime kernels, omitted):",
             "  %-48s %7s %12s %12s %12s" % ("kernel", "calls", "avg us", "min us", "max us")]
    lib = []
    for r in stats:
        rl, label = role(r["Name"])
        if rl is None or rl == "copy":
            continue
        lib.append((float(r["TotalDurationNs"]), label, int(r["Calls"]), float(r["AverageNs"]) / 1e3,
                    float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
    for _, label, calls, avg, mn, mx in sorted(lib, reverse=True):
        lines.append("  %-48s %7d %12.1f %12.1f %12.1f" % (label, calls, avg, mn, mx))
    if a.bench_json:
        with open(a.bench_json) as f:
            js = [json.loads(x) for x in f if x.startswith("{")]
        if js:
            b = js[-1]
            lines += ["", "bench.py line printed by the same run (its HIP-event timings, taken under the profiler):",
                      "  ms_per_step %.4f  value %.1f %s" % (b["ms_per_step"], b["value"], b["unit"])]
            for key, sub in (("", b), ("decode: ", b.get("decode"))):
                if sub and "roofline" in sub:
                    r = sub["roofline"]
                    lines.append("  %sroofline: kernel %s  kernel_ms %.4f  achieved %.1f %s  frac %.3f of %s peak %g" % (
                        key, r.get("kernel"), r.get("kernel_ms", float("nan")), r["achieved"], r["unit"], r["frac"],
                        r["bound"], r["peak"]))
    with open(a.out, "w") as f:
        f.write("\n".join(lines) + "\n")


def per_role(d, counter):
    """{role: (mean counter value per dispatch, dispatches)} and the copy dispatches' values."""
    acc, copies = {}, []
    for f in find(d, "counter_collection.csv"):
        for r in rows(f):
            if r["Counter_Name"] != counter:
                continue
            rl, _ = role(r["Kernel_Name"])
            v = float(r["Counter_Value"])
            if rl == "copy":
                copies.append((int(r.get("Dispatch_Id", 0) or 0), v))
            elif rl is not None:
                acc.setdefault(rl, []).append(v)
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}, [v for _, v in sorted(copies)]


def cmd_traffic(a):
    fetch, fcopy = per_role(a.fetch_dir, "FETCH_SIZE")
    write, wcopy = per_role(a.write_dir, "WRITE_SIZE")
    if len(fcopy) < 3 or len(wcopy) < 3:
        raise SystemExit("the calibration copies are missing (bench.py --copy-calibration)")
    cal = {"bytes": a.copy_bytes, "FETCH_SIZE_KiB": sum(fcopy[-3:]) / 3, "WRITE_SIZE_KiB": sum(wcopy[-3:]) / 3}
    kernels = {}
    for k in sorted(set(fetch) & set(write)):
        fb = fetch[k][0] * a.copy_bytes / cal["FETCH_SIZE_KiB"]
        wb = write[k][0] * a.copy_bytes / cal["WRITE_SIZE_KiB"]
        kernels[k] = {"FETCH_SIZE_KiB": fetch[k][0], "WRITE_SIZE_KiB": write[k][0], "dispatches": fetch[k][1],
                      "fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb}
    out = {"workload": a.workload, "source_hash": source_hash(),
           "sources": "every file of fp8_block_scaled_grouped_amd/csrc (kernels and compiled-in tables)",
           "commands": {"FETCH_SIZE": a.command_fetch, "WRITE_SIZE": a.command_write},
           "note": "KiB per dispatch averaged over the profiled dispatches of each kernel role; the last three "
                   "dispatches are a plain device copy of copy_calibration.bytes (__amd_rocclr_copyBuffer) "
                   "whose counters scale each counter to bytes",
           "kernels": kernels, "copy_calibration": cal}
    with open(a.out, "w") as f:
        json.dump(out, f, indent=1)
        f.write("\n")


def cmd_mfma(a):
    per = {}
    for f in find(a.dir, "counter_collection.csv"):
        for r in rows(f):
            rl, label = role(r["Kernel_Name"])
            if rl not in MODES.values() and rl != "fused_moe":
                continue
            key = (label, r.get("Dispatch_Id") or r.get("Correlation_Id"))
            d = per.setdefault(key, {"dur": (float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) if
                                     r.get("End_Timestamp") else float("nan")})
            d[r["Counter_Name"]] = d.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    by = {}
    for (label, _), d in per.items():
        by.setdefault(label, []).append(d)
    lines = []
    if not a.append:
        lines += ["rocprofv3 FP8 MFMA counters per libmoe355 GEMM kernel", "",
                  "GRBM_GUI_ACTIVE reads as the sum over the 8 XCDs (GUI / 8 / kernel duration gives the clock);",
                  "MFMA busy = SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / 8 x 1024 SIMDs); CU busy =",
                  "SQ_BUSY_CU_CYCLES / (GUI / 8 x 256); executed FP8 TFLOP/s = SQ_INSTS_VALU_MFMA_MOPS_F8 x 512 /",
                  "duration (one 16x16x128 MFMA counts 128 MOPs for 65,536 flops). Durations are under the profiler.", ""]
    lines += ["workload %s; command (<repo> = the repository root, <out> = any output directory):" % a.workload,
              "  " + a.command,
              "  %-44s %6s %9s %9s %8s %9s %10s" % ("kernel", "calls", "dur us", "clock GHz", "CU busy", "MFMA busy",
                                                    "exec TF/s")]
    for label, ds in sorted(by.items()):
        n = len(ds)
        dur = sum(d["dur"] for d in ds) / n  # ns
        gui = sum(d.get("GRBM_GUI_ACTIVE", 0) for d in ds) / n / 8
        busy = sum(d.get("SQ_VALU_MFMA_BUSY_CYCLES", 0) for d in ds) / n
        cu = sum(d.get("SQ_BUSY_CU_CYCLES", 0) for d in ds) / n
        mops = sum(d.get("SQ_INSTS_VALU_MFMA_MOPS_F8", 0) for d in ds) / n
        clk = gui / dur if dur > 0 else float("nan")
        lines.append("  %-44s %6d %9.1f %9.2f %7.1f%% %8.1f%% %10.0f" % (
            label, n, dur / 1e3, clk, 100 * cu / max(gui * 256, 1), 100 * busy / max(gui * 1024, 1),
            mops * 512 / max(dur, 1) / 1e3))
    with open(a.out, "a" if a.append else "w") as f:
        f.write("\n".join(lines) + "\n\n")


def mem_rows(d):
    """Per kernel label: averages over its dispatches of the memory-side counters."""
    per = {}
    for f in find(d, "counter_collection.csv"):
        for r in rows(f):
            rl, label = role(r["Kernel_Name"])
            if rl not in ("dense", "g1u1", "down", "combine", "fused_moe"):
                continue
            key = (label, r.get("Dispatch_Id") or r.get("Correlation_Id"))
            x = per.setdefault(key, {"dur": float(r["End_Timestamp"]) - float(r["Start_Timestamp"])})
            x[r["Counter_Name"]] = x.get(r["Counter_Name"], 0.0) + float(r["Counter_Value"])
    by = {}
    for (label, _), x in per.items():
        by.setdefault(label, []).append(x)
    out = {}
    for label, xs in by.items():
        n = len(xs)
        avg = lambda k: sum(x.get(k, 0.0) for x in xs) / n
        gui = avg("GRBM_GUI_ACTIVE") / 8  # cycles of one XCD (the counter sums the 8)
        req, lvl = avg("TCC_EA0_RDREQ_sum"), avg("TCC_EA0_RDREQ_LEVEL_sum")
        chan = gui * 128  # 16 L2 channels per XCD, 8 XCDs
        out[label] = {"calls": n, "dur_us": avg("dur") / 1e3, "clock_ghz": gui / max(avg("dur"), 1.0),
                      "reads": req, "latency_cycles": lvl / max(req, 1.0), "in_flight": lvl / max(gui, 1.0),
                      "dram_stall": avg("TCC_EA0_RDREQ_DRAM_CREDIT_STALL_sum") / max(chan, 1.0),
                      "gmi_stall": avg("TCC_EA0_RDREQ_GMI_CREDIT_STALL_sum") / max(chan, 1.0)}
    return out


def cmd_mem(a):
    lines = []
    if not a.append:
        lines += ["rocprofv3 memory-side counters per libmoe355 kernel (L2 misses)", "",
                  "reads = TCC_EA0_RDREQ_sum (requests from the L2s to memory, mostly 128 B); latency =",
                  "TCC_EA0_RDREQ_LEVEL_sum / reads (cycles from request to data); in flight = LEVEL_sum /",
                  "(GRBM_GUI_ACTIVE / 8), the mean number of such reads outstanding over the chip; DRAM / GMI",
                  "stall = TCC_EA0_RDREQ_{DRAM,GMI}_CREDIT_STALL_sum / (128 L2 channels x GUI / 8), the share of",
                  "cycles a channel's read interface waited for credits. Durations are under the profiler.", ""]
    lines += ["workload %s; command (<repo> = the repository root, <out> = any output directory):" % a.workload,
              "  " + a.command,
              "  %-44s %6s %9s %9s %12s %9s %10s %7s %7s" % ("kernel", "calls", "dur us", "clock GHz", "reads",
                                                              "latency", "in flight", "DRAM", "GMI")]
    for label, r in sorted(mem_rows(a.dir).items()):
        lines.append("  %-44s %6d %9.1f %9.2f %12.4g %9.0f %10.0f %6.2f%% %6.2f%%" % (
            label, r["calls"], r["dur_us"], r["clock_ghz"], r["reads"], r["latency_cycles"], r["in_flight"],
            100 * r["dram_stall"], 100 * r["gmi_stall"]))
    with open(a.out, "a" if a.append else "w") as f:
        f.write("\n".join(lines) + "\n\n")


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    k = sub.add_parser("kt")
    k.add_argument("--dir", required=True)
    k.add_argument("--title", required=True)
    k.add_argument("--command", required=True)
    k.add_argument("--bench-json")
    k.add_argument("--out", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch-dir", required=True)
    t.add_argument("--write-dir", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--command-fetch", required=True)
    t.add_argument("--command-write", required=True)
    t.add_argument("--out", required=True)
    m = sub.add_parser("mfma")
    m.add_argument("--dir", required=True)
    m.add_argument("--workload", required=True)
    m.add_argument("--command", required=True)
    m.add_argument("--append", action="store_true")
    m.add_argument("--out", required=True)
    e = sub.add_parser("mem")
    e.add_argument("--dir", required=True)
    e.add_argument("--workload", required=True)
    e.add_argument("--command", required=True)
    e.add_argument("--append", action="store_true")
    e.add_argument("--out", required=True)
    a = ap.parse_args()
    {"kt": cmd_kt, "traffic": cmd_traffic, "mfma": cmd_mfma, "mem": cmd_mem}[a.cmd](a)


if __name__ == "__main__":
    main()
