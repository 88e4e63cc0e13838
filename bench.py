#!/usr/bin/env python3
"""Benchmark of the MI355X attention backward (dQ, dK, dV).

One step = one whole backward (dq then main; with --dq-accumulate preprocess,
main, dq_convert) over one workload, by default the headline one: B=2, H=32,
Hk=8, Sq=Sk=4096, D=128, causal, bf16, inputs resident in HBM (--config picks
another of workloads.py, packed variable-length batches included).  Prints ONE
JSON line.

FLOP convention: 2.5 x the forward's 4*B*H*Sq*Sk*D, halved for causal (packed
batches: B*Sq*Sk replaced by the sum of the squared sequence lengths).  The
exact count over the visible (query, key) pairs (bottom-right causal
alignment) is reported beside it, since the convention undercounts Sq < Sk.
The roofline object is for the main kernel (the dominant one), timed with
HIP events recorded on the stream it is launched on.

Inputs: Q, K, V, dO from the seeded generator (workloads.py); O and LSE from a
plain fp32 torch forward on the GPU, one (sequence, head) at a time (input
preparation only, not timed).  The CPU baseline leg times the fp64 oracle on
a bounded sample.

--forward measures the forward kernel (O and LSE) on the same workload
instead and prints one JSON line of the same shape for it (not the headline
metric).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "bwd TFLOP/s (dQ+dK+dV) bf16 and % of MFMA peak, S=4096 D=128 causal GQA"
PEAK_BF16_TFLOPS = 2500.0     # MI355X published dense bf16 MFMA peak
PEAK_HBM_GBS = 8000.0         # MI355X published HBM3E bandwidth


# Sources of the key-tile kernel: the committed HBM-traffic summary applies to
# the kernel built from exactly these files (sha256 recorded with it).
KERNEL_SOURCES = ["attention_backward_fa2_amd/csrc/fa_main.hip",
                  "attention_backward_fa2_amd/csrc/fa_mfma.h",
                  "attention_backward_fa2_amd/csrc/fa_philox.h",
                  "attention_backward_fa2_amd/csrc/fa_internal.h"]
TRAFFIC_SUMMARY = "profiles/hbm_traffic_main_kernel_gqa_b2_h32_hk8_s4096_d128_causal.json"
TRACE_SUMMARY = "profiles/kernel_trace_gqa_b2_h32_hk8_s4096_d128_causal.md"
MAIN_KERNEL = "fa_bwd_main_kernel<128, false, false, false, false, 0>"
# The headline's other launch, the query-tile dQ kernel, and its sources.
DQ_KERNEL = "fa_bwd_dq_kernel<128, false, false, false, 0, false>"
DQ_SOURCES = ["attention_backward_fa2_amd/csrc/fa_dq.hip",
              "attention_backward_fa2_amd/csrc/fa_mfma.h",
              "attention_backward_fa2_amd/csrc/fa_philox.h",
              "attention_backward_fa2_amd/csrc/fa_internal.h"]


def kernel_source_hash(files=None):
    import hashlib
    h = hashlib.sha256()
    for f in files or KERNEL_SOURCES:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def committed_traffic():
    """Per-launch HBM bytes of the key-tile kernel from the committed counter
    summary, or None if there is none or the kernel changed since."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_sha256") != kernel_source_hash():
        return None
    return d.get("traffic_bytes_per_launch")


def committed_dq_traffic():
    """Per-launch HBM bytes of the dQ kernel from the same committed summary,
    or None if there is none or that kernel changed since."""
    path = os.path.join(ROOT, TRAFFIC_SUMMARY)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh).get("dq_kernel", {})
    if d.get("source_sha256") != kernel_source_hash(DQ_SOURCES):
        return None
    return d.get("traffic_bytes_per_launch")


PEAK_CLOCK_MHZ = 2400.0       # the clock the published peak is quoted at
CLOCK_SUMMARY = "profiles/clock_gqa_b2_h32_hk8_s4096_d128_causal.json"


def committed_clock():
    """Clock (MHz) the key-tile kernel ran at in the committed GRBM-counter
    profile, or None if there is none or the kernel changed since."""
    path = os.path.join(ROOT, CLOCK_SUMMARY)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        d = json.load(fh)
    if d.get("source_sha256") != kernel_source_hash():
        return None
    k = d.get("kernels", {}).get(MAIN_KERNEL)
    return {"mhz": k["mhz"]} if k else None


def tile_kernel_GBs(kms, headline):
    """Counter-measured HBM bytes per launch of the key-tile and dQ kernels
    (committed profile, current sources) over their HIP-event times."""
    if not headline:
        return {}
    out = {}
    for name, b in (("main", committed_traffic()), ("dq", committed_dq_traffic())):
        if b is not None and kms.get(name):
            out[name] = round(b / (kms[name] * 1e-3) / 1e9, 1)
    return out


def headline_path(args, wl):
    """True for the kernel and workload the committed profiles cover."""
    return (not args.dq_accumulate and wl.name == WORKLOAD_TAG and not wl.window
            and not wl.softcap and not wl.dropout)


def _csv_rows(path):
    import csv
    with open(path) as fh:
        return list(csv.DictReader(fh))


def _find(root, suffix):
    for dp, _, files in os.walk(root):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(dp, f)
    raise FileNotFoundError("%s under %s" % (suffix, root))


WORKLOAD_TAG = "gqa_b2_h32_hk8_s4096_d128_causal"
TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d {prof}/trace -o c3 -- "
             "python bench.py")
FWD_TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d {prof}/fwd_trace -o c3 -- "
                 "python bench.py --forward")
PMC_RUN = "python bench.py --no-cpu-baseline --steps 3 --warmup 1"
SQ_PASSES = [
    "SQ_WAVES SQ_WAVE_CYCLES SQ_BUSY_CYCLES SQ_WAIT_ANY SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY "
    "SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS",
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_VALU_MFMA_BUSY_CYCLES "
    "SQ_LDS_BANK_CONFLICT SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_VMEM",
    "TCC_HIT_sum TCC_MISS_sum TCC_REQ_sum"]


def _kname(raw):
    return raw.replace("void fa::", "").split("(fa::Params)")[0]


def _pmc_means(path):
    import collections
    acc = collections.defaultdict(list)
    for r in _csv_rows(path):
        acc[(r["Kernel_Name"], r["Counter_Name"])].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def summarize_variant_trace(trace_dir, bench_args, out_dir):
    """Write profiles/kernel_trace_<workload>.md from the outputs of
        rocprofv3 --kernel-trace --stats -f csv -d TRACE_DIR -o c3 --
            python bench.py BENCH_ARGS > TRACE_DIR.log
    (a variant of the headline workload: another head dim, window, cap,
    dropout or the forward), named for the workload its bench line reports."""
    stats = _csv_rows(_find(trace_dir, "kernel_stats.csv"))
    trace = _csv_rows(_find(trace_dir, "kernel_trace.csv"))
    bench_line = None
    with open(trace_dir.rstrip("/") + ".log") as fh:
        for line in fh:
            if line.startswith("{") and '"metric"' in line:
                bench_line = json.loads(line)
    steps, cfg = bench_line["steps"], bench_line["config"]
    per_kernel = {}
    for r in trace:
        if "fa::" in r["Kernel_Name"]:
            per_kernel.setdefault(_kname(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    rel = os.path.relpath(trace_dir, ROOT) if os.path.isabs(trace_dir) else trace_dir
    lines = ["# Kernel trace: %s%s" % ("forward, " if cfg.get("pass") == "forward" else "",
                                        cfg["workload"]), "",
             "Workload: `%s` (%s)." % (json.dumps(cfg), bench_line["metric"]), "",
             "Command (repo root, MI355X):", "",
             "    rocprofv3 --kernel-trace --stats -f csv -d %s -o c3 -- python bench.py %s" % (
                 rel, bench_args), "",
             "| kernel | calls | average (us) | min (us) | max (us) | average of the %d timed "
             "steps (us) |" % steps, "|---|---|---|---|---|---|"]
    for r in stats:
        if "fa::" in r["Name"]:
            name = _kname(r["Name"])
            timed = per_kernel[name][-steps:]
            lines.append("| %s | %s | %.1f | %.1f | %.1f | %.1f |" % (
                name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, sum(timed) / len(timed)))
    lines += ["", "Calls include the warm-up and any forward calls that produce the "
              "backward's inputs; the timed-steps column averages the last %d calls." % steps, "",
              "The same run's bench line: %.4f ms per step, %.1f TFLOP/s; per-kernel HIP-event "
              "times (ms per launch): `%s`." % (bench_line["ms_per_step"], bench_line["value"],
                                                json.dumps(bench_line.get("kernel_ms")))]
    fwd = "fwd_" if cfg.get("pass") == "forward" else ""
    path = os.path.join(out_dir, "kernel_trace_%s%s.md" % (fwd, cfg["workload"]))
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def summarize_profile(prof_dir, out_dir):
    """Write the profile summaries committed under profiles/ from the
    rocprofv3 outputs of the commands they list, run from the repo root
    with the outputs under PROF_DIR (trace/ + trace.log, FETCH_SIZE/,
    WRITE_SIZE/, copy_FETCH_SIZE/, copy_WRITE_SIZE/, sq1/, sq2/)."""
    # the commands as run: outputs under PROF_DIR (relative to the repo root)
    rel = os.path.relpath(prof_dir, ROOT) if os.path.isabs(prof_dir) else prof_dir.rstrip("/")

    def cmd(c):
        return c.replace("{prof}", rel)
    # -- kernel trace: per-kernel durations, all calls and the timed steps --
    stats = _csv_rows(_find(os.path.join(prof_dir, "trace"), "kernel_stats.csv"))
    trace = _csv_rows(_find(os.path.join(prof_dir, "trace"), "kernel_trace.csv"))
    bench_line = None
    with open(os.path.join(prof_dir, "trace.log")) as fh:
        for line in fh:
            if line.startswith("{") and '"metric"' in line:
                bench_line = json.loads(line)
    steps = bench_line["steps"]
    per_kernel = {}
    for r in trace:
        if "fa::" in r["Kernel_Name"]:
            per_kernel.setdefault(_kname(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    lines = ["# Kernel trace: %s" % WORKLOAD_TAG, "",
             "B=2, H=32, Hk=8, Sq=Sk=4096, D=128, causal, bf16; dQ by the separate "
             "query-tile kernel (the default path of `fa_bwd`).", "",
             "Command (repo root, MI355X):", "", "    " + cmd(TRACE_CMD), "",
             "| kernel | calls | average (us) | min (us) | max (us) | average of the %d timed "
             "steps (us) |" % steps, "|---|---|---|---|---|---|"]
    for r in stats:
        if "fa::" in r["Name"]:
            name = _kname(r["Name"])
            timed = per_kernel[name][-steps:]
            lines.append("| %s | %s | %.1f | %.1f | %.1f | %.1f |" % (
                name, r["Calls"], float(r["AverageNs"]) / 1e3, float(r["MinNs"]) / 1e3,
                float(r["MaxNs"]) / 1e3, sum(timed) / len(timed)))
    lines += ["", "Calls = warm-up + timed steps of bench.py (%d + %d)." % (
        bench_line["warmup"], steps), "",
        "The same run's bench line measured these kernels with HIP events on the launch "
        "stream (ms per launch): `%s`; whole step %.4f ms, %.1f TFLOP/s." % (
            json.dumps(bench_line["kernel_ms"]), bench_line["ms_per_step"],
            bench_line["value"])]
    with open(os.path.join(out_dir, os.path.basename(TRACE_SUMMARY)), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    # -- HBM traffic of the key-tile kernel, scaled by a plain copy --
    res = {"kernel": MAIN_KERNEL, "workload": WORKLOAD_TAG,
           "source_files": KERNEL_SOURCES, "source_sha256": kernel_source_hash(),
           "commands": [
               "rocprofv3 --pmc FETCH_SIZE -f csv -d {prof}/FETCH_SIZE -o c3 -- " + PMC_RUN,
               "rocprofv3 --pmc WRITE_SIZE -f csv -d {prof}/WRITE_SIZE -o c3 -- " + PMC_RUN,
               "rocprofv3 --pmc FETCH_SIZE -f csv -d {prof}/copy_FETCH_SIZE -o copy -- "
               "python bench.py --copy-calibration",
               "rocprofv3 --pmc WRITE_SIZE -f csv -d {prof}/copy_WRITE_SIZE -o copy -- "
               "python bench.py --copy-calibration"],
           "note": "kib_per_dispatch is the counter's mean over the kernel's dispatches; "
                   "scale_factor = copied bytes / (counter KiB * 1024) of a 1 GiB "
                   "device-to-device copy"}
    res["commands"] = [cmd(c) for c in res["commands"]]
    copy_bytes = float(1 << 30)
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        m = _pmc_means(_find(os.path.join(prof_dir, c), "counter_collection.csv"))
        kib, n = next(v for (k, cn), v in m.items() if MAIN_KERNEL in k and cn == c)
        cm = _pmc_means(_find(os.path.join(prof_dir, "copy_" + c), "counter_collection.csv"))
        ckib, cn_ = next(v for (k, cn), v in cm.items() if "copyBuffer" in k and cn == c)
        factor = copy_bytes / (ckib * 1024.0)
        res[c] = {"kib_per_dispatch": kib, "dispatches": n, "copy_kib_per_dispatch": ckib,
                  "copy_dispatches": cn_, "scale_factor": factor,
                  "bytes_per_launch": kib * 1024.0 * factor}
    res["traffic_bytes_per_launch"] = (res["FETCH_SIZE"]["bytes_per_launch"] +
                                       res["WRITE_SIZE"]["bytes_per_launch"])
    # The dQ kernel of the same runs, with its compulsory bytes: Q, dO, O
    # (for the row sums), K, V and LSE read, dQ and the two row vectors
    # written.
    import workloads as W
    wl = W.WORKLOADS[3]
    rows, krows = wl.batch * wl.seqlen_q * wl.heads, wl.batch * wl.seqlen_k * wl.heads_k
    dq = {"kernel": DQ_KERNEL, "source_files": DQ_SOURCES,
          "source_sha256": kernel_source_hash(DQ_SOURCES),
          "algorithmic_bytes_per_launch": (3 * rows * wl.head_dim * 2 + 2 * krows * wl.head_dim * 2
                                           + rows * 4 + rows * wl.head_dim * 2 + 2 * rows * 4)}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        m = _pmc_means(_find(os.path.join(prof_dir, c), "counter_collection.csv"))
        kib, n = next(v for (k, cn), v in m.items() if DQ_KERNEL in k and cn == c)
        dq[c] = {"kib_per_dispatch": kib, "dispatches": n,
                 "bytes_per_launch": kib * 1024.0 * res[c]["scale_factor"]}
    dq["traffic_bytes_per_launch"] = (dq["FETCH_SIZE"]["bytes_per_launch"] +
                                      dq["WRITE_SIZE"]["bytes_per_launch"])
    res["dq_kernel"] = dq
    with open(os.path.join(out_dir, os.path.basename(TRAFFIC_SUMMARY)), "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")

    # -- SQ counters per kernel --
    sq = {}
    for sub in ["sq%d" % (i + 1) for i in range(len(SQ_PASSES))]:
        if not os.path.isdir(os.path.join(prof_dir, sub)):
            continue
        for (k, c), (v, _) in _pmc_means(
                _find(os.path.join(prof_dir, sub), "counter_collection.csv")).items():
            if "fa::" in k:
                sq.setdefault(_kname(k), {})[c] = v
    names = sorted(sq)
    cols = sorted({c for d in sq.values() for c in d})
    lines = ["# SQ counters per dispatch: %s" % WORKLOAD_TAG, "", "Commands (repo root, MI355X):", ""]
    for i, cs in enumerate(SQ_PASSES):
        lines.append(cmd("    rocprofv3 --pmc %s -f csv -d {prof}/sq%d -o c3 -- %s") % (
            cs, i + 1, PMC_RUN))
    lines += ["", "| counter | " + " | ".join(names) + " |", "|---|" + "---|" * len(names)]
    for c in cols:
        lines.append("| %s | %s |" % (c, " | ".join("%.4g" % sq[n].get(c, float("nan"))
                                                      for n in names)))
    lines += ["", "Derived (SQ_VALU_MFMA_BUSY_CYCLES is summed over the SIMDs; TCC = the L2, "
              "summed over its channels and XCDs):", ""]
    for n in names:
        d = sq[n]
        if d.get("SQ_INSTS_MFMA"):
            lines.append("- %s: %.1f VALU instructions per MFMA; %.0f MFMA busy cycles per MFMA"
                         % (n, d["SQ_INSTS_VALU"] / d["SQ_INSTS_MFMA"],
                            d["SQ_VALU_MFMA_BUSY_CYCLES"] / d["SQ_INSTS_MFMA"]))
        if d.get("TCC_HIT_sum") is not None and d.get("TCC_MISS_sum"):
            lines.append("- %s: L2 hit rate %.3f (%.4g hits, %.4g misses, %.4g requests)"
                         % (n, d["TCC_HIT_sum"] / (d["TCC_HIT_sum"] + d["TCC_MISS_sum"]),
                            d["TCC_HIT_sum"], d["TCC_MISS_sum"], d.get("TCC_REQ_sum", float("nan"))))
    with open(os.path.join(out_dir, "sq_counters_%s.md" % WORKLOAD_TAG), "w") as fh:
        fh.write("\n".join(lines) + "\n")

    # -- forward kernel trace (if that run is present) --
    if os.path.isdir(os.path.join(prof_dir, "fwd_trace")):
        stats = _csv_rows(_find(os.path.join(prof_dir, "fwd_trace"), "kernel_stats.csv"))
        fwd_line = None
        with open(os.path.join(prof_dir, "fwd_trace.log")) as fh:
            for line in fh:
                if line.startswith("{") and '"metric"' in line:
                    fwd_line = json.loads(line)
        lines = ["# Kernel trace: forward, %s" % WORKLOAD_TAG, "",
                 "B=2, H=32, Hk=8, Sq=Sk=4096, D=128, causal, bf16; O and LSE by `fa_fwd`.",
                 "", "Command (repo root, MI355X):", "", "    " + cmd(FWD_TRACE_CMD), "",
                 "| kernel | calls | average (us) | min (us) | max (us) |", "|---|---|---|---|---|"]
        for r in stats:
            if "fa::" in r["Name"]:
                lines.append("| %s | %s | %.1f | %.1f | %.1f |" % (
                    _kname(r["Name"]), r["Calls"], float(r["AverageNs"]) / 1e3,
                    float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3))
        lines += ["", "Calls = warm-up + timed steps of `bench.py --forward` (%d + %d)." % (
            fwd_line["warmup"], fwd_line["steps"]), "",
            "The same run's bench line: %.4f ms per launch (HIP events on the launch stream), "
            "%.1f TFLOP/s on the forward's two products." % (fwd_line["ms_per_step"],
                                                             fwd_line["value"])]
        with open(os.path.join(out_dir, "kernel_trace_fwd_%s.md" % WORKLOAD_TAG), "w") as fh:
            fh.write("\n".join(lines) + "\n")
    print("wrote profile summaries to", out_dir)


CLOCK_CMD = ("rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE GRBM_COUNT -f csv -d {prof}/clock "
             "-o c3 -- " + PMC_RUN)
ACC_RUN = "python bench.py --dq-accumulate --no-cpu-baseline --steps 3 --warmup 1"
ACC_TRACE_CMD = ("rocprofv3 --kernel-trace --stats -f csv -d {prof}/acc_trace -o c3 -- "
                 "python bench.py --dq-accumulate --no-cpu-baseline")


def _agent(prof_sub):
    """The GPU agent's row of a rocprofv3 run's agent_info.csv."""
    return next(r for r in _csv_rows(_find(prof_sub, "agent_info.csv"))
                if r.get("Agent_Type") == "GPU")


def summarize_clock(prof_dir, out_dir):
    """profiles/clock_<workload>.json: the clock each kernel of the headline
    backward ran at, from the GRBM cycle counters of a kernel-trace run
    (PROF_DIR/clock): busy cycles per dispatch, summed by the counter over
    the accelerator's XCDs, over the dispatch's duration."""
    rel = os.path.relpath(prof_dir, ROOT) if os.path.isabs(prof_dir) else prof_dir.rstrip("/")
    sub = os.path.join(prof_dir, "clock")
    agent = _agent(sub)
    nxcc = int(agent["Num_Xcc"])
    durs = {}
    for r in _csv_rows(_find(sub, "kernel_trace.csv")):
        if "fa::" in r["Kernel_Name"]:
            durs.setdefault(_kname(r["Kernel_Name"]), []).append(
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    res = {"workload": WORKLOAD_TAG, "source_files": KERNEL_SOURCES,
           "source_sha256": kernel_source_hash(), "command": CLOCK_CMD.replace("{prof}", rel),
           "num_xcc": nxcc, "max_engine_clock_mhz": float(agent["Max_Engine_Clk_Fcompute"]),
           "note": "mhz = mean GRBM_GUI_ACTIVE per dispatch / num_xcc / mean dispatch duration "
                   "(same run); the published dense bf16 peak is quoted at 2400 MHz",
           "kernels": {}}
    for (k, c), (v, n) in _pmc_means(_find(sub, "counter_collection.csv")).items():
        if "fa::" in k and c == "GRBM_GUI_ACTIVE":
            name = _kname(k)
            d = sum(durs[name]) / len(durs[name])
            res["kernels"][name] = {"grbm_gui_active": v, "dispatches": n,
                                    "duration_us": d / 1e3, "mhz": round(v / nxcc / d * 1e3, 1)}
    path = os.path.join(out_dir, os.path.basename(CLOCK_SUMMARY))
    with open(path, "w") as fh:
        json.dump(res, fh, indent=1)
        fh.write("\n")
    return path


def summarize_accumulate(prof_dir, out_dir):
    """profiles/hbm_traffic_accumulate_mode_<workload>.md: the HBM-bound
    steps of the accumulate-mode backward (preprocess, dq_convert) and its
    key-tile kernel: durations from a kernel trace (PROF_DIR/acc_trace), HBM
    bytes from FETCH_SIZE / WRITE_SIZE runs (PROF_DIR/acc_FETCH_SIZE,
    acc_WRITE_SIZE) scaled by the plain-copy runs (copy_FETCH_SIZE,
    copy_WRITE_SIZE), and the algorithmic (compulsory) bytes."""
    rel = os.path.relpath(prof_dir, ROOT) if os.path.isabs(prof_dir) else prof_dir.rstrip("/")

    def cmd(c):
        return c.replace("{prof}", rel)
    bench_line = None
    with open(os.path.join(prof_dir, "acc_trace.log")) as fh:
        for line in fh:
            if line.startswith("{") and '"metric"' in line:
                bench_line = json.loads(line)
    cfg = bench_line["config"]
    rows, H, D = cfg["batch"] * cfg["seqlen_q"], cfg["heads"], cfg["head_dim"]
    dpad = next(d for d in (64, 96, 128, 192, 256) if d >= D)
    algo = {"preprocess": rows * H * (2 * D * 2 + 4 + 8) + rows * H * 4 * dpad,
            "dq_convert": rows * H * (4 * dpad + 2 * D)}
    trace = _csv_rows(_find(os.path.join(prof_dir, "acc_trace"), "kernel_trace.csv"))
    durs = {}
    for r in trace:
        if "fa::" in r["Kernel_Name"]:
            durs.setdefault(_kname(r["Kernel_Name"]), []).append(
                (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    copy_bytes = float(1 << 30)
    meas = {}
    for c in ("FETCH_SIZE", "WRITE_SIZE"):
        cm = _pmc_means(_find(os.path.join(prof_dir, "copy_" + c), "counter_collection.csv"))
        ckib, _ = next(v for (k, cn), v in cm.items() if "copyBuffer" in k and cn == c)
        factor = copy_bytes / (ckib * 1024.0)
        for (k, cn), (kib, n) in _pmc_means(
                _find(os.path.join(prof_dir, "acc_" + c), "counter_collection.csv")).items():
            if "fa::" in k and cn == c:
                meas.setdefault(_kname(k), {})[c] = (kib * 1024.0 * factor, factor)
    lines = ["# HBM traffic, accumulate mode: %s" % cfg["workload"], "",
             "dQ by fp32 partial adds in the key-tile kernel (`--dq-accumulate`, unordered "
             "atomics): preprocess, key-tile kernel, dq_convert.", "",
             "Commands (repo root, MI355X):", "",
             "    " + cmd(ACC_TRACE_CMD) + " > %s/acc_trace.log" % rel,
             "    rocprofv3 --pmc FETCH_SIZE -f csv -d %s/acc_FETCH_SIZE -o c3 -- %s" % (rel, ACC_RUN),
             "    rocprofv3 --pmc WRITE_SIZE -f csv -d %s/acc_WRITE_SIZE -o c3 -- %s" % (rel, ACC_RUN),
             "    rocprofv3 --pmc FETCH_SIZE -f csv -d %s/copy_FETCH_SIZE -o copy -- "
             "python bench.py --copy-calibration" % rel,
             "    rocprofv3 --pmc WRITE_SIZE -f csv -d %s/copy_WRITE_SIZE -o copy -- "
             "python bench.py --copy-calibration" % rel, "",
             "Counter bytes are FETCH_SIZE and WRITE_SIZE per dispatch scaled by what the same "
             "counters read for a 1 GiB device copy (factors %.3f and %.3f)." % (
                 next(iter(meas.values()))["FETCH_SIZE"][1],
                 next(iter(meas.values()))["WRITE_SIZE"][1]), "",
             "| kernel | mean duration (us) | algorithmic bytes | algorithmic GB/s | "
             "counter bytes read + written | counter GB/s |", "|---|---|---|---|---|---|"]
    for name in sorted(meas):
        d = sum(durs[name]) / len(durs[name])
        step = next((s for s in ("preprocess", "convert") if s in name), None)
        a = algo["dq_convert" if step == "convert" else "preprocess"] if step else None
        rd, wr = meas[name]["FETCH_SIZE"][0], meas[name]["WRITE_SIZE"][0]
        lines.append("| %s | %.1f | %s | %s | %.4g + %.4g | %.0f |" % (
            name, d, "%.4g" % a if a else "-", "%.0f" % (a / d / 1e3) if a else "-",
            rd, wr, (rd + wr) / d / 1e3))
    lines += ["", "Algorithmic bytes: preprocess reads O and dO (2 x 2 x D B per row and "
              "head), writes lse2 and rowdot (8 B) and clears the fp32 accumulator (4 x D_pad "
              "B); dq_convert reads the accumulator (4 x D_pad B) and writes dQ (2 x D B).  "
              "The key-tile kernel is MFMA-bound; its row shows the fp32 partial adds.", "",
              "The same run's bench line: %.4f ms per step, %.1f TFLOP/s, per-kernel HIP-event "
              "times (ms): `%s`, GB/s: `%s`." % (bench_line["ms_per_step"], bench_line["value"],
                                                json.dumps(bench_line["kernel_ms"]),
                                                json.dumps(bench_line.get("hbm_kernels_GBs")))]
    path = os.path.join(out_dir, "hbm_traffic_accumulate_mode_%s.md" % cfg["workload"])
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def mfma_ceiling(fa, torch, iters=4000, reps=3):
    """TFLOP/s of the library's MFMA probe (fa_probe_mfma_rate) in both
    operand modes, one workgroup of four waves per CU; best of `reps`."""
    lib = fa.load_library()
    blocks = torch.cuda.get_device_properties(0).multi_processor_count
    out = torch.zeros(blocks * 256, dtype=torch.float32, device="cuda:0")
    stream = torch.cuda.current_stream()
    res = {}
    for mode, name in ((0, "operands_in_registers"), (1, "a_operand_from_lds")):
        assert lib.fa_probe_mfma_rate(mode, blocks, 50, 1, out.data_ptr(), stream.cuda_stream) == 0
        best = None
        for r in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert lib.fa_probe_mfma_rate(mode, blocks, iters, 2 + r, out.data_ptr(),
                                          stream.cuda_stream) == 0
            e1.record(stream)
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            best = ms if best is None else min(best, ms)
        flops = blocks * 4.0 * 16 * iters * 32768
        tf = flops / (best * 1e-3) / 1e12
        res[name] = {"tflops": round(tf, 1), "frac_of_published_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                     "ns_per_mfma_per_wave": round(best * 1e6 / (16 * iters), 2)}
    return {"mfma_ceiling": res, "blocks": blocks, "waves_per_simd": 1,
            "instruction": "v_mfma_f32_32x32x16_bf16", "operands": "random bf16 bits",
            "published_peak_tflops": PEAK_BF16_TFLOPS}


def summarize_ceiling(prof_dir, out_dir):
    """profiles/mfma_ceiling_random_operands.md from
        python bench.py --mfma-ceiling > PROF_DIR/ceiling.log
        rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE GRBM_COUNT -f csv
            -d PROF_DIR/ceiling_clock -o probe -- python bench.py --mfma-ceiling"""
    rel = os.path.relpath(prof_dir, ROOT) if os.path.isabs(prof_dir) else prof_dir.rstrip("/")
    line = None
    with open(os.path.join(prof_dir, "ceiling.log")) as fh:
        for ln in fh:
            if ln.startswith("{") and "mfma_ceiling" in ln:
                line = json.loads(ln)
    sub = os.path.join(prof_dir, "ceiling_clock")
    nxcc = int(_agent(sub)["Num_Xcc"])
    trace = _csv_rows(_find(sub, "kernel_trace.csv"))
    cnt = _csv_rows(_find(sub, "counter_collection.csv"))
    durs = {}
    for r in trace:
        if "probe_kernel" in r["Kernel_Name"]:
            durs.setdefault(r["Kernel_Name"], []).append(
                int(r["End_Timestamp"]) - int(r["Start_Timestamp"]))
    gui = {}
    for r in cnt:
        if "probe_kernel" in r["Kernel_Name"] and r["Counter_Name"] == "GRBM_GUI_ACTIVE":
            gui.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    lines = ["# MFMA rate with random operands (v_mfma_f32_32x32x16_bf16, one wave per SIMD "
             "on every CU)", "",
             "Commands (repo root, MI355X):", "",
             "    python bench.py --mfma-ceiling > %s/ceiling.log" % rel,
             "    rocprofv3 --kernel-trace --pmc GRBM_GUI_ACTIVE GRBM_COUNT -f csv -d "
             "%s/ceiling_clock -o probe -- python bench.py --mfma-ceiling" % rel, "",
             "| operand supply | TFLOP/s | fraction of the published 2.5 PFLOP/s | ns per MFMA "
             "per wave |", "|---|---|---|---|"]
    for name, d in line["mfma_ceiling"].items():
        lines.append("| %s | %.1f | %.3f | %.2f |" % (name.replace("_", " "), d["tflops"],
                                                        d["frac_of_published_peak"],
                                                        d["ns_per_mfma_per_wave"]))
    lines += ["", "Clock during the probe (GRBM busy cycles / %d XCDs / dispatch duration, "
              "the profiled run; the long dispatches of each mode):" % nxcc, ""]
    for k in sorted(gui):
        ds = durs.get(k, [])
        pairs = sorted(zip(ds, gui[k]))[-3:]   # the long (timed) dispatches
        mhz = sum(g / nxcc / d * 1e3 for d, g in pairs) / len(pairs)
        lines.append("- `%s`: %.0f MHz over %d dispatches of %.1f ms" % (
            _kname(k).replace("(anonymous namespace)::", ""), mhz, len(pairs),
            sum(d for d, _ in pairs) / len(pairs) / 1e6))
    lines += ["", "The published peak assumes 2400 MHz; a 32x32x16 product takes 32 cycles "
              "per SIMD, so the rate at clock f is 2.5 PFLOP/s x f / 2400 MHz.  The probe's "
              "products have no other work between them: this is the rate the tile kernels' "
              "products can approach on data of this kind."]
    path = os.path.join(out_dir, "mfma_ceiling_random_operands.md")
    with open(path, "w") as fh:
        fh.write("\n".join(lines) + "\n")
    return path


def visible_pairs(Sq, Sk, causal, window=None):
    """(query, key) pairs of one (batch, head) that the products cover: the
    usual convention Sq*Sk, halved for causal, without a local window; the
    exact count of visible pairs with one (row i sees keys i + Sk - Sq - left
    .. i + Sk - Sq + right, clipped to the sequence)."""
    if window is None:
        return 0.5 * Sq * Sk if causal else float(Sq * Sk)
    import numpy as np
    left, right = window
    right = 0 if causal else right
    i = np.arange(Sq, dtype=np.int64) + (Sk - Sq)
    lo = np.maximum(0, i - left) if left >= 0 else np.zeros_like(i)
    hi = np.minimum(Sk - 1, i + right) if right >= 0 else np.full_like(i, Sk - 1)
    return float(np.maximum(0, hi - lo + 1).sum())


def conv_flops(B, H, Sq, Sk, D, causal, window=None):
    """Five products of 2*D FLOPs per visible (query, key) pair each."""
    return 2.5 * 4.0 * B * H * D * visible_pairs(Sq, Sk, causal, window)


def exact_pairs(Sq, Sk, causal, window=None):
    """The (query, key) pairs of one (sequence, head) that are visible: with
    the bottom-right causal rule (row i sees keys <= i + Sk - Sq) and any
    local window, counted exactly."""
    if not causal and window is None:
        return float(Sq * Sk)
    return visible_pairs(Sq, Sk, causal, window if window is not None else (-1, -1))


def workload_flops(wl, lens_q, lens_k):
    """(conventional FLOPs, exact visible-pair FLOPs) of one backward: five
    products of 2*D FLOPs per pair.  Packed batches sum over the sequences
    (the convention's B*Sq*Sk becomes the sum of Lq*Lk)."""
    H, D = wl.heads, wl.head_dim
    if wl.varlen:
        conv = sum(conv_flops(1, H, lq, lk, D, wl.causal, wl.window) for lq, lk in zip(lens_q, lens_k))
    else:
        conv = conv_flops(wl.batch, H, wl.seqlen_q, wl.seqlen_k, D, wl.causal, wl.window)
    exact = sum(2.5 * 4.0 * H * D * exact_pairs(lq, lk, wl.causal, wl.window)
                for lq, lk in zip(lens_q, lens_k))
    return conv, exact


def dq_add_bytes(wl, lens_q, lens_k):
    """Bytes of fp32 dQ partial adds of one accumulate-mode backward (method
    overhead): each 128-key tile adds its partial over the valid rows of
    every 64-row query tile it visits, head_dim columns of 4 bytes (the
    key-tile kernel's block bounds, causal bottom-right and window)."""
    left, right = wl.window if wl.window is not None else (-1, -1)
    if wl.causal:
        right = 0 if right < 0 else min(right, 0)
    total = 0
    for lq, lk in zip(lens_q, lens_k):
        off = lk - lq
        for n0 in range(0, lk, 128):
            first = max(0, n0 - off - right) if right >= 0 else 0
            last = min(lq - 1, min(lk - 1, n0 + 127) - off + left) if left >= 0 else lq - 1
            if first > last:
                continue
            m0, m1 = first // 64, last // 64 + 1
            total += sum(min(64, lq - 64 * m) for m in range(m0, m1))
    return total * wl.heads * wl.head_dim * 4


def forward_inputs_torch(q, k, v, scale, causal, window=None, softcap=0.0):
    """O (bf16) and natural-log LSE (fp32, (B,H,Sq)) by a plain fp32 torch
    forward, one (batch, head) at a time.  Dense bshd inputs on the GPU."""
    import torch
    B, Sq, H, D = q.shape
    Sk, Hk = k.shape[1], k.shape[2]
    G = H // Hk
    out = torch.empty_like(q)
    lse = torch.empty(B, H, Sq, dtype=torch.float32, device=q.device)
    masked = None
    if causal or window is not None:
        i = torch.arange(Sq, device=q.device)[:, None] + (Sk - Sq)
        j = torch.arange(Sk, device=q.device)[None, :]
        left, right = window if window is not None else (-1, -1)
        right = 0 if causal else right
        masked = torch.zeros(Sq, Sk, dtype=torch.bool, device=q.device)
        if right >= 0:
            masked |= j > i + right
        if left >= 0:
            masked |= j < i - left
    for b in range(B):
        for h in range(H):
            qh = q[b, :, h, :].float().contiguous()
            kt = k[b, :, h // G, :].float().t().contiguous()
            vh = v[b, :, h // G, :].float().contiguous()
            s = torch.matmul(qh, kt) * scale
            if softcap > 0:
                s = softcap * torch.tanh(s / softcap)
            if masked is not None:
                s.masked_fill_(masked, float("-inf"))
            l = torch.logsumexp(s, dim=-1)
            p = torch.exp(s - l[:, None])
            p = torch.nan_to_num(p, nan=0.0)
            out[b, :, h, :] = torch.matmul(p, vh).to(torch.bfloat16)
            lse[b, h] = l
    return out, lse


def forward_inputs_packed(q, k, v, lens_q, lens_k, scale, causal, window=None, softcap=0.0):
    """O and LSE of a packed batch ((total, H, D) tensors) by the same plain
    fp32 forward, one sequence at a time; LSE is (nseq, H, max_len_q), rows
    past a sequence's length -inf."""
    import torch
    nseq, H = len(lens_q), q.shape[1]
    out = torch.zeros_like(q)
    lse = torch.full((nseq, H, max(lens_q)), float("-inf"), dtype=torch.float32, device=q.device)
    oq = ok = 0
    for s_, (lq, lk) in enumerate(zip(lens_q, lens_k)):
        if lq and lk:
            o1, l1 = forward_inputs_torch(q[oq:oq + lq][None], k[ok:ok + lk][None],
                                          v[ok:ok + lk][None], scale, causal, window, softcap)
            out[oq:oq + lq] = o1[0]
            lse[s_, :, :lq] = l1[0]
        oq += lq
        ok += lk
    return out, lse


def cpu_model():
    """The host CPU's model name (from /proc/cpuinfo), or None."""
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(wl, units, inp=None):
    """fp64 oracle backward on a bounded sample: `units` (sequence, KV-head
    group) pairs of the workload, each its own exact sub-problem."""
    import numpy as np
    import workloads as W
    from oracle import oracle as O
    inp = inp if inp is not None else W.make_inputs(wl)
    G = wl.heads // wl.heads_k
    cu_q, cu_k = inp.cu_q.tolist(), inp.cu_k.tolist()
    t_total = 0.0
    flops = 0.0
    for (b, g) in units:
        hs = list(range(g * G, (g + 1) * G))

        def f64(t):
            return t.float().numpy().astype(np.float64)
        rq = slice(cu_q[b], cu_q[b + 1])
        rk = slice(cu_k[b], cu_k[b + 1])
        lq, lk = rq.stop - rq.start, rk.stop - rk.start
        q = f64(inp.packed(inp.q)[rq][:, hs])
        k = f64(inp.packed(inp.k)[rk][:, [g]])
        v = f64(inp.packed(inp.v)[rk][:, [g]])
        do = f64(inp.packed(inp.dout)[rq][:, hs])
        t0 = time.perf_counter()
        O.backward(q, k, v, do, [0, lq], [0, lk], wl.scale, wl.causal,
                   window=wl.window_sizes, softcap=wl.softcap, dropout=wl.dropout_f32,
                   drop_base=(b, g * G, wl.heads) if wl.dropout else None)
        t_total += time.perf_counter() - t0
        flops += conv_flops(1, G, lq, lk, wl.head_dim, wl.causal, wl.window)
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": O.num_threads(),
            "cpu_model": cpu_model(), "seconds": round(t_total, 2), "kind": "oracle",
            "sample": "%d of %d (%s, KV-head group) units of the workload, fp64 "
                      "contracted-Jacobian backward incl. its forward recompute, %.1f s"
                      % (len(units), (len(cu_q) - 1) * wl.heads_k,
                         "sequence" if wl.varlen else "batch", t_total)}


def workload_label(wl):
    """Shape words of a workload in the style of the headline metric
    ("S=4096 D=128 causal GQA")."""
    if wl.varlen:
        shape = "%d seqs L=%d..%d" % (wl.batch, wl.len_lo, wl.len_hi)
    elif wl.seqlen_q == wl.seqlen_k:
        shape = "S=%d" % wl.seqlen_q
    else:
        shape = "Sq=%d Sk=%d" % (wl.seqlen_q, wl.seqlen_k)
    heads = "MHA" if wl.heads == wl.heads_k else ("MQA" if wl.heads_k == 1 else "GQA")
    return "%s D=%d %s %s" % (shape, wl.head_dim, "causal" if wl.causal else "non-causal", heads)


def metric_name(base, wl):
    """The metric label with the workload's shape and extra features (the
    headline workload gives the base label unchanged)."""
    name = base.replace("S=4096 D=128 causal GQA", workload_label(wl))
    return name + window_suffix(wl)


def window_suffix(wl):
    suffix = "" if wl.window is None else ", local window (%d, %d)" % tuple(wl.window)
    suffix += ", softcap %g" % wl.softcap if wl.softcap > 0 else ""
    return suffix + (", dropout %g" % wl.dropout[0] if wl.dropout else "")


def main_kernel_name(fused, wl):
    local = wl.window is not None and wl.window[0] >= 0
    dpad = next(d for d in (64, 96, 128, 192, 256) if d >= wl.head_dim)
    # dropout mode: 2 when the keep words of the dQ pass are read (separate
    # dQ), 1 when drawn in the kernel (fused dQ)
    drop = 0 if wl.dropout is None else (1 if fused else 2)
    return "fa_bwd_main_kernel<%d, %s, false, %s, %s, %d>" % (
        dpad, str(bool(fused)).lower(), str(local).lower(), str(wl.softcap > 0).lower(), drop)


def fwd_kernel_name(wl):
    local = wl.window is not None and wl.window[0] >= 0
    dpad = next(d for d in (64, 96, 128, 192, 256) if d >= wl.head_dim)
    return "fa_fwd_kernel<%d, false, %s, %s, %s>" % (dpad, str(local).lower(),
                                                  str(wl.softcap > 0).lower(),
                                                  str(wl.dropout is not None).lower())


FWD_METRIC = "fwd TFLOP/s (O, LSE) bf16 and % of MFMA peak, S=4096 D=128 causal GQA"
FWD_KERNEL = "fa_fwd_kernel<128, false, false, false, false>"


def fwd_flops(B, H, Sq, Sk, D, causal, window=None):
    """The forward's two products (S = Q K^T, O = P V): 2*D FLOPs each per
    visible (query, key) pair (Sq*Sk pairs, halved for causal)."""
    return 4.0 * B * H * D * visible_pairs(Sq, Sk, causal, window)


def cpu_baseline_fwd(wl, units):
    """fp64 oracle forward on a bounded sample of (batch, head) units."""
    import numpy as np
    import workloads as W
    from oracle import oracle as O
    inp = W.make_inputs(wl)
    G = wl.heads // wl.heads_k
    t_total, flops = 0.0, 0.0
    cu_q = [0] + list(np.cumsum(inp.lens_q))
    cu_k = [0] + list(np.cumsum(inp.lens_k))
    for (b, h) in units:
        def f64(t):
            return t.float().numpy().astype(np.float64)
        if wl.varlen:   # sequence b of the packed batch
            q = f64(inp.q[cu_q[b]:cu_q[b + 1], [h]])
            k = f64(inp.k[cu_k[b]:cu_k[b + 1], [h // G]])
            v = f64(inp.v[cu_k[b]:cu_k[b + 1], [h // G]])
        else:
            q = f64(inp.q[b][:, [h]])
            k = f64(inp.k[b][:, [h // G]])
            v = f64(inp.v[b][:, [h // G]])
        lq, lk = q.shape[0], k.shape[0]
        t0 = time.perf_counter()
        O.forward(q, k, v, [0, lq], [0, lk], wl.scale, wl.causal,
                  window=wl.window_sizes, softcap=wl.softcap, dropout=wl.dropout_f32)
        t_total += time.perf_counter() - t0
        flops += fwd_flops(1, 1, lq, lk, wl.head_dim, wl.causal, wl.window)
    return {"value": flops / t_total / 1e12, "unit": "TFLOP/s", "cores": O.num_threads(),
            "kind": "oracle",
            "sample": "%d of %d (%s, head) units of the workload, fp64 forward, %.1f s"
                      % (len(units), len(inp.lens_q) * wl.heads,
                         "sequence" if wl.varlen else "batch", t_total)}


def bench_forward(args, wl, dev):
    import torch
    import workloads as W
    import attention_backward_fa2_amd as fa
    inp = W.make_inputs(wl)
    q, k, v = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v))
    out = torch.empty_like(q)
    kw = {}
    if wl.varlen:
        kw = dict(cu_seqlens_q=inp.cu_q.to(dev), cu_seqlens_k=inp.cu_k.to(dev),
                  max_seqlen_q=max(inp.lens_q), max_seqlen_k=max(inp.lens_k))
    lse = torch.empty(len(inp.lens_q), wl.heads, max(inp.lens_q), dtype=torch.float32,
                      device=dev)
    a = fa.make_fwd_args(q, k, v, out, lse, wl.scale, wl.causal, window=wl.window,
                         softcap=wl.softcap, dropout=wl.dropout, **kw)
    words = None
    if args.keep_words and wl.dropout:
        words = torch.empty(fa.keep_bytes(a) // 4, dtype=torch.int32, device=dev)
        a.dropout_keep_out = words.data_ptr()
        a.dropout_keep_out_bytes = words.numel() * 4
    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        fa.run_fwd(a, stream)
    torch.cuda.synchronize()
    K = args.steps
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for s in range(K):
        fa.run_fwd(a, stream)
        evs[s + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = evs[0].elapsed_time(evs[-1]) / K
    B, H, Hk, Sq, Sk, D = wl.batch, wl.heads, wl.heads_k, wl.seqlen_q, wl.seqlen_k, wl.head_dim
    # packed batches: exactly over the visible pairs of each sequence
    flops = sum(fwd_flops(1, H, lq, lk, D, wl.causal, wl.window)
                for lq, lk in zip(inp.lens_q, inp.lens_k))
    tf = flops / (ms * 1e-3) / 1e12
    rec = {
        "metric": metric_name(FWD_METRIC, wl), "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": K, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "heads": H, "heads_k": Hk,
                   "seqlen_q": Sq, "seqlen_k": Sk, "head_dim": D, "causal": wl.causal,
                   "window": list(wl.window) if wl.window else None,
                   "softcap": wl.softcap or None,
                   "dropout": wl.dropout[0] if wl.dropout else None, "pass": "forward",
                   "keep_words_out": words is not None},
        "pct_of_peak": round(100.0 * tf / PEAK_BF16_TFLOPS, 2),
        "flops_per_step": flops,
        "kernel_ms": {"fwd": round(ms, 4)},
        "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                     "traffic": None,
                     "kernel": fwd_kernel_name(wl),
                     "algorithmic_flops_per_launch": flops},
        "wall_s": round(wall, 3),
    }
    if not args.no_cpu_baseline:
        units = [(b, h) for b in range(len(inp.lens_q)) for h in range(H)]
        n = min(args.cpu_units, len(units))
        rec["cpu_baseline"] = cpu_baseline_fwd(wl, [units[(i * len(units)) // n]
                                                    for i in range(n)])
    print(json.dumps(rec), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--config", type=int, default=3, help="workload id (workloads.py)")
    ap.add_argument("--dq-accumulate", action="store_true",
                    help="form dQ by fp32 partial adds in the key-tile pass (+ convert) "
                         "instead of the separate query-tile pass")
    ap.add_argument("--deterministic", action="store_true",
                    help="with --dq-accumulate: ordered (bit-reproducible) partial adds")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--forward", action="store_true",
                    help="time the forward kernel (O, LSE) instead of the backward")
    ap.add_argument("--cpu-units", type=int, default=16)
    ap.add_argument("--window", type=int, nargs=2, metavar=("LEFT", "RIGHT"),
                    help="local window (negative = unbounded): times the workload with it")
    ap.add_argument("--softcap", type=float, default=0.0,
                    help="soft cap c > 0 of the scaled scores: times the workload with it")
    ap.add_argument("--head-dim", type=int, default=0,
                    help="head dim other than the workload's (up to 256): times the workload with it")
    ap.add_argument("--dropout", type=float, default=0.0,
                    help="dropout probability p > 0: times the workload with it (fixed seed)")
    ap.add_argument("--keep-words", action="store_true",
                    help="with --dropout: the forward writes the keep words and the backward "
                         "reads them instead of drawing the bits (with --forward: times the "
                         "forward writing them)")
    ap.add_argument("--summarize-profile", metavar="PROF_DIR",
                    help="write the profiles/ summaries from rocprofv3 outputs in PROF_DIR "
                         "(trace/, FETCH_SIZE/, WRITE_SIZE/, copy_FETCH_SIZE/, copy_WRITE_SIZE/)")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_ARGS"),
                    help="write profiles/kernel_trace_<workload>.md from a rocprofv3 kernel "
                         "trace of 'python bench.py BENCH_ARGS' in TRACE_DIR (log: TRACE_DIR.log)")
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="only time the library's MFMA rate probe (32x32x16 bf16 products on "
                         "random operands, one wave per SIMD on every CU): the rate the tile "
                         "kernels' products can approach at the clock the chip then runs")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of 1 GiB (4 times), the reference "
                         "kernel for scaling FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args()

    if args.summarize_profile:
        summarize_profile(args.summarize_profile, os.path.join(ROOT, "profiles"))
        if os.path.isdir(os.path.join(args.summarize_profile, "clock")):
            print(summarize_clock(args.summarize_profile, os.path.join(ROOT, "profiles")))
        if os.path.isdir(os.path.join(args.summarize_profile, "acc_trace")):
            print(summarize_accumulate(args.summarize_profile, os.path.join(ROOT, "profiles")))
        if os.path.isdir(os.path.join(args.summarize_profile, "ceiling_clock")):
            print(summarize_ceiling(args.summarize_profile, os.path.join(ROOT, "profiles")))
        return
    if args.summarize_trace:
        print(summarize_variant_trace(args.summarize_trace[0], args.summarize_trace[1],
                                      os.path.join(ROOT, "profiles")))
        return
    if args.gpus != 1:
        print("bench.py: the library runs on one GPU; --gpus %d is not supported "
              "(the backward splits into independent (batch, KV-head) units that need "
              "no communication; N GPUs would each run 1/N of them)" % args.gpus, file=sys.stderr)
        sys.exit(2)

    import torch
    import workloads as W
    import attention_backward_fa2_amd as fa

    if args.copy_calibration:
        n = 1 << 30
        src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        for _ in range(4):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_per_dispatch": {"read": n, "write": n},
                          "dispatches": 4}), flush=True)
        return

    if args.mfma_ceiling:
        print(json.dumps(mfma_ceiling(fa, torch)), flush=True)
        return
    fa.load_library()
    wl = W.WORKLOADS[args.config]
    if args.head_dim:
        import dataclasses
        wl = dataclasses.replace(wl, name=wl.name.replace("_d%d" % wl.head_dim, "_d%d" % args.head_dim),
                                 head_dim=int(args.head_dim))
    if args.window is not None:
        import dataclasses
        wl = dataclasses.replace(wl, name="%s_window%d_%d" % (wl.name, *args.window),
                                 window=tuple(args.window))
    if args.softcap > 0:
        import dataclasses
        wl = dataclasses.replace(wl, name="%s_softcap%g" % (wl.name, args.softcap),
                                 softcap=float(args.softcap))
    if args.dropout > 0:
        import dataclasses
        wl = dataclasses.replace(wl, name="%s_dropout%g%s" % (wl.name, args.dropout,
                                                              "_keepwords" if args.keep_words else ""),
                                 dropout=(float(args.dropout), 0x243F6A8885A308D3, 0))
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.forward:
        bench_forward(args, wl, dev)
        return
    inp = W.make_inputs(wl)
    q, k, v, do = (t.to(dev).contiguous() for t in (inp.q, inp.k, inp.v, inp.dout))
    kw = {}
    if wl.varlen:
        kw = dict(cu_seqlens_q=inp.cu_q.to(dev), cu_seqlens_k=inp.cu_k.to(dev),
                  max_seqlen_q=max(inp.lens_q), max_seqlen_k=max(inp.lens_k))
    keep_words = None
    if wl.dropout:
        # the backward needs the dropout forward's O: this library's forward
        o = torch.empty_like(q)
        lse = torch.empty(len(inp.lens_q), wl.heads, max(inp.lens_q), dtype=torch.float32,
                          device=dev)
        keep_words = fa.fa_fwd(q, k, v, o, lse, wl.scale, wl.causal, window=wl.window,
                               softcap=wl.softcap, dropout=wl.dropout, keep=args.keep_words,
                               **kw)
    elif wl.varlen:
        o, lse = forward_inputs_packed(q, k, v, inp.lens_q, inp.lens_k, wl.scale, wl.causal,
                                       wl.window, wl.softcap)
    else:
        o, lse = forward_inputs_torch(q, k, v, wl.scale, wl.causal, wl.window, wl.softcap)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    a = fa.make_args(do, q, k, v, o, lse, dq, dk, dv, wl.scale, wl.causal,
                     deterministic=args.deterministic, dq_accumulate=args.dq_accumulate,
                     window=wl.window, softcap=wl.softcap, dropout=wl.dropout,
                     dropout_keep=keep_words, **kw)
    # the steps of one backward, in the order fa_bwd enqueues them
    seq = ["preprocess", "main", "dq_convert"] if args.dq_accumulate else ["dq", "main"]
    ws = fa.alloc_workspace(a, dev)
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()

    def step(evs=None):
        if evs is None:
            fa.run(a, "all", stream)
            return
        evs[0].record(stream)
        for i, name in enumerate(seq):
            fa.run(a, name, stream)
            evs[i + 1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    K = args.steps
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(seq) + 1)] for _ in range(K)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(K):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    gpu_ms = evs[0][0].elapsed_time(evs[-1][-1])
    kms = {name: sum(e[i].elapsed_time(e[i + 1]) for e in evs) / K for i, name in enumerate(seq)}
    per_step = sorted(e[0].elapsed_time(e[-1]) for e in evs)
    main_ms = kms["main"]
    ms_per_step = gpu_ms / K

    B, H, Hk, Sq, Sk, D = wl.batch, wl.heads, wl.heads_k, wl.seqlen_q, wl.seqlen_k, wl.head_dim
    flops, exact = workload_flops(wl, inp.lens_q, inp.lens_k)
    value = flops / (ms_per_step * 1e-3) / 1e12
    # Algorithmic work per launch.  MFMA-bound kernels: the key-tile pass
    # does 4 of the 5 products (S, dP, dV, dK; + dQ in accumulate mode), the
    # separate dQ pass 3 (S, dP, dQ); FLOPs counted over the causal half like
    # the headline convention.  HBM-bound kernels: compulsory bytes (the
    # preprocess reads O and dO, writes lse2 / rowdot and clears the fp32
    # accumulator; dq_convert reads the accumulator and writes dQ).
    rows = sum(inp.lens_q)
    dpad = next(d for d in (64, 96, 128, 192, 256) if d >= D)
    gemm = flops / 5.0                   # one of the five products
    main_flops = 5 * gemm if args.dq_accumulate else 4 * gemm
    dq_flops = 0.0 if args.dq_accumulate else 3 * gemm
    pre_bytes = rows * H * (2 * D * 2 + 4 + 8) + rows * H * 4 * dpad   # accumulate mode
    conv_bytes = rows * H * (4 * dpad + 2 * D)
    main_tflops = main_flops / (main_ms * 1e-3) / 1e12
    add_bytes = dq_add_bytes(wl, inp.lens_q, inp.lens_k) if args.dq_accumulate else 0
    clock = committed_clock()
    off_flags = fa.workspace_layout(a).off_flags
    flags = ws[off_flags:off_flags + 16].cpu().view(torch.int32)

    rec = {
        "metric": metric_name(METRIC, wl),
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": wl.name, "batch": B, "heads": H, "heads_k": Hk,
                   "seqlen_q": Sq, "seqlen_k": Sk, "head_dim": D, "causal": wl.causal,
                   "window": list(wl.window) if wl.window else None,
                   "softcap": wl.softcap or None,
                   "dropout": wl.dropout[0] if wl.dropout else None,
                   "dq_mode": ("ordered" if args.deterministic else "atomic")
                   if args.dq_accumulate else "separate",
                   "keep_words": ("forward" if keep_words is not None else "drawn")
                   if wl.dropout else None},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "flops_per_step": flops,
        "ms_per_step_median": round(per_step[K // 2], 4),
        "ms_per_step_min": round(per_step[0], 4),
        "visible_flops_per_step": exact,
        "visible_tflops": round(exact / (ms_per_step * 1e-3) / 1e12, 2),
        # one exp2 per visible score (the method's count; this design's
        # separate dQ pass evaluates each a second time)
        "exp2_per_step": exact / (10.0 * D),
        "exp2_G_per_s": round(exact / (10.0 * D) / (ms_per_step * 1e-3) / 1e9, 1),
        "kernel_ms": {name: round(t, 4) for name, t in kms.items()},
        "kernel_tflops": {"main": round(main_tflops, 1)} if args.dq_accumulate else
        {"main": round(main_tflops, 1), "dq": round(dq_flops / (kms["dq"] * 1e-3) / 1e12, 1)},
        # HBM GB/s per kernel: the memory-bound kernels of the accumulate
        # mode over their compulsory bytes; in the default mode the two tile
        # kernels over the counter-measured bytes of the committed profile
        # (headline only), which shows how far below the HBM rate they run
        "hbm_kernels_GBs": {"preprocess": round(pre_bytes / (kms["preprocess"] * 1e-3) / 1e9, 1),
                            "dq_convert": round(conv_bytes / (kms["dq_convert"] * 1e-3) / 1e9, 1)}
        if args.dq_accumulate else tile_kernel_GBs(kms, headline_path(args, wl)),
        # accumulate mode: the fp32 dQ partial adds of the key-tile kernel
        # (method overhead beyond the compulsory bytes), and their rate over
        # that kernel's time
        "dq_partial_add": {"bytes": add_bytes,
                           "GBs_over_main": round(add_bytes / (main_ms * 1e-3) / 1e9, 1)}
        if args.dq_accumulate else None,
        "roofline": {"bound": "mfma", "achieved": round(main_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(main_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": committed_traffic() if headline_path(args, wl) else None,
                     "kernel": main_kernel_name(args.dq_accumulate, wl),
                     "algorithmic_flops_per_launch": main_flops},
        "wall_s": round(wall, 3),
        "ordered_wait_gave_up": bool(int(flags[0]) != 0),
    }
    if clock and headline_path(args, wl):
        # the dense bf16 peak scaled to the clock the kernel ran at (GRBM
        # cycle counters of the committed profile)
        pk = PEAK_BF16_TFLOPS * clock["mhz"] / PEAK_CLOCK_MHZ
        rec["roofline"]["clock_mhz"] = clock["mhz"]
        rec["roofline"]["peak_at_clock"] = round(pk, 1)
        rec["roofline"]["frac_at_clock"] = round(main_tflops / pk, 4)
    if not args.no_cpu_baseline:
        all_units = [(b, g) for b in range(len(inp.lens_q)) for g in range(Hk)]
        pick = [all_units[(i * len(all_units)) // args.cpu_units]
                for i in range(min(args.cpu_units, len(all_units)))]
        rec["cpu_baseline"] = cpu_baseline(wl, pick, inp)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
