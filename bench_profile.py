"""rocprofv3 runs behind the benchmark's roofline figures, and their summaries.

Runs bench.py (M = 8 round only, no CPU leg, plus one plain 1 GiB device copy)
three times under rocprofv3 -- a kernel trace with statistics, then a
FETCH_SIZE pass and a WRITE_SIZE pass, each in a run of its own -- and writes
short text summaries to profiles/:

  decode_round_m8_kernel_trace.md   per-kernel durations, per-shape decode
                                    averages, agreement with bench.py's own
                                    event-timed average launch
  decode_round_m8_hbm_counters.md   HBM bytes per decode launch from the two
                                    counter passes, each scaled by its reading
                                    for the plain copy of known size
  decode_kernel_traffic.json        the same bytes for bench.py, tagged with a
                                    hash of the decode kernel sources (bench.py
                                    reports them only while the hash matches)
  verify_topk_kernel_trace.md       the verify-width and top-k kernels (a whole
                                    bench run with few steps)
  prefill_m2048_mfma_counters.md    the prefill tile kernel's counted MFMA flops,
                                    rate against the bf16 peak, clock and MFMA
                                    busy fraction, LDS bank conflicts and VALU
                                    activity (two more counter passes)

Usage (on a machine with the GPU):  python3 bench_profile.py --out DIR
`--summarize-only` rebuilds the summaries from DIR without profiling.
"""
from __future__ import annotations

import argparse
import collections
import csv
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (host-only helpers; importing it touches no GPU)

BENCH_ARGS = ["--steps", "10", "--warmup", "2", "--no-cpu-baseline", "--no-sweep",
              "--calibration-copy"]
# The widths sweep, the verify-width rounds and the top-k timings (kernel
# trace only): the whole bench with few steps.
WIDE_ARGS = ["--steps", "4", "--warmup", "1", "--no-cpu-baseline"]
PASSES = (
    ("trace", ["--kernel-trace", "--stats"], 600, BENCH_ARGS),
    ("fetch", ["--pmc", "FETCH_SIZE"], 300, BENCH_ARGS),
    ("write", ["--pmc", "WRITE_SIZE"], 300, BENCH_ARGS),
    ("trace_wide", ["--kernel-trace", "--stats"], 600, WIDE_ARGS),
    # MFMA work and busy cycles of the prefill chunk (the same runs time it)
    ("mfma", ["--pmc", "SQ_INSTS_VALU_MFMA_MOPS_BF16", "SQ_VALU_MFMA_BUSY_CYCLES",
              "SQ_BUSY_CYCLES", "GRBM_GUI_ACTIVE"], 300, BENCH_ARGS),
    # ... and its LDS and VALU activity
    ("lds", ["--pmc", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE", "SQ_ACTIVE_INST_LDS",
             "SQ_WAIT_INST_LDS", "SQ_ACTIVE_INST_VALU", "SQ_VALU_MFMA_COEXEC_CYCLES",
             "GRBM_GUI_ACTIVE"], 300, BENCH_ARGS),
)
MFMA_COUNTERS = PASSES[4][1][1:]
LDS_COUNTERS = PASSES[5][1][1:]
VERIFY = "nvfp4::verify_kernel<"
TILE = "nvfp4::decode_tile_kernel<"
TOPK = "nvfp4::topk_"  # level and merge kernels
CALIB_BYTES = 1 << 30
DECODE = "nvfp4::decode_"  # decode_kernel< and decode_window_kernel<
# The prefill chunk's kernels, in bench.py's order: the default plan (on a
# 256-CU device whole tiles plus K pieces: tile kernel + K-piece sum kernel),
# the pieces schedule again by name, the stream-K schedule; then the round's
# four shapes at the chunk size, each under all three.
PREFILL_SK = "nvfp4::prefill_sk_kernel<"
PREFILL_PIECES = "nvfp4::prefill_kernel<"
PREFILL_SUM = "nvfp4::prefill_reduce_kernel<"


def chunk_dispatches(rows, name_of):
    """The prefill chunk's dispatches among `rows` (in time order; name_of(row)
    gives the kernel name): (tile kernel, K-piece sum kernel, stream-K kernel)
    lists.  The pieces dispatches are every one before the first stream-K
    dispatch; the stream-K ones are that first unbroken run."""
    pcs, psum, sk = [], [], []
    state = 0  # 0: before any stream-K dispatch, 1: in the first run, 2: after it
    for r in rows:
        n = name_of(r)
        if PREFILL_SK in n:
            if state < 2:
                state = 1
                sk.append(r)
        elif PREFILL_PIECES in n or PREFILL_SUM in n:
            if state == 1:
                state = 2
            if state == 0:
                (pcs if PREFILL_PIECES in n else psum).append(r)
    return pcs, psum, sk


COPY = "__amd_rocclr_copyBuffer"
# The achievable leg's one read of the whole weight arena: non-temporal
# 16-byte loads, the load type of the decode kernel's weight stream.
STREAM_READ_BIG = "nvfp4::stream_read_kernel"


def rocprof_cmd(flags, out_dir, args=BENCH_ARGS):
    return (["rocprofv3"] + flags + ["--output-format", "csv", "-d", out_dir, "-o", "run", "--",
                                     "python3", "-u", os.path.join(ROOT, "bench.py")] + args)


def shown(cmd):
    return " ".join(os.path.relpath(c, ROOT) if c.startswith(ROOT) else c for c in cmd)


def run_passes(out):
    env = dict(os.environ, TMPDIR="/tmp")
    for name, flags, limit, args in PASSES:
        d = os.path.join(out, name)
        cmd = rocprof_cmd(flags, d, args)
        print("== %s: %s" % (name, shown(cmd)), flush=True)
        with open(os.path.join(out, name + ".log"), "w") as log:
            r = subprocess.run(["timeout", "-s", "KILL", str(limit)] + cmd, cwd="/tmp", env=env,
                               stdout=log, stderr=subprocess.STDOUT)
        if r.returncode != 0:
            print("pass %s failed with status %d" % (name, r.returncode), flush=True)
            sys.exit(r.returncode)


def find_csv(d, suffix):
    for root, _, files in os.walk(d):
        for f in files:
            if f.endswith(suffix):
                return os.path.join(root, f)
    raise FileNotFoundError("no *%s under %s" % (suffix, d))


def bench_line(log_path):
    with open(log_path) as f:
        for line in f:
            if line.startswith("{\"metric\""):
                return json.loads(line)
    raise ValueError("no bench JSON line in " + log_path)


def short(name):
    n = name.split("(")[0]
    return n.replace("void ", "")


def summarize(out, dest):
    line = bench_line(os.path.join(out, "trace.log"))
    trace = list(csv.DictReader(open(find_csv(os.path.join(out, "trace"), "kernel_trace.csv"))))
    stats = list(csv.DictReader(open(find_csv(os.path.join(out, "trace"), "kernel_stats.csv"))))

    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    dec = [r for r in trace if DECODE in r["Kernel_Name"]]
    # the round's launches are those of the first replay's four shapes; the
    # other decode launches are the output head's
    round_keys = {(r["Kernel_Name"], r["Grid_Size_X"]) for r in dec[:4]}
    head = [r for r in dec if (r["Kernel_Name"], r["Grid_Size_X"]) not in round_keys]
    dec = [r for r in dec if (r["Kernel_Name"], r["Grid_Size_X"]) in round_keys]
    dur = lambda r: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    avg_us = lambda rs: sum(map(dur, rs)) / len(rs) / 1e3 if rs else float("nan")
    pcs, psum, sk = chunk_dispatches(trace, lambda r: r["Kernel_Name"])
    head_avg_us = sum(map(dur, head)) / len(head) / 1e3 if head else float("nan")

    # the first replay's first four launches are layer 0's qkv, o, gate_up, down
    layers = bench.LAYERS
    per_round = 4 * layers
    # bench.py's event time covers the timed replays only (after the warm-up
    # ones, before the single-replay spread): the same launches here
    t0 = line["warmup"] * per_round
    timed = dec[t0:t0 + line["steps"] * per_round]
    dec_avg_us = sum(map(dur, timed)) / len(timed) / 1e3
    names = {}
    for i, r in enumerate(dec[:4]):
        names[(r["Kernel_Name"], r["Grid_Size_X"])] = bench.ROUND_SHAPES[i]
    by_shape = collections.defaultdict(list)
    for r in dec:
        by_shape[(r["Kernel_Name"], r["Grid_Size_X"])].append(dur(r))

    roof = line["roofline"]
    algo = roof["avg_algorithmic_bytes_per_launch"]
    cmd_trace = shown(rocprof_cmd(PASSES[0][1], "OUT/trace"))
    md = []
    md.append("# Decode round (M = 8) and prefill chunk: kernel trace\n")
    md.append("Command (from the repository root, with `TMPDIR=/tmp`, run in /tmp):\n")
    md.append("    python3 bench_profile.py --out OUT\n")
    md.append("which runs, for this pass:\n")
    md.append("    " + cmd_trace + "\n")
    md.append("Workload: 27B-class round, 64 layers x {qkv 5120x7168, o 6144x5120, gate_up "
              "5120x34816, down 17408x5120} (K x N), NVFP4 weights, bf16 activations and "
              "outputs, M = 8 lanes, %d warm-up + %d timed graph replays (%d decode launches "
              "each); prefill chunk M = 2048, K = 5120, N = 17408.\n"
              % (line["warmup"], line["steps"], per_round))
    md.append("## Agreement with bench.py's event timing (same run)\n")
    md.append("| figure | bench.py (HIP events) | rocprofv3 kernel trace |")
    md.append("|---|---|---|")
    md.append("| decode kernel, average launch (us) | %.3f | %.3f |" % (roof["avg_launch_us"],
                                                                        dec_avg_us))
    md.append("| decode kernel, GB/s (algorithmic %d B per launch) | %.1f | %.1f |"
              % (algo, roof["achieved"], algo / (dec_avg_us * 1e-6) / 1e9))
    md.append("| M = 8 round (ms) | %.4f | %.4f (sum of kernel durations / replays) |"
              % (line["ms_per_step"], sum(map(dur, timed)) / (len(timed) / per_round) / 1e6))
    pc = line["prefill_chunk"]
    md.append("| prefill chunk, default plan (%s) (us) | %.2f | |" % (pc.get("default_schedule", "?"),
                                                                    pc["us"]))
    md.append("| prefill chunk, pieces schedule (us): tile kernel + K-piece sum kernel | %.2f | "
              "%.2f + %.2f = %.2f |" % (pc.get("pieces_us", float("nan")), avg_us(pcs),
                                        avg_us(psum) if psum else 0.0,
                                        avg_us(pcs) + (avg_us(psum) if psum else 0.0)))
    md.append("| prefill chunk, stream-K schedule (us) | %.2f | %.2f |"
              % (pc.get("stream_k_us", float("nan")), avg_us(sk)))
    for name, rs in pc.get("round_shapes", {}).items():
        md.append("| %s at M = 2048 (us): default (%s) / pieces / stream-K | %.2f / %.2f / %.2f "
                  "| |" % (name, rs["default_schedule"], rs["us"], rs["pieces_us"],
                           rs["stream_k_us"]))
    if "output_head" in line:
        md.append("| output head, M = 8, K = 5120, N = 152064, fp32 out (us) | %.2f | %.2f |"
                  % (line["output_head"]["us"], head_avg_us))
    md.append("")
    md.append("bench.py's average launch is the timed region's event time over the %d "
              "launches of a replay, so it includes the gaps between graph nodes; the "
              "trace's figure is kernel time only, over the same %d timed replays (launches "
              "%d .. %d of the %d decode launches in the trace; the per-shape table below "
              "takes all of them).\n" % (per_round, line["steps"], t0, t0 + len(timed) - 1,
                                          len(dec)))
    md.append("## Decode kernel per matrix shape\n")
    md.append("| matrix (K x N) | kernel | grid (threads) | launches | average (us) | "
              "algorithmic GB/s |")
    md.append("|---|---|---|---|---|---|")
    for key, ds in by_shape.items():
        name, K, N = names.get(key, ("?", 0, 0))
        nbytes = bench.weight_bytes(K, N) + 8 * K * 2 + 8 * N * 2
        avg = sum(ds) / len(ds)
        md.append("| %s %dx%d | %s | %s | %d | %.2f | %.1f |"
                  % (name, K, N, short(key[0]), key[1], len(ds), avg / 1e3, nbytes / avg))
    md.append("\n## All kernels in the run (rocprofv3 --stats)\n")
    md.append("| kernel | calls | average (us) | min (us) | max (us) | % of GPU time |")
    md.append("|---|---|---|---|---|---|")
    for r in stats[:14]:
        md.append("| %s | %s | %.2f | %.2f | %.2f | %s |"
                  % (short(r["Name"])[:90], r["Calls"], float(r["AverageNs"]) / 1e3,
                     float(r["MinNs"]) / 1e3, float(r["MaxNs"]) / 1e3, r["Percentage"]))
    md.append("\nKernels other than decode, prefill and the copy belong to building the "
              "inputs (weight draws, quantiser, packing) before the timed region.\n")
    with open(os.path.join(dest, "decode_round_m8_kernel_trace.md"), "w") as f:
        f.write("\n".join(md))

    # ---- counters
    def counter(pass_name):
        rows = list(csv.DictReader(open(find_csv(os.path.join(out, pass_name),
                                                 "counter_collection.csv"))))
        per = collections.defaultdict(float)
        meta = {}
        for r in rows:
            k = int(r["Dispatch_Id"])
            per[k] += float(r["Counter_Value"])
            meta[k] = (r["Kernel_Name"], r["Grid_Size"])
        dec_ids = sorted(k for k in per if DECODE in meta[k][0])
        keys = {meta[k] for k in dec_ids[:4]}  # the round's four shapes (not the head)
        dec_v = [per[k] for k in dec_ids if meta[k] in keys]
        cal = max(v for k, v in per.items() if COPY in meta[k][0])
        big = [v for k, v in per.items() if STREAM_READ_BIG in meta[k][0]]
        return dec_v, cal, len(dec_v), (sum(big) / len(big) if big else float("nan"))

    f_dec, f_cal, nf, f_big = counter("fetch")
    w_dec, w_cal, nw, _ = counter("write")
    f_factor = CALIB_BYTES / (f_cal * 1024)
    w_factor = CALIB_BYTES / (w_cal * 1024)
    arena = line["config"]["round_weight_bytes"]
    f_factor_nt = arena / (f_big * 1024)
    fetch_b = sum(f_dec) / nf * 1024 * f_factor
    write_b = sum(w_dec) / nw * 1024 * w_factor
    md = []
    md.append("# Decode kernel (M = 8 round): HBM traffic per launch\n")
    md.append("Commands (from the repository root, with `TMPDIR=/tmp`, run in /tmp), each a "
              "run of its own via `python3 bench_profile.py --out OUT`:\n")
    md.append("    " + shown(rocprof_cmd(PASSES[1][1], "OUT/fetch")))
    md.append("    " + shown(rocprof_cmd(PASSES[2][1], "OUT/write")) + "\n")
    md.append("Calibration: the same runs include one plain device copy of 1 GiB "
              "(`%s`, 1 GiB read and 1 GiB written).\n" % COPY)
    md.append("| counter | copy reading (KiB) | expected (KiB) | scale factor |")
    md.append("|---|---|---|---|")
    md.append("| FETCH_SIZE | %.0f | %d | %.4f |" % (f_cal, CALIB_BYTES // 1024, f_factor))
    md.append("| WRITE_SIZE | %.0f | %d | %.4f |\n" % (w_cal, CALIB_BYTES // 1024, w_factor))
    md.append("Cross-check of the FETCH_SIZE factor on the decode kernel's own load type: "
              "the same runs read the round's whole packed weight arena once with "
              "`nvfp4_stream_read` (non-temporal 16-byte loads, as the decode kernel's weight "
              "stream), %d bytes: FETCH_SIZE reads %.0f KiB, a factor of %.4f against %.4f "
              "for the copy.\n" % (arena, f_big, f_factor_nt, f_factor))
    md.append("| per decode launch (average over %d launches) | bytes |" % nf)
    md.append("|---|---|")
    md.append("| FETCH_SIZE x factor | %.0f |" % fetch_b)
    md.append("| WRITE_SIZE x factor | %.0f |" % write_b)
    md.append("| HBM traffic | %.0f |" % (fetch_b + write_b))
    md.append("| algorithmic (weights + activations in + bf16 out) | %d |" % algo)
    md.append("| traffic / algorithmic | %.3f |\n" % ((fetch_b + write_b) / algo))
    with open(os.path.join(dest, "decode_round_m8_hbm_counters.md"), "w") as f:
        f.write("\n".join(md))
    with open(os.path.join(dest, "decode_kernel_traffic.json"), "w") as f:
        json.dump({"kernel_source_hash": bench.kernel_source_hash(),
                   "fetch_bytes_per_launch": round(fetch_b),
                   "write_bytes_per_launch": round(write_b),
                   "algorithmic_bytes_per_launch": algo,
                   "launches": nf,
                   "fetch_scale": round(f_factor, 4), "write_scale": round(w_factor, 4),
                   "fetch_scale_nt_read": round(f_factor_nt, 4),
                   "workload": "M = 8 27B-class round, all 256 decode launches per replay"},
                  f, indent=1)
        f.write("\n")
    print("decode: trace %.3f us vs bench %.3f us; traffic %.0f B vs algorithmic %d B"
          % (dec_avg_us, roof["avg_launch_us"], fetch_b + write_b, algo))
    if os.path.isdir(os.path.join(out, "trace_wide")):
        summarize_wide(out, dest)
    if os.path.isdir(os.path.join(out, "mfma")):
        summarize_mfma(out, dest)


def counter_avgs(out, pass_name, counters):
    """Per-dispatch counter sums (over the device) averaged over the prefill
    chunk's pieces tile kernel and its stream-K kernel: ({counter: value},
    {counter: value}, dispatch counts)."""
    rows = list(csv.DictReader(open(find_csv(os.path.join(out, pass_name),
                                             "counter_collection.csv"))))
    per = collections.defaultdict(lambda: collections.defaultdict(float))
    name = {}
    for r in rows:
        k = int(r["Dispatch_Id"])
        per[k][r["Counter_Name"]] += float(r["Counter_Value"])
        name[k] = r["Kernel_Name"]
    pcs, _, sk = chunk_dispatches(sorted(name), lambda k: name[k])
    avg = lambda ids: {c: sum(per[k][c] for k in ids) / len(ids) for c in counters} if ids \
        else {c: float("nan") for c in counters}
    return avg(pcs), avg(sk), (len(pcs), len(sk))


def summarize_mfma(out, dest):
    """prefill_m2048_mfma_counters.md: the prefill chunk's MFMA work, for its
    pieces tile kernel (the default plan) and its stream-K kernel, from
    SQ_INSTS_VALU_MFMA_MOPS_BF16 (units of 512 flops) against the
    algorithmic 2 M K N, the rate over the kernel-trace duration against the
    2.5 PFLOP/s bf16 peak, the clock and the MFMA busy cycles; then the LDS
    and VALU pass."""
    a_pcs, a_sk, (n_pcs, n_sk) = counter_avgs(out, "mfma", MFMA_COUNTERS)
    trace = list(csv.DictReader(open(find_csv(os.path.join(out, "trace"), "kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    pcs, psum, sk = chunk_dispatches(trace, lambda r: r["Kernel_Name"])
    dur = lambda rs: sum(int(r["End_Timestamp"]) - int(r["Start_Timestamp"]) for r in rs) \
        / len(rs) / 1e3 if rs else float("nan")
    us = {"pcs": dur(pcs), "sk": dur(sk)}
    M, K, N = bench.PREFILL_SHAPE
    algo = 2.0 * M * K * N
    agent = [r for r in csv.DictReader(open(find_csv(os.path.join(out, "mfma"),
                                                     "agent_info.csv")))
             if r.get("Name", "").startswith("gfx")][0]
    xcc, simds = int(agent["Num_Xcc"]), int(agent["Simd_Count"])
    cus = int(agent["Cu_Count"]) if "Cu_Count" in agent else simds // 4
    md = ["# Prefill chunk (M = %d, K = %d, N = %d): MFMA, LDS and VALU counters\n" % (M, K, N)]
    md.append("Commands (from the repository root, with `TMPDIR=/tmp`, run in /tmp), each a run "
              "of its own via `python3 bench_profile.py --out OUT`:\n")
    md.append("    " + shown(rocprof_cmd(PASSES[4][1], "OUT/mfma")))
    md.append("    " + shown(rocprof_cmd(PASSES[5][1], "OUT/lds")))
    md.append("    " + shown(rocprof_cmd(PASSES[0][1], "OUT/trace")) + "\n")
    md.append("bench.py times the chunk with the default plan (whole tiles, the last round's "
              "tiles in K pieces: `%s...>` and its sum `%s...>`), with that schedule again by "
              "name, and with the stream-K schedule (`%s...>`). Counters per dispatch, summed "
              "over the device, averaged over the chunk's %d tile-kernel and %d stream-K "
              "dispatches of each run (the sum kernel issues no MFMA).\n"
              % (PREFILL_PIECES, PREFILL_SUM, PREFILL_SK, n_pcs, n_sk))
    md.append("| counter | pieces tile kernel | stream-K kernel |")
    md.append("|---|---|---|")
    for c in MFMA_COUNTERS:
        md.append("| %s | %.0f | %.0f |" % (c, a_pcs[c], a_sk[c]))

    def figs(a, t_us):
        flops = a["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512
        return {"flops": flops, "ratio": flops / algo, "us": t_us,
                "tflops": flops / t_us / 1e6, "frac": flops / t_us / 1e6 / 2500,
                "clk": a["GRBM_GUI_ACTIVE"] / xcc / (t_us * 1e3),
                "busy": a["SQ_VALU_MFMA_BUSY_CYCLES"] / (a["GRBM_GUI_ACTIVE"] / xcc * simds)}
    f_p, f_s = figs(a_pcs, us["pcs"]), figs(a_sk, us["sk"])
    md.append("\n| figure | pieces tile kernel | stream-K kernel |")
    md.append("|---|---|---|")
    md.append("| MFMA flops (MOPS_BF16 x 512) | %.4g | %.4g |" % (f_p["flops"], f_s["flops"]))
    md.append("| algorithmic flops 2 M K N | %.4g | %.4g |" % (algo, algo))
    md.append("| counted / algorithmic | %.4f | %.4f |" % (f_p["ratio"], f_s["ratio"]))
    md.append("| kernel-trace average (us) | %.2f | %.2f |" % (f_p["us"], f_s["us"]))
    md.append("| achieved bf16 MFMA rate (TFLOP/s) | %.1f | %.1f |" % (f_p["tflops"], f_s["tflops"]))
    md.append("| fraction of the 2.5 PFLOP/s dense bf16 peak | %.3f | %.3f |"
              % (f_p["frac"], f_s["frac"]))
    md.append("| clock while the kernel ran (GRBM_GUI_ACTIVE / %d XCDs / duration, GHz) "
              "| %.3f | %.3f |" % (xcc, f_p["clk"], f_s["clk"]))
    md.append("| MFMA pipes busy: SQ_VALU_MFMA_BUSY_CYCLES / (GRBM_GUI_ACTIVE / %d x %d SIMDs) "
              "| %.3f | %.3f |\n" % (xcc, simds, f_p["busy"], f_s["busy"]))
    md.append("The pieces schedule's figures are for its tile kernel alone (the K-piece sum "
              "kernel takes %.2f us more per call in the trace). SQ_VALU_MFMA_BUSY_CYCLES is the "
              "sum over SIMDs of cycles with an MFMA in flight: 32 per "
              "`v_mfma_f32_32x32x16_bf16` (MOPS / 2). The peak of 2.5 PFLOP/s assumes %d MHz; "
              "the clock counted during these kernels is lower, so the busy fraction at the "
              "running clock exceeds the fraction of peak.\n"
              % (dur(psum) if psum else 0.0, int(agent["Max_Engine_Clk_Fcompute"])))
    if os.path.isdir(os.path.join(out, "lds")):
        md += lds_table(out, a_pcs, a_sk, xcc, cus)
    with open(os.path.join(dest, "prefill_m2048_mfma_counters.md"), "w") as f:
        f.write("\n".join(md))
    print("prefill: counted MFMA flops %.4g / %.4g vs algorithmic %.4g; pieces %.2f us, "
          "stream-K %.2f us" % (f_p["flops"], f_s["flops"], algo, f_p["us"], f_s["us"]),
          flush=True)


def lds_table(out, m_pcs, m_sk, xcc, cus):
    """LDS and VALU activity of the two chunk kernels from the "lds" pass,
    with the derived figures by the expressions rocprofv3 -L gives for them
    (LDSBankConflict, LdsBankConflict, VALUBusy)."""
    a_pcs, a_sk, _ = counter_avgs(out, "lds", LDS_COUNTERS)
    md = ["## LDS and VALU activity\n", "| counter | pieces tile kernel | stream-K kernel |",
          "|---|---|---|"]
    for c in LDS_COUNTERS:
        md.append("| %s | %.0f | %.0f |" % (c, a_pcs[c], a_sk[c]))

    def figs(a, m):
        gui = a["GRBM_GUI_ACTIVE"] / xcc  # GRBM_GUI_ACTIVE of one XCD (the max over them)
        bank, idx = a["SQ_LDS_BANK_CONFLICT"], a["SQ_LDS_IDX_ACTIVE"]
        return (bank / (idx - bank), 100.0 * bank / gui / cus, 100.0 * idx / gui / cus,
                100.0 * a["SQ_ACTIVE_INST_VALU"] / cus / gui,
                a["SQ_VALU_MFMA_COEXEC_CYCLES"] / m["SQ_VALU_MFMA_BUSY_CYCLES"])
    p, k = figs(a_pcs, m_pcs), figs(a_sk, m_sk)
    md += ["\n| figure | pieces tile kernel | stream-K kernel |", "|---|---|---|",
           "| LDS bank-conflict cycles per conflict-free LDS cycle (LdsBankConflict: "
           "BANK_CONFLICT / (IDX_ACTIVE - BANK_CONFLICT)) | %.3f | %.3f |" % (p[0], k[0]),
           "| share of the kernel's time the LDS is stalled by bank conflicts "
           "(LDSBankConflict: 100 BANK_CONFLICT / GRBM_GUI_ACTIVE / %d CUs, %%) | %.1f | %.1f |"
           % (cus, p[1], k[1]),
           "| share of the kernel's time the LDS is active (100 IDX_ACTIVE / GRBM_GUI_ACTIVE / "
           "%d CUs, %%) | %.1f | %.1f |" % (cus, p[2], k[2]),
           "| VALUBusy (100 ACTIVE_INST_VALU / %d CUs / GRBM_GUI_ACTIVE, %%) | %.1f | %.1f |"
           % (cus, p[3], k[3]),
           "| cycles an MFMA and a VALU instruction issued together, per MFMA-busy cycle "
           "(VALU_MFMA_COEXEC / VALU_MFMA_BUSY of the MFMA pass) | %.3f | %.3f |" % (p[4], k[4])]
    md.append("\nThe two counter passes are separate runs of the same command.\n")
    return md


def summarize_wide(out, dest):
    """Verify-width rounds and top-k: per-kernel averages from the wide trace."""
    line = bench_line(os.path.join(out, "trace_wide.log"))
    trace = list(csv.DictReader(open(find_csv(os.path.join(out, "trace_wide"),
                                              "kernel_trace.csv"))))
    trace.sort(key=lambda r: int(r["Start_Timestamp"]))
    dur = lambda r: int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    md = ["# Verify-width rounds, narrow widths and top-k over the vocabulary: kernel trace\n"]
    md.append("Command (from the repository root, with `TMPDIR=/tmp`, run in /tmp):\n")
    md.append("    python3 bench_profile.py --out OUT\n")
    md.append("which runs, for this pass:\n")
    md.append("    " + shown(rocprof_cmd(PASSES[3][1], "OUT/trace_wide", WIDE_ARGS)) + "\n")
    md.append("## Verify-width rounds (64 layers, per-matrix graph; bench.py's round time beside)\n")
    ver = [r for r in trace if VERIFY in r["Kernel_Name"]]
    per_round = 4 * bench.LAYERS
    md.append("| M | bench.py round (ms) | trace: sum of kernel time per replay (ms) | "
              "qkv (us) | o (us) | gate_up (us) | down (us) |")
    md.append("|---|---|---|---|---|---|---|")
    # replays run M = 16, 32, 64 in order: 2 warm-up + max(5, steps // 2) timed each
    vr = line.get("verify_width_rounds", {})
    reps = 2 + max(5, 4 // 2)
    for i, M in enumerate((16, 32, 64)):
        seg = ver[i * reps * per_round:(i + 1) * reps * per_round]
        if len(seg) < per_round:
            continue
        shapes = collections.defaultdict(list)
        for j, r in enumerate(seg):
            shapes[j % 4].append(dur(r))
        avg = [sum(v) / len(v) / 1e3 for _, v in sorted(shapes.items())]
        md.append("| %d | %s | %.4f | %.2f | %.2f | %.2f | %.2f |"
                  % (M, vr.get(str(M), {}).get("round_ms", "-"),
                     sum(map(dur, seg)) / (len(seg) / per_round) / 1e6, *avg))
    md.append("\n## Narrow widths (M <= 4): the one-tile-per-workgroup kernel, per launch shape\n")
    md.append("From the same run's width sweep (M = 1..4 rounds), the projection (K = N = 5120, "
              "64 copies, M = 1, 2, 4) and the chained-MLP round (M = 1).  MR is the template's "
              "staged-row count (1, 2 or 4 rows).\n")
    md.append("| kernel (SBW, MR, bf16) | column tiles | waves per workgroup | matrix | launches | "
              "average (us) |")
    md.append("|---|---|---|---|---|---|")
    tiles_name = {448: "qkv 5120x7168", 2176: "gate_up 5120x34816", 9504: "head 5120x152064"}
    tgroups = collections.OrderedDict()
    for r in trace:
        if TILE in r["Kernel_Name"]:
            wg = int(r["Workgroup_Size_X"])
            key = (short(r["Kernel_Name"]), int(r["Grid_Size_X"]) // wg, wg // 64)
            tgroups.setdefault(key, []).append(dur(r))
    for (name, nt, waves), ds in tgroups.items():
        label = tiles_name.get(nt, "o 6144x5120" if (nt, waves) == (320, 12) else
                               "projection 5120x5120" if (nt, waves) == (320, 10) else "?")
        md.append("| %s | %d | %d | %s | %d | %.2f |" % (name.replace("nvfp4::", ""), nt, waves,
                                                          label, len(ds), sum(ds) / len(ds) / 1e3))
    md.append("\n## Top-k levels (per launch)\n")
    md.append("| kernel | grid X x Y (threads x rows) | launches | average (us) |")
    md.append("|---|---|---|---|")
    groups = collections.OrderedDict()
    for r in trace:
        if TOPK in r["Kernel_Name"]:
            key = (short(r["Kernel_Name"]), r["Grid_Size_X"], r.get("Grid_Size_Y", "1"))
            groups.setdefault(key, []).append(dur(r))
    for (name, gx, gy), ds in groups.items():
        md.append("| %s | %s x %s | %d | %.2f |" % (name, gx, gy, len(ds), sum(ds) / len(ds) / 1e3))
    md.append("\nbench.py's top-k figures (back-to-back calls, levels included): %s\n"
              % json.dumps(line.get("topk", {})))
    with open(os.path.join(dest, "verify_topk_kernel_trace.md"), "w") as f:
        f.write("\n".join(md))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--out", required=True, help="directory for rocprofv3 output and logs")
    ap.add_argument("--summarize-only", action="store_true")
    ap.add_argument("--dest", default=os.path.join(ROOT, "profiles"))
    args = ap.parse_args()
    out = os.path.abspath(args.out)
    os.makedirs(out, exist_ok=True)
    if not args.summarize_only:
        run_passes(out)
    os.makedirs(args.dest, exist_ok=True)
    summarize(out, args.dest)


if __name__ == "__main__":
    main()
