"""Benchmark of the NVFP4 weight-streaming decode round on one MI355X.

One step = one replay of the 27B-class decode round: 64 layers x {qkv
5120x7168, o 6144x5120, gate_up 5120x34816, down 17408x5120} (K x N), every
matrix streamed once for M lanes, captured in one HIP graph per width.  The
headline runs M = 8 lanes; the same run also times widths 1..8, the other
workloads of the same path (single projection, output head, prefill chunk,
verify widths, top-k, the chained MLP) and a plain streaming read of the same
bytes (the achievable rate).

Prints one JSON line (rank 0):
  value        = algorithmic bytes of the round (NVFP4 weights + bf16
                 activations in + bf16 outputs) / device time per round, GB/s
  roofline     = the decode kernel: average algorithmic bytes per launch over
                 the round's matrices / average launch duration (the timed
                 region's HIP event time over the round's launches) against
                 the MI355X HBM peak of 8 TB/s; `achievable` beside it is a
                 plain streaming read of the same weight bytes, timed here
  cpu_baseline = the CPU oracle timed on the host's cores on bounded samples
                 of the workloads (see cpu_baseline() below)

Inputs are synthetic (seeded N(0, 0.02) fp32 weights quantised on the GPU,
N(0, 1) bf16 activations) and resident in HBM before the timed region.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0
LAYERS = 64
ROUND_SHAPES = (("qkv", 5120, 7168), ("o", 6144, 5120), ("gate_up", 5120, 34816),
                ("down", 17408, 5120))
METRIC = "NVFP4 decode GEMM GB/s & % HBM peak at M=1..8; 27B-class round ms"
# The prefill chunk timed beside the round: M, K, N (bf16 out).
PREFILL_SHAPE = (2048, 5120, 17408)
# The single-projection config: K = N = 5120, bf16 out, widths 1, 2, 4, 8,
# over this many distinct weight copies chained in one graph (0.94 GB, well
# above the 256 MB Infinity Cache, so every call streams from HBM).
PROJ_K = PROJ_N = 5120
PROJ_COPIES = 64
# The output head: M = 8, K = 5120, N = 152064, fp32 logits; two weight copies
# alternate so consecutive calls never find their weights in a cache.
HEAD_K, HEAD_N = 5120, 152064


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode_kernel_traffic.json")
KERNEL_SOURCES = ("nvfp4_weight_streaming_amd/csrc/decode.hip",
                  "nvfp4_weight_streaming_amd/csrc/decode_device.h")


def kernel_source_hash():
    import hashlib
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic():
    """HBM bytes per decode launch from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, each scaled by its reading for a plain copy of
    known size), or None if the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_hash") != kernel_source_hash():
        return None
    return t


def weight_bytes(K, N):
    return K * N // 2 + K * N // 16


def gemm_bytes(M, K, N, out_bytes=2):
    """Algorithmic bytes of one GEMM: weights once, bf16 activations in, outputs."""
    return weight_bytes(K, N) + M * K * 2 + M * N * out_bytes


def round_bytes(M, layers=LAYERS):
    """Algorithmic bytes of one round: weights once, activations in and bf16
    outputs once."""
    return sum(gemm_bytes(M, K, N) for _, K, N in ROUND_SHAPES) * layers


def prefill_default_schedule(M, K, N):
    """The schedule a default plan runs a prefill of M rows with on this
    device: "stream-K" below one 256 x 256 tile per compute unit when at most
    3/4 of the units hold a tile (and every run is at least half a tile),
    else "pieces" (whole tiles, a last partial round cut along K)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = ((M + 255) // 256) * ((N + 255) // 256)
    nk = (K + 63) // 64
    applies = tiles % cus != 0 and tiles * nk // cus >= max(1, (nk + 1) // 2)
    return "stream-K" if applies and tiles < cus and 4 * tiles <= 3 * cus else "pieces"


def build_round(nv, seed=0, layers=LAYERS, max_M=8, log=None, shapes=ROUND_SHAPES):
    """Generate, quantise and pack every matrix of the round on the GPU (all
    packed planes in one arena, in round order).  Returns (round spec list,
    buffers kept alive; keep[0] is the arena)."""
    import torch
    import synth
    specs, keep = [], []
    total = sum(nv.nvfp4_packed_code_bytes(K, N) + nv.nvfp4_packed_scale_bytes(K, N)
                for _, K, N in shapes) * layers
    arena = torch.empty(total, dtype=torch.uint8, device="cuda")
    keep.append(arena)
    off = 0
    qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(), dtype=torch.uint8, device="cuda")
    ts_dev = torch.empty(layers * len(shapes), dtype=torch.float32, device="cuda")
    t0 = time.time()
    for layer in range(layers):
        for j, (name, K, N) in enumerate(shapes):
            idx = layer * len(shapes) + j
            sid = synth.stream_id(layer, name) if name in synth.PROJECTIONS else 5000 + idx
            w = synth.weights_device(seed, sid, N, K)
            codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
            scales = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda")
            nv.nvfp4_quantize(w, K, N, codes, scales, ts_dev[idx:idx + 1], qws)
            cb, sb = nv.nvfp4_packed_code_bytes(K, N), nv.nvfp4_packed_scale_bytes(K, N)
            cpk = arena[off:off + cb]
            spk = arena[off + cb:off + cb + sb]
            nv.nvfp4_pack(codes, scales, K, N, cpk, spk)
            del w, codes, scales
            act = synth.activations_device(seed, sid, max_M, K)
            out = torch.empty((max_M, N), dtype=torch.bfloat16, device="cuda")
            keep += [act, out]
            specs.append(dict(K=K, N=N, codes=cpk, scales=spk, tensor_scale=0.0, act=act,
                              out=out, out_dtype=nv.OUT_BF16, name=name, layer=layer,
                              arena_off=off, packed_bytes=cb + sb))
            off += cb + sb
        if log and layer % 16 == 15:
            torch.cuda.synchronize()
            log("  built layers 0..%d (%.1f s)" % (layer, time.time() - t0))
    ts = ts_dev.cpu().tolist()
    for s, t in zip(specs, ts):
        s["tensor_scale"] = t
    torch.cuda.synchronize()
    return specs, keep


def synth_act(spec, rows, seed=0):
    """bf16 activations [rows][K] for one matrix of the round (its own stream)."""
    import synth
    return synth.activations_device(seed, synth.stream_id(spec["layer"], spec["name"]), rows,
                                    spec["K"])


# ---- CPU baseline: the oracle as it stands, on the host's cores -----------------

def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_planes(pool, threads, sid, N, K, rows=None):
    """Canonical planes of a synthetic weight matrix quantised by the oracle
    (the tensor scale over the whole matrix; rows [0, rows) quantised)."""
    import numpy as np
    import oracle
    import synth
    W = synth.weights(0, sid, N, K)
    t = oracle.tensor_scale(W)
    R = N if rows is None else rows
    bounds = [R * i // threads for i in range(threads + 1)]
    parts = list(pool.map(lambda ab: oracle.quantize_rows(W[ab[0]:ab[1]], t),
                          zip(bounds[:-1], bounds[1:])))
    del W
    return (np.concatenate([c for c, _ in parts]), np.concatenate([s for _, s in parts]), t)


def _gpu_parity(gpu, planes, act_bits, M, K, N, out_dtype, y, S, rows=None):
    """Runs the library's GEMM (default plan for M rows) on the oracle's own
    planes and activations, and returns, over the first `rows` rows: max
    |out - y| / S, the largest fraction of the acceptance bound used (fp32
    outputs 2^-16 S; bf16 outputs that plus the store's rounding), and whether
    every output is within the bound."""
    import numpy as np
    import oracle
    nv, torch, stream = gpu
    c, s, t = planes
    rows = M if rows is None else rows
    with torch.cuda.stream(stream):
        pw = nv.PackedWeight.from_canonical(torch.from_numpy(c).cuda(), torch.from_numpy(s).cuda(),
                                            t, K, N, stream)
        act = torch.from_numpy(np.ascontiguousarray(act_bits).view(np.int16)).cuda()
        act = act.view(torch.bfloat16)
        g = nv.Gemm(M, K, N, out_dtype)
        dt = torch.float32 if out_dtype == nv.OUT_F32 else torch.bfloat16
        out = torch.empty((M, N), dtype=dt, device="cuda")
        g(pw, act, out, M=M, stream=stream)
    torch.cuda.synchronize()
    o = out[:rows].float().cpu().numpy().astype(np.float64)
    y, S = y[:rows], S[:rows]
    err = np.abs(o - y)
    bound = oracle.tolerance(S) if out_dtype == nv.OUT_F32 else oracle.tolerance_bf16(y, S)
    tiny = np.finfo(np.float64).tiny
    ratio = float((err / np.maximum(S, tiny)).max())
    used = float((err / np.maximum(bound, tiny)).max())
    return ratio, used, bool(np.all(err <= bound))


def cpu_baseline(threads=None, round_layers=None, gpu=None):
    """The CPU oracle (fp64, exact dequantisation), as it stands, timed on the
    host's cores on bounded samples of each workload.  Drawing and quantising
    inputs (with the oracle's quantiser, rows split over threads) is not
    timed; the oracle GEMM is.  Returns a dict: the headline sample (layers
    0..round_layers-1 of the round in full at M = 8, GB/s of weight bytes),
    and per-config seconds and rates:
      tiny       M = 1, K = 256, N = 512, in full
      projection M = 1, 2, 4, 8, K = N = 5120, in full
      head       M = 8, K = 5120, the first N/8 = 19008 of the 152064 rows
      prefill    8 of the 2048 rows, K = 5120, N = 17408 in full
    Rates for sampled configs are per unit of work, so they scale to the full
    config (the oracle's cost is linear in rows and in weights).
    With `gpu` = (nv, torch, stream), every oracle result except the head's
    is also compared with the library's output on the same planes and
    activations (default plans; the prefill chunk run at all 2048 rows):
    `max_err_over_S` and `within_bound` in each config's entry."""
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    import synth
    if threads is None:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    if round_layers is None:
        round_layers = int(os.environ.get("NVFP4_CPU_SAMPLE_LAYERS", "2"))
    oracle.build()
    per = {}

    def timed(act, planes):
        c, s, t = planes
        t0 = time.perf_counter()
        y, S = oracle.gemm(act, c, s, t, threads=threads)
        return time.perf_counter() - t0, y, S

    checks = []

    def parity(entry, planes, act, M, K, N, out_dtype, y, S, rows=None):
        if gpu is None:
            return
        ratio, used, ok = _gpu_parity(gpu, planes, act, M, K, N, out_dtype, y, S, rows)
        entry["max_err_over_S"] = float("%.3g" % ratio)
        entry["max_err_over_bound"] = float("%.3g" % used)
        entry["within_bound"] = ok
        checks.append(ok)

    nv = gpu[0] if gpu is not None else None

    with ThreadPoolExecutor(threads) as pool:
        # the round sample (the headline metric's unit: GB/s of weight bytes)
        dt, nbytes = 0.0, 0
        worst, worst_used, all_ok = 0.0, 0.0, True
        for layer in range(round_layers):
            for name, K, N in ROUND_SHAPES:
                sid = synth.stream_id(layer, name)
                planes = _oracle_planes(pool, threads, sid, N, K)
                act = synth.activations(0, sid, 8, K)
                sec, y, S = timed(act, planes)
                dt += sec
                nbytes += weight_bytes(K, N)
                if gpu is not None:
                    m = {}
                    parity(m, planes, act, 8, K, N, nv.OUT_BF16, y, S)
                    worst = max(worst, m["max_err_over_S"])
                    worst_used = max(worst_used, m["max_err_over_bound"])
                    all_ok = all_ok and m["within_bound"]
                del planes, y, S
        head_value = nbytes / dt / 1e9
        per["round_sample"] = {
            "layers": round_layers, "M": 8, "seconds": round(dt, 3),
            "weight_bytes": nbytes, "GB_s": round(head_value, 5),
            "est_full_round_s": round(dt * LAYERS / round_layers, 1)}
        if gpu is not None:
            per["round_sample"]["max_err_over_S"] = worst
            per["round_sample"]["max_err_over_bound"] = worst_used
            per["round_sample"]["within_bound"] = all_ok
        # tiny
        planes = _oracle_planes(pool, threads, 0, 512, 256)
        act = synth.activations(0, 0, 1, 256)
        sec, y, S = timed(act, planes)
        per["tiny"] = {"M": 1, "K": 256, "N": 512, "seconds": round(sec, 6)}
        parity(per["tiny"], planes, act, 1, 256, 512, nv and nv.OUT_F32, y, S)
        # projection
        planes = _oracle_planes(pool, threads, 100, PROJ_N, PROJ_K)
        proj = {}
        for M in (1, 2, 4, 8):
            act = synth.activations(0, 100, M, PROJ_K)
            sec, y, S = timed(act, planes)
            proj[str(M)] = {"seconds": round(sec, 4),
                            "GB_s": round(gemm_bytes(M, PROJ_K, PROJ_N) / sec / 1e9, 5)}
            parity(proj[str(M)], planes, act, M, PROJ_K, PROJ_N, nv and nv.OUT_BF16, y, S)
        per["projection"] = proj
        # output head, first N/8 rows
        rows = HEAD_N // 8
        planes = _oracle_planes(pool, threads, 9002, HEAD_N, HEAD_K, rows=rows)
        sec, y, S = timed(synth.activations(0, 9002, 8, HEAD_K), planes)
        per["head"] = {"M": 8, "rows": rows, "of_rows": HEAD_N, "seconds": round(sec, 3),
                       "GB_s": round(weight_bytes(HEAD_K, rows) / sec / 1e9, 5),
                       "est_full_s": round(sec * HEAD_N / rows, 2)}
        del planes, y, S
        # prefill chunk, the first 8 of its 2048 rows of activations
        PM, PK, PN = PREFILL_SHAPE
        planes = _oracle_planes(pool, threads, 9001, PN, PK)
        act = synth.activations(0, 9001, PM, PK)
        sec, y, S = timed(act[:8], planes)
        per["prefill"] = {"M_sampled": 8, "of_M": PM, "K": PK, "N": PN, "seconds": round(sec, 3),
                          "GFLOP_s": round(2.0 * 8 * PK * PN / sec / 1e9, 3),
                          "est_full_s": round(sec * PM / 8, 1)}
        parity(per["prefill"], planes, act, PM, PK, PN, nv and nv.OUT_BF16, y, S, rows=8)
        del planes, y, S
    desc = ("oracle GEMM (fp64, exact dequantisation) over layers 0..%d of the round in full "
            "(qkv, o, gate_up, down), M=8 lanes: %d weight bytes in %.2f s"
            % (round_layers - 1, nbytes, dt))
    res = {"value": round(head_value, 5), "unit": "GB/s", "cores": threads, "kind": "oracle",
           "sample": desc, "cpu_model": _cpu_model(), "per_config": per}
    if gpu is not None:
        res["gpu_outputs_within_bound"] = all(checks) and per["round_sample"]["within_bound"]
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="time only the M=8 round and the prefill chunk (profiling runs)")
    ap.add_argument("--calibration-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (for scaling memory counters)")
    ap.add_argument("--quiet", action="store_true")
    args = ap.parse_args()

    def log(msg):
        if not args.quiet:
            print(msg, file=sys.stderr, flush=True)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: this build has no multi-GPU path (the decode round "
              "of one card); run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import nvfp4_weight_streaming_amd as nv
    import synth

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    nv.lib()
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()  # default priority
    log("building the round (%d layers) ..." % args.layers)
    with torch.cuda.stream(stream):
        specs, keep = build_round(nv, layers=args.layers, log=log)
        ws_bytes = nv.nvfp4_round_workspace_bytes(specs, 8)
        ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
        plan = nv.nvfp4_round_create(specs, 8, ws, ws_bytes, stream)
    torch.cuda.synchronize()
    nodes = nv.nvfp4_round_graph_nodes(plan, 8)
    log("round graph: %d kernel nodes per width" % nodes)

    def time_events(fn, reps, warmup=2):
        """Mean device time per call (ms): one HIP event pair on `stream`
        around `reps` back-to-back calls."""
        for _ in range(warmup):
            fn()
        stream.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            fn()
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps

    # Headline: M = 8 lanes.  The timed region is the K replays between two
    # events on the replay stream, bracketed by device synchronisation.
    for _ in range(args.warmup):
        nv.nvfp4_round_run(plan, 8, stream)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        nv.nvfp4_round_run(plan, 8, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    ms8 = e0.elapsed_time(e1) / args.steps
    bytes8 = round_bytes(8, args.layers)
    gbs8 = bytes8 / (ms8 * 1e-3) / 1e9
    log("M=8 round: %.3f ms, %.1f GB/s (%.1f%% of 8 TB/s)" % (ms8, gbs8, 100 * gbs8 / HBM_PEAK_GBS))
    # The same K replays again, one event between consecutive ones: the spread
    # of single replays (median, minimum, maximum) beside the mean above.
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    evs[0].record(stream)
    for i in range(args.steps):
        nv.nvfp4_round_run(plan, 8, stream)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    each = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    replays = {"median_ms": round(each[len(each) // 2], 4), "min_ms": round(each[0], 4),
               "max_ms": round(each[-1], 4), "replays": args.steps}
    log("M=8 round, single replays: median %.3f ms, min %.3f, max %.3f"
        % (replays["median_ms"], replays["min_ms"], replays["max_ms"]))

    # Prefill chunk (M = 2048, K = 5120, N = 17408, bf16 out): the bf16 MFMA
    # kernel over dequantised tiles.  Timed right after the headline: after
    # minutes of sustained load the chip runs it at a lower clock.
    PM, PK, PN = PREFILL_SHAPE
    with torch.cuda.stream(stream):
        wp = synth.weights_device(0, 9001, PN, PK)
        ppw = nv.PackedWeight.quantize(wp, stream=stream)
        del wp
        pact = synth.activations_device(0, 9001, PM, PK)
        pout = torch.empty((PM, PN), dtype=torch.bfloat16, device="cuda")
        pg = nv.Gemm(PM, PK, PN, nv.OUT_BF16)
        # both schedules named, on the same data: whole tiles plus K pieces
        # of a last partial round, and stream-K
        pg_pieces = nv.Gemm(PM, PK, PN, nv.OUT_BF16, prefill_schedule=nv.PREFILL_PIECES)
        pg_sk = nv.Gemm(PM, PK, PN, nv.OUT_BF16, prefill_schedule=nv.PREFILL_STREAM_K)
    reps = max(3, args.steps // 4)
    p_us = time_events(lambda: pg(ppw, pact, pout, stream=stream), reps) * 1e3
    p_tflops = 2.0 * PM * PK * PN / (p_us * 1e-6) / 1e12
    log("prefill M=%d K=%d N=%d: %.1f us, %.1f TFLOP/s (%.1f%% of 2.5 PF bf16)"
        % (PM, PK, PN, p_us, p_tflops, 100 * p_tflops / BF16_MFMA_PEAK_TFLOPS))
    pp_us = time_events(lambda: pg_pieces(ppw, pact, pout, stream=stream), reps) * 1e3
    ps_us = time_events(lambda: pg_sk(ppw, pact, pout, stream=stream), reps) * 1e3
    log("prefill schedules: pieces %.1f us, stream-K %.1f us" % (pp_us, ps_us))
    prefill = {"M": PM, "K": PK, "N": PN, "us": round(p_us, 2), "TFLOP_s": round(p_tflops, 1),
               "frac_bf16_mfma_peak": round(p_tflops / BF16_MFMA_PEAK_TFLOPS, 4),
               "default_schedule": prefill_default_schedule(PM, PK, PN),
               "pieces_us": round(pp_us, 2), "stream_k_us": round(ps_us, 2)}
    del ppw, pg, pg_pieces, pg_sk

    # The round's four matrices at the chunk size (M = 2048, bf16 out): the
    # default plan, and the pieces schedule beside it on the same data.
    prefill_round = {}
    for name, RK, RN in ROUND_SHAPES:
        with torch.cuda.stream(stream):
            wr = synth.weights_device(0, 9100 + RK + RN, RN, RK)
            rpw = nv.PackedWeight.quantize(wr, stream=stream)
            del wr
            ract = pact[:, :RK] if RK <= PK else synth.activations_device(0, 9101, PM, RK)
            ract = ract.contiguous()
            rout = torch.empty((PM, RN), dtype=torch.bfloat16, device="cuda")
            rg = nv.Gemm(PM, RK, RN, nv.OUT_BF16)
            rgp = nv.Gemm(PM, RK, RN, nv.OUT_BF16, prefill_schedule=nv.PREFILL_PIECES)
            rgs = nv.Gemm(PM, RK, RN, nv.OUT_BF16, prefill_schedule=nv.PREFILL_STREAM_K)
        r_us = time_events(lambda: rg(rpw, ract, rout, stream=stream), reps) * 1e3
        rp_us = time_events(lambda: rgp(rpw, ract, rout, stream=stream), reps) * 1e3
        rs_us = time_events(lambda: rgs(rpw, ract, rout, stream=stream), reps) * 1e3
        fl = 2.0 * PM * RK * RN
        prefill_round[name] = {"K": RK, "N": RN, "us": round(r_us, 2),
                               "frac_bf16_mfma_peak": round(fl / (r_us * 1e-6) / 1e12
                                                            / BF16_MFMA_PEAK_TFLOPS, 4),
                               "default_schedule": prefill_default_schedule(PM, RK, RN),
                               "pieces_us": round(rp_us, 2), "stream_k_us": round(rs_us, 2)}
        log("prefill M=%d %s (K=%d N=%d): %.1f us (pieces %.1f, stream-K %.1f)"
            % (PM, name, RK, RN, r_us, rp_us, rs_us))
        del rpw, ract, rout, rg, rgp, rgs
    prefill["round_shapes"] = prefill_round
    del pact, pout

    # Achievable: a plain streaming read of the same weight bytes, (a) as one
    # read of the whole arena and (b) as a graph of 256 reads, one per matrix
    # with that matrix's byte size, the shape of the round graph.
    arena = keep[0]
    sink = torch.zeros(4, dtype=torch.int32, device="cuda")
    big_ms = time_events(lambda: nv.nvfp4_stream_read(arena, arena.numel(), sink, stream), 5)
    big_gbs = arena.numel() / (big_ms * 1e-3) / 1e9
    rg = torch.cuda.CUDAGraph()
    with torch.cuda.graph(rg, stream=stream):
        for s in specs:
            nv.nvfp4_stream_read(arena[s["arena_off"]:], s["packed_bytes"], sink)
    def replay_reads():
        with torch.cuda.stream(stream):
            rg.replay()
    graph_ms = time_events(replay_reads, 10)
    wbytes = sum(s["packed_bytes"] for s in specs)
    graph_gbs = wbytes / (graph_ms * 1e-3) / 1e9
    log("achievable: one read of the %.2f GB arena %.3f ms (%.1f GB/s); graph of %d reads "
        "%.3f ms (%.1f GB/s)" % (arena.numel() / 1e9, big_ms, big_gbs, len(specs), graph_ms,
                                 graph_gbs))
    del rg
    achievable = {"single_read_GB_s": round(big_gbs, 1), "single_read_ms": round(big_ms, 4),
                  "graph_of_reads_ms": round(graph_ms, 4), "graph_of_reads_GB_s": round(graph_gbs, 1),
                  "graph_nodes": len(specs),
                  "what": "nvfp4_stream_read over the round's packed weights: one read of the "
                          "whole arena, and a graph of one read per matrix"}

    sweep = {}
    for M in ([] if args.no_sweep else range(1, 9)):
        ms = time_events(lambda: nv.nvfp4_round_run(plan, M, stream), max(5, args.steps // 2))
        gbs = round_bytes(M, args.layers) / (ms * 1e-3) / 1e9
        sweep[str(M)] = {"round_ms": round(ms, 4), "GB_s": round(gbs, 1),
                         "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        log("M=%d round: %.3f ms (%.1f GB/s, %.1f%%)" % (M, ms, gbs, 100 * gbs / HBM_PEAK_GBS))

    # Single projection (K = N = 5120, bf16 out) over PROJ_COPIES distinct
    # weight copies chained in one graph: the per-GEMM mean at M = 1, 2, 4, 8.
    projection = {}
    if not args.no_sweep:
        with torch.cuda.stream(stream):
            pspecs, pkeep = build_round(nv, layers=PROJ_COPIES, shapes=(("proj", PROJ_K, PROJ_N),))
            pws_b = nv.nvfp4_round_workspace_bytes(pspecs, 8)
            pws = torch.zeros(max(pws_b, 16), dtype=torch.uint8, device="cuda")
            pplan = nv.nvfp4_round_create(pspecs, 8, pws, pws_b, stream)
        torch.cuda.synchronize()
        for M in (1, 2, 4, 8):
            ms = time_events(lambda: nv.nvfp4_round_run(pplan, M, stream), max(5, args.steps // 2))
            us = ms * 1e3 / PROJ_COPIES
            gbs = gemm_bytes(M, PROJ_K, PROJ_N) / (us * 1e-6) / 1e9
            projection[str(M)] = {"us_per_gemm": round(us, 3), "GB_s": round(gbs, 1),
                                  "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
            log("projection M=%d K=N=5120: %.2f us per GEMM (%.1f GB/s) over %d copies"
                % (M, us, gbs, PROJ_COPIES))
        nv.nvfp4_round_destroy(pplan)
        del pspecs, pkeep, pws

    # Output head (M = 8, K = 5120, N = 152064, fp32 logits), two weight copies
    # alternating, back-to-back calls between one pair of events.
    with torch.cuda.stream(stream):
        hpws = []
        for c in range(2):
            wh = synth.weights_device(0, 9002 + 10 * c, HEAD_N, HEAD_K)
            hpws.append(nv.PackedWeight.quantize(wh, stream=stream))
            del wh
        hact = synth.activations_device(0, 9002, 8, HEAD_K)
        hout = torch.empty((8, HEAD_N), dtype=torch.float32, device="cuda")
        hg = nv.Gemm(8, HEAD_K, HEAD_N, nv.OUT_F32)
    n_head = max(6, args.steps) // 2 * 2
    flip = [0]

    def head_call():
        hg(hpws[flip[0]], hact, hout, stream=stream)
        flip[0] ^= 1
    h_us = time_events(head_call, n_head) * 1e3
    h_bytes = gemm_bytes(8, HEAD_K, HEAD_N, out_bytes=4)
    h_gbs = h_bytes / (h_us * 1e-6) / 1e9

    # A plain read of the head's own weight bytes (one read of each packed
    # copy's codes and scales, alternating), the floor for this kernel.
    def head_read():
        hp = hpws[flip[0]]
        nv.nvfp4_stream_read(hp.codes, hp.codes.numel(), sink, stream)
        nv.nvfp4_stream_read(hp.scales, hp.scales.numel(), sink, stream)
        flip[0] ^= 1
    hr_us = time_events(head_read, n_head) * 1e3
    log("output head M=8 K=%d N=%d (fp32 out): %.1f us, %.1f GB/s (%.1f%% of 8 TB/s, %.1f%% of "
        "the single-read rate); a plain read of its weights %.1f us" % (
            HEAD_K, HEAD_N, h_us, h_gbs, 100 * h_gbs / HBM_PEAK_GBS, 100 * h_gbs / big_gbs,
            hr_us))
    head = {"M": 8, "K": HEAD_K, "N": HEAD_N, "out": "fp32", "us": round(h_us, 2),
            "algorithmic_bytes": h_bytes, "GB_s": round(h_gbs, 1),
            "frac_hbm_peak": round(h_gbs / HBM_PEAK_GBS, 4),
            "frac_of_achievable": round(h_gbs / big_gbs, 4), "weight_copies": 2,
            "plain_read_of_weights_us": round(hr_us, 2),
            "time_over_plain_read": round(h_us / hr_us, 4)}

    # Greedy sampling after the head: the argmax fused into the head's run
    # (nvfp4_gemm_run_argmax), against the head followed by the top-k kernel
    # with k = 1 (same plan, same weight copies).
    hidx = torch.empty(8, dtype=torch.int32, device="cuda")
    area_b = nv.nvfp4_gemm_argmax_area_bytes(hg.plan)
    area = torch.empty(area_b, dtype=torch.uint8, device="cuda")

    def head_argmax():
        hp = hpws[flip[0]]
        nv.nvfp4_gemm_run_argmax(hg.plan, 8, HEAD_K, HEAD_N, hp.codes, hp.scales, hp.tensor_scale,
                                 hact, hout, hidx, hg.workspace, area, area_b, stream)
        flip[0] ^= 1
    ha_us = time_events(head_argmax, n_head) * 1e3
    k1_idx = torch.empty((8, 1), dtype=torch.int32, device="cuda")
    k1_val = torch.empty((8, 1), dtype=torch.float32, device="cuda")
    k1_wsb = nv.nvfp4_topk_workspace_bytes(8, HEAD_N, 1)
    k1_ws = torch.empty(max(k1_wsb, 16), dtype=torch.uint8, device="cuda")

    def head_then_topk():
        head_call()
        nv.nvfp4_topk(hout, 8, HEAD_N, HEAD_N, 1, k1_idx, k1_val, k1_ws, k1_wsb, stream)
    ht_us = time_events(head_then_topk, n_head) * 1e3
    log("output head + greedy argmax: fused %.1f us; head then top-k (k=1) %.1f us"
        % (ha_us, ht_us))
    head["with_argmax_fused_us"] = round(ha_us, 2)
    head["then_topk_k1_us"] = round(ht_us, 2)
    del area, hidx, k1_idx, k1_val, k1_ws

    # Top-k over the vocabulary, the step after the head: on the head's own
    # logits (k = 1, the greedy argmax, and k = 8), and on 7 rows of a
    # 248320-entry vocabulary (the size class of the pages' drafter top-k).
    def time_topk(logits, k, reps=20):
        M, V = logits.shape
        idx = torch.empty((M, k), dtype=torch.int32, device="cuda")
        val = torch.empty((M, k), dtype=torch.float32, device="cuda")
        wsb = nv.nvfp4_topk_workspace_bytes(M, V, k)
        tws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        return time_events(lambda: nv.nvfp4_topk(logits, M, V, V, k, idx, val, tws, wsb, stream),
                           reps, warmup=3) * 1e3
    topk = {}
    if not args.no_sweep:
        for k in (1, 8):
            us = time_topk(hout, k)
            topk["head_M8_V%d_k%d" % (HEAD_N, k)] = {"us": round(us, 2)}
            log("top-k of the head's logits (M=8, V=%d, k=%d): %.2f us" % (HEAD_N, k, us))
        lg = torch.from_numpy(synth.logits(0, 9003, 7, 248320)).cuda()
        us = time_topk(lg, 7)
        topk["M7_V248320_k7"] = {"us": round(us, 2)}
        log("top-k M=7 V=248320 k=7: %.2f us" % us)
        del lg
    del hpws, hact, hout, hg

    # Chained MLP: the same round with each down matrix reading the SwiGLU of
    # its layer's gate_up output (made by gate_up's epilogue where its plan
    # allows, else by one more graph node per layer), so the gate_up -> down
    # pair is a dependent chain as in a forward pass.
    chained = {}
    if not args.no_sweep:
        with torch.cuda.stream(stream):
            cspecs = []
            for sp in specs:
                if sp["name"] == "down":
                    sp = dict(sp, act=torch.empty((8, sp["K"]), dtype=torch.bfloat16,
                                                  device="cuda"), act_op=nv.ACT_SWIGLU_PREV)
                cspecs.append(sp)
            cws_bytes = nv.nvfp4_round_workspace_bytes(cspecs, 8)
            cws = torch.zeros(max(cws_bytes, 16), dtype=torch.uint8, device="cuda")
            cplan = nv.nvfp4_round_create(cspecs, 8, cws, cws_bytes, stream)
        torch.cuda.synchronize()
        for M in (1, 8):
            ms = time_events(lambda: nv.nvfp4_round_run(cplan, M, stream), max(5, args.steps // 2))
            gbs = round_bytes(M, args.layers) / (ms * 1e-3) / 1e9
            chained[str(M)] = {"round_ms": round(ms, 4), "GB_s": round(gbs, 1),
                               "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4),
                               "graph_nodes": nv.nvfp4_round_graph_nodes(cplan, M)}
            log("chained-MLP round M=%d (SwiGLU between gate_up and down): %.3f ms, %.1f GB/s"
                % (M, ms, gbs))
        nv.nvfp4_round_destroy(cplan)
        del cspecs, cws

    # Verify widths (speculative decoding checks up to 7 drafts per lane in the
    # same pass: up to 8 x 8 = 64 rows): the same weights, 64-row activation
    # and output buffers, a round with one graph per width 1..64.
    verify = {}
    if not args.no_sweep:
        t_v = time.time()
        with torch.cuda.stream(stream):
            vspecs = []
            for sp in specs:
                vspecs.append(dict(sp, act=synth_act(sp, 64),
                                   out=torch.empty((64, sp["N"]), dtype=torch.bfloat16,
                                                   device="cuda")))
            vws_bytes = nv.nvfp4_round_workspace_bytes(vspecs, 64)
            vws = torch.zeros(max(vws_bytes, 16), dtype=torch.uint8, device="cuda")
            vplan = nv.nvfp4_round_create(vspecs, 64, vws, vws_bytes, stream)
        torch.cuda.synchronize()
        log("verify-width round (widths 1..64) built in %.1f s" % (time.time() - t_v))
        for M in (16, 32, 64):
            ms = time_events(lambda: nv.nvfp4_round_run(vplan, M, stream), max(5, args.steps // 2))
            gbs = round_bytes(M, args.layers) / (ms * 1e-3) / 1e9
            verify[str(M)] = {"round_ms": round(ms, 4), "GB_s": round(gbs, 1),
                              "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
            log("verify width M=%d: %.3f ms, %.1f GB/s (%.1f%% of 8 TB/s)"
                % (M, ms, gbs, 100 * gbs / HBM_PEAK_GBS))
        nv.nvfp4_round_destroy(vplan)
        del vspecs, vws

    # Roofline of the dominant kernel.  The M = 8 round graph runs nothing but
    # decode kernels, one per matrix, in sequence on `stream`, so its average
    # launch duration is the timed region's event time over the launches (it
    # includes the short gaps between graph nodes, so it is an upper bound).
    dk_us = ms8 * 1e3 / nodes
    avg_bytes = bytes8 / nodes
    achieved = avg_bytes / (dk_us * 1e-6) / 1e9
    log("decode kernel: %.2f us average launch, %.0f bytes average, %.1f GB/s (%.1f%% of the "
        "graph-of-reads rate)" % (dk_us, avg_bytes, achieved, 100 * achieved / graph_gbs))

    if args.calibration_copy:
        # A plain copy kernel of known size: 1 GiB read, 1 GiB written.
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    nv.nvfp4_round_destroy(plan)
    cpu = None
    if not args.no_cpu_baseline:
        t_c = time.time()
        cpu = cpu_baseline(gpu=(nv, torch, stream))
        log("cpu baseline: %.4f GB/s on %d threads (%s); leg took %.1f s"
            % (cpu["value"], cpu["cores"], cpu["cpu_model"], time.time() - t_c))

    tr = measured_traffic()
    traffic = None
    if tr is not None:
        traffic = round(tr["fetch_bytes_per_launch"] + tr["write_bytes_per_launch"])
    line = {
        "metric": METRIC,
        "value": round(gbs8, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms8, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "27B-class dense decode round: %d layers x {qkv 5120x7168, o 6144x5120, "
                        "gate_up 5120x34816, down 17408x5120} (K x N), NVFP4 weights "
                        "(E2M1 + E4M3 per 16 + fp32 per tensor), bf16 activations and outputs, "
                        "M=8 lanes, one hipGraph replay per round (one decode kernel per matrix)"
                        % args.layers,
            "lanes": 8,
            "round_weight_bytes": sum(weight_bytes(K, N) for _, K, N in ROUND_SHAPES) * args.layers,
            "round_bytes_m8": bytes8,
            "graph_kernel_nodes": nodes,
            "parallelism": "single GPU",
        },
        "frac_hbm_peak": round(gbs8 / HBM_PEAK_GBS, 4),
        "round_m8_single_replays": replays,
        "round_ms_m1_to_m8": {k: v["round_ms"] for k, v in sweep.items()},
        "round_sweep": sweep,
        "projection": projection,
        "verify_width_rounds": verify,
        "chained_mlp_rounds": chained,
        "roofline": {
            "bound": "hbm",
            "kernel": "nvfp4::decode_window_kernel (split-K decode, slices streamed in windows, "
                      "bf16 out), M=8",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(dk_us, 3),
            "avg_algorithmic_bytes_per_launch": round(avg_bytes),
            "launches_per_round": nodes,
            "traffic": traffic,
            "achievable": achievable,
            "frac_of_graph_of_reads": round(achieved / graph_gbs, 4),
        },
        "prefill_chunk": prefill,
        "output_head": head,
        "topk": topk,
        "cpu_baseline": cpu,
        "timed_wall_s": round(wall, 3),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
