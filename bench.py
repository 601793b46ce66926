"""Benchmark of the NVFP4 weight-streaming decode round on one MI355X.

One step = one replay of the 27B-class decode round: 64 layers x {qkv
5120x7168, o 6144x5120, gate_up 5120x34816, down 17408x5120} (K x N), every
matrix streamed once for M lanes, captured in one HIP graph per width.  The
headline runs M = 8 lanes; the same run also times widths 1..8.

Prints one JSON line (rank 0):
  value        = algorithmic bytes of the round (NVFP4 weights + bf16
                 activations in + bf16 outputs) / device time per round, GB/s
  roofline     = the decode kernel: average algorithmic bytes per launch over
                 the round's matrices / average launch duration (the timed
                 region's HIP event time over the round's launches) against
                 the MI355X HBM peak of 8 TB/s
  cpu_baseline = the CPU oracle timed on the host's cores on a bounded sample
                 of the same workload (see cpu_baseline() below)

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
LAYERS = 64
ROUND_SHAPES = (("qkv", 5120, 7168), ("o", 6144, 5120), ("gate_up", 5120, 34816),
                ("down", 17408, 5120))
METRIC = "NVFP4 decode GEMM GB/s & % HBM peak at M=1..8; 27B-class round ms"
# The prefill chunk timed beside the round: M, K, N (bf16 out).
PREFILL_SHAPE = (2048, 5120, 17408)


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


def round_bytes(M, layers=LAYERS):
    """Algorithmic bytes of one round: weights once, activations in and bf16
    outputs once."""
    b = 0
    for _, K, N in ROUND_SHAPES:
        b += weight_bytes(K, N) + M * K * 2 + M * N * 2
    return b * layers


def build_round(nv, seed=0, layers=LAYERS, max_M=8, log=None):
    """Generate, quantise and pack every matrix of the round on the GPU.
    Returns (round spec list, buffers kept alive, tensor scales)."""
    import torch
    import synth
    specs, keep = [], []
    total = sum(nv.nvfp4_packed_code_bytes(K, N) + nv.nvfp4_packed_scale_bytes(K, N)
                for _, K, N in ROUND_SHAPES) * layers
    arena = torch.empty(total, dtype=torch.uint8, device="cuda")
    keep.append(arena)
    off = 0
    qws = torch.empty(nv.nvfp4_quantize_workspace_bytes(), dtype=torch.uint8, device="cuda")
    ts_dev = torch.empty(layers * len(ROUND_SHAPES), dtype=torch.float32, device="cuda")
    t0 = time.time()
    for layer in range(layers):
        for j, (name, K, N) in enumerate(ROUND_SHAPES):
            idx = layer * len(ROUND_SHAPES) + j
            w = synth.weights_device(seed, synth.stream_id(layer, name), N, K)
            codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
            scales = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda")
            nv.nvfp4_quantize(w, K, N, codes, scales, ts_dev[idx:idx + 1], qws)
            cb, sb = nv.nvfp4_packed_code_bytes(K, N), nv.nvfp4_packed_scale_bytes(K, N)
            cpk = arena[off:off + cb]
            spk = arena[off + cb:off + cb + sb]
            off += cb + sb
            nv.nvfp4_pack(codes, scales, K, N, cpk, spk)
            del w, codes, scales
            act = synth.activations_device(seed, synth.stream_id(layer, name), max_M, K)
            out = torch.empty((max_M, N), dtype=torch.bfloat16, device="cuda")
            keep += [act, out]
            specs.append(dict(K=K, N=N, codes=cpk, scales=spk, tensor_scale=0.0, act=act,
                              out=out, out_dtype=nv.OUT_BF16, name=name, layer=layer))
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


def cpu_baseline(layers=None, lanes=8, threads=None):
    """The CPU oracle, as it stands, on a bounded sample of the round: the
    first `layers` layers' four matrices in full (default four layers, 335.5 M
    weights each), M = 8 lanes.  Drawing and quantising the sample (with the
    oracle's quantiser, rows split over threads) is not timed; the oracle GEMM
    is.  Returns (GB/s of NVFP4 weights processed, threads, sample
    description, seconds)."""
    from concurrent.futures import ThreadPoolExecutor
    import numpy as np
    import oracle
    import synth
    if threads is None:
        threads = int(os.environ.get("OMP_NUM_THREADS", "0")) or len(os.sched_getaffinity(0))
    if layers is None:
        layers = int(os.environ.get("NVFP4_CPU_SAMPLE_LAYERS", "4"))
    oracle.build()
    dt, nbytes = 0.0, 0
    with ThreadPoolExecutor(threads) as pool:
        for layer in range(layers):
            for name, K, N in ROUND_SHAPES:
                sid = synth.stream_id(layer, name)
                W = synth.weights(0, sid, N, K)
                t = oracle.tensor_scale(W)
                bounds = [N * i // threads for i in range(threads + 1)]
                parts = list(pool.map(lambda ab: oracle.quantize_rows(W[ab[0]:ab[1]], t),
                                      zip(bounds[:-1], bounds[1:])))
                del W
                codes = np.concatenate([c for c, _ in parts])
                scales = np.concatenate([s for _, s in parts])
                del parts
                act = synth.activations(0, sid, lanes, K)
                t0 = time.perf_counter()
                oracle.gemm(act, codes, scales, t, threads=threads)
                dt += time.perf_counter() - t0
                nbytes += weight_bytes(K, N)
    desc = ("oracle GEMM (fp64, exact dequantisation) over layer%s 0%s of the round in full "
            "(qkv, o, gate_up, down), M=%d lanes: %d weight bytes in %.2f s"
            % ("s" if layers > 1 else "", "..%d" % (layers - 1) if layers > 1 else "", lanes,
               nbytes, dt))
    return nbytes / dt / 1e9, threads, desc, dt


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--layers", type=int, default=LAYERS)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-sweep", action="store_true",
                    help="skip the M=1..8 sweep (profiling runs: keep only M=8 launches)")
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

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    nv.lib()
    torch.cuda.set_device(0)
    stream = torch.cuda.Stream()  # default priority
    log("building the round (%d layers) ..." % args.layers)
    plans, wss = {}, []
    with torch.cuda.stream(stream):
        specs, keep = build_round(nv, layers=args.layers, log=log)
        for mode in (nv.ROUND_PERSISTENT, nv.ROUND_PER_MATRIX, nv.ROUND_CHAIN):
            ws_bytes = nv.nvfp4_round_workspace_bytes(specs, 8, mode=mode)
            ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
            wss.append(ws)
            plans[mode] = nv.nvfp4_round_create(specs, 8, ws, ws_bytes, stream, mode=mode)
    torch.cuda.synchronize()
    nodes = {m: nv.nvfp4_round_graph_nodes(p, 8) for m, p in plans.items()}
    log("round graphs: persistent %d node(s), per-matrix %d nodes, chained %d node(s) per width"
        % (nodes[nv.ROUND_PERSISTENT], nodes[nv.ROUND_PER_MATRIX], nodes[nv.ROUND_CHAIN]))

    def time_round(plan, M, steps, warmup):
        """Mean device time per replay (ms): one HIP event pair around each
        replay, all on the stream the graph runs on."""
        for _ in range(warmup):
            nv.nvfp4_round_run(plan, M, stream)
        stream.synchronize()
        evs = []
        for _ in range(steps):
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            nv.nvfp4_round_run(plan, M, stream)
            b.record(stream)
            evs.append((a, b))
        torch.cuda.synchronize()
        return sum(a.elapsed_time(b) for a, b in evs) / steps

    headline = plans[nv.ROUND_PER_MATRIX]
    persistent = plans[nv.ROUND_PERSISTENT]
    # Headline: M = 8 lanes, the default round (one graph of per-matrix decode
    # kernels).  The timed region is the K replays bracketed by device
    # synchronisation.
    for _ in range(args.warmup):
        nv.nvfp4_round_run(headline, 8, stream)
    torch.cuda.synchronize()
    t_wall0 = time.perf_counter()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(args.steps):
        nv.nvfp4_round_run(headline, 8, stream)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall0
    ms8 = e0.elapsed_time(e1) / args.steps
    bytes8 = round_bytes(8, args.layers)
    gbs8 = bytes8 / (ms8 * 1e-3) / 1e9
    log("M=8 round: %.3f ms, %.1f GB/s (%.1f%% of 8 TB/s)" % (ms8, gbs8, 100 * gbs8 / HBM_PEAK_GBS))

    # Prefill chunk (M = 2048, K = 5120, N = 17408, bf16 out): the bf16 MFMA
    # kernel over dequantised tiles.  Timed right after the headline, before
    # the minutes of round sweeps below: timed after them, the same kernel
    # took 378-399 us instead of 334-345 us (the chip then runs it at a lower
    # clock; the counter pass shows 2.06 GHz even when timed early).
    import synth
    PM, PK, PN = PREFILL_SHAPE
    with torch.cuda.stream(stream):
        wp = synth.weights_device(0, 9001, PN, PK)
        ppw = nv.PackedWeight.quantize(wp, stream=stream)
        del wp
        pact = synth.activations_device(0, 9001, PM, PK)
        pout = torch.empty((PM, PN), dtype=torch.bfloat16, device="cuda")
        pg = nv.Gemm(PM, PK, PN, nv.OUT_BF16)
        for _ in range(2):
            pg(ppw, pact, pout, stream=stream)
        stream.synchronize()
        # back-to-back calls between one pair of events (throughput, as a
        # chunk loop issues them)
        n_pre = max(3, args.steps // 4)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n_pre):
            pg(ppw, pact, pout, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
    p_us = a.elapsed_time(b) / n_pre * 1e3
    p_tflops = 2.0 * PM * PK * PN / (p_us * 1e-6) / 1e12
    log("prefill M=%d K=%d N=%d: %.1f us, %.1f TFLOP/s (%.1f%% of 2.5 PF bf16)"
        % (PM, PK, PN, p_us, p_tflops, 100 * p_tflops / 2500.0))
    prefill = {"M": PM, "K": PK, "N": PN, "us": round(p_us, 2), "TFLOP_s": round(p_tflops, 1),
               "frac_bf16_mfma_peak": round(p_tflops / 2500.0, 4)}
    del ppw, pact, pout, pg

    sweep, sweep_ps, sweep_ch = {}, {}, {}
    for M in ([] if args.no_sweep else range(1, 9)):
        for mode, tab in ((nv.ROUND_PER_MATRIX, sweep), (nv.ROUND_PERSISTENT, sweep_ps),
                          (nv.ROUND_CHAIN, sweep_ch)):
            ms = time_round(plans[mode], M, max(5, args.steps // 2), 2)
            gbs = round_bytes(M, args.layers) / (ms * 1e-3) / 1e9
            tab[str(M)] = {"round_ms": round(ms, 4), "GB_s": round(gbs, 1),
                           "frac_hbm_peak": round(gbs / HBM_PEAK_GBS, 4)}
        log("M=%d: per-matrix graph %.3f ms (%.1f GB/s), persistent %.3f ms, chained %.3f ms "
            "(%.1f GB/s)" % (M, sweep[str(M)]["round_ms"], sweep[str(M)]["GB_s"],
                             sweep_ps[str(M)]["round_ms"], sweep_ch[str(M)]["round_ms"],
                             sweep_ch[str(M)]["GB_s"]))
    for mode in (nv.ROUND_PERSISTENT, nv.ROUND_CHAIN):
        flags = nv.nvfp4_round_status(plans[mode])
        assert flags == 0, "round form %d: a wait timed out (flags %d)" % (mode, flags)

    # Chained MLP: the same round with each down matrix reading the SwiGLU of
    # its layer's gate_up output (one more graph node per layer), so the
    # gate_up -> down pair is a dependent chain as in a forward pass.
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
            ms = time_round(cplan, M, max(5, args.steps // 2), 2)
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
    # and output buffers, a per-matrix round with one graph per width 1..64.
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
            ms = time_round(vplan, M, max(5, args.steps // 2), 2)
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
    launches = nodes[nv.ROUND_PER_MATRIX]
    dk_us = ms8 * 1e3 / launches
    avg_bytes = bytes8 / launches
    achieved = avg_bytes / (dk_us * 1e-6) / 1e9
    log("decode kernel: %.2f us average launch, %.0f bytes average, %.1f GB/s"
        % (dk_us, avg_bytes, achieved))


    # Output head (M = 8, K = 5120, N = 152064, fp32 logits): one decode launch
    # per call, default plan; back-to-back calls between one pair of events.
    HK, HN = 5120, 152064
    with torch.cuda.stream(stream):
        wh = synth.weights_device(0, 9002, HN, HK)
        hpw = nv.PackedWeight.quantize(wh, stream=stream)
        del wh
        hact = synth.activations_device(0, 9002, 8, HK)
        hout = torch.empty((8, HN), dtype=torch.float32, device="cuda")
        hg = nv.Gemm(8, HK, HN, nv.OUT_F32)
        for _ in range(3):
            hg(hpw, hact, hout, stream=stream)
        stream.synchronize()
        n_head = max(5, args.steps)
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(n_head):
            hg(hpw, hact, hout, stream=stream)
        b.record(stream)
        torch.cuda.synchronize()
    h_us = a.elapsed_time(b) / n_head * 1e3
    h_bytes = weight_bytes(HK, HN) + 8 * HK * 2 + 8 * HN * 4
    h_gbs = h_bytes / (h_us * 1e-6) / 1e9
    log("output head M=8 K=%d N=%d (fp32 out): %.1f us, %.1f GB/s (%.1f%% of 8 TB/s)"
        % (HK, HN, h_us, h_gbs, 100 * h_gbs / HBM_PEAK_GBS))
    head = {"M": 8, "K": HK, "N": HN, "out": "fp32", "us": round(h_us, 2),
            "algorithmic_bytes": h_bytes, "GB_s": round(h_gbs, 1),
            "frac_hbm_peak": round(h_gbs / HBM_PEAK_GBS, 4)}

    # Top-k over the vocabulary, the step after the head: on the head's own
    # logits (k = 1, the greedy argmax, and k = 8), and on 7 rows of a
    # 248320-entry vocabulary (the size class of the pages' drafter top-k).
    def time_topk(logits, k, reps=20):
        M, V = logits.shape
        idx = torch.empty((M, k), dtype=torch.int32, device="cuda")
        val = torch.empty((M, k), dtype=torch.float32, device="cuda")
        wsb = nv.nvfp4_topk_workspace_bytes(M, V, k)
        ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device="cuda")
        with torch.cuda.stream(stream):
            for _ in range(3):
                nv.nvfp4_topk(logits, M, V, V, k, idx, val, ws, wsb, stream)
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                nv.nvfp4_topk(logits, M, V, V, k, idx, val, ws, wsb, stream)
            b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / reps * 1e3
    import synth
    topk = {}
    for k in (1, 8):
        us = time_topk(hout, k)
        topk["head_M8_V%d_k%d" % (HN, k)] = {"us": round(us, 2)}
        log("top-k of the head's logits (M=8, V=%d, k=%d): %.2f us" % (HN, k, us))
    lg = torch.from_numpy(synth.logits(0, 9003, 7, 248320)).cuda()
    us = time_topk(lg, 7)
    topk["M7_V248320_k7"] = {"us": round(us, 2)}
    log("top-k M=7 V=248320 k=7: %.2f us" % us)
    del hpw, hact, hout, hg, lg

    if args.calibration_copy:
        # A plain copy kernel of known size: 1 GiB read, 1 GiB written.
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        v, thr, desc, dt = cpu_baseline()
        cpu = {"value": round(v, 5), "unit": "GB/s", "cores": thr, "kind": "oracle",
               "sample": desc}
        log("cpu baseline: %.4f GB/s on %d threads (%.1f s)" % (v, thr, dt))

    for p in plans.values():
        nv.nvfp4_round_destroy(p)
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
            "graph_kernel_nodes": nodes[nv.ROUND_PER_MATRIX],
            "parallelism": "single GPU",
        },
        "frac_hbm_peak": round(gbs8 / HBM_PEAK_GBS, 4),
        "round_ms_m1_to_m8": {k: v["round_ms"] for k, v in sweep.items()},
        "round_sweep": sweep,
        "round_sweep_persistent_kernel": sweep_ps,
        "round_sweep_chained": sweep_ch,
        "verify_width_rounds": verify,
        "chained_mlp_rounds": chained,
        "roofline": {
            "bound": "hbm",
            "kernel": "nvfp4::decode_window_kernel<WAVES, 1, true> (split-K decode, slices streamed "
                      "in windows of one superblock, bf16 out), M=8",
            "achieved": round(achieved, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(achieved / HBM_PEAK_GBS, 4),
            "avg_launch_us": round(dk_us, 3),
            "avg_algorithmic_bytes_per_launch": round(avg_bytes),
            "launches_per_round": 4 * args.layers,
            "traffic": traffic,
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
