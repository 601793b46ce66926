"""GPU parity of the decode-round driver (one captured HIP graph per width).

A round of 12 matrices (3 layers x the four projections of the 27B-class
structure, at the real K and 1/16 of the real N) is replayed at every width
M = 1..8 and every matrix's output is compared with the oracle.  Replays are
repeated with eager GEMM work between them, each checked, and the outputs are
poisoned before every replay so a skipped node shows; a canary region after
each output must stay untouched.  A second round feeds outputs into later
matrices' activations (overwriting buffers that earlier matrices read) to
check the ordering of the graph's launches."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bf16_bits, canary_out, check, dev, dev_bf16, host, pack, require_gpu

pytestmark = pytest.mark.gpu

SHAPES = (("qkv", 5120, 448), ("o", 6144, 320), ("gate_up", 5120, 2176), ("down", 17408, 320))


@pytest.fixture(scope="module")
def small_round():
    import torch
    nv = require_gpu()
    specs, ref = [], []
    for layer in range(3):
        for j, (name, K, N) in enumerate(SHAPES):
            sid = synth.stream_id(layer, name)
            W = synth.weights(1, sid, N, K)
            codes, scales, t = oracle.quantize(W)
            act = synth.activations(1, sid, 8, K)
            y, S = oracle.gemm(act, codes, scales, t)
            out_dtype = nv.OUT_F32 if (layer + j) % 3 == 0 else nv.OUT_BF16
            dt = torch.float32 if out_dtype == nv.OUT_F32 else torch.bfloat16
            pw = pack(nv, dev(codes), dev(scales), K, N, t)
            out, canary = canary_out(8, N, dt)
            specs.append(dict(K=K, N=N, codes=pw.codes, scales=pw.scales, tensor_scale=t,
                              act=dev_bf16(act), out=out, out_dtype=out_dtype, pw=pw,
                              canary=canary))
            ref.append((y, S))
    ws_bytes = nv.nvfp4_round_workspace_bytes(specs, 8)
    ws = torch.full((max(ws_bytes, 16),), 0x5A, dtype=torch.uint8, device="cuda")  # create zeroes it
    plan = nv.nvfp4_round_create(specs, 8, ws, ws_bytes)
    yield nv, plan, specs, ref
    nv.nvfp4_round_destroy(plan)
    del ws


def _poison(specs):
    for s in specs:
        s["out"].fill_(float("nan"))


def _check_all(nv, specs, ref, M, what):
    for i, (s, (y, S)) in enumerate(zip(specs, ref)):
        check(s["out"][:M], y[:M], S[:M], bf16=s["out_dtype"] == nv.OUT_BF16,
              what="%s matrix %d" % (what, i))
        s["canary"]("%s matrix %d" % (what, i))


def test_graph_nodes(small_round):
    nv, plan, specs, _ = small_round
    for M in range(1, 9):
        assert nv.nvfp4_round_graph_nodes(plan, M) == len(specs)


@pytest.mark.parametrize("M", range(1, 9))
def test_round_every_width(small_round, M):
    import torch
    nv, plan, specs, ref = small_round
    _poison(specs)
    nv.nvfp4_round_run(plan, M)
    torch.cuda.synchronize()
    _check_all(nv, specs, ref, M, "width %d" % M)


def test_replays_with_eager_work_between(small_round):
    import torch
    nv, plan, specs, ref = small_round
    s0 = specs[2]
    g = nv.Gemm(8, s0["K"], s0["N"], s0["out_dtype"])
    scratch = torch.empty_like(s0["out"])
    prev = None
    for rep in range(4):
        _poison(specs)
        nv.nvfp4_round_run(plan, 8)
        torch.cuda.synchronize()
        _check_all(nv, specs, ref, 8, "replay %d" % rep)
        now = [host(s["out"]).copy() for s in specs]
        if prev is not None:  # bitwise identical replays
            for a, b in zip(prev, now):
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8))
        prev = now
        g(s0["pw"], s0["act"], scratch)  # eager work between replays
        torch.cuda.synchronize()


def test_round_invalid_width(small_round):
    nv, plan, _, _ = small_round
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_round_run(plan, 9)
    assert e.value.message.startswith("M")


def test_round_outputs_feed_later_matrices():
    """Outputs of a round feed later matrices' activations, and buffers that
    earlier matrices read are overwritten and read again within the replay:
        m0: A -> B   m1: B -> A   m2: A -> C (fp32)   m3: A -> D
        m4: D -> B   m5: B -> E (fp32)
    Every replay starts from A = X0 and poisoned B..E.  Replays must repeat
    bit for bit, and the matrices whose inputs are still in place at the end
    (m2..m5) must match the oracle on those inputs."""
    import torch
    nv = require_gpu()
    dims = [(1024, 1536, "A", "B", nv.OUT_BF16), (1536, 1024, "B", "A", nv.OUT_BF16),
            (1024, 2048, "A", "C", nv.OUT_F32), (1024, 512, "A", "D", nv.OUT_BF16),
            (512, 1024, "D", "B", nv.OUT_BF16), (1024, 768, "B", "E", nv.OUT_F32)]
    bufs = {"A": torch.empty((8, 1024), dtype=torch.bfloat16, device="cuda"),
            "B": torch.empty((8, 1536), dtype=torch.bfloat16, device="cuda"),
            "C": torch.empty((8, 2048), dtype=torch.float32, device="cuda"),
            "D": torch.empty((8, 512), dtype=torch.bfloat16, device="cuda"),
            "E": torch.empty((8, 768), dtype=torch.float32, device="cuda")}
    x0 = dev_bf16(synth.activations(3, 7, 8, 1024))
    specs, planes = [], []
    for i, (K, N, a, o, dt) in enumerate(dims):
        W = synth.weights(3, 100 + i, N, K)
        codes, scales, t = oracle.quantize(W)
        pw = pack(nv, dev(codes), dev(scales), K, N, t)
        # B is [8][1536]; as m4's output it holds N = 1024 values per row and
        # as m5's input K = 1024: the row stride must be the layer's own width.
        out = bufs[o] if bufs[o].shape[1] == N else bufs[o].view(-1)[:8 * N].view(8, N)
        act = bufs[a] if bufs[a].shape[1] == K else bufs[a].view(-1)[:8 * K].view(8, K)
        specs.append(dict(K=K, N=N, codes=pw.codes, scales=pw.scales, tensor_scale=t, act=act,
                          out=out, out_dtype=dt, pw=pw))
        planes.append((codes, scales, t))

    def reset():
        bufs["A"].copy_(x0)
        for k in "BCDE":
            bufs[k].fill_(float("nan"))

    wsb = nv.nvfp4_round_workspace_bytes(specs, 8)
    ws = torch.zeros(max(wsb, 16), dtype=torch.uint8, device="cuda")
    plan = nv.nvfp4_round_create(specs, 8, ws, wsb)
    snaps = []
    try:
        for M in (8, 3, 8):
            reset()
            nv.nvfp4_round_run(plan, M)
            torch.cuda.synchronize()
            snaps.append((M, {k: host(v).copy() for k, v in bufs.items()}))
    finally:
        nv.nvfp4_round_destroy(plan)
    (_, a), (_, b) = snaps[0], snaps[2]
    for k in bufs:
        assert np.array_equal(a[k].view(np.uint8), b[k].view(np.uint8)), k
    # Oracle on the inputs left in place (width 8).
    for i in (2, 3, 4, 5):
        s = specs[i]
        codes, scales, t = planes[i]
        act = bf16_bits(s["act"])
        y, S = oracle.gemm(act, codes, scales, t)
        check(s["out"], y, S, bf16=s["out_dtype"] == nv.OUT_BF16, what="fed-forward m%d" % i)


# ---- verify widths (per-matrix round with max_M = 64) ----------------------------

@pytest.fixture(scope="module")
def verify_round():
    """One layer of the four projections at 1/16 of the real N, 64 rows of
    activations, a per-matrix round over widths 1..64."""
    import torch
    nv = require_gpu()
    specs, ref = [], []
    for j, (name, K, N) in enumerate(SHAPES):
        sid = synth.stream_id(7, name)
        W = synth.weights(2, sid, N, K)
        codes, scales, t = oracle.quantize(W)
        act = synth.activations(2, sid, 64, K)
        y, S = oracle.gemm(act, codes, scales, t)
        out_dtype = nv.OUT_F32 if j % 2 == 0 else nv.OUT_BF16
        dt = torch.float32 if out_dtype == nv.OUT_F32 else torch.bfloat16
        pw = pack(nv, dev(codes), dev(scales), K, N, t)
        out, canary = canary_out(64, N, dt)
        specs.append(dict(K=K, N=N, codes=pw.codes, scales=pw.scales, tensor_scale=t,
                          act=dev_bf16(act), out=out, out_dtype=out_dtype, pw=pw,
                          canary=canary))
        ref.append((y, S))
    ws_bytes = nv.nvfp4_round_workspace_bytes(specs, 64)
    ws = torch.full((max(ws_bytes, 16),), 0x5A, dtype=torch.uint8, device="cuda")
    plan = nv.nvfp4_round_create(specs, 64, ws, ws_bytes)
    yield nv, plan, specs, ref
    nv.nvfp4_round_destroy(plan)
    del ws


@pytest.mark.parametrize("M", [1, 8, 9, 16, 17, 33, 48, 64])
def test_verify_width_round(verify_round, M):
    import torch
    nv, plan, specs, ref = verify_round
    assert nv.nvfp4_round_graph_nodes(plan, M) == len(specs)
    for rep in range(2):  # counters must reset between replays
        _poison(specs)
        nv.nvfp4_round_run(plan, M)
        torch.cuda.synchronize()
        _check_all(nv, specs, ref, M, "verify round M=%d replay %d" % (M, rep))
