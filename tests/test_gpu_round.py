"""GPU parity of the decode-round driver (one captured HIP graph per width).

A round of 12 matrices (3 layers x the four projections of the 27B-class
structure, at the real K and 1/16 of the real N) is replayed at every width
M = 1..8 and every matrix's output is compared with the oracle.  Replays are
repeated with eager GEMM work between them, each checked, and the outputs are
poisoned before every replay so a skipped node shows."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import check, dev, dev_bf16, host, pack, require_gpu

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
            specs.append(dict(K=K, N=N, codes=pw.codes, scales=pw.scales, tensor_scale=t,
                              act=dev_bf16(act), out=torch.empty((8, N), dtype=dt, device="cuda"),
                              out_dtype=out_dtype, pw=pw))
            ref.append((y, S))
    plans = {}
    keep = []
    for mode in (nv.ROUND_PERSISTENT, nv.ROUND_PER_MATRIX):
        ws_bytes = nv.nvfp4_round_workspace_bytes(specs, 8, mode=mode)
        ws = torch.full((max(ws_bytes, 16),), 0x5A, dtype=torch.uint8, device="cuda")  # create zeroes it
        plans[mode] = nv.nvfp4_round_create(specs, 8, ws, ws_bytes, mode=mode)
        keep.append(ws)
    yield nv, plans, specs, ref
    for p in plans.values():
        nv.nvfp4_round_destroy(p)


def _poison(specs):
    for s in specs:
        s["out"].fill_(float("nan"))


def _check_all(nv, specs, ref, M, what):
    for i, (s, (y, S)) in enumerate(zip(specs, ref)):
        check(s["out"][:M], y[:M], S[:M], bf16=s["out_dtype"] == nv.OUT_BF16,
              what="%s matrix %d" % (what, i))


MODES = (0, 1)  # persistent, per-matrix


def test_graph_nodes(small_round):
    nv, plans, specs, _ = small_round
    for M in range(1, 9):
        assert nv.nvfp4_round_graph_nodes(plans[nv.ROUND_PER_MATRIX], M) == len(specs)
        assert nv.nvfp4_round_graph_nodes(plans[nv.ROUND_PERSISTENT], M) == 1


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M", range(1, 9))
def test_round_every_width(small_round, M, mode):
    import torch
    nv, plans, specs, ref = small_round
    _poison(specs)
    nv.nvfp4_round_run(plans[mode], M)
    torch.cuda.synchronize()
    _check_all(nv, specs, ref, M, "mode %d width %d" % (mode, M))
    assert nv.nvfp4_round_status(plans[mode]) == 0


@pytest.mark.parametrize("mode", MODES)
def test_replays_with_eager_work_between(small_round, mode):
    import torch
    nv, plans, specs, ref = small_round
    plan = plans[mode]
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


def test_both_forms_back_to_back(small_round):
    """The two forms replayed one after the other on the same buffers each
    match the oracle (their K slicing differs, so they need not agree bit for
    bit with each other)."""
    import torch
    nv, plans, specs, ref = small_round
    outs = {}
    for mode in MODES:
        _poison(specs)
        nv.nvfp4_round_run(plans[mode], 8)
        torch.cuda.synchronize()
        _check_all(nv, specs, ref, 8, "mode %d" % mode)
        outs[mode] = [host(s["out"]).copy() for s in specs]
    assert len(outs) == 2


def test_forced_wait_timeout_is_reported_and_recovers(small_round):
    """A spin limit of 0 makes every cross-matrix wait give up at once (the
    kernel still exits); the flag is reported, the counters re-armed, and the
    next replay with the normal limit is correct again."""
    import torch
    nv, plans, specs, ref = small_round
    plan = plans[nv.ROUND_PERSISTENT]
    nv.nvfp4_round_set_spin_limit(plan, 0)
    for _ in range(3):
        nv.nvfp4_round_run(plan, 8)
    torch.cuda.synchronize()
    flags = nv.nvfp4_round_status(plan)
    nv.nvfp4_round_set_spin_limit(plan, 1 << 16)
    assert flags in (0, 1)  # with no real wait needed the flag may stay clear
    _poison(specs)
    nv.nvfp4_round_run(plan, 8)
    torch.cuda.synchronize()
    _check_all(nv, specs, ref, 8, "after time-out")
    assert nv.nvfp4_round_status(plan) == 0


def test_round_invalid_width(small_round):
    nv, plans, _, _ = small_round
    for plan in plans.values():
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_round_run(plan, 9)
        assert e.value.message.startswith("M")
