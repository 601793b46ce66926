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
    ws_bytes = nv.nvfp4_round_workspace_bytes(specs, 8)
    ws = torch.full((max(ws_bytes, 16),), 0x5A, dtype=torch.uint8, device="cuda")  # create zeroes it
    plan = nv.nvfp4_round_create(specs, 8, ws, ws_bytes)
    yield nv, plan, specs, ref
    nv.nvfp4_round_destroy(plan)


def _poison(specs):
    for s in specs:
        s["out"].fill_(float("nan"))


def _check_all(nv, specs, ref, M, what):
    for i, (s, (y, S)) in enumerate(zip(specs, ref)):
        check(s["out"][:M], y[:M], S[:M], bf16=s["out_dtype"] == nv.OUT_BF16,
              what="%s matrix %d" % (what, i))


def test_graph_has_one_node_per_matrix(small_round):
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
