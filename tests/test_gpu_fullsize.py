"""Full-size parity: the 27B-class round and the output head, in the launch
configuration the benchmark times, checked on sampled output columns of
every matrix.

Weights are drawn on the GPU by the seeded generator (synth.weights_device);
the oracle reads the host copy of that same draw, computes the tensor scale
over the whole matrix, quantises the sampled rows itself and computes their
outputs.  The GPU's own quantised and packed planes are unpacked for those
rows and must equal the oracle's bit for bit."""
import numpy as np
import pytest

import bench
import oracle
import synth
from tests.gpu_util import bf16_bits, check, host, require_gpu

pytestmark = pytest.mark.gpu

# Every matrix of the round (64 layers x 4 projections), each on its own
# sampled columns: the first and last tiles' edges plus random ones.
SAMPLED = [(layer, name) for layer in range(64) for name in ("qkv", "o", "gate_up", "down")]


def _sample_cols(N, seed, n_random=48):
    rng = np.random.default_rng(seed)
    cols = set(rng.choice(N, n_random, replace=False).tolist())
    cols |= {0, 1, 15, 16, N - 17, N - 16, N - 1}
    return np.array(sorted(cols))


def _oracle_rows(nv, K, N, sid, cols, codes_packed, scales_packed, gpu_t, seed=0):
    """Oracle planes for the sampled rows, checked against the GPU's."""
    import torch
    W = synth.weights_device(seed, sid, N, K).cpu().numpy()
    t = oracle.tensor_scale(W)
    assert t == gpu_t, (t, gpu_t)
    c_ref, s_ref = oracle.quantize_rows(W[cols], t)
    c_gpu = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    s_gpu = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda")
    nv.nvfp4_unpack(codes_packed, scales_packed, K, N, c_gpu, s_gpu)
    sel = torch.from_numpy(cols).cuda()
    assert np.array_equal(host(c_gpu[sel]), c_ref)
    assert np.array_equal(host(s_gpu[sel]), s_ref)
    return c_ref, s_ref, t


@pytest.fixture(scope="module")
def full_round():
    import torch
    nv = require_gpu()
    specs, keep = bench.build_round(nv, layers=64)
    ws_bytes = nv.nvfp4_round_workspace_bytes(specs, 8)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    plan = nv.nvfp4_round_create(specs, 8, ws, ws_bytes)
    keep.append(ws)
    refs = {}
    for layer, name in SAMPLED:
        s = next(x for x in specs if x["layer"] == layer and x["name"] == name)
        cols = _sample_cols(s["N"], layer * 7 + len(name), n_random=16)
        c, sc, t = _oracle_rows(nv, s["K"], s["N"], synth.stream_id(layer, name), cols,
                                s["codes"], s["scales"], s["tensor_scale"])
        act = bf16_bits(s["act"])
        y, S = oracle.gemm(act, c, sc, t)  # [8][len(cols)]
        refs[(layer, name)] = (s, cols, y, S)
    yield nv, plan, specs, refs
    nv.nvfp4_round_destroy(plan)
    del keep


@pytest.mark.parametrize("M", [1, 5, 8])
def test_full_round_sampled(full_round, M):
    import torch
    nv, plan, specs, refs = full_round
    assert nv.nvfp4_round_graph_nodes(plan, M) == 256
    for s in specs:
        s["out"].fill_(float("nan"))
    nv.nvfp4_round_run(plan, M)
    torch.cuda.synchronize()
    for (layer, name), (s, cols, y, S) in refs.items():
        out = s["out"][:M][:, torch.from_numpy(cols).cuda()]
        check(out, y[:M], S[:M], bf16=True, what="layer %d %s M=%d" % (layer, name, M))
    # no matrix left unwritten
    for s in specs:
        assert not torch.isnan(s["out"][:M]).any()


def test_output_head_sampled():
    """Output head: M = 8, K = 5120, N = 152064, fp32 logits."""
    import torch
    nv = require_gpu()
    K, N, M = 5120, 152064, 8
    sid = 9000
    w = synth.weights_device(0, sid, N, K)
    pw = nv.PackedWeight.quantize(w)
    del w
    act = synth.activations_device(0, sid, M, K)
    g = nv.Gemm(M, K, N, nv.OUT_F32)
    out = torch.full((M, N), float("nan"), device="cuda")
    g(pw, act, out)
    torch.cuda.synchronize()
    cols = _sample_cols(N, 5)
    c, sc, t = _oracle_rows(nv, K, N, sid, cols, pw.codes, pw.scales, pw.tensor_scale)
    y, S = oracle.gemm(bf16_bits(act), c, sc, t)
    check(out[:, torch.from_numpy(cols).cuda()], y, S, bf16=False, what="head")
    assert not torch.isnan(out).any()
