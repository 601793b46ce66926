"""GPU parity of the SwiGLU step (bit for bit against the oracle) and of a
round that chains gate_up -> SwiGLU -> down (against the oracle, and bit for
bit against the same steps run as separate calls)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bf16_bits, check, dev, dev_bf16, host, pack, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _gate_up_bits(M, F, seed):
    """bf16 [M][2F]: N(0, 1) draws with special values planted."""
    x = synth.activations(seed, 77, M, 2 * F)
    rng = np.random.default_rng(seed)
    special = np.array([0x0000, 0x8000, 0x4300, 0xC300, 0x0001, 0x8001, 0x42C8, 0xC2C8,
                        0x3F80, 0xBF80, 0x7F7F, 0x0080], np.uint16)  # 0, -0, +-128, +-2^-133,
    #                                                  +-100, +-1, the largest, the smallest normal
    idx = rng.choice(x.size, min(x.size, 4 * len(special)), replace=False)
    x.flat[idx] = np.resize(special, len(idx))
    return x


@pytest.mark.parametrize("M,F", [(1, 1), (3, 7), (8, 17408), (64, 1000), (5, 4096)])
def test_swiglu_matches_oracle(nv, M, F):
    import torch
    gu = _gate_up_bits(M, F, M + F)
    out = torch.full((M, F), -1, dtype=torch.int16, device="cuda")
    nv.nvfp4_swiglu(dev_bf16(gu), M, F, out)
    torch.cuda.synchronize()
    got = host(out).view(np.uint16)
    want = oracle.swiglu(gu)
    bad = np.argwhere(got != want)
    assert bad.size == 0, (bad[:3], got[tuple(bad[0])], want[tuple(bad[0])])


# (K, F, widths, widths whose gate_up epilogue writes the SwiGLU itself):
# K = 512 (one superblock) keeps the SwiGLU kernel at every width; K = 2048
# (two K slices: the last workgroup's epilogue) and K = 1024 (one slice: every
# workgroup's epilogue) take the tile kernel up to 4 lanes and the fused
# epilogue from 5 on.
CHAINED = [(512, 1024, (1, 5, 8), ()), (2048, 1024, (1, 4, 5, 7, 8), (5, 7, 8)),
           (1024, 1024, (2, 5, 8), (5, 8))]


@pytest.mark.parametrize("K,F,widths,fused", CHAINED)
def test_chained_mlp_round(nv, K, F, widths, fused):
    """Two layers of x -> gate_up -> SwiGLU -> down, the down matrices reading
    the round-made SwiGLU of the gate_up outputs (made by the SwiGLU kernel, or
    by gate_up's own epilogue where its plan allows).  Every replay is checked
    against the oracle step by step: gate_up against oracle.gemm, the
    round-made activations bit for bit against oracle.swiglu of the gate_up
    output the round wrote, and down against oracle.gemm of those activations
    (bf16 bound).  It must also equal the same steps run as separate calls,
    bit for bit."""
    import torch
    specs, mats, planes = [], [], []
    for layer in range(2):
        for j, (k, n) in enumerate(((K, 2 * F), (F, K))):
            codes, scales = synth.random_planes(40 + layer, j, n, k)
            t = 2e-3 if j == 0 else 5e-4
            pw = pack(nv, dev(codes), dev(scales), k, n, t)
            if j == 0:
                x = synth.activations(41 + layer, 0, 8, k)
                act = dev_bf16(x)
            else:
                x = None
                act = torch.zeros((8, k), dtype=torch.bfloat16, device="cuda")  # round-made
            out = torch.empty((8, n), dtype=torch.bfloat16, device="cuda")
            specs.append(dict(K=k, N=n, codes=pw.codes, scales=pw.scales, tensor_scale=t,
                              act=act, out=out, out_dtype=nv.OUT_BF16,
                              act_op=nv.ACT_SWIGLU_PREV if j == 1 else nv.ACT_INPUT))
            mats.append(pw)
            planes.append((codes, scales, t, x))
    ws_bytes = nv.nvfp4_round_workspace_bytes(specs, 8)
    ws = torch.zeros(max(ws_bytes, 16), dtype=torch.uint8, device="cuda")
    plan = nv.nvfp4_round_create(specs, 8, ws, ws_bytes)
    try:
        for M in widths:
            # + two SwiGLU nodes where the gate_up epilogue does not make them
            assert nv.nvfp4_round_graph_nodes(plan, M) == len(specs) + (0 if M in fused else 2)
            for s in specs:
                s["out"].fill_(float("nan"))
            for s in specs[1::2]:
                s["act"].fill_(float("nan"))  # round-made: every value must be rewritten
            nv.nvfp4_round_run(plan, M)
            torch.cuda.synchronize()
            for layer in range(2):
                gu_s, dn_s = specs[2 * layer], specs[2 * layer + 1]
                # the oracle, step by step
                gc, gs, gt, gx = planes[2 * layer]
                dc, ds, dt, _ = planes[2 * layer + 1]
                y, S = oracle.gemm(gx[:M], gc, gs, gt)
                check(gu_s["out"][:M], y, S, bf16=True, what="gate_up M=%d" % M)
                gu_bits = bf16_bits(gu_s["out"][:M])
                h = oracle.swiglu(gu_bits)
                assert np.array_equal(bf16_bits(dn_s["act"][:M]), h), (M, layer)
                y, S = oracle.gemm(h, dc, ds, dt)
                check(dn_s["out"][:M], y, S, bf16=True, what="down M=%d" % M)
                # the same steps as separate calls
                g_ref = torch.empty((M, 2 * F), dtype=torch.bfloat16, device="cuda")
                nv.Gemm(M, K, 2 * F, nv.OUT_BF16)(mats[2 * layer], gu_s["act"][:M], g_ref)
                h_ref = torch.empty((M, F), dtype=torch.bfloat16, device="cuda")
                nv.nvfp4_swiglu(g_ref, M, F, h_ref)
                d_ref = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
                nv.Gemm(M, F, K, nv.OUT_BF16)(mats[2 * layer + 1], h_ref, d_ref)
                torch.cuda.synchronize()
                assert np.array_equal(bf16_bits(gu_s["out"][:M]), bf16_bits(g_ref)), (M, layer)
                assert np.array_equal(bf16_bits(dn_s["act"][:M]), bf16_bits(h_ref)), (M, layer)
                assert np.array_equal(bf16_bits(dn_s["out"][:M]), bf16_bits(d_ref)), (M, layer)
    finally:
        nv.nvfp4_round_destroy(plan)
