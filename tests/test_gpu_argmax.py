"""The output head's run with its argmax fused (nvfp4_gemm_run_argmax).

The logits must be bit-identical to a plain run of the same plan, and the
indices must equal both the host argmax of those logits (equal values to the
smaller column, -0.0 equal to +0.0) and the top-k kernel's k = 1 answer.
Shapes cover a K split (the last contributor of a group writes it), no split
(each workgroup writes its group), a single column, groups on only some XCDs
and a matrix wide enough for no split; ties are planted across groups of
different XCDs.  The area starts with arbitrary content."""
import numpy as np
import pytest

import synth
from tests.gpu_util import dev, dev_bf16, host, pack, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _host_argmax(logits):
    x = np.array(logits, dtype=np.float32)
    x[x == 0] = 0.0  # -0 and +0 compare equal; argmax takes the first maximum
    return np.argmax(x, axis=1).astype(np.int32)


def _run_both(nv, pw, act, M, K, N, reps=3):
    """Plain logits, then `reps` fused runs; returns (plain, fused logits, indices)."""
    import torch
    # (the decode kernel for every M, as the fused run: the narrow-width kernel
    # that a plain run may take for M <= 4 adds its sums in another order)
    g = nv.Gemm(8, K, N, nv.OUT_F32, tile_max_m=-1)
    plain = torch.full((M, N), float("nan"), device="cuda")
    g(pw, act[:M], plain, M=M)
    ab = nv.nvfp4_gemm_argmax_area_bytes(g.plan)
    # any content: the area starts as garbage (a previous run's keys of other data)
    area = torch.randint(0, 256, (ab,), dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(reps):
        logits = torch.full((M, N), float("nan"), device="cuda")
        idx = torch.full((M,), -7, dtype=torch.int32, device="cuda")
        nv.nvfp4_gemm_run_argmax(g.plan, M, K, N, pw.codes, pw.scales, pw.tensor_scale, act,
                                 logits, idx, g.workspace, area, ab)
        torch.cuda.synchronize()
        outs.append((host(logits), host(idx)))
    return host(plain), outs


SHAPES = [(8, 5120, 19008), (3, 5120, 7168), (8, 1040, 4099), (1, 16, 1), (5, 2576, 65563),
          (7, 512, 40)]


@pytest.mark.parametrize("M,K,N", SHAPES)
def test_argmax_run_matches_plain_run_and_topk(nv, M, K, N):
    import torch
    codes, scales = synth.random_planes(M + 11, N + K, N, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, 1.5e-3)
    act = dev_bf16(synth.activations(M + 12, K + N, M, K))
    plain, outs = _run_both(nv, pw, act, M, K, N)
    want = _host_argmax(plain)
    top_idx, _ = nv.topk(torch.from_numpy(plain).cuda(), 1)
    assert np.array_equal(host(top_idx)[:, 0], want)
    for logits, idx in outs:
        assert np.array_equal(logits.view(np.uint32), plain.view(np.uint32))
        assert np.array_equal(idx, want), (idx, want)


@pytest.mark.parametrize("M,K,N", [(8, 5120, 19008), (4, 2576, 65563)])
def test_argmax_run_ties_go_to_the_smaller_column(nv, M, K, N):
    """The largest column copied to columns of groups on other XCDs (and to a
    smaller column), so the maximum is tied across workgroups: the smallest of
    the copies must win in every run."""
    codes, scales = synth.random_planes(M + 21, N + 2 * K, N, K)
    scales = scales.copy()
    codes = codes.copy()
    hot = N - 5
    codes[hot] = 0x77  # every code +6 and the largest E4M3 scale: with non-negative
    scales[hot] = 0x7E  # activations this column's logits are each row's maximum
    copies = [N // 2 + 17, 64 * 3 + 1, 64 * 5 + 9]  # different 4-tile groups and XCDs
    for c in copies:
        codes[c] = codes[hot]
        scales[c] = scales[hot]
    pw = pack(nv, dev(codes), dev(scales), K, N, 1.0e-3)
    # one positive activation row pattern shared by every row: the same column wins each row
    act_bits = synth.activations(M + 22, K, 1, K)
    act_bits = act_bits & np.uint16(0x7FFF)  # sign bits cleared: every value >= 0
    act = dev_bf16(np.repeat(act_bits, M, axis=0))
    plain, outs = _run_both(nv, pw, act, M, K, N)
    want = _host_argmax(plain)
    assert (want == min(copies)).all(), want
    for logits, idx in outs:
        assert np.array_equal(logits.view(np.uint32), plain.view(np.uint32))
        assert np.array_equal(idx, want)


def test_argmax_run_all_equal_logits(nv):
    """Zero scales: every logit is +0 (tensor scale > 0) or -0 (< 0), all equal,
    so column 0 wins."""
    M, K, N = 8, 1024, 9000
    codes, _ = synth.random_planes(3, 4, N, K)
    scales = np.zeros((N, K // 16), dtype=np.uint8)
    for t in (2.0e-3, -2.0e-3):
        pw = pack(nv, dev(codes), dev(scales), K, N, t)
        act = dev_bf16(synth.activations(5, 6, M, K))
        plain, outs = _run_both(nv, pw, act, M, K, N, reps=2)
        assert (plain == 0).all()
        for logits, idx in outs:
            assert np.array_equal(logits.view(np.uint32), plain.view(np.uint32))
            assert (idx == 0).all(), idx
