"""GPU parity of the top-k over the vocabulary (the step after the output
head): indices equal and values bit-identical to the oracle, on random and
tie-heavy logits, one and several levels, strided rows, and the output head's
own logits computed by the oracle."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import dev, host, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


def _run(nv, x, k, ld=None):
    import torch
    M, V = x.shape
    if ld is None or ld == V:
        d = dev(x)
    else:
        pad = np.full((M, ld), np.nan, np.float32)  # past V: never read
        pad[:, :V] = x
        d = dev(pad)
    idx = torch.full((M, k), -7, dtype=torch.int32, device="cuda")
    val = torch.full((M, k), float("nan"), dtype=torch.float32, device="cuda")
    wsb = nv.nvfp4_topk_workspace_bytes(M, V, k)
    ws = torch.full((max(wsb, 16),), 0xA5, dtype=torch.uint8, device="cuda")
    nv.nvfp4_topk(d, M, V, ld or V, k, idx, val, ws if wsb else None, wsb)
    torch.cuda.synchronize()
    return host(idx), host(val)


def _check(x, k, got_idx, got_val, what):
    want_idx, want_val = oracle.topk(x, k)
    assert np.array_equal(got_idx, want_idx), (what, np.argwhere(got_idx != want_idx)[:3])
    assert np.array_equal(got_val.view(np.uint32), want_val.view(np.uint32)), what


# (M, V, k): one level (V <= 4096), two levels, three levels (many chunks x
# large k), the pages' vocabulary size class, ragged chunk tails.
SHAPES = [(1, 1, 1), (3, 7, 7), (2, 4096, 64), (5, 4097, 8), (4, 9000, 3), (8, 152064, 1),
          (8, 152064, 8), (8, 152064, 64), (64, 152064, 7), (7, 248320, 7), (2, 300000, 64)]


@pytest.mark.parametrize("M,V,k", SHAPES)
@pytest.mark.parametrize("ties", [False, True])
def test_topk_matches_oracle(nv, M, V, k, ties):
    x = synth.logits(3, M * 7 + V % 97 + k, M, V, ties=ties)
    got_idx, got_val = _run(nv, x, k)
    _check(x, k, got_idx, got_val, "topk %r ties=%s" % ((M, V, k), ties))


@pytest.mark.parametrize("M,V,k", [(2, 262144, 8), (2, 262145, 8), (3, 65536, 2)])
def test_topk_run_merge_bounds(nv, M, V, k):
    """After the first level, k <= 8 rows of at most 256 candidate runs are
    merged by one wave (4 runs per lane): exactly 256 runs, 257 (the level
    path), and a small k."""
    x = synth.logits(5, V + k, M, V, ties=True)
    got_idx, got_val = _run(nv, x, k)
    _check(x, k, got_idx, got_val, "merge bounds %r" % ((M, V, k),))


@pytest.mark.parametrize("k", [1, 5, 8])
def test_topk_all_winners_in_one_run(nv, k):
    """The k largest logits all in one 1024-entry unit (one candidate run
    supplies every output, so it is exhausted), with an equal-valued pair
    across two units for the last place."""
    M, V = 3, 152064
    x = synth.logits(6, 77 + k, M, V)
    for m in range(M):
        x[m, 5000:5000 + k] = 1000.0 + np.arange(k, dtype=np.float32)[::-1] * (m + 1)
        x[m, 90000] = x[m, 5000 + k - 1]  # ties with the k-th value, larger index
    got_idx, got_val = _run(nv, x, k)
    _check(x, k, got_idx, got_val, "one run k=%d" % k)


@pytest.mark.parametrize("M,V,ld,k", [(3, 5000, 5008, 5), (2, 100, 131, 64), (2, 64, 64, 64)])
def test_topk_strided_rows(nv, M, V, ld, k):
    x = synth.logits(4, V + ld, M, V, ties=True)
    got_idx, got_val = _run(nv, x, k, ld=ld)
    _check(x, k, got_idx, got_val, "strided %r" % ((M, V, ld, k),))


def test_topk_of_head_logits(nv):
    """The output head's logits (M = 8, K = 5120, a 20000-entry slice of the
    vocabulary), computed by the oracle GEMM and rounded to fp32, then the
    top-8 and the argmax."""
    K, N, M = 5120, 20000, 8
    W = synth.weights(0, 500, N, K)
    codes, scales, t = oracle.quantize(W)
    act = synth.activations(0, 500, M, K)
    y, _ = oracle.gemm(act, codes, scales, t)
    x = y.astype(np.float32)
    for k in (1, 8):
        got_idx, got_val = _run(nv, x, k)
        _check(x, k, got_idx, got_val, "head logits k=%d" % k)
