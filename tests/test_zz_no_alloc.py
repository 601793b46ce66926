"""GPU test of nvfp4_gemm_run_noalloc, the GEMM run without a workspace
argument for callers that cannot allocate: called through the C ABI, its
outputs equal those of nvfp4_gemm_run with a workspace (the same kernels) bit
for bit and match the oracle, on calls in a row whose split-K state shares
the one static scratch (a large decode, a verify width, then a smaller
decode); canaries after the outputs stay untouched.  A run that needs more
split-K state than the scratch holds is refused before anything runs."""
import ctypes

import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import bf16_bits, canary_out, check, dev, dev_bf16, host, pack, require_gpu

pytestmark = pytest.mark.gpu


def _noalloc(nv, plan, M, pw, act, out):
    import torch
    L = nv.lib()
    return L.nvfp4_gemm_run_noalloc(plan, M, pw.K, pw.N, pw.codes.data_ptr(),
                                    pw.scales.data_ptr(), ctypes.c_float(pw.tensor_scale),
                                    act.data_ptr(), out.data_ptr(),
                                    torch.cuda.current_stream().cuda_stream)


# (max_M, M, K, N, out dtype): split-K decode, a verify width, a smaller
# split-K decode (tile kernel off so the scratch is used).
CALLS = [(8, 8, 5120, 7168, 0), (64, 40, 6144, 1000, 1), (8, 6, 2048, 300, 1)]


def test_noalloc_equals_workspace_run_on_calls_in_a_row():
    import torch
    nv = require_gpu()
    for i, (max_M, M, K, N, dt) in enumerate(CALLS):
        codes, scales = synth.random_planes(70 + i, 71 + i, N, K)
        t = float(np.float32(np.random.default_rng(i).uniform(1e-4, 1e-2)))
        act = synth.activations(72 + i, 73 + i, M, K)
        pw = pack(nv, dev(codes), dev(scales), K, N, t)
        g = nv.Gemm(max_M, K, N, dt, tile_max_m=-1)
        assert g.ws_bytes > 0  # the workspace run needs split-K state
        torch_dt = torch.float32 if dt == nv.OUT_F32 else torch.bfloat16
        ref, ref_canary = canary_out(M, N, torch_dt)
        a = dev_bf16(act)
        g(pw, a, ref, M=M)
        got, got_canary = canary_out(M, N, torch_dt)
        st = _noalloc(nv, g.plan, M, pw, a, got)
        assert st == nv.OK, (st, nv.last_error())
        torch.cuda.synchronize()
        ref_canary("workspace run %d" % i)
        got_canary("noalloc run %d" % i)
        bits = (lambda x: host(x).view(np.uint32)) if dt == nv.OUT_F32 else bf16_bits
        assert np.array_equal(bits(got), bits(ref)), "call %d: noalloc differs from the workspace run" % i
        y, S = oracle.gemm(act, codes, scales, t)
        check(got, y, S, bf16=dt == nv.OUT_BF16, what="noalloc call %d" % i)


def test_noalloc_refuses_a_run_beyond_the_scratch():
    import torch
    nv = require_gpu()
    M, K, N = 2048, 5120, 17408  # prefill chunk: tens of MB of K-piece partial sums
    g = nv.Gemm(M, K, N, nv.OUT_BF16)
    pw = nv.PackedWeight(torch.zeros(nv.nvfp4_packed_code_bytes(K, N), dtype=torch.uint8,
                                     device="cuda"),
                         torch.zeros(nv.nvfp4_packed_scale_bytes(K, N), dtype=torch.uint8,
                                     device="cuda"), 1.0, K, N)
    a = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    st = _noalloc(nv, g.plan, M, pw, a, out)
    torch.cuda.synchronize()
    assert st == nv.EUNSUPPORTED, (st, nv.last_error())
    assert "static scratch" in nv.last_error(), nv.last_error()
    assert torch.isnan(out).all().item()  # nothing ran
