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
from tests.gpu_util import (bf16_bits, canary_out, check, dev, dev_bf16, half_block_rows, host,
                             pack, quarter_cols, require_gpu)

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


def test_noalloc_prefill_default_plan_falls_back_to_pieces():
    """o at M = 2048 (K = 6144, N = 5120: 160 tiles on 256 compute units): a
    default plan runs it with stream-K, whose slots do not fit the static
    scratch, so the no-allocation call runs whole tiles (no K split there):
    bit-identical to a workspace run of a pieces plan, and within the bound
    of the oracle on rows and columns that reach every wave of every tile."""
    import torch
    nv = require_gpu()
    M, K, N = 2048, 6144, 5120
    codes, scales = synth.random_planes(91, 92, N, K)
    t = 3.0e-3
    act = synth.activations(93, 94, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    a = dev_bf16(act)
    g = nv.Gemm(M, K, N, nv.OUT_BF16)
    gp = nv.Gemm(M, K, N, nv.OUT_BF16, prefill_schedule=nv.PREFILL_PIECES)
    ref, ref_canary = canary_out(M, N, torch.bfloat16)
    gp(pw, a, ref)
    got, got_canary = canary_out(M, N, torch.bfloat16)
    st = _noalloc(nv, g.plan, M, pw, a, got)
    assert st == nv.OK, (st, nv.last_error())
    torch.cuda.synchronize()
    ref_canary("pieces workspace run")
    got_canary("noalloc run")
    assert np.array_equal(bf16_bits(got), bf16_bits(ref))
    rows, cols = half_block_rows(M, 5), quarter_cols(N, 6)
    y, S = oracle.gemm(act[rows], codes[cols], scales[cols], t)
    sub = got[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
    check(sub, y, S, bf16=True, what="noalloc prefill fallback")


_CAPTURE_CHILD = r'''
import ctypes, sys
sys.path.insert(0, sys.argv[1])
import numpy as np
import torch
import nvfp4_weight_streaming_amd as nv
import synth
from tests.gpu_util import dev, dev_bf16, host, pack

M, K, N = 8, 2048, 300
codes, scales = synth.random_planes(91, 92, N, K)
pw = pack(nv, dev(codes), dev(scales), K, N, 0.003)
act = dev_bf16(synth.activations(93, 94, M, K))
g = nv.Gemm(8, K, N, nv.OUT_F32, tile_max_m=-1)
L = nv.lib()
side = torch.cuda.Stream()


def call(out, stream):
    return L.nvfp4_gemm_run_noalloc(g.plan, M, K, N, pw.codes.data_ptr(), pw.scales.data_ptr(),
                                    ctypes.c_float(pw.tensor_scale), act.data_ptr(),
                                    out.data_ptr(), stream.cuda_stream)


def nan_out():
    return torch.full((M, N), float("nan"), dtype=torch.float32, device="cuda")


torch.cuda.synchronize()
# 1. The first call on the device, under capture: refused, nothing recorded.
first = nan_out()
graph0 = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph0, stream=side):
    first.zero_()
    st = call(first, side)
print("first call under capture:", st, nv.last_error(), flush=True)
assert st == nv.ESTATE and "capture" in nv.last_error(), (st, nv.last_error())
# 2. An eager call sets the scratch up.
ref = nan_out()
st = call(ref, torch.cuda.current_stream())
assert st == nv.OK, (st, nv.last_error())
torch.cuda.synchronize()
assert not torch.isnan(ref).any().item()
# 3. Later calls may be captured: every replay equals the eager result bit for
# bit, with eager calls on the same scratch between the replays.
got = nan_out()
graph = torch.cuda.CUDAGraph()
with torch.cuda.graph(graph, stream=side):
    st = call(got, side)
assert st == nv.OK, (st, nv.last_error())
for r in range(3):
    got.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    assert np.array_equal(host(got).view(np.uint32), host(ref).view(np.uint32)), r
    between = nan_out()
    assert call(between, torch.cuda.current_stream()) == nv.OK
    torch.cuda.synchronize()
    assert np.array_equal(host(between).view(np.uint32), host(ref).view(np.uint32)), r
print("ok", flush=True)
'''


def test_noalloc_first_call_under_capture_is_refused_and_later_captures_replay():
    """In a fresh process (the scratch not yet set up on the device): a first
    call made under stream capture is refused (its clearing of the scratch
    would only be recorded); after one eager call, captured calls replay
    bit-identically to eager ones."""
    import os
    import subprocess
    import sys
    require_gpu()
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, "-c", _CAPTURE_CHILD, root], cwd=root,
                       capture_output=True, text=True, timeout=240)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout[-2000:], r.stderr[-3000:])
