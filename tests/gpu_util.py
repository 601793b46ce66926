"""Helpers shared by the GPU tests (not a test module).

The GPU tests fail -- they never skip -- when no GPU or no built library is
present: a GPU profile that silently skips would hide a broken build.
"""
from __future__ import annotations

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle  # noqa: E402  (the acceptance bounds)


def require_gpu():
    import torch
    import nvfp4_weight_streaming_amd as nv
    assert torch.cuda.is_available(), "no GPU visible: the gpu tests fail rather than skip"
    assert os.path.exists(nv.LIB_PATH), "libnvfp4.so is not built"
    nv.lib()
    return nv


def dev(a: np.ndarray):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits: np.ndarray):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda()
    return t.view(torch.bfloat16)


def host(t) -> np.ndarray:
    import torch
    if t.dtype == torch.bfloat16:
        return t.float().cpu().numpy().astype(np.float64)
    return t.cpu().numpy()


def bf16_bits(t) -> np.ndarray:
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def pack(nv, codes_dev, scales_dev, K, N, t):
    return nv.PackedWeight.from_canonical(codes_dev, scales_dev, t, K, N)


# Elements of a canary region placed right after an output buffer, and the
# bit patterns it holds (quiet NaNs no kernel writes): a store past the end of
# [M][N] (a ragged tile, a wrong row stride) changes them.
CANARY_ELEMS = 4096
_CANARY = {2: 0x7FA5, 4: 0x7FA5A5A5}


def canary_out(M, N, dtype):
    """An [M][N] output tensor (NaN-poisoned) followed in memory by a canary
    region.  Returns (out, assert_canary) where assert_canary(what) checks
    that the region is untouched."""
    import torch
    n = M * N
    buf = torch.empty(n + CANARY_ELEMS, dtype=dtype, device="cuda")
    buf[:n].fill_(float("nan"))
    ity = torch.int16 if buf.element_size() == 2 else torch.int32
    pattern = _CANARY[buf.element_size()]
    buf.view(ity)[n:] = pattern

    def assert_canary(what=""):
        tail = buf.view(ity)[n:]
        bad = int((tail != pattern).sum().item())
        assert bad == 0, "%s: %d canary elements after the output were overwritten" % (what, bad)

    return buf[:n].view(M, N), assert_canary


def run(nv, pw, act_dev, out_dtype, M=None, split_k=0, waves=0, chunks=0, max_M=None,
        windows=0, verify_waves=0, verify_windows=0, tile_max_m=0, tile_superblocks=0,
        verify_ranges=0, prefill_schedule=0):
    import torch
    M = act_dev.shape[0] if M is None else M
    g = nv.Gemm(max_M or M, pw.K, pw.N, out_dtype, split_k=split_k, waves=waves, chunks=chunks,
                windows=windows, verify_waves=verify_waves, verify_windows=verify_windows,
                tile_max_m=tile_max_m, tile_superblocks=tile_superblocks,
                verify_ranges=verify_ranges, prefill_schedule=prefill_schedule)
    dt = torch.float32 if out_dtype == nv.OUT_F32 else torch.bfloat16
    out, assert_canary = canary_out(M, pw.N, dt)
    g(pw, act_dev, out, M=M)
    torch.cuda.synchronize()
    assert_canary("M=%d K=%d N=%d" % (M, pw.K, pw.N))
    return out, g


def check(out, y, S, bf16: bool, what=""):
    """Element-wise acceptance: |out - y| <= 2^-16 S (fp32 outputs), plus the
    final bf16 rounding allowance for bf16 outputs."""
    o = host(out).astype(np.float64)
    assert o.shape == y.shape, (o.shape, y.shape)
    assert np.all(np.isfinite(o)), "non-finite output %s" % what
    err = np.abs(o - y)
    tol = oracle.tolerance_bf16(y, S) if bf16 else oracle.tolerance(S)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d outside bound; first %s out=%r y=%r S=%r" % (
            what, int(bad.sum()), bad.size, tuple(i), o[tuple(i)], y[tuple(i)], S[tuple(i)]))
    return float(np.max(err / np.maximum(S, 1e-300)))


def quarter_cols(N, seed):
    """A random column in every 64-column quarter of each 256-column block:
    with every row, that samples every wave's outputs of every tile (a wave
    owns one quarter of a tile's columns), the shared tiles' included."""
    rng = np.random.default_rng(seed)
    cols = {q + int(rng.integers(0, min(64, N - q))) for q in range(0, N, 64)}
    return np.array(sorted(cols | {0, N - 1}))


def half_block_rows(M, seed):
    """Two random rows of every 256-row block, one in each half (a wave owns
    one half of a tile's rows), plus the first and last rows."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1}
    for b in range(0, M, 256):
        for h in (0, 128):
            lo = b + h
            if lo < M:
                rows.add(lo + int(rng.integers(0, min(128, M - lo))))
    return np.array(sorted(rows))
