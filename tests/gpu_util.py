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


def run(nv, pw, act_dev, out_dtype, M=None, split_k=0, waves=0, chunks=0, kernel=0, tiles=0,
        max_M=None, windows=0, verify_waves=0, verify_windows=0):
    import torch
    M = act_dev.shape[0] if M is None else M
    g = nv.Gemm(max_M or M, pw.K, pw.N, out_dtype, split_k=split_k, waves=waves, chunks=chunks,
                kernel=kernel, tiles=tiles, windows=windows, verify_waves=verify_waves,
                verify_windows=verify_windows)
    dt = torch.float32 if out_dtype == nv.OUT_F32 else torch.bfloat16
    out = torch.full((M, pw.N), float("nan"), dtype=dt, device="cuda")  # poison
    g(pw, act_dev, out, M=M)
    torch.cuda.synchronize()
    return out, g


def check(out, y, S, bf16: bool, what=""):
    """Element-wise acceptance: |out - y| <= 2^-16 S (fp32 outputs), plus the
    final bf16 rounding allowance for bf16 outputs."""
    o = host(out).astype(np.float64)
    assert o.shape == y.shape, (o.shape, y.shape)
    assert np.all(np.isfinite(o)), "non-finite output %s" % what
    err = np.abs(o - y)
    tol = np.ldexp(S, -16)
    if bf16:
        tol = tol + np.ldexp(np.abs(y) + tol, -8)
    bad = err > tol
    if bad.any():
        i = np.argwhere(bad)[0]
        raise AssertionError("%s: %d of %d outside bound; first %s out=%r y=%r S=%r" % (
            what, int(bad.sum()), bad.size, tuple(i), o[tuple(i)], y[tuple(i)], S[tuple(i)]))
    return float(np.max(err / np.maximum(S, 1e-300)))
