"""NVFP4 oracle: plain CPU reference of the decode GEMM (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The HIP library never calls it and
shares no code with it.

It implements, on the CPU and in fp64 where the format allows exactness:

* decoders for the element types of the NVFP4 body format ("Models and
  artifacts", section "The artifact": 4-bit floating point with one scale per
  16 values) -- OCP MX FP4 E2M1 elements, OCP E4M3 (FN) block scales, bf16
  activations;
* the quantiser of the synthetic workload (tensor scale amax/(6*448), E4M3
  block scales with round-to-nearest-even and saturation, E2M1 values with
  round-to-nearest-even);
* the GEMM of the decode round ("Ignis" README, "The decode round": one pass
  over the weights serves all lanes): ``y[m][n] = sum_k a[m][k] * w[n][k]``
  with exact fp64 products, ascending-k fp64 sums, and ``S = sum |a*w|``.

* the SwiGLU step between gate_up and down (a reading of the shapes: the
  fused gate_up matrix has N = 2 x the down matrix's K): for bf16 [gate | up]
  halves, silu(g) * u = g * u / (1 + exp(-g)) in fp64, rounded once to bf16
  (nearest, ties to even);
* the top-k of the output head's logits ("Ignis" README, "Speculative
  decoding (DFlash2)": the drafter's top-k over the vocabulary, replaced by a
  row-split kernel with an identical answer): per row, the k largest values in
  descending order, equal values in ascending index order (IEEE comparison,
  so -0.0 and +0.0 are equal).

Every function here is pinned by ``tests/test_oracle_pins.py`` against tables,
library routines, closed forms and exact rational brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "nvfp4_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_lib = None


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (no HIP headers, no GPU code)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(
            ["gcc", "-O2", "-fPIC", "-shared", "-std=c11", "-ffp-contract=off",
             "-o", tmp, _SRC, "-lm", "-lpthread"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        lib = ctypes.CDLL(_LIB)
        c = ctypes
        u8p = c.POINTER(c.c_uint8)
        f32p = c.POINTER(c.c_float)
        f64p = c.POINTER(c.c_double)
        u16p = c.POINTER(c.c_uint16)
        lib.oracle_e2m1_value.argtypes = [c.c_int]
        lib.oracle_e2m1_value.restype = c.c_double
        lib.oracle_e4m3_value.argtypes = [c.c_int]
        lib.oracle_e4m3_value.restype = c.c_double
        lib.oracle_bf16_value.argtypes = [c.c_uint16]
        lib.oracle_bf16_value.restype = c.c_double
        lib.oracle_e4m3_encode.argtypes = [c.c_float]
        lib.oracle_e4m3_encode.restype = c.c_int
        lib.oracle_e2m1_encode.argtypes = [c.c_float]
        lib.oracle_e2m1_encode.restype = c.c_int
        lib.oracle_tensor_scale.argtypes = [f32p, c.c_size_t]
        lib.oracle_tensor_scale.restype = c.c_float
        lib.oracle_quantize_rows.argtypes = [f32p, c.c_int, c.c_int, c.c_int, c.c_float, u8p, u8p]
        lib.oracle_quantize_rows.restype = None
        lib.oracle_quantize.argtypes = [f32p, c.c_int, c.c_int, u8p, u8p]
        lib.oracle_quantize.restype = c.c_float
        lib.oracle_gemm.argtypes = [c.c_int, c.c_int, c.c_int, u8p, u8p, c.c_float, u16p,
                                    f64p, f64p, c.c_int]
        lib.oracle_gemm.restype = c.c_int
        _lib = lib
    return _lib


def _ptr(a: np.ndarray, ctype):
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(ctypes.POINTER(ctype))


# ---- element codecs ---------------------------------------------------------

def e2m1_value(code: int) -> float:
    return _load().oracle_e2m1_value(int(code))


def e4m3_value(byte: int) -> float:
    return _load().oracle_e4m3_value(int(byte))


def bf16_value(bits: int) -> float:
    return _load().oracle_bf16_value(int(bits))


def e4m3_encode(x: float) -> int:
    return _load().oracle_e4m3_encode(float(x))


def e2m1_encode(x: float) -> int:
    return _load().oracle_e2m1_encode(float(x))


# ---- quantiser --------------------------------------------------------------

def tensor_scale(w: np.ndarray) -> float:
    w = np.ascontiguousarray(w, dtype=np.float32)
    return float(_load().oracle_tensor_scale(_ptr(w, ctypes.c_float), w.size))


def quantize(w: np.ndarray):
    """Quantise an fp32 [N][K] matrix.  Returns (codes u8[N][K/2],
    scales u8[N][K/16], tensor_scale float)."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    assert K % 16 == 0
    codes = np.zeros((N, K // 2), np.uint8)
    scales = np.zeros((N, K // 16), np.uint8)
    t = _load().oracle_quantize(_ptr(w, ctypes.c_float), N, K, _ptr(codes, ctypes.c_uint8),
                                _ptr(scales, ctypes.c_uint8))
    return codes, scales, float(t)


def quantize_rows(w_rows: np.ndarray, t: float):
    """Quantise some rows of a matrix whose tensor scale ``t`` is already known."""
    w_rows = np.ascontiguousarray(w_rows, dtype=np.float32)
    R, K = w_rows.shape
    codes = np.zeros((R, K // 2), np.uint8)
    scales = np.zeros((R, K // 16), np.uint8)
    _load().oracle_quantize_rows(_ptr(w_rows, ctypes.c_float), K, 0, R, ctypes.c_float(t),
                                 _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8))
    return codes, scales


# ---- GEMM -------------------------------------------------------------------

def gemm(act_bits: np.ndarray, codes: np.ndarray, scales: np.ndarray, t: float,
         threads: int | None = None):
    """y[m][n] and S[m][n] in fp64 for bf16 activations ``act_bits`` (uint16
    [M][K]) and canonical planes of an [N][K] weight matrix."""
    act_bits = np.ascontiguousarray(act_bits, dtype=np.uint16)
    codes = np.ascontiguousarray(codes, dtype=np.uint8)
    scales = np.ascontiguousarray(scales, dtype=np.uint8)
    M, K = act_bits.shape
    N = codes.shape[0]
    assert codes.shape == (N, K // 2) and scales.shape == (N, K // 16)
    y = np.zeros((M, N), np.float64)
    S = np.zeros((M, N), np.float64)
    if threads is None:
        threads = os.cpu_count() or 1
    _load().oracle_gemm(M, K, N, _ptr(codes, ctypes.c_uint8), _ptr(scales, ctypes.c_uint8),
                        ctypes.c_float(t), _ptr(act_bits, ctypes.c_uint16),
                        _ptr(y, ctypes.c_double), _ptr(S, ctypes.c_double), int(threads))
    return y, S


def dequantize(codes: np.ndarray, scales: np.ndarray, t: float) -> np.ndarray:
    """The dequantised matrix, element by element, in fp64:
    w[n][k] = E2M1(code of k) * E4M3(scale of block k // 16) * t, with the code
    of k in the low nibble of byte k // 2 for even k and in the high nibble
    for odd k ("Models and artifacts", "The artifact": 4-bit values with one
    scale per 16).  Exact: at most 2 + 4 + 24 significant bits."""
    N = codes.shape[0]
    K = codes.shape[1] * 2
    lib = _load()
    e2 = np.array([lib.oracle_e2m1_value(c) for c in range(16)])
    e4 = np.array([lib.oracle_e4m3_value(b) for b in range(256)])
    lo = codes & 15
    hi = codes >> 4
    c = np.empty((N, K), np.int64)
    c[:, 0::2] = lo
    c[:, 1::2] = hi
    s = np.repeat(scales.astype(np.int64), 16, axis=1)
    return e2[c] * e4[s] * float(t)


def tolerance(S: np.ndarray) -> np.ndarray:
    """Per-element acceptance bound for fp32 outputs: 2^-16 * sum|a*w|."""
    return np.ldexp(S, -16)


def tolerance_bf16(y: np.ndarray, S: np.ndarray) -> np.ndarray:
    """Bound for outputs stored as bf16: the fp32 bound before the final
    rounding plus half a bf16 ulp of the (bounded) value.  bf16 has 8
    significant bits, so its round-to-nearest store moves a value by at most
    2^-8 of its magnitude (at the bottom of a binade)."""
    tol = np.ldexp(S, -16)
    return tol + np.ldexp(np.abs(y) + tol, -8)


def topk(logits: np.ndarray, k: int):
    """Top-k of each row of a float32 [M][V] array: (indices int32 [M][k],
    values float32 [M][k]), values descending, ties by ascending index.  The
    values are the input elements themselves (bit for bit)."""
    x = np.ascontiguousarray(logits, dtype=np.float32)
    M, V = x.shape
    assert 1 <= k <= V
    idx = np.empty((M, k), np.int32)
    for m in range(M):
        # lexsort's last key is the primary one: descending value, then index
        order = np.lexsort((np.arange(V), -x[m].astype(np.float64)))
        idx[m] = order[:k]
    vals = np.take_along_axis(x, idx.astype(np.int64), axis=1)
    return idx, vals


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float64 -> bf16 bits (uint16), rounded once to nearest, ties to even
    (no intermediate float32).  Overflow goes to infinity; NaN stays NaN."""
    x = np.asarray(x, np.float64)
    bits = x.view(np.uint64)
    sign = (bits >> np.uint64(63)).astype(np.uint16) << np.uint16(15)
    a = np.abs(x)
    out = np.zeros(x.shape, np.uint16)
    for i, (v, sg) in enumerate(zip(a.ravel(), sign.ravel())):
        if np.isnan(v):
            out.flat[i] = 0x7FC0
            continue
        if v == 0:
            out.flat[i] = sg
            continue
        # the two bf16 magnitudes around v, by exhaustive comparison of the
        # neighbouring exponents' grids: bf16 has 8 significant bits
        e = int(np.frexp(v)[1]) - 1  # v = m 2^e, 1 <= m < 2, exactly
        lo_e = max(e, -126)
        step = 2.0 ** (lo_e - 7)           # spacing of the 8-bit significand grid
        q = np.floor(v / step)
        lo, hi = q * step, (q + 1) * step
        if v - lo < hi - v:
            r = lo
        elif v - lo > hi - v:
            r = hi
        else:  # tie: the even significand
            r = lo if int(q) % 2 == 0 else hi
        r32 = np.float32(r) if r < 2.0 ** 128 else np.float32(np.inf)  # 2^128: overflow
        out.flat[i] = sg | (int(r32.view(np.uint32)) >> 16)
    return out


def swiglu(gate_up_bits: np.ndarray) -> np.ndarray:
    """bf16 bits [M][2F] -> bf16 bits [M][F]: silu(g) * u in fp64, g = first
    half, u = second half, rounded once to bf16."""
    gu = np.ascontiguousarray(gate_up_bits, dtype=np.uint16)
    M, F2 = gu.shape
    F = F2 // 2
    x = (gu.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    g, u = x[:, :F], x[:, F:]
    with np.errstate(over="ignore"):
        y = g * u / (1.0 + np.exp(-g))
    return bf16_round(y)
