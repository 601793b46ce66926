"""What re-quantising NVFP4 weights to the gfx950 scaled-MFMA FP4 format would
cost (CPU only; no kernel is built on it).

The artifact's body format is 4-bit floating point with a scale per 16 values
("Models and artifacts", "The artifact"); here that scale is E4M3, so a block
scale has mantissa bits.  gfx950's scaled FP4 MFMA takes OCP MX FP4 operands
instead: E2M1 elements with one E8M0 (power of two) scale per 32 values.
Using it for the weights means re-quantising every NVFP4 block pair into one
MX block.  These tests measure, against the oracle, how far the result of a
GEMM moves when that is done to the synthetic workload's weights:

* the MX quantiser follows OCP MX v1.0: X = 2^(floor(log2(amax)) - 2), the
  largest power of two of E2M1 being 2^2; elements round to nearest, ties to
  the even code, saturating at 6 (its E2M1 rounding is pinned against the
  oracle's encoder);
* it is applied to the exactly dequantised NVFP4 weights (the artifact's
  weights are NVFP4, not the fp32 originals), the tensor scale kept aside.

Run with -s to print the figures quoted in the design notes."""
import numpy as np
import pytest

import synth

E2M1_MAG = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_rne_magnitude(x):
    """|x| rounded to the nearest E2M1 magnitude, ties to the even code,
    saturating at 6 (vectorised)."""
    a = np.minimum(np.abs(x), 6.0)
    idx = np.searchsorted(E2M1_MAG, a)  # first magnitude >= a
    idx = np.clip(idx, 1, 7)
    lo, hi = E2M1_MAG[idx - 1], E2M1_MAG[idx]
    d_lo, d_hi = a - lo, hi - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (idx % 2 == 0))
    return np.where(take_hi, hi, lo)


def mx_fp4_requantize(w):
    """OCP MX FP4 (E2M1 elements, one E8M0 scale per 32 values along the last
    axis) quantisation of w; returns the dequantised values."""
    N, K = w.shape
    b = w.reshape(N, K // 32, 32)
    amax = np.abs(b).max(axis=2, keepdims=True)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2.0
    scale = np.where(amax > 0, np.exp2(e), 1.0)
    q = np.sign(b) * e2m1_rne_magnitude(b / scale)
    return (q * scale).reshape(N, K)


def test_e2m1_rounding_matches_the_oracle_encoder(oracle_mod):
    rng = np.random.default_rng(5)
    xs = np.concatenate([rng.uniform(-7, 7, 3000),
                         [0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0, 6.5, -0.25, -5.0, 0.0]])
    got = e2m1_rne_magnitude(xs)
    for x, g in zip(xs, got):
        c = oracle_mod.e2m1_encode(float(np.float32(x)))
        assert abs(oracle_mod.e2m1_value(c)) == g, (x, g, c)


def _requant_case(oracle_mod, N=64, K=5120, M=8, seed=3):
    W = synth.weights(seed, 77, N, K)
    codes, scales, t = oracle_mod.quantize(W)
    w_nv = oracle_mod.dequantize(codes, scales, 1.0)  # without the tensor scale
    w_mx = mx_fp4_requantize(w_nv)
    act = synth.activations(seed, 78, M, K)
    a = (act.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    y_nv, S = oracle_mod.gemm(act, codes, scales, t)
    y_mx = (a @ w_mx.T) * t
    return w_nv, w_mx, y_nv, y_mx, S


def test_mx_requantisation_moves_results_far_outside_the_parity_bound(oracle_mod):
    w_nv, w_mx, y_nv, y_mx, S = _requant_case(oracle_mod)
    changed = np.mean(w_mx != w_nv)
    rel_w = np.linalg.norm(w_mx - w_nv) / np.linalg.norm(w_nv)
    err = np.abs(y_mx - y_nv)
    outside = np.mean(err > np.ldexp(S, -16))
    rel_y = np.median(err / np.abs(y_nv))
    print("\nMX FP4 re-quantisation of NVFP4 weights (64 x 5120, N(0,0.02) source, M = 8):")
    print("  weights changed: %.1f%%, relative L2 weight error %.4f" % (100 * changed, rel_w))
    print("  GEMM outputs outside |err| <= 2^-16 S: %.1f%%; median |err|/|y| %.4f; "
          "median |err|/S %.2e" % (100 * outside, rel_y, np.median(err / S)))
    # E8M0 cannot carry the E4M3 scales' mantissa bits: most weights move
    # and nearly every output leaves the acceptance bound.
    assert changed > 0.3
    assert outside > 0.9


def test_mx_requantisation_is_exact_when_scales_are_powers_of_two(oracle_mod):
    """Sanity of the MX quantiser: NVFP4 blocks whose E4M3 scales are powers
    of two and equal within each 32-value block are MX blocks already (same
    scale, same codes), so re-quantisation changes nothing."""
    rng = np.random.default_rng(9)
    N, K = 8, 256
    codes = rng.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    # the largest element of each 32-block must reach the top binade of the
    # MX scale: force code 7 (6.0) at one position per 32 values
    codes[:, ::16] = (codes[:, ::16] & 0xF0) | 0x07
    exps = rng.integers(0, 15, size=(N, K // 32))
    s32 = (exps << 3).astype(np.uint8)  # E4M3 bytes of 2^(e-7), mantissa 0
    scales = np.repeat(s32, 2, axis=1)
    w = oracle_mod.dequantize(codes, scales, 1.0)
    assert np.array_equal(mx_fp4_requantize(w), w)
