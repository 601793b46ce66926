"""Pins of the CPU oracle against things other than itself.

* E2M1: the OCP MX FP4 table (tests/golden/e2m1_ocp_mx_fp4.txt).
* E4M3: torch's float8_e4m3fn decoder for all 256 bytes, the OCP FP8
  landmarks (tests/golden/e4m3_ocp_fp8_special.txt), and torch's
  round-to-nearest-even cast for the encoder below the saturation point.
* bf16: torch's bfloat16 decoder.
* Quantiser: hand-worked cases (tests/golden/quantiser_worked_cases.txt) and
  the nearest-value invariants on random N(0, 0.02) matrices.
* GEMM: exact rational brute force (Python fractions over the golden/torch
  tables), a closed form, one-hot reconstruction, zero scales.
* SwiGLU: the fp64 -> bf16 rounding against hand-worked cases
  (tests/golden/bf16_rounding_cases.txt) and torch's float32 -> bfloat16
  cast; silu against closed forms and the tanh form of the logistic function.
* Top-k: hand-worked cases (tests/golden/topk_worked_cases.txt), numpy's
  first-occurrence argmax (k = 1) and stable argsort (k = V), and order and
  selection invariants on random rows with many ties.
* A set of deliberately broken oracles (mistakes planted on the CPU) must
  fail these pins, which shows they can catch a dropped term, a swapped
  nibble order, a transposed operand or a wrong block index.
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import synth

pytestmark = pytest.mark.filterwarnings("ignore")


# ---- golden tables ----------------------------------------------------------

def _golden_e2m1(golden_dir):
    vals = {}
    with open(os.path.join(golden_dir, "e2m1_ocp_mx_fp4.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            c, v = line.split()
            vals[int(c, 16)] = float(v)
    assert len(vals) == 16
    return vals


def _torch_e4m3_table():
    b = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return b.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_bf16(bits):
    return torch.from_numpy(np.asarray(bits, np.uint16).view(np.int16)).view(
        torch.bfloat16).to(torch.float64).numpy()


# ---- element decoders -------------------------------------------------------

def test_e2m1_all_16_codes(oracle_mod, golden_dir):
    g = _golden_e2m1(golden_dir)
    for c in range(16):
        v = oracle_mod.e2m1_value(c)
        assert v == g[c], (c, v, g[c])
        assert math.copysign(1.0, v) == math.copysign(1.0, g[c])


def test_e4m3_all_256_bytes_match_torch(oracle_mod):
    ref = _torch_e4m3_table()
    for b in range(256):
        v = oracle_mod.e4m3_value(b)
        if math.isnan(ref[b]):
            assert math.isnan(v), b
        else:
            assert v == ref[b], (b, v, ref[b])
            assert math.copysign(1.0, v) == math.copysign(1.0, ref[b])


def test_e4m3_landmarks(oracle_mod, golden_dir):
    with open(os.path.join(golden_dir, "e4m3_ocp_fp8_special.txt")) as f:
        rows = [l.split() for l in f if l.strip() and not l.startswith("#")]
    assert len(rows) >= 10
    for b, v in rows:
        got = oracle_mod.e4m3_value(int(b, 16))
        if v == "nan":
            assert math.isnan(got)
        else:
            assert got == float(v), (b, got, v)
    finite_nonneg = [b for b in range(128) if not math.isnan(oracle_mod.e4m3_value(b))]
    assert len(finite_nonneg) == 127


def test_bf16_decode_matches_torch(oracle_mod):
    rng = np.random.default_rng(0)
    bits = np.concatenate([rng.integers(0, 65536, 4000), [0, 0x8000, 0x3F80, 0x0001, 0x7F7F]])
    bits = bits[((bits >> 7) & 0xFF) != 0xFF]  # finite patterns
    ref = _torch_bf16(bits.astype(np.uint16))
    for b, r in zip(bits, ref):
        assert oracle_mod.bf16_value(int(b)) == r


# ---- element encoders -------------------------------------------------------

def test_e4m3_encoder_matches_torch_rne_below_saturation(oracle_mod):
    table = _torch_e4m3_table()
    finite = sorted(set(float(table[b]) for b in range(127)))
    xs = list(finite)
    xs += [(a + b) / 2 for a, b in zip(finite[:-1], finite[1:])]      # every tie point
    xs += [np.nextafter(np.float32(x), np.float32(0)) for x in xs if x > 0]
    xs += [np.nextafter(np.float32(x), np.float32(1e9)) for x in xs]
    rng = np.random.default_rng(1)
    xs += list(rng.uniform(0, 464, 3000)) + list(np.exp(rng.uniform(-12, 6, 3000)))
    xs = np.array([x for x in xs if 0 <= x < 464], dtype=np.float32)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    for x, r in zip(xs, ref):
        assert oracle_mod.e4m3_encode(float(x)) == int(r), (float(x), int(r))


def test_e4m3_encoder_saturates(oracle_mod):
    for x in [448.0, 463.9, 464.0, 470.0, 1e6, float("inf")]:
        assert oracle_mod.e4m3_encode(x) == 0x7E


def test_e2m1_encoder_nearest_ties_to_even(oracle_mod, golden_dir):
    g = _golden_e2m1(golden_dir)
    mags = [g[c] for c in range(8)]
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}
    for x, c in ties.items():
        assert oracle_mod.e2m1_encode(x) == c
        assert oracle_mod.e2m1_encode(-x) == c | 8
    rng = np.random.default_rng(2)
    for x in np.concatenate([rng.uniform(-8, 8, 4000), np.linspace(-7, 7, 2801)]):
        x = float(np.float32(x))
        c = oracle_mod.e2m1_encode(x)
        assert (c >> 3) == (1 if math.copysign(1, x) < 0 else 0)
        best = min(abs(m - abs(x)) for m in mags)
        assert abs(mags[c & 7] - abs(x)) == best, (x, c)
    assert oracle_mod.e2m1_encode(100.0) == 7 and oracle_mod.e2m1_encode(-7.0) == 15


# ---- quantiser --------------------------------------------------------------

def _worked_cases(golden_dir):
    rows = []
    with open(os.path.join(golden_dir, "quantiser_worked_cases.txt")) as f:
        for line in f:
            if not line.startswith("row"):
                continue
            head, scale, codes = line.split("|")
            w = [float(v) for v in head.split(":")[1].split()]
            rows.append((w, int(scale.split(":")[1], 16),
                         [int(c, 16) for c in codes.split(":")[1].split()]))
    return rows


def test_quantiser_worked_cases(oracle_mod, golden_dir):
    rows = _worked_cases(golden_dir)
    W = np.array([r[0] for r in rows], np.float32)
    codes, scales, t = oracle_mod.quantize(W)
    assert t == 1.0
    for i, (_, sc, cs) in enumerate(rows):
        assert scales[i, 0] == sc, (i, scales[i, 0], sc)
        got = []
        for byte in codes[i]:
            got += [int(byte) & 15, int(byte) >> 4]
        assert got == cs, (i, got, cs)


def test_quantiser_invariants_random(oracle_mod, golden_dir):
    g = _golden_e2m1(golden_dir)
    e4 = _torch_e4m3_table()
    W = synth.weights(0, 7, 24, 256)
    codes, scales, t = oracle_mod.quantize(W)
    amax = float(np.max(np.abs(W)))
    assert t == float(np.float32(amax) / np.float32(2688.0))
    for n in range(W.shape[0]):
        for b in range(W.shape[1] // 16):
            blk = W[n, 16 * b:16 * b + 16]
            s = np.float32(np.float32(np.max(np.abs(blk))) / np.float32(6.0)) / np.float32(t)
            ref_sc = int(torch.tensor([float(s)], dtype=torch.float32).to(
                torch.float8_e4m3fn).view(torch.uint8)[0])
            assert scales[n, b] == ref_sc
            d = np.float32(e4[ref_sc]) * np.float32(t)
            for i in range(16):
                byte = codes[n, 8 * b + i // 2]
                c = (byte >> 4) if (i & 1) else (byte & 15)
                x = np.float32(blk[i]) / d
                err = abs(abs(g[c]) - abs(float(x)))
                assert err == min(abs(g[m] - abs(float(x))) for m in range(8))


def test_quantiser_zero_tensor(oracle_mod):
    codes, scales, t = oracle_mod.quantize(np.zeros((3, 32), np.float32))
    assert t == 0.0 and not codes.any() and not scales.any()


# ---- GEMM -------------------------------------------------------------------

def _exact(act_bits, codes, scales, t, golden_dir):
    """Exact rational y and S from the golden E2M1 table and torch's E4M3 and
    bf16 decoders."""
    g = _golden_e2m1(golden_dir)
    e4 = _torch_e4m3_table()
    a = _torch_bf16(act_bits)
    M, K = act_bits.shape
    N = codes.shape[0]
    tq = Fraction(float(t))
    y = [[Fraction(0)] * N for _ in range(M)]
    S = [[Fraction(0)] * N for _ in range(M)]
    for n in range(N):
        for k in range(K):
            byte = int(codes[n, k // 2])
            c = (byte >> 4) if (k & 1) else (byte & 15)
            w = Fraction(g[c]) * Fraction(float(e4[int(scales[n, k // 16])])) * tq
            for m in range(M):
                p = Fraction(float(a[m, k])) * w
                y[m][n] += p
                S[m][n] += abs(p)
    return y, S


def _random_case(seed, M, K, N):
    codes, scales = synth.random_planes(seed, 1, N, K)
    act = synth.activations(seed, 2, M, K)
    t = float(np.float32(np.random.default_rng(seed).uniform(1e-5, 2.0)))
    return act, codes, scales, t


def _check_brute_force(gemm, golden_dir, seeds=range(6)):
    shapes = [(1, 16, 1), (3, 32, 5), (8, 64, 8), (5, 48, 7), (2, 64, 3), (8, 16, 2)]
    for seed, (M, K, N) in zip(seeds, shapes):
        act, codes, scales, t = _random_case(seed, M, K, N)
        y, S = gemm(act, codes, scales, t)
        ey, eS = _exact(act, codes, scales, t, golden_dir)
        for m in range(M):
            for n in range(N):
                bound = float(eS[m][n]) * K * 2.0 ** -52 + 1e-300
                if abs(Fraction(float(y[m, n])) - ey[m][n]) > Fraction(bound):
                    return False
                if abs(float(S[m, n]) - float(eS[m][n])) > bound:
                    return False
    return True


def test_gemm_brute_force_fractions(oracle_mod, golden_dir):
    assert _check_brute_force(lambda *a: oracle_mod.gemm(*a, threads=2), golden_dir)


def test_gemm_closed_form_constant(oracle_mod, golden_dir):
    g = _golden_e2m1(golden_dir)
    e4 = _torch_e4m3_table()
    K, N = 256, 4
    one = synth._to_bf16_bits(np.ones((1, K), np.float32))
    for c, s, t in [(7, 0x7E, 0.25), (1, 0x01, 1.0), (0xB, 0x3A, 3.0e-5), (2, 0x38, 1.0)]:
        codes = np.full((N, K // 2), c | (c << 4), np.uint8)
        scales = np.full((N, K // 16), s, np.uint8)
        y, S = oracle_mod.gemm(one, codes, scales, np.float32(t))
        exact = K * g[c] * float(e4[s]) * float(np.float32(t))
        assert np.all(y == exact), (c, s, y[0, 0], exact)
        assert np.all(S == abs(exact))


def test_gemm_one_hot_reconstructs_weights(oracle_mod, golden_dir):
    g = _golden_e2m1(golden_dir)
    e4 = _torch_e4m3_table()
    K, N = 64, 6
    codes, scales = synth.random_planes(3, 4, N, K)
    t = float(np.float32(0.0123))
    eye = synth._to_bf16_bits(np.eye(K, dtype=np.float32))
    y, _ = oracle_mod.gemm(eye, codes, scales, t)
    for k in range(K):
        for n in range(N):
            byte = int(codes[n, k // 2])
            c = (byte >> 4) if (k & 1) else (byte & 15)
            assert y[k, n] == g[c] * float(e4[scales[n, k // 16]]) * t


def test_gemm_zero_scales_give_zero(oracle_mod):
    codes, _ = synth.random_planes(5, 6, 4, 128)
    act = synth.activations(5, 7, 3, 128)
    y, S = oracle_mod.gemm(act, codes, np.zeros((4, 8), np.uint8), 0.5)
    assert not y.any() and not S.any()


# ---- dequantisation -------------------------------------------------------------

def _dequant_pins(dequant, oracle_mod, golden_dir):
    """w[n][k] element-wise against (1) the exact value from the golden E2M1
    table, torch's E4M3 decoder and the canonical nibble order (low nibble =
    even k), and (2) the oracle GEMM with one-hot bf16 activation rows (row k
    of the identity returns column k of w, one exact product per output).
    Returns False on the first mismatch."""
    g = _golden_e2m1(golden_dir)
    e4 = _torch_e4m3_table()
    for seed, (K, N) in enumerate([(16, 1), (64, 6), (256, 9), (48, 48), (512, 3)]):
        codes, scales = synth.random_planes(60 + seed, 8, N, K)
        t = float(np.float32(np.random.default_rng(seed).uniform(1e-4, 3.0)))
        w = np.asarray(dequant(codes, scales, t))
        if w.shape != (N, K):
            return False
        for n in range(N):
            for k in range(K):
                byte = int(codes[n, k // 2])
                c = (byte >> 4) if (k & 1) else (byte & 15)
                exact = Fraction(g[c]) * Fraction(float(e4[int(scales[n, k // 16])])) * Fraction(t)
                if Fraction(float(w[n, k])) != exact:
                    return False
        eye = synth._to_bf16_bits(np.eye(K, dtype=np.float32))
        y, _ = oracle_mod.gemm(eye, codes, scales, t, threads=2)
        if not np.array_equal(w, y.T):
            return False
    return True


def test_dequantize_pins(oracle_mod, golden_dir):
    assert _dequant_pins(oracle_mod.dequantize, oracle_mod, golden_dir)


def _dequant_tiled(oracle_mod, codes, scales, t):
    """oracle.dequantize with one planted mistake: the block scales laid along
    K by tiling the row of scales instead of repeating each one 16 times."""
    N, K = codes.shape[0], codes.shape[1] * 2
    e2 = np.array([oracle_mod.e2m1_value(c) for c in range(16)])
    e4 = np.array([oracle_mod.e4m3_value(b) for b in range(256)])
    c = np.empty((N, K), np.int64)
    c[:, 0::2] = codes & 15
    c[:, 1::2] = codes >> 4
    s = np.tile(scales.astype(np.int64), (1, 16))
    return e2[c] * e4[s] * float(t)


DEQUANT_MUTANTS = {
    "nibble_order": lambda o, c, s, t: o.dequantize(_swap_nibbles(c), s, t),
    "block_shift": lambda o, c, s, t: o.dequantize(c, np.roll(s, 1, axis=1), t),
    "scales_tiled": _dequant_tiled,
    "sign_ignored": lambda o, c, s, t: o.dequantize((c & 0x77).astype(np.uint8), s, t),
    "no_tensor_scale": lambda o, c, s, t: o.dequantize(c, s, 1.0),
    "transposed": lambda o, c, s, t: o.dequantize(c, s, t).T,
}


@pytest.mark.parametrize("name", sorted(DEQUANT_MUTANTS))
def test_dequantize_planted_mistakes_fail_the_pins(oracle_mod, golden_dir, name):
    mutant = DEQUANT_MUTANTS[name]
    assert not _dequant_pins(lambda c, s, t: mutant(oracle_mod, c, s, t), oracle_mod, golden_dir)


# ---- acceptance bounds ------------------------------------------------------------

def test_tolerance_bounds(oracle_mod):
    """tolerance(S) is 2^-16 S.  tolerance_bf16(y, 0) admits the bf16 store of
    any value (the oracle's pinned fp64 -> bf16 rounding), including a tie at
    the bottom of a binade (1 + 2^-8 rounds to 1: error 2^-8 of the value),
    which a 2^-9 allowance would reject."""
    S = np.array([0.0, 1.0, 3.5e-3, 65.0])
    assert np.array_equal(oracle_mod.tolerance(S), S / 65536.0)
    rng = np.random.default_rng(11)
    y = np.concatenate([rng.standard_normal(2000) * 10.0 ** rng.uniform(-6, 6, 2000),
                        [1.0 + 2.0 ** -8, -(1.0 + 2.0 ** -8), 2.0 ** -126 * 1.5]])
    b = oracle_mod.bf16_round(y)
    stored = (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    err = np.abs(stored - y)
    assert np.all(err <= oracle_mod.tolerance_bf16(y, np.zeros_like(y)))
    assert err[-3] > np.ldexp(abs(y[-3]), -9)


# ---- planted mistakes must be caught ----------------------------------------

def _swap_nibbles(codes):
    return ((codes >> 4) | (codes << 4)).astype(np.uint8)


MUTANTS = {
    # low/high nibble order exchanged
    "nibble_order": lambda o, a, c, s, t: o.gemm(a, _swap_nibbles(c), s, t),
    # tensor scale dropped
    "no_tensor_scale": lambda o, a, c, s, t: o.gemm(a, c, s, 1.0),
    # block index off by one (scales shifted along K)
    "block_shift": lambda o, a, c, s, t: o.gemm(a, c, np.roll(s, 1, axis=1), t),
    # the last activation column dropped
    "dropped_term": lambda o, a, c, s, t: o.gemm(
        np.concatenate([a[:, :-1], np.zeros((a.shape[0], 1), np.uint16)], 1), c, s, t),
    # activations reversed along K (a transposed / mis-indexed operand)
    "reversed_k": lambda o, a, c, s, t: o.gemm(np.ascontiguousarray(a[:, ::-1]), c, s, t),
    # sign bit of the E2M1 code ignored
    "sign_ignored": lambda o, a, c, s, t: o.gemm(a, (c & 0x77).astype(np.uint8), s, t),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistakes_fail_brute_force(oracle_mod, golden_dir, name):
    mutant = MUTANTS[name]
    assert not _check_brute_force(lambda a, c, s, t: mutant(oracle_mod, a, c, s, t), golden_dir)


# ---- top-k --------------------------------------------------------------------

def _golden_topk(golden_dir):
    cases = []
    with open(os.path.join(golden_dir, "topk_worked_cases.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            row, k, idx = line.split("|")
            vals = np.array([float(v) for v in row.split(":")[1].split()], np.float32)
            cases.append((vals, int(k.split(":")[1]), [int(i) for i in idx.split(":")[1].split()]))
    assert len(cases) >= 7
    return cases


def _topk_pins(topk, golden_dir):
    """Every top-k pin, for the oracle and for planted mistakes."""
    for vals, k, want in _golden_topk(golden_dir):
        idx, got = topk(vals[None, :], k)
        assert idx[0].tolist() == want, (vals, k, idx[0].tolist(), want)
        assert np.array_equal(got[0].view(np.uint32), vals[want].view(np.uint32))
    rng = np.random.default_rng(5)
    for M, V, k in ((3, 50, 1), (2, 37, 37), (4, 200, 9), (1, 1000, 64)):
        # few distinct values (many ties), both zeros, some infinities
        pool = np.array([-np.inf, -2.5, -1, -0.0, 0.0, 0.5, 1, 1, 3, np.inf], np.float32)
        x = pool[rng.integers(0, len(pool), (M, V))]
        idx, got = topk(x, k)
        for m in range(M):
            if k == 1:
                assert idx[m, 0] == np.argmax(x[m])  # first occurrence of the maximum
            if k == V:
                assert idx[m].tolist() == np.argsort(-x[m], kind="stable").tolist()
            sel = idx[m].tolist()
            assert len(set(sel)) == k
            v = x[m, sel]
            for a in range(k - 1):  # descending; ties by ascending index
                assert v[a] > v[a + 1] or (v[a] == v[a + 1] and sel[a] < sel[a + 1])
            rest = np.setdiff1d(np.arange(V), sel)
            kth, kth_i = v[-1], sel[-1]
            assert np.all((x[m, rest] < kth) | ((x[m, rest] == kth) & (rest > kth_i)))


def test_topk_pins(oracle_mod, golden_dir):
    _topk_pins(oracle_mod.topk, golden_dir)


def _topk_mutant(kind):
    def f(x, k):
        x = np.asarray(x, np.float32)
        M, V = x.shape
        idx = np.empty((M, k), np.int32)
        for m in range(M):
            if kind == "ties_descending_index":
                order = np.lexsort((-np.arange(V), -x[m].astype(np.float64)))
            elif kind == "negative_zero_below":  # total order on the bits: -0 < +0
                key = x[m].view(np.int32).astype(np.int64)
                key = np.where(key < 0, -(key & 0x7FFFFFFF) - 1, key)
                order = np.lexsort((np.arange(V), -key))
            else:  # "ascending"
                order = np.lexsort((np.arange(V), x[m].astype(np.float64)))
            idx[m] = order[:k]
        return idx, np.take_along_axis(x, idx.astype(np.int64), axis=1)
    return f


@pytest.mark.parametrize("kind", ["ties_descending_index", "negative_zero_below", "ascending"])
def test_topk_planted_mistakes_fail_the_pins(golden_dir, kind):
    with pytest.raises(AssertionError):
        _topk_pins(_topk_mutant(kind), golden_dir)


# ---- SwiGLU -------------------------------------------------------------------

def _golden_bf16_rounding(golden_dir):
    cases = []
    with open(os.path.join(golden_dir, "bf16_rounding_cases.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            v, b = line.split()
            cases.append((float.fromhex(v), int(b, 16)))
    assert len(cases) >= 14
    return cases


def _bits_bf16(x):
    """float32 array -> bf16 bits by truncation (exact for bf16 values)."""
    return (np.asarray(x, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _swiglu_pins(bf16_round, swiglu, golden_dir):
    for v, want in _golden_bf16_rounding(golden_dir):
        got = int(bf16_round(np.array([v]))[0])
        assert got == want, (v.hex(), hex(got), hex(want))
    # torch rounds float32 -> bfloat16 to nearest-even; for float32 values the
    # single rounding from fp64 must agree
    rng = np.random.default_rng(11)
    x32 = (rng.standard_normal(4000) * np.exp2(rng.integers(-30, 30, 4000))).astype(np.float32)
    want = torch.from_numpy(x32).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_round(x32.astype(np.float64)), want)
    # silu: closed forms (g = 0 and u = 0 give zero; g = 100 makes the logistic
    # factor 1 in fp64, so the result is bf16(g * u)) and the tanh form
    # 1 / (1 + e^-g) = (1 + tanh(g / 2)) / 2, another library routine
    F = 256
    g = (rng.standard_normal(F) * 3).astype(np.float32)
    u = (rng.standard_normal(F) * 2).astype(np.float32)
    g[:4] = [0.0, -0.0, 100.0, -100.0]
    u[4:6] = [0.0, -0.0]
    gb, ub = _bits_bf16(g), _bits_bf16(u)
    gu = np.concatenate([gb, ub])[None, :]
    got = swiglu(gu)[0]
    gd = (gb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ud = (ub.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert got[0] in (0x0000, 0x8000) and got[1] in (0x0000, 0x8000)
    assert got[4] in (0x0000, 0x8000) and got[5] in (0x0000, 0x8000)
    assert got[2] == bf16_round(np.array([gd[2] * ud[2]]))[0]
    want = bf16_round(gd * ud * (1.0 + np.tanh(gd / 2.0)) / 2.0)
    assert np.array_equal(got[6:], want[6:]), np.argwhere(got[6:] != want[6:])[:3]
    # g = -100: the logistic factor is e^g to fp64 precision (another closed form)
    assert got[3] == bf16_round(np.array([gd[3] * ud[3] * np.exp(gd[3])]))[0]


def test_swiglu_pins(oracle_mod, golden_dir):
    _swiglu_pins(oracle_mod.bf16_round, oracle_mod.swiglu, golden_dir)


def _swiglu_mutant(oracle_mod, kind):
    def rnd(x):
        x = np.asarray(x, np.float64)
        if kind == "round_via_fp32":
            x32 = x.astype(np.float32)
            return _bits_bf16(x32) + ((x32.view(np.uint32) & 0xFFFF) > 0x8000).astype(np.uint16) \
                + (((x32.view(np.uint32) & 0xFFFF) == 0x8000) & (_bits_bf16(x32) & 1 == 1)).astype(np.uint16)
        if kind == "ties_away":
            out = oracle_mod.bf16_round(x)
            a = np.abs(x)
            for i, v in enumerate(a.ravel()):
                if v == 0 or not np.isfinite(v):
                    continue
                e = int(np.frexp(v)[1]) - 1
                step = 2.0 ** (max(e, -126) - 7)
                q = np.floor(v / step)
                if v - q * step == step / 2:
                    r = np.float32((q + 1) * step)
                    out.flat[i] = (out.flat[i] & 0x8000) | (int(r.view(np.uint32)) >> 16)
            return out
        return oracle_mod.bf16_round(x)

    def swi(gu_bits):
        gu = np.ascontiguousarray(gu_bits, dtype=np.uint16)
        M, F2 = gu.shape
        F = F2 // 2
        x = (gu.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        g, u = x[:, :F], x[:, F:]
        if kind == "halves_swapped":
            g, u = u, g
        with np.errstate(over="ignore"):
            y = g * u / (1.0 + np.exp(g if kind == "exp_sign" else -g))
        return rnd(y)
    return rnd, swi


@pytest.mark.parametrize("kind", ["round_via_fp32", "ties_away", "halves_swapped", "exp_sign"])
def test_swiglu_planted_mistakes_fail_the_pins(oracle_mod, golden_dir, kind):
    rnd, swi = _swiglu_mutant(oracle_mod, kind)
    with pytest.raises(AssertionError):
        _swiglu_pins(rnd, swi, golden_dir)
