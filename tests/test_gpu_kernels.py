"""GPU parity of the pack, quantise and GEMM kernels against the CPU oracle.

Every input comes from the seeded generator (synth); expected values come
only from the oracle.  Integer work (pack, quantiser codes) is compared
bit-exactly; GEMM outputs within |err| <= 2^-16 * sum|a*w| per element (plus
the final rounding allowance for bf16 outputs)."""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (bf16_bits, canary_out, check, dev, dev_bf16, half_block_rows, host,
                             pack, quarter_cols, require_gpu, run)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def nv():
    return require_gpu()


# ---- pack ---------------------------------------------------------------------

@pytest.mark.parametrize("K,N", [(16, 1), (48, 17), (512, 16), (1040, 100), (2576, 33),
                                 (5120, 48)])
def test_pack_unpack_roundtrip_bit_exact(nv, K, N):
    import torch
    codes, scales = synth.random_planes(11, K + N, N, K)
    cd, sd = dev(codes), dev(scales)
    pw = pack(nv, cd, sd, K, N, 1.0)
    pc = host(pw.codes)
    ps = host(pw.scales)
    # a permutation plus zero padding: byte histograms match
    hc = np.bincount(codes.ravel(), minlength=256)
    hc[0] += pc.size - codes.size
    assert np.array_equal(np.bincount(pc, minlength=256), hc)
    hs = np.bincount(scales.ravel(), minlength=256)
    hs[0] += ps.size - scales.size
    assert np.array_equal(np.bincount(ps, minlength=256), hs)
    c2 = torch.full_like(cd, 0xAB)
    s2 = torch.full_like(sd, 0xAB)
    nv.nvfp4_unpack(pw.codes, pw.scales, K, N, c2, s2)
    torch.cuda.synchronize()
    assert np.array_equal(host(c2), codes)
    assert np.array_equal(host(s2), scales)


# ---- quantiser ----------------------------------------------------------------

def _gpu_quantize(nv, W):
    import torch
    N, K = W.shape
    w = dev(W.astype(np.float32))
    codes = torch.empty((N, K // 2), dtype=torch.uint8, device="cuda")
    scales = torch.empty((N, K // 16), dtype=torch.uint8, device="cuda")
    ts = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(nv.nvfp4_quantize_workspace_bytes(), dtype=torch.uint8, device="cuda")
    nv.nvfp4_quantize(w, K, N, codes, scales, ts, ws)
    torch.cuda.synchronize()
    return host(codes), host(scales), float(host(ts)[0])


def _quantiser_cases():
    rng = np.random.default_rng(5)
    special = synth.weights(3, 9, 40, 64)
    special[0, :16] = 0.0                                   # zero block
    special[1, :16] = special[1, :16] * 1e-6                # block scale rounds to 0 / subnormal
    special[2, 16:32] = special[2, 16:32] * 1e-3
    special[3, :] = -0.0                                    # negative zeros
    special[4, 5] = 3.0                                     # a large value sets the tensor scale
    special[5, :16] = np.float32(6.375)                     # scale midpoint tie
    special[6, 32:48] = rng.uniform(-1e-4, 1e-4, 16)
    return [
        ("tiny_config", synth.weights(0, 0, 512, 256)),
        ("special", special),
        ("wide", synth.weights(0, 5, 64, 5120)),
    ]


@pytest.mark.parametrize("case", [c[0] for c in _quantiser_cases()])
def test_quantiser_bit_exact(nv, case):
    W = dict(_quantiser_cases())[case]
    c_ref, s_ref, t_ref = oracle.quantize(W)
    c, s, t = _gpu_quantize(nv, W)
    assert t == t_ref
    assert np.array_equal(s, s_ref)
    assert np.array_equal(c, c_ref)


def test_quantiser_worked_cases(nv, golden_dir):
    import os
    rows = []
    for line in open(os.path.join(golden_dir, "quantiser_worked_cases.txt")):
        if line.startswith("row"):
            head, sc, cs = line.split("|")
            rows.append(([float(v) for v in head.split(":")[1].split()], int(sc.split(":")[1], 16),
                         [int(x, 16) for x in cs.split(":")[1].split()]))
    W = np.array([r[0] for r in rows], np.float32)
    c, s, t = _gpu_quantize(nv, W)
    assert t == 1.0
    for i, (_, sc, cs) in enumerate(rows):
        assert s[i, 0] == sc
        got = []
        for byte in c[i]:
            got += [int(byte) & 15, int(byte) >> 4]
        assert got == cs, (i, got, cs)


# ---- GEMM -----------------------------------------------------------------------

def test_tiny_config_full_parity(nv):
    """M=1, K=256, N=512, fp32 out, seed 0; the GPU quantises and packs."""
    W = synth.weights(0, 0, 512, 256)
    c_ref, s_ref, t_ref = oracle.quantize(W)
    c, s, t = _gpu_quantize(nv, W)
    assert t == t_ref and np.array_equal(c, c_ref) and np.array_equal(s, s_ref)
    act = synth.activations(0, 0, 1, 256)
    pw = pack(nv, dev(c), dev(s), 256, 512, t)
    out, _ = run(nv, pw, dev_bf16(act), nv.OUT_F32)
    y, S = oracle.gemm(act, c_ref, s_ref, t_ref)
    check(out, y, S, bf16=False, what="tiny")


def test_one_hot_reconstructs_every_weight_exactly(nv):
    """Lane m of call i carries a one-hot activation at k = 8 i + m: every
    output equals one dequantised weight exactly, so the sweep reads the whole
    matrix back through the kernel and checks the packed layout and every
    index bit-exactly.  t is a power of two so w*t is exact in fp32."""
    K, N = 1040, 37
    codes, scales = synth.random_planes(21, 3, N, K)
    t = 2.0 ** -7
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    wref = oracle.dequantize(codes, scales, t)  # [N][K] fp64, exact
    eye = np.zeros((K, K), np.float32)
    np.fill_diagonal(eye, 1.0)
    bits = synth._to_bf16_bits(eye)
    g = nv.Gemm(8, K, N, nv.OUT_F32)
    import torch
    got = np.zeros((K, N))
    for k0 in range(0, K, 8):
        out = torch.full((8, N), float("nan"), device="cuda")
        g(pw, dev_bf16(bits[k0:k0 + 8]), out)
        got[k0:k0 + 8] = host(out)
    assert np.array_equal(got, wref.T)


@pytest.mark.parametrize("c,s,t", [(7, 0x7E, 0.25), (1, 0x01, 1.0), (0xB, 0x3A, 2.0 ** -20),
                                   (2, 0x38, 1.0)])
def test_closed_form_constant_weights(nv, c, s, t):
    K, N, M = 2048, 48, 8
    codes = np.full((N, K // 2), c | (c << 4), np.uint8)
    scales = np.full((N, K // 16), s, np.uint8)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    one = synth._to_bf16_bits(np.ones((M, K), np.float32))
    out, _ = run(nv, pw, dev_bf16(one), nv.OUT_F32)
    exact = K * oracle.e2m1_value(c) * oracle.e4m3_value(s) * t
    assert np.all(host(out) == exact)


def test_zero_scales_give_zero(nv):
    K, N = 512, 32
    codes, _ = synth.random_planes(4, 4, N, K)
    pw = pack(nv, dev(codes), dev(np.zeros((N, K // 16), np.uint8)), K, N, 1.0)
    out, _ = run(nv, pw, dev_bf16(synth.activations(4, 4, 8, K)), nv.OUT_F32)
    assert np.all(host(out) == 0.0)


RAGGED = [(1, 16, 1), (3, 48, 17), (8, 512, 16), (5, 1040, 100), (8, 2576, 33),
          (2, 5136, 515), (7, 12288, 40), (4, 256, 512), (6, 3072, 7)]


@pytest.mark.parametrize("M,K,N", RAGGED)
@pytest.mark.parametrize("bf16", [False, True])
def test_random_planes_ragged(nv, M, K, N, bf16):
    """Every code and every finite scale byte (subnormal ones included),
    shapes with ragged K and N tails, default plans."""
    codes, scales = synth.random_planes(M * 7 + K, N, N, K)
    t = float(np.float32(np.random.default_rng(K + N).uniform(1e-4, 1e-2)))
    act = synth.activations(M + K, N, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    out, _ = run(nv, pw, dev_bf16(act), nv.OUT_BF16 if bf16 else nv.OUT_F32)
    y, S = oracle.gemm(act, codes, scales, t)
    check(out, y, S, bf16=bf16, what="ragged %r" % ((M, K, N),))


@pytest.mark.parametrize("M,K,N", RAGGED)
@pytest.mark.parametrize("cfg", [dict(chunks=1, windows=2), dict(chunks=2, windows=3, waves=8),
                                 dict(chunks=1, windows=64)],
                         ids=["c1w2", "c2w3v8", "c1-all-of-K"])
def test_streamed_slices_ragged(nv, M, K, N, cfg):
    """The streamed-slice decode kernel on ragged K and N tails, with slices
    that end inside a window and K tails inside a superblock."""
    codes, scales = synth.random_planes(M * 5 + K, N + 1, N, K)
    t = 1.5e-3
    act = synth.activations(M + 3, K + N, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    out, _ = run(nv, pw, dev_bf16(act), nv.OUT_F32, **cfg)
    y, S = oracle.gemm(act, codes, scales, t)
    check(out, y, S, bf16=False, what="streamed %r %r" % ((M, K, N), cfg))


@pytest.mark.parametrize("M,bf16", [(8, False), (3, True)])
def test_wide_matrix_default_has_no_k_split(nv, M, bf16):
    """Column groups enough for 4 workgroups per compute unit (4098 tiles of
    16 on a 256-CU device): by default one slice covers all of K (windows of
    one superblock, the last one ragged) and no workspace is needed."""
    K, N = 528, 65563
    codes, scales = synth.random_planes(M + 40, N, N, K)
    t = 2.5e-3
    act = synth.activations(M + 41, K, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    out, g = run(nv, pw, dev_bf16(act), nv.OUT_BF16 if bf16 else nv.OUT_F32)
    import torch
    if torch.cuda.get_device_properties(0).multi_processor_count <= 256:
        assert g.ws_bytes == 0
    y, S = oracle.gemm(act, codes, scales, t)
    check(out, y, S, bf16=bf16, what="wide %r" % ((M, K, N),))


@pytest.mark.parametrize("M", [1, 2, 4, 8])
def test_projection_5120_full(nv, M):
    """The single-projection config: M lanes, K = N = 5120, quantised
    N(0, 0.02) weights, bf16 out; plus an fp32 plan checked to the strict bound."""
    K = N = 5120
    W = synth.weights(0, 100, N, K)
    c_ref, s_ref, t_ref = oracle.quantize(W)
    c, s, t = _gpu_quantize(nv, W)
    assert t == t_ref and np.array_equal(c, c_ref) and np.array_equal(s, s_ref)
    act = synth.activations(0, 100, M, K)
    pw = pack(nv, dev(c), dev(s), K, N, t)
    y, S = oracle.gemm(act, c_ref, s_ref, t_ref)
    out, _ = run(nv, pw, dev_bf16(act), nv.OUT_BF16)
    check(out, y, S, bf16=True, what="projection bf16 M=%d" % M)
    out32, _ = run(nv, pw, dev_bf16(act), nv.OUT_F32)
    check(out32, y, S, bf16=False, what="projection f32 M=%d" % M)


# ---- narrow widths: one workgroup per column tile over all of K ------------------

# Ragged K (inside a superblock, one superblock, below 512) and N (inside a
# tile), K needing 1..16 waves of 1..3 superblocks.
TILE = [(256, 512), (16, 3), (528, 40), (5120, 130), (6144, 33), (2576, 515), (17408, 20),
        (1040, 16)]


@pytest.mark.parametrize("K,N", TILE)
@pytest.mark.parametrize("sbw", [1, 2, 3])
def test_tile_kernel_forced(nv, K, N, sbw):
    """The tile kernel forced for M = 1..4 (both output dtypes) against the
    oracle; shapes whose K needs more than 16 waves of sbw superblocks are
    refused at plan time."""
    import math
    if math.ceil(-(-K // 512) / sbw) > 16:
        with pytest.raises(nv.Nvfp4Error):
            nv.Gemm(4, K, N, nv.OUT_F32, tile_max_m=4, tile_superblocks=sbw)
        return
    codes, scales = synth.random_planes(K + sbw, N + 17, N, K)
    t = float(np.float32(np.random.default_rng(K * N + sbw).uniform(1e-4, 1e-2)))
    act = synth.activations(K + 7, N + sbw, 4, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    for M in (1, 2, 3, 4):
        y, S = oracle.gemm(act[:M], codes, scales, t)
        for bf16 in (False, True):
            out, _ = run(nv, pw, dev_bf16(act[:M]), nv.OUT_BF16 if bf16 else nv.OUT_F32,
                         tile_max_m=4, tile_superblocks=sbw)
            check(out, y, S, bf16=bf16, what="tile K=%d N=%d sbw=%d M=%d" % (K, N, sbw, M))


def test_tile_kernel_repeats_bitwise_and_shares_a_plan_with_split_k(nv):
    """One plan serves M <= 4 with the tile kernel and M = 5..8 with the
    split-K kernel; repeated runs are bit-identical."""
    import torch
    K, N = 5120, 7168  # qkv: tile kernel up to M = 4 by default
    codes, scales = synth.random_planes(31, 32, N, K)
    t = 1.0e-3
    act = synth.activations(31, 33, 8, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    g = nv.Gemm(8, K, N, nv.OUT_F32)
    a = dev_bf16(act)
    for m in (1, 4, 5, 8, 2, 1):
        out = torch.full((m, N), float("nan"), dtype=torch.float32, device="cuda")
        g(pw, a[:m], out, M=m)
        again = torch.full_like(out, float("nan"))
        g(pw, a[:m], again, M=m)
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), host(again).view(np.uint32)), m
        y, S = oracle.gemm(act[:m], codes, scales, t)
        check(out, y, S, bf16=False, what="M=%d of a shared plan" % m)


CONFIGS = ([dict(chunks=c, waves=w) for w in (4, 8) for c in (1, 2, 3, 4)] +
           # streamed slices: several windows of `chunks` superblocks per workgroup
           [dict(chunks=c, waves=w, windows=n)
            for (w, c, n) in ((4, 1, 3), (4, 2, 2), (8, 2, 3), (8, 1, 5), (4, 2, 6), (8, 3, 2))])


@pytest.mark.parametrize("cfg", CONFIGS, ids=[str(sorted(c.items())) for c in CONFIGS])
def test_kernel_configurations_agree_and_are_deterministic(nv, cfg):
    M, K, N = 8, 6144, 1000
    codes, scales = synth.random_planes(8, 8, N, K)
    t = 3.0e-4
    act = synth.activations(8, 8, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    y, S = oracle.gemm(act, codes, scales, t)
    out1, g = run(nv, pw, dev_bf16(act), nv.OUT_F32, **cfg)
    check(out1, y, S, bf16=False, what=str(cfg))
    import torch
    out2 = torch.full_like(out1, float("nan"))
    for _ in range(3):  # the workspace counters must reset themselves
        g(pw, dev_bf16(act), out2)
    torch.cuda.synchronize()
    assert np.array_equal(host(out1).view(np.uint32), host(out2).view(np.uint32))


@pytest.mark.parametrize("M,K,N", [(8, 1536, 4096), (3, 2048, 64), (8, 17408, 40)])
def test_single_slice_and_long_k(nv, M, K, N):
    """No K split (K <= 2048: one slice per column group) and the longest K."""
    codes, scales = synth.random_planes(M, K, N, K)
    act = synth.activations(M, K, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, 0.002)
    out, _ = run(nv, pw, dev_bf16(act), nv.OUT_F32)
    y, S = oracle.gemm(act, codes, scales, 0.002)
    check(out, y, S, bf16=False, what="%r" % ((M, K, N),))


@pytest.mark.parametrize("M", [9, 20])
def test_more_than_eight_lanes(nv, M):
    K, N = 512, 64
    codes, scales = synth.random_planes(9, M, N, K)
    act = synth.activations(9, M, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, 0.01)
    out, _ = run(nv, pw, dev_bf16(act), nv.OUT_F32)
    y, S = oracle.gemm(act, codes, scales, 0.01)
    check(out, y, S, bf16=False, what="M=%d" % M)


def test_m_below_plan_max_and_bf16_rounding(nv):
    """A plan for 8 lanes run with fewer; bf16 out equals RNE of the fp32 out."""
    import torch
    K, N = 2048, 300
    codes, scales = synth.random_planes(12, 12, N, K)
    act = synth.activations(12, 12, 8, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, 0.003)
    g32 = nv.Gemm(8, K, N, nv.OUT_F32)
    g16 = nv.Gemm(8, K, N, nv.OUT_BF16)
    for M in (1, 3, 8):
        o32 = torch.full((M, N), float("nan"), device="cuda")
        o16 = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        g32(pw, dev_bf16(act[:M]), o32)
        g16(pw, dev_bf16(act[:M]), o16)
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(o16), bf16_bits(o32.to(torch.bfloat16)))
        y, S = oracle.gemm(act[:M], codes, scales, 0.003)
        check(o32, y, S, bf16=False, what="M=%d of 8" % M)


# ---- verify widths (8 < M <= 64: one weight pass, 16-row MFMA groups) ----------

# (M, K, N): every row-group count (M 9..16, ..64), ragged K inside a
# superblock and N inside a tile, one superblock (no split) and long K.
VERIFY = [(9, 512, 16), (16, 1040, 100), (17, 2576, 33), (31, 5136, 515), (33, 1536, 200),
          (48, 3072, 7), (49, 12288, 40), (64, 5120, 130), (64, 17408, 48), (24, 256, 1000)]


@pytest.mark.parametrize("M,K,N", VERIFY)
@pytest.mark.parametrize("bf16", [False, True])
def test_verify_width_ragged(nv, M, K, N, bf16):
    codes, scales = synth.random_planes(M * 7 + K, N + 5, N, K)
    t = float(np.float32(np.random.default_rng(K + N).uniform(1e-4, 1e-2)))
    act = synth.activations(M * 7 + 1, K + N, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    out, _ = run(nv, pw, dev_bf16(act), nv.OUT_BF16 if bf16 else nv.OUT_F32)
    y, S = oracle.gemm(act, codes, scales, t)
    check(out, y, S, bf16=bf16, what="verify %r" % ((M, K, N),))


@pytest.mark.parametrize("M,K,N", [(40, 5136, 515), (64, 3072, 300), (20, 12288, 70)])
@pytest.mark.parametrize("cfg", [dict(verify_waves=16), dict(verify_windows=3),
                                 dict(verify_waves=16, verify_windows=1),
                                 dict(verify_waves=8), dict(verify_waves=4, verify_windows=2),
                                 dict(verify_ranges=1), dict(verify_ranges=2, verify_waves=4),
                                 dict(verify_ranges=3, verify_waves=16)],
                         ids=["w16", "s3", "w16s1", "w8", "w4s2", "r1", "r2w4", "r3w16"])
def test_verify_width_configs(nv, M, K, N, cfg):
    """Non-default verify-width plans: 16 waves per workgroup, other slice
    lengths (ragged last slice, one superblock per slice), and equal ranges
    of each XCD's superblocks forced on shapes with a single column group,
    with groups on only some XCDs, and with every group split over many
    workgroups."""
    codes, scales = synth.random_planes(M + 71, K, N, K)
    t = 1.25e-3
    act = synth.activations(M + 72, N, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    out, _ = run(nv, pw, dev_bf16(act), nv.OUT_F32, **cfg)
    y, S = oracle.gemm(act, codes, scales, t)
    check(out, y, S, bf16=False, what="verify %r %r" % ((M, K, N), cfg))


def test_verify_width_rows_share_one_plan_and_repeat_bitwise(nv):
    """A plan with max_M = 64 serves every M (decode, verify), its split-K
    counters reset themselves, and repeated runs are bit-identical."""
    import torch
    K, N = 6144, 1000
    codes, scales = synth.random_planes(5, 6, N, K)
    t = 3.0e-4
    act = synth.activations(5, 7, 64, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    g = nv.Gemm(64, K, N, nv.OUT_F32)
    a = dev_bf16(act)
    for m in (64, 8, 17, 1, 40, 9, 64):
        out = torch.full((m, N), float("nan"), dtype=torch.float32, device="cuda")
        g(pw, a[:m], out, M=m)
        again = torch.full_like(out, float("nan"))
        g(pw, a[:m], again, M=m)
        torch.cuda.synchronize()
        assert np.array_equal(host(out).view(np.uint32), host(again).view(np.uint32)), m
        y, S = oracle.gemm(act[:m], codes, scales, t)
        check(out, y, S, bf16=False, what="M=%d of a max_M=64 plan" % m)


@pytest.mark.parametrize("K,N", [(16, 1), (16, 17), (32, 1), (528, 1)])
def test_smallest_shapes_through_every_kernel(nv, K, N):
    """The smallest K (one 16-value block) and N (one column) through every
    kernel one plan routes to: the tile kernel (M <= 4), split-K decode (5..8,
    and 1..8 with the tile kernel off), verify widths (9..64) and prefill
    (65, 300), both output dtypes, each against the oracle."""
    import torch
    codes, scales = synth.random_planes(K * 3 + N, K + 5, N, K)
    t = 2.0e-3
    act = synth.activations(K + N, 9, 300, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    a = dev_bf16(act)
    for tile in (0, -1):
        for dt, tdt in ((nv.OUT_F32, torch.float32), (nv.OUT_BF16, torch.bfloat16)):
            g = nv.Gemm(300, K, N, dt, tile_max_m=tile)
            for m in (1, 4, 5, 8, 9, 17, 40, 64, 65, 300):
                if tile == -1 and m > 8:
                    continue
                out, assert_canary = canary_out(m, N, tdt)
                g(pw, a[:m], out, M=m)
                torch.cuda.synchronize()
                assert_canary("K=%d N=%d M=%d" % (K, N, m))
                y, S = oracle.gemm(act[:m], codes, scales, t)
                check(out, y, S, bf16=dt == nv.OUT_BF16,
                      what="K=%d N=%d M=%d tile=%d" % (K, N, m, tile))


def test_verify_width_boundary_to_prefill(nv):
    """M = 64 is the last verify width and M = 65 the first prefill one."""
    K, N = 1024, 300
    codes, scales = synth.random_planes(11, 12, N, K)
    act = synth.activations(11, 13, 65, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, 0.002)
    for m in (64, 65):
        out, _ = run(nv, pw, dev_bf16(act[:m]), nv.OUT_F32, max_M=65)
        y, S = oracle.gemm(act[:m], codes, scales, 0.002)
        check(out, y, S, bf16=False, what="M=%d" % m)


# Default verify-width plans at full-size shapes that reach each branch of
# the plan: gate_up (K 5120, N 34816: more 4-tile groups than compute units ->
# above 16 rows one 8-wave workgroup per unit over equal ranges of its XCD's
# superblocks, 34 groups per XCD and about 10.6 superblocks per range; at 16
# rows two K slices per group), down (K 17408, N 5120: per-group slices sized
# to one workgroup per unit; long K -> 8 waves and slices of 6 superblocks at
# 17..48 rows) and a matrix wide enough for no K split at 16 rows and ranges
# of about two whole groups above (N = 65552, K = 1024).
# Last: equal ranges of 4-tile groups on a matrix wide enough that a range
# holds whole groups and runs on into the next.
VERIFY_FULL = [(5120, 34816, {}), (17408, 5120, {}), (1024, 65552, {}),
               (1024, 20000, dict(verify_ranges=1, verify_waves=4))]


@pytest.mark.parametrize("K,N,cfg", VERIFY_FULL)
def test_verify_width_default_plans_full_shapes(nv, K, N, cfg):
    import torch
    codes, scales = synth.random_planes(K + 3, N + 1, N, K)
    t = 2.5e-3
    act = synth.activations(K + 4, N + 2, 64, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    g = nv.Gemm(64, K, N, nv.OUT_BF16, **cfg)
    rng = np.random.default_rng(N)
    cols = set(rng.choice(N, 48, replace=False).tolist())
    cols |= {0, 15, 16, 63, 64, N // 2, N - 65, N - 64, N - 17, N - 16, N - 1}
    cols = np.array(sorted(cols))
    sel = torch.from_numpy(cols).cuda()
    y_all, S_all = oracle.gemm(act, codes[cols], scales[cols], t)
    a = dev_bf16(act)
    for M in (16, 32, 40, 64):
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        g(pw, a[:M], out, M=M)
        torch.cuda.synchronize()
        check(out[:, sel], y_all[:M], S_all[:M], bf16=True, what="verify M=%d K=%d N=%d" % (M, K, N))
        assert not torch.isnan(out).any().item(), "unwritten outputs at M=%d" % M


# ---- prefill (M > 8: dequantised tiles, bf16 MFMA) ------------------------------

# At most one tile per compute unit: all but the last split their tiles along K
# (fp32 partial sums and a second kernel); K = 256 is too short to split (4
# stages of 64).
@pytest.mark.parametrize("M,K,N", [(9, 512, 64), (64, 1024, 256), (300, 1040, 530),
                                   (513, 2048, 300), (256, 5120, 272), (40, 256, 1000)])
@pytest.mark.parametrize("bf16", [False, True])
def test_prefill_ragged(nv, M, K, N, bf16):
    codes, scales = synth.random_planes(M + 3 * K, N, N, K)
    t = float(np.float32(np.random.default_rng(M + N).uniform(1e-4, 1e-2)))
    act = synth.activations(M, K + N, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    out, _ = run(nv, pw, dev_bf16(act), nv.OUT_BF16 if bf16 else nv.OUT_F32)
    y, S = oracle.gemm(act, codes, scales, t)
    check(out, y, S, bf16=bf16, what="prefill %r" % ((M, K, N),))


def test_prefill_and_decode_share_a_workspace(nv):
    """One plan alternates prefill runs (K-split tiles: partial sums in the
    workspace) and decode runs (split-K counters in the same workspace): the
    prefill area must leave the decode counters zero."""
    import torch
    M, K, N = 513, 2048, 300
    codes, scales = synth.random_planes(77, N, N, K)
    t = 0.004
    act = synth.activations(77, K + N, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    g = nv.Gemm(M, K, N, nv.OUT_F32)
    a = dev_bf16(act)
    for m in (M, 8, M, 3, 8):
        out = torch.full((m, N), float("nan"), dtype=torch.float32, device="cuda")
        g(pw, a[:m], out, M=m)
        torch.cuda.synchronize()
        y, S = oracle.gemm(act[:m], codes, scales, t)
        check(out, y, S, bf16=False, what="M=%d after the other path" % m)


# ---- prefill, stream-K schedule ---------------------------------------------------

def _stream_k_shape(nv, M, K, N, default=False):
    """Whether stream-K applies to (M, K, N) on this device (tiles not a
    multiple of the compute units, every unit's run at least half a tile's K
    stages and one), or with default=True whether the default plan takes it
    (also fewer tiles than units, at most 3/4 of them)."""
    import torch
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    tiles = ((M + 255) // 256) * ((N + 255) // 256)
    nk = (K + 63) // 64
    applies = tiles % cus != 0 and tiles * nk // cus >= max(1, (nk + 1) // 2)
    if default:
        return applies and tiles < cus and 4 * tiles <= 3 * cus
    return applies


def _sk_case(nv, M, K, N, seed):
    codes, scales = synth.random_planes(seed, M + N, N, K)
    t = float(np.float32(np.random.default_rng(seed).uniform(1e-4, 1e-2)))
    act = synth.activations(seed + 1, K + N, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    cols = quarter_cols(N, seed)
    y, S = oracle.gemm(act, codes[cols], scales[cols], t)
    return pw, dev_bf16(act), cols, y, S


# Ragged M, N and K (K = 1040: a partial last stage; K = 16: one stage, so no
# tile is shared); 258 to 354 tiles on 256 compute units, and fewer tiles than
# units (136 and 188: runs shorter than a tile, up to three sharing one).
SK_SHAPES = [(300, 1040, 33000), (100, 2048, 66000), (600, 512, 30000), (300, 16, 40000),
             (512, 1040, 17408), (300, 2048, 24000)]


@pytest.mark.parametrize("M,K,N", SK_SHAPES)
@pytest.mark.parametrize("bf16", [False, True])
def test_prefill_stream_k_sampled(nv, M, K, N, bf16):
    import torch
    assert _stream_k_shape(nv, M, K, N)
    pw, a, cols, y, S = _sk_case(nv, M, K, N, M + K + N)
    out, _ = run(nv, pw, a, nv.OUT_BF16 if bf16 else nv.OUT_F32,
                 prefill_schedule=nv.PREFILL_STREAM_K)  # (canaries checked)
    check(out[:, torch.from_numpy(cols).cuda()], y, S, bf16=bf16,
          what="stream-K prefill %r" % ((M, K, N),))


# The round's other matrices at the chunk size, fewer tiles than compute units:
# o and down (160 tiles) run stream-K, runs of 60 and 170 stages sharing tiles
# two and three ways; qkv (224 tiles) runs its tiles whole, one per unit.
@pytest.mark.parametrize("name,K,N,sk", [("qkv", 5120, 7168, False), ("o", 6144, 5120, True),
                                         ("down", 17408, 5120, True)])
def test_prefill_round_shapes_at_chunk_size(nv, name, K, N, sk):
    import torch
    M = 2048
    if torch.cuda.get_device_properties(0).multi_processor_count == 256:
        assert _stream_k_shape(nv, M, K, N, default=True) == sk
    codes, scales = synth.random_planes(K + 1, N + 2, N, K)
    t = 2.5e-3
    act = synth.activations(K + 3, N + 4, M, K)
    pw = pack(nv, dev(codes), dev(scales), K, N, t)
    out, _ = run(nv, pw, dev_bf16(act), nv.OUT_BF16)
    rows, cols = half_block_rows(M, K), quarter_cols(N, N)
    y, S = oracle.gemm(act[rows], codes[cols], scales[cols], t)
    sub = out[torch.from_numpy(rows).cuda()][:, torch.from_numpy(cols).cuda()]
    check(sub, y, S, bf16=True, what="%s at M = 2048" % name)


def test_prefill_stream_k_deterministic_and_pieces_schedule(nv):
    """Repeated stream-K runs are bit-identical (a shared tile's sum does not
    depend on which contributor comes second); the pieces schedule, asked for
    by the plan, meets the same bound on the same shape."""
    import torch
    M, K, N = 300, 1040, 33000
    pw, a, cols, y, S = _sk_case(nv, M, K, N, 5)
    c = torch.from_numpy(cols).cuda()
    g = nv.Gemm(M, K, N, nv.OUT_F32, prefill_schedule=nv.PREFILL_STREAM_K)
    outs = []
    for _ in range(3):
        out = torch.full((M, N), float("nan"), device="cuda")
        g(pw, a, out)
        torch.cuda.synchronize()
        outs.append(out)
    for o in outs[1:]:
        assert np.array_equal(host(o).view(np.uint32), host(outs[0]).view(np.uint32))
    check(outs[0][:, c], y, S, bf16=False, what="stream-K")
    out, _ = run(nv, pw, a, nv.OUT_F32, prefill_schedule=nv.PREFILL_PIECES)
    check(out[:, c], y, S, bf16=False, what="pieces schedule")


def test_prefill_stream_k_fresh_slots_and_shared_workspace(nv):
    """One plan runs stream-K prefill on one weight matrix, decode, stream-K on
    another matrix, then the first again: the hand-off slots hold the previous
    run's sums when a run starts, and every run must read only its own; the
    counters must come back to zero for the decode kernel too."""
    import torch
    M, K, N = 600, 512, 30000
    cases = [_sk_case(nv, M, K, N, s) for s in (11, 12)]
    g = nv.Gemm(M, K, N, nv.OUT_F32, prefill_schedule=nv.PREFILL_STREAM_K)
    first = None
    for step, (ci, m) in enumerate([(0, M), (0, 8), (1, M), (0, M), (1, 5)]):
        pw, a, cols, y, S = cases[ci]
        c = torch.from_numpy(cols).cuda()
        out = torch.full((m, N), float("nan"), device="cuda")
        g(pw, a[:m], out, M=m)
        torch.cuda.synchronize()
        check(out[:, c], y[:m], S[:m], bf16=False, what="step %d (matrix %d, M = %d)" % (step, ci, m))
        if m == M and ci == 0:
            o = host(out)
            if first is None:
                first = o
            else:
                assert np.array_equal(o.view(np.uint32), first.view(np.uint32))


def test_prefill_chunk_config_sampled(nv):
    """The prefill-chunk config: M = 2048, K = 5120, N = 17408, quantised
    N(0, 0.02) weights, bf16 out; every row, sampled columns.  544 tiles on a
    256-CU device: the default plan's whole tiles with the last round's 32
    tiles in 8 K pieces each, and the stream-K schedule (224 of the tiles
    shared between two workgroups)."""
    import torch
    M, K, N = 2048, 5120, 17408
    W = synth.weights(0, 300, N, K)
    cols = np.array(sorted(set(np.random.default_rng(1).choice(N, 40, replace=False).tolist())
                           | {0, 255, 256, 16383, 16384, 16895, 17000, N - 1}))
    t = oracle.tensor_scale(W)
    c_ref, s_ref = oracle.quantize_rows(W[cols], t)
    c, s, tg = _gpu_quantize(nv, W)
    assert tg == t and np.array_equal(c[cols], c_ref) and np.array_equal(s[cols], s_ref)
    act = synth.activations(0, 300, M, K)
    pw = pack(nv, dev(c), dev(s), K, N, tg)
    y, S = oracle.gemm(act, c_ref, s_ref, t)
    for sch in (nv.PREFILL_AUTO, nv.PREFILL_STREAM_K):
        out, _ = run(nv, pw, dev_bf16(act), nv.OUT_BF16, prefill_schedule=sch)
        check(out[:, torch.from_numpy(cols).cuda()], y, S, bf16=True,
              what="prefill chunk, schedule %d" % sch)
