"""CPU tests of the C ABI: the library loads, exports every declared symbol,
sizes its packed planes, and refuses invalid requests (naming the parameter)
before it makes any HIP call, so none of this needs a GPU."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "nvfp4.h")


@pytest.fixture(scope="module")
def nv():
    import nvfp4_weight_streaming_amd as nv
    if not os.path.exists(nv.LIB_PATH):
        from nvfp4_weight_streaming_amd import build as b
        b.build()
    nv.lib()
    return nv


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(nvfp4_[a-z0-9_]+)\s*\(", text)))


def test_header_and_binding_agree(nv):
    declared = _declared_functions()
    assert len(declared) >= 15
    assert sorted(nv.EXPORTS) == declared


def test_width_constants_match_the_header(nv):
    text = open(HEADER).read()
    for name, value in (("NVFP4_DECODE_MAX_M", nv.DECODE_MAX_M),
                        ("NVFP4_VERIFY_MAX_M", nv.VERIFY_MAX_M)):
        m = re.search(r"#define\s+%s\s+(\d+)" % name, text)
        assert m and int(m.group(1)) == value, name


def test_library_exports_every_declared_symbol(nv):
    L = ctypes.CDLL(nv.LIB_PATH)
    for name in _declared_functions():
        assert hasattr(L, name), name


def test_status_strings(nv):
    assert nv.status_string(nv.OK) == "ok"
    assert nv.status_string(nv.EINVAL) == "invalid argument"
    assert nv.status_string(99) == "unknown status"
    assert nv.lib().nvfp4_version() >= 100


@pytest.mark.parametrize("K,N", [(256, 512), (5120, 5120), (5120, 7168), (6144, 5120),
                                 (5120, 34816), (17408, 5120), (5120, 152064), (48, 17)])
def test_packed_sizes(nv, K, N):
    Kp = -(-K // 512) * 512
    Np = -(-N // 16) * 16
    assert nv.nvfp4_packed_code_bytes(K, N) == Np * Kp // 2
    assert nv.nvfp4_packed_scale_bytes(K, N) == Np * Kp // 16


@pytest.mark.parametrize("K,N", [(0, 16), (8, 16), (24, 16), (16, 0), (-16, 4)])
def test_packed_sizes_invalid(nv, K, N):
    assert nv.nvfp4_packed_code_bytes(K, N) == 0
    assert nv.nvfp4_packed_scale_bytes(K, N) == 0


@pytest.mark.parametrize("args,word", [
    ((8, 24, 16, 0), "K"), ((8, 0, 16, 0), "K"), ((8, 256, 0, 0), "N"),
    ((0, 256, 16, 0), "max_M"), ((8, 256, 16, 7), "out_dtype")])
def test_gemm_create_rejects(nv, args, word):
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_gemm_create(*args)
    assert e.value.status == nv.EINVAL
    assert e.value.message.startswith(word)


def test_gemm_create_null_outputs(nv):
    L = nv.lib()
    ws = ctypes.c_size_t()
    assert L.nvfp4_gemm_create(None, 8, 256, 16, 0, ctypes.byref(ws)) == nv.EINVAL
    assert "plan" in nv.last_error()
    h = ctypes.c_void_p()
    assert L.nvfp4_gemm_create(ctypes.byref(h), 8, 256, 16, 0, None) == nv.EINVAL
    assert "workspace_bytes" in nv.last_error()


def test_gemm_create_size_limits(nv):
    """Shapes whose activation byte offsets would pass 2^31 in the kernels
    above 8 rows (64 rows of K values; 256-row prefill blocks) are refused."""
    for args in ((8, 1 << 24, 16, 1), (64, (1 << 24) + 16, 16, 1), (65, 1 << 22, 16, 1),
                 (2048, (1 << 22) + 512, 16, 1)):
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_gemm_create(*args)
        assert e.value.status == nv.EUNSUPPORTED and e.value.message.startswith("K"), args
    for args in ((64, (1 << 24) - 16, 16, 1), (65, (1 << 22) - 16, 16, 1)):
        plan, _ = nv.nvfp4_gemm_create(*args)
        nv.nvfp4_gemm_destroy(plan)


def test_gemm_config_validation(nv):
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_gemm_create(8, 5120, 5120, 1, split_k=0, waves=3)
    assert "waves" in e.value.message
    plan, ws = nv.nvfp4_gemm_create(8, 5120, 5120, 1, split_k=5, waves=8)
    assert ws > 0
    nv.nvfp4_gemm_destroy(plan)
    plan, ws = nv.nvfp4_gemm_create(8, 2048, 5120, 1, split_k=1, waves=4)
    assert ws == 0  # no K split: no partials, no counters
    nv.nvfp4_gemm_destroy(plan)
    # a workgroup holds at most 4 x 512 values of K, so K = 5120 needs 3 slices
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_gemm_create(8, 5120, 5120, 1, split_k=1)
    assert e.value.message.startswith("config.split_k")
    for bad in (0 - 1, 5):
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_gemm_create(8, 5120, 5120, 1, chunks=bad)
        assert e.value.message.startswith("config.chunks")
    plan, ws = nv.nvfp4_gemm_create(8, 5120, 5120, 1, chunks=4)
    assert ws > 0
    nv.nvfp4_gemm_destroy(plan)


def test_tile_kernel_config(nv):
    for bad, word in ((dict(tile_max_m=5), "config.tile_max_m"),
                      (dict(tile_max_m=-2), "config.tile_max_m"),
                      (dict(tile_superblocks=4), "config.tile_superblocks"),
                      (dict(tile_superblocks=-1), "config.tile_superblocks"),
                      # K = 17408: 34 superblocks, 34 waves of one
                      (dict(tile_max_m=2, tile_superblocks=1), "config.tile_max_m")):
        K = 17408 if bad.get("tile_superblocks") == 1 else 5120
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_gemm_create(8, K, 5120, 1, **bad)
        assert e.value.status == nv.EINVAL and e.value.message.startswith(word), e.value.message
    # the tile kernel needs no workspace: a plan that routes every width to it has none
    plan, ws = nv.nvfp4_gemm_create(4, 5120, 5120, 1, tile_max_m=4)
    assert ws >= 0
    nv.nvfp4_gemm_destroy(plan)
    for sbw in (1, 2, 3):
        plan, ws = nv.nvfp4_gemm_create(2, 2048, 100, 0, tile_max_m=2, tile_superblocks=sbw)
        nv.nvfp4_gemm_destroy(plan)


def test_gemm_run_argmax_validation(nv):
    """Errors the fused argmax run raises before launching anything."""
    f32, _ = nv.nvfp4_gemm_create(8, 5120, 1000, nv.OUT_F32)
    bf, _ = nv.nvfp4_gemm_create(8, 5120, 1000, nv.OUT_BF16)
    wide, _ = nv.nvfp4_gemm_create(16, 5120, 1000, nv.OUT_F32)
    # one slot of 8 row keys per 4-tile column group (1000 columns: 16 groups)
    need = nv.nvfp4_gemm_argmax_area_bytes(f32)
    assert need >= 16 * 64 and nv.nvfp4_gemm_argmax_area_bytes(bf) == 0
    p16, ok4 = 0x10000, 0x10004  # aligned stand-ins: nothing is dereferenced before validation
    base = dict(K=5120, N=1000, codes=p16, scales=p16, tensor_scale=1.0, act=p16, logits=p16,
                argmax=ok4, workspace=p16, area=p16, area_bytes=need)
    cases = [(bf, 8, {}, "plan"), (f32, 0, {}, "M"), (wide, 9, {}, "M"),
             (f32, 8, dict(argmax=None), "argmax"), (f32, 8, dict(argmax=0x10002), "argmax"),
             (f32, 8, dict(area=None), "area"), (f32, 8, dict(area=0x10008), "area"),
             (f32, 8, dict(area_bytes=need - 16), "area"), (f32, 8, dict(K=4096), "K")]
    try:
        for plan, M, over, word in cases:
            a = dict(base, **over)
            with pytest.raises(nv.Nvfp4Error) as e:
                nv.nvfp4_gemm_run_argmax(plan, M, a["K"], a["N"], a["codes"], a["scales"],
                                         a["tensor_scale"], a["act"], a["logits"], a["argmax"],
                                         a["workspace"], a["area"], a["area_bytes"], stream=0)
            assert e.value.status == nv.EINVAL and e.value.message.startswith(word), \
                (M, over, e.value.message)
    finally:
        for p in (f32, bf, wide):
            nv.nvfp4_gemm_destroy(p)


def test_verify_width_config(nv):
    for bad, word in ((dict(verify_waves=2), "config.verify_waves"),
                      (dict(verify_waves=32), "config.verify_waves"),
                      (dict(verify_windows=-1), "config.verify_windows"),
                      (dict(verify_ranges=-1), "config.verify_ranges"),
                      (dict(verify_ranges=5), "config.verify_ranges"),
                      (dict(verify_ranges=1, verify_windows=2), "config.verify_ranges")):
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_gemm_create(64, 5120, 5120, 1, **bad)
        assert e.value.message.startswith(word), e.value.message
    # a verify-width plan appends its own split-K area to the decode one
    p8, ws8 = nv.nvfp4_gemm_create(8, 5120, 5120, 1)
    p64, ws64 = nv.nvfp4_gemm_create(64, 5120, 5120, 1)
    assert ws64 > ws8 > 0
    nv.nvfp4_gemm_destroy(p8)
    nv.nvfp4_gemm_destroy(p64)


def test_prefill_schedule_config_and_workspace(nv):
    """prefill_schedule outside 0..2 is refused.  With the device's compute
    units taken as 256 when no GPU answers (the plan's own count otherwise),
    a prefill chunk of 544 tiles gets the stream-K area: counters, then two
    slots of 256 x 256 fp32 sums per workgroup's run; the pieces schedule
    instead holds its last round's K pieces (32 tiles x 8 pieces)."""
    for bad in (-1, 3):
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_gemm_create(2048, 5120, 17408, 1, prefill_schedule=bad)
        assert e.value.message.startswith("config.prefill_schedule"), e.value.message
    p, ws = nv.nvfp4_gemm_create(2048, 5120, 17408, 1)
    pp, wsp = nv.nvfp4_gemm_create(2048, 5120, 17408, 1, prefill_schedule=nv.PREFILL_PIECES)
    ps, wss = nv.nvfp4_gemm_create(2048, 5120, 17408, 1, prefill_schedule=nv.PREFILL_STREAM_K)
    try:
        assert ws == wss
        if not _gpu_visible():
            cus = 256
            slots = 2 * cus * 256 * 256 * 4          # two 256 x 256 fp32 slots per run
            counters = (2 * cus * 8 * 4 + 255) // 256 * 256  # per slot and wave
            assert ws - wsp == slots + counters - 32 * 8 * 256 * 256 * 4
    finally:
        for h in (p, pp, ps):
            nv.nvfp4_gemm_destroy(h)


def test_topk_validation_and_workspace(nv):
    L = nv.lib()
    assert nv.nvfp4_topk_workspace_bytes(8, 1024, 8) == 0       # one unit per row
    assert nv.nvfp4_topk_workspace_bytes(8, 152064, 8) > 0
    assert nv.nvfp4_topk_workspace_bytes(8, 100, 101) == 0      # k > V: invalid
    assert nv.nvfp4_topk_workspace_bytes(8, 100, 65) == 0       # k > 64: invalid
    for args, word in (((FAKE, 0, 10, 10, 1), "M"), ((FAKE, 2, 0, 10, 1), "V"),
                       ((FAKE, 2, 10, 9, 1), "ld"), ((FAKE, 2, 10, 10, 0), "k"),
                       ((FAKE, 2, 10, 10, 11), "k"), ((FAKE, 2, 100, 100, 65), "k"),
                       ((None, 2, 10, 10, 1), "logits")):
        assert L.nvfp4_topk(*args, FAKE, FAKE, None, 0, None) == nv.EINVAL
        assert nv.last_error().startswith(word), nv.last_error()
    assert L.nvfp4_topk(FAKE, 2, 10, 10, 1, None, FAKE, None, 0, None) == nv.EINVAL
    assert nv.last_error().startswith("idx")
    assert L.nvfp4_topk(FAKE + 2, 2, 10, 10, 1, FAKE, FAKE, None, 0, None) == nv.EINVAL
    assert "aligned" in nv.last_error()
    need = nv.nvfp4_topk_workspace_bytes(8, 152064, 8)
    assert L.nvfp4_topk(FAKE, 8, 152064, 152064, 8, FAKE, FAKE, FAKE, need - 1, None) == nv.EINVAL
    assert nv.last_error().startswith("workspace_bytes")


def test_workspace_sizes_for_round_shapes(nv):
    for K, N in [(5120, 7168), (6144, 5120), (5120, 34816), (17408, 5120), (5120, 152064)]:
        plan, ws = nv.nvfp4_gemm_create(8, K, N, 1)
        assert ws % 256 == 0
        nv.nvfp4_gemm_destroy(plan)


FAKE = 1 << 20  # a 16-byte-aligned non-null address; never dereferenced


@pytest.mark.parametrize("kw,word,status", [
    (dict(M=0), "M", 1), (dict(M=9), "M", 1), (dict(K=512), "K", 1), (dict(N=64), "N", 1),
    (dict(codes=None), "codes", 1), (dict(scales=None), "scales", 1), (dict(act=None), "act", 1),
    (dict(out=None), "out", 1), (dict(codes=FAKE + 4), "codes", 1),
    (dict(act=FAKE + 8), "act", 1), (dict(out=FAKE + 2), "out", 1),
    (dict(workspace=None), "workspace", 1), (dict(workspace=FAKE + 4), "workspace", 1)])
def test_gemm_run_validates_before_any_gpu_call(nv, kw, word, status):
    # a split-K plan: it needs a workspace, so every argument is checked
    plan, ws = nv.nvfp4_gemm_create(8, 5120, 5120, 1)
    assert ws > 0
    args = dict(M=4, K=5120, N=5120, codes=FAKE, scales=FAKE, act=FAKE, out=FAKE,
                workspace=FAKE)
    args.update(kw)
    try:
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_gemm_run(plan, args["M"], args["K"], args["N"], args["codes"],
                              args["scales"], 1.0, args["act"], args["out"], args["workspace"],
                              stream=0)
        assert e.value.status == status
        assert e.value.message.startswith(word)
    finally:
        nv.nvfp4_gemm_destroy(plan)


def test_gemm_run_bad_handle(nv):
    L = nv.lib()
    assert L.nvfp4_gemm_run(None, 1, 256, 16, FAKE, FAKE, ctypes.c_float(1.0), FAKE, FAKE,
                            None, None) == nv.ESTATE
    assert "plan" in nv.last_error()


def test_pack_and_quantize_validate(nv):
    L = nv.lib()
    assert L.nvfp4_pack(FAKE, FAKE, 24, 16, FAKE, FAKE, None) == nv.EINVAL
    assert nv.last_error().startswith("K")
    assert L.nvfp4_pack(None, FAKE, 32, 16, FAKE, FAKE, None) == nv.EINVAL
    assert nv.last_error().startswith("codes")
    assert L.nvfp4_pack(FAKE, FAKE, 32, 16, FAKE + 8, FAKE, None) == nv.EINVAL
    assert L.nvfp4_unpack(FAKE, FAKE, 32, 0, FAKE, FAKE, None) == nv.EINVAL
    assert nv.last_error().startswith("N")
    assert L.nvfp4_quantize(FAKE, 20, 4, FAKE, FAKE, FAKE, FAKE, None) == nv.EINVAL
    assert nv.last_error().startswith("K")
    assert L.nvfp4_quantize(FAKE, 32, 4, FAKE, FAKE, FAKE, None, None) == nv.EINVAL
    assert nv.last_error().startswith("workspace")
    assert nv.nvfp4_quantize_workspace_bytes() >= 4


def test_round_validation(nv):
    good = dict(K=256, N=32, codes=FAKE, scales=FAKE, tensor_scale=1.0, act=FAKE, out=FAKE,
                out_dtype=1)
    assert nv.nvfp4_round_workspace_bytes([good] * 3, 8) >= 0
    for bad, word in [(dict(K=20), "layers[1].K"), (dict(N=0), "layers[1].N"),
                      (dict(act=None), "layers[1]"), (dict(out_dtype=5), "layers[1].out_dtype"),
                      (dict(codes=FAKE + 1), "layers[1]")]:
        layers = [good, dict(good, **bad), good]
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_round_workspace_bytes(layers, 8)
        assert e.value.message.startswith(word), e.value.message
    # rounds take the verify widths too (up to 64 rows)
    assert nv.nvfp4_round_workspace_bytes([good] * 2, 64) >= 0
    with pytest.raises(nv.Nvfp4Error) as e:
        nv.nvfp4_round_workspace_bytes([good], 65)
    assert e.value.message.startswith("max_M")
    # chaining: SwiGLU of the previous output needs a previous bf16 matrix of N = 2 K
    gu = dict(good, K=256, N=64)
    dn = dict(good, K=32, N=256, act_op=nv.ACT_SWIGLU_PREV)
    assert nv.nvfp4_round_workspace_bytes([gu, dn], 8) >= 0
    for layers, word in (([dn], "layers[0].act_op"), ([good, dn], "layers[1].act_op"),
                         ([dict(gu, out_dtype=0), dn], "layers[1].act_op"),
                         ([gu, dict(dn, act_op=7)], "layers[1].act_op")):
        with pytest.raises(nv.Nvfp4Error) as e:
            nv.nvfp4_round_workspace_bytes(layers, 8)
        assert e.value.message.startswith(word), e.value.message
    L = nv.lib()
    for args, word in (((FAKE, 0, 4, FAKE, None), "M"), ((FAKE, 2, 0, FAKE, None), "F"),
                       ((None, 2, 4, FAKE, None), "gate_up"), ((FAKE, 2, 4, None, None), "out"),
                       ((FAKE + 1, 2, 4, FAKE, None), "gate_up/out")):
        assert L.nvfp4_swiglu(*args) == nv.EINVAL
        assert nv.last_error().startswith(word), nv.last_error()
    assert L.nvfp4_round_run(None, 1, None) == nv.ESTATE
    assert nv.nvfp4_round_graph_nodes(None, 1) == 0


def test_stream_read_validates(nv):
    L = nv.lib()
    sink = 0x10000
    for args, word in (((None, 1024, sink, None), "buf"), ((FAKE + 8, 1024, sink, None), "buf"),
                       ((FAKE, 0, sink, None), "bytes"), ((FAKE, 1000, sink, None), "bytes"),
                       ((FAKE, 1024, None, None), "sink"), ((FAKE, 1024, sink + 2, None), "sink")):
        assert L.nvfp4_stream_read(*args) == nv.EINVAL
        assert nv.last_error().startswith(word), nv.last_error()


def _gpu_visible():
    import torch
    return torch.cuda.is_available()


@pytest.mark.skipif("_gpu_visible()",
                    reason="forces a HIP runtime failure by launching with no device present; "
                           "with a GPU the same calls would run")
def test_hip_failure_is_returned_as_ehip(nv):
    """With no device, valid requests reach the HIP runtime, which fails: each
    entry point returns NVFP4_EHIP (it never aborts) and the message names the
    failing HIP call and carries the runtime's text."""
    L = nv.lib()
    sink = 0x10000
    st = L.nvfp4_stream_read(FAKE, 1 << 20, sink, None)
    assert st == nv.EHIP, (st, nv.last_error())
    msg = nv.last_error()
    assert "hip" in msg.lower() and "(" in msg, msg
    st = L.nvfp4_workspace_clear(FAKE, 4096, None)
    assert st == nv.EHIP, (st, nv.last_error())
    plan, ws = nv.nvfp4_gemm_create(8, 256, 16, 0)
    try:
        st = L.nvfp4_gemm_run(plan, 1, 256, 16, FAKE, FAKE, ctypes.c_float(1.0), FAKE, FAKE,
                              FAKE if ws else None, None)
        assert st == nv.EHIP, (st, nv.last_error())
    finally:
        nv.nvfp4_gemm_destroy(plan)
