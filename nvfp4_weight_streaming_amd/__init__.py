"""Python binding of libnvfp4 (the MI355X NVFP4 weight-streaming GEMM).

Argument marshalling only: every computation runs in the HIP kernels of
``libnvfp4.so``; torch is used for device memory and streams.  The functions
carry the names of the C entry points declared in ``include/nvfp4.h``.
Tensors are passed by device pointer; a ``stream`` argument defaults to
torch's current stream.  A failing call raises ``Nvfp4Error`` with the
library's message (which names the offending parameter).

If ``libnvfp4.so`` is missing, importing works but the first call raises: there
is no fallback path of any kind.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libnvfp4.so")

OK, EINVAL, EUNSUPPORTED, EHIP, ESTATE = 0, 1, 2, 3, 4
OUT_F32, OUT_BF16 = 0, 1
PREFILL_AUTO, PREFILL_PIECES, PREFILL_STREAM_K = 0, 1, 2
DECODE_MAX_M = 8
VERIFY_MAX_M = 64

# Every symbol include/nvfp4.h declares.
EXPORTS = (
    "nvfp4_status_string", "nvfp4_last_error", "nvfp4_version",
    "nvfp4_packed_code_bytes", "nvfp4_packed_scale_bytes", "nvfp4_pack", "nvfp4_unpack",
    "nvfp4_quantize_workspace_bytes", "nvfp4_quantize",
    "nvfp4_gemm_create", "nvfp4_gemm_create_ex", "nvfp4_gemm_destroy", "nvfp4_gemm_run",
    "nvfp4_gemm_run_noalloc", "nvfp4_gemm_argmax_area_bytes", "nvfp4_gemm_run_argmax",
    "nvfp4_workspace_clear",
    "nvfp4_round_workspace_bytes", "nvfp4_round_create", "nvfp4_round_run",
    "nvfp4_round_graph_nodes", "nvfp4_round_destroy",
    "nvfp4_topk_workspace_bytes", "nvfp4_topk", "nvfp4_swiglu", "nvfp4_stream_read",
)
TOPK_MAX_K = 64


class Nvfp4Error(RuntimeError):
    def __init__(self, status, message):
        super().__init__("%s (status %d): %s" % (_STATUS.get(status, "?"), status, message))
        self.status = status
        self.message = message


_STATUS = {OK: "ok", EINVAL: "EINVAL", EUNSUPPORTED: "EUNSUPPORTED", EHIP: "EHIP",
           ESTATE: "ESTATE"}


class GemmConfig(ctypes.Structure):
    _fields_ = [("split_k", ctypes.c_int), ("waves", ctypes.c_int), ("chunks", ctypes.c_int),
                ("windows", ctypes.c_int), ("verify_waves", ctypes.c_int),
                ("verify_windows", ctypes.c_int), ("tile_max_m", ctypes.c_int),
                ("tile_superblocks", ctypes.c_int), ("verify_ranges", ctypes.c_int),
                ("prefill_schedule", ctypes.c_int)]


class Layer(ctypes.Structure):
    _fields_ = [("K", ctypes.c_int), ("N", ctypes.c_int),
                ("codes_dev", ctypes.c_void_p), ("scales_dev", ctypes.c_void_p),
                ("tensor_scale", ctypes.c_float), ("act_dev", ctypes.c_void_p),
                ("out_dev", ctypes.c_void_p), ("out_dtype", ctypes.c_int),
                ("act_op", ctypes.c_int)]


ACT_INPUT, ACT_SWIGLU_PREV = 0, 1


_lib = None


def lib():
    """The loaded shared library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError("libnvfp4.so is not built (run __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        c = ctypes
        vp, sz, i = c.c_void_p, c.c_size_t, c.c_int
        L.nvfp4_status_string.argtypes = [i]
        L.nvfp4_status_string.restype = c.c_char_p
        L.nvfp4_last_error.argtypes = []
        L.nvfp4_last_error.restype = c.c_char_p
        L.nvfp4_version.restype = i
        L.nvfp4_packed_code_bytes.argtypes = [i, i]
        L.nvfp4_packed_code_bytes.restype = sz
        L.nvfp4_packed_scale_bytes.argtypes = [i, i]
        L.nvfp4_packed_scale_bytes.restype = sz
        L.nvfp4_pack.argtypes = [vp, vp, i, i, vp, vp, vp]
        L.nvfp4_unpack.argtypes = [vp, vp, i, i, vp, vp, vp]
        L.nvfp4_quantize_workspace_bytes.restype = sz
        L.nvfp4_quantize.argtypes = [vp, i, i, vp, vp, vp, vp, vp]
        L.nvfp4_gemm_create.argtypes = [c.POINTER(vp), i, i, i, i, c.POINTER(sz)]
        L.nvfp4_gemm_create_ex.argtypes = [c.POINTER(vp), i, i, i, i, c.POINTER(GemmConfig),
                                           c.POINTER(sz)]
        L.nvfp4_gemm_destroy.argtypes = [vp]
        L.nvfp4_gemm_destroy.restype = None
        L.nvfp4_gemm_run.argtypes = [vp, i, i, i, vp, vp, c.c_float, vp, vp, vp, vp]
        L.nvfp4_gemm_run_noalloc.argtypes = [vp, i, i, i, vp, vp, c.c_float, vp, vp, vp]
        L.nvfp4_gemm_run_argmax.argtypes = [vp, i, i, i, vp, vp, c.c_float, vp, vp, vp, vp, vp,
                                            sz, vp]
        L.nvfp4_gemm_argmax_area_bytes.argtypes = [vp]
        L.nvfp4_gemm_argmax_area_bytes.restype = sz
        L.nvfp4_workspace_clear.argtypes = [vp, sz, vp]
        L.nvfp4_round_workspace_bytes.argtypes = [c.POINTER(Layer), i, i, c.POINTER(sz)]
        L.nvfp4_round_create.argtypes = [c.POINTER(vp), c.POINTER(Layer), i, i, vp, sz, vp]
        L.nvfp4_round_run.argtypes = [vp, i, vp]
        L.nvfp4_round_graph_nodes.argtypes = [vp, i]
        L.nvfp4_round_destroy.argtypes = [vp]
        L.nvfp4_round_destroy.restype = None
        L.nvfp4_topk_workspace_bytes.argtypes = [i, i, i]
        L.nvfp4_topk_workspace_bytes.restype = sz
        L.nvfp4_topk.argtypes = [vp, i, i, i, i, vp, vp, vp, sz, vp]
        L.nvfp4_swiglu.argtypes = [vp, i, i, vp, vp]
        L.nvfp4_stream_read.argtypes = [vp, sz, vp, vp]
        for name in EXPORTS:
            getattr(L, name)
        _lib = L
    return _lib


def _check(status):
    if status != OK:
        raise Nvfp4Error(status, lib().nvfp4_last_error().decode(errors="replace"))


def _ptr(x):
    """Device pointer of a tensor, or an int / None passed through."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def last_error() -> str:
    return lib().nvfp4_last_error().decode(errors="replace")


def status_string(status: int) -> str:
    return lib().nvfp4_status_string(status).decode()


def nvfp4_packed_code_bytes(K: int, N: int) -> int:
    return lib().nvfp4_packed_code_bytes(K, N)


def nvfp4_packed_scale_bytes(K: int, N: int) -> int:
    return lib().nvfp4_packed_scale_bytes(K, N)


def nvfp4_pack(codes, scales, K, N, codes_packed, scales_packed, stream=None):
    _check(lib().nvfp4_pack(_ptr(codes), _ptr(scales), K, N, _ptr(codes_packed),
                            _ptr(scales_packed), _stream(stream)))


def nvfp4_unpack(codes_packed, scales_packed, K, N, codes, scales, stream=None):
    _check(lib().nvfp4_unpack(_ptr(codes_packed), _ptr(scales_packed), K, N, _ptr(codes),
                              _ptr(scales), _stream(stream)))


def nvfp4_quantize_workspace_bytes() -> int:
    return lib().nvfp4_quantize_workspace_bytes()


def nvfp4_quantize(w, K, N, codes, scales, tensor_scale, workspace, stream=None):
    _check(lib().nvfp4_quantize(_ptr(w), K, N, _ptr(codes), _ptr(scales), _ptr(tensor_scale),
                                _ptr(workspace), _stream(stream)))


def nvfp4_swiglu(gate_up, M, F, out, stream=None):
    _check(lib().nvfp4_swiglu(_ptr(gate_up), M, F, _ptr(out), _stream(stream)))


def nvfp4_stream_read(buf, nbytes, sink, stream=None):
    _check(lib().nvfp4_stream_read(_ptr(buf), nbytes, _ptr(sink), _stream(stream)))


def nvfp4_gemm_argmax_area_bytes(plan) -> int:
    return lib().nvfp4_gemm_argmax_area_bytes(plan)


def nvfp4_gemm_run_argmax(plan, M, K, N, codes, scales, tensor_scale, act, logits, argmax,
                          workspace, area, area_bytes, stream=None):
    _check(lib().nvfp4_gemm_run_argmax(plan, M, K, N, _ptr(codes), _ptr(scales),
                                       tensor_scale, _ptr(act), _ptr(logits),
                                       _ptr(argmax), _ptr(workspace), _ptr(area), area_bytes,
                                       _stream(stream)))


def nvfp4_topk_workspace_bytes(M, V, k) -> int:
    return lib().nvfp4_topk_workspace_bytes(M, V, k)


def nvfp4_topk(logits, M, V, ld, k, idx, val, workspace=None, workspace_bytes=0, stream=None):
    _check(lib().nvfp4_topk(_ptr(logits), M, V, ld, k, _ptr(idx), _ptr(val), _ptr(workspace),
                            workspace_bytes, _stream(stream)))


def topk(logits, k, stream=None):
    """(indices int32 [M][k], values [M][k]) of a device fp32 [M][V] tensor."""
    import torch
    M, V = logits.shape
    idx = torch.empty((M, k), dtype=torch.int32, device=logits.device)
    val = torch.empty((M, k), dtype=torch.float32, device=logits.device)
    wsb = nvfp4_topk_workspace_bytes(M, V, k)
    ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=logits.device) if wsb else None
    nvfp4_topk(logits, M, V, logits.stride(0), k, idx, val, ws, wsb, stream)
    return idx, val


def nvfp4_gemm_create(max_M, K, N, out_dtype, split_k=0, waves=0, chunks=0, windows=0,
                      verify_waves=0, verify_windows=0, tile_max_m=0, tile_superblocks=0,
                      verify_ranges=0, prefill_schedule=0):
    """Returns (plan handle, workspace bytes)."""
    h = ctypes.c_void_p()
    ws = ctypes.c_size_t()
    if (split_k or waves or chunks or windows or verify_waves or verify_windows or tile_max_m
            or tile_superblocks or verify_ranges or prefill_schedule):
        cfg = GemmConfig(split_k, waves, chunks, windows, verify_waves, verify_windows,
                         tile_max_m, tile_superblocks, verify_ranges, prefill_schedule)
        _check(lib().nvfp4_gemm_create_ex(ctypes.byref(h), max_M, K, N, out_dtype,
                                          ctypes.byref(cfg), ctypes.byref(ws)))
    else:
        _check(lib().nvfp4_gemm_create(ctypes.byref(h), max_M, K, N, out_dtype,
                                       ctypes.byref(ws)))
    return h.value, ws.value


def nvfp4_gemm_destroy(plan):
    lib().nvfp4_gemm_destroy(plan)


def nvfp4_gemm_run(plan, M, K, N, codes, scales, tensor_scale, act, out, workspace=None,
                   stream=None):
    _check(lib().nvfp4_gemm_run(plan, M, K, N, _ptr(codes), _ptr(scales),
                                ctypes.c_float(tensor_scale), _ptr(act), _ptr(out),
                                _ptr(workspace), _stream(stream)))


def nvfp4_gemm_run_noalloc(plan, M, K, N, codes, scales, tensor_scale, act, out, stream=None):
    _check(lib().nvfp4_gemm_run_noalloc(plan, M, K, N, _ptr(codes), _ptr(scales),
                                        ctypes.c_float(tensor_scale), _ptr(act), _ptr(out),
                                        _stream(stream)))


def nvfp4_workspace_clear(workspace, nbytes, stream=None):
    _check(lib().nvfp4_workspace_clear(_ptr(workspace), nbytes, _stream(stream)))


def _layers(layers):
    arr = (Layer * len(layers))()
    for i, l in enumerate(layers):
        arr[i] = Layer(l["K"], l["N"], _ptr(l["codes"]), _ptr(l["scales"]),
                       float(l["tensor_scale"]), _ptr(l["act"]), _ptr(l["out"]),
                       int(l.get("out_dtype", OUT_BF16)), int(l.get("act_op", ACT_INPUT)))
    return arr


def nvfp4_round_workspace_bytes(layers, max_M) -> int:
    ws = ctypes.c_size_t()
    _check(lib().nvfp4_round_workspace_bytes(_layers(layers), len(layers), max_M,
                                             ctypes.byref(ws)))
    return ws.value


def nvfp4_round_create(layers, max_M, workspace, workspace_bytes, stream=None):
    h = ctypes.c_void_p()
    _check(lib().nvfp4_round_create(ctypes.byref(h), _layers(layers), len(layers), max_M,
                                    _ptr(workspace), workspace_bytes, _stream(stream)))
    return h.value


def nvfp4_round_run(plan, M, stream=None):
    _check(lib().nvfp4_round_run(plan, M, _stream(stream)))


def nvfp4_round_graph_nodes(plan, M) -> int:
    return lib().nvfp4_round_graph_nodes(plan, M)


def nvfp4_round_destroy(plan):
    lib().nvfp4_round_destroy(plan)


# ---- convenience layer (still only marshalling) -----------------------------

class PackedWeight:
    """A K x N NVFP4 matrix in the packed layout on the GPU."""

    def __init__(self, codes_packed, scales_packed, tensor_scale: float, K: int, N: int):
        self.codes = codes_packed
        self.scales = scales_packed
        self.tensor_scale = float(tensor_scale)
        self.K = K
        self.N = N

    @staticmethod
    def alloc(K, N, device="cuda"):
        import torch
        c = torch.empty(nvfp4_packed_code_bytes(K, N), dtype=torch.uint8, device=device)
        s = torch.empty(nvfp4_packed_scale_bytes(K, N), dtype=torch.uint8, device=device)
        return c, s

    @classmethod
    def from_canonical(cls, codes, scales, tensor_scale, K, N, stream=None):
        """Pack canonical planes (device tensors [N][K/2], [N][K/16])."""
        c, s = cls.alloc(K, N, codes.device)
        nvfp4_pack(codes, scales, K, N, c, s, stream)
        return cls(c, s, tensor_scale, K, N)

    @classmethod
    def quantize(cls, w, stream=None, keep_canonical=False):
        """Quantise a device fp32 [N][K] tensor and pack it.  Reads the tensor
        scale back to the host (one synchronisation)."""
        import torch
        N, K = w.shape
        dev = w.device
        codes = torch.empty((N, K // 2), dtype=torch.uint8, device=dev)
        scales = torch.empty((N, K // 16), dtype=torch.uint8, device=dev)
        ts = torch.empty(1, dtype=torch.float32, device=dev)
        ws = torch.empty(nvfp4_quantize_workspace_bytes(), dtype=torch.uint8, device=dev)
        nvfp4_quantize(w, K, N, codes, scales, ts, ws, stream)
        pw = cls.from_canonical(codes, scales, 0.0, K, N, stream)
        pw.tensor_scale = float(ts.item())
        if keep_canonical:
            pw.canonical = (codes, scales)
        return pw


class Gemm:
    """A plan plus its workspace: ``Gemm(max_M, K, N, out_dtype)(w, act, out)``."""

    def __init__(self, max_M, K, N, out_dtype=OUT_BF16, split_k=0, waves=0, chunks=0,
                 windows=0, device="cuda", verify_waves=0, verify_windows=0, tile_max_m=0,
                 tile_superblocks=0, verify_ranges=0, prefill_schedule=0):
        import torch
        self.plan, self.ws_bytes = nvfp4_gemm_create(max_M, K, N, out_dtype, split_k, waves,
                                                     chunks, windows, verify_waves,
                                                     verify_windows, tile_max_m,
                                                     tile_superblocks, verify_ranges,
                                                     prefill_schedule)
        self.K, self.N, self.max_M, self.out_dtype = K, N, max_M, out_dtype
        self.workspace = None
        if self.ws_bytes:
            self.workspace = torch.zeros(self.ws_bytes, dtype=torch.uint8, device=device)

    def __call__(self, w: PackedWeight, act, out, M=None, stream=None):
        M = act.shape[0] if M is None else M
        nvfp4_gemm_run(self.plan, M, self.K, self.N, w.codes, w.scales, w.tensor_scale, act, out,
                       self.workspace, stream)
        return out

    def __del__(self):
        try:
            if self.plan:
                nvfp4_gemm_destroy(self.plan)
                self.plan = None
        except Exception:
            pass
