// C ABI: status reporting, GEMM plans and their validation.
//
// The shape of this boundary follows the "Ignis" README ("Ignis" intro and
// "Building it"): all GPU compute sits in a native library behind a flat,
// device-resident C ABI.  Requests that cannot be served are refused up front
// with the offending parameter named, rather than failing inside a kernel.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <new>

#include "common.h"

namespace nvfp4 {

static thread_local char g_last_error[512] = "";

int set_error(int status, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return status;
}

void clear_error() { g_last_error[0] = 0; }

int hip_fail(hipError_t e, const char* what) {
    return set_error(NVFP4_EHIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

__global__ void fill_zero_kernel(uint4* p, size_t n16) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (; i < n16; i += stride) p[i] = make_uint4(0, 0, 0, 0);
}

__global__ void fill_zero_bytes_kernel(uint8_t* p, size_t n) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) p[i] = 0;
}

int launch_fill_zero(void* p, size_t bytes, hipStream_t s) {
    if (bytes == 0) return NVFP4_OK;
    size_t n16 = bytes / 16;
    if (n16) {
        size_t blocks = (n16 + 255) / 256;
        if (blocks > 4096) blocks = 4096;
        hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)blocks), dim3(256), 0, s, (uint4*)p,
                           n16);
        NVFP4_HIP(hipGetLastError());
    }
    size_t tail = bytes - n16 * 16;
    if (tail) {
        hipLaunchKernelGGL(fill_zero_bytes_kernel, dim3(1), dim3(16), 0, s,
                           (uint8_t*)p + n16 * 16, tail);
        NVFP4_HIP(hipGetLastError());
    }
    return NVFP4_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15) == 0; }

int validate_run(const nvfp4_gemm_plan* p, int M, int K, int N, const void* codes,
                 const void* scales, const void* act, const void* out, const void* ws) {
    if (!p || p->magic != kGemmMagic) return set_error(NVFP4_ESTATE, "plan: invalid handle");
    if (K != p->K) return set_error(NVFP4_EINVAL, "K: %d differs from the plan's K=%d", K, p->K);
    if (N != p->N) return set_error(NVFP4_EINVAL, "N: %d differs from the plan's N=%d", N, p->N);
    if (M < 1 || M > p->max_M)
        return set_error(NVFP4_EINVAL, "M: %d outside [1, max_M=%d]", M, p->max_M);
    if (!codes) return set_error(NVFP4_EINVAL, "codes: NULL");
    if (!scales) return set_error(NVFP4_EINVAL, "scales: NULL");
    if (!act) return set_error(NVFP4_EINVAL, "act: NULL");
    if (!out) return set_error(NVFP4_EINVAL, "out: NULL");
    if (!aligned16(codes)) return set_error(NVFP4_EINVAL, "codes: not 16-byte aligned");
    if (!aligned16(scales)) return set_error(NVFP4_EINVAL, "scales: not 16-byte aligned");
    if (!aligned16(act)) return set_error(NVFP4_EINVAL, "act: not 16-byte aligned");
    if (((uintptr_t)out & 3) != 0) return set_error(NVFP4_EINVAL, "out: not 4-byte aligned");
    if (p->ws_bytes && !ws) return set_error(NVFP4_EINVAL, "workspace: NULL but the plan needs %zu bytes", p->ws_bytes);
    if (ws && !aligned16(ws)) return set_error(NVFP4_EINVAL, "workspace: not 16-byte aligned");
    return NVFP4_OK;
}

RunOffsets gemm_offsets(const nvfp4_gemm_plan* p) {
    return RunOffsets{p->dec.counter_bytes, p->ver.ws_off, p->ver.ws_off + p->ver.d.counter_bytes};
}

int run_gemm(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
             float ts, const uint16_t* act, void* out, void* ws, const RunOffsets& off,
             hipStream_t s) {
    const size_t partial_off = off.dec_partial;
    if (M > NVFP4_VERIFY_MAX_M && p->pre.enabled)
        return launch_prefill(p, M, codes, scales, ts, act, out, ws, s);
    if (M > NVFP4_DECODE_MAX_M && p->ver.enabled)
        return launch_verify(p, M, codes, scales, ts, act, out, ws, off.ver_counters,
                             off.ver_partial, s);
    if (p->str.enabled) {
        // Rows beyond 8 (when no prefill kernel applies) run as further passes.
        const size_t esz = p->out_dtype == NVFP4_OUT_BF16 ? 2 : 4;
        for (int m0 = 0; m0 < M; m0 += NVFP4_DECODE_MAX_M) {
            const int mm = M - m0 < NVFP4_DECODE_MAX_M ? M - m0 : NVFP4_DECODE_MAX_M;
            int st = stream_launch_gemm(p, mm, codes, scales, ts, act + (size_t)m0 * p->K,
                                        (char*)out + (size_t)m0 * p->N * esz, s);
            if (st) return st;
        }
        return NVFP4_OK;
    }
    return launch_decode(p, M, codes, scales, ts, act, out, ws, partial_off, s);
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

const char* nvfp4_status_string(int status) {
    switch (status) {
        case NVFP4_OK: return "ok";
        case NVFP4_EINVAL: return "invalid argument";
        case NVFP4_EUNSUPPORTED: return "unsupported";
        case NVFP4_EHIP: return "HIP runtime error";
        case NVFP4_ESTATE: return "invalid state";
        default: return "unknown status";
    }
}

const char* nvfp4_last_error(void) { return g_last_error; }

int nvfp4_version(void) { return 100; }

static int create_plan(nvfp4_gemm* plan, int max_M, int K, int N, int out_dtype,
                       const nvfp4_gemm_config* cfg, size_t* workspace_bytes) {
    clear_error();
    if (!plan) return set_error(NVFP4_EINVAL, "plan: NULL");
    *plan = nullptr;
    if (K < 16 || K % 16 != 0) return set_error(NVFP4_EINVAL, "K: %d is not a positive multiple of 16", K);
    if (N < 1) return set_error(NVFP4_EINVAL, "N: %d < 1", N);
    if (max_M < 1) return set_error(NVFP4_EINVAL, "max_M: %d < 1", max_M);
    if (K > (1 << 24)) return set_error(NVFP4_EUNSUPPORTED, "K: %d above 2^24", K);
    if (N > (1 << 26)) return set_error(NVFP4_EUNSUPPORTED, "N: %d above 2^26", N);
    if (max_M > (1 << 20)) return set_error(NVFP4_EUNSUPPORTED, "max_M: %d above 2^20", max_M);
    if (out_dtype != NVFP4_OUT_F32 && out_dtype != NVFP4_OUT_BF16)
        return set_error(NVFP4_EINVAL, "out_dtype: %d is neither F32 (0) nor BF16 (1)", out_dtype);
    if (!workspace_bytes) return set_error(NVFP4_EINVAL, "workspace_bytes: NULL");
    nvfp4_gemm_plan* p = new (std::nothrow) nvfp4_gemm_plan();
    if (!p) return set_error(NVFP4_EINVAL, "plan: out of host memory");
    p->magic = kGemmMagic;
    p->max_M = max_M;
    p->K = K;
    p->N = N;
    p->out_dtype = out_dtype;
    p->Kp = padded_k(K);
    p->Np = padded_n(N);
    const int kernel = cfg ? cfg->kernel : NVFP4_KERNEL_AUTO;
    int st = NVFP4_OK;
    if (kernel < NVFP4_KERNEL_AUTO || kernel > NVFP4_KERNEL_SPLITK)
        st = set_error(NVFP4_EINVAL, "config.kernel: %d is not AUTO, STREAM or SPLITK", kernel);
    const int tiles = cfg ? cfg->tiles : 0;
    if (!st && tiles != 0 && tiles != 2 && tiles != 4 && tiles != 8)
        st = set_error(NVFP4_EINVAL, "config.tiles: %d is not 2, 4 or 8", tiles);
    p->str.enabled = kernel == NVFP4_KERNEL_STREAM;
    p->str.tiles = tiles;
    if (!st) st = make_decode_config(K, N, max_M, cfg, &p->dec);
    if (!st) st = make_verify_config(K, N, max_M, cfg, &p->ver);
    if (!st) st = make_prefill_config(max_M, K, N, &p->pre);
    if (st != NVFP4_OK) {
        p->magic = 0;
        delete p;
        return st;
    }
    // [decode counters, partials][verify counters, partials][prefill partials]:
    // the counters must stay zero between runs, so no area overlaps another.
    auto align = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t dec_ws = p->str.enabled ? 0 : p->dec.ws_bytes;
    p->ver.ws_off = align(dec_ws);
    size_t end = p->ver.d.ws_bytes ? p->ver.ws_off + p->ver.d.ws_bytes : dec_ws;
    p->pre.ws_off = align(end);
    if (p->pre.ws_bytes) end = p->pre.ws_off + p->pre.ws_bytes;
    p->ws_bytes = end;
    *workspace_bytes = p->ws_bytes;
    *plan = p;
    return NVFP4_OK;
}

int nvfp4_gemm_create(nvfp4_gemm* plan, int max_M, int K, int N, int out_dtype,
                      size_t* workspace_bytes) {
    return create_plan(plan, max_M, K, N, out_dtype, nullptr, workspace_bytes);
}

int nvfp4_gemm_create_ex(nvfp4_gemm* plan, int max_M, int K, int N, int out_dtype,
                         const nvfp4_gemm_config* config, size_t* workspace_bytes) {
    return create_plan(plan, max_M, K, N, out_dtype, config, workspace_bytes);
}

void nvfp4_gemm_destroy(nvfp4_gemm plan) {
    if (plan && plan->magic == kGemmMagic) {
        plan->magic = 0;
        delete plan;
    }
}

int nvfp4_gemm_run(nvfp4_gemm plan, int M, int K, int N, const uint8_t* codes_dev,
                   const uint8_t* scales_dev, float tensor_scale, const uint16_t* act_dev,
                   void* out_dev, void* workspace_dev, void* stream) {
    clear_error();
    int st = validate_run(plan, M, K, N, codes_dev, scales_dev, act_dev, out_dev, workspace_dev);
    if (st != NVFP4_OK) return st;
    return run_gemm(plan, M, codes_dev, scales_dev, tensor_scale, act_dev, out_dev,
                    workspace_dev, gemm_offsets(plan), (hipStream_t)stream);
}

int nvfp4_workspace_clear(void* workspace_dev, size_t bytes, void* stream) {
    clear_error();
    if (bytes == 0) return NVFP4_OK;
    if (!workspace_dev) return set_error(NVFP4_EINVAL, "workspace: NULL");
    if (!aligned16(workspace_dev)) return set_error(NVFP4_EINVAL, "workspace: not 16-byte aligned");
    return launch_fill_zero(workspace_dev, bytes, (hipStream_t)stream);
}

}  // extern "C"
