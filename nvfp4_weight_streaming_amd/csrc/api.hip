// C ABI: status reporting, GEMM plans and their validation.
//
// The shape of this boundary follows the "Ignis" README ("Ignis" intro and
// "Building it"): all GPU compute sits in a native library behind a flat,
// device-resident C ABI.  Requests that cannot be served are refused up front
// with the offending parameter named, rather than failing inside a kernel.
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
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
    return RunOffsets{p->dec.counter_bytes, p->ver.ws_off, p->ver.ws_off + p->ver.d.counter_bytes,
                      p->pre.ws_off, p->pre.ws_off + p->pre.counter_bytes};
}

int run_gemm(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
             float ts, const uint16_t* act, void* out, void* ws, const RunOffsets& off,
             hipStream_t s) {
    const size_t partial_off = off.dec_partial;
    if (M > NVFP4_VERIFY_MAX_M && p->pre.enabled)
        return launch_prefill(p, M, codes, scales, ts, act, out, ws, off.pre_counters,
                              off.pre_partial, p->pre.schedule, s);
    if (M > NVFP4_DECODE_MAX_M && p->ver.enabled)
        return launch_verify(p, M, codes, scales, ts, act, out, ws, off.ver_counters,
                             off.ver_partial, s);
    if (M <= p->tile.max_m) return launch_tile(p, M, codes, scales, ts, act, out, s);
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
    // The verify-width and prefill kernels address activations with 32-bit
    // byte offsets: 64 rows of K bf16 values (verify widths), and a block of
    // 256 rows (prefill), must stay below 2^31 bytes.
    if (K >= (1 << 24)) return set_error(NVFP4_EUNSUPPORTED, "K: %d not below 2^24", K);
    if (max_M > NVFP4_VERIFY_MAX_M && K >= (1 << 22))
        return set_error(NVFP4_EUNSUPPORTED, "K: %d not below 2^22 with max_M = %d above %d "
                         "(32-bit activation offsets of the prefill kernel)", K, max_M,
                         NVFP4_VERIFY_MAX_M);
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
    int st = make_decode_config(K, N, max_M, cfg, &p->dec);
    if (!st) st = make_tile_config(K, N, max_M, cfg, &p->tile);
    if (!st) st = make_verify_config(K, N, max_M, cfg, &p->ver);
    if (!st) st = make_prefill_config(max_M, K, N, cfg, &p->pre);
    if (st != NVFP4_OK) {
        p->magic = 0;
        delete p;
        return st;
    }
    // [decode counters, partials][verify counters, partials][prefill counters, partials]:
    // the counters must stay zero between runs, so no area overlaps another.
    auto align = [](size_t v) { return (v + 255) & ~(size_t)255; };
    const size_t dec_ws = p->dec.ws_bytes;
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

size_t nvfp4_gemm_argmax_area_bytes(nvfp4_gemm plan) {
    if (!plan || plan->magic != kGemmMagic || plan->out_dtype != NVFP4_OUT_F32) return 0;
    return ((size_t)plan->dec.n_groups * 8 * sizeof(unsigned long long) + 255) / 256 * 256;
}

int nvfp4_gemm_run_argmax(nvfp4_gemm plan, int M, int K, int N, const uint8_t* codes_dev,
                          const uint8_t* scales_dev, float tensor_scale, const uint16_t* act_dev,
                          float* logits_dev, int* argmax_dev, void* workspace_dev,
                          void* area_dev, size_t area_bytes, void* stream) {
    clear_error();
    int st = validate_run(plan, M, K, N, codes_dev, scales_dev, act_dev, logits_dev,
                          workspace_dev);
    if (st != NVFP4_OK) return st;
    if (plan->out_dtype != NVFP4_OUT_F32)
        return set_error(NVFP4_EINVAL, "plan: bf16 outputs; the argmax run needs fp32 logits");
    if (M > NVFP4_DECODE_MAX_M)
        return set_error(NVFP4_EINVAL, "M: %d above %d for the argmax run", M, NVFP4_DECODE_MAX_M);
    if (!argmax_dev) return set_error(NVFP4_EINVAL, "argmax: NULL");
    if (((uintptr_t)argmax_dev & 3) != 0) return set_error(NVFP4_EINVAL, "argmax: not 4-byte aligned");
    if (!area_dev) return set_error(NVFP4_EINVAL, "area: NULL");
    if (!aligned16(area_dev)) return set_error(NVFP4_EINVAL, "area: not 16-byte aligned");
    const size_t need = nvfp4_gemm_argmax_area_bytes(plan);
    if (area_bytes < need)
        return set_error(NVFP4_EINVAL, "area: %zu bytes, the plan needs %zu", area_bytes, need);
    return launch_decode_argmax(plan, M, codes_dev, scales_dev, tensor_scale, act_dev,
                                logits_dev, workspace_dev, gemm_offsets(plan).dec_partial,
                                area_dev, argmax_dev, (hipStream_t)stream);
}

// ---- GEMM runs that allocate nothing ----------------------------------------------

// For callers that cannot allocate device memory (graph capture, serving loops,
// harnesses that forbid it): the split-K counters and partial sums live in a
// file-scope device array, one copy per GPU, instead of a caller workspace.
// The array's name is a host-side stand-in: host code uses only the device
// address hipGetSymbolAddress returns, looked up once per device with that
// device current.  Every call on a GPU shares that GPU's copy; calls that
// overlap on one GPU race.
}  // extern "C"

namespace nvfp4 {
// Layout: [split-K counters of every plan: kScratchCounters][partial sums].
// All plans share one counter region, which every run leaves zeroed again,
// so the region stays zero from one call to the next whatever plans
// alternate; partial sums need no initial value.
constexpr size_t kScratchBytes = (size_t)16 << 20;  // 16 MiB per GPU
constexpr size_t kScratchCounters = (size_t)64 << 10;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_ptr[64];

// The device address of this device's scratch, zero-filled by a kernel on
// `s` the first time it is used on the device.  That first use must not be
// under stream capture: the fill would only be recorded into the caller's
// graph, while later calls would take the scratch as already cleared.
static int scratch_for_current_device(hipStream_t s, void** ptr) {
    int dev = 0;
    NVFP4_HIP(hipGetDevice(&dev));
    if (dev < 0 || dev >= 64) return set_error(NVFP4_EUNSUPPORTED, "device %d: above 63", dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
        NVFP4_HIP(hipStreamIsCapturing(s, &cs));
        if (cs != hipStreamCaptureStatusNone)
            return set_error(NVFP4_ESTATE, "stream: the first call on device %d is under stream "
                             "capture; make one call outside capture first (it clears the "
                             "static scratch)", dev);
        void* p = nullptr;
        NVFP4_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
        const int st = launch_fill_zero(p, kScratchBytes, s);
        if (st) return st;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return NVFP4_OK;
}

static bool noalloc_fits(size_t counters, size_t partials) {
    return counters <= kScratchCounters && partials <= kScratchBytes - kScratchCounters;
}

// The prefill schedule a run of M rows takes without a workspace: the plan's,
// except that a default plan whose stream-K slots do not fit the scratch runs
// whole tiles and K pieces instead where those fit.
static int noalloc_prefill_schedule(const nvfp4_gemm_plan* p, int M) {
    size_t c = 0, q = 0;
    prefill_ws_need(p, M, p->pre.schedule, &c, &q);
    if (noalloc_fits(c, q) || p->pre.schedule != NVFP4_PREFILL_AUTO) return p->pre.schedule;
    prefill_ws_need(p, M, NVFP4_PREFILL_PIECES, &c, &q);
    return noalloc_fits(c, q) ? NVFP4_PREFILL_PIECES : p->pre.schedule;
}

// Counter and partial-sum bytes a run of M rows needs in that layout.
static void noalloc_need(const nvfp4_gemm_plan* p, int M, size_t* counters, size_t* partials) {
    *counters = *partials = 0;
    if (M > NVFP4_VERIFY_MAX_M && p->pre.enabled) {
        prefill_ws_need(p, M, noalloc_prefill_schedule(p, M), counters, partials);
    } else if (M > NVFP4_DECODE_MAX_M && p->ver.enabled) {
        *counters = p->ver.d.counter_bytes;
        *partials = p->ver.d.partial_bytes;
    } else if (M > p->tile.max_m) {
        *counters = p->dec.counter_bytes;
        *partials = p->dec.partial_bytes;
    }
}
}  // namespace nvfp4

extern "C" {

int nvfp4_gemm_run_noalloc(nvfp4_gemm plan, int M, int K, int N, const uint8_t* codes_dev,
                           const uint8_t* scales_dev, float tensor_scale, const uint16_t* act_dev,
                           void* out_dev, void* stream) {
    clear_error();
    // Validate everything first (the scratch stands in for the workspace), so
    // that nothing is launched on error.
    int st = validate_run(plan, M, K, N, codes_dev, scales_dev, act_dev, out_dev, (void*)256);
    if (st != NVFP4_OK) return st;
    size_t nc = 0, np = 0;
    noalloc_need(plan, M, &nc, &np);
    if (!noalloc_fits(nc, np))
        return set_error(NVFP4_EUNSUPPORTED, "M: %d needs %zu bytes of split-K counters and %zu of "
                         "partial sums, above the static scratch (%zu and %zu bytes; use "
                         "nvfp4_gemm_run with a workspace)", M, nc, np, kScratchCounters,
                         kScratchBytes - kScratchCounters);
    void* ws = nullptr;
    st = scratch_for_current_device((hipStream_t)stream, &ws);
    if (st) return st;
    const RunOffsets off{kScratchCounters, 0, kScratchCounters, 0, kScratchCounters};
    if (M > NVFP4_VERIFY_MAX_M && plan->pre.enabled)
        return launch_prefill(plan, M, codes_dev, scales_dev, tensor_scale, act_dev, out_dev, ws,
                              off.pre_counters, off.pre_partial,
                              noalloc_prefill_schedule(plan, M), (hipStream_t)stream);
    return run_gemm(plan, M, codes_dev, scales_dev, tensor_scale, act_dev, out_dev, ws, off,
                    (hipStream_t)stream);
}

int nvfp4_workspace_clear(void* workspace_dev, size_t bytes, void* stream) {
    clear_error();
    if (bytes == 0) return NVFP4_OK;
    if (!workspace_dev) return set_error(NVFP4_EINVAL, "workspace: NULL");
    if (!aligned16(workspace_dev)) return set_error(NVFP4_EINVAL, "workspace: not 16-byte aligned");
    return launch_fill_zero(workspace_dev, bytes, (hipStream_t)stream);
}

}  // extern "C"
