// Plain streaming read: the achievable HBM read rate that the decode kernels'
// weight stream is measured against.
//
// "Ignis" README, "What sets it apart", "The decode round": the round streams
// the weights at the card's memory bandwidth, so the useful ceiling for a
// decode kernel is what a kernel that only reads can reach on the same chip.
// Two load shapes, both non-temporal 16-byte loads (the streaming hint of the
// decode kernels' weight loads), by size:
//   - up to 512 MiB, one load per thread over as many 256-thread workgroups
//     as the buffer needs: in a graph of one read per matrix of the 27B-class
//     round this took 2.08 ms against 2.18 ms for the shape below;
//   - above, 8 loads per thread and step over 4 workgroups per compute unit,
//     striding over the buffer: 7.06 TB/s on a 4 GiB buffer on MI355X, above
//     1, 2 and 4 loads per step and other grid sizes.
// The loaded words are folded into one value so the loads are kept; that
// value is stored only if it equals an improbable constant.
#include "common.h"

namespace nvfp4 {

typedef unsigned int u32v4_t __attribute__((ext_vector_type(4)));
constexpr int kReadUnroll = 8;
constexpr int kReadThreads = 256;

__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const u32v4_t* __restrict__ p,
                                                                   size_t n16,
                                                                   unsigned int* __restrict__ sink) {
    const size_t step = (size_t)gridDim.x * kReadThreads * kReadUnroll;
    unsigned int acc = 0;
    for (size_t base = (size_t)blockIdx.x * kReadThreads * kReadUnroll + threadIdx.x; base < n16;
         base += step) {
        u32v4_t v[kReadUnroll];
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) {
            const size_t i = base + (size_t)u * kReadThreads;
            v[u] = i < n16 ? __builtin_nontemporal_load(p + i) : u32v4_t{0, 0, 0, 0};
        }
#pragma unroll
        for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    if (acc == 0x9E3779B9u) *sink = acc;
}

__global__ __launch_bounds__(kReadThreads) void stream_read1_kernel(const u32v4_t* __restrict__ p,
                                                                    size_t n16,
                                                                    unsigned int* __restrict__ sink) {
    const size_t i = (size_t)blockIdx.x * kReadThreads + threadIdx.x;
    if (i < n16) {
        const u32v4_t v = __builtin_nontemporal_load(p + i);
        const unsigned int acc = v.x ^ v.y ^ v.z ^ v.w;
        if (acc == 0x9E3779B9u) *sink = acc;
    }
}

constexpr size_t kReadOnePerThreadMax = (size_t)512 << 20;

}  // namespace nvfp4

using namespace nvfp4;

extern "C" int nvfp4_stream_read(const void* buf_dev, size_t bytes, unsigned int* sink_dev,
                                 void* stream) {
    clear_error();
    if (!buf_dev) return set_error(NVFP4_EINVAL, "buf: NULL");
    if ((uintptr_t)buf_dev & 15) return set_error(NVFP4_EINVAL, "buf: not 16-byte aligned");
    if (bytes == 0 || bytes % 16) return set_error(NVFP4_EINVAL, "bytes: %zu is not a positive multiple of 16", bytes);
    if (!sink_dev) return set_error(NVFP4_EINVAL, "sink: NULL");
    if ((uintptr_t)sink_dev & 3) return set_error(NVFP4_EINVAL, "sink: not 4-byte aligned");
    const size_t n16 = bytes / 16;
    if (bytes <= kReadOnePerThreadMax) {
        hipLaunchKernelGGL(stream_read1_kernel, dim3((unsigned)((n16 + kReadThreads - 1) / kReadThreads)),
                           dim3(kReadThreads), 0, (hipStream_t)stream, (const u32v4_t*)buf_dev, n16,
                           sink_dev);
        NVFP4_HIP(hipGetLastError());
        return NVFP4_OK;
    }
    const size_t per_block = (size_t)kReadThreads * kReadUnroll;
    size_t blocks = (n16 + per_block - 1) / per_block;
    const size_t cap = (size_t)4 * device_cus();
    if (blocks > cap) blocks = cap;
    hipLaunchKernelGGL(stream_read_kernel, dim3((unsigned)blocks), dim3(kReadThreads), 0,
                       (hipStream_t)stream, (const u32v4_t*)buf_dev, n16, sink_dev);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}
