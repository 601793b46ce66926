// Device quantiser: fp32 weights -> canonical NVFP4 planes.
//
// The format is the body format of "Models and artifacts" ("The artifact"):
// 4-bit floats (E2M1) with one scale per 16 values; the scale is an E4M3 byte
// and one fp32 factor per tensor covers the E4M3 range.  The recipe: tensor
// scale t = amax/(6*448); block scale (block amax / 6) / t rounded to E4M3
// nearest-even with saturation; each value w / (E4M3 * t) rounded to E2M1
// nearest-even, saturating at 6, sign kept.  Every step is fp32 with IEEE
// round-to-nearest-even (the division is the correctly rounded sequence).
#include "common.h"

namespace nvfp4 {

// Non-negative finite fp32 -> E4M3 (FN) code, nearest-even, saturating at 448.
__device__ __forceinline__ uint32_t e4m3_rne(float x) {
    if (!(x < 448.0f)) return 0x7Eu;  // includes +inf
    if (x < 0.015625f) {              // below the smallest normal 2^-6: steps of 2^-9
        return (uint32_t)rintf(x * 512.0f);  // exact scaling; 8 -> 0x08 = 2^-6
    }
    uint32_t u = __float_as_uint(x);
    int e = (int)(u >> 23) - 127;            // -6 .. 8
    uint32_t man = u & 0x7FFFFFu;
    uint32_t keep = man >> 20, rest = man & 0xFFFFFu;
    uint32_t code = ((uint32_t)(e + 7) << 3) | keep;
    if (rest > 0x80000u || (rest == 0x80000u && (keep & 1u))) code += 1;  // carries into e
    return code;
}

__device__ __forceinline__ float e4m3_to_f32(uint32_t c) {
    uint32_t e = (c >> 3) & 15u, m = c & 7u;
    if (e == 0) return (float)m * 0.001953125f;  // m * 2^-9, exact
    return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// |x| -> E2M1 magnitude code 0..7, nearest-even, saturating at 6.
__device__ __forceinline__ uint32_t e2m1_rne_mag(float a) {
    if (a <= 0.25f) return 0;
    if (a < 0.75f) return 1;
    if (a <= 1.25f) return 2;
    if (a < 1.75f) return 3;
    if (a <= 2.5f) return 4;
    if (a < 3.5f) return 5;
    if (a <= 5.0f) return 6;
    return 7;
}

__global__ void amax_kernel(const float4* __restrict__ w, size_t n4, unsigned int* amax_bits) {
    float m = 0.0f;
    size_t stride = (size_t)gridDim.x * blockDim.x;
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
        float4 v = w[i];
        m = fmaxf(m, fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w))));
    }
    for (int off = 32; off > 0; off >>= 1) m = fmaxf(m, __shfl_xor(m, off, 64));
    __shared__ float part[16];
    int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    if (lane == 0) part[wave] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < (int)(blockDim.x / 64); ++i) m = fmaxf(m, part[i]);
        // non-negative floats order like their bit patterns
        atomicMax(amax_bits, __float_as_uint(m));
    }
}

// One thread per block of 16 values.
__global__ void quantize_kernel(const float4* __restrict__ w, int K, size_t nblocks,
                                const unsigned int* __restrict__ amax_bits,
                                uint2* __restrict__ codes, uint8_t* __restrict__ scales,
                                float* __restrict__ tensor_scale) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    float t = __uint_as_float(*amax_bits) / 2688.0f;
    if (i == 0) *tensor_scale = t;
    if (i >= nblocks) return;
    float v[16];
    for (int q = 0; q < 4; ++q) {
        float4 x = w[i * 4 + q];
        v[4 * q] = x.x; v[4 * q + 1] = x.y; v[4 * q + 2] = x.z; v[4 * q + 3] = x.w;
    }
    float bamax = 0.0f;
    for (int j = 0; j < 16; ++j) bamax = fmaxf(bamax, fabsf(v[j]));
    uint32_t sc = 0;
    if (t > 0.0f) sc = e4m3_rne((bamax / 6.0f) / t);
    float d = e4m3_to_f32(sc) * t;
    uint32_t packed[2] = {0, 0};
    if (d > 0.0f) {
        for (int j = 0; j < 16; ++j) {
            float x = v[j] / d;
            uint32_t c = e2m1_rne_mag(fabsf(x)) | ((__float_as_uint(x) >> 28) & 8u);
            packed[j / 8] |= c << (4 * (j % 8));
        }
    }
    codes[i] = make_uint2(packed[0], packed[1]);
    scales[i] = (uint8_t)sc;
}

__global__ void zero_word_kernel(unsigned int* p) { *p = 0u; }

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

size_t nvfp4_quantize_workspace_bytes(void) { return 256; }

int nvfp4_quantize(const float* w, int K, int N, uint8_t* codes, uint8_t* scales,
                   float* tensor_scale, void* workspace, void* stream) {
    clear_error();
    if (K < 16 || K % 16 != 0) return set_error(NVFP4_EINVAL, "K: %d is not a positive multiple of 16", K);
    if (N < 1) return set_error(NVFP4_EINVAL, "N: %d < 1", N);
    if (!w) return set_error(NVFP4_EINVAL, "w: NULL");
    if (!codes) return set_error(NVFP4_EINVAL, "codes: NULL");
    if (!scales) return set_error(NVFP4_EINVAL, "scales: NULL");
    if (!tensor_scale) return set_error(NVFP4_EINVAL, "tensor_scale: NULL");
    if (!workspace) return set_error(NVFP4_EINVAL, "workspace: NULL");
    if (((uintptr_t)w & 15) || ((uintptr_t)codes & 7) || ((uintptr_t)tensor_scale & 3) ||
        ((uintptr_t)workspace & 3))
        return set_error(NVFP4_EINVAL, "w/codes/tensor_scale/workspace: misaligned (need 16/8/4/4 bytes)");
    hipStream_t s = (hipStream_t)stream;
    unsigned int* amax = (unsigned int*)workspace;
    size_t n4 = (size_t)N * K / 4, nblocks = (size_t)N * K / 16;
    hipLaunchKernelGGL(zero_word_kernel, dim3(1), dim3(1), 0, s, amax);
    NVFP4_HIP(hipGetLastError());
    size_t g = (n4 + 255) / 256;
    if (g > 8192) g = 8192;
    hipLaunchKernelGGL(amax_kernel, dim3((unsigned)g), dim3(256), 0, s, (const float4*)w, n4, amax);
    NVFP4_HIP(hipGetLastError());
    hipLaunchKernelGGL(quantize_kernel, dim3((unsigned)((nblocks + 255) / 256)), dim3(256), 0, s,
                       (const float4*)w, K, nblocks, amax, (uint2*)codes, scales, tensor_scale);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

}  // extern "C"
