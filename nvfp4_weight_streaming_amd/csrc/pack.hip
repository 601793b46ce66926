// Pack-time permutation of the canonical NVFP4 planes into the gfx950 layout.
//
// "Models and artifacts" ("The artifact") states that the engine's kernels read
// the weight planes as stored, with no conversion at load.  Here the only
// change at load is a bit-exact permutation, done once on the device, that
// puts every byte a wave needs for 4 MFMA steps into one 16-byte-per-lane
// (1 KiB per wave) coalesced load; the bytes themselves are unchanged.  The
// layout is described next to kTileN / kSuperK in common.h.
#include "common.h"

namespace nvfp4 {

// One thread per packed 16-byte lane chunk of codes.
__global__ void pack_codes_kernel(const uint8_t* __restrict__ canon, uint4* __restrict__ packed,
                                  int K, int N, int nsb, size_t total) {
    size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= total) return;
    size_t tile_sb = c / 256;
    int within = (int)(c % 256);
    int nt = (int)(tile_sb / nsb), sb = (int)(tile_sb % nsb);
    int kb = within / 64, lane = within % 64;
    int n = nt * kTileN + (lane & 15), g = lane >> 4;
    uint32_t w[4];
    for (int s = 0; s < 4; ++s) {
        int k0 = sb * kSuperK + kb * 128 + 32 * s + 8 * g;
        w[s] = 0;
        if (n < N && k0 < K)
            w[s] = *(const uint32_t*)(canon + (size_t)n * (K / 2) + k0 / 2);
    }
    packed[c] = make_uint4(w[0], w[1], w[2], w[3]);
}

// One thread per packed 16-byte scale chunk: (tile, superblock, column, half).
__global__ void pack_scales_kernel(const uint8_t* __restrict__ canon, uint4* __restrict__ packed,
                                   int K, int N, int nsb, size_t total) {
    size_t c = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (c >= total) return;
    size_t tile_sb = c / 32;
    int within = (int)(c % 32);
    int nt = (int)(tile_sb / nsb), sb = (int)(tile_sb % nsb);
    int col = within >> 1, p = within & 1;
    int n = nt * kTileN + col;
    int nblk = K / 16;
    uint8_t b[16];
    for (int kb = 0; kb < 4; ++kb)
        for (int s = 0; s < 4; ++s) {
            int blk = sb * (kSuperK / 16) + kb * 8 + 2 * s + p;
            b[kb * 4 + s] = (n < N && blk < nblk) ? canon[(size_t)n * nblk + blk] : 0;
        }
    uint32_t w[4];
    for (int i = 0; i < 4; ++i)
        w[i] = (uint32_t)b[4 * i] | ((uint32_t)b[4 * i + 1] << 8) | ((uint32_t)b[4 * i + 2] << 16) |
               ((uint32_t)b[4 * i + 3] << 24);
    packed[c] = make_uint4(w[0], w[1], w[2], w[3]);
}

// Inverse: one thread per canonical 4-byte code word (8 codes).
__global__ void unpack_codes_kernel(const uint8_t* __restrict__ packed, uint8_t* __restrict__ canon,
                                    int K, int N, int nsb, size_t total) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    int words_per_row = K / 8;
    int n = (int)(i / words_per_row);
    int k0 = (int)(i % words_per_row) * 8;
    int nt = n / kTileN, col = n % kTileN;
    int sb = k0 / kSuperK, r = k0 % kSuperK;
    int kb = r / 128, s = (r % 128) / 32, g = (r % 32) / 8;
    int lane = g * 16 + col;
    size_t off = (((size_t)nt * nsb + sb) * 256 + kb * 64 + lane) * 16 + 4 * s;
    *(uint32_t*)(canon + (size_t)n * (K / 2) + k0 / 2) = *(const uint32_t*)(packed + off);
}

// Inverse: one thread per canonical scale byte.
__global__ void unpack_scales_kernel(const uint8_t* __restrict__ packed,
                                     uint8_t* __restrict__ canon, int K, int N, int nsb,
                                     size_t total) {
    size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= total) return;
    int nblk = K / 16;
    int n = (int)(i / nblk), blk = (int)(i % nblk);
    int nt = n / kTileN, col = n % kTileN;
    int sb = blk / (kSuperK / 16), r = blk % (kSuperK / 16);
    int kb = r / 8, s = (r % 8) / 2, p = r % 2;
    size_t off = ((size_t)nt * nsb + sb) * kScaleBytesPerSuper + (col * 2 + p) * 16 + kb * 4 + s;
    canon[i] = packed[off];
}

static int validate_layout(int K, int N) {
    if (K < 16 || K % 16 != 0) return set_error(NVFP4_EINVAL, "K: %d is not a positive multiple of 16", K);
    if (N < 1) return set_error(NVFP4_EINVAL, "N: %d < 1", N);
    if (K > (1 << 24)) return set_error(NVFP4_EUNSUPPORTED, "K: %d above 2^24", K);
    if (N > (1 << 26)) return set_error(NVFP4_EUNSUPPORTED, "N: %d above 2^26", N);
    return NVFP4_OK;
}

static unsigned blocks_for(size_t n, int threads) { return (unsigned)((n + threads - 1) / threads); }

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

size_t nvfp4_packed_code_bytes(int K, int N) {
    if (K < 16 || K % 16 || N < 1 || K > (1 << 24) || N > (1 << 26)) return 0;
    return (size_t)padded_n(N) / kTileN * (padded_k(K) / kSuperK) * kCodeBytesPerSuper;
}

size_t nvfp4_packed_scale_bytes(int K, int N) {
    if (K < 16 || K % 16 || N < 1 || K > (1 << 24) || N > (1 << 26)) return 0;
    return (size_t)padded_n(N) / kTileN * (padded_k(K) / kSuperK) * kScaleBytesPerSuper;
}

int nvfp4_pack(const uint8_t* codes, const uint8_t* scales, int K, int N, uint8_t* codes_packed,
               uint8_t* scales_packed, void* stream) {
    clear_error();
    int st = validate_layout(K, N);
    if (st) return st;
    if (!codes || !scales || !codes_packed || !scales_packed)
        return set_error(NVFP4_EINVAL, "%s: NULL",
                         !codes ? "codes" : !scales ? "scales" : !codes_packed ? "codes_packed" : "scales_packed");
    if (((uintptr_t)codes & 3) || ((uintptr_t)codes_packed & 15) || ((uintptr_t)scales_packed & 15))
        return set_error(NVFP4_EINVAL, "codes/codes_packed/scales_packed: misaligned (need 4/16/16 bytes)");
    hipStream_t s = (hipStream_t)stream;
    int nsb = padded_k(K) / kSuperK;
    size_t tiles = (size_t)padded_n(N) / kTileN;
    size_t nc = tiles * nsb * 256, ns = tiles * nsb * 32;
    hipLaunchKernelGGL(pack_codes_kernel, dim3(blocks_for(nc, 256)), dim3(256), 0, s, codes,
                       (uint4*)codes_packed, K, N, nsb, nc);
    NVFP4_HIP(hipGetLastError());
    hipLaunchKernelGGL(pack_scales_kernel, dim3(blocks_for(ns, 256)), dim3(256), 0, s, scales,
                       (uint4*)scales_packed, K, N, nsb, ns);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

int nvfp4_unpack(const uint8_t* codes_packed, const uint8_t* scales_packed, int K, int N,
                 uint8_t* codes, uint8_t* scales, void* stream) {
    clear_error();
    int st = validate_layout(K, N);
    if (st) return st;
    if (!codes || !scales || !codes_packed || !scales_packed)
        return set_error(NVFP4_EINVAL, "%s: NULL",
                         !codes ? "codes" : !scales ? "scales" : !codes_packed ? "codes_packed" : "scales_packed");
    if (((uintptr_t)codes & 3) || ((uintptr_t)codes_packed & 15) || ((uintptr_t)scales_packed & 15))
        return set_error(NVFP4_EINVAL, "codes/codes_packed/scales_packed: misaligned (need 4/16/16 bytes)");
    hipStream_t s = (hipStream_t)stream;
    int nsb = padded_k(K) / kSuperK;
    size_t nc = (size_t)N * (K / 8), ns = (size_t)N * (K / 16);
    hipLaunchKernelGGL(unpack_codes_kernel, dim3(blocks_for(nc, 256)), dim3(256), 0, s,
                       codes_packed, codes, K, N, nsb, nc);
    NVFP4_HIP(hipGetLastError());
    hipLaunchKernelGGL(unpack_scales_kernel, dim3(blocks_for(ns, 256)), dim3(256), 0, s,
                       scales_packed, scales, K, N, nsb, ns);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

}  // extern "C"
