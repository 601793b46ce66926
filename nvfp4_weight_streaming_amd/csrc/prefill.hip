// Prefill GEMM (M > 8): a dense bf16 MFMA contraction over dequantised tiles.
//
// "Ignis" README, "The decode round": prefill runs in chunks interleaved with
// the decode rounds; at chunk sizes (thousands of rows) the NVFP4 GEMM is no
// longer bound by streaming the weights but by the matrix cores, so here every
// weight is dequantised once per block tile into LDS as exact bf16 and the
// block runs v_mfma_f32_32x32x16_bf16 over it.
//
// Dequantisation: w = E2M1 * E4M3 is exact in bf16 (at most 6 significant
// bits).  v_cvt_scalef32_pk_f32_fp4 (scale 1) gives the E2M1 values in fp32,
// one fp32 multiply applies the E4M3 block scale, and the conversion to bf16
// is exact.  The per-tensor fp32 scale is applied to the fp32 accumulators in
// the epilogue.
//
// Tiling: block tile 256 (rows of activations) x 256 (outputs) x 128 (K, one
// 128-value slice of the packed layout, so the weights are read as stored);
// 8 waves as 2 x 4, each owning 128 x 64 outputs as 4 x 2 MFMA tiles of 32 x 32
// (128 fp32 accumulators per lane).  The next K tile is loaded into registers
// while the current one is multiplied; LDS holds one activation tile and one
// dequantised weight tile.
#include "decode_device.h"

namespace nvfp4 {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

constexpr int kPBM = 256, kPBN = 256, kPBK = 128;
constexpr int kPThreads = 512;
constexpr int kPStride = kPBK + 8;  // LDS row: 128 bf16 + 16 B pad

// Register-held next tile: activations (8 x 16 B per thread) and packed
// weights (2 x 16 B of codes and 2 scale words per thread).
struct PTile {
    uint4 a[8];
    uint4 c[2];
    uint32_t s[2];
};

__device__ __forceinline__ void p_load(PTile& t, const uint16_t* __restrict__ act,
                                       const uint4* __restrict__ codes,
                                       const uint8_t* __restrict__ scales, int M, int K, int nsb,
                                       int n_tiles, int m0, int nt0, int kt) {
    const int k0 = kt * kPBK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int idx = threadIdx.x + i * kPThreads;  // 256 rows x 16 vectors
        const int r = idx >> 4, c = idx & 15;
        const int m = min(m0 + r, M - 1);
        const int k = min(k0 + 8 * c, K - 8);
        t.a[i] = *(const uint4*)(act + (size_t)m * K + k);
    }
    const int sb = k0 / kSuperK, kb = (k0 % kSuperK) / 128;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = threadIdx.x + i * kPThreads;  // 16 column tiles x 64 lanes
        const int tl = idx >> 6, lane = idx & 63;
        const int nt = min(nt0 + tl, n_tiles - 1);
        t.c[i] = codes[((size_t)nt * nsb + sb) * 256 + kb * 64 + lane];
        const int col = lane & 15, p = (lane >> 4) >> 1;
        t.s[i] = *(const uint32_t*)(scales + ((size_t)nt * nsb + sb) * kScaleBytesPerSuper +
                                    (col * 2 + p) * 16 + kb * 4);
    }
}

// 2 codes (byte B of w) times scale sc -> 2 bf16 packed in one word.
template <int B>
__device__ __forceinline__ uint32_t dequant2(uint32_t w, float sc) {
    const f32x2 v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
    const __bf16 lo = (__bf16)(v[0] * sc);
    const __bf16 hi = (__bf16)(v[1] * sc);
    uint16_t ul, uh;
    __builtin_memcpy(&ul, &lo, 2);
    __builtin_memcpy(&uh, &hi, 2);
    return (uint32_t)ul | ((uint32_t)uh << 16);
}

// 8 codes (one 4-byte word, low nibble first) times scale sc -> 8 bf16.
__device__ __forceinline__ uint4 dequant8(uint32_t w, float sc) {
    return make_uint4(dequant2<0>(w, sc), dequant2<1>(w, sc), dequant2<2>(w, sc),
                      dequant2<3>(w, sc));
}

// Step S of a packed 16-byte lane chunk: k = 32 S + 8 g .. + 7, block
// 2 S + g / 2, whose scale is byte S of the lane's scale word.
template <int S>
__device__ __forceinline__ void dequant_step(__bf16* row, int g, const uint4& cw, uint32_t sw) {
    const uint32_t w = S == 0 ? cw.x : S == 1 ? cw.y : S == 2 ? cw.z : cw.w;
    const float sc = __builtin_amdgcn_cvt_f32_fp8((int)sw, S);
    *(uint4*)(row + 32 * S + 8 * g) = dequant8(w, sc);
}

__device__ __forceinline__ void p_store(const PTile& t, __bf16* la, __bf16* lb, int M, int K,
                                        int m0, int kt) {
    const int k0 = kt * kPBK;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int idx = threadIdx.x + i * kPThreads;
        const int r = idx >> 4, c = idx & 15;
        const bool keep = m0 + r < M && k0 + 8 * c < K;
        uint4 v = t.a[i];
        v.x = keep ? v.x : 0u;
        v.y = keep ? v.y : 0u;
        v.z = keep ? v.z : 0u;
        v.w = keep ? v.w : 0u;
        *(uint4*)(la + r * kPStride + 8 * c) = v;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int idx = threadIdx.x + i * kPThreads;
        const int tl = idx >> 6, lane = idx & 63;
        const int col = lane & 15, g = lane >> 4;
        __bf16* row = lb + (tl * kTileN + col) * kPStride;  // weight row n of the tile
        dequant_step<0>(row, g, t.c[i], t.s[i]);
        dequant_step<1>(row, g, t.c[i], t.s[i]);
        dequant_step<2>(row, g, t.c[i], t.s[i]);
        dequant_step<3>(row, g, t.c[i], t.s[i]);
    }
}

template <bool BF16>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(
    const uint4* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ act, void* __restrict__ out, float ts, int M, int K, int N,
    int nsb, int n_tiles, int mblocks) {
    __shared__ __attribute__((aligned(16))) __bf16 la[kPBM * kPStride];
    __shared__ __attribute__((aligned(16))) __bf16 lb[kPBN * kPStride];

    // Column-block major order with the row blocks of one column block
    // adjacent in blockIdx, so consecutive workgroups share weight tiles.
    const int mb = blockIdx.x % mblocks, nb = blockIdx.x / mblocks;
    const int m0 = mb * kPBM, nt0 = nb * (kPBN / kTileN);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int wm = wave >> 2, wn = wave & 3;  // 2 x 4 waves, 128 x 64 each
    const int ktiles = (K + kPBK - 1) / kPBK;

    f32x16 acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

    PTile t;
    p_load(t, act, codes, scales, M, K, nsb, n_tiles, m0, nt0, 0);
    for (int kt = 0; kt < ktiles; ++kt) {
        __syncthreads();  // previous tile fully read
        p_store(t, la, lb, M, K, m0, kt);
        __syncthreads();
        if (kt + 1 < ktiles) p_load(t, act, codes, scales, M, K, nsb, n_tiles, m0, nt0, kt + 1);
        // 8 MFMA k-steps of 16 over the tile.
        const int r32 = lane & 31, kq = lane >> 5;
#pragma unroll
        for (int ks = 0; ks < kPBK / 16; ++ks) {
            const int kk = 16 * ks + 8 * kq;
            bf16x8 av[4], bv[2];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                av[i] = *(const bf16x8*)(la + (wm * 128 + 32 * i + r32) * kPStride + kk);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                bv[j] = *(const bf16x8*)(lb + (wn * 64 + 32 * j + r32) * kPStride + kk);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[j], acc[i][j], 0,
                                                                        0, 0);
        }
    }

    // Epilogue: C element (row, col) of a 32 x 32 tile in lane l, register r:
    // col = l % 32, row = 8 (r / 4) + 4 (l / 32) + r % 4.
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int n = nt0 * kTileN + wn * 64 + 32 * j + (lane & 31);
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * 128 + 32 * i + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (m < M && n < N) store_out<BF16>(out, (size_t)m * N + n, acc[i][j][r] * ts);
            }
        }
}

int make_prefill_config(int max_M, int K, int N, PrefillConfig* out) {
    (void)K;
    (void)N;
    out->enabled = max_M > NVFP4_DECODE_MAX_M;
    out->ws_bytes = 0;
    return NVFP4_OK;
}

int launch_prefill(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                   float ts, const uint16_t* act, void* out, void* ws, hipStream_t s) {
    (void)ws;
    const int mblocks = (M + kPBM - 1) / kPBM;
    const int nblocks = (p->Np + kPBN - 1) / kPBN;
    const int n_tiles = p->Np / kTileN, nsb = p->Kp / kSuperK;
    const dim3 grid((unsigned)(mblocks * nblocks));
    if (p->out_dtype == NVFP4_OUT_BF16)
        hipLaunchKernelGGL(prefill_kernel<true>, grid, dim3(kPThreads), 0, s, (const uint4*)codes,
                           scales, act, out, ts, M, p->K, p->N, nsb, n_tiles, mblocks);
    else
        hipLaunchKernelGGL(prefill_kernel<false>, grid, dim3(kPThreads), 0, s, (const uint4*)codes,
                           scales, act, out, ts, M, p->K, p->N, nsb, n_tiles, mblocks);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

}  // namespace nvfp4
