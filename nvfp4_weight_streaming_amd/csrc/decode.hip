// Decode GEMM: M <= 8 lanes served by one pass over NVFP4 weights.
//
// "Ignis" README, "The decode round": all decode lanes share one pass over the
// weights, so the round runs at the card's memory bandwidth ("Models and
// artifacts", "What differs, side by side": decode is bound by streaming the
// weights).  Every weight byte is read from HBM once per call; activations
// (at most 8 x K bf16) are staged once per workgroup in LDS.
//
// gfx950 mapping.  One wave owns a tile of 16 output columns and walks a K
// slice with v_mfma_f32_16x16x32_bf16:
//   B operand (32 k x 16 columns): the wave's weights.  Lane l holds column
//     l%16 and the K octet g = l/16 of each 32-k step: 4 code bytes, turned
//     into 8 exact bf16 values by v_cvt_scalef32_pk_bf16_fp4 with scale 1.
//     (That instruction applies only the exponent of its scale operand, so the
//     E4M3 block scale, which has mantissa bits, is applied separately.)
//   A operand (16 rows x 32 k): rows 0..7 carry the 8 lanes' activations for
//     the first 16-k block of the step (octets g = 0, 1) and zeros for the
//     second; rows 8..15 carry them for the second block (g = 2, 3) and zeros
//     for the first.  Each MFMA therefore returns, for every (lane, column),
//     the two 16-value block sums separately: output rows 4g..4g+3 of lane l
//     belong to block g/2, whose E4M3 scale the lane multiplies in with one
//     fp32 FMA per row.  Products are exact (bf16 x E2M1 fits the MFMA's fp32
//     product), block sums and the scaled accumulation are fp32.
//   The two row halves are added with one cross-lane exchange at the end.
// K is split over workgroups when the column count alone cannot fill the
// chip; partial sums go to a workspace and the last workgroup of a column
// group (an atomic counter) adds them in split order, so results are
// deterministic.  Workgroups of one column group are placed on one XCD
// (blockIdx % 8 selects the XCD), so their partials meet in one L2.
#include "common.h"

namespace nvfp4 {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;

constexpr int kLdsPad = 8;         // bf16 elements of padding per LDS row
constexpr int kMaxSlice = 5 * kSuperK;  // largest K slice one workgroup stages

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float x) {
    uint32_t u = __float_as_uint(x);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40u);  // quiet NaN
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

template <bool BF16>
__device__ __forceinline__ void store_out(void* out, size_t idx, float v) {
    if (BF16)
        ((uint16_t*)out)[idx] = f32_to_bf16_rne(v);
    else
        ((float*)out)[idx] = v;
}

// 8 E2M1 codes (4 bytes, low nibble first) -> 8 bf16 values in k order.
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16(uint32_t w) {
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// The packed bytes one wave streams per 512-k superblock: 4 code chunks (16 B
// per lane each, 4 MFMA steps apiece) and one 16-byte scale word per lane.
struct Chunk {
    uint4 c[4];
    uint4 s;
};

__device__ __forceinline__ void load_chunk(Chunk& x, const uint4* cp, const uint4* sp) {
    x.c[0] = cp[0];
    x.c[1] = cp[64];
    x.c[2] = cp[128];
    x.c[3] = cp[192];
    x.s = sp[0];
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// 128 k: four independent MFMAs (one per 32-k step), then the block scales.
// a: this lane's A-operand pointer for the first step of the 128.
__device__ __forceinline__ void kb_steps(float (&acc)[4], const uint4& cw, uint32_t sw,
                                         const __bf16* a) {
    f32x4 r[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8 av = *(const bf16x8*)(a + 32 * s);
        const bf16x8 bv = e2m1x8_to_bf16(word(cw, s));
        r[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
    const float s0 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 0);
    const float s1 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 1);
    const float s2 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 2);
    const float s3 = __builtin_amdgcn_cvt_f32_fp8((int)sw, 3);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        acc[j] = __builtin_fmaf(s0, r[0][j], acc[j]);
        acc[j] = __builtin_fmaf(s1, r[1][j], acc[j]);
        acc[j] = __builtin_fmaf(s2, r[2][j], acc[j]);
        acc[j] = __builtin_fmaf(s3, r[3][j], acc[j]);
    }
}

__device__ __forceinline__ void chunk_steps(float (&acc)[4], const Chunk& x, const __bf16* a) {
    kb_steps(acc, x.c[0], x.s.x, a);
    kb_steps(acc, x.c[1], x.s.y, a + 128);
    kb_steps(acc, x.c[2], x.s.z, a + 256);
    kb_steps(acc, x.c[3], x.s.w, a + 384);
}

template <int WAVES, bool BF16>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(
    const uint4* __restrict__ codes, const uint4* __restrict__ scales,
    const uint16_t* __restrict__ act, void* __restrict__ out, float* __restrict__ partial,
    unsigned int* __restrict__ counters, float ts, int M, int K, int N, int nsb,
    int sb_per_split, int splits, int n_groups, int n_tiles) {
    extern __shared__ uint4 lds_raw[];
    __shared__ int s_last;
    constexpr int kCols = WAVES * kTileN;

    const int b = blockIdx.x;
    const int xcd = b & 7, q = b >> 3;
    const int ng = (q / splits) * 8 + xcd;
    const int split = q - (q / splits) * splits;
    if (ng >= n_groups) return;  // whole workgroup: padding of the column groups to 8
    const int sb0 = split * sb_per_split;
    const int sb1 = min(sb0 + sb_per_split, nsb);
    const int klen = (sb1 - sb0) * kSuperK;
    const int stride = klen + kLdsPad;
    const int k0 = sb0 * kSuperK;
    __bf16* lds = (__bf16*)lds_raw;  // rows 0..M-1: activations; row M: zeros

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nt = ng * WAVES + wave;
    const int col = lane & 15, g = lane >> 4;
    const bool active = nt < n_tiles;
    const uint4* cp = codes + ((size_t)(active ? nt : 0) * nsb + sb0) * 256 + lane;
    const uint4* sp = scales + ((size_t)(active ? nt : 0) * nsb + sb0) * 32 + col * 2 + (g >> 1);
    // The first superblock's weights do not depend on the activations: issue
    // their loads before staging.
    Chunk A, B;
    if (active) load_chunk(A, cp, sp);

    // Stage this K slice of the activations (and one zero row) in LDS.
    const int noct = klen / 8;
    for (int idx = threadIdx.x; idx < (M + 1) * noct; idx += WAVES * 64) {
        int r = idx / noct, oct = idx - r * noct;
        int k = k0 + 8 * oct;
        uint4 v = make_uint4(0, 0, 0, 0);
        if (r < M && k < K) v = *(const uint4*)(act + (size_t)r * K + k);
        *(uint4*)(lds + r * stride + 8 * oct) = v;
    }
    __syncthreads();

    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (active) {
        // A-operand row of this lane: activation row `col` for its block half
        // (col < 8 pairs with octets 0,1; col >= 8 with octets 2,3), else zeros.
        const int m = col & 7;
        const bool live = ((col >> 3) == (g >> 1)) && (m < M);
        const __bf16* ap = lds + (live ? m : M) * stride + 8 * g;
        // Ping-pong over superblocks: the next one's loads are in flight while
        // this one computes.  The prefetch is unconditional (on the last
        // superblock it re-reads the current one, which the caches serve) so
        // the compiler can count outstanding loads exactly.
        int left = sb1 - sb0;  // superblocks still to compute, A loaded
        while (true) {
            int nx = left > 1 ? 1 : 0;
            load_chunk(B, cp + 256 * nx, sp + 32 * nx);
            chunk_steps(acc, A, ap);
            if (--left == 0) break;
            cp += 256;
            sp += 32;
            ap += kSuperK;
            nx = left > 1 ? 1 : 0;
            load_chunk(A, cp + 256 * nx, sp + 32 * nx);
            chunk_steps(acc, B, ap);
            if (--left == 0) break;
            cp += 256;
            sp += 32;
            ap += kSuperK;
        }
    }
    // Lanes g and g+2 hold the same (row, column) for the two block halves.
    for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], 32, 64);

    if (splits == 1) {
        if (lane < 32 && nt < n_tiles) {
            const int n = nt * kTileN + col;
            for (int j = 0; j < 4; ++j) {
                const int m = 4 * g + j;
                if (m < M && n < N) store_out<BF16>(out, (size_t)m * N + n, acc[j] * ts);
            }
        }
        return;
    }

    // Split K: publish this slice's partial sums, the last slice reduces.
    float* pbase = partial + (size_t)(ng * splits + split) * 8 * kCols;
    if (lane < 32 && nt < n_tiles) {
        for (int j = 0; j < 4; ++j) {
            const int m = 4 * g + j;
            if (m < M) pbase[m * kCols + wave * kTileN + col] = acc[j];
        }
    }
    __threadfence();
    __syncthreads();
    if (threadIdx.x == 0) {
        unsigned int old = atomicAdd(&counters[ng], 1u);
        s_last = (old == (unsigned int)(splits - 1));
    }
    __syncthreads();
    if (!s_last) return;
    __threadfence();
    const float* gbase = partial + (size_t)ng * splits * 8 * kCols;
    for (int idx = threadIdx.x; idx < M * kCols; idx += WAVES * 64) {
        const int m = idx / kCols, c = idx - m * kCols;
        const int n = ng * kCols + c;
        float sum = 0.f;
        for (int sp = 0; sp < splits; ++sp)
            sum += __builtin_nontemporal_load(gbase + (size_t)(sp * 8 + m) * kCols + c);
        if (n < N) store_out<BF16>(out, (size_t)m * N + n, sum * ts);
    }
    if (threadIdx.x == 0) counters[ng] = 0u;  // leave the workspace zeroed
}

// ---- plan ----------------------------------------------------------------------

int make_decode_config(int K, int N, int max_M, const nvfp4_gemm_config* cfg, DecodeConfig* d) {
    (void)max_M;
    int waves = (cfg && cfg->waves) ? cfg->waves : 4;
    if (waves != 2 && waves != 4 && waves != 8)
        return set_error(NVFP4_EINVAL, "config.waves: %d is not 2, 4 or 8", waves);
    const int n_tiles = padded_n(N) / kTileN;
    const int nsb = padded_k(K) / kSuperK;
    const int n_groups = (n_tiles + waves - 1) / waves;
    const int ng8 = round_up(n_groups, 8);
    const int max_sb = kMaxSlice / kSuperK;
    int splits;
    if (cfg && cfg->split_k) {
        if (cfg->split_k < 1) return set_error(NVFP4_EINVAL, "config.split_k: %d < 1", cfg->split_k);
        splits = cfg->split_k < nsb ? cfg->split_k : nsb;
    } else {
        // Aim for about four workgroups per CU (256 CUs).
        splits = (1024 + ng8 - 1) / ng8;
        if (splits > nsb) splits = nsb;
        if (splits < 1) splits = 1;
    }
    int sb_per = (nsb + splits - 1) / splits;
    if (sb_per > max_sb) sb_per = max_sb;
    splits = (nsb + sb_per - 1) / sb_per;
    d->waves = waves;
    d->splits = splits;
    d->sb_per_split = sb_per;
    d->n_groups = n_groups;
    d->grid = ng8 * splits;
    d->lds_bytes = (NVFP4_DECODE_MAX_M + 1) * (sb_per * kSuperK + kLdsPad) * 2;
    if (splits > 1) {
        size_t part = (size_t)ng8 * splits * 8 * waves * kTileN * sizeof(float);
        d->counter_off = (part + 255) / 256 * 256;
        d->ws_bytes = d->counter_off + ((size_t)ng8 * sizeof(unsigned int) + 255) / 256 * 256;
    } else {
        d->counter_off = 0;
        d->ws_bytes = 0;
    }
    return NVFP4_OK;
}

template <int WAVES, bool BF16>
static int launch_t(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                    float ts, const uint16_t* act, void* out, void* ws, hipStream_t s) {
    const DecodeConfig& d = p->dec;
    const int lds = (M + 1) * (d.sb_per_split * kSuperK + kLdsPad) * 2;
    float* partial = (float*)ws;
    unsigned int* counters = ws ? (unsigned int*)((char*)ws + d.counter_off) : nullptr;
    hipLaunchKernelGGL((decode_kernel<WAVES, BF16>), dim3(d.grid), dim3(WAVES * 64), lds, s,
                       (const uint4*)codes, (const uint4*)scales, act, out, partial, counters, ts,
                       M, p->K, p->N, p->Kp / kSuperK, d.sb_per_split, d.splits, d.n_groups,
                       p->Np / kTileN);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

template <bool BF16>
static int launch_w(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                    float ts, const uint16_t* act, void* out, void* ws, hipStream_t s) {
    switch (p->dec.waves) {
        case 2: return launch_t<2, BF16>(p, M, codes, scales, ts, act, out, ws, s);
        case 4: return launch_t<4, BF16>(p, M, codes, scales, ts, act, out, ws, s);
        default: return launch_t<8, BF16>(p, M, codes, scales, ts, act, out, ws, s);
    }
}

int launch_decode(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                  float ts, const uint16_t* act, void* out, void* ws, hipStream_t s) {
    const size_t esz = p->out_dtype == NVFP4_OUT_BF16 ? 2 : 4;
    // Rows beyond 8 (when no prefill kernel applies) run as further weight passes.
    for (int m0 = 0; m0 < M; m0 += NVFP4_DECODE_MAX_M) {
        const int mm = M - m0 < NVFP4_DECODE_MAX_M ? M - m0 : NVFP4_DECODE_MAX_M;
        const uint16_t* a = act + (size_t)m0 * p->K;
        void* o = (char*)out + (size_t)m0 * p->N * esz;
        int st = p->out_dtype == NVFP4_OUT_BF16
                     ? launch_w<true>(p, mm, codes, scales, ts, a, o, ws, s)
                     : launch_w<false>(p, mm, codes, scales, ts, a, o, ws, s);
        if (st) return st;
    }
    return NVFP4_OK;
}

}  // namespace nvfp4
