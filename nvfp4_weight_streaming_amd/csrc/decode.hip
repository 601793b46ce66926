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
constexpr int kMaxChunks = 4;  // superblocks of 512 k per wave (all loaded up front)

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

// One workgroup = WAVES column tiles (one per wave) x one K slice of up to
// NCH superblocks.  Every load a wave will need is issued before it computes
// anything: first its share of the activation slice, then all of its weight
// chunks; the activations are written to LDS as soon as they land (in-order
// completion counting lets the weights stay in flight), and the MFMA work on
// chunk c waits only for chunk c.
template <int WAVES, int NCH, bool BF16>
__global__ __launch_bounds__(WAVES * 64) void decode_kernel(
    const uint4* __restrict__ codes, const uint4* __restrict__ scales,
    const uint16_t* __restrict__ act, void* __restrict__ out, float* __restrict__ partial,
    unsigned int* __restrict__ counters, float ts, int M, int K, int N, int nsb, int splits,
    int n_groups, int n_tiles) {
    constexpr int kThreads = WAVES * 64;
    constexpr int kStride = NCH * kSuperK + kLdsPad;          // LDS row, bf16 elements
    constexpr int kVecs = 9 * NCH * (kSuperK / 8);            // 8 rows + zero row, 16 B each
    constexpr int kVecPerThread = (kVecs + kThreads - 1) / kThreads;
    constexpr int kCols = WAVES * kTileN;
    __shared__ __attribute__((aligned(16))) __bf16 lds[9 * kStride];
    __shared__ int s_last;

    const int b = blockIdx.x;
    const int xcd = b & 7, q = b >> 3;
    const int ng = (q / splits) * 8 + xcd;
    const int split = q - (q / splits) * splits;
    if (ng >= n_groups) return;  // whole workgroup: padding of the column groups to 8
    const int sb0 = split * NCH;
    const int nch = min(NCH, nsb - sb0);  // superblocks in this slice (>= 1)
    const int k0 = sb0 * kSuperK;
    const int row_vecs = nch * (kSuperK / 8);

    // 1. This thread's share of the activation slice (rows 0..7 and the zero
    //    row 8).  Loads are unconditional with clamped addresses; rows >= M,
    //    k >= K and the zero row are replaced by zeros when stored.
    uint4 av[kVecPerThread];
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
        const int idx = threadIdx.x + i * kThreads;
        const int r = idx / row_vecs, oct = idx - r * row_vecs;
        const int m = min(r, M - 1);
        const int k = min(k0 + 8 * oct, K - 8);
        av[i] = *(const uint4*)(act + (size_t)m * K + k);
    }

    // 2. All weight chunks of this wave's column tile and K slice.
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int nt = min(ng * WAVES + wave, n_tiles - 1);
    const int col = lane & 15, g = lane >> 4;
    const uint4* cp = codes + ((size_t)nt * nsb + sb0) * 256 + lane;
    const uint4* sp = scales + ((size_t)nt * nsb + sb0) * 32 + col * 2 + (g >> 1);
    Chunk w[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int cc = min(c, nch - 1);  // a short slice re-reads its last chunk (cache hit)
        load_chunk(w[c], cp + 256 * cc, sp + 32 * cc);
    }

    // 3. Activations to LDS.
#pragma unroll
    for (int i = 0; i < kVecPerThread; ++i) {
        const int idx = threadIdx.x + i * kThreads;
        const int r = idx / row_vecs, oct = idx - r * row_vecs;
        if (r < 9) {
            const int k = k0 + 8 * oct;
            const bool keep = r < M && k < K;
            uint4 v = av[i];
            v.x = keep ? v.x : 0u;
            v.y = keep ? v.y : 0u;
            v.z = keep ? v.z : 0u;
            v.w = keep ? v.w : 0u;
            *(uint4*)(lds + r * kStride + 8 * oct) = v;
        }
    }
    __syncthreads();

    // 4. MFMA over the slice.  A-operand row of this lane: activation row
    //    `col` for its block half (col < 8 pairs with octets 0,1; col >= 8
    //    with octets 2,3), else the zero row.
    const int m = col & 7;
    const bool live = ((col >> 3) == (g >> 1)) && (m < M);
    const __bf16* ap = lds + (live ? m : 8) * kStride + 8 * g;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if (c < nch) chunk_steps(acc, w[c], ap + c * kSuperK);

    // Lanes g and g+2 hold the same (row, column) for the two block halves.
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], 32, 64);
    const bool mine = lane < 32 && ng * WAVES + wave < n_tiles;

    if (splits == 1) {
        if (mine) {
            const int n = nt * kTileN + col;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int mm = 4 * g + j;
                if (mm < M && n < N) store_out<BF16>(out, (size_t)mm * N + n, acc[j] * ts);
            }
        }
        return;
    }

    // Split K.  The slices of one column group run on one XCD (blockIdx % 8).
    // Partial sums are written with agent-coherent (write-through) stores and
    // read back with agent-coherent loads, so the hand-off needs only the
    // store-completion wait before the counter increment -- no write-back of
    // the whole L2, which an agent-scope fence would cost every workgroup.
    float* pbase = partial + (size_t)(ng * splits + split) * 8 * kCols;
    if (mine) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int mm = 4 * g + j;
            if (mm < M)
                __hip_atomic_store(pbase + mm * kCols + wave * kTileN + col, acc[j],
                                   __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned int old =
            __hip_atomic_fetch_add(&counters[ng], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == (unsigned int)(splits - 1));
    }
    __syncthreads();
    if (!s_last) return;
    const float* gbase = partial + (size_t)ng * splits * 8 * kCols;
    for (int idx = threadIdx.x; idx < M * kCols; idx += kThreads) {
        const int mm = idx / kCols, c = idx - mm * kCols;
        const int n = ng * kCols + c;
        float sum = 0.f;
        for (int sp2 = 0; sp2 < splits; ++sp2)
            sum += __hip_atomic_load(gbase + (size_t)(sp2 * 8 + mm) * kCols + c, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
        if (n < N) store_out<BF16>(out, (size_t)mm * N + n, sum * ts);
    }
    if (threadIdx.x == 0)  // leave the counter zeroed for the next run
        __hip_atomic_store(&counters[ng], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---- plan ----------------------------------------------------------------------

int make_decode_config(int K, int N, int max_M, const nvfp4_gemm_config* cfg, DecodeConfig* d) {
    (void)max_M;
    int waves = (cfg && cfg->waves) ? cfg->waves : 4;
    if (waves != 4 && waves != 8)
        return set_error(NVFP4_EINVAL, "config.waves: %d is not 4 or 8", waves);
    const int n_tiles = padded_n(N) / kTileN;
    const int nsb = padded_k(K) / kSuperK;
    const int n_groups = (n_tiles + waves - 1) / waves;
    const int ng8 = round_up(n_groups, 8);
    int chunks;
    if (cfg && cfg->split_k) {
        if (cfg->split_k < 1) return set_error(NVFP4_EINVAL, "config.split_k: %d < 1", cfg->split_k);
        int sk = cfg->split_k < nsb ? cfg->split_k : nsb;
        chunks = (nsb + sk - 1) / sk;
        if (chunks > kMaxChunks)
            return set_error(NVFP4_EINVAL, "config.split_k: %d leaves %d superblocks of 512 per "
                             "slice, more than %d", cfg->split_k, chunks, kMaxChunks);
    } else if (cfg && cfg->chunks) {
        if (cfg->chunks < 1 || cfg->chunks > kMaxChunks)
            return set_error(NVFP4_EINVAL, "config.chunks: %d outside [1, %d]", cfg->chunks, kMaxChunks);
        chunks = cfg->chunks < nsb ? cfg->chunks : nsb;
    } else {
        // The largest slice (fewest partial sums) that still gives about
        // 1024 workgroups (four per CU on 256 CUs).
        chunks = kMaxChunks < nsb ? kMaxChunks : nsb;
        while (chunks > 1 && (long)ng8 * ((nsb + chunks - 1) / chunks) < 1024) --chunks;
    }
    const int splits = (nsb + chunks - 1) / chunks;
    d->waves = waves;
    d->chunks = chunks;
    d->splits = splits;
    d->n_groups = n_groups;
    d->grid = ng8 * splits;
    if (splits > 1) {
        d->counter_bytes = ((size_t)ng8 * sizeof(unsigned int) + 255) / 256 * 256;
        d->partial_bytes = (size_t)ng8 * splits * 8 * waves * kTileN * sizeof(float);
    } else {
        d->counter_bytes = 0;
        d->partial_bytes = 0;
    }
    d->ws_bytes = d->counter_bytes + d->partial_bytes;
    return NVFP4_OK;
}

template <int WAVES, int NCH, bool BF16>
static int launch_t(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                    float ts, const uint16_t* act, void* out, void* ws, size_t partial_off,
                    hipStream_t s) {
    const DecodeConfig& d = p->dec;
    unsigned int* counters = (unsigned int*)ws;
    float* partial = ws ? (float*)((char*)ws + partial_off) : nullptr;
    hipLaunchKernelGGL((decode_kernel<WAVES, NCH, BF16>), dim3(d.grid), dim3(WAVES * 64), 0, s,
                       (const uint4*)codes, (const uint4*)scales, act, out, partial, counters, ts,
                       M, p->K, p->N, p->Kp / kSuperK, d.splits, d.n_groups, p->Np / kTileN);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

template <int WAVES, bool BF16>
static int launch_c(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                    float ts, const uint16_t* act, void* out, void* ws, size_t po,
                    hipStream_t s) {
    switch (p->dec.chunks) {
        case 1: return launch_t<WAVES, 1, BF16>(p, M, codes, scales, ts, act, out, ws, po, s);
        case 2: return launch_t<WAVES, 2, BF16>(p, M, codes, scales, ts, act, out, ws, po, s);
        case 3: return launch_t<WAVES, 3, BF16>(p, M, codes, scales, ts, act, out, ws, po, s);
        default: return launch_t<WAVES, 4, BF16>(p, M, codes, scales, ts, act, out, ws, po, s);
    }
}

template <bool BF16>
static int launch_w(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                    float ts, const uint16_t* act, void* out, void* ws, size_t po,
                    hipStream_t s) {
    if (p->dec.waves == 8) return launch_c<8, BF16>(p, M, codes, scales, ts, act, out, ws, po, s);
    return launch_c<4, BF16>(p, M, codes, scales, ts, act, out, ws, po, s);
}

int launch_decode(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                  float ts, const uint16_t* act, void* out, void* ws, size_t partial_off,
                  hipStream_t s) {
    const size_t esz = p->out_dtype == NVFP4_OUT_BF16 ? 2 : 4;
    // Rows beyond 8 (when no prefill kernel applies) run as further weight passes.
    for (int m0 = 0; m0 < M; m0 += NVFP4_DECODE_MAX_M) {
        const int mm = M - m0 < NVFP4_DECODE_MAX_M ? M - m0 : NVFP4_DECODE_MAX_M;
        const uint16_t* a = act + (size_t)m0 * p->K;
        void* o = (char*)out + (size_t)m0 * p->N * esz;
        int st = p->out_dtype == NVFP4_OUT_BF16
                     ? launch_w<true>(p, mm, codes, scales, ts, a, o, ws, partial_off, s)
                     : launch_w<false>(p, mm, codes, scales, ts, a, o, ws, partial_off, s);
        if (st) return st;
    }
    return NVFP4_OK;
}

}  // namespace nvfp4
