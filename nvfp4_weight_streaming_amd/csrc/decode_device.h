// Device building blocks of the decode GEMM, shared by the split-K kernel
// (decode.hip) and the streaming kernels (stream.hip).  The operand mapping
// is described at the top of decode.hip.
#pragma once

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

// s_waitcnt immediates: vmcnt(n) with the other counters untouched; lgkmcnt(0).
constexpr int vmcnt_imm(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kLgkmcnt0 = 0xC07F;

// A barrier without the memory fence of __syncthreads: that fence would also
// wait for direct-to-LDS copies just issued.  The caller states with explicit
// waits what must be complete.
__device__ __forceinline__ void barrier_nofence() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Marks registers as redefined at this point (no instruction is emitted), so
// that work on them cannot be hoisted above the wait that precedes it.  Used
// after a window's final wait, where every load is complete: left free to move,
// the conversions of a window that both sides of a branch compute were hoisted
// above the branch, holding every converted value at once (190 registers).
__device__ __forceinline__ void opaque(uint32_t& v) { asm volatile("" : "+v"(v)); }
__device__ __forceinline__ void opaque(uint4& v) {
    asm volatile("" : "+v"(v.x), "+v"(v.y), "+v"(v.z), "+v"(v.w));
}

// 8 E2M1 codes (4 bytes, low nibble first) -> 8 bf16 values in k order.
__device__ __forceinline__ bf16x8 e2m1x8_to_bf16(uint32_t w) {
    bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 0);
    bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 1);
    bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 2);
    bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, 1.0f, 3);
    return bf16x8{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 E2M1 codes times the block scale sc -> 8 bf16 values in k order.  Exact:
// an E2M1 value has at most 2 significant bits and an E4M3 scale 4, so the
// fp32 product has at most 6 and converts to bf16 without rounding (and the
// exponent range of E2M1 x E4M3, 2^-10 .. 2688, is inside bf16's).
typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
template <int B>
__device__ __forceinline__ uint32_t e2m1x2_scaled(uint32_t w, float sc) {
    const auto v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, B);
    const f32x2v x = {v[0] * sc, v[1] * sc};
    const bf16x2v b = __builtin_convertvector(x, bf16x2v);
    uint32_t r;
    __builtin_memcpy(&r, &b, 4);
    return r;
}
__device__ __forceinline__ bf16x8 e2m1x8_scaled_bf16(uint32_t w, float sc) {
    const uint32_t r[4] = {e2m1x2_scaled<0>(w, sc), e2m1x2_scaled<1>(w, sc),
                           e2m1x2_scaled<2>(w, sc), e2m1x2_scaled<3>(w, sc)};
    bf16x8 v;
    __builtin_memcpy(&v, r, 16);
    return v;
}

// Activation row carried by A-operand row i (and i + 8) of the split-A MFMA:
// 2 (i mod 4) + i / 4.  Output row 4 g + j of a lane (g < 2) then belongs to
// activation row 2 j + g, so with M rows only j < ceil(M / 2) are live in any
// lane: kLiveJ(M) block-scale FMAs per MFMA instead of 4.
__device__ __forceinline__ int act_row(int i) { return 2 * (i & 3) + (i >> 2); }
__host__ __device__ constexpr int kLiveJ(int M) { return M >= 8 ? 4 : (M + 1) / 2; }

// The packed bytes one wave streams per 512-k superblock: 4 code chunks (16 B
// per lane each, 4 MFMA steps apiece) and one 16-byte scale word per lane.
struct Chunk {
    uint4 c[4];
    uint4 s;
};

// Weights are read once per call: non-temporal loads (the streaming hint), so
// they do not displace the activations and partial sums from the caches.
// Measured: 4% off the 27B-class round at M = 1 and at M = 8.
typedef unsigned int u32v4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const uint4* p) {
    const u32v4 v = __builtin_nontemporal_load((const u32v4*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ void load_chunk(Chunk& x, const uint4* cp, const uint4* sp) {
    x.c[0] = load_stream(cp);
    x.c[1] = load_stream(cp + 64);
    x.c[2] = load_stream(cp + 128);
    x.c[3] = load_stream(cp + 192);
    x.s = load_stream(sp);
}

__device__ __forceinline__ uint32_t word(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// 128 k: four independent MFMAs (one per 32-k step), then the block scales.
// a: this lane's A-operand pointer for the first step of the 128.
// J: output rows 0 .. J - 1 of each lane's four (4 g + j) are scaled and
// accumulated; with at most J activation rows the others hold only the
// zero rows' products and are never read.
template <int J = 4>
__device__ __forceinline__ void kb_steps(float (&acc)[4], const uint4& cw, uint32_t sw,
                                         const __bf16* a) {
    f32x4 r[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) {
        const bf16x8 av = *(const bf16x8*)(a + 32 * s);
        const bf16x8 bv = e2m1x8_to_bf16(word(cw, s));
        r[s] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
    }
    // the four E4M3 block scales, two per conversion
    const f32x2v s01 = __builtin_amdgcn_cvt_pk_f32_fp8((int)sw, false);
    const f32x2v s23 = __builtin_amdgcn_cvt_pk_f32_fp8((int)sw, true);
    const float s0 = s01[0], s1 = s01[1], s2 = s23[0], s3 = s23[1];
#pragma unroll
    for (int j = 0; j < J; ++j) {
        acc[j] = __builtin_fmaf(s0, r[0][j], acc[j]);
        acc[j] = __builtin_fmaf(s1, r[1][j], acc[j]);
        acc[j] = __builtin_fmaf(s2, r[2][j], acc[j]);
        acc[j] = __builtin_fmaf(s3, r[3][j], acc[j]);
    }
}

template <int J = 4>
__device__ __forceinline__ void chunk_steps(float (&acc)[4], const Chunk& x, const __bf16* a) {
    kb_steps<J>(acc, x.c[0], x.s.x, a);
    kb_steps<J>(acc, x.c[1], x.s.y, a + 128);
    kb_steps<J>(acc, x.c[2], x.s.z, a + 256);
    kb_steps<J>(acc, x.c[3], x.s.w, a + 384);
}

// Stage rows 0..7 of an activation K slice plus one zero row (row 8) into LDS
// (row stride kStride bf16).  ACTIVATION loads are issued here and written
// after `between()` runs, so the caller can issue its weight loads in between
// and they stay in flight.  Loads are unconditional with clamped addresses;
// rows >= M, k >= K and the zero row are stored as zeros.
template <int kThreads, int NCH, int kStride>
struct ActStage {
    static constexpr int kVecs = 9 * NCH * (kSuperK / 8);
    static constexpr int kPer = (kVecs + kThreads - 1) / kThreads;
    uint4 v[kPer];

    __device__ __forceinline__ void load(const uint16_t* act, int M, int K, int k0, int nch) {
        const int row_vecs = nch * (kSuperK / 8);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            const int r = idx / row_vecs, oct = idx - r * row_vecs;
            const int m = min(r, M - 1);
            const int k = min(k0 + 8 * oct, K - 8);
            v[i] = *(const uint4*)(act + (size_t)m * K + k);
        }
    }

    __device__ __forceinline__ void store(__bf16* lds, int M, int K, int k0, int nch) const {
        const int row_vecs = nch * (kSuperK / 8);
#pragma unroll
        for (int i = 0; i < kPer; ++i) {
            const int idx = threadIdx.x + i * kThreads;
            const int r = idx / row_vecs, oct = idx - r * row_vecs;
            if (r < 9) {
                const int k = k0 + 8 * oct;
                const bool keep = r < M && k < K;
                uint4 x = v[i];
                x.x = keep ? x.x : 0u;
                x.y = keep ? x.y : 0u;
                x.z = keep ? x.z : 0u;
                x.w = keep ? x.w : 0u;
                *(uint4*)(lds + r * kStride + 8 * oct) = x;
            }
        }
    }
};

// Sums, in split order, the `splits` partial sums of one column group (layout
// [split][kSplitRows rows][kCols]) for the outputs idx = threadIdx.x + r * kThreads,
// r < kR (row idx / kCols, column idx % kCols); only idx < n_out are valid.
// L2_LOCAL: the partials were written with plain stores into this XCD's L2;
// else with device-coherent stores, and they are read device-coherently.
// Every load of a batch of kSB = kBatch / kR splits, for all kR outputs, is
// issued before any is added, so a batch costs one memory round trip.  Within a wave that
// has valid outputs the output index is clamped to n_out - 1 (repeated
// addresses within a wave cost one request).
template <int kCols, int kThreads, int kR, bool L2_LOCAL, int kSplitRows = 8, int kBatch = 16>
__device__ __forceinline__ void sum_partials(const float* gbase, int splits, int n_out,
                                             float (&sum)[kR]) {
    static_assert(kR >= 1 && kR <= kBatch, "1 .. kBatch outputs per thread");
    constexpr int kSB = kBatch / kR;  // splits per batch: kBatch values in flight
#pragma unroll
    for (int r = 0; r < kR; ++r) sum[r] = 0.f;
    for (int s0 = 0; s0 < splits; s0 += kSB) {
        float v[kR][kSB];
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            // Waves with no valid output in this block issue nothing.
            const int wave0 = __builtin_amdgcn_readfirstlane((int)(threadIdx.x & ~63u)) + r * kThreads;
            const int idx = min((int)threadIdx.x + r * kThreads, n_out - 1);
            const int mm = idx / kCols, c = idx - mm * kCols;
#pragma unroll
            for (int t = 0; t < kSB; ++t) {
                v[r][t] = 0.f;
                if (wave0 < n_out && s0 + t < splits) {
                    const int off = ((s0 + t) * kSplitRows + mm) * kCols + c;
                    v[r][t] = L2_LOCAL ? gbase[off]
                                       : __hip_atomic_load(gbase + off, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
#pragma unroll
        for (int r = 0; r < kR; ++r)
#pragma unroll
            for (int t = 0; t < kSB; ++t)
                if (s0 + t < splits) sum[r] += v[r][t];
    }
}

}  // namespace nvfp4
