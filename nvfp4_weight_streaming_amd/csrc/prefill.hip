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
// Tiling: block tile 256 (rows of activations) x 256 (outputs), K in stages of
// 64.  LDS holds three stages of 256 x 64 activations and two of 256 x 64
// dequantised weights (160 KiB, one workgroup per compute unit).  8 waves as
// 2 x 4, each owning 128 x 64 outputs as 4 x 2 MFMA tiles of 32 x 32 (128 fp32
// accumulators per lane; two waves per SIMD, so 256 registers per lane in all).
// Activations run two
// stages ahead (direct-to-LDS copies); weights run two stages ahead in
// registers and are dequantised into LDS one stage ahead, the conversion
// interleaved with the multiplies; one barrier per stage.  LDS rows are 128
// bytes (8 segments of 16): segment j of row r sits in slot j ^ ((r / 2) % 8),
// so the 16 rows one operand read pass touches cover all banks once.
//
// Last round: the tiles beyond a multiple of the compute units' count would
// leave most of the chip idle in a last, partial round.  They are split along
// K instead, S pieces each (S = compute units / leftover tiles, at most one
// piece per 4 stages); every piece writes its fp32 accumulators to the
// workspace, and a second kernel adds the S partial sums of each output in
// piece order, applies the tensor scale and stores.  The pieces come first in
// the grid; the stream order makes every partial complete before the sum.
#include "decode_device.h"

namespace nvfp4 {

typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;

constexpr int kPBK = 64;          // K per stage
constexpr int kPWaves = 8;        // waves per workgroup: 2 x 4 of 128 x 64 outputs
constexpr int kPThreads = kPWaves * 64;
// s_waitcnt vmcnt(n) encodings (vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt fields at their maxima do not wait).
constexpr int vmcnt_enc(int n) { return (n & 15) | ((n >> 4) << 14) | 0x0F70; }
constexpr int kPWaitLgkm0 = 0xC07F;  // lgkmcnt(0)

struct PrefillLds {
    __bf16 a[3][256 * kPBK];  // activations [row][k], swizzled segments: 3 stages
    __bf16 b[2][256 * kPBK];  // dequantised weights [output][k], swizzled segments
};

// Slot of segment `seg` in LDS row `row`: seg ^ ((row / 2) % 8).  A 16-byte
// operand read serves 16 lanes (16 consecutive rows, one segment) per pass;
// with this key those 16 reads cover all 64 banks once.
__device__ __forceinline__ int swz_key(int row) { return (row >> 1) & 7; }
__device__ __forceinline__ int swz(int row, int seg) { return row * kPBK + 8 * (seg ^ swz_key(row)); }

// 8 codes (one 4-byte word, low nibble first) times scale sc -> 8 bf16.
// (exact: e2m1x2_scaled)
__device__ __forceinline__ uint4 dequant8(uint32_t w, float sc) {
    return make_uint4(e2m1x2_scaled<0>(w, sc), e2m1x2_scaled<1>(w, sc), e2m1x2_scaled<2>(w, sc),
                      e2m1x2_scaled<3>(w, sc));
}

// Global memory is read through buffer resources (base and size in scalar
// registers, a 32-bit offset per lane, a scalar offset per stage): compact
// addressing, and reads past the resource's size return zero.
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
constexpr int kRawBuffer = 0x00020000;  // buffer resource word 3: raw 32-bit data

__device__ __forceinline__ __amdgpu_buffer_rsrc_t prefill_rsrc(const void* base, size_t bytes) {
    const int n = bytes > 0x7FFFFFFFu ? 0x7FFFFFFF : (int)bytes;
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, kRawBuffer);
}

// Activations of one stage (BM rows x 64 k) go straight from global memory to
// LDS: one direct-to-LDS load moves 8 rows of 128 bytes; lane i fills slot
// i % 8 of row i / 8 with the segment that belongs there, (i % 8) ^ key(row).
// The resource covers rows m0 .. M-1 (rows past M read zero); k past K reads
// the next row (finite values; the weights past K are zero).  The NW waves
// take kL = BM / (8 NW) loads each; voff[i] is this lane's offset for load i.
template <int BM, int NW>
struct PrefillA {
    static constexpr int kL = BM / (8 * NW);
    __amdgpu_buffer_rsrc_t rsrc;
    int voff[kL];

    __device__ __forceinline__ void init(const uint16_t* act, int M, int K, int m0, int wave,
                                         int lane) {
        rsrc = prefill_rsrc(act + (size_t)m0 * K, (size_t)(M - m0) * K * 2);
#pragma unroll
        for (int i = 0; i < kL; ++i) {
            const int r = (wave * kL + i) * 8 + (lane >> 3);
            voff[i] = r * K * 2 + 16 * ((lane & 7) ^ swz_key(r));
        }
    }

    __device__ __forceinline__ void copy(__bf16* la, int kt, int wave) const {
#pragma unroll
        for (int i = 0; i < kL; ++i) {
            const int r0 = (wave * kL + i) * 8;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rsrc, (__attribute__((address_space(3))) void*)(la + r0 * kPBK), 16, voff[i],
                kt * kPBK * 2, 0, 0);
        }
    }
};

// Weights of one stage held in registers between their global loads and
// their (dequantising) LDS stores: BN / 16 column tiles x 64 lane slots of
// the packed layout; a stage of 64 k is half of a slot's 16 bytes (steps 2h,
// 2h+1 of 128-k chunk kb) plus bytes 2h, 2h+1 of its scale word.  The resources
// start at the block's first column tile and end at the last real one, so
// tiles past N read zero.
template <int BN, int NW>
struct PrefillB {
    static constexpr int kB = BN / 16 * 64 / (NW * 64);
    __amdgpu_buffer_rsrc_t rc, rs;
    int coff[kB], soff[kB];

    __device__ __forceinline__ void init(const uint8_t* codes, const uint8_t* scales, int nsb,
                                         int n_tiles, int nt0, int tid) {
        const size_t tiles = (size_t)(n_tiles - nt0);
        rc = prefill_rsrc(codes + (size_t)nt0 * nsb * kCodeBytesPerSuper,
                          tiles * nsb * kCodeBytesPerSuper);
        rs = prefill_rsrc(scales + (size_t)nt0 * nsb * kScaleBytesPerSuper,
                          tiles * nsb * kScaleBytesPerSuper);
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            const int u = tid + NW * 64 * i;
            const int t = u >> 6, ls = u & 63;
            const int col = ls & 15, p = (ls >> 4) >> 1;
            coff[i] = t * nsb * kCodeBytesPerSuper + ls * 16;
            soff[i] = t * nsb * kScaleBytesPerSuper + (col * 2 + p) * 16;
        }
    }
};

template <int BN, int NW>
struct PStage {
    static constexpr int kB = BN / 16 * 64 / (NW * 64);
    u32x2 c[kB];
    uint32_t s[kB];

    __device__ __forceinline__ void load(const PrefillB<BN, NW>& B, int kt) {
        const int k0 = kt * kPBK;
        const int sb = k0 / kSuperK, kb = (k0 % kSuperK) / 128, h = (k0 % 128) / 64;
        const int cso = sb * kCodeBytesPerSuper + kb * 1024 + h * 8;
        const int sso = sb * kScaleBytesPerSuper + kb * 4;
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            c[i] = __builtin_amdgcn_raw_buffer_load_b64(B.rc, B.coff[i], cso, 0);
            // the scale word of the whole 128-k chunk (steps 0..3); this
            // stage's two bytes are picked at the store
            s[i] = __builtin_amdgcn_raw_buffer_load_b32(B.rs, B.soff[i], sso, 0);
        }
    }

    // Piece q (0 .. 2 kB - 1) of the dequantised store: lane slot q / 2, word
    // q % 2 (8 values).
    template <int Q>
    __device__ __forceinline__ void store_piece(__bf16* lb, int kt, int tid) const {
        constexpr int i = Q / 2, w = Q % 2;
        const int h = (kt * kPBK % 128) / 64;
        const int u = tid + NW * 64 * i;
        const int ls = u & 63;
        const int col = (u >> 6) * 16 + (ls & 15), g = ls >> 4;
        const int sw = (int)(s[i] >> (16 * h));
        const float sc = __builtin_amdgcn_cvt_f32_fp8(sw, w);
        *(uint4*)(lb + swz(col, 4 * w + g)) = dequant8(w ? c[i].y : c[i].x, sc);
    }

    __device__ __forceinline__ void store(__bf16* lb, int kt, int tid) const {
        const int h = (kt * kPBK % 128) / 64;
#pragma unroll
        for (int i = 0; i < kB; ++i) {
            const int u = tid + NW * 64 * i;
            const int ls = u & 63;
            const int col = (u >> 6) * 16 + (ls & 15), g = ls >> 4;
            const int sw = (int)(s[i] >> (16 * h));
            const f32x2v s01 = __builtin_amdgcn_cvt_pk_f32_fp8(sw, false);
            const float s0 = s01[0], s1 = s01[1];
            // step 2h: k = 8 g .. 8 g + 7 of the stage; step 2h + 1: 32 further
            *(uint4*)(lb + swz(col, g)) = dequant8(c[i].x, s0);
            *(uint4*)(lb + swz(col, 4 + g)) = dequant8(c[i].y, s1);
        }
    }
};

// The MFMAs of one stage (64 k = 4 steps of 16) for this wave's (BM/64) x
// (BN/128) tiles, with the dequantised store of the next weight stage (`nx`,
// into the other LDS buffer) spread over the steps: after each step's
// multiplies are issued the wave converts and stores a share of it while the
// matrix cores work.  The operands of step ks + 1 are read before the
// multiplies of step ks.
template <int BM, int BN, int NW, int Q>
__device__ __forceinline__ void prefill_store_share(const PStage<BN, NW>& nx, __bf16* lbn,
                                                    int ktn, int ks, int tid) {
    constexpr int kPieces = 2 * PStage<BN, NW>::kB;
    // pieces ks * kPieces / 4 .. (ks + 1) * kPieces / 4 - 1
    if constexpr (Q < kPieces) {
        if (Q * 4 / kPieces == ks) nx.template store_piece<Q>(lbn, ktn, tid);
    }
}

// NW waves as (NW / 4) x 4: wave (wm, wn) owns rows wm * BM / (NW / 4) and
// columns wn * BN / 4, as TI x TJ MFMA tiles of 32 x 32.
constexpr int ptiles_i(int BM, int NW) { return BM / (NW / 4) / 32; }
constexpr int ptiles_j(int BN) { return BN / 4 / 32; }
template <int BM, int BN, int NW>
struct PTiles {
    static constexpr int WM = NW / 4;
    static constexpr int TI = ptiles_i(BM, NW), TJ = ptiles_j(BN);
};

template <int BM, int BN, int NW>
__device__ __forceinline__ void prefill_mma(
    f32x16 (&acc)[ptiles_i(BM, NW)][ptiles_j(BN)], const __bf16* la,
    const __bf16* lb, const PStage<BN, NW>& nx, __bf16* lbn, int ktn, int wm, int wn, int r32,
    int half, int tid) {
    constexpr int TI = PTiles<BM, BN, NW>::TI, TJ = PTiles<BM, BN, NW>::TJ;
    constexpr int WM = PTiles<BM, BN, NW>::WM;
    bf16x8 av[2][TI], bv[2][TJ];
    auto read = [&](int ks, int buf) {
        const int seg = 2 * ks + half;
#pragma unroll
        for (int i = 0; i < TI; ++i)
            av[buf][i] = *(const bf16x8*)(la + swz(wm * (BM / WM) + 32 * i + r32, seg));
#pragma unroll
        for (int j = 0; j < TJ; ++j)
            bv[buf][j] = *(const bf16x8*)(lb + swz(wn * (BN / 4) + 32 * j + r32, seg));
    };
    read(0, 0);
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int ks = 0; ks < kPBK / 16; ++ks) {
        const int buf = ks & 1;
        if (ks + 1 < kPBK / 16) read(ks + 1, buf ^ 1);
#pragma unroll
        for (int i = 0; i < TI; ++i)
#pragma unroll
            for (int j = 0; j < TJ; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[buf][i], bv[buf][j],
                                                                    acc[i][j], 0, 0, 0);
        prefill_store_share<BM, BN, NW, 0>(nx, lbn, ktn, ks, tid);
        prefill_store_share<BM, BN, NW, 1>(nx, lbn, ktn, ks, tid);
        prefill_store_share<BM, BN, NW, 2>(nx, lbn, ktn, ks, tid);
        prefill_store_share<BM, BN, NW, 3>(nx, lbn, ktn, ks, tid);
    }
    __builtin_amdgcn_s_setprio(0);
}

// This wave's share of the BM x BN block tile at (m0, n0) over K stages
// kt0 .. kt1 - 1 (kt1 > kt0), accumulated into acc from zero; wave w owns
// rows (w / 4) * BM / (NW / 4) and columns (w % 4) * BN/4, as TI x TJ MFMA
// tiles of 32 x 32 (PTiles).  On return, re-reads of the last stage may still
// be in flight into L (the prefetch runs two stages past the end): a caller
// that reuses L waits for them and for every wave first.  tid is the thread
// index (a caller looping over tiles passes it opaque, so that the addresses
// derived from it are not computed once before that loop and held).
template <int BM, int BN, int NW>
__device__ __forceinline__ void prefill_accumulate(
    f32x16 (&acc)[ptiles_i(BM, NW)][ptiles_j(BN)], PrefillLds& L,
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ act, int M, int K, int nsb, int n_tiles, int m0, int n0,
    int kt0, int kt1, int tid) {
    constexpr int TI = PTiles<BM, BN, NW>::TI, TJ = PTiles<BM, BN, NW>::TJ;
    // loads per thread per stage: weights (a code and a scale load per lane
    // slot) and activation copies
    constexpr int kWL = 2 * PStage<BN, NW>::kB, kAL = PrefillA<BM, NW>::kL;
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 2, wn = wave & 3;
    const int nt0 = n0 / kTileN;
    const int nks = kt1 - kt0;
    // absolute stage of relative stage u, clamped to the last one
    auto at = [&](int u) { return kt0 + min(u, nks - 1); };

    // (whole zero vectors: element-wise zeroing would read the previous
    // values, keeping a previous tile's accumulators alive into this one)
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) acc[i][j] = f32x16{};

    // Activations run two stages ahead in three LDS buffers (relative stage
    // u in buffer u % 3); weights run two stages ahead in registers (st0 /
    // st1 alternately hold stages u + 1 and u + 2) and are dequantised into
    // two LDS buffers (stage u in buffer u % 2).  Stages past the end re-read
    // the last one into buffers nobody reads again.
    PrefillA<BM, NW> A;
    A.init(act, M, K, m0, wave, lane);
    PrefillB<BN, NW> B;
    B.init(codes, scales, nsb, n_tiles, nt0, tid);
    PStage<BN, NW> st0, st1;
    A.copy(L.a[0], at(0), wave);
    st0.load(B, at(0));
    __builtin_amdgcn_s_waitcnt(vmcnt_enc(0));
    st0.store(L.b[0], at(0), tid);
    // The loads in flight when the loop starts are issued in the order the
    // loop itself leaves them at the end of each stage (weights of stage 1,
    // activation copy of stage 1, weights of stage 2), so the compiler's own
    // waits inside the loop are exact: a different order here merged with
    // the loop's at its head and made each stage wait for the next stage's
    // weights before dequantising.
    st0.load(B, at(1));
    A.copy(L.a[1], at(1), wave);
    st1.load(B, at(2));
    __builtin_amdgcn_s_waitcnt(kPWaitLgkm0);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    const int r32 = lane & 31, half = lane >> 5;
    // Per stage, issued in this order: activation copy of stage u + 2
    // (BM / 64 loads), the multiplies with the dequantised store of stage
    // u + 1 interleaved, the weight loads of stage u + 3 (BN / 64 loads).
    // Before the barrier the copy of stage u + 1 (issued one stage earlier)
    // must have landed: the loads after it may still be in flight.
    auto stage = [&](int u, PStage<BN, NW>& next, int u_next) {
        A.copy(L.a[(u + 2) % 3], at(u + 2), wave);
        __builtin_amdgcn_sched_barrier(0);
        prefill_mma<BM, BN, NW>(acc, L.a[u % 3], L.b[u & 1], next, L.b[(u + 1) & 1], at(u + 1),
                                wm, wn, r32, half, tid);
        __builtin_amdgcn_sched_barrier(0);
        next.load(B, at(u_next));
        __builtin_amdgcn_sched_barrier(0);
        // Then the barrier, without a memory fence (a fence would also wait
        // for the copy of stage u + 2 just issued): this wave's LDS stores
        // are complete, and the compiler may not move memory accesses across.
        __builtin_amdgcn_s_waitcnt(vmcnt_enc(2 * kWL + kAL));
        __builtin_amdgcn_s_waitcnt(kPWaitLgkm0);
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
    };
    // Unrolled by two so st0 and st1 keep fixed registers (copying a register
    // set whose loads are in flight would wait for them); an odd last stage
    // runs after the loop.
    int u = 0;
    for (; u + 1 < nks; u += 2) {
        stage(u, st0, u + 3);
        stage(u + 1, st1, u + 4);
    }
    if (u < nks) stage(u, st0, u + 3);
}

// Epilogue of a whole tile: element r of a 32 x 32 MFMA tile in lane l is
// (row 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32); acc * ts to out.
template <int BM, int BN, int NW, bool BF16>
__device__ __forceinline__ void prefill_store_tile(
    const f32x16 (&acc)[ptiles_i(BM, NW)][ptiles_j(BN)], void* __restrict__ out, float ts, int M,
    int N, int m0, int n0) {
    constexpr int TI = PTiles<BM, BN, NW>::TI, TJ = PTiles<BM, BN, NW>::TJ;
    constexpr int WM = PTiles<BM, BN, NW>::WM;
    // (the thread index made opaque here: in a loop over tiles the compiler
    // would otherwise compute these addresses once, before the loop, and
    // hold them in registers through the multiplies)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = tid >> 6, lane = tid & 63;
    const int wm = wave >> 2, wn = wave & 3;
    const int r32 = lane & 31, half = lane >> 5;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j) {
            const int n = n0 + wn * (BN / 4) + 32 * j + r32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int m = m0 + wm * (BM / WM) + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
                if (m < M && n < N) store_out<BF16>(out, (size_t)m * N + n, acc[i][j][r] * ts);
            }
        }
}

// Raw accumulators of a K piece to part (BM * BN floats, in register order:
// float4 ((((w TI + i) TJ + j) 4 + r / 4) 64 + lane) holds elements r .. r + 3
// of lane's MFMA tile (i, j) of wave w).
template <int BM, int BN, int NW>
__device__ __forceinline__ void prefill_store_piece(
    const f32x16 (&acc)[ptiles_i(BM, NW)][ptiles_j(BN)], float* __restrict__ part) {
    constexpr int TI = PTiles<BM, BN, NW>::TI, TJ = PTiles<BM, BN, NW>::TJ;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const int v = (((wave * TI + i) * TJ + j) * 4 + rq) * 64 + lane;
                *(float4*)(part + 4 * v) = make_float4(acc[i][j][4 * rq], acc[i][j][4 * rq + 1],
                                                       acc[i][j][4 * rq + 2], acc[i][j][4 * rq + 3]);
            }
}

// One block tile over K stages kt0 .. kt1 - 1, in a workgroup of its own.
// With part == nullptr the tile covers all of K and stores acc * ts to out;
// otherwise it stores its raw accumulators to part (prefill_store_piece).
template <int BM, int BN, int NW, bool BF16>
__device__ __forceinline__ void prefill_tile(PrefillLds& L, const uint8_t* __restrict__ codes,
                                             const uint8_t* __restrict__ scales,
                                             const uint16_t* __restrict__ act,
                                             void* __restrict__ out, float* __restrict__ part,
                                             float ts, int M, int K, int N, int nsb, int n_tiles,
                                             int m0, int n0, int kt0, int kt1) {
    f32x16 acc[ptiles_i(BM, NW)][ptiles_j(BN)];
    prefill_accumulate<BM, BN, NW>(acc, L, codes, scales, act, M, K, nsb, n_tiles, m0, n0, kt0,
                                   kt1, threadIdx.x);
    if (part)
        prefill_store_piece<BM, BN, NW>(acc, part);
    else
        prefill_store_tile<BM, BN, NW, BF16>(acc, out, ts, M, N, m0, n0);
}

constexpr int kPTile = 256;                      // block tile edge (rows and outputs)
constexpr int kPTileFloats = kPTile * kPTile;    // one piece's partial sums
constexpr int kPMinPieceStages = 4;              // K stages per piece, at least

// Tile t covers rows (t % mblocks) * 256 and outputs (t / mblocks) * 256.
// Workgroups 0 .. pieces - 1 are the K pieces of the last n_tail tiles
// (piece b: tile tiles - n_tail + b % n_tail, split b / n_tail, stages
// split * nk / S .. (split + 1) * nk / S - 1; its partial sums at part +
// b * 65536); the rest are whole tiles 0, 1, ...
template <bool BF16>
__global__ __launch_bounds__(kPThreads) void prefill_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ act, void* __restrict__ out, float* __restrict__ part, float ts,
    int M, int K, int N, int nsb, int n_tiles, int mblocks, int tiles, int n_tail, int splits) {
    __shared__ __attribute__((aligned(16))) PrefillLds L;
    const int nk = (K + kPBK - 1) / kPBK;
    const int pieces = n_tail * splits;
    const int b = blockIdx.x;
    if (b < pieces) {
        const int t = tiles - n_tail + b % n_tail, split = b / n_tail;
        prefill_tile<kPTile, kPTile, kPWaves, BF16>(
            L, codes, scales, act, out, part + (size_t)b * kPTileFloats, ts, M, K, N, nsb,
            n_tiles, (t % mblocks) * kPTile, (t / mblocks) * kPTile, split * nk / splits,
            (split + 1) * nk / splits);
    } else {
        const int t = b - pieces;
        prefill_tile<kPTile, kPTile, kPWaves, BF16>(L, codes, scales, act, out, nullptr, ts, M,
                                                    K, N, nsb, n_tiles, (t % mblocks) * kPTile,
                                                    (t / mblocks) * kPTile, 0, nk);
    }
}

// ---- stream-K schedule ----------------------------------------------------------
//
// The tiles' K stages are laid end to end (tile after tile, W = tiles * nk in
// all) and workgroup r of C (one per compute unit) takes the stages r W / C ..
// (r + 1) W / C - 1: every unit gets the same number of stages, with no last
// partial round.  The host takes this schedule when every run holds at least
// half a tile's stages (and one), so a tile is shared by at most three
// consecutive runs.  A run's parts are the last tile it touches if it only
// starts there (its head), the first tile if it does not take all of it (its
// tail), then its whole tiles, in that order, so the hand-offs of shared tiles
// happen early and spread over the run while other workgroups compute.

// Cache policy of the hand-off's stores and loads between XCDs: device scope
// (sc1), so that they bypass the XCDs' non-coherent cached copies.
constexpr int kPDeviceScope = 16;
constexpr int kPWaveFloats = 32 * 32 * PTiles<256, 256, kPWaves>::TI * PTiles<256, 256, kPWaves>::TJ;
constexpr int kPMaxShare = 3;  // runs sharing one tile, at most

// Scalar byte offset of float4 group g (64 lanes) of a slot.
__device__ __forceinline__ int sk_soff(int g) { return 1024 * g; }

// The run holding stage s: the largest q with W q / C <= s.
__device__ __forceinline__ int sk_run_of(long long s, long long W, int C) {
    return (int)(((s + 1) * C - 1) / W);
}

// Slot of run q's part in tile t: 2 q for the tile holding the run's first
// stage, 2 q + 1 for its last tile.
__device__ __forceinline__ int sk_slot(int q, int t, long long W, int C, int nk) {
    return 2 * q + (t == (int)(W * q / C / nk) ? 0 : 1);
}

// Hand-off of a shared tile, wave by wave (wave w of every contributor owns
// the same outputs): the wave stores its accumulators to its slot and, once
// the stores have completed, increments the tile's counter.  The wave that
// finds the other n - 1 increments already there finishes the tile, with a
// sum that is the same float whichever contributor comes last: with two
// terms it adds the other's slot to its registers (own + other in either
// order), with three it adds the three slots in run order, its own included.
// It zeroes the counter again and stores the outputs itself (a store after
// the hand-off, reached from both outcomes, would keep the accumulators
// alive through the loads).  With every contributor on one XCD
// (LOCAL) the slots and the counter live in that XCD's L2: plain stores and
// loads, an agent-scope atomic.  Otherwise the stores and loads are
// device-scope and the counter system-scope (coherent across XCDs).  Slots:
// float4 ((i TJ + j) 4 + r / 4) 64 + lane of slot s, wave w (at (s NW + w)
// kPWaveFloats floats) holds elements r .. r + 3 of lane's MFMA tile (i, j).
template <int BM, int BN, int NW, bool BF16, bool LOCAL>
__device__ __forceinline__ void prefill_handoff(f32x16 (&acc)[ptiles_i(BM, NW)][ptiles_j(BN)],
                                                float* __restrict__ slots,
                                                unsigned int* __restrict__ counters, int ctr,
                                                int me, int n, const int (&slot)[kPMaxShare],
                                                void* __restrict__ out, float ts, int M, int N,
                                                int m0, int n0) {
    constexpr int TI = PTiles<BM, BN, NW>::TI, TJ = PTiles<BM, BN, NW>::TJ;
    constexpr int kF = 32 * 32 * TI * TJ;  // floats per wave
    constexpr int kAux = LOCAL ? 0 : kPDeviceScope;
    // (the thread index opaque, as in prefill_store_tile)
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    auto rsrc_of = [&](int s) {
        return prefill_rsrc(slots + ((size_t)s * NW + wave) * kF, (size_t)kF * 4);
    };
    // (slot indices through scalar registers: the resources must be scalar)
    const int own = __builtin_amdgcn_readfirstlane(me == 0 ? slot[0] : me == 1 ? slot[1] : slot[2]);
    const __amdgpu_buffer_rsrc_t rm = rsrc_of(own);
    // float4 v of a slot at byte 16 lane + sk_soff(v / 64): the lane's part
    // in a vector register, the rest in the instruction's scalar offset (so
    // no per-float4 address registers are held)
    const int voff = 16 * lane;
#pragma unroll
    for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
#pragma unroll
            for (int rq = 0; rq < 4; ++rq) {
                const u32x4 x = {__float_as_uint(acc[i][j][4 * rq]),
                                 __float_as_uint(acc[i][j][4 * rq + 1]),
                                 __float_as_uint(acc[i][j][4 * rq + 2]),
                                 __float_as_uint(acc[i][j][4 * rq + 3])};
                __builtin_amdgcn_raw_buffer_store_b128(x, rm, voff, sk_soff((i * TJ + j) * 4 + rq),
                                                       kAux);
            }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    unsigned int* c = counters + (size_t)ctr * NW + wave;
    unsigned int old = 0;
    if (lane == 0)
        old = LOCAL ? __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                    : __hip_atomic_fetch_add(c, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    old = __builtin_amdgcn_readlane(old, 0);
    asm volatile("" ::: "memory");
    if (old != (unsigned int)(n - 1)) return;  // a later contributor finishes
    if (n == 2) {
        // Two terms: own + other is the same float in either order, so the
        // other's slot is added to the registers.
        const __amdgpu_buffer_rsrc_t ro =
            rsrc_of(__builtin_amdgcn_readfirstlane(me == 0 ? slot[1] : slot[0]));
        constexpr int kB2 = 2;
#pragma unroll
        for (int b0 = 0; b0 < TI * TJ; b0 += kB2) {
            u32x4 x[kB2 * 4];
#pragma unroll
            for (int q = 0; q < kB2 * 4; ++q)
                x[q] = __builtin_amdgcn_raw_buffer_load_b128(ro, voff, sk_soff(b0 * 4 + q), kAux);
#pragma unroll
            for (int q = 0; q < kB2 * 4; ++q) {
                const int i = (b0 + q / 4) / TJ, j = (b0 + q / 4) % TJ, rq = q % 4;
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[i][j][4 * rq + e] += __uint_as_float(x[q][e]);
            }
            asm volatile("" ::: "memory");
        }
        if (lane == 0) {
            if (LOCAL)
                __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            else
                __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        prefill_store_tile<BM, BN, NW, BF16>(acc, out, ts, M, N, m0, n0);
        return;
    }
    // Three terms: all slots in run order, this wave's own included (stored and waited
    // for above: the same values as its registers), so no term depends on
    // which contributor is adding; the sums go straight to the outputs, in
    // batches of kBatch MFMA tiles whose loads are in flight together.
    const __amdgpu_buffer_rsrc_t r0 = rsrc_of(slot[0]), r1 = rsrc_of(slot[1]);
    const __amdgpu_buffer_rsrc_t r2 = rsrc_of(slot[n == 3 ? 2 : 1]);
    constexpr int WM = PTiles<BM, BN, NW>::WM;
    const int wm = wave >> 2, wn = wave & 3, r32 = lane & 31, half = lane >> 5;
    constexpr int kBatch = 2;
    int vo = voff;
#pragma unroll
    for (int b0 = 0; b0 < TI * TJ; b0 += kBatch) {
        u32x4 x0[kBatch * 4], x1[kBatch * 4], x2[kBatch * 4];
#pragma unroll
        for (int q = 0; q < kBatch * 4; ++q) {
            const int so = sk_soff(b0 * 4 + q);
            x0[q] = __builtin_amdgcn_raw_buffer_load_b128(r0, vo, so, kAux);
            x1[q] = __builtin_amdgcn_raw_buffer_load_b128(r1, vo, so, kAux);
            if (n == 3) x2[q] = __builtin_amdgcn_raw_buffer_load_b128(r2, vo, so, kAux);
        }
        float last = 0.f;
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int i = (b0 + u) / TJ, j = (b0 + u) % TJ;
            const int nn = n0 + wn * (BN / 4) + 32 * j + r32;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int q = 4 * u + r / 4, e = r % 4;
                float sum = __uint_as_float(x0[q][e]) + __uint_as_float(x1[q][e]);
                if (n == 3) sum += __uint_as_float(x2[q][e]);
                const int m = m0 + wm * (BM / WM) + 32 * i + 8 * (r >> 2) + 4 * half + (r & 3);
                if (m < M && nn < N) store_out<BF16>(out, (size_t)m * N + nn, sum * ts);
                last = sum;
            }
        }
        // the next batch's offset depends on this batch's sums, so its loads
        // are not issued (and held in registers) before these are done
        asm volatile("" : "+v"(vo) : "v"(last));
    }
    if (lane == 0) {
        if (LOCAL)
            __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_store(c, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// Stream tile t covers rows (t / nblocks) * 256 and outputs (t % nblocks) *
// 256.  Run r covers stages lo .. hi - 1: tiles ta = lo / nk .. tb = (hi - 1)
// / nk, of which ta from stage ka = lo - ta nk and tb up to kb = hi - tb nk.
template <bool BF16>
__global__ __launch_bounds__(kPThreads) void prefill_sk_kernel(
    const uint8_t* __restrict__ codes, const uint8_t* __restrict__ scales,
    const uint16_t* __restrict__ act, void* __restrict__ out, float* __restrict__ slots,
    unsigned int* __restrict__ counters, float ts, int M, int K, int N, int nsb, int n_tiles,
    int nblocks, int tiles, int l2_local) {
    __shared__ __attribute__((aligned(16))) PrefillLds L;
    const int nk = (K + kPBK - 1) / kPBK;
    const long long W = (long long)tiles * nk;
    const int C = (int)gridDim.x;
    // Run r of workgroup b: with C a multiple of 8, the C / 8 workgroups of
    // one XCD (b % 8) take consecutive runs, and the stream holds the tiles
    // row block by row block, so an XCD works on the same rows of
    // activations (kept in its L2) across its column blocks.
    // (l2_local: workgroup b verified to run on XCD b % 8, and C % 8 == 0)
    const int r = C % 8 ? (int)blockIdx.x : (int)(blockIdx.x % 8) * (C / 8) + (int)blockIdx.x / 8;
    const long long lo = W * r / C, hi = W * (r + 1) / C;
    const int ta = (int)(lo / nk), tb = (int)((hi - 1) / nk);
    const int ka = (int)(lo - (long long)ta * nk), kb = (int)(hi - (long long)tb * nk);
    const int sh_b = ta != tb && kb != nk;              // a head in tile tb
    const int sh_a = ka != 0 || (ta == tb && kb != nk);  // a shared part in tile ta
    const int tw0 = ta + sh_a, n_whole = tb - sh_b - tw0 + 1;
    const int n_parts = sh_b + sh_a + (n_whole > 0 ? n_whole : 0);
    f32x16 acc[PTiles<kPTile, kPTile, kPWaves>::TI][PTiles<kPTile, kPTile, kPWaves>::TJ];
    for (int q = 0; q < n_parts; ++q) {
        // part q is of kind 0 (head of tb), 1 (the part of ta) or 2 (whole
        // tile tw0 + q - sh_b - sh_a)
        const int kind = q < sh_b ? 0 : q < sh_b + sh_a ? 1 : 2;
        const int t = kind == 0 ? tb : kind == 1 ? ta : tw0 + (q - sh_b - sh_a);
        const int kt0 = kind == 1 ? ka : 0;
        const int kt1 = kind == 0 || (kind == 1 && ta == tb) ? kb : nk;
        const int m0 = (t / nblocks) * kPTile, n0 = (t % nblocks) * kPTile;
        int tid = threadIdx.x;
        asm volatile("" : "+v"(tid));
        prefill_accumulate<kPTile, kPTile, kPWaves>(acc, L, codes, scales, act, M, K, nsb,
                                                    n_tiles, m0, n0, kt0, kt1, tid);
        // The part ended with a barrier after every wave's last LDS reads;
        // this wave's re-reads past the end (into its own rows and columns
        // of L) must land before the next part's first copies.  Waiting here,
        // before the epilogue, leaves the epilogue's stores in flight.
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        if (kind == 2) {
            prefill_store_tile<kPTile, kPTile, kPWaves, BF16>(acc, out, ts, M, N, m0, n0);
        } else {
            // the runs rf .. rf + n - 1 share tile t; its counter belongs to
            // run rf's slot there
            // (uniform values through scalar registers: the slot addresses
            // make buffer resources, which must be scalar)
            const int rf = __builtin_amdgcn_readfirstlane(sk_run_of((long long)t * nk, W, C));
            const int n = __builtin_amdgcn_readfirstlane(
                sk_run_of((long long)(t + 1) * nk - 1, W, C) - rf + 1);
            int slot[kPMaxShare];
#pragma unroll
            for (int i = 0; i < kPMaxShare; ++i)
                slot[i] = __builtin_amdgcn_readfirstlane(i < n ? sk_slot(rf + i, t, W, C, nk)
                                                               : sk_slot(rf, t, W, C, nk));
            const bool local = l2_local && rf / (C / 8) == (rf + n - 1) / (C / 8);
            if (local)
                prefill_handoff<kPTile, kPTile, kPWaves, BF16, true>(
                    acc, slots, counters, slot[0], r - rf, n, slot, out, ts, M, N, m0, n0);
            else
                prefill_handoff<kPTile, kPTile, kPWaves, BF16, false>(
                    acc, slots, counters, slot[0], r - rf, n, slot, out, ts, M, N, m0, n0);
        }
    }
}

// Sum of the split tiles' partials: thread p of tile q adds float4 p of its
// S pieces in piece order, scales by ts and stores the 4 outputs it maps to
// (the register order prefill_tile stores them in).
constexpr int kPReduceThreads = 256;
template <bool BF16>
__global__ __launch_bounds__(kPReduceThreads) void prefill_reduce_kernel(
    const float* __restrict__ part, void* __restrict__ out, float ts, int M, int N, int mblocks,
    int tiles, int n_tail, int splits) {
    constexpr int kBlocksPerTile = kPTileFloats / 4 / kPReduceThreads;
    constexpr int TI = PTiles<kPTile, kPTile, kPWaves>::TI;
    constexpr int TJ = PTiles<kPTile, kPTile, kPWaves>::TJ;
    constexpr int WM = PTiles<kPTile, kPTile, kPWaves>::WM;
    const int q = blockIdx.x / kBlocksPerTile;
    const int p = (blockIdx.x % kBlocksPerTile) * kPReduceThreads + threadIdx.x;
    const int t = tiles - n_tail + q;
    const int lane = p & 63, rq = (p >> 6) & 3, j = (p >> 8) % TJ, i = (p >> 8) / TJ % TI;
    const int wave = (p >> 8) / (TI * TJ);
    const int wm = wave >> 2, wn = wave & 3;
    const int n = (t / mblocks) * kPTile + wn * (kPTile / 4) + 32 * j + (lane & 31);
    const int m = (t % mblocks) * kPTile + wm * (kPTile / WM) + 32 * i + 8 * rq + 4 * (lane >> 5);
    if (n >= N || m >= M) return;
    // Batches of 8 pieces: every load of a batch is issued before any is
    // added (one memory round trip per batch).
    constexpr int kBatch = 8;
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s0 = 0; s0 < splits; s0 += kBatch) {
        float4 x[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int s = min(s0 + u, splits - 1);
            x[u] = *(const float4*)(part + (size_t)(s * n_tail + q) * kPTileFloats + 4 * p);
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
            if (s0 + u < splits) {
                v.x += x[u].x;
                v.y += x[u].y;
                v.z += x[u].z;
                v.w += x[u].w;
            }
    }
    const float e[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int r = 0; r < 4; ++r)
        if (m + r < M) store_out<BF16>(out, (size_t)(m + r) * N + n, e[r] * ts);
}

// How a run of M rows is laid out over the compute units: the stream-K
// schedule (below), or whole tiles with the tiles beyond whole rounds (one
// tile per compute unit at a time) split along K when at least two pieces
// each fit: n_tail tiles, S pieces each.
struct PrefillSplit {
    int tiles, n_tail, splits;
    bool stream;
};

static PrefillSplit prefill_split(int M, int K, int N, int cus, int schedule) {
    const int mblocks = (M + kPTile - 1) / kPTile, nblocks = (N + kPTile - 1) / kPTile;
    const int nk = (K + kPBK - 1) / kPBK;
    PrefillSplit s{mblocks * nblocks, 0, 1, false};
    const int left = s.tiles % cus;
    // Stream-K applies when every run holds at least half a tile's stages
    // (and one): then at most three runs share a tile.  By default it is
    // taken below one tile per unit when at most 3/4 of the units would have
    // a tile (measured 8-20% faster at 160 and 136 of 256 tiles, 11% slower
    // at 224); with more tiles than units the whole tiles plus K pieces of
    // the last round measured 1-4% faster, so stream-K there only on request.
    const long long per_run = (long long)s.tiles * nk / cus;
    const bool applies = left && per_run >= max(1, (nk + 1) / 2);
    const bool preferred = s.tiles < cus && 4 * s.tiles <= 3 * cus;
    if (applies && (schedule == NVFP4_PREFILL_STREAM_K ||
                    (schedule == NVFP4_PREFILL_AUTO && preferred))) {
        s.stream = true;
        return s;
    }
    const int S = left ? min(cus / left, nk / kPMinPieceStages) : 1;
    if (S >= 2) {
        s.n_tail = left;
        s.splits = S;
    }
    return s;
}

// Workspace of a run: [counters][partial sums] (stream-K: two slots per run,
// and a counter per slot and wave; pieces: no counters, the pieces' partial
// sums).
static void prefill_need(const PrefillSplit& s, int cus, size_t* counters, size_t* partials) {
    if (s.stream) {
        *counters = ((size_t)2 * cus * kPWaves * sizeof(unsigned int) + 255) & ~(size_t)255;
        *partials = (size_t)2 * cus * kPWaves * kPWaveFloats * sizeof(float);
    } else {
        *counters = 0;
        *partials = (size_t)s.n_tail * s.splits * kPTileFloats * sizeof(float);
    }
}

int make_prefill_config(int max_M, int K, int N, const nvfp4_gemm_config* cfg,
                        PrefillConfig* out) {
    out->enabled = max_M > NVFP4_VERIFY_MAX_M;
    out->ws_off = 0;
    out->ws_bytes = 0;
    out->counter_bytes = 0;
    out->schedule = cfg ? cfg->prefill_schedule : 0;
    out->cus = device_cus();
    if (out->schedule < 0 || out->schedule > NVFP4_PREFILL_STREAM_K)
        return set_error(NVFP4_EINVAL, "config.prefill_schedule: %d outside [0, %d]",
                         out->schedule, NVFP4_PREFILL_STREAM_K);
    if (!out->enabled) return NVFP4_OK;
    // The largest counter and partial-sum areas over every M the plan serves
    // (the layout depends on M only through the row blocks).
    size_t part = 0;
    for (int mb = 1; mb <= (max_M + kPTile - 1) / kPTile; ++mb) {
        size_t c = 0, p = 0;
        prefill_need(prefill_split(mb * kPTile, K, N, out->cus, out->schedule), out->cus, &c, &p);
        if (c > out->counter_bytes) out->counter_bytes = c;
        if (p > part) part = p;
    }
    out->ws_bytes = out->counter_bytes + part;
    return NVFP4_OK;
}

void prefill_ws_need(const nvfp4_gemm_plan* p, int M, int schedule, size_t* counters,
                     size_t* partials) {
    prefill_need(prefill_split(M, p->K, p->N, p->pre.cus, schedule), p->pre.cus, counters,
                 partials);
}

int launch_prefill(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                   float ts, const uint16_t* act, void* out, void* ws, size_t ctr_off,
                   size_t pre_off, int schedule, hipStream_t s) {
    const int n_tiles = p->Np / kTileN, nsb = p->Kp / kSuperK;
    const int mblocks = (M + kPTile - 1) / kPTile;
    const PrefillSplit sp = prefill_split(M, p->K, p->N, p->pre.cus, schedule);
    const bool bf16 = p->out_dtype == NVFP4_OUT_BF16;
    if (sp.stream) {
        // one workgroup per compute unit (the plan's count, which sized the
        // workspace and chose the schedule)
        float* slots = (float*)((char*)ws + pre_off);
        unsigned int* counters = (unsigned int*)((char*)ws + ctr_off);
        const dim3 grid((unsigned)p->pre.cus);
        const int l2_local = p->pre.cus % 8 == 0 && xcd_mapping_verified();
        if (bf16)
            hipLaunchKernelGGL(prefill_sk_kernel<true>, grid, dim3(kPThreads), 0, s, codes,
                               scales, act, out, slots, counters, ts, M, p->K, p->N, nsb, n_tiles,
                               sp.tiles / mblocks, sp.tiles, l2_local);
        else
            hipLaunchKernelGGL(prefill_sk_kernel<false>, grid, dim3(kPThreads), 0, s, codes,
                               scales, act, out, slots, counters, ts, M, p->K, p->N, nsb, n_tiles,
                               sp.tiles / mblocks, sp.tiles, l2_local);
        NVFP4_HIP(hipGetLastError());
        return NVFP4_OK;
    }
    const int pieces = sp.n_tail * sp.splits;
    float* part = pieces ? (float*)((char*)ws + pre_off) : nullptr;
    const dim3 grid((unsigned)(sp.tiles - sp.n_tail + pieces));
    if (bf16)
        hipLaunchKernelGGL(prefill_kernel<true>, grid, dim3(kPThreads), 0, s, codes, scales, act,
                           out, part, ts, M, p->K, p->N, nsb, n_tiles, mblocks, sp.tiles,
                           sp.n_tail, sp.splits);
    else
        hipLaunchKernelGGL(prefill_kernel<false>, grid, dim3(kPThreads), 0, s, codes, scales,
                           act, out, part, ts, M, p->K, p->N, nsb, n_tiles, mblocks, sp.tiles,
                           sp.n_tail, sp.splits);
    NVFP4_HIP(hipGetLastError());
    if (!pieces) return NVFP4_OK;
    const dim3 rgrid((unsigned)(sp.n_tail * (kPTileFloats / 4 / kPReduceThreads)));
    if (bf16)
        hipLaunchKernelGGL(prefill_reduce_kernel<true>, rgrid, dim3(kPReduceThreads), 0, s, part,
                           out, ts, M, p->N, mblocks, sp.tiles, sp.n_tail, sp.splits);
    else
        hipLaunchKernelGGL(prefill_reduce_kernel<false>, rgrid, dim3(kPReduceThreads), 0, s,
                           part, out, ts, M, p->N, mblocks, sp.tiles, sp.n_tail, sp.splits);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

}  // namespace nvfp4
