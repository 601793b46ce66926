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
//     product), block sums and the scaled accumulation are fp32.  A row i
//     (and i + 8) carries activation row 2 (i mod 4) + i / 4 (act_row), so
//     output row 4g + j holds activation row 2j + g (g mod 2) and with M
//     lanes only j < ceil(M / 2) need their FMAs (kLiveJ).
//   The two row halves are added with one cross-lane exchange at the end.
// K is split over workgroups when the column count alone cannot fill the
// chip; partial sums go to a workspace and the last workgroup of a column
// group (an atomic counter) adds them in split order, so results are
// deterministic.  Workgroups of one column group are placed on one XCD
// (blockIdx % 8 selects the XCD), so their partials meet in one L2.
#include "decode_device.h"
#include "swiglu_device.h"
#include <type_traits>

namespace nvfp4 {

// Argmax of each output row, fused into the output head's run (the step
// after the head: "Ignis" README, "Speculative decoding (DFlash2)", top-k over
// the vocabulary; k = 1 here).  Logit v at column n becomes the key
// (ord(v) << 32) | ~n of the top-k kernel: a larger key is a larger value, or
// an equal one at a smaller column (-0 equals +0).  The one workgroup that
// writes a column group's outputs folds their keys into LDS per row and
// stores the group's 8 row keys to its slot of the caller's area (plain
// stores, no atomics); argmax_merge_kernel then takes each row's maximum over
// the slots.  Measured at M = 8, N = 152064: the head with its argmax 75.8 us,
// the head alone 69.9, the head followed by the top-k kernel with k = 1 76.0:
// the second launch costs what the top-k launch did.  (A first form folded
// the keys into per-XCD words with L2 atomics and elected the last group by
// counters, with no second launch: every workgroup then waited for two atomic
// round trips, and the head with its argmax took 80.3 us against 76.5.)
struct ArgmaxRef {
    unsigned long long* area;    // [groups][8] row keys; null: no argmax
    unsigned long long* s_keys;  // LDS, 8 words
};

// The gate_up epilogue that also computes SwiGLU for the next matrix (a round
// whose down matrix takes the SwiGLU of gate_up's output): the column group
// holds gate columns 32 ng .. 32 ng + 31 (waves 0, 1) and the up columns F
// above them (waves 2, 3), so each output row's 32 h values can be formed from
// the group's own bf16 outputs, exactly as the SwiGLU kernel forms them.
struct SwigluRef {
    uint16_t* h;     // [M][F] bf16 (the down matrix's activations)
    int F;           // N / 2
    uint16_t* s_gu;  // LDS, 8 rows x 64 group columns of bf16 outputs
};

__device__ __forceinline__ unsigned long long argmax_key(float v, int n) {
    unsigned int b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0u;  // -0 -> +0
    const unsigned int o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((unsigned long long)o << 32) | (unsigned int)(~n);
}

// After a group's outputs are written and their keys folded into s_keys.
__device__ __forceinline__ void argmax_group_done(const ArgmaxRef& am, int ng) {
    __syncthreads();  // every output's key is in s_keys
    if (threadIdx.x < 8) am.area[(size_t)ng * 8 + threadIdx.x] = am.s_keys[threadIdx.x];
}

// Row m's argmax from the n_groups slots of the area (workgroup m, 256
// threads).  (One workgroup of 1024 threads reading whole slots and keeping
// all 8 rows measured slower: 78.7 us for the head with its argmax against
// 75.8.)
__global__ __launch_bounds__(256) void argmax_merge_kernel(const unsigned long long* __restrict__ area,
                                                           int n_groups, int* __restrict__ out) {
    __shared__ unsigned long long s_best[4];
    const int m = blockIdx.x;
    unsigned long long best = 0;
    for (int g = threadIdx.x; g < n_groups; g += 256) {
        const unsigned long long k = area[(size_t)g * 8 + m];
        best = k > best ? k : best;
    }
    for (int o = 32; o >= 1; o >>= 1) {
        const unsigned long long k = __shfl_xor(best, o, 64);
        best = k > best ? k : best;
    }
    if ((threadIdx.x & 63) == 0) s_best[threadIdx.x >> 6] = best;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < 4; ++w) best = s_best[w] > best ? s_best[w] : best;
        out[m] = (int)~(unsigned int)best;
    }
}

// The end of a workgroup: the two row halves of each lane's sums are added,
// then the outputs (one slice) or the split-K hand-off (several), and the
// argmax step when asked for.
template <int WAVES, bool BF16, bool SW = false>
__device__ __forceinline__ void decode_finish(float (&acc)[4], void* __restrict__ out,
                                              float* __restrict__ partial,
                                              unsigned int* __restrict__ counters, float ts,
                                              int M, int N, int splits, int n_tiles, int l2_local,
                                              int ng, int split, int nt, int* s_last,
                                              const ArgmaxRef& am,
                                              const SwigluRef& sw = SwigluRef{}) {
    static_assert(!SW || (WAVES == 4 && BF16), "SwiGLU epilogue: 4 waves, bf16 outputs");
    constexpr int kThreads = WAVES * 64;
    constexpr int kCols = WAVES * kTileN;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, g = lane >> 4;
    // Lanes g and g+2 hold the same (row, column) for the two block halves.
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], 32, 64);
    const bool mine = lane < 32 && ng * WAVES + wave < n_tiles;
    const bool amax = am.area != nullptr;  // (uniform)
    if (amax) {
        if (threadIdx.x < 8) am.s_keys[threadIdx.x] = 0;
        __syncthreads();
    }
    // Output (mm, n) = v: stored, and its key folded into the row's LDS word.
    auto emit = [&](int mm, int n, float v) {
        store_out<BF16>(out, (size_t)mm * N + n, v);
        if (amax)
            __hip_atomic_fetch_max(&am.s_keys[mm], argmax_key(v, n), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_WORKGROUP);
    };

    // (SW) h for the group's 32 columns from its stashed bf16 outputs.
    auto swiglu_tail = [&]() {
        if constexpr (SW) {
            __syncthreads();
            for (int t = threadIdx.x; t < M * 32; t += kThreads) {
                const int mm = t >> 5, jj = t & 31;
                sw.h[(size_t)mm * sw.F + 32 * ng + jj] =
                    swiglu_bf16(sw.s_gu[mm * 64 + jj], sw.s_gu[mm * 64 + 32 + jj]);
            }
        }
    };

    if (splits == 1) {
        if (mine) {
            const int n = nt * kTileN + col;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int mm = 2 * j + g;
                if (mm < M && n < N) {
                    emit(mm, n, acc[j] * ts);
                    if constexpr (SW) sw.s_gu[mm * 64 + wave * kTileN + col] = f32_to_bf16_rne(acc[j] * ts);
                }
            }
        }
        if (amax) argmax_group_done(am, ng);
        swiglu_tail();
        return;
    }

    // Split K.  The slices of one column group run on one XCD (blockIdx % 8
    // selects it, verified when the plan is made: l2_local), so their
    // partial sums meet in that XCD's L2: plain stores, a wait for their
    // completion, then the counter increment.  Without the verified mapping
    // the partials go through device-coherent (write-through) stores and
    // loads instead.  Either way the hand-off needs no agent-scope fence,
    // whose write-back of the whole L2 would cost every workgroup.
    float* pbase = partial + (size_t)(ng * splits + split) * 8 * kCols;
    if (mine) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int mm = 2 * j + g;
            if (mm < M) {
                float* dst = pbase + mm * kCols + wave * kTileN + col;
                if (l2_local)
                    *dst = acc[j];
                else
                    __hip_atomic_store(dst, acc[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        // (agent scope is a read-modify-write in this XCD's L2; without the
        // verified mapping the contributors may sit on several XCDs, so the
        // counter is then device-coherent)
        const unsigned int old =
            l2_local ? __hip_atomic_fetch_add(&counters[ng], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT)
                     : __hip_atomic_fetch_add(&counters[ng], 1u, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_SYSTEM);
        *s_last = (old == (unsigned int)(splits - 1));
    }
    __syncthreads();
    if (!*s_last) return;
    const float* gbase = partial + (size_t)ng * splits * 8 * kCols;
    constexpr int kR = (8 * kCols + kThreads - 1) / kThreads;
    float sum[kR];
    if (l2_local)
        sum_partials<kCols, kThreads, kR, true>(gbase, splits, M * kCols, sum);
    else
        sum_partials<kCols, kThreads, kR, false>(gbase, splits, M * kCols, sum);
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int idx = threadIdx.x + r * kThreads;
        const int mm = idx / kCols, c = idx - mm * kCols;
        int n = ng * kCols + c;
        if constexpr (SW) n = c < 32 ? 32 * ng + c : sw.F + 32 * ng + (c - 32);
        if (idx < M * kCols && n < N) {
            emit(mm, n, sum[r] * ts);
            if constexpr (SW) sw.s_gu[mm * 64 + c] = f32_to_bf16_rne(sum[r] * ts);
        }
    }
    if (threadIdx.x == 0) {  // leave the counter zeroed for the next run
        if (l2_local)
            __hip_atomic_store(&counters[ng], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_store(&counters[ng], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    if (amax) argmax_group_done(am, ng);
    swiglu_tail();
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
    int n_groups, int n_tiles, int l2_local, unsigned long long* __restrict__ amax_area) {
    constexpr int kThreads = WAVES * 64;
    constexpr int kStride = NCH * kSuperK + kLdsPad;          // LDS row, bf16 elements
    __shared__ __attribute__((aligned(16))) __bf16 lds[9 * kStride];
    __shared__ int s_last;
    __shared__ unsigned long long s_keys[8];

    const int b = blockIdx.x;
    const int xcd = b & 7, q = b >> 3;
    const int ng = (q / splits) * 8 + xcd;
    const int split = q - (q / splits) * splits;
    if (ng >= n_groups) return;  // whole workgroup: padding of the column groups to 8
    const int sb0 = split * NCH;
    const int nch = min(NCH, nsb - sb0);  // superblocks in this slice (>= 1)
    const int k0 = sb0 * kSuperK;

    // 1. This thread's share of the activation slice.
    ActStage<kThreads, NCH, kStride> stage;
    stage.load(act, M, K, k0, nch);

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
    stage.store(lds, M, K, k0, nch);
    __syncthreads();

    // 4. MFMA over the slice.  A-operand row of this lane: activation row
    //    `col` for its block half (col < 8 pairs with octets 0,1; col >= 8
    //    with octets 2,3), else the zero row.
    const int m = act_row(col & 7);
    const bool live = ((col >> 3) == (g >> 1)) && (m < M);
    const __bf16* ap = lds + (live ? m : 8) * kStride + 8 * g;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NCH; ++c)
        if (c < nch) chunk_steps(acc, w[c], ap + c * kSuperK);

    decode_finish<WAVES, BF16>(acc, out, partial, counters, ts, M, N, splits, n_tiles, l2_local,
                               ng, split, nt, &s_last,
                               ArgmaxRef{amax_area, s_keys});
}

// ---- long slices ------------------------------------------------------------------

// Long K slices: a workgroup's slice is `windows` windows of NCH superblocks.
// A wave keeps the weights of two windows in registers: those of window w + 1
// are issued before window w is computed, so the weight stream of the
// workgroup does not stop between windows.  The activations of a window are
// copied straight to LDS (buffer_load ... lds) into one of two buffers,
// issued right after that window's weights; a wave's loads complete in order,
// so waiting for window w's loads never waits for window w + 1's.  Every wave
// issues the same number of loads per window (clamped addresses, unused
// destinations), so the waits are constants.
//
// Code shape.  The compiler adds its own waits before any use of a loaded
// register or of LDS that a copy may be writing, from what it can prove at
// that point.  The loop is therefore written so that its proof is exact: the
// steady state issues the next window on every step (no branch around the
// issue; a runtime "is there a next window" branch merged the two paths'
// states and produced a wait for every load in flight, the next window's
// too), the last one or two windows are separate code, and scheduling
// barriers keep each window's compute between its own waits.  Measured in one
// process against the earlier shape: 64-layer round 7% faster at M = 1 and at
// M = 8, and the registers per lane fall from 122 to 76 (6 waves per SIMD
// instead of 4).
// J: output rows scaled per lane (kb_steps, kLiveJ of the lanes).
// SW: the gate_up epilogue with SwiGLU (SwigluRef): column group ng holds gate
// tiles 2 ng, 2 ng + 1 and up tiles n_tiles / 2 + 2 ng, + 1.
template <int WAVES, int NCH, bool BF16, int J = 4, bool SW = false>
__global__ __launch_bounds__(WAVES * 64) void decode_window_kernel(
    const uint4* __restrict__ codes, const uint4* __restrict__ scales,
    const uint16_t* __restrict__ act, void* __restrict__ out, float* __restrict__ partial,
    unsigned int* __restrict__ counters, float ts, int M, int K, int N, int nsb, int splits,
    int n_groups, int n_tiles, int l2_local, int windows,
    unsigned long long* __restrict__ amax_area, uint16_t* __restrict__ sw_h, int sw_F) {
    constexpr int kThreads = WAVES * 64;
    constexpr int kStride = NCH * kSuperK + kLdsPad;  // LDS row, bf16 elements
    constexpr int kSeg = 8 * NCH / WAVES;  // activation segments (1 KiB) per wave per window
    static_assert(8 * NCH % WAVES == 0, "activation segments divide over the waves");
    constexpr int kLoads = 5 * NCH + kSeg;  // loads a wave issues per window
    // Two separate arrays (not one of two rows): the compiler then sees that
    // copies into one buffer never alias reads of the other, and does not
    // make the reads wait for the copies in flight.
    __shared__ __attribute__((aligned(16))) __bf16 lds0[9 * kStride];
    __shared__ __attribute__((aligned(16))) __bf16 lds1[9 * kStride];
    __shared__ int s_last;
    __shared__ unsigned long long s_keys[8];
    __shared__ uint16_t s_gu[SW ? 8 * 64 : 1];

    const int b = blockIdx.x;
    const int xcd = b & 7, q = b >> 3;
    const int ng = (q / splits) * 8 + xcd;
    const int split = q - (q / splits) * splits;
    if (ng >= n_groups) return;  // whole workgroup: padding of the column groups to 8
    const int sb_begin = split * NCH * windows;
    const int ns = min(NCH * windows, nsb - sb_begin);  // superblocks in this slice (>= 1)
    const int nwin = (ns + NCH - 1) / NCH;

    // The wave index is uniform; saying so keeps the activation resources scalar.
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int nt = SW ? (wave < 2 ? 2 * ng + wave : (n_tiles >> 1) + 2 * ng + (wave - 2))
                      : min(ng * WAVES + wave, n_tiles - 1);
    const int col = lane & 15, g = lane >> 4;
    const uint4* cp = codes + ((size_t)nt * nsb + sb_begin) * 256 + lane;
    const uint4* sp = scales + ((size_t)nt * nsb + sb_begin) * 32 + col * 2 + (g >> 1);

    // Zero row (row 8) of both buffers; complete before the first window's barrier.
    for (int o = threadIdx.x; o < NCH * kSuperK / 8; o += kThreads) {
        *(uint4*)(lds0 + 8 * kStride + 8 * o) = make_uint4(0, 0, 0, 0);
        *(uint4*)(lds1 + 8 * kStride + 8 * o) = make_uint4(0, 0, 0, 0);
    }

    // Issues window w: weights into x, activation rows into buf.
    // Segment j of this wave is (row r, superblock c) = divmod(wave * kSeg + j,
    // NCH); rows >= M re-read row M - 1 and superblocks past the slice re-read
    // its last one (their destinations are never read).  Each row's resource
    // ends at the row's end, so values past K read as zero.
    auto issue = [&](int w, Chunk (&x)[NCH], __bf16* buf) {
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int sb = min(w * NCH + c, ns - 1);
            load_chunk(x[c], cp + 256 * sb, sp + 32 * sb);
        }
#pragma unroll
        for (int j = 0; j < kSeg; ++j) {
            const int seg = wave * kSeg + j;
            const int r = seg / NCH, c = seg - r * NCH;
            const int sb = min(w * NCH + c, ns - 1);
            const int k = (sb_begin + sb) * kSuperK;
            const uint16_t* row = act + (size_t)min(r, M - 1) * K + k;
            const int bytes = (K - k) * (int)sizeof(uint16_t);
            const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<uint16_t*>(row), 0, bytes, 0x00020000);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rs, (__attribute__((address_space(3))) void*)(buf + r * kStride + c * kSuperK),
                16, lane * 16, 0, 0, 0);
        }
    };

    const int m = act_row(col & 7);
    const bool live = ((col >> 3) == (g >> 1)) && (m < M);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    // Window w: wait for its loads (not for the next window's), then compute.
    // next (a compile-time true or false): window w + 1 exists and is issued
    // first, into y and nxt.
    auto step = [&](int w, auto next, Chunk (&x)[NCH], Chunk (&y)[NCH], const __bf16* cur,
                    __bf16* nxt) {
        // Every wave is done reading nxt (window w - 1).
        // (scheduling barriers: no instruction of the previous or next window's
        // compute moves across the issue and the waits)
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
        barrier_nofence();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(next)::value) {
            issue(w + 1, y, nxt);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        barrier_nofence();  // every wave's activation segments of window w are in LDS
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!decltype(next)::value) {
            // (all loads are complete here: marking the registers costs no wait)
#pragma unroll
            for (int c = 0; c < NCH; ++c) {
#pragma unroll
                for (int i = 0; i < 4; ++i) opaque(x[c].c[i]);
                opaque(x[c].s);
            }
        }
        const int nch = min(NCH, ns - w * NCH);
        const __bf16* ap = cur + (live ? m : 8) * kStride + 8 * g;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            if (c < nch) chunk_steps<J>(acc, x[c], ap + c * kSuperK);
    };
    using Yes = std::integral_constant<bool, true>;
    using No = std::integral_constant<bool, false>;
    Chunk wa[NCH], wb[NCH];
    issue(0, wa, lds0);
    int w = 0;
    for (; w + 2 < nwin; w += 2) {
        step(w, Yes{}, wa, wb, lds0, lds1);
        step(w + 1, Yes{}, wb, wa, lds1, lds0);
    }
    if (w + 1 < nwin) {
        step(w, Yes{}, wa, wb, lds0, lds1);
        step(w + 1, No{}, wb, wa, lds1, lds0);
    } else {
        step(w, No{}, wa, wb, lds0, lds1);
    }
    decode_finish<WAVES, BF16, SW>(acc, out, partial, counters, ts, M, N, splits, n_tiles,
                                   l2_local, ng, split, nt, &s_last, ArgmaxRef{amax_area, s_keys},
                                   SwigluRef{sw_h, sw_F, s_gu});
}

// ---- narrow widths: one workgroup per column tile ------------------------------------

// M <= 4 lanes.  With few activation rows a workgroup can afford the whole of
// K's activations (at most 4 x K bf16), so one workgroup owns one 16-column
// tile over all of K and its waves split K: wave p streams superblocks
// [p SBW, p SBW + SBW), issuing all of its weight loads and its activation
// rows (direct-to-LDS copies, into its own LDS rows) at once, then computes
// with the split-A MFMA of the decode kernel.  The waves' sums meet in LDS
// and are added in wave order, so there is no split-K hand-off between
// workgroups, no workspace and no atomic.  Lanes whose A-operand row is not a
// live activation row read a zero row.
//
// Measured in 64-node graphs on MI355X at M = 1 against the split-K kernel:
// qkv (5120 x 7168) 6.65 us against 8.15, o (6144 x 5120) 6.57 against 7.71,
// gate_up (5120 x 34816) 18.7 against 20.1, the output head at plain-read
// speed (64.0 us; a plain read of its bytes 64.2).  It loses at M = 8, where
// every workgroup re-stages 80 KB of activations per tile, and for long K
// (down, 34 superblocks), whose waves per workgroup leave one workgroup per
// compute unit.
template <int SBW, int MR, bool BF16>
__global__ __launch_bounds__(1024) void decode_tile_kernel(
    const uint4* __restrict__ codes, const uint4* __restrict__ scales,
    const uint16_t* __restrict__ act, void* __restrict__ out, float ts, int M, int K, int N,
    int nsb) {
    static_assert(MR >= 1 && MR <= 4, "at most 4 staged rows (M <= MR)");
    constexpr int kRow = SBW * kSuperK + kLdsPad;  // bf16 elements per staged row
    extern __shared__ __attribute__((aligned(16))) __bf16 tile_lds[];
    const int waves = blockDim.x >> 6;
    // The wave index is uniform; saying so keeps the activation resources scalar.
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int nt = blockIdx.x;
    const int col = lane & 15, g = lane >> 4;
    __bf16* zero = tile_lds;                                // one row of zeros
    __bf16* rows = tile_lds + kRow + wave * MR * kRow;      // this wave's MR rows
    float* red = (float*)(tile_lds + kRow + waves * MR * kRow);  // [waves][8][16]
    for (int o = threadIdx.x; o < kRow / 8; o += blockDim.x)
        *(uint4*)(zero + 8 * o) = make_uint4(0, 0, 0, 0);

    // Every wave has at least one superblock (waves = ceil(nsb / SBW)); the
    // last one may have fewer than SBW and re-reads its last (unused) one.
    const int sb0 = wave * SBW;
    const int ns = min(SBW, nsb - sb0);
    const uint4* cp = codes + ((size_t)nt * nsb + sb0) * 256 + lane;
    const uint4* sp = scales + ((size_t)nt * nsb + sb0) * 32 + col * 2 + (g >> 1);
    Chunk w[SBW];
#pragma unroll
    for (int c = 0; c < SBW; ++c) {
        const int cc = min(c, ns - 1);
        load_chunk(w[c], cp + 256 * cc, sp + 32 * cc);
    }
    // Activation rows r < M of this wave's K range, one 1 KiB copy per row
    // and superblock; each row's resource ends at the row's end, so values
    // past K read as zero.
#pragma unroll
    for (int r = 0; r < MR; ++r) {
        if (r < M) {
#pragma unroll
            for (int c = 0; c < SBW; ++c) {
                if (c < ns) {
                    const int k = (sb0 + c) * kSuperK;
                    const uint16_t* row = act + (size_t)r * K + k;
                    const int bytes = (K - k) * (int)sizeof(uint16_t);
                    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<uint16_t*>(row), 0, bytes, 0x00020000);
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        rs, (__attribute__((address_space(3))) void*)(rows + r * kRow + c * kSuperK),
                        16, lane * 16, 0, 0, 0);
                }
            }
        }
    }
    __syncthreads();  // the zero row is written
    __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));  // this wave's weights and rows have landed

    const int m = act_row(col & 7);
    const bool live = ((col >> 3) == (g >> 1)) && (m < M);
    const __bf16* ap = live ? (rows + m * kRow + 8 * g) : (zero + 8 * g);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < SBW; ++c)
        if (c < ns) chunk_steps<kLiveJ(MR)>(acc, w[c], ap + c * kSuperK);

    // Lanes g and g+2 hold the same (row, column) for the two block halves.
#pragma unroll
    for (int j = 0; j < kLiveJ(MR); ++j) acc[j] += __shfl_xor(acc[j], 32, 64);
    if (lane < 32) {
#pragma unroll
        for (int j = 0; j < 4; ++j) red[(wave * 8 + 2 * j + g) * kTileN + col] = acc[j];
    }
    __syncthreads();
    if ((int)threadIdx.x < M * kTileN) {
        const int mm = threadIdx.x / kTileN, c = threadIdx.x - mm * kTileN;
        float sum = 0.f;
        for (int p = 0; p < waves; ++p) sum += red[(p * 8 + mm) * kTileN + c];
        const int n = nt * kTileN + c;
        if (n < N) store_out<BF16>(out, (size_t)mm * N + n, sum * ts);
    }
}

static size_t tile_lds_bytes(int sbw, int mr, int waves) {
    const size_t row = (size_t)sbw * kSuperK + kLdsPad;
    return (row + (size_t)waves * mr * row) * 2 + (size_t)waves * 8 * kTileN * sizeof(float);
}

int make_tile_config(int K, int N, int max_M, const nvfp4_gemm_config* cfg, TileConfig* t) {
    *t = TileConfig{};
    const int n_tiles = padded_n(N) / kTileN;
    const int nsb = padded_k(K) / kSuperK;
    const int forced_m = cfg ? cfg->tile_max_m : 0;
    const int forced_sbw = cfg ? cfg->tile_superblocks : 0;
    if (forced_m < -1 || forced_m > 4)
        return set_error(NVFP4_EINVAL, "config.tile_max_m: %d outside [-1, 4]", forced_m);
    if (forced_sbw < 0 || forced_sbw > 3)
        return set_error(NVFP4_EINVAL, "config.tile_superblocks: %d outside [0, 3]", forced_sbw);
    if (forced_m == -1) return NVFP4_OK;
    // Defaults measured on MI355X over the round's shapes and the output
    // head: one superblock per wave while the tiles alone give each compute
    // unit fewer than 4 workgroups (qkv, o), two for wider matrices (gate_up,
    // the head); M up to 4 and up to 2 respectively; no tile kernel when K
    // would need more than 12 waves per workgroup (down).
    const bool wide = n_tiles >= 4 * device_cus();
    const int sbw = forced_sbw ? forced_sbw : (wide ? 2 : 1);
    const int waves = (nsb + sbw - 1) / sbw;
    if (waves > 16) {
        if (forced_m > 0)
            return set_error(NVFP4_EINVAL, "config.tile_max_m: K = %d needs %d waves of %d "
                             "superblocks, more than 16", K, waves, sbw);
        return NVFP4_OK;
    }
    int max_m = forced_m ? forced_m : (waves > 12 ? 0 : wide ? 2 : 4);
    if (max_m > max_M) max_m = max_M;
    if (max_m > 0 && tile_lds_bytes(sbw, max_m <= 1 ? 1 : max_m <= 2 ? 2 : 4, waves) > 160 * 1024)
        return set_error(NVFP4_EINVAL, "config.tile_superblocks: %d with %d waves needs more "
                         "LDS than a compute unit has", sbw, waves);
    t->max_m = max_m;
    t->sbw = sbw;
    t->waves = waves;
    return NVFP4_OK;
}

template <int SBW, int MR, bool BF16>
static int launch_tile_t(const nvfp4_gemm_plan* p, int M, const uint8_t* codes,
                         const uint8_t* scales, float ts, const uint16_t* act, void* out,
                         hipStream_t s) {
    const TileConfig& t = p->tile;
    const size_t lds = tile_lds_bytes(SBW, MR, t.waves);
    if (lds > 64 * 1024) {
        // above the default limit of dynamic LDS per workgroup
        NVFP4_HIP(hipFuncSetAttribute((const void*)decode_tile_kernel<SBW, MR, BF16>,
                                      hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds));
    }
    hipLaunchKernelGGL((decode_tile_kernel<SBW, MR, BF16>), dim3(p->Np / kTileN),
                       dim3(t.waves * 64), lds, s, (const uint4*)codes, (const uint4*)scales, act,
                       out, ts, M, p->K, p->N, p->Kp / kSuperK);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

template <int SBW, bool BF16>
static int launch_tile_m(const nvfp4_gemm_plan* p, int M, const uint8_t* codes,
                         const uint8_t* scales, float ts, const uint16_t* act, void* out,
                         hipStream_t s) {
    if (M <= 1) return launch_tile_t<SBW, 1, BF16>(p, M, codes, scales, ts, act, out, s);
    if (M <= 2) return launch_tile_t<SBW, 2, BF16>(p, M, codes, scales, ts, act, out, s);
    return launch_tile_t<SBW, 4, BF16>(p, M, codes, scales, ts, act, out, s);
}

template <bool BF16>
static int launch_tile_s(const nvfp4_gemm_plan* p, int M, const uint8_t* codes,
                         const uint8_t* scales, float ts, const uint16_t* act, void* out,
                         hipStream_t s) {
    switch (p->tile.sbw) {
        case 1: return launch_tile_m<1, BF16>(p, M, codes, scales, ts, act, out, s);
        case 2: return launch_tile_m<2, BF16>(p, M, codes, scales, ts, act, out, s);
        default: return launch_tile_m<3, BF16>(p, M, codes, scales, ts, act, out, s);
    }
}

int launch_tile(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                float ts, const uint16_t* act, void* out, hipStream_t s) {
    return p->out_dtype == NVFP4_OUT_BF16
               ? launch_tile_s<true>(p, M, codes, scales, ts, act, out, s)
               : launch_tile_s<false>(p, M, codes, scales, ts, act, out, s);
}

// ---- device facts ----------------------------------------------------------------

int device_cus() {
    static int cached[64];
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 256;
    }
    if (cached[dev]) return cached[dev];
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus < 1) {
        (void)hipGetLastError();
        cus = 256;  // MI355X; kept, so plans and launches agree
    }
    cached[dev] = cus;
    return cus;
}

// ---- XCD mapping check -----------------------------------------------------------

// Workgroups are dispatched to the 8 XCDs round-robin (workgroup b on XCD
// b % 8); the split-K hand-off relies on it to keep partial sums in one L2.
// Checked once per device by reading each workgroup's XCC_ID register.
constexpr int kProbeBlocks = 64;
__device__ unsigned int g_xcc_probe[kProbeBlocks];

__global__ void xcc_probe_kernel() {
    unsigned int v;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
    if (threadIdx.x == 0) g_xcc_probe[blockIdx.x] = v & 0xFu;
}

int xcd_mapping_verified() {
    static int cached[64];
    static bool init = false;
    if (!init) {
        for (int& c : cached) c = -1;
        init = true;
    }
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) {
        (void)hipGetLastError();
        return 0;
    }
    if (cached[dev] >= 0) return cached[dev];
    unsigned int h[kProbeBlocks];
    int ok = 0;
    hipLaunchKernelGGL(xcc_probe_kernel, dim3(kProbeBlocks), dim3(64), 0, 0);
    if (hipGetLastError() == hipSuccess && hipDeviceSynchronize() == hipSuccess &&
        hipMemcpyFromSymbol(h, HIP_SYMBOL(g_xcc_probe), sizeof(h), 0, hipMemcpyDeviceToHost) ==
            hipSuccess) {
        ok = 1;
        for (int b = 0; b < kProbeBlocks; ++b)
            if (h[b] != (unsigned int)(b % 8)) ok = 0;
    }
    (void)hipGetLastError();
    cached[dev] = ok;
    return ok;
}

// ---- plan ----------------------------------------------------------------------

int make_decode_config(int K, int N, int max_M, const nvfp4_gemm_config* cfg, DecodeConfig* d) {
    (void)max_M;
    const int n_tiles = padded_n(N) / kTileN;
    const int nsb = padded_k(K) / kSuperK;
    // Defaults measured on MI355X over the round's shapes (K = 5120..17408,
    // N = 5120..34816): slices of 2 windows of 1 superblock and 4 waves per
    // workgroup, except very long K (>= 16384): 6 windows of 1 superblock and
    // 8 waves.  (One window of 2 superblocks, resp. 3 superblocks and 8
    // waves, the best single-window forms, are 2% slower over the round.)
    // Column groups that alone give every compute unit 4 or more workgroups
    // (the output head: 2376) take no K split at all: one slice of the whole
    // K per workgroup, streamed window by window, and no hand-off (the head
    // at M = 8: 72 us against 94 with 5 splits).  The round's other matrices
    // keep their splits: two, of half of K each, when two workgroups per
    // group nearly fill the chip (qkv, 112 groups: 8.46 us against 9.02 with
    // 5 splits, gate_up, 544 groups: 21.9 against 22.3, at M = 8 in 64-node
    // graphs); fewer groups take the slices below.
    const bool long_k = nsb >= 32;
    const bool defaults = !(cfg && (cfg->split_k || cfg->chunks || cfg->windows));
    int waves = (cfg && cfg->waves) ? cfg->waves : (long_k ? 8 : 4);
    if (waves != 4 && waves != 8)
        return set_error(NVFP4_EINVAL, "config.waves: %d is not 4 or 8", waves);
    const int n_groups = (n_tiles + waves - 1) / waves;
    const bool wide = n_groups >= 4 * device_cus();
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
        chunks = 1;
    }
    const bool halves = !long_k && 8 * 2 * n_groups >= 7 * device_cus();
    // Fewer groups: as many K slices as still give every workgroup a compute
    // unit of its own, slices of at least 2 windows (o and the 5120 x 5120
    // projection, 80 groups: 3 slices, 7.9 us at M = 8 against 8.4 with the
    // 6 and 5 slices of 2 windows, and against 8.8 / 8.1 with 4 / 2 slices).
    const int fill = device_cus() / ng8 > 1 ? device_cus() / ng8 : 1;
    const int fill_windows = (nsb + fill - 1) / fill > 2 ? (nsb + fill - 1) / fill : 2;
    int windows = (cfg && cfg->windows) ? cfg->windows
                  : defaults ? (wide ? nsb : long_k ? 6 : halves ? (nsb + 1) / 2 : fill_windows)
                             : 1;
    if (windows < 1) return set_error(NVFP4_EINVAL, "config.windows: %d < 1", windows);
    if ((long long)windows * chunks > nsb) windows = (nsb + chunks - 1) / chunks;
    const int splits = (nsb + chunks * windows - 1) / (chunks * windows);
    d->l2_local = splits > 1 ? xcd_mapping_verified() : 0;
    d->waves = waves;
    d->chunks = chunks;
    d->windows = windows;
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

// The argmax step's area for a launch (null: none).
struct ArgmaxArgs {
    unsigned long long* area;
};

template <int WAVES, int NCH, bool BF16>
static int launch_t(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                    float ts, const uint16_t* act, void* out, void* ws, size_t partial_off,
                    const ArgmaxArgs& am, hipStream_t s) {
    const DecodeConfig& d = p->dec;
    unsigned int* counters = (unsigned int*)ws;
    float* partial = ws ? (float*)((char*)ws + partial_off) : nullptr;
    if (NCH == 1 && d.windows > 1 && M <= 6) {
        // fewer than 7 lanes: only the live output rows take their scales
#define NVFP4_WINDOW_J(JJ)                                                                     \
    hipLaunchKernelGGL((decode_window_kernel<WAVES, 1, BF16, JJ>), dim3(d.grid),               \
                       dim3(WAVES * 64), 0, s, (const uint4*)codes, (const uint4*)scales, act, \
                       out, partial, counters, ts, M, p->K, p->N, p->Kp / kSuperK, d.splits,   \
                       d.n_groups, p->Np / kTileN, d.l2_local, d.windows, am.area, nullptr, 0)
        if (kLiveJ(M) == 1)
            NVFP4_WINDOW_J(1);
        else if (kLiveJ(M) == 2)
            NVFP4_WINDOW_J(2);
        else
            NVFP4_WINDOW_J(3);
#undef NVFP4_WINDOW_J
    } else if (d.windows > 1)
        hipLaunchKernelGGL((decode_window_kernel<WAVES, NCH, BF16>), dim3(d.grid),
                           dim3(WAVES * 64), 0, s, (const uint4*)codes, (const uint4*)scales, act,
                           out, partial, counters, ts, M, p->K, p->N, p->Kp / kSuperK, d.splits,
                           d.n_groups, p->Np / kTileN, d.l2_local, d.windows, am.area, nullptr, 0);
    else
        hipLaunchKernelGGL((decode_kernel<WAVES, NCH, BF16>), dim3(d.grid), dim3(WAVES * 64), 0,
                           s, (const uint4*)codes, (const uint4*)scales, act, out, partial,
                           counters, ts, M, p->K, p->N, p->Kp / kSuperK, d.splits, d.n_groups,
                           p->Np / kTileN, d.l2_local, am.area);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

template <int WAVES, bool BF16>
static int launch_c(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                    float ts, const uint16_t* act, void* out, void* ws, size_t po,
                    const ArgmaxArgs& am, hipStream_t s) {
    switch (p->dec.chunks) {
        case 1: return launch_t<WAVES, 1, BF16>(p, M, codes, scales, ts, act, out, ws, po, am, s);
        case 2: return launch_t<WAVES, 2, BF16>(p, M, codes, scales, ts, act, out, ws, po, am, s);
        case 3: return launch_t<WAVES, 3, BF16>(p, M, codes, scales, ts, act, out, ws, po, am, s);
        default: return launch_t<WAVES, 4, BF16>(p, M, codes, scales, ts, act, out, ws, po, am, s);
    }
}

template <bool BF16>
static int launch_w(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                    float ts, const uint16_t* act, void* out, void* ws, size_t po,
                    const ArgmaxArgs& am, hipStream_t s) {
    if (p->dec.waves == 8)
        return launch_c<8, BF16>(p, M, codes, scales, ts, act, out, ws, po, am, s);
    return launch_c<4, BF16>(p, M, codes, scales, ts, act, out, ws, po, am, s);
}

int launch_decode(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                  float ts, const uint16_t* act, void* out, void* ws, size_t partial_off,
                  hipStream_t s) {
    const size_t esz = p->out_dtype == NVFP4_OUT_BF16 ? 2 : 4;
    const ArgmaxArgs none{nullptr};
    // Rows beyond 8 (when no prefill kernel applies) run as further weight passes.
    for (int m0 = 0; m0 < M; m0 += NVFP4_DECODE_MAX_M) {
        const int mm = M - m0 < NVFP4_DECODE_MAX_M ? M - m0 : NVFP4_DECODE_MAX_M;
        const uint16_t* a = act + (size_t)m0 * p->K;
        void* o = (char*)out + (size_t)m0 * p->N * esz;
        int st = p->out_dtype == NVFP4_OUT_BF16
                     ? launch_w<true>(p, mm, codes, scales, ts, a, o, ws, partial_off, none, s)
                     : launch_w<false>(p, mm, codes, scales, ts, a, o, ws, partial_off, none, s);
        if (st) return st;
    }
    return NVFP4_OK;
}

// A gate_up run whose epilogue also writes h = SwiGLU(output) for the next
// matrix (SwigluRef), in place of the separate SwiGLU kernel.  Applies when the
// plan takes the streamed-slice decode kernel at this width with 4-wave groups
// and bf16 outputs, and N is a multiple of 64 (whole gate/up group pairs).
bool decode_swiglu_fusable(const nvfp4_gemm_plan* p, int M) {
    const DecodeConfig& d = p->dec;
    return M >= 1 && M <= NVFP4_DECODE_MAX_M && M > p->tile.max_m && d.windows > 1 &&
           d.chunks == 1 && d.waves == 4 && p->out_dtype == NVFP4_OUT_BF16 && p->N % 64 == 0;
}

int launch_decode_swiglu(const nvfp4_gemm_plan* p, int M, const uint8_t* codes,
                         const uint8_t* scales, float ts, const uint16_t* act, void* out,
                         uint16_t* h, void* ws, size_t partial_off, hipStream_t s) {
    const DecodeConfig& d = p->dec;
    unsigned int* counters = (unsigned int*)ws;
    float* partial = ws ? (float*)((char*)ws + partial_off) : nullptr;
    const int F = p->N / 2;
#define NVFP4_SWIGLU_J(JJ)                                                                   \
    hipLaunchKernelGGL((decode_window_kernel<4, 1, true, JJ, true>), dim3(d.grid), dim3(256), 0, \
                       s, (const uint4*)codes, (const uint4*)scales, act, out, partial,       \
                       counters, ts, M, p->K, p->N, p->Kp / kSuperK, d.splits, d.n_groups,    \
                       p->Np / kTileN, d.l2_local, d.windows, nullptr, h, F)
    switch (kLiveJ(M)) {
        case 1: NVFP4_SWIGLU_J(1); break;
        case 2: NVFP4_SWIGLU_J(2); break;
        case 3: NVFP4_SWIGLU_J(3); break;
        default: NVFP4_SWIGLU_J(4); break;
    }
#undef NVFP4_SWIGLU_J
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

// M <= 8 rows of an fp32 plan through the decode kernel (never the narrow-width
// tile kernel), each column group's row keys to its slot of `area`, then the
// merge kernel: row m's argmax to argmax[m].
int launch_decode_argmax(const nvfp4_gemm_plan* p, int M, const uint8_t* codes,
                         const uint8_t* scales, float ts, const uint16_t* act, float* out,
                         void* ws, size_t partial_off, void* area, int* argmax,
                         hipStream_t s) {
    const ArgmaxArgs am{(unsigned long long*)area};
    const int st = launch_w<false>(p, M, codes, scales, ts, act, out, ws, partial_off, am, s);
    if (st) return st;
    hipLaunchKernelGGL(argmax_merge_kernel, dim3(M), dim3(256), 0, s,
                       (const unsigned long long*)area, p->dec.n_groups, argmax);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

}  // namespace nvfp4
