// Verify-width decode GEMM: 8 < M <= 64 rows served by one pass over NVFP4
// weights.
//
// "Ignis" README, "Speculative decoding (DFlash2)": a drafter proposes up to
// seven tokens per lane and the model checks them in the same pass, so one
// round multiplies lanes x (1 + drafts) <= 64 activation rows by each weight
// matrix.  That is still one read of every weight byte ("The decode round":
// the round streams the weights at the card's bandwidth); only the work per
// byte grows, up to 128 flops at M = 64.
//
// gfx950 mapping.  As in the M <= 8 kernel, one wave owns a tile of 16
// output columns and streams a K slice window by window (one 512-k
// superblock per window, the next window's loads in flight while the current
// one is computed), and a workgroup of WAVES tiles stages the activation rows
// of a window in LDS with direct-to-LDS copies.  The multiply differs:
//   B operand (32 k x 16 columns): each lane turns its 8 codes of the step
//     into 8 exact bf16 values of code x E4M3 block scale (at most 6
//     significant bits).  The 8 values of a lane lie in one 16-k block, so a
//     lane needs one scale per step.
//   A operand (16 rows x 32 k): 16 activation rows, one MFMA
//     (v_mfma_f32_16x16x32_bf16) per 16-row group accumulates into that
//     group's fp32 sums directly.
// The dequantisation (16 VALU operations per lane and step) is shared by the
// G = ceil(M / 16) MFMAs of the step.  Split-K and the deterministic
// last-workgroup hand-off are those of the M <= 8 kernel, for 16 G rows.
#include "decode_device.h"
#include <algorithm>
#include <type_traits>

namespace nvfp4 {

constexpr int kVerifyWaves = 4;       // waves per workgroup by default
constexpr int kVerifyWavesWide = 8;   // G = 4 with many column groups; long K at G = 2, 3

// End of a workgroup: outputs (one slice) or the split-K hand-off (several).
// acc[gi][j] holds row 16 gi + 4 (lane / 16) + j, column lane % 16 of the
// wave's tile.
template <int WAVES, int G, bool BF16>
__device__ __forceinline__ void verify_finish(const f32x4 (&acc)[G], void* __restrict__ out,
                                              float* __restrict__ partial,
                                              unsigned int* __restrict__ counters, float ts,
                                              int M, int N, int splits, int n_tiles, int l2_local,
                                              int ng, int split, int nt, int* s_last) {
    constexpr int kThreads = WAVES * 64;
    constexpr int kCols = WAVES * kTileN;
    constexpr int kRows = 16 * G;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, g = lane >> 4;
    const bool mine = ng * WAVES + wave < n_tiles;

    if (splits == 1) {
        if (mine) {
            const int n = nt * kTileN + col;
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int mm = 16 * gi + 4 * g + j;
                    if (mm < M && n < N) store_out<BF16>(out, (size_t)mm * N + n, acc[gi][j] * ts);
                }
        }
        return;
    }

    // Split K: the same hand-off as the M <= 8 kernel (partials in this XCD's
    // L2 when the workgroup-to-XCD mapping is verified, else device-coherent).
    float* pbase = partial + (size_t)(ng * splits + split) * kRows * kCols;
    if (mine) {
#pragma unroll
        for (int gi = 0; gi < G; ++gi)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int mm = 16 * gi + 4 * g + j;
                if (mm < M) {
                    float* dst = pbase + mm * kCols + wave * kTileN + col;
                    if (l2_local)
                        *dst = acc[gi][j];
                    else
                        __hip_atomic_store(dst, acc[gi][j], __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT);
                }
            }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (threadIdx.x == 0) {
        const unsigned int old =
            __hip_atomic_fetch_add(&counters[ng], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *s_last = (old == (unsigned int)(splits - 1));
    }
    __syncthreads();
    if (!*s_last) return;
    const float* gbase = partial + (size_t)ng * splits * kRows * kCols;
    constexpr int kR = kRows * kCols / kThreads;
    static_assert(kRows * kCols % kThreads == 0 && kR <= 16, "outputs divide over the threads");
    float sum[kR];
    if (l2_local)
        sum_partials<kCols, kThreads, kR, true, kRows>(gbase, splits, M * kCols, sum);
    else
        sum_partials<kCols, kThreads, kR, false, kRows>(gbase, splits, M * kCols, sum);
#pragma unroll
    for (int r = 0; r < kR; ++r) {
        const int idx = threadIdx.x + r * kThreads;
        const int mm = idx / kCols, c = idx - mm * kCols;
        const int n = ng * kCols + c;
        if (idx < M * kCols && n < N) store_out<BF16>(out, (size_t)mm * N + n, sum[r] * ts);
    }
    if (threadIdx.x == 0)  // leave the counter zeroed for the next run
        __hip_atomic_store(&counters[ng], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Window length (in 128-k chunks) for G row groups: with 48 or 64 rows a
// superblock's activations take 50-66 KiB of LDS per buffer, so the window is
// half a superblock and two workgroups fit on a compute unit.  At 32 rows the
// half-superblock window measured 6% faster over the round (more workgroups
// per compute unit); at 16 rows the whole superblock is 9% faster.
constexpr int verify_kbw(int G) { return G >= 2 ? 2 : 4; }

// Weights of one window: KBW code chunks (16 B per lane each, 4 MFMA steps
// apiece) and their KBW scale words (one E4M3 byte per step).
template <int KBW>
struct VWin {
    uint4 c[KBW];
    uint32_t s[KBW];
};

typedef unsigned int u32v2 __attribute__((ext_vector_type(2)));

// One workgroup = WAVES column tiles x one K slice of `slice_sb` superblocks,
// streamed in windows of 128 KBW k.  Window w's weights (KBW + 1 loads per
// lane) and activation rows (16 G rows) are issued before window w - 1 is
// computed; loads complete in order per wave, so the wait before window w is
// the constant vmcnt of one window's loads.
//
// LDS rows hold one window of one activation row, unpadded (1 KiB or 512 B),
// in 16-byte segments: segment j of row r sits in slot j ^ (r % 16).  An
// operand read serves 16 lanes (rows r0 .. r0 + 15, one segment) per pass and
// a row's bank group is its slot % 16, so those reads cover all banks once.
// A direct-to-LDS copy writes 1 KiB to consecutive slots (one row, or two
// rows of a half-superblock window); each lane fetches the segment its slot
// needs.  The copies address the whole activation buffer: k past K reads the
// next row (finite values; the weights there are zero) and the last row's
// tail reads zero.
template <int WAVES, int G, bool BF16>
__global__ __launch_bounds__(WAVES * 64) void verify_kernel(
    const uint4* __restrict__ codes, const uint4* __restrict__ scales,
    const uint16_t* __restrict__ act, void* __restrict__ out, float* __restrict__ partial,
    unsigned int* __restrict__ counters, float ts, int M, int K, int N, int nsb, int splits,
    int n_groups, int n_tiles, int l2_local, int slice_sb) {
    constexpr int KBW = verify_kbw(G);
    constexpr int kWinK = 128 * KBW;            // k per window = bf16 per LDS row
    constexpr int kWinPerSb = 4 / KBW;
    constexpr int kSlots = kWinK / 8;           // 16-byte segments per row: 64 or 32
    constexpr int kRows = 16 * G;
    constexpr int kRowsPerCopy = 64 / kSlots;   // rows one 1 KiB copy fills: 1 or 2
    constexpr int kCopies = kRows / kRowsPerCopy;
    constexpr int kSeg = (kCopies + WAVES - 1) / WAVES;  // copies per wave per window
    constexpr int kLoads = KBW + 1 + kSeg;      // loads a wave issues per window
    // Two separate arrays: the compiler then sees that copies into one never
    // alias reads of the other.
    __shared__ __attribute__((aligned(16))) __bf16 lds0[kRows * kWinK];
    __shared__ __attribute__((aligned(16))) __bf16 lds1[kRows * kWinK];
    __shared__ int s_last;

    const int b = blockIdx.x;
    const int xcd = b & 7, q = b >> 3;
    const int ng = (q / splits) * 8 + xcd;
    const int split = q - (q / splits) * splits;
    if (ng >= n_groups) return;  // whole workgroup: padding of the column groups to 8
    const int w_begin = split * slice_sb * kWinPerSb;                       // first window
    const int nwin = min(slice_sb * kWinPerSb, nsb * kWinPerSb - w_begin);  // >= 1

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int nt = min(ng * WAVES + wave, n_tiles - 1);
    const int col = lane & 15, g = lane >> 4;
    const uint4* cp = codes + (size_t)nt * nsb * 256 + lane;
    const uint4* sp = scales + (size_t)nt * nsb * 32 + col * 2 + (g >> 1);
    const __amdgpu_buffer_rsrc_t act_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(act), 0, M * K * (int)sizeof(uint16_t), 0x00020000);
    // This lane's slot in a copy: row r0 + lane / kSlots, slot lane % kSlots.
    const int c_row = lane / kSlots, c_slot = lane % kSlots;

    // Window w: weights into x, activation rows into buf.  Row r of the
    // window is activation row min(r, M - 1) (rows >= M are never stored).
    auto issue = [&](int w, VWin<KBW>& x, __bf16* buf) {
        const int gw = w_begin + min(w, nwin - 1);
        const int sb = gw / kWinPerSb, kb0 = (gw % kWinPerSb) * KBW;
#pragma unroll
        for (int i = 0; i < KBW; ++i) x.c[i] = load_stream(cp + 256 * sb + 64 * (kb0 + i));
        if constexpr (KBW == 4) {
            const uint4 v = load_stream(sp + 32 * sb);
            x.s[0] = v.x;
            x.s[1] = v.y;
            x.s[2] = v.z;
            x.s[3] = v.w;
        } else {
            const u32v2 v =
                __builtin_nontemporal_load((const u32v2*)(sp + 32 * sb) + (kb0 >> 1));
            x.s[0] = v.x;
            x.s[1] = v.y;
        }
        const int k = gw * kWinK;
#pragma unroll
        for (int j = 0; j < kSeg; ++j) {
            // copies past the last repeat it (same bytes to the same place)
            const int ci = min(wave * kSeg + j, kCopies - 1);
            const int r0 = ci * kRowsPerCopy, r = r0 + c_row;
            const int seg = c_slot ^ (r & 15);
            const int voff = ((min(r, M - 1) * K + k) + 8 * seg) * (int)sizeof(uint16_t);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                act_rs, (__attribute__((address_space(3))) void*)(buf + r0 * kWinK), 16, voff,
                0, 0, 0);
        }
    };

    f32x4 acc[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) acc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
    // A operand of this lane at step t: row col of each 16-row group, segment
    // 4 t + g, in slot (4 t + g) ^ col = 4 (t ^ (col / 4)) + (g ^ (col % 4)):
    // the four offsets for t % 4 = 0..3, plus 32 (t - t % 4) bf16.
    int a_off[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) a_off[u] = col * kWinK + 8 * (4 * (u ^ (col >> 2)) + (g ^ (col & 3)));
    // next (a compile-time true or false): window w + 1 exists and is issued
    // first, into y and nxt.  The loop has the decode kernel's shape (steady
    // state that always issues, separate last windows, scheduling barriers
    // around the waits), so the compiler adds no waits of its own: measured
    // 3-4% off the verify-width rounds.
    auto step = [&](int w, auto next, VWin<KBW>& x, VWin<KBW>& y, const __bf16* cur,
                    __bf16* nxt) {
        // (scheduling barriers: no instruction of the previous or next window's
        // compute moves across the issue and the waits)
        __builtin_amdgcn_sched_barrier(0);
        // Every wave is done reading nxt (window w - 1).
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
        barrier_nofence();  // every wave's activation rows of window w are in LDS
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!decltype(next)::value) {
            // (all loads are complete here: marking the registers costs no wait)
#pragma unroll
            for (int i = 0; i < KBW; ++i) {
                opaque(x.c[i]);
                opaque(x.s[i]);
            }
        }
        // Steps of 32 k.  The A fragments of step t + 1 are read before the
        // multiplies of step t, so no MFMA waits on a read issued just before.
        constexpr int kSteps = 4 * KBW;
        bf16x8 av[2][G];
        auto read_a = [&](int t, bf16x8 (&dst)[G]) {
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
                dst[gi] = *(const bf16x8*)(cur + a_off[t & 3] + 16 * gi * kWinK + 32 * (t & ~3));
        };
        read_a(0, av[0]);
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
            const int kb = t >> 2, s = t & 3;
            if (t + 1 < kSteps) read_a(t + 1, av[(t + 1) & 1]);
            // keep those reads ahead of this step's work (the scheduler would
            // otherwise move each read next to its use)
            __builtin_amdgcn_sched_barrier(0);
            const int sw = (int)x.s[kb];
            const float sc = s == 0   ? __builtin_amdgcn_cvt_f32_fp8(sw, 0)
                             : s == 1 ? __builtin_amdgcn_cvt_f32_fp8(sw, 1)
                             : s == 2 ? __builtin_amdgcn_cvt_f32_fp8(sw, 2)
                                      : __builtin_amdgcn_cvt_f32_fp8(sw, 3);
            const bf16x8 bv = e2m1x8_scaled_bf16(word(x.c[kb], s), sc);
#pragma unroll
            for (int gi = 0; gi < G; ++gi)
                acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[t & 1][gi], bv, acc[gi], 0,
                                                                  0, 0);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using Yes = std::integral_constant<bool, true>;
    using No = std::integral_constant<bool, false>;
    VWin<KBW> wa, wb;
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
    verify_finish<WAVES, G, BF16>(acc, out, partial, counters, ts, M, N, splits, n_tiles,
                                  l2_local, ng, split, nt, &s_last);
}

// One launch configuration: `waves` column tiles per workgroup, slices as
// below (no split for column groups that alone give every compute unit 4
// workgroups), a workspace for `rows` rows.
static void verify_launch_config(int n_tiles, int nsb, int waves, int rows,
                                 const nvfp4_gemm_config* cfg, int slice_sb,
                                 DecodeConfig& d) {
    d = DecodeConfig{};
    const int n_groups = (n_tiles + waves - 1) / waves;
    const int ng8 = round_up(n_groups, 8);
    const int cus = device_cus();
    const bool wide = n_groups >= 4 * cus;
    // Fewer column groups than compute units: as many K slices as still give
    // every workgroup its own compute unit.  A workgroup of 48-64 rows holds a
    // compute unit's LDS alone, so a grid a little larger than the unit count
    // runs a second, nearly empty round (qkv: 5 slices of 2 superblocks made
    // 280 workgroups; 4 slices of 3 make 224, and measured 17% faster).
    int windows;
    if (cfg && cfg->verify_windows)
        windows = cfg->verify_windows;
    else if (slice_sb)
        windows = slice_sb;
    else if (wide)
        windows = nsb;
    else if (ng8 < cus) {
        const int s = cus / ng8;
        windows = (nsb + s - 1) / s;
    } else  // many groups: two slices (gate_up, M = 16..64: 6-16% faster than 5 of 2)
        windows = nsb >= 32 ? 6 : (nsb + 1) / 2;
    if (windows > nsb) windows = nsb;
    const int splits = (nsb + windows - 1) / windows;
    d.l2_local = splits > 1 ? xcd_mapping_verified() : 0;
    d.waves = waves;
    d.chunks = 1;
    d.windows = windows;
    d.splits = splits;
    d.n_groups = n_groups;
    d.grid = ng8 * splits;
    if (splits > 1) {
        d.counter_bytes = ((size_t)ng8 * sizeof(unsigned int) + 255) / 256 * 256;
        d.partial_bytes = (size_t)ng8 * splits * rows * waves * kTileN * sizeof(float);
    }
    d.ws_bytes = d.counter_bytes + d.partial_bytes;
}

// Plan, per count G of 16-row groups: 4 waves per workgroup (measured over the
// 64-layer round against 8 throughout: M = 16 -7.6%, M = 40 -3%), except
//  - 8 for 49..64 rows when the column groups of 4 tiles outnumber the
//    compute units (gate_up: 7% faster there; qkv, o and down are 12%, 9%
//    and 3% faster with 4);
//  - 8, with K slices of 6 superblocks, for 17..48 rows of a long K (>= 32
//    superblocks: down), as the M <= 8 kernel's long-K plan (down, repeats
//    interleaved in one process: M = 17 18.2 us against 20.6, M = 32 19.4
//    against 21.4, M = 48 24.4 against 25.0; at 16 and 64 rows the 4-wave
//    plan stays faster).
// The launch configurations share one workspace area sized for the larger
// of each part.
int make_verify_config(int K, int N, int max_M, const nvfp4_gemm_config* cfg, VerifyConfig* v) {
    v->enabled = max_M > NVFP4_DECODE_MAX_M;
    v->ws_off = 0;
    v->rows = 0;
    for (DecodeConfig& g : v->g) g = DecodeConfig{};
    v->d = DecodeConfig{};
    if (!v->enabled) return NVFP4_OK;
    const int m = max_M < NVFP4_VERIFY_MAX_M ? max_M : NVFP4_VERIFY_MAX_M;
    v->rows = (m + 15) / 16 * 16;
    const int n_tiles = padded_n(N) / kTileN;
    const int nsb = padded_k(K) / kSuperK;
    const int forced = cfg ? cfg->verify_waves : 0;
    if (forced && forced != 4 && forced != 8 && forced != 16)
        return set_error(NVFP4_EINVAL, "config.verify_waves: %d is not 4, 8 or 16", forced);
    if (cfg && cfg->verify_windows < 0)
        return set_error(NVFP4_EINVAL, "config.verify_windows: %d < 0", cfg->verify_windows);
    const bool many = round_up((n_tiles + 3) / 4, 8) >= device_cus();
    const bool long_k = nsb >= 32;
    DecodeConfig& d = v->d;
    for (int G = 1; G <= v->rows / 16; ++G) {
        const bool long_mid = long_k && (G == 2 || G == 3);
        const int waves = forced ? forced
                          : (G == 4 && many) || long_mid ? kVerifyWavesWide : kVerifyWaves;
        verify_launch_config(n_tiles, nsb, waves, v->rows, cfg, !forced && long_mid ? 6 : 0,
                             v->g[G - 1]);
        d.counter_bytes = std::max(d.counter_bytes, v->g[G - 1].counter_bytes);
        d.partial_bytes = std::max(d.partial_bytes, v->g[G - 1].partial_bytes);
    }
    d.ws_bytes = d.counter_bytes + d.partial_bytes;
    return NVFP4_OK;
}

int launch_verify(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                  float ts, const uint16_t* act, void* out, void* ws, size_t counters_off,
                  size_t partial_off, hipStream_t s) {
    const int G = (M + 15) / 16;
    const DecodeConfig& d = p->ver.g[G - 1];
    unsigned int* counters = d.splits > 1 ? (unsigned int*)((char*)ws + counters_off) : nullptr;
    float* partial = d.splits > 1 ? (float*)((char*)ws + partial_off) : nullptr;
    const bool bf16 = p->out_dtype == NVFP4_OUT_BF16;
    const dim3 grid(d.grid), block(d.waves * 64);
    const int nsb = p->Kp / kSuperK, n_tiles = p->Np / kTileN;
#define NVFP4_VERIFY_LAUNCH(WW, GG, BB)                                                       \
    hipLaunchKernelGGL((verify_kernel<WW, GG, BB>), grid, block, 0, s, (const uint4*)codes,    \
                       (const uint4*)scales, act, out, partial, counters, ts, M, p->K, p->N,   \
                       nsb, d.splits, d.n_groups, n_tiles, d.l2_local, d.windows)
#define NVFP4_VERIFY_G(WW, BB)                              \
    switch (G) {                                            \
        case 1: NVFP4_VERIFY_LAUNCH(WW, 1, BB); break;      \
        case 2: NVFP4_VERIFY_LAUNCH(WW, 2, BB); break;      \
        case 3: NVFP4_VERIFY_LAUNCH(WW, 3, BB); break;      \
        default: NVFP4_VERIFY_LAUNCH(WW, 4, BB); break;     \
    }
    if (d.waves == 16) {
        if (bf16) NVFP4_VERIFY_G(16, true) else NVFP4_VERIFY_G(16, false)
    } else if (d.waves == 4) {
        if (bf16) NVFP4_VERIFY_G(4, true) else NVFP4_VERIFY_G(4, false)
    } else {
        if (bf16) NVFP4_VERIFY_G(8, true) else NVFP4_VERIFY_G(8, false)
    }
#undef NVFP4_VERIFY_G
#undef NVFP4_VERIFY_LAUNCH
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

}  // namespace nvfp4
