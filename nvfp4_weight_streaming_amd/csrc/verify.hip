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
// G = ceil(M / 16) MFMAs of the step.
//
// Work decomposition.  Column groups (WAVES tiles) are dealt to the 8 XCDs
// round-robin; on each XCD the groups' windows form one sequence (group by
// group, K order within a group), and the XCD's workgroups take equal
// contiguous ranges of it.  A range may end inside one group and go on into
// the next, so every compute unit gets the same number of windows whatever
// the matrix's shape (a per-group K split leaves some units a whole extra
// workgroup when the groups do not divide evenly), and a workgroup streams
// its windows without a pause at a group boundary: the next group's first
// window is in flight while the previous group's sums are handed off.  A
// group covered by several workgroups is added by the deterministic
// last-arriver hand-off of the M <= 8 kernel: each contributor stores its
// partial sums in its own slot, the last to arrive adds the slots in
// workgroup order.  The contributors of a group are consecutive workgroups
// of one XCD, so the partial sums stay in that XCD's L2.
#include "decode_device.h"
#include <algorithm>
#include <type_traits>

namespace nvfp4 {


// End of a group's windows in this workgroup: the outputs (the group is
// wholly this workgroup's, nc = 1), or the hand-off among the group's nc
// contributors, this one the ci-th.  acc[gi][j] holds row 16 gi + 4 (lane /
// 16) + j, column lane % 16 of the wave's tile.
template <int WAVES, int G, bool BF16>
__device__ __forceinline__ void verify_finish(const f32x4 (&acc)[G], void* __restrict__ out,
                                              float* __restrict__ partial,
                                              unsigned int* __restrict__ counters, float ts,
                                              int M, int N, int n_tiles, int l2_local, int ng,
                                              int nc, int ci, int slots, int* s_last) {
    constexpr int kThreads = WAVES * 64;
    constexpr int kCols = WAVES * kTileN;
    constexpr int kRows = 16 * G;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int col = lane & 15, g = lane >> 4;
    const bool mine = ng * WAVES + wave < n_tiles;
    // (M and N opaque here: the output row offsets and row masks are then
    // computed where they are used, not hoisted out of the window loop into
    // 4 G register pairs held for the whole kernel)
    asm volatile("" : "+s"(M), "+s"(N));

    if (nc == 1) {
        if (mine) {
            const int n = (ng * WAVES + wave) * kTileN + col;
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

    // Several contributors: the last-arriver hand-off of the M <= 8 kernel,
    // with each lane's sums stored in its own accumulator layout (slot c,
    // row group gi: one 16-byte word per thread), kept in this XCD's L2 when
    // the workgroup-to-XCD mapping is verified, else device-coherent.
    constexpr int kSlot = 4 * G * kThreads;  // floats per slot
    f32x4* slot0 = (f32x4*)(partial + (size_t)ng * slots * kSlot) + threadIdx.x;
    {
        f32x4* dst = slot0 + (size_t)ci * (kSlot / 4);
#pragma unroll
        for (int gi = 0; gi < G; ++gi) {
            if (l2_local) {
                dst[gi * kThreads] = acc[gi];
            } else {
                float* d4 = (float*)(dst + gi * kThreads);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    __hip_atomic_store(d4 + j, acc[gi][j], __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
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
        *s_last = (old == (unsigned int)(nc - 1));
    }
    __syncthreads();
    if (!*s_last) return;
    if (threadIdx.x == 0) {  // leave the counter zeroed for the next run
        if (l2_local)
            __hip_atomic_store(&counters[ng], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_store(&counters[ng], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    }
    if (!mine) return;
    // The slots in contributor order (this workgroup's own from registers):
    // the same sum whichever contributor arrives last.  Loads of kB slots are
    // in flight at once (one round trip per kB slots).
    constexpr int kB = G <= 2 ? 4 : 2;
    f32x4 sum[G];
#pragma unroll
    for (int gi = 0; gi < G; ++gi) sum[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
    for (int c0 = 0; c0 < nc; c0 += kB) {
        f32x4 v[kB][G];
#pragma unroll
        for (int u = 0; u < kB; ++u) {
            const int c = c0 + u;
            const f32x4* src = slot0 + (size_t)c * (kSlot / 4);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                if (c >= nc || c == ci) {
                    v[u][gi] = acc[gi];
                } else if (l2_local) {
                    v[u][gi] = src[gi * kThreads];
                } else {
                    const float* s4 = (const float*)(src + gi * kThreads);
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        v[u][gi][j] = __hip_atomic_load(s4 + j, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        }
#pragma unroll
        for (int u = 0; u < kB; ++u)
            if (c0 + u < nc)
#pragma unroll
                for (int gi = 0; gi < G; ++gi) sum[gi] += v[u][gi];
    }
    const int n = (ng * WAVES + wave) * kTileN + col;
#pragma unroll
    for (int gi = 0; gi < G; ++gi)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int mm = 16 * gi + 4 * g + j;
            if (mm < M && n < N) store_out<BF16>(out, (size_t)mm * N + n, sum[gi][j] * ts);
        }
}

// Contributors of window sequence positions: with T windows on an XCD split
// into Q equal ranges, range q is [floor(q T / Q), floor((q + 1) T / Q)), and
// position s lies in range floor(((s + 1) Q - 1) / T).
__host__ __device__ inline int verify_range_of(long long s, long long T, int Q) {
    return (int)(((s + 1) * Q - 1) / T);
}

// Window length in 128-k chunks: a whole superblock for 16 rows, half a
// superblock (the activations of a superblock of 64 rows are 64 KiB per
// buffer) for more.  At 16 rows the whole-superblock window halves the
// per-window latency paid per byte: qkv and o 8% faster than with half
// windows in the same plan.
constexpr int verify_kbw(int G) { return G == 1 ? 4 : 2; }

// Weights of one window: KBW code chunks (16 B per lane each, 4 MFMA steps
// apiece) and their KBW scale words (one E4M3 byte per step).
template <int KBW>
struct VWin {
    uint4 c[KBW];
    uint32_t s[KBW];
};

typedef unsigned int u32v2 __attribute__((ext_vector_type(2)));

// One workgroup = WAVES column tiles, streaming its range of the XCD's window
// sequence (windows of 128 KBW k).  Window i's weights (KBW + 1 loads per
// lane) and activation rows (16 G rows) are issued before window i - 1 is
// computed, across group boundaries too; loads complete in order per wave, so
// the wait before window i is the constant vmcnt of one window's loads.
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
    unsigned int* __restrict__ counters, float ts, int M, int K, int N, int nsb, int n_groups,
    int n_tiles, int l2_local, int per_xcd, int slots, int slice_sb) {
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

    // This workgroup's range of the XCD's window sequence: groups xcd,
    // xcd + 8, ... (local index j), nwg windows each.  Either one K slice of
    // slice_sb superblocks of one group (slice_sb > 0: `slots` slices per
    // group), or the q-th of per_xcd equal ranges of the XCD's superblocks.
    const int b = blockIdx.x;
    const int xcd = b & 7, q = b >> 3;
    const int n_x = (n_groups - xcd + 7) >> 3;
    const int nwg = nsb * kWinPerSb;
    const long long T = (long long)n_x * nsb;
    int start, len;
    if (slice_sb) {
        const int j = q / slots, sb0 = (q - j * slots) * slice_sb;
        if (j >= n_x) return;  // whole workgroup: padding of the groups to 8
        start = (j * nsb + sb0) * kWinPerSb;
        len = (min(nsb, sb0 + slice_sb) - sb0) * kWinPerSb;
    } else {
        start = kWinPerSb * (int)(T * q / per_xcd);
        len = kWinPerSb * (int)(T * (q + 1) / per_xcd) - start;
        if (len <= 0) return;  // whole workgroup: more ranges than superblocks
    }

    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int col = lane & 15, g = lane >> 4;
    const __amdgpu_buffer_rsrc_t act_rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(act), 0, M * K * (int)sizeof(uint16_t), 0x00020000);
    // This lane's slot in a copy: row r0 + lane / kSlots, slot lane % kSlots.
    const int c_row = lane / kSlots, c_slot = lane % kSlots;

    // Window i of the range (i < len): weights into x, activation rows into
    // buf.  Row r of the window is activation row min(r, M - 1) (rows >= M
    // are never stored).
    auto issue = [&](int i, VWin<KBW>& x, __bf16* buf) {
        const int it = start + i;
        const int j = it / nwg, w = it - j * nwg;
        const int nt = min((j * 8 + xcd) * WAVES + wave, n_tiles - 1);
        const uint4* cp = codes + (size_t)nt * nsb * 256 + lane;
        const uint4* sp = scales + (size_t)nt * nsb * 32 + col * 2 + (g >> 1);
        const int sb = w / kWinPerSb, kb0 = (w % kWinPerSb) * KBW;
#pragma unroll
        for (int u = 0; u < KBW; ++u) x.c[u] = load_stream(cp + 256 * sb + 64 * (kb0 + u));
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
        const int k = w * kWinK;
#pragma unroll
        for (int u = 0; u < kSeg; ++u) {
            // copies past the last repeat it (same bytes to the same place)
            const int ci = min(wave * kSeg + u, kCopies - 1);
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
    // next (a compile-time true or false): window i + 1 exists and is issued
    // first, into y and nxt.  The loop has the decode kernel's shape (steady
    // state that always issues, separate last windows, scheduling barriers
    // around the waits), so the compiler adds no waits of its own: measured
    // 3-4% off the verify-width rounds.
    auto step = [&](int i, auto next, VWin<KBW>& x, VWin<KBW>& y, const __bf16* cur,
                    __bf16* nxt) {
        // (scheduling barriers: no instruction of the previous or next window's
        // compute moves across the issue and the waits)
        __builtin_amdgcn_sched_barrier(0);
        // Every wave is done reading nxt (window i - 1).
        __builtin_amdgcn_s_waitcnt(kLgkmcnt0);
        barrier_nofence();
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (decltype(next)::value) {
            issue(i + 1, y, nxt);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(kLoads));
        } else {
            __builtin_amdgcn_s_waitcnt(vmcnt_imm(0));
        }
        barrier_nofence();  // every wave's activation rows of window i are in LDS
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (!decltype(next)::value) {
            // (all loads are complete here: marking the registers costs no wait)
#pragma unroll
            for (int u = 0; u < KBW; ++u) {
                opaque(x.c[u]);
                opaque(x.s[u]);
            }
        }
        // Steps of 32 k, software-pipelined: the MFMAs of step t are issued
        // one at a time, each followed by one A-fragment read and a share of
        // the dequantisation of step t + 1, so that the VALU work runs while
        // the matrix core is busy (the B operand is double-buffered).  The A
        // fragments of a step are read one step ahead, so no MFMA waits on a
        // read issued just before.
        constexpr int kSteps = 4 * KBW;
        // VALU operations of one step's dequantisation: the scale conversion,
        // then 4 per pair of codes.
        constexpr int kDeqOps = 17;
        // One A fragment per row group: the read for step t + 1 follows the
        // MFMA of step t that used the register.
        bf16x8 av[G];
        bf16x8 bv[2];
        auto read_a = [&](int t, int gi) {
            av[gi] = *(const bf16x8*)(cur + a_off[t & 3] + 16 * gi * kWinK + 32 * (t & ~3));
        };
        auto dequant = [&](int t) {
            const int kb = t >> 2, s4 = t & 3;
            const int sw = (int)x.s[kb];
            const float sc = s4 == 0   ? __builtin_amdgcn_cvt_f32_fp8(sw, 0)
                             : s4 == 1 ? __builtin_amdgcn_cvt_f32_fp8(sw, 1)
                             : s4 == 2 ? __builtin_amdgcn_cvt_f32_fp8(sw, 2)
                                       : __builtin_amdgcn_cvt_f32_fp8(sw, 3);
            return e2m1x8_scaled_bf16(word(x.c[kb], s4), sc);
        };
#pragma unroll
        for (int gi = 0; gi < G; ++gi) read_a(0, gi);
        bv[0] = dequant(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int t = 0; t < kSteps; ++t) {
            if (t + 1 < kSteps) bv[(t + 1) & 1] = dequant(t + 1);
#pragma unroll
            for (int gi = 0; gi < G; ++gi) {
                acc[gi] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[gi], bv[t & 1], acc[gi], 0,
                                                                  0, 0);
                if (t + 1 < kSteps) read_a(t + 1, gi);
            }
            if (t + 1 < kSteps) {
#pragma unroll
                for (int gi = 0; gi < G; ++gi) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
                    __builtin_amdgcn_sched_group_barrier(0x002, (kDeqOps + G - 1) / G, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using Yes = std::integral_constant<bool, true>;
    using No = std::integral_constant<bool, false>;
    // The hand-off of group j after its last window in this range (the next
    // group's first window is already in flight).
    auto finish = [&](int j) {
        int nc, ci;  // contributors of group j, and this workgroup's index among them
        if (slice_sb) {
            nc = slots;
            ci = q - (q / slots) * slots;
        } else {
            const int q_lo = verify_range_of((long long)j * nsb, T, per_xcd);
            nc = verify_range_of((long long)(j + 1) * nsb - 1, T, per_xcd) - q_lo + 1;
            ci = q - q_lo;
        }
        verify_finish<WAVES, G, BF16>(acc, out, partial, counters, ts, M, N, n_tiles, l2_local,
                                      j * 8 + xcd, nc, ci, slots, &s_last);
#pragma unroll
        for (int gi = 0; gi < G; ++gi) acc[gi] = f32x4{0.f, 0.f, 0.f, 0.f};
    };
    // A steady state that always issues the next window, then the last
    // windows apart: with the choice of issuing made inside the loop, the
    // compiler gave the two window register sets different places on the two
    // paths and, at the loop's end, copied them, waiting for the loads in
    // flight.
    VWin<KBW> wa, wb;
    issue(0, wa, lds0);
    int i = 0;
    if constexpr (kWinPerSb == 2) {
        // Superblock by superblock: window i (even) computes from (wa, lds0),
        // window i + 1 from (wb, lds1); a group ends only after an odd window.
        auto after_sb = [&](int e) {  // e: first window after the superblock
            const int it = start + e;
            const int j = (it - 1) / nwg;
            if (it == (j + 1) * nwg || e == len) finish(j);
        };
        for (; i + 2 < len; i += 2) {
            step(i, Yes{}, wa, wb, lds0, lds1);
            step(i + 1, Yes{}, wb, wa, lds1, lds0);
            after_sb(i + 2);
        }
        step(i, Yes{}, wa, wb, lds0, lds1);
        step(i + 1, No{}, wb, wa, lds1, lds0);
        after_sb(i + 2);
    } else {
        // Window = superblock: even windows compute from (wa, lds0), odd ones
        // from (wb, lds1), and a group may end after either.
        auto after = [&](int w) {
            const int it = start + w + 1;
            const int j = (it - 1) / nwg;
            if (it == (j + 1) * nwg || w + 1 == len) finish(j);
        };
        for (; i + 2 < len; i += 2) {
            step(i, Yes{}, wa, wb, lds0, lds1);
            after(i);
            step(i + 1, Yes{}, wb, wa, lds1, lds0);
            after(i + 1);
        }
        if (i + 1 < len) {
            step(i, Yes{}, wa, wb, lds0, lds1);
            after(i);
            step(i + 1, No{}, wb, wa, lds1, lds0);
            after(i + 1);
        } else {
            step(i, No{}, wa, wb, lds0, lds1);
            after(i);
        }
    }
}

// LDS of the kernel's own arrays for G row groups (two activation windows),
// and the LDS a workgroup requests in all when it must have a compute unit to
// itself (more than half of the 160 KiB).
constexpr int verify_static_lds(int G) { return 2 * 16 * G * 128 * verify_kbw(G) * 2; }
constexpr int kVerifyLdsPerUnit = 84 * 1024;

// Per-group K slices: `waves` column tiles per workgroup, each group's K cut
// into slices of slice_sb superblocks (one workgroup per slice; the last may
// be shorter); a workspace for `rows` rows.
static void verify_slices_config(int n_tiles, int nsb, int waves, int rows, int slice_sb,
                                 DecodeConfig& d) {
    d = DecodeConfig{};
    const int n_groups = (n_tiles + waves - 1) / waves;
    const int ng8 = round_up(n_groups, 8);
    if (slice_sb > nsb) slice_sb = nsb;
    const int splits = (nsb + slice_sb - 1) / slice_sb;
    d.waves = waves;
    d.chunks = 1;
    d.windows = slice_sb;
    d.splits = splits;
    d.n_groups = n_groups;
    d.per_xcd = ng8 / 8 * splits;
    d.slots = splits;
    d.grid = ng8 * splits;
    d.l2_local = splits > 1 ? xcd_mapping_verified() : 0;
    if (splits > 1) {
        d.counter_bytes = ((size_t)ng8 * sizeof(unsigned int) + 255) / 256 * 256;
        d.partial_bytes = (size_t)ng8 * splits * rows * waves * kTileN * sizeof(float);
    }
    d.ws_bytes = d.counter_bytes + d.partial_bytes;
}

// Equal ranges: `waves` column tiles per workgroup, `per_cu` workgroups per
// compute unit taking equal ranges of their XCD's superblocks (a range runs
// on from one group into the next); a workspace for `rows` rows.  With one
// workgroup per unit, each requests more than half a unit's LDS, so that the
// dispatcher cannot place two on one unit while another idles.
static void verify_ranges_config(int n_tiles, int nsb, int waves, int G, int rows, int per_cu,
                                 DecodeConfig& d) {
    d = DecodeConfig{};
    const int n_groups = (n_tiles + waves - 1) / waves;
    const int ng8 = round_up(n_groups, 8);
    // Every range non-empty on every XCD that has groups (an empty range
    // would be counted as a contributor that never arrives): at most as many
    // workgroups per XCD as the XCD with the fewest groups has superblocks.
    const long long t_min = (long long)std::max(1, n_groups / 8) * nsb;
    const long long q = std::max(1LL, std::min((long long)per_cu * std::max(1, device_cus() / 8),
                                               t_min));
    int slots = 1;
    for (int x = 0; x < 8; ++x) {
        const int n_x = (n_groups - x + 7) / 8;
        const long long t = (long long)n_x * nsb;
        for (int j = 0; j < n_x; ++j) {
            const int lo = verify_range_of((long long)j * nsb, t, (int)q);
            const int hi = verify_range_of((long long)(j + 1) * nsb - 1, t, (int)q);
            slots = std::max(slots, hi - lo + 1);
        }
    }
    d.waves = waves;
    d.chunks = 1;
    d.windows = 0;      // (equal ranges, not slices)
    d.splits = slots;   // most workgroups adding into one group
    d.n_groups = n_groups;
    d.per_xcd = (int)q;
    d.slots = slots;
    d.grid = 8 * (int)q;
    d.l2_local = slots > 1 ? xcd_mapping_verified() : 0;
    if (per_cu == 1) d.lds_pad = std::max(0, kVerifyLdsPerUnit - verify_static_lds(G));
    if (slots > 1) {
        d.counter_bytes = ((size_t)ng8 * sizeof(unsigned int) + 255) / 256 * 256;
        d.partial_bytes = (size_t)ng8 * slots * rows * waves * kTileN * sizeof(float);
    }
    d.ws_bytes = d.counter_bytes + d.partial_bytes;
}

// Default slice length for per-group slices: as many slices as still give
// every workgroup its own compute unit when the groups are fewer than the
// units (a workgroup of 48-64 rows holds a unit's LDS alone, so a grid a
// little larger than the unit count runs a second, nearly empty round); two
// for more groups (6 superblocks for a long K); none for groups that alone
// give every unit 4 workgroups.
static int verify_default_slice(int n_tiles, int nsb, int waves) {
    const int n_groups = (n_tiles + waves - 1) / waves;
    const int ng8 = round_up(n_groups, 8), cus = device_cus();
    if (n_groups >= 4 * cus) return nsb;
    if (ng8 < cus) {
        const int pieces = cus / ng8;
        return (nsb + pieces - 1) / pieces;
    }
    return nsb >= 32 ? 6 : (nsb + 1) / 2;
}

// Plan, per count G of 16-row groups (measured on the 27B-class round's
// shapes, per matrix, in one process against each alternative):
//  - 17..64 rows with more 4-tile column groups than compute units (gate_up):
//    one 8-wave workgroup per unit over equal ranges (M = 32: 35.7 us
//    against 38.7 with per-group slices; M = 64: 46.5 against 52.5);
//  - otherwise per-group slices of the default length, 4 waves, except for
//    a long K (>= 32 superblocks: down): slices of 6 superblocks, with 8
//    waves above 16 rows (M = 17: 18.2 us against 20.6, M = 32: 19.4
//    against 21.4, M = 48: 24.4 against 25.0, M = 64: 25.4 against 27.3
//    with 4 waves and 3 slices) and 4 waves up to 16 when the groups are
//    fewer than the units (M = 16: 15.9 against 16.4 with 3 slices).
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
    if (cfg && (cfg->verify_ranges < 0 || cfg->verify_ranges > 4))
        return set_error(NVFP4_EINVAL, "config.verify_ranges: %d is not 0..4", cfg->verify_ranges);
    if (cfg && cfg->verify_ranges && cfg->verify_windows)
        return set_error(NVFP4_EINVAL, "config.verify_ranges and config.verify_windows: both set");
    const int slice = cfg ? cfg->verify_windows : 0;
    const int ranges = cfg ? cfg->verify_ranges : 0;
    const bool many = round_up((n_tiles + 3) / 4, 8) >= device_cus();
    const bool long_k = nsb >= 32;
    DecodeConfig& d = v->d;
    for (int G = 1; G <= v->rows / 16; ++G) {
        DecodeConfig& c = v->g[G - 1];
        if (ranges || (!slice && G >= 2 && many)) {
            verify_ranges_config(n_tiles, nsb, forced ? forced : 8, G, v->rows,
                                 ranges ? ranges : 1, c);
        } else {
            const int waves = forced ? forced : long_k && G >= 2 ? 8 : 4;
            // (up to 16 rows only where the groups are fewer than the units)
            const bool few = round_up((n_tiles + waves - 1) / waves, 8) < device_cus();
            int sl = slice ? slice : verify_default_slice(n_tiles, nsb, waves);
            if (!slice && !forced && long_k && (G >= 2 || few)) sl = 6;
            verify_slices_config(n_tiles, nsb, waves, v->rows, sl, c);
        }
        d.counter_bytes = std::max(d.counter_bytes, c.counter_bytes);
        d.partial_bytes = std::max(d.partial_bytes, c.partial_bytes);
    }
    d.ws_bytes = d.counter_bytes + d.partial_bytes;
    return NVFP4_OK;
}

int launch_verify(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                  float ts, const uint16_t* act, void* out, void* ws, size_t counters_off,
                  size_t partial_off, hipStream_t s) {
    const int G = (M + 15) / 16;
    const DecodeConfig& d = p->ver.g[G - 1];
    unsigned int* counters = d.slots > 1 ? (unsigned int*)((char*)ws + counters_off) : nullptr;
    float* partial = d.slots > 1 ? (float*)((char*)ws + partial_off) : nullptr;
    const bool bf16 = p->out_dtype == NVFP4_OUT_BF16;
    const dim3 grid(d.grid), block(d.waves * 64);
    const int nsb = p->Kp / kSuperK, n_tiles = p->Np / kTileN;
#define NVFP4_VERIFY_LAUNCH(WW, GG, BB)                                                       \
    if (d.lds_pad > 64 * 1024) /* above the default limit of dynamic LDS */                    \
        NVFP4_HIP(hipFuncSetAttribute((const void*)verify_kernel<WW, GG, BB>,                  \
                                      hipFuncAttributeMaxDynamicSharedMemorySize, d.lds_pad));  \
    hipLaunchKernelGGL((verify_kernel<WW, GG, BB>), grid, block, d.lds_pad, s, (const uint4*)codes, \
                       (const uint4*)scales, act, out, partial, counters, ts, M, p->K, p->N,   \
                       nsb, d.n_groups, n_tiles, d.l2_local, d.per_xcd, d.slots, d.windows)
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
