// Chained decode round: every matrix of a round in one launch, the next
// matrix's weight stream running while the previous matrix finishes.
//
// "Ignis" README, "The decode round" (one pass over the weights serves every
// lane; the round replays a captured graph) and "Lineage" -> "Credits" (the
// decode kernels of a round are chained so that one GEMM's start overlaps the
// previous one's drain).  gfx950 has no launch attribute for such an overlap
// between kernels, so here the matrices of a round are the workgroups of one
// grid, in round order:
//   - a workgroup first issues every weight load of its slice (weights depend
//     on nothing), then waits until the previous matrix is complete, then
//     loads its activations and computes as the split-K decode kernel does
//     (decode.hip: same operand mapping, same slices, same hand-off);
//   - completion of matrix i is published in replicated flag words once the
//     last of its column groups has written its outputs.
// Forward progress.  A workgroup takes its place in the round from a ticket
// counter of the XCD it runs on (read from the hardware register), not from
// its workgroup index, because the order in which workgroups are dispatched
// is not specified.  Tickets are handed out in round order, so a workgroup
// holding a ticket of matrix i waits only on matrices < i whose tickets, on
// every XCD, were all taken earlier by workgroups that are resident or done,
// and which in turn wait only on earlier matrices: every wait ends.  This
// needs each XCD to run exactly its share of the grid, which the plan checks
// once by counting a probe launch's workgroups per XCD; every wait is also
// bounded (a time-out raises an error flag instead of hanging).
// Split K stays XCD-local: the slices of a column group hold tickets of one
// XCD (group = (ticket / splits) * 8 + xcd), so their partial sums meet in
// that XCD's L2.  Each matrix has its own counter and partial-sum region, so
// no address is written twice in a launch and no cached line can be stale.
#include <new>

#include "decode_device.h"

namespace nvfp4 {

constexpr int kChainWaves = 4;   // compute waves: one 16-column tile each
constexpr int kChainChunks = 2;  // superblocks of 512 k per K slice
constexpr int kChainFlagSlots = 64;
constexpr int kChainFlagStride = 4096;  // bytes: one flag word per memory channel
constexpr int kChainTicketWords = 64;   // words between the XCDs' ticket counters
constexpr int kChainMaxMats = 1 << 14;  // matrix index field of a ticket record

enum : unsigned int { kChainOutBf16 = 1u, kChainActCoherent = 2u };

// One ticket: a workgroup's share of one matrix, i.e. one K slice of one
// column group on the XCD that takes it (64 bytes, read with scalar loads).
struct alignas(64) ChainTicket {
    const uint4* codes;
    const uint4* scales;
    const uint16_t* act;
    void* out;
    float ts;
    int K, N, splits;
    int n_groups;
    int ng0;              // column group = ng0 + xcd (ng0 is a multiple of 8)
    unsigned int region;  // offset of the matrix's counters + partial sums, in 256-byte units
    unsigned int word;    // kChainOutBf16 | kChainActCoherent | index << 2 | split << 16
};
static_assert(sizeof(ChainTicket) == 64, "ChainTicket is one 64-byte record");

struct ChainSync {
    unsigned int* status;   // [0] error flags, [1] spin limit
    unsigned int* tickets;  // 8 counters, kChainTicketWords apart
    unsigned int* done;     // [n] finished column groups per matrix
    unsigned int* flags;    // kChainFlagSlots words, kChainFlagStride bytes apart
    char* regions;
};

__host__ __device__ inline size_t chain_counter_bytes(int n_groups) {
    return ((size_t)(n_groups + 7) / 8 * 8 * sizeof(unsigned int) + 255) / 256 * 256;
}

// The buffers a ticket names are accessed through buffer resources (base and
// size in scalar registers, 32-bit offsets).  Generic pointers read from
// memory would compile to flat accesses, which also count against the
// scalar-load wait counter: the first scalar wait after the weight loads would
// then wait for the whole weight stream.
typedef unsigned int cu32x4 __attribute__((ext_vector_type(4)));
constexpr int kChainRaw = 0x00020000;  // buffer resource word 3: raw 32-bit data
constexpr int kSc1 = 16;               // cache policy bits: device scope (sc1)
constexpr int kNt = 2;                 // cache policy bits: non-temporal (weights, read once)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t chain_rsrc(const void* base, size_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)bytes, kChainRaw);
}

template <int AUX>
__device__ __forceinline__ uint4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff) {
    const cu32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, (int)soff, AUX);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ unsigned int* chain_flag(unsigned int* flags, int slot) {
    return (unsigned int*)((char*)flags + (size_t)slot * kChainFlagStride);
}

// Device-coherent (sc1) store of output element idx.
__device__ __forceinline__ void store_coherent(__amdgpu_buffer_rsrc_t out, uint32_t idx, float v,
                                               bool bf16) {
    if (bf16)
        __builtin_amdgcn_raw_buffer_store_b16(f32_to_bf16_rne(v), out, (int)(idx * 2), 0, kSc1);
    else
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), out, (int)(idx * 4), 0, kSc1);
}

// WAVES compute waves and one stager wave.  The compute waves issue nothing
// but their weight loads before they compute: because a wave's loads complete
// in order, any later load of theirs would wait for the weights.  The stager
// takes the ticket, waits for the previous matrix and copies the activation
// slice straight into LDS, all while the weights are in flight.
template <int WAVES, int NCH>
__global__ __launch_bounds__((WAVES + 1) * 64) void chain_kernel(
    const ChainTicket* __restrict__ tickets, ChainSync sync, int n_mats, int per_xcd, int M) {
    constexpr int kAll = (WAVES + 1) * 64;
    constexpr int kStride = NCH * kSuperK + kLdsPad;  // LDS activation row, bf16
    constexpr int kCols = WAVES * kTileN;
    __shared__ __attribute__((aligned(16))) __bf16 lds[9 * kStride];
    __shared__ int s_ticket, s_last;

    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool stager = wave == WAVES;

    // 0. Place in the round: the next ticket of this XCD.
    unsigned int xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    const int xcd = (int)(xcc & 7u);
    if (stager && lane == 0) {
        unsigned int* ctr = sync.tickets + xcd * kChainTicketWords;
        const unsigned int t =
            __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        // The last workgroup of this XCD re-arms the counter for the next launch.
        if (t + 1 == (unsigned int)per_xcd)
            __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_ticket = (int)t;
    }
    __syncthreads();
    const int ticket = __builtin_amdgcn_readfirstlane(s_ticket);
    if (ticket >= per_xcd) return;  // not reached when every XCD runs its share

    const ChainTicket& d = tickets[ticket];
    const unsigned int word = d.word;
    const int index = (int)((word >> 2) & (kChainMaxMats - 1));
    const int split = (int)(word >> 16);
    const int ng = d.ng0 + xcd;
    if (ng >= d.n_groups) return;  // padding of the column groups to 8
    const int K = d.K, N = d.N, splits = d.splits;
    const int nsb = (K + kSuperK - 1) / kSuperK;
    const int n_tiles = (N + kTileN - 1) / kTileN;
    const int sb0 = split * NCH;
    const int nch = min(NCH, nsb - sb0);
    const int k0 = sb0 * kSuperK;
    const int col = lane & 15, g = lane >> 4;
    const int nt = min(ng * WAVES + wave, n_tiles - 1);

    Chunk w[NCH];
    if (!stager) {
        // 1. Every weight chunk of this wave's column tile and K slice.
        const __amdgpu_buffer_rsrc_t rc =
            chain_rsrc(d.codes, (size_t)n_tiles * nsb * kCodeBytesPerSuper);
        const __amdgpu_buffer_rsrc_t rs =
            chain_rsrc(d.scales, (size_t)n_tiles * nsb * kScaleBytesPerSuper);
        const uint32_t sbw = (uint32_t)(nt * nsb + sb0);  // first (tile, superblock)
        const uint32_t coff = sbw * kCodeBytesPerSuper + lane * 16;
        const uint32_t soff = sbw * kScaleBytesPerSuper + (col * 2 + (g >> 1)) * 16;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const uint32_t cc = (uint32_t)min(c, nch - 1);  // a short slice re-reads its last chunk
#pragma unroll
            for (int i = 0; i < 4; ++i)
                w[c].c[i] = bload16<kNt>(rc, coff + i * 1024, cc * kCodeBytesPerSuper);
            w[c].s = bload16<kNt>(rs, soff, cc * kScaleBytesPerSuper);
        }
    } else {
        // 2. Wait until the previous matrix is complete (its flag reads >= index).
        if (index > 0 && lane == 0) {
            const unsigned int* slot = chain_flag(sync.flags, (ticket * 8 + xcd) % kChainFlagSlots);
            const unsigned int limit = sync.status[1];
            unsigned int it = 0;
            while (__hip_atomic_load(slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                   (unsigned int)index) {
                if (++it > limit) {
                    __hip_atomic_fetch_or(sync.status, 1u, __ATOMIC_RELAXED,
                                          __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
                __builtin_amdgcn_s_sleep(8);
            }
        }
        // 3. Rows 0..M-1 of the activation slice, straight into LDS: one
        //    64-lane copy per row and superblock, through a resource that ends
        //    at the row's end (values past K read as zero).  Activations an
        //    earlier matrix of the launch wrote are read device-coherently.
        //    Rows M..7 are never read (their lanes select the zero row 8).
        const bool coherent = (word & kChainActCoherent) != 0;
        for (int r = 0; r < M; ++r) {
            for (int c = 0; c < nch; ++c) {
                const int k = k0 + c * kSuperK;
                const __amdgpu_buffer_rsrc_t ra =
                    chain_rsrc(d.act + (size_t)r * K + k, (size_t)(K - k) * sizeof(uint16_t));
                __attribute__((address_space(3))) void* dst =
                    (__attribute__((address_space(3))) void*)(lds + r * kStride + c * kSuperK);
                if (coherent)
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, lane * 16, 0, 0, kSc1);
                else
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, dst, 16, lane * 16, 0, 0, 0);
            }
        }
        for (int i = lane; i < NCH * kSuperK / 8; i += 64)
            *(uint4*)(lds + 8 * kStride + 8 * i) = make_uint4(0, 0, 0, 0);
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    __syncthreads();  // activations in LDS

    // 4. MFMA over the slice (operand mapping of decode.hip).
    const bool bf16 = (word & kChainOutBf16) != 0;
    const __amdgpu_buffer_rsrc_t out =
        chain_rsrc(d.out, (size_t)M * N * (bf16 ? sizeof(uint16_t) : sizeof(float)));
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    if (!stager) {
        const int m = col & 7;
        const bool live = ((col >> 3) == (g >> 1)) && (m < M);
        const __bf16* ap = lds + (live ? m : 8) * kStride + 8 * g;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
            if (c < nch) chunk_steps(acc, w[c], ap + c * kSuperK);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], 32, 64);
    }
    const bool mine = !stager && lane < 32 && ng * WAVES + wave < n_tiles;

    // 5. Outputs, written with device-coherent stores (a later matrix of the
    //    launch may read them as activations from another XCD).
    if (splits == 1) {
        if (mine) {
            const int n = nt * kTileN + col;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int mm = 4 * g + j;
                if (mm < M && n < N) store_coherent(out, (uint32_t)(mm * N + n), acc[j] * d.ts, bf16);
            }
        }
    } else {
        unsigned int* counters = (unsigned int*)(sync.regions + (size_t)d.region * 256);
        float* partial = (float*)((char*)counters + chain_counter_bytes(d.n_groups));
        float* pbase = partial + (size_t)(ng * splits + split) * 8 * kCols;
        if (mine) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int mm = 4 * g + j;
                if (mm < M) pbase[mm * kCols + wave * kTileN + col] = acc[j];
            }
        }
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __syncthreads();
        if (threadIdx.x == 0) {
            const unsigned int old = __hip_atomic_fetch_add(&counters[ng], 1u, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
            s_last = (old == (unsigned int)(splits - 1));
        }
        __syncthreads();
        if (!s_last) return;
        // The last slice adds the partial sums in split order.
        constexpr int kR = (8 * kCols + kAll - 1) / kAll;
        const float* gbase = partial + (size_t)ng * splits * 8 * kCols;
        float sum[kR];
        sum_partials<kCols, kAll, kR, true>(gbase, splits, M * kCols, sum);
#pragma unroll
        for (int r = 0; r < kR; ++r) {
            const int idx = threadIdx.x + r * kAll;
            const int mm = idx / kCols, c = idx - mm * kCols;
            const int n = ng * kCols + c;
            if (idx < M * kCols && n < N) store_coherent(out, (uint32_t)(mm * N + n), sum[r] * d.ts, bf16);
        }
        if (threadIdx.x == 0)  // re-armed for the next launch
            __hip_atomic_store(&counters[ng], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }

    // 6. This column group is final: count it; the matrix's last group
    //    publishes completion (the last matrix clears the flags instead).
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    if (wave == 0) {
        unsigned int pub = 0;
        if (lane == 0) {
            const unsigned int old = __hip_atomic_fetch_add(&sync.done[index], 1u,
                                                            __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
            if (old + 1 == (unsigned int)d.n_groups) {
                pub = 1;
                __hip_atomic_store(&sync.done[index], 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        pub = __shfl(pub, 0, 64);
        if (pub) {
            const unsigned int v = index == n_mats - 1 ? 0u : (unsigned int)(index + 1);
            __hip_atomic_store(chain_flag(sync.flags, lane), v, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Counts, per XCD, the workgroups of a launch of `blocks` workgroups.
__global__ void chain_count_kernel(unsigned int* counts) {
    unsigned int xcc;
    asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(counts + (xcc & 7u) * kChainTicketWords, 1u, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
}

// ---- host ---------------------------------------------------------------------

static size_t al256(size_t x) { return (x + 255) / 256 * 256; }

struct ChainShape {
    int splits, n_groups, ng8;
    size_t region_bytes;
};

static ChainShape chain_shape(int K, int N) {
    ChainShape s;
    const int nsb = padded_k(K) / kSuperK;
    const int n_tiles = padded_n(N) / kTileN;
    s.splits = (nsb + kChainChunks - 1) / kChainChunks;
    s.n_groups = (n_tiles + kChainWaves - 1) / kChainWaves;
    s.ng8 = round_up(s.n_groups, 8);
    s.region_bytes = s.splits > 1 ? chain_counter_bytes(s.n_groups) +
                                        al256((size_t)s.ng8 * s.splits * 8 * kChainWaves *
                                              kTileN * sizeof(float))
                                  : 0;
    return s;
}

size_t chain_round_layout(const nvfp4_layer* L, int n, ChainLayout* out) {
    ChainLayout& y = *out;
    y.n = n;
    size_t per_xcd = 0, regions = 0;
    for (int i = 0; i < n; ++i) {
        const ChainShape s = chain_shape(L[i].K, L[i].N);
        per_xcd += (size_t)(s.ng8 / 8) * s.splits;
        regions += s.region_bytes;
    }
    y.per_xcd = per_xcd;
    y.status_off = 0;
    y.tickets_off = 256;
    y.done_off = y.tickets_off + 8 * kChainTicketWords * sizeof(unsigned int);
    y.flags_off = (y.done_off + al256((size_t)n * sizeof(unsigned int)) + 4095) / 4096 * 4096;
    y.desc_off = y.flags_off + (size_t)kChainFlagSlots * kChainFlagStride;  // ticket records
    y.regions_off = y.desc_off + al256(per_xcd * sizeof(ChainTicket));
    y.total = y.regions_off + regions;
    return y.total;
}

static bool ranges_overlap(const void* a, size_t an, const void* b, size_t bn) {
    const uintptr_t x = (uintptr_t)a, y = (uintptr_t)b;
    return x < y + bn && y < x + an;
}

int chain_round_write(const nvfp4_layer* L, int n, int max_M, void* ws, const ChainLayout& y) {
    if (n >= kChainMaxMats)
        return set_error(NVFP4_EUNSUPPORTED, "n_layers: %d matrices exceed the chained round's %d",
                         n, kChainMaxMats - 1);
    if (y.per_xcd > (size_t)0x7FFFFFFF / 8)
        return set_error(NVFP4_EUNSUPPORTED, "layers: %zu workgroups per XCD exceed one launch",
                         y.per_xcd);
    for (int i = 0; i < n; ++i) {
        if ((size_t)padded_n(L[i].N) * padded_k(L[i].K) / 2 > 0x7FFFFFFFu)
            return set_error(NVFP4_EUNSUPPORTED,
                             "layers[%d]: more than 2 GiB of packed codes (chained round)", i);
        if (chain_shape(L[i].K, L[i].N).splits > 0xFFFF)
            return set_error(NVFP4_EUNSUPPORTED, "layers[%d].K: %d too long for the chained round",
                             i, L[i].K);
    }
    ChainTicket* tk = new (std::nothrow) ChainTicket[y.per_xcd ? y.per_xcd : 1];
    if (!tk) return set_error(NVFP4_EINVAL, "plan: out of host memory");
    size_t ticket = 0, region = 0;
    for (int i = 0; i < n; ++i) {
        const nvfp4_layer& l = L[i];
        const ChainShape s = chain_shape(l.K, l.N);
        // Activations written by an earlier matrix of the round are read with
        // device-coherent loads.
        bool coherent = false;
        const size_t in_bytes = (size_t)max_M * l.K * sizeof(uint16_t);
        for (int j = 0; j < i && !coherent; ++j) {
            const size_t esz = L[j].out_dtype == NVFP4_OUT_BF16 ? 2 : 4;
            coherent = ranges_overlap(l.act_dev, in_bytes, L[j].out_dev, (size_t)max_M * L[j].N * esz);
        }
        const unsigned int base = (l.out_dtype == NVFP4_OUT_BF16 ? kChainOutBf16 : 0u) |
                                  (coherent ? kChainActCoherent : 0u) | ((unsigned int)i << 2);
        const int nt = s.ng8 / 8 * s.splits;
        for (int q = 0; q < nt; ++q) {
            ChainTicket& d = tk[ticket + q];
            d.codes = (const uint4*)l.codes_dev;
            d.scales = (const uint4*)l.scales_dev;
            d.act = l.act_dev;
            d.out = l.out_dev;
            d.ts = l.tensor_scale;
            d.K = l.K;
            d.N = l.N;
            d.splits = s.splits;
            d.n_groups = s.n_groups;
            d.ng0 = q / s.splits * 8;
            d.region = (unsigned int)(region / 256);
            d.word = base | (unsigned int)(q % s.splits) << 16;
        }
        ticket += nt;
        region += s.region_bytes;
    }
    int st = NVFP4_OK;
    hipError_t e = hipMemcpy((char*)ws + y.desc_off, tk, y.per_xcd * sizeof(ChainTicket),
                             hipMemcpyHostToDevice);
    if (e != hipSuccess) st = hip_fail(e, "hipMemcpy(chain tickets)");
    delete[] tk;
    return st;
}

// Launches a grid of 8 * per_xcd one-wave workgroups and checks that each XCD
// ran exactly per_xcd of them (the chain's forward-progress argument needs
// it).  Uses and re-zeroes the ticket counters.  Synchronous.
int chain_check_dispatch(void* ws, const ChainLayout& y) {
    unsigned int* counts = (unsigned int*)((char*)ws + y.tickets_off);
    hipLaunchKernelGGL(chain_count_kernel, dim3((unsigned int)(8 * y.per_xcd)), dim3(64), 0, 0,
                       counts);
    NVFP4_HIP(hipGetLastError());
    unsigned int h[8 * kChainTicketWords];
    NVFP4_HIP(hipMemcpy(h, counts, sizeof(h), hipMemcpyDeviceToHost));
    NVFP4_HIP(hipMemset(counts, 0, sizeof(h)));
    NVFP4_HIP(hipDeviceSynchronize());
    for (int x = 0; x < 8; ++x)
        if (h[x * kChainTicketWords] != (unsigned int)y.per_xcd)
            return set_error(NVFP4_EUNSUPPORTED,
                             "mode: the chained round needs workgroups spread evenly over 8 XCDs "
                             "(XCD %d ran %u of %zu)", x, h[x * kChainTicketWords], y.per_xcd);
    return NVFP4_OK;
}

int chain_launch_round(int M, void* ws, const ChainLayout& y, hipStream_t s) {
    char* b = (char*)ws;
    ChainSync sync{(unsigned int*)(b + y.status_off), (unsigned int*)(b + y.tickets_off),
                   (unsigned int*)(b + y.done_off), (unsigned int*)(b + y.flags_off),
                   b + y.regions_off};
    hipLaunchKernelGGL((chain_kernel<kChainWaves, kChainChunks>),
                       dim3((unsigned int)(8 * y.per_xcd)), dim3((kChainWaves + 1) * 64), 0, s,
                       (const ChainTicket*)(b + y.desc_off), sync, y.n, (int)y.per_xcd, M);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

}  // namespace nvfp4
