// Streaming decode GEMM: the weight stream of a wave never stops.
//
// "Ignis" README, "The decode round": one pass over the NVFP4 weights serves
// every lane and the round runs at the card's memory bandwidth; its decode
// kernels are chained ("Credits": a programmatic-dependent-launch decode
// chain) so one GEMM's start overlaps the previous one's drain.
//
// Work decomposition (gfx950).  A workgroup has 8 compute waves and 2 stager
// waves.  It owns a column group of T column tiles (16 outputs each, one MFMA
// column block) for the whole of K: compute wave w works on tile w % T and on
// the K superblocks (512 values) congruent to w / T modulo P = 8 / T.  The P
// partial sums of a tile are added in LDS at the end in a fixed order, so
// there is no cross-workgroup reduction: no partial-sum traffic, no counters,
// no atomics on the data path.  T is chosen per matrix (small N: T = 2 so
// enough workgroups stream; large N: T = 8 so the activation staging is
// shared by more tiles).
//
// Compute waves issue nothing but weight loads.  Each keeps a ring of D
// superblocks in registers and refills one slot per step, D steps ahead; the
// look-ahead runs on into the workgroup's next task -- and, in the persistent
// round, into the next matrix.  Because a wave's loads complete in issue
// order, any other load on a compute wave would force the whole ring to land
// first; so the two stager waves load the activations, write the results
// and, in the persistent round, wait for the previous matrix and signal
// completion.  Under a saturated weight stream even cached loads take
// microseconds, so the activations of a whole K window (all of K up to 8704)
// are staged into LDS at once per task: the compute waves then run through
// their steps without synchronising until the window ends.
#include <new>

#include "decode_device.h"

namespace nvfp4 {

constexpr int kSCompute = 8;                          // compute waves
constexpr int kSStagers = 2;                          // stager waves
constexpr int kSThreads = (kSCompute + kSStagers) * 64;
constexpr int kSPmax = 4;                             // at most 4 K parts (T >= 2)
// Activations live in LDS for a whole window of K: 17 superblocks (8704
// values) x 9 rows (8 lanes and the zero row) of bf16, 154 KB -- one window
// covers every K up to 8704; longer K (17408) takes two windows.
constexpr int kSWinSb = 17;
constexpr int kSStride = kSWinSb * kSuperK + kLdsPad;  // LDS activation row (bf16)

struct alignas(16) StreamDesc {
    const uint4* codes;
    const uint4* scales;
    const uint16_t* act;
    void* out;
    float ts;
    int K, N, nsb;
    int n_tiles;
    int T;        // column tiles per workgroup (2, 4 or 8)
    int lgT;      // log2(T)
    int n_tasks;  // column groups: ceil(n_tiles / T)
    int steps;    // ceil(nsb / P), P = 8 / T
    int out_bf16;
    int rot;      // persistent round: task rotation over the grid
    int pad;
};

// Position of a workgroup in its stream of (matrix, task, step).
struct Cursor {
    int i;     // matrix (n_mats when past the end)
    int task;  // column group within the matrix
    int step;  // K step within the task
};

// Workgroup wg of G takes the tasks congruent to (wg + rot) modulo G.
__device__ __forceinline__ int first_task_of(int wg, int G, int rot) {
    return (wg + G - rot % G) % G;
}

template <class Descs>
__device__ __forceinline__ void cursor_seek(const Descs& D, int n_mats, int G, Cursor& c) {
    // From (c.i, c.task): first matrix >= c.i where c.task is a valid task.
    while (c.i < n_mats && c.task >= D(c.i).n_tasks) {
        ++c.i;
        if (c.i < n_mats) c.task = first_task_of((int)blockIdx.x, G, D(c.i).rot);
    }
}

template <class Descs>
__device__ __forceinline__ void cursor_first(const Descs& D, int n_mats, int G, Cursor& c) {
    c.i = 0;
    c.step = 0;
    c.task = first_task_of((int)blockIdx.x, G, D(0).rot);
    cursor_seek(D, n_mats, G, c);
}

template <class Descs>
__device__ __forceinline__ void cursor_advance(const Descs& D, int n_mats, int G, Cursor& c) {
    if (c.i >= n_mats) return;
    if (++c.step < D(c.i).steps) return;
    c.step = 0;
    c.task += G;
    cursor_seek(D, n_mats, G, c);
}

// Weight chunk of compute wave `wave` at cursor c.  Past the end, or for a
// part or tile out of range, a valid chunk is re-read instead (the caches
// serve it): every step issues the same number of loads, so the in-order
// completion count stays exact.
template <class Descs>
__device__ __forceinline__ void load_at(const Descs& D, int n_mats, const Cursor& c, int wave,
                                        int lane, Chunk& w) {
    const bool ok = c.i < n_mats;
    const StreamDesc& d = D(ok ? c.i : 0);
    const int task = ok ? c.task : 0, step = ok ? c.step : 0;
    const int t = wave & (d.T - 1), p = wave >> d.lgT;
    const int P = kSCompute >> d.lgT;
    const int nt = min(task * d.T + t, d.n_tiles - 1);
    const int sb = min(step * P + p, d.nsb - 1);
    const int col = lane & 15, g = lane >> 4;
    load_chunk(w, d.codes + ((size_t)nt * d.nsb + sb) * 256 + lane,
               d.scales + ((size_t)nt * d.nsb + sb) * 32 + col * 2 + (g >> 1));
}

// Stager waves: rows 0..M-1 of the activations of K range
// [k0, k0 + nsb_w*512) into LDS, with direct-to-LDS loads (no registers hold
// the data).  One load instruction fills 64 consecutive 16-byte vectors of one
// row, so row r, superblock j of the window is one instruction; the two stager
// waves take alternate instructions.  Rows >= M are never read (those MFMA rows read the
// zero row); K beyond the matrix (the padding of the last superblock) reads a
// clamped in-range address, harmless since the padding weights are zero.
__device__ __forceinline__ void stage_act(__bf16* buf, const uint16_t* act, int M, int K, int k0,
                                          int nsb_w, int swave, int lane) {
    for (int j = swave; j < M * nsb_w; j += kSStagers) {
        const int r = j / nsb_w, seg = j - r * nsb_w;
        const int k = min(k0 + 8 * (seg * 64 + lane), K - 8);
        __builtin_amdgcn_global_load_lds((const void*)(act + (size_t)r * K + k),
                                         (__attribute__((address_space(3))) void*)(
                                             buf + r * kSStride + seg * kSuperK),
                                         16, 0, 0);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <bool BF16>
__device__ __forceinline__ void store_result(void* out, size_t idx, float v, bool coherent) {
    if (coherent) {
        if (BF16)
            __hip_atomic_store((uint16_t*)out + idx, f32_to_bf16_rne(v), __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        else
            __hip_atomic_store((float*)out + idx, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        store_out<BF16>(out, idx, v);
    }
}

// Cross-matrix completion flags of the persistent round: completion of
// matrix i is published as the value i + 1 in kSFlagSlots words kSFlagStride
// bytes apart (different memory channels); each workgroup polls one slot, so
// the polling does not pile onto one address.
constexpr int kSFlagSlots = 64;
constexpr int kSFlagStride = 4096;

struct RoundSync {
    unsigned int* done;    // [n_mats] finished tasks per matrix
    unsigned int* status;  // [0] error flags, [1] spin limit
    unsigned int* flags;   // kSFlagSlots words, kSFlagStride apart
};

__device__ __forceinline__ unsigned int* sflag(unsigned int* flags, int slot) {
    return (unsigned int*)((char*)flags + (size_t)slot * kSFlagStride);
}

// The core.  Descs(i) returns matrix i's descriptor.  PERSISTENT: before the
// activations of matrix i are staged, matrix i-1 must be final; results are
// written with device-coherent stores; finished tasks are counted and a
// completed matrix is published.
template <int D, bool PERSISTENT, class Descs>
__device__ __forceinline__ void stream_tasks(const Descs& Ds, int n_mats, int M, RoundSync sync) {
    __shared__ __attribute__((aligned(16))) __bf16 lds[9 * kSStride];
    __shared__ float red[kSCompute][32][4];

    const int G = gridDim.x;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const bool stager = wave >= kSCompute;
    const int swave = wave - kSCompute;  // stager wave 0..1
    const int col = lane & 15, g = lane >> 4;

    // Zero row (row 8): written once, never overwritten.
    for (int idx = threadIdx.x; idx < kSStride / 8; idx += kSThreads)
        *(uint4*)(lds + 8 * kSStride + 8 * idx) = make_uint4(0, 0, 0, 0);

    Cursor cc;  // compute position (uniform over the workgroup)
    cursor_first(Ds, n_mats, G, cc);
    if (cc.i >= n_mats) return;
    Cursor pc = cc;  // compute waves' prefetch position, D steps ahead

    Chunk ring[D];
    if (!stager) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
            load_at(Ds, n_mats, pc, wave, lane, ring[q]);
            cursor_advance(Ds, n_mats, G, pc);
        }
    }
    unsigned int* my_flag =
        PERSISTENT ? sflag(sync.flags, (blockIdx.x * kSStagers + (wave - kSCompute)) % kSFlagSlots)
                   : nullptr;
    const unsigned int spin_limit = PERSISTENT ? sync.status[1] : 0u;
    int waited = 0;
    float acc[4] = {0.f, 0.f, 0.f, 0.f};

    while (cc.i < n_mats) {
#pragma unroll
        for (int q = 0; q < D; ++q) {
            if (cc.i < n_mats) {
                const StreamDesc& d = Ds(cc.i);
                const int P = kSCompute >> d.lgT;
                // Superblocks of K per window: whole steps, at most kSWinSb.
                const int win_steps = kSWinSb / P;
                const int w0 = cc.step - cc.step % win_steps;  // first step of this window
                if (cc.step == w0) {
                    // Window start (and, at step 0, task start): stage the
                    // activations of the window's K range.
                    if (cc.step == 0 && PERSISTENT && cc.i > waited) {
                        if (stager && lane == 0) {
                            unsigned int it = 0;
                            while (__hip_atomic_load(my_flag, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) < (unsigned int)cc.i) {
                                if (++it > spin_limit) {
                                    __hip_atomic_fetch_or(sync.status, 1u, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                                    break;
                                }
                                __builtin_amdgcn_s_sleep(8);
                            }
                        }
                        waited = cc.i;
                    }
                    if (cc.step != 0) __syncthreads();  // previous window fully read
                    if (stager) {
                        const int sb0 = w0 * P;
                        const int nsb_w = min(win_steps * P, d.nsb - sb0);
                        stage_act(lds, d.act, M, d.K, sb0 * kSuperK, nsb_w, swave, lane);
                    }
                    if (cc.step == 0) acc[0] = acc[1] = acc[2] = acc[3] = 0.f;
                    __syncthreads();
                }
                if (!stager) {
                    const int t = wave & (d.T - 1), p = wave >> d.lgT;
                    const bool live = ((col >> 3) == (g >> 1)) && ((col & 7) < M);
                    const int arow = live ? (col & 7) : 8;
                    if (cc.task * d.T + t < d.n_tiles && cc.step * P + p < d.nsb)
                        chunk_steps(acc, ring[q],
                                    lds + arow * kSStride + ((cc.step - w0) * P + p) * kSuperK +
                                        8 * g);
                    load_at(Ds, n_mats, pc, wave, lane, ring[q]);
                    cursor_advance(Ds, n_mats, G, pc);
                }
                if (cc.step == d.steps - 1) {
                    // Task end: the parts of each tile meet in LDS; stager wave 0
                    // adds them in order and writes the results.
                    if (!stager) {
#pragma unroll
                        for (int j = 0; j < 4; ++j) acc[j] += __shfl_xor(acc[j], 32, 64);
                        if (lane < 32) {
#pragma unroll
                            for (int j = 0; j < 4; ++j) red[wave][lane][j] = acc[j];
                        }
                    }
                    __syncthreads();
                    if (wave == kSCompute) {
                        for (int o = lane; o < d.T * 128; o += 64) {
                            const int t = o >> 7, l = (o >> 2) & 31, j = o & 3;
                            const int tile = cc.task * d.T + t;
                            const int n = tile * kTileN + (l & 15), mm = 4 * (l >> 4) + j;
                            if (tile < d.n_tiles && mm < M && n < d.N) {
                                float v = red[t][l][j];
                                for (int pp = 1; pp < P; ++pp) v += red[pp * d.T + t][l][j];
                                if (d.out_bf16)
                                    store_result<true>(d.out, (size_t)mm * d.N + n, v * d.ts,
                                                       PERSISTENT);
                                else
                                    store_result<false>(d.out, (size_t)mm * d.N + n, v * d.ts,
                                                        PERSISTENT);
                            }
                        }
                        if (PERSISTENT) {
                            // Results complete before the task counts as done.
                            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
                            unsigned int pub = 0;
                            if (lane == 0) {
                                const unsigned int old = __hip_atomic_fetch_add(
                                    &sync.done[cc.i], 1u, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
                                if (old + 1 == (unsigned int)d.n_tasks) {
                                    pub = 1;
                                    // Matrix complete: nobody reads its predecessor's
                                    // counter any more; the last matrix resets its own.
                                    if (cc.i > 0)
                                        __hip_atomic_store(&sync.done[cc.i - 1], 0u,
                                                           __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                                    if (cc.i == n_mats - 1)
                                        __hip_atomic_store(&sync.done[cc.i], 0u, __ATOMIC_RELAXED,
                                                           __HIP_MEMORY_SCOPE_AGENT);
                                }
                            }
                            pub = __shfl(pub, 0, 64);
                            if (pub) {
                                const unsigned int v =
                                    cc.i == n_mats - 1 ? 0u : (unsigned int)(cc.i + 1);
                                __hip_atomic_store(sflag(sync.flags, lane), v, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
                            }
                        }
                    }
                    // LDS (activations, red[]) is next written after the next
                    // task start's barrier, which every wave reaches only after
                    // this point.
                    __syncthreads();
                }
                cursor_advance(Ds, n_mats, G, cc);
            }
        }
    }
}

struct OneDesc {
    const StreamDesc& d;
    __device__ __forceinline__ const StreamDesc& operator()(int) const { return d; }
};

struct DescArray {
    const StreamDesc* p;
    __device__ __forceinline__ const StreamDesc& operator()(int i) const { return p[i]; }
};

template <int D>
__global__ __launch_bounds__(kSThreads) void stream_gemm_kernel(StreamDesc d, int M) {
    stream_tasks<D, false>(OneDesc{d}, 1, M, RoundSync{nullptr, nullptr, nullptr});
}

template <int D>
__global__ __launch_bounds__(kSThreads) void stream_round_kernel(const StreamDesc* __restrict__ descs,
                                                                 int n_mats, int M, RoundSync sync) {
    stream_tasks<D, true>(DescArray{descs}, n_mats, M, sync);
}

// ---- host side ----------------------------------------------------------------

constexpr int kStreamDepth = 3;

// Column tiles per workgroup: the widest (most sharing of the activation
// staging) that still leaves at least 128 workgroups streaming; at most 4 K
// parts (T >= 2).
static int choose_T(int n_tiles) {
    for (int T = 8; T >= 2; T >>= 1)
        if ((n_tiles + T - 1) / T >= 128) return T;
    return 2;
}

void stream_fill_desc(StreamDesc* d, int K, int N, const void* codes, const void* scales,
                      const uint16_t* act, void* out, float ts, int out_dtype, int T_override) {
    const int n_tiles = padded_n(N) / kTileN;
    d->codes = (const uint4*)codes;
    d->scales = (const uint4*)scales;
    d->act = act;
    d->out = out;
    d->ts = ts;
    d->K = K;
    d->N = N;
    d->nsb = padded_k(K) / kSuperK;
    d->n_tiles = n_tiles;
    d->T = T_override ? T_override : choose_T(n_tiles);
    d->lgT = d->T == 8 ? 3 : d->T == 4 ? 2 : 1;
    d->n_tasks = (n_tiles + d->T - 1) / d->T;
    const int P = kSCompute / d->T;
    d->steps = (d->nsb + P - 1) / P;
    d->out_bf16 = out_dtype == NVFP4_OUT_BF16;
    d->rot = 0;
    d->pad = 0;
}

int stream_launch_gemm(const nvfp4_gemm_plan* p, int M, const uint8_t* codes,
                       const uint8_t* scales, float ts, const uint16_t* act, void* out,
                       hipStream_t s) {
    StreamDesc d;
    stream_fill_desc(&d, p->K, p->N, codes, scales, act, out, ts, p->out_dtype, p->str.tiles);
    hipLaunchKernelGGL((stream_gemm_kernel<kStreamDepth>), dim3(d.n_tasks), dim3(kSThreads), 0, s,
                       d, M);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

int stream_round_grid(int* grid) {
    int dev = 0, cus = 0, per = 0;
    NVFP4_HIP(hipGetDevice(&dev));
    NVFP4_HIP(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev));
    NVFP4_HIP(hipOccupancyMaxActiveBlocksPerMultiprocessor(
        &per, (const void*)stream_round_kernel<kStreamDepth>, kSThreads, 0));
    if (per < 1) return set_error(NVFP4_EUNSUPPORTED, "round kernel: no resident workgroup fits");
    *grid = cus * per;
    return NVFP4_OK;
}

size_t stream_round_layout(int n, StreamRoundLayout* out) {
    auto al = [](size_t b) { return (b + 255) / 256 * 256; };
    out->done_off = 0;
    out->status_off = al((size_t)n * sizeof(unsigned int));
    out->desc_off = out->status_off + 256;  // status[0] flags, status[1] spin limit
    out->flags_off = out->desc_off + al((size_t)n * sizeof(StreamDesc));
    out->total = out->flags_off + (size_t)kSFlagSlots * kSFlagStride;
    return out->total;
}

int stream_round_write_descs(const nvfp4_layer* L, int n, int grid, void* ws,
                             const StreamRoundLayout& lay, hipStream_t s) {
    StreamDesc* h = new (std::nothrow) StreamDesc[n];
    if (!h) return set_error(NVFP4_EINVAL, "layers: out of host memory for descriptors");
    long long rot = 0;
    for (int i = 0; i < n; ++i) {
        stream_fill_desc(&h[i], L[i].K, L[i].N, L[i].codes_dev, L[i].scales_dev, L[i].act_dev,
                         L[i].out_dev, L[i].tensor_scale, L[i].out_dtype, 0);
        // Rotate each matrix's task-to-workgroup map so the workgroups left
        // without work by one matrix lead the next (and prefetch for it).
        h[i].rot = (int)(rot % grid);
        rot += h[i].n_tasks;
    }
    hipError_t e = hipMemcpyAsync((char*)ws + lay.desc_off, h, (size_t)n * sizeof(StreamDesc),
                                  hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    delete[] h;
    if (e != hipSuccess) return hip_fail(e, "hipMemcpyAsync(round descriptors)");
    return NVFP4_OK;
}

int stream_launch_round(int n, int M, int grid, void* ws, const StreamRoundLayout& lay,
                        hipStream_t s) {
    char* b = (char*)ws;
    RoundSync sync{(unsigned int*)(b + lay.done_off), (unsigned int*)(b + lay.status_off),
                   (unsigned int*)(b + lay.flags_off)};
    hipLaunchKernelGGL((stream_round_kernel<kStreamDepth>), dim3(grid), dim3(kSThreads), 0, s,
                       (const StreamDesc*)(b + lay.desc_off), n, M, sync);
    NVFP4_HIP(hipGetLastError());
    return NVFP4_OK;
}

}  // namespace nvfp4
