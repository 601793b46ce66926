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
#include "decode_device.h"

namespace nvfp4 {

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
    int n_groups, int n_tiles, int l2_local) {
    constexpr int kThreads = WAVES * 64;
    constexpr int kStride = NCH * kSuperK + kLdsPad;          // LDS row, bf16 elements
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
            const int mm = 4 * g + j;
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
        const unsigned int old =
            __hip_atomic_fetch_add(&counters[ng], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        s_last = (old == (unsigned int)(splits - 1));
    }
    __syncthreads();
    if (!s_last) return;
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
        const int n = ng * kCols + c;
        if (idx < M * kCols && n < N) store_out<BF16>(out, (size_t)mm * N + n, sum[r] * ts);
    }
    if (threadIdx.x == 0)  // leave the counter zeroed for the next run
        __hip_atomic_store(&counters[ng], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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

static int xcd_mapping_verified() {
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
    // N = 5120..152064): 2 superblocks per slice and 4 waves per workgroup,
    // except very long K (>= 16384), where 3 superblocks and 8 waves win.
    const bool long_k = nsb >= 32;
    int waves = (cfg && cfg->waves) ? cfg->waves : (long_k ? 8 : 4);
    if (waves != 4 && waves != 8)
        return set_error(NVFP4_EINVAL, "config.waves: %d is not 4 or 8", waves);
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
        chunks = long_k ? 3 : 2;
        if (chunks > nsb) chunks = nsb;
    }
    const int splits = (nsb + chunks - 1) / chunks;
    d->l2_local = splits > 1 ? xcd_mapping_verified() : 0;
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
                       M, p->K, p->N, p->Kp / kSuperK, d.splits, d.n_groups, p->Np / kTileN,
                       d.l2_local);
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
