// Top-k over the vocabulary: the step right after the output head.
//
// "Ignis" README, "Speculative decoding (DFlash2)": the drafter's vendored
// top-k gave one small thread group to each of seven rows of a 248k-entry
// vocabulary and was the bottleneck; its row-split replacement returns the
// same answer.  Here every row is split over many workgroups, and the answer
// is unique by construction: the k largest logits in descending order,
// equal values by ascending index, -0.0 equal to +0.0.
//
// Keys.  A logit v at index i becomes the 64-bit key (ord(v) << 32) | ~i,
// where ord maps float bits to an unsigned order (negative values
// complemented, non-negative ones with the sign bit set; -0 first becomes
// +0).  A larger key means a larger value, or an equal value at a smaller
// index, so keys are distinct and their descending order is the answer.  The
// smallest key of a finite or infinite logit is ord(-inf) << 32 > 0, so key
// 0 marks "no element".  NaN logits are out of contract.
//
// Levels.  A wave takes a unit of 1024 keys of a row (16 per lane, sorted in
// registers by a bitonic network), then k rounds: the wave's largest head
// key (a DPP butterfly within rows of 16 lanes, then the four rows' lanes
// read as scalars: no LDS, no barrier) is the next output, and the lane that
// held it shifts its list.  Level 0 reads the logits and writes k candidate
// keys per unit; while a row has more than one unit of candidates, the next
// level does the same over them.  The last level writes the indices and
// re-reads the values from the logits (bit for bit).  For k <= 8 and at most
// 256 units, one wave per row merges level 0's sorted runs instead of
// further levels (topk_merge_kernel).
#include "common.h"

namespace nvfp4 {

constexpr int kTopkThreads = 256;  // 4 waves, one unit each
constexpr int kTopkPer = 16;
constexpr int kTopkUnit = 64 * kTopkPer;  // 1024 keys per wave

typedef unsigned long long u64;

__device__ __forceinline__ u64 topk_key(float v, int i) {
    unsigned int b = __float_as_uint(v);
    if (b == 0x80000000u) b = 0u;  // -0 -> +0
    const unsigned int o = (b & 0x80000000u) ? ~b : (b | 0x80000000u);
    return ((u64)o << 32) | (unsigned int)(~i);
}

__device__ __forceinline__ u64 max64(u64 a, u64 b) { return a > b ? a : b; }

// Descending compare-exchange.
__device__ __forceinline__ void cex(u64& a, u64& b) {
    const u64 hi = max64(a, b), lo = a > b ? b : a;
    a = hi;
    b = lo;
}

// Bitonic sorting network over 16 registers, descending.
__device__ __forceinline__ void sort16(u64 (&x)[kTopkPer]) {
#pragma unroll
    for (int size = 2; size <= kTopkPer; size <<= 1)
#pragma unroll
        for (int stride = size >> 1; stride > 0; stride >>= 1)
#pragma unroll
            for (int i = 0; i < kTopkPer; ++i) {
                const int j = i ^ stride;
                if (j > i) {
                    // descending within blocks whose bit `size` is clear
                    if ((i & size) == 0)
                        cex(x[i], x[j]);
                    else
                        cex(x[j], x[i]);
                }
            }
}

// v from the lane that DPP control `ctrl` selects (both halves).
template <int CTRL>
__device__ __forceinline__ u64 dpp64(u64 v) {
    const int lo = __builtin_amdgcn_update_dpp((int)v, (int)v, CTRL, 0xF, 0xF, false);
    const int hi = __builtin_amdgcn_update_dpp((int)(v >> 32), (int)(v >> 32), CTRL, 0xF, 0xF,
                                               false);
    return ((u64)(unsigned int)hi << 32) | (unsigned int)lo;
}

__device__ __forceinline__ u64 lane64(u64 v, int lane) {
    const unsigned int lo = __builtin_amdgcn_readlane((int)v, lane);
    const unsigned int hi = __builtin_amdgcn_readlane((int)(v >> 32), lane);
    return ((u64)hi << 32) | lo;
}

// The wave's largest key, uniform.  Within each row of 16 lanes: swap lane
// pairs, then quad halves (quad_perm [1,0,3,2] and [2,3,0,1]), then the
// mirrors of each 8 and of the 16; every lane of a row then holds the row's
// maximum.  The four rows' maxima are read from lanes 0, 16, 32 and 48.
__device__ __forceinline__ u64 wave_max64(u64 v) {
    v = max64(v, dpp64<0xB1>(v));   // quad_perm [1,0,3,2]
    v = max64(v, dpp64<0x4E>(v));   // quad_perm [2,3,0,1]
    v = max64(v, dpp64<0x141>(v));  // row_half_mirror
    v = max64(v, dpp64<0x140>(v));  // row_mirror
    return max64(max64(lane64(v, 0), lane64(v, 16)), max64(lane64(v, 32), lane64(v, 48)));
}

// One level.  Row m's input: logits (LOGITS, n = V elements, stride ld) or
// keys (n = candidates per row, stride n).  Unit u of the row (wave
// blockIdx.x * 4 + wave): elements 1024 u .. 1024 u + 1023.  FINAL: one unit
// per row; writes idx/val [M][k].  Otherwise writes k keys per unit to
// out_keys [M][units][k].
template <bool LOGITS, bool FINAL>
__global__ __launch_bounds__(kTopkThreads) void topk_level_kernel(
    const float* __restrict__ logits, int ld, const u64* __restrict__ in_keys, int n, int k,
    int units, u64* __restrict__ out_keys, int* __restrict__ idx_out,
    float* __restrict__ val_out) {
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6));
    const int lane = threadIdx.x & 63;
    const int u = blockIdx.x * (kTopkThreads / 64) + wave, m = blockIdx.y;
    if (u >= units) return;  // whole wave
    // All 16 loads at once: clamped addresses, elements past n masked after.
    u64 x[kTopkPer];
    float v[kTopkPer];
#pragma unroll
    for (int j = 0; j < kTopkPer; ++j) {
        const int e = min(u * kTopkUnit + j * 64 + lane, n - 1);
        if (LOGITS)
            v[j] = logits[(size_t)m * ld + e];
        else
            x[j] = in_keys[(size_t)m * n + e];
    }
#pragma unroll
    for (int j = 0; j < kTopkPer; ++j) {
        const int e = u * kTopkUnit + j * 64 + lane;
        if (LOGITS) x[j] = topk_key(v[j], e);
        x[j] = e < n ? x[j] : 0;
    }
    if (k > 1) sort16(x);
    // Round r's key is kept by lane r; all stores (and the final value
    // gathers) go out together after the rounds.
    u64 kept = 0;
    if (k == 1) {
        u64 head = x[0];
#pragma unroll
        for (int j = 1; j < kTopkPer; ++j) head = max64(head, x[j]);
        kept = wave_max64(head);
    } else {
        // Each lane's list stays in place; `taken` counts its keys already
        // output, and its head is x[taken] (0 once all 16 are out), picked by
        // a select chain (linear in 16, and no register-array indexing).
        int taken = 0;
        for (int r = 0; r < k; ++r) {
            u64 head = 0;
#pragma unroll
            for (int j = 0; j < kTopkPer; ++j) head = taken == j ? x[j] : head;
            const u64 top = wave_max64(head);
            kept = lane == r ? top : kept;
            // the holder of `top` (keys are distinct: one lane) moves on
            taken += head == top ? 1 : 0;
        }
    }
    if (lane < k) {
        if (FINAL) {
            // kept is 0 only past the row's elements, and V >= k
            const int i = (int)~(unsigned int)(kept & 0xFFFFFFFFu);
            idx_out[(size_t)m * k + lane] = i;
            val_out[(size_t)m * k + lane] = logits[(size_t)m * ld + i];
        } else {
            out_keys[((size_t)m * units + u) * k + lane] = kept;
        }
    }
}

// The levels after the first, for k <= 8 and at most 256 units: a row's
// candidates are then u0 runs of k keys, each already sorted descending (lane
// r of a unit keeps its round-r key), and one wave per row merges them into
// the answer in k rounds, with no sort: lane l owns runs l, l + 64, l + 128
// and l + 192, its head is the largest current key of its runs, and each
// round outputs the wave's largest head and advances the run that held it.
// One launch instead of one or two further levels, each of which sorted its
// units again.
constexpr int kMergeRuns = 4;  // runs per lane
constexpr int kMergeMaxK = 8;
__global__ __launch_bounds__(64) void topk_merge_kernel(const float* __restrict__ logits, int ld,
                                                        const u64* __restrict__ in_keys,
                                                        int units, int k,
                                                        int* __restrict__ idx_out,
                                                        float* __restrict__ val_out) {
    const int lane = threadIdx.x, m = blockIdx.x;
    // All loads at once: clamped addresses, runs past `units` and keys past
    // k masked after.
    u64 x[kMergeRuns][kMergeMaxK];
#pragma unroll
    for (int r = 0; r < kMergeRuns; ++r)
#pragma unroll
        for (int j = 0; j < kMergeMaxK; ++j) {
            const int run = min(lane + 64 * r, units - 1), jj = min(j, k - 1);
            x[r][j] = in_keys[((size_t)m * units + run) * k + jj];
        }
#pragma unroll
    for (int r = 0; r < kMergeRuns; ++r)
#pragma unroll
        for (int j = 0; j < kMergeMaxK; ++j)
            x[r][j] = (lane + 64 * r < units && j < k) ? x[r][j] : 0;
    int taken[kMergeRuns] = {0, 0, 0, 0};
    u64 kept = 0;
    for (int t = 0; t < k; ++t) {
        u64 h[kMergeRuns];
#pragma unroll
        for (int r = 0; r < kMergeRuns; ++r) {
            u64 v = 0;  // 0 once the run is exhausted
#pragma unroll
            for (int j = 0; j < kMergeMaxK; ++j) v = taken[r] == j ? x[r][j] : v;
            h[r] = v;
        }
        const u64 top = wave_max64(max64(max64(h[0], h[1]), max64(h[2], h[3])));
        kept = lane == t ? top : kept;
        // keys are distinct: exactly one run of one lane held `top`
#pragma unroll
        for (int r = 0; r < kMergeRuns; ++r) taken[r] += h[r] == top ? 1 : 0;
    }
    if (lane < k) {
        // the row has at least k elements, so kept is a real key
        const int i = (int)~(unsigned int)(kept & 0xFFFFFFFFu);
        idx_out[(size_t)m * k + lane] = i;
        val_out[(size_t)m * k + lane] = logits[(size_t)m * ld + i];
    }
}

int topk_levels(int V, int k, int* units0) {
    int n = V, levels = 0, u0 = 0;
    do {
        const int u = (n + kTopkUnit - 1) / kTopkUnit;
        if (levels == 0) u0 = u;
        ++levels;
        if (u == 1) break;
        n = u * k;
    } while (true);
    *units0 = u0;
    return levels;
}

}  // namespace nvfp4

using namespace nvfp4;

extern "C" {

size_t nvfp4_topk_workspace_bytes(int M, int V, int k) {
    if (M < 1 || V < 1 || k < 1 || k > NVFP4_TOPK_MAX_K || k > V) return 0;
    int u0 = 0;
    topk_levels(V, k, &u0);
    // two candidate buffers: level l writes one, level l + 1 reads it
    const size_t one = (size_t)M * u0 * k * sizeof(u64);
    return u0 > 1 ? 2 * ((one + 255) / 256 * 256) : 0;
}

int nvfp4_topk(const float* logits_dev, int M, int V, int ld, int k, int* idx_dev,
               float* val_dev, void* workspace_dev, size_t workspace_bytes, void* stream) {
    clear_error();
    if (M < 1 || M > 65535) return set_error(NVFP4_EINVAL, "M: %d outside [1, 65535]", M);
    if (V < 1) return set_error(NVFP4_EINVAL, "V: %d < 1", V);
    if (ld < V) return set_error(NVFP4_EINVAL, "ld: %d < V = %d", ld, V);
    if (k < 1 || k > NVFP4_TOPK_MAX_K || k > V)
        return set_error(NVFP4_EINVAL, "k: %d outside [1, min(V, %d)]", k, NVFP4_TOPK_MAX_K);
    if (!logits_dev) return set_error(NVFP4_EINVAL, "logits: NULL");
    if (!idx_dev) return set_error(NVFP4_EINVAL, "idx: NULL");
    if (!val_dev) return set_error(NVFP4_EINVAL, "val: NULL");
    if (((uintptr_t)logits_dev | (uintptr_t)idx_dev | (uintptr_t)val_dev) & 3)
        return set_error(NVFP4_EINVAL, "logits/idx/val: not 4-byte aligned");
    if ((size_t)M * ld > 0x7FFFFFFFu)
        return set_error(NVFP4_EINVAL, "M * ld: %zu elements, more than 2^31 - 1", (size_t)M * ld);
    const size_t need = nvfp4_topk_workspace_bytes(M, V, k);
    if (workspace_bytes < need)
        return set_error(NVFP4_EINVAL, "workspace_bytes: %zu < %zu needed", workspace_bytes, need);
    if (need && !workspace_dev) return set_error(NVFP4_EINVAL, "workspace: NULL");
    if (need && ((uintptr_t)workspace_dev & 15))
        return set_error(NVFP4_EINVAL, "workspace: not 16-byte aligned");
    hipStream_t s = (hipStream_t)stream;
    int u0 = 0;
    const int levels = topk_levels(V, k, &u0);
    const size_t half = need / 2;
    u64* buf[2] = {(u64*)workspace_dev, need ? (u64*)((char*)workspace_dev + half) : nullptr};
    const dim3 block(kTopkThreads);
    constexpr int kWaves = kTopkThreads / 64;
    auto blocks = [](int units) { return (unsigned)((units + kWaves - 1) / kWaves); };
    if (levels == 1) {
        hipLaunchKernelGGL((topk_level_kernel<true, true>), dim3(1, M), block, 0, s, logits_dev,
                           ld, nullptr, V, k, 1, nullptr, idx_dev, val_dev);
        NVFP4_HIP(hipGetLastError());
        return NVFP4_OK;
    }
    hipLaunchKernelGGL((topk_level_kernel<true, false>), dim3(blocks(u0), M), block, 0, s,
                       logits_dev, ld, nullptr, V, k, u0, buf[0], nullptr, nullptr);
    NVFP4_HIP(hipGetLastError());
    if (k <= kMergeMaxK && u0 <= 64 * kMergeRuns) {
        hipLaunchKernelGGL(topk_merge_kernel, dim3(M), dim3(64), 0, s, logits_dev, ld, buf[0], u0,
                           k, idx_dev, val_dev);
        NVFP4_HIP(hipGetLastError());
        return NVFP4_OK;
    }
    int n = u0 * k, cur = 0;
    for (int l = 1; l < levels; ++l) {
        const int u = (n + kTopkUnit - 1) / kTopkUnit;
        if (l == levels - 1)
            hipLaunchKernelGGL((topk_level_kernel<false, true>), dim3(1, M), block, 0, s,
                               logits_dev, ld, buf[cur], n, k, 1, nullptr, idx_dev, val_dev);
        else
            hipLaunchKernelGGL((topk_level_kernel<false, false>), dim3(blocks(u), M), block, 0,
                               s, logits_dev, ld, buf[cur], n, k, u, buf[cur ^ 1], nullptr,
                               nullptr);
        NVFP4_HIP(hipGetLastError());
        cur ^= 1;
        n = u * k;
    }
    return NVFP4_OK;
}

}  // extern "C"
