// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/nvfp4.h"

namespace nvfp4 {

// ---- packed layout -----------------------------------------------------------
// A weight matrix is cut into column tiles of 16 outputs (one MFMA column
// block) and K superblocks of 512 values.  One (tile, superblock) holds:
//   codes : 4 KiB = [kb 0..3][lane 0..63][16 bytes]; lane l (column l%16, K
//           octet g = l/16) holds, for MFMA step s = 0..3, the 4 canonical code
//           bytes of k = sb*512 + kb*128 + 32*s + 8*g .. +7 at bytes 4s..4s+3.
//   scales: 512 B = [column 0..15][half p 0..1][kb 0..3][step s 0..3]: the
//           E4M3 byte of block (sb*512 + kb*128 + 32*s + 16*p) / 16.
// Tiles are stored column-tile major, superblocks ascending within a tile, so
// one wave streams one contiguous range per column tile.
constexpr int kTileN = 16;
constexpr int kSuperK = 512;
constexpr int kCodeBytesPerSuper = kTileN * kSuperK / 2;     // 4096
constexpr int kScaleBytesPerSuper = kTileN * kSuperK / 16;   // 512

inline int round_up(int x, int m) { return (x + m - 1) / m * m; }
inline int padded_k(int K) { return round_up(K, kSuperK); }
inline int padded_n(int N) { return round_up(N, kTileN); }

// ---- errors --------------------------------------------------------------------
int set_error(int status, const char* fmt, ...);
void clear_error();
int hip_fail(hipError_t e, const char* what);

#define NVFP4_HIP(call)                                           \
    do {                                                          \
        hipError_t e_ = (call);                                   \
        if (e_ != hipSuccess) return ::nvfp4::hip_fail(e_, #call); \
    } while (0)

// ---- plans ---------------------------------------------------------------------
struct DecodeConfig {
    int waves;          // column tiles (waves) per workgroup
    int chunks;         // superblocks of 512 k per window (loaded up front per wave)
    int windows;        // windows per K slice (> 1: the streaming decode_window_kernel)
    int splits;         // K slices
    int n_groups;       // column groups of `waves` tiles
    int grid;           // workgroups launched (n_groups padded to 8, times splits)
    int l2_local;       // split-K partials stay in one XCD's L2 (mapping verified)
    int per_xcd;        // verify widths: workgroups per XCD (equal ranges of its windows)
    int slots;          // verify widths: partial-sum slots per column group
    int lds_pad;        // verify widths: dynamic LDS bytes requested beyond the kernel's own
    // Workspace layout: [counters: counter_bytes][partial sums: partial_bytes].
    // Counters come first so that, when several plans share one workspace (a
    // round), no plan's partial sums ever overlap any plan's counters.
    size_t counter_bytes;
    size_t partial_bytes;
    size_t ws_bytes;    // counter_bytes + partial_bytes
};

// Verify widths (8 < M <= 64): the decode layout for 16 G rows, G = ceil(M / 16).
struct VerifyConfig {
    int enabled;   // max_M > 8
    int rows;      // rows the workspace holds: ceil(min(max_M, 64) / 16) * 16
    DecodeConfig g[4];  // launch config for G = 1..4 row groups of 16 (up to the plan's rows)
    DecodeConfig d;     // workspace envelope of both: counter and partial areas, ws_bytes
    size_t ws_off; // offset of its counters and partials in the plan's workspace
};

// Narrow widths (M <= 4): one workgroup per column tile over all of K, its
// waves splitting K and adding their sums in LDS (decode_tile_kernel).
struct TileConfig {
    int max_m;  // largest M routed to the tile kernel (0: none)
    int sbw;    // superblocks of 512 k per wave (1..3)
    int waves;  // waves per workgroup: ceil(K superblocks / sbw), 1..16
};

struct PrefillConfig {
    int enabled;
    int schedule;          // NVFP4_PREFILL_*: 0 by shape
    int cus;               // compute units the schedule and workspace are laid out for
    size_t ws_off;         // [counters][partial sums] of split tiles: offset in the workspace
    size_t counter_bytes;  // the counters' share (stream-K hand-offs; zero between runs)
    size_t ws_bytes;       // and the whole area (0: no M the plan serves splits)
};

}  // namespace nvfp4

struct nvfp4_gemm_plan {
    uint32_t magic;
    int max_M, K, N, out_dtype;
    int Kp, Np;
    nvfp4::DecodeConfig dec;
    nvfp4::TileConfig tile;
    nvfp4::VerifyConfig ver;
    nvfp4::PrefillConfig pre;
    size_t ws_bytes;
};

namespace nvfp4 {
constexpr uint32_t kGemmMagic = 0x4E564634u;  // "NVF4"
constexpr uint32_t kRoundMagic = 0x524F4E44u;

// Compute units of the current device (cached per device; 256 if the query fails).
int device_cus();
// Workgroup b runs on XCD b % 8 on the current device (checked once per device).
int xcd_mapping_verified();
int make_verify_config(int K, int N, int max_M, const nvfp4_gemm_config* cfg, VerifyConfig* out);
int make_decode_config(int K, int N, int max_M, const nvfp4_gemm_config* cfg, DecodeConfig* out);
int make_tile_config(int K, int N, int max_M, const nvfp4_gemm_config* cfg, TileConfig* out);
int make_prefill_config(int max_M, int K, int N, const nvfp4_gemm_config* cfg,
                        PrefillConfig* out);

// Launchers (no validation: callers validated).  Return NVFP4_OK or EHIP.
// ws: the workspace; partial_off: byte offset of the partial sums in it (the
// plan's own counter_bytes, or a larger value shared by the plans of a round).
int launch_decode(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                  float ts, const uint16_t* act, void* out, void* ws, size_t partial_off,
                  hipStream_t s);
int launch_decode_argmax(const nvfp4_gemm_plan* p, int M, const uint8_t* codes,
                         const uint8_t* scales, float ts, const uint16_t* act, float* out,
                         void* ws, size_t partial_off, void* area, int* argmax, hipStream_t s);
int launch_tile(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                float ts, const uint16_t* act, void* out, hipStream_t s);
int launch_verify(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                  float ts, const uint16_t* act, void* out, void* ws, size_t counters_off,
                  size_t partial_off, hipStream_t s);
// pre_off: byte offset of the K pieces' partial sums in ws (the plan's own
// pre.ws_off, or another place a caller lays out).
int launch_prefill(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
                   float ts, const uint16_t* act, void* out, void* ws, size_t ctr_off,
                   size_t pre_off, int schedule, hipStream_t s);
// Counter and partial-sum bytes a prefill run of M rows uses with `schedule`
// (an NVFP4_PREFILL_* value; a plan runs its own, pre.schedule).
void prefill_ws_need(const nvfp4_gemm_plan* p, int M, int schedule, size_t* counters,
                     size_t* partials);
int launch_fill_zero(void* p, size_t bytes, hipStream_t s);
int launch_swiglu(const uint16_t* gate_up, uint16_t* out, int M, int F, hipStream_t s);
// gate_up with the SwiGLU of its output written to h (round chaining); only
// where decode_swiglu_fusable holds.
bool decode_swiglu_fusable(const nvfp4_gemm_plan* p, int M);
int launch_decode_swiglu(const nvfp4_gemm_plan* p, int M, const uint8_t* codes,
                         const uint8_t* scales, float ts, const uint16_t* act, void* out,
                         uint16_t* h, void* ws, size_t partial_off, hipStream_t s);

// Shared validation of a GEMM run against its plan.
int validate_run(const nvfp4_gemm_plan* p, int M, int K, int N, const void* codes,
                 const void* scales, const void* act, const void* out, const void* ws);
// Where a run's split-K state sits in the workspace: a plan's own layout
// (gemm_offsets), or the shared counter and partial regions of a round.
struct RunOffsets {
    size_t dec_partial;   // decode partials (its counters start at 0)
    size_t ver_counters;  // verify-width counters
    size_t ver_partial;   // verify-width partials
    size_t pre_counters;  // prefill stream-K counters
    size_t pre_partial;   // prefill partial sums (stream-K slots or K pieces)
};
RunOffsets gemm_offsets(const nvfp4_gemm_plan* p);
int run_gemm(const nvfp4_gemm_plan* p, int M, const uint8_t* codes, const uint8_t* scales,
             float ts, const uint16_t* act, void* out, void* ws, const RunOffsets& off,
             hipStream_t s);
}  // namespace nvfp4
