/*
 * nvfp4.h -- C ABI of the MI355X (gfx950) NVFP4 weight-streaming GEMM library.
 *
 * What the library computes
 *   The decode round of "Ignis" (README, "What sets it apart", "The decode
 *   round"; and "Why ignis", tile "One round for every lane"): one pass over
 *   weights stored in NVFP4 serves every decode lane at once, so the round is
 *   bound by the bandwidth of streaming the weights.  The body format is the
 *   one "Models and artifacts" gives in "The artifact": 4-bit floating point
 *   with one scale per 16 values, read by the kernels as stored.
 *
 *     y[m][n] = tensor_scale * sum_k bf16(a[m][k]) * E2M1(code[n][k])
 *                                   * E4M3(scale[n][k/16])
 *
 *   for M lanes (rows of activations), K inputs and N outputs.  E2M1 is the
 *   OCP MX FP4 element, E4M3 the OCP FP8 "FN" type (max 448), tensor_scale an
 *   fp32 per-matrix factor.  Products are exact; sums are in fp32.
 *
 * Canonical weight planes (the format as produced by a quantiser)
 *   codes  : uint8 [N][K/2]; byte j of row n holds k = 2j in bits 0..3 and
 *            k = 2j+1 in bits 4..7.
 *   scales : uint8 [N][K/16]; one E4M3 byte per block of 16 consecutive k.
 *   Kernels read a packed permutation of these planes made once by
 *   nvfp4_pack (no conversion at load beyond that permutation).
 *
 * Conventions for every entry point
 *   - Pointers named *_dev are device pointers (e.g. from hipMalloc or a torch
 *     CUDA tensor); the caller owns all device memory.  The library allocates
 *     no device memory except the graph objects of a round plan.
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *     Every launch is asynchronous on that stream; no entry point synchronises
 *     except nvfp4_round_create (graph capture) and nvfp4_quantize (none: the
 *     tensor scale stays on the device).
 *   - Return value: NVFP4_OK or an error code.  On error nothing was launched
 *     and nvfp4_last_error() (thread-local) names the offending parameter.
 *     No entry point aborts, exits or throws.
 *   - NaN/Inf activations, NaN scale bytes (0x7F, 0xFF) and negative scales
 *     are outside the contract and are not checked.
 */
#ifndef NVFP4_H
#define NVFP4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum nvfp4_status {
    NVFP4_OK = 0,
    NVFP4_EINVAL = 1,       /* a parameter is invalid (named by nvfp4_last_error) */
    NVFP4_EUNSUPPORTED = 2, /* a legal request outside what this plan/build supports */
    NVFP4_EHIP = 3,         /* the HIP runtime returned an error (message carried) */
    NVFP4_ESTATE = 4        /* misuse of a handle (destroyed, wrong plan) */
};

enum nvfp4_out_dtype { NVFP4_OUT_F32 = 0, NVFP4_OUT_BF16 = 1 };

/* Largest number of lanes (activation rows) the decode kernel serves in one
 * weight pass. */
#define NVFP4_DECODE_MAX_M 8
/* Largest M of the verify-width decode kernel ("Ignis" README, "Speculative
 * decoding (DFlash2)": up to seven drafts per lane are checked in the same
 * pass, so 8 lanes x (1 + 7) rows); still one pass over the weights.  Larger
 * M goes to the prefill kernel. */
#define NVFP4_VERIFY_MAX_M 64

/* Prefill schedules (nvfp4_gemm_config.prefill_schedule) for M > 64, whose
 * 256 x 256 output tiles are spread over the compute units: */
enum nvfp4_prefill_schedule {
    NVFP4_PREFILL_AUTO = 0,     /* stream-K below one tile per compute unit (see
                                   nvfp4_gemm_run), else pieces */
    NVFP4_PREFILL_PIECES = 1,   /* whole tiles; the tiles of a last partial round cut
                                   along K into pieces, added by a second kernel */
    NVFP4_PREFILL_STREAM_K = 2  /* wherever it applies (tiles not a multiple of the
                                   compute units, runs of at least half a tile): every
                                   compute unit takes an equal run of the tiles' K
                                   stages laid end to end; a tile shared by two or three
                                   units is finished by the last */
};

/* Largest k of nvfp4_topk. */
#define NVFP4_TOPK_MAX_K 64

/* ---- status ----------------------------------------------------------------- */

/* Errors stay with the call that raised them: the credits of the pages' engine
 * ("Lineage", "Credits") list a per-request error boundary among its kernel
 * work, and here each entry point reports its own failure through its return
 * value and this thread's last-error text, launching nothing on a refused call
 * and leaving other plans, rounds and threads untouched. */

/* Static text of a status code. */
const char* nvfp4_status_string(int status);
/* Thread-local text of the last error raised on this thread ("" if none). */
const char* nvfp4_last_error(void);
/* Library version as an integer (major*10000 + minor*100 + patch). */
int nvfp4_version(void);

/* ---- packed layout ----------------------------------------------------------- */

/* Bytes of the packed code / scale planes for a K x N weight matrix.  They
 * include padding of K to a multiple of 512 and of N to a multiple of 16
 * (padding is zero codes and zero scales).  Return 0 for invalid K or N
 * (K % 16 != 0, K < 16, N < 1). */
size_t nvfp4_packed_code_bytes(int K, int N);
size_t nvfp4_packed_scale_bytes(int K, int N);

/* Permute canonical planes into the packed gfx950 layout (a bijection on the
 * non-padding bytes, bit-exact).  codes_dev: [N][K/2], scales_dev: [N][K/16];
 * outputs sized by the two functions above, 16-byte aligned.  Inputs and
 * outputs must not overlap. */
int nvfp4_pack(const uint8_t* codes_dev, const uint8_t* scales_dev, int K, int N,
               uint8_t* codes_packed_dev, uint8_t* scales_packed_dev, void* stream);

/* Inverse of nvfp4_pack (for tests and export). */
int nvfp4_unpack(const uint8_t* codes_packed_dev, const uint8_t* scales_packed_dev, int K,
                 int N, uint8_t* codes_dev, uint8_t* scales_dev, void* stream);

/* ---- quantiser ----------------------------------------------------------------- */

/* Quantise fp32 weights w_dev [N][K] (row-major, K % 16 == 0) to canonical
 * NVFP4 planes: tensor scale t = amax/(6*448); block scale = (block amax/6)/t
 * rounded to E4M3 (nearest-even, saturating at 448); each value w/(E4M3*t)
 * rounded to E2M1 (nearest-even, saturating at 6, sign kept; a block whose
 * decoded scale is 0 gets +0 codes).  All arithmetic fp32, round to nearest
 * even.  Writes codes_dev [N][K/2], scales_dev [N][K/16] and the fp32 tensor
 * scale to *tensor_scale_dev (device memory).  workspace_dev: at least
 * nvfp4_quantize_workspace_bytes() bytes, any content. */
size_t nvfp4_quantize_workspace_bytes(void);
int nvfp4_quantize(const float* w_dev, int K, int N, uint8_t* codes_dev, uint8_t* scales_dev,
                   float* tensor_scale_dev, void* workspace_dev, void* stream);

/* ---- GEMM plan --------------------------------------------------------------------- */

typedef struct nvfp4_gemm_plan* nvfp4_gemm;

/* Optional kernel configuration for nvfp4_gemm_create_ex; 0 fields mean
 * "choose automatically". */
typedef struct nvfp4_gemm_config {
    int split_k; /* decode: number of K slices (workgroups per column group) */
    int waves;   /* decode: waves per workgroup (column tiles of 16), 4 or 8 */
    int chunks;  /* decode: K values per slice in units of 512, 1..4 (when
                    split_k is 0) */
    int windows; /* decode: windows of `chunks` superblocks per K slice; above 1
                    a wave streams its slice, issuing the next window's loads
                    before computing the current one (0 or 1: one window) */
    int verify_waves;   /* verify widths (8 < M <= 64): waves (column tiles) per
                           workgroup, 4, 8 or 16 (0: by shape) */
    int verify_windows; /* verify widths: superblocks of 512 k per K slice of a
                           column group (0: by shape) */
    int tile_max_m;     /* widths M <= tile_max_m (at most 4) run the kernel with one
                           workgroup per 16-column tile over all of K, its waves
                           splitting K and adding in LDS (no workspace); 0: by shape
                           (up to 4 for matrices of fewer than 4 x compute-unit
                           tiles, 2 for wider ones, none when K needs more than 12
                           waves); -1: never */
    int tile_superblocks; /* that kernel: superblocks of 512 k per wave, 1..3 (0: by
                             shape) */
    int verify_ranges;  /* verify widths: 1..4 workgroups per compute unit taking
                           equal ranges of their XCD's superblocks, a range
                           running on from one column group into the next, in
                           place of per-group K slices (0: by shape; not with
                           verify_windows) */
    int prefill_schedule; /* M > 64: an nvfp4_prefill_schedule */
} nvfp4_gemm_config;

/* Create a plan for GEMMs of shape (M <= max_M) x K x N with the given output
 * dtype.  Validates K % 16 == 0, K >= 16, N >= 1, max_M >= 1, out_dtype;
 * returns NVFP4_EUNSUPPORTED for K >= 2^24, and for K >= 2^22 when max_M > 64
 * (the kernels above 8 rows address activations with 32-bit byte offsets).
 * The first plan made on a device also runs a one-off check of the device's
 * workgroup-to-XCD dispatch order (one tiny kernel and a synchronisation);
 * split-K plans use the cheaper in-L2 hand-off of partial sums only if it
 * holds.
 * *workspace_bytes receives the device workspace every run of this plan
 * needs (may be 0).  The workspace must be zero-filled before its first use
 * (nvfp4_workspace_clear or any zero fill); every run leaves its counter
 * region zeroed again.  A workspace belongs to one plan: runs of different
 * plans (or overlapping runs of one plan on different streams) must not share
 * it -- a round plan lays out one workspace for all of its matrices itself.
 * No device memory is allocated. */
int nvfp4_gemm_create(nvfp4_gemm* plan, int max_M, int K, int N, int out_dtype,
                      size_t* workspace_bytes);
int nvfp4_gemm_create_ex(nvfp4_gemm* plan, int max_M, int K, int N, int out_dtype,
                         const nvfp4_gemm_config* config, size_t* workspace_bytes);
void nvfp4_gemm_destroy(nvfp4_gemm plan);

/* Run out[m][n] = tensor_scale * sum_k act[m][k] * w[n][k] for m < M.
 *   codes_dev, scales_dev : packed planes (nvfp4_pack) of the K x N matrix
 *   act_dev               : bf16 bits [M][K] row-major, 16-byte aligned
 *   out_dev               : [M][N] row-major, fp32 or bf16 (plan's dtype;
 *                           bf16 is round-to-nearest-even of the fp32 result)
 *   workspace_dev         : the plan's workspace (16-byte aligned), or NULL
 *                           if the plan needs none
 * (K, N) must equal the plan's, 1 <= M <= max_M.  M <= 8 uses the decode
 * kernel and 8 < M <= 64 the verify-width decode kernel (each one pass over
 * the weights for all M rows); larger M uses the bf16 MFMA prefill kernel.
 * With fewer 256 x 256 output tiles than the device's compute units, at
 * most 3/4 of them, it runs the stream-K schedule (one workgroup per compute
 * unit, equal runs of K stages of at least half a tile; the fp32 partial
 * sums of a tile shared by two or three runs meet in the workspace and the
 * last contributor adds them in run order).  Otherwise whole tiles, with a
 * last partial round's tiles cut along K and a second kernel adding their
 * pieces.  nvfp4_gemm_config.prefill_schedule can ask for either wherever it
 * applies.  The workspace holds, in this order, the
 * decode, verify and prefill areas the plan's max_M needs.  For M > 8 and K not a
 * multiple of 512, every activation value must be finite: those kernels read
 * the tail of a row's last K window from the start of the next row and
 * multiply it by the zero weights past K (an infinity or NaN there would turn
 * into NaN sums of another row).  Rows of M <= 8 end at K.  Asynchronous; no
 * synchronisation. */
int nvfp4_gemm_run(nvfp4_gemm plan, int M, int K, int N, const uint8_t* codes_dev,
                   const uint8_t* scales_dev, float tensor_scale, const uint16_t* act_dev,
                   void* out_dev, void* workspace_dev, void* stream);

/* Bytes of the area nvfp4_gemm_run_argmax needs for this plan (one slot of
 * 8 row keys per column group of the decode kernel); 0 for an invalid handle
 * or a bf16 plan. */
size_t nvfp4_gemm_argmax_area_bytes(nvfp4_gemm plan);

/* The output head's step with greedy sampling fused in ("Ignis" README,
 * "Speculative decoding (DFlash2)": a top-k over the vocabulary follows the
 * head; here k = 1): runs nvfp4_gemm_run for 1 <= M <= min(8, max_M) rows of
 * an fp32 plan, always with the decode kernel (not the narrow-width one), and
 * also writes argmax_dev[m] = the column of the largest logit of row m, equal
 * values resolved to the smaller column and -0.0 equal to +0.0: the index
 * nvfp4_topk with k = 1 returns for the same logits, which are written to
 * logits_dev [M][N] as nvfp4_gemm_run writes them with the decode kernel
 * (for M <= 4 a plan may route nvfp4_gemm_run to the narrow-width kernel,
 * whose sums can differ in the last bits).  The workgroup that writes a
 * column group's logits also stores the group's row maxima; a second, small
 * kernel takes the maximum over the groups.  NaN logits are out of contract.
 *   argmax_dev  : int32 [M]
 *   area_dev    : area_bytes >= nvfp4_gemm_argmax_area_bytes(plan) bytes,
 *                 16-byte aligned, any content (every word read is written
 *                 first in the same call); owned by the call while it runs.
 * EINVAL for a bf16 plan, M outside [1, min(8, max_M)], a short area, or a
 * NULL or misaligned pointer, before anything is launched.  Asynchronous; no
 * synchronisation. */
int nvfp4_gemm_run_argmax(nvfp4_gemm plan, int M, int K, int N, const uint8_t* codes_dev,
                          const uint8_t* scales_dev, float tensor_scale, const uint16_t* act_dev,
                          float* logits_dev, int* argmax_dev, void* workspace_dev,
                          void* area_dev, size_t area_bytes, void* stream);

/* nvfp4_gemm_run for callers that cannot allocate device memory (code under
 * graph capture, tight serving loops, harnesses that forbid allocation): the
 * same kernels, with the split-K counters and partial sums in a static 16 MiB
 * device array per GPU (held until the process ends) instead of a caller
 * workspace.  Arguments as nvfp4_gemm_run, without the workspace.  Stream-K
 * prefill runs do not fit (their hand-off slots take 512 KiB per compute
 * unit): a default plan runs such an M with whole tiles and K pieces instead,
 * whose sums can differ from nvfp4_gemm_run's in the last bits.  A run that
 * still needs more than 16 MiB of that state (a large prefill chunk, or
 * stream-K asked for by the plan) returns NVFP4_EUNSUPPORTED and launches
 * nothing.  The first call on a device
 * zero-fills the array with one kernel on `stream`, so it must be made
 * outside stream capture (under capture it returns NVFP4_ESTATE and launches
 * nothing); later calls may be captured.  Every call on a GPU uses
 * that GPU's one array: calls that overlap on one GPU (other streams, other
 * threads) race and must be serialised by the caller.  Allocates nothing. */
int nvfp4_gemm_run_noalloc(nvfp4_gemm plan, int M, int K, int N, const uint8_t* codes_dev,
                           const uint8_t* scales_dev, float tensor_scale, const uint16_t* act_dev,
                           void* out_dev, void* stream);

/* Zero a workspace with a fill kernel (safe inside graph capture). */
int nvfp4_workspace_clear(void* workspace_dev, size_t bytes, void* stream);

/* ---- decode round ---------------------------------------------------------------------- */

/* Where a round matrix's activations come from (nvfp4_layer.act_op). */
enum nvfp4_act_op {
    NVFP4_ACT_INPUT = 0,       /* act_dev as the caller filled it */
    NVFP4_ACT_SWIGLU_PREV = 1  /* written by the round before this matrix:
                                  nvfp4_swiglu of the previous matrix's bf16
                                  output (its N must be 2 K): the gated MLP
                                  step between gate_up and down */
};

/* One matrix of a round.  act_dev holds max_M rows of K bf16 values, out_dev
 * max_M rows of N outputs.  act_op: nvfp4_act_op. */
typedef struct nvfp4_layer {
    int K, N;
    const uint8_t* codes_dev;  /* packed */
    const uint8_t* scales_dev; /* packed */
    float tensor_scale;
    const uint16_t* act_dev;
    void* out_dev;
    int out_dtype;
    int act_op;
} nvfp4_layer;

typedef struct nvfp4_round_plan* nvfp4_round;

/* Workspace a round over these layers needs (one split-K counter region and
 * one partial-sum region, shared by the matrices, which run one after the
 * other). */
int nvfp4_round_workspace_bytes(const nvfp4_layer* layers, int n_layers, int max_M,
                                size_t* workspace_bytes);

/* Capture one HIP graph per width M = 1..max_M (max_M <= 64), each running
 * the n_layers GEMMs in list order: the reference engine replays one CUDA
 * graph per batch width ("Ignis" README, "What sets it apart", "The decode
 * round").  The graph of width M holds one kernel launch per matrix (the
 * decode kernel for M <= 8, the verify-width kernel for the widths of
 * speculative verification above 8: "Ignis" README, "Speculative decoding
 * (DFlash2)"), plus one SwiGLU launch before each matrix whose act_op asks for
 * it -- except where the previous matrix (gate_up) runs the streamed-slice
 * decode kernel with 4-wave column groups, bf16 outputs and N a multiple of 64:
 * there its last epilogue per column group also writes the SwiGLU values (the
 * same bits nvfp4_swiglu gives), with its column groups pairing gate tiles
 * with the matching up tiles.  Launches are ordered on one stream, so matrix i+1 starts only once
 * every output of matrix i is written, the order of a forward pass in which
 * each matrix consumes the previous one's result.
 * The layer array is copied; the device buffers it names must stay valid
 * while the plan lives.  The workspace (nvfp4_round_workspace_bytes bytes,
 * 16-byte aligned) is zeroed here, then owned by the plan until it is
 * destroyed.  Synchronises `stream` (graph capture and upload).
 * Errors: EINVAL names the layer and field; EHIP carries the runtime's
 * message (nothing is left allocated). */
int nvfp4_round_create(nvfp4_round* plan, const nvfp4_layer* layers, int n_layers, int max_M,
                       void* workspace_dev, size_t workspace_bytes, void* stream);
/* Replay the graph of width M (1..max_M) on `stream`.  Asynchronous.
 * ESTATE for a destroyed or foreign handle, EINVAL for M out of range. */
int nvfp4_round_run(nvfp4_round plan, int M, void* stream);
/* Number of kernel nodes in the graph of width M (0 on error). */
int nvfp4_round_graph_nodes(nvfp4_round plan, int M);
void nvfp4_round_destroy(nvfp4_round plan);

/* ---- SwiGLU between gate_up and down ------------------------------------------ */

/* out[m][j] = silu(g) * u for g = gate_up[m][j], u = gate_up[m][F + j]
 * (bf16 [M][2F] in, bf16 [M][F] out, row-major), silu(g) = g / (1 + e^-g).
 * The pages leave the layer's non-GEMM steps unstated; this is the reading
 * the round's shapes support (gate_up N = 2 x down K).  Computed in fp64 and
 * rounded once to bf16 (nearest, ties to even).  Asynchronous on `stream`. */
int nvfp4_swiglu(const uint16_t* gate_up_dev, int M, int F, uint16_t* out_dev, void* stream);

/* ---- top-k over the vocabulary ---------------------------------------------- */

/* The step after the output head ("Ignis" README, "Speculative decoding
 * (DFlash2)": the drafter's top-k over the vocabulary, replaced by a
 * row-split kernel with the same answer).  For each row m < M of the fp32
 * logits [M][ld] (first V entries), writes the k largest values in
 * descending order to val_dev[m][0..k-1] and their indices to
 * idx_dev[m][0..k-1] (int32); equal values are listed by ascending index,
 * and -0.0 equals +0.0.  The answer is unique, so it is bit-identical to any
 * correct top-k; values are copied from the logits bit for bit.  NaN logits
 * are out of contract.  1 <= k <= min(V, NVFP4_TOPK_MAX_K), ld >= V,
 * M * ld < 2^31, pointers 4-byte aligned.
 *   workspace_dev: nvfp4_topk_workspace_bytes(M, V, k) bytes (16-byte
 *   aligned; 0 for V <= 1024), any content; owned by the call while it runs.
 * Asynchronous on `stream`; no synchronisation. */
size_t nvfp4_topk_workspace_bytes(int M, int V, int k);
int nvfp4_topk(const float* logits_dev, int M, int V, int ld, int k, int* idx_dev,
               float* val_dev, void* workspace_dev, size_t workspace_bytes, void* stream);

/* ---- measurement ------------------------------------------------------------- */

/* Read `bytes` bytes of buf_dev once with the streaming load shape of the
 * decode kernels' weight stream and no arithmetic: the achievable read rate
 * that the round, which streams the weights at the card's memory bandwidth
 * ("Ignis" README, "What sets it apart", "The decode round"), is measured
 * against.  buf_dev 16-byte aligned, bytes a positive multiple of 16;
 * sink_dev: one device word, written only if the folded value of the data
 * equals an improbable constant (it keeps the loads).  Asynchronous on
 * `stream`; EINVAL names a bad argument before anything is launched. */
int nvfp4_stream_read(const void* buf_dev, size_t bytes, unsigned int* sink_dev, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
