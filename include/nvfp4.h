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

/* Largest k of nvfp4_topk. */
#define NVFP4_TOPK_MAX_K 64

/* ---- status ----------------------------------------------------------------- */

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

/* Decode kernels (M <= 8). */
enum nvfp4_kernel {
    NVFP4_KERNEL_AUTO = 0,
    NVFP4_KERNEL_STREAM = 1, /* full-K column groups, per-wave weight ring */
    NVFP4_KERNEL_SPLITK = 2  /* K split over workgroups, last one reduces (default) */
};

/* Optional kernel configuration for nvfp4_gemm_create_ex; 0 fields mean
 * "choose automatically". */
typedef struct nvfp4_gemm_config {
    int split_k; /* SPLITK: number of K slices (workgroups per column group) */
    int waves;   /* SPLITK: waves per workgroup (column tiles of 16), 4 or 8 */
    int chunks;  /* SPLITK: K values per slice in units of 512, 1..4 (when
                    split_k is 0) */
    int kernel;  /* nvfp4_kernel */
    int tiles;   /* STREAM: column tiles of 16 per workgroup, 2, 4 or 8 */
    int windows; /* SPLITK: windows of `chunks` superblocks per K slice; above 1 a
                    wave streams its slice, issuing the next window's loads
                    before computing the current one (0 or 1: one window) */
    int verify_waves;   /* verify widths (8 < M <= 64): waves per workgroup, 4, 8
                           or 16 (0: 4 up to 48 rows, 8 above) */
    int verify_windows; /* verify widths: superblocks per K slice (0: by shape) */
} nvfp4_gemm_config;

/* Create a plan for GEMMs of shape (M <= max_M) x K x N with the given output
 * dtype.  Validates K % 16 == 0, K >= 16, N >= 1, max_M >= 1, out_dtype.
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
 * the weights for all M rows); larger M uses the bf16 MFMA prefill kernel,
 * and, when the 256 x 256 output tiles leave a last partial round on the
 * device's compute units, a second kernel that adds the fp32 partial sums of
 * those tiles' K pieces.  The workspace holds, in this order, the decode,
 * verify and prefill areas the plan's max_M needs.  Asynchronous; no
 * synchronisation. */
int nvfp4_gemm_run(nvfp4_gemm plan, int M, int K, int N, const uint8_t* codes_dev,
                   const uint8_t* scales_dev, float tensor_scale, const uint16_t* act_dev,
                   void* out_dev, void* workspace_dev, void* stream);

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
 * max_M rows of N outputs.  act_op: nvfp4_act_op (PER_MATRIX rounds only). */
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

/* Forms of a round (see nvfp4_round_create_ex). */
enum nvfp4_round_mode {
    NVFP4_ROUND_PERSISTENT = 0, /* one persistent kernel walks every matrix */
    NVFP4_ROUND_PER_MATRIX = 1, /* one decode kernel per matrix */
    NVFP4_ROUND_CHAIN = 2       /* one launch whose workgroups run the matrices in order */
};

/* Workspace a round over these layers needs in the given form (the default
 * form is NVFP4_ROUND_PER_MATRIX). */
int nvfp4_round_workspace_bytes(const nvfp4_layer* layers, int n_layers, int max_M,
                                size_t* workspace_bytes);
int nvfp4_round_workspace_bytes_ex(const nvfp4_layer* layers, int n_layers, int max_M, int mode,
                                   size_t* workspace_bytes);

/* Capture one HIP graph per width M = 1..max_M, each running the n_layers
 * GEMMs in list order, as the reference engine replays one graph per batch
 * width.  max_M <= 64 for PER_MATRIX (widths above 8, the verify widths of
 * speculative decoding, launch the verify-width kernel), <= 8 for the other
 * forms.  Matrix i+1 starts computing only once every output of matrix
 * i is written (the order of a forward pass in which each matrix consumes the
 * previous one's result).
 *   PER_MATRIX : the graph holds one decode (or verify-width) kernel launch
 *                per matrix.
 *   PERSISTENT : the graph holds one kernel whose resident workgroups walk
 *                every matrix; the next matrix's weights are fetched while the
 *                previous matrix finishes (no launch boundary between them).
 *                Outputs are written with device-coherent stores.  Its waits
 *                are bounded: a wait that times out raises a flag read by
 *                nvfp4_round_status (the results are then not valid).  The
 *                grid assumes it has the device to itself while it runs.
 *   CHAIN      : the graph holds one launch whose workgroups are the
 *                decode workgroups of every matrix, in list order ("Ignis"
 *                README, "Lineage": "Credits" -- the round's decode kernels
 *                are chained so that each GEMM's start overlaps the previous
 *                one's drain).  A workgroup issues its weight loads, then
 *                waits until the previous matrix is complete, then reads its
 *                activations.  Outputs are written with device-coherent
 *                stores; activations that overlap an earlier matrix's output
 *                are read with device-coherent loads.  Waits are bounded as in
 *                PERSISTENT.  Needs workgroups spread evenly over the 8 XCDs
 *                (checked here: NVFP4_EUNSUPPORTED otherwise).  The workspace
 *                holds a split-K region per matrix (about 10.5 MB per layer of
 *                the 27B-class round).
 * The layer array is copied; the device buffers it names must stay valid
 * while the plan lives.  The workspace (nvfp4_round_workspace_bytes_ex
 * bytes, 16-byte aligned) is zeroed and written here, then owned by the plan
 * until it is destroyed.  Synchronises `stream`.  nvfp4_round_create is the
 * PER_MATRIX form (measured faster on MI355X for the 27B-class round). */
int nvfp4_round_create(nvfp4_round* plan, const nvfp4_layer* layers, int n_layers, int max_M,
                       void* workspace_dev, size_t workspace_bytes, void* stream);
int nvfp4_round_create_ex(nvfp4_round* plan, const nvfp4_layer* layers, int n_layers, int max_M,
                          int mode, void* workspace_dev, size_t workspace_bytes, void* stream);
/* Error flags raised by the replays since the last call (bit 0: a wait timed
 * out), then cleared; after a time-out the plan's counters are also re-zeroed
 * so later replays are valid again.  Synchronises the device.  Always 0 for
 * PER_MATRIX. */
int nvfp4_round_status(nvfp4_round plan, unsigned int* flags);
/* Bound on the polling rounds of each wait of a PERSISTENT or CHAIN round (default
 * 2^16, tens of milliseconds).  Synchronises the device. */
int nvfp4_round_set_spin_limit(nvfp4_round plan, unsigned int limit);
/* Replay the graph of width M (1..max_M) on `stream`. */
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

#ifdef __cplusplus
}
#endif

#endif /* NVFP4_H */
