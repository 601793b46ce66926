/*
 * NVFP4 oracle: a plain, slow CPU implementation of what the weight-streaming
 * decode GEMM computes.  TEST INFRASTRUCTURE ONLY: the tests, the smoke check
 * and the benchmark's CPU-baseline leg are the only users.  It shares no code
 * with the HIP library and the HIP library never calls it.
 *
 * What it follows:
 *  - "Models and artifacts", section "The artifact": the body format is 4-bit
 *    floating point with one scale per 16 values.  The 4-bit element is the
 *    OCP Microscaling v1.0 FP4 E2M1 type (largest magnitude 6); the block scale
 *    is the OCP 8-bit E4M3 "FN" type (no infinities, largest finite 448); one
 *    fp32 scale per tensor multiplies every block scale.
 *  - "Ignis" README, "What sets it apart", "The decode round": one pass over
 *    these weights serves every decode lane, i.e. y[m][n] = sum_k a[m][k]*w[n][k]
 *    for M <= 8 lanes of bf16 activations.
 *  - The quantisation recipe of the synthetic workload: tensor scale
 *    t = amax/(6*448); block scale (block_amax/6)/t rounded to E4M3 with
 *    round-to-nearest-even and saturation; each value divided by the decoded
 *    block scale times t and rounded to E2M1, nearest-even, saturating.
 *
 * Canonical layout (the format, before any GPU packing): weights are N rows of
 * K values.  codes[n][K/2]: byte j holds k = 2j in its low nibble and k = 2j+1
 * in its high nibble.  scales[n][K/16]: one E4M3 byte per block of 16 values.
 *
 * Every floating-point decision (the quantiser) is taken in fp32 with
 * round-to-nearest-even, in the order the recipe states.  The GEMM forms every
 * product in fp64 (it is exact: 8 + 2 + 4 + 24 significant bits <= 53) and sums
 * in ascending k in fp64.
 */
#include <math.h>
#include <pthread.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

/* ---- element decoders (definitions written out) ------------------------- */

/* OCP MX FP4 E2M1: sign bit 3, exponent bits 2..1 (bias 1), mantissa bit 0.
 * Exponent field 0 is subnormal: magnitude = mantissa * 0.5. */
double oracle_e2m1_value(int code) {
    int sign = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double mag;
    if (e == 0)
        mag = m * 0.5;
    else
        mag = ldexp(1.0 + m / 2.0, e - 1);
    return sign ? -mag : mag;
}

/* OCP E4M3 "FN": sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0.
 * Exponent field 0 is subnormal (mantissa * 2^-9); exponent 15 with mantissa 7
 * is NaN; there is no infinity. */
double oracle_e4m3_value(int byte) {
    int sign = (byte >> 7) & 1;
    int e = (byte >> 3) & 15;
    int m = byte & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
double oracle_bf16_value(uint16_t bits) {
    uint32_t u = (uint32_t)bits << 16;
    float f;
    memcpy(&f, &u, 4);
    return (double)f;
}

/* ---- element encoders (nearest representable value, ties to even code) -- */

/* Round a non-negative fp32 value to E4M3 by searching the whole code table
 * for the nearest finite value; on a tie the code with mantissa LSB 0 wins.
 * Values above the largest finite value saturate to it (448). */
int oracle_e4m3_encode(float x) {
    double v = (double)x;
    int best = 0;
    double best_d = INFINITY;
    if (!(v >= 0.0))
        return 0; /* negative / NaN scales are outside the recipe */
    if (v > 448.0)
        v = 448.0; /* saturation: no infinity in E4M3 FN */
    for (int c = 0; c < 0x7F; ++c) { /* 0x00..0x7E: the finite non-negative codes */
        double d = fabs(oracle_e4m3_value(c) - v); /* exact in fp64 */
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return best;
}

/* Round |x| to the nearest E2M1 magnitude (codes 0..7), ties to the even code,
 * saturating at 6; the sign bit of x becomes bit 3 of the code. */
int oracle_e2m1_encode(float x) {
    double v = fabs((double)x);
    int best = 0;
    double best_d = INFINITY;
    for (int c = 0; c < 8; ++c) {
        double d = fabs(oracle_e2m1_value(c) - v);
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best = c;
            best_d = d;
        }
    }
    return best | (signbit(x) ? 8 : 0);
}

/* ---- quantiser ----------------------------------------------------------- */

/* Tensor scale t = amax / (6 * 448) in fp32. */
float oracle_tensor_scale(const float* w, size_t count) {
    float amax = 0.0f;
    for (size_t i = 0; i < count; ++i) {
        float a = fabsf(w[i]);
        if (a > amax)
            amax = a;
    }
    return amax / 2688.0f;
}

/* Quantise rows [n0, n1) of a row-major [N][K] fp32 matrix with a given tensor
 * scale t, writing those rows of the canonical code and scale planes.
 * K must be a multiple of 16.  A block whose decoded scale is 0 (tensor or
 * block all zero, or a block scale that rounds to 0) gets all codes +0. */
void oracle_quantize_rows(const float* w, int K, int n0, int n1, float t,
                          uint8_t* codes, uint8_t* scales) {
    for (int n = n0; n < n1; ++n) {
        const float* row = w + (size_t)n * K;
        for (int b = 0; b < K / 16; ++b) {
            const float* blk = row + 16 * b;
            float bamax = 0.0f;
            for (int i = 0; i < 16; ++i) {
                float a = fabsf(blk[i]);
                if (a > bamax)
                    bamax = a;
            }
            int sc = 0;
            if (t > 0.0f) {
                float s = (bamax / 6.0f) / t;
                sc = oracle_e4m3_encode(s);
            }
            scales[(size_t)n * (K / 16) + b] = (uint8_t)sc;
            float d = (float)oracle_e4m3_value(sc) * t; /* decoded scale, fp32 */
            for (int i = 0; i < 16; i += 2) {
                int c0 = 0, c1 = 0;
                if (d > 0.0f) {
                    c0 = oracle_e2m1_encode(blk[i] / d);
                    c1 = oracle_e2m1_encode(blk[i + 1] / d);
                }
                codes[(size_t)n * (K / 2) + 8 * b + i / 2] = (uint8_t)(c0 | (c1 << 4));
            }
        }
    }
}

/* Whole-matrix quantiser: returns the tensor scale. */
float oracle_quantize(const float* w, int N, int K, uint8_t* codes, uint8_t* scales) {
    float t = oracle_tensor_scale(w, (size_t)N * K);
    oracle_quantize_rows(w, K, 0, N, t, codes, scales);
    return t;
}

/* ---- dequantisation and the GEMM ---------------------------------------- */

/* w[n][k] = E2M1(code) * E4M3(block scale) * t, exact in fp64. */
double oracle_weight(const uint8_t* codes, const uint8_t* scales, int K, float t,
                     int n, int k) {
    uint8_t byte = codes[(size_t)n * (K / 2) + k / 2];
    int code = (k & 1) ? (byte >> 4) : (byte & 15);
    int sc = scales[(size_t)n * (K / 16) + k / 16];
    return oracle_e2m1_value(code) * oracle_e4m3_value(sc) * (double)t;
}

/* y[m][n] = sum_k a[m][k] * w[n][k] and S[m][n] = sum_k |a[m][k] * w[n][k]|
 * for columns n in [n0, n1); ascending k, fp64.  act is bf16 bits [M][K];
 * y and S are [M][N] row-major (S may be NULL). */
void oracle_gemm_cols(int M, int K, int N, const uint8_t* codes, const uint8_t* scales,
                      float t, const uint16_t* act, int n0, int n1, double* y, double* S) {
    for (int n = n0; n < n1; ++n) {
        for (int m = 0; m < M; ++m) {
            double acc = 0.0, mag = 0.0;
            for (int k = 0; k < K; ++k) {
                double p = oracle_bf16_value(act[(size_t)m * K + k]) *
                           oracle_weight(codes, scales, K, t, n, k);
                acc += p;
                mag += fabs(p);
            }
            y[(size_t)m * N + n] = acc;
            if (S)
                S[(size_t)m * N + n] = mag;
        }
    }
}

/* Threaded driver: splits the columns into `threads` contiguous ranges; each
 * output is still computed by oracle_gemm_cols exactly as above. */
typedef struct {
    int M, K, N, n0, n1;
    const uint8_t *codes, *scales;
    float t;
    const uint16_t* act;
    double *y, *S;
} oracle_job;

static void* oracle_job_run(void* p) {
    oracle_job* j = (oracle_job*)p;
    oracle_gemm_cols(j->M, j->K, j->N, j->codes, j->scales, j->t, j->act, j->n0, j->n1,
                     j->y, j->S);
    return NULL;
}

int oracle_gemm(int M, int K, int N, const uint8_t* codes, const uint8_t* scales, float t,
                const uint16_t* act, double* y, double* S, int threads) {
    if (threads < 1)
        threads = 1;
    if (threads > 256)
        threads = 256;
    if (threads > N)
        threads = N > 0 ? N : 1;
    pthread_t tid[256];
    oracle_job jobs[256];
    int started = 0;
    for (int i = 0; i < threads; ++i) {
        jobs[i] = (oracle_job){M, K, N, (int)((long long)N * i / threads),
                               (int)((long long)N * (i + 1) / threads), codes, scales, t, act,
                               y, S};
    }
    for (int i = 1; i < threads; ++i) {
        if (pthread_create(&tid[i], NULL, oracle_job_run, &jobs[i]) != 0)
            break;
        started = i;
    }
    oracle_job_run(&jobs[0]);
    for (int i = started + 1; i < threads; ++i) /* any range not started runs here */
        oracle_job_run(&jobs[i]);
    for (int i = 1; i <= started; ++i)
        pthread_join(tid[i], NULL);
    return threads;
}
