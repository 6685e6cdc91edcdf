/*
 * oracle.c -- plain CPU oracle for the quantized projection matmul.
 *
 * TEST INFRASTRUCTURE ONLY: called by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product library.  It shares no
 * code with the HIP path.  Built with gcc -O2 -fopenmp -ffp-contract=off and
 * no fast-math, so every float operation below is one IEEE operation in the
 * order written.  OpenMP only splits the outermost output loop; each output
 * is computed by one thread in the order written.
 *
 * Sources (web pages, cited by title and section):
 *  [P1] "The ONNX pack: weights to Q4NX, matmuls to our kernels, no VitisAI"
 *       (1bit.gg onnx-pack): sections "The three layers of the pack",
 *       "Why it folds without a new kernel", "What works today, and what
 *       does not", "A real Quark export, through the EP".
 *  [P2] "int8 inference" (onemodel docs): section "Product kernel (Int8Gemm)".
 *  [P4] "NPU engine: full ELFs, no xclbin": section "Q4NX chunks".
 *  [P5] "Zaya 8B Q4NX on the AMD NPU": sections "The bugs that were the
 *       work", "What's next", "Round 26".
 *
 * Parity pins for each routine are in tests/test_oracle_*.py.  None of the
 * routines here is "parity unpinned".
 */
#include "oracle.h"

#include <math.h>
#include <stddef.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the OpenMP loops use from now on (timing only; results do not
 * depend on it). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

static int64_t load_i8(const void *p, int u8, int64_t idx) {
    if (u8) return (int64_t)((const uint8_t *)p)[idx];
    return (int64_t)((const int8_t *)p)[idx];
}

/* [P2] "Product kernel (Int8Gemm)": sums are int32 and cannot overflow while
 * K * 255 * 128 < 2^31. */
int oracle_int8_bound_ok(int64_t K) {
    return K >= 0 && K * 255 * 128 < ((int64_t)1 << 31);
}

/* [P2] "Product kernel (Int8Gemm)": C[m,n] = sum_k (A[m,k]-zA)(B[k,n]-zB),
 * checked there against "a 64-bit naive reference".  This is that reference:
 * the definition itself, in int64, on the unshifted values. */
void oracle_int8_gemm_i64(const void *A, int a_u8, int64_t M, int64_t K, int64_t lda, int32_t zA,
                          const void *B, int b_u8, int64_t N, int64_t ldb, int32_t zB,
                          int64_t *Y, int64_t ldy) {
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t a = load_i8(A, a_u8, m * lda + k) - zA;
                int64_t b = load_i8(B, b_u8, k * ldb + n) - zB;
                acc += a * b;
            }
            Y[m * ldy + n] = acc;
        }
    }
}

/* [P1] "What works today": zero points per axis, one per activation row
 * (zA[m]) and one per weight column (zB[n]), the same axes as the per-axis
 * scales.  The plain definition, written out: Y[m,n] = sum_k (A[m,k] - zA[m])
 * (B[k,n] - zB[n]) in int64. */
void oracle_int8_gemm_axis_i64(const void *A, int a_u8, int64_t M, int64_t K, int64_t lda, const int32_t *zA,
                               const void *B, int b_u8, int64_t N, int64_t ldb, const int32_t *zB,
                               int64_t *Y, int64_t ldy) {
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            int64_t acc = 0;
            for (int64_t k = 0; k < K; ++k) {
                int64_t a = load_i8(A, a_u8, m * lda + k) - zA[m];
                int64_t b = load_i8(B, b_u8, k * ldb + n) - zB[n];
                acc += a * b;
            }
            Y[m * ldy + n] = acc;
        }
    }
}

void oracle_int8_gemm_at(const void *A, int a_u8, int64_t K, int64_t lda, int32_t zA,
                         const void *B, int b_u8, int64_t ldb, int32_t zB,
                         const int64_t *im, const int64_t *in, int64_t count, int64_t *out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i) {
        int64_t m = im[i], n = in[i], acc = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t a = load_i8(A, a_u8, m * lda + k) - zA;
            int64_t b = load_i8(B, b_u8, k * ldb + n) - zB;
            acc += a * b;
        }
        out[i] = acc;
    }
}

/* [P1] "Why it folds without a new kernel": the product is dequantised as
 * C = C_s32 * s_a[m] * s_w[n]; per-tensor and per-axis scales are the same
 * expression.  [P2] "Product kernel": optional bias in the epilogue.  The
 * oracle evaluates it in fp64; the bias is added after scaling. */
void oracle_epilogue_f64(const int64_t *Y, int64_t M, int64_t N, int64_t ldy,
                         const float *rs, const float *cs, float scale, const float *bias,
                         double *out) {
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        double r = rs ? (double)rs[m] : 1.0;
        for (int64_t n = 0; n < N; ++n) {
            double c = cs ? (double)cs[n] : 1.0;
            double v = (double)Y[m * ldy + n] * r * c * (double)scale;
            if (bias) v += (double)bias[n];
            out[m * N + n] = v;
        }
    }
}

/* [P1] "What works today": the readback folds both scales and the output
 * scale into one multiply per element, rounds half to even (ONNX), and adds
 * the output zero point after rounding, so that a tie resolves on the
 * unshifted value (adding an odd zero point first would flip which
 * neighbour is even).  [P1] "A real Quark
 * export": an exact int32 accumulator times an fp32 multiplier can land on
 * either side of a tie from a float-accumulating reference, so this chain is
 * fixed as the definition: every step below is one fp32 operation. */
int oracle_requant(const int64_t *Y, int64_t M, int64_t N, int64_t ldy,
                   const float *rs, const float *cs, float scale, const int32_t *bias_i32,
                   int32_t zp_out, int out_u8, int32_t *out) {
    const int64_t lo = out_u8 ? 0 : -128, hi = out_u8 ? 255 : 127;
    int bad = 0;
    for (int64_t m = 0; m < M; ++m) {
        float r = rs ? rs[m] : 1.0f;
        for (int64_t n = 0; n < N; ++n) {
            float c = cs ? cs[n] : 1.0f;
            int64_t acc = Y[m * ldy + n] + (bias_i32 ? (int64_t)bias_i32[n] : 0);
            if (acc < INT32_MIN || acc > INT32_MAX) { bad = 1; acc = 0; }
            float rc = r * c;
            float mult = rc * scale;
            float facc = (float)(int32_t)acc;  /* int32 -> fp32, round to nearest even */
            float v = facc * mult;
            /* clamp to a range where the conversion below is exact; the final
             * clamp makes this invisible in the result */
            if (v > 65536.0f) v = 65536.0f;
            if (v < -65536.0f) v = -65536.0f;
            float rr = rintf(v);               /* default rounding mode: half to even */
            int64_t q = (int64_t)rr + zp_out;
            if (q < lo) q = lo;
            if (q > hi) q = hi;
            out[m * N + n] = (int32_t)q;
        }
    }
    return bad ? -1 : 0;
}

/* [P1] "The three layers of the pack": packB quantises each column to int8
 * with scale = amax/127 and stores the column scales alongside; activations
 * are quantised per row with amax/127.  Rounding is half to even, the only
 * rounding the pages name; codes stay in [-127, 127]; an all-zero vector
 * gets scale 0 and codes 0. */
static void quantize_vec(const float *x, int64_t n, int64_t stride,
                         int8_t *q, int64_t qstride, float *scale_out) {
    float amax = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float a = fabsf(x[i * stride]);
        if (a > amax) amax = a;
    }
    if (amax == 0.0f) {
        *scale_out = 0.0f;
        for (int64_t i = 0; i < n; ++i) q[i * qstride] = 0;
        return;
    }
    float s = amax / 127.0f;
    *scale_out = s;
    for (int64_t i = 0; i < n; ++i) {
        float v = x[i * stride] / s;
        float r = rintf(v);
        if (r > 127.0f) r = 127.0f;
        if (r < -127.0f) r = -127.0f;
        q[i * qstride] = (int8_t)r;
    }
}

void oracle_pack_b_int8(const float *W, int64_t K, int64_t N, int64_t ldw,
                        int8_t *Q, float *scale, int32_t *colsum) {
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        quantize_vec(W + n, K, ldw, Q + n, N, &scale[n]);
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) s += Q[k * N + n];
        colsum[n] = (int32_t)s;
    }
}

/* [P2] "Product kernel": B is stored as int8, and a uint8 B is shifted by 128
 * into the int8 range; a raw (already quantised) B keeps scale 1.  [P1] "What
 * works today": the weight column sum is computed once and kept. */
void oracle_pack_b_raw(const void *B, int b_u8, int64_t K, int64_t N, int64_t ldb,
                       int8_t *Q, float *scale, int32_t *colsum) {
    for (int64_t n = 0; n < N; ++n) {
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k) {
            int64_t v = load_i8(B, b_u8, k * ldb + n) - (b_u8 ? 128 : 0);
            Q[k * N + n] = (int8_t)v;
            s += v;
        }
        scale[n] = 1.0f;
        colsum[n] = (int32_t)s;
    }
}

void oracle_quantize_rows_int8(const float *X, int64_t M, int64_t K, int64_t ldx,
                               int8_t *Q, float *scale) {
    int64_t m;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) quantize_vec(X + m * ldx, K, 1, Q + m * K, 1, &scale[m]);
}

/* ---------------------------------------------------------------- q4_1 --- */

/* bf16 is the upper half of an fp32; widening is exact. */
static double bf16_to_f64(uint16_t h) {
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)h << 16;
    return (double)v.f;
}

/* [P4] "Q4NX chunks": q4_1 blocks; [P5] "Round 26": W = q4*scale + zp with
 * per-(row, 32-col) bf16 scales and mins.  A block is 32 consecutive k of
 * one output column n: {bf16 d, bf16 m, 16 code bytes}; code byte j holds
 * element j in its low nibble and element j+16 in its high nibble.
 * q*d + m is exact in fp64 (4 + 8 significant bits). */
static double q4_1_value(const uint8_t *blocks, int64_t K, int64_t k, int64_t n) {
    const uint8_t *blk = blocks + (n * (K / 32) + k / 32) * 20;
    uint16_t d = (uint16_t)(blk[0] | (blk[1] << 8));
    uint16_t mn = (uint16_t)(blk[2] | (blk[3] << 8));
    int j = (int)(k % 32);
    int q = (j < 16) ? (blk[4 + j] & 0x0F) : (blk[4 + j - 16] >> 4);
    return (double)q * bf16_to_f64(d) + bf16_to_f64(mn);
}

void oracle_q4_1_decode(const uint8_t *blocks, int64_t K, int64_t N, double *W) {
    int64_t k;
#pragma omp parallel for schedule(static)
    for (k = 0; k < K; ++k)
        for (int64_t n = 0; n < N; ++n) W[k * N + n] = q4_1_value(blocks, K, k, n);
}

/* Y = X * W with W decoded exactly; fp64 products, summed in k order. */
void oracle_q4_1_matmul(const float *X, int64_t M, int64_t K, int64_t ldx,
                        const uint8_t *blocks, int64_t N, double *Y, int64_t ldy) {
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t k = 0; k < K; ++k)
                acc += (double)X[m * ldx + k] * q4_1_value(blocks, K, k, n);
            Y[m * ldy + n] = acc;
        }
    }
}

void oracle_q4_1_matmul_at(const float *X, int64_t K, int64_t ldx, const uint8_t *blocks,
                           const int64_t *im, const int64_t *in, int64_t count, double *out) {
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += (double)X[im[i] * ldx + k] * q4_1_value(blocks, K, k, in[i]);
        out[i] = acc;
    }
}

/* q4_1 weights against per-row int8 activations ([P1] "The three layers of
 * the pack", item 2: every matmul input quantised per row with amax/127;
 * [P4] "Q4NX chunks": W = q*d + m per block of 32 k).  The block form: per
 * block b of column n the integer dot D = sum_k q*xq and the integer row sum
 * S = sum_k xq are exact; then Y[m,n] = sa[m] * sum_b (d*D + mn*S), in fp64
 * with the blocks in k order. */
void oracle_q4_1_matmul_q8(const int8_t *Xq, const float *sa, int64_t M, int64_t K, int64_t ldq,
                           const uint8_t *blocks, int64_t N, double *Y, int64_t ldy) {
    const int64_t NB = K / 32;
    int64_t n;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t b = 0; b < NB; ++b) {
                const uint8_t *blk = blocks + (n * NB + b) * 20;
                const double d = bf16_to_f64((uint16_t)(blk[0] | (blk[1] << 8)));
                const double mn = bf16_to_f64((uint16_t)(blk[2] | (blk[3] << 8)));
                int64_t D = 0, S = 0;
                for (int j = 0; j < 32; ++j) {
                    const int64_t q = (j < 16) ? (blk[4 + j] & 0x0F) : (blk[4 + j - 16] >> 4);
                    const int64_t x = Xq[m * ldq + b * 32 + j];
                    D += q * x;
                    S += x;
                }
                acc += d * (double)D + mn * (double)S;
            }
            Y[m * ldy + n] = (double)sa[m] * acc;
        }
    }
}

/* [P5] "The bugs that were the work": the per-token expert ids are a strided
 * view (17 sorted experts per token, row stride 17 int32); only the first
 * n_expert_used of each row are used and they must be read through the
 * stride.  [P5] "What's next": gate/up experts read the shared activation
 * form [k, ntokens], i.e. token t's row for every slot (ldx_slot = 0); down
 * experts read a row of their own per (token, slot), the per-expert form
 * [k, n_expert_used, ntokens] (row at t*ldx + s*ldx_slot). */
int oracle_q4_1_matmul_id(const float *X, int64_t T, int64_t K, int64_t ldx, int64_t ldx_slot,
                          const uint8_t *experts, int64_t n_expert, int64_t N,
                          const int32_t *ids, int64_t ids_row_stride, int64_t n_used,
                          double *Y, int64_t ldy_slot, int64_t ldy_token) {
    const int64_t expert_bytes = (K / 32) * N * 20;
    for (int64_t t = 0; t < T; ++t)
        for (int64_t s = 0; s < n_used; ++s) {
            int32_t e = ids[t * ids_row_stride + s];
            if (e < 0 || e >= n_expert) return -1;
        }
    int64_t t;
#pragma omp parallel for schedule(static)
    for (t = 0; t < T; ++t) {
        for (int64_t s = 0; s < n_used; ++s) {
            int32_t e = ids[t * ids_row_stride + s];
            const uint8_t *W = experts + (int64_t)e * expert_bytes;
            for (int64_t n = 0; n < N; ++n) {
                double acc = 0.0;
                for (int64_t k = 0; k < K; ++k)
                    acc += (double)X[t * ldx + s * ldx_slot + k] * q4_1_value(W, K, k, n);
                Y[t * ldy_token + s * ldy_slot + n] = acc;
            }
        }
    }
    return 0;
}

int oracle_q4_1_matmul_id_at(const float *X, int64_t K, int64_t ldx, int64_t ldx_slot,
                             const uint8_t *experts, int64_t n_expert, int64_t N,
                             const int32_t *ids, int64_t ids_row_stride,
                             const int64_t *it, const int64_t *is, const int64_t *in,
                             int64_t count, double *out) {
    const int64_t expert_bytes = (K / 32) * N * 20;
    for (int64_t i = 0; i < count; ++i) {
        int32_t e = ids[it[i] * ids_row_stride + is[i]];
        if (e < 0 || e >= n_expert) return -1;
    }
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i) {
        int32_t e = ids[it[i] * ids_row_stride + is[i]];
        const uint8_t *W = experts + (int64_t)e * expert_bytes;
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k)
            acc += (double)X[it[i] * ldx + is[i] * ldx_slot + k] * q4_1_value(W, K, k, in[i]);
        out[i] = acc;
    }
    return 0;
}
