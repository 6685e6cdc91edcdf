/*
 * oracle.h -- plain CPU oracle for the quantized projection matmul.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library includes, links
 * or calls this code; only the tests, the smoke check and the benchmark's CPU
 * baseline leg do.  The oracle shares no code, header, table or constant with
 * the HIP path.
 *
 * Every routine is the plain definition (integer paths, int64) or the plain
 * step-by-step rule (quantisers, q4_1 decode, fp64 accumulation), written
 * from the web pages it cites, with no blocking, fusion or reordering.
 *
 * Conventions (shared with the public API, restated here on purpose):
 *   A      : M x K, row-major, leading dimension lda (elements)
 *   B      : K x N, row-major, leading dimension ldb (elements); one scale
 *            per output column n
 *   Y      : M x N, row-major
 *   q4_1   : canonical blocks of 20 bytes {bf16 d, bf16 m, 16 code bytes},
 *            stored [N][K/32]; block b of column n covers k = 32b .. 32b+31;
 *            code byte j holds element j (low nibble) and j+16 (high nibble);
 *            the value is W[k][n] = q * d + m.
 */
#ifndef QMM_ORACLE_H
#define QMM_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* 1 if K*255*128 < 2^31, the bound under which the int32 sums of the
 * shifted product cannot overflow ("int8 inference", "Product kernel"). */
int oracle_int8_bound_ok(int64_t K);

/* Y[m][n] = sum_k (A[m][k] - zA) * (B[k][n] - zB), int64, naive.
 * a_u8 / b_u8 select uint8 (1) or int8 (0) element types. */
void oracle_int8_gemm_i64(const void *A, int a_u8, int64_t M, int64_t K, int64_t lda, int32_t zA,
                          const void *B, int b_u8, int64_t N, int64_t ldb, int32_t zB,
                          int64_t *Y, int64_t ldy);

/* Per-axis zero points: zA[M] per activation row, zB[N] per weight column;
 * Y[m,n] = sum_k (A[m,k]-zA[m])(B[k,n]-zB[n]) in int64. */
void oracle_int8_gemm_axis_i64(const void *A, int a_u8, int64_t M, int64_t K, int64_t lda, const int32_t *zA,
                               const void *B, int b_u8, int64_t N, int64_t ldb, const int32_t *zB,
                               int64_t *Y, int64_t ldy);

/* The scalar-zero-point definition at `count` sampled positions (im[i], in[i]). */
void oracle_int8_gemm_at(const void *A, int a_u8, int64_t K, int64_t lda, int32_t zA,
                         const void *B, int b_u8, int64_t ldb, int32_t zB,
                         const int64_t *im, const int64_t *in, int64_t count, int64_t *out);

/* Float epilogue in fp64: y = Y * rs[m] * cs[n] * scale + bias[n].
 * rs, cs, bias may be NULL (1, 1, 0). Y has row stride ldy, out has N. */
void oracle_epilogue_f64(const int64_t *Y, int64_t M, int64_t N, int64_t ldy,
                         const float *rs, const float *cs, float scale, const float *bias,
                         double *out);

/* Requantising epilogue, the exact fp32 chain (one multiply per element,
 * round half to even, output zero point added after rounding):
 *   acc  = Y + bias_i32[n]                        (must fit int32)
 *   mult = fl32(fl32(rs[m] * cs[n]) * scale)
 *   v    = fl32(fl32(acc) * mult)
 *   y    = clamp(rne(v) + zp_out, lo, hi)         lo,hi = -128,127 or 0,255
 * Returns 0, or -1 if some acc does not fit int32. */
int oracle_requant(const int64_t *Y, int64_t M, int64_t N, int64_t ldy,
                   const float *rs, const float *cs, float scale, const int32_t *bias_i32,
                   int32_t zp_out, int out_u8, int32_t *out);

/* Symmetric per-vector int8 quantisation with scale = amax/127:
 * s = fl32(amax / 127); q = clamp(rne(fl32(x / s)), -127, 127); s = 0 and
 * q = 0 when amax = 0.  Applied per column of W (pack) or per row of X. */
void oracle_pack_b_int8(const float *W, int64_t K, int64_t N, int64_t ldw,
                        int8_t *Q /* K x N, ld N */, float *scale /* N */, int32_t *colsum /* N */);
void oracle_pack_b_raw(const void *B, int b_u8, int64_t K, int64_t N, int64_t ldb,
                       int8_t *Q /* K x N, ld N, shifted domain */, float *scale, int32_t *colsum);
void oracle_quantize_rows_int8(const float *X, int64_t M, int64_t K, int64_t ldx,
                               int8_t *Q /* M x K, ld K */, float *scale /* M */);

/* q4_1: decode to fp64 W (K x N, ld N), exact. */
void oracle_q4_1_decode(const uint8_t *blocks, int64_t K, int64_t N, double *W);

/* Y[m][n] = sum_k X[m][k] * (q*d + m) in fp64, sequential over k. */
void oracle_q4_1_matmul(const float *X, int64_t M, int64_t K, int64_t ldx,
                        const uint8_t *blocks, int64_t N, double *Y, int64_t ldy);
void oracle_q4_1_matmul_at(const float *X, int64_t K, int64_t ldx, const uint8_t *blocks,
                           const int64_t *im, const int64_t *in, int64_t count, double *out);

/* q4_1 weights x per-row int8 activations (codes Xq, scales sa):
 * Y[m,n] = sa[m] * sum_b (d[n,b] * sum_{k in b} q*xq + m[n,b] * sum_{k in b} xq),
 * integer block sums exact, the rest fp64. */
void oracle_q4_1_matmul_q8(const int8_t *Xq, const float *sa, int64_t M, int64_t K, int64_t ldq,
                           const uint8_t *blocks, int64_t N, double *Y, int64_t ldy);

/* MUL_MAT_ID: for t < T, s < n_used, e = ids[t*ids_row_stride + s],
 * Y[t][s][:] = x(t,s) * W_e, where the activation row x(t,s) starts at
 * X + t*ldx + s*ldx_slot: ldx_slot = 0 is the shared form (token t's row for
 * every slot), ldx_slot >= K the per-slot form.  Experts are canonical q4_1
 * matrices stored one after another (K/32*N blocks each).  Y element (t,s,n)
 * lives at t*ldy_token + s*ldy_slot + n.
 * Returns 0, or -1 if an id lies outside [0, n_expert). */
int oracle_q4_1_matmul_id(const float *X, int64_t T, int64_t K, int64_t ldx, int64_t ldx_slot,
                          const uint8_t *experts, int64_t n_expert, int64_t N,
                          const int32_t *ids, int64_t ids_row_stride, int64_t n_used,
                          double *Y, int64_t ldy_slot, int64_t ldy_token);
/* Sampled form: output (t[i], s[i], n[i]). */
int oracle_q4_1_matmul_id_at(const float *X, int64_t K, int64_t ldx, int64_t ldx_slot,
                             const uint8_t *experts, int64_t n_expert, int64_t N,
                             const int32_t *ids, int64_t ids_row_stride,
                             const int64_t *it, const int64_t *is, const int64_t *in,
                             int64_t count, double *out);

/* Number of OpenMP threads the oracle runs with. */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
