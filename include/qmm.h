/*
 * qmm.h -- C ABI of the quantized projection matmul library (libqmm.so) for
 * AMD Instinct MI355X (gfx950).
 *
 * The library computes the quantized projection matmul of a decoder LLM:
 *   - an int8 x int8 product with int32 accumulation and the zero-point
 *     correction epilogue, plus optional bias, requantisation or fp32 output;
 *   - per-column int8 weight packing (scale = amax/127) and per-row int8
 *     activation quantisation;
 *   - 4-bit q4_1 block weights (bf16 scale and min per 32 values) decoded
 *     inside the kernels, including the mixture-of-experts form that reads
 *     top-k expert ids through a strided view.
 *
 * Sources (web pages, by title and section):
 *  [P1] "The ONNX pack: weights to Q4NX, matmuls to our kernels, no VitisAI"
 *  [P2] "int8 inference" (onemodel docs), "Product kernel (Int8Gemm)"
 *  [P4] "NPU engine: full ELFs, no xclbin", "Q4NX chunks"
 *  [P5] "Zaya 8B Q4NX on the AMD NPU"
 *
 * Common rules for every entry point:
 *   - Pointers named as device pointers refer to GPU memory owned by the
 *     caller; the library never frees or retains them after the call.
 *   - Matrices are row-major with an explicit leading dimension in elements.
 *   - `stream` is a hipStream_t (NULL = the legacy default stream).  Every
 *     call only enqueues work on it and returns; nothing synchronises unless
 *     stated.
 *   - All arguments are checked on the host before anything is enqueued.  On
 *     an error status nothing is enqueued and no output is written.
 *   - QMM_ERR_UNSUPPORTED means well-formed but not covered (the caller is
 *     expected to fall back, as the pages' execution provider does for a
 *     shape it has no kernel for: [P1] "What the graph gives us").
 *   - Results do not depend on the launch configuration: integer outputs are
 *     exact, and floating-point outputs are bitwise reproducible run to run.
 *   - No call allocates device memory (the one device array the library
 *     owns, q4_1_matmul_id_noalloc's scratch, is part of its code object and
 *     placed by the HIP runtime when it loads the kernels on a GPU).  Results depend
 *     only on the arguments: the only state kept between calls is the
 *     process-wide check-mode flag (qmm_set_check), the per-thread
 *     diagnostics (qmm_last_hip_error, qmm_last_variant) and, for
 *     q4_1_matmul_id_noalloc, one library-owned scratch array per GPU.
 *   - Calls on different streams may run concurrently as long as they do not
 *     share an output or a workspace (and, for q4_1_matmul_id_noalloc, not
 *     on the same GPU).
 *   - Workspaces are scratch: no initial contents are needed, every call
 *     writes what it reads, and a workspace may be reused by any later call
 *     on the same stream.
 */
#ifndef QMM_H
#define QMM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    QMM_OK = 0,
    QMM_ERR_INVALID = 1,     /* null pointer, bad size, ld < width, bad zero point   */
    QMM_ERR_UNSUPPORTED = 2, /* valid but not covered (e.g. q4_1 with K % 32 != 0)   */
    QMM_ERR_WORKSPACE = 3,   /* workspace or packed buffer smaller than required     */
    QMM_ERR_HIP = 4          /* a HIP launch failed; see qmm_last_hip_error()         */
} qmm_status;

typedef enum { QMM_S8 = 0, QMM_U8 = 1 } qmm_i8type;

/* Output selectors for qmm_epilogue.outputs (bitwise OR). */
enum {
    QMM_OUT_I32 = 1, /* corrected int32 accumulator                               */
    QMM_OUT_F32 = 2, /* fp32: Y * row_scale[m] * col_scale[n] * scale + bias_f32[n] */
    QMM_OUT_I8 = 4,  /* requantised int8                                          */
    QMM_OUT_U8 = 8   /* requantised uint8 (exclusive with QMM_OUT_I8)             */
};

/*
 * Epilogue of int8_gemm ([P2] "Product kernel": zero-point correction,
 * optional bias, requantisation or float conversion; [P1] "Why it folds
 * without a new kernel" and "What works today": per-axis scales land in the
 * same epilogue, the output scale folds into one multiply per element, the
 * result rounds half to even and the output zero point is added after
 * rounding).
 *
 * With Y the corrected int32 accumulator (wrapping int32 arithmetic) and
 *   mult = fl32(fl32(rs[m] * cs[n]) * scale)   (rs = row_scale or 1,
 *                                               cs = col_scale or the packed
 *                                               weight's column scales)
 * the outputs are
 *   I32 : y_i32[m*ld_i32 + n] = Y
 *   F32 : y_f32[m*ld_f32 + n] = fl32(Y) * mult + bias_f32[n]      (bias 0 if NULL)
 *   I8/U8: acc = Y + bias_i32[n] (int32);  v = fl32(fl32(acc) * mult);
 *          y_q8[m*ld_q8 + n] = clamp(rne(v) + zp_out, -128..127 or 0..255)
 * Any combination of I32, F32 and one of I8/U8 may be requested at once.
 */
typedef struct {
    uint32_t outputs;
    int32_t *y_i32;          /* device, M x N, used with QMM_OUT_I32          */
    int64_t ld_i32;
    float *y_f32;            /* device, M x N, used with QMM_OUT_F32          */
    int64_t ld_f32;
    void *y_q8;              /* device, M x N int8/uint8, with QMM_OUT_I8/U8  */
    int64_t ld_q8;
    const float *row_scale;  /* device [M] or NULL (= 1)                      */
    const float *col_scale;  /* device [N] or NULL (= packed column scales)   */
    float scale;             /* per-tensor factor (e.g. s_x*s_w/s_y)          */
    const float *bias_f32;   /* device [N] or NULL; F32 output only           */
    const int32_t *bias_i32; /* device [N] or NULL; I8/U8 output only         */
    int32_t zp_out;          /* I8: -128..127, U8: 0..255                     */
} qmm_epilogue;

/* ------------------------------------------------------ int8 weight pack --- */

/* Bytes of a packed int8 weight buffer for a K x N weight. */
size_t qmm_pack_b_int8_bytes(int64_t K, int64_t N);

/*
 * pack_b_int8: [P1] "The three layers of the pack": quantise each weight
 * column to int8 with scale = amax/127 and store the column scales alongside
 * the packed buffer; done once per (tensor, K, N).
 *   W       device fp32 K x N, leading dimension ldw >= N (one column per
 *           output feature n).
 *   packed  device buffer of at least qmm_pack_b_int8_bytes(K, N) bytes,
 *           256-byte aligned.  Receives a 64-byte header, the codes in the
 *           library's tile layout, fp32 scale[N] and int32 colsum[N].
 * Per column: s = fl32(amax/127), q = clamp(rne(fl32(w/s)), -127, 127); an
 * all-zero column gets s = 0 and codes 0; colsum[n] = sum_k q.
 */
qmm_status pack_b_int8(const float *W, int64_t K, int64_t N, int64_t ldw,
                       void *packed, size_t packed_bytes, void *stream);

/*
 * pack_b_int8_raw: pack an already-quantised int8/uint8 weight ([P2]
 * "Product kernel": B is stored as int8 and a uint8 B is shifted by 128).
 * Codes are B (int8) or B - 128 (uint8); scales are 1; colsum is the sum of
 * the shifted codes ([P1] "What works today": the weight column sum is
 * computed once and kept).
 */
qmm_status pack_b_int8_raw(const void *B, qmm_i8type bt, int64_t K, int64_t N, int64_t ldb,
                           void *packed, size_t packed_bytes, void *stream);

/*
 * qmm_packed_b_check: synchronously read the header of a packed buffer and
 * check that it was written by this layout version for this K and N
 * (QMM_ERR_INVALID otherwise).  Optional; int8_gemm does not read the header.
 */
qmm_status qmm_packed_b_check(const void *packed, int64_t K, int64_t N, void *stream);

/*
 * quantize_rows_int8: [P1] "The three layers of the pack", item 2: every
 * matmul input is quantised per row with amax/127.
 *   X  device fp32 M x K (ldx >= K);  Xq device int8 M x K (ldq >= K);
 *   row_scale device fp32 [M].  Same rule as pack_b_int8, along rows.
 */
qmm_status quantize_rows_int8(const float *X, int64_t M, int64_t K, int64_t ldx,
                              int8_t *Xq, int64_t ldq, float *row_scale, void *stream);

/* ----------------------------------------------------------- int8 GEMM --- */

/* Workspace bytes int8_gemm needs for an M x K x N product (may be 0). */
size_t qmm_int8_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N);

/*
 * int8_gemm: [P2] "Product kernel (Int8Gemm)":
 *   S[m,n] = sum_k A'[m,k] * B'[k,n]        (int32; primes = shifted domain,
 *                                            A' = A - 128 for uint8 A)
 *   Y[m,n] = S - zA'*colSum[n] - zB'*(rowSum[m] - K*zA')
 * which equals sum_k (A[m,k]-zA)(B[k,n]-zB) exactly whenever that value fits
 * in int32 (always for K <= 33025), then the epilogue above.
 *   A        device, M x K int8 or uint8 (at), leading dimension lda >= K.
 *   zA       activation zero point in at's range.
 *   packedB  buffer written by pack_b_int8 / pack_b_int8_raw for this K, N.
 *   bt       element type the packed weight was given in (QMM_S8 for
 *            pack_b_int8); zB is in that type's range.
 *   workspace  device scratch of qmm_int8_gemm_workspace_bytes(M,K,N) bytes
 *            (256-byte aligned, any contents); NULL when
 *            that size is 0, which it is for every current kernel variant.
 * K must satisfy K*255*128 < 2^31 ([P2]: the sums cannot overflow below that
 * bound), else QMM_ERR_UNSUPPORTED.  M = 0 or N = 0 is a no-op.
 */
qmm_status int8_gemm(const void *A, qmm_i8type at, int64_t M, int64_t K, int64_t lda, int32_t zA,
                     const void *packedB, qmm_i8type bt, int64_t N, int32_t zB,
                     const qmm_epilogue *ep, void *workspace, size_t workspace_bytes,
                     void *stream);

/*
 * int8_gemm_per_axis: int8_gemm with a zero point per activation row and one
 * per weight column ([P1] "What works today": asymmetric zero points per
 * axis, on the same axes as the per-axis scales, folded into the epilogue):
 *   Y[m,n] = sum_k (A[m,k] - zA_row[m]) * (B[k,n] - zB_col[n])
 *          = S - zA'[m]*colSum[n] - zB'[n]*(rowSum[m] - K*zA'[m])  (int32)
 * then the same epilogue: per-axis scales come through ep->row_scale (s_x[m])
 * and ep->col_scale (s_w[n]), and the QDQ group "int8 in, int8 out" is the
 * I8/U8 output with ep->scale = 1/s_y and ep->zp_out = zp_y.
 *   zA_row   device int32 [M], each in at's range, or NULL (all 0)
 *   zB_col   device int32 [N], each in bt's range, or NULL (all 0)
 * The ranges are a precondition (device data, not checked on the host).
 * Every other argument, the bound on K and the error codes are int8_gemm's.
 */
qmm_status int8_gemm_per_axis(const void *A, qmm_i8type at, int64_t M, int64_t K, int64_t lda,
                              const int32_t *zA_row, const void *packedB, qmm_i8type bt, int64_t N,
                              const int32_t *zB_col, const qmm_epilogue *ep, void *workspace,
                              size_t workspace_bytes, void *stream);

/* Workspace bytes int8_gemm_dynamic needs (0 when the quantisation is fused,
 * see int8_gemm_dynamic). */
size_t qmm_int8_gemm_dynamic_workspace_bytes(int64_t M, int64_t K, int64_t N);

/*
 * int8_gemm_dynamic: the float MatMul route of [P1] "The three layers of the
 * pack" in one call: fp32 activations X (M x K, ldx >= K) are quantised per
 * row with amax/127 (the quantize_rows_int8 rule) and multiplied with a
 * weight packed by pack_b_int8 (zA = zB = 0); the epilogue uses the computed
 * row scales (ep->row_scale must be NULL).  Results are bit-identical to
 * quantize_rows_int8 followed by int8_gemm.  The quantisation runs inside
 * the product kernel (one launch) when K <= 4096 and the rows, cut into
 * G = 1, 2, 4 or 8 groups of R = ceil(M / G), give R' <= 16 and
 * R' * K <= 16384, R' = R rounded up to a power of 2 (G is the smallest one
 * with R' <= 8 if there is one, else the smallest one with R' <= 16); each
 * group is then a grid row that reads the weight once.  Otherwise the two
 * kernels run in turn.  Xq (M x K int8, ldq >= K) and row_scale ([M] fp32)
 * optionally receive the quantised rows and their scales; pass NULL to skip
 * them (the two-kernel form then keeps them in the workspace).
 */
qmm_status int8_gemm_dynamic(const float *X, int64_t M, int64_t K, int64_t ldx,
                             const void *packedB, int64_t N, const qmm_epilogue *ep,
                             int8_t *Xq, int64_t ldq, float *row_scale,
                             void *workspace, size_t workspace_bytes, void *stream);

/*
 * int8_gemm_dynamic_grouped: int8_gemm_dynamic over several weights that
 * read the same activations (a decoder layer's q, k and v projections, or
 * its gate and up projections), in one launch: [P1] "What works today, and
 * what does not": a decode-side win needs fewer, longer launches.  X (fp32
 * M x K, ldx >= K) is quantised per row with amax/127 once per row group
 * and multiplied with every item's weight; item i writes
 *   items[i].y_f32[m*ld_f32 + n] = fl32(Y_i) * fl32(fl32(rs[m]*cs_i[n])*scale)
 *                                  + bias_f32[n]          (bias 0 if NULL)
 * with Y_i the int32 product with weight i, rs the computed row scales and
 * cs_i the weight's packed column scales: bit for bit what int8_gemm_dynamic
 * with an F32-only epilogue (row_scale NULL, col_scale NULL, that scale and
 * bias) gives for each weight alone.
 *   items     host array of n_items (1..QMM_MAX_GROUP_ITEMS) descriptors; each
 *             packedB was written by pack_b_int8 for this K and its N; items
 *             with N = 0 are skipped.
 *   workspace device scratch of qmm_int8_gemm_dynamic_grouped_workspace_bytes
 *             (M, K) bytes (0, workspace may be NULL, whenever the rows cut
 *             into the row groups of int8_gemm_dynamic's one-launch form;
 *             otherwise the quantised rows and their scales, the rows
 *             quantised once and each item multiplied in a launch of its own).
 * Errors as int8_gemm_dynamic.
 */
#define QMM_MAX_GROUP_ITEMS 4
typedef struct {
    const void *packedB;     /* device, pack_b_int8 buffer for K x N           */
    int64_t N;
    float *y_f32;            /* device, M x N fp32 output                      */
    int64_t ld_f32;
    const float *bias_f32;   /* device [N] or NULL                             */
} qmm_dynamic_item;
size_t qmm_int8_gemm_dynamic_grouped_workspace_bytes(int64_t M, int64_t K);
qmm_status int8_gemm_dynamic_grouped(const float *X, int64_t M, int64_t K, int64_t ldx,
                                     const qmm_dynamic_item *items, int64_t n_items, float scale,
                                     void *workspace, size_t workspace_bytes, void *stream);

/* ---------------------------------------------------------------- q4_1 --- */

/*
 * Canonical q4_1 block ([P4] "Q4NX chunks"; [P5] "Round 26": W = q*scale +
 * min with bf16 scale and min per (row, 32-col) block): 32 consecutive k of
 * one output column n, 20 bytes:
 *   bytes 0-1  d  (bf16, little endian), bytes 2-3  m (bf16),
 *   bytes 4-19 codes: byte j holds element j (low nibble) and j+16 (high).
 * value(k) = q(k) * d + m.  A K x N weight is the array blocks[N][K/32].
 */
#define QMM_Q4_1_BLOCK_BYTES 20

/* Bytes of the device layout of a K x N q4_1 weight. */
size_t qmm_q4_1_packed_bytes(int64_t K, int64_t N);

/*
 * q4_1_repack: copy canonical blocks (device, [N][K/32] x 20 bytes) into the
 * library's tile layout (layout only, no arithmetic; [P5] "Milestones": one
 * raw blob plus a tile-major layout read by the kernel).  K % 32 != 0 gives
 * QMM_ERR_UNSUPPORTED.
 */
qmm_status q4_1_repack(const void *blocks, int64_t K, int64_t N,
                       void *packed, size_t packed_bytes, void *stream);

/* Workspace bytes q4_1_matmul needs for M rows. */
size_t qmm_q4_1_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N);

/*
 * q4_1_matmul: Y[m,n] = sum_k X[m,k] * (q[k,n]*d + m) with X fp32 (M x K,
 * ldx >= K), the weight in the layout written by q4_1_repack, Y fp32 (M x N,
 * ldy >= N).  Codes are decoded inside the kernel and kept exact; the
 * relative Frobenius error against exact arithmetic is below 1e-5.
 * workspace: device, >= qmm_q4_1_matmul_workspace_bytes(M,K,N), 256-byte
 * aligned, any contents (the k-split partial sums).  That size is
 * 0 for M <= 4, and for M <= 16 with K <= 1024 (one launch covers the whole
 * k range: no partial sums); workspace may then be NULL.
 */
qmm_status q4_1_matmul(const float *X, int64_t M, int64_t K, int64_t ldx,
                       const void *Wpacked, int64_t N, float *Y, int64_t ldy,
                       void *workspace, size_t workspace_bytes, void *stream);

/*
 * q4_1_matmul_q8: q4_1 weights against per-row int8 activations (the codes
 * and scales quantize_rows_int8 writes: [P1] "The three layers of the pack",
 * item 2; [P4] "Q4NX chunks" for W = q*d + m):
 *   Y[m,n] = row_scale[m] * sum_b ( d[n,b] * sum_{k in b} q[n,k]*Xq[m,k]
 *                                 + m[n,b] * sum_{k in b} Xq[m,k] )
 * Each block dot and row sum is exact (int32 MFMA); the combination is fp32.
 * It trades the fp32 activations of q4_1_matmul for int8 ones.
 *   Xq         device int8 M x K (ldq >= K); row_scale device fp32 [M]
 *   Wpacked    written by q4_1_repack for this K, N;  Y device fp32 M x N
 * K % 32 != 0 is QMM_ERR_UNSUPPORTED.  Rows run 16 per launch; no workspace.
 */
qmm_status q4_1_matmul_q8(const int8_t *Xq, const float *row_scale, int64_t M, int64_t K, int64_t ldq,
                          const void *Wpacked, int64_t N, float *Y, int64_t ldy, void *stream);

/* Workspace bytes q4_1_matmul_id needs. */
size_t qmm_q4_1_matmul_id_workspace_bytes(int64_t n_tokens, int64_t n_used, int64_t n_expert,
                                          int64_t K, int64_t N);

/*
 * q4_1_matmul_id: MUL_MAT_ID over stacked q4_1 experts ([P5] "The bugs that
 * were the work": the ids are a strided view and must be read through the
 * stride; "What's next": the shared activation form [k, ntokens]).
 * For t < n_tokens and s < n_used:
 *   e = ids[t*ids_row_stride + s];   Y[t*ldy_token + s*ldy_slot + n] = X[t] . W_e[:, n]
 *   X         device fp32 n_tokens x K (ldx >= K)
 *   Wexperts  device, n_expert weights in the q4_1_repack layout, expert e
 *             at byte offset e*expert_stride (>= qmm_q4_1_packed_bytes(K,N))
 *   ids       device int32, row stride ids_row_stride >= n_used; every used
 *             id must lie in [0, n_expert) (a precondition: pairs with other
 *             ids are skipped, and reported in check mode, qmm_set_check)
 * Tokens routed to each expert are grouped on the device (counting sort) and
 * run in one grouped launch.  workspace: >= qmm_q4_1_matmul_id_workspace_bytes,
 * 256-byte aligned, any contents (routing tables and split activations).
 */
qmm_status q4_1_matmul_id(const float *X, int64_t n_tokens, int64_t K, int64_t ldx,
                          const void *Wexperts, int64_t n_expert, int64_t N, size_t expert_stride,
                          const int32_t *ids, int64_t ids_row_stride, int64_t n_used,
                          float *Y, int64_t ldy_slot, int64_t ldy_token,
                          void *workspace, size_t workspace_bytes, void *stream);

/* Workspace bytes q4_1_matmul_id_per_slot needs. */
size_t qmm_q4_1_matmul_id_per_slot_workspace_bytes(int64_t n_tokens, int64_t n_used, int64_t n_expert,
                                                   int64_t K, int64_t N);

/*
 * q4_1_matmul_id_per_slot: MUL_MAT_ID whose activations hold a row of their
 * own per (token, slot), the per-expert form [k, n_expert_used, ntokens] the
 * down experts read ([P5] "What's next": reading token t's shared row for
 * every slot made every expert compute with the first slot's activation).
 * For t < n_tokens and s < n_used:
 *   e = ids[t*ids_row_stride + s];
 *   Y[t*ldy_token + s*ldy_slot + n] = X[t*ldx_token + s*ldx_slot + :] . W_e[:, n]
 *   X         device fp32, ldx_slot >= K, ldx_token >= n_used*ldx_slot
 * Every other argument, the error codes and the workspace rule are those of
 * q4_1_matmul_id; the workspace grows with n_tokens*n_used activation rows
 * instead of n_tokens.
 */
qmm_status q4_1_matmul_id_per_slot(const float *X, int64_t n_tokens, int64_t K, int64_t ldx_slot,
                                   int64_t ldx_token, const void *Wexperts, int64_t n_expert, int64_t N,
                                   size_t expert_stride, const int32_t *ids, int64_t ids_row_stride,
                                   int64_t n_used, float *Y, int64_t ldy_slot, int64_t ldy_token,
                                   void *workspace, size_t workspace_bytes, void *stream);

/*
 * q4_1_matmul_id_noalloc: q4_1_matmul_id for callers that cannot allocate
 * device memory or pass a workspace (code under HIP graph capture, serving
 * loops, harnesses that forbid allocation).  Same arguments, results (the
 * same kernels, bit for bit), error codes and check mode as q4_1_matmul_id,
 * without the workspace: the routing tables and split activations live in
 * a library-owned device array of QMM_NOALLOC_SCRATCH_BYTES per GPU, created
 * with the library's code object on each GPU it runs on and held until the
 * process ends.  The call itself allocates nothing and never synchronises
 * (outside check mode).
 *   - A call whose workspace (qmm_q4_1_matmul_id_workspace_bytes) exceeds
 *     QMM_NOALLOC_SCRATCH_BYTES returns QMM_ERR_WORKSPACE before anything
 *     is enqueued (16 MiB covers e.g. 512 tokens x top-8 over 128 experts
 *     at K = 2048, which needs about 4.5 MiB).
 *   - Every call on one GPU shares that GPU's array, and nothing in it needs
 *     to start at any value (each call writes everything it reads): calls
 *     that overlap in time on one GPU (different streams, or different host
 *     threads) race and may return wrong results; serialise them.
 *   - The GPU is the one `stream` belongs to (the current device for NULL).
 */
#define QMM_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
qmm_status q4_1_matmul_id_noalloc(const float *X, int64_t n_tokens, int64_t K, int64_t ldx,
                                  const void *Wexperts, int64_t n_expert, int64_t N, size_t expert_stride,
                                  const int32_t *ids, int64_t ids_row_stride, int64_t n_used,
                                  float *Y, int64_t ldy_slot, int64_t ldy_token, void *stream);

/* ------------------------------------------------------------- helpers --- */

const char *qmm_status_string(qmm_status s);
/* hipError_t of the last failed HIP call on this thread (0 if none). */
int qmm_last_hip_error(void);
/* Name of the kernel variant the last call on this thread launched
 * (diagnostics; "" before the first call).  With QMM_TRACE=1 in the
 * environment when the library loads, every call also prints its variant
 * (and the int8 products their launch plan) to stderr. */
const char *qmm_last_variant(void);

/*
 * Check mode, a debug aid (off by default; QMM_CHECK=1 in the environment
 * turns it on when the library loads).  While on, calls that can verify
 * device data do so and synchronise the stream: int8_gemm and
 * int8_gemm_per_axis read the packed weight's header (qmm_packed_b_check)
 * and return QMM_ERR_INVALID before launching if it does not match K and N;
 * q4_1_matmul_id and q4_1_matmul_id_per_slot return QMM_ERR_INVALID after the
 * call if an expert id lay outside [0, n_expert) (those pairs' outputs are
 * left unwritten, every other output is written).  The flag is process-wide.
 */
void qmm_set_check(int on);
int qmm_check_enabled(void);

#ifdef __cplusplus
}
#endif
#endif /* QMM_H */
