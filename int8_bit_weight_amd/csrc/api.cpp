// api.cpp -- the C ABI of libqmm.so: argument checks, launch planning and
// dispatch to the HIP kernels.  Everything is checked before anything is
// enqueued; on an error status nothing runs and no output is touched.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>

#include "qmm.h"
#include "qmm_internal.h"

namespace {

thread_local int g_last_hip_error = 0;
thread_local const char *g_last_variant = "";

qmm_status hip_status(hipError_t e) {
    if (e == hipSuccess) return QMM_OK;
    g_last_hip_error = (int)e;
    return QMM_ERR_HIP;
}

int env_int(const char *name, int dflt) {
    const char *v = std::getenv(name);
    if (!v || !*v) return dflt;
    return std::atoi(v);
}

bool trace_on() {
    static int t = env_int("QMM_TRACE", 0);
    return t != 0;
}

}  // namespace

namespace qmm {

// Check mode (QMM_CHECK=1 at load, or qmm_set_check): calls that can verify
// device data do so synchronously.
int g_check = env_int("QMM_CHECK", 0);

qmm_status record_status(hipError_t e, const char *variant) {
    g_last_variant = variant;
    if (trace_on()) fprintf(stderr, "qmm %s\n", variant);
    return hip_status(e);
}

// Decode (M <= 32): one workgroup per 16-column strip of the weight, with
// WAVES wavefronts (4, 8 or 16) splitting its k tiles and TPW (1, 2 or 4)
// tiles per wavefront per round, chosen so one round covers as much of K as
// possible.  With many strips (an output projection onto a vocabulary) and
// A small enough to sit in LDS, one wavefront per strip over the whole k
// range instead (the wide decode).  Prefill (M > 32): 256 x 128 MFMA tiles.
// Integer results are exact whatever the choice, and the fp32 epilogue is
// one per-element formula, so no output bit depends on it.  The wide decode
// starts at 1024 strips (measured: on the 0.6B projections, 64-384 strips,
// it was 1.2-2.4x slower per call; on 9496 strips 1.7x faster at M = 1 and
// 3.8x at M = 16).  QMM_WIDE_MIN_STRIPS overrides the threshold (tuning).
static int64_t wide_min_strips() {
    static int64_t v = env_int("QMM_WIDE_MIN_STRIPS", (int)kWideMinStrips);
    return v;
}
static bool use_wide(int64_t M, int64_t K, int64_t N) {
    const PackedBLayout L = packed_b_layout(K, N);
    const int mt = M <= 16 ? 1 : 2;
    return M <= 32 && L.NS >= wide_min_strips() && L.KT * mt <= kWideMaxTiles;
}

Int8Plan plan_int8_gemm(int64_t M, int64_t K, int64_t N, bool allow_wide) {
    Int8Plan pl{};
    const PackedBLayout L = packed_b_layout(K, N);
    if (allow_wide && use_wide(M, K, N)) {
        pl.variant = 2;
        pl.mt = M <= 16 ? 1 : 2;
        pl.grid = ceil_div(L.NS, kWideWaves);
    } else if (M <= 32) {
        pl.variant = 0;
        pl.mt = M <= 16 ? 1 : 2;
        // one round of 16 wavefronts covers K <= 4096 (up to 4 tiles each);
        // (waves, tiles per wave) is one of 4x1, 8x1, 16x1, 16x2, 16x4
        const int waves = L.KT <= 4 ? 4 : (L.KT <= 8 ? 8 : 16);
        int tpw = (int)ceil_div(L.KT, waves);
        tpw = tpw <= 1 ? 1 : (tpw <= 2 ? 2 : 4);
        pl.waves = waves;
        pl.tpw = tpw;
        pl.grid = L.NS;
    } else {
        pl.variant = 1;
        pl.grid = ceil_div(L.NS, 8) * ceil_div(M, 256);
    }
    return pl;
}

}  // namespace qmm

using namespace qmm;

extern "C" {

const char *qmm_status_string(qmm_status s) {
    switch (s) {
        case QMM_OK: return "ok";
        case QMM_ERR_INVALID: return "invalid argument";
        case QMM_ERR_UNSUPPORTED: return "unsupported case";
        case QMM_ERR_WORKSPACE: return "workspace or buffer too small";
        case QMM_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

int qmm_last_hip_error(void) { return g_last_hip_error; }
const char *qmm_last_variant(void) { return g_last_variant; }

void qmm_set_check(int on) { qmm::g_check = on ? 1 : 0; }
int qmm_check_enabled(void) { return qmm::g_check; }

size_t qmm_pack_b_int8_bytes(int64_t K, int64_t N) {
    if (K < 0 || N < 0) return 0;
    return (size_t)packed_b_layout(K, N).total;
}

static bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

static bool k_in_bound(int64_t K) { return K * 255 * 128 < ((int64_t)1 << 31); }

qmm_status pack_b_int8(const float *W, int64_t K, int64_t N, int64_t ldw, void *packed,
                       size_t packed_bytes, void *stream) {
    if (K <= 0 || N <= 0 || ldw < N || !W || !packed || !aligned(packed, 256) || !aligned(W, 4))
        return QMM_ERR_INVALID;
    if (K > INT32_MAX / 2 || N > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
    const PackedBLayout L = packed_b_layout(K, N);
    if (packed_bytes < (size_t)L.total) return QMM_ERR_WORKSPACE;
    g_last_variant = "pack_b_f32";
    return hip_status(launch_pack_b_f32(W, ldw, L, packed, (hipStream_t)stream));
}

qmm_status pack_b_int8_raw(const void *B, qmm_i8type bt, int64_t K, int64_t N, int64_t ldb,
                           void *packed, size_t packed_bytes, void *stream) {
    if (K <= 0 || N <= 0 || ldb < N || !B || !packed || !aligned(packed, 256) ||
        (bt != QMM_S8 && bt != QMM_U8))
        return QMM_ERR_INVALID;
    if (K > INT32_MAX / 2 || N > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
    const PackedBLayout L = packed_b_layout(K, N);
    if (packed_bytes < (size_t)L.total) return QMM_ERR_WORKSPACE;
    g_last_variant = "pack_b_raw";
    return hip_status(launch_pack_b_raw(B, bt == QMM_U8, ldb, L, packed, (hipStream_t)stream));
}

qmm_status qmm_packed_b_check(const void *packed, int64_t K, int64_t N, void *stream) {
    if (!packed || K <= 0 || N <= 0) return QMM_ERR_INVALID;
    PackedHeader h;
    hipError_t e = hipMemcpyAsync(&h, packed, sizeof(h), hipMemcpyDeviceToHost, (hipStream_t)stream);
    if (e == hipSuccess) e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_status(e);
    const PackedBLayout L = packed_b_layout(K, N);
    if (h.magic != kPackMagic || h.version != kPackVersion || h.K != K || h.N != N || h.Kp != L.Kp ||
        h.Np != L.Np || h.scale_off != L.scale_off || h.colsum_off != L.colsum_off || h.kind > kPackRawU8)
        return QMM_ERR_INVALID;
    return QMM_OK;
}

qmm_status quantize_rows_int8(const float *X, int64_t M, int64_t K, int64_t ldx, int8_t *Xq,
                              int64_t ldq, float *row_scale, void *stream) {
    if (M < 0 || K <= 0 || ldx < K || ldq < K) return QMM_ERR_INVALID;
    if (M == 0) return QMM_OK;
    if (!X || !Xq || !row_scale || !aligned(X, 4) || !aligned(row_scale, 4)) return QMM_ERR_INVALID;
    if (M > INT32_MAX || K > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
    g_last_variant = "quantize_rows";
    return hip_status(launch_quantize_rows(X, M, K, ldx, Xq, ldq, row_scale, (hipStream_t)stream));
}

size_t qmm_int8_gemm_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K <= 0 || N <= 0) return 0;
    return (size_t)plan_int8_gemm(M, K, N).ws_bytes;
}

// Output selection, leading dimensions and zero point (no pointer checks).
static qmm_status check_epilogue(const qmm_epilogue *ep, int64_t N) {
    const uint32_t outs = ep->outputs;
    if (outs == 0 || (outs & ~15u) || ((outs & QMM_OUT_I8) && (outs & QMM_OUT_U8))) return QMM_ERR_INVALID;
    if ((outs & QMM_OUT_I32) && ep->ld_i32 < N) return QMM_ERR_INVALID;
    if ((outs & QMM_OUT_F32) && ep->ld_f32 < N) return QMM_ERR_INVALID;
    if ((outs & (QMM_OUT_I8 | QMM_OUT_U8))) {
        if (ep->ld_q8 < N) return QMM_ERR_INVALID;
        const int32_t lo = (outs & QMM_OUT_U8) ? 0 : -128;
        if (ep->zp_out < lo || ep->zp_out > lo + 255) return QMM_ERR_INVALID;
    }
    return QMM_OK;
}

// Output pointers of a non-empty product.
static qmm_status check_epilogue_ptrs(const qmm_epilogue *ep) {
    const uint32_t outs = ep->outputs;
    if ((outs & QMM_OUT_I32) && (!ep->y_i32 || !aligned(ep->y_i32, 4))) return QMM_ERR_INVALID;
    if ((outs & QMM_OUT_F32) && (!ep->y_f32 || !aligned(ep->y_f32, 4))) return QMM_ERR_INVALID;
    if ((outs & (QMM_OUT_I8 | QMM_OUT_U8)) && !ep->y_q8) return QMM_ERR_INVALID;
    return QMM_OK;
}

static void fill_params(Int8GemmParams &p, int64_t M, int64_t K, int64_t N, const void *packedB,
                        const qmm_epilogue *ep) {
    const PackedBLayout L = packed_b_layout(K, N);
    const int8_t *base = (const int8_t *)packedB;
    p.M = (int)M;
    p.K = (int)K;
    p.N = (int)N;
    p.codes = base + L.codes_off;
    p.colsum = (const int32_t *)(base + L.colsum_off);
    p.KT = (int)L.KT;
    p.NS = (int)L.NS;
    p.outputs = ep->outputs;
    p.y_i32 = ep->y_i32;
    p.ld_i32 = ep->ld_i32;
    p.y_f32 = ep->y_f32;
    p.ld_f32 = ep->ld_f32;
    p.y_q8 = (int8_t *)ep->y_q8;
    p.ld_q8 = ep->ld_q8;
    p.q8_u8 = (ep->outputs & QMM_OUT_U8) != 0;
    p.row_scale = ep->row_scale;
    p.col_scale = ep->col_scale ? ep->col_scale : (const float *)(base + L.scale_off);
    p.scale = ep->scale;
    p.bias_f32 = ep->bias_f32;
    p.bias_i32 = ep->bias_i32;
    p.zp_out = ep->zp_out;
}

static void trace_gemm(const char *fn, const char *variant, int64_t M, int64_t K, int64_t N, const Int8Plan &plan) {
    if (trace_on())
        fprintf(stderr, "qmm %s variant=%s M=%lld K=%lld N=%lld grid=%lld waves=%d tpw=%d spw=%d\n", fn, variant,
                (long long)M, (long long)K, (long long)N, (long long)plan.grid, plan.waves, plan.tpw, plan.spw);
}

// int8_gemm and int8_gemm_per_axis: scalar zero points zA, zB, or one per
// row of A (za_row) and one per column of B (zb_col), device vectors in the
// caller's domain (a precondition, like the MoE ids: in the type's range).
static qmm_status gemm_call(const void *A, qmm_i8type at, int64_t M, int64_t K, int64_t lda, int32_t zA,
                            const int32_t *za_row, const void *packedB, qmm_i8type bt, int64_t N, int32_t zB,
                            const int32_t *zb_col, const qmm_epilogue *ep, void *workspace, size_t workspace_bytes,
                            void *stream, const char *fn) {
    if (M < 0 || N < 0 || K <= 0 || !ep || (at != QMM_S8 && at != QMM_U8) ||
        (bt != QMM_S8 && bt != QMM_U8))
        return QMM_ERR_INVALID;
    if (lda < K) return QMM_ERR_INVALID;
    const int32_t za_lo = at == QMM_U8 ? 0 : -128, zb_lo = bt == QMM_U8 ? 0 : -128;
    if (zA < za_lo || zA > za_lo + 255 || zB < zb_lo || zB > zb_lo + 255) return QMM_ERR_INVALID;
    qmm_status st = check_epilogue(ep, N);
    if (st != QMM_OK) return st;
    if (!k_in_bound(K) || M > INT32_MAX || N > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return QMM_OK;
    if (!A || !packedB || !aligned(packedB, 256) || check_epilogue_ptrs(ep) != QMM_OK) return QMM_ERR_INVALID;
    if ((za_row && !aligned(za_row, 4)) || (zb_col && !aligned(zb_col, 4))) return QMM_ERR_INVALID;
    if (g_check && qmm_packed_b_check(packedB, K, N, stream) != QMM_OK) return QMM_ERR_INVALID;
    const Int8Plan plan = plan_int8_gemm(M, K, N);
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < (size_t)plan.ws_bytes || !aligned(workspace, 256)))
        return QMM_ERR_WORKSPACE;

    Int8GemmParams p{};
    fill_params(p, M, K, N, packedB, ep);
    p.A = (const int8_t *)A;
    p.lda = lda;
    p.a_u8 = at == QMM_U8;
    p.a_vec = aligned(A, 16) && (lda % 16 == 0);
    p.zAs = zA - (at == QMM_U8 ? 128 : 0);
    p.zBs = zB - (bt == QMM_U8 ? 128 : 0);
    p.za_row = za_row;
    p.zb_col = zb_col;
    p.za_off = at == QMM_U8 ? 128 : 0;
    p.zb_off = bt == QMM_U8 ? 128 : 0;
    const char *variant = "";
    st = hip_status(launch_int8_gemm(plan, p, (hipStream_t)stream, &variant));
    g_last_variant = variant;
    trace_gemm(fn, variant, M, K, N, plan);
    return st;
}

qmm_status int8_gemm(const void *A, qmm_i8type at, int64_t M, int64_t K, int64_t lda, int32_t zA,
                     const void *packedB, qmm_i8type bt, int64_t N, int32_t zB,
                     const qmm_epilogue *ep, void *workspace, size_t workspace_bytes,
                     void *stream) {
    return gemm_call(A, at, M, K, lda, zA, nullptr, packedB, bt, N, zB, nullptr, ep, workspace, workspace_bytes,
                     stream, "int8_gemm");
}

qmm_status int8_gemm_per_axis(const void *A, qmm_i8type at, int64_t M, int64_t K, int64_t lda,
                              const int32_t *zA_row, const void *packedB, qmm_i8type bt, int64_t N,
                              const int32_t *zB_col, const qmm_epilogue *ep, void *workspace,
                              size_t workspace_bytes, void *stream) {
    // a NULL vector means zero points of 0 in the caller's domain: the scalar
    // 0 stands in for it (in range for both types; for a uint8 operand it is
    // -128 in the shifted domain, so the correction still runs)
    return gemm_call(A, at, M, K, lda, 0, zA_row, packedB, bt, N, 0, zB_col, ep, workspace, workspace_bytes,
                     stream, "int8_gemm_per_axis");
}

// The fused form quantises the activations inside the product: every
// workgroup quantises the rows it multiplies.  It is taken while
// E * K <= 16384 and K <= 4096 for some split of the rows into 1, 2, 4 or 8
// row groups (E = rows per group rounded up to a power of two, at most 16):
// then one workgroup keeps its rows' values in registers from the row
// maximum to the codes.  Beyond that the rows are quantised by a launch of
// their own.
static bool dynamic_fusable(int64_t M, int64_t K) {
    if (K > 4096) return false;
    for (int g : {1, 2, 4, 8}) {
        const int64_t r = (M + g - 1) / g;
        int64_t e = 1;
        while (e < r) e <<= 1;
        if (e <= 16 && e * K <= 16384) return true;
    }
    return false;
}
// Calls the wide decode takes (many columns) quantise in a launch of their
// own: there the weight bytes per workgroup are few next to a quantisation in
// every workgroup.
// The wide decode (>= 1024 strips) quantises inside while the rows, rounded
// up to a power of two, times K stay within 16384 values (at most 32 per
// thread of its 512) and X allows aligned 16-byte loads.
static bool dynamic_wide_fused(int64_t M, int64_t K, int64_t N, const float *X, int64_t ldx) {
    int64_t mp = 1;
    while (mp < M) mp <<= 1;
    return use_wide(M, K, N) && mp * K <= 16384 && K % 4 == 0 && aligned(X, 16) && ldx % 4 == 0;
}

static bool dynamic_fused(int64_t M, int64_t K, int64_t N) {
    return dynamic_fusable(M, K) && !use_wide(M, K, N);
}

// Shape of the fused launch: rows per row group and 16-column strips per
// workgroup (S = 1, 2, 4; the S strips share one quantisation of the rows).
// A workgroup reads rows * K * 4 bytes of activations (from L2) and
// S * K * 16 bytes of weights; the call costs about rounds * (those bytes),
// rounds = ceil(workgroups / 256 CUs).  The split with the fewest such bytes
// is taken, fewer rows per group on a tie (less quantisation per
// workgroup).  On MI355X this picked the fastest of all splits for every
// Qwen3-0.6B projection group at M = 1, 16 and 32, with workgroups of 16
// wavefronts and of 8 (the grouped q/k/v call at M = 32: 4 groups of 8 rows,
// 4 strips per workgroup, 5.3 us with 8 wavefronts against 9.7 us for one
// strip per 16-wavefront workgroup; counting 512 workgroups per round, as
// two 8-wavefront workgroups fit a CU, picked slower splits in 8 of 12
// cases).
struct DynShape {
    int64_t rows;  // rows per group (= M: one group)
    int spw;       // strips per workgroup
    int waves;     // wavefronts per workgroup
};
static DynShape dynamic_shape(int64_t M, int64_t K, int64_t NS) {
    constexpr int64_t kCUs = 256;
    DynShape best{M, 1, 8};
    int64_t best_cost = INT64_MAX, best_e = INT64_MAX;
    for (int g : {1, 2, 4, 8}) {
        const int64_t r = (M + g - 1) / g;
        int64_t e = 1;
        while (e < r) e <<= 1;
        if (e > 16 || e * K > 16384) continue;
        const int64_t groups = (M + r - 1) / r;
        for (int spw : {1, 2, 4}) {
            const int64_t wgs = ceil_div(NS, spw) * groups;
            const int64_t cost = ceil_div(wgs, kCUs) * (r * K * 4 + spw * K * 16);
            if (cost < best_cost || (cost == best_cost && e < best_e)) {
                best_cost = cost;
                best_e = e;
                best = DynShape{r, spw, 8};
            }
        }
    }
    // 8 wavefronts per workgroup, 4 where K <= 1024, S <= 2 and at least 192
    // workgroups run (a sweep of 2, 4, 8 and 16 over the Qwen3-0.6B groups:
    // 4 won exactly those cases, by 0.2-0.5 us, and lost the others) and a
    // lane's E * TPQ activations (TPQ = k tiles per wavefront, a power of
    // two >= KT / 4) stay within 32
    const int64_t wgs = ceil_div(NS, best.spw) * ceil_div(M, best.rows);
    int64_t e = 1, tpq = 1;
    while (e < best.rows) e <<= 1;
    while (tpq * 4 < ceil_div(K, 64)) tpq <<= 1;
    if (K <= 1024 && best.spw <= 2 && wgs >= 192 && e * tpq <= 32) best.waves = 4;
    return best;
}

size_t qmm_int8_gemm_dynamic_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K <= 0 || N <= 0) return 0;
    if (dynamic_fused(M, K, N)) return (size_t)plan_int8_gemm(dynamic_shape(M, K, packed_b_layout(K, N).NS).rows, K, N, false).ws_bytes;
    return (size_t)(round_up(M * K, 256) + round_up(4 * M, 256));
}

qmm_status int8_gemm_dynamic(const float *X, int64_t M, int64_t K, int64_t ldx, const void *packedB, int64_t N,
                             const qmm_epilogue *ep, int8_t *Xq, int64_t ldq, float *row_scale,
                             void *workspace, size_t workspace_bytes, void *stream) {
    if (M < 0 || N < 0 || K <= 0 || !ep || ldx < K) return QMM_ERR_INVALID;
    if (ep->row_scale) return QMM_ERR_INVALID;  // the row scales are the computed ones
    if (Xq && ldq < K) return QMM_ERR_INVALID;
    qmm_status st = check_epilogue(ep, N);
    if (st != QMM_OK) return st;
    if (!k_in_bound(K) || M > INT32_MAX / 2 || N > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return QMM_OK;
    if (!X || !packedB || !aligned(packedB, 256) || !aligned(X, 4) || (row_scale && !aligned(row_scale, 4)) ||
        check_epilogue_ptrs(ep) != QMM_OK)
        return QMM_ERR_INVALID;
    hipStream_t s = (hipStream_t)stream;
    if (dynamic_wide_fused(M, K, N, X, ldx)) {
        // the wide decode with the quantisation inside: one launch
        Int8GemmParams p{};
        fill_params(p, M, K, N, packedB, ep);
        p.X = X;
        p.ldx = ldx;
        p.x_vec = 1;
        p.xq_out = Xq;
        p.ldq = ldq;
        p.rs_out = row_scale;
        const char *variant = "";
        st = hip_status(launch_int8_gemm_dynamic_wide(p, s, &variant));
        g_last_variant = variant;
        trace_gemm("int8_gemm_dynamic", variant, M, K, N, plan_int8_gemm(M, K, N));
        return st;
    }
    if (!dynamic_fused(M, K, N)) {
        // The row quantiser, then the product.
        int8_t *q = Xq;
        float *rs = row_scale;
        int64_t lq = ldq;
        const size_t need = (q && rs) ? 0 : qmm_int8_gemm_dynamic_workspace_bytes(M, K, N);
        if (need > 0) {
            if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return QMM_ERR_WORKSPACE;
            if (!q) {
                q = (int8_t *)workspace;
                lq = K;
            }
            if (!rs) rs = (float *)((int8_t *)workspace + round_up(M * K, 256));
        }
        st = quantize_rows_int8(X, M, K, ldx, q, lq, rs, stream);
        if (st != QMM_OK) return st;
        qmm_epilogue e2 = *ep;
        e2.row_scale = rs;
        return int8_gemm(q, QMM_S8, M, K, lq, 0, packedB, QMM_S8, N, 0, &e2, nullptr, 0, stream);
    }
    // one round of the workgroup's wavefronts covers K <= 4096, so the
    // activations stay in registers between the amax and quantise passes
    const DynShape ds = dynamic_shape(M, K, packed_b_layout(K, N).NS);
    const int64_t rows = ds.rows;
    Int8Plan plan = plan_int8_gemm(rows, K, N, false);
    plan.spw = ds.spw;
    plan.waves = ds.waves;
    if (plan.ws_bytes > 0 && (!workspace || workspace_bytes < (size_t)plan.ws_bytes || !aligned(workspace, 256)))
        return QMM_ERR_WORKSPACE;
    Int8GemmParams p{};
    fill_params(p, M, K, N, packedB, ep);
    p.X = X;
    p.ldx = ldx;
    p.x_vec = aligned(X, 16) && (ldx % 4 == 0);
    p.xq_out = Xq;
    p.ldq = ldq;
    p.rs_out = row_scale;
    p.rpg = rows < M ? (int)rows : 0;
    const char *variant = "";
    st = hip_status(launch_int8_gemm_dynamic(plan, p, s, &variant));
    g_last_variant = variant;
    trace_gemm("int8_gemm_dynamic", variant, M, K, N, plan);
    return st;
}

static_assert(QMM_MAX_GROUP_ITEMS == kMaxGroups, "one grouped launch holds every item");

size_t qmm_int8_gemm_dynamic_grouped_workspace_bytes(int64_t M, int64_t K) {
    if (M <= 0 || K <= 0 || dynamic_fusable(M, K)) return 0;
    return (size_t)(round_up(M * K, 256) + round_up(4 * M, 256));
}

qmm_status int8_gemm_dynamic_grouped(const float *X, int64_t M, int64_t K, int64_t ldx,
                                     const qmm_dynamic_item *items, int64_t n_items, float scale,
                                     void *workspace, size_t workspace_bytes, void *stream) {
    if (M < 0 || K <= 0 || ldx < K || !items || n_items < 1 || n_items > QMM_MAX_GROUP_ITEMS)
        return QMM_ERR_INVALID;
    for (int64_t i = 0; i < n_items; ++i)
        if (items[i].N < 0 || items[i].ld_f32 < items[i].N) return QMM_ERR_INVALID;
    if (!k_in_bound(K) || M > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
    int64_t total_ns = 0;
    for (int64_t i = 0; i < n_items; ++i) {
        if (items[i].N > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
        total_ns += packed_b_layout(K, items[i].N).NS;
    }
    if (total_ns > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
    if (M == 0) return QMM_OK;
    if (!X || !aligned(X, 4)) return QMM_ERR_INVALID;
    for (int64_t i = 0; i < n_items; ++i) {
        if (items[i].N == 0) continue;
        const qmm_dynamic_item &it = items[i];
        if (!it.packedB || !aligned(it.packedB, 256) || !it.y_f32 || !aligned(it.y_f32, 4) ||
            (it.bias_f32 && !aligned(it.bias_f32, 4)))
            return QMM_ERR_INVALID;
        if (g_check && qmm_packed_b_check(it.packedB, K, it.N, stream) != QMM_OK) return QMM_ERR_INVALID;
    }
    if (!dynamic_fusable(M, K)) {
        // not fusable: quantise once, then one product per item
        const size_t need = qmm_int8_gemm_dynamic_grouped_workspace_bytes(M, K);
        if (!workspace || workspace_bytes < need || !aligned(workspace, 256)) return QMM_ERR_WORKSPACE;
        int8_t *q = (int8_t *)workspace;
        float *rs = (float *)((int8_t *)workspace + round_up(M * K, 256));
        qmm_status st = quantize_rows_int8(X, M, K, ldx, q, K, rs, stream);
        for (int64_t i = 0; i < n_items && st == QMM_OK; ++i) {
            if (items[i].N == 0) continue;
            qmm_epilogue e{};
            e.outputs = QMM_OUT_F32;
            e.y_f32 = items[i].y_f32;
            e.ld_f32 = items[i].ld_f32;
            e.row_scale = rs;
            e.scale = scale;
            e.bias_f32 = items[i].bias_f32;
            st = int8_gemm(q, QMM_S8, M, K, K, 0, items[i].packedB, QMM_S8, items[i].N, 0, &e, nullptr, 0, stream);
        }
        return st;
    }
    // one fused launch over the items' strips, row groups as in int8_gemm_dynamic
    DecodeGroups dg{};
    for (int i = 0; i < kMaxGroups; ++i) dg.strip_begin[i] = INT32_MAX;
    int n = 0, sb = 0;
    for (int64_t i = 0; i < n_items; ++i) {
        if (items[i].N == 0) continue;
        const PackedBLayout L = packed_b_layout(K, items[i].N);
        const int8_t *base = (const int8_t *)items[i].packedB;
        dg.codes[n] = base + L.codes_off;
        dg.colsum[n] = (const int32_t *)(base + L.colsum_off);
        dg.col_scale[n] = (const float *)(base + L.scale_off);
        dg.y_f32[n] = items[i].y_f32;
        dg.ld_f32[n] = items[i].ld_f32;
        dg.bias_f32[n] = items[i].bias_f32;
        dg.N[n] = (int)items[i].N;
        dg.strip_begin[n] = sb;
        sb += (int)L.NS;
        ++n;
    }
    if (n == 0) return QMM_OK;
    const DynShape ds = dynamic_shape(M, K, sb);
    const int64_t rows = ds.rows;
    Int8Plan plan = plan_int8_gemm(rows, K, 16, false);
    plan.spw = ds.spw;
    plan.waves = ds.waves;
    Int8GemmParams p{};
    qmm_epilogue e0{};
    e0.outputs = QMM_OUT_F32;
    e0.y_f32 = dg.y_f32[0];
    e0.ld_f32 = dg.ld_f32[0];
    e0.scale = scale;
    fill_params(p, M, K, dg.N[0], (const int8_t *)dg.codes[0] - kHeaderBytes, &e0);
    p.NS = sb;  // the grid: every item's strips
    p.X = X;
    p.ldx = ldx;
    p.x_vec = aligned(X, 16) && (ldx % 4 == 0);
    p.rpg = rows < M ? (int)rows : 0;
    const char *variant = "";
    const qmm_status st = hip_status(launch_int8_gemm_dynamic_grouped(plan, p, dg, (hipStream_t)stream, &variant));
    g_last_variant = variant;
    trace_gemm("int8_gemm_dynamic_grouped", variant, M, K, sb * 16, plan);
    return st;
}

}  // extern "C"
