// api_q4.cpp -- C ABI of the q4_1 path: argument checks, launch planning and
// dispatch.  Everything is checked before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>
#include <mutex>

#include "qmm.h"
#include "q4_internal.h"

namespace qmm {

// Set by every entry point (defined in api.cpp).
qmm_status record_status(hipError_t e, const char *variant);

// Dense q4_1: rows run in launches of up to 32 (one or two 16-row MFMA
// tiles).  A workgroup is 8 wavefronts x 2 strips = 256 columns and a k
// range of `qps` records (a multiple of the chunk, 2 records at 16 rows, 1
// at 32).  The k range is split S ways so that about `target` workgroups are
// in flight; the S partial results are summed in split order by a second
// kernel.  Fewer splits at larger M keep the partial traffic (S*M*N floats)
// small next to the weight bytes.
// Past 4096 strips k_q4_mm16 (16 strips per workgroup) has more workgroups
// than CUs: some CUs run several, each staging the same activations again,
// and the strips spread unevenly, where the persistent form spreads them
// evenly and stages once per CU.  Measured at K = 1024, M = 16 (us per call,
// k_q4_mm16 / persistent): 4096 strips 13.9 / 15.4, 6144 21.7 / 19.6,
// 8192 23.9 / 23.6, 9496 31.0 / 27.5, 16384 46.1 / 41.2.
constexpr int64_t kWideMm16Strips = 4096;

Q4Plan plan_q4_matmul(int64_t M, int64_t K, int64_t N) {
    Q4Plan pl{};
    const Q4Layout L = q4_layout(K, N);
    pl.rows_per_launch = M < 32 ? M : 32;
    // mt 0: one 16-row tile holding the three bf16 terms of up to 4 rows
    pl.mt = pl.rows_per_launch <= 4 ? 0 : pl.rows_per_launch <= 16 ? 1 : 2;
    pl.waves = 8;
    if (pl.mt == 0) {
        // k_q4_gemv: a workgroup owns one strip and its 4, 8 or 16
        // wavefronts split the k range, so one launch covers the whole
        // product.  The fewest wavefronts that leave at most 8 records each
        // (the kernel keeps them all in flight) and give about 2048
        // wavefronts in all; 16 when none does.
        // At one row the kernel keeps all of a wavefront's records in flight
        // and the tail after the last data arrives is one wavefront's records,
        // so at most 4 records each where the workgroup size allows.
        if (M == 1 && L.NQ <= 8 && L.NS >= 1024) {
            // k_q4_gemv1_wide: a wavefront per strip over its whole k range,
            // 8 strips per workgroup sharing one staging of the activations
            pl.cs = 8;
            pl.waves = 8;
            pl.S = 1;
            pl.qps = (int)L.NQ;
            pl.grid = ceil_div(L.NS, 8);
            pl.ws_part_off = 0;
            pl.ws_bytes = 0;
            return pl;
        }
        pl.cs = 1;
        pl.waves = 16;
        const int64_t rmax = M == 1 && ceil_div(L.NQ, 16) <= 4 ? 4 : 8;
        for (int w : {4, 8, 16}) {
            if (ceil_div(L.NQ, w) <= rmax && L.NS * w >= 2048) {
                pl.waves = w;
                break;
            }
        }
        pl.S = 1;
        pl.qps = (int)ceil_div(L.NQ, pl.waves);
        pl.grid = ceil_div(L.NS, pl.cs);
        pl.ws_part_off = 0;
        pl.ws_bytes = 0;
        return pl;
    }
    if (pl.mt == 1 && L.NQ <= 8 && L.NS > kWideMm16Strips) {
        // k_q4_mm16_wide: one workgroup per CU, each staging the whole k
        // range once for its contiguous run of strips (k_q4_mm16 would need
        // more workgroups than fit at once)
        pl.cs = 1;
        pl.S = 1;
        pl.qps = (int)L.NQ;
        pl.grid = 256;
        pl.ws_part_off = 0;
        pl.ws_bytes = 0;
        return pl;
    }
    if (pl.mt == 1) {
        // k_q4_mm16: 8 wavefronts x 2 strips per workgroup and at most 8
        // records (its whole k range is staged in LDS at once); the k range
        // is split as evenly as that allows
        const int64_t groups = ceil_div(L.NS, 16);
        const int64_t S = ceil_div(L.NQ, 8);
        pl.qps = (int)ceil_div(L.NQ, S);
        pl.S = (int)ceil_div(L.NQ, pl.qps);
        pl.grid = groups * pl.S;
        pl.ws_part_off = 0;
        pl.ws_bytes = pl.S > 1 ? round_up((int64_t)pl.S * pl.rows_per_launch * N * 4, 256) : 0;
        return pl;
    }
    const int64_t qc = pl.mt <= 1 ? 2 : 1;
    const int64_t groups = ceil_div(L.NS, 2 * pl.waves);
    const int64_t target = pl.rows_per_launch <= 4 ? 512 : 256;
    int64_t S = ceil_div(target, groups);
    const int64_t max_s = ceil_div(L.NQ, qc);
    if (S > max_s) S = max_s;
    if (S < 1) S = 1;
    int64_t qps = round_up(ceil_div(L.NQ, S), qc);
    S = ceil_div(L.NQ, qps);
    pl.S = (int)S;
    pl.qps = (int)qps;
    pl.grid = groups * S;
    pl.ws_part_off = 0;
    pl.ws_bytes = S > 1 ? round_up(S * pl.rows_per_launch * N * 4, 256) : 0;
    return pl;
}

MoePlan plan_q4_moe(int64_t T, int64_t n_used, int64_t E, int64_t K, int64_t N, bool per_slot) {
    MoePlan pl{};
    const int64_t P = T * n_used;
    const int64_t R = per_slot ? P : T;  // activation rows split
    pl.rpc = 32;
    pl.max_chunks = ceil_div(P, pl.rpc) + E;
    pl.ws_sorted_off = 0;
    pl.ws_chunk_off = round_up(P * 4, 256);
    pl.ws_misc_off = pl.ws_chunk_off + round_up(pl.max_chunks * 3 * 4, 256);
    // the activation split: fp16 terms (4 bytes per activation), block sums,
    // scale exponents
    const Q4Layout L = q4_layout(K, N);
    pl.ws_xs_off = pl.ws_misc_off + 512;
    pl.ws_xsum_off = pl.ws_xs_off + round_up(R * L.NB * 128, 256);
    pl.ws_xsc_off = pl.ws_xsum_off + round_up(R * L.NQ * 64, 256);
    pl.ws_bytes = pl.ws_xsc_off + round_up(R * 4, 256);
    return pl;
}

}  // namespace qmm

using namespace qmm;

// Rows run in launches of 32; a last launch of fewer rows is planned for its
// own row count (the M <= 4 or 5..16 kernels), so every k_q4_mm launch has
// 17..32 rows.  The workspace serves the larger of the two plans (launches
// run in turn on one stream and reuse it).
static int64_t q4_matmul_ws_bytes(int64_t M, int64_t K, int64_t N) {
    int64_t w = plan_q4_matmul(M < 32 ? M : 32, K, N).ws_bytes;
    if (M > 32 && M % 32 != 0) {
        const int64_t t = plan_q4_matmul(M % 32, K, N).ws_bytes;
        if (t > w) w = t;
    }
    return w;
}

static bool aligned_to(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

extern "C" {

size_t qmm_q4_1_packed_bytes(int64_t K, int64_t N) {
    if (K <= 0 || N <= 0 || K % 32 != 0) return 0;
    return (size_t)q4_layout(K, N).total;
}

qmm_status q4_1_repack(const void *blocks, int64_t K, int64_t N, void *packed, size_t packed_bytes,
                       void *stream) {
    if (K <= 0 || N <= 0 || !blocks || !packed || !aligned_to(packed, 256)) return QMM_ERR_INVALID;
    if (K % 32 != 0) return QMM_ERR_UNSUPPORTED;
    if (K > INT32_MAX / 2 || N > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
    const Q4Layout L = q4_layout(K, N);
    if (packed_bytes < (size_t)L.total) return QMM_ERR_WORKSPACE;
    return record_status(launch_q4_repack((const uint8_t *)blocks, L, (uint8_t *)packed, (hipStream_t)stream),
                         "q4_repack");
}

size_t qmm_q4_1_matmul_workspace_bytes(int64_t M, int64_t K, int64_t N) {
    if (M <= 0 || K <= 0 || N <= 0 || K % 32 != 0) return 0;
    return (size_t)q4_matmul_ws_bytes(M, K, N);
}

qmm_status q4_1_matmul(const float *X, int64_t M, int64_t K, int64_t ldx, const void *Wpacked, int64_t N,
                       float *Y, int64_t ldy, void *workspace, size_t workspace_bytes, void *stream) {
    if (M < 0 || K <= 0 || N < 0 || ldx < K || ldy < N) return QMM_ERR_INVALID;
    if (K % 32 != 0) return QMM_ERR_UNSUPPORTED;
    if (M > INT32_MAX / 2 || K > INT32_MAX / 2 || N > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return QMM_OK;
    if (!X || !Wpacked || !Y || !aligned_to(Wpacked, 256) || !aligned_to(X, 4) || !aligned_to(Y, 4))
        return QMM_ERR_INVALID;
    const Q4Layout L = q4_layout(K, N);
    const int64_t ws_need = q4_matmul_ws_bytes(M, K, N);
    if (ws_need > 0 && (!workspace || workspace_bytes < (size_t)ws_need || !aligned_to(workspace, 256)))
        return QMM_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipSuccess;
    const char *variant = "";
    for (int64_t r0 = 0; r0 < M && e == hipSuccess; r0 += 32) {
        const int64_t rows = (M - r0) < 32 ? (M - r0) : 32;
        const Q4Plan pl = plan_q4_matmul(rows, K, N);
        Q4Params p{};
        p.recs = (const uint8_t *)Wpacked;
        p.NQ = (int)L.NQ;
        p.NB = (int)L.NB;
        p.NS = (int)L.NS;
        p.N = (int)N;
        p.K = (int)K;
        p.X = X + r0 * ldx;
        p.ldx = ldx;
        p.x_vec = aligned_to(X, 16) && (ldx % 4 == 0);
        p.M = (int)rows;
        p.Y = Y + r0 * ldy;
        p.ldy = ldy;
        p.part = (float *)((uint8_t *)workspace + pl.ws_part_off);
        p.S = pl.S;
        p.qps = pl.qps;
        e = launch_q4_dense(p, pl.mt, pl.waves, pl.cs, pl.grid, s, &variant);
    }
    return record_status(e, variant);
}

qmm_status q4_1_matmul_q8(const int8_t *Xq, const float *row_scale, int64_t M, int64_t K, int64_t ldq,
                          const void *Wpacked, int64_t N, float *Y, int64_t ldy, void *stream) {
    if (M < 0 || K <= 0 || N < 0 || ldq < K || ldy < N) return QMM_ERR_INVALID;
    if (K % 32 != 0) return QMM_ERR_UNSUPPORTED;
    if (M > INT32_MAX / 2 || K > INT32_MAX / 2 || N > INT32_MAX / 2) return QMM_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return QMM_OK;
    if (!Xq || !row_scale || !Wpacked || !Y || !aligned_to(Wpacked, 256) || !aligned_to(row_scale, 4) ||
        !aligned_to(Y, 4))
        return QMM_ERR_INVALID;
    const Q4Layout L = q4_layout(K, N);
    hipError_t e = hipSuccess;
    const char *variant = "";
    // one launch per 16 rows (each reads the whole weight)
    for (int64_t r0 = 0; r0 < M && e == hipSuccess; r0 += 16) {
        Q4Q8Params p{};
        p.recs = (const uint8_t *)Wpacked;
        p.Xq = Xq + r0 * ldq;
        p.row_scale = row_scale + r0;
        p.Y = Y + r0 * ldy;
        p.ldq = ldq;
        p.ldy = ldy;
        p.NQ = (int)L.NQ;
        p.NS = (int)L.NS;
        p.N = (int)N;
        p.K = (int)K;
        p.M = (int)((M - r0) < 16 ? (M - r0) : 16);
        e = launch_q4_q8(p, (hipStream_t)stream, &variant);
    }
    return record_status(e, variant);
}

size_t qmm_q4_1_matmul_id_workspace_bytes(int64_t n_tokens, int64_t n_used, int64_t n_expert, int64_t K,
                                          int64_t N) {
    if (n_tokens <= 0 || n_used <= 0 || n_expert <= 0 || K <= 0 || N <= 0 || K % 32 != 0) return 0;
    return (size_t)plan_q4_moe(n_tokens, n_used, n_expert, K, N, false).ws_bytes;
}

size_t qmm_q4_1_matmul_id_per_slot_workspace_bytes(int64_t n_tokens, int64_t n_used, int64_t n_expert, int64_t K,
                                                   int64_t N) {
    if (n_tokens <= 0 || n_used <= 0 || n_expert <= 0 || K <= 0 || N <= 0 || K % 32 != 0) return 0;
    return (size_t)plan_q4_moe(n_tokens, n_used, n_expert, K, N, true).ws_bytes;
}

}  // extern "C"

// ------------------------------------------------ allocation-free MUL_MAT_ID ---
// q4_1_matmul_id_noalloc keeps its routing tables and split activations in
// this library-owned array instead of a caller workspace.  Each GPU the
// library runs on holds its own copy until the process ends.  In host code
// `scratch` names a host-side stand-in, not the device array: the device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current, and only that address is handed to the kernels.
static __device__ __align__(256) uint8_t scratch[QMM_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];  // device address of `scratch` per device (null until looked up)

// The scratch array's address on the device that runs `stream`.
hipError_t scratch_on(hipStream_t stream, void **out) {
    int dev = 0;
    hipError_t e = hipStreamGetDevice(stream, &dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        e = hipGetDevice(&cur);
        if (e != hipSuccess) return e;
        if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
        void *ptr = nullptr;
        e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
        if (cur != dev) {
            const hipError_t e2 = hipSetDevice(cur);
            if (e == hipSuccess) e = e2;
        }
        if (e != hipSuccess) return e;
        if (!ptr) return hipErrorInvalidSymbol;
        g_scratch_ptr[dev] = ptr;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}
}  // namespace

// Both MUL_MAT_ID forms: the shared one (ldx_slot = 0: token t's row for
// every slot) and the per-slot one (a row per (token, slot) pair).
static qmm_status moe_call(const float *X, int64_t n_tokens, int64_t K, int64_t ldx, int64_t ldx_slot,
                           bool per_slot, const void *Wexperts, int64_t n_expert, int64_t N, size_t expert_stride,
                           const int32_t *ids, int64_t ids_row_stride, int64_t n_used, float *Y, int64_t ldy_slot,
                           int64_t ldy_token, void *workspace, size_t workspace_bytes, void *stream,
                           bool use_scratch = false) {
    if (n_tokens < 0 || K <= 0 || N < 0 || n_expert <= 0 || n_used <= 0 || ids_row_stride < n_used ||
        ldy_slot < N || ldy_token < n_used * ldy_slot)
        return QMM_ERR_INVALID;
    if (per_slot ? (ldx_slot < K || ldx < n_used * ldx_slot) : ldx < K) return QMM_ERR_INVALID;
    if (K % 32 != 0) return QMM_ERR_UNSUPPORTED;
    if (n_expert > 8192 || n_tokens * n_used > INT32_MAX / 2 || K > INT32_MAX / 2 || N > INT32_MAX / 2)
        return QMM_ERR_UNSUPPORTED;
    if (n_tokens == 0 || N == 0) return QMM_OK;
    if (!X || !Wexperts || !ids || !Y || !aligned_to(Wexperts, 256) || !aligned_to(X, 4) || !aligned_to(Y, 4) ||
        !aligned_to(ids, 4))
        return QMM_ERR_INVALID;
    const Q4Layout L = q4_layout(K, N);
    if (expert_stride < (size_t)L.total || expert_stride % 256 != 0) return QMM_ERR_INVALID;
    // the product kernel addresses the split activations with 32-bit offsets
    const int64_t R = per_slot ? n_tokens * n_used : n_tokens;
    if (R * L.NB * 128 > (int64_t)UINT32_MAX || R * L.NQ * 64 > (int64_t)UINT32_MAX) return QMM_ERR_UNSUPPORTED;
    const MoePlan pl = plan_q4_moe(n_tokens, n_used, n_expert, K, N, per_slot);
    if (use_scratch) {
        // the library-owned array (allocation-free entry point)
        if (pl.ws_bytes > (int64_t)QMM_NOALLOC_SCRATCH_BYTES) return QMM_ERR_WORKSPACE;
        const hipError_t e = scratch_on((hipStream_t)stream, &workspace);
        if (e != hipSuccess) return record_status(e, "q4_moe_m32");
        workspace_bytes = QMM_NOALLOC_SCRATCH_BYTES;
    }
    if (!workspace || workspace_bytes < (size_t)pl.ws_bytes || !aligned_to(workspace, 256))
        return QMM_ERR_WORKSPACE;
    hipStream_t s = (hipStream_t)stream;
    uint8_t *ws = (uint8_t *)workspace;
    int32_t *sorted = (int32_t *)(ws + pl.ws_sorted_off);
    int32_t *chunk_info = (int32_t *)(ws + pl.ws_chunk_off);
    int32_t *misc = (int32_t *)(ws + pl.ws_misc_off);
    const bool xvec = aligned_to(X, 16) && (ldx % 4 == 0) && (ldx_slot % 4 == 0);
    MoeSplit sp{};
    sp.X = X;
    sp.ldx = ldx;
    sp.ldx_slot = per_slot ? ldx_slot : 0;
    sp.T = (int)n_tokens;
    sp.per = per_slot ? (int)n_used : 1;
    sp.R = (int)(per_slot ? n_tokens * n_used : n_tokens);
    sp.K = (int)K;
    sp.NB = (int)L.NB;
    sp.NQ = (int)L.NQ;
    sp.x_vec = xvec;
    sp.xs = ws + pl.ws_xs_off;
    sp.xsum = ws + pl.ws_xsum_off;
    sp.xsc = (int32_t *)(ws + pl.ws_xsc_off);
    sp.zeros = ws + pl.ws_misc_off + 256;
    hipError_t e = launch_moe_route(ids, ids_row_stride, n_tokens, n_used, n_expert, pl.rpc, sorted, chunk_info,
                                    misc, misc + 1, sp, s);
    const char *variant = "";
    if (e == hipSuccess) {
        Q4Params p{};
        p.recs = (const uint8_t *)Wexperts;
        p.expert_stride = (int64_t)expert_stride;
        p.NQ = (int)L.NQ;
        p.NB = (int)L.NB;
        p.NS = (int)L.NS;
        p.N = (int)N;
        p.K = (int)K;
        p.X = X;
        p.ldx = ldx;
        p.x_vec = xvec;
        p.Y = Y;
        p.sorted = sorted;
        p.chunk_info = chunk_info;
        p.nchunks = misc;
        p.n_used = (int)n_used;
        p.ldy_slot = ldy_slot;
        p.ldy_token = ldy_token;
        p.xs = sp.xs;
        p.xsum = sp.xsum;
        p.xsc = sp.xsc;
        p.zeros = sp.zeros;
        e = launch_q4_moe(p, per_slot, pl.max_chunks, s, &variant);
    }
    if (e == hipSuccess && g_check) {
        // the routing kernel flags ids outside [0, n_expert) (their pairs are
        // skipped, every other output is written)
        int32_t bad = 0;
        e = hipMemcpyAsync(&bad, misc + 1, sizeof(bad), hipMemcpyDeviceToHost, s);
        if (e == hipSuccess) e = hipStreamSynchronize(s);
        if (e == hipSuccess && bad) {
            record_status(e, variant);
            return QMM_ERR_INVALID;
        }
    }
    return record_status(e, variant);
}

extern "C" {

qmm_status q4_1_matmul_id(const float *X, int64_t n_tokens, int64_t K, int64_t ldx, const void *Wexperts,
                          int64_t n_expert, int64_t N, size_t expert_stride, const int32_t *ids,
                          int64_t ids_row_stride, int64_t n_used, float *Y, int64_t ldy_slot, int64_t ldy_token,
                          void *workspace, size_t workspace_bytes, void *stream) {
    return moe_call(X, n_tokens, K, ldx, 0, false, Wexperts, n_expert, N, expert_stride, ids, ids_row_stride,
                    n_used, Y, ldy_slot, ldy_token, workspace, workspace_bytes, stream);
}

qmm_status q4_1_matmul_id_per_slot(const float *X, int64_t n_tokens, int64_t K, int64_t ldx_slot,
                                   int64_t ldx_token, const void *Wexperts, int64_t n_expert, int64_t N,
                                   size_t expert_stride, const int32_t *ids, int64_t ids_row_stride, int64_t n_used,
                                   float *Y, int64_t ldy_slot, int64_t ldy_token, void *workspace,
                                   size_t workspace_bytes, void *stream) {
    return moe_call(X, n_tokens, K, ldx_token, ldx_slot, true, Wexperts, n_expert, N, expert_stride, ids,
                    ids_row_stride, n_used, Y, ldy_slot, ldy_token, workspace, workspace_bytes, stream);
}

}  // extern "C"

extern "C" qmm_status q4_1_matmul_id_noalloc(const float *X, int64_t n_tokens, int64_t K, int64_t ldx,
                                             const void *Wexperts, int64_t n_expert, int64_t N,
                                             size_t expert_stride, const int32_t *ids, int64_t ids_row_stride,
                                             int64_t n_used, float *Y, int64_t ldy_slot, int64_t ldy_token,
                                             void *stream) {
    return moe_call(X, n_tokens, K, ldx, 0, false, Wexperts, n_expert, N, expert_stride, ids, ids_row_stride,
                    n_used, Y, ldy_slot, ldy_token, nullptr, 0, stream, true);
}
