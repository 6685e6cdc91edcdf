// q4_internal.h -- internal declarations of the q4_1 path: the device
// record layout, the launch parameters of the dense, MoE and int8-activation
// kernels, their planners and launchers.
#pragma once

#include "qmm_internal.h"

namespace qmm {

// ------------------------------------------------------------------------
// q4_1 device layout.  A K x N q4_1 weight (blocks of 32 k per column) is
// stored as records of 4 consecutive blocks x 16 columns, strip-major:
//   record (strip, quad) at 64 + (strip*NQ + quad) * 1280, NQ = ceil(NB/4)
//   bytes [0, 1024): 64 lane chunks of 16 bytes.  Chunk `lane` holds, for
//       column lane%16 and k-octet g = lane/16, four 4-byte words, one per
//       block of the record; word i holds the codes of k = 32b + 8g + e,
//       e = 0..7, with element e in nibble 2e (e < 4) or 2(e-4)+1 (e >= 4),
//       so that (w & 0x0F0F0F0F) and ((w >> 4) & 0x0F0F0F0F) are the bytes of
//       elements 0..3 and 4..7 in order.
//   bytes [1024, 1280): for column c at 1024 + 16c, the bf16 pairs (d, m) of
//       the record's four blocks.
// Padding blocks and columns hold zero codes and d = m = 0.  A record is
// 16 x 128 weights in 1280 bytes: the canonical 5 bits per weight.
// ------------------------------------------------------------------------
constexpr int kQ4RecBytes = 1280;
constexpr uint32_t kQ4Magic = 0x31514d51u;  // "QMQ1"

struct Q4Layout {
    int64_t K, N, NB, NQ, NS, total;
};

inline Q4Layout q4_layout(int64_t K, int64_t N) {
    Q4Layout L;
    L.K = K;
    L.N = N;
    L.NB = K / 32;
    L.NQ = ceil_div(L.NB, 4);
    L.NS = ceil_div(N, 16);
    L.total = kHeaderBytes + L.NS * L.NQ * kQ4RecBytes;
    return L;
}

struct Q4Params {
    const uint8_t *recs;      // dense: the weight; MoE: expert 0
    int64_t expert_stride;    // MoE: bytes between experts
    int NQ, NB, NS, N, K;
    const float *X;           // fp32 activations (row stride ldx)
    int64_t ldx;
    int x_vec;                // 1: X and ldx allow aligned 16-byte loads
    int M;                    // dense rows in this launch
    float *Y;
    int64_t ldy;
    float *part;              // dense split-K partials [S][M][N]
    int S, qps;               // dense: splits, quads per split
    // MoE routing tables (device)
    const int32_t *sorted;    // pair ids grouped by expert
    const int32_t *chunk_info;  // [max_chunks][3]: expert, first row, rows
    const int32_t *nchunks;
    int n_used;
    int64_t ldy_slot, ldy_token;
    // MoE activations split once per call by the routing launch
    const uint8_t *xs;        // [R][NB][2][4] 16-byte pieces: two fp16 terms of x * 2^sc[a]
    const uint8_t *xsum;      // [R][NQ] 64 bytes: per bf16 term u < 3 the record's four block sums and 8 zero bytes, then 16 zero bytes
    const int32_t *xsc;       // [R] scale exponents sc[a] (R activation rows, see MoeSplit)
    const uint8_t *zeros;     // 256 zero bytes
};

// The MoE activation split (k_moe_route's extra workgroups): per token t,
// sc[t] = 15 - e with the token's max |x| = f 2^e, f in [0.5, 1); each piece
// (block b, k-octet g) of x * 2^sc as two fp16 terms, and each block's sum
// of x * 2^sc as three bf16 terms, four blocks (a record) per 16 bytes.
// q4_1 weights x per-row int8 activations (k_q4_q8): one launch per 16 rows.
struct Q4Q8Params {
    const uint8_t *recs;      // the weight (q4_1 device layout, with its header)
    const int8_t *Xq;         // int8 activation codes, row stride ldq
    const float *row_scale;   // [M] per-row scales
    float *Y;
    int64_t ldq, ldy;
    int NQ, NS, N, K, M;      // M <= 16 rows in this launch
};

hipError_t launch_q4_q8(const Q4Q8Params &p, hipStream_t s, const char **variant);

// The MoE activation split works on activation rows: R = T tokens (shared
// form, per = 1) or R = T * n_used (token, slot) pairs (per-slot form,
// per = n_used); row a starts at X + (a / per) * ldx + (a % per) * ldx_slot.
struct MoeSplit {
    const float *X;
    int64_t ldx, ldx_slot;
    int T, R, per, K, NB, NQ, x_vec;
    int tpt;  // threads per activation row (set by the launcher)
    uint8_t *xs, *xsum, *zeros;
    int32_t *xsc;
};

struct Q4Plan {
    int mt, waves, cs, S, qps;  // cs: mt 0, strips per workgroup; mt 1, 1 = k_q4_mm16_wide
    int64_t grid, rows_per_launch;
    int64_t ws_part_off, ws_bytes;
};

Q4Plan plan_q4_matmul(int64_t M, int64_t K, int64_t N);

struct MoePlan {
    int rpc;
    int64_t max_chunks;
    int64_t ws_sorted_off, ws_chunk_off, ws_misc_off, ws_xs_off, ws_xsum_off, ws_xsc_off, ws_bytes;
};

MoePlan plan_q4_moe(int64_t T, int64_t n_used, int64_t E, int64_t K, int64_t N, bool per_slot);

hipError_t launch_q4_repack(const uint8_t *blocks, const Q4Layout &L, uint8_t *packed, hipStream_t s);
hipError_t launch_q4_dense(const Q4Params &p, int mt, int waves, int cs, int64_t grid, hipStream_t s,
                           const char **variant);
hipError_t launch_moe_route(const int32_t *ids, int64_t ids_stride, int64_t T, int64_t n_used, int64_t E,
                            int rpc, int32_t *sorted, int32_t *chunk_info, int32_t *nchunks, int32_t *err,
                            const MoeSplit &sp, hipStream_t s);
// per_slot: the activation row of pair (t, s) is the pair itself, not token t
hipError_t launch_q4_moe(const Q4Params &p, bool per_slot, int64_t max_chunks, hipStream_t s, const char **variant);

}  // namespace qmm
