// qmm_internal.h -- device layouts and launcher declarations shared by the
// host dispatcher (api.cpp) and the HIP kernels.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "qmm.h"

namespace qmm {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v4f __attribute__((ext_vector_type(4)));

inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }
inline int64_t ceil_div(int64_t x, int64_t m) { return (x + m - 1) / m; }

// ------------------------------------------------------------------------
// Packed int8 weight.  The codes of a K x N weight are stored as 1 KiB tiles
// of 64 k x 16 n.  Inside a tile, 16-byte chunk `lane` (0..63) holds the 16
// consecutive k = 16*(lane/16) .. +15 of column lane%16: exactly the B operand
// one wavefront lane feeds to v_mfma_i32_16x16x64_i8, so a wavefront reads a
// tile with one fully coalesced 16-byte load per lane.  Tiles of one 16-column
// strip are contiguous along k (strip-major), so a K-range of one strip is one
// contiguous run of HBM.
//   byte offset of (k, n) = 64 + ((n/16)*KT + k/64)*1024
//                           + ((k%64)/16)*256 + (n%16)*16 + (k%16)
// followed by fp32 scale[Np] and int32 colsum[Np].  K is padded to a multiple
// of 64 and N to 16 with zero codes.
// ------------------------------------------------------------------------
constexpr int kTileK = 64;
constexpr int kTileN = 16;
constexpr int kTileBytes = 1024;
constexpr int64_t kHeaderBytes = 64;
constexpr uint32_t kPackMagic = 0x31424d51u;  // "QMB1"
constexpr uint32_t kPackVersion = 1;

enum PackKind : uint32_t { kPackF32 = 0, kPackRawS8 = 1, kPackRawU8 = 2 };

struct PackedHeader {
    uint32_t magic, version, kind, reserved;
    int64_t K, N, Kp, Np;
    int64_t scale_off, colsum_off;
};
static_assert(sizeof(PackedHeader) == 64, "header is 64 bytes");

struct PackedBLayout {
    int64_t K, N, Kp, Np, KT, NS;
    int64_t codes_off, scale_off, colsum_off, total;
};

inline PackedBLayout packed_b_layout(int64_t K, int64_t N) {
    PackedBLayout L;
    L.K = K;
    L.N = N;
    L.Kp = round_up(K > 0 ? K : 1, kTileK);
    L.Np = round_up(N > 0 ? N : 1, kTileN);
    L.KT = L.Kp / kTileK;
    L.NS = L.Np / kTileN;
    L.codes_off = kHeaderBytes;
    L.scale_off = L.codes_off + L.Kp * L.Np;
    L.colsum_off = L.scale_off + 4 * L.Np;
    L.total = L.colsum_off + 4 * L.Np;
    return L;
}

// ------------------------------------------------------------------------
// int8 GEMM launch parameters (passed by value as the kernel argument).
// ------------------------------------------------------------------------
struct Int8GemmParams {
    // 8-byte fields first, then the 4-byte ones: no padding, 240 bytes (the
    // decode calls measured 0.2 us slower per launch with this struct at 264
    // bytes, padded between its int and pointer fields)
    const int8_t *A;      // raw bytes of A (int8 or uint8)
    int64_t lda;
    // per-axis zero points (NULL: the scalars zAs, zBs): one per row of A, one
    // per column of B, in the caller's domain; za_off / zb_off (128 for uint8,
    // else 0) take them to the shifted domain
    const int32_t *za_row, *zb_col;
    const int8_t *codes;  // packed tiles
    const int32_t *colsum;
    // epilogue
    int32_t *y_i32;
    int64_t ld_i32;
    float *y_f32;
    int64_t ld_f32;
    int8_t *y_q8;
    int64_t ld_q8;
    const float *row_scale;  // NULL = 1
    const float *col_scale;  // never NULL (defaults to the packed scales)
    const float *bias_f32;
    const int32_t *bias_i32;
    // dynamic variant: fp32 activations quantised per row inside the kernel
    const float *X;
    int64_t ldx;
    int8_t *xq_out;        // optional copies of the quantised rows / scales
    int64_t ldq;
    float *rs_out;
    int M, K, N;
    int a_u8;             // 1: A is uint8 (flip the top bit to shift by 128)
    int a_vec;            // 1: A and lda allow aligned 16-byte loads
    int32_t zAs, zBs;     // zero points in the shifted (int8) domain
    int32_t za_off, zb_off;
    int KT, NS;           // k tiles, n strips
    uint32_t outputs;
    int q8_u8;
    float scale;
    int32_t zp_out;
    int x_vec;             // 1: X and ldx allow aligned 16-byte loads
    int rpg;               // > 0: rows per row group (blockIdx.y), each group an independent call
};

// The wide decode (one wavefront per strip over the whole k range) stages
// all of A' in LDS: at most this many 1 KiB operand tiles (k tiles x 16-row
// tiles), 64 KiB.  It is planned from this many 16-column strips on.
constexpr int kWideWaves = 8;        // strips (wavefronts) per workgroup
constexpr int kWideMaxTiles = 64;
constexpr int64_t kWideMinStrips = 1024;

struct Int8Plan {
    int variant;      // 0 = decode (M <= 32), 1 = prefill, 2 = wide decode (M <= 32, many columns)
    int mt;           // 16-row tiles (decode)
    int waves;        // waves per workgroup (decode)
    int tpw;          // k tiles per wave per round (decode)
    int64_t grid;
    int64_t ws_bytes; // workspace the plan needs (0 for every current variant)
};

// allow_wide = false: the per-strip decode for M <= 32 whatever N (the fused
// quantising launch has no wide form)
Int8Plan plan_int8_gemm(int64_t M, int64_t K, int64_t N, bool allow_wide = true);

hipError_t launch_pack_b_f32(const float *W, int64_t ldw, const PackedBLayout &L, void *packed,
                             hipStream_t s);
hipError_t launch_pack_b_raw(const void *B, int u8, int64_t ldb, const PackedBLayout &L,
                             void *packed, hipStream_t s);
hipError_t launch_quantize_rows(const float *X, int64_t M, int64_t K, int64_t ldx, int8_t *Xq,
                                int64_t ldq, float *row_scale, hipStream_t s);
// the prefill kernel (M > 32), launched by launch_int8_gemm
hipError_t launch_int8_prefill(const Int8GemmParams &p, hipStream_t s);
hipError_t launch_int8_gemm(const Int8Plan &plan, Int8GemmParams p, hipStream_t s,
                            const char **variant);
hipError_t launch_int8_gemm_dynamic(const Int8Plan &plan, Int8GemmParams p, hipStream_t s,
                                    const char **variant);

}  // namespace qmm

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
    const uint8_t *xsum;      // [R][NQ][3] 16 bytes: the record's four block sums (bf16 terms)
    const int32_t *xsc;       // [R] scale exponents sc[a] (R activation rows, see MoeSplit)
    const uint8_t *zero16;    // 16 zero bytes
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
    uint8_t *xs, *xsum, *zero16;
    int32_t *xsc;
};

struct Q4Plan {
    int mt, waves, cs, S, qps;  // cs: strips per workgroup of the M <= 4 kernel
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
