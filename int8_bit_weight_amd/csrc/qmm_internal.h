// qmm_internal.h -- device layouts and launcher declarations shared by the
// host dispatcher (api.cpp) and the int8 kernels; the q4_1 path's are in
// q4_internal.h.  gfx950 (CDNA4) only.
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

// check mode (qmm_set_check / QMM_CHECK=1): synchronous checks of device data
extern int g_check;

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

// Grouped fused decode: up to kMaxGroups weights that share the activations
// (one launch; the grid's strips are the items' strips back to back).  A
// second kernel argument, so the single-weight launches keep their
// argument size.
constexpr int kMaxGroups = 4;
struct DecodeGroups {
    const int8_t *codes[kMaxGroups];
    const int32_t *colsum[kMaxGroups];
    const float *col_scale[kMaxGroups];
    float *y_f32[kMaxGroups];
    const float *bias_f32[kMaxGroups];
    int64_t ld_f32[kMaxGroups];
    int strip_begin[kMaxGroups];  // first grid strip of each item; unused items: INT32_MAX
    int N[kMaxGroups];
};

// Wavefronts per workgroup of the fused quantising decode (k_int8_decode_q):
// 8, measured faster than 16 for every Qwen3-0.6B projection group at M = 1,
// 16 and 32 (fewer partial tiles to combine and less skew before the
// row-maximum barrier); 4 where K <= 1024, S <= 2 and >= 192 workgroups
// (faster there, slower everywhere else).  Int8Plan::waves carries it.

// The wide decode (one wavefront per strip over the whole k range) stages
// all of A' in LDS: at most this many 1 KiB operand tiles (k tiles x 16-row
// tiles), 64 KiB.  It is planned from this many 16-column strips on.
constexpr int kWideWaves = 8;        // strips (wavefronts) per workgroup
constexpr int kWideMaxTiles = 64;
// persistent wide decode (k_int8_decode_wide_qp): its grid (two workgroups
// per CU: measured 2-6 % faster than one on the lm_head), and the strips
// from which it is taken (at least one per wavefront)
constexpr int kWidePersistGrid = 512;
constexpr int64_t kWidePersistStrips = 4096;
constexpr int64_t kWideMinStrips = 1024;

struct Int8Plan {
    int variant;      // 0 = decode (M <= 32), 1 = prefill, 2 = wide decode (M <= 32, many columns)
    int mt;           // 16-row tiles (decode)
    int waves;        // waves per workgroup (decode; fused quantising decode: 4 or 8)
    int tpw;          // k tiles per wave per round (decode)
    int spw;          // 16-column strips per workgroup (fused quantising decode; 0 = 1)
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
hipError_t launch_int8_prefill(const Int8GemmParams &p, hipStream_t s, const char **variant);
hipError_t launch_int8_gemm(const Int8Plan &plan, Int8GemmParams p, hipStream_t s,
                            const char **variant);
// the wide decode with the quantisation inside (aligned X, K % 4 == 0)
hipError_t launch_int8_gemm_dynamic_wide(const Int8GemmParams &p, hipStream_t s, const char **variant);
hipError_t launch_int8_gemm_dynamic(const Int8Plan &plan, Int8GemmParams p, hipStream_t s,
                                    const char **variant);
// grouped form: p.NS is the total strip count of the items; p's per-weight
// fields are ignored (taken from g)
hipError_t launch_int8_gemm_dynamic_grouped(const Int8Plan &plan, Int8GemmParams p, const DecodeGroups &g,
                                            hipStream_t s, const char **variant);

}  // namespace qmm
