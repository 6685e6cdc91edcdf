// k_q4_1.hip -- q4_1 path kernels for gfx950 (CDNA4, wave64):
//   * repack of canonical q4_1 blocks into the record layout (qmm_internal.h)
//   * the q4_1 product on MFMA (v_mfma_f32_16x16x32_bf16) with fp32
//     activations split in-kernel into three bf16 terms (x = x0 + x1 + x2,
//     near exact): one 32-k block is one MFMA k-step, so each block gets a
//     fresh accumulator and
//       Y += d * (sum_k q*x) + m * (sum_k x)
//     ("NPU engine: full ELFs, no xclbin", "Q4NX chunks": q4_1 blocks;
//     "Zaya 8B Q4NX on the AMD NPU", "Round 26": W = q*scale + min with bf16
//     scale and min per (row, 32-col) block)
//   * MUL_MAT_ID routing: a counting sort of the (token, slot) pairs by
//     expert into chunks of rows, read through the strided id view ("Zaya
//     8B", "The bugs that were the work"), and one grouped launch over all
//     chunks (the grouped-dispatch cost lesson of "Round 25p"); the routing
//     launch also splits every token once into two fp16 terms under a
//     power-of-two scale, which the grouped product multiplies with
//     v_mfma_f32_16x16x32_f16 (two MFMAs per block instead of three).
//
// Codes stay exact: bytes 0..15 read as OCP e4m3 are exactly q * 2^-9, and
// v_cvt_scalef32_pk_bf16_fp8 (or _f16_fp8) with scale 2^9 turns two of them
// into two exact bf16 (fp16) integers per instruction.
#include <type_traits>
#include <utility>

#include "q4_internal.h"

namespace qmm {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef int v2i __attribute__((ext_vector_type(2)));
typedef float v2f __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef _Float16 v2h __attribute__((ext_vector_type(2)));
template <int N> using ic = std::integral_constant<int, N>;

// f(ic<0>{}), ..., f(ic<N-1>{})
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(ic<I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Eight 4-bit codes (record nibble order) -> eight exact bf16 values in k order.
// Each conversion yields one packed pair; the four pairs are the four dwords
// of the MFMA operand as they are (a bit cast, no element shuffling).
__device__ __forceinline__ v8bf decode8(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu;
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
    const v4i r = {__builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false)),
                   __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true)),
                   __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false)),
                   __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true))};
    return __builtin_bit_cast(v8bf, r);
}

// The same eight codes as exact fp16 values (the f16 form of the conversion).
__device__ __forceinline__ v8h decode8h(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu;
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
    const v4i r = {__builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false)),
                   __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true)),
                   __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false)),
                   __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true))};
    return __builtin_bit_cast(v8h, r);
}

// ---------------------------------------------------------------- repack ---
// One thread per (record, lane chunk).  Canonical block of column n, block b:
// 20 bytes at blocks + (n*NB + b)*20: d (bf16), m (bf16), 16 code bytes with
// element j in the low nibble of byte j (j < 16) or the high nibble of byte
// j-16.
__global__ __launch_bounds__(256) void k_q4_repack(const uint8_t *__restrict__ blocks, int NB, int N,
                                                   int NQ, int64_t nrec, uint8_t *__restrict__ base,
                                                   PackedHeader h) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid == 0) *(PackedHeader *)base = h;
    uint8_t *recs = base + kHeaderBytes;
    const int64_t rec = gid >> 6;
    const int lane = (int)(gid & 63);
    if (rec >= nrec) return;
    const int strip = (int)(rec / NQ);
    const int quad = (int)(rec % NQ);
    const int c = lane & 15;
    const int g = lane >> 4;
    const int n = strip * 16 + c;
    uint32_t w[4];
    uint32_t dm[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int b = quad * 4 + i;
        w[i] = 0u;
        dm[i] = 0u;
        if (n < N && b < NB) {
            const uint8_t *blk = blocks + ((int64_t)n * NB + b) * 20;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int j = 8 * g + e;
                const uint32_t q = (j < 16) ? (blk[4 + j] & 0x0Fu) : (uint32_t)(blk[4 + j - 16] >> 4);
                const int pos = e < 4 ? 2 * e : 2 * (e - 4) + 1;
                w[i] |= q << (4 * pos);
            }
            dm[i] = (uint32_t)blk[0] | ((uint32_t)blk[1] << 8) | ((uint32_t)blk[2] << 16) | ((uint32_t)blk[3] << 24);
        }
    }
    uint8_t *dst = recs + rec * kQ4RecBytes;
    *(v4i *)(dst + lane * 16) = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
    if (g == 0) *(v4i *)(dst + 1024 + c * 16) = v4i{(int)dm[0], (int)dm[1], (int)dm[2], (int)dm[3]};
}

// ----------------------------------------------------------- the product ---
// Workgroup = WAVES wavefronts; each wavefront owns C column strips (16 C
// columns) and all MT*16 rows of the workgroup's row set.  The k range is
// walked in chunks of QC records (4 QC blocks of 32 k).  Per block b and
// column n the product needs d_bn * sum_k(q x) + m_bn * sum_k(x):
//   * activations: the workgroup reads its rows' fp32 values for the next
//     chunk and splits each into three bf16 terms, x = x0 + x1 + x2 (the
//     conversions round to nearest; both differences are exact in fp32, and
//     x2 is exact in bf16).  The terms are stored in LDS as MFMA A fragments
//     (double buffered).  Each block's sum of x (fixed order) is split the
//     same way and stored as a second A operand whose k index is the block
//     of the chunk.  Only rows that exist are staged; fragments of absent
//     rows only reach accumulator rows that are never stored (an MFMA output
//     row depends on its own A row alone);
//   * weights: each wavefront streams its strips' records (16 bytes of codes
//     and 16 bytes of (d, m) per lane per record), one chunk ahead in
//     registers: with QC >= 2 a record's registers are refilled with the
//     next chunk's record as soon as its last block is used; with QC == 1
//     two register sets alternate and the chunk loop is unrolled by two;
//   * d term, per block and strip: codes -> exact bf16, three MFMAs into a
//     fresh accumulator, then y += d * acc;
//   * m term, per chunk and strip: the chunk's m values as a bf16 B operand
//     (k = block) against the split block sums, three MFMAs accumulating
//     over the whole k range.
//   blockIdx -> (strip group, k split); rows 0..M-1 (17 <= M <= 32 per
//   launch: the host plans a last launch of fewer rows for k_q4_gemv or
//   k_q4_mm16; k_q4_moe is the grouped product).
// Loads are never inside branches (a load in a branch makes the compiler wait
// for it where the branch ends, which would serialise the prefetch): indices
// past the valid range are clamped to valid memory.  A record past the range
// takes its (d, m) from the last 16 bytes of the packed header, which are
// zero, so it adds nothing.  XVEC: X and ldx allow aligned 16-byte loads.
//
// LDS layout of one 16-row A fragment (1 KiB): in MFMA lane order, the
// 16-byte piece of (row r, k-octet g) at slot 16 g + r, the slot lane 16 g + r
// reads, and the staging stores fill consecutive slots from consecutive
// threads.  Contiguous 16-byte-per-lane accesses measured free of LDS bank
// conflicts; an XOR swizzle of the rows by k-octet (16 g + (r ^ f(g)),
// f = {0, 6, 10, 12}) measured 2-way conflicted on every operand read.

// Two floats -> packed bf16 pair (round to nearest even), and the pair's
// residuals x - bf16(x), exact in fp32.
__device__ __forceinline__ uint32_t pk_bf16(float a, float b) {
    const v2bf r = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, r);
}
__device__ __forceinline__ float bf16_lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
// s_waitcnt on the vector memory counter only (gfx9 encoding: vmcnt in bits
// 3:0 and 15:14; expcnt and lgkmcnt left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt_q4() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
__device__ __forceinline__ float bf16_hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

template <int MT, int WAVES, int C, int QC, int MINW, bool XVEC, int RS = 2, int XD = 1>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(MINW, 8))) void k_q4_mm(Q4Params p) {
    constexpr int NT = WAVES * 64;
    constexpr int ROWS = MT * 16;
    constexpr int NF = 3;  // A fragments (bf16 terms) per block and row tile
    constexpr int SPG = C * WAVES;
    constexpr int BPC = 4 * QC;
    static_assert(BPC <= 8, "the m-term operand holds at most 8 blocks per chunk");
    constexpr int PIECES = BPC * ROWS * 4;  // (block, row, k-octet) pieces of a chunk at most
    constexpr int PPT = (PIECES + NT - 1) / NT;
    // weight register sets.  QC >= 2: one set; each record's registers are
    // refilled with the next chunk's record right after their last use.
    // QC == 1: RS sets; chunk c loads chunk c + RS - 1's records into the set
    // chunk c - 1 used when it starts (RS - 1 chunks in flight).
    constexpr int NSET = QC >= 2 ? 1 : RS;
    static_assert(NSET == 1 || NSET == 2 || NSET == 4, "record sets");
    // activation register sets: chunk c loads chunk c + XD's activations
    // (XD > 1 needs the chunk loop unrolled by XD: one set per unrolled chunk)
    static_assert(XD == 1 || XD == NSET, "activation sets follow the record sets");
    constexpr int ADB = MT == 1 ? 2 : 1;   // A fragment register sets
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][BPC][NF][MT][1024];
    // block sums as A fragments: row r, block bl at byte 16 r + 2 bl (k-octet
    // 0); k-octets 1..3 and blocks past BPC stay zero
    __shared__ __attribute__((aligned(16))) uint8_t sXM[2][NF][MT][1024];
    __shared__ int64_t sRow[ROWS];  // element offset of each row of X

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    // wave-uniform, so record addresses are computed in scalar registers
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int groups = (p.NS + SPG - 1) / SPG;
    const int sg = blockIdx.x % groups;
    const int job = blockIdx.x / groups;

    const uint8_t *hdr = p.recs;
    const int nrows = p.M;
    const int q0 = job * p.qps;
    const int q1 = min(p.NQ, q0 + p.qps);
    const uint8_t *recs = hdr + kHeaderBytes;
    if (tid < nrows) sRow[tid] = (int64_t)tid * p.ldx;
    for (int o = tid * 16; o < (int)sizeof(sXM); o += NT * 16) *(v4i *)(&sXM[0][0][0][0] + o) = v4i{0, 0, 0, 0};
    __syncthreads();

    // ---- activation staging.  piece -> (r = piece % 16, g = piece / 16 % 4,
    // tile = piece / 64 % MT, block = piece / 64 / MT): a wavefront's 64
    // pieces are one fragment, lane order.  Rows past nrows read row
    // nrows - 1 and stage zeros (their MFMA output rows are never stored);
    // both row tiles are always multiplied (see the note on k_q4_moe).
    int pbl[PPT], pg[PPT], prow[PPT], pdst[PPT];
    int64_t psrc[PPT];
    bool pok[PPT], pon[PPT];
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int idx = tid + i * NT;
        const int pc = min(idx, PIECES - 1);
        const int r = pc & 15, g = (pc >> 4) & 3, tile = (pc >> 6) % MT, blk = (pc >> 6) / MT;
        const int row = tile * 16 + r;
        prow[i] = row;
        pg[i] = g;
        pbl[i] = blk;
        pok[i] = idx < PIECES && row < nrows;
        pon[i] = idx < PIECES;
        psrc[i] = sRow[min(row, nrows - 1)] + g * 8;
        pdst[i] = (blk * 3 * MT + tile) * 1024 + (g * 16 + r) * 16;
    }
    float xr[XD][PPT][8];
    bool xok[XD][PPT];
    auto gload_a = [&](int qc, auto X_) {
        constexpr int xs = decltype(X_)::value;
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            const int b = qc * 4 + pbl[i];
            xok[xs][i] = pok[i] && b < p.NB;
            const float *src = p.X + psrc[i] + min(b, p.NB - 1) * 32;
            if (XVEC) {
                const v4f lo = *(const v4f *)src;
                const v4f hi = *(const v4f *)(src + 4);
                xr[xs][i][0] = lo[0]; xr[xs][i][1] = lo[1]; xr[xs][i][2] = lo[2]; xr[xs][i][3] = lo[3];
                xr[xs][i][4] = hi[0]; xr[xs][i][5] = hi[1]; xr[xs][i][6] = hi[2]; xr[xs][i][7] = hi[3];
            } else {
#pragma unroll
                for (int e = 0; e < 8; ++e) xr[xs][i][e] = src[e];
            }
        }
    };
    auto sstore_a = [&](int buf, auto X_) {
        constexpr int xs = decltype(X_)::value;
#pragma unroll
        for (int i = 0; i < PPT; ++i) {
            if (!pon[i]) continue;  // wave-uniform
            float bsum = 0.0f;
            uint32_t w[3][4];
#pragma unroll
            for (int e = 0; e < 8; e += 2) {
                const float x0 = xok[xs][i] ? xr[xs][i][e] : 0.0f;
                const float x1 = xok[xs][i] ? xr[xs][i][e + 1] : 0.0f;
                bsum += x0;
                bsum += x1;
                const uint32_t t0 = pk_bf16(x0, x1);
                const float r0 = x0 - bf16_lo_f32(t0), r1 = x1 - bf16_hi_f32(t0);
                const uint32_t t1 = pk_bf16(r0, r1);
                const uint32_t t2 = pk_bf16(r0 - bf16_lo_f32(t1), r1 - bf16_hi_f32(t1));
                w[0][e >> 1] = t0;
                w[1][e >> 1] = t1;
                w[2][e >> 1] = t2;
            }
            // the four k-octets of one (row, block) sit in lanes r, r+16, r+32, r+48
            bsum += __shfl_xor(bsum, 16);
            bsum += __shfl_xor(bsum, 32);
            {
#pragma unroll
                for (int tt = 0; tt < 3; ++tt)
                    *(v4i *)(&sA[buf][0][0][0][0] + pdst[i] + tt * MT * 1024) =
                        v4i{(int)w[tt][0], (int)w[tt][1], (int)w[tt][2], (int)w[tt][3]};
                if (pg[i] == 0) {
                    const uint32_t s0 = pk_bf16(bsum, 0.0f);
                    const float sr = bsum - bf16_lo_f32(s0);
                    const uint32_t s1 = pk_bf16(sr, 0.0f);
                    const uint32_t s2 = pk_bf16(sr - bf16_lo_f32(s1), 0.0f);
                    uint8_t *xm = &sXM[buf][0][prow[i] >> 4][0] + (prow[i] & 15) * 16 + pbl[i] * 2;
                    *(uint16_t *)(xm) = (uint16_t)s0;
                    *(uint16_t *)(xm + MT * 1024) = (uint16_t)s1;
                    *(uint16_t *)(xm + 2 * MT * 1024) = (uint16_t)s2;
                }
            }
        }
    };

    // ---- weight records.  Strips past the last read the last strip (their
    // columns are never stored); records past the range read the last record
    // of the range for codes and the header's zero tail for (d, m).
    const int strip_base = sg * SPG + wave * C;
    v4i bc[NSET][QC][C], bs[NSET][QC][C];
    auto gload_rec = [&](int quad, v4i (&dc)[C], v4i (&ds)[C]) {
        const int qq = min(quad, q1 - 1);
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int strip = min(strip_base + j, p.NS - 1);
            const uint8_t *rec = recs + ((int64_t)strip * p.NQ + qq) * kQ4RecBytes;
            const uint8_t *dmp = quad < q1 ? rec + 1024 + (uint32_t)(lane & 15) * 16u : hdr + kHeaderBytes - 16;
            dc[j] = *(const v4i *)(rec + (uint32_t)lane * 16u);
            ds[j] = *(const v4i *)dmp;
        }
    };

    v4f acc_y[MT][C], acc_m[MT][C];
#pragma unroll
    for (int rt = 0; rt < MT; ++rt)
#pragma unroll
        for (int j = 0; j < C; ++j) {
            acc_y[rt][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
            acc_m[rt][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }

    const int a_off = lane * 16;
    const int nchunk = (q1 - q0 + QC - 1) / QC;

    // One chunk: c = chunk index, buf = its LDS buffer, S = its weight set
    // (and activation set when XD > 1).  Chunk c + XD's activations (clamped
    // to the last chunk) and chunk c + NSET - 1's records are loaded first;
    // chunk c + 1's activations are split into LDS at the end.
    auto chunk = [&](int c, int buf, auto S_) {
        constexpr int S = decltype(S_)::value;
        constexpr int XS = XD == 1 ? 0 : S;
        const int qn = q0 + min(c + XD, nchunk - 1) * QC;
        if (NSET >= 2) {
            // unclamped: chunks past the range (the padding of the last
            // unrolled step) get d = m = 0
            constexpr int SN = (S + NSET - 1) % NSET;
#pragma unroll
            for (int q = 0; q < QC; ++q)
                gload_rec(q0 + (c + NSET - 1) * QC + q, bc[SN][q], bs[SN][q]);
        }
        gload_a(qn, ic<XS>{});
        v8bf a[ADB][MT][NF];
        auto lds_a = [&](int bl, v8bf (&ad)[MT][NF]) {
#pragma unroll
            for (int rt = 0; rt < MT; ++rt)
#pragma unroll
                for (int t = 0; t < NF; ++t) ad[rt][t] = *(const v8bf *)(&sA[buf][bl][t][rt][a_off]);
        };
        // m values of the chunk's blocks as bf16 pairs (k = block), packed
        // before the records' registers are refilled
        uint32_t mw[C][4];
#pragma unroll
        for (int j = 0; j < C; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) mw[j][t] = 0u;
        if (ADB == 2) lds_a(0, a[0]);
#pragma unroll
        for (int bl = 0; bl < BPC; ++bl) {
            const int q = bl >> 2, i = bl & 3;
            const int ab = ADB == 2 ? (bl & 1) : 0;
            if (ADB == 2) {
                if (bl + 1 < BPC) lds_a(bl + 1, a[(bl + 1) & 1]);
            } else {
                lds_a(bl, a[0]);
            }
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const v8bf bop = decode8((uint32_t)bc[S][q][j][i]);
                const float d = bf16_lo_f32((uint32_t)bs[S][q][j][i]);
#pragma unroll
                for (int rt = 0; rt < MT; ++rt) {
                    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                    for (int t = 0; t < NF; ++t)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[ab][rt][t], bop, acc, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc_y[rt][j][v] = fmaf(d, acc[v], acc_y[rt][j][v]);
                }
            }
            // pin the accumulators here: otherwise the compiler sinks every
            // block's update to the end of the chunk and keeps all the MFMA
            // results alive until then
#pragma unroll
            for (int rt = 0; rt < MT; ++rt)
#pragma unroll
                for (int j = 0; j < C; ++j) asm volatile("" : "+v"(acc_y[rt][j]));
            if (i == 3) {
#pragma unroll
                for (int j = 0; j < C; ++j) {
                    // high halves (m) of blocks (0, 1) and (2, 3) of the record
                    mw[j][2 * q] = __builtin_amdgcn_perm((uint32_t)bs[S][q][j][1], (uint32_t)bs[S][q][j][0], 0x07060302u);
                    mw[j][2 * q + 1] = __builtin_amdgcn_perm((uint32_t)bs[S][q][j][3], (uint32_t)bs[S][q][j][2], 0x07060302u);
                }
                if (NSET == 1) gload_rec(qn + q, bc[0][q], bs[0][q]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
#pragma unroll
        for (int rt = 0; rt < MT; ++rt) {
            v8bf xm[NF];
#pragma unroll
            for (int t = 0; t < NF; ++t) xm[t] = *(const v8bf *)(&sXM[buf][t][rt][lane * 16]);
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const v8bf mop = __builtin_bit_cast(v8bf, v4i{(int)mw[j][0], (int)mw[j][1], (int)mw[j][2], (int)mw[j][3]});
#pragma unroll
                for (int t = 0; t < NF; ++t)
                    acc_m[rt][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xm[t], mop, acc_m[rt][j], 0, 0, 0);
            }
        }
        sstore_a(buf ^ 1, ic<(XS + 1) % XD>{});
        __syncthreads();
    };

    if (nchunk > 0) {
        static_for<XD>([&](auto X_) { gload_a(q0 + min(decltype(X_)::value, nchunk - 1) * QC, X_); });
        static_for<(NSET > 1 ? NSET - 1 : 1)>([&](auto S_) {
            constexpr int st = decltype(S_)::value;
#pragma unroll
            for (int q = 0; q < QC; ++q) gload_rec(q0 + st * QC + q, bc[st][q], bs[st][q]);
        });
        sstore_a(0, ic<0>{});
    }
    __syncthreads();
    if (NSET == 1) {
        for (int c = 0; c < nchunk; ++c) chunk(c, c & 1, ic<0>{});
    } else {
        // steps of NSET chunks; the last step's chunks past the range have
        // records with d = m = 0
        for (int c = 0; c < nchunk; c += NSET)
            static_for<NSET>([&](auto J) {
                constexpr int j = decltype(J)::value;
                chunk(c + j, j & 1, J);
            });
    }

#pragma unroll
    for (int rt = 0; rt < MT; ++rt)
#pragma unroll
        for (int j = 0; j < C; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = rt * 16 + 4 * (lane >> 4) + v;
                const int n = (strip_base + j) * 16 + (lane & 15);
                if (row < nrows && n < p.N) {
                    const float val = acc_y[rt][j][v] + acc_m[rt][j][v];
                    if (p.S == 1) {
                        p.Y[(int64_t)row * p.ldy + n] = val;
                    } else {
                        p.part[((int64_t)job * p.M + row) * p.N + n] = val;
                    }
                }
            }
}

// ------------------------------------------------ the product, M <= 4 ---
// Decode-shaped product (at most 4 activation rows).  One MFMA 16-row tile
// holds the three bf16 terms of each row (rows 4m, 4m+1, 4m+2 of the tile),
// so a block and strip cost one MFMA.  A workgroup owns C strips and the
// whole k range, which its W wavefronts split: wavefront w takes records
// [w qpw, (w+1) qpw).  Each wavefront streams its records through a ring of
// D register slots (codes, (d, m) words and the record's 128 activations per
// row), so D records per strip are in flight; nothing waits on another
// wavefront until the end, where the W partial sums are added in wavefront
// order through LDS.  No second launch and no workspace.
//   * activations: each lane loads 16 bytes (4 values of one row) of the
//     record, splits them into the three bf16 terms and writes the terms to
//     the wavefront's own LDS area; a lane of the A operand (row 4m+t,
//     k-octet g) then reads its 8 terms of each block with one ds_read_b128.
//     LDS operations of one wavefront complete in order, so no barrier.
//   * m term: the lanes that split the activations also add them up per
//     block (own values, then a DPP reduction inside 8 or 16 lanes); one
//     lane per (row, block) writes the sum to the wavefront's LDS area and
//     every output lane (row m, column c) reads its row's four sums with one
//     ds_read_b128, so y += d (sum of the three d-term outputs) + m (sum).
//   * records past the wavefront's range read its last record for codes and
//     activations and the header's zero tail for (d, m): they add nothing.
//     Blocks past K in the last record have d = m = 0 in the packed layout;
//     their activation reads are clamped inside the row.
template <int W, int C, int D, int MR, bool XVEC>
__global__ __launch_bounds__(W * 64) void k_q4_gemv(Q4Params p) {
    static_assert(MR == 1 || MR == 2 || MR == 4, "activation rows per launch");
    // per wavefront: terms of the current record, [row][term][k] bf16, a
    // term plane padded to 160 elements (320 bytes) so that the (term,
    // k-octet) pieces one operand read touches sit in distinct bank groups.
    // A-operand lanes of absent rows read row M - 1 and those of the unused
    // fourth term read term 2: an MFMA output row depends on its own A row
    // only, and outputs of absent rows and of the fourth term are never used.
    constexpr int TP = 160;
    __shared__ __attribute__((aligned(16))) uint16_t sT[W][4][3][TP];
    __shared__ __attribute__((aligned(16))) float sXS[W][4][4];  // block sums [row][block] of the record
    __shared__ float sRed[W][C][64];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int strip0 = blockIdx.x * C;
    const int q0 = min(wave * p.qps, p.NQ);
    const int q1 = min(q0 + p.qps, p.NQ);
    const uint8_t *hdr = p.recs;
    const uint8_t *recs = hdr + kHeaderBytes;
    const int M = p.M;  // 1 .. MR

    // A operand lane: row 4 am + at of the tile, k-octet ag
    const int am = (lane & 15) >> 2, at = lane & 3, ag = lane >> 4;
    const int a_rd = ((am < M ? am : M - 1) * 3 + (at < 3 ? at : 2)) * TP + 8 * ag;  // element offset in sT[wave]
    // activation loads: XL values of row xrow at k = xk of the record
    constexpr int XL = MR == 1 ? 2 : 4;         // values per lane per load
    constexpr int XH = MR == 4 ? 2 : 1;         // loads per lane per record
    const int xk = MR == 1 ? 2 * lane : 4 * (lane & 31);

    v4i wc[D][C], wd[D][C];
    float xv[D][XH][XL];
    auto gload = [&](auto S, int q) {
        constexpr int s = decltype(S)::value;
        const bool pad = q >= q1;
        const int qq = min(q, q1 - 1);
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int strip = min(strip0 + j, p.NS - 1);
            const uint8_t *rec = recs + ((int64_t)strip * p.NQ + qq) * kQ4RecBytes;
            wc[s][j] = *(const v4i *)(rec + (uint32_t)lane * 16u);
            wd[s][j] = *(const v4i *)(pad ? hdr + kHeaderBytes - 16 : rec + 1024 + (uint32_t)(lane & 15) * 16u);
        }
        const int k = min(qq * 128 + xk, p.K - XL);
#pragma unroll
        for (int h = 0; h < XH; ++h) {
            const int row = MR == 1 ? 0 : min(2 * h + (lane >> 5), M - 1);
            const float *src = p.X + (int64_t)row * p.ldx + k;
            if (XVEC && XL == 4) {
                const v4f v = *(const v4f *)src;
#pragma unroll
                for (int e = 0; e < 4; ++e) xv[s][h][e] = v[e];
            } else if (XVEC) {
                const v2f v = *(const v2f *)src;
                xv[s][h][0] = v[0];
                xv[s][h][1] = v[1];
            } else {
#pragma unroll
                for (int e = 0; e < XL; ++e) xv[s][h][e] = src[e];
            }
        }
    };

    const v4f zero = {0.0f, 0.0f, 0.0f, 0.0f};
    // lanes of one (row, block) of the activation loads: 16 at one row (2
    // values each), 8 otherwise (4 values each); the last of them holds the sum
    constexpr int XG = MR == 1 ? 16 : 8;
    float y[C];
#pragma unroll
    for (int j = 0; j < C; ++j) y[j] = 0.0f;

    // record in slot S: stage its activation terms, then 4 blocks x (C + 1) MFMAs
    auto record = [&](auto S) {
        constexpr int s = decltype(S)::value;
#pragma unroll
        for (int h = 0; h < XH; ++h) {
            uint32_t t[3][XL / 2];
#pragma unroll
            for (int e = 0; e < XL; e += 2) {
                const float x0 = xv[s][h][e], x1 = xv[s][h][e + 1];
                const uint32_t t0 = pk_bf16(x0, x1);
                const float r0 = x0 - bf16_lo_f32(t0), r1 = x1 - bf16_hi_f32(t0);
                const uint32_t t1 = pk_bf16(r0, r1);
                t[0][e >> 1] = t0;
                t[1][e >> 1] = t1;
                t[2][e >> 1] = pk_bf16(r0 - bf16_lo_f32(t1), r1 - bf16_hi_f32(t1));
            }
            const int row = MR == 1 ? 0 : 2 * h + (lane >> 5);
#pragma unroll
            for (int tt = 0; tt < 3; ++tt) {
                if (XL == 4)
                    *(v2i *)(&sT[wave][row][tt][xk]) = v2i{(int)t[tt][0], (int)t[tt][1]};
                else
                    *(uint32_t *)(&sT[wave][row][tt][xk]) = t[tt][0];
            }
            float bs = xv[s][h][0];
#pragma unroll
            for (int e = 1; e < XL; ++e) bs += xv[s][h][e];
            // inclusive prefix sums inside each row of 16 lanes (row_shr 1, 2, 4, 8)
            bs += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bs), 0x111, 0xF, 0xF, true));
            bs += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bs), 0x112, 0xF, 0xF, true));
            bs += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bs), 0x114, 0xF, 0xF, true));
            if (XG == 16)
                bs += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bs), 0x118, 0xF, 0xF, true));
            if ((lane & (XG - 1)) == XG - 1) sXS[wave][row][(xk >> 5) & 3] = bs;
        }
        const v4f xs4 = *(const v4f *)(&sXS[wave][lane >> 4][0]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v8bf a = *(const v8bf *)(&sT[wave][0][0][0] + a_rd + 32 * i);
            const float xs = xs4[i];
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, decode8((uint32_t)wc[s][j][i]), zero, 0, 0, 0);
                const uint32_t dm = (uint32_t)wd[s][j][i];
                y[j] = fmaf(bf16_lo_f32(dm), (acc[0] + acc[1]) + acc[2], y[j]);
                y[j] = fmaf(bf16_hi_f32(dm), xs, y[j]);
            }
            // pin the sums here: otherwise the compiler sinks every block's
            // update to the end of the loop and keeps all MFMA results alive
#pragma unroll
            for (int j = 0; j < C; ++j) asm volatile("" : "+v"(y[j]));
        }
    };

    // steps of D records; the last step's records past the range are the
    // zero-weight padding described above (no load sits in a branch, so the
    // ring stays in flight)
    if (q0 < q1) {
        static_for<D>([&](auto S) { gload(S, q0 + decltype(S)::value); });
        for (int q = q0; q < q1; q += D) {
            static_for<D>([&](auto S) {
                record(S);
                gload(S, q + decltype(S)::value + D);
                // keep each record's work in its own step (hoisting the next
                // records' activation work ahead costs registers)
                __builtin_amdgcn_sched_barrier(0);
            });
        }
    }

    // y of lane (row lane >> 4, column lane & 15) of each strip; rows past M hold zeros
#pragma unroll
    for (int j = 0; j < C; ++j) sRed[wave][j][lane] = y[j];
    __syncthreads();
    for (int o = threadIdx.x; o < C * 64; o += W * 64) {
        const int j = o >> 6, l = o & 63;
        const int m = l >> 4;
        const int n = (strip0 + j) * 16 + (l & 15);
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) v += sRed[w][j][l];
        if (m < M && n < p.N && strip0 + j < p.NS) p.Y[(int64_t)m * p.ldy + n] = v;
    }
}

// M = 1 with at most QMAX records per wavefront: the same split of the k
// range as k_q4_gemv, but each wavefront stages the activation terms and
// block sums of its whole k range (at most 128 QMAX values) once; their loads
// go out first (they come from L2, ahead of the records' HBM traffic).  A
// record's remaining work is per block one LDS operand read, the code decode,
// one MFMA and two fma.  Every record of the wavefront is loaded at the start,
// so a wavefront whose data comes late has little left to do; the fewer
// records per wavefront, the shorter that tail (4 where the planner can).
template <int W, int QMAX, bool XVEC>
__global__ __launch_bounds__(W * 64) void k_q4_gemv1(Q4Params p) {
    static_assert(QMAX == 4 || QMAX == 8, "records per wavefront");
    constexpr int D = QMAX;
    constexpr int XPL = QMAX * 128 / 64;  // activation values per lane
    // term planes of the range padded by 64 bytes (a plane is 256 QMAX bytes,
    // so the stride is 64 mod 256): the (term, k-octet) pieces of one operand
    // read sit in distinct bank groups.  Lanes of the unused fourth term read
    // term 2 and rows 1..3 of the tile repeat row 0 (outputs never used).
    constexpr int TPL = QMAX * 128 + 32;
    __shared__ __attribute__((aligned(16))) uint16_t sT[W][3][TPL];
    __shared__ __attribute__((aligned(16))) float sXS[W][QMAX * 4];  // block sums of the range
    __shared__ float sRed[W][16];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int strip = min((int)blockIdx.x, p.NS - 1);
    const int q0 = min(wave * p.qps, p.NQ);
    const int q1 = min(q0 + p.qps, p.NQ);
    const uint8_t *hdr = p.recs;
    const uint8_t *recs = hdr + kHeaderBytes;

    v4i wc[D], wd[D];
    auto gload = [&](auto S, int q) {
        constexpr int s = decltype(S)::value;
        const bool pad = q >= q1;
        const int qq = min(q, q1 - 1);
        const uint8_t *rec = recs + ((int64_t)strip * p.NQ + qq) * kQ4RecBytes;
        // non-temporal: each record is read once (4096 x 14336: 9.5 -> 8.9 us)
        wc[s] = __builtin_nontemporal_load((const v4i *)(rec + (uint32_t)lane * 16u));
        wd[s] = __builtin_nontemporal_load(
            (const v4i *)(pad ? hdr + kHeaderBytes - 16 : rec + 1024 + (uint32_t)(lane & 15) * 16u));
    };
    float y = 0.0f;
    if (q0 < q1) {
        // activations k0 + XPL L .. + XPL - 1 of the range (clamped inside the
        // row: values past the range or past K meet zero-weight records or blocks)
        const int k = min(q0 * 128 + XPL * lane, p.K - XPL);
        float x[XPL];
        if (XVEC) {
#pragma unroll
            for (int u = 0; u < XPL / 4; ++u) {
                const v4f v = *(const v4f *)(p.X + k + 4 * u);
                x[4 * u] = v[0]; x[4 * u + 1] = v[1]; x[4 * u + 2] = v[2]; x[4 * u + 3] = v[3];
            }
        } else {
#pragma unroll
            for (int e = 0; e < XPL; ++e) x[e] = p.X[k + e];
        }
        __builtin_amdgcn_sched_barrier(0);
        static_for<D>([&](auto S) { gload(S, q0 + decltype(S)::value); });
        __builtin_amdgcn_sched_barrier(0);
        uint32_t t[3][XPL / 2];
        float bs = 0.0f;
#pragma unroll
        for (int e = 0; e < XPL; e += 2) {
            const float x0 = x[e], x1 = x[e + 1];
            bs += x0;
            bs += x1;
            const uint32_t t0 = pk_bf16(x0, x1);
            const float r0 = x0 - bf16_lo_f32(t0), r1 = x1 - bf16_hi_f32(t0);
            const uint32_t t1 = pk_bf16(r0, r1);
            t[0][e >> 1] = t0;
            t[1][e >> 1] = t1;
            t[2][e >> 1] = pk_bf16(r0 - bf16_lo_f32(t1), r1 - bf16_hi_f32(t1));
        }
#pragma unroll
        for (int tt = 0; tt < 3; ++tt)
#pragma unroll
            for (int u = 0; u < XPL / 8; ++u)
                *(v4i *)(&sT[wave][tt][XPL * lane + 8 * u]) =
                    v4i{(int)t[tt][4 * u], (int)t[tt][4 * u + 1], (int)t[tt][4 * u + 2], (int)t[tt][4 * u + 3]};
        // a block (32 values) is 32 / XPL lanes: the last of them holds the sum
        bs += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bs), 0x111, 0xF, 0xF, true));
        if (XPL == 8)
            bs += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bs), 0x112, 0xF, 0xF, true));
        constexpr int LPB = 32 / XPL;
        if ((lane & (LPB - 1)) == LPB - 1) sXS[wave][lane / LPB] = bs;

        // A operand lane: term at (<= 2) of row 0, k-octet ag
        const int at = lane & 3, ag = lane >> 4;
        const int a_rd = (at < 3 ? at : 2) * TPL + 8 * ag;
        auto record = [&](auto S, int qi) {
            constexpr int s = decltype(S)::value;
            const v4f xs4 = *(const v4f *)(&sXS[wave][4 * qi]);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v8bf a = *(const v8bf *)(&sT[wave][0][0] + a_rd + qi * 128 + 32 * i);
                const v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, decode8((uint32_t)wc[s][i]),
                                                                       v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                const uint32_t dm = (uint32_t)wd[s][i];
                y = fmaf(bf16_lo_f32(dm), (acc[0] + acc[1]) + acc[2], y);
                y = fmaf(bf16_hi_f32(dm), xs4[i], y);
                asm volatile("" : "+v"(y));
            }
        };
        static_for<D>([&](auto S) { record(S, decltype(S)::value); });
    }

    // lanes 0..15 hold the columns (row 0 of the tile's output rows 0..3)
    if (lane < 16) sRed[wave][lane] = y;
    __syncthreads();
    if (threadIdx.x < 16) {
        float v = 0.0f;
#pragma unroll
        for (int w = 0; w < W; ++w) v += sRed[w][threadIdx.x];
        const int n = strip * 16 + (int)threadIdx.x;
        if ((int)blockIdx.x < p.NS && n < p.N) p.Y[n] = v;
    }
}

// M = 1 over many strips with at most 8 records each (K <= 1024, e.g. an
// lm_head): 8 wavefronts per workgroup, each owning one 16-column strip over
// its whole k range, so the activation terms and block sums are staged once
// per workgroup for 8 strips (k_q4_gemv1 stages them once per strip) and no
// wavefront's partial sum meets another's.  Wavefronts 0 and 1 stage records
// 0-3 and 4-7 with k_q4_gemv1's rule (three bf16 terms, the same padded term
// planes and block sums), one barrier, then every wavefront runs the records
// of its strip, all loaded at the start, with k_q4_gemv1's per-block
// arithmetic (one fma chain over the whole k range: no partial sums).
template <bool XVEC>
__global__ __launch_bounds__(512) void k_q4_gemv1_wide(Q4Params p) {
    constexpr int W = 8, QMAX = 8, D = QMAX, XPL = 8;
    constexpr int TPL = QMAX * 128 + 32;
    __shared__ __attribute__((aligned(16))) uint16_t sT[3][TPL];
    __shared__ __attribute__((aligned(16))) float sXS[QMAX * 4];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int strip_raw = (int)blockIdx.x * W + wave;
    const int strip = min(strip_raw, p.NS - 1);
    const int nq = p.NQ;
    const uint8_t *hdr = p.recs;
    const uint8_t *recs = hdr + kHeaderBytes;

    // staging: wavefront w < 2 takes activations 512 w + 8 L .. + 7 (clamped
    // inside the row: values past K meet zero-weight blocks)
    float x[XPL];
    if (wave < 2) {
        const int k = min(512 * wave + XPL * lane, p.K - XPL);
        if (XVEC) {
#pragma unroll
            for (int u = 0; u < XPL / 4; ++u) {
                const v4f v = *(const v4f *)(p.X + k + 4 * u);
                x[4 * u] = v[0]; x[4 * u + 1] = v[1]; x[4 * u + 2] = v[2]; x[4 * u + 3] = v[3];
            }
        } else {
#pragma unroll
            for (int e = 0; e < XPL; ++e) x[e] = p.X[k + e];
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    v4i wc[D], wd[D];
    static_for<D>([&](auto S) {
        constexpr int q = decltype(S)::value;
        const bool pad = q >= nq;
        const uint8_t *rec = recs + ((int64_t)strip * nq + min(q, nq - 1)) * kQ4RecBytes;
        // non-temporal: each record is read once (19.5 -> 18.1 us on the lm_head)
        wc[q] = __builtin_nontemporal_load((const v4i *)(rec + (uint32_t)lane * 16u));
        wd[q] = __builtin_nontemporal_load(
            (const v4i *)(pad ? hdr + kHeaderBytes - 16 : rec + 1024 + (uint32_t)(lane & 15) * 16u));
    });
    __builtin_amdgcn_sched_barrier(0);
    if (wave < 2) {
        uint32_t t[3][XPL / 2];
        float bs = 0.0f;
#pragma unroll
        for (int e = 0; e < XPL; e += 2) {
            const float x0 = x[e], x1 = x[e + 1];
            bs += x0;
            bs += x1;
            const uint32_t t0 = pk_bf16(x0, x1);
            const float r0 = x0 - bf16_lo_f32(t0), r1 = x1 - bf16_hi_f32(t0);
            const uint32_t t1 = pk_bf16(r0, r1);
            t[0][e >> 1] = t0;
            t[1][e >> 1] = t1;
            t[2][e >> 1] = pk_bf16(r0 - bf16_lo_f32(t1), r1 - bf16_hi_f32(t1));
        }
#pragma unroll
        for (int tt = 0; tt < 3; ++tt)
#pragma unroll
            for (int u = 0; u < XPL / 8; ++u)
                *(v4i *)(&sT[tt][512 * wave + XPL * lane + 8 * u]) =
                    v4i{(int)t[tt][4 * u], (int)t[tt][4 * u + 1], (int)t[tt][4 * u + 2], (int)t[tt][4 * u + 3]};
        // a block (32 values) is 4 lanes: the last of them holds the sum
        bs += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bs), 0x111, 0xF, 0xF, true));
        bs += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, bs), 0x112, 0xF, 0xF, true));
        if ((lane & 3) == 3) sXS[16 * wave + lane / 4] = bs;
    }
    // LDS barrier without a memory fence (the record loads stay in flight)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    float y = 0.0f;
    const int at = lane & 3, ag = lane >> 4;
    const int a_rd = (at < 3 ? at : 2) * TPL + 8 * ag;
    static_for<D>([&](auto S) {
        constexpr int qi = decltype(S)::value;
        const v4f xs4 = *(const v4f *)(&sXS[4 * qi]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const v8bf a = *(const v8bf *)(&sT[0][0] + a_rd + qi * 128 + 32 * i);
            const v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, decode8((uint32_t)wc[qi][i]),
                                                                   v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
            const uint32_t dm = (uint32_t)wd[qi][i];
            y = fmaf(bf16_lo_f32(dm), (acc[0] + acc[1]) + acc[2], y);
            y = fmaf(bf16_hi_f32(dm), xs4[i], y);
            asm volatile("" : "+v"(y));
        }
    });
    // lanes 0..15 hold the strip's columns (row 0 of the tile)
    const int n = strip * 16 + lane;
    if (lane < 16 && strip_raw < p.NS && n < p.N) p.Y[n] = y;
}

// ------------------- staging shared by the 16-row whole-range kernels ---
// k_q4_mm16 and k_q4_mm16_wide (8 wavefronts) split the activations of their
// whole k range (32 blocks from block b0) into LDS once.  Each wavefront
// owns two rows, r = 2 wave + lane / 32; piece p = (block p / 4, k-octet
// p % 4) of its row is 8 activations, and lane L holds pieces L % 32 + 32 i,
// so a row's maximum, scale and block sums never leave its wavefront (no
// barrier before the split).  Rows past M read row M - 1 (they reach only
// outputs that are never stored) and blocks past K read the last block,
// whose copies meet zero (d, m) in the padded records, so no value needs
// masking: the row maxima and the products of the real rows and blocks are
// those of the real values.
template <int PPT, bool XVEC>
__device__ __forceinline__ void load_pieces16(const float *X, int64_t ldx, int M, int NB, int lane, int wave,
                                              int b0, float (&xr)[PPT][8]) {
    const int r = 2 * wave + (lane >> 5);
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int pc = (lane & 31) + 32 * i;
        const int g = pc & 3, bl = pc >> 2;
        const int b = b0 + bl;
        const float *src = X + (int64_t)min(r, M - 1) * ldx + min(b, NB - 1) * 32 + g * 8;
        if (XVEC) {
            const v4f lo = *(const v4f *)src;
            const v4f hi = *(const v4f *)(src + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                xr[i][e] = lo[e];
                xr[i][4 + e] = hi[e];
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) xr[i][e] = src[e];
        }
    }
}

// The split of the held pieces: the row's scale exponent sc (sc = 15 - e for
// max |x| = f 2^e, f in [0.5, 1); into s_sc[row] for the epilogue), then the
// two fp16 terms of x 2^sc at sA[bl][term] in MFMA lane order and the
// unscaled block sums (the four k-octets of a block lie in four consecutive
// lanes), three bf16 terms, into the m-term operands sXM (row r, block bl at
// byte 16 r + 2 (bl % 8) of sXM[bl / 8]; k-octets 1..3 of each operand stay
// zero).  Ends with an LDS-only barrier (no memory fence: record loads may
// be in flight).
template <int WAVES, int NBLK, int PPT>
__device__ __forceinline__ void stage16(int tid, int lane, int wave, const float (&xr)[PPT][8],
                                        uint8_t (*sA)[2][1024], uint8_t (*sXM)[3][1024], int *s_sc) {
    static_assert(WAVES == 8 && NBLK * 4 == 32 * PPT, "two rows per wavefront, 32 lanes a row");
    constexpr int NT = WAVES * 64;
    constexpr int NG = (NBLK + 7) / 8;
    for (int o = tid * 16; o < NG * 3 * 768; o += NT * 16) {
        const int f = o / 768;
        *(v4i *)(&sXM[0][0][0] + f * 1024 + 256 + o % 768) = v4i{0, 0, 0, 0};
    }
    const int r = 2 * wave + (lane >> 5);
    float am = 0.0f;
#pragma unroll
    for (int i = 0; i < PPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(xr[i][e]));
#pragma unroll
    for (int m = 16; m >= 1; m >>= 1) am = fmaxf(am, __shfl_xor(am, m));
    const int sc = am > 0.0f ? 15 - __builtin_amdgcn_frexp_expf(am) : 0;
    if ((lane & 31) == 0) s_sc[r] = sc;
#pragma unroll
    for (int i = 0; i < PPT; ++i) {
        const int pc = (lane & 31) + 32 * i;
        const int g = pc & 3, bl = pc >> 2;
        float bsum = 0.0f;
        uint32_t w[2][4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float x0 = xr[i][e];
            const float x1 = xr[i][e + 1];
            bsum += x0;
            bsum += x1;
            const float s0 = __builtin_ldexpf(x0, sc), s1 = __builtin_ldexpf(x1, sc);
            const v2h a0 = {(_Float16)s0, (_Float16)s1};
            const v2h a1 = {(_Float16)(s0 - (float)a0[0]), (_Float16)(s1 - (float)a0[1])};
            w[0][e >> 1] = __builtin_bit_cast(uint32_t, a0);
            w[1][e >> 1] = __builtin_bit_cast(uint32_t, a1);
        }
        bsum += __shfl_xor(bsum, 1);
        bsum += __shfl_xor(bsum, 2);
#pragma unroll
        for (int t = 0; t < 2; ++t)
            *(v4i *)(&sA[bl][t][(g * 16 + r) * 16]) = v4i{(int)w[t][0], (int)w[t][1], (int)w[t][2], (int)w[t][3]};
        if (g == 0) {
            const uint32_t s0 = pk_bf16(bsum, 0.0f);
            const float sr = bsum - bf16_lo_f32(s0);
            const uint32_t s1 = pk_bf16(sr, 0.0f);
            const uint32_t s2 = pk_bf16(sr - bf16_lo_f32(s1), 0.0f);
            uint8_t *xm = &sXM[bl >> 3][0][r * 16 + (bl & 7) * 2];
            *(uint16_t *)(xm) = (uint16_t)s0;
            *(uint16_t *)(xm + 1024) = (uint16_t)s1;
            *(uint16_t *)(xm + 2048) = (uint16_t)s2;
        }
    }
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// ----------------------------------------- the product, 5 <= M <= 16 ---
// One 16-row MFMA tile of activation rows, two MFMAs (one per fp16 term)
// per block and strip.  A workgroup of WAVES wavefronts owns
// WAVES * C strips and a k range of at most QMAX records; the grid splits
// the k range S ways and k_q4_finalize adds the S partial sums.  What
// differs from k_q4_mm is the order of the work: the workgroup splits the
// activations of its whole k range into LDS once, right at the start (every
// wavefront's activation loads are issued before any record load), and the
// records then stream through a ring of R register slots per wavefront with
// no barrier after the staging one.  (Chunk by chunk, each chunk's
// activation loads, split and barrier sat between the weight loads and the
// MFMAs.)
//   * staging: piece (block bl, k-octet g, row r) = 8 activations, loaded
//     with two 16-byte loads ahead of the record loads.  Each row first
//     gets a power-of-two scale over the workgroup's k range (sc = 15 - e,
//     max |x| = f 2^e, f in [0.5, 1); a row's pieces all sit in one
//     wavefront, so no barrier precedes the split): every x 2^sc lies below
//     2^15, and its two fp16 terms h0 = fp16(x 2^sc), h1 = fp16(x 2^sc - h0)
//     hold it to ~2^-22 relative (the scaling and the subtraction are
//     exact).  The terms are stored at sA[bl][term] in MFMA lane order (lane
//     16 g + r), against the exact fp16 codes; the epilogue multiplies the
//     d term by 2^-sc (each k split undoes its own scale).  Rows past M and
//     blocks past K stage copies of row M - 1 and of the last block (outputs
//     never stored; zero (d, m)).  The (unscaled) block
//     sums (the four k-octets of a (row, block) lie in lanes r, r+16, r+32,
//     r+48 of one wavefront) are split the same way into the m-term A
//     operand: row r, block bl at byte 16 r + 2 (bl % 8) of sXM[bl / 8].
//   * records past the workgroup's range take the last record's codes and
//     the header's zero tail for (d, m): they add nothing.
template <int WAVES, int C, int QMAX, int R, bool XVEC>
__global__ __launch_bounds__(WAVES * 64) void k_q4_mm16(Q4Params p) {
    constexpr int NT = WAVES * 64;
    constexpr int NBLK = 4 * QMAX;
    constexpr int NG = (NBLK + 7) / 8;  // m-term operands of 8 blocks
    constexpr int PIECES = NBLK * 64;
    static_assert(PIECES % NT == 0 && NBLK % 8 == 0, "pieces per thread");
    static_assert(R >= 1 && R <= QMAX, "record ring");
    constexpr int PPT = PIECES / NT;
    constexpr int SPG = WAVES * C;
    __shared__ __attribute__((aligned(16))) uint8_t sA[NBLK][2][1024];
    __shared__ __attribute__((aligned(16))) uint8_t sXM[NG][3][1024];
    __shared__ int s_sc[16];  // the rows' scale exponents

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int groups = (p.NS + SPG - 1) / SPG;
    const int sg = blockIdx.x % groups;
    const int job = blockIdx.x / groups;
    const int q0 = job * p.qps;
    const int q1 = min(p.NQ, q0 + p.qps);
    const int M = p.M;
    const uint8_t *hdr = p.recs;
    const uint8_t *recs = hdr + kHeaderBytes;

    // ---- activation loads (first: the staging waits for them alone)
    float xr[PPT][8];
    load_pieces16<PPT, XVEC>(p.X, p.ldx, M, p.NB, lane, wave, q0 * 4, xr);

    // every wavefront's activation loads go out before any record load: the
    // memory pipeline returns them in order, and the staging needs them first
    __builtin_amdgcn_s_barrier();
    // ---- the wavefront's records in k order, through a ring of R slots:
    // the first R now, record q + R as soon as record q is used
    const int strip_base = sg * SPG + wave * C;
    v4i wc[R][C], wd[R][C];
    auto gload_rec = [&](int q, v4i (&dc)[C], v4i (&dd)[C]) {
        const int qq = min(q0 + q, q1 - 1);
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int strip = min(strip_base + j, p.NS - 1);
            const uint8_t *rec = recs + ((int64_t)strip * p.NQ + qq) * kQ4RecBytes;
            // non-temporal: each record is read once (measured 4 % faster
            // at M = 16; the hint made the M = 1 kernels no faster)
            dc[j] = __builtin_nontemporal_load((const v4i *)(rec + (uint32_t)lane * 16u));
            dd[j] = __builtin_nontemporal_load((const v4i *)(q0 + q < q1 ? rec + 1024 + (uint32_t)(lane & 15) * 16u : hdr + kHeaderBytes - 16));
        }
    };
#pragma unroll
    for (int q = 0; q < R; ++q) gload_rec(q, wc[q], wd[q]);

    // ---- staging (its last barrier is LDS-only: a memory fence would wait
    // for the record loads still in flight)
    stage16<WAVES, NBLK, PPT>(tid, lane, wave, xr, sA, sXM, s_sc);

    // ---- the product
    v4f acc_y[C], acc_m[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
        acc_y[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
        acc_m[j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int a_off = lane * 16;
    uint32_t mw[2][C][2];  // m values of the last two records, bf16 pairs (k = block)
#pragma unroll
    for (int q = 0; q < QMAX; ++q) {
        const int sl = q % R;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int bl = 4 * q + i;
            v8h a[2];
#pragma unroll
            for (int t = 0; t < 2; ++t) a[t] = *(const v8h *)(&sA[bl][t][a_off]);
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const v8h bop = decode8h((uint32_t)wc[sl][j][i]);
                const float d = bf16_lo_f32((uint32_t)wd[sl][j][i]);
                v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = 0; t < 2; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], bop, acc, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc_y[j][v] = fmaf(d, acc[v], acc_y[j][v]);
            }
            // keep each block's update here (else the compiler sinks them all
            // to the end and keeps every MFMA result alive)
#pragma unroll
            for (int j = 0; j < C; ++j) asm volatile("" : "+v"(acc_y[j]));
        }
        // the record's m values (high halves of its four (d, m) words), then
        // its slot takes record q + R
#pragma unroll
        for (int j = 0; j < C; ++j) {
            mw[q & 1][j][0] = __builtin_amdgcn_perm((uint32_t)wd[sl][j][1], (uint32_t)wd[sl][j][0], 0x07060302u);
            mw[q & 1][j][1] = __builtin_amdgcn_perm((uint32_t)wd[sl][j][3], (uint32_t)wd[sl][j][2], 0x07060302u);
        }
        if (q + R < QMAX) gload_rec(q + R, wc[sl], wd[sl]);
        if (q & 1) {
            // m term of records q-1 and q: their 8 m values (k = block) against
            // the split block sums
            v8bf xm[3];
#pragma unroll
            for (int t = 0; t < 3; ++t) xm[t] = *(const v8bf *)(&sXM[q >> 1][t][a_off]);
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const v4i mv = {(int)mw[0][j][0], (int)mw[0][j][1], (int)mw[1][j][0], (int)mw[1][j][1]};
                const v8bf mop = __builtin_bit_cast(v8bf, mv);
#pragma unroll
                for (int t = 0; t < 3; ++t)
                    acc_m[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xm[t], mop, acc_m[j], 0, 0, 0);
            }
        }
    }

    int esc[4];  // -sc of this lane's output rows
#pragma unroll
    for (int v = 0; v < 4; ++v) esc[v] = -s_sc[4 * (lane >> 4) + v];
#pragma unroll
    for (int j = 0; j < C; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = 4 * (lane >> 4) + v;
            const int n = (strip_base + j) * 16 + (lane & 15);
            if (row < M && n < p.N) {
                const float val = __builtin_ldexpf(acc_y[j][v], esc[v]) + acc_m[j][v];
                if (p.S == 1)
                    p.Y[(int64_t)row * p.ldy + n] = val;
                else
                    p.part[((int64_t)job * M + row) * p.N + n] = val;
            }
        }
}

// 5 <= M <= 16 over many strips with at most 8 records each (K <= 1024,
// e.g. an lm_head): a persistent form of k_q4_mm16.  The grid is at most one
// workgroup per CU; workgroup b of G owns a contiguous run of NS / G or
// NS / G + 1 strips, stages the activations of the whole k range once
// (stage16) and each wavefront then runs the strips first + wave,
// first + wave + WAVES, ... one at a time over their whole k range (per
// block two fp16 MFMAs and y += d acc, the m term per two records, the
// strip's outputs stored straight to Y: no k split).  The records stream
// through 8 register slots: slot q holds record q of the current strip and,
// once its four blocks are used, takes record q of the wavefront's next
// strip, so the next strip's loads are in flight while the current one is
// multiplied.  (k_q4_mm16 over more strips than CUs x 16 runs more
// workgroups than CUs, and each of them stages the same activations again.)
template <int WAVES, bool XVEC>
__global__ __launch_bounds__(WAVES * 64) void k_q4_mm16_wide(Q4Params p) {
    constexpr int NT = WAVES * 64, QMAX = 8, NBLK = 4 * QMAX, NG = NBLK / 8;
    static_assert(NBLK * 64 % NT == 0, "pieces per thread");
    constexpr int PPT = NBLK * 64 / NT;
    __shared__ __attribute__((aligned(16))) uint8_t sA[NBLK][2][1024];
    __shared__ __attribute__((aligned(16))) uint8_t sXM[NG][3][1024];
    __shared__ int s_sc[16];  // the rows' scale exponents

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // workgroup b of G: NS / G strips, one more for b < NS % G
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    const int sq = p.NS / G, sr = p.NS % G;
    const int first = b * sq + min(b, sr);
    const int cnt = sq + (b < sr ? 1 : 0);
    const int nst = max(0, (cnt - wave + WAVES - 1) / WAVES);  // this wavefront's strips
    const int nq = p.NQ;
    const uint8_t *hdr = p.recs;
    const uint8_t *recs = hdr + kHeaderBytes;

    float xr[PPT][8];
    load_pieces16<PPT, XVEC>(p.X, p.ldx, p.M, p.NB, lane, wave, 0, xr);
    // every wavefront's activation loads go out before any record load
    __builtin_amdgcn_s_barrier();

    // records past the k range take the last record's codes and the header's
    // zero tail for (d, m): they add nothing
    v4i wc[QMAX], wd[QMAX];
    auto gload = [&](int st, int q, v4i &dc, v4i &dd) {
        const uint8_t *rec = recs + ((int64_t)st * nq + min(q, nq - 1)) * kQ4RecBytes;
        dc = __builtin_nontemporal_load((const v4i *)(rec + (uint32_t)lane * 16u));
        dd = __builtin_nontemporal_load(
            (const v4i *)(q < nq ? rec + 1024 + (uint32_t)(lane & 15) * 16u : hdr + kHeaderBytes - 16));
    };
    int strip = min(first + wave, p.NS - 1);
    static_for<QMAX>([&](auto Q) {
        constexpr int q = decltype(Q)::value;
        gload(strip, q, wc[q], wd[q]);
    });

    stage16<WAVES, NBLK, PPT>(tid, lane, wave, xr, sA, sXM, s_sc);

    int esc[4];  // -sc of this lane's output rows
#pragma unroll
    for (int v = 0; v < 4; ++v) esc[v] = -s_sc[4 * (lane >> 4) + v];
    const int a_off = lane * 16;

    // one strip; NEXT: refill each slot with the same record of the
    // wavefront's next strip (inlined: the slots must stay in registers)
    auto run_strip = [&](auto NEXT) __attribute__((always_inline)) {
        constexpr bool next = decltype(NEXT)::value;
        const int ahead = strip + WAVES;
        v4f acc_y = {0.0f, 0.0f, 0.0f, 0.0f}, acc_m = {0.0f, 0.0f, 0.0f, 0.0f};
        uint32_t mw[2][2];  // m values of the last two records, bf16 pairs (k = block)
        static_for<QMAX>([&](auto Q) {
            constexpr int q = decltype(Q)::value;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int bl = 4 * q + i;
                v8h a[2];
#pragma unroll
                for (int t = 0; t < 2; ++t) a[t] = *(const v8h *)(&sA[bl][t][a_off]);
                const v8h bop = decode8h((uint32_t)wc[q][i]);
                const float d = bf16_lo_f32((uint32_t)wd[q][i]);
                v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int t = 0; t < 2; ++t) acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t], bop, acc, 0, 0, 0);
#pragma unroll
                for (int v = 0; v < 4; ++v) acc_y[v] = fmaf(d, acc[v], acc_y[v]);
                asm volatile("" : "+v"(acc_y));
            }
            mw[q & 1][0] = __builtin_amdgcn_perm((uint32_t)wd[q][1], (uint32_t)wd[q][0], 0x07060302u);
            mw[q & 1][1] = __builtin_amdgcn_perm((uint32_t)wd[q][3], (uint32_t)wd[q][2], 0x07060302u);
            if constexpr (next) gload(ahead, q, wc[q], wd[q]);
            if constexpr ((q & 1) != 0) {
                v8bf xm[3];
#pragma unroll
                for (int t = 0; t < 3; ++t) xm[t] = *(const v8bf *)(&sXM[q >> 1][t][a_off]);
                const v4i mv = {(int)mw[0][0], (int)mw[0][1], (int)mw[1][0], (int)mw[1][1]};
                const v8bf mop = __builtin_bit_cast(v8bf, mv);
#pragma unroll
                for (int t = 0; t < 3; ++t) acc_m = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xm[t], mop, acc_m, 0, 0, 0);
            }
        });
        const int n = strip * 16 + (lane & 15);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = 4 * (lane >> 4) + v;
            if (row < p.M && n < p.N) p.Y[(int64_t)row * p.ldy + n] = __builtin_ldexpf(acc_y[v], esc[v]) + acc_m[v];
        }
        strip += WAVES;
    };
    for (int i = 0; i + 1 < nst; ++i) run_strip(std::true_type{});
    if (nst > 0) run_strip(std::false_type{});
}

// Sum of the k-split partials in split order.  Loads go out eight at a time
// (independent, clamped to the last split; extra ones are not added) so that
// a thread waits for one memory latency per eight splits, not per split.
__global__ __launch_bounds__(256) void k_q4_finalize(const float *__restrict__ part, int S, int M, int N,
                                                     float *__restrict__ Y, int64_t ldy) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)M * N) return;
    const int64_t m = gid / N, n = gid % N;
    const int64_t stride = (int64_t)M * N;
    float acc = 0.0f;
    for (int s0 = 0; s0 < S; s0 += 8) {
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = part[min(s0 + u, S - 1) * stride + gid];
#pragma unroll
        for (int u = 0; u < 8; ++u)
            if (s0 + u < S) acc += v[u];
    }
    Y[m * ldy + n] = acc;
}

// -------------------------------------------------- grouped MoE product ---
// One workgroup per (chunk of <= 32 rows of one expert, group of WAVES * C
// strips); chunks come from the routing table, past-the-end workgroups exit.
// The activations arrive split (k_moe_route's other workgroups): per chunk
// (one record, four blocks) the workgroup gathers its rows' 16-byte pieces
// of the split buffers (each lane its own row's address) into registers,
// three fragments per wavefront, together with the next record, and stores
// them into the other stage of a two-stage LDS ring at the end of the
// chunk; one barrier per chunk.  (A global_load_lds copy made the compiler
// wait for every load in flight before the stage's reads.)
//   * d term, per block, strip and 16-row tile: two MFMAs
//     (v_mfma_f32_16x16x32_f16: the fp16 terms against the exact fp16
//     codes) into a fresh accumulator, then y += d * acc;
//   * m term, per record, strip and tile: one bf16 MFMA, accumulated into
//     y, whose A operand holds the three bf16 terms of the record's four
//     block sums in k-octets 0, 1, 2 (k = 8 term + block; the rest zero) and
//     whose B operand holds the record's four m values in every k-octet;
//   * the epilogue undoes the token's scale: Y = y * 2^-sc[t].
// Rows past the chunk repeat its last row (their outputs are not stored);
// blocks past K read the last block (their d = m = 0).  A chunk of <= 16
// rows runs a one-tile copy of the whole job, chosen at kernel entry; inside
// a copy every tile is multiplied: no branch may sit between an MFMA and the
// VALU instructions that read its result.  A VALU read of an MFMA
// destination needs wait states the hardware does not enforce (the compiler
// emits 8 for v_mfma_f32_16x16x32_f16 on straight-line code), and with a
// wave-uniform branch skipping the second tile's MFMAs, the built code read
// the first tile's accumulator one instruction after its MFMA on the
// branch-taken path (the wait was only on the fall-through path), so every
// chunk of <= 16 rows summed stale accumulator registers.
// One job's product with MT 16-row tiles.
constexpr int kMoeTileRows = 16;
template <int MT, int WAVES, int C, bool PER_SLOT>
__device__ __forceinline__ void moe_job(const Q4Params &p, uint8_t *sS0, uint8_t *sS1, const int *sTok,
                                        const int64_t *sYoff, const int *sYexp, int sg, int expert, int nrows) {
    constexpr int SPG = WAVES * C;
    constexpr int NFD = 4 * 2 * MT;  // d-term fragments per chunk: block x term x tile
    constexpr int NFM = MT;          // m-term fragments: one per tile
    constexpr int FPW = (NFD + NFM + WAVES - 1) / WAVES;  // fragments copied per wavefront
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint8_t *hdr = p.recs + (int64_t)expert * p.expert_stride;
    const uint8_t *recs = hdr + kHeaderBytes;
    const int NQ = p.NQ;

    // ---- gather sources: fragment f = wave + WAVES i of the stage (clamped:
    // the wavefronts with fewer fragments store the last one again, the same
    // bytes to the same place); d term f = (block * 2 + term) * MT + tile,
    // m term f - NFD = tile.  Lane (row r, k-octet g) of a tile.  Every load
    // of the loop is a uniform base (the buffer and the record's offset,
    // scalar registers) plus a per-lane 32-bit offset fixed for the job (the
    // lane's row and k-octet): no vector address arithmetic per record.  A
    // record's block-sum entry is 64 bytes, 16 per k-octet: term g's four
    // sums and 8 zero bytes for g < 3, zeros for g = 3.
    const int r = lane & 15, g = lane >> 4;
    const int a_off = lane * 16;
    uint32_t fvoff[FPW];
    int foff[FPW], fblk[FPW];
    bool fisd[FPW];
#pragma unroll
    for (int i = 0; i < FPW; ++i) {
        const int f = min(wave + WAVES * i, NFD + NFM - 1);
        foff[i] = f * 1024;
        const bool isd = f < NFD;
        const int u = (f / MT) & 1;
        const int tile = isd ? f % MT : f - NFD;
        const uint32_t tok = (uint32_t)sTok[tile * 16 + r];
        fvoff[i] = isd ? tok * (uint32_t)(p.NB * 128) + (uint32_t)(u * 64 + g * 16)
                       : tok * (uint32_t)(NQ * 64) + (uint32_t)(g * 16);
        fisd[i] = isd;
        fblk[i] = isd ? f / (2 * MT) : 0;
    }
    // gathers of record q (clamped to the last record) into registers, and
    // their stores into stage ST
    v4i fr[FPW];
    auto fload = [&](int q) {
        const int qq = min(q, NQ - 1);
#pragma unroll
        for (int i = 0; i < FPW; ++i) {
            const uint8_t *base = fisd[i] ? p.xs + (int64_t)min(qq * 4 + fblk[i], p.NB - 1) * 128
                                          : p.xsum + (int64_t)qq * 64;
            fr[i] = *(const v4i *)(base + fvoff[i]);
        }
    };
    auto fstore = [&](auto ST) {
        constexpr int st = decltype(ST)::value;
        uint8_t *base = st == 0 ? sS0 : sS1;
#pragma unroll
        for (int i = 0; i < FPW; ++i) *(v4i *)(base + foff[i] + a_off) = fr[i];
    };

    // ---- weight records: two register sets, record q + 1 loaded while q computes
    const int strip_base = sg * SPG + wave * C;
    const uint8_t *srec[C];  // the wavefront's strips' first records (uniform)
#pragma unroll
    for (int j = 0; j < C; ++j) srec[j] = recs + (int64_t)min(strip_base + j, p.NS - 1) * NQ * kQ4RecBytes;
    const uint32_t c_off = (uint32_t)lane * 16u, dm_off = (uint32_t)(lane & 15) * 16u;
    v4i bc[2][C], bd[2][C];
    auto gload_rec = [&](int q, v4i (&dc)[C], v4i (&dd)[C]) {
        const int qq = min(q, NQ - 1);
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const uint8_t *rec = srec[j] + qq * kQ4RecBytes;
            // plain loads (no non-temporal hint): an expert split into two
            // chunks reads its records twice, the second time from cache.
            // Record NQ (odd NQ's last pair): (d, m) from the zero region,
            // so it adds exactly zero.
            dc[j] = *(const v4i *)(rec + c_off);
            dd[j] = *(const v4i *)((q < NQ ? rec + 1024 : p.zeros) + dm_off);
        }
    };

    v4f y[MT][C];
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int j = 0; j < C; ++j) y[t][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    // chunk q in stage ST with record set ST
    auto chunk = [&](auto ST, int q) {
        constexpr int st = decltype(ST)::value;
        // stage st was stored at the end of the previous chunk (LDS only: no
        // memory fence, which would wait for the loads in flight)
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        fload(q + 1);
        gload_rec(q + 1, bc[st ^ 1], bd[st ^ 1]);
        const uint8_t *A = st == 0 ? sS0 : sS1;
        const uint8_t *Mf = A + NFD * 1024;
#pragma unroll
        for (int bl = 0; bl < 4; ++bl) {
            v8h a[MT][2];
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int u = 0; u < 2; ++u) a[t][u] = *(const v8h *)(A + ((bl * 2 + u) * MT + t) * 1024 + a_off);
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const uint32_t cw = (uint32_t)bc[st][j][bl];
                const uint32_t lo = cw & 0x0F0F0F0Fu, hi = (cw >> 4) & 0x0F0F0F0Fu;
                const v2h p0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, false);
                const v2h p1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 512.0f, true);
                const v2h p2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, false);
                const v2h p3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 512.0f, true);
                const v8h bop = {p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
                const float d = bf16_lo_f32((uint32_t)bd[st][j][bl]);
#pragma unroll
                for (int t = 0; t < MT; ++t) {
                    v4f acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t][0], bop, v4f{0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[t][1], bop, acc, 0, 0, 0);
#pragma unroll
                    for (int v = 0; v < 4; ++v) y[t][j][v] = fmaf(d, acc[v], y[t][j][v]);
                }
            }
            // keep each block's update here (else the compiler sinks them to
            // the end of the chunk and keeps every MFMA result alive)
#pragma unroll
            for (int t = 0; t < MT; ++t)
#pragma unroll
                for (int j = 0; j < C; ++j) asm volatile("" : "+v"(y[t][j]));
        }
#pragma unroll
        for (int t = 0; t < MT; ++t) {
            const v8bf xm = *(const v8bf *)(Mf + t * 1024 + a_off);
#pragma unroll
            for (int j = 0; j < C; ++j) {
                // every lane of column n holds its m values: the same in each k-octet
                const v4i mv = {(int)__builtin_amdgcn_perm((uint32_t)bd[st][j][1], (uint32_t)bd[st][j][0], 0x07060302u),
                                (int)__builtin_amdgcn_perm((uint32_t)bd[st][j][3], (uint32_t)bd[st][j][2], 0x07060302u), 0, 0};
                const v8bf mop = __builtin_bit_cast(v8bf, mv);
                y[t][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xm, mop, y[t][j], 0, 0, 0);
            }
        }
        // chunk q + 1's pieces into the other stage (read after the next barrier)
        fstore(ic<st ^ 1>{});
    };

    fload(0);
    gload_rec(0, bc[0], bd[0]);
    fstore(ic<0>{});
    // pairs of chunks (NQ >= 1: a do-while keeps the first record loads
    // ahead of the first stores); at odd NQ the last pair's second chunk is
    // record NQ, whose (d, m) come from the header's zero tail: it adds
    // exactly zero
    int q = 0;
    do {
        chunk(ic<0>{}, q);
        chunk(ic<1>{}, q + 1);
        q += 2;
    } while (q < NQ);

#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int row = t * 16 + 4 * (lane >> 4) + v;
            float *yrow = p.Y + sYoff[row];
            const int ex = sYexp[row];
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const int n = (strip_base + j) * 16 + (lane & 15);
                if (row < nrows && n < p.N) yrow[n] = __builtin_ldexpf(y[t][j][v], ex);
            }
        }
}


// The kernel: a job's chunk of <= 16 rows runs the one-tile copy of the
// product (about half the MFMA and VALU work of the two-tile copy); the
// routing lists these chunks last, so the workgroups dispatched once the
// first ones finish get the cheapest jobs.  The copy is chosen at entry,
// before any MFMA: inside each copy no branch sits between an MFMA and the
// instructions that read its result.
template <int WAVES, int C, int MINW, bool PER_SLOT>
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(MINW, 8))) void k_q4_moe(Q4Params p) {
    constexpr int ROWS = 32, SPG = WAVES * C;
    constexpr int STAGE = (4 * 2 * 2 + 2) * 1024;  // the two-tile copy's fragments
    // stage = the chunk's fragments: d term [block][term][tile], then m term [term][tile]
    __shared__ __attribute__((aligned(16))) uint8_t sS0[STAGE], sS1[STAGE];
    __shared__ int sTok[ROWS];
    __shared__ int64_t sYoff[ROWS];  // output row of each chunk row (token, slot)
    __shared__ int sYexp[ROWS];      // -sc of its activation row

    const int tid = threadIdx.x;
    const int groups = (p.NS + SPG - 1) / SPG;
    // Workgroup ids go round-robin over the 8 XCDs (each with its own L2):
    // workgroup b runs on XCD b % 8, which takes chunks x, x + 8, x + 16, ...
    // and all strip groups of each of them, one after another, so that a
    // chunk's activation pieces are fetched into one L2 and read there by
    // every strip group.  Chunks keep the routing table's order (full chunks
    // first) across the XCDs.
    const int x = blockIdx.x % 8, l = blockIdx.x / 8;
    const int sg = l % groups;
    const int job = (l / groups) * 8 + x;
    if (job >= *p.nchunks) return;
    const int expert = __builtin_amdgcn_readfirstlane(p.chunk_info[job * 3 + 0]);
    const int row0 = __builtin_amdgcn_readfirstlane(p.chunk_info[job * 3 + 1]);
    const int nrows = __builtin_amdgcn_readfirstlane(p.chunk_info[job * 3 + 2]);
    // activation row of each row of the chunk: the token (shared form) or the
    // (token, slot) pair itself (per-slot form); for the epilogue its output
    // row and scale exponent (one division per row here rather than per
    // output element)
    if (tid < ROWS) {
        const int pair = p.sorted[row0 + min(tid, nrows - 1)];
        const int tk = pair / p.n_used;
        const int sl = pair - tk * p.n_used;
        sTok[tid] = PER_SLOT ? pair : tk;
        sYoff[tid] = (int64_t)tk * p.ldy_token + (int64_t)sl * p.ldy_slot;
        sYexp[tid] = -p.xsc[PER_SLOT ? pair : tk];
    }
    __syncthreads();
    if (nrows <= kMoeTileRows)
        moe_job<1, WAVES, C, PER_SLOT>(p, sS0, sS1, sTok, sYoff, sYexp, sg, expert, nrows);
    else
        moe_job<2, WAVES, C, PER_SLOT>(p, sS0, sS1, sTok, sYoff, sYexp, sg, expert, nrows);
}

// ------------------------------------------------------ MoE routing sort ---
// One workgroup.  Counts the used (token, slot) pairs per expert (ids read
// once, through the row stride, and kept in registers), scans the counts,
// scatters pair ids into per-expert runs and writes the chunk table (expert,
// first row, rows) with at most `rpc` rows per chunk.  Pairs whose id lies
// outside [0, E) are left out (their outputs are not written) and flagged in
// *err.  Rows inside an expert's run may come in any order: each output row
// depends on its own activation row only.  The scan is parallel: each thread
// sums a run of consecutive experts, a wavefront scan and a scan of the
// wavefront totals give every run its offsets.  The chunk table lists the
// full chunks (rpc rows) of every expert first, then the partial chunks of
// more than 16 rows, then those of at most 16 rows.
//
// The launch's other workgroups split the activations for the grouped
// product, 1024 / tpt tokens per workgroup, tpt = 64, 128 or 256 threads per
// token (the token's 16-byte pieces rounded up to a power of two, at most
// 256, so that few threads idle at small K): the token's max |x|
// fixes a power-of-two scale 2^sc with sc = 15 - e (max |x| = f 2^e, f in
// [0.5, 1)), so that every scaled value lies below 2^15 and the two fp16
// terms h0 = fp16(x 2^sc), h1 = fp16(x 2^sc - h0) hold it to about 2^-22
// relative (the scaling is exact; the subtraction is exact in fp32).  The
// block sums of the scaled values (32 k, fixed order: 8 values per thread,
// then the four k-octets) are split into three bf16 terms, as the m term's
// A operand: one 64-byte entry per record, term u's four sums and 8 zero
// bytes at 16 u, 16 zero bytes at 48.
__device__ void moe_split_token(const MoeSplit &sp, int t, int ltid, float *s_max) {
    const int lane = ltid & 63, wl = ltid >> 6;  // wavefront of the token (0 .. tpt / 64 - 1)
    const int tpt = sp.tpt;
    // activation row t: token t (shared form), or pair t = token * per + slot
    const float *xr = sp.X + (int64_t)(t / sp.per) * sp.ldx + (int64_t)(t % sp.per) * sp.ldx_slot;
    const int npc = sp.NQ * 16;  // pieces (block, k-octet), whole records
    auto load8 = [&](int pc, float (&v)[8]) {
        const int b = pc >> 2, g = pc & 3;
        const bool ok = b < sp.NB;
        const float *src = xr + (int64_t)min(b, sp.NB - 1) * 32 + g * 8;
        if (sp.x_vec) {
            const v4f lo = *(const v4f *)src, hi = *(const v4f *)(src + 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[e] = ok ? lo[e] : 0.0f;
                v[4 + e] = ok ? hi[e] : 0.0f;
            }
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) v[e] = ok ? src[e] : 0.0f;
        }
    };
    float am = 0.0f;
    for (int pc = ltid; pc < npc; pc += tpt) {
        float v[8];
        load8(pc, v);
#pragma unroll
        for (int e = 0; e < 8; ++e) am = fmaxf(am, fabsf(v[e]));
    }
#pragma unroll
    for (int d = 32; d >= 1; d >>= 1) am = fmaxf(am, __shfl_xor(am, d));
    if (lane == 0) s_max[wl] = am;
    __syncthreads();
    float tm = s_max[0];
    for (int w = 1; w < tpt / 64; ++w) tm = fmaxf(tm, s_max[w]);
    const int sc = 15 - __builtin_amdgcn_frexp_expf(tm);
    if (ltid == 0) sp.xsc[t] = sc;
    for (int pc0 = 0; pc0 < npc; pc0 += tpt) {  // uniform trip count: the shuffles below
        const int pc = pc0 + ltid;
        const int b = pc >> 2, g = pc & 3;
        float v[8];
        load8(min(pc, npc - 1), v);
        float bs = 0.0f;
        uint32_t h[2][4];
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
            const float x0 = __builtin_ldexpf(v[e], sc), x1 = __builtin_ldexpf(v[e + 1], sc);
            bs += x0;
            bs += x1;
            const v2h a0 = {(_Float16)x0, (_Float16)x1};
            const v2h a1 = {(_Float16)(x0 - (float)a0[0]), (_Float16)(x1 - (float)a0[1])};
            h[0][e >> 1] = __builtin_bit_cast(uint32_t, a0);
            h[1][e >> 1] = __builtin_bit_cast(uint32_t, a1);
        }
        if (pc < npc && b < sp.NB) {
#pragma unroll
            for (int u = 0; u < 2; ++u)
                *(v4i *)(sp.xs + (((int64_t)t * sp.NB + b) * 2 + u) * 64 + g * 16) =
                    v4i{(int)h[u][0], (int)h[u][1], (int)h[u][2], (int)h[u][3]};
        }
        // block sum over the four k-octets (lanes 4b'..4b'+3), then the four
        // blocks of the record (lanes 16q'..16q'+15) into its first lane
        bs += __shfl_xor(bs, 1);
        bs += __shfl_xor(bs, 2);
        float s4[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) s4[k] = __shfl(bs, (lane & ~15) + 4 * k);
        if (pc < npc && (pc & 15) == 0) {
            uint32_t w[3][2];
#pragma unroll
            for (int k = 0; k < 4; k += 2) {
                const uint32_t t0 = pk_bf16(s4[k], s4[k + 1]);
                const float r0 = s4[k] - bf16_lo_f32(t0), r1 = s4[k + 1] - bf16_hi_f32(t0);
                const uint32_t t1 = pk_bf16(r0, r1);
                const uint32_t t2 = pk_bf16(r0 - bf16_lo_f32(t1), r1 - bf16_hi_f32(t1));
                w[0][k >> 1] = t0;
                w[1][k >> 1] = t1;
                w[2][k >> 1] = t2;
            }
            const int q = pc >> 4;
            // the record's 64-byte entry, one k-octet of the m-term operand
            // per 16 bytes: term u's four block sums and 8 zero bytes at
            // 16 u, zeros in the last 16
            v4i *e = (v4i *)(sp.xsum + ((int64_t)t * sp.NQ + q) * 64);
#pragma unroll
            for (int u = 0; u < 3; ++u) e[u] = v4i{(int)w[u][0], (int)w[u][1], 0, 0};
            e[3] = v4i{0, 0, 0, 0};
        }
    }
}

// inclusive prefix sum over the 64 lanes of a wavefront: rows of 16 lanes
// by DPP row shifts (bound_ctrl: a lane whose source lies before its row
// adds 0), then the last lane of row 0 into row 1 and of row 2 into row 3
// (row_bcast:15), and of row 1 into rows 2 and 3 (row_bcast:31); a row the
// row mask leaves out adds `old`, 0
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_add_src(int v) { return __builtin_amdgcn_update_dpp(0, v, CTRL, ROWS, 0xF, true); }
__device__ __forceinline__ int wave_incl_sum(int v) {
    v += dpp_add_src<0x111, 0xF>(v);  // row_shr:1
    v += dpp_add_src<0x112, 0xF>(v);  // row_shr:2
    v += dpp_add_src<0x114, 0xF>(v);  // row_shr:4
    v += dpp_add_src<0x118, 0xF>(v);  // row_shr:8
    v += dpp_add_src<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_add_src<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3
    return v;
}

constexpr int kRoutePairsPerThread = 8;  // pairs held in registers per pass
__global__ __launch_bounds__(1024) void k_moe_route(const int32_t *__restrict__ ids, int64_t ids_stride, int T,
                                                    int n_used, int E, int rpc, int32_t *__restrict__ sorted,
                                                    int32_t *__restrict__ chunk_info, int32_t *__restrict__ nchunks,
                                                    int32_t *__restrict__ err, MoeSplit sp) {
    if (blockIdx.x > 0) {
        __shared__ float s_max[16][4];
        const int grp = threadIdx.x / sp.tpt;
        const int t = ((int)blockIdx.x - 1) * (1024 / sp.tpt) + grp;
        if (blockIdx.x == 1 && threadIdx.x < 16) ((v4i *)sp.zeros)[threadIdx.x] = v4i{0, 0, 0, 0};
        // rows past R repeat row R - 1 (the same values, written again)
        moe_split_token(sp, min(t, sp.R - 1), threadIdx.x % sp.tpt, s_max[grp]);
        return;
    }
    extern __shared__ int32_t sh[];
    int32_t *cnt = sh;           // [E] register-held pairs per expert (their ranks: the atomics' old values)
    int32_t *cnt2 = sh + E;      // [E] pairs per expert past the register-held ones
    int32_t *off = sh + 2 * E;   // [E] first sorted row of the expert
    int32_t *fill = sh + 3 * E;  // [E] pairs of cnt2 scattered so far
    __shared__ int s_bad;
    const int tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int P = T * n_used;
    for (int e = tid; e < E; e += 1024) {
        cnt[e] = 0;
        cnt2[e] = 0;
        fill[e] = 0;
    }
    if (tid == 0) s_bad = 0;
    __syncthreads();
    // ---- ids of the first pass in registers, each with its rank inside its
    // expert (the counting atomic's old value); larger P loops (re-reading)
    int ev[kRoutePairsPerThread], rk[kRoutePairsPerThread];
#pragma unroll
    for (int u = 0; u < kRoutePairsPerThread; ++u) {
        const int pr = tid + 1024 * u;
        ev[u] = pr < P ? ids[(int64_t)(pr / n_used) * ids_stride + pr % n_used] : -1;
    }
    bool bad = false;
#pragma unroll
    for (int u = 0; u < kRoutePairsPerThread; ++u) {
        const int pr = tid + 1024 * u;
        rk[u] = 0;
        if (pr < P) {
            if (ev[u] >= 0 && ev[u] < E) rk[u] = atomicAdd(&cnt[ev[u]], 1);
            else bad = true;
        }
    }
    for (int pr = tid + 1024 * kRoutePairsPerThread; pr < P; pr += 1024) {
        const int e = ids[(int64_t)(pr / n_used) * ids_stride + pr % n_used];
        if (e >= 0 && e < E) atomicAdd(&cnt2[e], 1);
        else bad = true;
    }
    if (bad) s_bad = 1;
    // LDS barrier: the counts are LDS only (no memory fence)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // ---- scan and chunk table (wavefront 0; lane l owns experts
    // [l EPW, (l+1) EPW)): pairs, full chunks, partial chunks of more than
    // one tile of rows (the product's two-tile copy) and partial chunks of at
    // most one tile (its one-tile copy, about half the work), listed in that
    // order: the workgroups that start last, once the first ones finish, get
    // the cheapest jobs
    if (wave == 0) {
        constexpr int small = kMoeTileRows;
        const int EPW = (E + 63) / 64;
        const int e0 = min(lane * EPW, E), e1 = min(e0 + EPW, E);
        int lc = 0, lf = 0, lb = 0, ls = 0;
        for (int e = e0; e < e1; ++e) {
            const int c = cnt[e] + cnt2[e], r = c % rpc;
            lc += c;
            lf += c / rpc;
            lb += r > small;
            ls += r != 0 && r <= small;
        }
        const int ic = wave_incl_sum(lc), iF = wave_incl_sum(lf), ib = wave_incl_sum(lb), is = wave_incl_sum(ls);
        const int nfull = __builtin_amdgcn_readlane(iF, 63), nbig = __builtin_amdgcn_readlane(ib, 63);
        const int nsmall = __builtin_amdgcn_readlane(is, 63);
        int o = ic - lc, fo = iF - lf, bo = nfull + ib - lb, so = nfull + nbig + is - ls;
        for (int e = e0; e < e1; ++e) {
            const int c = cnt[e] + cnt2[e], nf = c / rpc, r = c % rpc;
            off[e] = o;
            for (int k = 0; k < nf; ++k) {
                chunk_info[(fo + k) * 3 + 0] = e;
                chunk_info[(fo + k) * 3 + 1] = o + k * rpc;
                chunk_info[(fo + k) * 3 + 2] = rpc;
            }
            fo += nf;
            if (r != 0) {
                int &po = r > small ? bo : so;
                chunk_info[po * 3 + 0] = e;
                chunk_info[po * 3 + 1] = o + nf * rpc;
                chunk_info[po * 3 + 2] = r;
                ++po;
            }
            o += c;
        }
        if (lane == 0) {
            *nchunks = nfull + nbig + nsmall;
            *err = s_bad;
        }
    }
    // the scatter needs the offsets alone: an LDS barrier with no memory
    // fence (a fence would wait for the chunk table's stores, which drain
    // together with the scatter's)
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // ---- scatter: register-held pairs at their rank, the others after them
#pragma unroll
    for (int u = 0; u < kRoutePairsPerThread; ++u) {
        const int pr = tid + 1024 * u;
        if (pr < P && ev[u] >= 0 && ev[u] < E) sorted[off[ev[u]] + rk[u]] = pr;
    }
    for (int pr = tid + 1024 * kRoutePairsPerThread; pr < P; pr += 1024) {
        const int e = ids[(int64_t)(pr / n_used) * ids_stride + pr % n_used];
        if (e >= 0 && e < E) sorted[off[e] + cnt[e] + atomicAdd(&fill[e], 1)] = pr;
    }
}

}  // namespace

// ------------------------------------------------------------ launchers ---

hipError_t launch_q4_repack(const uint8_t *blocks, const Q4Layout &L, uint8_t *packed, hipStream_t s) {
    const int64_t nrec = L.NS * L.NQ;
    const int64_t threads = nrec * 64;
    PackedHeader h = {kQ4Magic, kPackVersion, 0u, 0u, L.K, L.N, L.NB, L.NS, 0, 0};
    hipLaunchKernelGGL(k_q4_repack, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, s, blocks, (int)L.NB,
                       (int)L.N, (int)L.NQ, nrec, packed, h);
    return hipGetLastError();
}

hipError_t launch_q4_dense(const Q4Params &p, int mt, int waves, int cs, int64_t grid, hipStream_t s,
                           const char **variant) {
    const dim3 g((unsigned)grid), b(512);
    if (mt == 0) {
        // k_q4_gemv<W, 1, D, MR, XVEC>: one strip per workgroup, p.qps records per wavefront
        *variant = "q4_gemv_m4";
        const dim3 bw(waves * 64);
        const int mr = p.M == 1 ? 1 : p.M == 2 ? 2 : 4;
        bool ok = true;
        auto go = [&](auto W_, auto MR_) {
            constexpr int Wv = decltype(W_)::value, MRv = decltype(MR_)::value;
            // all of a wavefront's records in flight at once (8 slots; 4 at
            // four rows, where each slot also holds 8 activation values)
            constexpr int Dv = MRv == 4 ? 4 : 8;
            if (p.x_vec)
                hipLaunchKernelGGL((k_q4_gemv<Wv, 1, Dv, MRv, true>), g, bw, 0, s, p);
            else
                hipLaunchKernelGGL((k_q4_gemv<Wv, 1, Dv, MRv, false>), g, bw, 0, s, p);
        };
        auto by_m = [&](auto W_) {
            if (mr == 1) go(W_, ic<1>{});
            else if (mr == 2) go(W_, ic<2>{});
            else go(W_, ic<4>{});
        };
        // one row and at most 8 records per wavefront: activations staged once
        auto go1 = [&](auto W_) {
            constexpr int Wv = decltype(W_)::value;
            *variant = "q4_gemv_m1";
            if (p.qps <= 4) {
                if (p.x_vec)
                    hipLaunchKernelGGL((k_q4_gemv1<Wv, 4, true>), g, bw, 0, s, p);
                else
                    hipLaunchKernelGGL((k_q4_gemv1<Wv, 4, false>), g, bw, 0, s, p);
            } else {
                if (p.x_vec)
                    hipLaunchKernelGGL((k_q4_gemv1<Wv, 8, true>), g, bw, 0, s, p);
                else
                    hipLaunchKernelGGL((k_q4_gemv1<Wv, 8, false>), g, bw, 0, s, p);
            }
        };
        const bool one = p.M == 1 && p.qps <= 8;
        if (cs == 8) {
            // one row, at most 8 records per strip, 8 strips per workgroup
            *variant = "q4_gemv_m1_wide";
            if (p.M != 1 || p.NQ > 8 || waves != 8) return hipErrorInvalidValue;
            if (p.x_vec)
                hipLaunchKernelGGL((k_q4_gemv1_wide<true>), g, b, 0, s, p);
            else
                hipLaunchKernelGGL((k_q4_gemv1_wide<false>), g, b, 0, s, p);
            return hipGetLastError();
        }
        if (cs != 1) ok = false;
        else if (one && waves == 4) go1(ic<4>{});
        else if (one && waves == 8) go1(ic<8>{});
        else if (one && waves == 16) go1(ic<16>{});
        else if (waves == 4) by_m(ic<4>{});
        else if (waves == 8) by_m(ic<8>{});
        else if (waves == 16) by_m(ic<16>{});
        else ok = false;
        if (!ok) return hipErrorInvalidValue;
        return hipGetLastError();
    } else if (mt == 1 && cs == 1) {
        // k_q4_mm16_wide: one workgroup per CU at most, strips in contiguous
        // ranges, the whole k range (at most 8 records) staged once
        *variant = "q4_mm16_wide";
        if (p.NQ > 8 || p.M > 16 || p.S != 1 || waves != 8 || grid > p.NS) return hipErrorInvalidValue;
        if (p.x_vec)
            hipLaunchKernelGGL((k_q4_mm16_wide<8, true>), g, b, 0, s, p);
        else
            hipLaunchKernelGGL((k_q4_mm16_wide<8, false>), g, b, 0, s, p);
        return hipGetLastError();
    } else if (mt == 1 && waves == 8) {
        // k_q4_mm16<8, 2, 8, 2, XVEC>: at most 8 records per workgroup, 2 in flight
        // per wavefront (measured: 4, 6 and 8 in flight were 2-12 % slower)
        *variant = "q4_mm16";
        if (p.qps > 8 || p.M > 16) return hipErrorInvalidValue;
        if (p.x_vec)
            hipLaunchKernelGGL((k_q4_mm16<8, 2, 8, 2, true>), g, b, 0, s, p);
        else
            hipLaunchKernelGGL((k_q4_mm16<8, 2, 8, 2, false>), g, b, 0, s, p);
    } else if (mt == 2 && waves == 8) {
        *variant = "q4_mm_m32";
        if (p.x_vec)
            hipLaunchKernelGGL((k_q4_mm<2, 8, 2, 1, 4, true>), g, b, 0, s, p);
        else
            hipLaunchKernelGGL((k_q4_mm<2, 8, 2, 1, 4, false>), g, b, 0, s, p);
    } else {
        return hipErrorInvalidValue;
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || p.S == 1) return e;
    const int64_t n = (int64_t)p.M * p.N;
    hipLaunchKernelGGL(k_q4_finalize, dim3((unsigned)ceil_div(n, 256)), dim3(256), 0, s, p.part, p.S, p.M, p.N,
                       p.Y, p.ldy);
    return hipGetLastError();
}

hipError_t launch_moe_route(const int32_t *ids, int64_t ids_stride, int64_t T, int64_t n_used, int64_t E,
                            int rpc, int32_t *sorted, int32_t *chunk_info, int32_t *nchunks, int32_t *err,
                            const MoeSplit &sp, hipStream_t s) {
    const size_t shmem = (size_t)E * 4 * sizeof(int32_t);
    // workgroup 0 routes; workgroups 1.. split 1024 / tpt activation rows each
    MoeSplit spl = sp;
    const int npc = sp.NQ * 16;
    spl.tpt = npc > 128 ? 256 : (npc > 64 ? 128 : 64);
    const unsigned grid = 1u + (unsigned)ceil_div(sp.R, 1024 / spl.tpt);
    hipLaunchKernelGGL(k_moe_route, dim3(grid), dim3(1024), shmem, s, ids, ids_stride, (int)T, (int)n_used, (int)E,
                       rpc, sorted, chunk_info, nchunks, err, spl);
    return hipGetLastError();
}

hipError_t launch_q4_moe(const Q4Params &p, bool per_slot, int64_t max_chunks, hipStream_t s,
                         const char **variant) {
    // 4 wavefronts x 4 strips: each A fragment read from LDS feeds four
    // strips' MFMAs (half the LDS reads per MFMA of 8 x 2, which tied the
    // LDS bandwidth to the MFMA rate); 168 VGPRs, three workgroups per CU
    constexpr int WAVES = 4, C = 4;
    const int64_t groups = ceil_div(p.NS, C * WAVES);
    *variant = "q4_moe_m32";
    // 8 XCDs x groups x (chunk slots per XCD)
    const dim3 g((unsigned)(8 * groups * ceil_div(max_chunks, 8))), b(WAVES * 64);
    if (per_slot)
        hipLaunchKernelGGL((k_q4_moe<WAVES, C, 3, true>), g, b, 0, s, p);
    else
        hipLaunchKernelGGL((k_q4_moe<WAVES, C, 3, false>), g, b, 0, s, p);
    return hipGetLastError();
}

}  // namespace qmm
