// k_q4_1.hip -- q4_1 path kernels for gfx950 (CDNA4, wave64):
//   * repack of canonical q4_1 blocks into the record layout (qmm_internal.h)
//   * activation split: x = x0 + x1 + x2 with bf16 terms (near exact), plus
//     fp32 block sums of x
//   * the q4_1 product on MFMA (v_mfma_f32_16x16x32_bf16): one 32-k block is
//     one MFMA k-step, so each block gets a fresh accumulator and
//       Y += d * (sum_k q*x) + m * (sum_k x)
//     ("NPU engine: full ELFs, no xclbin", "Q4NX chunks": q4_1 blocks;
//     "Zaya 8B Q4NX on the AMD NPU", "Round 26": W = q*scale + min with bf16
//     scale and min per (row, 32-col) block)
//   * MUL_MAT_ID routing: a counting sort of the (token, slot) pairs by
//     expert into chunks of rows, read through the strided id view ("Zaya
//     8B", "The bugs that were the work"), and one grouped launch over all
//     chunks (the grouped-dispatch cost lesson of "Round 25p").
//
// Codes stay exact: bytes 0..15 read as OCP e4m3 are exactly q * 2^-9, and
// v_cvt_scalef32_pk_bf16_fp8 with scale 2^9 turns two of them into two exact
// bf16 integers per instruction.
#include "qmm_internal.h"

namespace qmm {

namespace {

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

constexpr int KCB = 8;  // blocks per LDS-staged activation chunk (two records)

__device__ __forceinline__ uint32_t bf16_rne_bits(float x) {
    uint32_t u = __float_as_uint(x);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ __forceinline__ float bf16_bits_f32(uint32_t h) { return __uint_as_float(h << 16); }

// Eight 4-bit codes (record nibble order) -> eight exact bf16 values in k order.
__device__ __forceinline__ v8bf decode8(uint32_t w) {
    const uint32_t lo = w & 0x0F0F0F0Fu;
    const uint32_t hi = (w >> 4) & 0x0F0F0F0Fu;
    const v2bf a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, false);
    const v2bf b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 512.0f, true);
    const v2bf c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, false);
    const v2bf d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 512.0f, true);
    v8bf r = {a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
    return r;
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

// ---------------------------------------------------- activation split ---
// One thread per (row, k).  x0 = bf16(x), x1 = bf16(x - x0), x2 = bf16(x - x0 - x1)
// (both differences are exact in fp32), stored [row][block][term][32].  The
// 32 lanes of a block also sum x in a fixed butterfly order.
__global__ __launch_bounds__(256) void k_q4_xsplit(const float *__restrict__ X, int64_t ldx, int R, int NB,
                                                   uint16_t *__restrict__ xsp, float *__restrict__ xs) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t per_row = (int64_t)NB * 32;
    const bool valid = gid < (int64_t)R * per_row;
    const int64_t row = gid / per_row;
    const int64_t rem = gid % per_row;
    const int64_t b = rem >> 5;
    const int j = (int)(rem & 31);
    const float x = valid ? X[row * ldx + b * 32 + j] : 0.0f;
    const uint32_t t0 = bf16_rne_bits(x);
    const float r1 = x - bf16_bits_f32(t0);
    const uint32_t t1 = bf16_rne_bits(r1);
    const float r2 = r1 - bf16_bits_f32(t1);
    const uint32_t t2 = bf16_rne_bits(r2);
    float s = x;
#pragma unroll
    for (int off = 16; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (valid) {
        uint16_t *dst = xsp + ((row * NB + b) * 3) * 32 + j;
        dst[0] = (uint16_t)t0;
        dst[32] = (uint16_t)t1;
        dst[64] = (uint16_t)t2;
        if (j == 0) xs[row * NB + b] = s;
    }
}

// ----------------------------------------------------------- the product ---
// Workgroup = WAVES wavefronts; each wavefront owns 4 column strips (64
// columns) and all MT*16 rows of the workgroup's row set.  The split
// activations of the rows are staged in LDS in chunks of KCB blocks (double
// buffered, next chunk's global loads issued before the current chunk's
// MFMAs) and shared by all wavefronts; each wavefront streams its strips'
// records (16 bytes of codes + 16 bytes of (d,m) per lane per record, one
// record prefetched ahead) and keeps its outputs in registers across the
// whole k range.
//   dense: blockIdx -> (strip group, k split); rows 0..M-1.
//   MoE:   blockIdx -> (strip group, row chunk); the chunk table gives the
//          expert and the sorted (token, slot) pairs of its rows.
template <int MT, int WAVES, bool MOE>
__global__ __launch_bounds__(WAVES * 64) void k_q4_mm(Q4Params p) {
    constexpr int NT = WAVES * 64;
    constexpr int ROWS = MT * 16;
    constexpr int SPW = 4;
    constexpr int SPG = SPW * WAVES;
    constexpr int APIECES = KCB * 3 * ROWS * 4;
    constexpr int APT = (APIECES + NT - 1) / NT;
    constexpr int XPIECES = KCB * ROWS;
    constexpr int XPT = (XPIECES + NT - 1) / NT;
    __shared__ __attribute__((aligned(16))) uint8_t sA[2][KCB][3][MT][1024];
    __shared__ __attribute__((aligned(16))) float sXS[2][KCB][ROWS];
    __shared__ int sTok[ROWS];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int groups = (p.NS + SPG - 1) / SPG;
    const int sg = blockIdx.x % groups;
    const int job = blockIdx.x / groups;

    const uint8_t *recs = p.recs;
    int nrows, row0 = 0, q0, q1;
    if (MOE) {
        if (job >= *p.nchunks) return;
        const int expert = p.chunk_info[job * 3 + 0];
        row0 = p.chunk_info[job * 3 + 1];
        nrows = p.chunk_info[job * 3 + 2];
        recs += (int64_t)expert * p.expert_stride;
        q0 = 0;
        q1 = p.NQ;
    } else {
        nrows = p.M;
        q0 = job * p.qps;
        q1 = min(p.NQ, q0 + p.qps);
    }
    recs += kHeaderBytes;
    if (tid < ROWS) sTok[tid] = (tid < nrows) ? (MOE ? p.sorted[row0 + tid] / p.n_used : tid) : -1;
    __syncthreads();

    v4i stg[APT];
    float stx[XPT];
    auto gload_chunk = [&](int qc) {
        const int b0 = qc * 4;
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int idx = tid + i * NT;
            v4i v = {0, 0, 0, 0};
            if (idx < APIECES) {
                const int g = idx & 3;
                const int t = (idx >> 2) % 3;
                const int rest = (idx >> 2) / 3;
                const int row = rest % ROWS;
                const int b = b0 + rest / ROWS;
                const int tok = sTok[row];
                if (tok >= 0 && b < p.NB)
                    v = *(const v4i *)(p.xsp + (((int64_t)tok * p.NB + b) * 3 + t) * 32 + g * 8);
            }
            stg[i] = v;
        }
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int idx = tid + i * NT;
            float v = 0.0f;
            if (idx < XPIECES) {
                const int row = idx % ROWS;
                const int b = b0 + idx / ROWS;
                const int tok = sTok[row];
                if (tok >= 0 && b < p.NB) v = p.xs[(int64_t)tok * p.NB + b];
            }
            stx[i] = v;
        }
    };
    auto sstore_chunk = [&](int buf) {
#pragma unroll
        for (int i = 0; i < APT; ++i) {
            const int idx = tid + i * NT;
            if (idx < APIECES) {
                const int g = idx & 3;
                const int t = (idx >> 2) % 3;
                const int rest = (idx >> 2) / 3;
                const int row = rest % ROWS;
                const int bl = rest / ROWS;
                *(v4i *)(&sA[buf][bl][t][row >> 4][(g * 16 + (row & 15)) * 16]) = stg[i];
            }
        }
#pragma unroll
        for (int i = 0; i < XPT; ++i) {
            const int idx = tid + i * NT;
            if (idx < XPIECES) sXS[buf][idx / ROWS][idx % ROWS] = stx[i];
        }
    };

    const int strip_base = sg * SPG + wave * SPW;
    auto load_rec = [&](int quad, v4i *codes, v4i *sc) {
#pragma unroll
        for (int j = 0; j < SPW; ++j) {
            const int strip = strip_base + j;
            if (strip < p.NS && quad < q1) {
                const uint8_t *rec = recs + ((int64_t)strip * p.NQ + quad) * kQ4RecBytes;
                codes[j] = *(const v4i *)(rec + lane * 16);
                sc[j] = *(const v4i *)(rec + 1024 + (lane & 15) * 16);
            } else {
                codes[j] = v4i{0, 0, 0, 0};
                sc[j] = v4i{0, 0, 0, 0};
            }
        }
    };

    v4f acc_y[MT][SPW];
#pragma unroll
    for (int rt = 0; rt < MT; ++rt)
#pragma unroll
        for (int j = 0; j < SPW; ++j) acc_y[rt][j] = v4f{0.0f, 0.0f, 0.0f, 0.0f};

    const int nchunk = (q1 - q0 + 1) / 2;
    if (nchunk > 0) {
        gload_chunk(q0);
        sstore_chunk(0);
    }
    __syncthreads();
    v4i codes[SPW], sc[SPW], ncodes[SPW], nsc[SPW];
    if (nchunk > 0) load_rec(q0, codes, sc);
    for (int c = 0; c < nchunk; ++c) {
        const int buf = c & 1;
        const int qc = q0 + 2 * c;
        if (c + 1 < nchunk) gload_chunk(qc + 2);
#pragma unroll
        for (int qq = 0; qq < 2; ++qq) {
            const int quad = qc + qq;
            load_rec(quad + 1, ncodes, nsc);  // prefetch (zeros past the range)
            if (quad < q1) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int bl = qq * 4 + i;
                    v8bf a[MT][3];
                    v4f xsv[MT];
#pragma unroll
                    for (int rt = 0; rt < MT; ++rt) {
#pragma unroll
                        for (int t = 0; t < 3; ++t) a[rt][t] = *(const v8bf *)(&sA[buf][bl][t][rt][lane * 16]);
                        xsv[rt] = *(const v4f *)(&sXS[buf][bl][rt * 16 + 4 * (lane >> 4)]);
                    }
#pragma unroll
                    for (int j = 0; j < SPW; ++j) {
                        const v8bf bop = decode8((uint32_t)codes[j][i]);
                        const uint32_t dm = (uint32_t)sc[j][i];
                        const float d = bf16_bits_f32(dm & 0xFFFFu);
                        const float mn = bf16_bits_f32(dm >> 16);
#pragma unroll
                        for (int rt = 0; rt < MT; ++rt) {
                            v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt][0], bop, acc, 0, 0, 0);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt][1], bop, acc, 0, 0, 0);
                            acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[rt][2], bop, acc, 0, 0, 0);
#pragma unroll
                            for (int v = 0; v < 4; ++v) {
                                acc_y[rt][j][v] = fmaf(d, acc[v], acc_y[rt][j][v]);
                                acc_y[rt][j][v] = fmaf(mn, xsv[rt][v], acc_y[rt][j][v]);
                            }
                        }
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < SPW; ++j) {
                codes[j] = ncodes[j];
                sc[j] = nsc[j];
            }
        }
        if (c + 1 < nchunk) sstore_chunk(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int rt = 0; rt < MT; ++rt)
#pragma unroll
        for (int j = 0; j < SPW; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int row = rt * 16 + 4 * (lane >> 4) + v;
                const int n = (strip_base + j) * 16 + (lane & 15);
                if (row < nrows && n < p.N) {
                    const float val = acc_y[rt][j][v];
                    if (MOE) {
                        const int pair = p.sorted[row0 + row];
                        const int t = pair / p.n_used;
                        const int s = pair - t * p.n_used;
                        p.Y[(int64_t)t * p.ldy_token + (int64_t)s * p.ldy_slot + n] = val;
                    } else if (p.S == 1) {
                        p.Y[(int64_t)row * p.ldy + n] = val;
                    } else {
                        p.part[((int64_t)job * p.M + row) * p.N + n] = val;
                    }
                }
            }
}

// Sum of the k-split partials in split order.
__global__ __launch_bounds__(256) void k_q4_finalize(const float *__restrict__ part, int S, int M, int N,
                                                     float *__restrict__ Y, int64_t ldy) {
    const int64_t gid = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (gid >= (int64_t)M * N) return;
    const int64_t m = gid / N, n = gid % N;
    float acc = 0.0f;
    for (int s = 0; s < S; ++s) acc += part[((int64_t)s * M + m) * N + n];
    Y[m * ldy + n] = acc;
}

// ------------------------------------------------------ MoE routing sort ---
// One workgroup.  Counts the used (token, slot) pairs per expert (ids read
// through the row stride), scans the counts, scatters pair ids into
// per-expert runs and writes the chunk table (expert, first row, rows) with
// at most `rpc` rows per chunk.  Pairs whose id lies outside [0, E) are left
// out (their outputs are not written) and flagged in *err.  Rows inside an
// expert's run may come in any order: each output row depends on its own
// activation row only.
__global__ __launch_bounds__(1024) void k_moe_route(const int32_t *__restrict__ ids, int64_t ids_stride, int T,
                                                    int n_used, int E, int rpc, int32_t *__restrict__ sorted,
                                                    int32_t *__restrict__ chunk_info, int32_t *__restrict__ nchunks,
                                                    int32_t *__restrict__ err) {
    extern __shared__ int32_t sh[];
    int32_t *cnt = sh;
    int32_t *off = sh + E;
    int32_t *coff = sh + 2 * E;
    int32_t *fill = sh + 3 * E;
    __shared__ int s_bad;
    const int tid = threadIdx.x;
    const int P = T * n_used;
    for (int e = tid; e < E; e += 1024) {
        cnt[e] = 0;
        fill[e] = 0;
    }
    if (tid == 0) s_bad = 0;
    __syncthreads();
    for (int pr = tid; pr < P; pr += 1024) {
        const int e = ids[(int64_t)(pr / n_used) * ids_stride + pr % n_used];
        if (e >= 0 && e < E)
            atomicAdd(&cnt[e], 1);
        else
            s_bad = 1;
    }
    __syncthreads();
    if (tid == 0) {
        int o = 0, co = 0;
        for (int e = 0; e < E; ++e) {
            off[e] = o;
            coff[e] = co;
            o += cnt[e];
            co += (cnt[e] + rpc - 1) / rpc;
        }
        *nchunks = co;
        *err = s_bad;
    }
    __syncthreads();
    for (int pr = tid; pr < P; pr += 1024) {
        const int e = ids[(int64_t)(pr / n_used) * ids_stride + pr % n_used];
        if (e >= 0 && e < E) sorted[off[e] + atomicAdd(&fill[e], 1)] = pr;
    }
    for (int e = tid; e < E; e += 1024) {
        const int nc = (cnt[e] + rpc - 1) / rpc;
        for (int c = 0; c < nc; ++c) {
            const int idx = coff[e] + c;
            chunk_info[idx * 3 + 0] = e;
            chunk_info[idx * 3 + 1] = off[e] + c * rpc;
            chunk_info[idx * 3 + 2] = min(rpc, cnt[e] - c * rpc);
        }
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

hipError_t launch_q4_xsplit(const float *X, int64_t ldx, int64_t R, int64_t NB, uint16_t *xsp, float *xs,
                            hipStream_t s) {
    const int64_t threads = R * NB * 32;
    hipLaunchKernelGGL(k_q4_xsplit, dim3((unsigned)ceil_div(threads, 256)), dim3(256), 0, s, X, ldx, (int)R,
                       (int)NB, xsp, xs);
    return hipGetLastError();
}

hipError_t launch_q4_dense(const Q4Params &p, int mt, int waves, int64_t grid, hipStream_t s,
                           const char **variant) {
    if (mt == 1 && waves == 4) {
        *variant = "q4_mm_m16";
        hipLaunchKernelGGL((k_q4_mm<1, 4, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
    } else if (mt == 2 && waves == 4) {
        *variant = "q4_mm_m32";
        hipLaunchKernelGGL((k_q4_mm<2, 4, false>), dim3((unsigned)grid), dim3(256), 0, s, p);
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
                            hipStream_t s) {
    const size_t shmem = (size_t)E * 4 * sizeof(int32_t);
    hipLaunchKernelGGL(k_moe_route, dim3(1), dim3(1024), shmem, s, ids, ids_stride, (int)T, (int)n_used, (int)E,
                       rpc, sorted, chunk_info, nchunks, err);
    return hipGetLastError();
}

hipError_t launch_q4_moe(const Q4Params &p, int64_t max_chunks, hipStream_t s, const char **variant) {
    constexpr int WAVES = 6;
    const int64_t groups = ceil_div(p.NS, 4 * WAVES);
    *variant = "q4_mm_moe_m32";
    hipLaunchKernelGGL((k_q4_mm<2, WAVES, true>), dim3((unsigned)(groups * max_chunks)), dim3(WAVES * 64), 0, s, p);
    return hipGetLastError();
}

}  // namespace qmm
