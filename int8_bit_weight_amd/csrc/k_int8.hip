// k_int8.hip -- int8 path kernels for gfx950 (CDNA4, wave64):
//   * packB: per-column int8 quantisation into the MFMA tile layout
//   * per-row int8 activation quantisation
//   * the decode forms of the int8 x int8 -> int32 GEMM with the
//     zero-point correction epilogue (M <= 32: HBM streaming of the weight
//     tiles; per 16-column strip with k split over a workgroup's wavefronts,
//     with the row quantisation inside, or one wavefront per strip for many
//     columns), and the launch dispatch (the prefill kernel, M > 32, is in
//     k_int8_prefill.hip).
//
// Arithmetic follows "int8 inference" (onemodel docs), "Product kernel
// (Int8Gemm)", and "The ONNX pack: weights to Q4NX, matmuls to our kernels,
// no VitisAI", sections "The three layers of the pack", "Why it folds
// without a new kernel" and "What works today, and what does not".
#include <type_traits>
#include <utility>

#include "qmm_internal.h"

namespace qmm {

namespace {

#include "int8_common.h"

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

template <int CTRL, int ROWS = 0xF>
__device__ __forceinline__ float dpp_f(float x) {
    // rows outside ROWS keep x
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, x), __builtin_bit_cast(int, x),
                                                                 CTRL, ROWS, 0xF, false));
}

// Maximum over each group of L consecutive lanes (L a power of two <= 64),
// in every lane of the group, with DPP lane moves (VALU; no LDS round trip,
// as __shfl_xor's ds_bpermute takes): quad permutations [1,0,3,2] and
// [2,3,0,1] and the half-row and row mirrors leave every lane of a group of
// 2, 4, 8, 16 with its maximum; the row broadcasts of lanes 15 and 31 carry
// it into lanes 31 and 63, read back with readlane.  (The permlane16/32
// swap builtins were not usable here: with both operands the same value the
// compiler took the swap's first result for both.)
template <int L>
__device__ __forceinline__ float group_max(float v) {
    static_assert(L >= 1 && L <= 64 && (L & (L - 1)) == 0, "L is a power of two <= 64");
    if constexpr (L >= 2) v = fmaxf(v, dpp_f<0xB1>(v));
    if constexpr (L >= 4) v = fmaxf(v, dpp_f<0x4E>(v));
    if constexpr (L >= 8) v = fmaxf(v, dpp_f<0x141>(v));
    if constexpr (L >= 16) v = fmaxf(v, dpp_f<0x140>(v));
    if constexpr (L >= 32) {
        // rows 1 and 3 take the maximum with lane 15 of the row before: lanes
        // 31 and 63 then hold their 32-lane half's maximum
        v = fmaxf(v, dpp_f<0x142, 0xA>(v));
        if constexpr (L == 32) {
            const float lo = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 31));
            const float hi = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
            v = (threadIdx.x & 63) < 32 ? lo : hi;
        } else {
            // rows 2 and 3 take the maximum with lane 31: lane 63 holds the wave's
            v = fmaxf(v, dpp_f<0x143, 0xC>(v));
            v = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
        }
    }
    return v;
}

// Symmetric int8 code of x for scale s (s > 0): clamp(rne(x / s), -127, 127).
// The division is IEEE correctly rounded (hipcc's default for fp32 '/').
__device__ __forceinline__ int quant_code(float x, float s) {
    float r = rintf(x / s);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    return (int)r;
}

// ---------------------------------------------------------------- packB ---
// One workgroup per 16-column strip.  Pass 1: column amax (fp32 source).
// Pass 2: each thread produces the 16 codes of one MFMA lane chunk (16
// consecutive k of one column) and stores them with one 16-byte store.
template <bool RAW>
__global__ __launch_bounds__(256) void k_pack_b(const void *__restrict__ Bsrc, int64_t ld, int u8,
                                                int K, int N, int KT, int8_t *__restrict__ codes,
                                                float *__restrict__ scale,
                                                int32_t *__restrict__ colsum,
                                                PackedHeader *__restrict__ header, PackedHeader h) {
    const int strip = blockIdx.x;
    const int t = threadIdx.x;
    const int c = t & 15;
    const int r = t >> 4;
    const int n = strip * kTileN + c;
    __shared__ float s_part[16][17];
    __shared__ int s_sum[16][17];
    __shared__ float s_scale[16];

    if (blockIdx.x == 0 && t == 0) *header = h;

    if (!RAW) {
        const float *W = (const float *)Bsrc;
        float amax = 0.0f;
        if (n < N)
            for (int k = r; k < K; k += 16) amax = fmaxf(amax, fabsf(W[(int64_t)k * ld + n]));
        s_part[r][c] = amax;
        __syncthreads();
        if (t < 16) {
            float a = 0.0f;
            for (int i = 0; i < 16; ++i) a = fmaxf(a, s_part[i][t]);
            s_scale[t] = (a == 0.0f) ? 0.0f : a / 127.0f;
        }
    } else if (t < 16) {
        s_scale[t] = (strip * kTileN + t < N) ? 1.0f : 0.0f;
    }
    __syncthreads();
    const float s = s_scale[c];

    const int lane = t & 63;
    const int g = lane >> 4;
    int csum = 0;
    for (int tile = t >> 6; tile < KT; tile += 4) {
        const int k0 = tile * kTileK + g * 16;
        uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const int k = k0 + j;
            int q = 0;
            if (n < N && k < K) {
                if (RAW) {
                    const uint8_t b = ((const uint8_t *)Bsrc)[(int64_t)k * ld + n];
                    q = u8 ? (int)b - 128 : (int)(int8_t)b;
                } else if (s > 0.0f) {
                    q = quant_code(((const float *)Bsrc)[(int64_t)k * ld + n], s);
                }
            }
            csum += q;
            w[j >> 2] |= (uint32_t)(q & 0xFF) << (8 * (j & 3));
        }
        v4i out = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        *(v4i *)(codes + ((int64_t)strip * KT + tile) * kTileBytes + lane * 16) = out;
    }
    s_sum[r][c] = csum;
    __syncthreads();
    if (t < 16) {
        int acc = 0;
        for (int i = 0; i < 16; ++i) acc += s_sum[i][t];
        colsum[strip * kTileN + t] = acc;
        scale[strip * kTileN + t] = s_scale[t];
    }
}

// x / s rounded to nearest, bit-identical to the IEEE quotient: y = 1/s is
// correctly rounded (one IEEE division per lane), two residual corrections
// with fma bring x*y to within one ulp and then, by Markstein's theorem
// (a faithful quotient plus RN(residual) times a correctly rounded
// reciprocal rounds to the correctly rounded quotient), to RN(x/s).  The
// theorem needs no underflow or overflow: callers use it for normal s and
// take the IEEE division otherwise.
__device__ __forceinline__ float div_by(float x, float s, float y) {
    const float q0 = x * y;
    const float q1 = fmaf(fmaf(-q0, s, x), y, q0);
    return fmaf(fmaf(-q1, s, x), y, q1);
}

// Codes of 4 values for scale s > 0 with y = 1/s (k_quantize_rows rule:
// clamp(rne(x / s), -127, 127)), packed little-endian; `fast` selects the
// division above, else the IEEE division.
__device__ __forceinline__ uint32_t quant4(const float (&x)[4], float s, float y, bool fast) {
    float q[4];
    bool ok = fast;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        q[j] = div_by(x[j], s, y);
        ok = ok && fabsf(q[j]) <= 256.0f;
    }
    // the IEEE division only where the fast quotient may be off, decided per
    // wavefront (both quotients are the correctly rounded one where ok)
    if (!__all(ok)) {
#pragma unroll
        for (int j = 0; j < 4; ++j) q[j] = ok ? q[j] : x[j] / s;
    }
    uint32_t w = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        float r = rintf(q[j]);
        r = fminf(fmaxf(r, -127.0f), 127.0f);
        w |= (uint32_t)((int)r & 0xFF) << (8 * j);
    }
    return w;
}

// ------------------------------------------------------- row quantiser ---
// One workgroup (256 threads) per row.  VEC (X and Xq rows 16- and 4-byte
// aligned, K a multiple of 4, K <= 4096): every thread loads its up to 16
// values with 16-byte loads at once, keeps them in registers through the
// row maximum and writes 4 codes per 4-byte store.  Otherwise two strided
// passes over the row.
template <bool VEC>
__global__ __launch_bounds__(256) void k_quantize_rows(const float *__restrict__ X, int64_t ldx,
                                                       int K, int8_t *__restrict__ Xq, int64_t ldq,
                                                       float *__restrict__ row_scale) {
    const int64_t m = blockIdx.x;
    const int t = threadIdx.x;
    const float *x = X + m * ldx;
    int8_t *q = Xq + m * ldq;
    __shared__ float s_red[4];
    float amax = 0.0f;
    float v[4][4];
    if (VEC) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = (t + 256 * i) * 4;
            const v4f l = *(const v4f *)(x + min(k, K - 4));
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                v[i][e] = k < K ? l[e] : 0.0f;
                amax = fmaxf(amax, fabsf(v[i][e]));
            }
        }
    } else {
        for (int k = t; k < K; k += 256) amax = fmaxf(amax, fabsf(x[k]));
    }
    amax = wave_max_f(amax);
    if ((t & 63) == 0) s_red[t >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
    const float s = (amax == 0.0f) ? 0.0f : amax / 127.0f;
    const float y = 1.0f / s;
    const bool fast = s >= 0x1p-100f && s <= 0x1p100f;
    if (VEC) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int k = (t + 256 * i) * 4;
            if (k < K) *(uint32_t *)(q + k) = s > 0.0f ? quant4(v[i], s, y, fast) : 0u;
        }
    } else {
        for (int k = t; k < K; k += 256) q[k] = (s > 0.0f) ? (int8_t)quant_code(x[k], s) : (int8_t)0;
    }
    if (t == 0) row_scale[m] = s;
}

// --------------------------------------------------------- decode GEMM ---
// Loads of the decode kernels are never inside branches (a load in a branch
// makes the compiler wait for it where the branch ends, which serialises the
// memory round trips): rows, k and tiles past the valid range are clamped to
// valid memory and the values are masked where they are used.  AVEC (A or X
// 16-byte aligned, ld and K multiples of 16) selects 16-byte loads.

// 16 fp32 activations of row `row`, k = k0 .. k0+15 (zero outside M x K).
template <bool AVEC>
__device__ __forceinline__ void load_x16(const Int8GemmParams &p, int row, int k0, float (&x)[16]) {
    const int r = min(row, p.M - 1);
    const float *src = p.X + (int64_t)r * p.ldx;
    if (AVEC) {
        const bool ok = row < p.M && k0 < p.K;
        const float *s = src + min(k0, p.K - 16);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const v4f v = *(const v4f *)(s + 4 * j);
#pragma unroll
            for (int e = 0; e < 4; ++e) x[4 * j + e] = ok ? v[e] : 0.0f;
        }
    } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const float v = src[min(k0 + j, p.K - 1)];
            x[j] = (row < p.M && k0 + j < p.K) ? v : 0.0f;
        }
    }
}

// Codes of 16 activations for row scale s (same rule as k_quantize_rows).
__device__ __forceinline__ v4i quant16(const float (&x)[16], float s) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
    if (s > 0.0f) {
#pragma unroll
        for (int j = 0; j < 16; ++j) w[j >> 2] |= (uint32_t)(quant_code(x[j], s) & 0xFF) << (8 * (j & 3));
    }
    return v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}


// M <= 16*MT on quantised activations.  One workgroup per 16-column strip;
// its WAVES wavefronts split the k tiles round-robin (wave w takes tiles w,
// w+WAVES, ...), TPW tiles per round, and every load of a round (one 16-byte
// weight load per lane per tile, a contiguous 1 KiB per tile, and the
// matching activation loads) is issued before its first MFMA.  The
// epilogue's column and row operands are fetched with the first round.  The
// waves' 16x16 int32 tiles are summed in LDS in wave order and the epilogue
// runs in the same workgroup: no cross-workgroup traffic, no workspace.
template <int MT, int WAVES, int TPW, bool HAS_ZB, bool AVEC>
__global__ __launch_bounds__(WAVES * 64) void k_int8_decode(Int8GemmParams p) {
    constexpr int NE = MT * 256;  // elements of the (MT*16) x 16 output tile
    constexpr int NT = WAVES * 64;
    constexpr int EPT = (NE + NT - 1) / NT;  // epilogue elements per thread
    constexpr int ROWS = MT * 16;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int strip = blockIdx.x;
    const int8_t *strip_codes = p.codes + (int64_t)strip * p.KT * kTileBytes + lane * 16;

    v4i acc[MT], accr[MT];
#pragma unroll
    for (int r = 0; r < MT; ++r) {
        acc[r] = v4i{0, 0, 0, 0};
        accr[r] = v4i{0, 0, 0, 0};
    }
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    const ColOps col = load_colops_c(p, strip * kTileN + (threadIdx.x & 15));
    float rs[EPT];
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int m = min((int)(threadIdx.x + i * NT) >> 4, p.M - 1);
        // without row scales the (discarded) load reads col_scale[0], which
        // exists for any N >= 1; col_scale[m] could lie past a caller's N
        const float v = *(p.row_scale ? p.row_scale + m : p.col_scale);
        rs[i] = p.row_scale ? v : 1.0f;
    }

    for (int base = wave; base < p.KT; base += WAVES * TPW) {
        v4i bf[TPW], af[TPW][MT];
#pragma unroll
        for (int i = 0; i < TPW; ++i) {
            const int kt = base + i * WAVES;
            bf[i] = *(const v4i *)(strip_codes + (int64_t)min(kt, p.KT - 1) * kTileBytes);
#pragma unroll
            for (int r = 0; r < MT; ++r)
                af[i][r] = load_a16<AVEC>(p, r * 16 + (lane & 15), kt * kTileK + (lane >> 4) * 16);
        }
#pragma unroll
        for (int i = 0; i < TPW; ++i)
#pragma unroll
            for (int r = 0; r < MT; ++r) {
                acc[r] = mfma_i8(af[i][r], bf[i], acc[r]);
                if (HAS_ZB) accr[r] = mfma_i8(af[i][r], ones, accr[r]);
            }
    }

    __shared__ int32_t s_red[WAVES][ROWS][17];
    __shared__ int32_t s_redr[WAVES][ROWS];
    __shared__ int32_t s_rowsum[ROWS];
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int row = r * 16 + 4 * (lane >> 4) + i;
            s_red[wave][row][lane & 15] = acc[r][i];
            if (HAS_ZB && (lane & 15) == 0) s_redr[wave][row] = accr[r][i];
        }
    __syncthreads();
    if (HAS_ZB) {
        if (threadIdx.x < ROWS) {
            int32_t rsum = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) rsum += s_redr[w][threadIdx.x];
            s_rowsum[threadIdx.x] = rsum;
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < EPT; ++i) {
        const int e = threadIdx.x + i * NT;
        const int m = e >> 4;
        const int n = strip * kTileN + (e & 15);
        if (e < NE && m < p.M && n < p.N) {
            int32_t v = 0;
#pragma unroll
            for (int w = 0; w < WAVES; ++w) v += s_red[w][m][e & 15];
            epilogue_store_c(p, m, n, (uint32_t)v, HAS_ZB ? s_rowsum[m] : 0, HAS_ZB, rs[i], row_za(p, m), col);
        }
    }
}

// Decode over many columns (M <= 16*MT, N of tens of thousands, such as an
// output projection onto a vocabulary): one wavefront per 16-column strip
// over its whole k range, kWideWaves strips per workgroup.  The workgroup
// copies A' (shifted domain) into LDS once, in MFMA operand order (tile kt,
// row tile r: lane l's 16 bytes are row 16 r + l % 16, k = 64 kt + 16 (l / 16)
// .. +15), so each wavefront streams only its own strip's weight tiles,
// through a ring of D register stages issued before the A copy, and no
// wavefront waits for another after that copy: the epilogue runs straight
// from the MFMA accumulators (lane l holds rows 4 (l / 16) + i, column
// l % 16).  The per-strip workgroups of k_int8_decode instead split one
// strip's k range over their wavefronts and sum the pieces in LDS, which
// costs a reduction and a barrier per 16 columns.  Loads past the last tile
// re-read the last tile (clamped), never out of range.
template <int MT, int D, bool HAS_ZB, bool AVEC>
__global__ __launch_bounds__(kWideWaves * 64) void k_int8_decode_wide(Int8GemmParams p) {
    extern __shared__ v4i s_a[];  // [KT][MT][64]
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int strip_raw = (int)blockIdx.x * kWideWaves + wave;
    const bool strip_ok = strip_raw < p.NS;
    const int strip = min(strip_raw, p.NS - 1);
    const int8_t *codes = p.codes + (int64_t)strip * p.KT * kTileBytes + lane * 16;
    const int last = p.KT - 1;

    v4i bf[D];
#pragma unroll
    for (int i = 0; i < D; ++i) bf[i] = *(const v4i *)(codes + (int64_t)min(i, last) * kTileBytes);
    const ColOps col = load_colops_c(p, strip * kTileN + (lane & 15));
    float rs[MT][4];
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = min(r * 16 + 4 * (lane >> 4) + i, p.M - 1);
            const float v = *(p.row_scale ? p.row_scale + m : p.col_scale);
            rs[r][i] = p.row_scale ? v : 1.0f;
        }
    const int na = p.KT * MT * 64;
    for (int u = threadIdx.x; u < na; u += kWideWaves * 64) {
        const int l = u & 63;
        const int rt = (u >> 6) % MT;
        const int kt = (u >> 6) / MT;
        s_a[u] = load_a16<AVEC>(p, rt * 16 + (l & 15), kt * kTileK + (l >> 4) * 16);
    }
    __syncthreads();

    v4i acc[MT], accr[MT];
#pragma unroll
    for (int r = 0; r < MT; ++r) {
        acc[r] = v4i{0, 0, 0, 0};
        accr[r] = v4i{0, 0, 0, 0};
    }
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    for (int kt0 = 0; kt0 < p.KT; kt0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int kt = kt0 + i;
            if (kt < p.KT) {
#pragma unroll
                for (int r = 0; r < MT; ++r) {
                    const v4i a = s_a[(kt * MT + r) * 64 + lane];
                    acc[r] = mfma_i8(a, bf[i], acc[r]);
                    if (HAS_ZB) accr[r] = mfma_i8(a, ones, accr[r]);
                }
            }
            bf[i] = *(const v4i *)(codes + (int64_t)min(kt + D, last) * kTileBytes);
        }
    }

    const int n = strip * kTileN + (lane & 15);
#pragma unroll
    for (int r = 0; r < MT; ++r)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = r * 16 + 4 * (lane >> 4) + i;
            if (strip_ok && m < p.M && n < p.N)
                epilogue_store_c(p, m, n, (uint32_t)acc[r][i], HAS_ZB ? accr[r][i] : 0, HAS_ZB, rs[r][i],
                                 row_za(p, m), col);
        }
}

// Wide decode with the per-row quantisation inside (int8_gemm_dynamic over
// >= 1024 strips, MP * K <= 16384): the quantiser and the product in one
// launch.  The workgroup's 512 threads take MP rows (M rounded up to a power
// of two), 512 / MP threads a row, each thread CPT 16-byte chunks of it at a
// stride of 512 / MP chunks, so a wavefront's loads are contiguous.  The
// chunk loads go out first, then the wavefront's weight tiles (as in
// k_int8_decode_wide), so the row maxima wait for the activations alone.
// Row maxima combine by DPP lane moves inside a wavefront and through LDS
// across the wavefronts of a row; every thread then quantises its chunks
// with the k_quantize_rows rule (bit for bit its codes and scales) straight
// into the LDS copy of the rows' codes in operand order.  Rows past M
// quantise row M - 1 again and operand rows past MP are never written: both
// reach only outputs that are not stored; k past K multiplies the zero codes
// of the padded weight.  Workgroup 0 also writes the codes and scales out
// when asked.
template <int MP, int CPT>
__device__ __forceinline__ void wide_q_load(const Int8GemmParams &p, int tid, v4f (&xv)[CPT]) {
    constexpr int TPR = kWideWaves * 64 / MP;
    const int r = tid / TPR, j = tid % TPR;
    const int nch = p.K >> 2;
    const float *xrow = p.X + (int64_t)min(r, p.M - 1) * p.ldx;
#pragma unroll
    for (int i = 0; i < CPT; ++i) xv[i] = *(const v4f *)(xrow + 4 * min(j + i * TPR, nch - 1));
}

// s_amax: [MP][wavefronts per row]; s_scale: [MP].  Ends with a barrier
// (LDS only: the weight loads in flight are not waited for).
template <int MT, int MP, int CPT>
__device__ __forceinline__ void wide_q_quantize(const Int8GemmParams &p, int tid, int lane, int wave,
                                                const v4f (&xv)[CPT], v4i *s_a, float *s_amax, float *s_scale) {
    constexpr int TPR = kWideWaves * 64 / MP;  // threads per row
    constexpr int L = TPR < 64 ? TPR : 64;     // lanes of a row in one wavefront
    constexpr int WPR = TPR / L;               // wavefronts per row
    static_assert(MP <= 16 * MT && (MP & (MP - 1)) == 0, "rows");
    const int r = tid / TPR, j = tid % TPR;
    const int nch = p.K >> 2;
    // row maxima (chunks past K count as zeros)
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < CPT; ++i)
        if (j + i * TPR < nch)
#pragma unroll
            for (int e = 0; e < 4; ++e) a = fmaxf(a, fabsf(xv[i][e]));
    a = group_max<L>(a);
    if constexpr (WPR > 1) {
        if (lane == 0) s_amax[r * WPR + wave % WPR] = a;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < WPR; ++w) a = fmaxf(a, s_amax[r * WPR + w]);
    }
    const float s = (a == 0.0f) ? 0.0f : a / 127.0f;
    const float y = 1.0f / s;
    const bool fast = s >= 0x1p-100f && s <= 0x1p100f;
    if (j == 0) {
        s_scale[r] = s;
        if (p.rs_out && blockIdx.x == 0 && r < p.M) p.rs_out[r] = s;
    }
    // codes into the operand copy: 4 codes of chunk c = k 4c .. 4c + 3 of
    // row r sit in the 16-byte operand of (k tile, row tile, lane (4c % 64) / 16
    // * 16 + r % 16) at byte 4c % 16
    uint8_t *sa = (uint8_t *)s_a;
#pragma unroll
    for (int i = 0; i < CPT; ++i) {
        const int c = j + i * TPR;
        if (c < nch) {
            const float xs[4] = {xv[i][0], xv[i][1], xv[i][2], xv[i][3]};
            const uint32_t w = s > 0.0f ? quant4(xs, s, y, fast) : 0u;
            const int k = 4 * c, kt = k >> 6, kk = k & 63;
            const int op = (kt * MT + (r >> 4)) * 64 + (kk >> 4) * 16 + (r & 15);
            *(uint32_t *)(sa + op * 16 + (kk & 15)) = w;
            if (p.xq_out && blockIdx.x == 0 && r < p.M) {
                int8_t *dst = p.xq_out + (int64_t)r * p.ldq + k;
#pragma unroll
                for (int e = 0; e < 4; ++e) dst[e] = (int8_t)(w >> (8 * e));
            }
        }
    }
    __syncthreads();
}

template <int MT, int D, int MP, int CPT>
__global__ __launch_bounds__(kWideWaves * 64) void k_int8_decode_wide_q(Int8GemmParams p) {
    constexpr int WPR = (kWideWaves * 64 / MP) / ((kWideWaves * 64 / MP) < 64 ? (kWideWaves * 64 / MP) : 64);
    extern __shared__ v4i s_a[];  // [KT][MT][64]
    __shared__ float s_amax[MP * WPR];
    __shared__ float s_scale[MP];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int strip_raw = (int)blockIdx.x * kWideWaves + wave;
    const bool strip_ok = strip_raw < p.NS;
    const int strip = min(strip_raw, p.NS - 1);
    const int8_t *codes = p.codes + (int64_t)strip * p.KT * kTileBytes + lane * 16;
    const int last = p.KT - 1;

    v4f xv[CPT];
    wide_q_load<MP, CPT>(p, tid, xv);
    v4i bf[D];
#pragma unroll
    for (int i = 0; i < D; ++i) bf[i] = *(const v4i *)(codes + (int64_t)min(i, last) * kTileBytes);
    const ColOps col = load_colops_c(p, strip * kTileN + (lane & 15));
    wide_q_quantize<MT, MP, CPT>(p, tid, lane, wave, xv, s_a, s_amax, s_scale);

    v4i acc[MT];
#pragma unroll
    for (int t = 0; t < MT; ++t) acc[t] = v4i{0, 0, 0, 0};
    for (int kt0 = 0; kt0 < p.KT; kt0 += D) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            const int kt = kt0 + i;
            if (kt < p.KT) {
#pragma unroll
                for (int t = 0; t < MT; ++t) acc[t] = mfma_i8(s_a[(kt * MT + t) * 64 + lane], bf[i], acc[t]);
            }
            bf[i] = *(const v4i *)(codes + (int64_t)min(kt + D, last) * kTileBytes);
        }
    }

    const int n = strip * kTileN + (lane & 15);
#pragma unroll
    for (int t = 0; t < MT; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = t * 16 + 4 * (lane >> 4) + i;
            if (strip_ok && m < p.M && n < p.N)
                epilogue_store_c(p, m, n, (uint32_t)acc[t][i], 0, false, s_scale[min(m, MP - 1)], 0, col);
        }
}

// A persistent form of k_int8_decode_wide_q for M <= 16 and K <= 1024 (at
// most 16 k tiles) over many strips: two workgroups per CU (at most 128
// VGPRs); workgroup b of G owns a contiguous run of NS / G or NS / G + 1
// strips and quantises the rows once, then each wavefront runs the strips
// first + wave, first + wave + 8, ... in turn.  Register slot i holds k tile i of the
// current strip and, once it is multiplied, takes tile i of the wavefront's
// next strip (the column operands of the next strip are loaded likewise), so
// the next strip's loads are in flight while one is multiplied.  Per strip
// the arithmetic and the epilogue are k_int8_decode_wide_q's.  All 16 tiles
// are multiplied whatever KT is: operand tiles KT..15 are zero in LDS (and
// their weight slots re-read tile KT - 1), so no branch sits between an MFMA
// and the instructions that read its result.
template <int MP, int CPT>
__global__ __launch_bounds__(kWideWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 8))) void k_int8_decode_wide_qp(
    Int8GemmParams p) {
    constexpr int D = 16;
    constexpr int WPR = (kWideWaves * 64 / MP) / ((kWideWaves * 64 / MP) < 64 ? (kWideWaves * 64 / MP) : 64);
    __shared__ v4i s_a[D * 64];  // 16 operand tiles, those past KT zero
    __shared__ float s_amax[MP * WPR];
    __shared__ float s_scale[MP];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    // workgroup b of G: NS / G strips, one more for b < NS % G
    const int G = (int)gridDim.x, b = (int)blockIdx.x;
    const int sq = p.NS / G, sr = p.NS % G;
    const int first = b * sq + min(b, sr);
    const int cnt = sq + (b < sr ? 1 : 0);
    const int nst = max(0, (cnt - wave + kWideWaves - 1) / kWideWaves);  // this wavefront's strips
    const int KT = p.KT, last = KT - 1;
    const int8_t *codes = p.codes + lane * 16;
    int strip = min(first + wave, p.NS - 1);

    v4f xv[CPT];
    wide_q_load<MP, CPT>(p, tid, xv);
    v4i bf[D];
#pragma unroll
    // weight tiles non-temporal: each is read once (lm_head 29.7 -> 26.0 us at M = 1)
    for (int i = 0; i < D; ++i)
        bf[i] = __builtin_nontemporal_load((const v4i *)(codes + ((int64_t)strip * KT + min(i, last)) * kTileBytes));
    ColRaw col = load_colraw(p, strip * kTileN + (lane & 15));
    for (int u = KT * 64 + tid; u < D * 64; u += kWideWaves * 64) s_a[u] = v4i{0, 0, 0, 0};
    wide_q_quantize<1, MP, CPT>(p, tid, lane, wave, xv, s_a, s_amax, s_scale);
    float rs[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) rs[i] = s_scale[min(4 * (lane >> 4) + i, MP - 1)];

    // one strip; NEXT: refill the slots and column operands from the
    // wavefront's next strip (inlined: the slots must stay in registers)
    auto run_strip = [&](auto NEXT) __attribute__((always_inline)) {
        constexpr bool next = decltype(NEXT)::value;
        const int ahead = strip + kWideWaves;
        v4i acc = {0, 0, 0, 0};
#pragma unroll
        for (int i = 0; i < D; ++i) {
            acc = mfma_i8(s_a[i * 64 + lane], bf[i], acc);
            if constexpr (next)
                bf[i] = __builtin_nontemporal_load((const v4i *)(codes + ((int64_t)ahead * KT + min(i, last)) * kTileBytes));
            // keeps each tile's operand read next to its MFMA (hoisted, the
            // 16 reads held 64 more registers and spilled)
            asm volatile("" ::: "memory");
        }
        ColRaw cn = col;
        if constexpr (next) cn = load_colraw(p, ahead * kTileN + (lane & 15));
        const ColOps co = colops_of(p, col);
        const int n = strip * kTileN + (lane & 15);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int m = 4 * (lane >> 4) + i;
            if (m < p.M && n < p.N) epilogue_store_c(p, m, n, (uint32_t)acc[i], 0, false, rs[i], 0, co);
        }
        col = cn;
        strip = ahead;
    };
    for (int i = 0; i + 1 < nst; ++i) run_strip(std::true_type{});
    if (nst > 0) run_strip(std::false_type{});
}

// Fused dynamic quantisation for small M x K (the planner takes it while
// E * K <= 16384, E = rows of a row group rounded up to a power of two <= 16,
// and K <= 4096; row groups run as the grid's second dimension).  A
// workgroup of WAVES (8, or 4 where planned) wavefronts covers S consecutive
// 16-column strips:
//   1. every wavefront loads the activations of its TPQ k tiles (tile t
//      belongs to wave t % WAVES; 64 / E lanes per row, E values per lane and
//      tile, so every lane does real work even at M = 1; at most 32 values
//      per lane), then its weight tiles;
//   2. row maxima combine across the lanes of a row (DPP lane moves) and the
//      waves (LDS, one barrier); each lane forms its row's scale amax/127 and
//      quantises its values with the k_quantize_rows rule into an LDS copy of
//      the rows' codes, laid out as MFMA A operands (E rows of 64 bytes per
//      k tile);
//   3. the WAVES / S wavefronts of a strip take its k tiles round-robin, one
//      16x16x64 MFMA per tile with A from LDS (rows >= E read as zero);
//   4. the strip's wavefronts' int32 tiles are summed in LDS and the
//      epilogue runs in the same workgroup.
// All S strips share the one quantisation, so the activations are read
// from L2 once per S strips: S > 1 pays where M * K is large next to a
// strip's weights.  At S = 1 every wave only multiplies the tiles it
// quantised itself and no barrier separates phases 2 and 3.
// GROUPED: the grid's strips are those of up to kMaxGroups weights that
// share the activations, back to back; each wavefront takes its strip's
// item (weight, width, epilogue operands) from `g` and works on the item's
// own strip index (every item is the same computation as a call of its
// own).
struct NoGroups {};
template <bool GROUPED>
using GroupArg = std::conditional_t<GROUPED, DecodeGroups, NoGroups>;

template <int WAVES, int E, int TPQ, int S, bool AVEC, bool GROUPED>
__global__ __launch_bounds__(WAVES * 64) void k_int8_decode_q(Int8GemmParams p, GroupArg<GROUPED> g) {
    constexpr int WPS = WAVES / S;         // wavefronts per strip
    constexpr int TPB = TPQ * S;           // weight tiles per wavefront (bound)
    constexpr int L = 64 / E;              // lanes per row
    static_assert(WAVES == 4 || WAVES == 8, "4 or 8 wavefronts");
    static_assert(E == 1 || E == 2 || E == 4 || E == 8 || E == 16, "E is a power of two <= 16");
    static_assert((S == 1 || S == 2 || S == 4) && WAVES % S == 0, "S divides the wavefronts");
    static_assert(E * TPQ <= 32, "at most 32 activations per lane");
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int slot = wave / WPS, kg = wave % WPS;
    // the quantised rows and scales are written once, by workgroup x = 0
    const bool writer = blockIdx.x == 0;
    const int gstrip = (int)blockIdx.x * S + slot;
    const bool strip_ok = gstrip < p.NS;
    int strip = min(gstrip, p.NS - 1);
    if constexpr (GROUPED) {
        const int it = (strip >= g.strip_begin[1]) + (strip >= g.strip_begin[2]) + (strip >= g.strip_begin[3]);
        strip -= g.strip_begin[it];
        p.codes = g.codes[it];
        p.colsum = g.colsum[it];
        p.col_scale = g.col_scale[it];
        p.y_f32 = g.y_f32[it];
        p.ld_f32 = g.ld_f32[it];
        p.bias_f32 = g.bias_f32[it];
        p.N = g.N[it];
    }
    // (after the item's operands: the row offsets apply to its output)
    if (p.rpg > 0) {
        // row group blockIdx.y: rows [y rpg, y rpg + rpg) of the call, quantised
        // and multiplied on their own (the weights are read once per group)
        const int r0 = (int)blockIdx.y * p.rpg;
        p.M = min(p.rpg, p.M - r0);
        p.X += (int64_t)r0 * p.ldx;
        if (p.y_i32) p.y_i32 += (int64_t)r0 * p.ld_i32;
        if (p.y_f32) p.y_f32 += (int64_t)r0 * p.ld_f32;
        if (p.y_q8) p.y_q8 += (int64_t)r0 * p.ld_q8;
        if (p.xq_out) p.xq_out += (int64_t)r0 * p.ldq;
        if (p.rs_out) p.rs_out += r0;
    }
    const int m = lane / L;                    // row of this lane's values
    const int kl = (lane % L) * E;             // their first k within a tile
    const bool row_ok = m < p.M;
    const int KT = p.KT;

    // loads: activations, weight tiles, the epilogue's column operands
    float x[TPQ][E];
    v4i bf[TPB];
    {
        const float *src = p.X + (int64_t)min(m, p.M - 1) * p.ldx;
#pragma unroll
        for (int t = 0; t < TPQ; ++t) {
            const int k0 = (wave + t * WAVES) * kTileK + kl;
            const bool ok = row_ok && k0 < p.K;
            if (AVEC && E >= 4) {
                const float *s = src + min(k0, p.K - E);
#pragma unroll
                for (int j = 0; j < E; j += 4) {
                    const v4f v = *(const v4f *)(s + j);
#pragma unroll
                    for (int e = 0; e < 4; ++e) x[t][j + e] = ok ? v[e] : 0.0f;
                }
            } else {
#pragma unroll
                for (int j = 0; j < E; ++j) {
                    const float v = src[min(k0 + j, p.K - 1)];
                    x[t][j] = (ok && k0 + j < p.K) ? v : 0.0f;
                }
            }
        }
        const int8_t *cs = p.codes + (int64_t)strip * KT * kTileBytes + lane * 16;
        // the weight tiles with the non-temporal hint: read once per call,
        // they then displace less of what later calls read again (the
        // activations; measured 3 % on the Qwen3-0.6B decode step)
#pragma unroll
        for (int j = 0; j < TPB; ++j)
            bf[j] = __builtin_nontemporal_load((const v4i *)(cs + (int64_t)min(kg + j * WPS, KT - 1) * kTileBytes));
    }
    const ColOps col = load_colops_c(p, strip * kTileN + (lane & 15));

    __shared__ __attribute__((aligned(16))) float s_amax[E][WAVES];  // [row][wave]
    __shared__ float s_scale[E];
    __shared__ __attribute__((aligned(16))) int8_t s_q[TPQ * WAVES][E][64];  // [k tile][row][k]
    // partial tiles, [row][column][wave]: a strip's waves are contiguous, so
    // an output's sum reads them with 16-byte loads (the row pitch of 20
    // keeps those loads aligned)
    __shared__ __attribute__((aligned(16))) int32_t s_red[E][16][WAVES + 4];

    float a = 0.0f;
#pragma unroll
    for (int t = 0; t < TPQ; ++t)
#pragma unroll
        for (int j = 0; j < E; ++j) a = fmaxf(a, fabsf(x[t][j]));
    a = group_max<L>(a);
    if (lane % L == 0) s_amax[m][wave] = a;
    __syncthreads();
    a = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; w += 4) {
        const v4f v = *(const v4f *)(&s_amax[m][w]);
        a = fmaxf(fmaxf(a, fmaxf(v[0], v[1])), fmaxf(v[2], v[3]));
    }
    const float s = (a == 0.0f) ? 0.0f : a / 127.0f;
    if (wave == 0 && lane % L == 0) {
        s_scale[m] = s;
        if (p.rs_out && writer && row_ok) p.rs_out[m] = s;
    }
    const float y = 1.0f / s;
    const bool fast_s = s >= 0x1p-100f && s <= 0x1p100f;

#pragma unroll
    for (int t = 0; t < TPQ; ++t) {
        // codes: clamp(rne(x / s), -127, 127), 0 for an all-zero row
        float qv[E];
        bool fast = fast_s;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            qv[j] = div_by(x[t][j], s, y);
            fast = fast && fabsf(qv[j]) <= 256.0f;
        }
        // the IEEE division where the fast quotient may be off (a scale
        // outside [2^-100, 2^100], a quotient past 256), decided per
        // wavefront: as a per-lane select the compiler computed the division
        // for every value (half the quantisation phase)
        if (!__all(fast)) {
#pragma unroll
            for (int j = 0; j < E; ++j) qv[j] = fast ? qv[j] : x[t][j] / s;
        }
        uint32_t w[(E + 3) / 4];
#pragma unroll
        for (int i = 0; i < (E + 3) / 4; ++i) w[i] = 0u;
#pragma unroll
        for (int j = 0; j < E; ++j) {
            float r = rintf(qv[j]);
            r = fminf(fmaxf(r, -127.0f), 127.0f);
            const uint32_t c = s > 0.0f ? (uint32_t)((int)r & 0xFF) : 0u;
            w[j >> 2] |= c << (8 * (j & 3));
        }
        // tiles past KT (only in the last round of a wave) are never read
        int8_t *qdst = &s_q[wave + t * WAVES][m][kl];
        if constexpr (E == 1) *(uint8_t *)qdst = (uint8_t)w[0];
        else if constexpr (E == 2) *(uint16_t *)qdst = (uint16_t)w[0];
        else if constexpr (E == 4) *(uint32_t *)qdst = w[0];
        else if constexpr (E == 8) *(uint64_t *)qdst = (uint64_t)w[0] | ((uint64_t)w[1] << 32);
        else *(v4i *)qdst = v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
        const int k0 = (wave + t * WAVES) * kTileK + kl;
        if (p.xq_out && writer && row_ok && k0 < p.K) {
            int8_t *dst = p.xq_out + (int64_t)m * p.ldq + k0;
            for (int j = 0; j < E && k0 + j < p.K; ++j) dst[j] = (int8_t)(w[j >> 2] >> (8 * (j & 3)));
        }
    }
    if constexpr (S == 1) __builtin_amdgcn_wave_barrier();
    else __syncthreads();

    // A operands: lane (row lane % 16, k-group lane / 16); rows >= E are zero.
    // Tiles past KT multiply zero weights (no branch around the MFMA).
    v4i acc = v4i{0, 0, 0, 0};
    const int ar = lane & 15;
#pragma unroll
    for (int j = 0; j < TPB; ++j) {
        const int kt = kg + j * WPS;
        const int ktc = min(kt, TPQ * WAVES - 1);
        v4i af = *(const v4i *)(&s_q[ktc][ar < E ? ar : 0][(lane >> 4) * 16]);
        if (ar >= E || kt >= KT) af = v4i{0, 0, 0, 0};
        acc = mfma_i8(af, bf[j], acc);
    }
    __builtin_amdgcn_wave_barrier();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * (lane >> 4) + i;
        if (r < E) s_red[r][lane & 15][wave] = acc[i];
    }
    __syncthreads();
    // the strip's outputs: E rows x 16 columns over its WPS wavefronts
    // (summed in wave order: int32, so the order changes no bit)
    const int n = strip * kTileN + (lane & 15);
    for (int e = kg * 64 + lane; e < E * 16; e += WPS * 64) {
        const int mo = e >> 4;
        if (strip_ok && mo < p.M && n < p.N) {
            const int32_t *src = &s_red[mo][e & 15][slot * WPS];
            uint32_t v = 0u;  // wrapping int32 sum
            if constexpr (WPS % 4 == 0) {
#pragma unroll
                for (int ww = 0; ww < WPS; ww += 4) {
                    const v4i t = *(const v4i *)(src + ww);
                    v += ((uint32_t)t[0] + (uint32_t)t[1]) + ((uint32_t)t[2] + (uint32_t)t[3]);
                }
            } else {
#pragma unroll
                for (int ww = 0; ww < WPS; ++ww) v += (uint32_t)src[ww];
            }
            epilogue_store_c(p, mo, n, v, 0, false, s_scale[mo], 0, col);
        }
    }
}

template <int MT, int WAVES, int TPW, bool AVEC>
hipError_t launch_decode(const Int8GemmParams &p, hipStream_t s) {
    if (p.zBs != 0 || p.zb_col)
        hipLaunchKernelGGL((k_int8_decode<MT, WAVES, TPW, true, AVEC>), dim3((unsigned)p.NS), dim3(WAVES * 64), 0,
                           s, p);
    else
        hipLaunchKernelGGL((k_int8_decode<MT, WAVES, TPW, false, AVEC>), dim3((unsigned)p.NS), dim3(WAVES * 64),
                           0, s, p);
    return hipGetLastError();
}

template <int MT, int D, bool AVEC>
hipError_t launch_wide_d(const Int8GemmParams &p, hipStream_t s) {
    const dim3 grid((unsigned)ceil_div(p.NS, kWideWaves));
    const size_t lds = (size_t)p.KT * MT * 64 * sizeof(v4i);
    if (p.zBs != 0 || p.zb_col)
        hipLaunchKernelGGL((k_int8_decode_wide<MT, D, true, AVEC>), grid, dim3(kWideWaves * 64), lds, s, p);
    else
        hipLaunchKernelGGL((k_int8_decode_wide<MT, D, false, AVEC>), grid, dim3(kWideWaves * 64), lds, s, p);
    return hipGetLastError();
}

template <int MT, bool AVEC>
hipError_t launch_wide(const Int8GemmParams &p, hipStream_t s) {
    if (p.KT * MT > kWideMaxTiles) return hipErrorInvalidValue;
    if (p.KT <= 8) return launch_wide_d<MT, 8, AVEC>(p, s);
    return launch_wide_d<MT, 16, AVEC>(p, s);
}

template <int MT, int D, int MP>
hipError_t launch_wide_q_mp(const Int8GemmParams &p, hipStream_t s) {
    const dim3 grid((unsigned)ceil_div(p.NS, kWideWaves));
    const size_t lds = (size_t)p.KT * MT * 64 * sizeof(v4i);
    const int cpt = (int)ceil_div(p.K / 4, kWideWaves * 64 / MP);
    if (cpt <= 1)
        hipLaunchKernelGGL((k_int8_decode_wide_q<MT, D, MP, 1>), grid, dim3(kWideWaves * 64), lds, s, p);
    else if (cpt <= 2)
        hipLaunchKernelGGL((k_int8_decode_wide_q<MT, D, MP, 2>), grid, dim3(kWideWaves * 64), lds, s, p);
    else if (cpt <= 4)
        hipLaunchKernelGGL((k_int8_decode_wide_q<MT, D, MP, 4>), grid, dim3(kWideWaves * 64), lds, s, p);
    else if (cpt <= 8)
        hipLaunchKernelGGL((k_int8_decode_wide_q<MT, D, MP, 8>), grid, dim3(kWideWaves * 64), lds, s, p);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

template <int MT, int D>
hipError_t launch_wide_q_d(const Int8GemmParams &p, hipStream_t s) {
    // more than 16 rows: two row tiles, the rows rounded up to 32
    if constexpr (MT == 2) {
        return launch_wide_q_mp<2, D, 32>(p, s);
    } else {
        if (p.M <= 1) return launch_wide_q_mp<1, D, 1>(p, s);
        if (p.M <= 2) return launch_wide_q_mp<1, D, 2>(p, s);
        if (p.M <= 4) return launch_wide_q_mp<1, D, 4>(p, s);
        if (p.M <= 8) return launch_wide_q_mp<1, D, 8>(p, s);
        return launch_wide_q_mp<1, D, 16>(p, s);
    }
}

// (waves, tiles per wave) pairs the planner uses: 4x1, 8x1, 16x1, 16x2, 16x4.
template <int MT, bool AVEC>
hipError_t launch_decode_shape(const Int8GemmParams &p, int waves, int tpw, hipStream_t s) {
    if (waves == 4 && tpw == 1) return launch_decode<MT, 4, 1, AVEC>(p, s);
    if (waves == 8 && tpw == 1) return launch_decode<MT, 8, 1, AVEC>(p, s);
    if (waves == 16 && tpw == 1) return launch_decode<MT, 16, 1, AVEC>(p, s);
    if (waves == 16 && tpw == 2) return launch_decode<MT, 16, 2, AVEC>(p, s);
    if (waves == 16 && tpw == 4) return launch_decode<MT, 16, 4, AVEC>(p, s);
    return hipErrorInvalidValue;
}

}  // namespace

// ------------------------------------------------------------ launchers ---

hipError_t launch_pack_b_f32(const float *W, int64_t ldw, const PackedBLayout &L, void *packed,
                             hipStream_t s) {
    PackedHeader h = {kPackMagic, kPackVersion, kPackF32, 0u, L.K, L.N, L.Kp, L.Np, L.scale_off, L.colsum_off};
    int8_t *base = (int8_t *)packed;
    hipLaunchKernelGGL((k_pack_b<false>), dim3((unsigned)L.NS), dim3(256), 0, s, (const void *)W, ldw, 0,
                       (int)L.K, (int)L.N, (int)L.KT, base + L.codes_off, (float *)(base + L.scale_off),
                       (int32_t *)(base + L.colsum_off), (PackedHeader *)base, h);
    return hipGetLastError();
}

hipError_t launch_pack_b_raw(const void *B, int u8, int64_t ldb, const PackedBLayout &L,
                             void *packed, hipStream_t s) {
    PackedHeader h = {kPackMagic, kPackVersion, u8 ? (uint32_t)kPackRawU8 : (uint32_t)kPackRawS8, 0u,
                      L.K, L.N, L.Kp, L.Np, L.scale_off, L.colsum_off};
    int8_t *base = (int8_t *)packed;
    hipLaunchKernelGGL((k_pack_b<true>), dim3((unsigned)L.NS), dim3(256), 0, s, B, ldb, u8, (int)L.K,
                       (int)L.N, (int)L.KT, base + L.codes_off, (float *)(base + L.scale_off),
                       (int32_t *)(base + L.colsum_off), (PackedHeader *)base, h);
    return hipGetLastError();
}

hipError_t launch_quantize_rows(const float *X, int64_t M, int64_t K, int64_t ldx, int8_t *Xq,
                                int64_t ldq, float *row_scale, hipStream_t s) {
    const bool vec = K <= 4096 && K % 4 == 0 && ldx % 4 == 0 && ldq % 4 == 0 && ((uintptr_t)X % 16) == 0 &&
                     ((uintptr_t)Xq % 4) == 0;
    if (vec)
        hipLaunchKernelGGL(k_quantize_rows<true>, dim3((unsigned)M), dim3(256), 0, s, X, ldx, (int)K, Xq, ldq,
                           row_scale);
    else
        hipLaunchKernelGGL(k_quantize_rows<false>, dim3((unsigned)M), dim3(256), 0, s, X, ldx, (int)K, Xq, ldq,
                           row_scale);
    return hipGetLastError();
}

hipError_t launch_int8_gemm(const Int8Plan &plan, Int8GemmParams p, hipStream_t s,
                            const char **variant) {
    if (plan.variant == 2) {
        *variant = plan.mt == 1 ? "int8_decode_wide_m16" : "int8_decode_wide_m32";
        const bool avec = p.a_vec && (p.K % 16) == 0;
        if (plan.mt == 1) return avec ? launch_wide<1, true>(p, s) : launch_wide<1, false>(p, s);
        return avec ? launch_wide<2, true>(p, s) : launch_wide<2, false>(p, s);
    }
    if (plan.variant == 0) {
        *variant = plan.mt == 1 ? "int8_decode_m16" : "int8_decode_m32";
        const bool avec = p.a_vec && (p.K % 16) == 0;
        if (plan.mt == 1)
            return avec ? launch_decode_shape<1, true>(p, plan.waves, plan.tpw, s)
                        : launch_decode_shape<1, false>(p, plan.waves, plan.tpw, s);
        return avec ? launch_decode_shape<2, true>(p, plan.waves, plan.tpw, s)
                    : launch_decode_shape<2, false>(p, plan.waves, plan.tpw, s);
    }
    return launch_int8_prefill(p, s, variant);
}

template <int WAVES, int E, int TPQ, int S, bool GROUPED>
hipError_t launch_dyn(const Int8GemmParams &p, const DecodeGroups &dg, bool avec, hipStream_t s) {
    const unsigned groups = p.rpg > 0 ? (unsigned)((p.M + p.rpg - 1) / p.rpg) : 1u;
    const dim3 g((unsigned)((p.NS + S - 1) / S), groups), b(WAVES * 64);
    GroupArg<GROUPED> ga{};
    if constexpr (GROUPED) ga = dg;
    if (E >= 4 && avec)
        hipLaunchKernelGGL((k_int8_decode_q<WAVES, E, TPQ, S, true, GROUPED>), g, b, 0, s, p, ga);
    else
        hipLaunchKernelGGL((k_int8_decode_q<WAVES, E, TPQ, S, false, GROUPED>), g, b, 0, s, p, ga);
    return hipGetLastError();
}

// strips per workgroup: 1, 2 or 4 (4 only with 8 wavefronts)
template <int WAVES, int E, int TPQ, bool GROUPED>
hipError_t launch_dyn_s(const Int8GemmParams &p, const DecodeGroups &dg, int spw, bool avec, hipStream_t s) {
    if (spw == 1) return launch_dyn<WAVES, E, TPQ, 1, GROUPED>(p, dg, avec, s);
    if (spw == 2) return launch_dyn<WAVES, E, TPQ, 2, GROUPED>(p, dg, avec, s);
    if constexpr (WAVES == 8) {
        if (spw == 4) return launch_dyn<WAVES, E, TPQ, 4, GROUPED>(p, dg, avec, s);
    }
    return hipErrorInvalidValue;
}

// k tiles per wavefront: the power of two >= KT / WAVES.  With 8 wavefronts
// the planner's bound E * K <= 16384 keeps E * TPQ <= 32 (for KT in
// (2^a, 2^(a+1)]: E <= 2^(7-a), TPQ <= 2^(a-2)); 4 wavefronts are planned
// only for KT <= 16 (TPQ <= 4).
template <int WAVES, int E, bool GROUPED>
hipError_t launch_dyn_tpq(const Int8GemmParams &p, const DecodeGroups &dg, int spw, bool avec, hipStream_t s) {
    constexpr int W = WAVES;
    if (p.KT <= W) return launch_dyn_s<WAVES, E, 1, GROUPED>(p, dg, spw, avec, s);
    if constexpr (E * 2 <= 32) {
        if (p.KT <= 2 * W) return launch_dyn_s<WAVES, E, 2, GROUPED>(p, dg, spw, avec, s);
    }
    if constexpr (E * 4 <= 32) {
        if (p.KT <= 4 * W) return launch_dyn_s<WAVES, E, 4, GROUPED>(p, dg, spw, avec, s);
    }
    if constexpr (E * 8 <= 32 && WAVES == 8) {
        if (p.KT <= 8 * W) return launch_dyn_s<WAVES, E, 8, GROUPED>(p, dg, spw, avec, s);
    }
    return hipErrorInvalidValue;
}

template <int E, bool GROUPED>
hipError_t launch_dyn_w(const Int8GemmParams &p, const DecodeGroups &dg, int waves, int spw, bool avec,
                        hipStream_t s) {
    if (waves == 4) return launch_dyn_tpq<4, E, GROUPED>(p, dg, spw, avec, s);
    if (waves == 8) return launch_dyn_tpq<8, E, GROUPED>(p, dg, spw, avec, s);
    return hipErrorInvalidValue;
}

template <bool GROUPED>
hipError_t launch_dyn_rows(const Int8Plan &plan, const Int8GemmParams &p, const DecodeGroups &dg, hipStream_t s) {
    const int rows = p.rpg > 0 ? p.rpg : p.M;  // rows one workgroup quantises
    if (plan.variant != 0 || rows > 16 || p.KT > 64 || p.zBs != 0 || p.zb_col || p.za_row)
        return hipErrorInvalidValue;
    const bool v = p.x_vec && (p.K % 16) == 0;
    const int spw = plan.spw > 0 ? plan.spw : 1;
    const int w = plan.waves > 0 ? plan.waves : 8;
    // E: values per lane, the rows rounded up to a power of two
    if (rows <= 1) return launch_dyn_w<1, GROUPED>(p, dg, w, spw, v, s);
    if (rows <= 2) return launch_dyn_w<2, GROUPED>(p, dg, w, spw, v, s);
    if (rows <= 4) return launch_dyn_w<4, GROUPED>(p, dg, w, spw, v, s);
    if (rows <= 8) return launch_dyn_w<8, GROUPED>(p, dg, w, spw, v, s);
    return launch_dyn_w<16, GROUPED>(p, dg, w, spw, v, s);
}

template <int MP>
hipError_t launch_wide_qp_mp(const Int8GemmParams &p, unsigned grid, hipStream_t s) {
    // K <= 1024: at most K / 4 = 256 chunks a row over 512 / MP threads, so
    // CPT <= MP / 2 (1 below four rows)
    const int cpt = (int)ceil_div(p.K / 4, kWideWaves * 64 / MP);
    auto go = [&](auto C) {
        hipLaunchKernelGGL((k_int8_decode_wide_qp<MP, decltype(C)::value>), dim3(grid), dim3(kWideWaves * 64), 0, s,
                           p);
        return hipGetLastError();
    };
    if (cpt <= 1) return go(std::integral_constant<int, 1>{});
    if constexpr (MP >= 4)
        if (cpt <= 2) return go(std::integral_constant<int, 2>{});
    if constexpr (MP >= 8)
        if (cpt <= 4) return go(std::integral_constant<int, 4>{});
    if constexpr (MP >= 16)
        if (cpt <= 8) return go(std::integral_constant<int, 8>{});
    return hipErrorInvalidValue;
}

hipError_t launch_int8_gemm_dynamic_wide(const Int8GemmParams &p, hipStream_t s, const char **variant) {
    const int mt = p.M <= 16 ? 1 : 2;
    *variant = mt == 1 ? "int8_dynamic_wide_m16" : "int8_dynamic_wide_m32";
    if (p.KT * mt > kWideMaxTiles || p.K % 4 != 0 || !p.x_vec) return hipErrorInvalidValue;
    if (mt == 1 && p.KT <= 16 && p.NS >= kWidePersistStrips) {
        // two workgroups per CU, each quantising the rows once
        *variant = "int8_dynamic_wide_m16p";
        const unsigned g = kWidePersistGrid;
        if (p.M <= 1) return launch_wide_qp_mp<1>(p, g, s);
        if (p.M <= 2) return launch_wide_qp_mp<2>(p, g, s);
        if (p.M <= 4) return launch_wide_qp_mp<4>(p, g, s);
        if (p.M <= 8) return launch_wide_qp_mp<8>(p, g, s);
        return launch_wide_qp_mp<16>(p, g, s);
    }
    if (mt == 1) return p.KT <= 8 ? launch_wide_q_d<1, 8>(p, s) : launch_wide_q_d<1, 16>(p, s);
    return p.KT <= 8 ? launch_wide_q_d<2, 8>(p, s) : launch_wide_q_d<2, 16>(p, s);
}

hipError_t launch_int8_gemm_dynamic(const Int8Plan &plan, Int8GemmParams p, hipStream_t s,
                                    const char **variant) {
    // names carry the strips per workgroup
    static const char *const names[2][3] = {{"int8_dynamic_m16", "int8_dynamic_m16_s2", "int8_dynamic_m16_s4"},
                                            {"int8_dynamic_groups", "int8_dynamic_groups_s2",
                                             "int8_dynamic_groups_s4"}};
    *variant = names[p.rpg > 0][plan.spw == 4 ? 2 : (plan.spw == 2 ? 1 : 0)];
    return launch_dyn_rows<false>(plan, p, DecodeGroups{}, s);
}

hipError_t launch_int8_gemm_dynamic_grouped(const Int8Plan &plan, Int8GemmParams p, const DecodeGroups &g,
                                            hipStream_t s, const char **variant) {
    *variant = plan.spw == 4 ? "int8_dynamic_grouped_s4" : (plan.spw == 2 ? "int8_dynamic_grouped_s2" : "int8_dynamic_grouped");
    return launch_dyn_rows<true>(plan, p, g, s);
}

}  // namespace qmm
