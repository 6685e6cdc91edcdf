// k_q4_q8.hip -- q4_1 weights against per-row int8 activations on gfx950.
//
//   Y[m,n] = sa[m] * sum_b ( d[n,b] * sum_{k in b} q[n,k] * xq[m,k]
//                          + m[n,b] * sum_{k in b} xq[m,k] )
//
// "The ONNX pack", "The three layers of the pack", item 2 (every matmul input
// quantised per row with amax/127) and "NPU engine: full ELFs, no xclbin",
// "Q4NX chunks" (W = q*d + m per block of 32 k).  One block of 32 k is one
// v_mfma_i32_16x16x32_i8: the 4-bit codes widen to int8 in two VALU ops per
// 8 codes (the record layout already holds elements 0..3 in the even nibbles
// and 4..7 in the odd ones) and the block dot comes out exact in int32.  A
// second MFMA against an all-ones operand gives the block's row sums for the
// m term.  The fp32 combination y += d*float(D) + m*float(S) is the only
// rounding.
#include "q4_internal.h"

namespace qmm {

namespace {

typedef long i8x8;  // eight int8 operand bytes of one lane

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Eight 4-bit codes of one record word as eight int8 operand bytes, in k order.
__device__ __forceinline__ i8x8 widen_codes(uint32_t w) {
    const uint64_t lo = w & 0x0F0F0F0Fu, hi = (w >> 4) & 0x0F0F0F0Fu;
    return (i8x8)(lo | (hi << 32));
}

// One workgroup per 16-column strip; its WAVES wavefronts take the strip's
// records round-robin (record q to wavefront q % WAVES), R records in flight
// per wavefront, and add their 16 x 16 partial results in LDS in wavefront
// order (deterministic).  Rows 16 (launch's rows) and up read row M-1 and are
// zeroed; records past NQ read record NQ-1 and get d = m = 0; blocks past K
// inside the last record are padding with zero codes and d = m = 0.  Loads
// are never inside branches.  AVEC: Xq and ldq allow aligned 8-byte loads.
template <int WAVES, int R, bool AVEC>
__global__ __launch_bounds__(WAVES * 64) void k_q4_q8(Q4Q8Params p) {
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int strip = blockIdx.x;
    const int r = lane & 15, g = lane >> 4;  // operand lane: row (A) / column (B), k-octet
    const bool row_ok = r < p.M;
    const int8_t *xrow = p.Xq + (int64_t)min(r, p.M - 1) * p.ldq + 8 * g;
    const uint8_t *recs = p.recs + kHeaderBytes + (int64_t)strip * p.NQ * kQ4RecBytes;
    const int kmax = p.K - 32;  // first k of the last block
    const i8x8 ones = 0x0101010101010101L;

    float y[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int q0 = wave; q0 < p.NQ; q0 += WAVES * R) {
        v4i cw[R], dm[R];
        i8x8 a[R][4];
#pragma unroll
        for (int t = 0; t < R; ++t) {
            const int q = min(q0 + WAVES * t, p.NQ - 1);
            const uint8_t *rec = recs + (int64_t)q * kQ4RecBytes;
            cw[t] = *(const v4i *)(rec + lane * 16);
            dm[t] = *(const v4i *)(rec + 1024 + r * 16);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int k0 = min(128 * q + 32 * i, kmax);
                if (AVEC) {
                    a[t][i] = *(const i8x8 *)(xrow + k0);
                } else {
                    uint64_t v = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) v |= (uint64_t)(uint8_t)xrow[k0 + e] << (8 * e);
                    a[t][i] = (i8x8)v;
                }
            }
        }
#pragma unroll
        for (int t = 0; t < R; ++t) {
            const bool rec_ok = q0 + WAVES * t < p.NQ;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const i8x8 av = row_ok ? a[t][i] : (i8x8)0;
                const v4i D = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, widen_codes((uint32_t)cw[t][i]),
                                                                    v4i{0, 0, 0, 0}, 0, 0, 0);
                const v4i S = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, ones, v4i{0, 0, 0, 0}, 0, 0, 0);
                const uint32_t w = rec_ok ? (uint32_t)dm[t][i] : 0u;
                const float d = bf16_lo(w), m = bf16_hi(w);
#pragma unroll
                for (int v = 0; v < 4; ++v) y[v] = fmaf(m, (float)S[v], fmaf(d, (float)D[v], y[v]));
            }
        }
    }

    // lane holds rows 4 g + v, column r of the strip
    __shared__ float s_red[WAVES][16][17];
#pragma unroll
    for (int v = 0; v < 4; ++v) s_red[wave][4 * g + v][r] = y[v];
    __syncthreads();
    if (threadIdx.x < 256) {
        const int row = threadIdx.x >> 4, col = threadIdx.x & 15;
        const int n = strip * 16 + col;
        float acc = 0.0f;
#pragma unroll
        for (int w = 0; w < WAVES; ++w) acc += s_red[w][row][col];
        const float sa = p.row_scale[min(row, p.M - 1)];
        if (row < p.M && n < p.N) p.Y[(int64_t)row * p.ldy + n] = acc * sa;
    }
}

template <int WAVES, int R>
hipError_t launch_q4q8_w(const Q4Q8Params &p, bool avec, hipStream_t s) {
    const dim3 grid((unsigned)p.NS), block(WAVES * 64);
    if (avec)
        hipLaunchKernelGGL((k_q4_q8<WAVES, R, true>), grid, block, 0, s, p);
    else
        hipLaunchKernelGGL((k_q4_q8<WAVES, R, false>), grid, block, 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_q8(const Q4Q8Params &p, hipStream_t s, const char **variant) {
    // 8 wavefronts per strip (4 below 16 records), 2 records in flight per
    // wavefront: measured best of 4/8/16 wavefronts x 2/4/8 records on the
    // 8B shapes (32 and 112 records per strip); deeper rings or more
    // wavefronts than records load clamped duplicates and were up to 6x
    // slower
    const bool avec = ((uintptr_t)p.Xq % 8) == 0 && (p.ldq % 8) == 0;
    *variant = "q4_q8_m16";
    return p.NQ >= 16 ? launch_q4q8_w<8, 2>(p, avec, s) : launch_q4q8_w<4, 2>(p, avec, s);
}

}  // namespace qmm
