// k_int8_prefill.hip -- the int8 x int8 -> int32 prefill GEMM for gfx950
// (M > 32): LDS-staged tiles, v_mfma_i32_32x32x32_i8, the zero-point
// correction epilogue of "int8 inference" (onemodel docs), "Product kernel
// (Int8Gemm)", and "The ONNX pack", "What works today, and what does not".
#include <type_traits>
#include <utility>

#include "qmm_internal.h"

namespace qmm {

namespace {

#include "int8_common.h"

// -------------------------------------------------------- prefill GEMM ---
// 256 x 128 output tile per workgroup, k step 64, 4 wavefronts in a 2 x 2
// grid each owning 128 x 64: 4 x 2 tiles of v_mfma_i32_32x32x32_i8 (two per
// tile and k step, 128 int32 accumulators per lane).  The 32 x 32 form
// issues one MFMA per 32 cycles even at one wavefront per SIMD (the 16 x 16
// x 64 form reached 2.5 POP/s there, 3.3 at four waves).  A 32 x 32 x 32
// operand takes, for lane L, row (or column) L % 32 and the 16-k chunk
// 2 h + L / 32 of k half h.
//
// Power, not issue, bounds this kernel on random int8 data: the shader
// clock (s_memtime against the 100 MHz s_memrealtime, per workgroup over the
// k loop) runs at 1.83 GHz for the MFMAs alone (554 cycles a k step: the 16
// MFMAs' 512 and the barrier), 1.70 GHz once the operand reads from LDS are
// added and 1.40 GHz with the global-to-LDS copies as well, where the loop
// takes 614 cycles a step.  Fewer cycles a step are bought partly back by
// the clock.
//
// Aligned path (FAST): activations and weight tiles are copied global-to-LDS
// (global_load_lds_dwordx4: no register round trip, no LDS store
// instructions) two k steps at a time into a ring of three pair buffers (see
// the loop); a pair's activations are whole 128-byte rows (copies of 64
// bytes per row, half a cache line, kept the copy path a third slower), laid
// out so that the MFMA operand reads are free of bank conflicts.  General
// path (unaligned A or ragged K): activations are staged through registers
// into 16-row fragments of 64 k in LDS, weights are loaded straight into a
// ring of PF_DEPTH register stages.
//
// In a general-path A fragment the 16-byte piece of (row r, k-chunk g) sits
// at slot 4 r + (g ^ t(r)), t(r) = ((r >> 1) ^ (r >> 3)) & 3: the MFMA reads
// (lane L: row L % 16, one chunk) touch distinct 16-byte bank groups in
// every 8 and every 16 consecutive lanes.  Row and column epilogue operands
// are staged in LDS once.
constexpr int PF_BM = 256, PF_BN = 128, PF_DEPTH = 4;

__device__ __forceinline__ int pf_chunk_perm(int r) { return ((r >> 1) ^ (r >> 3)) & 3; }
// pair layout: chunk swizzle of row r8 (0..7) of a block of parity bp
__device__ __forceinline__ int pf_pair_swz(int r8, int bp) { return (r8 >> 1) | (bp << 2); }
__device__ __forceinline__ int pf_slot(int r, int g) { return 4 * r + (g ^ pf_chunk_perm(r)); }

template <int N>
using ic = std::integral_constant<int, N>;

// f(ic<0>{}), f(ic<1>{}), ..., f(ic<N-1>{})
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
    (f(ic<I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F &&f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Instruction order of one k step of the register-staged path.  With one
// wavefront per SIMD nothing else hides a wait, and left to itself the
// scheduler moves the LDS operand reads for the next step down next to their
// first use (each pair of MFMAs then waits for an LDS round trip).  The order
// pinned here puts one memory instruction between consecutive MFMAs: the
// next step's 8 operand reads, the 4 activation stores, then the 8 global
// loads (two per MFMA).  Of the placements tried (stores grouped at the
// start or the end of the step, loads before the stores) this was fastest.
template <bool HAS_ZB>
__device__ __forceinline__ void pf_schedule_staged() {
    constexpr int MFMA = 0x008, VMEM_RD = 0x020, DS_RD = 0x100, DS_WR = 0x200;
    static_for<8>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(DS_RD, 1, 0);
    });
    static_for<4>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(DS_WR, 1, 0);
    });
    static_for<4>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(VMEM_RD, 2, 0);
    });
    if constexpr (HAS_ZB) __builtin_amdgcn_sched_group_barrier(MFMA, 4, 0);
}

// Step order of the pair path: the 12 operand reads for the next step and
// the step's 6 copies spread between the 16 MFMAs.
template <bool HAS_ZB>
__device__ __forceinline__ void pf_schedule_pair() {
    constexpr int MFMA = 0x008, VMEM = 0x060, DS_RD = 0x100;
    static_for<6>([&](auto) {
        __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(DS_RD, 1, 0);
        __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
        __builtin_amdgcn_sched_group_barrier(DS_RD, 1, 0);
        __builtin_amdgcn_sched_group_barrier(VMEM, 1, 0);
    });
    __builtin_amdgcn_sched_group_barrier(MFMA, 4, 0);
    if constexpr (HAS_ZB) __builtin_amdgcn_sched_group_barrier(MFMA, 4, 0);
}

// s_waitcnt that waits for the vector memory counter only (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at their maxima)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt((63 & 15) | (7 << 4) | (0 << 8) | (3 << 14)); }

// Workgroup barrier for LDS written by this workgroup's own LDS stores and
// by global-to-LDS copies whose completion the caller has already waited for
// (vmcnt).  __syncthreads' release fence would also wait for every
// outstanding global load, including the weight operands and the copies of
// later stages that are meant to stay in flight across the barrier.  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// FAST (A 16-byte aligned, lda % 16 == 0, K % 64 == 0): every global load is
// unconditional, so loads issued for later stages stay in flight (a load
// inside a branch makes the compiler wait for it at the branch's end).  Rows
// past M read row M - 1 and strips past the last read the last strip; those
// products land in outputs that are never stored.  The FAST path copies the
// activations global-to-LDS; the general path stages them through registers
// (masked, shifted for uint8 A, stored to LDS).  FLIP (uint8 A on the FAST
// path): the copies land unshifted and each step flips its own operand
// registers before its MFMAs.
template <bool HAS_ZB, bool FAST, bool FLIP>
__global__ __launch_bounds__(256) void k_int8_prefill(Int8GemmParams p) {
    constexpr int AF = PF_BM / 16;      // A fragments per stage
    constexpr int BF = PF_BN / 16;      // B fragments per stage
    constexpr int ACH = AF * 64 / 256;  // 16-byte A chunks per thread per stage (4)
    constexpr int SA = AF * 1024;  // bytes of one activation stage
    constexpr int SB = BF * 1024;  // bytes of one weight stage (FAST: in LDS after the activations)
    // activation stages in LDS: three for the register-staged path
    __shared__ __attribute__((aligned(16))) int8_t sA[FAST ? 1 : 3][FAST ? 16 : SA];
    // FAST: three pair buffers, each two k steps (128 k) of activations
    // (32 KiB) and weight tiles (16 KiB); one array per buffer, so that the
    // compiler can tell a read of one buffer from copies still landing in
    // another (it waits for every outstanding global-to-LDS copy before a
    // read it cannot separate from them)
    constexpr int SPA = 2 * SA, SPB = 2 * SB;
    constexpr int SP = FAST ? SPA + SPB : 16;
    __shared__ __attribute__((aligned(16))) int8_t sP0[SP], sP1[SP], sP2[SP];
    auto pair_buf = [&](auto B) -> int8_t * {
        constexpr int b = decltype(B)::value;
        if constexpr (b == 0) return sP0;
        else if constexpr (b == 1) return sP1;
        else return sP2;
    };
    __shared__ __attribute__((aligned(16))) float s_rs[PF_BM];
    __shared__ int32_t s_za[PF_BM];
    __shared__ ColOps s_col[PF_BN];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    // Tile order: workgroup ids go round-robin over the 8 XCDs, so id w is
    // first renumbered XCD-major (each XCD's workgroups get consecutive
    // numbers), then numbers run through groups of 4 row tiles column by
    // column: an XCD's resident workgroups share 4 row tiles and a run of
    // column tiles, about a fifth less data through its L2 than a row of
    // tiles (measured 1-3 % faster on the M = 2048 shapes).
    const int tiles_n = (p.NS + BF - 1) / BF;
    const int tiles_m = (p.M + PF_BM - 1) / PF_BM;
    int w = blockIdx.x;
    if (gridDim.x % 8 == 0) w = (w % 8) * (gridDim.x / 8) + w / 8;
    constexpr int GM = 4;
    const int gq = w / (GM * tiles_n), gr = w % (GM * tiles_n);
    const int gm = min(GM, tiles_m - gq * GM);
    const int bm = gq * GM + gr % gm;
    const int bn = gr / gm;
    const int m0 = bm * PF_BM;
    const int strip0 = bn * BF;
    const int KT = p.KT;

    // FAST: a pair buffer holds 128 k of the workgroup's 256 rows as 1 KiB
    // blocks of 8 rows x 128 bytes (whole 128-byte lines of A: copies of 64
    // bytes per row measured a third slower).  Block b holds rows 8 b .. 8 b + 7;
    // the 16-byte chunk c (0..7: k 16 c .. 16 c + 15 of the pair) of row
    // 8 b + r8 sits at slot 8 r8 + (c ^ pf_pair_swz(r8, b)), so a copy's lane L
    // (landing in slot L) reads chunk (L % 8) ^ swz of row 8 b + L / 8, and the
    // MFMA operand reads of 16 consecutive lanes (16 rows, one chunk) touch
    // 16 distinct 16-byte bank groups.  Wave w copies blocks 8 w .. 8 w + 7.
    const int a_r8 = lane >> 3;
    const int a_c0 = (lane & 7) ^ pf_pair_swz(a_r8, 0), a_c1 = (lane & 7) ^ pf_pair_swz(a_r8, 1);
    const int a_row0 = m0 + 64 * wave + a_r8;
    // weight operands of this wave: column tile t (32 columns, strips
    // 2t and 2t+1 of the wave's 4), k half h; strips past the last read the
    // last one (their columns are never stored)
    const int8_t *b_src[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int strip = min(strip0 + wn * 4 + t * 2 + ((lane & 31) >> 4), p.NS - 1);
        b_src[t] = p.codes + (int64_t)strip * KT * kTileBytes;
    }
    v4i ra[PF_DEPTH][ACH], rb[PF_DEPTH][2][2];
    int a_dst[ACH];  // general path: LDS byte offset of thread's piece i of a stage
#pragma unroll
    for (int i = 0; i < ACH; ++i) {
        const int c = tid + 256 * i;
        const int r = c >> 2;
        a_dst[i] = (r >> 4) * 1024 + pf_slot(r & 15, c & 3) * 16;
    }
    // operand read offsets inside a 1 KiB fragment, per k half: chunk 2 h + L / 32
    int a_rd[2], b_rd[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        a_rd[h] = pf_slot(lane & 15, 2 * h + (lane >> 5)) * 16;
        b_rd[h] = ((2 * h + (lane >> 5)) * 16 + (lane & 15)) * 16;  // inside a packed 1 KiB tile
    }
    // FAST: A operand of row R = 32 t + L % 32 of the wave's 128 rows, chunk
    // 4 hs + 2 h + L / 32 of the pair (hs: which k step of the pair): block
    // R / 8, slot 8 (R % 8) + (chunk ^ swz); the tile adds 4 KiB, the wave's
    // row half 16 KiB
    int ap_rd[2][2];
    {
        const int r8 = lane & 7, blk = (lane & 31) >> 3;
        const int swz = pf_pair_swz(r8, blk & 1);
#pragma unroll
        for (int hs = 0; hs < 2; ++hs)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                ap_rd[hs][h] = wm * 16384 + blk * 1024 + (8 * r8 + ((4 * hs + 2 * h + (lane >> 5)) ^ swz)) * 16;
    }
    auto gload = [&](auto slot, int kt) {
        constexpr int sl = decltype(slot)::value;
#pragma unroll
        for (int t = 0; t < 2; ++t)
#pragma unroll
            for (int h = 0; h < 2; ++h) rb[sl][t][h] = *(const v4i *)(b_src[t] + (int64_t)kt * kTileBytes + b_rd[h]);
        if (FAST) return;
#pragma unroll
        for (int i = 0; i < ACH; ++i) {
            const int c = tid + 256 * i;  // (row, k-chunk) = (c >> 2, c & 3)
            ra[sl][i] = load_a16<false>(p, m0 + (c >> 2), kt * kTileK + (c & 3) * 16);
        }
    };
    // FAST: weight tiles of the workgroup's 8 strips: wave w copies strips
    // 2 w and 2 w + 1 (lane L copies 16-byte chunk L of the packed tile, so
    // the LDS image is the tile as stored)
    const int8_t *bt_src[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
        const int strip = min(strip0 + 2 * wave + u, p.NS - 1);
        bt_src[u] = p.codes + (int64_t)strip * KT * kTileBytes + lane * 16;
    }
    // FAST: the activations of pair q (k steps 2 q and 2 q + 1) into pair
    // buffer BUF: 8 copies per wave, each 8 whole rows of 128 bytes; bytes
    // past K (an odd step count's last pair, pairs past the end) read the
    // row's last 16 bytes, which no MFMA of a real step reads
    auto dload_a = [&](auto BUF, int q, auto U0, auto U1) {
        constexpr int b = decltype(BUF)::value;
        const int kb0 = min(q * 2 * kTileK + a_c0 * 16, p.K - 16);
        const int kb1 = min(q * 2 * kTileK + a_c1 * 16, p.K - 16);
#pragma unroll
        for (int u = decltype(U0)::value; u < decltype(U1)::value; ++u) {
            const int row = min(a_row0 + 8 * u, p.M - 1);
            __builtin_amdgcn_global_load_lds((const void *)(p.A + (int64_t)row * p.lda + ((u & 1) ? kb1 : kb0)),
                                             (__attribute__((address_space(3))) void *)(pair_buf(ic<b>{}) + (8 * wave + u) * 1024),
                                             16, 0, 0);
        }
    };
    // FAST: the weight tiles of pair q into pair buffer BUF: 4 copies per
    // wave (strips 2 w, 2 w + 1 for both k steps; tiles past K read the last)
    auto dload_b = [&](auto BUF, int q) {
        constexpr int b = decltype(BUF)::value;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int kt = min(2 * q + (u >> 1), KT - 1);
            __builtin_amdgcn_global_load_lds((const void *)(bt_src[u & 1] + (int64_t)kt * kTileBytes),
                                             (__attribute__((address_space(3))) void *)(pair_buf(ic<b>{}) + SPA + (u >> 1) * SB + (2 * wave + (u & 1)) * 1024),
                                             16, 0, 0);
        }
    };
    auto sstore = [&](auto slot, int buf) {
        constexpr int sl = decltype(slot)::value;
#pragma unroll
        for (int i = 0; i < ACH; ++i) *(v4i *)(&sA[buf][a_dst[i]]) = ra[sl][i];
    };

    v16i acc[4][2];
    v16i accr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        accr[i] = v16i{};
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16i{};
    }
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};

    // activation operands, double-buffered in registers: a step's operands
    // are read from LDS during the previous step's MFMAs.  [tile][k half]
    v4i fa[2][4][2];
    // FAST: weight operands from LDS as well, double-buffered like fa: [tile][k half]
    v4i fb[2][2][2];
    auto lds_frags_at = [&](auto F, const int8_t *base) {
        constexpr int f = decltype(F)::value;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 4; ++t)
                fa[f][t][h] = *(const v4i *)(base + (wm * 8 + t * 2 + ((lane & 31) >> 4)) * 1024 + a_rd[h]);
    };
    auto lds_frags = [&](auto F, int buf) { lds_frags_at(F, &sA[buf][0]); };
    // FAST: step operands from pair buffer base, k step HS of the pair
    auto lds_frags_pair = [&](auto F, auto HS, const int8_t *base) {
        constexpr int f = decltype(F)::value, hs = decltype(HS)::value;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 4; ++t) fa[f][t][h] = *(const v4i *)(base + t * 4096 + ap_rd[hs][h]);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int t = 0; t < 2; ++t)
                fb[f][t][h] = *(const v4i *)(base + SPA + hs * SB + (wn * 4 + t * 2 + ((lane & 31) >> 4)) * 1024 + b_rd[h]);
    };
    // step k: activation set F, weight operands from register slot S (FAST:
    // from operand set F)
    auto mfmas = [&](auto F, auto S) {
        constexpr int f = decltype(F)::value, sl = decltype(S)::value;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
#pragma unroll
                for (int j = 0; j < 2; ++j)
                    acc[i][j] = mfma32_i8(fa[f][i][h], FAST ? fb[f][j][h] : rb[sl][j][h], acc[i][j]);
                if (HAS_ZB) accr[i] = mfma32_i8(fa[f][i][h], ones, accr[i]);
            }
    };

    if constexpr (FAST) {
        // Pair q (k steps 2 q, 2 q + 1) lives in pair buffer q % 3.  Step k
        // reads step k+1's operands, runs the MFMAs of step k and issues 6 of
        // the 12 copies of pair k / 2 + 2 per wavefront (even k: activation
        // copies 0-5; odd k: activation copies 6-7 and the 4 weight copies).
        // That pair's buffer held pair k / 2 - 1, last read in step k - 2
        // (for step k - 1); the barrier after step k - 2 (even) follows each
        // wavefront's wait for its LDS reads, so no copy overwrites data a
        // wavefront still reads.  Only even steps end with a wait and a
        // barrier: step k + 1 (odd) reads step k + 2, the first of pair
        // k / 2 + 1, whose copies were all issued in steps k - 2 and k - 1,
        // so at most the 6 copies of step k may remain outstanding; an odd
        // step's next step reads its own pair, already published.
        dload_a(ic<0>{}, 0, ic<0>{}, ic<8>{});
        dload_b(ic<0>{}, 0);
        dload_a(ic<1>{}, 1, ic<0>{}, ic<8>{});
        dload_b(ic<1>{}, 1);
        __builtin_amdgcn_sched_barrier(0);
        wait_vmcnt<12>();
        lds_barrier();
        lds_frags_pair(ic<0>{}, ic<0>{}, pair_buf(ic<0>{}));
        wait_lgkmcnt0();
        // step base + j, base a multiple of 6 (j fixes the buffers)
        auto pstep = [&](auto J, int kt) {
            constexpr int j = decltype(J)::value;
            lds_frags_pair(ic<(j + 1) & 1>{}, ic<(j + 1) & 1>{}, pair_buf(ic<((j + 1) / 2) % 3>{}));
            if constexpr (FLIP) {
                // uint8 activations: the flip happens on this step's operands,
                // read (and waited for) before the previous barrier
#pragma unroll
                for (int t = 0; t < 4; ++t)
#pragma unroll
                    for (int h = 0; h < 2; ++h) fa[j & 1][t][h] ^= 0x80808080;
            }
            mfmas(ic<j & 1>{}, ic<0>{});
            if constexpr ((j & 1) == 0) {
                dload_a(ic<(j / 2 + 2) % 3>{}, kt / 2 + 2, ic<0>{}, ic<6>{});
                pf_schedule_pair<HAS_ZB>();
                __builtin_amdgcn_sched_barrier(0);
                wait_vmcnt<6>();
                lds_barrier();
            } else {
                dload_a(ic<((j - 1) / 2 + 2) % 3>{}, (kt - 1) / 2 + 2, ic<6>{}, ic<8>{});
                dload_b(ic<((j - 1) / 2 + 2) % 3>{}, (kt - 1) / 2 + 2);
                pf_schedule_pair<HAS_ZB>();
                __builtin_amdgcn_sched_barrier(0);
            }
        };
        const int KT6 = KT - KT % 6;
        for (int base = 0; base < KT6; base += 6)
            static_for<6>([&](auto J) { pstep(J, base + decltype(J)::value); });
        static_for<5>([&](auto J) {
            if (KT6 + decltype(J)::value < KT) pstep(J, KT6 + decltype(J)::value);
        });
        wait_vmcnt<0>();
    } else {
    // General path.  Stage s: register slot s % PF_DEPTH, LDS buffer s % 3,
    // activation operand set s % 2.  Step k: read step k+1's activation
    // operands (LDS buffer written in step k-1, published by its barrier),
    // MFMAs of step k (weight operands in slot k % PF_DEPTH, loaded PF_DEPTH
    // steps ago), store stage k+2's activations (its buffer was last read for
    // step k-1, whose reads completed before the MFMAs of step k-1), load
    // stage k+PF_DEPTH into slot k % PF_DEPTH, barrier.
    const int KTD = KT - KT % PF_DEPTH;
    static_for<PF_DEPTH>([&](auto S) { gload(S, min(decltype(S)::value, KT - 1)); });
    sstore(ic<0>{}, 0);
    sstore(ic<1 % PF_DEPTH>{}, 1);
    __syncthreads();
    lds_frags(ic<0>{}, 0);
    auto step = [&](auto J, int kt) {
        constexpr int j = decltype(J)::value;
        lds_frags(ic<(j + 1) & 1>{}, (kt + 1) % 3);
        mfmas(ic<j & 1>{}, J);
        sstore(ic<(j + 2) % PF_DEPTH>{}, (kt + 2) % 3);
        gload(ic<j>{}, min(kt + PF_DEPTH, KT - 1));
        pf_schedule_staged<HAS_ZB>();
        __syncthreads();
    };
    static_assert(PF_DEPTH % 2 == 0, "fragment sets alternate with the unrolled steps");
    static_assert(PF_DEPTH >= 3, "stage k+2 is stored in step k: it must have been loaded in an earlier step");
    for (int base = 0; base < KTD; base += PF_DEPTH)
        static_for<PF_DEPTH>([&](auto J) { step(J, base + decltype(J)::value); });
    static_for<PF_DEPTH - 1>([&](auto J) {
        if (KTD + decltype(J)::value < KT) step(J, KTD + decltype(J)::value);
    });
    }

    // ---- epilogue.  Row scales and column operands are staged in LDS (the
    // A/B buffers are no longer needed); the common case (fp32 output, no
    // zero points, a whole tile inside M x N) runs without per-element
    // branches.
    for (int r = tid; r < PF_BM; r += 256) {
        const int m = min(m0 + r, p.M - 1);
        const float v = *(p.row_scale ? p.row_scale + m : p.col_scale);
        s_rs[r] = p.row_scale ? v : 1.0f;
        s_za[r] = row_za(p, m);
    }
    if (tid < PF_BN) s_col[tid] = load_colops_c(p, strip0 * kTileN + tid);
    __syncthreads();
    const bool whole = m0 + PF_BM <= p.M && (strip0 + BF) * kTileN <= p.N;
    // accumulator element e of tile (i, j): row i*32 + 8 (e / 4) + 4 (L / 32) + e % 4,
    // column j*32 + L % 32 of the wavefront's 128 x 64 block
    if (!HAS_ZB && p.outputs == QMM_OUT_F32 && p.zAs == 0 && !p.za_row && whole) {
        float cm[2], cb[2];
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const ColOps c = s_col[wn * 64 + j * 32 + (lane & 31)];
            cm[j] = c.cs;
            cb[j] = c.bias_f;
        }
        float *ybase = p.y_f32 + (int64_t)(m0 + wm * 128 + 4 * (lane >> 5)) * p.ld_f32 + strip0 * kTileN +
                       wn * 64 + (lane & 31);
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                const int r0 = i * 32 + 8 * g;
                const v4f rs = *(const v4f *)(&s_rs[wm * 128 + r0 + 4 * (lane >> 5)]);
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    float *yrow = ybase + (int64_t)(r0 + v) * p.ld_f32;
#pragma unroll
                    for (int j = 0; j < 2; ++j) {
                        const float mult = (rs[v] * cm[j]) * p.scale;
                        yrow[j * 32] = fmaf((float)acc[i][j][4 * g + v], mult, cb[j]);
                    }
                }
            }
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int cl = wn * 64 + j * 32 + (lane & 31);
            const int n = strip0 * kTileN + cl;
#pragma unroll
            for (int e = 0; e < 16; ++e) {
                const int rl = wm * 128 + i * 32 + 8 * (e >> 2) + 4 * (lane >> 5) + (e & 3);
                const int m = m0 + rl;
                if (m < p.M && n < p.N)
                    epilogue_store_c(p, m, n, (uint32_t)acc[i][j][e], HAS_ZB ? accr[i][e] : 0, HAS_ZB, s_rs[rl],
                                     s_za[rl], s_col[cl]);
            }
        }
}


// ------------------------------------------------ wide-tile prefill ---
// 256 x 224 output tile (14 strips) per workgroup of 8 wavefronts in a 4 x 2
// grid, each owning 64 rows x 112 columns: 4 x 7 tiles of
// v_mfma_i32_16x16x64_i8 (112 int32 accumulators per lane), two wavefronts
// per SIMD.  It serves shapes whose 256 x 224 tiles fill the CUs in fewer
// rounds of work than the 256 x 128 ones (M = 2048, N = 14336: 512 tiles in
// two rounds against 896 in three and a half), for 16-byte aligned A and
// K % 128 == 0.  Per k step a workgroup copies 23 KB for 3.7 M int8
// operations (the 256 x 128 tile: 24 KB for 4.2 M) and each wavefront reads
// 11 KB of operands from LDS for its 28 MFMAs.
//
// A pair buffer holds two k steps: the 256 rows' activations in the pair
// layout of k_int8_prefill (32 KiB) and the 14 strips' packed weight tiles of
// both steps as stored (28 KiB); two pair buffers (120 KiB).  The 16 x 16 x
// 64 operand of lane L is row (column) L % 16 and 16-k chunk L / 16 of the
// step: for A, chunk c = 4 hs + L / 16 of the pair, in block row / 8 at slot
// 8 (row % 8) + (c ^ swz), so 16 consecutive lanes touch 16 distinct 16-byte
// bank groups; for B, chunk L of the tile.
//
// Pair q sits in buffer q % 2.  Step 2q reads the operands of step 2q+1 and
// runs the MFMAs of step 2q.  Step 2q+1 waits for this wavefront's copies of
// pair q+1 (the only ones in flight), then a barrier: every wavefront has
// its copies of pair q+1 landed and its reads of buffer q % 2 done (step
// 2q+1's operands were read during step 2q).  It then issues the copies of
// pair q+2 into buffer q % 2, reads the operands of step 2q+2 from the other
// buffer and runs its own MFMAs.  Copies and reads past the last pair read
// clamped addresses and land in a buffer no later step reads.
constexpr int PW_S = 14;  // strips of the wide tile (224 columns)

// S strips per tile (14: the 256 x 224 tile), S / 2 per wavefront column
template <int S, bool HAS_ZB, bool FLIP>
__global__ __launch_bounds__(512) void k_int8_prefill_w(Int8GemmParams p) {
    constexpr int BN = 16 * S, JW = S / 2;
    constexpr int NB = (2 * S + 7) / 8;  // weight-tile copies per wavefront and pair
    static_assert(S % 2 == 0 && NB <= 4, "tile width");
    constexpr int SPA = 2 * PF_BM * kTileK;   // a pair's activations: 32 KiB
    constexpr int SPB1 = S * kTileBytes;     // one step's weight tiles (14 KiB at S = 14)
    constexpr int SP = SPA + 2 * SPB1;       // 60 KiB at S = 14
    __shared__ __attribute__((aligned(16))) int8_t sP0[SP], sP1[SP];
    __shared__ __attribute__((aligned(16))) float s_rs[PF_BM];
    __shared__ int32_t s_za[PF_BM];
    __shared__ ColOps s_col[BN];
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave >> 1, wn = wave & 1;
    // tile order of k_int8_prefill: XCD-major renumbering, then groups of 4
    // row tiles walked column by column
    const int tiles_n = (p.NS + S - 1) / S;
    const int tiles_m = (p.M + PF_BM - 1) / PF_BM;
    int w = blockIdx.x;
    if (gridDim.x % 8 == 0) w = (w % 8) * (gridDim.x / 8) + w / 8;
    constexpr int GM = 4;
    const int gq = w / (GM * tiles_n), gr = w % (GM * tiles_n);
    const int gm = min(GM, tiles_m - gq * GM);
    const int bm = gq * GM + gr % gm;
    const int bn = gr / gm;
    const int m0 = bm * PF_BM;
    const int strip0 = bn * S;
    const int KT = p.KT, NP = KT / 2;

    // copies of pair q, 4 + NB per wavefront: activation blocks 4 w .. 4 w + 3
    // (rows 32 w + 8 u + L / 8, whole 128-byte rows), and weight tiles
    // i = w + 8 u of the pair's 2 S (strip i % S of step i / S; where 2 S is
    // not a multiple of 8, the wavefronts past the last tile copy it again:
    // the same bytes to the same place)
    const int a_r8 = lane >> 3;
    const int a_c0 = (lane & 7) ^ pf_pair_swz(a_r8, 0), a_c1 = (lane & 7) ^ pf_pair_swz(a_r8, 1);
    const int a_row0 = m0 + 32 * wave + a_r8;
    const int8_t *bt_src[NB];
    int bt_dst[NB], bt_hs[NB];
#pragma unroll
    for (int u = 0; u < NB; ++u) {
        const int i = min(wave + 8 * u, 2 * S - 1);
        const int sl = i % S, hs = i / S;
        bt_src[u] = p.codes + (int64_t)min(strip0 + sl, p.NS - 1) * KT * kTileBytes + lane * 16;
        bt_dst[u] = SPA + hs * SPB1 + sl * kTileBytes;
        bt_hs[u] = hs;
    }
    auto copy_pair = [&](auto BUF, int q) {
        int8_t *buf = decltype(BUF)::value ? sP1 : sP0;
        const int kb0 = min(q * 2 * kTileK + a_c0 * 16, p.K - 16);
        const int kb1 = min(q * 2 * kTileK + a_c1 * 16, p.K - 16);
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int row = min(a_row0 + 8 * u, p.M - 1);
            __builtin_amdgcn_global_load_lds((const void *)(p.A + (int64_t)row * p.lda + ((u & 1) ? kb1 : kb0)),
                                             (__attribute__((address_space(3))) void *)(buf + (4 * wave + u) * 1024),
                                             16, 0, 0);
        }
#pragma unroll
        for (int u = 0; u < NB; ++u) {
            const int kt = min(2 * q + bt_hs[u], KT - 1);
            __builtin_amdgcn_global_load_lds((const void *)(bt_src[u] + (int64_t)kt * kTileBytes),
                                             (__attribute__((address_space(3))) void *)(buf + bt_dst[u]), 16, 0, 0);
        }
    };

    // operand offsets: A of row tile t (adds 2 KiB per tile) and step hs; B of
    // the wavefront's strip j (adds 1 KiB per strip) and step hs
    int a_rd[2], b_rd[2];
    {
        const int R = lane & 15, r8 = R & 7, blk = 8 * wm + (R >> 3);
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
            const int c = 4 * hs + (lane >> 4);
            a_rd[hs] = blk * 1024 + (8 * r8 + (c ^ pf_pair_swz(r8, blk & 1))) * 16;
            b_rd[hs] = SPA + hs * SPB1 + JW * wn * kTileBytes + lane * 16;
        }
    }
    v4i fa[2][4], fb[2][JW];
    auto read_ops = [&](auto F, auto HS, const int8_t *buf) {
        constexpr int f = decltype(F)::value, hs = decltype(HS)::value;
#pragma unroll
        for (int t = 0; t < 4; ++t) fa[f][t] = *(const v4i *)(buf + a_rd[hs] + t * 2048);
#pragma unroll
        for (int j = 0; j < JW; ++j) fb[f][j] = *(const v4i *)(buf + b_rd[hs] + j * kTileBytes);
    };
    v4i acc[4][JW], accr[4];
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        accr[t] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < JW; ++j) acc[t][j] = v4i{0, 0, 0, 0};
    }
    const v4i ones = {0x01010101, 0x01010101, 0x01010101, 0x01010101};
    auto mfmas = [&](auto F) {
        constexpr int f = decltype(F)::value;
        if constexpr (FLIP) {
            // uint8 activations land unshifted: shift this step's operands
#pragma unroll
            for (int t = 0; t < 4; ++t) fa[f][t] ^= 0x80808080;
        }
#pragma unroll
        for (int j = 0; j < JW; ++j)
#pragma unroll
            for (int t = 0; t < 4; ++t) acc[t][j] = mfma_i8(fa[f][t], fb[f][j], acc[t][j]);
        if constexpr (HAS_ZB) {
#pragma unroll
            for (int t = 0; t < 4; ++t) accr[t] = mfma_i8(fa[f][t], ones, accr[t]);
        }
    };
    // instruction order of a step: the 4 + JW operand reads (and, in odd
    // steps, the 4 + NB copies first) spread between its 4 JW MFMAs
    auto schedule = [&](auto ODD) {
        constexpr int MFMA = 0x008, VMEM = 0x060, DS_RD = 0x100;
        constexpr int odd = decltype(ODD)::value, NC = odd ? 4 + NB : 0;
        if constexpr (odd) {
            static_for<NC>([&](auto) {
                __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
                __builtin_amdgcn_sched_group_barrier(VMEM, 1, 0);
            });
        }
        static_for<4 + JW>([&](auto) {
            __builtin_amdgcn_sched_group_barrier(MFMA, 1, 0);
            __builtin_amdgcn_sched_group_barrier(DS_RD, 1, 0);
        });
        __builtin_amdgcn_sched_group_barrier(MFMA, 4 * JW - NC - (4 + JW), 0);
        if constexpr (HAS_ZB) __builtin_amdgcn_sched_group_barrier(MFMA, 4, 0);
    };

    copy_pair(ic<0>{}, 0);
    copy_pair(ic<1>{}, 1);
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt<4 + NB>();
    lds_barrier();
    read_ops(ic<0>{}, ic<0>{}, sP0);
    auto pair = [&](auto BUF, int q) {
        constexpr int b = decltype(BUF)::value;
        const int8_t *cur = b ? sP1 : sP0;
        const int8_t *nxt = b ? sP0 : sP1;
        // step 2q
        read_ops(ic<1>{}, ic<1>{}, cur);
        mfmas(ic<0>{});
        schedule(ic<0>{});
        __builtin_amdgcn_sched_barrier(0);
        // step 2q + 1
        wait_vmcnt<0>();
        lds_barrier();
        copy_pair(BUF, q + 2);
        read_ops(ic<0>{}, ic<0>{}, nxt);
        mfmas(ic<1>{});
        schedule(ic<1>{});
        __builtin_amdgcn_sched_barrier(0);
    };
    int q = 0;
    for (; q + 1 < NP; q += 2) {
        pair(ic<0>{}, q);
        pair(ic<1>{}, q + 1);
    }
    if (q < NP) pair(ic<0>{}, q);
    wait_vmcnt<0>();

    // ---- epilogue (as k_int8_prefill's): row and column operands in LDS
    for (int r = tid; r < PF_BM; r += 512) {
        const int m = min(m0 + r, p.M - 1);
        const float v = *(p.row_scale ? p.row_scale + m : p.col_scale);
        s_rs[r] = p.row_scale ? v : 1.0f;
        s_za[r] = row_za(p, m);
    }
    if (tid < BN) s_col[tid] = load_colops_c(p, strip0 * kTileN + tid);
    __syncthreads();
    const bool whole = m0 + PF_BM <= p.M && (strip0 + S) * kTileN <= p.N;
    // element e of tile (t, j): row 64 wm + 16 t + 4 (L / 16) + e, column
    // 112 wn + 16 j + L % 16 of the workgroup's tile
    if (!HAS_ZB && p.outputs == QMM_OUT_F32 && p.zAs == 0 && !p.za_row && whole) {
        float cm[JW], cb[JW];
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const ColOps c = s_col[16 * JW * wn + 16 * j + (lane & 15)];
            cm[j] = c.cs;
            cb[j] = c.bias_f;
        }
        float *ybase = p.y_f32 + (int64_t)(m0 + 64 * wm + 4 * (lane >> 4)) * p.ld_f32 + strip0 * kTileN +
                       16 * JW * wn + (lane & 15);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const v4f rs = *(const v4f *)(&s_rs[64 * wm + 16 * t + 4 * (lane >> 4)]);
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                float *yrow = ybase + (int64_t)(16 * t + e) * p.ld_f32;
#pragma unroll
                for (int j = 0; j < JW; ++j) {
                    const float mult = (rs[e] * cm[j]) * p.scale;
                    yrow[16 * j] = fmaf((float)acc[t][j][e], mult, cb[j]);
                }
            }
        }
        return;
    }
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
        for (int j = 0; j < JW; ++j) {
            const int cl = 16 * JW * wn + 16 * j + (lane & 15);
            const int n = strip0 * kTileN + cl;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                const int rl = 64 * wm + 16 * t + 4 * (lane >> 4) + e;
                const int m = m0 + rl;
                if (m < p.M && n < p.N)
                    epilogue_store_c(p, m, n, (uint32_t)acc[t][j][e], HAS_ZB ? accr[t][e] : 0, HAS_ZB, s_rs[rl],
                                     s_za[rl], s_col[cl]);
            }
        }
}

}  // namespace

// The 256 x 224 tile where its tiles fill the CUs in fewer rounds of work:
// each CU's share, rounds of tiles times strips per tile, against the 256 x
// 128 tile's (aligned A, K % 128 == 0 only).
static bool use_wide_tile(const Int8GemmParams &p) {
    constexpr int64_t kCUs = 256;
    if (!p.a_vec || p.K % (2 * kTileK) != 0) return false;
    const int64_t tm = ceil_div(p.M, PF_BM);
    const int64_t t128 = ceil_div(p.NS, PF_BN / kTileN) * tm, t224 = ceil_div(p.NS, PW_S) * tm;
    return ceil_div(t224, kCUs) * PW_S < ceil_div(t128, kCUs) * (PF_BN / kTileN);
}

hipError_t launch_int8_prefill(const Int8GemmParams &p, hipStream_t s, const char **variant) {
    const bool has_zb = p.zBs != 0 || p.zb_col;
    if (use_wide_tile(p)) {
        *variant = "int8_prefill_256x224";
        const dim3 grid((unsigned)(ceil_div(p.NS, PW_S) * ceil_div(p.M, PF_BM))), b(512);
        if (has_zb && p.a_u8)
            hipLaunchKernelGGL((k_int8_prefill_w<PW_S, true, true>), grid, b, 0, s, p);
        else if (has_zb)
            hipLaunchKernelGGL((k_int8_prefill_w<PW_S, true, false>), grid, b, 0, s, p);
        else if (p.a_u8)
            hipLaunchKernelGGL((k_int8_prefill_w<PW_S, false, true>), grid, b, 0, s, p);
        else
            hipLaunchKernelGGL((k_int8_prefill_w<PW_S, false, false>), grid, b, 0, s, p);
        return hipGetLastError();
    }
    *variant = "int8_prefill_256x128";
    dim3 grid((unsigned)(ceil_div(p.NS, PF_BN / kTileN) * ceil_div(p.M, PF_BM)));
    const bool fast = p.a_vec && (p.K % kTileK) == 0;
    const dim3 b(256);
    if (has_zb) {
        if (fast && p.a_u8)
            hipLaunchKernelGGL((k_int8_prefill<true, true, true>), grid, b, 0, s, p);
        else if (fast)
            hipLaunchKernelGGL((k_int8_prefill<true, true, false>), grid, b, 0, s, p);
        else
            hipLaunchKernelGGL((k_int8_prefill<true, false, false>), grid, b, 0, s, p);
    } else {
        if (fast && p.a_u8)
            hipLaunchKernelGGL((k_int8_prefill<false, true, true>), grid, b, 0, s, p);
        else if (fast)
            hipLaunchKernelGGL((k_int8_prefill<false, true, false>), grid, b, 0, s, p);
        else
            hipLaunchKernelGGL((k_int8_prefill<false, false, false>), grid, b, 0, s, p);
    }
    return hipGetLastError();
}

}  // namespace qmm
