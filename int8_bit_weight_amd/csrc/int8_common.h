// int8_common.h -- device helpers shared by the int8 kernels (k_int8.hip:
// packB, row quantiser, decode; k_int8_prefill.hip: prefill): the epilogue
// with the zero-point correction, its column operands, the 16-byte A loads
// and the int8 MFMA forms.  Included inside namespace qmm's anonymous
// namespace of each source.
#pragma once
// ------------------------------------------------------------- epilogue ---
// Zero-point correction in wrapping int32, then the requested outputs.
//   Y    = S - zA'*colsum[n] - zB'*(rowsum[m] - K*zA')
// (zA' per row and zB' per column with per-axis zero points: the same
// expansion of sum_k (a - zA')(b - zB'), each product with its own pair)
//   mult = fl32(fl32(rs[m]*cs[n]) * scale)
//   F32  = fma(fl32(Y), mult, bias_f32[n])
//   I8/U8: v = fl32(fl32(Y + bias_i32[n]) * mult); clamp(rne(v) + zp_out)
// Column operands of the epilogue for one output column.
struct ColOps {
    int32_t colsum;
    float cs;
    float bias_f;
    int32_t bias_i;
    int32_t zb;  // zB' of the column (shifted domain)
};

// zA' of row m (shifted domain).  Called in the epilogues, after the main
// loads: the load sits in a branch only on the per-axis path.
__device__ __forceinline__ int32_t row_za(const Int8GemmParams &p, int m) {
    return p.za_row ? p.za_row[m] - p.za_off : p.zAs;
}


__device__ __forceinline__ void epilogue_store_c(const Int8GemmParams &p, int m, int n, uint32_t S,
                                                 int32_t rowsum, bool has_zb, float rs, int32_t za,
                                                 const ColOps &c) {
    uint32_t Y = S - (uint32_t)za * (uint32_t)c.colsum;
    if (has_zb) Y -= (uint32_t)c.zb * ((uint32_t)rowsum - (uint32_t)p.K * (uint32_t)za);
    const int32_t y = (int32_t)Y;
    if (p.outputs & QMM_OUT_I32) p.y_i32[(int64_t)m * p.ld_i32 + n] = y;
    if (p.outputs & (QMM_OUT_F32 | QMM_OUT_I8 | QMM_OUT_U8)) {
        const float rc = rs * c.cs;
        const float mult = rc * p.scale;
        if (p.outputs & QMM_OUT_F32) p.y_f32[(int64_t)m * p.ld_f32 + n] = fmaf((float)y, mult, c.bias_f);
        if (p.outputs & (QMM_OUT_I8 | QMM_OUT_U8)) {
            const uint32_t acc = Y + (uint32_t)c.bias_i;
            float v = (float)(int32_t)acc * mult;
            v = fminf(fmaxf(v, -65536.0f), 65536.0f);
            int q = (int)rintf(v) + p.zp_out;
            const int lo = p.q8_u8 ? 0 : -128, hi = p.q8_u8 ? 255 : 127;
            q = q < lo ? lo : (q > hi ? hi : q);
            p.y_q8[(int64_t)m * p.ld_q8 + n] = (int8_t)(uint8_t)q;
        }
    }
}

// 16 bytes of A' (shifted domain) for row `row`, k = k0 .. k0+15; zero where
// row >= M or k >= K.  uint8 A is shifted by flipping the top bit.
template <bool AVEC>
__device__ __forceinline__ v4i load_a16(const Int8GemmParams &p, int row, int k0) {
    const int r = min(row, p.M - 1);
    const int8_t *src = p.A + (int64_t)r * p.lda;
    const uint32_t flip = p.a_u8 ? 0x80808080u : 0u;
    uint32_t w[4];
    if (AVEC) {
        const bool ok = row < p.M && k0 < p.K;
        const v4i v = *(const v4i *)(src + min(k0, p.K - 16));
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = ok ? ((uint32_t)v[i] ^ flip) : 0u;
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = 0u;
#pragma unroll
        for (int j = 0; j < 16; ++j) {
            const uint32_t b = (uint8_t)src[min(k0 + j, p.K - 1)] ^ (flip & 0xFFu);
            w[j >> 2] |= (row < p.M && k0 + j < p.K ? b : 0u) << (8 * (j & 3));
        }
    }
    return v4i{(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
}

// Epilogue operands of column n (loaded for every thread; columns past N
// read column N-1 and are never stored).  Null operands read a valid array
// and are replaced by 0.
// The column operands as loaded (every load in range: absent vectors read
// another column vector instead), and the operands they give.  Kept apart so
// that a kernel loading the next strip's operands ahead does not wait for
// those loads where it selects.
struct ColRaw {
    int32_t colsum, bi, zb;
    float cs, bf;
};

__device__ __forceinline__ ColRaw load_colraw(const Int8GemmParams &p, int n) {
    const int c = min(n, p.N - 1);
    ColRaw r;
    r.bf = (p.bias_f32 ? p.bias_f32 : p.col_scale)[c];
    r.bi = (p.bias_i32 ? p.bias_i32 : p.colsum)[c];
    r.zb = (p.zb_col ? p.zb_col : p.colsum)[c];
    r.colsum = p.colsum[c];
    r.cs = p.col_scale[c];
    return r;
}

__device__ __forceinline__ ColOps colops_of(const Int8GemmParams &p, const ColRaw &r) {
    ColOps o;
    o.colsum = r.colsum;
    o.cs = r.cs;
    o.bias_f = p.bias_f32 ? r.bf : 0.0f;
    o.bias_i = p.bias_i32 ? r.bi : 0;
    o.zb = p.zb_col ? r.zb - p.zb_off : p.zBs;
    return o;
}

__device__ __forceinline__ ColOps load_colops_c(const Int8GemmParams &p, int n) {
    return colops_of(p, load_colraw(p, n));
}

__device__ __forceinline__ v4i mfma_i8(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ v16i mfma32_i8(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}
