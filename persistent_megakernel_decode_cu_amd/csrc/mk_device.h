// mk_device.h - device helpers shared by the resident interpreter and the
// one-kernel-per-op baseline (bf16 unpacking, wave reductions, the
// activation layout, the attention block update and the op epilogues).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mk_isa.h"
#include "mk_kernels.h"

namespace mk {

#define MK_LDS __attribute__((address_space(3)))
#define MK_CONST __attribute__((address_space(4)))

typedef unsigned int v4u __attribute__((ext_vector_type(4)));
typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef float v4f __attribute__((ext_vector_type(4)));

// Uniform read through the scalar data cache (read-only data: queues, event
// table, page table, lengths, tokens, weight pointer table).
template <typename T>
__device__ __forceinline__ T sload(const T *p, int64_t i) {
    return ((const MK_CONST T *)p)[i];
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }

// binary32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Butterfly sums and maxima: every lane ends with the same value, and the
// combination order is fixed, so results are bit-reproducible.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ float group16_sum(float v) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
    return v;
}
__device__ __forceinline__ float group16_max(float v) {
#pragma unroll
    for (int off = 8; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 64));
    return v;
}

// 8 bf16 weights (one 16-byte chunk) times 8 activations
__device__ __forceinline__ float dot8(v4u w, v4f a0, v4f a1) {
    float s = bf_lo(w.x) * a0.x;
    s = fmaf(bf_hi(w.x), a0.y, s);
    s = fmaf(bf_lo(w.y), a0.z, s);
    s = fmaf(bf_hi(w.y), a0.w, s);
    s = fmaf(bf_lo(w.z), a1.x, s);
    s = fmaf(bf_hi(w.z), a1.y, s);
    s = fmaf(bf_lo(w.w), a1.z, s);
    s = fmaf(bf_hi(w.w), a1.w, s);
    return s;
}

// Activation layout in LDS for a matvec input of length K: element i of
// 16-byte weight chunk ci = i / 8 sits where lane ci % 64 of pass ci / 64
// reads it with two conflict-free 16-byte LDS reads.
__device__ __forceinline__ int act_index(int i) {
    const int ci = i >> 3, e8 = i & 7;
    return ((((ci >> 6) << 1) + (e8 >> 2)) << 8) + ((ci & 63) << 2) + (e8 & 3);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// Online-softmax state of one wave for up to 8 query heads of one kv group:
// lanes are (head-in-pass hl = lane / 16, j = lane % 16); pass p covers heads
// 4p .. 4p+3. m and l are replicated over the 16 lanes of a head; o holds
// dims 4j .. 4j+3 of that head.
struct AttnState {
    float m[2], l[2], o[2][4];
};

__device__ __forceinline__ void attn_init(AttnState &s) {
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        s.m[p] = -1e30f;
        s.l[p] = 0.0f;
#pragma unroll
        for (int e = 0; e < 4; ++e) s.o[p][e] = 0.0f;
    }
}

// One 16-position K/V block. `kchunk(j, ch)` returns 16 bytes (8 bf16) of K
// row j, dims 8ch .. 8ch+7; `vpart(j, q)` returns 8 bytes (4 bf16) of V row
// j, dims 4q .. 4q+3. q_lds: rotated queries [G][68] fp32. nvalid: positions
// of the block that exist (the rest are masked).
template <typename KF, typename VF>
__device__ __forceinline__ void attn_block(AttnState &st, const MK_LDS float *q_lds, int G, int nvalid, int lane,
                                           KF kchunk, VF vpart) {
    const int hl = lane >> 4, j = lane & 15;
    const int npass = (G + 3) >> 2;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        if (p >= npass) break;
        const int hq = p * 4 + hl;
        const bool active = hq < G;
        float s = 0.0f;
        if (active && j < nvalid) {
            const MK_LDS float *qh = q_lds + hq * 68;
#pragma unroll
            for (int kk = 0; kk < 8; ++kk) {
                const int ch = (kk + j) & 7;  // rotate the chunk order across lanes: fewer bank conflicts
                v4u kw = kchunk(j, ch);
                v4f a0 = *(const MK_LDS v4f *)(qh + ch * 8);
                v4f a1 = *(const MK_LDS v4f *)(qh + ch * 8 + 4);
                s += dot8(kw, a0, a1);
            }
            s *= 0.125f;  // 1 / sqrt(64)
        } else {
            s = -INFINITY;
        }
        const float mb = group16_max(s);
        const float mnew = fmaxf(st.m[p], mb);
        const float alpha = __expf(st.m[p] - mnew);
        const float pj = (s == -INFINITY) ? 0.0f : __expf(s - mnew);
        const float ls = group16_sum(pj);
        st.l[p] = st.l[p] * alpha + ls;
#pragma unroll
        for (int e = 0; e < 4; ++e) st.o[p][e] *= alpha;
        for (int jj = 0; jj < nvalid; ++jj) {
            const float pw = __shfl(pj, (hl << 4) + jj, 64);
            v2u vv = vpart(jj, j);
            st.o[p][0] = fmaf(pw, bf_lo(vv.x), st.o[p][0]);
            st.o[p][1] = fmaf(pw, bf_hi(vv.x), st.o[p][1]);
            st.o[p][2] = fmaf(pw, bf_lo(vv.y), st.o[p][2]);
            st.o[p][3] = fmaf(pw, bf_hi(vv.y), st.o[p][3]);
        }
        st.m[p] = mnew;
    }
}

// Writes a wave's state as partials [G][68] (o[64], m, l).
__device__ __forceinline__ void attn_store(const AttnState &st, MK_LDS float *part, int G, int lane) {
    const int hl = lane >> 4, j = lane & 15;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
        const int hq = p * 4 + hl;
        if (hq < G) {
            MK_LDS float *ph = part + hq * 68;
#pragma unroll
            for (int e = 0; e < 4; ++e) ph[j * 4 + e] = st.o[p][e];
            if (j == 0) {
                ph[64] = st.m[p];
                ph[65] = st.l[p];
            }
        }
    }
}


// Merge partial softmax states (o, m, l) of `n` sources in source order;
// lanes are dims. Sources are global (gsrc) or LDS (lsrc), `stride` floats
// apart, laid out [o 0..63, m, l].
__device__ __forceinline__ void merge_parts(const float *gsrc, const MK_LDS float *lsrc, int n, int stride, int lane,
                                            float *o, float *m, float *l) {
    float M = -1e30f;
    for (int i = 0; i < n; ++i) {
        const float mi = gsrc ? gsrc[i * stride + 64] : lsrc[i * stride + 64];
        M = fmaxf(M, mi);
    }
    float L = 0.0f, O = 0.0f;
    for (int i = 0; i < n; ++i) {
        const float mi = gsrc ? gsrc[i * stride + 64] : lsrc[i * stride + 64];
        const float li = gsrc ? gsrc[i * stride + 65] : lsrc[i * stride + 65];
        const float oi = gsrc ? gsrc[i * stride + lane] : lsrc[i * stride + lane];
        const float f = expf(mi - M);
        L = fmaf(li, f, L);
        O = fmaf(oi, f, O);
    }
    *o = O;
    *m = M;
    *l = L;
}

// (value, index) order of the greedy pick: larger value, then lower index
__device__ __forceinline__ bool amax_better(float v, int i, float bv, int bi) {
    return v > bv || (v == bv && i < bi);
}

// residual-stream source of request b, element i: the stream itself, or at
// layer 0 the embedding row of the token / the given hidden vector
__device__ __forceinline__ float x_input(const KParams &P, int b, int i, bool from_input, int tok) {
    if (!from_input) return P.x[(int64_t)b * P.H + i];
    if (P.has_embed) return bf2f(P.embed[(int64_t)tok * P.H + i]);
    return P.hidden_in[(int64_t)b * P.H + i];
}

__device__ __forceinline__ int clamp_token(const KParams &P, int b) {
    const int t = P.tokens_in[b];
    return (t < 0 || t >= P.V) ? 0 : t;
}

__device__ __forceinline__ int op_k(const KParams &P, int op) {
    if (op == OP_OPROJ) return P.nq * P.d;
    if (op == OP_DOWN) return P.F;
    return P.H;
}

// Output of one row r for request b of a matvec op (all but the LM head's
// argmax): v0 is the row's dot product, v1 the up-projection's for UPGATE.
__device__ __forceinline__ void row_epilogue(const KParams &P, int op, int flags, int r, int b, float v0, float v1) {
    if (op == OP_QKV) {
        P.qkv[(int64_t)b * (P.nq + 2 * P.nkv) * P.d + r] = v0;
    } else if (op == OP_OPROJ) {
        const bool from_input = (flags & F_X_FROM_INPUT) != 0;
        const int tok = (from_input && P.has_embed) ? clamp_token(P, b) : 0;
        P.x[(int64_t)b * P.H + r] = x_input(P, b, r, from_input, tok) + v0;
    } else if (op == OP_UPGATE) {
        P.act[(int64_t)b * P.F + r] = silu(v0) * v1;
    } else if (op == OP_DOWN) {
        const float nx = P.x[(int64_t)b * P.H + r] + v0;
        P.x[(int64_t)b * P.H + r] = nx;
        if ((flags & F_WRITE_HIDDEN) && P.hidden_out) P.hidden_out[(int64_t)b * P.H + r] = nx;
    } else if (op == OP_LMHEAD) {
        if (P.logits_out) P.logits_out[(int64_t)b * P.V + r] = v0;
    }
}

}  // namespace mk
