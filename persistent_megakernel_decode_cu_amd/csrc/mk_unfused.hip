// mk_unfused.hip - the conventional path: one kernel launch per op, with
// every intermediate materialised in HBM between launches.
//
// "Inference MegaKernel" (shaojiemike.top), section "why conventional
// inference still has bubbles": a step as Norm, QKV GEMM, RoPE, Attention,
// residual, MLP and sampling kernels advanced by host launches, each
// boundary adding launch, tail and materialisation time to T_e2e. This is the
// comparison baseline; it uses the same op math (mk_device.h) as the
// resident interpreter.
#include "mk_device.h"

namespace mk {

namespace {

constexpr int UF_THREADS = 256;
constexpr int UF_WAVES = UF_THREADS / 64;

__device__ __forceinline__ const uint16_t *uf_w(const KParams &P, int layer, int k) {
    return (const uint16_t *)(uintptr_t)P.wtab[(int64_t)layer * 8 + k];
}

// u[b] = rmsnorm(source_b) * w; source: residual stream or layer-0 input
__global__ __launch_bounds__(UF_THREADS) void uf_norm(KParams P, int layer, int which, int from_input, float *u) {
    const uint16_t *wn = which < 0 ? P.final_norm : uf_w(P, layer, which);
    __shared__ float red[UF_WAVES];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int tok = (from_input && P.has_embed) ? clamp_token(P, b) : 0;
    if (from_input && P.has_embed && tid == 0) {
        const int t = P.tokens_in[b];
        if (t < 0 || t >= P.V) atomicCAS(P.err, 0, (ERR_RANGE << 28));
    }
    float ss = 0.0f;
    for (int i = tid; i < P.H; i += UF_THREADS) {
        const float v = x_input(P, b, i, from_input != 0, tok);
        ss = fmaf(v, v, ss);
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.0f;
    for (int w = 0; w < UF_WAVES; ++w) tot += red[w];
    const float inv = 1.0f / sqrtf(tot / (float)P.H + P.eps);
    for (int i = tid; i < P.H; i += UF_THREADS)
        u[(int64_t)b * P.H + i] = x_input(P, b, i, from_input != 0, tok) * inv * bf2f(wn[i]);
}

// One row per wave; in: [B, K] fp32 plain layout.
template <int NB>
__global__ __launch_bounds__(UF_THREADS) void uf_matvec(KParams P, int op, int layer, int flags, const float *in) {
    __shared__ float am_v[UF_WAVES][MAX_B];
    __shared__ int am_i[UF_WAVES][MAX_B];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int K = op_k(P, op);
    const int nchunk = K >> 3;
    const int rows = op == OP_QKV ? (P.nq + 2 * P.nkv) * P.d
                     : op == OP_UPGATE ? P.F
                     : op == OP_LMHEAD ? P.V
                                       : P.H;
    const uint16_t *W0 = op == OP_QKV ? uf_w(P, layer, 1)
                         : op == OP_OPROJ ? uf_w(P, layer, 2)
                         : op == OP_UPGATE ? uf_w(P, layer, 4)
                         : op == OP_DOWN ? uf_w(P, layer, 6)
                                         : P.embed;
    const uint16_t *W1 = op == OP_UPGATE ? uf_w(P, layer, 5) : nullptr;
    const int r = blockIdx.x * UF_WAVES + wave;
    float dot[2][NB];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int b = 0; b < NB; ++b) dot[m][b] = 0.0f;
    if (r < rows) {
        const int nm = op == OP_UPGATE ? 2 : 1;
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            if (m >= nm) break;
            const uint16_t *Wr = (m ? W1 : W0) + (int64_t)r * K;
            float acc[NB];
#pragma unroll
            for (int b = 0; b < NB; ++b) acc[b] = 0.0f;
            for (int ci = lane; ci < nchunk; ci += 64) {
                const v4u w = *(const v4u *)(Wr + ci * 8);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    const v4f a0 = *(const v4f *)(in + (int64_t)b * K + ci * 8);
                    const v4f a1 = *(const v4f *)(in + (int64_t)b * K + ci * 8 + 4);
                    acc[b] += dot8(w, a0, a1);
                }
            }
#pragma unroll
            for (int b = 0; b < NB; ++b) dot[m][b] = wave_sum(acc[b]);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (lane == b) row_epilogue(P, op, flags, r, b, dot[0][b], dot[1][b]);
    }
    if (op == OP_LMHEAD) {
#pragma unroll
        for (int b = 0; b < NB; ++b)
            if (lane == b) {
                const float v = r < rows ? dot[0][b] : -INFINITY;
                if (v != v) atomicCAS(P.err, 0, (ERR_NAN << 28));
                am_v[wave][b] = v;
                am_i[wave][b] = r < rows ? r : 0x7fffffff;
            }
        __syncthreads();
        if (wave == 0 && lane < NB) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int w = 0; w < UF_WAVES; ++w)
                if (amax_better(am_v[w][lane], am_i[w][lane], bv, bi)) {
                    bv = am_v[w][lane];
                    bi = am_i[w][lane];
                }
            P.lm_part[((int64_t)blockIdx.x * P.B + lane) * 2] = bv;
            ((int32_t *)P.lm_part)[((int64_t)blockIdx.x * P.B + lane) * 2 + 1] = bi;
        }
    }
}

// RoPE on the queries (-> qrot) and keys, K/V append as bf16 at position p.
__global__ __launch_bounds__(UF_THREADS) void uf_rope_append(KParams P, int layer, float *qrot) {
    const int b = blockIdx.x, lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int QKVN = (P.nq + 2 * P.nkv) * P.d, QD = P.nq * P.d;
    int p = P.kv_lens[b];
    if (p < 0 || p >= P.T * P.max_pages) {
        if (threadIdx.x == 0) atomicCAS(P.err, 0, (ERR_RANGE << 28));
        return;
    }
    int page = P.page_table[(int64_t)b * P.max_pages + (p >> 4)];
    if (page < 0 || page >= P.n_pages) {
        if (threadIdx.x == 0) atomicCAS(P.err, 0, (ERR_RANGE << 28));
        return;
    }
    const float2 cs = P.rope[(int64_t)p * 32 + (lane & 31)];
    const float *row = P.qkv + (int64_t)b * QKVN;
    const size_t layer_pool = (size_t)P.n_pages * P.nkv * 16 * 64;
    for (int t = wave; t < P.nq + 2 * P.nkv; t += UF_WAVES) {
        const float *src = row + t * 64;  // q heads, then k heads, then v heads
        const float xi = src[lane];
        float out = xi;
        if (t < P.nq + P.nkv) {
            const float xp = src[lane ^ 32];
            out = rope_rotate(xi, xp, cs, lane < 32);
        }
        if (t < P.nq) {
            qrot[(int64_t)b * QD + t * 64 + lane] = out;
        } else {
            const bool is_k = t < P.nq + P.nkv;
            const int g = is_k ? t - P.nq : t - P.nq - P.nkv;
            uint16_t *pool = is_k ? P.k_pool : P.v_pool;
            pool[(size_t)layer * layer_pool + ((size_t)page * P.nkv + g) * 1024 + (p & 15) * 64 + lane] = f2bf(out);
        }
    }
}

// The attention split of the step (mk_device.h), computed by each wave that
// needs it from the request lengths.
__device__ __forceinline__ void uf_split(const KParams &P, int T, int lane, int (&nb)[MAX_B], int (&n)[MAX_B]) {
#pragma unroll
    for (int b = 0; b < MAX_B; ++b) nb[b] = b < P.B ? attn_nblocks(P.kv_lens[b], P.T * P.max_pages) : 0;
    attn_split_counts(nb, P.B, T, P.attn_split == SPLIT_BALANCED, lane, n);
}

// One attention tile (tile c of kv head g: the request and K/V blocks the
// split gives it) per workgroup of N_COMPUTE_WAVES waves: wave w folds blocks
// blo + w, blo + w + N_COMPUTE_WAVES, ... into its own softmax state and the
// head waves merge the waves' states in wave order - the same split, lane
// layout and order as an attention tile of the resident interpreter.
constexpr int UF_ATTN_THREADS = N_COMPUTE_WAVES * 64;

template <int G>
__global__ __launch_bounds__(UF_ATTN_THREADS) void uf_attn(KParams P, int layer, const float *qrot) {
    constexpr int NW = N_COMPUTE_WAVES;
    __shared__ float q[MAX_G * 64];
    __shared__ float st[attn_state_floats(MAX_G)];
    const int c = blockIdx.x, g = blockIdx.y, T = gridDim.x;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int nb[MAX_B], n[MAX_B], b, blo, bhi;
    bool last;
    uf_split(P, T, lane, nb, n);
    attn_split_tile(nb, n, c, b, blo, bhi, last);
    const int p = P.kv_lens[b];
    if (p < 0 || p >= P.T * P.max_pages) return;  // flagged by uf_rope_append
    for (int i = threadIdx.x; i < G * 64; i += UF_ATTN_THREADS) q[i] = qrot[(int64_t)b * P.nq * 64 + (g * G) * 64 + i];
    __syncthreads();
    const size_t layer_pool = (size_t)P.n_pages * P.nkv * 16 * 64;
    MK_LDS float *sts = (MK_LDS float *)st;
    AttnAcc<G> a;
    attn_acc_init(a);
    const int t0 = lane >> 3;
    for (int blk = blo + wave; blk < bhi; blk += NW) {
        int page = P.page_table[(int64_t)b * P.max_pages + blk];
        if (page < 0 || page >= P.n_pages) page = 0;
        const size_t off = (size_t)layer * layer_pool + ((size_t)page * P.nkv + g) * 1024;
        const v4u *kb = (const v4u *)(P.k_pool + off);
        const v4u *vb = (const v4u *)(P.v_pool + off);
        const int pos0 = blk * 16 + t0;
        attn_acc_block<G>(a, (const MK_LDS float *)q, lane, kb[lane], kb[64 + lane], vb[lane], vb[64 + lane],
                          pos0 <= p, pos0 + 8 <= p);
    }
    if (blo + wave < bhi) {
        float o[G], l[G];
        attn_acc_finish<G>(a, lane, o, l);
        attn_acc_store<G>(a, o, l, sts, wave, lane);
    }
    __syncthreads();
    if (wave < G) {
        const int nw = min(NW, bhi - blo);
        float O, M, L;
        merge_init(O, M, L);
        for (int w = 0; w < nw; ++w) {
            const MK_LDS float *s = sts + (w * G + wave) * ATTN_PART;
            merge_step(O, M, L, s[lane], s[64], s[65]);
        }
        float *dst = P.attn_part + (((int64_t)g * T + c) * G + wave) * ATTN_PART_STRIDE;
        dst[lane] = O;
        if (lane == 0) {
            dst[64] = M;
            dst[65] = L;
        }
    }
}

// The states of each request's tiles merged in tile order, then o = O / L:
// one wave per query head of the kv group.
__global__ __launch_bounds__(64 * MAX_G) void uf_attn_merge(KParams P, int T) {
    const int g = blockIdx.x, b = blockIdx.y, lane = threadIdx.x & 63, hq = threadIdx.x >> 6;
    const int G = P.nq / P.nkv;
    if (hq >= G) return;  // whole waves: the block has 64 G threads
    int nb[MAX_B], n[MAX_B];
    uf_split(P, T, lane, nb, n);
    const int first = attn_split_first(n, b), nt = attn_split_first(n, b + 1) - first;
    float O, M, L;
    merge_init(O, M, L);
    for (int c = first; c < first + nt; ++c) {
        const float *src = P.attn_part + (((int64_t)g * T + c) * G + hq) * ATTN_PART_STRIDE;
        merge_step(O, M, L, src[lane], src[64], src[65]);
    }
    P.o[(int64_t)b * P.nq * P.d + (g * G + hq) * 64 + lane] = O / L;
}

// greedy token per request over the LM-head blocks' partials: 1024 threads
// take the partials round-robin, then the waves and the workgroup reduce
// (the pick is a maximum under a total order, so the order does not matter)
constexpr int UF_AMAX_THREADS = 1024;
__global__ __launch_bounds__(UF_AMAX_THREADS) void uf_argmax(KParams P, int nslot) {
    __shared__ float sv[UF_AMAX_THREADS / 64];
    __shared__ int si[UF_AMAX_THREADS / 64];
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    float bv = -INFINITY;
    int bi = 0x7fffffff;
    for (int t = tid; t < nslot; t += UF_AMAX_THREADS) {
        const float v = P.lm_part[((int64_t)t * P.B + b) * 2];
        const int i = ((const int32_t *)P.lm_part)[((int64_t)t * P.B + b) * 2 + 1];
        if (amax_better(v, i, bv, bi)) {
            bv = v;
            bi = i;
        }
    }
    for (int off = 32; off >= 1; off >>= 1) {
        const float ov = __shfl_xor(bv, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (amax_better(ov, oi, bv, bi)) {
            bv = ov;
            bi = oi;
        }
    }
    if (lane == 0) {
        sv[wave] = bv;
        si[wave] = bi;
    }
    __syncthreads();
    if (tid == 0) {
        for (int w = 1; w < UF_AMAX_THREADS / 64; ++w)
            if (amax_better(sv[w], si[w], bv, bi)) {
                bv = sv[w];
                bi = si[w];
            }
        if (P.has_embed) P.tokens_out[b] = bi;
        if (P.kv_lens_out) P.kv_lens_out[b] = P.kv_lens[b] + 1;
    }
}

__global__ void k_rope_table(float2 *t, int capacity, int d, double theta) {
    const int half = d / 2;
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i >= (int64_t)capacity * half) return;
    const int pos = (int)(i / half), k = (int)(i % half);
    const double freq = pow(theta, -2.0 * (double)k / (double)d);
    const double ang = (double)pos * freq;
    t[i] = make_float2((float)cos(ang), (float)sin(ang));
}

template <int NB>
hipError_t uf_mv(const KParams &p, int op, int layer, int flags, const float *in, hipStream_t s) {
    const int rows = op == OP_QKV ? (p.nq + 2 * p.nkv) * p.d : op == OP_UPGATE ? p.F : op == OP_LMHEAD ? p.V : p.H;
    hipLaunchKernelGGL(uf_matvec<NB>, dim3((rows + UF_WAVES - 1) / UF_WAVES), dim3(UF_THREADS), 0, s, p, op, layer,
                       flags, in);
    return hipGetLastError();
}

hipError_t uf_mv_any(const KParams &p, int op, int layer, int flags, const float *in, hipStream_t s) {
    switch (p.B) {
        case 1: return uf_mv<1>(p, op, layer, flags, in, s);
        case 2: return uf_mv<2>(p, op, layer, flags, in, s);
        case 3: return uf_mv<3>(p, op, layer, flags, in, s);
        case 4: return uf_mv<4>(p, op, layer, flags, in, s);
        case 5: return uf_mv<5>(p, op, layer, flags, in, s);
        case 6: return uf_mv<6>(p, op, layer, flags, in, s);
        case 7: return uf_mv<7>(p, op, layer, flags, in, s);
        default: return uf_mv<8>(p, op, layer, flags, in, s);
    }
}

}  // namespace

hipError_t launch_unfused(const KParams &p, float *u, float *qrot, hipStream_t s) {
#define MK_TRY(x)                                 \
    do {                                          \
        hipError_t e_ = (x);                      \
        if (e_ != hipSuccess) return e_;          \
    } while (0)
    const int nt = p.B * p.attn_chunks;  // attention tiles per kv head
    for (int l = 0; l < p.L; ++l) {
        const int first = l == 0 ? F_X_FROM_INPUT : 0;
        const bool last = l == p.L - 1;
        hipLaunchKernelGGL(uf_norm, dim3(p.B), dim3(UF_THREADS), 0, s, p, l, 0, l == 0 ? 1 : 0, u);
        MK_TRY(hipGetLastError());
        MK_TRY(uf_mv_any(p, OP_QKV, l, first, u, s));
        hipLaunchKernelGGL(uf_rope_append, dim3(p.B), dim3(UF_THREADS), 0, s, p, l, qrot);
        MK_TRY(hipGetLastError());
        {
            const dim3 grid(nt, p.nkv), blk(UF_ATTN_THREADS);
            switch (p.nq / p.nkv) {
                case 1: hipLaunchKernelGGL(uf_attn<1>, grid, blk, 0, s, p, l, (const float *)qrot); break;
                case 2: hipLaunchKernelGGL(uf_attn<2>, grid, blk, 0, s, p, l, (const float *)qrot); break;
                case 3: hipLaunchKernelGGL(uf_attn<3>, grid, blk, 0, s, p, l, (const float *)qrot); break;
                case 4: hipLaunchKernelGGL(uf_attn<4>, grid, blk, 0, s, p, l, (const float *)qrot); break;
                case 5: hipLaunchKernelGGL(uf_attn<5>, grid, blk, 0, s, p, l, (const float *)qrot); break;
                case 6: hipLaunchKernelGGL(uf_attn<6>, grid, blk, 0, s, p, l, (const float *)qrot); break;
                case 7: hipLaunchKernelGGL(uf_attn<7>, grid, blk, 0, s, p, l, (const float *)qrot); break;
                default: hipLaunchKernelGGL(uf_attn<8>, grid, blk, 0, s, p, l, (const float *)qrot); break;
            }
        }
        MK_TRY(hipGetLastError());
        hipLaunchKernelGGL(uf_attn_merge, dim3(p.nkv, p.B), dim3(64 * (p.nq / p.nkv)), 0, s, p, nt);
        MK_TRY(hipGetLastError());
        MK_TRY(uf_mv_any(p, OP_OPROJ, l, first, p.o, s));
        hipLaunchKernelGGL(uf_norm, dim3(p.B), dim3(UF_THREADS), 0, s, p, l, 3, 0, u);
        MK_TRY(hipGetLastError());
        MK_TRY(uf_mv_any(p, OP_UPGATE, l, 0, u, s));
        MK_TRY(uf_mv_any(p, OP_DOWN, l, last ? F_WRITE_HIDDEN : 0, p.act, s));
    }
    if (p.has_embed) {
        hipLaunchKernelGGL(uf_norm, dim3(p.B), dim3(UF_THREADS), 0, s, p, 0, -1, 0, u);
        MK_TRY(hipGetLastError());
        MK_TRY(uf_mv_any(p, OP_LMHEAD, p.L, 0, u, s));
    }
    hipLaunchKernelGGL(uf_argmax, dim3(p.B), dim3(UF_AMAX_THREADS), 0, s, p,
                       p.has_embed ? (p.V + UF_WAVES - 1) / UF_WAVES : 0);
    MK_TRY(hipGetLastError());
    return hipSuccess;
#undef MK_TRY
}

hipError_t launch_rope_table(float2 *table, int capacity, int d, double theta, hipStream_t s) {
    const int64_t n = (int64_t)capacity * (d / 2);
    hipLaunchKernelGGL(k_rope_table, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, table, capacity, d, theta);
    return hipGetLastError();
}

}  // namespace mk
