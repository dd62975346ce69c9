// mk_device.h - device helpers shared by the resident interpreter and the
// one-kernel-per-op baseline (bf16 unpacking, wave reductions, the
// activation layout, the attention block update and the op epilogues).
#pragma once
#include <hip/hip_fp16.h>
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

// s_waitcnt vmcnt(n) that is also a compiler barrier: no memory access moves
// across it (the plain builtin is not one, and a store sinking below it, or a
// flag store rising above it, would publish data that has not arrived).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Device-coherent vector accesses (scope bit sc1): they neither hit nor
// leave behind lines that another XCD's L2 may hold stale, so data exchanged
// between workgroups within one launch can move through them without the
// agent-scope cache write-back and invalidate that a release or acquire fence
// costs. Completion (s_waitcnt vmcnt(0)) of such a store makes it visible at
// device scope; the compiler tracks these loads and stores like any other.
constexpr int CP_SC1 = 16;  // cache-policy operand: sc1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void *base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ v4f coherent_load16f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    const v4u v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, CP_SC1);
    return v4f{__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w)};
}
__device__ __forceinline__ float coherent_load4f(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, off, 0, CP_SC1));
}
__device__ __forceinline__ void coherent_store4f(__amdgpu_buffer_rsrc_t r, uint32_t off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, off, 0, CP_SC1);
}

// Tagged activations: one 64-bit word per value, low half the fp32 bits,
// high half the tag of the step that wrote it. A single 64-bit access is
// atomic, so a reader that sees the tag sees the value written with it.
__device__ __forceinline__ void tput(__amdgpu_buffer_rsrc_t r, uint32_t idx, float v, uint32_t tag) {
    __builtin_amdgcn_raw_buffer_store_b64(v2u{__float_as_uint(v), tag}, r, idx * 8u, 0, CP_SC1);
}
__device__ __forceinline__ v2u tget(__amdgpu_buffer_rsrc_t r, uint32_t idx) {
    return __builtin_amdgcn_raw_buffer_load_b64(r, idx * 8u, 0, CP_SC1);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tres(const uint64_t *base, uint32_t words) {
    return coherent_rsrc(base, words * 8u);
}

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf2f(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
// binary16 halves of a 32-bit word, and binary32 -> binary16 (round to nearest even)
__device__ __forceinline__ float h_lo(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w & 0xffffu))); }
__device__ __forceinline__ float h_hi(uint32_t w) { return __half2float(__ushort_as_half((unsigned short)(w >> 16))); }
__device__ __forceinline__ uint16_t f2h(float f) { return __half_as_ushort(__float2half_rn(f)); }

// binary32 -> bf16, round to nearest even (NaN kept quiet).
__device__ __forceinline__ uint16_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40u);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

// Sum over the 64 lanes of a wave, returned to every lane (a scalar): DPP
// row shifts by 1, 2, 4, 8 make lane 15 of each row its row's sum, two row
// broadcasts carry rows 0 and 2 into rows 1 and 3 and then rows 0-1 into
// rows 2-3, and lane 63 ends with the total. Every step is a VALU op; the
// combination order is fixed, so results are bit-reproducible.
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_shift0(float v) {
    // lanes without a source (outside the row, or masked rows) read 0
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, true));
}
__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_shift0<0x111, 0xf>(v);  // row_shr:1
    v += dpp_shift0<0x112, 0xf>(v);  // row_shr:2
    v += dpp_shift0<0x114, 0xf>(v);  // row_shr:4
    v += dpp_shift0<0x118, 0xf>(v);  // row_shr:8
    v += dpp_shift0<0x142, 0xa>(v);  // row_bcast:15 into rows 1 and 3
    v += dpp_shift0<0x143, 0xc>(v);  // row_bcast:31 into rows 2 and 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
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

// A pair of binary16 values (the operand of the packed fp16 dot product).
typedef _Float16 h2v __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h2v as_h2(uint32_t w) { return __builtin_bit_cast(h2v, w); }
// a bf16 pair (low, high half) as a binary16 pair, each rounded to nearest even
__device__ __forceinline__ h2v bf_pair_h2(uint32_t w) { return h2v{(_Float16)bf_lo(w), (_Float16)bf_hi(w)}; }

// dot8 with the weights already converted to fp32 (the same arithmetic)
__device__ __forceinline__ float dot8f(const float (&w)[8], v4f a0, v4f a1) {
    float s = w[0] * a0.x;
    s = fmaf(w[1], a0.y, s);
    s = fmaf(w[2], a0.z, s);
    s = fmaf(w[3], a0.w, s);
    s = fmaf(w[4], a1.x, s);
    s = fmaf(w[5], a1.y, s);
    s = fmaf(w[6], a1.z, s);
    s = fmaf(w[7], a1.w, s);
    return s;
}

// Activation layout in LDS for a matvec input of length K: element i of
// 16-byte weight chunk ci = i / 8 sits where lane ci % 64 of pass ci / 64
// reads it with two conflict-free 16-byte LDS reads.
__device__ __forceinline__ int act_index(int i) {
    const int ci = i >> 3, e8 = i & 7;
    return ((((ci >> 6) << 1) + (e8 >> 2)) << 8) + ((ci & 63) << 2) + (e8 & 3);
}

// Rotate-half RoPE of element i (lane) of a 64-wide head: x_i cos - x_{i+32}
// sin for i < 32, x_i cos + x_{i-32} sin above; xp is the partner element.
// Written with explicit fmaf so that every kernel rounds it the same way.
__device__ __forceinline__ float rope_rotate(float xi, float xp, float2 cs, bool low_half) {
    return low_half ? fmaf(xi, cs.x, -(xp * cs.y)) : fmaf(xi, cs.x, xp * cs.y);
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + expf(-z)); }

// A matvec's activations held in registers at batch 1 with K = 2048: lane
// l's 32 inputs, chunk 64 j + l, elements 8 (64 j + l) + e.
struct RegAct {
    float o[4][8];
};

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// Sum over the 8 lanes of a lane group: quad swaps (lane ^ 1, lane ^ 2), then
// the half-row mirror (lane i <-> 7 - i), which pairs the two quads.
__device__ __forceinline__ float sum8lanes(float v) {
    v += dpp_f<0xB1>(v);   // quad_perm [1, 0, 3, 2]
    v += dpp_f<0x4E>(v);   // quad_perm [2, 3, 0, 1]
    v += dpp_f<0x141>(v);  // row_half_mirror
    return v;
}


// Cross-lane exchanges among the 8 lane groups of a wave (lanes 8 apart):
// the value of lane l ^ 8 (rows of 16 lanes rotated by 8), and the gfx950
// lane swaps, which hand back (a with its upper 32 lanes replaced by b's
// lower 32, b with its lower 32 replaced by a's upper 32) and the same with
// rows of 16 lanes (a's odd rows against b's even rows).
__device__ __forceinline__ float xor8(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xf, 0xf, false));
}
__device__ __forceinline__ float swap32_add(float a, float b) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_add(float a, float b) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_max(float a) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap16_max(float a) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(a), false, false);
    return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// maximum of a value that is the same on the 8 lanes of each group, over
// the groups; every lane gets it
__device__ __forceinline__ float group_max(float v) {
    v = swap32_max(v);
    v = swap16_max(v);
    return fmaxf(v, xor8(v));
}

// Attention over one tile's K/V blocks (16 positions of one kv head each),
// wave by wave: wave w folds blocks w, w + N_COMPUTE_WAVES, ... of the tile,
// in order, into an online-softmax state per query head of the group, kept
// in registers. The lane layout of a block follows the K/V page: lane l holds
// the 16-byte chunk l of K and of V, i.e. dims dd = 8 (l % 8) .. dd + 7 of
// positions t0 = l / 8 and t0 + 8; a position's score q_h . K_t / sqrt(64)
// is the sum over its 8 lanes. Per block and head the wave's running
// maximum M (the same on every lane) rises to the block's, every sum is
// scaled by exp(M_old - M_new), and each lane adds exp(S - M) and
// exp(S - M) V over ITS two positions to its L and to O over its 8 dims;
// positions past the new one score -inf and their values count as zero (a
// missing position may hold any bit pattern). At the end of the tile the 8
// lane groups are added, which gives the wave's state (o[64], m, l) of each
// head; the tile's state is then the merge of the waves' states in wave
// order (merge_step below). No barrier between blocks; the O of the tile is
// unnormalised.
// Above four heads per group the 8 dims x G heads of deferred sums would
// not fit beside the interpreter's other registers: there each block's
// products are summed over the lane groups at once (the halving below), so
// that a lane carries one dim per head and the weight sums are whole.
template <int G>
constexpr bool ATTN_SUM_PER_BLOCK = G > 4;
template <int G>
constexpr int ATTN_ACC_DIMS = ATTN_SUM_PER_BLOCK<G> ? 1 : 8;

template <int G>
struct AttnAcc {
    float O[G][ATTN_ACC_DIMS<G>];  // head h: dims dd .. dd + 7 over the lane's positions (or the lane's dim, summed)
    float L[G];                    // the lane's positions' weights (or the wave's, summed)
    float M[G];                    // the wave's running maximum score
};

template <int G>
__device__ __forceinline__ void attn_acc_init(AttnAcc<G> &a) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
#pragma unroll
        for (int i = 0; i < ATTN_ACC_DIMS<G>; ++i) a.O[h][i] = 0.0f;
        a.L[h] = 0.0f;
        a.M[h] = -1e30f;
    }
}

// Eight values per lane (dims dd .. dd + 7 of the lane's group) added over
// the 8 lane groups by halving: lanes 32 apart add dims 0-3 (lower half) or
// 4-7 (upper half), then rows 16 apart two of those, then lanes 8 apart one
// (each sum of two lanes is the same on both). Lane l ends with dim
// 8 (l % 8) + l / 8.
__device__ __forceinline__ float group_sum_dims(const float (&v)[8], int lane) {
    const bool hi8 = (lane & 8) != 0;
    float v4[4], v2[2];
#pragma unroll
    for (int i = 0; i < 4; ++i) v4[i] = swap32_add(v[i], v[i + 4]);
#pragma unroll
    for (int i = 0; i < 2; ++i) v2[i] = swap16_add(v4[i], v4[i + 2]);
    const float keep = hi8 ? v2[1] : v2[0], send = hi8 ? v2[0] : v2[1];
    return keep + xor8(send);
}
// a value that is the same on the 8 lanes of each group, summed over the
// groups (the same halving), on every lane
__device__ __forceinline__ float group_sum(float v) {
    v = swap32_add(v, v);
    v = swap16_add(v, v);
    return v + xor8(v);
}

// One block into the wave's state; q: the group's rotated queries [G][64]
// fp32 in LDS; ok0 / ok1: positions t0 and t0 + 8 are at or before the new
// one.
template <int G>
__device__ __forceinline__ void attn_acc_block(AttnAcc<G> &a, const MK_LDS float *q, int lane, v4u k0, v4u k1,
                                               v4u v0, v4u v1, bool ok0, bool ok1) {
    const int dd = (lane & 7) * 8;
    if (!ok0) v0 = v4u{0u, 0u, 0u, 0u};
    if (!ok1) v1 = v4u{0u, 0u, 0u, 0u};
    const float va[8] = {bf_lo(v0.x), bf_hi(v0.x), bf_lo(v0.y), bf_hi(v0.y),
                         bf_lo(v0.z), bf_hi(v0.z), bf_lo(v0.w), bf_hi(v0.w)};
    const float vb[8] = {bf_lo(v1.x), bf_hi(v1.x), bf_lo(v1.y), bf_hi(v1.y),
                         bf_lo(v1.z), bf_hi(v1.z), bf_lo(v1.w), bf_hi(v1.w)};
#pragma unroll
    for (int h = 0; h < G; ++h) {
        const v4f qa = *(const MK_LDS v4f *)(q + h * 64 + dd);
        const v4f qb = *(const MK_LDS v4f *)(q + h * 64 + dd + 4);
        float s0 = sum8lanes(dot8(k0, qa, qb)) * 0.125f;  // 1 / sqrt(64)
        float s1 = sum8lanes(dot8(k1, qa, qb)) * 0.125f;
        if (!ok0) s0 = -INFINITY;
        if (!ok1) s1 = -INFINITY;
        const float Mn = fmaxf(a.M[h], group_max(fmaxf(s0, s1)));
        const float sc = __expf(a.M[h] - Mn);
        const float p0 = __expf(s0 - Mn), p1 = __expf(s1 - Mn);
        if constexpr (ATTN_SUM_PER_BLOCK<G>) {
            float t[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) t[i] = fmaf(p1, vb[i], p0 * va[i]);
            a.O[h][0] = fmaf(a.O[h][0], sc, group_sum_dims(t, lane));
            a.L[h] = fmaf(a.L[h], sc, group_sum(p0 + p1));
        } else {
            a.L[h] = fmaf(a.L[h], sc, p0 + p1);
#pragma unroll
            for (int i = 0; i < 8; ++i) a.O[h][i] = fmaf(p1, vb[i], fmaf(p0, va[i], a.O[h][i] * sc));
        }
        a.M[h] = Mn;
    }
}

// The wave's state of every head: lane l's o[h] holds dim 8 (l % 8) + l / 8
// and l[h] the head's weight sum, on every lane (the deferred sums added
// over the lane groups now, or already whole).
template <int G>
__device__ __forceinline__ void attn_acc_finish(const AttnAcc<G> &a, int lane, float (&o)[G], float (&l)[G]) {
#pragma unroll
    for (int h = 0; h < G; ++h) {
        if constexpr (ATTN_SUM_PER_BLOCK<G>) {
            o[h] = a.O[h][0];
            l[h] = a.L[h];
        } else {
            o[h] = group_sum_dims(a.O[h], lane);
            l[h] = group_sum(a.L[h]);
        }
    }
}

// The wave's finished states into st[(w G + h) ATTN_PART + ...] (o[64], m, l).
template <int G>
__device__ __forceinline__ void attn_acc_store(const AttnAcc<G> &a, const float (&o)[G], const float (&l)[G],
                                               MK_LDS float *st, int w, int lane) {
    const int dim = (lane & 7) * 8 + (lane >> 3);
#pragma unroll
    for (int h = 0; h < G; ++h) {
        MK_LDS float *d = st + (w * G + h) * ATTN_PART;
        d[dim] = o[h];
        if (lane == 0) {
            d[64] = a.M[h];
            d[65] = l[h];
        }
    }
}

// Softmax-state merge, one source at a time in a fixed order: (O, M, L)
// absorbs (o, m, l). Every merge of attention states (the waves of a tile,
// the chunks of a kv head) goes through this step, in source order.
__device__ __forceinline__ void merge_step(float &O, float &M, float &L, float o, float m, float l) {
    const float mn = fmaxf(M, m);
    const float a = __expf(M - mn), b = __expf(m - mn);
    O = fmaf(O, a, o * b);
    L = fmaf(L, a, l * b);
    M = mn;
}
__device__ __forceinline__ void merge_init(float &O, float &M, float &L) {
    O = 0.0f;
    M = -1e30f;
    L = 0.0f;
}

// ------------------------------------------------------------ attention split
// "Inference MegaKernel" (shaojiemike.top), section "hand-written whole-model
// MegaKernel / limits": a queue fixed before the step cannot follow requests
// whose lengths differ. The queue here stays fixed - each kv head has T
// attention instructions ("tiles") - but what each tile does is decided on
// the device at every step, from the requests' current lengths: every wave
// that needs the split computes it from the same inputs, so all agree
// without exchanging anything.
//
// Request b covers nb[b] = ceil((p_b + 1) / 16) K/V blocks (positions
// 0..p_b). Balanced: s is the smallest tile size, in blocks, for which
// ceil(nb[b] / s) tiles per request fit in T; request b gets that many tiles,
// the T - sum spare tiles go to the request with the most blocks (the lowest
// index of those), and each request's blocks are cut evenly over its tiles,
// tile j of n getting [j nb / n, (j + 1) nb / n). Per request: T / B tiles
// each. Tiles are numbered request by request; the last tile of a request
// holds its block of position p_b.

// blocks of a request whose newest position is p (clamped to the capacity;
// an out-of-range length is reported by the attention staging)
__device__ __forceinline__ int attn_nblocks(int p, int cap) {
    p = p < 0 ? 0 : (p >= cap ? cap - 1 : p);
    return (p + 16) >> 4;
}

// n[b]: tiles of request b (0 for b >= B). Every lane of the wave takes
// part (the search for s tries 64 sizes at once) and gets the same counts;
// nb and B are the same on every lane; 1 <= B <= T <= MAX_ATTN_TILES.
__device__ __forceinline__ void attn_split_counts(const int (&nb)[MAX_B], int B, int T, bool balanced, int lane,
                                                  int (&n)[MAX_B]) {
    if (!balanced) {
#pragma unroll
        for (int b = 0; b < MAX_B; ++b) n[b] = b < B ? T / B : 0;
        return;
    }
    int N = 0, mx = 0, bm = 0;
#pragma unroll
    for (int b = 0; b < MAX_B; ++b)
        if (b < B) {
            N += nb[b];
            if (nb[b] > mx) {
                mx = nb[b];
                bm = b;
            }
        }
    // f(s) = sum ceil(nb / s) does not increase with s; f(mx) = B <= T, and
    // f(s) <= N / s + B <= T once s >= N / (T - B); f(s) >= N / s > T below
    // ceil(N / T). Each pass tries 64 sizes spread over [lo, hi] (the last
    // one hi) and keeps the gap below the first that fits.
    int lo = max(1, (N + T - 1) / T), hi = mx;
    if (T > B) hi = min(hi, (N + T - B - 1) / (T - B));
    while (lo < hi) {
        const int stride = (hi - lo + 62) / 63;
        const int cand = min(hi, lo + stride * lane);
        int f = 0;
#pragma unroll
        for (int b = 0; b < MAX_B; ++b)
            if (b < B) f += (nb[b] + cand - 1) / cand;
        const uint64_t ok = __builtin_amdgcn_ballot_w64(f <= T);
        const int k = (int)__builtin_ctzll(ok);  // lane 63 holds hi, which fits
        const int ck = __builtin_amdgcn_readlane(cand, k);
        lo = k == 0 ? ck : __builtin_amdgcn_readlane(cand, k - 1) + 1;
        hi = ck;
    }
    int used = 0;
#pragma unroll
    for (int b = 0; b < MAX_B; ++b) {
        n[b] = b < B ? (nb[b] + lo - 1) / lo : 0;
        used += n[b];
    }
#pragma unroll
    for (int b = 0; b < MAX_B; ++b)
        if (b == bm) n[b] += T - used;
}

// Tile t (< sum n): its request b, blocks [lo, hi) of it, and whether it is
// the request's last tile.
__device__ __forceinline__ void attn_split_tile(const int (&nb)[MAX_B], const int (&n)[MAX_B], int t, int &b, int &lo,
                                                int &hi, bool &last) {
    int first = 0, rb = -1, rn = 1, rnb = 0, rf = 0;
#pragma unroll
    for (int j = 0; j < MAX_B; ++j) {
        if (rb < 0 && t < first + n[j]) {
            rb = j;
            rn = n[j];
            rnb = nb[j];
            rf = first;
        }
        first += n[j];
    }
    const int jj = t - rf;
    b = rb;
    lo = jj * rnb / rn;
    hi = (jj + 1) * rnb / rn;
    last = jj == rn - 1;
}

// first tile of request b
__device__ __forceinline__ int attn_split_first(const int (&n)[MAX_B], int b) {
    int f = 0;
#pragma unroll
    for (int j = 0; j < MAX_B; ++j)
        if (j < b) f += n[j];
    return f;
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
