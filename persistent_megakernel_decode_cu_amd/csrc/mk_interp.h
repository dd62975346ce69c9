// mk_interp.h - the resident decode interpreter for gfx950 (device code).
//
// Included once per padded batch size by mk_interp_b{1,2,4,8}.hip, which
// instantiate the kernel for each supported head grouping.
//
// "Inference MegaKernel" (shaojiemike.top), section "hand-written whole-model
// MegaKernel / principle, schedule and dataflow": one grid sized to the
// compute-unit count stays resident for the step; each workgroup walks its
// own instruction queue, waits for the inputs of each instruction, runs the
// op body and publishes its results for the consumers on other units. The
// page's design targets one-die GPUs with a coherent L2, so its waits are on
// counters that producers bump after a fence. gfx950 has eight L2s, one per
// XCD, kept coherent only by agent-scope cache write-back / invalidate, and
// measured on this chip a fenced counter hop across 256 workgroups costs
// 7-15 us. So this interpreter moves every activation that crosses compute
// units as a tagged 64-bit word (fp32 value, step tag) written and read with
// device-coherent (sc1) accesses: a consumer polls the data itself, with no
// fence and no counter, and a single 64-bit access makes value and tag
// atomic. Counters are kept only to elect the one workgroup that merges split
// attention chunks and the LM-head argmax.
//
// One workgroup per compute unit, N_COMPUTE_WAVES wave64s, all alike. The
// page leases on-chip pages to prefetch the next op's weights while the
// counter wait is still pending; here each wave keeps PREFETCH_SLICES 4 KiB
// weight slices (or 16-position K/V blocks) in flight in its own registers,
// and the stream of slices runs straight across instruction boundaries: the
// weights and K/V blocks of the next instruction are already landing while
// the wave polls that instruction's inputs. At an instruction boundary the
// waves stage the inputs into LDS together (RMSNorm recomputed where the op
// consumes a norm; RoPE and the K/V append for attention), then each takes
// its round-robin share of rows (or K/V blocks) from the slice stream. The
// last wave to finish an instruction runs its merges. Waves synchronise
// through LDS counters only; every wait loop is bounded by a watchdog, after
// which the wave records an error and the grid drains instead of hanging.
#pragma once
#include "mk_device.h"

namespace mk {

namespace {

// LDS misc area, in 32-bit words
enum : int {
    M_ABORT = 0,
    M_ARRIVE = 1,  // compute-wave barrier arrivals
    M_FIN = 2,     // waves finished with an instruction's slices
    M_DONE = 3,    // instructions fully finished (incl. their merges)
    M_AFIN = 4,    // attention heads merged over the waves (G per instruction)
    M_NQ = 5,      // instructions in the queue (the index of its END), found while copying it
    M_KVLEN = 8,   // [MAX_B] lengths of the requests (read once at start)
    M_NORM = 16,   // [4][MAX_B] sums of squares
    M_AMAX = 64,   // [NC][MAX_B][2] per-wave argmax (value, index)
    // the attention split of a step, one of two areas by
    // the step's parity: the first tile of each request ([MAX_B + 1], at 0),
    // then per tile its request (| 256 on a request's last tile) and its
    // blocks lo | hi << 16 (two words, at SPLIT_TILE)
    M_SPLIT = 256,
    SPLIT_TILE = 16,
    SPLIT_WORDS = SPLIT_TILE + 2 * MAX_ATTN_TILES,
};

constexpr int NC = N_COMPUTE_WAVES;
static_assert(M_AMAX + NC * MAX_B * 2 <= M_SPLIT && M_SPLIT + 2 * SPLIT_WORDS <= MISC_BYTES / 4, "LDS misc area");
// At a padded batch of 8 every matvec input is staged in LDS as binary16,
// request b's K values contiguous at b K (8 requests' fp32 inputs of 8192
// would not fit in LDS, and the batched products read each activation once
// per weight row: binary16 halves those reads and feeds the packed fp16 dot
// product). A norm's input is gathered as fp32 past that area first.
template <int NB>
constexpr bool ACT16 = NB == 8;
constexpr int D = PREFETCH_SLICES;

// Every lane reads the same LDS word; readfirstlane makes that visible to the
// compiler, so that control flow on these flags stays uniform (and the slice
// cursors stay in scalar registers).
__device__ __forceinline__ uint32_t lds_ld(MK_LDS uint32_t *p) {
    return __builtin_amdgcn_readfirstlane(__hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
}
// A word written once before the workgroup's first barrier (the request
// lengths): a plain read, made visibly uniform. An acquire load here would
// wait for the wave's outstanding global loads, the weight slices in flight.
__device__ __forceinline__ uint32_t lds_ld_const(const MK_LDS uint32_t *p) {
    return __builtin_amdgcn_readfirstlane(*p);
}
__device__ __forceinline__ void lds_st(MK_LDS uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ uint32_t lds_add(MK_LDS uint32_t *p, uint32_t v) {
    return __hip_atomic_fetch_add(p, v, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// The lane's index, recomputed where it is used by an opaque two-instruction
// sequence the compiler neither hoists nor merges: lane-derived addresses are
// then rebuilt next to their use instead of living across the whole kernel,
// where register pressure spills them and each reload waits behind every
// weight slice in flight.
__device__ __forceinline__ int lane_id() {
    int l;
    asm volatile("v_mbcnt_lo_u32_b32 %0, -1, 0\n\tv_mbcnt_hi_u32_b32 %0, -1, %0" : "=v"(l));
    return l;
}

// Lane lane ^ m's value (a cross-lane LDS permute addressed with lane_id():
// the runtime's shuffle takes the lane index from a builtin the compiler
// hoists to the kernel's start, where it is spilled and reloaded behind the
// slices in flight).
__device__ __forceinline__ int shfl_xor_i(int v, int m) {
    return __builtin_amdgcn_ds_bpermute((lane_id() ^ m) << 2, v);
}
__device__ __forceinline__ float shfl_xor_f(float v, int m) { return __int_as_float(shfl_xor_i(__float_as_int(v), m)); }

struct Ctx {
    MK_LDS uint32_t *misc;
    const MK_LDS int32_t *q;  // this CU's queue, LDS_INSTR_WORDS words per instruction
    MK_LDS float *act;   // matvec inputs of all requests, or the attention staging
    MK_LDS float *xrow;  // residual rows of the instruction (O projection, down projection)
    int cu, w;
    int nq;              // instructions in this unit's queue (the index of its END)
    bool kv_pending;     // this wave appended a K/V entry in the current attention tile
    uint32_t nbar;
    __device__ __forceinline__ int lane() const { return lane_id(); }
    uint32_t tag;        // copies of kernel arguments the helpers need: taking
    int64_t watchdog;    // the argument block's address would move it to
    int32_t *err;        // private memory
    int32_t *host_err;
    int pending_timeout; // instruction whose LDS-only barrier timed out (-1: none), raised on exit
};

__device__ __forceinline__ void raise_err(Ctx &c, int code, int pc) {
    const int32_t v = (code << 28) | ((c.cu & 0xfff) << 16) | (pc & 0xffff);
    if (atomicCAS(c.err, 0, v) == 0 && c.host_err)
        __hip_atomic_store(c.host_err, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
    lds_st(c.misc + M_ABORT, 1u);
}

// A boolean every lane agrees on, made visibly uniform: return paths that
// pass through lane-conditional code (an error report by lane 0) would
// otherwise make the compiler treat the caller's loop control as divergent.
__device__ __forceinline__ bool uni(bool b) { return __builtin_amdgcn_readfirstlane((int)b) != 0; }

// Wait until *p >= v; false (after raising an error on timeout) if the
// workgroup aborts.
__device__ __forceinline__ bool lds_wait_ge(Ctx &c, MK_LDS uint32_t *p, uint32_t v, int pc) {
    // a target every lane agrees on, made visibly uniform: otherwise the
    // loop's exit is taken for divergent, and so is every value that flows
    // through a barrier in a loop
    v = __builtin_amdgcn_readfirstlane(v);
    if (lds_ld(p) >= v) return true;
    int64_t spins = 0;
    while (lds_ld(p) < v) {
        if (lds_ld(c.misc + M_ABORT)) return false;
        if (++spins > c.watchdog) {
            raise_err(c, ERR_TIMEOUT, pc);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    return true;
}

// barrier of the workgroup's waves (one arrival per wave)
__device__ __forceinline__ bool cbar(Ctx &c, int pc) {
    c.nbar++;
    if (c.lane() == 0) lds_add(c.misc + M_ARRIVE, 1u);
    return lds_wait_ge(c, c.misc + M_ARRIVE, (uint32_t)NC * c.nbar, pc);
}

// Barrier of the workgroup's waves (the same arrival count as cbar) that
// orders only their LDS accesses, with LDS-only fences: a full release would
// first wait for the wave's outstanding global loads, which are the weight
// slices in flight. On a timeout it raises the abort flag and leaves the
// error to be recorded once the wave has left its loops (so that no global
// atomic sits in them).
__device__ __forceinline__ bool lbar(Ctx &c, int pc) {
    c.nbar++;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (c.lane() == 0)
        __hip_atomic_fetch_add(c.misc + M_ARRIVE, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    const uint32_t target = __builtin_amdgcn_readfirstlane((uint32_t)NC * c.nbar);
    int64_t spins = 0;
    while (__builtin_amdgcn_readfirstlane(
               __hip_atomic_load(c.misc + M_ARRIVE, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)) < target) {
        if (__builtin_amdgcn_readfirstlane(
                __hip_atomic_load(c.misc + M_ABORT, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP)))
            return false;
        if (++spins > c.watchdog) {
            c.pending_timeout = pc;
            __hip_atomic_store(c.misc + M_ABORT, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    return true;
}

// LDS counter increment that publishes the wave's earlier LDS accesses only
// (see lbar); returns the old value, read by lane 0
__device__ __forceinline__ uint32_t lds_add_local(MK_LDS uint32_t *p, uint32_t v) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// word `w` of instruction pc, from the LDS copy of the queue
__device__ __forceinline__ int32_t iw(const Ctx &c, int pc, int w) {
    return __builtin_amdgcn_readfirstlane(c.q[pc * LDS_INSTR_WORDS + w]);
}

// Words [w0, w0 + 4) of instruction pc as one 16-byte LDS read (every lane
// the same address): the reads of a record issue together and wait once,
// where a read per word would wait a full LDS round trip each.
typedef int32_t iv4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ iv4 iw4(const Ctx &c, int pc, int w0) {
    return *(const MK_LDS iv4 *)(c.q + pc * LDS_INSTR_WORDS + w0);
}
__device__ __forceinline__ int32_t rfl(int32_t v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t rfl64(int32_t lo, int32_t hi) {
    return (uint64_t)(uint32_t)rfl(lo) | ((uint64_t)(uint32_t)rfl(hi) << 32);
}
static_assert(W_OP == 0 && W_LAYER == 1 && W_R0 == 2 && W_R1 == 3 && W_B == 4 && W_G == 5 && W_C == 6 &&
                  W_NCH == 7 && W_FLAGS == 8 && W_MERGE == 9 && W_SLOT == 10 && W_NSLOT == 11 && W_MCTR == 13 &&
                  W_MNEED == 14 && W_WA == 16 && W_WB == 18 && W_WN == 20 && LDS_INSTR_WORDS % 4 == 0 &&
                  W_WN + 4 <= LDS_INSTR_WORDS,
              "instruction record layout read by iw4");

// The attention split of a step (mk_device.h): every wave writes it, from
// the lengths all waves read, into the step's area at its own start of the
// step (the same values whichever wave writes last), and reads back only
// what it wrote itself. The area of step s is rewritten at step s + 2, which
// no wave starts before every wave has finished step s. The interpreter for
// a single request has no table (its split is the even cut of its blocks).
__device__ __forceinline__ MK_LDS uint32_t *split_area(const Ctx &c, int step) {
    return c.misc + M_SPLIT + (step & 1) * SPLIT_WORDS;
}
// a word of the step's split, as this wave wrote it
__device__ __forceinline__ uint32_t split_word(const Ctx &c, int step, int i) {
    return __builtin_amdgcn_readfirstlane(split_area(c, step)[i]);
}
template <int NB>
__device__ __forceinline__ void split_build(const KParams &P, Ctx &c, int step) {
    if constexpr (NB == 1) return;  // one request: the cursors cut its blocks evenly themselves
    const int lane = lane_id(), T = P.B * P.attn_chunks, cap = P.T * P.max_pages;
    int nb[MAX_B], n[MAX_B];
#pragma unroll
    for (int b = 0; b < MAX_B; ++b)
        nb[b] = b < P.B ? attn_nblocks((int)lds_ld_const(c.misc + M_KVLEN + b) + step, cap) : 0;
    attn_split_counts(nb, P.B, T, P.attn_split == SPLIT_BALANCED, lane, n);
    MK_LDS uint32_t *a = split_area(c, step);
    for (int t = lane; t < T; t += WAVE) {
        int b, lo, hi;
        bool last;
        attn_split_tile(nb, n, t, b, lo, hi, last);
        a[SPLIT_TILE + 2 * t] = (uint32_t)b | (last ? 256u : 0u);
        a[SPLIT_TILE + 2 * t + 1] = (uint32_t)lo | ((uint32_t)hi << 16);
    }
    if (lane <= P.B) a[lane] = (uint32_t)attn_split_first(n, lane);
    // the wave's lanes read one another's words: its LDS accesses stay in order
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
}

// Reads the tagged words idx(k), k < n (n <= N, per lane), until each
// carries the step's tag, handing every value to put(k, v). All outstanding
// loads are issued before any tag is checked. False on abort or timeout.
template <int N, typename IDX, typename PUT>
__device__ __forceinline__ bool tgather(Ctx &c, __amdgpu_buffer_rsrc_t r, int n, IDX idx, PUT put, int pc) {
    static_assert(N >= 1 && N <= 48, "gather width");
    const uint32_t tag = c.tag;
    uint64_t pend = n <= 0 ? 0ull : (n >= N ? ((1ull << N) - 1ull) : ((1ull << n) - 1ull));
    int64_t spins = 0;
    for (;;) {
        v2u wv[N];
#pragma unroll
        for (int k = 0; k < N; ++k)
            if (pend & (1ull << k)) wv[k] = tget(r, idx(k));
#pragma unroll
        for (int k = 0; k < N; ++k)
            if ((pend & (1ull << k)) && wv[k].y == tag) {
                put(k, __uint_as_float(wv[k].x));
                pend &= ~(1ull << k);
            }
        if (__builtin_amdgcn_ballot_w64(pend != 0) == 0) return true;
        if (lds_ld(c.misc + M_ABORT)) return false;
        // a producer on another unit may have failed: then this data never comes
        if ((++spins & 63) == 0 &&
            __builtin_amdgcn_readfirstlane(__hip_atomic_load(c.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))) {
            lds_st(c.misc + M_ABORT, 1u);
            return false;
        }
        if (spins > c.watchdog) {
            raise_err(c, ERR_TIMEOUT, pc);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
    }
}

// Gathers words [lo, hi) of a tagged vector into fn(i, v), the lane taking
// i = lo + lane + 64 k, in rounds of up to 16 words per lane.
template <typename FN>
__device__ __forceinline__ bool tgather_range(Ctx &c, __amdgpu_buffer_rsrc_t r, int lo, int hi, FN fn, int pc) {
    for (int base = lo; base < hi; base += 64 * 16) {
        const int first = base + c.lane();
        const int n = first < hi ? min(16, (hi - first + 63) / 64) : 0;
        if (!tgather<16>(
                c, r, n, [&](int k) { return (uint32_t)(first + 64 * k); },
                [&](int k, float v) { fn(first + 64 * k, v); }, pc))
            return false;
    }
    return true;
}

// Gathers the flattened tagged vector src[0, B K) (B requests of K words)
// with every wave of the workgroup, W words per lane and round, handing
// word (b, i) to put(b, i, v): the gathers of all requests share their
// rounds, where one gather per request would pay one round trip each.
template <int W = 16, typename PUT>
__device__ __forceinline__ bool tgather_batch(Ctx &c, const uint64_t *src, int B, int K, PUT put, int pc) {
    const int total = B * K;
    const __amdgpu_buffer_rsrc_t r = tres(src, (uint32_t)total);
    const float invK = 1.0f / (float)K;
    constexpr int STRIDE = NC * 64;
    for (int base = 0; base < total; base += STRIDE * W) {
        const int first = base + c.w * 64 + c.lane();
        const int n = first < total ? min(W, (total - first + STRIDE - 1) / STRIDE) : 0;
        if (!tgather<W>(
                c, r, n, [&](int k) { return (uint32_t)(first + STRIDE * k); },
                [&](int k, float v) {
                    const int j = first + STRIDE * k;
                    int b = (int)((float)j * invK);  // j < 2^24: off by at most one
                    if (b * K > j) --b;
                    if ((b + 1) * K <= j) ++b;
                    put(b, j - b * K, v);
                },
                pc))
            return false;
    }
    return true;
}

// ------------------------------------------------------------ slice stream

// A wave's position in its stream of slices: instruction pc, unit u (a row,
// a row pair, or a K/V block; the wave's units are w, w + NC, ...), slice s
// of the unit. An instruction in which the wave has no unit still yields one
// empty slice, so that the wave passes through its staging and merges.
struct Cur {
    int step;  // decode step of the launch (a resident launch runs several)
    int pc, op, layer, r0, nu, sp, spm, u, s, K;
    int b, g, blo, p;
    uint32_t rowb;
    uint64_t wa, wb;  // matvec: base of the op's first (gate) and second (up) weight matrix
};

// Instruction pc of step `step` (its END past the queue). The cursors never
// cross a step's END themselves: the main loop restarts them at the next
// step (logic for that here, in the slice loop's path, costs the whole step
// dearly in code quality).
template <int NB>
__device__ __forceinline__ void cur_load(const KParams &P, const Ctx &c, Cur &k, int pc, int step) {
    k.step = step;
    k.pc = pc;
    k.op = OP_END;
    k.u = c.w;
    k.s = 0;
    k.nu = 0;
    k.sp = 1;
    k.spm = 1;
    k.K = 0;
    k.rowb = 0;
    k.wa = k.wb = (uint64_t)(uintptr_t)P.wtab;
    if (pc >= c.nq) return;
    const iv4 a = iw4(c, pc, W_OP), bw = iw4(c, pc, W_B), wq = iw4(c, pc, W_WA);
    k.op = rfl(a[0]);
    if (k.op == OP_END) return;
    k.layer = rfl(a[1]);
    k.r0 = rfl(a[2]);
    if (k.op == OP_ATTN) {
        k.g = rfl(bw[1]);
        const int t = rfl(bw[2]), cap = P.T * P.max_pages;
        int lo, hi;
        if constexpr (NB == 1) {  // one request: tile t of T takes blocks [t nb / T, (t + 1) nb / T)
            const int nb = attn_nblocks((int)lds_ld_const(c.misc + M_KVLEN) + step, cap);
            const uint32_t T = (uint32_t)rfl(bw[3]), rT = (uint32_t)rfl(a[3]);
            k.b = 0;
            // n / T as the high word of n ceil(2^32 / T) (the queue holds the
            // multiplier): exact, since n <= 32 * 65536 and T <= 32
            lo = (int)(T == 1 ? (uint32_t)t * nb : __umulhi((uint32_t)t * nb, rT));
            hi = (int)(T == 1 ? (uint32_t)(t + 1) * nb : __umulhi((uint32_t)(t + 1) * nb, rT));
        } else {
            const uint32_t w0 = split_word(c, step, SPLIT_TILE + 2 * t), w1 = split_word(c, step, SPLIT_TILE + 2 * t + 1);
            k.b = (int)(w0 & (MAX_B - 1));
            lo = (int)(w1 & 0xffffu);
            hi = (int)(w1 >> 16);
        }
        int p = (int)lds_ld_const(c.misc + M_KVLEN + k.b) + step;
        if (p < 0 || p >= cap) p = 0;  // the staging raises the error
        k.p = p;
        k.blo = lo;
        k.nu = hi - lo;
    } else if (k.op == OP_AMERGE) {
        k.nu = 0;  // streams nothing: one empty slice
    } else if (k.op > OP_END && k.op < OP_COUNT) {
        k.K = op_k(P, k.op);
        k.rowb = (uint32_t)k.K * 2;
        k.spm = (int)((k.rowb + SLICE_BYTES - 1) / SLICE_BYTES);
        k.sp = (k.op == OP_UPGATE ? 2 : 1) * k.spm;
        k.nu = rfl(a[3]) - k.r0;
        k.wa = rfl64(wq[0], wq[1]);
        k.wb = rfl64(wq[2], wq[3]);
    }
    // an unknown opcode yields one empty slice; its staging raises the error
}

template <int NB>
__device__ __forceinline__ void cur_next(const KParams &P, const Ctx &c, Cur &k) {
    if (k.op == OP_END) return;
    if (k.u < k.nu) {
        if (++k.s == k.sp) {
            k.s = 0;
            k.u += NC;
        }
        if (k.u < k.nu) return;
    }
    cur_load<NB>(P, c, k, k.pc + 1, k.step);
}

// Buffer resource words for a byte range (gfx950 raw buffer, stride 0):
// loads beyond `bytes` read as zero.
__device__ __forceinline__ v4u rsrc_words(const void *base, uint32_t bytes) {
    const uint64_t a = (uint64_t)(uintptr_t)base;
    return v4u{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, 0x00020000u};
}

// The slices live in registers the compiler never allocates: the kernel asks
// for an occupancy of 3 waves per SIMD, which caps the compiler at 168 VGPRs
// (v0-v167), and slot k occupies v[SLOT_VGPR0 + 16 k, +16). Only the inline
// assembly below names them (their clobber lists make the kernel allocate
// them), so no compiler-generated instruction can read, copy or spill a slot
// while its loads are in flight; the loads are untracked by the compiler, and
// the only wait on them is the s_waitcnt in slot_take(). check_isa.py proves
// these properties on the compiled code.
constexpr int SLOT_VGPR0 = 168;
static_assert(SLOT_VGPR0 + 16 * D <= 256, "slots beyond the VGPR file");

template <int K>
__device__ __forceinline__ void slot_loads(uint32_t o, v4u ra, v4u rb, bool coherent);
template <int K>
__device__ __forceinline__ void slot_take(v2u (&x)[8], int n_wait);


// The four loads of a slot: weights non-temporal (streamed once); K/V blocks
// device-coherent (sc1), since a resident launch appends entries on one XCD
// and reads them back on another with no kernel boundary in between.
#define MK_SLOT_LOADS_ASM(V0, V1, V2, V3, POL)                                        \
    "s_nop 4\n\t"                                                                      \
    "buffer_load_dwordx4 v[" V0 "], %0, %1, 0 offen " POL " ; slot_load\n\t"             \
    "buffer_load_dwordx4 v[" V1 "], %0, %1, 0 offen offset:1024 " POL " ; slot_load\n\t" \
    "buffer_load_dwordx4 v[" V2 "], %0, %2, 0 offen " POL " ; slot_load\n\t"             \
    "buffer_load_dwordx4 v[" V3 "], %0, %2, 0 offen offset:1024 " POL " ; slot_load"
template <>
__device__ __forceinline__ void slot_loads<0>(uint32_t o, v4u ra, v4u rb, bool coherent) {
    if (coherent)
        asm volatile(MK_SLOT_LOADS_ASM("168:171", "172:175", "176:179", "180:183", "sc1")
                     :
                     : "v"(o), "s"(ra), "s"(rb)
                     : "memory", "v168", "v169", "v170", "v171", "v172", "v173", "v174", "v175", "v176", "v177", "v178", "v179", "v180", "v181", "v182", "v183");
    else
        asm volatile(MK_SLOT_LOADS_ASM("168:171", "172:175", "176:179", "180:183", "nt")
                     :
                     : "v"(o), "s"(ra), "s"(rb)
                     : "memory", "v168", "v169", "v170", "v171", "v172", "v173", "v174", "v175", "v176", "v177", "v178", "v179", "v180", "v181", "v182", "v183");
}
template <>
__device__ __forceinline__ void slot_loads<1>(uint32_t o, v4u ra, v4u rb, bool coherent) {
    if (coherent)
        asm volatile(MK_SLOT_LOADS_ASM("184:187", "188:191", "192:195", "196:199", "sc1")
                     :
                     : "v"(o), "s"(ra), "s"(rb)
                     : "memory", "v184", "v185", "v186", "v187", "v188", "v189", "v190", "v191", "v192", "v193", "v194", "v195", "v196", "v197", "v198", "v199");
    else
        asm volatile(MK_SLOT_LOADS_ASM("184:187", "188:191", "192:195", "196:199", "nt")
                     :
                     : "v"(o), "s"(ra), "s"(rb)
                     : "memory", "v184", "v185", "v186", "v187", "v188", "v189", "v190", "v191", "v192", "v193", "v194", "v195", "v196", "v197", "v198", "v199");
}
template <>
__device__ __forceinline__ void slot_loads<2>(uint32_t o, v4u ra, v4u rb, bool coherent) {
    if (coherent)
        asm volatile(MK_SLOT_LOADS_ASM("200:203", "204:207", "208:211", "212:215", "sc1")
                     :
                     : "v"(o), "s"(ra), "s"(rb)
                     : "memory", "v200", "v201", "v202", "v203", "v204", "v205", "v206", "v207", "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215");
    else
        asm volatile(MK_SLOT_LOADS_ASM("200:203", "204:207", "208:211", "212:215", "nt")
                     :
                     : "v"(o), "s"(ra), "s"(rb)
                     : "memory", "v200", "v201", "v202", "v203", "v204", "v205", "v206", "v207", "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215");
}
template <>
__device__ __forceinline__ void slot_loads<3>(uint32_t o, v4u ra, v4u rb, bool coherent) {
    if (coherent)
        asm volatile(MK_SLOT_LOADS_ASM("216:219", "220:223", "224:227", "228:231", "sc1")
                     :
                     : "v"(o), "s"(ra), "s"(rb)
                     : "memory", "v216", "v217", "v218", "v219", "v220", "v221", "v222", "v223", "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231");
    else
        asm volatile(MK_SLOT_LOADS_ASM("216:219", "220:223", "224:227", "228:231", "nt")
                     :
                     : "v"(o), "s"(ra), "s"(rb)
                     : "memory", "v216", "v217", "v218", "v219", "v220", "v221", "v222", "v223", "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231");
}
#undef MK_SLOT_LOADS_ASM
template <>
__device__ __forceinline__ void slot_take<0>(v2u (&x)[8], int n_wait) {
    if (n_wait == 0)  // a constant at every call site
        asm volatile("s_waitcnt vmcnt(0) ; slot_wait" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(%0) ; slot_wait" ::"i"(4 * (D - 1)) : "memory");
    asm volatile(
        "v_mov_b64 %0, v[168:169] ; slot_take\n\t"
        "v_mov_b64 %1, v[170:171] ; slot_take\n\t"
        "v_mov_b64 %2, v[172:173] ; slot_take\n\t"
        "v_mov_b64 %3, v[174:175] ; slot_take\n\t"
        "v_mov_b64 %4, v[176:177] ; slot_take\n\t"
        "v_mov_b64 %5, v[178:179] ; slot_take\n\t"
        "v_mov_b64 %6, v[180:181] ; slot_take\n\t"
        "v_mov_b64 %7, v[182:183] ; slot_take"
        : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7])
        :
        : "memory", "v168", "v169", "v170", "v171", "v172", "v173", "v174", "v175", "v176", "v177", "v178", "v179", "v180", "v181", "v182", "v183");
}
template <>
__device__ __forceinline__ void slot_take<1>(v2u (&x)[8], int n_wait) {
    if (n_wait == 0)  // a constant at every call site
        asm volatile("s_waitcnt vmcnt(0) ; slot_wait" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(%0) ; slot_wait" ::"i"(4 * (D - 1)) : "memory");
    asm volatile(
        "v_mov_b64 %0, v[184:185] ; slot_take\n\t"
        "v_mov_b64 %1, v[186:187] ; slot_take\n\t"
        "v_mov_b64 %2, v[188:189] ; slot_take\n\t"
        "v_mov_b64 %3, v[190:191] ; slot_take\n\t"
        "v_mov_b64 %4, v[192:193] ; slot_take\n\t"
        "v_mov_b64 %5, v[194:195] ; slot_take\n\t"
        "v_mov_b64 %6, v[196:197] ; slot_take\n\t"
        "v_mov_b64 %7, v[198:199] ; slot_take"
        : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7])
        :
        : "memory", "v184", "v185", "v186", "v187", "v188", "v189", "v190", "v191", "v192", "v193", "v194", "v195", "v196", "v197", "v198", "v199");
}
template <>
__device__ __forceinline__ void slot_take<2>(v2u (&x)[8], int n_wait) {
    if (n_wait == 0)  // a constant at every call site
        asm volatile("s_waitcnt vmcnt(0) ; slot_wait" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(%0) ; slot_wait" ::"i"(4 * (D - 1)) : "memory");
    asm volatile(
        "v_mov_b64 %0, v[200:201] ; slot_take\n\t"
        "v_mov_b64 %1, v[202:203] ; slot_take\n\t"
        "v_mov_b64 %2, v[204:205] ; slot_take\n\t"
        "v_mov_b64 %3, v[206:207] ; slot_take\n\t"
        "v_mov_b64 %4, v[208:209] ; slot_take\n\t"
        "v_mov_b64 %5, v[210:211] ; slot_take\n\t"
        "v_mov_b64 %6, v[212:213] ; slot_take\n\t"
        "v_mov_b64 %7, v[214:215] ; slot_take"
        : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7])
        :
        : "memory", "v200", "v201", "v202", "v203", "v204", "v205", "v206", "v207", "v208", "v209", "v210", "v211", "v212", "v213", "v214", "v215");
}
template <>
__device__ __forceinline__ void slot_take<3>(v2u (&x)[8], int n_wait) {
    if (n_wait == 0)  // a constant at every call site
        asm volatile("s_waitcnt vmcnt(0) ; slot_wait" ::: "memory");
    else
        asm volatile("s_waitcnt vmcnt(%0) ; slot_wait" ::"i"(4 * (D - 1)) : "memory");
    asm volatile(
        "v_mov_b64 %0, v[216:217] ; slot_take\n\t"
        "v_mov_b64 %1, v[218:219] ; slot_take\n\t"
        "v_mov_b64 %2, v[220:221] ; slot_take\n\t"
        "v_mov_b64 %3, v[222:223] ; slot_take\n\t"
        "v_mov_b64 %4, v[224:225] ; slot_take\n\t"
        "v_mov_b64 %5, v[226:227] ; slot_take\n\t"
        "v_mov_b64 %6, v[228:229] ; slot_take\n\t"
        "v_mov_b64 %7, v[230:231] ; slot_take"
        : "=v"(x[0]), "=v"(x[1]), "=v"(x[2]), "=v"(x[3]), "=v"(x[4]), "=v"(x[5]), "=v"(x[6]), "=v"(x[7])
        :
        : "memory", "v216", "v217", "v218", "v219", "v220", "v221", "v222", "v223", "v224", "v225", "v226", "v227", "v228", "v229", "v230", "v231");
}

// Issues the loads of the slice at the cursor into slot K: always four
// 16-byte buffer loads per lane (two per 2 KiB half), so that the count of
// loads in flight per slot is fixed; bytes outside the slice read as zero.
template <int K>
__device__ __forceinline__ void issue(const KParams &P, const Cur &k, int lane) {
    const char *a = (const char *)P.wtab, *b = (const char *)P.wtab;
    uint32_t na = 0, nb = 0;
    if (k.op != OP_END && k.u < k.nu) {
        if (k.op == OP_ATTN) {
            const int blk = k.blo + k.u;
            int page = sload(P.page_table, (int64_t)k.b * P.max_pages + blk);
            if (page < 0 || page >= P.n_pages) page = 0;  // the staging raises the error
            const size_t off = (((size_t)k.layer * P.n_pages + page) * P.nkv + k.g) * 2048;
            a = (const char *)P.k_pool + off;
            b = (const char *)P.v_pool + off;
            na = nb = 2048;
        } else {
            const int m = k.s >= k.spm ? 1 : 0, part = k.s - m * k.spm;
            const uint32_t col0 = (uint32_t)part * SLICE_BYTES;
            a = (const char *)(uintptr_t)(m ? k.wb : k.wa) + ((uint32_t)(k.r0 + k.u) * k.rowb + col0);
            const uint32_t nbytes = min((uint32_t)SLICE_BYTES, k.rowb - col0);
            na = min(nbytes, 2048u);
            nb = nbytes - na;
            b = a + 2048;
        }
    }
    slot_loads<K>((uint32_t)lane * 16, rsrc_words(a, na), rsrc_words(b, nb), k.op == OP_ATTN && P.n_steps > 1);
}

// Waits until at most N vector memory operations are outstanding (N = 0 or
// 4 (D - 1)) and copies slot K into compiler registers. With D slots issued
// in order and four loads per slot, 4 (D - 1) waits exactly for slot K.
template <int K, int N>
__device__ __forceinline__ void take_slot(v4u (&r)[4]) {
    static_assert(N == 0 || N == 4 * (D - 1), "wait counts");
    v2u x[8];
    slot_take<K>(x, N);
#pragma unroll
    for (int j = 0; j < 4; ++j) r[j] = v4u{x[2 * j].x, x[2 * j].y, x[2 * j + 1].x, x[2 * j + 1].y};
}

// ------------------------------------------------------------ instruction

struct Ins {
    int step;  // decode step of the launch
    int gpc;   // step * (queue length) + pc: the instruction's index in the LDS counts
    int pc, op, layer, r0, r1, flags, b, g, c, nch, p, merge, slot, nslot, mctr, mneed;
    int nblk;     // attention: K/V blocks of the tile
    bool alast;   // attention: the tile holds its request's newest position (and appends it)
    uint64_t wn;  // norm weight of the op's input
    // a matvec's tagged output: the layer's vector of every request (request
    // b's row r is word b * os + r of B * os)
    uint64_t *ob;
    int os;
    int64_t *tr;
};

template <int NB>
struct Acc {
    float a0[NB], a1[NB];  // dot products of the current unit (gate/up for UPGATE)
    float bv[NB];          // LM head: best value and index so far
    int bi[NB];
    float g;               // batched UPGATE: lane b holds request b's finished gate product
    bool nan;
};

// Batched kernels accumulate an UPGATE unit's gate and up products in one
// register per request: when the gate half of the unit ends, its reduced
// product is parked in lane b (Acc::g) and the register starts the up half.
// The sums and their order are unchanged; the slice loop carries NB fewer
// live values, which it would otherwise spill.
template <int NB>
constexpr bool ONE_ACC = NB > 1;

// Request b's input token: the caller's at the launch's first step, and at
// each later step of a resident launch the token the previous step's LM
// head published (polled like any tagged activation). -1 on abort.
__device__ __forceinline__ int token_of(const KParams &P, Ctx &c, int b, const Ins &in) {
    int t;
    if (in.step == 0) {
        t = sload(P.tokens_in, b);
    } else {
        float v = 0.0f;
        const uint32_t tag = c.tag;
        c.tag = tag - 1u;  // the previous step's
        const bool ok = tgather<1>(
            c, tres(P.ttok, (uint32_t)(P.n_steps * P.B)), 1,
            [&](int) { return (uint32_t)((in.step - 1) * P.B + b); }, [&](int, float x) { v = x; }, in.pc);
        c.tag = tag;
        if (!ok) return -1;
        t = __builtin_amdgcn_readfirstlane(__float_as_int(v));
    }
    if (t < 0 || t >= P.V) {
        if (c.lane() == 0) raise_err(c, ERR_RANGE, in.pc);
        t = 0;
    }
    return t;
}

// Copies the norm weights wn[0, H) (bf16) into the LDS area at nw_off with
// 1 KiB wave loads that write LDS directly (no registers held, no wait of
// their own): issued before the input polls, they land under the same waits.
// Wave w < 4 copies KiB w, w + 4, ...; lanes past the vector re-read its last
// 16 bytes into the area's padding.
__device__ __forceinline__ void prefetch_norm_w(const KParams &P, const Ctx &c, const uint16_t *wn) {
    if (c.w >= 4) return;
    const int bytes = P.H * 2;
    MK_LDS char *dst = (MK_LDS char *)c.misc + P.nw_off;
    for (int kib = c.w; kib * 1024 < bytes; kib += 4) {
        const int off = min(kib * 1024 + c.lane() * 16, bytes - 16);
        __builtin_amdgcn_global_load_lds((const __attribute__((address_space(1))) void *)((const char *)wn + off),
                                         (__attribute__((address_space(3))) void *)(dst + kib * 1024), 16, 0, 0);
    }
}

// The batched norm (several requests, x_v with v > 0): request b's words
// are gathered by its NC / NB waves, each holding the baseline partition's
// "virtual waves" v0 .. v0 + VPW - 1 (elements i = 64 v + lane + 256 k) in
// registers, so the sums of squares run in the baseline's order straight
// from the gathered words; the fp32 words also land in the staging area for
// the scaling pass. Words of the wave, in gather order j: virtual wave
// v0 + j % VPW, k = j / VPW.
template <int NB>
__device__ __forceinline__ bool norm_gather_batched(const KParams &P, Ctx &c, const Ins &in, int xv) {
    static_assert(NB == 2 || NB == 4 || NB == 8, "batched norm");
    constexpr int R = NC / NB, VPW = 4 / R;  // waves per request; virtual waves per wave
    const int H = P.H, lane = c.lane(), b = c.w / R, v0 = (c.w % R) * VPW;
    if (b >= P.B) return true;
    const int nw = VPW * (H / 256);  // words per lane (H is a multiple of 256)
    const __amdgpu_buffer_rsrc_t r = tres(P.tx + ((size_t)(xv - 1) * P.B + b) * H, (uint32_t)H);
    auto xs = [&](int i) -> MK_LDS float & {
        if constexpr (ACT16<NB>) return c.act[(NB * H) / 2 + b * H + i];
        else return c.act[b * P.act_stride + act_index(i)];
    };
    auto elem = [&](int j) { return 64 * (v0 + j % VPW + 4 * (j / VPW)) + lane; };
    float ss[VPW];
#pragma unroll
    for (int v = 0; v < VPW; ++v) ss[v] = 0.0f;
    for (int j0 = 0; j0 < nw; j0 += 16) {  // uniform bound; 16 is a multiple of VPW
        float x[16];
        if (!tgather<16>(
                c, r, min(16, nw - j0), [&](int k) { return (uint32_t)elem(j0 + k); },
                [&](int k, float v) { x[k] = v; }, in.pc))
            return false;
#pragma unroll
        for (int k = 0; k < 16; ++k)
            if (j0 + k < nw) {
                ss[k % VPW] = fmaf(x[k], x[k], ss[k % VPW]);
                xs(elem(j0 + k)) = x[k];
            }
    }
    MK_LDS float *norm = (MK_LDS float *)(c.misc + M_NORM);
#pragma unroll
    for (int v = 0; v < VPW; ++v) {
        const float t = wave_sum(ss[v]);
        if (lane == 0) norm[(v0 + v) * MAX_B + b] = t;
    }
    return true;
}

// ... and the scaling pass of the batched norm: request b's R waves split its
// elements in chunks of 8 (16-byte LDS accesses), scaled by its inverse RMS
// (the four partial sums added in the baseline's order) and the norm weight.
template <int NB>
__device__ __forceinline__ void norm_scale_batched(const KParams &P, Ctx &c) {
    constexpr int R = NC / NB;
    const int H = P.H, lane = c.lane(), b = c.w / R, r = c.w % R;
    if (b >= P.B) return;
    const MK_LDS float *norm = (const MK_LDS float *)(c.misc + M_NORM);
    float tot = 0.0f;
    for (int v = 0; v < 4; ++v) tot += norm[v * MAX_B + b];
    const float inv = 1.0f / sqrtf(tot / (float)H + P.eps);
    const MK_LDS uint16_t *nwl = (const MK_LDS uint16_t *)((MK_LDS char *)c.misc + P.nw_off);
    const int per = H / 8 / R;  // chunks of this wave
    for (int ci = r * per + lane; ci < (r + 1) * per; ci += 64) {
        const v4u wv = *(const MK_LDS v4u *)(nwl + ci * 8);
        const float wn[8] = {bf_lo(wv.x), bf_hi(wv.x), bf_lo(wv.y), bf_hi(wv.y),
                             bf_lo(wv.z), bf_hi(wv.z), bf_lo(wv.w), bf_hi(wv.w)};
        if constexpr (ACT16<NB>) {
            const MK_LDS float *xs = c.act + (NB * H) / 2 + b * H + ci * 8;
            const v4f a = *(const MK_LDS v4f *)xs, e = *(const MK_LDS v4f *)(xs + 4);
            const float xv[8] = {a.x, a.y, a.z, a.w, e.x, e.y, e.z, e.w};
            uint32_t h[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                h[q] = (uint32_t)f2h(xv[2 * q] * inv * wn[2 * q]) |
                       ((uint32_t)f2h(xv[2 * q + 1] * inv * wn[2 * q + 1]) << 16);
            *(MK_LDS v4u *)((MK_LDS uint16_t *)c.act + b * H + ci * 8) = v4u{h[0], h[1], h[2], h[3]};
        } else {
            // act_index: chunk ci's first four values, then its last four 256 floats on
            MK_LDS float *xs = c.act + b * P.act_stride + act_index(ci * 8);
            v4f a = *(MK_LDS v4f *)xs, e = *(MK_LDS v4f *)(xs + 256);
            a = v4f{a.x * inv * wn[0], a.y * inv * wn[1], a.z * inv * wn[2], a.w * inv * wn[3]};
            e = v4f{e.x * inv * wn[4], e.y * inv * wn[5], e.z * inv * wn[6], e.w * inv * wn[7]};
            *(MK_LDS v4f *)xs = a;
            *(MK_LDS v4f *)(xs + 256) = e;
        }
    }
}

// act[b] <- rmsnorm(x_v[b]) * wn in the matvec layout (x_0: the layer-0
// input). The elements i = 64 w + lane + 256 k of each request are summed
// as four "virtual waves" w = 0..3 in that order, then added w by w, which is
// the reduction of the one-kernel-per-op baseline's norm, so both paths
// agree bit for bit.
template <int NB>
__device__ __forceinline__ bool stage_norm(const KParams &P, Ctx &c, const Ins &in, const uint16_t *wn, int xv) {
    const int H = P.H, lane = c.lane(), w = c.w;
    MK_LDS float *norm = (MK_LDS float *)(c.misc + M_NORM);
    const int first = w * 64 + lane;
    const int n = first < H ? (H - first + 255) / 256 : 0;  // this lane's elements
    const int nmax = (H - w * 64 + 255) / 256;               // lane 0's: the most
    prefetch_norm_w(P, c, wn);
    if constexpr (NB > 1) {
        if (xv != 0) {
            if (!norm_gather_batched<NB>(P, c, in, xv)) return false;
            // the norm-weight copies (waves 0..3) have landed
            if (w < 4) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            if (!cbar(c, in.pc)) return false;
            norm_scale_batched<NB>(P, c);
            return cbar(c, in.pc);
        }
    }
    // the fp32 input of request b, element i: in the matvec layout, or with
    // binary16 staging contiguous past the binary16 area
    auto xs = [&](int b, int i) -> MK_LDS float & {
        if constexpr (ACT16<NB>) return c.act[(NB * H) / 2 + b * H + i];
        else return c.act[b * P.act_stride + act_index(i)];
    };
    if (w < 4) {
        for (int b = 0; b < P.B; ++b) {
            if (xv == 0) {
                const int tok = P.has_embed ? token_of(P, c, b, in) : 0;
                if (tok < 0) return false;
                for (int i = first; i < H; i += 256) xs(b, i) = x_input(P, b, i, true, tok);
            } else {
                const __amdgpu_buffer_rsrc_t r = tres(P.tx + ((size_t)(xv - 1) * P.B + b) * H, (uint32_t)H);
                // the loop bound is uniform: an early return from a loop whose
                // trip count differs per lane would make the caller's control
                // flow divergent
                for (int k0 = 0; k0 < nmax; k0 += 16)
                    if (!tgather<16>(
                            c, r, n - k0, [&](int k) { return (uint32_t)(first + 256 * (k0 + k)); },
                            [&](int k, float v) { xs(b, first + 256 * (k0 + k)) = v; }, in.pc))
                        return false;
            }
            float ss = 0.0f;
            for (int i = first; i < H; i += 256) {
                const float v = xs(b, i);
                ss = fmaf(v, v, ss);
            }
            ss = wave_sum(ss);
            if (lane == 0) norm[w * MAX_B + b] = ss;
        }
    }
    // the norm-weight copies have landed (the polls waited for every load
    // issued before them; the embedding path has no polls)
    if (w < 4) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (!cbar(c, in.pc)) return false;
    // batch 1 with H = 2048: every wave applies the norm as it loads its
    // register activations (norm_scale, at entry to the slices), so the
    // inputs stay unscaled here and neither a scaling pass nor a second
    // barrier is needed
    if (NB == 1 && H == 2048) return true;
    if (w < 4) {
        const MK_LDS uint16_t *nw = (const MK_LDS uint16_t *)((MK_LDS char *)c.misc + P.nw_off);
        for (int b = 0; b < P.B; ++b) {
            float tot = 0.0f;
            for (int v = 0; v < 4; ++v) tot += norm[v * MAX_B + b];
            const float inv = 1.0f / sqrtf(tot / (float)H + P.eps);
            if constexpr (ACT16<NB>) {
                MK_LDS uint16_t *a16 = (MK_LDS uint16_t *)c.act + b * H;
                for (int i = first; i < H; i += 256) a16[i] = f2h(xs(b, i) * inv * bf2f(nw[i]));
            } else {
                for (int i = first; i < H; i += 256) xs(b, i) = xs(b, i) * inv * bf2f(nw[i]);
            }
        }
    }
    return cbar(c, in.pc);
}

// xrow[b][j] <- x_v[b][r0 + j] for the instruction's rows (x_0: the input)
template <int NB>
__device__ __forceinline__ bool stage_rows(const KParams &P, Ctx &c, const Ins &in, int xv) {
    const int nr = in.r1 - in.r0;
    if (NB > 1 && xv != 0 && P.B * nr <= NC * 64) {  // every (request, row) word in one round
        const __amdgpu_buffer_rsrc_t r = tres(P.tx + (size_t)(xv - 1) * P.B * P.H, (uint32_t)(P.B * P.H));
        const int L = c.w * 64 + c.lane();
        const int b = nr > 0 ? L / nr : 0, j = L - b * nr;
        return tgather<1>(
            c, r, L < P.B * nr ? 1 : 0, [&](int) { return (uint32_t)(b * P.H + in.r0 + j); },
            [&](int, float v) { c.xrow[b * P.xrow_stride + j] = v; }, in.pc);
    }
    for (int b = 0; b < P.B; ++b) {
        MK_LDS float *xr = c.xrow + b * P.xrow_stride;
        if (xv == 0) {
            const int tok = P.has_embed ? token_of(P, c, b, in) : 0;
            if (tok < 0) return false;
            for (int j = c.w * 64 + c.lane(); j < nr; j += NC * 64) xr[j] = x_input(P, b, in.r0 + j, true, tok);
        } else {
            const __amdgpu_buffer_rsrc_t r = tres(P.tx + ((size_t)(xv - 1) * P.B + b) * P.H, (uint32_t)P.H);
            for (int j0 = c.w * 64; j0 < nr; j0 += NC * 64) {
                const int j = j0 + c.lane();
                if (!tgather<1>(
                        c, r, j < nr ? 1 : 0, [&](int) { return (uint32_t)(in.r0 + j); },
                        [&](int, float v) { xr[j] = v; }, in.pc))
                    return false;
            }
        }
    }
    return true;
}

// act[b] <- src[b][0, K) in the matvec layout (A16: rounded to binary16, in
// the 16-bit layout); src: tagged [B][K]
template <bool A16, int NB>
__device__ __forceinline__ bool stage_copy(const KParams &P, Ctx &c, const Ins &in, const uint64_t *src, int K) {
    // batch 8: the down projection's eight inputs of F words are the
    // largest gather; twice the words in flight per round halve its rounds
    if (NB > 1)
        return tgather_batch<A16 ? 32 : 16>(
            c, src, P.B, K,
            [&](int b, int i, float v) {
                if (A16) ((MK_LDS uint16_t *)c.act + b * K)[i] = f2h(v);
                else c.act[b * P.act_stride + act_index(i)] = v;
            },
            in.pc);
    const int per = K / NC;
    for (int b = 0; b < P.B; ++b) {
        MK_LDS float *a = c.act + b * P.act_stride;
        MK_LDS uint16_t *a16 = (MK_LDS uint16_t *)c.act + b * K;
        const __amdgpu_buffer_rsrc_t r = tres(src + (size_t)b * K, (uint32_t)K);
        if (!tgather_range(
                c, r, c.w * per, (c.w + 1) * per,
                [&](int i, float v) {
                    if (A16) a16[i] = f2h(v);
                    else a[act_index(i)] = v;
                },
                in.pc))
            return false;
    }
    return true;
}

// AMERGE: the softmax states (o, m, l) that the attention tiles of request
// b and kv head g published - the request's tiles of this step's split, in
// tile order - are gathered into LDS (the activation area, which no other
// part of a merge uses) by all waves, MAX_ATTN_CHUNKS tiles at a time, and
// merged in tile order, one wave per query head of the group (lane = dim);
// then o = O / L is published for the O projection, which reads only the
// merged outputs.

// nc gathered states (in LDS) into head h's running state, in tile order:
// eight states' reads at a time, then their merge steps (the registers of
// all sixteen would spill)
template <int G>
__device__ __forceinline__ void merge_states(const Ctx &c, int nc, int h, int lane, float &O, float &M, float &L) {
    for (int k0 = 0; k0 < nc; k0 += 8) {
        float o[8], m[8], l[8];
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (k0 + k < nc) {
                const MK_LDS float *src = c.act + ((k0 + k) * G + h) * ATTN_PART;
                o[k] = src[lane];
                m[k] = src[64];
                l[k] = src[65];
            }
#pragma unroll
        for (int k = 0; k < 8; ++k)
            if (k0 + k < nc) merge_step(O, M, L, o[k], m[k], l[k]);
    }
}

template <int NB, int G>
__device__ __forceinline__ bool stage_amerge(const KParams &P, Ctx &c, const Ins &in) {
    const int T = in.nch, lane = c.lane(), QD = P.nq * P.d;
    const __amdgpu_buffer_rsrc_t ro = tres(P.to + ((size_t)in.layer * P.B + in.b) * QD, (uint32_t)QD);
    if constexpr (NB == 1) {
        // one request: its T (<= MAX_ATTN_CHUNKS) tiles in one gather (the
        // round loop below measured slower here)
        const int n = T * G * ATTN_PART, per = (n + NC - 1) / NC;
        const __amdgpu_buffer_rsrc_t rp = tres(P.tpart + ((size_t)in.layer * P.nkv + in.g) * n, (uint32_t)n);
        if (!tgather_range(
                c, rp, c.w * per, min(n, (c.w + 1) * per), [&](int i, float v) { c.act[i] = v; }, in.pc))
            return false;
        if (!cbar(c, in.pc)) return false;
        if (c.w < G && T <= MAX_ATTN_CHUNKS) {
            float O, M, L;
            merge_init(O, M, L);
            merge_states<G>(c, T, c.w, lane, O, M, L);
            tput(ro, (uint32_t)((in.g * G + c.w) * 64 + lane), O / L, c.tag);
        }
        return true;
    }
    const int first = (int)split_word(c, in.step, in.b), nt = (int)split_word(c, in.step, in.b + 1) - first;
    const size_t base = (((size_t)in.layer * P.nkv + in.g) * T + first) * G * ATTN_PART;
    float O, M, L;
    merge_init(O, M, L);
    for (int c0 = 0; uni(c0 < nt); c0 += MAX_ATTN_CHUNKS) {
        const int nc = min(MAX_ATTN_CHUNKS, nt - c0);
        const int n = nc * G * ATTN_PART, per = (n + NC - 1) / NC;
        const __amdgpu_buffer_rsrc_t rp = tres(P.tpart + base + (size_t)c0 * G * ATTN_PART, (uint32_t)n);
        if (!tgather_range(
                c, rp, c.w * per, min(n, (c.w + 1) * per), [&](int i, float v) { c.act[i] = v; }, in.pc))
            return false;
        if (!cbar(c, in.pc)) return false;
        if (c.w < G) merge_states<G>(c, nc, c.w, lane, O, M, L);
        // the head waves have read these states before the next ones land
        if (c0 + MAX_ATTN_CHUNKS < nt && !cbar(c, in.pc)) return false;
    }
    if (c.w < G) tput(ro, (uint32_t)((in.g * G + c.w) * 64 + lane), O / L, c.tag);
    return true;
}

// Attention staging: the group's queries rotated (fp32, act[0, G*64)), and
// the new K/V entry rotated and rounded to bf16 (act + G*64 as uint16 [2][64]);
// the last chunk also appends that entry to the cache.
template <int G>
__device__ __forceinline__ bool stage_attn(const KParams &P, Ctx &c, const Ins &in) {
    const int lane = c.lane();
    const int QD = P.nq * P.d, QKVN = QD + 2 * P.nkv * P.d;
    const int b = in.b, g = in.g, p = in.p;
    const bool last = in.alast;
    MK_LDS uint16_t *kvn = (MK_LDS uint16_t *)(c.act + G * 64);
    const __amdgpu_buffer_rsrc_t r = tres(P.tqkv + ((size_t)in.layer * P.B + b) * QKVN, (uint32_t)QKVN);
    const float2 cs = P.rope[(int64_t)p * 32 + (lane & 31)];
    for (int t = c.w; t < G + 2; t += NC) {
        const int row0 = t < G ? (g * G + t) * 64 : (t == G ? QD + g * 64 : QD + P.nkv * 64 + g * 64);
        float xi = 0.0f;
        if (!tgather<1>(
                c, r, 1, [&](int) { return (uint32_t)(row0 + lane); }, [&](int, float v) { xi = v; }, in.pc))
            return false;
        float out = xi;
        if (t <= G) {  // queries and the key are rotated; the value is not
            const float xp = shfl_xor_f(xi, 32);
            out = rope_rotate(xi, xp, cs, lane < 32);
        }
        if (t < G) {
            c.act[t * 64 + lane] = out;
        } else {
            const uint16_t hb = f2bf(out);
            kvn[(t - G) * 64 + lane] = hb;
            if (last) {
                int page = sload(P.page_table, (int64_t)b * P.max_pages + (p >> 4));
                if (page < 0 || page >= P.n_pages) {
                    if (lane == 0) raise_err(c, ERR_RANGE, in.pc);
                    page = 0;
                }
                uint16_t *pool = t == G ? P.k_pool : P.v_pool;
                const uint16_t *entry = pool + (((size_t)in.layer * P.n_pages + page) * P.nkv + g) * 1024 + (p & 15) * 64;
                // one address for the wave, visibly (a buffer resource must be uniform)
                const uint64_t ea = (uint64_t)(uintptr_t)entry;
                uint16_t *dst = (uint16_t *)(uintptr_t)rfl64((int32_t)(uint32_t)ea, (int32_t)(uint32_t)(ea >> 32));
                // device-coherent: the later steps of a resident launch read
                // the entry back on other XCDs, with no kernel boundary
                // between (the wave waits for it before it leaves the tile)
                __builtin_amdgcn_raw_buffer_store_b16(hb, coherent_rsrc(dst, 128), (uint32_t)lane * 2, 0, CP_SC1);
                c.kv_pending = true;
            }
        }
    }
    return cbar(c, in.pc);
}

template <int NB, int G>
__device__ __forceinline__ bool enter(const KParams &P, Ctx &c, const Cur &k, Ins &in, Acc<NB> &acc, RegAct &ra) {
    const int pc = k.pc;
    in.pc = pc;
    in.step = k.step;
    in.gpc = k.step * c.nq + pc;
    c.tag = P.tag + (uint32_t)k.step;
    const iv4 a = iw4(c, pc, W_OP), bw = iw4(c, pc, W_B), fw = iw4(c, pc, W_FLAGS), mw = iw4(c, pc, 12),
              nw = iw4(c, pc, W_WN);
    in.op = rfl(a[0]);
    in.layer = rfl(a[1]);
    in.r0 = rfl(a[2]);
    in.r1 = rfl(a[3]);
    in.b = rfl(bw[0]);
    in.g = rfl(bw[1]);
    in.c = rfl(bw[2]);
    in.nch = rfl(bw[3]);
    in.flags = rfl(fw[0]);
    in.merge = rfl(fw[1]);
    in.slot = rfl(fw[2]);
    in.nslot = rfl(fw[3]);
    in.mctr = rfl(mw[W_MCTR - 12]);
    in.mneed = rfl(mw[W_MNEED - 12]);
    in.wn = rfl64(nw[0], nw[1]);
    switch (in.op) {
        case OP_QKV:
            in.os = (P.nq + 2 * P.nkv) * P.d;
            in.ob = P.tqkv + (size_t)in.layer * P.B * in.os;
            break;
        case OP_OPROJ:
            in.os = P.H;
            in.ob = P.tx + (size_t)(2 * in.layer) * P.B * P.H;
            break;
        case OP_UPGATE:
            in.os = P.F;
            in.ob = P.tact + (size_t)in.layer * P.B * P.F;
            break;
        case OP_DOWN:
            in.os = P.H;
            in.ob = P.tx + (size_t)(2 * in.layer + 1) * P.B * P.H;
            break;
        default:
            in.os = 0;
            in.ob = nullptr;
            break;
    }
    in.tr = P.trace ? P.trace + ((int64_t)c.cu * P.Q + pc) * TRACE_WORDS : nullptr;
    const bool tracer = in.tr && c.w == 0 && c.lane() == 0;
    if (tracer) in.tr[TR_START] = wall_clock64();
    // the previous instruction is finished, merges included: its LDS areas are free
    if (!lds_wait_ge(c, c.misc + M_DONE, (uint32_t)in.gpc, pc)) return false;
    bool ok = true;
    switch (in.op) {
        case OP_QKV:
            ok = stage_norm<NB>(P, c, in, (const uint16_t *)(uintptr_t)in.wn, (in.flags & F_X_FROM_INPUT) ? 0 : 2 * in.layer);
            break;
        case OP_UPGATE: ok = stage_norm<NB>(P, c, in, (const uint16_t *)(uintptr_t)in.wn, 2 * in.layer + 1); break;
        case OP_LMHEAD: ok = stage_norm<NB>(P, c, in, (const uint16_t *)(uintptr_t)in.wn, 2 * P.L); break;
        case OP_OPROJ:
            ok = stage_rows<NB>(P, c, in, (in.flags & F_X_FROM_INPUT) ? 0 : 2 * in.layer) &&
                 stage_copy<ACT16<NB>, NB>(P, c, in, P.to + (size_t)in.layer * P.B * P.nq * P.d, P.nq * P.d) && cbar(c, pc);
            break;
        case OP_DOWN:
            ok = stage_rows<NB>(P, c, in, 2 * in.layer + 1) &&
                 stage_copy<ACT16<NB>, NB>(P, c, in, P.tact + (size_t)in.layer * P.B * P.F, P.F) && cbar(c, pc);
            break;
        case OP_ATTN: {
            // the cursor's request and blocks of this tile at this step
            in.b = k.b;
            in.nblk = k.nu;
            // the tile holding the request's newest position appends it
            if constexpr (NB == 1)
                in.alast = in.c == in.nch - 1;
            else
                in.alast = (split_word(c, in.step, SPLIT_TILE + 2 * in.c) & 256u) != 0;
            const int p = (int)lds_ld_const(c.misc + M_KVLEN + k.b) + in.step;
            if (p < 0 || p >= P.T * P.max_pages) {
                if (c.lane() == 0) raise_err(c, ERR_RANGE, pc);
                return false;
            }
            in.p = p;
            ok = stage_attn<G>(P, c, in);
            break;
        }
        case OP_AMERGE: ok = stage_amerge<NB, G>(P, c, in); break;
        default:
            if (c.lane() == 0) raise_err(c, ERR_OPCODE, pc);
            return false;
    }
    if (!ok) return false;
    if (tracer) in.tr[TR_READY] = wall_clock64();
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        acc.a0[b] = 0.0f;
        acc.a1[b] = 0.0f;
        acc.bv[b] = -INFINITY;
        acc.bi[b] = 0x7fffffff;
    }
    if constexpr (NB > 1) {
        // batched kernels keep the LM head's running best of request b in the
        // wave's LDS slot (lane b reads and writes it), not in registers the
        // slice loop would have to spill
        if (in.op == OP_LMHEAD && c.lane() < P.B) {
            MK_LDS float *am = (MK_LDS float *)(c.misc + M_AMAX);
            am[(c.w * MAX_B + c.lane()) * 2] = -INFINITY;
            ((MK_LDS int32_t *)am)[(c.w * MAX_B + c.lane()) * 2 + 1] = 0x7fffffff;
        }
    }
    acc.nan = false;
    if (NB == 1 && in.op != OP_ATTN && k.K == 2048) {
        // the lane's activations: chunk 64 j + lane, elements 8 (64 j + lane) + e
        const bool normed = in.op == OP_QKV || in.op == OP_UPGATE || in.op == OP_LMHEAD;
        float inv = 1.0f;
        if (normed) {  // the same sum and order as a staged norm's scaling pass
            const MK_LDS float *norm = (const MK_LDS float *)(c.misc + M_NORM);
            float tot = 0.0f;
            for (int v = 0; v < 4; ++v) tot += norm[v * MAX_B];
            inv = 1.0f / sqrtf(tot / (float)P.H + P.eps);
        }
        const MK_LDS uint16_t *nw = (const MK_LDS uint16_t *)((MK_LDS char *)c.misc + P.nw_off);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const v4f a = *(const MK_LDS v4f *)(c.act + j * 512 + c.lane() * 4);
            const v4f b = *(const MK_LDS v4f *)(c.act + j * 512 + 256 + c.lane() * 4);
            ra.o[j][0] = a.x; ra.o[j][1] = a.y; ra.o[j][2] = a.z; ra.o[j][3] = a.w;
            ra.o[j][4] = b.x; ra.o[j][5] = b.y; ra.o[j][6] = b.z; ra.o[j][7] = b.w;
            if (normed) {
                const v4u wq = *(const MK_LDS v4u *)(nw + (j * 64 + c.lane()) * 8);
                const float wf[8] = {bf_lo(wq.x), bf_hi(wq.x), bf_lo(wq.y), bf_hi(wq.y),
                                     bf_lo(wq.z), bf_hi(wq.z), bf_lo(wq.w), bf_hi(wq.w)};
#pragma unroll
                for (int e = 0; e < 8; ++e) ra.o[j][e] = ra.o[j][e] * inv * wf[e];
            }
        }
    }
    return true;
}

// Output of row `row` for request b (lane b), v0 the row's dot product, v1
// the up projection's for UPGATE.
__device__ __forceinline__ void emit_row(const KParams &P, Ctx &c, const Ins &in, int row, int b, float v0, float v1) {
    const bool last_step = in.step == P.n_steps - 1;  // a resident launch returns its last step's logits and hidden
    float v;
    switch (in.op) {
        case OP_QKV: v = v0; break;
        case OP_OPROJ: v = c.xrow[b * P.xrow_stride + (row - in.r0)] + v0; break;
        case OP_UPGATE: v = silu(v0) * v1; break;
        case OP_DOWN:
            v = c.xrow[b * P.xrow_stride + (row - in.r0)] + v0;
            if ((in.flags & F_WRITE_HIDDEN) && P.hidden_out && last_step) P.hidden_out[(int64_t)b * P.H + row] = v;
            break;
        default:
            if (P.logits_out && last_step) P.logits_out[(int64_t)b * P.V + row] = v0;
            return;
    }
    tput(tres(in.ob, (uint32_t)(P.B * in.os)), (uint32_t)(b * in.os + row), v, c.tag);
}

// The eight requests' dot products of a unit summed over the wave's 64
// lanes together: three exchanges with the lanes 32, 16 and 8 apart, each
// halving the values a lane carries, then a sum over 8 adjacent lanes;
// request b's total ends in lanes 8 b .. 8 b + 7. (Eight separate wave sums
// and eight one-lane emits per unit cost several times the unit's products
// at this batch.)
__device__ __forceinline__ float reduce8(const float (&v)[8]) {
    const int lane = lane_id();
    const bool h5 = (lane & 32) != 0, h4 = (lane & 16) != 0, h3 = (lane & 8) != 0;
    float a[4], e[2];
#pragma unroll
    for (int k = 0; k < 4; ++k) a[k] = (h5 ? v[k + 4] : v[k]) + shfl_xor_f(h5 ? v[k] : v[k + 4], 32);
#pragma unroll
    for (int k = 0; k < 2; ++k) e[k] = (h4 ? a[k + 2] : a[k]) + shfl_xor_f(h4 ? a[k] : a[k + 2], 16);
    return sum8lanes((h3 ? e[1] : e[0]) + shfl_xor_f(h3 ? e[0] : e[1], 8));
}

// Row `row`'s outputs of the eight requests, written by lanes 8 b (request
// b = lane / 8, the value pair its lane group holds), through the
// instruction's output resource, which spans all requests (uniform).
__device__ __forceinline__ void emit_rows8(const KParams &P, Ctx &c, const Ins &in, int row, float v0, float v1) {
    const int lane = lane_id(), b = lane >> 3;
    if ((lane & 7) != 0 || b >= P.B) return;
    const bool last_step = in.step == P.n_steps - 1;
    float v;
    switch (in.op) {
        case OP_QKV: v = v0; break;
        case OP_OPROJ: v = c.xrow[b * P.xrow_stride + (row - in.r0)] + v0; break;
        case OP_UPGATE: v = silu(v0) * v1; break;
        case OP_DOWN:
            v = c.xrow[b * P.xrow_stride + (row - in.r0)] + v0;
            if ((in.flags & F_WRITE_HIDDEN) && P.hidden_out && last_step) P.hidden_out[(int64_t)b * P.H + row] = v;
            break;
        default: {
            if (P.logits_out && last_step) P.logits_out[(int64_t)b * P.V + row] = v0;
            // the wave's running best of request b (its rows rise, so ties
            // keep the lowest index)
            MK_LDS float *am = (MK_LDS float *)(c.misc + M_AMAX);
            const int at = (c.w * MAX_B + b) * 2;
            if (v0 > am[at]) {
                am[at] = v0;
                ((MK_LDS int32_t *)am)[at + 1] = row;
            }
            return;
        }
    }
    tput(tres(in.ob, (uint32_t)(P.B * in.os)), (uint32_t)(b * in.os + row), v, c.tag);
}

// End of a slice at a padded batch of 8: at the end of an UPGATE unit's gate
// half its eight sums are parked in acc.g (request b's in lanes 8 b ..), at
// the end of a unit its outputs are written.
template <int NB>
__device__ __forceinline__ void unit_end8(const KParams &P, Ctx &c, const Cur &k, const Ins &in, Acc<NB> &acc) {
    static_assert(NB == 8 && ONE_ACC<NB>, "batch-8 epilogue");
    const bool gate_done = in.op == OP_UPGATE && k.s == k.spm - 1;
    if (!gate_done && k.s != k.sp - 1) return;
    const float s = reduce8(acc.a0);
#pragma unroll
    for (int b = 0; b < NB; ++b) acc.a0[b] = 0.0f;
    if (gate_done) {
        acc.g = s;
        return;
    }
    const bool up = in.op == OP_UPGATE;
    const float v0 = up ? acc.g : s;
    if (in.op == OP_LMHEAD && __builtin_amdgcn_ballot_w64((lane_id() >> 3) < P.B && v0 != v0) != 0) acc.nan = true;
    emit_rows8(P, c, in, k.r0 + k.u, v0, up ? s : 0.0f);
}

// Slice (part, m) of unit u: the lane's 16-byte chunks ci = 256 part + 64 j +
// lane, j < 4, times the activations of those chunks, added in j order to
// the unit's dot product (m: gate or up matrix of UPGATE). Three forms with
// the same arithmetic: at batch 1 with K = 2048 the activations sit in
// registers (xr.o[j]), loaded once per instruction; a full slice converts its
// weights once and reads each request's activations from LDS right before
// that request's products (at a padded batch of 8 the down projection's
// input is staged as binary16, the only way 8 requests' 8192-wide inputs fit
// in LDS); a slice past the end of a short row guards each chunk.
template <int NB>
__device__ __forceinline__ void consume_mv(const KParams &P, Ctx &c, const Cur &k, const Ins &in, const v4u (&r)[4],
                                           Acc<NB> &acc, const RegAct &xr) {
    const int lane = c.lane();
    const int m = k.s >= k.spm ? 1 : 0, part = k.s - m * k.spm;
    if (NB == 1 && k.K == 2048) {
        float a = m ? acc.a1[0] : acc.a0[0];
#pragma unroll
        for (int j = 0; j < 4; ++j)
            a += dot8(r[j], v4f{xr.o[j][0], xr.o[j][1], xr.o[j][2], xr.o[j][3]},
                      v4f{xr.o[j][4], xr.o[j][5], xr.o[j][6], xr.o[j][7]});
        acc.a0[0] = m ? acc.a0[0] : a;
        acc.a1[0] = m ? a : acc.a1[0];
    } else if (ACT16<NB> && k.K >= (part + 1) * 2048) {
        // binary16 staging: the slice's weights as binary16 pairs once (bf16
        // to binary16 with round-to-nearest-even; the weights' magnitudes lie
        // far inside its range), then per request eight 16-byte activation
        // reads and packed fp16 dot products accumulating in fp32
        h2v wh[4][4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wh[j][0] = bf_pair_h2(r[j].x);
            wh[j][1] = bf_pair_h2(r[j].y);
            wh[j][2] = bf_pair_h2(r[j].z);
            wh[j][3] = bf_pair_h2(r[j].w);
        }
        // request b + 1's four activation reads are issued before request
        // b's products, so that LDS latency overlaps the arithmetic instead
        // of being waited out read by read
        const MK_LDS uint16_t *a0p = (const MK_LDS uint16_t *)c.act + part * 2048 + lane * 8;
        v4u xn[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) xn[j] = *(const MK_LDS v4u *)(a0p + j * 512);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float a = ONE_ACC<NB> ? acc.a0[b] : (m ? acc.a1[b] : acc.a0[b]);
            v4u xc[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) xc[j] = xn[j];
            if (b + 1 < NB) {
#pragma unroll
                for (int j = 0; j < 4; ++j) xn[j] = *(const MK_LDS v4u *)(a0p + (b + 1) * k.K + j * 512);
            }
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const v4u x = xc[j];
                a = __builtin_amdgcn_fdot2(wh[j][0], as_h2(x.x), a, false);
                a = __builtin_amdgcn_fdot2(wh[j][1], as_h2(x.y), a, false);
                a = __builtin_amdgcn_fdot2(wh[j][2], as_h2(x.z), a, false);
                a = __builtin_amdgcn_fdot2(wh[j][3], as_h2(x.w), a, false);
            }
            if constexpr (ONE_ACC<NB>) {
                acc.a0[b] = a;
            } else {
                acc.a0[b] = m ? acc.a0[b] : a;
                acc.a1[b] = m ? a : acc.a1[b];
            }
        }
    } else if (!ACT16<NB> && k.K >= (part + 1) * 2048) {
        // the slice's weights as fp32 once; then each request's activations
        // are read right before its products, so that few are live at once
        float wf[4][8];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            wf[j][0] = bf_lo(r[j].x);
            wf[j][1] = bf_hi(r[j].x);
            wf[j][2] = bf_lo(r[j].y);
            wf[j][3] = bf_hi(r[j].y);
            wf[j][4] = bf_lo(r[j].z);
            wf[j][5] = bf_hi(r[j].z);
            wf[j][6] = bf_lo(r[j].w);
            wf[j][7] = bf_hi(r[j].w);
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float a = ONE_ACC<NB> ? acc.a0[b] : (m ? acc.a1[b] : acc.a0[b]);
            const MK_LDS float *ab = c.act + b * P.act_stride + part * 2048 + lane * 4;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                a += dot8f(wf[j], *(const MK_LDS v4f *)(ab + j * 512), *(const MK_LDS v4f *)(ab + j * 512 + 256));
            if constexpr (ONE_ACC<NB>) {
                acc.a0[b] = a;
            } else {
                acc.a0[b] = m ? acc.a0[b] : a;
                acc.a1[b] = m ? a : acc.a1[b];
            }
        }
    } else {
        const int nchunk = k.K >> 3;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int ci = part * 256 + j * 64 + lane;
            if (ci < nchunk) {
                const int base = ((ci >> 6) << 9) + ((ci & 63) << 2);
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    float d;
                    if constexpr (ACT16<NB>) {
                        const v4u x = *(const MK_LDS v4u *)((const MK_LDS uint16_t *)c.act + b * k.K + ci * 8);
                        d = dot8(r[j], v4f{h_lo(x.x), h_hi(x.x), h_lo(x.y), h_hi(x.y)},
                                 v4f{h_lo(x.z), h_hi(x.z), h_lo(x.w), h_hi(x.w)});
                    } else {
                        const MK_LDS float *a = c.act + b * P.act_stride + base;
                        d = dot8(r[j], *(const MK_LDS v4f *)a, *(const MK_LDS v4f *)(a + 256));
                    }
                    if (ONE_ACC<NB> || m == 0) acc.a0[b] += d;
                    else acc.a1[b] += d;
                }
            }
        }
    }
    if constexpr (NB == 8) {
        unit_end8(P, c, k, in, acc);
        return;
    }
    if constexpr (ONE_ACC<NB>) {
        if (in.op == OP_UPGATE && k.s == k.spm - 1) {  // the unit's gate half is complete
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const float gsum = wave_sum(acc.a0[b]);
                if (lane == b) acc.g = gsum;
                acc.a0[b] = 0.0f;
            }
            return;
        }
    }
    if (k.s != k.sp - 1) return;
    // unit complete: reduce, write, reset
    const int row = k.r0 + k.u;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        float v0, v1;
        if (ONE_ACC<NB> && in.op == OP_UPGATE) {
            v0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc.g), b));
            v1 = wave_sum(acc.a0[b]);
        } else {
            v0 = wave_sum(acc.a0[b]);
            v1 = in.op == OP_UPGATE ? wave_sum(acc.a1[b]) : 0.0f;
        }
        acc.a0[b] = 0.0f;
        acc.a1[b] = 0.0f;
        if (b < P.B) {
            if (lane == b) emit_row(P, c, in, row, b, v0, v1);
            if (in.op == OP_LMHEAD) {
                if (v0 != v0) acc.nan = true;
                // a wave's rows rise, so ties keep the lowest index
                if constexpr (NB == 1) {
                    if (v0 > acc.bv[b]) {
                        acc.bv[b] = v0;
                        acc.bi[b] = row;
                    }
                } else if (lane == b) {
                    MK_LDS float *am = (MK_LDS float *)(c.misc + M_AMAX);
                    const int at = (c.w * MAX_B + b) * 2;
                    if (v0 > am[at]) {
                        am[at] = v0;
                        ((MK_LDS int32_t *)am)[at + 1] = row;
                    }
                }
            }
        }
    }
}

// The LDS area of an attention tile's wave states ([N_COMPUTE_WAVES][G]
// [ATTN_PART]): after the staged queries ([G][64] fp32) and the new K/V
// entry (bf16 [2][64], 64 floats' room).
template <int G>
__device__ __forceinline__ MK_LDS float *attn_states(const Ctx &c) {
    return c.act + G * 64 + 64;
}

// One K/V block of an attention tile into the wave's softmax state: the new
// entry replaces whatever the cache slot held.
template <int G>
__device__ __forceinline__ void attn_fold_block(Ctx &c, const Cur &k, const Ins &in, const v4u (&r)[4], AttnAcc<G> &a) {
    const int lane = c.lane();
    const int blk = k.blo + k.u;
    v4u k0 = r[0], k1 = r[1], v0 = r[2], v1 = r[3];
    const int t0 = lane >> 3;
    if (blk == (in.p >> 4)) {
        const int j = in.p & 15, dd = (lane & 7) * 8;
        const MK_LDS uint16_t *kvn = (const MK_LDS uint16_t *)(c.act + G * 64);
        const v4u nk = *(const MK_LDS v4u *)(kvn + dd), nv = *(const MK_LDS v4u *)(kvn + 64 + dd);
        if (t0 == j) {
            k0 = nk;
            v0 = nv;
        }
        if (t0 + 8 == j) {
            k1 = nk;
            v1 = nv;
        }
    }
    const int pos0 = blk * 16 + t0;
    attn_acc_block<G>(a, c.act, lane, k0, k1, v0, v1, pos0 <= in.p, pos0 + 8 <= in.p);
}

// Elects the last of the instruction's merge-event finishers (one per step).
__device__ __forceinline__ bool elect_last(const KParams &P, Ctx &c, const Ins &in) {
    const int32_t need = (int32_t)((int64_t)(P.step_epoch + in.step) * in.mneed);
    int32_t old = 0;
    if (c.lane() == 0)
        old = __hip_atomic_fetch_add(P.counters + (int64_t)in.mctr * CTR_STRIDE, 1, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT);
    old = __builtin_amdgcn_readfirstlane(old);  // lane 0's: every lane is active here
    return old + 1 == need;
}

// The start counter: every workgroup bumps it once it has read kv_lens, so
// a step that writes kv_lens_out (which may alias kv_lens) first checks that
// every workgroup of the grid has taken its copy. `first` is a value read
// earlier; by the end of a step the count is normally complete already.
__device__ __forceinline__ int32_t started_count(const KParams &P) {
    return __hip_atomic_load(P.counters + (int64_t)P.start_ctr * CTR_STRIDE, __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ bool wait_all_started(const KParams &P, Ctx &c, int32_t first, int pc) {
    const int32_t need = (int32_t)((int64_t)P.epoch * P.n_cus);
    int32_t v = __builtin_amdgcn_readfirstlane(first);
    int64_t spins = 0;
    while (v < need) {
        if (++spins > c.watchdog) {
            raise_err(c, ERR_TIMEOUT, pc);
            return false;
        }
        __builtin_amdgcn_s_sleep(1);
        v = __builtin_amdgcn_readfirstlane(started_count(P));
    }
    return true;
}

// Run by the last wave to finish an instruction's slices.
template <int G>
__device__ __forceinline__ bool finish(const KParams &P, Ctx &c, const Ins &in) {
    const int lane = c.lane();
    const uint32_t tag = c.tag;
    const bool last_step = in.step == P.n_steps - 1;
    if (in.op == OP_LMHEAD) {
        const MK_LDS float *am = (const MK_LDS float *)(c.misc + M_AMAX);
        const __amdgpu_buffer_rsrc_t rl = tres(P.tlm, (uint32_t)(in.nslot * P.B * 2));
        if (lane < P.B) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int w = 0; w < NC; ++w) {
                const float v = am[(w * MAX_B + lane) * 2];
                const int i = ((const MK_LDS int32_t *)am)[(w * MAX_B + lane) * 2 + 1];
                if (amax_better(v, i, bv, bi)) {
                    bv = v;
                    bi = i;
                }
            }
            tput(rl, (uint32_t)((in.slot * P.B + lane) * 2), bv, tag);
            tput(rl, (uint32_t)((in.slot * P.B + lane) * 2 + 1), __int_as_float(bi), tag);
        }
        if (!elect_last(P, c, in)) return true;
        if (in.tr && lane == 0) in.tr[TR_ELECT] = wall_clock64();
        const int32_t started = P.kv_lens_out && last_step ? started_count(P) : 0;  // read now, checked before the write
        // the argmax is a maximum under a total order: any combination order gives the same token
        if (!tgather_range(
                c, rl, 0, in.nslot * P.B * 2, [&](int i, float v) { c.act[i] = v; }, in.pc))
            return false;
        if (in.tr && lane == 0) in.tr[TR_GATHER] = wall_clock64();
        // per request: each lane takes slots lane, lane + 64, ..., then an
        // xor butterfly over the wave leaves every lane with the maximum
        for (int b = 0; b < P.B; ++b) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
            for (int t = lane; t < in.nslot; t += 64) {
                const float v = c.act[(t * P.B + b) * 2];
                const int i = __float_as_int(c.act[(t * P.B + b) * 2 + 1]);
                if (amax_better(v, i, bv, bi)) {
                    bv = v;
                    bi = i;
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const float ov = shfl_xor_f(bv, o);
                const int oi = shfl_xor_i(bi, o);
                if (amax_better(ov, oi, bv, bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (lane == 0) {
                P.tokens_out[(int64_t)in.step * P.B + b] = bi;
                // the next step of a resident launch embeds this token
                if (!last_step) tput(tres(P.ttok, (uint32_t)(P.n_steps * P.B)), (uint32_t)(in.step * P.B + b),
                                     __int_as_float(bi), tag);
            }
        }
        if (P.kv_lens_out && last_step) {
            if (!wait_all_started(P, c, started, in.pc)) return false;
            if (lane < P.B) P.kv_lens_out[lane] = (int32_t)c.misc[M_KVLEN + lane] + P.n_steps;
        }
        return true;
    }
    if ((in.flags & F_STEP_FINAL) && in.merge >= 0) {  // last layer's down projection without an LM head
        if (elect_last(P, c, in) && P.kv_lens_out) {
            if (!wait_all_started(P, c, started_count(P), in.pc)) return false;
            if (lane < P.B) P.kv_lens_out[lane] = (int32_t)c.misc[M_KVLEN + lane] + P.n_steps;
        }
    }
    return true;
}

template <int NB, int G>
__device__ __forceinline__ bool leave(const KParams &P, Ctx &c, const Ins &in, Acc<NB> &acc) {
    const int lane = c.lane();
    if (in.op == OP_LMHEAD) {
        if constexpr (NB == 1) {  // batched kernels kept the running best there already
            MK_LDS float *am = (MK_LDS float *)(c.misc + M_AMAX);
            if (lane == 0 && P.B > 0) {
                am[(c.w * MAX_B) * 2] = acc.bv[0];
                ((MK_LDS int32_t *)am)[(c.w * MAX_B) * 2 + 1] = acc.bi[0];
            }
        }
        if (acc.nan && lane == 0) raise_err(c, ERR_NAN, in.pc);
    }
    uint32_t old = 0;
    if (lane == 0) old = lds_add(c.misc + M_FIN, 1u);
    old = __builtin_amdgcn_readfirstlane(old);  // lane 0's: every lane is active here
    if (in.tr && lane == 0 && old == (uint32_t)NC * in.gpc) in.tr[TR_FIRST] = wall_clock64();
    if (in.tr && lane == 0 && old == (uint32_t)NC * (in.gpc + 1) - 1) in.tr[TR_LAST] = wall_clock64();
    if (in.op == OP_ATTN) return true;  // the attention loop published the tile and ended it
    if (old != (uint32_t)NC * (in.gpc + 1) - 1) return true;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
    if (!finish<G>(P, c, in)) return false;
    if (in.tr && lane == 0) in.tr[TR_END] = wall_clock64();
    if (lane == 0) lds_add(c.misc + M_DONE, 1u);
    return true;
}

// Slot operations with a run-time slot index (a uniform scalar): one small
// case per slot, so the code that consumes a slice exists once.
__device__ __forceinline__ void take_any(int k, v4u (&r)[4]) {
    switch (k) {
        case 0: take_slot<0, 4 * (D - 1)>(r); break;
        case 1: take_slot<1, 4 * (D - 1)>(r); break;
        case 2: take_slot<2, 4 * (D - 1)>(r); break;
        default: take_slot<3, 4 * (D - 1)>(r); break;
    }
}
__device__ __forceinline__ void issue_any(int k, const KParams &P, const Cur &cur, int lane) {
    switch (k) {
        case 0: issue<0>(P, cur, lane); break;
        case 1: issue<1>(P, cur, lane); break;
        case 2: issue<2>(P, cur, lane); break;
        default: issue<3>(P, cur, lane); break;
    }
}

// An attention tile, outside the matvec slice loop (its softmax state
// would otherwise share that loop's registers): the wave takes its blocks
// (units w, w + NC, ...) from the slice stream in order, keeping the stream
// D slices ahead, and folds each into its own state, with no barrier; a
// wave without any block consumes its one empty slice. The waves holding
// blocks then leave their states in LDS, and after one barrier wave h < G
// merges head h's states in wave order and publishes the result as the
// tile's (o, m, l); the last head published ends the instruction. False on
// abort.
// A wave that appended the step's K/V entry waits for that store before it
// leaves the tile, in a resident launch (after its part of the tile, so
// the tile is not held up): every later instruction of this unit starts once
// all its waves have left, so everything the unit publishes afterwards - and
// with it the next step's token - follows the completed append. A single
// step needs no wait: the kernel's end completes every store.
__device__ __forceinline__ bool attn_tile_left(const KParams &P, Ctx &c) {
    if (P.n_steps > 1 && c.kv_pending) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    c.kv_pending = false;
    return true;
}

template <int NB, int G>
__device__ __forceinline__ bool attn_tile(const KParams &P, Ctx &c, Cur &ic, Cur &cc, const Ins &in, int &slot) {
    AttnAcc<G> a;
    attn_acc_init(a);
    const int pc = in.pc, lane = c.lane();
    // the cursor leaves the instruction after the wave's last block (or its
    // empty slice)
    while (uni(cc.pc == pc && cc.step == in.step && cc.op == OP_ATTN)) {
        v4u buf[4];
        take_any(slot, buf);
        if (cc.u < cc.nu) attn_fold_block<G>(c, cc, in, buf, a);
        issue_any(slot, P, ic, lane);
        cur_next<NB>(P, c, ic);
        cur_next<NB>(P, c, cc);
        slot = slot + 1 == D ? 0 : slot + 1;
    }
    MK_LDS float *st = attn_states<G>(c);
    if (c.w < in.nblk) {
        float o[G], l[G];
        attn_acc_finish<G>(a, lane, o, l);
        attn_acc_store<G>(a, o, l, st, c.w, lane);
    }
    if (!uni(lbar(c, pc))) return false;
    if (c.w >= G) return attn_tile_left(P, c);
    const int h = c.w, nw = min(NC, in.nblk);
    float O, M, L;
    merge_init(O, M, L);
    for (int w = 0; w < nw; ++w) {
        const MK_LDS float *s = st + (w * G + h) * ATTN_PART;
        merge_step(O, M, L, s[lane], s[64], s[65]);
    }
    const size_t pbase = (((size_t)in.layer * P.nkv + in.g) * in.nch + in.c) * G * ATTN_PART;
    const __amdgpu_buffer_rsrc_t rp = tres(P.tpart + pbase, (uint32_t)(G * ATTN_PART));
    tput(rp, (uint32_t)(h * ATTN_PART + lane), O, c.tag);
    if (lane == 0) {
        tput(rp, (uint32_t)(h * ATTN_PART + 64), M, c.tag);
        tput(rp, (uint32_t)(h * ATTN_PART + 65), L, c.tag);
    }
    uint32_t m = 0;
    if (lane == 0) m = lds_add_local(c.misc + M_AFIN, 1u);
    m = __builtin_amdgcn_readfirstlane(m);
    // a tile's publishes all end before the next tile's begin, so the count
    // reaches a multiple of G exactly at its last publish
    if ((m + 1) % G != 0) return attn_tile_left(P, c);
    if (in.tr && lane == 0) in.tr[TR_END] = wall_clock64();
    if (lane == 0) lds_add_local(c.misc + M_DONE, 1u);
    return attn_tile_left(P, c);
}

// The wave's main loop. Slices are consumed in the order they were issued,
// so the slot being consumed always has the other D - 1 slots issued after
// it, and a wait for all but the 4 (D - 1) newest loads is a wait for
// exactly this slot. At an instruction boundary the wave leaves the previous instruction
// and enters the next one while the slices already issued stay in flight.
// A resident launch runs its steps one after the other: past a step's END
// the slots hold empty loads, which the wave waits for before it restarts
// its cursors at the next step's first instruction and refills its window
// (that step's layer 0 waits for this step's token anyway).
template <int NB, int G>
__device__ __forceinline__ void run(const KParams &P, Ctx &c) {
    static_assert(D >= 2 && D <= 4, "two to four slots");
    Cur ic, cc;
    Ins in{};
    bool ok = true;
    for (int step = 0; uni(ok && step < P.n_steps); ++step) {
        // a step starts with its first D slices issued; the slots the
        // previous step left hold empty loads issued past its END
        if (step > 0) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        split_build<NB>(P, c, step);
        cur_load<NB>(P, c, ic, 0, step);
        cur_load<NB>(P, c, cc, 0, step);
        issue<0>(P, ic, c.lane());
        cur_next<NB>(P, c, ic);
        issue<1>(P, ic, c.lane());
        cur_next<NB>(P, c, ic);
        if constexpr (D > 2) {
            issue<2>(P, ic, c.lane());
            cur_next<NB>(P, c, ic);
        }
        if constexpr (D > 3) {
            issue<3>(P, ic, c.lane());
            cur_next<NB>(P, c, ic);
        }
        int slot = 0;
        while (uni(cc.op != OP_END)) {
            // per-instruction accumulators and register activations: nothing of
            // them lives from one instruction to the next (an attention tile never
            // holds a matvec's registers). The record `in` stays outside, which
            // keeps the compiler's view of the cursors uniform.
            Acc<NB> acc;
            RegAct ra;
            if (!uni(enter<NB, G>(P, c, cc, in, acc, ra))) {
                ok = false;
                break;
            }
            if (cc.op == OP_ATTN) {
                if (!uni(attn_tile<NB, G>(P, c, ic, cc, in, slot))) {
                    ok = false;
                    break;
                }
            } else {
                for (;;) {
                    v4u buf[4];
                    take_any(slot, buf);
                    const bool empty = cc.u >= cc.nu;
                    if (!empty) consume_mv<NB>(P, c, cc, in, buf, acc, ra);
                    const bool last = empty || (cc.s == cc.sp - 1 && cc.u + NC >= cc.nu);
                    issue_any(slot, P, ic, c.lane());
                    cur_next<NB>(P, c, ic);
                    cur_next<NB>(P, c, cc);
                    slot = slot + 1 == D ? 0 : slot + 1;
                    if (uni(last)) break;
                }
            }
            if (!uni(leave<NB, G>(P, c, in, acc))) {
                ok = false;
                break;
            }
        }
    }
    // no load may still be writing a slot register when the wave ends
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    if (c.pending_timeout >= 0) raise_err(c, ERR_TIMEOUT, c.pending_timeout);
}

}  // namespace

// Occupancy target 3 caps the compiler at SLOT_VGPR0 VGPRs; the slot
// registers above make the kernel's real count 232 (2 waves per SIMD, which
// one 8-wave workgroup per compute unit needs).
template <int NB, int G>
__global__ __attribute__((amdgpu_flat_work_group_size(BLOCK_THREADS, BLOCK_THREADS), amdgpu_waves_per_eu(3, 3))) void mk_megakernel(
    KParams P) {
    extern __shared__ char lds_raw[];
    MK_LDS char *lds = (MK_LDS char *)lds_raw;
    Ctx c;
    c.misc = (MK_LDS uint32_t *)lds;
    c.q = (const MK_LDS int32_t *)(lds + P.queue_off);
    c.xrow = (MK_LDS float *)(lds + P.xrow_off);
    c.act = (MK_LDS float *)(lds + P.act_off);
    c.cu = blockIdx.x;
    c.w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    c.nbar = 0;
    c.tag = P.tag;
    c.watchdog = P.watchdog;
    c.err = P.err;
    c.host_err = P.host_err;
    c.pending_timeout = -1;
    c.kv_pending = false;
    for (int i = threadIdx.x; i < MISC_BYTES / 4; i += BLOCK_THREADS) c.misc[i] = i == M_NQ ? (uint32_t)P.Q : 0u;
    __syncthreads();
    // the CU's queue and the request lengths are read once, here: scalar
    // reads of them later in the step would miss in caches that the weight
    // stream has long since flushed
    {
        MK_LDS int32_t *q = (MK_LDS int32_t *)(lds + P.queue_off);
        const int32_t *src = P.queue + (int64_t)c.cu * P.Q * INSTR_WORDS;
        for (int i = threadIdx.x; i < P.Q * LDS_INSTR_WORDS; i += BLOCK_THREADS) {
            const int32_t v = src[(i / LDS_INSTR_WORDS) * INSTR_WORDS + i % LDS_INSTR_WORDS];
            q[i] = v;
            if (i % LDS_INSTR_WORDS == W_OP && v == OP_END)
                __hip_atomic_fetch_min(c.misc + M_NQ, (uint32_t)(i / LDS_INSTR_WORDS), __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_WORKGROUP);
        }
        if (threadIdx.x < (unsigned)P.B) c.misc[M_KVLEN + threadIdx.x] = (uint32_t)P.kv_lens[threadIdx.x];
    }
    __syncthreads();
    c.nq = (int)__builtin_amdgcn_readfirstlane(c.misc[M_NQ]);
    // the lengths are in LDS (their loads have returned): count this
    // workgroup as started
    if (threadIdx.x == 0)
        __hip_atomic_fetch_add(P.counters + (int64_t)P.start_ctr * CTR_STRIDE, 1, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    run<NB, G>(P, c);
}

}  // namespace mk
