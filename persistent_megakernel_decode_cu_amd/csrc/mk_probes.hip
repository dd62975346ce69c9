// mk_probes.hip - measurement kernels behind the mk_debug_* exports: the
// latency of one dependency hop between workgroups, and the read bandwidth of
// one resident workgroup per compute unit streaming through registers.
#include "mk_device.h"

namespace mk {

namespace {

enum : int { PM_LANDED = 1, PM_ABORT = 2, PM_WPOS = 16 };
// shape of the ring probe: one loader wave, PNC consumer waves, 1 KiB granules
constexpr int PNC = 8;
constexpr int P_WAVES = PNC + 2;
constexpr int P_THREADS = P_WAVES * 64;
constexpr int P_GRANULE = 1024;
constexpr int P_MISC = 4096;

__device__ __forceinline__ uint32_t lds_ld(MK_LDS uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP);
}
__device__ __forceinline__ void lds_st(MK_LDS uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// HBM -> LDS, 16 bytes per active lane at lds_addr + 16 * lane. Issued from
// inline assembly so that the compiler does not conservatively wait for the
// transfer before unrelated LDS accesses; the loader tracks completion with
// its own vmcnt waits. m0 carries the LDS base; nothing else in this kernel
// uses m0.
__device__ __forceinline__ void dma16(const void *gptr, uint32_t lds_addr) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 1\n\t"
        "global_load_lds_dwordx4 %1, off"
        :
        : "s"(lds_addr), "v"(gptr)
        : "memory");
}

}  // namespace


// A chain of grid-wide hops. Round r: every workgroup waits until all
// workgroups finished round r - 1, optionally acquires at agent scope, reads
// the 8-float slices all workgroups wrote in round r - 1 and writes its own,
// optionally releases at agent scope and signals. Kernel time / rounds is the
// cost of one hop on the critical path.
// variant bits: 0 no release fence, 1 no acquire fence, 2 exchange the
// slices, 3 tree signal (16-way group counters, then a top counter whose last
// arriver raises 16 replicated flags; each workgroup polls one replica)
// instead of one shared counter per round, 4 spread the exchanged vector
// (128-byte line i at i * 4 KiB), 5 read it with plain loads instead of
// device-coherent ones.
// ctr layout (int32 words): shared-counter mode uses word r * 32 for round r;
// tree mode puts the top counter at word 0, group g at (1 + g) * 1024 and
// replica k at (1 + groups + k) * 1024.
constexpr int HOP_SPREAD = 1024;  // words: 4 KiB

__device__ __forceinline__ int hop_xidx(int e, bool spread) { return spread ? (e >> 5) * HOP_SPREAD + (e & 31) : e; }

__global__ __launch_bounds__(64) void mk_hop_probe(int32_t *ctr, float *xbuf, int rounds, int variant,
                                                   int64_t watchdog, int32_t *res) {
    const int cu = blockIdx.x, n = gridDim.x, lane = threadIdx.x;
    const bool rel = !(variant & 1), acq = !(variant & 2), data = (variant & 4) != 0;
    const bool tree = (variant & 8) != 0, spread = (variant & 16) != 0, plain = (variant & 32) != 0;
    const int ngroups = (n + 15) / 16, grp = cu / 16, gsize = min(16, n - grp * 16);
    const int nx = n * 8;
    const int xlen = spread ? ((nx + 31) / 32) * HOP_SPREAD : nx;
    float acc = 0.0f;
    for (int r = 0; r < rounds; ++r) {
        if (r > 0) {
            int64_t spins = 0;
            const int32_t *pp = tree ? ctr + (1 + ngroups + (cu & 15)) * HOP_SPREAD : ctr + (int64_t)r * CTR_STRIDE;
            const int32_t target = tree ? r : n;
            while (__hip_atomic_load(pp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < target) {
                if (++spins > watchdog) {
                    if (lane == 0) atomicAdd(res, 1);
                    return;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            wait_vmcnt<0>();
            if (acq) {
                __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                wait_vmcnt<0>();
            }
        }
        if (data) {
            // 16-byte chunks: chunk c holds floats 4c .. 4c + 3 (one 128-byte
            // line = 8 chunks)
            float *src = xbuf + (size_t)(r & 1) * xlen;
            const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(src, xlen * 4);
            const int nch = nx / 4;
            v4f part = {0.0f, 0.0f, 0.0f, 0.0f};
            for (int c = lane; c < nch; c += 64) {
                const int off = hop_xidx(c * 4, spread) * 4;
                part += plain ? *(const v4f *)((const char *)src + off) : coherent_load16f(rs, off);
            }
            acc += part.x + part.y + part.z + part.w;
            if (lane < 8) {
                float *dst = xbuf + (size_t)((r + 1) & 1) * xlen + hop_xidx(cu * 8 + lane, spread);
                if (plain) *dst = acc;
                else __hip_atomic_store(dst, acc, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        wait_vmcnt<0>();
        if (rel) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
        if (lane == 0) {
            if (tree) {
                const int32_t og = __hip_atomic_fetch_add(ctr + (1 + grp) * HOP_SPREAD, 1, __ATOMIC_RELAXED,
                                                          __HIP_MEMORY_SCOPE_AGENT);
                if (og == gsize * (r + 1) - 1) {
                    if (acq) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    if (rel) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                    const int32_t ot = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    if (ot == ngroups * (r + 1) - 1) {
                        if (acq) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                        if (rel) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                        for (int k = 0; k < 16; ++k)
                            __hip_atomic_store(ctr + (1 + ngroups + k) * HOP_SPREAD, r + 1, __ATOMIC_RELAXED,
                                               __HIP_MEMORY_SCOPE_AGENT);
                    }
                }
            } else {
                __hip_atomic_fetch_add(ctr + (int64_t)(r + 1) * CTR_STRIDE, 1, __ATOMIC_RELAXED,
                                       __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
    if (acc == 1234.5f) res[1] = 1;
}

hipError_t hop_probe(int32_t *ctr, float *xbuf, int n_cus, int rounds, int variant, int32_t *res) {
    int64_t wd = (int64_t)1 << 22;
    void *args[] = {&ctr, &xbuf, &rounds, &variant, &wd, &res};
    return hipLaunchCooperativeKernel((const void *)mk_hop_probe, dim3(n_cus), dim3(64), args, 0, nullptr);
}

// Epoch-tagged exchange (each fp32 value travels with its round number in
// one 64-bit word, so a reader that sees the tag also sees the value). Round
// r: every workgroup writes its `per` values tagged r + 1 into buffer r & 1,
// then reads all n * per words until every tag is r + 1; no counters, no
// fences. Kernel time / rounds is the hop cost. buf: 2 * n * per uint64.
__global__ __launch_bounds__(64) void mk_ll_probe(uint64_t *buf, int per, int copies, int rounds,
                                                  int64_t watchdog, int32_t *res) {
    const int cu = blockIdx.x, n = gridDim.x, lane = threadIdx.x;
    const int total = n * per;
    float acc = 0.0f;
    for (int r = 0; r < rounds; ++r) {
        // copy c of round r at (r & 1) * copies + c; workgroup b reads copy b % copies
        uint64_t *cur0 = buf + (size_t)(r & 1) * copies * total;
        const __amdgpu_buffer_rsrc_t ws = coherent_rsrc(cur0, (uint32_t)total * copies * 8);
        for (int c = 0; c < copies; ++c)
            for (int i = lane; i < per; i += 64) {
                const uint32_t v = __float_as_uint(acc + (float)i);
                __builtin_amdgcn_raw_buffer_store_b64(v2u{v, (uint32_t)(r + 1)}, ws,
                                                      (uint32_t)(c * total + cu * per + i) * 8, 0, CP_SC1);
            }
        const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(cur0 + (size_t)(cu % copies) * total, (uint32_t)total * 8);
        // wait for everyone's words of this round, re-reading only missing ones
        float sum = 0.0f;
        for (int base = 0; base < total; base += 64 * 32) {
            uint32_t pending = 0;
            for (int k = 0; k < 32; ++k)
                if (base + k * 64 + lane < total) pending |= 1u << k;
            int64_t spins = 0;
            while (__builtin_amdgcn_ballot_w64(pending != 0) != 0) {
                // issue every outstanding load first, then check the tags
                v2u w[32];
#pragma unroll
                for (int k = 0; k < 32; ++k)
                    if (pending & (1u << k))
                        w[k] = __builtin_amdgcn_raw_buffer_load_b64(rs, (uint32_t)(base + k * 64 + lane) * 8, 0,
                                                                    CP_SC1);
#pragma unroll
                for (int k = 0; k < 32; ++k)
                    if ((pending & (1u << k)) && w[k].y == (uint32_t)(r + 1)) {
                        pending &= ~(1u << k);
                        sum += __uint_as_float(w[k].x);
                    }
                if (++spins > watchdog) {
                    if (lane == 0) atomicAdd(res, 1);
                    return;
                }
                if (__builtin_amdgcn_ballot_w64(pending != 0) != 0) __builtin_amdgcn_s_sleep(1);
            }
        }
        acc += wave_sum(sum) * 1e-30f;
    }
    if (acc == 1234.5f) res[1] = 1;
}

hipError_t ll_probe(uint64_t *buf, int n_cus, int per, int copies, int rounds, int32_t *res) {
    int64_t wd = (int64_t)1 << 22;
    void *args[] = {&buf, &per, &copies, &rounds, &wd, &res};
    return hipLaunchCooperativeKernel((const void *)mk_ll_probe, dim3(n_cus), dim3(64), args, 0, nullptr);
}

// One workgroup per compute unit, blockDim / 64 waves; each wave streams
// 4 KiB slices (slice k of wave w of workgroup b at ((k * grid + b) * waves +
// w) * 4 KiB) with D slices in flight in registers, XOR-folding each landed
// slice.
template <int D>
__global__ __launch_bounds__(P_THREADS, 1) void mk_regstream_probe(const v4u *src, int64_t n_slices,
                                                                        uint32_t *out) {
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nw = blockDim.x >> 6;
    const int64_t gw = (int64_t)blockIdx.x * nw + w, stride = (int64_t)gridDim.x * nw;
    v4u buf[D][4];
    uint32_t acc = 0;
    auto issue = [&](v4u(&r)[4], int64_t s) {
        if (s < n_slices) {
            const v4u *g = src + s * 256 + lane;
#pragma unroll
            for (int j = 0; j < 4; ++j) r[j] = g[j * 64];
        }
    };
#pragma unroll
    for (int i = 0; i < D; ++i) issue(buf[i], gw + i * stride);
    for (int64_t s = gw; s < n_slices; s += D * stride) {
#pragma unroll
        for (int i = 0; i < D; ++i) {
            if (s + i * stride < n_slices) {
#pragma unroll
                for (int j = 0; j < 4; ++j) acc ^= buf[i][j].x ^ buf[i][j].y ^ buf[i][j].z ^ buf[i][j].w;
            }
            issue(buf[i], s + (i + D) * stride);
        }
    }
    if (acc == 0x9e3779b9u) out[0] = acc;
}

hipError_t regstream_probe(const void *src, size_t bytes, int blocks, int threads, int depth, uint32_t *out) {
    const int64_t n = (int64_t)(bytes / 4096);
    const v4u *s = (const v4u *)src;
    switch (depth) {
        case 1: hipLaunchKernelGGL(mk_regstream_probe<1>, dim3(blocks), dim3(threads), 0, 0, s, n, out); break;
        case 2: hipLaunchKernelGGL(mk_regstream_probe<2>, dim3(blocks), dim3(threads), 0, 0, s, n, out); break;
        case 3: hipLaunchKernelGGL(mk_regstream_probe<3>, dim3(blocks), dim3(threads), 0, 0, s, n, out); break;
        case 4: hipLaunchKernelGGL(mk_regstream_probe<4>, dim3(blocks), dim3(threads), 0, 0, s, n, out); break;
        default: hipLaunchKernelGGL(mk_regstream_probe<6>, dim3(blocks), dim3(threads), 0, 0, s, n, out); break;
    }
    return hipGetLastError();
}

// Cross-XCD message-passing litmus. Workgroup 2k writes, workgroup 2k+1 (on
// another XCD under the round-robin placement) reads. Per round r the writer
// stores r into n words and raises a flag; the reader first reads the words
// with plain loads (planting possibly stale copies in its caches), waits for
// the flag, then reads them again with plain loads (stale ones counted into
// res[0]) and with device-coherent loads (res[1]); then it acknowledges the
// round. res[2] counts watchdog expiries.
// mode 0: plain stores, agent-scope release fence before the flag, agent-scope
//   acquire fence after it (the fenced protocol);
// mode 1: device-coherent stores, s_waitcnt vmcnt(0) before the flag, no
//   fences (the coherent-access protocol).
__global__ __launch_bounds__(256) void mk_litmus(int32_t *data, int32_t *flags, int n, int rounds, int mode,
                                                 int64_t watchdog, int32_t *res) {
    const int pair = blockIdx.x >> 1, role = blockIdx.x & 1, tid = threadIdx.x;
    int32_t *d = data + (size_t)pair * n;
    int32_t *flag = flags + pair * 64, *ack = flags + pair * 64 + 32;
    const __amdgpu_buffer_rsrc_t rs = coherent_rsrc(d, (uint32_t)n * 4);
    int stale_plain = 0, stale_coh = 0, sink = 0;
    for (int r = 1; r <= rounds; ++r) {
        if (role == 0) {
            if (tid == 0) {
                int64_t spins = 0;
                while (__hip_atomic_load(ack, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < r - 1) {
                    if (++spins > watchdog) {
                        atomicAdd(res + 2, 1);
                        __hip_atomic_store(flag, 1 << 30, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            __syncthreads();
            for (int i = tid; i < n; i += 256) {
                if (mode == 1) coherent_store4f(rs, (uint32_t)i * 4, __int_as_float(r));
                else d[i] = r;
            }
            wait_vmcnt<0>();
            __syncthreads();
            if (tid == 0) {
                if (mode == 0) __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __hip_atomic_store(flag, r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        } else {
            for (int i = tid; i < n; i += 256) sink += d[i];
            if (tid == 0) {
                int64_t spins = 0;
                while (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < r) {
                    if (++spins > watchdog) {
                        atomicAdd(res + 2, 1);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                wait_vmcnt<0>();
                if (mode == 0) {
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    wait_vmcnt<0>();
                }
            }
            __syncthreads();
            for (int i = tid; i < n; i += 256) {
                stale_plain += d[i] != r;
                stale_coh += __float_as_int(coherent_load4f(rs, (uint32_t)i * 4)) != r;
            }
            wait_vmcnt<0>();
            __syncthreads();
            if (tid == 0) __hip_atomic_store(ack, r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
    if (stale_plain) atomicAdd(res, stale_plain);
    if (stale_coh) atomicAdd(res + 1, stale_coh);
    if (sink == 0x7fffffff) res[3] = sink;
}

hipError_t litmus(int pairs, int n, int rounds, int mode, int32_t *data, int32_t *flags, int32_t *res) {
    int64_t wd = (int64_t)1 << 22;
    void *args[] = {&data, &flags, &n, &rounds, &mode, &wd, &res};
    hipError_t e = hipLaunchCooperativeKernel((const void *)mk_litmus, dim3(2 * pairs), dim3(256), args, 0, nullptr);
    if (e != hipSuccess) return e;
    return hipDeviceSynchronize();
}

// One wave: DMA n granules into LDS at byte offset `off` exactly as the
// loader does, wait, then copy those LDS bytes out with ordinary loads.
__global__ __launch_bounds__(64) void mk_dma_probe(const char *src, char *dst, int n, int off) {
    extern __shared__ char lds_raw[];
    MK_LDS char *lds = (MK_LDS char *)lds_raw;
    const int lane = threadIdx.x;
    for (int i = lane; i < LDS_LIMIT / 4; i += 64) ((MK_LDS uint32_t *)lds)[i] = 0u;
    __syncthreads();
    const uint32_t base = (uint32_t)(uintptr_t)lds + (uint32_t)off;
    if (n < 0) {
        // two transfers, one m0 value, the second with instruction offset 1024
        const char *g = src + lane * 16;
        asm volatile(
            "s_mov_b32 m0, %0\n\t"
            "s_nop 1\n\t"
            "global_load_lds_dwordx4 %1, off\n\t"
            "global_load_lds_dwordx4 %1, off offset:1024"
            :
            : "s"(base), "v"(g)
            : "memory");
        n = 2;
    } else {
        for (int k = 0; k < n; ++k)
            dma16(src + (size_t)k * P_GRANULE + lane * 16, __builtin_amdgcn_readfirstlane(base + k * P_GRANULE));
    }
    wait_vmcnt<0>();
    for (int k = 0; k < n; ++k) {
        const v4u v = *(const MK_LDS v4u *)(lds + off + k * P_GRANULE + lane * 16);
        *(v4u *)(dst + (size_t)k * P_GRANULE + lane * 16) = v;
    }
}

hipError_t dma_probe(const void *src, void *dst, int n_kib, int off_kib) {
    hipError_t e = hipFuncSetAttribute((const void *)mk_dma_probe, hipFuncAttributeMaxDynamicSharedMemorySize,
                                       LDS_LIMIT);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mk_dma_probe, dim3(1), dim3(64), LDS_LIMIT, 0, (const char *)src, (char *)dst, n_kib,
                       off_kib * P_GRANULE);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipDeviceSynchronize();
}

// Ring protocol probe: wave 0 streams n granules of a known pattern through
// a ring of `ring` granules exactly as the loader does (issue, keep `depth`
// in flight, publish landed); PNC consumer waves take granules round-robin,
// wait for them to land, check every word and release them. `variant` 1
// makes the loader read back one word of the newest landed granule before
// publishing. Counts mismatching words into errs[0] and granules checked
// into errs[1].
__global__ __launch_bounds__(P_THREADS, 1) void mk_ring_probe(const uint32_t *src, int n, int ring, int depth,
                                                                   int variant, int64_t watchdog, int32_t *errs) {
    extern __shared__ char lds_raw[];
    MK_LDS char *lds = (MK_LDS char *)lds_raw;
    MK_LDS uint32_t *misc = (MK_LDS uint32_t *)lds;
    MK_LDS char *rb = lds + P_MISC;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    src += (size_t)blockIdx.x * n * 256;
    for (int i = threadIdx.x; i < P_MISC / 4; i += P_THREADS) misc[i] = 0;
    __syncthreads();
    const int nl = (variant >> 8) & 15;
    const int gb = ((variant >> 12) & 15) ? ((variant >> 12) & 15) : 1;  // granules per DMA batch: 1 or 4
    const bool regs = (variant >> 16) & 1;                                // register-staged loaders
    const bool inter = (variant >> 17) & 1;  // batch t of workgroup b at (t * gridDim.x + b) * 4 KiB
    const bool plain = (variant >> 18) & 1;  // ordinary loads instead of non-temporal ones
    variant &= 255;
    if (inter) src -= (size_t)blockIdx.x * n * 256;  // undo the per-block slice
    if (regs && nl >= 1) {
        // nl loader waves; batch t = 4 granules issued by loader t % nl with
        // ordinary 16-byte loads into registers, 4 batches in flight, then
        // written into the ring once its slots are free
        const int ncons = P_WAVES - nl;
        const int nbatch = n / 4;
        if (wave < nl) {
            uint32_t mine = 0, lim = ring;
            v4u ra[4], rbuf[4], rc[4], rd[4];
            auto issue = [&](v4u (&r)[4], int t) {
                if (t < nbatch) {
                    const size_t bt = inter ? (size_t)t * gridDim.x + blockIdx.x : (size_t)t;
                    const v4u *g = (const v4u *)(src + bt * 4 * 256) + lane;
                    if (plain) {
#pragma unroll
                        for (int i = 0; i < 4; ++i) r[i] = g[i * 64];
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i) r[i] = __builtin_nontemporal_load(g + i * 64);
                    }
                }
            };
            auto commit = [&](v4u (&r)[4], int t) -> bool {
                if (t >= nbatch) return true;
                const uint32_t k = (uint32_t)t * 4;
                if (k + 4 > lim) {
                    int64_t spins = 0;
                    for (;;) {
                        uint32_t mn = lds_ld(misc + PM_WPOS);
                        for (int w = 1; w < ncons; ++w) mn = min(mn, lds_ld(misc + PM_WPOS + w));
                        lim = __builtin_amdgcn_readfirstlane(mn + ring);
                        if (k + 4 <= lim) break;
                        if (++spins > watchdog) {
                            lds_st(misc + PM_ABORT, 1u);
                            return false;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) *(MK_LDS v4u *)(rb + ((k + i) % ring) * P_GRANULE + lane * 16) = r[i];
                mine += 4;
                asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                __hip_atomic_store(misc + PM_LANDED + 32 + wave, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
                return true;
            };
            const int step = nl;
            int t = wave;
            issue(ra, t);
            issue(rbuf, t + step);
            issue(rc, t + 2 * step);
            issue(rd, t + 3 * step);
            for (; t < nbatch; t += 4 * step) {
                if (!commit(ra, t)) return;
                issue(ra, t + 4 * step);
                if (!commit(rbuf, t + step)) return;
                issue(rbuf, t + 5 * step);
                if (!commit(rc, t + 2 * step)) return;
                issue(rc, t + 6 * step);
                if (!commit(rd, t + 3 * step)) return;
                issue(rd, t + 7 * step);
            }
        } else {
            const int w = wave - nl;
            int bad = 0, seen = 0;
            for (int g = w; g < nbatch * 4; g += ncons) {
                const int tb = g / 4;
                const int j = tb % nl;
                const uint32_t need = (uint32_t)((tb / nl + 1) * 4);
                int64_t spins = 0;
                while (lds_ld(misc + PM_LANDED + 32 + j) < need) {
                    if (lds_ld(misc + PM_ABORT) == 1u || ++spins > watchdog) {
                        if (lane == 0) atomicAdd(errs + 2, 1);
                        return;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                const v4u v = *(const MK_LDS v4u *)(rb + (g % ring) * P_GRANULE + lane * 16);
                const uint32_t e = (uint32_t)g * 256u + lane * 4u;
                if (variant == 4)
                    bad += (v.x ^ v.y ^ v.z ^ v.w) == 0x12345678u;
                else
                    bad += (v.x != src[e]) + (v.y != src[e + 1]) + (v.z != src[e + 2]) + (v.w != src[e + 3]);
                ++seen;
                const int gn = g + ncons;
                if (lane == 0) lds_st(misc + PM_WPOS + w, (uint32_t)(gn < nbatch * 4 ? gn : nbatch * 4));
            }
            if (lane == 0) lds_st(misc + PM_WPOS + w, (uint32_t)(nbatch * 4));
            bad = (int)wave_sum((float)bad);
            if (lane == 0) {
                atomicAdd(errs, bad);
                atomicAdd(errs + 1, seen);
            }
        }
        return;
    }
    if (nl >= 1) {
        // nl loader waves; batch t (granules [t*gb, t*gb+gb)) is issued by
        // loader t % nl with one m0 write; consumers are waves nl .. P_WAVES-1
        // and wait on the issuing loader's own landed count (in granules)
        const int ncons = P_WAVES - nl;
        const int nbatch = n / gb;
        if (wave < nl) {
            const uint32_t ring_lds = (uint32_t)(uintptr_t)rb;
            uint32_t mine = 0, pub = 0, lim = ring;
            for (int t = wave; t < nbatch; t += nl) {
                const uint32_t k = (uint32_t)t * gb;  // first granule of the batch
                if (k + gb > lim) {
                    int64_t spins = 0;
                    for (;;) {
                        wait_vmcnt<0>();
                        pub = mine;
                        lds_st(misc + PM_LANDED + 32 + wave, mine);
                        uint32_t mn = lds_ld(misc + PM_WPOS);
                        for (int w = 1; w < ncons; ++w) mn = min(mn, lds_ld(misc + PM_WPOS + w));
                        lim = __builtin_amdgcn_readfirstlane(mn + ring);
                        if (k + gb <= lim) break;
                        if (++spins > watchdog) {
                            lds_st(misc + PM_ABORT, 1u);
                            return;
                        }
                        __builtin_amdgcn_s_sleep(1);
                    }
                }
                const size_t kk = inter ? ((size_t)t * gridDim.x + blockIdx.x) * gb : (size_t)k;
                const char *g = (const char *)(src + kk * 256 + lane * 4);
                const uint32_t l = __builtin_amdgcn_readfirstlane(ring_lds + (k % ring) * P_GRANULE);
                if (gb == 4) {
                    asm volatile(
                        "s_mov_b32 m0, %0\n\t"
                        "s_nop 1\n\t"
                        "global_load_lds_dwordx4 %1, off\n\t"
                        "global_load_lds_dwordx4 %1, off offset:1024\n\t"
                        "global_load_lds_dwordx4 %1, off offset:2048\n\t"
                        "global_load_lds_dwordx4 %1, off offset:3072"
                        :
                        : "s"(l), "v"(g)
                        : "memory");
                } else {
                    dma16(g, l);
                }
                mine += gb;
                uint32_t dd;
                switch (depth) {
                    case 8: wait_vmcnt<8>(); dd = 8; break;
                    case 32: wait_vmcnt<32>(); dd = 32; break;
                    case 48: wait_vmcnt<48>(); dd = 48; break;
                    case 56: wait_vmcnt<56>(); dd = 56; break;
                    default: wait_vmcnt<16>(); dd = 16; break;
                }
                if (mine > dd && mine - dd > pub) {
                    pub = mine - dd;
                    lds_st(misc + PM_LANDED + 32 + wave, pub);
                }
            }
            wait_vmcnt<0>();
            lds_st(misc + PM_LANDED + 32 + wave, mine);
        } else {
            const int w = wave - nl;
            int bad = 0, seen = 0;
            for (int g = w; g < nbatch * gb; g += ncons) {
                const int t = g / gb;
                const int j = t % nl;
                const uint32_t need = (uint32_t)((t / nl + 1) * gb);
                int64_t spins = 0;
                while (lds_ld(misc + PM_LANDED + 32 + j) < need) {
                    if (lds_ld(misc + PM_ABORT) == 1u || ++spins > watchdog) {
                        if (lane == 0) atomicAdd(errs + 2, 1);
                        return;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                const v4u v = *(const MK_LDS v4u *)(rb + (g % ring) * P_GRANULE + lane * 16);
                const uint32_t e = (uint32_t)g * 256u + lane * 4u;
                if (variant == 4)
                    bad += (v.x ^ v.y ^ v.z ^ v.w) == 0x12345678u;
                else
                    bad += (v.x != src[e]) + (v.y != src[e + 1]) + (v.z != src[e + 2]) + (v.w != src[e + 3]);
                ++seen;
                const int gn = g + ncons;
                if (lane == 0) lds_st(misc + PM_WPOS + w, (uint32_t)(gn < nbatch * gb ? gn : nbatch * gb));
            }
            if (lane == 0) lds_st(misc + PM_WPOS + w, (uint32_t)(nbatch * gb));
            bad = (int)wave_sum((float)bad);
            if (lane == 0) {
                atomicAdd(errs, bad);
                atomicAdd(errs + 1, seen);
            }
        }
        return;
    }
    if (wave == 0) {
        const uint32_t ring_lds = (uint32_t)(uintptr_t)rb;
        uint32_t issued = 0, slot = 0, lim = ring, pub = 0;
        for (int k = 0; k < n; ++k) {
            if (issued >= lim) {
                int64_t spins = 0;
                for (;;) {
                    wait_vmcnt<0>();
                    pub = issued;
                    lds_st(misc + PM_LANDED, issued);
                    uint32_t mn = lds_ld(misc + PM_WPOS);
                    for (int w = 1; w < PNC; ++w) mn = min(mn, lds_ld(misc + PM_WPOS + w));
                    lim = __builtin_amdgcn_readfirstlane(mn + ring);
                    if (issued < lim) break;
                    if (++spins > watchdog) {
                        lds_st(misc + PM_ABORT, 1u);
                        return;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
            }
            dma16(src + (size_t)k * 256 + lane * 4, __builtin_amdgcn_readfirstlane(ring_lds + slot * P_GRANULE));
            ++issued;
            slot = (slot + 1 == (uint32_t)ring) ? 0 : slot + 1;
            switch (depth) {
                case 0: wait_vmcnt<0>(); break;
                case 8: wait_vmcnt<8>(); break;
                case 40: wait_vmcnt<40>(); break;
                default: wait_vmcnt<56>(); break;
            }
            if (issued > (uint32_t)depth && issued - depth > pub) {
                pub = issued - depth;
                if (variant == 1) {
                    const uint32_t s2 = (pub - 1) % ring;
                    const uint32_t v = *(volatile MK_LDS uint32_t *)(rb + s2 * P_GRANULE + lane * 16);
                    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
                    if (v == 0xdeadbeefu) misc[PM_ABORT] = 2;
                }
                lds_st(misc + PM_LANDED, pub);
            }
        }
        wait_vmcnt<0>();
        lds_st(misc + PM_LANDED, issued);
    } else if (wave == 1) {
        // variant 2: agent-scope acquire fences, variant 3: release fences,
        // issued by a second wave while the loader streams
        if (variant >= 2) {
            int64_t spins = 0;
            while (lds_ld(misc + PM_LANDED) < (uint32_t)n && lds_ld(misc + PM_ABORT) != 1u && ++spins < watchdog) {
                (void)__hip_atomic_load(errs + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (variant == 2) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                else __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
                __builtin_amdgcn_s_sleep(2);
            }
        }
    } else if (wave >= 2) {
        const int w = wave - 2;
        int bad = 0, seen = 0;
        for (int g = w; g < n; g += PNC) {
            int64_t spins = 0;
            while (lds_ld(misc + PM_LANDED) < (uint32_t)(g + 1)) {
                if (lds_ld(misc + PM_ABORT) == 1u || ++spins > watchdog) {
                    if (lane == 0) atomicAdd(errs + 2, 1);
                    return;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            const v4u v = *(const MK_LDS v4u *)(rb + (g % ring) * P_GRANULE + lane * 16);
            const uint32_t e = (uint32_t)g * 256u + lane * 4u;
            if (variant == 4)
                bad += (v.x ^ v.y ^ v.z ^ v.w) == 0x12345678u;
            else
                bad += (v.x != src[e]) + (v.y != src[e + 1]) + (v.z != src[e + 2]) + (v.w != src[e + 3]);
            ++seen;
            const int gn = g + PNC;
            if (lane == 0) lds_st(misc + PM_WPOS + w, (uint32_t)(gn < n ? gn : n));
        }
        if (lane == 0) lds_st(misc + PM_WPOS + w, (uint32_t)n);
        bad = (int)wave_sum((float)bad);
        if (lane == 0) {
            atomicAdd(errs, bad);
            atomicAdd(errs + 1, seen);
        }
    }
}

hipError_t ring_probe(const void *src, int n, int ring, int depth, int variant, int32_t *errs, int blocks) {
    const int lds = P_MISC + ring * P_GRANULE;
    hipError_t e = hipFuncSetAttribute((const void *)mk_ring_probe, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(mk_ring_probe, dim3(blocks), dim3(P_THREADS), lds, 0, (const uint32_t *)src, n, ring,
                       depth, variant, (int64_t)1 << 22, errs);
    return hipGetLastError();
}

// Plain HBM streaming read: every thread sums 16-byte loads; the achievable
// read bandwidth of the chip.
__global__ __launch_bounds__(256) void mk_stream_probe(const v4u *src, size_t n16, uint32_t *out) {
    uint32_t acc = 0;
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    for (; i + 3 * stride < n16; i += 4 * stride) {
        const v4u a = src[i], b = src[i + stride], c = src[i + 2 * stride], d = src[i + 3 * stride];
        acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
    }
    for (; i < n16; i += stride) {
        const v4u a = src[i];
        acc ^= a.x ^ a.y ^ a.z ^ a.w;
    }
    if (acc == 0x9e3779b9u) out[0] = acc;
}

hipError_t stream_probe(const void *src, size_t bytes, int blocks, uint32_t *out) {
    hipLaunchKernelGGL(mk_stream_probe, dim3(blocks), dim3(256), 0, 0, (const v4u *)src, bytes / 16, out);
    return hipGetLastError();
}

// Plain device copy of n16 16-byte words: each word is read once and written
// once, so its traffic counters calibrate those of the other kernels.
__global__ __launch_bounds__(256) void mk_copy_probe(const v4u *src, v4u *dst, size_t n16) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n16; i += stride) dst[i] = src[i];
}

hipError_t copy_probe(const void *src, void *dst, size_t bytes, hipStream_t s) {
    hipLaunchKernelGGL(mk_copy_probe, dim3(2048), dim3(256), 0, s, (const v4u *)src, (v4u *)dst, bytes / 16);
    return hipGetLastError();
}

}  // namespace mk
