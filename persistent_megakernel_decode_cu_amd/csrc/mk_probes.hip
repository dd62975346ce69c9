// mk_probes.hip - measurement kernels behind the mk_debug_* exports: the
// latency of one dependency hop between workgroups (fenced counters and
// tagged words), a cross-XCD visibility litmus of the tagged-word protocol,
// the read bandwidth of one resident workgroup per compute unit streaming
// through registers, and a plain copy of known size that calibrates the
// traffic counters.
#include "mk_device.h"

namespace mk {

namespace {

// launch bound of the register-stream probe (launched with up to 512 threads)
constexpr int P_THREADS = 640;

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

// The attention split of mk_device.h for a batch of kv lengths per case, one
// wave per case.
__global__ __launch_bounds__(64) void mk_split_probe(const int32_t *kv, int B, int T, int mode, int cap, int32_t *out) {
    const int cs = blockIdx.x, lane = threadIdx.x;
    int nb[MAX_B], n[MAX_B];
#pragma unroll
    for (int b = 0; b < MAX_B; ++b) nb[b] = b < B ? attn_nblocks(kv[(int64_t)cs * B + b], cap) : 0;
    attn_split_counts(nb, B, T, mode == SPLIT_BALANCED, lane, n);
    int32_t *o = out + (int64_t)cs * (4 * T + B + 1);
    for (int t = lane; t < T; t += 64) {
        int b, lo, hi;
        bool last;
        attn_split_tile(nb, n, t, b, lo, hi, last);
        o[4 * t] = b;
        o[4 * t + 1] = lo;
        o[4 * t + 2] = hi;
        o[4 * t + 3] = last ? 1 : 0;
    }
    if (lane <= B) o[4 * T + lane] = attn_split_first(n, lane);
}

hipError_t split_probe(const int32_t *kv, int n_cases, int B, int T, int mode, int cap, int32_t *out) {
    hipLaunchKernelGGL(mk_split_probe, dim3(n_cases), dim3(64), 0, nullptr, kv, B, T, mode, cap, out);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return hipDeviceSynchronize();
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
