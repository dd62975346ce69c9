// mk_kernels.h - kernel parameter block and host launchers (internal).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mk {

// Everything a step needs, passed by value as the kernel argument block.
struct KParams {
    // schedule
    const int32_t *queue;     // [n_cus, Q, INSTR_WORDS]
    const int32_t *events;    // [n_events, EV_WORDS] merge events
    int32_t *counters;        // [n_counters * CTR_STRIDE]
    int32_t Q, epoch, n_cus;  // epoch: launches so far, this one included (start counter)
    int32_t start_ctr;        // counter every workgroup bumps once it has read kv_lens
    uint32_t tag;             // the first step's tag on every exchanged activation (never 0); step s uses tag + s
    int32_t n_steps;          // greedy decode steps this launch runs (the grid stays resident across them)
    int32_t step_epoch;       // merge-event epoch of the first step (steps so far, this one included)
    uint64_t *ttok;           // [n_steps][B] tagged tokens each step hands to the next, or null (one step)
    int32_t queue_off, xrow_off, act_off, nw_off;  // LDS byte offsets
    int32_t act_stride;       // floats per request in the activation area
    int32_t xrow_stride;      // floats per request in the residual-row area
    int64_t watchdog;
    // model
    int32_t L, H, nq, nkv, d, F, V, has_embed, B, T, max_pages;
    float eps;
    const uint16_t *embed;
    const uint16_t *final_norm;
    const uint64_t *wtab;     // [L, 8]: attn_norm, wqkv, wo, mlp_norm, w_gate, w_up, w_down, -
    const float2 *rope;       // [capacity, d/2] (cos, sin)
    // step io
    const int32_t *tokens_in;
    const float *hidden_in;
    const int32_t *kv_lens;
    uint16_t *k_pool, *v_pool;
    int32_t n_pages;
    const int32_t *page_table;
    int32_t *tokens_out, *kv_lens_out;
    float *logits_out, *hidden_out;
    // resident interpreter: tagged activations, 64-bit words (low: fp32 bits,
    // high: tag), each written once per step
    uint64_t *tx;      // [2L][B][H]: x_1 .. x_{2L} (x_v at index v - 1)
    uint64_t *tqkv;    // [L][B][(nq + 2 nkv) d]
    uint64_t *tact;    // [L][B][F]
    uint64_t *tpart;   // [L][nkv][B chunks][G][ATTN_PART] attention tile states
    uint64_t *to;      // [L][B][nq d] merged attention outputs
    uint64_t *tlm;     // [lm slots][B][2] argmax partials (value, index)
    int32_t attn_chunks;  // tiles per request, on average: each kv head has B attn_chunks tiles
    int32_t attn_split;   // SPLIT_BALANCED or SPLIT_PER_REQUEST
    // one-kernel-per-op baseline scratch (fp32, overwritten in place)
    float *x;          // [B, H] residual stream
    float *qkv;        // [B, (nq + 2 nkv) d]
    float *o;          // [B, nq d] attention output
    float *act;        // [B, F] gated MLP activation
    float *attn_part;  // [nkv, B chunks, G, ATTN_PART_STRIDE]
    float *lm_part;    // [lm slots, B, 2]
    int32_t *err;      // device error word
    int32_t *host_err; // mapped host mirror of the error word
    int64_t *trace;    // [n_cus, Q, TRACE_WORDS] or null
};

constexpr int ATTN_PART_STRIDE = 68;

// The resident interpreter exists for B in 1..8 and G = nq / nkv in {1, 2, 4, 8}.
bool megakernel_supports(int B, int G);
hipError_t fill_u32(uint32_t *p, size_t n, uint32_t v, hipStream_t s);
hipError_t launch_megakernel(const KParams &p, int lds_bytes, hipStream_t s);
// The file-scope device array behind mk_decode_step_static, one per device.
constexpr size_t STATIC_SCRATCH_BYTES = (size_t)64 << 20;  // MK_STATIC_SCRATCH_BYTES of mk.h
hipError_t static_scratch_setup(int device);  // with `device` current; once per device
void *static_scratch(int device);             // its device address, or null before set-up
hipError_t setup_megakernel(int B, int G, int lds_bytes);
hipError_t megakernel_occupancy(int B, int G, int lds_bytes, int *blocks_per_cu);
hipError_t launch_unfused(const KParams &p, float *u_scratch, float *qrot, hipStream_t s);
hipError_t copy_probe(const void *src, void *dst, size_t bytes, hipStream_t s);
hipError_t litmus(int pairs, int n, int rounds, int mode, int32_t *data, int32_t *flags, int32_t *res);
hipError_t split_probe(const int32_t *kv, int n_cases, int B, int T, int mode, int cap, int32_t *out);
hipError_t hop_probe(int32_t *ctr, float *xbuf, int n_cus, int rounds, int variant, int32_t *res);
hipError_t ll_probe(uint64_t *buf, int n_cus, int per, int copies, int rounds, int32_t *res);
hipError_t regstream_probe(const void *src, size_t bytes, int blocks, int threads, int depth, uint32_t *out);
hipError_t launch_rope_table(float2 *table, int capacity, int d, double theta, hipStream_t s);

}  // namespace mk
