/* mk.h - C ABI of a persistent decode megakernel for AMD Instinct MI355X
 * (CDNA4, gfx950).
 *
 * One call runs one decode step of a Llama-style dense decoder (batch 1 to
 * 8): RMSNorm, QKV matvec, RoPE with K/V append, GQA attention over a paged
 * K/V cache, O projection with residual, SiLU-gated MLP with residual, and
 * (for models with an embedding) the tied LM head with greedy argmax.
 *
 * The operation follows "Inference MegaKernel" (shaojiemike.top):
 *   - section "why conventional inference still has bubbles": the op chain of
 *     a step, and the end-to-end time equation T_e2e = sum of kernel, launch,
 *     tail and materialisation times plus communication, whose launch, tail
 *     and materialisation terms a resident kernel removes;
 *   - section "unified framework": the lowering chain kernel graph -> tile
 *     graph -> per-SM queue + event counters -> resident worker, and the
 *     four obligations (data visibility, progress, capacity, resources);
 *   - section "hand-written whole-model MegaKernel / principle, schedule and
 *     dataflow": a host script builds the tile DAG and writes one instruction
 *     queue per compute unit; one model binding passes weights, K/V cache,
 *     activations and counters in as objects; a grid sized to the unit count
 *     runs an interpreter loop that fetches an instruction, waits on its
 *     counters, leases on-chip pages, runs the op body, fences and publishes
 *     completions; and the object table (queue [S,Q,32] int32 for the whole
 *     kernel, weights per model instance, paged K/V per request, counters per
 *     dependency interval).
 *
 * Conventions for every call:
 *   - Return value: MK_OK (0) or a positive mk_status code. The text of the
 *     last error on the calling thread is returned by mk_last_error().
 *   - No C++ exception crosses the ABI. One host thread uses a handle at a
 *     time.
 *   - "device pointer" means memory on the handle's HIP device; "host
 *     pointer" means ordinary process memory. The library never frees memory
 *     it did not allocate.
 *   - Streams are passed as `void *` holding a hipStream_t (NULL = the null
 *     stream).
 */
#ifndef MK_H
#define MK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mk_status {
    MK_OK = 0,
    MK_EINVAL = 1,      /* an argument is invalid (null, shape, range) */
    MK_ENOSCHED = 2,    /* mk_decode_step before a successful mk_build_schedule */
    MK_ECAPACITY = 3,   /* queue, LDS staging, attention chunking or K/V
                           pages cannot cover the configured maximum
                           (capacity obligation of the "unified framework"
                           section) */
    MK_ERESOURCE = 4,   /* the resident grid cannot be co-resident at one
                           workgroup per CU (resource obligation) */
    MK_EHIP = 5,        /* a HIP runtime call failed */
    MK_ETIMEOUT = 6,    /* sticky: a device wait exceeded the watchdog bound
                           and the grid bailed out instead of hanging */
    MK_EDEVICE = 7      /* sticky: the device raised an error (invalid opcode,
                           token or page id out of range, NaN logit) */
} mk_status;

typedef enum mk_mode {
    MK_MODE_MEGAKERNEL = 0, /* one resident grid per step */
    MK_MODE_UNFUSED = 1     /* one kernel launch per op (comparison baseline) */
} mk_mode;

/* How the attention work of a step is shared out ("Inference MegaKernel",
 * shaojiemike.top, section "hand-written whole-model MegaKernel / limits": a
 * queue fixed before the step cannot follow requests of different lengths).
 * Each kv head has batch x attn_chunks attention tiles in the queues; which
 * request and which K/V blocks a tile covers is computed on the device at
 * every step from the requests' lengths then, the same way in both modes of
 * mk_mode. Request b covers nb_b = ceil((kv_len_b + 1) / 16) blocks. */
typedef enum mk_attn_split {
    /* the smallest tile size s (blocks) with sum_b ceil(nb_b / s) <= tiles;
     * request b gets ceil(nb_b / s) tiles, the spare ones go to the request
     * with the most blocks (lowest index among equals); each request's
     * blocks are cut evenly over its tiles */
    MK_SPLIT_BALANCED = 0,
    /* attn_chunks tiles per request, whatever its length */
    MK_SPLIT_PER_REQUEST = 1
} mk_attn_split;

/* Model shape and capacity. Requirements: head_dim == 64; n_q_heads a
 * multiple of n_kv_heads with n_q_heads / n_kv_heads <= 8; hidden, ffn and
 * n_q_heads * head_dim each a multiple of 512 or equal to 256; page_tokens
 * == 16; 1 <= max_batch <= 8. */
typedef struct mk_config {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    int32_t has_embed;          /* 1: token in, tied LM head, greedy token
                                   out; 0: hidden vector in and out, no head */
    float rms_eps, rope_theta;
    int32_t max_batch;
    int32_t page_tokens;        /* K/V positions per page, 16 */
    int32_t max_pages_per_req;  /* page-table columns, 1..65535; a request may
                                   hold up to max_pages_per_req * page_tokens
                                   positions */
    int32_t device;             /* HIP device ordinal */
} mk_config;

/* Per-layer weights: device pointers to bf16, row-major [out, in]. */
typedef struct mk_layer_weights {
    const void *attn_norm;  /* [H] */
    const void *wqkv;       /* [(nq + 2 nkv) d, H], rows [q heads | k heads | v heads] */
    const void *wo;         /* [H, nq d] */
    const void *mlp_norm;   /* [H] */
    const void *w_gate;     /* [F, H] */
    const void *w_up;       /* [F, H] */
    const void *w_down;     /* [H, F] */
} mk_layer_weights;

typedef struct mk_weights {
    const void *embed;                /* device [V, H] bf16, also the LM head; NULL if has_embed == 0 */
    const void *final_norm;           /* device [H] bf16; NULL if has_embed == 0 */
    const mk_layer_weights *layers;   /* host array of n_layers entries */
} mk_weights;

typedef struct mk_schedule_desc {
    int32_t batch;           /* requests per step, 1..max_batch */
    int32_t n_cus;           /* compute units of the grid; 0 = the device's count */
    int32_t mode;            /* mk_mode */
    int32_t max_kv_len;      /* the largest kv_lens[b] a step will see; sizes
                                the attention split; <= capacity - 1 */
    int32_t attn_chunks;     /* attention tiles per request, on average: each kv
                                head gets batch x attn_chunks tiles; 0 = auto;
                                at most 32, batch x attn_chunks at most 128
                                (else MK_EINVAL) */
    int32_t trace;           /* 1: record per-instruction device timestamps */
    int64_t watchdog_spins;  /* bound of every device wait loop; 0 = default */
    int32_t attn_split;      /* how a kv head's tiles are shared out over the
                                requests, on the device at every step, from
                                the current lengths: MK_SPLIT_BALANCED (0)
                                or MK_SPLIT_PER_REQUEST (1) */
    int32_t reserved1;       /* must be 0 */
} mk_schedule_desc;

/* Buffers of one step. All device pointers; the caller owns them. The new
 * K/V entry of request b is written at position kv_lens[b]. tokens_out may
 * alias tokens_in (every read of the tokens feeds the layer-0 activations,
 * which the LM head depends on) and kv_lens_out may alias kv_lens (the
 * resident grid writes them only after every workgroup has counted itself
 * started, which it does once it holds its copy of the lengths). */
typedef struct mk_step_io {
    const int32_t *tokens_in;   /* [B] (has_embed == 1) */
    const float *hidden_in;     /* [B, H] fp32 (has_embed == 0) */
    const int32_t *kv_lens;     /* [B], current lengths */
    void *k_pool;               /* bf16 [L, n_pages, nkv, page_tokens, d] */
    void *v_pool;               /* same shape */
    int32_t n_pages;            /* pages per layer in each pool */
    const int32_t *page_table;  /* [B, max_pages_per_req] page ids */
    int32_t *tokens_out;        /* [B] greedy tokens (has_embed == 1) */
    int32_t *kv_lens_out;       /* [B] = kv_lens + 1, or NULL */
    float *logits_out;          /* [B, V] fp32, or NULL */
    float *hidden_out;          /* [B, H] fp32 residual stream after the last layer, or NULL */
} mk_step_io;

typedef struct mk_handle mk_handle;

/* Binds a model to a device ("hand-written whole-model MegaKernel" section:
 * the one model-specific binding; weights live in HBM for the model
 * instance). Weights are BORROWED: the caller keeps them alive and
 * unchanged until mk_destroy. The handle owns its RoPE table, activation
 * scratch and counters. Errors: MK_EINVAL (null pointer, unsupported shape),
 * MK_EHIP (no device, allocation failure). *out is set only on MK_OK. */
int mk_create(const mk_config *cfg, const mk_weights *w, mk_handle **out);

/* Builds the tile DAG of a step for a batch size, validates it, linearises
 * it into one instruction queue per CU ([n_cus, Q, 32] int32, a subsequence
 * of one global topological order each) and uploads it ("principle,
 * schedule and dataflow" section: the host script that builds the DAG and
 * tensorises each SM's plan). Rebuilding replaces the previous schedule and
 * resets the counters. Errors: MK_EINVAL, MK_ECAPACITY (over capacity),
 * MK_ERESOURCE (not co-resident at one workgroup per CU), MK_EHIP. */
int mk_build_schedule(mk_handle *h, const mk_schedule_desc *s);

/* Runs one decode step on `stream` (a hipStream_t), asynchronously: no host
 * synchronisation ("principle, schedule and dataflow" section: the resident
 * grid and its interpreter loop). In MK_MODE_MEGAKERNEL this is one
 * cooperative launch of 256 (n_cus) workgroups. Errors: MK_ENOSCHED,
 * MK_EINVAL, MK_EHIP, and the sticky MK_ETIMEOUT / MK_EDEVICE raised by an
 * earlier step's device watchdog or error flag (seen once that step has
 * finished; mk_sync_status waits for it). After a sticky error the handle
 * needs mk_build_schedule before the next step. */
int mk_decode_step(mk_handle *h, const mk_step_io *io, void *stream);

/* Runs n_steps consecutive greedy decode steps in one launch whose grid stays
 * resident across them ("Inference MegaKernel", section "MPK compiler and
 * runtime": the kernel stays resident between tokens; here the step count is
 * fixed at the launch instead of a host shutdown flag). Step s embeds the
 * token step s - 1 chose and attends over kv_lens + s entries, exactly as
 * n_steps calls of mk_decode_step would; between steps no workgroup exits, so
 * the next step's first weights stream while the previous step's LM head
 * finishes. Needs MK_MODE_MEGAKERNEL and an embedding (has_embed == 1).
 * io as for mk_decode_step, except: tokens_in [B] holds step 0's tokens;
 * tokens_out is [n_steps][B] (step-major); kv_lens_out (optional) receives
 * kv_lens + n_steps; logits_out and hidden_out (optional) receive the last
 * step's values; every request's kv_lens + n_steps - 1 must be within the
 * schedule's max_kv_len. The first call with a larger n_steps * B than
 * before allocates a small device buffer (tagged tokens) and synchronises
 * `stream`. Errors: as mk_decode_step, and MK_EINVAL for n_steps < 1 or
 * above 2^20, a schedule in MK_MODE_UNFUSED, or a model without embedding.
 * A device-side range error (a length past the page capacity) is reported
 * like any other device error. */
int mk_decode_steps(mk_handle *h, const mk_step_io *io, int32_t n_steps, void *stream);

/* mk_decode_step for callers that cannot allocate device memory at the call
 * or around it (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). It runs the same resident interpreter, but the
 * step's exchange words and counters live in a file-scope device array of
 * MK_STATIC_SCRATCH_BYTES (64 MiB) per device, which the library sets up in
 * mk_create and holds until the process ends; the call itself allocates and
 * frees nothing. Every call on a device shares that array and keeps the last
 * call's contents: each call first clears the part its schedule uses (on
 * `stream`, with a fill kernel), so calls that overlap on one device race
 * and must be ordered by the caller (one stream, or events). The handle's
 * own exchange buffers and step tag are untouched, so the handle also stays
 * valid for mk_decode_step. Arguments, layouts and sticky errors as
 * mk_decode_step. Errors: MK_ENOSCHED; MK_EINVAL (also: the schedule is not
 * MK_MODE_MEGAKERNEL); MK_ECAPACITY when the schedule's exchange buffers
 * exceed MK_STATIC_SCRATCH_BYTES (the 16-layer 1B shape needs about 4.4 MB
 * at batch 1 and 35 MB at batch 8); MK_EHIP. */
#define MK_STATIC_SCRATCH_BYTES (64u << 20)
int mk_decode_step_static(mk_handle *h, const mk_step_io *io, void *stream);

/* Ends the lifetimes the object table of the "principle, schedule and
 * dataflow" section gives to what a binding owns: the queue and counters
 * (the resident kernel's and the dependency intervals' objects) and the
 * per-instance scratch. Waits for the handle's device work, then frees
 * everything the handle allocated; never touches borrowed buffers (weights,
 * K/V pools, step io). NULL is a no-op. No error is reported. */
void mk_destroy(mk_handle *h);

/* The text behind the last non-MK_OK status on the calling thread: the
 * capacity and resource obligations of the "unified framework" section are
 * checked before any launch and reported here with the quantity that failed,
 * and a device wait that hit its watchdog or a device-side range/NaN check
 * (the progress and visibility obligations) is reported with the failing
 * compute unit and instruction. Thread-local; valid until the next call on
 * the same thread; never NULL ("no error" before any failure). */
const char *mk_last_error(void);

/* Waits for the handle's device work on `stream` and returns the sticky
 * status (MK_OK, MK_ETIMEOUT or MK_EDEVICE) with the failing CU and
 * instruction in mk_last_error(). */
int mk_sync_status(mk_handle *h, void *stream);

/* Schedule facts for reports and tests. */
typedef struct mk_schedule_info {
    int32_t n_cus, queue_len, n_instr, n_events, n_counters;
    int32_t attn_chunks, prefetch_slices, lds_bytes, block_threads;
    int64_t stream_bytes_max_cu;   /* largest per-CU streamed byte count of a step at max_kv_len */
    int64_t stream_bytes_total;    /* streamed bytes of a step over all CUs at max_kv_len */
    int32_t launches_per_step;     /* 1 for the megakernel, kernel count for MK_MODE_UNFUSED */
} mk_schedule_info;

int mk_get_schedule_info(const mk_handle *h, mk_schedule_info *out);

/* Copies the trace of the last step (when built with trace = 1) into the
 * host buffer `out` of `cap` int64 values: for each CU and queue slot,
 * MK_TRACE_WORDS device-clock stamps (100 MHz): {start, inputs staged, end
 * (merges included), first wave done, last wave done, merge finisher elected,
 * merge inputs gathered, unused}; 0 where a stamp does not apply. Returns the
 * number of values written through *n. */
#define MK_TRACE_WORDS 8
int mk_read_trace(mk_handle *h, int64_t *out, size_t cap, size_t *n);

/* ---- debugging aids ---- */

/* Copies the last layer's activation `which` of the previous step (0:
 * residual stream x after the last layer [B, H], 1: qkv [B, (nq + 2 nkv) d],
 * 2: attention output o [B, nq d], 3: gated MLP activation [B, F]) as fp32
 * into the host buffer `out` of `bytes` bytes, after synchronising the
 * device. In MK_MODE_UNFUSED these are the baseline's scratch buffers; in
 * MK_MODE_MEGAKERNEL the value halves of the last layer's tagged exchange
 * words. Errors: MK_EINVAL, MK_ENOSCHED, MK_EHIP. */
int mk_debug_copy_scratch(mk_handle *h, int which, void *out, size_t bytes);

/* Plain device copy of `bytes` (a multiple of 16) from src_dev to dst_dev on
 * `stream` (a hipStream_t, NULL: the null stream), each byte read and written
 * once: the reference whose HBM traffic counters (FETCH_SIZE, WRITE_SIZE)
 * scale those measured for the decode kernels. Asynchronous. Errors:
 * MK_EINVAL (null pointer, size not a positive multiple of 16), MK_EHIP. */
int mk_debug_copy_probe(const void *src_dev, void *dst_dev, size_t bytes, void *stream);

/* Cross-XCD message-passing litmus: `pairs` writer/reader workgroup pairs
 * (co-resident, cooperative launch) run `rounds` rounds over `n_words` int32
 * words each (data_dev: pairs * n_words int32; flags_dev: pairs * 64 int32,
 * zeroed). The reader plants possibly stale copies with plain loads, waits
 * for the writer's flag and counts words that are not the round's value:
 * res_dev[0] with plain loads, res_dev[1] with device-coherent loads;
 * res_dev[2] counts watchdog expiries (device int32[4], zeroed).
 * mode 0: plain stores, agent-scope release fence before the flag and
 * acquire fence after it. mode 1: device-coherent stores, completion wait
 * before the flag, no fences (the protocol of the resident interpreter, in
 * which only the device-coherent count must be zero). Synchronous. Errors:
 * MK_EINVAL, MK_EHIP. */
int mk_debug_litmus(int pairs, int n_words, int rounds, int mode, int32_t *data_dev, int32_t *flags_dev,
                    int32_t *res_dev);

/* The attention split (mk_attn_split) as the device computes it, for
 * n_cases batches of `batch` requests: kv_lens_dev [n_cases][batch] int32
 * (each clamped to 0..capacity - 1, as a step does); `tiles` per kv head
 * (batch <= tiles <= 128, a multiple of batch for MK_SPLIT_PER_REQUEST);
 * out_dev [n_cases][4 tiles + batch + 1] int32: per tile its request, first
 * block, end block and 1 on a request's last tile, then the first tile of
 * each request and `tiles`. One wave per case; synchronous. Errors:
 * MK_EINVAL, MK_EHIP. */
int mk_debug_attn_split(const int32_t *kv_lens_dev, int n_cases, int batch, int tiles, int mode, int capacity,
                        int32_t *out_dev);

/* Dependency-hop latency: a cooperative grid of n_cus one-wave workgroups
 * runs `rounds` grid-wide hops (wait for every workgroup's previous round,
 * optionally acquire, optionally exchange 8 floats per workgroup, optionally
 * release, signal). ctr_dev: ctr_words int32, zeroed by the caller, at least
 * max((rounds + 1) * 32, (17 + ceil(n_cus / 16)) * 1024); xbuf_dev:
 * xbuf_floats floats, at least 2 * ceil(n_cus / 4) * 1024; res_dev: 2 int32
 * (res[0] counts watchdog expiries). variant bits: 0 no release fence, 1 no
 * acquire fence, 2 exchange the floats, 3 tree of 16-way counters with
 * replicated release flags instead of one shared counter, 4 spread the
 * exchanged vector one 128-byte line per 4 KiB, 5 plain loads and stores for
 * the exchange instead of device-coherent ones. Asynchronous on the null
 * stream. */
int mk_debug_hop_probe(int32_t *ctr_dev, size_t ctr_words, float *xbuf_dev, size_t xbuf_floats, int n_cus,
                       int rounds, int variant, int32_t *res_dev);
/* Epoch-tagged exchange latency: a cooperative grid of n_cus one-wave
 * workgroups runs `rounds` rounds; in each, every workgroup writes `per`
 * 64-bit (value, round) words into each of `copies` (1..16) copies of the
 * exchange vector and then reads all n_cus * per words of copy
 * (workgroup % copies) until each carries the round. buf_dev: buf_words
 * uint64, at least 2 * copies * n_cus * per, zeroed by the caller; res_dev:
 * 2 int32 (res[0] counts watchdog expiries). Asynchronous on the null
 * stream. */
int mk_debug_ll_probe(uint64_t *buf_dev, size_t buf_words, int n_cus, int per, int copies, int rounds,
                      int32_t *res_dev);
/* Read bandwidth of `blocks` workgroups of `threads` threads streaming the
 * first floor(bytes / 4096) 4 KiB slices of src through registers with
 * `depth` (1..6) slices in flight per wave. out_dev: one uint32 sink.
 * Asynchronous on the null stream. */
int mk_debug_regstream_probe(const void *src, size_t bytes, int blocks, int threads, int depth, void *out_dev);

/* ---- host-only planning (no HIP call; usable without a GPU) ---- */

typedef struct mk_plan mk_plan;

/* Builds the same schedule mk_build_schedule would, on the host only.
 * `s->n_cus` must be given (non-zero). Errors as mk_build_schedule. */
int mk_plan_create(const mk_config *cfg, const mk_schedule_desc *s, mk_plan **out);
void mk_plan_destroy(mk_plan *p);
int mk_plan_info(const mk_plan *p, mk_schedule_info *out);
/* Copies the encoded queues [n_cus, Q, 32] int32 into `out` (cap int32s). */
int mk_plan_queue(const mk_plan *p, int32_t *out, size_t cap);
/* Copies the event table [n_events, 16] int32 into `out`. */
int mk_plan_events(const mk_plan *p, int32_t *out, size_t cap);

#ifdef __cplusplus
}
#endif
#endif /* MK_H */
