#include <algorithm>
// mk_api.cpp - the C ABI (include/mk.h): model binding, schedule upload,
// step launch, sticky device errors.
//
// "Inference MegaKernel" (shaojiemike.top), section "hand-written
// whole-model MegaKernel / principle, schedule and dataflow": one
// model-specific binding passes weights, K/V cache, activations and counters
// to the resident run as objects; its object table fixes their lifetimes
// (weights per model instance, K/V per request, queue and counters per
// kernel). The "unified framework" section's capacity and resource
// obligations are checked here before any launch.
#include <hip/hip_runtime.h>

#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "mk.h"
#include "mk_isa.h"
#include "mk_kernels.h"
#include "mk_sched.h"

namespace mk {

namespace {
thread_local std::string g_last_error = "no error";
}

int set_error(int code, const std::string &msg) {
    g_last_error = msg;
    return code;
}

}  // namespace mk

using mk::set_error;

#define MK_HIP(call)                                                                                \
    do {                                                                                            \
        hipError_t e_ = (call);                                                                     \
        if (e_ != hipSuccess)                                                                       \
            return set_error(MK_EHIP, std::string(#call) + " failed: " + hipGetErrorString(e_)); \
    } while (0)

struct mk_handle {
    mk_config cfg{};
    int n_cus_dev = 0;
    uint64_t *wtab = nullptr;
    std::vector<uint64_t> wtab_host;  // [L, 8] device addresses of the layer weights
    const void *embed = nullptr, *final_norm = nullptr;
    float2 *rope = nullptr;
    int capacity = 0;
    int32_t *err = nullptr;
    int32_t *host_err = nullptr;      // pinned, mapped
    int32_t *host_err_dev = nullptr;  // device view of host_err
    // schedule
    bool built = false;
    mk::Plan plan;
    int32_t *queue = nullptr, *events = nullptr, *counters = nullptr;
    float *x = nullptr, *qkv = nullptr, *o = nullptr, *act = nullptr, *attn_part = nullptr, *lm_part = nullptr;
    float *u = nullptr, *qrot = nullptr;
    uint64_t *tx = nullptr, *tqkv = nullptr, *to = nullptr, *tact = nullptr, *tpart = nullptr, *tlm = nullptr;
    uint32_t tag = 0;  // tag of the last step's activations (never 0 on the device)
    uint64_t *ttok = nullptr;  // [ttok_cap] tagged tokens a resident launch hands from step to step
    size_t ttok_cap = 0;
    int64_t *trace = nullptr;
    int64_t epoch = 0;  // launches since the counters were last cleared (start counter)
    int64_t steps = 0;  // decode steps since then (merge events)
    int32_t max_need = 1;
    int sticky = MK_OK;
};

namespace {

template <typename T>
void dfree(T *&p) {
    if (p) (void)hipFree((void *)p);
    p = nullptr;
}

void free_schedule(mk_handle *h) {
    dfree(h->queue);
    dfree(h->events);
    dfree(h->counters);
    dfree(h->x);
    dfree(h->qkv);
    dfree(h->o);
    dfree(h->act);
    dfree(h->attn_part);
    dfree(h->lm_part);
    dfree(h->u);
    dfree(h->qrot);
    dfree(h->tx);
    dfree(h->tqkv);
    dfree(h->to);
    dfree(h->tact);
    dfree(h->tpart);
    dfree(h->tlm);
    dfree(h->ttok);
    h->ttok_cap = 0;
    dfree(h->trace);
    h->built = false;
}

template <typename T>
int dalloc(T *&p, size_t count) {
    void *v = nullptr;
    hipError_t e = hipMalloc(&v, count * sizeof(T) + 256);
    if (e != hipSuccess) return set_error(MK_EHIP, std::string("hipMalloc failed: ") + hipGetErrorString(e));
    e = hipMemset(v, 0, count * sizeof(T) + 256);
    if (e != hipSuccess) return set_error(MK_EHIP, std::string("hipMemset failed: ") + hipGetErrorString(e));
    p = (T *)v;
    return MK_OK;
}

int decode_err(int32_t v) {
    const int code = (v >> 28) & 0xf;
    const int cu = (v >> 16) & 0xfff, pc = v & 0xffff;
    const char *what = code == mk::ERR_TIMEOUT ? "watchdog timeout"
                       : code == mk::ERR_OPCODE ? "invalid opcode"
                       : code == mk::ERR_RANGE ? "token, length or page id out of range"
                       : code == mk::ERR_NAN ? "NaN logit"
                                             : "device error";
    const int rc = code == mk::ERR_TIMEOUT ? MK_ETIMEOUT : MK_EDEVICE;
    return set_error(rc, std::string("device reported ") + what + " (cu " + std::to_string(cu) + ", instruction " +
                             std::to_string(pc) + "); rebuild the schedule");
}

}  // namespace

// Writes each instruction's operand addresses (weight matrices, norm
// weight) into its words, so that the interpreter reads them with the
// instruction instead of chasing the weight table.
static void bind_operands(const mk_handle *h, mk::Plan &plan) {
    auto put64 = [](int32_t *w, int at, uint64_t v) {
        w[at] = (int32_t)(uint32_t)v;
        w[at + 1] = (int32_t)(uint32_t)(v >> 32);
    };
    for (size_t i = 0; i + mk::INSTR_WORDS <= plan.queue.size(); i += mk::INSTR_WORDS) {
        int32_t *w = &plan.queue[i];
        const int op = w[mk::W_OP], l = w[mk::W_LAYER];
        uint64_t wa = 0, wb = 0, wn = 0;
        auto tab = [&](int k) { return h->wtab_host[(size_t)l * 8 + k]; };
        switch (op) {
            case mk::OP_QKV: wa = tab(1); wn = tab(0); break;
            case mk::OP_OPROJ: wa = tab(2); break;
            case mk::OP_UPGATE: wa = tab(4); wb = tab(5); wn = tab(3); break;
            case mk::OP_DOWN: wa = tab(6); break;
            case mk::OP_LMHEAD:
                wa = (uint64_t)(uintptr_t)h->embed;
                wn = (uint64_t)(uintptr_t)h->final_norm;
                break;
            default: break;
        }
        if (op != mk::OP_UPGATE) wb = wa;
        put64(w, mk::W_WA, wa);
        put64(w, mk::W_WB, wb);
        put64(w, mk::W_WN, wn);
    }
}

// Where mk_decode_step_static puts a schedule's exchange words and counters
// inside the device's static scratch: the same buffers mk_build_schedule
// allocates for the resident interpreter, each 256-byte aligned.
struct StaticLayout {
    char *base;
    size_t bytes;  // used, from base
    uint64_t *tx, *tqkv, *to, *tact, *tpart, *tlm;
    int32_t *counters;
};

static int static_layout(const mk_handle *h, char *base, StaticLayout *sl) {
    const mk_config &c = h->cfg;
    const mk::Plan &P = h->plan;
    const size_t B = (size_t)P.desc.batch, L = (size_t)c.n_layers, G = (size_t)(c.n_q_heads / c.n_kv_heads);
    const size_t QKV = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, QD = (size_t)c.n_q_heads * c.head_dim;
    size_t off = 0;
    auto take = [&](size_t bytes) {
        char *p = base + off;
        off += (bytes + 255) / 256 * 256;
        return p;
    };
    sl->base = base;
    sl->tx = (uint64_t *)take(2 * L * B * c.hidden * 8);
    sl->tqkv = (uint64_t *)take(L * B * QKV * 8);
    sl->to = (uint64_t *)take(L * B * QD * 8);
    sl->tact = (uint64_t *)take(L * B * c.ffn * 8);
    sl->tpart = (uint64_t *)take(L * B * c.n_kv_heads * P.attn_chunks * G * mk::ATTN_PART * 8);
    sl->tlm = (uint64_t *)take((size_t)std::max(P.n_lm_slots, 1) * B * 2 * 8);
    sl->counters = (int32_t *)take((size_t)(P.n_counters + 1) * mk::CTR_STRIDE * 4);
    sl->bytes = off;
    if (off > mk::STATIC_SCRATCH_BYTES)
        return set_error(MK_ECAPACITY, "this schedule's exchange buffers need " + std::to_string(off) +
                                           " bytes; the static scratch holds " +
                                           std::to_string(mk::STATIC_SCRATCH_BYTES));
    return MK_OK;
}

extern "C" {

const char *mk_last_error(void) { return mk::g_last_error.c_str(); }

int mk_create(const mk_config *cfg, const mk_weights *w, mk_handle **out) {
    try {
        if (!cfg || !w || !out) return set_error(MK_EINVAL, "null argument");
        if (int rc = mk::check_config(*cfg)) return rc;
        if (!w->layers) return set_error(MK_EINVAL, "weights.layers is null");
        if (cfg->has_embed && (!w->embed || !w->final_norm))
            return set_error(MK_EINVAL, "embed and final_norm are required with has_embed = 1");
        for (int l = 0; l < cfg->n_layers; ++l) {
            const mk_layer_weights &lw = w->layers[l];
            if (!lw.attn_norm || !lw.wqkv || !lw.wo || !lw.mlp_norm || !lw.w_gate || !lw.w_up || !lw.w_down)
                return set_error(MK_EINVAL, "null weight pointer in layer " + std::to_string(l));
        }
        int ndev = 0;
        MK_HIP(hipGetDeviceCount(&ndev));
        if (cfg->device < 0 || cfg->device >= ndev) return set_error(MK_EINVAL, "device ordinal out of range");
        MK_HIP(hipSetDevice(cfg->device));
        hipDeviceProp_t prop;
        MK_HIP(hipGetDeviceProperties(&prop, cfg->device));
        if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0)
            return set_error(MK_EINVAL, std::string("built for gfx950, device is ") + prop.gcnArchName);
        // the device's static scratch (mk_decode_step_static): its address,
        // looked up once per device with the device current
        MK_HIP(mk::static_scratch_setup(cfg->device));

        mk_handle *h = new (std::nothrow) mk_handle();
        if (!h) return set_error(MK_EINVAL, "out of host memory");
        h->cfg = *cfg;
        h->n_cus_dev = prop.multiProcessorCount;
        h->embed = w->embed;
        h->final_norm = w->final_norm;
        auto fail = [&](int rc) {
            mk_destroy(h);
            return rc;
        };
        std::vector<uint64_t> tab((size_t)cfg->n_layers * 8, 0);
        for (int l = 0; l < cfg->n_layers; ++l) {
            const mk_layer_weights &lw = w->layers[l];
            const void *ptrs[7] = {lw.attn_norm, lw.wqkv, lw.wo, lw.mlp_norm, lw.w_gate, lw.w_up, lw.w_down};
            for (int k = 0; k < 7; ++k) tab[(size_t)l * 8 + k] = (uint64_t)(uintptr_t)ptrs[k];
        }
        h->wtab_host = tab;
        if (int rc = dalloc(h->wtab, tab.size())) return fail(rc);
        if (hipMemcpy(h->wtab, tab.data(), tab.size() * 8, hipMemcpyHostToDevice) != hipSuccess)
            return fail(set_error(MK_EHIP, "hipMemcpy of the weight table failed"));
        h->capacity = cfg->max_pages_per_req * cfg->page_tokens;
        if (int rc = dalloc(h->rope, (size_t)h->capacity * (cfg->head_dim / 2))) return fail(rc);
        if (mk::launch_rope_table(h->rope, h->capacity, cfg->head_dim, (double)cfg->rope_theta, nullptr) !=
            hipSuccess)
            return fail(set_error(MK_EHIP, "RoPE table kernel failed to launch"));
        if (int rc = dalloc(h->err, 1)) return fail(rc);
        if (hipHostMalloc((void **)&h->host_err, 64, hipHostMallocMapped) != hipSuccess)
            return fail(set_error(MK_EHIP, "hipHostMalloc failed"));
        *h->host_err = 0;
        if (hipHostGetDevicePointer((void **)&h->host_err_dev, h->host_err, 0) != hipSuccess)
            return fail(set_error(MK_EHIP, "hipHostGetDevicePointer failed"));
        if (hipDeviceSynchronize() != hipSuccess) return fail(set_error(MK_EHIP, "device synchronisation failed"));
        *out = h;
        return MK_OK;
    } catch (...) {
        return set_error(MK_EINVAL, "internal error in mk_create");
    }
}

int mk_build_schedule(mk_handle *h, const mk_schedule_desc *s) {
    try {
        if (!h || !s) return set_error(MK_EINVAL, "null argument");
        MK_HIP(hipSetDevice(h->cfg.device));
        mk_schedule_desc d = *s;
        if (d.n_cus == 0) d.n_cus = h->n_cus_dev;
        if (d.n_cus < 0) return set_error(MK_EINVAL, "n_cus must be >= 0");
        if (d.watchdog_spins <= 0) d.watchdog_spins = (int64_t)1 << 22;
        mk::Plan plan;
        if (int rc = mk::build_plan(h->cfg, d, plan)) return rc;
        const int G = h->cfg.n_q_heads / h->cfg.n_kv_heads;
        if (d.mode == MK_MODE_MEGAKERNEL) {
            if (!mk::megakernel_supports(d.batch, G))
                return set_error(MK_EINVAL, "no resident interpreter for this batch and head grouping");
            MK_HIP(mk::setup_megakernel(d.batch, G, plan.lds_bytes));
            int per_cu = 0;
            MK_HIP(mk::megakernel_occupancy(d.batch, G, plan.lds_bytes, &per_cu));
            if (per_cu < 1 || d.n_cus > h->n_cus_dev * per_cu)
                return set_error(MK_ERESOURCE, "resident grid of " + std::to_string(d.n_cus) +
                                                   " workgroups is not co-resident (" + std::to_string(per_cu) +
                                                   " per CU, " + std::to_string(h->n_cus_dev) + " CUs)");
        }
        MK_HIP(hipDeviceSynchronize());
        free_schedule(h);
        h->plan = plan;
        const mk_config &c = h->cfg;
        const int B = d.batch;
        const size_t QKV = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, QD = (size_t)c.n_q_heads * c.head_dim;
        const size_t kmax = std::max<size_t>(c.hidden, std::max<size_t>(c.ffn, QD));
        const size_t lm_slots =
            c.has_embed ? std::max<size_t>((size_t)plan.n_lm_slots, (size_t)(c.vocab + 3) / 4) : 1;
        int rc = MK_OK;
        if (!rc) rc = dalloc(h->queue, std::max<size_t>(plan.queue.size(), 32));
        if (!rc) rc = dalloc(h->events, std::max<size_t>(plan.events.size(), 16));
        // the merge events' counters, then the start counter
        if (!rc) rc = dalloc(h->counters, (size_t)(plan.n_counters + 1) * mk::CTR_STRIDE);
        if (d.mode == MK_MODE_UNFUSED) {  // the baseline's scratch, overwritten in place by its kernels
            if (!rc) rc = dalloc(h->x, (size_t)B * c.hidden);
            if (!rc) rc = dalloc(h->qkv, (size_t)B * QKV);
            if (!rc) rc = dalloc(h->o, (size_t)B * QD);
            if (!rc) rc = dalloc(h->act, (size_t)B * c.ffn);
            if (!rc)
                rc = dalloc(h->attn_part, (size_t)B * c.n_kv_heads * plan.attn_chunks * G * mk::ATTN_PART_STRIDE);
            if (!rc) rc = dalloc(h->lm_part, lm_slots * B * 2);
            if (!rc) rc = dalloc(h->u, (size_t)B * kmax);
            if (!rc) rc = dalloc(h->qrot, (size_t)B * QD);
        } else {  // tagged activations, each written once per step
            const size_t L = (size_t)c.n_layers;
            if (!rc) rc = dalloc(h->tx, 2 * L * B * c.hidden);
            if (!rc) rc = dalloc(h->tqkv, L * B * QKV);
            if (!rc) rc = dalloc(h->to, L * B * QD);
            if (!rc) rc = dalloc(h->tact, L * B * c.ffn);
            if (!rc) rc = dalloc(h->tpart, L * B * c.n_kv_heads * plan.attn_chunks * G * mk::ATTN_PART);
            if (!rc) rc = dalloc(h->tlm, (size_t)std::max(plan.n_lm_slots, 1) * B * 2);
        }
        if (!rc && d.trace) rc = dalloc(h->trace, (size_t)plan.n_cus * plan.Q * MK_TRACE_WORDS);
        if (rc) {
            free_schedule(h);
            return rc;
        }
        bind_operands(h, h->plan);
        if (!h->plan.queue.empty())
            MK_HIP(hipMemcpy(h->queue, h->plan.queue.data(), h->plan.queue.size() * 4, hipMemcpyHostToDevice));
        if (!plan.events.empty())
            MK_HIP(hipMemcpy(h->events, plan.events.data(), plan.events.size() * 4, hipMemcpyHostToDevice));
        h->max_need = std::max(1, plan.n_cus);  // the start counter counts every workgroup
        for (int e = 0; e < plan.n_events; ++e)
            h->max_need = std::max(h->max_need, plan.events[(size_t)e * mk::EV_WORDS + mk::EV_NEED]);
        MK_HIP(hipMemset(h->err, 0, 4));
        *h->host_err = 0;
        h->sticky = MK_OK;
        h->epoch = 0;
        h->steps = 0;
        h->tag = 0;
        MK_HIP(hipDeviceSynchronize());
        h->built = true;
        return MK_OK;
    } catch (...) {
        return set_error(MK_EINVAL, "internal error in mk_build_schedule");
    }
}

static int decode_step(mk_handle *h, const mk_step_io *io, void *stream, const StaticLayout *sl, int n_steps) {
    try {
        if (!h || !io) return set_error(MK_EINVAL, "null argument");
        if (!h->built) return set_error(MK_ENOSCHED, "mk_decode_step before mk_build_schedule");
        if (h->sticky != MK_OK) return set_error(h->sticky, "a previous step failed; rebuild the schedule");
        const int32_t herr = __atomic_load_n(h->host_err, __ATOMIC_ACQUIRE);
        if (herr != 0) {
            h->sticky = decode_err(herr);
            return h->sticky;
        }
        const mk_config &c = h->cfg;
        if (!io->kv_lens || !io->k_pool || !io->v_pool || !io->page_table)
            return set_error(MK_EINVAL, "kv_lens, k_pool, v_pool and page_table are required");
        if (c.has_embed && (!io->tokens_in || !io->tokens_out))
            return set_error(MK_EINVAL, "tokens_in and tokens_out are required with an embedding");
        if (!c.has_embed && !io->hidden_in) return set_error(MK_EINVAL, "hidden_in is required without an embedding");
        if (io->n_pages < 1) return set_error(MK_EINVAL, "n_pages must be positive");
        hipStream_t st = (hipStream_t)stream;
        const mk::Plan &P = h->plan;
        if (n_steps < 1) return set_error(MK_EINVAL, "n_steps must be positive");
        if (n_steps > 1) {
            if (P.desc.mode != MK_MODE_MEGAKERNEL)
                return set_error(MK_EINVAL, "several steps per launch need the resident interpreter (MK_MODE_MEGAKERNEL)");
            if (!c.has_embed) return set_error(MK_EINVAL, "several steps per launch need an embedding (greedy tokens feed back)");
            if (n_steps > (1 << 20)) return set_error(MK_EINVAL, "n_steps above 2^20");
            const size_t need = (size_t)n_steps * P.desc.batch;
            if (need > h->ttok_cap) {
                MK_HIP(hipStreamSynchronize(st));
                dfree(h->ttok);
                h->ttok_cap = 0;
                if (int rc = dalloc(h->ttok, need)) return rc;
                h->ttok_cap = need;
            }
        }
        mk::KParams k{};
        k.n_steps = n_steps;
        k.ttok = n_steps > 1 ? h->ttok : nullptr;
        if (sl) {
            // the static scratch keeps whatever the last call on this device
            // left there: clear the part this schedule uses (a fill kernel,
            // which a captured graph replays correctly), then run as the first
            // step on cleared buffers
            MK_HIP(mk::fill_u32((uint32_t *)sl->base, sl->bytes / 4, 0u, st));
            k.epoch = 1;
            k.step_epoch = 1;
            k.tag = 1;
        } else {
            // epoch-based counters (one start-counter epoch per launch, one
            // merge epoch per step): re-zero before the int32 counts could wrap
            if ((h->steps + n_steps) * (int64_t)h->max_need >= ((int64_t)1 << 30)) {
                MK_HIP(mk::fill_u32((uint32_t *)h->counters, (size_t)(P.n_counters + 1) * mk::CTR_STRIDE, 0u, st));
                h->epoch = 0;
                h->steps = 0;
            }
            h->epoch++;
            k.epoch = (int32_t)h->epoch;
            k.step_epoch = (int32_t)(h->steps + 1);
            h->steps += n_steps;
            // step s of the launch tags its activations tag + s; tags only
            // grow, so no word left by an earlier launch carries one of them
            // (the buffers start at tag 0, which no step uses)
            if ((uint64_t)h->tag + (uint64_t)n_steps > 0xffffffffull)
                return set_error(MK_EINVAL, "activation tags exhausted; rebuild the schedule");
            k.tag = h->tag + 1;
            h->tag += (uint32_t)n_steps;
        }
        k.queue = h->queue;
        k.events = h->events;
        k.counters = sl ? sl->counters : h->counters;
        k.start_ctr = P.n_counters;
        k.Q = P.Q;
        k.n_cus = P.n_cus;
        k.queue_off = P.queue_off;
        k.xrow_off = P.xrow_off;
        k.act_off = P.act_off;
        k.nw_off = P.nw_off;
        k.act_stride = P.act_stride;
        k.xrow_stride = P.xrow_stride;
        k.watchdog = P.desc.watchdog_spins;
        k.L = c.n_layers;
        k.H = c.hidden;
        k.nq = c.n_q_heads;
        k.nkv = c.n_kv_heads;
        k.d = c.head_dim;
        k.F = c.ffn;
        k.V = c.vocab;
        k.has_embed = c.has_embed;
        k.B = P.desc.batch;
        k.T = c.page_tokens;
        k.max_pages = c.max_pages_per_req;
        k.eps = c.rms_eps;
        k.embed = (const uint16_t *)h->embed;
        k.final_norm = (const uint16_t *)h->final_norm;
        k.wtab = h->wtab;
        k.rope = h->rope;
        k.tokens_in = io->tokens_in;
        k.hidden_in = io->hidden_in;
        k.kv_lens = io->kv_lens;
        k.k_pool = (uint16_t *)io->k_pool;
        k.v_pool = (uint16_t *)io->v_pool;
        k.n_pages = io->n_pages;
        k.page_table = io->page_table;
        k.tokens_out = io->tokens_out;
        k.kv_lens_out = io->kv_lens_out;
        k.logits_out = io->logits_out;
        k.hidden_out = io->hidden_out;
        k.x = h->x;
        k.qkv = h->qkv;
        k.o = h->o;
        k.act = h->act;
        k.attn_part = h->attn_part;
        k.lm_part = h->lm_part;
        k.tx = sl ? sl->tx : h->tx;
        k.tqkv = sl ? sl->tqkv : h->tqkv;
        k.to = sl ? sl->to : h->to;
        k.tact = sl ? sl->tact : h->tact;
        k.tpart = sl ? sl->tpart : h->tpart;
        k.tlm = sl ? sl->tlm : h->tlm;
        k.attn_chunks = P.attn_chunks;
        k.attn_split = P.desc.attn_split;
        k.err = h->err;
        k.host_err = h->host_err_dev;
        k.trace = h->trace;
        hipError_t e;
        if (P.desc.mode == MK_MODE_MEGAKERNEL) {
            e = mk::launch_megakernel(k, P.lds_bytes, st);
        } else {
            e = mk::launch_unfused(k, h->u, h->qrot, st);
        }
        if (e != hipSuccess) return set_error(MK_EHIP, std::string("launch failed: ") + hipGetErrorString(e));
        return MK_OK;
    } catch (...) {
        return set_error(MK_EINVAL, "internal error in a decode step");
    }
}

int mk_decode_step(mk_handle *h, const mk_step_io *io, void *stream) { return decode_step(h, io, stream, nullptr, 1); }

int mk_decode_steps(mk_handle *h, const mk_step_io *io, int32_t n_steps, void *stream) {
    return decode_step(h, io, stream, nullptr, n_steps);
}

int mk_decode_step_static(mk_handle *h, const mk_step_io *io, void *stream) {
    try {
        if (!h || !io) return set_error(MK_EINVAL, "null argument");
        if (!h->built) return set_error(MK_ENOSCHED, "mk_decode_step_static before mk_build_schedule");
        if (h->plan.desc.mode != MK_MODE_MEGAKERNEL)
            return set_error(MK_EINVAL, "mk_decode_step_static runs the resident interpreter: build the schedule "
                                        "in MK_MODE_MEGAKERNEL");
        void *base = mk::static_scratch(h->cfg.device);
        if (!base) return set_error(MK_EHIP, "the static scratch of this device was not set up by mk_create");
        StaticLayout sl{};
        if (int rc = static_layout(h, (char *)base, &sl)) return rc;
        return decode_step(h, io, stream, &sl, 1);
    } catch (...) {
        return set_error(MK_EINVAL, "internal error in mk_decode_step_static");
    }
}

int mk_sync_status(mk_handle *h, void *stream) {
    if (!h) return set_error(MK_EINVAL, "null argument");
    MK_HIP(hipSetDevice(h->cfg.device));
    MK_HIP(hipStreamSynchronize((hipStream_t)stream));
    int32_t v = 0;
    MK_HIP(hipMemcpy(&v, h->err, 4, hipMemcpyDeviceToHost));
    if (v != 0) {
        h->sticky = decode_err(v);
        return h->sticky;
    }
    if (h->sticky != MK_OK) return set_error(h->sticky, "a previous step failed; rebuild the schedule");
    return MK_OK;
}

void mk_destroy(mk_handle *h) {
    if (!h) return;
    (void)hipSetDevice(h->cfg.device);
    (void)hipDeviceSynchronize();
    free_schedule(h);
    dfree(h->wtab);
    dfree(h->rope);
    dfree(h->err);
    if (h->host_err) (void)hipHostFree(h->host_err);
    delete h;
}

int mk_get_schedule_info(const mk_handle *h, mk_schedule_info *out) {
    if (!h || !out) return set_error(MK_EINVAL, "null argument");
    if (!h->built) return set_error(MK_ENOSCHED, "no schedule");
    const mk::Plan &P = h->plan;
    std::memset(out, 0, sizeof *out);
    out->n_cus = P.n_cus;
    out->queue_len = P.Q;
    out->n_instr = P.n_instr;
    out->n_events = P.n_events;
    out->n_counters = P.n_counters;
    out->attn_chunks = P.attn_chunks;
    out->prefetch_slices = mk::PREFETCH_SLICES;
    out->lds_bytes = P.lds_bytes;
    out->block_threads = mk::BLOCK_THREADS;
    out->stream_bytes_max_cu = P.stream_max_cu;
    out->stream_bytes_total = P.stream_total;
    out->launches_per_step = P.launches;
    return MK_OK;
}

int mk_debug_copy_scratch(mk_handle *h, int which, void *out, size_t bytes) {
    if (!h || !out) return set_error(MK_EINVAL, "null argument");
    if (!h->built) return set_error(MK_ENOSCHED, "no schedule");
    const mk_config &c = h->cfg;
    const size_t B = (size_t)h->plan.desc.batch, L = (size_t)c.n_layers;
    const size_t QKV = (size_t)(c.n_q_heads + 2 * c.n_kv_heads) * c.head_dim, QD = (size_t)c.n_q_heads * c.head_dim;
    const bool mega = h->plan.desc.mode == MK_MODE_MEGAKERNEL;
    size_t n = 0;
    const void *src = nullptr;
    switch (which) {
        case 0: n = B * c.hidden; src = mega ? (const void *)(h->tx + (2 * L - 1) * n) : h->x; break;
        case 1: n = B * QKV; src = mega ? (const void *)(h->tqkv + (L - 1) * n) : h->qkv; break;
        case 2: n = B * QD; src = mega ? (const void *)(h->to + (L - 1) * n) : h->o; break;
        case 3: n = B * c.ffn; src = mega ? (const void *)(h->tact + (L - 1) * n) : h->act; break;
        default: return set_error(MK_EINVAL, "unknown scratch buffer");
    }
    if (bytes < n * 4) return set_error(MK_EINVAL, "buffer too small");
    MK_HIP(hipSetDevice(c.device));
    MK_HIP(hipDeviceSynchronize());
    if (!mega) {
        MK_HIP(hipMemcpy(out, src, n * 4, hipMemcpyDeviceToHost));
        return MK_OK;
    }
    // tagged words: fp32 bits in the low half, the step tag in the high half
    std::vector<uint64_t> words(n);
    MK_HIP(hipMemcpy(words.data(), src, n * 8, hipMemcpyDeviceToHost));
    uint32_t *o32 = (uint32_t *)out;
    for (size_t i = 0; i < n; ++i) o32[i] = (uint32_t)words[i];
    return MK_OK;
}

int mk_debug_copy_probe(const void *src_dev, void *dst_dev, size_t bytes, void *stream) {
    if (!src_dev || !dst_dev || bytes < 16 || bytes % 16) return set_error(MK_EINVAL, "bad copy arguments");
    MK_HIP(mk::copy_probe(src_dev, dst_dev, bytes, (hipStream_t)stream));
    return MK_OK;
}

int mk_debug_litmus(int pairs, int n_words, int rounds, int mode, int32_t *data_dev, int32_t *flags_dev,
                    int32_t *res_dev) {
    if (pairs < 1 || pairs > 128 || n_words < 1 || rounds < 1 || mode < 0 || mode > 1 || !data_dev || !flags_dev ||
        !res_dev)
        return set_error(MK_EINVAL, "bad litmus arguments");
    MK_HIP(mk::litmus(pairs, n_words, rounds, mode, data_dev, flags_dev, res_dev));
    return MK_OK;
}

int mk_debug_attn_split(const int32_t *kv_lens_dev, int n_cases, int batch, int tiles, int mode, int capacity,
                        int32_t *out_dev) {
    if (!kv_lens_dev || !out_dev || n_cases < 1 || n_cases > 65535 || batch < 1 || batch > mk::MAX_B ||
        tiles < batch || tiles > mk::MAX_ATTN_TILES || capacity < 1 || capacity > 65535 * 16 ||
        (mode != mk::SPLIT_BALANCED && mode != mk::SPLIT_PER_REQUEST) ||
        (mode == mk::SPLIT_PER_REQUEST && tiles % batch != 0))
        return set_error(MK_EINVAL, "bad attention split arguments");
    MK_HIP(mk::split_probe(kv_lens_dev, n_cases, batch, tiles, mode, capacity, out_dev));
    return MK_OK;
}

int mk_debug_hop_probe(int32_t *ctr_dev, size_t ctr_words, float *xbuf_dev, size_t xbuf_floats, int n_cus,
                       int rounds, int variant, int32_t *res_dev) {
    if (!ctr_dev || !xbuf_dev || !res_dev || n_cus < 1 || n_cus > 1024 || rounds < 1 || rounds > 100000 ||
        variant < 0 || variant > 63)
        return set_error(MK_EINVAL, "bad probe arguments");
    const size_t groups = (size_t)(n_cus + 15) / 16;
    const size_t need_ctr = std::max((size_t)(rounds + 1) * 32, (1 + groups + 16) * 1024);
    const size_t need_x = 2 * (((size_t)n_cus * 8 + 31) / 32) * 1024;
    if (ctr_words < need_ctr || xbuf_floats < need_x) return set_error(MK_EINVAL, "probe buffers too small");
    MK_HIP(mk::hop_probe(ctr_dev, xbuf_dev, n_cus, rounds, variant, res_dev));
    return MK_OK;
}

int mk_debug_ll_probe(uint64_t *buf_dev, size_t buf_words, int n_cus, int per, int copies, int rounds,
                      int32_t *res_dev) {
    if (!buf_dev || !res_dev || n_cus < 1 || n_cus > 1024 || per < 1 || per > 4096 || copies < 1 || copies > 16 ||
        rounds < 1 || rounds > 100000 || (size_t)n_cus * per * copies * 8 >= ((size_t)1 << 31))
        return set_error(MK_EINVAL, "bad probe arguments");
    if (buf_words < 2 * (size_t)n_cus * per * copies) return set_error(MK_EINVAL, "probe buffer too small");
    MK_HIP(mk::ll_probe(buf_dev, n_cus, per, copies, rounds, res_dev));
    return MK_OK;
}

int mk_debug_regstream_probe(const void *src, size_t bytes, int blocks, int threads, int depth, void *out_dev) {
    if (!src || !out_dev || blocks < 1 || bytes < 4096 || threads < 64 || threads > mk::BLOCK_THREADS ||
        threads % 64 != 0 || depth < 1 || depth > 6)
        return set_error(MK_EINVAL, "bad probe arguments");
    MK_HIP(mk::regstream_probe(src, bytes, blocks, threads, depth, (uint32_t *)out_dev));
    return MK_OK;
}

int mk_read_trace(mk_handle *h, int64_t *out, size_t cap, size_t *n) {
    if (!h || !out || !n) return set_error(MK_EINVAL, "null argument");
    if (!h->built || !h->trace) return set_error(MK_EINVAL, "schedule was not built with trace = 1");
    const size_t need = (size_t)h->plan.n_cus * h->plan.Q * MK_TRACE_WORDS;
    if (cap < need) return set_error(MK_EINVAL, "buffer too small");
    MK_HIP(hipSetDevice(h->cfg.device));
    MK_HIP(hipDeviceSynchronize());
    MK_HIP(hipMemcpy(out, h->trace, need * 8, hipMemcpyDeviceToHost));
    *n = need;
    return MK_OK;
}

}  // extern "C"
