// mk_sched.cpp - host scheduler of the decode megakernel (pure C++, no HIP).
//
// "Inference MegaKernel" (shaojiemike.top):
//   - "unified framework": kernel graph -> tile/task graph -> per-SM queue +
//     event counters -> resident worker; the capacity obligation (queues,
//     rings and K/V pages must cover the configured maximum) and the
//     resource obligation (the largest body must not stop the launch).
//   - "hand-written whole-model MegaKernel / principle, schedule and
//     dataflow": start from a fixed Llama configuration, cut every op into
//     tiles, build the dependency DAG, assign tiles statically to each SM's
//     queue; a producer bumps a counter when its tile is done and a consumer
//     waits only for the count it needs.
//   - "MPK compiler and runtime" (its Figure 4): events connect only the tiles
//     that really depend on each other; the compile passes end with a
//     linearisation of ready tasks.
//
// What this file does, in order:
//   1. cut every op of every layer into tiles: a contiguous row range per
//      compute unit for each matvec (rows handed out by a least-loaded-first
//      fill over streamed bytes, so compute units that also carry attention
//      chunks get fewer rows of the next op), and one tile per (request, kv
//      head, K/V chunk) for attention;
//   2. create the events: one per (layer, kv group) for the QKV -> attention
//      edges (only the QKV tiles whose rows feed that group bump it), one per
//      layer for each later op boundary, and last-finisher merge counters for
//      the attention chunks and the LM-head argmax;
//   3. order all tiles in one global topological order (layer by layer, op
//      by op); each compute unit's queue is the subsequence of its tiles,
//      which makes every queue consistent with one order and so rules out
//      deadlock while all workgroups are co-resident (progress obligation);
//   4. encode each queue as [Q, 32] int32 words (mk_isa.h) and size the LDS
//      split between the activation area and the weight ring.
#include "mk_sched.h"

#include <algorithm>
#include <cstring>
#include <queue>

namespace mk {

namespace {

int ceil_div(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

bool k_supported(int k) { return k == 256 || (k >= 512 && k % 512 == 0); }

struct Tile {
    int op = OP_END, layer = 0, r0 = 0, r1 = 0, b = 0, g = 0, c = 0, nch = 0, flags = 0;
    std::vector<int> waits, pubs;
    int merge = -1, slot = 0, nslot = 0;
    int cu = 0;
    int64_t bytes = 0;
};

struct Ev {
    int kind = EVK_WAIT;
    int need = 0;
};

// Least-loaded-first: hand out n units of `unit_bytes` one at a time to the
// compute unit with the smallest cumulative streamed bytes (ties: lowest
// index). Returns the unit count per compute unit.
std::vector<int> fill_units(int n, int64_t unit_bytes, std::vector<int64_t> &cum) {
    const int S = (int)cum.size();
    std::vector<int> cnt(S, 0);
    using E = std::pair<int64_t, int>;
    std::priority_queue<E, std::vector<E>, std::greater<E>> pq;
    for (int c = 0; c < S; ++c) pq.push({cum[c], c});
    for (int i = 0; i < n; ++i) {
        E e = pq.top();
        pq.pop();
        cnt[e.second]++;
        e.first += unit_bytes;
        cum[e.second] = e.first;
        pq.push(e);
    }
    return cnt;
}

int pick_least(const std::vector<int64_t> &cum) {
    int best = 0;
    for (int c = 1; c < (int)cum.size(); ++c)
        if (cum[c] < cum[best]) best = c;
    return best;
}

}  // namespace

int check_config(const mk_config &c) {
    if (c.n_layers < 1 || c.hidden < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1)
        return set_error(MK_EINVAL, "layers, hidden and head counts must be positive");
    if (c.head_dim != 64) return set_error(MK_EINVAL, "head_dim must be 64");
    if (c.n_q_heads % c.n_kv_heads != 0 || c.n_q_heads / c.n_kv_heads > MAX_G)
        return set_error(MK_EINVAL, "n_q_heads must be a multiple of n_kv_heads with at most 8 q heads per kv head");
    if (!k_supported(c.hidden) || !k_supported(c.ffn) || !k_supported(c.n_q_heads * c.head_dim))
        return set_error(MK_EINVAL, "hidden, ffn and n_q_heads*head_dim must each be 256 or a multiple of 512");
    if (c.page_tokens != 16) return set_error(MK_EINVAL, "page_tokens must be 16");
    if (c.max_batch < 1 || c.max_batch > MAX_B) return set_error(MK_EINVAL, "max_batch must be in 1..8");
    if (c.max_pages_per_req < 1) return set_error(MK_EINVAL, "max_pages_per_req must be positive");
    if (c.has_embed != 0 && c.has_embed != 1) return set_error(MK_EINVAL, "has_embed must be 0 or 1");
    if (c.has_embed && c.vocab < 1) return set_error(MK_EINVAL, "vocab must be positive with an embedding");
    if (!(c.rms_eps >= 0.0f) || !(c.rope_theta > 0.0f)) return set_error(MK_EINVAL, "bad rms_eps or rope_theta");
    return MK_OK;
}

void attn_chunk_blocks(int kv_len, int page_tokens, int c, int nch, int *lo, int *hi) {
    const int nb = (kv_len + 1 + page_tokens - 1) / page_tokens;  // blocks covering positions 0..kv_len
    *lo = (int)((int64_t)c * nb / nch);
    *hi = (int)((int64_t)(c + 1) * nb / nch);
}

int64_t instr_stream_bytes(const mk_config &cfg, const int32_t *ins, int kv_len) {
    const int64_t H = cfg.hidden, F = cfg.ffn, QD = (int64_t)cfg.n_q_heads * cfg.head_dim;
    const int64_t rows = ins[W_R1] - ins[W_R0];
    switch (ins[W_OP]) {
        case OP_QKV: return rows * H * 2;
        case OP_OPROJ: return rows * QD * 2;
        case OP_UPGATE: return rows * H * 2 * 2;
        case OP_DOWN: return rows * F * 2;
        case OP_LMHEAD: return rows * H * 2;
        case OP_ATTN: {
            int lo, hi;
            attn_chunk_blocks(kv_len, cfg.page_tokens, ins[W_C], ins[W_NCH], &lo, &hi);
            return (int64_t)(hi - lo) * 2 * cfg.page_tokens * cfg.head_dim * 2;
        }
        default: return 0;
    }
}

int unfused_launches(const mk_config &cfg) {
    // per layer: norm, qkv, rope+append, attention chunks, merge, o-proj,
    // norm, up/gate, down; then final norm, LM head, argmax
    return cfg.n_layers * 9 + (cfg.has_embed ? 3 : 1);
}

int build_plan(const mk_config &cfg, const mk_schedule_desc &desc, Plan &P) {
    if (int rc = check_config(cfg)) return rc;
    P = Plan{};
    P.cfg = cfg;
    P.desc = desc;
    const int B = desc.batch, S = desc.n_cus;
    if (B < 1 || B > cfg.max_batch) return set_error(MK_EINVAL, "batch must be in 1..max_batch");
    if (S < 1) return set_error(MK_EINVAL, "n_cus must be positive");
    if (desc.mode != MK_MODE_MEGAKERNEL && desc.mode != MK_MODE_UNFUSED)
        return set_error(MK_EINVAL, "unknown mode");
    const int T = cfg.page_tokens, cap = cfg.max_pages_per_req * T;
    int maxlen = desc.max_kv_len > 0 ? desc.max_kv_len : cap - 1;
    if (maxlen > cap - 1 || maxlen < 0)
        return set_error(MK_ECAPACITY, "max_kv_len exceeds the page capacity of a request");
    P.max_kv_len = maxlen;
    const int nb_max = (maxlen + 1 + T - 1) / T;
    int C = desc.attn_chunks > 0 ? desc.attn_chunks : std::max(1, ceil_div(nb_max, 16));
    C = std::min(C, nb_max);
    P.attn_chunks = C;
    P.n_cus = S;

    const int L = cfg.n_layers, H = cfg.hidden, F = cfg.ffn, d = cfg.head_dim;
    const int nq = cfg.n_q_heads, nkv = cfg.n_kv_heads, G = nq / nkv, QD = nq * d;
    const int QKV = (nq + 2 * nkv) * d;

    // LDS split: activation area (matvec inputs of all requests, or the
    // attention staging) + misc flags + the weight ring.
    const int kmax = std::max(H, std::max(F, QD));
    const int attn_floats = G * 68 + 2 * 64 + N_COMPUTE_WAVES * G * 68;
    P.act_floats = std::max(B * ((kmax + 511) / 512 * 512), attn_floats);
    const int act_bytes = ceil_div((int64_t)P.act_floats * 4, 1024) * 1024;
    P.ring_granules = (LDS_LIMIT - MISC_BYTES - act_bytes) / GRANULE;
    if (desc.ring_kib < 0) return set_error(MK_EINVAL, "ring_kib must be >= 0");
    if (desc.dma_inflight < 0 || desc.dma_inflight > 57) return set_error(MK_EINVAL, "dma_inflight must be in 0..57");
    if (desc.ring_kib > 0) {
        if (desc.ring_kib > P.ring_granules)
            return set_error(MK_ECAPACITY, "ring_kib exceeds the LDS left next to the activation area");
        P.ring_granules = desc.ring_kib;
    }
    P.lds_bytes = MISC_BYTES + act_bytes + P.ring_granules * GRANULE;

    if (desc.mode == MK_MODE_UNFUSED) {
        P.launches = unfused_launches(cfg);
        P.n_lm_slots = cfg.has_embed ? ceil_div(cfg.vocab, 64) : 0;
        return MK_OK;
    }
    P.launches = 1;

    // largest unit a compute wave holds in the ring at once
    const int max_unit = std::max({ceil_div((int64_t)2 * H * 2, GRANULE), ceil_div((int64_t)F * 2, GRANULE),
                                   ceil_div((int64_t)QD * 2, GRANULE), ceil_div((int64_t)2 * T * d * 2, GRANULE)});
    if (P.ring_granules < 2 * max_unit + 2)
        return set_error(MK_ECAPACITY, "batch too large: the LDS ring cannot hold two units of the largest op "
                                       "next to the activation area (" + std::to_string(P.act_floats * 4) + " B)");

    std::vector<Tile> tiles;
    std::vector<Ev> evs;
    auto new_ev = [&](int kind) { evs.push_back(Ev{kind, 0}); return (int)evs.size() - 1; };
    std::vector<int64_t> cum(S, 0);

    // rows of one matvec op, one tile per compute unit that receives rows
    auto matvec_op = [&](int op, int layer, int rows, int64_t unit_bytes, const std::vector<int> &waits,
                         int flags) -> std::vector<int> {
        std::vector<int> cnt = fill_units(rows, unit_bytes, cum);
        std::vector<int> ids;
        int r = 0;
        for (int c = 0; c < S; ++c) {
            if (cnt[c] == 0) continue;
            Tile t;
            t.op = op;
            t.layer = layer;
            t.r0 = r;
            t.r1 = r + cnt[c];
            t.cu = c;
            t.waits = waits;
            t.flags = flags;
            t.bytes = (int64_t)cnt[c] * unit_bytes;
            r += cnt[c];
            tiles.push_back(t);
            ids.push_back((int)tiles.size() - 1);
        }
        return ids;
    };

    int ev_prev = -1;  // event: residual stream of this layer is complete
    for (int l = 0; l < L; ++l) {
        const int first = l == 0 ? F_X_FROM_INPUT : 0;
        // --- QKV
        std::vector<int> w0;
        if (ev_prev >= 0) w0.push_back(ev_prev);
        std::vector<int> qkv_ids = matvec_op(OP_QKV, l, QKV, (int64_t)H * 2, w0, first);
        // per-group events when every tile feeds few groups, else one event
        auto groups_of = [&](const Tile &t) {
            std::vector<int> gs;
            for (int g = 0; g < nkv; ++g) {
                const int rq0 = g * G * d, rq1 = (g + 1) * G * d;
                const int rk0 = QD + g * d, rk1 = rk0 + d;
                const int rv0 = QD + nkv * d + g * d, rv1 = rv0 + d;
                auto hit = [&](int a, int b) { return t.r0 < b && a < t.r1; };
                if (hit(rq0, rq1) || hit(rk0, rk1) || hit(rv0, rv1)) gs.push_back(g);
            }
            return gs;
        };
        bool per_group = true;
        for (int id : qkv_ids)
            if ((int)groups_of(tiles[id]).size() > MAX_PUB) per_group = false;
        std::vector<int> ev_qkv(nkv);
        if (per_group) {
            for (int g = 0; g < nkv; ++g) ev_qkv[g] = new_ev(EVK_WAIT);
            for (int id : qkv_ids)
                for (int g : groups_of(tiles[id])) tiles[id].pubs.push_back(ev_qkv[g]);
        } else {
            int e = new_ev(EVK_WAIT);
            for (int g = 0; g < nkv; ++g) ev_qkv[g] = e;
            for (int id : qkv_ids) tiles[id].pubs.push_back(e);
        }
        // --- attention chunks; the last chunk of each (b, g) to finish merges
        const int ev_attn = new_ev(EVK_WAIT);
        for (int b = 0; b < B; ++b)
            for (int g = 0; g < nkv; ++g) {
                const int ev_merge = new_ev(EVK_MERGE);
                for (int c = 0; c < C; ++c) {
                    Tile t;
                    t.op = OP_ATTN;
                    t.layer = l;
                    t.b = b;
                    t.g = g;
                    t.c = c;
                    t.nch = C;
                    t.waits = {ev_qkv[g]};
                    t.pubs = {ev_attn};
                    t.merge = ev_merge;
                    t.slot = c;
                    t.nslot = C;
                    int lo, hi;
                    attn_chunk_blocks(maxlen, T, c, C, &lo, &hi);
                    t.bytes = (int64_t)(hi - lo) * 2 * T * d * 2;
                    t.cu = pick_least(cum);
                    cum[t.cu] += t.bytes;
                    tiles.push_back(t);
                }
            }
        // --- O projection + residual
        const int ev_o = new_ev(EVK_WAIT);
        for (int id : matvec_op(OP_OPROJ, l, H, (int64_t)QD * 2, {ev_attn}, first)) tiles[id].pubs.push_back(ev_o);
        // --- up/gate + SiLU
        const int ev_ug = new_ev(EVK_WAIT);
        for (int id : matvec_op(OP_UPGATE, l, F, (int64_t)H * 4, {ev_o}, 0)) tiles[id].pubs.push_back(ev_ug);
        // --- down + residual
        const bool last = l == L - 1;
        std::vector<int> down_ids = matvec_op(OP_DOWN, l, H, (int64_t)F * 2, {ev_ug}, last ? F_WRITE_HIDDEN : 0);
        if (!last || cfg.has_embed) {
            const int ev_d = new_ev(EVK_WAIT);
            for (int id : down_ids) tiles[id].pubs.push_back(ev_d);
            ev_prev = ev_d;
        } else {
            const int ev_fin = new_ev(EVK_MERGE);
            for (size_t i = 0; i < down_ids.size(); ++i) {
                Tile &t = tiles[down_ids[i]];
                t.merge = ev_fin;
                t.slot = (int)i;
                t.nslot = (int)down_ids.size();
                t.flags |= F_STEP_FINAL;
            }
        }
    }
    if (cfg.has_embed) {
        std::vector<int> lm_ids = matvec_op(OP_LMHEAD, L, cfg.vocab, (int64_t)H * 2, {ev_prev}, F_STEP_FINAL);
        const int ev_lm = new_ev(EVK_MERGE);
        for (size_t i = 0; i < lm_ids.size(); ++i) {
            Tile &t = tiles[lm_ids[i]];
            t.merge = ev_lm;
            t.slot = (int)i;
            t.nslot = (int)lm_ids.size();
        }
        P.n_lm_slots = (int)lm_ids.size();
    }

    // event needs: producers per step
    for (const Tile &t : tiles) {
        if (t.op == OP_ATTN) continue;  // attention publishes once per (b, g), below
        for (int e : t.pubs) evs[e].need++;
    }
    for (const Tile &t : tiles)
        if (t.op == OP_ATTN && t.c == 0) evs[t.pubs[0]].need++;
    for (const Tile &t : tiles)
        if (t.merge >= 0) evs[t.merge].need = t.nslot;
    for (const Tile &t : tiles) {
        if ((int)t.waits.size() > MAX_WAIT || (int)t.pubs.size() > MAX_PUB)
            return set_error(MK_ECAPACITY, "instruction has too many waits or completions");
    }

    // per-CU queues in the global order
    std::vector<std::vector<int>> per_cu(S);
    for (int i = 0; i < (int)tiles.size(); ++i) per_cu[tiles[i].cu].push_back(i);
    int Q = 1;
    for (auto &v : per_cu) Q = std::max(Q, (int)v.size() + 1);
    P.Q = Q;
    P.n_instr = (int)tiles.size();
    P.queue.assign((size_t)S * Q * INSTR_WORDS, 0);
    for (int c = 0; c < S; ++c) {
        int64_t bytes = 0;
        for (size_t k = 0; k < per_cu[c].size(); ++k) {
            const int id = per_cu[c][k];
            const Tile &t = tiles[id];
            int32_t *w = &P.queue[((size_t)c * Q + k) * INSTR_WORDS];
            w[W_OP] = t.op;
            w[W_LAYER] = t.layer;
            w[W_R0] = t.r0;
            w[W_R1] = t.r1;
            w[W_B] = t.b;
            w[W_G] = t.g;
            w[W_C] = t.c;
            w[W_NCH] = t.nch;
            w[W_FLAGS] = t.flags;
            w[W_NWAIT] = (int)t.waits.size();
            for (size_t j = 0; j < t.waits.size(); ++j) w[W_WAIT + j] = t.waits[j];
            w[W_NPUB] = (int)t.pubs.size();
            for (size_t j = 0; j < t.pubs.size(); ++j) w[W_PUB + j] = t.pubs[j];
            w[W_MERGE] = t.merge;
            w[W_SLOT] = t.slot;
            w[W_NSLOT] = t.nslot;
            w[W_SEQ] = id;
            bytes += t.bytes;
        }
        // END is the zero-filled word after the last instruction
        P.stream_total += bytes;
        P.stream_max_cu = std::max(P.stream_max_cu, bytes);
    }
    P.n_events = (int)evs.size();
    P.n_counters = P.n_events;
    P.events.assign((size_t)P.n_events * EV_WORDS, 0);
    for (int e = 0; e < P.n_events; ++e) {
        P.events[(size_t)e * EV_WORDS + EV_CTR] = e;
        P.events[(size_t)e * EV_WORDS + EV_NEED] = evs[e].need;
        P.events[(size_t)e * EV_WORDS + EV_KIND] = evs[e].kind;
    }
    return MK_OK;
}

}  // namespace mk

// ------------------------------------------------------------ C ABI (plans)

struct mk_plan {
    mk::Plan p;
};

extern "C" {

int mk_plan_create(const mk_config *cfg, const mk_schedule_desc *s, mk_plan **out) {
    if (!cfg || !s || !out) return mk::set_error(MK_EINVAL, "null argument");
    if (s->n_cus <= 0) return mk::set_error(MK_EINVAL, "mk_plan_create needs n_cus > 0");
    mk_plan *p = new (std::nothrow) mk_plan();
    if (!p) return mk::set_error(MK_EINVAL, "out of host memory");
    int rc = mk::build_plan(*cfg, *s, p->p);
    if (rc) {
        delete p;
        return rc;
    }
    *out = p;
    return MK_OK;
}

void mk_plan_destroy(mk_plan *p) { delete p; }

int mk_plan_info(const mk_plan *p, mk_schedule_info *out) {
    if (!p || !out) return mk::set_error(MK_EINVAL, "null argument");
    const mk::Plan &P = p->p;
    std::memset(out, 0, sizeof *out);
    out->n_cus = P.n_cus;
    out->queue_len = P.Q;
    out->n_instr = P.n_instr;
    out->n_events = P.n_events;
    out->n_counters = P.n_counters;
    out->attn_chunks = P.attn_chunks;
    out->ring_granules = P.ring_granules;
    out->lds_bytes = P.lds_bytes;
    out->block_threads = mk::BLOCK_THREADS;
    out->stream_bytes_max_cu = P.stream_max_cu;
    out->stream_bytes_total = P.stream_total;
    out->launches_per_step = P.launches;
    return MK_OK;
}

int mk_plan_queue(const mk_plan *p, int32_t *out, size_t cap) {
    if (!p || !out) return mk::set_error(MK_EINVAL, "null argument");
    if (cap < p->p.queue.size()) return mk::set_error(MK_EINVAL, "buffer too small");
    std::memcpy(out, p->p.queue.data(), p->p.queue.size() * sizeof(int32_t));
    return MK_OK;
}

int mk_plan_events(const mk_plan *p, int32_t *out, size_t cap) {
    if (!p || !out) return mk::set_error(MK_EINVAL, "null argument");
    if (cap < p->p.events.size()) return mk::set_error(MK_EINVAL, "buffer too small");
    std::memcpy(out, p->p.events.data(), p->p.events.size() * sizeof(int32_t));
    return MK_OK;
}

}  // extern "C"
