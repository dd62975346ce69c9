// mk_sched.cpp - host scheduler of the decode megakernel (pure C++, no HIP).
//
// "Inference MegaKernel" (shaojiemike.top):
//   - "unified framework": kernel graph -> tile/task graph -> per-SM queue +
//     event counters -> resident worker; the capacity obligation (queues,
//     on-chip buffers and K/V pages must cover the configured maximum) and
//     the resource obligation (the largest body must not stop the launch).
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
//      fill over streamed bytes, restarted at each op that follows a hop;
//      the O projection's fill counts the layer's QKV and attention bytes,
//      so compute units that also carry attention chunks get fewer of its
//      rows), and one tile per (request, kv head, K/V chunk) for attention;
//   2. create the merge events: last-finisher counters for the attention
//      chunks of each (layer, request, kv head), the LM-head argmax, and the
//      end of a step without an LM head. The data edges need no event: every
//      activation carries the step's tag, a consumer waits for the tags of
//      exactly what it reads, and each buffer is written once per step;
//   3. order all tiles in one global topological order (layer by layer, op
//      by op); each compute unit's queue is the subsequence of its tiles,
//      which makes every queue consistent with one order and so rules out
//      deadlock while all workgroups are co-resident (progress obligation);
//   4. encode each queue as [Q, 32] int32 words (mk_isa.h) and lay out the
//      LDS of a workgroup (residual rows, activations, attention states).
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
    int merge = -1, slot = 0, nslot = 0;
    int cu = 0;
    int64_t bytes = 0;
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
    if (c.max_pages_per_req < 1 || c.max_pages_per_req > 65535)
        return set_error(MK_EINVAL, "max_pages_per_req must be in 1..65535");
    if (c.has_embed != 0 && c.has_embed != 1) return set_error(MK_EINVAL, "has_embed must be 0 or 1");
    if (c.has_embed && c.vocab < 1) return set_error(MK_EINVAL, "vocab must be positive with an embedding");
    if (!(c.rms_eps >= 0.0f) || !(c.rope_theta > 0.0f)) return set_error(MK_EINVAL, "bad rms_eps or rope_theta");
    return MK_OK;
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
    if (desc.attn_split != SPLIT_BALANCED && desc.attn_split != SPLIT_PER_REQUEST)
        return set_error(MK_EINVAL, "unknown attn_split");
    if (desc.reserved1 != 0) return set_error(MK_EINVAL, "reserved fields must be 0");
    const int T = cfg.page_tokens, cap = cfg.max_pages_per_req * T;
    int maxlen = desc.max_kv_len > 0 ? desc.max_kv_len : cap - 1;
    if (maxlen > cap - 1 || maxlen < 0)
        return set_error(MK_ECAPACITY, "max_kv_len exceeds the page capacity of a request");
    P.max_kv_len = maxlen;
    const int nb_max = (maxlen + 1 + T - 1) / T;
    // enough chunks that one chunk's K/V blocks fit in its workgroup's
    // prefetch window (N_COMPUTE_WAVES waves x PREFETCH_SLICES blocks)
    if (desc.attn_chunks > MAX_ATTN_CHUNKS)
        return set_error(MK_EINVAL, "attn_chunks above " + std::to_string(MAX_ATTN_CHUNKS));
    if ((int64_t)B * desc.attn_chunks > MAX_ATTN_TILES)
        return set_error(MK_EINVAL, "batch x attn_chunks above " + std::to_string(MAX_ATTN_TILES));
    // about one K/V block per wave on half the waves (one wave per SIMD,
    // which then has the vector unit to itself): attention is short
    // arithmetic on few units, so it is spread wide; with more requests there
    // are more tiles already, and half the chunk cap, and no more tiles than
    // compute units (a unit's second tile would start only after its first,
    // while the balanced split already evens out the tiles' sizes). Long K/V
    // at batch <= 2: two blocks per wave, up to one tile per compute unit
    // (1b-kv8192: 32 tiles per request took 953 us per step against 1041 at
    // 16, 1088 at 48; at 1b-kv1024 16 stays best)
    int C = desc.attn_chunks > 0
                ? desc.attn_chunks
                : std::min(B <= 2 ? AUTO_ATTN_CHUNKS : AUTO_ATTN_CHUNKS / 2,
                           std::max(1, ceil_div(nb_max, N_COMPUTE_WAVES / 2)));
    if (desc.attn_chunks <= 0 && B <= 2)
        C = std::max(C, std::min({MAX_ATTN_CHUNKS, ceil_div(nb_max, 2 * N_COMPUTE_WAVES),
                                  std::max(1, S / (B * cfg.n_kv_heads))}));
    if (desc.attn_chunks <= 0 && B > 2) C = std::min(C, std::max(1, S / (B * cfg.n_kv_heads)));
    C = std::min(C, nb_max);
    P.attn_chunks = C;
    P.n_cus = S;

    const int L = cfg.n_layers, H = cfg.hidden, F = cfg.ffn, d = cfg.head_dim;
    const int nq = cfg.n_q_heads, nkv = cfg.n_kv_heads, G = nq / nkv, QD = nq * d;
    const int QKV = (nq + 2 * nkv) * d;

    if (desc.mode == MK_MODE_UNFUSED) {
        P.launches = unfused_launches(cfg);
        P.n_lm_slots = cfg.has_embed ? ceil_div(cfg.vocab, 64) : 0;
        return MK_OK;
    }
    P.launches = 1;
    if (G != 1 && G != 2 && G != 4 && G != 8)
        return set_error(MK_EINVAL, "the resident interpreter needs n_q_heads / n_kv_heads in {1, 2, 4, 8}");

    std::vector<Tile> tiles;
    std::vector<int> ev_need;  // merge events
    auto new_merge = [&](int need) {
        ev_need.push_back(need);
        return (int)ev_need.size() - 1;
    };
    std::vector<int64_t> cum(S, 0);

    // rows of one matvec op, one tile per compute unit that receives rows
    auto matvec_op = [&](int op, int layer, int rows, int64_t unit_bytes, int flags) -> std::vector<int> {
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
            t.flags = flags;
            t.bytes = (int64_t)cnt[c] * unit_bytes;
            r += cnt[c];
            tiles.push_back(t);
            ids.push_back((int)tiles.size() - 1);
        }
        return ids;
    };

    for (int l = 0; l < L; ++l) {
        const int first = l == 0 ? F_X_FROM_INPUT : 0;
        // Every unit starts an op that follows a hop at about the same time,
        // so the fill starts afresh there (QKV, UPGATE, DOWN, LM head); the
        // O projection continues from the QKV and attention bytes, so that
        // units carrying attention chunks get fewer of its rows.
        std::fill(cum.begin(), cum.end(), 0);
        matvec_op(OP_QKV, l, QKV, (int64_t)H * 2, first);
        // B x C attention tiles per kv head, each publishing one softmax
        // state: which request and K/V blocks a tile takes is decided on the
        // device at every step (the attention split), so each is charged an
        // equal share of the batch's K/V at max_kv_len; then one merge per
        // (request, kv head), on the least-loaded unit
        const int TT = B * C;
        for (int g = 0; g < nkv; ++g)
            for (int c = 0; c < TT; ++c) {
                // a single request's split is fixed: tile c of its blocks
                const int64_t blocks = B == 1 ? (int64_t)(c + 1) * nb_max / TT - (int64_t)c * nb_max / TT
                                              : (int64_t)ceil_div((int64_t)B * nb_max, TT);
                Tile t;
                t.op = OP_ATTN;
                t.layer = l;
                t.b = -1;
                t.g = g;
                t.c = c;
                t.nch = TT;
                // ceil(2^32 / TT): a single request's interpreter divides by TT with it
                t.r1 = TT > 1 ? (int32_t)(uint32_t)(((1ull << 32) + TT - 1) / TT) : 0;
                t.merge = -1;
                t.slot = c;
                t.nslot = TT;
                t.bytes = blocks * 2 * T * d * 2;
                t.cu = pick_least(cum);
                cum[t.cu] += t.bytes;
                tiles.push_back(t);
            }
        for (int b = 0; b < B; ++b)
            for (int g = 0; g < nkv; ++g) {
                Tile t;
                t.op = OP_AMERGE;
                t.layer = l;
                t.b = b;
                t.g = g;
                t.nch = TT;
                // ceil(2^32 / TT): a single request's interpreter divides by TT with it
                t.r1 = TT > 1 ? (int32_t)(uint32_t)(((1ull << 32) + TT - 1) / TT) : 0;
                t.merge = -1;
                t.bytes = 0;  // streams nothing
                t.cu = pick_least(cum);
                // charged at the whole O projection: a merge ends after the
                // attention tiles, later than any other unit's inputs arrive,
                // so its unit takes none of the O projection's rows (unless
                // every unit carries a merge), which would otherwise end last
                // and hold back the MLP
                cum[t.cu] += (int64_t)H * QD * 2;
                tiles.push_back(t);
            }
        matvec_op(OP_OPROJ, l, H, (int64_t)QD * 2, first);
        std::fill(cum.begin(), cum.end(), 0);
        matvec_op(OP_UPGATE, l, F, (int64_t)H * 4, 0);
        std::fill(cum.begin(), cum.end(), 0);
        const bool last = l == L - 1;
        std::vector<int> down_ids = matvec_op(OP_DOWN, l, H, (int64_t)F * 2, last ? F_WRITE_HIDDEN : 0);
        if (last && !cfg.has_embed) {  // the last down-projection tile to finish ends the step
            const int ev = new_merge((int)down_ids.size());
            for (size_t i = 0; i < down_ids.size(); ++i) {
                Tile &t = tiles[down_ids[i]];
                t.merge = ev;
                t.slot = (int)i;
                t.nslot = (int)down_ids.size();
                t.flags |= F_STEP_FINAL;
            }
        }
    }
    if (cfg.has_embed) {
        std::fill(cum.begin(), cum.end(), 0);
        std::vector<int> lm_ids = matvec_op(OP_LMHEAD, L, cfg.vocab, (int64_t)H * 2, F_STEP_FINAL);
        const int ev = new_merge((int)lm_ids.size());
        for (size_t i = 0; i < lm_ids.size(); ++i) {
            Tile &t = tiles[lm_ids[i]];
            t.merge = ev;
            t.slot = (int)i;
            t.nslot = (int)lm_ids.size();
        }
        P.n_lm_slots = (int)lm_ids.size();
    }

    // per-CU queues in the global order
    std::vector<std::vector<int>> per_cu(S);
    for (int i = 0; i < (int)tiles.size(); ++i) per_cu[tiles[i].cu].push_back(i);
    int Q = 1;
    for (auto &v : per_cu) Q = std::max(Q, (int)v.size() + 1);
    P.Q = Q;
    P.n_instr = (int)tiles.size();
    P.queue.assign((size_t)S * Q * INSTR_WORDS, 0);
    int max_rows_x = 1;  // residual rows an O- or down-projection tile stages
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
            w[W_MERGE] = t.merge;
            w[W_SLOT] = t.slot;
            w[W_NSLOT] = t.nslot;
            w[W_SEQ] = id;
            w[W_MCTR] = t.merge;  // the merge event's counter is its index
            w[W_MNEED] = t.merge >= 0 ? ev_need[t.merge] : 0;
            bytes += t.bytes;
            if (t.op == OP_OPROJ || t.op == OP_DOWN) max_rows_x = std::max(max_rows_x, t.r1 - t.r0);
        }
        // END is the zero-filled word after the last instruction
        P.stream_total += bytes;
        P.stream_max_cu = std::max(P.stream_max_cu, bytes);
    }
    P.n_events = (int)ev_need.size();
    P.n_counters = P.n_events;
    P.events.assign((size_t)P.n_events * EV_WORDS, 0);
    for (int e = 0; e < P.n_events; ++e) {
        P.events[(size_t)e * EV_WORDS + EV_CTR] = e;
        P.events[(size_t)e * EV_WORDS + EV_NEED] = ev_need[e];
        P.events[(size_t)e * EV_WORDS + EV_KIND] = EVK_MERGE;
    }

    // LDS layout (capacity obligation: everything a tile stages must fit)
    const int NBP = B <= 1 ? 1 : B <= 2 ? 2 : B <= 4 ? 4 : 8;  // requests the interpreter is compiled for
    // at a padded batch of 8 every matvec input is staged as binary16 (half
    // the bytes), a norm's input first gathered as fp32 past it (1.5 H
    // floats per request); otherwise every input is fp32
    const int kmax = NBP == 8 ? std::max({(3 * H + 1) / 2, (QD + 1) / 2, (F + 1) / 2}) : std::max(H, std::max(F, QD));
    P.act_stride = (kmax + 511) / 512 * 512;
    P.xrow_stride = (max_rows_x + 3) / 4 * 4;
    // matvec inputs; attention staging (queries, new K/V entry) and the
    // tile's wave states; an AMERGE's tile states (MAX_ATTN_CHUNKS at a
    // time); LM-head partials
    const int64_t act_floats =
        std::max<int64_t>({(int64_t)NBP * P.act_stride, (int64_t)G * 64 + 64 + attn_state_floats(G),
                           (int64_t)std::min(B * C, MAX_ATTN_CHUNKS) * G * ATTN_PART,
                           (int64_t)P.n_lm_slots * B * 2});
    auto up256 = [](int64_t x) { return (x + 255) / 256 * 256; };
    const int64_t queue_off = MISC_BYTES;  // the CU's queue, LDS_INSTR_WORDS words per instruction
    const int64_t xrow_off = queue_off + up256((int64_t)Q * LDS_INSTR_WORDS * 4);
    const int64_t act_off = xrow_off + up256((int64_t)NBP * P.xrow_stride * 4);
    // the norm weights of a staged RMSNorm, copied in whole 1 KiB wave loads
    const int64_t nw_off = act_off + up256(act_floats * 4);
    const int64_t lds = nw_off + ((int64_t)H * 2 + 1023) / 1024 * 1024;
    if (lds > LDS_LIMIT)
        return set_error(MK_ECAPACITY, "a tile's on-chip staging needs " + std::to_string(lds) +
                                           " bytes of LDS (limit " + std::to_string(LDS_LIMIT) +
                                           "): the activation area holds " + std::to_string(NBP) + " x " +
                                           std::to_string(P.act_stride) + " floats");
    P.queue_off = (int)queue_off;
    P.xrow_off = (int)xrow_off;
    P.act_off = (int)act_off;
    P.nw_off = (int)nw_off;
    P.lds_bytes = (int)lds;
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
    out->prefetch_slices = mk::PREFETCH_SLICES;
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
