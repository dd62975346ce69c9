/* oracle.c - plain, slow CPU reference for one decode step of a Llama-style
 * dense decoder.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the product path. It shares no code
 * with the HIP library. Single thread, sequential sums in index order, no
 * blocking, no fusion, no reordering.
 *
 * Source of the computation: "Inference MegaKernel" (shaojiemike.top).
 *   [bubbles]  section "why conventional inference still has bubbles": a
 *              decode step is Norm, QKV GEMM, RoPE, Attention, residual, MLP
 *              and sampling, in that order.
 *   [flow]     section "hand-written whole-model MegaKernel / principle,
 *              schedule and dataflow": the interpreter dispatches RMS_NORM,
 *              QKV_MATVEC, ATTENTION, MLP_UP_GATE, MLP_DOWN and LM_HEAD; its
 *              object table puts the weights in HBM for the model's lifetime
 *              and the K/V cache in per-layer pages owned by the request.
 * The page names the ops but not their formulas. The formulas below are the
 * plain Llama definitions; each place where the page leaves a choice open
 * carries a "Reading:" note.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

#ifdef ORACLE_REAL_FLOAT
#define R_SQRT sqrtf
#define R_EXP expf
#else
#define R_SQRT sqrt
#define R_EXP exp
#endif

/* ------------------------------------------------------------------ bf16 */

float oracle_bf16_to_f32(uint16_t h)
{
    /* bf16 is the upper half of a binary32 pattern. */
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Value of a bf16 pattern used as a rounding candidate. The pattern after the
 * largest finite one stands for 2^128, the next value of an unbounded
 * exponent range, so that overflow follows round-to-nearest-even. */
static double candidate_value(uint16_t h)
{
    if ((h & 0x7fffu) == 0x7f80u)
        return (h & 0x8000u) ? -ldexp(1.0, 128) : ldexp(1.0, 128);
    return (double)oracle_bf16_to_f32(h);
}

uint16_t oracle_f32_to_bf16(float f)
{
    /* Round to nearest, ties to even, from the definition: the two bf16
     * values that bracket f are the truncation `lo` and the next pattern away
     * from zero `hi`; take the nearer, and on a tie the one whose last
     * mantissa bit is 0. NaN maps to a quiet NaN of the same sign. */
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if (isnan(f))
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u);
    uint16_t lo = (uint16_t)(u >> 16);
    if ((u & 0xffffu) == 0)
        return lo; /* exactly representable, includes +-0 and +-inf */
    uint16_t hi = (uint16_t)(lo + 1u);
    double dlo = fabs((double)f - candidate_value(lo));
    double dhi = fabs(candidate_value(hi) - (double)f);
    if (dlo < dhi)
        return lo;
    if (dhi < dlo)
        return hi;
    return (lo & 1u) ? hi : lo;
}

static oracle_real wv(const uint16_t *w, size_t i)
{
    return (oracle_real)oracle_bf16_to_f32(w[i]);
}

/* ------------------------------------------------------------- single ops */

/* RMS_NORM body ([flow]). Reading: epsilon inside the square root, the mean
 * taken over the hidden size, the weight applied after normalisation, no
 * scaling of the embedding. */
void oracle_rmsnorm(const oracle_real *x, const uint16_t *w, int32_t n,
                    double eps, oracle_real *out)
{
    oracle_real ss = 0;
    for (int32_t i = 0; i < n; ++i)
        ss += x[i] * x[i];
    oracle_real inv = (oracle_real)1 / R_SQRT(ss / (oracle_real)n + (oracle_real)eps);
    for (int32_t i = 0; i < n; ++i)
        out[i] = (x[i] * inv) * wv(w, (size_t)i);
}

/* The matvec of QKV_MATVEC, MLP_UP_GATE, MLP_DOWN and LM_HEAD ([flow]):
 * y[r] = sum_c W[r, c] x[c], W row-major [rows, cols] in bf16. */
void oracle_matvec(const uint16_t *W, int32_t rows, int32_t cols,
                   const oracle_real *x, oracle_real *y)
{
    for (int32_t r = 0; r < rows; ++r) {
        oracle_real acc = 0;
        for (int32_t c = 0; c < cols; ++c)
            acc += wv(W, (size_t)r * (size_t)cols + (size_t)c) * x[c];
        y[r] = acc;
    }
}

/* RoPE ([bubbles] lists it as its own kernel). Reading: the rotate-half
 * pairing (i, i + d/2) with frequency theta^(-2i/d) and angle pos * freq,
 * evaluated in double; no frequency scaling. */
void oracle_rope(oracle_real *v, int32_t n_heads, int32_t head_dim,
                 int32_t pos, double theta)
{
    int32_t half = head_dim / 2;
    for (int32_t h = 0; h < n_heads; ++h) {
        oracle_real *x = v + (size_t)h * (size_t)head_dim;
        for (int32_t i = 0; i < half; ++i) {
            double freq = pow(theta, -2.0 * (double)i / (double)head_dim);
            double ang = (double)pos * freq;
            oracle_real c = (oracle_real)cos(ang), s = (oracle_real)sin(ang);
            oracle_real a = x[i], b = x[i + half];
            x[i] = a * c - b * s;
            x[i + half] = b * c + a * s;
        }
    }
}

/* SiLU of the gated MLP: z / (1 + e^-z). */
oracle_real oracle_silu(oracle_real z)
{
    return z / ((oracle_real)1 + R_EXP(-z));
}

/* Greedy sampling ([bubbles] "sampling"). The decision is taken on the
 * binary32 value of each logit, the precision in which the GPU path holds
 * its logits. Reading: the lowest index wins a tie; a NaN logit is an
 * error (-1). */
int32_t oracle_argmax(const oracle_real *v, int32_t n)
{
    int32_t best = -1;
    float bv = 0.0f;
    for (int32_t i = 0; i < n; ++i) {
        float f = (float)v[i];
        if (isnan(f))
            return -1;
        if (best < 0 || f > bv) {
            best = i;
            bv = f;
        }
    }
    return best;
}

/* Address of one cached row (position `pos`, kv head `g`) inside one layer's
 * pool [n_pages, nkv, page_tokens, d]. */
static size_t kv_row(const oracle_dims *dm, const int32_t *page_row,
                     int32_t pos, int32_t g)
{
    int32_t page = page_row[pos / dm->page_tokens];
    int32_t slot = pos % dm->page_tokens;
    return (((size_t)page * (size_t)dm->n_kv_heads + (size_t)g)
                * (size_t)dm->page_tokens + (size_t)slot)
           * (size_t)dm->head_dim;
}

/* ATTENTION body ([flow]) over the paged cache ([flow] object table).
 * Reading: query head h uses kv head h / (nq / nkv) (contiguous groups);
 * scores are scaled by 1/sqrt(d); no mask beyond the length; the softmax is
 * the plain definition with the maximum subtracted. */
void oracle_attention(const oracle_dims *dm, const oracle_real *q,
                      const uint16_t *k_layer, const uint16_t *v_layer,
                      const int32_t *page_row, int32_t pos,
                      oracle_real *out)
{
    int32_t d = dm->head_dim, G = dm->n_q_heads / dm->n_kv_heads;
    int32_t n = pos + 1;
    oracle_real scale = (oracle_real)1 / R_SQRT((oracle_real)d);
    oracle_real *s = (oracle_real *)malloc(sizeof(oracle_real) * (size_t)n);
    for (int32_t h = 0; h < dm->n_q_heads; ++h) {
        int32_t g = h / G;
        const oracle_real *qh = q + (size_t)h * (size_t)d;
        oracle_real m = 0;
        for (int32_t j = 0; j < n; ++j) {
            size_t base = kv_row(dm, page_row, j, g);
            oracle_real dot = 0;
            for (int32_t c = 0; c < d; ++c)
                dot += qh[c] * wv(k_layer, base + (size_t)c);
            s[j] = dot * scale;
            if (j == 0 || s[j] > m)
                m = s[j];
        }
        oracle_real z = 0;
        for (int32_t j = 0; j < n; ++j) {
            s[j] = R_EXP(s[j] - m);
            z += s[j];
        }
        oracle_real *oh = out + (size_t)h * (size_t)d;
        for (int32_t c = 0; c < d; ++c)
            oh[c] = 0;
        for (int32_t j = 0; j < n; ++j) {
            size_t base = kv_row(dm, page_row, j, g);
            oracle_real p = s[j] / z;
            for (int32_t c = 0; c < d; ++c)
                oh[c] += p * wv(v_layer, base + (size_t)c);
        }
    }
    free(s);
}

/* ------------------------------------------------------------ decode step */

int32_t oracle_decode_step(const oracle_dims *dm, const oracle_weights *w,
                           uint16_t *k_pool, uint16_t *v_pool,
                           const int32_t *page_table, int32_t batch,
                           const int32_t *tokens_in,
                           const oracle_real *hidden_in,
                           const int32_t *kv_lens,
                           oracle_real *logits_out, oracle_real *hidden_out,
                           int32_t *tokens_out)
{
    const int32_t L = dm->n_layers, H = dm->hidden, nq = dm->n_q_heads,
                  nkv = dm->n_kv_heads, d = dm->head_dim, F = dm->ffn,
                  V = dm->vocab, T = dm->page_tokens;
    const int32_t QKV = (nq + 2 * nkv) * d;
    const size_t layer_pool = (size_t)dm->n_pages * (size_t)nkv * (size_t)T * (size_t)d;
    int32_t rc = 0;

    oracle_real *x = malloc(sizeof(oracle_real) * (size_t)H);
    oracle_real *u = malloc(sizeof(oracle_real) * (size_t)H);
    oracle_real *qkv = malloc(sizeof(oracle_real) * (size_t)QKV);
    oracle_real *o = malloc(sizeof(oracle_real) * (size_t)(nq * d));
    oracle_real *t = malloc(sizeof(oracle_real) * (size_t)H);
    oracle_real *gt = malloc(sizeof(oracle_real) * (size_t)F);
    oracle_real *up = malloc(sizeof(oracle_real) * (size_t)F);
    oracle_real *logits = dm->has_embed ? malloc(sizeof(oracle_real) * (size_t)V) : NULL;

    for (int32_t b = 0; b < batch && rc == 0; ++b) {
        const int32_t *page_row = page_table + (size_t)b * (size_t)dm->max_pages_per_req;
        /* Reading: the new token sits at position p = current length
         * (0-based) and attends to p + 1 positions, itself included. */
        int32_t p = kv_lens[b];
        if (p < 0 || p >= dm->max_pages_per_req * T) {
            rc = -1;
            break;
        }
        for (int32_t j = 0; j <= p / T; ++j)
            if (page_row[j] < 0 || page_row[j] >= dm->n_pages)
                rc = -1;
        if (rc)
            break;

        /* Reading: the step starts from the embedding row of the token (no
         * embedding kernel is named on the page), or from the given hidden
         * vector when the model has no embedding. */
        if (dm->has_embed) {
            int32_t tok = tokens_in[b];
            if (tok < 0 || tok >= V) {
                rc = -1;
                break;
            }
            for (int32_t i = 0; i < H; ++i)
                x[i] = wv(w->embed, (size_t)tok * (size_t)H + (size_t)i);
        } else {
            for (int32_t i = 0; i < H; ++i)
                x[i] = hidden_in[(size_t)b * (size_t)H + (size_t)i];
        }

        for (int32_t l = 0; l < L; ++l) {
            uint16_t *kl = k_pool + (size_t)l * layer_pool;
            uint16_t *vl = v_pool + (size_t)l * layer_pool;
            /* Norm, QKV GEMM, RoPE. */
            oracle_rmsnorm(x, w->attn_norm + (size_t)l * (size_t)H, H, dm->rms_eps, u);
            oracle_matvec(w->wqkv + (size_t)l * (size_t)QKV * (size_t)H, QKV, H, u, qkv);
            oracle_real *q = qkv, *k = qkv + (size_t)nq * (size_t)d,
                        *v = qkv + (size_t)(nq + nkv) * (size_t)d;
            oracle_rope(q, nq, d, p, dm->rope_theta);
            oracle_rope(k, nkv, d, p, dm->rope_theta);
            /* Reading: the cache holds rotated keys; the new entry is stored
             * as bf16 (round to nearest even of its binary32 value) before
             * the attention reads it, so the attention sees exactly what a
             * later step will read back. */
            for (int32_t g = 0; g < nkv; ++g) {
                size_t row = kv_row(dm, page_row, p, g);
                for (int32_t c = 0; c < d; ++c) {
                    kl[row + (size_t)c] = oracle_f32_to_bf16((float)k[(size_t)g * (size_t)d + (size_t)c]);
                    vl[row + (size_t)c] = oracle_f32_to_bf16((float)v[(size_t)g * (size_t)d + (size_t)c]);
                }
            }
            /* Attention. */
            oracle_attention(dm, q, kl, vl, page_row, p, o);
            /* Residual: x += W_o o. Reading: the O projection is part of the
             * attention block, added to the residual stream ("residual" in
             * the op chain of [bubbles]). */
            oracle_matvec(w->wo + (size_t)l * (size_t)H * (size_t)(nq * d), H, nq * d, o, t);
            for (int32_t i = 0; i < H; ++i)
                x[i] += t[i];
            /* MLP: norm, gate and up projections, SiLU gating, down
             * projection, residual. */
            oracle_rmsnorm(x, w->mlp_norm + (size_t)l * (size_t)H, H, dm->rms_eps, u);
            oracle_matvec(w->w_gate + (size_t)l * (size_t)F * (size_t)H, F, H, u, gt);
            oracle_matvec(w->w_up + (size_t)l * (size_t)F * (size_t)H, F, H, u, up);
            for (int32_t i = 0; i < F; ++i)
                gt[i] = oracle_silu(gt[i]) * up[i];
            oracle_matvec(w->w_down + (size_t)l * (size_t)H * (size_t)F, H, F, gt, t);
            for (int32_t i = 0; i < H; ++i)
                x[i] += t[i];
        }

        if (hidden_out)
            for (int32_t i = 0; i < H; ++i)
                hidden_out[(size_t)b * (size_t)H + (size_t)i] = x[i];

        if (dm->has_embed) {
            /* LM_HEAD ([flow]) with the final norm; the head is the
             * embedding table (tied). Then greedy sampling. */
            oracle_rmsnorm(x, w->final_norm, H, dm->rms_eps, u);
            oracle_matvec(w->embed, V, H, u, logits);
            if (logits_out)
                for (int32_t i = 0; i < V; ++i)
                    logits_out[(size_t)b * (size_t)V + (size_t)i] = logits[i];
            int32_t tok = oracle_argmax(logits, V);
            if (tok < 0)
                rc = -2;
            if (tokens_out)
                tokens_out[b] = tok;
        }
    }

    free(x); free(u); free(qkv); free(o); free(t); free(gt); free(up); free(logits);
    return rc;
}
