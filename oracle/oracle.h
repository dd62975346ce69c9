/* oracle.h - interface of the CPU oracle for one decode step of a
 * Llama-style dense decoder.
 *
 * TEST INFRASTRUCTURE ONLY. Only tests, the smoke check and the benchmark's
 * CPU-baseline leg may load this library. The product path (the HIP library
 * under persistent_megakernel_decode_cu_amd/) never links, imports or calls
 * it, and this file shares no code or header with it.
 *
 * What is computed follows "Inference MegaKernel" (shaojiemike.top):
 *   - section "why conventional inference still has bubbles": the op chain
 *     Norm -> QKV GEMM -> RoPE -> Attention -> residual -> MLP -> sampling;
 *   - section "hand-written whole-model MegaKernel / principle, schedule and
 *     dataflow": the op bodies RMS_NORM, QKV_MATVEC, ATTENTION, MLP_UP_GATE,
 *     MLP_DOWN, LM_HEAD of the interpreter, and the object table (weights
 *     fixed in HBM, per-layer paged K/V cache owned by the request).
 * The page does not spell out the Llama arithmetic; every such detail is a
 * reading, listed where it is used in oracle.c.
 *
 * Scalar type: `oracle_real` is double unless ORACLE_REAL_FLOAT is defined,
 * in which case the same source builds a single-precision variant.
 */
#ifndef MK_ORACLE_H
#define MK_ORACLE_H

#include <stdint.h>

#ifdef ORACLE_REAL_FLOAT
typedef float oracle_real;
#else
typedef double oracle_real;
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Model shape. `has_embed` = 1: the input is a token id, the embedding
 * table is also the LM head (tied), and the step ends with logits and the
 * greedy token. `has_embed` = 0: the input is a hidden vector, there is no
 * head, and the step ends with the residual stream (one-layer block case). */
typedef struct oracle_dims {
    int32_t n_layers, hidden, n_q_heads, n_kv_heads, head_dim, ffn, vocab;
    int32_t has_embed;
    int32_t page_tokens;          /* KV positions per page (16) */
    int32_t max_pages_per_req;    /* columns of the page table */
    int32_t n_pages;              /* pages per layer in the K and V pools */
    double rms_eps, rope_theta;
} oracle_dims;

/* bf16 weights (raw uint16 bit patterns), row-major [out, in], stacked over
 * layers. Rows of wqkv are [q heads | k heads | v heads]. */
typedef struct oracle_weights {
    const uint16_t *embed;        /* [V, H] or NULL */
    const uint16_t *final_norm;   /* [H] or NULL */
    const uint16_t *attn_norm;    /* [L, H] */
    const uint16_t *wqkv;         /* [L, (nq + 2 nkv) d, H] */
    const uint16_t *wo;           /* [L, H, nq d] */
    const uint16_t *mlp_norm;     /* [L, H] */
    const uint16_t *w_gate;       /* [L, F, H] */
    const uint16_t *w_up;         /* [L, F, H] */
    const uint16_t *w_down;       /* [L, H, F] */
} oracle_weights;

/* bf16 <-> binary32 */
float    oracle_bf16_to_f32(uint16_t h);
uint16_t oracle_f32_to_bf16(float f);

/* Single ops, each on plain contiguous vectors. */
void oracle_rmsnorm(const oracle_real *x, const uint16_t *w, int32_t n,
                    double eps, oracle_real *out);
void oracle_matvec(const uint16_t *W, int32_t rows, int32_t cols,
                   const oracle_real *x, oracle_real *y);
void oracle_rope(oracle_real *v, int32_t n_heads, int32_t head_dim,
                 int32_t pos, double theta);
oracle_real oracle_silu(oracle_real z);
int32_t oracle_argmax(const oracle_real *v, int32_t n);

/* Decode attention of one request in one layer. q: [nq, d], already rotated.
 * The cache rows for positions 0..pos (inclusive) are read from the pools
 * through `page_row` (this request's row of the page table). out: [nq, d]. */
void oracle_attention(const oracle_dims *dims, const oracle_real *q,
                      const uint16_t *k_layer, const uint16_t *v_layer,
                      const int32_t *page_row, int32_t pos,
                      oracle_real *out);

/* One decode step for a batch of B requests. k_pool/v_pool are
 * [L, n_pages, nkv, page_tokens, d] bf16 and receive the new entry of every
 * request at position kv_lens[b]. Outputs may be NULL except tokens_out when
 * has_embed = 1. Returns 0, or a negative code: -1 invalid lengths or page
 * table entry, -2 a NaN logit. */
int32_t oracle_decode_step(const oracle_dims *dims, const oracle_weights *w,
                           uint16_t *k_pool, uint16_t *v_pool,
                           const int32_t *page_table, int32_t batch,
                           const int32_t *tokens_in,
                           const oracle_real *hidden_in,
                           const int32_t *kv_lens,
                           oracle_real *logits_out, oracle_real *hidden_out,
                           int32_t *tokens_out);

#ifdef __cplusplus
}
#endif
#endif
