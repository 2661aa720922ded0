/*
 * CPU oracle for the DeepSeek-V3.2 sparse-attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  This is the plain, slow, obviously-correct
 * statement of what the hot path computes, written from the pages in fp64.
 * Only the test-suite, the smoke check and the benchmark's CPU-baseline leg
 * may load it.  It shares no source, header, table or helper with the GPU
 * library, and the GPU library never calls it.
 *
 * Sources (the pages this follows):
 *  - atlas.klimoza.dev, DeepSeek-V3.2-Exp, MoE block, "All 43 steps": the index
 *    score S^I = 1/(sqrt 64 * sqrt 128) * sum_h w_{t,h} ReLU(Q^I_{h,t} . k^I_s),
 *    the causal mask M added to it, and the top-2048 selection mask M^sel.
 *  - nnterp encyclopedia, deepseek_v32, section 03 ("Up to 2048 tokens the
 *    sparse attention is plain causal attention") and section 04: unselected
 *    keys get zero probability, rows sum to one over the selection, the
 *    selection is int32 [batch, query, min(index_topk, keys)].
 *  - the same MoE-block step list for latent attention: k^C = c^KV W_UK,
 *    v = c^KV W_UV, K_i = [K^C_i ; k^R] with one rotary key shared by all heads.
 *
 * Conventions (readings where the pages are silent):
 *  - query t of a sequence sits at position q_pos(t) = S - T + t and sees keys
 *    s <= q_pos(t) (the diagonal included);
 *  - top-K orders by (score descending, index ascending); -0 equals +0; NaN and
 *    -inf are never selected; the chosen indices are written in ascending
 *    order and the row is padded with -1 up to min(K, S);
 *  - the index scale is applied after the head sum, in fp32;
 *  - sparse attention over an index row skips entries that are -1 or outside
 *    [0, S) and counts duplicates as given; a row with no valid entry yields
 *    o = 0 and lse = -inf.
 *
 * Data types: DSA_ORC_F32 = 0, DSA_ORC_BF16 = 1 (uint16 bit patterns),
 * DSA_ORC_FP8 = 2 (OCP E4M3FN bytes with one ue8m0 scale byte per 128-element
 * block; value = e4m3 * 2^(byte - 127)).
 *
 * Row-list calling convention: each routine works on n query rows; row r of
 * the call is query (row_b[r], row_t[r]).  Per-query inputs (q_idx, w, q) and
 * outputs are passed compactly, [n, ...]; per-sequence tensors (k_idx, kv) are
 * passed whole, [B, S, ...].  All routines return 0 on success, nonzero on a
 * bad argument.
 */
#ifndef DSA_ORACLE_H
#define DSA_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { DSA_ORC_F32 = 0, DSA_ORC_BF16 = 1, DSA_ORC_FP8 = 2 };

typedef struct {
  int32_t B, T, S;      /* batch, queries per sequence, keys per sequence */
  int32_t HI, DI;       /* indexer heads, indexer head width */
  int32_t H, Dc, Dr;    /* MLA heads, latent width, rotary width */
  int32_t K;            /* top-k */
  float idx_scale;      /* index-score prefactor */
  float sm_scale;       /* softmax scale */
  int32_t idx_dtype;    /* q_idx / k_idx */
  int32_t w_dtype;      /* w */
  int32_t mla_dtype;    /* q / kv */
} orc_shape;

/* Index scores, [n, S] fp32, future keys -inf. */
int orc_indexer_scores(const orc_shape* sh, int32_t n, const int32_t* row_b,
                       const int32_t* row_t, const void* q_idx_rows,
                       const uint8_t* q_sf_rows, const void* k_idx,
                       const uint8_t* k_sf, const void* w_rows, float* scores);

/* The same with per-sequence context lengths (ragged batch; the padding mask
 * of the nnterp page, section 02): sequence b has seq_lens[b] <= S valid keys
 * and its queries sit at q_pos(t) = seq_lens[b] - T + t.  seq_lens NULL: all S. */
int orc_indexer_scores_ragged(const orc_shape* sh, int32_t n, const int32_t* row_b,
                              const int32_t* row_t, const int32_t* seq_lens,
                              const void* q_idx_rows, const uint8_t* q_sf_rows,
                              const void* k_idx, const uint8_t* k_sf, const void* w_rows,
                              float* scores);

/* Top-K selection of n score rows of length S -> [n, min(K, S)] int32. */
int orc_topk(const orc_shape* sh, int32_t n, const float* scores, int32_t* idx);

/* Absorbed sparse latent attention over index rows of width W.
 * o [n, H, Dc] fp64, lse [n, H] fp64, probs [n, H, W] fp64 (nullable). */
int orc_sparse_mla(const orc_shape* sh, int32_t n, const int32_t* row_b,
                   const void* q_rows, const void* kv, const int32_t* idx,
                   int32_t W, double* o, double* lse, double* probs);

/* Dense causal latent attention over every key s <= q_pos(t).
 * o [n, H, Dc] fp64, lse [n, H] fp64. */
int orc_dense_mla(const orc_shape* sh, int32_t n, const int32_t* row_b,
                  const int32_t* row_t, const void* q_rows, const void* kv,
                  double* o, double* lse);

/* Explicit (non-absorbed) latent attention of one query over nkeys keys, fp64.
 * qC [H, Dn], qR [H, Dr], c [nkeys, Dc], r [nkeys, Dr],
 * W_UK [Dc, H*Dn] and W_UV [Dc, H*Dv] (column block h belongs to head h).
 * out [H, Dv]. */
int orc_explicit_mla(int32_t H, int32_t Dc, int32_t Dn, int32_t Dv, int32_t Dr,
                     int32_t nkeys, double sm_scale, const double* qC,
                     const double* qR, const double* c, const double* r,
                     const double* W_UK, const double* W_UV, double* out);

/* Cache fill and indexer inputs for n tokens (the step before the path).
 * x [n, D] bf16 hidden states; W [768, D] bf16 joint projection in Linear
 * layout, rows 0-511 the latent down-projection W_DKV, 512-575 the rotary key
 * W_KR, 576-703 the indexer key wk, 704-767 the head-weight projection W_w.
 * With p = W x (fp64 sums of exact products) and eps = 1e-6:
 *   kv_out [n, 576] = [ RMSNorm(p[0:512]) * kv_gamma ;
 *                       rotary part: pair (2i, 2i+1) of p[512:576] turned by
 *                       (rope_cos[t, i], rope_sin[t, i]) into dims i, i + 32 ]
 *   k_out [n, 128]  = LayerNorm(p[576:704]) * k_gamma + k_beta
 *   w_out [n, 64]   = p[704:768]
 * The rotation angles are the caller's (rope_cos / rope_sin [n, 32]). */
int orc_cache_fill(int32_t n, int32_t D, const uint16_t* x, const uint16_t* W,
                   const float* kv_gamma, const float* k_gamma, const float* k_beta,
                   const float* rope_cos, const float* rope_sin, double* kv_out,
                   double* k_out, double* w_out);

/* ue8m0 + OCP E4M3FN quantisation of one block of len values: the scale is
 * 2^e with e the smallest integer such that 448 2^e >= max |y| (byte e + 127;
 * an all-zero block gets byte 127), and each code is y / 2^e rounded to the
 * nearest E4M3 value, ties to the even code. */
int orc_quantize_e4m3_block(const double* y, int32_t len, uint8_t* codes, uint8_t* scale_byte);

/* The indexer query Q^I = c^Q wq_b of n tokens: cq [n, Dq] and wq_b
 * [out_dim, Dq] bf16 (Linear layout; out_dim = 64 heads x 128, row 128 h + d
 * is head h, dim d), q [n, out_dim] fp64. */
int orc_indexer_query(int32_t n, int32_t Dq, const uint16_t* cq, const uint16_t* wq_b,
                      int32_t out_dim, double* q);

/* Absorption either side of the sparse attention (the MoE-block step list:
 * k^C = c^KV W_UK and v = c^KV W_UV; the nnterp module tree's kv_b_proj
 * 512 -> heads x (key dims + value dims)).  kv_b is kv_b_proj's Linear
 * weight [H (Dn + Dv), Dc]: rows h (Dn + Dv) + e, e < Dn, are head h's key
 * dims, the next Dv rows its value dims.  All values fp64.
 *
 * orc_absorb_query: qb [n, H, Dn + Dr] (q^C then q^pe per head), rope_cos and
 * rope_sin [n, Dr / 2]; q [n, H, Dc + Dr]: q[t,h,c] = sum_e q^C[e] kv_b[h (Dn
 * + Dv) + e][c], then pair (2i, 2i+1) of q^pe turned by angle i into dims
 * Dc + i and Dc + Dr/2 + i (the cached rotary key's layout). */
int orc_absorb_query(int32_t n, int32_t H, int32_t Dc, int32_t Dn, int32_t Dv, int32_t Dr,
                     const double* qb, const double* kv_b, const double* rope_cos,
                     const double* rope_sin, double* q);

/* orc_absorb_output: o [n, H, Dc] latent contexts; out [n, H Dv] with
 * out[t, h Dv + d] = sum_c o[t,h,c] kv_b[h (Dn + Dv) + Dn + d][c]. */
int orc_absorb_output(int32_t n, int32_t H, int32_t Dc, int32_t Dn, int32_t Dv,
                      const double* o, const double* kv_b, double* out);

/* A Linear layer on bf16 operands (o_proj / wo): out [n, Dout] =
 * x [n, Din] W^T with W [Dout, Din]; fp64 sums of exact products. */
int orc_linear_bf16(int32_t n, int32_t Din, int32_t Dout, const uint16_t* x, const uint16_t* W,
                    double* out);

#ifdef __cplusplus
}
#endif
#endif
