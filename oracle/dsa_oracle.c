/*
 * CPU oracle for the DeepSeek-V3.2 sparse-attention hot path.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU library.  Plain loops in
 * fp64, no blocking, no fusion, no reordering beyond the definitions below.
 * The readings taken where the pages are silent are listed in dsa_oracle.h.
 */
#include "dsa_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* storage formats -> exact fp64 values                                      */
/* ------------------------------------------------------------------------ */

static double bf16_value(uint16_t bits) {
  uint32_t u = (uint32_t)bits << 16;
  float f;
  memcpy(&f, &u, sizeof f);
  return (double)f;
}

/* OCP E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits; the
 * all-ones exponent with all-ones mantissa is NaN; there is no infinity. */
static double e4m3_value(uint8_t code) {
  int sign = (code >> 7) & 1;
  int e = (code >> 3) & 0xF;
  int m = code & 0x7;
  double v;
  if (e == 0xF && m == 0x7) return NAN;
  if (e == 0)
    v = ldexp((double)m / 8.0, -6);
  else
    v = ldexp(1.0 + (double)m / 8.0, e - 7);
  return sign ? -v : v;
}

/* ue8m0 scale byte: 2^(byte - 127); 0xFF is NaN */
static double ue8m0_value(uint8_t byte) {
  if (byte == 0xFF) return NAN;
  return ldexp(1.0, (int)byte - 127);
}

/* Element i of a tensor stored as dtype (fp8 handled by the caller). */
static double load_value(const void* base, int dtype, int64_t i) {
  if (dtype == DSA_ORC_F32) return (double)((const float*)base)[i];
  return bf16_value(((const uint16_t*)base)[i]);
}

/* Element i of an indexer tensor; fp8 applies its 128-block scale. */
static double load_index_value(const void* base, const uint8_t* sf, int dtype,
                               int64_t row, int32_t width, int32_t d) {
  int64_t i = row * width + d;
  if (dtype == DSA_ORC_FP8) {
    int32_t nblk = width / 128;
    return e4m3_value(((const uint8_t*)base)[i]) * ue8m0_value(sf[row * nblk + d / 128]);
  }
  return load_value(base, dtype, i);
}

static int check_shape(const orc_shape* sh) {
  if (!sh) return 1;
  if (sh->B <= 0 || sh->T <= 0 || sh->S <= 0 || sh->T > sh->S) return 1;
  if (sh->HI <= 0 || sh->DI <= 0 || sh->H <= 0 || sh->Dc <= 0 || sh->Dr < 0) return 1;
  if (sh->K <= 0) return 1;
  if (sh->idx_dtype == DSA_ORC_FP8 && sh->DI % 128 != 0) return 1;
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Index score (MoE-block step list: S^I, then S~^I = S^I + M)               */
/* ------------------------------------------------------------------------ */

/* Sequence b holds L_b valid keys at positions 0 .. L_b - 1 (L_b = S when
 * seq_lens is NULL); its T queries are the last T positions, q_pos(t) =
 * L_b - T + t, and key s is visible when s <= q_pos(t) (so never when
 * s >= L_b).  A query with q_pos < 0 sees no key. */
int orc_indexer_scores_ragged(const orc_shape* sh, int32_t n, const int32_t* row_b,
                              const int32_t* row_t, const int32_t* seq_lens,
                              const void* q_idx_rows, const uint8_t* q_sf_rows,
                              const void* k_idx, const uint8_t* k_sf, const void* w_rows,
                              float* scores) {
  if (check_shape(sh) || n < 0) return 1;
  const int32_t S = sh->S, HI = sh->HI, DI = sh->DI;
  for (int32_t r = 0; r < n; ++r) {
    const int32_t b = row_b[r], t = row_t[r];
    if (b < 0 || b >= sh->B || t < 0 || t >= sh->T) return 1;
    const int32_t L = seq_lens ? seq_lens[b] : S;
    if (L < 0 || L > S) return 1;
    const int32_t q_pos = L - sh->T + t;
    for (int32_t s = 0; s < S; ++s) {
      if (s > q_pos) { /* causal mask M: a future key (or past the sequence) */
        scores[(int64_t)r * S + s] = -INFINITY;
        continue;
      }
      double acc = 0.0; /* sum_h w[t,h] * ReLU(Q^I[h,t] . k^I[s]) */
      for (int32_t h = 0; h < HI; ++h) {
        double dot = 0.0;
        for (int32_t d = 0; d < DI; ++d) {
          double qv = load_index_value(q_idx_rows, q_sf_rows, sh->idx_dtype,
                                       (int64_t)r * HI + h, DI, d);
          double kvv = load_index_value(k_idx, k_sf, sh->idx_dtype,
                                        (int64_t)b * S + s, DI, d);
          dot += qv * kvv;
        }
        double relu = dot > 0.0 ? dot : 0.0;
        double wv = load_value(w_rows, sh->w_dtype, (int64_t)r * HI + h);
        acc += wv * relu;
      }
      /* the prefactor is applied once, after the head sum, in fp32 */
      float accf = (float)acc;
      scores[(int64_t)r * S + s] = sh->idx_scale * accf;
    }
  }
  return 0;
}

int orc_indexer_scores(const orc_shape* sh, int32_t n, const int32_t* row_b,
                       const int32_t* row_t, const void* q_idx_rows,
                       const uint8_t* q_sf_rows, const void* k_idx,
                       const uint8_t* k_sf, const void* w_rows, float* scores) {
  return orc_indexer_scores_ragged(sh, n, row_b, row_t, NULL, q_idx_rows, q_sf_rows, k_idx,
                                   k_sf, w_rows, scores);
}

/* ------------------------------------------------------------------------ */
/* Top-K selection (MoE-block step list: M^sel keeps s in top_2048(S~^I_t))  */
/* ------------------------------------------------------------------------ */

typedef struct {
  float score;
  int32_t index;
} scored_key;

/* (score descending, index ascending); -0 == +0 because the comparison is on
 * values, not bits */
static int by_score_then_index(const void* pa, const void* pb) {
  const scored_key* a = (const scored_key*)pa;
  const scored_key* b = (const scored_key*)pb;
  if (a->score > b->score) return -1;
  if (a->score < b->score) return 1;
  return (a->index > b->index) - (a->index < b->index);
}

static int by_value(const void* pa, const void* pb) {
  int32_t a = *(const int32_t*)pa, b = *(const int32_t*)pb;
  return (a > b) - (a < b);
}

int orc_topk(const orc_shape* sh, int32_t n, const float* scores, int32_t* idx) {
  if (check_shape(sh) || n < 0) return 1;
  const int32_t S = sh->S;
  const int32_t Keff = sh->K < S ? sh->K : S;
  scored_key* cand = (scored_key*)malloc(sizeof(scored_key) * (size_t)S);
  if (!cand) return 1;
  for (int32_t r = 0; r < n; ++r) {
    const float* row = scores + (int64_t)r * S;
    int32_t m = 0;
    for (int32_t s = 0; s < S; ++s) {
      float v = row[s];
      if (isnan(v) || (isinf(v) && v < 0)) continue; /* never selectable */
      cand[m].score = v;
      cand[m].index = s;
      ++m;
    }
    qsort(cand, (size_t)m, sizeof(scored_key), by_score_then_index);
    int32_t take = m < Keff ? m : Keff;
    int32_t* out = idx + (int64_t)r * Keff;
    for (int32_t j = 0; j < take; ++j) out[j] = cand[j].index;
    qsort(out, (size_t)take, sizeof(int32_t), by_value);
    for (int32_t j = take; j < Keff; ++j) out[j] = -1;
  }
  free(cand);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Latent attention, absorbed form.                                          */
/* logit_j = sm_scale * (q[0:Dc] . c_j + q[Dc:Dc+Dr] . r_j) with the row      */
/* kv_j = [c_j ; r_j]; p = softmax over the index row; o = sum_j p_j c_j.    */
/* ------------------------------------------------------------------------ */

static double mla_logit(const orc_shape* sh, const void* q_rows, int64_t qrow,
                        const void* kv, int64_t kvrow) {
  const int32_t D = sh->Dc + sh->Dr;
  double dot = 0.0;
  for (int32_t d = 0; d < D; ++d) /* latent part and rotary part together */
    dot += load_value(q_rows, sh->mla_dtype, qrow * D + d) *
           load_value(kv, sh->mla_dtype, kvrow * D + d);
  return (double)sh->sm_scale * dot;
}

/* Softmax-weighted sum over a list of key rows (keys[j] < 0: skipped). */
static void attend(const orc_shape* sh, const void* q_rows, int64_t qrow,
                   const void* kv, int32_t b, const int32_t* keys, int32_t nk,
                   double* o, double* lse, double* probs, double* logit) {
  const int32_t S = sh->S, D = sh->Dc + sh->Dr, Dc = sh->Dc;
  double m = -INFINITY;
  for (int32_t j = 0; j < nk; ++j) {
    if (keys[j] < 0) continue;
    logit[j] = mla_logit(sh, q_rows, qrow, kv, (int64_t)b * S + keys[j]);
    if (logit[j] > m) m = logit[j];
  }
  for (int32_t d = 0; d < Dc; ++d) o[d] = 0.0;
  if (m == -INFINITY) { /* no valid key */
    *lse = -INFINITY;
    if (probs)
      for (int32_t j = 0; j < nk; ++j) probs[j] = 0.0;
    return;
  }
  double l = 0.0;
  for (int32_t j = 0; j < nk; ++j)
    if (keys[j] >= 0) l += exp(logit[j] - m);
  for (int32_t j = 0; j < nk; ++j) {
    double p = keys[j] >= 0 ? exp(logit[j] - m) / l : 0.0;
    if (probs) probs[j] = p;
    if (keys[j] < 0) continue;
    for (int32_t d = 0; d < Dc; ++d)
      o[d] += p * load_value(kv, sh->mla_dtype, ((int64_t)b * S + keys[j]) * D + d);
  }
  *lse = m + log(l);
}

int orc_sparse_mla(const orc_shape* sh, int32_t n, const int32_t* row_b,
                   const void* q_rows, const void* kv, const int32_t* idx,
                   int32_t W, double* o, double* lse, double* probs) {
  if (check_shape(sh) || n < 0 || W < 0) return 1;
  const int32_t H = sh->H, Dc = sh->Dc, S = sh->S;
  int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)(W > 0 ? W : 1));
  double* logit = (double*)malloc(sizeof(double) * (size_t)(W > 0 ? W : 1));
  if (!keys || !logit) { free(keys); free(logit); return 1; }
  for (int32_t r = 0; r < n; ++r) {
    const int32_t b = row_b[r];
    if (b < 0 || b >= sh->B) { free(keys); free(logit); return 1; }
    for (int32_t j = 0; j < W; ++j) { /* out-of-range entries are skipped */
      int32_t s = idx[(int64_t)r * W + j];
      keys[j] = (s >= 0 && s < S) ? s : -1;
    }
    for (int32_t h = 0; h < H; ++h) {
      int64_t qh = (int64_t)r * H + h;
      attend(sh, q_rows, qh, kv, b, keys, W, o + qh * Dc, lse + qh,
             probs ? probs + qh * W : NULL, logit);
    }
  }
  free(keys);
  free(logit);
  return 0;
}

int orc_dense_mla(const orc_shape* sh, int32_t n, const int32_t* row_b,
                  const int32_t* row_t, const void* q_rows, const void* kv,
                  double* o, double* lse) {
  if (check_shape(sh) || n < 0) return 1;
  const int32_t H = sh->H, Dc = sh->Dc, S = sh->S;
  int32_t* keys = (int32_t*)malloc(sizeof(int32_t) * (size_t)S);
  double* logit = (double*)malloc(sizeof(double) * (size_t)S);
  if (!keys || !logit) { free(keys); free(logit); return 1; }
  for (int32_t r = 0; r < n; ++r) {
    const int32_t b = row_b[r], t = row_t[r];
    if (b < 0 || b >= sh->B || t < 0 || t >= sh->T) { free(keys); free(logit); return 1; }
    const int32_t q_pos = S - sh->T + t;
    for (int32_t s = 0; s < S; ++s) keys[s] = s <= q_pos ? s : -1;
    for (int32_t h = 0; h < H; ++h) {
      int64_t qh = (int64_t)r * H + h;
      attend(sh, q_rows, qh, kv, b, keys, S, o + qh * Dc, lse + qh, NULL, logit);
    }
  }
  free(keys);
  free(logit);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Explicit latent attention (MoE-block step list): per head h,              */
/* K^C_h[s] = c_s W_UK,h ; V_h[s] = c_s W_UV,h ; K = [K^C_h ; r_s] ;          */
/* logits = sm_scale * (qC_h . K^C_h[s] + qR_h . r_s) ; out_h = sum p V_h.   */
/* ------------------------------------------------------------------------ */

int orc_explicit_mla(int32_t H, int32_t Dc, int32_t Dn, int32_t Dv, int32_t Dr,
                     int32_t nkeys, double sm_scale, const double* qC,
                     const double* qR, const double* c, const double* r,
                     const double* W_UK, const double* W_UV, double* out) {
  if (H <= 0 || Dc <= 0 || Dn <= 0 || Dv <= 0 || Dr < 0 || nkeys <= 0) return 1;
  double* logit = (double*)malloc(sizeof(double) * (size_t)nkeys);
  if (!logit) return 1;
  for (int32_t h = 0; h < H; ++h) {
    double m = -INFINITY;
    for (int32_t s = 0; s < nkeys; ++s) {
      double dot = 0.0;
      for (int32_t e = 0; e < Dn; ++e) {
        double kc = 0.0; /* K^C_h[s][e] = sum_d c[s][d] W_UK[d][h*Dn+e] */
        for (int32_t d = 0; d < Dc; ++d)
          kc += c[(int64_t)s * Dc + d] * W_UK[(int64_t)d * H * Dn + h * Dn + e];
        dot += qC[(int64_t)h * Dn + e] * kc;
      }
      for (int32_t e = 0; e < Dr; ++e)
        dot += qR[(int64_t)h * Dr + e] * r[(int64_t)s * Dr + e];
      logit[s] = sm_scale * dot;
      if (logit[s] > m) m = logit[s];
    }
    double l = 0.0;
    for (int32_t s = 0; s < nkeys; ++s) l += exp(logit[s] - m);
    for (int32_t e = 0; e < Dv; ++e) {
      double acc = 0.0;
      for (int32_t s = 0; s < nkeys; ++s) {
        double v = 0.0; /* V_h[s][e] = sum_d c[s][d] W_UV[d][h*Dv+e] */
        for (int32_t d = 0; d < Dc; ++d)
          v += c[(int64_t)s * Dc + d] * W_UV[(int64_t)d * H * Dv + h * Dv + e];
        acc += exp(logit[s] - m) / l * v;
      }
      out[(int64_t)h * Dv + e] = acc;
    }
  }
  free(logit);
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Cache fill and indexer inputs, the step before the path (MoE-block step   */
/* list: c^KV = x W_DKV, c^KV normalised, k^pe = x W_KR rotated, w = x W_w;  */
/* the indexer's key projection wk with k_norm, a LayerNorm with affine and  */
/* bias, from the nnterp deepseek_v32 module tree; the joint down-projection */
/* split [512, 64], then the latent norm and the key rotation, from the     */
/* mla-kv excerpt of the atlas "DeepSeek-V3.2-Exp . Attention input" page). */
/* ------------------------------------------------------------------------ */

#define ORC_FILL_LAT 512
#define ORC_FILL_ROPE 64
#define ORC_FILL_IDX 128
#define ORC_FILL_W 64
#define ORC_FILL_COLS (ORC_FILL_LAT + ORC_FILL_ROPE + ORC_FILL_IDX + ORC_FILL_W)
#define ORC_NORM_EPS 1e-6

int orc_cache_fill(int32_t n, int32_t D, const uint16_t* x, const uint16_t* W,
                   const float* kv_gamma, const float* k_gamma, const float* k_beta,
                   const float* rope_cos, const float* rope_sin, double* kv_out,
                   double* k_out, double* w_out) {
  if (n < 0 || D <= 0 || !x || !W || !kv_gamma || !k_gamma || !k_beta || !rope_cos ||
      !rope_sin || !kv_out || !k_out || !w_out)
    return 1;
  double p[ORC_FILL_COLS];
  for (int32_t t = 0; t < n; ++t) {
    /* the joint projection: p_j = sum_d x[d] W[j][d] */
    for (int32_t j = 0; j < ORC_FILL_COLS; ++j) {
      double acc = 0.0;
      for (int32_t d = 0; d < D; ++d)
        acc += bf16_value(x[(int64_t)t * D + d]) * bf16_value(W[(int64_t)j * D + d]);
      p[j] = acc;
    }
    double* kv = kv_out + (int64_t)t * (ORC_FILL_LAT + ORC_FILL_ROPE);
    /* c^KV: RMSNorm over the 512 latent dims, then the gain */
    double ms = 0.0;
    for (int32_t i = 0; i < ORC_FILL_LAT; ++i) ms += p[i] * p[i];
    ms /= ORC_FILL_LAT;
    const double inv_rms = 1.0 / sqrt(ms + ORC_NORM_EPS);
    for (int32_t i = 0; i < ORC_FILL_LAT; ++i) kv[i] = p[i] * inv_rms * kv_gamma[i];
    /* k^pe: pair (2i, 2i + 1) is turned by angle i of this token and lands in
     * rotary dims i and i + 32 */
    const double* kpe = p + ORC_FILL_LAT;
    for (int32_t i = 0; i < ORC_FILL_ROPE / 2; ++i) {
      const double c = rope_cos[(int64_t)t * (ORC_FILL_ROPE / 2) + i];
      const double s = rope_sin[(int64_t)t * (ORC_FILL_ROPE / 2) + i];
      const double a = kpe[2 * i], b = kpe[2 * i + 1];
      kv[ORC_FILL_LAT + i] = a * c - b * s;
      kv[ORC_FILL_LAT + ORC_FILL_ROPE / 2 + i] = a * s + b * c;
    }
    /* k^I: LayerNorm over its 128 dims (population variance), gain and bias */
    const double* y = p + ORC_FILL_LAT + ORC_FILL_ROPE;
    double mean = 0.0;
    for (int32_t i = 0; i < ORC_FILL_IDX; ++i) mean += y[i];
    mean /= ORC_FILL_IDX;
    double var = 0.0;
    for (int32_t i = 0; i < ORC_FILL_IDX; ++i) var += (y[i] - mean) * (y[i] - mean);
    var /= ORC_FILL_IDX;
    const double inv_std = 1.0 / sqrt(var + ORC_NORM_EPS);
    for (int32_t i = 0; i < ORC_FILL_IDX; ++i)
      k_out[(int64_t)t * ORC_FILL_IDX + i] = (y[i] - mean) * inv_std * k_gamma[i] + k_beta[i];
    /* w: the head weights, as projected */
    for (int32_t i = 0; i < ORC_FILL_W; ++i)
      w_out[(int64_t)t * ORC_FILL_W + i] = p[ORC_FILL_LAT + ORC_FILL_ROPE + ORC_FILL_IDX + i];
  }
  return 0;
}

/* OCP E4M3FN code of |v| <= 448, round to nearest, ties to the even code */
static uint8_t e4m3_code_of(double v) {
  const uint8_t sign = (v < 0 || (v == 0 && signbit(v))) ? 0x80 : 0x00;
  double a = fabs(v);
  if (a >= 448.0) return sign | 0x7E;
  if (a < ldexp(1.0, -6)) { /* subnormal: steps of 2^-9 */
    const double q = a * 512.0;
    double r = floor(q);
    const double f = q - r;
    if (f > 0.5 || (f == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
    return sign | (uint8_t)r; /* r == 8 is the smallest normal, code 0x08 */
  }
  int e;
  const double m = frexp(a, &e); /* a = m 2^e, m in [0.5, 1) */
  int E = e - 1;                 /* a = (2m) 2^E, 2m in [1, 2) */
  const double q = (2.0 * m - 1.0) * 8.0;
  double r = floor(q);
  const double f = q - r;
  if (f > 0.5 || (f == 0.5 && fmod(r, 2.0) != 0.0)) r += 1.0;
  if (r == 8.0) { r = 0.0; ++E; }
  if (E + 7 > 15 || (E + 7 == 15 && r == 7.0)) return sign | 0x7E;
  return sign | (uint8_t)(((E + 7) << 3) | (int)r);
}

int orc_quantize_e4m3_block(const double* y, int32_t len, uint8_t* codes, uint8_t* scale_byte) {
  if (!y || !codes || !scale_byte || len <= 0) return 1;
  double amax = 0.0;
  for (int32_t i = 0; i < len; ++i) amax = fmax(amax, fabs(y[i]));
  /* the smallest e with 448 2^e >= amax (0 for an all-zero block), held    */
  /* to the range of the scale byte e + 127: never below -127 (a block whose */
  /* largest magnitude is under 448 2^-127 keeps the scale 2^-127)           */
  int e = 0;
  if (amax > 0.0) {
    e = (int)ceil(log2(amax / 448.0));
    while (ldexp(448.0, e - 1) >= amax) --e;
    while (ldexp(448.0, e) < amax) ++e;
    if (e < -127) e = -127;
  }
  *scale_byte = (uint8_t)(e + 127);
  for (int32_t i = 0; i < len; ++i) codes[i] = e4m3_code_of(ldexp(y[i], -e));
  return 0;
}

/* The indexer query: Q^I = c^Q wq_b (the indexer's wq_b in the nnterp
 * deepseek_v32 module tree), per token, fp64 sums of exact products. */
int orc_indexer_query(int32_t n, int32_t Dq, const uint16_t* cq, const uint16_t* wq_b,
                      int32_t out_dim, double* q) {
  if (n < 0 || Dq <= 0 || out_dim <= 0 || !cq || !wq_b || !q) return 1;
  for (int32_t t = 0; t < n; ++t)
    for (int32_t j = 0; j < out_dim; ++j) {
      double acc = 0.0;
      for (int32_t d = 0; d < Dq; ++d)
        acc += bf16_value(cq[(int64_t)t * Dq + d]) * bf16_value(wq_b[(int64_t)j * Dq + d]);
      q[(int64_t)t * out_dim + j] = acc;
    }
  return 0;
}

/* ------------------------------------------------------------------------ */
/* Absorption either side of the sparse attention.                          */

int orc_absorb_query(int32_t n, int32_t H, int32_t Dc, int32_t Dn, int32_t Dv, int32_t Dr,
                     const double* qb, const double* kv_b, const double* rope_cos,
                     const double* rope_sin, double* q) {
  if (n < 0 || H <= 0 || Dc <= 0 || Dn <= 0 || Dv <= 0 || Dr < 0 || Dr % 2) return 1;
  const int32_t in_w = Dn + Dr, out_w = Dc + Dr, head_rows = Dn + Dv;
  for (int32_t t = 0; t < n; ++t)
    for (int32_t h = 0; h < H; ++h) {
      const double* qc = qb + ((int64_t)t * H + h) * in_w;
      double* qo = q + ((int64_t)t * H + h) * out_w;
      /* latent part: the head's q^C through its key half of kv_b */
      for (int32_t c = 0; c < Dc; ++c) {
        double acc = 0.0;
        for (int32_t e = 0; e < Dn; ++e)
          acc += qc[e] * kv_b[((int64_t)h * head_rows + e) * Dc + c];
        qo[c] = acc;
      }
      /* rotary part: pair (2i, 2i+1) of q^pe turned by angle i */
      const double* pe = qc + Dn;
      for (int32_t i = 0; i < Dr / 2; ++i) {
        const double cs = rope_cos[(int64_t)t * (Dr / 2) + i];
        const double sn = rope_sin[(int64_t)t * (Dr / 2) + i];
        const double a = pe[2 * i], b = pe[2 * i + 1];
        qo[Dc + i] = a * cs - b * sn;
        qo[Dc + Dr / 2 + i] = a * sn + b * cs;
      }
    }
  return 0;
}

int orc_absorb_output(int32_t n, int32_t H, int32_t Dc, int32_t Dn, int32_t Dv,
                      const double* o, const double* kv_b, double* out) {
  if (n < 0 || H <= 0 || Dc <= 0 || Dn <= 0 || Dv <= 0) return 1;
  const int32_t head_rows = Dn + Dv;
  for (int32_t t = 0; t < n; ++t)
    for (int32_t h = 0; h < H; ++h) {
      const double* ol = o + ((int64_t)t * H + h) * Dc;
      for (int32_t d = 0; d < Dv; ++d) {
        /* the head's value half of kv_b: rows after its Dn key rows */
        const double* wv = kv_b + ((int64_t)h * head_rows + Dn + d) * Dc;
        double acc = 0.0;
        for (int32_t c = 0; c < Dc; ++c) acc += ol[c] * wv[c];
        out[((int64_t)t * H + h) * Dv + d] = acc;
      }
    }
  return 0;
}

int orc_linear_bf16(int32_t n, int32_t Din, int32_t Dout, const uint16_t* x, const uint16_t* W,
                    double* out) {
  if (n < 0 || Din <= 0 || Dout <= 0 || !x || !W || !out) return 1;
  for (int32_t t = 0; t < n; ++t)
    for (int32_t j = 0; j < Dout; ++j) {
      double acc = 0.0;
      for (int32_t i = 0; i < Din; ++i)
        acc += bf16_value(x[(int64_t)t * Din + i]) * bf16_value(W[(int64_t)j * Din + i]);
      out[(int64_t)t * Dout + j] = acc;
    }
  return 0;
}
