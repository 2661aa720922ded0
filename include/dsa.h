/*
 * libdsa: DeepSeek-V3.2 sparse attention hot path on AMD Instinct MI355X
 * (gfx950).  Lightning-indexer scores -> per-query top-K -> absorbed sparse
 * latent attention, as hand-written HIP kernels behind a plain C ABI.
 *
 * Where each operation is defined:
 *  - index score and causal mask: atlas.klimoza.dev, DeepSeek-V3.2-Exp, MoE
 *    block, "All 43 steps": S^I_{t,s} = 1/(sqrt 64 sqrt 128) sum_h w_{t,h}
 *    ReLU(Q^I_{h,t} . k^I_s); S~^I = S^I + M;
 *  - selection: the same step list, M^sel keeps s in top_2048(S~^I_t); the
 *    nnterp deepseek_v32 page, section 03, gives the result's layout, int32
 *    [batch, query, min(index_topk, keys)];
 *  - sparse latent attention: the same step list (k^C = c^KV W_UK, v = c^KV
 *    W_UV, K_i = [K^C_i ; k^R], the same rotary key for every head), taken in
 *    absorbed form (q_lat_h = W_UK,h q^C_h, output = per-head 512-wide latent
 *    context before W_UV), with the nnterp deepseek_v32 semantics of section
 *    03/04: zero probability outside the selection, rows summing to one over
 *    it, a written index list used as written.
 *
 * Conventions shared by every entry point:
 *  - Memory.  Every tensor pointer is caller-owned DEVICE memory, row-major
 *    and contiguous, 16-byte aligned.  The library allocates nothing; scratch
 *    comes from the caller's workspace, sized by dsa_workspace_bytes().
 *  - Streams.  Work is enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream).  Calls return after enqueueing: results are valid once the
 *    stream has reached them.  No call synchronises the host.
 *  - Positions.  Query t of a sequence sits at position q_pos(t) = S - T + t
 *    and sees keys s <= q_pos(t).  Decode is T = 1 (sees all S keys); causal
 *    prefill is T = S.
 *  - Errors.  A call returns DSA_OK or an error code and enqueues nothing on
 *    error (argument errors are detected on the host before any launch).
 *    dsa_last_error() gives a thread-local message for the last failure.
 *  - Outputs are fully overwritten, so a failed call can simply be repeated.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The enumerations cross the ABI as 32-bit integers.  Compiled as C++ they
 * have a fixed int32_t underlying type, so every int32 value a caller passes
 * is a value of the type (an unknown one is rejected by the call). */
#ifdef __cplusplus
#define DSA_ENUM(tag) enum tag : int32_t
#else
#define DSA_ENUM(tag) enum tag
#endif

typedef DSA_ENUM(dsa_status_e) {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = 1, /* null pointer, bad size, misaligned pointer */
  DSA_ERR_UNSUPPORTED = 2, /* dtype or shape combination without a kernel */
  DSA_ERR_WORKSPACE = 3,   /* workspace missing or too small */
  DSA_ERR_HIP = 4          /* a HIP runtime call or launch failed */
} dsa_status_t;

typedef DSA_ENUM(dsa_dtype_e) {
  DSA_F32 = 0,
  DSA_BF16 = 1,
  DSA_FP8_E4M3 = 2 /* OCP E4M3FN bytes with one ue8m0 scale byte per 128 elements */
} dsa_dtype_t;

/* Problem description.  The DeepSeek-V3.2 sizes (config_671B_v3.2.json on the
 * atlas block-input page) are HI x DI = 64 x 128, H = 128, Dc = 512, Dr = 64,
 * K = 2048. */
typedef struct {
  int32_t B, T, S;   /* batch, queries per sequence, keys per sequence (T <= S) */
  int32_t HI, DI;    /* indexer heads and head width */
  int32_t H, Dc, Dr; /* latent-attention heads, latent width, rotary width */
  int32_t K;         /* top-k; rows hold K_eff = min(K, S) indices */
  float idx_scale;   /* index prefactor, 1/(sqrt(HI) sqrt(DI)) on the pages */
  float sm_scale;    /* softmax scale on the logits (1/sqrt(192) for the V3.2 head) */
  int32_t idx_dtype; /* dsa_dtype_t of q_idx and k_idx: F32, BF16 or FP8_E4M3 */
  int32_t w_dtype;   /* dsa_dtype_t of w: F32 or BF16 */
  int32_t mla_dtype; /* dsa_dtype_t of q, kv and o: F32 or BF16 */
} dsa_shape_t;

typedef DSA_ENUM(dsa_entry_e) {
  DSA_ENTRY_TOPK = 0,
  DSA_ENTRY_SPARSE_MLA = 1,
  DSA_ENTRY_FORWARD = 2,
  DSA_ENTRY_INDEXER_TOPK = 3
} dsa_entry_t;

/*
 * Index scores (the atlas MoE-block step list: S^I and the causal mask M).
 *   q_idx  [B, T, HI, DI]  idx_dtype
 *   q_sf   [B, T, HI, DI/128] uint8 ue8m0 scales (FP8 only, else NULL)
 *   k_idx  [B, S, DI]      idx_dtype
 *   k_sf   [B, S, DI/128]  uint8 ue8m0 scales (FP8 only, else NULL)
 *   w      [B, T, HI]      w_dtype
 *   scores [B, T, S]       fp32 output: idx_scale * sum_h w_h ReLU(q_h . k_s)
 *                          for s <= q_pos(t), -inf for future keys.
 * The head sum accumulates in fp32 and the prefactor multiplies it once, in
 * fp32.  FP8 requires DI % 128 == 0.
 */
dsa_status_t dsa_indexer_scores(const dsa_shape_t* shape, const void* q_idx,
                                const uint8_t* q_sf, const void* k_idx,
                                const uint8_t* k_sf, const void* w, float* scores,
                                void* stream);

/*
 * Index scores of a ragged batch: sequence b holds seq_lens[b] valid keys at
 * positions 0 .. seq_lens[b] - 1 of its S-row cache, and its T queries are its
 * last T positions, q_pos(t) = seq_lens[b] - T + t (the padding
 * attention_mask of the nnterp deepseek_v32 page, section 02, read as
 * per-sequence context lengths).  Key s is scored when s <= q_pos(t); every
 * other entry of the row, including those of keys past seq_lens[b], is -inf.
 *   seq_lens [B] int32, device memory, 4-byte aligned (NULL: every sequence
 *            holds S keys, which is dsa_indexer_scores); values are clamped
 *            to [0, S]; a query with q_pos(t) < 0 gets a row of -inf.
 * Other arguments and errors as dsa_indexer_scores.
 */
dsa_status_t dsa_indexer_scores_ragged(const dsa_shape_t* shape, const int32_t* seq_lens,
                                       const void* q_idx, const uint8_t* q_sf,
                                       const void* k_idx, const uint8_t* k_sf, const void* w,
                                       float* scores, void* stream);

/*
 * Top-K selection per score row (the step list's M^sel; layout from the
 * nnterp deepseek_v32 page, section 03).
 *   scores [B, T, S] fp32 (as written by dsa_indexer_scores, or any values)
 *   idx    [B, T, K_eff] int32 output, K_eff = min(K, S)
 * Selects the K_eff largest scores by (value descending, index ascending);
 * -0 equals +0; NaN and -inf are never selected.  Each row lists the chosen
 * indices in ascending order and is padded with -1 when fewer than K_eff
 * scores are selectable.  The result is exact (no approximation).
 * ws/ws_bytes: workspace of at least dsa_workspace_bytes(shape, DSA_ENTRY_TOPK)
 * bytes (may be NULL/0 when that is 0); its contents before the call do not
 * matter, and calls sharing one workspace must not overlap.  B*T <= 65535 and
 * S <= 8388608, else DSA_ERR_UNSUPPORTED before any launch.
 */
dsa_status_t dsa_topk(const dsa_shape_t* shape, const float* scores, int32_t* idx,
                      void* ws, size_t ws_bytes, void* stream);

/*
 * Index scores and top-K selection in one launch, for decode (the fused
 * streaming indexer -> top-K; the steps S^I + M and M^sel of the atlas
 * DeepSeek-V3.2-Exp MoE-block step list, layout from the nnterp deepseek_v32
 * page, section 03).  Covers the V3.2 indexer (HI = 64, DI = 128, BF16 or
 * FP8_E4M3 keys) with fewer than 8 queries per sequence and S <= 262144;
 * other shapes return DSA_ERR_UNSUPPORTED before any launch.
 *   q_idx, q_sf, k_idx, k_sf, w: as dsa_indexer_scores
 *   seq_lens: as dsa_indexer_scores_ragged (NULL: every sequence holds S keys)
 *   idx [B, T, K_eff] int32 output: exactly dsa_topk of the scores
 *       dsa_indexer_scores would give (same order, ties, padding)
 * ws: at least dsa_workspace_bytes(shape, DSA_ENTRY_INDEXER_TOPK) bytes; the
 * row scores ([B, T, S] fp32 at its start) stay there after the call, the
 * rest holds per-row counters and histograms, valid whatever the workspace
 * held before.  Calls sharing one workspace must not overlap.  Each key
 * block's workgroup stores its scores and adds its block's histogram to its
 * row's; the last one of the row selects (its row's scores are read back
 * once more, from the caches).
 */
dsa_status_t dsa_indexer_topk(const dsa_shape_t* shape, const int32_t* seq_lens,
                              const void* q_idx, const uint8_t* q_sf, const void* k_idx,
                              const uint8_t* k_sf, const void* w, int32_t* idx, void* ws,
                              size_t ws_bytes, void* stream);

/*
 * Sparse latent attention in absorbed form over the listed keys.
 *   q   [B, T, H, Dc+Dr] mla_dtype: per head, the absorbed latent query
 *       (W_UK,h q^C_h, Dc wide) followed by the rotary query (Dr wide)
 *   kv  [B, S, Dc+Dr]    mla_dtype: per key, the normalised latent c^KV (Dc)
 *       followed by the rotary key k^R (Dr), shared by all heads
 *   idx [B, T, K_eff]    int32 key indices; entries that are -1 or outside
 *       [0, S) are skipped; duplicates count as written
 *   o   [B, T, H, Dc]    mla_dtype output: sum_j p_j c_j with
 *       p = softmax_j(sm_scale * (q_lat . c_j + q_rot . r_j))
 *   lse [B, T, H]        fp32 output (nullable): log sum_j exp(logit_j)
 * A row with no valid index gives o = 0 and lse = -inf.  Accumulation is in
 * fp32.  ws: at least dsa_workspace_bytes(shape, DSA_ENTRY_SPARSE_MLA) bytes.
 * A build with -DDSA_DEBUG checks the rows on the device first and returns
 * DSA_ERR_INVALID_ARG for entries outside [-1, S) (it synchronizes the
 * stream to read the check back); its top-K entry points also check their
 * own output (entries in [-1, S), valid entries ascending, -1 padding last).
 */
dsa_status_t dsa_sparse_mla_fwd(const dsa_shape_t* shape, const void* q,
                                const void* kv, const int32_t* idx, void* o,
                                float* lse, void* ws, size_t ws_bytes, void* stream);

/*
 * The whole hot path: index scores -> top-K -> sparse latent attention.
 * Arguments as above; idx_out [B, T, K_eff] (nullable) receives the selection.
 * ws: at least dsa_workspace_bytes(shape, DSA_ENTRY_FORWARD) bytes (it holds
 * the [B, T, S] fp32 scores, the selection when idx_out is NULL, and the
 * scratch of the two later steps).
 */
dsa_status_t dsa_forward(const dsa_shape_t* shape, const void* q_idx,
                         const uint8_t* q_sf, const void* k_idx, const uint8_t* k_sf,
                         const void* w, const void* q, const void* kv,
                         int32_t* idx_out, void* o, float* lse, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * The whole hot path over a ragged batch: the index scores as
 * dsa_indexer_scores_ragged (seq_lens as there), then top-K (rows of a short
 * sequence are padded with -1 once its visible keys are exhausted) and the
 * sparse latent attention over the selection.  Other arguments, workspace and
 * errors as dsa_forward (same workspace size).
 */
dsa_status_t dsa_forward_ragged(const dsa_shape_t* shape, const int32_t* seq_lens,
                                const void* q_idx, const uint8_t* q_sf, const void* k_idx,
                                const uint8_t* k_sf, const void* w, const void* q, const void* kv,
                                int32_t* idx_out, void* o, float* lse, void* ws,
                                size_t ws_bytes, void* stream);

/*
 * dsa_forward for callers that cannot allocate device memory (code being
 * captured into a HIP graph, tight serving loops, harnesses that forbid
 * hipMalloc): the same computation with no ws argument.  Its scratch (the
 * scores, the selection when idx_out is NULL, the later steps' scratch) lives
 * in a device array that the library itself holds on every GPU it runs on:
 * 64 MiB (67108864 bytes), reserved when the library's code is loaded on that
 * GPU and kept until the process ends.  The call allocates nothing.
 *   - A shape whose dsa_workspace_bytes(shape, DSA_ENTRY_FORWARD) exceeds
 *     64 MiB returns DSA_ERR_WORKSPACE before any launch (every decode
 *     workload of the V3.2 shapes fits; a long prefill's [T, S] scores do not).
 *   - All calls on one GPU share that GPU's array: calls that may overlap on
 *     one GPU (several host threads, or several streams without an ordering
 *     between them) race and give undefined results.  Calls ordered on one
 *     stream are safe; nothing carries over from one call to the next.
 *   - The first call on a GPU looks up the array's device address
 *     (DSA_ERR_HIP if the runtime cannot give it).
 * Other arguments, results and errors as dsa_forward.
 */
dsa_status_t dsa_forward_noalloc(const dsa_shape_t* shape, const void* q_idx,
                                 const uint8_t* q_sf, const void* k_idx, const uint8_t* k_sf,
                                 const void* w, const void* q, const void* kv,
                                 int32_t* idx_out, void* o, float* lse, void* stream);

/*
 * Cache fill and indexer inputs for N new tokens, the step before the path
 * (atlas.klimoza.dev, DeepSeek-V3.2-Exp MoE block, "All 43 steps": c^KV =
 * x W_DKV and its RMSNorm, k^pe = x W_KR rotated, w = x W_w; the indexer key
 * wk with k_norm, a LayerNorm with gain and bias, from the nnterp
 * deepseek_v32 module tree; the [512, 64] split of the joint down-projection,
 * then the latent norm and the key rotation, from the mla-kv excerpt of the
 * atlas "DeepSeek-V3.2-Exp · Attention input" page).  With p = W x (fp32
 * accumulation):
 *   x         [N, D] bf16   the tokens' attention inputs; D % 64 == 0
 *   W         [768, D] bf16 joint projection in Linear layout (row j holds
 *             output j's weights): rows 0-511 W_DKV, 512-575 W_KR,
 *             576-703 wk, 704-767 W_w
 *   kv_gamma  [512] fp32    gain of the latent RMSNorm (eps 1e-6)
 *   k_gamma, k_beta [128] fp32  gain and bias of the indexer key LayerNorm
 *             (eps 1e-6, population variance)
 *   rope_cos, rope_sin [N, 32] fp32  the rotation of pair i for token n (the
 *             frequencies, YaRN or not, are the caller's)
 *   slots     [N] int64     the cache row each token fills (b * S + position
 *             for caches laid out [B, S, ...]); a negative slot skips the
 *             cache writes of that token.  Slots must be rows of the caches.
 *   kv_cache  [rows, 576] kv_dtype (BF16 or F32): row slots[n] receives
 *             [RMSNorm(p[0:512]) * kv_gamma ; p[512:576] with pair (2i, 2i+1)
 *             turned into dims i and i + 32, the layout the nnterp page
 *             states for this model]
 *   k_cache   [rows, 128] k_dtype (BF16, F32, or FP8_E4M3 codes):
 *             LayerNorm(p[576:704]) * k_gamma + k_beta; for FP8 the row's
 *             ue8m0 scale byte goes to k_sf[slots[n]] (2^e with e the smallest
 *             integer such that 448 2^e >= max |value|; codes round to
 *             nearest, ties to even)
 *   w_out     [N, 64] w_dtype (BF16 or F32): p[704:768], the head weights of
 *             the token's query
 * Every pointer is device memory, 16-byte aligned.  ws: at least
 * dsa_cache_fill_workspace_bytes(N, D) bytes (fp32 partial projections).
 * Errors as the other entry points (checked on the host before any launch).
 */
dsa_status_t dsa_cache_fill(int32_t N, int32_t D, const void* x, const void* W,
                            const float* kv_gamma, const float* k_gamma, const float* k_beta,
                            const float* rope_cos, const float* rope_sin, const int64_t* slots,
                            int32_t kv_dtype, void* kv_cache, int32_t k_dtype, void* k_cache,
                            uint8_t* k_sf, int32_t w_dtype, void* w_out, void* ws,
                            size_t ws_bytes, void* stream);
/* Workspace bytes of dsa_cache_fill on the current device ((size_t)-1 for
 * invalid sizes). */
size_t dsa_cache_fill_workspace_bytes(int32_t N, int32_t D);

/*
 * The indexer query of N tokens: Q^I = c^Q wq_b (the nnterp deepseek_v32
 * module tree: the indexer's wq_b maps the 1536-wide normalised query latent
 * to 64 heads x 128; the bar over Q^I in the score is read as this query).
 *   cq     [N, Dq] bf16      normalised query latents; Dq % 64 == 0 (1536)
 *   wq_b   [8192, Dq] bf16   Linear layout: row 128 h + d is head h, dim d
 *   q_out  [N, 64, 128] q_dtype (BF16, F32, or FP8_E4M3 codes), fp32
 *          accumulation; for FP8 each (token, head) row gets its ue8m0 scale in
 *          q_sf [N, 64] (the quantiser of dsa_cache_fill's keys)
 * Every pointer is device memory, 16-byte aligned.  ws: at least
 * dsa_indexer_query_workspace_bytes(N, Dq) bytes (fp32 partial projections).
 */
dsa_status_t dsa_indexer_query(int32_t N, int32_t Dq, const void* cq, const void* wq_b,
                               int32_t q_dtype, void* q_out, uint8_t* q_sf, void* ws,
                               size_t ws_bytes, void* stream);
/* Workspace bytes of dsa_indexer_query ((size_t)-1 for invalid sizes). */
size_t dsa_indexer_query_workspace_bytes(int32_t N, int32_t Dq);

/*
 * Absorption products either side of the sparse attention (the step list of
 * the atlas.klimoza.dev DeepSeek-V3.2-Exp page: k^C = c^KV W_UK and
 * v = c^KV W_UV; the nnterp deepseek_v32 module tree: kv_b_proj 512 ->
 * 32768 = 128 heads x (128 key dims + 128 value dims), q_b_proj's 192 per
 * head = 128 + 64 rotary, o_proj 16384 -> 7168).  Absorbed, head h's query
 * meets the latent rows through q_lat,h = W_UK,h q^C_h and its output
 * leaves through W_UV,h o_lat,h, then wo.
 *
 * kv_b is kv_b_proj's weight in Linear layout, [H * 256, 512] bf16: rows
 * 256 h .. 256 h + 127 are head h's key half, the next 128 its value half.
 * H is the number of heads the caller holds (128 for the whole model).
 */

/* W_UK in the form dsa_absorb_query reads: w_uk_t [H, 512, 128] bf16 with
 * w_uk_t[h][c][e] = kv_b[256 h + e][c] (a transpose, once per weight set).
 * Device pointers, 16-byte aligned; w_uk_t must not overlap kv_b. */
dsa_status_t dsa_absorb_prepare(int32_t H, const void* kv_b, void* w_uk_t, void* stream);

/*
 * The sparse attention's query of N tokens from q_b_proj's output:
 *   qb   [N, H, 192] bf16: per head q^C (128) then q^pe (64, pairs (2i, 2i+1))
 *   w_uk_t [H, 512, 128] bf16 from dsa_absorb_prepare
 *   rope_cos, rope_sin [N, 32] fp32: the rotation of pair i for token n
 *   q    [N, H, 576] q_dtype (BF16 or F32): q[n, h, c] = sum_e qb[n, h, e]
 *        kv_b[256 h + e][c] for c < 512 (fp32 accumulation), then pair i of
 *        q^pe turned into dims 512 + i and 544 + i (the cached key's layout)
 * Device pointers, 16-byte aligned; no workspace.
 */
dsa_status_t dsa_absorb_query(int32_t N, int32_t H, const void* qb, const void* w_uk_t,
                              const float* rope_cos, const float* rope_sin, int32_t q_dtype,
                              void* q, void* stream);

/*
 * Head outputs from the latent contexts of N tokens:
 *   o_lat [N, H, 512] bf16: dsa_sparse_mla_fwd's o
 *   out   [N, H * 128] out_dtype (BF16 or F32): out[n, 128 h + d] =
 *         sum_c o_lat[n, h, c] kv_b[256 h + 128 + d][c] (fp32 accumulation),
 *         the heads' outputs concatenated, the input o_proj / wo takes
 * Device pointers, 16-byte aligned; no workspace.
 */
dsa_status_t dsa_absorb_output(int32_t N, int32_t H, const void* o_lat, const void* kv_b,
                               int32_t out_dtype, void* out, void* stream);

/*
 * The output projection wo (o_proj): out [N, Dout] = premix [N, Din] wo^T
 * with wo [Dout, Din] bf16 in Linear layout (16384 -> 7168 for the model),
 * fp32 accumulation, out_dtype BF16 or F32.  Din % 64 == 0, Dout % 128 == 0.
 * ws: at least dsa_output_projection_workspace_bytes(N, Din, Dout) bytes
 * (fp32 partial sums when few tokens split the reduction; 0 otherwise, and
 * ws may then be NULL).  Device pointers, 16-byte aligned.
 */
dsa_status_t dsa_output_projection(int32_t N, int32_t Din, int32_t Dout, const void* premix,
                                   const void* wo, int32_t out_dtype, void* out, void* ws,
                                   size_t ws_bytes, void* stream);
/* Workspace bytes of dsa_output_projection on the current device
 * ((size_t)-1 for invalid sizes). */
size_t dsa_output_projection_workspace_bytes(int32_t N, int32_t Din, int32_t Dout);

/* Workspace bytes an entry point needs for `shape` on the current device
 * (0 if none).  Returns (size_t)-1 when the shape is invalid. */
size_t dsa_workspace_bytes(const dsa_shape_t* shape, int32_t entry);

/*
 * Kernel timing, for measurement only.  Between dsa_timing_begin() and
 * dsa_timing_end(), each kernel the library launches (from any host thread)
 * carries a pair of HIP events that the runtime stamps with that dispatch's
 * own begin and end on the device (hipExtLaunchKernel), on the stream it is
 * launched on; outside a session launches carry none.  dsa_timing_end()
 * waits for the recorded events, ends the session and writes one record per
 * kernel name, in order of first launch, into out[0 .. max_out-1];
 * *n_out (nullable) receives the number of distinct kernels.  The first
 * 65536 launches of a session are timed; later ones are only counted, in
 * `dropped` of their kernel's record.  Events come from a pool the library
 * keeps for the life of the process.
 * Errors: DSA_ERR_INVALID_ARG if a session is already active (begin) or none
 * is (end), or out is NULL with max_out > 0; DSA_ERR_HIP if an event call
 * fails (the session is ended).
 */
typedef struct {
  char name[48];    /* kernel name, e.g. "mla_mfma" */
  int32_t launches; /* timed launches */
  int32_t dropped;  /* launches beyond the session's capacity (not timed) */
  double total_ms, min_ms, max_ms;
} dsa_kernel_time_t;

dsa_status_t dsa_timing_begin(void);
dsa_status_t dsa_timing_end(dsa_kernel_time_t* out, int32_t max_out, int32_t* n_out);

/* Static description of a status code. */
const char* dsa_status_str(dsa_status_t status);

/* Thread-local detail of the last failed call on this thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif
