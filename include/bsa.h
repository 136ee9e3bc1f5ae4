/*
 * bsa.h -- C ABI of libbsa: block-sparse attention with summary-based block
 * routing for AMD Instinct MI355X (gfx950).
 *
 * The method (three stages, each one call here):
 *   Stage 0  bsa_summarize      keys of every block of B tokens are pooled into
 *                               one summary vector ("DashAttention" page,
 *                               section "Estágio 0: Resumo de Blocos Locais");
 *            bsa_summarize_blocks  one block per sequence, for a growing
 *                               decode cache.
 *   Stage 1  bsa_route_topk     every query block (prefill) or query token
 *            bsa_route_entmax   (decode) scores the summaries and selects a set
 *                               of blocks: top-k ("DashAttention", Declaração do
 *                               Problema; "Gist Sparse Attention", section 2,
 *                               item 3) or the support of alpha-entmax
 *                               ("DashAttention", Estágio 1, equation
 *                               w = alpha-entmax(gamma z)), whose threshold is
 *                               found by bisection started from a 16-bin
 *                               histogram ("AdaSplash-2", section 2.A).
 *   Stage 2  bsa_attend_prefill exact softmax attention over the tokens of the
 *            bsa_attend_decode  selected blocks only, causal prefill or one
 *                               query token per sequence ("DashAttention",
 *                               Contribuições item 4: prefill and incremental
 *                               decode).
 *            bsa_attend_backward  gradients of the prefill attention for a
 *                               fixed selection, zero blocks skipped.
 *            bsa_route_entmax_backward  the gradient through the entmax
 *                               routing weights to the queries and keys.
 *            bsa_token_mask     per-token selections (BSA_TOKEN) as active-block
 *                               masks of 64-query tiles.
 *            bsa_attend_entmax  token-level alpha-entmax attention
 *                               ("AdaSplash-2"), dense causal, zero tiles
 *                               skipped; bsa_attend_entmax_backward its
 *                               gradients.
 *   Decode   bsa_decode_topk    Stage 1 (top-k) and Stage 2 for one decode
 *                               step in a single launch (bsa_decode_topk_paged,
 *                               bsa_summarize_blocks_paged: the same over a
 *                               paged K/V cache).
 *
 * Conventions shared by every call
 *   - Tensors are device pointers owned by the caller.  The library never
 *     allocates device memory; scratch space is the caller's `ws` buffer of at
 *     least bsa_workspace_size(...) bytes (NULL allowed when that size is 0),
 *     except in bsa_decode_topk_noalloc, which uses a static device array of
 *     the library instead.
 *   - Q, K, V, O are [batch, heads, tokens, head_dim] with head_dim contiguous
 *     and explicit element strides for (batch, head, token).  Base pointers
 *     must be 16-byte aligned and strides multiples of 8 elements (bf16) or 4
 *     elements (fp32).
 *   - Summaries S are fp32 [batch, n_kv_heads, n_blk, head_dim] contiguous,
 *     n_blk = ceil(kv_len / block).
 *   - GQA: query head h reads KV head h / (n_q_heads / n_kv_heads).
 *   - Selections are int32 [batch, n_kv_heads, n_rows, width], ascending block
 *     ids padded with -1, plus a count [batch, n_kv_heads, n_rows].  n_rows is
 *     ceil(q_len / block) in prefill, q_len in token mode and 1 in decode.
 *   - Every call is asynchronous on `stream` (a hipStream_t; NULL = the null
 *     stream) and returns BSA_OK or a negative bsa_status.  Arguments are
 *     validated on the host before anything is enqueued: on an error nothing
 *     runs and bsa_last_error() (thread-local) describes it.  A failed kernel
 *     launch returns BSA_ERR_DEVICE.
 *   - Device-side integer inputs (kv_lens, idx, cnt) are trusted for values
 *     but never dereferenced out of bounds: lengths are clamped to
 *     [1, kv_len], counts to [0, width], and block ids outside the valid range
 *     are skipped.
 *   - The library holds no state besides that static array; calls on
 *     different streams may overlap as long as their output buffers and
 *     workspaces do not (bsa_decode_topk_noalloc calls on one GPU never may).
 */
#ifndef BSA_H
#define BSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { BSA_F32 = 0, BSA_BF16 = 1 } bsa_dtype;

typedef enum {
  BSA_OK = 0,
  BSA_ERR_INVALID = -1,     /* malformed arguments */
  BSA_ERR_UNSUPPORTED = -2, /* well-formed but outside the supported set */
  BSA_ERR_DEVICE = -3,      /* a HIP launch failed */
  BSA_ERR_WORKSPACE = -4    /* ws_bytes smaller than bsa_workspace_size() */
} bsa_status;

/* BSA_TOKEN: causal prefill routed per query token ("DashAttention",
 * Estágio 1 routes each query): the routing rows are the q_len query tokens,
 * token t's own block is t / B, and attention runs over 64-query tiles with
 * per-token masks (bsa_token_mask). */
typedef enum { BSA_PREFILL = 0, BSA_DECODE = 1, BSA_TOKEN = 2 } bsa_mode;

/* Forced blocks: always in the selection, never counted as routed. */
enum {
  BSA_FORCE_DIAG = 1u,  /* prefill: the query block's own (diagonal) block;
                           token: the block holding the token;
                           decode: the block holding the query (= TAIL) */
  BSA_FORCE_FIRST = 2u, /* block 0 */
  BSA_FORCE_TAIL = 4u   /* decode only: the last, possibly partial, block */
};

typedef enum {
  BSA_OP_SUMMARIZE = 0,
  BSA_OP_ROUTE_TOPK = 1,
  BSA_OP_ROUTE_ENTMAX = 2,
  BSA_OP_ATTEND_PREFILL = 3,
  BSA_OP_ATTEND_DECODE = 4,
  BSA_OP_DECODE_TOPK = 5,
  BSA_OP_ATTEND_PREFILL_PRIOR = 6, /* bsa_attend_prefill with wsel != NULL */
  BSA_OP_ATTEND_BACKWARD = 7,      /* bsa_attend_backward; k_or_cap = k_max */
  BSA_OP_ROUTE_ENTMAX_BACKWARD = 8, /* bsa_route_entmax_backward */
  BSA_OP_ATTEND_ENTMAX_BACKWARD = 9, /* bsa_attend_entmax_backward */
  BSA_OP_ATTEND_BACKWARD_PRIOR = 10  /* bsa_attend_backward with wsel; k_or_cap = k_max */
} bsa_op;

/* Problem description, read only during the call. */
typedef struct bsa_shape {
  int32_t batch;      /* >= 1 */
  int32_t n_q_heads;  /* Hq >= 1 */
  int32_t n_kv_heads; /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;   /* d: 64 or 128 */
  int32_t block;      /* B: 64 or 128 */
  int32_t dtype;      /* bsa_dtype of Q, K and V */
  int32_t mode;       /* bsa_mode */
  int32_t reserved;   /* must be 0 */
  int64_t q_len;      /* prefill, token: N (== kv_len); decode: 1 */
  int64_t kv_len;     /* prefill, token: N; decode: capacity of the K/V cache */
  int64_t q_stride[3]; /* element strides of Q for (batch, head, token) */
  int64_t k_stride[3];
  int64_t v_stride[3];
  int64_t o_stride[3];
} bsa_shape;

/*
 * A paged K/V cache (decode): a pool of num_pages pages of `block` tokens
 * each.  Logical block j of sequence b is page table[b * max_pages + j]
 * (device int32, owned by the caller; an entry outside [0, num_pages) means
 * no page: its rows read as zero).  Element (kv head g, token t of
 * the block, c) of page p of K sits at p * k_page_stride + g * k_stride[1] +
 * t * k_stride[2] + c (V alike with v_page_stride and v_stride); k_stride[0]
 * and v_stride[0] are not used.  max_pages must be >= n_blk (ceil(kv_len /
 * block)); page strides are multiples of 8 (bf16) or 4 (fp32) elements.
 */
typedef struct bsa_pages {
  const int32_t *table;
  int32_t max_pages; /* row length of table */
  int32_t num_pages; /* pages in the pool, >= 1 */
  int64_t k_page_stride;
  int64_t v_page_stride;
} bsa_pages;

/*
 * Stage 0 -- block summaries ("DashAttention", Estágio 0).
 *   K     [batch, Hkv, kv_len, d] in shape->dtype.
 *   qbar  NULL: the zero-initialised learned query, i.e. the uniform mean of
 *         the block's keys.  Otherwise fp32 [Hkv, d]: summary = sum_t w_t k_t
 *         with w = softmax over the block of qbar . k_t / sqrt(d).
 *   S     out, fp32 [batch, Hkv, n_blk, d].  A trailing partial block averages
 *         the tokens present.  In decode only complete blocks are ever read by
 *         the router, so S can be computed once and kept (a summary is fixed
 *         once its block is complete).
 * Errors: BSA_ERR_INVALID (null K or S, bad shape), BSA_ERR_UNSUPPORTED.
 */
int bsa_summarize(const bsa_shape *shape, const void *K, const float *qbar, float *S,
                  void *stream);

/*
 * Stage 0 for a growing decode cache ("DashAttention", Estágio 0: a block's
 * summary is computed once, when the block is complete, and then reused).
 * Recomputes one block summary per sequence instead of the whole cache: for
 * sequence b, S[b, :, blk[b], :] from the keys of block blk[b] (a block
 * reaching past kv_len averages the tokens present, as in bsa_summarize).
 *   blk   int32 [batch] on the device: the block index of each sequence, or
 *         any value outside [0, n_blk) for none.  After appending a token at
 *         position L_b - 1, the block that just completed is L_b / B - 1 when
 *         L_b % B == 0.
 *   K, qbar, S as bsa_summarize (S holds the earlier summaries; only the
 *         named blocks are written).
 * Errors: BSA_ERR_INVALID (null K, S or blk, bad shape), BSA_ERR_UNSUPPORTED.
 */
int bsa_summarize_blocks(const bsa_shape *shape, const void *K, const float *qbar,
                         const int32_t *blk, float *S, void *stream);

/*
 * bsa_summarize_blocks over a paged key cache (see bsa_pages): S[b, :, blk[b]]
 * from the keys of the page holding block blk[b] of sequence b (a negative
 * table entry skips the sequence).  The block is summarised over
 * min(block, kv_len - blk[b] * block) rows, as in bsa_summarize_blocks.
 * Errors: as bsa_summarize_blocks, plus BSA_ERR_INVALID for a NULL or short
 * page table.
 */
int bsa_summarize_blocks_paged(const bsa_shape *shape, const bsa_pages *pages, const void *K,
                               const float *qbar, const int32_t *blk, float *S, void *stream);

/*
 * Stage 1, top-k ("DashAttention", Declaração do Problema; "Gist Sparse
 * Attention", section 2, item 3).
 *   Routing query of a row: prefill -- the mean of the query block's queries,
 *   per head; decode and token mode -- the query itself.  The score of block j for KV head g
 *   is score_scale * sum over the group's query heads of qhat_h . S_j
 *   (score_scale 0 means 1/sqrt(d)).
 *   Candidates: prefill row i -- blocks j <= i (causal); token row t -- blocks
 *   j <= t / B; decode -- complete blocks j < floor((L-1)/B), L = kv_lens[b]
 *   (NULL: every L = kv_len).
 *   Forced blocks (force_flags, BSA_FORCE_*) are always selected; the other
 *   k_total - #forced are the best candidates by (score desc, block asc).
 *   idx   out int32 [batch, Hkv, n_rows, k_total] ascending, -1 padded.
 *   cnt   out int32 [batch, Hkv, n_rows].
 *   scores_out  NULL, or fp32 [batch, Hkv, n_rows, n_blk]: candidate scores,
 *         -inf for non-candidates.
 *   ws    prefill: bsa_workspace_size(BSA_OP_ROUTE_TOPK, ...) bytes.  Decode:
 *         with that much ws the summaries are scored by several workgroups
 *         per row (partitioned); with ws NULL one workgroup per row routes.
 * Errors: BSA_ERR_INVALID (k_total < #forced or < 1, TAIL in prefill, null
 * pointers, bad shape), BSA_ERR_UNSUPPORTED, BSA_ERR_WORKSPACE.
 */
int bsa_route_topk(const bsa_shape *shape, const void *Q, const float *S,
                   const int32_t *kv_lens, int32_t k_total, uint32_t force_flags,
                   float score_scale, int32_t *idx, int32_t *cnt, float *scores_out, void *ws,
                   size_t ws_bytes, void *stream);

/*
 * Stage 1, alpha-entmax ("DashAttention", Estágio 1; threshold per
 * "AdaSplash-2", sections 1 and 2.A).  Per query head and row:
 *   x_j = (alpha-1) * gamma * score_scale * qhat_h . S_j over the candidates
 *   (prefill row i: j < i; token row t: j < t / B; decode: complete blocks
 *   before the tail; forced blocks excluded), tau from a 16-bin histogram of x_max - x on [0, 1)
 *   bracketing the root, then at most max_iter bisection steps, stopping once
 *   no x lies inside the bracket; the exact tau of the resolved support is
 *   used, else the bracket's lower end.  p_j = [x_j - tau]_+^(1/(alpha-1)),
 *   renormalised.  The heads of a KV group average p; the blocks with a
 *   positive average are kept, cut to the `cap` largest (ties: lower block)
 *   when more; forced blocks are added.
 *   idx   out int32 [batch, Hkv, n_rows, cap + #forced], cnt as above.
 *   probs_out NULL or fp32 [batch, Hq, n_rows, n_blk] (0 outside candidates).
 *   tau_out   NULL or fp32 [batch, Hq, n_rows] (NaN for rows without
 *             candidates).
 *   wsel_out  NULL or fp32 [batch, Hkv, n_rows, cap + #forced], the layout of
 *             idx: the routing weight w of each listed block -- the group's
 *             mean probability for a routed block, 1 for a forced block (it
 *             has no routing score), 0 in the padding.  Input of the
 *             prior-induced softmax of bsa_attend_prefill.
 * Errors: BSA_ERR_INVALID (alpha <= 1, n_bins != 16, max_iter outside
 * [0, 32], cap < 1, TAIL in prefill), BSA_ERR_UNSUPPORTED, BSA_ERR_WORKSPACE.
 */
int bsa_route_entmax(const bsa_shape *shape, const void *Q, const float *S,
                     const int32_t *kv_lens, float alpha, float gamma, int32_t n_bins,
                     int32_t max_iter, int32_t cap, uint32_t force_flags, float score_scale,
                     int32_t *idx, int32_t *cnt, float *probs_out, float *tau_out,
                     float *wsel_out, void *ws, size_t ws_bytes, void *stream);

/*
 * Stage 2, causal prefill ("DashAttention", Estágio 2 without routing bias).
 * For query t of head h: softmax over the tokens t' <= t of the blocks in
 * idx[b, g(h), t / B, 0:cnt] of (q_t . k_t') * sm_scale (0 means 1/sqrt(d)),
 * times V.  An empty token set gives 0.
 *   O     out [batch, Hq, q_len, d] with o_stride, dtype o_dtype: shape->dtype
 *         or BSA_F32 (full-precision output for bf16 inputs).
 *   k_max width of idx.
 *   sm_scale  >= 0; 0 means 1/sqrt(d).
 *   wsel, sigma  prior-induced softmax ("DashAttention", Estágio 2): NULL for
 *         the plain softmax, else fp32 routing weights in the layout of idx
 *         (wsel_out of bsa_route_entmax).  The softmax is taken against the
 *         reference g that gives each key of listed block j the weight
 *         w_j^sigma, i.e. those keys' logits gain sigma * ln w_j; a listed
 *         block with w_j <= 0 is dropped (g = 0).  sigma must be finite.
 *   Token mode (shape->mode == BSA_TOKEN): idx/cnt (and wsel) are per-token
 *   [batch, Hkv, q_len, k_max] and query t attends over idx[b, g(h), t, :cnt].
 *   The call first builds the 64-query tile masks of bsa_token_mask in ws
 *   (bsa_workspace_size(BSA_OP_ATTEND_PREFILL, ...) bytes, or
 *   BSA_OP_ATTEND_PREFILL_PRIOR with wsel, which adds each tile's per-query
 *   bias; 256-byte aligned, scratch afterwards), then attends tile by tile
 *   over the active blocks, masking each query's scores on blocks its token
 *   did not select.  In prefill mode ws is unused.
 *   lse   NULL, or out fp32 [batch, Hq, q_len] contiguous: for every query the
 *         natural log of its softmax normaliser, ln sum exp(logit) over the
 *         keys it attends (logits with the prior bias when wsel is given);
 *         -inf for a query that attends nothing.  bsa_attend_backward reads it.
 * Errors: BSA_ERR_INVALID, BSA_ERR_UNSUPPORTED, BSA_ERR_WORKSPACE.
 */
int bsa_attend_prefill(const bsa_shape *shape, const void *Q, const void *K, const void *V,
                       const int32_t *idx, const int32_t *cnt, int32_t k_max, float sm_scale,
                       const float *wsel, float sigma, void *O, int32_t o_dtype, float *lse,
                       void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of Stage 2, causal prefill with block rows or per-token
 * selections: the gradients of bsa_attend_prefill's output for a fixed
 * selection (the selection itself
 * gets none; with a prior, the routing weights do).  The pages single out the backward pass as
 * where training time goes and skip its zero blocks ("AdaSplash-2", section
 * 4); training the sparse attention end to end is "DashAttention",
 * Contribuições item 1.  For query t of head h with weights P_tu over its
 * attended keys u (recomputed from lse) and upstream gradient dO_t:
 *   Delta_t = dO_t . O_t,  dS_tu = P_tu (dO_t . v_u - Delta_t),
 *   dQ_t = sm_scale sum_u dS_tu k_u,
 *   dK_u = sm_scale sum_t dS_tu q_t,  dV_u = sum_t P_tu dO_t,
 * the key sums running over every query head of the KV group.  Only the
 * (query block, selected block) pairs are visited: once from the query side
 * for dQ, once from the key side for dK and dV (rows that selected a block
 * are gathered from a transposed copy of the selection; blocks selected by
 * many rows are split over several workgroups and their parts summed in a
 * fixed order, so results are deterministic).
 *   Q, K, V, idx, cnt, k_max, sm_scale, wsel, sigma  as given to
 *         bsa_attend_prefill (bf16 only; the entries of a row must be
 *         distinct, as the routing calls produce them; wsel NULL: no prior).
 *   Token mode (shape->mode == BSA_TOKEN; "DashAttention", Estágio 1 routes
 *         every query token): idx/cnt (and wsel) per token as in
 *         bsa_attend_prefill.  The call first builds the 64-query tile masks
 *         of bsa_token_mask in ws; the rows of both walks are then those
 *         tiles, and a query's weights on a block its token did not choose
 *         are zero.
 *   dwsel NULL, or out fp32 in the layout of idx (needs wsel; block rows:
 *         k_max <= 80): dL/dw_j = sigma / w_j * sum of dS_tu over the entry's
 *         (query, key) pairs of every query head of the group (the logits of
 *         block j carry sigma ln w_j); 0 for entries beyond cnt, with
 *         w_j <= 0, or (token mode) for a block after the token.
 *         bsa_route_entmax_backward carries it to Q and K.
 *   O     the forward output, o_dtype (bf16 or BSA_F32), with o_stride.
 *   dO    bf16 [batch, Hq, q_len, d] with o_stride.
 *   lse   fp32 [batch, Hq, q_len] written by bsa_attend_prefill.
 *   dQ, dK, dV  out, g_dtype (bf16 or BSA_F32), with the strides of Q, K, V;
 *         every element is written (0 for keys no query attends).
 *   ws    bsa_workspace_size(BSA_OP_ATTEND_BACKWARD, shape, k_max) bytes
 *         without a prior, BSA_OP_ATTEND_BACKWARD_PRIOR with wsel (the same
 *         for block rows; token mode adds the tiles' per-query bias and the
 *         sums behind dwsel), 256-byte aligned; scratch afterwards.
 * Errors: BSA_ERR_INVALID (mode BSA_DECODE, null pointers),
 * BSA_ERR_UNSUPPORTED (fp32 inputs, more than 16384 blocks (token mode:
 * 4096), strides, alignment), BSA_ERR_WORKSPACE.
 */
int bsa_attend_backward(const bsa_shape *shape, const void *Q, const void *K, const void *V,
                        const void *O, int32_t o_dtype, const void *dO, const float *lse,
                        const int32_t *idx, const int32_t *cnt, int32_t k_max, float sm_scale,
                        const float *wsel, float sigma, float *dwsel, void *dQ, void *dK,
                        void *dV, int32_t g_dtype, void *ws, size_t ws_bytes, void *stream);

/*
 * Backward of Stage 1, alpha-entmax routing of prefill block rows (or, with
 * shape->mode == BSA_TOKEN, of every query token: each token is a row whose
 * routing query is its own query and whose candidates are the blocks before
 * its own): the part of the gradient that flows through the routing weights
 * into the queries and
 * the keys ("DashAttention", Estágio 1: entmax routing is differentiable, so
 * gradients pass the routing decision back to the block summaries of
 * Estágio 0).  With w_j = (1/G) sum_h p_hj the listed routed blocks' weights
 * (forced blocks have none), dp_hj = dw_j / G; with g = p^(2-alpha) on the
 * support, the logits z_hj = gamma * score_scale * qhat_h . S_j get
 * dz_j = g_j (dp_j - <g, dp> / sum g); then
 *   dqhat_h = gamma * score_scale * sum_j dz_hj S_j,
 *   dS_j = gamma * score_scale * sum over the group's heads and rows of dz q-hat,
 * and the mean pools give every query of row r dqhat / (tokens of the row;
 * 1 for a token row) and every key of block j dS_j / (tokens of the block) (summaries with a
 * zero learned query).  These are ADDED to dQ and dK (run after
 * bsa_attend_backward wrote the attention part).
 *   Q      the forward's queries (the routing queries are recomputed).
 *   S      fp32 [batch, Hkv, n_blk, d]: the summaries the routing used.
 *   probs  fp32 [batch, Hq, n_rows, n_blk]: probs_out of bsa_route_entmax.
 *   idx, cnt, width  the selection of bsa_route_entmax.
 *   dwsel  fp32, layout of idx: from bsa_attend_backward.
 *   alpha, gamma, score_scale  as given to bsa_route_entmax (0: 1/sqrt(d)).
 *   dQ, dK in/out, g_dtype (input dtype or BSA_F32), strides of Q and K.
 *   ws     bsa_workspace_size(BSA_OP_ROUTE_ENTMAX_BACKWARD, shape, 0) bytes.
 * Errors: BSA_ERR_INVALID (mode BSA_DECODE, alpha <= 1, null pointers),
 * BSA_ERR_UNSUPPORTED, BSA_ERR_WORKSPACE.
 */
int bsa_route_entmax_backward(const bsa_shape *shape, const void *Q, const float *S,
                              const float *probs, const int32_t *idx, const int32_t *cnt,
                              int32_t width, const float *dwsel, float alpha, float gamma,
                              float score_scale, void *dQ, void *dK, int32_t g_dtype, void *ws,
                              size_t ws_bytes, void *stream);

/*
 * Token-level alpha-entmax attention, causal prefill ("AdaSplash-2", sections
 * 1 and 2): the weights of query t over its keys j <= t are
 * p = alpha-entmax(z_t), x_j = (alpha-1) z_j = (alpha-1) sm_scale q_t . k_j,
 * p_j = [x_j - tau_t]_+^(1/(alpha-1)) with sum_j p_j = 1 (exact zeros outside
 * the support); o_t = sum_j p_j v_j, with the weights renormalised by their
 * sum.  tau_t is bracketed by a 16-bin histogram of x_max - x on [0, 1)
 * ("AdaSplash-2", 2.A), then refined by `refine` steps of the hybrid solver
 * of 2.B: Halley for alpha <= 1.5, Newton for 1.5 < alpha <= 2, and for
 * alpha > 2 a secant through the bracket ends (Illinois halving of a kept
 * end), with bisection whenever a step would leave the bracket; key tiles of
 * 64 with no x above the bracket's lower end are skipped in the later
 * passes.  The mass has a kink of unbounded slope at every key when
 * alpha > 2, so the secant needs more steps there than the 1-2 that suffice
 * up to alpha = 2 (about 8 at alpha = 2.5 and 12 at alpha = 3 for the
 * output to settle within 1e-2).
 *   Q, K, V bf16 [batch, H, N, d] (q_len == kv_len == N <= 131072);
 *   O [batch, Hq, N, d] bf16 or fp32 (o_dtype); sm_scale 0 means 1/sqrt(d).
 *   alpha in (1, 16]; refine in [0, 24] (0: tau = the histogram lower bound).
 *   tau_out NULL or fp32 [batch, Hq, N]: the threshold used, in units of x.
 *   live_out NULL or uint32 [batch, Hkv, T, ceil(T / 32)], T = ceil(N / 64):
 *         bit j % 32 of word j / 32 of row (b, g, i) is set when key tile j
 *         holds an x above the bracket's lower end for some query of query
 *         tile i and some query head of KV head g -- a superset of the tiles
 *         with nonzero weights, which bsa_attend_entmax_backward then walks
 *         alone.  With refine = 0 every causal tile is set.  Written whole.
 * Errors: BSA_ERR_INVALID (alpha <= 1, refine outside [0, 24], bad shape),
 * BSA_ERR_UNSUPPORTED (alpha > 16, fp32 inputs, N > 131072, strides).
 */
int bsa_attend_entmax(const bsa_shape *shape, const void *Q, const void *K, const void *V,
                      float alpha, int32_t refine, float sm_scale, void *O, int32_t o_dtype,
                      float *tau_out, uint32_t *live_out, void *stream);

/*
 * Backward of the token-level alpha-entmax attention ("AdaSplash-2",
 * sections 1 and 4: entmax attention is trained, and its backward skips the
 * zero blocks).  With the forward's threshold tau_t (tau_out, x units), the
 * weights of query t are recomputed as p_j = [x_j - tau_t]_+^(1/(alpha-1)) / Z_t
 * (Z_t their sum) and, with dP_j = dO_t . v_j and g = p^(2-alpha) on the
 * support, the entmax vector-Jacobian product gives
 *   dz_j = g_j (dP_j - <g, dP> / sum g),   z_j = sm_scale q_t . k_j,
 *   dQ_t = sm_scale sum_j dz_j k_j,  dK_j = sm_scale sum_t dz_tj q_t,
 *   dV_j = sum_t p_tj dO_t  (key sums over the group's query heads).
 * A first walk over each query's causal key tiles gathers Z and <g, dP> /
 * sum g, a second forms dQ over the tiles where the walk found weight; the
 * key side walks the query tiles from each key tile on.  Products for keys
 * outside every support of a tile are zero.
 *   Q, K, V bf16 [batch, H, N, d] as given to bsa_attend_entmax (shape with
 *         mode BSA_PREFILL, block 64, N <= 131072); alpha in (1, 2];
 *         sm_scale 0: 1/sqrt(d).
 *   dO    bf16 [batch, Hq, N, d] with o_stride.
 *   tau   fp32 [batch, Hq, N]: tau_out of bsa_attend_entmax.
 *   live  NULL (walk every causal tile) or live_out of the same
 *         bsa_attend_entmax call: both sides then visit only its tiles.
 *   dQ, dK, dV  out, g_dtype (bf16 or BSA_F32), strides of Q, K, V.
 *   ws    bsa_workspace_size(BSA_OP_ATTEND_ENTMAX_BACKWARD, shape, 0) bytes.
 * Errors: BSA_ERR_INVALID, BSA_ERR_UNSUPPORTED (fp32 inputs, block != 64,
 * alpha > 2, N > 131072, strides), BSA_ERR_WORKSPACE.
 */
int bsa_attend_entmax_backward(const bsa_shape *shape, const void *Q, const void *K,
                               const void *V, const void *dO, const float *tau,
                               const uint32_t *live, float alpha,
                               float sm_scale, void *dQ, void *dK, void *dV, int32_t g_dtype,
                               void *ws, size_t ws_bytes, void *stream);

/*
 * Active-block masks of per-token selections ("DashAttention", Estágio 2,
 * Implementação: the attention kernel iterates over the active blocks of a
 * bit-packed mask).  Queries are grouped in tiles of 64 tokens,
 * ntile = ceil(q_len / 64).  For each (b, g, tile):
 *   uidx  out int32 [batch, Hkv, ntile, n_blk]: the blocks selected by at
 *         least one of the tile's tokens, ascending, -1 padded;
 *   ucnt  out int32 [batch, Hkv, ntile]: their number;
 *   ubits out uint64 [batch, Hkv, ntile, n_blk]: for entry e, bit r is set
 *         when token 64*tile + r has uidx[e] among idx[b, g, token, :cnt];
 *         0 padded.
 *   idx/cnt  per-token selections [batch, Hkv, q_len, width] (shape->mode
 *         must be BSA_TOKEN); entries outside [0, n_blk) are ignored.
 * Errors: BSA_ERR_INVALID, BSA_ERR_UNSUPPORTED (more than 4096 blocks).
 */
int bsa_token_mask(const bsa_shape *shape, const int32_t *idx, const int32_t *cnt, int32_t width,
                   int32_t *uidx, int32_t *ucnt, uint64_t *ubits, void *stream);

/*
 * Stage 2, decode: one query token per sequence at position L-1
 * (L = kv_lens[b], NULL: kv_len), attending to the tokens t' < L of the blocks
 * in idx[b, g(h), 0, 0:cnt].  One launch: each (batch, KV head) row is
 * handled by one or more workgroups (the GQA group split across them) that
 * stream the selected blocks and merge their partial softmax states on chip.
 *   Q [batch, Hq, 1, d]; K, V [batch, Hkv, kv_len, d]; O [batch, Hq, 1, d].
 *   ws is unused (may be NULL).
 * Errors: BSA_ERR_INVALID, BSA_ERR_UNSUPPORTED (more than 8 query heads per
 * workgroup after splitting, or a row whose scores do not fit in LDS).
 */
int bsa_attend_decode(const bsa_shape *shape, const void *Q, const void *K, const void *V,
                      const int32_t *kv_lens, const int32_t *idx, const int32_t *cnt,
                      int32_t k_max, float sm_scale, void *O, int32_t o_dtype, void *ws,
                      size_t ws_bytes, void *stream);

/*
 * Decode step: top-k routing over the cached summaries S (exactly as
 * bsa_route_topk in decode mode) followed by attention on that selection
 * (as bsa_attend_decode), without the selection round-tripping through the
 * caller.  When the GQA group has at most 8 query heads and fewer than 256
 * blocks are routed, every (batch, KV head) row is served by several
 * workgroups over disjoint data: a routing kernel keeps each summary slice's
 * exact local top-k in ws, and an attention kernel merges them, attends its
 * share of the selected blocks into a partial softmax state in ws, and a
 * combine kernel merges a row's partial states into O.  Otherwise one
 * workgroup per row does everything in one launch and ws is unused.
 *   idx, cnt  NULL, or outputs as in bsa_route_topk (both or neither).
 *   ws        bsa_workspace_size(BSA_OP_DECODE_TOPK, shape, k_total) bytes,
 *             256-byte aligned; its contents need no initialisation and are
 *             scratch afterwards.  Calls sharing one ws must not overlap.
 * Errors: as bsa_route_topk and bsa_attend_decode.
 */
int bsa_decode_topk(const bsa_shape *shape, const void *Q, const void *K, const void *V,
                    const float *S, const int32_t *kv_lens, int32_t k_total,
                    uint32_t force_flags, float score_scale, float sm_scale, int32_t *idx,
                    int32_t *cnt, void *O, int32_t o_dtype, void *ws, size_t ws_bytes,
                    void *stream);

/*
 * bsa_decode_topk over a paged K/V cache ("Gist Sparse Attention", section
 * 2: only the selected blocks are fetched, so a cache stored in pages is read
 * page by page through the sequence's table).  Routing reads the logical
 * summaries S exactly as bsa_decode_topk; the attention reads each selected
 * block from its page, rows at or past L as zero.  Same workspace, outputs
 * and errors as bsa_decode_topk, plus BSA_ERR_INVALID for a NULL or short
 * page table.  Results equal bsa_decode_topk on the gathered cache.
 */
int bsa_decode_topk_paged(const bsa_shape *shape, const bsa_pages *pages, const void *Q,
                          const void *K, const void *V, const float *S, const int32_t *kv_lens,
                          int32_t k_total, uint32_t force_flags, float score_scale,
                          float sm_scale, int32_t *idx, int32_t *cnt, void *O, int32_t o_dtype,
                          void *ws, size_t ws_bytes, void *stream);

/*
 * bsa_decode_topk with no workspace argument, for callers that cannot
 * allocate device memory: code recorded into a HIP graph, tight serving
 * loops, harnesses that forbid hipMalloc.  It calls no allocator.  The
 * scratch that the partitioned decode path needs (routing candidates and
 * partial softmax states, used when batch x n_kv_heads is small) lives in a
 * static device array of the library, BSA_STATIC_SCRATCH_BYTES on each GPU
 * the library runs on, held until the process ends; every slot a call reads
 * is written earlier in the same call, so no clearing is needed.  All calls
 * on one GPU share that array: calls that overlap on one GPU (other streams,
 * other threads) race and must be serialised by the caller.  A shape whose
 * scratch would exceed the array returns BSA_ERR_UNSUPPORTED before anything
 * is enqueued.  Arguments, outputs and other errors as bsa_decode_topk.
 */
#define BSA_STATIC_SCRATCH_BYTES (4u << 20)
int bsa_decode_topk_noalloc(const bsa_shape *shape, const void *Q, const void *K,
                            const void *V, const float *S, const int32_t *kv_lens,
                            int32_t k_total, uint32_t force_flags, float score_scale,
                            float sm_scale, int32_t *idx, int32_t *cnt, void *O,
                            int32_t o_dtype, void *stream);

/* Scratch bytes needed by `op` for this shape; k_or_cap is k_total (top-k),
 * cap (entmax) or k_max (attend).  Returns 0 when none is needed or the
 * arguments are invalid. */
size_t bsa_workspace_size(int32_t op, const bsa_shape *shape, int32_t k_or_cap);

/* Thread-local description of the last error ("" if none). */
const char *bsa_last_error(void);

/* Library version string. */
const char *bsa_version(void);

#ifdef __cplusplus
}
#endif

#endif /* BSA_H */
