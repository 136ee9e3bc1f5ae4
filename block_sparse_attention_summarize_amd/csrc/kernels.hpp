// Launch interface between the host layer (api.cpp) and the gfx950 kernels.
// Every launcher enqueues on `stream` and returns the launch status.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

// Strides are in elements; the head_dim stride is 1.
struct Strides3 {
  int64_t b, h, t;
};

struct SummarizeArgs {
  const void* K;
  Strides3 ks;
  const float* qbar;  // nullptr -> mean
  float* S;           // [batch, hkv, nblk, d]
  const int32_t* blk;  // nullptr: every block; else [batch] the one block per sequence, -1 none
  // paged K (nullptr: contiguous with ks): block j of sequence b is page
  // table[b * max_pages + j], its element (g, t, c) at page * page_k + g * ks.h + t * ks.t + c
  const int32_t* table;
  int max_pages, num_pages;
  int64_t page_k;
  int batch, hkv, d, B, nblk;
  int64_t kv_len;
  bool bf16;
};
hipError_t launch_summarize(const SummarizeArgs& a, hipStream_t stream);

// Routing query of every row.  Prefill: mean over the query block, decode
// and per-token routing (B = 1): the query itself.  group_sum: add the heads of each KV group (top-k) and
// write [batch, hkv, nrow, d]; otherwise [batch, hq, nrow, d].
struct QPoolArgs {
  const void* Q;
  Strides3 qs;
  float* qhat;
  int batch, hq, hkv, d, B, nrow;
  int64_t q_len;
  bool bf16, group_sum;
};
hipError_t launch_qpool(const QPoolArgs& a, hipStream_t stream);

// Candidate range and forced blocks of a routing row are derived on the
// device from (mode, row, kv_lens) exactly as documented in bsa.h.
struct RowRule {
  int mode;       // 0 prefill (row = query block), 1 decode, 2 prefill routed per token
  int entmax;     // 1: prefill candidates exclude the diagonal
  uint32_t force;
  int B;
  int64_t kv_len;
  const int32_t* kv_lens;  // decode, may be null
};

// scores[row, j] = scale * qhat[row] . S[b, g, j] for candidate j, -inf else.
// qhat holds `qheads` heads per batch (the KV heads for top-k, whose q-hat is
// already summed over the group, or the query heads for entmax); head h reads
// the summaries of KV head h / group.
struct ScoreArgs {
  const float* qhat;  // [batch, qheads, nrow, d]
  const float* S;     // [batch, hkv, nblk, d]
  float* scores;      // [batch, qheads, nrow, nblk]
  int batch, hkv, qheads, group, nrow, nblk, d;
  float scale;
  RowRule rule;
};
// fill: also write -inf over whole tiles beyond every row's candidates (a
// caller-visible score matrix); otherwise only tiles holding candidates.
hipError_t launch_scores(const ScoreArgs& a, hipStream_t stream, bool fill);

struct SelectArgs {
  const float* scores;  // [rows, nblk]
  int32_t* idx;         // [rows, k_total]
  int32_t* cnt;         // [rows]
  int batch, hkv, nrow, nblk, k_total;
  RowRule rule;
};
hipError_t launch_select_topk(const SelectArgs& a, hipStream_t stream);

struct EntmaxArgs {
  int32_t* idx;       // [batch, hkv, nrow, width]
  int32_t* cnt;
  float* probs;       // optional [batch, hq, nrow, nblk]
  float* tau;         // optional [batch, hq, nrow]
  float* wsel;        // optional [batch, hkv, nrow, width]: group-mean p of each listed
                      // block, 1 for forced blocks, 0 padded
  float* xbuf;        // logits from the scores kernel [batch, hq, nrow, nblk]; overwritten
                      // with the probabilities
  int batch, hq, hkv, nrow, nblk, width, cap, max_iter;
  float alpha;
  int tourn;  // set by the launcher: cap below the tournament slice and its buffers fit
  RowRule rule;
};
hipError_t launch_route_entmax(const EntmaxArgs& a, hipStream_t stream);

struct AttendArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  Strides3 qs, ks, vs, os;
  const int32_t* idx;  // [batch, hkv, nrow, k_max]
  const int32_t* cnt;
  // Per-token selections: nullptr for block rows (row i = queries [iB, iB+B)).
  // Otherwise row i is the query tile [64i, 64i+64), idx/cnt its active
  // blocks and bits[row, e] the tile's tokens that selected block idx[row, e].
  const uint64_t* bits;
  // Prior-induced softmax (nullptr: plain softmax).  Block rows: wsel holds
  // the routing weight w of every entry of idx (layout of idx); the scores of
  // its keys gain sigma * ln w, and an entry with w <= 0 is skipped.  Token
  // tiles: tbias [row, entry, 64 queries] holds that bias per query already
  // (-inf where the query's token did not select the block).
  const float* wsel;
  const float* tbias;
  float sigma;
  // optional [batch, hq, q_len]: ln of the softmax normaliser of every query,
  // ln sum_u exp(sm_scale q.k_u + bias_u) over its attended keys (-inf: none)
  float* lse;
  int batch, hq, hkv, d, B, k_max, nrow, nblk;
  int64_t q_len, kv_len;
  float sm_scale;
  bool bf16, out_f32;
};
hipError_t launch_attend_prefill(const AttendArgs& a, hipStream_t stream);

// Gradients of the causal block-sparse prefill attention (bf16, q_len ==
// kv_len == n) for a fixed selection idx/cnt [batch, hkv, nrow, k_max]: block
// rows, or (tok) 64-query tiles listing the union of their tokens' blocks.
// dQ, dK, dV are written with the strides of Q, K, V (elements of the
// gradient dtype); dO has the strides of O.
struct BwdArgs {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  void* dQ;
  void* dK;
  void* dV;
  Strides3 qs, ks, vs, os;
  const float* lse;  // [batch, hq, n] from the forward
  const int32_t* idx;
  const int32_t* cnt;
  // prior-induced softmax (nullptr: none): routing weights in the layout of
  // idx; entries with w <= 0 are skipped, listed keys' logits gain sigma ln w
  const float* wsel;
  float sigma;
  float* dwsel;      // optional out, layout of idx: dL/dw (needs wsel)
  float* dbpart;     // workspace [batch * hkv * nrow, units, k_max]: per-unit sums of dS
  // workspace
  float* delta;      // [batch, hq, n]: dO . O
  uint32_t* bits;    // [batch * hkv, nwords, nblk]: bit r % 32 of word r / 32 = row r selected block j
  int4* items;       // [max_items] (pair, block, chunk, partial slot or -1)
  int4* red;         // [max_red] (pair, block, first slot, chunks)
  int* counters;     // [2]: items, red
  float* part;       // [slots, 2, B, d]: dK then dV partials of split blocks
  int batch, hq, hkv, d, B, k_max, nrow, nblk, nwords, chunk, max_items, max_red;
  int units;         // query-side units per row (query heads of a group x query sub-tiles)
  int64_t n;
  float sm_scale;
  bool bf16, o_f32, g_f32;
  // token-level entmax attention (dense causal, B = 64; idx, cnt, the plan
  // and lse unused): tau per query [batch, hq, n] in units of
  // x = (alpha - 1) sm_scale q.k; zbuf (workspace [batch, hq, n]) receives
  // each query's normaliser, delta its <g, dP> / sum g
  bool ent;
  float alpha;
  const float* tau;
  float* zbuf;
  const uint32_t* live;  // optional [batch * hkv, nrow, nlw]: the forward's live key tiles
  int nlw;
  // per-token selections: a row is a 64-query tile (rowq = 64; block rows
  // have rowq = B) whose list idx/cnt is the union of its tokens' blocks
  // (bsa_token_mask), each entry with the word of the tokens that chose it
  bool tok;
  int rowq;
  const uint64_t* tbits;  // [batch * hkv * nrow, k_max]
  const float* tbias;     // nullptr, or [.., k_max, 64]: sigma ln w (or -inf) per query
  int32_t* tpos;          // workspace [batch * hkv, nblk, nrow]: list entry of block j in row r
  float* dbtok;           // workspace [batch * hkv * nrow, k_max, nparts, 64]: dS sums (dL/dw)
  int nparts;             // query-side workgroups that share one query's heads, at most
  // per-token lists and weights, for dL/dw [batch, hkv, n, width]
  const int32_t* pidx;
  const int32_t* pcnt;
  const float* pw;
  int pwidth;
};
int attend_bwd_units(int group, int B);  // units per row of the query side
int attend_bwd_max_prior_width();        // k_max limit when dL/dw is requested
int attend_bwd_tok_parts(int group);     // nparts of the token-mode dL/dw sums
hipError_t launch_attend_backward(const BwdArgs& a, hipStream_t stream);

// Routing part of the gradient of entmax-routed prefill (block rows, or a
// row per query token): dL/dw of the listed blocks -> dQ, dK (added to the
// caller's gradients).
struct RouteBwdArgs {
  const float* qhat;   // [batch, hq, nrow, d] routing queries (workspace)
  const float* S;      // [batch, hkv, nblk, d] summaries
  const float* probs;  // [batch, hq, nrow, nblk] the routing probabilities
  const int32_t* idx;  // [batch, hkv, nrow, width]
  const int32_t* cnt;
  const float* dwsel;  // layout of idx
  float* dz;           // [batch, hq, nrow, nblk] workspace: dL/d(q-hat . S)
  float* dqh;          // [batch, hq, nrow, d] workspace: dL/d(q-hat)
  float* dsp;          // [batch, hq, ksplit, nblk, d] workspace: each head's (and row
                       // range's) part of dL/dS
  void* dQ;
  void* dK;
  Strides3 qs, ks;     // of dQ, dK (elements of the gradient dtype)
  int batch, hq, hkv, d, B, nrow, nblk, width;
  int rowq;    // queries pooled per row: B (block rows) or 1 (token rows)
  int rowdiv;  // row r's own block is r / rowdiv: 1 (block rows) or B (token rows)
  int ksplit;  // row ranges the key-side product is split into
  int64_t n;
  float alpha, fscale;  // fscale = gamma * score_scale
  bool g_f32;
};
int route_bwd_key_splits(int nrow);  // ksplit for nrow routing rows
hipError_t launch_route_entmax_backward(const RouteBwdArgs& a, hipStream_t stream);

// Active blocks of every 64-query tile from per-token selections
// idx/cnt [batch, hkv, q_len, width]: uidx/ucnt the ascending union over the
// tile's tokens (-1 padded to nblk), ubits the tokens that selected each.
struct TokenMaskArgs {
  const int32_t* idx;
  const int32_t* cnt;
  int32_t* uidx;   // [batch, hkv, ntile, nblk]
  int32_t* ucnt;   // [batch, hkv, ntile]
  uint64_t* ubits; // [batch, hkv, ntile, nblk]
  // optional prior: per-token weights wsel [batch, hkv, q_len, width] ->
  // ubias [batch, hkv, ntile, nblk, 64] = sigma * ln w (-inf: not selected)
  const float* wsel;
  float* ubias;
  float sigma;
  int batch, hkv, width, nblk, ntile;
  int64_t q_len;
};
hipError_t launch_token_mask(const TokenMaskArgs& a, hipStream_t stream);

// Token-level alpha-entmax attention, causal prefill (bf16 Q/K/V, q_len ==
// kv_len == n): o_t = sum_{j<=t} p_tj v_j, p_t = alpha-entmax of
// (alpha-1) sm_scale q_t . k_j; `refine` hybrid steps after the histogram
// bracket.
struct EntmaxAttnArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  Strides3 qs, ks, vs, os;
  float* tau;  // optional [batch, hq, n]: the threshold used, in units of x
  uint32_t* live;  // optional [batch, hkv, ntile, nlw]: key tiles with some x above the
                   // bracket's lower end, per query tile (union over the group's heads)
  int batch, hq, hkv, d, refine;
  int64_t n;
  float sm_scale, alpha;
  bool out_f32;
};
int entmax_attend_max_tiles();
hipError_t launch_entmax_attend(const EntmaxAttnArgs& a, hipStream_t stream);

// Single-token decode: routing (route = 1) and/or attention (attend = 1) for
// every (batch, KV head) row, hsplit workgroups per row splitting the query
// heads.  Without routing, the selection is read from idx/cnt.
struct DecodeArgs {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  Strides3 qs, ks, vs, os;
  const float* S;          // [batch, hkv, nblk, d] summaries
  const int32_t* kv_lens;  // may be null
  int32_t* idx;            // [batch, hkv, 1, k_total]: out when routing, else in
  int32_t* cnt;
  int batch, hq, hkv, d, B, nblk, k_total, hsplit, route, attend, lds_floats;
  int64_t kv_len;
  uint32_t force;
  float score_scale, sm_scale;
  bool bf16, out_f32;
  // paged K/V (nullptr: contiguous [batch, hkv, kv_len, d] with ks/vs):
  // logical block j of sequence b is page table[b * max_pages + j], whose
  // element (g, t, c) sits at page * page_k + g * ks.h + t * ks.t + c (V alike)
  const int32_t* table;
  int max_pages, num_pages;  // pages outside [0, num_pages) read as zero
  int64_t page_k, page_v;
  // partitioned decode (parts workgroups per row over disjoint data)
  int parts, mpad;       // candidates kept per partition (>= routed count)
  uint32_t* cand_key;    // [rows, parts, mpad] order-preserving score keys
  int32_t* cand_id;      // [rows, parts, mpad] block ids, -1 = none
  float* part;           // [rows, parts, G, d + 2] partial softmax states
};
int decode_lds_floats(int nblk, int d, int gs_max);
int decode_sel_ints(int nblk, int k_total);  // LDS ints after the floats
hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t stream);
// Partitioned decode step: routing kernel then attention kernel.  With
// attend = 0 the second kernel only merges the candidates into idx/cnt.
hipError_t launch_decode_parts(const DecodeArgs& a, hipStream_t stream);

}  // namespace bsa
