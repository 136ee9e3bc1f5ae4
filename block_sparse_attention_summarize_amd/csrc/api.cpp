// Host side of the C ABI in include/bsa.h: argument validation (before
// anything is enqueued), workspace carving and kernel dispatch.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <mutex>
#include <string>

#include "bsa.h"
#include "kernels.hpp"

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

int ok() {
  g_err.clear();
  return BSA_OK;
}

int device_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(BSA_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

int64_t nblk_of(const bsa_shape* s) { return (s->kv_len + s->block - 1) / s->block; }
// Routing rows: query blocks (prefill), query tokens (token), one (decode).
int64_t nrow_of(const bsa_shape* s) {
  if (s->mode == BSA_TOKEN) return s->q_len;
  return s->mode == BSA_PREFILL ? (s->q_len + s->block - 1) / s->block : 1;
}
// 64-query tiles of per-token attention.
int64_t ntile_of(const bsa_shape* s) { return (s->q_len + 63) / 64; }
constexpr int64_t kMaxTokenBlocks = 4096;  // one LDS word per block in the mask kernel (32 KiB)
int popcount3(uint32_t f) { return (f & 1u) + ((f >> 1) & 1u) + ((f >> 2) & 1u); }
int elem_bytes(int32_t dt) { return dt == BSA_BF16 ? 2 : 4; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape checks shared by every entry point.
int check_shape(const bsa_shape* s) {
  if (!s) return fail(BSA_ERR_INVALID, "shape is NULL");
  if (s->batch < 1 || s->n_q_heads < 1 || s->n_kv_heads < 1)
    return fail(BSA_ERR_INVALID, "batch, n_q_heads and n_kv_heads must be >= 1");
  if (s->n_q_heads % s->n_kv_heads != 0)
    return fail(BSA_ERR_INVALID, "n_q_heads (%d) must be a multiple of n_kv_heads (%d)",
                s->n_q_heads, s->n_kv_heads);
  if (s->mode != BSA_PREFILL && s->mode != BSA_DECODE && s->mode != BSA_TOKEN)
    return fail(BSA_ERR_INVALID, "mode must be BSA_PREFILL, BSA_DECODE or BSA_TOKEN");
  if (s->reserved != 0) return fail(BSA_ERR_INVALID, "reserved field must be 0");
  if (s->kv_len < 1) return fail(BSA_ERR_INVALID, "kv_len must be >= 1");
  if (s->mode != BSA_DECODE && s->q_len != s->kv_len)
    return fail(BSA_ERR_INVALID, "prefill needs q_len == kv_len (got %lld, %lld)",
                (long long)s->q_len, (long long)s->kv_len);
  if (s->mode == BSA_DECODE && s->q_len != 1)
    return fail(BSA_ERR_INVALID, "decode needs q_len == 1 (got %lld)", (long long)s->q_len);
  if (s->dtype != BSA_F32 && s->dtype != BSA_BF16)
    return fail(BSA_ERR_UNSUPPORTED, "dtype %d is not supported (BSA_F32, BSA_BF16)", s->dtype);
  if (s->head_dim != 64 && s->head_dim != 128)
    return fail(BSA_ERR_UNSUPPORTED, "head_dim %d is not supported (64, 128)", s->head_dim);
  if (s->block != 64 && s->block != 128)
    return fail(BSA_ERR_UNSUPPORTED, "block %d is not supported (64, 128)", s->block);
  const int64_t nblk = nblk_of(s);
  const int64_t nrow = nrow_of(s);
  // grids are 1-D with one workgroup per (batch, head, block) at most
  const int64_t worst = static_cast<int64_t>(s->batch) * s->n_q_heads * nblk * 2;
  const int64_t rows = static_cast<int64_t>(s->batch) * s->n_q_heads * nrow;
  if (worst >= (int64_t(1) << 31) || rows >= (int64_t(1) << 31) ||
      nblk * nrow >= (int64_t(1) << 40))
    return fail(BSA_ERR_UNSUPPORTED, "problem too large for one launch");
  return BSA_OK;
}

int check_strides(const char* name, const int64_t st[3], int32_t dtype) {
  const int64_t q = dtype == BSA_BF16 ? 8 : 4;
  for (int k = 0; k < 3; ++k) {
    if (st[k] < 0) return fail(BSA_ERR_INVALID, "%s stride %d is negative", name, k);
    if (st[k] % q != 0)
      return fail(BSA_ERR_UNSUPPORTED, "%s stride %d (%lld) must be a multiple of %lld elements",
                  name, k, (long long)st[k], (long long)q);
  }
  return BSA_OK;
}

int check_ptr(const char* name, const void* p) {
  if (!p) return fail(BSA_ERR_INVALID, "%s is NULL", name);
  if (!aligned16(p)) return fail(BSA_ERR_UNSUPPORTED, "%s must be 16-byte aligned", name);
  return BSA_OK;
}

bsa::Strides3 st3(const int64_t s[3]) { return bsa::Strides3{s[0], s[1], s[2]}; }

bsa::RowRule rule_of(const bsa_shape* s, int entmax, uint32_t force, const int32_t* kv_lens) {
  bsa::RowRule r;
  r.mode = s->mode;
  r.entmax = entmax;
  r.force = force;
  r.B = s->block;
  r.kv_len = s->kv_len;
  r.kv_lens = s->mode == BSA_DECODE ? kv_lens : nullptr;
  return r;
}

int check_force(const bsa_shape* s, uint32_t force) {
  if (force & ~7u) return fail(BSA_ERR_INVALID, "unknown force flags 0x%x", force);
  if (s->mode != BSA_DECODE && (force & BSA_FORCE_TAIL))
    return fail(BSA_ERR_INVALID, "BSA_FORCE_TAIL is only meaningful in decode");
  return BSA_OK;
}

// Workgroups per decode row: the GQA group is split over hsplit workgroups
// (at most 8 query heads each) until the grid covers the 256 CUs.
int decode_hsplit(const bsa_shape* s) {
  const int G = s->n_q_heads / s->n_kv_heads;
  const int64_t rows = static_cast<int64_t>(s->batch) * s->n_kv_heads;
  int h = 1;
  while (G / h > 8 || (G % (2 * h) == 0 && rows * h < 256)) h *= 2;
  return G % h == 0 ? h : -1;
}
int gs_template(int gs) { return gs <= 1 ? 1 : gs <= 2 ? 2 : gs <= 4 ? 4 : 8; }

// Partitioned decode: `parts` workgroups per row over disjoint data, so that
// the grid covers the 256 CUs; used when the GQA group has at most 8 heads and
// fewer than 256 blocks are routed.
int decode_parts(const bsa_shape* s, int32_t k_total, uint32_t force) {
  const int G = s->n_q_heads / s->n_kv_heads;
  const int64_t rows = static_cast<int64_t>(s->batch) * s->n_kv_heads;
  const int m = k_total - popcount3(force);
  if (G > 8 || m >= 256) return 0;
  // Splitting pays only when one workgroup per row would leave most CUs
  // idle: at 128 rows (2 parts) the single fused launch is faster (72 us
  // against 83 us for 16 x 8 rows of 128k tokens), since a part's share is
  // too small to keep enough loads in flight.
  int parts = static_cast<int>((256 + rows - 1) / rows);
  if (parts < 3) return 0;
  parts = parts > 8 ? 8 : parts;
  const int64_t per = (nblk_of(s) + parts - 1) / parts;
  const int64_t cap = ((per + 255) / 256) * k_total;
  if (per * 4 + cap * 16 > 96 * 1024) return 0;
  const int64_t tot = static_cast<int64_t>(parts) * k_total;
  const int64_t cap2 = ((tot + 255) / 256) * k_total;
  if (k_total * 4 + cap2 * 16 + k_total * 8 + 8 * 8 * (s->head_dim + 2) * 4 > 96 * 1024) return 0;
  return parts;
}
struct DecodeWs {
  size_t cand, part, total;
};
DecodeWs decode_ws(const bsa_shape* s, int parts, int32_t k_total, bool attend) {
  const size_t rows = static_cast<size_t>(s->batch) * s->n_kv_heads;
  const size_t G = s->n_q_heads / s->n_kv_heads;
  DecodeWs w;
  w.cand = align_up(rows * parts * k_total * 4);
  w.part = attend ? align_up(rows * parts * G * (s->head_dim + 2) * 4) : 0;
  w.total = parts > 0 ? 2 * w.cand + w.part : 0;
  return w;
}

// LDS floats of the fused decode kernel; -1 when the row does not fit.
int decode_lds(const bsa_shape* s, int hsplit, int32_t width) {
  const int gs = gs_template((s->n_q_heads / s->n_kv_heads) / hsplit);
  const int64_t nblk = nblk_of(s);
  const int64_t f = bsa::decode_lds_floats(static_cast<int>(nblk), s->head_dim, gs);
  if (nblk > (int64_t(1) << 24)) return -1;
  if ((f + bsa::decode_sel_ints(static_cast<int>(nblk), width)) * 4 > 96 * 1024) return -1;
  return static_cast<int>(f);
}

// Decode routing normally runs the fused kernel with no scratch; the
// size returned also covers the three-kernel path used when scores_out is
// requested.
size_t ws_route_topk(const bsa_shape* s, int32_t k_total = 0, uint32_t force = 0) {
  if (s->mode == BSA_DECODE && k_total > 0) {
    const int parts = decode_parts(s, k_total, force);
    if (parts > 0) return decode_ws(s, parts, k_total, false).total;
  }
  const size_t rows = static_cast<size_t>(s->batch) * s->n_kv_heads * nrow_of(s);
  return align_up(rows * s->head_dim * 4) + align_up(rows * nblk_of(s) * 4);
}
size_t ws_route_entmax(const bsa_shape* s) {
  const size_t hrows = static_cast<size_t>(s->batch) * s->n_q_heads * nrow_of(s);
  return align_up(hrows * s->head_dim * 4) + align_up(hrows * nblk_of(s) * 4);
}
// Per-token attention: the tile masks (uidx, ubits, ucnt) and, with a prior,
// the per-query bias of every listed block (ubias) live in ws.
struct MaskWs {
  size_t uidx, ubits, ucnt, ubias, total;
};
MaskWs mask_ws(const bsa_shape* s, bool prior) {
  const size_t rows = static_cast<size_t>(s->batch) * s->n_kv_heads * ntile_of(s);
  MaskWs w;
  w.uidx = align_up(rows * nblk_of(s) * 4);
  w.ubits = align_up(rows * nblk_of(s) * 8);
  w.ucnt = align_up(rows * 4);
  w.ubias = prior ? align_up(rows * nblk_of(s) * 64 * 4) : 0;
  w.total = w.uidx + w.ubits + w.ucnt + w.ubias;
  return w;
}
// Backward: Delta, the transposed selection, the work plan and the partial
// sums of key blocks split over several work items.
constexpr int kBwdChunk = 32;                  // query blocks per key-side work item
constexpr int64_t kMaxBwdBlocks = 16384;       // one LDS word per key block when marking
// Per-token selections (BSA_TOKEN) add the tile masks of bsa_token_mask (the
// rows are 64-query tiles listing the union of their tokens' blocks), the
// position of every block in each tile's list and, with a prior, the tiles'
// per-query bias and the per-(entry, query) sums of dS behind dL/dw.
struct BwdWs {
  size_t delta, bits, items, red, counters, part, dbpart, tpos, uidx, ubits, ucnt, ubias, dbtok,
      total;
  int64_t max_items, max_red, slots, nwords, nrow;
};
BwdWs bwd_ws(const bsa_shape* s, int32_t k_max, bool prior) {
  BwdWs w{};
  const bool tok = s->mode == BSA_TOKEN;
  const int64_t npair = static_cast<int64_t>(s->batch) * s->n_kv_heads;
  const int64_t nblk = nblk_of(s);
  const int64_t nrow = tok ? ntile_of(s) : nrow_of(s);
  const int64_t rowq = tok ? 64 : s->block;
  const int64_t k = tok ? nblk : std::max<int64_t>(1, std::min<int64_t>(k_max, nblk));
  // (row, block) pairs with the block starting at or before the row's last
  // query: sum over rows of min(k, that many blocks)
  int64_t per = 0;
  for (int64_t r = 0; r < nrow; ++r) per += std::min<int64_t>(k, ((r + 1) * rowq - 1) / s->block + 1);
  const int64_t E = npair * per;
  w.nrow = nrow;
  w.nwords = (nrow + 31) / 32;
  w.max_items = npair * nblk + (E + kBwdChunk - 1) / kBwdChunk;
  w.max_red = std::min<int64_t>(npair * nblk, E / (kBwdChunk + 1) + 1);
  w.slots = E / kBwdChunk + w.max_red + 1;
  w.delta = align_up(static_cast<size_t>(s->batch) * s->n_q_heads * s->q_len * 4);
  w.bits = align_up(static_cast<size_t>(npair * w.nwords * nblk) * 4);
  w.items = align_up(static_cast<size_t>(w.max_items) * 16);
  w.red = align_up(static_cast<size_t>(w.max_red) * 16);
  w.counters = align_up(8);
  w.part = align_up(static_cast<size_t>(w.slots) * 2 * s->block * s->head_dim * 4);
  // per-unit sums of dS for dL/dw (the prior's gradient)
  w.dbpart = tok ? 0
                 : align_up(static_cast<size_t>(npair * nrow) *
                            bsa::attend_bwd_units(s->n_q_heads / s->n_kv_heads, s->block) *
                            std::max<int32_t>(k_max, 1) * 4);
  if (tok) {
    const size_t rl = static_cast<size_t>(npair * nrow * nblk);  // (row, list entry) slots
    w.tpos = align_up(rl * 4);
    w.uidx = align_up(rl * 4);
    w.ubits = align_up(rl * 8);
    w.ucnt = align_up(static_cast<size_t>(npair * nrow) * 4);
    w.ubias = prior ? align_up(rl * 64 * 4) : 0;
    w.dbtok = prior ? align_up(rl * bsa::attend_bwd_tok_parts(s->n_q_heads / s->n_kv_heads) * 64 * 4)
                    : 0;
  }
  w.total = w.delta + w.bits + w.items + w.red + w.counters + w.part + w.dbpart + w.tpos +
            w.uidx + w.ubits + w.ucnt + w.ubias + w.dbtok;
  return w;
}
// Routing backward: the routing queries and dL/d(logit) of every head-row.
struct RouteBwdWs {
  size_t qhat, dz, dqh, dsp, total;
};
RouteBwdWs route_bwd_ws(const bsa_shape* s) {
  const size_t rows = static_cast<size_t>(s->batch) * s->n_q_heads * nrow_of(s);
  RouteBwdWs w{};
  w.qhat = align_up(rows * s->head_dim * 4);
  w.dz = align_up(rows * nblk_of(s) * 4);
  w.dqh = align_up(rows * s->head_dim * 4);
  w.dsp = align_up(static_cast<size_t>(s->batch) * s->n_q_heads *
                   bsa::route_bwd_key_splits(static_cast<int>(nrow_of(s))) * nblk_of(s) *
                   s->head_dim * 4);
  w.total = w.qhat + w.dz + w.dqh + w.dsp;
  return w;
}
int check_ws(void* ws, size_t ws_bytes, size_t need) {
  if (ws_bytes < need)
    return fail(BSA_ERR_WORKSPACE, "workspace of %zu bytes is smaller than the %zu needed",
                ws_bytes, need);
  if (need > 0 && !ws) return fail(BSA_ERR_INVALID, "ws is NULL");
  if (need > 0 && (reinterpret_cast<uintptr_t>(ws) % kAlign) != 0)
    return fail(BSA_ERR_UNSUPPORTED, "ws must be %zu-byte aligned", kAlign);
  return BSA_OK;
}

// Fills the fused decode kernel's arguments shared by the three decode calls.
// A paged K/V cache: the table, its row length and the page strides.
int check_pages(const bsa_shape* s, const bsa_pages* pg) {
  if (!pg) return fail(BSA_ERR_INVALID, "pages is NULL");
  if (!pg->table) return fail(BSA_ERR_INVALID, "pages->table is NULL");
  if (pg->num_pages < 1) return fail(BSA_ERR_INVALID, "pages->num_pages must be >= 1");
  if (pg->max_pages < nblk_of(s))
    return fail(BSA_ERR_INVALID, "pages->max_pages (%d) must cover the %lld blocks of kv_len",
                pg->max_pages, (long long)nblk_of(s));
  const int64_t q = s->dtype == BSA_BF16 ? 8 : 4;
  if (pg->k_page_stride < 0 || pg->v_page_stride < 0)
    return fail(BSA_ERR_INVALID, "page strides must be >= 0");
  if (pg->k_page_stride % q != 0 || pg->v_page_stride % q != 0)
    return fail(BSA_ERR_UNSUPPORTED, "page strides must be multiples of %lld elements",
                (long long)q);
  return BSA_OK;
}

int decode_args(const bsa_shape* s, const void* Q, const void* K, const void* V,
                       const float* S, const int32_t* kv_lens, int32_t* idx, int32_t* cnt,
                       int32_t width, uint32_t force, float score_scale, float sm_scale, void* O,
                       int32_t o_dtype, int route, int attend, bsa::DecodeArgs& a,
                       const bsa_pages* pg = nullptr) {
  int rc;
  a = bsa::DecodeArgs{};
  if (s->mode != BSA_DECODE) return fail(BSA_ERR_INVALID, "decode calls need BSA_DECODE");
  if ((rc = check_ptr("Q", Q)) != BSA_OK) return rc;
  if ((rc = check_strides("Q", s->q_stride, s->dtype)) != BSA_OK) return rc;
  if (!std::isfinite(score_scale) || !std::isfinite(sm_scale) || sm_scale < 0.f)
    return fail(BSA_ERR_INVALID, "scales must be finite and sm_scale >= 0 (0: 1/sqrt(d))");
  if (route && (rc = check_ptr("S", S)) != BSA_OK) return rc;
  if (attend) {
    if ((rc = check_ptr("K", K)) != BSA_OK) return rc;
    if ((rc = check_ptr("V", V)) != BSA_OK) return rc;
    if ((rc = check_ptr("O", O)) != BSA_OK) return rc;
    if (o_dtype != s->dtype && o_dtype != BSA_F32)
      return fail(BSA_ERR_UNSUPPORTED, "o_dtype must be the input dtype or BSA_F32");
    if ((rc = check_strides("K", s->k_stride, s->dtype)) != BSA_OK) return rc;
    if ((rc = check_strides("V", s->v_stride, s->dtype)) != BSA_OK) return rc;
    if ((rc = check_strides("O", s->o_stride, o_dtype)) != BSA_OK) return rc;
    if (s->k_stride[2] < s->head_dim || s->v_stride[2] < s->head_dim)
      return fail(BSA_ERR_INVALID, "K/V token stride must be >= head_dim");
    // one head's rows (of a sequence, or of a page) are addressed with
    // 32-bit byte offsets
    const int64_t esz = elem_bytes(s->dtype);
    const int64_t rows = pg ? s->block : s->kv_len;
    if ((rows + 256) * s->k_stride[2] * esz >= (int64_t(1) << 31) ||
        (rows + 256) * s->v_stride[2] * esz >= (int64_t(1) << 31))
      return fail(BSA_ERR_UNSUPPORTED, "K/V: one head spans more than 2 GiB");
    if (pg) {
      if ((rc = check_pages(s, pg)) != BSA_OK) return rc;
      a.table = pg->table;
      a.max_pages = pg->max_pages;
      a.num_pages = pg->num_pages;
      a.page_k = pg->k_page_stride;
      a.page_v = pg->v_page_stride;
    }
  }
  const int hsplit = attend ? decode_hsplit(s) : 1;
  if (hsplit < 1)
    return fail(BSA_ERR_UNSUPPORTED, "decode needs n_q_heads/n_kv_heads to split into <= 8 heads");
  const int lds = decode_lds(s, hsplit, width);
  if (lds < 0) return fail(BSA_ERR_UNSUPPORTED, "decode row too long for one workgroup's LDS");
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.qs = st3(s->q_stride);
  a.ks = st3(s->k_stride);
  a.vs = st3(s->v_stride);
  a.os = st3(s->o_stride);
  a.S = S;
  a.kv_lens = kv_lens;
  a.idx = idx;
  a.cnt = cnt;
  a.batch = s->batch;
  a.hq = s->n_q_heads;
  a.hkv = s->n_kv_heads;
  a.d = s->head_dim;
  a.B = s->block;
  a.nblk = static_cast<int>(nblk_of(s));
  a.k_total = width;
  a.hsplit = hsplit;
  a.route = route;
  a.attend = attend;
  a.lds_floats = lds;
  a.kv_len = s->kv_len;
  a.force = force;
  a.score_scale = score_scale != 0.f ? score_scale : 1.f / std::sqrt(static_cast<float>(s->head_dim));
  a.sm_scale = sm_scale != 0.f ? sm_scale : 1.f / std::sqrt(static_cast<float>(s->head_dim));
  a.bf16 = s->dtype == BSA_BF16;
  a.out_f32 = o_dtype == BSA_F32;
  return BSA_OK;
}

}  // namespace

extern "C" {

const char* bsa_last_error(void) { return g_err.c_str(); }

const char* bsa_version(void) { return "libbsa 0.1 (gfx950)"; }

size_t bsa_workspace_size(int32_t op, const bsa_shape* s, int32_t k_or_cap) {
  if (check_shape(s) != BSA_OK) return 0;
  switch (op) {
    case BSA_OP_ROUTE_TOPK:
      // decode: the size also admits the partitioned path for any force flags
      return s->mode == BSA_DECODE ? std::max(ws_route_topk(s), ws_route_topk(s, k_or_cap, 7u))
                                   : ws_route_topk(s);
    case BSA_OP_DECODE_TOPK: {
      if (s->mode != BSA_DECODE || k_or_cap < 1) return 0;
      const int parts = decode_parts(s, k_or_cap, 7u);
      return parts > 0 ? decode_ws(s, parts, k_or_cap, true).total : 0;
    }
    case BSA_OP_ROUTE_ENTMAX:
      return ws_route_entmax(s);
    case BSA_OP_ATTEND_PREFILL:
      return s->mode == BSA_TOKEN ? mask_ws(s, false).total : 0;
    case BSA_OP_ATTEND_PREFILL_PRIOR:
      return s->mode == BSA_TOKEN ? mask_ws(s, true).total : 0;
    case BSA_OP_ATTEND_BACKWARD:
    case BSA_OP_ATTEND_BACKWARD_PRIOR:
      return (s->mode == BSA_PREFILL || s->mode == BSA_TOKEN) && k_or_cap >= 1
                 ? bwd_ws(s, k_or_cap, op == BSA_OP_ATTEND_BACKWARD_PRIOR).total
                 : 0;
    case BSA_OP_ROUTE_ENTMAX_BACKWARD:
      return s->mode == BSA_PREFILL || s->mode == BSA_TOKEN ? route_bwd_ws(s).total : 0;
    case BSA_OP_ATTEND_ENTMAX_BACKWARD:
      // each query's <g, dP> / sum g and normaliser
      return s->mode == BSA_PREFILL
                 ? 2 * align_up(static_cast<size_t>(s->batch) * s->n_q_heads * s->q_len * 4)
                 : 0;
    default:
      return 0;
  }
}

int bsa_summarize(const bsa_shape* s, const void* K, const float* qbar, float* S, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if ((rc = check_ptr("K", K)) != BSA_OK) return rc;
  if ((rc = check_ptr("S", S)) != BSA_OK) return rc;
  if (qbar && !aligned16(qbar)) return fail(BSA_ERR_UNSUPPORTED, "qbar must be 16-byte aligned");
  if ((rc = check_strides("K", s->k_stride, s->dtype)) != BSA_OK) return rc;
  bsa::SummarizeArgs a{};
  a.K = K;
  a.ks = st3(s->k_stride);
  a.qbar = qbar;
  a.S = S;
  a.blk = nullptr;
  a.batch = s->batch;
  a.hkv = s->n_kv_heads;
  a.d = s->head_dim;
  a.B = s->block;
  a.nblk = static_cast<int>(nblk_of(s));
  a.kv_len = s->kv_len;
  a.bf16 = s->dtype == BSA_BF16;
  return device_status(bsa::launch_summarize(a, static_cast<hipStream_t>(stream)), "summarize");
}

int bsa_summarize_blocks(const bsa_shape* s, const void* K, const float* qbar, const int32_t* blk,
                         float* S, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if ((rc = check_ptr("K", K)) != BSA_OK) return rc;
  if ((rc = check_ptr("S", S)) != BSA_OK) return rc;
  if (!blk) return fail(BSA_ERR_INVALID, "blk must not be NULL");
  if (qbar && !aligned16(qbar)) return fail(BSA_ERR_UNSUPPORTED, "qbar must be 16-byte aligned");
  if ((rc = check_strides("K", s->k_stride, s->dtype)) != BSA_OK) return rc;
  bsa::SummarizeArgs a{};
  a.K = K;
  a.ks = st3(s->k_stride);
  a.qbar = qbar;
  a.S = S;
  a.blk = blk;
  a.batch = s->batch;
  a.hkv = s->n_kv_heads;
  a.d = s->head_dim;
  a.B = s->block;
  a.nblk = static_cast<int>(nblk_of(s));
  a.kv_len = s->kv_len;
  a.bf16 = s->dtype == BSA_BF16;
  return device_status(bsa::launch_summarize(a, static_cast<hipStream_t>(stream)),
                       "summarize_blocks");
}

int bsa_route_topk(const bsa_shape* s, const void* Q, const float* S, const int32_t* kv_lens,
                   int32_t k_total, uint32_t force, float score_scale, int32_t* idx, int32_t* cnt,
                   float* scores_out, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if ((rc = check_force(s, force)) != BSA_OK) return rc;
  if (k_total < 1 || k_total < popcount3(force))
    return fail(BSA_ERR_INVALID, "k_total (%d) must be >= 1 and >= the number of forced blocks",
                k_total);
  if (!std::isfinite(score_scale)) return fail(BSA_ERR_INVALID, "score_scale must be finite");
  if ((rc = check_ptr("Q", Q)) != BSA_OK) return rc;
  if ((rc = check_ptr("S", S)) != BSA_OK) return rc;
  if (!idx || !cnt) return fail(BSA_ERR_INVALID, "idx and cnt must not be NULL");
  if (scores_out && !aligned16(scores_out))
    return fail(BSA_ERR_UNSUPPORTED, "scores_out must be 16-byte aligned");
  if ((rc = check_strides("Q", s->q_stride, s->dtype)) != BSA_OK) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (s->mode == BSA_DECODE && scores_out == nullptr) {
    bsa::DecodeArgs da{};
    if ((rc = decode_args(s, Q, nullptr, nullptr, S, kv_lens, idx, cnt, k_total, force,
                          score_scale, 0.f, nullptr, s->dtype, 1, 0, da)) != BSA_OK)
      return rc;
    const int parts = decode_parts(s, k_total, force);
    const DecodeWs dw = decode_ws(s, parts, k_total, false);
    if (parts > 0 && ws != nullptr && ws_bytes >= dw.total &&
        (reinterpret_cast<uintptr_t>(ws) % kAlign) == 0) {
      // partitioned routing: every CU streams a distinct slice of the summaries
      char* base = static_cast<char*>(ws);
      da.parts = parts;
      da.mpad = k_total;
      da.cand_key = reinterpret_cast<uint32_t*>(base);
      da.cand_id = reinterpret_cast<int32_t*>(base + dw.cand);
      da.part = nullptr;
      return device_status(bsa::launch_decode_parts(da, st), "route_topk/decode");
    }
    // one workgroup per row, scores never leave LDS
    return device_status(bsa::launch_decode_fused(da, st), "route_topk/decode");
  }
  const int nrow = static_cast<int>(nrow_of(s));
  const int nblk = static_cast<int>(nblk_of(s));
  const size_t rows = static_cast<size_t>(s->batch) * s->n_kv_heads * nrow;
  if ((rc = check_ws(ws, ws_bytes, ws_route_topk(s))) != BSA_OK) return rc;
  float* qhat = static_cast<float*>(ws);
  float* scores = scores_out ? scores_out
                             : reinterpret_cast<float*>(static_cast<char*>(ws) +
                                                        align_up(rows * s->head_dim * 4));
  bsa::QPoolArgs qp;
  qp.Q = Q;
  qp.qs = st3(s->q_stride);
  qp.qhat = qhat;
  qp.batch = s->batch;
  qp.hq = s->n_q_heads;
  qp.hkv = s->n_kv_heads;
  qp.d = s->head_dim;
  qp.B = s->mode == BSA_TOKEN ? 1 : s->block;  // token rows: the query itself
  qp.nrow = nrow;
  qp.q_len = s->q_len;
  qp.bf16 = s->dtype == BSA_BF16;
  qp.group_sum = true;
  hipError_t e = bsa::launch_qpool(qp, st);
  if (e != hipSuccess) return device_status(e, "route_topk/qpool");
  bsa::ScoreArgs sa;
  sa.qhat = qhat;
  sa.S = S;
  sa.scores = scores;
  sa.batch = s->batch;
  sa.hkv = s->n_kv_heads;
  sa.qheads = s->n_kv_heads;  // q-hat summed over each group
  sa.group = 1;
  sa.nrow = nrow;
  sa.nblk = nblk;
  sa.d = s->head_dim;
  sa.scale = score_scale != 0.f ? score_scale : 1.f / std::sqrt(static_cast<float>(s->head_dim));
  sa.rule = rule_of(s, 0, force, kv_lens);
  e = bsa::launch_scores(sa, st, scores_out != nullptr);
  if (e != hipSuccess) return device_status(e, "route_topk/scores");
  bsa::SelectArgs se;
  se.scores = scores;
  se.idx = idx;
  se.cnt = cnt;
  se.batch = s->batch;
  se.hkv = s->n_kv_heads;
  se.nrow = nrow;
  se.nblk = nblk;
  se.k_total = k_total;
  se.rule = sa.rule;
  return device_status(bsa::launch_select_topk(se, st), "route_topk/select");
}

int bsa_route_entmax(const bsa_shape* s, const void* Q, const float* S, const int32_t* kv_lens,
                     float alpha, float gamma, int32_t n_bins, int32_t max_iter, int32_t cap,
                     uint32_t force, float score_scale, int32_t* idx, int32_t* cnt,
                     float* probs_out, float* tau_out, float* wsel_out, void* ws, size_t ws_bytes,
                     void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if ((rc = check_force(s, force)) != BSA_OK) return rc;
  if (!(alpha > 1.f) || !std::isfinite(alpha)) return fail(BSA_ERR_INVALID, "alpha must be > 1");
  if (!std::isfinite(gamma)) return fail(BSA_ERR_INVALID, "gamma must be finite");
  if (n_bins != 16) return fail(BSA_ERR_INVALID, "n_bins must be 16 (got %d)", n_bins);
  if (max_iter < 0 || max_iter > 32)
    return fail(BSA_ERR_INVALID, "max_iter must be in [0, 32] (got %d)", max_iter);
  if (cap < 1) return fail(BSA_ERR_INVALID, "cap must be >= 1 (got %d)", cap);
  if (!std::isfinite(score_scale)) return fail(BSA_ERR_INVALID, "score_scale must be finite");
  if ((rc = check_ptr("Q", Q)) != BSA_OK) return rc;
  if ((rc = check_ptr("S", S)) != BSA_OK) return rc;
  if (!idx || !cnt) return fail(BSA_ERR_INVALID, "idx and cnt must not be NULL");
  if ((rc = check_strides("Q", s->q_stride, s->dtype)) != BSA_OK) return rc;
  if ((rc = check_ws(ws, ws_bytes, ws_route_entmax(s))) != BSA_OK) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const int nrow = static_cast<int>(nrow_of(s));
  const int nblk = static_cast<int>(nblk_of(s));
  const size_t hrows = static_cast<size_t>(s->batch) * s->n_q_heads * nrow;
  float* qhat = static_cast<float*>(ws);
  float* xbuf = reinterpret_cast<float*>(static_cast<char*>(ws) + align_up(hrows * s->head_dim * 4));
  bsa::QPoolArgs qp;
  qp.Q = Q;
  qp.qs = st3(s->q_stride);
  qp.qhat = qhat;
  qp.batch = s->batch;
  qp.hq = s->n_q_heads;
  qp.hkv = s->n_kv_heads;
  qp.d = s->head_dim;
  qp.B = s->mode == BSA_TOKEN ? 1 : s->block;
  qp.nrow = nrow;
  qp.q_len = s->q_len;
  qp.bf16 = s->dtype == BSA_BF16;
  qp.group_sum = false;
  hipError_t e = bsa::launch_qpool(qp, st);
  if (e != hipSuccess) return device_status(e, "route_entmax/qpool");
  const float scale =
      score_scale != 0.f ? score_scale : 1.f / std::sqrt(static_cast<float>(s->head_dim));
  // logits x = (alpha - 1) gamma score_scale q-hat . s of every query head,
  // -inf outside the candidates
  bsa::ScoreArgs sa;
  sa.qhat = qhat;
  sa.S = S;
  sa.scores = xbuf;
  sa.batch = s->batch;
  sa.hkv = s->n_kv_heads;
  sa.qheads = s->n_q_heads;
  sa.group = s->n_q_heads / s->n_kv_heads;
  sa.nrow = nrow;
  sa.nblk = nblk;
  sa.d = s->head_dim;
  sa.scale = (alpha - 1.f) * gamma * scale;
  sa.rule = rule_of(s, 1, force, kv_lens);
  e = bsa::launch_scores(sa, st, false);
  if (e != hipSuccess) return device_status(e, "route_entmax/scores");
  bsa::EntmaxArgs ea;
  ea.idx = idx;
  ea.cnt = cnt;
  ea.probs = probs_out;
  ea.tau = tau_out;
  ea.wsel = wsel_out;
  ea.xbuf = xbuf;
  ea.batch = s->batch;
  ea.hq = s->n_q_heads;
  ea.hkv = s->n_kv_heads;
  ea.nrow = nrow;
  ea.nblk = nblk;
  ea.width = cap + popcount3(force);
  ea.cap = cap;
  ea.max_iter = max_iter;
  ea.alpha = alpha;
  ea.rule = rule_of(s, 1, force, kv_lens);
  return device_status(bsa::launch_route_entmax(ea, st), "route_entmax");
}

static int attend_common(const bsa_shape* s, const void* Q, const void* K, const void* V,
                         const int32_t* idx, const int32_t* cnt, int32_t k_max, float sm_scale,
                         void* O, int32_t o_dtype, bsa::AttendArgs& a) {
  int rc;
  if ((rc = check_ptr("Q", Q)) != BSA_OK) return rc;
  if ((rc = check_ptr("K", K)) != BSA_OK) return rc;
  if ((rc = check_ptr("V", V)) != BSA_OK) return rc;
  if ((rc = check_ptr("O", O)) != BSA_OK) return rc;
  if (!idx || !cnt) return fail(BSA_ERR_INVALID, "idx and cnt must not be NULL");
  if (k_max < 1) return fail(BSA_ERR_INVALID, "k_max must be >= 1");
  if (!std::isfinite(sm_scale) || sm_scale < 0.f)
    return fail(BSA_ERR_INVALID, "sm_scale must be finite and >= 0 (0: 1/sqrt(d))");
  if (o_dtype != s->dtype && o_dtype != BSA_F32)
    return fail(BSA_ERR_UNSUPPORTED, "o_dtype must be the input dtype or BSA_F32");
  if ((rc = check_strides("Q", s->q_stride, s->dtype)) != BSA_OK) return rc;
  if ((rc = check_strides("K", s->k_stride, s->dtype)) != BSA_OK) return rc;
  if ((rc = check_strides("V", s->v_stride, s->dtype)) != BSA_OK) return rc;
  if ((rc = check_strides("O", s->o_stride, o_dtype)) != BSA_OK) return rc;
  // rows of one head are addressed with 32-bit offsets and must not overlap
  const int64_t esz = elem_bytes(s->dtype);
  const struct { const char* n; const int64_t* st; int64_t len; } heads[3] = {
      {"Q", s->q_stride, s->q_len}, {"K", s->k_stride, s->kv_len}, {"V", s->v_stride, s->kv_len}};
  for (const auto& hd : heads) {
    if (hd.st[2] < s->head_dim)
      return fail(BSA_ERR_INVALID, "%s token stride must be >= head_dim", hd.n);
    if ((hd.len + 128) * hd.st[2] * esz >= (int64_t(1) << 31))
      return fail(BSA_ERR_UNSUPPORTED, "%s: one head spans more than 2 GiB", hd.n);
  }
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.qs = st3(s->q_stride);
  a.ks = st3(s->k_stride);
  a.vs = st3(s->v_stride);
  a.os = st3(s->o_stride);
  a.idx = idx;
  a.cnt = cnt;
  a.bits = nullptr;
  a.wsel = nullptr;
  a.tbias = nullptr;
  a.sigma = 0.f;
  a.lse = nullptr;
  a.batch = s->batch;
  a.hq = s->n_q_heads;
  a.hkv = s->n_kv_heads;
  a.d = s->head_dim;
  a.B = s->block;
  a.k_max = k_max;
  a.nrow = static_cast<int>(nrow_of(s));
  a.nblk = static_cast<int>(nblk_of(s));
  a.q_len = s->q_len;
  a.kv_len = s->kv_len;
  a.sm_scale = sm_scale != 0.f ? sm_scale : 1.f / std::sqrt(static_cast<float>(s->head_dim));
  a.bf16 = s->dtype == BSA_BF16;
  a.out_f32 = o_dtype == BSA_F32;
  return BSA_OK;
}

static int token_mask_args(const bsa_shape* s, const int32_t* idx, const int32_t* cnt,
                           int32_t width, int32_t* uidx, int32_t* ucnt, uint64_t* ubits,
                           bsa::TokenMaskArgs& m) {
  if (s->mode != BSA_TOKEN) return fail(BSA_ERR_INVALID, "per-token masks need BSA_TOKEN");
  if (!idx || !cnt) return fail(BSA_ERR_INVALID, "idx and cnt must not be NULL");
  if (!uidx || !ucnt || !ubits) return fail(BSA_ERR_INVALID, "uidx, ucnt and ubits must not be NULL");
  if (width < 1) return fail(BSA_ERR_INVALID, "width must be >= 1");
  if (nblk_of(s) > kMaxTokenBlocks)
    return fail(BSA_ERR_UNSUPPORTED, "per-token masks support at most %lld blocks",
                (long long)kMaxTokenBlocks);
  m.idx = idx;
  m.cnt = cnt;
  m.uidx = uidx;
  m.ucnt = ucnt;
  m.ubits = ubits;
  m.batch = s->batch;
  m.hkv = s->n_kv_heads;
  m.width = width;
  m.nblk = static_cast<int>(nblk_of(s));
  m.ntile = static_cast<int>(ntile_of(s));
  m.q_len = s->q_len;
  m.wsel = nullptr;
  m.ubias = nullptr;
  m.sigma = 0.f;
  return BSA_OK;
}

int bsa_token_mask(const bsa_shape* s, const int32_t* idx, const int32_t* cnt, int32_t width,
                   int32_t* uidx, int32_t* ucnt, uint64_t* ubits, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  bsa::TokenMaskArgs m;
  if ((rc = token_mask_args(s, idx, cnt, width, uidx, ucnt, ubits, m)) != BSA_OK) return rc;
  return device_status(bsa::launch_token_mask(m, static_cast<hipStream_t>(stream)), "token_mask");
}

int bsa_attend_prefill(const bsa_shape* s, const void* Q, const void* K, const void* V,
                       const int32_t* idx, const int32_t* cnt, int32_t k_max, float sm_scale,
                       const float* wsel, float sigma, void* O, int32_t o_dtype, float* lse,
                       void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if (s->mode == BSA_DECODE)
    return fail(BSA_ERR_INVALID, "bsa_attend_prefill needs BSA_PREFILL or BSA_TOKEN");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return fail(BSA_ERR_UNSUPPORTED, "lse must be 4-byte aligned");
  if (!std::isfinite(sigma)) return fail(BSA_ERR_INVALID, "sigma must be finite");
  if (wsel && !aligned16(wsel)) return fail(BSA_ERR_UNSUPPORTED, "wsel must be 16-byte aligned");
  bsa::AttendArgs a;
  if ((rc = attend_common(s, Q, K, V, idx, cnt, k_max, sm_scale, O, o_dtype, a)) != BSA_OK)
    return rc;
  a.lse = lse;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (s->mode == BSA_TOKEN) {
    // per-token selections -> tile masks (and prior bias) in ws -> masked
    // tile attention
    const MaskWs mw = mask_ws(s, wsel != nullptr);
    if ((rc = check_ws(ws, ws_bytes, mw.total)) != BSA_OK) return rc;
    char* base = static_cast<char*>(ws);
    bsa::TokenMaskArgs m;
    if ((rc = token_mask_args(s, idx, cnt, k_max, reinterpret_cast<int32_t*>(base),
                              reinterpret_cast<int32_t*>(base + mw.uidx + mw.ubits),
                              reinterpret_cast<uint64_t*>(base + mw.uidx), m)) != BSA_OK)
      return rc;
    if (wsel) {
      m.wsel = wsel;
      m.sigma = sigma;
      m.ubias = reinterpret_cast<float*>(base + mw.uidx + mw.ubits + mw.ucnt);
    }
    const hipError_t e = bsa::launch_token_mask(m, st);
    if (e != hipSuccess) return device_status(e, "attend_prefill/token_mask");
    a.idx = m.uidx;
    a.cnt = m.ucnt;
    a.bits = m.ubits;
    a.tbias = m.ubias;
    a.k_max = m.nblk;
    a.nrow = m.ntile;
  } else if (wsel) {
    a.wsel = wsel;
    a.sigma = sigma;
  }
  return device_status(bsa::launch_attend_prefill(a, st), "attend_prefill");
}

int bsa_attend_decode(const bsa_shape* s, const void* Q, const void* K, const void* V,
                      const int32_t* kv_lens, const int32_t* idx, const int32_t* cnt,
                      int32_t k_max, float sm_scale, void* O, int32_t o_dtype, void* ws,
                      size_t ws_bytes, void* stream) {
  (void)ws;
  (void)ws_bytes;
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if (s->mode != BSA_DECODE) return fail(BSA_ERR_INVALID, "bsa_attend_decode needs BSA_DECODE");
  if (!idx || !cnt) return fail(BSA_ERR_INVALID, "idx and cnt must not be NULL");
  if (k_max < 1) return fail(BSA_ERR_INVALID, "k_max must be >= 1");
  bsa::DecodeArgs a;
  if ((rc = decode_args(s, Q, K, V, nullptr, kv_lens, const_cast<int32_t*>(idx),
                        const_cast<int32_t*>(cnt), k_max, 0u, 0.f, sm_scale, O, o_dtype, 0, 1,
                        a)) != BSA_OK)
    return rc;
  return device_status(bsa::launch_decode_fused(a, static_cast<hipStream_t>(stream)),
                       "attend_decode");
}

static int decode_topk_impl(const bsa_shape* s, const bsa_pages* pg, const void* Q,
                            const void* K, const void* V, const float* S,
                            const int32_t* kv_lens, int32_t k_total, uint32_t force,
                            float score_scale, float sm_scale, int32_t* idx, int32_t* cnt,
                            void* O, int32_t o_dtype, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if ((rc = check_force(s, force)) != BSA_OK) return rc;
  if (k_total < 1 || k_total < popcount3(force))
    return fail(BSA_ERR_INVALID, "k_total (%d) must be >= 1 and >= the number of forced blocks",
                k_total);
  if ((idx == nullptr) != (cnt == nullptr))
    return fail(BSA_ERR_INVALID, "idx and cnt must both be given or both be NULL");
  bsa::DecodeArgs a;
  if ((rc = decode_args(s, Q, K, V, S, kv_lens, idx, cnt, k_total, force, score_scale, sm_scale,
                        O, o_dtype, 1, 1, a, pg)) != BSA_OK)
    return rc;
  const int parts = decode_parts(s, k_total, force);
  const DecodeWs dw = decode_ws(s, parts, k_total, true);
  if ((rc = check_ws(ws, ws_bytes, dw.total)) != BSA_OK) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  if (parts == 0)
    return device_status(bsa::launch_decode_fused(a, st), "decode_topk");
  char* base = static_cast<char*>(ws);
  a.parts = parts;
  a.mpad = k_total;
  a.cand_key = reinterpret_cast<uint32_t*>(base);
  a.cand_id = reinterpret_cast<int32_t*>(base + dw.cand);
  a.part = reinterpret_cast<float*>(base + 2 * dw.cand);
  return device_status(bsa::launch_decode_parts(a, st), "decode_topk");
}

int bsa_attend_backward(const bsa_shape* s, const void* Q, const void* K, const void* V,
                        const void* O, int32_t o_dtype, const void* dO, const float* lse,
                        const int32_t* idx, const int32_t* cnt, int32_t k_max, float sm_scale,
                        const float* wsel, float sigma, float* dwsel, void* dQ, void* dK,
                        void* dV, int32_t g_dtype, void* ws, size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  const bool tok = s->mode == BSA_TOKEN;
  if (s->mode != BSA_PREFILL && !tok)
    return fail(BSA_ERR_INVALID, "bsa_attend_backward needs BSA_PREFILL or BSA_TOKEN");
  if (s->dtype != BSA_BF16)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_attend_backward supports bf16 inputs only");
  bsa::AttendArgs f;
  if ((rc = attend_common(s, Q, K, V, idx, cnt, k_max, sm_scale, const_cast<void*>(O), o_dtype,
                          f)) != BSA_OK)
    return rc;
  if ((rc = check_ptr("dO", dO)) != BSA_OK) return rc;
  if ((rc = check_ptr("dQ", dQ)) != BSA_OK) return rc;
  if ((rc = check_ptr("dK", dK)) != BSA_OK) return rc;
  if ((rc = check_ptr("dV", dV)) != BSA_OK) return rc;
  if (!lse) return fail(BSA_ERR_INVALID, "lse is NULL");
  if ((reinterpret_cast<uintptr_t>(lse) & 3u) != 0)
    return fail(BSA_ERR_UNSUPPORTED, "lse must be 4-byte aligned");
  if (g_dtype != s->dtype && g_dtype != BSA_F32)
    return fail(BSA_ERR_UNSUPPORTED, "g_dtype must be the input dtype or BSA_F32");
  if (!std::isfinite(sigma)) return fail(BSA_ERR_INVALID, "sigma must be finite");
  if (dwsel && !wsel) return fail(BSA_ERR_INVALID, "dwsel needs wsel");
  if ((wsel && (reinterpret_cast<uintptr_t>(wsel) & 3u) != 0) ||
      (dwsel && (reinterpret_cast<uintptr_t>(dwsel) & 3u) != 0))
    return fail(BSA_ERR_UNSUPPORTED, "wsel and dwsel must be 4-byte aligned");
  if (!tok && dwsel && k_max > bsa::attend_bwd_max_prior_width())
    return fail(BSA_ERR_UNSUPPORTED, "dwsel supports k_max <= %d with block rows",
                bsa::attend_bwd_max_prior_width());
  if (tok && nblk_of(s) > kMaxTokenBlocks)
    return fail(BSA_ERR_UNSUPPORTED, "per-token selections support at most %lld blocks",
                (long long)kMaxTokenBlocks);
  if ((rc = check_strides("dO", s->o_stride, s->dtype)) != BSA_OK) return rc;
  if ((rc = check_strides("dQ/dK/dV", s->q_stride, g_dtype)) != BSA_OK) return rc;
  const int64_t gsz = elem_bytes(g_dtype), osz = elem_bytes(o_dtype);
  if (s->o_stride[2] < s->head_dim) return fail(BSA_ERR_INVALID, "O token stride must be >= head_dim");
  if ((s->q_len + 128) * s->o_stride[2] * std::max(osz, gsz) >= (int64_t(1) << 31) ||
      (s->q_len + 128) * std::max({s->q_stride[2], s->k_stride[2], s->v_stride[2]}) * gsz >=
          (int64_t(1) << 31))
    return fail(BSA_ERR_UNSUPPORTED, "one head spans more than 2 GiB");
  if (nblk_of(s) > kMaxBwdBlocks)
    return fail(BSA_ERR_UNSUPPORTED, "the backward supports at most %lld blocks",
                (long long)kMaxBwdBlocks);
  const BwdWs bw = bwd_ws(s, k_max, wsel != nullptr);
  if (bw.max_items >= (int64_t(1) << 31)) return fail(BSA_ERR_UNSUPPORTED, "problem too large");
  if ((rc = check_ws(ws, ws_bytes, bw.total)) != BSA_OK) return rc;
  char* base = static_cast<char*>(ws);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    char* p = base + off;
    off += bytes;
    return p;
  };
  const hipStream_t st = static_cast<hipStream_t>(stream);
  bsa::BwdArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.dO = dO;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.qs = f.qs;
  a.ks = f.ks;
  a.vs = f.vs;
  a.os = f.os;
  a.lse = lse;
  a.idx = idx;
  a.cnt = cnt;
  a.delta = reinterpret_cast<float*>(take(bw.delta));
  a.bits = reinterpret_cast<uint32_t*>(take(bw.bits));
  a.items = reinterpret_cast<int4*>(take(bw.items));
  a.red = reinterpret_cast<int4*>(take(bw.red));
  a.counters = reinterpret_cast<int*>(take(bw.counters));
  a.part = reinterpret_cast<float*>(take(bw.part));
  float* dbpart = reinterpret_cast<float*>(take(bw.dbpart));
  a.sigma = wsel ? sigma : 0.f;
  a.dwsel = dwsel;
  a.units = bsa::attend_bwd_units(s->n_q_heads / s->n_kv_heads, tok ? 64 : s->block);
  a.rowq = s->block;
  if (tok) {
    // the tiles' masks (and per-query prior bias) first, as the forward builds them
    a.tpos = reinterpret_cast<int32_t*>(take(bw.tpos));
    int32_t* uidx = reinterpret_cast<int32_t*>(take(bw.uidx));
    uint64_t* ubits = reinterpret_cast<uint64_t*>(take(bw.ubits));
    int32_t* ucnt = reinterpret_cast<int32_t*>(take(bw.ucnt));
    float* ubias = reinterpret_cast<float*>(take(bw.ubias));
    float* dbtok = reinterpret_cast<float*>(take(bw.dbtok));
    bsa::TokenMaskArgs m;
    if ((rc = token_mask_args(s, idx, cnt, k_max, uidx, ucnt, ubits, m)) != BSA_OK) return rc;
    if (wsel) {
      m.wsel = wsel;
      m.sigma = sigma;
      m.ubias = ubias;
    }
    const hipError_t e = bsa::launch_token_mask(m, st);
    if (e != hipSuccess) return device_status(e, "attend_backward/token_mask");
    a.tok = true;
    a.rowq = 64;
    a.idx = uidx;
    a.cnt = ucnt;
    a.tbits = ubits;
    a.tbias = m.ubias;
    a.dbtok = dwsel ? dbtok : nullptr;
    a.nparts = bsa::attend_bwd_tok_parts(s->n_q_heads / s->n_kv_heads);
    a.pidx = idx;
    a.pcnt = cnt;
    a.pw = wsel;
    a.pwidth = k_max;
  } else {
    a.wsel = wsel;
    a.dbpart = dwsel ? dbpart : nullptr;
  }
  a.batch = s->batch;
  a.hq = s->n_q_heads;
  a.hkv = s->n_kv_heads;
  a.d = s->head_dim;
  a.B = s->block;
  a.k_max = tok ? f.nblk : k_max;
  a.nrow = static_cast<int>(bw.nrow);
  a.nblk = f.nblk;
  a.nwords = static_cast<int>(bw.nwords);
  a.chunk = kBwdChunk;
  a.max_items = static_cast<int>(bw.max_items);
  a.max_red = static_cast<int>(bw.max_red);
  a.n = s->q_len;
  a.sm_scale = f.sm_scale;
  a.bf16 = true;
  a.o_f32 = o_dtype == BSA_F32;
  a.g_f32 = g_dtype == BSA_F32;
  static_assert(kBwdChunk <= 64, "chunk rows are staged in a 64-entry LDS list");
  return device_status(bsa::launch_attend_backward(a, st), "attend_backward");
}

int bsa_route_entmax_backward(const bsa_shape* s, const void* Q, const float* S,
                              const float* probs, const int32_t* idx, const int32_t* cnt,
                              int32_t width, const float* dwsel, float alpha, float gamma,
                              float score_scale, void* dQ, void* dK, int32_t g_dtype, void* ws,
                              size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  const bool tok = s->mode == BSA_TOKEN;
  if (s->mode != BSA_PREFILL && !tok)
    return fail(BSA_ERR_INVALID, "bsa_route_entmax_backward needs BSA_PREFILL or BSA_TOKEN");
  if ((rc = check_ptr("Q", Q)) != BSA_OK) return rc;
  if ((rc = check_ptr("S", S)) != BSA_OK) return rc;
  if ((rc = check_ptr("probs", probs)) != BSA_OK) return rc;
  if ((rc = check_ptr("dQ", dQ)) != BSA_OK) return rc;
  if ((rc = check_ptr("dK", dK)) != BSA_OK) return rc;
  if (!idx || !cnt || !dwsel) return fail(BSA_ERR_INVALID, "idx, cnt and dwsel must not be NULL");
  if (width < 1) return fail(BSA_ERR_INVALID, "width must be >= 1");
  if (!(alpha > 1.f) || !std::isfinite(alpha)) return fail(BSA_ERR_INVALID, "alpha must be > 1");
  if (!std::isfinite(gamma) || !std::isfinite(score_scale) || score_scale < 0.f)
    return fail(BSA_ERR_INVALID, "gamma must be finite and score_scale finite and >= 0");
  if (g_dtype != s->dtype && g_dtype != BSA_F32)
    return fail(BSA_ERR_UNSUPPORTED, "g_dtype must be the input dtype or BSA_F32");
  if ((rc = check_strides("Q", s->q_stride, s->dtype)) != BSA_OK) return rc;
  if ((rc = check_strides("dQ/dK", s->q_stride, g_dtype)) != BSA_OK) return rc;
  if ((rc = check_strides("dK", s->k_stride, g_dtype)) != BSA_OK) return rc;
  const RouteBwdWs w = route_bwd_ws(s);
  if ((rc = check_ws(ws, ws_bytes, w.total)) != BSA_OK) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  bsa::QPoolArgs qa{};
  qa.Q = Q;
  qa.qs = st3(s->q_stride);
  qa.qhat = reinterpret_cast<float*>(base);
  qa.batch = s->batch;
  qa.hq = s->n_q_heads;
  qa.hkv = s->n_kv_heads;
  qa.d = s->head_dim;
  qa.B = tok ? 1 : s->block;  // token rows: the query itself
  qa.nrow = static_cast<int>(nrow_of(s));
  qa.q_len = s->q_len;
  qa.bf16 = s->dtype == BSA_BF16;
  qa.group_sum = false;
  hipError_t e = bsa::launch_qpool(qa, st);
  if (e != hipSuccess) return device_status(e, "route_entmax_backward/qpool");
  bsa::RouteBwdArgs a{};
  a.qhat = qa.qhat;
  a.S = S;
  a.probs = probs;
  a.idx = idx;
  a.cnt = cnt;
  a.dwsel = dwsel;
  a.dz = reinterpret_cast<float*>(base + w.qhat);
  a.dqh = reinterpret_cast<float*>(base + w.qhat + w.dz);
  a.dsp = reinterpret_cast<float*>(base + w.qhat + w.dz + w.dqh);
  a.dQ = dQ;
  a.dK = dK;
  a.qs = st3(s->q_stride);
  a.ks = st3(s->k_stride);
  a.batch = s->batch;
  a.hq = s->n_q_heads;
  a.hkv = s->n_kv_heads;
  a.d = s->head_dim;
  a.B = s->block;
  a.nrow = qa.nrow;
  a.rowq = qa.B;
  a.rowdiv = tok ? s->block : 1;
  a.ksplit = bsa::route_bwd_key_splits(a.nrow);
  a.nblk = static_cast<int>(nblk_of(s));
  a.width = width;
  a.n = s->q_len;
  a.alpha = alpha;
  a.fscale = gamma * (score_scale != 0.f ? score_scale
                                          : 1.f / std::sqrt(static_cast<float>(s->head_dim)));
  a.g_f32 = g_dtype == BSA_F32;
  return device_status(bsa::launch_route_entmax_backward(a, st), "route_entmax_backward");
}

int bsa_attend_entmax_backward(const bsa_shape* s, const void* Q, const void* K, const void* V,
                               const void* dO, const float* tau, const uint32_t* live,
                               float alpha, float sm_scale,
                               void* dQ, void* dK, void* dV, int32_t g_dtype, void* ws,
                               size_t ws_bytes, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if (s->mode != BSA_PREFILL)
    return fail(BSA_ERR_INVALID, "bsa_attend_entmax_backward needs BSA_PREFILL");
  if (s->dtype != BSA_BF16)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_attend_entmax_backward supports bf16 inputs only");
  if (s->block != 64)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_attend_entmax_backward works on 64-token tiles (block 64)");
  if (!(alpha > 1.f) || !std::isfinite(alpha)) return fail(BSA_ERR_INVALID, "alpha must be > 1");
  if (alpha > 2.f) return fail(BSA_ERR_UNSUPPORTED, "alpha > 2 is not supported");
  bsa::AttendArgs f;
  const int32_t one = 1;
  if ((rc = attend_common(s, Q, K, V, &one, &one, 1, sm_scale, const_cast<void*>(dO), s->dtype,
                          f)) != BSA_OK)
    return rc;
  if ((rc = check_ptr("dQ", dQ)) != BSA_OK) return rc;
  if ((rc = check_ptr("dK", dK)) != BSA_OK) return rc;
  if ((rc = check_ptr("dV", dV)) != BSA_OK) return rc;
  if (!tau) return fail(BSA_ERR_INVALID, "tau is NULL");
  if ((reinterpret_cast<uintptr_t>(tau) & 3u) != 0)
    return fail(BSA_ERR_UNSUPPORTED, "tau must be 4-byte aligned");
  if (live && (reinterpret_cast<uintptr_t>(live) & 3u) != 0)
    return fail(BSA_ERR_UNSUPPORTED, "live must be 4-byte aligned");
  if ((s->q_len + 63) / 64 > 2048)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_attend_entmax_backward supports at most %d tokens",
                64 * 2048);
  if (g_dtype != s->dtype && g_dtype != BSA_F32)
    return fail(BSA_ERR_UNSUPPORTED, "g_dtype must be the input dtype or BSA_F32");
  if ((rc = check_strides("dQ/dK/dV", s->q_stride, g_dtype)) != BSA_OK) return rc;
  const size_t per = align_up(static_cast<size_t>(s->batch) * s->n_q_heads * s->q_len * 4);
  if ((rc = check_ws(ws, ws_bytes, 2 * per)) != BSA_OK) return rc;
  char* base = static_cast<char*>(ws);
  bsa::BwdArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.dO = dO;
  a.dQ = dQ;
  a.dK = dK;
  a.dV = dV;
  a.qs = f.qs;
  a.ks = f.ks;
  a.vs = f.vs;
  a.os = f.os;
  a.delta = reinterpret_cast<float*>(base);
  a.zbuf = reinterpret_cast<float*>(base + per);
  a.batch = s->batch;
  a.hq = s->n_q_heads;
  a.hkv = s->n_kv_heads;
  a.d = s->head_dim;
  a.B = 64;
  a.rowq = 64;
  a.k_max = 1;
  a.nrow = f.nrow;
  a.nblk = f.nblk;
  a.n = s->q_len;
  a.sm_scale = f.sm_scale;
  a.bf16 = true;
  a.g_f32 = g_dtype == BSA_F32;
  a.ent = true;
  a.alpha = alpha;
  a.tau = tau;
  a.live = live;
  a.nlw = static_cast<int>((f.nrow + 31) / 32);
  return device_status(bsa::launch_attend_backward(a, static_cast<hipStream_t>(stream)),
                       "attend_entmax_backward");
}

int bsa_attend_entmax(const bsa_shape* s, const void* Q, const void* K, const void* V,
                      float alpha, int32_t refine, float sm_scale, void* O, int32_t o_dtype,
                      float* tau_out, uint32_t* live_out, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if (s->mode != BSA_PREFILL) return fail(BSA_ERR_INVALID, "bsa_attend_entmax needs BSA_PREFILL");
  if (s->dtype != BSA_BF16) return fail(BSA_ERR_UNSUPPORTED, "bsa_attend_entmax takes bf16 inputs");
  if (!(alpha > 1.f) || !std::isfinite(alpha)) return fail(BSA_ERR_INVALID, "alpha must be > 1");
  if (alpha > 16.f)
    return fail(BSA_ERR_UNSUPPORTED, "bsa_attend_entmax supports 1 < alpha <= 16 (got %g)",
                static_cast<double>(alpha));
  if (refine < 0 || refine > 24)
    return fail(BSA_ERR_INVALID, "refine must be in [0, 24] (got %d)", refine);
  if ((s->q_len + 63) / 64 > bsa::entmax_attend_max_tiles())
    return fail(BSA_ERR_UNSUPPORTED, "bsa_attend_entmax supports at most %d tokens",
                64 * bsa::entmax_attend_max_tiles());
  if (tau_out && !aligned16(tau_out)) return fail(BSA_ERR_UNSUPPORTED, "tau_out must be 16-byte aligned");
  if (live_out && (reinterpret_cast<uintptr_t>(live_out) & 3u) != 0)
    return fail(BSA_ERR_UNSUPPORTED, "live_out must be 4-byte aligned");
  // the shared argument checks of the attention calls (a dummy selection)
  bsa::AttendArgs t;
  static const int32_t one = 0;
  if ((rc = attend_common(s, Q, K, V, &one, &one, 1, sm_scale, O, o_dtype, t)) != BSA_OK)
    return rc;
  bsa::EntmaxAttnArgs a{};
  a.Q = Q;
  a.K = K;
  a.V = V;
  a.O = O;
  a.qs = t.qs;
  a.ks = t.ks;
  a.vs = t.vs;
  a.os = t.os;
  a.tau = tau_out;
  a.live = live_out;
  a.batch = s->batch;
  a.hq = s->n_q_heads;
  a.hkv = s->n_kv_heads;
  a.d = s->head_dim;
  a.refine = refine;
  a.n = s->q_len;
  a.sm_scale = t.sm_scale;
  a.alpha = alpha;
  a.out_f32 = o_dtype == BSA_F32;
  return device_status(bsa::launch_entmax_attend(a, static_cast<hipStream_t>(stream)),
                       "attend_entmax");
}

int bsa_decode_topk(const bsa_shape* s, const void* Q, const void* K, const void* V,
                    const float* S, const int32_t* kv_lens, int32_t k_total, uint32_t force,
                    float score_scale, float sm_scale, int32_t* idx, int32_t* cnt, void* O,
                    int32_t o_dtype, void* ws, size_t ws_bytes, void* stream) {
  return decode_topk_impl(s, nullptr, Q, K, V, S, kv_lens, k_total, force, score_scale, sm_scale,
                          idx, cnt, O, o_dtype, ws, ws_bytes, stream);
}

}  // extern "C"

namespace {

// Scratch of bsa_decode_topk_noalloc: one copy per GPU, created with the
// code object.  In host code `scratch` names a host-side stand-in, not the
// device array: its device address comes from hipGetSymbolAddress, taken
// once per device with that device current, and only that address is ever
// handed to kernels.
__device__ __align__(256) unsigned char scratch[BSA_STATIC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;

int static_scratch(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(BSA_ERR_DEVICE, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(BSA_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      const hipError_t ge = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (ge != hipSuccess || !p)
        return fail(BSA_ERR_DEVICE, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(ge));
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return BSA_OK;
}

}  // namespace

extern "C" {

int bsa_decode_topk_noalloc(const bsa_shape* s, const void* Q, const void* K, const void* V,
                            const float* S, const int32_t* kv_lens, int32_t k_total,
                            uint32_t force, float score_scale, float sm_scale, int32_t* idx,
                            int32_t* cnt, void* O, int32_t o_dtype, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if (s->mode != BSA_DECODE) return fail(BSA_ERR_INVALID, "bsa_decode_topk_noalloc needs BSA_DECODE");
  if ((rc = check_force(s, force)) != BSA_OK) return rc;
  if (k_total < 1 || k_total < popcount3(force))
    return fail(BSA_ERR_INVALID, "k_total (%d) must be >= 1 and >= the number of forced blocks",
                k_total);
  if ((idx == nullptr) != (cnt == nullptr))
    return fail(BSA_ERR_INVALID, "idx and cnt must both be given or both be NULL");
  {
    // every argument is checked before the device is touched
    bsa::DecodeArgs probe;
    if ((rc = decode_args(s, Q, K, V, S, kv_lens, idx, cnt, k_total, force, score_scale, sm_scale,
                          O, o_dtype, 1, 1, probe, nullptr)) != BSA_OK)
      return rc;
  }
  const int parts = decode_parts(s, k_total, force);
  const size_t need = decode_ws(s, parts, k_total, true).total;
  if (need > BSA_STATIC_SCRATCH_BYTES)
    return fail(BSA_ERR_UNSUPPORTED,
                "this shape needs %zu bytes of scratch; the static array holds %zu",
                need, static_cast<size_t>(BSA_STATIC_SCRATCH_BYTES));
  void* ws = nullptr;
  if (need > 0 && (rc = static_scratch(&ws)) != BSA_OK) return rc;
  return decode_topk_impl(s, nullptr, Q, K, V, S, kv_lens, k_total, force, score_scale, sm_scale,
                          idx, cnt, O, o_dtype, ws, need, stream);
}

int bsa_decode_topk_paged(const bsa_shape* s, const bsa_pages* pages, const void* Q,
                          const void* K, const void* V, const float* S, const int32_t* kv_lens,
                          int32_t k_total, uint32_t force, float score_scale, float sm_scale,
                          int32_t* idx, int32_t* cnt, void* O, int32_t o_dtype, void* ws,
                          size_t ws_bytes, void* stream) {
  if (!pages) return fail(BSA_ERR_INVALID, "pages is NULL");
  return decode_topk_impl(s, pages, Q, K, V, S, kv_lens, k_total, force, score_scale, sm_scale,
                          idx, cnt, O, o_dtype, ws, ws_bytes, stream);
}

int bsa_summarize_blocks_paged(const bsa_shape* s, const bsa_pages* pages, const void* K,
                               const float* qbar, const int32_t* blk, float* S, void* stream) {
  int rc;
  if ((rc = check_shape(s)) != BSA_OK) return rc;
  if ((rc = check_pages(s, pages)) != BSA_OK) return rc;
  if ((rc = check_ptr("K", K)) != BSA_OK) return rc;
  if ((rc = check_ptr("S", S)) != BSA_OK) return rc;
  if (!blk) return fail(BSA_ERR_INVALID, "blk must not be NULL");
  if (qbar && !aligned16(qbar)) return fail(BSA_ERR_UNSUPPORTED, "qbar must be 16-byte aligned");
  if ((rc = check_strides("K", s->k_stride, s->dtype)) != BSA_OK) return rc;
  bsa::SummarizeArgs a{};
  a.K = K;
  a.ks = st3(s->k_stride);
  a.qbar = qbar;
  a.S = S;
  a.blk = blk;
  a.table = pages->table;
  a.max_pages = pages->max_pages;
  a.num_pages = pages->num_pages;
  a.page_k = pages->k_page_stride;
  a.batch = s->batch;
  a.hkv = s->n_kv_heads;
  a.d = s->head_dim;
  a.B = s->block;
  a.nblk = static_cast<int>(nblk_of(s));
  a.kv_len = s->kv_len;
  a.bf16 = s->dtype == BSA_BF16;
  return device_status(bsa::launch_summarize(a, static_cast<hipStream_t>(stream)),
                       "summarize_blocks_paged");
}

}  // extern "C"
