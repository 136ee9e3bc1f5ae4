// Backward of Stage 2: gradients of the causal block-sparse attention for a
// fixed selection ("AdaSplash-2", section 4: the backward pass dominates
// training time and only the nonzero blocks are visited; "DashAttention",
// Contribuições item 1: training through the sparse attention).
//
// With P the softmax weights recomputed from the forward's log-normaliser,
// Delta_t = dO_t . O_t and dS = P (dP - Delta), dP = dO V^T:
//   dQ = sm_scale dS K,  dK = sm_scale dS^T Q,  dV = P^T dO.
//
//   bwd_mark      bit r of word (r/32, j) of a KV head says that query block r
//                 selected key block j: the selection transposed, written
//                 whole (no atomics on global memory, nothing to clear).
//   bwd_plan      one workgroup: per key block the number of selecting rows,
//                 split into chunks of `chunk` rows; a flat list of work items
//                 (key block, chunk) ordered by (batch, KV head) then block,
//                 and the list of blocks whose chunks must be summed.  The
//                 items running at a time then belong to one or two KV heads,
//                 whose query and upstream-gradient rows (read once per
//                 selecting block) stay in the memory-side cache; within a
//                 head the blocks near the start, selected most, go first.
//   bwd_dq        query side, the forward's walk: one workgroup per (batch,
//                 KV head, query block, unit group) over the row's selected
//                 key tiles staged in LDS.  S^T = K Q^T and dP^T = V dO^T on
//                 bf16 MFMA, dS^T in fp32, dQ^T += K^T dS^T.  Also writes
//                 Delta for the key side.
//   bwd_dkv       key side: one workgroup per work item; each wave keeps 16
//                 keys' K and V fragments in registers and the rows' Q / dO
//                 tiles of every query head of the group stream through LDS.
//                 S = Q K^T, dP = dO V^T, dV^T += dO^T P, dK^T += Q^T dS.
//   bwd_reduce    blocks split into several chunks: the chunks' fp32 partials
//                 summed in chunk order (deterministic), then stored.
// Every gradient element is written exactly once; keys no query attends get 0.
//
// Per-token selections ("DashAttention", Estágio 1 routes every query and
// Estágio 2 masks each token to its own blocks): the rows are 64-query tiles
// whose lists are the unions of their tokens' blocks, each entry with the
// word of the tokens that chose it (and, with a prior, every token's own bias);
// both sides then zero P for the queries outside the word.  dL/dw of a token's
// entry is sigma / w times the sum of dS over the block's keys and the group's
// heads: the query side leaves per (entry, query) sums in order, and
// bwd_dwsel_tok maps each token's own entries onto them.
#include <algorithm>
#include <type_traits>

#include "common.hpp"
#include "kernels.hpp"
#include "walk.hpp"

namespace bsa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 lds_v4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kPlanThreads = 1024;
constexpr int kMaxTilesBwd = 256;  // tile-list chunk staged in LDS (query side)
constexpr int kMaxEntTilesDq = 2048;  // entmax query side: key tiles of one sequence
constexpr int kMaxPriorEntries = 80;  // list width with a prior (per-wave sums in LDS)
constexpr int kBwdQT = 2, kBwdNW = 4;  // query side: 16-query tiles per wave, waves

__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// A 64-row tile of D bf16 columns in LDS, rows padded by 16 elements: both
// the row fragments (16 rows x one 16-byte chunk per lane group) and the
// transposing reads (8 rows x 32 bytes per half-wave) then run without bank
// conflicts (measured with the LDS bank-conflict counter on gfx950; an XOR
// swizzle of the chunks conflicts on the row fragments).
template <int D>
struct Swz {
  static constexpr int ST = D + 16;  // row stride, elements
  // element offset of 16-byte chunk c of row r
  __device__ static __forceinline__ int at(int r, int c) { return r * ST + (c << 3); }
};

// Transposed MFMA operand from a row-major tile: lane l gets column
// 16 dt + l%16 of rows 32 kk + 4 (l/16) + e and 32 kk + 16 + 4 (l/16) + e,
// e < 4 (the key order of a packed probability fragment).
template <int D>
__device__ __forceinline__ uint4 tr_frag(const uint16_t* tile, int kk, int dt, int lane) {
  const int s16 = lane & 15;
  const int r = kk * 32 + (lane >> 4) * 4 + (s16 >> 2);
  const uint16_t* p = tile + Swz<D>::at(r, 2 * dt + ((s16 & 3) >> 1)) + 4 * (s16 & 1);
  const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p));
  const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(p + 16 * Swz<D>::ST));
  const uint2 u0 = __builtin_bit_cast(uint2, r0), u1 = __builtin_bit_cast(uint2, r1);
  return make_uint4(u0.x, u0.y, u1.x, u1.y);
}

// Row fragment: lane l gets row 16 rt + l%16, columns 32 ks + 8 (l/16) .. +7.
template <int D>
__device__ __forceinline__ uint4 row_frag(const uint16_t* tile, int rt, int ks, int lane) {
  return *reinterpret_cast<const uint4*>(tile + Swz<D>::at(rt * 16 + (lane & 15), ks * 4 + (lane >> 4)));
}

// Four fp32 weights per lane of two 16-row accumulator tiles -> one bf16
// operand fragment over 32 rows (rows 32kk + 4G + e, 32kk + 16 + 4G + e).
__device__ __forceinline__ uint4 pack_frag(const f32x4& a, const f32x4& b) {
  return make_uint4(pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                    pack_bf16x2(b[2], b[3]));
}

// Sum over the four lanes l, l^16, l^32, l^48.
__device__ __forceinline__ float xsum16(float v) { return swap32_sum(swap16_sum(v)); }

__device__ __forceinline__ int wave_incl_scan(int v) {
  const int lane = lane_id();
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const int t = __shfl_up(v, o, kWave);
    if (lane >= o) v += t;
  }
  return v;
}

// Exclusive prefix of v over the workgroup and its total.
template <int NT>
__device__ __forceinline__ int block_scan_int(int v, int* wave_tot, int& total) {
  constexpr int NW = NT / kWave;
  const int incl = wave_incl_scan(v);
  const int w = threadIdx.x / kWave;
  if (lane_id() == kWave - 1) wave_tot[w] = incl;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const int t = wave_tot[k];
    off += k < w ? t : 0;
    tot += t;
  }
  __syncthreads();
  total = tot;
  return off + incl - v;
}

// ---------------------------------------------------------------------------
// Transposed selection and work plan
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bwd_mark(BwdArgs a) {
  extern __shared__ uint32_t words[];  // [nblk]
  const int tid = threadIdx.x;
  const int wd = blockIdx.x % a.nwords;
  const int64_t pair = blockIdx.x / a.nwords;
  for (int j = tid; j < a.nblk; j += 256) words[j] = 0u;
  __syncthreads();
  const int r0 = wd * 32;
  const int nr = a.nrow - r0 < 32 ? a.nrow - r0 : 32;
  for (int e = tid; e < nr * a.k_max; e += 256) {
    const int rr = e / a.k_max, s = e - rr * a.k_max;
    const int64_t row = pair * a.nrow + r0 + rr;
    const int c = a.cnt[row];
    if (s < (c > a.k_max ? a.k_max : c)) {
      const int j = a.idx[row * a.k_max + s];
      // block j is attended by row r only when it starts at or before the
      // row's last query (j <= r for block rows, query and key blocks both B long)
      const bool live = !a.wsel || a.wsel[row * a.k_max + s] > 0.f;  // the prior drops w <= 0
      if (j >= 0 && j < a.nblk &&
          static_cast<int64_t>(j) * a.B <= static_cast<int64_t>(r0 + rr + 1) * a.rowq - 1 && live) {
        atomicOr(&words[j], 1u << rr);
        // token tiles: where block j sits in the row's list (read by the key side)
        if (a.tpos) a.tpos[(pair * a.nblk + j) * a.nrow + r0 + rr] = s;
      }
    }
  }
  __syncthreads();
  uint32_t* out = a.bits + (pair * a.nwords + wd) * a.nblk;
  for (int j = tid; j < a.nblk; j += 256) out[j] = words[j];
}

__global__ __launch_bounds__(kPlanThreads) void bwd_plan(BwdArgs a) {
  __shared__ int wave_tot[kPlanThreads / kWave];
  const int tid = threadIdx.x;
  const int npair = a.batch * a.hkv;
  const int64_t total = static_cast<int64_t>(npair) * a.nblk;
  int ibase = 0, sbase = 0, rbase = 0;
  for (int64_t x0 = 0; x0 < total; x0 += kPlanThreads) {
    const int64_t x = x0 + tid;
    int p = 0, j = 0, nch = 0;
    if (x < total) {
      p = static_cast<int>(x / a.nblk);
      j = static_cast<int>(x % a.nblk);
      const uint32_t* col = a.bits + static_cast<int64_t>(p) * a.nwords * a.nblk + j;
      int c = 0;
      for (int w = 0; w < a.nwords; ++w) c += __popc(col[static_cast<int64_t>(w) * a.nblk]);
      nch = c == 0 ? 1 : (c + a.chunk - 1) / a.chunk;  // an empty block still writes zeros
    }
    const bool multi = nch > 1;
    int ti, ts, tr;
    const int io = block_scan_int<kPlanThreads>(nch, wave_tot, ti);
    const int so = block_scan_int<kPlanThreads>(multi ? nch : 0, wave_tot, ts);
    const int ro = block_scan_int<kPlanThreads>(multi ? 1 : 0, wave_tot, tr);
    for (int c = 0; c < nch; ++c)
      a.items[ibase + io + c] = make_int4(p, j, c, multi ? sbase + so + c : -1);
    if (multi) a.red[rbase + ro] = make_int4(p, j, sbase + so, nch);
    ibase += ti;
    sbase += ts;
    rbase += tr;
  }
  if (tid == 0) {
    a.counters[0] = ibase;
    a.counters[1] = rbase;
  }
}

// ---------------------------------------------------------------------------
// Query side: dQ (and Delta)
// ---------------------------------------------------------------------------
template <int D>
struct DqLds {
  alignas(16) uint16_t k[2][64 * Swz<D>::ST];
  alignas(16) uint16_t v[2][64 * Swz<D>::ST];
};

// Entmax weights of a score: t = x - tau with x = (alpha - 1) sm_scale s;
// on the support (t > 0) the unnormalised weight t^(1/(alpha-1)) and the
// Jacobian weight t^((2-alpha)/(alpha-1)) (p^(2-alpha) up to the
// normaliser's power), with the closed forms of alpha = 1.5 and 2.
__device__ __forceinline__ void ent_pow(float t, float alpha, float ib, float ig, float& pb,
                                        float& pg) {
  if (alpha == 1.5f) {
    pb = t * t;
    pg = t;
  } else if (alpha == 2.f) {
    pb = t;
    pg = 1.f;
  } else {
    const float l2 = __log2f(t);
    pb = __builtin_amdgcn_exp2f(ib * l2);
    pg = __builtin_amdgcn_exp2f(ig * l2);
  }
}

// The query-side workgroups holding some head of the queries of sub-tile qs
// (units qs*G .. qs*G+G-1, NW units a workgroup) are first_wg .. last_wg.
__device__ __host__ inline int dq_first_wg(int qs, int G, int NW) { return qs * G / NW; }
__device__ __host__ inline int dq_last_wg(int qs, int G, int NW) { return (qs * G + G - 1) / NW; }

// QT query tiles of 16 per wavefront, NW wavefronts; a unit is one query head
// x 16 QT queries of the row, as in the forward kernel.  ENT: the
// token-level entmax attention (dense causal, tau per query): a first walk
// over the tiles gathers each query's normaliser and the VJP's mean
// <g, dP> / sum g, the second forms dz and dQ.  TOK: per-token selections
// (rows are 64-query tiles): a query whose token did not choose the tile's
// block gets P = 0, and with a prior each query's bias is its own sigma ln w;
// the sums of dS per (entry, query) over the group's heads (for dL/dw) go to
// dbtok, one part per workgroup holding some of those heads.
template <int D, int QT, int NW, bool ENT, bool TOK>
__global__ __launch_bounds__(NW * 64, 8 / NW) void bwd_dq(BwdArgs a, int wpb) {
  constexpr int NT = NW * 64;
  constexpr int QPW = 16 * QT;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int CPR = D / 8;
  constexpr int KTOT = 64 * CPR;
  constexpr int KITEMS = (KTOT + NT - 1) / NT;
  __shared__ DqLds<D> lds;
  __shared__ int lds_tiles[kMaxTilesBwd];
  __shared__ int lds_tent[kMaxTilesBwd];    // list entry of each tile
  __shared__ float lds_tbias[kMaxTilesBwd];  // prior bias of its block, score units
  __shared__ float lds_db[TOK ? 1 : NW][kMaxPriorEntries];  // per wave: dL/d(bias) per list entry
  __shared__ uint64_t lds_tbits[TOK ? kMaxTilesBwd : 1];   // TOK: the entry's token word
  __shared__ float lds_dbq[TOK ? 2 : 1][NW][16 * QT];      // TOK: per wave, per query: sum of dS
  // ENT: per wave, the key tiles where some of its queries has weight (found
  // by the gathering walk; the second walk skips the others)
  __shared__ uint32_t lds_wlive[ENT ? NW : 1][ENT ? kMaxEntTilesDq / 32 : 1];
  __shared__ int lds_ntiles;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int G = a.hq / a.hkv;
  const int nsub = a.B / 64;
  const int qsub = a.rowq / QPW;
  const int units = G * qsub;
  int pair, i, sub;
  map_wg(blockIdx.x, a.batch * a.hkv, a.nrow, wpb, pair, i, sub);
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int u = sub * NW + w;
  const bool active = u < units;
  const int hh = active ? u % G : 0;
  const int qs = active ? u / G : 0;
  const int h = g * G + hh;
  const int qpos0 = i * a.rowq + qs * QPW;
  int qs_max = 0;
  for (int uu = sub * NW; uu < sub * NW + NW && uu < units; ++uu) qs_max = max(qs_max, uu / G);
  int64_t qmax = static_cast<int64_t>(i) * a.rowq + qs_max * QPW + QPW - 1;
  if (qmax > a.n - 1) qmax = a.n - 1;

  const int64_t rowid = static_cast<int64_t>(pair) * a.nrow + i;
  int n = 0;
  if constexpr (!ENT) {
    n = a.cnt[rowid];
    n = n < 0 ? 0 : (n > a.k_max ? a.k_max : n);
  }
  TileWalk walk{a.idx + rowid * a.k_max, n, nsub, a.B, a.nblk, a.n, qmax};

  const auto rk = make_rsrc(static_cast<const uint16_t*>(a.K) + b * a.ks.b + g * a.ks.h,
                            head_bytes(a.n, a.ks.t, D, 2));
  const auto rv = make_rsrc(static_cast<const uint16_t*>(a.V) + b * a.vs.b + g * a.vs.h,
                            head_bytes(a.n, a.vs.t, D, 2));
  const uint32_t kst = static_cast<uint32_t>(a.ks.t * 2), vst = static_cast<uint32_t>(a.vs.t * 2);

  // Q and dO fragments (B operands): lane l holds query 16qt + l%16,
  // d = 32ks + 8(l/16) .. +7; rows past n read as zero.
  uint4 qf[QT][KS], df[QT][KS];
  float dl[QT], lse2[QT];
  const int64_t hrow = (static_cast<int64_t>(b) * a.hq + h) * a.n;
  if constexpr (ENT) {
    // entmax: Q and dO fragments, and tau (x units) in place of lse
    const auto rq = make_rsrc(static_cast<const uint16_t*>(a.Q) + b * a.qs.b + h * a.qs.h,
                              active ? head_bytes(a.n, a.qs.t, D, 2) : 0u);
    const auto rdo = make_rsrc(static_cast<const uint16_t*>(a.dO) + b * a.os.b + h * a.os.h,
                               active ? head_bytes(a.n, a.os.t, D, 2) : 0u);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int64_t t = qpos0 + qt * 16 + (lane & 15);
      const uint32_t tq = static_cast<uint32_t>(t);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c0 = ks * 32 + (lane >> 4) * 8;
        qf[qt][ks] = buf_load16(rq, tq * static_cast<uint32_t>(a.qs.t * 2) + c0 * 2);
        df[qt][ks] = buf_load16(rdo, tq * static_cast<uint32_t>(a.os.t * 2) + c0 * 2);
      }
      lse2[qt] = t < a.n ? a.tau[hrow + t] : INFINITY;  // past the end: no support
      dl[qt] = 0.f;
    }
  } else {
    const uint32_t qbytes = active ? head_bytes(a.n, a.qs.t, D, 2) : 0u;
    const uint32_t obytes = active ? head_bytes(a.n, a.os.t, D, a.o_f32 ? 4 : 2) : 0u;
    const auto rq = make_rsrc(static_cast<const uint16_t*>(a.Q) + b * a.qs.b + h * a.qs.h, qbytes);
    const auto rdo = make_rsrc(static_cast<const uint16_t*>(a.dO) + b * a.os.b + h * a.os.h,
                               active ? head_bytes(a.n, a.os.t, D, 2) : 0u);
    const int oes = a.o_f32 ? 4 : 2;
    const auto ro = make_rsrc(static_cast<const uint8_t*>(a.O) + (b * a.os.b + h * a.os.h) * oes,
                              obytes);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const int64_t t = qpos0 + qt * 16 + (lane & 15);
      const uint32_t tq = static_cast<uint32_t>(t);
      float part = 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c0 = ks * 32 + (lane >> 4) * 8;
        qf[qt][ks] = buf_load16(rq, tq * static_cast<uint32_t>(a.qs.t * 2) + c0 * 2);
        df[qt][ks] = buf_load16(rdo, tq * static_cast<uint32_t>(a.os.t * 2) + c0 * 2);
        float ov[8];
        if (a.o_f32)
          buf_load8_f32<float>(ro, tq * static_cast<uint32_t>(a.os.t * 4) + c0 * 4, ov);
        else
          buf_load8_f32<uint16_t>(ro, tq * static_cast<uint32_t>(a.os.t * 2) + c0 * 2, ov);
        const uint4 dv = df[qt][ks];
        part = fmaf(bf16_lo(dv.x), ov[0], part);
        part = fmaf(bf16_hi(dv.x), ov[1], part);
        part = fmaf(bf16_lo(dv.y), ov[2], part);
        part = fmaf(bf16_hi(dv.y), ov[3], part);
        part = fmaf(bf16_lo(dv.z), ov[4], part);
        part = fmaf(bf16_hi(dv.z), ov[5], part);
        part = fmaf(bf16_lo(dv.w), ov[6], part);
        part = fmaf(bf16_hi(dv.w), ov[7], part);
      }
      dl[qt] = xsum16(part);
      float L = t < a.n ? a.lse[hrow + t] : -INFINITY;
      // a query without weights (no key, or past the end) gets P = 0
      lse2[qt] = L > -INFINITY ? L * kLog2e : INFINITY;
      if (active && lane < 16 && t < a.n) a.delta[hrow + t] = dl[qt];
    }
  }

  f32x4 acc[DT][QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt)
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) acc[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  const float sc = a.sm_scale * kLog2e;

  uint4 kreg[KITEMS], vreg[KITEMS];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (KTOT % NT == 0 || flat < KTOT) {
        kreg[it] = buf_load16(rk, static_cast<uint32_t>(k0 + r) * kst + c * 16);
        vreg[it] = buf_load16(rv, static_cast<uint32_t>(k0 + r) * vst + c * 16);
      }
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (KTOT % NT == 0 || flat < KTOT) {
        *reinterpret_cast<uint4*>(&lds.k[buf][Swz<D>::at(r, c)]) = kreg[it];
        *reinterpret_cast<uint4*>(&lds.v[buf][Swz<D>::at(r, c)]) = vreg[it];
      }
    }
  };

  if (!TOK && a.dbpart)
    for (int e = lane; e < a.k_max; e += 64) lds_db[w][e] = 0.f;
  if constexpr (ENT)
    for (int e = lane; e < kMaxEntTilesDq / 32; e += 64) lds_wlive[w][e] = 0u;
  // entmax: per query column the sums over its keys of t^(1/(alpha-1)) (the
  // normaliser Z), of g dP and of g (g = t^((2-alpha)/(alpha-1)))
  const float a1s = (a.alpha - 1.f) * a.sm_scale;
  const float ib = 1.f / (a.alpha - 1.f), ig = (2.f - a.alpha) / (a.alpha - 1.f);
  float zs[QT], gds[QT], gs[QT], zf[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) zs[qt] = gds[qt] = gs[qt] = zf[qt] = 0.f;
  // entmax: all causal tiles, walked twice
  const int nraw = ENT ? static_cast<int>(qmax / 64) + 1 : n * nsub;
  // TOK with a prior: this lane's query columns' bias for the current and the
  // next tile (logit units, -inf where the token did not choose the block)
  float bcur[QT], bnxt[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) bcur[qt] = bnxt[qt] = 0.f;
  auto load_bias = [&](int tt, float (&dst)[QT]) {
    const float* bp = a.tbias + (rowid * a.k_max + lds_tent[tt]) * 64 + qs * QPW + (lane & 15);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) dst[qt] = bp[qt * 16];
  };
  const bool tok_bias = TOK && a.tbias != nullptr && active;
  float dbacc = 0.f;  // TOK, wave 0: this query's dS sum over the entry's tiles and heads

  // one walk over the tiles; entmax runs the gathering walk (0) first
  auto walk_pass = [&](auto pass_c) {
  constexpr int pass = decltype(pass_c)::value;
  for (int base = 0; base < nraw; base += kMaxTilesBwd) {
    if (w == 0) {
      int c = 0;
      for (int r = 0; r < kMaxTilesBwd && base + r < nraw; r += 64) {
        const int T = base + r + lane;
        int64_t k0 = T >= nraw ? -1 : (ENT ? 64 * static_cast<int64_t>(T) : walk.key0(T));
        // entmax with the forward's live tiles: only those have weights
        if (ENT && a.live && k0 >= 0 && !((a.live[rowid * a.nlw + (T >> 5)] >> (T & 31)) & 1u))
          k0 = -1;
        float tb = 0.f;
        if (!ENT && a.wsel && k0 >= 0) {
          // the prior: sigma ln w of the tile's block, dropped when w <= 0
          const float wv = a.wsel[rowid * a.k_max + T / nsub];
          if (wv > 0.f)
            tb = a.sigma * __logf(wv) / a.sm_scale;
          else
            k0 = -1;
        }
        const uint64_t mk = __ballot(k0 >= 0);
        if (k0 >= 0) {
          const int pos = c + lanes_below(mk);
          lds_tiles[pos] = static_cast<int>(k0);
          lds_tent[pos] = T / nsub;
          lds_tbias[pos] = tb;
          if constexpr (TOK) lds_tbits[pos] = a.tbits[rowid * a.k_max + T / nsub];
        }
        c += __popcll(mk);
      }
      if (lane == 0) lds_ntiles = c;
    }
    __syncthreads();
    const int ntiles = lds_ntiles;
    int buf = 0;
    if (ntiles > 0) {
      load_tile(lds_tiles[0]);
      if (tok_bias) load_bias(0, bcur);
      store_tile(0);
    }
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int k0 = lds_tiles[t];
      const bool more = t + 1 < ntiles;
      if (more) {
        load_tile(lds_tiles[t + 1]);
        if (tok_bias) load_bias(t + 1, bnxt);
      }
      // TOK: bit 16qt + c says whether query qpos0 + 16qt + c chose the
      // tile's block; a wave none of whose queries did has nothing to add
      const uint64_t qbits = TOK ? lds_tbits[t] >> (qs * QPW) : ~0ull;
      const bool wave_on = !TOK || (qbits & (QPW == 64 ? ~0ull : (1ull << QPW) - 1)) != 0;
      float dcol[QT];  // TOK: per query column, the sum of dS over the tile
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) dcol[qt] = 0.f;
      // a wave whose queries all precede the tile has nothing to add, and
      // (entmax, second walk) nor has one none of whose queries weights it
      const bool wave_live =
          !ENT || pass == 0 ||
          ((__builtin_amdgcn_readfirstlane(lds_wlive[w][(k0 >> 6) >> 5]) >> ((k0 >> 6) & 31)) & 1u);
      if (active && k0 <= qpos0 + QPW - 1 && wave_on && wave_live) {
        const uint16_t* kt_ = lds.k[buf];
        const uint16_t* vt_ = lds.v[buf];
        // exponent offset per query column: the bias minus lse
        float eoff[QT];
        const float tbs = lds_tbias[t] * sc;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          if constexpr (TOK) {
            const bool on = (qbits >> (qt * 16 + (lane & 15))) & 1ull;
            eoff[qt] = on ? (tok_bias ? bcur[qt] * kLog2e : 0.f) - lse2[qt] : -INFINITY;
          } else {
            eoff[qt] = tbs - lse2[qt];
          }
        }
        float dbs = 0.f;  // this wave's sum of dS over the tile (prior gradient)
        // S^T and dP^T, one 16-key slice at a time (lane l holds keys
        // 16kt + 4(l/16) + j of query column 16qt + l%16), turned into dS^T
        // and packed two slices per bf16 operand
        const bool diag = k0 + 63 > qpos0;
        const int rel0 = k0 - qpos0 + (lane >> 4) * 4 - (lane & 15);
        uint4 dsf[QT][2];
        f32x4 dsp[QT];
        bool pair_live[2];
        bool live_pair = false;  // entmax: some weight in the current pair of slices
        bool tile_live = false;  // entmax: some weight in the tile
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          f32x4 s[QT], dp[QT];
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            s[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
            dp[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
          if constexpr (ENT && pass == 0) {
            // S first: a 16-key slice outside every support of the wave's
            // queries has no dP, dz or dQ work (zero blocks skipped)
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              const uint4 kf = row_frag<D>(kt_, kt, ks, lane);
#pragma unroll
              for (int qt = 0; qt < QT; ++qt) s[qt] = mfma16(kf, qf[qt][ks], s[qt]);
            }
            bool any = false;
#pragma unroll
            for (int qt = 0; qt < QT; ++qt)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                any |= fmaf(s[qt][j], a1s, -lse2[qt]) > 0.f &&
                       !(diag && rel0 + kt * 16 + j - qt * 16 > 0);
            const bool live = __ballot(any) != 0;
            live_pair = (kt & 1) ? (live_pair || live) : live;
            tile_live |= live;
            if (live) {
#pragma unroll
              for (int ks = 0; ks < KS; ++ks) {
                const uint4 vf = row_frag<D>(vt_, kt, ks, lane);
#pragma unroll
                for (int qt = 0; qt < QT; ++qt) dp[qt] = mfma16(vf, df[qt][ks], dp[qt]);
              }
            }
          } else {
#pragma unroll
            for (int ks = 0; ks < KS; ++ks) {
              const uint4 kf = row_frag<D>(kt_, kt, ks, lane);
              const uint4 vf = row_frag<D>(vt_, kt, ks, lane);
#pragma unroll
              for (int qt = 0; qt < QT; ++qt) {
                s[qt] = mfma16(kf, qf[qt][ks], s[qt]);
                dp[qt] = mfma16(vf, df[qt][ks], dp[qt]);
              }
            }
            if constexpr (ENT) {
              // the dQ products of a pair of slices outside every support are skipped
              bool any = false;
#pragma unroll
              for (int qt = 0; qt < QT; ++qt)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                  any |= fmaf(s[qt][j], a1s, -lse2[qt]) > 0.f &&
                         !(diag && rel0 + kt * 16 + j - qt * 16 > 0);
              const bool live = __ballot(any) != 0;
              live_pair = (kt & 1) ? (live_pair || live) : live;
            }
          }
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            f32x4 ds;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const bool masked = diag && rel0 + kt * 16 + j - qt * 16 > 0;  // key after query
              if constexpr (ENT) {
                const float tt = fmaf(s[qt][j], a1s, -lse2[qt]);
                float pb = 0.f, pg = 0.f;
                if (tt > 0.f && !masked) ent_pow(tt, a.alpha, ib, ig, pb, pg);
                if constexpr (pass == 0) {
                  zs[qt] += pb;
                  gds[qt] = fmaf(pg, dp[qt][j], gds[qt]);
                  gs[qt] += pg;
                }
                if constexpr (pass == 1) ds[j] = zf[qt] * pg * (dp[qt][j] - dl[qt]);
              } else {
                float p = __builtin_amdgcn_exp2f(fmaf(s[qt][j], sc, eoff[qt]));
                if (masked) p = 0.f;
                ds[j] = p * (dp[qt][j] - dl[qt]);
                if constexpr (TOK)
                  dcol[qt] += ds[j];
                else
                  dbs += ds[j];
              }
            }
            if constexpr (pass == 1) {
              if (kt & 1)
                dsf[qt][kt >> 1] = pack_frag(dsp[qt], ds);
              else
                dsp[qt] = ds;
            }
          }
          if (kt & 1) pair_live[kt >> 1] = !ENT || live_pair;
        }
        // dQ^T += K^T dS^T
        if constexpr (pass == 1) {
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            if (!pair_live[kk]) continue;  // entmax: both slices outside every support
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              const uint4 kf = tr_frag<D>(kt_, kk, dt, lane);
#pragma unroll
              for (int qt = 0; qt < QT; ++qt) acc[dt][qt] = mfma16(kf, dsf[qt][kk], acc[dt][qt]);
            }
          }
        }
        if constexpr (ENT && pass == 0) {
          // (only this wave writes its words; the walks see the same tiles)
          if (lane == 0 && tile_live) lds_wlive[w][(k0 >> 6) >> 5] |= 1u << ((k0 >> 6) & 31);
        }
        if (!ENT && !TOK && a.dbpart) {
          // this unit's part of dL/d(bias) of the tile's list entry (a block
          // of two tiles adds twice)
          dbs = wave_sum(dbs);
          if (lane == 0) lds_db[w][lds_tent[t]] += dbs;
        }
      }
      if constexpr (TOK) {
        if (a.dbtok) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            const float v = xsum16(dcol[qt]);
            if (lane < 16) lds_dbq[buf][w][qt * 16 + lane] = v;
          }
        }
      }
      if (more) store_tile(buf ^ 1);
      if constexpr (TOK) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) bcur[qt] = bnxt[qt];
      }
      __syncthreads();
      if constexpr (TOK) {
        if (a.dbtok && w == 0) {
          // query `lane` of the row: add the heads this workgroup holds, and
          // store once the entry's last tile is done
          const int qsq = lane / QPW;
          bool mine = false;
#pragma unroll
          for (int w2 = 0; w2 < NW; ++w2) {
            const int u2 = sub * NW + w2;
            if (u2 < units && u2 / G == qsq) {
              dbacc += lds_dbq[buf][w2][lane % QPW];
              mine = true;
            }
          }
          const int e = lds_tent[t];
          if (t + 1 == ntiles || lds_tent[t + 1] != e) {
            if (mine)
              a.dbtok[((rowid * a.k_max + e) * a.nparts + sub - dq_first_wg(qsq, G, NW)) * 64 + lane] =
                  dbacc;
            dbacc = 0.f;
          }
        }
      }
      buf ^= 1;
    }
  }
  if constexpr (ENT && pass == 0) {
    // each query's normaliser and VJP mean, shared with the key side
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float z = xsum16(zs[qt]), gsum = xsum16(gs[qt]), gd = xsum16(gds[qt]);
      dl[qt] = gsum > 0.f ? gd / gsum : 0.f;
      // g = (t^(1/(alpha-1)) / Z)^(2-alpha) = t^((2-alpha)/(alpha-1)) Z^(alpha-2)
      zf[qt] = z > 0.f ? __builtin_amdgcn_exp2f((a.alpha - 2.f) * __log2f(z)) : 0.f;
      const int64_t t = qpos0 + qt * 16 + (lane & 15);
      if (active && lane < 16 && t < a.n) {
        a.delta[hrow + t] = dl[qt];
        a.zbuf[hrow + t] = z;
      }
    }
  }
  };
  if constexpr (ENT) walk_pass(std::integral_constant<int, 0>{});
  walk_pass(std::integral_constant<int, 1>{});

  if (!active) return;
  if (!TOK && a.dbpart)
    for (int e = lane; e < a.k_max; e += 64)
      a.dbpart[(rowid * a.units + u) * a.k_max + e] = lds_db[w][e];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int64_t t = qpos0 + qt * 16 + (lane & 15);
    if (t >= a.n) continue;
    const int64_t off = b * a.qs.b + h * a.qs.h + t * a.qs.t;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d0 = dt * 16 + (lane >> 4) * 4;
      const f32x4 v = acc[dt][qt] * a.sm_scale;
      if (a.g_f32) {
        *reinterpret_cast<float4*>(static_cast<float*>(a.dQ) + off + d0) = make_float4(v[0], v[1], v[2], v[3]);
      } else {
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dQ) + off + d0) =
            make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Key side: dK, dV
// ---------------------------------------------------------------------------
template <int D>
struct DkvLds {
  alignas(16) uint16_t q[2][64 * Swz<D>::ST];
  alignas(16) uint16_t o[2][64 * Swz<D>::ST];  // dO
  alignas(16) float lse2[2][64];
  alignas(16) float dl[2][64];
};
constexpr int kMaxChunk = 64;
constexpr int kMaxEntRows = 2048;  // entmax key side: query tiles a key tile can have

// NW = B / 16 wavefronts, wave w owning keys 16w .. 16w+15 of the block.
// ENT: the token-level entmax attention; one item per (KV head, key block),
// its rows every query block from the key block on (dense causal).
// Token tiles (a.tok): a query whose token did not choose block j, or whose
// bias is -inf, gets P = 0, and a prior's bias enters through the query's
// exponent offset (lse - bias).
template <int D, int NW, bool ENT>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dkv(BwdArgs a) {
  constexpr int NT = NW * 64;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int CPR = D / 8;
  constexpr int QTOT = 64 * CPR;
  constexpr int QITEMS = (QTOT + NT - 1) / NT;
  constexpr int B = NW * 16;
  __shared__ DkvLds<D> lds;
  __shared__ int rows[kMaxChunk];
  __shared__ float rbias[kMaxChunk];  // prior bias of block j in each row, score units
  __shared__ int rent[kMaxChunk];     // token tiles: the list entry of block j in each row
  __shared__ float lds_iz[ENT ? 2 : 1][64];  // entmax: 1 / Z of each query
  __shared__ float lds_zf[ENT ? 2 : 1][64];  // entmax: Z^(alpha-2)
  __shared__ uint16_t erows[ENT ? kMaxEntRows : 1];  // entmax with live tiles: the query tiles
  __shared__ int lds_nr;

  int pair, j, chunk = 0, slot = -1;
  if constexpr (ENT) {
    // key blocks near the start have the most rows: they go first
    const int npair = a.batch * a.hkv;
    j = static_cast<int>(blockIdx.x / npair);
    pair = static_cast<int>(blockIdx.x % npair);
  } else {
    if (static_cast<int>(blockIdx.x) >= a.counters[0]) return;
    const int4 item = a.items[blockIdx.x];
    pair = item.x;
    j = item.y;
    chunk = item.z;
    slot = item.w;
  }
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int G = a.hq / a.hkv;

  // rows of this chunk: ranks [chunk * a.chunk, +a.chunk) among the set bits
  // of block j's column, ascending
  if (ENT) {
    if (!a.live) {
      if (tid == 0) lds_nr = a.nrow - j;
    } else if (w == 0) {
      // the query tiles from j on whose live row holds key tile j
      int c = 0;
      for (int base = j; base < a.nrow; base += 64) {
        const int i = base + lane;
        const bool on = i < a.nrow &&
                        ((a.live[(static_cast<int64_t>(pair) * a.nrow + i) * a.nlw + (j >> 5)] >>
                          (j & 31)) & 1u);
        const uint64_t mk = __ballot(on);
        if (on) erows[c + lanes_below(mk)] = static_cast<uint16_t>(i);
        c += __popcll(mk);
      }
      if (lane == 0) lds_nr = c;
    }
  } else if (w == 0) {
    const int lo = chunk * a.chunk, hi = lo + a.chunk;
    const uint32_t* col = a.bits + static_cast<int64_t>(pair) * a.nwords * a.nblk + j;
    int base = 0;
    for (int w0 = 0; w0 < a.nwords && base < hi; w0 += 64) {
      const int wi = w0 + lane;
      uint32_t word = wi < a.nwords ? col[static_cast<int64_t>(wi) * a.nblk] : 0u;
      const int pc = __popc(word);
      const int incl = wave_incl_scan(pc);
      int rank = base + incl - pc;
      while (word != 0u && rank < hi) {
        const int bit = __builtin_ctz(word);
        word &= word - 1u;
        if (rank >= lo) rows[rank - lo] = wi * 32 + bit;
        ++rank;
      }
      base += __shfl(incl, 63, kWave);
    }
    if (lane == 0) lds_nr = base <= lo ? 0 : (base < hi ? base : hi) - lo;
  }

  // K and V fragments of this wave's keys (B operands of S = Q K^T and
  // dP = dO V^T): lane l holds key 16w + l%16, d = 32ks + 8(l/16) .. +7
  const int64_t key0 = static_cast<int64_t>(j) * B + w * 16;
  uint4 kf[KS], vf[KS];
  {
    const auto rk = make_rsrc(static_cast<const uint16_t*>(a.K) + b * a.ks.b + g * a.ks.h,
                              head_bytes(a.n, a.ks.t, D, 2));
    const auto rv = make_rsrc(static_cast<const uint16_t*>(a.V) + b * a.vs.b + g * a.vs.h,
                              head_bytes(a.n, a.vs.t, D, 2));
    const uint32_t t = static_cast<uint32_t>(key0 + (lane & 15));
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      const int c0 = ks * 32 + (lane >> 4) * 8;
      kf[ks] = buf_load16(rk, t * static_cast<uint32_t>(a.ks.t * 2) + c0 * 2);
      vf[ks] = buf_load16(rv, t * static_cast<uint32_t>(a.vs.t * 2) + c0 * 2);
    }
  }
  f32x4 dk[DT], dv[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    dk[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
    dv[dt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  __syncthreads();
  const int nr = lds_nr;
  if (!ENT && a.tok)
    for (int i = tid; i < nr; i += NT) rent[i] = a.tpos[(static_cast<int64_t>(pair) * a.nblk + j) * a.nrow + rows[i]];
  if (!ENT && a.wsel) {
    // the routing weight of block j in each row's list: 8 threads per row
    // scan the entries (a row lists j once; rows only hold j when w > 0)
    for (int i = tid / 8; i < nr; i += NT / 8) {
      const int64_t row = static_cast<int64_t>(pair) * a.nrow + rows[i];
      const int c = min(a.cnt[row], a.k_max);
      for (int e = tid % 8; e < c; e += 8)
        if (a.idx[row * a.k_max + e] == j)
          rbias[i] = a.sigma * __logf(a.wsel[row * a.k_max + e]) / a.sm_scale;
    }
  }
  __syncthreads();
  // queries per row: 64 whenever the key block is (block rows of 64, token
  // tiles, entmax), so the unit arithmetic below folds to constants there
  const int rowq = (ENT || B == 64) ? 64 : a.rowq;
  const int qtiles = rowq / 64;           // 64-query tiles per row
  const int nunits = nr * G * qtiles;     // (row, head, query tile), row-major
  const float sc = a.sm_scale * kLog2e;

  uint4 qreg[QITEMS], oreg[QITEMS];
  float lreg = 0.f, dreg = 0.f, zreg = 0.f;
  // unit u -> query head and first query position
  auto unit_of = [&](int uu, int& h, int64_t& t0) {
    const int qq = uu % qtiles;
    const int rest = uu / qtiles;
    h = g * G + rest % G;
    const int row = ENT ? (a.live ? static_cast<int>(erows[rest / G]) : j + rest / G) : rows[rest / G];
    t0 = static_cast<int64_t>(row) * rowq + qq * 64;
  };
  auto load_unit = [&](int uu) {
    int h;
    int64_t t0;
    unit_of(uu, h, t0);
    const int ri = uu / qtiles / G;  // slot of the unit's row
    (void)ri;
    const auto rq = make_rsrc(static_cast<const uint16_t*>(a.Q) + b * a.qs.b + h * a.qs.h,
                              head_bytes(a.n, a.qs.t, D, 2));
    const auto rdo = make_rsrc(static_cast<const uint16_t*>(a.dO) + b * a.os.b + h * a.os.h,
                               head_bytes(a.n, a.os.t, D, 2));
#pragma unroll
    for (int it = 0; it < QITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (QTOT % NT == 0 || flat < QTOT) {
        const uint32_t t = static_cast<uint32_t>(t0 + r);
        qreg[it] = buf_load16(rq, t * static_cast<uint32_t>(a.qs.t * 2) + c * 16);
        oreg[it] = buf_load16(rdo, t * static_cast<uint32_t>(a.os.t * 2) + c * 16);
      }
    }
    if (tid < 64) {
      const int64_t t = t0 + tid;
      const int64_t hrow = (static_cast<int64_t>(b) * a.hq + h) * a.n;
      if constexpr (ENT) {
        lreg = t < a.n ? a.tau[hrow + t] : INFINITY;  // past the end: no support
        zreg = t < a.n ? a.zbuf[hrow + t] : 0.f;
      } else {
        const float L = t < a.n ? a.lse[hrow + t] : -INFINITY;
        float bias = 0.f;
        bool on = L > -INFINITY;
        if (a.tok) {
          // the query's own choice of block j and its bias
          const int64_t le = (static_cast<int64_t>(pair) * a.nrow + rows[ri]) * a.k_max + rent[ri];
          on = on && ((a.tbits[le] >> tid) & 1ull);
          if (a.tbias) {
            bias = a.tbias[le * 64 + tid];
            on = on && bias > -INFINITY;
          }
        }
        lreg = on ? (L - bias) * kLog2e : INFINITY;
      }
      dreg = t < a.n ? a.delta[hrow + t] : 0.f;
    }
  };
  auto store_unit = [&](int buf) {
#pragma unroll
    for (int it = 0; it < QITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (QTOT % NT == 0 || flat < QTOT) {
        *reinterpret_cast<uint4*>(&lds.q[buf][Swz<D>::at(r, c)]) = qreg[it];
        *reinterpret_cast<uint4*>(&lds.o[buf][Swz<D>::at(r, c)]) = oreg[it];
      }
    }
    if (tid < 64) {
      lds.lse2[buf][tid] = lreg;
      lds.dl[buf][tid] = dreg;
      if constexpr (ENT) {
        lds_iz[buf][tid] = zreg > 0.f ? 1.f / zreg : 0.f;
        lds_zf[buf][tid] = zreg > 0.f ? __builtin_amdgcn_exp2f((a.alpha - 2.f) * __log2f(zreg)) : 0.f;
      }
    }
  };

  int buf = 0;
  if (nunits > 0) {
    load_unit(0);
    store_unit(0);
  }
  __syncthreads();
  for (int uu = 0; uu < nunits; ++uu) {
    const bool more = uu + 1 < nunits;
    if (more) load_unit(uu + 1);
    int h;
    int64_t t0;
    unit_of(uu, h, t0);
    (void)h;
    // nothing to add when every key of the wave follows every query of the tile
    if (key0 <= t0 + 63) {
      const uint16_t* qt_ = lds.q[buf];
      const uint16_t* ot_ = lds.o[buf];
      // S and dP tiles: lane l holds queries 16qt + 4(l/16) + e of key 16w + l%16
      f32x4 s[4], dp[4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        s[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
      const bool diag = key0 + 15 > t0;
      const int64_t rel0 = key0 + (lane & 15) - t0 - (lane >> 4) * 4;  // key - query at qt = e = 0
      bool live = true;
      if constexpr (ENT) {
        // S first: keys outside every support of the tile's queries have no
        // dP, dV or dK work (zero blocks skipped)
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int qt = 0; qt < 4; ++qt) s[qt] = mfma16(row_frag<D>(qt_, qt, ks, lane), kf[ks], s[qt]);
        const float a1s_ = (a.alpha - 1.f) * a.sm_scale;
        bool any = false;
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const float4 L = *reinterpret_cast<const float4*>(&lds.lse2[buf][qt * 16 + (lane >> 4) * 4]);
          const float Lv[4] = {L.x, L.y, L.z, L.w};
#pragma unroll
          for (int e = 0; e < 4; ++e)
            any |= fmaf(s[qt][e], a1s_, -Lv[e]) > 0.f && !(diag && rel0 - qt * 16 - e > 0);
        }
        live = __ballot(any) != 0;
        if (live)
#pragma unroll
          for (int ks = 0; ks < KS; ++ks)
#pragma unroll
            for (int qt = 0; qt < 4; ++qt) dp[qt] = mfma16(row_frag<D>(ot_, qt, ks, lane), vf[ks], dp[qt]);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks)
#pragma unroll
          for (int qt = 0; qt < 4; ++qt) {
            s[qt] = mfma16(row_frag<D>(qt_, qt, ks, lane), kf[ks], s[qt]);
            dp[qt] = mfma16(row_frag<D>(ot_, qt, ks, lane), vf[ks], dp[qt]);
          }
      }
      const float tbs = !ENT && a.wsel ? rbias[uu / qtiles / G] * sc : 0.f;  // the row's prior bias
      const float a1s = (a.alpha - 1.f) * a.sm_scale;
      const float ib = 1.f / (a.alpha - 1.f), ig = (2.f - a.alpha) / (a.alpha - 1.f);
      f32x4 p[4], ds[4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const int qo = qt * 16 + (lane >> 4) * 4;
        const float4 L = *reinterpret_cast<const float4*>(&lds.lse2[buf][qo]);
        const float4 Dl = *reinterpret_cast<const float4*>(&lds.dl[buf][qo]);
        const float Lv[4] = {L.x, L.y, L.z, L.w};
        const float Dv[4] = {Dl.x, Dl.y, Dl.z, Dl.w};
        float Iz[4] = {0.f, 0.f, 0.f, 0.f}, Zf[4] = {0.f, 0.f, 0.f, 0.f};
        if constexpr (ENT) {
          const float4 iz = *reinterpret_cast<const float4*>(&lds_iz[buf][qo]);
          const float4 zf = *reinterpret_cast<const float4*>(&lds_zf[buf][qo]);
          Iz[0] = iz.x; Iz[1] = iz.y; Iz[2] = iz.z; Iz[3] = iz.w;
          Zf[0] = zf.x; Zf[1] = zf.y; Zf[2] = zf.z; Zf[3] = zf.w;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bool masked = diag && rel0 - qt * 16 - e > 0;  // key after query
          if constexpr (ENT) {
            // entmax weights from tau (x units): p = t^(1/(alpha-1)) / Z and
            // dz = Z^(alpha-2) t^((2-alpha)/(alpha-1)) (dP - <g, dP> / sum g)
            const float tt = fmaf(s[qt][e], a1s, -Lv[e]);
            float pb = 0.f, pg = 0.f;
            if (tt > 0.f && !masked) ent_pow(tt, a.alpha, ib, ig, pb, pg);
            p[qt][e] = pb * Iz[e];
            ds[qt][e] = Zf[e] * pg * (dp[qt][e] - Dv[e]);
          } else {
            float pv = __builtin_amdgcn_exp2f(fmaf(s[qt][e], sc, tbs - Lv[e]));
            if (masked) pv = 0.f;
            p[qt][e] = pv;
            ds[qt][e] = pv * (dp[qt][e] - Dv[e]);
          }
        }
      }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        if (!live) break;
        const uint4 pf = pack_frag(p[2 * kk], p[2 * kk + 1]);
        const uint4 sf = pack_frag(ds[2 * kk], ds[2 * kk + 1]);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          dv[dt] = mfma16(tr_frag<D>(ot_, kk, dt, lane), pf, dv[dt]);
          dk[dt] = mfma16(tr_frag<D>(qt_, kk, dt, lane), sf, dk[dt]);
        }
      }
    }
    if (more) store_unit(buf ^ 1);
    __syncthreads();
    buf ^= 1;
  }

  // lane l holds dK^T / dV^T rows d = 16dt + 4(l/16) + e of key 16w + l%16
  const int64_t key = key0 + (lane & 15);
  if (slot >= 0) {
    float* pk = a.part + static_cast<int64_t>(slot) * 2 * B * D + (w * 16 + (lane & 15)) * D;
    float* pv = pk + B * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d0 = dt * 16 + (lane >> 4) * 4;
      *reinterpret_cast<float4*>(pk + d0) = make_float4(dk[dt][0], dk[dt][1], dk[dt][2], dk[dt][3]);
      *reinterpret_cast<float4*>(pv + d0) = make_float4(dv[dt][0], dv[dt][1], dv[dt][2], dv[dt][3]);
    }
    return;
  }
  if (key >= a.n) return;
  const int64_t ok = b * a.ks.b + g * a.ks.h + key * a.ks.t;
  const int64_t ov = b * a.vs.b + g * a.vs.h + key * a.vs.t;
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int d0 = dt * 16 + (lane >> 4) * 4;
    const f32x4 k4 = dk[dt] * a.sm_scale;
    const f32x4 v4 = dv[dt];
    if (a.g_f32) {
      *reinterpret_cast<float4*>(static_cast<float*>(a.dK) + ok + d0) = make_float4(k4[0], k4[1], k4[2], k4[3]);
      *reinterpret_cast<float4*>(static_cast<float*>(a.dV) + ov + d0) = make_float4(v4[0], v4[1], v4[2], v4[3]);
    } else {
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dK) + ok + d0) =
          make_uint2(pack_bf16x2(k4[0], k4[1]), pack_bf16x2(k4[2], k4[3]));
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.dV) + ov + d0) =
          make_uint2(pack_bf16x2(v4[0], v4[1]), pack_bf16x2(v4[2], v4[3]));
    }
  }
}

// Sum of the chunk partials of a split block, in chunk order; kRedSlices
// workgroups share each block.
constexpr int kRedSlices = 16;
__global__ __launch_bounds__(256) void bwd_reduce(BwdArgs a) {
  const int item = blockIdx.x / kRedSlices, slice = blockIdx.x % kRedSlices;
  if (item >= a.counters[1]) return;
  const int4 r = a.red[item];
  const int pair = r.x, j = r.y, s0 = r.z, ns = r.w;
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int64_t bd = static_cast<int64_t>(a.B) * a.d;
  const int64_t per = 2 * bd / kRedSlices;  // a multiple of 4 (B * d >= 4096)
  for (int64_t e = slice * per + threadIdx.x * 4; e < (slice + 1) * per; e += 256 * 4) {
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int s = 0; s < ns; ++s) {
      const float4 v = *reinterpret_cast<const float4*>(a.part + (s0 + s) * 2 * bd + e);
      acc.x += v.x;
      acc.y += v.y;
      acc.z += v.z;
      acc.w += v.w;
    }
    const bool isv = e >= bd;
    const int64_t rem = isv ? e - bd : e;
    const int64_t key = static_cast<int64_t>(j) * a.B + rem / a.d;
    const int c = static_cast<int>(rem % a.d);
    if (key >= a.n) continue;
    if (!isv) {
      acc.x *= a.sm_scale;
      acc.y *= a.sm_scale;
      acc.z *= a.sm_scale;
      acc.w *= a.sm_scale;
    }
    const int64_t off = isv ? b * a.vs.b + g * a.vs.h + key * a.vs.t + c
                            : b * a.ks.b + g * a.ks.h + key * a.ks.t + c;
    void* dst = isv ? a.dV : a.dK;
    if (a.g_f32)
      *reinterpret_cast<float4*>(static_cast<float*>(dst) + off) = acc;
    else
      *reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + off) =
          make_uint2(pack_bf16x2(acc.x, acc.y), pack_bf16x2(acc.z, acc.w));
  }
}

// dL/dw of every list entry: sigma / w times the units' sums of dS.
__global__ __launch_bounds__(64) void bwd_dwsel(BwdArgs a) {
  const int64_t rowid = blockIdx.x;
  const int c = a.cnt[rowid];
  for (int e = threadIdx.x; e < a.k_max; e += 64) {
    float acc = 0.f;
    for (int u = 0; u < a.units; ++u) acc += a.dbpart[(rowid * a.units + u) * a.k_max + e];
    const float wv = a.wsel[rowid * a.k_max + e];
    a.dwsel[rowid * a.k_max + e] = e < c && wv > 0.f ? a.sigma / wv * acc : 0.f;
  }
}

// Token tiles: dL/dw of every token's list entry, sigma / w times the sum of
// dS over the entry's keys and the group's heads (the parts of the query-side
// workgroups holding those heads, in order).  Four threads per token, each
// taking every fourth entry.
constexpr int kDwTok = 4;
__global__ __launch_bounds__(64 * kDwTok) void bwd_dwsel_tok(BwdArgs a) {
  const int64_t rowid = blockIdx.x;  // (pair, tile)
  const int64_t pair = rowid / a.nrow;
  const int q = threadIdx.x & 63, s0 = threadIdx.x >> 6;
  const int64_t t = (rowid % a.nrow) * 64 + q;
  if (t >= a.n) return;
  const int G = a.hq / a.hkv;
  constexpr int QPW = 16 * kBwdQT;
  const int qsq = q / QPW;
  const int np = dq_last_wg(qsq, G, kBwdNW) - dq_first_wg(qsq, G, kBwdNW) + 1;  // parts, in order
  int c = a.cnt[rowid];
  c = c < 0 ? 0 : (c > a.k_max ? a.k_max : c);
  const int32_t* list = a.idx + rowid * a.k_max;
  const int64_t prow = (pair * a.n + t) * a.pwidth;
  int pc = a.pcnt[pair * a.n + t];
  pc = pc < 0 ? 0 : (pc > a.pwidth ? a.pwidth : pc);
  for (int s = s0; s < a.pwidth; s += kDwTok) {
    float out = 0.f;
    const int j = s < pc ? a.pidx[prow + s] : -1;
    const float wv = s < pc ? a.pw[prow + s] : 0.f;
    // a block after the token attends nothing; w <= 0 drops the block
    if (j >= 0 && j < a.nblk && wv > 0.f && static_cast<int64_t>(j) * a.B <= t) {
      int lo = 0, hi = c;  // the tile's list is ascending
      while (lo < hi) {
        const int mid = (lo + hi) >> 1;
        if (list[mid] < j)
          lo = mid + 1;
        else
          hi = mid;
      }
      if (lo < c && list[lo] == j) {
        float acc = 0.f;
        for (int p = 0; p < np; ++p) acc += a.dbtok[((rowid * a.k_max + lo) * a.nparts + p) * 64 + q];
        out = a.sigma / wv * acc;
      }
    }
    a.dwsel[prow + s] = out;
  }
}

template <int D>
hipError_t bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  const int npair = a.batch * a.hkv;
  constexpr int QT = kBwdQT, NW = kBwdNW;
  const int G = a.hq / a.hkv;
  const int units = G * (a.rowq / (16 * QT));
  const int wpb = (units + NW - 1) / NW;
  const dim3 gq(static_cast<unsigned>(npair) * a.nrow * wpb);
  if (a.ent) {
    // token-level entmax attention: B = 64 rows, dense causal
    hipLaunchKernelGGL((bwd_dq<D, QT, NW, true, false>), gq, dim3(NW * 64), 0, stream, a, wpb);
    hipLaunchKernelGGL((bwd_dkv<D, 4, true>), dim3(static_cast<unsigned>(npair) * a.nblk),
                       dim3(256), 0, stream, a);
    return hipGetLastError();
  }
  if (a.tok)
    hipLaunchKernelGGL((bwd_dq<D, QT, NW, false, true>), gq, dim3(NW * 64), 0, stream, a, wpb);
  else
    hipLaunchKernelGGL((bwd_dq<D, QT, NW, false, false>), gq, dim3(NW * 64), 0, stream, a, wpb);
  if (a.B == 64)
    hipLaunchKernelGGL((bwd_dkv<D, 4, false>), dim3(a.max_items), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((bwd_dkv<D, 8, false>), dim3(a.max_items), dim3(512), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

int attend_bwd_units(int group, int B) { return group * (B / (16 * kBwdQT)); }
int attend_bwd_max_prior_width() { return kMaxPriorEntries; }
int attend_bwd_tok_parts(int group) {
  int m = 1;
  for (int qs = 0; qs < 64 / (16 * kBwdQT); ++qs)
    m = std::max(m, dq_last_wg(qs, group, kBwdNW) - dq_first_wg(qs, group, kBwdNW) + 1);
  return m;
}

hipError_t launch_attend_backward(const BwdArgs& a, hipStream_t stream) {
  const unsigned npair = static_cast<unsigned>(a.batch) * a.hkv;
  if (a.ent) return a.d == 64 ? bwd_bf16<64>(a, stream) : bwd_bf16<128>(a, stream);
  hipLaunchKernelGGL(bwd_mark, dim3(npair * a.nwords), dim3(256), a.nblk * sizeof(uint32_t), stream, a);
  hipLaunchKernelGGL(bwd_plan, dim3(1), dim3(kPlanThreads), 0, stream, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (!a.bf16) return hipErrorInvalidValue;  // fp32 path not built
  e = a.d == 64 ? bwd_bf16<64>(a, stream) : bwd_bf16<128>(a, stream);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_reduce, dim3(a.max_red * kRedSlices), dim3(256), 0, stream, a);
  if (a.dwsel && a.tok)
    hipLaunchKernelGGL(bwd_dwsel_tok, dim3(static_cast<unsigned>(npair) * a.nrow), dim3(64 * kDwTok), 0,
                       stream, a);
  else if (a.dwsel)
    hipLaunchKernelGGL(bwd_dwsel, dim3(static_cast<unsigned>(npair) * a.nrow), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bsa
