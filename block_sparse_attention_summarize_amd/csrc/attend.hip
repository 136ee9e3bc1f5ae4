// Stage 2: exact softmax attention restricted to the tokens of the selected
// blocks ("DashAttention", Declaração do Problema: fine-grained softmax over
// the selected tokens; Estágio 2 with the routing bias switched off).
//
//   attend_prefill_bf16   gathered-KV causal prefill on bf16 MFMA.
//                         A workgroup (4 wavefronts) owns one (batch, KV head,
//                         query block) and up to 4 "units" of 32 queries x one
//                         query head of the GQA group, so every K/V tile it
//                         stages in LDS serves several heads.  S^T = K Q^T
//                         and O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16
//                         with fp32 accumulation; the online softmax is fp32.
//                         V stays row-major in LDS and its transposed MFMA
//                         operand comes from ds_read_b64_tr_b16.
//   attend_prefill_f32    fp32 inputs: one query per lane, VALU dot products
//                         (fp32 matrix rate is not the bound at these sizes).
// With per-token selections (TOK) a row is a tile of 64 queries whose list
// holds the blocks any of its tokens selected, each with a 64-bit word of the
// tokens that did; a query's scores on a block its token did not select are
// masked to -inf ("DashAttention", Estágio 2, Implementação: active blocks
// from a bit-packed mask).
// With a prior (BIAS) the scores of every key of a listed block gain the
// routing bias sigma * ln w of that block (block rows) or of that block for
// that query (token tiles), the prior-induced softmax of Estágio 2.
// Single-token decode lives in decode.hip.
#include "common.hpp"
#include "kernels.hpp"
#include "walk.hpp"

namespace bsa {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short v4i16 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma16(const uint4& a, const uint4& b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
}

// Double-buffered K and V tiles, both row-major (64 keys x D).  Row padding
// spreads each read instruction over all 64 banks: K fragments read 16 B from
// 16 rows (a 16-B pad staggers rows by 4 banks); the transposing V reads take
// 32 B from each of 8 rows per half-wave (a 32-B pad staggers rows by 8).
template <int D>
struct PrefillLds {
  static constexpr int KST = D + 8;   // K row stride (bf16 elements)
  static constexpr int VST = D + 16;  // V row stride
  alignas(16) uint16_t k[2][64 * KST];
  alignas(16) uint16_t v[2][64 * VST];
};

constexpr float kRescale = 8.f;  // lazy rescale threshold, log2 units

// Max over the four lanes l, l^16, l^32, l^48 (VALU lane swaps, no LDS).
__device__ __forceinline__ float xmax16(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max3f(float a, float b, float c) {
  return __builtin_fmaxf(a, __builtin_fmaxf(b, c));
}
constexpr int kMaxTiles = 1024;  // tile-list chunk staged in LDS
constexpr int kMaxTilesTok = 512;  // the same with a 64-bit token word per tile

// QT query tiles of 16 per wavefront, NW wavefronts per workgroup.  A "unit"
// is one query head x 16*QT queries of the query block; the workgroup's
// wavefronts take NW consecutive units of the same (batch, KV head, block),
// so they share every K/V tile staged in LDS.
template <int D, int QT, int NW, bool OUT_F32, bool TOK, bool BIAS>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attend_prefill_bf16(AttendArgs a, int wpb) {
  constexpr int NT = NW * 64;
  constexpr int QPW = 16 * QT;  // queries per wave
  constexpr int KS = D / 32;    // k-steps of S^T = K Q^T
  constexpr int DT = D / 16;    // 16-row d tiles of O^T
  constexpr int CPR = D / 8;    // 16-byte chunks per row
  constexpr int KTOT = 64 * CPR;                // 16-byte chunks per K (or V) tile
  constexpr int KITEMS = (KTOT + NT - 1) / NT;  // per thread
  constexpr int MAXT = TOK ? kMaxTilesTok : kMaxTiles;
  __shared__ PrefillLds<D> lds;
  __shared__ int lds_tiles[MAXT];
  __shared__ uint64_t lds_tbits[TOK ? MAXT : 1];
  // BIAS: the tile's bias in score units (block rows) or its list entry (token tiles)
  __shared__ float lds_tbias[BIAS && !TOK ? MAXT : 1];
  __shared__ int lds_tent[BIAS && TOK ? MAXT : 1];
  __shared__ int lds_ntiles;
  using L = PrefillLds<D>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int G = a.hq / a.hkv;
  const int nsub = a.B / 64;
  const int qb = TOK ? 64 : a.B;  // queries per row
  const int qsub = qb / QPW;      // query sub-blocks per row
  const int units = G * qsub;
  int pair, i, sub;
  map_wg(blockIdx.x, a.batch * a.hkv, a.nrow, wpb, pair, i, sub);
  const int b = pair / a.hkv, g = pair % a.hkv;

  const int u = sub * NW + w;
  const bool active = u < units;
  const int hh = active ? u % G : 0;
  const int qs = active ? u / G : 0;
  const int h = g * G + hh;
  const int qpos0 = i * qb + qs * QPW;
  int qs_max = 0;
  for (int uu = sub * NW; uu < sub * NW + NW && uu < units; ++uu) qs_max = max(qs_max, uu / G);
  int64_t qmax = static_cast<int64_t>(i) * qb + qs_max * QPW + QPW - 1;
  if (qmax > a.q_len - 1) qmax = a.q_len - 1;

  const int64_t rowid = static_cast<int64_t>(pair) * a.nrow + i;
  int n = a.cnt[rowid];
  n = n < 0 ? 0 : (n > a.k_max ? a.k_max : n);
  TileWalk walk{a.idx + rowid * a.k_max, n, nsub, a.B, a.nblk, a.kv_len, qmax};
  // the first 64 list entries are read before the count arrives, so the two
  // loads overlap instead of following each other
  int jpre = -1;
  if (w == 0 && lane < a.k_max * nsub) jpre = walk.list[lane / nsub];

  const auto rk = make_rsrc(static_cast<const uint16_t*>(a.K) + b * a.ks.b + g * a.ks.h,
                            head_bytes(a.kv_len, a.ks.t, D, 2));
  const auto rv = make_rsrc(static_cast<const uint16_t*>(a.V) + b * a.vs.b + g * a.vs.h,
                            head_bytes(a.kv_len, a.vs.t, D, 2));
  const uint32_t kst = static_cast<uint32_t>(a.ks.t * 2), vst = static_cast<uint32_t>(a.vs.t * 2);

  // Q fragments (B operand of S^T = K Q^T): lane l holds query 16qt + l%16,
  // d = 32ks + 8(l/16) .. +7.  Rows past q_len read as zero.
  uint4 qf[QT][KS];
  {
    const auto rq = make_rsrc(static_cast<const uint16_t*>(a.Q) + b * a.qs.b + h * a.qs.h,
                              active ? head_bytes(a.q_len, a.qs.t, D, 2) : 0u);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const uint32_t t = static_cast<uint32_t>(qpos0 + qt * 16 + (lane & 15));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[qt][ks] = buf_load16(rq, t * static_cast<uint32_t>(a.qs.t * 2) + (ks * 32 + (lane >> 4) * 8) * 2);
    }
  }

  f32x4 o[DT][QT];
  f32x4 lsum[QT];
  float m[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    lsum[qt] = f32x4{0.f, 0.f, 0.f, 0.f};
    m[qt] = -INFINITY;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const float sc = a.sm_scale * kLog2e;
  const float inv_sm = 1.f / a.sm_scale;
  const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
  // token tiles with a prior: this lane's query columns' bias for the current
  // and the next tile (score units)
  float bcur[QT], bnxt[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) bcur[qt] = bnxt[qt] = 0.f;
  auto load_bias = [&](int tt, float (&dst)[QT]) {
    const float* bp = a.tbias + (rowid * a.k_max + lds_tent[tt]) * 64 + qs * QPW + (lane & 15);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) dst[qt] = bp[qt * 16] * inv_sm;
  };

  uint4 kreg[KITEMS];
  uint4 vreg[KITEMS];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (KTOT % NT == 0 || flat < KTOT)
        kreg[it] = buf_load16(rk, static_cast<uint32_t>(k0 + r) * kst + c * 16);
    }
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (KTOT % NT == 0 || flat < KTOT)
        vreg[it] = buf_load16(rv, static_cast<uint32_t>(k0 + r) * vst + c * 16);
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (KTOT % NT == 0 || flat < KTOT)
        *reinterpret_cast<uint4*>(&lds.k[buf][r * L::KST + c * 8]) = kreg[it];
    }
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (KTOT % NT == 0 || flat < KTOT)
        *reinterpret_cast<uint4*>(&lds.v[buf][r * L::VST + c * 8]) = vreg[it];
    }
  };

  // The workgroup's tiles (valid, not entirely in its future) are compacted
  // into LDS by wave 0, kMaxTiles raw entries at a time, so the main loop
  // reads its next key offset from LDS instead of a dependent global load.
  const int nraw = n * nsub;
  for (int base = 0; base < nraw; base += MAXT) {
    if (w == 0) {
      int c = 0;
      for (int r = 0; r < MAXT && base + r < nraw; r += 64) {
        const int T = base + r + lane;
        int64_t k0 = T >= nraw ? -1 : (T < 64 ? walk.key0_of(jpre, T) : walk.key0(T));
        float tb = 0.f;
        if constexpr (BIAS && !TOK) {
          // routing weight of the tile's block: w <= 0 drops it, else ln-bias
          if (k0 >= 0) {
            const float wv = a.wsel[rowid * a.k_max + T / nsub];
            if (wv > 0.f)
              tb = a.sigma * __logf(wv) * inv_sm;
            else
              k0 = -1;
          }
        }
        const uint64_t mk = __ballot(k0 >= 0);
        if (k0 >= 0) {
          const int pos = c + lanes_below(mk);
          lds_tiles[pos] = static_cast<int>(k0);
          if constexpr (TOK) lds_tbits[pos] = a.bits[rowid * a.k_max + T / nsub];
          if constexpr (BIAS && !TOK) lds_tbias[pos] = tb;
          if constexpr (BIAS && TOK) lds_tent[pos] = T / nsub;
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
      if constexpr (BIAS && TOK) load_bias(0, bcur);
      store_tile(0);
    }
    // Drain every outstanding vector load (the Q fragments) here, so that the
    // loop's only pending loads are the next tile's prefetch and the MFMAs on
    // the current tile never wait for it.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int k0 = lds_tiles[t];
      const bool more = t + 1 < ntiles;
      if (more) {
        load_tile(lds_tiles[t + 1]);
        if constexpr (BIAS && TOK) load_bias(t + 1, bnxt);
      }
      // bias of the tile for each query column (score units)
      float tb[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        if constexpr (BIAS && TOK)
          tb[qt] = bcur[qt];
        else if constexpr (BIAS)
          tb[qt] = lds_tbias[t];
        else
          tb[qt] = 0.f;
      }
      // TOK: bit 16qt + c says whether query qpos0 + 16qt + c selected the
      // tile's block; a wave none of whose queries did skips the tile
      uint64_t qbits = ~0ull;
      if constexpr (TOK) qbits = lds_tbits[t] >> (qs * QPW);

      if (active && (!TOK || (qbits & (QPW == 64 ? ~0ull : (1ull << QPW) - 1)) != 0)) {
        // S^T tiles: lane l holds keys 16kt + 4(l/16) + j of query column 16qt + l%16.
        // The two MFMA phases run at raised wave priority, so the SIMD's other
        // wavefront, in its softmax, yields the matrix unit to them (measured
        // ~2 % faster at the 32k GQA workload).
        __builtin_amdgcn_s_setprio(1);
        f32x4 s[4][QT];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) s[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            const uint4 kf = *reinterpret_cast<const uint4*>(
                &lds.k[buf][(kt * 16 + (lane & 15)) * L::KST + ks * 32 + (lane >> 4) * 8]);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) s[kt][qt] = mfma16(kf, qf[qt][ks], s[kt][qt]);
          }
        }
        if constexpr (TOK) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
            if (!((qbits >> (qt * 16 + (lane & 15))) & 1ull))
#pragma unroll
              for (int kt = 0; kt < 4; ++kt) s[kt][qt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        }
        // causal mask, only on tiles that reach past the wave's first query
        if (k0 + 63 > qpos0) {
          const int rel0 = k0 - qpos0 + (lane >> 4) * 4 - (lane & 15);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt)
#pragma unroll
            for (int kt = 0; kt < 4; ++kt)
#pragma unroll
              for (int j = 0; j < 4; ++j)
                if (rel0 + kt * 16 + j - qt * 16 > 0) s[kt][qt][j] = -INFINITY;
        }
        __builtin_amdgcn_s_setprio(0);
        // running max per query; the accumulators are rescaled only when it
        // grows by more than 2^kRescale (p stays <= 2^kRescale, exact after
        // normalising)
        float mx[QT];
        bool grow = false;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          // 16 values in 8 three-input maxes
          const float t0 = max3f(s[0][qt][0], s[0][qt][1], s[0][qt][2]);
          const float t1 = max3f(s[0][qt][3], s[1][qt][0], s[1][qt][1]);
          const float t2 = max3f(s[1][qt][2], s[1][qt][3], s[2][qt][0]);
          const float t3 = max3f(s[2][qt][1], s[2][qt][2], s[2][qt][3]);
          const float t4 = max3f(s[3][qt][0], s[3][qt][1], s[3][qt][2]);
          const float t5 = max3f(t0, t1, t2);
          const float t6 = max3f(t3, t4, s[3][qt][3]);
          float v = fmaxf(t5, t6);
          v = xmax16(v);
          mx[qt] = BIAS ? (v + tb[qt]) * sc : v * sc;
          grow |= mx[qt] > m[qt] + kRescale;
        }
        if (__ballot(grow) != 0) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            const float mn = fmaxf(m[qt], mx[qt]);
            const float f = mn == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m[qt] - mn);
            m[qt] = mn;
            lsum[qt] *= f;
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) o[dt][qt] *= f;
          }
        }
        uint4 pf[QT][2];
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          float nb = m[qt] == -INFINITY ? 0.f : -m[qt];
          if constexpr (BIAS) nb = fmaf(tb[qt], sc, nb);
          float p[4][4];
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int j = 0; j < 4; ++j) p[kt][j] = __builtin_amdgcn_exp2f(fmaf(s[kt][qt][j], sc, nb));
#pragma unroll
          for (int kk = 0; kk < 2; ++kk) {
            pf[qt][kk].x = pack_bf16x2(p[2 * kk][0], p[2 * kk][1]);
            pf[qt][kk].y = pack_bf16x2(p[2 * kk][2], p[2 * kk][3]);
            pf[qt][kk].z = pack_bf16x2(p[2 * kk + 1][0], p[2 * kk + 1][1]);
            pf[qt][kk].w = pack_bf16x2(p[2 * kk + 1][2], p[2 * kk + 1][3]);
          }
        }
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) lsum[qt] = mfma16(ones, pf[qt][kk], lsum[qt]);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) {
            // V^T fragment by two transposing reads of the row-major V tile:
            // keys 32kk + 4G + e and 32kk + 16 + 4G + e (G = lane/16) for
            // column 16dt + lane%16, the key order of the P fragment
            const int s16 = lane & 15;
            const uint16_t* vp = &lds.v[buf][(kk * 32 + (lane >> 4) * 4 + (s16 >> 2)) * L::VST +
                                             dt * 16 + 4 * (s16 & 3)];
            typedef __attribute__((address_space(3))) v4i16 lds_v4;
            const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp));
            const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp + 16 * L::VST));
            const uint2 u0 = __builtin_bit_cast(uint2, r0), u1 = __builtin_bit_cast(uint2, r1);
            const uint4 vf = make_uint4(u0.x, u0.y, u1.x, u1.y);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) o[dt][qt] = mfma16(vf, pf[qt][kk], o[dt][qt]);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if (more) store_tile(buf ^ 1);
      if constexpr (BIAS && TOK) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) bcur[qt] = bnxt[qt];
      }
      __syncthreads();
      buf ^= 1;
    }
  }

  if (!active) return;
  uint8_t* Ob = static_cast<uint8_t*>(a.O);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    // every row of the ones-product holds the column sum of the bf16 weights
    const float lt = lsum[qt][0];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t t = qpos0 + qt * 16 + (lane & 15);
    if (t >= a.q_len) continue;
    // the normaliser in natural-log units (m and the scores are log2 units)
    if (a.lse && lane < 16)
      a.lse[(static_cast<int64_t>(b) * a.hq + h) * a.q_len + t] =
          lt > 0.f ? (m[qt] + __log2f(lt)) * kLn2 : -INFINITY;
    const int64_t off = b * a.os.b + h * a.os.h + t * a.os.t;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d0 = dt * 16 + (lane >> 4) * 4;
      const f32x4 v = o[dt][qt] * inv;
      if constexpr (OUT_F32) {
        *reinterpret_cast<float4*>(reinterpret_cast<float*>(Ob) + off + d0) =
            make_float4(v[0], v[1], v[2], v[3]);
      } else {
        uint2 pk;
        pk.x = pack_bf16x2(v[0], v[1]);
        pk.y = pack_bf16x2(v[2], v[3]);
        *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(Ob) + off + d0) = pk;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// fp32 prefill: one query per lane, 32-key tiles in LDS read by broadcast.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(64) void attend_prefill_f32(AttendArgs a) {
  constexpr int KT = 32;
  __shared__ float ks[KT][D];
  __shared__ float vs[KT][D];
  const int lane = threadIdx.x;
  const bool tok = a.bits != nullptr;  // rows are 64-query tiles
  const int nsub = tok ? 1 : a.B / 64;
  const int qb = tok ? 64 : a.B;
  // grid: (b, h, i, qs)
  int id = blockIdx.x;
  const int qs = id % nsub;
  id /= nsub;
  const int i = id % a.nrow;
  id /= a.nrow;
  const int h = id % a.hq;
  const int b = id / a.hq;
  const int G = a.hq / a.hkv;
  const int g = h / G;
  const int64_t qpos0 = static_cast<int64_t>(i) * qb + qs * 64;
  const int64_t t = qpos0 + lane;
  int64_t qmax = qpos0 + 63;
  if (qmax > a.q_len - 1) qmax = a.q_len - 1;
  const float* Qg = static_cast<const float*>(a.Q) + b * a.qs.b + h * a.qs.h;
  const float* Kg = static_cast<const float*>(a.K) + b * a.ks.b + g * a.ks.h;
  const float* Vg = static_cast<const float*>(a.V) + b * a.vs.b + g * a.vs.h;
  const float sc = a.sm_scale * kLog2e;
  float q[D], o[D];
#pragma unroll
  for (int c = 0; c < D; ++c) {
    q[c] = t < a.q_len ? Qg[t * a.qs.t + c] * sc : 0.f;
    o[c] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int64_t rowid = (static_cast<int64_t>(b) * a.hkv + g) * a.nrow + i;
  int n = a.cnt[rowid];
  n = n < 0 ? 0 : (n > a.k_max ? a.k_max : n);
  const int32_t* list = a.idx + rowid * a.k_max;
  for (int s = 0; s < n; ++s) {
    const int j = list[s];
    if (j < 0 || j >= a.nblk) continue;
    // this lane's token selected block j (always, for block rows)
    bool on = !tok || ((a.bits[rowid * a.k_max + s] >> lane) & 1ull);
    // prior: bias of the block for this query, log2 units (scores are too)
    float bias2 = 0.f;
    if (a.tbias) {
      bias2 = a.tbias[(rowid * a.k_max + s) * 64 + lane] * kLog2e;
    } else if (a.wsel) {
      const float wv = a.wsel[rowid * a.k_max + s];
      if (!(wv > 0.f)) continue;
      bias2 = a.sigma * __log2f(wv);
    }
    on = on && bias2 != -INFINITY;
    for (int64_t k0 = static_cast<int64_t>(j) * a.B; k0 < static_cast<int64_t>(j + 1) * a.B;
         k0 += KT) {
      if (k0 > qmax || k0 >= a.kv_len) break;
      __syncthreads();
      for (int e = lane; e < KT * D; e += 64) {
        const int r = e / D, c = e % D;
        const int64_t tt = k0 + r;
        ks[r][c] = tt < a.kv_len ? Kg[tt * a.ks.t + c] : 0.f;
        vs[r][c] = tt < a.kv_len ? Vg[tt * a.vs.t + c] : 0.f;
      }
      __syncthreads();
      float sv[KT];
      float mx = -INFINITY;
#pragma unroll
      for (int r = 0; r < KT; ++r) {
        float acc = 0.f;
#pragma unroll
        for (int c = 0; c < D; ++c) acc = fmaf(q[c], ks[r][c], acc);
        const int64_t key = k0 + r;
        sv[r] = (key > t || key >= a.kv_len || !on) ? -INFINITY : acc + bias2;
        mx = fmaxf(mx, sv[r]);
      }
      const float mnew = fmaxf(m, mx);
      const float base = mnew == -INFINITY ? 0.f : mnew;
      const float alpha = exp2f(m - base);
      m = mnew;
      l *= alpha;
#pragma unroll
      for (int c = 0; c < D; ++c) o[c] *= alpha;
#pragma unroll
      for (int r = 0; r < KT; ++r) {
        const float p = exp2f(sv[r] - base);
        l += p;
#pragma unroll
        for (int c = 0; c < D; ++c) o[c] = fmaf(p, vs[r][c], o[c]);
      }
    }
  }
  if (t >= a.q_len) return;
  if (a.lse)
    a.lse[(static_cast<int64_t>(b) * a.hq + h) * a.q_len + t] =
        l > 0.f ? (m + __log2f(l)) * kLn2 : -INFINITY;
  const float inv = l > 0.f ? 1.f / l : 0.f;
  float* Og = static_cast<float*>(a.O) + b * a.os.b + h * a.os.h + t * a.os.t;
#pragma unroll
  for (int c = 0; c < D; ++c) Og[c] = o[c] * inv;
}

template <int D, int QT, int NW, bool TOK, bool BIAS>
hipError_t prefill_bf16_launch(const AttendArgs& a, hipStream_t stream) {
  const int G = a.hq / a.hkv;
  const int units = G * ((TOK ? 64 : a.B) / (16 * QT));
  const int wpb = (units + NW - 1) / NW;
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * a.nrow * wpb;
  if (a.out_f32)
    hipLaunchKernelGGL((attend_prefill_bf16<D, QT, NW, true, TOK, BIAS>), dim3(grid),
                       dim3(NW * 64), 0, stream, a, wpb);
  else
    hipLaunchKernelGGL((attend_prefill_bf16<D, QT, NW, false, TOK, BIAS>), dim3(grid),
                       dim3(NW * 64), 0, stream, a, wpb);
  return hipGetLastError();
}

template <int D>
hipError_t prefill_bf16_dispatch(const AttendArgs& a, hipStream_t stream) {
  if (a.bits)
    return a.tbias ? prefill_bf16_launch<D, 2, 4, true, true>(a, stream)
                   : prefill_bf16_launch<D, 2, 4, true, false>(a, stream);
  return a.wsel ? prefill_bf16_launch<D, 2, 4, false, true>(a, stream)
                : prefill_bf16_launch<D, 2, 4, false, false>(a, stream);
}

}  // namespace

hipError_t launch_attend_prefill(const AttendArgs& a, hipStream_t stream) {
  if (a.bf16) return a.d == 64 ? prefill_bf16_dispatch<64>(a, stream) : prefill_bf16_dispatch<128>(a, stream);
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hq * a.nrow * (a.bits ? 1 : a.B / 64);
  if (a.d == 64)
    hipLaunchKernelGGL(attend_prefill_f32<64>, dim3(grid), dim3(64), 0, stream, a);
  else
    hipLaunchKernelGGL(attend_prefill_f32<128>, dim3(grid), dim3(64), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bsa
