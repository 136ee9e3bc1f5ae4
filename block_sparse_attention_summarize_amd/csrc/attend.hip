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
//   attend_prefill_pp     the same computation for plain block rows with many
//                         key tiles: eight wavefronts in two groups half a
//                         tile apart, alternating MFMA and softmax phases.
//   attend_prefill_f32    fp32 inputs: each query over D/16 lanes, VALU dot products
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
#include "lds_tiles.hpp"
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

// K and V tiles (64 keys x D, bf16) in NBUF rotating buffers, filled by
// direct-to-LDS loads.  Rows are unpadded; the 16-byte chunks of a row are
// XOR-swizzled so that the K fragment reads (16 rows x 16 bytes per half-wave)
// and the transposing V reads (8 rows x 32 bytes) hit every bank once.
template <int D, int NBUF = 3>
struct PpLds {
  static constexpr int NC = D / 8;     // 16-byte chunks per row
  static constexpr int RPL = 16 / NC;  // rows per 256-byte bank line
  __host__ __device__ static constexpr int kswz(int r) { return (r / RPL) & (NC - 1); }
  __host__ __device__ static constexpr int vswz(int r) { return ((r / RPL) & (NC / 2 - 1)) << 1; }
  alignas(16) uint16_t k[NBUF][64 * D];
  alignas(16) uint16_t v[NBUF][64 * D];
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
constexpr int kPingPongMinTiles = 32;  // list width (in 64-key tiles) from which the
                                       // ping-pong kernel serves plain block rows

// QT query tiles of 16 per wavefront, NW wavefronts per workgroup.  A "unit"
// is one query head x 16*QT queries of the query block; the workgroup's
// wavefronts take NW consecutive units of the same (batch, KV head, block),
// so they share every K/V tile staged in LDS.
template <int D, int QT, int NW, bool OUT_F32, bool TOK, bool BIAS>
__global__ __launch_bounds__(NW * 64, 8 / NW) void attend_prefill_bf16(AttendArgs a, int wpb) {
  constexpr int QPW = 16 * QT;  // queries per wave
  constexpr int KS = D / 32;    // k-steps of S^T = K Q^T
  constexpr int DT = D / 16;    // 16-row d tiles of O^T
  constexpr int NC = D / 8;     // 16-byte chunks per row
  constexpr int NI = 64 * NC / 64 / NW;  // 1 KB direct-to-LDS loads per wave per tensor
  static_assert(NI >= 1 && NI * NW * 64 == 64 * NC, "tile split over the wavefronts");
  constexpr int MAXT = TOK ? kMaxTilesTok : kMaxTiles;
  __shared__ PpLds<D, 2> lds;
  __shared__ int lds_tiles[MAXT];
  __shared__ uint64_t lds_tbits[TOK ? MAXT : 1];
  // BIAS: the tile's bias in score units (block rows) or its list entry (token tiles)
  __shared__ float lds_tbias[BIAS && !TOK ? MAXT : 1];
  __shared__ int lds_tent[BIAS && TOK ? MAXT : 1];
  __shared__ int lds_ntiles;
  using L = PpLds<D, 2>;

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

  const auto rk = make_desc(static_cast<const uint16_t*>(a.K) + b * a.ks.b + g * a.ks.h,
                            head_bytes(a.kv_len, a.ks.t, D, 2));
  const auto rv = make_desc(static_cast<const uint16_t*>(a.V) + b * a.vs.b + g * a.vs.h,
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

  // direct-to-LDS loads: wave instruction it fills bytes [1 KB (w NI + it),
  // +1 KB) of a tile; lane l's 16 bytes land at chunk q = 64 (w NI + it) + l,
  // i.e. row q / NC, physical chunk q % NC, which holds logical chunk p ^ swz(row)
  uint32_t koff[NI], voff[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int q = (w * NI + it) * 64 + lane;
    const int r = q / NC, p = q % NC;
    koff[it] = static_cast<uint32_t>(r) * kst + ((p ^ L::kswz(r)) * 16);
    voff[it] = static_cast<uint32_t>(r) * vst + ((p ^ L::vswz(r)) * 16);
  }
  auto load_tile = [&](int k0, int buf) {
    const uint32_t kb = static_cast<uint32_t>(k0) * kst, vb = static_cast<uint32_t>(k0) * vst;
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      lds_dma16(rk, &lds.k[buf][(w * NI + it) * 512], koff[it] + kb);
      lds_dma16(rv, &lds.v[buf][(w * NI + it) * 512], voff[it] + vb);
    }
  };
  // this lane's K fragment offset (elements) per k-step and V transposing-read
  // offset per d tile at rows 0-15 (the swizzles repeat every 16 rows)
  int kfo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int r = lane & 15;
    kfo[ks] = r * D + ((ks * 4 + (lane >> 4)) ^ L::kswz(r)) * 8;
  }
  int vfo[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int s16 = lane & 15;
    const int r = (lane >> 4) * 4 + (s16 >> 2);
    const int c = dt * 2 + ((s16 & 3) >> 1);
    vfo[dt] = r * D + (c ^ L::vswz(r)) * 8 + (s16 & 1) * 4;
  }

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
      load_tile(lds_tiles[0], 0);
      if constexpr (BIAS && TOK) load_bias(0, bcur);
    }
    // Drain every outstanding vector load (the Q fragments, tile 0) here, so
    // that the loop's only pending loads are the next tile's and the MFMAs on
    // the current tile never wait for them.
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0)
    __syncthreads();
    for (int t = 0; t < ntiles; ++t) {
      const int k0 = lds_tiles[t];
      const bool more = t + 1 < ntiles;
      // the other buffer's last reads (tile t - 1) ended at the barrier
      if (more) {
        load_tile(lds_tiles[t + 1], buf ^ 1);
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
            const uint4 kf = *reinterpret_cast<const uint4*>(&lds.k[buf][kfo[ks] + kt * 16 * D]);
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
            const uint16_t* vp = &lds.v[buf][vfo[dt] + kk * 32 * D];
            typedef __attribute__((address_space(3))) v4i16 lds_v4;
            const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp));
            const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp + 16 * D));
            const uint2 u0 = __builtin_bit_cast(uint2, r0), u1 = __builtin_bit_cast(uint2, r1);
            const uint4 vf = make_uint4(u0.x, u0.y, u1.x, u1.y);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) o[dt][qt] = mfma16(vf, pf[qt][kk], o[dt][qt]);
          }
        }
      }
      __builtin_amdgcn_s_setprio(0);
      if constexpr (BIAS && TOK) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) bcur[qt] = bnxt[qt];
      }
      __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): tile t + 1 is in LDS
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
// fp32 prefill: each query is spread over LPQ = D/16 lanes (16 dimensions
// each), 64 queries per group of LPQ wavefronts, and a workgroup holds
// NS = 16/LPQ such groups for the same 64 queries: the workgroup's tiles of 32
// keys are listed in LDS, group g takes tiles g, g + NS, ..., staging each (K
// and V, 16-byte loads by every thread of the group, rows past the sequence
// read as zero) into its two LDS buffers, the next tile's loads in flight
// while the current one is used.  q.k is summed over the query's lanes; each
// of them runs the same online softmax for its dimensions of o.  At the end
// the groups' (m, l, o) are merged through LDS.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(1024) void attend_prefill_f32(AttendArgs a) {
  constexpr int LPQ = D / 16;     // lanes per query
  constexpr int NTG = 64 * LPQ;   // threads of a group: 64 queries
  constexpr int NS = 16 / LPQ;    // groups (key splits)
  constexpr int KT = 32;          // keys per tile
  constexpr int F4 = KT * D / 4;  // 16-byte chunks per tile and tensor
  constexpr int PT = F4 / NTG;    // per thread
  static_assert(PT * NTG == F4 && (LPQ == 4 || LPQ == 8), "tile split over a group");
  constexpr int MAXT = 256;       // tile-list chunk staged in LDS
  // [group][buffer][K, V]; reused for the merge once every tile is done
  __shared__ float4 kv[NS][2][2][F4];
  static_assert(sizeof(kv) >= (NS * NTG * 16 + NS * 64 * 2) * sizeof(float), "merge area");
  __shared__ int tk0[MAXT];  // first key of the tile
  __shared__ int tent[MAXT];  // its list entry
  __shared__ int ntl;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int grp = tid / NTG;
  const int gt = tid % NTG;
  const int qi = gt / LPQ;  // query of the block
  const int ds = gt % LPQ;  // dimensions [16 ds, 16 ds + 16)
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
  const int64_t t = qpos0 + qi;
  int64_t qmax = qpos0 + 63;
  if (qmax > a.q_len - 1) qmax = a.q_len - 1;
  const float* Qg = static_cast<const float*>(a.Q) + b * a.qs.b + h * a.qs.h;
  const auto rk = make_rsrc(static_cast<const float*>(a.K) + b * a.ks.b + g * a.ks.h,
                            head_bytes(a.kv_len, a.ks.t, D, 4));
  const auto rv = make_rsrc(static_cast<const float*>(a.V) + b * a.vs.b + g * a.vs.h,
                            head_bytes(a.kv_len, a.vs.t, D, 4));
  const uint32_t kst = static_cast<uint32_t>(a.ks.t * 4), vst = static_cast<uint32_t>(a.vs.t * 4);
  const float sc = a.sm_scale * kLog2e;
  float q[16], o[16];
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4) {
    const float4 v = t < a.q_len ? *reinterpret_cast<const float4*>(Qg + t * a.qs.t + ds * 16 + c4 * 4)
                                 : make_float4(0.f, 0.f, 0.f, 0.f);
    q[c4 * 4 + 0] = v.x * sc;
    q[c4 * 4 + 1] = v.y * sc;
    q[c4 * 4 + 2] = v.z * sc;
    q[c4 * 4 + 3] = v.w * sc;
  }
#pragma unroll
  for (int c = 0; c < 16; ++c) o[c] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int64_t rowid = (static_cast<int64_t>(b) * a.hkv + g) * a.nrow + i;
  int n = a.cnt[rowid];
  n = n < 0 ? 0 : (n > a.k_max ? a.k_max : n);
  const int32_t* list = a.idx + rowid * a.k_max;
  const int tpb = a.B / KT;  // tiles per block

  float4 kr[PT], vr[PT];
  auto load_tile = [&](int k0) {
#pragma unroll
    for (int it = 0; it < PT; ++it) {
      const int f = gt + NTG * it;
      const uint32_t r = static_cast<uint32_t>(k0 + f / (D / 4)), c = f % (D / 4);
      kr[it] = __builtin_bit_cast(float4, buf_load16(rk, r * kst + c * 16));
      vr[it] = __builtin_bit_cast(float4, buf_load16(rv, r * vst + c * 16));
    }
  };
  auto store_tile = [&](int buf) {
#pragma unroll
    for (int it = 0; it < PT; ++it) {
      kv[grp][buf][0][gt + NTG * it] = kr[it];
      kv[grp][buf][1][gt + NTG * it] = vr[it];
    }
  };
  // sum over the query's LPQ consecutive lanes (every one of them gets it)
  auto qsum = [&](float v) {
    v += dppf<0xB1>(v);  // lane ^ 1
    v += dppf<0x4E>(v);  // lane ^ 2
    if constexpr (LPQ == 8) v += dppf<0x141>(v);  // the other quad of the 8-lane half
    return v;
  };

  const int nraw = n * tpb;
  for (int base = 0; base < nraw; base += MAXT) {
    if (tid < 64) {
      int c = 0;
      for (int r = 0; r < MAXT && base + r < nraw; r += 64) {
        const int T = base + r + lane;
        bool ok = T < nraw;
        int k0 = 0;
        if (ok) {
          const int j = list[T / tpb];
          ok = j >= 0 && j < a.nblk;
          if (ok) {
            const int64_t kk = static_cast<int64_t>(j) * a.B + (T % tpb) * KT;
            ok = kk <= qmax && kk < a.kv_len;
            if (ok && a.wsel && !a.tbias) ok = a.wsel[rowid * a.k_max + T / tpb] > 0.f;
            k0 = static_cast<int>(kk);
          }
        }
        const uint64_t mk = __ballot(ok);
        if (ok) {
          tk0[c + lanes_below(mk)] = k0;
          tent[c + lanes_below(mk)] = T / tpb;
        }
        c += __popcll(mk);
      }
      if (lane == 0) ntl = c;
    }
    __syncthreads();
    const int nt = ntl;
    if (grp < nt) {
      load_tile(tk0[grp]);
      store_tile(0);
    }
    __syncthreads();
    const int nit = (nt + NS - 1) / NS;
    for (int it = 0; it < nit; ++it) {
      const int buf = it & 1;
      const int cur = it * NS + grp, nxt = cur + NS;
      if (nxt < nt) load_tile(tk0[nxt]);
      if (cur < nt) {
        const int k0 = tk0[cur], s = tent[cur];
        // this query's token selected the block (always, for block rows), and
        // the prior's bias of the block for it, log2 units (scores are too)
        bool on = !tok || ((a.bits[rowid * a.k_max + s] >> qi) & 1ull);
        float bias2 = 0.f;
        if (a.tbias)
          bias2 = a.tbias[(rowid * a.k_max + s) * 64 + qi] * kLog2e;
        else if (a.wsel)
          bias2 = a.sigma * __log2f(a.wsel[rowid * a.k_max + s]);
        on = on && bias2 != -INFINITY;
        // 8 keys at a time, each group its own online-softmax step; the loop
        // is kept rolled so that a group's LDS reads are not all hoisted
#pragma unroll 1
        for (int r0 = 0; r0 < KT; r0 += 8) {
          const float4* kb = &kv[grp][buf][0][r0 * (D / 4) + ds * 4];
          const float4* vb = &kv[grp][buf][1][r0 * (D / 4) + ds * 4];
          float sv[8];
          float mx = -INFINITY;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            float acc = 0.f;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
              const float4 kq = kb[r * (D / 4) + c4];
              acc = fmaf(q[c4 * 4 + 0], kq.x, acc);
              acc = fmaf(q[c4 * 4 + 1], kq.y, acc);
              acc = fmaf(q[c4 * 4 + 2], kq.z, acc);
              acc = fmaf(q[c4 * 4 + 3], kq.w, acc);
            }
            acc = qsum(acc);
            const int64_t key = k0 + r0 + r;
            sv[r] = (key > t || key >= a.kv_len || !on) ? -INFINITY : acc + bias2;
            mx = fmaxf(mx, sv[r]);
          }
          const float mnew = fmaxf(m, mx);
          const float bse = mnew == -INFINITY ? 0.f : mnew;
          const float alpha = exp2f(m - bse);
          m = mnew;
          l *= alpha;
#pragma unroll
          for (int c = 0; c < 16; ++c) o[c] *= alpha;
#pragma unroll
          for (int r = 0; r < 8; ++r) {
            const float p = exp2f(sv[r] - bse);
            l += p;
#pragma unroll
            for (int c4 = 0; c4 < 4; ++c4) {
              const float4 vv = vb[r * (D / 4) + c4];
              o[c4 * 4 + 0] = fmaf(p, vv.x, o[c4 * 4 + 0]);
              o[c4 * 4 + 1] = fmaf(p, vv.y, o[c4 * 4 + 1]);
              o[c4 * 4 + 2] = fmaf(p, vv.z, o[c4 * 4 + 2]);
              o[c4 * 4 + 3] = fmaf(p, vv.w, o[c4 * 4 + 3]);
            }
          }
        }
      }
      // the other buffer's last reads (this group's previous tile) ended at
      // the last barrier
      if (nxt < nt) store_tile(buf ^ 1);
      __syncthreads();
    }
  }
  // merge the groups: every group's state to LDS (the tile buffers are free:
  // the last barrier ended their reads), then group 0 combines
  float* mo = reinterpret_cast<float*>(&kv[0][0][0][0]);  // [NS][NTG][16]
  float* ml = mo + NS * NTG * 16;                            // [NS][64][2]
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4)
    *reinterpret_cast<float4*>(mo + (grp * NTG + gt) * 16 + c4 * 4) =
        make_float4(o[c4 * 4], o[c4 * 4 + 1], o[c4 * 4 + 2], o[c4 * 4 + 3]);
  if (ds == 0) {
    ml[(grp * 64 + qi) * 2] = m;
    ml[(grp * 64 + qi) * 2 + 1] = l;
  }
  __syncthreads();
  if (grp != 0 || t >= a.q_len) return;
  float M = -INFINITY;
#pragma unroll
  for (int gg = 0; gg < NS; ++gg) M = fmaxf(M, ml[(gg * 64 + qi) * 2]);
  const float bse = M == -INFINITY ? 0.f : M;
  float L = 0.f;
#pragma unroll
  for (int c = 0; c < 16; ++c) o[c] = 0.f;
#pragma unroll
  for (int gg = 0; gg < NS; ++gg) {
    const float f = exp2f(ml[(gg * 64 + qi) * 2] - bse);
    L = fmaf(ml[(gg * 64 + qi) * 2 + 1], f, L);
#pragma unroll
    for (int c4 = 0; c4 < 4; ++c4) {
      const float4 v = *reinterpret_cast<const float4*>(mo + (gg * NTG + gt) * 16 + c4 * 4);
      o[c4 * 4 + 0] = fmaf(v.x, f, o[c4 * 4 + 0]);
      o[c4 * 4 + 1] = fmaf(v.y, f, o[c4 * 4 + 1]);
      o[c4 * 4 + 2] = fmaf(v.z, f, o[c4 * 4 + 2]);
      o[c4 * 4 + 3] = fmaf(v.w, f, o[c4 * 4 + 3]);
    }
  }
  if (a.lse && ds == 0)
    a.lse[(static_cast<int64_t>(b) * a.hq + h) * a.q_len + t] =
        L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  const float inv = L > 0.f ? 1.f / L : 0.f;
  float* Og = static_cast<float*>(a.O) + b * a.os.b + h * a.os.h + t * a.os.t + ds * 16;
#pragma unroll
  for (int c4 = 0; c4 < 4; ++c4)
    *reinterpret_cast<float4*>(Og + c4 * 4) =
        make_float4(o[c4 * 4] * inv, o[c4 * 4 + 1] * inv, o[c4 * 4 + 2] * inv, o[c4 * 4 + 3] * inv);
}

// ---------------------------------------------------------------------------
// Ping-pong variant for plain block rows (no token masks, no prior).  Eight
// wavefronts per workgroup, one workgroup per CU: waves 0-3 and 4-7 share the
// four SIMDs pairwise and run the same tile sequence half a tile apart.  Each
// wavefront alternates a matrix phase (P V of the previous tile, then S^T of
// the current one) and a vector phase (the current tile's online softmax), and
// every phase ends at a workgroup barrier, so on each SIMD one wavefront's
// MFMAs run while the other's softmax occupies the VALU.  K/V tiles arrive
// through direct-to-LDS buffer loads into three rotating buffers (unpadded,
// 16-byte chunks XOR-swizzled per row for conflict-free fragment reads).
// ---------------------------------------------------------------------------

template <int D, bool OUT_F32>
__global__ __launch_bounds__(512, 1) void attend_prefill_pp(AttendArgs a, int wpb) {
  constexpr int NW = 8, QT = 2, QPW = 32;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int NC = D / 8;
  constexpr int NI = 64 * NC / 64 / NW;  // 1 KB DMA instructions per wave per tensor
  __shared__ PpLds<D> lds;
  __shared__ int lds_tiles[kMaxTiles];
  __shared__ int lds_ntiles;
  using L = PpLds<D>;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int grp = w >> 2;  // 0: leads, 1: half a tile behind
  const int G = a.hq / a.hkv;
  const int nsub = a.B / 64;
  const int qsub = a.B / QPW;
  const int units = G * qsub;
  int pair, i, sub;
  map_wg(blockIdx.x, a.batch * a.hkv, a.nrow, wpb, pair, i, sub);
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int u = sub * NW + w;
  const bool active = u < units;
  const int hh = active ? u % G : 0;
  const int qs = active ? u / G : 0;
  const int h = g * G + hh;
  const int qpos0 = i * a.B + qs * QPW;
  int qs_max = 0;
  for (int uu = sub * NW; uu < sub * NW + NW && uu < units; ++uu) qs_max = max(qs_max, uu / G);
  int64_t qmax = static_cast<int64_t>(i) * a.B + qs_max * QPW + QPW - 1;
  if (qmax > a.q_len - 1) qmax = a.q_len - 1;

  const int64_t rowid = static_cast<int64_t>(pair) * a.nrow + i;
  int n = a.cnt[rowid];
  n = n < 0 ? 0 : (n > a.k_max ? a.k_max : n);
  TileWalk walk{a.idx + rowid * a.k_max, n, nsub, a.B, a.nblk, a.kv_len, qmax};
  int jpre = -1;
  if (w == 0 && lane < a.k_max * nsub) jpre = walk.list[lane / nsub];

  const auto rk = make_desc(static_cast<const uint16_t*>(a.K) + b * a.ks.b + g * a.ks.h,
                            head_bytes(a.kv_len, a.ks.t, D, 2));
  const auto rv = make_desc(static_cast<const uint16_t*>(a.V) + b * a.vs.b + g * a.vs.h,
                            head_bytes(a.kv_len, a.vs.t, D, 2));
  const uint32_t kst = static_cast<uint32_t>(a.ks.t * 2), vst = static_cast<uint32_t>(a.vs.t * 2);

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
  const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);

  // DMA: wave instruction it fills bytes [1 KB (w NI + it), +1 KB) of a
  // tile; lane l's 16 bytes land at LDS chunk q = 64 (w NI + it) + l, i.e.
  // row q / NC, physical chunk q % NC, which holds logical chunk p ^ swz(row)
  uint32_t koff[NI], voff[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int q = (w * NI + it) * 64 + lane;
    const int r = q / NC, p = q % NC;
    koff[it] = static_cast<uint32_t>(r) * kst + ((p ^ L::kswz(r)) * 16);
    voff[it] = static_cast<uint32_t>(r) * vst + ((p ^ L::vswz(r)) * 16);
  }
  auto load_tile = [&](int k0, int buf) {
    const uint32_t kb = static_cast<uint32_t>(k0) * kst, vb = static_cast<uint32_t>(k0) * vst;
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      lds_dma16(rk, &lds.k[buf][(w * NI + it) * 512], koff[it] + kb);
      lds_dma16(rv, &lds.v[buf][(w * NI + it) * 512], voff[it] + vb);
    }
  };
  // this lane's K fragment offset (elements) per k-step and V transposing-read
  // offset per d tile, at key tile 0 / the first 16 rows: the swizzles depend
  // only on the row within its 16-row (K) or 8-row (V) group, so the other key
  // tiles and halves are the same offsets plus a constant
  int kfo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int r = lane & 15;
    kfo[ks] = r * D + ((ks * 4 + (lane >> 4)) ^ L::kswz(r)) * 8;
  }
  int vfo[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int s16 = lane & 15;
    const int r = (lane >> 4) * 4 + (s16 >> 2);
    const int c = dt * 2 + ((s16 & 3) >> 1);
    vfo[dt] = r * D + (c ^ L::vswz(r)) * 8 + (s16 & 1) * 4;
  }
  static_assert(L::kswz(16) == L::kswz(0) && L::vswz(16) == L::vswz(0) &&
                L::vswz(32) == L::vswz(0), "swizzles repeat every 16 rows");

  f32x4 s[4][QT];
  uint4 pf[QT][2];
  // matrix phase: P V of tile tp (weights pf) and S^T = K Q^T of tile ts
  auto pv_part = [&](int tp) {
    const uint16_t* vb = lds.v[tp % 3];
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) lsum[qt] = mfma16(ones, pf[qt][kk], lsum[qt]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        typedef __attribute__((address_space(3))) v4i16 lds_v4;
        const uint16_t* vp = vb + vfo[dt] + kk * 32 * D;
        const v4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp));
        const v4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp + 16 * D));
        const uint2 u0 = __builtin_bit_cast(uint2, r0), u1 = __builtin_bit_cast(uint2, r1);
        const uint4 vf = make_uint4(u0.x, u0.y, u1.x, u1.y);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) o[dt][qt] = mfma16(vf, pf[qt][kk], o[dt][qt]);
      }
    }
  };
  auto s_part = [&](int ts) {
    const uint16_t* kb = lds.k[ts % 3];
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[kt][qt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const uint4 kf = *reinterpret_cast<const uint4*>(kb + kfo[ks] + kt * 16 * D);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[kt][qt] = mfma16(kf, qf[qt][ks], s[kt][qt]);
      }
    }
  };
  auto mphase = [&](int tp, int ts) {
    __builtin_amdgcn_s_setprio(1);
    if (tp >= 0 && ts >= 0) {
      // the steady state: both products in one scheduling region, P V first
      // in program order (S^T first measured 26 % slower); eight fragment
      // reads ahead, then one read per MFMA (measured 3-4 % faster than
      // ordering the two products separately)
      pv_part(tp);
      s_part(ts);
      __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
      for (int r = 0; r < 40; ++r) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 28, 0);
    } else {
      if (tp >= 0) {
        pv_part(tp);
        // issue order: eight fragment reads ahead, then two MFMAs per two reads
        __builtin_amdgcn_sched_group_barrier(0x100, 8, 0);
#pragma unroll
        for (int r = 0; r < 12; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 12, 0);
      }
      if (ts >= 0) {
        s_part(ts);
        __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
#pragma unroll
        for (int r = 0; r < 10; ++r) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 12, 1);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // vector phase: online softmax of s (tile at key k0) into pf
  auto vphase = [&](int k0) {
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
    float mx[QT];
    bool grow = false;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float t0 = max3f(s[0][qt][0], s[0][qt][1], s[0][qt][2]);
      const float t1 = max3f(s[0][qt][3], s[1][qt][0], s[1][qt][1]);
      const float t2 = max3f(s[1][qt][2], s[1][qt][3], s[2][qt][0]);
      const float t3 = max3f(s[2][qt][1], s[2][qt][2], s[2][qt][3]);
      const float t4 = max3f(s[3][qt][0], s[3][qt][1], s[3][qt][2]);
      const float t5 = max3f(t0, t1, t2);
      const float t6 = max3f(t3, t4, s[3][qt][3]);
      float v = fmaxf(t5, t6);
      v = xmax16(v);
      mx[qt] = v * sc;
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
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float nb = m[qt] == -INFINITY ? 0.f : -m[qt];
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
  };

  const int nraw = n * nsub;
  for (int base = 0; base < nraw; base += kMaxTiles) {
    if (w == 0) {
      int c = 0;
#pragma clang loop unroll(disable)
      for (int r = 0; r < kMaxTiles && base + r < nraw; r += 64) {
        const int T = base + r + lane;
        const int64_t k0 = T >= nraw ? -1 : (T < 64 ? walk.key0_of(jpre, T) : walk.key0(T));
        const uint64_t mk = __ballot(k0 >= 0);
        if (k0 >= 0) lds_tiles[c + lanes_below(mk)] = static_cast<int>(k0);
        c += __popcll(mk);
      }
      if (lane == 0) lds_ntiles = c;
    }
    __syncthreads();
    const int ntiles = lds_ntiles;
    if (ntiles > 0) load_tile(lds_tiles[0], 0);
    __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): Q fragments and tile 0
    __syncthreads();
    // Slot sl: group 0 runs its phase sl, group 1 its phase sl - 1; phase 2t
    // is the matrix phase (P V of tile t-1, S^T of tile t), phase 2t+1 the
    // softmax of tile t.  Tile t is read in slots 2t .. 2t+3; its loads go
    // out at slot 2t-2 (into the buffer tile t-3 left at slot 2t-3) and are
    // complete before the barrier that ends slot 2t-1.
    const int nslots = 2 * ntiles + 2;
#pragma clang loop unroll(disable)
    for (int sl = 0; sl < nslots; ++sl) {
      if (!(sl & 1) && (sl >> 1) + 1 < ntiles) load_tile(lds_tiles[(sl >> 1) + 1], ((sl >> 1) + 1) % 3);
      const int ph = sl - grp;
      if (active && ph >= 0) {
        const int t = ph >> 1;
        if (!(ph & 1))
          mphase(t >= 1 ? t - 1 : -1, t < ntiles ? t : -1);
        else if (t < ntiles)
          vphase(lds_tiles[t]);
      }
      if (sl & 1) __builtin_amdgcn_s_waitcnt(0x0F70);  // vmcnt(0): this slot pair's loads
      __syncthreads();
    }
  }

  if (!active) return;
  uint8_t* Ob = static_cast<uint8_t*>(a.O);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const float lt = lsum[qt][0];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t t = qpos0 + qt * 16 + (lane & 15);
    if (t >= a.q_len) continue;
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

template <int D>
hipError_t prefill_pp_launch(const AttendArgs& a, hipStream_t stream) {
  const int G = a.hq / a.hkv;
  const int units = G * (a.B / 32);
  const int wpb = (units + 7) / 8;
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * a.nrow * wpb;
  if (a.out_f32)
    hipLaunchKernelGGL((attend_prefill_pp<D, true>), dim3(grid), dim3(512), 0, stream, a, wpb);
  else
    hipLaunchKernelGGL((attend_prefill_pp<D, false>), dim3(grid), dim3(512), 0, stream, a, wpb);
  return hipGetLastError();
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
  if (a.wsel) return prefill_bf16_launch<D, 2, 4, false, true>(a, stream);
  // rows of many key tiles: the ping-pong kernel (measured 3-5 % faster at 64
  // tiles a row); short rows keep two independent 4-wave workgroups per CU,
  // which hide each other's tails better (16 tiles a row: ~6 % faster)
  return a.k_max * (a.B / 64) >= kPingPongMinTiles ? prefill_pp_launch<D>(a, stream)
                                                   : prefill_bf16_launch<D, 2, 4, false, false>(a, stream);
}

}  // namespace

hipError_t launch_attend_prefill(const AttendArgs& a, hipStream_t stream) {
  if (a.bf16) return a.d == 64 ? prefill_bf16_dispatch<64>(a, stream) : prefill_bf16_dispatch<128>(a, stream);
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hq * a.nrow * (a.bits ? 1 : a.B / 64);
  if (a.d == 64)
    hipLaunchKernelGGL(attend_prefill_f32<64>, dim3(grid), dim3(1024), 0, stream, a);
  else
    hipLaunchKernelGGL(attend_prefill_f32<128>, dim3(grid), dim3(1024), 0, stream, a);
  return hipGetLastError();
}

}  // namespace bsa
