// Single-token decode, routing and attention in one launch.
//
// One workgroup of 512 threads owns one (batch, KV head) row and a slice of
// its query heads (hsplit workgroups per row split the GQA group, so that
// 128 rows still fill all 256 CUs).  Phase R ("DashAttention", Declaração do
// Problema; cached block summaries of Estágio 0): the routing query is the sum
// of the group's query heads, the summaries of the complete blocks before the
// query's own block are streamed from HBM with several 16-byte loads in
// flight per lane, scored in fp32, and the top-k (forced blocks added, ties
// to the lower block id) is selected by the exact radix select in LDS.
// Phase A: the selected blocks are streamed in chunks of keys, each wavefront
// keeping an online softmax per query head; the wavefronts' partial states
// are merged in LDS.  Decode is bound by HBM transfers (summaries + the
// selected K/V), so everything stays on the VALU.
// PAGED: the K/V cache is a pool of pages of B tokens; the selection is
// translated through the sequence's page table into LDS once, and each chunk
// load builds its buffer resource over its page (rows past the sequence
// length read as zero, as in the contiguous layout).
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace bsa {

namespace {

constexpr int kNT = 512;
constexpr int kNW = kNT / kWave;
constexpr int kUnroll = 16;  // summary loads in flight per lane
constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ void xcd_row(int id, int rows, int hsplit, int& row, int& hs) {
  // the hsplit workgroups of a row share its summaries and K/V through one L2
  if (rows % 8 == 0) {
    const int x = id % 8, s = id / 8;
    hs = s % hsplit;
    row = (s / hsplit) * 8 + x;
  } else {
    row = id / hsplit;
    hs = id % hsplit;
  }
}

template <typename T, int D, int GS, bool PAGED>
__global__ __launch_bounds__(kNT) void decode_fused(DecodeArgs a) {
  constexpr int LPK = D / 8;       // lanes per key row (8 elements each)
  constexpr int KPI = kWave / LPK;  // keys per wave load instruction
  // keys per chunk: two chunks of K and V are in registers at once, so the
  // chunk shrinks as the head slice (accumulators) or the element size grows
  constexpr int CK = sizeof(T) == 2 ? (GS <= 2 ? 32 : 16) : (GS <= 1 ? 16 : 8);
  constexpr int KPC = CK / KPI;     // load instructions per chunk
  static_assert(KPC >= 1, "chunk shorter than one load instruction");
  constexpr int LPR = D / 4;       // lanes per fp32 summary row
  constexpr int RPW = kWave / LPR;  // summary rows per wave load instruction
  extern __shared__ float dyn[];    // [nblk] scores, then the merge buffer
  __shared__ float qh[D];
  __shared__ float qa[GS][D];
  // bf16 with up to 4 heads: q.k by packed bf16 dot products from the
  // queries as stored (more heads keep the fp32 form: registers)
  constexpr bool kDot = sizeof(T) == 2 && GS <= 4;
  __shared__ uint16_t qr[kDot ? GS : 1][D];
  __shared__ int hist[256];
  __shared__ int bcast[2];
  __shared__ int wave_tot[kNW];
  __shared__ int sel_n;
  int* sel = reinterpret_cast<int*>(dyn + a.lds_floats);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int w = tid >> 6;
  const int rows = a.batch * a.hkv;
  int row, hs;
  xcd_row(blockIdx.x, rows, a.hsplit, row, hs);
  const int b = row / a.hkv, g = row % a.hkv;
  const int G = a.hq / a.hkv;
  const int gs = G / a.hsplit;  // heads of this workgroup (<= GS)
  const int h0 = g * G + hs * gs;
  int64_t L = a.kv_lens ? static_cast<int64_t>(a.kv_lens[b]) : a.kv_len;
  L = L < 1 ? 1 : (L > a.kv_len ? a.kv_len : L);
  const T* Qb = static_cast<const T*>(a.Q) + b * a.qs.b;
  const float scl = a.sm_scale * kLog2e;
  auto qval = [&](int h, int c) {
    const T* qp = Qb + h * a.qs.h;
    if constexpr (sizeof(T) == 2)
      return bf16_to_f32(qp[c]);
    else
      return static_cast<float>(qp[c]);
  };
  // the attention's query heads, scaled for exp2
  auto load_qa = [&]() {
    for (int e = tid; e < gs * D; e += kNT) {
      const int hh = e / D, c = e % D;
      if constexpr (kDot)
        qr[hh][c] = (Qb + (h0 + hh) * a.qs.h)[c];
      else
        qa[hh][c] = qval(h0 + hh, c) * scl;
    }
  };

  if (a.route) {
    RowRule rule;
    rule.mode = 1;
    rule.entmax = 0;
    rule.force = a.force;
    rule.B = a.B;
    rule.kv_len = a.kv_len;
    rule.kv_lens = a.kv_lens;
    const RowInfo ri = row_info(rule, b, 0);
    const int n = ri.cand_end;
    // Stream the summaries of the candidates.  Wavefront w takes the slices
    // of kSel candidates w, w + kNW, ... (its own contiguous rows), in rounds
    // of kUnroll loads per lane with the next round in flight, and the scores
    // go to LDS.  With a top-m below kSel a wavefront selects the exact top-m
    // of each slice it finished at once (wave_topm, no barrier: the slices end
    // at different times, so this first round of the tournament overlaps the
    // other wavefronts' streaming); its survivors, in id order and padded
    // with -1, wait in bk0/bi0 for the remaining rounds.
    const int c4 = lane % LPR;
    const auto rs = make_rsrc(a.S + static_cast<int64_t>(row) * a.nblk * D,
                              static_cast<uint32_t>(n) * D * 4);  // candidates only
    constexpr int RROWS = RPW * kUnroll;  // rows per wavefront round
    constexpr int RPS = kSel / RROWS;     // rounds per slice
    static_assert(kSel % RROWS == 0, "slice of whole rounds");
    const int nslice = (n + kSel - 1) / kSel;
    const int nq = nslice > w ? ((nslice - 1 - w) / kNW + 1) * RPS : 0;  // this wavefront's rounds
    auto round_row0 = [&](int q) { return (w + (q / RPS) * kNW) * kSel + (q % RPS) * RROWS; };
    // two register buffers: the next round's loads are in flight while the
    // current one is reduced (rows past n read as zero, nothing is written)
    uint4 va[kUnroll], vb[kUnroll];
    auto issue = [&](int q, uint4 (&v)[kUnroll]) {
      const int r0 = q < nq ? round_row0(q) : n;
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t j = static_cast<uint32_t>(r0 + u * RPW + lane / LPR);
        v[u] = buf_load16(rs, j * (D * 4) + c4 * 16);
      }
    };
    int m = a.k_total - ri.nforced;
    m = m < 0 ? 0 : m;
    const bool waves_first = m > 0 && m < kSel;
    const int cap = nslice * (m > 0 ? m : 1);
    uint32_t* bk0 = reinterpret_cast<uint32_t*>(sel + a.k_total);
    int32_t* bi0 = reinterpret_cast<int32_t*>(bk0 + cap);
    uint32_t* bk1 = reinterpret_cast<uint32_t*>(bi0 + cap);
    int32_t* bi1 = reinterpret_cast<int32_t*>(bk1 + cap);
    uint32_t* fk = reinterpret_cast<uint32_t*>(bi1 + cap);
    int32_t* fi = reinterpret_cast<int32_t*>(fk + a.k_total);
    // the first round of summaries is requested before the query heads, so
    // the two reads' latencies overlap; then the attention heads and the
    // routing query (the group's sum)
    if (nq > 0) issue(0, va);
    load_qa();
    for (int c = tid; c < D; c += kNT) {
      float s = 0.f;
      for (int hh = 0; hh < G; ++hh) s += qval(g * G + hh, c);
      qh[c] = s;
    }
    __syncthreads();
    const float4 q4 = reinterpret_cast<const float4*>(qh)[c4];
    auto reduce = [&](int q, const uint4 (&v)[kUnroll]) {
      const int r0 = round_row0(q);
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = r0 + u * RPW + lane / LPR;
        float p = q4.x * __uint_as_float(v[u].x);
        p = fmaf(q4.y, __uint_as_float(v[u].y), p);
        p = fmaf(q4.z, __uint_as_float(v[u].z), p);
        p = fmaf(q4.w, __uint_as_float(v[u].w), p);
        p = lane_sum<LPR>(p);
        if (c4 == 0 && j < n) dyn[j] = p * a.score_scale;
      }
      if (!waves_first || q % RPS != RPS - 1) return;
      // the slice is complete: its exact top-m (element e of lane l is
      // candidate r0 + 64 e + l, so ties go to the lower id)
      __builtin_amdgcn_wave_barrier();
      const int sl = w + (q / RPS) * kNW;
      uint32_t key[4];
      bool valid[4], pick[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = sl * kSel + e * kWave + lane;
        valid[e] = i < n && !is_forced(ri, i);
        key[e] = valid[e] ? float_key(dyn[i]) : 0u;
      }
      wave_topm<4>(key, valid, m, pick);
      int cnt = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t mk = __ballot(pick[e]);
        if (pick[e]) {
          const int pos = sl * m + cnt + lanes_below(mk);
          bk0[pos] = key[e];
          bi0[pos] = sl * kSel + e * kWave + lane;
        }
        cnt += __popcll(mk);
      }
      for (int t = cnt + lane; t < m; t += kWave) bi0[sl * m + t] = -1;
    };
    for (int q = 0; q < nq; q += 2) {
      issue(q + 1, vb);
      reduce(q, va);
      if (q + 1 >= nq) break;
      issue(q + 2, va);
      reduce(q + 1, vb);
    }
    __syncthreads();
    const int n_elig = n - ri.nforced_below(n);
    auto get = [&](int e, uint32_t& key) -> bool {
      if (e >= n || is_forced(ri, e)) return false;
      key = float_key(dyn[e]);
      return true;
    };
    int32_t* gidx = a.idx ? a.idx + static_cast<int64_t>(row) * a.k_total : nullptr;
    const bool write = gidx != nullptr && hs == 0;
    if (m < kSel) {
      // the remaining rounds over the slices' survivors (per-wave exact top-m
      // of 256-entry slices, ballot bit-splitting, until one slice is left);
      // forced blocks added around the routed ids, which lie strictly between
      // them
      const int len = nslice * m;
      const int nr = m == 0 ? 0
                            : tournament<kNT>(
                                  len, m,
                                  [&](int i, uint32_t& key, int32_t& id, bool& valid) {
                                    valid = i < len && bi0[i] >= 0;
                                    key = valid ? bk0[i] : 0u;
                                    id = valid ? bi0[i] : -1;
                                  },
                                  bk1, bi1, bk0, bi0, fk, fi, a.k_total);
      const int lead = (ri.f0 == 0 && (a.force & 2u)) ? 1 : 0;
      for (int q = tid; q < nr; q += kNT) sel[lead + q] = fi[q];
      if (tid == 0) {
        int c = lead + nr;
        if (lead) sel[0] = 0;
        if (!lead && ri.f0 >= 0) sel[c++] = ri.f0;
        if (ri.f1 >= 0) sel[c++] = ri.f1;
        sel_n = c;
      }
      __syncthreads();
      if (write) {
        const int c = sel_n;
        for (int p = tid; p < a.k_total; p += kNT) gidx[p] = p < c ? sel[p] : -1;
        if (tid == 0 && a.cnt) a.cnt[row] = c;
      }
    } else {
      const int c = select_and_write<kNT>(
          ri, ri.span, m, n_elig, get,
          [&](int p, int e) {
            sel[p] = e;
            if (write) gidx[p] = e;
          },
          a.k_total, hist, bcast, wave_tot);
      if (tid == 0) {
        sel_n = c;
        if (write && a.cnt) a.cnt[row] = c;
      }
      __syncthreads();
    }
  } else {
    load_qa();
    int c = a.cnt[row];
    c = c < 0 ? 0 : (c > a.k_total ? a.k_total : c);
    for (int p = tid; p < c; p += kNT) sel[p] = a.idx[static_cast<int64_t>(row) * a.k_total + p];
    if (tid == 0) sel_n = c;
    __syncthreads();
  }
  if (!a.attend) return;

  // ---- attention over the selected blocks for heads h0 .. h0+gs-1 ----
  const int nsel = sel_n;
  const int cpb = a.B / CK;  // chunks per block
  const int nchunk = nsel * cpb;
  // paged: the selected blocks' pages (the selection buffers past sel[k_total]
  // are free once the selection is made)
  int* pgs = sel + a.k_total;
  if constexpr (PAGED) {
    for (int q = tid; q < nsel; q += kNT) {
      const int j = sel[q];
      const int pg = (j >= 0 && j < a.nblk && j < a.max_pages)
                         ? a.table[static_cast<int64_t>(b) * a.max_pages + j] : -1;
      pgs[q] = pg >= 0 && pg < a.num_pages ? pg : -1;
    }
    __syncthreads();
  }
  // K/V rows at or past L read as zero through the buffer resources
  const auto rk = make_rsrc(static_cast<const T*>(a.K) + b * a.ks.b + g * a.ks.h,
                            head_bytes(L, a.ks.t, D, sizeof(T)));
  const auto rv = make_rsrc(static_cast<const T*>(a.V) + b * a.vs.b + g * a.vs.h,
                            head_bytes(L, a.vs.t, D, sizeof(T)));
  const uint32_t kst = static_cast<uint32_t>(a.ks.t * sizeof(T));
  const uint32_t vst = static_cast<uint32_t>(a.vs.t * sizeof(T));
  const int c8 = lane % LPK, kg = lane / LPK;
  float m[GS], l[GS], o[GS][8];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    m[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }
  constexpr int RPL = sizeof(T) == 2 ? 1 : 2;  // 16-byte loads per 8 elements
  // Chunk ch covers keys [t0, t0 + CK) of selected block sel[ch / cpb];
  // invalid chunks load from an out-of-range offset (zeros) and are masked.
  auto chunk_t0 = [&](int ch) -> int {
    if (ch >= nchunk) return -1;
    const int j = sel[ch / cpb];
    return (j >= 0 && j < a.nblk) ? j * a.B + (ch % cpb) * CK : -1;
  };
  auto issue = [&](int ch, uint4 (&kb)[KPC][RPL], uint4 (&vb)[KPC][RPL]) {
    int t0 = chunk_t0(ch);
    auto rkc = rk, rvc = rv;
    if constexpr (PAGED) {
      // the chunk's page (wave-uniform): rows [0, L - jB) of it are valid
      const int pg = t0 < 0 ? -1 : __builtin_amdgcn_readfirstlane(pgs[ch / cpb]);
      const int j = t0 < 0 ? 0 : t0 / a.B;
      const int64_t rows = pg < 0 ? 0 : (L - static_cast<int64_t>(j) * a.B < a.B
                                             ? L - static_cast<int64_t>(j) * a.B : a.B);
      const int64_t pgo = pg < 0 ? 0 : pg;
      rkc = make_rsrc(static_cast<const T*>(a.K) + pgo * a.page_k + g * a.ks.h,
                      head_bytes(rows, a.ks.t, D, sizeof(T)));
      rvc = make_rsrc(static_cast<const T*>(a.V) + pgo * a.page_v + g * a.vs.h,
                      head_bytes(rows, a.vs.t, D, sizeof(T)));
      if (pg < 0) t0 = -1;
      else t0 -= j * a.B;  // page-relative
    }
#pragma unroll
    for (int it = 0; it < KPC; ++it) {
      const uint32_t t = static_cast<uint32_t>(t0 + it * KPI + kg);
      const uint32_t ko = t0 < 0 ? 0xFFFFFF00u : t * kst + c8 * 8 * sizeof(T);
      const uint32_t vo = t0 < 0 ? 0xFFFFFF00u : t * vst + c8 * 8 * sizeof(T);
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        kb[it][r] = buf_load16(rkc, ko + 16 * r);
        vb[it][r] = buf_load16(rvc, vo + 16 * r);
      }
    }
  };
  auto unpack = [&](const uint4 (&u)[RPL], float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
      x[0] = bf16_lo(u[0].x); x[1] = bf16_hi(u[0].x);
      x[2] = bf16_lo(u[0].y); x[3] = bf16_hi(u[0].y);
      x[4] = bf16_lo(u[0].z); x[5] = bf16_hi(u[0].z);
      x[6] = bf16_lo(u[0].w); x[7] = bf16_hi(u[0].w);
    } else {
      x[0] = __uint_as_float(u[0].x); x[1] = __uint_as_float(u[0].y);
      x[2] = __uint_as_float(u[0].z); x[3] = __uint_as_float(u[0].w);
      x[4] = __uint_as_float(u[RPL - 1].x); x[5] = __uint_as_float(u[RPL - 1].y);
      x[6] = __uint_as_float(u[RPL - 1].z); x[7] = __uint_as_float(u[RPL - 1].w);
    }
  };
  // kDot: the lane's 8 query elements of each head as bf16 pairs; q.k by
  // packed bf16 dot products (exact products, fp32 sums), scaled after the
  // reduction over the key's lanes; each V slice is unpacked once for all
  // heads
  uint4 qp[kDot ? GS : 1];
  if constexpr (kDot) {
#pragma unroll
    for (int hh = 0; hh < GS; ++hh)
      qp[hh] = hh < gs ? *reinterpret_cast<const uint4*>(&qr[hh][c8 * 8]) : make_uint4(0u, 0u, 0u, 0u);
  }
  auto dot8 = [&](const uint4& k, const uint4& q) {
    float acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.x),
                                                __builtin_bit_cast(bf16x2_t, q.x), 0.f, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.y),
                                          __builtin_bit_cast(bf16x2_t, q.y), acc, false);
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.z),
                                          __builtin_bit_cast(bf16x2_t, q.z), acc, false);
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, k.w),
                                           __builtin_bit_cast(bf16x2_t, q.w), acc, false);
  };
  auto compute = [&](int ch, const uint4 (&kb)[KPC][RPL], const uint4 (&vb)[KPC][RPL]) {
    const int t0 = chunk_t0(ch);
    if (t0 < 0) return;
    bool ok[KPC];
#pragma unroll
    for (int it = 0; it < KPC; ++it) ok[it] = t0 + it * KPI + kg < L;
    if constexpr (kDot) {
      float sv[GS][KPC];
#pragma unroll
      for (int hh = 0; hh < GS; ++hh) {
        if (hh >= gs) break;
#pragma unroll
        for (int it = 0; it < KPC; ++it) {
          const float acc = lane_sum<LPK>(dot8(kb[it][0], qp[hh]));
          sv[hh][it] = ok[it] ? acc * scl : -INFINITY;
        }
      }
      float base[GS], ls[GS];
#pragma unroll
      for (int hh = 0; hh < GS; ++hh) {
        if (hh >= gs) break;
        float mx = -INFINITY;
#pragma unroll
        for (int it = 0; it < KPC; ++it) mx = fmaxf(mx, sv[hh][it]);
        if constexpr (LPK == 8) mx = fmaxf(mx, __shfl_xor(mx, 8, kWave));
        mx = swap32_max(swap16_max(mx));
        const float mn = fmaxf(m[hh], mx);
        base[hh] = mn == -INFINITY ? 0.f : mn;
        const float f = __builtin_amdgcn_exp2f(m[hh] - base[hh]);
        m[hh] = mn;
        ls[hh] = 0.f;
        l[hh] *= f;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] *= f;
      }
#pragma unroll
      for (int it = 0; it < KPC; ++it) {
        float vv[8];
        unpack(vb[it], vv);
#pragma unroll
        for (int hh = 0; hh < GS; ++hh) {
          if (hh >= gs) break;
          const float p = __builtin_amdgcn_exp2f(sv[hh][it] - base[hh]);
          ls[hh] += p;
#pragma unroll
          for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(p, vv[e], o[hh][e]);
        }
      }
#pragma unroll
      for (int hh = 0; hh < GS; ++hh) {
        if (hh >= gs) break;
        l[hh] += ls[hh];
      }
    } else {
  #pragma unroll
      for (int hh = 0; hh < GS; ++hh) {
        if (hh >= gs) break;
        float s[KPC];
        float mx = -INFINITY;
  #pragma unroll
        for (int it = 0; it < KPC; ++it) {
          float kv[8];
          unpack(kb[it], kv);
          float acc = 0.f;
  #pragma unroll
          for (int e = 0; e < 8; ++e) acc = fmaf(kv[e], qa[hh][c8 * 8 + e], acc);
          acc = lane_sum<LPK>(acc);
          s[it] = ok[it] ? acc : -INFINITY;
          mx = fmaxf(mx, s[it]);
        }
        if constexpr (LPK == 8) mx = fmaxf(mx, __shfl_xor(mx, 8, kWave));
        mx = swap32_max(swap16_max(mx));
        const float mn = fmaxf(m[hh], mx);
        const float base = mn == -INFINITY ? 0.f : mn;
        const float f = __builtin_amdgcn_exp2f(m[hh] - base);
        m[hh] = mn;
        float ls = 0.f;
  #pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] *= f;
  #pragma unroll
        for (int it = 0; it < KPC; ++it) {
          const float p = __builtin_amdgcn_exp2f(s[it] - base);
          float vv[8];
          unpack(vb[it], vv);
          ls += p;
  #pragma unroll
          for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(p, vv[e], o[hh][e]);
        }
        l[hh] = l[hh] * f + ls;
      }
    }
  };
  {
    uint4 ka[KPC][RPL], va2[KPC][RPL], kb2[KPC][RPL], vb2[KPC][RPL];
    if (w < nchunk) issue(w, ka, va2);
    for (int ch = w; ch < nchunk; ch += 2 * kNW) {
      issue(ch + kNW, kb2, vb2);
      compute(ch, ka, va2);
      if (ch + kNW >= nchunk) break;
      issue(ch + 2 * kNW, ka, va2);
      compute(ch + kNW, kb2, vb2);
    }
  }
  // reduce over the key groups of the wave (lanes sharing c8), then merge the
  // waves: merge[w][hh] = {m, l, o[D]}
  float* merge = dyn;
  constexpr int PART = D + 2;
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    if (hh >= gs) break;
    float lt = l[hh];
    if constexpr (LPK == 8) lt += __shfl_xor(lt, 8, kWave);
    lt = swap32_sum(swap16_sum(lt));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = o[hh][e];
      if constexpr (LPK == 8) v += __shfl_xor(v, 8, kWave);
      v = swap32_sum(swap16_sum(v));
      if (kg == 0) merge[(w * GS + hh) * PART + 2 + c8 * 8 + e] = v;
    }
    if (lane == 0) {
      merge[(w * GS + hh) * PART + 0] = m[hh];
      merge[(w * GS + hh) * PART + 1] = lt;
    }
  }
  __syncthreads();
  for (int e = tid; e < gs * D; e += kNT) {
    const int hh = e / D, c = e % D;
    float M = -INFINITY;
    for (int ww = 0; ww < kNW; ++ww) M = fmaxf(M, merge[(ww * GS + hh) * PART]);
    const float base = M == -INFINITY ? 0.f : M;
    float ls = 0.f, acc = 0.f;
    for (int ww = 0; ww < kNW; ++ww) {
      const float* pp = merge + (ww * GS + hh) * PART;
      const float f = __builtin_amdgcn_exp2f(pp[0] - base);
      ls += f * pp[1];
      acc += f * pp[2 + c];
    }
    const float v = ls > 0.f ? acc / ls : 0.f;
    const int64_t off = b * a.os.b + (h0 + hh) * a.os.h + c;
    if (a.out_f32)
      static_cast<float*>(a.O)[off] = v;
    else
      static_cast<uint16_t*>(a.O)[off] = f32_to_bf16(v);
  }
}

template <typename T, int D, int GS, bool PAGED>
hipError_t launch_gs_p(const DecodeArgs& a, hipStream_t stream) {
  const size_t dyn = (static_cast<size_t>(a.lds_floats) + decode_sel_ints(a.nblk, a.k_total)) * 4;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_fused<T, D, GS, PAGED>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * a.hsplit;
  hipLaunchKernelGGL((decode_fused<T, D, GS, PAGED>), dim3(grid), dim3(kNT), dyn, stream, a);
  return hipGetLastError();
}
template <typename T, int D, int GS>
hipError_t launch_gs(const DecodeArgs& a, hipStream_t stream) {
  return a.table ? launch_gs_p<T, D, GS, true>(a, stream) : launch_gs_p<T, D, GS, false>(a, stream);
}

template <typename T, int D>
hipError_t launch_t(const DecodeArgs& a, hipStream_t stream) {
  const int gs = a.hq / a.hkv / a.hsplit;
  if (gs <= 1) return launch_gs<T, D, 1>(a, stream);
  if (gs <= 2) return launch_gs<T, D, 2>(a, stream);
  if (gs <= 4) return launch_gs<T, D, 4>(a, stream);
  return launch_gs<T, D, 8>(a, stream);
}

}  // namespace

int decode_lds_floats(int nblk, int d, int gs_max) {
  const int merge = kNW * gs_max * (d + 2);
  return nblk > merge ? nblk : merge;
}

int decode_sel_ints(int nblk, int k_total) {
  // the selection, then (top-m below kSel) four tournament buffers and its
  // output keys and ids; a paged cache reuses them for the selection's pages
  // (at least k_total ints)
  const long cap = ((static_cast<long>(nblk) + kSel - 1) / kSel) * (k_total > 0 ? k_total : 1);
  const long tb = k_total < kSel ? 4 * cap + 2 * k_total : 0;
  return static_cast<int>(k_total + (tb > k_total ? tb : k_total));
}

hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t stream) {
  if (a.bf16) return a.d == 64 ? launch_t<uint16_t, 64>(a, stream) : launch_t<uint16_t, 128>(a, stream);
  return a.d == 64 ? launch_t<float, 64>(a, stream) : launch_t<float, 128>(a, stream);
}

}  // namespace bsa

// ===========================================================================
// Partitioned decode step: every (batch, KV head) row is served by `parts`
// workgroups that stream disjoint data, so all CUs pull distinct bytes.
//   decode_route_part   partition p scores the candidate blocks
//                       [p*per, (p+1)*per) and keeps its exact local top-m
//                       (a block in the global top-m is in its partition's
//                       top-m under the same tie rule).
//   decode_attend_part  merges the parts' candidates into the row's top-m,
//                       adds the forced blocks, attends a contiguous share of
//                       the selected blocks for every query head and writes
//                       its partial softmax state.
//   decode_combine      merges the parts' partial states of a row into O.
// ===========================================================================
namespace bsa {
namespace {

__device__ __forceinline__ void part_map(int id, int rows, int parts, int& row, int& p) {
  if (rows % 8 == 0) {  // the parts of a row on one XCD (shared L2)
    const int x = id % 8, s = id / 8;
    p = s % parts;
    row = (s / parts) * 8 + x;
  } else {
    row = id / parts;
    p = id % parts;
  }
}


template <int D>
__global__ __launch_bounds__(kNT) void decode_route_part(DecodeArgs a) {
  constexpr int LPR = D / 4;
  constexpr int RPW = kWave / LPR;
  extern __shared__ float dyn[];  // [per] scores, then 2 x 2 x tournament buffers
  __shared__ float qh[D];
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rows = a.batch * a.hkv;
  int row, p;
  part_map(blockIdx.x, rows, a.parts, row, p);
  const int b = row / a.hkv, g = row % a.hkv;
  const int G = a.hq / a.hkv;
  RowRule rule;
  rule.mode = 1;
  rule.entmax = 0;
  rule.force = a.force;
  rule.B = a.B;
  rule.kv_len = a.kv_len;
  rule.kv_lens = a.kv_lens;
  const RowInfo ri = row_info(rule, b, 0);
  const int n = ri.cand_end;
  const int per = (n + a.parts - 1) / a.parts;
  const int lo = p * per < n ? p * per : n;
  const int hi = lo + per < n ? lo + per : n;
  const int len = hi - lo;
  int m = a.k_total - ri.nforced;
  m = m < 0 ? 0 : m;
  if (a.bf16) {
    const uint16_t* Qb = static_cast<const uint16_t*>(a.Q) + b * a.qs.b;
    for (int c = tid; c < D; c += kNT) {
      float s = 0.f;
      for (int hh = 0; hh < G; ++hh) s += bf16_to_f32(Qb[(g * G + hh) * a.qs.h + c]);
      qh[c] = s;
    }
  } else {
    const float* Qb = static_cast<const float*>(a.Q) + b * a.qs.b;
    for (int c = tid; c < D; c += kNT) {
      float s = 0.f;
      for (int hh = 0; hh < G; ++hh) s += Qb[(g * G + hh) * a.qs.h + c];
      qh[c] = s;
    }
  }
  __syncthreads();
  const int c4 = lane % LPR;
  const float4 q4 = reinterpret_cast<const float4*>(qh)[c4];
  const auto rs = make_rsrc(a.S + (static_cast<int64_t>(row) * a.nblk + lo) * D,
                            static_cast<uint32_t>(len) * D * 4);
  constexpr int STEP = kNW * RPW;
  constexpr int ROUND = STEP * kUnroll;
  uint4 va[kUnroll], vb[kUnroll];
  auto issue = [&](int base, uint4 (&v)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const uint32_t j = static_cast<uint32_t>(base + u * STEP + w * RPW + lane / LPR);
      v[u] = buf_load16(rs, j * (D * 4) + c4 * 16);
    }
  };
  auto reduce = [&](int base, const uint4 (&v)[kUnroll]) {
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int j = base + u * STEP + w * RPW + lane / LPR;
      float s = q4.x * __uint_as_float(v[u].x);
      s = fmaf(q4.y, __uint_as_float(v[u].y), s);
      s = fmaf(q4.z, __uint_as_float(v[u].z), s);
      s = fmaf(q4.w, __uint_as_float(v[u].w), s);
      s = lane_sum<LPR>(s);
      if (c4 == 0 && j < len) dyn[j] = s * a.score_scale;
    }
  };
  if (len > 0) issue(0, va);
  for (int base = 0; base < len; base += 2 * ROUND) {
    issue(base + ROUND, vb);
    reduce(base, va);
    if (base + ROUND >= len) break;
    issue(base + 2 * ROUND, va);
    reduce(base + ROUND, vb);
  }
  __syncthreads();
  // local top-m of the partition, kept in block-id order
  const int cap = ((len + kSel - 1) / kSel) * m;
  uint32_t* bk0 = reinterpret_cast<uint32_t*>(dyn + a.lds_floats);
  int32_t* bi0 = reinterpret_cast<int32_t*>(bk0 + cap);
  uint32_t* bk1 = reinterpret_cast<uint32_t*>(bi0 + cap);
  int32_t* bi1 = reinterpret_cast<int32_t*>(bk1 + cap);
  const int64_t off = (static_cast<int64_t>(row) * a.parts + p) * a.mpad;
  tournament<kNT>(
      len, m,
      [&](int i, uint32_t& key, int32_t& id, bool& valid) {
        const int j = lo + i;
        valid = i < len && !is_forced(ri, j);
        key = valid ? float_key(dyn[i]) : 0u;
        id = j;
      },
      bk0, bi0, bk1, bi1, a.cand_key + off, a.cand_id + off, a.mpad);
}

template <typename T, int D, int GS, bool PAGED>
__global__ __launch_bounds__(kNT) void decode_attend_part(DecodeArgs a) {
  constexpr int LPK = D / 8;
  constexpr int KPI = kWave / LPK;
  constexpr int CK = sizeof(T) == 2 ? (GS <= 2 ? 32 : 16) : (GS <= 1 ? 16 : 8);
  constexpr int KPC = CK / KPI;
  constexpr int RPL = sizeof(T) == 2 ? 1 : 2;
  constexpr int PART = D + 2;
  extern __shared__ float dyn[];
  __shared__ float qa[GS][D];
  __shared__ int sel_n;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int rows = a.batch * a.hkv;
  int row, p;
  part_map(blockIdx.x, rows, a.attend ? a.parts : 1, row, p);
  const int b = row / a.hkv, g = row % a.hkv;
  const int G = a.hq / a.hkv;
  RowRule rule;
  rule.mode = 1;
  rule.entmax = 0;
  rule.force = a.force;
  rule.B = a.B;
  rule.kv_len = a.kv_len;
  rule.kv_lens = a.kv_lens;
  const RowInfo ri = row_info(rule, b, 0);
  int64_t L = a.kv_lens ? static_cast<int64_t>(a.kv_lens[b]) : a.kv_len;
  L = L < 1 ? 1 : (L > a.kv_len ? a.kv_len : L);
  int m = a.k_total - ri.nforced;
  m = m < 0 ? 0 : m;
  // ---- merge the parts' candidates (already in block-id order) ----
  const int total = a.parts * a.mpad;
  int* sel = reinterpret_cast<int*>(dyn);  // [k_total]
  uint32_t* bk0 = reinterpret_cast<uint32_t*>(sel + a.k_total);
  const int cap = ((total + kSel - 1) / kSel) * (m > 0 ? m : 1);
  int32_t* bi0 = reinterpret_cast<int32_t*>(bk0 + cap);
  uint32_t* bk1 = reinterpret_cast<uint32_t*>(bi0 + cap);
  int32_t* bi1 = reinterpret_cast<int32_t*>(bk1 + cap);
  uint32_t* fk = reinterpret_cast<uint32_t*>(bi1 + cap);
  int32_t* fi = reinterpret_cast<int32_t*>(fk + a.mpad);
  const uint32_t* ck = a.cand_key + static_cast<int64_t>(row) * total;
  const int32_t* ci = a.cand_id + static_cast<int64_t>(row) * total;
  const int nr = tournament<kNT>(
      total, m,
      [&](int i, uint32_t& key, int32_t& id, bool& valid) {
        id = i < total ? ci[i] : -1;
        valid = id >= 0;
        key = valid ? ck[i] : 0u;
      },
      bk0, bi0, bk1, bi1, fk, fi, a.mpad);
  if (tid == 0) {
    // ascending: block 0 when forced first, the routed ids (all between),
    // then the row's own block when forced (f0 <= f1 and both bracket the
    // candidates, which lie strictly between them)
    int c = 0;
    const bool lead = ri.f0 == 0 && (a.force & 2u);
    if (lead) sel[c++] = 0;
    for (int q = 0; q < nr; ++q) sel[c++] = fi[q];
    if (!lead && ri.f0 >= 0) sel[c++] = ri.f0;
    if (ri.f1 >= 0) sel[c++] = ri.f1;
    sel_n = c;
  }
  __syncthreads();
  const int nsel = sel_n;
  if (a.idx != nullptr && p == 0) {
    int32_t* gidx = a.idx + static_cast<int64_t>(row) * a.k_total;
    for (int q = tid; q < a.k_total; q += kNT) gidx[q] = q < nsel ? sel[q] : -1;
    if (tid == 0) a.cnt[row] = nsel;
  }
  if (!a.attend) return;

  // ---- attention over this part's share of the selected blocks ----
  const float scl = a.sm_scale * kLog2e;
  for (int e = tid; e < G * D; e += kNT) {
    const int hh = e / D, c = e % D;
    const T* qp = static_cast<const T*>(a.Q) + b * a.qs.b + (g * G + hh) * a.qs.h;
    float v;
    if constexpr (sizeof(T) == 2)
      v = bf16_to_f32(qp[c]);
    else
      v = qp[c];
    qa[hh][c] = v * scl;
  }
  __syncthreads();
  const int s0 = (nsel * p) / a.parts, s1 = (nsel * (p + 1)) / a.parts;
  const int cpb = a.B / CK;
  const int nchunk = (s1 - s0) * cpb;
  // paged: the selected blocks' pages, over the (finished) tournament buffers
  int* pgs = reinterpret_cast<int*>(bk0);
  if constexpr (PAGED) {
    for (int q = tid; q < nsel; q += kNT) {
      const int j = sel[q];
      const int pg = (j >= 0 && j < a.nblk && j < a.max_pages)
                         ? a.table[static_cast<int64_t>(b) * a.max_pages + j] : -1;
      pgs[q] = pg >= 0 && pg < a.num_pages ? pg : -1;
    }
    __syncthreads();
  }
  const auto rk = make_rsrc(static_cast<const T*>(a.K) + b * a.ks.b + g * a.ks.h,
                            head_bytes(L, a.ks.t, D, sizeof(T)));
  const auto rv = make_rsrc(static_cast<const T*>(a.V) + b * a.vs.b + g * a.vs.h,
                            head_bytes(L, a.vs.t, D, sizeof(T)));
  const uint32_t kst = static_cast<uint32_t>(a.ks.t * sizeof(T));
  const uint32_t vst = static_cast<uint32_t>(a.vs.t * sizeof(T));
  const int c8 = lane % LPK, kg = lane / LPK;
  float mm[GS], l[GS], o[GS][8];
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    mm[hh] = -INFINITY;
    l[hh] = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[hh][e] = 0.f;
  }
  auto chunk_t0 = [&](int ch) -> int {
    if (ch >= nchunk) return -1;
    const int j = sel[s0 + ch / cpb];
    return (j >= 0 && j < a.nblk) ? j * a.B + (ch % cpb) * CK : -1;
  };
  auto issue = [&](int ch, uint4 (&kb)[KPC][RPL], uint4 (&vb)[KPC][RPL]) {
    int t0 = chunk_t0(ch);
    auto rkc = rk, rvc = rv;
    if constexpr (PAGED) {
      // the chunk's page (wave-uniform): rows [0, L - jB) of it are valid
      const int pg = t0 < 0 ? -1 : __builtin_amdgcn_readfirstlane(pgs[s0 + ch / cpb]);
      const int j = t0 < 0 ? 0 : t0 / a.B;
      const int64_t rows = pg < 0 ? 0 : (L - static_cast<int64_t>(j) * a.B < a.B
                                             ? L - static_cast<int64_t>(j) * a.B : a.B);
      const int64_t pgo = pg < 0 ? 0 : pg;
      rkc = make_rsrc(static_cast<const T*>(a.K) + pgo * a.page_k + g * a.ks.h,
                      head_bytes(rows, a.ks.t, D, sizeof(T)));
      rvc = make_rsrc(static_cast<const T*>(a.V) + pgo * a.page_v + g * a.vs.h,
                      head_bytes(rows, a.vs.t, D, sizeof(T)));
      if (pg < 0) t0 = -1;
      else t0 -= j * a.B;  // page-relative
    }
#pragma unroll
    for (int it = 0; it < KPC; ++it) {
      const uint32_t t = static_cast<uint32_t>(t0 + it * KPI + kg);
      const uint32_t ko = t0 < 0 ? 0xFFFFFF00u : t * kst + c8 * 8 * sizeof(T);
      const uint32_t vo = t0 < 0 ? 0xFFFFFF00u : t * vst + c8 * 8 * sizeof(T);
#pragma unroll
      for (int r = 0; r < RPL; ++r) {
        kb[it][r] = buf_load16(rkc, ko + 16 * r);
        vb[it][r] = buf_load16(rvc, vo + 16 * r);
      }
    }
  };
  auto unpack = [&](const uint4 (&u)[RPL], float (&x)[8]) {
    if constexpr (sizeof(T) == 2) {
      x[0] = bf16_lo(u[0].x); x[1] = bf16_hi(u[0].x);
      x[2] = bf16_lo(u[0].y); x[3] = bf16_hi(u[0].y);
      x[4] = bf16_lo(u[0].z); x[5] = bf16_hi(u[0].z);
      x[6] = bf16_lo(u[0].w); x[7] = bf16_hi(u[0].w);
    } else {
      x[0] = __uint_as_float(u[0].x); x[1] = __uint_as_float(u[0].y);
      x[2] = __uint_as_float(u[0].z); x[3] = __uint_as_float(u[0].w);
      x[4] = __uint_as_float(u[RPL - 1].x); x[5] = __uint_as_float(u[RPL - 1].y);
      x[6] = __uint_as_float(u[RPL - 1].z); x[7] = __uint_as_float(u[RPL - 1].w);
    }
  };
  auto compute = [&](int ch, const uint4 (&kb)[KPC][RPL], const uint4 (&vb)[KPC][RPL]) {
    const int t0 = chunk_t0(ch);
    if (t0 < 0) return;
    bool ok[KPC];
#pragma unroll
    for (int it = 0; it < KPC; ++it) ok[it] = t0 + it * KPI + kg < L;
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      if (hh >= G) break;
      float s[KPC];
      float mx = -INFINITY;
#pragma unroll
      for (int it = 0; it < KPC; ++it) {
        float kv[8];
        unpack(kb[it], kv);
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(kv[e], qa[hh][c8 * 8 + e], acc);
        acc = lane_sum<LPK>(acc);
        s[it] = ok[it] ? acc : -INFINITY;
        mx = fmaxf(mx, s[it]);
      }
      if constexpr (LPK == 8) mx = fmaxf(mx, __shfl_xor(mx, 8, kWave));
      mx = swap32_max(swap16_max(mx));
      const float mn = fmaxf(mm[hh], mx);
      const float base = mn == -INFINITY ? 0.f : mn;
      const float f = __builtin_amdgcn_exp2f(mm[hh] - base);
      mm[hh] = mn;
      float ls = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) o[hh][e] *= f;
#pragma unroll
      for (int it = 0; it < KPC; ++it) {
        const float pw = __builtin_amdgcn_exp2f(s[it] - base);
        float vv[8];
        unpack(vb[it], vv);
        ls += pw;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(pw, vv[e], o[hh][e]);
      }
      l[hh] = l[hh] * f + ls;
    }
  };
  {
    uint4 ka[KPC][RPL], va2[KPC][RPL], kb2[KPC][RPL], vb2[KPC][RPL];
    if (w < nchunk) issue(w, ka, va2);
    for (int ch = w; ch < nchunk; ch += 2 * kNW) {
      issue(ch + kNW, kb2, vb2);
      compute(ch, ka, va2);
      if (ch + kNW >= nchunk) break;
      issue(ch + 2 * kNW, ka, va2);
      compute(ch + kNW, kb2, vb2);
    }
  }
  // merge the waves in LDS (reusing the candidate area), then publish the
  // workgroup's partial state
  float* merge = reinterpret_cast<float*>(fi + a.mpad);
#pragma unroll
  for (int hh = 0; hh < GS; ++hh) {
    if (hh >= G) break;
    float lt = l[hh];
    if constexpr (LPK == 8) lt += __shfl_xor(lt, 8, kWave);
    lt = swap32_sum(swap16_sum(lt));
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      float v = o[hh][e];
      if constexpr (LPK == 8) v += __shfl_xor(v, 8, kWave);
      v = swap32_sum(swap16_sum(v));
      if (kg == 0) merge[(w * GS + hh) * PART + 2 + c8 * 8 + e] = v;
    }
    if (lane == 0) {
      merge[(w * GS + hh) * PART + 0] = mm[hh];
      merge[(w * GS + hh) * PART + 1] = lt;
    }
  }
  __syncthreads();
  float* mypart = a.part + (static_cast<int64_t>(row) * a.parts + p) * G * PART;
  for (int e = tid; e < G * PART; e += kNT) {
    const int hh = e / PART, c = e % PART;
    float M = -INFINITY;
    for (int ww = 0; ww < kNW; ++ww) M = fmaxf(M, merge[(ww * GS + hh) * PART]);
    float v;
    if (c == 0) {
      v = M;
    } else {
      const float base = M == -INFINITY ? 0.f : M;
      v = 0.f;
      for (int ww = 0; ww < kNW; ++ww) {
        const float* pp = merge + (ww * GS + hh) * PART;
        v += __builtin_amdgcn_exp2f(pp[0] - base) * pp[c];
      }
    }
    mypart[e] = v;
  }
}

// Merges the parts' partial softmax states of a row and writes O.  A kernel
// of its own: the stream order publishes the partial states across XCDs
// (the L2s of different XCDs are not coherent, and an agent-scope fence per
// workgroup would write back and invalidate a whole L2 each time).
__global__ __launch_bounds__(256) void decode_combine(DecodeArgs a) {
  constexpr int PART_PAD = 2;
  const int row = blockIdx.x;
  const int b = row / a.hkv, g = row % a.hkv;
  const int G = a.hq / a.hkv;
  const int part_w = a.d + PART_PAD;
  const float* rp = a.part + static_cast<int64_t>(row) * a.parts * G * part_w;
  for (int e = threadIdx.x; e < G * a.d; e += blockDim.x) {
    const int hh = e / a.d, c = e % a.d;
    float M = -INFINITY;
    for (int q = 0; q < a.parts; ++q) M = fmaxf(M, rp[(q * G + hh) * part_w]);
    const float base = M == -INFINITY ? 0.f : M;
    float ls = 0.f, acc = 0.f;
    for (int q = 0; q < a.parts; ++q) {
      const float* pp = rp + (q * G + hh) * part_w;
      const float f = __builtin_amdgcn_exp2f(pp[0] - base);
      ls += f * pp[1];
      acc += f * pp[2 + c];
    }
    const float v = ls > 0.f ? acc / ls : 0.f;
    const int64_t off = b * a.os.b + (g * G + hh) * a.os.h + c;
    if (a.out_f32)
      static_cast<float*>(a.O)[off] = v;
    else
      static_cast<uint16_t*>(a.O)[off] = f32_to_bf16(v);
  }
}

template <typename T, int D, int GS, bool PAGED>
hipError_t launch_attend_part_p(const DecodeArgs& a, size_t dyn, hipStream_t stream) {
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(
        reinterpret_cast<const void*>(&decode_attend_part<T, D, GS, PAGED>),
        hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * (a.attend ? a.parts : 1);
  hipLaunchKernelGGL((decode_attend_part<T, D, GS, PAGED>), dim3(grid), dim3(kNT), dyn, stream, a);
  return hipGetLastError();
}

template <typename T, int D, int GS>
hipError_t launch_attend_part(const DecodeArgs& a, size_t dyn, hipStream_t stream) {
  hipError_t e = a.table ? launch_attend_part_p<T, D, GS, true>(a, dyn, stream)
                         : launch_attend_part_p<T, D, GS, false>(a, dyn, stream);
  if (e != hipSuccess || !a.attend) return e;
  hipLaunchKernelGGL(decode_combine, dim3(a.batch * a.hkv), dim3(256), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_attend_part_t(const DecodeArgs& a, size_t dyn, hipStream_t stream) {
  const int G = a.hq / a.hkv;
  if (G <= 1) return launch_attend_part<T, D, 1>(a, dyn, stream);
  if (G <= 2) return launch_attend_part<T, D, 2>(a, dyn, stream);
  if (G <= 4) return launch_attend_part<T, D, 4>(a, dyn, stream);
  return launch_attend_part<T, D, 8>(a, dyn, stream);
}

}  // namespace

hipError_t launch_decode_parts(const DecodeArgs& a, hipStream_t stream) {
  const int rows = a.batch * a.hkv;
  int m = a.k_total;  // upper bound of the routed count
  // routing kernel LDS: partition scores + two tournament ping-pong buffers
  const int per = (a.nblk + a.parts - 1) / a.parts;
  const int cap1 = ((per + kSel - 1) / kSel) * m;
  const size_t dyn1 = static_cast<size_t>(per) * 4 + static_cast<size_t>(cap1) * 16;
  static bool attr = false;
  if (!attr) {
    hipError_t e;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_route_part<64>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024)) != hipSuccess)
      return e;
    if ((e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_route_part<128>),
                                 hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024)) != hipSuccess)
      return e;
    attr = true;
  }
  DecodeArgs r = a;
  r.lds_floats = per;
  const unsigned grid1 = static_cast<unsigned>(rows) * a.parts;
  if (a.d == 64)
    hipLaunchKernelGGL(decode_route_part<64>, dim3(grid1), dim3(kNT), dyn1, stream, r);
  else
    hipLaunchKernelGGL(decode_route_part<128>, dim3(grid1), dim3(kNT), dyn1, stream, r);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int G = a.hq / a.hkv;
  const int gs = G <= 1 ? 1 : G <= 2 ? 2 : G <= 4 ? 4 : 8;
  const int total = a.parts * a.mpad;
  const int cap2 = ((total + kSel - 1) / kSel) * (m > 0 ? m : 1);
  size_t dyn2 = static_cast<size_t>(a.k_total) * 4 + static_cast<size_t>(cap2) * 16 +
                static_cast<size_t>(a.mpad) * 8;
  dyn2 += static_cast<size_t>(kNW) * gs * (a.d + 2) * 4;
  if (a.bf16)
    return a.d == 64 ? launch_attend_part_t<uint16_t, 64>(a, dyn2, stream)
                     : launch_attend_part_t<uint16_t, 128>(a, dyn2, stream);
  return a.d == 64 ? launch_attend_part_t<float, 64>(a, dyn2, stream)
                   : launch_attend_part_t<float, 128>(a, dyn2, stream);
}

}  // namespace bsa
