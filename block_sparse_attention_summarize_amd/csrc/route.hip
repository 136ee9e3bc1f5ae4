// Stage 1: block routing.
//
//   scores_tiled    coarse scores of every candidate block against the row's
//   scores_kernel   routing query ("DashAttention", Declaração do Problema:
//                   coarse attention scores between queries and block
//                   summaries).  fp32 throughout: selections must agree with
//                   an fp64 reference whenever the k-th/(k+1)-th gap exceeds
//                   1e-4, so no reduced-precision matrix cores here.  Prefill
//                   rows of one KV head share its summaries, so the scores are
//                   a small GEMM tiled 64 x 64 through LDS (scores_tiled);
//                   decode rows each have their own summaries and are a GEMV
//                   streamed from memory (scores_kernel).
//   select_kernel   top-k with forced blocks and the lower-index tie rule
//                   ("Gist Sparse Attention", section 2 item 3).  Exact radix
//                   select on order-preserving uint32 keys (4 passes of 8
//                   bits over an LDS histogram), then an ordered ballot scan
//                   that resolves ties toward lower block ids and writes the
//                   ascending list.
//   entmax_kernel   alpha-entmax support per query head ("DashAttention",
//                   Estágio 1) over logits produced by the scores kernels,
//                   with the threshold bracketed by a 16-bin LDS histogram
//                   and refined by bisection ("AdaSplash-2", 2.A),
//                   GQA-averaged probabilities, cap by the same radix select.
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace bsa {

namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kChunk = 128;  // candidate blocks scored per workgroup

// ---------------------------------------------------------------------------
// Decode scores (one row per (b, g), its own summaries).  d/4 lanes share one
// summary row (a float4 each); the dot is finished with a butterfly over those
// lanes.
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kThreads) void scores_kernel(ScoreArgs a) {
  constexpr int LPR = D / 4;           // lanes per summary row
  constexpr int RPW = kWave / LPR;     // rows per wave step
  const int nchunk = (a.nblk + kChunk - 1) / kChunk;
  const int chunk = blockIdx.x % nchunk;
  const int rowid = blockIdx.x / nchunk;  // (b, q-hat head, row)
  const int row = rowid % a.nrow;
  const int bh = rowid / a.nrow;
  const int b = bh / a.qheads;
  const int bg = b * a.hkv + (bh % a.qheads) / a.group;
  const RowInfo ri = row_info(a.rule, b, row);
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int c = lane % LPR;
  const float4 q = reinterpret_cast<const float4*>(a.qhat + static_cast<int64_t>(rowid) * D)[c];
  const float* Sg = a.S + static_cast<int64_t>(bg) * a.nblk * D;
  float* out = a.scores + static_cast<int64_t>(rowid) * a.nblk;
  const int j0 = chunk * kChunk;
  for (int jj = w * RPW + lane / LPR; jj < kChunk; jj += kWaves * RPW) {
    const int j = j0 + jj;
    if (j >= a.nblk) break;
    float s = -INFINITY;
    if (j < ri.cand_end) {
      const float4 v = reinterpret_cast<const float4*>(Sg + static_cast<int64_t>(j) * D)[c];
      float p = q.x * v.x;
      p = fmaf(q.y, v.y, p);
      p = fmaf(q.z, v.z, p);
      p = fmaf(q.w, v.w, p);
      p = group_sum<LPR>(p);
      s = p * a.scale;
    }
    if (c == 0) out[j] = s;
  }
}

// ---------------------------------------------------------------------------
// Prefill and per-token scores: one workgroup per 64 rows x 64 blocks tile of
// one (b, q-hat head).  The q-hat and summary tiles are staged in LDS (rows
// padded by 4 floats; reads outside the rows present return zeros), and the
// tile runs on the fp32 matrix cores: wavefront w owns rows 16w..16w+15 as
// four 16 x 16 accumulators (v_mfma_f32_16x16x4_f32).
// Lane l reads 4 consecutive d of its row (A) and of its block (B) from LDS
// and feeds them to four MFMAs, so each MFMA's k-slice is {c, c+4, c+8, c+12}
// of a 16-wide d chunk: the dot products run over every d exactly once, in
// fp32 products and fp32 accumulation as on the VALU.  Unless `fill`, tiles
// right of every row's candidates (the candidate end grows with the row) are
// not written at all (their readers only look at the candidates).  A
// workgroup takes `jgroup` consecutive block tiles of its row tile: the rows'
// fragments are read from LDS into registers once and only the summaries are
// staged per block tile (many rows, as with per-token routing, re-read them
// far less often), the next tile's loads in flight in registers while the
// current tile's products run, then stored to the other of two LDS buffers.
// ---------------------------------------------------------------------------
constexpr int kTile = 64;
constexpr int kPad = 4;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int D>
__global__ __launch_bounds__(kThreads) void scores_mfma(ScoreArgs a, int fill, int jgroup) {
  // two staging buffers: the row tile is staged in buf[1] once and read into
  // registers, after which buf[1] takes every other block tile
  __shared__ float buf[2][kTile][D + kPad];
  const int nrt = (a.nrow + kTile - 1) / kTile;
  const int njt = (a.nblk + kTile - 1) / kTile;
  const int ngt = (njt + jgroup - 1) / jgroup;
  int id = blockIdx.x;
  const int gt = id % ngt;
  id /= ngt;
  const int rt = id % nrt;
  const int bh = id / nrt;  // (b, q-hat head)
  const int b = bh / a.qheads;
  const int sg_row = b * a.hkv + (bh % a.qheads) / a.group;
  const int r0 = rt * kTile;
  const int rn = a.nrow - r0 < kTile ? a.nrow - r0 : kTile;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int ce = a.rule.entmax ? 0 : 1;
  const int tok_b = a.rule.mode == 2 ? a.rule.B : 1;
  const int jend = (r0 + rn - 1) / tok_b + ce;  // blocks past every row's candidates
  constexpr int V4 = D / 4;
  constexpr int KC = D / 16;
  constexpr int PF = kTile * V4 / kThreads;  // 16-byte loads per thread and tile
  static_assert(PF * kThreads == kTile * V4, "tile split over the threads");
  const int lr = lane & 15, lk = (lane >> 4) * 4;
  // the workgroup's block tiles: [jt0, jtc) hold candidates, [jtc, jt1) do not
  const int jt0 = gt * jgroup;
  const int jt1 = njt < (gt + 1) * jgroup ? njt : (gt + 1) * jgroup;
  const int jtlast = (jend + kTile - 1) / kTile;  // first tile with no candidate
  const int jtc = jt1 < jtlast ? jt1 : jtlast;
  uint4 pre[PF];
  // summaries of block tile jt into registers (rows past n_blk read as zero)
  auto fetch = [&](int jt) {
    const int j0 = jt * kTile;
    const int jn = a.nblk - j0 < kTile ? a.nblk - j0 : kTile;
    const auto rs = make_rsrc(a.S + (static_cast<int64_t>(sg_row) * a.nblk + j0) * D,
                              static_cast<uint32_t>(jn) * D * 4);
#pragma unroll
    for (int i = 0; i < PF; ++i) pre[i] = buf_load16(rs, static_cast<uint32_t>(tid + i * kThreads) * 16);
  };
  auto put = [&](int k) {
#pragma unroll
    for (int i = 0; i < PF; ++i) {
      const int e = tid + i * kThreads, r = e / V4, c = e % V4;
      *reinterpret_cast<uint4*>(&buf[k][r][c * 4]) = pre[i];
    }
  };
  if (jt0 < jtc) {
    {
      const float* qg = a.qhat + (static_cast<int64_t>(bh) * a.nrow + r0) * D;
      const auto rq = make_rsrc(qg, static_cast<uint32_t>(rn) * D * 4);
      uint4 qv[PF];
#pragma unroll
      for (int i = 0; i < PF; ++i) qv[i] = buf_load16(rq, static_cast<uint32_t>(tid + i * kThreads) * 16);
      fetch(jt0);
#pragma unroll
      for (int i = 0; i < PF; ++i) {
        const int e = tid + i * kThreads, r = e / V4, c = e % V4;
        *reinterpret_cast<uint4*>(&buf[1][r][c * 4]) = qv[i];
      }
      put(0);
    }
    __syncthreads();
    float4 av[KC];  // this lane's row fragments, read once
#pragma unroll
    for (int k = 0; k < KC; ++k) av[k] = *reinterpret_cast<const float4*>(&buf[1][16 * w + lr][16 * k + lk]);
    __syncthreads();  // buf[1] is free for the second block tile
    for (int jt = jt0; jt < jtc; ++jt) {
      const int cur = (jt - jt0) & 1;
      const bool more = jt + 1 < jtc;
      if (more) fetch(jt + 1);  // in flight during this tile's products
      const int j0 = jt * kTile;
      const int jn = a.nblk - j0 < kTile ? a.nblk - j0 : kTile;
      float* out = a.scores + (static_cast<int64_t>(bh) * a.nrow + r0) * a.nblk + j0;
      f32x4_t acc[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int k = 0; k < KC; ++k) {
        float4 bv[4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) bv[ct] = *reinterpret_cast<const float4*>(&buf[cur][16 * ct + lr][16 * k + lk]);
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[k].x, bv[ct].x, acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[k].y, bv[ct].y, acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[k].z, bv[ct].z, acc[ct], 0, 0, 0);
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av[k].w, bv[ct].w, acc[ct], 0, 0, 0);
        }
      }
      // the next tile into the other buffer (last read before the previous
      // barrier), ahead of this tile's stores so that the wait for its loads
      // does not also wait for them
      if (more) put(cur ^ 1);
      // lane l holds rows 16w + 4(l/16) + i, block 16ct + l%16
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = 16 * w + (lane >> 4) * 4 + i;
        const int cend = (r0 + r) / tok_b + ce - j0;
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int j = 16 * ct + lr;
          if (r < rn && j < jn)
            out[static_cast<int64_t>(r) * a.nblk + j] = j < cend ? acc[ct][i] * a.scale : -INFINITY;
        }
      }
      __syncthreads();
    }
  }
  if (!fill) return;
  // right of the last row's candidates
  for (int jt = jtc > jt0 ? jtc : jt0; jt < jt1; ++jt) {
    const int j0 = jt * kTile;
    const int jn = a.nblk - j0 < kTile ? a.nblk - j0 : kTile;
    float* out = a.scores + (static_cast<int64_t>(bh) * a.nrow + r0) * a.nblk + j0;
    for (int e = tid; e < kTile * kTile; e += kThreads) {
      const int r = e / kTile, j = e % kTile;
      if (r < rn && j < jn) out[static_cast<int64_t>(r) * a.nblk + j] = -INFINITY;
    }
  }
}

// ---------------------------------------------------------------------------
// Top-k select, one workgroup per row.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void select_kernel(SelectArgs a) {
  __shared__ int hist[256];
  __shared__ int bcast[2];
  __shared__ int wave_tot[kWaves];
  const int rowid = blockIdx.x;
  const int row = rowid % a.nrow;
  const int b = rowid / (a.nrow * a.hkv);
  const RowInfo ri = row_info(a.rule, b, row);
  const float* sc = a.scores + static_cast<int64_t>(rowid) * a.nblk;
  const int n_elig = ri.cand_end - ri.nforced_below(ri.cand_end);
  int m = a.k_total - ri.nforced;
  m = m < 0 ? 0 : m;
  auto get = [&](int e, uint32_t& key) -> bool {
    if (e >= ri.cand_end || is_forced(ri, e)) return false;
    key = float_key(sc[e]);
    return true;
  };
  int32_t* idx = a.idx + static_cast<int64_t>(rowid) * a.k_total;
  const int c = select_and_write<kThreads>(
      ri, ri.span, m, n_elig, get, [&](int p, int e) { idx[p] = e; }, a.k_total, hist, bcast,
      wave_tot);
  if (threadIdx.x == 0) a.cnt[rowid] = c;
}

// ---------------------------------------------------------------------------
// alpha-entmax routing, one workgroup per (b, g, row); wave w handles the
// query heads w, w+4, ... of the group.  The logits of each head live in the
// workspace row xbuf[head][0:nblk] (L1/L2 resident across the passes).
// ---------------------------------------------------------------------------

// [x - t]_+^(1/(alpha-1))
__device__ __forceinline__ float emass(float x, float t, float alpha) {
  const float d = x - t;
  if (!(d > 0.f)) return 0.f;
  if (alpha == 1.5f) return d * d;
  if (alpha == 2.f) return d;
  return powf(d, 1.f / (alpha - 1.f));
}

// [x - t]_+^(1/(alpha-1)) in fp64 (the bracket and bisection state)
__device__ __forceinline__ double emass_d(double x, double t, double alpha) {
  const double d = x - t;
  if (!(d > 0.0)) return 0.0;
  if (alpha == 1.5) return d * d;
  if (alpha == 2.0) return d;
  return pow(d, 1.0 / (alpha - 1.0));
}

// Root of sum_k c_k [e_k - tau]_+^(1/(alpha-1)) = 1 for the 16 bin values
// e_k = xm - (k + off) / 16 (descending) with counts c_k (in LDS): sort-based
// closed forms for alpha in {1.5, 2}, 64 bisection steps on [e_0 - 1, e_0]
// otherwise.  fp64: the closed forms cancel (1 - Q) when few bins are in the
// support.
struct BinVals {
  double xm;
  int off;
  __device__ double operator[](int k) const { return xm - static_cast<double>(k + off) * 0.0625; }
};
__device__ inline double solve_bins(const BinVals& e, const int* c, double alpha) {
  if (alpha == 2.0 || alpha == 1.5) {
    double n = 0.0, s1 = 0.0;
    for (int r = 0; r < 16; ++r) {
      if (c[r] == 0) continue;
      const double cr = static_cast<double>(c[r]);
      n += cr;
      s1 += cr * e[r];
      double tau;
      if (alpha == 2.0) {
        tau = (s1 - 1.0) / n;
      } else {
        const double M = s1 / n;
        double Q = 0.0;  // squared deviations, recomputed for accuracy
        for (int k = 0; k <= r; ++k) {
          const double dv = e[k] - M;
          Q += static_cast<double>(c[k]) * dv * dv;
        }
        if (Q > 1.0) continue;
        tau = M - sqrt((1.0 - Q) / n);
      }
      int nx = r + 1;
      while (nx < 16 && c[nx] == 0) ++nx;
      if (tau < e[r] && (nx >= 16 || tau >= e[nx])) return tau;
    }
  }
  double lo = e[0] - 1.0, hi = e[0];
  for (int it = 0; it < 64; ++it) {
    const double mid = 0.5 * (lo + hi);
    double f = 0.0;
    for (int r = 0; r < 16; ++r) f += static_cast<double>(c[r]) * emass_d(e[r], mid, alpha);
    if (f >= 1.0)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

// IN_LDS: the group's logit rows are copied once into LDS (G * nblk floats of
// dynamic LDS) and every pass runs there; otherwise the passes read the
// workspace rows in place.
template <bool IN_LDS>
__global__ __launch_bounds__(kThreads) void entmax_kernel(EntmaxArgs a) {
  extern __shared__ float xsh[];
  __shared__ int hist[256];
  __shared__ int bcast[2];
  __shared__ int wave_tot[kWaves];
  __shared__ int bins[kWaves][16];
  const int G = a.hq / a.hkv;
  const int rowid = blockIdx.x;  // (b, g, row)
  const int row = rowid % a.nrow;
  const int bg = rowid / a.nrow;
  const int g = bg % a.hkv;
  const int b = bg / a.hkv;
  const RowInfo ri = row_info(a.rule, b, row);
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int n = ri.cand_end;  // candidate range; forced ids inside are excluded
  // logits of head g*G + hh of this row, from the scores kernel
  auto grow_of = [&](int hh) {
    return a.xbuf + ((static_cast<int64_t>(b) * a.hq + g * G + hh) * a.nrow + row) * a.nblk;
  };
  auto xrow_of = [&](int hh) {
    return IN_LDS ? xsh + static_cast<int64_t>(hh) * a.nblk : grow_of(hh);
  };
  const float alpha = a.alpha;
  if constexpr (IN_LDS) {
    for (int hh = 0; hh < G; ++hh) {
      const float* src = grow_of(hh);
      for (int j = threadIdx.x; j < n; j += kThreads)
        xsh[hh * a.nblk + j] = is_forced(ri, j) ? -INFINITY : src[j];
    }
    __syncthreads();
  }

  for (int hh = w; hh < G; hh += kWaves) {
    const int h = g * G + hh;
    const int64_t hrow = (static_cast<int64_t>(b) * a.hq + h) * a.nrow + row;
    float* x = xrow_of(hh);
    // forced blocks inside the candidate range take no part in the entmax
    if (!IN_LDS && lane == 0) {
      if (ri.f0 >= 0 && ri.f0 < n) x[ri.f0] = -INFINITY;
      if (ri.f1 >= 0 && ri.f1 < n) x[ri.f1] = -INFINITY;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
    __builtin_amdgcn_wave_barrier();
    // number of eligible candidates and the maximum
    float xmax = -INFINITY;
    int ne = 0;
    for (int j = lane; j < n; j += kWave) {
      const float v = x[j];
      if (v != -INFINITY) {
        xmax = fmaxf(xmax, v);
        ++ne;
      }
    }
    xmax = wave_max(xmax);
    ne = wave_sum_i(ne);
    float tau = __builtin_nanf("");
    if (ne > 0) {
      // 16-bin histogram of u = xmax - x on [0, 1)
      if (lane < 16) bins[w][lane] = 0;
      __builtin_amdgcn_wave_barrier();
      for (int j = lane; j < n; j += kWave) {
        const float v = x[j];
        if (v == -INFINITY) continue;
        const float u = xmax - v;
        if (u < 1.f) {
          int bin = static_cast<int>(floorf(u * 16.f));
          bin = bin > 15 ? 15 : bin;
          atomicAdd(&bins[w][bin], 1);
        }
      }
      __builtin_amdgcn_wave_barrier();
      const double ad = alpha, xm = xmax;
      // lower bin edges bound tau from below, upper edges from above
      const double tau_lo = solve_bins(BinVals{xm, 1}, bins[w], ad);
      const double tau_hi = solve_bins(BinVals{xm, 0}, bins[w], ad);
      // bracket and bisection in fp64, like the threshold they converge to
      double lo = fmax(tau_lo, xm - 1.0);
      double hi = fmin(tau_hi, xm - pow(static_cast<double>(ne), 1.0 - ad));
      bool resolved = false;
      for (int it = 0;; ++it) {
        int inside = 0;
        for (int j = lane; j < n; j += kWave) {
          const double v = x[j];
          inside |= (v > lo && v <= hi) ? 1 : 0;
        }
        if (__ballot(inside) == 0) {
          resolved = true;
          break;
        }
        if (it >= a.max_iter) break;
        const double mid = 0.5 * (lo + hi);
        double f = 0.0;
        for (int j = lane; j < n; j += kWave) f += emass_d(x[j], mid, ad);
        f = wave_sum_d(f);
        if (f >= 1.0)
          lo = mid;
        else
          hi = mid;
      }
      tau = static_cast<float>(lo);
      if (resolved) {
        // exact threshold of the support {x > lo}.  The closed forms are
        // evaluated in fp64: for alpha = 1.5, 1 - Q cancels when the support
        // is small, and fp32 would lose digits that tau itself does not lose.
        double s1 = 0.0;
        int ns = 0;
        for (int j = lane; j < n; j += kWave) {
          const float v = x[j];
          if (v > lo) {
            s1 += v;
            ++ns;
          }
        }
        s1 = wave_sum_d(s1);
        ns = wave_sum_i(ns);
        const double nsd = static_cast<double>(ns);
        if (alpha == 2.f) {
          tau = static_cast<float>((s1 - 1.0) / nsd);
        } else if (alpha == 1.5f) {
          const double M = s1 / nsd;
          double Q = 0.0;
          for (int j = lane; j < n; j += kWave) {
            const double v = x[j];
            if (v > lo) Q += (v - M) * (v - M);
          }
          Q = wave_sum_d(Q);
          tau = static_cast<float>(M - sqrt(fmax((1.0 - Q) / nsd, 0.0)));
        } else {
          double l2 = lo, h2 = lo + 1.0;  // the root is below max x <= lo + 1
          for (int it = 0; it < 64; ++it) {
            const double mid = 0.5 * (l2 + h2);
            double f = 0.0;
            for (int j = lane; j < n; j += kWave) {
              const double v = x[j];
              if (v > lo) f += emass_d(v, mid, ad);
            }
            f = wave_sum_d(f);
            if (f >= 1.0)
              l2 = mid;
            else
              h2 = mid;
          }
          tau = static_cast<float>(0.5 * (l2 + h2));
        }
      }
      // probabilities, renormalised; stored over the logits
      float z = 0.f;
      for (int j = lane; j < n; j += kWave) z += emass(x[j], tau, alpha);
      z = wave_sum(z);
      const float iz = 1.f / z;
      for (int j = lane; j < n; j += kWave) x[j] = emass(x[j], tau, alpha) * iz;
    } else {
      for (int j = lane; j < n; j += kWave) x[j] = 0.f;
    }
    if (a.tau && lane == 0) a.tau[hrow] = tau;
    if (a.probs) {
      float* pr = a.probs + hrow * a.nblk;
      for (int j = lane; j < a.nblk; j += kWave) pr[j] = j < n ? x[j] : 0.f;
    }
  }
  __syncthreads();
  // GQA: mean probability over the group's heads; keep the positive ones,
  // capped (per-wave tournament below kSel, radix select otherwise).
  const float invG = 1.f / static_cast<float>(G);
  const int64_t hstride = IN_LDS ? a.nblk : static_cast<int64_t>(a.nrow) * a.nblk;  // between heads
  const float* xrow = xrow_of(0);
  auto wbar = [&](int e) {
    float s = 0.f;
    for (int hh = 0; hh < G; ++hh) s += xrow[static_cast<int64_t>(hh) * hstride + e];
    return s * invG;
  };
  int32_t* idx = a.idx + static_cast<int64_t>(rowid) * a.width;
  if (a.tourn) {
    // buffers after the logit rows (if those are in LDS)
    const int capb = ((n + kSel - 1) / kSel) * a.cap;
    uint32_t* bk0 = reinterpret_cast<uint32_t*>(xsh + (IN_LDS ? G * a.nblk : 0));
    int32_t* bi0 = reinterpret_cast<int32_t*>(bk0 + capb);
    uint32_t* bk1 = reinterpret_cast<uint32_t*>(bi0 + capb);
    int32_t* bi1 = reinterpret_cast<int32_t*>(bk1 + capb);
    uint32_t* fk = reinterpret_cast<uint32_t*>(bi1 + capb);
    int32_t* fi = reinterpret_cast<int32_t*>(fk + a.cap);
    const int nr = tournament<kThreads>(
        n, a.cap,
        [&](int i, uint32_t& key, int32_t& id, bool& valid) {
          float v = 0.f;
          valid = false;
          if (i < n && !is_forced(ri, i)) {
            v = wbar(i);
            valid = v > 0.f;
          }
          key = valid ? float_key(v) : 0u;
          id = i;
        },
        bk0, bi0, bk1, bi1, fk, fi, a.cap);
    // ascending: block 0 when forced first, the routed ids (strictly between
    // the forced ones), then the row's own block when forced
    const int lead = (ri.f0 == 0 && (a.rule.force & 2u)) ? 1 : 0;
    const int tail0 = (!lead && ri.f0 >= 0) ? ri.f0 : -1;
    const int total = lead + nr + (tail0 >= 0) + (ri.f1 >= 0);
    float* wsel = a.wsel ? a.wsel + static_cast<int64_t>(rowid) * a.width : nullptr;
    for (int p = threadIdx.x; p < a.width; p += kThreads) {
      int v = -1;
      float wv = 0.f;
      if (p < lead) {
        v = 0;
        wv = 1.f;
      } else if (p < lead + nr) {
        v = fi[p - lead];
        wv = wsel ? wbar(v) : 0.f;
      } else if (p < total) {
        v = (p == lead + nr && tail0 >= 0) ? tail0 : ri.f1;
        wv = 1.f;
      }
      idx[p] = v;
      if (wsel) wsel[p] = wv;
    }
    if (threadIdx.x == 0) a.cnt[rowid] = total;
    return;
  }
  int npos = 0;
  for (int e = threadIdx.x; e < n; e += kThreads) npos += (!is_forced(ri, e) && wbar(e) > 0.f) ? 1 : 0;
  npos = wave_sum_i(npos);
  if (lane == 0) wave_tot[w] = npos;
  __syncthreads();
  int n_elig = 0;
#pragma unroll
  for (int k = 0; k < kWaves; ++k) n_elig += wave_tot[k];
  __syncthreads();
  auto get = [&](int e, uint32_t& key) -> bool {
    if (e >= n || is_forced(ri, e)) return false;
    const float v = wbar(e);
    if (!(v > 0.f)) return false;
    key = float_key(v);
    return true;
  };
  float* wsel = a.wsel ? a.wsel + static_cast<int64_t>(rowid) * a.width : nullptr;
  const int c = select_and_write<kThreads>(
      ri, ri.span, a.cap, n_elig, get,
      [&](int p, int e) {
        idx[p] = e;
        if (wsel) wsel[p] = e < 0 ? 0.f : (is_forced(ri, e) ? 1.f : wbar(e));
      },
      a.width, hist, bcast, wave_tot);
  if (threadIdx.x == 0) a.cnt[rowid] = c;
}

// ---------------------------------------------------------------------------
// alpha-entmax routing of short rows (<= 64 E candidates), one wavefront per
// (b, g, row) and four rows per workgroup with no barrier between them: the
// many short rows of per-token routing.  The wave keeps a head's logits in
// registers (element e of lane l is block e*64 + l), runs the same histogram
// bracket, bisection and exact threshold as entmax_kernel head by head,
// accumulates the group's probabilities and takes the capped support with a
// register top-m.
// ---------------------------------------------------------------------------

__device__ __forceinline__ double readlane_d(double v, int l) {
  const uint2 u = __builtin_bit_cast(uint2, v);
  return __builtin_bit_cast(double, make_uint2(__builtin_amdgcn_readlane(u.x, l),
                                               __builtin_amdgcn_readlane(u.y, l)));
}

// Sum over the 16 lanes of each row (DPP within the row), for a double.
__device__ __forceinline__ double row16_sum_d(double v) {
  v += dppd<0xB1>(v);
  v += dppd<0x4E>(v);
  v += dppd<0x141>(v);
  v += dppd<0x140>(v);
  return v;
}
// Inclusive prefix sum over the 16 lanes of each row (DPP row shifts; lanes
// shifted in from outside the row read 0).
__device__ __forceinline__ int row16_scan_i(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, true);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, true);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, true);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, true);  // row_shr:8
  return v;
}

// Both histogram bounds of tau (the roots of the binned equation with every
// bin's mass at its lower and at its upper edge, as solve_bins), relative to
// xm, in one pass: lanes 0-15 hold bin r = lane with value -(r+1)/16, lanes
// 16-31 bin r = lane-16 with value -r/16, and lane r of each row tries the
// closed form of the prefix of bins 0..r.  The counts and the first and
// second moments of the bin offsets are integers, so the prefix moments and
// the variance numerator are exact.  `cl` is the count of bin lane & 15 on
// lanes < 32.  Other alpha, or no valid prefix: 64 bisection steps on
// [e_0 - 1, e_0] per row.  Returns (lower bound, upper bound).
__device__ inline double2 bin_bounds(int cl, double alpha) {
  const int lane = lane_id();
  const int r = lane & 15;
  const int off = lane < 16 ? 1 : 0;
  const bool act = lane < 32;
  const int c = act ? cl : 0;
  const int kk = r + off;  // bin value -kk/16
  const uint64_t nz = __ballot(act && c > 0);
  double tau = 0.0;
  bool ok = false;
  if (alpha == 2.0 || alpha == 1.5) {
    const int n = row16_scan_i(c);
    const int b1 = row16_scan_i(c * kk);
    const int a2 = row16_scan_i(c * kk * kk);
    const double nd = static_cast<double>(n);
    const double s1 = -static_cast<double>(b1) * 0.0625;  // sum of c e
    ok = act && c > 0;
    if (alpha == 2.0) {
      tau = (s1 - 1.0) / nd;
    } else {
      // sum c (e - M)^2 = (n a2 - b1^2) / (256 n), exact numerator
      const int64_t num = static_cast<int64_t>(n) * a2 - static_cast<int64_t>(b1) * b1;
      const double Q = static_cast<double>(num) / (256.0 * nd);
      ok = ok && !(Q > 1.0);
      tau = s1 / nd - sqrt(fmax((1.0 - Q) / nd, 0.0));
    }
    const uint64_t rowbits = (nz >> (lane & 48)) & 0xFFFFull;
    const uint64_t above = rowbits >> (r + 1);
    const int nx = above ? r + 1 + __builtin_ctzll(above) : 16;
    ok = ok && tau < -static_cast<double>(kk) * 0.0625 &&
         (nx >= 16 || tau >= -static_cast<double>(nx + off) * 0.0625);
  }
  const uint64_t vm = __ballot(ok);
  const uint32_t mlo = static_cast<uint32_t>(vm & 0xFFFFull);
  const uint32_t mhi = static_cast<uint32_t>((vm >> 16) & 0xFFFFull);
  double2 out;
  if (mlo && mhi) {
    out.x = readlane_d(tau, __builtin_ctz(mlo));
    out.y = readlane_d(tau, 16 + __builtin_ctz(mhi));
    return out;
  }
  double lo = -static_cast<double>(off) * 0.0625 - 1.0, hi = -static_cast<double>(off) * 0.0625;
  for (int it = 0; it < 64; ++it) {
    const double mid = 0.5 * (lo + hi);
    double f = act ? static_cast<double>(c) * emass_d(-static_cast<double>(kk) * 0.0625, mid, alpha)
                   : 0.0;
    f = row16_sum_d(f);
    if (f >= 1.0)
      lo = mid;
    else
      hi = mid;
  }
  const double t = 0.5 * (lo + hi);
  out.x = mlo ? readlane_d(tau, __builtin_ctz(mlo)) : readlane_d(t, 0);
  out.y = mhi ? readlane_d(tau, 16 + __builtin_ctz(mhi)) : readlane_d(t, 16);
  return out;
}

// Threshold of one head's logits held K per lane (-inf: not a candidate):
// bisection on [lo, hi] in fp64 until no logit lies inside the bracket (at
// most max_iter steps), then the exact threshold of the resolved support, or
// the bracket's lower end when unresolved.
template <int K>
__device__ inline float entmax_tau(const float (&x)[K], double lo, double hi, float alpha,
                                   int max_iter) {
  const double ad = alpha;
  bool resolved = false;
  for (int it = 0;; ++it) {
    bool inside = false;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      const double v = x[e];
      inside |= v > lo && v <= hi;
    }
    if (__ballot(inside) == 0) {
      resolved = true;
      break;
    }
    if (it >= max_iter) break;
    const double mid = 0.5 * (lo + hi);
    double f = 0.0;
#pragma unroll
    for (int e = 0; e < K; ++e) f += emass_d(x[e], mid, ad);
    f = wave_sum_d(f);
    if (f >= 1.0)
      lo = mid;
    else
      hi = mid;
  }
  if (!resolved) return static_cast<float>(lo);
  double s1 = 0.0;
  int ns = 0;
#pragma unroll
  for (int e = 0; e < K; ++e)
    if (x[e] > lo) {
      s1 += x[e];
      ++ns;
    }
  s1 = wave_sum_d(s1);
  ns = wave_sum_i(ns);
  const double nsd = static_cast<double>(ns);
  if (alpha == 2.f) return static_cast<float>((s1 - 1.0) / nsd);
  if (alpha == 1.5f) {
    const double M = s1 / nsd;
    double Q = 0.0;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      const double v = x[e];
      if (v > lo) Q += (v - M) * (v - M);
    }
    Q = wave_sum_d(Q);
    return static_cast<float>(M - sqrt(fmax((1.0 - Q) / nsd, 0.0)));
  }
  double l2 = lo, h2 = lo + 1.0;
  for (int it = 0; it < 64; ++it) {
    const double mid = 0.5 * (l2 + h2);
    double f = 0.0;
#pragma unroll
    for (int e = 0; e < K; ++e) {
      const double v = x[e];
      if (v > lo) f += emass_d(v, mid, ad);
    }
    f = wave_sum_d(f);
    if (f >= 1.0)
      l2 = mid;
    else
      h2 = mid;
  }
  return static_cast<float>(0.5 * (l2 + h2));
}

// AK: alpha known at compile time (1: 1.5, 2: 2; 0: the run-time a.alpha), so
// that the closed-form cases carry no pow() code and its registers.
template <int E, int MINW, int AK>
__global__ __launch_bounds__(kThreads, MINW) void entmax_rows_kernel(EntmaxArgs a) {
  __shared__ int bins[kWaves][16];
  __shared__ float live_x[kWaves][kWave];
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int64_t rowid = static_cast<int64_t>(blockIdx.x) * kWaves + w;  // (b, g, row)
  if (rowid >= static_cast<int64_t>(a.batch) * a.hkv * a.nrow) return;
  const int G = a.hq / a.hkv;
  const int row = static_cast<int>(rowid % a.nrow);
  const int64_t bg = rowid / a.nrow;
  const int g = static_cast<int>(bg % a.hkv);
  const int b = static_cast<int>(bg / a.hkv);
  const RowInfo ri = row_info(a.rule, b, row);
  const int n = ri.cand_end;  // <= 64 E
  const float alpha = AK == 1 ? 1.5f : AK == 2 ? 2.f : a.alpha;
  const double ad = alpha;
  float wsum[E];
#pragma unroll
  for (int e = 0; e < E; ++e) wsum[e] = 0.f;
  for (int hh = 0; hh < G; ++hh) {
    const int64_t hrow = (static_cast<int64_t>(b) * a.hq + g * G + hh) * a.nrow + row;
    const float* xr = a.xbuf + hrow * a.nblk;
    float x[E];
    float xmax = -INFINITY;
    int ne = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int j = e * kWave + lane;
      x[e] = (j < n && !is_forced(ri, j)) ? xr[j] : -INFINITY;
      if (x[e] != -INFINITY) {
        xmax = fmaxf(xmax, x[e]);
        ++ne;
      }
    }
    xmax = wave_max(xmax);
    ne = wave_sum_i(ne);
    float tau = __builtin_nanf("");
    float iz = 0.f;  // 1 / sum of the unnormalised masses (0: no candidates)
    if (ne > 0) {
      // 16-bin histogram of u = xmax - x on [0, 1)
      if (lane < 16) bins[w][lane] = 0;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const float u = xmax - x[e];
        if (x[e] != -INFINITY && u < 1.f) {
          int bin = static_cast<int>(floorf(u * 16.f));
          bin = bin > 15 ? 15 : bin;
          atomicAdd(&bins[w][bin], 1);
        }
      }
      __builtin_amdgcn_wave_barrier();
      const int cl = lane < 32 ? bins[w][lane & 15] : 0;
      const double xm = xmax;
      const double2 tb = bin_bounds(cl, ad);
      const double nterm = alpha == 1.5f ? 1.0 / sqrt(static_cast<double>(ne))
                           : alpha == 2.f ? 1.0 / static_cast<double>(ne)
                                          : pow(static_cast<double>(ne), 1.0 - ad);
      const double lo = fmax(xm + tb.x, xm - 1.0);
      const double hi = fmin(xm + tb.y, xm - nterm);
      // logits at or below lo never carry mass for a threshold in the
      // bracket: pack the others one per lane when they fit
      int nlive = 0;
#pragma unroll
      for (int e = 0; e < E; ++e) nlive += __popcll(__ballot(static_cast<double>(x[e]) > lo));
      if (nlive <= kWave) {
        int base = 0;
#pragma unroll
        for (int e = 0; e < E; ++e) {
          const bool live = static_cast<double>(x[e]) > lo;
          const uint64_t mk = __ballot(live);
          if (live) live_x[w][base + lanes_below(mk)] = x[e];
          base += __popcll(mk);
        }
        __builtin_amdgcn_wave_barrier();
        const float xl[1] = {lane < nlive ? live_x[w][lane] : -INFINITY};
        __builtin_amdgcn_wave_barrier();
        tau = entmax_tau<1>(xl, lo, hi, alpha, a.max_iter);
      } else {
        tau = entmax_tau<E>(x, lo, hi, alpha, a.max_iter);
      }
      float z = 0.f;
#pragma unroll
      for (int e = 0; e < E; ++e) z += emass(x[e], tau, alpha);
      z = wave_sum(z);
      iz = 1.f / z;
#pragma unroll
      for (int e = 0; e < E; ++e) wsum[e] += emass(x[e], tau, alpha) * iz;
    }
    if (a.tau && lane == 0) a.tau[hrow] = tau;
    if (a.probs) {
      float* pr = a.probs + hrow * a.nblk;
#pragma unroll
      for (int e = 0; e < E; ++e) {
        const int j = e * kWave + lane;
        if (j < a.nblk) pr[j] = (j < n && ne > 0) ? emass(x[e], tau, alpha) * iz : 0.f;
      }
      for (int j = E * kWave + lane; j < a.nblk; j += kWave) pr[j] = 0.f;
    }
  }
  // GQA: mean probability over the group's heads; keep the positive ones,
  // capped at the `cap` largest (lower block first on ties)
  const float invG = 1.f / static_cast<float>(G);
  float wb[E];
  uint32_t key[E];
  bool valid[E], sel[E];
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const int j = e * kWave + lane;
    wb[e] = wsum[e] * invG;
    valid[e] = j < n && !is_forced(ri, j) && wb[e] > 0.f;
    key[e] = valid[e] ? float_key(wb[e]) : 0u;
  }
  const int nr = wave_topm<E>(key, valid, a.cap, sel);
  // ascending: block 0 when forced first, the routed ids (strictly between
  // the forced ones), then the row's own block when forced
  int32_t* idx = a.idx + rowid * a.width;
  float* wsel = a.wsel ? a.wsel + rowid * a.width : nullptr;
  const int lead = (ri.f0 == 0 && (a.rule.force & 2u)) ? 1 : 0;
  const int tail0 = (!lead && ri.f0 >= 0) ? ri.f0 : -1;
  const int total = lead + nr + (tail0 >= 0) + (ri.f1 >= 0);
  int base = lead;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const uint64_t mk = __ballot(sel[e]);
    if (sel[e]) {
      const int pos = base + lanes_below(mk);
      idx[pos] = e * kWave + lane;
      if (wsel) wsel[pos] = wb[e];
    }
    base += __popcll(mk);
  }
  for (int q = lane; q < a.width; q += kWave) {
    if (q >= lead && q < lead + nr) continue;
    int v = -1;
    float wv = 0.f;
    if (q < lead) {
      v = 0;
      wv = 1.f;
    } else if (q < total) {
      v = (q == lead + nr && tail0 >= 0) ? tail0 : ri.f1;
      wv = 1.f;
    }
    idx[q] = v;
    if (wsel) wsel[q] = wv;
  }
  if (lane == 0) a.cnt[rowid] = total;
}

}  // namespace

hipError_t launch_scores(const ScoreArgs& a, hipStream_t stream, bool fill) {
  if (a.rule.mode != 1) {
    // block tiles per workgroup: enough row tiles to fill the chip with one
    // workgroup each when rows are many (per-token routing), else one
    const int nrt = (a.nrow + kTile - 1) / kTile, njt = (a.nblk + kTile - 1) / kTile;
    const int64_t rowtiles = static_cast<int64_t>(a.batch) * a.qheads * nrt;
    const int jgroup = rowtiles >= 4096 ? njt : 1;
    const unsigned tiles = static_cast<unsigned>(nrt) *
                           static_cast<unsigned>((njt + jgroup - 1) / jgroup);
    const unsigned grid = static_cast<unsigned>(a.batch) * a.qheads * tiles;
    const int f = fill ? 1 : 0;
    if (a.d == 64)
      hipLaunchKernelGGL(scores_mfma<64>, dim3(grid), dim3(kThreads), 0, stream, a, f, jgroup);
    else
      hipLaunchKernelGGL(scores_mfma<128>, dim3(grid), dim3(kThreads), 0, stream, a, f, jgroup);
    return hipGetLastError();
  }
  const int nchunk = (a.nblk + kChunk - 1) / kChunk;
  const unsigned grid = static_cast<unsigned>(a.batch) * a.qheads * a.nrow * nchunk;
  if (a.d == 64)
    hipLaunchKernelGGL(scores_kernel<64>, dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL(scores_kernel<128>, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_select_topk(const SelectArgs& a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * a.nrow;
  hipLaunchKernelGGL(select_kernel, dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

hipError_t launch_route_entmax(const EntmaxArgs& a, hipStream_t stream) {
  if (a.rule.mode == 2 && a.nblk <= 16 * kWave) {
    // per-token rows: many short rows, one wavefront each
    const int64_t rows = static_cast<int64_t>(a.batch) * a.hkv * a.nrow;
    const unsigned grid = static_cast<unsigned>((rows + kWaves - 1) / kWaves);
    const bool small = a.nblk <= 8 * kWave;
    if (a.alpha == 1.5f) {
      if (small)
        hipLaunchKernelGGL((entmax_rows_kernel<8, 3, 1>), dim3(grid), dim3(kThreads), 0, stream, a);
      else
        hipLaunchKernelGGL((entmax_rows_kernel<16, 1, 1>), dim3(grid), dim3(kThreads), 0, stream, a);
    } else if (a.alpha == 2.f) {
      if (small)
        hipLaunchKernelGGL((entmax_rows_kernel<8, 3, 2>), dim3(grid), dim3(kThreads), 0, stream, a);
      else
        hipLaunchKernelGGL((entmax_rows_kernel<16, 1, 2>), dim3(grid), dim3(kThreads), 0, stream, a);
    } else {
      if (small)
        hipLaunchKernelGGL((entmax_rows_kernel<8, 3, 0>), dim3(grid), dim3(kThreads), 0, stream, a);
      else
        hipLaunchKernelGGL((entmax_rows_kernel<16, 1, 0>), dim3(grid), dim3(kThreads), 0, stream, a);
    }
    return hipGetLastError();
  }
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * a.nrow;
  const size_t rows = static_cast<size_t>(a.hq / a.hkv) * a.nblk * sizeof(float);
  const size_t capb = ((static_cast<size_t>(a.nblk) + kSel - 1) / kSel) * a.cap;
  const size_t tb = (4 * capb + 2 * static_cast<size_t>(a.cap)) * 4;
  EntmaxArgs b = a;
  b.tourn = a.cap < kSel && tb <= 48 * 1024;
  const size_t extra = b.tourn ? tb : 0;
  if (rows + extra <= 64 * 1024)
    hipLaunchKernelGGL(entmax_kernel<true>, dim3(grid), dim3(kThreads), rows + extra, stream, b);
  else
    hipLaunchKernelGGL(entmax_kernel<false>, dim3(grid), dim3(kThreads), extra, stream, b);
  return hipGetLastError();
}

}  // namespace bsa
