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
// Prefill scores: one workgroup per 64 rows x 64 blocks tile of one (b, g).
// The q-hat and summary tiles are staged in LDS (rows padded by 4 floats);
// thread (tr, tj) accumulates rows tr + 16m and blocks tj + 16n, m, n < 4.
// Tiles right of every row's candidates only write -inf (the candidate end
// grows with the row in prefill).
// ---------------------------------------------------------------------------
constexpr int kTile = 64;
constexpr int kPad = 4;

template <int D>
__global__ __launch_bounds__(kThreads) void scores_tiled(ScoreArgs a) {
  __shared__ float qs[kTile][D + kPad];
  __shared__ float ss[kTile][D + kPad];
  const int nrt = (a.nrow + kTile - 1) / kTile;
  const int njt = (a.nblk + kTile - 1) / kTile;
  int id = blockIdx.x;
  const int jt = id % njt;
  id /= njt;
  const int rt = id % nrt;
  const int bh = id / nrt;  // (b, q-hat head)
  const int b = bh / a.qheads;
  const int sg_row = b * a.hkv + (bh % a.qheads) / a.group;
  const int r0 = rt * kTile, j0 = jt * kTile;
  const int rn = a.nrow - r0 < kTile ? a.nrow - r0 : kTile;
  const int jn = a.nblk - j0 < kTile ? a.nblk - j0 : kTile;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  float* out = a.scores + (static_cast<int64_t>(bh) * a.nrow + r0) * a.nblk + j0;
  // candidates of row r: blocks before own(r) (entmax) or up to it (top-k),
  // own(r) = r for query-block rows and r / B for token rows
  const int ce = a.rule.entmax ? 0 : 1;
  const int tok_b = a.rule.mode == 2 ? a.rule.B : 1;
  if (j0 >= (r0 + rn - 1) / tok_b + ce) {  // right of the last row's candidates
    for (int e = tid; e < kTile * kTile; e += kThreads) {
      const int r = e / kTile, j = e % kTile;
      if (r < rn && j < jn) out[static_cast<int64_t>(r) * a.nblk + j] = -INFINITY;
    }
    return;
  }
  constexpr int V4 = D / 4;
  const float* qg = a.qhat + (static_cast<int64_t>(bh) * a.nrow + r0) * D;
  const float* sg = a.S + (static_cast<int64_t>(sg_row) * a.nblk + j0) * D;
  // rows past the ends read as zeros (buffer loads outside the extent)
  const auto rq = make_rsrc(qg, static_cast<uint32_t>(rn) * D * 4);
  const auto rs = make_rsrc(sg, static_cast<uint32_t>(jn) * D * 4);
  for (int e = tid; e < kTile * V4; e += kThreads) {
    const int r = e / V4, c = e % V4;
    *reinterpret_cast<uint4*>(&qs[r][c * 4]) = buf_load16(rq, static_cast<uint32_t>(e) * 16);
    *reinterpret_cast<uint4*>(&ss[r][c * 4]) = buf_load16(rs, static_cast<uint32_t>(e) * 16);
  }
  __syncthreads();
  const int tr = w * 4 + lane / 16, tj = lane % 16;
  float acc[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m)
#pragma unroll
    for (int n = 0; n < 4; ++n) acc[m][n] = 0.f;
#pragma unroll 2
  for (int k = 0; k < D; k += 4) {
    float4 qv[4], sv[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) qv[m] = *reinterpret_cast<const float4*>(&qs[tr + 16 * m][k]);
#pragma unroll
    for (int n = 0; n < 4; ++n) sv[n] = *reinterpret_cast<const float4*>(&ss[tj + 16 * n][k]);
#pragma unroll
    for (int m = 0; m < 4; ++m)
#pragma unroll
      for (int n = 0; n < 4; ++n) {
        float t = acc[m][n];
        t = fmaf(qv[m].x, sv[n].x, t);
        t = fmaf(qv[m].y, sv[n].y, t);
        t = fmaf(qv[m].z, sv[n].z, t);
        t = fmaf(qv[m].w, sv[n].w, t);
        acc[m][n] = t;
      }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int r = tr + 16 * m;
    const int cend = (r0 + r) / tok_b + ce - j0;
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int j = tj + 16 * n;
      if (r < rn && j < jn)
        out[static_cast<int64_t>(r) * a.nblk + j] = j < cend ? acc[m][n] * a.scale : -INFINITY;
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

}  // namespace

hipError_t launch_scores(const ScoreArgs& a, hipStream_t stream) {
  if (a.rule.mode != 1) {
    const unsigned tiles = static_cast<unsigned>((a.nrow + kTile - 1) / kTile) *
                           static_cast<unsigned>((a.nblk + kTile - 1) / kTile);
    const unsigned grid = static_cast<unsigned>(a.batch) * a.qheads * tiles;
    if (a.d == 64)
      hipLaunchKernelGGL(scores_tiled<64>, dim3(grid), dim3(kThreads), 0, stream, a);
    else
      hipLaunchKernelGGL(scores_tiled<128>, dim3(grid), dim3(kThreads), 0, stream, a);
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
