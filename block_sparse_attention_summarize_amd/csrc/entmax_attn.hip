// Token-level alpha-entmax attention, causal prefill ("AdaSplash-2", sections
// 1 and 2).  For query t the weights over its keys j <= t are
// p = alpha-entmax(z), x_j = (alpha-1) z_j = (alpha-1) sm_scale q_t . k_j,
// p_j = [x_j - tau_t]_+^(1/(alpha-1)) with tau_t the normaliser (sum p = 1),
// and o_t = sum_j p_j v_j.
//
// A workgroup (4 wavefronts, 32 queries x one query head each, like the
// softmax prefill kernel) owns 64 queries of a (batch, KV head) pair and
// walks the causal key tiles several times, keeping Q in registers:
//   1. row maxima of x;
//   2. a 16-bin histogram of x_max - x on [0, 1) per query (2.A: tau lies in
//      [x_max - 1, x_max]); its closed-form roots with every count at its bin's
//      lower and upper edge bracket tau;
//   3. `refine` passes of the hybrid step of 2.B from the bracket's lower end
//      (Halley for alpha <= 1.5, Newton for 1.5 < alpha <= 2, and for
//      alpha > 2 a secant through the bracket ends with the Illinois halving;
//      each kept inside the bracket, else bisection), the first of which also
//      marks the key tiles holding any x above that lower end;
//   4. the output: only the marked tiles (a tile with every x <= tau has zero
//      weight), p on the matrix cores against V, normalised by its sum.
// S^T = K Q^T and O^T += V^T P^T run on v_mfma_f32_16x16x32_bf16 as in the
// softmax kernel (V's transposed operand from ds_read_b64_tr_b16).
#include "common.hpp"
#include "kernels.hpp"

namespace bsa {

namespace {

typedef __bf16 ebf16x8 __attribute__((ext_vector_type(8)));
typedef float ef32x4 __attribute__((ext_vector_type(4)));
typedef short ev4i16 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ ef32x4 emfma(const uint4& a, const uint4& b, ef32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(ebf16x8, a),
                                                __builtin_bit_cast(ebf16x8, b), c, 0, 0, 0);
}

// Sum / max over the four lanes l, l^16, l^32, l^48 (the lanes holding one
// query column of an S^T fragment).
__device__ __forceinline__ float col_max(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float col_sum(float v) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  v = __uint_as_float(r[0]) + __uint_as_float(r[1]);
  r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// [d]_+^(1/(alpha-1)) and the first two derivatives' magnitudes with respect
// to tau (d = x - tau > 0): m = d^e, m1 = e d^(e-1), m2 = e (e-1) d^(e-2).
struct Mass {
  float m, m1, m2;
};
__device__ __forceinline__ Mass mass3(float d, float alpha, float e) {
  Mass r{0.f, 0.f, 0.f};
  if (!(d > 0.f)) return r;
  if (alpha == 1.5f) {
    r.m = d * d;
    r.m1 = 2.f * d;
    r.m2 = 2.f;
  } else if (alpha == 2.f) {
    r.m = d;
    r.m1 = 1.f;
  } else {
    const float p = __builtin_amdgcn_exp2f(e * __builtin_amdgcn_logf(d));  // log2
    r.m = p;
    r.m1 = e * p / d;
    r.m2 = e * (e - 1.f) * p / (d * d);
  }
  return r;
}
__device__ __forceinline__ float mass1(float d, float alpha, float e) {
  if (!(d > 0.f)) return 0.f;
  if (alpha == 1.5f) return d * d;
  if (alpha == 2.f) return d;
  return __builtin_amdgcn_exp2f(e * __builtin_amdgcn_logf(d));
}

// Root of sum_k c_k [e_k - tau]_+^(1/(alpha-1)) = 1 over the 16 bin values
// e_k = xm - (k + off)/16, as the routing kernels' solve_bins (per lane, its
// own query's counts): prefix closed forms for alpha 1.5 and 2, else 64
// bisection steps on [e_0 - 1, e_0].
__device__ inline double bins_root(const int (&c)[16], double xm, int off, double alpha) {
  auto ev = [&](int k) { return xm - static_cast<double>(k + off) * 0.0625; };
  if (alpha == 2.0 || alpha == 1.5) {
    double n = 0.0, s1 = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (c[r] == 0) continue;
      n += c[r];
      s1 += c[r] * ev(r);
      double tau;
      if (alpha == 2.0) {
        tau = (s1 - 1.0) / n;
      } else {
        const double M = s1 / n;
        double Q = 0.0;
#pragma unroll
        for (int k = 0; k <= r; ++k) {
          const double dv = ev(k) - M;
          Q += c[k] * dv * dv;
        }
        if (Q > 1.0) continue;
        tau = M - sqrt((1.0 - Q) / n);
      }
      int nx = 16;
#pragma unroll
      for (int k = 15; k > r; --k)
        if (c[k] != 0) nx = k;
      if (tau < ev(r) && (nx >= 16 || tau >= ev(nx))) return tau;
    }
  }
  double lo = ev(0) - 1.0, hi = ev(0);
  const double e = 1.0 / (alpha - 1.0);
  for (int it = 0; it < 64; ++it) {
    const double mid = 0.5 * (lo + hi);
    double f = 0.0;
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (c[r] != 0 && ev(r) > mid) f += c[r] * pow(ev(r) - mid, e);
    if (f >= 1.0)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

template <int D>
struct EntLds {
  static constexpr int KST = D + 8;
  static constexpr int VST = D + 16;
  alignas(16) uint16_t k[2][64 * KST];
  alignas(16) uint16_t v[2][64 * VST];
};

constexpr int kMaxKeyTiles = 2048;  // 64-key tiles of one sequence (N <= 131072)

template <int D, int QT, int NW, bool OUT_F32>
__global__ __launch_bounds__(NW * 64, 8 / NW) void entmax_attn_bf16(EntmaxAttnArgs a, int wpb) {
  constexpr int NT = NW * 64;
  constexpr int QPW = 16 * QT;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int CPR = D / 8;
  constexpr int KTOT = 64 * CPR;
  constexpr int KITEMS = (KTOT + NT - 1) / NT;
  __shared__ EntLds<D> lds;
  __shared__ uint32_t live[kMaxKeyTiles / 32];
  __shared__ int lds_list[kMaxKeyTiles];
  __shared__ int lds_n;
  using L = EntLds<D>;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.hq / a.hkv;
  const int nqt = static_cast<int>((a.n + 63) / 64);
  const int units = G * (64 / QPW);
  // heavy (late) query tiles first; the workgroups of a (pair, tile) adjacent
  const int id = blockIdx.x;
  const int sub = id % wpb;
  const int rest = id / wpb;
  const int pair = rest % (a.batch * a.hkv);
  const int i = nqt - 1 - rest / (a.batch * a.hkv);
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int u = sub * NW + w;
  const bool active = u < units;
  const int hh = active ? u % G : 0;
  const int qs = active ? u / G : 0;
  const int h = g * G + hh;
  const int qpos0 = i * 64 + qs * QPW;
  const int ntile = i + 1;  // causal key tiles 0..i

  const auto rk = make_rsrc(static_cast<const uint16_t*>(a.K) + b * a.ks.b + g * a.ks.h,
                            head_bytes(a.n, a.ks.t, D, 2));
  const auto rv = make_rsrc(static_cast<const uint16_t*>(a.V) + b * a.vs.b + g * a.vs.h,
                            head_bytes(a.n, a.vs.t, D, 2));
  const uint32_t kst = static_cast<uint32_t>(a.ks.t * 2), vst = static_cast<uint32_t>(a.vs.t * 2);

  uint4 qf[QT][KS];
  {
    const auto rq = make_rsrc(static_cast<const uint16_t*>(a.Q) + b * a.qs.b + h * a.qs.h,
                              active ? head_bytes(a.n, a.qs.t, D, 2) : 0u);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const uint32_t t = static_cast<uint32_t>(qpos0 + qt * 16 + (lane & 15));
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        qf[qt][ks] = buf_load16(rq, t * static_cast<uint32_t>(a.qs.t * 2) + (ks * 32 + (lane >> 4) * 8) * 2);
    }
  }
  const float alpha = a.alpha;
  const float e = 1.f / (alpha - 1.f);
  const float cx = (alpha - 1.f) * a.sm_scale;  // x = cx * s

  uint4 kreg[KITEMS], vreg[KITEMS];
  auto load_k = [&](int k0) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (KTOT % NT == 0 || flat < KTOT)
        kreg[it] = buf_load16(rk, static_cast<uint32_t>(k0 + r) * kst + c * 16);
    }
  };
  auto load_v = [&](int k0) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (KTOT % NT == 0 || flat < KTOT)
        vreg[it] = buf_load16(rv, static_cast<uint32_t>(k0 + r) * vst + c * 16);
    }
  };
  auto store_k = [&](int buf) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (KTOT % NT == 0 || flat < KTOT)
        *reinterpret_cast<uint4*>(&lds.k[buf][r * L::KST + c * 8]) = kreg[it];
    }
  };
  auto store_v = [&](int buf) {
#pragma unroll
    for (int it = 0; it < KITEMS; ++it) {
      const int flat = tid + NT * it;
      const int r = flat / CPR, c = flat % CPR;
      if (KTOT % NT == 0 || flat < KTOT)
        *reinterpret_cast<uint4*>(&lds.v[buf][r * L::VST + c * 8]) = vreg[it];
    }
  };
  // S^T of the tile in buffer buf, causal-masked: s[kt][qt][j] is key
  // 16kt + 4(l/16) + j of query column 16qt + l%16
  auto scores = [&](int buf, int k0, ef32x4 (&s)[4][QT]) {
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[kt][qt] = ef32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const uint4 kf = *reinterpret_cast<const uint4*>(
            &lds.k[buf][(kt * 16 + (lane & 15)) * L::KST + ks * 32 + (lane >> 4) * 8]);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[kt][qt] = emfma(kf, qf[qt][ks], s[kt][qt]);
      }
    }
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
  };
  // One pass over the key tiles in lds_list[0, lds_n): K (and V) staged with
  // the next tile's loads in flight; body(t, buf, k0) per tile.
  auto pass = [&](bool with_v, auto&& body) {
    const int nt = lds_n;
    int buf = 0;
    if (nt > 0) {
      load_k(lds_list[0] * 64);
      if (with_v) load_v(lds_list[0] * 64);
      store_k(0);
      if (with_v) store_v(0);
    }
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      const int k0 = lds_list[t] * 64;
      const bool more = t + 1 < nt;
      if (more) {
        load_k(lds_list[t + 1] * 64);
        if (with_v) load_v(lds_list[t + 1] * 64);
      }
      if (active) body(t, buf, k0);
      if (more) {
        store_k(buf ^ 1);
        if (with_v) store_v(buf ^ 1);
      }
      __syncthreads();
      buf ^= 1;
    }
  };
  auto list_all = [&]() {
    for (int t = tid; t < ntile; t += NT) lds_list[t] = t;
    if (tid == 0) lds_n = ntile;
    __syncthreads();
  };

  // ---- pass 1: row maxima of s, and each tile's maximum over the
  // workgroup's queries (order-preserving keys, LDS atomics over the V
  // buffers: [ntile] after the histogram's place) ----
  uint32_t* tkey = reinterpret_cast<uint32_t*>(&lds.v[0][0]) + NW * QT * 256;
  static_assert((NW * QT * 256 + kMaxKeyTiles + 1) * 4 <= sizeof(lds.v), "tile maxima do not fit");
  for (int t = tid; t <= ntile; t += NT) tkey[t] = 0u;  // tkey[ntile]: the threshold
  list_all();
  float smax[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) smax[qt] = -INFINITY;
  pass(false, [&](int t, int buf, int k0) {
    ef32x4 s[4][QT];
    scores(buf, k0, s);
    float tm = -INFINITY;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float m = -INFINITY;
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) m = fmaxf(m, s[kt][qt][j]);
      smax[qt] = fmaxf(smax[qt], m);
      tm = fmaxf(tm, m);
    }
    tm = wave_max(tm);
    if (lane == 0) atomicMax(&tkey[lds_list[t]], float_key(tm));
  });
  float xmax[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) xmax[qt] = cx * col_max(smax[qt]);
  {
    // Keys below x_max - 1 of their query carry no weight (tau >= x_max - 1),
    // so every later pass visits only the tiles whose maximum exceeds the
    // smallest x_max - 1 over the workgroup's queries (a superset).
    float thr = INFINITY;  // in units of s
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
      if (qpos0 + qt * 16 + (lane & 15) < a.n) thr = fminf(thr, (xmax[qt] - 1.f) / cx);
    thr = -wave_max(-thr);
    if (active && lane == 0) atomicMax(&tkey[ntile], ~float_key(thr));  // max of ~key = min
    __syncthreads();
    const uint32_t tk = ~tkey[ntile];  // key of the smallest threshold
    if (w == 0) {
      int c = 0;
      for (int base = 0; base < ntile; base += 64) {
        const int t = base + lane;
        const bool on = t < ntile && tkey[t] > tk;
        const uint64_t mk = __ballot(on);
        if (on) lds_list[c + lanes_below(mk)] = t;
        c += __popcll(mk);
      }
      if (lane == 0) lds_n = c;
    }
    __syncthreads();
  }

  // ---- pass 2: histogram of xmax - x on [0, 1) ----
  // counts per (wave, query column, bin) in LDS atomics, over the V buffers
  // (unused until the output pass)
  int* hist = reinterpret_cast<int*>(&lds.v[0][0]);  // [NW][QT][16 columns][16 bins]
  static_assert(NW * QT * 16 * 16 * 4 <= sizeof(lds.v), "histogram does not fit");
  for (int e2 = tid; e2 < NW * QT * 256; e2 += NT) hist[e2] = 0;
  __syncthreads();
  int* myh = hist + w * QT * 256 + (lane & 15) * 16;
  pass(false, [&](int, int buf, int k0) {
    ef32x4 s[4][QT];
    scores(buf, k0, s);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt)
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float uu = xmax[qt] - cx * s[kt][qt][j];
          if (uu < 1.f) {  // -inf scores give +inf
            int bin = static_cast<int>(uu * 16.f);
            bin = bin > 15 ? 15 : bin;
            atomicAdd(myh + qt * 256 + bin, 1);
          }
        }
  });
  // bracket per query column (fp64)
  // bracket [lo, hi]: h = mass - 1 >= 0 at lo, < 0 at hi
  double lo[QT], hi[QT], tau[QT];
  // alpha > 2: the mass values at the bracket ends (valid once the end has
  // been evaluated: side bit 1 lo, bit 2 hi) and which end the last iterate
  // replaced, for the bracketed secant.  No NaN sentinels: this file is built
  // without NaN semantics.
  double hlo[QT], hhi[QT];
  int side[QT], have[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    hlo[qt] = hhi[qt] = 0.0;
    side[qt] = have[qt] = 0;
  }
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    int cnt[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) cnt[k] = myh[qt * 256 + k];
    const int64_t qpos = qpos0 + qt * 16 + (lane & 15);
    const double nkeys = static_cast<double>(qpos < a.n ? qpos + 1 : 1);
    const double xm = xmax[qt];
    const double tl = bins_root(cnt, xm, 1, alpha);
    const double th = bins_root(cnt, xm, 0, alpha);
    const double nterm = alpha == 1.5f ? 1.0 / sqrt(nkeys)
                         : alpha == 2.f ? 1.0 / nkeys : pow(nkeys, 1.0 - static_cast<double>(alpha));
    lo[qt] = fmax(tl, xm - 1.0);
    hi[qt] = fmin(th, xm - nterm);
    if (!(hi[qt] >= lo[qt])) hi[qt] = lo[qt];
    tau[qt] = lo[qt];
  }

  // ---- pass 3: hybrid refinement; the first pass marks the live tiles ----
  for (int t = tid; t < kMaxKeyTiles / 32; t += NT) live[t] = 0u;
  __syncthreads();
  for (int it = 0; it < a.refine; ++it) {
    const bool mark = it == 0;
    float f0[QT], f1[QT], f2[QT];
    float tf[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      f0[qt] = f1[qt] = f2[qt] = 0.f;
      tf[qt] = static_cast<float>(tau[qt]);
    }
    pass(false, [&](int t, int buf, int k0) {
      ef32x4 s[4][QT];
      scores(buf, k0, s);
      bool any = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float d = cx * s[kt][qt][j] - tf[qt];
            any |= d > 0.f;
            const Mass r = mass3(d, alpha, e);
            f0[qt] += r.m;
            f1[qt] += r.m1;
            f2[qt] += r.m2;
          }
      if (mark && __ballot(any) != 0ull && lane == 0) atomicOr(&live[lds_list[t] >> 5], 1u << (lds_list[t] & 31));
    });
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const double h0 = static_cast<double>(col_sum(f0[qt])) - 1.0;
      const double d1 = col_sum(f1[qt]);  // -dh/dtau
      const double d2 = col_sum(f2[qt]);  // d2h/dtau2
      // the iterate replaces the bracket end on its side; for alpha > 2 the
      // other end's mass value is halved when it is kept twice in a row
      // (Illinois), so the secant cannot stall on one side
      if (h0 >= 0.0) {
        if (side[qt] > 0) hhi[qt] *= 0.5;
        lo[qt] = tau[qt];
        hlo[qt] = h0;
        side[qt] = 1;
        have[qt] |= 1;
      } else {
        if (side[qt] < 0) hlo[qt] *= 0.5;
        hi[qt] = tau[qt];
        hhi[qt] = h0;
        side[qt] = -1;
        have[qt] |= 2;
      }
      double nt;
      if (alpha <= 1.5f) {
        nt = tau[qt] + 2.0 * h0 * d1 / (2.0 * d1 * d1 - h0 * d2);  // Halley
      } else if (alpha <= 2.f) {
        nt = tau[qt] + h0 / d1;  // Newton
      } else {
        // secant through the bracket ends (bisection until both are known):
        // the mass has a kink of unbounded slope at every key, which defeats
        // the derivative steps
        nt = (have[qt] == 3 && hlo[qt] > hhi[qt])
                 ? lo[qt] + hlo[qt] * (hi[qt] - lo[qt]) / (hlo[qt] - hhi[qt])
                 : 0.5 * (lo[qt] + hi[qt]);
      }
      if (!(nt >= lo[qt] && nt <= hi[qt])) nt = (h0 == 0.0) ? tau[qt] : 0.5 * (lo[qt] + hi[qt]);
      tau[qt] = nt;
    }
    if (mark) {
      // the output and later refinements visit only tiles with some x > lo
      __syncthreads();
      if (a.live) {
        // the workgroup's marks, OR-ed into its query tile's row (the other
        // workgroups of the tile hold other heads of the group)
        uint32_t* row = a.live + (static_cast<int64_t>(pair) * nqt + i) * ((nqt + 31) / 32);
        for (int t = tid; t <= (ntile - 1) >> 5; t += NT)
          if (live[t] != 0u) atomicOr(row + t, live[t]);
      }
      if (w == 0) {
        int c = 0;
        for (int base = 0; base < ntile; base += 64) {
          const int t = base + lane;
          const bool on = t < ntile && ((live[t >> 5] >> (t & 31)) & 1u);
          const uint64_t mk = __ballot(on);
          if (on) lds_list[c + lanes_below(mk)] = t;
          c += __popcll(mk);
        }
        if (lane == 0) lds_n = c;
      }
      __syncthreads();
    }
  }
  if (a.refine == 0) {
    // no refinement: every tile is visited (and every causal tile is live)
    list_all();
    if (a.live && sub == 0) {
      uint32_t* row = a.live + (static_cast<int64_t>(pair) * nqt + i) * ((nqt + 31) / 32);
      for (int t = tid; t <= (ntile - 1) >> 5; t += NT)
        row[t] = (t < (ntile >> 5)) ? ~0u : (1u << (ntile & 31)) - 1u;
    }
  }

  // ---- pass 4: output over the live tiles ----
  ef32x4 o[DT][QT], lsum[QT];
  float tf[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    lsum[qt] = ef32x4{0.f, 0.f, 0.f, 0.f};
    tf[qt] = static_cast<float>(tau[qt]);
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) o[dt][qt] = ef32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint4 ones = make_uint4(0x3f803f80u, 0x3f803f80u, 0x3f803f80u, 0x3f803f80u);
  pass(true, [&](int, int buf, int k0) {
    ef32x4 s[4][QT];
    scores(buf, k0, s);
    uint4 pf[QT][2];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float p[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) p[kt][j] = mass1(cx * s[kt][qt][j] - tf[qt], alpha, e);
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        pf[qt][kk].x = pack_bf16x2(p[2 * kk][0], p[2 * kk][1]);
        pf[qt][kk].y = pack_bf16x2(p[2 * kk][2], p[2 * kk][3]);
        pf[qt][kk].z = pack_bf16x2(p[2 * kk + 1][0], p[2 * kk + 1][1]);
        pf[qt][kk].w = pack_bf16x2(p[2 * kk + 1][2], p[2 * kk + 1][3]);
      }
    }
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) lsum[qt] = emfma(ones, pf[qt][kk], lsum[qt]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        const int s16 = lane & 15;
        const uint16_t* vp = &lds.v[buf][(kk * 32 + (lane >> 4) * 4 + (s16 >> 2)) * L::VST +
                                         dt * 16 + 4 * (s16 & 3)];
        typedef __attribute__((address_space(3))) ev4i16 lds_v4;
        const ev4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp));
        const ev4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp + 16 * L::VST));
        const uint2 u0 = __builtin_bit_cast(uint2, r0), u1 = __builtin_bit_cast(uint2, r1);
        const uint4 vf = make_uint4(u0.x, u0.y, u1.x, u1.y);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) o[dt][qt] = emfma(vf, pf[qt][kk], o[dt][qt]);
      }
    }
  });

  if (!active) return;
  uint8_t* Ob = static_cast<uint8_t*>(a.O);
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) {
    const int64_t t = qpos0 + qt * 16 + (lane & 15);
    if (t >= a.n) continue;
    if (a.tau && (lane >> 4) == 0) a.tau[(static_cast<int64_t>(b) * a.hq + h) * a.n + t] = tf[qt];
    const float lt = lsum[qt][0];
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    const int64_t off = b * a.os.b + h * a.os.h + t * a.os.t;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) {
      const int d0 = dt * 16 + (lane >> 4) * 4;
      const ef32x4 v = o[dt][qt] * inv;
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

// Clears the live-tile rows before the attention ORs its marks into them.
__global__ __launch_bounds__(256) void clear_words(uint32_t* p, int64_t n) {
  const int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (e < n) p[e] = 0u;
}

template <int D>
hipError_t entmax_launch(const EntmaxAttnArgs& a, hipStream_t stream) {
  constexpr int QT = 2, NW = 4;
  const int G = a.hq / a.hkv;
  const int units = G * (64 / (16 * QT));
  const int wpb = (units + NW - 1) / NW;
  const int nqt = static_cast<int>((a.n + 63) / 64);
  if (a.live) {
    const int64_t words = static_cast<int64_t>(a.batch) * a.hkv * nqt * ((nqt + 31) / 32);
    hipLaunchKernelGGL(clear_words, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0,
                       stream, a.live, words);
  }
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * nqt * wpb;
  if (a.out_f32)
    hipLaunchKernelGGL((entmax_attn_bf16<D, QT, NW, true>), dim3(grid), dim3(NW * 64), 0, stream,
                       a, wpb);
  else
    hipLaunchKernelGGL((entmax_attn_bf16<D, QT, NW, false>), dim3(grid), dim3(NW * 64), 0, stream,
                       a, wpb);
  return hipGetLastError();
}

}  // namespace

int entmax_attend_max_tiles() { return kMaxKeyTiles; }

hipError_t launch_entmax_attend(const EntmaxAttnArgs& a, hipStream_t stream) {
  return a.d == 64 ? entmax_launch<64>(a, stream) : entmax_launch<128>(a, stream);
}

}  // namespace bsa
