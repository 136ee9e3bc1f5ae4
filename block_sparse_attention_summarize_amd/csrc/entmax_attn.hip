// Token-level alpha-entmax attention, causal prefill ("AdaSplash-2", sections
// 1 and 2).  For query t the weights over its keys j <= t are
// p = alpha-entmax(z), x_j = (alpha-1) z_j = (alpha-1) sm_scale q_t . k_j,
// p_j = [x_j - tau_t]_+^(1/(alpha-1)) with tau_t the normaliser (sum p = 1),
// and o_t = sum_j p_j v_j.
//
// A workgroup of 8 wavefronts (32 queries x one query head each) owns the 64
// queries of a query tile for up to four heads of a GQA group, keeps Q in
// registers and walks the causal 64-key tiles several times:
//   1. row maxima of x, and each wavefront's maximum per tile;
//   2. a 16-bin histogram of x_max - x on [0, 1) per query (2.A: tau lies in
//      [x_max - 1, x_max]); its closed-form roots with every count at its bin's
//      lower and upper edge bracket tau;
//   3. `refine` passes of the hybrid step of 2.B from the bracket's lower end
//      (Halley for alpha <= 1.5, Newton for 1.5 < alpha <= 2, and for
//      alpha > 2 a secant through the bracket ends with the Illinois halving;
//      each kept inside the bracket: a Halley step outside it falls back to
//      the Newton step, then bisection), the first of which also
//      marks, per wavefront, the key tiles holding any x above that lower end;
//   4. the output: only the marked tiles (a tile with every x <= tau has zero
//      weight), p on the matrix cores against V, normalised by its sum.
// Each pass after the first visits only the tiles some wavefront can use, and
// a wavefront skips the others: pass 2 the tiles whose maximum reaches
// x_max - 1 of one of its queries, the first refinement those reaching the
// bracket's lower end, the rest those it marked.  K and V tiles arrive by
// direct-to-LDS loads in groups (three tiles a group in the K-only passes,
// two in the output), the next group loading while the wavefronts work
// through the current one with no barrier in between, so that a wavefront
// busy on one tile of a group does not hold the others up for the rest.
// The products run on v_mfma_f32_16x16x32_bf16 (V's transposed operand from
// ds_read_b64_tr_b16).
#include "common.hpp"
#include "kernels.hpp"
#include "lds_tiles.hpp"
#include "walk.hpp"

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

// Root of sum_k c_k [e_k - tau]_+^(1/(alpha-1)) = 1 over the NB bin values
// e_k = xm - (k + off)/16 (per lane, its own query's counts); closed forms
// for alpha 1.5 and 2, else 64 bisection steps on [e_0 - 1, e_0].
template <int NB>
__device__ inline double bins_root(const int (&c)[NB], double xm, int off, double alpha) {
  auto ev = [&](int k) { return xm - static_cast<double>(k + off) * 0.0625; };
  if (alpha == 2.0 || alpha == 1.5) {
    // The mass at tau = e_j comes from the bins above it: with u_k = (k +
    // off)/16 and prefix sums n, s1, s2 over k < j of c_k, c_k u_k, c_k u_k^2
    // it is n u_j - s1 (alpha 2) or n u_j^2 - 2 u_j s1 + s2 (alpha 1.5).  The
    // root lies below the last e_j where that is < 1 and at or above the first
    // where it is >= 1, so exactly the bins above that e_j hold its support.
    double n = 0.0, s1 = 0.0, s2 = 0.0;
    double nj = 0.0, s1j = 0.0, s2j = 0.0;
    bool found = false;
#pragma unroll
    for (int r = 0; r < NB; ++r) {
      const double ur = static_cast<double>(r + off) * 0.0625;
      const double f = alpha == 2.0 ? n * ur - s1 : (n * ur - 2.0 * s1) * ur + s2;
      if (!found && f >= 1.0) {
        found = true;
        nj = n;
        s1j = s1;
        s2j = s2;
      }
      n += c[r];
      s1 += c[r] * ur;
      s2 += c[r] * ur * ur;
    }
    if (!found) {
      nj = n;
      s1j = s1;
      s2j = s2;
    }
    if (nj == 0.0) return ev(0) - 1.0;  // no scores (a column past the sequence)
    if (alpha == 2.0) return xm - (s1j + 1.0) / nj;
    // n (u - s1/n)^2 + (s2 - s1^2/n) = 1 on the support, u above the mean
    const double Q = s2j - s1j * s1j / nj;
    return xm - s1j / nj - sqrt(fmax(1.0 - Q, 0.0) / nj);
  }
  double lo = ev(0) - 1.0, hi = ev(0);
  const double e = 1.0 / (alpha - 1.0);
  for (int it = 0; it < 64; ++it) {
    const double mid = 0.5 * (lo + hi);
    double f = 0.0;
#pragma unroll
    for (int r = 0; r < NB; ++r)
      if (c[r] != 0 && ev(r) > mid) f += c[r] * pow(ev(r) - mid, e);
    if (f >= 1.0)
      lo = mid;
    else
      hi = mid;
  }
  return 0.5 * (lo + hi);
}

constexpr int kMaxKeyTiles = 2048;  // 64-key tiles of one sequence (N <= 131072)
constexpr int kEw = 8;               // wavefronts per workgroup

// Each wavefront's tile maxima (16-bit order keys, rounded up) and the
// histograms, kept from the first pass to the first refinement.
struct EntAux {
  uint16_t tmx[kEw][kMaxKeyTiles];
  int hist[kEw][2][16][16];  // [wave][query tile][query column][bin]
};

// LDS of one workgroup.  The passes stage their tiles in groups: the K-only
// passes GK tiles a group in two sets of K slots, followed by the EntAux; the
// output pass GO tiles a group in two sets of K and V slots over the same
// space.
template <int D>
struct EntLds {
  static constexpr int TILE = 64 * D;  // elements of one tile
  static constexpr int GK = 3, GO = 2;
  static constexpr int AUX_OFF = 2 * GK * TILE * 2;  // bytes
  static constexpr int KONLY_BYTES = AUX_OFF + static_cast<int>(sizeof(EntAux));
  static constexpr int KV_BYTES = 4 * GO * TILE * 2;
  static constexpr int POOL = KONLY_BYTES > KV_BYTES ? KONLY_BYTES : KV_BYTES;
  alignas(16) unsigned char pool[POOL];
  uint32_t live[kEw][kMaxKeyTiles / 32];  // per wavefront: tiles with some x above its bracket
  uint64_t words[kMaxKeyTiles / 64];       // on-bits of a tile list being built
  int list[kMaxKeyTiles];
  uint32_t thr[kEw];                       // per wavefront: 16-bit key of its tile threshold
  int n;
  __device__ uint16_t* slot(int i) { return reinterpret_cast<uint16_t*>(pool) + i * TILE; }
  __device__ EntAux& aux() { return *reinterpret_cast<EntAux*>(pool + AUX_OFF); }
};

// Upper 16 bits of the order key of v, rounded up: a tile whose maximum m
// exceeds a threshold t has key16_up(m) > float_key(t) >> 16.
__device__ __forceinline__ uint32_t key16_up(float v) {
  const uint32_t k = float_key(v);
  const uint32_t r = (k >> 16) + ((k & 0xFFFFu) != 0u);
  return r > 0xFFFFu ? 0xFFFFu : r;
}

template <int D, bool OUT_F32>
__global__ __launch_bounds__(512, 1) void entmax_attn_bf16(EntmaxAttnArgs a, int wpb) {
  constexpr int NW = kEw, QT = 2, QPW = 32;
  constexpr int KS = D / 32;
  constexpr int DT = D / 16;
  constexpr int NC = D / 8;
  constexpr int NI = NC / NW;  // 1 KB direct-to-LDS loads per wavefront per tile and tensor
  static_assert(NI >= 1, "head dimension below 64");
  __shared__ EntLds<D> lds;
  using Z = SwzTile<D>;

  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.hq / a.hkv;
  const int nqt = static_cast<int>((a.n + 63) / 64);
  const int units = G * (64 / QPW);
  int pair, i, sub;
  map_wg(blockIdx.x, a.batch * a.hkv, nqt, wpb, pair, i, sub);
  const int b = pair / a.hkv, g = pair % a.hkv;
  const int u = sub * NW + w;
  const bool active = u < units;
  const int hh = active ? u % G : 0;
  const int qs = active ? u / G : 0;
  const int h = g * G + hh;
  const int qpos0 = i * 64 + qs * QPW;
  const int ntile = i + 1;  // causal key tiles 0..i
  bool valid[QT];           // this lane's query columns lie inside the sequence
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) valid[qt] = active && qpos0 + qt * 16 + (lane & 15) < a.n;

  const auto rk = make_desc(static_cast<const uint16_t*>(a.K) + b * a.ks.b + g * a.ks.h,
                            head_bytes(a.n, a.ks.t, D, 2));
  const auto rv = make_desc(static_cast<const uint16_t*>(a.V) + b * a.vs.b + g * a.vs.h,
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

  // direct-to-LDS loads: wavefront instruction it fills bytes [1 KB (w NI + it),
  // +1 KB) of a tile; lane l's 16 bytes land at chunk q = 64 (w NI + it) + l,
  // i.e. row q / NC, physical chunk q % NC, which holds logical chunk p ^ swz(row)
  uint32_t koff[NI], voff[NI];
#pragma unroll
  for (int it = 0; it < NI; ++it) {
    const int q = (w * NI + it) * 64 + lane;
    const int r = q / NC, p = q % NC;
    koff[it] = static_cast<uint32_t>(r) * kst + ((p ^ Z::kswz(r)) * 16);
    voff[it] = static_cast<uint32_t>(r) * vst + ((p ^ Z::vswz(r)) * 16);
  }
  // the tile at key k0: K into slot ks and, when vs >= 0, V into slot vs
  auto load_tile = [&](int k0, int ks, int vs) {
    const uint32_t kb = static_cast<uint32_t>(k0) * kst, vb = static_cast<uint32_t>(k0) * vst;
#pragma unroll
    for (int it = 0; it < NI; ++it) {
      lds_dma16(rk, lds.slot(ks) + (w * NI + it) * 512, koff[it] + kb);
      if (vs >= 0) lds_dma16(rv, lds.slot(vs) + (w * NI + it) * 512, voff[it] + vb);
    }
  };
  // fragment offsets (elements) at key tile rows 0-15; the swizzles repeat
  // every 16 rows, so the other rows are these plus a constant
  int kfo[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    const int r = lane & 15;
    kfo[ks] = r * D + ((ks * 4 + (lane >> 4)) ^ Z::kswz(r)) * 8;
  }
  int vfo[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) {
    const int s16 = lane & 15;
    const int r = (lane >> 4) * 4 + (s16 >> 2);
    const int c = dt * 2 + ((s16 & 3) >> 1);
    vfo[dt] = r * D + (c ^ Z::vswz(r)) * 8 + (s16 & 1) * 4;
  }

  // S^T of the K tile at kb: s[kt][qt][j] is key 16kt + 4(l/16) + j of query
  // column 16qt + l%16
  ef32x4 s[4][QT];
  auto scores = [&](const uint16_t* kb) {
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kt = 0; kt < 4; ++kt)
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) s[kt][qt] = ef32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
#pragma unroll
      for (int kt = 0; kt < 4; ++kt) {
        const uint4 kf = *reinterpret_cast<const uint4*>(kb + kfo[ks] + kt * 16 * D);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) s[kt][qt] = emfma(kf, qf[qt][ks], s[kt][qt]);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 6, 1);
#pragma unroll
    for (int r = 0; r < 10; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 1);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, 12, 1);
    __builtin_amdgcn_s_setprio(0);
  };
  // causal mask of the scores of the tile at key k0
  auto mask = [&](int k0) {
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
  // the largest of this lane's 16 scores of query tile qt
  auto lane_max = [&](int qt) {
    const float t0 = fmaxf(fmaxf(s[0][qt][0], s[0][qt][1]), fmaxf(s[0][qt][2], s[0][qt][3]));
    const float t1 = fmaxf(fmaxf(s[1][qt][0], s[1][qt][1]), fmaxf(s[1][qt][2], s[1][qt][3]));
    const float t2 = fmaxf(fmaxf(s[2][qt][0], s[2][qt][1]), fmaxf(s[2][qt][2], s[2][qt][3]));
    const float t3 = fmaxf(fmaxf(s[3][qt][0], s[3][qt][1]), fmaxf(s[3][qt][2], s[3][qt][3]));
    return fmaxf(fmaxf(t0, t1), fmaxf(t2, t3));
  };

  // One pass over lds.list[0, n) in groups of GS entries: between two
  // barriers every wavefront runs body(t, kb, vb) for the entries t of one
  // group (it skips those it has no use for), while the next group's K (and V)
  // tiles load into the other set of slots.
  auto run = [&](auto gs, bool with_v, auto&& body) {
    constexpr int GS = decltype(gs)::value;
    const int n = lds.n;
    auto load_group = [&](int g) {
      for (int e = 0; e < GS && g * GS + e < n; ++e) {
        const int sl = (g & 1) * GS + e;
        load_tile(lds.list[g * GS + e] * 64, sl, with_v ? 2 * GS + sl : -1);
      }
    };
    load_group(0);
    wait_vm<0>();
    __syncthreads();
    const int ng = (n + GS - 1) / GS;
#pragma clang loop unroll(disable)
    for (int g = 0; g < ng; ++g) {
      if (g + 1 < ng) load_group(g + 1);
      if (active) {
#pragma unroll
        for (int e = 0; e < GS; ++e) {
          const int t = g * GS + e;
          const int sl = (g & 1) * GS + e;
          if (t < n) body(t, lds.slot(sl), lds.slot(2 * GS + sl));
        }
      }
      wait_vm<0>();
      __syncthreads();
    }
  };
  using GK = std::integral_constant<int, EntLds<D>::GK>;
  using GO = std::integral_constant<int, EntLds<D>::GO>;
  // lds.list = the tiles t < ntile with on(t), ascending
  auto build_list = [&](auto&& on) {
    for (int c = w; c * 64 < ntile; c += NW) {
      const int t = c * 64 + lane;
      const uint64_t m = __ballot(t < ntile && on(t));
      if (lane == 0) lds.words[c] = m;
    }
    __syncthreads();
    if (w == 0) {
      int base = 0;
      for (int c = 0; c * 64 < ntile; ++c) {
        const uint64_t m = lds.words[c];
        if ((m >> lane) & 1ull) lds.list[base + lanes_below(m)] = c * 64 + lane;
        base += __popcll(m);
      }
      if (lane == 0) lds.n = base;
    }
    __syncthreads();
  };
  // this wavefront's tile threshold (the smallest of t over its valid query
  // columns, as a 16-bit key; none: no tile) published for the lists
  auto set_thr = [&](float t0, float t1) {
    float t = fminf(valid[0] ? t0 : INFINITY, valid[1] ? t1 : INFINITY);
    t = -wave_max(-t);
    const uint32_t k = t == INFINITY ? 0xFFFFu : (float_key(t) >> 16);
    if (lane == 0) lds.thr[w] = active ? k : 0xFFFFu;
    return k;
  };
  auto over_thr = [&](int t) {
    bool on = false;
#pragma unroll
    for (int v = 0; v < NW; ++v) on |= lds.aux().tmx[v][t] > lds.thr[v];
    return on;
  };
  auto any_live = [&](int t) {
    uint32_t m = 0u;
#pragma unroll
    for (int v = 0; v < NW; ++v) m |= lds.live[v][t >> 5];
    return ((m >> (t & 31)) & 1u) != 0u;
  };
  // wave-uniform: entry t of the list is above this wavefront's threshold
  auto above = [&](int t, uint32_t k) {
    return __builtin_amdgcn_readfirstlane(lds.aux().tmx[w][lds.list[t]]) > k;
  };
  auto is_live = [&](int t) {
    const int j = lds.list[t];
    return ((__builtin_amdgcn_readfirstlane(lds.live[w][j >> 5]) >> (j & 31)) & 1u) != 0u;
  };

  // ---- pass 1: row maxima of s and each wavefront's tile maxima ----
  for (int t = tid; t < ntile; t += 512) lds.list[t] = t;
  for (int t = tid; t < NW * (kMaxKeyTiles / 32); t += 512) (&lds.live[0][0])[t] = 0u;
  if (tid == 0) lds.n = ntile;
  __syncthreads();
  float smax[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) smax[qt] = -INFINITY;
  run(GK{}, false, [&](int t, const uint16_t* kb, const uint16_t*) {
    scores(kb);
    mask(lds.list[t] * 64);
    float tm = -INFINITY;
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float m = lane_max(qt);
      smax[qt] = fmaxf(smax[qt], m);
      tm = fmaxf(tm, valid[qt] ? m : -INFINITY);
    }
    tm = wave_max(tm);
    if (lane == 0) lds.aux().tmx[w][lds.list[t]] = static_cast<uint16_t>(key16_up(tm));
  });
  float xmax[QT];
#pragma unroll
  for (int qt = 0; qt < QT; ++qt) xmax[qt] = cx * col_max(smax[qt]);
  // keys with x <= x_max - 1 carry no weight (tau >= x_max - 1): the later
  // passes skip every tile whose maximum lies below that for all of a
  // wavefront's queries
  const uint32_t thr1 = set_thr((xmax[0] - 1.f) / cx, (xmax[1] - 1.f) / cx);
  for (int e2 = tid; e2 < NW * QT * 256; e2 += 512) (&lds.aux().hist[0][0][0][0])[e2] = 0;
  __syncthreads();
  build_list(over_thr);

  // ---- pass 2: histogram of x_max - x on [0, 1) per query column ----
  run(GK{}, false, [&](int t, const uint16_t* kb, const uint16_t*) {
    if (!above(t, thr1)) return;
    scores(kb);
    mask(lds.list[t] * 64);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      if (__ballot(xmax[qt] - cx * lane_max(qt) < 1.f) == 0ull) continue;
      int* hq = &lds.aux().hist[w][qt][lane & 15][0];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float uu = xmax[qt] - cx * s[kt][qt][j];
          if (uu < 1.f) {  // -inf scores give +inf
            const int bin = static_cast<int>(uu * 16.f);
            atomicAdd(hq + (bin > 15 ? 15 : bin), 1);
          }
        }
    }
  });
  // bracket per query column (fp64): h = mass - 1 >= 0 at lo, < 0 at hi
  double lo[QT], hi[QT], tau[QT];
  // alpha > 2: the mass values at the bracket ends (valid once the end has
  // been evaluated: have bit 1 lo, bit 2 hi) and which end the last iterate
  // replaced, for the bracketed secant.  No NaN sentinels: this file is built
  // without NaN semantics.
  double hlo[QT], hhi[QT];
  int side[QT], have[QT];
  // (a lambda called with constant arguments rather than a loop the compiler
  // may keep rolled, which would move these arrays to scratch memory)
  auto bracket = [&](int qt) {
    hlo[qt] = hhi[qt] = 0.0;
    side[qt] = have[qt] = 0;
    int cnt[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) cnt[k] = lds.aux().hist[w][qt][lane & 15][k];
    const int64_t qpos = qpos0 + qt * 16 + (lane & 15);
    const double nkeys = static_cast<double>(qpos < a.n ? qpos + 1 : 1);
    const double xm = xmax[qt];
    const double tl = bins_root<16>(cnt, xm, 1, alpha);
    const double th = bins_root<16>(cnt, xm, 0, alpha);
    const double nterm = alpha == 1.5f ? 1.0 / sqrt(nkeys)
                         : alpha == 2.f ? 1.0 / nkeys : pow(nkeys, 1.0 - static_cast<double>(alpha));
    lo[qt] = fmax(tl, xm - 1.0);
    hi[qt] = fmin(th, xm - nterm);
    if (!(hi[qt] >= lo[qt])) hi[qt] = lo[qt];
    tau[qt] = lo[qt];
  };
  static_assert(QT == 2, "two query tiles per wavefront");
  bracket(0);
  bracket(1);
  __syncthreads();  // the histograms are read before the thresholds move
  // every later pass visits only keys above the bracket's lower end
  const uint32_t thr2 = set_thr(static_cast<float>(lo[0]) / cx, static_cast<float>(lo[1]) / cx);
  __syncthreads();
  if (a.refine > 0) build_list(over_thr);

  // ---- pass 3: hybrid refinement; the first pass marks the live tiles ----
  for (int it = 0; it < a.refine; ++it) {
    const bool mark = it == 0;
    float f0[QT], f1[QT], f2[QT];
    float tf[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      f0[qt] = f1[qt] = f2[qt] = 0.f;
      tf[qt] = static_cast<float>(tau[qt]);
    }
    auto relevant = [&](int t) { return mark ? above(t, thr2) : is_live(t); };
    const bool closed = alpha == 1.5f || alpha == 2.f;
    run(GK{}, false, [&](int t, const uint16_t* kb, const uint16_t*) {
          if (!relevant(t)) return;
          scores(kb);
          mask(lds.list[t] * 64);
          bool any = false;
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            const float dm = valid[qt] ? cx * lane_max(qt) - tf[qt] : -INFINITY;
            if (__ballot(dm > 0.f) == 0ull) continue;
            any = true;
            if (closed) {
              // alpha 1.5 and 2: the sums of d_+^2, d_+ and [d > 0], from
              // which the mass and its derivatives follow after the column sums
#pragma unroll
              for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const float d = fmaf(cx, s[kt][qt][j], -tf[qt]);
                  const float dp = fmaxf(d, 0.f);
                  f0[qt] = fmaf(dp, dp, f0[qt]);
                  f1[qt] += dp;
                  f2[qt] += d > 0.f ? 1.f : 0.f;
                }
            } else {
              // [d]_+^(1/(alpha-1)) and its first two derivatives' magnitudes
#pragma unroll
              for (int kt = 0; kt < 4; ++kt)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                  const Mass r = mass3(fmaf(cx, s[kt][qt][j], -tf[qt]), alpha, e);
                  f0[qt] += r.m;
                  f1[qt] += r.m1;
                  f2[qt] += r.m2;
                }
            }
          }
          if (mark && any && lane == 0) {
            const int j = lds.list[t];
            lds.live[w][j >> 5] |= 1u << (j & 31);
          }
        });
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const double a0 = col_sum(f0[qt]), a1 = col_sum(f1[qt]), a2 = col_sum(f2[qt]);
      // mass - 1, -dh/dtau and d2h/dtau2: alpha 1.5: sum d^2, 2 sum d, 2 count;
      // alpha 2: sum d, count, 0; otherwise the sums as accumulated
      const double h0 = (alpha == 2.f ? a1 : a0) - 1.0;
      const double d1 = alpha == 1.5f ? 2.0 * a1 : alpha == 2.f ? a2 : a1;
      const double d2 = alpha == 1.5f ? 2.0 * a2 : alpha == 2.f ? 0.0 : a2;
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
      // for alpha <= 2 the mass is convex and decreasing in tau, so a Newton
      // step from the root's left stays between the iterate and the root: it
      // replaces a Halley step that leaves the bracket (Halley overshoots
      // where keys leave the support between the iterate and the root), and
      // bisection is the last resort
      if (alpha <= 1.5f && !(nt >= lo[qt] && nt <= hi[qt])) nt = tau[qt] + h0 / d1;
      if (!(nt >= lo[qt] && nt <= hi[qt])) nt = (h0 == 0.0) ? tau[qt] : 0.5 * (lo[qt] + hi[qt]);
      tau[qt] = nt;
    }
    if (mark) {
      // the output and later refinements visit only tiles with some x > lo
      build_list(any_live);
      if (a.live) {
        // the marks of every wavefront, OR-ed into the query tile's row (other
        // workgroups of the tile hold other heads of the group)
        uint32_t* row = a.live + (static_cast<int64_t>(pair) * nqt + i) * ((nqt + 31) / 32);
        for (int t = tid; t <= (ntile - 1) >> 5; t += 512) {
          uint32_t m = 0u;
#pragma unroll
          for (int v = 0; v < NW; ++v) m |= lds.live[v][t];
          if (m != 0u) atomicOr(row + t, m);
        }
      }
    }
  }
  if (a.refine == 0) {
    // no refinement: every causal tile is visited, and every one is live
    for (int t = tid; t < ntile; t += 512) lds.list[t] = t;
    if (tid == 0) lds.n = ntile;
    if (a.live && sub == 0) {
      uint32_t* row = a.live + (static_cast<int64_t>(pair) * nqt + i) * ((nqt + 31) / 32);
      for (int t = tid; t <= (ntile - 1) >> 5; t += 512)
        row[t] = (t < (ntile >> 5)) ? ~0u : (1u << (ntile & 31)) - 1u;
    }
    __syncthreads();
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
  const bool all_live = a.refine == 0;
  uint4 pf[QT][2];
  auto out_rel = [&](int t) { return all_live || is_live(t); };
  run(GO{}, true, [&](int t, const uint16_t* kb, const uint16_t* vb) {
    if (!out_rel(t)) return;
    scores(kb);
    mask(lds.list[t] * 64);
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      float p[4][4];
#pragma unroll
      for (int kt = 0; kt < 4; ++kt)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float d = fmaf(cx, s[kt][qt][j], -tf[qt]);
          p[kt][j] = alpha == 1.5f ? fmaxf(d, 0.f) * fmaxf(d, 0.f)
                     : alpha == 2.f ? fmaxf(d, 0.f) : mass1(d, alpha, e);
        }
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        pf[qt][kk].x = pack_bf16x2(p[2 * kk][0], p[2 * kk][1]);
        pf[qt][kk].y = pack_bf16x2(p[2 * kk][2], p[2 * kk][3]);
        pf[qt][kk].z = pack_bf16x2(p[2 * kk + 1][0], p[2 * kk + 1][1]);
        pf[qt][kk].w = pack_bf16x2(p[2 * kk + 1][2], p[2 * kk + 1][3]);
      }
    }
    // O^T += V^T P^T and the weight sums (an MFMA against ones)
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) lsum[qt] = emfma(ones, pf[qt][kk], lsum[qt]);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        typedef __attribute__((address_space(3))) ev4i16 lds_v4;
        const uint16_t* vp = vb + vfo[dt] + kk * 32 * D;
        const ev4i16 r0 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp));
        const ev4i16 r1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4*)(vp + 16 * D));
        const uint2 u0 = __builtin_bit_cast(uint2, r0), u1 = __builtin_bit_cast(uint2, r1);
        const uint4 vf = make_uint4(u0.x, u0.y, u1.x, u1.y);
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) o[dt][qt] = emfma(vf, pf[qt][kk], o[dt][qt]);
      }
    }
    __builtin_amdgcn_s_setprio(0);
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
  const int G = a.hq / a.hkv;
  const int units = G * 2;  // 32-query halves of a 64-query tile x heads of the group
  const int wpb = (units + kEw - 1) / kEw;
  const int nqt = static_cast<int>((a.n + 63) / 64);
  if (a.live) {
    const int64_t words = static_cast<int64_t>(a.batch) * a.hkv * nqt * ((nqt + 31) / 32);
    hipLaunchKernelGGL(clear_words, dim3(static_cast<unsigned>((words + 255) / 256)), dim3(256), 0,
                       stream, a.live, words);
  }
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * nqt * wpb;
  if (a.out_f32)
    hipLaunchKernelGGL((entmax_attn_bf16<D, true>), dim3(grid), dim3(kEw * 64), 0, stream, a, wpb);
  else
    hipLaunchKernelGGL((entmax_attn_bf16<D, false>), dim3(grid), dim3(kEw * 64), 0, stream, a, wpb);
  return hipGetLastError();
}

}  // namespace

int entmax_attend_max_tiles() { return kMaxKeyTiles; }

hipError_t launch_entmax_attend(const EntmaxAttnArgs& a, hipStream_t stream) {
  return a.d == 64 ? entmax_launch<64>(a, stream) : entmax_launch<128>(a, stream);
}

}  // namespace bsa
