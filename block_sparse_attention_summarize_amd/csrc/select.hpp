// Routing-row rules and exact workgroup-wide top-m selection, shared by the
// routing kernels and the fused decode kernel.
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace bsa {

struct RowInfo {
  int cand_end;  // candidates are [0, cand_end)
  int own;       // the row's own block (diagonal / tail)
  int f0, f1;    // forced blocks, -1 when absent (scalars: no private array)
  int nforced;
  int span;      // every block id that can appear in the selection is < span
  __device__ int nforced_below(int n) const { return (f0 >= 0 && f0 < n) + (f1 >= 0 && f1 < n); }
};

// Candidate range and forced blocks of one routing row, as documented in bsa.h.
__device__ inline RowInfo row_info(const RowRule& r, int b, int row) {
  RowInfo ri;
  if (r.mode != 1) {  // prefill: row = query block; token: row = query token
    ri.own = r.mode == 2 ? row / r.B : row;
    ri.cand_end = r.entmax ? ri.own : ri.own + 1;
  } else {
    int64_t L = r.kv_lens ? static_cast<int64_t>(r.kv_lens[b]) : r.kv_len;
    L = L < 1 ? 1 : (L > r.kv_len ? r.kv_len : L);
    ri.own = static_cast<int>((L - 1) / r.B);
    ri.cand_end = ri.own;
  }
  const bool first = (r.force & 2u) != 0;
  const bool own_forced = (r.force & 1u) || (r.mode == 1 && (r.force & 4u));
  ri.f0 = first ? 0 : (own_forced ? ri.own : -1);
  ri.f1 = (first && own_forced && ri.own != 0) ? ri.own : -1;
  ri.nforced = (ri.f0 >= 0) + (ri.f1 >= 0);
  ri.span = ri.own + 1 > ri.cand_end ? ri.own + 1 : ri.cand_end;
  return ri;
}

__device__ inline bool is_forced(const RowInfo& ri, int j) { return j == ri.f0 || j == ri.f1; }

// ---------------------------------------------------------------------------
// Workgroup-wide helpers for NT threads.
// ---------------------------------------------------------------------------

// Exclusive prefix count of `flag` over the workgroup in thread order.
template <int NT>
__device__ inline int block_scan(int flag, int* wave_tot, int& total) {
  constexpr int NW = NT / kWave;
  const uint64_t m = __ballot(flag);
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  if (lane == 0) wave_tot[w] = __popcll(m);
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < NW; ++k) {
    const int v = wave_tot[k];
    off += k < w ? v : 0;
    tot += v;
  }
  __syncthreads();
  total = tot;
  return off + lanes_below(m);
}

// Radix select: the key T of the m-th largest eligible element (1 <= m <=
// #eligible) and how many elements equal to T belong to the top m.
// `get(e, key)` returns whether element e is eligible and its key.
template <int NT, typename Get>
__device__ inline void radix_select(int n, int m, Get get, int* hist, int* bcast, uint32_t& T,
                                    int& need) {
  uint32_t prefix = 0, pmask = 0;
  int remaining = m;
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    for (int k = threadIdx.x; k < 256; k += NT) hist[k] = 0;
    __syncthreads();
    for (int e = threadIdx.x; e < n; e += NT) {
      uint32_t key;
      if (get(e, key) && (key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (threadIdx.x < kWave) {
      // lane l owns bins 4l..4l+3; suffix sums from the top bin down
      const int l = threadIdx.x;
      const int h0 = hist[4 * l], h1 = hist[4 * l + 1], h2 = hist[4 * l + 2], h3 = hist[4 * l + 3];
      const int own = h0 + h1 + h2 + h3;
      int incl = own;  // sum over lanes >= l
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_down(incl, o, kWave);
        incl += (l + o < kWave) ? v : 0;
      }
      const int above = incl - own;  // elements in bins above this lane's bins
      if (above < remaining && incl >= remaining) {
        int cum = above, bin = 4 * l + 3;
        const int hv[4] = {h0, h1, h2, h3};
        for (int k = 3; k >= 0; --k) {
          if (cum + hv[k] >= remaining) {
            bin = 4 * l + k;
            break;
          }
          cum += hv[k];
        }
        bcast[0] = bin;
        bcast[1] = remaining - cum;
      }
    }
    __syncthreads();
    const uint32_t bin = static_cast<uint32_t>(bcast[0]);
    remaining = bcast[1];
    prefix |= bin << shift;
    pmask |= 255u << shift;
    __syncthreads();
  }
  T = prefix;
  need = remaining;
}

// Writes the ascending selection (forced blocks + the routed top m of the
// eligible elements, ties to lower ids) to idx[0:width], pads with -1 and
// returns the count.  Elements range over [0, span).
template <int NT, typename Get, typename Out>
__device__ inline int select_and_write(const RowInfo& ri, int span, int m, int n_elig, Get get,
                                       Out out, int width, int* hist, int* bcast, int* wave_tot) {
  uint32_t T = 0;
  int need = 0;
  const bool all = m >= n_elig;
  if (!all && m > 0) radix_select<NT>(span, m, get, hist, bcast, T, need);
  int carry_eq = 0, carry_sel = 0;
  for (int base = 0; base < span; base += NT) {
    const int e = base + static_cast<int>(threadIdx.x);
    uint32_t key = 0;
    const bool elig = e < span && get(e, key);
    const bool eq = elig && !all && m > 0 && key == T;
    int tot_eq;
    const int r_eq = block_scan<NT>(eq ? 1 : 0, wave_tot, tot_eq) + carry_eq;
    bool sel;
    if (e >= span)
      sel = false;
    else if (is_forced(ri, e))
      sel = true;
    else if (!elig || m == 0)
      sel = false;
    else if (all)
      sel = true;
    else
      sel = key > T || (eq && r_eq < need);
    int tot_sel;
    const int pos = block_scan<NT>(sel ? 1 : 0, wave_tot, tot_sel) + carry_sel;
    if (sel && pos < width) out(pos, e);
    carry_eq += tot_eq;
    carry_sel += tot_sel;
  }
  for (int p = carry_sel + static_cast<int>(threadIdx.x); p < width; p += NT) out(p, -1);
  return carry_sel < width ? carry_sel : width;
}

}  // namespace bsa

namespace bsa {

// Exact top-m of up to 64*E elements held by one wavefront: element e of lane
// l is element number e*64 + l, and that number must follow the block-id order
// (lower number = lower id), so ties resolve toward the lower id.  Finds the
// m-th largest key with an MSB-first bitwise search (ballot counts, no LDS,
// no barriers), then takes every larger key and the first `need` equal keys.
// sel[e] is set for the selected elements; returns how many were selected.
// Invalid elements take key 0, below every valid key (the order-preserving
// key of a float is 0 only for a NaN with the sign bit set, which is treated
// as invalid), so the search compares keys alone.
template <int E>
__device__ inline int wave_topm(const uint32_t (&key)[E], const bool (&valid)[E], int m,
                                bool (&sel)[E]) {
  uint32_t k[E];
  int nvalid = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) {
    k[e] = valid[e] ? key[e] : 0u;
    nvalid += __popcll(__ballot(k[e] != 0u));
  }
  if (m >= nvalid) {
#pragma unroll
    for (int e = 0; e < E; ++e) sel[e] = k[e] != 0u;
    return nvalid;
  }
  if (m <= 0) {
#pragma unroll
    for (int e = 0; e < E; ++e) sel[e] = false;
    return 0;
  }
  // T ends as the m-th largest key: the largest value with >= m keys >= T.
  // Two bits per step: the counts at T|11, T|10 and T|01 (in that order they
  // can only grow) decide both bits at once, as two one-bit steps would, with
  // three independent ballot chains instead of two dependent ones.
  uint32_t T = 0;
#pragma unroll
  for (int bit = 30; bit >= 0; bit -= 2) {
    const uint32_t c3 = T | (3u << bit), c2 = T | (2u << bit), c1 = T | (1u << bit);
    int n3 = 0, n2 = 0, n1 = 0;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      n3 += __popcll(__ballot(k[e] >= c3));
      n2 += __popcll(__ballot(k[e] >= c2));
      n1 += __popcll(__ballot(k[e] >= c1));
    }
    T = n3 >= m ? c3 : (n2 >= m ? c2 : (n1 >= m ? c1 : T));
  }
  int greater = 0;
#pragma unroll
  for (int e = 0; e < E; ++e) greater += __popcll(__ballot(k[e] > T));
  const int need = m - greater;
  int before = 0;  // tied elements with a lower element number
#pragma unroll
  for (int e = 0; e < E; ++e) {
    const bool tie = k[e] == T;
    const uint64_t mk = __ballot(tie);
    const int rank = before + lanes_below(mk);
    sel[e] = k[e] > T || (tie && rank < need);
    before += __popcll(mk);
  }
  return m;
}


constexpr int kSel = 256;  // elements per wave-level selection slice (4 per lane)

// Reduces `len` (key, id) candidates held in LDS in id order (src) to their
// top-m, also in id order, by rounds of per-wave slice selections; returns
// the final count.  The result is left in `out` (mpad entries, -1 padded).
// Requires m < kSel.  `load(i, key, id, valid)` reads element i of the first
// round's source.
template <int NT, typename Load>
__device__ int tournament(int len, int m, Load load, uint32_t* bufk0, int32_t* bufi0,
                          uint32_t* bufk1, int32_t* bufi1, uint32_t* outk, int32_t* outi,
                          int mpad) {
  constexpr int NW = NT / kWave;
  __shared__ int final_count;
  const int lane = lane_id(), w = threadIdx.x / kWave;
  uint32_t* srck = nullptr;
  int32_t* srci = nullptr;
  uint32_t* dk = bufk0;
  int32_t* di = bufi0;
  bool first = true;
  for (;;) {
    const int nslice = (len + kSel - 1) / kSel;
    const bool last = nslice <= 1;
    for (int sl = w; sl < (nslice > 0 ? nslice : 1); sl += NW) {
      uint32_t key[4];
      int32_t id[4];
      bool valid[4], sel[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = sl * kSel + e * kWave + lane;
        if (first) {
          load(i, key[e], id[e], valid[e]);
          valid[e] = valid[e] && i < len;
        } else {
          valid[e] = i < len && srci[i] >= 0;
          key[e] = valid[e] ? srck[i] : 0u;
          id[e] = valid[e] ? srci[i] : -1;
        }
      }
      wave_topm<4>(key, valid, m, sel);
      uint32_t* ok = last ? outk : dk + sl * m;
      int32_t* oi = last ? outi : di + sl * m;
      const int width = last ? mpad : m;
      int base = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint64_t mk = __ballot(sel[e]);
        if (sel[e]) {
          const int pos = base + lanes_below(mk);
          ok[pos] = key[e];
          oi[pos] = id[e];
        }
        base += __popcll(mk);
      }
      for (int q = base + lane; q < width; q += kWave) oi[q] = -1;
      if (last && lane == 0) final_count = base;
    }
    __syncthreads();
    if (last) break;
    len = nslice * m;
    srck = dk;
    srci = di;
    dk = (dk == bufk0) ? bufk1 : bufk0;
    di = (di == bufi0) ? bufi1 : bufi0;
    first = false;
  }
  return final_count;
}

}  // namespace bsa
