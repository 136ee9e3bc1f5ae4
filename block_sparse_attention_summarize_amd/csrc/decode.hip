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
// Phase A: the selected blocks are streamed in 32-key chunks, each wavefront
// keeping an online softmax per query head; the wavefronts' partial states
// are merged in LDS.  Decode is bound by HBM transfers (summaries + the
// selected K/V), so everything stays on the VALU.
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

template <typename T, int D, int GS>
__global__ __launch_bounds__(kNT) void decode_fused(DecodeArgs a) {
  constexpr int LPK = D / 8;       // lanes per key row (8 elements each)
  constexpr int KPI = kWave / LPK;  // keys per wave load instruction
  constexpr int KPC = 32 / KPI;     // load instructions per 32-key chunk
  constexpr int LPR = D / 4;       // lanes per fp32 summary row
  constexpr int RPW = kWave / LPR;  // summary rows per wave load instruction
  extern __shared__ float dyn[];    // [nblk] scores, then the merge buffer
  __shared__ float qh[D];
  __shared__ float qa[GS][D];
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

  if (a.route) {
    // routing query: sum of the group's query heads
    for (int c = tid; c < D; c += kNT) {
      float s = 0.f;
      for (int hh = 0; hh < G; ++hh) {
        const T* qp = Qb + (g * G + hh) * a.qs.h;
        if constexpr (sizeof(T) == 2)
          s += bf16_to_f32(qp[c]);
        else
          s += qp[c];
      }
      qh[c] = s;
    }
    __syncthreads();
    RowRule rule;
    rule.mode = 1;
    rule.entmax = 0;
    rule.force = a.force;
    rule.B = a.B;
    rule.kv_len = a.kv_len;
    rule.kv_lens = a.kv_lens;
    const RowInfo ri = row_info(rule, b, 0);
    const int n = ri.cand_end;
    // stream the summaries of the candidates, kUnroll loads in flight per lane
    const int c4 = lane % LPR;
    const float4 q4 = reinterpret_cast<const float4*>(qh)[c4];
    const auto rs = make_rsrc(a.S + static_cast<int64_t>(row) * a.nblk * D,
                              static_cast<uint32_t>(n) * D * 4);  // candidates only
    constexpr int STEP = kNW * RPW;  // rows per workgroup load round
    for (int base = 0; base < n; base += STEP * kUnroll) {
      uint4 v[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const uint32_t j = static_cast<uint32_t>(base + u * STEP + w * RPW + lane / LPR);
        v[u] = buf_load16(rs, j * (D * 4) + c4 * 16);  // rows >= n read as zero
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        const int j = base + u * STEP + w * RPW + lane / LPR;
        float p = q4.x * __uint_as_float(v[u].x);
        p = fmaf(q4.y, __uint_as_float(v[u].y), p);
        p = fmaf(q4.z, __uint_as_float(v[u].z), p);
        p = fmaf(q4.w, __uint_as_float(v[u].w), p);
        p = lane_sum<LPR>(p);
        if (c4 == 0 && j < n) dyn[j] = p * a.score_scale;
      }
    }
    __syncthreads();
    int n_elig = n;
    for (int f = 0; f < ri.nforced; ++f) n_elig -= ri.forced[f] < n ? 1 : 0;
    int m = a.k_total - ri.nforced;
    m = m < 0 ? 0 : m;
    auto get = [&](int e, uint32_t& key) -> bool {
      if (e >= n || is_forced(ri, e)) return false;
      key = float_key(dyn[e]);
      return true;
    };
    int32_t* gidx = a.idx ? a.idx + static_cast<int64_t>(row) * a.k_total : nullptr;
    const bool write = gidx != nullptr && hs == 0;
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
  } else {
    int c = a.cnt[row];
    c = c < 0 ? 0 : (c > a.k_total ? a.k_total : c);
    for (int p = tid; p < c; p += kNT) sel[p] = a.idx[static_cast<int64_t>(row) * a.k_total + p];
    if (tid == 0) sel_n = c;
    __syncthreads();
  }
  if (!a.attend) return;

  // ---- attention over the selected blocks for heads h0 .. h0+gs-1 ----
  const float scl = a.sm_scale * kLog2e;
  for (int e = tid; e < gs * D; e += kNT) {
    const int hh = e / D, c = e % D;
    const T* qp = Qb + (h0 + hh) * a.qs.h;
    float v;
    if constexpr (sizeof(T) == 2)
      v = bf16_to_f32(qp[c]);
    else
      v = qp[c];
    qa[hh][c] = v * scl;
  }
  __syncthreads();
  const int nsel = sel_n;
  const int cpb = a.B / 32;  // 32-key chunks per block
  const int nchunk = nsel * cpb;
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
  for (int ch = w; ch < nchunk; ch += kNW) {
    const int j = sel[ch / cpb];
    if (j < 0 || j >= a.nblk) continue;
    const int t0 = j * a.B + (ch % cpb) * 32;
    float kv[KPC][8], vv[KPC][8];
    bool ok[KPC];
#pragma unroll
    for (int it = 0; it < KPC; ++it) {
      const int t = t0 + it * KPI + kg;
      ok[it] = t < L;
      buf_load8_f32<T>(rk, static_cast<uint32_t>(t) * kst + c8 * 8 * sizeof(T), kv[it]);
    }
#pragma unroll
    for (int it = 0; it < KPC; ++it) {
      const int t = t0 + it * KPI + kg;
      buf_load8_f32<T>(rv, static_cast<uint32_t>(t) * vst + c8 * 8 * sizeof(T), vv[it]);
    }
#pragma unroll
    for (int hh = 0; hh < GS; ++hh) {
      if (hh >= gs) break;
      float s[KPC];
      float mx = -INFINITY;
#pragma unroll
      for (int it = 0; it < KPC; ++it) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc = fmaf(kv[it][e], qa[hh][c8 * 8 + e], acc);
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
        ls += p;
#pragma unroll
        for (int e = 0; e < 8; ++e) o[hh][e] = fmaf(p, vv[it][e], o[hh][e]);
      }
      l[hh] = l[hh] * f + ls;
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

template <typename T, int D, int GS>
hipError_t launch_gs(const DecodeArgs& a, hipStream_t stream) {
  const size_t dyn = static_cast<size_t>(a.lds_floats) * 4 + static_cast<size_t>(a.k_total) * 4;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&decode_fused<T, D, GS>),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, 96 * 1024);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * a.hsplit;
  hipLaunchKernelGGL((decode_fused<T, D, GS>), dim3(grid), dim3(kNT), dyn, stream, a);
  return hipGetLastError();
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

hipError_t launch_decode_fused(const DecodeArgs& a, hipStream_t stream) {
  if (a.bf16) return a.d == 64 ? launch_t<uint16_t, 64>(a, stream) : launch_t<uint16_t, 128>(a, stream);
  return a.d == 64 ? launch_t<float, 64>(a, stream) : launch_t<float, 128>(a, stream);
}

}  // namespace bsa
