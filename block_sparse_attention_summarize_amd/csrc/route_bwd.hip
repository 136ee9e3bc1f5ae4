// Backward of the entmax routing of prefill block rows, or of every query
// token (a row per token, its routing query the token's own query): the
// gradient of the loss with respect to the routing weights (dL/dw of the
// listed blocks, from the prior-induced softmax's backward) carried to the
// queries and keys ("DashAttention", Estágio 1: unlike top-k, entmax routing
// is differentiable, so gradients reach the block summaries of Estágio 0).
//
//   entmax_vjp_rows  one wavefront per (batch, query head, row): the listed
//                    routed block j of the head's KV group has w_j = mean over
//                    the group of p_j, so dp_j = dw_j / G; with g = p^(2-alpha)
//                    on the support, dz_j = g_j (dp_j - <g, dp> / sum g),
//                    scaled by gamma * score_scale (the logits' factor).
//   route_bwd_gemm   dqhat = dz S (over the row's candidates) and each head's
//                    part of dS_j = sum over rows of dz q-hat, the rows split
//                    into ranges of kKeyRows (one partial each, summed in
//                    order when spread): fp32 products on MFMA tiles staged in
//                    LDS.
//   route_bwd_spread the mean pools' adjoint: dQ_t += dqhat_row / (tokens in
//                    the row; 1 for token rows), dK_u += (sum over the
//                    group's heads of the parts) / (tokens in the block),
//                    four elements a thread.
#include "common.hpp"
#include "kernels.hpp"

namespace bsa {

namespace {

constexpr int kVjpThreads = 256;  // four rows a workgroup, one wavefront each
constexpr int kVjpRows = kVjpThreads / kWave;
constexpr int kKeyRows = 1024;     // rows per partial of the key-side product
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// g = p^(2-alpha) on the support (alpha = 1.5: sqrt p; alpha = 2: 1)
__device__ __forceinline__ float entmax_g(float p, float alpha, float expo) {
  if (!(p > 0.f)) return 0.f;
  if (alpha == 1.5f) return __builtin_sqrtf(p);
  if (alpha == 2.f) return 1.f;
  return __builtin_amdgcn_exp2f(expo * __log2f(p));
}

__global__ __launch_bounds__(kVjpThreads) void entmax_vjp_rows(RouteBwdArgs a, int64_t nrows) {
  extern __shared__ uint32_t listed[];  // [kVjpRows][nwords]: the row's listed blocks
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nwords = (a.nblk + 31) / 32;
  uint32_t* mark = listed + wv * nwords;
  for (int k = lane; k < nwords; k += kWave) mark[k] = 0u;
  const int64_t hrow = static_cast<int64_t>(blockIdx.x) * kVjpRows + wv;  // (b * hq + h) * nrow + r
  const bool live = hrow < nrows;
  const int r = static_cast<int>(hrow % a.nrow);
  const int64_t bh = hrow / a.nrow;
  const int h = static_cast<int>(bh % a.hq);
  const int64_t b = bh / a.hq;
  const int G = a.hq / a.hkv;
  const int64_t rowid = (b * a.hkv + h / G) * a.nrow + r;
  const float* p = a.probs + hrow * a.nblk;
  float* dz = a.dz + hrow * a.nblk;
  const float expo = 2.f - a.alpha;
  float sg = 0.f;
  if (live)
    for (int j = lane; j < a.nblk; j += kWave) sg += entmax_g(p[j], a.alpha, expo);
  sg = wave_sum(sg);
  int c = live ? a.cnt[rowid] : 0;
  c = c < 0 ? 0 : (c > a.width ? a.width : c);
  const int32_t* list = a.idx + rowid * a.width;
  const float* dw = a.dwsel + rowid * a.width;
  const float invG = 1.f / static_cast<float>(G);
  __syncthreads();  // marks cleared
  float sgd = 0.f;
  for (int e = lane; e < c; e += kWave) {
    const int j = list[e];
    // forced blocks are no candidates (p = 0) and so carry no gradient
    if (j >= 0 && j < a.nblk) {
      sgd += entmax_g(p[j], a.alpha, expo) * dw[e] * invG;
      atomicOr(&mark[j >> 5], 1u << (j & 31));
    }
  }
  sgd = wave_sum(sgd);
  __syncthreads();  // marks set
  if (!live) return;
  const float m = sg > 0.f ? sgd / sg : 0.f;
  // unlisted blocks, then the listed ones: every dz written once
  for (int j = lane; j < a.nblk; j += kWave)
    if (!((mark[j >> 5] >> (j & 31)) & 1u)) dz[j] = -a.fscale * entmax_g(p[j], a.alpha, expo) * m;
  for (int e = lane; e < c; e += kWave) {
    const int j = list[e];
    if (j >= 0 && j < a.nblk) dz[j] = a.fscale * entmax_g(p[j], a.alpha, expo) * (dw[e] * invG - m);
  }
}

// The same for rows of whole float4s (n_blk % 4 == 0, n_blk <= kVjpVecMax):
// each lane reads four probabilities at a time and keeps their g in
// registers (up to kVjpCache * 256 blocks; the rest is read again), the
// listed blocks' dw / G sit in LDS beside their marks, and dz is written in
// one pass of 16-byte stores.
constexpr int kVjpCache = 8;     // 256-block chunks whose g stay in registers
constexpr int kVjpVecMax = 3840;  // keeps the dynamic LDS within 64 KB

__global__ __launch_bounds__(kVjpThreads) void entmax_vjp_rows_vec(RouteBwdArgs a, int64_t nrows) {
  extern __shared__ uint32_t vlds[];  // [kVjpRows][nwords marks, n_blk dw / G]
  const int lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
  const int nblk = a.nblk;
  const int nwords = (nblk + 31) / 32;
  uint32_t* mark = vlds + wv * (nwords + nblk);
  float* dwl = reinterpret_cast<float*>(mark + nwords);
  for (int k = lane; k < nwords; k += kWave) mark[k] = 0u;
  const int64_t hrow = static_cast<int64_t>(blockIdx.x) * kVjpRows + wv;  // (b * hq + h) * nrow + r
  const bool live = hrow < nrows;
  const int r = static_cast<int>(hrow % a.nrow);
  const int64_t bh = hrow / a.nrow;
  const int h = static_cast<int>(bh % a.hq);
  const int64_t b = bh / a.hq;
  const int G = a.hq / a.hkv;
  const int64_t rowid = (b * a.hkv + h / G) * a.nrow + r;
  const float* p = a.probs + hrow * nblk;
  float* dz = a.dz + hrow * nblk;
  const float expo = 2.f - a.alpha;
  auto g4 = [&](int j) {
    const float4 v = *reinterpret_cast<const float4*>(p + j);
    return make_float4(entmax_g(v.x, a.alpha, expo), entmax_g(v.y, a.alpha, expo),
                       entmax_g(v.z, a.alpha, expo), entmax_g(v.w, a.alpha, expo));
  };
  float4 gc[kVjpCache];
  float sg = 0.f;
  if (live) {
#pragma unroll
    for (int ch = 0; ch < kVjpCache; ++ch) {
      const int j = ch * 256 + lane * 4;
      gc[ch] = j < nblk ? g4(j) : make_float4(0.f, 0.f, 0.f, 0.f);
      sg += (gc[ch].x + gc[ch].y) + (gc[ch].z + gc[ch].w);
    }
    for (int j = kVjpCache * 256 + lane * 4; j < nblk; j += 256) {
      const float4 gv = g4(j);
      sg += (gv.x + gv.y) + (gv.z + gv.w);
    }
  }
  sg = wave_sum(sg);
  int c = live ? a.cnt[rowid] : 0;
  c = c < 0 ? 0 : (c > a.width ? a.width : c);
  const int32_t* list = a.idx + rowid * a.width;
  const float* dw = a.dwsel + rowid * a.width;
  const float invG = 1.f / static_cast<float>(G);
  __syncthreads();  // marks cleared
  float sgd = 0.f;
  for (int e = lane; e < c; e += kWave) {
    const int j = list[e];
    // forced blocks are no candidates (p = 0) and so carry no gradient
    if (j >= 0 && j < nblk) {
      const float dv = dw[e] * invG;
      sgd += entmax_g(p[j], a.alpha, expo) * dv;
      dwl[j] = dv;
      atomicOr(&mark[j >> 5], 1u << (j & 31));
    }
  }
  sgd = wave_sum(sgd);
  __syncthreads();  // marks and dw set
  if (!live) return;
  const float m = sg > 0.f ? sgd / sg : 0.f;
  auto put = [&](int j, const float4& gv) {
    float gg[4] = {gv.x, gv.y, gv.z, gv.w};
    float o[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int jj = j + q;
      const bool listed = (mark[jj >> 5] >> (jj & 31)) & 1u;
      o[q] = a.fscale * gg[q] * ((listed ? dwl[jj] : 0.f) - m);
    }
    *reinterpret_cast<float4*>(dz + j) = make_float4(o[0], o[1], o[2], o[3]);
  };
#pragma unroll
  for (int ch = 0; ch < kVjpCache; ++ch) {
    const int j = ch * 256 + lane * 4;
    if (j < nblk) put(j, gc[ch]);
  }
  for (int j = kVjpCache * 256 + lane * 4; j < nblk; j += 256) put(j, g4(j));
}

// Batched fp32 product on MFMA tiles, C[64 x D] = A[64 x K] B[K x D] per
// workgroup, with A read through element strides (so it may be a transposed
// view of dz) and both tiles staged in LDS with K contiguous.
//   KEY = false: rows r of head h, K = the blocks before r's own block
//                r / rowdiv: A = dz[h][r][j], B = S[g][j][c] -> dqhat[h][r][c].
//   KEY = true:  rows j (key blocks), one head h of the group, K = the rows
//                whose own block follows j: A = dz[h][r][j],
//                B = qhat[h][r][c] -> that head's part of dS[g][j][c] (the
//                parts are summed when spread).
constexpr int kGT = 64;      // output rows per workgroup, K per chunk
constexpr int kGPad = 4;     // LDS row padding (floats)

template <int D, bool KEY>
__global__ __launch_bounds__(256) void route_bwd_gemm(RouteBwdArgs a) {
  constexpr int KS = kGT + kGPad;
  __shared__ float As[kGT][KS];  // [m][k]
  __shared__ float Bs[D][KS];    // [c][k]
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int G = a.hq / a.hkv;
  const int mtot = KEY ? a.nblk : a.nrow;  // output rows
  const int nmt = (mtot + kGT - 1) / kGT;
  const int ks = KEY ? static_cast<int>(blockIdx.x % a.ksplit) : 0;  // row range (key side)
  const int xi = KEY ? static_cast<int>(blockIdx.x / a.ksplit) : static_cast<int>(blockIdx.x);
  const int mt = xi % nmt;
  const int64_t bh = xi / nmt;  // (b, h)
  const int m0 = mt * kGT;
  const int mrows = mtot - m0 < kGT ? mtot - m0 : kGT;
  f32x4_t acc[D / 16];
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one K chunk of 64 staged and multiplied
  // A's contiguous dimension (k when ak == 1, else m) is read four floats at a
  // time when its stride keeps them 16-byte aligned (vec), B's rows always
  auto chunk = [&](const float* abase, int64_t am, int64_t ak, int kn, const float* bbase,
                   bool vec) {
    __syncthreads();
    if (vec) {
      for (int e = tid; e < kGT * kGT / 4; e += 256) {
        const int o = e / (kGT / 4), i4 = (e % (kGT / 4)) * 4;  // outer, inner (contiguous)
        const int m = ak == 1 ? o : i4, k = ak == 1 ? i4 : o;
        const bool in = ak == 1 ? (m < mrows && k < kn) : (k < kn && m < mrows);
        float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
        if (in) {
          const int lim = ak == 1 ? kn - k : mrows - m;  // valid elements from here
          const float* src = abase + m * am + k * ak;
          if (lim >= 4) {
            v = *reinterpret_cast<const float4*>(src);
          } else {
            const int64_t st = ak == 1 ? 1 : am;
            v.x = src[0];
            if (lim > 1) v.y = src[st];
            if (lim > 2) v.z = src[2 * st];
          }
        }
        if (ak == 1) {
          *reinterpret_cast<float4*>(&As[m][k]) = v;
        } else {
          As[m][k] = v.x;
          As[m + 1][k] = v.y;
          As[m + 2][k] = v.z;
          As[m + 3][k] = v.w;
        }
      }
    } else {
      for (int e = tid; e < kGT * kGT; e += 256) {
        // walk the contiguous dimension of A across neighbouring threads
        const int m = ak == 1 ? e / kGT : e % kGT;
        const int k = ak == 1 ? e % kGT : e / kGT;
        As[m][k] = (m < mrows && k < kn) ? abase[m * am + k * ak] : 0.f;
      }
    }
    for (int e = tid; e < kGT * D / 4; e += 256) {
      const int k = e / (D / 4), c = (e % (D / 4)) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (k < kn) v = *reinterpret_cast<const float4*>(bbase + static_cast<int64_t>(k) * D + c);
      Bs[c][k] = v.x;
      Bs[c + 1][k] = v.y;
      Bs[c + 2][k] = v.z;
      Bs[c + 3][k] = v.w;
    }
    __syncthreads();
    const int lr = lane & 15, lk = (lane >> 4) * 4;
#pragma unroll 4
    for (int kc = 0; kc < kGT; kc += 16) {
      const float4 av = *reinterpret_cast<const float4*>(&As[16 * w + lr][kc + lk]);
#pragma unroll
      for (int ct = 0; ct < D / 16; ++ct) {
        const float4 bv = *reinterpret_cast<const float4*>(&Bs[16 * ct + lr][kc + lk]);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.x, bv.x, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.y, bv.y, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.z, bv.z, acc[ct], 0, 0, 0);
        acc[ct] = __builtin_amdgcn_mfma_f32_16x16x4f32(av.w, bv.w, acc[ct], 0, 0, 0);
      }
    }
  };

  const int64_t b = bh / a.hq;
  const int h = static_cast<int>(bh % a.hq), g = h / G;
  const int64_t hrow = bh * a.nrow;
  const bool vec = a.nblk % 4 == 0;  // dz rows of whole float4s
  if constexpr (!KEY) {
    const float* S = a.S + (b * a.hkv + g) * a.nblk * D;
    // candidates of rows m0.. are the blocks before their own blocks
    const int kend = (m0 + mrows - 1) / a.rowdiv;
    for (int k0 = 0; k0 < kend; k0 += kGT)
      chunk(a.dz + (hrow + m0) * a.nblk + k0, a.nblk, 1, kend - k0 < kGT ? kend - k0 : kGT,
            S + static_cast<int64_t>(k0) * D, vec);
  } else {
    // rows whose own block follows block m0 hold it among their candidates;
    // this workgroup takes those in its range
    const int rend = min(a.nrow, (ks + 1) * kKeyRows);
    for (int r0 = max((m0 + 1) * a.rowdiv, ks * kKeyRows); r0 < rend; r0 += kGT)
      chunk(a.dz + (hrow + r0) * a.nblk + m0, 1, a.nblk, rend - r0 < kGT ? rend - r0 : kGT,
            a.qhat + (hrow + r0) * D, vec);
  }
  // lane l holds rows 16w + 4(l/16) + i, columns 16ct + l%16 (the key side's
  // empty ranges store zeros)
  float* out = (KEY ? a.dsp + (bh * a.ksplit + ks) * a.nblk * D : a.dqh + hrow * D) +
               static_cast<int64_t>(m0) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 16 * w + (lane >> 4) * 4 + i;
    if (m < mrows)
#pragma unroll
      for (int ct = 0; ct < D / 16; ++ct) out[m * D + 16 * ct + (lane & 15)] = acc[ct][i];
  }
}

// The key side's partials of one KV head (its heads' and row ranges' parts)
// summed in order into the first part, so that the tokens of a block read
// one value instead of every part.  Four elements per thread.
__global__ __launch_bounds__(256) void route_bwd_sum_parts(float* dsp, int parts, int64_t slab,
                                                           int64_t total) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;  // in [groups, slab]
  if (e >= total) return;
  const int64_t grp = e / slab, off = e % slab;
  float* base = dsp + grp * parts * slab + off;
  float4 v = *reinterpret_cast<const float4*>(base);
  for (int p = 1; p < parts; ++p) {
    const float4 x = *reinterpret_cast<const float4*>(base + p * slab);
    v.x += x.x;
    v.y += x.y;
    v.z += x.z;
    v.w += x.w;
  }
  *reinterpret_cast<float4*>(base) = v;
}

// The mean pools' adjoint, added to the gradient: every token of block r
// gets src[r] / (tokens of the block), summed over the first `parts` of the
// `pstride` consecutive parts of each head of src (the group's heads for dK,
// one head for dQ).  Four elements per thread; blockIdx.y is the batch.
template <typename GT>
__global__ __launch_bounds__(256) void route_bwd_spread(const float* src, int parts, int pstride,
                                                        void* dst, Strides3 st, int heads,
                                                        int nrow, int B, int64_t n, int d) {
  const int64_t e = (static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x) * 4;
  const int64_t per_head = n * d;
  if (e >= heads * per_head) return;
  const int64_t b = blockIdx.y, hd = e / per_head;
  const int64_t rem = e % per_head;
  const int64_t t = rem / d;
  const int c = static_cast<int>(rem % d);
  const int r = static_cast<int>(t / B);
  const int nt = static_cast<int>(n - static_cast<int64_t>(r) * B < B ? n - static_cast<int64_t>(r) * B : B);
  float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
  for (int p = 0; p < parts; ++p) {
    const float4 x = *reinterpret_cast<const float4*>(
        src + (((b * heads + hd) * pstride + p) * nrow + r) * d + c);
    v.x += x.x;
    v.y += x.y;
    v.z += x.z;
    v.w += x.w;
  }
  const float inv = 1.f / static_cast<float>(nt);
  const int64_t off = b * st.b + hd * st.h + t * st.t + c;
  if constexpr (sizeof(GT) == 4) {
    float4* q = reinterpret_cast<float4*>(static_cast<float*>(dst) + off);
    float4 o = *q;
    o.x += v.x * inv;
    o.y += v.y * inv;
    o.z += v.z * inv;
    o.w += v.w * inv;
    *q = o;
  } else {
    uint2* q = reinterpret_cast<uint2*>(static_cast<uint16_t*>(dst) + off);
    const uint2 o = *q;
    *q = make_uint2(pack_bf16x2(bf16_lo(o.x) + v.x * inv, bf16_hi(o.x) + v.y * inv),
                    pack_bf16x2(bf16_lo(o.y) + v.z * inv, bf16_hi(o.y) + v.w * inv));
  }
}

}  // namespace

int route_bwd_key_splits(int nrow) { return (nrow + kKeyRows - 1) / kKeyRows; }

hipError_t launch_route_entmax_backward(const RouteBwdArgs& a, hipStream_t stream) {
  const int64_t rows = static_cast<int64_t>(a.batch) * a.hq * a.nrow;
  const unsigned vgrid = static_cast<unsigned>((rows + kVjpRows - 1) / kVjpRows);
  if (a.nblk % 4 == 0 && a.nblk <= kVjpVecMax) {
    const size_t lds_bytes = static_cast<size_t>(kVjpRows) * ((a.nblk + 31) / 32 + a.nblk) * 4;
    hipLaunchKernelGGL(entmax_vjp_rows_vec, dim3(vgrid), dim3(kVjpThreads), lds_bytes, stream, a, rows);
  } else {
    const size_t mark_bytes = static_cast<size_t>(kVjpRows) * ((a.nblk + 31) / 32) * 4;
    hipLaunchKernelGGL(entmax_vjp_rows, dim3(vgrid), dim3(kVjpThreads), mark_bytes, stream, a, rows);
  }
  const unsigned bh = static_cast<unsigned>(a.batch) * a.hq;
  const dim3 gq(bh * static_cast<unsigned>((a.nrow + kGT - 1) / kGT));
  const dim3 gk(bh * static_cast<unsigned>((a.nblk + kGT - 1) / kGT) * a.ksplit);
  if (a.d == 64) {
    hipLaunchKernelGGL((route_bwd_gemm<64, false>), gq, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((route_bwd_gemm<64, true>), gk, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((route_bwd_gemm<128, false>), gq, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((route_bwd_gemm<128, true>), gk, dim3(256), 0, stream, a);
  }
  const int G = a.hq / a.hkv;
  // many key-side parts (row ranges): summed once per KV head first
  const int kparts = G * a.ksplit;
  const int ksum = a.ksplit > 1 ? 1 : kparts;
  if (a.ksplit > 1) {
    const int64_t slab = static_cast<int64_t>(a.nblk) * a.d;
    const int64_t total = static_cast<int64_t>(a.batch) * a.hkv * slab;
    hipLaunchKernelGGL(route_bwd_sum_parts, dim3(static_cast<unsigned>((total / 4 + 255) / 256)),
                       dim3(256), 0, stream, a.dsp, kparts, slab, total);
  }
  auto grid_of = [&](int heads) {
    const int64_t elems = static_cast<int64_t>(heads) * a.n * a.d / 4;
    return dim3(static_cast<unsigned>((elems + 255) / 256), static_cast<unsigned>(a.batch));
  };
  if (a.g_f32) {
    hipLaunchKernelGGL(route_bwd_spread<float>, grid_of(a.hq), dim3(256), 0, stream, a.dqh, 1, 1,
                       a.dQ, a.qs, a.hq, a.nrow, a.rowq, a.n, a.d);
    hipLaunchKernelGGL(route_bwd_spread<float>, grid_of(a.hkv), dim3(256), 0, stream, a.dsp,
                       ksum, kparts, a.dK, a.ks, a.hkv, a.nblk, a.B, a.n, a.d);
  } else {
    hipLaunchKernelGGL(route_bwd_spread<uint16_t>, grid_of(a.hq), dim3(256), 0, stream, a.dqh, 1,
                       1, a.dQ, a.qs, a.hq, a.nrow, a.rowq, a.n, a.d);
    hipLaunchKernelGGL(route_bwd_spread<uint16_t>, grid_of(a.hkv), dim3(256), 0, stream, a.dsp,
                       ksum, kparts, a.dK, a.ks, a.hkv, a.nblk, a.B, a.n, a.d);
  }
  return hipGetLastError();
}

}  // namespace bsa
