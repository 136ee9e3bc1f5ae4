// Backward of the entmax routing of prefill block rows, or of every query
// token (a row per token, its routing query the token's own query): the
// gradient of the loss with respect to the routing weights (dL/dw of the
// listed blocks, from the prior-induced softmax's backward) carried to the
// queries and keys ("DashAttention", Estágio 1: unlike top-k, entmax routing
// is differentiable, so gradients reach the block summaries of Estágio 0).
//
//   entmax_vjp_rows  one workgroup per (batch, query head, row): the listed
//                    routed block j of the head's KV group has w_j = mean over
//                    the group of p_j, so dp_j = dw_j / G; with g = p^(2-alpha)
//                    on the support, dz_j = g_j (dp_j - <g, dp> / sum g),
//                    scaled by gamma * score_scale (the logits' factor).
//   route_bwd_gemm   dqhat = dz S (over the row's candidates) and each head's
//                    part of dS_j = sum over rows of dz q-hat: fp32 products
//                    on MFMA tiles staged in LDS.
//   route_bwd_spread the mean pools' adjoint: dQ_t += dqhat_row / (tokens in
//                    the row; 1 for token rows), dK_u += (sum over the
//                    group's heads of the parts) / (tokens in the block),
//                    four elements a thread.
#include "common.hpp"
#include "kernels.hpp"

namespace bsa {

namespace {

constexpr int kVjpThreads = 256;
typedef float f32x4_t __attribute__((ext_vector_type(4)));

template <int NT>
__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (lane_id() == 0) red[w] = v;
  __syncthreads();
  float t = 0.f;
#pragma unroll
  for (int k = 0; k < NT / kWave; ++k) t += red[k];
  return t;
}

__device__ __forceinline__ float entmax_g(float p, float expo) {
  return p > 0.f ? __builtin_amdgcn_exp2f(expo * __log2f(p)) : 0.f;
}

__global__ __launch_bounds__(kVjpThreads) void entmax_vjp_rows(RouteBwdArgs a) {
  __shared__ float red[kVjpThreads / kWave];
  const int64_t hrow = blockIdx.x;  // (b * hq + h) * nrow + r
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
  for (int j = threadIdx.x; j < a.nblk; j += kVjpThreads) sg += entmax_g(p[j], expo);
  sg = block_sum<kVjpThreads>(sg, red);
  int c = a.cnt[rowid];
  c = c < 0 ? 0 : (c > a.width ? a.width : c);
  const int32_t* list = a.idx + rowid * a.width;
  const float* dw = a.dwsel + rowid * a.width;
  const float invG = 1.f / static_cast<float>(G);
  float sgd = 0.f;
  for (int e = threadIdx.x; e < c; e += kVjpThreads) {
    const int j = list[e];
    // forced blocks are no candidates (p = 0) and so carry no gradient
    if (j >= 0 && j < a.nblk) sgd += entmax_g(p[j], expo) * dw[e] * invG;
  }
  sgd = block_sum<kVjpThreads>(sgd, red);
  const float m = sg > 0.f ? sgd / sg : 0.f;
  for (int j = threadIdx.x; j < a.nblk; j += kVjpThreads)
    dz[j] = -a.fscale * entmax_g(p[j], expo) * m;
  __syncthreads();  // the listed blocks' values below replace these
  for (int e = threadIdx.x; e < c; e += kVjpThreads) {
    const int j = list[e];
    if (j >= 0 && j < a.nblk) {
      const float g = entmax_g(p[j], expo);
      if (g > 0.f) dz[j] = a.fscale * g * (dw[e] * invG - m);
    }
  }
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
  const int mt = blockIdx.x % nmt;
  const int64_t bh = blockIdx.x / nmt;  // (b, h)
  const int m0 = mt * kGT;
  const int mrows = mtot - m0 < kGT ? mtot - m0 : kGT;
  f32x4_t acc[D / 16];
#pragma unroll
  for (int ct = 0; ct < D / 16; ++ct) acc[ct] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // one K chunk of 64 staged and multiplied
  auto chunk = [&](const float* abase, int64_t am, int64_t ak, int kn, const float* bbase) {
    __syncthreads();
    for (int e = tid; e < kGT * kGT; e += 256) {
      // walk the contiguous dimension of A across neighbouring threads
      const int m = ak == 1 ? e / kGT : e % kGT;
      const int k = ak == 1 ? e % kGT : e / kGT;
      As[m][k] = (m < mrows && k < kn) ? abase[m * am + k * ak] : 0.f;
    }
    for (int e = tid; e < kGT * D; e += 256) {
      const int k = e / D, c = e % D;
      Bs[c][k] = k < kn ? bbase[static_cast<int64_t>(k) * D + c] : 0.f;
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
  if constexpr (!KEY) {
    const float* S = a.S + (b * a.hkv + g) * a.nblk * D;
    // candidates of rows m0.. are the blocks before their own blocks
    const int kend = (m0 + mrows - 1) / a.rowdiv;
    for (int k0 = 0; k0 < kend; k0 += kGT)
      chunk(a.dz + (hrow + m0) * a.nblk + k0, a.nblk, 1, kend - k0 < kGT ? kend - k0 : kGT,
            S + static_cast<int64_t>(k0) * D);
  } else {
    // rows whose own block follows block m0 hold it among their candidates
    for (int r0 = (m0 + 1) * a.rowdiv; r0 < a.nrow; r0 += kGT)
      chunk(a.dz + (hrow + r0) * a.nblk + m0, 1, a.nblk, a.nrow - r0 < kGT ? a.nrow - r0 : kGT,
            a.qhat + (hrow + r0) * D);
  }
  // lane l holds rows 16w + 4(l/16) + i, columns 16ct + l%16
  float* out = (KEY ? a.dsp + bh * a.nblk * D : a.dqh + hrow * D) + static_cast<int64_t>(m0) * D;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = 16 * w + (lane >> 4) * 4 + i;
    if (m < mrows)
#pragma unroll
      for (int ct = 0; ct < D / 16; ++ct) out[m * D + 16 * ct + (lane & 15)] = acc[ct][i];
  }
}

// The mean pools' adjoint, added to the gradient: every token of block r
// gets src[r] / (tokens of the block), summed over `parts` consecutive heads
// of src (the group's heads for dK, one head for dQ).  Four elements per
// thread; blockIdx.y is the batch.
template <typename GT>
__global__ __launch_bounds__(256) void route_bwd_spread(const float* src, int parts, void* dst,
                                                        Strides3 st, int heads, int nrow, int B,
                                                        int64_t n, int d) {
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
        src + (((b * heads + hd) * parts + p) * nrow + r) * d + c);
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

hipError_t launch_route_entmax_backward(const RouteBwdArgs& a, hipStream_t stream) {
  const unsigned rows = static_cast<unsigned>(a.batch) * a.hq * a.nrow;
  hipLaunchKernelGGL(entmax_vjp_rows, dim3(rows), dim3(kVjpThreads), 0, stream, a);
  const unsigned bh = static_cast<unsigned>(a.batch) * a.hq;
  const dim3 gq(bh * static_cast<unsigned>((a.nrow + kGT - 1) / kGT));
  const dim3 gk(bh * static_cast<unsigned>((a.nblk + kGT - 1) / kGT));
  if (a.d == 64) {
    hipLaunchKernelGGL((route_bwd_gemm<64, false>), gq, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((route_bwd_gemm<64, true>), gk, dim3(256), 0, stream, a);
  } else {
    hipLaunchKernelGGL((route_bwd_gemm<128, false>), gq, dim3(256), 0, stream, a);
    hipLaunchKernelGGL((route_bwd_gemm<128, true>), gk, dim3(256), 0, stream, a);
  }
  const int G = a.hq / a.hkv;
  auto grid_of = [&](int heads) {
    const int64_t elems = static_cast<int64_t>(heads) * a.n * a.d / 4;
    return dim3(static_cast<unsigned>((elems + 255) / 256), static_cast<unsigned>(a.batch));
  };
  if (a.g_f32) {
    hipLaunchKernelGGL(route_bwd_spread<float>, grid_of(a.hq), dim3(256), 0, stream, a.dqh, 1,
                       a.dQ, a.qs, a.hq, a.nrow, a.rowq, a.n, a.d);
    hipLaunchKernelGGL(route_bwd_spread<float>, grid_of(a.hkv), dim3(256), 0, stream, a.dsp, G,
                       a.dK, a.ks, a.hkv, a.nblk, a.B, a.n, a.d);
  } else {
    hipLaunchKernelGGL(route_bwd_spread<uint16_t>, grid_of(a.hq), dim3(256), 0, stream, a.dqh, 1,
                       a.dQ, a.qs, a.hq, a.nrow, a.rowq, a.n, a.d);
    hipLaunchKernelGGL(route_bwd_spread<uint16_t>, grid_of(a.hkv), dim3(256), 0, stream, a.dsp, G,
                       a.dK, a.ks, a.hkv, a.nblk, a.B, a.n, a.d);
  }
  return hipGetLastError();
}

}  // namespace bsa
