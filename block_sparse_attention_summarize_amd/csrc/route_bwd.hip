// Backward of the entmax routing of prefill block rows: the gradient of the
// loss with respect to the routing weights (dL/dw of the listed blocks, from
// the prior-induced softmax's backward) carried to the queries and keys
// ("DashAttention", Estágio 1: unlike top-k, entmax routing is
// differentiable, so gradients reach the block summaries of Estágio 0).
//
//   entmax_vjp_rows  one workgroup per (batch, query head, row): the listed
//                    routed block j of the head's KV group has w_j = mean over
//                    the group of p_j, so dp_j = dw_j / G; with g = p^(2-alpha)
//                    on the support, dz_j = g_j (dp_j - <g, dp> / sum g),
//                    scaled by gamma * score_scale (the logits' factor).
//   route_bwd_q      dqhat = dz S (over the row's candidates), spread over the
//                    row's queries: dQ_t += dqhat / (tokens in the row).
//   route_bwd_k      dS_j = sum over the group's heads and rows of dz q-hat,
//                    spread over the block's keys: dK_u += dS / (tokens).
#include "common.hpp"
#include "kernels.hpp"

namespace bsa {

namespace {

constexpr int kVjpThreads = 256;

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

template <typename T>
__device__ __forceinline__ void add_to(void* base, int64_t off, float v) {
  if constexpr (sizeof(T) == 4) {
    static_cast<float*>(base)[off] += v;
  } else {
    uint16_t* q = static_cast<uint16_t*>(base) + off;
    *q = f32_to_bf16(bf16_to_f32(*q) + v);
  }
}

// One workgroup (d threads) per (batch, query head, row).
template <typename GT>
__global__ __launch_bounds__(128) void route_bwd_q(RouteBwdArgs a) {
  const int64_t hrow = blockIdx.x;
  const int r = static_cast<int>(hrow % a.nrow);
  const int64_t bh = hrow / a.nrow;
  const int h = static_cast<int>(bh % a.hq);
  const int64_t b = bh / a.hq;
  const int g = h / (a.hq / a.hkv);
  const int c = threadIdx.x;
  const float* dz = a.dz + hrow * a.nblk;
  const float* S = a.S + (b * a.hkv + g) * a.nblk * a.d;
  float acc0 = 0.f, acc1 = 0.f;
  // candidates are the blocks before the row's own
  int j = 0;
  for (; j + 1 < r; j += 2) {
    acc0 = fmaf(dz[j], S[static_cast<int64_t>(j) * a.d + c], acc0);
    acc1 = fmaf(dz[j + 1], S[static_cast<int64_t>(j + 1) * a.d + c], acc1);
  }
  if (j < r) acc0 = fmaf(dz[j], S[static_cast<int64_t>(j) * a.d + c], acc0);
  const int64_t t0 = static_cast<int64_t>(r) * a.B;
  const int nr = static_cast<int>(a.n - t0 < a.B ? a.n - t0 : a.B);
  const float v = (acc0 + acc1) / static_cast<float>(nr);
  const int64_t base = b * a.qs.b + h * a.qs.h;
  for (int t = 0; t < nr; ++t) add_to<GT>(a.dQ, base + (t0 + t) * a.qs.t + c, v);
}

// One workgroup (d threads) per (batch, KV head, key block).
template <typename GT>
__global__ __launch_bounds__(128) void route_bwd_k(RouteBwdArgs a) {
  const int j = static_cast<int>(blockIdx.x % a.nblk);
  const int64_t bg = blockIdx.x / a.nblk;
  const int g = static_cast<int>(bg % a.hkv);
  const int64_t b = bg / a.hkv;
  const int G = a.hq / a.hkv;
  const int c = threadIdx.x;
  float acc0 = 0.f, acc1 = 0.f;
  for (int hh = 0; hh < G; ++hh) {
    const int64_t hb = (b * a.hq + g * G + hh) * a.nrow;
    // rows after j have block j among their candidates
    int r = j + 1;
    for (; r + 1 < a.nrow; r += 2) {
      acc0 = fmaf(a.dz[(hb + r) * a.nblk + j], a.qhat[(hb + r) * a.d + c], acc0);
      acc1 = fmaf(a.dz[(hb + r + 1) * a.nblk + j], a.qhat[(hb + r + 1) * a.d + c], acc1);
    }
    if (r < a.nrow) acc0 = fmaf(a.dz[(hb + r) * a.nblk + j], a.qhat[(hb + r) * a.d + c], acc0);
  }
  const int64_t u0 = static_cast<int64_t>(j) * a.B;
  const int nj = static_cast<int>(a.n - u0 < a.B ? a.n - u0 : a.B);
  const float v = (acc0 + acc1) / static_cast<float>(nj);
  const int64_t base = b * a.ks.b + g * a.ks.h;
  for (int u = 0; u < nj; ++u) add_to<GT>(a.dK, base + (u0 + u) * a.ks.t + c, v);
}

}  // namespace

hipError_t launch_route_entmax_backward(const RouteBwdArgs& a, hipStream_t stream) {
  const unsigned rows = static_cast<unsigned>(a.batch) * a.hq * a.nrow;
  hipLaunchKernelGGL(entmax_vjp_rows, dim3(rows), dim3(kVjpThreads), 0, stream, a);
  const unsigned kblocks = static_cast<unsigned>(a.batch) * a.hkv * a.nblk;
  if (a.g_f32) {
    hipLaunchKernelGGL(route_bwd_q<float>, dim3(rows), dim3(a.d), 0, stream, a);
    hipLaunchKernelGGL(route_bwd_k<float>, dim3(kblocks), dim3(a.d), 0, stream, a);
  } else {
    hipLaunchKernelGGL(route_bwd_q<uint16_t>, dim3(rows), dim3(a.d), 0, stream, a);
    hipLaunchKernelGGL(route_bwd_k<uint16_t>, dim3(kblocks), dim3(a.d), 0, stream, a);
  }
  return hipGetLastError();
}

}  // namespace bsa
