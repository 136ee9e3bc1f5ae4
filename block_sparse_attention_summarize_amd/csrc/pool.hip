// Stage 0 and the routing-query pool: bandwidth-bound reductions over blocks
// of B tokens ("DashAttention", Estágio 0: a block summary is the mean of the
// block's keys when the learned query is zero, or its local softmax-weighted
// average otherwise).
//
// One workgroup of 256 threads per (batch, head, block).  Every thread loads
// 16-byte (bf16) or 32-byte (fp32) slices of a row, so a row of d elements is
// covered by d/8 consecutive threads and a wavefront reads whole rows
// back-to-back (fully coalesced).  Partial sums of the row groups meet in LDS.
#include "common.hpp"
#include "kernels.hpp"

namespace bsa {

namespace {

constexpr int kThreads = 256;

template <typename T, int D, bool LEARNED>
__global__ __launch_bounds__(kThreads) void summarize_kernel(SummarizeArgs a) {
  constexpr int TPR = D / 8;           // threads per row
  constexpr int RG = kThreads / TPR;   // row groups
  __shared__ float red[RG][D];
  __shared__ float wts[128];

  const int tid = threadIdx.x;
  // all blocks: one workgroup per (b, g, block); one block per sequence:
  // one workgroup per (b, g) for the block blk[b] (none when out of range)
  const int bg = a.blk ? static_cast<int>(blockIdx.x) : static_cast<int>(blockIdx.x) / a.nblk;
  const int g = bg % a.hkv;
  const int b = bg / a.hkv;
  const int j = a.blk ? a.blk[b] : static_cast<int>(blockIdx.x) % a.nblk;
  if (j < 0 || j >= a.nblk) return;
  const int64_t t0 = static_cast<int64_t>(j) * a.B;
  const int64_t rem = a.kv_len - t0;
  const int cnt = static_cast<int>(rem < a.B ? rem : a.B);
  const T* base = static_cast<const T*>(a.K) + b * a.ks.b + g * a.ks.h + t0 * a.ks.t;
  if (a.table) {  // paged cache: the block's page holds its B rows
    if (j >= a.max_pages) return;
    const int pg = a.table[static_cast<int64_t>(b) * a.max_pages + j];
    if (pg < 0 || pg >= a.num_pages) return;
    base = static_cast<const T*>(a.K) + static_cast<int64_t>(pg) * a.page_k + g * a.ks.h;
  }
  const int c = tid % TPR;
  const int r0 = tid / TPR;

  if constexpr (LEARNED) {
    // weights w_t = softmax_t(qbar . k_t / sqrt(d)) over the block's tokens
    float qv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) qv[e] = a.qbar[g * D + c * 8 + e];
    const float sc = rsqrtf(static_cast<float>(D));
    for (int r = r0; r < cnt; r += RG) {
      float kv[8];
      load8_f32<T>(base + r * a.ks.t + c * 8, kv);
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 8; ++e) s = fmaf(qv[e], kv[e], s);
      s = group_sum<TPR>(s);
      if (c == 0) wts[r] = s * sc;
    }
    __syncthreads();
    float mx = -INFINITY;
    for (int r = 0; r < cnt; ++r) mx = fmaxf(mx, wts[r]);
    float z = 0.f;
    for (int r = 0; r < cnt; ++r) z += __expf(wts[r] - mx);
    __syncthreads();
    for (int r = tid; r < cnt; r += kThreads) wts[r] = __expf(wts[r] - mx) / z;
    __syncthreads();
  }

  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int r = r0; r < cnt; r += RG) {
    float kv[8];
    load8_f32<T>(base + r * a.ks.t + c * 8, kv);
    const float w = LEARNED ? wts[r] : 1.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = fmaf(w, kv[e], acc[e]);
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r0][c * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) s += red[r][tid];
    if (!LEARNED) s = s / static_cast<float>(cnt);
    a.S[(static_cast<int64_t>(bg) * a.nblk + j) * D + tid] = s;
  }
}

// Routing query: per row, sum over `nh` heads of the mean over the block's
// queries (nh = group size for top-k, 1 for entmax).
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void qpool_kernel(QPoolArgs a) {
  constexpr int TPR = D / 8;
  constexpr int RG = kThreads / TPR;
  __shared__ float red[RG][D];
  const int tid = threadIdx.x;
  const int nout = a.group_sum ? a.hkv : a.hq;
  const int nh = a.group_sum ? a.hq / a.hkv : 1;
  const int i = blockIdx.x % a.nrow;
  const int bo = blockIdx.x / a.nrow;
  const int o = bo % nout;
  const int b = bo / nout;
  const int64_t t0 = static_cast<int64_t>(i) * a.B;
  const int64_t rem = a.q_len - t0;
  const int cnt = static_cast<int>(rem < a.B ? rem : a.B);
  const int c = tid % TPR;
  const int r0 = tid / TPR;
  float acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = 0.f;
  for (int hh = 0; hh < nh; ++hh) {
    const int h = o * nh + hh;
    const T* base = static_cast<const T*>(a.Q) + b * a.qs.b + h * a.qs.h + t0 * a.qs.t;
    for (int r = r0; r < cnt; r += RG) {
      float qv[8];
      load8_f32<T>(base + r * a.qs.t + c * 8, qv);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[e] += qv[e];
    }
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) red[r0][c * 8 + e] = acc[e];
  __syncthreads();
  if (tid < D) {
    float s = 0.f;
#pragma unroll
    for (int r = 0; r < RG; ++r) s += red[r][tid];
    a.qhat[(static_cast<int64_t>(bo) * a.nrow + i) * D + tid] = s / static_cast<float>(cnt);
  }
}

// Per-token routing query (rows of one token): q-hat[b, o, t] = sum over the
// nh heads of group o of q[b, h, t], one thread per 8 elements of a row.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void qtok_kernel(QPoolArgs a, int64_t total) {
  constexpr int CPR = D / 8;
  const int64_t e = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
  if (e >= total) return;
  const int nout = a.group_sum ? a.hkv : a.hq;
  const int nh = a.group_sum ? a.hq / a.hkv : 1;
  const int c = static_cast<int>(e % CPR);
  const int64_t r = e / CPR;  // (b, o, t)
  const int64_t t = r % a.q_len;
  const int64_t bo = r / a.q_len;
  const int o = static_cast<int>(bo % nout);
  const int64_t b = bo / nout;
  float acc[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) acc[k] = 0.f;
  for (int hh = 0; hh < nh; ++hh) {
    float qv[8];
    load8_f32<T>(static_cast<const T*>(a.Q) + b * a.qs.b + (o * nh + hh) * a.qs.h + t * a.qs.t +
                     c * 8,
                 qv);
#pragma unroll
    for (int k = 0; k < 8; ++k) acc[k] += qv[k];
  }
  float4* out = reinterpret_cast<float4*>(a.qhat + r * D + c * 8);
  out[0] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  out[1] = make_float4(acc[4], acc[5], acc[6], acc[7]);
}

template <typename T, int D>
hipError_t summarize_dispatch(const SummarizeArgs& a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * (a.blk ? 1 : a.nblk);
  if (a.qbar)
    hipLaunchKernelGGL((summarize_kernel<T, D, true>), dim3(grid), dim3(kThreads), 0, stream, a);
  else
    hipLaunchKernelGGL((summarize_kernel<T, D, false>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t qpool_dispatch(const QPoolArgs& a, hipStream_t stream) {
  const int nout = a.group_sum ? a.hkv : a.hq;
  if (a.B == 1) {
    const int64_t total = static_cast<int64_t>(a.batch) * nout * a.q_len * (D / 8);
    const unsigned grid = static_cast<unsigned>((total + kThreads - 1) / kThreads);
    hipLaunchKernelGGL((qtok_kernel<T, D>), dim3(grid), dim3(kThreads), 0, stream, a, total);
    return hipGetLastError();
  }
  const unsigned grid = static_cast<unsigned>(a.batch) * nout * a.nrow;
  hipLaunchKernelGGL((qpool_kernel<T, D>), dim3(grid), dim3(kThreads), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_summarize(const SummarizeArgs& a, hipStream_t stream) {
  if (a.bf16) {
    return a.d == 64 ? summarize_dispatch<uint16_t, 64>(a, stream)
                     : summarize_dispatch<uint16_t, 128>(a, stream);
  }
  return a.d == 64 ? summarize_dispatch<float, 64>(a, stream)
                   : summarize_dispatch<float, 128>(a, stream);
}

hipError_t launch_qpool(const QPoolArgs& a, hipStream_t stream) {
  if (a.bf16) {
    return a.d == 64 ? qpool_dispatch<uint16_t, 64>(a, stream)
                     : qpool_dispatch<uint16_t, 128>(a, stream);
  }
  return a.d == 64 ? qpool_dispatch<float, 64>(a, stream) : qpool_dispatch<float, 128>(a, stream);
}

}  // namespace bsa
