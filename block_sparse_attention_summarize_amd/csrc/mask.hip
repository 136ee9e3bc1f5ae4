// Active-block masks of 64-query tiles from per-token selections
// ("DashAttention", Estágio 2, Implementação: the attention walks the active
// blocks given by a bit-packed mask).  For every (batch, KV head, tile) the
// blocks any of the tile's tokens selected are listed in ascending order, each
// with a 64-bit word whose bit r says whether token 64 * tile + r selected it.
//
// One workgroup per tile: the tile's selection rows are contiguous, so they
// are read coalesced and OR-ed into one LDS word per block (ds_or_b64); a
// workgroup scan then compacts the non-zero words in block order.  With
// routing weights, the tile's prior bias sigma * ln w of every (listed block,
// query) is laid out next to it, -inf where the query did not select the
// block (the prior-induced softmax of Estágio 2).
#include "common.hpp"
#include "kernels.hpp"
#include "select.hpp"

namespace bsa {

namespace {

constexpr int kMaskThreads = 256;

__global__ __launch_bounds__(kMaskThreads) void token_mask_kernel(TokenMaskArgs a) {
  extern __shared__ unsigned long long words[];  // [nblk], then the bias pass's int posmap[nblk]
  __shared__ int cnts[64];
  __shared__ int wave_tot[kMaskThreads / kWave];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x % a.ntile;
  const int64_t bg = blockIdx.x / a.ntile;
  const int64_t t0 = static_cast<int64_t>(tile) * 64;
  const int ntok = a.q_len - t0 < 64 ? static_cast<int>(a.q_len - t0) : 64;
  for (int j = tid; j < a.nblk; j += kMaskThreads) words[j] = 0ull;
  if (tid < 64) {
    int c = tid < ntok ? a.cnt[bg * a.q_len + t0 + tid] : 0;
    cnts[tid] = c < 0 ? 0 : (c > a.width ? a.width : c);
  }
  __syncthreads();
  const int32_t* src = a.idx + (bg * a.q_len + t0) * a.width;
  for (int e = tid; e < ntok * a.width; e += kMaskThreads) {
    const int r = e / a.width;
    if (e - r * a.width < cnts[r]) {
      const int j = src[e];
      if (j >= 0 && j < a.nblk) atomicOr(&words[j], 1ull << r);
    }
  }
  __syncthreads();
  const int64_t out = (bg * a.ntile + tile) * a.nblk;
  int base = 0;
  for (int j0 = 0; j0 < a.nblk; j0 += kMaskThreads) {
    const int j = j0 + tid;
    const unsigned long long wv = j < a.nblk ? words[j] : 0ull;
    int tot;
    const int pos = base + block_scan<kMaskThreads>(wv != 0ull, wave_tot, tot);
    if (wv != 0ull) {
      a.uidx[out + pos] = j;
      a.ubits[out + pos] = wv;
      if (a.ubias) reinterpret_cast<int*>(words + a.nblk)[j] = pos;
    }
    base += tot;
  }
  if (a.ubias) {
    // every (listed block, query) slot starts at -inf; the selecting tokens
    // then write their own (a barrier orders the two stores to one slot)
    float* ub = a.ubias + out * 64;
    for (int e = tid; e < base * 64; e += kMaskThreads) ub[e] = -INFINITY;
    __syncthreads();
    const int* posmap = reinterpret_cast<const int*>(words + a.nblk);
    const float* wsrc = a.wsel + (bg * a.q_len + t0) * a.width;
    for (int e = tid; e < ntok * a.width; e += kMaskThreads) {
      const int r = e / a.width;
      if (e - r * a.width < cnts[r]) {
        const int j = src[e];
        if (j >= 0 && j < a.nblk) {
          const float wv = wsrc[e];
          ub[posmap[j] * 64 + r] = wv > 0.f ? a.sigma * __logf(wv) : -INFINITY;
        }
      }
    }
  }
  for (int u = base + tid; u < a.nblk; u += kMaskThreads) {
    a.uidx[out + u] = -1;
    a.ubits[out + u] = 0ull;
  }
  if (tid == 0) a.ucnt[bg * a.ntile + tile] = base;
}

}  // namespace

hipError_t launch_token_mask(const TokenMaskArgs& a, hipStream_t stream) {
  const unsigned grid = static_cast<unsigned>(a.batch) * a.hkv * a.ntile;
  const size_t lds = static_cast<size_t>(a.nblk) * (sizeof(unsigned long long) + (a.ubias ? 4 : 0));
  hipLaunchKernelGGL(token_mask_kernel, dim3(grid), dim3(kMaskThreads), lds, stream, a);
  return hipGetLastError();
}

}  // namespace bsa
