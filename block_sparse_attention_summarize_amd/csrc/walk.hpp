// Walk of a query block's selected key blocks as 64-key tiles, and the
// workgroup order of the gathered prefill kernels (forward and the query-side
// backward share both).
#pragma once

#include "common.hpp"

namespace bsa {

// Walk of the selected blocks as 64-key tiles: tile index T covers block
// idx[T / nsub] (nsub = B/64 tiles per block) at offset (T % nsub) * 64.
struct TileWalk {
  const int32_t* list;
  int n;       // number of list entries to use
  int nsub;
  int B;
  int nblk;
  int64_t kv_len;
  int64_t qmax;  // last query position of the workgroup

  // key0 of tile T, or -1 when the tile is invalid or entirely in the future.
  __device__ __forceinline__ int64_t key0(int T) const { return key0_of(list[T / nsub], T); }
  // the same with the list entry j = list[T / nsub] already read
  __device__ __forceinline__ int64_t key0_of(int j, int T) const {
    if (j < 0 || j >= nblk) return -1;
    const int64_t k0 = static_cast<int64_t>(j) * B + (T % nsub) * 64;
    if (k0 > qmax || k0 >= kv_len) return -1;
    return k0;
  }
  __device__ __forceinline__ int next(int T) const {
    for (++T; T < n * nsub; ++T)
      if (key0(T) >= 0) return T;
    return -1;
  }
};

// Map workgroup id -> (pair = b*hkv + g, query block i, sub-unit).  Heavy
// query blocks (larger i select more blocks) go first, and when the
// (batch, KV head) pairs divide evenly over the 8 XCDs (workgroups are
// dispatched round-robin over them) every workgroup of a pair lands on the
// same XCD, so the pair's K/V stays in one L2.
__device__ __forceinline__ void map_wg(int id, int npair, int nrow, int wpb, int& pair, int& i,
                                       int& sub) {
  const int total = npair * nrow * wpb;
  if (npair % 8 == 0 && total % 8 == 0) {
    const int x = id % 8, s = id / 8;
    const int per = (npair / 8) * wpb;
    const int ir = s / per, rest = s % per;
    pair = x + 8 * (rest / wpb);
    sub = rest % wpb;
    i = nrow - 1 - ir;
    return;
  }
  if (8 % npair == 0 && nrow % (8 / npair) == 0) {
    const int xpp = 8 / npair;
    const int x = id % 8, s = id / 8;
    pair = x % npair;
    const int r = x / npair;
    const int ir = (s / wpb) * xpp + r;
    sub = s % wpb;
    i = nrow - 1 - ir;
    return;
  }
  const int ir = id / (npair * wpb);
  const int rest = id % (npair * wpb);
  pair = rest / wpb;
  sub = rest % wpb;
  i = nrow - 1 - ir;
}

}  // namespace bsa
