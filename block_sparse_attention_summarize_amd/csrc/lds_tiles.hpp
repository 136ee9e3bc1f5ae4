// 64-row bf16 tiles staged in LDS by direct-to-LDS buffer loads, for the
// attention kernels that stage K and V that way.  Rows are unpadded; the
// 16-byte chunks of a row are XOR-swizzled so that the MFMA fragment reads
// hit every bank once:
//   K fragments (16 rows x 16 bytes per half-wave): chunk p of row r sits at
//     p ^ kswz(r);
//   V transposing reads (ds_read_b64_tr_b16, 8 rows x 32 bytes per half-wave):
//     chunk p of row r sits at p ^ vswz(r), an even XOR so that a 32-byte pair
//     of chunks stays adjacent.
#pragma once

#include "common.hpp"

namespace bsa {

template <int D>
struct SwzTile {
  static constexpr int NC = D / 8;     // 16-byte chunks per row
  static constexpr int RPL = 16 / NC;  // rows per 256-byte bank line
  __host__ __device__ static constexpr int kswz(int r) { return (r / RPL) & (NC - 1); }
  __host__ __device__ static constexpr int vswz(int r) { return ((r / RPL) & (NC / 2 - 1)) << 1; }
};
static_assert(SwzTile<128>::kswz(16) == SwzTile<128>::kswz(0) &&
                  SwzTile<128>::vswz(16) == SwzTile<128>::vswz(0) &&
                  SwzTile<64>::kswz(16) == SwzTile<64>::kswz(0) &&
                  SwzTile<64>::vswz(16) == SwzTile<64>::vswz(0),
              "swizzles repeat every 16 rows");

// 16 bytes per lane from buffer offset voff into LDS at lds + 16 * lane (the
// wave's 1 KB block starts at lds, which must be wave-uniform).  A plain
// function, not a lambda or template, so that the host pass of every kernel
// that calls it sees one definition.
__device__ __forceinline__ void lds_dma16(__amdgpu_buffer_rsrc_t r, void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16,
                                           voff, 0, 0, 0);
}

// s_waitcnt vmcnt(N): all but the N youngest vector memory operations of this
// wave (register and direct-to-LDS loads retire in issue order) have landed.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

}  // namespace bsa
