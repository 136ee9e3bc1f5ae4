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
// wave's 1 KB block starts at lds, which must be wave-uniform).  The load is
// issued from assembly, so the compiler does not know that it writes LDS and
// inserts no wait for it before later LDS reads: it cannot tell the rotating
// tile buffers apart and would otherwise wait for every load in flight,
// including those just issued for a later tile (measured 3.5 % of the long
// prefill).  Callers order the loads with their own vmcnt waits and barriers.
// The descriptor is the one make_rsrc builds (base, stride 0, extent,
// raw-buffer flags), held in SGPRs.  Plain functions, not lambdas or
// templates, so that the host pass of every kernel that calls them sees one
// definition.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 make_desc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  u32x4 d;
  d.x = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a));
  d.y = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(a >> 32) & 0xFFFFu);
  d.z = __builtin_amdgcn_readfirstlane(bytes);
  d.w = 0x00020000u;
  return d;
}
__device__ __forceinline__ void lds_dma16(const u32x4& d, const void* lds, uint32_t voff) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(
          (const __attribute__((address_space(3))) void*)lds)));
  // M0 (the load's LDS base, read when the instruction issues) is saved and
  // restored around it, so the compiler's view of M0 is unchanged
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\tbuffer_load_dwordx4 %2, %3, 0 offen lds\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(d)
      : "memory");
}

// s_waitcnt vmcnt(N): all but the N youngest vector memory operations of this
// wave (register and direct-to-LDS loads retire in issue order) have landed.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 16, "vmcnt field");
  __builtin_amdgcn_s_waitcnt(0x0F70 | N);
}

}  // namespace bsa
