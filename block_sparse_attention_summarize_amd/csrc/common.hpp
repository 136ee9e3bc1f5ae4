// Device-side helpers shared by the gfx950 kernels of libbsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bsa {

constexpr int kWave = 64;

// bf16 <-> fp32.  bf16 values are carried as raw uint16 bit patterns.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}
// Round to nearest, ties to even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
// Two floats -> two bf16 (round to nearest even) in one v_cvt_pk_bf16_f32.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Load 8 consecutive elements of a row as fp32 (bf16 or fp32 storage).
template <typename T>
__device__ __forceinline__ void load8_f32(const T* p, float (&v)[8]);

template <>
__device__ __forceinline__ void load8_f32<uint16_t>(const uint16_t* p, float (&v)[8]) {
  uint4 u = *reinterpret_cast<const uint4*>(p);
  v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
  v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
  v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
  v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
}

template <>
__device__ __forceinline__ void load8_f32<float>(const float* p, float (&v)[8]) {
  float4 a = *reinterpret_cast<const float4*>(p);
  float4 b = *reinterpret_cast<const float4*>(p + 4);
  v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
  v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
}

// Butterfly reductions across `width` consecutive lanes (width a power of 2).
template <int width>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
template <int width>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = width / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}

// Sums over W consecutive lanes (W in 8, 16, 32, 64) with DPP moves inside
// 16-lane rows and gfx950 lane swaps across rows: VALU only, no LDS crossbar.
template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float swap16_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float swap16_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float swap32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
template <int W>
__device__ __forceinline__ float lane_sum(float v) {
  static_assert(W == 8 || W == 16 || W == 32 || W == 64, "lane_sum width");
  v += dppf<0xB1>(v);   // quad_perm [1,0,3,2]: lane ^ 1
  v += dppf<0x4E>(v);   // quad_perm [2,3,0,1]: lane ^ 2
  v += dppf<0x141>(v);  // row_half_mirror: the other quad of the 8-lane half
  if constexpr (W >= 16) v += dppf<0x140>(v);  // row_mirror: the other half of the row
  if constexpr (W >= 32) v = swap16_sum(v);
  if constexpr (W >= 64) v = swap32_sum(v);
  return v;
}
// Whole-wave reductions with the same DPP / lane-swap sequence (every lane
// ends with the result).  32-bit values move as they are; a double moves as
// its two halves through the same permutation.
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t v) {
  return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}
template <typename Op>
__device__ __forceinline__ uint32_t wave_reduce_u(uint32_t v, Op op) {
  v = op(v, dppu<0xB1>(v));
  v = op(v, dppu<0x4E>(v));
  v = op(v, dppu<0x141>(v));
  v = op(v, dppu<0x140>(v));
  auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
  v = op(r[0], r[1]);
  r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
  return op(r[0], r[1]);
}
__device__ __forceinline__ float wave_sum(float v) { return lane_sum<kWave>(v); }
__device__ __forceinline__ float wave_max(float v) {
  return __uint_as_float(wave_reduce_u(__float_as_uint(v), [](uint32_t x, uint32_t y) {
    return __float_as_uint(fmaxf(__uint_as_float(x), __uint_as_float(y)));
  }));
}
__device__ __forceinline__ int wave_sum_i(int v) {
  return static_cast<int>(wave_reduce_u(static_cast<uint32_t>(v), [](uint32_t x, uint32_t y) { return x + y; }));
}
template <int CTRL>
__device__ __forceinline__ double dppd(double v) {
  const uint2 u = __builtin_bit_cast(uint2, v);
  return __builtin_bit_cast(double, make_uint2(dppu<CTRL>(u.x), dppu<CTRL>(u.y)));
}
__device__ __forceinline__ double wave_sum_d(double v) {
  v += dppd<0xB1>(v);
  v += dppd<0x4E>(v);
  v += dppd<0x141>(v);
  v += dppd<0x140>(v);
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint2 u = __builtin_bit_cast(uint2, v);
    const auto lo = k == 0 ? __builtin_amdgcn_permlane16_swap(u.x, u.x, false, false)
                           : __builtin_amdgcn_permlane32_swap(u.x, u.x, false, false);
    const auto hi = k == 0 ? __builtin_amdgcn_permlane16_swap(u.y, u.y, false, false)
                           : __builtin_amdgcn_permlane32_swap(u.y, u.y, false, false);
    v = __builtin_bit_cast(double, make_uint2(lo[0], hi[0])) +
        __builtin_bit_cast(double, make_uint2(lo[1], hi[1]));
  }
  return v;
}

// Order-preserving map of fp32 to uint32: a > b (as floats) <=> key(a) > key(b).
// -0 and +0 map to distinct adjacent keys; NaN is not expected.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

// Raw buffer resource over [base, base + bytes): loads at offsets past the end
// return zeros, so ragged tails need no branches (and no serialising waits).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), 0x00020000);
}
__device__ __forceinline__ uint4 buf_load16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, static_cast<int>(off), 0, 0));
}
// Byte extent of one head's rows [0, len) with token stride st (elements).
__device__ __forceinline__ uint32_t head_bytes(int64_t len, int64_t st, int d, int esz) {
  return len < 1 ? 0u : static_cast<uint32_t>(((len - 1) * st + d) * esz);
}
// 8 consecutive elements at byte offset `off` as fp32 (bf16 or fp32 storage).
template <typename T>
__device__ __forceinline__ void buf_load8_f32(__amdgpu_buffer_rsrc_t r, uint32_t off, float (&v)[8]) {
  if constexpr (sizeof(T) == 2) {
    const uint4 u = buf_load16(r, off);
    v[0] = bf16_lo(u.x); v[1] = bf16_hi(u.x);
    v[2] = bf16_lo(u.y); v[3] = bf16_hi(u.y);
    v[4] = bf16_lo(u.z); v[5] = bf16_hi(u.z);
    v[6] = bf16_lo(u.w); v[7] = bf16_hi(u.w);
  } else {
    const uint4 a = buf_load16(r, off), b = buf_load16(r, off + 16);
    v[0] = __uint_as_float(a.x); v[1] = __uint_as_float(a.y);
    v[2] = __uint_as_float(a.z); v[3] = __uint_as_float(a.w);
    v[4] = __uint_as_float(b.x); v[5] = __uint_as_float(b.y);
    v[6] = __uint_as_float(b.z); v[7] = __uint_as_float(b.w);
  }
}

// Number of set bits of `mask` below this lane.
__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

}  // namespace bsa
