// Device helpers shared by the gfx950 kernels of libswa: vector types,
// bf16 <-> fp32 conversion, DPP lane reductions, XCD-aware work mapping.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace swa {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr float kLog2e = 1.4426950408889634f;

// Workgroup and work-item indices read straight from the hardware registers.
// Under this library's float flags (no IEEE mode) the blockIdx / threadIdx
// accessors stay calls into the device library, which is built with IEEE mode
// on and so cannot be inlined; a call also hides that the workgroup index is
// uniform, and loops bounded by it would branch per lane.
__device__ __forceinline__ int wg_x() { return (int)__builtin_amdgcn_workgroup_id_x(); }
__device__ __forceinline__ int wg_y() { return (int)__builtin_amdgcn_workgroup_id_y(); }
__device__ __forceinline__ int wg_z() { return (int)__builtin_amdgcn_workgroup_id_z(); }
__device__ __forceinline__ int thread_x() { return (int)__builtin_amdgcn_workitem_id_x(); }
constexpr int kNumXcd = 8;  // MI355X: 8 accelerator complex dies, 32 CUs each

// bf16 bit patterns packed two per 32-bit word: low half is the first element.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Two fp32 -> packed bf16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2 v = {(__bf16)a, (__bf16)b};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float fdot2_bf16(uint32_t a, uint32_t b, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, a), __builtin_bit_cast(bf16x2, b), c, false);
}

// DPP lane movements (within rows of 16 lanes).
template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xf, 0xf, false));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7-i inside each group of 8
constexpr int kDppRowRor8 = 0x128;    // lane i <- lane (i+8) mod 16 inside each row of 16

// Sum over the 8 lanes of each aligned group of 8; every lane gets the sum.
__device__ __forceinline__ float sum8(float x) {
  x += dpp_f<kDppXor1>(x);
  x += dpp_f<kDppXor2>(x);
  x += dpp_f<kDppHalfMirror>(x);
  return x;
}

// max / sum over the lane pair {l, l ^ 16} (or {l, l ^ 32}), through the gfx950
// row-swap instructions (plain VALU, no LDS round trip).  permlane16_swap(x, x)
// returns x with rows 1 and 3 replaced by rows 0 and 2, and x with rows 0 and 2
// replaced by rows 1 and 3 (a row is 16 lanes; likewise halves of 32 lanes for
// permlane32_swap).  In every lane the two results are its own value and its
// partner's, so no lane select is needed and both lanes of a pair get the same
// value.
__device__ __forceinline__ float max_pair16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_pair16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float add_pair32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Reductions over lanes {l, l^8, l^16, ...}: combine groups of 8 lanes.
__device__ __forceinline__ float max_over_groups8(float x) {
  x = fmaxf(x, dpp_f<kDppRowRor8>(x));
  return max_pair32(max_pair16(x));
}
__device__ __forceinline__ float sum_over_groups8(float x) {
  x += dpp_f<kDppRowRor8>(x);
  return add_pair32(add_pair16(x));
}

// Sum of an int over the 64 lanes of a wave (every lane must be active).
__device__ __forceinline__ int wave_sum_i32(int x) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) x += __shfl_xor(x, m);
  return x;
}

// Workgroups are dispatched to the XCDs round-robin (id mod 8).  Give each XCD
// a contiguous range of logical work items so that the workgroups resident on
// one XCD at a time work on neighbouring tiles and share that XCD's L2.
__device__ __forceinline__ int xcd_logical_id(int hw_id, int n) {
  const int x = hw_id % kNumXcd;
  const int q = hw_id / kNumXcd;
  const int per = n / kNumXcd, rem = n % kNumXcd;
  const int start = x * per + (x < rem ? x : rem);
  return start + q;
}

}  // namespace swa
