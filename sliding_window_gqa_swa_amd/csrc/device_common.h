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

// Inclusive prefix sum of an int over the 64 lanes of a wave (every lane
// active), on DPP: shifts by 1, 2, 4 and 8 lanes within each row of 16 (lanes
// shifted in from outside the row add 0), then the total of row 0 added to
// rows 1 and 3 (row_bcast:15) and the total of rows 0-1 to rows 2 and 3
// (row_bcast:31).  Rows outside the row mask keep the old value 0.
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, false);  // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, false);  // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, false);  // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, false);  // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

// One DPP step of the float scans below: x's value from the lane Ctrl names
// (row_shr:n or row_bcast), `ident` where that lane is outside the row or the
// row is masked off.
template <int Ctrl, int RowMask>
__device__ __forceinline__ float dpp_f32(float x, float ident) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(__builtin_bit_cast(int, ident), __builtin_bit_cast(int, x),
                                                               Ctrl, RowMask, 0xf, false));
}
// Maximum and sum of a float over the 64 lanes of a wave (every lane active),
// as the scan of wave_incl_scan_i32 with max / add; the result (lane 63 of the
// scan) is returned uniform.
__device__ __forceinline__ float wave_max_f32(float x) {
  const float ni = -INFINITY;
  x = fmaxf(x, dpp_f32<0x111, 0xf>(x, ni));
  x = fmaxf(x, dpp_f32<0x112, 0xf>(x, ni));
  x = fmaxf(x, dpp_f32<0x114, 0xf>(x, ni));
  x = fmaxf(x, dpp_f32<0x118, 0xf>(x, ni));
  x = fmaxf(x, dpp_f32<0x142, 0xa>(x, ni));
  x = fmaxf(x, dpp_f32<0x143, 0xc>(x, ni));
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  x += dpp_f32<0x111, 0xf>(x, 0.f);
  x += dpp_f32<0x112, 0xf>(x, 0.f);
  x += dpp_f32<0x114, 0xf>(x, 0.f);
  x += dpp_f32<0x118, 0xf>(x, 0.f);
  x += dpp_f32<0x142, 0xa>(x, 0.f);
  x += dpp_f32<0x143, 0xc>(x, 0.f);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 63));
}
// Lane `i` (uniform) of a float.
__device__ __forceinline__ float lane_f32(float x, int i) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), i));
}

// Merge of n >= 1 partial results of one output row (unnormalised output
// sums, running max in log2 units, weight sum): returns
// sum_j w_j row_j[col] / sum_j w_j l_j with w_j = exp2(m_j - max_j m_j).
// Called by every thread of whole waves, one thread per column col.
// ml_at(j) points at partial j's (max, sum), row_at(j) at its value for this
// thread's column.  Lane i handles the (max, sum) of partials i, i + 64, ...;
// the first 64 pairs and the first kMergeBatch row values are loaded before
// any arithmetic, so a merge of up to kMergeBatch partials waits for memory
// once.  The max and the weight sum are wave reductions; each partial's
// weight is broadcast to the threads that add its row, and the rows add in
// partial order.  A partial whose max is -inf (no keys) has weight 0.
constexpr int kMergeBatch = 8;
template <class MlAt, class RowAt>
__device__ __forceinline__ float merge_partials(int n, int lane, MlAt ml_at, RowAt row_at) {
  float m0 = -INFINITY, l0 = 0.f;
  if (lane < n) {
    const float *q = ml_at(lane);
    m0 = q[0];
    l0 = q[1];
  }
  float a0[kMergeBatch];
#pragma unroll
  for (int i = 0; i < kMergeBatch; i++) a0[i] = *row_at(i < n ? i : n - 1);
  float mx = m0;
  for (int c0 = 64; c0 < n; c0 += 64)
    if (c0 + lane < n) mx = fmaxf(mx, ml_at(c0 + lane)[0]);
  mx = wave_max_f32(mx);
  float ls = 0.f, os = 0.f;
  for (int c0 = 0; c0 < n; c0 += 64) {
    const int cn = n - c0 < 64 ? n - c0 : 64;
    float m = m0, l = l0;
    if (c0 > 0) {
      m = -INFINITY;
      l = 0.f;
      if (lane < cn) {
        const float *q = ml_at(c0 + lane);
        m = q[0];
        l = q[1];
      }
    }
    const float w = (lane < cn && m != -INFINITY) ? exp2f(m - mx) : 0.f;
    ls += w * l;
    for (int i0 = 0; i0 < cn; i0 += kMergeBatch) {
      float av[kMergeBatch];
      if (c0 == 0 && i0 == 0) {
#pragma unroll
        for (int i = 0; i < kMergeBatch; i++) av[i] = a0[i];
      } else {
#pragma unroll
        for (int i = 0; i < kMergeBatch; i++) av[i] = *row_at(c0 + (i0 + i < cn ? i0 + i : cn - 1));
      }
#pragma unroll
      for (int i = 0; i < kMergeBatch; i++)
        if (i0 + i < cn) os += lane_f32(w, i0 + i) * av[i];
    }
  }
  return os / wave_sum_f32(ls);
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
