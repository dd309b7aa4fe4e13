// Device-side vector types and small helpers for the gfx950 kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <cstdint>

namespace ringattn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_huge_valf();

// Workgroups are handed to the 8 XCDs of an MI355X round-robin by linear
// id.  This maps a hardware id to a logical id such that each XCD receives
// one contiguous range of logical ids (neighbouring tiles that read the same
// K/V then share that XCD's L2).
__device__ __forceinline__ int xcd_contiguous_id(int hw_id, int total) {
  constexpr int kXcds = 8;
  const int xcd = hw_id % kXcds;
  const int local = hw_id / kXcds;
  const int per = total / kXcds;
  const int extra = total % kXcds;
  return xcd < extra ? xcd * (per + 1) + local : extra * (per + 1) + (xcd - extra) * per + local;
}

__device__ __forceinline__ float wave_max_xor32(float x) {
  return fmaxf(x, __shfl_xor(x, 32, 64));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Transposing LDS read: within each group of 16 lanes, lane i receives element
// (i % 4) of the four 16-bit values addressed by lanes 4e + i/4, e = 0..3.
__device__ __forceinline__ s16x4 lds_read_tr16(const uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) s16x4*)(p));
}

__device__ __forceinline__ bf16x8 join_bf16x4(s16x4 lo, s16x4 hi) {
  typedef short s16x8 __attribute__((ext_vector_type(8)));
  s16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

}  // namespace ringattn
