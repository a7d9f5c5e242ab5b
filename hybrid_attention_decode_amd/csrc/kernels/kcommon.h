// Device helpers shared by the gfx950 kernels of this library.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace had {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// bf16 bit pattern -> float (exact).
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(static_cast<uint32_t>(b) << 16); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = static_cast<__bf16>(x);
  return __builtin_bit_cast(uint16_t, b);
}
// Two floats -> packed bf16 pair (lo in bits 0..15), round to nearest even.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t v;
  v.x = static_cast<__bf16>(lo);
  v.y = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// acc + a.lo*b.lo + a.hi*b.hi with bf16 pairs and an fp32 accumulator
// (v_dot2c_f32_bf16).
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a), __builtin_bit_cast(bf16x2_t, b), acc,
                                         false);
}

// DPP lane permutations (gfx9 encodings).
enum : int {
  DPP_QUAD_XOR1 = 0xB1,   // quad_perm [1,0,3,2]
  DPP_QUAD_XOR2 = 0x4E,   // quad_perm [2,3,0,1]
  DPP_ROW_HALF_MIRROR = 0x141,  // lane i <-> 7-i inside each group of 8
  DPP_ROW_ROR4 = 0x124,   // rotate by 4 inside each 16-lane row
  DPP_ROW_ROR8 = 0x128    // rotate by 8 inside each 16-lane row (= xor 8)
};

template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float shfl_xor_f(float x, int mask) {
  const int lane = __lane_id();
  return __int_as_float(__builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __float_as_int(x)));
}

// x of lanes l and l ^ 16 (l ^ 32): v_permlane16_swap exchanges the upper
// 16 lanes of each 32-lane half of its first operand with the lower 16 of
// its second (v_permlane32_swap the upper 32 lanes of the first with the
// lower 32 of the second), so with both operands x its two results hold x of
// lane l and of lane l ^ 16 (l ^ 32), in either order
__device__ __forceinline__ float sum_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(p[0]) + __uint_as_float(p[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto p = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto p = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(p[0]), __uint_as_float(p[1]));
}

__device__ __forceinline__ uint32_t perm_b32(uint32_t hi, uint32_t lo, uint32_t sel) {
  return __builtin_amdgcn_perm(hi, lo, sel);
}

__device__ __forceinline__ void set_err(int32_t* d_err, int bits) {
  if (d_err) atomicOr(d_err, bits);
}

constexpr float kLog2e = 1.4426950408889634f;

// Word 3 of a raw buffer resource on gfx9 (32-bit data format, no swizzle;
// range checking against num_records on), and the non-temporal cache-policy
// bit of a buffer instruction on gfx950.
constexpr int kBufferRsrcWord3 = 0x00020000;
constexpr int kBufferNT = 2;

}  // namespace had
