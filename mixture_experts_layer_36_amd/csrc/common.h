// Shared device helpers of libmoe's kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

// 16-byte vector of elements: 8 bf16 or 4 fp32.
template <typename T> struct Vec16;
template <> struct Vec16<float> { static constexpr int N = 4; };
template <> struct Vec16<bf16> { static constexpr int N = 8; };

__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T> __device__ __forceinline__ T from_f32(float v);
template <> __device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }

// Unpack a 16-byte vector into N floats.
template <typename T>
__device__ __forceinline__ void unpack16(const u32x4& v, float* out);
template <>
__device__ __forceinline__ void unpack16<float>(const u32x4& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(v[i]);
}
template <>
__device__ __forceinline__ void unpack16<bf16>(const u32x4& v, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(v[i] << 16);
    out[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}

// Pack N floats into a 16-byte vector (bf16: round to nearest even).
template <typename T>
__device__ __forceinline__ u32x4 pack16(const float* in);
template <>
__device__ __forceinline__ u32x4 pack16<float>(const float* in) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = __float_as_uint(in[i]);
  return v;
}
__device__ __forceinline__ unsigned bf16_bits(float f) {
  bf16 b = (bf16)f;
  return (unsigned)__builtin_bit_cast(unsigned short, b);
}
// two floats rounded to bf16 (to nearest even, as a single conversion does),
// a in the low half: one v_cvt_pk_bf16_f32 instead of two conversions, a
// shift and an or
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ unsigned pack_bf16x2(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}
template <>
__device__ __forceinline__ u32x4 pack16<bf16>(const float* in) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = pack_bf16x2(in[2 * i], in[2 * i + 1]);
  return v;
}

// Transposing LDS read (ds_read_b64_tr_b16): within each 16-lane group,
// lane j addresses 4 consecutive 16-bit columns of row j / 4 of a 4 x 16
// block, and lane i receives column i's 4 values (rows 0..3).  p is an LDS
// address, 8-byte aligned.
typedef short i16x4_lds_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  typedef __attribute__((address_space(3))) i16x4_lds_t lds_i16x4;
  const i16x4_lds_t v =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(const __attribute__((address_space(3))) char*)p);
  return __builtin_bit_cast(u32x2, v);
}

__device__ __forceinline__ u32x4 ld16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// Wave-level reductions over lanes that differ only in the low log2(W) bits.
template <int W>
__device__ __forceinline__ float group_sum(float v) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
template <int W>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int m = W / 2; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}

}  // namespace moe
