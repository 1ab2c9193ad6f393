// Internal helpers shared by the HIP kernels and the host orchestration of
// libortho.so.  gfx950 (CDNA4) only.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ortho {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef double doublex4 __attribute__((ext_vector_type(4)));

// Most matrices one launch may address through its pointer tables.  Larger
// groups are issued as several launches.
constexpr int kMaxBatch = 32;

// One operand as a kernel sees it: a pointer per group member, a leading
// dimension shared by the group, its logical extent and whether 16-byte vector
// access is legal for every member.
struct MatArg {
  const void* p[kMaxBatch];
  int64_t ld;
  int rows;
  int cols;
  int vec;
};

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// Round to nearest even (lowers to v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ bf16 to_bf16(float x) { return static_cast<bf16>(x); }

__device__ __forceinline__ uint16_t to_bf16_bits(float x) {
  return __builtin_bit_cast(uint16_t, static_cast<bf16>(x));
}

// Four fp32 values as four bf16 (RNE), packed for one 8-byte store.
__device__ __forceinline__ uint2 pack_bf16x4(floatx4 v) {
  return make_uint2(to_bf16_bits(v[0]) | (uint32_t(to_bf16_bits(v[1])) << 16),
                    to_bf16_bits(v[2]) | (uint32_t(to_bf16_bits(v[3])) << 16));
}

// x = hi + lo + O(2^-16 |x|): hi is x rounded to bf16, lo is the exact fp32
// remainder rounded to bf16.
__device__ __forceinline__ void split_bf16(float x, bf16& hi, bf16& lo) {
  hi = to_bf16(x);
  lo = to_bf16(x - static_cast<float>(hi));
}

// Value of element (r, c) of a storage-typed matrix as fp32.
template <typename T>
__device__ __forceinline__ float load_as_f32(const T* p, int64_t idx);
template <>
__device__ __forceinline__ float load_as_f32<float>(const float* p, int64_t idx) { return p[idx]; }
template <>
__device__ __forceinline__ float load_as_f32<uint16_t>(const uint16_t* p, int64_t idx) {
  return bf16_bits_to_f32(p[idx]);
}

template <typename T>
__device__ __forceinline__ void store_from_f32(T* p, int64_t idx, float v);
template <>
__device__ __forceinline__ void store_from_f32<float>(float* p, int64_t idx, float v) { p[idx] = v; }
template <>
__device__ __forceinline__ void store_from_f32<uint16_t>(uint16_t* p, int64_t idx, float v) {
  p[idx] = to_bf16_bits(v);
}

// Four consecutive elements of row r starting at column c (c % 4 == 0), as fp32.
template <typename T>
__device__ __forceinline__ float4 load4(const T* row, int c, int limit, bool vec);

template <>
__device__ __forceinline__ float4 load4<float>(const float* row, int c, int limit, bool vec) {
  if (vec && c + 4 <= limit) return *reinterpret_cast<const float4*>(row + c);
  float t[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) t[j] = (c + j < limit) ? row[c + j] : 0.f;
  return make_float4(t[0], t[1], t[2], t[3]);
}

template <>
__device__ __forceinline__ float4 load4<uint16_t>(const uint16_t* row, int c, int limit, bool vec) {
  if (vec && c + 4 <= limit) {
    uint2 u = *reinterpret_cast<const uint2*>(row + c);
    return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                       __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
  }
  float t[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) t[j] = (c + j < limit) ? bf16_bits_to_f32(row[c + j]) : 0.f;
  return make_float4(t[0], t[1], t[2], t[3]);
}

// Four consecutive elements as stored (fp32: float4, bf16 bits: uint2), and
// their fp32 values.
template <typename T> struct Raw4;
template <> struct Raw4<float> { typedef float4 type; };
template <> struct Raw4<uint16_t> { typedef uint2 type; };

__device__ __forceinline__ float4 raw_to_f4(const float4& v) { return v; }
__device__ __forceinline__ float4 raw_to_f4(const uint2& u) {
  return make_float4(__uint_as_float(u.x << 16), __uint_as_float(u.x & 0xffff0000u),
                     __uint_as_float(u.y << 16), __uint_as_float(u.y & 0xffff0000u));
}

__device__ __forceinline__ float f4_get(const float4& v, int j) {
  return j == 0 ? v.x : (j == 1 ? v.y : (j == 2 ? v.z : v.w));
}

}  // namespace ortho
