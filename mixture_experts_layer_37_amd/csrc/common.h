// Shared device helpers for the gfx950 MoE kernels: bf16 conversion, vector types and the
// MFMA operand types. Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

constexpr int kWave = 64;
constexpr int kMaxExperts = 256;
constexpr int kMaxTopK = 16;
constexpr int kCountBlockTokens = 1024;   // tokens per permute histogram block
constexpr int kRouteFlagGroup = 16;       // tokens per route flag word

typedef uint16_t bf16_t;                  // raw bfloat16 bits
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte store with the nontemporal hint, for rows written once and not read back soon.
__device__ __forceinline__ void st_stream(uint4* p, uint4 v) {
  const u32x4 w = {v.x, v.y, v.z, v.w};
  __builtin_nontemporal_store(w, (u32x4*)p);
}

__device__ __forceinline__ float bf16_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bfloat16, round to nearest, ties to even; NaN -> quiet NaN.
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// Two floats -> two packed bfloat16 (lo in bits 0..15), round to nearest, ties to even: one
// v_cvt_pk_bf16_f32 on gfx950 (a NaN stays a quiet NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// Element storage helpers: bf16 is stored as raw 16-bit patterns.
template <typename T> struct Elem;
template <> struct Elem<bf16_t> {
  static __device__ __forceinline__ float load(const bf16_t* p) { return bf16_to_f32(*p); }
  static __device__ __forceinline__ bf16_t from_f32(float f) { return (bf16_t)f32_to_bf16(f); }
  static __device__ __forceinline__ float to_f32(bf16_t v) { return bf16_to_f32(v); }
};
template <> struct Elem<float> {
  static __device__ __forceinline__ float load(const float* p) { return *p; }
  static __device__ __forceinline__ float from_f32(float f) { return f; }
  static __device__ __forceinline__ float to_f32(float v) { return v; }
};

__device__ __forceinline__ int lane_id() { return threadIdx.x & (kWave - 1); }

}  // namespace moe
