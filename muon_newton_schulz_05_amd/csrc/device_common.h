// device_common.h -- small device helpers shared by the HIP kernels (gfx950).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "layout.h"

namespace muon {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16_t;
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

// Two floats -> one register of two bfloat16 (round to nearest even, low half first).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// Four packed registers as a matrix-core operand of eight bfloat16.
__device__ __forceinline__ bf16x8_t as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8_t, v);
}

// Pointers into device memory read from tables are generic for the compiler;
// casting them to the global address space gives global_* instructions with a
// uniform base and 32-bit lane offsets instead of flat 64-bit addressing.
#define MUON_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ MUON_GLOBAL T* as_global(T* p) {
  return (MUON_GLOBAL T*)p;
}
template <typename T>
__device__ __forceinline__ const MUON_GLOBAL T* as_global(const T* p) {
  return (const MUON_GLOBAL T*)p;
}

// float -> bfloat16 bits, round to nearest even (v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ uint16_t to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ float from_bf16(uint16_t h) {
  return __uint_as_float((uint32_t)h << 16);
}

// Element loads/stores by run-time dtype (0 = float32, 1 = bfloat16 bits).
__device__ __forceinline__ float load_as_f32(const void* base, int64_t idx, int dtype) {
  return dtype == 0 ? static_cast<const float*>(base)[idx]
                    : from_bf16(static_cast<const uint16_t*>(base)[idx]);
}
__device__ __forceinline__ void store_from_f32(void* base, int64_t idx, int dtype, float v) {
  if (dtype == 0) static_cast<float*>(base)[idx] = v;
  else static_cast<uint16_t*>(base)[idx] = to_bf16(v);
}

// Workspace element type of X: float (fp32 mode) or bfloat16 bits.
template <typename T> __device__ __forceinline__ T cvt_x(float v);
template <> __device__ __forceinline__ float cvt_x<float>(float v) { return v; }
template <> __device__ __forceinline__ uint16_t cvt_x<uint16_t>(float v) { return to_bf16(v); }
__device__ __forceinline__ float x_to_f32(float v) { return v; }
__device__ __forceinline__ float x_to_f32(uint16_t v) { return from_bf16(v); }

// Fixed-order sum across a 64-lane wavefront (butterfly; every lane gets the total).
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

// Shape factor f of the update of a slice with oriented shape [m, n]
// (m <= n), stored transposed ([n, m], R > C) or not ([m, n]).
__device__ __forceinline__ float update_factor(int scale_mode, int64_t m, int64_t n, int transposed) {
  if (scale_mode == 1) return transposed ? sqrtf((float)n / (float)m) : 1.f;  // sqrt(max(1, R / C))
  if (scale_mode == 2) return 0.2f * sqrtf((float)n);                        // 0.2 sqrt(max(R, C))
  return 1.f;
}

}  // namespace muon
