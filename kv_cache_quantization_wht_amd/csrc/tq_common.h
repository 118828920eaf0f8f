// Device helpers shared by the library's kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tq {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float floatx4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16_bits_to_float(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }

__device__ __forceinline__ float half_bits_to_float(uint16_t b) {
  _Float16 h;
  __builtin_memcpy(&h, &b, 2);
  return (float)h;
}

// Round to fp16, ties to even.
__device__ __forceinline__ uint16_t float_to_half_bits(float f) {
  _Float16 h = (_Float16)f;
  uint16_t b;
  __builtin_memcpy(&b, &h, 2);
  return b;
}

// Element i of an input row of dtype 0 (f32), 1 (bf16) or 2 (f16), widened to fp32.
__device__ __forceinline__ float load_elem(const void *p, int64_t i, int dtype) {
  if (dtype == 0) return ((const float *)p)[i];
  if (dtype == 1) return bf16_bits_to_float(((const uint16_t *)p)[i]);
  return half_bits_to_float(((const uint16_t *)p)[i]);
}

}  // namespace tq
