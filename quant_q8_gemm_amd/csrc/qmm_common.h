// qmm_common.h -- small device helpers shared by the library's HIP kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace qmm {

typedef int v2i __attribute__((ext_vector_type(2)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// Empty asm that claims to modify v: the value must be produced before this
// point and cannot be recomputed after it.  Emits no instruction; used to keep
// software-pipeline stages where they are written.
template <class T>
__device__ __forceinline__ void pin(T& v) {
  asm volatile("" : "+v"(v));
}

// A pointer every lane of the wave holds, moved to scalar registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ float f16_bits_to_float(uint32_t bits) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)bits);
}

}  // namespace qmm
