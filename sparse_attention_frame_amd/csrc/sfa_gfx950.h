// gfx950 building blocks shared by the attention and prologue kernels: operand vector
// types, address-space pointer types, bf16 packing and the wait on outstanding vector
// memory operations.
#pragma once
#include "sfa_internal.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_void_ptr;
typedef __attribute__((address_space(3))) i16x4* lds_i16x4_ptr;
typedef __attribute__((address_space(1))) void* global_void_ptr;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats rounded to bf16 (round to nearest even) in one 32-bit word, lo first.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Wait until at most N of this wave's vector-memory operations (the LDS DMAs
// of younger stages, loads, stores) are still in flight.
template <int N>
__device__ inline void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

}  // namespace
