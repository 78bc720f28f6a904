// Device helpers shared by the forward and backward kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <math.h>

namespace sdpa07 {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

constexpr float kLn2 = 0.693147180559945309f;
// Buffer resource word 3 for raw (untyped) loads on gfx9-family parts, and an
// offset past any num_records bound (such loads return zeros).
constexpr int kBufferFlags = 0x00020000;
constexpr int kOutOfRange = (int)0x80000000u;
typedef int i32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Mfma16;
template <>
struct Mfma16<__bf16> {
  using v8 = bf16x8;
  static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
};
template <>
struct Mfma16<_Float16> {
  using v8 = f16x8;
  static __device__ __forceinline__ f32x16 mma(v8 a, v8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
};

// Value of x held by the lane 32 positions away (the other half-wave).
__device__ __forceinline__ float other_half(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  // Lanes < 32 receive the upper half in sw[1]; lanes >= 32 the lower in sw[0].
  const unsigned o = (threadIdx.x & 32) ? sw[0] : sw[1];
  return __builtin_bit_cast(float, o);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Pins the computation of x before this point of the instruction stream (an
// empty volatile asm that reads x: volatile asms keep their order, so x's
// producers cannot sink past it). Used to keep softmax work interleaved with
// the MFMAs it is meant to overlap.
template <typename X>
__device__ __forceinline__ void pin(const X& x) {
  asm volatile("" ::"v"(x));
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

typedef float f32x2 __attribute__((ext_vector_type(2)));

template <typename T>
struct Pack2;
template <>
struct Pack2<__bf16> {
  using type = bf16x2;
};
template <>
struct Pack2<_Float16> {
  using type = f16x2;
};

// acc + h.x + h.y for a packed pair of 16-bit values (one v_dot2 with ones).
template <typename T>
__device__ __forceinline__ float dot2_ones(typename Pack2<T>::type h, float acc);
template <>
__device__ __forceinline__ float dot2_ones<__bf16>(bf16x2 h, float acc) {
  const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(h, one, acc, false);
}
template <>
__device__ __forceinline__ float dot2_ones<_Float16>(f16x2 h, float acc) {
  const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
  return __builtin_amdgcn_fdot2(h, one, acc, false);
}

}  // namespace
}  // namespace sdpa07
