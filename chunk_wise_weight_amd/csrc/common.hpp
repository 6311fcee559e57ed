// Shared device types and helpers for the gfx950 (CDNA4) kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ttt {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

// Elements of T per 16-byte chunk (the unit of every global and LDS access).
template <typename T> struct Vec;
template <> struct Vec<bf16> { static constexpr int V = 8; };
template <> struct Vec<float> { static constexpr int V = 4; };

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }

// Round-to-nearest-even float -> bf16 on the raw bits (NaN kept quiet).
__device__ __forceinline__ unsigned bf16_bits_rne(float f) {
  unsigned u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) {
  unsigned short b = (unsigned short)bf16_bits_rne(x);
  return __builtin_bit_cast(bf16, b);
}

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two floats to packed bf16 with round-to-nearest-even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ unsigned pack2_bf16(float a, float b) {
  return __builtin_bit_cast(unsigned, __builtin_convertvector((f32x2){a, b}, bf16x2));
}

// Store four consecutive values (8 bytes for bf16, 16 bytes for fp32).
__device__ __forceinline__ void store4(bf16* p, float a, float b, float c, float d) {
  *reinterpret_cast<u32x2*>(p) = (u32x2){pack2_bf16(a, b), pack2_bf16(c, d)};
}
__device__ __forceinline__ void store4(float* p, float a, float b, float c, float d) {
  *reinterpret_cast<f32x4*>(p) = (f32x4){a, b, c, d};
}

// Load four consecutive values widened to fp32.
__device__ __forceinline__ f32x4 load4(const bf16* p) {
  u32x2 w = *reinterpret_cast<const u32x2*>(p);
  return (f32x4){__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xffff0000u),
                 __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xffff0000u)};
}
__device__ __forceinline__ f32x4 load4(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
// The same as a non-temporal (streaming) load: for data read once, so that it
// does not displace what the caches hold for the other waves.
__device__ __forceinline__ f32x4 load4_stream(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}

// Widen one 16-byte chunk of bf16 to 8 floats / of fp32 to 4 floats.
__device__ __forceinline__ void unpack8(u32x4 w, float* o) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}

// Logistic function and SiLU from the hardware exponential and reciprocal
// (v_exp_f32, v_rcp_f32, about 1 ulp each) rather than an IEEE division
// sequence.  exp(-x) overflowing to +inf for very negative x gives 0.
__device__ __forceinline__ float sigmoid_f(float x) { return __builtin_amdgcn_rcpf(1.0f + __expf(-x)); }
__device__ __forceinline__ float silu_f(float x) { return x * sigmoid_f(x); }

}  // namespace ttt
