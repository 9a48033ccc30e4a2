// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;   // MFMA operand
typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int WAVE = 64;
constexpr int MOE_MAX_K = 8;   // largest top-k the kernels accept

// --- scalar conversions --------------------------------------------------
__device__ __forceinline__ float to_f32(float v) { return v; }
__device__ __forceinline__ float to_f32(bf16 v) { return (float)v; }

template <typename T>
__device__ __forceinline__ T from_f32(float v);
template <>
__device__ __forceinline__ float from_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16 from_f32<bf16>(float v) { return (bf16)v; }  // RNE

// --- activations ---------------------------------------------------------
// exact (erf) GELU, z * Phi(z)
__device__ __forceinline__ float gelu_erf(float z) {
  return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}
// SiLU, z * sigmoid(z)
__device__ __forceinline__ float silu(float z) {
  return z / (1.0f + __expf(-z));
}

// Logistic sigmoid 1 / (1 + e^-z) (per-expert router scoring).
__device__ __forceinline__ float sigmoid_f(float z) {
  return 1.0f / (1.0f + __expf(-z));
}

// --- 16-byte vector type punning ----------------------------------------
union V16 {
  u32x4 u;
  bf16x8 h;
  float f[4];
  uint16_t s[8];
};

__device__ __forceinline__ u32x4 ldg16(const void* p) {
  return *reinterpret_cast<const u32x4*>(p);
}
__device__ __forceinline__ void stg16(void* p, u32x4 v) {
  *reinterpret_cast<u32x4*>(p) = v;
}

// bf16x8 from 8 floats (RNE)
__device__ __forceinline__ bf16x8 pack_bf16x8(const float* f) {
  bf16x8 r;
#pragma unroll
  for (int i = 0; i < 8; ++i) r[i] = (bf16)f[i];
  return r;
}

// Split a float into three bf16 parts with v == hi + mid + lo up to the
// last bit or two of v's 24-bit significand; each difference below is exact
// in float32, so products of the parts with a bf16 value are exact.
__device__ __forceinline__ void split3(float v, bf16& hi, bf16& mid, bf16& lo) {
  hi = (bf16)v;
  float r1 = v - (float)hi;
  mid = (bf16)r1;
  float r2 = r1 - (float)mid;
  lo = (bf16)r2;
}

// --- wave reductions (fixed butterfly order: deterministic) -------------
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, WAVE));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, WAVE);
  return v;
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
