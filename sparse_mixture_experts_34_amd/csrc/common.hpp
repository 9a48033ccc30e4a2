// Device helpers shared by the gfx950 kernels of the MoE layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;   // MFMA operand
typedef __attribute__((ext_vector_type(2))) float f32x2;
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
// erf-form GELU, z * Phi(z), Phi(z) = (1 + erf(z / sqrt 2)) / 2.  erfc of
// u = |z| / sqrt 2 comes from Abramowitz & Stegun 7.1.26 (absolute error at
// most 1.5e-7): erfc(u) ~ q = t (a1 + t (a2 + t (a3 + t (a4 + t a5))))
// exp(-u^2), t = 1 / (1 + p u); then Phi(z) = q / 2 for z < 0 (no
// cancellation in 1 + erf) and 1 - q / 2 otherwise.  About a dozen
// instructions with the hardware reciprocal and exponential, against the
// library erff's branchy sequence, which was most of the GELU GEMMs'
// epilogue; in float32 the result stays within 4.2e-7 of the exact GELU
// (the erff form: 4.5e-7, and 100% relative error below z = -3).
__device__ __forceinline__ float gelu_erf(float z) {
  const float u = fabsf(z) * 0.70710678118654752f;
  const float t = __builtin_amdgcn_rcpf(fmaf(0.3275911f, u, 1.0f));
  float poly = fmaf(1.061405429f, t, -1.453152027f);
  poly = fmaf(poly, t, 1.421413741f);
  poly = fmaf(poly, t, -0.284496736f);
  poly = fmaf(poly, t, 0.254829592f);
  const float hq = 0.5f * (poly * t) * __expf(-u * u);
  return z * (z < 0.f ? hq : 1.0f - hq);
}
// SiLU, z * sigmoid(z), with the hardware reciprocal (about 1 ulp; the
// result is rounded to bf16 next) instead of an IEEE division: the
// division's ten-instruction sequence was a third of the tiled GEMM's
// epilogue.  For z below about -88, exp overflows, the reciprocal is 0 and
// the result is -0 (the exact value is below 1e-36 in magnitude).
__device__ __forceinline__ float silu(float z) {
  return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
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

// Split a float into three bf16 parts with v == hi + mid + lo exactly for
// every float with 2^-100 <= |v| < 2^120 (each part takes the next 8 bits of
// the 24-bit significand, the rounding residue moving its sign into the next
// part; outside that range the last part can underflow bf16 or hi can round
// to infinity); each difference below is exact in float32, so products of
// the parts with a bf16 value are exact.
__device__ __forceinline__ void split3(float v, bf16& hi, bf16& mid, bf16& lo) {
  hi = (bf16)v;
  float r1 = v - (float)hi;
  mid = (bf16)r1;
  float r2 = r1 - (float)mid;
  lo = (bf16)r2;
}

// --- wave reductions ------------------------------------------------------
// DPP lane moves (gfx9 controls): partner within a quad, then within 8 and
// 16 lanes by mirroring, then row 0 -> 1 and 2 -> 3 (row_bcast:15) and
// row 1 -> 2, 3 (row_bcast:31); lane 63 then holds the result, which is
// read back to every lane.  Fixed order: deterministic.  Every lane of the
// wave must be active.
constexpr int DPP_QUAD_1032 = 0xB1;     // quad_perm [1,0,3,2]
constexpr int DPP_QUAD_2301 = 0x4E;     // quad_perm [2,3,0,1]
constexpr int DPP_ROW_MIRROR = 0x140;
constexpr int DPP_ROW_HALF_MIRROR = 0x141;
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;

// lane's value moved by CTRL (rows outside ROWMASK return `old`)
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ int dpp_i(int old, int v) {
  return __builtin_amdgcn_update_dpp(old, v, CTRL, ROWMASK, 0xf, false);
}
template <int CTRL, int ROWMASK = 0xf>
__device__ __forceinline__ float dpp_f(float old, float v) {
  return __builtin_bit_cast(
      float, dpp_i<CTRL, ROWMASK>(__builtin_bit_cast(int, old),
                                  __builtin_bit_cast(int, v)));
}
__device__ __forceinline__ float lane63(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
  v = fmaxf(v, dpp_f<DPP_QUAD_1032>(v, v));
  v = fmaxf(v, dpp_f<DPP_QUAD_2301>(v, v));
  v = fmaxf(v, dpp_f<DPP_ROW_HALF_MIRROR>(v, v));
  v = fmaxf(v, dpp_f<DPP_ROW_MIRROR>(v, v));
  v = fmaxf(v, dpp_f<DPP_ROW_BCAST15, 0xa>(v, v));
  v = fmaxf(v, dpp_f<DPP_ROW_BCAST31, 0xc>(v, v));
  return lane63(v);
}
__device__ __forceinline__ float wave_sum(float v) {
  v += dpp_f<DPP_QUAD_1032>(0.f, v);
  v += dpp_f<DPP_QUAD_2301>(0.f, v);
  v += dpp_f<DPP_ROW_HALF_MIRROR>(0.f, v);
  v += dpp_f<DPP_ROW_MIRROR>(0.f, v);
  v += dpp_f<DPP_ROW_BCAST15, 0xa>(0.f, v);
  v += dpp_f<DPP_ROW_BCAST31, 0xc>(0.f, v);
  return lane63(v);
}

__device__ __forceinline__ int ceil_div(int a, int b) { return (a + b - 1) / b; }

}  // namespace moe
