// Combine: gate-weighted sum of the expert outputs back into token order,
// plus the shared expert and the residual.
//
// out[t] = x[t] + shared[t] + sum over kept slots j of gate[t,j] * y[row]
// (randomcommits.com "Mixture-of-Experts routing", How a sparse MoE layer
// works: weighted sum of the chosen experts, added through the residual;
// foundry.adhana.ai "Mixture-of-Experts routing", Concept).  A dropped slot
// (slot_of = -1) adds nothing and the surviving gates keep their values
// (letsbuildsolutions.com "How Mixture of Experts Works", Token Dropping and
// Overflow Handling, zero output).
//
// One workgroup per token; each thread owns 8 consecutive features (one
// 16-byte bf16 vector or two float4 vectors), so every row is read and
// written with full-width coalesced accesses.  Accumulation is float32 in
// the fixed order residual, shared, slot 0..k-1, then one rounding.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

template <typename T>
__device__ __forceinline__ void load8(const T* p, float* f);
// bf16 rows (x, the expert outputs) are each read once here: non-temporal
// loads (the DeepSeek-V3 combine 131 -> 117 us)
template <>
__device__ __forceinline__ void load8<bf16>(const bf16* p, float* f) {
  V16 v;
  v.u = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)v.h[i];
}
template <>
__device__ __forceinline__ void load8<float>(const float* p, float* f) {
  V16 a, b;
  a.u = ldg16(p);
  b.u = ldg16(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[i] = a.f[i];
    f[4 + i] = b.f[i];
  }
}
template <typename T>
__device__ __forceinline__ void store8(T* p, const float* f);
template <>
__device__ __forceinline__ void store8<bf16>(bf16* p, const float* f) {
  V16 v;
  v.h = pack_bf16x8(f);
  stg16(p, v.u);
}
template <>
__device__ __forceinline__ void store8<float>(float* p, const float* f) {
  V16 a, b;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a.f[i] = f[i];
    b.f[i] = f[4 + i];
  }
  stg16(p, a.u);
  stg16(p + 4, b.u);
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(
    const T* __restrict__ x, const T* __restrict__ y,
    const int32_t* __restrict__ slot_of, const float* __restrict__ gate,
    T* __restrict__ out, int T_, int d, int k, int n_shared) {
  const int t = blockIdx.x;
  int rows[MOE_MAX_K];
  float g[MOE_MAX_K];
#pragma unroll
  for (int j = 0; j < MOE_MAX_K; ++j) {
    rows[j] = -1;
    g[j] = 0.f;
    if (j < k) {
      rows[j] = slot_of[(size_t)t * k + j];
      g[j] = gate[(size_t)t * k + j];
    }
  }
  const T* ysh = n_shared ? y + ((size_t)T_ * k + t) * d : nullptr;
  for (int c = threadIdx.x * 8; c < d; c += blockDim.x * 8) {
    float acc[8];
    if (x) {
      load8<T>(x + (size_t)t * d + c, acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    }
    if (ysh) {
      float v[8];
      load8<T>(ysh + c, v);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += v[i];
    }
#pragma unroll
    for (int j = 0; j < MOE_MAX_K; ++j) {
      if (rows[j] >= 0) {
        float v[8];
        load8<T>(y + (size_t)rows[j] * d + c, v);
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] += g[j] * v[i];
      }
    }
    store8<T>(out + (size_t)t * d + c, acc);
  }
}

}  // namespace

hipError_t launch_combine(int dtype, const void* x, const void* y,
                          const int32_t* slot_of, const float* gate,
                          void* out, int T, int d, int k, int n_shared,
                          hipStream_t s) {
  if (T == 0) return hipSuccess;
  const int threads = d >= 2048 ? 256 : (d >= 512 ? 64 : 64);
  if (dtype == 1)
    combine_kernel<bf16><<<T, threads, 0, s>>>(
        (const bf16*)x, (const bf16*)y, slot_of, gate, (bf16*)out, T, d, k,
        n_shared);
  else
    combine_kernel<float><<<T, threads, 0, s>>>(
        (const float*)x, (const float*)y, slot_of, gate, (float*)out, T, d, k,
        n_shared);
  return hipGetLastError();
}

}  // namespace moe
