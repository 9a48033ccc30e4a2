// Device helpers shared by the expert-FFN translation units (ffn.hip: the
// bf16 and float32 schedules; ffn_q4.hip: the 4-bit stream schedule).
#pragma once

#include "common.hpp"
#include "kernels.hpp"

namespace moe {
namespace {

// Waves per workgroup of the stream schedules; they split K.
constexpr int ST_WAVES = 4;

enum { UP_SWIGLU = 0, UP_GELU = 1, DOWN = 2 };

struct Group {
  int rows;     // rows of this group
  int out0;     // first output row
  bool shared;
};

__device__ __forceinline__ Group group_of(int g, const int32_t* offsets, int E,
                                          int T, int k) {
  Group r;
  if (g < E) {
    r.out0 = offsets[g];
    r.rows = offsets[g + 1] - r.out0;
    r.shared = false;
  } else {
    r.out0 = T * k;
    r.rows = T;
    r.shared = true;
  }
  return r;
}

// Row of the A operand for output row index i (0-based inside the group).
template <int MODE, typename ET>
__device__ __forceinline__ const ET* a_row(const FfnArgs& a, const Group& gr,
                                           int i, int K) {
  if (MODE == DOWN) return (const ET*)a.h + (size_t)(gr.out0 + i) * K;
  const int tok = gr.shared ? i : a.perm[gr.out0 + i] / a.k;
  return (const ET*)a.x + (size_t)tok * K;
}

// A wave-uniform pointer in scalar registers (the value is the same in every
// lane; this only tells the compiler so).
__device__ __forceinline__ const char* uniform_ptr(const char* p) {
  const uint64_t v = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const char*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

}  // namespace
}  // namespace moe
