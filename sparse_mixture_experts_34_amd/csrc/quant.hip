// Group-wise 4-bit round-to-nearest quantisation of bf16 expert weights
// (letsbuildsolutions.com "How Mixture of Experts Works", Production
// Considerations: storing expert weights in 4 bits cuts Mixtral 8x7B's
// weights from about 93 GB to about 26 GB).  The plain reading kept here:
// one (scale, offset) pair per group of 128 consecutive weights of a row,
// scale = (max - min) / 15, code = rint((w - min) / scale) in 0..15.
//
// One thread per 32-bit code word (eight consecutive weights), 16 threads
// per group: the group's min and max meet through lane shuffles inside the
// 16-lane segment.  Codes are decided in float32 with correctly rounded
// division, so they do not depend on how the division is compiled.
//
// Word layout: nibble i holds weight 2i for i < 4 and weight 2(i-4)+1 for
// i >= 4, so a word turns into bf16 MFMA operand pairs (even weight low,
// odd weight high) with one shift and one mask per pair.  Words are stored
// in the GEMM's operand order: a 1024-byte tile per 16 rows x one group,
// slot m = row%16 + 16*kq holding weights kq*32..kq*32+31 of the group as
// words h = 0..3, so one wave reads a tile with one contiguous load; the
// (scale, offset) pairs of the 16 rows of a group share a 128-byte tile.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int QW = Q4_GROUP / 8;   // code words (threads) per group

__global__ __launch_bounds__(256) void quantize_int4_kernel(
    const bf16* __restrict__ w, long long n_groups, int K,
    uint32_t* __restrict__ codes, float* __restrict__ qparams) {
  const long long tg = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long g = tg / QW;          // group id: row * (K/128) + index
  const int j = (int)(tg % QW);         // word inside the group
  if (g >= n_groups) return;            // whole 16-lane segments
  const int gpr = K / Q4_GROUP;
  const long long row = g / gpr;
  const int gi = (int)(g % gpr);
  const size_t base = (size_t)row * K + (size_t)gi * Q4_GROUP + j * 8;
  V16 v;
  v.u = ldg16(w + base);
  float f[8];
  float lo, hi;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (float)v.h[i];
  lo = hi = f[0];
#pragma unroll
  for (int i = 1; i < 8; ++i) {
    lo = fminf(lo, f[i]);
    hi = fmaxf(hi, f[i]);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    lo = fminf(lo, __shfl_xor(lo, o, QW));
    hi = fmaxf(hi, __shfl_xor(hi, o, QW));
  }
  const float s = __fdiv_rn(hi - lo, 15.0f);
  uint32_t word = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int q = 0;
    if (s != 0.0f) {
      const float r = rintf(__fdiv_rn(f[i] - lo, s));
      q = (int)fminf(fmaxf(r, 0.0f), 15.0f);
    }
    const int nib = (i & 1) ? 4 + (i >> 1) : (i >> 1);
    word |= (uint32_t)q << (4 * nib);
  }
  const size_t tile = (size_t)(row >> 4) * gpr + gi;
  const int slot = (int)(row & 15) + 16 * (j >> 2);
  codes[tile * 256 + slot * 4 + (j & 3)] = word;
  if (j == 0) {
    const size_t qi = (tile * 16 + (size_t)(row & 15)) * 2;
    qparams[qi] = s;
    qparams[qi + 1] = lo;
  }
}

}  // namespace

hipError_t launch_quantize_int4(const void* w, long long rows, int K,
                                void* codes, float* qparams, hipStream_t s) {
  const long long n_groups = rows * (K / Q4_GROUP);
  if (n_groups == 0) return hipSuccess;
  const long long threads = n_groups * QW;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  quantize_int4_kernel<<<blocks, 256, 0, s>>>((const bf16*)w, n_groups, K,
                                              (uint32_t*)codes, qparams);
  return hipGetLastError();
}

// bf16 weights in tiled order: one thread per 16-byte piece p of the
// output; tile t = p / 64 (row block rb = t / (K/32), column block kb =
// t % (K/32)), piece u = p % 64 holds row 16*rb + u % 16, columns
// 32*kb + 8*(u / 16) .. +8.  Output writes are contiguous.
namespace {
__global__ __launch_bounds__(256) void tile_bf16_kernel(
    const bf16* __restrict__ w, long long n_pieces, int K,
    bf16* __restrict__ out) {
  const long long p = (long long)blockIdx.x * 256 + threadIdx.x;
  if (p >= n_pieces) return;
  const int kbs = K / 32;
  const long long t = p >> 6;
  const int u = (int)(p & 63);
  const long long rb = t / kbs;
  const int kb = (int)(t - rb * kbs);
  const long long row = rb * 16 + (u & 15);
  const size_t src = (size_t)row * K + (size_t)kb * 32 + (u >> 4) * 8;
  stg16(out + (size_t)p * 8, ldg16(w + src));
}
}  // namespace

hipError_t launch_tile_bf16(const void* w, long long rows, int K, void* out,
                            hipStream_t s) {
  const long long n = rows * (K / 8);
  if (n == 0) return hipSuccess;
  tile_bf16_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(
      (const bf16*)w, n, K, (bf16*)out);
  return hipGetLastError();
}

}  // namespace moe
