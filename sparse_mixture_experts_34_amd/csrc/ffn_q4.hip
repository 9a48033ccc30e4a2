// Expert FFNs with 4-bit weights: the stream schedule of the bf16 decode
// path (ffn.hip) over group-wise quantised codes, dequantised inside the
// GEMM (letsbuildsolutions.com "How Mixture of Experts Works", Production
// Considerations: quantization for MoE).  Used at every batch size: a
// decode-path format; larger batches stay correct, re-streaming the weights
// once per 32 rows of an expert.
//
// This file is compiled with the MFMA accumulators in ordinary VGPRs
// (-amdgpu-mfma-vgpr-form; the build script adds it for this file only):
// the per-group partial sums are read back by VALU right after their MFMAs,
// and from accumulation registers every read would first cost a copy.
#include "common.hpp"
#include "ffn_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

// The stream schedule's work split (16*CG columns per workgroup, 4 waves
// splitting K) with one K step per quantisation group of 128 weights.  Lane
// (col, kq) takes weights kq*32 .. kq*32+31 of the group in its row: 16
// code bytes, i.e. four words, each word one 16x16x32 MFMA B operand.  The
// codes are stored tiled in exactly this lane order (1024 bytes per 16 rows
// x group), so a wave reads a tile with one fully coalesced load, and the
// 16 rows' (scale, offset) pairs with one 128-byte line.  A
// word becomes eight bf16 with one shift and one and-or per pair: the bits
// 0x4300 | q are exactly the bf16 number 128 + q, so the MFMAs sum
// x * (128 + q) over the group, and one more MFMA per 32 weights against
// bf16 ones gives the group's sum of x.  Then
//   sum x * (lo + q*s) = s * sum x*(128 + q) + (lo - 128*s) * sum x
// folds the group's scale and offset in after its MFMAs.  The A operand
// takes the same weights in natural order (lane kq: kq*32 + 8h + 0..7 for
// MFMA h), matching the code word layout (even weights in the low
// half-words, odd weights in the high half-words).
template <int MODE>
__device__ __forceinline__ void group_weights_q4(
    const FfnArgs& a, int g, bool shared, int N, int K, const uint8_t*& c0,
    const uint8_t*& c1, const float*& q0, const float*& q1,
    const void*& bias) {
  const size_t cmat = (size_t)N * (K / 2);              // code bytes
  const size_t qmat = (size_t)N * (K / Q4_GROUP) * 2;   // floats
  c1 = nullptr;
  q1 = nullptr;
  if (MODE == DOWN) {
    c0 = shared ? (const uint8_t*)a.sw2 : (const uint8_t*)a.w2 + (size_t)g * cmat;
    q0 = shared ? a.sw2q : a.w2q + (size_t)g * qmat;
    bias = shared ? a.sb2
                  : (a.b2 ? (const char*)a.b2 + (size_t)g * N * 2 : nullptr);
  } else {
    c0 = shared ? (const uint8_t*)a.sw1 : (const uint8_t*)a.w1 + (size_t)g * cmat;
    q0 = shared ? a.sw1q : a.w1q + (size_t)g * qmat;
    if (MODE == UP_SWIGLU) {
      c1 = shared ? (const uint8_t*)a.sw_up
                  : (const uint8_t*)a.w_up + (size_t)g * cmat;
      q1 = shared ? a.sw_upq : a.w_upq + (size_t)g * qmat;
      bias = nullptr;
    } else {
      bias = shared ? a.sb1 : (const char*)a.b1 + (size_t)g * N * 2;
    }
  }
}

template <int NMAT, int RT, int CG>
struct Q4Buf {
  u32x4 code[NMAT][CG];   // 32 codes of one weight row, four words
  f32x2 qp[NMAT][CG];     // that row's (scale, offset) for the group
  u32x4 a[RT][4];         // 32 bf16 of one token row per row tile
};

// One code word -> the eight bf16 of an MFMA B operand: element pair j is
// nibbles j and j + 4, each or-ed into bf16 128.0.  mask and magic arrive in
// registers so that every element pair is one three-operand and-or (with
// literal constants the compiler emits a separate and and or).
__device__ __forceinline__ bf16x8 q4_operand(uint32_t word, uint32_t mask,
                                              uint32_t magic) {
  V16 r;
  r.u[0] = (word & mask) | magic;
  r.u[1] = ((word >> 4) & mask) | magic;
  r.u[2] = ((word >> 8) & mask) | magic;
  r.u[3] = ((word >> 12) & mask) | magic;
  return r.h;
}

using gchar = const __attribute__((address_space(1))) char;

// QL: each wave copies the (scale, offset) tiles of its whole K range into
// LDS once (whole 16-byte chunks, coalesced) and reads each step's pair
// from there; otherwise every step loads its pairs (8 bytes per lane, 16
// distinct per instruction) beside the codes.  Those per-step loads cost
// about an eighth of the up GEMM's time: as many load instructions as the
// codes for a sixteenth of the bytes.
extern __shared__ __attribute__((aligned(16))) char q4_lds[];

// LDS bytes the QL variant needs (dynamic; its waves' pair tiles)
constexpr int q4_ql_bytes(int ngroups, int nmat, int cg) {
  return ST_WAVES * nmat * cg * ((ngroups + ST_WAVES - 1) / ST_WAVES) * 128;
}
constexpr int Q4_QL_MAX = 64 * 1024;

template <int MODE, int RT, int CG, int PF, bool QL>
__global__ __launch_bounds__(ST_WAVES * 64) void ffn_stream_q4_kernel(FfnArgs a) {
  constexpr int NMAT = MODE == UP_SWIGLU ? 2 : 1;
  __shared__ f32x4 red[ST_WAVES - 1][NMAT * CG * RT][64];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = blockIdx.y;
  const Group gr = group_of(g, a.offsets, a.E, a.T, a.k);
  if (gr.rows <= 0) return;                 // uniform over the workgroup
  const int N = MODE == DOWN ? a.d : a.d_ff;
  const int K = MODE == DOWN ? a.d_ff : a.d;
  const int n0 = blockIdx.x * 16 * CG;
  if (n0 >= N) return;                      // uniform over the workgroup
  const uint8_t* cm[2];
  const float* qm[2];
  const void* biasv;
  group_weights_q4<MODE>(a, g, gr.shared, N, K, cm[0], cm[1], qm[0], qm[1],
                         biasv);

  const int col = lane & 15;   // B: weight row n0+16c+col; A: token row
  const int kq = lane >> 4;    // 32-weight quarter of the group
  const int ngroups = K / Q4_GROUP;
  const int s_beg = wave * ngroups / ST_WAVES;
  const int my_steps = (wave + 1) * ngroups / ST_WAVES - s_beg;
  // code and (scale, offset) tiles: wave-uniform bases (scalar registers)
  // plus 32-bit lane offsets, so each load takes one offset register
  gchar* crow[NMAT][CG];
  gchar* qrow[NMAT][CG];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      // 16-row block of column group c (a partial last group re-reads the
      // last block and stores nothing for it)
      const int nb = min((n0 + 16 * c) >> 4, N / 16 - 1);
      const size_t tile = (size_t)nb * ngroups + s_beg;
      crow[m][c] = (gchar*)uniform_ptr((const char*)cm[m] + tile * 1024);
      qrow[m][c] = (gchar*)uniform_ptr((const char*)qm[m] + tile * 128);
    }
  const uint32_t c_lane = lane * 16, q_lane = col * 8;
  // QL: this wave's pair tiles, [m][c][step] x 128 bytes
  const int spw = (ngroups + ST_WAVES - 1) / ST_WAVES;
  char* qw = q4_lds + (size_t)wave * (NMAT * CG * spw * 128);
  if constexpr (QL) {
    // all of a lane's chunks in flight at once, then into LDS (QJ: chunks
    // per lane per tile at the largest QL size)
    constexpr int QJ = Q4_QL_MAX / (ST_WAVES * NMAT * CG * 1024);
    u32x4 qt[NMAT][CG][QJ];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int j = 0; j < QJ; ++j) {
          const int i = lane + 64 * j;
          if (i < my_steps * 8)
            qt[m][c][j] = *reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(
                qrow[m][c] + (uint32_t)i * 16u);
        }
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int j = 0; j < QJ; ++j) {
          const int i = lane + 64 * j;
          if (i < my_steps * 8)
            *reinterpret_cast<u32x4*>(qw + (m * CG + c) * spw * 128 + i * 16) = qt[m][c][j];
        }
  }
  V16 ones;
  ones.u = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  uint32_t mask, magic;   // nibble pair mask, bf16 128.0 in both halves
  asm("s_mov_b32 %0, %1" : "=s"(mask) : "i"(0x000F000F));
  asm("s_mov_b32 %0, %1" : "=s"(magic) : "i"(0x43004300));

  for (int rg = 0; rg < gr.rows; rg += RT * 16) {
    const int ntile = min(RT, (gr.rows - rg + 15) >> 4);
    const bf16* arow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int i = min(rg + t * 16 + col, gr.rows - 1);
      arow[t] = a_row<MODE, bf16>(a, gr, i, K) + s_beg * Q4_GROUP + kq * 32;
    }
    f32x4 acc[NMAT][CG][RT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[m][c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    Q4Buf<NMAT, RT, CG> buf[PF];
    auto load = [&](Q4Buf<NMAT, RT, CG>& b, int s) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int c = 0; c < CG; ++c) {
          // codes stream once: non-temporal (the scale/offset pairs,
          // 1/16 of the bytes, measured better as ordinary loads)
          b.code[m][c] = __builtin_nontemporal_load(
              reinterpret_cast<const __attribute__((address_space(1))) u32x4*>(
                  crow[m][c] + (c_lane + (uint32_t)s * 1024)));
          if constexpr (!QL)
            b.qp[m][c] = *reinterpret_cast<const __attribute__((address_space(1))) f32x2*>(
                qrow[m][c] + (q_lane + (uint32_t)s * 128));
        }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if (t < ntile) {
#pragma unroll
          for (int h = 0; h < 4; ++h) b.a[t][h] = ldg16(arow[t] + s * Q4_GROUP + h * 8);
        }
      }
    };
    auto compute = [&](const Q4Buf<NMAT, RT, CG>& b, int st) {
      f32x2 qp[NMAT][CG];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int c = 0; c < CG; ++c)
          qp[m][c] = QL ? *reinterpret_cast<const f32x2*>(
                              qw + ((m * CG + c) * spw + st) * 128 + col * 8)
                        : b.qp[m][c];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if (t < ntile) {
          f32x4 xs = f32x4{0.f, 0.f, 0.f, 0.f};
          f32x4 pg[NMAT][CG];
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int c = 0; c < CG; ++c) pg[m][c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int h = 0; h < 4; ++h) {
            V16 av;
            av.u = b.a[t][h];
            xs = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av.h, ones.h, xs, 0, 0, 0);
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int c = 0; c < CG; ++c)
                pg[m][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    av.h, q4_operand(b.code[m][c][h], mask, magic), pg[m][c], 0, 0, 0);
          }
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int c = 0; c < CG; ++c) {
              const float sc = qp[m][c].x;
              const float cl = qp[m][c].y - 128.0f * sc;
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[m][c][t][r] =
                    fmaf(cl, xs[r], fmaf(sc, pg[m][c][r], acc[m][c][t][r]));
            }
        }
      }
    };
#pragma unroll
    for (int p = 0; p < PF; ++p)
      if (p < my_steps) load(buf[p], p);
    for (int s0 = 0; s0 < my_steps; s0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        const int st = s0 + p;
        if (st < my_steps) {
          compute(buf[p], st);
          if (st + PF < my_steps) load(buf[p], st + PF);
        }
      }
    }

    // K-split reduction: waves 1..3 park their sums, wave 0 adds in order
    if (wave > 0) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
          for (int t = 0; t < RT; ++t)
            red[wave - 1][(m * CG + c) * RT + t][lane] = acc[m][c][t];
    }
    __syncthreads();
    if (wave == 0) {
#pragma unroll
      for (int w = 0; w < ST_WAVES - 1; ++w)
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int c = 0; c < CG; ++c)
#pragma unroll
            for (int t = 0; t < RT; ++t)
              acc[m][c][t] += red[w][(m * CG + c) * RT + t][lane];
      // epilogue: lane holds column n0+16c+col, rows rg + 16t + 4*kq + r
      bf16* outp = (bf16*)(MODE == DOWN ? a.y : a.h);
#pragma unroll
      for (int c = 0; c < CG; ++c) {
        const int n = n0 + 16 * c + col;
        if (n >= N) continue;
        float bias = 0.f;
        if (MODE != UP_SWIGLU && biasv) bias = (float)((const bf16*)biasv)[n];
#pragma unroll
        for (int t = 0; t < RT; ++t) {
          if (t < ntile) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const int i = rg + t * 16 + kq * 4 + r;
              if (i < gr.rows) {
                float v;
                if (MODE == UP_SWIGLU)
                  v = silu(acc[0][c][t][r]) * acc[NMAT - 1][c][t][r];
                else if (MODE == UP_GELU) v = gelu_erf(acc[0][c][t][r] + bias);
                else v = acc[0][c][t][r] + bias;
                outp[(size_t)(gr.out0 + i) * N + n] = (bf16)v;
              }
            }
          }
        }
      }
    }
    __syncthreads();   // red is reused by the next row group
  }
}

// 16*cg columns per workgroup: as many as the grid allows while it still
// covers the chip.  cg 4 only for the down kernel with one row tile: the
// up kernel (two matrices) or two row tiles at cg 4 would need more
// registers than two waves per SIMD leave.
template <int MODE, int RT, int CG, int PF>
void launch_q4_shape(const FfnArgs& a, dim3 grid, hipStream_t s) {
  constexpr int NMAT = MODE == UP_SWIGLU ? 2 : 1;
  const int K = MODE == DOWN ? a.d_ff : a.d;
  const int qb = q4_ql_bytes(K / Q4_GROUP, NMAT, CG);
  if (qb <= Q4_QL_MAX)
    ffn_stream_q4_kernel<MODE, RT, CG, PF, true><<<grid, ST_WAVES * 64, qb, s>>>(a);
  else
    ffn_stream_q4_kernel<MODE, RT, CG, PF, false><<<grid, ST_WAVES * 64, 0, s>>>(a);
}

template <int MODE>
hipError_t launch_q4(const FfnArgs& a, hipStream_t s) {
  const int N = MODE == DOWN ? a.d : a.d_ff;
  const int G = a.E + a.n_shared;
  const auto blocks = [&](int cols) { return (long long)((N + cols - 1) / cols) * G; };
  const bool rt1 = a.T <= 16;   // a token picks an expert at most once
  const int cg = MODE == DOWN && rt1 && blocks(64) >= 512 ? 4 : (blocks(32) >= 512 ? 2 : 1);
  dim3 grid((N + 16 * cg - 1) / (16 * cg), G);
  if (cg == 4) {
    // no in-wave prefetch: 132 VGPRs, and the waves of the other
    // workgroup on the CU cover the load latency (down GEMM 50.3 -> 48.1 us
    // against a two-step ring)
    if constexpr (MODE == DOWN) launch_q4_shape<MODE, 1, 4, 1>(a, grid, s);
  } else if (cg == 2) {
    if (rt1) launch_q4_shape<MODE, 1, 2, 2>(a, grid, s);
    else launch_q4_shape<MODE, 2, 2, 2>(a, grid, s);
  } else {
    if (rt1) launch_q4_shape<MODE, 1, 1, 3>(a, grid, s);
    else launch_q4_shape<MODE, 2, 1, 2>(a, grid, s);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_q4_up(const FfnArgs& a, hipStream_t s) {
  if (a.act == 1) return launch_q4<UP_SWIGLU>(a, s);
  return launch_q4<UP_GELU>(a, s);
}

hipError_t launch_q4_down(const FfnArgs& a, hipStream_t s) {
  return launch_q4<DOWN>(a, s);
}

}  // namespace moe
