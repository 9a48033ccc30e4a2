// Expert FFNs over each expert's kept rows: the dense contraction of the
// layer, run as grouped GEMMs on bf16 MFMA with float32 accumulation.
//
// Every expert runs once over the batch of tokens grouped to it
// (hassanahmed.net "Mixture of Experts explained": a real kernel groups
// tokens by expert and runs each expert once; letsbuildsolutions.com "How
// Mixture of Experts Works", Gating Mechanism: grouped GEMM instead of the
// per-expert loop).  Experts are GELU MLPs with biases (randomcommits.com
// "Mixture-of-Experts routing", How a sparse MoE layer works) or SwiGLU
// w_down(silu(w_gate x) * w_up x) without biases (getnybble.com "Mixture of
// Experts (MoE)", Implementing a complete MoE layer), plus an optional
// always-on shared expert (same page, DeepSeek-V3).
//
// Groups: g < E is routed expert g, rows [offsets[g], offsets[g+1]) of the
// output, A-row r taken from x[perm[r] / k] (gather on load, no permuted
// copy of x); g == E is the shared expert, rows T*k + t for t < T.
//
//   up    H[r, n]  = act(A[r,:] . W1[g, n, :]) (SwiGLU: silu(gate) * up)
//   down  Y[r, n]  = H[r,:] . W2[g, n, :] (+ b2)
//
// Three bf16 schedules, picked on the host from the shapes only (average
// assignments per expert T*k/E):
//   stream  up to 64 (decode): a workgroup owns 32 output columns, its
//           waves split K, and each streams its weight rows once from HBM
//           straight into MFMA B registers (16x16x32) with a 3-deep register
//           prefetch ring; the handful of token rows ride along as the A
//           operand; partial sums meet in LDS.
//   panel   up to 256 (many experts, moderate batch): a workgroup owns up to
//           256 rows of one expert and 256 weight rows over all of K; the
//           weights stream once from HBM into MFMA B registers, the token
//           rows are shared through LDS.
//   tiled   more (prefill): 256-row by 256-column workgroup tiles,
//           A and B loaded straight into XOR-swizzled LDS stages, 32x32x16
//           MFMAs, the activation fused into the epilogue, the output tile
//           staged through LDS for 16-byte row stores, and each XCD's last
//           round of tiles split along K over its CUs.
// 4-bit weights use the stream schedule at every batch size; float32
// problems use a plain float32 kernel (same grouping).  bf16 weights may
// also come in tiled order (wquant 2, moe_tile_bf16: 1 KiB tiles of 16 rows
// x 32 columns in 16x16x32 operand order); every bf16 schedule has a
// variant (template flag TW) that loads those tiles as they are.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

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

template <int MODE>
__device__ __forceinline__ void group_weights(const FfnArgs& a, int g,
                                              bool shared, int N, int K,
                                              const void*& w0,
                                              const void*& w1,
                                              const void*& bias) {
  const size_t esz = a.dtype == 1 ? 2 : 4;
  const size_t mat = (size_t)N * K * esz;
  if (MODE == DOWN) {
    w0 = shared ? a.sw2 : (const char*)a.w2 + (size_t)g * mat;
    w1 = nullptr;
    const void* b = shared ? a.sb2 : (a.b2 ? (const char*)a.b2 + (size_t)g * N * esz : nullptr);
    bias = b;
  } else if (MODE == UP_SWIGLU) {
    w0 = shared ? a.sw1 : (const char*)a.w1 + (size_t)g * mat;
    w1 = shared ? a.sw_up : (const char*)a.w_up + (size_t)g * mat;
    bias = nullptr;
  } else {
    w0 = shared ? a.sw1 : (const char*)a.w1 + (size_t)g * mat;
    w1 = nullptr;
    bias = shared ? a.sb1 : (const char*)a.b1 + (size_t)g * N * esz;
  }
}

// ===========================================================================
// stream schedule (bf16)
// ===========================================================================
// A workgroup owns 32 output columns (two groups of 16) of one group; its 4
// waves split the K steps into contiguous quarters, stream their weight rows
// into registers (3-deep prefetch ring) and add their partial sums through
// LDS in the fixed order 0,1,2,3.  Two column groups per workgroup halve the
// token-row (A) reads per weight byte.
//
// Weight loads are non-temporal and cover whole 128-byte lines: a load
// instruction reads 8 rows x 128 bytes (lane l: row l / 8, bytes 16 * (l %
// 8) of the step), which streams HBM at the rate of a plain sequential read
// (the MFMA operand order, 16 rows x 4 interleaved 16-byte pieces per
// instruction, reads the same bytes about 10% slower).  Each step's weight
// registers then pass through a per-wave LDS slot into MFMA B order.
constexpr int ST_WAVES = 4;
constexpr int ST_KSTEP = 64;         // K per step (two 16x16x32 MFMAs)
constexpr int ST_PF = 3;             // prefetch ring depth (steps)

template <int NMAT, int RT, int CG>
struct StreamBuf {
  u32x4 b[NMAT][CG][2];      // rows 8h + lane/8 of group c, 16 bytes each
  u32x4 a[RT][2];            // 16 bf16 of one token row per row tile
};

// CG = 16-column groups per workgroup.
// TW: weights in tiled order (one 1 KiB tile per MFMA B operand, read
// straight into registers; no reshuffle).
template <int MODE, int RT, int CG, bool TW>
__global__ __launch_bounds__(ST_WAVES * 64) void ffn_stream_kernel(FfnArgs a) {
  constexpr int NMAT = MODE == UP_SWIGLU ? 2 : 1;
  __shared__ f32x4 red[ST_WAVES - 1][NMAT * CG * RT][64];
  __shared__ u32x4 xs[TW ? 1 : ST_WAVES][NMAT * CG * 2][64];   // reshuffle
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int g = blockIdx.y;
  const Group gr = group_of(g, a.offsets, a.E, a.T, a.k);
  if (gr.rows <= 0) return;                 // uniform over the workgroup
  const int N = MODE == DOWN ? a.d : a.d_ff;
  const int K = MODE == DOWN ? a.d_ff : a.d;
  const int n0 = blockIdx.x * 16 * CG;
  if (n0 >= N) return;                      // uniform over the workgroup
  const void *w0v, *w1v, *biasv;
  group_weights<MODE>(a, g, gr.shared, N, K, w0v, w1v, biasv);
  const bf16* wm[2] = {(const bf16*)w0v, (const bf16*)w1v};

  const int col = lane & 15;   // B: weight row n0+col; A: token row
  const int kq = lane >> 4;    // 16-wide k slice of the 64-wide step
  const int nsteps = K / ST_KSTEP;
  const int s_beg = wave * nsteps / ST_WAVES;
  const int my_steps = (wave + 1) * nsteps / ST_WAVES - s_beg;
  // A operand of MFMA h: 8 elements at koff + 8h (row-major weights:
  // piece 2kq + h of the step) or koff + 32h (tiled weights: the tile's
  // columns 8kq .. 8kq + 7 of each 32-column block)
  const int koff = s_beg * ST_KSTEP + kq * (TW ? 8 : 16);
  constexpr int AH = TW ? 32 : 8;
  // tiled weights: the tile of rows n0 + 16c (clamped to the last row
  // block) and the wave's first 32-column block, this lane's 16 bytes
  const bf16* btile[NMAT][CG];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int c = 0; c < CG; ++c)
      btile[m][c] = wm[m] +
                    ((size_t)min((n0 >> 4) + c, N / 16 - 1) * (K / 32) + 2 * s_beg) * 512 +
                    lane * 8;
  // weight rows 16c + 8h + lane/8 of column group c, bytes 16 * (lane % 8)
  // of each step; a partial last group re-reads row N-1 and stores nothing
  // for it
  const bf16* brow[NMAT][CG][2];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int h = 0; h < 2; ++h)
        brow[m][c][h] = wm[m] +
                        (size_t)min(n0 + 16 * c + 8 * h + (lane >> 3), N - 1) * K +
                        s_beg * ST_KSTEP + (lane & 7) * 8;
  // MFMA B order: lane (col, kq), MFMA h holds row col, 16-byte piece
  // 2kq + h of the step (the A operand below takes the same pieces); in the
  // load order that is register col / 8, lane 8 * (col % 8) + 2kq + h
  const int xsrc = col >> 3, xlane = 8 * (col & 7) + 2 * kq;

  for (int rg = 0; rg < gr.rows; rg += RT * 16) {
    const int ntile = min(RT, (gr.rows - rg + 15) >> 4);
    const bf16* arow[RT];
#pragma unroll
    for (int t = 0; t < RT; ++t) {
      const int i = min(rg + t * 16 + col, gr.rows - 1);
      arow[t] = a_row<MODE, bf16>(a, gr, i, K) + koff;
    }
    f32x4 acc[NMAT][CG][RT];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int t = 0; t < RT; ++t) acc[m][c][t] = f32x4{0.f, 0.f, 0.f, 0.f};

    StreamBuf<NMAT, RT, CG> buf[ST_PF];
    auto load = [&](StreamBuf<NMAT, RT, CG>& b, int s) {
      const int k0 = s * ST_KSTEP;
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            b.b[m][c][h] = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                TW ? btile[m][c] + (size_t)(2 * s + h) * 512 : brow[m][c][h] + k0));
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if (t < ntile) {
          b.a[t][0] = ldg16(arow[t] + k0);
          b.a[t][1] = ldg16(arow[t] + k0 + AH);
        }
      }
    };
    // the step's weight registers into this wave's LDS slot (load order);
    // the slot's previous reads are done (in-order LDS within a wave)
    auto stage = [&](const StreamBuf<NMAT, RT, CG>& b) {
      if constexpr (TW) return;
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            xs[wave][(m * CG + c) * 2 + h][lane] = b.b[m][c][h];
    };
    auto compute = [&](const StreamBuf<NMAT, RT, CG>& b) {
      u32x4 wb[NMAT][CG][2];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int c = 0; c < CG; ++c)
#pragma unroll
          for (int h = 0; h < 2; ++h)
            wb[m][c][h] = TW ? b.b[m][c][h]
                             : xs[TW ? 0 : wave][(m * CG + c) * 2 + xsrc][xlane + h];
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if (t < ntile) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            V16 av;
            av.u = b.a[t][h];
#pragma unroll
            for (int m = 0; m < NMAT; ++m)
#pragma unroll
              for (int c = 0; c < CG; ++c) {
                V16 bv;
                bv.u = wb[m][c][h];
                acc[m][c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                    av.h, bv.h, acc[m][c][t], 0, 0, 0);
              }
          }
        }
      }
    };
#pragma unroll
    for (int p = 0; p < ST_PF; ++p)
      if (p < my_steps) load(buf[p], p);
    for (int s0 = 0; s0 < my_steps; s0 += ST_PF) {
#pragma unroll
      for (int p = 0; p < ST_PF; ++p) {
        const int s = s0 + p;
        if (s < my_steps) {
          stage(buf[p]);
          const StreamBuf<NMAT, RT, CG> cur = buf[p];
          if (s + ST_PF < my_steps) load(buf[p], s + ST_PF);
          compute(cur);
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

// ===========================================================================
// stream schedule, 4-bit weights
// ===========================================================================
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
  float2 qp[NMAT][CG];    // that row's (scale, offset) for the group
  u32x4 a[RT][4];         // 32 bf16 of one token row per row tile
};

__device__ __forceinline__ bf16x8 q4_operand(uint32_t word) {
  V16 r;
  r.u[0] = 0x43004300u | (word & 0x000F000Fu);
  r.u[1] = 0x43004300u | ((word >> 4) & 0x000F000Fu);
  r.u[2] = 0x43004300u | ((word >> 8) & 0x000F000Fu);
  r.u[3] = 0x43004300u | ((word >> 12) & 0x000F000Fu);
  return r.h;
}

template <int MODE, int RT, int CG, int PF>
__global__ __launch_bounds__(ST_WAVES * 64) void ffn_stream_q4_kernel(FfnArgs a) {
  constexpr int NMAT = MODE == UP_SWIGLU ? 2 : 1;
  __shared__ f32x4 red[ST_WAVES - 1][NMAT * CG * RT][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
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
  const uint8_t* crow[NMAT][CG];
  const float2* qrow[NMAT][CG];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int c = 0; c < CG; ++c) {
      // 16-row block of column group c (a partial last group re-reads the
      // last block and stores nothing for it)
      const int nb = min((n0 + 16 * c) >> 4, N / 16 - 1);
      const size_t tile = (size_t)nb * ngroups + s_beg;
      crow[m][c] = cm[m] + tile * 1024 + lane * 16;
      qrow[m][c] = (const float2*)qm[m] + tile * 16 + col;
    }
  V16 ones;
  ones.u = u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};

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
              reinterpret_cast<const u32x4*>(crow[m][c] + (size_t)s * 1024));
          b.qp[m][c] = qrow[m][c][s * 16];
        }
#pragma unroll
      for (int t = 0; t < RT; ++t) {
        if (t < ntile) {
#pragma unroll
          for (int h = 0; h < 4; ++h) b.a[t][h] = ldg16(arow[t] + s * Q4_GROUP + h * 8);
        }
      }
    };
    auto compute = [&](const Q4Buf<NMAT, RT, CG>& b) {
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
                    av.h, q4_operand(b.code[m][c][h]), pg[m][c], 0, 0, 0);
          }
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int c = 0; c < CG; ++c) {
              const float sc = b.qp[m][c].x;
              const float cl = b.qp[m][c].y - 128.0f * sc;
#pragma unroll
              for (int r = 0; r < 4; ++r)
                acc[m][c][t][r] += sc * pg[m][c][r] + cl * xs[r];
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
          compute(buf[p]);
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

// ===========================================================================
// tiled schedule (bf16)
// ===========================================================================
// Workgroup tile BM x 256 (BM = 256) over BK = 64 slices of K, eight waves
// (two per SIMD) in a 2 x 4 grid, each wave (BM/2) x 64 of 32x32x16 MFMA
// tiles.
//
// A and B slices go from global memory straight into LDS (direct-to-LDS
// loads, 16 bytes per lane, one instruction = 8 rows x 128 bytes, so every
// row segment is read whole).  LDS rows are 128 bytes; 16-byte chunk c of
// row r sits at position c ^ key(r) so that the MFMA operand reads (32 rows,
// one chunk) spread over all banks.  The key depends only on the low row
// bits, which makes the swizzled offset of a lane the same for every 32-row
// tile: one register per K-substep, tile offsets are immediates.  Two stages
// live in four distinct arrays so the compiler sees that the stage being
// loaded never aliases the stage being read: the next slice loads during the
// MFMAs.
//
// Tile order: logical tiles run expert by expert, and inside an expert
// n-block by n-block with the m-tiles innermost, so neighbouring tiles share
// weight (B) slices and token (A) slices.  Workgroups are handed to the 8
// XCDs round-robin by id; the id is remapped so that each XCD receives a
// contiguous run of logical tiles and its L2 serves the shared slices.
constexpr int TL_BN = 256;   // B rows per tile (SwiGLU: 128 gate + 128 up)
constexpr int N_XCD = 8;
// One configuration is launched: 256-row tiles, two 64-wide K stages (one
// slice in flight).  The template also takes narrower slices and deeper
// rings (NS stages, NS - 1 slices in flight); 128-row tiles with six 32-wide
// stages and 256-row tiles with four 32-wide stages both measured slower at
// every batch size past the panel range.
constexpr int TL_WAVES = 8;

// Logical tiles run group by group, n-block by n-block, row tiles (m)
// innermost; group g has ceil(rows/BM) * NB of them.  Whole workgroup of
// NTHR (>= number of groups) threads: thread g < G gets its group's first
// logical tile (excl) and end (incl) from a prefix scan (wave shuffles, then
// wave totals through LDS); every thread gets the total.
template <int NTHR>
__device__ void tile_scan(const FfnArgs& a, int G, int BM, int NB, int& excl,
                          int& incl, int& total) {
  __shared__ int s_wsum[NTHR / 64];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  int span = 0;
  if (t < G) {
    const int rows = t < a.E ? a.offsets[t + 1] - a.offsets[t] : a.T;
    span = ((rows + BM - 1) / BM) * NB;
  }
  incl = span;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  if (lane == 63) s_wsum[wave] = incl;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < NTHR / 64; ++w) {
    const int ws = s_wsum[w];
    if (w < wave) base += ws;
    total += ws;
  }
  incl += base;
  excl = incl - span;
}

// (group, first row, n-block) of logical tile L into s_info, by the thread
// whose group holds it; false for L past the last tile.  Whole workgroup.
__device__ __forceinline__ bool publish_tile(int G, int BM, int NB, int L,
                                             int excl, int incl, int* s_info) {
  const int t = threadIdx.x;
  if (t < G && L >= excl && L < incl) {
    const int nt = (incl - excl) / NB;
    const int r = L - excl;
    const int nb = r / nt;
    s_info[0] = t;
    s_info[1] = (r - nb * nt) * BM;
    s_info[2] = nb;
  }
  __syncthreads();
  return s_info[1] >= 0;
}

// Panel schedule: workgroups reach the 8 XCDs round-robin by id (slot =
// id / 8 on XCD id % 8); runs of NB logical tiles (one panel's n-blocks,
// which share its token rows) are dealt to the XCDs in turn, so XCD x's
// slot j takes tile ((j / NB) * 8 + x) * NB + j % NB.  False for a
// workgroup with no tile (the grid is an upper bound).
template <int NTHR>
__device__ bool find_panel_tile(const FfnArgs& a, int G, int BM, int NB,
                                int* s_info) {
  if (threadIdx.x == 0) s_info[1] = -1;
  int excl, incl, total;
  tile_scan<NTHR>(a, G, BM, NB, excl, incl, total);
  const int slot = blockIdx.x / N_XCD;
  const int L = ((slot / NB) * N_XCD + blockIdx.x % N_XCD) * NB + slot % NB;
  return publish_tile(G, BM, NB, L, excl, incl, s_info);
}

// Tiled schedule: XCD x takes the contiguous run of ceil(total / 8)
// logical tiles from x * ceil(total / 8), so its L2 serves the weight and
// token slices neighbouring tiles share.  The run of n tiles fills
// R = n / cpx whole rounds of the XCD's cpx CUs; the lo = n - R*cpx tiles
// left over would leave most CUs idle in a last round, so (given a split
// workspace, and when s = min(cpx / lo, nk) >= 2) each is cut into s K
// ranges spread over the CUs.  s_info: group, first row, n-block, first and
// end K slice, split item (-1: whole tile), counter index, pieces s.  False
// for a workgroup with no work.
template <int NTHR>
__device__ bool find_tile_split(const FfnArgs& a, int G, int BM, int NB,
                                int nk, int* s_info) {
  if (threadIdx.x == 0) s_info[1] = -1;
  int excl, incl, total;
  tile_scan<NTHR>(a, G, BM, NB, excl, incl, total);
  const int x = blockIdx.x % N_XCD, slot = blockIdx.x / N_XCD;
  const int per = (total + N_XCD - 1) / N_XCD;
  const int first = x * per;
  const int n = max(0, min(per, total - first));
  const int cpx = a.split_part ? a.split_cpx : 0;
  const int R = cpx > 0 ? n / cpx : 0;
  const int lo = n - R * cpx;
  const int sp = (cpx > 0 && lo > 0) ? min(cpx / lo, nk) : 1;
  int L = total, kb = 0, ke = nk, item = -1, ctr = 0;
  if (sp < 2) {
    if (slot < n) L = first + slot;
  } else if (slot < R * cpx) {
    L = first + slot;
  } else {
    const int q = slot - R * cpx;
    if (q < lo * sp) {
      const int tl = q / sp, c = q - tl * sp;
      L = first + R * cpx + tl;
      kb = c * nk / sp;
      ke = (c + 1) * nk / sp;
      item = x * cpx + q;
      ctr = x * cpx + tl;
    }
  }
  if (threadIdx.x == 0) {
    s_info[3] = kb;
    s_info[4] = ke;
    s_info[5] = item;
    s_info[6] = ctr;
    s_info[7] = sp;
  }
  return publish_tile(G, BM, NB, L, excl, incl, s_info);
}

typedef __attribute__((address_space(3))) void lds_void_t;
typedef __attribute__((address_space(1))) void glb_void_t;

// 16 bytes per lane from global memory straight into LDS: lane l's bytes land
// at lds_base + 16*l (lds_base must be the same for the whole wave).  The
// instruction has no destination registers.  It is written as inline asm so
// that the compiler does not track it: its own waitcnt analysis would
// otherwise make every later LDS read wait for all loads in flight.  The
// kernel orders these loads itself with s_waitcnt vmcnt at each slice
// barrier; a compiler-generated vmcnt wait can only wait longer (vector
// loads complete in order).
__device__ __forceinline__ void dma16(const void* src, bf16* lds_base) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      (uint32_t)(uintptr_t)(lds_void_t*)lds_base);   // wave-uniform
  asm volatile(
      "s_mov_b32 m0, %1\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, off"
      :
      : "v"(src), "s"(m0)
      : "memory", "m0");
}

// End of a K slice: wait until at most N of this wave's vector-memory loads
// (the later slices' direct-to-LDS loads) are in flight and all its LDS
// reads are done, then meet the other waves.  A plain s_barrier: the
// workgroup fence of __syncthreads would also wait for the later slices.
template <int N>
__device__ __forceinline__ void slice_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)\n\ts_barrier" ::"n"(N)
               : "memory");
}

// LDS geometry of one K slice of BK bf16 per row: rows of BK*2 bytes, CPR
// 16-byte chunks per row; chunk c of row r sits at position c ^ key(r).  The
// key spreads a 32-row MFMA operand read (one chunk of 32 consecutive rows)
// over all LDS banks and depends only on the row's low bits, so it is the
// same for every 32-row tile.
template <int BK>
struct SliceGeom {
  static constexpr int CPR = BK / 8;         // chunks per row
  static constexpr int RPI = 64 / CPR;       // rows per load instruction
  static constexpr int SUB = BK / 16;        // 32x32x16 MFMA K-substeps
  __device__ static int key(int r) {
    return BK == 64 ? (r >> 1) & 7 : (r >> 2) & 3;
  }
};

// TW: weights in tiled order: a B slice is 16 row blocks x 2 column
// blocks of 1 KiB tiles, each loaded by one direct-to-LDS instruction and
// kept in tile order in LDS (BK = 64).
template <int MODE, int BM, int BK, int NS, int WAVES, bool TW>
__global__ __launch_bounds__(WAVES * 64, 1) void ffn_tiled_kernel(FfnArgs a,
                                                                  int NB) {
  using Geo = SliceGeom<BK>;
  constexpr int TL_THREADS = WAVES * 64;
  constexpr int WGN = WAVES / 2;      // waves along N (2 along M)
  constexpr int WM = BM / 2;          // rows per wave
  constexpr int WN = TL_BN / WGN;     // B rows per wave (128 or 64)
  constexpr int MT = WM / 32;         // 32-row MFMA tiles per wave
  constexpr int NT = WN / 32;         // 32-col MFMA tiles per wave
  constexpr int IA = BM / Geo::RPI / WAVES;      // A loads per wave, slice
  constexpr int IB = TL_BN / Geo::RPI / WAVES;   // B loads per wave, slice
  constexpr int PER = IA + IB;                      // loads per wave, slice
  constexpr int D = NS - 1;                         // slices in flight
  constexpr int SA = BM * BK, SB = TL_BN * BK;      // elements per slice
  static_assert(IA >= 1 && IB >= 1, "every wave loads A and B rows");
  static_assert(!TW || (BK == 64 && IB * WAVES * Geo::RPI == TL_BN &&
                        TL_BN / 16 * 2 == IB * WAVES),
                "tiled weights: one 1 KiB tile per B load instruction");
  // NS stages of A and B slices; every stage index below is a compile-time
  // constant, so the compiler can see that the stage being loaded never
  // aliases the stage being read and does not make LDS reads wait for the
  // loads in flight.
  static_assert(NS >= 2 && NS <= 6, "2 to 6 stages");
  __shared__ __attribute__((aligned(16))) bf16 A0[SA];
  __shared__ __attribute__((aligned(16))) bf16 A1[SA];
  __shared__ __attribute__((aligned(16))) bf16 A2[NS > 2 ? SA : 8];
  __shared__ __attribute__((aligned(16))) bf16 A3[NS > 3 ? SA : 8];
  __shared__ __attribute__((aligned(16))) bf16 A4[NS > 4 ? SA : 8];
  __shared__ __attribute__((aligned(16))) bf16 A5[NS > 5 ? SA : 8];
  __shared__ __attribute__((aligned(16))) bf16 B0[SB];
  __shared__ __attribute__((aligned(16))) bf16 B1[SB];
  __shared__ __attribute__((aligned(16))) bf16 B2[NS > 2 ? SB : 8];
  __shared__ __attribute__((aligned(16))) bf16 B3[NS > 3 ? SB : 8];
  __shared__ __attribute__((aligned(16))) bf16 B4[NS > 4 ? SB : 8];
  __shared__ __attribute__((aligned(16))) bf16 B5[NS > 5 ? SB : 8];
  __shared__ int s_info[9];
  // stage s's arrays (s is a constant after unrolling, so each access names
  // one distinct object)
  auto As = [&](int st) -> bf16* {
    switch (st) {
      case 0: return A0;
      case 1: return A1;
      case 2: return A2;
      case 3: return A3;
      case 4: return A4;
      default: return A5;
    }
  };
  auto Bs = [&](int st) -> bf16* {
    switch (st) {
      case 0: return B0;
      case 1: return B1;
      case 2: return B2;
      case 3: return B3;
      case 4: return B4;
      default: return B5;
    }
  };

  const int G = a.E + a.n_shared;
  const int Kd = MODE == DOWN ? a.d_ff : a.d;
  if (!find_tile_split<TL_THREADS>(a, G, BM, NB, Kd / BK, s_info)) return;
  const int g = s_info[0], r0 = s_info[1], nb = s_info[2];
  const int kb = s_info[3], ke = s_info[4], item = s_info[5];
  const Group gr = group_of(g, a.offsets, a.E, a.T, a.k);
  const int N = MODE == DOWN ? a.d : a.d_ff;
  const int K = MODE == DOWN ? a.d_ff : a.d;
  const int ncols = MODE == UP_SWIGLU ? TL_BN / 2 : TL_BN;   // outputs per tile
  const int nbase = nb * ncols;
  const void *w0v, *w1v, *biasv;
  group_weights<MODE>(a, g, gr.shared, N, K, w0v, w1v, biasv);

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WGN, wn = wave % WGN;
  const int l31 = lane & 31, q = lane >> 5;

  // Loads: wave w fills A rows [w*IA*RPI, (w+1)*IA*RPI) and B rows likewise,
  // RPI rows per instruction; lane l covers row RPI*i + l/CPR, LDS position
  // l%CPR, i.e. global chunk (l%CPR) ^ key(row).  32-bit element offsets.
  const int lr = lane / Geo::CPR;
  const int lp = lane % Geo::CPR;
  const bf16* abase_g = (const bf16*)(MODE == DOWN ? a.h : a.x);
  uint32_t ao[IA];
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int row = (wave * IA + i) * Geo::RPI + lr;
    const int ai = min(r0 + row, gr.rows - 1);
    const int arow_g = MODE == DOWN ? gr.out0 + ai
                                    : (gr.shared ? ai : a.perm[gr.out0 + ai] / a.k);
    ao[i] = (uint32_t)arow_g * (uint32_t)K + ((lp ^ Geo::key(row)) << 3);
  }
  // B rows: SwiGLU block b = r >> 6 holds gate cols [32b, 32b+32) in rows
  // [64b, 64b+32) and the matching up cols in [64b+32, 64b+64), so wave
  // column wn's two N-tiles are a gate tile and its up tile.
  uint32_t bo[IB];
  const bf16* bb[IB];
#pragma unroll
  for (int i = 0; i < IB; ++i) {
    const int row = (wave * IB + i) * Geo::RPI + lr;
    int wrow;
    if (MODE == UP_SWIGLU) {
      bb[i] = (const bf16*)(((row >> 5) & 1) ? w1v : w0v);
      wrow = nbase + 32 * (row >> 6) + (row & 31);
    } else {
      bb[i] = (const bf16*)w0v;
      wrow = nbase + row;
    }
    wrow = min(wrow, N - 1);
    bo[i] = (uint32_t)wrow * (uint32_t)K + ((lp ^ Geo::key(row)) << 3);
    if constexpr (TW) {
      // instruction ii = wave * IB + i loads tile (row block ii / 2 of the
      // slice's B rows, column block ii % 2): weight row block of LDS rows
      // 16 * (ii / 2) .. +15 (SwiGLU: gate or up rows, as above)
      const int ii = wave * IB + i;
      const int r0 = 16 * (ii >> 1);
      int wr0;
      if (MODE == UP_SWIGLU) {
        bb[i] = (const bf16*)(((r0 >> 5) & 1) ? w1v : w0v);
        wr0 = nbase + 32 * (r0 >> 6) + (r0 & 31);
      } else {
        bb[i] = (const bf16*)w0v;
        wr0 = nbase + r0;
      }
      const int rbg = min(wr0 >> 4, N / 16 - 1);
      bo[i] = ((uint32_t)rbg * (uint32_t)(K / 32) + (uint32_t)(ii & 1)) * 512u +
              (uint32_t)(lane * 8);
    }
  }
  auto issue = [&](int kt, bf16* Ad, bf16* Bd) {
    const int k0 = (kb + kt) * BK;
#pragma unroll
    for (int i = 0; i < IA; ++i)
      dma16(abase_g + ao[i] + k0, Ad + (wave * IA + i) * Geo::RPI * BK);
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      if constexpr (TW)
        dma16(bb[i] + bo[i] + (size_t)(kb + kt) * 1024, Bd + (wave * IB + i) * 512);
      else
        dma16(bb[i] + bo[i] + k0, Bd + (wave * IB + i) * Geo::RPI * BK);
    }
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

  const int nk = ke - kb;   // K slices of this piece
  // MFMA operand rows: A rows wm*WM + 32i + l31, B rows wn*64 + 32j + l31;
  // their swizzle key is key(l31) for every tile
  const int akey = Geo::key(l31);
  const int arow0 = (wm * WM + l31) * BK;
  const int brow0 = (wn * WN + l31) * BK;
  // tiled weights in LDS: row l31 of N-tile j is row block
  // (wn*WN + 32j)/16 + l31/16, piece 16*(chunk % 4) + l31 % 16 of column
  // block chunk / 4 (chunk 2ss + q)
  const int tb0 = ((wn * WN) / 16 + (l31 >> 4)) * 1024 + (l31 & 15) * 8 + q * 128;
  // Operands of substep ss+1 are read from LDS before the MFMAs of substep
  // ss are issued, so LDS latency overlaps matrix work.  Two register sets
  // of operands, alternating by substep.
  V16 av[2][MT], bv[2][NT];
  auto fetch = [&](const bf16* Ab, const bf16* Bb, int ss, int set) {
    const int pos = ((ss * 2 + q) ^ akey) << 3;
    const bf16* ap = Ab + arow0 + pos;
    const bf16* bp = TW ? Bb + tb0 + (ss >> 1) * 512 + (ss & 1) * 256 : Bb + brow0 + pos;
    constexpr int BJ = TW ? 2048 : 32 * BK;   // next N-tile
#pragma unroll
    for (int i = 0; i < MT; ++i)
      av[set][i].u = *reinterpret_cast<const u32x4*>(ap + i * 32 * BK);
#pragma unroll
    for (int j = 0; j < NT; ++j)
      bv[set][j].u = *reinterpret_cast<const u32x4*>(bp + j * BJ);
  };
  auto mfmas = [&](int set) {
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[set][i].h, bv[set][j].h, acc[i][j], 0, 0, 0);
  };
  // schedule: the next substep's LDS reads interleaved one by one with this
  // substep's MFMAs
  auto interleave = [&]() {
#pragma unroll
    for (int r = 0; r < MT + NT; ++r) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // one DS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, MT * NT - (MT + NT), 0);
  };
  // The MFMAs of a slice's last substep are issued after the slice barrier,
  // behind the next slice's first LDS reads, so the matrix cores work while
  // those reads are in flight.  Their operands are in registers already (the
  // barrier waited for the reads), so the stage they came from may be
  // refilled meanwhile.  Before the first slice the deferred set holds
  // zeros: its MFMAs add exact zeros.
  constexpr int LS = (Geo::SUB - 1) & 1;   // register set of the last substep
  auto compute_deferred = [&](const bf16* Ab, const bf16* Bb) {
    fetch(Ab, Bb, 0, 0);
    mfmas(LS);   // the previous slice's last substep
    __builtin_amdgcn_sched_group_barrier(0x100, MT + NT, 0);
    __builtin_amdgcn_sched_group_barrier(0x008, MT * NT, 0);
#pragma unroll
    for (int ss = 0; ss + 1 < Geo::SUB; ++ss) {
      const int cur = ss & 1;
      fetch(Ab, Bb, ss + 1, cur ^ 1);
      mfmas(cur);
      interleave();
    }
  };
#pragma unroll
  for (int i = 0; i < MT; ++i) av[LS][i].u = u32x4{0u, 0u, 0u, 0u};
#pragma unroll
  for (int j = 0; j < NT; ++j) bv[LS][j].u = u32x4{0u, 0u, 0u, 0u};

  // Prologue: slices 0..D-1 in flight (clamped to the last slice when the
  // piece is shorter), then wait for slice 0.
#pragma unroll
  for (int s = 0; s < D; ++s) issue(min(s, nk - 1), As(s), Bs(s));
  slice_barrier<(D - 1) * PER>();
  // Main loop, NS slices per trip with constant stage indices.  Slice k
  // reads stage k % NS; before it, slice k + D is issued into stage
  // (k + D) % NS, last read by slice k - 1 (one barrier ago).  After slice k
  // the wave waits until slice k + 1 has landed: all later slices may stay
  // in flight.  The slice body has no branch: near the end the last slice
  // is issued again into the stage just freed (D redundant slices per tile,
  // never read), so every slice issues PER loads and the wait count is
  // constant; the loads, the first LDS reads and the MFMAs of a slice
  // schedule as one block.
  for (int kt = 0; kt < nk; kt += NS) {
#pragma unroll
    for (int u = 0; u < NS; ++u) {
      const int k = kt + u;
      if (k < nk) {
        issue(min(k + D, nk - 1), As((u + D) % NS), Bs((u + D) % NS));
        compute_deferred(As(u), Bs(u));
        slice_barrier<(D - 1) * PER>();
      }
    }
  }
  mfmas(LS);   // the last slice's last substep
  // the redundant tail slices land before the stages are reused below
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // ---- a K piece of a split tile: park the partial sums; the last piece
  // to arrive adds them all in piece order and stores the tile ----
  if (item >= 0) {
    static_assert(MT * NT * 16 * TL_THREADS <= SPLIT_TILE_FLOATS, "split tile");
    const int ctr = s_info[6], sp = s_info[7];
    // 16-byte partials: float4 (i, j, v4) of thread tid at
    // ((i*NT + j)*4 + v4)*TL_THREADS + tid
    f32x4* pp = reinterpret_cast<f32x4*>(a.split_part + (size_t)item * SPLIT_TILE_FLOATS);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j)
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
          pp[((i * NT + j) * 4 + v4) * TL_THREADS + tid] =
              f32x4{acc[i][j][4 * v4], acc[i][j][4 * v4 + 1],
                    acc[i][j][4 * v4 + 2], acc[i][j][4 * v4 + 3]};
    __threadfence();
    __syncthreads();
    if (tid == 0) s_info[8] = atomicAdd(a.split_cnt + ctr, 1);
    __syncthreads();
    if (s_info[8] != sp - 1) return;   // uniform: another piece finishes it
    __threadfence();
    // pieces of a tile are consecutive items (tile tl of the XCD: items
    // x*cpx + tl*sp + 0 .. sp-1); this one is piece pc.  Sum in piece
    // order, one 32x32 accumulator tile at a time (its four loads per
    // piece issued together).
    const int pc = (item % a.split_cpx) % sp;
    const f32x4* p0 = reinterpret_cast<const f32x4*>(
        a.split_part + (size_t)(item - pc) * SPLIT_TILE_FLOATS);
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
      for (int j = 0; j < NT; ++j) {
        f32x4 sum[4];
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4) sum[v4] = f32x4{0.f, 0.f, 0.f, 0.f};
        for (int q = 0; q < sp; ++q) {
          f32x4 pv[4];
          if (q == pc) {
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
              pv[v4] = f32x4{acc[i][j][4 * v4], acc[i][j][4 * v4 + 1],
                             acc[i][j][4 * v4 + 2], acc[i][j][4 * v4 + 3]};
          } else {
#pragma unroll
            for (int v4 = 0; v4 < 4; ++v4)
              pv[v4] = p0[(size_t)q * (SPLIT_TILE_FLOATS / 4) +
                          ((i * NT + j) * 4 + v4) * TL_THREADS + tid];
          }
#pragma unroll
          for (int v4 = 0; v4 < 4; ++v4) sum[v4] += pv[v4];
        }
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * v4 + e] = sum[v4][e];
      }
    if (tid == 0) a.split_cnt[ctr] = 0;   // ready for the next launch
  }

  // ---- epilogue: activation, stage the bf16 tile in LDS, store rows ----
  // The output tile (BM x ncols bf16, row-major) is staged in the A stages
  // and, past their end, in the B stages.
  static_assert(BM * TL_BN <= NS * (SA + SB), "output tile fits the LDS");
  __syncthreads();
  auto ot = [&](int row, int col) -> bf16& {
    const int idx = row * ncols + col;
    const int st = idx / SA;
    if (st < NS) return As(st)[idx - st * SA];
    const int rb = idx - NS * SA;
    return Bs(rb / SB)[rb % SB];
  };
  // 32x32 accumulator layout: lane holds column lane&31; item v is row
  // (v&3) + 4*(lane>>5) + 8*(v>>2).
#pragma unroll
  for (int i = 0; i < MT; ++i) {
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int row = wm * WM + 32 * i + (v & 3) + 4 * q + 8 * (v >> 2);
      if (MODE == UP_SWIGLU) {
        // N-tiles (2p, 2p+1) are a gate tile and its up tile
#pragma unroll
        for (int p = 0; p < NT / 2; ++p) {
          const int c = 32 * (wn * (NT / 2) + p) + l31;
          const float h = silu(acc[i][2 * p][v]) * acc[i][2 * p + 1][v];
          ot(row, c) = (bf16)h;
        }
      } else {
#pragma unroll
        for (int j = 0; j < NT; ++j) {
          const int c = wn * WN + 32 * j + l31;
          const int n = min(nbase + c, N - 1);
          const float bias = biasv ? (float)((const bf16*)biasv)[n] : 0.f;
          float v2 = acc[i][j][v] + bias;
          if (MODE == UP_GELU) v2 = gelu_erf(v2);
          ot(row, c) = (bf16)v2;
        }
      }
    }
  }
  __syncthreads();
  bf16* outp = (bf16*)(MODE == DOWN ? a.y : a.h);
  const int cpr = ncols / 8;   // 16-byte chunks per output row
  for (int idx = tid; idx < BM * cpr; idx += TL_THREADS) {
    const int row = idx / cpr, ch = idx - row * cpr;
    const int i = r0 + row;
    const int n = nbase + ch * 8;
    if (i < gr.rows && n < N) {
      const u32x4 v = *reinterpret_cast<const u32x4*>(&ot(row, ch * 8));
      stg16(outp + (size_t)(gr.out0 + i) * N + n, v);
    }
  }
}


// ===========================================================================
// panel schedule (bf16)
// ===========================================================================
// For experts with a few hundred rows each (many experts, moderate batch):
// the layer is weight-bound there, so every weight byte should cross HBM
// once.  A workgroup owns a panel of up to PN_BM rows of one group and 16*CG
// weight rows per wave (256 per workgroup: SwiGLU 128 gate + the matching
// 128 up rows, else 256 output columns), over the whole of K.  Each wave
// streams its own weight rows from HBM into a register ring, in whole
// 128-byte lines that a per-wave LDS slot reshuffles into 16x16x32 B
// operand order (or, with tiled weights, as 1 KiB tiles already in that
// order); the panel's token rows (A) are read once per workgroup with
// ordinary loads, written to a double-buffered, XOR-swizzled LDS slice and
// read by all eight waves.
// Row tiles past the panel's rows issue no MFMAs and no loads, so a ragged
// expert costs its own rows, not a full tile.  Every load is an ordinary
// compiler-visible load, so the compiler's waits are exact: a wait for one
// slice never waits for later weight loads.
constexpr int PN_KSTEP = 64;     // K per step (two 16x16x32 MFMAs)
// Panel configuration (measured on the DeepSeek-V3 and Switch workloads;
// 192- and 128-row panels, two steps of lookahead, 4 waves x 64 weight rows
// and two 4-wave workgroups per CU were all slower):
constexpr int PN_BM = 256;    // rows per panel
constexpr int PN_L = 1;       // steps of lookahead
constexpr int PN_W = 8;       // waves per workgroup
constexpr int PN_NBG = 2;     // 16-row weight groups per wave
constexpr int PN_RA = 4;      // LDS operand reads issued ahead of the MFMAs


// LDS slice: BM rows of 128 bytes; 16-byte chunk c of row r sits at
// position c ^ ((r >> 1) & 7).
__device__ __forceinline__ int pn_key(int r) { return (r >> 1) & 7; }

// End of a step: this wave's LDS writes and reads are done, then meet the
// other waves.  No vmcnt wait: loads for later steps stay in flight.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int V>
struct IntC {
  static constexpr int value = V;
};

template <int NMAT, int CG>
struct PanelB {
  u32x4 b[NMAT][CG][2];
};

constexpr int pn_gcd(int x, int y) { return y == 0 ? x : pn_gcd(y, x % y); }
constexpr int pn_lcm(int x, int y) { return x / pn_gcd(x, y) * y; }

// BM rows per panel; L steps of lookahead for both operands: step s stores
// A step s+1 into LDS and issues A step s+1+L and weight step s+1+L, so L
// register sets of A and L+1 weight slots are live.  A and weight loads of
// one step are issued together, A first: vector loads complete in order, so
// a wait for A step s+1 also waits for weight step s, which step s needs
// anyway, and for nothing later.
// W waves per workgroup, NBG groups of 16 weight rows per wave (SwiGLU:
// NBG/2 gate groups and the matching up groups).
// TW: weights in tiled order (each weight load reads one 1 KiB tile in MFMA
// operand order; no reshuffle).
template <int MODE, int BM, int L, int W, int NBG, bool TW>
__global__ __launch_bounds__(W * 64, 1) void ffn_panel_kernel(FfnArgs a,
                                                              int NB) {
  constexpr int NMAT = MODE == UP_SWIGLU ? 2 : 1;
  constexpr int CG = NBG / NMAT;                   // 16-column groups / wave
  constexpr int MT = BM / 16;                      // 16-row tiles per panel
  constexpr int COLS = W * 16 * CG;                // output columns / panel
  constexpr int SL = BM * PN_KSTEP;                // elements per slice
  constexpr int AI = BM * PN_KSTEP / 8 / (W * 64); // A loads / lane
  constexpr int NSLOT = L + 1;                     // weight ring slots
  static_assert(CG * NMAT == NBG && AI * W * 64 * 8 == SL, "shape");
  __shared__ __attribute__((aligned(16))) bf16 S0[SL];
  __shared__ __attribute__((aligned(16))) bf16 S1[SL];
  __shared__ u32x4 xs[TW ? 1 : W][NMAT * CG * 2][64];   // reshuffle per wave
  __shared__ int s_info[3];

  const int G = a.E + a.n_shared;
  if (!find_panel_tile<W * 64>(a, G, BM, NB, s_info)) return;
  const int g = s_info[0], r0 = s_info[1], nb = s_info[2];
  const Group gr = group_of(g, a.offsets, a.E, a.T, a.k);
  const int N = MODE == DOWN ? a.d : a.d_ff;
  const int K = MODE == DOWN ? a.d_ff : a.d;
  const int nvalid = min(BM, gr.rows - r0);
  const int ntile = (nvalid + 15) >> 4;
  const void *w0v, *w1v, *biasv;
  group_weights<MODE>(a, g, gr.shared, N, K, w0v, w1v, biasv);
  const bf16* wm[2] = {(const bf16*)w0v, (const bf16*)w1v};

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, kq = lane >> 4;
  const int nbase = nb * COLS;

  // A loads: thread covers rows (i*512 + tid) / 8, chunk tid % 8 of each
  // step (8 threads read one row's 128 bytes); 32-bit element offsets.
  // Rows past the panel re-read its last row (one cached line per
  // instruction): every load is unconditional, which keeps the compiler's
  // wait counts exact across the loop.
  const bf16* abase = (const bf16*)(MODE == DOWN ? a.h : a.x);
  uint32_t ao[AI];
  int lo[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = (i * W * 64 + tid) >> 3;
    const int p = tid & 7;
    const int ri = r0 + min(row, nvalid - 1);
    const int arow_g = MODE == DOWN ? gr.out0 + ri
                                    : (gr.shared ? ri : a.perm[gr.out0 + ri] / a.k);
    ao[i] = (uint32_t)arow_g * (uint32_t)K + (uint32_t)(p << 3);
    lo[i] = row * PN_KSTEP + ((p ^ pn_key(row)) << 3);
  }
  // B: wave column group c holds weight rows nbase + 16*(wave*CG + c) + col.
  // MFMA h of a 64-wide step contracts k-chunk kq + 4h (8 elements) of lane
  // group kq, for A and B alike: with this order the A operand reads of
  // 16 rows x 4 chunks hit every LDS bank once (the order 2kq + h measured
  // about three conflict cycles per read).  A partial last block re-reads
  // row N-1 and stores nothing for it.
  // Weights are loaded in whole 128-byte lines (register h of group c: rows
  // 8h + lane/8, bytes 16 * (lane % 8) of the step; half lines per
  // instruction were slower: DeepSeek-V3 layer 5.75 against 5.51 ms) and
  // pass through a per-wave LDS slot into MFMA order: row col, chunk
  // kq + 4h is register col / 8, lane 8 * (col % 8) + kq + 4h.  Plain loads:
  // the non-temporal hint was mixed here (Switch faster, DeepSeek slower).
  uint32_t boff[CG][2];   // element offsets (same rows in every matrix)
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      boff[c][h] = (uint32_t)min(nbase + 16 * (wave * CG + c) + 8 * h + (lane >> 3), N - 1) *
                       (uint32_t)K + (uint32_t)((lane & 7) * 8);
  const int xsrc = col >> 3, xlane = 8 * (col & 7) + kq;
  // tiled weights: element offset of group c's tile at column block 0
  // (rows clamped to the last row block), this lane's 16 bytes
  uint32_t toff[CG];
#pragma unroll
  for (int c = 0; c < CG; ++c)
    toff[c] = (uint32_t)min((nbase >> 4) + wave * CG + c, N / 16 - 1) *
                  (uint32_t)(K / 32) * 512u + (uint32_t)(lane * 8);
  // MFMA A operand of row tile t, half h: row 16t + col, chunk kq + 4h; the
  // swizzle key of row 16t + col is key(col) for every t.
  const int aoff0 = col * PN_KSTEP + ((kq ^ pn_key(col)) << 3);
  const int aoff1 = col * PN_KSTEP + (((kq + 4) ^ pn_key(col)) << 3);

  const int nk = K / PN_KSTEP;
  u32x4 ar[L][AI];
  // Loads past the last step re-read the last step (cached, never used).
  // the first NA of this thread's A loads (rows below NA * W * 64 / 8)
  auto loadA = [&](auto nac, u32x4 (&r)[AI], int s) {
    constexpr int NA = decltype(nac)::value;
    const int k0 = min(s, nk - 1) * PN_KSTEP;
#pragma unroll
    for (int i = 0; i < NA; ++i) r[i] = ldg16(abase + ao[i] + k0);
  };
  auto storeA = [&](auto nac, const u32x4 (&r)[AI], bf16* S) {
    constexpr int NA = decltype(nac)::value;
#pragma unroll
    for (int i = 0; i < NA; ++i) *reinterpret_cast<u32x4*>(S + lo[i]) = r[i];
  };
  PanelB<NMAT, CG> ring[NSLOT];
  auto loadB = [&](PanelB<NMAT, CG>& b, int s) {
    const int k0 = min(s, nk - 1) * PN_KSTEP;
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h)
          // tiled weights: non-temporal (measured faster there; on the
          // row-major lines the hint was mixed)
          b.b[m][c][h] = TW ? __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
                                  wm[m] + toff[c] + (uint32_t)(2 * min(s, nk - 1) + h) * 512u))
                            : ldg16(wm[m] + boff[c][h] + k0);
  };
  // a weight slot into this wave's LDS slot (load order), then back in MFMA
  // order; the slot's earlier reads are done (in-order LDS within a wave)
  auto stageB = [&](const PanelB<NMAT, CG>& b) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int c = 0; c < CG; ++c)
#pragma unroll
        for (int h = 0; h < 2; ++h) xs[wave][(m * CG + c) * 2 + h][lane] = b.b[m][c][h];
  };

  f32x4 acc[NMAT][CG][MT];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int c = 0; c < CG; ++c)
#pragma unroll
      for (int t = 0; t < MT; ++t) acc[m][c][t] = f32x4{0.f, 0.f, 0.f, 0.f};
  // The K loop for NT active row tiles (a compile-time count, so the loop
  // body is straight-line code: the compiler pipelines the LDS operand reads
  // with the MFMAs and its wait counts stay exact).  Tiles past the panel's
  // rows up to NT hold copies of its last row; their sums are not stored.
  auto kloop = [&](auto ntc) {
    constexpr int NT = decltype(ntc)::value;
    // A rows 0 .. NT*16-1 only: loads per thread
    constexpr int NA = (NT * 16 * 8 + W * 64 - 1) / (W * 64);
    static_assert(NA >= 1 && NA <= AI, "A loads");
    const IntC<NA> na{};
    // MFMAs of one step: half h outermost, so the two MFMAs into one
    // accumulator are a tile sweep apart
    // Per MFMA half h: the half's weight operands are read back from the
    // wave's reshuffle slot (MFMA order), then the A operand of each tile.
    auto compute = [&](const bf16* S, const PanelB<NMAT, CG>& b) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        V16 bw[NMAT][CG];
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int c = 0; c < CG; ++c)
            bw[m][c].u = TW ? b.b[m][c][h]
                            : xs[TW ? 0 : wave][(m * CG + c) * 2 + xsrc][xlane + 4 * h];
        const bf16* sa = S + (h ? aoff1 : aoff0);
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          V16 f;
          f.u = *reinterpret_cast<const u32x4*>(sa + t * 16 * PN_KSTEP);
#pragma unroll
          for (int m = 0; m < NMAT; ++m)
#pragma unroll
            for (int c = 0; c < CG; ++c)
              acc[m][c][t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f.h, bw[m][c].h, acc[m][c][t], 0, 0, 0);
        }
      }
      // order: the first half's weight reads and PN_RA A reads ahead, then
      // each tile's MFMAs followed by the next read (the second half's
      // weight reads come in that stream ahead of its A reads)
      constexpr int NM = NMAT * CG;
      constexpr int RA = PN_RA < 2 * NT ? PN_RA : 2 * NT;
      constexpr int BR = TW ? 0 : NM;   // weight reads of a half from LDS
      __builtin_amdgcn_sched_group_barrier(0x100, BR + RA, 0);   // DS reads
#pragma unroll
      for (int i = 0; i < 2 * NT + BR - RA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, NM, 0);   // MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, RA * NM - BR * NM, 0);
    };
    // Step s (u = s mod U): reads slice s % 2 and weight slot s % (L+1);
    // first writes A step s+1 (register set (s+1) % L) into the other
    // slice, whose readers finished at the last barrier, and its weight
    // slot into the wave's reshuffle slot; reloads the A set and refills
    // the weight slot with step s+1+L, then runs the MFMAs (which read the
    // weights back from the reshuffle slot in MFMA order).
    auto step = [&](int s, int u) {
      bf16* cur = (u & 1) ? S1 : S0;
      bf16* nxt = (u & 1) ? S0 : S1;
      storeA(na, ar[(u + 1) % L], nxt);
      if constexpr (TW) {
        // the MFMAs read the weight slot itself, then it is refilled
        loadA(na, ar[(u + 1) % L], s + 1 + L);
        compute(cur, ring[u % NSLOT]);
        loadB(ring[u % NSLOT], s + 1 + L);
      } else {
        stageB(ring[u % NSLOT]);
        loadA(na, ar[(u + 1) % L], s + 1 + L);
        loadB(ring[u % NSLOT], s + 1 + L);
        compute(cur, ring[u % NSLOT]);
      }
      lds_barrier();
    };
    // prologue in the loop's issue order: A step 0 into S0, then A step j
    // (register set j % L) and weight step j for j = 1..L; weight step 0
    // right after A step 0
    loadA(na, ar[0], 0);
    loadB(ring[0], 0);
    storeA(na, ar[0], S0);
#pragma unroll
    for (int j = 1; j <= L; ++j) {
      loadA(na, ar[j % L], j);
      loadB(ring[j], j);
    }
    lds_barrier();
    // whole trips of U steps (constant slice, set and slot indices), then
    // the remaining steps
    constexpr int U = pn_lcm(2, pn_lcm(L, NSLOT));
    const int ntrip = nk / U;
    for (int tr = 0; tr < ntrip; ++tr) {
#pragma unroll
      for (int u = 0; u < U; ++u) step(tr * U + u, u);
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
      if (ntrip * U + u < nk) step(ntrip * U + u, u);
  };
  // two instances: panels filling at most half the tiles run the half-size
  // loop (more instances overflow the register file)
  static_assert(MT % 2 == 0, "half panel");
  if (ntile > MT / 2) kloop(IntC<MT>{});
  else kloop(IntC<MT / 2>{});

  // epilogue: lane holds column n of group c and rows 16t + 4kq + r
  bf16* outp = (bf16*)(MODE == DOWN ? a.y : a.h);
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const int n = nbase + 16 * (wave * CG + c) + col;
    if (n >= N) continue;
    float bias = 0.f;
    if (MODE != UP_SWIGLU && biasv) bias = (float)((const bf16*)biasv)[n];
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < ntile) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 16 * t + 4 * kq + r;
          if (i < nvalid) {
            float v;
            if (MODE == UP_SWIGLU)
              v = silu(acc[0][c][t][r]) * acc[NMAT - 1][c][t][r];
            else if (MODE == UP_GELU) v = gelu_erf(acc[0][c][t][r] + bias);
            else v = acc[0][c][t][r] + bias;
            outp[(size_t)(gr.out0 + r0 + i) * N + n] = (bf16)v;
          }
        }
      }
    }
  }
}

// ===========================================================================
// float32 schedule
// ===========================================================================
// Linear row-tile id -> (group, first row); false past the last tile.
// Whole workgroup.
__device__ bool find_tile(const FfnArgs& a, int G, int BM, int tile, int* s_info) {
  if (threadIdx.x == 0) {
    int acc = 0, g = 0, r0 = -1;
    for (; g < G; ++g) {
      const int rows = g < a.E ? a.offsets[g + 1] - a.offsets[g] : a.T;
      const int nt = (rows + BM - 1) / BM;
      if (tile < acc + nt) {
        r0 = (tile - acc) * BM;
        break;
      }
      acc += nt;
    }
    s_info[0] = g;
    s_info[1] = r0;
  }
  __syncthreads();
  return s_info[1] >= 0;
}

constexpr int F32_BM = 16;
constexpr int F32_BN = 64;

template <int MODE>
__global__ __launch_bounds__(256) void ffn_f32_kernel(FfnArgs a) {
  __shared__ int s_info[2];
  const int G = a.E + a.n_shared;
  if (!find_tile(a, G, F32_BM, blockIdx.x, s_info)) return;
  const int g = s_info[0], r0 = s_info[1];
  const Group gr = group_of(g, a.offsets, a.E, a.T, a.k);
  const int N = MODE == DOWN ? a.d : a.d_ff;
  const int K = MODE == DOWN ? a.d_ff : a.d;
  const void *w0v, *w1v, *biasv;
  group_weights<MODE>(a, g, gr.shared, N, K, w0v, w1v, biasv);
  const float* w0 = (const float*)w0v;
  const float* w1 = (const float*)w1v;
  const float* bias = (const float*)biasv;
  float* outp = (float*)(MODE == DOWN ? a.y : a.h);
  const int c = blockIdx.y * F32_BN + (threadIdx.x & 63);
  for (int rr = threadIdx.x >> 6; rr < F32_BM; rr += 4) {
    const int i = r0 + rr;
    if (i >= gr.rows || c >= N) continue;
    const float* ar = a_row<MODE, float>(a, gr, i, K);
    float s0 = 0.f, s1 = 0.f;
    for (int kk = 0; kk < K; ++kk) {
      s0 = fmaf(ar[kk], w0[(size_t)c * K + kk], s0);
      if (MODE == UP_SWIGLU) s1 = fmaf(ar[kk], w1[(size_t)c * K + kk], s1);
    }
    float v;
    if (MODE == UP_SWIGLU) v = silu(s0) * s1;
    else if (MODE == UP_GELU) v = gelu_erf(s0 + bias[c]);
    else v = s0 + (bias ? bias[c] : 0.f);
    outp[(size_t)(gr.out0 + i) * N + c] = v;
  }
}

template <int MODE, bool TW>
hipError_t launch_mode(const FfnArgs& a, hipStream_t s, int sched, int rt,
                       int max_tiles) {
  const int N = MODE == DOWN ? a.d : a.d_ff;
  const int G = a.E + a.n_shared;
  if (sched == 0) {
    // two column groups per workgroup unless that leaves too few
    // workgroups to cover the chip
    const int cg = (long long)((N + 31) / 32) * G >= 512 ? 2 : 1;
    dim3 grid((N + 16 * cg - 1) / (16 * cg), G);
    if (cg == 2) {
      if (rt == 1) ffn_stream_kernel<MODE, 1, 2, TW><<<grid, ST_WAVES * 64, 0, s>>>(a);
      else if (rt == 2) ffn_stream_kernel<MODE, 2, 2, TW><<<grid, ST_WAVES * 64, 0, s>>>(a);
      else ffn_stream_kernel<MODE, 4, 2, TW><<<grid, ST_WAVES * 64, 0, s>>>(a);
    } else {
      if (rt == 1) ffn_stream_kernel<MODE, 1, 1, TW><<<grid, ST_WAVES * 64, 0, s>>>(a);
      else if (rt == 2) ffn_stream_kernel<MODE, 2, 1, TW><<<grid, ST_WAVES * 64, 0, s>>>(a);
      else ffn_stream_kernel<MODE, 4, 1, TW><<<grid, ST_WAVES * 64, 0, s>>>(a);
    }
  } else if (sched == 1) {
    // 256-row tiles; max_tiles counts m-tiles.  With
    // a split workspace each XCD may need up to split_cpx more workgroups
    // for the pieces of its last round; their counters start at zero.
    const int ncols = MODE == UP_SWIGLU ? TL_BN / 2 : TL_BN;
    const int NB = (N + ncols - 1) / ncols;
    long long tiles = (long long)max_tiles * NB;
    tiles = (tiles + N_XCD - 1) / N_XCD * N_XCD;
    if (a.split_part) {
      tiles += (long long)N_XCD * a.split_cpx;
      const hipError_t e = launch_fill_zero32(a.split_cnt, (long long)N_XCD * a.split_cpx, s);
      if (e != hipSuccess) return e;
    }
    ffn_tiled_kernel<MODE, 256, 64, 2, TL_WAVES, TW>
        <<<(unsigned)tiles, TL_WAVES * 64, 0, s>>>(a, NB);
  } else if (sched == 4) {
    // max_tiles counts panels of PN_BM rows
    constexpr int cols = PN_W * 16 * (MODE == UP_SWIGLU ? PN_NBG / 2 : PN_NBG);
    const int NB = (N + cols - 1) / cols;
    long long tiles = (long long)(max_tiles + N_XCD - 1) / N_XCD * N_XCD * NB;
    ffn_panel_kernel<MODE, PN_BM, PN_L, PN_W, PN_NBG, TW><<<(unsigned)tiles, PN_W * 64, 0, s>>>(a, NB);
  } else {
    dim3 grid(max_tiles, (N + F32_BN - 1) / F32_BN);
    ffn_f32_kernel<MODE><<<grid, 256, 0, s>>>(a);
  }
  return hipGetLastError();
}

}  // namespace

int device_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      n <= 0)
    return 256;
  return n;
}

// Schedule choice from shapes only (no device readback):
//   f32 -> float32 kernel; bf16 with at most 64 assignments per expert on
//   average -> stream; up to 256 -> panel; otherwise tiled.
int ffn_schedule(int dtype, int T, int k, int E) {
  if (dtype != 1) return 2;
  const long long tk = (long long)T * k;
  if (tk <= 64LL * E) return 0;        // stream
  if (tk <= 256LL * E) return 4;       // panel
  return 1;                            // tiled, 256-row tiles
}

namespace {
struct Plan {
  int sched, rt, max_tiles;
};
Plan plan_of(const FfnArgs& a) {
  Plan p;
  p.sched = ffn_schedule(a.dtype, a.T, a.k, a.E);
  const long long tk = (long long)a.T * a.k;
  p.rt = 4;
  if (p.sched == 0) {
    const int maxrows = a.T;   // a token picks an expert at most once
    p.rt = maxrows <= 16 ? 1 : (maxrows <= 32 ? 2 : 4);
  }
  const int bm = p.sched == 1 ? 256 : (p.sched == 4 ? PN_BM : F32_BM);
  p.max_tiles = (int)((tk + bm - 1) / bm) + a.E +
                (a.n_shared ? (a.T + bm - 1) / bm : 0);
  return p;
}
}  // namespace

// 4-bit weights: the weight-streaming schedule at every batch size (a
// decode-path format; larger batches stay correct, re-streaming the
// weights once per 32 rows of an expert).
template <int MODE>
hipError_t launch_q4(const FfnArgs& a, hipStream_t s) {
  const int N = MODE == DOWN ? a.d : a.d_ff;
  const int G = a.E + a.n_shared;
  const int cg = (long long)((N + 31) / 32) * G >= 512 ? 2 : 1;
  dim3 grid((N + 16 * cg - 1) / (16 * cg), G);
  const bool rt1 = a.T <= 16;   // a token picks an expert at most once
  if (cg == 2) {
    if (rt1) ffn_stream_q4_kernel<MODE, 1, 2, 2><<<grid, ST_WAVES * 64, 0, s>>>(a);
    else ffn_stream_q4_kernel<MODE, 2, 2, 2><<<grid, ST_WAVES * 64, 0, s>>>(a);
  } else {
    if (rt1) ffn_stream_q4_kernel<MODE, 1, 1, 3><<<grid, ST_WAVES * 64, 0, s>>>(a);
    else ffn_stream_q4_kernel<MODE, 2, 1, 2><<<grid, ST_WAVES * 64, 0, s>>>(a);
  }
  return hipGetLastError();
}

hipError_t launch_expert_up(const FfnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.wquant == 1) {   // 4-bit codes
    if (a.act == 1) return launch_q4<UP_SWIGLU>(a, s);
    return launch_q4<UP_GELU>(a, s);
  }
  const Plan p = plan_of(a);
  if (a.wquant == 2) {   // bf16 weights in tiled order
    if (a.act == 1) return launch_mode<UP_SWIGLU, true>(a, s, p.sched, p.rt, p.max_tiles);
    return launch_mode<UP_GELU, true>(a, s, p.sched, p.rt, p.max_tiles);
  }
  if (a.act == 1) return launch_mode<UP_SWIGLU, false>(a, s, p.sched, p.rt, p.max_tiles);
  return launch_mode<UP_GELU, false>(a, s, p.sched, p.rt, p.max_tiles);
}

hipError_t launch_expert_down(const FfnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.wquant == 1) return launch_q4<DOWN>(a, s);   // 4-bit codes
  const Plan p = plan_of(a);
  if (a.wquant == 2) return launch_mode<DOWN, true>(a, s, p.sched, p.rt, p.max_tiles);
  return launch_mode<DOWN, false>(a, s, p.sched, p.rt, p.max_tiles);
}

}  // namespace moe
