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
//           in whole 128-byte lines into a register prefetch ring (three
//           steps; two for the one-row-tile down GEMM), reordered into
//           16x16x32 MFMA B order through a per-wave LDS slot; the handful
//           of token rows ride along as the A operand; partial sums meet in
//           LDS.
//   panel   up to 256 (many experts, moderate batch): a workgroup owns up to
//           256 rows of one expert and 256 weight rows over all of K; the
//           weights stream once from HBM the same way (lines, per-wave LDS
//           reorder), the token rows go straight into LDS and are shared by
//           the workgroup's waves.
//   tiled   more (prefill): 256-row by 256-column workgroup tiles,
//           A and B loaded straight into XOR-swizzled LDS stages, 32x32x16
//           MFMAs, the activation fused into the epilogue, the output tile
//           staged through LDS for 16-byte row stores, and each XCD's last
//           round of tiles split along K over its CUs.
// 4-bit weights use the stream schedule at every batch size (ffn_q4.hip); float32
// problems use a plain float32 kernel (same grouping).  bf16 weights may
// also come in tiled order (wquant 2, moe_tile_bf16: 1 KiB tiles of 16 rows
// x 32 columns in 16x16x32 operand order); every bf16 schedule has a
// variant (template flag TW) that loads those tiles as they are.
#include <utility>

#include "common.hpp"
#include "ffn_common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

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
// into registers (a prefetch ring of ST_PF steps; two for the one-row-tile
// down GEMM, below) and add their partial sums through LDS in the fixed
// order 0,1,2,3.  Two column groups per workgroup halve the token-row (A)
// reads per weight byte.
//
// Weight loads are non-temporal and cover whole 128-byte lines: a load
// instruction reads 8 rows x 128 bytes (lane l: row l / 8, bytes 16 * (l %
// 8) of the step), which streams HBM at the rate of a plain sequential read
// (the MFMA operand order, 16 rows x 4 interleaved 16-byte pieces per
// instruction, reads the same bytes about 10% slower).  Each step's weight
// registers then pass through a per-wave LDS slot into MFMA B order.
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
  // prefetch ring depth: the one-row-tile down GEMM takes two steps, which
  // leaves it under 128 VGPRs, four workgroups per CU: the decode down
  // GEMM's 1024 workgroups are then all resident at once instead of
  // running 1.33 rounds of three per CU
  constexpr int PF = (MODE == DOWN && RT == 1) ? 2 : ST_PF;
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

    StreamBuf<NMAT, RT, CG> buf[PF];
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
    for (int p = 0; p < PF; ++p)
      if (p < my_steps) load(buf[p], p);
    for (int s0 = 0; s0 < my_steps; s0 += PF) {
#pragma unroll
      for (int p = 0; p < PF; ++p) {
        const int s = s0 + p;
        if (s < my_steps) {
          stage(buf[p]);
          const StreamBuf<NMAT, RT, CG> cur = buf[p];
          if (s + PF < my_steps) load(buf[p], s + PF);
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
// tile: one register per K-substep, tile offsets are immediates.  A and B
// have rings of their own (NSA and NSB stages, each stage a distinct array
// so the compiler sees that the stage being loaded never aliases the stage
// being read): 160 KiB of LDS holds five 32 KiB slices, so the operand
// that streams from HBM gets three stages (two slices in flight) and the
// other two.
//
// Tile order: logical tiles run expert by expert, and inside an expert
// n-block by n-block with the m-tiles innermost, so neighbouring tiles share
// weight (B) slices and token (A) slices.  Workgroups are handed to the 8
// XCDs round-robin by id; the id is remapped so that each XCD receives a
// contiguous run of logical tiles and its L2 serves the shared slices.
constexpr int TL_BN = 256;   // B rows per tile (SwiGLU: 128 gate + 128 up)
constexpr int N_XCD = 8;
// One tile shape is launched: 256-row tiles over 64-wide K slices.  The
// template also takes narrower slices and deeper rings; 128-row tiles with
// six 32-wide stages and 256-row tiles with four 32-wide stages both
// measured slower at every batch size past the panel range.
constexpr int TL_WAVES = 8;
// Stages per ring: the up GEMMs' weights stream from HBM (the token rows
// are re-read from L2 and the memory-side cache), so B gets the third
// stage; the down GEMM's A (the hidden rows, written by the up GEMM) is the
// larger stream, so A gets it.  Mixtral-shaped prefill, same box: one
// slice in flight for both, up 3.42 ms and down 1.79 ms; two B slices for
// up 3.29 ms; two A slices for down 1.65 ms.
constexpr int tl_nsa(int mode) { return mode == DOWN ? 3 : 2; }
constexpr int tl_nsb(int mode) { return mode == DOWN ? 2 : 3; }

// Logical tiles run group by group, n-block by n-block, row tiles (m)
// innermost; group g has ceil(rows/BM) * NB of them.  Whole workgroup of
// NTHR (>= number of groups) threads: thread g < G gets its group's first
// logical tile (excl) and end (incl) from a prefix scan (wave shuffles, then
// wave totals through s_wsum, NTHR / 64 ints of LDS); every thread gets the
// total.
template <int NTHR>
__device__ void tile_scan(const FfnArgs& a, int G, int BM, int NB,
                          int* s_wsum, int& excl, int& incl, int& total) {
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
// slot j takes tile ((j / NB) * 8 + x) * NB + j % NB.  Logical tiles run
// group by group and panel by panel with the n-blocks innermost; with
// by_cost, workgroups (which start roughly in id order) take the expensive
// panels first: every panel with more than BM/2 rows (the full-size K loop,
// about twice the matrix work of a half panel) of every group, then each
// group's half panel (its last panel when that holds at most BM/2 rows).
// The up GEMMs use it: in group order DeepSeek-V3's up GEMM left the CUs
// idle 8% of the time at its end (the last CU finishing 270 us after the
// average), and the order took it from 3100 to 3063 us.  The down GEMMs'
// panels are short (38-83 us against 130-286 us there) and ran 1.5-2%
// slower in that order, so they keep group order.  False for a workgroup
// with no tile (the grid is an upper bound).
template <int NTHR>
__device__ bool find_panel_tile(const FfnArgs& a, int G, int BM, int NB,
                                bool by_cost, int* s_info) {
  __shared__ int s_wsum[2][NTHR / 64];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  if (t == 0) s_info[1] = -1;
  // this thread's group: full-loop panels nf and half panels nh (0 or 1;
  // without by_cost every panel counts in the first class)
  int nf = 0, nh = 0, np = 0;
  if (t < G) {
    const int rows = t < a.E ? a.offsets[t + 1] - a.offsets[t] : a.T;
    np = (rows + BM - 1) / BM;
    nh = (by_cost && np > 0 && rows - (np - 1) * BM <= BM / 2) ? 1 : 0;
    nf = np - nh;
  }
  // inclusive prefix sums of the two classes' tile counts (wave shuffles,
  // then wave totals through LDS)
  int inf = nf * NB, inh = nh * NB;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int vf = __shfl_up(inf, o, 64), vh = __shfl_up(inh, o, 64);
    if (lane >= o) {
      inf += vf;
      inh += vh;
    }
  }
  if (lane == 63) {
    s_wsum[0][wave] = inf;
    s_wsum[1][wave] = inh;
  }
  __syncthreads();
  int bf = 0, bh = 0, tf = 0;
#pragma unroll
  for (int w = 0; w < NTHR / 64; ++w) {
    const int wf = s_wsum[0][w], wh = s_wsum[1][w];
    if (w < wave) {
      bf += wf;
      bh += wh;
    }
    tf += wf;
  }
  inf += bf;
  inh += bh;
  const int slot = blockIdx.x / N_XCD;
  const int L = ((slot / NB) * N_XCD + blockIdx.x % N_XCD) * NB + slot % NB;
  if (t < G) {
    const int ef = inf - nf * NB, eh = tf + inh - nh * NB;
    if (L >= ef && L < inf) {          // full-loop panel (L - ef) / NB
      s_info[0] = t;
      s_info[1] = ((L - ef) / NB) * BM;
      s_info[2] = (L - ef) % NB;
    } else if (L >= eh && L < eh + nh * NB) {   // the half panel
      s_info[0] = t;
      s_info[1] = (np - 1) * BM;
      s_info[2] = L - eh;
    }
  }
  __syncthreads();
  return s_info[1] >= 0;
}

// Tiled schedule: XCD x takes the contiguous run of ceil(total / 8)
// logical tiles from x * ceil(total / 8), so its L2 serves the weight and
// token slices neighbouring tiles share.  The run of n tiles fills
// R = n / cpx whole rounds of the XCD's cpx CUs; the lo = n - R*cpx tiles
// left over would leave most CUs idle in a last round, so (given a split
// workspace, and when s = min(cpx / lo, nk) >= 2) each is cut into s K
// ranges spread over the CUs.  s_info (TL_INFO ints of LDS, then the scan's
// NTHR / 64): group, first row, n-block, first and end K slice, split item
// (-1: whole tile), counter index, pieces s.  False for a workgroup with no
// work.
constexpr int TL_INFO = 16;
// A split costs about as much as 50 K slices of a tile (the partial tiles'
// stores, the device-scope fence that makes them visible to the other
// pieces, and the sum): a last round is split only when that takes at
// least TL_SPLIT_MIN_SAVED slices off it, into at most TL_SPLIT_MAX pieces.
constexpr int TL_SPLIT_MIN_SAVED = 48;
constexpr int TL_SPLIT_MAX = 8;
template <int NTHR>
__device__ bool find_tile_split(const FfnArgs& a, int G, int BM, int NB,
                                int nk, int* s_info) {
  if (threadIdx.x == 0) s_info[1] = -1;
  int excl, incl, total;
  tile_scan<NTHR>(a, G, BM, NB, s_info + TL_INFO, excl, incl, total);
  const int x = blockIdx.x % N_XCD, slot = blockIdx.x / N_XCD;
  const int per = (total + N_XCD - 1) / N_XCD;
  const int first = x * per;
  const int n = max(0, min(per, total - first));
  const int cpx = a.split_part ? a.split_cpx : 0;
  const int R = cpx > 0 ? n / cpx : 0;
  const int lo = n - R * cpx;
  int sp = (cpx > 0 && lo > 0) ? min(min(cpx / lo, nk), TL_SPLIT_MAX) : 1;
  if (nk - nk / sp < TL_SPLIT_MIN_SAVED) sp = 1;
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
// at the wave's LDS address + 16*l.  The instruction has no destination
// registers.  It is written as inline asm so that the compiler does not
// track it: its own waitcnt analysis would otherwise make every later LDS
// read wait for all loads in flight.  The kernel orders these loads itself
// with s_waitcnt vmcnt at each slice barrier; a compiler-generated vmcnt
// wait can only wait longer (vector loads complete in order).
// The load uses a wave-uniform 64-bit base in scalar registers and a 32-bit
// per-lane byte offset (the scalar-base addressing form): one vector
// register per load instead of a 64-bit address, and no 64-bit vector add.
// The wave's 64 x 16 bytes land at LDS byte address lds + IMM (lds
// uniform; IMM a constant folded into the m0 write, so that the compiler
// does not keep one register per load for the LDS addresses).  The scalar
// add writes SCC, which the clobber list declares.
template <int IMM>
__device__ __forceinline__ void dma16s(const void* sbase, uint32_t voff,
                                       uint32_t lds) {
  asm volatile(
      "s_add_u32 m0, %2, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %0, %1"
      :
      : "v"(voff), "s"(sbase), "s"(lds), "n"(IMM)
      : "memory", "m0", "scc");
}

// dma16s for loads I... of a wave: load i from sbase(i) at offset voff[i]
// into LDS lds + i * STRIDE.
template <int STRIDE, typename SB, int... I>
__device__ __forceinline__ void dma16s_seq(SB sbase, const uint32_t* voff,
                                           uint32_t lds,
                                           std::integer_sequence<int, I...>) {
  (dma16s<I * STRIDE>(sbase(I), voff[I], lds), ...);
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

constexpr int pn_gcd(int x, int y) { return y == 0 ? x : pn_gcd(y, x % y); }
constexpr int pn_lcm(int x, int y) { return x / pn_gcd(x, y) * y; }

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
template <int MODE, int BM, int BK, int NSA, int NSB, int WAVES, bool TW>
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
  // NSA stages of A slices and NSB of B slices: DA and DB slices in flight
  constexpr int DA = NSA - 1, DB = NSB - 1;
  constexpr int DMAX = DA > DB ? DA : DB;
  // Each slice issues the A slice DA ahead and the B slice DB ahead, the one
  // with less lookahead first; a slice's end waits until only the loads
  // issued after the last one the next slice needs are in flight.
  constexpr int WAITN = DA == DB ? (DA - 1) * PER
                      : DA > DB ? IA + (DB - 1) * PER : IB + (DA - 1) * PER;
  constexpr int SA = BM * BK, SB = TL_BN * BK;      // elements per slice
  static_assert(IA >= 1 && IB >= 1, "every wave loads A and B rows");
  static_assert(!TW || (BK == 64 && IB * WAVES * Geo::RPI == TL_BN &&
                        TL_BN / 16 * 2 == IB * WAVES),
                "tiled weights: one 1 KiB tile per B load instruction");
  // Every stage index below is a compile-time constant, so the compiler can
  // see that the stage being loaded never aliases the stage being read and
  // does not make LDS reads wait for the loads in flight.
  static_assert(NSA >= 2 && NSA <= 6 && NSB >= 2 && NSB <= 6 &&
                DA - DB <= 1 && DB - DA <= 1, "2 to 6 stages, lookaheads within one");
  __shared__ __attribute__((aligned(16))) bf16 A0[SA];
  __shared__ __attribute__((aligned(16))) bf16 A1[SA];
  __shared__ __attribute__((aligned(16))) bf16 A2[NSA > 2 ? SA : 8];
  __shared__ __attribute__((aligned(16))) bf16 A3[NSA > 3 ? SA : 8];
  __shared__ __attribute__((aligned(16))) bf16 A4[NSA > 4 ? SA : 8];
  __shared__ __attribute__((aligned(16))) bf16 A5[NSA > 5 ? SA : 8];
  __shared__ __attribute__((aligned(16))) bf16 B0[SB];
  __shared__ __attribute__((aligned(16))) bf16 B1[SB];
  __shared__ __attribute__((aligned(16))) bf16 B2[NSB > 2 ? SB : 8];
  __shared__ __attribute__((aligned(16))) bf16 B3[NSB > 3 ? SB : 8];
  __shared__ __attribute__((aligned(16))) bf16 B4[NSB > 4 ? SB : 8];
  __shared__ __attribute__((aligned(16))) bf16 B5[NSB > 5 ? SB : 8];
  // stage s's arrays (s is a constant after unrolling, so each access names
  // one distinct object; stages past NSA or NSB are never named, so their
  // placeholder arrays take no LDS)
  auto As = [&](int st) -> bf16* {
    if constexpr (NSA > 5) if (st == 5) return A5;
    if constexpr (NSA > 4) if (st == 4) return A4;
    if constexpr (NSA > 3) if (st == 3) return A3;
    if constexpr (NSA > 2) if (st == 2) return A2;
    return st == 1 ? A1 : A0;
  };
  auto Bs = [&](int st) -> bf16* {
    if constexpr (NSB > 5) if (st == 5) return B5;
    if constexpr (NSB > 4) if (st == 4) return B4;
    if constexpr (NSB > 3) if (st == 3) return B3;
    if constexpr (NSB > 2) if (st == 2) return B2;
    return st == 1 ? B1 : B0;
  };
  // The tile's parameters and the tile scan's scratch live in the last A
  // stage: its first load is issued by slice 0, after the prologue's
  // barrier, and every wave has read them into scalar registers before it
  // (the split path's counter slot is used after the loads have landed).
  static_assert(SA * 2 >= (TL_INFO + TL_THREADS / 64) * 4, "tile info fits");
  int* const s_info = reinterpret_cast<int*>(As(NSA - 1));

  const int G = a.E + a.n_shared;
  const int Kd = MODE == DOWN ? a.d_ff : a.d;
  if (!find_tile_split<TL_THREADS>(a, G, BM, NB, Kd / BK, s_info)) return;
  // tile parameters are workgroup-uniform: keep them in scalar registers
  const int g = __builtin_amdgcn_readfirstlane(s_info[0]);
  const int r0 = __builtin_amdgcn_readfirstlane(s_info[1]);
  const int nb = __builtin_amdgcn_readfirstlane(s_info[2]);
  const int kb = __builtin_amdgcn_readfirstlane(s_info[3]);
  const int ke = __builtin_amdgcn_readfirstlane(s_info[4]);
  const int item = __builtin_amdgcn_readfirstlane(s_info[5]);
  const int sp_ctr = __builtin_amdgcn_readfirstlane(s_info[6]);
  const int sp_n = __builtin_amdgcn_readfirstlane(s_info[7]);
  Group gr = group_of(g, a.offsets, a.E, a.T, a.k);
  gr.out0 = __builtin_amdgcn_readfirstlane(gr.out0);
  gr.rows = __builtin_amdgcn_readfirstlane(gr.rows);
  const int N = MODE == DOWN ? a.d : a.d_ff;
  const int K = MODE == DOWN ? a.d_ff : a.d;
  const int ncols = MODE == UP_SWIGLU ? TL_BN / 2 : TL_BN;   // outputs per tile
  const int nbase = nb * ncols;
  const void *w0v, *w1v, *biasv;
  group_weights<MODE>(a, g, gr.shared, N, K, w0v, w1v, biasv);

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WGN, wn = wave % WGN;
  const int l31 = lane & 31, q = lane >> 5;

  // Loads: wave w fills A rows [w*IA*RPI, (w+1)*IA*RPI) and B rows likewise,
  // RPI = 8 rows per instruction; lane l covers row RPI*i + l/8, LDS position
  // l%8, i.e. global chunk (l%8) ^ key(row).  An instruction's first row is a
  // multiple of 8, so key(row) = (l/8)/2 ^ (4 if the instruction index is
  // odd): one per-lane chunk offset for even and one for odd instructions.
  // Each load instruction has a wave-uniform base (scalar registers) and a
  // 32-bit per-lane byte offset.  A: the byte offset of the lane's row from
  // x (up GEMMs, token rows gathered through perm, T*d*2 < 2^32 bytes) or
  // from the group's first H row (down GEMM), rows past the group's end
  // repeating its last row: one register per load, kept across the K loop
  // (reading them back from an LDS table instead made each issue wait for
  // the operand reads in flight; up GEMM 3420 -> 3570 us).  B: the uniform
  // part is the instruction's first weight row (its 8 rows lie in one
  // matrix and, N being a multiple of 64, all inside it or all past it, so
  // a past group is clamped whole to the last 8 rows), the per-lane part
  // row l/8 of the 8 and the chunk: two registers for all B loads.
  static_assert(BK == 64 && Geo::RPI == 8 && IA % 2 == 0 && IB % 2 == 0,
                "load layout");
  const int lr = lane >> 3;
  const int lp = lane & 7;
  const uint32_t ch_even = (uint32_t)((lp ^ (lr >> 1)) << 4);
  const uint32_t ch_odd = (uint32_t)((lp ^ ((lr >> 1) | 4)) << 4);
  const char* abase = MODE == DOWN
      ? (const char*)a.h + (size_t)gr.out0 * K * 2
      : (const char*)a.x;
  uint32_t ao[IA];   // per-lane A offsets, live across the K loop
#pragma unroll
  for (int i = 0; i < IA; ++i) {
    const int ai = min(r0 + (wave * IA + i) * Geo::RPI + lr, gr.rows - 1);
    const int arow = MODE == DOWN ? ai
                                  : (gr.shared ? ai : a.perm[gr.out0 + ai] / a.k);
    ao[i] = (uint32_t)arow * ((uint32_t)K * 2u) + ((i & 1) ? ch_odd : ch_even);
  }
  // B rows: SwiGLU block b = r >> 6 holds gate cols [32b, 32b+32) in rows
  // [64b, 64b+32) and the matching up cols in [64b+32, 64b+64), so wave
  // column wn's two N-tiles are a gate tile and its up tile.
  const size_t bskip = TW ? (size_t)(nbase >> 4) * (K / 32) * 512
                          : (size_t)nbase * K;
  const char* bm0 = (const char*)((const bf16*)w0v + bskip);
  const char* bm1 = MODE == UP_SWIGLU
      ? (const char*)((const bf16*)w1v + bskip) : bm0;
  const uint32_t b_lane = TW ? (uint32_t)(lane * 16)
                             : (uint32_t)lr * ((uint32_t)K * 2u);
  // uniform part of B load i: its matrix and byte offset from that matrix's
  // tile base
  auto b_part = [&](int i, bool& up) -> uint32_t {
    if constexpr (TW) {
      // instruction ii = wave * IB + i loads tile (row block ii / 2 of the
      // slice's B rows, column block ii % 2)
      const int ii = wave * IB + i;
      const int t0 = 16 * (ii >> 1);
      int wr0;
      if (MODE == UP_SWIGLU) {
        up = ((t0 >> 5) & 1) != 0;
        wr0 = nbase + 32 * (t0 >> 6) + (t0 & 31);
      } else {
        up = false;
        wr0 = nbase + t0;
      }
      const int rbg = min(wr0 >> 4, N / 16 - 1);
      return ((uint32_t)(rbg - (nbase >> 4)) * (uint32_t)(K / 32) +
              (uint32_t)(ii & 1)) * 1024u;
    } else {
      const int row0 = (wave * IB + i) * Geo::RPI;
      int wrow0;
      if (MODE == UP_SWIGLU) {
        up = ((row0 >> 5) & 1) != 0;
        wrow0 = nbase + 32 * (row0 >> 6) + (row0 & 31);
      } else {
        up = false;
        wrow0 = nbase + row0;
      }
      wrow0 = min(wrow0, N - 8);
      return (uint32_t)(wrow0 - nbase) * ((uint32_t)K * 2u);
    }
  };
  // LDS byte addresses of the stages (link-time constants) and of this
  // wave's first load in a stage
  auto lds_of = [](const void* p) -> uint32_t {
    return (uint32_t)(uintptr_t)(lds_void_t*)p;
  };
  const uint32_t a_lds[6] = {lds_of(A0), lds_of(A1), lds_of(A2),
                             lds_of(A3), lds_of(A4), lds_of(A5)};
  const uint32_t b_lds[6] = {lds_of(B0), lds_of(B1), lds_of(B2),
                             lds_of(B3), lds_of(B4), lds_of(B5)};
  constexpr int ASTR = Geo::RPI * BK * 2;            // LDS bytes per A load
  constexpr int BSTR = TW ? 1024 : Geo::RPI * BK * 2;
  const uint32_t a_w = (uint32_t)(wave * IA * ASTR);
  const uint32_t b_w = (uint32_t)(wave * IB * BSTR);
  auto issue_a = [&](int kt, int st) {
    const char* ak = abase + (size_t)(kb + kt) * BK * 2;
    dma16s_seq<ASTR>([&](int) { return ak; }, ao, a_lds[st] + a_w,
                     std::make_integer_sequence<int, IA>());
  };
  auto issue_b = [&](int kt, int st) {
    const size_t kw = TW ? (size_t)(kb + kt) * 2048 : (size_t)(kb + kt) * BK * 2;
    uint32_t bo[IB];
    const char* bs[IB];
#pragma unroll
    for (int i = 0; i < IB; ++i) {
      bool up;
      const uint32_t u = b_part(i, up);
      bs[i] = uniform_ptr((up ? bm1 : bm0) + kw + u);
      bo[i] = TW ? b_lane : b_lane + ((i & 1) ? ch_odd : ch_even);
    }
    dma16s_seq<BSTR>([&](int i) { return bs[i]; }, bo, b_lds[st] + b_w,
                     std::make_integer_sequence<int, IB>());
  };
  // The loads slice k issues: A slice k + DA and B slice k + DB, clamped to
  // the piece's last slice, into stages (u + DA) % NSA and (u + DB) % NSB,
  // u = k mod lcm(NSA, NSB) a constant after unrolling.  The prologue runs
  // this for k = u = -DMAX .. -1, issuing only slices >= 0.
  const int nk = ke - kb;   // K slices of this piece
  auto issue = [&](int u, int k) {
    const int sa = u + DA, sb = u + DB;
    if (DA > DB) {
      if (sb >= 0) issue_b(min(k + DB, nk - 1), sb % NSB);
      if (sa >= 0) issue_a(min(k + DA, nk - 1), sa % NSA);
    } else {
      if (sa >= 0) issue_a(min(k + DA, nk - 1), sa % NSA);
      if (sb >= 0) issue_b(min(k + DB, nk - 1), sb % NSB);
    }
  };

  f32x16 acc[MT][NT];
#pragma unroll
  for (int i = 0; i < MT; ++i)
#pragma unroll
    for (int j = 0; j < NT; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

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

  // Prologue: A slices 0..DA-1 and B slices 0..DB-1 in flight (clamped to
  // the last slice when the piece is shorter), in the order the main loop
  // keeps, then wait for slice 0.
#pragma unroll
  for (int j = -DMAX; j < 0; ++j) issue(j, j);
  slice_barrier<WAITN>();
  // Main loop, lcm(NSA, NSB) slices per trip with constant stage indices.
  // Slice k reads A stage k % NSA and B stage k % NSB; before it, A slice
  // k + DA and B slice k + DB are issued into the stages slice k - 1 read
  // (one barrier ago).  After slice k the wave waits until slice k + 1 has
  // landed: all later loads may stay in flight.  The slice body has no
  // branch: near the end the last slice is issued again into the stage just
  // freed (redundant loads, never read), so every slice issues PER loads and
  // the wait count is constant; the loads, the first LDS reads and the MFMAs
  // of a slice schedule as one block.
  constexpr int U = pn_lcm(NSA, NSB);
  for (int kt = 0; kt < nk; kt += U) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kt + u;
      if (k < nk) {
        issue(u, k);
        compute_deferred(As(u % NSA), Bs(u % NSB));
        slice_barrier<WAITN>();
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
    const int ctr = sp_ctr, sp = sp_n;
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
    // order, this piece's own partial read back like the others, one 32x32
    // accumulator tile at a time with the loads of four pieces issued
    // together (indices past the last piece re-read it and are not added).
    static_assert(TL_SPLIT_MAX % 4 == 0, "pieces in batches of four");
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
#pragma unroll
        for (int q0 = 0; q0 < TL_SPLIT_MAX; q0 += 4) {
          if (q0 < sp) {
            f32x4 pv[4][4];
#pragma unroll
            for (int u = 0; u < 4; ++u)
#pragma unroll
              for (int v4 = 0; v4 < 4; ++v4)
                pv[u][v4] = p0[(size_t)min(q0 + u, sp - 1) * (SPLIT_TILE_FLOATS / 4) +
                               ((i * NT + j) * 4 + v4) * TL_THREADS + tid];
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (q0 + u < sp)
#pragma unroll
                for (int v4 = 0; v4 < 4; ++v4) sum[v4] += pv[u][v4];
          }
        }
#pragma unroll
        for (int v4 = 0; v4 < 4; ++v4)
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[i][j][4 * v4 + e] = sum[v4][e];
      }
    if (tid == 0) a.split_cnt[ctr] = 0;   // ready for the next launch
  }

  // ---- epilogue: activation, stage the bf16 tile in LDS, store rows ----
  // The output tile (BM x NCOLS bf16, row-major) is staged in the A stages
  // and, past their end, in the B stages, RPS rows per stage.  A wave's
  // 32-row MFMA tile lies in one stage, and so does each pass of the store
  // loop; the stage is picked with scalar code (a wave-uniform index), so
  // every LDS access is one base register plus a constant offset.
  constexpr int NCOLS = MODE == UP_SWIGLU ? TL_BN / 2 : TL_BN;
  constexpr int RPS = SA / NCOLS;           // staged rows per stage
  constexpr int CPR = NCOLS / 8;            // 16-byte chunks per row
  constexpr int PASSES = BM * CPR / TL_THREADS;
  constexpr int PPS = SA / 8 / TL_THREADS;  // store passes per stage
  static_assert(SA == SB && RPS % 32 == 0 && (SA / 8) % TL_THREADS == 0 &&
                BM * NCOLS <= NSA * SA + NSB * SB, "output tile staging");
  typedef __attribute__((address_space(3))) bf16 lds_bf16;
  typedef __attribute__((address_space(3))) u32x4 lds_u32x4;
  auto stage_lds = [&](int st) -> uint32_t {   // st: wave-uniform
    uint32_t r = a_lds[0];
#pragma unroll
    for (int s2 = 1; s2 < NSA; ++s2)
      if (st == s2) r = a_lds[s2];
#pragma unroll
    for (int s2 = 0; s2 < NSB; ++s2)
      if (st == NSA + s2) r = b_lds[s2];
    return r;
  };
  __syncthreads();
  // this lane's bias of each of its N-tiles' columns (GELU up and down)
  float bias_j[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) {
    const int n = min(nbase + wn * WN + 32 * j + l31, N - 1);
    bias_j[j] = (MODE != UP_SWIGLU && biasv) ? (float)((const bf16*)biasv)[n] : 0.f;
  }
  // 32x32 accumulator layout: lane holds column lane&31; item v is row
  // (v&3) + 4*(lane>>5) + 8*(v>>2).  One accumulator tile (SwiGLU: a gate
  // tile and its up tile) at a time, each copied out whole, so that every
  // index into the accumulator array is a constant.
  auto out_tile = [&](int i, int c, const f32x16& t0, const f32x16& t1,
                      float bias) {
    const int row0 = wm * WM + 32 * i;   // wave-uniform
    const int st = row0 / RPS;
    lds_bf16* p = (lds_bf16*)(uintptr_t)(
        stage_lds(st) + 2u * (uint32_t)((row0 - st * RPS + 4 * q) * NCOLS + c));
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      float h;
      if (MODE == UP_SWIGLU) {
        h = silu(t0[v]) * t1[v];
      } else {
        h = t0[v] + bias;
        if (MODE == UP_GELU) h = gelu_erf(h);
      }
      p[((v & 3) + 8 * (v >> 2)) * NCOLS] = (bf16)h;
    }
  };
#pragma unroll
  for (int i = 0; i < MT; ++i) {
    if (MODE == UP_SWIGLU) {
      // N-tiles (2p, 2p+1) are a gate tile and its up tile
#pragma unroll
      for (int p = 0; p < NT / 2; ++p)
        out_tile(i, 32 * (wn * (NT / 2) + p) + l31, acc[i][2 * p],
                 acc[i][2 * p + 1], 0.f);
    } else {
#pragma unroll
      for (int j = 0; j < NT; ++j)
        out_tile(i, wn * WN + 32 * j + l31, acc[i][j], acc[i][j], bias_j[j]);
    }
  }
  __syncthreads();
  bf16* outp = (bf16*)(MODE == DOWN ? a.y : a.h);
#pragma unroll
  for (int ps = 0; ps < PASSES; ++ps) {
    const int idx = ps * TL_THREADS + tid;   // 16-byte chunk of the tile
    const int row = idx / CPR, ch = idx - row * CPR;
    const int i = r0 + row;
    const int n = nbase + ch * 8;
    if (i < gr.rows && n < N) {
      const u32x4 v = *(const lds_u32x4*)(uintptr_t)(
          stage_lds(ps / PPS) + 16u * (uint32_t)(idx - (ps / PPS) * (SA / 8)));
      // non-temporal: the tile is not read again by this launch, and its
      // lines would otherwise push the shared A and B slices out of L2
      __builtin_nontemporal_store(
          v, reinterpret_cast<u32x4*>(outp + (size_t)(gr.out0 + i) * N + n));
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
// order); the panel's token rows (A) go once per workgroup from global
// memory straight into a ring of three XOR-swizzled LDS slices (direct-to-
// LDS loads, two steps ahead) and are read by all eight waves.  (Through
// registers and LDS stores, as first built, the A path cost about an eighth
// of the DeepSeek-V3 up GEMM: 3371 -> 3177 us, Switch down 325 -> 304 us.)
// Row tiles past the panel's rows issue no MFMAs and no loads, so a ragged
// expert costs its own rows, not a full tile.  The weight loads are
// ordinary compiler-visible loads; the A loads are not, and each step ends
// with a wait counted for the loads issued after the next step's A.
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


// BM rows per panel; L = 1: step s issues A step s+2 (direct-to-LDS, a
// ring of three slices) and weight step s+2 (L+1 register slots), A first.
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
  __shared__ __attribute__((aligned(16))) bf16 S2[SL];
  __shared__ u32x4 xs[TW ? 1 : W][NMAT * CG * 2][64];   // reshuffle per wave
  __shared__ int s_info[3];

  const int G = a.E + a.n_shared;
  if (!find_panel_tile<W * 64>(a, G, BM, NB, MODE != DOWN, s_info)) return;
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

  // A slices go from global memory straight into LDS (direct-to-LDS
  // loads, 16 bytes per lane, one instruction = 8 rows x 128 bytes): load i
  // of wave w covers rows 64i + 8w + lane/8 of the panel, LDS position
  // lane % 8 of its row, i.e. global chunk (lane % 8) ^ key(row); the key of
  // those rows depends only on w and lane/8.  Each lane keeps one 32-bit
  // byte offset per load from a wave-uniform base: the token row from x (up
  // GEMMs, through perm; T*d*2 < 2^32 bytes) or the row from the group's
  // first H row (down GEMM).  Rows past the panel re-read its last row.
  const char* abase = MODE == DOWN ? (const char*)a.h + (size_t)gr.out0 * K * 2
                                   : (const char*)a.x;
  uint32_t ao[AI];
#pragma unroll
  for (int i = 0; i < AI; ++i) {
    const int row = i * 64 + wave * 8 + (lane >> 3);
    const int ri = r0 + min(row, nvalid - 1);
    const int arow = MODE == DOWN ? ri
                                  : (gr.shared ? ri : a.perm[gr.out0 + ri] / a.k);
    ao[i] = (uint32_t)arow * ((uint32_t)K * 2u) +
            (uint32_t)(((lane & 7) ^ pn_key(row)) << 4);
  }
  // LDS byte address of this wave's first A load in each slice (uniform)
  const uint32_t a_w = (uint32_t)__builtin_amdgcn_readfirstlane(wave * 8 * PN_KSTEP * 2);
  const uint32_t a_lds[3] = {(uint32_t)(uintptr_t)(lds_void_t*)S0 + a_w,
                             (uint32_t)(uintptr_t)(lds_void_t*)S1 + a_w,
                             (uint32_t)(uintptr_t)(lds_void_t*)S2 + a_w};
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
  // kq + 4h is register col / 8, row col % 8, chunk kq + 4h.  In the slot,
  // chunk ch of row r of register b sits at position 8r + (ch ^ (r/2) ^ 4b),
  // so that the 16 lanes of an MFMA-order read (16 rows, one chunk) and of a
  // store (two rows, eight chunks) fall on distinct banks of a 256-byte
  // window (unswizzled, the reads met 8-way conflicts: 1.9e8 conflict
  // cycles per DeepSeek-V3 up GEMM).  Plain loads: the non-temporal hint
  // was mixed here (Switch faster, DeepSeek slower).
  uint32_t boff[CG][2];   // element offsets (same rows in every matrix)
#pragma unroll
  for (int c = 0; c < CG; ++c)
#pragma unroll
    for (int h = 0; h < 2; ++h)
      boff[c][h] = (uint32_t)min(nbase + 16 * (wave * CG + c) + 8 * h + (lane >> 3), N - 1) *
                       (uint32_t)K + (uint32_t)((lane & 7) * 8);
  const int xsrc = col >> 3;
  // slot positions: this lane's store of register b, and its MFMA-order
  // read of half h
  const int xst[2] = {(lane & 56) | ((lane & 7) ^ (lane >> 4)),
                      (lane & 56) | ((lane & 7) ^ (lane >> 4) ^ 4)};
  const int xrd[2] = {8 * (col & 7) + (kq ^ ((col & 7) >> 1) ^ (xsrc << 2)),
                      8 * (col & 7) + ((kq + 4) ^ ((col & 7) >> 1) ^ (xsrc << 2))};
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
  // A step s into slice st: the first NA of this lane's loads (rows below
  // NA * 64); loads past the last step re-read the last step (never used)
  auto dmaA = [&](auto nac, int st, int s) {
    constexpr int NA = decltype(nac)::value;
    const char* ak = uniform_ptr(abase + (size_t)min(s, nk - 1) * PN_KSTEP * 2);
    dma16s_seq<64 * PN_KSTEP * 2>([&](int) { return ak; }, ao, a_lds[st],
                                  std::make_integer_sequence<int, NA>());
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
        for (int h = 0; h < 2; ++h) xs[wave][(m * CG + c) * 2 + h][xst[h]] = b.b[m][c][h];
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
                            : xs[TW ? 0 : wave][(m * CG + c) * 2 + xsrc][xrd[h]];
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
    // Step s (u = s mod U): reads A slice s % 3 and weight slot s % 2.
    // It issues A step s+2 into slice (s+2) % 3, whose readers finished at
    // the last barrier, then refills the weight slot with step s+2 (after
    // the slot went to the wave's reshuffle slot; with tiled weights, after
    // the MFMAs that read the slot itself), and runs the MFMAs (row-major
    // weights read back from the reshuffle slot in MFMA order).  Every step
    // issues NA A loads, then BL weight loads, so at its end the loads
    // issued after A step s+1 number BL + NA + BL: waiting for at most that
    // many leaves the later steps in flight.  (The compiler's own wait for
    // a weight slot counts only the weight loads; it also waits for the A
    // step issued before the slot's successor, which that step needs one
    // step later anyway.)
    static_assert(L == 1, "A ring of three slices, weights two steps ahead");
    constexpr int BL = NMAT * CG * 2;   // weight loads per step
    constexpr int WAITN = 2 * BL + NA;
    auto S = [&](int i) -> bf16* { return i == 0 ? S0 : (i == 1 ? S1 : S2); };
    auto step = [&](int s, int u) {
      bf16* cur = S(u % 3);
      if constexpr (TW) {
        dmaA(na, (u + 2) % 3, s + 2);
        compute(cur, ring[u % NSLOT]);
        loadB(ring[u % NSLOT], s + 2);
      } else {
        stageB(ring[u % NSLOT]);
        dmaA(na, (u + 2) % 3, s + 2);
        loadB(ring[u % NSLOT], s + 2);
        compute(cur, ring[u % NSLOT]);
      }
      slice_barrier<WAITN>();
    };
    // prologue in the loop's issue order: A step 0, weight step 0, A step
    // 1, weight step 1; then wait for A step 0
    dmaA(na, 0, 0);
    loadB(ring[0], 0);
    dmaA(na, 1, 1);
    loadB(ring[1], 1);
    slice_barrier<WAITN>();
    // whole trips of U steps (constant slice and slot indices), then the
    // remaining steps
    constexpr int U = pn_lcm(3, NSLOT);
    const int ntrip = nk / U;
    for (int tr = 0; tr < ntrip; ++tr) {
#pragma unroll
      for (int u = 0; u < U; ++u) step(tr * U + u, u);
    }
#pragma unroll
    for (int u = 0; u < U - 1; ++u)
      if (ntrip * U + u < nk) step(ntrip * U + u, u);
  };
  // three instances: panels filling at most half or three quarters of the
  // tiles run a shorter loop
  static_assert(MT % 4 == 0, "half and three-quarter panels");
  if (ntile > MT * 3 / 4) kloop(IntC<MT>{});
  else if (ntile > MT / 2) kloop(IntC<MT * 3 / 4>{});
  else kloop(IntC<MT / 2>{});
  // the redundant tail A loads land in LDS before the workgroup can end
  // (the next workgroup on this CU may take the same LDS)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // epilogue: lane holds column n of group c and rows 16t + 4kq + r.  The
  // stores take a wave-uniform base (the panel's first output row, in scalar
  // registers) and a 32-bit lane offset (rows < 256, so the offset stays
  // below 256 * N elements), and a row tile that lies wholly inside the
  // panel stores without per-lane row checks.  (With a 64-bit address
  // multiply and a row check per element the stores took 5.3 us per panel
  // of the DeepSeek-V3 down GEMM, against a 58 us K loop.)
  typedef __attribute__((address_space(1))) bf16 gbf16;
  typedef __attribute__((address_space(1))) char gchar8;
  gchar8* obase = (gchar8*)uniform_ptr(
      (const char*)((bf16*)(MODE == DOWN ? a.y : a.h) + (size_t)(gr.out0 + r0) * N));
  const uint32_t row_bytes = (uint32_t)N * 2u;
  auto store = [&](uint32_t byte, bf16 v) { *(gbf16*)(obase + byte) = v; };
#pragma unroll
  for (int c = 0; c < CG; ++c) {
    const int n = nbase + 16 * (wave * CG + c) + col;
    if (n >= N) continue;
    float bias = 0.f;
    if (MODE != UP_SWIGLU && biasv) bias = (float)((const bf16*)biasv)[n];
    const uint32_t o0 = (uint32_t)(4 * kq) * row_bytes + (uint32_t)n * 2u;
    auto val = [&](int t, int r) -> bf16 {
      float v;
      if (MODE == UP_SWIGLU)
        v = silu(acc[0][c][t][r]) * acc[NMAT - 1][c][t][r];
      else if (MODE == UP_GELU) v = gelu_erf(acc[0][c][t][r] + bias);
      else v = acc[0][c][t][r] + bias;
      return (bf16)v;
    };
#pragma unroll
    for (int t = 0; t < MT; ++t) {
      if (t < ntile) {
        // the activation once, outside the two store paths (inlined into
        // both it doubled the GELU kernel's epilogue code and slowed it)
        bf16 v4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v4[r] = val(t, r);
        if (16 * t + 16 <= nvalid) {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            store(o0 + (uint32_t)(16 * t + r) * row_bytes, v4[r]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r)
            if (16 * t + 4 * kq + r < nvalid)
              store(o0 + (uint32_t)(16 * t + r) * row_bytes, v4[r]);
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
    ffn_tiled_kernel<MODE, 256, 64, tl_nsa(MODE), tl_nsb(MODE), TL_WAVES, TW>
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

hipError_t launch_expert_up(const FfnArgs& a, hipStream_t s) {
  if (a.T == 0) return hipSuccess;
  if (a.wquant == 1) return launch_q4_up(a, s);   // 4-bit codes
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
  if (a.wquant == 1) return launch_q4_down(a, s);   // 4-bit codes
  const Plan p = plan_of(a);
  if (a.wquant == 2) return launch_mode<DOWN, true>(a, s, p.sched, p.rt, p.max_tiles);
  return launch_mode<DOWN, false>(a, s, p.sched, p.rt, p.max_tiles);
}

}  // namespace moe
