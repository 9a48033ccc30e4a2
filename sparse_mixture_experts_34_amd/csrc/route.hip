// Route: router linear, softmax, top-k, renormalised gates.
//
// The router is one linear layer from the hidden state to E scores,
// followed by a softmax over all E experts and a top-k choice whose chosen
// probabilities are renormalised to sum to one (randomcommits.com
// "Mixture-of-Experts routing", How a sparse MoE layer works;
// letsbuildsolutions.com "How Mixture of Experts Works", Gating Mechanism;
// getnybble.com "Mixture of Experts (MoE)", The router).  The router runs
// in float32 (letsbuildsolutions.com, Dense vs Sparse).
//
// Kernel 1 (router_logits): logits = x . Wr^T on bf16 MFMA.  Wr is float32;
// each weight is split exactly into hi + mid + lo bf16 parts, so with bf16
// x every product is exact in float32 and the three MFMAs accumulate a
// float32-accurate dot product at matrix-core speed.  A float32 x is split
// the same way (six part products).  64 tokens x 64 experts per
// workgroup, the K dimension split over its four waves and, for small T,
// across workgroups (the partial sums are added, in a fixed order, by
// kernel 2).  Past 2048 bf16 tokens a wide variant takes 256 tokens per
// workgroup and shares each split weight slice through LDS.
//
// Kernel 2 (route_select): one wave per token.  Sum the K-split partials,
// add the router bias, softmax (max-subtracted), choose k experts by k
// rounds of wave argmax on (key, index) with equal keys going to the lower
// index, gates = exp-values of the chosen experts over their sum.  Each
// workgroup also writes the sum over its tokens of the probabilities
// (fixed order) for the aux loss.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int RL_THREADS = 256;
constexpr int RL_EXP_TILE = 64;   // experts per workgroup (4 MFMA N-tiles)
constexpr int RL_KSTEP = 64;      // K per step (two 16x16x32 MFMAs)

// Load 16 consecutive x values as float.
template <typename XT>
__device__ __forceinline__ void load16(const XT* p, float* out);

template <>
__device__ __forceinline__ void load16<bf16>(const bf16* p, float* out) {
  V16 a, b;
  a.u = ldg16(p);
  b.u = ldg16(p + 8);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    out[i] = (float)a.h[i];
    out[8 + i] = (float)b.h[i];
  }
}
template <>
__device__ __forceinline__ void load16<float>(const float* p, float* out) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    V16 v;
    v.u = ldg16(p + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * i + j] = v.f[j];
  }
}

// XPARTS: 1 for bf16 x (exact), 3 for float32 x.
// TT: token tiles of 16 per wave.
template <typename XT, int XPARTS, int TT>
__global__ __launch_bounds__(RL_THREADS) void router_logits_kernel(
    const XT* __restrict__ x, const float* __restrict__ wr,
    float* __restrict__ part, int T, int d, int E, int ksplit) {
  __shared__ float red[3][TT * 16 * RL_EXP_TILE];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 15;   // token row (A) / expert row (B) in a tile
  const int kq = lane >> 4;    // which 16-wide k slice of the 64-wide step
  const int t0 = blockIdx.x * (TT * 16);
  const int e0 = blockIdx.y * RL_EXP_TILE;
  const int ks = blockIdx.z;
  const int klen = d / ksplit;             // multiple of 64 (host checks)
  const int kbeg = ks * klen;
  const int nsteps = klen / RL_KSTEP;
  const int ntile = min(4, (E - e0 + 15) >> 4);
  const int ttok = min(TT, (T - t0 + 15) >> 4);

  const XT* xr[TT];
#pragma unroll
  for (int i = 0; i < TT; ++i) {
    int t = min(t0 + 16 * i + row, T - 1);
    xr[i] = x + (size_t)t * d + kbeg + kq * 16;
  }
  const float* wrow[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    int e = min(e0 + 16 * j + row, E - 1);
    wrow[j] = wr + (size_t)e * d + kbeg + kq * 16;
  }

  f32x4 acc[TT][4];
#pragma unroll
  for (int i = 0; i < TT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int s = wave; s < nsteps; s += 4) {
    const int k0 = s * RL_KSTEP;
    // A operands: x rows, split into XPARTS bf16 parts, two 8-wide halves
    bf16x8 a[TT][XPARTS][2];
#pragma unroll
    for (int i = 0; i < TT; ++i) {
      float xv[16];
      load16<XT>(xr[i] + k0, xv);
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          bf16 pr[3];
          split3(xv[8 * h + q], pr[0], pr[1], pr[2]);
#pragma unroll
          for (int p = 0; p < XPARTS; ++p) a[i][p][h][q] = pr[p];
        }
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < ntile) {
        float wv[16];
        load16<float>(wrow[j] + k0, wv);
        bf16x8 b[3][2];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            bf16 hi, mid, lo;
            split3(wv[8 * h + q], hi, mid, lo);
            b[0][h][q] = hi;
            b[1][h][q] = mid;
            b[2][h][q] = lo;
          }
#pragma unroll
        for (int i = 0; i < TT; ++i) {
          if (i < ttok) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              f32x4 c = acc[i][j];
              // parts whose ranks sum to <= 2 (hi=0, mid=1, lo=2)
#pragma unroll
              for (int pa = 0; pa < XPARTS; ++pa)
#pragma unroll
                for (int pb = 0; pb < 3; ++pb)
                  if (pa + pb <= 2)
                    c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                        a[i][pa][h], b[pb][h], c, 0, 0, 0);
              acc[i][j] = c;
            }
          }
        }
      }
    }
  }

  // Reduce the four waves' partial sums in the fixed order 0,1,2,3.
  // Accumulator layout: lane holds column (expert) lane&15 and rows
  // (tokens) 4*(lane>>4) + r.
  if (wave > 0) {
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int m = 16 * i + 4 * kq + r, n = 16 * j + row;
          red[wave - 1][m * RL_EXP_TILE + n] = acc[i][j][r];
        }
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int i = 0; i < TT; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          int m = 16 * i + 4 * kq + r, n = 16 * j + row;
          float v = acc[i][j][r];
          v += red[0][m * RL_EXP_TILE + n];
          v += red[1][m * RL_EXP_TILE + n];
          v += red[2][m * RL_EXP_TILE + n];
          int t = t0 + m, e = e0 + n;
          if (t < T && e < E) part[((size_t)ks * T + t) * E + e] = v;
        }
  }
}

// Large batches (bf16 x): 256 tokens x 64 experts per workgroup, the four
// waves on 64 tokens each.  Each K step's 64 x 64 router-weight slice is
// loaded once per workgroup (wave w loads expert tile w), split into its
// three bf16 parts and kept in LDS in MFMA operand order for all four waves,
// so the float32 weights cross L2 once per 256 tokens instead of once per 64.
// Double-buffered LDS, one barrier per step; each wave loads the next step's
// x and weights while it computes.  A wave adds its steps in order and
// writes its own tokens' partial logits (no cross-wave reduction).
constexpr int RLW_TT = 4;                            // 16-token tiles per wave
constexpr int RLW_TOK = ROUTE_WAVES * RLW_TT * 16;   // tokens per workgroup
constexpr int RLW_MAX_KSPLIT = 8;                    // K slices at most

__global__ __launch_bounds__(RL_THREADS) void router_logits_wide_kernel(
    const bf16* __restrict__ x, const float* __restrict__ wr,
    float* __restrict__ part, int T, int d, int E, int ksplit) {
  // [stage][expert tile][part * 2 + half][lane]
  __shared__ u32x4 bs[2][4][6][64];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int row = lane & 15;
  const int kq = lane >> 4;
  const int t0 = blockIdx.x * RLW_TOK + wave * (RLW_TT * 16);
  const int e0 = blockIdx.y * RL_EXP_TILE;
  const int ks = blockIdx.z;
  const int klen = d / ksplit;   // multiple of 64 (host checks)
  const int kbeg = ks * klen;
  const int nsteps = klen / RL_KSTEP;
  const int ntile = min(4, (E - e0 + 15) >> 4);
  const int ttok = max(0, min(RLW_TT, (T - t0 + 15) >> 4));   // this wave

  const bf16* xr[RLW_TT];
#pragma unroll
  for (int i = 0; i < RLW_TT; ++i) {
    const int t = min(t0 + 16 * i + row, T - 1);
    xr[i] = x + (size_t)t * d + kbeg + kq * 16;
  }
  // this wave's expert tile of the weight slice (rows past E re-read the
  // last expert; their parts are never used)
  const bool wload = wave < ntile;
  const float* wrow =
      wr + (size_t)min(e0 + 16 * wave + row, E - 1) * d + kbeg + kq * 16;

  f32x4 acc[RLW_TT][4];
#pragma unroll
  for (int i = 0; i < RLW_TT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // raw operands of the next step: x as the two bf16x8 halves, weights as
  // 16 floats
  u32x4 xn[RLW_TT][2], wn[4];
  auto fetch = [&](int s) {
    const int k0 = s * RL_KSTEP;
#pragma unroll
    for (int i = 0; i < RLW_TT; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) xn[i][h] = ldg16(xr[i] + k0 + 8 * h);
    if (wload) {
#pragma unroll
      for (int q = 0; q < 4; ++q) wn[q] = ldg16(wrow + k0 + 4 * q);
    }
  };
  if (nsteps > 0) fetch(0);
  for (int s = 0; s < nsteps; ++s) {
    const int st = s & 1;
    V16 xc[RLW_TT][2];
#pragma unroll
    for (int i = 0; i < RLW_TT; ++i)
#pragma unroll
      for (int h = 0; h < 2; ++h) xc[i][h].u = xn[i][h];
    if (wload) {
      // split the 16 weights into hi / mid / lo, two 8-wide halves each
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        V16 hi, mid, lo;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
          V16 w;
          w.u = wn[(8 * h + q) >> 2];
          bf16 a, b, c;
          split3(w.f[q & 3], a, b, c);
          hi.h[q] = a;
          mid.h[q] = b;
          lo.h[q] = c;
        }
        bs[st][wave][0 + h][lane] = hi.u;
        bs[st][wave][2 + h][lane] = mid.u;
        bs[st][wave][4 + h][lane] = lo.u;
      }
    }
    if (s + 1 < nsteps) fetch(s + 1);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (j < ntile) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          V16 b[3];
#pragma unroll
          for (int pb = 0; pb < 3; ++pb) b[pb].u = bs[st][j][2 * pb + h][lane];
#pragma unroll
          for (int i = 0; i < RLW_TT; ++i) {
            if (i < ttok) {
              f32x4 c = acc[i][j];
#pragma unroll
              for (int pb = 0; pb < 3; ++pb)
                c = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xc[i][h].h,
                                                            b[pb].h, c, 0, 0, 0);
              acc[i][j] = c;
            }
          }
        }
      }
    }
  }
  // accumulator layout: lane holds expert 16j + (lane & 15) and tokens
  // 16i + 4*(lane >> 4) + r
#pragma unroll
  for (int i = 0; i < RLW_TT; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = t0 + 16 * i + 4 * kq + r, e = e0 + 16 * j + row;
        if (t < T && e < E) part[((size_t)ks * T + t) * E + e] = acc[i][j][r];
      }
}

// One token's choice from its float32 logits l (router bias included; lane
// holds experts lane + 64c, -inf past E): the selection keys (the logit, or
// with a selection bias the logit or sigmoid score plus the bias), the
// scores (softmax, or per-expert sigmoid), k rounds of wave argmax on (key,
// index) with equal keys going to the lower index, and the gates; lane j < k
// writes slot j of token t.  Adds the token's scores scaled to sum to 1 to
// psum (the aux loss's P).  Whole wave.
template <int MAXC>
__device__ __forceinline__ void select_token(
    const float (&l)[MAXC], int t, int lane, const float* __restrict__ select_bias,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out,
    float (&psum)[MAXC], int E, int k, int scoring, int raw) {
  float key[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = lane + 64 * c;
    // sigmoid scores with a selection bias: the bias is on the score scale;
    // otherwise the logit orders the choice
    key[c] = e >= E ? -INFINITY
             : select_bias ? (scoring ? sigmoid_f(l[c]) : l[c]) + select_bias[e]
                           : l[c];
  }
  // per-token scores: softmax probs, or sigmoid scores; P accumulates
  // the scores scaled to sum to 1
  float m = -INFINITY, inv;
  float ex[MAXC], se = 0.f;
  if (!scoring) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) m = fmaxf(m, l[c]);
    m = wave_max(m);
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = lane + 64 * c;
      ex[c] = (e < E) ? __expf(l[c] - m) : 0.f;
      se += ex[c];
    }
  } else {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = lane + 64 * c;
      ex[c] = (e < E) ? sigmoid_f(l[c]) : 0.f;
      se += ex[c];
    }
  }
  se = wave_sum(se);
  inv = 1.0f / se;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) psum[c] += ex[c] * inv;

  // k rounds of wave argmax on (key desc, index asc); lane j keeps the
  // winner of round j (slot j) and its logit.
  bool taken[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) taken[c] = (lane + 64 * c) >= E;
  int my_idx = 0;
  float my_l = -INFINITY;
  for (int j = 0; j < k; ++j) {
    float bk = -INFINITY, bl = -INFINITY;
    int bi = 0x7fffffff;
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      // indices rise with c: strict > keeps the lower index on ties
      if (!taken[c] && (bi == 0x7fffffff || key[c] > bk)) {
        bk = key[c];
        bi = lane + 64 * c;
        bl = l[c];
      }
    }
    // wave argmax on (key desc, index asc): a total order, so the DPP
    // steps of the wave reductions give the same winner in any order
    auto take = [&](float ok, int oi, float ol) {
      const bool better = (oi != 0x7fffffff) &&
                          (bi == 0x7fffffff || ok > bk || (ok == bk && oi < bi));
      if (better) {
        bk = ok;
        bi = oi;
        bl = ol;
      }
    };
#define MOE_ARGMAX_STEP(CTRL, RM)                                       \
    take(dpp_f<CTRL, RM>(bk, bk), dpp_i<CTRL, RM>(bi, bi),           \
         dpp_f<CTRL, RM>(bl, bl))
    MOE_ARGMAX_STEP(DPP_QUAD_1032, 0xf);
    MOE_ARGMAX_STEP(DPP_QUAD_2301, 0xf);
    MOE_ARGMAX_STEP(DPP_ROW_HALF_MIRROR, 0xf);
    MOE_ARGMAX_STEP(DPP_ROW_MIRROR, 0xf);
    MOE_ARGMAX_STEP(DPP_ROW_BCAST15, 0xa);
    MOE_ARGMAX_STEP(DPP_ROW_BCAST31, 0xc);
#undef MOE_ARGMAX_STEP
    bk = lane63(bk);
    bi = __builtin_amdgcn_readlane(bi, 63);
    bl = lane63(bl);
    // every lane now holds the same winner
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
      if (lane + 64 * c == bi) taken[c] = true;
    if (lane == j) {
      my_idx = bi;
      my_l = bl;
    }
  }
  // gates.  Softmax, renormalised: chosen probabilities over their sum,
  // i.e. a softmax over the chosen logits (the shared normaliser
  // cancels).  Softmax, raw: the chosen probability.  Sigmoid: the chosen
  // score, over the chosen scores' sum when renormalised.
  float g;
  if (!scoring) {
    if (!raw) {
      const float mc = wave_max(lane < k ? my_l : -INFINITY);
      const float ej = lane < k ? __expf(my_l - mc) : 0.f;
      const float sj = wave_sum(ej);
      g = ej / sj;
    } else {
      g = __expf(my_l - m) * inv;
    }
  } else {
    const float sc = lane < k ? sigmoid_f(my_l) : 0.f;
    if (!raw) {
      const float sj = wave_sum(sc);
      g = sc / sj;
    } else {
      g = sc;
    }
  }
  if (lane < k) {
    idx_out[(size_t)t * k + lane] = my_idx;
    gate_out[(size_t)t * k + lane] = g;
  }
}

constexpr int RS_WAVES = ROUTE_WAVES;

// MAXC experts per lane (E <= 64*MAXC), KSM = largest K split, PF: load the
// next token's partial logits while the current token is processed (used
// when a wave handles several tokens; the K split is then at most
// RLW_MAX_KSPLIT).
template <int MAXC, int KSM, bool PF>
__global__ __launch_bounds__(RS_WAVES * 64) void route_select_kernel(
    const float* __restrict__ part, int ksplit,
    const float* __restrict__ router_bias,
    const float* __restrict__ select_bias, float* __restrict__ logits_out,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out,
    float* __restrict__ partials, int T, int E, int k, int tpw, int scoring,
    int raw) {
  __shared__ float psum_s[RS_WAVES][256];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  float psum[MAXC];
#pragma unroll
  for (int c = 0; c < MAXC; ++c) psum[c] = 0.f;

  const int tbeg = (blockIdx.x * RS_WAVES + wave) * tpw;
  const int tend = min(tbeg + tpw, T);
  // pvn: the partial logits being fetched (the next token's with PF), pvc:
  // the current token's (a copy taken at the top of each token, so every
  // register index is a compile-time constant)
  float pvn[MAXC][KSM], pvc[MAXC][KSM];
  auto fetch = [&](int t) {
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = lane + 64 * c;
#pragma unroll
      for (int s = 0; s < KSM; ++s)
        pvn[c][s] = (e < E && s < ksplit)
                        ? part[((size_t)s * T + t) * E + e] : 0.f;
    }
  };
  if (PF && tbeg < tend) fetch(tbeg);
  for (int i = 0; i < tpw; ++i) {
    const int t = tbeg + i;
    if (t >= tend) break;   // wave-uniform
    if (!PF) fetch(t);
#pragma unroll
    for (int c = 0; c < MAXC; ++c)
#pragma unroll
      for (int s = 0; s < KSM; ++s) pvc[c][s] = pvn[c][s];
    if (PF && t + 1 < tend) fetch(t + 1);
    float l[MAXC];
#pragma unroll
    for (int c = 0; c < MAXC; ++c) {
      const int e = lane + 64 * c;
      l[c] = -INFINITY;
      if (e < E) {
        // K-slice partial sums added in slice order
        float v = pvc[c][0];
#pragma unroll
        for (int s = 1; s < KSM; ++s)
          if (s < ksplit) v += pvc[c][s];
        if (router_bias) v += router_bias[e];
        l[c] = v;
        if (logits_out) logits_out[(size_t)t * E + e] = v;
      }
    }
    select_token<MAXC>(l, t, lane, select_bias, idx_out, gate_out, psum, E,
                       k, scoring, raw);
  }
  // per-block probability partial sums, waves added in order 0..3
  for (int e = lane; e < 256; e += 64) psum_s[wave][e] = 0.f;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) psum_s[wave][lane + 64 * c] = psum[c];
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    float v = psum_s[0][e];
    v += psum_s[1][e];
    v += psum_s[2][e];
    v += psum_s[3][e];
    partials[(size_t)blockIdx.x * E + e] = v;
  }
}

// Fused route for small batches with few experts (decode): one workgroup
// per token runs the router linear, the softmax, the top-k and the gates in
// one launch.  The router GEMM is float32 on the vector units (a handful of
// tokens leaves the matrix cores nothing to fill): thread i takes the K
// chunks of 8 at 8i, 8i + 8*RF_THREADS, ... for every expert, adding the
// products in K order; each expert's 256 partial sums are reduced within
// each 16-lane row by DPP butterflies (quad, half-row and row mirrors, so
// every lane of a row holds the same sum) and the 16 row sums added in a
// fixed order through LDS.  Wave 0 then scores, chooses and gates the token
// with the select kernel's own code.  The token's scores scaled to sum to 1
// are its row of the probability partials (one row per token).
constexpr int RF_THREADS = 256;
constexpr int RF_MAXE = 8;       // experts per token held in registers
constexpr int RF_MAXT = 128;     // tokens (workgroups) the fused path takes

template <typename XT>
__device__ __forceinline__ void load8f(const XT* p, float* out);
template <>
__device__ __forceinline__ void load8f<bf16>(const bf16* p, float* out) {
  V16 a;
  a.u = ldg16(p);
#pragma unroll
  for (int i = 0; i < 8; ++i) out[i] = (float)a.h[i];
}
template <>
__device__ __forceinline__ void load8f<float>(const float* p, float* out) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    V16 v;
    v.u = ldg16(p + 4 * i);
#pragma unroll
    for (int j = 0; j < 4; ++j) out[4 * i + j] = v.f[j];
  }
}

template <typename XT>
__global__ __launch_bounds__(RF_THREADS) void route_fused_kernel(
    const XT* __restrict__ x, const float* __restrict__ wr,
    const float* __restrict__ router_bias,
    const float* __restrict__ select_bias, float* __restrict__ logits_out,
    int32_t* __restrict__ idx_out, float* __restrict__ gate_out,
    float* __restrict__ partials, int d, int E, int k, int scoring,
    int raw) {
  __shared__ float red[RF_MAXE][RF_THREADS / 16];
  const int t = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  float acc[RF_MAXE];
#pragma unroll
  for (int e = 0; e < RF_MAXE; ++e) acc[e] = 0.f;
  const XT* xr = x + (size_t)t * d;
  // RF_U chunks per thread per trip, all their loads issued before the
  // first product (one memory latency per trip, not one per chunk); chunks
  // past d are skipped, the products still added in K order
  constexpr int RF_U = 2;
  for (int k0 = tid * 8; k0 < d; k0 += RF_U * RF_THREADS * 8) {
    float xv[RF_U][8];
    V16 w[RF_U][RF_MAXE][2];
#pragma unroll
    for (int u = 0; u < RF_U; ++u) {
      const int kk = k0 + u * RF_THREADS * 8;
      if (kk < d) {
        load8f<XT>(xr + kk, xv[u]);
#pragma unroll
        for (int e = 0; e < RF_MAXE; ++e) {
          if (e < E) {
            w[u][e][0].u = ldg16(wr + (size_t)e * d + kk);
            w[u][e][1].u = ldg16(wr + (size_t)e * d + kk + 4);
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < RF_U; ++u) {
      if (k0 + u * RF_THREADS * 8 < d) {
#pragma unroll
        for (int e = 0; e < RF_MAXE; ++e) {
          if (e < E) {
            float a = acc[e];
#pragma unroll
            for (int j = 0; j < 4; ++j) a = fmaf(xv[u][j], w[u][e][0].f[j], a);
#pragma unroll
            for (int j = 0; j < 4; ++j)
              a = fmaf(xv[u][4 + j], w[u][e][1].f[j], a);
            acc[e] = a;
          }
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < RF_MAXE; ++e) {
    if (e < E) {
      float v = acc[e];
      v += dpp_f<DPP_QUAD_1032>(0.f, v);
      v += dpp_f<DPP_QUAD_2301>(0.f, v);
      v += dpp_f<DPP_ROW_HALF_MIRROR>(0.f, v);
      v += dpp_f<DPP_ROW_MIRROR>(0.f, v);
      if ((lane & 15) == 0) red[e][wave * 4 + (lane >> 4)] = v;
    }
  }
  __syncthreads();
  if (wave != 0) return;
  float l[1] = {-INFINITY};
  if (lane < E) {
    float v = red[lane][0];
#pragma unroll
    for (int r = 1; r < RF_THREADS / 16; ++r) v += red[lane][r];
    if (router_bias) v += router_bias[lane];
    l[0] = v;
    if (logits_out) logits_out[(size_t)t * E + lane] = v;
  }
  float psum[1] = {0.f};
  select_token<1>(l, t, lane, select_bias, idx_out, gate_out, psum, E, k,
                  scoring, raw);
  if (lane < E) partials[(size_t)t * E + lane] = psum[0];
}

// Column means of the per-block probability partials [nblk, E], in a fixed
// order: 64 experts per workgroup, PM_PARTS strided parts per expert (part
// p adds blocks p, p + PM_PARTS, ...), then the parts added in order.
constexpr int PM_PARTS = 16;
__global__ __launch_bounds__(64 * PM_PARTS) void prob_mean_kernel(
    const float* __restrict__ partials, float* __restrict__ pm, int nblk,
    int T, int E) {
  __shared__ float part[PM_PARTS][64];
  const int lane = threadIdx.x & 63, p = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  float v = 0.f;
  if (e < E) {
#pragma unroll 4
    for (int b = p; b < nblk; b += PM_PARTS) v += partials[(size_t)b * E + e];
  }
  part[p][lane] = v;
  __syncthreads();
  if (p == 0 && e < E) {
    float sum = 0.f;
#pragma unroll
    for (int q = 0; q < PM_PARTS; ++q) sum += part[q][lane];
    pm[e] = T > 0 ? sum / (float)T : 0.f;
  }
}

}  // namespace

// Batches that take the wide router kernel: bf16 x past 2048 tokens (the
// batches whose select waves handle several tokens each).
static bool router_wide(int T, int dtype) { return dtype == 1 && route_tpw(T) > 1; }

// Number of K slices for the router GEMM: each slice a whole number of
// 64-wide steps (at least 4), the largest split that keeps the grid within
// about 1024 workgroups (wide kernel: 512 workgroups of 256 tokens, at most
// RLW_MAX_KSPLIT slices), so that small batches and wide routers still fill
// the chip with independent load chains.
int router_ksplit(int T, int d, int E, int dtype) {
  const int steps = d / RL_KSTEP;
  const long long etiles = (E + RL_EXP_TILE - 1) / RL_EXP_TILE;
  if (router_wide(T, dtype)) {
    const long long blocks = (long long)((T + RLW_TOK - 1) / RLW_TOK) * etiles;
    int best = 1;
    for (int ks = 2; ks <= RLW_MAX_KSPLIT; ks *= 2) {
      if (steps % ks != 0 || steps / ks < 4 || blocks * ks > 512) break;
      best = ks;
    }
    return best;
  }
  const int tt = dtype == 1 ? 64 : 16;
  const long long blocks = (long long)((T + tt - 1) / tt) * etiles;
  // a wave of the select kernel that handles several tokens sums at most
  // RLW_MAX_KSPLIT slices per token; float32 x keeps two
  const int kmax = route_tpw(T) > 1 ? 2 : ROUTER_MAX_KSPLIT;
  int best = 1;
  for (int ks = 2; ks <= kmax; ++ks) {
    if (steps % ks != 0 || steps / ks < 4) continue;
    if (blocks * ks > 1024) break;
    best = ks;
  }
  return best;
}

hipError_t launch_router_logits_partial(int dtype, const void* x,
                                        const float* wr, float* part, int T,
                                        int d, int E, int ksplit,
                                        hipStream_t s) {
  if (router_wide(T, dtype)) {
    dim3 grid((T + RLW_TOK - 1) / RLW_TOK, (E + RL_EXP_TILE - 1) / RL_EXP_TILE,
              ksplit);
    router_logits_wide_kernel<<<grid, RL_THREADS, 0, s>>>(
        (const bf16*)x, wr, part, T, d, E, ksplit);
  } else if (dtype == 1) {
    dim3 grid((T + 63) / 64, (E + RL_EXP_TILE - 1) / RL_EXP_TILE, ksplit);
    router_logits_kernel<bf16, 1, 4><<<grid, RL_THREADS, 0, s>>>(
        (const bf16*)x, wr, part, T, d, E, ksplit);
  } else {
    dim3 grid((T + 15) / 16, (E + RL_EXP_TILE - 1) / RL_EXP_TILE, ksplit);
    router_logits_kernel<float, 3, 1><<<grid, RL_THREADS, 0, s>>>(
        (const float*)x, wr, part, T, d, E, ksplit);
  }
  return hipGetLastError();
}

hipError_t launch_route_select_from(const float* part, int ksplit,
                                    const float* router_bias,
                                    const float* select_bias, float* logits,
                                    int32_t* idx, float* gate,
                                    float* partials, int T, int E, int k,
                                    int scoring, int raw, hipStream_t s) {
  const int tpw = route_tpw(T);
  const dim3 grid(route_blocks(T)), block(RS_WAVES * 64);
#define MOE_SELECT(C, KS, PF)                                                 \
  route_select_kernel<C, KS, PF><<<grid, block, 0, s>>>(                      \
      part, ksplit, router_bias, select_bias, logits, idx, gate, partials, T, \
      E, k, tpw, scoring, raw)
  const int mc = (E + 63) / 64;
  if (tpw > 1) {   // several tokens per wave: K split <= 8, prefetch
    if (mc == 1) MOE_SELECT(1, RLW_MAX_KSPLIT, true);
    else if (mc == 2) MOE_SELECT(2, RLW_MAX_KSPLIT, true);
    else MOE_SELECT(4, RLW_MAX_KSPLIT, true);
  } else {
    if (mc == 1) MOE_SELECT(1, ROUTER_MAX_KSPLIT, false);
    else if (mc == 2) MOE_SELECT(2, ROUTER_MAX_KSPLIT, false);
    else MOE_SELECT(4, ROUTER_MAX_KSPLIT, false);
  }
#undef MOE_SELECT
  return hipGetLastError();
}

bool route_fused(int T, int E) { return T <= RF_MAXT && E <= RF_MAXE; }

int route_partial_rows(int T, int E) {
  return route_fused(T, E) ? T : route_blocks(T);
}

hipError_t launch_route_fused(int dtype, const void* x, const float* wr,
                              const float* router_bias,
                              const float* select_bias, float* logits,
                              int32_t* idx, float* gate, float* partials,
                              int T, int d, int E, int k, int scoring,
                              int raw, hipStream_t s) {
  if (dtype == 1)
    route_fused_kernel<bf16><<<T, RF_THREADS, 0, s>>>(
        (const bf16*)x, wr, router_bias, select_bias, logits, idx, gate,
        partials, d, E, k, scoring, raw);
  else
    route_fused_kernel<float><<<T, RF_THREADS, 0, s>>>(
        (const float*)x, wr, router_bias, select_bias, logits, idx, gate,
        partials, d, E, k, scoring, raw);
  return hipGetLastError();
}

hipError_t launch_prob_mean(const float* partials, float* prob_mean, int nblk,
                            int T, int E, hipStream_t s) {
  prob_mean_kernel<<<(E + 63) / 64, 64 * PM_PARTS, 0, s>>>(partials, prob_mean,
                                                           nblk, T, E);
  return hipGetLastError();
}

namespace {
// select_bias[e] += gamma * sign(sum(counts) - E * counts[e]) (exact sign)
__global__ void update_select_bias_kernel(const int32_t* __restrict__ counts,
                                          float* __restrict__ bias,
                                          float gamma, int E) {
  __shared__ long long total_s;
  if (threadIdx.x == 0) {
    long long tot = 0;
    for (int e = 0; e < E; ++e) tot += counts[e];
    total_s = tot;
  }
  __syncthreads();
  for (int e = threadIdx.x; e < E; e += blockDim.x) {
    const long long d = total_s - (long long)E * counts[e];
    const float sg = d > 0 ? 1.0f : (d < 0 ? -1.0f : 0.0f);
    bias[e] = bias[e] + gamma * sg;
  }
}
}  // namespace

hipError_t launch_update_select_bias(const int32_t* counts, float* bias,
                                     float gamma, int E, hipStream_t s) {
  update_select_bias_kernel<<<1, 256, 0, s>>>(counts, bias, gamma, E);
  return hipGetLastError();
}

}  // namespace moe
