// Internal launchers of the MoE kernels (host side).  The C ABI in abi.hip
// validates arguments and sizes the workspace; these only enqueue.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

namespace moe {

// Route-select: 4 waves per workgroup, route_tpw(T) tokens per wave (one
// token per wave for small batches, up to 16 for large ones, so that about
// 512 workgroups cover the batch).  A workgroup writes one row of
// probability partial sums.
constexpr int ROUTE_WAVES = 4;
inline int route_tpw(int T) {
  const int t = (T + 2047) / 2048;
  return t < 1 ? 1 : (t > 16 ? 16 : t);
}
inline int route_blocks(int T) {
  const int per = ROUTE_WAVES * route_tpw(T);
  return (T + per - 1) / per;
}
// Largest K split of the router GEMM.
constexpr int ROUTER_MAX_KSPLIT = 16;
// Assignments (token, slot) handled by one wave in the dispatch kernels.
constexpr int DISPATCH_CHUNK = 256;
// Chunks (one per wave) per dispatch workgroup.
constexpr int DISPATCH_WAVES = 4;

inline int dispatch_chunks(long long tk) {
  return (int)((tk + DISPATCH_CHUNK - 1) / DISPATCH_CHUNK);
}

// ---- route -----------------------------------------------------------------
// K slices of the router GEMM (partial logits [ksplit, T, E] in workspace).
int router_ksplit(int T, int d, int E, int dtype);
// part[ks, t, e] = sum over slice ks of x[t,:] . Wr[e,:]  (float32).
hipError_t launch_router_logits_partial(int dtype, const void* x,
                                        const float* wr, float* part, int T,
                                        int d, int E, int ksplit,
                                        hipStream_t s);
// Sum the slices (+ router bias), score (softmax, or sigmoid when
// scoring = 1), top-k, gates (renormalised unless raw = 1), and per-block
// probability partial sums [route_blocks(T), E].  logits may be null.
hipError_t launch_route_select_from(const float* part, int ksplit,
                                    const float* router_bias,
                                    const float* select_bias, float* logits,
                                    int32_t* idx, float* gate,
                                    float* partials, int T, int E, int k,
                                    int scoring, int raw, hipStream_t s);
// Small batches with few experts (decode) take one fused kernel: router
// linear, scores, top-k, gates and one row of probability partials per
// token.  route_partial_rows: rows of partials the route step writes
// (T fused, route_blocks(T) otherwise).
bool route_fused(int T, int E);
int route_partial_rows(int T, int E);
hipError_t launch_route_fused(int dtype, const void* x, const float* wr,
                              const float* router_bias,
                              const float* select_bias, float* logits,
                              int32_t* idx, float* gate, float* partials,
                              int T, int d, int E, int k, int scoring,
                              int raw, hipStream_t s);
// select_bias[e] += gamma * sign(mean count - counts[e]).
hipError_t launch_update_select_bias(const int32_t* counts, float* bias,
                                     float gamma, int E, hipStream_t s);
// prob_mean[e] = sum_b partials[b,e] / T (fixed order).
hipError_t launch_prob_mean(const float* partials, float* prob_mean, int nblk,
                            int T, int E, hipStream_t s);

// ---- dispatch --------------------------------------------------------------
// counts/offsets/perm/slot_of/n_dropped and optionally prob_mean + aux.
// `partials` (route partial sums, nblk rows) may be given instead of a
// finished prob_mean; then prob_mean_out receives the mean.
struct DispatchArgs {
  const int32_t* idx;
  const float* prob_mean_in;   // or nullptr
  const float* partials;       // or nullptr
  int n_partials;
  float* prob_mean_out;        // written when partials != nullptr
  int32_t* counts;
  int32_t* offsets;
  int32_t* perm;
  int32_t* slot_of;
  int32_t* n_dropped;
  float* aux;                  // or nullptr
  int32_t* chunk_ws;           // [nchunks, E]
  int T, E, k, capacity;
  float aux_coef;
};
hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s);

// Overflow reassignment after launch_dispatch (which wrote the cut's
// offsets into off0 and slot_of with -1 for drops; perm is rewritten).
struct ReassignArgs {
  int32_t* idx;           // [T*k] in/out
  float* gate;            // [T*k] in/out
  const float* logits;    // [T, E]
  const int32_t* off0;    // [E+1] offsets after the cut
  int32_t* offsets;       // [E+1] out
  int32_t* perm;          // [T*k] out
  int32_t* slot_of;       // [T*k] in (after the cut) / out
  int32_t* n_dropped;     // [1] out
  int32_t* rslot;         // [T*k] workspace: rank among an expert's moved
  int32_t* newe;          // [T*k] workspace: the moved slot's new expert
  int T, E, k, capacity, scoring, raw;
  uint32_t key0, key1;
};
hipError_t launch_reassign(const ReassignArgs& a, hipStream_t s);

// ---- expert FFN ------------------------------------------------------------
struct FfnArgs {
  int dtype, act;
  int T, d, E, k, d_ff, n_shared;
  const void* x;
  const int32_t* perm;
  const int32_t* offsets;
  const void *w1, *w_up, *w2, *b1, *b2;
  const void *sw1, *sw_up, *sw2, *sb1, *sb2;
  void* h;   // [T*k + n_shared*T, d_ff] workspace
  void* y;   // [T*k + n_shared*T, d]
  // wquant = 2: bf16 matrices in tiled order (moe_tile_bf16).
  // 4-bit weights: wquant = 1, matrices hold codes, *q the (scale, offset)
  // pairs per group of Q4_GROUP weights
  int wquant;
  const float *w1q, *w_upq, *w2q, *sw1q, *sw_upq, *sw2q;
  // tiled schedule, last round split along K (optional workspace): one
  // partial tile of SPLIT_TILE_FLOATS floats and one counter per CU for
  // split_cpx CUs per XCD; split_part == nullptr: no split
  float* split_part;
  int32_t* split_cnt;
  int split_cpx;
};
constexpr int SPLIT_TILE_FLOATS = 256 * 256;
// CUs of the current device (persistent and split grids)
int device_cus();
hipError_t launch_expert_up(const FfnArgs& a, hipStream_t s);
hipError_t launch_expert_down(const FfnArgs& a, hipStream_t s);
// the same with 4-bit weights (wquant 1; called by the two above)
hipError_t launch_q4_up(const FfnArgs& a, hipStream_t s);
hipError_t launch_q4_down(const FfnArgs& a, hipStream_t s);

// ---- 4-bit weights ---------------------------------------------------------
constexpr int Q4_GROUP = 128;   // weights per (scale, offset) pair
hipError_t launch_quantize_int4(const void* w, long long rows, int K,
                                void* codes, float* qparams, hipStream_t s);
// bf16 [rows, K] -> tiled order (16 x 32 tiles in 16x16x32 operand order)
hipError_t launch_tile_bf16(const void* w, long long rows, int K, void* out,
                            hipStream_t s);

// ---- combine ---------------------------------------------------------------
hipError_t launch_combine(int dtype, const void* x, const void* y,
                          const int32_t* slot_of, const float* gate,
                          void* out, int T, int d, int k, int n_shared,
                          hipStream_t s);

// ---- misc ------------------------------------------------------------------
// Writes zeros (int32 / float32) - used for the T = 0 outputs.
hipError_t launch_fill_zero32(void* p, long long n, hipStream_t s);

}  // namespace moe
