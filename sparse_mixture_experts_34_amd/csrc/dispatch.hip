// Dispatch: group (token, slot) assignments by expert under a capacity cut,
// and the load-balance aux loss.
//
// For each expert the assignments routed to it are ranked in ascending
// token order; ranks below the capacity are kept, the rest dropped (their
// MoE output is zero and the residual carries the token) - randomcommits.com
// "Mixture-of-Experts routing", How a sparse MoE layer works (the capacity
// check on a row-major nonzero of the routing mask);
// letsbuildsolutions.com "How Mixture of Experts Works", The Capacity
// Factor and Token Dropping and Overflow Handling.  The aux loss is
// alpha * E * sum_e f_e P_e with f_e the pre-capacity fraction of
// assignments routed to e per token and P_e the mean router probability
// (same page, The Load Balancing Problem).
//
// Assignment a = t*k + j.  For a fixed expert, ascending a is ascending t
// (a token never picks an expert twice), so the stable order is the
// assignment order.  The work splits into chunks of 256 consecutive
// assignments, one wave each:
//   count   per-chunk expert histogram (LDS integer atomics: the final
//           counts do not depend on their order)
//   scan    one workgroup: per expert, exclusive scan over chunks (chunk
//           base ranks), counts, kept = min(count, capacity), offsets =
//           exclusive scan of kept over experts, n_dropped, prob mean and
//           aux loss (fixed-order sums)
//   scatter per chunk, 64 assignments at a time: an assignment's rank is its
//           chunk base plus the number of earlier same-expert assignments
//           (earlier rounds: LDS counter; same round: lanes below it)
// Small batches (at most 4 chunks) run all three in one workgroup.
#include "common.hpp"
#include "kernels.hpp"

namespace moe {

namespace {

constexpr int DW = DISPATCH_WAVES;
constexpr int CH = DISPATCH_CHUNK;

// Histogram of chunk `c` into hist[0..E) (must start at zero).
// Expert ids outside [0, E) are ignored here and dropped by the scatter.
__device__ __forceinline__ void count_chunk(const int32_t* __restrict__ idx,
                                            long long tk, int E, int c,
                                            int* hist, int lane) {
  for (int r = 0; r < CH / 64; ++r) {
    long long a = (long long)c * CH + r * 64 + lane;
    if (a < tk) {
      const int e = idx[a];
      if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);
    }
  }
}

// Rank and scatter the assignments of chunk c.  base[e] holds the chunk's
// base rank per expert and is advanced in place.
__device__ __forceinline__ void scatter_chunk(
    const int32_t* __restrict__ idx, long long tk, int c, int* base,
    const int32_t* offsets, int E, int32_t* __restrict__ perm,
    int32_t* __restrict__ slot_of, int lane) {
  const long long c0 = (long long)c * CH;
  const int rounds = (int)min((long long)(CH / 64), (tk - c0 + 63) / 64);
  for (int r = 0; r < rounds; ++r) {
    const long long a = c0 + r * 64 + lane;
    int e = a < tk ? idx[a] : -1;
    if ((unsigned)e >= (unsigned)E) e = -1;
    int before = 0;
#pragma unroll 16
    for (int l = 0; l < 64; ++l) {
      const int v = __builtin_amdgcn_readlane(e, l);
      before += (v == e && l < lane) ? 1 : 0;
    }
    const int rank = e >= 0 ? base[e] + before : 0;
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0);
    if (e >= 0) atomicAdd(&base[e], 1);
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_s_waitcnt(0);
    if (a < tk && e < 0) slot_of[a] = -1;
    if (e >= 0) {
      const int keep = offsets[e + 1] - offsets[e];
      if (rank < keep) {
        const int p = offsets[e] + rank;
        perm[p] = (int32_t)a;
        slot_of[a] = p;
      } else {
        slot_of[a] = -1;
      }
    }
  }
  // perm rows past the kept total are set to -1
  const int total = offsets[E];
  for (int r = 0; r < rounds; ++r) {
    const long long p = c0 + r * 64 + lane;
    if (p < tk && p >= total) perm[p] = -1;
  }
}

// Scan over chunks and experts, executed by one workgroup of NTHR threads.
// chunk[c*E + e] holds per-chunk counts on entry and chunk base ranks on
// exit.  Writes counts, offsets, n_dropped, prob mean and aux.
//
// Each expert gets TPE threads (a power of two, at most NTHR / E, no more
// than the chunks and partial rows need): thread j scans a
// contiguous range of chunks and sums an interleaved share of the
// probability partial rows; the TPE pieces are combined in the fixed order
// j = 0, 1, ... (deterministic).  red_* hold NTHR entries.
template <int NTHR>
__device__ void scan_all(int* chunk, int nchunks, const DispatchArgs& a,
                         int32_t* offsets_out, int* red_i, float* red_f) {
  const int t = threadIdx.x;
  const int E = a.E;
  // threads per expert: enough to split the chunk scan and the partial
  // rows, at most NTHR / E (the pieces are combined serially)
  const int n_part = a.partials ? a.n_partials : 0;
  const int need = max(max(nchunks, (n_part + 15) / 16), 1);
  int tpe = 1;
  while (tpe < need && tpe * 2 * E <= NTHR) tpe *= 2;
  // expert-minor: consecutive lanes take consecutive experts of one chunk
  // row, so the chunk and partial loads are coalesced
  const bool act = t < tpe * E;
  const int e = act ? t % E : E, j = act ? t / E : 0;
  // ---- per-chunk counts -> chunk base ranks, per-expert totals ----------
  const int cpt = (nchunks + tpe - 1) / tpe;
  const int c0 = min(j * cpt, nchunks), c1 = min(c0 + cpt, nchunks);
  int local = 0;
  if (act) {
#pragma unroll 8
    for (int c = c0; c < c1; ++c) local += chunk[c * E + e];
  }
  red_i[t] = local;
  __syncthreads();
  int base = 0, count = 0;
  if (act) {
    for (int jj = 0; jj < tpe; ++jj) {
      const int v = red_i[jj * E + e];
      if (jj < j) base += v;
      count += v;
    }
    int run = base;
    for (int c = c0; c < c1; ++c) {
      const int v = chunk[c * E + e];
      chunk[c * E + e] = run;
      run += v;
    }
  }
  __syncthreads();
  // ---- kept counts, exclusive scan over experts --------------------------
  const int kept_e = (act && j == 0)
                         ? (a.capacity > 0 ? min(count, a.capacity) : count)
                         : 0;
  if (t < 256) red_i[t] = 0;
  __syncthreads();
  if (act && j == 0) red_i[e] = kept_e;
  __syncthreads();
  for (int o = 1; o < E; o <<= 1) {   // entries >= E stay 0
    int v = (t < 256 && t >= o) ? red_i[t - o] : 0;
    __syncthreads();
    if (t < 256) red_i[t] += v;
    __syncthreads();
  }
  if (act && j == 0) {
    const int incl = red_i[e];
    a.counts[e] = count;
    offsets_out[e] = incl - kept_e;
    if (e == E - 1) {
      offsets_out[E] = incl;
      *a.n_dropped = (int32_t)((long long)a.T * a.k - incl);
    }
  }
  // ---- probability mean (fixed-order sums) and aux loss ------------------
  float pm_part = 0.f;
  if (act && a.partials) {
    float accs[4] = {0.f, 0.f, 0.f, 0.f};
    int q = 0;
#pragma unroll 4
    for (int b = j; b < a.n_partials; b += tpe) {
      accs[q & 3] += a.partials[(size_t)b * E + e];
      ++q;
    }
    pm_part = (accs[0] + accs[1]) + (accs[2] + accs[3]);
  }
  __syncthreads();
  red_f[t] = pm_part;
  __syncthreads();
  float term = 0.f;
  if (act && j == 0) {
    float pm;
    if (a.partials) {
      float v = 0.f;
      for (int jj = 0; jj < tpe; ++jj) v += red_f[jj * E + e];
      pm = v / (float)a.T;
      if (a.prob_mean_out) a.prob_mean_out[e] = pm;
    } else {
      pm = a.prob_mean_in ? a.prob_mean_in[e] : 0.f;
    }
    term = ((float)count / (float)a.T) * pm;
  }
  __syncthreads();
  if (t < 256) red_f[t] = 0.f;
  __syncthreads();
  if (act && j == 0) red_f[e] = term;
  __syncthreads();
  int half = 1;
  while (half * 2 < E) half *= 2;     // terms >= E are 0
  for (int o = half; o >= 1; o >>= 1) {
    if (t < o) red_f[t] += red_f[t + o];
    __syncthreads();
  }
  if (t == 0 && a.aux) *a.aux = a.aux_coef * (float)E * red_f[0];
}

__global__ __launch_bounds__(DW * 64) void dispatch_count_kernel(
    const int32_t* __restrict__ idx, long long tk, int nchunks, int E,
    int32_t* __restrict__ chunk_ws) {
  __shared__ int hist[DW][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  for (int e = lane; e < 256; e += 64) hist[wave][e] = 0;
  __syncthreads();
  const int c = blockIdx.x * DW + wave;
  if (c < nchunks) count_chunk(idx, tk, E, c, hist[wave], lane);
  __syncthreads();
  if (c < nchunks)
    for (int e = lane; e < E; e += 64) chunk_ws[(size_t)c * E + e] = hist[wave][e];
}

constexpr int SCAN_THREADS = 1024;

__global__ __launch_bounds__(SCAN_THREADS) void dispatch_scan_kernel(
    DispatchArgs a, int nchunks) {
  __shared__ int red_i[SCAN_THREADS];
  __shared__ float red_f[SCAN_THREADS];
  scan_all<SCAN_THREADS>(a.chunk_ws, nchunks, a, a.offsets, red_i, red_f);
}

__global__ __launch_bounds__(DW * 64) void dispatch_scatter_kernel(
    DispatchArgs a, int nchunks) {
  __shared__ int base[DW][256];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = blockIdx.x * DW + wave;
  const long long tk = (long long)a.T * a.k;
  if (c >= nchunks) return;   // no workgroup barrier below
  for (int e = lane; e < a.E; e += 64) base[wave][e] = a.chunk_ws[(size_t)c * a.E + e];
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_s_waitcnt(0);
  scatter_chunk(a.idx, tk, c, base[wave], a.offsets, a.E, a.perm, a.slot_of,
                lane);
}

// Decode-sized batches (at most 64 assignments and 64 experts): the whole
// dispatch in one wave, with no workgroup barrier.  Lane a holds assignment
// a (token a / k, slot a % k) and, as an expert, lane e; one ballot per
// expert gives its count and every assignment's rank among its expert's in
// ascending a (= ascending token); kept counts are scanned across lanes;
// an assignment is kept iff its rank is below the capacity, at row
// offsets[e] + rank.  The probability partial rows are added in row order
// per expert, the aux terms by the fixed DPP butterfly of wave_sum.  An
// expert index outside [0, E) is neither counted nor kept.
__global__ __launch_bounds__(64) void dispatch_wave_kernel(DispatchArgs a) {
  const int lane = threadIdx.x;
  const int tk = a.T * a.k;
  const int E = a.E;
  int my_e = lane < tk ? a.idx[lane] : -1;
  if (my_e >= E) my_e = -1;
  int cnt = 0, rank = 0;
  for (int e = 0; e < E; ++e) {
    const uint64_t m = __ballot(my_e == e);
    if (lane == e) cnt = __popcll(m);
    if (my_e == e) rank = __popcll(m & ((1ull << lane) - 1ull));
  }
  const int kept = lane < E ? (a.capacity > 0 ? min(cnt, a.capacity) : cnt) : 0;
  int incl = kept;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o, 64);
    if (lane >= o) incl += v;
  }
  const int excl = incl - kept;
  const int total = __shfl(incl, 63, 64);
  if (lane < E) {
    a.counts[lane] = cnt;
    a.offsets[lane] = excl;
  }
  if (lane == 0) {
    a.offsets[E] = total;
    *a.n_dropped = tk - total;
  }
  const int base = __shfl(excl, my_e < 0 ? 0 : my_e, 64);
  if (lane < tk) {
    const bool keep = my_e >= 0 && (a.capacity <= 0 || rank < a.capacity);
    const int slot = keep ? base + rank : -1;
    a.slot_of[lane] = slot;
    if (keep) a.perm[slot] = lane;
    if (lane >= total) a.perm[lane] = -1;
  }
  // probability means and the aux loss
  float pm = 0.f;
  if (lane < E) {
    if (a.partials) {
      float v = 0.f;
      for (int r = 0; r < a.n_partials; ++r) v += a.partials[(size_t)r * E + lane];
      pm = v / (float)a.T;
      if (a.prob_mean_out) a.prob_mean_out[lane] = pm;
    } else {
      pm = a.prob_mean_in ? a.prob_mean_in[lane] : 0.f;
    }
  }
  const float term = wave_sum(lane < E ? ((float)cnt / (float)a.T) * pm : 0.f);
  if (lane == 0 && a.aux) *a.aux = a.aux_coef * (float)E * term;
}

// Everything in one workgroup when there are at most DW chunks.
__global__ __launch_bounds__(256) void dispatch_small_kernel(DispatchArgs a,
                                                             int nchunks) {
  __shared__ int chunk[DW * 256];
  __shared__ int red_i[256];
  __shared__ float red_f[256];
  __shared__ int32_t offs[257];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const long long tk = (long long)a.T * a.k;
  for (int i = threadIdx.x; i < DW * 256; i += 256) chunk[i] = 0;
  __syncthreads();
  if (wave < nchunks) count_chunk(a.idx, tk, a.E, wave, chunk + wave * a.E, lane);
  __syncthreads();
  scan_all<256>(chunk, nchunks, a, offs, red_i, red_f);
  __syncthreads();
  for (int e = threadIdx.x; e <= a.E; e += 256) a.offsets[e] = offs[e];
  if (wave < nchunks)
    scatter_chunk(a.idx, tk, wave, chunk + wave * a.E, offs, a.E, a.perm,
                  a.slot_of, lane);
}

// ---------------------------------------------------------------------------
// Overflow by random reassignment (letsbuildsolutions.com "How Mixture of
// Experts Works", Token Dropping and Overflow Handling: overflow tokens go
// to expert slots with room left, weighted by the new expert's router
// probability).  Dropped assignments are visited in ascending id; each
// takes a free slot drawn with Philox4x32-10.  In general the walk is
// sequential (a token's own experts leave the candidates): one wave, lanes
// = experts (4 per lane), the draws of a 64-assignment chunk computed in
// parallel.  With one slot per token the draws' ranges are known in
// advance and the walk is decoded in parallel (reassign_k1_kernel).
// ---------------------------------------------------------------------------

// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
// As Easy as 1, 2, 3", SC 2011): word 0 of the output block.
__device__ __forceinline__ uint32_t philox_word0(uint32_t c0, uint32_t c1,
                                                 uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c0), lo0 = 0xD2511F53u * c0;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c2), lo1 = 0xCD9E8D57u * c2;
    const uint32_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  return c0;
}

__device__ __forceinline__ int wave_incl_scan(int v, int lane) {
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int u = __shfl_up(v, o, 64);
    if (lane >= o) v += u;
  }
  return v;
}

__device__ __forceinline__ int rdlane(int v, int l) {
  return __builtin_amdgcn_readlane(v, l);
}

// The sequential walk.  Lane l holds experts l + 64c (c < MAXC): their
// free slots and the exclusive prefix of free slots over all experts in
// ascending order, kept up to date by -1 past the chosen expert, so a pick
// needs no scan: the token's own experts are taken out of the prefix with
// a few scalar reads, and one ballot finds the expert holding slot r.
// Writes the new expert (newe) and its rank among the expert's moved rows
// (rslot) for every moved assignment, -1 elsewhere, then the offsets.
// KK >= k: slots per token handled (unused ones hold expert -1).
template <int MAXC, int KK>
__global__ __launch_bounds__(64) void reassign_kernel(ReassignArgs a) {
  const int lane = threadIdx.x;
  const long long tk = (long long)a.T * a.k;
  const int E = a.E, k = a.k;
  int spare[MAXC], pre[MAXC], moved[MAXC];
  int run = 0;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = lane + 64 * c;
    spare[c] = e < E ? a.capacity - (a.off0[e + 1] - a.off0[e]) : 0;
    moved[c] = 0;
    const int inc = wave_incl_scan(spare[c], lane);
    pre[c] = run + inc - spare[c];
    run += rdlane(inc, 63);
  }
  int total = run;                       // free slots left (uniform)
  int endv[MAXC];                        // inclusive prefix (one slot/token)
#pragma unroll
  for (int c = 0; c < MAXC; ++c) endv[c] = pre[c] + spare[c];
  int cur_t = -1;
  int cur_e[KK];
#pragma unroll
  for (int jj = 0; jj < KK; ++jj) cur_e[jj] = -1;

  // per-lane view of assignment base + lane: dropped?, token, its experts
  auto load = [&](long long base, bool& drop, int& tok, int* te) {
    const long long aid = base + lane;
    drop = false;
    tok = (int)(aid / k);
    if (aid < tk) {
      const int ea = a.idx[aid];
      drop = a.slot_of[aid] < 0 && (unsigned)ea < (unsigned)E;
    }
#pragma unroll
    for (int jj = 0; jj < KK; ++jj)
      te[jj] = (aid < tk && jj < k) ? a.idx[(size_t)tok * k + jj] : -1;
  };
  bool drop_n;
  int tok_n, te_n[KK];
  load(0, drop_n, tok_n, te_n);
  for (long long base = 0; base < tk; base += 64) {
    const bool drop = drop_n;
    const int tok = tok_n;
    int te[KK];
#pragma unroll
    for (int jj = 0; jj < KK; ++jj) te[jj] = te_n[jj];
    if (base + 64 < tk) load(base + 64, drop_n, tok_n, te_n);   // prefetch
    const long long aid = base + lane;
    uint64_t mask = __ballot(drop);
    int my_rank = -1, my_e = -1;
    if constexpr (KK == 1) {
      // One slot per token: nothing to exclude, and every pick takes one
      // free slot, so the j-th dropped lane of this chunk draws from
      // total - j slots.  Its slot r is known before the walk; the walk
      // only finds the expert holding slot r among the slots still free:
      // the number of experts whose free slots end at or before r (end =
      // inclusive prefix of free slots, kept up to date by -1 from the
      // chosen expert on).
      if (mask && total > 0) {
        const uint32_t x = drop ? philox_word0((uint32_t)aid,
                                               (uint32_t)(aid >> 32), 0u, 0u,
                                               a.key0, a.key1)
                                : 0u;
        const int j = (int)__builtin_amdgcn_mbcnt_hi(
            (uint32_t)(mask >> 32),
            __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
        const int av = total - j;
        const int rl = (drop && av > 0)
                           ? (int)(((unsigned long long)x * (unsigned)av) >> 32)
                           : 0;
        // every dropped lane gets a slot while slots last (av > 0)
        const int npick = min(__popcll(mask), total);
        for (int i = 0; i < npick; ++i) {
          const int b = __ffsll((unsigned long long)mask) - 1;
          mask &= mask - 1;
          const int rb = rdlane(rl, b);
          int e_new = 0;
#pragma unroll
          for (int c = 0; c < MAXC; ++c)
            e_new += __popcll(__ballot(endv[c] <= rb));
          // e_new < E: slot rb < total, the last expert's end
          int rank;
          if constexpr (MAXC == 1) {
            rank = rdlane(moved[0], e_new);
          } else {
            rank = 0;
#pragma unroll
            for (int c = 0; c < MAXC; ++c)
              if (c == (e_new >> 6)) rank = rdlane(moved[c], e_new & 63);
          }
#pragma unroll
          for (int c = 0; c < MAXC; ++c) {
            const int e = lane + 64 * c;
            endv[c] -= e >= e_new ? 1 : 0;
            moved[c] += e == e_new ? 1 : 0;
          }
          if (lane == b) {
            my_e = e_new;
            my_rank = rank;
          }
        }
        total -= npick;
      }
    } else if (mask && total > 0) {
      const uint32_t x = drop ? philox_word0((uint32_t)aid,
                                             (uint32_t)(aid >> 32), 0u, 0u,
                                             a.key0, a.key1)
                              : 0u;
      while (mask) {
        const int b = __ffsll((unsigned long long)mask) - 1;
        mask &= mask - 1;
        // free slots of the token's own experts leave the candidate set.
        // With one slot per token that expert is the one that overflowed,
        // which has no free slot: nothing to exclude.
        int sx[KK];
        int excl = 0;
        int j = 0;
#pragma unroll
        for (int jj = 0; jj < KK; ++jj) sx[jj] = 0;
        if constexpr (KK > 1) {
          const int t = rdlane(tok, b);
          j = (int)((base + b) - (long long)t * k);
          if (t != cur_t) {
            cur_t = t;
#pragma unroll
            for (int jj = 0; jj < KK; ++jj) cur_e[jj] = rdlane(te[jj], b);
          }
#pragma unroll
          for (int jj = 0; jj < KK; ++jj) {
            const int e = cur_e[jj];
            if ((unsigned)e < (unsigned)E) {
              int v = 0;
#pragma unroll
              for (int c = 0; c < MAXC; ++c)
                if ((e >> 6) == c) v = rdlane(spare[c], e & 63);
              sx[jj] = v;
              excl += v;
            }
          }
        }
        const int avail = total - excl;
        if (avail <= 0) continue;        // stays dropped
        const uint32_t xb = (uint32_t)rdlane((int)x, b);
        const int r = (int)(((unsigned long long)xb * (unsigned)avail) >> 32);
        int e_new = -1;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
          const int e = lane + 64 * c;
          int adj = pre[c];
          bool mine = false;
          if constexpr (KK > 1) {
#pragma unroll
            for (int jj = 0; jj < KK; ++jj) {
              adj -= cur_e[jj] < e ? sx[jj] : 0;
              mine |= cur_e[jj] == e;
            }
          }
          const int w = (e < E && !mine) ? spare[c] : 0;
          const uint64_t hit = __ballot(w > 0 && adj <= r && r < adj + w);
          if (e_new < 0 && hit)
            e_new = (__ffsll((unsigned long long)hit) - 1) + 64 * c;
        }
        const int owner = e_new & 63, c_sel = e_new >> 6;
        int rank = 0;
#pragma unroll
        for (int c = 0; c < MAXC; ++c) {
          if (c == c_sel) rank = rdlane(moved[c], owner);
          const int e = lane + 64 * c;
          if (c == c_sel && lane == owner) {
            moved[c] += 1;
            spare[c] -= 1;
          }
          if (e > e_new) pre[c] -= 1;
        }
        total -= 1;
        if constexpr (KK > 1) {
#pragma unroll
          for (int jj = 0; jj < KK; ++jj)
            if (jj == j) cur_e[jj] = e_new;
        }
        if (lane == b) {
          my_rank = rank;
          my_e = e_new;
        }
      }
    }
    if (aid < tk) {
      a.rslot[aid] = my_rank;
      a.newe[aid] = my_e;
    }
  }
  // offsets over the kept plus moved rows (ascending expert)
  run = 0;
#pragma unroll
  for (int c = 0; c < MAXC; ++c) {
    const int e = lane + 64 * c;
    const int kept = e < E ? (a.off0[e + 1] - a.off0[e]) + moved[c] : 0;
    const int inc = wave_incl_scan(kept, lane);
    if (e < E) a.offsets[e] = run + inc - kept;
    run += rdlane(inc, 63);
  }
  if (lane == 0) {
    a.offsets[E] = run;
    *a.n_dropped = (int32_t)(tk - run);
  }
}

// One slot per token (k = 1): the token's own expert overflowed, so it has
// no free slot and every expert with room is a candidate; every draw while
// slots last succeeds, so the j-th dropped assignment draws r_j =
// floor(x_j * (M - j) / 2^32) over the M - j slots still free, with no
// dependence on where the earlier draws landed.  Draw j takes the r_j-th
// slot that remains (free slots laid out in ascending expert order), so the
// walk is the decoding of an inversion table: position p_j in the initial
// layout.  It is decoded bottom-up in LDS like a merge sort: a block of
// draws holds its positions, sorted, relative to the layout left by all
// earlier blocks; merging block A with the block B after it maps each b of
// B to b + #{i : a_i - i <= b} (the b-th slot not taken by A) and each a_i
// of A keeps its position; both land at their merged index, found by one
// binary search in the other block.  Then p_j gives the expert, and each
// draw's rank among its expert's moved rows (in draw order) comes from
// per-wave ballot counts.  Same outputs as reassign_kernel.
constexpr int RP_THREADS = 1024;
constexpr int RP_WAVES = RP_THREADS / 64;
constexpr int RP_MAXP = 16384;   // draws (two 64 KB LDS buffers)
constexpr int RP_MAXE = 512;     // experts (per-wave count tables)
constexpr int RP_PER = RP_MAXP / RP_THREADS;   // draws per thread

// Exclusive prefix of v over the workgroup (RP_THREADS threads) and the
// total; s_w holds RP_WAVES ints.  Whole workgroup.
__device__ __forceinline__ int rp_block_scan(int v, int* s_w, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) s_w[wave] = inc;
  __syncthreads();
  int base = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < RP_WAVES; ++w) {
    const int x = s_w[w];
    if (w < wave) base += x;
    total += x;
  }
  __syncthreads();
  return base + inc - v;
}

// WQ: 64-expert slots per lane for the per-wave counts (E <= 64 * WQ).
template <int WQ>
__global__ __launch_bounds__(RP_THREADS) void reassign_k1_kernel(ReassignArgs a) {
  __shared__ uint32_t buf0[RP_MAXP];
  __shared__ uint32_t buf1[RP_MAXP];
  __shared__ int s_pre[RP_MAXE + 1];   // exclusive prefix of free slots
  __shared__ int s_mv[RP_MAXE];        // moved rows per expert
  __shared__ int s_w[RP_WAVES];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tk = a.T;                  // k = 1
  const int E = a.E;
  int32_t* drops = a.perm;             // scratch: ids of the drawing drops

  // free slots per expert and their exclusive prefix; M = s_pre[E]
  for (int e0 = 0; e0 <= E; e0 += RP_THREADS) {
    const int e = e0 + tid;
    const int sp = e < E ? a.capacity - (a.off0[e + 1] - a.off0[e]) : 0;
    int tot;
    const int ex = rp_block_scan(sp, s_w, tot);
    const int carry = e0 == 0 ? 0 : s_pre[e0];
    __syncthreads();
    if (e <= E) s_pre[e] = carry + ex;
    if (e < E) s_mv[e] = 0;
    __syncthreads();
  }
  const int M = s_pre[E];

  // dropped assignments in ascending id; the first M of them draw
  int nd = 0;
  for (int b0 = 0; b0 < tk; b0 += RP_THREADS) {
    const int aid = b0 + tid;
    bool drop = false;
    if (aid < tk) {
      drop = a.slot_of[aid] < 0 && (unsigned)a.idx[aid] < (unsigned)E;
      a.rslot[aid] = -1;
      a.newe[aid] = -1;
    }
    int tot;
    const int pos = nd + rp_block_scan(drop ? 1 : 0, s_w, tot);
    if (drop && pos < M) drops[pos] = aid;
    nd += tot;
  }
  const int P = min(nd, M);
  __syncthreads();

  // draw j: r_j over the M - j free slots, packed (r << 16) | j
  for (int j = tid; j < P; j += RP_THREADS) {
    const uint32_t aid = (uint32_t)drops[j];
    const uint32_t x = philox_word0(aid, 0u, 0u, 0u, a.key0, a.key1);
    const uint32_t r = (uint32_t)(((unsigned long long)x * (unsigned)(M - j)) >> 32);
    buf0[j] = (r << 16) | (uint32_t)j;
  }
  __syncthreads();

  uint32_t* cur = buf0;
  uint32_t* nxt = buf1;
  for (int h = 1; h < P; h <<= 1) {
    for (int i = tid; i < P; i += RP_THREADS) {
      const int s0 = i & ~(2 * h - 1);
      const int off = i - s0;
      const uint32_t v = cur[i];
      const int pos = (int)(v >> 16);
      if (off < h) {
        // A element: its merged index adds the B positions below its
        // count of untaken slots
        const int b0 = s0 + h;
        const int bn = max(0, min(s0 + 2 * h, P) - b0);
        const int ap = pos - off;
        int lo = 0, hi = bn;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((int)(cur[b0 + mid] >> 16) < ap) lo = mid + 1;
          else hi = mid;
        }
        nxt[s0 + off + lo] = v;
      } else {
        // B element (A is a full block of h): skip the slots A took
        const int jb = off - h;
        int lo = 0, hi = h;
        while (lo < hi) {
          const int mid = (lo + hi) >> 1;
          if ((int)(cur[s0 + mid] >> 16) - mid <= pos) lo = mid + 1;
          else hi = mid;
        }
        nxt[s0 + jb + lo] = ((uint32_t)(pos + lo) << 16) | (v & 0xFFFFu);
      }
    }
    __syncthreads();
    uint32_t* t = cur;
    cur = nxt;
    nxt = t;
  }

  // expert of each position (the one whose free slots hold it), by draw
  for (int i = tid; i < P; i += RP_THREADS) {
    const uint32_t v = cur[i];
    const int pos = (int)(v >> 16);
    int lo = 0, hi = E;   // last e with s_pre[e] <= pos
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (s_pre[mid] <= pos) lo = mid;
      else hi = mid - 1;
    }
    nxt[v & 0xFFFFu] = (uint32_t)lo;
  }
  __syncthreads();
  const uint32_t* ebd = nxt;   // expert by draw
  int* cnt = (int*)cur;        // [RP_WAVES][E] counts, reused LDS

  // Ranks in draw order.  Wave w takes draws [w*Q, (w+1)*Q), 64 at a
  // time; lane l keeps the wave's count of experts l + 64q in wc[q].  In a
  // chunk, each distinct expert is taken once: one ballot finds its draws,
  // their ranks follow the count so far in lane order, and the owning lane
  // adds them.  Pass 1 counts, the waves' counts are prefixed per expert,
  // pass 2 ranks (earlier waves, earlier chunks, lower lanes).
  const int Q = ((P + RP_WAVES - 1) / RP_WAVES + 63) & ~63;
  const int jbeg = wave * Q, jend = min(P, jbeg + Q);
  int wc[WQ];
  auto walk = [&](bool ranks) {
    for (int c = jbeg; c < jend; c += 64) {
      const int j = c + lane;
      const bool valid = j < jend;
      const int e = valid ? (int)ebd[j] : -1;
      int rank = -1;
      uint64_t mask = __ballot(valid);
      while (mask) {
        const int l0 = __ffsll((unsigned long long)mask) - 1;
        const int e0 = rdlane(e, l0);
        const uint64_t m = __ballot(valid && e == e0);
        int base = 0;
#pragma unroll
        for (int q = 0; q < WQ; ++q)
          if ((e0 >> 6) == q) base = rdlane(wc[q], e0 & 63);
        if (e == e0)
          rank = base + (int)__builtin_amdgcn_mbcnt_hi(
                            (uint32_t)(m >> 32),
                            __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
#pragma unroll
        for (int q = 0; q < WQ; ++q)
          if ((e0 >> 6) == q && lane == (e0 & 63)) wc[q] += __popcll(m);
        mask &= ~m;
      }
      if (ranks && valid) {
        const int aid = drops[j];
        a.newe[aid] = e;
        a.rslot[aid] = rank;
      }
    }
  };
#pragma unroll
  for (int q = 0; q < WQ; ++q) wc[q] = 0;
  walk(false);
#pragma unroll
  for (int q = 0; q < WQ; ++q)
    if (lane + 64 * q < E) cnt[wave * E + lane + 64 * q] = wc[q];
  __syncthreads();
  for (int e = tid; e < E; e += RP_THREADS) {
    int run = 0;
    for (int w = 0; w < RP_WAVES; ++w) {
      const int x = cnt[w * E + e];
      cnt[w * E + e] = run;
      run += x;
    }
    s_mv[e] = run;
  }
  __syncthreads();
#pragma unroll
  for (int q = 0; q < WQ; ++q)
    wc[q] = lane + 64 * q < E ? cnt[wave * E + lane + 64 * q] : 0;
  walk(true);
  __syncthreads();

  // offsets over the kept plus moved rows (ascending expert)
  int run = 0;
  for (int e0 = 0; e0 < E; e0 += RP_THREADS) {
    const int e = e0 + tid;
    const int kept = e < E ? (a.off0[e + 1] - a.off0[e]) + s_mv[e] : 0;
    int tot;
    const int ex = rp_block_scan(kept, s_w, tot);
    if (e < E) a.offsets[e] = run + ex;
    run += tot;
  }
  if (tid == 0) {
    a.offsets[E] = run;
    *a.n_dropped = (int32_t)(tk - run);
  }
}

// New rows: an expert's kept assignments keep their order and shift by the
// rows moved into earlier experts; its moved ones follow them.  A moved
// slot's gate: the new expert's score under the token's normaliser (its
// original choice; all experts for raw softmax gates).  idx still holds
// the original choice here.
__global__ void reassign_rebuild_kernel(ReassignArgs a) {
  const long long tk = (long long)a.T * a.k;
  const long long aid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (aid >= tk) return;
  const int old = a.slot_of[aid];
  const int rk = a.rslot[aid];
  int ns = -1;
  if (old >= 0) {
    const int e = a.idx[aid];
    ns = old + (a.offsets[e] - a.off0[e]);
  } else if (rk >= 0) {
    const int e = a.newe[aid];
    ns = a.offsets[e] + (a.off0[e + 1] - a.off0[e]) + rk;
    const int t = (int)(aid / a.k);
    const float* lg = a.logits + (size_t)t * a.E;
    const int32_t* oi = a.idx + (size_t)t * a.k;
    float g;
    if (!a.scoring) {
      float m = -INFINITY, ssum = 0.f;
      if (!a.raw) {
        for (int jj = 0; jj < a.k; ++jj)
          if ((unsigned)oi[jj] < (unsigned)a.E) m = fmaxf(m, lg[oi[jj]]);
        for (int jj = 0; jj < a.k; ++jj)
          if ((unsigned)oi[jj] < (unsigned)a.E) ssum += __expf(lg[oi[jj]] - m);
      } else {
        for (int x = 0; x < a.E; ++x) m = fmaxf(m, lg[x]);
        for (int x = 0; x < a.E; ++x) ssum += __expf(lg[x] - m);
      }
      g = __expf(lg[e] - m) / ssum;
    } else {
      float ssum = 0.f;
      if (!a.raw)
        for (int jj = 0; jj < a.k; ++jj)
          if ((unsigned)oi[jj] < (unsigned)a.E) ssum += sigmoid_f(lg[oi[jj]]);
      g = sigmoid_f(lg[e]) / (a.raw ? 1.f : ssum);
    }
    a.gate[aid] = g;
  }
  a.slot_of[aid] = ns;
  if (ns >= 0) a.perm[ns] = (int32_t)aid;
  if (aid >= a.offsets[a.E]) a.perm[aid] = -1;
}

// The moved slots' new experts, after every gate was computed from the
// original choice.
__global__ void reassign_commit_kernel(ReassignArgs a) {
  const long long tk = (long long)a.T * a.k;
  const long long aid = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (aid < tk && a.rslot[aid] >= 0) a.idx[aid] = a.newe[aid];
}

__global__ void fill_zero32_kernel(uint32_t* p, long long n) {
  long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

}  // namespace

hipError_t launch_dispatch(const DispatchArgs& a, hipStream_t s) {
  const long long tk = (long long)a.T * a.k;
  const int nchunks = dispatch_chunks(tk);
  if (tk <= 64 && a.E <= 64) {
    dispatch_wave_kernel<<<1, 64, 0, s>>>(a);
    return hipGetLastError();
  }
  if (nchunks <= DW) {
    dispatch_small_kernel<<<1, 256, 0, s>>>(a, nchunks);
    return hipGetLastError();
  }
  const int blocks = (nchunks + DW - 1) / DW;
  dispatch_count_kernel<<<blocks, DW * 64, 0, s>>>(a.idx, tk, nchunks, a.E,
                                                   a.chunk_ws);
  dispatch_scan_kernel<<<1, SCAN_THREADS, 0, s>>>(a, nchunks);
  dispatch_scatter_kernel<<<blocks, DW * 64, 0, s>>>(a, nchunks);
  return hipGetLastError();
}

hipError_t launch_reassign(const ReassignArgs& a, hipStream_t s) {
  const long long tk = (long long)a.T * a.k;
  if (tk == 0) return hipSuccess;
#define MOE_REASSIGN(C)                                              \
  do {                                                               \
    if (a.k == 1) reassign_kernel<C, 1><<<1, 64, 0, s>>>(a);         \
    else if (a.k == 2) reassign_kernel<C, 2><<<1, 64, 0, s>>>(a);    \
    else if (a.k <= 4) reassign_kernel<C, 4><<<1, 64, 0, s>>>(a);    \
    else reassign_kernel<C, 8><<<1, 64, 0, s>>>(a);                  \
  } while (0)
  // k = 1 within the LDS bounds: the parallel decode (draws are at most
  // min(T, E * capacity); positions and draw ids fit 16 bits)
  const long long slots = (long long)a.E * a.capacity;
  if (a.k == 1 && a.E <= RP_MAXE && slots <= 65536 &&
      (tk < slots ? tk : slots) <= RP_MAXP) {
    if (a.E <= 64) reassign_k1_kernel<1><<<1, RP_THREADS, 0, s>>>(a);
    else if (a.E <= 128) reassign_k1_kernel<2><<<1, RP_THREADS, 0, s>>>(a);
    else if (a.E <= 256) reassign_k1_kernel<4><<<1, RP_THREADS, 0, s>>>(a);
    else reassign_k1_kernel<8><<<1, RP_THREADS, 0, s>>>(a);
  } else if (a.E <= 64) MOE_REASSIGN(1);
  else if (a.E <= 128) MOE_REASSIGN(2);
  else MOE_REASSIGN(4);
#undef MOE_REASSIGN
  const unsigned blocks = (unsigned)((tk + 255) / 256);
  reassign_rebuild_kernel<<<blocks, 256, 0, s>>>(a);
  reassign_commit_kernel<<<blocks, 256, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_fill_zero32(void* p, long long n, hipStream_t s) {
  if (n <= 0) return hipSuccess;
  const int bs = 256;
  fill_zero32_kernel<<<(unsigned)((n + bs - 1) / bs), bs, 0, s>>>((uint32_t*)p, n);
  return hipGetLastError();
}

}  // namespace moe
