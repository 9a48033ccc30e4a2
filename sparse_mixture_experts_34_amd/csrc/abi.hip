// C ABI of the MoE layer: argument validation, workspace layout, launches.
// Every entry point validates everything on the host before enqueuing the
// first kernel, so an error status means nothing was enqueued.
#include <math.h>
#include <string.h>

#include <mutex>

#include <hip/hip_runtime.h>

#include "../../include/moe.h"
#include "kernels.hpp"

namespace moe {
int ffn_schedule(int dtype, int T, int k, int E);
}

namespace {

using namespace moe;

constexpr size_t ALIGN = 256;

size_t align_up(size_t v) { return (v + ALIGN - 1) / ALIGN * ALIGN; }

struct Layout {
  int ksplit;
  int nrb;       // route blocks
  int nchunks;   // dispatch chunks
  size_t part, idx, gate, rpart, pmean, chunk, counts, offsets, perm, slot,
      ndrop, aux, h, y, logits, off0, rslot, newe, split_part, split_cnt,
      total;
  int split_cpx;   // CUs per XCD the split area holds (0: none)
};

// split: whether the tiled expert GEMMs get the K-split area (the no-alloc
// entry point's layout has none; its tiled GEMMs then never split).
Layout make_layout(const moe_problem& p, bool split = true) {
  Layout L;
  const long long T = p.T, E = p.n_experts, k = p.top_k;
  const long long rows = T * k + (long long)p.n_shared * T;
  const size_t esz = p.dtype == MOE_DTYPE_BF16 ? 2 : 4;
  L.ksplit = router_ksplit(p.T, p.d_model, p.n_experts, p.dtype);
  L.nrb = route_partial_rows(p.T, p.n_experts);
  L.nchunks = dispatch_chunks(T * k);
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off = align_up(off + (bytes ? bytes : 1));
    return o;
  };
  L.part = take((size_t)L.ksplit * T * E * 4);
  L.idx = take((size_t)T * k * 4);
  L.gate = take((size_t)T * k * 4);
  L.rpart = take((size_t)L.nrb * E * 4);
  L.pmean = take((size_t)E * 4);
  L.chunk = take((size_t)L.nchunks * E * 4);
  L.counts = take((size_t)E * 4);
  L.offsets = take((size_t)(E + 1) * 4);
  L.perm = take((size_t)T * k * 4);
  L.slot = take((size_t)T * k * 4);
  L.ndrop = take(4);
  L.aux = take(4);
  L.h = take((size_t)rows * p.d_ff * esz);
  L.y = take((size_t)rows * p.d_model * esz);
  // overflow reassignment: router logits, the cut's offsets, moved ranks
  const bool re = p.overflow == MOE_OVERFLOW_REASSIGN;
  L.logits = take(re ? (size_t)T * E * 4 : 0);
  L.off0 = take(re ? (size_t)(E + 1) * 4 : 0);
  L.rslot = take(re ? (size_t)T * k * 4 : 0);
  L.newe = take(re ? (size_t)T * k * 4 : 0);
  // tiled expert GEMMs (bf16 weights): one partial tile and one counter
  // per CU for the K-split last round
  const int sched = ffn_schedule(p.dtype, p.T, p.top_k, p.n_experts);
  L.split_cpx = (split && p.wquant != MOE_WQUANT_INT4 && sched == 1)
                    ? device_cus() / 8 : 0;
  L.split_part = take((size_t)8 * L.split_cpx * SPLIT_TILE_FLOATS * 4);
  L.split_cnt = take((size_t)8 * L.split_cpx * 4);
  L.total = off;
  return L;
}

int32_t check_problem(const moe_problem* p) {
  if (!p) return MOE_EINVAL;
  if (p->T < 0 || p->n_experts < 1 || p->n_experts > MOE_MAX_EXPERTS)
    return MOE_EINVAL;
  if (p->top_k < 1 || p->top_k > p->n_experts) return MOE_EINVAL;
  if (p->top_k > MOE_MAX_TOP_K) return MOE_ENOTSUP;
  if (p->d_model <= 0 || p->d_ff <= 0) return MOE_EINVAL;
  if (p->d_model % 64 != 0 || p->d_ff % 64 != 0) return MOE_ENOTSUP;
  if (p->n_shared != 0 && p->n_shared != 1) return MOE_EINVAL;
  if (p->act != MOE_ACT_GELU && p->act != MOE_ACT_SWIGLU) return MOE_EINVAL;
  if (p->dtype != MOE_DTYPE_F32 && p->dtype != MOE_DTYPE_BF16)
    return MOE_EINVAL;
  if (!isfinite(p->aux_coef)) return MOE_EINVAL;
  if (p->wquant != MOE_WQUANT_NONE && p->wquant != MOE_WQUANT_INT4 &&
      p->wquant != MOE_WQUANT_BF16_TILED)
    return MOE_EINVAL;
  if (p->wquant == MOE_WQUANT_BF16_TILED && p->dtype != MOE_DTYPE_BF16)
    return MOE_ENOTSUP;
  if (p->scoring != MOE_SCORING_SOFTMAX && p->scoring != MOE_SCORING_SIGMOID)
    return MOE_EINVAL;
  if (p->raw_gates != 0 && p->raw_gates != 1) return MOE_EINVAL;
  if (p->overflow != MOE_OVERFLOW_DROP && p->overflow != MOE_OVERFLOW_REASSIGN)
    return MOE_EINVAL;
  if (p->wquant == MOE_WQUANT_INT4 &&
      (p->dtype != MOE_DTYPE_BF16 || p->d_model % MOE_Q4_GROUP != 0 ||
       p->d_ff % MOE_Q4_GROUP != 0))
    return MOE_ENOTSUP;
  const long long rows = (long long)p->T * p->top_k + (long long)p->n_shared * p->T;
  if (rows >= (1LL << 31)) return MOE_ENOTSUP;
  // the GEMMs address a row-major activation matrix and one expert's
  // weight matrix with 32-bit element offsets
  const long long wide = p->d_model > p->d_ff ? p->d_model : p->d_ff;
  if ((rows + p->T) * wide >= (1LL << 32) ||
      (long long)p->d_model * p->d_ff >= (1LL << 32))
    return MOE_ENOTSUP;
  // (this also keeps x under 2^32 bytes, 2*T*d <= (T*k + T)*d, so the
  // 256-row GEMM tiles can gather its rows with 32-bit byte offsets)
  return MOE_OK;
}

int32_t check_ws(const moe_problem* p, const void* ws, size_t ws_bytes) {
  const Layout L = make_layout(*p);
  if (ws_bytes < L.total) return MOE_EWORKSPACE;
  if (!ws && L.total) return MOE_EINVAL;
  if (((uintptr_t)ws) % ALIGN) return MOE_EINVAL;
  return MOE_OK;
}

int32_t check_weights(const moe_problem* p, const moe_expert_weights* w) {
  if (!w) return MOE_EINVAL;
  if (p->act == MOE_ACT_SWIGLU) {
    if (!w->w1 || !w->w_up || !w->w2) return MOE_EINVAL;
    if (w->b1 || w->b2) return MOE_EINVAL;
    if (p->n_shared &&
        (!w->shared_w1 || !w->shared_w_up || !w->shared_w2 || w->shared_b1 ||
         w->shared_b2))
      return MOE_EINVAL;
  } else {
    if (!w->w1 || !w->w2 || !w->b1 || !w->b2) return MOE_EINVAL;
    if (w->w_up) return MOE_EINVAL;
    if (p->n_shared && (!w->shared_w1 || !w->shared_w2 || !w->shared_b1 ||
                        !w->shared_b2 || w->shared_w_up))
      return MOE_EINVAL;
  }
  if (p->wquant == MOE_WQUANT_INT4) {
    // every quantised matrix needs its (scale, offset) pairs
    if (!w->w1_q || !w->w2_q) return MOE_EINVAL;
    if (p->act == MOE_ACT_SWIGLU && !w->w_up_q) return MOE_EINVAL;
    if (p->n_shared) {
      if (!w->shared_w1_q || !w->shared_w2_q) return MOE_EINVAL;
      if (p->act == MOE_ACT_SWIGLU && !w->shared_w_up_q) return MOE_EINVAL;
    }
  }
  return MOE_OK;
}

int32_t status_of(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_EHIP; }

// Step 1 for T > 0: the fused kernel for small batches with few experts,
// otherwise the router GEMM (K-split partial logits in `part`) and the
// select kernel.  Writes rpart, the route_partial_rows(T, E) rows of
// probability partials.
hipError_t route_on(const moe_problem* p, const void* x, const float* w_router,
                    const float* router_bias, const float* select_bias,
                    float* logits, int32_t* idx, float* gate, float* part,
                    float* rpart, int ksplit, hipStream_t stream) {
  if (route_fused(p->T, p->n_experts))
    return launch_route_fused(p->dtype, x, w_router, router_bias,
                              select_bias, logits, idx, gate, rpart, p->T,
                              p->d_model, p->n_experts, p->top_k, p->scoring,
                              p->raw_gates, stream);
  hipError_t e = launch_router_logits_partial(p->dtype, x, w_router, part,
                                              p->T, p->d_model, p->n_experts,
                                              ksplit, stream);
  if (e != hipSuccess) return e;
  return launch_route_select_from(part, ksplit, router_bias, select_bias,
                                  logits, idx, gate, rpart, p->T,
                                  p->n_experts, p->top_k, p->scoring,
                                  p->raw_gates, stream);
}

#define MOE_TRY(expr)                                    \
  do {                                                   \
    hipError_t e_ = (expr);                              \
    if (e_ != hipSuccess) return status_of(e_);          \
  } while (0)

FfnArgs ffn_args(const moe_problem* p, const void* x, const int32_t* perm,
                 const int32_t* offsets, const moe_expert_weights* w, void* h,
                 void* y) {
  FfnArgs a;
  a.dtype = p->dtype;
  a.act = p->act;
  a.T = p->T;
  a.d = p->d_model;
  a.E = p->n_experts;
  a.k = p->top_k;
  a.d_ff = p->d_ff;
  a.n_shared = p->n_shared;
  a.x = x;
  a.perm = perm;
  a.offsets = offsets;
  a.w1 = w->w1;
  a.w_up = w->w_up;
  a.w2 = w->w2;
  a.b1 = w->b1;
  a.b2 = w->b2;
  a.sw1 = w->shared_w1;
  a.sw_up = w->shared_w_up;
  a.sw2 = w->shared_w2;
  a.sb1 = w->shared_b1;
  a.sb2 = w->shared_b2;
  a.wquant = p->wquant;
  a.w1q = w->w1_q;
  a.w_upq = w->w_up_q;
  a.w2q = w->w2_q;
  a.sw1q = w->shared_w1_q;
  a.sw_upq = w->shared_w_up_q;
  a.sw2q = w->shared_w2_q;
  a.h = h;
  a.y = y;
  a.split_part = nullptr;
  a.split_cnt = nullptr;
  a.split_cpx = 0;
  return a;
}

// The K-split area of the workspace, when the layout has one.
void with_split(FfnArgs& a, const Layout& L, char* ws) {
  if (L.split_cpx > 0) {
    a.split_part = (float*)(ws + L.split_part);
    a.split_cnt = (int32_t*)(ws + L.split_cnt);
    a.split_cpx = L.split_cpx;
  }
}

}  // namespace

namespace {

ReassignArgs reassign_args(const moe_problem* p, int32_t* idx, float* gate,
                           const float* logits, const int32_t* off0,
                           int32_t* offsets, int32_t* perm, int32_t* slot_of,
                           int32_t* n_dropped, int32_t* rslot,
                           int32_t* newe) {
  ReassignArgs r;
  r.idx = idx;
  r.gate = gate;
  r.logits = logits;
  r.off0 = off0;
  r.offsets = offsets;
  r.perm = perm;
  r.slot_of = slot_of;
  r.n_dropped = n_dropped;
  r.rslot = rslot;
  r.newe = newe;
  r.T = p->T;
  r.E = p->n_experts;
  r.k = p->top_k;
  r.capacity = p->capacity;
  r.scoring = p->scoring;
  r.raw = p->raw_gates;
  r.key0 = (uint32_t)(p->overflow_seed & 0xFFFFFFFFu);
  r.key1 = (uint32_t)(p->overflow_seed >> 32);
  return r;
}

// Scratch of moe_layer_forward_noalloc: the workspace of that entry point,
// a device global of the library's code object, so each GPU the library
// runs on holds its own copy until the process ends.  Host code never
// uses the name as an address (on the host it is only a stand-in for the
// symbol); the device address comes from hipGetSymbolAddress, looked up
// once per device with that device current, and is what kernels receive.
static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
char* g_scratch_ptr[MAX_DEVICES];   // scratch's address on each device

int32_t scratch_of_current_device(char** out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return MOE_EHIP;
  if (dev < 0 || dev >= MAX_DEVICES) return MOE_ENOTSUP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr)
      return MOE_EHIP;
    g_scratch_ptr[dev] = (char*)ptr;
  }
  *out = g_scratch_ptr[dev];
  return MOE_OK;
}

// Steps 1-5 of the layer, enqueued with the workspace wsb laid out as L.
// Arguments are validated by the callers.
int32_t layer_forward_in(const moe_problem* p, const void* x,
                         const float* w_router, const float* router_bias,
                         const float* select_bias,
                         const moe_expert_weights* w, void* out,
                         float* aux_loss, int32_t* counts, int32_t* n_dropped,
                         int32_t* topk_idx, char* wsb, const Layout& L,
                         hipStream_t stream) {
  if (p->T == 0) {
    if (aux_loss) MOE_TRY(launch_fill_zero32(aux_loss, 1, stream));
    if (counts) MOE_TRY(launch_fill_zero32(counts, p->n_experts, stream));
    if (n_dropped) MOE_TRY(launch_fill_zero32(n_dropped, 1, stream));
    return MOE_OK;
  }
  int32_t* idx = topk_idx ? topk_idx : (int32_t*)(wsb + L.idx);
  float* gate = (float*)(wsb + L.gate);
  float* part = (float*)(wsb + L.part);
  float* rpart = (float*)(wsb + L.rpart);
  const bool reassign =
      p->overflow == MOE_OVERFLOW_REASSIGN && p->capacity > 0;
  float* logits = reassign ? (float*)(wsb + L.logits) : nullptr;
  MOE_TRY(route_on(p, x, w_router, router_bias, select_bias, logits, idx,
                   gate, part, rpart, L.ksplit, stream));
  DispatchArgs a;
  a.idx = idx;
  a.prob_mean_in = nullptr;
  a.partials = rpart;
  a.n_partials = L.nrb;
  a.prob_mean_out = (float*)(wsb + L.pmean);
  a.counts = counts ? counts : (int32_t*)(wsb + L.counts);
  a.offsets = (int32_t*)(wsb + L.offsets);
  a.perm = (int32_t*)(wsb + L.perm);
  a.slot_of = (int32_t*)(wsb + L.slot);
  a.n_dropped = n_dropped ? n_dropped : (int32_t*)(wsb + L.ndrop);
  a.aux = aux_loss ? aux_loss : (float*)(wsb + L.aux);
  a.chunk_ws = (int32_t*)(wsb + L.chunk);
  a.T = p->T;
  a.E = p->n_experts;
  a.k = p->top_k;
  a.capacity = p->capacity;
  a.aux_coef = p->aux_coef;
  if (reassign) a.offsets = (int32_t*)(wsb + L.off0);
  MOE_TRY(launch_dispatch(a, stream));
  if (reassign) {
    a.offsets = (int32_t*)(wsb + L.offsets);
    MOE_TRY(launch_reassign(
        reassign_args(p, idx, gate, logits, (int32_t*)(wsb + L.off0),
                      a.offsets, a.perm, a.slot_of, a.n_dropped,
                      (int32_t*)(wsb + L.rslot), (int32_t*)(wsb + L.newe)),
        stream));
  }
  void* y = wsb + L.y;
  FfnArgs f = ffn_args(p, x, a.perm, a.offsets, w, wsb + L.h, y);
  with_split(f, L, wsb);
  MOE_TRY(launch_expert_up(f, stream));
  MOE_TRY(launch_expert_down(f, stream));
  MOE_TRY(launch_combine(p->dtype, x, y, a.slot_of, gate, out, p->T,
                         p->d_model, p->top_k, p->n_shared, stream));
  return MOE_OK;
}

}  // namespace

extern "C" {

int32_t moe_capacity(int32_t T, int32_t top_k, int32_t n_experts,
                     int32_t cf_num, int32_t cf_den) {
  if (T < 0 || top_k < 1 || n_experts < 1 || cf_num <= 0 || cf_den <= 0)
    return -1;
  const long long num = (long long)cf_num * T * top_k;
  const long long den = (long long)cf_den * n_experts;
  const long long c = num / den;
  if (c >= (1LL << 31)) return -1;
  return c < 1 ? 1 : (int32_t)c;
}

int32_t moe_workspace_bytes(const moe_problem* p, size_t* bytes) {
  int32_t st = check_problem(p);
  if (st) return st;
  if (!bytes) return MOE_EINVAL;
  *bytes = make_layout(*p).total;
  return MOE_OK;
}

int32_t moe_route(const moe_problem* p, const void* x, const float* w_router,
                  const float* router_bias, const float* select_bias,
                  float* logits, int32_t* topk_idx, float* topk_gate,
                  float* prob_mean, void* ws, size_t ws_bytes,
                  hipStream_t stream) {
  int32_t st = check_problem(p);
  if (st) return st;
  if (!prob_mean) return MOE_EINVAL;
  if (p->T > 0 && (!x || !w_router || !topk_idx || !topk_gate))
    return MOE_EINVAL;
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if (p->T == 0) return status_of(launch_fill_zero32(prob_mean, p->n_experts, stream));
  const Layout L = make_layout(*p);
  char* w = (char*)ws;
  float* part = (float*)(w + L.part);
  float* rpart = (float*)(w + L.rpart);
  MOE_TRY(route_on(p, x, w_router, router_bias, select_bias, logits,
                   topk_idx, topk_gate, part, rpart, L.ksplit, stream));
  MOE_TRY(launch_prob_mean(rpart, prob_mean, L.nrb, p->T, p->n_experts,
                           stream));
  return MOE_OK;
}

int32_t moe_dispatch(const moe_problem* p, const int32_t* topk_idx,
                     const float* prob_mean, int32_t* counts,
                     int32_t* offsets, int32_t* perm, int32_t* slot_of,
                     int32_t* n_dropped, float* aux_loss, void* ws,
                     size_t ws_bytes, hipStream_t stream) {
  int32_t st = check_problem(p);
  if (st) return st;
  // reassignment needs the gates and logits: moe_dispatch_reassign
  if (p->overflow != MOE_OVERFLOW_DROP) return MOE_EINVAL;
  if (!counts || !offsets || !n_dropped) return MOE_EINVAL;
  if (p->T > 0 && (!topk_idx || !perm || !slot_of)) return MOE_EINVAL;
  if (aux_loss && !prob_mean) return MOE_EINVAL;
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if (p->T == 0) {
    MOE_TRY(launch_fill_zero32(counts, p->n_experts, stream));
    MOE_TRY(launch_fill_zero32(offsets, p->n_experts + 1, stream));
    MOE_TRY(launch_fill_zero32(n_dropped, 1, stream));
    if (aux_loss) MOE_TRY(launch_fill_zero32(aux_loss, 1, stream));
    return MOE_OK;
  }
  const Layout L = make_layout(*p);
  DispatchArgs a;
  a.idx = topk_idx;
  a.prob_mean_in = prob_mean;
  a.partials = nullptr;
  a.n_partials = 0;
  a.prob_mean_out = nullptr;
  a.counts = counts;
  a.offsets = offsets;
  a.perm = perm;
  a.slot_of = slot_of;
  a.n_dropped = n_dropped;
  a.aux = aux_loss;
  a.chunk_ws = (int32_t*)((char*)ws + L.chunk);
  a.T = p->T;
  a.E = p->n_experts;
  a.k = p->top_k;
  a.capacity = p->capacity;
  a.aux_coef = p->aux_coef;
  return status_of(launch_dispatch(a, stream));
}


int32_t moe_dispatch_reassign(const moe_problem* p, int32_t* topk_idx,
                              float* topk_gate, const float* logits,
                              const float* prob_mean, int32_t* counts,
                              int32_t* offsets, int32_t* perm,
                              int32_t* slot_of, int32_t* n_dropped,
                              float* aux_loss, void* ws, size_t ws_bytes,
                              hipStream_t stream) {
  int32_t st = check_problem(p);
  if (st) return st;
  if (p->overflow != MOE_OVERFLOW_REASSIGN) return MOE_EINVAL;
  if (!counts || !offsets || !n_dropped) return MOE_EINVAL;
  if (p->T > 0 && (!topk_idx || !topk_gate || !logits || !perm || !slot_of))
    return MOE_EINVAL;
  if (aux_loss && !prob_mean) return MOE_EINVAL;
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if (p->T == 0) {
    MOE_TRY(launch_fill_zero32(counts, p->n_experts, stream));
    MOE_TRY(launch_fill_zero32(offsets, p->n_experts + 1, stream));
    MOE_TRY(launch_fill_zero32(n_dropped, 1, stream));
    if (aux_loss) MOE_TRY(launch_fill_zero32(aux_loss, 1, stream));
    return MOE_OK;
  }
  const Layout L = make_layout(*p);
  char* wsb = (char*)ws;
  const bool cut = p->capacity > 0;
  int32_t* off0 = cut ? (int32_t*)(wsb + L.off0) : offsets;
  DispatchArgs a;
  a.idx = topk_idx;
  a.prob_mean_in = prob_mean;
  a.partials = nullptr;
  a.n_partials = 0;
  a.prob_mean_out = nullptr;
  a.counts = counts;
  a.offsets = off0;
  a.perm = perm;
  a.slot_of = slot_of;
  a.n_dropped = n_dropped;
  a.aux = aux_loss;
  a.chunk_ws = (int32_t*)(wsb + L.chunk);
  a.T = p->T;
  a.E = p->n_experts;
  a.k = p->top_k;
  a.capacity = p->capacity;
  a.aux_coef = p->aux_coef;
  MOE_TRY(launch_dispatch(a, stream));
  if (cut)
    MOE_TRY(launch_reassign(
        reassign_args(p, topk_idx, topk_gate, logits, off0, offsets, perm,
                      slot_of, n_dropped, (int32_t*)(wsb + L.rslot),
                      (int32_t*)(wsb + L.newe)),
        stream));
  return MOE_OK;
}

int32_t moe_expert_ffn(const moe_problem* p, const void* x,
                       const int32_t* perm, const int32_t* offsets,
                       const moe_expert_weights* w, void* y, void* ws,
                       size_t ws_bytes, hipStream_t stream) {
  int32_t st = check_problem(p);
  if (st) return st;
  if ((st = check_weights(p, w))) return st;
  if (p->T > 0 && (!x || !perm || !offsets || !y)) return MOE_EINVAL;
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  if (p->T == 0) return MOE_OK;
  const Layout L = make_layout(*p);
  FfnArgs a = ffn_args(p, x, perm, offsets, w, (char*)ws + L.h, y);
  with_split(a, L, (char*)ws);
  MOE_TRY(launch_expert_up(a, stream));
  return status_of(launch_expert_down(a, stream));
}

int32_t moe_expert_up(const moe_problem* p, const void* x,
                      const int32_t* perm, const int32_t* offsets,
                      const moe_expert_weights* w, void* h, void* ws,
                      size_t ws_bytes, hipStream_t stream) {
  int32_t st = check_problem(p);
  if (st) return st;
  if ((st = check_weights(p, w))) return st;
  if (p->T > 0 && (!x || !perm || !offsets || !h)) return MOE_EINVAL;
  if (ws && (st = check_ws(p, ws, ws_bytes))) return st;
  if (p->T == 0) return MOE_OK;
  FfnArgs a = ffn_args(p, x, perm, offsets, w, h, nullptr);
  if (ws) with_split(a, make_layout(*p), (char*)ws);
  return status_of(launch_expert_up(a, stream));
}

int32_t moe_expert_down(const moe_problem* p, const void* h,
                        const int32_t* offsets, const moe_expert_weights* w,
                        void* y, void* ws, size_t ws_bytes,
                        hipStream_t stream) {
  int32_t st = check_problem(p);
  if (st) return st;
  if ((st = check_weights(p, w))) return st;
  if (p->T > 0 && (!h || !offsets || !y)) return MOE_EINVAL;
  if (ws && (st = check_ws(p, ws, ws_bytes))) return st;
  if (p->T == 0) return MOE_OK;
  FfnArgs a = ffn_args(p, nullptr, nullptr, offsets, w, (void*)h, y);
  if (ws) with_split(a, make_layout(*p), (char*)ws);
  return status_of(launch_expert_down(a, stream));
}

int32_t moe_combine(const moe_problem* p, const void* x_residual,
                    const void* y, const int32_t* slot_of,
                    const float* topk_gate, void* out, hipStream_t stream) {
  int32_t st = check_problem(p);
  if (st) return st;
  if (p->T > 0 && (!y || !slot_of || !topk_gate || !out)) return MOE_EINVAL;
  if (p->T == 0) return MOE_OK;
  return status_of(launch_combine(p->dtype, x_residual, y, slot_of, topk_gate,
                                  out, p->T, p->d_model, p->top_k,
                                  p->n_shared, stream));
}

int32_t moe_layer_forward(const moe_problem* p, const void* x,
                          const float* w_router, const float* router_bias,
                          const float* select_bias,
                          const moe_expert_weights* w, void* out,
                          float* aux_loss, int32_t* counts,
                          int32_t* n_dropped, int32_t* topk_idx, void* ws,
                          size_t ws_bytes, hipStream_t stream) {
  int32_t st = check_problem(p);
  if (st) return st;
  if ((st = check_weights(p, w))) return st;
  if (p->T > 0 && (!x || !w_router || !out)) return MOE_EINVAL;
  if ((st = check_ws(p, ws, ws_bytes))) return st;
  return layer_forward_in(p, x, w_router, router_bias, select_bias, w, out,
                          aux_loss, counts, n_dropped, topk_idx, (char*)ws,
                          make_layout(*p), stream);
}

int32_t moe_layer_forward_noalloc(const moe_problem* p, const void* x,
                                  const float* w_router,
                                  const float* router_bias,
                                  const float* select_bias,
                                  const moe_expert_weights* w, void* out,
                                  float* aux_loss, int32_t* counts,
                                  int32_t* n_dropped, int32_t* topk_idx,
                                  hipStream_t stream) {
  int32_t st = check_problem(p);
  if (st) return st;
  if ((st = check_weights(p, w))) return st;
  if (p->T > 0 && (!x || !w_router || !out)) return MOE_EINVAL;
  const Layout L = make_layout(*p, false);
  if (L.total > (size_t)MOE_NOALLOC_SCRATCH_BYTES) return MOE_EWORKSPACE;
  char* sp = nullptr;
  if ((st = scratch_of_current_device(&sp))) return st;
  return layer_forward_in(p, x, w_router, router_bias, select_bias, w, out,
                          aux_loss, counts, n_dropped, topk_idx, sp, L,
                          stream);
}

int32_t moe_quantize_int4(const void* w, int64_t rows, int32_t K,
                          void* codes, float* qparams, hipStream_t stream) {
  if (rows < 0) return MOE_EINVAL;
  if (K <= 0 || K % MOE_Q4_GROUP != 0 || rows % 16 != 0) return MOE_ENOTSUP;
  if (rows > 0 && (!w || !codes || !qparams)) return MOE_EINVAL;
  // one thread per code word: the grid (rows * K / 8 threads) must fit the
  // 32-bit dispatch size
  if ((long long)rows * (K / 8) >= (1LL << 32) - 256) return MOE_ENOTSUP;
  return status_of(launch_quantize_int4(w, rows, K, codes, qparams, stream));
}

int32_t moe_tile_bf16(const void* w, int64_t rows, int32_t K, void* out,
                      hipStream_t stream) {
  if (rows < 0) return MOE_EINVAL;
  if (K <= 0 || K % 32 != 0 || rows % 16 != 0) return MOE_ENOTSUP;
  if (rows > 0 && (!w || !out)) return MOE_EINVAL;
  // one thread per 16-byte piece: the grid must fit the 32-bit dispatch size
  if ((long long)rows * (K / 8) >= (1LL << 32) - 256) return MOE_ENOTSUP;
  return status_of(launch_tile_bf16(w, rows, K, out, stream));
}

int32_t moe_update_select_bias(const moe_problem* p, const int32_t* counts,
                               float* select_bias, float gamma,
                               hipStream_t stream) {
  int32_t st = check_problem(p);
  if (st) return st;
  if (!counts || !select_bias || !isfinite(gamma)) return MOE_EINVAL;
  return status_of(launch_update_select_bias(counts, select_bias, gamma,
                                             p->n_experts, stream));
}

const char* moe_status_string(int32_t status) {
  switch (status) {
    case MOE_OK: return "MOE_OK: success";
    case MOE_EINVAL: return "MOE_EINVAL: invalid argument";
    case MOE_ENOTSUP: return "MOE_ENOTSUP: shape or type not supported";
    case MOE_EWORKSPACE: return "MOE_EWORKSPACE: workspace too small";
    case MOE_EHIP: return "MOE_EHIP: kernel launch failed";
    default: return "unknown MoE status";
  }
}

}  // extern "C"
