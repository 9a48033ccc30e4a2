"""Plain fp64 CPU statement of the sparse MoE layer forward pass.

TEST INFRASTRUCTURE ONLY: see the package docstring.  Written for a reader
who checks it against the pages by eye; nothing here is blocked, fused or
reordered beyond the pages' own per-expert grouping, and every function cites
the passage it follows.  Page tags ([RC], [LBS], [HA], [GN], [FA]) are
expanded in ``oracle/__init__.py``.

Conventions
-----------
* Inputs arrive as numpy arrays (bf16 tensors are handed over as the float32
  arrays holding the same values).  All arithmetic below is float64, except
  the router logits, which are rounded once to float32: [LBS] "Dense vs
  Sparse" states the router runs in float32 while the rest may be bfloat16,
  so the top-k decision is taken on float32 logits, as the GPU takes it.
* Stacked expert weights follow ``nn.Linear`` storage ([out, in], the input
  dimension contiguous) with a leading expert axis:
  GELU experts ``w1 [E,d_ff,d], b1 [E,d_ff], w2 [E,d,d_ff], b2 [E,d]``;
  SwiGLU experts ``w_gate, w_up [E,d_ff,d], w_down [E,d,d_ff]``;
  an always-on shared expert uses the same names with a ``shared_`` prefix
  and no expert axis.  Any object whose ``[e]`` gives an array works, so a
  caller may fetch one expert at a time.
* Assignment id ``a = t*k + j`` names slot ``j`` of token ``t`` ([LBS]
  "Gating Mechanism": the flattened expert ids, token = flat position // k).
"""

from __future__ import annotations

import math

import numpy as np
from scipy.special import erf as _erf

F64 = np.float64


# ---------------------------------------------------------------------------
# Scalars
# ---------------------------------------------------------------------------

def capacity(T: int, k: int, E: int, cf_num: int, cf_den: int) -> int:
    """Per-expert token capacity.

    [LBS] "The Capacity Factor": the ideal share is T*k/E assignments per
    expert; capacity is that share times the capacity factor, truncated to
    an integer, and never below 1.  The factor is taken as the exact
    rational cf_num/cf_den so that e.g. 1.1 cannot truncate to the wrong
    integer through a binary floating-point product.
    """
    if T < 0 or k < 1 or E < 1 or cf_num <= 0 or cf_den <= 0:
        raise ValueError("capacity: need T>=0, k>=1, E>=1, cf>0")
    return max((cf_num * T * k) // (cf_den * E), 1)


def gelu(z):
    """Exact (erf) GELU, z * Phi(z): the default ``nn.GELU`` inside the
    Linear-GELU-Linear expert of [RC] "How a sparse MoE layer works"."""
    z = np.asarray(z, F64)
    return 0.5 * z * (1.0 + _erf(z / math.sqrt(2.0)))


def silu(z):
    """SiLU, z * sigmoid(z), the gate nonlinearity of the SwiGLU expert in
    [GN] "Implementing a complete MoE layer"."""
    z = np.asarray(z, F64)
    with np.errstate(over="ignore"):
        return z / (1.0 + np.exp(-z))


def softmax(logits):
    """Row softmax over the expert axis ([RC], [LBS] "Gating Mechanism",
    [GN] "The router"); the row maximum is subtracted first."""
    l = np.asarray(logits, F64)
    if l.shape[-1] == 0:
        return l.copy()
    m = l.max(axis=-1, keepdims=True)
    e = np.exp(l - m)
    return e / e.sum(axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# Step 1: route
# ---------------------------------------------------------------------------

def sigmoid(z):
    """Logistic sigmoid 1 / (1 + e^-z), the per-expert scoring function
    ([FA] "The knobs": per-expert sigmoid scoring as the alternative to a
    softmax over all experts).  Float64."""
    z = np.asarray(z, F64)
    out = np.empty_like(z)
    pos = z >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-z[pos]))
    ez = np.exp(z[~pos])
    out[~pos] = ez / (1.0 + ez)
    return out


def _logits64(x, w_router, router_bias=None):
    l = np.asarray(x, F64) @ np.asarray(w_router, F64).T
    if router_bias is not None:
        l = l + np.asarray(router_bias, F64)
    return l


def route(x, w_router, k, router_bias=None, select_bias=None,
          scoring="softmax", renormalize=True):
    """Router linear, scoring, top-k and (renormalised) gates.

    * logits = x . W_r^T (+ router bias): one linear layer from the hidden
      state to E scores ([RC] "How a sparse MoE layer works"; [LBS]
      "Gating Mechanism" uses no bias; [GN] "The router").  Rounded once to
      float32, the router precision [LBS] "Dense vs Sparse" gives.
    * probs = softmax(logits) over all E experts.
    * The k experts with the largest key are chosen, in descending key
      order; equal keys go to the lower expert index.  The key is the
      float32 logit, plus (float32 add) a per-expert selection bias when
      one is given: [GN] "DeepSeek-V3" adds a per-expert bias to the
      routing scores to choose experts; here it moves the choice only, the
      gates and probs still come from the unbiased softmax.  Choosing on the
      logits is choosing on the probs, softmax being monotone.
    * gate[t, j] = probs[t, idx[t, j]] / sum over the k chosen probs
      ([RC]; [LBS] "Gating Mechanism"; [GN] "The router"; [FA] "Concept").

    Variants ([FA] "The knobs": scoring by a softmax over all experts or a
    per-expert sigmoid, and whether the chosen gates are renormalised to
    sum to 1):
    * ``scoring="sigmoid"``: scores = sigmoid(logits) per expert.  Without
      a selection bias the key is the logit (the same order, sigmoid being
      monotone); with one, the bias is added to the float32 score, the
      scale DeepSeek-V3's routing scores live on ([GN] "DeepSeek-V3").
      ``probs`` (the P of the aux loss) are each token's scores divided by
      their sum over all experts, so they sum to 1 as softmax probs do.
    * ``renormalize=False``: gate[t, j] is the chosen score itself
      (softmax prob or sigmoid score), not divided by the chosen sum.

    Returns a dict: logits (float32 [T,E]), keys (float32 [T,E]),
    idx (int64 [T,k]), gate (float64 [T,k]), probs (float64 [T,E]),
    scores (float64 [T,E]).
    """
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(w_router).shape[0]
    if not 1 <= k <= E:
        raise ValueError("route: need 1 <= k <= E")
    if scoring not in ("softmax", "sigmoid"):
        raise ValueError("route: scoring is softmax or sigmoid")
    logits = _logits64(x, w_router, router_bias).astype(np.float32)
    if scoring == "softmax":
        scores = softmax(logits)
        probs = scores
        keys = logits.copy()
        if select_bias is not None:
            keys = (keys + np.asarray(select_bias, np.float32)).astype(
                np.float32)
    else:
        scores = sigmoid(logits)
        probs = scores / scores.sum(axis=1, keepdims=True) if T else scores
        if select_bias is None:
            keys = logits.copy()
        else:
            keys = (scores.astype(np.float32) +
                    np.asarray(select_bias, np.float32)).astype(np.float32)
    idx = np.zeros((T, k), np.int64)
    for t in range(T):
        # sort by key descending, then by expert index ascending
        order = sorted(range(E), key=lambda e: (-float(keys[t, e]), e))
        idx[t] = order[:k]
    chosen = np.take_along_axis(scores, idx, axis=1)
    if renormalize and T:
        gate = chosen / chosen.sum(axis=1, keepdims=True)
    else:
        gate = chosen
    return {"logits": logits, "keys": keys, "idx": idx, "gate": gate,
            "probs": probs, "scores": scores}


def topk_margin(x, w_router, k, router_bias=None, select_bias=None,
                scoring="softmax"):
    """Smallest gap between consecutive sorted selection keys around the
    top-k boundary, per token, in float64 (no float32 rounding).

    For keys sorted descending, kappa_(1) >= kappa_(2) >= ..., the gaps
    kappa_(j) - kappa_(j+1) for j = 1..k (j = 1..k-1 when k = E) decide
    both the chosen set and the slot order; a token whose smallest gap is
    tiny can flip under float32 summation order.  Used only to build test
    inputs whose routing is unique at float32 resolution.
    """
    keys = _logits64(x, w_router, router_bias)
    if select_bias is not None:
        if scoring == "sigmoid":
            keys = sigmoid(keys)
        keys = keys + np.asarray(select_bias, F64)
    E = keys.shape[1]
    s = -np.sort(-keys, axis=1)
    last = min(k, E - 1)
    if last < 1:
        return np.full(keys.shape[0], np.inf)
    gaps = s[:, :last] - s[:, 1:last + 1]
    return gaps.min(axis=1)


# ---------------------------------------------------------------------------
# Step 2: dispatch (capacity cut, grouping by expert)
# ---------------------------------------------------------------------------

def dispatch(idx, E, cap):
    """Group assignments by expert under a per-expert capacity.

    The rule ([RC] "How a sparse MoE layer works", the capacity check; [LBS]
    "The Capacity Factor" and "Token Dropping and Overflow Handling",
    zero-output strategy): an expert accepts the assignments routed to it in
    ascending token order until it holds ``cap`` of them; the rest are
    dropped (their MoE output is zero and the residual carries the token).
    cap <= 0 means no limit.

    Stated here as ranks: visiting the assignments a = t*k + j in ascending
    a (so ascending token, a token's k experts being distinct), the rank of
    a is the number of earlier assignments to the same expert; a is kept
    iff its rank is below ``cap``.  Kept assignments of expert e occupy
    rows offsets[e] + rank of the grouped batch, offsets being the
    exclusive scan of the per-expert kept counts.

    Returns counts[E] (assignments routed, before the cut), kept[E],
    offsets[E+1], perm[offsets[E]] (assignment id held by each grouped row),
    slot_of[T*k] (grouped row of each assignment, -1 if dropped) and
    n_dropped.
    """
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    expert_of = idx.reshape(-1)
    counts = np.zeros(E, np.int64)
    rank = np.zeros(T * k, np.int64)
    for a in range(T * k):
        e = int(expert_of[a])
        rank[a] = counts[e]
        counts[e] += 1
    keep = rank >= 0 if cap <= 0 else rank < cap
    kept = counts.copy() if cap <= 0 else np.minimum(counts, cap)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    slot_of = np.full(T * k, -1, np.int64)
    slot_of[keep] = offsets[expert_of[keep]] + rank[keep]
    perm = np.zeros(int(offsets[E]), np.int64)
    perm[slot_of[keep]] = np.nonzero(keep)[0]
    n_dropped = int(T * k - offsets[E])
    return {"counts": counts, "kept": kept, "offsets": offsets,
            "perm": perm, "slot_of": slot_of, "n_dropped": n_dropped}


# ---------------------------------------------------------------------------
# Overflow by random reassignment
# ---------------------------------------------------------------------------

_PHILOX_M = (0xD2511F53, 0xCD9E8D57)
_PHILOX_W = (0x9E3779B9, 0xBB67AE85)
_U32 = 0xFFFFFFFF


def philox4x32(ctr, key, rounds=10):
    """The Philox4x32-10 counter-based generator (Salmon, Moraes, Dror and
    Shaw, "Parallel Random Numbers: As Easy as 1, 2, 3", SC 2011): a round
    multiplies words 0 and 2 of the 128-bit counter by two fixed 32-bit
    multipliers and mixes the high and low halves of the products with
    words 1 and 3 and the 64-bit key; the key advances by two Weyl
    constants between rounds.  Returns the four 32-bit output words."""
    c = [int(v) & _U32 for v in ctr]
    k = [int(v) & _U32 for v in key]
    for r in range(rounds):
        if r:
            k = [(k[0] + _PHILOX_W[0]) & _U32, (k[1] + _PHILOX_W[1]) & _U32]
        p0 = _PHILOX_M[0] * c[0]
        p1 = _PHILOX_M[1] * c[2]
        c = [(p1 >> 32) ^ c[1] ^ k[0], p1 & _U32,
             (p0 >> 32) ^ c[3] ^ k[1], p0 & _U32]
    return c


def _reassign_candidates(spare, mine):
    """Experts with a free slot that the token does not already use, in
    ascending index."""
    return [e for e in range(len(spare)) if spare[e] > 0 and e not in mine]


def _pick_slot(x, cand, spare):
    """The expert holding free slot r = floor(x * total / 2^32) when the
    candidates' free slots are laid out in ascending expert order."""
    r = (x * sum(spare[e] for e in cand)) >> 32
    for e in cand:
        if r < spare[e]:
            return e
        r -= spare[e]
    raise AssertionError("unreachable: r < total")


def _reassigned_gate(scores_t, orig_idx_t, e, renormalize):
    """The new expert's score under the token's own normaliser."""
    norm = scores_t[orig_idx_t].sum() if renormalize else 1.0
    return scores_t[e] / norm


def dispatch_reassign(idx, scores, gate, E, cap, seed, renormalize=True):
    """Capacity dispatch with overflow reassigned at random ([LBS] "Token
    Dropping and Overflow Handling", random reassignment: an overflow token
    goes to a randomly chosen expert slot that still has room, weighted by
    that expert's router probability).

    Plain reading of the steps the page leaves open:
    * first the capacity cut of :func:`dispatch` (first ``cap`` per expert
      in token order kept); spare[e] = cap - kept[e];
    * the dropped assignments a = t*k + j are visited in ascending a; each
      draws one 32-bit word x = philox4x32((a, 0, 0, 0), (seed low 32 bits,
      seed high 32 bits))[0] and picks a free slot uniformly: with the
      candidate experts (spare > 0 and not already one of token t's
      experts) in ascending index, r = floor(x * total / 2^32) over
      total = sum of their spare slots selects the expert whose slot range
      holds r; that expert's spare drops by one.  With no candidate the
      assignment stays dropped;
    * the new gate is the reassigned expert's score (softmax probability
      or sigmoid score) under the token's own normaliser: divided by the
      sum of the scores of its originally chosen experts when gates are
      renormalised, as is;
    * each expert's rows are its kept assignments in token order followed
      by its reassigned ones in the order they were placed.
    counts (for the aux loss) stay the routing decisions before the cut.

    Returns the :func:`dispatch` dict plus ``idx`` and ``gate`` (updated
    copies) and ``n_reassigned``."""
    idx = np.asarray(idx, np.int64)
    T, k = idx.shape
    base = dispatch(idx, E, cap)
    new_idx = idx.copy()
    new_gate = np.array(gate, np.float64, copy=True)
    extra = [[] for _ in range(E)]
    if cap > 0:
        scores = np.asarray(scores, np.float64)
        spare = [cap - int(base["kept"][e]) for e in range(E)]
        key = (int(seed) & _U32, (int(seed) >> 32) & _U32)
        for a in range(T * k):
            if base["slot_of"][a] >= 0:
                continue
            t, j = divmod(a, k)
            cand = _reassign_candidates(spare,
                                        set(int(e) for e in new_idx[t]))
            if not cand:
                continue
            e = _pick_slot(philox4x32((a, 0, 0, 0), key)[0], cand, spare)
            spare[e] -= 1
            new_idx[t, j] = e
            new_gate[t, j] = _reassigned_gate(scores[t], idx[t], e,
                                              renormalize)
            extra[e].append(a)
    kept = np.array([base["kept"][e] + len(extra[e]) for e in range(E)],
                    np.int64)
    offsets = np.zeros(E + 1, np.int64)
    offsets[1:] = np.cumsum(kept)
    perm = []
    slot_of = np.full(T * k, -1, np.int64)
    for e in range(E):
        rows = list(base["perm"][base["offsets"][e]:base["offsets"][e + 1]])
        for a in rows + extra[e]:
            slot_of[a] = len(perm)
            perm.append(int(a))
    return {"counts": base["counts"], "kept": kept, "offsets": offsets,
            "perm": np.asarray(perm, np.int64), "slot_of": slot_of,
            "n_dropped": int(T * k - offsets[E]), "idx": new_idx,
            "gate": new_gate,
            "n_reassigned": int(sum(len(x) for x in extra))}


# ---------------------------------------------------------------------------
# Steps 3-4: expert FFNs over each expert's kept rows
# ---------------------------------------------------------------------------

def _ffn(X, act, w1, w_up, w2, b1, b2):
    """One expert on a batch of rows X [n, d] (float64).

    GELU expert: Linear(d, d_ff) with bias, exact GELU, Linear(d_ff, d)
    with bias ([RC] "How a sparse MoE layer works").  SwiGLU expert:
    w_down(silu(w_gate x) * w_up x), no biases ([GN] "Implementing a
    complete MoE layer"; "Mixtral 8x7B" gives the three matrices).
    """
    if act == "gelu":
        h = gelu(X @ np.asarray(w1, F64).T + np.asarray(b1, F64))
        return h @ np.asarray(w2, F64).T + np.asarray(b2, F64)
    if act == "swiglu":
        g = X @ np.asarray(w1, F64).T
        u = X @ np.asarray(w_up, F64).T
        return (silu(g) * u) @ np.asarray(w2, F64).T
    raise ValueError(f"unknown activation {act!r}")


def _expert_args(weights, act, e):
    if act == "gelu":
        return (weights["w1"][e], None, weights["w2"][e],
                weights["b1"][e], weights["b2"][e])
    return (weights["w_gate"][e], weights["w_up"][e], weights["w_down"][e],
            None, None)


def _shared_args(weights, act):
    if act == "gelu":
        return (weights["shared_w1"], None, weights["shared_w2"],
                weights["shared_b1"], weights["shared_b2"])
    return (weights["shared_gate"], weights["shared_up"],
            weights["shared_down"], None, None)


def expert_ffn(x, perm, offsets, weights, act, k, n_shared=0, tokens=None):
    """Run every expert once over the rows grouped to it.

    Row r in [offsets[e], offsets[e+1]) of the result is expert e applied
    to token perm[r] // k: the pages' per-expert loop (gather the tokens an
    expert received, run the expert on them as one batch) from [RC], [LBS]
    "Gating Mechanism" and [HA].  With an always-on shared expert ([GN]
    "DeepSeek-V3", the shared expert pattern; [FA] "The knobs",
    n_shared_experts) row T*k + t holds the shared expert applied to token
    t.  Rows in [offsets[E], T*k) are unused and left zero.

    If ``tokens`` is given, only rows belonging to those tokens are
    computed (the rest stay zero); the arithmetic per row is unchanged.
    """
    x = np.asarray(x)
    T, d = x.shape
    E = len(offsets) - 1
    y = np.zeros((T * k + n_shared * T, d), F64)
    want = None
    if tokens is not None:
        want = np.zeros(T, bool)
        want[np.asarray(tokens, np.int64)] = True
    for e in range(E):
        rows = np.arange(offsets[e], offsets[e + 1])
        t_of = np.asarray(perm, np.int64)[rows] // k
        if want is not None:
            sel = want[t_of]
            rows, t_of = rows[sel], t_of[sel]
        if rows.size == 0:
            continue
        y[rows] = _ffn(np.asarray(x[t_of], F64), act,
                       *_expert_args(weights, act, e))
    if n_shared:
        ts = np.arange(T) if want is None else np.nonzero(want)[0]
        if ts.size:
            y[T * k + ts] = _ffn(np.asarray(x[ts], F64), act,
                                 *_shared_args(weights, act))
    return y


# ---------------------------------------------------------------------------
# Step 5: combine
# ---------------------------------------------------------------------------

def combine(x_residual, y, slot_of, gate, k, n_shared=0, T=None,
            tokens=None):
    """Gate-weighted combine back into token order, plus the residual.

    out[t] = x[t] + (shared row of t) + sum over kept slots j of
    gate[t, j] * y[slot_of[t*k + j]].  A dropped slot adds nothing and the
    surviving gates are not renormalised ([RC] "How a sparse MoE layer
    works": the weights are taken before the capacity cut, and the residual
    is added at the end; [LBS] "Token Dropping and Overflow Handling",
    zero output; [FA] "Concept": the sum of gate times expert output).
    ``x_residual=None`` omits the residual, as the [LBS], [HA] and [GN]
    snippets do.  ``tokens`` restricts the rows computed.
    """
    gate = np.asarray(gate, F64)
    if T is None:
        T = gate.shape[0]
    d = y.shape[1]
    ts = np.arange(T) if tokens is None else np.asarray(tokens, np.int64)
    out = np.zeros((ts.size, d), F64)
    for i, t in enumerate(ts):
        acc = np.zeros(d, F64)
        if x_residual is not None:
            acc += np.asarray(x_residual[t], F64)
        if n_shared:
            acc += y[T * k + t]
        for j in range(k):
            s = slot_of[t * k + j]
            if s >= 0:
                acc += gate[t, j] * y[s]
        out[i] = acc
    return out


# ---------------------------------------------------------------------------
# Step 6: auxiliary load-balance loss
# ---------------------------------------------------------------------------

def aux_loss(counts, probs, alpha):
    """Switch-style load-balance loss alpha * E * sum_e f_e * P_e.

    f_e = (assignments routed to e over all k slots, before any capacity
    cut) / T and P_e = mean over tokens of the full-softmax probability of
    e ([LBS] "The Load Balancing Problem"; [GN] "Load balancing and expert
    collapse" puts alpha inside, as here).  T = 0 gives 0.
    """
    probs = np.asarray(probs, F64)
    T, E = probs.shape
    if T == 0:
        return 0.0
    f = np.asarray(counts, F64) / T
    P = probs.mean(axis=0)
    return float(alpha * E * np.sum(f * P))


# ---------------------------------------------------------------------------
# The whole layer
# ---------------------------------------------------------------------------

def layer_forward(x, w_router, weights, *, k, cap, act, n_shared=0,
                  alpha=0.01, router_bias=None, select_bias=None,
                  residual=True, tokens=None, scoring="softmax",
                  renormalize=True, reassign_seed=None):
    """Route, dispatch, expert FFNs, combine and aux loss, in that order.

    With ``tokens`` the routing, dispatch and aux loss still cover every
    token (capacity depends on the whole batch, [FA] "Effect"), while
    expert outputs and the combined output are produced for those tokens
    only; ``out`` then has one row per listed token.
    """
    x = np.asarray(x)
    T = x.shape[0]
    E = np.asarray(w_router).shape[0]
    r = route(x, w_router, k, router_bias, select_bias, scoring, renormalize)
    if reassign_seed is None:
        dsp = dispatch(r["idx"], E, cap)
    else:
        dsp = dispatch_reassign(r["idx"], r["scores"], r["gate"], E, cap,
                                reassign_seed, renormalize)
        r = dict(r)
        r["idx"], r["gate"] = dsp.pop("idx"), dsp.pop("gate")
    y = expert_ffn(x, dsp["perm"], dsp["offsets"], weights, act, k,
                   n_shared, tokens)
    out = combine(x if residual else None, y, dsp["slot_of"], r["gate"], k,
                  n_shared, T, tokens)
    aux = aux_loss(dsp["counts"], r["probs"], alpha)
    res = dict(r)
    res.update(dsp)
    res.update({"y": y, "out": out, "aux": aux,
                "prob_mean": r["probs"].mean(axis=0) if T else
                np.zeros(E, F64)})
    return res


def update_select_bias(select_bias, counts, gamma):
    """One step of the auxiliary-loss-free balancing of [GN] "DeepSeek-V3":
    the selection bias of an over-loaded expert goes down and that of an
    under-loaded expert goes up.  The page gives no step rule; the plain
    reading kept here moves every bias by a fixed gamma towards balance:
    b_e <- b_e + gamma * sign(mean count - count_e), where count_e are the
    pre-capacity assignments of the step and the mean is sum(counts) / E.
    The sign is decided exactly (sum(counts) - E * count_e in integers);
    the update is one float32 addition."""
    c = np.asarray(counts, np.int64)
    E = c.shape[0]
    sgn = np.sign(c.sum() - E * c).astype(np.float32)
    b = np.asarray(select_bias, np.float32)
    return (b + np.float32(gamma) * sgn).astype(np.float32)


# ---------------------------------------------------------------------------
# 4-bit expert weights (decode path)
# ---------------------------------------------------------------------------
# [LBS] "Production Considerations", Quantization for MoE: storing expert
# weights in 4 bits shrinks Mixtral 8x7B's weights from about 93 GB to about
# 26 GB; the calibrated methods the page names need data, so the reading
# kept here is plain round-to-nearest with one affine pair (scale, offset)
# per group of Q4_GROUP consecutive input-dimension weights of one output
# row.  The code of every weight is an integer decided by floating point,
# so the decision is taken in float32 with correctly rounded division, the
# precision the GPU quantiser uses.

Q4_GROUP = 128


def quantize_int4(w):
    """Group-wise 4-bit round-to-nearest codes of a weight matrix.

    ``w`` [rows, K] (K a multiple of 128) holds bf16 values as float32.  Per
    group of 128 consecutive weights of a row: lo = min, hi = max,
    s = (hi - lo) / 15, code q = rint((w - lo) / s) clamped to 0..15
    (ties to even); a constant group gets s = 0 and q = 0.  The weight is
    represented as lo + q * s.  Returns ``(q [rows, K] uint8, scale
    [rows, K/128] float32, offset [rows, K/128] float32)``."""
    w = np.asarray(w, np.float32)
    rows, K = w.shape
    assert K % Q4_GROUP == 0
    g = w.reshape(rows, K // Q4_GROUP, Q4_GROUP)
    lo = g.min(axis=2)
    hi = g.max(axis=2)
    s = ((hi - lo) / np.float32(15.0)).astype(np.float32)
    const = s == 0
    safe = np.where(const, np.float32(1.0), s)[..., None]
    v = (g - lo[..., None]) / safe                      # float32 arithmetic
    q = np.clip(np.rint(v), 0, 15)
    q = np.where(const[..., None], 0, q).astype(np.uint8)
    return q.reshape(rows, K), s, lo.astype(np.float32)


def dequantize_int4(q, scale, offset):
    """Weights represented by 4-bit codes: offset + q * scale per group, in
    float64 ([rows, K])."""
    q = np.asarray(q, F64)
    rows, K = q.shape
    s = np.repeat(np.asarray(scale, F64), Q4_GROUP, axis=1)
    o = np.repeat(np.asarray(offset, F64), Q4_GROUP, axis=1)
    return o + q * s
