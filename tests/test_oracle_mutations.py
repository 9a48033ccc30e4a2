"""Plant plausible mistakes into the CPU oracle (on the CPU, via
monkeypatch) and check that at least one pin catches each of them."""

import math

import numpy as np
import pytest

import int4_format
import oracle
import oracle.moe as om
import oracle_pins

F64 = np.float64


def _patch(monkeypatch, name, fn):
    monkeypatch.setattr(om, name, fn)
    if hasattr(oracle, name):
        monkeypatch.setattr(oracle, name, fn)


_route = om.route
_dispatch = om.dispatch
_combine = om.combine
_ffn = om._ffn
_aux = om.aux_loss
_capacity = om.capacity
_expert_ffn = om.expert_ffn


def m_no_renormalise(mp):
    def route(*a, **k):
        r = _route(*a, **k)
        r["gate"] = np.take_along_axis(r["probs"], r["idx"], axis=1)
        return r
    _patch(mp, "route", route)


def m_tie_to_higher_index(mp):
    def route(x, w_router, k, router_bias=None, select_bias=None,
              scoring="softmax", renormalize=True):
        r = _route(x, w_router, k, router_bias, select_bias, scoring,
                   renormalize)
        keys = r["keys"]
        E = keys.shape[1]
        for t in range(keys.shape[0]):
            order = sorted(range(E), key=lambda e: (-float(keys[t, e]), -e))
            r["idx"][t] = order[:k]
        ch = np.take_along_axis(r["scores"], r["idx"], axis=1)
        r["gate"] = ch / ch.sum(1, keepdims=True) if renormalize else ch
        return r
    _patch(mp, "route", route)


def m_bias_in_gates(mp):
    def route(x, w_router, k, router_bias=None, select_bias=None,
              scoring="softmax", renormalize=True):
        r = _route(x, w_router, k, router_bias, select_bias, scoring,
                   renormalize)
        if select_bias is not None and scoring == "softmax":
            p = om.softmax(r["keys"])
            ch = np.take_along_axis(p, r["idx"], axis=1)
            r["gate"] = ch / ch.sum(1, keepdims=True) if renormalize else ch
        return r
    _patch(mp, "route", route)


def m_capacity_by_slot(mp):
    def dispatch(idx, E, cap):
        idx = np.asarray(idx)
        T, k = idx.shape
        r = _dispatch(idx, E, 0)
        perm, slot_of = [], np.full(T * k, -1, np.int64)
        kept = np.zeros(E, np.int64)
        for e in range(E):
            slots, rows = np.nonzero(idx.T == e)   # slot-major order
            n = rows.size if cap <= 0 else min(rows.size, cap)
            kept[e] = n
            for t, j in zip(rows[:n], slots[:n]):
                slot_of[t * k + j] = len(perm)
                perm.append(t * k + j)
        r.update(kept=kept, perm=np.asarray(perm), slot_of=slot_of,
                 n_dropped=int(T * k - kept.sum()))
        r["offsets"] = np.concatenate([[0], np.cumsum(kept)])
        return r
    _patch(mp, "dispatch", dispatch)


def m_keep_last(mp):
    def dispatch(idx, E, cap):
        idx = np.asarray(idx)
        T, k = idx.shape
        r = _dispatch(idx, E, 0)
        perm, slot_of = [], np.full(T * k, -1, np.int64)
        kept = np.zeros(E, np.int64)
        for e in range(E):
            rows, slots = np.nonzero(idx == e)
            n = rows.size if cap <= 0 else min(rows.size, cap)
            kept[e] = n
            for t, j in zip(rows[rows.size - n:], slots[rows.size - n:]):
                slot_of[t * k + j] = len(perm)
                perm.append(t * k + j)
        r.update(kept=kept, perm=np.asarray(perm), slot_of=slot_of,
                 n_dropped=int(T * k - kept.sum()))
        r["offsets"] = np.concatenate([[0], np.cumsum(kept)])
        return r
    _patch(mp, "dispatch", dispatch)


def m_renormalise_survivors(mp):
    def combine(x_residual, y, slot_of, gate, k, n_shared=0, T=None,
                tokens=None):
        g = np.array(gate, F64)
        for t in range(g.shape[0]):
            keep = [slot_of[t * k + j] >= 0 for j in range(k)]
            s = sum(g[t, j] for j in range(k) if keep[j])
            if 0 < s:
                g[t] = g[t] / s
        return _combine(x_residual, y, slot_of, g, k, n_shared, T, tokens)
    _patch(mp, "combine", combine)


def m_transposed_w2(mp):
    def ffn(X, act, w1, w_up, w2, b1, b2):
        w2 = np.asarray(w2)
        if w2.shape[0] == w2.shape[1]:
            w2 = w2.T
        return _ffn(X, act, w1, w_up, w2, b1, b2)
    _patch(mp, "_ffn", ffn)


def m_drop_bias_b2(mp):
    def ffn(X, act, w1, w_up, w2, b1, b2):
        if b2 is not None:
            b2 = np.zeros_like(np.asarray(b2, F64))
        return _ffn(X, act, w1, w_up, w2, b1, b2)
    _patch(mp, "_ffn", ffn)


def m_gelu_tanh(mp):
    def gelu(z):
        z = np.asarray(z, F64)
        return 0.5 * z * (1 + np.tanh(math.sqrt(2 / math.pi)
                                      * (z + 0.044715 * z ** 3)))
    _patch(mp, "gelu", gelu)


def m_silu_is_sigmoid(mp):
    def silu(z):
        z = np.asarray(z, F64)
        return 1.0 / (1.0 + np.exp(-z))
    _patch(mp, "silu", silu)


def m_swap_gate_up(mp):
    def ffn(X, act, w1, w_up, w2, b1, b2):
        if act == "swiglu":
            return _ffn(X, act, w_up, w1, w2, b1, b2)
        return _ffn(X, act, w1, w_up, w2, b1, b2)
    _patch(mp, "_ffn", ffn)


def m_aux_post_capacity(mp):
    def layer_forward(*a, **kw):
        r = _layer(*a, **kw)
        r["aux"] = _aux(r["kept"], r["probs"], kw.get("alpha", 0.01))
        return r
    _patch(mp, "layer_forward", layer_forward)

    def aux_loss(counts, probs, alpha):
        c = np.minimum(np.asarray(counts), 2)
        return _aux(c, probs, alpha)
    _patch(mp, "aux_loss", aux_loss)


def m_aux_no_E(mp):
    def aux_loss(counts, probs, alpha):
        E = np.asarray(probs).shape[1]
        return _aux(counts, probs, alpha) / E
    _patch(mp, "aux_loss", aux_loss)


def m_capacity_ceil(mp):
    def capacity(T, k, E, cf_num, cf_den):
        return max(1, -(-(cf_num * T * k) // (cf_den * E)))
    _patch(mp, "capacity", capacity)


def m_softmax_no_shift(mp):
    def softmax(l):
        l = np.asarray(l, F64)
        with np.errstate(over="ignore", invalid="ignore"):
            e = np.exp(l)
            return e / e.sum(-1, keepdims=True)
    _patch(mp, "softmax", softmax)


def m_no_shared(mp):
    def expert_ffn(x, perm, offsets, weights, act, k, n_shared=0,
                   tokens=None):
        y = _expert_ffn(x, perm, offsets, weights, act, k, n_shared, tokens)
        T = np.asarray(x).shape[0]
        y[T * k:] = 0.0
        return y
    _patch(mp, "expert_ffn", expert_ffn)


def m_token_from_assignment_by_E(mp):
    # a wrong index: token = a // E instead of a // k
    def expert_ffn(x, perm, offsets, weights, act, k, n_shared=0,
                   tokens=None):
        E = len(offsets) - 1
        return _expert_ffn(x, perm, offsets, weights, act, E, n_shared,
                           tokens) if E != k else \
            _expert_ffn(x, perm, offsets, weights, act, k, n_shared, tokens)
    _patch(mp, "expert_ffn", expert_ffn)


_layer = om.layer_forward
_quantize = om.quantize_int4
_dequantize = om.dequantize_int4


def m_q4_floor(mp):
    def quantize_int4(w):
        w = np.asarray(w, np.float32)
        rows, K = w.shape
        g = w.reshape(rows, K // 128, 128)
        lo, hi = g.min(axis=2), g.max(axis=2)
        s = ((hi - lo) / np.float32(15.0)).astype(np.float32)
        safe = np.where(s == 0, np.float32(1), s)
        q = np.clip(np.floor((g - lo[..., None]) / safe[..., None]), 0, 15)
        q = np.where(s[..., None] == 0, 0, q).astype(np.uint8)
        return q.reshape(rows, K), s, lo
    _patch(mp, "quantize_int4", quantize_int4)


def m_q4_sixteen_steps(mp):
    def quantize_int4(w):
        q, s, o = _quantize(w)
        return q, (s * np.float32(15.0 / 16.0)).astype(np.float32), o
    _patch(mp, "quantize_int4", quantize_int4)


def m_q4_dequant_no_offset(mp):
    def dequantize_int4(q, scale, offset):
        return _dequantize(q, scale, np.zeros_like(np.asarray(offset)))
    _patch(mp, "dequantize_int4", dequantize_int4)


def m_q4_pack_untiled(mp):
    # the right words, stored row by row instead of in MFMA tiles
    def pack_int4(q):
        q = np.asarray(q, np.uint32)
        rows, K = q.shape
        k8 = q.reshape(rows, K // 8, 8)
        word = np.zeros((rows, K // 8), np.uint32)
        for i in range(4):
            word |= k8[:, :, 2 * i] << np.uint32(4 * i)
            word |= k8[:, :, 2 * i + 1] << np.uint32(16 + 4 * i)
        return word.astype("<u4").view(np.uint8).reshape(rows, K // 2)
    # the format helper the GPU byte comparisons use
    mp.setattr(int4_format, "pack_int4", pack_int4)


def m_q4_qparams_row_major(mp):
    def pack_qparams(scale, offset):
        return np.stack([np.asarray(scale, np.float32),
                         np.asarray(offset, np.float32)], axis=-1)
    mp.setattr(int4_format, "pack_qparams", pack_qparams)


def m_sigmoid_bias_on_logits(mp):
    def route(x, w_router, k, router_bias=None, select_bias=None,
              scoring="softmax", renormalize=True):
        r = _route(x, w_router, k, router_bias, select_bias, scoring,
                   renormalize)
        if scoring == "sigmoid" and select_bias is not None:
            r2 = _route(x, w_router, k, router_bias, select_bias, "softmax",
                        renormalize)
            r["idx"] = r2["idx"]
            ch = np.take_along_axis(r["scores"], r["idx"], 1)
            r["gate"] = ch / ch.sum(1, keepdims=True) if renormalize else ch
        return r
    _patch(mp, "route", route)


def m_raw_gates_renormalised(mp):
    def route(x, w_router, k, router_bias=None, select_bias=None,
              scoring="softmax", renormalize=True):
        return _route(x, w_router, k, router_bias, select_bias, scoring, True)
    _patch(mp, "route", route)


def m_sigmoid_probs_unnormalised(mp):
    def route(x, w_router, k, router_bias=None, select_bias=None,
              scoring="softmax", renormalize=True):
        r = _route(x, w_router, k, router_bias, select_bias, scoring,
                   renormalize)
        if scoring == "sigmoid":
            r["probs"] = r["scores"]
        return r
    _patch(mp, "route", route)


def m_bias_update_wrong_sign(mp):
    _upd = om.update_select_bias

    def update_select_bias(select_bias, counts, gamma):
        return _upd(select_bias, counts, -gamma)
    _patch(mp, "update_select_bias", update_select_bias)


def m_reassign_own_expert_allowed(mp):
    mp.setattr(om, "_reassign_candidates",
               lambda spare, mine: [e for e in range(len(spare))
                                    if spare[e] > 0])


def m_reassign_uniform_over_experts(mp):
    def pick(x, cand, spare):
        return cand[(x * len(cand)) >> 32]
    mp.setattr(om, "_pick_slot", pick)


def m_reassign_gate_unnormalised(mp):
    mp.setattr(om, "_reassigned_gate",
               lambda scores_t, orig_idx_t, e, renormalize: scores_t[e])


def m_reassign_gate_new_normaliser(mp):
    # normalised over the token's experts after the move instead of the
    # experts it originally chose
    _disp = om.dispatch_reassign

    def dispatch_reassign(idx, scores, gate, E, cap, seed, renormalize=True):
        r = _disp(idx, scores, gate, E, cap, seed, renormalize)
        if renormalize:
            sc = np.asarray(scores, np.float64)
            moved = np.argwhere(r["idx"] != np.asarray(idx))
            for t, j in moved:
                r["gate"][t, j] = sc[t, r["idx"][t, j]] / \
                    sc[t, r["idx"][t]].sum()
        return r
    _patch(mp, "dispatch_reassign", dispatch_reassign)


def m_reassign_gate_softmax_under_sigmoid(mp):
    # under sigmoid scoring, the moved slot weighted by the softmax
    # probability of the new expert
    _disp = om.dispatch_reassign

    def dispatch_reassign(idx, scores, gate, E, cap, seed, renormalize=True):
        sc = np.asarray(scores, np.float64)
        if sc.size and not np.allclose(sc.sum(axis=1), 1.0):
            with np.errstate(divide="ignore"):
                sc = om.softmax(np.log(sc) - np.log1p(-sc))
        return _disp(idx, sc, gate, E, cap, seed, renormalize)
    _patch(mp, "dispatch_reassign", dispatch_reassign)


def m_philox_swapped_products(mp):
    _ph = om.philox4x32

    def philox4x32(ctr, key, rounds=10):
        c = [int(v) & 0xFFFFFFFF for v in ctr]
        k = [int(v) & 0xFFFFFFFF for v in key]
        for r in range(rounds):
            if r:
                k = [(k[0] + 0x9E3779B9) & 0xFFFFFFFF,
                     (k[1] + 0xBB67AE85) & 0xFFFFFFFF]
            p0 = 0xD2511F53 * c[0]
            p1 = 0xCD9E8D57 * c[2]
            # high halves mixed with the wrong words
            c = [(p0 >> 32) ^ c[1] ^ k[0], p1 & 0xFFFFFFFF,
                 (p1 >> 32) ^ c[3] ^ k[1], p0 & 0xFFFFFFFF]
        return c
    _patch(mp, "philox4x32", philox4x32)
    del _ph


MUTATIONS = [m_no_renormalise, m_tie_to_higher_index, m_bias_in_gates,
             m_capacity_by_slot, m_keep_last, m_renormalise_survivors,
             m_transposed_w2, m_drop_bias_b2, m_gelu_tanh, m_silu_is_sigmoid,
             m_swap_gate_up, m_aux_post_capacity, m_aux_no_E,
             m_capacity_ceil, m_softmax_no_shift, m_no_shared,
             m_token_from_assignment_by_E, m_q4_floor, m_q4_sixteen_steps,
             m_q4_dequant_no_offset, m_q4_pack_untiled,
             m_q4_qparams_row_major, m_sigmoid_bias_on_logits,
             m_raw_gates_renormalised, m_sigmoid_probs_unnormalised,
             m_bias_update_wrong_sign, m_reassign_own_expert_allowed,
             m_reassign_uniform_over_experts, m_reassign_gate_unnormalised,
             m_reassign_gate_new_normaliser,
             m_reassign_gate_softmax_under_sigmoid,
             m_philox_swapped_products]


@pytest.mark.parametrize("mutate", MUTATIONS, ids=[m.__name__ for m in
                                                   MUTATIONS])
def test_some_pin_catches(mutate, monkeypatch):
    mutate(monkeypatch)
    caught = []
    for pin in oracle_pins.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught {mutate.__name__}"
