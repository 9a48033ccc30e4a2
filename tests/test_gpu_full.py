"""Parity at the full workload sizes, in the launch configuration the
benchmark times.

* The whole layer (moe_layer_forward, one call): routing decisions,
  per-expert counts and the drop count for every token; the aux loss; the
  combined output and its MoE part (output minus residual) on a sample of
  tokens the oracle evaluates one by one (its routing and capacity still
  cover the whole batch).
* Dispatch (moe_dispatch, or moe_dispatch_reassign for the reassigning
  Switch layer) on the GPU router's own top-k at full size: offsets, the
  permutation, the slot map and so the drop set, bit for bit against the
  oracle.  These batches run 1 to 128 chunks of 256 assignments.
* The expert FFN (moe_expert_ffn) on the oracle's grouping: every row of
  the largest expert's group against the oracle.  On the Mixtral-shaped
  prefill layer also the last expert, whose tiles end the last XCD's run
  of tiles in both GEMMs (the down GEMM's last round is split along K, and
  its last row tile is partial); on the DeepSeek-V3-shaped layer also the always-on
  shared expert (all 4096 rows).
"""

import time

import numpy as np
import pytest
import torch

import oracle
import sparse_mixture_experts_34_amd as moe
from gpu_helpers import (AUX_RTOL, GATE_TOL, TOL, gpu_dispatch,
                         gpu_expert_ffn, gpu_layer, gpu_route, host, log,
                         make, oracle_layer, oracle_route, rel_inf)
from sparse_mixture_experts_34_amd import synth

pytestmark = pytest.mark.gpu

FULL = ["mixtral_decode", "mixtral_prefill", "switch_top1_cf1",
        "switch_top1_cf125", "switch_top1_cf1_reassign", "deepseek_v3"]
SAMPLES = {"mixtral_decode": 16, "mixtral_prefill": 48, "switch_top1_cf1": 48,
           "switch_top1_cf125": 48, "switch_top1_cf1_reassign": 48,
           "deepseek_v3": 10}


@pytest.fixture(scope="module", params=FULL)
def full(request):
    """One full workload's inputs at a time (the device holds one); a
    module-scoped fixture, so pytest runs every test of a workload before
    drawing the next."""
    wl = synth.WORKLOADS[request.param]
    torch.cuda.empty_cache()
    inp = make(wl)
    yield wl, inp
    del inp
    torch.cuda.empty_cache()


def test_full_size_layer(full):
    wl, inp = full
    name = wl.name
    t0 = time.time()
    g = gpu_layer(inp, wl)
    log(f"  {name}: gpu layer done ({time.time() - t0:.1f}s incl. first "
        f"launch)")
    rng = np.random.default_rng(7)
    n = min(SAMPLES[name], wl.T)
    tokens = np.unique(np.concatenate([[0, wl.T - 1],
                                       rng.choice(wl.T, n, replace=False)]))
    t0 = time.time()
    o = oracle_layer(inp, wl, tokens=tokens, lazy=True)
    log(f"  {name}: oracle ({len(tokens)} sampled tokens) "
        f"{time.time() - t0:.1f}s")
    idx = host(g["idx"])
    flips = int((idx != o["idx"]).any(axis=1).sum())
    log(f"  {name}: routing flips {flips}, counts {o['counts'].tolist()[:8]}"
        f"..., dropped {o['n_dropped']} ({o['n_dropped'] / (wl.T * wl.top_k):.2%})")
    assert flips == 0
    assert host(g["counts"]).tolist() == o["counts"].tolist()
    assert int(host(g["n_dropped"])[0]) == o["n_dropped"]
    aux = float(host(g["aux"])[0])
    assert abs(aux - o["aux"]) <= AUX_RTOL * abs(o["aux"]), (aux, o["aux"])
    out = host(g["out"][torch.as_tensor(tokens, device=g["out"].device)])
    err = rel_inf(out, o["out"])
    x = host(inp["x"])[tokens]
    derr = rel_inf(out - x, o["out"] - x)
    log(f"  {name}: sampled out rel err {err:.2e} (moe delta {derr:.2e})")
    assert np.isfinite(out).all()
    assert err <= TOL[wl.dtype]
    # the MoE part alone (the residual x ~ N(0, 1) would hide its errors)
    assert derr <= TOL[wl.dtype]
    g2 = gpu_layer(inp, wl)
    assert torch.equal(g["out"], g2["out"])


def _dropped(slot_of):
    return np.nonzero(np.asarray(slot_of) < 0)[0].tolist()


def _oracle_grouping(inp, wl):
    r = oracle_route(inp, wl)
    if wl.overflow == "reassign":
        return oracle.dispatch_reassign(r["idx"], r["scores"], r["gate"],
                                        wl.n_experts, wl.capacity,
                                        wl.overflow_seed, not wl.raw_gates)
    return oracle.dispatch(r["idx"], wl.n_experts, wl.capacity)


def test_full_size_dispatch(full):
    wl, inp = full
    name = wl.name
    T, k, E = wl.T, wl.top_k, wl.n_experts
    gr = gpu_route(inp, wl)
    r = oracle_route(inp, wl)
    gidx = host(gr["idx"])
    assert (gidx == r["idx"]).all(), "routing differs from the oracle"
    nchunks = (T * k + 255) // 256
    if wl.overflow == "reassign":
        want = oracle.dispatch_reassign(r["idx"], r["scores"], r["gate"], E,
                                        wl.capacity, wl.overflow_seed,
                                        not wl.raw_gates)
        dev = "cuda"
        p = moe.problem_for(wl)
        ws = moe.workspace(p, dev)
        idx, gate = gr["idx"], gr["gate"]
        got = {
            "counts": torch.full((E,), -7, dtype=torch.int32, device=dev),
            "offsets": torch.full((E + 1,), -7, dtype=torch.int32,
                                  device=dev),
            "perm": torch.full((T * k,), -7, dtype=torch.int32, device=dev),
            "slot_of": torch.full((T * k,), -7, dtype=torch.int32,
                                  device=dev),
            "n_dropped": torch.full((1,), -7, dtype=torch.int32, device=dev),
            "aux": torch.full((1,), float("nan"), device=dev)}
        moe.moe_dispatch_reassign(p, idx, gate, gr["logits"], gr["prob_mean"],
                                  got["counts"], got["offsets"], got["perm"],
                                  got["slot_of"], got["n_dropped"],
                                  got["aux"], ws)
        torch.cuda.synchronize()
        assert host(idx).tolist() == want["idx"].tolist()
        assert np.abs(host(gate) - want["gate"]).max() <= GATE_TOL
        extra = f", reassigned {want['n_reassigned']}"
    else:
        want = oracle.dispatch(r["idx"], E, wl.capacity)
        got = gpu_dispatch(gidx, host(gr["prob_mean"]), wl)
        extra = ""
    assert host(got["counts"]).tolist() == want["counts"].tolist()
    assert host(got["offsets"]).tolist() == want["offsets"].tolist()
    total = int(want["offsets"][-1])
    perm = host(got["perm"])
    assert perm[:total].tolist() == want["perm"].tolist()
    assert (perm[total:T * k] == -1).all()
    slot = host(got["slot_of"])[:T * k]
    assert slot.tolist() == want["slot_of"].tolist()
    assert _dropped(slot) == _dropped(want["slot_of"])
    assert int(host(got["n_dropped"])[0]) == want["n_dropped"]
    log(f"  {name}: {nchunks} dispatch chunks, perm/slot_of/offsets bit for "
        f"bit, {want['n_dropped']} dropped{extra}")


def _tiles_of_groups(rows, bm, nb):
    """Logical tile ranges [first, end) of each group (row tiles times
    column blocks), in the order the tiled schedule numbers them."""
    spans = [((r + bm - 1) // bm) * nb for r in rows]
    ends = np.cumsum(spans)
    return [(int(e - s), int(e)) for s, e in zip(spans, ends)]


def _split_tiles(total, cpx, nk):
    """Logical tiles whose last round the tiled schedule splits along K:
    each XCD's contiguous run leaves lo tiles after its whole rounds; they
    are cut into s = min(cpx // lo, nk, 8) pieces when s >= 2 and the split
    takes at least 48 of the nk K slices off the last round."""
    per = (total + 7) // 8
    out = []
    for xcd in range(8):
        first = xcd * per
        n = max(0, min(per, total - first))
        whole = n // cpx
        lo = n - whole * cpx
        if lo > 0:
            s = min(cpx // lo, nk, 8)
            if s >= 2 and nk - nk // s >= 48:
                out += list(range(first + whole * cpx, first + n))
    return out


def _expert_rows_check(inp, wl, o_disp, e, label):
    """Every row of group e (e == E: the shared expert) of the GPU's expert
    FFN against the oracle's."""
    T, k, E = wl.T, wl.top_k, wl.n_experts
    y = gpu_expert_ffn(inp, o_disp["perm"], o_disp["offsets"], wl)
    w = synth.oracle_weights(inp, wl, lazy=True)
    xh = host(inp["x"])
    t0 = time.time()
    if e < E:
        a, b = int(o_disp["offsets"][e]), int(o_disp["offsets"][e + 1])
        perm_e = o_disp["perm"][a:b]
        offs_e = np.zeros(E + 1, np.int64)
        offs_e[e + 1:] = b - a
        want = oracle.expert_ffn(xh, perm_e, offs_e, w, wl.act, k)[:b - a]
        got = host(y[a:b])
    else:
        a, b = T * k, T * k + T
        want = oracle.expert_ffn(xh, np.zeros(0, np.int64),
                                 np.zeros(E + 1, np.int64), w, wl.act, k,
                                 n_shared=1)[T * k:]
        got = host(y[a:b])
    err = rel_inf(got, want)
    log(f"  {wl.name}: {label}: {b - a} rows x {wl.d_model}, rel err "
        f"{err:.2e} (oracle {time.time() - t0:.1f}s)")
    assert np.isfinite(got).all()
    assert err <= TOL[wl.dtype]


def test_full_size_expert_rows(full):
    """The largest routed expert's whole row group on every workload; on the
    Mixtral-shaped prefill layer also the last expert (its tiles take the
    K-split last round of the last XCD in the down GEMM, and its last row
    tile is partial); on the DeepSeek-V3-shaped layer also the shared
    expert."""
    wl, inp = full
    d = _oracle_grouping(inp, wl)
    rows = np.diff(d["offsets"]).tolist()
    e = int(np.argmax(rows))
    _expert_rows_check(inp, wl, d, e, f"largest expert {e} ({rows[e]} rows)")
    if wl.name == "mixtral_prefill":
        e = wl.n_experts - 1
        cpx = torch.cuda.get_device_properties(0).multi_processor_count // 8
        for gemm, nb, nk in (("up", (wl.d_ff + 127) // 128, wl.d_model // 64),
                             ("down", (wl.d_model + 255) // 256, wl.d_ff // 64)):
            spans = _tiles_of_groups(rows, 256, nb)
            split = set(_split_tiles(spans[-1][1], cpx, nk))
            mine = set(range(*spans[e]))
            log(f"  {gemm} GEMM: {spans[-1][1]} tiles, {len(split)} split "
                f"along K, {len(split & mine)} of them in expert {e}")
            if gemm == "down":
                assert split & mine, "expert must own tiles of the K-split round"
        assert rows[e] % 256 != 0, "expert must end in a partial row tile"
        _expert_rows_check(inp, wl, d, e, f"expert {e} ({rows[e]} rows)")
    if wl.n_shared:
        _expert_rows_check(inp, wl, d, wl.n_experts, "shared expert")
