"""GPU parity of the expert FFN (moe_expert_ffn) against the CPU oracle on
hand-made groupings whose per-expert row counts sit on every boundary of the
bf16 schedules: empty experts, one row, 15/16/17 rows (16-row MFMA tiles),
127/128/129 rows (half and full 256-row panels), 144/160/161/193 rows (the
three-quarter panel loop and just past it), 255/256/257 rows (one or
two panels or 256-row tiles), with and without a shared expert,
odd numbers of 64-wide K steps and partial weight blocks.  The schedule is
chosen from T, k and E only (stream up to 64 assignments per expert on
average, panel up to 256, tiled beyond), so each case fixes T*k/E and then
places the counts freely (rows past offsets[E] are unused).  Each case runs
through moe_expert_ffn (with workspace: the tiled schedule may split its
last round along K), through moe_expert_up + moe_expert_down without a
workspace (never split) and with one (split as in moe_expert_ffn), with the
weights row-major and in moe_tile_bf16's tiled order.  Outputs are compared by max |gpu - oracle| /
max |oracle| over the computed rows (2e-2, bf16)."""

from dataclasses import replace

import numpy as np
import pytest
import torch

import oracle
from gpu_helpers import TOL, gpu_expert_ffn, host, log
import sparse_mixture_experts_34_amd as moe
from sparse_mixture_experts_34_amd import synth

pytestmark = pytest.mark.gpu

W = synth.Workload

# (workload, per-expert row counts); the comment names the schedule
CASES = [
    # stream: T*k <= 64*E
    (W("ffnb_stream", T=200, d_model=192, n_experts=8, top_k=2, d_ff=320,
       act="swiglu", dtype="bf16", capacity=0, seed_index=40),
     [0, 1, 15, 16, 17, 33, 64, 65]),
    # panel: 64*E < T*k <= 256*E; half (<=128 rows) and full panels, two
    # panels, an empty expert, shared expert over 500 rows (two panels)
    (W("ffnb_panel_swiglu", T=500, d_model=192, n_experts=4, top_k=2,
       d_ff=320, act="swiglu", dtype="bf16", capacity=0, n_shared=1,
       seed_index=41),
     [128, 129, 0, 257]),
    (W("ffnb_panel_swiglu_b", T=500, d_model=192, n_experts=4, top_k=2,
       d_ff=320, act="swiglu", dtype="bf16", capacity=0, seed_index=42),
     [1, 127, 255, 256]),
    # the three-quarter panel loop (129-192 rows: 12 row tiles) from 144 to
    # 161 rows, and just past it
    (W("ffnb_panel_swiglu_c", T=500, d_model=192, n_experts=4, top_k=2,
       d_ff=320, act="swiglu", dtype="bf16", capacity=0, seed_index=51),
     [144, 160, 161, 193]),
    (W("ffnb_panel_gelu", T=500, d_model=256, n_experts=4, top_k=2,
       d_ff=448, act="gelu", dtype="bf16", capacity=0, n_shared=1,
       seed_index=43),
     [15, 16, 17, 385]),
    # tiled: T*k > 256*E; a ragged and a two-tile expert, shared expert
    (W("ffnb_tiled_shared", T=400, d_model=192, n_experts=2, top_k=2, d_ff=320,
       act="swiglu", dtype="bf16", capacity=0, n_shared=1, seed_index=44),
     [127, 385]),
    # tiled, many rows per expert
    (W("ffnb_tiled", T=2100, d_model=128, n_experts=2, top_k=1,
       d_ff=384, act="gelu", dtype="bf16", capacity=0, seed_index=45),
     [255, 1025]),
    # tiled with K = 4096 in both GEMMs: 64 tiles each, 8 left per XCD
    # after no whole round, so with a workspace both last rounds are split
    # into 4 K pieces
    (W("ffnb_tiled_ksplit", T=700, d_model=4096, n_experts=2, top_k=1,
       d_ff=4096, act="gelu", dtype="bf16", capacity=0, seed_index=48),
     [300, 385]),
    # panel with few panels and a long K (the Switch-shaped down GEMM's
    # situation): 128 K steps in the GELU down GEMM (biases, a two-panel
    # expert), then in a SwiGLU up GEMM with the shared expert's two panels
    (W("ffnb_panel_longk_down", T=600, d_model=512, n_experts=4, top_k=1,
       d_ff=8192, act="gelu", dtype="bf16", capacity=0, seed_index=49),
     [130, 0, 257, 200]),
    (W("ffnb_panel_longk_up", T=300, d_model=8192, n_experts=4, top_k=2,
       d_ff=256, act="swiglu", dtype="bf16", capacity=0, n_shared=1,
       seed_index=50),
     [100, 129, 0, 256]),
]


def _grouping(counts, T, k, seed):
    """perm/offsets for the given counts: expert e's rows are distinct
    tokens (as routing makes them), slot j drawn at random."""
    rng = np.random.default_rng(seed)
    assert sum(counts) <= T * k and max(counts) <= T
    perm = []
    for c in counts:
        toks = np.sort(rng.choice(T, size=c, replace=False))
        perm.extend(int(t) * k + int(rng.integers(k)) for t in toks)
    offsets = np.concatenate([[0], np.cumsum(counts)]).astype(np.int32)
    return np.asarray(perm, np.int32), offsets


def _gpu_up_down(inp, perm, offsets, wl, with_ws=False):
    """moe_expert_up then moe_expert_down, with or without a workspace."""
    p = moe.problem_for(wl)
    dev = inp["x"].device
    ws = (torch.empty(moe.moe_workspace_bytes(p), dtype=torch.uint8,
                      device=dev) if with_ws else None)
    rows = wl.T * wl.top_k + wl.n_shared * wl.T
    h = torch.full((rows, wl.d_ff), float("nan"), dtype=wl.torch_dtype,
                   device=dev)
    y = torch.full((rows, wl.d_model), float("nan"), dtype=wl.torch_dtype,
                   device=dev)
    pt = torch.full((max(wl.T * wl.top_k, 1),), -1, dtype=torch.int32,
                    device=dev)
    if perm.size:
        pt[:perm.size] = torch.as_tensor(perm, device=dev)
    ot = torch.as_tensor(offsets, device=dev)
    moe.moe_expert_up(p, inp["x"], pt, ot, inp, h, ws)
    moe.moe_expert_down(p, h, ot, inp, y, ws)
    torch.cuda.synchronize()
    return y


def _errors(y, ref, offsets, counts, rows):
    assert np.isfinite(y[rows]).all()
    err = np.abs(y[rows] - ref[rows]).max() / np.abs(ref[rows]).max()
    # per expert too, so a wrong small group cannot hide behind a big one
    worst = 0.0
    for e in range(len(counts)):
        r = np.arange(offsets[e], offsets[e + 1])
        if r.size:
            worst = max(worst, np.abs(y[r] - ref[r]).max()
                        / np.abs(ref[r]).max())
    return err, worst


@pytest.mark.parametrize("tiled", [False, True], ids=["rowmajor", "tiled"])
@pytest.mark.parametrize("wl,counts", CASES, ids=[c[0].name for c in CASES])
def test_expert_ffn_boundaries(wl, counts, tiled):
    log(f"ffn boundaries {wl.name} ({'tiled' if tiled else 'row-major'} "
        f"weights): counts {counts}")
    inp = synth.make_inputs(wl, device="cuda")
    perm, offsets = _grouping(counts, wl.T, wl.top_k, wl.seed())
    ref = oracle.expert_ffn(host(inp["x"]), perm, offsets,
                            synth.oracle_weights(inp, wl), wl.act, wl.top_k,
                            n_shared=wl.n_shared)
    if tiled:
        wl = replace(wl, wquant="bf16_tiled")
        inp = moe.tile_weights(inp)
    y = host(gpu_expert_ffn(inp, perm, offsets, wl)).astype(np.float64)
    T, k = wl.T, wl.top_k
    rows = np.arange(offsets[-1])
    if wl.n_shared:
        rows = np.concatenate([rows, T * k + np.arange(T)])
    err, worst = _errors(y, ref, offsets, counts, rows)
    y2 = host(_gpu_up_down(inp, perm, offsets, wl)).astype(np.float64)
    err2, worst2 = _errors(y2, ref, offsets, counts, rows)
    y3 = host(_gpu_up_down(inp, perm, offsets, wl, with_ws=True)).astype(
        np.float64)
    err3, worst3 = _errors(y3, ref, offsets, counts, rows)
    log(f"  moe_expert_ffn rel err {err:.2e} (worst expert {worst:.2e}); "
        f"up+down {err2:.2e} ({worst2:.2e}); with workspace {err3:.2e} "
        f"({worst3:.2e})")
    assert max(err, worst, err2, worst2, err3, worst3) <= TOL["bf16"]

