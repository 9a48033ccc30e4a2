"""Repeated layer calls give bit-identical results on one device.

Every reduction in the library has a fixed order; the one integer atomic
(the K pieces of a split tile in the tiled GEMMs) only decides which piece
adds the partial sums, which it does in piece order.  Each schedule runs the
layer three times through one workspace, with another problem's call in
between (its split counters and partial tiles share the workspace area), and
every output must match the first call bit for bit."""

from dataclasses import replace

import pytest
import torch

from gpu_helpers import make
import sparse_mixture_experts_34_amd as moe
from sparse_mixture_experts_34_amd import synth

pytestmark = pytest.mark.gpu

W = synth.Workload
CASES = [
    # stream
    W("det_stream", T=40, d_model=256, n_experts=8, top_k=2, d_ff=512,
      act="swiglu", dtype="bf16", capacity=0, seed_index=50),
    # panel, shared expert
    W("det_panel", T=500, d_model=192, n_experts=4, top_k=2, d_ff=320,
      act="swiglu", dtype="bf16", capacity=0, n_shared=1, seed_index=51),
    # tiled, drops, the up GEMM's last round split along K (K = 4096: 64
    # slices, 3 tiles left per XCD, 8 pieces)
    W("det_tiled_drops", T=1500, d_model=4096, n_experts=4, top_k=2,
      d_ff=256, act="gelu", dtype="bf16", capacity=700, seed_index=52),
    # tiled, the down GEMM's last round split along K (K = 4096)
    W("det_tiled", T=4200, d_model=256, n_experts=2, top_k=1, d_ff=4096,
      act="swiglu", dtype="bf16", capacity=0, seed_index=53),
]
# the same schedules with tiled bf16 weights
CASES += [replace(w, name=w.name + "_tw", wquant="bf16_tiled")
          for w in CASES[1:]]
OTHER = W("det_other", T=3000, d_model=128, n_experts=2, top_k=1, d_ff=256,
          act="gelu", dtype="bf16", capacity=0, seed_index=54)


def _layer(inp, wl, ws):
    p = moe.problem_for(wl)
    if wl.wquant == "bf16_tiled":
        inp = dict(inp, **{n: v for n, v in moe.tile_weights(inp).items()
                           if n in moe.QUANT_MATRICES})
    dev = inp["x"].device
    out = torch.empty_like(inp["x"])
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    counts = torch.empty(wl.n_experts, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    moe.moe_layer_forward(p, inp["x"], inp["w_router"], inp["router_bias"],
                          inp["select_bias"], moe.expert_weights(inp), out,
                          aux, counts, nd, None, ws)
    return out, aux, counts, nd


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_repeated_calls_bit_identical(wl):
    inp = make(wl)
    other = make(OTHER)
    dev = inp["x"].device
    # one workspace big enough for both problems
    nbytes = max(moe.moe_workspace_bytes(moe.problem_for(w))
                 for w in (wl, OTHER))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    first = _layer(inp, wl, ws)
    torch.cuda.synchronize()
    for _ in range(2):
        _layer(other, OTHER, ws)
        again = _layer(inp, wl, ws)
        torch.cuda.synchronize()
        for a, b in zip(first, again):
            assert torch.equal(a, b)
