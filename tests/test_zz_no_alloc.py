"""moe_layer_forward_noalloc (the layer without a caller workspace: its
intermediates live in the library's per-GPU scratch) against
moe_layer_forward on the same inputs, through the C ABI.

Each case makes two calls in a row, the second on a smaller batch, so the
second call runs over what the first left in the scratch.  Where no tile of
the 256-row GEMM schedule is split along K (moe_layer_forward splits the
last round of that schedule, the no-alloc entry never does) the two entry
points run the same kernels in the same order and must agree bit for bit;
otherwise the outputs agree within the bf16 tolerance and the routing,
counts and drops bit for bit."""

import ctypes

import numpy as np
import pytest
import torch

import sparse_mixture_experts_34_amd as moe
from sparse_mixture_experts_34_amd import binding
from gpu_helpers import TOL, gpu_layer, host, log, make, rel_inf
from sparse_mixture_experts_34_amd import synth

pytestmark = pytest.mark.gpu

W = synth.Workload
CASES = [
    # Mixtral-shaped decode (stream schedule), then 5 tokens
    (synth.WORKLOADS["mixtral_decode"], 5, True),
    # GELU experts with a shared expert and capacity drops (panel
    # schedule), then a smaller batch (stream schedule)
    (W("na_gelu_shared_drops", T=700, d_model=256, n_experts=8, top_k=2,
       d_ff=512, act="gelu", dtype="bf16", capacity=150, n_shared=1,
       zipf_s=0.5, seed_index=90), 37, True),
    # 256-row tiled schedule (T*k > 256*E), then the panel schedule; K of
    # 256 and 384 is too short for moe_layer_forward to split a last round
    (W("na_tiled", T=1500, d_model=256, n_experts=4, top_k=2, d_ff=384,
       act="swiglu", dtype="bf16", capacity=0, seed_index=91), 300, True),
    # the same schedule with K = 4096 in the down GEMM, whose last round
    # moe_layer_forward splits along K
    (W("na_tiled_ksplit", T=1500, d_model=256, n_experts=4, top_k=2,
       d_ff=4096, act="swiglu", dtype="bf16", capacity=0, seed_index=92),
     300, False),
    # float32 problem
    (synth.WORKLOADS["tiny_gelu_f32"], 9, True),
]


def noalloc_layer(inp, wl):
    p = moe.problem_for(wl)
    dev = inp["x"].device
    T, E, k = wl.T, wl.n_experts, wl.top_k
    res = {
        "out": torch.full_like(inp["x"], float("nan")),
        "aux": torch.full((1,), float("nan"), device=dev),
        "counts": torch.full((E,), -7, dtype=torch.int32, device=dev),
        "n_dropped": torch.full((1,), -7, dtype=torch.int32, device=dev),
        "idx": torch.full((max(T, 1), k), -7, dtype=torch.int32, device=dev),
    }
    moe.moe_layer_forward_noalloc(p, inp["x"], inp["w_router"],
                                  inp["router_bias"], inp["select_bias"],
                                  inp, res["out"], res["aux"], res["counts"],
                                  res["n_dropped"], res["idx"])
    torch.cuda.synchronize()
    return res


@pytest.mark.parametrize("wl,T2,exact", CASES,
                         ids=[c[0].name for c in CASES])
def test_noalloc_matches_layer_forward(wl, T2, exact):
    for w in (wl, wl.sized(T=T2)):
        inp = make(w)
        ref = gpu_layer(inp, w)
        got = noalloc_layer(inp, w)
        for key in ("idx", "counts", "n_dropped"):
            assert torch.equal(got[key], ref[key]), (w.name, key)
        if exact:
            assert torch.equal(got["out"], ref["out"]), w.name
            assert torch.equal(got["aux"], ref["aux"]), w.name
        else:
            err = rel_inf(host(got["out"]), host(ref["out"]))
            log(f"  {w.name}: no-alloc vs workspace entry rel err {err:.2e}")
            assert err <= TOL[w.dtype]
            assert abs(float(got["aux"].item()) - float(ref["aux"].item())) \
                <= 1e-6 * abs(float(ref["aux"].item()))
        assert np.isfinite(host(got["out"])).all()
        del inp, ref, got
    torch.cuda.empty_cache()


def test_noalloc_rejects_oversized_problem():
    wl = synth.WORKLOADS["mixtral_prefill"]
    p = moe.problem_for(wl)
    x = torch.zeros(1, device="cuda")
    w = binding.moe_expert_weights(x.data_ptr(), x.data_ptr(), x.data_ptr())
    # refused on the host (nothing is enqueued, nothing is read)
    st = binding._lib.moe_layer_forward_noalloc(
        ctypes.byref(p), x.data_ptr(), x.data_ptr(), None, None,
        ctypes.byref(w), x.data_ptr(), None, None, None, None, None)
    assert st == moe.MOE_EWORKSPACE
