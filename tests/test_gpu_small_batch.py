"""The layer on decode-sized batches against the CPU oracle.

Batches of a few dozen tokens take the small-batch paths: with at most 8
experts the fused route kernel (one workgroup per token), otherwise the
router GEMM split along K into up to 16 slices and one token per select
wave; with at most 64 assignments and 64 experts the one-wave dispatch,
otherwise the whole dispatch in one workgroup.  Each case checks the layer's expert
indices, counts, drop count and output against the oracle (indices and
counts bit for bit, aux within 1e-4 relative, output within the dtype
tolerance), and, where nothing is reassigned, the indices against
moe_route's and the counts and drop count against moe_dispatch's on those
indices, and a second call bit for bit."""

import numpy as np
import pytest
import torch

from gpu_helpers import (AUX_RTOL, TOL, gpu_dispatch, gpu_layer, gpu_route,
                         host, log, make, oracle_layer, rel_inf)
from sparse_mixture_experts_34_amd import synth

pytestmark = pytest.mark.gpu

W = synth.Workload
CASES = [
    W("sb_decode_e8", T=16, d_model=256, n_experts=8, top_k=2, d_ff=256,
      act="swiglu", dtype="bf16", capacity=0, router_std=0.02, seed_index=60),
    W("sb_one_token", T=1, d_model=128, n_experts=8, top_k=2, d_ff=128,
      act="swiglu", dtype="bf16", capacity=0, seed_index=61),
    # two experts per select lane; sigmoid scores with a selection bias
    W("sb_t31_e100_k3_sigmoid", T=31, d_model=128, n_experts=100, top_k=3,
      d_ff=64, act="gelu", dtype="bf16", capacity=0, scoring="sigmoid",
      select_bias_std=0.1, seed_index=62),
    # four experts per select lane, k = 8, shared expert
    W("sb_t32_e256_k8_shared", T=32, d_model=128, n_experts=256, top_k=8,
      d_ff=64, act="swiglu", dtype="bf16", capacity=0, n_shared=1,
      seed_index=63),
    # float32 with capacity drops
    W("sb_t20_f32_drops", T=20, d_model=64, n_experts=4, top_k=2, d_ff=128,
      act="gelu", dtype="f32", capacity=6, seed_index=64),
    # top-1, raw gates, skewed router, drops
    W("sb_t24_raw_drops", T=24, d_model=128, n_experts=16, top_k=1,
      d_ff=128, act="gelu", dtype="bf16", capacity=2, zipf_s=1.1,
      raw_gates=True, seed_index=65),
    # overflow reassigned after the capacity cut
    W("sb_t32_reassign", T=32, d_model=128, n_experts=16, top_k=1, d_ff=128,
      act="gelu", dtype="bf16", capacity=3, zipf_s=1.1, seed_index=66,
      overflow="reassign", overflow_seed=21),
    W("sb_t33", T=33, d_model=128, n_experts=8, top_k=2, d_ff=128,
      act="swiglu", dtype="bf16", capacity=0, seed_index=67),
    # fused route with a router bias and a selection bias, capacity drops in
    # the one-wave dispatch
    W("sb_t30_e8_biases_drops", T=30, d_model=256, n_experts=8, top_k=2,
      d_ff=128, act="swiglu", dtype="bf16", capacity=6, zipf_s=0.8,
      select_bias_std=0.1, seed_index=68),
    # fused route with sigmoid scores, a selection bias and raw gates
    W("sb_t29_e6_sigmoid_bias_raw", T=29, d_model=192, n_experts=6, top_k=3,
      d_ff=64, act="gelu", dtype="bf16", capacity=0, scoring="sigmoid",
      select_bias_std=0.1, raw_gates=True, seed_index=69),
    # decode size at the one-wave dispatch's limit (64 assignments), router
    # and selection biases, capacity drops
    W("sb_t16_e8_k4_biases_drops", T=16, d_model=256, n_experts=8, top_k=4,
      d_ff=128, act="swiglu", dtype="bf16", capacity=6, zipf_s=0.8,
      select_bias_std=0.1, seed_index=72),
    # 80 assignments at decode size: the one-workgroup dispatch
    W("sb_t16_e8_k5", T=16, d_model=128, n_experts=8, top_k=5, d_ff=64,
      act="swiglu", dtype="bf16", capacity=0, seed_index=73),
    # three experts, top-1 sigmoid scores with a selection bias, raw gates
    W("sb_t7_e3_k1_sigmoid_raw", T=7, d_model=192, n_experts=3, top_k=1,
      d_ff=64, act="gelu", dtype="bf16", capacity=0, scoring="sigmoid",
      select_bias_std=0.1, raw_gates=True, seed_index=74),
    # d = 320 (a partial trip of the fused route's K loop), shared expert
    W("sb_t12_e6_gelu_shared", T=12, d_model=320, n_experts=6, top_k=2,
      d_ff=128, act="gelu", dtype="bf16", capacity=0, n_shared=1,
      seed_index=75),
    # the fused route writing logits for overflow reassignment at decode size
    W("sb_t16_reassign", T=16, d_model=128, n_experts=8, top_k=1, d_ff=64,
      act="gelu", dtype="bf16", capacity=1, zipf_s=1.1, seed_index=76,
      overflow="reassign", overflow_seed=5),
    # float32 at decode size
    W("sb_t16_f32", T=16, d_model=64, n_experts=8, top_k=2, d_ff=64,
      act="swiglu", dtype="f32", capacity=0, seed_index=77),
    # the largest batch of the fused route (128 tokens, 256 assignments:
    # the one-workgroup dispatch)
    W("sb_t128_e8", T=128, d_model=128, n_experts=8, top_k=2, d_ff=64,
      act="swiglu", dtype="bf16", capacity=0, seed_index=70),
    # just past the fused route (129 tokens: router GEMM + select)
    W("sb_t129_e8", T=129, d_model=128, n_experts=8, top_k=2, d_ff=64,
      act="swiglu", dtype="bf16", capacity=0, seed_index=71),
]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_small_batch_layer(wl):
    inp = make(wl)
    o = oracle_layer(inp, wl)
    g = gpu_layer(inp, wl)
    idx = host(g["idx"])
    assert idx.tolist() == o["idx"].tolist()
    assert host(g["counts"]).tolist() == o["counts"].tolist()
    assert int(host(g["n_dropped"])[0]) == o["n_dropped"]
    aux = float(host(g["aux"])[0])
    assert abs(aux - o["aux"]) <= AUX_RTOL * abs(o["aux"])
    err = rel_inf(host(g["out"]), o["out"])
    x = host(inp["x"])
    derr = rel_inf(host(g["out"]) - x, o["out"] - x)
    log(f"  {wl.name}: out rel err {err:.2e} (moe delta {derr:.2e}), "
        f"dropped {o['n_dropped']}, reassigned {o.get('n_reassigned', 0)}")
    if "drops" in wl.name:
        assert o["n_dropped"] > 0, "workload must exercise the capacity cut"
    assert err <= TOL[wl.dtype]
    assert derr <= TOL[wl.dtype]
    if wl.overflow == "reassign":
        assert o["n_reassigned"] > 0, "workload must exercise reassignment"
        return
    # the separate entry points agree with the layer
    r = gpu_route(inp, wl)
    assert np.array_equal(host(r["idx"]), idx)
    d = gpu_dispatch(host(r["idx"]), host(r["prob_mean"]), wl)
    assert torch.equal(d["counts"], g["counts"])
    assert torch.equal(d["n_dropped"], g["n_dropped"])
    # repeated calls are bit-identical
    g2 = gpu_layer(inp, wl)
    assert torch.equal(g["out"], g2["out"])
    assert torch.equal(g["aux"], g2["aux"])
