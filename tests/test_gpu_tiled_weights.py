"""bf16 expert weights in the GEMMs' tiled order (MOE_WQUANT_BF16_TILED).

moe_tile_bf16 is a permutation; it is checked bit for bit against the
order its header defines, written here with numpy reshapes (tile (rb, kb)
of 16 rows x 32 columns at tile index rb*(K/32) + kb, piece 16*q + r =
row 16*rb + r, columns 32*kb + 8*q .. +8).  The layer with tiled weights
is compared with the CPU oracle on the row-major weights, on every bf16
schedule (stream, panel, tiled), to the bf16 tolerance, and routing,
counts and drops bit for bit."""

import numpy as np
import pytest
import torch

from gpu_helpers import (AUX_RTOL, TOL, gpu_layer, host, log, make,
                         oracle_layer, rel_inf)
import sparse_mixture_experts_34_amd as moe
from sparse_mixture_experts_34_amd import synth

pytestmark = pytest.mark.gpu

W = synth.Workload


def tiled_reference(w):
    """The tiled order of a [rows, K] bf16 array (as uint16 bits)."""
    rows, K = w.shape
    t = w.reshape(rows // 16, 16, K // 32, 4, 8).transpose(0, 2, 3, 1, 4)
    return np.ascontiguousarray(t).reshape(rows, K)


@pytest.mark.parametrize("rows,K", [(16, 32), (48, 96), (256, 4096),
                                    (8 * 64, 192)])
def test_tile_bf16_bit_exact(rows, K):
    g = torch.Generator(device="cpu").manual_seed(rows * 7 + K)
    w = torch.randn(rows, K, generator=g).to(torch.bfloat16)
    out = torch.full_like(w, float("nan")).cuda()
    moe.moe_tile_bf16(w.cuda(), out)
    torch.cuda.synchronize()
    got = out.cpu().view(torch.int16).numpy()
    want = tiled_reference(w.view(torch.int16).numpy())
    assert np.array_equal(got, want)


CASES = [
    # stream: T*k <= 64*E
    W("tw_stream_swiglu", T=40, d_model=256, n_experts=8, top_k=2, d_ff=512,
      act="swiglu", dtype="bf16", capacity=0, seed_index=60,
      wquant="bf16_tiled"),
    W("tw_stream_gelu_shared", T=24, d_model=192, n_experts=4, top_k=2,
      d_ff=320, act="gelu", dtype="bf16", capacity=0, n_shared=1,
      seed_index=61, wquant="bf16_tiled"),
    # panel: 64*E < T*k <= 256*E (partial last weight block: d_ff 320)
    W("tw_panel_swiglu_shared", T=500, d_model=192, n_experts=4, top_k=2,
      d_ff=320, act="swiglu", dtype="bf16", capacity=0, n_shared=1,
      seed_index=62, wquant="bf16_tiled"),
    W("tw_panel_gelu_drops", T=3000, d_model=256, n_experts=16, top_k=1,
      d_ff=448, act="gelu", dtype="bf16", capacity=200, zipf_s=0.3,
      seed_index=63, wquant="bf16_tiled"),
    # tiled: T*k > 256*E, ragged M, partial N blocks; the up GEMM's last
    # round split along K (K = 4096: 4 tiles left per XCD, 8 pieces)
    W("tw_tiled_swiglu", T=2200, d_model=4096, n_experts=2, top_k=1,
      d_ff=384, act="swiglu", dtype="bf16", capacity=0, seed_index=64,
      wquant="bf16_tiled"),
    W("tw_tiled_gelu_shared_drops", T=2100, d_model=320, n_experts=2,
      top_k=2, d_ff=384, act="gelu", dtype="bf16", capacity=2000,
      n_shared=1, seed_index=65, wquant="bf16_tiled"),
]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_tiled_weights_layer(wl):
    inp = make(wl)
    o = oracle_layer(inp, wl)
    g = gpu_layer(moe.tile_weights(inp), wl)
    assert host(g["idx"]).tolist() == o["idx"].tolist()
    assert host(g["counts"]).tolist() == o["counts"].tolist()
    assert int(host(g["n_dropped"])[0]) == o["n_dropped"]
    aux = float(host(g["aux"])[0])
    assert abs(aux - o["aux"]) <= AUX_RTOL * abs(o["aux"])
    out = host(g["out"])
    err = rel_inf(out, o["out"])
    x = host(inp["x"])
    derr = rel_inf(out - x, o["out"] - x)
    log(f"  {wl.name}: out rel err {err:.2e} (moe delta {derr:.2e})")
    assert np.isfinite(out).all()
    assert err <= TOL["bf16"]
    assert derr <= TOL["bf16"]


@pytest.mark.parametrize("name", ["deepseek_v3_tiled", "mixtral_prefill_tiled"])
def test_tiled_weights_full_size_sampled(name):
    wl = synth.WORKLOADS[name]
    torch.cuda.empty_cache()
    inp = make(wl)
    g = gpu_layer(moe.tile_weights(inp), wl)
    tokens = np.array([0, 1, wl.T // 2, wl.T - 1])
    o = oracle_layer(inp, wl, tokens=tokens, lazy=True)
    assert host(g["idx"]).tolist() == o["idx"].tolist()
    assert host(g["counts"]).tolist() == o["counts"].tolist()
    out = host(g["out"][torch.as_tensor(tokens, device="cuda")])
    err = rel_inf(out, o["out"])
    log(f"  {name}: sampled out rel err {err:.2e}")
    assert err <= TOL["bf16"]
