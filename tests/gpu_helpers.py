"""Helpers for the GPU parity tests: run each C-ABI step through the Python
binding and compute the oracle's answer on the same seeded inputs."""

from __future__ import annotations

import sys
import time

import numpy as np
import torch

import oracle
import sparse_mixture_experts_34_amd as moe
from sparse_mixture_experts_34_amd import synth

# Output tolerance: max |gpu - oracle| / max |oracle| over the tensor.
TOL = {"bf16": 2e-2, "f32": 1e-4}
GATE_TOL = 1e-5
AUX_RTOL = 1e-4


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def rel_inf(a, b) -> float:
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if b.size == 0:
        return 0.0
    den = np.abs(b).max()
    if den == 0:
        return float(np.abs(a).max())
    return float(np.abs(a - b).max() / den)


def host(t):
    return t.detach().to("cpu").numpy() if t.dtype != torch.bfloat16 else \
        t.detach().to("cpu", torch.float32).numpy()


def make(wl, margin=True, device="cuda"):
    t0 = time.time()
    inp = synth.make_inputs(wl, device=device,
                            margin_fn=oracle.topk_margin if margin else None)
    log(f"  inputs {wl.name}: {time.time() - t0:.1f}s, "
        f"redraws={inp['redraws']}")
    return inp


def oracle_route(inp, wl):
    return oracle.route(host(inp["x"]), host(inp["w_router"]), wl.top_k,
                        None if inp["router_bias"] is None
                        else host(inp["router_bias"]),
                        None if inp["select_bias"] is None
                        else host(inp["select_bias"]),
                        scoring=wl.scoring, renormalize=not wl.raw_gates)


def gpu_route(inp, wl, ws=None):
    p = moe.problem_for(wl)
    dev = inp["x"].device
    ws = moe.workspace(p, dev) if ws is None else ws
    T, E, k = wl.T, wl.n_experts, wl.top_k
    out = {
        "logits": torch.full((T, E), float("nan"), device=dev),
        "idx": torch.full((T, k), -7, dtype=torch.int32, device=dev),
        "gate": torch.full((T, k), float("nan"), device=dev),
        "prob_mean": torch.full((E,), float("nan"), device=dev),
    }
    moe.moe_route(p, inp["x"], inp["w_router"], inp["router_bias"],
                  inp["select_bias"], out["logits"], out["idx"], out["gate"],
                  out["prob_mean"], ws)
    torch.cuda.synchronize()
    return out


def gpu_dispatch(idx_np, prob_mean_np, wl, ws=None, device="cuda"):
    p = moe.problem_for(wl)
    ws = moe.workspace(p, device) if ws is None else ws
    T, E, k = wl.T, wl.n_experts, wl.top_k
    idx = torch.as_tensor(np.asarray(idx_np, np.int32).reshape(T, k),
                          device=device)
    pm = torch.as_tensor(np.asarray(prob_mean_np, np.float32), device=device)
    out = {
        "counts": torch.full((E,), -7, dtype=torch.int32, device=device),
        "offsets": torch.full((E + 1,), -7, dtype=torch.int32, device=device),
        "perm": torch.full((max(T * k, 1),), -7, dtype=torch.int32,
                           device=device),
        "slot_of": torch.full((max(T * k, 1),), -7, dtype=torch.int32,
                              device=device),
        "n_dropped": torch.full((1,), -7, dtype=torch.int32, device=device),
        "aux": torch.full((1,), float("nan"), device=device),
    }
    moe.moe_dispatch(p, idx, pm, out["counts"], out["offsets"], out["perm"],
                     out["slot_of"], out["n_dropped"], out["aux"], ws)
    torch.cuda.synchronize()
    return out


def check_dispatch(g, o, wl):
    T, k = wl.T, wl.top_k
    assert host(g["counts"]).tolist() == o["counts"].tolist()
    assert host(g["offsets"]).tolist() == o["offsets"].tolist()
    total = int(o["offsets"][-1])
    perm = host(g["perm"])
    assert perm[:total].tolist() == o["perm"].tolist()
    assert (perm[total:T * k] == -1).all()
    assert host(g["slot_of"])[:T * k].tolist() == o["slot_of"].tolist()
    assert int(host(g["n_dropped"])[0]) == o["n_dropped"]


def rows_of(o, wl):
    """Rows of y the GPU writes: routed rows [0, offsets[E]) and shared."""
    total = int(o["offsets"][-1])
    r = list(range(total))
    if wl.n_shared:
        r += list(range(wl.T * wl.top_k, wl.T * wl.top_k + wl.T))
    return np.asarray(r, np.int64)


def gpu_expert_ffn(inp, perm_np, offsets_np, wl, ws=None):
    p = moe.problem_for(wl)
    dev = inp["x"].device
    ws = moe.workspace(p, dev) if ws is None else ws
    rows = wl.T * wl.top_k + wl.n_shared * wl.T
    y = torch.full((rows, wl.d_model), float("nan"), dtype=wl.torch_dtype,
                   device=dev)
    perm = torch.full((max(wl.T * wl.top_k, 1),), -1, dtype=torch.int32,
                      device=dev)
    pn = np.asarray(perm_np, np.int32)
    if pn.size:
        perm[:pn.size] = torch.as_tensor(pn, device=dev)
    offs = torch.as_tensor(np.asarray(offsets_np, np.int32), device=dev)
    moe.moe_expert_ffn(p, inp["x"], perm, offs, inp, y, ws)
    torch.cuda.synchronize()
    return y


def gpu_combine(inp, y_np, slot_np, gate_np, wl, residual=True):
    p = moe.problem_for(wl)
    dev = inp["x"].device
    y = torch.as_tensor(np.asarray(y_np, np.float32), device=dev) \
        .to(wl.torch_dtype)
    slot = torch.as_tensor(np.asarray(slot_np, np.int32), device=dev)
    gate = torch.as_tensor(np.asarray(gate_np, np.float32), device=dev)
    out = torch.full_like(inp["x"], float("nan"))
    moe.moe_combine(p, inp["x"] if residual else None, y, slot, gate, out)
    torch.cuda.synchronize()
    return out, host(y)


def gpu_layer(inp, wl, ws=None):
    p = moe.problem_for(wl)
    dev = inp["x"].device
    ws = moe.workspace(p, dev) if ws is None else ws
    T, E, k = wl.T, wl.n_experts, wl.top_k
    res = {
        "out": torch.full_like(inp["x"], float("nan")),
        "aux": torch.full((1,), float("nan"), device=dev),
        "counts": torch.full((E,), -7, dtype=torch.int32, device=dev),
        "n_dropped": torch.full((1,), -7, dtype=torch.int32, device=dev),
        "idx": torch.full((max(T, 1), k), -7, dtype=torch.int32, device=dev),
    }
    moe.moe_layer_forward(p, inp["x"], inp["w_router"], inp["router_bias"],
                          inp["select_bias"], inp, res["out"], res["aux"],
                          res["counts"], res["n_dropped"], res["idx"], ws)
    torch.cuda.synchronize()
    return res


def oracle_layer(inp, wl, tokens=None, lazy=False):
    return oracle.layer_forward(
        host(inp["x"]), host(inp["w_router"]),
        synth.oracle_weights(inp, wl, lazy=lazy), k=wl.top_k,
        cap=wl.capacity, act=wl.act, n_shared=wl.n_shared,
        alpha=wl.aux_coef,
        router_bias=None if inp["router_bias"] is None
        else host(inp["router_bias"]),
        select_bias=None if inp["select_bias"] is None
        else host(inp["select_bias"]),
        tokens=tokens, scoring=wl.scoring, renormalize=not wl.raw_gates,
        reassign_seed=wl.overflow_seed if wl.overflow == "reassign"
        else None)
