#!/usr/bin/env python3
"""Benchmark of the sparse MoE layer forward pass on one MI355X.

A step is one full layer forward (route, dispatch, expert up and down
GEMMs, combine, aux loss) over one batch of seeded synthetic inputs already
resident in HBM.  The default workload is the Mixtral-shaped decode layer
(T=16 tokens, d_model 4096, 8 SwiGLU experts of d_ff 14336, top-2, bf16).

Prints one JSON line.  Besides the headline tokens/s it reports
  roofline      the dominant kernel's achieved GB/s or TFLOP/s against the
                MI355X peak (HBM 8 TB/s, dense bf16 MFMA 2.5 PFLOP/s), with
                the kernel's duration taken from HIP events recorded on the
                launch stream in a second timed pass that runs the layer as
                its separate C-ABI steps;
  layer_roofline the whole step against max(F / 2.5 PFLOP/s, B / 8 TB/s);
  cpu_baseline  the CPU oracle timed on this host on a bounded sample, with
                the GPU output's error on the sampled tokens;
  mixtral_prefill  (default decode run only) the same record for the
                Mixtral-shaped prefill layer (T=8192), the MFMA-bound half of
                the metric, timed after the decode layer.
"""

from __future__ import annotations

import argparse
import hashlib
import re
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM = 8.0e12          # bytes/s
PEAK_BF16 = 2.5e15         # dense bf16 MFMA FLOP/s
PEAK_F32_VALU = 157.3e12   # fp32 vector FLOP/s
METRIC = ("MoE layer fwd tokens/s + % of bf16 MFMA / HBM roofline "
          "(Mixtral-shaped layer)")
# oracle sample (tokens whose expert outputs the oracle evaluates); routing
# and dispatch of the oracle always cover the whole batch
CPU_SAMPLE = {"mixtral_decode": 16, "mixtral_decode_int4": 2,
              "mixtral_decode_tiled": 16, "mixtral_prefill_tiled": 48,
              "switch_top1_cf1_tiled": 256, "deepseek_v3_tiled": 12,
              "mixtral_prefill": 48,
              "switch_top1_cf1": 256, "switch_top1_cf125": 256,
              "switch_top1_cf1_reassign": 256,
              "deepseek_v3": 12, "tiny_gelu_f32": 64}
# the oracle is timed over whole passes of its sample until this much CPU
# time has run (at most CPU_MAX_PASSES passes)
CPU_SECONDS = 10.0
CPU_MAX_PASSES = 30


def parse():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixtral_decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true",
                    help="with the default decode workload, skip the "
                    "Mixtral-shaped prefill record (the MFMA-bound half)")
    ap.add_argument("--cpu-tokens", type=int, default=None)
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="after the benchmark, run a plain device-to-device "
                    "copy of this many MiB three times (a known-size "
                    "reference for the profiler's HBM byte counters)")
    return ap.parse_args()


# the sources the expert GEMM kernels are compiled from
GEMM_SOURCES = ("common.hpp", "kernels.hpp", "ffn_common.hpp", "ffn.hip",
                "ffn_q4.hip")


def code_only(text: str) -> str:
    """A C++ source without its comments and with its white space collapsed:
    what the compiler sees of it (these sources hold no string literal with
    a comment marker), so a comment-only edit leaves the digest alone."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    return " ".join(text.split())


def kernel_sources_digest() -> str:
    d = os.path.join(ROOT, "sparse_mixture_experts_34_amd", "csrc")
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(f.encode())
        h.update(code_only(open(os.path.join(d, f)).read()).encode())
    return h.hexdigest()[:16]


def load_traffic(workload: str, kernel: str):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 PMC
    summary, if it was taken on the current kernel sources."""
    p = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_pmc.json")
    if not os.path.exists(p):
        return None
    rec = json.load(open(p))
    if rec.get("kernel_sources_digest") != kernel_sources_digest():
        return None
    return rec.get("hbm_bytes_per_launch")


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not "
              "supported (this layer's benchmark is a single-GPU kernel "
              "benchmark; multi-GPU expert parallelism is not built)",
              file=sys.stderr)
        sys.exit(2)

    import torch

    from sparse_mixture_experts_34_amd import synth

    wl = synth.WORKLOADS[args.workload]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    res, bf16_inp, gpu = measure(wl, args.steps, args.warmup, dev)
    res = {"metric": METRIC, **res}
    if args.workload == "mixtral_decode" and not args.no_prefill:
        # the compute-bound half of the metric: the Mixtral-shaped prefill
        # layer, timed the same way after the decode layer
        pre, _, _ = measure(synth.WORKLOADS["mixtral_prefill"],
                            min(args.steps, 20), min(args.warmup, 5), dev)
        torch.cuda.empty_cache()
        res["mixtral_prefill"] = {
            n: pre[n] for n in ("value", "unit", "ms_per_step", "config",
                                "roofline", "layer_roofline", "kernels_us",
                                "step_ms_percentiles", "routing", "steps",
                                "warmup")}
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(wl, bf16_inp, args.cpu_tokens,
                                           gpu_idx=gpu["idx"],
                                           gpu_out=gpu["out"])
    print(json.dumps(res), flush=True)
    if args.copy_calibration_mib > 0:
        copy_calibration(args.copy_calibration_mib)


def measure(wl, steps, warmup, dev):
    """Time one workload: K whole-layer steps (the headline), then the same
    layer as its separate C-ABI steps with HIP events on the launch stream
    (per-kernel durations, dominant-kernel roofline).  Returns the record,
    the bf16 inputs and the GPU's routing and output of the last step."""
    import numpy as np
    import torch

    import sparse_mixture_experts_34_amd as moe
    from sparse_mixture_experts_34_amd import synth

    inp = synth.make_inputs(wl, device=dev)
    p = moe.problem_for(wl)
    ws = moe.workspace(p, dev)
    T, E, k, d, f = wl.T, wl.n_experts, wl.top_k, wl.d_model, wl.d_ff
    rows = T * k + wl.n_shared * T
    dt = wl.torch_dtype
    # Two copies of the expert weights, used on alternate steps: a step's
    # weights were last read two steps earlier, with the other copy read in
    # between, so the 256 MB memory-side cache gives no reuse across steps.
    q4 = wl.wquant == "int4"
    tw = wl.wquant == "bf16_tiled"
    bf16_inp = inp
    if q4:
        # 4-bit expert weights, quantised on the device before timing
        inp = moe.quantize_weights(bf16_inp)
    elif tw:
        # bf16 expert weights in the GEMMs' tiled order, reordered on the
        # device before timing
        inp = moe.tile_weights(bf16_inp)
    wnames = [n for n in inp if n in moe.QUANT_MATRICES or
              n.endswith("_q") or n in ("b1", "b2", "shared_b1", "shared_b2")]
    inp_b = dict(inp)
    for n in wnames:
        if inp[n] is not None:
            inp_b[n] = inp[n].clone()
    Ws = [moe.expert_weights(inp), moe.expert_weights(inp_b)]
    W = Ws[0]

    out = torch.empty_like(inp["x"])
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    counts = torch.empty(E, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)

    def step(i, ev=None):
        if ev is not None:
            ev[0].record()
        moe.moe_layer_forward(p, inp["x"], inp["w_router"],
                              inp["router_bias"], inp["select_bias"],
                              Ws[i & 1], out, aux, counts, nd, None, ws)
        if ev is not None:
            ev[1].record()

    # ---- headline pass: K whole-layer calls ------------------------------
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(i)
    torch.cuda.synchronize()
    t_step = (time.perf_counter() - t0) / steps
    # per-step spread: a second pass with HIP events around every call
    sev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
           for _ in range(steps)]
    for i in range(steps):
        step(i, sev[i])
    torch.cuda.synchronize()
    st = np.array([e[0].elapsed_time(e[1]) for e in sev])

    cnt = counts.cpu().tolist()
    n_dropped = int(nd.item())
    kept_total = T * k - n_dropped
    F, B = moe.flops_and_bytes(wl, cnt, kept_total)
    t_roof = max(F / PEAK_BF16, B / PEAK_HBM)

    # ---- kernel pass: the same layer as its C-ABI steps, HIP events ------
    reassign = wl.overflow == "reassign" and wl.capacity > 0
    logits = (torch.empty(T, E, dtype=torch.float32, device=dev)
              if reassign else None)
    idx = torch.empty(T, k, dtype=torch.int32, device=dev)
    gate = torch.empty(T, k, dtype=torch.float32, device=dev)
    pm = torch.empty(E, dtype=torch.float32, device=dev)
    offs = torch.empty(E + 1, dtype=torch.int32, device=dev)
    perm = torch.empty(T * k, dtype=torch.int32, device=dev)
    slot = torch.empty(T * k, dtype=torch.int32, device=dev)
    h = torch.empty(rows, f, dtype=dt, device=dev)
    y = torch.empty(rows, d, dtype=dt, device=dev)
    out2 = torch.empty_like(out)
    names = ["route", "dispatch", "expert_up", "expert_down", "combine"]

    def step_parts(ev, i):
        W = Ws[i & 1]
        ev[0].record()
        moe.moe_route(p, inp["x"], inp["w_router"], inp["router_bias"],
                      inp["select_bias"], logits, idx, gate, pm, ws)
        ev[1].record()
        if reassign:
            moe.moe_dispatch_reassign(p, idx, gate, logits, pm, counts, offs,
                                      perm, slot, nd, aux, ws)
        else:
            moe.moe_dispatch(p, idx, pm, counts, offs, perm, slot, nd, aux,
                             ws)
        ev[2].record()
        moe.moe_expert_up(p, inp["x"], perm, offs, W, h, ws)
        ev[3].record()
        moe.moe_expert_down(p, h, offs, W, y, ws)
        ev[4].record()
        moe.moe_combine(p, inp["x"], y, slot, gate, out2)
        ev[5].record()

    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(6)]
           for _ in range(steps)]
    for i in range(warmup):
        step_parts(evs[0], i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step_parts(evs[i], i)
    torch.cuda.synchronize()
    t_parts = (time.perf_counter() - t0) / steps
    per = {n: float(np.mean([e[j].elapsed_time(e[j + 1]) for e in evs]))
           * 1e-3 for j, n in enumerate(names)}
    same = bool(torch.equal(out, out2))

    # dominant kernel: the longest single-kernel step (up or down GEMM)
    krn = gemm_work(wl, cnt, kept_total)
    touched = sum(1 for c in cnt if c > 0) + wl.n_shared
    dom = max(krn, key=lambda n: per[n])
    kb, kf, kt = krn[dom]["bytes"], krn[dom]["flops"], per[dom]
    if wl.dtype == "bf16":
        bound = "mfma" if kf / kb > PEAK_BF16 / PEAK_HBM else "hbm"
    else:
        bound = "alu" if kf / kb > PEAK_F32_VALU / PEAK_HBM else "hbm"
    if bound == "hbm":
        achieved, peak, unit = kb / kt / 1e9, PEAK_HBM / 1e9, "GB/s"
    elif bound == "mfma":
        achieved, peak, unit = kf / kt / 1e12, PEAK_BF16 / 1e12, "TFLOP/s"
    else:
        achieved, peak, unit = kf / kt / 1e12, PEAK_F32_VALU / 1e12, \
            "TFLOP/s"
    kname = {"expert_up": "ffn_up", "expert_down": "ffn_down"}[dom]
    roof = {"kernel": kname, "bound": bound, "achieved": round(achieved, 3),
            "peak": peak, "unit": unit, "frac": round(achieved / peak, 4),
            "traffic": load_traffic(wl.name, kname),
            "algorithmic_bytes": kb, "algorithmic_flops": kf,
            "avg_launch_us": round(kt * 1e6, 3)}

    # routing health (production checks the pages recommend)
    uniform = T * k / E
    healthy = all(abs(c - uniform) <= 0.2 * uniform for c in cnt)
    drop_frac = n_dropped / max(T * k, 1)

    res = {
        "value": round(T / t_step, 3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(t_step * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic (seeded; random-init weights of the layer shape)",
        "config": {"workload": wl.name, "T": T, "d_model": d,
                   "n_experts": E, "top_k": k, "d_ff": f, "act": wl.act,
                   "capacity": wl.capacity, "n_shared": wl.n_shared,
                   "expert_weights": "int4 (group 128, fp32 scale/offset)"
                   if q4 else (wl.dtype + " (tiled order)" if tw
                               else wl.dtype),
                   "scoring": wl.scoring, "raw_gates": wl.raw_gates,
                   "overflow": wl.overflow},
        "roofline": roof,
        "layer_roofline": {
            "flops": F, "bytes": B, "t_roof_us": round(t_roof * 1e6, 2),
            "frac": round(t_roof / t_step, 4),
            "tflops": round(F / t_step / 1e12, 2),
            "hbm_gbps": round(B / t_step / 1e9, 1),
            "bound": "mfma" if F / PEAK_BF16 > B / PEAK_HBM else "hbm"},
        "kernels_us": {n: round(v * 1e6, 2) for n, v in per.items()},
        "parts_ms_per_step": round(t_parts * 1e3, 4),
        "step_ms_percentiles": {
            "p10": round(float(np.percentile(st, 10)), 4),
            "p50": round(float(np.percentile(st, 50)), 4),
            "p90": round(float(np.percentile(st, 90)), 4)},
        "weight_copies": 2,
        "parts_match_layer_output": same,
        "routing": {"counts": cnt, "touched_experts": touched - wl.n_shared,
                    "kept_assignments": kept_total,
                    "n_dropped": n_dropped,
                    "drop_fraction": round(drop_frac, 5),
                    "within_20pct_of_uniform": healthy,
                    "drop_alert_over_2pct": drop_frac > 0.02,
                    "aux_loss": float(aux.item())},
    }
    gpu = {"idx": idx.cpu().numpy(), "out": out.float().cpu().numpy()}
    return res, bf16_inp, gpu


def copy_calibration(mib):
    """A plain copy of known size: reads and writes mib MiB per launch."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes": n * 4}), flush=True)


def kept_total_rows(kept_total, wl):
    return kept_total + wl.n_shared * wl.T


def gemm_work(wl, counts, kept_total):
    """Algorithmic bytes and FLOPs of each expert GEMM launch: the touched
    experts' weights (and GELU biases) once, plus the rows it reads and
    writes (A rows of K elements, output rows of N); 2 FLOPs per
    multiply-add over the kept and shared rows."""
    d, f = wl.d_model, wl.d_ff
    esz = 2 if wl.dtype == "bf16" else 4
    touched = sum(1 for c in counts if c > 0) + wl.n_shared
    nmat_up = 2 if wl.act == "swiglu" else 1
    if wl.wquant == "int4":
        # codes (half a byte per weight) + float32 (scale, offset) per 128
        qb = lambda n: n // 2 + (n // 128) * 8
        up_w = touched * (nmat_up * qb(f * d) +
                          (f * esz if wl.act == "gelu" else 0))
        dn_w = touched * (qb(d * f) + (d * esz if wl.act == "gelu" else 0))
    else:
        up_w = touched * (nmat_up * f * d +
                          (f if wl.act == "gelu" else 0)) * esz
        dn_w = touched * (d * f + (d if wl.act == "gelu" else 0)) * esz
    rows = kept_total_rows(kept_total, wl)
    return {
        "expert_up": {"bytes": up_w + rows * (d + f) * esz,
                      "flops": 2 * rows * d * f * nmat_up},
        "expert_down": {"bytes": dn_w + rows * (f + d) * esz,
                        "flops": 2 * rows * d * f},
    }


def cpu_baseline(wl, inp, n_tokens=None, gpu_idx=None, gpu_out=None):
    """The CPU oracle (float64, numpy/OpenBLAS) on a bounded sample: routing
    and capacity dispatch over the whole batch plus the expert FFNs and
    combine of a token sample.  Weights are copied to host memory before
    the clock starts.  With ``gpu_idx``, also counts the tokens whose
    selected experts differ from the oracle's (expected 0); with
    ``gpu_out`` (the GPU layer's output, host array), reports its error on
    the sampled tokens: max |gpu - oracle| / max |oracle| of the output and
    of its MoE part (output minus residual)."""
    import numpy as np
    import torch
    from threadpoolctl import threadpool_info

    import oracle
    from sparse_mixture_experts_34_amd import synth

    n = min(n_tokens or CPU_SAMPLE.get(wl.name, 16), wl.T)
    rng = np.random.default_rng(0)
    tokens = np.sort(rng.choice(wl.T, n, replace=False))
    hx = lambda t: None if t is None else t.to("cpu", torch.float32).numpy()
    x, wr = hx(inp["x"]), hx(inp["w_router"])
    rb, sb = hx(inp["router_bias"]), hx(inp["select_bias"])
    # route once (untimed) to find the experts the sample needs
    renorm = not wl.raw_gates
    reseed = wl.overflow_seed if wl.overflow == "reassign" else None
    r = oracle.route(x, wr, wl.top_k, rb, sb, wl.scoring, renorm)
    ridx = r["idx"]
    if reseed is not None and wl.capacity > 0:
        ridx = oracle.dispatch_reassign(r["idx"], r["scores"], r["gate"],
                                        wl.n_experts, wl.capacity, reseed,
                                        renorm)["idx"]
    need = sorted(set(int(e) for e in ridx[tokens].ravel()))
    flips = None
    if gpu_idx is not None:
        flips = int((np.asarray(gpu_idx) != ridx).any(axis=1).sum())
    names = (["w1", "b1", "w2", "b2"] if wl.act == "gelu"
             else ["w_gate", "w_up", "w_down"])
    w = {}
    # 4-bit weights: the oracle evaluates the weights its own codes
    # represent (quantised and dequantised here, before the clock starts)
    q4 = wl.wquant == "int4"

    def prep(a, name):
        if not q4 or name.startswith("b") or name.startswith("shared_b"):
            return a
        q, sc, off = oracle.quantize_int4(a.reshape(-1, a.shape[-1]))
        return oracle.dequantize_int4(q, sc, off).reshape(a.shape)

    for nme in names:
        full = {}
        for e in need:
            full[e] = prep(hx(inp[nme][e]), nme)
        w[nme] = full
    for nme in list(inp):
        if nme.startswith("shared_"):
            w[nme] = prep(hx(inp[nme]), nme)
    def run():
        return oracle.layer_forward(x, wr, w, k=wl.top_k, cap=wl.capacity,
                                    act=wl.act, n_shared=wl.n_shared,
                                    alpha=wl.aux_coef, router_bias=rb,
                                    select_bias=sb, tokens=tokens,
                                    scoring=wl.scoring, renormalize=renorm,
                                    reassign_seed=reseed)

    # whole passes over the sample until about CPU_SECONDS of work (a batch
    # smaller than that is timed over repeated passes)
    t0 = time.perf_counter()
    o = run()
    dt = time.perf_counter() - t0
    passes = 1
    while dt < CPU_SECONDS and passes < CPU_MAX_PASSES:
        t0 = time.perf_counter()
        run()
        dt += time.perf_counter() - t0
        passes += 1
    threads = max([i.get("num_threads", 1) for i in threadpool_info()
                   if i.get("internal_api") in ("openblas", "mkl", "blis")]
                  or [1])
    errs = {}
    if gpu_out is not None:
        def rel(a, b):
            den = np.abs(b).max()
            return float(np.abs(a - b).max() / den) if den else 0.0
        g = np.asarray(gpu_out, np.float64)[tokens]
        xs = np.asarray(x, np.float64)[tokens]
        errs = {"out_rel_err_vs_gpu": rel(g, o["out"]),
                "moe_delta_rel_err_vs_gpu": rel(g - xs, o["out"] - xs)}
    return {"value": round(n * passes / dt, 4), "unit": "tokens/s",
            "cores": len(os.sched_getaffinity(0)), "blas_threads": threads,
            "kind": "oracle", "seconds": round(dt, 3), "passes": passes,
            "routing_flips_vs_gpu": flips, **errs,
            "sample": ("4-bit weights quantised and dequantised by the oracle "
                       "before timing; " if q4 else "") +
                      f"{n} of {wl.T} tokens: float64 routing + capacity "
                      f"dispatch over all {wl.T} tokens, expert FFNs and "
                      f"combine for the {n} sampled tokens, {passes} "
                      f"timed passes"}


if __name__ == "__main__":
    main()
