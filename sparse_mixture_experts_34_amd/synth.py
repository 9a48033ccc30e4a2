"""Seeded synthetic workloads for the sparse MoE layer.

This module only draws numbers: it holds the workload shapes and the seeded
random inputs and performs none of the layer's arithmetic.  Both the HIP path
(tests, benchmark) and the CPU oracle (tests) consume the bytes it produces.

Shapes follow the pages: Mixtral 8x7B's expert (d_model 4096, intermediate
14,336, 8 experts, top-2: getnybble.com "Mixture of Experts (MoE)",
"Mixtral 8x7B"), a Switch-style top-1 layer with many experts (same page,
"Load balancing and expert collapse"), and DeepSeek-V3's 256 routed experts,
top-8, plus one always-on shared expert (same page, "DeepSeek-V3").

Distribution readings (no page fixes them):
* ``N(0, 1/d_in)`` is read as a variance (std = 1/sqrt(d_in)); a router
  ``std`` is a standard deviation.
* The Switch layer's Zipf(s) expert popularity is a fixed router-logit bias
  ``-s * ln(e + 1)``: the log of the Zipf mass up to a constant.
* DeepSeek-V3's per-expert selection bias is ``N(0, std)`` float32.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

ACTS = ("gelu", "swiglu")
DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}
BASE_SEED = 20261203


@dataclass(frozen=True)
class Workload:
    name: str
    T: int
    d_model: int
    n_experts: int
    top_k: int
    d_ff: int
    act: str                      # "gelu" | "swiglu"
    dtype: str                    # "f32" | "bf16"
    capacity: int                 # <= 0: no limit
    n_shared: int = 0
    aux_coef: float = 0.01
    router_std: float | None = None   # None: 1/sqrt(d_model)
    zipf_s: float = 0.0               # router bias -s*ln(e+1) when > 0
    select_bias_std: float = 0.0      # > 0: DeepSeek-style selection bias
    seed_index: int = 0
    wquant: str | None = None         # "int4" | "bf16_tiled" (see binding)
    scoring: str = "softmax"          # router scores: softmax | sigmoid
    raw_gates: bool = False           # gates without renormalisation
    overflow: str = "drop"            # drop | reassign (random free slot)
    overflow_seed: int = 0            # key of the reassignment draws
    notes: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def torch_dtype(self):
        return DTYPES[self.dtype]

    def seed(self) -> int:
        return BASE_SEED + self.seed_index

    def sized(self, **kw) -> "Workload":
        """A copy with some sizes changed (name gets a suffix)."""
        tag = ",".join(f"{k}={v}" for k, v in sorted(kw.items()))
        return replace(self, name=f"{self.name}[{tag}]", **kw)


# Capacities below are the integers the capacity rule (ideal share T*k/E
# times the factor, truncated, at least 1) gives at these sizes:
# 64*2/4*1.25 = 40, 16384/64*1.0 = 256, 16384/64*1.25 = 320.
WORKLOADS = {
    "tiny_gelu_f32": Workload(
        "tiny_gelu_f32", T=64, d_model=64, n_experts=4, top_k=2, d_ff=128,
        act="gelu", dtype="f32", capacity=40, seed_index=0),
    "mixtral_decode": Workload(
        "mixtral_decode", T=16, d_model=4096, n_experts=8, top_k=2,
        d_ff=14336, act="swiglu", dtype="bf16", capacity=0,
        router_std=0.02, seed_index=1),
    # the decode layer above with its expert weights in 4 bits (same seed,
    # so the same bf16 weights before quantisation)
    "mixtral_decode_int4": Workload(
        "mixtral_decode_int4", T=16, d_model=4096, n_experts=8, top_k=2,
        d_ff=14336, act="swiglu", dtype="bf16", capacity=0,
        router_std=0.02, seed_index=1, wquant="int4"),
    "mixtral_prefill": Workload(
        "mixtral_prefill", T=8192, d_model=4096, n_experts=8, top_k=2,
        d_ff=14336, act="swiglu", dtype="bf16", capacity=0,
        router_std=0.02, seed_index=2),
    "switch_top1_cf1": Workload(
        "switch_top1_cf1", T=16384, d_model=2048, n_experts=64, top_k=1,
        d_ff=8192, act="gelu", dtype="bf16", capacity=256, zipf_s=1.1,
        seed_index=3),
    "switch_top1_cf125": Workload(
        "switch_top1_cf125", T=16384, d_model=2048, n_experts=64, top_k=1,
        d_ff=8192, act="gelu", dtype="bf16", capacity=320, zipf_s=1.1,
        seed_index=3),
    # the Switch layer at capacity factor 1.0 with overflow reassigned to
    # free slots at random instead of dropped
    "switch_top1_cf1_reassign": Workload(
        "switch_top1_cf1_reassign", T=16384, d_model=2048, n_experts=64,
        top_k=1, d_ff=8192, act="gelu", dtype="bf16", capacity=256,
        zipf_s=1.1, seed_index=3, overflow="reassign",
        overflow_seed=20261203),
    "deepseek_v3": Workload(
        "deepseek_v3", T=4096, d_model=7168, n_experts=256, top_k=8,
        d_ff=2048, act="swiglu", dtype="bf16", capacity=0, n_shared=1,
        select_bias_std=0.1, seed_index=4),
}
# The same layers with their bf16 expert weights stored in the GEMMs' tiled
# order (same seeds, so the same weight values).
for _n in ("mixtral_decode", "mixtral_prefill", "switch_top1_cf1",
           "deepseek_v3"):
    WORKLOADS[_n + "_tiled"] = replace(WORKLOADS[_n], name=_n + "_tiled",
                                       wquant="bf16_tiled")
del _n


def weight_shapes(wl: Workload) -> dict:
    """Shapes of every weight tensor of the layer, ``nn.Linear`` storage
    ([out, in]) stacked over experts."""
    E, d, f = wl.n_experts, wl.d_model, wl.d_ff
    s = {"w_router": (E, d)}
    if wl.act == "gelu":
        s.update(w1=(E, f, d), b1=(E, f), w2=(E, d, f), b2=(E, d))
        if wl.n_shared:
            s.update(shared_w1=(f, d), shared_b1=(f,), shared_w2=(d, f),
                     shared_b2=(d,))
    else:
        s.update(w_gate=(E, f, d), w_up=(E, f, d), w_down=(E, d, f))
        if wl.n_shared:
            s.update(shared_gate=(f, d), shared_up=(f, d),
                     shared_down=(d, f))
    return s


def param_count(wl: Workload, active: bool = False) -> int:
    """Parameter count of the layer's weights (router included).  With
    ``active``, only the k routed experts a token runs plus shared experts
    and the router are counted."""
    shapes = weight_shapes(wl)
    per_expert = 0
    total = 0
    for name, shp in shapes.items():
        n = math.prod(shp)
        if name == "w_router" or name.startswith("shared_"):
            total += n
        else:
            total += n
            per_expert += n // wl.n_experts
    if not active:
        return total
    return total - per_expert * (wl.n_experts - wl.top_k)


def _randn(shape, gen, device, std, dtype):
    t = torch.randn(*shape, generator=gen, device=device,
                    dtype=torch.float32)
    if std != 1.0:
        t.mul_(std)
    return t.to(dtype)


def _row_seed(seed: int, t: int, attempt: int) -> int:
    return (seed * 1_000_003 + t * 7919 + attempt * 104_729) % (2 ** 62)


def make_inputs(wl: Workload, device="cpu", seed: int | None = None,
                margin_fn=None, min_margin: float = 1e-4,
                max_attempts: int = 64) -> dict:
    """Draw every input of the layer for workload ``wl``.

    Draw order on one generator: x, router weight, router/selection bias,
    then per expert e = 0..E-1 its matrices and biases in the order
    (w1|w_gate, w_up, w2|w_down, b1, b2), then the shared expert.  Floats
    are drawn as float32 normals and rounded (RNE) to the workload dtype;
    the router weight and the biases on the router stay float32.

    ``margin_fn(x64, w_router64, k, router_bias64, select_bias64, scoring)``
    may return a per-token top-k margin; tokens at or below ``min_margin``
    get their x row redrawn from a per-(token, attempt) generator.  The number
    of redraws is returned under ``"redraws"``.
    """
    seed = wl.seed() if seed is None else seed
    dev = torch.device(device)
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    dt = wl.torch_dtype
    T, d, E, f = wl.T, wl.d_model, wl.n_experts, wl.d_ff
    out = {}
    out["x"] = _randn((T, d), gen, dev, 1.0, dt)
    rstd = wl.router_std if wl.router_std is not None else 1.0 / math.sqrt(d)
    out["w_router"] = _randn((E, d), gen, dev, rstd, torch.float32)
    out["router_bias"] = None
    if wl.zipf_s > 0:
        rb = torch.tensor([-wl.zipf_s * math.log(e + 1.0) for e in range(E)],
                          dtype=torch.float32)
        out["router_bias"] = rb.to(dev)
    out["select_bias"] = None
    if wl.select_bias_std > 0:
        out["select_bias"] = _randn((E,), gen, dev, wl.select_bias_std,
                                    torch.float32)
    sd, sf = 1.0 / math.sqrt(d), 1.0 / math.sqrt(f)
    if wl.act == "gelu":
        names = [("w1", (f, d), sd), ("w2", (d, f), sf), ("b1", (f,), sd),
                 ("b2", (d,), sf)]
    else:
        names = [("w_gate", (f, d), sd), ("w_up", (f, d), sd),
                 ("w_down", (d, f), sf)]
    for name, shp, _ in names:
        out[name] = torch.empty((E,) + shp, dtype=dt, device=dev)
    for e in range(E):
        for name, shp, std in names:
            out[name][e] = _randn(shp, gen, dev, std, dt)
    if wl.n_shared:
        for name, shp, std in names:
            key = {"w_gate": "shared_gate", "w_up": "shared_up",
                   "w_down": "shared_down"}.get(name, "shared_" + name)
            out[key] = _randn(shp, gen, dev, std, dt)
    out["redraws"] = 0
    if margin_fn is not None and T > 0:
        _redraw_close_tokens(out, wl, seed, dev, margin_fn, min_margin,
                             max_attempts)
    return out


def _host64(t):
    return None if t is None else t.detach().to("cpu", torch.float64).numpy()


def _redraw_close_tokens(inp, wl, seed, dev, margin_fn, min_margin,
                         max_attempts):
    wr = _host64(inp["w_router"])
    rb = _host64(inp["router_bias"])
    sb = _host64(inp["select_bias"])
    x = inp["x"]
    bad = np.nonzero(margin_fn(_host64(x), wr, wl.top_k, rb, sb, wl.scoring)
                     <= min_margin)[0]
    for t in bad:
        t = int(t)
        for attempt in range(max_attempts):
            g = torch.Generator(device=dev)
            g.manual_seed(_row_seed(seed, t, attempt))
            row = _randn((1, wl.d_model), g, dev, 1.0, wl.torch_dtype)
            m = margin_fn(_host64(row), wr, wl.top_k, rb, sb,
                          wl.scoring)[0]
            inp["redraws"] += 1
            if m > min_margin:
                x[t] = row[0]
                break
        else:
            raise RuntimeError(f"token {t}: no row with margin > "
                               f"{min_margin} in {max_attempts} draws")


def host_f32(t):
    """A tensor's values as a float32 numpy array on the host (bf16 values
    are exactly representable in float32)."""
    return None if t is None else t.detach().to("cpu", torch.float32).numpy()


class ExpertView:
    """``[e]`` gives expert e of a stacked device tensor as a host float32
    array, fetched on demand (keeps host memory small for big layers)."""

    def __init__(self, stacked):
        self.t = stacked

    def __getitem__(self, e):
        return host_f32(self.t[e])

    def __len__(self):
        return self.t.shape[0]


def oracle_weights(inp: dict, wl: Workload, lazy: bool = False) -> dict:
    """The weight dict in the form the CPU oracle reads."""
    names = (["w1", "b1", "w2", "b2"] if wl.act == "gelu"
             else ["w_gate", "w_up", "w_down"])
    w = {}
    for n in names:
        w[n] = ExpertView(inp[n]) if lazy else host_f32(inp[n])
    for n in list(inp):
        if n.startswith("shared_"):
            w[n] = host_f32(inp[n])
    return w
