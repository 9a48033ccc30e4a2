"""MI355X (gfx950) sparse mixture-of-experts layer forward pass.

Thin Python binding over the C ABI of ``libmoe.so`` (declared in
``include/moe.h``).  The functions below have the C entry points' names and
only marshal arguments: tensors become device pointers, ``None`` becomes
NULL, and the stream defaults to torch's current stream.  Every step of the
layer runs in the HIP kernels; there is no Python or CPU fallback.  If the
library is not built the import of the binding fails loudly.

PyTorch is used only for device memory and streams.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch  # must precede the library load: one HIP runtime per process

from . import synth  # noqa: F401  (seeded workloads)

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK, MOE_EINVAL, MOE_ENOTSUP, MOE_EWORKSPACE, MOE_EHIP = 0, -1, -2, -3, -4
MOE_ACT_GELU, MOE_ACT_SWIGLU = 0, 1
MOE_DTYPE_F32, MOE_DTYPE_BF16 = 0, 1
MOE_WQUANT_NONE, MOE_WQUANT_INT4, MOE_WQUANT_BF16_TILED = 0, 1, 2
MOE_SCORING_SOFTMAX, MOE_SCORING_SIGMOID = 0, 1
MOE_OVERFLOW_DROP, MOE_OVERFLOW_REASSIGN = 0, 1
OVERFLOW = {"drop": MOE_OVERFLOW_DROP, "reassign": MOE_OVERFLOW_REASSIGN}
SCORING = {"softmax": MOE_SCORING_SOFTMAX, "sigmoid": MOE_SCORING_SIGMOID}
MOE_Q4_GROUP = 128
MOE_NOALLOC_SCRATCH_BYTES = 32 << 20
WQUANT = {None: MOE_WQUANT_NONE, "none": MOE_WQUANT_NONE,
          "int4": MOE_WQUANT_INT4, "bf16_tiled": MOE_WQUANT_BF16_TILED}
ACT = {"gelu": MOE_ACT_GELU, "swiglu": MOE_ACT_SWIGLU}
DTYPE = {"f32": MOE_DTYPE_F32, "bf16": MOE_DTYPE_BF16}
TORCH_DTYPE = {MOE_DTYPE_F32: torch.float32, MOE_DTYPE_BF16: torch.bfloat16}


class MoEError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {moe_status_string(status)} ({status})")


class moe_problem(ctypes.Structure):
    _fields_ = [("T", ctypes.c_int32), ("d_model", ctypes.c_int32),
                ("n_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("d_ff", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("capacity", ctypes.c_int32), ("act", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("aux_coef", ctypes.c_float),
                ("wquant", ctypes.c_int32), ("scoring", ctypes.c_int32),
                ("raw_gates", ctypes.c_int32), ("overflow", ctypes.c_int32),
                ("overflow_seed", ctypes.c_uint64)]


class moe_expert_weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("w1", "w_up", "w2", "b1", "b2", "shared_w1", "shared_w_up",
                 "shared_w2", "shared_b1", "shared_b2", "w1_q", "w_up_q",
                 "w2_q", "shared_w1_q", "shared_w_up_q", "shared_w2_q")]


_P = ctypes.POINTER(moe_problem)
_W = ctypes.POINTER(moe_expert_weights)
_V = ctypes.c_void_p
_SZ = ctypes.c_size_t
_I32 = ctypes.c_int32

_SIGS = {
    "moe_capacity": (_I32, [_I32, _I32, _I32, _I32, _I32]),
    "moe_workspace_bytes": (_I32, [_P, ctypes.POINTER(_SZ)]),
    "moe_route": (_I32, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, _SZ, _V]),
    "moe_dispatch": (_I32, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V, _SZ,
                            _V]),
    "moe_expert_ffn": (_I32, [_P, _V, _V, _V, _W, _V, _V, _SZ, _V]),
    "moe_expert_up": (_I32, [_P, _V, _V, _V, _W, _V, _V, _SZ, _V]),
    "moe_expert_down": (_I32, [_P, _V, _V, _W, _V, _V, _SZ, _V]),
    "moe_combine": (_I32, [_P, _V, _V, _V, _V, _V, _V]),
    "moe_layer_forward": (_I32, [_P, _V, _V, _V, _V, _W, _V, _V, _V, _V, _V,
                                 _V, _SZ, _V]),
    "moe_layer_forward_noalloc": (_I32, [_P, _V, _V, _V, _V, _W, _V, _V, _V,
                                         _V, _V, _V]),
    "moe_quantize_int4": (_I32, [_V, ctypes.c_int64, _I32, _V, _V, _V]),
    "moe_tile_bf16": (_I32, [_V, ctypes.c_int64, _I32, _V, _V]),
    "moe_update_select_bias": (_I32, [_P, _V, _V, ctypes.c_float, _V]),
    "moe_dispatch_reassign": (_I32, [_P, _V, _V, _V, _V, _V, _V, _V, _V, _V,
                                     _V, _V, _SZ, _V]),
    "moe_status_string": (ctypes.c_char_p, [_I32]),
}
EXPORTS = tuple(_SIGS)


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is not built; run "
            "`python -m sparse_mixture_experts_34_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = _load()


def library_path() -> str:
    return LIB_PATH


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------

def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


_F32, _I32T, _U8 = torch.float32, torch.int32, torch.uint8


def _arg(t, dtype, name):
    """Device pointer of a tensor argument after checking what the C side
    cannot see: the tensor lives on a GPU, is contiguous and has the
    element type the entry point reads.  ``None`` is NULL and a plain int
    is taken as a raw device address (unchecked)."""
    if t is None or isinstance(t, int):
        return _ptr(t)
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch.Tensor, got {type(t)}")
    if t.device.type != "cuda":
        raise ValueError(f"{name}: must be a GPU tensor (got {t.device})")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous (row-major)")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    return t.data_ptr()


def _ws(ws):
    """(pointer, bytes) of a workspace tensor; it is counted in bytes, so
    it must be uint8."""
    if ws is None:
        return None, 0
    return _arg(ws, _U8, "ws"), ws.numel()


def _act(p):
    """torch dtype of the problem's activations, experts and outputs."""
    return TORCH_DTYPE.get(p.dtype)


def _weights(p, weights):
    """The C weights struct, each tensor checked for device, contiguity and
    the element type the problem's weight format implies."""
    if isinstance(weights, moe_expert_weights):
        return weights
    act = _act(p)
    mat = _U8 if p.wquant == MOE_WQUANT_INT4 else act
    for n, t in weights.items():
        if not isinstance(t, torch.Tensor):
            continue
        if n in QUANT_MATRICES:
            _arg(t, mat, n)
        elif n.endswith("_q") and n[:-2] in QUANT_MATRICES:
            _arg(t, _F32, n)
        elif n in ("b1", "b2", "shared_b1", "shared_b2"):
            _arg(t, act, n)
    return expert_weights(weights)


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status, where):
    if status != MOE_OK:
        raise MoEError(status, where)


def problem(T, d_model, n_experts, top_k, d_ff, *, n_shared=0, capacity=0,
            act="swiglu", dtype="bf16", aux_coef=0.01,
            wquant=None, scoring="softmax",
            raw_gates=False, overflow="drop",
            overflow_seed=0) -> moe_problem:
    return moe_problem(T, d_model, n_experts, top_k, d_ff, n_shared, capacity,
                       ACT[act] if isinstance(act, str) else act,
                       DTYPE[dtype] if isinstance(dtype, str) else dtype,
                       aux_coef,
                       WQUANT[wquant] if not isinstance(wquant, int)
                       else wquant,
                       SCORING[scoring] if isinstance(scoring, str)
                       else scoring, int(raw_gates),
                       OVERFLOW[overflow] if isinstance(overflow, str)
                       else overflow, int(overflow_seed))


def problem_for(wl) -> moe_problem:
    """The C problem struct of a :class:`synth.Workload`."""
    return problem(wl.T, wl.d_model, wl.n_experts, wl.top_k, wl.d_ff,
                   n_shared=wl.n_shared, capacity=wl.capacity, act=wl.act,
                   dtype=wl.dtype, aux_coef=wl.aux_coef,
                   wquant=getattr(wl, "wquant", None),
                   scoring=getattr(wl, "scoring", "softmax"),
                   raw_gates=getattr(wl, "raw_gates", False),
                   overflow=getattr(wl, "overflow", "drop"),
                   overflow_seed=getattr(wl, "overflow_seed", 0))


def expert_weights(w: dict) -> moe_expert_weights:
    """C weights struct from a dict of device tensors keyed like the
    layer's weights (w1/w2/b1/b2 or w_gate/w_up/w_down, shared_*).  For
    4-bit weights the matrices hold codes and ``<name>_q`` their
    (scale, offset) pairs."""
    get = lambda *names: next((_ptr(w[n]) for n in names
                               if w.get(n) is not None), None)
    q = lambda *names: get(*[n + "_q" for n in names])
    return moe_expert_weights(
        get("w1", "w_gate"), get("w_up"), get("w2", "w_down"), get("b1"),
        get("b2"), get("shared_w1", "shared_gate"), get("shared_up"),
        get("shared_w2", "shared_down"), get("shared_b1"), get("shared_b2"),
        q("w1", "w_gate"), q("w_up"), q("w2", "w_down"),
        q("shared_w1", "shared_gate"), q("shared_up"),
        q("shared_w2", "shared_down"))


# ---------------------------------------------------------------------------
# the C entry points
# ---------------------------------------------------------------------------

def moe_status_string(status: int) -> str:
    return _lib.moe_status_string(status).decode()


def moe_capacity(T, top_k, n_experts, cf_num, cf_den) -> int:
    return int(_lib.moe_capacity(T, top_k, n_experts, cf_num, cf_den))


def moe_workspace_bytes(p: moe_problem) -> int:
    n = _SZ(0)
    _check(_lib.moe_workspace_bytes(ctypes.byref(p), ctypes.byref(n)),
           "moe_workspace_bytes")
    return n.value


def workspace(p: moe_problem, device="cuda") -> torch.Tensor:
    """A workspace tensor of the size the library asks for (256-byte
    aligned: torch's caching allocator aligns blocks to 512 bytes)."""
    n = moe_workspace_bytes(p)
    ws = torch.empty(max(n, 1), dtype=torch.uint8, device=device)
    assert ws.data_ptr() % 256 == 0
    return ws


def moe_route(p, x, w_router, router_bias, select_bias, logits, topk_idx,
              topk_gate, prob_mean, ws, stream=None):
    wp, wn = _ws(ws)
    _check(_lib.moe_route(ctypes.byref(p), _arg(x, _act(p), "x"),
                          _arg(w_router, _F32, "w_router"),
                          _arg(router_bias, _F32, "router_bias"),
                          _arg(select_bias, _F32, "select_bias"),
                          _arg(logits, _F32, "logits"),
                          _arg(topk_idx, _I32T, "topk_idx"),
                          _arg(topk_gate, _F32, "topk_gate"),
                          _arg(prob_mean, _F32, "prob_mean"), wp, wn,
                          _stream(stream)), "moe_route")


def moe_dispatch(p, topk_idx, prob_mean, counts, offsets, perm, slot_of,
                 n_dropped, aux_loss, ws, stream=None):
    wp, wn = _ws(ws)
    _check(_lib.moe_dispatch(ctypes.byref(p),
                             _arg(topk_idx, _I32T, "topk_idx"),
                             _arg(prob_mean, _F32, "prob_mean"),
                             _arg(counts, _I32T, "counts"),
                             _arg(offsets, _I32T, "offsets"),
                             _arg(perm, _I32T, "perm"),
                             _arg(slot_of, _I32T, "slot_of"),
                             _arg(n_dropped, _I32T, "n_dropped"),
                             _arg(aux_loss, _F32, "aux_loss"), wp, wn,
                             _stream(stream)), "moe_dispatch")


def moe_expert_ffn(p, x, perm, offsets, weights, y, ws, stream=None):
    w = _weights(p, weights)
    wp, wn = _ws(ws)
    _check(_lib.moe_expert_ffn(ctypes.byref(p), _arg(x, _act(p), "x"),
                               _arg(perm, _I32T, "perm"),
                               _arg(offsets, _I32T, "offsets"),
                               ctypes.byref(w), _arg(y, _act(p), "y"), wp, wn,
                               _stream(stream)), "moe_expert_ffn")


def moe_expert_up(p, x, perm, offsets, weights, h, ws=None, stream=None):
    w = _weights(p, weights)
    wp, wn = _ws(ws)
    _check(_lib.moe_expert_up(ctypes.byref(p), _arg(x, _act(p), "x"),
                              _arg(perm, _I32T, "perm"),
                              _arg(offsets, _I32T, "offsets"),
                              ctypes.byref(w), _arg(h, _act(p), "h"), wp, wn,
                              _stream(stream)), "moe_expert_up")


def moe_expert_down(p, h, offsets, weights, y, ws=None, stream=None):
    w = _weights(p, weights)
    wp, wn = _ws(ws)
    _check(_lib.moe_expert_down(ctypes.byref(p), _arg(h, _act(p), "h"),
                                _arg(offsets, _I32T, "offsets"),
                                ctypes.byref(w), _arg(y, _act(p), "y"), wp,
                                wn, _stream(stream)), "moe_expert_down")


def moe_combine(p, x_residual, y, slot_of, topk_gate, out, stream=None):
    _check(_lib.moe_combine(ctypes.byref(p),
                            _arg(x_residual, _act(p), "x_residual"),
                            _arg(y, _act(p), "y"),
                            _arg(slot_of, _I32T, "slot_of"),
                            _arg(topk_gate, _F32, "topk_gate"),
                            _arg(out, _act(p), "out"),
                            _stream(stream)), "moe_combine")


def moe_layer_forward(p, x, w_router, router_bias, select_bias, weights, out,
                      aux_loss, counts, n_dropped, topk_idx, ws,
                      stream=None):
    w = _weights(p, weights)
    wp, wn = _ws(ws)
    _check(_lib.moe_layer_forward(ctypes.byref(p), _arg(x, _act(p), "x"),
                                  _arg(w_router, _F32, "w_router"),
                                  _arg(router_bias, _F32, "router_bias"),
                                  _arg(select_bias, _F32, "select_bias"),
                                  ctypes.byref(w), _arg(out, _act(p), "out"),
                                  _arg(aux_loss, _F32, "aux_loss"),
                                  _arg(counts, _I32T, "counts"),
                                  _arg(n_dropped, _I32T, "n_dropped"),
                                  _arg(topk_idx, _I32T, "topk_idx"), wp, wn,
                                  _stream(stream)), "moe_layer_forward")


def moe_layer_forward_noalloc(p, x, w_router, router_bias, select_bias,
                              weights, out, aux_loss, counts, n_dropped,
                              topk_idx, stream=None):
    w = _weights(p, weights)
    _check(_lib.moe_layer_forward_noalloc(
        ctypes.byref(p), _arg(x, _act(p), "x"),
        _arg(w_router, _F32, "w_router"),
        _arg(router_bias, _F32, "router_bias"),
        _arg(select_bias, _F32, "select_bias"), ctypes.byref(w),
        _arg(out, _act(p), "out"), _arg(aux_loss, _F32, "aux_loss"),
        _arg(counts, _I32T, "counts"), _arg(n_dropped, _I32T, "n_dropped"),
        _arg(topk_idx, _I32T, "topk_idx"), _stream(stream)),
        "moe_layer_forward_noalloc")


def moe_quantize_int4(w, codes, qparams, stream=None):
    """4-bit codes of a bf16 matrix (or stack of matrices) ``w`` whose last
    axis is the input dimension K: ``codes`` uint8 [..., K/2], ``qparams``
    float32 [..., K/128, 2]."""
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    _check(_lib.moe_quantize_int4(_arg(w, torch.bfloat16, "w"), rows, K,
                                  _arg(codes, _U8, "codes"),
                                  _arg(qparams, _F32, "qparams"),
                                  _stream(stream)),
           "moe_quantize_int4")


def moe_tile_bf16(w, out, stream=None):
    """``out`` (same shape and size as the bf16 matrix or stack ``w``, last
    axis K) gets ``w`` in the GEMMs' tiled order."""
    K = w.shape[-1]
    rows = w.numel() // K if K else 0
    _check(_lib.moe_tile_bf16(_arg(w, torch.bfloat16, "w"), rows, K,
                              _arg(out, torch.bfloat16, "out"),
                              _stream(stream)),
           "moe_tile_bf16")


def moe_dispatch_reassign(p, topk_idx, topk_gate, logits, prob_mean, counts,
                          offsets, perm, slot_of, n_dropped, aux_loss, ws,
                          stream=None):
    wp, wn = _ws(ws)
    _check(_lib.moe_dispatch_reassign(
        ctypes.byref(p), _arg(topk_idx, _I32T, "topk_idx"),
        _arg(topk_gate, _F32, "topk_gate"), _arg(logits, _F32, "logits"),
        _arg(prob_mean, _F32, "prob_mean"), _arg(counts, _I32T, "counts"),
        _arg(offsets, _I32T, "offsets"), _arg(perm, _I32T, "perm"),
        _arg(slot_of, _I32T, "slot_of"), _arg(n_dropped, _I32T, "n_dropped"),
        _arg(aux_loss, _F32, "aux_loss"), wp, wn, _stream(stream)),
        "moe_dispatch_reassign")


def moe_update_select_bias(p, counts, select_bias, gamma, stream=None):
    _check(_lib.moe_update_select_bias(ctypes.byref(p),
                                       _arg(counts, _I32T, "counts"),
                                       _arg(select_bias, _F32, "select_bias"),
                                       gamma, _stream(stream)),
           "moe_update_select_bias")


QUANT_MATRICES = ("w1", "w2", "w_gate", "w_up", "w_down", "shared_w1",
                  "shared_w2", "shared_gate", "shared_up", "shared_down")


def quantize_weights(inp: dict, stream=None) -> dict:
    """A copy of a weights dict with every expert matrix replaced by its
    4-bit codes (same key) and (scale, offset) pairs (key + ``_q``), made
    on the device by :func:`moe_quantize_int4`.  Biases and the router stay
    as they are."""
    out = dict(inp)
    for n in QUANT_MATRICES:
        w = inp.get(n)
        if w is None:
            continue
        K = w.shape[-1]
        codes = torch.empty(*w.shape[:-1], K // 2, dtype=torch.uint8,
                            device=w.device)
        qp = torch.empty(*w.shape[:-1], K // MOE_Q4_GROUP, 2,
                         dtype=torch.float32, device=w.device)
        moe_quantize_int4(w, codes, qp, stream)
        out[n] = codes
        out[n + "_q"] = qp
    return out


def tile_weights(inp: dict, stream=None) -> dict:
    """A copy of a weights dict with every bf16 expert matrix replaced by
    its tiled-order copy (same key, same shape), made on the device by
    :func:`moe_tile_bf16`, for problems with wquant "bf16_tiled".  Biases
    and the router stay as they are."""
    out = dict(inp)
    for n in QUANT_MATRICES:
        w = inp.get(n)
        if w is None:
            continue
        t = torch.empty_like(w)
        moe_tile_bf16(w, t, stream)
        out[n] = t
    return out


# ---------------------------------------------------------------------------
# convenience: allocate outputs and run the whole layer
# ---------------------------------------------------------------------------

def layer_forward(inp: dict, wl, ws=None, stream=None, return_routing=False):
    """Run the layer on the inputs of :func:`synth.make_inputs` (device
    tensors).  Returns ``out``, ``aux``, ``counts``, ``n_dropped`` (and
    ``topk_idx`` when asked) as device tensors."""
    p = problem_for(wl)
    dev = inp["x"].device
    if ws is None:
        ws = workspace(p, dev)
    out = torch.empty_like(inp["x"])
    aux = torch.empty(1, dtype=torch.float32, device=dev)
    counts = torch.empty(wl.n_experts, dtype=torch.int32, device=dev)
    nd = torch.empty(1, dtype=torch.int32, device=dev)
    idx = (torch.empty(wl.T, wl.top_k, dtype=torch.int32, device=dev)
           if return_routing else None)
    moe_layer_forward(p, inp["x"], inp["w_router"], inp.get("router_bias"),
                      inp.get("select_bias"), inp, out, aux, counts, nd, idx,
                      ws, stream)
    res = {"out": out, "aux": aux, "counts": counts, "n_dropped": nd}
    if return_routing:
        res["topk_idx"] = idx
    return res


def flops_and_bytes(wl, counts, kept_total) -> tuple:
    """Algorithmic FLOPs and HBM bytes of one layer forward: 2 FLOPs per
    multiply-add over the kept assignments (plus shared rows) and the
    router; bytes of the touched experts' weights once plus x, out, the
    router weight and biases.  ``counts`` are per-expert pre-capacity
    assignment counts."""
    esz = 2 if wl.dtype == "bf16" else 4
    d, f, E = wl.d_model, wl.d_ff, wl.n_experts
    per_expert = (3 if wl.act == "swiglu" else 2) * d * f
    bias = (f + d) if wl.act == "gelu" else 0
    rows = kept_total + wl.n_shared * wl.T
    flops = 2 * rows * per_expert + 2 * wl.T * d * E
    touched = sum(1 for c in counts if c > 0) + wl.n_shared
    if getattr(wl, "wquant", None) == "int4":
        # codes (half a byte per weight) plus a float32 (scale, offset) per
        # group of 128 weights
        w_bytes = per_expert // 2 + (per_expert // MOE_Q4_GROUP) * 8 \
            + bias * esz
    else:
        w_bytes = (per_expert + bias) * esz
    byts = (touched * w_bytes + 2 * wl.T * d * esz
            + E * d * 4 + (E * 4 if wl.zipf_s > 0 else 0)
            + (E * 4 if wl.select_bias_std > 0 else 0))
    return flops, byts


__all__ = [n for n in dir() if n.startswith("moe_")] + [
    "problem", "problem_for", "expert_weights", "workspace", "layer_forward",
    "quantize_weights", "tile_weights", "QUANT_MATRICES",
    "flops_and_bytes", "MoEError", "synth", "library_path", "EXPORTS"]
