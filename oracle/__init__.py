"""CPU oracle for the sparse mixture-of-experts layer forward pass.

TEST INFRASTRUCTURE ONLY.  This package is the slow, plain, fp64 statement of
what the layer computes; it exists so the HIP path can be checked against it.
Only the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it.  The product path (the C-ABI library and its Python binding) never
imports, links or calls anything here, and this package shares no code with it.

Sources (web pages on sparse mixture-of-experts layers):
  [RC]  randomcommits.com, "Mixture-of-Experts routing" post
  [LBS] letsbuildsolutions.com, "How Mixture of Experts Works: Sparse Gating,
        Expert Routing, and the Architecture Behind Efficient Large Language
        Models"
  [HA]  hassanahmed.net, "Mixture of Experts explained"
  [GN]  getnybble.com, "Mixture of Experts (MoE) - conditional computation at
        scale"
  [FA]  foundry.adhana.ai, "Mixture-of-Experts routing"

Every function in :mod:`oracle.moe` is pinned by a ``-m "not gpu"`` test
against something other than itself (closed forms, hand-counted cases, a
brute-force dense evaluation, library routines).  Nothing here is
"parity unpinned" except where a docstring says so.
"""

from .moe import (  # noqa: F401
    capacity,
    gelu,
    silu,
    softmax,
    sigmoid,
    update_select_bias,
    route,
    topk_margin,
    dispatch,
    philox4x32,
    dispatch_reassign,
    expert_ffn,
    combine,
    aux_loss,
    layer_forward,
    Q4_GROUP,
    quantize_int4,
    dequantize_int4,
)
