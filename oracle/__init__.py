"""CPU oracle for pre-gated multi-adapter low-rank projection.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
execute this package: only the test suite, the smoke check in
__graft_entry__.py and the CPU-baseline leg of bench.py use it.  It shares no
code with the HIP library (rank_pregate_amd/csrc) and does not import the
rank_pregate_amd package.

What it computes (AdaFuse, "Accelerating Dynamic Adapter Inference via
Token-Level Pre-Gating and Fused Kernel Optimization", technical summary §2):

  * §2.A token-level pre-gating: one light linear router scores each token once
    (logits = x . Wg), the top-k adapters are chosen, and that choice is held
    for every later layer and projection.
  * the decoder layer around the projections (§2.B decoding step 4 runs the
    base model; §4 measures Llama-family 7B models): RMSNorm, residual adds and
    the silu(gate) * up MLP activation, with bf16 rounding at each operation's
    output (decoder_layer).
  * §2.B SGMM / decoding procedure: the chosen LoRA experts are applied together
    with the backbone projection in one pass.  In factorised form
        y[t] = W0 x[t] + sum_j g[t,j] * B_{e(t,j)} (A_{e(t,j)} x[t]),
    which in exact arithmetic equals projecting with the merged weight
    W0 + sum_j g_j B_e A_e (the pages' merge / infer / unmerge steps).

Modules:
  reference -- NumPy fp64 implementation (library matmul / sort as steps).
  brute     -- pure-Python loops for tiny inputs (independent formulation).

Every function is pinned by tests/test_oracle_pins.py against brute force,
closed forms and invariants; none is "parity unpinned".
"""
from . import reference, brute  # noqa: F401
from .reference import (  # noqa: F401
    widen, router_logits, select_topk, topk_margin, softmax_gates, pregate, segment, sgmm,
    round_bf16, rmsnorm, silu_mul, decoder_layer,
)
