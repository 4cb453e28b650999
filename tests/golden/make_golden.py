"""Write the golden fixtures in this folder.

Inputs come from the seeded generator (rank_pregate_amd.datagen.custom_case);
every expected value is computed by oracle.brute (plain Python loops; exact
integer arithmetic when the inputs are integers).  Nothing here calls the HIP
library.  Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import numpy as np  # noqa: E402

from oracle import brute  # noqa: E402
from rank_pregate_amd import datagen  # noqa: E402

CITATION = ("AdaFuse: Accelerating Dynamic Adapter Inference via Token-Level Pre-Gating and Fused Kernel "
            "Optimization (gist.science summary), technical summary §2.A token-level pre-gating and §2.B "
            "SGMM / decoding procedure steps 1-3.  The page prints no worked example; these expected values "
            "are the method's definition evaluated by brute force.")


def widen(a, dt):
    return datagen.bf16_bits_to_f32(a).astype(np.float64) if dt == "bf16" else a.astype(np.float64)


def make(name, seed, T, d_in, d_out, E, r, k, dtype, integer_range, tie_cols=None):
    c = datagen.custom_case(seed, T, d_in, d_out, E, r, dtype=dtype, b_scale=1.0, integer_range=integer_range)
    if tie_cols:
        a, b = tie_cols
        c["Wg"][:, b] = c["Wg"][:, a]
    x, Wg, W0, A, B = (widen(c[n], dtype) for n in ("x", "Wg", "W0", "A", "B"))
    if integer_range is not None:
        x, Wg, W0, A, B = (v.astype(np.int64).tolist() for v in (x, Wg, W0, A, B))
    else:
        x, Wg, W0, A, B = (v.tolist() for v in (x, Wg, W0, A, B))
    logits = brute.logits(x, Wg)
    idx = [brute.topk([float(v) for v in row], k) for row in logits]
    gate = [brute.gates([float(v) for v in row], chosen) for row, chosen in zip(logits, idx)]
    exact = integer_range is not None and k == 1
    if exact:
        gate_used = [[1] * k for _ in range(T)]
    else:
        gate_used = gate
    offsets, perm = brute.segments(idx, E)
    y = brute.projection(x, W0, A, B, idx, gate_used)
    fixture = {
        "name": name, "citation": CITATION, "dtype": dtype, "T": T, "d_in": d_in, "d_out": d_out,
        "E": E, "r": r, "k": k, "exact": exact,
        "note": ("integer inputs, top-1: every product and sum is an exact integer in fp32/fp64"
                 if exact else "real-valued gates; compare with a tolerance"),
        "inputs": {n: np.asarray(c[n]).tolist() for n in ("x", "Wg", "W0", "A", "B")},
        "expected": {"topk_idx": idx, "topk_gate": gate, "seg_offsets": offsets, "pair_perm": perm,
                     "y": y},
    }
    with open(os.path.join(HERE, name + ".json"), "w") as fh:
        json.dump(fixture, fh)
    print("wrote", name)


if __name__ == "__main__":
    make("exact_int_top1_bf16", 1, T=8, d_in=32, d_out=24, E=4, r=8, k=1, dtype="bf16",
         integer_range=2, tie_cols=(1, 3))
    make("exact_int_top1_f32", 2, T=10, d_in=24, d_out=40, E=5, r=8, k=1, dtype="f32",
         integer_range=3, tie_cols=(0, 4))
    make("top2_bf16", 3, T=6, d_in=16, d_out=24, E=6, r=8, k=2, dtype="bf16", integer_range=None)
