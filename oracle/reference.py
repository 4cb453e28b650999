"""NumPy fp64 oracle (test infrastructure only; see oracle/__init__.py).

Source of every step: the AdaFuse page (gist.science summary of
"AdaFuse: Accelerating Dynamic Adapter Inference via Token-Level Pre-Gating
and Fused Kernel Optimization"), technical summary §2.A (pre-gating) and
§2.B (SGMM kernel and the five-step decoding procedure).  Where the page is
silent, the reading taken is stated in the function's docstring.
"""
from __future__ import annotations

from typing import Optional, Sequence, Tuple

import numpy as np


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Exact fp64 view of an input as uploaded to the device.

    dtype "bf16": `a` holds bfloat16 bit patterns (uint16); a bfloat16 value is
    the float32 whose upper 16 bits are those bits and whose lower 16 are zero.
    dtype "f32": `a` is float32.
    """
    if dtype == "bf16":
        b = np.ascontiguousarray(a, dtype=np.uint16)
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    if dtype == "f32":
        return np.asarray(a, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def router_logits(x: np.ndarray, Wg: np.ndarray) -> np.ndarray:
    """Router scores, §2.A: one linear map per token, logits[t,e] = sum_i x[t,i] Wg[i,e].

    Reading: the "lightweight router" is a single bias-free linear layer
    Wg[d_in, E] (the toy workload's router is Wg[512x4]).  fp64 matmul.
    """
    return np.asarray(x, np.float64) @ np.asarray(Wg, np.float64)


def select_topk(logits: np.ndarray, k: int) -> np.ndarray:
    """Top-k adapter choice per token, §2.B step 2.

    Adapters are ranked on the fp64 logits by (logit descending, index
    ascending): an exact tie goes to the lower index.  Returns int32 [T, k],
    best first.
    """
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    if not (0 <= k <= E):
        raise ValueError("k out of range")
    e_ids = np.broadcast_to(np.arange(E), (T, E))
    order = np.lexsort((e_ids, -l), axis=-1)  # primary key: -logit, secondary: index
    return order[:, :k].astype(np.int32)


def topk_margin(logits: np.ndarray, k: int) -> np.ndarray:
    """Per-token gap between the k-th and (k+1)-th largest logit (fp64); +inf when k == E.

    Tokens with a gap below the device's rounding error may legitimately
    select differently; tests report them instead of asserting on them.
    """
    l = np.sort(np.asarray(logits, np.float64), axis=1)[:, ::-1]
    T, E = l.shape
    if k >= E or k == 0:
        return np.full(T, np.inf)
    return l[:, k - 1] - l[:, k]


def softmax_gates(logits: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """Gate weights over the chosen adapters (reading: softmax over the k selected logits).

    g[t,j] = exp(l[t,idx_j] - l[t,idx_0]) / sum_j' exp(l[t,idx_j'] - l[t,idx_0]).
    For k = 1 this is exactly 1.  Equal to a softmax over all E renormalised
    over the selected k.  fp64.
    """
    l = np.asarray(logits, np.float64)
    T, k = idx.shape
    if k == 0:
        return np.zeros((T, 0))
    sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    z = np.exp(sel - sel[:, :1])
    return z / z.sum(axis=1, keepdims=True)


def pregate(x: np.ndarray, Wg: np.ndarray, k: int) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """§2.A + §2.B steps 1-2: score once, choose top-k, weight the choice.

    Returns (idx int32 [T,k], gate fp64 [T,k], logits fp64 [T,E]).
    """
    logits = router_logits(x, Wg)
    idx = select_topk(logits, k)
    return idx, softmax_gates(logits, idx), logits


def segment(idx: np.ndarray, E: int) -> Tuple[np.ndarray, np.ndarray]:
    """Group the (token, slot) pairs by adapter: the segments SGMM runs over.

    A pair p = t*k + j names slot j of token t.  offsets[e] .. offsets[e+1]
    is adapter e's segment in `perm`, which lists the pair ids grouped by
    adapter (ascending e) and, inside a segment, in ascending p (a stable
    order).  Empty segments have offsets[e] == offsets[e+1].
    Returns (offsets int32 [E+1], perm int32 [T*k]).
    """
    flat = np.asarray(idx, np.int64).ravel()
    if flat.size and (flat.min() < 0 or flat.max() >= E):
        raise ValueError("adapter index out of range")
    counts = np.bincount(flat, minlength=E)
    offsets = np.zeros(E + 1, dtype=np.int64)
    np.cumsum(counts, out=offsets[1:])
    perm = np.argsort(flat, kind="stable")
    return offsets.astype(np.int32), perm.astype(np.int32)


def sgmm(x: np.ndarray, W0: np.ndarray, A: np.ndarray, B: np.ndarray, idx: np.ndarray,
         gate: np.ndarray, tokens: Optional[Sequence[int]] = None) -> np.ndarray:
    """Base projection plus the gated low-rank deltas of each token's chosen adapters.

    y[t] = W0 x[t] + sum_j gate[t,j] * B[idx[t,j]] (A[idx[t,j]] x[t])

    Shapes: x [T, d_in], W0 [d_out, d_in], A [E, r, d_in], B [E, d_out, r],
    idx/gate [T, k].  Evaluated per token over its chosen adapters (a plain
    loop); the base term is one library matmul.  `tokens` restricts the
    evaluation to a subset of rows (returned in that order).  fp64.
    """
    x = np.asarray(x, np.float64)
    W0 = np.asarray(W0, np.float64)
    A = np.asarray(A, np.float64)
    B = np.asarray(B, np.float64)
    gate = np.asarray(gate, np.float64)
    rows = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens, np.int64)
    y = x[rows] @ W0.T
    k = idx.shape[1] if idx.ndim == 2 else 0
    for out_row, t in enumerate(rows):
        for j in range(k):
            e = int(idx[t, j])
            u = A[e] @ x[t]                 # rank-r intermediate
            y[out_row] += gate[t, j] * (B[e] @ u)
    return y


# ----------------------------------------------------------------------------- decoder layer
# Whole-step chaining around the adapted projections.  Decoding step 4 of the
# AdaFuse page (technical summary §2.B) runs the base model's standard
# inference between the projections; §4 measures Llama2-7B / Mistral-7B, whose
# decoder layer normalises with RMSNorm, adds residuals and gates its MLP with
# silu(gate) * up (gate and up packed into one wide operation on the
# "FlashSVD v1.5" page, La Solución).  Reading: the activations that cross
# from one operation to the next are bf16 tensors (the interface dtype), so
# each operation's output is rounded once to bf16, round-to-nearest-even.

def round_bf16(a: np.ndarray) -> np.ndarray:
    """Nearest bfloat16 value of each element (ties to the even significand), as fp64.

    bfloat16 keeps 8 significant bits: for |a| in [2^e, 2^(e+1)) the spacing is
    2^(e-7); a is divided by that spacing, rounded half-to-even, and scaled back.
    Finite normal-range inputs only.
    """
    a = np.asarray(a, np.float64)
    out = np.zeros_like(a)
    nz = a != 0
    e = np.floor(np.log2(np.abs(a[nz])))
    step = np.exp2(e - 7)
    q = a[nz] / step
    # guard the exponent against log2 landing one off at powers of two
    big = np.abs(q) >= 256
    step = np.where(big, step * 2, step)
    q = a[nz] / step
    small = np.abs(q) < 128
    step = np.where(small, step / 2, step)
    out[nz] = np.round(a[nz] / step) * step  # np.round: half to even
    return out


def rmsnorm(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of each row: x[t] * gamma / sqrt(mean_i x[t,i]^2 + eps).  fp64."""
    x = np.asarray(x, np.float64)
    ms = np.mean(x * x, axis=1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(gamma, np.float64)[None, :]


def silu_mul(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """Gated MLP activation: silu(g) * u with silu(g) = g / (1 + exp(-g)).  fp64."""
    g = np.asarray(g, np.float64)
    return g / (1.0 + np.exp(-g)) * np.asarray(u, np.float64)


def decoder_layer(h: np.ndarray, w: dict, idx: np.ndarray, gate: np.ndarray, eps: float,
                  rnd=round_bf16) -> np.ndarray:
    """One decode-step layer around the adapted projections; returns the next residual stream.

    w maps "gamma1", "gamma2" to [d] and "q","k","v","o","gate","up","down" to
    (W0, A, B) triples.  Every projection applies the step's routing (idx,
    gate) through `sgmm`.  Reading (attention is outside the method): the
    token attends to a single cached position, whose softmax weight is 1, so
    the attention output equals v.  Each operation's output passes through
    `rnd` (bf16 rounding by default):

        n1 = rnd(rmsnorm(h, gamma1))
        q, k, v = rnd(proj(n1))                  (q and k feed only the attention)
        h1 = rnd(h + proj_o(v))                  residual inside the one rounding
        n2 = rnd(rmsnorm(h1, gamma2))
        g, u = rnd(proj_gate(n2)), rnd(proj_up(n2))
        m = rnd(silu(g) * u)
        h2 = rnd(h1 + proj_down(m))
    """
    def proj(x, name):
        W0, A, B = w[name]
        return sgmm(x, W0, A, B, idx, gate)

    n1 = rnd(rmsnorm(h, w["gamma1"], eps))
    v = rnd(proj(n1, "v"))
    h1 = rnd(np.asarray(h, np.float64) + proj(v, "o"))
    n2 = rnd(rmsnorm(h1, w["gamma2"], eps))
    g = rnd(proj(n2, "gate"))
    u = rnd(proj(n2, "up"))
    m = rnd(silu_mul(g, u))
    return rnd(h1 + proj(m, "down"))
