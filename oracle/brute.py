"""Pure-Python brute force for tiny inputs (test infrastructure only).

An independent formulation of each step of the AdaFuse pre-gated projection
(technical summary §2.A pre-gating, §2.B SGMM / decoding procedure), used to
pin oracle/reference.py.  It uses no NumPy arithmetic: plain loops over Python
numbers.  With integer-valued inputs every result is an exact integer.
"""
from __future__ import annotations

import itertools
import math
from typing import List, Sequence, Tuple


def _tolist(a):
    return a.tolist() if hasattr(a, "tolist") else a


def logits(x, Wg) -> List[List[float]]:
    """l[t][e] = sum over i of x[t][i] * Wg[i][e], summed in index order."""
    x, Wg = _tolist(x), _tolist(Wg)
    T, d = len(x), len(Wg)
    E = len(Wg[0]) if d else 0
    out = []
    for t in range(T):
        row = []
        for e in range(E):
            s = 0
            for i in range(d):
                s += x[t][i] * Wg[i][e]
            row.append(s)
        out.append(row)
    return out


def topk(l_row: Sequence[float], k: int) -> List[int]:
    """The unique k-subset S whose every member outranks every non-member.

    Rank order: higher logit first; between equal logits the lower index
    first.  Found by enumerating all k-subsets (E small), then listed best
    first.
    """
    E = len(l_row)

    def beats(a, b):
        return l_row[a] > l_row[b] or (l_row[a] == l_row[b] and a < b)

    found = []
    for S in itertools.combinations(range(E), k):
        rest = [e for e in range(E) if e not in S]
        if all(beats(a, b) for a in S for b in rest):
            found.append(S)
    assert len(found) == 1, "rank order is total, so exactly one subset dominates"
    S = list(found[0])
    # order the members: a member's place = number of members that beat it
    placed = [None] * k
    for a in S:
        placed[sum(1 for b in S if b != a and beats(b, a))] = a
    return placed


def gates(l_row: Sequence[float], chosen: Sequence[int]) -> List[float]:
    """Softmax over the chosen logits (math.exp; no shift needed at test sizes)."""
    w = [math.exp(l_row[e]) for e in chosen]
    s = sum(w)
    return [v / s for v in w]


def segments(idx, E: int) -> Tuple[List[int], List[int]]:
    """For each adapter in turn, scan all pairs in order and collect those that chose it."""
    idx = _tolist(idx)
    T = len(idx)
    k = len(idx[0]) if T else 0
    perm, offsets = [], [0]
    for e in range(E):
        for t in range(T):
            for j in range(k):
                if idx[t][j] == e:
                    perm.append(t * k + j)
        offsets.append(len(perm))
    return offsets, perm


def projection(x, W0, A, B, idx, gate) -> List[List[float]]:
    """y[t][o] = sum_i W0[o][i] x[t][i] + sum_j g[t][j] sum_c B[e][o][c] sum_i A[e][c][i] x[t][i]."""
    x, W0, A, B, idx, gate = map(_tolist, (x, W0, A, B, idx, gate))
    T = len(x)
    d_out, d_in = len(W0), len(W0[0])
    k = len(idx[0]) if T else 0
    y = []
    for t in range(T):
        row = []
        for o in range(d_out):
            s = 0
            for i in range(d_in):
                s += W0[o][i] * x[t][i]
            for j in range(k):
                e = idx[t][j]
                r = len(A[e])
                delta = 0
                for c in range(r):
                    u = 0
                    for i in range(d_in):
                        u += A[e][c][i] * x[t][i]
                    delta += B[e][o][c] * u
                s += gate[t][j] * delta
            row.append(s)
        y.append(row)
    return y


def bf16_grid_nearest(v: float) -> float:
    """Nearest bfloat16 value by walking the representable grid (ties: even last significand bit).

    A bfloat16 is the float32 whose upper 16 bits are the pattern; the two
    patterns around v are found from v's float32 bits and compared directly.
    """
    import struct
    if v == 0.0:
        return 0.0
    bits = struct.unpack("<I", struct.pack("<f", v))[0] & 0xFFFF0000  # a pattern at or toward zero from v
    lo = struct.unpack("<f", struct.pack("<I", bits))[0]
    hi = struct.unpack("<f", struct.pack("<I", bits + 0x10000))[0]  # next pattern away from zero
    if abs(lo) > abs(v):  # float32 rounding of v went past it: step back one pattern
        lo, hi = struct.unpack("<f", struct.pack("<I", bits - 0x10000))[0], lo
        bits -= 0x10000
    dl, dh = abs(v - lo), abs(hi - v)
    if dl < dh:
        return lo
    if dh < dl:
        return hi
    return lo if (bits >> 16) % 2 == 0 else hi


def decoder_layer(h, w, idx, gate, eps: float):
    """The decoder layer of oracle.reference.decoder_layer without the bf16 rounding, in loops.

    n1 = rmsnorm(h, gamma1); v = proj_v(n1); h1 = h + proj_o(v);
    n2 = rmsnorm(h1, gamma2); m = silu(proj_gate(n2)) * proj_up(n2); h2 = h1 + proj_down(m).
    """
    h = [list(map(float, r)) for r in _tolist(h)]

    def norm(x, gamma):
        gamma = _tolist(gamma)
        out = []
        for row in x:
            ms = sum(v * v for v in row) / len(row)
            inv = 1.0 / math.sqrt(ms + eps)
            out.append([row[i] * inv * gamma[i] for i in range(len(row))])
        return out

    def proj(x, name):
        W0, A, B = w[name]
        return projection(x, W0, A, B, idx, gate)

    def add(a, b):
        return [[a[t][i] + b[t][i] for i in range(len(a[t]))] for t in range(len(a))]

    n1 = norm(h, w["gamma1"])
    h1 = add(h, proj(proj(n1, "v"), "o"))
    n2 = norm(h1, w["gamma2"])
    g, u = proj(n2, "gate"), proj(n2, "up")
    m = [[g[t][i] / (1.0 + math.exp(-g[t][i])) * u[t][i] for i in range(len(g[t]))] for t in range(len(g))]
    return add(h1, proj(m, "down"))
