"""Pin checks for the CPU oracle, written against an implementation object.

Each check takes `impl` (a module or namespace exposing the oracle's
functions) and raises AssertionError when the implementation disagrees with
something fixed independently of it: brute force on tiny inputs
(oracle.brute), closed forms, exact integer arithmetic, or invariants of the
method (AdaFuse technical summary §2.A pre-gating and §2.B SGMM / decoding
procedure).  tests/test_oracle_pins.py runs them on the real oracle;
tests/test_oracle_mutants.py runs them on deliberately broken copies to show
that each plausible mistake is caught.
"""
from __future__ import annotations

import math

import numpy as np

from oracle import brute


def _rng(seed):
    return np.random.default_rng(np.random.SeedSequence([4242, seed]))


# ----------------------------------------------------------------------------- router

def check_logits_brute(impl):
    g = _rng(1)
    x = g.standard_normal((5, 7))
    Wg = g.standard_normal((7, 4))
    ref = np.array(brute.logits(x, Wg))
    np.testing.assert_allclose(impl.router_logits(x, Wg), ref, rtol=1e-12, atol=1e-12)
    # integer inputs: exact
    xi = g.integers(-4, 5, (6, 9)).astype(float)
    Wi = g.integers(-4, 5, (9, 5)).astype(float)
    assert np.array_equal(impl.router_logits(xi, Wi), np.array(brute.logits(xi, Wi)))


def check_topk_brute(impl):
    g = _rng(2)
    for E in range(1, 8):
        for k in range(1, E + 1):
            # values from a small set so that exact ties are frequent
            l = g.integers(-3, 4, (12, E)).astype(np.float64) * 0.5
            got = impl.select_topk(l, k)
            for t in range(l.shape[0]):
                assert list(got[t]) == brute.topk(list(l[t]), k), (E, k, t, l[t], got[t])


def check_topk_ties_lowest_index(impl):
    # duplicate router columns give exactly equal logits; the lower index must win
    g = _rng(3)
    x = g.standard_normal((16, 10))
    Wg = g.standard_normal((10, 6))
    Wg[:, 4] = Wg[:, 1]
    Wg[:, 5] = Wg[:, 1]
    l = impl.router_logits(x, Wg)
    idx = impl.select_topk(l, 2)
    for t in range(16):
        chosen = set(idx[t].tolist())
        if 1 in chosen or 4 in chosen or 5 in chosen:
            # among the three equal columns the lowest index comes first
            tied = [e for e in idx[t].tolist() if e in (1, 4, 5)]
            assert tied == sorted([1, 4, 5])[: len(tied)], (t, idx[t])


def check_topk_invariant(impl):
    g = _rng(4)
    l = g.standard_normal((200, 32))
    for k in (1, 2, 5):
        idx = impl.select_topk(l, k)
        assert idx.dtype == np.int32 and idx.shape == (200, k)
        for t in range(200):
            sel = l[t, idx[t]]
            rest = np.delete(l[t], idx[t])
            assert sel.min() >= rest.max()
            assert np.all(np.diff(sel) <= 0), "best first"
            assert len(set(idx[t].tolist())) == k


def check_topk_ranks_exact_logits(impl):
    # the ranking follows the logits themselves: a gap far below fp32
    # resolution still decides, and only an exact tie goes to the lower index
    l = np.array([[1.0, 1.0 + 1e-12, -1.0], [1.0, 1.0, -1.0], [2.0 ** -30, 0.0, 2.0 ** -30 * (1 + 2.0 ** -40)]])
    assert impl.select_topk(l, 1)[:, 0].tolist() == [1, 0, 2]
    assert impl.select_topk(l, 2).tolist() == [[1, 0], [0, 1], [2, 0]]


# ----------------------------------------------------------------------------- gates

def check_gates_closed_form(impl):
    l = np.array([[math.log(3.0), 0.0, -5.0]])
    idx = np.array([[0, 1]], dtype=np.int32)
    np.testing.assert_allclose(impl.softmax_gates(l, idx), [[0.75, 0.25]], rtol=0, atol=1e-15)
    g = _rng(5)
    l = g.standard_normal((50, 8)) * 3
    idx = impl.select_topk(l, 2)
    gt = impl.softmax_gates(l, idx)
    l0 = l[np.arange(50), idx[:, 0]]
    l1 = l[np.arange(50), idx[:, 1]]
    np.testing.assert_allclose(gt[:, 0], 1.0 / (1.0 + np.exp(l1 - l0)), rtol=1e-13)
    np.testing.assert_allclose(gt.sum(1), 1.0, rtol=1e-14)
    assert np.all(gt[:, 0] >= gt[:, 1])
    idx1 = impl.select_topk(l, 1)
    assert np.all(impl.softmax_gates(l, idx1) == 1.0)


def check_gates_brute(impl):
    g = _rng(6)
    l = g.standard_normal((10, 6))
    for k in (1, 2, 3):
        idx = impl.select_topk(l, k)
        gt = impl.softmax_gates(l, idx)
        for t in range(10):
            np.testing.assert_allclose(gt[t], brute.gates(list(l[t]), idx[t].tolist()), rtol=1e-13)


def check_pregate_composes(impl):
    g = _rng(7)
    x = g.standard_normal((9, 12))
    Wg = g.standard_normal((12, 5))
    idx, gate, logits = impl.pregate(x, Wg, 2)
    bl = brute.logits(x, Wg)
    for t in range(9):
        assert list(idx[t]) == brute.topk(bl[t], 2)
        np.testing.assert_allclose(gate[t], brute.gates(bl[t], idx[t].tolist()), rtol=1e-12)


# ----------------------------------------------------------------------------- segments

def check_segment_brute(impl):
    g = _rng(8)
    for (T, E, k) in [(1, 1, 1), (7, 3, 1), (20, 5, 2), (33, 9, 3), (64, 4, 4)]:
        idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
        off, perm = impl.segment(idx, E)
        boff, bperm = brute.segments(idx, E)
        assert off.tolist() == boff and perm.tolist() == bperm, (T, E, k)


def check_segment_invariants(impl):
    g = _rng(9)
    T, E, k = 300, 40, 2
    idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    off, perm = impl.segment(idx, E)
    assert off.dtype == np.int32 and perm.dtype == np.int32
    assert off[0] == 0 and off[-1] == T * k and np.all(np.diff(off) >= 0)
    np.testing.assert_array_equal(np.diff(off), np.bincount(idx.ravel(), minlength=E))
    assert sorted(perm.tolist()) == list(range(T * k))
    flat = idx.ravel()
    for e in range(E):
        seg = perm[off[e]:off[e + 1]]
        assert np.all(flat[seg] == e)
        assert np.all(np.diff(seg) > 0), "stable: ascending pair id inside a segment"


def check_segment_empty_and_edge(impl):
    off, perm = impl.segment(np.zeros((0, 2), np.int32), 5)
    assert off.tolist() == [0] * 6 and perm.size == 0
    idx = np.full((4, 1), 2, np.int32)  # every token on adapter 2: segments 0,1,3 empty
    off, perm = impl.segment(idx, 4)
    assert off.tolist() == [0, 0, 0, 4, 4] and perm.tolist() == [0, 1, 2, 3]
    try:
        impl.segment(np.array([[5]], np.int32), 4)
    except ValueError:
        pass
    else:
        raise AssertionError("out-of-range adapter index must be rejected")


# ----------------------------------------------------------------------------- projection

def _tiny_case(seed, T=4, d_in=6, d_out=5, E=3, r=2, k=2, integer=False):
    g = _rng(seed)
    if integer:
        draw = lambda s: g.integers(-3, 4, s).astype(np.float64)  # noqa: E731
    else:
        draw = lambda s: g.standard_normal(s)  # noqa: E731
    x, W0, A, B = draw((T, d_in)), draw((d_out, d_in)), draw((E, r, d_in)), draw((E, d_out, r))
    idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    gate = np.ones((T, k)) if integer else g.uniform(0.1, 1.0, (T, k))
    return x, W0, A, B, idx, gate


def check_sgmm_brute(impl):
    for seed, kw in [(10, {}), (11, dict(T=3, d_in=5, d_out=8, E=4, r=3, k=3)), (12, dict(k=1))]:
        x, W0, A, B, idx, gate = _tiny_case(seed, **kw)
        np.testing.assert_allclose(impl.sgmm(x, W0, A, B, idx, gate),
                                   np.array(brute.projection(x, W0, A, B, idx, gate)),
                                   rtol=1e-12, atol=1e-12)


def check_sgmm_exact_integer(impl):
    x, W0, A, B, idx, gate = _tiny_case(13, T=5, d_in=16, d_out=9, E=4, r=4, k=2, integer=True)
    got = impl.sgmm(x, W0, A, B, idx, gate)
    want = np.array(brute.projection(x.astype(int).tolist(), W0.astype(int).tolist(),
                                     A.astype(int).tolist(), B.astype(int).tolist(),
                                     idx.tolist(), [[1] * 2] * 5), dtype=np.float64)
    assert np.array_equal(got, want)


def check_sgmm_plain_lora(impl):
    # E = 1, k = 1, gate 1: the textbook LoRA form x W0^T + (x A^T) B^T
    g = _rng(14)
    x, W0 = g.standard_normal((7, 10)), g.standard_normal((6, 10))
    A, B = g.standard_normal((1, 3, 10)), g.standard_normal((1, 6, 3))
    idx, gate = np.zeros((7, 1), np.int32), np.ones((7, 1))
    np.testing.assert_allclose(impl.sgmm(x, W0, A, B, idx, gate),
                               np.matmul(x, W0.T) + np.matmul(np.matmul(x, A[0].T), B[0].T),
                               rtol=1e-12, atol=1e-12)


def check_sgmm_merged_weight(impl):
    # the pages' merge -> infer view: with one fixed choice for every token the
    # fused result equals projecting through W0 + sum_j g_j B_ej A_ej
    g = _rng(15)
    T, d_in, d_out, E, r = 9, 12, 7, 5, 3
    x, W0 = g.standard_normal((T, d_in)), g.standard_normal((d_out, d_in))
    A, B = g.standard_normal((E, r, d_in)), g.standard_normal((E, d_out, r))
    for choice, gs in [((3,), (1.0,)), ((4, 1), (0.7, 0.3))]:
        W = W0.copy()
        for e, gv in zip(choice, gs):
            W += gv * (B[e] @ A[e])
        idx = np.tile(np.array(choice, np.int32), (T, 1))
        gate = np.tile(np.array(gs), (T, 1))
        np.testing.assert_allclose(impl.sgmm(x, W0, A, B, idx, gate), x @ W.T, rtol=1e-11, atol=1e-11)


def check_sgmm_zero_B_and_k0(impl):
    x, W0, A, B, idx, gate = _tiny_case(16, T=6, d_in=8, d_out=5)
    base = impl.sgmm(x, W0, A, np.zeros_like(B), idx, gate)
    assert np.array_equal(base, x @ W0.T)
    assert np.array_equal(impl.sgmm(x, W0, A, B, idx[:, :0], gate[:, :0]), x @ W0.T)


def check_sgmm_token_permutation(impl):
    x, W0, A, B, idx, gate = _tiny_case(17, T=11, d_in=9, d_out=6, E=4, r=2, k=2)
    p = _rng(18).permutation(11)
    y = impl.sgmm(x, W0, A, B, idx, gate)
    yp = impl.sgmm(x[p], W0, A, B, idx[p], gate[p])
    np.testing.assert_allclose(yp, y[p], rtol=1e-13, atol=1e-13)


def check_sgmm_linearity(impl):
    x, W0, A, B, idx, gate = _tiny_case(19, T=6, d_in=8, d_out=7, E=3, r=2, k=2)
    y0 = impl.sgmm(x, W0, A, B, idx[:, :0], gate[:, :0])
    d1 = impl.sgmm(x, W0, A, B, idx, gate) - y0
    np.testing.assert_allclose(impl.sgmm(x, W0, A, 2.5 * B, idx, gate) - y0, 2.5 * d1, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(impl.sgmm(x, W0, A, B, idx, 3.0 * gate) - y0, 3.0 * d1, rtol=1e-11, atol=1e-12)
    # slots add independently
    dj = sum(impl.sgmm(x, W0, A, B, idx[:, j:j + 1], gate[:, j:j + 1]) - y0 for j in range(2))
    np.testing.assert_allclose(dj, d1, rtol=1e-11, atol=1e-12)


def check_sgmm_token_subset(impl):
    x, W0, A, B, idx, gate = _tiny_case(20, T=8)
    y = impl.sgmm(x, W0, A, B, idx, gate)
    np.testing.assert_allclose(impl.sgmm(x, W0, A, B, idx, gate, tokens=[5, 1, 7]), y[[5, 1, 7]], rtol=1e-14)


# ----------------------------------------------------------------------------- decoder layer

def check_round_bf16_grid(impl):
    # against the representable grid walked pattern by pattern, and hand-made ties
    g = _rng(30)
    x = g.standard_normal(3000) * 10.0 ** g.integers(-6, 6, 3000)
    want = np.array([brute.bf16_grid_nearest(float(v)) for v in x])
    assert np.array_equal(impl.round_bf16(x), want)
    ties = np.array([1 + 2.0 ** -8, 1 + 3 * 2.0 ** -8, 255.5, -(1 + 2.0 ** -8), 3 * 2.0 ** -9 + 2.0 ** -1])
    assert np.array_equal(impl.round_bf16(ties), [1.0, 1 + 2.0 ** -6, 256.0, -1.0, 0.5078125])
    exact = np.array([1.0, -0.5, 3.0, 2.0 ** -20, 1 + 2.0 ** -7])
    assert np.array_equal(impl.round_bf16(exact), exact)


def check_rmsnorm_closed_forms(impl):
    g = _rng(31)
    gamma = g.uniform(0.5, 2.0, 6)
    # a constant row c normalises to sign(c) * gamma (eps = 0)
    x = np.array([[3.0] * 6, [-0.25] * 6])
    np.testing.assert_allclose(impl.rmsnorm(x, gamma, 0.0), np.array([gamma, -gamma]), rtol=1e-14)
    # [3, 4]: mean square 12.5
    np.testing.assert_allclose(impl.rmsnorm(np.array([[3.0, 4.0]]), np.ones(2), 0.0),
                               [[3 / math.sqrt(12.5), 4 / math.sqrt(12.5)]], rtol=1e-14)
    # scale invariance and unit mean square (eps = 0, gamma = 1)
    x = g.standard_normal((4, 10))
    y = impl.rmsnorm(x, np.ones(10), 0.0)
    np.testing.assert_allclose(impl.rmsnorm(7.5 * x, np.ones(10), 0.0), y, rtol=1e-13)
    np.testing.assert_allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-13)
    # eps enters under the square root: a zero row stays zero, a tiny row is damped
    assert np.array_equal(impl.rmsnorm(np.zeros((1, 4)), np.ones(4), 1e-5), np.zeros((1, 4)))
    np.testing.assert_allclose(impl.rmsnorm(np.array([[1e-3, 1e-3]]), np.ones(2), 1e-6),
                               [[1e-3 / math.sqrt(2e-6)] * 2], rtol=1e-13)


def check_silu_mul_values(impl):
    # sigma(x) = (1 + tanh(x / 2)) / 2: silu(g) = g * sigma(g)
    g = np.array([[0.0, 1.0, -1.0, 2.0, -3.5]])
    want = g * (1 + np.tanh(g / 2)) / 2
    np.testing.assert_allclose(impl.silu_mul(g, np.ones_like(g)), want, rtol=1e-14, atol=1e-300)
    # odd part: silu(x) - silu(-x) = x; linear in u; the gate is the argument of silu
    x = _rng(32).standard_normal((3, 7))
    one = np.ones_like(x)
    np.testing.assert_allclose(impl.silu_mul(x, one) - impl.silu_mul(-x, one), x, rtol=1e-13, atol=1e-14)
    u = _rng(33).standard_normal((3, 7))
    np.testing.assert_allclose(impl.silu_mul(x, 2.0 * u), 2.0 * impl.silu_mul(x, u), rtol=1e-14)
    assert np.array_equal(impl.silu_mul(np.zeros((1, 3)), np.array([[5.0, -1.0, 2.0]])), np.zeros((1, 3)))


def _layer_case(seed, T=3, d=8, ff=12, E=3, r=2, k=2):
    g = _rng(seed)
    w = {"gamma1": g.uniform(0.5, 1.5, d), "gamma2": g.uniform(0.5, 1.5, d)}
    for name, (o, i) in {"q": (d, d), "k": (d, d), "v": (d, d), "o": (d, d), "gate": (ff, d), "up": (ff, d),
                         "down": (d, ff)}.items():
        w[name] = (g.standard_normal((o, i)) / math.sqrt(i), g.standard_normal((E, r, i)) / math.sqrt(i),
                   0.3 * g.standard_normal((E, o, r)))
    h = g.standard_normal((T, d))
    idx = np.stack([g.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    gate = g.uniform(0.1, 1.0, (T, k))
    return h, w, idx, gate


def _zero(w, name):
    W0, A, B = w[name]
    return (np.zeros_like(W0), A, np.zeros_like(B))


def check_decoder_layer_brute(impl):
    ident = lambda a: np.asarray(a, np.float64)  # noqa: E731
    for seed in (40, 41):
        h, w, idx, gate = _layer_case(seed)
        np.testing.assert_allclose(impl.decoder_layer(h, w, idx, gate, 1e-5, rnd=ident),
                                   np.array(brute.decoder_layer(h, w, idx, gate, 1e-5)), rtol=1e-11, atol=1e-12)


def check_decoder_layer_passthrough(impl):
    h, w, idx, gate = _layer_case(42)
    h = impl.round_bf16(h)
    # o and down zero: both residual adds pass h through unchanged
    w2 = dict(w, o=_zero(w, "o"), down=_zero(w, "down"))
    assert np.array_equal(impl.decoder_layer(h, w2, idx, gate, 1e-5), h)
    # up zero: the MLP adds silu(g) * 0 = 0, so the layer is h + o(v) alone (o still live)
    w3 = dict(w, up=_zero(w, "up"))
    w4 = dict(w, up=_zero(w, "up"), down=_zero(w, "down"))
    assert np.array_equal(impl.decoder_layer(h, w3, idx, gate, 1e-5), impl.decoder_layer(h, w4, idx, gate, 1e-5))
    # ... while a zero gate projection makes silu(0) = 0 as well, but a live up alone must not
    w5 = dict(w, gate=_zero(w, "gate"))
    assert np.array_equal(impl.decoder_layer(h, w5, idx, gate, 1e-5), impl.decoder_layer(h, w4, idx, gate, 1e-5))


def check_decoder_layer_token_permutation(impl):
    h, w, idx, gate = _layer_case(43, T=6)
    p = _rng(44).permutation(6)
    y = impl.decoder_layer(h, w, idx, gate, 1e-5)
    assert np.array_equal(impl.decoder_layer(h[p], w, idx[p], gate[p], 1e-5), y[p])


ALL_CHECKS = [v for k, v in sorted(globals().items()) if k.startswith("check_")]
