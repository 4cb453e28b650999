"""Plant plausible mistakes in copies of the oracle (on the CPU) and show the pins catch each one."""
import types

import numpy as np
import pytest

from oracle import reference
from tests import oracle_pins


def _mutant(**overrides):
    ns = types.SimpleNamespace(**{n: getattr(reference, n) for n in (
        "router_logits", "select_topk", "topk_margin", "softmax_gates", "pregate", "segment", "sgmm",
        "round_bf16", "rmsnorm", "silu_mul", "decoder_layer")})
    for k, v in overrides.items():
        setattr(ns, k, v)
    # keep pregate composed from the (possibly mutated) parts
    if "pregate" not in overrides:
        def pregate(x, Wg, k):
            l = ns.router_logits(x, Wg)
            idx = ns.select_topk(l, k)
            return idx, ns.softmax_gates(l, idx), l
        ns.pregate = pregate
    # and the decoder layer from the (possibly mutated) elementwise parts
    if "decoder_layer" not in overrides:
        ns.decoder_layer = _layer_variant(None, ns)
    return ns


def _layer_variant(kind, ns=None):
    def layer(h, w, idx, gate, eps, rnd=None):
        parts = ns if ns is not None else reference
        rnd = rnd or parts.round_bf16

        def proj(x, name):
            return parts.sgmm(x, *w[name], idx, gate)
        n1 = rnd(parts.rmsnorm(h, w["gamma1"], eps))
        attn = rnd(proj(n1, "q" if kind == "attention_from_q" else "v"))
        h1 = rnd((0 if kind == "no_residual_o" else np.asarray(h, np.float64)) + proj(attn, "o"))
        n2 = rnd(parts.rmsnorm(h1, w["gamma1" if kind == "gamma1_twice" else "gamma2"], eps))
        g, u = rnd(proj(n2, "gate")), rnd(proj(n2, "up"))
        m = rnd(parts.silu_mul(g, u))
        return rnd((0 if kind == "no_residual_down" else h1) + proj(m, "down"))
    return layer


def _round_toward_zero(a):
    a = np.asarray(a, np.float64)
    r = reference.round_bf16(a)
    step = np.exp2(np.floor(np.log2(np.abs(np.where(a == 0, 1, a)))) - 7)
    return np.where(np.abs(r) > np.abs(a), r - np.sign(a) * step, r)


def _round_ties_away(a):
    a = np.asarray(a, np.float64)
    r = reference.round_bf16(a)
    e = np.floor(np.log2(np.abs(np.where(a == 0, 1, a))))
    step = np.exp2(e - 7)
    tie = np.abs(a / step - np.trunc(a / step)) == 0.5
    return np.where(tie, np.sign(a) * (np.abs(np.trunc(a / step)) + 1) * step, r)


def _rmsnorm_no_sqrt(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / (np.mean(x * x, axis=1, keepdims=True) + eps) * gamma


def _rmsnorm_eps_outside(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / (np.sqrt(np.mean(x * x, axis=1, keepdims=True)) + eps) * gamma


def _rmsnorm_sum(x, gamma, eps):
    x = np.asarray(x, np.float64)
    return x / np.sqrt(np.sum(x * x, axis=1, keepdims=True) + eps) * gamma


def _silu_on_up(g, u):
    return reference.silu_mul(u, g)


def _silu_sign(g, u):
    g = np.asarray(g, np.float64)
    return g / (1.0 + np.exp(g)) * u


def _sgmm_variant(kind):
    def sgmm(x, W0, A, B, idx, gate, tokens=None):
        x, W0, A, B, gate = (np.asarray(a, np.float64) for a in (x, W0, A, B, gate))
        rows = np.arange(x.shape[0]) if tokens is None else np.asarray(tokens)
        y = x[rows] @ W0.T
        k = idx.shape[1]
        for o, t in enumerate(rows):
            for j in range(k):
                e = int(idx[t, j])
                if kind == "gate_slot_swapped":
                    gv = gate[t, (j + 1) % k]
                elif kind == "gate_dropped":
                    gv = 1.0
                else:
                    gv = gate[t, j]
                if kind == "first_adapter_only":
                    e = int(idx[t, 0])
                u = A[e] @ x[t]
                if kind == "sign":
                    gv = -gv
                if kind == "A_transposed_use":
                    # reads A's rows as if they were indexed by the output (square-ish misuse)
                    u = A[e][:, ::-1] @ x[t]
                y[o] += gv * (B[e] @ u)
                if kind == "delta_dropped_for_last_slot" and j == k - 1:
                    y[o] -= gv * (B[e] @ u)
        return y
    return sgmm


def _topk_highest_index_wins(logits, k):
    l = np.asarray(logits, np.float64)
    T, E = l.shape
    e_ids = np.broadcast_to(np.arange(E)[::-1], (T, E))
    order = np.lexsort((e_ids, -l), axis=-1)
    return order[:, :k].astype(np.int32)


def _topk_rounds_to_fp32(logits, k):
    # ranks logits rounded to fp32: near-equal logits collapse into false ties
    return reference.select_topk(np.asarray(logits, np.float64).astype(np.float32).astype(np.float64), k)


def _topk_ascending(logits, k):
    return reference.select_topk(-np.asarray(logits), k)


def _segment_unstable(idx, E):
    off, perm = reference.segment(idx, E)
    perm = perm.copy()
    for e in range(E):
        perm[off[e]:off[e + 1]] = perm[off[e]:off[e + 1]][::-1]
    return off, perm


def _segment_inclusive(idx, E):
    off, perm = reference.segment(idx, E)
    return np.concatenate([off[1:], off[-1:]]).astype(np.int32), perm


def _gates_full_softmax(logits, idx):
    l = np.asarray(logits, np.float64)
    z = np.exp(l - l.max(1, keepdims=True))
    z = z / z.sum(1, keepdims=True)
    return np.take_along_axis(z, idx.astype(np.int64), axis=1)


def _gates_wrong_shift(logits, idx):
    l = np.asarray(logits, np.float64)
    sel = np.take_along_axis(l, idx.astype(np.int64), axis=1)
    z = np.exp(sel)
    return z / z.sum(1, keepdims=True) * (1 + 1e-9 * sel.shape[1])


def _logits_transposed_weight(x, Wg):
    x, Wg = np.asarray(x, np.float64), np.asarray(Wg, np.float64)
    return x @ Wg[::-1]


MUTANTS = {
    "logits_weight_rows_reversed": dict(router_logits=_logits_transposed_weight),
    "topk_ties_to_highest": dict(select_topk=_topk_highest_index_wins),
    "topk_decides_in_fp32": dict(select_topk=_topk_rounds_to_fp32),
    "topk_ascending": dict(select_topk=_topk_ascending),
    "gates_over_all_E": dict(softmax_gates=_gates_full_softmax),
    "gates_not_normalised_exactly": dict(softmax_gates=_gates_wrong_shift),
    "segment_unstable": dict(segment=_segment_unstable),
    "segment_inclusive_offsets": dict(segment=_segment_inclusive),
    "sgmm_gate_slot_swapped": dict(sgmm=_sgmm_variant("gate_slot_swapped")),
    "sgmm_gate_dropped": dict(sgmm=_sgmm_variant("gate_dropped")),
    "sgmm_first_adapter_only": dict(sgmm=_sgmm_variant("first_adapter_only")),
    "sgmm_sign": dict(sgmm=_sgmm_variant("sign")),
    "sgmm_A_misindexed": dict(sgmm=_sgmm_variant("A_transposed_use")),
    "sgmm_last_slot_dropped": dict(sgmm=_sgmm_variant("delta_dropped_for_last_slot")),
    "round_bf16_toward_zero": dict(round_bf16=_round_toward_zero),
    "round_bf16_ties_away": dict(round_bf16=_round_ties_away),
    "rmsnorm_no_sqrt": dict(rmsnorm=_rmsnorm_no_sqrt),
    "rmsnorm_eps_outside_sqrt": dict(rmsnorm=_rmsnorm_eps_outside),
    "rmsnorm_sum_not_mean": dict(rmsnorm=_rmsnorm_sum),
    "silu_on_up": dict(silu_mul=_silu_on_up),
    "silu_sign": dict(silu_mul=_silu_sign),
    "layer_no_residual_o": dict(decoder_layer=_layer_variant("no_residual_o")),
    "layer_no_residual_down": dict(decoder_layer=_layer_variant("no_residual_down")),
    "layer_attention_from_q": dict(decoder_layer=_layer_variant("attention_from_q")),
    "layer_gamma1_twice": dict(decoder_layer=_layer_variant("gamma1_twice")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    impl = _mutant(**MUTANTS[name])
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(impl)
        except (AssertionError, ValueError, IndexError):
            caught.append(check.__name__)
    assert caught, f"no pin detects mutant {name}"
