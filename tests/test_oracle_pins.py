"""CPU oracle pinned against brute force, closed forms, invariants and golden fixtures."""
import json
import os

import numpy as np
import pytest

import oracle
from oracle import reference
from tests import oracle_pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.mark.parametrize("check", oracle_pins.ALL_CHECKS, ids=lambda f: f.__name__)
def test_pin(check):
    check(reference)


def _golden_files():
    return sorted(f for f in os.listdir(GOLDEN) if f.endswith(".json"))


@pytest.mark.parametrize("name", _golden_files())
def test_golden_fixture(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        g = json.load(fh)
    assert g["citation"]
    dt = g["dtype"]
    arr = lambda key: np.array(g["inputs"][key], dtype=np.uint16 if dt == "bf16" else np.float32)  # noqa: E731
    x, Wg, W0, A, B = (oracle.widen(arr(n), dt) for n in ("x", "Wg", "W0", "A", "B"))
    k, E = g["k"], g["E"]
    idx, gate, logits = oracle.pregate(x, Wg, k)
    exp = g["expected"]
    assert idx.tolist() == exp["topk_idx"]
    np.testing.assert_allclose(gate, np.array(exp["topk_gate"]), rtol=0, atol=1e-12)
    off, perm = oracle.segment(idx, E)
    assert off.tolist() == exp["seg_offsets"] and perm.tolist() == exp["pair_perm"]
    y = oracle.sgmm(x, W0, A, B, idx, gate)
    if g["exact"]:
        assert np.array_equal(y, np.array(exp["y"], dtype=np.float64))
    else:
        np.testing.assert_allclose(y, np.array(exp["y"]), rtol=1e-12, atol=1e-12)


def test_widen_bf16_exact():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x7F7F], dtype=np.uint16)
    w = oracle.widen(bits, "bf16")
    assert w[0] == 1.0 and w[1] == -1.0 and w[3] == 0.0
    assert w[2] == 3.140625
    assert w[4] == (1.0 + 127.0 / 128.0) * 2.0 ** 127  # largest finite bfloat16


def test_margin():
    l = np.array([[3.0, 1.0, 2.0], [0.0, 0.0, -1.0]])
    np.testing.assert_array_equal(reference.topk_margin(l, 1), [1.0, 0.0])
    np.testing.assert_array_equal(reference.topk_margin(l, 3), [np.inf, np.inf])
