"""Seeded synthetic inputs for the pre-gated multi-adapter projection.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no router, no top-k, no segmentation, no projection), so
that both the HIP path and the CPU oracle can be fed from it without sharing
any computation.

Workloads follow the shapes of AdaFuse ("Accelerating Dynamic Adapter
Inference via Token-Level Pre-Gating and Fused Kernel Optimization",
section 4, experiments on Llama2-7B / Mistral-7B): hidden size 4096, MLP width
11008, 32 layers.  No trained weights or datasets are used: every tensor is
drawn from a seeded normal law,

    x ~ N(0, 1),  W0, A, Wg ~ N(0, 1/fan_in),  B ~ b_scale * N(0, 1/r)

with b_scale = 0.1 by default.  bf16 tensors are produced from fp32 draws by
round-to-nearest-even and are returned as uint16 bit patterns (numpy has no
bfloat16); fp32 tensors are returned as float32.

Seeds: workload i uses numpy SeedSequence entropy [1000 + i, layer, tensor
code, projection code], so every tensor of every layer can be regenerated on
its own without drawing the others.
"""
from __future__ import annotations

import dataclasses
import os
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

# ----------------------------------------------------------------------------
# workload table
# ----------------------------------------------------------------------------

PROJ_CODES = {"q": 0, "k": 1, "v": 2, "o": 3, "gate": 4, "up": 5, "down": 6, "single": 7}
TENSOR_CODES = {"x": 0, "W0": 1, "A": 2, "B": 3, "Wg": 4, "x_router": 5, "zipf": 6,
                "x_attn": 7, "x_o": 8, "x_d": 9, "h0": 10, "gamma1": 11, "gamma2": 12}


@dataclasses.dataclass(frozen=True)
class Group:
    """Projections that read the same input and are issued as one call."""
    name: str
    projs: Tuple[str, ...]
    d_in: int
    d_out: int
    x_name: str  # which per-layer input feeds the group


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    index: int          # 1-based; seeds derive from 1000 + index
    dtype: str          # "f32" or "bf16"
    T: int
    d: int              # router input width (= hidden size)
    E: int
    r: int
    k: int
    layers: int
    groups: Tuple[Group, ...]
    assignment: str     # "router" or "zipf"
    zipf_s: float = 0.0
    description: str = ""

    @property
    def n_proj_per_layer(self) -> int:
        return sum(len(g.projs) for g in self.groups)


D, INTER = 4096, 11008
_ATTN = (Group("qkv", ("q", "k", "v"), D, D, "x_attn"), Group("o", ("o",), D, D, "x_o"))
_MLP = (Group("gate_up", ("gate", "up"), D, INTER, "x_attn"), Group("down", ("down",), INTER, D, "x_d"))

WORKLOADS: Dict[str, Workload] = {
    "toy_f32": Workload(
        "toy_f32", 1, "f32", T=64, d=512, E=4, r=8, k=1, layers=1,
        groups=(Group("single", ("single",), 512, 512, "x_attn"),), assignment="router",
        description="single 512->512 projection, fp32, T=64, E=4 adapters r=8, top-1, router Wg[512x4]"),
    "decode_qkvo": Workload(
        "decode_qkvo", 2, "bf16", T=32, d=D, E=8, r=16, k=2, layers=1, groups=_ATTN,
        assignment="router",
        description="one Llama-7B-shaped layer's q/k/v/o projections, bf16 decode, T=32, E=8 r=16 top-2"),
    "prefill_mlp": Workload(
        "prefill_mlp", 3, "bf16", T=4096, d=D, E=32, r=64, k=1, layers=1, groups=_MLP,
        assignment="zipf", zipf_s=1.1,
        description="MLP gate/up 4096->11008 and down 11008->4096 prefill, bf16, T=4096, E=32 r=64, "
                    "top-1 Zipf(1.1) token-to-adapter assignment"),
    "decode_many_adapters": Workload(
        "decode_many_adapters", 4, "bf16", T=256, d=D, E=256, r=16, k=2, layers=1,
        groups=_ATTN + _MLP, assignment="router",
        description="one layer q/k/v/o + MLP, bf16 decode, T=256, E=256 r=16 top-2 (segments of 1-3 tokens)"),
    "decode_32layer": Workload(
        "decode_32layer", 5, "bf16", T=64, d=D, E=16, r=8, k=2, layers=32, groups=_ATTN + _MLP,
        assignment="router",
        description="full 32-layer decode step, bf16, T=64, E=16 r=8 top-2, router once at layer 0"),
}

WORKLOAD_ORDER = ["toy_f32", "decode_qkvo", "prefill_mlp", "decode_many_adapters", "decode_32layer"]


# ----------------------------------------------------------------------------
# number formats
# ----------------------------------------------------------------------------

def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round-to-nearest-even); return uint16 bits.

    Inputs are finite by construction (normal draws), so NaN handling is not needed.
    """
    a = np.ascontiguousarray(a, dtype=np.float32)
    bits = a.view(np.uint32)
    bias = ((bits >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((bits + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32 (for building inputs)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------

def _rng(wl: Workload, layer: int, tensor: str, proj: str = "single") -> np.random.Generator:
    ss = np.random.SeedSequence([1000 + wl.index, layer, TENSOR_CODES[tensor], PROJ_CODES[proj]])
    return np.random.default_rng(ss)


_CHUNK = 1 << 22


def _normal(rng_seed: np.random.SeedSequence, shape, std: float, nthreads: int = 0) -> np.ndarray:
    """fp32 normal draws with standard deviation `std`, filled in parallel chunks.

    Chunk c is drawn from child seed c of `rng_seed`, so the result does not
    depend on the number of threads.
    """
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, (n + _CHUNK - 1) // _CHUNK)
    children = rng_seed.spawn(nchunks)
    s = np.float32(std)

    def fill(c):
        lo, hi = c * _CHUNK, min(n, (c + 1) * _CHUNK)
        g = np.random.default_rng(children[c])
        g.standard_normal(hi - lo, dtype=np.float32, out=out[lo:hi])
        out[lo:hi] *= s

    if nthreads <= 0:
        nthreads = min(16, len(os.sched_getaffinity(0)))
    if nchunks == 1 or nthreads == 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(nthreads) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(shape)


def _seed(wl: Workload, layer: int, tensor: str, proj: str = "single") -> np.random.SeedSequence:
    return np.random.SeedSequence([1000 + wl.index, layer, TENSOR_CODES[tensor], PROJ_CODES[proj]])


def _fmt(wl: Workload, a: np.ndarray) -> np.ndarray:
    return a if wl.dtype == "f32" else f32_to_bf16_bits(a)


def router_input(wl: Workload) -> np.ndarray:
    """Token activations the router scores: the input of layer 0's first group."""
    return layer_input(wl, 0, wl.groups[0].x_name)


def router_weight(wl: Workload, layer: int = 0) -> np.ndarray:
    """Wg[d, E], N(0, 1/d): the pre-gating router (layer 0), or the router of `layer` when every
    layer routes on its own (the per-layer routing baseline)."""
    return _fmt(wl, _normal(_seed(wl, layer, "Wg"), (wl.d, wl.E), 1.0 / np.sqrt(wl.d)))


def layer_input(wl: Workload, layer: int, x_name: str) -> np.ndarray:
    width = {g.x_name: g.d_in for g in wl.groups}[x_name]
    return _fmt(wl, _normal(_seed(wl, layer, x_name), (wl.T, width), 1.0))


def residual_input(wl: Workload) -> np.ndarray:
    """h0 [T, d], N(0, 1): the residual stream entering layer 0 of the chained decoder layers."""
    return _fmt(wl, _normal(_seed(wl, 0, "h0"), (wl.T, wl.d), 1.0))


def norm_weight(wl: Workload, layer: int, which: str) -> np.ndarray:
    """RMSNorm weight gamma [d] of `layer` ("gamma1" before attention, "gamma2" before the MLP):
    1 + N(0, 0.1^2)."""
    g = 1.0 + _normal(_seed(wl, layer, which), (wl.d,), 0.1)
    return _fmt(wl, g.astype(np.float32))


@dataclasses.dataclass
class ProjWeights:
    W0: np.ndarray  # [d_out, d_in]
    A: np.ndarray   # [E, r, d_in]
    B: np.ndarray   # [E, d_out, r]


def proj_weights(wl: Workload, layer: int, group: Group, proj: str, b_scale: float = 0.1,
                 zero_B: bool = False) -> ProjWeights:
    d_in, d_out, E, r = group.d_in, group.d_out, wl.E, wl.r
    W0 = _normal(_seed(wl, layer, "W0", proj), (d_out, d_in), 1.0 / np.sqrt(d_in))
    A = _normal(_seed(wl, layer, "A", proj), (E, r, d_in), 1.0 / np.sqrt(d_in))
    if zero_B:
        B = np.zeros((E, d_out, r), dtype=np.float32)
    else:
        B = _normal(_seed(wl, layer, "B", proj), (E, d_out, r), b_scale / np.sqrt(r))
    return ProjWeights(_fmt(wl, W0), _fmt(wl, A), _fmt(wl, B))


def zipf_assignment(wl: Workload) -> Tuple[np.ndarray, np.ndarray]:
    """Forced token-to-adapter assignment with P(e) proportional to (e+1)^-s.

    Drawn i.i.d. per (token, slot) by inverse CDF on the seeded uniform stream;
    a token never receives the same adapter twice (redrawn slots walk to the
    next free adapter).  Gates are 1/k each.  Returns (idx int32 [T,k],
    gate float32 [T,k]).
    """
    rng = _rng(wl, 0, "zipf")
    w = (np.arange(1, wl.E + 1, dtype=np.float64)) ** (-wl.zipf_s)
    cdf = np.cumsum(w / w.sum())
    cdf[-1] = 1.0
    u = rng.random((wl.T, wl.k))
    idx = np.searchsorted(cdf, u, side="right").astype(np.int32)
    idx = np.minimum(idx, wl.E - 1)
    for t in range(wl.T):
        seen = set()
        for j in range(wl.k):
            e = int(idx[t, j])
            while e in seen:
                e = (e + 1) % wl.E
            idx[t, j] = e
            seen.add(e)
    gate = np.full((wl.T, wl.k), 1.0 / wl.k, dtype=np.float32)
    return idx, gate


# ----------------------------------------------------------------------------
# small hand-shaped cases (edge cases and exact-integer inputs)
# ----------------------------------------------------------------------------

def custom_case(seed: int, T: int, d_in: int, d_out: int, E: int, r: int, dtype: str = "bf16",
                b_scale: float = 0.1, integer_range: Optional[int] = None) -> dict:
    """A free-form single-projection case for edge-case tests.

    With integer_range=m every tensor holds integers in [-m, m], so every
    product and partial sum stays exactly representable in fp32 and bf16 for
    the small sizes these cases use.
    """
    rng = np.random.default_rng(np.random.SeedSequence([77, seed, T, d_in, d_out, E, r]))
    if integer_range is not None:
        m = integer_range

        def draw(shape, std):
            return rng.integers(-m, m + 1, size=shape).astype(np.float32)
    else:
        def draw(shape, std):
            return (rng.standard_normal(shape, dtype=np.float32) * np.float32(std)).astype(np.float32)

    x = draw((T, d_in), 1.0)
    W0 = draw((d_out, d_in), 1.0 / np.sqrt(d_in))
    A = draw((E, r, d_in), 1.0 / np.sqrt(d_in))
    B = draw((E, d_out, r), b_scale / np.sqrt(r))
    Wg = draw((d_in, E), 1.0 / np.sqrt(d_in))
    conv = (lambda a: a) if dtype == "f32" else f32_to_bf16_bits
    return dict(x=conv(x), W0=conv(W0), A=conv(A), B=conv(B), Wg=conv(Wg), dtype=dtype)


def uniform_indices(seed: int, T: int, E: int, k: int) -> np.ndarray:
    """Random distinct adapter indices per token (for tests that bypass the router)."""
    rng = np.random.default_rng(np.random.SeedSequence([91, seed, T, E, k]))
    idx = np.empty((T, k), dtype=np.int32)
    for t in range(T):
        idx[t] = rng.choice(E, size=k, replace=False)
    return idx


def random_gates(seed: int, T: int, k: int) -> np.ndarray:
    """Positive per-slot gate weights (not normalised; the projection is linear in them)."""
    rng = np.random.default_rng(np.random.SeedSequence([92, seed, T, k]))
    return rng.uniform(0.1, 1.0, size=(T, k)).astype(np.float32)
