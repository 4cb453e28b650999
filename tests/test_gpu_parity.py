"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bars (AdaFuse technical summary §2.A-§2.B defines what is computed):
  * topk_idx, seg_offsets, pair_perm: bit-exact (ties to the lowest index).
    The oracle ranks its fp64 logits, the device its fp32 sums; a token whose
    k-th and (k+1)-th oracle logits lie within twice the fp32 accumulation
    bound of each other may choose either way and is reported (the seeded
    workloads have none).  Exact ties (integer inputs, duplicated router
    columns) are exact on both sides and must match.
  * topk_gate: |dg| <= 1e-5 (fp32 softmax of logits carrying the fp32
    accumulation error, which reaches ~1e-5 for d_in = 4096: a top-2 gate
    moves by at most a quarter of the logit difference's error, plus a few
    ulp); 1e-6 where the logits are exact (integer inputs).
  * y, fp32: max|y - ref| <= 1e-4 max|ref| and |y - ref| <= 1e-4 |ref| where
    |ref| >= 1e-2 max|ref|.
  * y, bf16: max|y - ref| <= 2e-2 max|ref| (per projection output).
  * exact-integer inputs: bit-exact.
"""
import json
import os
import sys

import numpy as np
import pytest

import oracle
from rank_pregate_amd import datagen

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rank_pregate_amd as rp  # noqa: E402
from rank_pregate_amd.workload import DeviceWorkload, to_device, to_host  # noqa: E402

DEV = torch.device("cuda:0")
EPS32 = 2.0 ** -24


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def widen(a, dt):
    return oracle.widen(a, dt)


def dl_widen(t, dt):
    return widen(to_host(t), dt)


def logit_bound(x64, Wg64):
    """Worst-case fp32 accumulation error of the router sum (d terms)."""
    d = x64.shape[1]
    return 1.01 * d * EPS32 * (np.abs(x64) @ np.abs(Wg64)) + 1e-30


def check_y(y_dev, ref, dt, what=""):
    got = dl_widen(y_dev, dt)
    m = np.abs(ref).max()
    err = np.abs(got - ref)
    if dt == "bf16":
        assert err.max() <= 2e-2 * m, f"{what}: max err {err.max():.3e} > 2e-2*{m:.3e}"
    else:
        assert err.max() <= 1e-4 * m, f"{what}: max err {err.max():.3e} > 1e-4*{m:.3e}"
        big = np.abs(ref) >= 1e-2 * m
        rel = err[big] / np.abs(ref[big])
        assert rel.max() <= 1e-4, f"{what}: max rel err {rel.max():.3e}"
    return err.max() / m


def compare_routing(idx_dev, gate_dev, logits_dev, x64, Wg64, k):
    """Oracle pre-gate vs device; returns the mask of tokens that agree."""
    idx_ref, gate_ref, l_ref = oracle.pregate(x64, Wg64, k)
    bound = logit_bound(x64, Wg64)
    if logits_dev is not None:
        l_dev = logits_dev.cpu().numpy().astype(np.float64)
        assert np.all(np.abs(l_dev - l_ref) <= bound), "router logits outside the fp32 accumulation bound"
    idx = idx_dev.cpu().numpy()
    same = np.all(idx == idx_ref, axis=1)
    # near ties: the k-th and (k+1)-th logits closer than twice the bound
    srt = np.sort(l_ref, axis=1)[:, ::-1]
    E = l_ref.shape[1]
    near = np.zeros(len(idx), bool)
    if k < E:
        kth = np.take_along_axis(l_ref, idx_ref[:, k - 1:k].astype(np.int64), 1)[:, 0]
        gap = kth - srt[:, k]
        bmax = bound.max(axis=1)
        near = gap <= 2 * bmax
    for t in np.nonzero(~same)[0]:
        assert near[t], f"token {t}: idx {idx[t]} vs oracle {idx_ref[t]} with a clear margin"
        # the device's choice must be a valid top-k within the bound
        chosen = l_ref[t, idx[t]]
        rest = np.delete(l_ref[t], idx[t])
        assert chosen.min() >= rest.max() - 2 * bound[t].max()
    if (~same).any():
        say(f"near-tie tokens choosing differently: {int((~same).sum())}")
    g = gate_dev.cpu().numpy().astype(np.float64)
    assert np.abs(g[same] - gate_ref[same]).max(initial=0) <= 1e-5
    return same, idx_ref, gate_ref


# --------------------------------------------------------------------------- pre-gating

@pytest.mark.parametrize("name", datagen.WORKLOAD_ORDER)
def test_pregate_workload(name):
    say("pregate", name)
    wl = datagen.WORKLOADS[name]
    x, Wg = datagen.router_input(wl), datagen.router_weight(wl)
    xd, Wgd = to_device(x, wl.dtype, DEV), to_device(Wg, wl.dtype, DEV)
    logits = torch.empty((wl.T, wl.E), dtype=torch.float32, device=DEV)
    idx, gate = rp.pregate(xd, Wgd, wl.k, logits=logits)
    torch.cuda.synchronize()
    same, _, _ = compare_routing(idx, gate, logits, widen(x, wl.dtype), widen(Wg, wl.dtype), wl.k)
    assert same.all(), "seeded workloads are chosen free of near ties"


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,d,E,k", [(7, 64, 6, 2), (65, 128, 200, 3), (16, 256, 1024, 8), (3, 32, 1, 1),
                                     (300, 64, 200, 3),   # two-token tiles, 512 threads
                                     (600, 64, 100, 2),   # four-token tiles, 512 threads
                                     (400, 32, 8, 1),     # two-token tiles, 128 threads
                                     (700, 32, 16, 2)])   # four-token tiles, 128 threads
def test_pregate_exact_ties(dt, T, d, E, k):
    """Integer inputs give exact logits; duplicated router columns tie exactly -> lowest index."""
    say("pregate ties", dt, T, d, E, k)
    rng = np.random.default_rng(T * 1000 + E)
    x = rng.integers(-2, 3, (T, d)).astype(np.float32)
    Wg = rng.integers(-2, 3, (d, E)).astype(np.float32)
    if E >= 4:
        Wg[:, E - 1] = Wg[:, 0]
        Wg[:, E // 2] = Wg[:, 1]
    conv = datagen.f32_to_bf16_bits if dt == "bf16" else (lambda a: a)
    xd, Wgd = to_device(conv(x), dt, DEV), to_device(conv(Wg), dt, DEV)
    idx, gate = rp.pregate(xd, Wgd, k)
    torch.cuda.synchronize()
    idx_ref, gate_ref, _ = oracle.pregate(x.astype(np.float64), Wg.astype(np.float64), k)
    np.testing.assert_array_equal(idx.cpu().numpy(), idx_ref)
    assert np.abs(gate.cpu().numpy() - gate_ref).max() <= 1e-6


@pytest.mark.parametrize("T", [1, 255, 256, 257, 512, 513, 1030])
@pytest.mark.parametrize("E", [8, 296, 300])
def test_pregate_tile_sizes(T, E):
    """Router tiles of one, two or four tokens (chosen from T; E = 8, 300) and the matrix-core
    router's 16-token tiles (E = 296) give logits within the fp32 accumulation bound and the
    oracle's top-k away from near ties."""
    say("pregate tile sizes", T, E)
    rng = np.random.default_rng(7 * T + E)
    d, k = 256, 2
    x = datagen.f32_to_bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    Wg = datagen.f32_to_bf16_bits(rng.standard_normal((d, E), dtype=np.float32) / np.float32(16.0))
    xd, Wgd = to_device(x, "bf16", DEV), to_device(Wg, "bf16", DEV)
    logits = torch.empty((T, E), dtype=torch.float32, device=DEV)
    idx, gate = rp.pregate(xd, Wgd, k, logits=logits)
    torch.cuda.synchronize()
    compare_routing(idx, gate, logits, widen(x, "bf16"), widen(Wg, "bf16"), k)


# --------------------------------------------------------------------------- segmentation

@pytest.mark.parametrize("T,k,E", [(1, 1, 1), (32, 2, 8), (64, 1, 4), (256, 2, 256), (4096, 1, 32),
                                   (300, 3, 1024), (5000, 8, 64), (17, 2, 1000), (0, 2, 8), (20, 0, 8)])
def test_segment(T, k, E):
    say("segment", T, k, E)
    idx = datagen.uniform_indices(T + 7 * k + E, T, E, k) if k > 0 else np.zeros((T, 0), np.int32)
    if T >= 10 and E > 4 and k > 0:
        idx[: T // 2, 0] = 3  # a big segment plus many empty ones
        for t in range(T // 2):
            if k > 1 and 3 in idx[t, 1:]:
                idx[t, 1:][idx[t, 1:] == 3] = 4 if idx[t, 0] != 4 else 5
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    idx_d = torch.from_numpy(idx).to(DEV) if idx.size else torch.zeros((T, k), dtype=torch.int32, device=DEV)
    off, perm = rp.segment(idx_d, E)
    torch.cuda.synchronize()
    off_ref, perm_ref = oracle.segment(idx, E)
    np.testing.assert_array_equal(off.cpu().numpy(), off_ref)
    if T * k:
        np.testing.assert_array_equal(perm.cpu().numpy()[: T * k], perm_ref)


def test_segment_counts_out_of_range():
    say("segment out-of-range")
    idx = np.array([[0, 5], [9, 1], [-1, 2], [3, 4]], np.int32)
    ws = torch.zeros(256, dtype=torch.uint8, device=DEV)
    off, perm = rp.segment(torch.from_numpy(idx).to(DEV), 6, ws=ws)
    torch.cuda.synchronize()
    assert int(ws[:4].view(torch.int32).item()) == 2
    valid = [(p, e) for p, e in enumerate(idx.ravel().tolist()) if 0 <= e < 6]
    want_perm = [p for e in range(6) for p, ee in valid if ee == e]
    assert off.cpu().numpy()[-1] == len(valid)
    assert perm.cpu().numpy()[: len(valid)].tolist() == want_perm


# --------------------------------------------------------------------------- fused projection

def _golden(name):
    with open(os.path.join(GOLDEN, name)) as fh:
        return json.load(fh)


@pytest.mark.parametrize("name", ["exact_int_top1_bf16.json", "exact_int_top1_f32.json", "top2_bf16.json"])
def test_golden_end_to_end(name):
    """Golden fixtures (expected values by brute force): router, segments and projection."""
    say("golden", name)
    g = _golden(name)
    dt = g["dtype"]
    npdt = np.uint16 if dt == "bf16" else np.float32
    inp = {n: np.array(g["inputs"][n], dtype=npdt) for n in ("x", "Wg", "W0", "A", "B")}
    dev = {n: to_device(v, dt, DEV) for n, v in inp.items()}
    idx, gate = rp.pregate(dev["x"], dev["Wg"], g["k"])
    off, perm = rp.segment(idx, g["E"])
    (y,) = rp.sgmm_fused([(dev["W0"], dev["A"], dev["B"])], dev["x"], g["E"], g["r"], g["k"], idx, gate, off, perm)
    torch.cuda.synchronize()
    exp = g["expected"]
    assert idx.cpu().numpy().tolist() == exp["topk_idx"]
    assert off.cpu().numpy().tolist() == exp["seg_offsets"]
    assert perm.cpu().numpy()[: g["T"] * g["k"]].tolist() == exp["pair_perm"]
    ref = np.array(exp["y"], dtype=np.float64)
    if g["exact"]:
        if dt == "bf16":
            want = datagen.f32_to_bf16_bits(ref.astype(np.float32))  # exact ints, rounded once
            np.testing.assert_array_equal(to_host(y), want)
        else:
            np.testing.assert_array_equal(to_host(y).astype(np.float64), ref)
    else:
        check_y(y, ref, dt, name)


@pytest.mark.parametrize("d_out,d_in", [(48, 96), (32, 160), (64, 256)])
def test_pack_w0_layout(d_out, d_in):
    """rp_pack_w0 writes the documented block order: chunks of four block columns, each chunk's blocks
    row block by row block (ragged last chunks included), checked against a NumPy placement."""
    say("pack_w0", d_out, d_in)
    rng = np.random.default_rng(4)
    W = datagen.f32_to_bf16_bits(rng.standard_normal((d_out, d_in), dtype=np.float32))
    packed = to_host(rp.pack_w0(to_device(W, "bf16", DEV))).reshape(-1)
    want = np.empty(d_out * d_in, np.uint16)
    nb, n_rb = d_in // 32, d_out // 16
    for rb in range(n_rb):
        for cb in range(nb):
            g = cb // 4
            nbg = min(4, nb - 4 * g)
            o = (4 * g * n_rb + rb * nbg + cb - 4 * g) * 512
            for q in range(64):
                row, col = rb * 16 + q % 16, cb * 32 + (q // 16) * 8
                want[o + 8 * q:o + 8 * q + 8] = W[row, col:col + 8]
    np.testing.assert_array_equal(packed, want)


def _run_projection_case(T, d_in, d_outs, E, r, k, dt, seed, b_scale=0.1, zero_B=False, idx=None, gate=None,
                         tiled=False, ws=None):
    """Random single-group case through route-free inputs; returns max error ratio."""
    rng = np.random.default_rng(seed)
    conv = datagen.f32_to_bf16_bits if dt == "bf16" else (lambda a: a.astype(np.float32))
    x = conv(rng.standard_normal((T, d_in), dtype=np.float32))
    projs, hw = [], []
    for d_out in d_outs:
        W0 = conv(rng.standard_normal((d_out, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
        A = conv(rng.standard_normal((E, r, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
        B = np.zeros((E, d_out, r), np.float32) if zero_B else \
            rng.standard_normal((E, d_out, r), dtype=np.float32) * np.float32(b_scale / np.sqrt(r))
        B = conv(B)
        hw.append((W0, A, B))
        W0d = to_device(W0, dt, DEV)
        projs.append((rp.pack_w0(W0d) if tiled else W0d, to_device(A, dt, DEV), to_device(B, dt, DEV)))
    if idx is None:
        idx = datagen.uniform_indices(seed, T, E, k)
    if gate is None:
        gate = datagen.random_gates(seed, T, k)
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, np.int32)).to(DEV)
    gate_d = torch.from_numpy(np.ascontiguousarray(gate, np.float32)).to(DEV)
    off, perm = rp.segment(idx_d, E)
    xd = to_device(x, dt, DEV)
    ys = rp.sgmm_fused(projs, xd, E, r, k, idx_d, gate_d, off, perm, ws=ws)
    torch.cuda.synchronize()
    x64 = widen(x, dt)
    worst = 0.0
    for (W0, A, B), y in zip(hw, ys):
        ref = oracle.sgmm(x64, widen(W0, dt), widen(A, dt), widen(B, dt), idx, gate.astype(np.float64))
        worst = max(worst, check_y(y, ref, dt, f"T={T} d_in={d_in} d_out={W0.shape[0]}"))
    return worst, ys


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,d_in,d_outs,E,r,k", [
    (1, 64, [64], 4, 8, 1),            # single token
    (33, 72, [200], 5, 16, 2),         # ragged T, d_in % 16 == 8, d_out not a tile multiple
    (64, 256, [128, 96], 16, 8, 2),    # two projections, different widths
    (100, 128, [64, 64, 64], 9, 32, 3),
    (48, 256, [128], 100, 16, 2),      # decode, E > 32: shrink over segment chunks
    (24, 512, [192], 12, 32, 2),       # decode, E*r > 128: lane-by-lane expand over dense u
    (64, 256, [128], 8, 16, 4),        # decode, more u pieces than the staged expand holds
    (64, 4096, [4096], 16, 8, 2),      # decode, four token tiles, full width
    (256, 512, [256], 256, 16, 2),     # many adapters, 1-3 tokens per segment
    (257, 256, [136], 7, 64, 1),       # first prefill size, ragged
    (300, 264, [128, 40], 12, 128, 2),  # prefill, k=2, r=128
    (1000, 512, [512], 32, 64, 1),
    (1100, 256, [200], 9, 16, 2),      # 256-token tiles of eight waves, ragged T and d_out
    (300, 128, [96], 6, 8, 1),         # top-1 expand, r = 8 (rank columns past r are zero)
    (200, 256, [128, 64], 10, 32, 1),  # top-1 expand, r = 32, 128-token tiles
])
def test_projection_shapes(dt, T, d_in, d_outs, E, r, k):
    say("projection", dt, T, d_in, d_outs, E, r, k)
    _run_projection_case(T, d_in, d_outs, E, r, k, dt, seed=T + d_in + E)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,d_in,d_outs,E,r,k", [
    (200, 8200, [136], 6, 16, 2),       # K split two ways, ragged last stage and tile
    (130, 12288, [256, 64], 5, 32, 2),  # K split three ways, two projections
    (1030, 12288, [128], 6, 16, 2),     # 256-token tiles, K split three ways
])
def test_projection_long_k(dt, T, d_in, d_outs, E, r, k):
    """Long K.  bf16: the prefill GEMM splits K over few row tiles and sums the partial tiles in
    split order.  fp32: every sum over K runs in 64-column partials (the 1e-4 elementwise bar
    holds at d_in = 12288).  The workspace is exactly rp_sgmm_workspace_size bytes."""
    say("projection long K", dt, T, d_in, d_outs, E, r, k)
    code = rp.RP_BF16 if dt == "bf16" else rp.RP_F32
    n = rp.sgmm_workspace_size(len(d_outs), T, d_in, sum(d_outs), E, r, k, code)
    ws = rp.track_workspace(torch.zeros(n, dtype=torch.uint8, device=DEV))
    _run_projection_case(T, d_in, d_outs, E, r, k, dt, seed=T + d_in + E, ws=ws)


@pytest.mark.parametrize("T,d_in,d_out,E,r,k,dt", [
    (32, 256, 128, 8, 16, 2, "bf16"),   # decode, adapters applied by row tiles of the stacked A
    (48, 256, 96, 40, 16, 3, "bf16"),   # decode, E > 32: segment-chunk shrink
    (100, 128, 64, 8, 16, 2, "bf16"),   # prefill
    (16, 64, 64, 4, 8, 2, "f32"),
])
def test_projection_duplicate_adapters(T, d_in, d_out, E, r, k, dt):
    """A token may name one adapter in two slots (the C ABI allows it): both gated terms count."""
    say("duplicate adapters", T, d_in, d_out, E, r, k, dt)
    idx = datagen.uniform_indices(5 + T, T, E, k)
    idx[::3, 1] = idx[::3, 0]
    gate = datagen.random_gates(5 + T, T, k)
    _run_projection_case(T, d_in, [d_out], E, r, k, dt, seed=T + 3, b_scale=1.0, idx=idx, gate=gate)


@pytest.mark.parametrize("T,d_in,d_outs,E,r,k", [
    (1, 64, [64], 4, 8, 1),
    (33, 96, [208], 5, 16, 2),          # 208 rows: last 64-row tile a quarter full
    (16, 160, [80], 4, 8, 2),           # a full 128-column chunk and a one-block chunk
    (32, 1120, [320], 8, 16, 2),        # K split four ways, last chunk of three blocks
    (64, 256, [128, 96], 16, 8, 2),
    (48, 4096, [4096], 8, 16, 2),
    (100, 128, [64, 64, 64], 9, 32, 3),  # tiled order through the prefill path
    (300, 256, [208, 48], 12, 64, 1),
    (1024, 256, [128, 64], 12, 32, 2),  # 256-token tiles, every stage whole (no clamps)
    (1040, 96, [208], 5, 16, 1),        # 256-token tiles, last stage half past d_in
])
def test_projection_tiled_w0(T, d_in, d_outs, E, r, k):
    say("projection tiled", T, d_in, d_outs, E, r, k)
    _run_projection_case(T, d_in, d_outs, E, r, k, "bf16", seed=T + 7 * d_in + E, tiled=True)


@pytest.mark.parametrize("T,d_in,d_outs,E,r,k", [
    (64, 4096, [512], 16, 8, 2),             # 4 tiles of 128 rows: the most K splits a phase takes
    (40, 1000, [1200], 12, 16, 2),           # ragged K (8 chunks, the last partial) and a ragged last tile
    (64, 11008, [256], 16, 8, 2),            # long K: at least the long-K split count
    (50, 2048, [4096, 4096, 1024], 8, 16, 2),  # 72 tiles over three projections
    (64, 4096, [11008], 16, 8, 2),           # 86 tiles: few splits, several items past the CUs' count
])
def test_decode_phase_splits(T, d_in, d_outs, E, r, k):
    """Decode launches of 128-row tiles that leave CUs free: the K splits come from the planner's
    estimate of the phase (1 to 4 backbone splits, up to 8 for the shrink); outputs against the oracle
    and bit-identical on a second call."""
    say("phase splits", T, d_in, d_outs, E, r, k)
    _, ys = _run_projection_case(T, d_in, d_outs, E, r, k, "bf16", seed=T + d_in + len(d_outs), b_scale=1.0)
    first = [y.clone() for y in ys]
    _, ys2 = _run_projection_case(T, d_in, d_outs, E, r, k, "bf16", seed=T + d_in + len(d_outs), b_scale=1.0)
    for a, b in zip(first, ys2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "phase splits changed between calls"


@pytest.mark.parametrize("T,d_in,d_outs,E,r,k", [
    (256, 4096, [4096, 1024], 256, 16, 2),   # many adapters, one token tile of 256
    (65, 512, [520, 128], 64, 8, 3),         # 128-token tile, ragged output tile (second half past d_out)
    (200, 12288, [256], 96, 16, 2),          # long K on few tiles: split-K partials, then the fp32 base
    (130, 256, [192, 64, 320], 40, 8, 4),    # four slots, three projections
    (100, 1024, [384, 136], 48, 32, 2),      # rank 32, two token blocks, ragged 64-row block
    (90, 256, [136], 45, 16, 2),             # odd E, two token blocks, one ragged 64-row block
    (70, 512, [200], 30, 32, 2),             # rank 32, T just past the decode path
])
def test_prefill_split_expand(T, d_in, d_outs, E, r, k):
    """Prefill shapes with many small segments: the GEMM stores fp32 base tiles and the expand runs as a
    launch of its own (per token, each slot's adapter rows read directly); outputs against the oracle,
    bit-identical on a second call."""
    say("split expand", T, d_in, d_outs, E, r, k)
    _, ys = _run_projection_case(T, d_in, d_outs, E, r, k, "bf16", seed=T + E + k, b_scale=1.0)
    first = [y.clone() for y in ys]
    _, ys2 = _run_projection_case(T, d_in, d_outs, E, r, k, "bf16", seed=T + E + k, b_scale=1.0)
    for a, b in zip(first, ys2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "split expand changed between calls"


@pytest.mark.parametrize("T", [32, 300])
def test_projection_zero_B_is_base(T):
    say("zero B", T)
    _, ys = _run_projection_case(T, 256, [128], 8, 16, 2, "bf16", seed=5, zero_B=True)
    _, ys0 = _run_projection_case(T, 256, [128], 8, 16, 0, "bf16", seed=5)
    assert torch.equal(ys[0], ys0[0]), "B = 0 must reproduce the base projection bit for bit"


@pytest.mark.parametrize("T", [48, 512])
def test_projection_single_adapter_merged(T):
    """Every token on one adapter with gate 1: equals x (W0 + B A)^T (merged weight formed on the host)."""
    say("merged weight", T)
    d_in, d_out, E, r = 128, 96, 3, 16
    idx = np.full((T, 1), 2, np.int32)
    gate = np.ones((T, 1), np.float32)
    rng = np.random.default_rng(11)
    conv = datagen.f32_to_bf16_bits
    x = conv(rng.standard_normal((T, d_in), dtype=np.float32))
    W0 = conv(rng.standard_normal((d_out, d_in), dtype=np.float32) * np.float32(0.1))
    A = conv(rng.standard_normal((E, r, d_in), dtype=np.float32) * np.float32(0.1))
    B = conv(rng.standard_normal((E, d_out, r), dtype=np.float32) * np.float32(0.3))
    dv = [to_device(a, "bf16", DEV) for a in (x, W0, A, B)]
    idx_d, gate_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(gate).to(DEV)
    off, perm = rp.segment(idx_d, E)
    (y,) = rp.sgmm_fused([(dv[1], dv[2], dv[3])], dv[0], E, r, 1, idx_d, gate_d, off, perm)
    torch.cuda.synchronize()
    x64, W64, A64, B64 = (widen(a, "bf16") for a in (x, W0, A, B))
    merged = W64 + B64[2] @ A64[2]
    check_y(y, x64 @ merged.T, "bf16", "merged")


@pytest.mark.parametrize("T", [64, 512])
def test_token_permutation(T):
    say("token permutation", T)
    rng = np.random.default_rng(3)
    p = rng.permutation(T)
    d_in, d_out, E, r, k = 256, 128, 8, 16, 2
    idx = datagen.uniform_indices(1, T, E, k)
    gate = datagen.random_gates(1, T, k)
    conv = datagen.f32_to_bf16_bits
    x = conv(rng.standard_normal((T, d_in), dtype=np.float32))
    W0 = conv(rng.standard_normal((d_out, d_in), dtype=np.float32) / np.float32(16))
    A = conv(rng.standard_normal((E, r, d_in), dtype=np.float32) / np.float32(16))
    B = conv(rng.standard_normal((E, d_out, r), dtype=np.float32) / np.float32(4))
    W = [to_device(a, "bf16", DEV) for a in (W0, A, B)]

    def run(xx, ii, gg):
        ii_d, gg_d = torch.from_numpy(np.ascontiguousarray(ii)).to(DEV), torch.from_numpy(np.ascontiguousarray(gg)).to(DEV)
        off, perm = rp.segment(ii_d, E)
        (y,) = rp.sgmm_fused([tuple(W)], to_device(np.ascontiguousarray(xx), "bf16", DEV), E, r, k, ii_d, gg_d, off, perm)
        torch.cuda.synchronize()
        return y

    y = run(x, idx, gate)
    yp = run(x[p], idx[p], gate[p])
    ref = oracle.sgmm(widen(x, "bf16"), widen(W0, "bf16"), widen(A, "bf16"), widen(B, "bf16"), idx, gate.astype(np.float64))
    check_y(yp, ref[p], "bf16", "permuted")
    bit = np.array_equal(to_host(yp), to_host(y)[p])
    say(f"permuted output bit-identical: {bit}")


# --------------------------------------------------------------------------- routing inside the projection launch

def _fused_case(T, d_in, d_outs, E, r, k, dt, seed, tiled=False, ws=None):
    """rp_route_sgmm_fused against the separate calls (routing bit for bit) and the oracle (y)."""
    rng = np.random.default_rng(seed)
    conv = datagen.f32_to_bf16_bits if dt == "bf16" else (lambda a: a.astype(np.float32))
    x = conv(rng.standard_normal((T, d_in), dtype=np.float32))
    Wg = conv(rng.standard_normal((d_in, E), dtype=np.float32) / np.float32(np.sqrt(d_in)))
    projs, hw = [], []
    for d_out in d_outs:
        W0 = conv(rng.standard_normal((d_out, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
        A = conv(rng.standard_normal((E, r, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
        B = conv(rng.standard_normal((E, d_out, r), dtype=np.float32) * np.float32(1.0 / np.sqrt(r)))
        hw.append((W0, A, B))
        W0d = to_device(W0, dt, DEV)
        projs.append((rp.pack_w0(W0d) if tiled else W0d, to_device(A, dt, DEV), to_device(B, dt, DEV)))
    xd, Wgd = to_device(x, dt, DEV), to_device(Wg, dt, DEV)
    ys, idx, gate, off, perm = rp.route_sgmm_fused(projs, xd, Wgd, E, r, k, ws=ws)
    idx2, gate2 = rp.pregate(xd, Wgd, k)
    off2, perm2 = rp.segment(idx2, E)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx2), "fused router indices differ from rp_pregate"
    assert torch.equal(gate.view(torch.int32), gate2.view(torch.int32)), "fused gates differ from rp_pregate"
    assert torch.equal(off, off2) and torch.equal(perm[: T * k], perm2[: T * k]), "fused segments differ"
    x64, Wg64 = widen(x, dt), widen(Wg, dt)
    same, idx_ref, gate_ref = compare_routing(idx, gate, None, x64, Wg64, k)
    assert same.all(), "seeds are chosen free of near ties"
    off_ref, perm_ref = oracle.segment(idx_ref, E)
    np.testing.assert_array_equal(off.cpu().numpy(), off_ref)
    np.testing.assert_array_equal(perm.cpu().numpy()[: T * k], perm_ref)
    worst = 0.0
    for (W0, A, B), y in zip(hw, ys):
        ref = oracle.sgmm(x64, widen(W0, dt), widen(A, dt), widen(B, dt), idx_ref, gate_ref)
        worst = max(worst, check_y(y, ref, dt, f"fused T={T} d_in={d_in} d_out={W0.shape[0]} E={E}"))
    return worst


@pytest.mark.parametrize("T,d_in,d_outs,E,r,k,dt", [
    (1, 64, [64], 4, 8, 1, "bf16"),                   # one token, one router tile
    (17, 256, [96, 32], 40, 16, 2, "bf16"),           # E > 32: shrink over segment chunks
    (32, 4096, [4096, 4096, 4096], 8, 16, 2, "bf16"),  # decode q|k|v shape
    (64, 512, [256], 16, 8, 2, "bf16"),               # 64 tokens (four token tiles)
    (48, 1024, [512], 1024, 32, 8, "bf16"),           # E = 1024: two-token router tiles, k = 8
    (5, 128, [128], 3, 128, 3, "bf16"),               # r = 128
    (100, 256, [128], 8, 16, 2, "bf16"),              # prefill shape: three launches
    (100, 200, [64], 200, 8, 3, "bf16"),              # matrix-core router, split form: ragged K, two column chunks
    (257, 4096, [128], 256, 16, 2, "bf16"),           # matrix-core router, split form: 17 token tiles, ragged last
    (16, 128, [64], 4, 8, 1, "f32"),                  # fp32: three launches
])
def test_route_fused(T, d_in, d_outs, E, r, k, dt):
    say("route fused", T, d_in, d_outs, E, r, k, dt)
    _fused_case(T, d_in, d_outs, E, r, k, dt, seed=31 + T + E)


def test_route_fused_tiled():
    say("route fused tiled")
    _fused_case(32, 1024, [512, 256], 8, 16, 2, "bf16", seed=77, tiled=True)


def test_workspace_shared_across_call_kinds():
    """One workspace through a sequence of fused, separate and differently shaped calls: each
    call starts from the control state the previous one left."""
    say("workspace sequence")
    ws = rp.track_workspace(torch.zeros(64 << 20, dtype=torch.uint8, device=DEV))
    shapes = [(32, 512, [256, 128], 8, 16, 2), (9, 256, [64], 40, 8, 1), (64, 256, [128], 16, 32, 2)]
    for rep in range(3):
        for i, (T, d_in, d_outs, E, r, k) in enumerate(shapes):
            _fused_case(T, d_in, d_outs, E, r, k, "bf16", seed=100 + i, ws=ws)
            _run_projection_case(T, d_in, d_outs, E, r, k, "bf16", seed=200 + i, ws=ws)


# --------------------------------------------------------------------------- multi-group steps

def _group_weights(rng, d_in, d_outs, E, r, dt, b_scale=1.0):
    conv = datagen.f32_to_bf16_bits if dt == "bf16" else (lambda a: a.astype(np.float32))
    hw, dev = [], []
    for d_out in d_outs:
        W0 = conv(rng.standard_normal((d_out, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
        A = conv(rng.standard_normal((E, r, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
        B = conv(rng.standard_normal((E, d_out, r), dtype=np.float32) * np.float32(b_scale / np.sqrt(r)))
        hw.append((W0, A, B))
        dev.append((to_device(W0, dt, DEV), to_device(A, dt, DEV), to_device(B, dt, DEV)))
    return hw, dev


@pytest.mark.parametrize("T,specs,E,r,k,route", [
    (32, [(512, [256, 128, 128]), (256, [512]), (512, [384])], 8, 16, 2, True),   # routing inside, three groups
    (17, [(256, [96]), (96, [256])], 40, 16, 2, False),                            # E > 32, routing given
    (64, [(256, [128, 64]), (128, [256])], 16, 8, 2, True),                         # T = 64: routing launched first
    (100, [(128, [64]), (64, [128])], 8, 16, 2, True),                              # prefill shapes, group by group
    (9, [(128, [64])] * 11, 6, 8, 1, True),                                        # more groups than one launch holds
])
def test_step_groups(T, specs, E, r, k, route):
    """rp_sgmm_step: every group against the oracle with the step's routing."""
    say("step", T, len(specs), E, r, k, route)
    rng = np.random.default_rng(T * 7 + len(specs))
    dt = "bf16"
    conv = datagen.f32_to_bf16_bits
    groups, hws, xs = [], [], []
    for d_in, d_outs in specs:
        hw, dev = _group_weights(rng, d_in, d_outs, E, r, dt)
        x = conv(rng.standard_normal((T, d_in), dtype=np.float32))
        xs.append(x)
        hws.append(hw)
        groups.append(([dv for dv in dev], to_device(x, dt, DEV)))
    Wg = conv(rng.standard_normal((specs[0][0], E), dtype=np.float32) / np.float32(np.sqrt(specs[0][0])))
    if route:
        ys, idx, gate, off, perm = rp.sgmm_step(groups, E, r, k, Wg=to_device(Wg, dt, DEV))
        torch.cuda.synchronize()
        same, idx_ref, gate_ref = compare_routing(idx, gate, None, widen(xs[0], dt), widen(Wg, dt), k)
        assert same.all()
        off_ref, perm_ref = oracle.segment(idx_ref, E)
        np.testing.assert_array_equal(off.cpu().numpy(), off_ref)
        np.testing.assert_array_equal(perm.cpu().numpy()[: T * k], perm_ref)
    else:
        idx_ref = datagen.uniform_indices(T, T, E, k)
        gate_ref = datagen.random_gates(T, T, k).astype(np.float64)
        idx_d = torch.from_numpy(idx_ref).to(DEV)
        gate_d = torch.from_numpy(gate_ref.astype(np.float32)).to(DEV)
        off, perm = rp.segment(idx_d, E)
        ys, *_ = rp.sgmm_step(groups, E, r, k, topk_idx=idx_d, topk_gate=gate_d, seg_offsets=off, pair_perm=perm)
        torch.cuda.synchronize()
    for gi, (hw, gys) in enumerate(zip(hws, ys)):
        x64 = widen(xs[gi], dt)
        for (W0, A, B), y in zip(hw, gys):
            ref = oracle.sgmm(x64, widen(W0, dt), widen(A, dt), widen(B, dt), idx_ref, gate_ref)
            check_y(y, ref, dt, f"step group {gi} d_out={W0.shape[0]}")


@pytest.mark.parametrize("T", [32, 64])
def test_step_chained(T):
    """A group whose input is an earlier group's output in the same call (x_from_call): the later
    group must read what the earlier one wrote."""
    say("step chained", T)
    rng = np.random.default_rng(400 + T)
    dt, E, r, k = "bf16", 8, 16, 2
    conv = datagen.f32_to_bf16_bits
    d = 256
    hw0, dev0 = _group_weights(rng, d, [d, 128], E, r, dt)
    hw1, dev1 = _group_weights(rng, d, [192], E, r, dt)
    hw2, dev2 = _group_weights(rng, 192, [256], E, r, dt)
    x0 = conv(rng.standard_normal((T, d), dtype=np.float32))
    y0 = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    y1 = torch.empty((T, 192), dtype=torch.bfloat16, device=DEV)
    idx = datagen.uniform_indices(T + 1, T, E, k)
    gate = datagen.random_gates(T + 1, T, k)
    idx_d, gate_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(gate).to(DEV)
    off, perm = rp.segment(idx_d, E)
    groups = [([dev0[0] + (y0,), dev0[1]], to_device(x0, dt, DEV)),
              ([dev1[0] + (y1,)], y0, 1),
              ([dev2[0]], y1, 1)]
    for rep in range(3):  # NaN-filled outputs each time: a read before the write would show
        y0.fill_(float("nan"))
        y1.fill_(float("nan"))
        ys, *_ = rp.sgmm_step(groups, E, r, k, topk_idx=idx_d, topk_gate=gate_d, seg_offsets=off, pair_perm=perm)
        torch.cuda.synchronize()
        g64 = gate.astype(np.float64)
        ref0 = oracle.sgmm(widen(x0, dt), *(widen(a, dt) for a in hw0[0]), idx, g64)
        check_y(y0, ref0, dt, "chained group 0")
        ref1 = oracle.sgmm(dl_widen(y0, dt), *(widen(a, dt) for a in hw1[0]), idx, g64)
        check_y(y1, ref1, dt, "chained group 1")
        ref2 = oracle.sgmm(dl_widen(y1, dt), *(widen(a, dt) for a in hw2[0]), idx, g64)
        check_y(ys[2][0], ref2, dt, "chained group 2")


@pytest.mark.parametrize("T", [20, 64])
def test_step_chained_residual(T):
    """A dependent group whose residual is the earlier group's output: y1 = W1 x + adapters, then
    y2 = y1 + W2 y1 + adapters in the same call, read only after y1 is written (NaN-filled before)."""
    say("step chained residual", T)
    rng = np.random.default_rng(900 + T)
    dt, E, r, k = "bf16", 8, 16, 2
    conv = datagen.f32_to_bf16_bits
    d = 512
    hw0, dev0 = _group_weights(rng, d, [d], E, r, dt)
    hw1, dev1 = _group_weights(rng, d, [d], E, r, dt)
    x0 = conv(rng.standard_normal((T, d), dtype=np.float32))
    y0 = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    y1 = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    idx = datagen.uniform_indices(T + 3, T, E, k)
    gate = datagen.random_gates(T + 3, T, k)
    idx_d, gate_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(gate).to(DEV)
    off, perm = rp.segment(idx_d, E)
    groups = [([dev0[0] + (y0,)], to_device(x0, dt, DEV)), ([dev1[0] + (y1, y0)], y0, 1)]
    for rep in range(2):
        y0.fill_(float("nan"))
        y1.fill_(float("nan"))
        rp.sgmm_step(groups, E, r, k, topk_idx=idx_d, topk_gate=gate_d, seg_offsets=off, pair_perm=perm)
        torch.cuda.synchronize()
        g64 = gate.astype(np.float64)
        ref0 = oracle.sgmm(widen(x0, dt), *(widen(a, dt) for a in hw0[0]), idx, g64)
        check_y(y0, ref0, dt, "residual chain: group 0")
        got0 = dl_widen(y0, dt)
        ref1 = oracle.sgmm(got0, *(widen(a, dt) for a in hw1[0]), idx, g64) + got0
        check_y(y1, ref1, dt, "residual chain: group 1")


@pytest.mark.parametrize("T,d,ff", [(9, 512, 2048), (9, 512, 11008), (64, 512, 11008), (64, 4096, 11008)])
def test_step_chained_wide(T, d, ff):
    """gate|up -> down chained in one launch at widths whose K splits are padded to the load ring: the
    dependent group's weight slots fill before its wait, while its input still holds NaN."""
    say("step chained wide", T, d, ff)
    rng = np.random.default_rng(T + ff + d)
    dt, E, r, k = "bf16", 16, 8, 2
    conv = datagen.f32_to_bf16_bits
    hw0, dev0 = _group_weights(rng, d, [ff, ff], E, r, dt)
    hw1, dev1 = _group_weights(rng, ff, [d], E, r, dt)
    x0 = conv(rng.standard_normal((T, d), dtype=np.float32))
    g = torch.full((T, ff), float("nan"), dtype=torch.bfloat16, device=DEV)
    u = torch.full((T, ff), float("nan"), dtype=torch.bfloat16, device=DEV)
    idx = datagen.uniform_indices(T + 7, T, E, k)
    gate = datagen.random_gates(T + 7, T, k)
    idx_d, gate_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(gate).to(DEV)
    off, perm = rp.segment(idx_d, E)
    groups = [([dev0[0] + (g,), dev0[1] + (u,)], to_device(x0, dt, DEV)), ([dev1[0]], u, 1)]
    ys, *_ = rp.sgmm_step(groups, E, r, k, topk_idx=idx_d, topk_gate=gate_d, seg_offsets=off, pair_perm=perm)
    torch.cuda.synchronize()
    g64 = gate.astype(np.float64)
    ref_u = oracle.sgmm(widen(x0, dt), *(widen(a, dt) for a in hw0[1]), idx, g64)
    check_y(u, ref_u, dt, "chained wide: up")
    ref = oracle.sgmm(dl_widen(u, dt), *(widen(a, dt) for a in hw1[0]), idx, g64)
    check_y(ys[1][0], ref, dt, "chained wide: down")


@pytest.mark.parametrize("T", [32, 64])
def test_step_skip_dependency(T):
    """Independent groups do not wait, a dependent one waits for every earlier group: group 2 reads
    group 0's output across an independent group 1."""
    say("step skip dependency", T)
    rng = np.random.default_rng(500 + T)
    dt, E, r, k = "bf16", 8, 16, 2
    conv = datagen.f32_to_bf16_bits
    d = 256
    hw0, dev0 = _group_weights(rng, d, [d], E, r, dt)
    hw1, dev1 = _group_weights(rng, d, [4096], E, r, dt)
    hw2, dev2 = _group_weights(rng, d, [128], E, r, dt)
    hw3, dev3 = _group_weights(rng, d, [512], E, r, dt)
    x0 = conv(rng.standard_normal((T, d), dtype=np.float32))
    x1 = conv(rng.standard_normal((T, d), dtype=np.float32))
    y0 = torch.empty((T, d), dtype=torch.bfloat16, device=DEV)
    idx = datagen.uniform_indices(T + 2, T, E, k)
    gate = datagen.random_gates(T + 2, T, k)
    idx_d, gate_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(gate).to(DEV)
    off, perm = rp.segment(idx_d, E)
    x0_d, x1_d = to_device(x0, dt, DEV), to_device(x1, dt, DEV)
    groups = [([dev0[0] + (y0,)], x0_d), ([dev1[0]], x1_d), ([dev2[0]], y0, 1), ([dev3[0]], x1_d)]
    g64 = gate.astype(np.float64)
    for rep in range(3):
        y0.zero_()
        ys, *_ = rp.sgmm_step(groups, E, r, k, topk_idx=idx_d, topk_gate=gate_d, seg_offsets=off, pair_perm=perm)
        torch.cuda.synchronize()
        ref0 = oracle.sgmm(widen(x0, dt), *(widen(a, dt) for a in hw0[0]), idx, g64)
        check_y(y0, ref0, dt, "group 0")
        check_y(ys[1][0], oracle.sgmm(widen(x1, dt), *(widen(a, dt) for a in hw1[0]), idx, g64), dt, "group 1")
        ref2 = oracle.sgmm(dl_widen(y0, dt), *(widen(a, dt) for a in hw2[0]), idx, g64)
        check_y(ys[2][0], ref2, dt, "group 2")
        check_y(ys[3][0], oracle.sgmm(widen(x1, dt), *(widen(a, dt) for a in hw3[0]), idx, g64), dt, "group 3")


def test_adapter_sensitivity():
    """B without the 0.1 factor: a wrong adapter or gate could not hide under the bf16 tolerance."""
    say("adapter sensitivity")
    T, d, E, r, k = 32, 4096, 8, 16, 2
    idx = datagen.uniform_indices(9, T, E, k)
    gate = datagen.random_gates(9, T, k)
    worst, ys = _run_projection_case(T, d, [d], E, r, k, "bf16", seed=9, b_scale=1.0, idx=idx, gate=gate)
    assert worst < 2e-2
    # the oracle with the two slots' gates swapped differs from the device output beyond the tolerance
    rng = np.random.default_rng(9)
    x = datagen.f32_to_bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
    W0 = datagen.f32_to_bf16_bits(rng.standard_normal((d, d), dtype=np.float32) / np.float32(np.sqrt(d)))
    A = datagen.f32_to_bf16_bits(rng.standard_normal((E, r, d), dtype=np.float32) / np.float32(np.sqrt(d)))
    B = datagen.f32_to_bf16_bits(rng.standard_normal((E, d, r), dtype=np.float32) * np.float32(1.0 / np.sqrt(r)))
    wrong = oracle.sgmm(widen(x, "bf16"), widen(W0, "bf16"), widen(A, "bf16"), widen(B, "bf16"), idx,
                        gate[:, ::-1].astype(np.float64))
    got = dl_widen(ys[0], "bf16")
    assert np.abs(got - wrong).max() > 2e-2 * np.abs(wrong).max()


# --------------------------------------------------------------------------- the workloads end to end

def _oracle_routing(wl):
    x64 = widen(datagen.router_input(wl), wl.dtype)
    Wg64 = widen(datagen.router_weight(wl), wl.dtype)
    if wl.assignment == "zipf":
        idx, gate = datagen.zipf_assignment(wl)
        return idx, gate.astype(np.float64)
    idx, gate, _ = oracle.pregate(x64, Wg64, wl.k)
    return idx, gate


_WL_CACHE = {}


def _device_workload(name):
    """The full-size workload on the device (every layer), built once per test session (all five
    together hold about 15 GB of device memory)."""
    if name not in _WL_CACHE:
        wl = datagen.WORKLOADS[name]
        _WL_CACHE[name] = DeviceWorkload(wl, DEV, per_layer_router=wl.layers > 1)
    return _WL_CACHE[name]


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", datagen.WORKLOAD_ORDER)
def test_workload_end_to_end(name):
    """Full-size workloads in the launch configuration the bench times (every layer of the 32-layer
    step, every token row of the prefill), each output against the oracle."""
    wl = datagen.WORKLOADS[name]
    say("workload", name, "generating + uploading")
    dw = _device_workload(name)
    dw.step()
    torch.cuda.synchronize()
    say("workload", name, "ran; checking")
    idx_ref, gate_ref = _oracle_routing(wl)
    if wl.assignment == "router":
        same, _, _ = compare_routing(dw.topk_idx, dw.topk_gate, None, widen(datagen.router_input(wl), wl.dtype),
                                     widen(datagen.router_weight(wl), wl.dtype), wl.k)
        assert same.all()
    off_ref, perm_ref = oracle.segment(idx_ref, wl.E)
    np.testing.assert_array_equal(dw.seg_offsets.cpu().numpy(), off_ref)
    np.testing.assert_array_equal(dw.pair_perm.cpu().numpy()[: wl.T * wl.k], perm_ref)
    for l in dw.layers:
        worst = 0.0
        for g in wl.groups:
            x64 = widen(datagen.layer_input(wl, l, g.x_name), wl.dtype)
            for p in g.projs:
                w = datagen.proj_weights(wl, l, g, p)
                ref = oracle.sgmm(x64, widen(w.W0, wl.dtype), widen(w.A, wl.dtype), widen(w.B, wl.dtype),
                                  idx_ref, gate_ref)
                del w
                worst = max(worst, check_y(dw.outputs[(l, p)], ref, wl.dtype, f"{name} layer {l} {p}"))
        say(f"{name} layer {l}: worst max|err|/max|ref| = {worst:.2e}")


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", datagen.WORKLOAD_ORDER)
def test_determinism_repeat(name):
    """Ten steps of each full-size workload give bit-identical outputs and routing (split-K partials
    are summed in split order, claimed items and hand-offs do not change any sum's order)."""
    say("determinism", name)
    dw = _device_workload(name)
    dw.step()
    torch.cuda.synchronize()
    first = {key: v.clone() for key, v in dw.outputs.items()}
    route0 = [t.clone() for t in (dw.topk_idx, dw.topk_gate, dw.seg_offsets, dw.pair_perm)]
    for rep in range(1, 10):
        dw.step()
        torch.cuda.synchronize()
        for key, v in dw.outputs.items():
            assert torch.equal(v.view(torch.int16) if v.dtype == torch.bfloat16 else v.view(torch.int32),
                               first[key].view(torch.int16) if v.dtype == torch.bfloat16 else first[key].view(torch.int32)), \
                f"{name}: step {rep} output {key} differs from step 0"
        for a, b in zip((dw.topk_idx, dw.topk_gate, dw.seg_offsets, dw.pair_perm), route0):
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name}: step {rep} routing differs"


# --------------------------------------------------------------------------- baselines on the same kernels

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,d_in,d_outs,E,r,k", [
    (32, 256, [256, 128], 8, 16, 2),
    (9, 512, [320], 5, 128, 3),          # r = 128, ragged rows
    (100, 128, [64], 3, 8, 1),           # segments longer than one 16-pair chunk
    (20, 64, [512], 40, 32, 2),          # most segments empty
])
def test_adapter_apply(dt, T, d_in, d_outs, E, r, k):
    """rp_adapter_apply: a base launch (k = 0) then one launch per adapter equals the fused projection
    (the oracle), including tokens that name one adapter in two slots."""
    say("adapter apply", dt, T, d_in, d_outs, E, r, k)
    rng = np.random.default_rng(T + E + r)
    conv = datagen.f32_to_bf16_bits if dt == "bf16" else (lambda a: a.astype(np.float32))
    hw, dev = [], []
    for d_out in d_outs:
        W0 = conv(rng.standard_normal((d_out, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
        A = conv(rng.standard_normal((E, r, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
        B = conv(rng.standard_normal((E, d_out, r), dtype=np.float32) / np.float32(np.sqrt(r)))
        hw.append((W0, A, B))
        dev.append(tuple(to_device(a, dt, DEV) for a in (W0, A, B)) + (torch.empty((T, d_out), dtype=torch.bfloat16 if dt == "bf16" else torch.float32, device=DEV),))
    idx = datagen.uniform_indices(T + 1, T, E, k)
    if k > 1:
        idx[::4, 1] = idx[::4, 0]
    gate = datagen.random_gates(T + 1, T, k)
    x = conv(rng.standard_normal((T, d_in), dtype=np.float32))
    xd = to_device(x, dt, DEV)
    idx_d, gate_d = torch.from_numpy(idx).to(DEV), torch.from_numpy(gate).to(DEV)
    off, perm = rp.segment(idx_d, E)
    rp.sgmm_fused(dev, xd, E, r, 0)
    for e in range(E):
        rp.adapter_apply(dev, xd, E, r, k, e, gate_d, off, perm)
    torch.cuda.synchronize()
    x64 = widen(x, dt)
    for (W0, A, B), d in zip(hw, dev):
        ref = oracle.sgmm(x64, widen(W0, dt), widen(A, dt), widen(B, dt), idx, gate.astype(np.float64))
        check_y(d[3], ref, dt, "adapter apply")


@pytest.mark.timeout(900)
def test_ablation_per_layer_routing():
    """The router re-run at every layer of the 32-layer step (each layer on its own router and
    input): every layer's routing bit-exact and every output against the oracle."""
    name = "decode_32layer"
    wl = datagen.WORKLOADS[name]
    dw = _device_workload(name)
    say("per-layer routing", name)
    dw.run_per_layer_routing()
    torch.cuda.synchronize()
    for l in dw.layers:
        x_r = datagen.layer_input(wl, l, wl.groups[0].x_name)
        Wg_l = datagen.router_weight(wl, l)
        idx_d, gate_d, off_d, perm_d = dw.layer_routing[l]
        same, idx_ref, gate_ref = compare_routing(idx_d, gate_d, None, widen(x_r, wl.dtype), widen(Wg_l, wl.dtype),
                                                  wl.k)
        assert same.all(), f"layer {l}: near ties"
        off_ref, perm_ref = oracle.segment(idx_ref, wl.E)
        np.testing.assert_array_equal(off_d.cpu().numpy(), off_ref)
        np.testing.assert_array_equal(perm_d.cpu().numpy()[: wl.T * wl.k], perm_ref)
        worst = 0.0
        for g in wl.groups:
            x64 = widen(datagen.layer_input(wl, l, g.x_name), wl.dtype)
            for p in g.projs:
                w = datagen.proj_weights(wl, l, g, p)
                ref = oracle.sgmm(x64, widen(w.W0, wl.dtype), widen(w.A, wl.dtype), widen(w.B, wl.dtype),
                                  idx_ref, gate_ref)
                worst = max(worst, check_y(dw.outputs[(l, p)], ref, wl.dtype, f"per-layer L{l} {p}"))
        say(f"per-layer routing layer {l}: worst {worst:.2e}")


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode_qkvo", "decode_many_adapters", "decode_32layer"])
def test_ablation_unfused(name):
    """Pre-gating once, then a base launch and one launch per adapter for every group: every output
    against the oracle."""
    wl = datagen.WORKLOADS[name]
    dw = _device_workload(name)
    say("unfused", name)
    for y in dw.outputs.values():
        y.zero_()
    dw.run_unfused()
    torch.cuda.synchronize()
    idx_ref, gate_ref = _oracle_routing(wl)
    for l in dw.layers:
        worst = 0.0
        for g in wl.groups:
            x64 = widen(datagen.layer_input(wl, l, g.x_name), wl.dtype)
            for p in g.projs:
                w = datagen.proj_weights(wl, l, g, p)
                ref = oracle.sgmm(x64, widen(w.W0, wl.dtype), widen(w.A, wl.dtype), widen(w.B, wl.dtype),
                                  idx_ref, gate_ref)
                worst = max(worst, check_y(dw.outputs[(l, p)], ref, wl.dtype, f"unfused {name} L{l} {p}"))
        say(f"unfused {name} layer {l}: worst {worst:.2e}")


def _unpack_tiled(packed, d_out, d_in):
    """Row-major [d_out, d_in] from the tiled order (chunks of four 16x32 blocks, each chunk's blocks
    row block by row block; a block's 64 groups of 8 columns, group q = row q%16, columns 8*(q//16)+)."""
    flat = np.asarray(packed).reshape(-1)
    out = np.empty((d_out, d_in), flat.dtype)
    nb, n_rb = d_in // 32, d_out // 16
    for rb in range(n_rb):
        for cb in range(nb):
            g = cb // 4
            nbg = min(4, nb - 4 * g)
            o = (4 * g * n_rb + rb * nbg + cb - 4 * g) * 512
            blk = flat[o:o + 512].reshape(4, 16, 8)  # [column group][row][8 columns]
            out[rb * 16:rb * 16 + 16, cb * 32:cb * 32 + 32] = blk.transpose(1, 0, 2).reshape(16, 32)
    return out


def _ulp_bf16(v):
    """Spacing of bfloat16 numbers at |v| (8 significant bits)."""
    a = np.maximum(np.abs(v), 2.0 ** -126)
    return 2.0 ** (np.floor(np.log2(a)) - 7)


@pytest.mark.parametrize("dt,tiled", [("bf16", False), ("bf16", True), ("f32", False)])
@pytest.mark.parametrize("d_out,d_in,E,r,sel", [
    (256, 512, 6, 16, [2, 5]),
    (96, 1024, 4, 128, [3]),            # r = 128: several LDS stages of rank columns
    (160, 4096, 8, 8, [7, 0, 7]),       # an adapter named twice; ragged row tile
])
def test_merge_infer_unmerge(dt, tiled, d_out, d_in, E, r, sel):
    """The pages' literal decoding steps for one token: merging its adapters into W0 gives
    W0 + sum_j g_j B_j A_j to one rounding of W0's type; the backbone alone on the merged W0 equals
    the factorised fused projection (and the oracle); unmerging restores W0 up to rounding."""
    if tiled and dt != "bf16":
        pytest.skip("the tiled order is bf16 only")
    say("merge", dt, tiled, d_out, d_in, E, r, sel)
    rng = np.random.default_rng(d_out + d_in + r)
    conv = datagen.f32_to_bf16_bits if dt == "bf16" else (lambda a: a.astype(np.float32))
    W0 = conv(rng.standard_normal((d_out, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
    A = conv(rng.standard_normal((E, r, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
    B = conv(rng.standard_normal((E, d_out, r), dtype=np.float32) / np.float32(np.sqrt(r)))
    x = conv(rng.standard_normal((1, d_in), dtype=np.float32))
    g = datagen.random_gates(d_in, 1, len(sel))[0]
    W0d = to_device(W0, dt, DEV)
    W0t = rp.pack_w0(W0d) if tiled else W0d.clone()
    Ad, Bd, xd = (to_device(a, dt, DEV) for a in (A, B, x))
    sel_d = torch.tensor(sel, dtype=torch.int32, device=DEV)
    g_d = torch.from_numpy(g).to(DEV)
    # merge
    rp.merge_adapters(W0t, Ad, Bd, sel_d, g_d, 1.0)
    W0_64, A64, B64 = widen(W0, dt), widen(A, dt), widen(B, dt)
    exact = W0_64 + sum(float(gj) * (B64[e] @ A64[e]) for e, gj in zip(sel, g))
    (y_merged,) = rp.sgmm_fused([(W0t, Ad, Bd)], xd, E, r, 0)
    torch.cuda.synchronize()
    if not tiled:
        got = widen(to_host(W0t), dt)
        if dt == "bf16":
            slack = 2.0 ** -20 * np.abs(exact).max()  # the fp32 rank sum where W0 and the delta cancel
            assert np.all(np.abs(got - exact) <= _ulp_bf16(exact) + slack), "merged W0 beyond one bf16 ulp"
        else:
            assert np.abs(got - exact).max() <= 1e-5 * np.abs(exact).max()
    # the backbone on the merged W0 = x (W0 + sum g B A)^T = the factorised projection
    ref = widen(x, dt)
    ref_y = ref @ exact.T
    check_y(y_merged, ref_y, dt, "backbone on the merged weight")
    idx = torch.tensor([sel], dtype=torch.int32, device=DEV)
    gate = torch.from_numpy(g[None, :].copy()).to(DEV)
    off, perm = rp.segment(idx, E)
    (y_fact,) = rp.sgmm_fused([(W0d, Ad, Bd)], xd, E, r, len(sel), idx, gate, off, perm)
    torch.cuda.synchronize()
    check_y(y_fact, oracle.sgmm(ref, W0_64, A64, B64, np.array([sel], np.int32), g[None, :].astype(np.float64)),
            dt, "factorised")
    # unmerge: W0 back up to the two roundings
    rp.merge_adapters(W0t, Ad, Bd, sel_d, g_d, -1.0)
    torch.cuda.synchronize()
    after = to_host(W0t)
    a64 = widen(_unpack_tiled(after, d_out, d_in) if tiled else after, dt)
    drift = np.abs(a64 - W0_64)
    changed = float((drift > 0).mean())
    if dt == "bf16":
        # the merge rounds at the merged value's scale, the unmerge at the original's
        bound = 0.5 * _ulp_bf16(exact) + 0.5 * _ulp_bf16(W0_64) + 2.0 ** -19 * np.abs(exact).max()
        assert np.all(drift <= bound), "unmerge drift beyond the two roundings"
    else:
        assert drift.max() <= 1e-5 * np.abs(exact).max()
    say(f"unmerge: {100 * changed:.2f}% of W0 elements differ from the original (max {drift.max():.2e})")


@pytest.mark.parametrize("T,d_in,d_outs,E,r,k", [
    (20, 8000, [4096, 520], 8, 16, 2),   # ragged last chunk, ragged row tile, split K
    (64, 2000, [4096, 4096], 16, 8, 2),  # 64 tokens (eight-wave, 128-row tiles), ragged K
    (32, 4096, [4096], 40, 16, 2),       # pair-chunk shrink items (E * r beyond the dense form)
    (32, 4096, [4096], 8, 16, 0),        # base only
])
def test_decode_shapes_repeat(T, d_in, d_outs, E, r, k):
    """Decode-kernel shapes at the edges of its item kinds (ragged K chunk and row tile, both tile
    heights, both shrink forms, no adapters): outputs against the oracle, and bit-identical on a
    second call."""
    say("decode shape", T, d_in, d_outs, E, r, k)
    _, ys = _run_projection_case(T, d_in, d_outs, E, r, k, "bf16", seed=T + d_in + E, b_scale=1.0)
    first = [y.clone() for y in ys]
    _, ys2 = _run_projection_case(T, d_in, d_outs, E, r, k, "bf16", seed=T + d_in + E, b_scale=1.0)
    for a, b in zip(first, ys2):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16)), "decode result changed between calls"


def test_fused_step_two_groups():
    """Routing inside the decode launch feeding two groups (three projections, then one)."""
    say("fused step, two groups")
    T, E, r, k, d = 9, 8, 16, 2, 2048
    rng = np.random.default_rng(99)
    conv = datagen.f32_to_bf16_bits
    hw0, dev0 = _group_weights(rng, d, [d, d, d], E, r, "bf16")
    hw1, dev1 = _group_weights(rng, d, [d], E, r, "bf16")
    x0 = conv(rng.standard_normal((T, d), dtype=np.float32))
    x1 = conv(rng.standard_normal((T, d), dtype=np.float32))
    Wg = conv(rng.standard_normal((d, E), dtype=np.float32) / np.float32(np.sqrt(d)))
    groups = [(dev0, to_device(x0, "bf16", DEV)), (dev1, to_device(x1, "bf16", DEV))]
    ys, idx, gate, off, perm = rp.sgmm_step(groups, E, r, k, Wg=to_device(Wg, "bf16", DEV))
    torch.cuda.synchronize()
    same, idx_ref, gate_ref = compare_routing(idx, gate, None, widen(x0, "bf16"), widen(Wg, "bf16"), k)
    assert same.all()
    for hw, xin, gys in ((hw0, x0, ys[0]), (hw1, x1, ys[1])):
        for (W0, A, B), y in zip(hw, gys):
            ref = oracle.sgmm(widen(xin, "bf16"), widen(W0, "bf16"), widen(A, "bf16"), widen(B, "bf16"), idx_ref,
                              gate_ref)
            check_y(y, ref, "bf16", "fused step, two groups")


def test_step_split_expand_routed_graph():
    """Routed prefill-sized step with many small segments: routing and shrink run on the library's second
    stream beside the base GEMM, joined before the expand.  Outputs against the oracle; a HIP graph of
    the call, replayed three times with eager work between the replays, reproduces the eager outputs
    bit for bit."""
    say("split expand, routed, graph")
    T, E, r, k = 256, 96, 16, 2
    rng = np.random.default_rng(123)
    conv = datagen.f32_to_bf16_bits
    specs = [(1024, [1024, 512]), (768, [640])]
    hws, groups, xs = [], [], []
    for d_in, d_outs in specs:
        hw, dv = _group_weights(rng, d_in, d_outs, E, r, "bf16", b_scale=1.0)
        x = conv(rng.standard_normal((T, d_in), dtype=np.float32))
        ys = [torch.empty((T, d), dtype=torch.bfloat16, device=DEV) for d in d_outs]
        hws.append(hw)
        xs.append(x)
        groups.append(([p + (y,) for p, y in zip(dv, ys)], to_device(x, "bf16", DEV)))
    Wg = conv(rng.standard_normal((specs[0][0], E), dtype=np.float32) / np.float32(np.sqrt(specs[0][0])))
    Wg_d = to_device(Wg, "bf16", DEV)
    idx = torch.empty((T, k), dtype=torch.int32, device=DEV)
    gate = torch.empty((T, k), dtype=torch.float32, device=DEV)
    off = torch.empty(E + 1, dtype=torch.int32, device=DEV)
    perm = torch.empty(T * k, dtype=torch.int32, device=DEV)
    ws = torch.zeros(rp.step_workspace_size(groups, E, r, k), dtype=torch.uint8, device=DEV)
    stream = torch.cuda.Stream(device=DEV)
    outs = [y for g in groups for (_, _, _, y) in g[0]]
    with torch.cuda.stream(stream):
        rp.sgmm_step(groups, E, r, k, Wg=Wg_d, topk_idx=idx, topk_gate=gate, seg_offsets=off, pair_perm=perm,
                     ws=ws, stream=stream)
        stream.synchronize()
        eager = [y.clone() for y in outs]
        same, idx_ref, gate_ref = compare_routing(idx, gate, None, widen(xs[0], "bf16"), widen(Wg, "bf16"), k)
        assert same.all()
        for hw, x, (projs, _) in zip(hws, xs, groups):
            for (W0, A, B), (_, _, _, y) in zip(hw, projs):
                ref = oracle.sgmm(widen(x, "bf16"), widen(W0, "bf16"), widen(A, "bf16"), widen(B, "bf16"), idx_ref,
                                  gate_ref)
                check_y(y, ref, "bf16", "split expand, routed")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            rp.sgmm_step(groups, E, r, k, Wg=Wg_d, topk_idx=idx, topk_gate=gate, seg_offsets=off, pair_perm=perm,
                         ws=ws, stream=stream)
        for rep in range(3):
            for y in outs:
                y.fill_(float("nan"))
            idx.fill_(-1)
            stream.synchronize()
            g.replay()
            stream.synchronize()
            for a, b in zip(eager, outs):
                assert torch.equal(a.view(torch.int16), b.view(torch.int16)), f"graph replay {rep} differs"


# --------------------------------------------------------------------------- whole decoder layers

@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("T,d", [(1, 64), (9, 256), (64, 4096), (130, 11008), (3, 65536)])
def test_rmsnorm(dt, T, d):
    """rp_rmsnorm against the oracle's fp64 RMSNorm rounded to the output dtype, in place too."""
    say("rmsnorm", dt, T, d)
    rng = np.random.default_rng(T + d)
    conv = datagen.f32_to_bf16_bits if dt == "bf16" else (lambda a: a.astype(np.float32))
    x = conv(rng.standard_normal((T, d), dtype=np.float32) * np.float32(3.0))
    g = conv((1.0 + 0.1 * rng.standard_normal(d)).astype(np.float32))
    xd, gd = to_device(x, dt, DEV), to_device(g, dt, DEV)
    y = rp.rmsnorm(xd, gd, 1e-5)
    x2 = xd.clone()
    rp.rmsnorm(x2, gd, 1e-5, out=x2)
    torch.cuda.synchronize()
    ref = oracle.rmsnorm(widen(x, dt), widen(g, dt), 1e-5)
    got = dl_widen(y, dt)
    if dt == "bf16":
        # one rounding of an fp32 value within a few ulp of the fp64 one: at most one bf16 step apart
        step = np.abs(oracle.round_bf16(ref)) * 2.0 ** -7 + 1e-30
        assert np.all(np.abs(got - ref) <= step), f"max err {np.abs(got - ref).max():.3e}"
    else:
        assert np.all(np.abs(got - ref) <= 1e-5 * np.abs(ref) + 1e-6)
    assert torch.equal(x2.view(torch.int16) if dt == "bf16" else x2, y.view(torch.int16) if dt == "bf16" else y)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_silu_mul(dt):
    say("silu_mul", dt)
    rng = np.random.default_rng(5)
    T, d = 33, 1000 if dt == "f32" else 1024
    conv = datagen.f32_to_bf16_bits if dt == "bf16" else (lambda a: a.astype(np.float32))
    g = conv(rng.standard_normal((T, d), dtype=np.float32) * np.float32(4.0))
    u = conv(rng.standard_normal((T, d), dtype=np.float32))
    m = rp.silu_mul(to_device(g, dt, DEV), to_device(u, dt, DEV))
    torch.cuda.synchronize()
    ref = oracle.silu_mul(widen(g, dt), widen(u, dt))
    got = dl_widen(m, dt)
    tol = (np.abs(ref) * (2.0 ** -7 if dt == "bf16" else 4e-6)) + 1e-30
    assert np.all(np.abs(got - ref) <= tol), f"max err {np.abs(got - ref).max():.3e}"


@pytest.mark.parametrize("dt,T,d_in,d_out,E", [("bf16", 9, 256, 192, 8), ("bf16", 64, 512, 256, 8),
                                               ("bf16", 300, 256, 384, 8), ("bf16", 160, 256, 384, 64),
                                               ("f32", 16, 128, 64, 8)])
@pytest.mark.parametrize("in_place", [False, True])
def test_projection_residual(dt, T, d_in, d_out, E, in_place):
    """y = residual + W0 x + adapters, one rounding; the residual may be y itself (updated in place).
    (160 tokens over 64 adapters takes the prefill path whose expand is a launch of its own.)"""
    say("residual", dt, T, d_in, d_out, E, in_place)
    rng = np.random.default_rng(T + d_out)
    conv = datagen.f32_to_bf16_bits if dt == "bf16" else (lambda a: a.astype(np.float32))
    r, k = 16, 2
    x = conv(rng.standard_normal((T, d_in), dtype=np.float32))
    W0 = conv(rng.standard_normal((d_out, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
    A = conv(rng.standard_normal((E, r, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
    B = conv(rng.standard_normal((E, d_out, r), dtype=np.float32) / np.float32(np.sqrt(r)))
    res = conv(rng.standard_normal((T, d_out), dtype=np.float32) * np.float32(2.0))
    idx, gate = datagen.uniform_indices(T, T, E, k), datagen.random_gates(T, T, k)
    idx_d = torch.from_numpy(idx.astype(np.int32)).to(DEV)
    gate_d = torch.from_numpy(gate.astype(np.float32)).to(DEV)
    off, perm = rp.segment(idx_d, E)
    res_d = to_device(res, dt, DEV)
    y = res_d if in_place else torch.empty_like(res_d)
    groups = [([(to_device(W0, dt, DEV), to_device(A, dt, DEV), to_device(B, dt, DEV), y, res_d)],
               to_device(x, dt, DEV))]
    rp.sgmm_step(groups, E, r, k, topk_idx=idx_d, topk_gate=gate_d, seg_offsets=off, pair_perm=perm)
    torch.cuda.synchronize()
    ref = widen(res, dt) + oracle.sgmm(widen(x, dt), widen(W0, dt), widen(A, dt), widen(B, dt), idx,
                                       gate.astype(np.float64))
    check_y(y, ref, dt, "residual")


def _act_case(dt, T, d_in, d_ff, seed):
    rng = np.random.default_rng(seed)
    conv = datagen.f32_to_bf16_bits if dt == "bf16" else (lambda a: a.astype(np.float32))
    E, r, k = 8, 16, 2
    x = to_device(conv(rng.standard_normal((T, d_in), dtype=np.float32)), dt, DEV)
    projs = []
    for _ in range(2):
        projs.append(tuple(to_device(conv(a), dt, DEV) for a in (
            rng.standard_normal((d_ff, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)),
            rng.standard_normal((E, r, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)),
            rng.standard_normal((E, d_ff, r), dtype=np.float32) / np.float32(np.sqrt(r)))))
    idx_d = torch.from_numpy(datagen.uniform_indices(seed, T, E, k).astype(np.int32)).to(DEV)
    gate_d = torch.from_numpy(datagen.random_gates(seed, T, k).astype(np.float32)).to(DEV)
    off, perm = rp.segment(idx_d, E)
    return x, projs, (E, r, k), (idx_d, gate_d, off, perm)


@pytest.mark.parametrize("dt,T,d_in,d_ff", [("bf16", 9, 256, 512), ("bf16", 64, 512, 1024), ("bf16", 32, 4096, 11008),
                                            ("bf16", 100, 256, 384), ("f32", 16, 128, 256)])
def test_act_matches_separate(dt, T, d_in, d_ff):
    """A (gate, up) group with RP_ACT_SILU_MUL gives, bit for bit, rp_silu_mul of the group's own outputs
    (fused epilogue for decode shapes, a separate launch otherwise), and up is left as it was."""
    say("act", dt, T, d_in, d_ff)
    x, projs, (E, r, k), rt = _act_case(dt, T, d_in, d_ff, seed=T + d_ff)
    idx_d, gate_d, off, perm = rt
    plain, _, _, _, _ = rp.sgmm_step([(list(projs), x)], E, r, k, topk_idx=idx_d, topk_gate=gate_d,
                                     seg_offsets=off, pair_perm=perm)
    m_sep = rp.silu_mul(plain[0][0], plain[0][1])
    fused, _, _, _, _ = rp.sgmm_step([(list(projs), x, 0, rp.RP_ACT_SILU_MUL)], E, r, k, topk_idx=idx_d,
                                     topk_gate=gate_d, seg_offsets=off, pair_perm=perm)
    torch.cuda.synchronize()
    as_bits = (lambda t: t.view(torch.int16)) if dt == "bf16" else (lambda t: t.view(torch.int32))
    assert torch.equal(as_bits(fused[0][1]), as_bits(plain[0][1])), "up output changed"
    assert torch.equal(as_bits(fused[0][0]), as_bits(m_sep)), "fused activation differs from rp_silu_mul"


def _chain_workload(name_idx, dt, T, d, ff, E, r, k, layers):
    G = datagen.Group
    groups = (G("qkv", ("q", "k", "v"), d, d, "x_attn"), G("o", ("o",), d, d, "x_o"),
              G("gate_up", ("gate", "up"), d, ff, "x_attn"), G("down", ("down",), ff, d, "x_d"))
    return datagen.Workload(f"chain_{name_idx}", name_idx, dt, T=T, d=d, E=E, r=r, k=k, layers=layers,
                            groups=groups, assignment="router")


@pytest.mark.parametrize("index,dt,T,d,ff,E,r,k,layers", [
    (61, "bf16", 9, 256, 512, 8, 8, 2, 2),        # small decode, routing inside the first launch
    (62, "bf16", 64, 4096, 11008, 16, 8, 2, 2),   # the 32-layer decode step's shapes, two layers
    (63, "bf16", 100, 256, 384, 40, 16, 2, 2),    # prefill shapes: residual in the GEMM, activation as a launch
    (64, "f32", 16, 128, 256, 4, 8, 1, 2),        # fp32
])
def test_decoder_layer_chain(index, dt, T, d, ff, E, r, k, layers):
    """Whole decoder layers around the adapted projections, inputs chained (RMSNorm -> q|k|v -> o + residual ->
    RMSNorm -> gate|up with silu(g)*u -> down + residual), routing once on layer 0's normalised input:
    the residual stream after every layer against the oracle's decoder_layer (bf16 rounding at each
    operation's output for bf16)."""
    say("chain", dt, T, d, ff, E, r, k, layers)
    wl = _chain_workload(index, dt, T, d, ff, E, r, k, layers)
    dw = DeviceWorkload(wl, DEV, b_scale=1.0)
    dw.run_chained()
    torch.cuda.synchronize()
    rnd = oracle.round_bf16 if dt == "bf16" else (lambda a: np.asarray(a, np.float64))
    h0 = widen(datagen.residual_input(wl), dt)
    Wg = widen(datagen.router_weight(wl), dt)
    ws = []
    for l in range(layers):
        w = {g: widen(datagen.norm_weight(wl, l, g), dt) for g in ("gamma1", "gamma2")}
        for g in wl.groups:
            for p in g.projs:
                pw = datagen.proj_weights(wl, l, g, p, b_scale=1.0)
                w[p] = (widen(pw.W0, dt), widen(pw.A, dt), widen(pw.B, dt))
        ws.append(w)
    n1 = rnd(oracle.rmsnorm(h0, ws[0]["gamma1"], 1e-5))
    same, idx_ref, gate_ref = compare_routing(dw.topk_idx, dw.topk_gate, None, n1, Wg, k)
    assert same.all(), "seeds are chosen free of near ties"
    h = h0
    for l in range(layers):
        h = oracle.decoder_layer(h, ws[l], idx_ref, gate_ref, 1e-5, rnd=rnd)
    err = check_y(dw.chain_h, h, dt, f"chain after {layers} layers")
    say(f"chain: max error {err:.2e} of max|h|")
    # a dependent group in the launch of the group it reads: the same splits, so the same bits
    separate = dw.chain_h.clone()
    dw.chain_h.zero_()
    dw.run_chained(dependent=True)
    torch.cuda.synchronize()
    assert torch.equal(dw.chain_h, separate), "dependent launches differ from one launch per group"
