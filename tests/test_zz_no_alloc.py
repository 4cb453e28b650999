"""rp_sgmm_step_noalloc (rp_sgmm_step with the library's static workspace) against rp_sgmm_step
with a workspace of its own, through the C ABI: two calls in a row, the second with fewer tokens.

Bars: routing (topk_idx, seg_offsets, pair_perm) bit-exact; gates within 1e-5 of the oracle;
outputs within 2e-2 * max|ref| of rp_sgmm_step's (bf16) -- they run the same kernels, so they are
also expected to be bit-identical, which is reported -- and of the fp64 oracle.
"""
import sys

import numpy as np
import pytest

import oracle
from rank_pregate_amd import datagen

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():  # pragma: no cover - CPU container
    pytest.skip("no GPU", allow_module_level=True)

import rank_pregate_amd as rp  # noqa: E402
from rank_pregate_amd.workload import to_device, to_host  # noqa: E402

DEV = torch.device("cuda:0")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def _weights(rng, d_in, d_outs, E, r):
    conv = datagen.f32_to_bf16_bits
    hw = []
    for d_out in d_outs:
        W0 = conv(rng.standard_normal((d_out, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
        A = conv(rng.standard_normal((E, r, d_in), dtype=np.float32) / np.float32(np.sqrt(d_in)))
        B = conv(rng.standard_normal((E, d_out, r), dtype=np.float32) / np.float32(np.sqrt(r)))
        hw.append((W0, A, B))
    return hw


def _check_bf16(got_t, ref, what):
    got = oracle.widen(to_host(got_t), "bf16")
    m = np.abs(ref).max()
    err = np.abs(got - ref).max()
    assert err <= 2e-2 * m, f"{what}: max err {err:.3e} > 2e-2*{m:.3e}"


def test_noalloc_matches_step_twice():
    d, E, r, k = 1024, 8, 16, 2
    rng = np.random.default_rng(2718)
    hw_qkv = _weights(rng, d, [d, 256, 256], E, r)
    hw_o = _weights(rng, d, [d], E, r)
    Wg = datagen.f32_to_bf16_bits(rng.standard_normal((d, E), dtype=np.float32) / np.float32(np.sqrt(d)))
    dev_w = lambda hw: [tuple(to_device(a, "bf16", DEV) for a in w) for w in hw]  # noqa: E731
    W_qkv, W_o, Wg_d = dev_w(hw_qkv), dev_w(hw_o), to_device(Wg, "bf16", DEV)
    for call, T in enumerate((32, 9)):
        say("noalloc call", call, "T", T)
        x = datagen.f32_to_bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
        xo = datagen.f32_to_bf16_bits(rng.standard_normal((T, d), dtype=np.float32))
        xd, xod = to_device(x, "bf16", DEV), to_device(xo, "bf16", DEV)
        groups = [(W_qkv, xd), (W_o, xod)]
        ys_a, idx_a, gate_a, off_a, perm_a = rp.sgmm_step_noalloc(groups, E, r, k, Wg=Wg_d)
        ws = rp.track_workspace(torch.zeros(rp.step_workspace_size(groups, E, r, k), dtype=torch.uint8, device=DEV))
        ys_b, idx_b, gate_b, off_b, perm_b = rp.sgmm_step(groups, E, r, k, Wg=Wg_d, ws=ws)
        torch.cuda.synchronize()
        # routing: bit-exact against the entry point with its own workspace and against the oracle
        assert torch.equal(idx_a, idx_b) and torch.equal(off_a, off_b)
        assert torch.equal(perm_a[: T * k], perm_b[: T * k])
        assert torch.equal(gate_a.view(torch.int32), gate_b.view(torch.int32))
        x64, Wg64 = oracle.widen(x, "bf16"), oracle.widen(Wg, "bf16")
        idx_ref, gate_ref, _ = oracle.pregate(x64, Wg64, k)
        np.testing.assert_array_equal(idx_a.cpu().numpy(), idx_ref)
        assert np.abs(gate_a.cpu().numpy() - gate_ref).max() <= 1e-5
        off_ref, perm_ref = oracle.segment(idx_ref, E)
        np.testing.assert_array_equal(off_a.cpu().numpy(), off_ref)
        np.testing.assert_array_equal(perm_a.cpu().numpy()[: T * k], perm_ref)
        bitwise = True
        for gi, (hw, xin) in enumerate(((hw_qkv, x), (hw_o, xo))):
            xin64 = oracle.widen(xin, "bf16")
            for pi, (W0, A, B) in enumerate(hw):
                ya, yb = ys_a[gi][pi], ys_b[gi][pi]
                _check_bf16(ya, oracle.widen(to_host(yb), "bf16"), f"call {call} group {gi} proj {pi} vs rp_sgmm_step")
                ref = oracle.sgmm(xin64, *(oracle.widen(t, "bf16") for t in (W0, A, B)), idx_ref, gate_ref)
                _check_bf16(ya, ref, f"call {call} group {gi} proj {pi} vs oracle")
                bitwise &= torch.equal(ya.view(torch.int16), yb.view(torch.int16))
        say(f"call {call}: outputs bit-identical to rp_sgmm_step: {bitwise}")


def test_noalloc_rejects_beyond_static_workspace():
    # 4 projections x 4096 tokens x 8 slots x rank 128 of fp32 u alone exceed 64 MiB
    FAKE = 1 << 20
    import ctypes
    proj = (rp.RpProj * 4)(*[rp.RpProj(FAKE, FAKE, FAKE, FAKE, 256, 256, 0, 0)] * 4)
    g = (rp.RpGroup * 1)(rp.RpGroup(ctypes.cast(proj, ctypes.POINTER(rp.RpProj)), 4, 0, FAKE, 256, 256))
    st = rp.lib().rp_sgmm_step_noalloc(g, 1, 4096, 16, 128, 8, None, FAKE, FAKE, FAKE, FAKE, rp.RP_BF16, None)
    assert st == rp.RP_ERR_WORKSPACE and "static" in rp.last_error()
