"""Host-only checks of the C ABI: the library loads, exports what the header
declares, and rejects bad arguments before touching the GPU."""
import ctypes
import os
import re

import pytest

import rank_pregate_amd as rp

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rank_pregate.h")

pytestmark = pytest.mark.skipif(not os.path.exists(rp.LIB_PATH), reason="library not built")

FAKE = 1 << 20  # a 16-byte aligned non-null address; never dereferenced (validation fails first)


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rp_[a-z0-9_]+)\s*\(", text)))


def test_header_symbols_exported():
    L = rp.lib()
    names = _declared()
    assert set(names) == set(rp.EXPORTED), names
    for n in names:
        assert hasattr(L, n), n


def test_abi_version():
    assert rp.abi_version() == 7


@pytest.mark.parametrize("ws,nbytes", [(None, 1 << 16), (FAKE + 16, 1 << 16), (FAKE, 4096)])
def test_workspace_status_rejects(ws, nbytes):
    wo, bad = ctypes.c_int32(7), ctypes.c_int32(7)
    st = rp.lib().rp_workspace_status(ws, nbytes, 0, ctypes.byref(wo), ctypes.byref(bad), None)
    assert st == rp.RP_ERR_WORKSPACE and rp.last_error()
    assert wo.value == 7 and bad.value == 7  # nothing read


def test_missing_library_fails_loudly(monkeypatch):
    monkeypatch.setattr(rp, "_lib", None)
    monkeypatch.setattr(rp, "LIB_PATH", "/nonexistent/librank_pregate.so")
    with pytest.raises(RuntimeError, match="no CPU fallback"):
        rp.lib()


def _pregate(**kw):
    a = dict(x=FAKE, T=4, d_in=64, ld_x=64, Wg=FAKE, E=8, k=2, dt=rp.RP_BF16, idx=FAKE, gate=FAKE, logits=None,
             stream=None)
    a.update(kw)
    return rp.lib().rp_pregate(a["x"], a["T"], a["d_in"], a["ld_x"], a["Wg"], a["E"], a["k"], a["dt"], a["idx"],
                               a["gate"], a["logits"], a["stream"])


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), rp.RP_ERR_INVALID_ARG),
    (dict(k=9, E=16), rp.RP_ERR_INVALID_ARG),
    (dict(k=3, E=2), rp.RP_ERR_INVALID_ARG),
    (dict(E=0), rp.RP_ERR_INVALID_ARG),
    (dict(E=1025), rp.RP_ERR_INVALID_ARG),
    (dict(T=-1), rp.RP_ERR_INVALID_ARG),
    (dict(d_in=60, ld_x=64), rp.RP_ERR_INVALID_ARG),
    (dict(ld_x=60), rp.RP_ERR_INVALID_ARG),
    (dict(x=None), rp.RP_ERR_INVALID_ARG),
    (dict(Wg=FAKE + 8), rp.RP_ERR_INVALID_ARG),
    (dict(idx=None), rp.RP_ERR_INVALID_ARG),
    (dict(dt=7), rp.RP_ERR_INVALID_ARG),
])
def test_pregate_rejects(kw, status):
    assert _pregate(**kw) == status
    assert rp.last_error()


def test_pregate_T0_is_noop():
    assert _pregate(T=0, x=None, idx=None, gate=None) == rp.RP_OK


def _segment(**kw):
    a = dict(idx=FAKE, T=4, k=2, E=8, off=FAKE, perm=FAKE, ws=FAKE, ws_bytes=256)
    a.update(kw)
    return rp.lib().rp_segment(a["idx"], a["T"], a["k"], a["E"], a["off"], a["perm"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=9), rp.RP_ERR_INVALID_ARG),
    (dict(E=0), rp.RP_ERR_INVALID_ARG),
    (dict(off=None), rp.RP_ERR_INVALID_ARG),
    (dict(idx=None), rp.RP_ERR_INVALID_ARG),
    (dict(ws=None), rp.RP_ERR_INVALID_ARG),
    (dict(ws_bytes=3), rp.RP_ERR_WORKSPACE),
    (dict(off=FAKE + 2), rp.RP_ERR_INVALID_ARG),
])
def test_segment_rejects(kw, status):
    assert _segment(**kw) == status


def _sgmm(projs=None, **kw):
    a = dict(n_proj=1, x=FAKE, T=32, d_in=256, ld_x=256, E=8, r=16, k=2, idx=FAKE, gate=FAKE, off=FAKE, perm=FAKE,
             dt=rp.RP_BF16, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    if projs is None:
        projs = [rp.RpProj(FAKE, FAKE, FAKE, FAKE, 128, 128, 0, 0)]
    arr = (rp.RpProj * max(1, len(projs)))(*projs)
    return rp.lib().rp_sgmm_fused(arr, a["n_proj"], a["x"], a["T"], a["d_in"], a["ld_x"], a["E"], a["r"], a["k"],
                                  a["idx"], a["gate"], a["off"], a["perm"], a["dt"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_proj=0), rp.RP_ERR_INVALID_ARG),
    (dict(n_proj=5), rp.RP_ERR_INVALID_ARG),
    (dict(r=12), rp.RP_ERR_UNSUPPORTED),
    (dict(r=256), rp.RP_ERR_UNSUPPORTED),
    (dict(k=9), rp.RP_ERR_INVALID_ARG),
    (dict(k=3, E=2), rp.RP_ERR_INVALID_ARG),
    (dict(E=2000), rp.RP_ERR_INVALID_ARG),
    (dict(d_in=100, ld_x=104), rp.RP_ERR_INVALID_ARG),
    (dict(ld_x=200), rp.RP_ERR_INVALID_ARG),
    (dict(x=FAKE + 4), rp.RP_ERR_INVALID_ARG),
    (dict(idx=None), rp.RP_ERR_INVALID_ARG),
    (dict(ws=None), rp.RP_ERR_WORKSPACE),
    (dict(ws=FAKE + 16), rp.RP_ERR_WORKSPACE),
    (dict(T=-5), rp.RP_ERR_INVALID_ARG),
])
def test_sgmm_rejects(kw, status):
    assert _sgmm(**kw) == status
    assert rp.last_error()


@pytest.mark.parametrize("proj,status", [
    (rp.RpProj(FAKE, FAKE, FAKE, FAKE, 100, 104, 0, 0), rp.RP_ERR_INVALID_ARG),   # d_out % 8
    (rp.RpProj(FAKE, FAKE, FAKE, FAKE, 128, 120, 0, 0), rp.RP_ERR_INVALID_ARG),   # ld_y < d_out
    (rp.RpProj(None, FAKE, FAKE, FAKE, 128, 128, 0, 0), rp.RP_ERR_INVALID_ARG),   # null W0
    (rp.RpProj(FAKE, FAKE + 2, FAKE, FAKE, 128, 128, 0, 0), rp.RP_ERR_INVALID_ARG),  # misaligned A
    (rp.RpProj(FAKE, FAKE, FAKE, FAKE, 128, 128, 7, 0), rp.RP_ERR_INVALID_ARG),   # unknown layout
    (rp.RpProj(FAKE, FAKE, FAKE, FAKE, 128, 128, 0, 3), rp.RP_ERR_INVALID_ARG),   # reserved != 0
    (rp.RpProj(FAKE, FAKE, FAKE, FAKE, 136, 136, 1, 0), rp.RP_ERR_UNSUPPORTED),   # tiled needs d_out % 16
])
def test_sgmm_rejects_projection(proj, status):
    assert _sgmm(projs=[proj]) == status


def test_sgmm_tiled_needs_bf16_and_d_in_multiple_of_32():
    proj = rp.RpProj(FAKE, FAKE, FAKE, FAKE, 128, 128, 1, 0)
    assert _sgmm(projs=[proj], dt=rp.RP_F32) == rp.RP_ERR_UNSUPPORTED
    assert _sgmm(projs=[proj], d_in=264, ld_x=264) == rp.RP_ERR_UNSUPPORTED


@pytest.mark.parametrize("args,status", [
    ((FAKE, FAKE + (1 << 24), 128, 256, 0), rp.RP_ERR_UNSUPPORTED),   # fp32
    ((FAKE, FAKE + (1 << 24), 120, 256, 1), rp.RP_ERR_INVALID_ARG),   # d_out % 16
    ((FAKE, FAKE + (1 << 24), 128, 200, 1), rp.RP_ERR_INVALID_ARG),   # d_in % 32
    ((FAKE, FAKE + 1024, 128, 256, 1), rp.RP_ERR_INVALID_ARG),        # overlap
    ((None, FAKE, 128, 256, 1), rp.RP_ERR_INVALID_ARG),
])
def test_pack_w0_rejects(args, status):
    s, d, n, k, dt = args
    assert rp.lib().rp_pack_w0(s, d, n, k, dt, None) == status


def test_sgmm_T0_is_noop():
    assert _sgmm(T=0, x=None, ws=None) == rp.RP_OK


def test_sgmm_k0_needs_no_adapter_buffers_in_validation():
    # k = 0 with null routing buffers passes validation up to the workspace check
    assert _sgmm(k=0, idx=None, gate=None, off=None, perm=None, ws=None) == rp.RP_ERR_WORKSPACE


def test_workspace_sizes():
    L = rp.lib()
    assert L.rp_segment_workspace_size(32, 2, 8) >= 4
    b = L.rp_sgmm_workspace_size(3, 32, 4096, 3 * 4096, 8, 16, 2, rp.RP_BF16)
    assert b >= 3 * 32 * 2 * 16 * 4 and b % 256 == 0
    assert L.rp_sgmm_workspace_size(3, 32, 4096, 3 * 4096, 8, 12, 2, rp.RP_BF16) == 0
    assert L.rp_sgmm_workspace_size(0, 32, 4096, 4096, 8, 16, 2, rp.RP_BF16) == 0
    # prefill sizes need no split-K partials: only the rank-r intermediates
    big = L.rp_sgmm_workspace_size(2, 4096, 4096, 22016, 32, 64, 1, rp.RP_BF16)
    assert big >= 2 * 4096 * 64 * 4


def _route(projs=None, **kw):
    a = dict(n_proj=1, x=FAKE, T=32, d_in=256, ld_x=256, Wg=FAKE, E=8, r=16, k=2, dt=rp.RP_BF16, idx=FAKE,
             gate=FAKE, off=FAKE, perm=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    if projs is None:
        projs = [rp.RpProj(FAKE, FAKE, FAKE, FAKE, 128, 128, 0, 0)]
    arr = (rp.RpProj * max(1, len(projs)))(*projs)
    return rp.lib().rp_route_sgmm_fused(arr, a["n_proj"], a["x"], a["T"], a["d_in"], a["ld_x"], a["Wg"], a["E"],
                                        a["r"], a["k"], a["dt"], a["idx"], a["gate"], a["off"], a["perm"], a["ws"],
                                        a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(k=0), rp.RP_ERR_INVALID_ARG),           # routing needs k >= 1
    (dict(k=9), rp.RP_ERR_INVALID_ARG),
    (dict(E=0), rp.RP_ERR_INVALID_ARG),
    (dict(r=12), rp.RP_ERR_UNSUPPORTED),
    (dict(Wg=None), rp.RP_ERR_INVALID_ARG),
    (dict(Wg=FAKE + 8), rp.RP_ERR_INVALID_ARG),
    (dict(idx=None), rp.RP_ERR_INVALID_ARG),
    (dict(perm=None), rp.RP_ERR_INVALID_ARG),
    (dict(off=FAKE + 2), rp.RP_ERR_INVALID_ARG),
    (dict(ws=None), rp.RP_ERR_WORKSPACE),
    (dict(x=FAKE + 4), rp.RP_ERR_INVALID_ARG),
    (dict(n_proj=5), rp.RP_ERR_INVALID_ARG),
])
def test_route_sgmm_rejects(kw, status):
    assert _route(**kw) == status
    assert rp.last_error()


def test_route_sgmm_T0_is_noop():
    assert _route(T=0, x=None, Wg=None, idx=None, gate=None, off=None, perm=None, ws=None) == rp.RP_OK


def _step(groups=None, n_groups=None, **kw):
    a = dict(T=32, E=8, r=16, k=2, Wg=None, idx=FAKE, gate=FAKE, off=FAKE, perm=FAKE, dt=rp.RP_BF16, ws=FAKE,
             ws_bytes=1 << 30)
    a.update(kw)
    proj = (rp.RpProj * 1)(rp.RpProj(FAKE, FAKE, FAKE, FAKE, 128, 128, 0, 0))
    if groups is None:
        groups = [rp.RpGroup(ctypes.cast(proj, ctypes.POINTER(rp.RpProj)), 1, 0, FAKE, 256, 256)] * 2
    arr = (rp.RpGroup * max(1, len(groups)))(*groups)
    n = len(groups) if n_groups is None else n_groups
    return rp.lib().rp_sgmm_step(arr, n, a["T"], a["E"], a["r"], a["k"], a["Wg"], a["idx"], a["gate"], a["off"],
                                 a["perm"], a["dt"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(n_groups=0), rp.RP_ERR_INVALID_ARG),
    (dict(n_groups=4097), rp.RP_ERR_INVALID_ARG),
    (dict(r=12), rp.RP_ERR_UNSUPPORTED),
    (dict(k=9), rp.RP_ERR_INVALID_ARG),
    (dict(idx=None), rp.RP_ERR_INVALID_ARG),      # routing given: inputs needed
    (dict(Wg=FAKE, k=0), rp.RP_ERR_INVALID_ARG),  # routing computed: k >= 1
    (dict(Wg=FAKE + 8), rp.RP_ERR_INVALID_ARG),
    (dict(ws=None), rp.RP_ERR_WORKSPACE),
    (dict(ws_bytes=1024), rp.RP_ERR_WORKSPACE),
])
def test_step_rejects(kw, status):
    assert _step(**kw) == status
    assert rp.last_error()


def test_step_rejects_bad_group():
    proj = (rp.RpProj * 1)(rp.RpProj(FAKE, FAKE, FAKE, FAKE, 100, 104, 0, 0))  # d_out % 8
    good = (rp.RpProj * 1)(rp.RpProj(FAKE, FAKE, FAKE, FAKE, 128, 128, 0, 0))
    g_bad = rp.RpGroup(ctypes.cast(proj, ctypes.POINTER(rp.RpProj)), 1, 0, FAKE, 256, 256)
    g_ok = rp.RpGroup(ctypes.cast(good, ctypes.POINTER(rp.RpProj)), 1, 0, FAKE, 256, 256)
    assert _step(groups=[g_ok, g_bad]) == rp.RP_ERR_INVALID_ARG
    assert "group 1" in rp.last_error()
    g_flag = rp.RpGroup(ctypes.cast(good, ctypes.POINTER(rp.RpProj)), 1, 2, FAKE, 256, 256)
    assert _step(groups=[g_ok, g_flag]) == rp.RP_ERR_INVALID_ARG


def test_step_T0_is_noop():
    assert _step(T=0, idx=None, gate=None, off=None, perm=None, ws=None) == rp.RP_OK


def test_step_workspace_size():
    L = rp.lib()
    proj = (rp.RpProj * 3)(*[rp.RpProj(FAKE, FAKE, FAKE, FAKE, 4096, 4096, 0, 0)] * 3)
    g = rp.RpGroup(ctypes.cast(proj, ctypes.POINTER(rp.RpProj)), 3, 0, FAKE, 4096, 4096)
    arr = (rp.RpGroup * 10)(*[g] * 10)
    one = L.rp_sgmm_step_workspace_size(arr, 1, 32, 8, 16, 2, rp.RP_BF16)
    ten = L.rp_sgmm_step_workspace_size(arr, 10, 32, 8, 16, 2, rp.RP_BF16)
    assert one > 0 and one % 256 == 0
    # eight groups share one launch's workspace; later launches reuse it
    assert ten >= one and ten <= 8 * one
    assert L.rp_sgmm_step_workspace_size(arr, 0, 32, 8, 16, 2, rp.RP_BF16) == 0
    assert L.rp_sgmm_step_workspace_size(arr, 1, 32, 8, 12, 2, rp.RP_BF16) == 0


@pytest.mark.parametrize("T,d_in,d_outs", [(200, 8200, [136]), (256, 11008, [4096]), (130, 12288, [256, 64]),
                                           (1100, 12288, [128])])
def test_prefill_workspace_covers_split_k(T, d_in, d_outs):
    """A single bf16 prefill group may split K: rp_sgmm_workspace_size covers its partial tiles,
    and agrees with the step size of the same group."""
    L = rp.lib()
    E, r, k = 6, 16, 2
    n = len(d_outs)
    proj = (rp.RpProj * n)(*[rp.RpProj(FAKE, FAKE, FAKE, FAKE, d, d, 0, 0) for d in d_outs])
    g = rp.RpGroup(ctypes.cast(proj, ctypes.POINTER(rp.RpProj)), n, 0, FAKE, d_in, d_in)
    single = L.rp_sgmm_workspace_size(n, T, d_in, sum(d_outs), E, r, k, rp.RP_BF16)
    step = L.rp_sgmm_step_workspace_size((rp.RpGroup * 1)(g), 1, T, E, r, k, rp.RP_BF16)
    u_only = 131072 + ((n * T * k * r * 4 + 255) // 256) * 256  # two 64 KiB control blocks, then u
    tiles = sum((d + 127) // 128 for d in d_outs)
    partials = ((tiles + 7) // 8 * 8) * ((T + 127) // 128) * 2 * 128 * 128 * 4  # at least two splits
    assert single >= u_only + partials
    assert step >= u_only + partials


def _noalloc(groups=None, **kw):
    a = dict(T=32, E=8, r=16, k=2, Wg=None, idx=FAKE, gate=FAKE, off=FAKE, perm=FAKE, dt=rp.RP_BF16)
    a.update(kw)
    proj = (rp.RpProj * 1)(rp.RpProj(FAKE, FAKE, FAKE, FAKE, 128, 128, 0, 0))
    if groups is None:
        groups = [rp.RpGroup(ctypes.cast(proj, ctypes.POINTER(rp.RpProj)), 1, 0, FAKE, 256, 256)]
    arr = (rp.RpGroup * len(groups))(*groups)
    return rp.lib().rp_sgmm_step_noalloc(arr, len(groups), a["T"], a["E"], a["r"], a["k"], a["Wg"], a["idx"],
                                         a["gate"], a["off"], a["perm"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(r=12), rp.RP_ERR_UNSUPPORTED),
    (dict(k=9), rp.RP_ERR_INVALID_ARG),
    (dict(idx=None), rp.RP_ERR_INVALID_ARG),
    (dict(Wg=FAKE, k=0), rp.RP_ERR_INVALID_ARG),
])
def test_noalloc_rejects(kw, status):
    """The static-workspace variant validates like rp_sgmm_step, before any device call."""
    assert _noalloc(**kw) == status
    assert rp.last_error()


def test_noalloc_rejects_beyond_static_workspace_cpu():
    proj = (rp.RpProj * 4)(*[rp.RpProj(FAKE, FAKE, FAKE, FAKE, 256, 256, 0, 0)] * 4)
    g = rp.RpGroup(ctypes.cast(proj, ctypes.POINTER(rp.RpProj)), 4, 0, FAKE, 256, 256)
    assert _noalloc(groups=[g], T=4096, E=16, r=128, k=8) == rp.RP_ERR_WORKSPACE
    assert "static" in rp.last_error()


def test_noalloc_T0_is_noop():
    assert _noalloc(T=0, idx=None, gate=None, off=None, perm=None) == rp.RP_OK
