"""Device-resident synthetic workloads and the pre-gated decode/prefill step.

A step is the whole hot path once (AdaFuse technical summary §2.A-§2.B):
route the router input once (rp_pregate), group pairs by adapter
(rp_segment), then every projection group of every layer in dependency order
(q|k|v -> o -> gate|up -> down) through rp_sgmm_step, which runs them in
order inside multi-group launches.  The same gate and segments serve every
layer.  By default the routing runs inside the step's first launch, since the
router's input is the first group's input.

Inputs come from rank_pregate_amd.datagen (seeded); weights are uploaded
once and stay resident in HBM.  `copies` > 1 keeps several copies of the
weights and rotates through them step by step, so repeated steps do not hit
the on-chip caches.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

from . import datagen
from . import pregate as rp_pregate, segment as rp_segment, sgmm_fused as rp_sgmm_fused
from . import route_sgmm_fused as rp_route_sgmm_fused, sgmm_step as rp_sgmm_step, step_workspace_size
from . import sgmm_workspace_size, segment_workspace_size, pack_w0, RP_BF16, RP_F32


def to_device(a: np.ndarray, dtype: str, device):
    """Upload a datagen array: uint16 bf16 bits -> torch.bfloat16, float32 -> torch.float32."""
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device)
        return t.view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def to_host(t) -> np.ndarray:
    """Download: torch.bfloat16 -> uint16 bits, float32 -> float32."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
    return t.detach().cpu().numpy()


@dataclasses.dataclass
class DevProj:
    W0: object
    A: object
    B: object


class DeviceWorkload:
    def __init__(self, wl: datagen.Workload, device="cuda:0", layers: Optional[List[int]] = None,
                 b_scale: float = 0.1, copies: int = 1, packed: bool = True):
        import torch
        self.wl = wl
        self.device = torch.device(device)
        self.layers = list(range(wl.layers)) if layers is None else list(layers)
        self.copies = copies
        dt = wl.dtype
        tdt = torch.bfloat16 if dt == "bf16" else torch.float32
        self.code = RP_BF16 if dt == "bf16" else RP_F32
        up = lambda a: to_device(a, dt, self.device)  # noqa: E731
        # backbone weights in the tiled order the kernels stream fastest (one-time repack)
        self.packed = packed and dt == "bf16" and all(g.d_out % 16 == 0 and g.d_in % 32 == 0 for g in wl.groups)
        upw = (lambda a: pack_w0(up(a))) if self.packed else up
        self.x_router = up(datagen.router_input(wl))
        self.Wg = up(datagen.router_weight(wl))
        # per layer: inputs by name and weights by projection (copy 0)
        self.inputs: Dict[Tuple[int, str], object] = {}
        self.weights: List[Dict[Tuple[int, str], DevProj]] = [dict()]
        for l in self.layers:
            for g in wl.groups:
                if (l, g.x_name) not in self.inputs:
                    self.inputs[(l, g.x_name)] = up(datagen.layer_input(wl, l, g.x_name))
                for p in g.projs:
                    w = datagen.proj_weights(wl, l, g, p, b_scale=b_scale)
                    self.weights[0][(l, p)] = DevProj(upw(w.W0), up(w.A), up(w.B))
                    del w
        for c in range(1, copies):
            self.weights.append({key: DevProj(v.W0.clone(), v.A.clone(), v.B.clone())
                                 for key, v in self.weights[0].items()})
        T, k, E = wl.T, wl.k, wl.E
        self.topk_idx = torch.empty((T, k), dtype=torch.int32, device=self.device)
        self.topk_gate = torch.empty((T, k), dtype=torch.float32, device=self.device)
        self.seg_offsets = torch.empty(E + 1, dtype=torch.int32, device=self.device)
        self.pair_perm = torch.empty(max(1, T * k), dtype=torch.int32, device=self.device)
        self.seg_ws = torch.zeros(segment_workspace_size(T, k, E), dtype=torch.uint8, device=self.device)
        # the choice the projections use: the router's, or a forced (Zipf) one
        self.sel_idx, self.sel_gate = self.topk_idx, self.topk_gate
        if wl.assignment == "zipf":
            fi, fg = datagen.zipf_assignment(wl)
            self.sel_idx = torch.from_numpy(fi).to(self.device)
            self.sel_gate = torch.from_numpy(fg).to(self.device)
        self.outputs: Dict[Tuple[int, str], object] = {}
        for g in wl.groups:
            for l in self.layers:
                for p in g.projs:
                    self.outputs[(l, p)] = torch.empty((T, g.d_out), dtype=tdt, device=self.device)
        ws_bytes = step_workspace_size(self.step_groups(0), E, wl.r, k)
        self.ws = torch.zeros(ws_bytes, dtype=torch.uint8, device=self.device)
        self.step_count = 0

    # -- the hot path --------------------------------------------------------
    def route(self, stream=None):
        wl = self.wl
        # with a forced assignment the router still runs (its cost stays in the
        # step) but the segments follow the forced choice
        rp_pregate(self.x_router, self.Wg, wl.k, self.topk_idx, self.topk_gate, stream=stream)
        rp_segment(self.sel_idx, wl.E, self.seg_offsets, self.pair_perm, ws=self.seg_ws, stream=stream)

    def step_groups(self, copy: int = 0):
        """The step's projection groups in dependency order: (projs, x) per (layer, group)."""
        W = self.weights[copy]
        groups = []
        for l in self.layers:
            for g in self.wl.groups:
                projs = [(W[(l, p)].W0, W[(l, p)].A, W[(l, p)].B, self.outputs[(l, p)]) for p in g.projs]
                groups.append((projs, self.inputs[(l, g.x_name)]))
        return groups

    def can_fuse_route(self) -> bool:
        """The router's input is layer 0's first group input and its choice is the one used."""
        return self.layers[0] == 0 and self.sel_idx is self.topk_idx

    def run(self, copy: int = 0, fused: bool = True, k: Optional[int] = None, n_groups: Optional[int] = None,
            stream=None):
        """One step: routing, then every projection group in order (rp_sgmm_step).  With `fused` the
        router and the segmentation run inside the step's first launch; k = 0 gives the base projections
        only.  n_groups limits the step to its first groups (for timing one launch)."""
        wl = self.wl
        kk = wl.k if k is None else k
        groups = self.step_groups(copy)
        if n_groups is not None:
            groups = groups[:n_groups]
        if kk > 0 and fused and self.can_fuse_route():
            rp_sgmm_step(groups, wl.E, wl.r, kk, Wg=self.Wg, topk_idx=self.topk_idx, topk_gate=self.topk_gate,
                         seg_offsets=self.seg_offsets, pair_perm=self.pair_perm, ws=self.ws, stream=stream)
            return
        if kk > 0:
            self.route(stream)
        rp_sgmm_step(groups, wl.E, wl.r, kk, topk_idx=self.sel_idx if kk else None,
                     topk_gate=self.sel_gate if kk else None, seg_offsets=self.seg_offsets if kk else None,
                     pair_perm=self.pair_perm if kk else None, ws=self.ws, stream=stream)

    def project(self, copy: int = 0, k: Optional[int] = None, stream=None):
        """Every projection group with the routing already in place (no routing work)."""
        wl = self.wl
        kk = wl.k if k is None else k
        rp_sgmm_step(self.step_groups(copy), wl.E, wl.r, kk, topk_idx=self.sel_idx if kk else None,
                     topk_gate=self.sel_gate if kk else None, seg_offsets=self.seg_offsets if kk else None,
                     pair_perm=self.pair_perm if kk else None, ws=self.ws, stream=stream)

    def step(self, stream=None, fused: bool = True):
        self.run(self.step_count % self.copies, fused=fused, stream=stream)
        self.step_count += 1

    def group_bytes(self, gi: int, n_touched: int, k: Optional[int] = None) -> int:
        """Algorithmic bytes of projection group number gi of the step (weights, touched adapters, input, outputs)."""
        wl = self.wl
        kk = wl.k if k is None else k
        g = wl.groups[gi % len(wl.groups)]
        bpe = 2 if wl.dtype == "bf16" else 4
        b = wl.T * g.d_in * bpe
        for _ in g.projs:
            b += g.d_out * g.d_in * bpe + wl.T * g.d_out * bpe
            if kk > 0:
                b += n_touched * wl.r * (g.d_in + g.d_out) * bpe
        return b

    def routing_bytes(self) -> int:
        """Router weight and input, and the routing arrays."""
        wl = self.wl
        bpe = 2 if wl.dtype == "bf16" else 4
        return wl.d * wl.E * bpe + wl.T * wl.d * bpe + wl.T * wl.k * 8 + (wl.E + 1) * 4 + wl.T * wl.k * 4

    # -- accounting ------------------------------------------------------------
    def algorithmic_bytes(self, n_touched: int, k: Optional[int] = None) -> int:
        """Bytes the method must move per step: every W0 once, the touched
        adapters' A and B once, each distinct input and every output once, the
        router weight, and the small routing arrays."""
        wl = self.wl
        kk = wl.k if k is None else k
        bpe = 2 if wl.dtype == "bf16" else 4
        b = 0
        for l in self.layers:
            names = set()
            for g in wl.groups:
                for _ in g.projs:
                    b += g.d_out * g.d_in * bpe
                    if kk > 0:
                        b += n_touched * wl.r * (g.d_in + g.d_out) * bpe
                    b += wl.T * g.d_out * bpe
                if g.x_name not in names:
                    names.add(g.x_name)
                    b += wl.T * g.d_in * bpe
        b += wl.d * wl.E * bpe + wl.T * wl.d * bpe  # router weight and router input
        b += wl.T * wl.k * 8 + (wl.E + 1) * 4 + wl.T * wl.k * 4  # idx, gate, offsets, perm
        return b

    def algorithmic_flops(self, k: Optional[int] = None) -> int:
        wl = self.wl
        kk = wl.k if k is None else k
        f = 2 * wl.T * wl.d * wl.E
        for _ in self.layers:
            for g in wl.groups:
                for _ in g.projs:
                    f += 2 * wl.T * g.d_in * g.d_out + 2 * wl.T * kk * wl.r * (g.d_in + g.d_out)
        return f
