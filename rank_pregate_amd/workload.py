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
from . import sgmm_workspace_size, segment_workspace_size, pack_w0, track_workspace, RP_BF16, RP_F32
from . import adapter_apply as rp_adapter_apply, merge_adapters as rp_merge_adapters
from . import rmsnorm as rp_rmsnorm, silu_mul as rp_silu_mul, RP_ACT_SILU_MUL


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


CHAIN_EPS = 1e-5  # RMSNorm epsilon of the chained decoder layers


class DeviceWorkload:
    def __init__(self, wl: datagen.Workload, device="cuda:0", layers: Optional[List[int]] = None,
                 b_scale: float = 0.1, copies: int = 1, packed: bool = True, per_layer_router: bool = False):
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
        # one workspace for every call kind made here: the whole step, each group on its own without
        # adapters (the unfused baseline), and one token's step with and without adapters (fewer
        # tiles per launch split K further, so a smaller call can need more)
        groups0 = self.step_groups(0)
        sizes = [step_workspace_size(groups0, E, wl.r, k)]
        sizes += [step_workspace_size([g], E, wl.r, 0) for g in groups0]
        if dt == "bf16":
            tok = self.token_groups(0)
            sizes += [step_workspace_size(tok, E, wl.r, k), step_workspace_size(tok, E, wl.r, 0)]
        self.ws = track_workspace(torch.zeros(max(sizes), dtype=torch.uint8, device=self.device))
        self.step_count = 0
        # per-layer routing baseline: a router per layer on that layer's first input
        self.layer_routing: Dict[int, Tuple] = {}
        self.Wg_layer: Dict[int, object] = {}
        if per_layer_router:
            for l in self.layers:
                self.Wg_layer[l] = up(datagen.router_weight(wl, l))
                self.layer_routing[l] = (
                    torch.empty((T, k), dtype=torch.int32, device=self.device),
                    torch.empty((T, k), dtype=torch.float32, device=self.device),
                    torch.empty(E + 1, dtype=torch.int32, device=self.device),
                    torch.empty(max(1, T * k), dtype=torch.int32, device=self.device))

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

    # -- baselines on the same kernels (AdaFuse technical summary §1 and §4) ---
    def run_per_layer_routing(self, copy: int = 0, stream=None):
        """The router re-run at every layer (per-layer dynamic adapters): each layer's groups in one
        rp_sgmm_step call that first routes that layer's input with that layer's router."""
        wl = self.wl
        if not self.layer_routing:
            raise RuntimeError("build the workload with per_layer_router=True")
        groups = self.step_groups(copy)
        n = len(wl.groups)
        for i, l in enumerate(self.layers):
            idx, gate, off, perm = self.layer_routing[l]
            rp_sgmm_step(groups[i * n:(i + 1) * n], wl.E, wl.r, wl.k, Wg=self.Wg_layer[l], topk_idx=idx,
                         topk_gate=gate, seg_offsets=off, pair_perm=perm, ws=self.ws, stream=stream)

    def run_unfused(self, copy: int = 0, stream=None):
        """Pre-gating once, then per projection group a base launch (k = 0) followed by one launch
        per adapter adding its gated delta (the unfused "simple fusion" form)."""
        wl = self.wl
        self.route(stream)
        for projs, x in self.step_groups(copy):
            rp_sgmm_fused(projs, x, wl.E, wl.r, 0, ws=self.ws, stream=stream)
            for e in range(wl.E):
                rp_adapter_apply(projs, x, wl.E, wl.r, wl.k, e, self.sel_gate, self.seg_offsets, self.pair_perm,
                                 stream=stream)

    # -- one token: the pages' literal merge -> infer -> unmerge, and the factorised form
    def _token_buffers(self):
        import torch
        if not hasattr(self, "tok_idx"):
            wl, dev = self.wl, self.device
            self.tok_idx = torch.empty((1, wl.k), dtype=torch.int32, device=dev)
            self.tok_gate = torch.empty((1, wl.k), dtype=torch.float32, device=dev)
            self.tok_off = torch.empty(wl.E + 1, dtype=torch.int32, device=dev)
            self.tok_perm = torch.empty(max(1, wl.k), dtype=torch.int32, device=dev)
            tdt = self.outputs[next(iter(self.outputs))].dtype
            self.tok_out = {key: torch.empty((1, y.shape[1]), dtype=tdt, device=dev) for key, y in self.outputs.items()}

    def token_groups(self, copy: int = 0, token: int = 0):
        """The step's groups for one token (row `token` of every input), writing tok_out."""
        self._token_buffers()
        W = self.weights[copy]
        groups = []
        for l in self.layers:
            for g in self.wl.groups:
                x = self.inputs[(l, g.x_name)][token:token + 1]
                groups.append(([(W[(l, p)].W0, W[(l, p)].A, W[(l, p)].B, self.tok_out[(l, p)]) for p in g.projs], x))
        return groups

    def run_token_fused(self, copy: int = 0, token: int = 0, stream=None):
        """One token through the factorised fused path (routing inside the step)."""
        wl = self.wl
        groups = self.token_groups(copy, token)
        rp_sgmm_step(groups, wl.E, wl.r, wl.k, Wg=self.Wg, topk_idx=self.tok_idx, topk_gate=self.tok_gate,
                     seg_offsets=self.tok_off, pair_perm=self.tok_perm, ws=self.ws, stream=stream)

    def run_token_merged(self, copy: int = 0, token: int = 0, stream=None):
        """AdaFuse's literal decoding steps 1-5 for one token: route it, merge its k adapters into every
        W0 of the step, run the backbone alone (k = 0), unmerge them."""
        wl = self.wl
        groups = self.token_groups(copy, token)
        rp_pregate(self.x_router[token:token + 1], self.Wg, wl.k, self.tok_idx, self.tok_gate, stream=stream)
        sel, w = self.tok_idx[0], self.tok_gate[0]
        W = self.weights[copy]
        for pw in W.values():
            rp_merge_adapters(pw.W0, pw.A, pw.B, sel, w, 1.0, stream=stream)
        rp_sgmm_step(groups, wl.E, wl.r, 0, ws=self.ws, stream=stream)
        for pw in W.values():
            rp_merge_adapters(pw.W0, pw.A, pw.B, sel, w, -1.0, stream=stream)

    # -- whole decoder layers around the projections (chained inputs) --------
    def prepare_chain(self):
        """Residual stream, norm output and per-layer RMSNorm weights of the chained layers (uploads and
        allocates: call before recording run_chained into a graph)."""
        import torch
        if hasattr(self, "chain_h"):
            return
        wl, dev = self.wl, self.device
        names = [g.name for g in wl.groups]
        if names != ["qkv", "o", "gate_up", "down"]:
            raise RuntimeError("chained layers need the q|k|v, o, gate|up, down groups")
        up = lambda a: to_device(a, wl.dtype, dev)  # noqa: E731
        self.chain_h0 = up(datagen.residual_input(wl))
        self.chain_h = torch.empty_like(self.chain_h0)
        self.chain_n = torch.empty_like(self.chain_h0)
        self.chain_gamma = {(l, w): up(datagen.norm_weight(wl, l, w)) for l in self.layers
                            for w in ("gamma1", "gamma2")}
        attn, mlp = self.chain_groups(0)[0]
        need = max(step_workspace_size(part, wl.E, wl.r, wl.k) for part in [attn, mlp] + [[g] for g in attn + mlp])
        if need > self.ws.numel():
            self.ws = track_workspace(torch.zeros(need, dtype=torch.uint8, device=dev))

    def chain_groups(self, copy: int = 0):
        """Per layer, the two launches' groups of a chained decoder layer:
        ([q|k|v on n1, o on v with residual h -> h], [gate|up on n2 with silu(g)*u, down on m with residual h -> h]).
        Layer 0's o reads the residual from h0 (so every step starts from the same stream)."""
        W, wl = self.weights[copy], self.wl
        out = []
        for i, l in enumerate(self.layers):
            P = lambda p: (W[(l, p)].W0, W[(l, p)].A, W[(l, p)].B)  # noqa: E731
            res = self.chain_h0 if i == 0 else self.chain_h
            v = self.outputs[(l, "v")]
            qkv = ([P("q") + (self.outputs[(l, "q")],), P("k") + (self.outputs[(l, "k")],), P("v") + (v,)],
                   self.chain_n)
            o = ([P("o") + (self.chain_h, res)], v, 1)
            g_out = self.outputs[(l, "gate")]
            gate_up = ([P("gate") + (g_out,), P("up") + (self.outputs[(l, "up")],)], self.chain_n, 0,
                       RP_ACT_SILU_MUL)
            down = ([P("down") + (self.chain_h, self.chain_h)], g_out, 1)
            out.append(([qkv, o], [gate_up, down]))
        return out

    def run_chained(self, copy: int = 0, stream=None, dependent: bool = False):
        """Every layer as a whole decoder layer (RMSNorm, q|k|v, o + residual, RMSNorm, gate|up with the
        fused silu(g)*u, down + residual), inputs chained from the outputs before them; the routing runs
        inside the first launch, on layer 0's normalised input.  The residual stream ends in chain_h.

        Each projection group is a launch of its own; with `dependent` a group that reads the group before
        it shares that group's launch instead (it waits there for every tile of it).  Both give the same
        bits."""
        self.prepare_chain()
        wl = self.wl
        first = True

        def launch(groups):
            nonlocal first
            route = dict(Wg=self.Wg) if first else {}
            first = False
            rp_sgmm_step(groups, wl.E, wl.r, wl.k, topk_idx=self.topk_idx, topk_gate=self.topk_gate,
                         seg_offsets=self.seg_offsets, pair_perm=self.pair_perm, ws=self.ws, stream=stream, **route)

        for i, (l, (attn, mlp)) in enumerate(zip(self.layers, self.chain_groups(copy))):
            rp_rmsnorm(self.chain_h0 if i == 0 else self.chain_h, self.chain_gamma[(l, "gamma1")], CHAIN_EPS,
                       out=self.chain_n, stream=stream)
            for part in ([attn] if dependent else [[g] for g in attn]):
                launch(part)
            rp_rmsnorm(self.chain_h, self.chain_gamma[(l, "gamma2")], CHAIN_EPS, out=self.chain_n, stream=stream)
            for part in ([mlp] if dependent else [[g] for g in mlp]):
                launch(part)

    def run_variant(self, variant: str, copy: int = 0, stream=None):
        if variant == "fused":
            self.run(copy, stream=stream)
        elif variant == "per_layer_routing":
            self.run_per_layer_routing(copy, stream=stream)
        elif variant == "unfused":
            self.run_unfused(copy, stream=stream)
        elif variant == "token_fused":
            self.run_token_fused(copy, stream=stream)
        elif variant == "token_merge_unmerge":
            self.run_token_merged(copy, stream=stream)
        elif variant == "chained_layers":
            self.run_chained(copy, stream=stream)
        elif variant == "chained_layers_dependent":
            self.run_chained(copy, stream=stream, dependent=True)
        else:
            raise ValueError(variant)

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

    def group_flops(self, gi: int, k: Optional[int] = None) -> int:
        """Algorithmic FLOPs of projection group number gi of the step."""
        wl = self.wl
        kk = wl.k if k is None else k
        g = wl.groups[gi % len(wl.groups)]
        return len(g.projs) * (2 * wl.T * g.d_in * g.d_out + 2 * wl.T * kk * wl.r * (g.d_in + g.d_out))

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
