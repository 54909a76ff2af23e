"""MoELayer: holds the device buffers of one layer and issues the C-ABI calls
in order (route + permute as one moe_route_plan call -> grouped_ffn ->
combine).  Torch provides the device memory and the stream; nothing here
computes."""
from __future__ import annotations

import numpy as np

from . import (MOE_BLOB_ROUTED, MOE_BLOB_SHARED, MOE_F32, moe_blob_bytes, moe_combine,
               moe_grouped_ffn, moe_pack_experts, moe_permute, moe_route, moe_route_plan,
               moe_workspace_bytes)


def pack_blob(desc, kind, gate, gate_s, up, up_s, down, down_s) -> np.ndarray:
    """Canonical host weights -> host blob (numpy uint8) via moe_pack_experts."""
    blob = np.empty(moe_blob_bytes(desc, kind), np.uint8)
    c = lambda a: None if a is None else np.ascontiguousarray(a)
    return moe_pack_experts(desc, kind, c(gate), c(gate_s), c(up), c(up_s), c(down), c(down_s),
                            blob)


class MoELayer:
    def __init__(self, desc, k: int, T_max: int, device="cuda"):
        import torch
        self.torch = torch
        self.desc, self.k, self.T_max, self.device = desc, k, T_max, device
        d, E = desc.d, desc.n_experts
        n = T_max * k
        f32, i32 = torch.float32, torch.int32
        act = torch.float32 if desc.act == MOE_F32 else torch.bfloat16
        z = lambda shape, dt: torch.empty(shape, dtype=dt, device=device)
        self.logits = z((max(T_max, 1), E), f32)
        self.ids = z((max(n, 1),), i32)
        self.w = z((max(n, 1),), f32)
        self.offsets = z((E + 1,), i32)
        self.perm = z((max(n, 1),), i32)
        self.inv_perm = z((max(n, 1),), i32)
        self.out_assign = z((max(n, 1), d), f32)
        self.shared_out = z((max(T_max, 1), d), f32) if desc.n_shared else None
        self.y = z((max(T_max, 1), d), act)
        self.ws_bytes = moe_workspace_bytes(desc, T_max, k)
        # zeroed once: its first 16 bytes are moe_route_plan's block counters
        self.workspace = torch.zeros((self.ws_bytes,), dtype=torch.uint8, device=device)
        self.router_w = self.bias = self.routed_blob = self.shared_blob = None

    def set_weights(self, router_w, routed_blob, shared_blob=None, bias=None):
        """Device tensors (router weights [E, d] act dtype, blobs uint8)."""
        self.router_w, self.routed_blob, self.shared_blob, self.bias = (
            router_w, routed_blob, shared_blob, bias)

    def route(self, x, T):
        moe_route(self.desc, T, self.k, x, self.router_w, self.bias, self.logits, self.ids,
                  self.w)

    def permute(self, x, T):
        moe_permute(self.desc, T, self.k, x, self.ids, self.offsets, self.perm, self.inv_perm,
                    self.workspace, self.ws_bytes)

    def route_plan(self, x, T):
        """route and permute as one call (one launch when T <= 32, bf16)."""
        moe_route_plan(self.desc, T, self.k, x, self.router_w, self.bias, self.logits, self.ids,
                       self.w, self.offsets, self.perm, self.inv_perm, self.workspace,
                       self.ws_bytes)

    def grouped_ffn(self, x, T):
        moe_grouped_ffn(self.desc, T, self.k, x, self.w, self.offsets, self.perm,
                        self.routed_blob, self.shared_blob, self.out_assign, self.shared_out,
                        self.workspace, self.ws_bytes)

    def combine(self, T):
        moe_combine(self.desc, T, self.k, self.out_assign, self.inv_perm, self.shared_out, self.y)

    def forward(self, x, T=None):
        """x: device tensor [T, d] (act dtype).  Returns a view of y [T, d]."""
        T = x.shape[0] if T is None else T
        assert T <= self.T_max
        self.route_plan(x, T)
        self.grouped_ffn(x, T)
        self.combine(T)
        return self.y[:T]

    def capture(self, x, T=None):
        """Record the layer's calls on x (a static device buffer) into one HIP
        graph; replaying it reruns the layer on whatever x then holds, with the
        weights bound at capture time.  Returns the torch graph object."""
        import torch
        T = x.shape[0] if T is None else T
        self.forward(x, T)  # warm: first launches of each kernel happen outside capture
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            self.forward(x, T)
        return g


def blobs_from_inputs(desc, inputs: dict):
    """Pack the routed (and shared) expert blobs of a workloads.generate() dict."""
    routed = pack_blob(desc, MOE_BLOB_ROUTED, inputs["wg"], inputs.get("wg_s"), inputs["wu"],
                       inputs.get("wu_s"), inputs["wd"], inputs.get("wd_s"))
    shared = None
    if desc.n_shared:
        shared = pack_blob(desc, MOE_BLOB_SHARED, inputs["sg"], inputs.get("sg_s"), inputs["su"],
                           inputs.get("su_s"), inputs["sd"], inputs.get("sd_s"))
    return routed, shared
