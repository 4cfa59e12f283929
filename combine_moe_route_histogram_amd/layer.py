"""Buffers and call sequences of one MoE layer step over the C ABI.

torch is used only to allocate device memory; every computation is one of the
library's entry points, called in the order of the layer (UniEP article,
section 1.1 and Figure 1): route -> dispatch -> expert FFN -> combine, then the
mirror image for the backward.
"""
from __future__ import annotations

import torch

from . import (BF16, F32, Dims, moe_combine, moe_combine_bwd, moe_dispatch, moe_dispatch_bwd,
               moe_dispatch_ffn, moe_expert_ffn_bwd, moe_expert_ffn_bwd_data, moe_expert_ffn_bwd_weight,
               moe_expert_ffn_down, moe_expert_ffn_up, moe_ffn_combine, moe_route, moe_route_bwd,
               moe_sync_status, moe_workspace_bytes)


def make_dims(T, H, E, K, I, n_shared=0, dtype="bf16", I_shared=None) -> Dims:
    return Dims(T=T, H=H, E=E, K=K, I=I, n_shared=n_shared, I_shared=I_shared,
                dtype=BF16 if dtype == "bf16" else F32)


class Buffers:
    """Every intermediate and output of one forward + backward step."""

    def __init__(self, d: Dims, device="cuda", backward=True):
        dt, T, H, E, K, I, Ns = d.torch_dtype, d.T, d.H, d.E, d.K, d.I, d.n_shared
        R, RA = d.R, d.RA
        z = lambda *s, dtype=dt: torch.empty(*s, dtype=dtype, device=device)
        i32, f32 = torch.int32, torch.float32
        self.d = d
        self.ws = z(max(moe_workspace_bytes(d), 256), dtype=torch.uint8)
        self.topk_idx = z(T, K, dtype=i32)
        self.topk_w = z(T, K, dtype=f32)
        self.counts = z(E, dtype=i32)
        self.offsets = z(E + 1, dtype=i32)
        self.slot = z(T, K, dtype=i32)
        self.slot_src = z(R, dtype=i32)
        self.x_perm = z(R, H)
        self.ab = z(RA, 2 * I)
        self.h = z(RA, I)
        self.y = z(RA, H)
        self.out = z(T, H)
        if backward:
            self.dy = z(R, H)
            self.dtopk_w = z(T, K, dtype=f32)
            self.dab = z(RA, 2 * I)
            self.dx_rows = z(RA, H)
            self.dx = z(T, H)
            self.dlogits = z(T, E, dtype=f32)
            self.dw1 = z(E, H, I, dtype=f32)
            self.dw3 = z(E, H, I, dtype=f32)
            self.dw2 = z(E, I, H, dtype=f32)
            self.dws1 = z(Ns, H, I, dtype=f32) if Ns else None
            self.dws3 = z(Ns, H, I, dtype=f32) if Ns else None
            self.dws2 = z(Ns, I, H, dtype=f32) if Ns else None


def route(b: Buffers, p: dict, stream=None):
    moe_route(b.d, p["logits"], b.topk_idx, b.topk_w, b.counts, b.offsets, b.slot, b.slot_src,
              b.ws, stream)


def forward(b: Buffers, p: dict, fused: bool = False, stream=None):
    """route -> dispatch -> expert FFN -> combine.  p holds the device inputs."""
    d = b.d
    route(b, p, stream)
    if fused:
        moe_dispatch_ffn(d, p["x"], b.slot_src, b.slot, b.offsets, p["w1"], p["w3"], p.get("ws1"),
                         p.get("ws3"), b.x_perm, b.ab, b.h, b.ws, stream)
        moe_ffn_combine(d, b.h, b.offsets, p["w2"], p.get("ws2"), b.slot, b.topk_w, b.y, b.out,
                        b.ws, stream)
    else:
        moe_dispatch(d, p["x"], b.slot, b.x_perm, stream)
        moe_expert_ffn_up(d, b.x_perm, p["x"], b.offsets, p["w1"], p["w3"], p.get("ws1"),
                          p.get("ws3"), b.ab, b.h, b.ws, stream)
        moe_expert_ffn_down(d, b.h, b.offsets, p["w2"], p.get("ws2"), b.y, b.ws, stream)
        moe_combine(d, b.y, b.slot, b.topk_w, b.out, stream)


def backward(b: Buffers, p: dict, fused: bool = False, stream=None):
    """combine_bwd -> FFN input grads (B) -> FFN weight grads (W) -> dispatch_bwd -> route_bwd.
    fused: B and W in one launch, W filling the gaps of B (moe_expert_ffn_bwd)."""
    d = b.d
    moe_combine_bwd(d, p["dout"], b.y, b.slot, b.topk_w, b.dy, b.dtopk_w, stream)
    if fused:
        moe_expert_ffn_bwd(d, b.dy, p.get("dout"), b.offsets, p["w1"], p["w3"], p["w2"],
                           p.get("ws1"), p.get("ws3"), p.get("ws2"), b.ab, b.x_perm, p["x"], b.h,
                           b.dab, b.dx_rows, b.dw1, b.dw3, b.dw2, b.dws1, b.dws3, b.dws2, b.ws,
                           stream)
    else:
        moe_expert_ffn_bwd_data(d, b.dy, p.get("dout"), b.offsets, p["w1"], p["w3"], p["w2"],
                                p.get("ws1"), p.get("ws3"), p.get("ws2"), b.ab, b.dab, b.dx_rows,
                                b.ws, stream)
        moe_expert_ffn_bwd_weight(d, b.x_perm, p["x"], b.h, b.dy, p.get("dout"), b.dab, b.offsets,
                                  b.dw1, b.dw3, b.dw2, b.dws1, b.dws3, b.dws2, b.ws, stream)
    moe_dispatch_bwd(d, b.dx_rows, b.slot, b.dx, stream)
    moe_route_bwd(d, b.dtopk_w, b.topk_w, b.topk_idx, b.dlogits, stream)


def check(stream=None):
    """Wait for the step's work and raise MoeError (MOE_ETIMEOUT) if a bounded
    wait inside a persistent kernel gave up, which leaves invalid results."""
    moe_sync_status(stream)
