"""Builds a GQE layer on the GPU from a synthetic workload and runs it (no reference code here:
the comparison with the CPU oracle lives in the tests)."""
from __future__ import annotations

import numpy as np
import torch

from .gqe import GQEAttention, TORCH_DTYPES, upload_weights
from .inputs import Workload, make_inputs


def build_layer(wl: Workload, inputs: dict | None = None, device: str = "cuda:0"):
    """Returns (layer, x on the device, host inputs)."""
    inputs = make_inputs(wl) if inputs is None else inputs
    w = upload_weights(inputs, device, wl.dtype)
    if wl.dense_gqa:
        w["w_router"] = None
        w["b_router"] = None
    if not wl.shared_head:
        w["w_q_shared"] = None
        w["w_o_shared"] = None
    if wl.variant != "gqe" or wl.dense_gqa:
        w["w_o_rslot"] = None
    layer = GQEAttention(wl.dim, wl.num_query_experts, wl.num_kv_heads, wl.top_k, wl.head_dim,
                         wl.variant, wl.shared_head, wl.shared_kv_group, wl.dtype, wl.dense_gqa,
                         weights=w, rope_base=wl.rope_base)
    x = torch.from_numpy(np.ascontiguousarray(inputs["x"])).to(device=device,
                                                               dtype=TORCH_DTYPES[wl.dtype])
    return layer, x, inputs


def run_layer(layer: GQEAttention, x: torch.Tensor, routing: bool = True) -> dict:
    """One forward; returns host copies of y (float64), routing and the balance statistics."""
    B, S, _ = x.shape
    ridx = rw = None
    if routing and not layer.cfg.dense_gqa:
        ridx = torch.full((B, S, layer.G, layer.k), -1, dtype=torch.int32, device=x.device)
        rw = torch.full((B, S, layer.G, layer.k), -1.0, dtype=torch.float32, device=x.device)
    y = layer(x, route_idx=ridx, route_w=rw)
    torch.cuda.synchronize()
    out = dict(y=y.float().cpu().numpy().astype(np.float64).reshape(B * S, -1))
    if ridx is not None:
        out["idx"] = ridx.cpu().numpy().reshape(B * S, layer.G, layer.k)
        out["w"] = rw.cpu().numpy().reshape(B * S, layer.G, layer.k)
    out.update(layer.aux_stats())
    return out


def build_moe(wl, inputs: dict | None = None, device: str = "cuda:0"):
    """MoE-MLP layer of a MoeWorkload: returns (layer, x on the device, host inputs)."""
    from .gqe import MoEMLP
    from .inputs import make_moe_inputs
    inputs = make_moe_inputs(wl) if inputs is None else inputs

    def dev(a, dt):
        return None if a is None else torch.from_numpy(np.ascontiguousarray(a)).to(device=device, dtype=dt)

    w = dict(w_router=dev(inputs["w_router"], torch.float32), b_router=dev(inputs["b_router"], torch.float32),
             w1=dev(inputs["w1"], torch.bfloat16), w2=dev(inputs["w2"], torch.bfloat16))
    layer = MoEMLP(wl.dim, wl.num_experts, wl.top_k, wl.d_ff, wl.activation, weights=w)
    x = dev(inputs["x"], torch.bfloat16)
    return layer, x, inputs
