"""Seeded synthetic inputs for the GQE forward pass (shared by the tests, the benchmark and
the smoke check).  This module holds none of the layer's arithmetic: it only draws random
numbers and rounds them to the storage precision.

Recipe (the pages' workload is a 250M-parameter LM prefilling FineWeb-Edu text; the corpus
and trained weights are not available, so seeded Gaussians of the same shapes stand in):

* generator ``numpy.random.default_rng(seed)`` (PCG64), ``standard_normal(dtype=float32)``;
* fixed draw order x, W_r, W_q, W_qs, W_k, W_v, W_o, W_oR, W_os -- every tensor is drawn
  every time, so the three output variants of one seed share identical weights;
* x ~ N(0, 1); projection weights ~ N(0, 0.02^2); router weights ~ N(0, router_std^2);
* an optional +bias on local expert 0 of each group;
* optional stress settings for peaked attention: a larger std of the query and key projections
  (``qk_std``) and a ramp that scales x up along the sequence (``x_ramp``);
* then round-to-nearest-even to bf16 for bf16 workloads (the router stays fp32).
"""
from __future__ import annotations

from dataclasses import dataclass, field, replace

import numpy as np


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 by round-to-nearest-even, returned as float32 holding the bf16 value."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return (u.astype(np.uint32) << 16).view(np.float32)


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-exact."""
    return (np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)


@dataclass(frozen=True)
class Workload:
    """One layer configuration plus the shape and seed of its synthetic input."""
    name: str
    dim: int
    num_query_experts: int
    num_kv_heads: int
    top_k: int
    head_dim: int | None
    batch: int
    seq: int
    dtype: str = "bf16"               # storage / compute type of x, weights, y
    variant: str = "gqe"
    shared_head: bool = True
    shared_kv_group: int = 0
    seed: int = 0
    router_std: float | None = None   # None -> 1/sqrt(dim) (logits ~ N(0, 1))
    router_bias_first: float = 0.0    # added to local expert 0 of every group
    dense_gqa: bool = False           # all-active GQA baseline on the same weights
    rope_base: float = 0.0            # rotary position embedding base (0: none, as on the pages)
    qk_std: float = 0.02              # std of the query and key projections (W_q, W_qs, W_k)
    x_ramp: float = 0.0               # x[b, s] scaled by 1 + x_ramp * s / (S - 1): growing norms

    @property
    def dh(self) -> int:
        return self.head_dim if self.head_dim else self.dim // self.num_query_experts

    @property
    def tokens(self) -> int:
        return self.batch * self.seq

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


# The five workloads of the measurement plan.  Names say what they are.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", 64, 4, 2, 1, 16, 1, 32, dtype="f32", seed=0,
                          router_std=0.02),
    "main_b8_s2048": Workload("main_b8_s2048", 768, 16, 8, 1, 48, 8, 2048, seed=0),
    "long_s16384": Workload("long_s16384", 768, 16, 8, 1, 48, 1, 16384, seed=0),
    "long_s32768": Workload("long_s32768", 768, 16, 8, 1, 48, 1, 32768, seed=0),
    "k2_skew_b4_s4096": Workload("k2_skew_b4_s4096", 1024, 16, 8, 2, 64, 4, 4096, seed=0,
                                 router_std=2.70 / np.sqrt(1024.0), router_bias_first=2.0),
    "ablation_gqe_b2_s8192": Workload("ablation_gqe_b2_s8192", 768, 16, 8, 1, 48, 2, 8192,
                                      seed=1, variant="gqe"),
    "ablation_weighted_b2_s8192": Workload("ablation_weighted_b2_s8192", 768, 16, 8, 1, 48, 2,
                                           8192, seed=1, variant="weighted_concat"),
    "ablation_hard_b2_s8192": Workload("ablation_hard_b2_s8192", 768, 16, 8, 1, 48, 2, 8192,
                                       seed=1, variant="hard_concat"),
}


def gqa_of(wl: Workload) -> Workload:
    """The all-active GQA baseline on the same draws: every expert is a head (k = N/G),
    plain concatenation, no shared head, no router."""
    return wl.with_(name=wl.name + "_gqa", top_k=wl.num_query_experts // wl.num_kv_heads,
                    variant="hard_concat", shared_head=False, dense_gqa=True)


def make_inputs(wl: Workload) -> dict:
    """Draw x and all weights for ``wl``.  Returns float32 arrays (bf16-exact when the
    workload is bf16) in the layouts of the C ABI:
    x [B, S, d]; w_router [d, N] fp32; b_router [N] fp32; w_q [N, d, dh]; w_q_shared [d, dh];
    w_k, w_v [d, G*dh]; w_o [N, dh, d]; w_o_rslot [G, dh, d]; w_o_shared [dh, d]."""
    d, N, G, dh = wl.dim, wl.num_query_experts, wl.num_kv_heads, wl.dh
    rng = np.random.default_rng(wl.seed)

    def draw(shape, std):
        return (rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std))

    rstd = wl.router_std if wl.router_std is not None else 1.0 / np.sqrt(d)
    out = {
        "x": draw((wl.batch, wl.seq, d), 1.0),
        "w_router": draw((d, N), rstd),
        "w_q": draw((N, d, dh), wl.qk_std),
        "w_q_shared": draw((d, dh), wl.qk_std),
        "w_k": draw((d, G * dh), wl.qk_std),
        "w_v": draw((d, G * dh), 0.02),
        "w_o": draw((N, dh, d), 0.02),
        "w_o_rslot": draw((G, dh, d), 0.02),
        "w_o_shared": draw((dh, d), 0.02),
    }
    if wl.x_ramp:
        ramp = 1.0 + wl.x_ramp * np.arange(wl.seq, dtype=np.float32) / np.float32(max(wl.seq - 1, 1))
        out["x"] = out["x"] * ramp.astype(np.float32)[None, :, None]
    b = np.zeros(N, np.float32)
    if wl.router_bias_first:
        b[:: N // G] = np.float32(wl.router_bias_first)
    out["b_router"] = b
    if wl.dtype == "bf16":
        for key in ("x", "w_q", "w_q_shared", "w_k", "w_v", "w_o", "w_o_rslot",
                    "w_o_shared"):
            out[key] = round_bf16(out[key])
    return out


# ----------------------------------------------------------------------------- top-k MoE-MLP
@dataclass(frozen=True)
class MoeWorkload:
    """A top-k MoE-MLP layer and its input: tokens x [T, dim] routed to top_k of num_experts
    two-layer expert MLPs of hidden width d_ff."""
    name: str
    dim: int
    num_experts: int
    top_k: int
    d_ff: int
    tokens: int
    activation: str = "gelu"
    seed: int = 0
    router_bias_first: float = 0.0    # > 0: bias added to expert 0's logit (skewed routing)
    router_std: float | None = None   # router weight std (default 1/sqrt(dim): logits ~ N(0, 1))
    router_bias: bool = False         # pass a (zero unless skewed) router bias to the layer

    def with_(self, **kw) -> "MoeWorkload":
        return replace(self, **kw)


# 2 of 8 experts active (the tutorial's example) at the main setting's width and token count, a
# skewed 16-expert layer, and a small ragged case.
MOE_WORKLOADS = {
    "moe_tiny": MoeWorkload("moe_tiny", 64, 4, 2, 128, 100),
    "moe_e8_k2_t16384": MoeWorkload("moe_e8_k2_t16384", 768, 8, 2, 3072, 16384),
    "moe_skew_e16_k2_t4096": MoeWorkload("moe_skew_e16_k2_t4096", 1024, 16, 2, 2048, 4096,
                                         router_std=2.70 / np.sqrt(1024.0), router_bias_first=2.0,
                                         router_bias=True),
}


def make_moe_inputs(wl: MoeWorkload) -> dict:
    """Draw x and the weights for ``wl`` (float32 arrays, x / w1 / w2 bf16-exact):
    x [T, d] ~ N(0, 1); w_router [d, E] ~ N(0, router_std^2); b_router [E] (None unless
    ``router_bias``); w1 [E, d, d_ff] ~ N(0, 1/d); w2 [E, d_ff, d] ~ N(0, 1/d_ff)."""
    d, E, dff = wl.dim, wl.num_experts, wl.d_ff
    rng = np.random.default_rng(wl.seed)

    def draw(shape, std):
        return rng.standard_normal(size=shape, dtype=np.float32) * np.float32(std)

    rstd = wl.router_std if wl.router_std is not None else 1.0 / np.sqrt(d)
    out = {"x": round_bf16(draw((wl.tokens, d), 1.0)), "w_router": draw((d, E), rstd),
           "w1": round_bf16(draw((E, d, dff), 1.0 / np.sqrt(d))),
           "w2": round_bf16(draw((E, dff, d), 1.0 / np.sqrt(dff)))}
    b = None
    if wl.router_bias:
        b = np.zeros(E, np.float32)
        b[0] = np.float32(wl.router_bias_first)
    out["b_router"] = b
    return out
