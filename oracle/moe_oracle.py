"""Top-k mixture-of-experts MLP -- CPU oracle.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg
of ``bench.py`` may import this module.  Plain NumPy in float64; no code is shared with the HIP
library.

What it computes (cseroadmap tutorial "Grouped-query attention and mixture of experts", section
"Mixture of experts (MoE)": the ``moe_layer`` sketch and the consequences listed under it):

  1. router probabilities  p[t] = softmax_e(x[t] W_r + b_r)            (softmax over all E experts)
  2. selection             the top_k experts of largest probability, best first
  3. mixing weights        w[t, r] = p[t, e_r] / sum_r' p[t, e_r']     (renormalised over the chosen)
  4. output                y[t] = sum_r w[t, r] f_{e_r}(x[t])

Readings where the page is silent (each listed in the design notes):
  * an expert is a two-layer MLP without biases, f_e(x) = act(x W1[e]) W2[e], W1 [E, d, d_ff],
    W2 [E, d_ff, d]; act is GELU in its exact form 0.5 h (1 + erf(h / sqrt 2)) or ReLU;
  * the sketch's router has no bias; an optional b_r is accepted (it only shifts logits) so that
    skewed routing can be set up; the logits are formed in float64;
  * ranking uses the logits (the softmax is monotone); equal logits go to the lower expert index;
  * ``hidden="bf16"`` rounds the hidden activation to bf16 (round to nearest even) before the second
    product -- the precision in which a bf16 layer stores it; ``hidden=None`` keeps it exact;
  * load statistics as for the attention router: share_e = count_e / (T top_k), the mean
    probability P_e, and the Switch-style balance loss E sum_e share_e P_e.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erf

ACTIVATIONS = ("gelu", "relu")


def round_bf16(a: np.ndarray) -> np.ndarray:
    """float64 -> float32 -> bf16 (round to nearest, ties to even) -> float64."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def act(h: np.ndarray, kind: str) -> np.ndarray:
    """The expert's elementwise activation."""
    if kind == "gelu":
        return 0.5 * h * (1.0 + erf(h / np.sqrt(2.0)))
    if kind == "relu":
        return np.maximum(h, 0.0)
    raise ValueError(kind)


def router(x, w_router, top_k: int, b_router=None) -> dict:
    """Steps 1-3: logits, probabilities, the top_k choices (best first) and their weights."""
    x = np.asarray(x, dtype=np.float64)
    logits = x @ np.asarray(w_router, dtype=np.float64)
    if b_router is not None:
        logits = logits + np.asarray(b_router, dtype=np.float64)[None, :]
    T, E = logits.shape
    z = np.exp(logits - logits.max(axis=1, keepdims=True))
    p = z / z.sum(axis=1, keepdims=True)
    # descending logit, ties to the lower index: a stable sort of the negated logits
    order = np.argsort(-logits, axis=1, kind="stable")
    idx = order[:, :top_k].astype(np.int32)
    psel = np.take_along_axis(p, idx, axis=1)
    w = psel / psel.sum(axis=1, keepdims=True)
    srt = np.take_along_axis(logits, order, axis=1)
    gap = srt[:, top_k - 1] - srt[:, top_k] if top_k < E else np.full(T, np.inf)
    return dict(logits=logits, p=p, idx=idx, w=w, gap=gap)


def weights_for(p, idx) -> np.ndarray:
    """Renormalised weights of given choices (used when a near tie was decided the other way)."""
    psel = np.take_along_axis(p, np.asarray(idx, dtype=np.int64), axis=1)
    return psel / psel.sum(axis=1, keepdims=True)


def forward(x, w: dict, top_k: int, activation: str = "gelu", idx=None, hidden=None) -> dict:
    """Step 4 for every token: y [T, d], plus the routing and the hidden activations of each
    (token, rank) pair, h [T, top_k, d_ff]."""
    x = np.asarray(x, dtype=np.float64)
    r = router(x, w["w_router"], top_k, w.get("b_router"))
    if idx is None:
        idx = r["idx"]
        mix = r["w"]
    else:
        idx = np.asarray(idx, dtype=np.int32)
        mix = weights_for(r["p"], idx)
    W1 = np.asarray(w["w1"], dtype=np.float64)
    W2 = np.asarray(w["w2"], dtype=np.float64)
    T, d = x.shape
    E, _, dff = W1.shape
    y = np.zeros((T, W2.shape[2]))
    h_all = np.zeros((T, top_k, dff))
    for e in range(E):
        tok, rank = np.nonzero(idx == e)
        if tok.size == 0:
            continue
        h = act(x[tok] @ W1[e], activation)
        if hidden == "bf16":
            h = round_bf16(h)
        h_all[tok, rank] = h
        y[tok] += mix[tok, rank][:, None] * (h @ W2[e])
    return dict(y=y, h=h_all, idx=idx, w=mix, p=r["p"], logits=r["logits"], gap=r["gap"])


def stats(p, idx, num_experts: int) -> dict:
    """Per-expert token counts and shares, mean router probabilities, the balance loss."""
    idx = np.asarray(idx)
    T, k = idx.shape
    counts = np.bincount(idx.ravel(), minlength=num_experts).astype(np.int64)
    share = counts / float(T * k)
    mean_p = np.asarray(p, dtype=np.float64).mean(axis=0)
    return dict(counts=counts, share=share, mean_p=mean_p, aux=float(num_experts * np.sum(share * mean_p)))
