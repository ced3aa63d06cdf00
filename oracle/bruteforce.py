"""Whole-layer NumPy float64 brute force of the GQE forward pass, for tiny shapes only.

TEST INFRASTRUCTURE ONLY (see gqe_oracle.py).  Written independently of gqe_oracle.c: it
materialises full matrices (all N expert queries, the full masked score matrix per head, the
dense one-hot expansion of the output concatenation) instead of looping per token, so a
slip in either implementation shows up as a disagreement between the two.

Follows the README "Algorithm Overview" (in-group softmax, then top-k; shared head; dense KV),
"Parameters"/"Ablations" (variants), the explainer's "Output Construction", and the tutorial's
moe_layer sketch (softmax of x @ router_w, argsort for the top_k, renormalised mix).
"""
from __future__ import annotations

import numpy as np


def layer(cfg, B, S, x, w):
    d, N, G, k, dh = cfg.dim, cfg.num_query_experts, cfg.num_kv_heads, cfg.top_k, cfg.dh
    n = N // G
    T = B * S
    x = np.asarray(x, np.float64).reshape(T, d)
    Wr = np.asarray(w["w_router"], np.float64)
    br = np.zeros(N) if w.get("b_router") is None else np.asarray(w["b_router"], np.float64)
    logits = x @ Wr + br                                    # [T, N]
    lg = logits.reshape(T, G, n)
    ex = np.exp(lg - lg.max(axis=2, keepdims=True))
    p = (ex / ex.sum(axis=2, keepdims=True))                # [T, G, n]
    order = np.argsort(-lg, axis=2, kind="stable")          # ties -> lower index first
    sel = order[:, :, :k]                                   # [T, G, k] local ids
    psel = np.take_along_axis(p, sel, axis=2)
    wts = psel / psel.sum(axis=2, keepdims=True)
    idx = sel + (np.arange(G) * n)[None, :, None]

    Wq = np.asarray(w["w_q"], np.float64)                   # [N, d, dh]
    q_all = np.einsum("td,edh->teh", x, Wq)                 # every expert, then select
    Wk = np.asarray(w["w_k"], np.float64).reshape(d, G, dh)
    Wv = np.asarray(w["w_v"], np.float64).reshape(d, G, dh)
    Kx = np.einsum("td,dgh->tgh", x, Wk).reshape(B, S, G, dh)
    base = float(getattr(cfg, "rope_base", 0.0) or 0.0)
    if base > 0:
        # rotary position embedding as complex multiplication: the pair (v[2i], v[2i+1]) is the
        # complex number v[2i] + i v[2i+1], multiplied by exp(i m base^(-2i/dh))
        pos = getattr(cfg, "pos0", 0) + np.arange(S)
        rot = np.exp(1j * pos[:, None] * base ** (-np.arange(0, dh, 2) / dh))   # [S, dh/2]

        def rope(v):  # v [B, S, heads, dh]
            z = (v[..., 0::2] + 1j * v[..., 1::2]) * rot[None, :, None, :]
            out = np.empty_like(v)
            out[..., 0::2], out[..., 1::2] = z.real, z.imag
            return out
        Kx = rope(Kx)
        q_all = rope(q_all.reshape(B, S, N, dh)).reshape(T, N, dh)
    Vx = np.einsum("td,dgh->tgh", x, Wv).reshape(B, S, G, dh)
    mask = np.tril(np.ones((S, S), bool))

    def attn(qh, g):
        """qh [B, S, dh] queries attending to group g; returns [B, S, dh]."""
        sc = np.einsum("bsh,bth->bst", qh, Kx[:, :, g, :]) / np.sqrt(dh)
        sc = np.where(mask[None], sc, -np.inf)
        a = np.exp(sc - sc.max(axis=2, keepdims=True))
        a = a / a.sum(axis=2, keepdims=True)
        return np.einsum("bst,bth->bsh", a, Vx[:, :, g, :])

    # attention output of every expert head (all N), then pick by the routing
    o_all = np.zeros((T, N, dh))
    for e in range(N):
        o_all[:, e, :] = attn(q_all[:, e, :].reshape(B, S, dh), e // n).reshape(T, dh)

    Wo = np.asarray(w["w_o"], np.float64)                   # [N, dh, d]
    # dense one-hot coefficient matrix over all N expert slots
    coef = np.zeros((T, N))
    pf = p.reshape(T, N)
    for g in range(G):
        for r in range(k):
            e = idx[:, g, r]
            if cfg.variant == "weighted_concat":
                coef[np.arange(T), e] = pf[np.arange(T), e]
            else:
                coef[np.arange(T), e] = 1.0
    y = np.einsum("te,teh,ehd->td", coef, o_all, Wo)
    if cfg.variant == "gqe":
        WoR = np.asarray(w["w_o_rslot"], np.float64)        # [G, dh, d]
        for g in range(G):
            slot = np.zeros((T, dh))
            for r in range(k):
                slot += wts[:, g, r:r + 1] * o_all[np.arange(T), idx[:, g, r], :]
            y += slot @ WoR[g]
    q_s = o_s = None
    if cfg.shared_head:
        q_s = x @ np.asarray(w["w_q_shared"], np.float64)
        if base > 0:
            q_s = rope(q_s.reshape(B, S, 1, dh)).reshape(T, dh)
        o_s = attn(q_s.reshape(B, S, dh), cfg.shared_kv_group).reshape(T, dh)
        y += o_s @ np.asarray(w["w_o_shared"], np.float64)
    return dict(y=y, logits=logits, p=pf, idx=idx.astype(np.int32), w=wts, o_all=o_all,
                K=Kx.reshape(T, G, dh), V=Vx.reshape(T, G, dh), o_s=o_s)
