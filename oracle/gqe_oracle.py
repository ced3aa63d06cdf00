"""Grouped Query Experts (GQE) forward pass -- CPU oracle (Python side).

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this module.  It loads ``liboracle.so`` built from
``gqe_oracle.c`` (plain loops, fp64 accumulation) and shares no code with the HIP library.

The method (web pages on GQE):
  * "GQE: Grouped Query Experts" README, "Algorithm Overview" / "Parameters" / "Ablations";
  * gist.science explainer, "Technical Summary" -> "Architecture and Routing";
  * cseroadmap tutorial "Grouped-query attention and mixture of experts", "Mixture of experts".

Every array handed to the C code is float64 (inputs that the GPU reads as bf16 are first
rounded to bf16 by the input generator and then widened exactly).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqe_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

VARIANTS = {"gqe": 0, "weighted_concat": 1, "hard_concat": 2}


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (OpenMP over independent tokens)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


class _Cfg(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "dim", "num_query_experts", "num_kv_heads", "top_k", "head_dim", "variant",
        "shared_head", "shared_kv_group", "pos0", "pad_")] + [("rope_base", ctypes.c_double)]


@dataclass(frozen=True)
class OracleConfig:
    dim: int
    num_query_experts: int = 16
    num_kv_heads: int = 8
    top_k: int = 1
    head_dim: int | None = None   # None -> dim // num_query_experts ("Parameters")
    variant: str = "gqe"
    shared_head: bool = True
    shared_kv_group: int = 0
    rope_base: float = 0.0        # rotary position embedding base (RoFormer); 0 = none
    pos0: int = 0                 # position of the first token of every sequence

    @property
    def dh(self) -> int:
        return self.head_dim if self.head_dim else self.dim // self.num_query_experts

    @property
    def n(self) -> int:
        return self.num_query_experts // self.num_kv_heads

    @property
    def h_act(self) -> int:
        return self.num_kv_heads * self.top_k + (1 if self.shared_head else 0)

    def c(self) -> _Cfg:
        return _Cfg(self.dim, self.num_query_experts, self.num_kv_heads, self.top_k, self.dh,
                    VARIANTS[self.variant], int(self.shared_head), self.shared_kv_group, self.pos0, 0,
                    float(self.rope_base))


_lib = None


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        C = ctypes.POINTER(_Cfg)
        lib.gqe_oracle_router.argtypes = [C, I64, P, P, P, P, P, P, P, P]
        lib.gqe_oracle_aux.argtypes = [C, I64, P, P, P, P, P, P]
        lib.gqe_oracle_kv.argtypes = [C, I64, I64, P, P, P, P, P]
        lib.gqe_oracle_bucket.argtypes = [C, I64, P, P, P, P]
        lib.gqe_oracle_rows.argtypes = [C, I64, I64, P, P, P, P, P, P, P, P, P, P, P, I64, P,
                                        P, P]
        lib.gqe_oracle_backward.argtypes = [C, I64, I64] + [P] * 12 + [ctypes.c_double] + [P] * 10
        for f in (lib.gqe_oracle_router, lib.gqe_oracle_aux, lib.gqe_oracle_kv,
                  lib.gqe_oracle_rows, lib.gqe_oracle_bucket, lib.gqe_oracle_backward):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def router(cfg: OracleConfig, x, w_router, b_router=None) -> dict:
    """Logits, in-group softmax p, top-k idx (global expert ids), renormalised w, gap."""
    lib = _load()
    x = _f64(x).reshape(-1, cfg.dim)
    T = x.shape[0]
    N, G, k = cfg.num_query_experts, cfg.num_kv_heads, cfg.top_k
    Wr = _f64(w_router)
    br = None if b_router is None else _f64(b_router)
    out = dict(logits=np.zeros((T, N)), p=np.zeros((T, N)),
               idx=np.zeros((T, G, k), np.int32), w=np.zeros((T, G, k)),
               gap=np.zeros((T, G)))
    cc = cfg.c()
    rc = lib.gqe_oracle_router(ctypes.byref(cc), T, _ptr(x), _ptr(Wr), _ptr(br),
                               _ptr(out["logits"]), _ptr(out["p"]), _ptr(out["idx"]),
                               _ptr(out["w"]), _ptr(out["gap"]))
    if rc != 0:
        raise ValueError("oracle router: invalid configuration")
    return out


def bucket(cfg: OracleConfig, idx) -> dict:
    """Stable bucketing of the (t, g, r) assignments by expert: offs [N+1], perm [T*G*k]
    (token ids), inv [T, G, k] (position of each assignment in perm)."""
    lib = _load()
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    N, G, k = cfg.num_query_experts, cfg.num_kv_heads, cfg.top_k
    T = idx.size // (G * k)
    offs = np.zeros(N + 1, np.int64)
    perm = np.zeros(T * G * k, np.int64)
    inv = np.zeros((T, G, k), np.int64)
    cc = cfg.c()
    if lib.gqe_oracle_bucket(ctypes.byref(cc), T, _ptr(idx), _ptr(offs), _ptr(perm), _ptr(inv)) != 0:
        raise MemoryError("oracle bucket")
    return dict(offs=offs, perm=perm, inv=inv)


def aux(cfg: OracleConfig, p, idx) -> dict:
    """Per-expert counts, mean probability, Switch-style aux loss (unscaled), head count."""
    lib = _load()
    p = _f64(p)
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    T = p.shape[0]
    N = cfg.num_query_experts
    counts = np.zeros(N, np.int64)
    mean_prob = np.zeros(N)
    a = np.zeros(1)
    heads = np.zeros(1, np.int32)
    cc = cfg.c()
    lib.gqe_oracle_aux(ctypes.byref(cc), T, _ptr(p), _ptr(idx), _ptr(counts), _ptr(mean_prob),
                       _ptr(a), _ptr(heads))
    return dict(counts=counts, mean_prob=mean_prob, aux=float(a[0]),
                active_heads=int(heads[0]))


def kv(cfg: OracleConfig, x, w_k, w_v, S: int | None = None):
    """Dense K and V for every token: [T, G, dh] each (sequences of S tokens; S = T when None:
    the positions matter only with the rotary embedding)."""
    lib = _load()
    x = _f64(x).reshape(-1, cfg.dim)
    T = x.shape[0]
    G, dh = cfg.num_kv_heads, cfg.dh
    K = np.zeros((T, G, dh))
    V = np.zeros((T, G, dh))
    cc = cfg.c()
    lib.gqe_oracle_kv(ctypes.byref(cc), T, T if S is None else S, _ptr(x), _ptr(_f64(w_k)),
                      _ptr(_f64(w_v)), _ptr(K), _ptr(V))
    return K, V


def rows(cfg: OracleConfig, B: int, S: int, x, p, idx, w, K, V, rows_list, want_qo=False):
    """Layer output y [len(rows), d] for the given global token ids (b*S + s)."""
    lib = _load()
    x = _f64(x).reshape(-1, cfg.dim)
    rws = np.ascontiguousarray(rows_list, dtype=np.int64)
    nr = rws.shape[0]
    y = np.zeros((nr, cfg.dim))
    q = np.zeros((nr, cfg.h_act, cfg.dh)) if want_qo else None
    o = np.zeros((nr, cfg.h_act, cfg.dh)) if want_qo else None
    wq, wqs, wo, wor, wos = (_f64(w[k]) for k in ("w_q", "w_q_shared", "w_o", "w_o_rslot",
                                                  "w_o_shared"))
    cc = cfg.c()
    rc = lib.gqe_oracle_rows(ctypes.byref(cc), B, S, _ptr(x), _ptr(_f64(p)),
                             _ptr(np.ascontiguousarray(idx, np.int32)), _ptr(wq), _ptr(wqs),
                             _ptr(_f64(K)), _ptr(_f64(V)), _ptr(wo), _ptr(wor), _ptr(wos),
                             _ptr(rws), nr, _ptr(y), _ptr(q), _ptr(o))
    if rc != 0:
        raise ValueError("oracle rows: invalid configuration")
    return (y, q, o) if want_qo else y


def forward(cfg: OracleConfig, B: int, S: int, x, w: dict, rows_list=None, want_qo=False,
            idx_override=None) -> dict:
    """The whole layer: routing, aux statistics, dense K/V, and y for ``rows_list``
    (all tokens when None).  ``idx_override`` (same shape as idx) replaces the oracle's
    selection for chosen tokens -- used only where the logit gap is below the near-tie
    bound, where either choice is correct."""
    x = _f64(x).reshape(B * S, cfg.dim)
    r = router(cfg, x, w["w_router"], w.get("b_router"))
    idx = r["idx"] if idx_override is None else np.ascontiguousarray(idx_override, np.int32)
    st = aux(cfg, r["p"], idx)
    K, V = kv(cfg, x, w["w_k"], w["w_v"], S)
    if rows_list is None:
        rows_list = np.arange(B * S)
    res = rows(cfg, B, S, x, r["p"], idx, w, K, V, rows_list, want_qo=want_qo)
    out = dict(r)
    out.update(st)
    out["idx_used"] = idx
    out["K"], out["V"] = K, V
    if want_qo:
        out["y"], out["q"], out["o"] = res
    else:
        out["y"] = res
    out["rows"] = np.asarray(rows_list)
    return out


def decode(cfg: OracleConfig, x_hist, w: dict, pos, idx_new=None) -> dict:
    """One decode step with a dense KV cache (README "Algorithm Overview": the KV heads stay dense
    and unchanged, so GQA's KV cache is kept; explainer "Architecture and Routing", "Dense KV
    Path").  The new token of sequence b sits at position pos[b] after the cached positions
    0 .. pos[b]-1 of x_hist[b]; the cache holds exactly their keys and values, so the token's
    output is row pos[b] of the causal forward pass over x_hist[b, :pos[b]+1].  That is how it is
    computed here (no cache of its own: the definition, written out).

    x_hist [B, >= max(pos)+1, d]; idx_new optional [B, G, k] routing of the new tokens that replaces
    the oracle's (only where a decision is near-tied).  Returns y [B, d] and the new tokens'
    logits, p, idx, w, gap."""
    x_hist = np.asarray(x_hist)
    B = x_hist.shape[0]
    G, k = cfg.num_kv_heads, cfg.top_k
    out = dict(y=np.zeros((B, cfg.dim)), logits=np.zeros((B, cfg.num_query_experts)),
               p=np.zeros((B, cfg.num_query_experts)), idx=np.zeros((B, G, k), np.int32),
               w=np.zeros((B, G, k)), gap=np.zeros((B, G)))
    for b, p in enumerate(int(v) for v in pos):
        xs = _f64(x_hist[b, :p + 1]).reshape(p + 1, cfg.dim)
        override = None
        if idx_new is not None:
            override = router(cfg, xs, w["w_router"], w.get("b_router"))["idx"]
            override[p] = np.asarray(idx_new)[b]
        r = forward(cfg, 1, p + 1, xs, w, rows_list=[p], idx_override=override)
        out["y"][b] = r["y"][0]
        for key in ("logits", "p", "idx", "w", "gap"):
            out[key][b] = r[key][p]
    return out


GRAD_KEYS = ("x", "w_router", "b_router", "w_q", "w_q_shared", "w_k", "w_v", "w_o", "w_o_rslot", "w_o_shared")


def backward(cfg: OracleConfig, B: int, S: int, x, w: dict, dy, aux_coef: float = 0.0, idx=None) -> dict:
    """Gradients of L = sum(dy * y) + aux_coef * aux with respect to x and every weight (the
    training half of the method: README "Usage" trains with lm_loss + 0.01 * aux; the explainer's
    "Output Construction" notes that the renormalised slot is the loss's differentiable path to the
    router).  The routing ``idx`` [T, G, k] is held fixed (the oracle's own when None).
    Returns a dict keyed like the weights, plus "x"."""
    lib = _load()
    T = B * S
    d, N, G, k, dh = cfg.dim, cfg.num_query_experts, cfg.num_kv_heads, cfg.top_k, cfg.dh
    x = _f64(x).reshape(T, d)
    if idx is None:
        idx = router(cfg, x, w["w_router"], w.get("b_router"))["idx"]
    idx = np.ascontiguousarray(idx, dtype=np.int32)
    br = np.zeros(N) if w.get("b_router") is None else _f64(w["b_router"])
    ins = [x, _f64(w["w_router"]), br, _f64(w["w_q"]), _f64(w["w_q_shared"]), _f64(w["w_k"]),
           _f64(w["w_v"]), _f64(w["w_o"]), _f64(w["w_o_rslot"]), _f64(w["w_o_shared"])]
    out = {"x": np.zeros((T, d)), "w_router": np.zeros((d, N)), "b_router": np.zeros(N),
           "w_q": np.zeros((N, d, dh)), "w_q_shared": np.zeros((d, dh)), "w_k": np.zeros((d, G * dh)),
           "w_v": np.zeros((d, G * dh)), "w_o": np.zeros((N, dh, d)), "w_o_rslot": np.zeros((G, dh, d)),
           "w_o_shared": np.zeros((dh, d))}
    cc = cfg.c()
    rc = lib.gqe_oracle_backward(ctypes.byref(cc), B, S, *[_ptr(a) for a in ins[:9]], _ptr(ins[9]),
                                 _ptr(idx), _ptr(_f64(dy).reshape(T, d)), float(aux_coef),
                                 *[_ptr(out[kk]) for kk in GRAD_KEYS])
    if rc != 0:
        raise ValueError("oracle backward: invalid configuration")
    return out


def loss(cfg: OracleConfig, B: int, S: int, x, w: dict, dy, aux_coef: float, idx) -> float:
    """L = sum(dy * y) + aux_coef * aux with the routing held at ``idx`` (for finite differences)."""
    T = B * S
    x = _f64(x).reshape(T, cfg.dim)
    r = router(cfg, x, w["w_router"], w.get("b_router"))
    out = forward(cfg, B, S, x, w, idx_override=idx)
    st = aux(cfg, r["p"], idx)
    return float(np.sum(_f64(dy).reshape(T, cfg.dim) * out["y"]) + aux_coef * st["aux"])
