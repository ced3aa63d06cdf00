"""Thin ctypes binding of libgqe (C ABI in include/gqe.h).

Argument marshalling only: every step of the forward pass runs in the library's HIP kernels.
PyTorch supplies device memory and streams.  The functions keep the C names; ``GQEAttention``
and ``collect_aux_loss`` wrap them in the shape of the README's usage example
(``attn = GQEAttention(dim=768, num_query_experts=16, num_kv_heads=8, top_k=1)``,
``y = attn(x)``, ``collect_aux_loss(attn)``).
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgqe.so")

VARIANTS = {"gqe": 0, "weighted_concat": 1, "hard_concat": 2}
DTYPES = {"f32": 0, "bf16": 1}
TORCH_DTYPES = {"f32": torch.float32, "bf16": torch.bfloat16}
ERRORS = {0: "GQE_OK", -1: "GQE_ERR_INVALID_CONFIG", -2: "GQE_ERR_NULL_POINTER",
          -3: "GQE_ERR_MISALIGNED", -4: "GQE_ERR_UNSUPPORTED", -5: "GQE_ERR_WORKSPACE",
          -6: "GQE_ERR_SHAPE", -7: "GQE_ERR_HIP", -8: "GQE_ERR_STATE"}
EXPORTS = ("gqe_init", "gqe_packed_weights_bytes", "gqe_pack_weights", "gqe_workspace_bytes",
           "gqe_forward", "gqe_forward_static", "gqe_aux_stats", "gqe_workspace_layout", "gqe_bucket", "gqe_profile_enable",
           "gqe_profile_read", "gqe_profile_read_kernels", "gqe_attention_schedule", "gqe_kv_export",
           "gqe_decode_workspace_bytes", "gqe_decode", "gqe_backward_workspace_bytes", "gqe_backward",
           "gqe_destroy", "gqe_last_error") + (
           "gqe_moe_init", "gqe_moe_packed_weights_bytes", "gqe_moe_pack_weights", "gqe_moe_workspace_bytes",
           "gqe_moe_forward", "gqe_moe_stats", "gqe_moe_workspace_layout", "gqe_moe_profile_enable",
           "gqe_moe_profile_read_kernels", "gqe_moe_destroy")
ACTIVATIONS = {"gelu": 0, "relu": 1}
# kernel timing slots of gqe_moe_profile_read_kernels
MOE_KERNELS = ("moe_router", "moe_router_stats", "moe_bucket", "moe_up", "moe_down", "moe_combine")
STAGES = ("router", "projection", "attention", "combine")
# kernel timing slots of gqe_profile_read_kernels, in launch order
KERNELS = ("router", "router_stats", "projection", "key_norms", "attention_prep", "attention", "attention_merge",
           "combine", "decode_projection", "decode_attention", "decode_merge", "decode_combine",
           "backward_output", "backward_attention", "backward_weights", "backward_dx", "attention_schedule")
GRAD_FIELDS = ("dx", "d_router", "d_router_bias", "d_q", "d_q_shared", "d_k", "d_v", "d_o", "d_o_rslot",
               "d_o_shared")


class GqeError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"{ERRORS.get(code, code)}: {msg}")
        self.code = code


class Config(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "dim", "num_query_experts", "num_kv_heads", "top_k", "head_dim", "variant",
        "shared_head", "shared_kv_group", "dtype", "causal", "dense_gqa")] + [("rope_base", ctypes.c_float)]


class Weights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in (
        "w_router", "b_router", "w_q", "w_q_shared", "w_k", "w_v", "w_o", "w_o_rslot",
        "w_o_shared")]


class Grads(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in GRAD_FIELDS]


class MoeConfig(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("dim", "num_experts", "top_k", "d_ff", "activation", "dtype")]


class MoeWeights(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("w_router", "b_router", "w1", "w2")]


_lib = None


def lib():
    """Load libgqe.so; fails loudly when the HIP library has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                               "(hipcc for gfx950); there is no fallback")
        L = ctypes.CDLL(LIB_PATH)
        P, I64, SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
        L.gqe_init.argtypes = [ctypes.POINTER(Config), ctypes.POINTER(Weights), ctypes.POINTER(P)]
        L.gqe_packed_weights_bytes.argtypes = [P, ctypes.POINTER(SZ)]
        L.gqe_pack_weights.argtypes = [P, P, SZ, P]
        L.gqe_workspace_bytes.argtypes = [P, I64, I64, ctypes.POINTER(SZ)]
        L.gqe_forward.argtypes = [P, P, P, I64, I64, P, SZ, P, P, P]
        L.gqe_forward_static.argtypes = [P, P, P, I64, I64, P, P, P]
        L.gqe_aux_stats.argtypes = [P, P, P, P, P, P]
        L.gqe_workspace_layout.argtypes = [P, I64, I64, P, P]
        L.gqe_bucket.argtypes = [P, P, P, P, P]
        L.gqe_profile_enable.argtypes = [P, ctypes.c_int]
        L.gqe_profile_read.argtypes = [P, P, P]
        L.gqe_profile_read_kernels.argtypes = [P, P, P]
        L.gqe_attention_schedule.argtypes = [P, I64, I64, P, I64, P, I64, P]
        L.gqe_kv_export.argtypes = [P, P, P, P, I64, I64, I64]
        L.gqe_decode_workspace_bytes.argtypes = [P, I64, I64, ctypes.POINTER(SZ)]
        L.gqe_decode.argtypes = [P, P, P, I64, P, P, P, I64, P, SZ, P, P, P]
        L.gqe_backward_workspace_bytes.argtypes = [P, I64, I64, ctypes.POINTER(SZ)]
        L.gqe_backward.argtypes = [P, P, P, I64, I64, ctypes.c_double, P, P, SZ, ctypes.POINTER(Grads), P]
        L.gqe_moe_init.argtypes = [ctypes.POINTER(MoeConfig), ctypes.POINTER(MoeWeights), ctypes.POINTER(P)]
        L.gqe_moe_packed_weights_bytes.argtypes = [P, ctypes.POINTER(SZ)]
        L.gqe_moe_pack_weights.argtypes = [P, P, SZ, P]
        L.gqe_moe_workspace_bytes.argtypes = [P, I64, ctypes.POINTER(SZ)]
        L.gqe_moe_forward.argtypes = [P, P, P, I64, P, SZ, P, P, P]
        L.gqe_moe_stats.argtypes = [P, P, P, P, P]
        L.gqe_moe_workspace_layout.argtypes = [P, I64, P]
        L.gqe_moe_profile_enable.argtypes = [P, ctypes.c_int]
        L.gqe_moe_profile_read_kernels.argtypes = [P, P, P]
        L.gqe_moe_destroy.argtypes = [P]
        L.gqe_moe_destroy.restype = None
        L.gqe_destroy.argtypes = [P]
        L.gqe_destroy.restype = None
        L.gqe_last_error.argtypes = []
        L.gqe_last_error.restype = ctypes.c_char_p
        for f in ("gqe_init", "gqe_packed_weights_bytes", "gqe_pack_weights",
                  "gqe_workspace_bytes", "gqe_forward", "gqe_forward_static", "gqe_aux_stats", "gqe_workspace_layout", "gqe_bucket",
                  "gqe_profile_enable", "gqe_profile_read", "gqe_profile_read_kernels",
                  "gqe_attention_schedule", "gqe_kv_export", "gqe_decode_workspace_bytes", "gqe_decode",
                  "gqe_backward_workspace_bytes", "gqe_backward", "gqe_moe_init", "gqe_moe_packed_weights_bytes",
                  "gqe_moe_pack_weights", "gqe_moe_workspace_bytes", "gqe_moe_forward", "gqe_moe_stats",
                  "gqe_moe_workspace_layout", "gqe_moe_profile_enable", "gqe_moe_profile_read_kernels"):
            getattr(L, f).restype = ctypes.c_int
        _lib = L
    return _lib


def _check(rc: int):
    if rc != 0:
        raise GqeError(rc, gqe_last_error())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


# ------------------------------------------------------------------------- C names
def gqe_last_error() -> str:
    return lib().gqe_last_error().decode()


def gqe_init(cfg: Config, weights: Weights) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(lib().gqe_init(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(h)))
    return h


def gqe_packed_weights_bytes(h) -> int:
    n = ctypes.c_size_t()
    _check(lib().gqe_packed_weights_bytes(h, ctypes.byref(n)))
    return n.value


def gqe_pack_weights(h, packed: torch.Tensor, stream=None):
    _check(lib().gqe_pack_weights(h, _ptr(packed), packed.numel() * packed.element_size(),
                                  _stream(stream)))


def gqe_workspace_bytes(h, batch: int, seq: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().gqe_workspace_bytes(h, batch, seq, ctypes.byref(n)))
    return n.value


def gqe_forward(h, x: torch.Tensor, y: torch.Tensor, batch: int, seq: int,
                workspace: torch.Tensor, stream=None, route_idx=None, route_w=None):
    _check(lib().gqe_forward(h, _ptr(x), _ptr(y), batch, seq, _ptr(workspace),
                             workspace.numel() * workspace.element_size(), _stream(stream),
                             _ptr(route_idx), _ptr(route_w)))


def gqe_forward_static(h, x: torch.Tensor, y: torch.Tensor, batch: int, seq: int, stream=None,
                       route_idx=None, route_w=None):
    """The forward on the library's static per-GPU scratch (no workspace argument)."""
    _check(lib().gqe_forward_static(h, _ptr(x), _ptr(y), batch, seq, _stream(stream), _ptr(route_idx),
                                    _ptr(route_w)))


STATIC_SCRATCH_BYTES = 64 << 20


def gqe_bucket(h, offs: torch.Tensor, perm: torch.Tensor, inv: torch.Tensor, stream=None):
    _check(lib().gqe_bucket(h, _stream(stream), _ptr(offs), _ptr(perm), _ptr(inv)))


def gqe_aux_stats(h, n_experts: int, stream=None) -> dict:
    counts = np.zeros(n_experts, np.int64)
    mean = np.zeros(n_experts, np.float64)
    aux = np.zeros(1, np.float64)
    heads = np.zeros(1, np.int32)
    _check(lib().gqe_aux_stats(h, _stream(stream), counts.ctypes.data_as(ctypes.c_void_p),
                               mean.ctypes.data_as(ctypes.c_void_p),
                               aux.ctypes.data_as(ctypes.c_void_p),
                               heads.ctypes.data_as(ctypes.c_void_p)))
    return dict(counts=counts, mean_prob=mean, aux=float(aux[0]), active_heads=int(heads[0]))


def gqe_workspace_layout(h, batch: int, seq: int):
    offs = (ctypes.c_size_t * 12)()
    dims = (ctypes.c_int64 * 4)()
    _check(lib().gqe_workspace_layout(h, batch, seq, offs, dims))
    return list(offs), list(dims)


def gqe_profile_enable(h, enable: bool):
    _check(lib().gqe_profile_enable(h, int(enable)))


def gqe_profile_read(h):
    ms = (ctypes.c_double * 4)()
    n = ctypes.c_int64()
    _check(lib().gqe_profile_read(h, ms, ctypes.byref(n)))
    return dict(zip(STAGES, list(ms))), n.value


def gqe_profile_read_kernels(h):
    ms = (ctypes.c_double * len(KERNELS))()
    n = ctypes.c_int64()
    _check(lib().gqe_profile_read_kernels(h, ms, ctypes.byref(n)))
    return dict(zip(KERNELS, list(ms))), n.value


def gqe_attention_schedule(h, batch: int, seq: int):
    """The attention work schedule (host only): jobs [n, 8] and merges [m, 8] int32 (numpy), the
    number of partial slots and the chunk cap in key tiles."""
    import numpy as np
    counts = (ctypes.c_int64 * 4)()
    _check(lib().gqe_attention_schedule(h, batch, seq, None, 0, None, 0, counts))
    jobs = np.zeros((max(counts[0], 1), 8), dtype=np.int32)
    merges = np.zeros((max(counts[1], 1), 8), dtype=np.int32)
    _check(lib().gqe_attention_schedule(h, batch, seq, jobs.ctypes.data_as(ctypes.c_void_p), jobs.shape[0],
                                        merges.ctypes.data_as(ctypes.c_void_p), merges.shape[0], counts))
    return jobs[:counts[0]], merges[:counts[1]], int(counts[2]), int(counts[3])


def gqe_kv_export(h, kcache: torch.Tensor, vcache: torch.Tensor, b0: int = 0, stream=None):
    """Keys and values of the last forward -> cache rows b0 .. b0+B-1 ([rows, G, s_max, d_h])."""
    _check(lib().gqe_kv_export(h, _stream(stream), _ptr(kcache), _ptr(vcache), kcache.shape[0],
                               kcache.shape[2], b0))


def gqe_decode_workspace_bytes(h, batch: int, s_max: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().gqe_decode_workspace_bytes(h, batch, s_max, ctypes.byref(n)))
    return n.value


def gqe_decode(h, x: torch.Tensor, y: torch.Tensor, pos: torch.Tensor, kcache: torch.Tensor,
               vcache: torch.Tensor, workspace: torch.Tensor, stream=None, route_idx=None, route_w=None):
    _check(lib().gqe_decode(h, _ptr(x), _ptr(y), x.shape[0], _ptr(pos), _ptr(kcache), _ptr(vcache),
                            kcache.shape[2], _ptr(workspace), workspace.numel() * workspace.element_size(),
                            _stream(stream), _ptr(route_idx), _ptr(route_w)))


def gqe_backward_workspace_bytes(h, batch: int, seq: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().gqe_backward_workspace_bytes(h, batch, seq, ctypes.byref(n)))
    return n.value


def gqe_backward(h, x: torch.Tensor, dy: torch.Tensor, batch: int, seq: int, aux_coef: float,
                 fwd_workspace: torch.Tensor, workspace: torch.Tensor, grads: dict, stream=None):
    g = Grads(*[_ptr(grads.get(f)) for f in GRAD_FIELDS])
    _check(lib().gqe_backward(h, _ptr(x), _ptr(dy), batch, seq, float(aux_coef), _ptr(fwd_workspace),
                              _ptr(workspace), workspace.numel() * workspace.element_size(), ctypes.byref(g),
                              _stream(stream)))


def gqe_destroy(h):
    if h:
        lib().gqe_destroy(h)


# ------------------------------------------------------------------------- C names: MoE-MLP
def gqe_moe_init(cfg: MoeConfig, weights: MoeWeights) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(lib().gqe_moe_init(ctypes.byref(cfg), ctypes.byref(weights), ctypes.byref(h)))
    return h


def gqe_moe_packed_weights_bytes(h) -> int:
    n = ctypes.c_size_t()
    _check(lib().gqe_moe_packed_weights_bytes(h, ctypes.byref(n)))
    return n.value


def gqe_moe_pack_weights(h, packed: torch.Tensor, stream=None):
    _check(lib().gqe_moe_pack_weights(h, _ptr(packed), packed.numel() * packed.element_size(), _stream(stream)))


def gqe_moe_workspace_bytes(h, tokens: int) -> int:
    n = ctypes.c_size_t()
    _check(lib().gqe_moe_workspace_bytes(h, tokens, ctypes.byref(n)))
    return n.value


def gqe_moe_forward(h, x: torch.Tensor, y: torch.Tensor, tokens: int, ws: torch.Tensor, stream=None,
                    route_idx: torch.Tensor | None = None, route_w: torch.Tensor | None = None):
    _check(lib().gqe_moe_forward(h, _ptr(x), _ptr(y), tokens, _ptr(ws), ws.numel(), _stream(stream),
                                 _ptr(route_idx), _ptr(route_w)))


def gqe_moe_stats(h, n_experts: int, stream=None) -> dict:
    counts = (ctypes.c_int64 * n_experts)()
    mean = (ctypes.c_double * n_experts)()
    aux = ctypes.c_double()
    _check(lib().gqe_moe_stats(h, _stream(stream), counts, mean, ctypes.byref(aux)))
    return dict(counts=np.array(counts[:], dtype=np.int64), mean_prob=np.array(mean[:]), aux=aux.value)


def gqe_moe_workspace_layout(h, tokens: int):
    offs = (ctypes.c_size_t * 7)()
    _check(lib().gqe_moe_workspace_layout(h, tokens, offs))
    return list(offs)


def gqe_moe_profile_enable(h, enable: bool):
    _check(lib().gqe_moe_profile_enable(h, int(enable)))


def gqe_moe_profile_read_kernels(h):
    ms = (ctypes.c_double * len(MOE_KERNELS))()
    n = ctypes.c_int64()
    _check(lib().gqe_moe_profile_read_kernels(h, ms, ctypes.byref(n)))
    return dict(zip(MOE_KERNELS, ms[:])), n.value


def gqe_moe_destroy(h):
    lib().gqe_moe_destroy(h)


# ------------------------------------------------------------------------- module wrapper
class MoEMLP:
    """Top-k mixture-of-experts MLP (the tutorial's moe_layer with expert MLPs): weights are device
    tensors w_router [d, E] f32, b_router [E] f32 or None, w1 [E, d, d_ff] bf16, w2 [E, d_ff, d] bf16."""

    WEIGHT_KEYS = ("w_router", "b_router", "w1", "w2")

    def __init__(self, dim: int, num_experts: int, top_k: int, d_ff: int, activation: str = "gelu",
                 weights: dict | None = None, stream=None):
        if weights is None:
            raise ValueError("weights (device tensors) are required")
        self.dim, self.E, self.k, self.d_ff = dim, num_experts, top_k, d_ff
        self.cfg = MoeConfig(dim, num_experts, top_k, d_ff, ACTIVATIONS[activation], DTYPES["bf16"])
        self._w = {k: weights.get(k) for k in self.WEIGHT_KEYS}
        self.weights = MoeWeights(*[_ptr(self._w[k]) for k in self.WEIGHT_KEYS])
        self.h = gqe_moe_init(self.cfg, self.weights)
        self.device = self._w["w1"].device
        self.packed = torch.empty(max(gqe_moe_packed_weights_bytes(self.h), 256), dtype=torch.uint8,
                                  device=self.device)
        gqe_moe_pack_weights(self.h, self.packed, stream)
        self._ws = None

    def workspace(self, tokens: int) -> torch.Tensor:
        nbytes = max(gqe_moe_workspace_bytes(self.h, tokens), 256)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self._ws

    def __call__(self, x: torch.Tensor, y: torch.Tensor | None = None, stream=None, route_idx=None,
                 route_w=None) -> torch.Tensor:
        if x.dim() != 2 or x.shape[1] != self.dim or x.dtype != torch.bfloat16 or not x.is_contiguous():
            raise ValueError("x must be a contiguous [tokens, dim] bf16 tensor")
        if y is None:
            y = torch.empty_like(x)
        T = x.shape[0]
        gqe_moe_forward(self.h, x, y, T, self.workspace(T), stream, route_idx, route_w)
        return y

    def stats(self, stream=None) -> dict:
        return gqe_moe_stats(self.h, self.E, stream)

    def intermediates(self, tokens: int) -> dict:
        """Views of the last forward's bucketing, hidden activations and expert outputs."""
        offs = gqe_moe_workspace_layout(self.h, tokens)
        ws = self._ws
        P = tokens * self.k

        def view(off, shape, dt, es):
            n = int(np.prod(shape))
            return ws[off:off + n * es].view(dt).view(*shape)

        return dict(offs=view(offs[0], (self.E + 1,), torch.int32, 4), perm=view(offs[1], (P,), torch.int32, 4),
                    inv=view(offs[2], (tokens, self.k), torch.int32, 4),
                    h=view(offs[3], (P, self.d_ff), torch.bfloat16, 2), Y=view(offs[4], (P, self.dim), torch.float32, 4),
                    idx=view(offs[5], (tokens, self.k), torch.int32, 4),
                    w=view(offs[6], (tokens, self.k), torch.float32, 4))

    def close(self):
        if self.h:
            gqe_moe_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class GQEAttention:
    """GQEAttention(dim, num_query_experts=16, num_kv_heads=8, top_k=1, head_dim=None,
    variant="gqe") as in the README; weights are device tensors in the C ABI layouts."""

    WEIGHT_KEYS = ("w_router", "b_router", "w_q", "w_q_shared", "w_k", "w_v", "w_o",
                   "w_o_rslot", "w_o_shared")

    def __init__(self, dim: int, num_query_experts: int = 16, num_kv_heads: int = 8,
                 top_k: int = 1, head_dim: int | None = None, variant: str = "gqe",
                 shared_head: bool = True, shared_kv_group: int = 0, dtype: str = "bf16",
                 dense_gqa: bool = False, weights: dict | None = None, stream=None, rope_base: float = 0.0):
        if weights is None:
            raise ValueError("weights (device tensors) are required")
        self.dtype = dtype
        self.N = num_query_experts
        self.G = num_kv_heads
        self.k = top_k
        self.dim = dim
        self.cfg = Config(dim, num_query_experts, num_kv_heads, top_k, head_dim or 0,
                          VARIANTS[variant], int(shared_head), shared_kv_group, DTYPES[dtype], 1,
                          int(dense_gqa), float(rope_base))
        self._w = {k: weights.get(k) for k in self.WEIGHT_KEYS}   # keep alive
        self.weights = Weights(*[_ptr(self._w[k]) for k in self.WEIGHT_KEYS])
        self.h = gqe_init(self.cfg, self.weights)
        dev = next(v.device for v in self._w.values() if v is not None)
        self.device = dev
        self.packed = torch.empty(max(gqe_packed_weights_bytes(self.h), 256), dtype=torch.uint8,
                                  device=dev)
        gqe_pack_weights(self.h, self.packed, stream)
        self._ws = None
        self._ws_shape = None
        self._dws = None
        self.dh = int(head_dim or dim // num_query_experts)

    def workspace(self, batch: int, seq: int) -> torch.Tensor:
        nbytes = gqe_workspace_bytes(self.h, batch, seq)
        if self._ws is None or self._ws.numel() < nbytes:
            self._ws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        return self._ws

    def __call__(self, x: torch.Tensor, y: torch.Tensor | None = None, stream=None,
                 route_idx=None, route_w=None) -> torch.Tensor:
        B, S, d = x.shape
        if d != self.dim or x.dtype != TORCH_DTYPES[self.dtype] or not x.is_contiguous():
            raise ValueError("x must be a contiguous [B, S, dim] tensor of the layer's dtype")
        if y is None:
            y = torch.empty_like(x)
        ws = self.workspace(B, S)
        gqe_forward(self.h, x, y, B, S, ws, stream, route_idx, route_w)
        return y

    def aux_stats(self, stream=None) -> dict:
        return gqe_aux_stats(self.h, self.N, stream)

    # ---- backward pass
    def backward(self, x: torch.Tensor, dy: torch.Tensor, aux_coef: float = 0.0, stream=None) -> dict:
        """Gradients of sum(dy * y) + aux_coef * aux for the last forward (which must have been on
        this x): float32 tensors keyed like gqe_grads_t (dx, d_router, ..., d_o_shared)."""
        B, S, d = x.shape
        if dy.shape != x.shape or dy.dtype != x.dtype or not dy.is_contiguous():
            raise ValueError("dy must be a contiguous tensor like x")
        dh, N, G = self.dh, self.N, self.G
        f32 = dict(dtype=torch.float32, device=self.device)
        shapes = {"dx": (B, S, d), "d_router": (d, N), "d_router_bias": (N,), "d_q": (N, d, dh),
                  "d_q_shared": (d, dh), "d_k": (d, G * dh), "d_v": (d, G * dh), "d_o": (N, dh, d),
                  "d_o_rslot": (G, dh, d), "d_o_shared": (dh, d)}
        if self.cfg.dense_gqa:
            shapes.pop("d_router"), shapes.pop("d_router_bias")
        if not self.cfg.shared_head:
            shapes.pop("d_q_shared"), shapes.pop("d_o_shared")
        if self.cfg.dense_gqa or self.cfg.variant != VARIANTS["gqe"]:
            shapes.pop("d_o_rslot")
        grads = {k: torch.empty(v, **f32) for k, v in shapes.items()}
        nbytes = gqe_backward_workspace_bytes(self.h, B, S)
        bws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=self.device)
        gqe_backward(self.h, x, dy, B, S, aux_coef, self._ws, bws, grads, stream)
        return grads

    # ---- decode with a dense KV cache
    def kv_cache(self, batch: int, s_max: int):
        """Empty K and V caches [batch, G, s_max, d_h] of the layer's dtype."""
        shape = (batch, self.G, s_max, self.dh)
        td = TORCH_DTYPES[self.dtype]
        return (torch.empty(shape, dtype=td, device=self.device),
                torch.empty(shape, dtype=td, device=self.device))

    def export_kv(self, kcache: torch.Tensor, vcache: torch.Tensor, b0: int = 0, stream=None):
        """Writes the keys and values of the last forward into cache rows b0 .. b0+B-1."""
        self._check_cache(kcache, vcache)
        gqe_kv_export(self.h, kcache, vcache, b0, stream)

    def decode(self, x: torch.Tensor, pos: torch.Tensor, kcache: torch.Tensor, vcache: torch.Tensor,
               y: torch.Tensor | None = None, stream=None, route_idx=None, route_w=None) -> torch.Tensor:
        """One decode step: x [B, dim] (new token of every sequence), pos [B] int32 on the device
        (its position = tokens already cached); appends its K/V to the caches and returns y [B, dim]."""
        B, d = x.shape
        if d != self.dim or x.dtype != TORCH_DTYPES[self.dtype] or not x.is_contiguous():
            raise ValueError("x must be a contiguous [B, dim] tensor of the layer's dtype")
        if pos.dtype != torch.int32 or pos.shape != (B,) or not pos.is_contiguous():
            raise ValueError("pos must be a contiguous int32 tensor [B]")
        self._check_cache(kcache, vcache)
        if kcache.shape[0] < B:
            raise ValueError("the caches have fewer rows than the batch")
        if y is None:
            y = torch.empty_like(x)
        nbytes = gqe_decode_workspace_bytes(self.h, B, kcache.shape[2])
        if self._dws is None or self._dws.numel() < nbytes:
            self._dws = torch.empty(nbytes, dtype=torch.uint8, device=self.device)
        gqe_decode(self.h, x, y, pos, kcache, vcache, self._dws, stream, route_idx, route_w)
        return y

    def _check_cache(self, kcache, vcache):
        td = TORCH_DTYPES[self.dtype]
        for c in (kcache, vcache):
            if (c.dim() != 4 or c.shape[1] != self.G or c.shape[3] != self.dh or c.dtype != td
                    or not c.is_contiguous()):
                raise ValueError("caches must be contiguous [rows, G, s_max, d_h] tensors of the layer's dtype")
        if kcache.shape != vcache.shape:
            raise ValueError("kcache and vcache must have the same shape")

    def bucket(self, batch: int, seq: int, stream=None) -> dict:
        """Global token-to-expert bucketing of the last forward (device int32 tensors)."""
        G, k = self.cfg.num_kv_heads, self.cfg.top_k
        offs = torch.empty(self.N + 1, dtype=torch.int32, device=self.device)
        perm = torch.empty(batch * seq * G * k, dtype=torch.int32, device=self.device)
        inv = torch.empty((batch * seq, G, k), dtype=torch.int32, device=self.device)
        gqe_bucket(self.h, offs, perm, inv, stream)
        return dict(offs=offs, perm=perm, inv=inv)

    def intermediates(self, batch: int, seq: int) -> dict:
        """Views of Q_act, K, V^T, O_act and the routing buffers inside the workspace."""
        offs, dims = gqe_workspace_layout(self.h, batch, seq)
        H, S_pad = dims[0], dims[1]
        es = 2 if self.dtype == "bf16" else 4
        td = TORCH_DTYPES[self.dtype]
        dh = int(self.cfg.head_dim or self.dim // self.N)
        ws = self._ws
        T = batch * seq

        def view(off, shape, dt, esz):
            n = int(np.prod(shape))
            return ws[off:off + n * esz].view(dt).reshape(shape)

        return dict(
            q=view(offs[0], (batch, H, seq, dh), td, es),
            k=view(offs[1], (batch, self.G, S_pad, dh), td, es),
            vt=view(offs[2], (batch, self.G, dh, S_pad), td, es),
            o=view(offs[3], (batch, seq, H, dh), td, es),
            idx=view(offs[4], (T, self.G, self.k), torch.int32, 4),
            w=view(offs[5], (T, self.G, self.k), torch.float32, 4),
            psel=view(offs[6], (T, self.G, self.k), torch.float32, 4),
            kn=view(offs[8], (batch, self.G, S_pad), torch.float32, 4),
            knt=view(offs[9], (batch, self.G, S_pad // 64), torch.float32, 4),
            jobs=view(offs[10], (dims[3], 8), torch.int32, 4),
            merges_offset=offs[11],
            matrix_core=bool(dims[2]),
        )

    def close(self):
        if self.h:
            gqe_destroy(self.h)
            self.h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def collect_aux_loss(attn: GQEAttention, stream=None) -> float:
    """README 'Usage': the load-balancing loss of the last forward (unscaled)."""
    return attn.aux_stats(stream)["aux"]


def vt_unpermute(vt: torch.Tensor) -> torch.Tensor:
    """Undo the key slotting of V^T (bits 2 and 3 of the key offset inside every 16-key chunk
    are swapped) -> [..., d_h, S_pad] in key order."""
    S_pad = vt.shape[-1]
    pos = np.arange(S_pad)
    o = pos & 15
    slot = (o & ~12) | ((o & 4) << 1) | ((o & 8) >> 1)
    src = (pos & ~15) | slot
    return vt[..., torch.as_tensor(src, device=vt.device)]


def upload_weights(w: dict, device, dtype: str) -> dict:
    """Host arrays from inputs.make_inputs -> device tensors of the ABI dtypes."""
    td = TORCH_DTYPES[dtype]
    out = {}
    for k, v in w.items():
        if k == "x":
            continue
        t = torch.from_numpy(np.ascontiguousarray(v))
        out[k] = t.to(device=device, dtype=torch.float32 if k in ("w_router", "b_router") else td)
    return out
