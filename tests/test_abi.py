"""The C ABI without a GPU: the library loads, exports every entry point declared in
include/gqe.h, and rejects bad arguments on the host before any device call."""
import ctypes
import os
import re

import pytest

from sparse_moe_query_amd import gqe

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "gqe.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(gqe_[a-z_]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("gqe_init", "gqe_forward", "gqe_aux_stats", "gqe_workspace_bytes",
              "gqe_pack_weights", "gqe_destroy", "gqe_last_error"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = gqe.lib()
    for n in _declared():
        assert hasattr(L, n), n
    assert set(_declared()) == set(gqe.EXPORTS)


def _cfg(**kw):
    base = dict(dim=768, num_query_experts=16, num_kv_heads=8, top_k=1, head_dim=0, variant=0,
                shared_head=1, shared_kv_group=0, dtype=1, causal=1, dense_gqa=0, rope_base=0.0)
    base.update(kw)
    return gqe.Config(*[base[f] for f, _ in gqe.Config._fields_])


def _weights(**kw):
    # fake but aligned addresses: gqe_init only validates them and never dereferences
    base = {f: 0x10000 * (i + 1) for i, (f, _) in enumerate(gqe.Weights._fields_)}
    base.update(kw)
    return gqe.Weights(*[base[f] for f, _ in gqe.Weights._fields_])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(num_query_experts=12, num_kv_heads=8), -1, "divisible"),
    (dict(top_k=0), -1, "top_k"),
    (dict(top_k=3), -1, "top_k"),
    (dict(dim=0), -1, "dim"),
    (dict(dim=8, num_query_experts=16), -1, "head_dim"),
    (dict(head_dim=-2), -1, "head_dim"),
    (dict(variant=3), -1, "variant"),
    (dict(dtype=7), -1, "dtype"),
    (dict(shared_kv_group=8), -1, "shared_kv_group"),
    (dict(causal=0), -4, "causal"),
    (dict(dense_gqa=1), -1, "dense_gqa"),
    (dict(num_query_experts=128, num_kv_heads=8), -4, "64"),
    (dict(head_dim=256), -4, "head_dim"),
    (dict(rope_base=-1.0), -1, "rope_base"),
    (dict(rope_base=float("nan")), -1, "rope_base"),
    (dict(rope_base=10000.0, dim=420, num_query_experts=12, num_kv_heads=4, head_dim=35), -1, "even"),
])
def test_init_rejects_bad_configs(kw, code, msg):
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_init(_cfg(**kw), _weights())
    assert e.value.code == code
    assert msg in str(e.value)


def test_init_rejects_null_and_misaligned_weights():
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_init(_cfg(), _weights(w_router=None))
    assert e.value.code == -2
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_init(_cfg(), _weights(w_o_rslot=None))
    assert e.value.code == -2
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_init(_cfg(), _weights(w_k=0x10008))
    assert e.value.code == -3
    # hard_concat needs no renormalised-slot projection, no shared head needs no shared weights
    h = gqe.gqe_init(_cfg(variant=2, shared_head=0), _weights(w_o_rslot=None, w_q_shared=None,
                                                              w_o_shared=None))
    gqe.gqe_destroy(h)


def test_host_side_sizes_and_state_errors():
    h = gqe.gqe_init(_cfg(), _weights())
    try:
        ws = gqe.gqe_workspace_bytes(h, 8, 2048)
        assert ws > 8 * 2048 * 9 * 48 * 2 * 2   # at least Q_act and O_act
        assert gqe.gqe_packed_weights_bytes(h) >= 768 * 16 * 8
        with pytest.raises(gqe.GqeError) as e:
            gqe.gqe_workspace_bytes(h, 0, 10)
        assert e.value.code == -6
        offs, dims = gqe.gqe_workspace_layout(h, 2, 100)
        assert dims[0] == 9 and dims[1] == 128
        assert len(set(offs)) == 12          # every buffer, the attention schedule tables included
        assert dims[3] > 0                   # attention jobs
        # forward before the weights are packed -> state error, no device call
        L = gqe.lib()
        rc = L.gqe_forward(h, ctypes.c_void_p(0x1000), ctypes.c_void_p(0x200000), 1, 1,
                           ctypes.c_void_p(0x400000), 1 << 30, None, None, None)
        assert rc == -8
        rc = L.gqe_aux_stats(h, None, None, None, None, None)
        assert rc == -8
    finally:
        gqe.gqe_destroy(h)
    assert gqe.gqe_last_error() == "" or isinstance(gqe.gqe_last_error(), str)


def test_decode_host_side_errors():
    """Decode entry points check sizes, support and call order on the host."""
    h = gqe.gqe_init(_cfg(), _weights())
    try:
        n = gqe.gqe_decode_workspace_bytes(h, 64, 8192)
        # float32 queries and merged outputs, and per-chunk partials of every (sequence, group)
        assert n >= 64 * 9 * 48 * 4 * 2 + 64 * 8 * 32 * 2 * 50 * 4
        for bad in ((0, 10), (4, 0), (1 << 21, 8)):
            with pytest.raises(gqe.GqeError) as e:
                gqe.gqe_decode_workspace_bytes(h, *bad)
            assert e.value.code == -6
        L = gqe.lib()
        P = ctypes.c_void_p
        args = [P(0x1000), P(0x200000), 1, P(0x300000), P(0x400000), P(0x500000), 16, P(0x600000),
                1 << 30, None, None, None]
        assert L.gqe_decode(h, *args) == -8          # weights not packed yet
        args[3] = None
        assert L.gqe_decode(h, *args) == -2          # no positions
        assert L.gqe_kv_export(h, None, P(0x400000), P(0x500000), 1, 16, 0) == -8  # no forward yet
    finally:
        gqe.gqe_destroy(h)
    # head_dim 20 in bf16: 40-byte cache rows are not whole 16-byte units
    h = gqe.gqe_init(_cfg(dim=320, head_dim=20), _weights())
    try:
        with pytest.raises(gqe.GqeError) as e:
            gqe.gqe_decode_workspace_bytes(h, 2, 64)
        assert e.value.code == -4
    finally:
        gqe.gqe_destroy(h)


# ----------------------------------------------------------------------------- top-k MoE-MLP
def _moe_cfg(**kw):
    base = dict(dim=768, num_experts=8, top_k=2, d_ff=3072, activation=0, dtype=1)
    base.update(kw)
    return gqe.MoeConfig(*[base[f] for f, _ in gqe.MoeConfig._fields_])


def _moe_weights(**kw):
    base = {f: 0x20000 * (i + 1) for i, (f, _) in enumerate(gqe.MoeWeights._fields_)}
    base.update(kw)
    return gqe.MoeWeights(*[base[f] for f, _ in gqe.MoeWeights._fields_])


@pytest.mark.parametrize("kw,code,msg", [
    (dict(num_experts=0), -1, "num_experts"),
    (dict(top_k=0), -1, "top_k"),
    (dict(top_k=9), -1, "top_k"),
    (dict(dim=0), -1, "dim"),
    (dict(d_ff=0), -1, "d_ff"),
    (dict(activation=2), -1, "activation"),
    (dict(dtype=0), -4, "bf16"),
    (dict(num_experts=17, top_k=2), -4, "16"),
    (dict(dim=100), -4, "multiples of 32"),
    (dict(d_ff=3000), -4, "multiples of 32"),
])
def test_moe_init_rejects_bad_configs(kw, code, msg):
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_moe_init(_moe_cfg(**kw), _moe_weights())
    assert e.value.code == code
    assert msg in str(e.value)


def test_moe_host_side_errors_and_sizes():
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_moe_init(_moe_cfg(), _moe_weights(w1=None))
    assert e.value.code == -2
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_moe_init(_moe_cfg(), _moe_weights(w2=0x20008))
    assert e.value.code == -3
    h = gqe.gqe_moe_init(_moe_cfg(), _moe_weights(b_router=None))
    try:
        d, E, k, dff, T = 768, 8, 2, 3072, 1000
        packed = gqe.gqe_moe_packed_weights_bytes(h)
        assert packed >= d * 16 * 8 + 2 * E * d * dff * 2
        ws = gqe.gqe_moe_workspace_bytes(h, T)
        assert ws >= T * k * (dff * 2 + d * 4)   # hidden bf16 + expert outputs float32
        assert gqe.gqe_moe_workspace_bytes(h, 0) >= 0
        offs = gqe.gqe_moe_workspace_layout(h, T)
        assert all(o % 256 == 0 for o in offs) and len(set(offs)) == 7
        with pytest.raises(gqe.GqeError) as e:
            gqe.gqe_moe_workspace_bytes(h, -1)
        assert e.value.code == -6
        with pytest.raises(gqe.GqeError) as e:
            gqe.gqe_moe_workspace_bytes(h, 1 << 30)   # tokens * top_k >= 2^31
        assert e.value.code == -6
        L = gqe.lib()
        # forward before packing, stats before any forward: state errors, no device call
        assert L.gqe_moe_forward(h, 0x1000, 0x2000, 4, 0x10000, 1 << 30, None, None, None) == -8
        assert L.gqe_moe_stats(h, None, None, None, None) == -8
        assert L.gqe_moe_forward(None, 0x1000, 0x2000, 4, 0x10000, 1 << 30, None, None, None) == -2
    finally:
        gqe.gqe_moe_destroy(h)
