"""GPU parity of the decode step with a dense KV cache, through the C ABI, against the oracle.

The cache is filled the way a user fills it: a forward pass (prefill) of each sequence's prefix,
then gqe_kv_export into that sequence's cache row.  Then several decode steps append one token
per sequence each (ragged positions, including an empty cache); every step's output is compared
with the oracle's decode (row p of the causal forward over the prefix 0..p), and its routing
with the oracle's router.
"""
import numpy as np
import pytest
import torch

from sparse_moe_query_amd.inputs import Workload
from tests import parity

pytestmark = pytest.mark.gpu


def _wl(name, d=768, N=16, G=8, k=1, dh=48, B=4, S=310, **kw):
    return Workload(name, d, N, G, k, dh, B, S, **kw)


def _prefill(layer, x, lens, s_max):
    """Caches [B, G, s_max, d_h] holding the K/V of x[b, :lens[b]] (forward + export per row)."""
    kc, vc = layer.kv_cache(x.shape[0], s_max)
    kc.zero_()
    vc.zero_()
    for b, L in enumerate(lens):
        if L == 0:
            continue
        layer(x[b:b + 1, :L])
        layer.export_kv(kc, vc, b0=b)
    return kc, vc


def _decode_steps(wl, lens, steps, s_max):
    from sparse_moe_query_amd.runner import build_layer
    print(f"[gpu] decode {wl.name} B={wl.batch} lens={lens} steps={steps} s_max={s_max} d={wl.dim} "
          f"k={wl.top_k} dh={wl.dh} {wl.dtype} {wl.variant}", flush=True)
    layer, x, inp = build_layer(wl)
    kc, vc = _prefill(layer, x, lens, s_max)
    B = wl.batch
    reps = []
    for t in range(steps):
        pos = [L + t for L in lens]
        xn = torch.stack([x[b, p] for b, p in enumerate(pos)]).contiguous()
        pd = torch.tensor(pos, dtype=torch.int32, device=x.device)
        ridx = rw = None
        if not wl.dense_gqa:
            ridx = torch.full((B, wl.num_kv_heads, wl.top_k), -1, dtype=torch.int32, device=x.device)
            rw = torch.full((B, wl.num_kv_heads, wl.top_k), -1.0, dtype=torch.float32, device=x.device)
        y = layer.decode(xn, pd, kc, vc, route_idx=ridx, route_w=rw)
        torch.cuda.synchronize()
        yh = y.float().cpu().numpy().astype(np.float64)
        ih = ridx.cpu().numpy() if ridx is not None else None
        wh = rw.cpu().numpy() if rw is not None else None
        reps.append(parity.compare_decode(wl, yh, ih, wh, inp, pos))
    print(f"[gpu]   y_err per step {[round(r['y_err'], 5) for r in reps]}", flush=True)
    return layer, x, inp, kc, vc, reps


CASES = [
    # main setting, ragged prefixes: empty cache, one tile, past one 256-key chunk
    (_wl("dec_main"), [0, 63, 257, 300], 3, 320),
    (Workload("dec_tiny_fp32", 64, 4, 2, 1, 16, 3, 40, dtype="f32", router_std=0.02), [1, 17, 35], 2, 40),
    (_wl("dec_k2_skew", d=1024, k=2, dh=64, B=2, S=600, router_std=2.70 / 32.0, router_bias_first=2.0),
     [300, 555], 2, 600),
    (_wl("dec_weighted", B=2, S=200, variant="weighted_concat", seed=1), [100, 190], 2, 256),
    (_wl("dec_hard_noshared", B=2, S=200, variant="hard_concat", shared_head=False, seed=2), [5, 150], 2, 256),
    (_wl("dec_shared_group3", B=2, S=200, shared_kv_group=3, seed=3), [40, 199], 1, 200),
    (_wl("dec_gqa", B=2, S=300, k=2, variant="hard_concat", shared_head=False, dense_gqa=True, seed=4),
     [128, 290], 2, 300),
    (_wl("dec_dh32_k2", d=256, N=8, G=4, k=2, dh=32, B=3, S=520, seed=5), [0, 256, 511], 2, 520),
    (_wl("dec_f32_dh32", d=64, N=4, G=2, k=1, dh=32, B=2, S=300, dtype="f32", router_std=0.3, seed=6),
     [129, 290], 2, 300),
]


@pytest.mark.parametrize("wl,lens,steps,s_max", CASES, ids=[c[0].name for c in CASES])
def test_decode_matches_oracle(wl, lens, steps, s_max):
    _decode_steps(wl, lens, steps, s_max)


def test_decode_long_cache():
    """One sequence with 8000 cached keys: 32 chunks merged, s_max a multiple of the chunk."""
    _decode_steps(_wl("dec_long", B=1, S=8002, seed=7), [8000], 2, 8192)


def test_export_is_the_forward_kv():
    """The exported cache rows are the forward pass's K and V, bit for bit (data movement only)."""
    from sparse_moe_query_amd.gqe import vt_unpermute
    from sparse_moe_query_amd.runner import build_layer
    wl = _wl("export", B=2, S=150, seed=8)
    layer, x, _ = build_layer(wl)
    layer(x)
    kc, vc = layer.kv_cache(3, 160)
    kc.zero_()
    vc.zero_()
    layer.export_kv(kc, vc, b0=1)
    torch.cuda.synchronize()
    it = layer.intermediates(wl.batch, wl.seq)
    k_ref = it["k"][:, :, :wl.seq]
    v_ref = vt_unpermute(it["vt"])[:, :, :, :wl.seq].transpose(2, 3)
    assert torch.equal(kc[1:3, :, :wl.seq], k_ref)
    assert torch.equal(vc[1:3, :, :wl.seq], v_ref)
    assert not torch.count_nonzero(kc[0]) and not torch.count_nonzero(kc[1:, :, wl.seq:])
    assert not torch.count_nonzero(vc[0])


def test_decode_deterministic_and_invalid_positions():
    """Two identical steps give identical bits; a position outside [0, s_max) gives a NaN row and
    leaves that sequence's cache untouched while the other sequences are still correct."""
    from sparse_moe_query_amd.runner import build_layer
    wl = _wl("dec_invalid", B=3, S=100, seed=9)
    print("[gpu] decode invalid positions", flush=True)
    layer, x, inp = build_layer(wl)
    s_max = 96
    kc, vc = _prefill(layer, x, [50, 60, 70], s_max)
    pos = torch.tensor([50, s_max, -1], dtype=torch.int32, device=x.device)
    xn = torch.stack([x[0, 50], x[1, 60], x[2, 70]]).contiguous()
    k_before, v_before = kc[1:].clone(), vc[1:].clone()
    ridx = torch.full((3, wl.num_kv_heads, wl.top_k), -1, dtype=torch.int32, device=x.device)
    rw = torch.full((3, wl.num_kv_heads, wl.top_k), -1.0, dtype=torch.float32, device=x.device)
    y1 = layer.decode(xn, pos, kc, vc, route_idx=ridx, route_w=rw).clone()
    y2 = layer.decode(xn, pos, kc, vc).clone()
    torch.cuda.synchronize()
    assert torch.equal(y1[:1], y2[:1])   # (NaN rows never compare equal)
    assert torch.isnan(y1[1:].float()).all() and torch.isnan(y2[1:].float()).all()
    assert torch.equal(kc[1:], k_before) and torch.equal(vc[1:], v_before)
    inp1 = dict(inp)
    inp1["x"] = inp["x"][:1]
    parity.compare_decode(wl.with_(batch=1), y1[:1].float().cpu().numpy().astype(np.float64),
                          ridx[:1].cpu().numpy(), rw[:1].cpu().numpy(), inp1, [50])


ROPE_CASES = [
    (_wl("dec_rope_main", rope_base=10000.0, seed=30), [0, 63, 257, 300], 2, 320),
    (_wl("dec_rope_k2", d=1024, k=2, dh=64, B=2, S=600, rope_base=10000.0, seed=31), [300, 555], 2, 600),
    (Workload("dec_rope_f32", 64, 4, 2, 1, 16, 2, 40, dtype="f32", router_std=0.02, rope_base=500.0, seed=32),
     [5, 30], 2, 40),
]


@pytest.mark.parametrize("wl,lens,steps,s_max", ROPE_CASES, ids=[c[0].name for c in ROPE_CASES])
def test_decode_rope_matches_oracle(wl, lens, steps, s_max):
    """Rotary embedding in decode: the new key is rotated at its position before it is cached; the
    cached keys come rotated from the forward pass."""
    _decode_steps(wl, lens, steps, s_max)
