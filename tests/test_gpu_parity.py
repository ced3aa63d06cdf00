"""GPU parity: the HIP library through its C ABI against the CPU oracle.

Small shapes are compared on every token and stage by stage (Q_act, K, V, O_act, y); they span
several tiles of every kernel and end in ragged tails.  The full-size workloads are compared on
sampled tokens (both ends of every sequence, tile boundaries, random positions) plus the full
routing and statistics.
"""
import sys

import numpy as np
import pytest
import torch

from sparse_moe_query_amd.inputs import WORKLOADS, Workload, gqa_of, make_inputs
from tests import parity

pytestmark = pytest.mark.gpu


def _run(wl, inputs=None, rows=None, want_qo=False):
    from sparse_moe_query_amd.runner import build_layer, run_layer
    print(f"[gpu] {wl.name} B={wl.batch} S={wl.seq} d={wl.dim} N={wl.num_query_experts} "
          f"G={wl.num_kv_heads} k={wl.top_k} dh={wl.dh} {wl.dtype} {wl.variant}", flush=True)
    layer, x, inp = build_layer(wl, inputs)
    gpu = run_layer(layer, x)
    rep = parity.compare(wl, gpu, inp, rows=rows, want_qo=want_qo)
    return layer, x, inp, gpu, rep


def _small(name, d=768, N=16, G=8, k=1, dh=48, B=2, S=200, **kw):
    return Workload(name, d, N, G, k, dh, B, S, **kw)


SMALL = [
    WORKLOADS["tiny_fp32"],
    _small("main_ragged", B=2, S=200),
    _small("main_one_tile", B=1, S=64),
    _small("main_short", B=3, S=17),
    _small("main_single_pos", B=4, S=1),
    _small("k2_skew_ragged", d=1024, k=2, dh=64, B=1, S=333,
           router_std=2.70 / 32.0, router_bias_first=2.0),
    _small("weighted_ragged", B=1, S=130, variant="weighted_concat", seed=1),
    _small("hard_ragged", B=1, S=130, variant="hard_concat", seed=1),
    _small("no_shared", B=2, S=96, shared_head=False, seed=2),
    _small("shared_group3", B=1, S=160, shared_kv_group=3, seed=3),
    _small("n4_k2", N=16, G=4, k=2, dh=64, d=512, B=1, S=150, seed=4),
    _small("dh32_f32", d=64, N=4, G=2, k=1, dh=32, B=1, S=70, dtype="f32", router_std=0.3),
    _small("gqa_small", B=2, S=150, k=2, variant="hard_concat", shared_head=False,
           dense_gqa=True),
    _small("dh32_bf16_k2", d=256, N=8, G=4, k=2, dh=32, B=1, S=150, seed=5),
    _small("dh32_weighted", d=384, N=8, G=4, k=1, dh=32, B=2, S=77, variant="weighted_concat", seed=6),
    _small("n1_groups_hard", d=512, N=8, G=8, k=1, dh=64, B=1, S=140, variant="hard_concat", seed=7),
    _small("weighted_k2", d=512, N=16, G=4, k=2, dh=48, B=1, S=129, variant="weighted_concat", seed=8),
    # several hundred positions: many key tiles per attention item, every token checked
    _small("long_s1000", B=1, S=1000, seed=9),
    _small("long_k2_dh64", d=1024, k=2, dh=64, B=1, S=700, seed=10),
    _small("long_dh32_k2", d=256, N=8, G=4, k=2, dh=32, B=2, S=900, seed=11),
    _small("long_gqa", B=1, S=800, k=2, variant="hard_concat", shared_head=False, dense_gqa=True, seed=12),
    # routing skewed toward local expert 0 (about 85 % and 76 % of the tokens) and a ragged last
    # tile: the projection's routed and dense waves multiply every row-block count from 1 to 8
    _small("skew_k1_partial_tile", B=2, S=242, router_bias_first=1.5, seed=14),
    _small("skew_k1_dh32", d=256, N=8, G=4, k=1, dh=32, B=1, S=300, router_bias_first=1.0, seed=15),
    # bf16 with a hidden size that is not a multiple of 64: scalar projection and combine, matrix-core
    # attention on a schedule built by its own kernel
    _small("bf16_d96_scalar_proj", d=96, N=8, G=4, k=1, dh=32, B=2, S=700, seed=13),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_every_token_and_stage(wl):
    layer, x, inp, gpu, rep = _run(wl, want_qo=True)
    inter = layer.intermediates(wl.batch, wl.seq)
    B, S, G, dh, H = wl.batch, wl.seq, wl.num_kv_heads, wl.dh, inter["q"].shape[1]
    K = rep["K"].reshape(B, S, G, dh).transpose(0, 2, 1, 3)
    V = rep["V"].reshape(B, S, G, dh).transpose(0, 2, 1, 3)
    kg = inter["k"].float().cpu().numpy()[:, :, :S]
    from sparse_moe_query_amd.gqe import vt_unpermute
    vg = vt_unpermute(inter["vt"]).float().cpu().numpy()[:, :, :, :S].transpose(0, 1, 3, 2)
    assert parity.within_rounding(kg, K, wl.dtype), parity.rel_err_rows(kg, K)
    assert parity.within_rounding(vg, V, wl.dtype), parity.rel_err_rows(vg, V)
    # Q_act is stored pre-scaled by log2(e)/sqrt(d_h) (the attention works in log2 units)
    qscale = np.float32(1.4426950408889634 / np.sqrt(dh))
    qg = inter["q"].float().cpu().numpy().transpose(0, 2, 1, 3).reshape(B * S, H, dh) / qscale
    og = inter["o"].float().cpu().numpy().reshape(B * S, H, dh)
    assert parity.within_rounding(qg, rep["q_ref"], wl.dtype), parity.rel_err_rows(qg, rep["q_ref"])
    assert parity.rel_err_rows(og, rep["o_ref"], parity.Y_STORAGE_U[wl.dtype]) <= (1e-4 if wl.dtype == "f32" else 2e-2)
    print(f"[gpu] {wl.name}: y_err={rep['y_err']:.2e} (global {rep['y_err_global']:.2e}) "
          f"near_ties={rep['near_ties']}", flush=True)


def test_router_ties_take_lower_index():
    """All-equal logits (W_r = 0, b_r = 0): every group picks its lowest local indices."""
    wl = _small("ties", B=1, S=100, k=1)
    inp = make_inputs(wl)
    inp["w_router"][:] = 0
    inp["b_router"][:] = 0
    _, _, _, gpu, _ = _run(wl, inputs=inp)
    assert np.all(gpu["idx"][:, :, 0] == np.arange(8) * 2)
    assert np.all(gpu["w"] == 1.0)


def test_deterministic_reruns():
    from sparse_moe_query_amd.runner import build_layer, run_layer
    wl = _small("determinism", B=2, S=257)
    layer, x, _ = build_layer(wl)
    a = run_layer(layer, x)
    b = run_layer(layer, x)
    np.testing.assert_array_equal(a["y"], b["y"])
    np.testing.assert_array_equal(a["idx"], b["idx"])
    np.testing.assert_array_equal(a["counts"], b["counts"])
    np.testing.assert_array_equal(a["mean_prob"], b["mean_prob"])


@pytest.mark.parametrize("wl", [_small("knt_s128", B=2, S=128), _small("knt_s320", B=3, S=320, seed=2),
                                _small("knt_ragged", B=2, S=200, seed=3)], ids=lambda w: w.name)
def test_key_norm_tile_maxima(wl):
    """The attention's range test reads the largest key norm of every 64-key tile: it must be
    the maximum of that tile's key norms (bit-exact: the square root is monotone and correctly
    rounded), and each key norm the norm of the stored-before-rounding key within float32."""
    from sparse_moe_query_amd.runner import build_layer, run_layer
    layer, x, _ = build_layer(wl)
    run_layer(layer, x)
    inter = layer.intermediates(wl.batch, wl.seq)
    kn = inter["kn"].cpu().numpy()[:, :, :wl.seq]
    knt = inter["knt"].cpu().numpy()
    S = wl.seq
    for j in range(knt.shape[2]):
        ref = kn[:, :, 64 * j:min(64 * (j + 1), S)].max(axis=2)
        np.testing.assert_array_equal(knt[:, :, j], ref)
    kg = inter["k"].float().cpu().numpy()[:, :, :S]
    np.testing.assert_allclose(kn, np.sqrt((kg.astype(np.float64) ** 2).sum(-1)), rtol=2e-2)
    layer.close()


def test_abi_errors_on_device():
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.runner import build_layer
    wl = _small("errors", B=1, S=64)
    layer, x, _ = build_layer(wl)
    y = torch.empty_like(x)
    small = torch.empty(128, dtype=torch.uint8, device=x.device)
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_forward(layer.h, x, y, 1, 64, small)
    assert e.value.code == -5
    ws = layer.workspace(1, 64)
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_forward(layer.h, x, x, 1, 64, ws)
    assert e.value.code == -1
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_forward(layer.h, x, y, 0, 64, ws)
    assert e.value.code == -6


BUCKET = [_small("bucket_main_ragged", B=2, S=200), _small("bucket_k2", d=1024, k=2, dh=64, B=1, S=333,
                                                              router_std=2.70 / 32.0, router_bias_first=2.0),
          _small("bucket_n4_k2", N=16, G=4, k=2, dh=64, d=512, B=1, S=150, seed=4),
          _small("bucket_n1", d=512, N=8, G=8, k=1, dh=64, B=1, S=70, variant="hard_concat", seed=7),
          WORKLOADS["main_b8_s2048"], WORKLOADS["k2_skew_b4_s4096"]]


@pytest.mark.parametrize("wl", BUCKET, ids=[w.name for w in BUCKET])
def test_bucket_bit_exact(wl):
    """Global bucketing of the forward's routing = the oracle's stable counting sort of the same
    decisions (integer result: bit-exact), on small ragged and full-size workloads."""
    from oracle import gqe_oracle as go
    from sparse_moe_query_amd.runner import build_layer, run_layer
    print(f"[gpu] bucket {wl.name} B={wl.batch} S={wl.seq} N={wl.num_query_experts} G={wl.num_kv_heads} "
          f"k={wl.top_k}", flush=True)
    layer, x, _ = build_layer(wl)
    run_layer(layer, x)
    b = layer.bucket(wl.batch, wl.seq)
    torch.cuda.synchronize()
    idx = layer.intermediates(wl.batch, wl.seq)["idx"].cpu().numpy()
    ref = go.bucket(parity.oracle_cfg(wl), idx)
    assert np.array_equal(b["offs"].cpu().numpy().astype(np.int64), ref["offs"])
    assert np.array_equal(b["perm"].cpu().numpy().astype(np.int64), ref["perm"])
    assert np.array_equal(b["inv"].cpu().numpy().astype(np.int64), ref["inv"])
    layer.close()


def test_bucket_errors():
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.runner import build_layer, run_layer
    wl = _small("bucket_errors", B=1, S=64)
    layer, x, _ = build_layer(wl)
    with pytest.raises(gqe.GqeError) as e:
        layer.bucket(1, 64)
    assert e.value.code == -8  # no forward yet
    run_layer(layer, x)
    t = torch.empty(4, dtype=torch.int32, device=x.device)
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_bucket(layer.h, t, torch.empty(0), t)
    assert e.value.code == -2  # empty tensor -> NULL pointer
    layer.close()
    g = gqa_of(_small("bucket_gqa", B=1, S=64, k=2, variant="hard_concat", shared_head=False))
    layer, x, _ = build_layer(g)
    run_layer(layer, x)
    with pytest.raises(gqe.GqeError) as e:
        layer.bucket(1, 64)
    assert e.value.code == -8  # dense GQA has no routing
    layer.close()


FULL = [WORKLOADS[k] for k in ("main_b8_s2048", "long_s16384", "long_s32768",
                               "k2_skew_b4_s4096", "ablation_gqe_b2_s8192",
                               "ablation_weighted_b2_s8192", "ablation_hard_b2_s8192")]
FULL.append(gqa_of(WORKLOADS["long_s16384"]))


@pytest.mark.parametrize("wl", FULL, ids=[w.name for w in FULL])
def test_full_size_sampled(wl):
    rows = parity.sample_rows(wl.batch, wl.seq)
    _, _, _, gpu, rep = _run(wl, rows=rows)
    print(f"[gpu] {wl.name}: y_err={rep['y_err']:.2e} on {rep['rows']} rows, "
          f"near_ties={rep['near_ties']}, top1 share of local expert 0="
          f"{rep.get('top1_share_local0', float('nan')):.3f}", flush=True)
    sys.stdout.flush()


ROPE = [
    _small("rope_main_ragged", B=2, S=200, rope_base=10000.0, seed=20),
    _small("rope_k2_dh64", d=1024, k=2, dh=64, B=1, S=333, rope_base=10000.0, seed=21,
           router_std=2.70 / 32.0, router_bias_first=2.0),
    _small("rope_dh32_weighted", d=384, N=8, G=4, k=1, dh=32, B=2, S=130, variant="weighted_concat",
           rope_base=500.0, seed=22),
    _small("rope_f32_scalar", d=64, N=4, G=2, k=1, dh=16, B=1, S=70, dtype="f32", router_std=0.3,
           rope_base=10000.0, seed=23),
    _small("rope_gqa", B=1, S=150, k=2, variant="hard_concat", shared_head=False, dense_gqa=True,
           rope_base=10000.0, seed=24),
    # long positions: angles of thousands of radians per pair
    _small("rope_long_s3000", B=1, S=3000, rope_base=10000.0, seed=25),
]


@pytest.mark.parametrize("wl", ROPE, ids=[w.name for w in ROPE])
def test_rope_parity(wl):
    """Optional rotary position embedding: every token against the oracle (rotation in float64)."""
    rows = None if wl.tokens <= 1000 else parity.sample_rows(wl.batch, wl.seq, n=96, seed=3)
    _run(wl, rows=rows)


# Peaked attention: query and key projections with std 0.2 (ten times the default) put
# max|q| * max|k| far above the range where the kernel may skip the running maximum (64 in log2
# units), so every key tile takes the online-softmax step; a ramp that scales x up along the
# sequence makes the scores grow along the keys, so the running maximum keeps rising by more than
# the lazy threshold (2^8) and the accumulators are rescaled.  Shapes where the schedule splits
# items, so the merge combines chunks with non-zero offsets.  Every token is checked.
PEAKED = [
    _small("peaked_dh48_k1", B=1, S=1000, qk_std=0.2, seed=30),
    _small("peaked_dh48_k1_ramp", B=1, S=1000, qk_std=0.2, x_ramp=3.0, seed=31),
    _small("peaked_dh48_k2", d=512, N=16, G=4, k=2, dh=48, B=1, S=1000, qk_std=0.2, x_ramp=1.0, seed=32),
    _small("peaked_dh32_k2", d=256, N=8, G=4, k=2, dh=32, B=1, S=1000, qk_std=0.3, seed=33),
    _small("peaked_dh32_k1_ramp", d=384, N=8, G=4, k=1, dh=32, B=1, S=1000, qk_std=0.2, x_ramp=3.0, seed=34),
    _small("peaked_dh64_k2_ramp", d=1024, k=2, dh=64, B=1, S=1000, qk_std=0.2, x_ramp=3.0, seed=35),
    _small("peaked_dh64_k1", d=1024, k=1, dh=64, B=1, S=1000, qk_std=0.2, seed=36),
]

FAST_BOUND = 64.0   # log2 units: the kernel skips the running maximum only below this bound


@pytest.mark.parametrize("wl", PEAKED, ids=[w.name for w in PEAKED])
def test_online_softmax_branch(wl):
    """Scores this peaked make the output ill-conditioned in bf16: rounding q and k once to bf16
    (the layer's storage precision, 2^-9 relative) moves a score by up to |q| |k| 2^-8, about one
    unit of log2 here, which re-weights the softmax by tens of percent.  So the stages are
    checked one by one: Q, K, V against the oracle within one rounding, the attention output
    against float64 softmax attention over the kernel's own stored bf16 Q, K, V (the check of
    the online-softmax branch), routing and statistics exactly; the end-to-end output error is
    recorded, not held to the bar."""
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.gqe import vt_unpermute
    from sparse_moe_query_amd.runner import build_layer, run_layer
    print(f"[gpu] {wl.name} B={wl.batch} S={wl.seq} d={wl.dim} N={wl.num_query_experts} "
          f"G={wl.num_kv_heads} k={wl.top_k} dh={wl.dh} qk_std={wl.qk_std} x_ramp={wl.x_ramp}", flush=True)
    layer, x, inp = build_layer(wl)
    gpu = run_layer(layer, x)
    rep = parity.compare(wl, gpu, inp, want_qo=True, check_y=False)
    B, S, dh, G = wl.batch, wl.seq, wl.dh, wl.num_kv_heads
    jobs, merges, nslots, chunk = gqe.gqe_attention_schedule(layer.h, B, S)
    assert chunk > 0 and len(merges) > 0, "the shape must split attention items"
    inter = layer.intermediates(B, S)
    q = inter["q"].float().cpu().numpy().astype(np.float64)          # [B, H, S, dh], log2 units
    knt = inter["knt"].cpu().numpy().astype(np.float64)[:, :, :(S + 63) // 64]
    qn = np.sqrt((q ** 2).sum(-1))
    # every query norm times every tile's largest key norm exceeds the bound: no tile of any wave
    # can take the fast path (the kernel's per-wave query bound is at least the largest norm)
    assert qn.min() * knt.min() > FAST_BOUND, (qn.min(), knt.min())
    H = q.shape[1]
    # stored Q, K, V = the exact values rounded once
    qscale = np.float32(1.4426950408889634 / np.sqrt(dh))
    qg = q.transpose(0, 2, 1, 3).reshape(B * S, H, dh) / qscale
    assert parity.within_rounding(qg, rep["q_ref"], wl.dtype)
    kg = inter["k"].float().cpu().numpy().astype(np.float64)
    vg = vt_unpermute(inter["vt"]).float().cpu().numpy().astype(np.float64).transpose(0, 1, 3, 2)
    Kx = rep["K"].reshape(B, S, G, dh).transpose(0, 2, 1, 3)
    Vx = rep["V"].reshape(B, S, G, dh).transpose(0, 2, 1, 3)
    assert parity.within_rounding(kg[:, :, :S], Kx, wl.dtype)
    assert parity.within_rounding(vg[:, :, :S], Vx, wl.dtype)
    # the attention output against float64 attention over the stored operands: the kernel's own
    # roundings are P to bf16 (2^-9 relative, the same P forms the row sums) and O to bf16
    og = inter["o"].float().cpu().numpy().astype(np.float64).reshape(B, S, H, dh)
    oref = parity.attention_from_stored(q, kg, vg, G, wl.top_k, wl.shared_kv_group, S)
    o_err = parity.rel_err_rows(og, oref, parity.Y_STORAGE_U[wl.dtype])
    parity.record(dict(kind="attention_stage", workload=wl.name, o_err=o_err, o_err_raw=parity.rel_err_rows(og, oref),
                       bar=1e-2))
    assert o_err <= 1e-2, f"attention output {o_err:.3e} x row RMS from float64 attention over the stored operands"
    if wl.x_ramp:
        # scores of late queries rise along the keys by more than the lazy threshold (2^8)
        k = inter["k"].float().cpu().numpy().astype(np.float64)[0, 0, :S]   # group 0, batch 0
        rises = 0
        for pos in (S - 1, S // 2, S - 200):
            s = k[:pos + 1] @ q[0, 0, pos]
            tiles = [s[i:i + 64].max() for i in range(0, pos + 1, 64)]
            rises += int(np.max(np.maximum.accumulate(tiles)) - tiles[0] > 8.0)
        assert rises > 0
    print(f"[gpu] {wl.name}: attention stage {o_err:.2e}; end to end y_err={rep['y_err']:.2e} "
          f"raw {rep['y_err_raw']:.2e} (recorded); chunk cap {chunk}, "
          f"{len(merges)} merged items, min|q|*min knt = {qn.min() * knt.min():.1f}", flush=True)
    layer.close()
