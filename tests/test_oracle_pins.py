"""Pins for the CPU oracle: facts fixed by the pages and by mathematics, checked without a GPU.

Each test names the passage or the mathematical fact it rests on.  Chosen so that a dropped
term, a wrong sign or index, a transposed operand or a wrong tie rule anywhere in the oracle
fails at least one of them:

* router   -- numpy matmul + scipy softmax (library routines), brute force over k-subsets,
              the all-equal-logits tie case, k=1 => w=1, sum w = 1;
* aux      -- closed forms (k = n => 1, collapse => n, uniform p => 1), count totals;
* bucketing-- numpy's stable argsort of the expert ids (brute force), bucket sizes = counts,
              perm o inv = identity, tokens ascending in every bucket, k = n => every bucket is
              0..T-1;
* attention-- S=1 => o = v_0; W_k = 0 => causal running mean of V;
* layer    -- k = N/G + hard concat + no shared head is textbook GQA: torch's
              scaled_dot_product_attention (float64); label permutations of experts and groups;
              identical experts; the variant relations; locality and causality;
              and agreement with an independently written numpy brute force.
"""
import json
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import bruteforce
from oracle import gqe_oracle as go
from sparse_moe_query_amd.inputs import Workload, make_inputs, round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _wl(d=32, N=4, G=2, k=1, dh=8, B=2, S=9, seed=0, variant="gqe", shared=True, skv=0,
        rstd=None, bias=0.0):
    return Workload("pin", d, N, G, k, dh, B, S, dtype="f32", variant=variant,
                    shared_head=shared, shared_kv_group=skv, seed=seed, router_std=rstd,
                    router_bias_first=bias)


def _cfg(wl):
    return go.OracleConfig(wl.dim, wl.num_query_experts, wl.num_kv_heads, wl.top_k, wl.dh,
                           wl.variant, wl.shared_head, wl.shared_kv_group)


def _fwd(wl, w=None, **kw):
    w = make_inputs(wl) if w is None else w
    return go.forward(_cfg(wl), wl.batch, wl.seq, w["x"], w, **kw), w


# ----------------------------------------------------------------------------- golden
def test_head_accounting_golden():
    """README 'Algorithm Overview': N=16, G=8, k=1 computes 9 of 16 query heads."""
    with open(os.path.join(GOLDEN, "head_accounting.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        cfg = go.OracleConfig(768, c["num_query_experts"], c["num_kv_heads"], c["top_k"],
                              None, "gqe", c["shared_head"])
        T = 5
        N = c["num_query_experts"]
        rng = np.random.default_rng(0)
        r = go.router(cfg, rng.standard_normal((T, 768)), rng.standard_normal((768, N)) / 28)
        st = go.aux(cfg, r["p"], r["idx"])
        assert st["active_heads"] == c["active_heads"]
        assert r["idx"].shape[1] * r["idx"].shape[2] == c["routed_active"]
        assert cfg.dh == 768 // 16  # README 'Parameters': head_dim defaults to dim // N


def test_moe_properties_golden():
    """Tutorial 'Mixture of experts': exactly top_k distinct experts, weights sum to 1."""
    with open(os.path.join(GOLDEN, "moe_properties.json")) as f:
        props = json.load(f)
    for k, N, G in ((1, 4, 2), (2, 8, 2), (3, 12, 3)):
        wl = _wl(d=24, N=N, G=G, k=k, S=11, rstd=0.5)
        w = make_inputs(wl)
        cfg = _cfg(wl)
        r = go.router(cfg, w["x"], w["w_router"], w["b_router"])
        n = N // G
        for g in range(G):
            sel = r["idx"][:, g, :]
            assert props["exactly_k_distinct_per_group"]
            assert all(len(set(row)) == k for row in sel.tolist())
            assert np.all((sel >= g * n) & (sel < (g + 1) * n))
        np.testing.assert_allclose(r["w"].sum(axis=2), props["renormalised_weights_sum"],
                                   rtol=0, atol=1e-15)


# ----------------------------------------------------------------------------- router
def test_router_logits_and_softmax_match_library():
    """README 'Algorithm Overview': softmax over experts inside each group.  Logits are
    x @ W_r + b_r (tutorial moe_layer), checked with numpy's matmul; p with scipy's softmax."""
    wl = _wl(d=40, N=12, G=3, k=2, S=13, rstd=0.3, bias=0.7)
    w = make_inputs(wl)
    r = go.router(_cfg(wl), w["x"], w["w_router"], w["b_router"])
    x = w["x"].reshape(-1, wl.dim).astype(np.float64)
    ref_l = x @ w["w_router"].astype(np.float64) + w["b_router"].astype(np.float64)
    np.testing.assert_allclose(r["logits"], ref_l, rtol=1e-13, atol=1e-13)
    ref_p = scipy.special.softmax(ref_l.reshape(-1, 3, 4), axis=2).reshape(-1, 12)
    np.testing.assert_allclose(r["p"], ref_p, rtol=1e-12, atol=1e-15)


def test_router_topk_bruteforce_subsets():
    """Top-k = the k-subset with the largest total logit (unique for continuous draws);
    the rank order inside the selection is descending logit."""
    import itertools
    wl = _wl(d=16, N=10, G=2, k=3, S=25, rstd=1.0)
    w = make_inputs(wl)
    r = go.router(_cfg(wl), w["x"], w["w_router"], w["b_router"])
    n = 5
    for t in range(r["logits"].shape[0]):
        for g in range(2):
            lg = r["logits"][t, g * n:(g + 1) * n]
            best = max(itertools.combinations(range(n), 3), key=lambda s: sum(lg[list(s)]))
            got = r["idx"][t, g] - g * n
            assert sorted(got.tolist()) == sorted(best)
            assert np.all(np.diff(lg[got]) < 0)
            rest = sorted(set(range(n)) - set(best))
            assert r["gap"][t, g] == pytest.approx(lg[got[-1]] - max(lg[rest]), abs=1e-15)


def test_router_all_equal_logits_tie_break():
    """Equal logits: the lower local index wins, p = 1/n, w = 1/k, gap = 0."""
    wl = _wl(d=16, N=12, G=3, k=2, S=7)
    w = make_inputs(wl)
    w["w_router"][:] = 0
    w["b_router"][:] = 0
    r = go.router(_cfg(wl), w["x"], w["w_router"], w["b_router"])
    n = 4
    for g in range(3):
        assert np.all(r["idx"][:, g, 0] == g * n) and np.all(r["idx"][:, g, 1] == g * n + 1)
    assert np.all(r["p"] == 0.25) and np.all(r["w"] == 0.5) and np.all(r["gap"] == 0)


def test_router_k1_weight_is_one_and_k_eq_n_gap_inf():
    wl = _wl(d=16, N=8, G=4, k=1, S=9, rstd=1.0)
    w = make_inputs(wl)
    r = go.router(_cfg(wl), w["x"], w["w_router"], w["b_router"])
    assert np.all(r["w"] == 1.0)
    wl2 = wl.with_(top_k=2)
    r2 = go.router(_cfg(wl2), w["x"], w["w_router"], w["b_router"])
    assert np.all(np.isinf(r2["gap"]))


# ----------------------------------------------------------------------------- bucketing
@pytest.mark.parametrize("N,G,k,T,seed", [(4, 2, 1, 37, 0), (16, 8, 1, 200, 1), (16, 4, 2, 150, 2),
                                          (8, 8, 1, 20, 3), (32, 8, 3, 64, 4)])
def test_bucket_is_stable_sort_by_expert(N, G, k, T, seed):
    """Bucketing = stable sort of the (t, g, r) assignments by expert id: compared with numpy's
    stable argsort (brute force); sizes equal the per-expert counts; perm o inv = identity;
    tokens strictly ascending inside every bucket."""
    rng = np.random.default_rng(seed)
    n = N // G
    idx = np.zeros((T, G, k), np.int32)
    for t in range(T):
        for g in range(G):
            idx[t, g] = g * n + rng.permutation(n)[:k]
    cfg = go.OracleConfig(64, N, G, k, 16)
    b = go.bucket(cfg, idx)
    flat = idx.reshape(-1)
    order = np.argsort(flat, kind="stable")
    assert np.array_equal(b["perm"], order // (G * k))
    pos = np.empty_like(order)
    pos[order] = np.arange(order.size)
    assert np.array_equal(b["inv"].reshape(-1), pos)
    counts = np.bincount(flat, minlength=N)
    assert np.array_equal(np.diff(b["offs"]), counts) and b["offs"][0] == 0
    assert np.array_equal(b["perm"][b["inv"].reshape(-1)], np.repeat(np.arange(T), G * k))
    for e in range(N):
        seg = b["perm"][b["offs"][e]:b["offs"][e + 1]]
        assert np.all(np.diff(seg) > 0)


def test_bucket_all_experts_chosen_is_identity_per_bucket():
    """k = n: every expert receives every token, so each bucket is 0..T-1 in order."""
    N, G, T = 8, 4, 33
    n = N // G
    idx = np.zeros((T, G, n), np.int32)
    for g in range(G):
        idx[:, g, :] = g * n + np.arange(n)[::-1]   # rank order does not matter to the buckets
    b = go.bucket(go.OracleConfig(64, N, G, n, 16), idx)
    assert np.array_equal(b["offs"], np.arange(N + 1) * T)
    assert np.array_equal(b["perm"], np.tile(np.arange(T), N))


# ----------------------------------------------------------------------------- aux
def test_aux_closed_forms():
    """Switch-style balance loss (README 'Algorithm Overview'): n * sum_e f_e P_e per group,
    averaged.  k = n -> exactly 1; all tokens to one expert with p = 1 -> n; uniform p with
    every token on one expert -> 1; per-group counts sum to T*k."""
    wl = _wl(d=16, N=8, G=2, k=4, S=17, rstd=1.0)
    w = make_inputs(wl)
    cfg = _cfg(wl)
    r = go.router(cfg, w["x"], w["w_router"], w["b_router"])
    st = go.aux(cfg, r["p"], r["idx"])
    assert st["aux"] == pytest.approx(1.0, abs=1e-13)
    T = wl.tokens
    assert np.all(st["counts"] == T)

    wl1 = wl.with_(top_k=1)
    cfg1 = _cfg(wl1)
    b = np.zeros(8, np.float32)
    b[::4] = 1000.0
    r = go.router(cfg1, w["x"], w["w_router"], b)
    st = go.aux(cfg1, r["p"], r["idx"])
    assert st["aux"] == pytest.approx(4.0, abs=1e-13)
    assert st["counts"].tolist() == [T, 0, 0, 0, T, 0, 0, 0]

    r = go.router(cfg1, w["x"], np.zeros_like(w["w_router"]), None)
    st = go.aux(cfg1, r["p"], r["idx"])
    assert st["aux"] == pytest.approx(1.0, abs=1e-13)
    np.testing.assert_allclose(st["mean_prob"], 0.25, rtol=1e-15)

    wl3 = _wl(d=16, N=12, G=3, k=2, S=23, rstd=1.0)
    w3 = make_inputs(wl3)
    cfg3 = _cfg(wl3)
    r = go.router(cfg3, w3["x"], w3["w_router"], None)
    st = go.aux(cfg3, r["p"], r["idx"])
    assert st["counts"].reshape(3, 4).sum(axis=1).tolist() == [wl3.tokens * 2] * 3
    np.testing.assert_allclose(st["mean_prob"], r["p"].mean(axis=0), rtol=1e-14)


# ----------------------------------------------------------------------------- attention
def test_attention_single_position_returns_v0():
    """Causal attention over one key returns that key's value exactly."""
    wl = _wl(d=24, N=4, G=2, k=1, dh=8, B=3, S=1, rstd=1.0)
    out, w = _fwd(wl, want_qo=True)
    V = out["V"].reshape(3, 1, 2, 8)
    for b in range(3):
        for v in range(3):
            g = out["idx_used"][b, v] // 2 if v < 2 else 0
            g = v if v < 2 else 0
            np.testing.assert_allclose(out["o"][b, v], V[b, 0, g], rtol=0, atol=1e-15)


def test_attention_zero_keys_is_causal_running_mean():
    """W_k = 0 makes every score 0, so o_t is the mean of v_0..v_t."""
    wl = _wl(d=24, N=4, G=2, k=1, dh=8, B=2, S=12, rstd=1.0)
    w = make_inputs(wl)
    w["w_k"][:] = 0
    out, _ = _fwd(wl, w, want_qo=True)
    V = out["V"].reshape(2, 12, 2, 8)
    mean = np.cumsum(V, axis=1) / np.arange(1, 13)[None, :, None, None]
    o = out["o"].reshape(2, 12, 3, 8)
    for v, g in ((0, 0), (1, 1), (2, 0)):
        np.testing.assert_allclose(o[:, :, v], mean[:, :, g], rtol=0, atol=1e-14)


# ----------------------------------------------------------------------------- layer
def _gqa_sdpa(wl, w):
    """Textbook GQA (tutorial 'Multi-head, multi-query and grouped-query attention'):
    N query heads, G shared KV heads, concat then output projection -- via torch."""
    B, S, d, N, G, dh = wl.batch, wl.seq, wl.dim, wl.num_query_experts, wl.num_kv_heads, wl.dh
    x = torch.tensor(w["x"], dtype=torch.float64).reshape(B, S, d)
    Wq = torch.tensor(w["w_q"], dtype=torch.float64)
    q = torch.stack([x @ Wq[e] for e in range(N)], dim=1)                      # [B,N,S,dh]
    k = (x @ torch.tensor(w["w_k"], dtype=torch.float64)).reshape(B, S, G, dh).transpose(1, 2)
    v = (x @ torch.tensor(w["w_v"], dtype=torch.float64)).reshape(B, S, G, dh).transpose(1, 2)
    k = k.repeat_interleave(N // G, dim=1)
    v = v.repeat_interleave(N // G, dim=1)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
    Wo = torch.tensor(w["w_o"], dtype=torch.float64).reshape(N * dh, d)
    return (o.transpose(1, 2).reshape(B * S, N * dh) @ Wo).numpy()


@pytest.mark.parametrize("N,G,dh", [(4, 2, 8), (6, 3, 4), (8, 2, 16)])
def test_k_equals_n_hard_concat_is_gqa(N, G, dh):
    """k = N/G with plain concatenation and no shared head reduces to GQA."""
    wl = _wl(d=32, N=N, G=G, k=N // G, dh=dh, B=2, S=10, variant="hard_concat", shared=False,
             rstd=1.0)
    out, w = _fwd(wl)
    np.testing.assert_allclose(out["y"], _gqa_sdpa(wl, w), rtol=1e-10, atol=1e-12)


def test_gqe_with_zero_extra_projections_is_gqa():
    """With W_oR = 0 and W_os = 0 the 'gqe' variant at k = N/G is again GQA."""
    wl = _wl(d=32, N=4, G=2, k=2, dh=8, B=2, S=10, variant="gqe", shared=True, rstd=1.0)
    w = make_inputs(wl)
    w["w_o_rslot"][:] = 0
    w["w_o_shared"][:] = 0
    out, _ = _fwd(wl, w)
    np.testing.assert_allclose(out["y"], _gqa_sdpa(wl, w), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("variant,k", [("gqe", 1), ("gqe", 2), ("weighted_concat", 2),
                                       ("hard_concat", 1)])
def test_expert_label_permutation(variant, k):
    """Relabelling the experts inside each group (router columns, biases, W_q, W_o together)
    leaves y unchanged and maps the selected ids by the same permutation."""
    wl = _wl(d=32, N=8, G=2, k=k, dh=8, B=2, S=9, variant=variant, rstd=1.0, bias=0.3)
    out, w = _fwd(wl)
    rng = np.random.default_rng(5)
    perm = np.concatenate([g * 4 + rng.permutation(4) for g in range(2)])
    w2 = dict(w)
    w2["w_router"] = w["w_router"][:, perm]
    w2["b_router"] = w["b_router"][perm]
    w2["w_q"] = w["w_q"][perm]
    w2["w_o"] = w["w_o"][perm]
    out2, _ = _fwd(wl, w2)
    np.testing.assert_allclose(out2["y"], out["y"], rtol=1e-12, atol=1e-13)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(np.sort(perm[out2["idx"]], axis=2),
                                  np.sort(out["idx"], axis=2))
    assert inv.shape == perm.shape


def test_group_permutation_moves_shared_group():
    """Relabelling the GQA groups (router column blocks, W_q blocks, K/V heads, W_o blocks,
    W_oR) with the shared head's KV group moved along leaves y unchanged."""
    N, G, dh, n = 6, 3, 8, 2
    wl = _wl(d=32, N=N, G=G, k=1, dh=dh, B=2, S=9, rstd=1.0, bias=0.2, skv=1)
    out, w = _fwd(wl)
    gp = np.array([2, 0, 1])
    eperm = np.concatenate([np.arange(g * n, (g + 1) * n) for g in gp])
    cperm = np.concatenate([np.arange(g * dh, (g + 1) * dh) for g in gp])
    w2 = dict(w)
    w2["w_router"] = w["w_router"][:, eperm]
    w2["b_router"] = w["b_router"][eperm]
    w2["w_q"] = w["w_q"][eperm]
    w2["w_o"] = w["w_o"][eperm]
    w2["w_k"] = w["w_k"][:, cperm]
    w2["w_v"] = w["w_v"][:, cperm]
    w2["w_o_rslot"] = w["w_o_rslot"][gp]
    new_skv = int(np.where(gp == 1)[0][0])
    out2, _ = _fwd(wl.with_(shared_kv_group=new_skv), w2)
    np.testing.assert_allclose(out2["y"], out["y"], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("variant", ["gqe", "hard_concat"])
def test_identical_experts_equal_single_expert(variant):
    """Tutorial 'Mixture of experts': with identical experts the layer equals a single
    expert -- so y does not depend on which expert the router picks."""
    wl = _wl(d=32, N=8, G=2, k=1, dh=8, B=2, S=9, variant=variant, rstd=1.0)
    w = make_inputs(wl)
    for g in range(2):
        w["w_q"][g * 4:(g + 1) * 4] = w["w_q"][g * 4]
        w["w_o"][g * 4:(g + 1) * 4] = w["w_o"][g * 4]
    out, _ = _fwd(wl, w)
    w2 = dict(w)
    w2["w_router"] = np.random.default_rng(9).standard_normal(w["w_router"].shape).astype(
        np.float32)
    out2, _ = _fwd(wl, w2)
    assert np.any(out2["idx"] != out["idx"])
    np.testing.assert_allclose(out2["y"], out["y"], rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("k", [2, 3])
def test_identical_experts_renormalised_slot_at_k_above_one(k):
    """Tutorial 'Mixture of experts' (identical experts make the mixture one expert) at k >= 2,
    variant gqe, n = 4 > k: every chosen expert of a group then gives the same head output o, so
    the hard-concat part is k o W_o[g] and the renormalised slot is (sum_r w_r) o W_oR[g] = o W_oR[g]
    -- the layer must equal the k = 1 layer whose expert projection is k W_o[g], whatever the
    routing.  A slot weighted by the raw probabilities (their sum is below 1 when k < n), by 1 per
    choice, or by any weights not summing to one fails this."""
    wl = _wl(d=32, N=8, G=2, k=k, dh=8, B=2, S=9, variant="gqe", rstd=0.1, seed=3)
    w = make_inputs(wl)
    for g in range(2):
        w["w_q"][g * 4:(g + 1) * 4] = w["w_q"][g * 4]
        w["w_o"][g * 4:(g + 1) * 4] = w["w_o"][g * 4]
    out, _ = _fwd(wl, w)
    p_sel = np.take_along_axis(out["p"].reshape(wl.tokens, 2, 4), out["idx"] % 4, axis=2).sum(axis=2)
    assert np.mean(p_sel) < 0.95  # raw probabilities of the chosen experts do not sum to one
    w1 = dict(w)
    w1["w_o"] = float(k) * w["w_o"].astype(np.float64)  # exact: no float32 rounding of 3 W_o
    one, _ = _fwd(wl.with_(top_k=1), w1)
    np.testing.assert_allclose(out["y"], one["y"], rtol=1e-11, atol=1e-13)
    w2 = dict(w)
    w2["w_router"] = np.random.default_rng(17).standard_normal(w["w_router"].shape).astype(np.float32)
    out2, _ = _fwd(wl, w2)
    assert np.any(out2["idx"] != out["idx"])
    np.testing.assert_allclose(out2["y"], out["y"], rtol=1e-11, atol=1e-13)


def test_weighted_concat_pairs_each_probability_with_its_expert():
    """README 'Ablations' (weighted_concat: each selected expert's slot scaled by its router
    probability) at k = 2 of n = 4, one position per sequence: every head output is then v_0 of
    its group, so with W_o[e] = c_e M (distinct scalars c_e) the output is
    (sum_r p[e_r] c_{e_r}) v_0 M -- the scalar, recovered from y, checks that each probability is
    paired with its own expert's projection.  The router's p and idx are pinned on their own."""
    wl = _wl(d=32, N=4, G=1, k=2, dh=8, B=7, S=1, variant="weighted_concat", shared=False,
             rstd=0.1, seed=5)
    w = make_inputs(wl)
    c = np.array([1.0, 8.0, 64.0, 512.0], np.float32)  # powers of two: c_e M is exact
    w["w_o"] = c[:, None, None] * w["w_o"][0][None]
    out, _ = _fwd(wl, w)
    base, _ = _fwd(wl.with_(variant="hard_concat", top_k=1, num_query_experts=1),
                   dict(w, w_q=w["w_q"][:1], w_o=w["w_o"][:1], w_router=w["w_router"][:, :1],
                        b_router=w["b_router"][:1]))  # one expert, coefficient 1: v_0 M
    T = wl.tokens
    scal = np.einsum("td,td->t", out["y"], base["y"]) / np.einsum("td,td->t", base["y"], base["y"])
    want = (out["p"][np.arange(T)[:, None], out["idx"][:, 0, :]] * c[out["idx"][:, 0, :]]).sum(axis=1)
    np.testing.assert_allclose(scal, want, rtol=1e-10)


@pytest.mark.parametrize("k,n,G", [(2, 4, 1), (3, 4, 2), (2, 3, 2)])
def test_gqe_slot_is_weighted_mix_divided_by_selected_mass(k, n, G):
    """Explainer 'Output Construction' (renormalised weighted-sum slot) against README
    'Ablations' (weighted_concat): with W_o[e] = W_oR[g] for every expert of group g and no shared
    head, weighted_concat gives sum_g sum_r p_r o_r W_oR[g]; the gqe slot alone (W_o = 0) gives
    sum_g sum_r (p_r / sum_sel p) o_r W_oR[g].  With one group the two differ exactly by the factor
    sum_sel p per token; with several groups, zeroing every W_oR but one isolates each group."""
    N = n * G
    wl = _wl(d=32, N=N, G=G, k=k, dh=8, B=2, S=11, variant="gqe", shared=False, rstd=0.1, seed=7)
    w = make_inputs(wl)
    for gsel in range(G):
        wg = dict(w)
        wg["w_o_rslot"] = w["w_o_rslot"].copy()
        wg["w_o_rslot"][np.arange(G) != gsel] = 0
        wg["w_o"] = np.repeat(wg["w_o_rslot"], n, axis=0)
        yw, _ = _fwd(wl.with_(variant="weighted_concat"), wg)
        wz = dict(wg, w_o=np.zeros_like(wg["w_o"]))
        ys, _ = _fwd(wl, wz)
        T = wl.tokens
        p_sel = yw["p"][np.arange(T)[:, None], yw["idx"][:, gsel, :]].sum(axis=1)
        assert np.mean(p_sel) < 0.95
        np.testing.assert_allclose(ys["y"] * p_sel[:, None], yw["y"], rtol=1e-10, atol=1e-14)


def test_weighted_concat_scales_slot_by_router_probability():
    """README 'Ablations': weighted_concat has no renormalised slot; each selected expert's
    slot is weighted by its router probability.  With one group's projection kept and the
    shared projection zeroed, y_weighted = p_sel * y_hard token by token."""
    wl = _wl(d=32, N=6, G=3, k=1, dh=8, B=2, S=9, rstd=1.0)
    w = make_inputs(wl)
    w["w_o"][2:] = 0          # keep group 0 only
    w["w_o_shared"][:] = 0
    yw, _ = _fwd(wl.with_(variant="weighted_concat"), w)
    yh, _ = _fwd(wl.with_(variant="hard_concat"), w)
    psel = yw["p"][np.arange(wl.tokens), yw["idx"][:, 0, 0]]
    np.testing.assert_allclose(yw["y"], psel[:, None] * yh["y"], rtol=1e-12, atol=1e-14)


def test_gqe_slot_adds_renormalised_mix():
    """Explainer 'Output Construction': gqe = hard concat + renormalised weighted-sum slot.
    At k = 1 the slot is the selected output itself, so W_oR[g] = W_o of group g makes
    the routed part exactly twice the hard-concat one."""
    wl = _wl(d=32, N=6, G=3, k=1, dh=8, B=2, S=9, rstd=1.0)
    w = make_inputs(wl)
    for g in range(3):
        w["w_o"][2 * g + 1] = w["w_o"][2 * g]
        w["w_o_rslot"][g] = w["w_o"][2 * g]
    w["w_o_shared"][:] = 0
    yg, _ = _fwd(wl.with_(variant="gqe"), w)
    yh, _ = _fwd(wl.with_(variant="hard_concat"), w)
    np.testing.assert_allclose(yg["y"], 2 * yh["y"], rtol=1e-12, atol=1e-14)


def test_locality_of_routing():
    """README 'Algorithm Overview': the KV path is dense and unchanged, so the weights of an
    expert that token t did not select cannot change y_t."""
    wl = _wl(d=32, N=8, G=2, k=1, dh=8, B=1, S=12, rstd=1.0)
    out, w = _fwd(wl)
    t = 7
    unused = sorted(set(range(8)) - set(out["idx"][t].ravel().tolist()))[0]
    w2 = dict(w)
    w2["w_q"] = w["w_q"].copy()
    w2["w_o"] = w["w_o"].copy()
    w2["w_q"][unused] += 1.0
    w2["w_o"][unused] -= 1.0
    out2, _ = _fwd(wl, w2)
    np.testing.assert_array_equal(out2["y"][t], out["y"][t])


def test_causality():
    """Causal mask: changing the token at position s0 leaves every earlier output unchanged."""
    wl = _wl(d=32, N=4, G=2, k=1, dh=8, B=1, S=12, rstd=1.0)
    out, w = _fwd(wl)
    w2 = dict(w)
    w2["x"] = w["x"].copy()
    w2["x"][0, 6] += 3.0
    out2, _ = _fwd(wl, w2)
    np.testing.assert_array_equal(out2["y"][:6], out["y"][:6])
    assert np.any(out2["y"][6] != out["y"][6])


@pytest.mark.parametrize("N,G,k,variant,shared,skv", [
    (4, 2, 1, "gqe", True, 0), (8, 2, 2, "gqe", True, 1), (8, 4, 1, "weighted_concat", True, 3),
    (12, 3, 2, "weighted_concat", False, 0), (6, 2, 3, "hard_concat", True, 1),
    (4, 4, 1, "gqe", False, 0)])
def test_c_oracle_matches_numpy_bruteforce(N, G, k, variant, shared, skv):
    wl = _wl(d=24, N=N, G=G, k=k, dh=8, B=2, S=11, variant=variant, shared=shared, skv=skv,
             rstd=0.8, bias=0.4)
    out, w = _fwd(wl, want_qo=True)
    bf = bruteforce.layer(_cfg(wl), wl.batch, wl.seq, w["x"], w)
    np.testing.assert_array_equal(out["idx"], bf["idx"])
    np.testing.assert_allclose(out["p"], bf["p"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(out["w"], bf["w"], rtol=1e-13, atol=1e-15)
    np.testing.assert_allclose(out["y"], bf["y"], rtol=1e-11, atol=1e-13)
    T = wl.tokens
    o_routed = bf["o_all"][np.arange(T)[:, None], out["idx"].reshape(T, G * k)]
    np.testing.assert_allclose(out["o"][:, :G * k], o_routed, rtol=1e-11, atol=1e-13)


def test_bf16_rounding_matches_torch():
    """The generator's fp32 -> bf16 rounding is round-to-nearest-even, as torch's cast."""
    a = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 7
    a[:4] = [1.00390625, 1.01171875, -2.0078125, 3.0]   # exact ties and a representable
    ref = torch.tensor(a).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(round_bf16(a), ref)


def test_inputs_are_seeded_and_ordered():
    wl = _wl(d=16, N=4, G=2, k=1, dh=4, S=5)
    a, b = make_inputs(wl), make_inputs(wl)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    c = make_inputs(wl.with_(variant="hard_concat"))
    np.testing.assert_array_equal(a["w_o_shared"], c["w_o_shared"])


@pytest.mark.parametrize("variant,k,shared", [("gqe", 1, True), ("weighted_concat", 2, True),
                                              ("hard_concat", 2, False)])
def test_decode_is_last_row_of_prefix_bruteforce(variant, k, shared):
    """Decode with a dense KV cache (README "Algorithm Overview", explainer "Dense KV Path"): the
    new token's output equals the last row of the independently written numpy brute force run
    over the sequence's prefix, for ragged positions (0 = empty cache)."""
    wl = _wl(d=24, N=8, G=2, k=k, dh=8, B=3, S=13, variant=variant, shared=shared, rstd=0.9, bias=0.3)
    w = make_inputs(wl)
    pos = [0, 5, 12]
    dec = go.decode(_cfg(wl), w["x"], w, pos)
    for b, p in enumerate(pos):
        bf = bruteforce.layer(_cfg(wl), 1, p + 1, w["x"][b, :p + 1], w)
        np.testing.assert_allclose(dec["y"][b], bf["y"][p], rtol=1e-11, atol=1e-13)
        np.testing.assert_array_equal(dec["idx"][b], bf["idx"][p])


def test_decode_ignores_tokens_after_its_position():
    """Causality seen from the cache: a decode step reads positions 0 .. pos only, so whatever
    follows pos in the history (future tokens, padding) does not change its output."""
    wl = _wl(d=24, N=4, G=2, k=1, dh=8, B=2, S=10, rstd=1.0)
    w = make_inputs(wl)
    pos = [3, 9]
    ref = go.decode(_cfg(wl), w["x"], w, pos)["y"]
    x2 = w["x"].copy()
    x2[0, 4:] = 100.0
    got = go.decode(_cfg(wl), x2, w, pos)["y"]
    np.testing.assert_array_equal(got, ref)
    x2[1, 2] += 1.0   # a cached token of sequence 1 does change it
    assert np.any(go.decode(_cfg(wl), x2, w, pos)["y"][1] != ref[1])


def _rope_cfg(wl, base, pos0=0):
    c = _cfg(wl)
    return go.OracleConfig(c.dim, c.num_query_experts, c.num_kv_heads, c.top_k, c.head_dim, c.variant,
                           c.shared_head, c.shared_kv_group, rope_base=base, pos0=pos0)


@pytest.mark.parametrize("variant,k,base", [("gqe", 1, 10000.0), ("weighted_concat", 2, 500.0),
                                            ("hard_concat", 1, 10.0)])
def test_rope_c_oracle_matches_complex_bruteforce(variant, k, base):
    """Rotary embedding (RoFormer; not on the pages, optional): the C oracle's real 2x2 rotations
    agree with the brute force's complex multiplications by exp(i m base^(-2i/dh))."""
    wl = _wl(d=24, N=8, G=2, k=k, dh=8, B=2, S=11, variant=variant, rstd=0.8)
    w = make_inputs(wl)
    cfg = _rope_cfg(wl, base)
    out = go.forward(cfg, wl.batch, wl.seq, w["x"], w)
    bf = bruteforce.layer(cfg, wl.batch, wl.seq, w["x"], w)
    np.testing.assert_allclose(out["y"], bf["y"], rtol=1e-10, atol=1e-12)
    plain = go.forward(_cfg(wl), wl.batch, wl.seq, w["x"], w)
    # the rotation is not a no-op
    assert np.max(np.abs(out["y"] - plain["y"])) > 1e-2 * np.sqrt(np.mean(plain["y"] ** 2))


def test_rope_depends_only_on_relative_positions():
    """q_m . k_n after the rotation depends on m - n only (RoFormer's defining property), so moving
    every position of a sequence by the same offset leaves the layer output unchanged."""
    wl = _wl(d=24, N=4, G=2, k=1, dh=8, B=1, S=12, rstd=1.0)
    w = make_inputs(wl)
    ref = go.forward(_rope_cfg(wl, 10000.0), 1, wl.seq, w["x"], w)["y"]
    for off in (1, 777, 40000):
        got = go.forward(_rope_cfg(wl, 10000.0, pos0=off), 1, wl.seq, w["x"], w)["y"]
        np.testing.assert_allclose(got, ref, rtol=1e-9, atol=1e-11)
    got = go.forward(_rope_cfg(wl, 10000.0, pos0=5), 1, wl.seq, w["x"], w)["K"]
    k0 = go.forward(_rope_cfg(wl, 10000.0), 1, wl.seq, w["x"], w)["K"]
    assert np.max(np.abs(got - k0)) > 1e-2 * np.sqrt(np.mean(k0 ** 2))   # the keys themselves move


def test_rope_at_position_zero_is_identity():
    """Position 0 rotates by angle 0: a one-token sequence is the same with and without RoPE."""
    wl = _wl(d=24, N=4, G=2, k=1, dh=8, B=3, S=1, rstd=1.0)
    w = make_inputs(wl)
    a = go.forward(_rope_cfg(wl, 10000.0), wl.batch, 1, w["x"], w)["y"]
    b = go.forward(_cfg(wl), wl.batch, 1, w["x"], w)["y"]
    np.testing.assert_array_equal(a, b)


def test_rope_decode_is_last_row_of_prefix_bruteforce():
    wl = _wl(d=24, N=8, G=2, k=2, dh=8, B=2, S=9, rstd=0.9)
    w = make_inputs(wl)
    cfg = _rope_cfg(wl, 10000.0)
    pos = [4, 8]
    dec = go.decode(cfg, w["x"], w, pos)
    for b, p in enumerate(pos):
        bf = bruteforce.layer(cfg, 1, p + 1, w["x"][b, :p + 1], w)
        np.testing.assert_allclose(dec["y"][b], bf["y"][p], rtol=1e-10, atol=1e-12)


# ---------------------------------------------------------------- backward pass
def _fd_check(cfg, B, S, w, dy, aux_coef, n_coords=5, seed=0, eps=1e-5):
    """Central finite differences of the oracle's loss against its analytic gradients, at random
    coordinates of x and of every weight (the routing held at the unperturbed decision)."""
    rng = np.random.default_rng(seed)
    T = B * S
    idx = go.router(cfg, np.asarray(w["x"], np.float64).reshape(T, cfg.dim), w["w_router"],
                    w.get("b_router"))["idx"]
    g = go.backward(cfg, B, S, w["x"], w, dy, aux_coef, idx)
    worst = 0.0
    for key in go.GRAD_KEYS:
        if key == "w_q_shared" or key == "w_o_shared":
            if not cfg.shared_head:
                continue
        if key == "w_o_rslot" and cfg.variant != "gqe":
            continue
        arr = np.asarray(w[key], np.float64)
        for _ in range(n_coords):
            pos = tuple(int(rng.integers(0, s)) for s in arr.shape)
            wp, wm = dict(w), dict(w)
            ap, am = arr.copy(), arr.copy()
            ap[pos] += eps
            am[pos] -= eps
            wp[key], wm[key] = ap, am
            fd = (go.loss(cfg, B, S, wp["x"], wp, dy, aux_coef, idx)
                  - go.loss(cfg, B, S, wm["x"], wm, dy, aux_coef, idx)) / (2 * eps)
            an = g[key].reshape(arr.shape)[pos]
            scale = max(1e-3, np.max(np.abs(g[key])))
            worst = max(worst, abs(fd - an) / scale)
            assert abs(fd - an) <= 1e-6 * scale, (key, pos, fd, an)
    return g, worst


@pytest.mark.parametrize("variant,k,shared,rope", [("gqe", 2, True, 0.0), ("gqe", 1, True, 10000.0),
                                                   ("weighted_concat", 1, True, 0.0),
                                                   ("weighted_concat", 2, False, 500.0),
                                                   ("hard_concat", 2, True, 0.0)])
def test_backward_matches_finite_differences(variant, k, shared, rope):
    """Training half of the method (README "Usage": lm_loss + 0.01 * aux): the oracle's analytic
    gradients of sum(dy * y) + 0.01 aux equal central finite differences of its own forward pass,
    for every tensor, with the renormalised slot (k = 2), the weighted_concat probabilities, the
    shared head and the rotary embedding exercised."""
    wl = _wl(d=16, N=8, G=2, k=k, dh=4, B=2, S=5, variant=variant, shared=shared, rstd=1.0, bias=0.3)
    w = make_inputs(wl)
    cfg = _rope_cfg(wl, rope)
    dy = np.random.default_rng(7).standard_normal((wl.tokens, wl.dim))
    _fd_check(cfg, wl.batch, wl.seq, w, dy, 0.01)


def test_backward_router_gradient_needs_more_than_one_choice():
    """With one choice per group the renormalised weight is identically 1 and hard concat has no
    router coefficient, so the LM loss sends no gradient to the router (only the aux loss does);
    with two choices (gqe) or the raw probability (weighted_concat) it does."""
    for variant, k, coef, zero in (("gqe", 1, 0.0, True), ("hard_concat", 2, 0.0, True),
                                   ("gqe", 2, 0.0, False), ("weighted_concat", 1, 0.0, False),
                                   ("gqe", 1, 0.01, False)):
        wl = _wl(d=16, N=8, G=2, k=k, dh=4, B=1, S=6, variant=variant, rstd=1.0)
        w = make_inputs(wl)
        dy = np.random.default_rng(3).standard_normal((wl.tokens, wl.dim))
        g = go.backward(_cfg(wl), 1, wl.seq, w["x"], w, dy, coef)
        if zero:
            assert np.all(g["w_router"] == 0) and np.all(g["b_router"] == 0), (variant, k)
        else:
            assert np.max(np.abs(g["w_router"])) > 1e-8, (variant, k, coef)


def test_backward_gqa_case_matches_torch_autograd():
    """k = N/G, hard concat, no shared head is textbook GQA: torch autograd (float64) of an
    independently written GQA layer with scaled_dot_product_attention gives the same gradients."""
    N, G, d, dh, S = 4, 2, 16, 4, 7
    wl = _wl(d=d, N=N, G=G, k=N // G, dh=dh, B=1, S=S, variant="hard_concat", shared=False, rstd=1.0)
    w = make_inputs(wl)
    dy = np.random.default_rng(5).standard_normal((S, d))
    g = go.backward(_cfg(wl), 1, S, w["x"], w, dy, 0.0)
    t = {k: torch.tensor(np.asarray(w[k], np.float64), requires_grad=True)
         for k in ("x", "w_q", "w_k", "w_v", "w_o")}
    x = t["x"].reshape(S, d)
    q = torch.einsum("sd,edh->esh", x, t["w_q"])                       # [N, S, dh]
    kk = (x @ t["w_k"]).reshape(S, G, dh).permute(1, 0, 2)               # [G, S, dh]
    vv = (x @ t["w_v"]).reshape(S, G, dh).permute(1, 0, 2)
    rep = N // G
    o = torch.nn.functional.scaled_dot_product_attention(
        q, kk.repeat_interleave(rep, 0), vv.repeat_interleave(rep, 0), is_causal=True)
    y = torch.einsum("esh,ehd->sd", o, t["w_o"])
    (y * torch.tensor(dy)).sum().backward()
    for key in ("x", "w_q", "w_k", "w_v", "w_o"):
        np.testing.assert_allclose(g[key].reshape(t[key].shape), t[key].grad.numpy(), rtol=1e-9, atol=1e-12)
