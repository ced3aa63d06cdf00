"""Pins of the MoE-MLP oracle (``oracle/moe_oracle.py``) to facts outside itself: the tutorial's
printed numbers and listed properties, library routines for the softmax / error function / bf16
rounding, brute force over expert subsets, the dense all-experts formulation, and closed forms."""
import itertools
import json
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

from oracle import moe_oracle as mo

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _weights(rng, d, E, dff, std_r=1.0, std=0.1):
    return dict(w_router=rng.standard_normal((d, E)) * std_r / np.sqrt(d),
                w1=rng.standard_normal((E, d, dff)) * std, w2=rng.standard_normal((E, dff, d)) * std)


def test_round_bf16_matches_torch():
    rng = np.random.default_rng(0)
    a = np.concatenate([rng.standard_normal(4000) * 10.0 ** rng.integers(-6, 6, 4000),
                        # exact ties between two bf16 values: both parities of the last kept bit
                        np.array([1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0, -0.0])])
    want = torch.tensor(a.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(mo.round_bf16(a), want)


def test_activations_closed_forms():
    h = np.linspace(-6, 6, 1001)
    np.testing.assert_allclose(mo.act(h, "gelu"), h * scipy.stats.norm.cdf(h), rtol=1e-13, atol=1e-15)
    assert mo.act(np.array([1.0]), "gelu")[0] == pytest.approx(0.8413447460685429, abs=1e-15)
    np.testing.assert_array_equal(mo.act(h, "relu"), np.where(h > 0, h, 0.0))


@pytest.mark.parametrize("E,k", [(6, 1), (6, 2), (5, 3)])
def test_router_matches_library_softmax_and_subset_bruteforce(E, k):
    rng = np.random.default_rng(E * 10 + k)
    T, d = 40, 12
    x = rng.standard_normal((T, d))
    w = _weights(rng, d, E, 4)
    b = rng.standard_normal(E) * 0.3
    r = mo.router(x, w["w_router"], k, b)
    p_lib = torch.softmax(torch.tensor(x @ w["w_router"] + b), dim=1).numpy()
    np.testing.assert_allclose(r["p"], p_lib, rtol=1e-12)
    for t in range(T):
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(r["logits"][t, list(s)]))
        assert set(r["idx"][t]) == set(best)
        assert list(r["idx"][t]) == sorted(best, key=lambda e: -r["logits"][t, e])
        assert r["w"][t].sum() == pytest.approx(1.0, abs=1e-14)
        np.testing.assert_allclose(r["w"][t], p_lib[t, r["idx"][t]] / p_lib[t, r["idx"][t]].sum(), rtol=1e-12)


def test_tie_break_zero_router():
    """W_r = 0: every logit equal, so the choices are experts 0 .. k-1 with weight 1/k."""
    x = np.random.default_rng(1).standard_normal((7, 5))
    r = mo.router(x, np.zeros((5, 8)), 3)
    assert (r["idx"] == np.array([0, 1, 2])).all()
    np.testing.assert_allclose(r["w"], 1.0 / 3.0)
    np.testing.assert_allclose(r["p"], 1.0 / 8.0)


@pytest.mark.parametrize("activation", mo.ACTIVATIONS)
@pytest.mark.parametrize("k", [1, 2, 4])
def test_identical_experts_equal_a_single_expert(activation, k):
    """The tutorial's check of the mixing: with identical experts the layer is one expert."""
    rng = np.random.default_rng(k)
    T, d, E, dff = 30, 16, 6, 24
    x = rng.standard_normal((T, d))
    w1 = rng.standard_normal((d, dff)) * 0.3
    w2 = rng.standard_normal((dff, d)) * 0.3
    w = dict(w_router=rng.standard_normal((d, E)), w1=np.repeat(w1[None], E, 0), w2=np.repeat(w2[None], E, 0))
    h = x @ w1
    single = (0.5 * h * (1 + scipy.special.erf(h / np.sqrt(2))) if activation == "gelu" else np.maximum(h, 0)) @ w2
    np.testing.assert_allclose(mo.forward(x, w, k, activation)["y"], single, rtol=1e-12, atol=1e-13)


@pytest.mark.parametrize("activation", mo.ACTIVATIONS)
def test_dense_mixture_bruteforce(activation):
    """Every expert run on every token, mixed by a dense [T, E] weight matrix that is zero for the
    unchosen experts (no gathering), equals the oracle's routed computation."""
    rng = np.random.default_rng(5)
    T, d, E, dff, k = 50, 10, 5, 7, 2
    x = rng.standard_normal((T, d))
    w = _weights(rng, d, E, dff, std=0.5)
    out = mo.forward(x, w, k, activation)
    M = np.zeros((T, E))
    for t in range(T):
        for r in range(k):
            M[t, out["idx"][t, r]] += out["w"][t, r]
    dense = np.zeros((T, d))
    for e in range(E):
        dense += M[:, e:e + 1] * (mo.act(x @ w["w1"][e], activation) @ w["w2"][e])
    np.testing.assert_allclose(out["y"], dense, rtol=1e-12, atol=1e-13)
    for t in range(T):   # exactly k distinct experts, weights sum to 1
        assert len(set(out["idx"][t])) == k


def test_all_experts_active_is_the_softmax_mixture():
    rng = np.random.default_rng(6)
    T, d, E, dff = 20, 8, 4, 6
    x = rng.standard_normal((T, d))
    w = _weights(rng, d, E, dff, std=0.5)
    out = mo.forward(x, w, E, "relu")
    p = torch.softmax(torch.tensor(x @ w["w_router"]), dim=1).numpy()
    want = sum(p[:, e:e + 1] * (np.maximum(x @ w["w1"][e], 0) @ w["w2"][e]) for e in range(E))
    np.testing.assert_allclose(out["y"], want, rtol=1e-12, atol=1e-13)
    assert np.isinf(out["gap"]).all()


def test_relu_with_positive_operands_is_linear():
    rng = np.random.default_rng(7)
    T, d, E, dff, k = 25, 6, 4, 5, 2
    x = np.abs(rng.standard_normal((T, d)))
    w = _weights(rng, d, E, dff)
    w["w1"] = np.abs(w["w1"])
    out = mo.forward(x, w, k, "relu")
    for t in range(T):
        lin = sum(out["w"][t, r] * (x[t] @ w["w1"][out["idx"][t, r]] @ w["w2"][out["idx"][t, r]]) for r in range(k))
        np.testing.assert_allclose(out["y"][t], lin, rtol=1e-12, atol=1e-13)


def test_expert_relabelling():
    rng = np.random.default_rng(8)
    T, d, E, dff, k = 40, 8, 6, 5, 2
    x = rng.standard_normal((T, d))
    w = _weights(rng, d, E, dff, std=0.5)
    perm = rng.permutation(E)
    wp = dict(w_router=w["w_router"][:, perm], w1=w["w1"][perm], w2=w["w2"][perm])
    a, b = mo.forward(x, w, k), mo.forward(x, wp, k)
    np.testing.assert_allclose(a["y"], b["y"], rtol=1e-12, atol=1e-13)
    np.testing.assert_array_equal(perm[b["idx"]], a["idx"])


def test_golden_active_parameters_and_even_share():
    g = json.load(open(os.path.join(GOLDEN, "moe_mlp_tutorial.json")))
    E, k = g["experts"], g["active"]
    rng = np.random.default_rng(9)
    T, d, dff = 64, 8, 12
    x = rng.standard_normal((T, d))
    w = _weights(rng, d, E, dff)
    out = mo.forward(x, w, k)
    per_expert = w["w1"][0].size + w["w2"][0].size
    for t in range(T):
        used = len(set(out["idx"][t])) * per_expert
        assert used / (E * per_expert) == g["active_param_fraction"]
    # routing that cycles through the experts: every expert gets the even share
    logits_pick = np.zeros((E * 4, E))
    for t in range(E * 4):
        logits_pick[t, [(t + r) % E for r in range(k)]] = [5.0 - r for r in range(k)]
    r = mo.router(logits_pick, np.eye(E), k)
    st = mo.stats(r["p"], r["idx"], E)
    np.testing.assert_allclose(st["share"], g["even_share"])


def test_balance_loss_closed_forms():
    E, k, T = 8, 2, 16
    x = np.ones((T, 3))
    st = mo.stats(mo.router(x, np.zeros((3, E)), k)["p"], mo.router(x, np.zeros((3, E)), k)["idx"], E)
    assert st["aux"] == pytest.approx(1.0)   # uniform probabilities
    # collapse: every token to experts {0, 1} with probability ~1 on expert 0
    r = mo.router(x, np.zeros((3, E)), k, b_router=np.array([60.0, 30.0] + [0.0] * (E - 2)))
    st = mo.stats(r["p"], r["idx"], E)
    np.testing.assert_allclose(st["share"][:2], 0.5)
    assert st["aux"] == pytest.approx(E * 0.5, rel=1e-9)


def test_hidden_rounding_is_only_the_stored_precision():
    rng = np.random.default_rng(10)
    T, d, E, dff, k = 30, 16, 4, 32, 2
    x = rng.standard_normal((T, d))
    w = _weights(rng, d, E, dff, std=0.3)
    a, b = mo.forward(x, w, k), mo.forward(x, w, k, hidden="bf16")
    np.testing.assert_array_equal(b["h"], mo.round_bf16(a["h"]))
    assert np.max(np.abs(a["y"] - b["y"])) < 2.0 ** -7 * np.max(np.abs(a["y"]))
