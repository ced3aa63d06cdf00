"""GPU parity of the backward pass, of decode and of the top-k MoE-MLP over seeded draws of the
layer's configuration.

As in test_gpu_random_configs.py, the parameters and shapes come from fixed seeds (the same cases
every run), restricted to what each entry point supports: the backward takes head dims that are
multiples of 16 and at most 16 experts per group; decode takes 16-byte cache rows, at most eight
active heads per group and at most 8192 slot dims per token; the MoE-MLP takes bf16, at most 16
experts and sizes that are multiples of 32.  The checks are those of the hand-picked cases
(tests/test_gpu_backward.py, tests/test_gpu_decode.py, tests/test_gpu_moe.py).
"""
from __future__ import annotations

import numpy as np
import pytest

from sparse_moe_query_amd.inputs import MoeWorkload, Workload
from tests.test_gpu_backward import _check as check_backward
from tests.test_gpu_decode import _decode_steps
from tests.test_gpu_moe import test_moe_matches_oracle as check_moe

pytestmark = pytest.mark.gpu


def _draw(r, name: str, dhs, B_max: int, S_max: int) -> Workload:
    G = int(r.choice([1, 2, 4, 8]))
    n = int(r.choice([1, 2, 3, 4]))
    k = int(r.integers(1, min(n, 3) + 1))
    dtype = "f32" if r.random() < 0.2 else "bf16"
    dh = int(r.choice(dhs))
    d = int(r.choice([64, 128, 192, 256, 384, 512]))
    variant = str(r.choice(["gqe", "weighted_concat", "hard_concat"]))
    shared = bool(r.random() < 0.7)
    skv = int(r.integers(0, G))
    rope = 10000.0 if r.random() < 0.3 else 0.0
    B = int(r.integers(1, B_max + 1))
    S = int(r.integers(2, S_max + 1))
    return Workload(f"{name}_d{d}_N{G * n}_G{G}_k{k}_dh{dh}_{dtype}_{variant}_s{int(shared)}_B{B}_S{S}"
                    + ("_rope" if rope else ""), d, G * n, G, k, dh, B, S, dtype=dtype, variant=variant,
                    shared_head=shared, shared_kv_group=skv, seed=int(r.integers(0, 1 << 16)),
                    rope_base=rope, router_std=0.3 if dtype == "f32" else None)


def _decode_ok(wl: Workload) -> bool:
    es = 2 if wl.dtype == "bf16" else 4
    s = int(wl.shared_head)
    slots = wl.num_kv_heads * wl.top_k + (wl.num_kv_heads if wl.variant == "gqe" else 0) + s
    return ((wl.dh * es) % 16 == 0 and wl.dh <= 128 and (wl.dim * es) % 16 == 0 and wl.top_k + s <= 8
            and slots <= 192 and slots * wl.dh <= 8192)


BWD = [_draw(np.random.default_rng(8100 + i), f"rbwd{i:02d}", [16, 32, 48, 64, 128], 2, 160) for i in range(10)]

DEC = []
_i = 0
while len(DEC) < 10:
    _w = _draw(np.random.default_rng(8200 + _i), f"rdec{_i:02d}", [16, 24, 32, 40, 48, 64, 80, 128], 3, 300)
    _i += 1
    if _decode_ok(_w):
        DEC.append(_w)


@pytest.mark.parametrize("wl", BWD, ids=[w.name for w in BWD])
def test_random_backward(wl):
    check_backward(wl)


@pytest.mark.parametrize("wl", DEC, ids=[w.name for w in DEC])
def test_random_decode(wl):
    r = np.random.default_rng(len(wl.name))
    # ragged prefixes (an empty cache among them when the batch allows), two steps each
    lens = sorted(int(v) for v in r.integers(0, max(1, wl.seq - 2), size=wl.batch))
    lens[0] = 0
    _decode_steps(wl, lens, 2, wl.seq)


def _moe_draw(i: int) -> MoeWorkload:
    r = np.random.default_rng(8300 + i)
    E = int(r.integers(1, 17))
    k = int(r.integers(1, min(E, 4) + 1))
    d = int(r.choice([64, 96, 128, 192, 256, 320]))
    dff = int(r.choice([32, 64, 96, 160, 256, 512]))
    T = int(r.integers(1, 601))
    act = str(r.choice(["gelu", "relu"]))
    return MoeWorkload(f"rmoe{i:02d}_d{d}_E{E}_k{k}_ff{dff}_T{T}_{act}", d, E, k, dff, T, activation=act,
                       seed=500 + i)


MOE = [_moe_draw(i) for i in range(8)]


@pytest.mark.parametrize("wl", MOE, ids=[w.name for w in MOE])
def test_random_moe(wl):
    check_moe(wl)
