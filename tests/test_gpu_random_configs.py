"""GPU parity over a seeded sweep of layer configurations (every token and stage against the oracle).

The hand-picked cases in test_gpu_parity.py follow the pages' workloads; this sweep draws the
layer's parameters (hidden size, experts, groups, top-k, head dim, variant, shared head and its
group, rotary embedding, storage type) and the input shape from fixed seeds, so both the
matrix-core path (bf16, head dims 32 / 48 / 64, hidden sizes that tile by 64) and the scalar path
(everything else the method allows) meet combinations nobody chose.  The draw is fixed: the same
cases run every time.
"""
from __future__ import annotations

import numpy as np
import pytest

from sparse_moe_query_amd.inputs import Workload
from tests import parity

pytestmark = pytest.mark.gpu


def _draw(i: int) -> Workload:
    r = np.random.default_rng(7000 + i)
    G = int(r.choice([1, 2, 4, 8]))
    n = int(r.choice([1, 2, 3, 4]))
    N = G * n
    k = int(r.integers(1, min(n, 3) + 1))
    dtype = "f32" if r.random() < 0.2 else "bf16"
    dh = int(r.choice([16, 24, 32, 40, 48, 64, 80, 128]))
    d = int(r.choice([64, 96, 128, 192, 256, 384, 512]))
    variant = str(r.choice(["gqe", "weighted_concat", "hard_concat"]))
    shared = bool(r.random() < 0.7)
    skv = int(r.integers(0, G))
    rope = 10000.0 if r.random() < 0.3 else 0.0
    B = int(r.integers(1, 4))
    S = int(r.integers(1, 301))
    return Workload(f"rand{i:02d}_d{d}_N{N}_G{G}_k{k}_dh{dh}_{dtype}_{variant}_s{int(shared)}_B{B}_S{S}"
                    + ("_rope" if rope else ""), d, N, G, k, dh, B, S, dtype=dtype, variant=variant,
                    shared_head=shared, shared_kv_group=skv, seed=300 + i, rope_base=rope,
                    router_std=0.3 if dtype == "f32" else None)


CASES = [_draw(i) for i in range(24)]


@pytest.mark.parametrize("wl", CASES, ids=[w.name for w in CASES])
def test_random_config_every_token(wl):
    from sparse_moe_query_amd.runner import build_layer, run_layer
    print(f"[gpu] {wl.name}", flush=True)
    layer, x, inp = build_layer(wl)
    gpu = run_layer(layer, x)
    rep = parity.compare(wl, gpu, inp)
    print(f"[gpu]   y_err={rep['y_err']:.2e} near_ties={rep['near_ties']} "
          f"matrix_core={layer.intermediates(wl.batch, wl.seq)['matrix_core']}", flush=True)
    layer.close()
