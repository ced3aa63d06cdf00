"""GPU: gqe_forward_static, the forward for callers that cannot allocate device memory (it runs on
the library's static per-GPU scratch array instead of a caller workspace), against gqe_forward on
the same inputs -- two calls in a row, the second with a smaller input -- and against the oracle.
Runs alone in a fresh process as well as after the other tests."""
import numpy as np
import pytest
import torch

from sparse_moe_query_amd.inputs import Workload
from tests import parity

pytestmark = pytest.mark.gpu


def _forward_both(layer, x, B, S):
    from sparse_moe_query_amd import gqe
    G, k = layer.G, layer.k
    out = {}
    for name in ("workspace", "static"):
        y = torch.full_like(x, float("nan"))
        ridx = torch.full((B, S, G, k), -1, dtype=torch.int32, device=x.device)
        rw = torch.full((B, S, G, k), -1.0, dtype=torch.float32, device=x.device)
        torch.cuda.synchronize()
        alloc0 = torch.cuda.memory_allocated()
        if name == "workspace":
            gqe.gqe_forward(layer.h, x, y, B, S, layer.workspace(B, S), route_idx=ridx, route_w=rw)
        else:
            gqe.gqe_forward_static(layer.h, x, y, B, S, route_idx=ridx, route_w=rw)
            torch.cuda.synchronize()
            assert torch.cuda.memory_allocated() == alloc0
        torch.cuda.synchronize()
        st = layer.aux_stats()
        out[name] = dict(y=y.clone(), idx=ridx.clone(), w=rw.clone(), stats=st)
    return out


def test_static_forward_matches_workspace_forward():
    from sparse_moe_query_amd.runner import build_layer
    wl = Workload("static_main", 768, 16, 8, 1, 48, 2, 300, seed=40)
    layer, x, inp = build_layer(wl)
    small = Workload("static_small", 768, 16, 8, 1, 48, 1, 100, seed=40)
    xs = x[:1, :100].contiguous()
    for (B, S, xx, w) in ((2, 300, x, wl), (1, 100, xs, small)):
        print(f"[gpu] static forward B={B} S={S}", flush=True)
        out = _forward_both(layer, xx, B, S)
        a, b = out["workspace"], out["static"]
        assert torch.equal(a["y"], b["y"]), "outputs differ"
        assert torch.equal(a["idx"], b["idx"]) and torch.equal(a["w"], b["w"])
        np.testing.assert_array_equal(a["stats"]["counts"], b["stats"]["counts"])
        np.testing.assert_array_equal(a["stats"]["mean_prob"], b["stats"]["mean_prob"])
        assert a["stats"]["aux"] == b["stats"]["aux"]
        # and the oracle's bar for the static result
        inp_w = dict(inp, x=inp["x"][:B, :S])
        gpu = dict(y=b["y"].float().cpu().numpy().astype(np.float64).reshape(B * S, -1),
                   idx=b["idx"].cpu().numpy().reshape(B * S, 8, 1), w=b["w"].cpu().numpy().reshape(B * S, 8, 1))
        gpu.update(b["stats"])
        rep = parity.compare(w, gpu, inp_w)
        print(f"[gpu]   equal to gqe_forward; y_err {rep['y_err']:.2e}", flush=True)
    layer.close()


def test_static_forward_rejects_shapes_beyond_its_scratch():
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.runner import build_layer
    wl = Workload("static_big", 768, 16, 8, 1, 48, 1, 64, seed=41)
    layer, x, _ = build_layer(wl)
    B, S = 1, 16384
    assert gqe.gqe_workspace_bytes(layer.h, B, S) > gqe.STATIC_SCRATCH_BYTES
    xb = torch.zeros((B, S, wl.dim), dtype=x.dtype, device=x.device)
    y = torch.empty_like(xb)
    with pytest.raises(gqe.GqeError) as e:
        gqe.gqe_forward_static(layer.h, xb, y, B, S)
    assert e.value.code == -5 and "static scratch" in str(e.value)
    layer.close()
