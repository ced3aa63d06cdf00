"""GPU: the attention work schedule built by every forward in its workspace, and the forward's
promise to allocate nothing and copy nothing (so that it can run under HIP graph capture).

The device builder (integer work) must write exactly the tables the host planner returns."""
import numpy as np
import pytest
import torch

from sparse_moe_query_amd.inputs import WORKLOADS, Workload, gqa_of
from tests import parity

pytestmark = pytest.mark.gpu


def _small(name, d=768, N=16, G=8, k=1, dh=48, B=2, S=200, **kw):
    return Workload(name, d, N, G, k, dh, B, S, **kw)


SHAPES = [
    WORKLOADS["main_b8_s2048"],
    WORKLOADS["long_s16384"],
    WORKLOADS["long_s32768"],
    WORKLOADS["k2_skew_b4_s4096"],
    gqa_of(WORKLOADS["long_s16384"]),
    _small("sched_s1000", B=1, S=1000),
    _small("sched_short", B=3, S=17),
    _small("sched_single", B=4, S=1),
    _small("sched_group3", B=2, S=700, shared_kv_group=3),
    _small("sched_dh32_k2", d=256, N=8, G=4, k=2, dh=32, B=2, S=900),
    # hidden size not a multiple of 64: scalar projection, so the schedule kernel of its own
    _small("sched_own_kernel", d=96, N=8, G=4, k=1, dh=32, B=2, S=900),
]


@pytest.mark.parametrize("wl", SHAPES, ids=[w.name for w in SHAPES])
def test_device_schedule_equals_host_schedule(wl):
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.runner import build_layer, run_layer
    print(f"[gpu] schedule {wl.name} B={wl.batch} S={wl.seq} k={wl.top_k} dh={wl.dh}", flush=True)
    layer, x, _ = build_layer(wl)
    run_layer(layer, x, routing=False)
    jobs, merges, nslots, chunk = gqe.gqe_attention_schedule(layer.h, wl.batch, wl.seq)
    inter = layer.intermediates(wl.batch, wl.seq)
    dj = inter["jobs"].cpu().numpy()
    np.testing.assert_array_equal(dj, jobs)
    if len(merges):
        off = inter["merges_offset"]
        dm = layer._ws[off:off + merges.size * 4].view(torch.int32).reshape(-1, 8).cpu().numpy()
        np.testing.assert_array_equal(dm, merges)
    print(f"[gpu]   {len(jobs)} jobs, {len(merges)} merges, chunk cap {chunk}", flush=True)
    layer.close()


def test_forward_of_a_fresh_shape_allocates_nothing():
    """gqe_forward of a shape the handle has never seen: device memory in use (torch's
    allocator and the device's free memory) is the same before and after, and the result matches
    the oracle."""
    from sparse_moe_query_amd.runner import build_layer, run_layer
    wl = _small("noalloc_fresh", B=1, S=1000, seed=3)
    layer, x, inp = build_layer(wl)
    warm = torch.zeros((2, 300, wl.dim), dtype=x.dtype, device=x.device)
    layer(warm)                                  # every kernel loaded, another shape
    ws = layer.workspace(1, 1000)                # the caller's workspace, allocated up front
    y = torch.empty_like(x)
    torch.cuda.synchronize()
    alloc0 = torch.cuda.memory_allocated()
    free0 = torch.cuda.mem_get_info()[0]
    from sparse_moe_query_amd import gqe
    gqe.gqe_forward(layer.h, x, y, 1, 1000, ws)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == alloc0
    assert torch.cuda.mem_get_info()[0] == free0
    gpu = run_layer(layer, x)
    parity.compare(wl, gpu, inp)
    layer.close()


def test_forward_replays_in_a_hip_graph():
    """The forward captured in a HIP graph and replayed three times, with other work and
    synchronisations in between, gives the eager result bit for bit every time."""
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.runner import build_layer
    wl = _small("graph_main", B=2, S=700, seed=4)
    layer, x, _ = build_layer(wl)
    ws = layer.workspace(2, 700)
    y_eager = torch.empty_like(x)
    gqe.gqe_forward(layer.h, x, y_eager, 2, 700, ws)
    torch.cuda.synchronize()
    ref = y_eager.clone()
    y = torch.zeros_like(x)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        gqe.gqe_forward(layer.h, x, y, 2, 700, ws)   # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gqe.gqe_forward(layer.h, x, y, 2, 700, ws)
    for r in range(3):
        y.zero_()
        junk = torch.randn(1024, 1024, device=x.device) @ torch.randn(1024, 1024, device=x.device)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, ref), f"replay {r} differs"
        del junk
    layer.close()
