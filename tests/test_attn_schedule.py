"""The attention work schedule (host logic, no GPU): every key tile of every (batch, group,
block of positions) item is processed by exactly one job, jobs are dispatched longest first, and
each split item's chunks own consecutive partial slots that one merge record combines."""
import math

import numpy as np
import pytest

from sparse_moe_query_amd import gqe

COLS, TILE = 256, 64


def _handle(d=768, N=16, G=8, k=1, dh=48, shared=1, skv=0, dense=0, variant=0):
    cfg = gqe.Config(d, N, G, k, dh, variant, shared, skv, 1, 1, dense)
    base = {f: 0x10000 * (i + 1) for i, (f, _) in enumerate(gqe.Weights._fields_)}
    if dense:
        base["w_router"] = base["b_router"] = 0
    w = gqe.Weights(*[base[f] for f, _ in gqe.Weights._fields_])
    return gqe.gqe_init(cfg, w)


def _items(G, k, shared, skv, B, S):
    out = set()
    for g in range(G):
        nh = k + (1 if shared and g == skv else 0)
        P = COLS // nh
        for b in range(B):
            for p0 in range(0, S, P):
                np_ = min(P, S - p0)
                out.add((b, g, nh, p0, np_, (p0 + np_ - 1) // TILE + 1))
    return out


CASES = [
    dict(B=8, S=2048), dict(B=1, S=16384), dict(B=1, S=32768), dict(B=2, S=8192),
    dict(B=1, S=1000), dict(B=3, S=17), dict(B=4, S=1), dict(B=1, S=200, skv=3),
    dict(B=4, S=4096, d=1024, k=2, dh=64), dict(B=1, S=700, d=1024, k=2, dh=64),
    dict(B=1, S=16384, k=2, variant=2, shared=0, dense=1), dict(B=2, S=900, d=256, N=8, G=4, k=2, dh=32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_schedule_covers_every_tile_once(case):
    c = dict(d=768, N=16, G=8, k=1, dh=48, shared=1, skv=0, dense=0, variant=0)
    c.update(case)
    B, S = c.pop("B"), c.pop("S")
    h = _handle(**c)
    try:
        jobs, merges, nslots, chunk = gqe.gqe_attention_schedule(h, B, S)
        ws_with = gqe.gqe_workspace_bytes(h, B, S)
    finally:
        gqe.gqe_destroy(h)
    items = _items(c["G"], c["k"], c["shared"], c["skv"], B, S)
    # lengths never increase along the dispatch order
    lens = jobs[:, 6] - jobs[:, 5]
    assert np.all(lens > 0)
    assert np.all(np.diff(lens) <= 0)
    # coverage: the jobs of an item tile [0, kt_end) exactly once
    seen = {}
    for j in jobs:
        key = tuple(int(v) for v in j[:5])
        seen.setdefault(key, []).append((int(j[5]), int(j[6]), int(j[7])))
    got_items = {key + (max(e for _, e, _ in v),) for key, v in seen.items()}
    assert got_items == items
    used_slots = []
    for key, v in seen.items():
        v.sort()
        assert v[0][0] == 0
        for (a0, e0, _), (a1, _, _) in zip(v, v[1:]):
            assert e0 == a1
        if len(v) == 1:
            assert v[0][2] == -1
        else:
            assert all(s >= 0 for _, _, s in v)
            used_slots += [s for _, _, s in v]
    # slots: each used once, 0 .. nslots-1; a merge record per split item with its chunk run
    assert sorted(used_slots) == list(range(nslots))
    assert len(merges) == sum(1 for v in seen.values() if len(v) > 1)
    for m in merges:
        key = tuple(int(x) for x in m[:5])
        v = seen[key]
        assert int(m[6]) == len(v) <= 32
        assert [s for _, _, s in v] == list(range(int(m[5]), int(m[5]) + int(m[6])))
    # chunk cap respected, and the workspace holds the partial results
    if chunk:
        assert lens.max() <= max(chunk, math.ceil(max(i[5] for i in items) / 32))
    assert ws_with >= nslots * COLS * (c["dh"] + 2) * 4


def test_long_items_are_split_at_16k():
    """At seq 16384 the last item reads all 256 key tiles, longer than the average load of a
    work-group slot; the schedule must split it."""
    h = _handle()
    try:
        jobs, merges, nslots, chunk = gqe.gqe_attention_schedule(h, 1, 16384)
    finally:
        gqe.gqe_destroy(h)
    assert chunk > 0 and len(merges) > 0
    assert (jobs[:, 6] - jobs[:, 5]).max() < 256



def _canonical(G, k, shared, skv, B, S, chunk):
    """The dispatch order written out from its definition: templates (group, item, chunk) in that
    order, sorted by key-tile count (longest first, ties keep template order), each repeated for
    the B sequences; split items own B ss + b nc + c slots and merge record B mi + b."""
    tpl, merges, ss, mi = [], [], 0, 0
    for g in range(G):
        nh = k + (1 if shared and g == skv else 0)
        P = COLS // nh
        for i in range((S + P - 1) // P):
            p0, np_ = i * P, min(P, S - i * P)
            kt = (p0 + np_ - 1) // TILE + 1
            nc = 1 if chunk <= 0 or kt <= chunk else min(-(-kt // chunk), 32)
            for c in range(nc):
                tpl.append((g, nh, p0, np_, c * kt // nc, (c + 1) * kt // nc, nc, c, ss if nc > 1 else -1))
            if nc > 1:
                merges += [(b, g, nh, p0, np_, B * ss + b * nc, nc, 0) for b in range(B)]
                ss += nc
                mi += 1
    order = sorted(range(len(tpl)), key=lambda t: (-(tpl[t][5] - tpl[t][4]), t))
    jobs = []
    for t in order:
        g, nh, p0, np_, a, e, nc, c, s0 = tpl[t]
        for b in range(B):
            jobs.append((b, g, nh, p0, np_, a, e, B * s0 + b * nc + c if s0 >= 0 else -1))
    return np.array(jobs, np.int32).reshape(-1, 8), np.array(merges, np.int32).reshape(-1, 8)


@pytest.mark.parametrize("case", CASES, ids=lambda c: "-".join(f"{k}{v}" for k, v in c.items()))
def test_schedule_follows_its_canonical_order(case):
    """The tables equal the order written out from its definition (the device builder of every
    forward writes the same tables; a GPU test compares them bit for bit)."""
    c = dict(d=768, N=16, G=8, k=1, dh=48, shared=1, skv=0, dense=0, variant=0)
    c.update(case)
    B, S = c.pop("B"), c.pop("S")
    h = _handle(**c)
    try:
        jobs, merges, nslots, chunk = gqe.gqe_attention_schedule(h, B, S)
    finally:
        gqe.gqe_destroy(h)
    k = c["N"] // c["G"] if c["dense"] else c["k"]
    ej, em = _canonical(c["G"], k, c["shared"] and not c["dense"], c["skv"], B, S, chunk)
    np.testing.assert_array_equal(jobs, ej)
    np.testing.assert_array_equal(merges.reshape(-1, 8), em)
