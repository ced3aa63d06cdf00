"""Benchmark of the GQE forward (prefill) pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-long] [--no-decode] [--only-main]
                [--profile-workload NAME] [--copy-calibration]

One step = one gqe_forward over the main-setting workload (dim 768, N=16, G=8, k=1, head_dim 48,
shared head, variant gqe, batch 8 x seq 2048, bf16) with x and the packed weights resident in HBM.
Prints ONE JSON line (stdout): tokens/s of that workload (K timed forwards, bracketed by device
synchronisations); the roofline of its dominant kernel (its algorithmic work per launch over its
average launch duration, from HIP events recorded on the forward's stream right before and after
every kernel during K more forwards; HBM traffic from the committed rocprofv3 counter summary
when it was taken on the current kernel source, else null); the CPU
oracle timed on a bounded sample; and, as extra fields, the all-active GQA baseline, the
long-context runs (seq 16384 and 32768) and a decode step with a dense KV cache (64 sequences with
8192 cached positions each, same layer shape).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2500.0   # TFLOP/s, MI355X dense bf16 matrix
PEAK_FP64 = 78.6     # TFLOP/s, MI355X fp64 (matrix and vector)
PEAK_HBM = 8000.0    # GB/s
PEAK_FP32 = 157.3    # TFLOP/s, MI355X float32 vector (float32 layers' backward)

# kernel slot -> (source file of the kernel, stage of the algorithmic-work table)
KERNEL_SOURCES = {
    "router": ("k_router.hip", "router"),
    "projection": ("k_proj.hip", "projection"),
    "attention": ("k_attn.hip", "attention"),
    "combine": ("k_combine.hip", "combine"),
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(wl) -> dict:
    """Algorithmic work of one forward, per stage: flops (active heads only; causal attention
    counts S(S+1)/2 score entries per head) and HBM bytes (each tensor read or written once,
    bf16 = 2 bytes)."""
    T, d, N, G, dh = wl.tokens, wl.dim, wl.num_query_experts, wl.num_kv_heads, wl.dh
    k = wl.top_k
    H = G * k + (1 if wl.shared_head else 0)
    B, S = wl.batch, wl.seq
    es = 2 if wl.dtype == "bf16" else 4
    slots = N if wl.dense_gqa else G * k + (G if wl.variant == "gqe" else 0) + (1 if wl.shared_head else 0)
    gk = G * k
    out = {
        "router": dict(flops=0.0 if wl.dense_gqa else 2.0 * T * d * N,
                       bytes=0.0 if wl.dense_gqa else T * d * es + d * N * 8 + T * gk * 12.0),
        "projection": dict(flops=2.0 * T * d * dh * (2 * G + H),
                           bytes=T * d * es + d * dh * (2 * G + (N if wl.dense_gqa else N + (1 if wl.shared_head else 0))) * es
                           + T * (H + 2 * G) * dh * es + T * G * 4.0),
        "attention": dict(flops=4.0 * dh * H * B * S * (S + 1) / 2.0,
                          bytes=(B * H * S * dh + 2 * B * G * S * dh + T * H * dh) * es),
        "combine": dict(flops=2.0 * T * d * dh * slots,
                        bytes=(T * H * dh + T * d) * es + d * dh * (N + G + 1) * es + T * gk * 12.0),
    }
    out["layer_flops"] = sum(v["flops"] for v in out.values() if isinstance(v, dict))
    return out


def source_hash(fname: str) -> str:
    """Hash of a kernel source and the helpers it includes (ties counter summaries to code)."""
    h = hashlib.sha256()
    for f in (fname, "gqe_common.h"):
        with open(os.path.join(ROOT, "sparse_moe_query_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str, source: str | None = None):
    """HBM bytes per launch of ``kernel`` on ``workload`` from profiles/traffic_<kernel>_<workload>.md,
    if that summary was taken on the current source (its 'source hash' line matches)."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source hash:\s*([0-9a-f]+)", text)
    m_bytes = re.search(r"HBM bytes per launch \(scaled\):\s*([0-9.eE+]+)", text)
    src = source or KERNEL_SOURCES[kernel][0]
    if not m_hash or not m_bytes or m_hash.group(1) != source_hash(src):
        return None
    return float(m_bytes.group(1))


def committed_mfma_busy(kernel: str, workload: str):
    """Measured matrix-core busy fraction of ``kernel`` on ``workload`` (SQ_VALU_MFMA_BUSY_CYCLES over
    the SIMDs' active cycles) from profiles/counters_<kernel>_<workload>.md, if that summary was taken
    on the current source."""
    path = os.path.join(ROOT, "profiles", f"counters_{kernel}_{workload}.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m_hash = re.search(r"source hash:\s*([0-9a-f]+)", text)
    m_busy = re.search(r"mfma_busy:\s*([0-9.eE+-]+)", text)
    if not m_hash or not m_busy or m_hash.group(1) != source_hash(KERNEL_SOURCES[kernel][0]):
        return None
    return float(m_busy.group(1))


def run_workload(wl, steps, warmup, profile=True):
    import torch
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.runner import build_layer
    layer, x, _ = build_layer(wl)
    y = torch.empty_like(x)
    for _ in range(warmup):
        layer(x, y)
    # timed steps: nothing but the forwards on the stream
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer(x, y)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms = (t1 - t0) * 1e3 / steps
    # the same number of steps again with HIP events around every kernel (per-kernel durations)
    kern, n = {}, 0
    if profile:
        gqe.gqe_profile_enable(layer.h, True)
        for _ in range(steps):
            layer(x, y)
        torch.cuda.synchronize()
        kern, n = gqe.gqe_profile_read_kernels(layer.h)
        gqe.gqe_profile_enable(layer.h, False)
    kernel_ms = {k: v / max(n, 1) for k, v in kern.items()}
    path = layer.intermediates(wl.batch, wl.seq)["matrix_core"]
    layer.close()
    del layer, x, y
    torch.cuda.empty_cache()
    return ms, kernel_ms, path


def stages_of(kernel_ms: dict) -> dict:
    g = kernel_ms.get
    return {"router": g("router", 0) + g("router_stats", 0),
            "projection": g("projection", 0) + g("key_norms", 0),
            "attention": g("attention_prep", 0) + g("attention", 0) + g("attention_merge", 0),
            "combine": g("combine", 0)}


def attn_step_ms(kernel_ms: dict) -> float:
    """The attention step: the attention kernel plus the merge of items split along the key range
    (0 when the schedule splits nothing)."""
    return kernel_ms.get("attention", 0.0) + kernel_ms.get("attention_merge", 0.0)


def roofline(kernel: str, ms: float, alg: dict, workload: str, merge_ms: float = 0.0) -> dict:
    """``ms`` is the kernel's own average launch duration (what rocprofv3 reports for it); for the
    attention kernel, ``achieved`` also charges the merge kernel's time (``merge_ms``)."""
    stage = KERNEL_SOURCES[kernel][1]
    f = alg[stage]["flops"] / ((ms + merge_ms) * 1e-3) / 1e12
    peak = PEAK_FP64 if kernel == "router" else PEAK_BF16
    r = dict(bound="mfma", achieved=f, peak=peak, unit="TFLOP/s", frac=f / peak)
    r["kernel"] = kernel
    r["kernel_ms"] = ms
    r["merge_ms"] = merge_ms
    r["traffic"] = committed_traffic(kernel, workload)
    r["algorithmic_bytes"] = alg[stage]["bytes"]
    r["algorithmic_hbm_frac"] = alg[stage]["bytes"] / (ms * 1e-3) / 1e9 / PEAK_HBM
    return r


# Decode: the main-setting layer, one new token for each of `batch` sequences with `ctx` cached positions.
DECODE_WORKLOADS = {"decode_b64_ctx8192": ("main_b8_s2048", 64, 8192)}
KV_STD = 0.02 * 768 ** 0.5   # std of x @ W_k for x ~ N(0, 1), W_k ~ N(0, 0.02^2), d = 768


def decode_algorithmic(wl, batch: int, ctx: int) -> dict:
    """Bytes the decode attention must move: the K and V cache rows of positions 0..ctx of every
    (sequence, group), read once (the queries, partials and outputs are a few hundred KB)."""
    es = 2 if wl.dtype == "bf16" else 4
    kv = 2.0 * batch * wl.num_kv_heads * (ctx + 1) * wl.dh * es
    return dict(attention_bytes=kv)


def run_decode(name: str, steps: int, warmup: int, gqa: bool = False, profile: bool = True):
    """Decode steps at a fixed position (the new token at position ctx; each step rewrites the same
    cache slot with the same values): wall time per step and per-kernel HIP-event durations."""
    import torch
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.inputs import WORKLOADS, gqa_of
    from sparse_moe_query_amd.runner import build_layer
    base, batch, ctx = DECODE_WORKLOADS[name]
    wl = WORKLOADS[base].with_(name=name, batch=batch, seq=1)
    if gqa:
        wl = gqa_of(wl)
    layer, x, _ = build_layer(wl)          # x [batch, 1, d]: the new tokens
    x = x.reshape(batch, wl.dim)
    kc, vc = layer.kv_cache(batch, ctx + 64)
    gen = torch.Generator(device=x.device)
    gen.manual_seed(1234)
    kc.normal_(0.0, KV_STD, generator=gen)
    vc.normal_(0.0, KV_STD, generator=gen)
    pos = torch.full((batch,), ctx, dtype=torch.int32, device=x.device)
    y = torch.empty_like(x)
    for _ in range(warmup):
        layer.decode(x, pos, kc, vc, y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer.decode(x, pos, kc, vc, y)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    kern, n = {}, 0
    if profile:
        gqe.gqe_profile_enable(layer.h, True)
        for _ in range(steps):
            layer.decode(x, pos, kc, vc, y)
        torch.cuda.synchronize()
        kern, n = gqe.gqe_profile_read_kernels(layer.h)
        gqe.gqe_profile_enable(layer.h, False)
    kernel_ms = {k: v / max(n, 1) for k, v in kern.items() if v > 0}
    assert torch.isfinite(y.float()).all(), "decode produced non-finite outputs"
    layer.close()
    del layer, x, y, kc, vc
    torch.cuda.empty_cache()
    return wl, batch, ctx, ms, kernel_ms


def decode_report(steps: int, warmup: int) -> dict:
    name = "decode_b64_ctx8192"
    log(f"[bench] {name}")
    wl, batch, ctx, ms, km = run_decode(name, steps, warmup)
    log(f"[bench] {name} gqa")
    _, _, _, g_ms, g_km = run_decode(name, steps, warmup, gqa=True)
    a = decode_algorithmic(wl, batch, ctx)
    att = km.get("decode_attention", 0.0) + km.get("decode_merge", 0.0)
    g_att = g_km.get("decode_attention", 0.0) + g_km.get("decode_merge", 0.0)
    gbs = a["attention_bytes"] / (att * 1e-3) / 1e9
    log(f"[bench] {name}: {ms:.3f} ms/step (GQA {g_ms:.3f}), attention {gbs:.0f} GB/s; kernels {km}")
    return dict(workload=name, batch=batch, cached_positions=ctx, ms_per_step=ms,
                tokens_s=batch / (ms / 1e3), kernel_ms=km,
                roofline=dict(bound="hbm", kernel="decode_attention", achieved=gbs, peak=PEAK_HBM,
                              unit="GB/s", frac=gbs / PEAK_HBM, kernel_ms=km.get("decode_attention", 0.0),
                              merge_ms=km.get("decode_merge", 0.0), algorithmic_bytes=a["attention_bytes"],
                              traffic=committed_traffic("decode_attention", name, "k_decode.hip")),
                gqa_ms_per_step=g_ms, gqa_kernel_ms=g_km, speedup_layer=g_ms / ms,
                speedup_attention=g_att / att if att > 0 else None)


def backward_flops(wl) -> float:
    """Multiply-add work of one backward pass, per the chain rule of the forward's contractions
    (2 flops per multiply-add): every forward GEMM appears twice (input and weight gradient), the
    causal attention five times over its S(S+1)/2 score entries per head (the recomputed scores,
    the log-sum-exp pass, do . v, dq, dk and dv: 6 d_h-long products per entry, counted as 6)."""
    alg = algorithmic(wl)
    dh, B, S = wl.dh, wl.batch, wl.seq
    H = wl.num_kv_heads * wl.top_k + (1 if wl.shared_head else 0)
    att = 2.0 * dh * H * B * S * (S + 1) / 2.0 * 6
    return 2 * (alg["projection"]["flops"] + alg["combine"]["flops"]) + att


def run_backward(wl, steps, warmup, aux_coef=0.01):
    """Forward once, then backward passes of sum(dy * y) + aux_coef * aux on the stored forward."""
    import numpy as np
    import torch
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.runner import build_layer
    layer, x, _ = build_layer(wl)
    gen = torch.Generator(device=x.device)
    gen.manual_seed(4321)
    dy = torch.empty_like(x).normal_(0.0, 1.0, generator=gen)
    layer(x)
    for _ in range(warmup):
        layer.backward(x, dy, aux_coef)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g = layer.backward(x, dy, aux_coef)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gqe.gqe_profile_enable(layer.h, True)
    for _ in range(steps):
        layer.backward(x, dy, aux_coef)
    torch.cuda.synchronize()
    kern, n = gqe.gqe_profile_read_kernels(layer.h)
    gqe.gqe_profile_enable(layer.h, False)
    km = {k: v / max(n, 1) for k, v in kern.items() if v > 0}
    finite = all(bool(torch.isfinite(v).all()) for v in g.values())
    layer.close()
    del layer, x, dy, g
    torch.cuda.empty_cache()
    return ms, km, finite


def backward_stage_flops(wl) -> dict:
    """Algorithmic flops of each timed backward stage (2 per multiply-add).  output: the per-slot
    projections dy W_slot^T (the combine's contraction once); weights: every forward GEMM's weight
    gradient (projection and combine contractions once each); dx: the projections' input gradient;
    attention: six d_h-long products per causal score entry and head."""
    alg = algorithmic(wl)
    dh, B, S = wl.dh, wl.batch, wl.seq
    H = wl.num_kv_heads * wl.top_k + (1 if wl.shared_head else 0)
    pr, cb = alg["projection"]["flops"], alg["combine"]["flops"]
    return {"backward_output": cb, "backward_attention": 2.0 * dh * H * B * S * (S + 1) / 2.0 * 6,
            "backward_weights": pr + cb, "backward_dx": pr}


def backward_report(steps: int, warmup: int) -> dict:
    from sparse_moe_query_amd.inputs import WORKLOADS
    wl = WORKLOADS["main_b8_s2048"]
    log("[bench] backward main_b8_s2048")
    ms, km, finite = run_backward(wl, steps, warmup)
    fl = backward_flops(wl)
    tf = fl / (ms * 1e-3) / 1e12
    # bf16 layers: every stage is matrix-core work except the router's float32 pieces
    peak = PEAK_BF16 if wl.dtype == "bf16" else PEAK_FP32
    bound = "mfma" if wl.dtype == "bf16" else "alu"
    stages = {}
    for k, f in backward_stage_flops(wl).items():
        if k in km:
            a = f / (km[k] * 1e-3) / 1e12
            stages[k] = dict(bound=bound, achieved=a, peak=peak, unit="TFLOP/s", frac=a / peak, flops=f, ms=km[k])
    dom = max(stages, key=lambda k: stages[k]["ms"]) if stages else None
    log(f"[bench] backward: {ms:.3f} ms ({tf:.1f} TFLOP/s overall); kernels {km}")
    roof = dict(stages[dom], kernel=dom) if dom else None
    return dict(workload=wl.name, ms=ms, tokens_s=wl.tokens / (ms / 1e3), kernel_ms=km, finite=finite,
                aux_coef=0.01, flops=fl, tflops=tf, stages=stages, roofline=roof)


def moe_flops(wl) -> dict:
    """Algorithmic flops of the MoE-MLP's expert products (2 per multiply-add, only the chosen
    experts' rows): up = T k d d_ff, down = T k d_ff d."""
    f = 2.0 * wl.tokens * wl.top_k * wl.dim * wl.d_ff
    return {"moe_up": f, "moe_down": f}


def run_moe(wl, steps, warmup):
    """Forwards of the MoE-MLP layer on resident inputs: ms per forward (device-synchronised wall
    clock over `steps`), then the same number with per-kernel HIP events."""
    import torch
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.runner import build_moe
    layer, x, _ = build_moe(wl)
    y = torch.empty_like(x)
    for _ in range(warmup):
        layer(x, y)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer(x, y)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gqe.gqe_moe_profile_enable(layer.h, True)
    for _ in range(steps):
        layer(x, y)
    torch.cuda.synchronize()
    kern, n = gqe.gqe_moe_profile_read_kernels(layer.h)
    gqe.gqe_moe_profile_enable(layer.h, False)
    km = {k: v / max(n, 1) for k, v in kern.items() if v > 0}
    st = layer.stats()
    layer.close()
    return ms, km, st


def moe_report(steps: int, warmup: int) -> dict:
    """The top-k MoE-MLP (2 of 8 experts, d 768, d_ff 3072, 16384 tokens) and its skewed
    16-expert variant: time per forward, tokens/s, expert-product rooflines (bf16 matrix core)."""
    from sparse_moe_query_amd.inputs import MOE_WORKLOADS
    out = {}
    for name in ("moe_e8_k2_t16384", "moe_skew_e16_k2_t4096"):
        wl = MOE_WORKLOADS[name]
        log(f"[bench] {name}")
        ms, km, st = run_moe(wl, steps, warmup)
        fl = moe_flops(wl)
        kr = {}
        for k, f in fl.items():
            if k in km:
                a = f / (km[k] * 1e-3) / 1e12
                kr[k] = dict(bound="mfma", achieved=a, peak=PEAK_BF16, unit="TFLOP/s", frac=a / PEAK_BF16,
                             flops=f, kernel_ms=km[k], traffic=committed_traffic(k, name, "k_moe.hip"))
        dom = max(kr, key=lambda k: kr[k]["kernel_ms"]) if kr else None
        share = (st["counts"] / max(1, wl.tokens * wl.top_k)).tolist()
        out[name] = dict(ms=ms, tokens_s=wl.tokens / (ms / 1e3), kernel_ms=km,
                         tflops=sum(fl.values()) / (ms * 1e-3) / 1e12,
                         roofline=dict(kr[dom], kernel=dom) if dom else None, kernels=kr,
                         expert_share=share, aux=st["aux"],
                         config=dict(dim=wl.dim, num_experts=wl.num_experts, top_k=wl.top_k, d_ff=wl.d_ff,
                                     tokens=wl.tokens, activation=wl.activation,
                                     router_bias_first=wl.router_bias_first))
        log(f"[bench] {name}: {ms:.3f} ms, kernels {km}")
    return out


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_seconds(wl, b: int = 0) -> float:
    """Wall-clock seconds of the oracle forward of sequence b of the workload (all its tokens;
    input generation excluded)."""
    from oracle import gqe_oracle as go
    from sparse_moe_query_amd.inputs import make_inputs
    inp = make_inputs(wl)
    cfg = go.OracleConfig(wl.dim, wl.num_query_experts, wl.num_kv_heads, wl.top_k, wl.dh,
                          wl.variant, wl.shared_head, wl.shared_kv_group)
    x = inp["x"].reshape(wl.batch, wl.seq, wl.dim)
    t0 = time.perf_counter()
    go.forward(cfg, 1, wl.seq, x[b % wl.batch], inp)
    return time.perf_counter() - t0


def cpu_baseline(wl, min_seconds=10.0):
    """The oracle as it stands, on whole sequences of the workload (all of their tokens), repeated
    over the batch until at least ``min_seconds`` of CPU work have been timed; then the per-config
    plan on bounded samples (one whole sequence per run): the tiny float32 layer as the median of 3
    runs; the skewed k = 2 layer and each ablation variant once (a median of 3 at these lengths
    would add minutes of CPU time to every run)."""
    from oracle import gqe_oracle as go
    from sparse_moe_query_amd.inputs import WORKLOADS, make_inputs
    inp = make_inputs(wl)
    cfg = go.OracleConfig(wl.dim, wl.num_query_experts, wl.num_kv_heads, wl.top_k, wl.dh,
                          wl.variant, wl.shared_head, wl.shared_kv_group)
    go.build(force=False)
    x = inp["x"].reshape(wl.batch, wl.seq, wl.dim)
    done, elapsed, b = 0, 0.0, 0
    while elapsed < min_seconds:
        t0 = time.perf_counter()
        go.forward(cfg, 1, wl.seq, x[b % wl.batch], inp)
        elapsed += time.perf_counter() - t0
        done += wl.seq
        b += 1
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    plan = {}
    for name, runs in (("tiny_fp32", 3), ("k2_skew_b4_s4096", 1), ("ablation_gqe_b2_s8192", 1),
                       ("ablation_weighted_b2_s8192", 1), ("ablation_hard_b2_s8192", 1)):
        w = WORKLOADS[name]
        t = sorted(_oracle_seconds(w, r) for r in range(runs))[runs // 2]
        plan[name] = dict(tokens_s=w.seq / t, seconds_per_sequence=t, runs=runs, seq=w.seq)
    return dict(value=done / elapsed, unit="tokens/s", cores=threads, kind="oracle",
                sample=f"{b} whole sequences of the workload (seq {wl.seq}, all tokens, cycling over its "
                       f"batch of {wl.batch}), fp64 plain loops, {elapsed:.1f} s",
                cpu_model=cpu_model(), per_config=plan)


def config_report(steps: int) -> dict:
    """The skewed k = 2 layer and the three output variants of the ablation sweep, each timed as
    the main workload is, beside the all-active GQA run of the same kernels on the same inputs
    (the ablation variants share their weights, so one GQA run serves the three)."""
    from sparse_moe_query_amd.inputs import WORKLOADS, gqa_of
    out = {}
    gqa_cache = {}
    for name in ("k2_skew_b4_s4096", "ablation_gqe_b2_s8192", "ablation_weighted_b2_s8192", "ablation_hard_b2_s8192"):
        wl = WORKLOADS[name]
        log(f"[bench] {name}")
        ms, kern, _ = run_workload(wl, steps, 2)
        g = gqa_of(wl)
        key = (g.dim, g.seed, g.batch, g.seq, g.head_dim, g.top_k)
        if key not in gqa_cache:
            log(f"[bench] {name} gqa")
            gqa_cache[key] = run_workload(g, steps, 2)[:2]
        g_ms, g_kern = gqa_cache[key]
        a = algorithmic(wl)
        at = a["attention"]["flops"] / (attn_step_ms(kern) * 1e-3) / 1e12
        out[name] = dict(tokens_s=wl.tokens / (ms / 1e3), ms=ms, kernel_ms=kern, layer_gflop=a["layer_flops"] / 1e9,
                         layer_tflops=a["layer_flops"] / (ms * 1e-3) / 1e12, attn_tflops=at,
                         attn_frac_peak=at / PEAK_BF16, gqa_ms=g_ms, gqa_kernel_ms=g_kern,
                         speedup_layer=g_ms / ms, speedup_attention=attn_step_ms(g_kern) / attn_step_ms(kern))
        log(f"[bench] {name}: {ms:.3f} ms (GQA {g_ms:.3f} ms), attn {at:.0f} TFLOP/s")
    return out


def copy_calibration(nbytes=256 << 20, reps=3):
    """A plain device copy of known size, for scaling the HBM byte counters of a profiled run."""
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").normal_()
    b = torch.empty_like(a)
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"[bench] copy calibration: {reps} copies of {nbytes} bytes (read {nbytes}, write {nbytes})")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-moe", action="store_true")
    ap.add_argument("--only-main", action="store_true", help="main workload only (for profilers)")
    ap.add_argument("--profile-workload", default=None,
                    help="run only this named workload (inputs.WORKLOADS, or NAME_gqa for its "
                         "all-active GQA baseline) for --steps forwards; for profilers")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="with --profile-workload: also run a plain 256 MiB device copy")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU: this build has no multi-GPU path (asked for {args.gpus}).",
              file=sys.stderr)
        sys.exit(2)
    if os.environ.get("WORLD_SIZE", "1") != "1":
        print("bench.py runs as a single process on one GPU.", file=sys.stderr)
        sys.exit(2)

    import torch
    from sparse_moe_query_amd.inputs import WORKLOADS, gqa_of

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    if args.profile_workload in DECODE_WORKLOADS or (args.profile_workload or "")[:-4] in DECODE_WORKLOADS:
        name = args.profile_workload
        gqa = name.endswith("_gqa")
        if args.copy_calibration:
            copy_calibration()
        wl, _, _, ms, kernel_ms = run_decode(name[:-4] if gqa else name, args.steps, args.warmup, gqa=gqa)
        print(json.dumps({"workload": wl.name, "ms_per_step": ms, "kernel_ms": kernel_ms,
                          "source_hash": source_hash("k_decode.hip")}), flush=True)
        return
    from sparse_moe_query_amd.inputs import MOE_WORKLOADS
    if args.profile_workload in MOE_WORKLOADS:
        if args.copy_calibration:
            copy_calibration()
        ms, km, _ = run_moe(MOE_WORKLOADS[args.profile_workload], args.steps, args.warmup)
        print(json.dumps({"workload": args.profile_workload, "ms_per_step": ms, "kernel_ms": km,
                          "source_hash": source_hash("k_moe.hip")}), flush=True)
        return
    if args.profile_workload == "backward_main_b8_s2048":
        if args.copy_calibration:
            copy_calibration()
        ms, km, _ = run_backward(WORKLOADS["main_b8_s2048"], args.steps, args.warmup)
        print(json.dumps({"workload": args.profile_workload, "ms_per_step": ms, "kernel_ms": km,
                          "source_hash": source_hash("k_backward.hip")}), flush=True)
        return
    if args.profile_workload:
        name = args.profile_workload
        wl = gqa_of(WORKLOADS[name[:-4]]) if name.endswith("_gqa") else WORKLOADS[name]
        if args.copy_calibration:
            copy_calibration()
        ms, kernel_ms, _ = run_workload(wl, args.steps, args.warmup)
        print(json.dumps({"workload": wl.name, "ms_per_step": ms, "kernel_ms": kernel_ms,
                          "source_hash": {k: source_hash(v[0]) for k, v in KERNEL_SOURCES.items()}}),
              flush=True)
        return
    main_wl = WORKLOADS["main_b8_s2048"]
    log(f"[bench] main workload {main_wl.name}: warmup {args.warmup}, steps {args.steps}")
    ms, kernel_ms, path = run_workload(main_wl, args.steps, args.warmup)
    alg = algorithmic(main_wl)
    tokens_s = main_wl.tokens / (ms / 1e3)
    stage_ms = stages_of(kernel_ms)
    log(f"[bench] {ms:.3f} ms/step, {tokens_s:.3e} tokens/s; kernels (ms) {kernel_ms}")
    dom = max(KERNEL_SOURCES, key=lambda k: kernel_ms.get(k, 0.0))
    mrg = lambda k: kernel_ms.get("attention_merge", 0.0) if k == "attention" else 0.0
    rl = roofline(dom, kernel_ms[dom], alg, main_wl.name, mrg(dom))
    kernels = {k: roofline(k, kernel_ms[k], alg, main_wl.name, mrg(k)) for k in KERNEL_SOURCES if kernel_ms.get(k, 0) > 0}
    kernels = {k: {kk: v[kk] for kk in ("kernel_ms", "achieved", "frac", "algorithmic_hbm_frac", "traffic")}
               for k, v in kernels.items()}
    for k in kernels:
        kernels[k]["mfma_busy"] = committed_mfma_busy(k, main_wl.name)

    result = {
        "metric": "GQE prefill tokens/s + attn TFLOP/s (% MFMA peak), d=768 N=16 G=8 k=1",
        "value": tokens_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) x, N(0,0.02^2) weights, router logits ~ N(0,1))",
        "config": {"workload": main_wl.name, "dim": 768, "num_query_experts": 16, "num_kv_heads": 8,
                   "top_k": 1, "head_dim": 48, "shared_head": True, "variant": "gqe", "batch": 8,
                   "seq": 2048, "causal": True, "matrix_core_stages": path},
        "roofline": rl,
        "attn_tflops": alg["attention"]["flops"] / (attn_step_ms(kernel_ms) * 1e-3) / 1e12,
        "kernels": kernels,
        "stage_ms": stage_ms,
    }
    result["attn_frac_peak"] = result["attn_tflops"] / PEAK_BF16

    if not args.only_main:
        # the all-active GQA baseline at the main setting
        g_ms, g_kern, _ = run_workload(gqa_of(main_wl), args.steps, args.warmup)
        result["main_gqa"] = dict(ms_per_step=g_ms, speedup_layer=g_ms / ms,
                                  speedup_attention=attn_step_ms(g_kern) / attn_step_ms(kernel_ms))
    if not args.no_long and not args.only_main:
        long = {}
        for name, steps in (("long_s16384", max(5, args.steps // 3)), ("long_s32768", max(3, args.steps // 6))):
            wl = WORKLOADS[name]
            log(f"[bench] {name}")
            l_ms, l_kern, _ = run_workload(wl, steps, 2)
            log(f"[bench] {name} gqa")
            g_ms, g_kern, _ = run_workload(gqa_of(wl), steps, 2)
            a = algorithmic(wl)
            ga = algorithmic(gqa_of(wl))
            at = a["attention"]["flops"] / (attn_step_ms(l_kern) * 1e-3) / 1e12
            gat = ga["attention"]["flops"] / (attn_step_ms(g_kern) * 1e-3) / 1e12
            long[name] = dict(tokens_s=wl.tokens / (l_ms / 1e3), ms=l_ms, kernel_ms=l_kern,
                              attn_tflops=at, attn_frac_peak=at / PEAK_BF16,
                              attn_mfma_busy=committed_mfma_busy("attention", name),
                              gqa_ms=g_ms, gqa_kernel_ms=g_kern, gqa_attn_tflops=gat,
                              speedup_layer=g_ms / l_ms,
                              speedup_attention=attn_step_ms(g_kern) / attn_step_ms(l_kern))
            log(f"[bench] {name}: {l_ms:.3f} ms (GQA {g_ms:.3f} ms) attn {at:.0f} TFLOP/s")
        result["long_context"] = long
    if not args.no_long and not args.only_main:
        result["configs"] = config_report(max(5, args.steps // 3))
    if not args.no_decode and not args.only_main:
        result["decode"] = decode_report(max(10, args.steps), args.warmup)
    if not args.no_moe and not args.only_main:
        result["moe_mlp"] = moe_report(max(10, args.steps), args.warmup)
    if not args.no_backward and not args.only_main:
        result["backward"] = backward_report(3, 1)
    if not args.no_cpu and not args.only_main:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(main_wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
