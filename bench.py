"""Benchmark of the GQE forward (prefill) pass on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu] [--no-long] [--only-main]

One step = one gqe_forward over the main-setting workload (dim 768, N=16, G=8, k=1, head_dim 48,
shared head, variant gqe, batch 8 x seq 2048, bf16) with x and the packed weights resident in HBM.
Prints ONE JSON line (stdout): tokens/s of that workload, the roofline of its dominant kernel
(stage times from HIP events recorded on the forward's stream during the timed steps), the CPU
oracle timed on a bounded sample, and -- as extra fields -- the long-context runs (seq 16384 and
32768) with the all-active GQA baseline on the same inputs and kernels.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16 = 2500.0   # TFLOP/s, MI355X dense bf16 matrix
PEAK_FP64 = 78.6     # TFLOP/s, MI355X fp64 vector
PEAK_HBM = 8000.0    # GB/s


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def algorithmic(wl) -> dict:
    """Algorithmic work of one forward, per stage: flops (active heads only) and HBM bytes
    (each tensor read or written once, bf16 = 2 bytes)."""
    T, d, N, G, dh = wl.tokens, wl.dim, wl.num_query_experts, wl.num_kv_heads, wl.dh
    k = wl.top_k
    H = G * k + (1 if wl.shared_head else 0)
    B, S = wl.batch, wl.seq
    es = 2 if wl.dtype == "bf16" else 4
    slots = N if wl.dense_gqa else G * k + (G if wl.variant == "gqe" else 0) + (1 if wl.shared_head else 0)
    gk = G * k
    out = {
        "router": dict(flops=0.0 if wl.dense_gqa else 2.0 * T * d * N,
                       bytes=0.0 if wl.dense_gqa else T * d * es + T * gk * 12.0),
        "projection": dict(flops=2.0 * T * d * dh * (2 * G + H),
                           bytes=T * d * es + d * dh * (2 * G + (N if wl.dense_gqa else N + (1 if wl.shared_head else 0))) * es
                           + T * (H + 2 * G) * dh * es),
        "attention": dict(flops=4.0 * dh * H * B * S * (S + 1) / 2.0,
                          bytes=(B * H * S * dh + 2 * B * G * S * dh + T * H * dh) * es),
        "combine": dict(flops=2.0 * T * d * dh * slots,
                        bytes=(T * H * dh + T * d) * es + d * dh * (N + G + 1) * es + T * gk * 12.0),
    }
    out["layer_flops"] = sum(v["flops"] for v in out.values() if isinstance(v, dict))
    return out


def run_workload(wl, steps, warmup, profile=True):
    import torch
    from sparse_moe_query_amd import gqe
    from sparse_moe_query_amd.runner import build_layer
    layer, x, _ = build_layer(wl)
    y = torch.empty_like(x)
    for _ in range(warmup):
        layer(x, y)
    torch.cuda.synchronize()
    if profile:
        gqe.gqe_profile_enable(layer.h, True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        layer(x, y)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    stages, n = (gqe.gqe_profile_read(layer.h) if profile else ({}, 0))
    if profile:
        gqe.gqe_profile_enable(layer.h, False)
    ms = (t1 - t0) * 1e3 / steps
    stage_ms = {k: v / max(n, 1) for k, v in stages.items()}
    path = layer.intermediates(wl.batch, wl.seq)["matrix_core"]
    layer.close()
    del layer, x, y
    torch.cuda.empty_cache()
    return ms, stage_ms, path


def cpu_baseline(wl):
    """The oracle as it stands, on one sequence of the workload (all of its tokens)."""
    from oracle import gqe_oracle as go
    from sparse_moe_query_amd.inputs import make_inputs
    one = wl.with_(batch=1)
    inp = make_inputs(one)
    cfg = go.OracleConfig(one.dim, one.num_query_experts, one.num_kv_heads, one.top_k, one.dh,
                          one.variant, one.shared_head, one.shared_kv_group)
    go.build(force=False)
    t0 = time.perf_counter()
    go.forward(cfg, 1, one.seq, inp["x"], inp)
    t1 = time.perf_counter()
    threads = int(os.environ.get("OMP_NUM_THREADS", len(os.sched_getaffinity(0))))
    return dict(value=one.tokens / (t1 - t0), unit="tokens/s", cores=threads, kind="oracle",
                sample=f"one sequence of the workload: batch 1 x seq {one.seq} (all tokens), "
                       f"fp64 plain loops, {t1 - t0:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-long", action="store_true")
    ap.add_argument("--only-main", action="store_true", help="main workload only (for profilers)")
    ap.add_argument("--profile-workload", default=None,
                    help="run only this named workload (inputs.WORKLOADS, or NAME_gqa for its "
                         "all-active GQA baseline) for --steps forwards; for profilers")
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
    if args.profile_workload:
        name = args.profile_workload
        wl = gqa_of(WORKLOADS[name[:-4]]) if name.endswith("_gqa") else WORKLOADS[name]
        ms, stage_ms, _ = run_workload(wl, args.steps, args.warmup)
        print(json.dumps({"workload": wl.name, "ms_per_step": ms, "stage_ms": stage_ms}), flush=True)
        return
    main_wl = WORKLOADS["main_b8_s2048"]
    log(f"[bench] main workload {main_wl.name}: warmup {args.warmup}, steps {args.steps}")
    ms, stage_ms, path = run_workload(main_wl, args.steps, args.warmup)
    alg = algorithmic(main_wl)
    tokens_s = main_wl.tokens / (ms / 1e3)
    dom = max(stage_ms, key=lambda k: stage_ms[k])
    log(f"[bench] {ms:.3f} ms/step, {tokens_s:.3e} tokens/s; stages (ms) {stage_ms}")

    def roof(stage, sms, a):
        f = a[stage]["flops"] / (sms * 1e-3) / 1e12
        if stage == "router":
            return dict(bound="alu", achieved=f, peak=PEAK_FP64, unit="TFLOP/s", frac=f / PEAK_FP64)
        return dict(bound="mfma", achieved=f, peak=PEAK_BF16, unit="TFLOP/s", frac=f / PEAK_BF16)

    roofline = roof(dom, stage_ms[dom], alg)
    roofline["kernel"] = dom
    roofline["traffic"] = None
    stages = {k: dict(ms=v, **{kk: vv for kk, vv in roof(k, v, alg).items() if kk in ("achieved", "frac", "bound")})
              for k, v in stage_ms.items() if v > 0}

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
        "roofline": roofline,
        "attn_tflops": alg["attention"]["flops"] / (stage_ms["attention"] * 1e-3) / 1e12,
        "stages": stages,
    }
    result["attn_frac_peak"] = result["attn_tflops"] / PEAK_BF16

    if not args.only_main:
        # the all-active GQA baseline at the main setting
        g_ms, g_stage, _ = run_workload(gqa_of(main_wl), args.steps, args.warmup)
        result["main_gqa"] = dict(ms_per_step=g_ms, speedup_layer=g_ms / ms,
                                  speedup_attention=g_stage["attention"] / stage_ms["attention"])
    if not args.no_long and not args.only_main:
        long = {}
        for name, steps in (("long_s16384", max(5, args.steps // 3)), ("long_s32768", max(3, args.steps // 6))):
            wl = WORKLOADS[name]
            log(f"[bench] {name}")
            l_ms, l_stage, _ = run_workload(wl, steps, 2)
            log(f"[bench] {name} gqa")
            g_ms, g_stage, _ = run_workload(gqa_of(wl), steps, 2)
            a = algorithmic(wl)
            ga = algorithmic(gqa_of(wl))
            at = a["attention"]["flops"] / (l_stage["attention"] * 1e-3) / 1e12
            gat = ga["attention"]["flops"] / (g_stage["attention"] * 1e-3) / 1e12
            long[name] = dict(tokens_s=wl.tokens / (l_ms / 1e3), ms=l_ms, stage_ms=l_stage,
                              attn_tflops=at, attn_frac_peak=at / PEAK_BF16,
                              gqa_ms=g_ms, gqa_stage_ms=g_stage, gqa_attn_tflops=gat,
                              speedup_layer=g_ms / l_ms,
                              speedup_attention=g_stage["attention"] / l_stage["attention"])
            log(f"[bench] {name}: {l_ms:.3f} ms (GQA {g_ms:.3f} ms) attn {at:.0f} TFLOP/s")
        result["long_context"] = long
    if not args.no_cpu and not args.only_main:
        log("[bench] cpu baseline (oracle)")
        result["cpu_baseline"] = cpu_baseline(main_wl)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
