#!/usr/bin/env python3
"""Throughput of the POET-X layer hot path on one GPU.

One step = CNP build of R and P, forward, backward to dq_R / dq_P / dx, and
(for the Llama-8B MLP up-projection workload) one merge W0 <- R W0 P followed
by the permuted-frame weight rebuild, all on synthetic seeded inputs already
resident in HBM. Prints one JSON line on stdout; progress goes to stderr.

The dominant kernel's roofline fraction comes from HIP events recorded by the
library around each of its steps inside the timed region; the CPU baseline is
the float64 oracle timed on a bounded token sample of the same workload.
"""

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "POET-X layer fwd+bwd tokens/s at Llama-8B shapes; % of MFMA/HBM peak on 1 GPU"
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(cfg, seconds_hint=20.0):
    """Time the float64 oracle on token samples of the workload and extrapolate
    linearly in T (the oracle's cost is a fixed part - CNP maps, their
    adjoints, the merge - plus a part proportional to the token count)."""
    import numpy as np
    import oracle as O
    from orthogonal_equivalence_amd import synth
    try:
        import threadpoolctl
        threads = max((i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()), default=1)
    except Exception:  # pragma: no cover - informational only
        threads = os.cpu_count() or 1
    L = synth.make_layer(cfg, 0)
    W0 = O.dequantize(L["W0_raw"], L["w_scale"]) if cfg.weight == "i8" else L["W0"].astype(np.float64)
    args = (W0, L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], cfg.b_r, cfg.b_p)
    t_small, t_big = 256, 512
    times = {}
    for T in (t_small, t_big):
        A = synth.make_activations(cfg, 0, T=T)
        t0 = time.perf_counter()
        O.backward(A["X"], A["dZ"], *args)   # includes the forward
        times[T] = time.perf_counter() - t0
        log(f"[cpu_baseline] oracle fwd+bwd on {T} tokens: {times[T]:.2f} s")
    t_merge = 0.0
    if cfg.merge:
        t0 = time.perf_counter()
        O.merge(*args)
        t_merge = time.perf_counter() - t0
        log(f"[cpu_baseline] oracle merge: {t_merge:.2f} s")
    per_tok = max((times[t_big] - times[t_small]) / (t_big - t_small), 0.0)
    fixed = max(times[t_small] - per_tok * t_small, 0.0)
    step = fixed + per_tok * cfg.T + t_merge
    return {
        "value": cfg.T / step,
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "sample": (f"float64 oracle fwd+bwd on {t_small} and {t_big} tokens of the {cfg.name} workload"
                   f"{' plus one full merge' if cfg.merge else ''}, extrapolated linearly in T to "
                   f"{cfg.T} tokens ({step:.1f} s per step; {sum(times.values()) + t_merge:.1f} s measured)"),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="llama8b_mlp_up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-yardstick", action="store_true")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs the layer on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the multi-GPU path (data parallel over token shards with one all-reduce of the packed "
              "gradients) is not part of this build", file=sys.stderr)
        sys.exit(2)

    import torch
    from orthogonal_equivalence_amd import synth
    from orthogonal_equivalence_amd import poetx as px
    from orthogonal_equivalence_amd.device import DeviceLayer, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    cfg = synth.CONFIGS[args.workload]
    log(f"[bench] workload {cfg.name}: T={cfg.T} m={cfg.m} n={cfg.n} b={cfg.b_r}/{cfg.b_p} "
        f"{cfg.act}/{cfg.weight} merge={cfg.merge}")
    L = synth.make_layer(cfg, 0)
    A = synth.make_activations(cfg, 0)
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, cfg.T)
    dl.load(L)
    x = to_device(A["X_raw"], cfg.act)
    dz = to_device(A["dZ_raw"], cfg.act)
    del A
    z = dl.act_tensor(cfg.T, cfg.n)
    dx = dl.act_tensor(cfg.T, cfg.m)
    dq_r = torch.empty_like(dl.q_r)
    dq_p = torch.empty_like(dl.q_p)
    dl.prepare()

    def step():
        dl.cnp_build()
        dl.forward(x, z)
        dl.backward(dz, dq_r, dq_p, dx)
        if cfg.merge:
            dl.merge()
            dl.prepare()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")

    stream = torch.cuda.current_stream()
    px.poetx_profile_enable(1)
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    px.poetx_profile_enable(0)
    per = {}
    for i in range(px.poetx_profile_count()):
        name, ms = px.poetx_profile_get(i)
        s = per.setdefault(name, [0.0, 0])
        s[0] += ms
        s[1] += 1
    ms_step = ms_total / args.steps
    log(f"[bench] {args.steps} timed steps: {ms_step:.3f} ms/step")
    kernels = {k: round(v[0] / v[1], 4) for k, v in sorted(per.items())}
    log("[bench] per-step breakdown (ms): " + json.dumps(kernels))

    flops_gemm = 2.0 * cfg.T * cfg.m * cfg.n
    g = [per[k] for k in ("gemm_dense_fwd", "gemm_dense_bwd") if k in per]
    g_ms = sum(v[0] for v in g) / max(sum(v[1] for v in g), 1)
    bf16 = cfg.act == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    achieved = flops_gemm / (g_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": None,
                "kernel": "dense W0 product (gemm_dense_fwd and gemm_dense_bwd launches)",
                "flops_per_launch": flops_gemm, "avg_launch_ms": round(g_ms, 4)}

    fwd_bwd_names = [k for k in per if k.startswith(("cnp_build", "gather", "apply", "gemm", "scatter",
                                                     "grad", "cnp_bwd"))]
    ms_fwd_bwd = sum(per[k][0] for k in fwd_bwd_names) / args.steps
    ms_merge = sum(per[k][0] for k in per if k.startswith(("merge", "prepare"))) / args.steps

    yard = None
    if not args.no_yardstick and bf16:
        # the same shape through torch.nn.functional.linear (hipBLASLt), fwd + bwd with dW
        w = torch.randn(cfg.n, cfg.m, dtype=torch.bfloat16, device="cuda", requires_grad=True)
        xi = x.detach().clone().requires_grad_(True)
        for it in range(8):
            if it == 3:
                torch.cuda.synchronize()
                e0 = torch.cuda.Event(enable_timing=True)
                e1 = torch.cuda.Event(enable_timing=True)
                e0.record()
            out = torch.nn.functional.linear(xi, w)
            out.backward(dz)
        e1.record()
        torch.cuda.synchronize()
        yard = round(e0.elapsed_time(e1) / 5, 4)
        del w, xi, out

    line = {
        "metric": METRIC,
        "value": round(cfg.T / (ms_step * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if bf16 else "f32",
        "data": "synthetic (seeded N(0,1) activations, N(0,0.02^2) weight, N(0,1e-3^2) packed skew params)",
        "config": {"workload": cfg.name, "tokens": cfg.T, "m": cfg.m, "n": cfg.n, "b_r": cfg.b_r,
                   "b_p": cfg.b_p, "weight": cfg.weight,
                   "step": "cnp_build+forward+backward" + ("+merge+weight_prepare" if cfg.merge else "")},
        "roofline": roofline,
        "cpu_baseline": None,
        "fwd_bwd_ms": round(ms_fwd_bwd, 4),
        "fwd_bwd_tokens_per_s": round(cfg.T / (ms_fwd_bwd * 1e-3), 1),
        "merge_prepare_ms": round(ms_merge, 4),
        "tokens_per_s_merge_every_200": round(cfg.T / ((ms_fwd_bwd + ms_merge / 200) * 1e-3), 1),
        "kernels_ms": kernels,
        "torch_linear_fwd_bwd_ms": yard,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
