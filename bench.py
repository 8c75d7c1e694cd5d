#!/usr/bin/env python3
"""Throughput of the POET-X layer hot path on one GPU.

One step = CNP build of R and P, forward, backward to dq_R / dq_P / dx, and
(for the Llama-8B MLP up-projection workload) one merge cycle: new draws of
both permutations and W0 <- R W0 P written into their frame, all on
synthetic seeded inputs already resident in HBM. Prints one JSON line on
stdout; progress goes to stderr.

The step time comes from a timed pass of K steps with nothing else on the
stream. A second timed pass of K steps runs with the library's HIP-event log
on (an event pair on the launch stream around each of its kernel steps); the
dominant kernel's roofline fraction and the per-kernel table come from it.
Further passes, timed the same way: the step without its merge cycle (the
forward + backward throughput and, with the difference, the merge cycle's
wall-clock cost), the memory variant, and the step of every other workload.
The CPU baseline is the float64 oracle timed on the same workload (whole, or
a token sample when the whole would take too long).
"""

import argparse
import dataclasses
import itertools
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "POET-X layer fwd+bwd tokens/s at Llama-8B shapes; % of MFMA/HBM peak on 1 GPU"

# The pages' own figures, on an H100 (zhichai.net digest of arXiv:2603.05500):
# the CNP forward before and after its fused kernel, section "3. Cayley-Neumann
# 参数化优化", and the single-layer latency of POET-X fast, section "4. 定制 CUDA
# Kernel 层", for which neither the layer shape nor the passes timed are given.
# Reported as context beside the matching figures measured here, not as targets.
PAGES_H100 = {"cnp_forward_unfused_ms": 0.316, "cnp_forward_fused_ms": 0.107, "layer_latency_ms": 1.38}
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_F32_TFLOPS = 157.3     # MI355X dense fp32 MFMA
PEAK_HBM_GBS = 8000.0
MERGE_SEED = 2026  # seed of the permutation draws that follow each merge


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def cpu_baseline(cfg, budget_s=30.0):
    """Time the float64 oracle on the workload. Two token samples (256, 512)
    give its cost as a fixed part (CNP maps, their adjoints) plus a part
    proportional to the token count; if a whole step is predicted to fit the
    budget it is then run on all of the workload's tokens and that time is
    used, else the linear extrapolation is."""
    import numpy as np
    import oracle as O
    from orthogonal_equivalence_amd import synth
    blas = "unknown"
    try:
        import threadpoolctl
        info = threadpoolctl.threadpool_info()
        threads = max((i.get("num_threads", 1) for i in info), default=1)
        blas = ", ".join(sorted({f"{i.get('internal_api', '?')} {i.get('version', '')}".strip()
                                 for i in info if i.get("user_api") == "blas"})) or blas
    except Exception:  # pragma: no cover - informational only
        threads = os.cpu_count() or 1
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            cpu_model = next((ln.split(":", 1)[1].strip() for ln in fh if ln.startswith("model name")), cpu_model)
    except OSError:  # pragma: no cover - informational only
        pass
    L = synth.make_layer(cfg, 0)
    if cfg.weight in ("i8", "f8"):
        W0 = (O.dequantize if cfg.weight == "i8" else O.dequantize_fp8)(L["W0_raw"], L["w_scale"])
    else:
        W0 = L["W0"].astype(np.float64)
    args = (W0, L["q_r"], L["q_p"], L["perm_r"], L["perm_p"], cfg.b_r, cfg.b_p)

    def fwd_bwd(T):
        A = synth.make_activations(cfg, 0, T=T)
        t0 = time.perf_counter()
        O.backward(A["X"], A["dZ"], *args)   # includes the forward
        dt = time.perf_counter() - t0
        log(f"[cpu_baseline] oracle fwd+bwd on {T} tokens: {dt:.2f} s")
        return dt

    t_small, t_big = 256, 512
    times = {T: fwd_bwd(T) for T in (t_small, t_big)}
    t_merge = 0.0
    if cfg.merge:
        t0 = time.perf_counter()
        if cfg.weight in ("i8", "f8"):
            O.merge_xq(L["W0_raw"], L["w_scale"], *args[1:], fmt=cfg.weight)
        else:
            O.merge(*args)
        t_merge = time.perf_counter() - t0
        log(f"[cpu_baseline] oracle merge: {t_merge:.2f} s")
    per_tok = max((times[t_big] - times[t_small]) / (t_big - t_small), 0.0)
    fixed = max(times[t_small] - per_tok * t_small, 0.0)
    predicted = fixed + per_tok * cfg.T
    if predicted <= budget_s:
        t_full = fwd_bwd(cfg.T)
        step = t_full + t_merge
        sample = (f"float64 oracle fwd+bwd on all {cfg.T} tokens of the {cfg.name} workload"
                  f"{' plus one full merge' if cfg.merge else ''} ({step:.1f} s per step)")
    else:
        step = predicted + t_merge
        sample = (f"float64 oracle fwd+bwd on {t_small} and {t_big} tokens of the {cfg.name} workload"
                  f"{' plus one full merge' if cfg.merge else ''}, extrapolated linearly in T to "
                  f"{cfg.T} tokens ({step:.1f} s per step; {sum(times.values()) + t_merge:.1f} s measured)")
    return {"value": cfg.T / step, "unit": "tokens/s", "cores": int(threads), "kind": "oracle", "sample": sample,
            "cpu_model": cpu_model, "blas": blas}


GEMM_SOURCES = ("gemm_dense.hip", "gemm.hpp", "common.hpp")


def gemm_source_sha256():
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        with open(os.path.join(ROOT, "orthogonal_equivalence_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def measured_traffic(workload):
    """HBM bytes per dense-product launch from the committed counter summary
    (rocprofv3 FETCH_SIZE and WRITE_SIZE passes, each scaled by the same
    counter's reading for a plain copy of known size), or None when there is
    none for this workload or the kernel's sources changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"gemm_dense_hbm_traffic_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith(("#", " ")):
                k, v = line.split(":", 1)
                kv[k.strip()] = v.strip()
    if kv.get("kernel_source_sha256") != gemm_source_sha256():
        log(f"[bench] {os.path.basename(path)} was taken on other kernel sources; traffic not reported")
        return None
    try:
        return float(kv["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def algorithmic_work(cfg):
    """(bytes, flops) each profiled step must move / compute at the layer's
    shape: block-diagonal work only (never dense m x m or n x n rotations),
    one pass over each operand, one G plane per CNP block."""
    es = 4 if cfg.act == "f32" else 2
    wes = {"f32": 4, "bf16": 2, "i8": 1, "f8": 1}[cfg.weight]
    T, m, n, br, bp = cfg.T, cfg.m, cfg.n, cfg.b_r, cfg.b_p
    nr, np_ = -(-m // br), -(-n // bp)
    pr = nr * br * (br - 1) // 2
    pp = np_ * bp * (bp - 1) // 2
    blk = nr * br * br + np_ * bp * bp
    cube = nr * br ** 3 + np_ * bp ** 3
    dense = (2.0 * T * m * n, es * T * m + wes * m * n + es * T * n)
    w = {
        "cnp_build": (4 * (pr + pp) + es * blk, 4.0 * cube),
        "cnp_build_r": (4 * pr + es * nr * br * br, 4.0 * nr * br ** 3),
        "cnp_build_p": (4 * pp + es * np_ * bp * bp, 4.0 * np_ * bp ** 3),
        "gather_x": (2 * es * T * m, 0.0),
        "apply_r_fwd": (2 * es * T * m, 2.0 * T * m * br),
        "gemm_dense_fwd": (dense[1], dense[0]),
        "apply_p_fwd": (2 * es * T * n, 2.0 * T * n * bp),
        "scatter_z": (2 * es * T * n, 0.0),
        "gather_dz": (2 * es * T * n, 0.0),
        "apply_p_bwd": (2 * es * T * n, 2.0 * T * n * bp),
        "fold_h_bwd": (2 * wes * m * n, 2.0 * m * n * bp),
        "grad_h": (2 * es * T * n + 4 * np_ * bp * bp, 2.0 * T * n * bp),
        "gemm_dense_bwd": (dense[1], dense[0]),
        "apply_r_bwd": (2 * es * T * m, 2.0 * T * m * br),
        "grad_g": (2 * es * T * m + 4 * nr * br * br, 2.0 * T * m * br),
        "grad_gh": (2 * es * T * (m + n) + 4 * blk, 2.0 * T * (m * br + n * bp)),
        "scatter_dx": (2 * es * T * m, 0.0),
        "cnp_bwd": (4 * blk + 8 * (pr + pp), 10.0 * cube),
        "merge_left": (2 * wes * m * n, 2.0 * m * n * br),
        "merge_transpose": (2 * wes * m * n, 0.0),
        "merge_right": (2 * wes * m * n, 2.0 * m * n * bp),
        "merge_reframe": (2 * wes * m * n, 0.0),
    }
    return w


def kernel_roofline(cfg, per):
    """Per profiled step: time, algorithmic rates, the fraction of the binding
    roof, t_roof / t with t_roof = max(flops / MFMA peak, bytes / HBM peak), and
    the fractions of the HBM and of the MFMA peak separately."""
    peak_f = (PEAK_BF16_TFLOPS if cfg.act == "bf16" else PEAK_F32_TFLOPS) * 1e12
    peak_b = PEAK_HBM_GBS * 1e9
    work = algorithmic_work(cfg)
    out = {}
    for name, (tot, cnt) in sorted(per.items()):
        if name not in work or cnt == 0:
            continue
        nbytes, flops = work[name]
        t = tot / cnt * 1e-3
        t_roof = max(flops / peak_f, nbytes / peak_b)
        out[name] = {"ms": round(t * 1e3, 4), "bound": "mfma" if flops / peak_f > nbytes / peak_b else "hbm",
                     "GB/s": round(nbytes / t / 1e9, 1), "TFLOP/s": round(flops / t / 1e12, 1),
                     "frac": round(t_roof / t, 4), "frac_hbm": round(nbytes / t / peak_b, 4),
                     "frac_mfma": round(flops / t / peak_f, 4)}
    return out


# The other single-GPU workloads of the pages' Llama runs, timed as extra
# lines of the same report (the tiny float32 layer is launch-bound and left out).
OTHER_WORKLOADS = ("llama3b_proj", "llama13b_q_proj", "llama13b_down_proj", "xq_llama8b_mlp_up",
                   "xf8_llama8b_mlp_up")


def time_workload(cfg, steps, warmup):
    """ms per step (CNP build + forward + backward) of one workload on fresh
    device buffers, with W warmup steps and K timed ones between two
    synchronisations, then the dense products' average launch times from a
    logged pass."""
    import torch
    from orthogonal_equivalence_amd import synth
    from orthogonal_equivalence_amd import poetx as px
    from orthogonal_equivalence_amd.device import DeviceLayer, to_device

    L = synth.make_layer(cfg, 0)
    A = synth.make_activations(cfg, 0)
    dl = DeviceLayer(cfg.m, cfg.n, cfg.b_r, cfg.b_p, cfg.act, cfg.weight, cfg.T)
    dl.load(L)
    x = to_device(A["X_raw"], cfg.act)
    dz = to_device(A["dZ_raw"], cfg.act)
    del A, L
    z = dl.act_tensor(cfg.T, cfg.n)
    dx = dl.act_tensor(cfg.T, cfg.m)
    dq_r, dq_p = torch.empty_like(dl.q_r), torch.empty_like(dl.q_p)

    def step():
        dl.cnp_build()
        dl.forward(x, z)
        dl.backward(dz, dq_r, dq_p, dx)

    for _ in range(warmup):
        step()
    st = torch.cuda.current_stream()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0.record(st)
    for _ in range(steps):
        step()
    t1.record(st)
    torch.cuda.synchronize()
    ms = t0.elapsed_time(t1) / steps
    px.poetx_profile_enable(1)
    for _ in range(3):
        step()
    px.poetx_profile_enable(0)
    g = {}
    for i in range(px.poetx_profile_count()):
        name, t = px.poetx_profile_get(i)
        if name.startswith("gemm_dense"):
            g.setdefault(name, []).append(t)
    out = {"tokens": cfg.T, "m": cfg.m, "n": cfg.n, "b": cfg.b_r, "weight": cfg.weight,
           "ms_per_step": round(ms, 4), "tokens_per_s": round(cfg.T / (ms * 1e-3), 1)}
    flops = 2.0 * cfg.T * cfg.m * cfg.n
    for name, ts in sorted(g.items()):
        avg = sum(ts) / len(ts)
        out[name + "_ms"] = round(avg, 4)
        out[name + "_frac_mfma"] = round(flops / (avg * 1e-3) / (PEAK_BF16_TFLOPS * 1e12), 4)
    del dl
    torch.cuda.empty_cache()
    return out


def copy_probe(mib):
    """Plain device-to-device copies of a known size (the calibration for the
    HBM byte counters: a profiler reads FETCH_SIZE / WRITE_SIZE off these)."""
    import torch
    n = mib * (1 << 20) // 2
    src = torch.ones(n, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    log(f"[bench] copy probe: 3 copies of {mib} MiB")
    del src, dst


def main():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="llama8b_mlp_up")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-yardstick", action="store_true")
    ap.add_argument("--no-mem-variant", action="store_true",
                    help="skip the memory variant's timed pass (profiling runs)")
    ap.add_argument("--no-spread", action="store_true",
                    help="skip the per-step warm and cold spread passes (profiling runs)")
    ap.add_argument("--merge", action="store_true",
                    help="include one merge and the weight rebuild in every step (the 8B MLP-up workload always does)")
    ap.add_argument("--no-other-workloads", action="store_true",
                    help="skip the timed steps of the workloads other than --workload")
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="run three plain copies of this many MiB first (counter calibration)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs the layer on one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the multi-GPU path (data parallel over token shards with one all-reduce of the packed "
              "gradients) is not implemented", file=sys.stderr)
        sys.exit(2)

    import torch
    from orthogonal_equivalence_amd import synth
    from orthogonal_equivalence_amd import poetx as px
    from orthogonal_equivalence_amd.device import DeviceLayer, to_device

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.copy_probe_mib > 0:
        copy_probe(args.copy_probe_mib)
    cfg = synth.CONFIGS[args.workload]
    if args.merge and not cfg.merge:
        cfg = dataclasses.replace(cfg, merge=True)
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
    draws = itertools.count(1)
    # a merge leaves q = 0; each step starts from the seeded nonzero q (a
    # device copy standing in for the optimizer's update, inside the timed
    # step), so that every step builds and applies real rotations
    q_step_r = dl.q_r.clone()
    q_step_p = dl.q_p.clone()

    def optimizer_stand_in():
        if cfg.merge:
            dl.q_r.copy_(q_step_r)
            dl.q_p.copy_(q_step_p)

    # what a training loop runs at a merge: a new draw of both permutations
    # (started on a second stream at the top of the step, so that it runs
    # beside the forward and backward), then W0 <- R W0 P with q <- 0 written
    # into their frame
    draw_now = [None]

    def begin_draw():
        draw_now[0] = next(draws)
        dl.begin_draw(MERGE_SEED, 0, draw_now[0])

    def merge_cycle():
        dl.merge_cycle(MERGE_SEED, 0, draw_now[0])

    def step():
        optimizer_stand_in()
        if cfg.merge:
            begin_draw()
        dl.cnp_build()
        dl.forward(x, z)
        dl.backward(dz, dq_r, dq_p, dx)
        if cfg.merge:
            merge_cycle()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    log(f"[bench] {args.warmup} warmup steps done")

    stream = torch.cuda.current_stream()

    def timed(steps, fn=step):
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0.record(stream)
        for _ in range(steps):
            fn()
        t1.record(stream)
        torch.cuda.synchronize()
        return t0.elapsed_time(t1)

    # pass 1: the step as a caller runs it (value, ms_per_step)
    ms_total = timed(args.steps)
    # pass 2: the same steps with the library's per-step HIP-event log on
    # (each logged step adds an event pair on the stream): per-kernel times
    # for the roofline
    px.poetx_profile_enable(1)
    ms_logged = timed(args.steps)
    px.poetx_profile_enable(0)
    per = {}
    for i in range(px.poetx_profile_count()):
        name, ms = px.poetx_profile_get(i)
        s = per.setdefault(name, [0.0, 0])
        s[0] += ms
        s[1] += 1
    ms_step = ms_total / args.steps
    log(f"[bench] {args.steps} timed steps: {ms_step:.3f} ms/step "
        f"({ms_logged / args.steps:.3f} ms/step with the per-kernel log)")
    kernels = {k: round(v[0] / v[1], 4) for k, v in sorted(per.items())}
    log("[bench] per-step breakdown (ms): " + json.dumps(kernels))

    # pass 3: the memory variant of the same step (the forward saves nothing,
    # the backward recomputes X1, X2 and Y1 from x), timed like pass 1
    def step_mem():
        optimizer_stand_in()
        if cfg.merge:
            begin_draw()
        dl.cnp_build()
        dl.forward_mem(x, z)
        dl.backward_mem(x, dz, dq_r, dq_p, dx)
        if cfg.merge:
            merge_cycle()

    variant_mem = None
    if not args.no_mem_variant:
        for _ in range(2):
            step_mem()
        ms_mem = timed(args.steps, step_mem) / args.steps
        log(f"[bench] memory variant: {ms_mem:.3f} ms/step")
        variant_mem = {"ms_per_step": round(ms_mem, 4), "tokens_per_s": round(cfg.T / (ms_mem * 1e-3), 1),
                       "activation_bytes_kept_per_layer": 0,
                       "saving_variant_activation_bytes_per_layer": px.poetx_saved_bytes(dl.L, cfg.T)}

    # pass 4: spread of single-step times, warm (back to back) and cold (a
    # 1 GiB write before each step evicts the 256 MB last-level cache and
    # every L2, so the step starts with nothing of its inputs cached)
    def step_spread(steps, before):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
        torch.cuda.synchronize()
        for a, b in evs:
            if before is not None:
                before()
            a.record(stream)
            step()
            b.record(stream)
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)
        at = lambda f: ms[int(round(f * (len(ms) - 1)))]  # noqa: E731
        return {"median_ms": round(at(0.5), 4), "p10_ms": round(at(0.1), 4), "p90_ms": round(at(0.9), 4)}

    spread = None
    if not args.no_spread:
        evict = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
        spread = {"warm": step_spread(args.steps, None), "cold": step_spread(args.steps, evict.zero_),
                  "cold_evict_bytes": evict.numel() * 4}
        del evict
        log(f"[bench] step spread: {json.dumps(spread)}")

    flops_gemm = 2.0 * cfg.T * cfg.m * cfg.n
    g = [per[k] for k in ("gemm_dense_fwd", "gemm_dense_bwd") if k in per]
    g_ms = sum(v[0] for v in g) / max(sum(v[1] for v in g), 1)
    bf16 = cfg.act == "bf16"
    peak = PEAK_BF16_TFLOPS if bf16 else PEAK_F32_TFLOPS
    achieved = flops_gemm / (g_ms * 1e-3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(achieved / peak, 4), "traffic": measured_traffic(cfg.name),
                "kernel": "dense W0 product (gemm_dense_fwd and gemm_dense_bwd launches)",
                "flops_per_launch": flops_gemm, "avg_launch_ms": round(g_ms, 4)}

    # pass 5: the step without its merge cycle, timed like pass 1 (q stays
    # nonzero without a merge, so no copy is needed); the merge cycle's
    # wall-clock cost is the difference of the two passes
    def step_fwd_bwd():
        dl.cnp_build()
        dl.forward(x, z)
        dl.backward(dz, dq_r, dq_p, dx)

    if cfg.merge:
        ms_fwd_bwd = timed(args.steps, step_fwd_bwd) / args.steps
        ms_merge = ms_step - ms_fwd_bwd
        optimizer_stand_in()
        log(f"[bench] without the merge cycle: {ms_fwd_bwd:.3f} ms/step (merge cycle {ms_merge:.3f} ms)")
    else:
        ms_fwd_bwd, ms_merge = ms_step, None
    # the merge cycle's kernels on the launch stream; the permutation draws
    # run on a second stream beside the step's forward and backward, so their
    # (overlapping) time is reported on its own
    ms_merge_kernels = sum(per[k][0] for k in per if k.startswith("merge")) / args.steps
    ms_draws = sum(per[k][0] for k in per if k.startswith("sample_perm")) / args.steps

    # pass 6: every other workload's step (CNP build, forward, backward; no
    # merge), timed like pass 1, plus its dense products from a logged pass
    others = None
    if not args.no_other_workloads:
        others = {}
        for name in OTHER_WORKLOADS:
            if name == cfg.name:
                continue
            others[name] = time_workload(synth.CONFIGS[name], args.steps, args.warmup)
            log(f"[bench] {name}: {json.dumps(others[name])}")

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
                   "step": ("q_update(copy)+" if cfg.merge else "") + "cnp_build+forward+backward"
                   + ("+perm_draw(side stream)+merge_into_new_frame" if cfg.merge else "")},
        "roofline": roofline,
        "cpu_baseline": None,
        "ms_per_step_with_kernel_log": round(ms_logged / args.steps, 4),
        "fwd_bwd_ms": round(ms_fwd_bwd, 4),
        "fwd_bwd_tokens_per_s": round(cfg.T / (ms_fwd_bwd * 1e-3), 1),
        "merge_cycle_ms": None if ms_merge is None else round(ms_merge, 4),
        "merge_cycle_kernels_ms": round(ms_merge_kernels, 4),
        "perm_draws_ms_on_side_stream": round(ms_draws, 4),
        "tokens_per_s_merge_every_200": (None if ms_merge is None else
                                         round(cfg.T / ((ms_fwd_bwd + ms_merge / 200) * 1e-3), 1)),
        "other_workloads": others,
        "step_spread": spread,
        "variant_mem": variant_mem,
        "kernels_ms": kernels,
        "kernel_roofline": kernel_roofline(cfg, per),
        "torch_linear_fwd_bwd_ms": yard,
        "pages_context": {
            "device": "NVIDIA H100, the pages' setting; shapes not stated",
            **PAGES_H100,
            "cnp_build_ms_here": kernels.get("cnp_build"),
            "layer_fwd_bwd_ms_here": round(ms_fwd_bwd, 4),
        },
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(cfg)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
