#!/usr/bin/env python3
"""Attention-forward benchmark on one MI355X.

One step = one attention forward pass (every stage of the fused kernel) over
the long-sequence workload: B=1, H_q=32, H_kv=8, N=16384, d=128, causal, bf16,
K scaled by 2. Inputs are generated once and are resident in HBM before the
timed region. Prints ONE JSON line.

  value       = algorithmic FLOPs / wall time per step (TFLOP/s), with the
                FLOPs 2·B·H_q·N_q·N_kv·(d_qk + d_v), halved when causal
  roofline    = the kernel's own launch time, from HIP events recorded on the
                stream the kernel is launched on, against the bf16 dense MFMA
                peak (256 CUs x 4096 flop/clk x 2.4 GHz = 2516.6 TFLOP/s):
                `achieved` from the average launch; the median (the primary
                figure), min and p90 beside it; the shader clock the
                chip held under the same load (an in-kernel probe, untimed,
                after the timed steps) and the fraction of the MFMA rate at
                that clock; then the dense bf16 MFMA rate the chip sustains
                on toggling operands (a probe kernel on every CU, also after
                the timed steps) and the kernel's fraction of it
  cpu_baseline= the fp64 oracle timed on the host over a bounded row sample;
                `cores` is the threads it used, `host_cores` and
                `affinity_cores` what the host has and allows
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 256 * 4096 * 2.4e9 / 1e12  # 2516.6
PEAK_HBM_GBS = 8000.0  # MI355X HBM3E
PROFILES = os.path.join(ROOT, "profiles")
METRIC = "attention fwd TFLOP/s on 1 MI355X + % of bf16 MFMA peak (causal FLOPs /2)"
DROPOUT_SEED = 1234


def kernel_source_sha(split: bool = False, wide_split: bool = False) -> str:
    """Hash of the sources an attention profile was taken on: the host code,
    the tile layer and RoPE, plus the main and wide kernels (wide_split: and
    the split-KV header the wide split kernel includes), or, for the d 64 /
    128 split-KV path, its own kernel and the main kernel header it includes."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "accelerator_programming_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        if split:
            take = name in ("attn_fwd.hip", "attn_fwd_kernel.hpp", "attn_split_kernel.hpp", "tile.hpp", "rope.hpp")
        else:
            take = name.startswith("attn_fwd") or name in ("tile.hpp", "rope.hpp") or (
                wide_split and name == "attn_split_kernel.hpp")
        if take:
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def gemm_source_sha() -> str:
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "accelerator_programming_amd", "csrc")
    for name in ("gemm_kernel.hpp", "tile_gemm.hip", "tile.hpp"):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


def wide_split_path(w, single_pass=False) -> bool:
    """Wide heads with V inside K, not causal: timed through the split-KV
    entry point (64-row tiles over key ranges, then the merge) unless
    single_pass asks for attn_fwd_run."""
    return w.dqk == 576 and w.v_from_k and not w.causal and not w.decode and not single_pass


def kernel_name(w, dropout=False, rope=False, single_pass=False):
    """The kernel the library launches for workload w (as rocprofv3 names it)."""
    causal = "true" if w.causal else "false"
    if w.decode:
        return "attn::attn_split_kernel<%d> + attn::attn_split_merge<%d>" % (w.dqk, w.dqk)
    if wide_split_path(w, single_pass):
        return "attn::attn_fwd_wide_vk_split_kernel<576, 512> + attn::attn_split_merge_wide<512>"
    if w.dqk == 576:
        # V given as the leading columns of K takes the kernel that stages K only
        return "attn::attn_fwd_wide_%skernel<576, 512, %s>" % ("vk_" if w.v_from_k else "", causal)
    return "attn::attn_fwd_kernel<%d, %s, %s%s>" % (
        w.dqk, causal, "__bf16" if str(w.dtype) == "torch.bfloat16" else "float",
        ", true" if dropout else (", false, true" if rope else ""))


def traffic_for_current_kernel(workload_name: str, tag: str, sha=None):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it was taken on other kernel sources or another workload."""
    try:
        with open(os.path.join(PROFILES, "%s_traffic.json" % tag)) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_sha") != (sha or kernel_source_sha()) or t.get("workload") != workload_name:
        return None
    return t.get("bytes_per_launch")


def cpu_baseline(w, q, k, v, target_s: float, threads: int, drop_thr: int = 0):
    """Time the oracle on a sample of rows sized for roughly target_s seconds."""
    import numpy as np
    import torch

    import oracle
    from accelerator_programming_amd.inputs import sample_rows

    Q = q.float().cpu().numpy()
    K = k.float().cpu().numpy()
    V = v.float().cpu().numpy() if not w.v_from_k else np.ascontiguousarray(
        k[..., : w.dv].float().cpu().numpy())

    def row_flops(rows):
        keys = (rows[:, 2] + 1) if w.causal else torch.full((rows.shape[0],), w.Nkv)
        return float((2.0 * keys.double() * (w.dqk + w.dv)).sum())

    def timed(n):
        rows = sample_rows(w, n, seed=123)
        t0 = time.perf_counter()
        _, _, used = oracle.attention_fp64(Q, K, V, w.causal, w.softmax_scale, rows=rows,
                                           threads=threads, drop_thr=drop_thr, seed=DROPOUT_SEED)
        return time.perf_counter() - t0, row_flops(rows), used, rows.shape[0]

    dt, fl, used, n = timed(max(threads * 4, 64))
    n2 = int(min(max(n * target_s / max(dt, 1e-3), n), 200000))
    dt, fl, used, n = timed(n2)
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        **cpu_info(used),
        "kind": "oracle",
        "sample": "%d seeded (b,h,i) rows of %s, each row's unmasked keys only; %.1f s wall, "
                  "%.3g FLOP" % (n, w.name, dt, fl),
    }


def gemm_cpu_baseline(w, a, b, target_s: float, threads: int):
    """Time the fp64 GEMM oracle on a sample of C rows sized for about target_s."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle.gemm import gemm_fp64

    A = a.float().cpu().numpy()
    B = b.float().cpu().numpy()
    rng = np.random.default_rng(123)

    def timed(n):
        rows = rng.integers(0, w.M, n)
        with threadpool_limits(limits=threads):
            t0 = time.perf_counter()
            gemm_fp64(A, B, rows=rows)
            return time.perf_counter() - t0, 2.0 * n * w.N * w.K, n

    dt, fl, n = timed(64)
    n2 = int(min(max(n * target_s / max(dt, 1e-3), n), w.M))
    dt, fl, n = timed(n2)
    return {
        "value": fl / dt / 1e12,
        "unit": "TFLOP/s",
        **cpu_info(threads),
        "kind": "oracle",
        "sample": "%d seeded rows of C of %s (fp64 product through numpy's BLAS, %d threads); "
                  "%.1f s wall, %.3g FLOP" % (n, w.name, threads, dt, fl),
    }


def settle(run, args):
    """Run the untimed warmup steps and fix the timed step count. With the
    defaults (-1): warm up for at least 5 steps and 0.3 s, then time at
    least 20 steps and about 0.2 s of work. Returns (warmup, steps) used."""
    import torch
    if args.warmup >= 0:
        for _ in range(args.warmup):
            run()
        torch.cuda.synchronize()
        warm, per_step = args.warmup, None
    else:
        warm = 0
        t0 = time.perf_counter()
        while warm < 5 or time.perf_counter() - t0 < 0.3:
            run()
            warm += 1
            if warm % 5 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        per_step = (time.perf_counter() - t0) / warm
    if args.steps > 0:
        steps = args.steps
    else:
        if per_step is None:
            t0 = time.perf_counter()
            run()
            torch.cuda.synchronize()
            per_step = time.perf_counter() - t0
        steps = max(20, int(0.2 / max(per_step, 1e-6)))
    return warm, steps


def clock_probe(run, stream, launch_ms: float, rounds: int = 4):
    """The shader clock under this load, measured on the GPU: after the timed
    steps the same launches keep running on `stream` (untimed), in rounds of
    at least 2 ms of launches (launch_ms each), and beside each round a probe
    kernel on a second stream (default priority) puts one wave in each of 256
    workgroups; each wave counts shader cycles (s_memtime) against the
    constant-rate counter (s_memrealtime) over 1 ms. Returns the median, min
    and max over all probe waves, or None if the probe library is not
    built."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "accelerator_programming_amd", "libattn_tile_selftest.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.tile_selftest_clock.restype = ctypes.c_int
    lib.tile_selftest_clock.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint,
                                        ctypes.c_uint, ctypes.c_void_p]
    lib.tile_selftest_wallclock_khz.restype = ctypes.c_int
    khz = lib.tile_selftest_wallclock_khz()
    if khz <= 0:
        return None
    n = 256
    side = torch.cuda.Stream()
    out = torch.zeros(rounds, 2 * n, dtype=torch.int64, device="cuda")
    ticks = khz  # 1 ms
    torch.cuda.synchronize()
    per_round = max(3, int(math.ceil(2.0 / max(launch_ms, 1e-3))))
    for r in range(rounds):
        for _ in range(per_round):
            run()
        # the probe starts while this round's launches are still running
        if lib.tile_selftest_clock(out[r].data_ptr(), n, ticks, 200000, side.cuda_stream) != 0:
            return None
        torch.cuda.synchronize()
    o = out.view(-1, 2).cpu().double()
    mhz = sorted((o[:, 0] / o[:, 1] * khz / 1e3).tolist())
    return {"median_mhz": round(mhz[len(mhz) // 2], 1), "min_mhz": round(mhz[0], 1),
            "max_mhz": round(mhz[-1], 1), "samples": len(mhz),
            "source": "s_memtime cycles over 1 ms of s_memrealtime in one wave per workgroup "
                      "of a probe kernel run beside further untimed launches after the timed steps"}


def launch_stats(ms):
    """Per-launch kernel times (HIP events): average, median, min, p90."""
    xs = sorted(ms)
    n = len(xs)
    return {"avg": sum(xs) / n, "median": xs[n // 2], "min": xs[0],
            "p90": xs[min(n - 1, int(math.ceil(0.9 * n)) - 1)]}


def timed_launches(run, steps, stream):
    """Time exactly `steps` launches of run(): wall clock around all of them
    (synchronised on both sides) and HIP events around each one, recorded on
    the stream the kernels are launched on. Then, untimed, the shader clock
    under the same load (clock_probe). Returns (wall_s, per-launch ms, clock
    summary)."""
    import torch
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        run()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    return wall, ms, clock_probe(run, stream, sorted(ms)[len(ms) // 2])


def kernel_times(ms, clock, work, unit_scale, peak_at_clock=None):
    """The roofline's timing block: per-launch statistics in ms, the rate at
    the median launch, and (for MFMA-bound kernels) the fraction of the
    dense bf16 rate at the sampled clock."""
    st = launch_stats(ms)
    out = {"kernel_ms_avg": round(st["avg"], 4), "kernel_ms_median": round(st["median"], 4),
           "kernel_ms_min": round(st["min"], 4), "kernel_ms_p90": round(st["p90"], 4),
           "launches": len(ms),
           "achieved_at_median": round(work / (st["median"] * 1e-3) / unit_scale, 2),
           "sclk": clock}
    if peak_at_clock and clock:
        peak = 256 * 4096 * clock["median_mhz"] * 1e6 / 1e12
        out["frac_at_sampled_clock"] = round(work / (st["avg"] * 1e-3) / 1e12 / peak, 4)
    return out


def mfma_sustained(rounds: int = 1, iters: int = 120000):
    """The dense bf16 MFMA rate this chip sustains on operands that toggle
    like real data: a probe kernel with one 8-wave workgroup on each of the
    256 CUs, every wave issuing iters x 16 v_mfma_f32_32x32x16_bf16 fed from
    LDS (hashed bf16 values in [-2, 2)), about 80 ms per launch. One untimed
    launch, then `rounds` timed ones (HIP events); the shader clock from each
    wave's s_memtime cycles over its s_memrealtime ticks. Returns one dict
    per timed round, or None if the probe library is not built."""
    import ctypes

    import torch
    path = os.path.join(ROOT, "accelerator_programming_amd", "libattn_tile_selftest.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.tile_selftest_mfma_rate.restype = ctypes.c_int
    lib.tile_selftest_mfma_rate.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint,
                                            ctypes.c_void_p]
    lib.tile_selftest_wallclock_khz.restype = ctypes.c_int
    khz = lib.tile_selftest_wallclock_khz()
    nb = 256
    out = torch.zeros(nb * 16, dtype=torch.int64, device="cuda")
    stream = torch.cuda.current_stream()
    flops = nb * 8 * iters * 16 * 2.0 * 32 * 32 * 16
    res = []
    torch.cuda.synchronize()
    for r in range(rounds + 1):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        if lib.tile_selftest_mfma_rate(out.data_ptr(), nb, iters, stream.cuda_stream) != 0:
            return None
        e1.record(stream)
        torch.cuda.synchronize()
        if r == 0:
            continue
        ms = e0.elapsed_time(e1)
        o = out.view(-1, 2).cpu().double()
        mhz = sorted((o[:, 0] / o[:, 1] * khz / 1e3).tolist()) if khz > 0 else [0.0]
        tf = flops / (ms * 1e-3) / 1e12
        res.append({"tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
                    "clock_mhz_median": round(mhz[len(mhz) // 2], 1), "ms": round(ms, 3),
                    "mfma_per_wave": iters * 16})
    return res


def sustained_block(achieved: float):
    """For an MFMA-bound line: the probe's sustained rate on this chip, run
    after the timed steps, and the kernel's fraction of it."""
    res = mfma_sustained(rounds=1)
    if not res:
        return {}
    r = res[-1]
    return {"sustained_mfma": {**r, "achieved_frac": round(achieved / r["tflops"], 4),
                               "source": "probe kernel: 8 waves on each CU issuing "
                                         "v_mfma_f32_32x32x16_bf16 from LDS on hashed bf16 "
                                         "operands (bench.py --mfma-ceiling)"}}


def mfma_ceiling_main(rounds: int = 3) -> int:
    """--mfma-ceiling: the probe alone, `rounds` timed launches."""
    import torch
    torch.cuda.set_device(0)
    res = mfma_sustained(rounds=rounds)
    if not res:
        print("bench.py: the MFMA rate probe is not built or did not launch", file=sys.stderr)
        return 2
    for i, r in enumerate(res):
        print("round %d: %.3f ms, %.1f TFLOP/s (%.1f %% of %.1f), shader clock %.0f MHz" % (
            i + 1, r["ms"], r["tflops"], 100 * r["frac_of_peak"], PEAK_BF16_TFLOPS,
            r["clock_mhz_median"]), file=sys.stderr, flush=True)
    best = max(res, key=lambda x: x["tflops"])
    line = {"metric": "sustained dense bf16 MFMA rate, toggling operands, all CUs",
            "value": best["tflops"], "unit": "TFLOP/s", "higher_is_better": True,
            "peak": round(PEAK_BF16_TFLOPS, 1), "frac_of_peak": best["frac_of_peak"],
            "clock_mhz_median": best["clock_mhz_median"], "rounds": res,
            "config": {"workload": "MFMA rate probe", "workgroups": 256, "waves_per_simd": 2,
                       "mfma": "v_mfma_f32_32x32x16_bf16"}}
    print(json.dumps(line), flush=True)
    return 0


def cpu_info(threads_used: int) -> dict:
    """Host cores: the count the OS reports and the ones this process may use."""
    return {"cores": threads_used, "host_cores": os.cpu_count(),
            "affinity_cores": len(os.sched_getaffinity(0))}


def gemm_main(args, w) -> int:
    """One step = one C = A·Bᵀ launch over the workload's full shape."""
    import torch

    from accelerator_programming_amd import gemm
    from accelerator_programming_amd.inputs import make_gemm_inputs

    torch.cuda.set_device(0)
    a, b = make_gemm_inputs(w, "cuda")
    c = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    stream = torch.cuda.current_stream()
    args.warmup, args.steps = settle(lambda: gemm.gemm_nt(a, b, out=c, stream=stream), args)
    wall, kern_ms, clock = timed_launches(lambda: gemm.gemm_nt(a, b, out=c, stream=stream),
                                          args.steps, stream)
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    ms_per_step = wall * 1e3 / args.steps
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_avg_ms * 1e-3) / 1e12
    finite = bool(torch.isfinite(c).all().item())
    sustained = sustained_block(achieved)
    cpu = None
    if not args.no_cpu_baseline:
        threads = min(16, len(os.sched_getaffinity(0)))
        cpu = gemm_cpu_baseline(w, a, b, args.cpu_seconds, threads)
    line = {
        "metric": "bf16 GEMM C = A·Bᵀ TFLOP/s on 1 MI355X",
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, resident in HBM)",
        "config": {"workload": w.name, "M": w.M, "N": w.N, "K": w.K,
                   "gflop_per_step": round(flops / 1e9, 3), "parallelism": "single-gpu",
                   "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "outputs_finite": finite},
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2),
                     "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                     "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic_for_current_kernel(w.name, "tile_gemm_" + args.config,
                                                           gemm_source_sha()),
                     **kernel_times(kern_ms, clock, flops, 1e12, peak_at_clock=True),
                     **sustained,
                     "kernel": "attn::gemm_bf16_nt_kernel"},
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0 if finite else 1


def rope_main(args) -> int:
    """R1: the standalone RoPE kernel over the Q of the long-sequence workload
    ([1, 32, 16384, 128] bf16, base 500000): bound by HBM, each byte read and
    written once."""
    import torch

    from accelerator_programming_amd import attn
    from accelerator_programming_amd.inputs import C4, make_inputs

    torch.cuda.set_device(0)
    q, _, _ = make_inputs(C4, "cuda")
    y = torch.empty_like(q)
    base = args.rope or 500000.0
    stream = torch.cuda.current_stream()
    args.warmup, args.steps = settle(lambda: attn.attn_rope_bf16(q, y, base, stream), args)
    wall, kern_list, clock = timed_launches(lambda: attn.attn_rope_bf16(q, y, base, stream),
                                            args.steps, stream)
    kern_ms = sum(kern_list) / len(kern_list)
    nbytes = 2 * q.numel() * q.element_size()
    gbs = nbytes / (kern_ms * 1e-3) / 1e9
    line = {
        "metric": "RoPE GB/s on 1 MI355X (bytes read + written)",
        "value": round(nbytes / (wall / args.steps) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall * 1e3 / args.steps, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs, resident in HBM)",
        "config": {"workload": "R1_rope_B1_H32_N16384_d128", "base": base,
                   "parallelism": "single-gpu", "bytes_per_step": nbytes},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                     "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                     "traffic": traffic_for_current_kernel("R1_rope_B1_H32_N16384_d128",
                                                           "attn_rope_R1"),
                     **kernel_times(kern_list, clock, nbytes, 1e9),
                     "kernel": "attn::rope_bf16_kernel"},
        "cpu_baseline": None,
    }
    print(json.dumps(line), flush=True)
    return 0


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=-1,
                    help="timed steps (default: at least 20 and at least 0.2 s of work)")
    ap.add_argument("--warmup", type=int, default=-1,
                    help="untimed steps first (default: at least 5 and at least 0.3 s of work, "
                         "so that the clock has settled)")
    ap.add_argument("--config", default="C4",
                    help="workload C1..C5 (the metric is quoted on C4), D1/D2 (split-KV decode) "
                         "or G1/G2 (the bf16 GEMM of the projections)")
    ap.add_argument("--dropout", type=float, default=0.0, metavar="P",
                    help="attention workloads: run with dropout at probability P (steps of 1/256) "
                         "through attn_fwd_run_dropout")
    ap.add_argument("--rope", type=float, default=0.0, metavar="BASE",
                    help="attention workloads: RoPE(Q), RoPE(K) with this base through "
                         "attn_fwd_run_rope (R1 times the standalone RoPE kernel)")
    ap.add_argument("--single-pass", action="store_true",
                    help="wide heads with V inside K (C5): time attn_fwd_run instead of the "
                         "split-KV entry point")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--mfma-ceiling", action="store_true",
                    help="instead of attention: the sustained dense bf16 MFMA rate of this chip "
                         "on toggling operands (a probe kernel, every CU busy), with the clock "
                         "it held")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of attention: copy a MIB-MiB buffer 3 times (a reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE to bytes)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(asked for --gpus %d)" % args.gpus, file=sys.stderr)
        return 2

    import torch

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": 4 * n, "bytes_written": 4 * n,
                          "launches": 3}), flush=True)
        return 0

    if args.mfma_ceiling:
        return mfma_ceiling_main()

    from accelerator_programming_amd import attn
    from accelerator_programming_amd.inputs import GEMM_WORKLOADS, WORKLOADS, make_inputs

    if args.config in GEMM_WORKLOADS:
        return gemm_main(args, GEMM_WORKLOADS[args.config])
    if args.config == "R1":
        return rope_main(args)
    w = WORKLOADS[args.config]
    torch.cuda.set_device(0)
    q, k, v = make_inputs(w, "cuda")
    B, Hq, N = w.B, w.Hq, w.Nq
    o = torch.empty((B, Hq, N, w.dv), dtype=q.dtype, device="cuda")
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device="cuda")
    op = attn.AttnFwd(q, k, v, w.causal, w.softmax_scale, o)
    if w.decode or wide_split_path(w, args.single_pass):
        # split-KV path; its workspace is allocated here, outside the timed steps
        ws = torch.empty(attn.attn_fwd_split_workspace_bytes(op.plan, 0), dtype=torch.uint8,
                         device="cuda")
        op.run = lambda q, k, v, o, lse, stream=None: op.run_split(q, k, v, o, lse, 0, ws, stream)
    if args.rope:
        if w.decode or w.dqk == 576 or w.dtype != torch.bfloat16:
            print("bench.py: RoPE is served by the bf16 d = 64 / 128 kernel only", file=sys.stderr)
            return 2
        k_rot = torch.empty(attn.lib().attn_fwd_rope_workspace_bytes(op.plan), dtype=torch.uint8,
                            device="cuda")
        op.run = lambda q, k, v, o, lse, stream=None: op.run_rope(q, k, v, o, lse, args.rope,
                                                                  k_rot, stream)
    drop_thr = int(args.dropout * 256)
    if drop_thr and args.rope:
        print("bench.py: --dropout and --rope are separate paths", file=sys.stderr)
        return 2
    if drop_thr:
        if w.decode or w.dqk == 576:
            print("bench.py: dropout is served by the d = 64 / 128 kernel only", file=sys.stderr)
            return 2
        op.run = lambda q, k, v, o, lse, stream=None: op.run_dropout(q, k, v, o, lse, args.dropout,
                                                                     DROPOUT_SEED, stream)
    stream = torch.cuda.current_stream()
    args.warmup, args.steps = settle(lambda: op.run(q, k, v, o, lse, stream=stream), args)

    wall, kern_ms, clock = timed_launches(lambda: op.run(q, k, v, o, lse, stream=stream),
                                          args.steps, stream)
    op.close()
    kern_avg_ms = sum(kern_ms) / len(kern_ms)
    ms_per_step = wall * 1e3 / args.steps
    flops = w.flops()
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_avg_ms * 1e-3) / 1e12
    gbs = w.io_bytes() / (kern_avg_ms * 1e-3) / 1e9  # algorithmic bytes (each tensor once)
    finite = bool(torch.isfinite(o).all().item() and torch.isfinite(lse).all().item())
    sustained = {} if w.decode else sustained_block(achieved)

    cpu = None
    if not args.no_cpu_baseline:
        threads = min(16, len(os.sched_getaffinity(0)))
        cpu = cpu_baseline(w, q, k, v, args.cpu_seconds, threads, drop_thr)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.dtype == torch.bfloat16 else "fp32-in/bf16-mfma",
        "data": "synthetic (seeded N(0,1) inputs, resident in HBM)",
        "config": {"workload": w.name, "B": w.B, "H_q": w.Hq, "H_kv": w.Hkv, "N_q": w.Nq,
                   "N_kv": w.Nkv, "d_qk": w.dqk, "d_v": w.dv, "causal": w.causal,
                   "gflop_per_step": round(flops / 1e9, 3), "parallelism": "single-gpu",
                   "pct_of_bf16_peak": round(100 * value / PEAK_BF16_TFLOPS, 2),
                   "dropout": drop_thr / 256.0,
                   "rope_base": args.rope or None,
                   "outputs_finite": finite},
        "roofline": ({"bound": "mfma", "achieved": round(achieved, 2),
                      "peak": round(PEAK_BF16_TFLOPS, 1), "unit": "TFLOP/s",
                      "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                      "traffic": traffic_for_current_kernel(
                          w.name, "attn_fwd_" + args.config + ("_dropout" if drop_thr else "")
                          + ("_rope" if args.rope else "") + ("_single_pass" if args.single_pass else ""),
                          kernel_source_sha(wide_split=wide_split_path(w, args.single_pass))),
                      **kernel_times(kern_ms, clock, flops, 1e12, peak_at_clock=True),
                      **sustained,
                      "kernel": ("attn::rope_bf16_kernel (K) + " if args.rope else "")
                      + kernel_name(w, drop_thr > 0, args.rope > 0, args.single_pass)} if not w.decode else
                     {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                      "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                      "traffic": traffic_for_current_kernel(w.name, "attn_split_" + args.config,
                                                                  kernel_source_sha(split=True)),
                      **kernel_times(kern_ms, clock, w.io_bytes(), 1e9),
                      "tflops": round(achieved, 2),
                      "kernel": kernel_name(w)}),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)
    return 0 if finite else 1


if __name__ == "__main__":
    sys.exit(main())
