#!/usr/bin/env python3
"""Benchmark of the fused conv + norm forward path on one MI355X.

A step is one call of cnf_forward on one batch of seeded synthetic input that
is already resident in device memory.  The headline workload is the largest
single-GPU configuration: ConvTranspose2d 64->64 k3 groups 8 on
128 x 64 x 256 x 256 -> GELU (erf) -> GroupNorm(8) with affine (page
"Kimi-K2.6__l2_p19"), 2.15 GB in and 2.18 GB out.  Every other workload is
measured the same way and listed under "per_workload" in the same JSON line.

Metric: effective TFLOP/s = 2 * N * C_out * |conv output grid| * (C_in/groups)
* k^ndim / time (the nominal conv FLOPs), plus ms per step.  `value` and
`ms_per_step` time K back-to-back steps (inputs resident).  Each workload also
reports cold single steps (ms_cold_*), each after a 512 MB write that evicts
L2 and MALL; the cold median is the primary per-workload figure.

"roofline" puts the dominant kernel's ALGORITHMIC work per launch against the
MI355X peak of the unit that bounds it.  The dominant kernel's launch
duration is measured live: every timed step goes through cnf_forward_timed,
which records a HIP event pair around that kernel on the launch stream.
"traffic" (and per workload "counter_hbm_gbs") come from rocprofv3
FETCH_SIZE / WRITE_SIZE runs summarised in profiles/traffic.json, used only
while the kernel's sources are the ones measured.  "cpu_baseline" is the fp64
oracle timed on the host cores on a bounded sample of each workload.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_FP32_TFLOPS = 157.3     # MI355X dense fp32 (MFMA and packed vector)
PEAK_MFMA_TFLOPS = {"f32": 157.3, "bf16": 2500.0, "f16": 2500.0}  # dense MFMA per input type
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E
HEADLINE = "convt2d_gelu_gn_n128"
CSRC = os.path.join(ROOT, "convolution_normalization_forward_amd", "csrc")

# Dominant kernel of each workload (the launch cnf_forward_timed brackets), as
# rocprofv3 names it (prefix match), its source file, the unit that bounds it,
# and the ALGORITHMIC work per launch (the per-unit figure x the units one
# launch processes):
#   softmax-pool: per pooled window 64 voxels x 16 ch x C_in*k^3 MAC x 2 FLOP
#                 (the 25% of conv voxels no window reads are not counted).
#   gn-mean, small, implicit GEMMs (fp32 at stride 1 or 2, 16-bit): the full
#                 conv, nominal FLOPs (the 16-bit one against the bf16 peak).
#   convt (single write): HBM, x and w read once + the fp32 output written once.
#   upsample2:    the stride-2 transposed conv's single-write kernel: HBM,
#                 x read once + the output written once.
DOMINANT = {
    "conv2d_in_div_n2": ("small_conv_norm_kernel", "k_small_conv_norm.hip", "mfma"),
    "conv3d_softmax_pool_n128": ("conv3d_softmax_pool_kernel", "k_conv3d_softmax_pool.hip", "mfma"),
    "conv3d_hswish_gn_mean_n1024": ("conv3d_k4_gn_mean_kernel", "k_conv3d_gn_mean.hip", "mfma"),
    "conv2d_in_div_n128": ("conv2d_igemm_kernel<128, 0, 1, false>", "k_conv2d_igemm.hip", "mfma"),
    "convt2d_gelu_gn_n128": ("convt2d_gn_fused_kernel<2, 0>", "k_convt2d_gn_fused.hip", "hbm"),
    "convt2d_dense_gelu_gn_n128": ("conv2d_igemm_kernel<64, 2, 1, true>", "k_conv2d_igemm.hip", "mfma"),
    "conv2d_s2p1_in_div_n128": ("conv2d_igemm_kernel<128, 0, 2, false>", "k_conv2d_igemm.hip", "mfma"),
    "convt2d_s2_gelu_gn_n128": ("upsample2_gn_fused_kernel<2, false>", "k_convt2d_gn_fused.hip", "hbm"),
    "conv2d_in_div_n128_bf16": ("conv2d_igemm16_kernel<128, 0, 1>", "k_conv2d_igemm.hip", "mfma"),
    "convt2d_gelu_gn_n128_bf16": ("convt2d_gn_fused_kernel<2, 1>", "k_convt2d_gn_fused.hip", "hbm"),
    "convt2d_gelu_gn_n128_bf16x3": ("convt2d_gn_fused_kernel<2, 3>", "k_convt2d_gn_fused.hip", "hbm"),
    "convt2d_s2_gelu_gn_n128_bf16x3": ("upsample2_gn_fused_kernel<2, true>", "k_convt2d_gn_fused.hip", "hbm"),
}


def conv_out_grid(wl):
    """Conv output extents (D = 1 for 2-D), with stride, padding, dilation."""
    k, s, p, d = wl["kernel"], wl["stride"], wl["padding"], wl["dilation"]

    def ext(L):
        if wl["kind"] == "conv_transpose":
            return (L - 1) * s - 2 * p + d * (k - 1) + wl["output_padding"] + 1
        return (L + 2 * p - d * (k - 1) - 1) // s + 1
    D, H, W = wl["in_dims"]
    return (ext(D) if wl["ndim"] == 3 else 1, ext(H), ext(W))


def nominal_flops(wl):
    """2 x outputs x (C_in/groups) x taps per output.  A transposed conv with
    stride s reaches each output with k^ndim / s^ndim taps on average."""
    Do, Ho, Wo = conv_out_grid(wl)
    taps = wl["kernel"] ** wl["ndim"]
    if wl["kind"] == "conv_transpose":
        taps /= wl["stride"] ** wl["ndim"]
    return 2.0 * wl["N"] * wl["C_out"] * Do * Ho * Wo * (wl["C_in"] // wl["groups"]) * taps


def algorithmic_flops(wl):
    if wl["reduce"] == "maxpool":
        Do, Ho, Wo = conv_out_grid(wl)
        P = wl["pool_kernel"] ** wl["pool_repeats"]
        windows = wl["N"] * (Do // P) * (Ho // P) * (Wo // P)
        K = (wl["C_in"] // wl["groups"]) * wl["kernel"] ** wl["ndim"]
        return 2.0 * windows * P ** 3 * wl["C_out"] * K
    return nominal_flops(wl)


def algorithmic_bytes(wl):
    """Minimum HBM bytes: read x, w (in their element type), b, gamma, beta once;
    write the fp32 output once."""
    import cnf_inputs
    n = 1
    for v in cnf_inputs.x_shape(wl):
        n *= v
    w = 1
    for v in cnf_inputs.w_shape(wl):
        w *= v
    Do, Ho, Wo = conv_out_grid(wl)
    if wl["reduce"] == "mean":
        out = wl["N"] * wl["C_out"]
    elif wl["reduce"] == "maxpool":
        P = wl["pool_kernel"] ** wl["pool_repeats"]
        out = wl["N"] * wl["C_out"] * (Do // P) * (Ho // P) * (Wo // P) * (2 if wl["want_argmax"] else 1)
    else:
        out = wl["N"] * wl["C_out"] * Do * Ho * Wo
    es = 2.0 if wl.get("dtype", "f32") in ("bf16", "f16") else 4.0   # x and w element size
    return es * (n + w) + 4.0 * (3 * wl["C_out"] + out)


def dominant_work(wl, bound):
    """Algorithmic work of one launch of the dominant kernel: FLOP or bytes."""
    return algorithmic_bytes(wl) if bound == "hbm" else algorithmic_flops(wl)


def kernel_source_digest(name):
    """Digest of the sources the workload's dominant kernel is built from."""
    h = hashlib.sha256()
    for f in (DOMINANT[name][1], "device.h", "kernels.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(f.encode() + fh.read())
    return h.hexdigest()[:16]


def load_traffic(name):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, or None if absent or taken on different kernel sources."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    e = t.get(name)
    if not e or e.get("kernel_source_digest") != kernel_source_digest(name):
        return None
    return e.get("hbm_bytes_per_launch")


def _events(n):
    import torch
    return [torch.cuda.Event(enable_timing=True) for _ in range(n)]


def _pairs(n, stream):
    """n (before, after) event pairs for cnf_forward_timed, each recorded once
    so that its HIP handle exists."""
    ev = list(zip(_events(n), _events(n)))
    for a, b in ev:
        a.record(stream)
        b.record(stream)
    return ev


def time_workload(name, steps, warmup, dev, flush=None, cold_reps=None):
    import numpy as np
    import torch

    import cnf_inputs
    import convolution_normalization_forward_amd as cnf

    wl = cnf_inputs.workload(name)
    plan = cnf.Plan(cnf.make_desc(wl))
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.get("dtype", "f32")]
    # x ~ N(0, 1), drawn on the device from a seeded generator; the conv and
    # norm parameters are the workload's seeded draws
    g = torch.Generator(device=dev)
    g.manual_seed(20_000 + wl["id"])
    x = torch.randn(cnf_inputs.x_shape(wl), generator=g, device=dev).to(dt)
    t = {k: (torch.from_numpy(v).to(dev) if v is not None else None)
         for k, v in cnf_inputs.gen_params(wl).items()}
    t["w"] = t["w"].to(dt)
    out, idx, ws = plan.allocate(dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step(ev=None):
        if ev is None:
            st = cnf.cnf_forward(plan.handle, x, t["w"], t["b"], t["gamma"], t["beta"], out, idx,
                                 ws, plan.workspace_bytes, sp)
        else:
            st = cnf.cnf_forward_timed(plan.handle, x, t["w"], t["b"], t["gamma"], t["beta"], out,
                                       idx, ws, plan.workspace_bytes, sp, ev[0].cuda_event,
                                       ev[1].cuda_event)
        if st != cnf.CNF_OK:
            raise cnf.CnfError(st, "cnf_forward")

    # one event pair per timed step around the dominant kernel
    kev = _pairs(steps, stream)
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly `steps` back-to-back steps between one pair of HIP
    # events recorded on the launch stream, synchronised on both sides
    e0, e1 = _events(2)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(steps):
        step(kev[i])
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    kms = np.array([a.elapsed_time(b) for a, b in kev])
    # cold steps: before each, overwrite a buffer larger than the MALL (256 MB) so
    # no input, weight or output line is left in L2 / MALL; then time one step
    if cold_reps is None:
        cold_reps = 50 if ms < 1.0 else 10
    cold, cold_k = [], []
    if flush is not None:
        ce = [(a, b, c, d) for (a, b), (c, d) in zip(_pairs(cold_reps, stream),
                                                      _pairs(cold_reps, stream))]
        torch.cuda.synchronize()
        for i, (a, b, c, d) in enumerate(ce):
            flush.fill_(float(i))
            a.record(stream)
            step((c, d))
            b.record(stream)
            b.synchronize()
            cold.append(a.elapsed_time(b))
            cold_k.append(c.elapsed_time(d))
    cold = np.array(cold) if cold else None
    cold_k = np.array(cold_k) if cold_k else None
    fl = nominal_flops(wl)
    ab = algorithmic_bytes(wl)
    kern, src, bound = DOMINANT[name]
    work = dominant_work(wl, bound)
    k_ms = float(kms.mean())
    if bound == "hbm":
        k_ach, k_peak, k_unit = work / (k_ms * 1e-3) / 1e9, PEAK_HBM_GBS, "GB/s"
    else:
        k_peak = PEAK_MFMA_TFLOPS[wl.get("dtype", "f32")]
        k_ach, k_unit = work / (k_ms * 1e-3) / 1e12, "TFLOP/s"
    traffic = load_traffic(name)
    cold_med = float(np.median(cold)) if cold is not None else None
    res = {
        "workload": name,
        "family": plan.describe().split()[0].split("=")[1],
        "primary": "ms_cold_median",
        "ms_cold_median": cold_med,
        "ms_cold_min": float(cold.min()) if cold is not None else None,
        "ms": ms,
        "ms_wall_per_step": wall * 1e3 / steps,
        "effective_tflops": fl / (ms * 1e-3) / 1e12,
        "effective_tflops_cold": fl / (cold_med * 1e-3) / 1e12 if cold_med else None,
        "nominal_gflop": fl / 1e9,
        "algorithmic_gflop": algorithmic_flops(wl) / 1e9,
        "algorithmic_gb": ab / 1e9,
        "frac_fp32_peak": fl / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
        "frac_mfma_peak_own_dtype": fl / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS[wl.get("dtype", "f32")],
        "frac_hbm_peak_algorithmic": ab / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "dtype": wl.get("dtype", "f32"),
        "f32_math": wl.get("f32_math", "native"),
        "dominant_kernel": kern,
        "bound": bound,
        "dominant_ms_mean": k_ms,
        "dominant_ms_min": float(kms.min()),
        "dominant_ms_cold_median": float(np.median(cold_k)) if cold_k is not None else None,
        "dominant_achieved": k_ach,
        "dominant_peak": k_peak,
        "dominant_unit": k_unit,
        "dominant_frac": k_ach / k_peak,
        "counter_hbm_bytes_per_launch": traffic,
        "counter_hbm_gbs": traffic / (k_ms * 1e-3) / 1e9 if traffic else None,
        "counter_frac_hbm": traffic / (k_ms * 1e-3) / 1e9 / PEAK_HBM_GBS if traffic else None,
    }
    del x, out, idx, ws, t, plan
    return wl, res


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            return next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")), None)
    except OSError:
        return None


def cpu_baseline(name, seconds):
    """The fp64 oracle, as it stands, on the host cores: passes over the
    workload's samples 0, 1, 2, ... (doubling the samples per pass while a
    pass is short) until `seconds` of oracle time; only the oracle is timed."""
    import cnf_inputs
    import oracle

    wl = cnf_inputs.workload(name)
    p = cnf_inputs.gen_params(wl)
    N = wl["N"]
    fl_sample = nominal_flops(wl) / N
    el, done, n = 0.0, 0, 1
    while el < seconds:
        idx = [(done + j) % N for j in range(n)]
        x = cnf_inputs.gen_x(wl, idx)
        t0 = time.perf_counter()
        oracle.forward(dict(wl, N=n), x, **p)
        dt = time.perf_counter() - t0
        el += dt
        done += n
        if dt < 0.25 and n < 64:
            n *= 2
    per_sample = el / done
    return {
        "value": fl_sample * done / el / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"fp64 oracle over {done} samples of {name} (samples 0..{min(done, N) - 1}, "
                  f"full conv grid each), {el:.1f} s of oracle time",
        "samples": done,
        "oracle_seconds": el,
        "ms_per_sample": per_sample * 1e3,
        "full_batch_seconds_extrapolated": per_sample * N,
        "cpu_model": cpu_model(),
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true", help="measure the named workload only")
    ap.add_argument("--cold-reps", type=int, default=None,
                    help="cold single steps per workload (default 50 below 1 ms, else 10)")
    ap.add_argument("--cpu-seconds", type=float, default=20.0,
                    help="oracle seconds for the headline workload's CPU baseline")
    ap.add_argument("--cpu-seconds-other", type=float, default=4.0,
                    help="oracle seconds for every other workload's CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--print-maps", action="store_true",
                    help="at the end, print the executable mappings of the loaded shared "
                         "objects to stderr (to attribute frames of a crash at process exit)")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="first run 5 plain device copies of this many MiB (a known-size "
                         "kernel for scaling HBM byte counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py runs on one GPU only: every workload here is one GPU's whole problem "
              "and the forward has no cross-GPU step; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch

    import cnf_inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.copy_calibration_mib:
        n = args.copy_calibration_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(5):
            torch.mul(src, 1.0, out=dst)  # one plain read stream + one write stream
        torch.cuda.synchronize()
        print(f"[bench] copy calibration: 5 copies of {args.copy_calibration_mib} MiB",
              file=sys.stderr, flush=True)
        del src, dst
    flush = torch.empty(512 * (1 << 20) // 4, dtype=torch.float32, device=dev)
    names = [args.workload] if args.only else \
        [args.workload] + [n for n in cnf_inputs.WORKLOAD_ORDER if n != args.workload]
    per = {}
    head_wl = None
    for nm in names:
        print(f"[bench] {nm}: timing {args.steps} steps after {args.warmup} warm-up",
              file=sys.stderr, flush=True)
        wl, r = time_workload(nm, args.steps, args.warmup, dev, flush, args.cold_reps)
        per[nm] = r
        if nm == args.workload:
            head_wl = wl
        torch.cuda.empty_cache()
    del flush
    torch.cuda.synchronize()
    h = per[args.workload]

    roof = {"bound": h["bound"], "achieved": h["dominant_achieved"], "peak": h["dominant_peak"],
            "unit": h["dominant_unit"], "frac": h["dominant_frac"],
            "traffic": h["counter_hbm_bytes_per_launch"], "kernel": h["dominant_kernel"],
            "kernel_ms_mean": h["dominant_ms_mean"],
            "work_per_launch": dominant_work(head_wl, h["bound"])}

    if not args.no_cpu_baseline:
        for nm in names:
            s = args.cpu_seconds if nm == args.workload else args.cpu_seconds_other
            print(f"[bench] cpu baseline {nm}: oracle for ~{s:.0f} s", file=sys.stderr, flush=True)
            per[nm]["cpu_baseline"] = cpu_baseline(nm, s)
    cpu = per[args.workload].get("cpu_baseline")

    line = {
        "metric": "fused conv+norm fwd effective TFLOP/s",
        "value": h["effective_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms"],
        "ms_cold_median": h["ms_cold_median"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": h["dtype"],
        "data": "synthetic",
        "config": {"workload": args.workload, "N": head_wl["N"], "C_in": head_wl["C_in"],
                   "C_out": head_wl["C_out"], "in_dims": list(head_wl["in_dims"]),
                   "kernel": head_wl["kernel"], "groups": head_wl["groups"],
                   "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_workload": list(per.values()),
    }
    print(json.dumps(line), flush=True)
    if args.print_maps:
        with open("/proc/self/maps") as f:
            for l in f:
                if " r-xp " in l and ".so" in l:
                    sys.stderr.write("[maps] " + l)
        sys.stderr.flush()


if __name__ == "__main__":
    main()
