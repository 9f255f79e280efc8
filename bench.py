#!/usr/bin/env python3
"""Benchmark of the fused conv + norm forward path on one MI355X.

A step is one call of cnf_forward on one batch of seeded synthetic input that
is already resident in device memory.  The headline workload is the Conv3d
3->16 k3 -> channel softmax -> MaxPool3d(2) x2 problem at batch 128
(page "Kimi-K2.6__l2_p6"); every other workload is measured the same way and
listed under "per_workload" in the same JSON line.

Metric: effective TFLOP/s = 2 * N * C_out * |conv output grid| * (C_in/groups)
* k^ndim / time (the nominal conv FLOPs), plus ms per step.  `value` and
`ms_per_step` time K back-to-back steps (inputs resident; whatever the 256 MB
MALL keeps between steps); each workload also reports cold single steps
(ms_cold_*), each after a 512 MB write that evicts L2 and MALL.  "roofline" puts
the dominant kernel's ALGORITHMIC work per launch against the MI355X peak of
the unit that bounds it, timed with HIP events on the launch stream.
"cpu_baseline" is the fp64 oracle timed on the host cores on a bounded sample.

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
HEADLINE = "conv3d_softmax_pool_n128"

# Dominant kernel of each workload, as named by rocprofv3 (prefix match), its
# bounding unit, and the ALGORITHMIC work per launch: the per-unit figure x the
# units one launch processes (see the per-unit notes below).
#   softmax-pool: per pooled window 64 voxels x 16 ch x C_in*k^3 MAC x 2.
#   gn-mean:      per sample, the full conv (nothing skipped) -> nominal FLOPs.
#   small:        the full conv -> nominal FLOPs.
#   igemm:        the full conv -> nominal FLOPs.
#   convt:        HBM bound: x read once + the output written once (fp32).
#   upsample2:    the stride-2 transposed conv's normalising pass (mode 2): x read
#                 once + the output written once (a statistics pass precedes it).
DOMINANT = {
    "conv2d_in_div_n2": ("small_conv_norm_kernel", "mfma"),
    "conv3d_softmax_pool_n128": ("conv3d_softmax_pool_kernel", "mfma"),
    "conv3d_hswish_gn_mean_n1024": ("conv3d_k4_gn_mean_kernel", "mfma"),
    "conv2d_in_div_n128": ("conv2d_igemm_kernel<128", "mfma"),
    "convt2d_gelu_gn_n128": ("convt2d_gn_fused_kernel<2, 0>", "mfma"),
    "convt2d_dense_gelu_gn_n128": ("conv2d_igemm_kernel<64", "mfma"),
    "conv2d_s2p1_in_div_n128": ("gen_conv_kernel<false, 4, 1, 0>", "mfma"),
    "convt2d_s2_gelu_gn_n128": ("upsample2_conv_kernel<2, 2>", "hbm"),
    "conv2d_in_div_n128_bf16": ("gen_conv_kernel<false, 4, 1, 1>", "mfma"),
    "convt2d_gelu_gn_n128_bf16": ("convt2d_gn_fused_kernel<2, 1>", "mfma"),
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


def kernel_source_digest():
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "convolution_normalization_forward_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, f), "rb") as fh:
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
    if not e or e.get("kernel_source_digest") != kernel_source_digest():
        return None
    return e.get("hbm_bytes_per_launch")


def time_workload(name, steps, warmup, dev, flush=None, cold_reps=10):
    import numpy as np
    import torch

    import cnf_inputs
    import convolution_normalization_forward_amd as cnf

    wl = cnf_inputs.workload(name)
    plan = cnf.Plan(cnf.make_desc(wl))
    p = cnf_inputs.gen_params(wl)
    dt = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}[wl.get("dtype", "f32")]
    x = torch.from_numpy(cnf_inputs.gen_x(wl)).to(dev).to(dt)
    t = {k: (torch.from_numpy(v).to(dev) if v is not None else None) for k, v in p.items()}
    t["w"] = t["w"].to(dt)
    out, idx, ws = plan.allocate(dev)
    stream = torch.cuda.current_stream()
    sp = stream.cuda_stream

    def step():
        st = cnf.cnf_forward(plan.handle, x, t["w"], t["b"], t["gamma"], t["beta"], out, idx, ws,
                             plan.workspace_bytes, sp)
        if st != cnf.CNF_OK:
            raise cnf.CnfError(st, "cnf_forward")

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # timed region: exactly `steps` back-to-back steps between one pair of HIP
    # events recorded on the launch stream, synchronised on both sides
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for _ in range(steps):
        step()
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = e0.elapsed_time(e1) / steps
    # per-step event pairs as well (include each launch's own latency)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(min(steps, 20))]
    for a, b in ev:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) for a, b in ev])
    # cold steps: before each, overwrite a buffer larger than the MALL (256 MB) so
    # no input, weight or output line is left in L2 / MALL; then time one step
    cold = []
    if flush is not None:
        for i in range(cold_reps):
            flush.fill_(float(i))
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            step()
            b.record(stream)
            b.synchronize()
            cold.append(a.elapsed_time(b))
    cold = np.array(cold) if cold else None
    fl = nominal_flops(wl)
    afl = algorithmic_flops(wl)
    ab = algorithmic_bytes(wl)
    kern, bound = DOMINANT[name]
    res = {
        "workload": name,
        "family": plan.describe().split()[0].split("=")[1],
        "ms": ms,
        "ms_single_launch_mean": float(per.mean()),
        "ms_single_launch_min": float(per.min()),
        "ms_wall_per_step": wall * 1e3 / steps,
        "ms_cold_median": float(np.median(cold)) if cold is not None else None,
        "ms_cold_min": float(cold.min()) if cold is not None else None,
        "effective_tflops": fl / (ms * 1e-3) / 1e12,
        "nominal_gflop": fl / 1e9,
        "algorithmic_gflop": afl / 1e9,
        "algorithmic_gb": ab / 1e9,
        "frac_fp32_peak": fl / (ms * 1e-3) / 1e12 / PEAK_FP32_TFLOPS,
        "frac_mfma_peak_own_dtype": fl / (ms * 1e-3) / 1e12 / PEAK_MFMA_TFLOPS[wl.get("dtype", "f32")],
        "frac_hbm_peak_algorithmic": ab / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "dtype": wl.get("dtype", "f32"),
        "dominant_kernel": kern,
        "bound": bound,
    }
    del x, out, idx, ws, t
    torch.cuda.empty_cache()
    return wl, res


def cpu_baseline(name, seconds):
    """The fp64 oracle, as it stands, on the host cores: whole batches of the
    workload's first samples, repeated until `seconds` of wall time."""
    import cnf_inputs
    import oracle

    wl = cnf_inputs.workload(name)
    p = cnf_inputs.gen_params(wl)
    n = min(wl["N"], 16)
    x = cnf_inputs.gen_x(wl, range(n))
    wl_n = dict(wl, N=n)
    done = 0
    t0 = time.perf_counter()
    while True:
        oracle.forward(wl_n, x, **p)
        done += 1
        el = time.perf_counter() - t0
        if el >= seconds:
            break
    fl = nominal_flops(wl_n) * done
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            model = next((l.split(":", 1)[1].strip() for l in f if l.startswith("model name")),
                         None)
    except OSError:
        pass
    per_sample = el / (done * n)
    return {
        "value": fl / el / 1e12,
        "unit": "TFLOP/s",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"fp64 oracle on samples 0..{n - 1} of {name} (full conv grid), "
                  f"{done} passes in {el:.1f} s",
        "subset_seconds": el,
        "ms_per_sample": per_sample * 1e3,
        "full_batch_seconds_extrapolated": per_sample * wl["N"],
        "cpu_model": model,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--only", action="store_true", help="measure the named workload only")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
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
        wl, r = time_workload(nm, args.steps, args.warmup, dev, flush)
        per[nm] = r
        if nm == args.workload:
            head_wl = wl
    h = per[args.workload]

    kern, bound = DOMINANT[args.workload]
    if bound == "mfma":
        achieved = algorithmic_flops(head_wl) / (h["ms"] * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP32_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_FP32_TFLOPS}
    else:
        achieved = algorithmic_bytes(head_wl) / (h["ms"] * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS}
    roof["kernel"] = kern
    roof["traffic"] = load_traffic(args.workload)

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline: oracle for ~{args.cpu_seconds:.0f} s", file=sys.stderr,
              flush=True)
        cpu = cpu_baseline(args.workload, args.cpu_seconds)

    line = {
        "metric": "fused conv+norm fwd effective TFLOP/s",
        "value": h["effective_tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": h["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "N": head_wl["N"], "C_in": head_wl["C_in"],
                   "C_out": head_wl["C_out"], "in_dims": list(head_wl["in_dims"]),
                   "kernel": head_wl["kernel"], "parallelism": "single-gpu"},
        "roofline": roof,
        "cpu_baseline": cpu,
        "per_workload": list(per.values()),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
