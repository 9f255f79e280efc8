"""Seeded synthetic workloads and inputs for the fused conv + norm forward path.

This module holds data only: the workload shapes and options, and the seeded
random tensors fed to both the HIP library and the fp64 oracle.  It contains
none of the method's arithmetic and imports neither side.

Workloads (shapes and options as the four source pages state their problems):
  * conv2d_in_div_n2      Conv2d 8->16 k3 on 2x8x32x32, InstanceNorm2d, /2.
                          A shrunken form of the l2_p17 problem, sized so the
                          oracle covers every element in well under a second.
  * conv3d_softmax_pool_n128
                          Conv3d 3->16 k3 on 128x3x16x32x32, softmax over the
                          channels, MaxPool3d(2) twice  (page l2_p6).
  * conv3d_hswish_gn_mean_n1024
                          Conv3d 3->16 k4 on 1024x3x16x32x32, HardSwish,
                          GroupNorm(4) with affine, mean over D,H,W (l2_p27).
  * conv2d_in_div_n128    Conv2d 64->128 k3 on 128x64x128x128,
                          InstanceNorm2d (no affine), /2  (page l2_p17).
  * convt2d_gelu_gn_n128  ConvTranspose2d 64->64 k3 s1 groups 8 on
                          128x64x256x256, exact GELU, GroupNorm(8) with affine
                          (page l2_p19).
  * convt2d_dense_gelu_gn_n128
                          the same with groups = 1 (dense 64->64 transposed
                          conv, K = 576): the other reading of l2_p19's problem.
  * conv2d_s2p1_in_div_n128
                          l2_p17's chain with a strided, padded conv: Conv2d
                          64->128 k3 stride 2 padding 1 on 128x64x128x128
                          (-> 64x64), InstanceNorm2d, /2.
  * conv2d_in_div_n128_bf16, convt2d_gelu_gn_n128_bf16
                          the l2_p17 and l2_p19 problems with x and w in bf16
                          (fp32 accumulation and epilogue).
  * convt2d_gelu_gn_n128_bf16x3, convt2d_s2_gelu_gn_n128_bf16x3
                          the l2_p19 problem and its upsampling form in fp32,
                          the contraction on three bf16 pieces of each fp32
                          operand (f32_math).
  * convt2d_s2_gelu_gn_n128
                          l2_p19's chain as an upsampling layer:
                          ConvTranspose2d 64->64 k3 stride 2 padding 1
                          output_padding 1 groups 8 on 128x64x128x128
                          (-> 256x256, the page's output size), GELU,
                          GroupNorm(8) with affine.

Element types: with dtype "bf16" or "f16", x and the conv weight are drawn as
above and rounded to that type (round to nearest even); they are returned as
float32 arrays holding exactly the rounded values, so the oracle and the
library see the same numbers (bias, gamma and beta stay fp32).

Distributions: x ~ N(0, 1) (or U[0, 1) as a second parity set, the
distribution the pages' own harness used); conv weight and bias ~
U(-1/sqrt(fan_in), 1/sqrt(fan_in)) with fan_in = (C_in/groups) * k^ndim;
gamma ~ U(0.5, 1.5); beta ~ N(0, 0.1).  Every tensor comes from NumPy's PCG64
seeded with (1000 * workload id + tensor id[, sample]) so any one sample of x
can be drawn without drawing the others.
"""
from __future__ import annotations

import math

import numpy as np

# Tensor ids inside a workload's seed space.
_TID_X, _TID_W, _TID_B, _TID_GAMMA, _TID_BETA = 1, 2, 3, 4, 5

_BASE = dict(ndim=2, kind="conv", groups=1, has_bias=1, act="none", norm="none",
             num_groups=1, eps=1e-5, affine=0, divide_by=1.0, reduce="none",
             pool_kernel=0, pool_repeats=0, want_argmax=0, stride=1, padding=0, dilation=1,
             output_padding=0, dtype="f32", f32_math="native")


def _wl(**kw):
    d = dict(_BASE)
    d.update(kw)
    return d


WORKLOADS = {
    "conv2d_in_div_n2": _wl(
        id=1, ndim=2, N=2, C_in=8, C_out=16, in_dims=(1, 32, 32), kernel=3,
        norm="instance", num_groups=16, divide_by=2.0),
    "conv3d_softmax_pool_n128": _wl(
        id=2, ndim=3, N=128, C_in=3, C_out=16, in_dims=(16, 32, 32), kernel=3,
        act="softmax", reduce="maxpool", pool_kernel=2, pool_repeats=2,
        want_argmax=1),
    "conv3d_hswish_gn_mean_n1024": _wl(
        id=3, ndim=3, N=1024, C_in=3, C_out=16, in_dims=(16, 32, 32), kernel=4,
        act="hardswish", norm="group", num_groups=4, affine=1, reduce="mean"),
    "conv2d_in_div_n128": _wl(
        id=4, ndim=2, N=128, C_in=64, C_out=128, in_dims=(1, 128, 128), kernel=3,
        norm="instance", num_groups=128, divide_by=2.0),
    "convt2d_gelu_gn_n128": _wl(
        id=5, ndim=2, kind="conv_transpose", N=128, C_in=64, C_out=64,
        in_dims=(1, 256, 256), kernel=3, groups=8, act="gelu", norm="group",
        num_groups=8, affine=1),
    "convt2d_dense_gelu_gn_n128": _wl(
        id=6, ndim=2, kind="conv_transpose", N=128, C_in=64, C_out=64,
        in_dims=(1, 256, 256), kernel=3, groups=1, act="gelu", norm="group",
        num_groups=8, affine=1),
    "conv2d_s2p1_in_div_n128": _wl(
        id=7, ndim=2, N=128, C_in=64, C_out=128, in_dims=(1, 128, 128), kernel=3,
        stride=2, padding=1, norm="instance", num_groups=128, divide_by=2.0),
    "convt2d_s2_gelu_gn_n128": _wl(
        id=8, ndim=2, kind="conv_transpose", N=128, C_in=64, C_out=64,
        in_dims=(1, 128, 128), kernel=3, groups=8, stride=2, padding=1,
        output_padding=1, act="gelu", norm="group", num_groups=8, affine=1),
}

# 16-bit-input forms of the l2_p17 and l2_p19 problems (x and w in bf16, fp32
# accumulation and epilogue): the second input precision.
WORKLOADS["conv2d_in_div_n128_bf16"] = dict(WORKLOADS["conv2d_in_div_n128"], id=9, dtype="bf16")
WORKLOADS["convt2d_gelu_gn_n128_bf16"] = dict(WORKLOADS["convt2d_gelu_gn_n128"], id=10,
                                              dtype="bf16")
# The l2_p19 problem in fp32 with the contraction on three bf16 pieces of each
# operand (fp32 accuracy; the library's f32_math option).
WORKLOADS["convt2d_gelu_gn_n128_bf16x3"] = dict(WORKLOADS["convt2d_gelu_gn_n128"], id=11,
                                                f32_math="bf16x3")
WORKLOADS["convt2d_s2_gelu_gn_n128_bf16x3"] = dict(WORKLOADS["convt2d_s2_gelu_gn_n128"], id=12,
                                                   f32_math="bf16x3")

# The workloads the pages state (the others vary their geometry or precision).
PAGE_WORKLOADS = [n for n in WORKLOADS if WORKLOADS[n]["id"] <= 6]

# Order in which the workloads are listed (smallest first).
WORKLOAD_ORDER = list(WORKLOADS)


def workload(name: str, **overrides) -> dict:
    """A copy of a named workload, optionally with fields replaced (e.g. N)."""
    d = dict(WORKLOADS[name])
    d.update(overrides)
    d["name"] = name
    return d


def x_shape(wl: dict, n: int | None = None) -> tuple:
    D, H, W = wl["in_dims"]
    n = wl["N"] if n is None else n
    sp = (D, H, W) if wl["ndim"] == 3 else (H, W)
    return (n, wl["C_in"]) + sp


def w_shape(wl: dict) -> tuple:
    k, g = wl["kernel"], wl["groups"]
    ks = (k,) * wl["ndim"]
    if wl["kind"] == "conv_transpose":
        return (wl["C_in"], wl["C_out"] // g) + ks
    return (wl["C_out"], wl["C_in"] // g) + ks


def round_to(a: np.ndarray, dtype: str) -> np.ndarray:
    """float32 array rounded to bf16 / fp16 (nearest even), returned as float32."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "f16":
        return a.astype(np.float16).astype(np.float32)
    if dtype == "bf16":
        u = a.view(np.uint32).astype(np.uint64)
        u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
        return u.astype(np.uint32).view(np.float32)
    raise ValueError(dtype)


def fan_in(wl: dict) -> int:
    return (wl["C_in"] // wl["groups"]) * wl["kernel"] ** wl["ndim"]


def _rng(wl: dict, tid: int, *extra: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64([1000 * wl["id"] + tid, *extra]))


def gen_x(wl: dict, samples=None, dist: str = "normal", seed_offset: int = 0) -> np.ndarray:
    """x for the listed samples (default: all), float32, C-contiguous.

    Sample n is always drawn from its own stream, so gen_x(wl, [5]) equals
    gen_x(wl)[5:6].
    """
    if samples is None:
        samples = range(wl["N"])
    samples = list(samples)
    shp = x_shape(wl, len(samples))
    out = np.empty(shp, dtype=np.float32)
    per = shp[1:]
    for i, n in enumerate(samples):
        r = _rng(wl, _TID_X, n, seed_offset)
        if dist == "normal":
            out[i] = r.standard_normal(per, dtype=np.float32)
        elif dist == "uniform":
            out[i] = r.random(per, dtype=np.float32)
        else:
            raise ValueError(dist)
    return round_to(out, wl.get("dtype", "f32"))


def gen_params(wl: dict, seed_offset: int = 0) -> dict:
    """Conv weight and bias, and the norm's gamma / beta (None when unused)."""
    bound = 1.0 / math.sqrt(fan_in(wl))
    w = _rng(wl, _TID_W, seed_offset).uniform(-bound, bound, w_shape(wl)).astype(np.float32)
    w = round_to(w, wl.get("dtype", "f32"))
    b = None
    if wl["has_bias"]:
        b = _rng(wl, _TID_B, seed_offset).uniform(-bound, bound, (wl["C_out"],)).astype(np.float32)
    gamma = beta = None
    if wl["norm"] != "none" and wl["affine"]:
        gamma = _rng(wl, _TID_GAMMA, seed_offset).uniform(0.5, 1.5, (wl["C_out"],)).astype(np.float32)
        beta = (0.1 * _rng(wl, _TID_BETA, seed_offset).standard_normal((wl["C_out"],))).astype(np.float32)
    return dict(w=w, b=b, gamma=gamma, beta=beta)


def subset(wl: dict, k: int) -> list:
    """A seeded subset of k sample indices that always holds 0 and N-1."""
    N = wl["N"]
    if k >= N:
        return list(range(N))
    r = np.random.Generator(np.random.PCG64(7000 + wl["id"]))
    mid = r.choice(np.arange(1, N - 1), size=max(k - 2, 0), replace=False)
    return sorted({0, N - 1, *map(int, mid)})
