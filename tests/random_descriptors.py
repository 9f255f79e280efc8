"""Seeded random small descriptors for the general family's sweep test.

Each case is a workload dict (the shape of cnf_inputs.WORKLOADS entries) drawn
from a fixed seed: 2-D or 3-D, conv or transposed conv, random channel counts,
groups, kernel, stride, padding, dilation, output_padding, activation, norm,
divide, reduction and input element type.  Only descriptors with valid output
extents are kept.  Data only: no arithmetic of the method.
"""
from __future__ import annotations

import numpy as np


def _extent(L, k, s, p, d, op, tr):
    if tr:
        return (L - 1) * s - 2 * p + d * (k - 1) + op + 1
    num = L + 2 * p - d * (k - 1) - 1
    return num // s + 1 if num >= 0 else 0


def cases(n: int, seed: int = 2024, first_id: int = 900) -> list:
    r = np.random.Generator(np.random.PCG64(seed))
    out = []
    while len(out) < n:
        nd = int(r.choice([2, 3], p=[0.7, 0.3]))
        tr = bool(r.random() < 0.4)
        G = int(r.choice([1, 1, 2, 3, 4]))
        cig = int(r.integers(1, 9 if nd == 3 else 13))
        cog = int(r.integers(1, 13 if G > 1 else 40))
        k = int(r.choice([1, 2, 3, 3, 4, 5])) if nd == 2 else int(r.choice([1, 2, 3]))
        s = int(r.choice([1, 1, 2, 3]))
        d = int(r.choice([1, 1, 2]))
        p = int(r.integers(0, k))
        op = int(r.integers(0, max(s, d))) if tr else 0
        dims = [1] + [int(r.integers(3, 20)) for _ in range(2)] if nd == 2 else \
            [int(r.integers(2, 8)) for _ in range(3)]
        ext = [_extent(L, k, s, p, d, op, tr) for L in (dims if nd == 3 else dims[1:])]
        if min(ext) < 1 or int(np.prod(ext)) > 4096:
            continue
        C_out = G * cog
        act = str(r.choice(["none", "hardswish", "gelu", "gelu_tanh", "softmax"]))
        norm = str(r.choice(["none", "group", "instance"]))
        ng = 1
        if norm == "group":
            divs = [g for g in range(1, C_out + 1) if C_out % g == 0]
            ng = int(r.choice(divs))
        red = str(r.choice(["none", "none", "mean", "maxpool"]))
        pk = pr = 0
        if red == "maxpool":
            pk, pr = int(r.choice([2, 3])), 1
            if min(ext) < pk:
                red = "none"
                pk = 0
        wl = dict(id=first_id + len(out), ndim=nd, kind="conv_transpose" if tr else "conv",
                  N=int(r.integers(1, 3)), C_in=G * cig, C_out=C_out, in_dims=tuple(dims),
                  kernel=k, groups=G, has_bias=int(r.random() < 0.8), act=act, norm=norm,
                  num_groups=ng, eps=1e-5, affine=int(norm != "none" and r.random() < 0.5),
                  divide_by=float(r.choice([1.0, 2.0, 0.5])), reduce=red, pool_kernel=pk,
                  pool_repeats=pr, want_argmax=int(red == "maxpool" and r.random() < 0.6),
                  stride=s, padding=p, dilation=d, output_padding=op,
                  dtype=str(r.choice(["f32", "f32", "bf16", "f16"])), name=f"random{seed}_{len(out)}")
        out.append(wl)
    return out
