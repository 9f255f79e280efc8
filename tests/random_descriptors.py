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


def specialised_cases(n: int, seed: int = 31) -> list:
    """Seeded random shapes inside the specialised families' supported sets
    (implicit GEMM, single-write and two-pass transposed conv, softmax-pool,
    GroupNorm-mean, small conv), all at stride 1 and no padding unless the
    family takes padding."""
    r = np.random.Generator(np.random.PCG64(seed))
    base = dict(eps=1e-5, has_bias=1, stride=1, padding=0, dilation=1, output_padding=0,
                dtype="f32", pool_kernel=0, pool_repeats=0, want_argmax=0, divide_by=1.0,
                affine=0, norm="none", num_groups=1, reduce="none", act="none", groups=1)
    acts = ["none", "hardswish", "gelu", "gelu_tanh"]
    out = []
    i = 0
    while len(out) < n:
        fam = ["igemm", "convt_fused", "convt", "softmax_pool", "gn_mean", "small"][i % 6]
        i += 1
        wl = dict(base, id=1100 + len(out), name=f"spec{seed}_{len(out)}_{fam}")
        act = str(r.choice(acts))
        if fam == "igemm":
            co = int(r.choice([64, 128]))
            norm = str(r.choice(["none", "group", "instance"]))
            wl.update(ndim=2, kind=str(r.choice(["conv", "conv_transpose"])), N=int(r.integers(1, 3)),
                      C_in=int(r.choice([4, 8, 12, 16, 32])), C_out=co,
                      in_dims=(1, int(r.integers(3, 40)), int(r.integers(3, 90))), kernel=3,
                      act=act, norm=norm, num_groups=int(r.choice([1, 8, 16])) if norm == "group" else co,
                      affine=int(norm != "none" and r.random() < 0.5), padding=int(r.integers(0, 3)),
                      divide_by=float(r.choice([1.0, 2.0])))
        elif fam in ("convt_fused", "convt"):
            G = int(r.choice([1, 2, 4, 8]))
            W = 256 if fam == "convt_fused" else int(r.integers(3, 60))
            # the single-write kernel takes heights whose (H + 3) // 2 two-row steps
            # split into whole 4-step slices: H = 8m - 3 or 8m - 2
            H = (8 * int(r.integers(1, 6)) - int(r.choice([2, 3])) if fam == "convt_fused"
                 else int(r.integers(1, 40)))
            wl.update(ndim=2, kind="conv_transpose", N=int(r.integers(1, 3)), C_in=8 * G, C_out=8 * G,
                      in_dims=(1, H, W), kernel=3, groups=G, act=act,
                      norm="group", num_groups=G, affine=int(r.random() < 0.5))
        elif fam == "softmax_pool":
            two = bool(r.random() < 0.7)
            wl.update(ndim=3, kind="conv", N=int(r.integers(1, 3)), C_in=3, C_out=16,
                      in_dims=tuple(int(r.integers(6, 20)) for _ in range(3)), kernel=3,
                      act=str(r.choice(["softmax", "softmax", "none", "gelu_tanh"])), reduce="maxpool",
                      pool_kernel=2 if two else 4, pool_repeats=2 if two else 1,
                      want_argmax=int(r.random() < 0.7))
        elif fam == "gn_mean":
            wl.update(ndim=3, kind="conv", N=int(r.integers(1, 4)), C_in=3, C_out=16,
                      in_dims=(int(r.integers(4, 12)), int(r.integers(4, 20)), int(r.integers(4, 33))),
                      kernel=4, act=act, norm="group", num_groups=int(r.choice([1, 2, 4, 8, 16])),
                      affine=int(r.random() < 0.5), reduce="mean")
        else:
            nd = int(r.choice([2, 3]))
            dims = (1, int(r.integers(3, 33)), int(r.integers(3, 33))) if nd == 2 else \
                tuple(int(r.integers(3, 11)) for _ in range(3))
            wl.update(ndim=nd, kind="conv", N=int(r.integers(1, 3)),
                      C_in=int(r.choice([1, 3, 4, 8])) if nd == 2 else int(r.choice([1, 3])),
                      C_out=16, in_dims=dims, kernel=3, act=act,
                      norm=str(r.choice(["instance", "group", "none"])), num_groups=4,
                      reduce=str(r.choice(["none", "mean"])), divide_by=float(r.choice([1.0, 2.0])))
            if wl["norm"] == "instance":
                wl["num_groups"] = 16
        out.append(wl)
    return out
