"""The oracle's composition of the steps, per workload, on tiny inputs.

Each workload's chain (conv -> activation -> norm -> divide -> reduction) is
re-derived here with NumPy array code written differently from the oracle's
loops (windows + tensordot, vectorised statistics, reshape pooling) and a
different erf (math.erf via a vectorised call), so a wrong step order or a
wrong axis in the composition fails.  Sizes are shrunk; options are the
workloads' own.
"""
import math

import numpy as np
import pytest

import cnf_inputs
import oracle
from test_oracle_pins import _conv_numpy

_erf = np.vectorize(math.erf)


def _convt_numpy(x, w, b, G):
    # gather form: y[i, j] = sum x[i - a, j - e] w[a, e]
    N, Ci, H, W = x.shape
    _, cog, k, _ = w.shape
    Co = cog * G
    cig = Ci // G
    xp = np.pad(x.astype(np.float64), ((0, 0), (0, 0), (k - 1, k - 1), (k - 1, k - 1)))
    y = np.zeros((N, Co, H + k - 1, W + k - 1))
    for co in range(Co):
        g, col = divmod(co, cog)
        for c in range(cig):
            ci = g * cig + c
            for a in range(k):
                for e in range(k):
                    y[:, co] += w[ci, col, a, e] * xp[:, ci, k - 1 - a:k - 1 - a + H + k - 1,
                                                      k - 1 - e:k - 1 - e + W + k - 1]
    if b is not None:
        y += b.astype(np.float64)[None, :, None, None]
    return y


def _conv_torch(wl, x, p):
    # strided / padded / dilated geometry: torch's float64 CPU routines
    import torch
    import torch.nn.functional as F
    t = lambda a: None if a is None else torch.from_numpy(a.astype(np.float64))  # noqa: E731
    geo = dict(stride=wl["stride"], padding=wl["padding"], dilation=wl["dilation"],
               groups=wl["groups"])
    nd = wl["ndim"]
    if wl["kind"] == "conv_transpose":
        fn = F.conv_transpose2d if nd == 2 else F.conv_transpose3d
        return fn(t(x), t(p["w"]), t(p["b"]), output_padding=wl["output_padding"], **geo).numpy()
    fn = F.conv2d if nd == 2 else F.conv3d
    return fn(t(x), t(p["w"]), t(p["b"]), **geo).numpy()


def _reference_numpy(wl, x, p):
    if (wl["stride"], wl["padding"], wl["dilation"], wl["output_padding"]) != (1, 0, 1, 0):
        y = _conv_torch(wl, x, p)
    elif wl["kind"] == "conv_transpose":
        y = _convt_numpy(x, p["w"], p["b"], wl["groups"])
    else:
        y = _conv_numpy(x, p["w"], p["b"], wl["groups"])
    if wl["act"] == "hardswish":
        y = np.where(y <= -3, 0.0, np.where(y >= 3, y, y * (y + 3) / 6))
    elif wl["act"] == "gelu":
        y = y * 0.5 * (1 + _erf(y / math.sqrt(2)))
    elif wl["act"] == "softmax":
        e = np.exp(y - y.max(1, keepdims=True))
        y = e / e.sum(1, keepdims=True)
    if wl["norm"] != "none":
        G = wl["C_out"] if wl["norm"] == "instance" else wl["num_groups"]
        N, C = y.shape[:2]
        yg = y.reshape(N, G, -1)
        mu = yg.mean(2, keepdims=True)
        var = yg.var(2, keepdims=True)
        y = ((yg - mu) / np.sqrt(var + wl["eps"])).reshape(y.shape)
        if wl["affine"]:
            sh = (1, C) + (1,) * (y.ndim - 2)
            y = y * p["gamma"].astype(np.float64).reshape(sh) + p["beta"].astype(np.float64).reshape(sh)
    y = y / wl["divide_by"]
    if wl["reduce"] == "mean":
        return y.reshape(y.shape[0], y.shape[1], -1).mean(2)
    if wl["reduce"] == "maxpool":
        P = wl["pool_kernel"] ** wl["pool_repeats"]
        N, C, D, H, W = y.shape
        Dp, Hp, Wp = D // P, H // P, W // P
        c = y[:, :, :Dp * P, :Hp * P, :Wp * P].reshape(N, C, Dp, P, Hp, P, Wp, P)
        return c.max(axis=(3, 5, 7))
    return y


SMALL = {
    "conv2d_in_div_n2": dict(N=2),
    "conv3d_softmax_pool_n128": dict(N=2, in_dims=(10, 11, 13)),
    "conv3d_hswish_gn_mean_n1024": dict(N=2, in_dims=(7, 9, 8)),
    "conv2d_in_div_n128": dict(N=1, C_in=8, C_out=16, in_dims=(1, 12, 11)),
    "convt2d_gelu_gn_n128": dict(N=2, C_in=16, C_out=16, in_dims=(1, 9, 10), groups=8,
                                 num_groups=8),
    "convt2d_dense_gelu_gn_n128": dict(N=2, C_in=6, C_out=8, in_dims=(1, 7, 9), num_groups=4),
    "conv2d_s2p1_in_div_n128": dict(N=1, C_in=8, C_out=16, in_dims=(1, 13, 12)),
    "convt2d_s2_gelu_gn_n128": dict(N=2, C_in=16, C_out=16, in_dims=(1, 6, 7)),
    "conv2d_in_div_n128_bf16": dict(N=1, C_in=8, C_out=16, in_dims=(1, 12, 11)),
    "convt2d_gelu_gn_n128_bf16": dict(N=2, C_in=16, C_out=16, in_dims=(1, 9, 10), groups=8,
                                      num_groups=8),
    "convt2d_gelu_gn_n128_bf16x3": dict(N=2, C_in=16, C_out=16, in_dims=(1, 9, 10), groups=8,
                                        num_groups=8),
    "convt2d_s2_gelu_gn_n128_bf16x3": dict(N=2, C_in=16, C_out=16, in_dims=(1, 6, 7)),
}


@pytest.mark.parametrize("name", cnf_inputs.WORKLOAD_ORDER)
@pytest.mark.parametrize("dist", ["normal", "uniform"])
def test_oracle_chain_matches_independent_numpy(name, dist):
    wl = cnf_inputs.workload(name, **SMALL[name])
    x = cnf_inputs.gen_x(wl, dist=dist)
    p = cnf_inputs.gen_params(wl)
    out, idx = oracle.forward(wl, x, **p)
    ref = _reference_numpy(wl, x, p)
    assert out.shape == ref.shape
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    if wl["reduce"] == "mean":
        cf, _ = oracle.forward(wl, x, **p, closed_form_mean=True)
        np.testing.assert_allclose(cf, out, rtol=1e-10, atol=1e-12)


def test_sixteen_bit_rounding_matches_torch():
    """round_to (the input generator's bf16 / fp16 rounding) equals torch's
    conversions bit for bit, including exact ties (round half to even)."""
    import torch
    r = np.random.Generator(np.random.PCG64(5))
    a = (r.standard_normal(4096) * np.exp2(r.integers(-20, 12, 4096))).astype(np.float32)
    # exact bf16 ties: low 16 bits = 0x8000, both parities of the kept part
    u = a.view(np.uint32).copy()
    u[:64] = (u[:64] & 0xFFFF0000) | 0x8000
    u[64:128] = (u[64:128] & 0xFFFE0000) | 0x00018000
    a = u.view(np.float32)
    for dt, tt in (("bf16", torch.bfloat16), ("f16", torch.float16)):
        got = cnf_inputs.round_to(a, dt)
        ref = torch.from_numpy(a).to(tt).to(torch.float32).numpy()
        np.testing.assert_array_equal(got.view(np.uint32), ref.view(np.uint32))
    wl = cnf_inputs.workload("conv2d_in_div_n2", dtype="bf16")
    x = cnf_inputs.gen_x(wl)
    assert (x.view(np.uint32) & 0xFFFF == 0).all()      # representable in bf16
    w = cnf_inputs.gen_params(wl)["w"]
    assert (w.view(np.uint32) & 0xFFFF == 0).all()


def test_inputs_are_per_sample_streams():
    wl = cnf_inputs.workload("conv3d_hswish_gn_mean_n1024", N=6)
    full = cnf_inputs.gen_x(wl)
    np.testing.assert_array_equal(cnf_inputs.gen_x(wl, [4]), full[4:5])
    np.testing.assert_array_equal(cnf_inputs.gen_x(wl, [1, 5]), full[[1, 5]])
    assert full.dtype == np.float32 and full.flags.c_contiguous
    p = cnf_inputs.gen_params(wl)
    bound = 1 / math.sqrt(3 * 64)
    assert np.abs(p["w"]).max() <= bound and np.abs(p["b"]).max() <= bound
    assert (p["gamma"] >= 0.5).all() and (p["gamma"] <= 1.5).all()
    s = cnf_inputs.subset(cnf_inputs.workload("conv2d_in_div_n128"), 4)
    assert s[0] == 0 and s[-1] == 127 and len(s) == 4
