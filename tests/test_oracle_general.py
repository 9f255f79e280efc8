"""Pins of the oracle's general convolution, transposed convolution and
per-axis max pool (stride, zero padding, dilation, output_padding; 2-D and
3-D).  CPU only.

Each function is tied to something other than itself:
  * torch's CPU convolutions and max pool in float64 (library routines of
    the same definitions);
  * identities that hold by the mathematics, checked against the separately
    written stride-1 oracle functions: zero padding is a padded input,
    stride is subsampling, dilation is a kernel with zeros inserted, the
    transposed conv is the adjoint of the conv;
  * the output sizes the pages print (l2_p19 first trace: 256 -> 258;
    l2_p6 trace: 14 -> 7 -> 3 under the floor-mode pool formula).
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle

RTOL, ATOL = 1e-12, 1e-12


def _rand(shape, seed):
    return np.random.Generator(np.random.PCG64(seed)).standard_normal(shape).astype(np.float32)


def _t(a):
    return torch.from_numpy(np.asarray(a, dtype=np.float64))


# --------------------------------------------------------------- output sizes
def test_output_size_formulas_page_values():
    # l2_p19 first trace: H_out = (256-1)*1 - 0 + 1*(3-1) + 0 + 1 = 258.
    assert oracle.conv_transpose_extent(256, 3) == 258
    # l2_p6 trace: conv 16x32x32 with k3 -> 14x30x30; pool formula with
    # padding 0, dilation 1, stride = kernel = 2 gives 7x15x15, then 3x7x7.
    assert [oracle.conv_extent(L, 3) for L in (16, 32, 32)] == [14, 30, 30]
    assert [oracle.conv_extent(L, 2, stride=2) for L in (14, 30)] == [7, 15]
    assert [oracle.conv_extent(L, 2, stride=2) for L in (7, 15)] == [3, 7]
    # Hand-computed general cases.
    assert oracle.conv_extent(128, 3, stride=2, padding=1) == 64
    assert oracle.conv_extent(32, 3, dilation=2) == 28
    assert oracle.conv_extent(5, 7) == 0          # kernel larger than input: empty
    assert oracle.conv_transpose_extent(64, 3, stride=2, padding=1, output_padding=1) == 128
    assert oracle.conv_transpose_extent(10, 3, dilation=3, padding=2) == 12


# --------------------------------------------------------------- conv vs torch
CONV_CASES = [
    # ndim, N, Ci, Co, G, L, k, stride, padding, dilation
    (2, 2, 4, 6, 1, 11, 3, 2, 1, 1),
    (2, 1, 6, 4, 2, 9, 3, 1, 2, 2),
    (2, 2, 3, 5, 1, 12, 5, 3, 2, 1),
    (2, 1, 4, 4, 4, 10, 3, 2, 0, 3),     # depthwise
    (2, 1, 2, 3, 1, 7, 1, 2, 0, 1),      # 1x1 strided
    (3, 1, 3, 4, 1, 8, 3, 2, 1, 1),
    (3, 2, 4, 4, 2, 7, 2, 1, 1, 2),
]


@pytest.mark.parametrize("case", CONV_CASES)
def test_general_conv_matches_torch(case):
    nd, N, Ci, Co, G, L, k, s, p, d = case
    x = _rand((N, Ci) + (L,) * nd, 11)
    w = _rand((Co, Ci // G) + (k,) * nd, 12)
    b = _rand((Co,), 13)
    got = oracle.conv(x, w, b, G, stride=s, padding=p, dilation=d)
    fn = F.conv2d if nd == 2 else F.conv3d
    ref = fn(_t(x), _t(w), _t(b), stride=s, padding=p, dilation=d, groups=G).numpy()
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)


def test_general_conv_per_axis_parameters_match_torch():
    x = _rand((1, 3, 6, 9, 8), 21)
    w = _rand((4, 3, 2, 3, 3), 22)
    got = oracle.conv(x, w, None, 1, stride=(1, 2, 3), padding=(0, 1, 2), dilation=(2, 1, 2))
    ref = F.conv3d(_t(x), _t(w), stride=(1, 2, 3), padding=(0, 1, 2), dilation=(2, 1, 2)).numpy()
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)


def test_general_conv_at_defaults_equals_stride1_function():
    x = _rand((2, 4, 9, 10), 31)
    w = _rand((6, 2, 3, 3), 32)
    b = _rand((6,), 33)
    # Force the general function with explicit per-axis defaults.
    got = oracle._conv_general(x, w, b, 2, (1, 1), (0, 0), (1, 1))
    ref = oracle.conv(x, w, b, 2)
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)


# --------------------------------------------------------- conv identities
def test_padding_is_a_zero_padded_input():
    x = _rand((1, 3, 7, 8), 41)
    w = _rand((5, 3, 3, 3), 42)
    got = oracle.conv(x, w, None, 1, padding=2)
    ref = oracle.conv(np.pad(x, ((0, 0), (0, 0), (2, 2), (2, 2))), w, None, 1)
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)


def test_stride_is_subsampling_of_the_stride1_conv():
    x = _rand((1, 2, 6, 13, 11), 51)
    w = _rand((3, 2, 3, 3, 3), 52)
    got = oracle.conv(x, w, None, 1, stride=(2, 3, 2))
    full = oracle.conv(x, w, None, 1)
    np.testing.assert_allclose(got, full[:, :, ::2, ::3, ::2], rtol=RTOL, atol=ATOL)


def test_dilation_is_a_kernel_with_zeros_inserted():
    x = _rand((1, 3, 15, 14), 61)
    w = _rand((4, 3, 3, 3), 62)
    d = 3
    wd = np.zeros((4, 3, 1 + d * 2, 1 + d * 2), np.float32)
    wd[:, :, ::d, ::d] = w
    got = oracle.conv(x, w, None, 1, dilation=d)
    ref = oracle.conv(x, wd, None, 1)
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)


# --------------------------------------------------- transposed conv pins
CONVT_CASES = [
    # ndim, N, Ci, Co, G, L, k, stride, padding, dilation, output_padding
    (2, 2, 4, 6, 1, 7, 3, 2, 1, 1, 1),
    (2, 1, 6, 4, 2, 6, 3, 3, 0, 1, 2),
    (2, 1, 4, 4, 4, 5, 3, 1, 1, 2, 0),   # depthwise, dilated
    (2, 2, 3, 5, 1, 6, 4, 2, 2, 1, 0),
    (2, 1, 8, 8, 8, 9, 3, 1, 0, 1, 0),   # the page's shape family, small
    (3, 1, 3, 4, 1, 4, 3, 2, 1, 1, 1),
    (3, 1, 4, 2, 2, 3, 2, 1, 0, 2, 1),
]


@pytest.mark.parametrize("case", CONVT_CASES)
def test_general_conv_transpose_matches_torch(case):
    nd, N, Ci, Co, G, L, k, s, p, d, op = case
    x = _rand((N, Ci) + (L,) * nd, 71)
    w = _rand((Ci, Co // G) + (k,) * nd, 72)
    b = _rand((Co,), 73)
    got = oracle.conv_transpose(x, w, b, G, stride=s, padding=p, dilation=d, output_padding=op)
    fn = F.conv_transpose2d if nd == 2 else F.conv_transpose3d
    ref = fn(_t(x), _t(w), _t(b), stride=s, padding=p, output_padding=op, groups=G,
             dilation=d).numpy()
    assert got.shape == ref.shape
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)


def test_general_conv_transpose_at_defaults_equals_stride1_function():
    x = _rand((2, 4, 6, 5), 81)
    w = _rand((4, 3, 3, 3), 82)
    b = _rand((6,), 83)
    got = oracle.conv_transpose(x, w, b, 2, stride=(1, 1), padding=(0, 0))  # tuple: general path
    ref = oracle.conv_transpose2d(x, w, b, 2)
    np.testing.assert_allclose(got, ref, rtol=RTOL, atol=ATOL)


@pytest.mark.parametrize("nd,s,p,d,G", [(2, 2, 1, 1, 1), (2, 3, 2, 2, 2), (3, 2, 1, 1, 1),
                                        (2, 1, 0, 1, 1), (3, 1, 2, 2, 2)])
def test_transposed_conv_is_the_adjoint_of_the_conv(nd, s, p, d, G):
    """<conv(x), y> = <x, conv_transpose(y)> with the conv's weight, stride,
    padding and dilation; output_padding picks the transposed output size
    that equals x's size (the extents the conv's floor discards)."""
    Ci, Co, k, L = 4, 6, 3, 11
    x = _rand((1, Ci) + (L,) * nd, 91).astype(np.float64)
    w = _rand((Co, Ci // G) + (k,) * nd, 92)
    cx = oracle.conv(x, w, None, G, stride=s, padding=p, dilation=d)
    Lo = cx.shape[-1]
    op = L - oracle.conv_transpose_extent(Lo, k, s, p, d)
    assert 0 <= op < max(s, d)
    y = _rand(cx.shape, 93)
    ty = oracle.conv_transpose(y, w, None, G, stride=s, padding=p, dilation=d, output_padding=op)
    assert ty.shape == x.shape
    lhs = float(np.sum(cx * y.astype(np.float64)))
    rhs = float(np.sum(x * ty))
    assert abs(lhs - rhs) <= 1e-10 * max(1.0, abs(lhs))


# --------------------------------------------------------------- max pool
@pytest.mark.parametrize("k,H,W", [(2, 9, 8), (3, 10, 11), (1, 4, 5)])
def test_2d_pool_matches_torch_values_and_indices(k, H, W):
    y = _rand((2, 3, H, W), 101).astype(np.float64)
    out, idx = oracle.maxpool3d(y[:, :, None], (1, k, k))
    ro, ri = F.max_pool2d(_t(y), k, return_indices=True)
    np.testing.assert_array_equal(out[:, :, 0], ro.numpy())
    np.testing.assert_array_equal(idx[:, :, 0], ri.numpy())


def test_3d_pool_per_axis_kernel_matches_torch():
    y = _rand((1, 2, 7, 9, 8), 111).astype(np.float64)
    out, idx = oracle.maxpool3d(y, (2, 3, 2))
    ro, ri = F.max_pool3d(_t(y), (2, 3, 2), return_indices=True)
    np.testing.assert_array_equal(out, ro.numpy())
    np.testing.assert_array_equal(idx, ri.numpy())


def test_repeated_2d_pool_through_forward_matches_composed_torch_pools():
    """A 2-D workload with a 3-pool applied twice: the oracle's forward pools
    H and W only (D stays 1), and the carried argmax equals torch's second
    index looked up in its first."""
    wl = dict(id=0, ndim=2, kind="conv", N=1, C_in=2, C_out=3, in_dims=(1, 20, 19), kernel=3,
              groups=1, has_bias=0, act="none", norm="none", num_groups=1, eps=1e-5, affine=0,
              divide_by=1.0, reduce="maxpool", pool_kernel=3, pool_repeats=2, want_argmax=1)
    x = _rand((1, 2, 20, 19), 121)
    w = _rand((3, 2, 3, 3), 122)
    out, idx = oracle.forward(wl, x, w)
    y = _t(oracle.conv(x, w))
    p1, i1 = F.max_pool2d(y, 3, return_indices=True)
    p2, i2 = F.max_pool2d(p1, 3, return_indices=True)
    assert out.shape == (1, 3, 1, 2, 1)
    np.testing.assert_array_equal(out[:, :, 0], p2.numpy())
    composed = torch.gather(i1.flatten(2), 2, i2.flatten(2)).reshape(i2.shape)
    np.testing.assert_array_equal(idx[:, :, 0], composed.numpy())


def test_general_forward_strided_conv_gn_matches_torch_chain():
    """The whole chain on a strided, padded, dilated grouped conv: conv ->
    GELU -> GroupNorm -> divide, against torch's float64 modules."""
    wl = dict(id=0, ndim=2, kind="conv", N=2, C_in=4, C_out=8, in_dims=(1, 13, 12), kernel=3,
              groups=2, has_bias=1, act="gelu", norm="group", num_groups=2, eps=1e-5, affine=1,
              divide_by=3.0, reduce="none", pool_kernel=0, pool_repeats=0, want_argmax=0,
              stride=2, padding=2, dilation=2)
    x = _rand((2, 4, 13, 12), 131)
    w = _rand((8, 2, 3, 3), 132)
    b = _rand((8,), 133)
    g = np.linspace(0.5, 1.5, 8).astype(np.float32)
    bt = np.linspace(-0.2, 0.2, 8).astype(np.float32)
    out, _ = oracle.forward(wl, x, w, b, g, bt)
    y = F.conv2d(_t(x), _t(w), _t(b), stride=2, padding=2, dilation=2, groups=2)
    y = F.gelu(y)
    y = F.group_norm(y, 2, _t(g), _t(bt), eps=1e-5) / 3.0
    np.testing.assert_allclose(out, y.numpy(), rtol=1e-10, atol=1e-10)


@pytest.mark.parametrize("s,p,op", list(itertools.product((1, 2), (0, 1), (0, 1)))[:6])
def test_general_forward_conv_transpose3d_in_affine_matches_torch_chain(s, p, op):
    if op >= s:
        pytest.skip("output_padding must be below the stride")
    wl = dict(id=0, ndim=3, kind="conv_transpose", N=1, C_in=4, C_out=4, in_dims=(3, 4, 5),
              kernel=3, groups=2, has_bias=1, act="hardswish", norm="instance", num_groups=4,
              eps=1e-5, affine=1, divide_by=1.0, reduce="mean", pool_kernel=0, pool_repeats=0,
              want_argmax=0, stride=s, padding=p, dilation=1, output_padding=op)
    x = _rand((1, 4, 3, 4, 5), 141)
    w = _rand((4, 2, 3, 3, 3), 142)
    b = _rand((4,), 143)
    g = np.array([0.7, 1.1, 1.3, 0.9], np.float32)
    bt = np.array([0.1, -0.1, 0.05, 0.0], np.float32)
    out, _ = oracle.forward(wl, x, w, b, g, bt)
    y = F.conv_transpose3d(_t(x), _t(w), _t(b), stride=s, padding=p, output_padding=op, groups=2)
    y = F.hardswish(y)
    y = F.instance_norm(y, weight=_t(g), bias=_t(bt), eps=1e-5)
    np.testing.assert_allclose(out, y.mean(dim=(2, 3, 4)).numpy(), rtol=1e-10, atol=1e-10)
