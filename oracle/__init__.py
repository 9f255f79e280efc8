"""fp64 CPU oracle for the fused conv + norm forward path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.  It
shares no code with the HIP library (different language, different headers,
different loop structure) and does not import it.

The primitives live in cnf_oracle.c (plain nested loops in double); this file
loads them with ctypes and chains them in the order the pages state each
problem.  See the header of cnf_oracle.c for the page names ([p27], [p17],
[p6], [p19]) used in the citations.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "cnf_oracle.c")
# CNF_ORACLE_LIB selects another build of the oracle (the ASan one, say)
_LIB_PATH = os.environ.get("CNF_ORACLE_LIB") or os.path.join(_HERE, "liboracle.so")
_ASAN_LIB_PATH = os.path.join(_HERE, "liboracle_asan.so")
_lib = None


def build(force: bool = True, asan: bool = False) -> str:
    """Compile the oracle with gcc (-O2, strict IEEE, OpenMP).  asan=True:
    with ROCm's clang and AddressSanitizer instead (the HIP library's
    host-ASan build uses that compiler's runtime, so both share one), into
    liboracle_asan.so."""
    path = _ASAN_LIB_PATH if asan else _LIB_PATH
    if force or not os.path.exists(path):
        tmp = path + ".tmp"
        cc = ["/opt/rocm/llvm/bin/clang", "-fsanitize=address", "-fno-omit-frame-pointer",
              "-shared-libasan"] if asan else ["gcc"]
        omp = ["-fopenmp=libgomp"] if asan else ["-fopenmp"]
        subprocess.check_call(cc + ["-O2", "-fno-fast-math", "-ffp-contract=off"] + omp +
                              ["-std=c11", "-Wall", "-shared", "-fPIC", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, path)
    return path


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    P, I, L, D = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_double
    lib.orc_conv.argtypes = [I] * 10 + [P] * 4
    lib.orc_conv.restype = I
    lib.orc_conv_transpose2d.argtypes = [I] * 8 + [P] * 4
    lib.orc_conv_transpose2d.restype = I
    for f in ("orc_hardswish", "orc_gelu_erf", "orc_gelu_tanh"):
        getattr(lib, f).argtypes = [P, L]
        getattr(lib, f).restype = None
    lib.orc_softmax_channel.argtypes = [P, I, I, L]
    lib.orc_group_norm.argtypes = [P, I, I, L, I, D, P, P]
    lib.orc_divide.argtypes = [P, L, D]
    lib.orc_mean_spatial.argtypes = [P, I, I, L, P]
    lib.orc_conv_general.argtypes = [I] * 10 + [P] * 7
    lib.orc_conv_general.restype = I
    lib.orc_conv_transpose_general.argtypes = [I] * 10 + [P] * 8
    lib.orc_conv_transpose_general.restype = I
    lib.orc_maxpool3d.argtypes = [P, P, I, I, I, I, I, I, I, I, P, P]
    lib.orc_maxpool3d.restype = I
    lib.orc_gn_mean_closed_form.argtypes = [P, I, I, L, I, D, P, P, P]
    lib.orc_num_threads.restype = I
    _lib = lib
    return lib


def _f32(a):
    if a is None:
        return None
    return np.ascontiguousarray(a, dtype=np.float32)


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def num_threads() -> int:
    return _load().orc_num_threads()


# ---------------------------------------------------------------- primitives
def _axes3(v, two_d, neutral):
    """Per-axis (D, H, W) parameters; a 2-D problem has the neutral value on D."""
    v = (v,) * (2 if two_d else 3) if isinstance(v, int) else tuple(v)
    if two_d:
        v = (neutral,) + v
    return (ctypes.c_int * 3)(*v)


def conv_extent(L, k, stride=1, padding=0, dilation=1):
    """floor((L + 2p - d(k-1) - 1) / s) + 1 ([p6] integer output-size passage)."""
    num = L + 2 * padding - dilation * (k - 1) - 1
    return num // stride + 1 if num >= 0 else 0


def conv_transpose_extent(L, k, stride=1, padding=0, dilation=1, output_padding=0):
    """(L - 1)s - 2p + d(k - 1) + op + 1 ([p19] first trace, output-size formula)."""
    return (L - 1) * stride - 2 * padding + dilation * (k - 1) + output_padding + 1


def conv(x, w, b=None, groups=1, stride=1, padding=0, dilation=1):
    """Grouped cross-correlation (2-D or 3-D).

    x: (N, Ci, [D,] H, W); w: (Co, Ci/groups, [kd,] kh, kw).  Returns float64.
    Stride 1, no padding, dilation 1 runs orc_conv; anything else runs
    orc_conv_general (stride, zero padding, dilation; an int applies to every
    spatial axis, a tuple gives one value per axis).
    """
    if (stride, padding, dilation) != (1, 0, 1):
        return _conv_general(x, w, b, groups, stride, padding, dilation)
    x, w, b = _f32(x), _f32(w), _f32(b)
    two_d = x.ndim == 4
    if two_d:
        x5 = x[:, :, None]
        w5 = w[:, :, None]
    else:
        x5, w5 = x, w
    N, Ci, D, H, W = x5.shape
    Co, _, kd, kh, kw = w5.shape
    y = np.empty((N, Co, D - kd + 1, H - kh + 1, W - kw + 1), dtype=np.float64)
    rc = _load().orc_conv(N, Ci, D, H, W, Co, groups, kd, kh, kw,
                          _ptr(np.ascontiguousarray(x5)), _ptr(np.ascontiguousarray(w5)),
                          _ptr(b), _ptr(y))
    if rc != 0:
        raise ValueError("orc_conv: bad shape")
    return y[:, :, 0] if two_d else y


def _conv_general(x, w, b, groups, stride, padding, dilation):
    x, w, b = _f32(x), _f32(w), _f32(b)
    two_d = x.ndim == 4
    x5 = x[:, :, None] if two_d else x
    w5 = w[:, :, None] if two_d else w
    N, Ci, D, H, W = x5.shape
    Co, _, kd, kh, kw = w5.shape
    s, p, dl = _axes3(stride, two_d, 1), _axes3(padding, two_d, 0), _axes3(dilation, two_d, 1)
    dims = [conv_extent(L, k, s[i], p[i], dl[i]) for i, (L, k) in enumerate(((D, kd), (H, kh), (W, kw)))]
    y = np.empty((N, Co, *dims), dtype=np.float64)
    rc = _load().orc_conv_general(N, Ci, D, H, W, Co, groups, kd, kh, kw, s, p, dl,
                                  _ptr(np.ascontiguousarray(x5)), _ptr(np.ascontiguousarray(w5)),
                                  _ptr(b), _ptr(y))
    if rc != 0:
        raise ValueError("orc_conv_general: bad shape")
    return y[:, :, 0] if two_d else y


def conv_transpose(x, w, b=None, groups=1, stride=1, padding=0, dilation=1, output_padding=0):
    """Grouped transposed conv, 2-D or 3-D, w: (Ci, Co/groups, [kd,] kh, kw).

    2-D with stride 1, no padding, dilation 1 runs orc_conv_transpose2d;
    anything else runs orc_conv_transpose_general.
    """
    x, w, b = _f32(x), _f32(w), _f32(b)
    two_d = x.ndim == 4
    if two_d and (stride, padding, dilation, output_padding) == (1, 0, 1, 0):
        return conv_transpose2d(x, w, b, groups)
    x5 = x[:, :, None] if two_d else x
    w5 = w[:, :, None] if two_d else w
    N, Ci, D, H, W = x5.shape
    _, cog, kd, kh, kw = w5.shape
    Co = cog * groups
    s, p = _axes3(stride, two_d, 1), _axes3(padding, two_d, 0)
    dl, op = _axes3(dilation, two_d, 1), _axes3(output_padding, two_d, 0)
    dims = [conv_transpose_extent(L, k, s[i], p[i], dl[i], op[i])
            for i, (L, k) in enumerate(((D, kd), (H, kh), (W, kw)))]
    y = np.empty((N, Co, *dims), dtype=np.float64)
    rc = _load().orc_conv_transpose_general(N, Ci, D, H, W, Co, groups, kd, kh, kw, s, p, dl, op,
                                            _ptr(np.ascontiguousarray(x5)),
                                            _ptr(np.ascontiguousarray(w5)), _ptr(b), _ptr(y))
    if rc != 0:
        raise ValueError("orc_conv_transpose_general: bad shape")
    return y[:, :, 0] if two_d else y


def conv_transpose2d(x, w, b=None, groups=1):
    """Stride-1, unpadded, grouped transposed conv. w: (Ci, Co/groups, kh, kw)."""
    x, w, b = _f32(x), _f32(w), _f32(b)
    N, Ci, H, W = x.shape
    _, cog, kh, kw = w.shape
    Co = cog * groups
    y = np.empty((N, Co, H + kh - 1, W + kw - 1), dtype=np.float64)
    rc = _load().orc_conv_transpose2d(N, Ci, H, W, Co, groups, kh, kw,
                                      _ptr(x), _ptr(w), _ptr(b), _ptr(y))
    if rc != 0:
        raise ValueError("orc_conv_transpose2d: bad shape")
    return y


def _inplace(fn, y):
    y = np.ascontiguousarray(y, dtype=np.float64).copy()
    fn(_ptr(y), y.size)
    return y


def hardswish(y):
    return _inplace(_load().orc_hardswish, y)


def gelu_erf(y):
    return _inplace(_load().orc_gelu_erf, y)


def gelu_tanh(y):
    return _inplace(_load().orc_gelu_tanh, y)


def softmax_channel(y):
    y = np.ascontiguousarray(y, dtype=np.float64).copy()
    N, C = y.shape[:2]
    _load().orc_softmax_channel(_ptr(y), N, C, int(np.prod(y.shape[2:])))
    return y


def group_norm(y, num_groups, eps=1e-5, gamma=None, beta=None):
    y = np.ascontiguousarray(y, dtype=np.float64).copy()
    N, C = y.shape[:2]
    gamma, beta = _f32(gamma), _f32(beta)
    _load().orc_group_norm(_ptr(y), N, C, int(np.prod(y.shape[2:])), num_groups, eps,
                           _ptr(gamma), _ptr(beta))
    return y


def instance_norm(y, eps=1e-5):
    return group_norm(y, y.shape[1], eps)


def divide(y, d):
    y = np.ascontiguousarray(y, dtype=np.float64).copy()
    _load().orc_divide(_ptr(y), y.size, float(d))
    return y


def mean_spatial(y):
    y = np.ascontiguousarray(y, dtype=np.float64)
    N, C = y.shape[:2]
    out = np.empty((N, C), dtype=np.float64)
    _load().orc_mean_spatial(_ptr(y), N, C, int(np.prod(y.shape[2:])), _ptr(out))
    return out


def maxpool3d(y, k, idx=None):
    """One floor-mode max pool with kernel = stride = k on (N, C, D, H, W);
    k is an int (every axis) or a (kd, kh, kw) tuple.  Returns (out, argmax)."""
    y = np.ascontiguousarray(y, dtype=np.float64)
    N, C, D, H, W = y.shape
    kd, kh, kw = (k, k, k) if isinstance(k, int) else tuple(k)
    shp = (N, C, D // kd, H // kh, W // kw)
    out = np.empty(shp, dtype=np.float64)
    oidx = np.empty(shp, dtype=np.int64)
    if idx is not None:
        idx = np.ascontiguousarray(idx, dtype=np.int64)
    rc = _load().orc_maxpool3d(_ptr(y), _ptr(idx), N, C, D, H, W, kd, kh, kw,
                               _ptr(out), _ptr(oidx))
    if rc != 0:
        raise ValueError("orc_maxpool3d: bad kernel")
    return out, oidx


def gn_mean_closed_form(h, num_groups, eps=1e-5, gamma=None, beta=None):
    h = np.ascontiguousarray(h, dtype=np.float64)
    N, C = h.shape[:2]
    out = np.empty((N, C), dtype=np.float64)
    gamma, beta = _f32(gamma), _f32(beta)
    _load().orc_gn_mean_closed_form(_ptr(h), N, C, int(np.prod(h.shape[2:])), num_groups,
                                    eps, _ptr(gamma), _ptr(beta), _ptr(out))
    return out


# ---------------------------------------------------------------- composition
def pre_norm(wl: dict, x, w, b):
    """Conv (or transposed conv) followed by the activation, in float64."""
    geo = dict(stride=wl.get("stride", 1), padding=wl.get("padding", 0),
               dilation=wl.get("dilation", 1))
    if wl["kind"] == "conv_transpose":
        y = conv_transpose(x, w, b, wl["groups"], output_padding=wl.get("output_padding", 0), **geo)
    else:
        y = conv(x, w, b, wl["groups"], **geo)
    act = wl["act"]
    if act == "hardswish":
        y = hardswish(y)
    elif act == "gelu":
        y = gelu_erf(y)
    elif act == "gelu_tanh":
        y = gelu_tanh(y)
    elif act == "softmax":
        y = softmax_channel(y)
    elif act != "none":
        raise ValueError(act)
    return y


def forward(wl: dict, x, w, b=None, gamma=None, beta=None, closed_form_mean=False):
    """Whole path for one workload on the given samples.

    Returns (out, argmax): out in float64 with the library's output shape,
    argmax (int64 flat index into each (n, c) conv grid) or None.
    Order of steps: conv -> activation -> norm -> divide -> reduction
    ([p27] mean after GroupNorm; [p17] divide after InstanceNorm; [p6]
    softmax, then the two pools; [p19] GELU then GroupNorm).
    """
    y = pre_norm(wl, x, w, b)
    norm = wl["norm"]
    if norm != "none":
        G = wl["C_out"] if norm == "instance" else wl["num_groups"]
        g, bt = (gamma, beta) if wl["affine"] else (None, None)
        if wl["reduce"] == "mean" and closed_form_mean:
            return gn_mean_closed_form(y, G, wl["eps"], g, bt), None
        y = group_norm(y, G, wl["eps"], g, bt)
    if wl["divide_by"] != 1.0:
        y = divide(y, wl["divide_by"])
    red = wl["reduce"]
    if red == "none":
        return y, None
    if red == "mean":
        return mean_spatial(y), None
    if red == "maxpool":
        p = wl["pool_kernel"]
        k = (p, p, p)
        if y.ndim == 4:  # 2-D: pool H and W only, keep D = 1
            y = y[:, :, None]
            k = (1, p, p)
        idx = None
        for _ in range(wl["pool_repeats"]):
            y, idx = maxpool3d(y, k, idx)
        return y, idx
    raise ValueError(red)
