"""CPU checks of the C ABI: the library loads, exports every symbol that
include/cnf.h declares, validates descriptors and rejects bad calls before
launching anything.  No compute call is made here (no GPU)."""
import os
import re

import pytest

import cnf_inputs
import convolution_normalization_forward_amd as cnf

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    src = open(os.path.join(ROOT, "include", "cnf.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return set(re.findall(r"\b(cnf_[a-z_]+)\s*\(", src))


def test_library_exports_every_declared_symbol():
    lib = cnf.load_library()
    names = _declared()
    assert {"cnf_plan_create", "cnf_forward", "cnf_plan_destroy"} <= names
    for n in names:
        assert hasattr(lib, n), n
    assert set(cnf.EXPORTED) == names


def test_abi_version_and_status_strings():
    assert cnf.cnf_abi_version() == cnf.CNF_ABI_VERSION
    for s in range(8):
        assert cnf.cnf_status_string(s).startswith("CNF_")
    assert cnf.cnf_status_string(99) == "CNF_ERR_UNKNOWN"


@pytest.mark.parametrize("name", cnf_inputs.WORKLOAD_ORDER)
def test_every_workload_plans_with_expected_shape(name):
    wl = cnf_inputs.workload(name)
    plan = cnf.Plan(cnf.make_desc(wl))
    exp = {
        "conv2d_in_div_n2": (2, 16, 30, 30),
        "conv3d_softmax_pool_n128": (128, 16, 3, 7, 7),
        "conv3d_hswish_gn_mean_n1024": (1024, 16),
        "conv2d_in_div_n128": (128, 128, 126, 126),
        "convt2d_gelu_gn_n128": (128, 64, 258, 258),
        "convt2d_dense_gelu_gn_n128": (128, 64, 258, 258),
    }[name]
    assert plan.out_shape == exp
    assert "family=" in plan.describe()


def _desc(name="conv3d_hswish_gn_mean_n1024", **over):
    return cnf.make_desc(cnf_inputs.workload(name, **over))


@pytest.mark.parametrize("mutate,status", [
    (lambda d: setattr(d, "abi_version", 99), cnf.CNF_ERR_ABI),
    (lambda d: setattr(d, "ndim", 4), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "N", -1), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "groups", 2), cnf.CNF_ERR_INVALID_DESC),      # 2 does not divide C_in=3
    (lambda d: setattr(d, "num_groups", 5), cnf.CNF_ERR_INVALID_DESC),  # 5 does not divide 16
    (lambda d: setattr(d, "eps", 0.0), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "eps", -1.0), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "divide_by", 0.0), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "divide_by", float("nan")), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "kernel", 40), cnf.CNF_ERR_INVALID_DESC),     # output extent < 1
    (lambda d: setattr(d, "kernel", 0), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "act", 9), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "reduce", 7), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "want_argmax", 1), cnf.CNF_ERR_INVALID_DESC),  # argmax without a pool
    (lambda d: setattr(d, "C_out", 24), cnf.CNF_ERR_UNSUPPORTED),        # valid, no kernel family
    (lambda d: setattr(d, "kernel", 5), cnf.CNF_ERR_UNSUPPORTED),
])
def test_descriptor_validation(mutate, status):
    d = _desc()
    mutate(d)
    assert cnf.cnf_plan_create_status(d) == status


def test_pool_larger_than_output_is_invalid():
    d = _desc("conv3d_softmax_pool_n128", pool_kernel=2, pool_repeats=4)
    assert cnf.cnf_plan_create_status(d) == cnf.CNF_ERR_INVALID_DESC


def test_2d_requires_unit_depth():
    d = _desc("conv2d_in_div_n2")
    d.in_dims[0] = 2
    assert cnf.cnf_plan_create_status(d) == cnf.CNF_ERR_INVALID_DESC


def test_null_arguments():
    lib = cnf.load_library()
    import ctypes
    h = ctypes.c_void_p()
    assert lib.cnf_plan_create(None, ctypes.byref(h)) == cnf.CNF_ERR_NULL
    assert lib.cnf_plan_create(ctypes.byref(_desc()), None) == cnf.CNF_ERR_NULL
    assert lib.cnf_plan_workspace_size(None, None) == cnf.CNF_ERR_NULL
    assert lib.cnf_plan_describe(None, None, 0) == cnf.CNF_ERR_NULL
    lib.cnf_plan_destroy(None)  # ignored


def test_forward_rejects_bad_pointers_before_launch():
    # every check below fires before any HIP call, so this runs without a GPU
    plan = cnf.Plan(_desc())
    A = 1 << 20  # a fake, 16-byte-aligned "device" address; never dereferenced
    f = lambda *a: cnf.cnf_forward(plan.handle, *a, stream=0)  # noqa: E731
    assert f(None, A, A, A, A, A, None, None, 0) == cnf.CNF_ERR_NULL
    assert f(A, A, None, A, A, A, None, None, 0) == cnf.CNF_ERR_NULL       # bias required
    assert f(A, A, A, None, A, A, None, None, 0) == cnf.CNF_ERR_NULL       # gamma required
    assert f(A, A, A, A, A, A, A, None, 0) == cnf.CNF_ERR_NULL             # argmax not wanted
    assert f(A + 4, A, A, A, A, A, None, None, 0) == cnf.CNF_ERR_ALIGNMENT
    assert f(A, A, A, A, A, A + 8, None, None, 0) == cnf.CNF_ERR_ALIGNMENT
    big = cnf.Plan(_desc("conv2d_in_div_n128"))
    assert big.workspace_bytes > 0
    g = lambda *a: cnf.cnf_forward(big.handle, *a, stream=0)  # noqa: E731
    assert g(A, A, A, None, None, A, None, None, 0) == cnf.CNF_ERR_WORKSPACE
    assert g(A, A, A, None, None, A, None, A, big.workspace_bytes - 1) == cnf.CNF_ERR_WORKSPACE


def test_workspace_sizes_are_what_the_partials_need():
    p4 = cnf.Plan(_desc("conv2d_in_div_n128"))
    tiles = 2 * 32   # 126 = 64 + 62 columns, 126 rows in blocks of 4
    assert p4.workspace_bytes == 128 * tiles * 128 * 3 * 4 + 64 * 9 * 128 * 4
    p5 = cnf.Plan(_desc("convt2d_gelu_gn_n128"))
    # the larger of the single-write kernel's slice triples (16 B header +
    # 1024 units x 32 slices x 16 B) and the two-pass fallback's per-channel
    # row-block triples (128 x 64 channels x 65 row blocks x 12 B)
    assert p5.workspace_bytes == max(16 + 1024 * 32 * 16, 128 * 64 * 65 * 3 * 4)
    assert cnf.Plan(_desc()).workspace_bytes == 0


def test_supported_matrix_edges():
    # combinations a family advertises are exactly the ones it launches
    ok = [("conv3d_softmax_pool_n128", dict(act="gelu_tanh")),
          ("convt2d_gelu_gn_n128", dict(num_groups=4)),
          ("convt2d_gelu_gn_n128", dict(num_groups=16)),
          ("convt2d_gelu_gn_n128", dict(norm="instance")),
          ("convt2d_gelu_gn_n128", dict(act="gelu_tanh")),
          ("conv2d_in_div_n128", dict(affine=1)),
          ("conv3d_hswish_gn_mean_n1024", dict(act="gelu_tanh"))]
    for name, over in ok:
        assert cnf.cnf_plan_create_status(_desc(name, **over)) == cnf.CNF_OK, (name, over)
    bad = [("conv3d_softmax_pool_n128", dict(kernel=2, act="hardswish")),
           ("conv3d_softmax_pool_n128", dict(C_in=1, act="none"))]
    for name, over in bad:
        assert cnf.cnf_plan_create_status(_desc(name, **over)) == cnf.CNF_ERR_UNSUPPORTED, (name, over)
