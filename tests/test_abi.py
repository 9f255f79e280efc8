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


def test_missing_library_fails_loudly(monkeypatch, tmp_path):
    # no CPU fallback: without libcnf.so the binding raises instead of computing
    monkeypatch.setattr(cnf, "_lib", None)
    monkeypatch.setattr(cnf, "LIB_PATH", str(tmp_path / "libcnf.so"))
    with pytest.raises(ImportError):
        cnf.load_library()
    with pytest.raises(ImportError):
        cnf.Plan(cnf.make_desc(cnf_inputs.workload("conv2d_in_div_n2")))


def test_abi_version_and_status_strings():
    assert cnf.cnf_abi_version() == cnf.CNF_ABI_VERSION
    for s in range(11):
        assert cnf.cnf_status_string(s).startswith("CNF_")
        assert cnf.cnf_status_string(s) != "CNF_ERR_UNKNOWN"
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
        "conv2d_s2p1_in_div_n128": (128, 128, 64, 64),
        "convt2d_s2_gelu_gn_n128": (128, 64, 256, 256),
        "conv2d_in_div_n128_bf16": (128, 128, 126, 126),
        "convt2d_gelu_gn_n128_bf16": (128, 64, 258, 258),
        "convt2d_gelu_gn_n128_bf16x3": (128, 64, 258, 258),
        "convt2d_s2_gelu_gn_n128_bf16x3": (128, 64, 256, 256),
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
    (lambda d: setattr(d, "stride", 0), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "dilation", 0), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "padding", -1), cnf.CNF_ERR_INVALID_DESC),
    (lambda d: setattr(d, "output_padding", 1), cnf.CNF_ERR_INVALID_DESC),  # conv: must be 0
    (lambda d: setattr(d, "dilation", 9), cnf.CNF_ERR_INVALID_DESC),        # dilated kernel > input
    (lambda d: setattr(d, "C_out", 24), cnf.CNF_OK),          # no specialised family: general one
    (lambda d: setattr(d, "kernel", 5), cnf.CNF_OK),
    (lambda d: setattr(d, "stride", 3), cnf.CNF_OK),
    (lambda d: (setattr(d, "padding", 2), setattr(d, "dilation", 2)), cnf.CNF_OK),
    (lambda d: [d.in_dims.__setitem__(i, 1024) for i in range(3)], cnf.CNF_ERR_UNSUPPORTED),
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
    tiles = 4 * 16   # 126 columns in tiles of 32, 126 rows in tiles of 8
    # partials, the [ci][tap][co] weight copy, one (scale, shift) per (n, c)
    assert p4.workspace_bytes == 128 * tiles * 128 * 3 * 4 + 64 * 9 * 128 * 4 + 128 * 128 * 8
    p5 = cnf.Plan(_desc("convt2d_gelu_gn_n128"))
    # the larger of the single-write kernel's slice triples (1024 units x 32
    # slices x 16 B) and the two-pass fallback's per-channel row-block triples
    # (128 x 64 channels x 65 row blocks x 12 B), then the 16-byte status word
    # of the bounded waits
    assert p5.workspace_bytes == max(1024 * 32 * 16, 128 * 64 * 65 * 3 * 4) + 16
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
    # ... and the combinations no specialised family takes go to the general one
    other = [("conv3d_softmax_pool_n128", dict(kernel=2, act="hardswish")),
             ("conv3d_softmax_pool_n128", dict(C_in=1, act="none"))]
    for name, over in other:
        assert "family=generic" in cnf.Plan(_desc(name, **over)).describe(), (name, over)


def test_transposed_conv_output_padding_rule():
    # 0 <= output_padding < max(stride, dilation)
    d = _desc("convt2d_gelu_gn_n128", output_padding=1)
    assert cnf.cnf_plan_create_status(d) == cnf.CNF_ERR_INVALID_DESC
    for s, dl, op, st in [(2, 1, 1, cnf.CNF_OK), (2, 1, 2, cnf.CNF_ERR_INVALID_DESC),
                          (1, 3, 2, cnf.CNF_OK), (1, 3, 3, cnf.CNF_ERR_INVALID_DESC)]:
        d = _desc("convt2d_gelu_gn_n128", stride=s, dilation=dl, output_padding=op)
        assert cnf.cnf_plan_create_status(d) == st, (s, dl, op)


@pytest.mark.parametrize("name,over,shape", [
    # conv: floor((L + 2p - d(k-1) - 1) / s) + 1
    ("conv2d_in_div_n128", dict(stride=2, padding=1, dilation=2), (128, 128, 63, 63)),
    ("conv2d_in_div_n128", dict(dilation=2, padding=2), (128, 128, 128, 128)),
    ("conv3d_hswish_gn_mean_n1024", dict(stride=2, reduce="none"), (1024, 16, 7, 15, 15)),
    # transposed: (L - 1)s - 2p + d(k-1) + op + 1
    ("convt2d_gelu_gn_n128", dict(stride=2, padding=1, output_padding=1), (128, 64, 512, 512)),
    ("convt2d_gelu_gn_n128", dict(stride=3, dilation=2), (128, 64, 770, 770)),
    ("convt2d_gelu_gn_n128", dict(ndim=3, in_dims=(4, 8, 8), stride=2), (128, 64, 9, 17, 17)),
    # 2-D pool of a strided conv: H and W pooled, D = 1 kept
    ("conv2d_in_div_n2", dict(stride=2, reduce="maxpool", pool_kernel=3, pool_repeats=1),
     (2, 16, 1, 5, 5)),
])
def test_general_geometry_output_shapes(name, over, shape):
    plan = cnf.Plan(_desc(name, **over))
    assert plan.out_shape == shape
    assert "family=generic" in plan.describe()


def test_padded_stride1_convs_use_the_implicit_gemm():
    for name, over, shape in [("conv2d_in_div_n128", dict(padding=1), (128, 128, 128, 128)),
                              ("conv2d_in_div_n128", dict(padding=2), (128, 128, 130, 130)),
                              ("convt2d_dense_gelu_gn_n128", dict(padding=1), (128, 64, 256, 256)),
                              ("convt2d_dense_gelu_gn_n128", dict(padding=2), (128, 64, 254, 254))]:
        plan = cnf.Plan(_desc(name, **over))
        assert "conv2d_igemm" in plan.describe(), (name, over)
        assert plan.out_shape == shape
    # beyond k - 1, or dilated, or strided past 2: the general family
    for over in (dict(padding=3), dict(padding=1, dilation=2), dict(padding=1, stride=3),
                 dict(padding=3, stride=2)):
        assert "family=generic" in cnf.Plan(_desc("conv2d_in_div_n128", **over)).describe(), over


def test_stride2_convs_use_the_implicit_gemm():
    # floor((L + 2p - 3) / 2) + 1, padding 0..2, both channel counts; a
    # transposed conv at stride 2 stays on the general family
    for name, over, shape in [("conv2d_in_div_n128", dict(stride=2, padding=1), (128, 128, 64, 64)),
                              ("conv2d_in_div_n128", dict(stride=2), (128, 128, 63, 63)),
                              ("conv2d_in_div_n128", dict(stride=2, padding=2), (128, 128, 65, 65)),
                              ("conv2d_in_div_n128", dict(stride=2, C_out=64, num_groups=64),
                               (128, 64, 63, 63))]:
        plan = cnf.Plan(_desc(name, **over))
        assert "conv2d_igemm" in plan.describe(), (name, over)
        assert plan.out_shape == shape
    # stride 2 takes input channels in pairs
    assert "family=generic" in cnf.Plan(_desc("conv2d_in_div_n128", stride=2, C_in=3)).describe()
    assert "family=generic" in cnf.Plan(_desc("convt2d_dense_gelu_gn_n128", stride=2)).describe()


def test_sixteen_bit_inputs_plan_on_the_general_family(monkeypatch):
    """16-bit x and w run on the general family, except the grouped 3x3
    ConvTranspose2d + GroupNorm shape of the single-write kernel, which widens
    them on load (its workspace also holds the general family's: its
    fallback), and unpadded stride-1 Conv2d with 64 / 128 output channels,
    W % 8 == 0 and C_in % 16 == 0, which the 16-bit implicit GEMM takes."""
    d = _desc("conv2d_in_div_n128")
    d.dtype = 3
    assert cnf.cnf_plan_create_status(d) == cnf.CNF_ERR_INVALID_DESC
    for dt in ("bf16", "f16"):
        for name in cnf_inputs.PAGE_WORKLOADS:
            plan = cnf.Plan(_desc(name, dtype=dt))
            fam = {"convt2d_gelu_gn_n128": "family=convt2d_grouped8_gn_fused",
                   "conv2d_in_div_n128": "family=conv2d_igemm16"}.get(name, "family=generic")
            assert fam in plan.describe() and f"dtype={dt}" in plan.describe(), (name, plan.describe())
        # the same shape at another width is not the single-write kernel's
        p = cnf.Plan(_desc("convt2d_gelu_gn_n128", dtype=dt, in_dims=(1, 64, 200)))
        assert "family=generic" in p.describe()
        fused = cnf.Plan(_desc("convt2d_gelu_gn_n128", dtype=dt))
        os.environ["CNF_FORCE_GENERIC"] = "1"
        try:
            gen = cnf.Plan(_desc("convt2d_gelu_gn_n128", dtype=dt))
        finally:
            del os.environ["CNF_FORCE_GENERIC"]
        assert "family=generic" in gen.describe()
        assert fused.workspace_bytes >= gen.workspace_bytes
    # the 16-bit implicit GEMM's conditions
    for over in (dict(in_dims=(1, 128, 124)), dict(C_in=24), dict(padding=1), dict(stride=2),
                 dict(C_out=96, num_groups=96)):
        assert "family=generic" in cnf.Plan(_desc("conv2d_in_div_n128", dtype="bf16", **over)).describe(), over
    for over in (dict(in_dims=(1, 9, 8)), dict(C_in=16, C_out=64, num_groups=64)):
        assert "family=conv2d_igemm16" in cnf.Plan(_desc("conv2d_in_div_n128", dtype="f16", **over)).describe(), over
    # its workspace: [N][tiles of 16 rows x 32 columns][C_out][3] partials, the
    # [C_in / 16][tap][co][16] 16-bit weight copy, [N][C_out] (scale, shift)
    p = cnf.Plan(_desc("conv2d_in_div_n128", dtype="bf16"))
    assert p.workspace_bytes == 128 * (8 * 4) * 128 * 3 * 4 + 64 * 9 * 128 * 2 + 128 * 128 * 8
    # 16-bit packed weights of the general family: 16 K entries per step (4 per
    # lane), 2-byte elements
    monkeypatch.setenv("CNF_FORCE_GENERIC", "1")
    p = cnf.Plan(_desc("conv2d_in_div_n128", dtype="bf16"))
    monkeypatch.delenv("CNF_FORCE_GENERIC")
    S = 126 * 126
    T = -(-126 // 1) * -(-126 // 64)   # one-row tiles of 64 columns
    wp = 1 * 9 * 16 * (64 // 16) * 2 * 16 * 4 * 2   # taps x 16 x steps x cobN x 16 x NB x 2 B
    assert p.workspace_bytes == _align(wp) + _align(128 * 128 * T * 16) + _align(128 * 128 * 8)


def test_f32_math_option():
    """f32_math: NATIVE or BF16X3, anything else is an invalid descriptor; the
    split form is named only where the plan's kernel has it (the two
    single-write grouped transposed convs with fp32 inputs), every other plan
    contracts fp32 natively and says nothing."""
    d = _desc("convt2d_gelu_gn_n128")
    d.f32_math = 2
    assert cnf.cnf_plan_create_status(d) == cnf.CNF_ERR_INVALID_DESC
    d.f32_math = -1
    assert cnf.cnf_plan_create_status(d) == cnf.CNF_ERR_INVALID_DESC
    split = cnf.Plan(_desc("convt2d_gelu_gn_n128", f32_math="bf16x3"))
    native = cnf.Plan(_desc("convt2d_gelu_gn_n128"))
    assert "family=convt2d_grouped8_gn_fused" in split.describe()
    assert "contraction=bf16x3" in split.describe()
    assert "contraction=" not in native.describe()
    # the same kernel and workspace either way
    assert split.workspace_bytes == native.workspace_bytes
    up = cnf.Plan(_desc("convt2d_s2_gelu_gn_n128", f32_math="bf16x3"))
    assert "family=convt2d_s2_grouped8_gn_fused" in up.describe() and "contraction=bf16x3" in up.describe()
    for name, over in (("conv2d_in_div_n128", {}), ("conv3d_softmax_pool_n128", {}),
                       ("convt2d_gelu_gn_n128", dict(dtype="bf16")),
                       ("convt2d_gelu_gn_n128", dict(in_dims=(1, 64, 200)))):
        p = cnf.Plan(_desc(name, f32_math="bf16x3", **over))
        assert "contraction=" not in p.describe(), (name, over)


def test_family_routing():
    # the page configurations keep their specialised families ...
    fams = {n: cnf.Plan(_desc(n)).describe().split()[0] for n in cnf_inputs.PAGE_WORKLOADS}
    assert not any("generic" in f for f in fams.values()), fams
    # the other workloads: the 16-bit form of the transposed conv and its
    # stride-2 upsampling form run on single-write kernels, the strided conv on
    # the implicit GEMM, the 16-bit conv on the 16-bit implicit GEMM, the rest
    # on the general family
    special = {"convt2d_gelu_gn_n128_bf16": "family=convt2d_grouped8_gn_fused",
               "convt2d_gelu_gn_n128_bf16x3": "family=convt2d_grouped8_gn_fused",
               "convt2d_s2_gelu_gn_n128_bf16x3": "family=convt2d_s2_grouped8_gn_fused",
               "convt2d_s2_gelu_gn_n128": "family=convt2d_s2_grouped8_gn_fused",
               "conv2d_s2p1_in_div_n128": "family=conv2d_igemm",
               "conv2d_in_div_n128_bf16": "family=conv2d_igemm16"}
    for n in set(cnf_inputs.WORKLOAD_ORDER) - set(cnf_inputs.PAGE_WORKLOADS):
        assert special.get(n, "family=generic") in cnf.Plan(_desc(n)).describe(), n
    # ... and CNF_FORCE_GENERIC=1 sends them to the general one
    os.environ["CNF_FORCE_GENERIC"] = "1"
    try:
        for n in cnf_inputs.WORKLOAD_ORDER:
            assert "family=generic" in cnf.Plan(_desc(n)).describe(), n
    finally:
        del os.environ["CNF_FORCE_GENERIC"]
    assert "generic" not in cnf.Plan(_desc("conv2d_in_div_n2")).describe()


def _align(v):
    return (v + 255) // 256 * 256


def _packed_weights(G, taps, Cgi, Cgo):
    # [group tiles][taps][K steps x 4][channel blocks of 16, NB per wave] floats;
    # groups of at most 8 output channels go P to a tile, 4/P K entries each
    pw2 = 1
    while pw2 < Cgo:
        pw2 *= 2
    P = min(4, 16 // pw2) if (Cgo <= 8 and G >= 2) else 1
    steps = -(-Cgi // (4 // P))
    cob = (Cgo + 15) // 16
    NB = 1 if P > 1 else 4 if cob >= 4 else 2 if cob >= 2 else 1
    cobN = 1 if P > 1 else (cob + NB - 1) // NB
    return _align(-(-G // P) * taps * 4 * steps * cobN * 16 * NB * 4)


def test_general_workspace_layout_sizes(monkeypatch):
    # InstanceNorm, no reduction: packed weights, per-tile triples (16 B),
    # per-channel scale/shift (8 B)
    monkeypatch.setenv("CNF_FORCE_GENERIC", "1")
    p = cnf.Plan(_desc("conv2d_in_div_n128", stride=2, padding=1))
    monkeypatch.delenv("CNF_FORCE_GENERIC")
    S = 64 * 64
    T = (S + 63) // 64
    assert p.workspace_bytes == (_packed_weights(1, 9, 64, 128) + _align(128 * 128 * T * 16)
                                 + _align(128 * 128 * 8))
    # plain conv, nothing after it: the packed weights only
    p = cnf.Plan(_desc("conv2d_in_div_n2", stride=2, norm="none", divide_by=1.0))
    assert p.workspace_bytes == _packed_weights(1, 9, 8, 16)
    # softmax + two 2-pools with argmax: staged conv output, then two ping-pong
    # value + index buffers of the first pool's size
    p = cnf.Plan(_desc("conv3d_softmax_pool_n128", padding=1))
    S = 16 * 32 * 32
    pool1 = 128 * 16 * 8 * 16 * 16
    assert p.workspace_bytes == (_packed_weights(1, 27, 3, 16) + _align(128 * 16 * S * 4)
                                 + 4 * _align(pool1 * 4))
    # strided (upsampling) transposed conv: the single-write plan keeps room for
    # its general-family fallback (stride^2 phases of ceil(256/2)^2 positions
    # each), then its 16-byte wait flag
    p = cnf.Plan(_desc("convt2d_s2_gelu_gn_n128"))
    T = 4 * (128 * 128 // 64)
    assert p.workspace_bytes == (_packed_weights(8, 9, 8, 8) + _align(128 * 64 * T * 16)
                                 + _align(128 * 64 * 8)) + 16


def test_descriptor_layout_matches_the_c_header(tmp_path):
    """sizeof and every field offset of cnf_desc, as gcc lays it out from the
    header, equal the ctypes mirror."""
    import ctypes
    import subprocess
    fields = [f for f, _ in cnf.cnf_desc._fields_]
    src = tmp_path / "layout.c"
    body = "".join(f'    printf("{f} %zu\\n", offsetof(cnf_desc, {f}));\n' for f in fields)
    src.write_text('#include <stdio.h>\n#include <stddef.h>\n#include "cnf.h"\n'
                   'int main(void) {\n    printf("size %zu\\n", sizeof(cnf_desc));\n'
                   + body + "    return 0;\n}\n")
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c11", f"-I{os.path.join(ROOT, 'include')}", str(src),
                           "-o", str(exe)])
    got = dict(l.split() for l in subprocess.check_output([str(exe)], text=True).splitlines())
    assert int(got["size"]) == ctypes.sizeof(cnf.cnf_desc)
    for f in fields:
        assert int(got[f]) == getattr(cnf.cnf_desc, f).offset, f
