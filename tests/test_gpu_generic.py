"""GPU parity of the general kernel family (stride, zero padding, dilation,
output_padding, 2-D and 3-D transposed conv, any channel counts and groups,
2-D pools) against the fp64 oracle, every element.  Also runs the page
configurations, at small sizes, through the general family
(CNF_FORCE_GENERIC=1) so its kernels are checked on those shapes too.

Tolerance as everywhere: |gpu - ref| <= 2e-4 + 1e-3 |ref|; pooling argmax
exact where the window's top two oracle values are further apart than that.
"""
import os
import sys

import pytest

torch = pytest.importorskip("torch")

import cnf_inputs  # noqa: E402
import oracle  # noqa: E402
from parity import check_argmax, check_close, oracle_pre_pool, run_gpu  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(name, force=False, dist="normal", **over):
    wl = cnf_inputs.workload(name, **over)
    _say(f"[generic] {name} {over} force={force} dist={dist}")
    x = cnf_inputs.gen_x(wl, dist=dist)
    p = cnf_inputs.gen_params(wl)
    if force:
        os.environ["CNF_FORCE_GENERIC"] = "1"
    try:
        plan, out, idx = run_gpu(wl, x, p)
    finally:
        os.environ.pop("CNF_FORCE_GENERIC", None)
    assert "family=generic" in plan.describe(), plan.describe()
    ref, ref_idx = oracle.forward(wl, x, **p)
    err = check_close(out.cpu().numpy(), ref, f"{name} {over}")
    if wl["want_argmax"]:
        Pk = wl["pool_kernel"] ** wl["pool_repeats"]
        excl = check_argmax(idx.cpu().numpy(), out.cpu().numpy(), ref_idx, oracle_pre_pool(wl, x, p), Pk, name)
        _say(f"    argmax ok, {excl} near-tie windows excluded")
    _say(f"    max_abs_err={err:.3e}")


GENERAL_CASES = [
    # 2-D conv: stride + padding, InstanceNorm + divide (l2_p17's chain, strided)
    ("conv2d_in_div_n2", dict(stride=2, padding=1)),
    # dilation, channel counts off the 16-row tile, groups with 8 output channels each
    ("conv2d_in_div_n2", dict(C_in=6, C_out=24, groups=3, in_dims=(1, 23, 29), dilation=2,
                              padding=2, act="hardswish", norm="group", num_groups=4, affine=1,
                              divide_by=1.0)),
    # depthwise, k5, stride 2, GELU, no norm, divide
    ("conv2d_in_div_n2", dict(C_in=8, C_out=8, groups=8, kernel=5, stride=2, in_dims=(1, 31, 26),
                              act="gelu", norm="none", divide_by=3.0)),
    # 1x1 conv, stride 3, one output channel, ragged input-channel chunk (70 = 17*4 + 2)
    ("conv2d_in_div_n2", dict(C_in=70, C_out=1, kernel=1, stride=3, in_dims=(1, 20, 22),
                              norm="none", divide_by=1.0)),
    # 40 output channels per group: three 16-row blocks, the last ragged; GroupNorm spanning
    # two conv groups
    ("conv2d_in_div_n2", dict(C_in=4, C_out=80, groups=2, in_dims=(1, 13, 15), padding=1,
                              norm="group", num_groups=1, affine=1, act="gelu_tanh")),
    # 3-D conv, stride 2 + padding, HardSwish + GroupNorm + mean (l2_p27's chain, strided)
    ("conv3d_hswish_gn_mean_n1024", dict(N=2, in_dims=(9, 14, 17), stride=2, padding=1)),
    ("conv3d_hswish_gn_mean_n1024", dict(N=2, in_dims=(8, 10, 12), dilation=2, norm="none",
                                         affine=0, divide_by=2.0)),
    # 3-D conv with padding + channel softmax + two 2-pools + argmax (l2_p6's chain, padded)
    ("conv3d_softmax_pool_n128", dict(N=2, in_dims=(10, 12, 14), padding=1)),
    ("conv3d_softmax_pool_n128", dict(N=1, in_dims=(13, 16, 16), stride=2, kernel=2,
                                      pool_kernel=2, pool_repeats=1)),
    # softmax followed by a norm, no reduction
    ("conv3d_softmax_pool_n128", dict(N=2, in_dims=(6, 9, 11), reduce="none", pool_kernel=0,
                                      pool_repeats=0, want_argmax=0, norm="instance",
                                      num_groups=16)),
    # 2-D pools (H and W only), with a norm in front: pool 3 once, pool 2 twice
    ("conv2d_in_div_n2", dict(in_dims=(1, 26, 31), act="gelu", reduce="maxpool", pool_kernel=3,
                              pool_repeats=1, want_argmax=1)),
    ("conv2d_in_div_n2", dict(in_dims=(1, 30, 27), stride=1, padding=1, reduce="maxpool",
                              pool_kernel=2, pool_repeats=2, want_argmax=1, norm="group",
                              num_groups=4, affine=1)),
    ("conv2d_in_div_n2", dict(in_dims=(1, 30, 27), padding=1, reduce="maxpool", pool_kernel=2,
                              pool_repeats=3, want_argmax=0, norm="none", divide_by=1.0)),
    # transposed conv, stride 2 + padding + output_padding, 8-channel groups, GELU +
    # GroupNorm (l2_p19's chain, upsampling)
    ("convt2d_gelu_gn_n128", dict(N=2, in_dims=(1, 9, 13), stride=2, padding=1,
                                  output_padding=1)),
    # stride 3 with dilation 2, dense, tanh GELU + affine InstanceNorm
    ("convt2d_gelu_gn_n128", dict(N=1, C_in=12, C_out=20, groups=1, in_dims=(1, 7, 8), stride=3,
                                  dilation=2, output_padding=2, act="gelu_tanh", norm="instance")),
    # padding larger than the kernel reach on one side, depthwise
    ("convt2d_gelu_gn_n128", dict(N=2, C_in=8, C_out=8, groups=8, in_dims=(1, 12, 10), stride=2,
                                  padding=2, num_groups=2, act="none")),
    # 3-D transposed conv, stride 2, then mean (closed-form reduction) and a divide
    ("convt2d_gelu_gn_n128", dict(N=2, ndim=3, C_in=8, C_out=16, groups=2, in_dims=(3, 5, 6),
                                  stride=2, output_padding=1, act="hardswish", num_groups=4,
                                  reduce="mean", divide_by=2.0)),
    # transposed conv into a pool with argmax
    ("convt2d_gelu_gn_n128", dict(N=1, C_in=8, C_out=8, groups=1, in_dims=(1, 10, 11), stride=2,
                                  num_groups=1, reduce="maxpool", pool_kernel=2, pool_repeats=2,
                                  want_argmax=1)),
    # phases of unequal size (output extents not multiples of the stride), 3-D dilated
    ("convt2d_gelu_gn_n128", dict(N=1, in_dims=(1, 7, 9), stride=3, padding=2, output_padding=1)),
    ("convt2d_gelu_gn_n128", dict(N=1, ndim=3, C_in=8, C_out=8, groups=1, num_groups=2,
                                  in_dims=(3, 4, 5), stride=2, dilation=2, output_padding=1)),
    # wide outputs (one-row, 64-column tiles) with ragged last column tiles
    ("convt2d_s2_gelu_gn_n128", dict(N=2, in_dims=(1, 9, 30))),
    ("convt2d_s2_gelu_gn_n128", dict(N=1, C_in=8, C_out=8, groups=1, num_groups=2,
                                     in_dims=(1, 5, 40), stride=3, output_padding=2)),
    # several conv groups per 16-row MFMA tile (block-diagonal weights): 3 channels
    # per group with 3 groups, depthwise with 5 groups (last tile partly empty),
    # a transposed conv with 7 groups of 1 output channel
    ("conv2d_in_div_n2", dict(N=2, C_in=9, C_out=9, groups=3, in_dims=(1, 11, 13), padding=1,
                              norm="group", num_groups=3, affine=1)),
    ("conv2d_in_div_n2", dict(N=2, C_in=5, C_out=5, groups=5, in_dims=(1, 12, 50), stride=2,
                              norm="none", divide_by=1.0, act="hardswish")),
    ("convt2d_gelu_gn_n128", dict(N=2, C_in=14, C_out=7, groups=7, num_groups=7,
                                  in_dims=(1, 6, 9), stride=2)),
    # stride-1 page shapes through non-default padding (the specialised families decline)
    ("convt2d_gelu_gn_n128", dict(N=1, in_dims=(1, 20, 30), padding=1)),
    ("conv2d_in_div_n128", dict(N=1, C_in=16, in_dims=(1, 25, 40), padding=3)),
    # planes of at least 4096 outputs: the flat apply pass (chunks spanning two planes)
    ("conv2d_in_div_n2", dict(N=2, C_out=24, in_dims=(1, 66, 70), padding=1, norm="group",
                              num_groups=6, affine=1)),
    # stride-2 3x3 transposed conv over 8-channel groups: its own direct conv stage
    # (ragged rows and column blocks, narrow and exact widths, a 1x1 input, no
    # statistics, a norm group spanning two conv groups, InstanceNorm)
    ("convt2d_s2_gelu_gn_n128", dict(N=1, in_dims=(1, 7, 70))),
    ("convt2d_s2_gelu_gn_n128", dict(N=3, C_in=16, C_out=16, groups=2, num_groups=2,
                                     in_dims=(1, 13, 5), act="hardswish")),
    ("convt2d_s2_gelu_gn_n128", dict(N=2, in_dims=(1, 6, 64), norm="instance", affine=1)),
    ("convt2d_s2_gelu_gn_n128", dict(N=2, C_in=8, C_out=8, groups=1, num_groups=1,
                                     in_dims=(1, 1, 1))),
    ("convt2d_s2_gelu_gn_n128", dict(N=2, in_dims=(1, 5, 33), norm="none", divide_by=2.0,
                                     act="gelu_tanh")),
    ("convt2d_s2_gelu_gn_n128", dict(N=1, in_dims=(1, 10, 20), num_groups=4)),
]


@pytest.mark.parametrize("name,over", GENERAL_CASES)
def test_general_family_every_element(name, over):
    _case(name, **over)


FORCED = [
    ("conv2d_in_div_n2", {}),
    ("conv3d_softmax_pool_n128", dict(N=2)),
    ("conv3d_hswish_gn_mean_n1024", dict(N=3)),
    ("conv2d_in_div_n128", dict(N=1, C_in=16, in_dims=(1, 30, 70))),
    ("convt2d_gelu_gn_n128", dict(N=1, in_dims=(1, 19, 33))),
    ("convt2d_dense_gelu_gn_n128", dict(N=1, C_in=8, in_dims=(1, 12, 20))),
    # l2_p17's chain strided (the implicit GEMM takes these unforced)
    ("conv2d_in_div_n2", dict(N=1, C_in=64, C_out=128, in_dims=(1, 21, 19), stride=2, padding=1)),
    ("conv2d_s2p1_in_div_n128", dict(N=2, C_in=12, in_dims=(1, 7, 130))),
]


@pytest.mark.parametrize("name,over", FORCED)
def test_page_configurations_through_the_general_family(name, over):
    _case(name, force=True, **over)


# 16-bit inputs (x and w rounded to bf16 / fp16 by the input generator, so the
# oracle sees the same values); the products are exact in fp32 and accumulate in
# fp32, so the same tolerance applies.
SIXTEEN_BIT_CASES = [
    ("conv2d_in_div_n2", {}),
    ("conv2d_in_div_n128", dict(N=1, C_in=16, in_dims=(1, 66, 66))),  # flat apply pass
    ("conv2d_in_div_n128", dict(N=1, C_in=16, in_dims=(1, 30, 70))),
    ("conv3d_hswish_gn_mean_n1024", dict(N=2)),
    ("conv3d_softmax_pool_n128", dict(N=2)),
    ("convt2d_gelu_gn_n128", dict(N=1, in_dims=(1, 19, 33))),
    ("convt2d_dense_gelu_gn_n128", dict(N=1, C_in=24, in_dims=(1, 12, 20))),
    ("conv2d_s2p1_in_div_n128", dict(N=2, C_in=40, in_dims=(1, 21, 70))),
    ("convt2d_s2_gelu_gn_n128", dict(N=2, in_dims=(1, 9, 30))),
    ("conv2d_in_div_n2", dict(C_in=6, C_out=24, groups=3, in_dims=(1, 23, 29), dilation=2,
                              padding=2, act="hardswish", norm="group", num_groups=4, affine=1,
                              divide_by=1.0)),
    ("conv2d_in_div_n2", dict(C_in=8, C_out=8, groups=8, kernel=5, stride=2, in_dims=(1, 31, 26),
                              act="gelu", norm="none", divide_by=3.0)),
    ("conv2d_in_div_n2", dict(C_in=70, C_out=1, kernel=1, stride=3, in_dims=(1, 20, 22),
                              norm="none", divide_by=1.0)),
    ("convt2d_gelu_gn_n128", dict(N=2, ndim=3, C_in=8, C_out=16, groups=2, in_dims=(3, 5, 6),
                                  stride=2, output_padding=1, act="hardswish", num_groups=4,
                                  reduce="mean", divide_by=2.0)),
    ("conv2d_in_div_n2", dict(in_dims=(1, 30, 27), stride=1, padding=1, reduce="maxpool",
                              pool_kernel=2, pool_repeats=2, want_argmax=1, norm="group",
                              num_groups=4, affine=1)),
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("name,over", SIXTEEN_BIT_CASES)
def test_sixteen_bit_inputs_every_element(name, over, dtype):
    _case(name, dtype=dtype, **over)


def _stride2_cases(count, seed=4242):
    """Seeded shapes for the stride-2 3x3 transposed conv over 8-channel groups (the
    general family's direct stage): sizes, groups, activation, norm, affine, divide."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        g = int(rng.integers(1, 5))
        norm = ["group", "instance", "none"][int(rng.integers(0, 3))]
        over = dict(N=int(rng.integers(1, 4)), C_in=8 * g, C_out=8 * g, groups=g,
                    in_dims=(1, int(rng.integers(1, 40)), int(rng.integers(1, 140))),
                    act=["gelu", "gelu_tanh", "hardswish", "none"][int(rng.integers(0, 4))],
                    norm=norm, affine=int(rng.integers(0, 2)) if norm != "none" else 0,
                    divide_by=[1.0, 2.0][int(rng.integers(0, 2))])
        if norm == "group":
            over["num_groups"] = [d for d in (1, 2, 4, 8) if (8 * g) % d == 0][int(rng.integers(0, 4))]
        out.append(over)
    return out


STRIDE2_CASES = _stride2_cases(12)


@pytest.mark.parametrize("over", STRIDE2_CASES)
def test_stride2_transposed_conv_random_shapes(over):
    _case("convt2d_s2_gelu_gn_n128", **over)


import random_descriptors  # noqa: E402

RANDOM_CASES = random_descriptors.cases(48) + random_descriptors.cases(48, seed=77, first_id=950)


@pytest.mark.parametrize("wl", RANDOM_CASES, ids=[w["name"] for w in RANDOM_CASES])
def test_random_descriptor_sweep(wl):
    """48 seeded random small descriptors (geometry, groups, activation, norm,
    reduction, input type), every element against the oracle."""
    _say(f"[random] {wl}")
    x = cnf_inputs.gen_x(wl)
    p = cnf_inputs.gen_params(wl)
    plan, out, idx = run_gpu(wl, x, p)
    ref, ref_idx = oracle.forward(wl, x, **p)
    err = check_close(out.cpu().numpy(), ref, wl["name"])
    if wl["want_argmax"]:
        Pk = wl["pool_kernel"] ** wl["pool_repeats"]
        excl = check_argmax(idx.cpu().numpy(), out.cpu().numpy(), ref_idx, oracle_pre_pool(wl, x, p), Pk, wl["name"])
        _say(f"    argmax ok, {excl} near-tie windows excluded")
    _say(f"    {plan.describe().split()[0][:20]} max_abs_err={err:.3e}")


SPECIALISED_CASES = random_descriptors.specialised_cases(36)


@pytest.mark.parametrize("wl", SPECIALISED_CASES, ids=[w["name"] for w in SPECIALISED_CASES])
def test_random_specialised_family_sweep(wl):
    """36 seeded random shapes inside the specialised families' supported sets
    (whichever family the planner picks), every element against the oracle."""
    _say(f"[random-spec] {wl}")
    x = cnf_inputs.gen_x(wl)
    p = cnf_inputs.gen_params(wl)
    plan, out, idx = run_gpu(wl, x, p)
    ref, ref_idx = oracle.forward(wl, x, **p)
    err = check_close(out.cpu().numpy(), ref, wl["name"])
    if wl["want_argmax"]:
        Pk = wl["pool_kernel"] ** wl["pool_repeats"]
        excl = check_argmax(idx.cpu().numpy(), out.cpu().numpy(), ref_idx, oracle_pre_pool(wl, x, p), Pk, wl["name"])
        _say(f"    argmax ok, {excl} near-tie windows excluded")
    _say(f"    {plan.describe().split()[0][:40]} max_abs_err={err:.3e}")


def test_general_family_uniform_inputs():
    _case("conv2d_in_div_n2", dist="uniform", stride=2, padding=1, norm="group", num_groups=2,
          affine=1)


def test_general_family_repeatable_bitwise():
    wl = cnf_inputs.workload("conv2d_in_div_n2", C_in=6, C_out=24, groups=3, stride=2, padding=1,
                             norm="group", num_groups=4, affine=1)
    x = cnf_inputs.gen_x(wl)
    p = cnf_inputs.gen_params(wl)
    _, a, _ = run_gpu(wl, x, p)
    _, b, _ = run_gpu(wl, x, p)
    assert torch.equal(a, b)
