"""GPU parity: the HIP path through the C ABI against the fp64 oracle.

Small cases cover every element (several tiles and ragged tails per kernel
family, other option combinations, both input distributions); full-size
cases run the whole batch in the launch configuration the benchmark times
and compare the seeded sample subset the oracle can afford (samples are
independent).  Tolerance: |gpu - ref| <= 2e-4 + 1e-3 |ref| element-wise;
pooling argmax exact wherever the window's top two oracle values are
further apart than that tolerance.
"""
import sys

import numpy as np
import pytest

torch = pytest.importorskip("torch")

import cnf_inputs  # noqa: E402
import oracle  # noqa: E402
from parity import check_argmax, check_close, oracle_pre_pool, run_gpu  # noqa: E402

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _case(name, dist="normal", **over):
    wl = cnf_inputs.workload(name, **over)
    _say(f"[parity] {name} {over} dist={dist}")
    x = cnf_inputs.gen_x(wl, dist=dist)
    p = cnf_inputs.gen_params(wl)
    plan, out, idx = run_gpu(wl, x, p)
    ref, ref_idx = oracle.forward(wl, x, **p)
    err = check_close(out.cpu().numpy(), ref, f"{name} {over}")
    if ref_idx is not None:
        Pk = wl["pool_kernel"] ** wl["pool_repeats"]
        excl = check_argmax(idx.cpu().numpy(), ref_idx, oracle_pre_pool(wl, x, p), Pk, name)
        _say(f"    argmax ok, {excl} near-tie windows excluded")
    _say(f"    {plan.describe().split()[0]} max_abs_err={err:.3e}")


# ---------------------------------------------------------------- small, every element
SMALL_CASES = [
    # small conv, one workgroup per sample
    ("conv2d_in_div_n2", {}),
    ("conv2d_in_div_n2", dict(N=3, in_dims=(1, 17, 23))),
    ("conv2d_in_div_n2", dict(N=2, norm="group", num_groups=4, affine=1, act="hardswish",
                              divide_by=1.0)),
    ("conv2d_in_div_n2", dict(N=1, C_in=3, in_dims=(1, 9, 40), act="gelu")),
    # conv3d + softmax + 4^3 pool
    ("conv3d_softmax_pool_n128", dict(N=3)),
    ("conv3d_softmax_pool_n128", dict(N=2, in_dims=(10, 14, 22))),
    ("conv3d_softmax_pool_n128", dict(N=2, in_dims=(11, 9, 13), pool_kernel=4, pool_repeats=1)),
    ("conv3d_softmax_pool_n128", dict(N=2, act="none")),
    # conv3d k4 + GroupNorm + mean
    ("conv3d_hswish_gn_mean_n1024", dict(N=3)),
    ("conv3d_hswish_gn_mean_n1024", dict(N=2, in_dims=(9, 20, 32))),
    ("conv3d_hswish_gn_mean_n1024", dict(N=2, num_groups=2, affine=0)),
    ("conv3d_hswish_gn_mean_n1024", dict(N=2, num_groups=16, act="gelu")),
    ("conv3d_hswish_gn_mean_n1024", dict(N=2, norm="none", affine=0, divide_by=3.0)),
    # conv2d 64->128 implicit GEMM + InstanceNorm + divide
    ("conv2d_in_div_n128", dict(N=2, C_in=8, in_dims=(1, 20, 70))),
    ("conv2d_in_div_n128", dict(N=1, C_in=64, in_dims=(1, 19, 131))),
    ("conv2d_in_div_n128", dict(N=2, C_in=12, in_dims=(1, 9, 9), norm="group", num_groups=32,
                                affine=1)),
    # grouped ConvTranspose2d + GELU + GroupNorm
    ("convt2d_gelu_gn_n128", dict(N=2, C_in=16, C_out=16, groups=2, num_groups=2,
                                  in_dims=(1, 13, 20))),
    ("convt2d_gelu_gn_n128", dict(N=1, in_dims=(1, 7, 36))),
    ("convt2d_gelu_gn_n128", dict(N=2, C_in=8, C_out=8, groups=1, num_groups=1,
                                  in_dims=(1, 5, 4), act="none")),
    # single-write cooperative transposed conv (W = 256): odd output height
    # (last step with one row), column tiles with masked rows, units that do
    # not fill a round, tail steps spread as extra row tiles, several rounds
    # with the XCD-grouped slice mapping; heights it does not take run the
    # two-pass kernels
    ("convt2d_gelu_gn_n128", dict(N=2, C_in=16, C_out=16, groups=2, num_groups=2,
                                  in_dims=(1, 30, 256))),
    ("convt2d_gelu_gn_n128", dict(N=1, in_dims=(1, 21, 256))),
    ("convt2d_gelu_gn_n128", dict(N=3, C_in=8, C_out=8, groups=1, num_groups=1,
                                  in_dims=(1, 1, 256), act="hardswish")),
    ("convt2d_gelu_gn_n128", dict(N=3, in_dims=(1, 127, 256), act="none")),  # odd tail step
    ("convt2d_gelu_gn_n128", dict(N=3, in_dims=(1, 126, 256))),
    ("convt2d_gelu_gn_n128", dict(N=3, in_dims=(1, 128, 256), act="hardswish")),
    ("convt2d_gelu_gn_n128", dict(N=2, in_dims=(1, 256, 256))),
    # tanh-form GELU in every family that takes an activation
    ("conv2d_in_div_n2", dict(N=2, act="gelu_tanh")),
    ("conv3d_softmax_pool_n128", dict(N=2, act="gelu_tanh")),
    ("conv3d_hswish_gn_mean_n1024", dict(N=2, act="gelu_tanh")),
    ("convt2d_gelu_gn_n128", dict(N=2, in_dims=(1, 30, 256), act="gelu_tanh")),
    ("convt2d_gelu_gn_n128", dict(N=2, in_dims=(1, 9, 20), act="gelu_tanh")),
    # norm groups other than the conv groups, InstanceNorm, affine InstanceNorm
    ("convt2d_gelu_gn_n128", dict(N=2, in_dims=(1, 11, 28), num_groups=4)),
    ("convt2d_gelu_gn_n128", dict(N=2, in_dims=(1, 11, 28), num_groups=16)),
    ("convt2d_gelu_gn_n128", dict(N=2, in_dims=(1, 30, 256), num_groups=2)),
    ("convt2d_gelu_gn_n128", dict(N=2, in_dims=(1, 13, 20), norm="instance", affine=1)),
    ("conv2d_in_div_n128", dict(N=2, C_in=8, in_dims=(1, 21, 37), affine=1)),
    # implicit GEMM with 64 output channels (8-row tiles) and with an activation
    ("conv2d_in_div_n128", dict(N=2, C_in=8, C_out=64, in_dims=(1, 19, 70), norm="group",
                                num_groups=8, affine=1)),
    ("conv2d_in_div_n128", dict(N=1, C_in=12, in_dims=(1, 13, 40), act="hardswish")),
    # implicit GEMM second pass: the divide alone (uniform scale), no pass at all, and
    # one GroupNorm group over all 128 channels (each lane folds many tile partials)
    ("conv2d_in_div_n128", dict(N=2, C_in=8, in_dims=(1, 17, 45), norm="none")),
    ("conv2d_in_div_n128", dict(N=1, C_in=8, in_dims=(1, 12, 66), norm="none", divide_by=1.0,
                                act="gelu")),
    ("conv2d_in_div_n128", dict(N=2, C_in=8, in_dims=(1, 30, 140), norm="group", num_groups=1,
                                affine=1)),
    # planes of at least 4096 outputs: the flat apply pass (chunks spanning two planes,
    # a ragged last chunk; with statistics and divide-only)
    ("conv2d_in_div_n128", dict(N=3, C_in=8, in_dims=(1, 66, 70))),
    ("conv2d_in_div_n128", dict(N=1, C_in=8, C_out=64, in_dims=(1, 66, 66), norm="none")),
    # dense transposed conv (groups 1) on the implicit GEMM: padded input, flipped kernel
    ("convt2d_dense_gelu_gn_n128", dict(N=2, C_in=8, C_out=64, in_dims=(1, 9, 20))),
    ("convt2d_dense_gelu_gn_n128", dict(N=2, C_in=16, C_out=128, in_dims=(1, 14, 61),
                                        norm="instance", act="gelu_tanh")),
    ("convt2d_dense_gelu_gn_n128", dict(N=1, C_in=64, in_dims=(1, 33, 66))),
    # zero-padded stride-1 convs ("same" padding) and padded dense transposed convs on
    # the implicit GEMM
    ("conv2d_in_div_n128", dict(N=2, C_in=8, in_dims=(1, 20, 70), padding=1)),
    ("conv2d_in_div_n128", dict(N=1, C_in=12, C_out=64, in_dims=(1, 9, 33), padding=2,
                                act="gelu", norm="group", num_groups=8, affine=1)),
    ("convt2d_dense_gelu_gn_n128", dict(N=2, C_in=8, in_dims=(1, 11, 19), padding=1)),
    ("convt2d_dense_gelu_gn_n128", dict(N=1, C_in=8, C_out=128, in_dims=(1, 12, 40), padding=2,
                                        norm="instance")),
]


@pytest.mark.parametrize("name,over", SMALL_CASES)
def test_small_every_element(name, over):
    _case(name, **over)


@pytest.mark.parametrize("name,over", [
    ("conv2d_in_div_n2", {}),
    ("conv3d_softmax_pool_n128", dict(N=2)),
    ("conv3d_hswish_gn_mean_n1024", dict(N=2)),
    ("conv2d_in_div_n128", dict(N=1, C_in=16, in_dims=(1, 30, 40))),
    ("convt2d_gelu_gn_n128", dict(N=1, in_dims=(1, 10, 24))),
])
def test_small_uniform_inputs(name, over):
    # the pages' own harness fed U[0,1) inputs: larger means, harder statistics
    _case(name, dist="uniform", **over)


# ---------------------------------------------------------------- full size, sampled
FULL_SUBSET = {
    "conv2d_in_div_n2": 2,
    "conv3d_softmax_pool_n128": 16,
    "conv3d_hswish_gn_mean_n1024": 8,
    "conv2d_in_div_n128": 2,
    "convt2d_gelu_gn_n128": 2,
    "convt2d_dense_gelu_gn_n128": 2,
    "conv2d_s2p1_in_div_n128": 2,
    "convt2d_s2_gelu_gn_n128": 2,
    "conv2d_in_div_n128_bf16": 2,
    "convt2d_gelu_gn_n128_bf16": 2,
}


@pytest.mark.parametrize("name", cnf_inputs.WORKLOAD_ORDER)
def test_full_size_sampled(name):
    wl = cnf_inputs.workload(name)
    _say(f"[parity-full] {name} N={wl['N']}")
    x = cnf_inputs.gen_x(wl)
    p = cnf_inputs.gen_params(wl)
    plan, out, idx = run_gpu(wl, x, p)
    sub = cnf_inputs.subset(wl, FULL_SUBSET[name])
    del x
    got = out[sub].cpu().numpy()
    del out
    torch.cuda.empty_cache()
    xs = cnf_inputs.gen_x(wl, sub)
    ref, ref_idx = oracle.forward(wl, xs, **p)
    err = check_close(got, ref, name)
    if ref_idx is not None:
        Pk = wl["pool_kernel"] ** wl["pool_repeats"]
        excl = check_argmax(idx[sub].cpu().numpy(), ref_idx, oracle_pre_pool(wl, xs, p), Pk, name)
        _say(f"    argmax ok, {excl} near-tie windows excluded")
    _say(f"    {plan.describe().split()[0]} samples={sub} max_abs_err={err:.3e}")


def test_repeatable_bitwise():
    # every kernel merges statistics in a fixed order: two runs agree bit for bit
    for name, over in [("conv3d_hswish_gn_mean_n1024", dict(N=4)),
                       ("convt2d_gelu_gn_n128", dict(N=1, in_dims=(1, 20, 24))),
                       ("conv2d_in_div_n128", dict(N=1, C_in=8, in_dims=(1, 40, 40)))]:
        wl = cnf_inputs.workload(name, **over)
        x = cnf_inputs.gen_x(wl)
        p = cnf_inputs.gen_params(wl)
        _, a, _ = run_gpu(wl, x, p)
        _, b, _ = run_gpu(wl, x, p)
        assert torch.equal(a, b), name


def _fused_slices(Ho):
    # slices per unit of the single-write kernel: at most 32, four steps each
    nst = (Ho + 1) // 2
    return min(32, nst // 4)


# 16-bit x and w through the single-write kernel (widened to fp32 on load): the
# oracle takes the same rounded inputs, so the fp32 tolerance applies.  Shapes:
# one unit; ragged last step with every slice carrying a single row tile; the
# tanh GELU and HardSwish forms; several samples and groups per round.
SIXTEEN_BIT_FUSED = [
    dict(N=1, in_dims=(1, 21, 256)),
    dict(N=3, in_dims=(1, 127, 256), act="none"),
    dict(N=2, in_dims=(1, 30, 256), act="gelu_tanh"),
    dict(N=2, in_dims=(1, 46, 256), act="hardswish"),
    dict(N=5, in_dims=(1, 14, 256)),
]


def _sixteen_bit_fused_random(count, seed=5151):
    """Seeded shapes the single-write kernel takes: W = 256 and heights whose
    output half-rows split evenly into four-step slices (H = 8k - 3 or 8k - 2)."""
    import numpy as np
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(count):
        g = int(rng.integers(1, 5))
        H = 8 * int(rng.integers(1, 9)) - int(rng.integers(2, 4))
        out.append(dict(N=int(rng.integers(1, 4)), C_in=8 * g, C_out=8 * g, groups=g, num_groups=g,
                        in_dims=(1, H, 256),
                        act=["gelu", "gelu_tanh", "hardswish", "none"][int(rng.integers(0, 4))]))
    return out


SIXTEEN_BIT_FUSED += _sixteen_bit_fused_random(6)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("over", SIXTEEN_BIT_FUSED)
def test_sixteen_bit_single_write_every_element(over, dtype):
    wl = cnf_inputs.workload("convt2d_gelu_gn_n128", dtype=dtype, **over)
    _say(f"[parity-16] {over} {dtype}")
    x = cnf_inputs.gen_x(wl)
    p = cnf_inputs.gen_params(wl)
    plan, out, _ = run_gpu(wl, x, p)
    assert "fused" in plan.describe(), plan.describe()
    ref, _ = oracle.forward(wl, x, **p)
    err = check_close(out.cpu().numpy(), ref, f"fused {dtype} {over}")
    _say(f"    max_abs_err={err:.3e}")


def test_fused_convt_wait_never_times_out():
    # the single-write kernel raises a flag (workspace word 0) if a
    # cross-workgroup wait hit its bound; it must stay 0.  Every slice's
    # triple (count, mean, M2, count) sits at float 4 + 4 (unit * S + slice).
    import convolution_normalization_forward_amd as cnf
    wl = cnf_inputs.workload("convt2d_gelu_gn_n128", N=6, in_dims=(1, 70, 256))
    plan = cnf.Plan(cnf.make_desc(wl))
    assert "fused" in plan.describe()
    x = cnf_inputs.gen_x(wl)
    p = cnf_inputs.gen_params(wl)
    dev = "cuda:0"
    t = {k: torch.from_numpy(v).to(dev) for k, v in p.items()}
    out, _, ws = plan.allocate(dev)
    ws.fill_(0xFF)
    for _ in range(3):
        st = cnf.cnf_forward(plan.handle, torch.from_numpy(x).to(dev), t["w"], t["b"], t["gamma"],
                             t["beta"], out, None, ws, plan.workspace_bytes)
        assert st == cnf.CNF_OK
    torch.cuda.synchronize()
    U = wl["N"] * wl["groups"]
    Ho, Wo = plan.out_shape[2], plan.out_shape[3]
    S = _fused_slices(Ho)
    words = ws[:16].view(torch.int32).cpu()
    assert int(words[0]) == 0, "cross-workgroup wait timed out"
    tri = ws[16: 16 + 16 * U * S].view(torch.float32).cpu().numpy().reshape(U, S, 4)
    assert (tri[:, :, 0] > 0).all() and (tri[:, :, 0] == tri[:, :, 3]).all()
    # the slices of a unit partition its 8 x Ho x Wo outputs
    assert (tri[:, :, 0].sum(axis=1) == 8 * Ho * Wo).all()
    ref, _ = oracle.forward(wl, x, **p)
    check_close(out.cpu().numpy(), ref, "fused convt repeated")


def test_empty_batch_is_a_noop():
    import convolution_normalization_forward_amd as cnf
    wl = cnf_inputs.workload("conv3d_hswish_gn_mean_n1024")
    plan = cnf.Plan(cnf.make_desc(wl, N=0))
    assert plan.out_shape == (0, 16)
    p = cnf_inputs.gen_params(wl)
    dev = "cuda:0"
    x = torch.empty((0, 3, 16, 32, 32), device=dev)
    t = {k: torch.from_numpy(v).to(dev) for k, v in p.items()}
    out = torch.empty((1, 16), device=dev)  # a valid pointer; nothing may be written
    out.fill_(7.0)
    st = cnf.cnf_forward(plan.handle, torch.empty(4, device=dev), t["w"], t["b"], t["gamma"],
                         t["beta"], out, None, None, 0)
    torch.cuda.synchronize()
    assert st == cnf.CNF_OK
    assert (out == 7.0).all()
    del x
