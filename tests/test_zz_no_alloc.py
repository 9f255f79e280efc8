"""cnf_forward_noalloc (the library's fixed device scratch as the workspace)
against cnf_forward (a caller workspace) through the C ABI.

Two calls of the no-allocation entry point in a row, the second on a smaller
input, so whatever the first call left in the shared scratch must not reach
the second one's results.  Outputs are compared to the parity tolerance
(|a - b| <= 2e-4 + 1e-3 |b|), argmax indices exactly.  Inputs are seeded
normal draws made on the device (both entry points see the same tensors).
"""
import sys

import pytest

torch = pytest.importorskip("torch")

import cnf_inputs  # noqa: E402
import convolution_normalization_forward_amd as cnf  # noqa: E402
from parity import ATOL, RTOL  # noqa: E402

_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _inputs(wl, seed, dev="cuda:0"):
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    dt = _DT[wl.get("dtype", "f32")]
    x = torch.randn(cnf_inputs.x_shape(wl), generator=g, device=dev).to(dt)
    p = cnf_inputs.gen_params(wl)
    t = {k: (torch.from_numpy(v).to(dev) if v is not None else None) for k, v in p.items()}
    t["w"] = t["w"].to(dt)
    return x, t


def _with_workspace(plan, x, t):
    out, idx, ws = plan.allocate(x.device)
    if ws is not None:
        ws.fill_(0xA5)
    st = cnf.cnf_forward(plan.handle, x, t["w"], t["b"], t["gamma"], t["beta"], out, idx, ws,
                         plan.workspace_bytes)
    assert st == cnf.CNF_OK, cnf.cnf_status_string(st)
    return out, idx


def _no_alloc(plan, x, t):
    out, idx, _ = plan.allocate(x.device)
    out.fill_(float("nan"))
    st = cnf.cnf_forward_noalloc(plan.handle, x, t["w"], t["b"], t["gamma"], t["beta"], out, idx)
    assert st == cnf.CNF_OK, cnf.cnf_status_string(st)
    return out, idx


def _same(a, b, what):
    assert a.shape == b.shape, what
    assert torch.isfinite(a).all(), f"{what}: non-finite output"
    bad = (a - b).abs() > ATOL + RTOL * b.abs()
    assert not bad.any(), f"{what}: {int(bad.sum())} of {b.numel()} outside tolerance"


# (workload, first call, second call on a smaller input); first calls leave
# partial statistics and wait flags in the scratch that the second must not see
CASES = [
    # the benchmark's configuration: single-write transposed conv, 128 x 64 x 256 x 256
    ("convt2d_gelu_gn_n128", {}, dict(N=2, in_dims=(1, 62, 256))),
    # implicit GEMM + norm passes; per-tile partials sized by the larger plan
    ("conv2d_in_div_n128", dict(N=3, in_dims=(1, 64, 64)), dict(N=1, in_dims=(1, 20, 70))),
    # general family: strided conv + InstanceNorm
    ("conv2d_s2p1_in_div_n128", dict(N=2, in_dims=(1, 40, 40)), dict(N=1, in_dims=(1, 18, 22))),
    # 16-bit inputs through the single-write kernel
    ("convt2d_gelu_gn_n128_bf16", dict(N=3, in_dims=(1, 126, 256)), dict(N=1, in_dims=(1, 30, 256))),
    # no workspace at all; argmax
    ("conv3d_softmax_pool_n128", dict(N=3), dict(N=1)),
]


@pytest.mark.gpu
@pytest.mark.parametrize("name,first,second", CASES)
def test_no_alloc_matches_workspace_entry(name, first, second):
    plans, refs, gots = [], [], []
    for k, over in enumerate((first, second)):
        wl = cnf_inputs.workload(name, **over)
        plan = cnf.Plan(cnf.make_desc(wl))
        assert plan.workspace_bytes <= cnf.CNF_NOALLOC_SCRATCH_BYTES
        _say(f"[no-alloc] {name} {over} workspace={plan.workspace_bytes} {plan.describe().split()[0]}")
        x, t = _inputs(wl, 9100 + k)
        plans.append((plan, x, t))
        refs.append(_with_workspace(plan, x, t))
    torch.cuda.synchronize()
    # the two no-allocation calls back to back, larger first
    for plan, x, t in plans:
        gots.append(_no_alloc(plan, x, t))
    torch.cuda.synchronize()
    for k, ((out, idx), (ref, ref_idx)) in enumerate(zip(gots, refs)):
        _same(out, ref, f"{name} call {k}")
        if ref_idx is not None:
            assert torch.equal(idx, ref_idx), f"{name} call {k}: argmax differs"
    # the first plan once more, after the smaller call left its partials
    plan, x, t = plans[0]
    out, idx = _no_alloc(plan, x, t)
    torch.cuda.synchronize()
    _same(out, refs[0][0], f"{name} repeated first call")


@pytest.mark.gpu
def test_no_alloc_rejects_plans_beyond_the_scratch():
    # 128 x 64 x 128 x 128 upsampling transposed conv: its per-tile partials
    # need 128 MiB, more than the fixed 64 MiB scratch
    wl = cnf_inputs.workload("convt2d_s2_gelu_gn_n128")
    plan = cnf.Plan(cnf.make_desc(wl))
    assert plan.workspace_bytes > cnf.CNF_NOALLOC_SCRATCH_BYTES
    dev = "cuda:0"
    t = {k: (torch.from_numpy(v).to(dev) if v is not None else None)
         for k, v in cnf_inputs.gen_params(wl).items()}
    x = torch.zeros(16, device=dev)
    out = torch.full((4,), 7.0, device=dev)
    st = cnf.cnf_forward_noalloc(plan.handle, x, t["w"], t["b"], t["gamma"], t["beta"], out, None)
    assert st == cnf.CNF_ERR_SCRATCH, cnf.cnf_status_string(st)
    torch.cuda.synchronize()
    assert (out == 7.0).all()
