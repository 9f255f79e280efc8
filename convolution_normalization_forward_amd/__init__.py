"""Python binding of the fused conv + norm forward library (include/cnf.h).

Thin ctypes marshalling over libcnf.so: the same entry points and names as
the C ABI, plus a descriptor builder and a convenience `forward` that
allocates the output and workspace with torch.  Every step of the path runs
in the library's HIP kernels; there is no Python or CPU compute path, and an
attempt to run without the built library raises.

torch is imported before the library is loaded so that libcnf.so binds to
the same HIP runtime instance torch uses (same soname), and device pointers
and streams from torch are valid for it.
"""
from __future__ import annotations

import ctypes
import os

import torch  # noqa: F401  (loads the HIP runtime first; see module docstring)

_HERE = os.path.dirname(os.path.abspath(__file__))
# CNF_LIB_PATH selects another build of the library (the host-ASan one, say)
LIB_PATH = os.environ.get("CNF_LIB_PATH") or os.path.join(_HERE, "libcnf.so")

CNF_ABI_VERSION = 5

# cnf_status
CNF_OK = 0
CNF_ERR_NULL = 1
CNF_ERR_INVALID_DESC = 2
CNF_ERR_UNSUPPORTED = 3
CNF_ERR_WORKSPACE = 4
CNF_ERR_ALIGNMENT = 5
CNF_ERR_HIP = 6
CNF_ERR_ABI = 7
CNF_ERR_NOMEM = 8
CNF_ERR_WAIT_TIMEOUT = 9
CNF_ERR_SCRATCH = 10
CNF_NOALLOC_SCRATCH_BYTES = 64 << 20

CNF_CONV, CNF_CONV_TRANSPOSE = 0, 1
ACT = {"none": 0, "hardswish": 1, "gelu": 2, "softmax": 3, "gelu_tanh": 4}
NORM = {"none": 0, "group": 1, "instance": 2}
REDUCE = {"none": 0, "mean": 1, "maxpool": 2}
DTYPE = {"f32": 0, "bf16": 1, "f16": 2}
F32_MATH = {"native": 0, "bf16x3": 1}

EXPORTED = ("cnf_plan_create", "cnf_plan_output_shape", "cnf_plan_workspace_size",
            "cnf_forward", "cnf_plan_destroy", "cnf_status_string", "cnf_plan_describe",
            "cnf_abi_version", "cnf_forward_timed", "cnf_forward_check", "cnf_forward_noalloc")


class cnf_desc(ctypes.Structure):
    _fields_ = [
        ("abi_version", ctypes.c_int32),
        ("ndim", ctypes.c_int32),
        ("kind", ctypes.c_int32),
        ("N", ctypes.c_int32),
        ("C_in", ctypes.c_int32),
        ("C_out", ctypes.c_int32),
        ("in_dims", ctypes.c_int32 * 3),
        ("kernel", ctypes.c_int32),
        ("groups", ctypes.c_int32),
        ("has_bias", ctypes.c_int32),
        ("act", ctypes.c_int32),
        ("norm", ctypes.c_int32),
        ("num_groups", ctypes.c_int32),
        ("eps", ctypes.c_float),
        ("affine", ctypes.c_int32),
        ("divide_by", ctypes.c_float),
        ("reduce", ctypes.c_int32),
        ("pool_kernel", ctypes.c_int32),
        ("pool_repeats", ctypes.c_int32),
        ("want_argmax", ctypes.c_int32),
        ("stride", ctypes.c_int32),
        ("padding", ctypes.c_int32),
        ("dilation", ctypes.c_int32),
        ("output_padding", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("f32_math", ctypes.c_int32),
    ]


class CnfError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {cnf_status_string(status)}")


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libcnf.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: run __graft_entry__.build() "
                          "(or python convolution_normalization_forward_amd/_build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    lib.cnf_plan_create.argtypes = [ctypes.POINTER(cnf_desc), ctypes.POINTER(P)]
    lib.cnf_plan_create.restype = ctypes.c_int
    lib.cnf_plan_output_shape.argtypes = [P, ctypes.POINTER(ctypes.c_int64), ctypes.POINTER(ctypes.c_int32)]
    lib.cnf_plan_output_shape.restype = ctypes.c_int
    lib.cnf_plan_workspace_size.argtypes = [P, ctypes.POINTER(ctypes.c_size_t)]
    lib.cnf_plan_workspace_size.restype = ctypes.c_int
    lib.cnf_forward.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P]
    lib.cnf_forward.restype = ctypes.c_int
    lib.cnf_plan_destroy.argtypes = [P]
    lib.cnf_plan_destroy.restype = None
    lib.cnf_status_string.argtypes = [ctypes.c_int]
    lib.cnf_status_string.restype = ctypes.c_char_p
    lib.cnf_plan_describe.argtypes = [P, ctypes.c_char_p, ctypes.c_size_t]
    lib.cnf_plan_describe.restype = ctypes.c_int
    lib.cnf_abi_version.argtypes = []
    lib.cnf_abi_version.restype = ctypes.c_int32
    lib.cnf_forward_timed.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_size_t, P, P, P]
    lib.cnf_forward_timed.restype = ctypes.c_int
    lib.cnf_forward_check.argtypes = [P, P, ctypes.c_size_t, P]
    lib.cnf_forward_check.restype = ctypes.c_int
    lib.cnf_forward_noalloc.argtypes = [P, P, P, P, P, P, P, P, P]
    lib.cnf_forward_noalloc.restype = ctypes.c_int
    _lib = lib
    return lib


# ------------------------------------------------------------ C-ABI mirrors
def cnf_status_string(status: int) -> str:
    return load_library().cnf_status_string(int(status)).decode()


def cnf_abi_version() -> int:
    return int(load_library().cnf_abi_version())


def cnf_plan_create(desc: cnf_desc) -> int:
    """Returns the plan handle (an int); raises CnfError on failure."""
    h = ctypes.c_void_p()
    st = load_library().cnf_plan_create(ctypes.byref(desc), ctypes.byref(h))
    if st != CNF_OK:
        raise CnfError(st, "cnf_plan_create")
    return h.value


def cnf_plan_create_status(desc: cnf_desc) -> int:
    """The raw status of cnf_plan_create (the plan, if any, is destroyed)."""
    h = ctypes.c_void_p()
    st = load_library().cnf_plan_create(ctypes.byref(desc), ctypes.byref(h))
    if st == CNF_OK:
        load_library().cnf_plan_destroy(h)
    return st


def cnf_plan_output_shape(plan: int) -> tuple:
    dims = (ctypes.c_int64 * 5)()
    rank = ctypes.c_int32()
    st = load_library().cnf_plan_output_shape(plan, dims, ctypes.byref(rank))
    if st != CNF_OK:
        raise CnfError(st, "cnf_plan_output_shape")
    return tuple(int(dims[i]) for i in range(rank.value))


def cnf_plan_workspace_size(plan: int) -> int:
    n = ctypes.c_size_t()
    st = load_library().cnf_plan_workspace_size(plan, ctypes.byref(n))
    if st != CNF_OK:
        raise CnfError(st, "cnf_plan_workspace_size")
    return int(n.value)


def cnf_plan_describe(plan: int) -> str:
    buf = ctypes.create_string_buffer(512)
    st = load_library().cnf_plan_describe(plan, buf, 512)
    if st != CNF_OK:
        raise CnfError(st, "cnf_plan_describe")
    return buf.value.decode()


def cnf_plan_destroy(plan: int) -> None:
    if plan:
        load_library().cnf_plan_destroy(plan)


def _ptr(t) -> int | None:
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def cnf_forward(plan: int, x, w, b, gamma, beta, out, argmax, workspace, workspace_bytes: int,
                stream=None) -> int:
    """Launch the path; tensors may be torch tensors (device) or raw ints.

    Returns the cnf_status (0 on success); does not synchronise.
    """
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load_library().cnf_forward(plan, _ptr(x), _ptr(w), _ptr(b), _ptr(gamma),
                                          _ptr(beta), _ptr(out), _ptr(argmax), _ptr(workspace),
                                          int(workspace_bytes), stream))


def cnf_forward_timed(plan: int, x, w, b, gamma, beta, out, argmax, workspace,
                      workspace_bytes: int, stream, event_before: int, event_after: int) -> int:
    """cnf_forward that also records the two hipEvent_t handles (ints) right
    before and after the plan's dominant kernel.  Returns the cnf_status."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load_library().cnf_forward_timed(plan, _ptr(x), _ptr(w), _ptr(b), _ptr(gamma),
                                                _ptr(beta), _ptr(out), _ptr(argmax),
                                                _ptr(workspace), int(workspace_bytes), stream,
                                                event_before, event_after))


def cnf_forward_check(plan: int, workspace, workspace_bytes: int, stream=None) -> int:
    """Waits for the stream; CNF_ERR_WAIT_TIMEOUT if the last call's
    cross-workgroup wait gave up, else CNF_OK.  Returns the cnf_status."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load_library().cnf_forward_check(plan, _ptr(workspace), int(workspace_bytes),
                                                stream))


def cnf_forward_noalloc(plan: int, x, w, b, gamma, beta, out, argmax, stream=None) -> int:
    """cnf_forward on the library's fixed device scratch (no workspace, no
    allocation).  Returns the cnf_status; does not synchronise."""
    if stream is None:
        stream = torch.cuda.current_stream().cuda_stream
    return int(load_library().cnf_forward_noalloc(plan, _ptr(x), _ptr(w), _ptr(b), _ptr(gamma),
                                                  _ptr(beta), _ptr(out), _ptr(argmax), stream))


# ------------------------------------------------------------ conveniences
def make_desc(wl: dict, N: int | None = None) -> cnf_desc:
    """Descriptor from a workload dict (see cnf_inputs.WORKLOADS)."""
    d = cnf_desc()
    d.abi_version = CNF_ABI_VERSION
    d.ndim = wl["ndim"]
    d.kind = CNF_CONV_TRANSPOSE if wl["kind"] == "conv_transpose" else CNF_CONV
    d.N = wl["N"] if N is None else N
    d.C_in, d.C_out = wl["C_in"], wl["C_out"]
    for i, v in enumerate(wl["in_dims"]):
        d.in_dims[i] = v
    d.kernel, d.groups, d.has_bias = wl["kernel"], wl["groups"], wl["has_bias"]
    d.act, d.norm = ACT[wl["act"]], NORM[wl["norm"]]
    d.num_groups = wl["num_groups"]
    d.eps, d.affine, d.divide_by = wl["eps"], wl["affine"], wl["divide_by"]
    d.reduce = REDUCE[wl["reduce"]]
    d.pool_kernel, d.pool_repeats = wl["pool_kernel"], wl["pool_repeats"]
    d.want_argmax = wl["want_argmax"]
    d.stride, d.padding = wl.get("stride", 1), wl.get("padding", 0)
    d.dilation, d.output_padding = wl.get("dilation", 1), wl.get("output_padding", 0)
    d.dtype = DTYPE[wl.get("dtype", "f32")]
    d.f32_math = F32_MATH[wl.get("f32_math", "native")]
    return d


class Plan:
    """RAII wrapper: plan + output shape + workspace size."""

    def __init__(self, desc: cnf_desc):
        self.desc = desc
        self.handle = cnf_plan_create(desc)
        self.out_shape = cnf_plan_output_shape(self.handle)
        self.workspace_bytes = cnf_plan_workspace_size(self.handle)

    def describe(self) -> str:
        return cnf_plan_describe(self.handle)

    def __del__(self):
        h = getattr(self, "handle", None)
        if h:
            try:
                cnf_plan_destroy(h)
            except Exception:  # interpreter shutdown
                pass
            self.handle = None

    def allocate(self, device="cuda"):
        out = torch.empty(self.out_shape, dtype=torch.float32, device=device)
        argmax = (torch.empty(self.out_shape, dtype=torch.int32, device=device)
                  if self.desc.want_argmax else None)
        ws = (torch.empty(max(self.workspace_bytes, 1), dtype=torch.uint8, device=device)
              if self.workspace_bytes else None)
        return out, argmax, ws

    def forward(self, x, w, b=None, gamma=None, beta=None, out=None, argmax=None, workspace=None,
                stream=None):
        if out is None:
            out, argmax, workspace = self.allocate(x.device)
        st = cnf_forward(self.handle, x, w, b, gamma, beta, out, argmax, workspace,
                         self.workspace_bytes, stream)
        if st != CNF_OK:
            raise CnfError(st, "cnf_forward")
        return out, argmax
