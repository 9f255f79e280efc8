"""Build libcnf.so (the HIP library behind include/cnf.h) for gfx950.

Each source is compiled with hipcc in parallel into _build/, then linked into
convolution_normalization_forward_amd/libcnf.so.  Packed-fp32 instruction
selection is switched off for all device code.

build(asan=True) (or `python -m convolution_normalization_forward_amd._build
--asan`) builds libcnf_asan.so into _build_asan/ with AddressSanitizer on the
host code only (device code is built as usual).  Loading it needs clang's ASan
runtime preloaded (asan_runtime() names it) and CNF_LIB_PATH pointing at it;
the binding honours CNF_LIB_PATH.
"""
from __future__ import annotations

import concurrent.futures as cf
import glob
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libcnf.so")
BUILD_ASAN = os.path.join(ROOT, "_build_asan")
LIB_ASAN = os.path.join(PKG, "libcnf_asan.so")
# host-side AddressSanitizer (each -fsanitize= behind -Xarch_host: the device
# code is not instrumented)
ASAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fno-omit-frame-pointer"]
ARCH = os.environ.get("CNF_OFFLOAD_ARCH", "gfx950")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
    f"-I{INCLUDE}", f"-I{CSRC}",
]


# Extra flags per source.  The softmax-pool kernel's inputs and intermediates are
# finite (softmax of finite logits), so NaN-aware min/max is not needed there and
# the DPP row reductions fold into single v_max_f32_dpp / v_add_f32_dpp ops.
FILE_FLAGS = {"k_conv3d_softmax_pool.hip": ["-fno-honor-nans", "-mllvm", "-amdgpu-mfma-vgpr-form"],
              # the general conv's accumulators are loop-carried VGPRs; the default
              # heuristic put the MFMAs on AGPRs and copied every accumulator both
              # ways around each group of MFMAs
              "k_generic.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"]}


def sources():
    return sorted(glob.glob(os.path.join(CSRC, "*.hip")) + glob.glob(os.path.join(CSRC, "*.cpp")))


def asan_runtime() -> str:
    """Path of the ASan runtime shared library of the ROCm clang that hipcc drives."""
    import glob as _glob
    hits = sorted(_glob.glob("/opt/rocm/llvm/lib/clang/*/lib/linux/libclang_rt.asan-x86_64.so"))
    if not hits:
        raise RuntimeError("no libclang_rt.asan-x86_64.so under /opt/rocm/llvm")
    return hits[-1]


def _compile(src: str, asan: bool = False) -> str:
    obj = os.path.join(BUILD_ASAN if asan else BUILD, os.path.basename(src) + ".o")
    cmd = [HIPCC] + FLAGS + (ASAN_FLAGS if asan else []) + FILE_FLAGS.get(os.path.basename(src), []) + \
        ["-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stdout}\n{r.stderr}")
    # host-pass feature warnings are expected; surface anything else
    other = [l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l and l.strip()]
    if other:
        sys.stderr.write("\n".join(other) + "\n")
    return obj


def build(verbose: bool = True, asan: bool = False) -> str:
    out = LIB_ASAN if asan else LIB
    os.makedirs(BUILD_ASAN if asan else BUILD, exist_ok=True)
    srcs = sources()
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, asan), srcs))
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + \
        (["-Xarch_host", "-fsanitize=address", "-shared-libasan"] if asan else []) + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)
    if verbose:
        print(f"built {out} from {len(srcs)} sources")
    return out


if __name__ == "__main__":
    build(asan="--asan" in sys.argv[1:])
