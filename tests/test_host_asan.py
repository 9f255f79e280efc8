"""Host AddressSanitizer run of the CPU suite.

The C oracle and the host side of the C ABI (descriptor validation, output
shape and workspace arithmetic, family selection, argument checks before any
launch) are built with -fsanitize=address (the HIP library's device code is
built as usual) and the CPU test files run against those builds in a child
process, with the ASan runtime preloaded into the Python interpreter.  Any
ASan report fails the run (halt_on_error).  Leak checking is off: the
interpreter and the ROCm runtime keep allocations alive until exit.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
# every CPU test file but this one
FILES = ["tests/test_abi.py", "tests/test_gelu_form.py", "tests/test_oracle_compose.py",
         "tests/test_oracle_general.py", "tests/test_oracle_pins.py", "tests/test_parity_helpers.py"]


def test_cpu_suite_under_host_asan():
    from convolution_normalization_forward_amd import _build
    import oracle
    try:
        runtime = _build.asan_runtime()
    except RuntimeError as e:
        pytest.skip(str(e))
    lib = _build.build(verbose=False, asan=True)
    olib = oracle.build(force=True, asan=True)
    env = dict(os.environ, LD_PRELOAD=runtime, CNF_LIB_PATH=lib, CNF_ORACLE_LIB=olib,
               ASAN_OPTIONS="detect_leaks=0:verify_asan_link_order=0:halt_on_error=1")
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-m", "not gpu",
                        "-p", "no:cacheprovider"] + FILES + [
                        "-o", "addopts="],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = r.stdout + r.stderr
    assert "AddressSanitizer" not in out, out[-4000:]
    assert r.returncode == 0, out[-4000:]
    # the instrumented builds were the ones loaded
    probe = subprocess.run([sys.executable, "-c",
                            "import sys; sys.path.insert(0, '.');"
                            "import convolution_normalization_forward_amd as c, oracle;"
                            "c.load_library(); oracle._load();"
                            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if '_asan.so' in l}))"],
                           cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert lib in probe.stdout and olib in probe.stdout, probe.stdout + probe.stderr[-2000:]
