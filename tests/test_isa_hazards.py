"""gfx950 assembly of every kernel source, scanned for a store hazard.

A vector-memory store of more than 8 bytes reads its data registers after
issue; a VALU instruction that overwrites them on the next instruction can
reach them first.  On gfx950 the compiler was seen to merge two 8-byte
buffer stores into one 16-byte store and follow it directly with a VALU
write of its data register (the last lanes then stored the new value).  The
kernels are written so that no such pair is formed; this test compiles each
source to gfx950 assembly with the library's own flags and fails on any
>8-byte store whose data VGPRs a VALU instruction overwrites within the next
two instructions with no s_nop between.
"""
import concurrent.futures as cf
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _regs(tok):
    tok = tok.strip().rstrip(",")
    m = re.match(r"v\[(\d+):(\d+)\]", tok)
    if m:
        return set(range(int(m.group(1)), int(m.group(2)) + 1))
    m = re.match(r"v(\d+)$", tok)
    return {int(m.group(1))} if m else set()


def store_hazards(asm_text):
    ins = [l.strip() for l in asm_text.splitlines()]
    ins = [l for l in ins if l and not l.startswith((";", ".")) and not l.endswith(":")]
    hits = []
    for i, t in enumerate(ins):
        op = t.split()[0]
        if not re.match(r"(buffer|global|flat)_store_(dwordx[34]|b96|b128)$", op):
            continue
        args = t[len(op):].split(",")
        data = _regs(args[0]) if op.startswith("buffer") else _regs(args[1])
        for j in (1, 2):
            if i + j >= len(ins):
                break
            n = ins[i + j]
            nop = n.split()[0]
            if nop.startswith("s_nop"):
                break
            if nop.startswith("v_") and not nop.startswith(("v_mfma", "v_readlane", "v_readfirstlane")):
                if _regs(n[len(nop):].split(",")[0]) & data:
                    hits.append((t, n))
                    break
    return hits


def test_scanner_finds_the_pattern():
    bad = "buffer_store_dwordx4 v[0:3], v10, s[4:7], 0 offen\n  v_mul_f32_e32 v0, v1, v2\n"
    assert store_hazards(bad)
    assert not store_hazards(bad.replace("v_mul_f32_e32 v0", "v_mul_f32_e32 v9"))
    assert not store_hazards("buffer_store_dwordx2 v[0:1], v10, s[4:7], 0 offen\n  v_mul_f32_e32 v0, v1, v2\n")
    assert not store_hazards("global_store_dwordx4 v[8:9], v[0:3], off\n  s_nop 0\n  v_mov_b32_e32 v1, 0\n")
    assert store_hazards("global_store_dwordx4 v[8:9], v[0:3], off\n  v_mov_b32_e32 v1, 0\n")


def _asm(src, out_dir):
    from convolution_normalization_forward_amd import _build
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [_build.HIPCC] + _build.FLAGS + _build.FILE_FLAGS.get(os.path.basename(src), []) + \
        ["-x", "hip", "--cuda-device-only", "-S", src, "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as fh:
        return src, fh.read()


def test_no_kernel_overwrites_wide_store_data(tmp_path):
    from convolution_normalization_forward_amd import _build
    if not os.path.exists(_build.HIPCC):
        pytest.skip("no hipcc")
    srcs = [s for s in _build.sources() if s.endswith(".hip")]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        results = list(ex.map(lambda s: _asm(s, str(tmp_path)), srcs))
    bad = {os.path.basename(s): store_hazards(a)[:3] for s, a in results if store_hazards(a)}
    assert not bad, bad
