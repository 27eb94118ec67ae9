"""A guard on the compiled kernels (CPU only: hipcc cross-compiles gfx950).

The dQ kernel of the attention backward once wrote its keep mask as a
per-element branch, `if (!(j < N && keep_pair(...))) s[r] = -inf`, on the
16-register score vector of a 32x32 MFMA, with keep_pair itself a
short-circuit `dist >= 0 && dist < w`.  The compiler turned each element's
assignment into an exec-masked block with nothing in it: it had written -inf
into a copy of the vector ahead of the branch, reused that register as a
temporary inside the branch and copied the unmasked score back for every lane
with j < N.  Pairs outside the source's distance range kept their scores and
dQ came out O(1) wrong.  Either the unsigned one-compare form of keep_pair or
a select instead of the branch compiles correctly; the kernels use selects.

The signature of that miscompile in the assembly is an `s_and_saveexec_b64
sX, ...` followed directly by `s_or_b64 exec, exec, sX`: a divergent block
whose body was lost.  This test compiles every HIP source of the library to
gfx950 assembly and requires that no kernel contains one.

The same compilation reports each kernel's resources: no kernel may use
scratch (register spills) apart from any listed in KNOWN_SPILLS.  A
change that makes the compiler index an accumulator array dynamically (an
epilogue loop it stops unrolling) shows up here as hundreds of bytes per lane.
"""
import concurrent.futures as cf
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "distance_adaptive_dual_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")


def empty_exec_blocks(asm: str):
    """(function, line) of every exec-masked block with an empty body."""
    lines = [l.strip() for l in asm.splitlines()]
    fn, hits = None, []
    for i, l in enumerate(lines):
        m = re.match(r"^(_Z\w+):", l)
        if m:
            fn = m.group(1)
        m = re.match(r"s_and_saveexec_b64 (s\[\d+:\d+\]), ", l)
        if not m:
            continue
        k = i + 1
        while k < len(lines) and (not lines[k] or lines[k][0] in ";."):
            k += 1
        if k < len(lines) and lines[k] == "s_or_b64 exec, exec, " + m.group(1):
            hits.append((fn, i + 1))
    return hits


def test_detector_finds_an_empty_block():
    asm = "\n".join(["_Zkernel:", "  s_and_saveexec_b64 s[8:9], s[6:7]", "; comment",
                     "  s_or_b64 exec, exec, s[8:9]", "  s_and_saveexec_b64 s[4:5], vcc",
                     "  v_mov_b32_e32 v1, 0", "  s_or_b64 exec, exec, s[4:5]"])
    assert empty_exec_blocks(asm) == [("_Zkernel", 2)]


# Kernels allowed to spill: none.  (The attention backward's dK/dV kernel
# spilled while a per-lane V column gather let the compiler hoist one 64-bit
# offset per element out of its source loop; the forward's epilogue held a
# per-lane output address across the pass loop.)
KNOWN_SPILLS = ()


def _compile(src, out_dir):
    out = os.path.join(out_dir, os.path.basename(src) + ".s")
    cmd = [HIPCC, "-O3", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature",
           "-Xclang", "-packed-fp32-ops", "-I", os.path.join(ROOT, "include"), "-I", CSRC, "-S",
           "--cuda-device-only", "-Rpass-analysis=kernel-resource-usage", src, "-o", out]
    r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    assert r.returncode == 0, r.stdout[-2000:]
    with open(out) as fh:
        return os.path.basename(src), fh.read(), r.stdout


@pytest.fixture(scope="module")
def compiled():
    srcs = sorted(os.path.join(CSRC, f) for f in os.listdir(CSRC) if f.endswith(".hip"))
    tmp = tempfile.mkdtemp(prefix="dar_asm_")
    try:
        with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
            return list(ex.map(lambda s: _compile(s, tmp), srcs))
    finally:
        shutil.rmtree(tmp, ignore_errors=True)


def scratch_by_kernel(remarks: str):
    """{kernel: scratch bytes per lane} from the resource-usage remarks."""
    out, name = {}, None
    for line in remarks.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            out[name] = int(m.group(1))
    return out


def test_no_kernel_has_an_empty_exec_block(compiled):
    bad = {name: empty_exec_blocks(asm)[:3] for name, asm, _ in compiled if empty_exec_blocks(asm)}
    assert not bad, bad


def test_no_unexpected_register_spills(compiled):
    sizes = {}
    for _, _, remarks in compiled:
        sizes.update(scratch_by_kernel(remarks))
    assert len(sizes) > 20  # the remarks were parsed
    bad = {k: v for k, v in sizes.items() if v > 0 and not any(s in k for s in KNOWN_SPILLS)}
    assert not bad, bad
