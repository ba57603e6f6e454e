"""CPU check of the compiled GEMM kernels (gfx950 assembly, no device).

The GEMM epilogues read their accumulators with inline `v_accvgpr_read`
(so that the compiler keeps them in AGPRs until they are consumed).  The
compiler's hazard check does not look inside inline assembly, so two
orderings must hold by construction and are checked here on the code the
compiler actually emits:
  * an inline read of an accumulator comes at least 18 wait states after
    the last MFMA that wrote it (a 16-pass MFMA result is not interlocked
    against a VALU read);
  * no compiler-generated AGPR write (a copy of an accumulator moved
    through VGPRs) lands on an accumulator shortly before an inline read
    of it.
Distances are counted within basic blocks (a label restarts them); the
epilogue reads sit in straight-line code after the tile boundary.
"""
import os
import re
import subprocess
import tempfile

import pytest

from combine_afd_slot_amd import build

KERNELS = ["_ZN3afd6k_gemmILi1EEEvNS_6DevCtxEPKiNS_7WeightsEi", "_ZN3afd6k_gemmILi2EEEvNS_6DevCtxEPKiNS_7WeightsEi"]
MIN_MFMA_TO_READ = 18


@pytest.fixture(scope="module")
def asm():
    with tempfile.TemporaryDirectory() as d:
        out = os.path.join(d, "k.s")
        cmd = [build.hipcc(), f"--offload-arch={build.ARCH}", "-O3", "-std=c++17", "--cuda-device-only", "-S",
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
               f"-I{os.path.join(build.ROOT, 'include')}", "-x", "hip",
               os.path.join(build.CSRC, "afd_kernels.hip"), "-o", out]
        r = subprocess.run(cmd, capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-2000:]
        return open(out).read()


def _body(asm, name):
    i = asm.index(name + ":")
    return asm[i:asm.index(".Lfunc_end", i)].split("\n")


def _scan(lines):
    """Minimum wait-state distance from an MFMA write / a compiler AGPR write
    to a later inline read of the same AGPR, within straight-line code."""
    inasm = False
    since_mfma, since_write = {}, {}
    d_mfma, d_write = [], []
    for raw in lines:
        t = raw.strip()
        if t.startswith(";;#ASMSTART"):
            inasm = True
            continue
        if t.startswith(";;#ASMEND"):
            inasm = False
            continue
        if not t or t.startswith(";") or (t.startswith(".") and not t.endswith(":")):
            continue
        if t.endswith(":"):  # a block boundary: distances restart (conservative for fall-through)
            since_mfma, since_write = {}, {}
            continue
        m = re.match(r"s_nop (\d+)", t)
        ws = int(m.group(1)) + 1 if m else 1
        for dct in (since_mfma, since_write):
            for k in dct:
                dct[k] += ws
        m = re.match(r"v_mfma\S+ a\[(\d+):(\d+)\]", t)
        if m:
            for r in range(int(m.group(1)), int(m.group(2)) + 1):
                since_mfma[r] = 0
        m = re.match(r"v_accvgpr_write_b32 a(\d+), (\S+)", t)
        if m and not inasm:
            since_write[int(m.group(1))] = 0
        m = re.match(r"v_accvgpr_read_b32 v\d+, a(\d+)", t)
        if m and inasm:
            a = int(m.group(1))
            if a in since_mfma:
                d_mfma.append(since_mfma[a])
            if a in since_write:
                d_write.append(since_write[a])
    return d_mfma, d_write


@pytest.mark.parametrize("name", KERNELS, ids=["gemm1", "gemm2"])
def test_accumulator_reads_are_hazard_free(asm, name):
    lines = _body(asm, name)
    n_inline = sum(1 for i, l in enumerate(lines) if "v_accvgpr_read" in l and i and ";;#ASMSTART" in lines[i - 1])
    assert n_inline > 0
    d_mfma, d_write = _scan(lines)
    assert not d_mfma or min(d_mfma) >= MIN_MFMA_TO_READ, min(d_mfma)
    # compiler AGPR writes are the accumulator zeroing of the next tile, far
    # from any read; a copy right before a read means accumulators went
    # through VGPRs
    assert not d_write or min(d_write) >= 64, min(d_write)
    compiler_reads = 0
    inasm = False
    for l in lines:
        t = l.strip()
        if t.startswith(";;#ASMSTART"):
            inasm = True
        elif t.startswith(";;#ASMEND"):
            inasm = False
        elif t.startswith("v_accvgpr_read") and not inasm:
            compiler_reads += 1
    assert compiler_reads == 0, compiler_reads
