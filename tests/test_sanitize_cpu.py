"""CPU: host AddressSanitizer / UndefinedBehaviorSanitizer builds.

The CPU oracle (oracle/afd_oracle.c) and the library's host-only protocol
code (afd_host.cpp: layout, configuration checks, header codec, argument
refusals; afd_proto.h: field sizes, inbound checks) are rebuilt with
-fsanitize=address,undefined on the host side and run through drivers in
tests/sanitize/ that reach every entry point on small and degenerate inputs.
No GPU is touched (the kernel launches are stubbed out in the library
build).  A sanitizer report or a failed check fails the test.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SAN = os.path.join(HERE, "sanitize")
ENV = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:halt_on_error=1",
           UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1", OMP_NUM_THREADS="2")


def _run(exe):
    r = subprocess.run([str(exe)], env=ENV, capture_output=True, text=True, timeout=300)
    text = r.stdout + r.stderr
    assert "AddressSanitizer" not in text and "runtime error:" not in text, text[-4000:]
    assert r.returncode == 0, text[-4000:]
    return text


def test_oracle_under_sanitizers(tmp_path):
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc not found")
    exe = tmp_path / "oracle_san"
    subprocess.run([gcc, "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=undefined", "-fopenmp", "-ffp-contract=off", "-std=c11",
                    os.path.join(ROOT, "oracle", "afd_oracle.c"), os.path.join(SAN, "oracle_driver.c"),
                    "-o", str(exe), "-lm"], check=True, capture_output=True, text=True)
    assert "0 failure(s)" in _run(exe)


def test_host_protocol_code_under_sanitizers(tmp_path):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not found")
    exe = tmp_path / "host_san"
    # host-side sanitizers only: each -fsanitize= follows -Xarch_host
    cmd = [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", f"-I{os.path.join(ROOT, 'include')}",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=undefined", "-x", "hip",
           os.path.join(ROOT, "combine_afd_slot_amd", "csrc", "afd_host.cpp"),
           os.path.join(SAN, "launch_stubs.cpp"), os.path.join(SAN, "host_driver.cpp"), "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "0 failure(s)" in _run(exe)
