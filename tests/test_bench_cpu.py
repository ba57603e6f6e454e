"""CPU: bench.py's host-side logic (no device).

* more than one GPU is refused before anything touches a device;
* the roofline arithmetic: flops and bytes of a step against the counts
  written out by hand from each workload's sizes;
* the counter-derived HBM traffic is reported only for the kernel source it
  was measured on.
"""
import hashlib
import json
import os
import subprocess
import sys

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from combine_afd_slot_amd.inputs import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


# Gate/up: 2 products of H x I per routed pair (gate and up, 2 flops per
# multiply-add) and of H x Is per token; down: half of that.
@pytest.mark.parametrize("name,gflop", [
    ("prefill", 566.94),  # 6*2048*(1408*4096*6 + 2816*4096) / 1e9
    ("fanin4", 1964.897),  # same sizes, 14196 tokens
    ("skew", 6494.0),     # 6*7168*(2048*8192*8 + 2048*8192) / 1e9
    ("decode", 17.7167),  # 6*2048*(1408*128*6 + 2816*128) / 1e9
])
def test_step_flops(name, gflop):
    wl = WORKLOADS[name]
    a = bench.algorithmic(wl, np.ones(wl.num_experts, dtype=np.int64))
    assert a["flops"] / 1e9 == pytest.approx(gflop, rel=2e-4)
    assert a["gemm_gate_up_swiglu"]["flops"] == pytest.approx(2 * a["gemm_down"]["flops"], rel=1e-12)


def test_decode_step_bytes():
    """Decode streams every expert's weights once: 64 experts x 3 x 1408 x
    2048 bf16 values, the shared expert's 3 x 2816 x 2048, plus the token
    rows in and out (128 x 2048 bf16 each way) and the logits (128 x 64
    fp32)."""
    wl = WORKLOADS["decode"]
    a = bench.algorithmic(wl, np.ones(wl.num_experts, dtype=np.int64))
    expect = 64 * 3 * 1408 * 2048 * 2 + 3 * 2816 * 2048 * 2 + 2 * 128 * 2048 * 2 + 128 * 64 * 4
    assert a["bytes"] == expect
    assert abs(a["bytes"] / 1e9 - 1.143) < 1e-3
    # experts with no rows are not streamed
    c = np.ones(wl.num_experts, dtype=np.int64)
    c[:4] = 0
    b = bench.algorithmic(wl, c)
    assert a["bytes"] - b["bytes"] == 4 * 3 * 1408 * 2048 * 2


def test_traffic_only_for_the_measured_source(tmp_path, monkeypatch):
    src_dir = tmp_path / "combine_afd_slot_amd" / "csrc"
    src_dir.mkdir(parents=True)
    (tmp_path / "profiles").mkdir()
    src = src_dir / "afd_kernels.hip"
    src.write_bytes(b"// kernels\n")
    sha = hashlib.sha256(src.read_bytes()).hexdigest()
    wl = WORKLOADS["decode"]
    side = {"workload": "decode", "kernel_source_sha256": sha,
            "bytes_per_launch": {"gemm_gate_up_swiglu": {"read": 768e6, "written": 3e6}}}
    (tmp_path / "profiles" / "hbm_bytes_decode.json").write_text(json.dumps(side))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.measured_traffic(wl, "gemm_gate_up_swiglu") == 771000000
    assert bench.measured_traffic(wl, "gemm_down") is None
    src.write_bytes(b"// kernels, changed\n")
    assert bench.measured_traffic(wl, "gemm_gate_up_swiglu") is None
    assert bench.measured_traffic(WORKLOADS["prefill"], "gemm_gate_up_swiglu") is None  # no summary
