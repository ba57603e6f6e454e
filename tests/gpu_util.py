"""Helpers shared by the GPU tests (not collected: no test_ prefix)."""
import sys

import numpy as np

# Output tolerance: per token row, max_h |gpu - ref| / max_h |ref| <= 2e-2
# (bf16 inputs and weights, fp32 accumulation, bf16 intermediates and output).
ROW_REL_TOL = 2e-2


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def row_rel_err(gpu, ref):
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    if gpu.size == 0:
        return 0.0
    den = np.abs(ref).max(axis=1)
    num = np.abs(gpu - ref).max(axis=1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max())


def check_routing(r, ref, wl):
    """Bit-exact ids / counts / offsets / perm / inv / split offsets; weights close."""
    T = wl.total_tokens
    assert r["off"].tolist() == [0] + np.cumsum(wl.seq_lens).tolist()
    np.testing.assert_array_equal(r["ids"], ref["ids"])
    np.testing.assert_array_equal(r["counts"], ref["counts"])
    np.testing.assert_array_equal(r["expert_offsets"], ref["expert_offsets"])
    np.testing.assert_array_equal(r["perm"], ref["perm"])
    np.testing.assert_array_equal(r["inv"], ref["inv"])
    assert r["ids"].shape == (T, wl.top_k)
    np.testing.assert_allclose(r["w"], ref["w"], rtol=2e-6, atol=1e-7)
