"""The oracle reproduces its stored tiny-workload values (regression pin).

tests/golden/tiny_oracle.json is written by tests/golden/make_golden.py,
which calls only oracle/ and the input generator.
"""
import json
import os

import numpy as np

from combine_afd_slot_amd.inputs import WORKLOADS, make_inputs

GOLD = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "tiny_oracle.json")


def test_tiny_golden(orc):
    d = json.load(open(GOLD))
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    r = orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], inp["Ws13"], inp["Ws2"], K=wl.top_k)
    assert r["off"].tolist() == d["split_offsets"]
    assert r["counts"].tolist() == d["expert_counts"]
    assert r["expert_offsets"].tolist() == d["expert_offsets"]
    assert r["ids"].tolist() == d["ids"]
    assert r["perm"].tolist() == d["perm"]
    np.testing.assert_allclose(r["w"], np.array(d["w"]), rtol=1e-15)
    np.testing.assert_allclose(r["out"][[0, 19], :4], np.array(d["out_rows_0_19_first4"]), rtol=1e-12)
    np.testing.assert_allclose(r["out"].sum(), d["out_sum"], rtol=1e-12)
    np.testing.assert_allclose(np.abs(r["out"]).sum(), d["out_abs_sum"], rtol=1e-12)
