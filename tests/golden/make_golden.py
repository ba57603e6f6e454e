"""Write the stored oracle values for the tiny workload.

Calls only the CPU oracle (oracle/) and the seeded input generator; no value
here comes from the HIP library.  Run from the repository root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from combine_afd_slot_amd.inputs import WORKLOADS, make_inputs  # noqa: E402
from oracle import oracle  # noqa: E402


def main():
    wl = WORKLOADS["tiny"]
    inp = make_inputs(wl)
    r = oracle.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], inp["Ws13"], inp["Ws2"], K=wl.top_k)
    doc = {
        "source": "CPU oracle (oracle/afd_oracle.c) on the tiny workload, generator recipe 'stream', seed 0",
        "seq_lens": list(wl.seq_lens),
        "split_offsets": r["off"].tolist(),
        "expert_counts": r["counts"].tolist(),
        "expert_offsets": r["expert_offsets"].tolist(),
        "ids": r["ids"].tolist(),
        "w": [[float(v) for v in row] for row in r["w"]],
        "perm": r["perm"].tolist(),
        "out_rows_0_19_first4": [[float(v) for v in r["out"][t, :4]] for t in (0, 19)],
        "out_sum": float(r["out"].sum()),
        "out_abs_sum": float(abs(r["out"]).sum()),
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_oracle.json")
    with open(path, "w") as f:
        json.dump(doc, f, indent=1)
    print("wrote", path)


if __name__ == "__main__":
    main()
