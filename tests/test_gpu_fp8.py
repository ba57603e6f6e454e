"""GPU: the fp8 W1 path (w1_fp8 = 1).

"[RFC]: Async AFD for Prefill on Ascend NPU", "Architecture": the routed W1
+ SwiGLU grouped GEMM, quantised.  Token rows and W13 / Ws13 rows are
quantised to OCP FP8 E4M3 with one scale per row; the gate/up GEMMs run on
the codes (block-scaled MFMA, unit block scales) with both row scales
applied before SwiGLU; the down GEMM stays bf16.  Every output row is
checked against the oracle's fp8 path (oracle.ffn_fp8, pinned on the CPU)
within the row tolerance, and must differ from the bf16 path's.
"""
import numpy as np
import pytest

from combine_afd_slot_amd.driver import FfnSession
from combine_afd_slot_amd.inputs import make_inputs, small_workload
from gpu_util import ROW_REL_TOL, row_rel_err, say

pytestmark = pytest.mark.gpu

WLS = [
    small_workload("fp8_shared", seq_lens=(37, 0, 70), hidden=128, num_experts=12, top_k=3, intermediate=96,
                   shared_intermediate=64, token_cap=72, w1_fp8=1),
    small_workload("fp8_routed_only", seq_lens=(19, 33), hidden=64, num_experts=8, top_k=2, intermediate=48,
                   shared_intermediate=0, token_cap=40, w1_fp8=1),
    small_workload("fp8_ragged", seq_lens=(150, 61), hidden=256, num_experts=40, top_k=6, intermediate=200,
                   shared_intermediate=136, token_cap=160, zipf_bias=1.0, w1_fp8=1),
    small_workload("fp8_wide", seq_lens=(64, 64), hidden=1024, num_experts=8, top_k=2, intermediate=256,
                   shared_intermediate=256, token_cap=64, w1_fp8=1),
    # rows longer than the 4096 values the quantising wavefront keeps in registers
    small_workload("fp8_long_rows", seq_lens=(9, 14), hidden=4608, num_experts=4, top_k=2, intermediate=64,
                   shared_intermediate=64, token_cap=16, w1_fp8=1),
]


@pytest.mark.parametrize("wl", WLS, ids=lambda w: w.name)
def test_fp8_against_oracle(orc, wl):
    inp = make_inputs(wl)
    ref = orc.ffn_fp8(inp["x"], inp["l"], inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"), K=wl.top_k,
                      rsf=wl.routed_scaling_factor, renorm=wl.renormalize)
    with FfnSession(wl, inp, poll_timeout_us=200_000) as s:
        s.step()
        assert s.status().status == 0
        out = [o.copy() for o in s.outputs_f32()]
    errs = [row_rel_err(o, ref[p]) for p, o in enumerate(out)]
    say(f"[fp8] {wl.name}: max row rel err {max(errs):.3e}")
    assert max(errs) <= ROW_REL_TOL
    import dataclasses
    with FfnSession(dataclasses.replace(wl, w1_fp8=0), inp, poll_timeout_us=200_000) as s:
        s.step()
        bf = s.outputs_f32()
    assert any(o.size and not np.array_equal(o, bf[p]) for p, o in enumerate(out))


@pytest.mark.parametrize("wl", WLS[:3], ids=lambda w: w.name)
def test_fp8_attention_routed_same_bits(wl):
    """An attention-routed window quantises each arriving row on the FFN side;
    pair rows are copies of their token's row, so every GEMM row gets the
    codes and scale of the FFN-routed path and the outputs are the same bits."""
    import dataclasses
    inp = make_inputs(wl)
    with FfnSession(wl, inp, poll_timeout_us=200_000) as s:
        s.step()
        assert s.status().status == 0
        base = [o.copy() for o in s.outputs_f32()]
    with FfnSession(dataclasses.replace(wl, attention_routes=1), inp, poll_timeout_us=200_000) as s:
        s.step()
        assert s.status().status == 0
        for p, o in enumerate(s.outputs_f32()):
            np.testing.assert_array_equal(o, base[p])
