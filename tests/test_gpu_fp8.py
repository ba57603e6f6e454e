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


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "prefill"])
def test_fp8_full_size_every_row(orc, name):
    """The fp8 W1 path on the full-size decode and prefill workloads: every
    output row against the oracle's fp8 path."""
    import dataclasses
    from combine_afd_slot_amd.inputs import WORKLOADS
    wl = dataclasses.replace(WORKLOADS[name], w1_fp8=1)
    say(f"[fp8-full] {name}: generating inputs")
    inp = make_inputs(wl)
    with FfnSession(wl, inp) as s:
        say(f"[fp8-full] {name}: GPU run")
        s.step()
        st = s.status()
        assert st.status == 0 and st.total_tokens == wl.total_tokens
        out = [o.copy() for o in s.outputs_f32()]
    say(f"[fp8-full] {name}: oracle fp8 path on all {wl.total_tokens} tokens")
    ref = orc.ffn_fp8(inp["x"], inp["l"], inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"), K=wl.top_k,
                      rsf=wl.routed_scaling_factor, renorm=wl.renormalize)
    errs = [row_rel_err(o, ref[p]) for p, o in enumerate(out)]
    say(f"[fp8-full] {name}: max row rel err {max(errs):.3e} over all {wl.total_tokens} rows")
    assert max(errs) <= ROW_REL_TOL


@pytest.mark.parametrize("F,shared_rank", [(2, 1), (4, 0)])
def test_fp8_expert_segments_same_bits(F, shared_rank):
    """fp8 W1 on attention-routed windows split into F expert segments: each
    rank's FFN side quantises only the rows of its experts (its row count
    comes from its group lists), and the sender's combine over the ranks
    gives the FFN-routed fp8 run's outputs bit for bit."""
    import dataclasses
    from combine_afd_slot_amd import afd
    wl = WLS[2]  # 40 experts, top-6, ragged lengths, Zipf bias
    E, H = wl.num_experts, wl.hidden
    El = E // F
    inp = make_inputs(wl)
    with FfnSession(wl, inp, poll_timeout_us=200_000) as s:
        s.step()
        assert s.status().status == 0
        base = [o.copy() for o in s.outputs_f32()]
    sess = []
    try:
        for r in range(F):
            rwl = dataclasses.replace(wl, attention_routes=1, num_experts=El, route_experts=E, expert_offset=r * El,
                                      shared_intermediate=wl.shared_intermediate if r == shared_rank else 0)
            rinp = dict(inp, W13=inp["W13"][r * El:(r + 1) * El], W2=inp["W2"][r * El:(r + 1) * El])
            if r != shared_rank:
                rinp["Ws13"] = rinp["Ws2"] = None
            sess.append(FfnSession(rwl, rinp, poll_timeout_us=200_000))
        for x in sess:
            x.pack_all()
        for x in sess:
            x.run()
            x.ffn_stream.synchronize()
            assert x.status().status == 0
        torch = sess[0].torch
        out = [torch.empty((n, H), dtype=torch.bfloat16, device=sess[0].dev) for n in wl.seq_lens]
        wins = [x.win for x in sess]
        for p, n in enumerate(wl.seq_lens):
            afd.afd_slot_unpack_ranks(wins, p, 0, n, out[p].data_ptr() if n else 0,
                                      sess[0].peer_streams[p].cuda_stream)
        for ps in sess[0].peer_streams:
            ps.synchronize()
        for p, o in enumerate(out):
            for x in sess:
                assert x.peer_status(p).status == 0
            np.testing.assert_array_equal(o.float().cpu().numpy(), base[p])
    finally:
        for x in sess:
            x.close()


@pytest.mark.timeout(900)
def test_fp8_skew_sampled_rows(orc):
    """The fp8 W1 path on the full-size skew workload (2 x 4096 tokens, H
    7168, 256 experts, top-8, Zipf bias): every 16th row of each peer, its
    last row and every row whose token chose a light expert (1-15 rows),
    against the oracle's fp8 path over those tokens alone (a token's output
    row depends on that token only; its token-row scale too)."""
    import dataclasses
    from combine_afd_slot_amd.inputs import WORKLOADS
    wl = dataclasses.replace(WORKLOADS["skew"], w1_fp8=1)
    say("[fp8-skew] generating inputs")
    inp = make_inputs(wl)
    with FfnSession(wl, inp) as s:
        say("[fp8-skew] GPU run")
        s.step()
        st = s.status()
        assert st.status == 0 and st.total_tokens == wl.total_tokens
        out = [o.copy() for o in s.outputs_f32()]
        r = s.routing()
    counts, ids, off = r["counts"], r["ids"], r["off"]
    light = np.flatnonzero((counts >= 1) & (counts <= 15))
    chose_light = np.isin(ids, light).any(axis=1)
    assert light.size > 0 and chose_light.any()
    errs = []
    for p, n in enumerate(wl.seq_lens):
        rows = np.zeros(n, dtype=bool)
        rows[::16] = True
        rows[n - 1] = True
        rows |= chose_light[off[p]:off[p] + n]
        idx = np.flatnonzero(rows)
        say(f"[fp8-skew] peer {p}: oracle fp8 path on {idx.size} of {n} rows")
        ref = orc.ffn_fp8([inp["x"][p][idx]], [inp["l"][p][idx]], inp["W13"], inp["W2"], inp.get("Ws13"),
                          inp.get("Ws2"), K=wl.top_k, rsf=wl.routed_scaling_factor, renorm=wl.renormalize)
        errs.append(row_rel_err(out[p][idx], ref[0]))
    say(f"[fp8-skew] {int(light.size)} light experts; max row rel err {max(errs):.3e}")
    assert max(errs) <= ROW_REL_TOL
