"""GPU parity: the HIP path through the C ABI against the CPU oracle.

Routing ids, per-expert counts and offsets, the dispatch permutation and its
inverse, and the split offsets must match bit for bit; outputs within 2e-2
per-row relative error.  Every output row is compared, on the small
workloads and on the four full-size ones (the skew workload one peer at a
time); the full-size inputs also go through an attention-routed window,
whose outputs must be the same bits.
"""
import dataclasses

import numpy as np
import pytest

from combine_afd_slot_amd.driver import FfnSession
from combine_afd_slot_amd.inputs import WORKLOADS, make_inputs, small_workload
from gpu_util import ROW_REL_TOL, check_routing, row_rel_err, say

pytestmark = pytest.mark.gpu


def _run_and_check_full(orc, wl):
    say(f"[parity] {wl.name} seq_lens={wl.seq_lens} H={wl.hidden} E={wl.num_experts} K={wl.top_k} "
        f"I={wl.intermediate} Is={wl.shared_intermediate}")
    inp = make_inputs(wl)
    ref = orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"),
                  K=wl.top_k, rsf=wl.routed_scaling_factor, renorm=wl.renormalize)
    with FfnSession(wl, inp) as s:
        s.step()
        st = s.status()
        assert st.status == 0, st.status
        assert st.total_tokens == wl.total_tokens
        check_routing(s.routing(), ref, wl)
        outs = s.outputs_f32()
        for p in range(wl.num_peers):
            assert s.peer_status(p).status == 0
            err = row_rel_err(outs[p], ref["out_p"][p])
            assert err <= ROW_REL_TOL, (p, err)
    return ref


def test_tiny(orc):
    _run_and_check_full(orc, WORKLOADS["tiny"])


SMALL = [
    # empty peer, widths that are not multiples of the 64-wide tile halves
    small_workload(),
    # several row tiles per expert, ragged tails everywhere
    small_workload("multi_tile", seq_lens=(300, 173), hidden=192, num_experts=6, top_k=2,
                   intermediate=136, shared_intermediate=264, token_cap=300),
    # no shared expert, K = E, routed scaling factor
    small_workload("k_eq_e", seq_lens=(33, 1), hidden=64, num_experts=5, top_k=5, intermediate=48,
                   shared_intermediate=0, token_cap=40, routed_scaling_factor=2.5),
    # top-1, many experts (two logits per lane), no renormalisation
    small_workload("top1_e100", seq_lens=(50, 70, 9), hidden=128, num_experts=100, top_k=1,
                   intermediate=64, shared_intermediate=64, token_cap=80, renormalize=0),
    # many peers, E=256 (four logits per lane), K=8
    small_workload("e256", seq_lens=(5, 17, 0, 29, 3, 64, 1, 40), hidden=256, num_experts=256, top_k=8,
                   intermediate=128, shared_intermediate=128, token_cap=64),
    # depth tails in both GEMMs (hidden, intermediate and the shared width not
    # multiples of the 32-deep step; the shared width below one step)
    small_workload("depth_tails", seq_lens=(45, 20), hidden=72, num_experts=7, top_k=3, intermediate=40,
                   shared_intermediate=24, token_cap=48),
]


@pytest.mark.parametrize("wl", SMALL, ids=[w.name for w in SMALL])
def test_small_workloads(orc, wl):
    _run_and_check_full(orc, wl)


def test_ties_and_negative_zero(orc):
    wl = small_workload("ties", seq_lens=(40, 24), hidden=64, num_experts=16, top_k=4, intermediate=64,
                        shared_intermediate=0, token_cap=64)
    inp = make_inputs(wl)
    L = inp["L"]
    L[::2] = np.round(L[::2])          # many exact ties
    L[1::4] = 0.5                       # all-equal rows
    L[3::8, 3] = -0.0
    L[3::8, 5] = 0.0
    off = np.concatenate([[0], np.cumsum(wl.seq_lens)])
    inp["l"] = [L[off[p]:off[p + 1]] for p in range(wl.num_peers)]
    ref = orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], K=wl.top_k)
    with FfnSession(wl, inp) as s:
        s.step()
        assert s.status().status == 0
        check_routing(s.routing(), ref, wl)


def _gpu_full_size(wl, inp, name):
    """One FFN-routed run and one attention-routed run of the same inputs;
    returns (routing artefacts, FFN-routed outputs per peer as float32).
    The attention-routed outputs must be the same bits."""
    with FfnSession(wl, inp) as s, FfnSession(dataclasses.replace(wl, attention_routes=1), inp) as sa:
        say(f"[parity-full] {name}: GPU run")
        s.step()
        st = s.status()
        assert st.status == 0 and st.total_tokens == wl.total_tokens, st.status
        for p in range(wl.num_peers):
            assert s.peer_status(p).status == 0
        routing = s.routing()
        out = [o.copy() for o in s.outputs_f32()]
        say(f"[parity-full] {name}: attention-routed run")
        sa.step()
        assert sa.status().status == 0
        for p, o in enumerate(sa.outputs_f32()):
            np.testing.assert_array_equal(o, out[p])
    return routing, out


def _oracle_routing(orc, wl, inp):
    ids, w = orc.route(inp["L"], wl.top_k, wl.renormalize)
    counts, eoff, perm, inv = orc.dispatch(ids, wl.num_experts)
    return {"ids": ids, "w": w, "counts": counts, "expert_offsets": eoff, "perm": perm, "inv": inv}


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["decode", "prefill", "fanin4"])
def test_full_size_every_row(orc, name):
    """Full-size workloads, in the launch configuration the benchmark times:
    routing artefacts bit-exact on every token, and every output row of every
    peer within the row tolerance of the whole oracle path."""
    wl = WORKLOADS[name]
    say(f"[parity-full] {name}: generating inputs")
    inp = make_inputs(wl)
    routing, out = _gpu_full_size(wl, inp, name)
    check_routing(routing, _oracle_routing(orc, wl, inp), wl)
    say(f"[parity-full] {name}: oracle on all {wl.total_tokens} tokens")
    ref = orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"), K=wl.top_k,
                  rsf=wl.routed_scaling_factor, renorm=wl.renormalize)
    errs = [row_rel_err(out[p], ref["out_p"][p]) for p in range(wl.num_peers)]
    say(f"[parity-full] {name}: max row rel err per peer {['%.3e' % e for e in errs]} "
        f"over all {wl.total_tokens} rows")
    assert max(errs) <= ROW_REL_TOL


@pytest.fixture(scope="module")
def skew_run(orc):
    """The skew workload (2 x 4096 tokens, H 7168, 256 experts, top-8, Zipf
    bias) run once on the GPU for the per-peer oracle checks below."""
    wl = WORKLOADS["skew"]
    say("[parity-full] skew: generating inputs")
    inp = make_inputs(wl)
    routing, out = _gpu_full_size(wl, inp, "skew")
    check_routing(routing, _oracle_routing(orc, wl, inp), wl)
    c = routing["counts"]
    say(f"[parity-full] skew: expert rows max {c.max()} (expert {int(c.argmax())}), "
        f"{int((c == 0).sum())} experts empty, {int(((c > 0) & (c < 16)).sum())} with 1-15 rows")
    yield wl, inp, out
    out.clear()
    inp.clear()


@pytest.mark.timeout(900)
@pytest.mark.parametrize("peer", [0, 1])
def test_full_size_skew_every_row(orc, skew_run, peer):
    """Every output row of one skew peer against the oracle run over that
    peer's tokens alone (each token's row depends on that token only)."""
    wl, inp, out = skew_run
    say(f"[parity-full] skew: oracle on peer {peer}'s {wl.seq_lens[peer]} tokens")
    ref = orc.ffn([inp["x"][peer]], [inp["l"][peer]], inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"),
                  K=wl.top_k, rsf=wl.routed_scaling_factor, renorm=wl.renormalize)
    err = row_rel_err(out[peer], ref["out"])
    say(f"[parity-full] skew: peer {peer} max row rel err {err:.3e} over all {wl.seq_lens[peer]} rows")
    assert err <= ROW_REL_TOL
