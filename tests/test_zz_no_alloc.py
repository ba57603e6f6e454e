"""GPU: the allocation-free window (afd_window_create_static).

The window of afd_window_create_static lives in the library's static device
array instead of a hipMalloc'd buffer; every other entry point runs the same
kernels on it.  Two static windows in a row, the second smaller (it reuses
the array the first left behind), must give the outputs of windows from
afd_window_create bit for bit, routing bit-exact against the oracle and every
row within the oracle's row tolerance.
"""
import numpy as np
import pytest

from combine_afd_slot_amd import afd
from combine_afd_slot_amd.driver import FfnSession
from combine_afd_slot_amd.inputs import WORKLOADS, make_inputs, small_workload
from gpu_util import ROW_REL_TOL, check_routing, row_rel_err, say

pytestmark = pytest.mark.gpu

# the decode-shaped workload (8 peers x 16 tokens, H 2048, 64 experts), then
# a smaller one with an empty peer and ragged tiles
WLS = [WORKLOADS["decode"],
       small_workload("static_small", seq_lens=(37, 0, 90), hidden=256, num_experts=12, top_k=3, intermediate=200,
                      shared_intermediate=136, token_cap=96)]


def _run(wl, inp, static):
    with FfnSession(wl, inp, static_window=static) as s:
        lay = s.layout
        s.step()
        st = s.status()
        assert st.status == 0, afd.status_string(st.status)
        for p in range(wl.num_peers):
            assert s.peer_status(p).status == 0
        return lay, s.routing(), [o.copy() for o in s.outputs_f32()]


def test_static_window_matches_allocated_window(orc):
    inps = [make_inputs(wl) for wl in WLS]
    refs = []
    for wl, inp in zip(WLS, inps):
        lay, r, out = _run(wl, inp, static=False)
        assert lay.total_bytes <= afd.AFD_STATIC_WINDOW_BYTES
        refs.append((r, out))
    for i, (wl, inp) in enumerate(zip(WLS, inps)):
        say(f"[no-alloc] static window {i}: {wl.name} ({wl.total_tokens} tokens)")
        _, r, out = _run(wl, inp, static=True)
        orc_ref = orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"),
                          K=wl.top_k, rsf=wl.routed_scaling_factor, renorm=wl.renormalize)
        check_routing(r, orc_ref, wl)
        for p in range(wl.num_peers):
            np.testing.assert_array_equal(out[p], refs[i][1][p])
            assert row_rel_err(out[p], orc_ref["out_p"][p]) <= ROW_REL_TOL, (i, p)


def test_one_static_window_per_device():
    wl = WLS[1]
    cfg = afd.make_config(wl.num_peers, wl.token_cap, wl.hidden, wl.num_experts, wl.top_k, wl.intermediate,
                          wl.shared_intermediate)
    w = afd.afd_window_create_static(cfg)
    try:
        with pytest.raises(afd.AfdError) as ei:
            afd.afd_window_create_static(cfg)
        assert ei.value.code == afd.AFD_ERR_INVALID
        with pytest.raises(afd.AfdError) as ei:
            afd.afd_profile_enable(w, 1)
        assert ei.value.code == afd.AFD_ERR_INVALID
    finally:
        afd.afd_window_destroy(w)
    # released: a new one opens
    afd.afd_window_destroy(afd.afd_window_create_static(cfg))
