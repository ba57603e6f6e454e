"""GPU: any-ready runs (afd_ffn_run_ready).

"[RFC]: Async AFD for Prefill on Ascend NPU", "Asynchronous work-item
contract" (the FFN side may take any ready replica without waiting for the
others, and must not starve one) and "[RFC]: Async GPU Connector", "Risks and
alternatives" (a device-side wait on the flag array with a rotating scan
start).  Every token's output row depends on that token alone, so the rows a
peer gets back from a run over a subset of the peers must equal, bit for bit,
the rows of a run over all of them; they are also checked against the oracle.
"""
import numpy as np
import pytest

from combine_afd_slot_amd import afd
from combine_afd_slot_amd.driver import FfnSession
from combine_afd_slot_amd.inputs import make_inputs, small_workload
from gpu_util import ROW_REL_TOL, row_rel_err, say

pytestmark = pytest.mark.gpu

WL = small_workload("any_ready", seq_lens=(21, 13, 34), hidden=128, num_experts=8, top_k=2, intermediate=64,
                    shared_intermediate=64, token_cap=40)


def _full_run(s):
    s.step(layer=0)
    assert s.status().status == 0
    return [o.copy() for o in s.outputs_f32()]


def _sync_peers(s, peers):
    for p in peers:
        s.peer_streams[p].synchronize()


def _run_ready(s, max_peers, gather_us=0):
    afd.afd_ffn_run_ready(s.win, 0, 0, s.packed.data_ptr(), max_peers, gather_us, s.ffn_stream.cuda_stream)
    return s.status()


def _check_peer(s, orc_out, full, p):
    o = s.outputs_f32()[p]
    np.testing.assert_array_equal(o, full[p])
    assert row_rel_err(o, orc_out[p]) <= ROW_REL_TOL


def test_serves_the_ready_subset(orc):
    inp = make_inputs(WL)
    ref = orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], inp["Ws13"], inp["Ws2"], K=WL.top_k)["out_p"]
    with FfnSession(WL, inp, poll_timeout_us=200_000) as s:
        full = _full_run(s)
        # peers 0 and 2 publish; peer 1 has not yet
        s.pack(0)
        s.pack(2)
        _sync_peers(s, (0, 2))
        st = _run_ready(s, max_peers=3)
        say(f"[any-ready] served {st.served_mask:#x} T={st.total_tokens}")
        assert st.status == 0 and st.served_mask == 0b101
        assert st.total_tokens == WL.seq_lens[0] + WL.seq_lens[2]
        # peer 1 was not answered; 0 and 2 were
        assert afd.afd_window_poll(s.win, 1, 3) == [2, 1, 2]
        for p in (0, 2):
            s.unpack(p)
        _sync_peers(s, (0, 2))
        for p in (0, 2):
            assert s.peer_status(p).status == 0
            _check_peer(s, ref, full, p)
        # peer 1 publishes later and is served alone
        s.pack(1)
        _sync_peers(s, (1,))
        st = _run_ready(s, max_peers=3)
        assert st.status == 0 and st.served_mask == 0b010 and st.total_tokens == WL.seq_lens[1]
        s.unpack(1)
        _sync_peers(s, (1,))
        assert s.peer_status(1).status == 0
        _check_peer(s, ref, full, 1)


def test_round_robin_with_one_peer_per_run(orc):
    inp = make_inputs(WL)
    ref = orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], inp["Ws13"], inp["Ws2"], K=WL.top_k)["out_p"]
    with FfnSession(WL, inp, poll_timeout_us=200_000) as s:
        full = _full_run(s)
        order = []
        for rnd in range(2):
            s.pack_all()
            for _ in range(3):
                st = _run_ready(s, max_peers=1)
                assert st.status == 0 and bin(st.served_mask).count("1") == 1
                p = st.served_mask.bit_length() - 1
                order.append(p)
                s.unpack(p)
                _sync_peers(s, (p,))
                assert s.peer_status(p).status == 0
                _check_peer(s, ref, full, p)
        say(f"[any-ready] service order {order}")
        # every peer once per round, in rotating order
        assert sorted(order[:3]) == [0, 1, 2] and sorted(order[3:]) == [0, 1, 2]
        assert all((order[i + 1] - order[i]) % 3 == 1 for i in range(len(order) - 1))


def test_nothing_ready_times_out_then_recovers(orc):
    inp = make_inputs(WL)
    with FfnSession(WL, inp, poll_timeout_us=20_000) as s:
        full = _full_run(s)
        st = _run_ready(s, max_peers=3)
        assert st.status == afd.AFD_ERR_TIMEOUT and st.served_mask == 0 and st.failed_peer == -1
        s.pack_all()
        st = _run_ready(s, max_peers=3, gather_us=1000)
        assert st.status == 0 and st.served_mask == 0b111
        s.unpack_all()
        for p, o in enumerate(s.outputs_f32()):
            np.testing.assert_array_equal(o, full[p])


def test_max_peers_caps_the_work_item(orc):
    inp = make_inputs(WL)
    with FfnSession(WL, inp, poll_timeout_us=200_000) as s:
        full = _full_run(s)
        s.pack_all()
        st = _run_ready(s, max_peers=2)
        assert st.status == 0 and bin(st.served_mask).count("1") == 2
        first = [p for p in range(3) if st.served_mask >> p & 1]
        st2 = _run_ready(s, max_peers=2)
        rest = [p for p in range(3) if st2.served_mask >> p & 1]
        assert st2.status == 0 and sorted(first + rest) == [0, 1, 2]
        s.unpack_all()
        for p, o in enumerate(s.outputs_f32()):
            np.testing.assert_array_equal(o, full[p])


def test_layer_table_any_ready(orc):
    inp = make_inputs(WL)
    with FfnSession(WL, inp, poll_timeout_us=200_000) as s:
        full = _full_run(s)
        afd.afd_layer_table_set(s.win, [s.packed.data_ptr()], s.ffn_stream.cuda_stream)
        s.pack(1, 0, 0)
        _sync_peers(s, (1,))
        afd.afd_ffn_run_ready(s.win, 0, -1, 0, 3, 0, s.ffn_stream.cuda_stream)
        st = s.status()
        assert st.status == 0 and st.served_mask == 0b010
        s.unpack(1)
        _sync_peers(s, (1,))
        np.testing.assert_array_equal(s.outputs_f32()[1], full[1])


def test_run_ready_argument_errors():
    inp = make_inputs(WL)
    with FfnSession(WL, inp, poll_timeout_us=20_000) as s:
        st_ = s.ffn_stream.cuda_stream
        pw = s.packed.data_ptr()
        for args in ((0, 0, pw, 0, 0), (0, 0, pw, 4, 0), (0, 0, pw, 2, -1), (0, 0, pw, 2, 20_001),
                     (1, 0, pw, 2, 0), (0, 0, 0, 2, 0), (0, 0, pw + 16, 2, 0), (0, -1, 0, 2, 0)):
            with pytest.raises(afd.AfdError) as ei:
                afd.afd_ffn_run_ready(s.win, *args, st_)
            assert ei.value.code == afd.AFD_ERR_INVALID, args
