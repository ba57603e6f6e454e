"""Scenarios of tests/test_gpu_concurrent.py, run in a child process.

Each scenario enqueues an FFN-side call first and lets the peers publish
while its wait kernel spins on another stream.  That needs the FFN stream
and the peer streams on distinct hardware queues; a process that has
already used many streams may have two of them on one queue (the runtime
shares its few queues among all streams), so the scenarios run in a fresh
process with a few more queues (GPU_MAX_HW_QUEUES=8), one after the other.
Usage: python tests/concurrent_scenarios.py OUT.json -- writes, per
scenario, "ok" or the failure text.  Not collected by pytest.
"""
import json
import os
import sys
import traceback

sys.path.insert(0, os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import time

import numpy as np

from combine_afd_slot_amd import afd
from combine_afd_slot_amd.driver import FfnSession, _dev_bf16
from combine_afd_slot_amd.inputs import make_inputs, small_workload
from gpu_util import ROW_REL_TOL, row_rel_err, say

# two peers, several GEMM tiles per expert, so a run takes long enough for
# the pack of a later stage to overlap it
WL = small_workload("concurrent", seq_lens=(300, 500), hidden=1024, num_experts=16, top_k=4, intermediate=512,
                    shared_intermediate=512, token_cap=512, ring_depth=2)
TIMEOUT_US = 1_000_000
DELAY_S = 0.02


def _oracle(orc, inp, wl=WL):
    return orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], inp["Ws13"], inp["Ws2"], K=wl.top_k,
                   rsf=wl.routed_scaling_factor, renorm=wl.renormalize)["out_p"]


def _pending(s):
    """An event after everything enqueued on the FFN stream so far."""
    ev = s.torch.cuda.Event()
    ev.record(s.ffn_stream)
    return ev


def _assert_waiting(ev, what):
    time.sleep(DELAY_S)
    assert not ev.query(), f"{what} finished before any peer published"


def _sync_all(s):
    s.ffn_stream.synchronize()
    for ps in s.peer_streams:
        ps.synchronize()


def _check_outputs(s, ref, base, peers=(0, 1)):
    for p in peers:
        st = s.peer_status(p)
        assert st.status == 0, (p, afd.status_string(st.status))
        o = s.outputs_f32()[p]
        if base is not None:
            np.testing.assert_array_equal(o, base[p])
        err = row_rel_err(o, ref[p])
        assert err <= ROW_REL_TOL, (p, err)


def run_waits_then_peers_publish(orc, early):
    inp = make_inputs(WL)
    ref = _oracle(orc, inp)
    with FfnSession(WL, inp, poll_timeout_us=TIMEOUT_US) as s:
        s.step()
        assert s.status().status == 0
        base = [o.copy() for o in s.outputs_f32()]
        for p in early:
            s.pack(p)
            s.peer_streams[p].synchronize()
        s.run()
        ev = _pending(s)
        _assert_waiting(ev, "afd_ffn_run")
        say(f"[concurrent] FFN run waiting; peers {[p for p in (0, 1) if p not in early]} publish now")
        for p in (0, 1):
            if p not in early:
                s.pack(p)
            s.unpack(p)
        _sync_all(s)
        st = s.status()
        assert st.status == 0, afd.status_string(st.status)
        assert st.total_tokens == WL.total_tokens
        _check_outputs(s, ref, base)


def ready_run_gathers_a_peer_that_arrives_during_the_window(orc):
    """afd_ffn_run_ready: peer 0 is ready when the run starts, peer 1
    publishes inside the gather window; both are served in one run."""
    inp = make_inputs(WL)
    ref = _oracle(orc, inp)
    with FfnSession(WL, inp, poll_timeout_us=TIMEOUT_US) as s:
        s.step()
        base = [o.copy() for o in s.outputs_f32()]
        s.pack(0)
        s.peer_streams[0].synchronize()
        afd.afd_ffn_run_ready(s.win, 0, 0, s.packed.data_ptr(), 2, 800_000, s.ffn_stream.cuda_stream)
        ev = _pending(s)
        _assert_waiting(ev, "the any-ready run")
        s.pack(1)
        for p in (0, 1):
            s.unpack(p)
        _sync_all(s)
        st = s.status()
        say(f"[concurrent] any-ready served {st.served_mask:#x}")
        assert st.status == 0 and st.served_mask == 0b11 and st.total_tokens == WL.total_tokens
        _check_outputs(s, ref, base)


def ready_run_waits_for_the_first_peer(orc):
    """afd_ffn_run_ready with nothing ready: the run spins until peer 1
    publishes and serves it alone (no gather window); peer 0's later
    message is served by the next run, which is also enqueued first."""
    inp = make_inputs(WL)
    ref = _oracle(orc, inp)
    with FfnSession(WL, inp, poll_timeout_us=TIMEOUT_US) as s:
        s.step()
        base = [o.copy() for o in s.outputs_f32()]
        for p in (1, 0):
            afd.afd_ffn_run_ready(s.win, 0, 0, s.packed.data_ptr(), 2, 0, s.ffn_stream.cuda_stream)
            ev = _pending(s)
            _assert_waiting(ev, "the any-ready run")
            s.pack(p)
            s.unpack(p)
            _sync_all(s)
            st = s.status()
            assert st.status == 0 and st.served_mask == 1 << p, (p, st.status, st.served_mask)
            assert st.total_tokens == WL.seq_lens[p]
            _check_outputs(s, ref, base, peers=(p,))


def _dev_inputs(s, inp):
    torch = s.torch
    x = [_dev_bf16(torch, a, s.dev) for a in inp["x"]]
    lg = [torch.from_numpy(np.ascontiguousarray(a)).to(s.dev) for a in inp["l"]]
    out = [torch.empty((n, s.wl.hidden), dtype=torch.bfloat16, device=s.dev) for n in s.wl.seq_lens]
    return x, lg, out


def _pack(s, stage, layer, bufs, p):
    x, lg, _ = bufs
    afd.afd_slot_pack(s.win, p, stage, layer, s.wl.seq_lens[p], x[p].data_ptr(), lg[p].data_ptr(), 0,
                      s.peer_streams[p].cuda_stream)


def _unpack(s, stage, bufs, p):
    afd.afd_slot_unpack(s.win, p, stage, s.wl.seq_lens[p], bufs[2][p].data_ptr(), s.peer_streams[p].cuda_stream)


def ring_depth_two_next_stage_published_while_the_first_runs(orc):
    """Ring depth 2: stage 0's messages are in; runs on stages 0 and 1 are
    enqueued back to back; the peers pack stage 1 at once (while stage 0's
    run computes and stage 1's wait spins), then unpack both stages."""
    inps = [make_inputs(WL.with_(seed=40)), make_inputs(WL.with_(seed=41), with_weights=False)]
    for k in ("W13", "W2", "Ws13", "Ws2"):  # one layer: both stages use the first draw's weights
        inps[1][k] = inps[0][k]
    refs = [_oracle(orc, inp) for inp in inps]
    with FfnSession(WL, inps[0], poll_timeout_us=TIMEOUT_US) as s:
        s.step()
        assert s.status().status == 0
        bufs = [_dev_inputs(s, inp) for inp in inps]
        s.torch.cuda.synchronize(s.dev)
        for p in (0, 1):
            _pack(s, 0, 0, bufs[0], p)
        for ps in s.peer_streams:
            ps.synchronize()
        s.run(stage=0)
        s.run(stage=1)
        for p in (0, 1):
            _pack(s, 1, 0, bufs[1], p)
            _unpack(s, 0, bufs[0], p)
            _unpack(s, 1, bufs[1], p)
        _sync_all(s)
        for stage in (0, 1):
            st = s.status(stage)
            assert st.status == 0, (stage, afd.status_string(st.status))
            for p in (0, 1):
                assert s.peer_status(p, stage).status == 0
                o = bufs[stage][2][p].float().cpu().numpy()
                err = row_rel_err(o, refs[stage][p])
                assert err <= ROW_REL_TOL, (stage, p, err)


def serve_loop_with_peers_publishing_during_the_loop(orc):
    """afd_ffn_serve: four items (stages 0, 1, 0, 1) enqueued before any
    message exists; the peers then send item by item with host delays,
    reusing each stage once its reply is unpacked (the ring rule), and
    every item's rows are checked."""
    n_items = 4
    inps = [make_inputs(WL.with_(seed=60 + i), with_weights=False) for i in range(n_items)]
    base_inp = make_inputs(WL)
    for inp in inps:
        for k in ("W13", "W2", "Ws13", "Ws2"):
            inp[k] = base_inp[k]
    with FfnSession(WL, base_inp, poll_timeout_us=TIMEOUT_US) as s:
        st_ = s.ffn_stream.cuda_stream
        afd.afd_layer_table_set(s.win, [s.packed.data_ptr()], st_)
        bufs = [_dev_inputs(s, inp) for inp in inps]
        s.torch.cuda.synchronize(s.dev)
        afd.afd_ffn_serve(s.win, 0, n_items, 0, 0, st_)
        ev = _pending(s)
        _assert_waiting(ev, "the serve loop")
        for i in range(n_items):
            stage = i % 2
            for p in (0, 1):
                _pack(s, stage, 0, bufs[i], p)
                _unpack(s, stage, bufs[i], p)
            time.sleep(DELAY_S / 4)
        assert afd.afd_ffn_serve_result(s.win, st_) == (afd.AFD_OK, n_items, -1)
        for stage in (0, 1):  # the words hold each stage's last unpack (items 2 and 3)
            for p in (0, 1):
                assert s.peer_status(p, stage).status == 0, (stage, p)
        for i in range(n_items):
            ref = _oracle(orc, inps[i])
            for p in (0, 1):
                o = bufs[i][2][p].float().cpu().numpy()
                err = row_rel_err(o, ref[p])
                assert err <= ROW_REL_TOL, (i, p, err)


SCENARIOS = {
    "run_waits_then_peers_publish[none_early]": lambda orc: run_waits_then_peers_publish(orc, ()),
    "run_waits_then_peers_publish[peer0_early]": lambda orc: run_waits_then_peers_publish(orc, (0,)),
    "ready_run_gathers_a_peer_that_arrives_during_the_window": ready_run_gathers_a_peer_that_arrives_during_the_window,
    "ready_run_waits_for_the_first_peer": ready_run_waits_for_the_first_peer,
    "ring_depth_two_next_stage_published_while_the_first_runs": ring_depth_two_next_stage_published_while_the_first_runs,
    "serve_loop_with_peers_publishing_during_the_loop": serve_loop_with_peers_publishing_during_the_loop,
}


def main(out):
    from oracle import oracle as orc
    orc.lib()
    res = {}
    for name, fn in SCENARIOS.items():
        say(f"[concurrent] {name}")
        try:
            fn(orc)
            res[name] = "ok"
        except Exception:
            res[name] = traceback.format_exc()
            say(res[name])
        with open(out, "w") as f:
            json.dump(res, f)


if __name__ == "__main__":
    main(sys.argv[1])
