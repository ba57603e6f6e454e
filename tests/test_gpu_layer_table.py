"""GPU: layer-select runs (device layer table) and the captured FFN loop.

"[RFC]: Async AFD for Prefill on Ascend NPU", "Architecture" (layer-select
operators: an address table of every layer's weights and a layer index kept
on the device) and "FFN execution modes" (eager mode; graph mode: the loop
over work items captured once and replayed, fixed-shape buffers, a fixed
iteration count, device-side spinning on the ready flags, serialized buffer
reuse).  Each layer has its own seeded weights; every run is checked against
the oracle with the weights of the layer its headers name, and the replays
of the captured loop bit for bit against eager layer-table runs of the same
inputs.  The loop also runs on an attention-routed window, where every stage
of the ring keeps its own routing state on the peer side.
"""
import dataclasses

import numpy as np
import pytest

from combine_afd_slot_amd import afd
from combine_afd_slot_amd.driver import FfnSession, _dev_bf16
from combine_afd_slot_amd.inputs import make_inputs, small_workload
from gpu_util import ROW_REL_TOL, row_rel_err, say

pytestmark = pytest.mark.gpu

WL = small_workload("layers", seq_lens=(21, 0, 34), hidden=128, num_experts=8, top_k=2, intermediate=64,
                    shared_intermediate=64, token_cap=40)
N_LAYERS = 3
HDR_LAYER = 5  # AFD_HDR_LAYER: header word of layer_idx


def _layer_weights(wl, n):
    return [make_inputs(wl.with_(seed=50 + i)) for i in range(n)]


def _pack_layers(s, ws):
    """Upload and pack each layer's weights; returns (packed buffers, keep-alive list)."""
    torch = s.torch
    nbytes = s.layout.packed_weight_bytes
    packed, keep = [], []
    for w in ws:
        t = [_dev_bf16(torch, w[k], s.dev) for k in ("W13", "W2", "Ws13", "Ws2")]
        buf = torch.empty(nbytes, dtype=torch.uint8, device=s.dev)
        torch.cuda.synchronize(s.dev)
        afd.afd_weights_pack(s.win, *(x.data_ptr() for x in t), buf.data_ptr(), nbytes, s.ffn_stream.cuda_stream)
        s.ffn_stream.synchronize()
        packed.append(buf)
        keep.append(t)
    return packed, keep


def _oracle(orc, wl, inp, w):
    return orc.ffn(inp["x"], inp["l"], w["W13"], w["W2"], w["Ws13"], w["Ws2"], K=wl.top_k)["out_p"]


def _ret_header(s, peer, stage):
    L = s.layout
    off = L.ret_off + (L.in_slots_off - L.in_off) + (peer * s.wl.ring_depth + stage) * L.slot_bytes + L.field_off[0]
    return np.frombuffer(afd.afd_debug_read(s.win, off, 4 * 12), np.int32)


def _in_header(s, peer, stage):
    L = s.layout
    off = L.in_slots_off + (peer * s.wl.ring_depth + stage) * L.slot_bytes + L.field_off[0]
    return np.frombuffer(afd.afd_debug_read(s.win, off, 4 * 12), np.int32).copy(), off


def test_layer_table_selects_weights_on_the_device(orc):
    ws = _layer_weights(WL, N_LAYERS)
    with FfnSession(WL, make_inputs(WL), poll_timeout_us=200_000, weights=False) as s:
        packed, keep = _pack_layers(s, ws)
        afd.afd_layer_table_set(s.win, [b.data_ptr() for b in packed], s.ffn_stream.cuda_stream)
        for i, layer in enumerate((2, 0, 1, 2)):
            inp = make_inputs(WL.with_(seed=200 + i), with_weights=False)
            s.set_inputs(inp)
            say(f"[layer-table] run {i} layer {layer}")
            s.pack_all(0, layer)
            afd.afd_ffn_run_table(s.win, 0, s.ffn_stream.cuda_stream)
            s.ffn_stream.synchronize()
            st = s.status()
            assert st.status == 0, st.status
            for p in range(WL.num_peers):
                if WL.seq_lens[p]:
                    assert _ret_header(s, p, 0)[HDR_LAYER] == layer
            s.unpack_all()
            ref = _oracle(orc, WL, inp, ws[layer])
            for p, o in enumerate(s.outputs_f32()):
                err = row_rel_err(o, ref[p])
                assert err <= ROW_REL_TOL, (i, layer, p, err)


def test_layer_table_errors(orc):
    ws = _layer_weights(WL, 2)
    with FfnSession(WL, make_inputs(WL), poll_timeout_us=200_000, weights=False) as s:
        st_ = s.ffn_stream.cuda_stream
        # no table yet
        with pytest.raises(afd.AfdError) as ei:
            afd.afd_ffn_run_table(s.win, 0, st_)
        assert ei.value.code == afd.AFD_ERR_INVALID
        packed, keep = _pack_layers(s, ws)
        for bad in ([], [packed[0].data_ptr() + 16], [packed[0].data_ptr(), 0]):
            with pytest.raises(afd.AfdError) as ei:
                afd.afd_layer_table_set(s.win, bad, st_)
            assert ei.value.code == afd.AFD_ERR_INVALID
        with pytest.raises(afd.AfdError) as ei:
            afd.afd_ffn_run_table(s.win, 1, st_)  # stage out of range (ring depth 1)
        assert ei.value.code == afd.AFD_ERR_INVALID
        afd.afd_layer_table_set(s.win, [b.data_ptr() for b in packed], st_)
        inp = make_inputs(WL.with_(seed=300), with_weights=False)
        s.set_inputs(inp)

        # the peers' headers disagree on the layer: nothing consumed or published
        s.pack(0, 0, 1)
        s.pack(1, 0, 1)
        s.pack(2, 0, 0)
        for ps in s.peer_streams:
            ps.synchronize()
        afd.afd_ffn_run_table(s.win, 0, st_)
        st = s.status()
        assert st.status == afd.AFD_ERR_HEADER and st.failed_peer == 2, (st.status, st.failed_peer)
        assert afd.afd_window_poll(s.win, 1, 3) == [0, 0, 0]
        # a layer past the table: every header names layer 2 of a 2-entry table
        saved = []
        for p in range(3):
            hw, off = _in_header(s, p, 0)
            saved.append((hw.copy(), off))
            hw[HDR_LAYER] = 2
            afd.afd_debug_write(s.win, off, hw.tobytes())
        afd.afd_ffn_run_table(s.win, 0, st_)
        st = s.status()
        assert st.status == afd.AFD_ERR_HEADER, st.status
        # all headers name layer 1: the run goes through with layer 1's weights
        for hw, off in saved:
            hw[HDR_LAYER] = 1
            afd.afd_debug_write(s.win, off, hw.tobytes())
        afd.afd_ffn_run_table(s.win, 0, st_)
        s.ffn_stream.synchronize()
        assert s.status().status == 0
        s.unpack_all()
        ref = _oracle(orc, WL, inp, ws[1])
        for p, o in enumerate(s.outputs_f32()):
            assert row_rel_err(o, ref[p]) <= ROW_REL_TOL


LOOP_WL = small_workload("loop", seq_lens=(21, 34), hidden=128, num_experts=8, top_k=2, intermediate=64,
                         shared_intermediate=64, token_cap=40, ring_depth=4)


def _dev_inputs(s, inp):
    torch = s.torch
    x = [_dev_bf16(torch, a, s.dev) for a in inp["x"]]
    lg = [torch.from_numpy(np.ascontiguousarray(a)).to(s.dev) for a in inp["l"]]
    out = [torch.empty((n, s.wl.hidden), dtype=torch.bfloat16, device=s.dev) for n in s.wl.seq_lens]
    return x, lg, out


@pytest.mark.parametrize("attention_routes", [0, 1])
def test_captured_loop_replays(orc, attention_routes):
    """Four runs on stages 1, 2, 3, 0 (ring depth 4) captured once and
    replayed three times, with eager runs and host synchronization between
    the replays.  Each replay's messages are packed and complete before it is
    launched, and unpacked after it, so no stream waits on the device for
    work queued on another (a waiting kernel may hold a hardware queue that
    other streams share); the stages are reused across replays."""
    wl = dataclasses.replace(LOOP_WL, attention_routes=attention_routes)
    ws = _layer_weights(wl, N_LAYERS)
    layers = (1, 0, 2, 1)
    n_runs, R, first = len(layers), wl.ring_depth, 1
    with FfnSession(wl, make_inputs(wl), poll_timeout_us=500_000, weights=False) as s:
        torch = s.torch
        packed, keep = _pack_layers(s, ws)
        afd.afd_layer_table_set(s.win, [b.data_ptr() for b in packed], s.ffn_stream.cuda_stream)
        loop = afd.afd_ffn_loop_create(s.win, n_runs, first, s.ffn_stream.cuda_stream)
        try:
            for rep in range(3):
                inps = [make_inputs(wl.with_(seed=1000 + 10 * rep + i), with_weights=False) for i in range(n_runs)]
                bufs = [_dev_inputs(s, inp) for inp in inps]
                torch.cuda.synchronize(s.dev)
                say(f"[loop] replay {rep}: enqueue peers and the loop")

                stage = [(first + i) % R for i in range(n_runs)]
                for i in range(n_runs):
                    x, lg, _ = bufs[i]
                    for p in range(wl.num_peers):
                        afd.afd_slot_pack(s.win, p, stage[i], layers[i], wl.seq_lens[p], x[p].data_ptr(),
                                          lg[p].data_ptr(), 0, s.peer_streams[p].cuda_stream)
                for ps in s.peer_streams:
                    ps.synchronize()
                afd.afd_ffn_loop_launch(loop, s.ffn_stream.cuda_stream)
                s.ffn_stream.synchronize()
                for i in range(n_runs):
                    out = bufs[i][2]
                    for p in range(wl.num_peers):
                        afd.afd_slot_unpack(s.win, p, stage[i], wl.seq_lens[p], out[p].data_ptr(),
                                            s.peer_streams[p].cuda_stream)
                for ps in s.peer_streams:
                    ps.synchronize()
                say(f"[loop] replay {rep}: check")
                for stg in range(R):
                    assert s.status(stg).status == 0
                    for p in range(wl.num_peers):
                        assert s.peer_status(p, stg).status == 0
                graph_out = [[o.float().cpu().numpy() for o in b[2]] for b in bufs]
                for i in range(n_runs):
                    ref = _oracle(orc, wl, inps[i], ws[layers[i]])
                    for p in range(wl.num_peers):
                        err = row_rel_err(graph_out[i][p], ref[p])
                        assert err <= ROW_REL_TOL, (rep, i, p, err)
                # eager layer-table runs of the same inputs give the same bits
                for i in range(n_runs):
                    s.set_inputs(inps[i])
                    s.pack_all(stage[i], layers[i])
                    afd.afd_ffn_run_table(s.win, stage[i], s.ffn_stream.cuda_stream)
                    s.ffn_stream.synchronize()
                    assert s.status(stage[i]).status == 0
                    s.unpack_all(stage[i])
                    for p, o in enumerate(s.outputs_f32()):
                        np.testing.assert_array_equal(o, graph_out[i][p])
        finally:
            afd.afd_ffn_loop_destroy(loop)


def test_loop_create_argument_errors():
    with FfnSession(LOOP_WL, make_inputs(LOOP_WL), weights=True) as s:
        st_ = s.ffn_stream.cuda_stream
        with pytest.raises(afd.AfdError) as ei:  # no layer table
            afd.afd_ffn_loop_create(s.win, 2, 0, st_)
        assert ei.value.code == afd.AFD_ERR_INVALID
        afd.afd_layer_table_set(s.win, [s.packed.data_ptr()], st_)
        for n, first, stream in ((0, 0, st_), (2, 4, st_), (2, -1, st_), (2, 0, 0)):
            with pytest.raises(afd.AfdError) as ei:
                afd.afd_ffn_loop_create(s.win, n, first, stream)
            assert ei.value.code == afd.AFD_ERR_INVALID
        afd.afd_profile_enable(s.win, 1)
        with pytest.raises(afd.AfdError) as ei:
            afd.afd_ffn_loop_create(s.win, 2, 0, st_)
        assert ei.value.code == afd.AFD_ERR_INVALID
        afd.afd_profile_enable(s.win, 0)
        afd.afd_ffn_loop_destroy(None)


SERVE_WL = small_workload("serve", seq_lens=(21, 34), hidden=128, num_experts=8, top_k=2, intermediate=64,
                          shared_intermediate=64, token_cap=40, ring_depth=2)


@pytest.mark.parametrize("attention_routes", [0, 1])
def test_serve_loop(orc, attention_routes):
    """The connector-driven loop (afd_ffn_serve): items run back to back with
    no host synchronisation; the first timeout or shutdown stops the loop on
    the device and the items after it consume nothing."""
    wl = dataclasses.replace(SERVE_WL, attention_routes=attention_routes)
    ws = _layer_weights(wl, 2)
    with FfnSession(wl, make_inputs(wl), poll_timeout_us=20_000, weights=False) as s:
        torch = s.torch
        st_ = s.ffn_stream.cuda_stream
        with pytest.raises(afd.AfdError) as ei:  # no layer table yet
            afd.afd_ffn_serve(s.win, 0, 2, 0, 0, st_)
        assert ei.value.code == afd.AFD_ERR_INVALID
        packed, keep = _pack_layers(s, ws)
        afd.afd_layer_table_set(s.win, [b.data_ptr() for b in packed], st_)
        for args in ((0, 0, 0, 0), (2, 1, 0, 0), (0, 1, 3, 0), (0, 1, 1, 20_001)):
            with pytest.raises(afd.AfdError) as ei:
                afd.afd_ffn_serve(s.win, *args, st_)
            assert ei.value.code == afd.AFD_ERR_INVALID, args

        def pack(stage, layer, inp, peers=(0, 1), flags=0):
            x, lg, out = _dev_inputs(s, inp)
            torch.cuda.synchronize(s.dev)
            for p in peers:
                n = 0 if flags else wl.seq_lens[p]
                afd.afd_slot_pack(s.win, p, stage, layer, n, x[p].data_ptr() if n else 0,
                                  lg[p].data_ptr() if n else 0, flags, s.peer_streams[p].cuda_stream)
            for ps in s.peer_streams:
                ps.synchronize()
            return out

        def unpack(stage, out, peers=(0, 1)):
            for p in peers:
                afd.afd_slot_unpack(s.win, p, stage, wl.seq_lens[p], out[p].data_ptr(), s.peer_streams[p].cuda_stream)
            for ps in s.peer_streams:
                ps.synchronize()
            return [o.float().cpu().numpy() for o in out]

        # two items ready (stage 0 layer 1, stage 1 layer 0); the third times out, the fourth is skipped
        inps = [make_inputs(wl.with_(seed=700 + i), with_weights=False) for i in range(3)]
        outs = [pack(0, 1, inps[0]), pack(1, 0, inps[1])]
        say("[serve] four items, two ready")
        afd.afd_ffn_serve(s.win, 0, 4, 0, 0, st_)
        assert afd.afd_ffn_serve_result(s.win, st_) == (afd.AFD_ERR_TIMEOUT, 2, 2)
        for stage, layer, out, inp in ((0, 1, outs[0], inps[0]), (1, 0, outs[1], inps[1])):
            got = unpack(stage, out)
            ref = _oracle(orc, wl, inp, ws[layer])
            for p in range(wl.num_peers):
                assert row_rel_err(got[p], ref[p]) <= ROW_REL_TOL, (stage, p)
        # every peer sends the shutdown sentinel on stage 0: the loop stops at its first item
        pack(0, 0, inps[2], flags=afd.AFD_FLAG_SHUTDOWN)
        say("[serve] shutdown")
        afd.afd_ffn_serve(s.win, 0, 3, 0, 0, st_)
        assert afd.afd_ffn_serve_result(s.win, st_) == (afd.AFD_SHUTDOWN, 0, 0)
        # any-ready items: only peer 1 has a message on stage 1
        out = pack(1, 1, inps[2], peers=(1,))
        say("[serve] any-ready")
        afd.afd_ffn_serve(s.win, 1, 2, 2, 0, st_)
        assert afd.afd_ffn_serve_result(s.win, st_) == (afd.AFD_ERR_TIMEOUT, 1, 1)
        got = unpack(1, out, peers=(1,))
        ref = _oracle(orc, wl, inps[2], ws[1])
        assert row_rel_err(got[1], ref[1]) <= ROW_REL_TOL
