"""GPU protocol tests: slot contents, flags, and the failure paths, each forced
from the host (a withheld publish, a corrupted header written with
afd_debug_write, a repeated flag value).  Every kernel still exits normally:
waits are bounded by a short poll timeout.

Sources: "[RFC]: Async GPU Connector" ("Window and slot layout": slot fields,
header self-check, shutdown bit, seq flags; "Capacity and ring depth":
overflow raises, ring exhaustion is an error; "Risks and alternatives":
echo_seq turns a mismatched reply into an explicit error) and "Data on the
wire" (shape checks).
"""
import numpy as np
import pytest

from combine_afd_slot_amd import afd
from combine_afd_slot_amd.driver import FfnSession
from combine_afd_slot_amd.inputs import WORKLOADS, make_inputs, small_workload, bf16_to_f32
from gpu_util import ROW_REL_TOL, row_rel_err, say
from oracle import protocol as ref

pytestmark = pytest.mark.gpu

TINY = WORKLOADS["tiny"]


def _session(wl=TINY, timeout_us=20_000, inp=None):
    inp = make_inputs(wl) if inp is None else inp
    return FfnSession(wl, inp, poll_timeout_us=timeout_us), inp


def _slot_off(s, win_off, peer, stage):
    L = s.layout
    first = L.in_slots_off - L.in_off
    return win_off + first + (peer * s.wl.ring_depth + stage) * L.slot_bytes


def _read_header(s, which, peer, stage=0):
    L = s.layout
    base = L.in_off if which == 0 else L.ret_off
    off = _slot_off(s, base, peer, stage) + L.field_off[0]
    raw = afd.afd_debug_read(s.win, off, 4 * (12 + s.wl.num_experts))
    return np.frombuffer(raw, np.int32).copy(), off


def _oracle_out(orc, wl, inp):
    return orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], inp.get("Ws13"), inp.get("Ws2"), K=wl.top_k)


def test_pack_writes_slot_fields_and_flag():
    say("[protocol] pack slot contents")
    s, inp = _session()
    with s:
        s.pack_all(layer=3)
        L = s.layout
        E, H = TINY.num_experts, TINY.hidden
        for p, n in enumerate(TINY.seq_lens):
            so = _slot_off(s, L.in_off, p, 0)
            rx = np.frombuffer(afd.afd_debug_read(s.win, so + L.field_off[2], 2 * n * H), np.uint16)
            sx = np.frombuffer(afd.afd_debug_read(s.win, so + L.field_off[4], 2 * n * H), np.uint16)
            rt = np.frombuffer(afd.afd_debug_read(s.win, so + L.field_off[1], 4 * n * E), np.float32)
            si = np.frombuffer(afd.afd_debug_read(s.win, so + L.field_off[3], 4 * n), np.int32)
            np.testing.assert_array_equal(rx.reshape(n, H), inp["x"][p])
            np.testing.assert_array_equal(sx.reshape(n, H), inp["x"][p])
            np.testing.assert_array_equal(rt.reshape(n, E), inp["l"][p])
            np.testing.assert_array_equal(si, np.arange(n))
            hw, _ = _read_header(s, 0, p)
            d = ref.decode_header(hw, E)
            assert d["seq"] == 1 and d["layer_idx"] == 3 and d["stage_idx"] == 0
            assert d["num_tokens"] == n and d["shared_tokens"] == n and d["src_peer"] == p
            assert not d["shutdown"]
        assert afd.afd_window_poll(s.win, 0, TINY.num_peers) == [1, 1]
        assert afd.afd_window_poll(s.win, 1, TINY.num_peers) == [0, 0]


def test_return_header_and_flags():
    s, inp = _session()
    with s:
        s.step(layer=2)
        s.pack_all(layer=2)
        s.run(layer=2)
        s.ffn_stream.synchronize()
        assert afd.afd_window_poll(s.win, 1, 2) == [2, 2]
        for p in range(2):
            hw, _ = _read_header(s, 1, p)
            d = ref.decode_header(hw, TINY.num_experts)
            assert d["echo_seq"] == 2 and d["seq"] == 2 and d["num_tokens"] == TINY.seq_lens[p]
            assert d["layer_idx"] == 2 and d["src_peer"] == p
            assert d["counts"].sum() == TINY.seq_lens[p] * TINY.top_k
        s.unpack_all()
        assert all(s.peer_status(p).status == 0 for p in range(2))


def test_routed_only_window(orc):
    """No shared expert on the FFN side: the routed-only protocol ("[RFC]:
    Async AFD for Prefill on Ascend NPU", "Shared-expert ownership").  The
    slots have no shared fields, messages and replies carry shared_tokens =
    0, the output is the routed branch alone, and a message that claims
    shared rows is a header error."""
    wl = small_workload("routed_only", seq_lens=(19, 0, 30), hidden=64, num_experts=8, top_k=2,
                        intermediate=48, shared_intermediate=0, token_cap=32)
    inp = make_inputs(wl)
    with FfnSession(wl, inp, poll_timeout_us=200_000) as s:
        L = s.layout
        assert L.field_bytes[3] == 0 and L.field_bytes[4] == 0
        assert L.slot_bytes == sum(ref.align_up(L.field_bytes[i]) for i in range(3))
        s.pack_all(layer=1)
        for p, n in enumerate(wl.seq_lens):
            so = _slot_off(s, L.in_off, p, 0)
            rx = np.frombuffer(afd.afd_debug_read(s.win, so + L.field_off[2], 2 * n * wl.hidden), np.uint16)
            np.testing.assert_array_equal(rx.reshape(n, wl.hidden), inp["x"][p])
            d = ref.decode_header(_read_header(s, 0, p)[0], wl.num_experts)
            assert d["num_tokens"] == n and d["routed_tokens"] == n and d["shared_tokens"] == 0
        s.run(layer=1)
        s.ffn_stream.synchronize()
        assert s.status().status == 0
        for p, n in enumerate(wl.seq_lens):
            if n:
                d = ref.decode_header(_read_header(s, 1, p)[0], wl.num_experts)
                assert d["num_tokens"] == n and d["shared_tokens"] == 0
        s.unpack_all()
        r = orc.ffn(inp["x"], inp["l"], inp["W13"], inp["W2"], None, None, K=wl.top_k)
        for p, o in enumerate(s.outputs_f32()):
            assert row_rel_err(o, r["out_p"][p]) <= ROW_REL_TOL
        # a message with shared rows on a routed-only window
        s.pack_all(layer=1)
        hw, off = _read_header(s, 0, 2)
        bad = hw.copy()
        bad[ref.WORD["shared_tokens"]] = wl.seq_lens[2]
        afd.afd_debug_write(s.win, off, bad.tobytes())
        s.run(layer=1)
        st = s.status()
        assert st.status == afd.AFD_ERR_HEADER and st.failed_peer == 2
        afd.afd_debug_write(s.win, off, hw.tobytes())
        s.run(layer=1)
        s.ffn_stream.synchronize()
        assert s.status().status == 0
        s.unpack_all()


def test_missing_peer_times_out_then_recovers(orc):
    say("[protocol] timeout (20 ms bound), then recovery")
    s, inp = _session(timeout_us=20_000)
    with s:
        s.pack(0)
        s.peer_streams[0].synchronize()
        s.run()
        st = s.status()
        assert st.status == afd.AFD_ERR_TIMEOUT and st.failed_peer == 1
        assert afd.afd_window_poll(s.win, 1, 2) == [0, 0]  # nothing published
        s.pack(1)
        s.peer_streams[1].synchronize()
        s.run()
        assert s.status().status == 0  # peer 0's message was not consumed by the failed run
        s.ffn_stream.synchronize()
        s.unpack_all()
        r = _oracle_out(orc, TINY, inp)
        for p, o in enumerate(s.outputs_f32()):
            assert row_rel_err(o, r["out_p"][p]) <= ROW_REL_TOL


def test_stale_flag_is_not_consumed_twice():
    s, inp = _session(timeout_us=20_000)
    with s:
        s.step()
        # re-announce the old seq: the FFN mirror has already seen it
        s.run()
        st = s.status()
        assert st.status == afd.AFD_ERR_TIMEOUT


def test_shutdown_bit():
    s, inp = _session()
    with s:
        s.pack(0, flags=afd.AFD_FLAG_SHUTDOWN)
        s.pack(1)
        for q in s.peer_streams:
            q.synchronize()
        s.run()
        st = s.status()
        assert st.status == afd.AFD_SHUTDOWN
        assert afd.afd_window_poll(s.win, 1, 2) == [0, 0]


@pytest.mark.parametrize("word,value", [(ref.WORD["magic"], 0x0BADF00D), (ref.WORD["version"], 9),
                                        (ref.WORD["n_counts"], 3), (ref.WORD["layer_idx"], 77),
                                        (ref.WORD["num_tokens"], 99), (ref.WORD["src_peer"], 0)])
def test_corrupt_header_rejected_then_fixed(orc, word, value):
    s, inp = _session()
    with s:
        s.pack_all()
        hw, off = _read_header(s, 0, 1)
        bad = hw.copy()
        bad[word] = value
        afd.afd_debug_write(s.win, off, bad.tobytes())
        s.run()
        st = s.status()
        assert st.status == afd.AFD_ERR_HEADER and st.failed_peer == 1
        assert afd.afd_window_poll(s.win, 1, 2) == [0, 0]
        afd.afd_debug_write(s.win, off, hw.tobytes())
        s.run()
        assert s.status().status == 0
        s.ffn_stream.synchronize()
        s.unpack_all()
        r = _oracle_out(orc, TINY, inp)
        for p, o in enumerate(s.outputs_f32()):
            assert row_rel_err(o, r["out_p"][p]) <= ROW_REL_TOL


def test_echo_seq_mismatch_is_an_error():
    s, inp = _session()
    with s:
        s.pack_all()
        s.run()
        s.ffn_stream.synchronize()
        hw, off = _read_header(s, 1, 0)
        bad = hw.copy()
        bad[ref.WORD["echo_seq"]] += 5
        afd.afd_debug_write(s.win, off, bad.tobytes())
        s.out[0].fill_(7.0)
        s.torch.cuda.synchronize()
        s.unpack_all()
        st = s.peer_status(0)
        assert st.status == afd.AFD_ERR_SEQ and st.failed_peer == 0
        assert (s.out[0].float() == 7.0).all().item()  # nothing copied
        assert s.peer_status(1).status == 0


def test_host_errors_capacity_ring_shape():
    s, inp = _session()
    with s:
        with pytest.raises(afd.AfdError) as ei:
            s.pack(0, seq_len=TINY.token_cap + 1)
        assert ei.value.code == afd.AFD_ERR_CAPACITY
        s.pack(0)
        with pytest.raises(afd.AfdError) as ei:
            s.pack(0)
        assert ei.value.code == afd.AFD_ERR_RING
        with pytest.raises(afd.AfdError) as ei:
            afd.afd_slot_unpack(s.win, 0, 0, TINY.seq_lens[0] + 1, s.out[0].data_ptr(),
                                s.peer_streams[0].cuda_stream)
        assert ei.value.code == afd.AFD_ERR_SHAPE
        with pytest.raises(afd.AfdError) as ei:
            afd.afd_slot_pack(s.win, 5, 0, 0, 1, s.x[0].data_ptr(), s.l[0].data_ptr(), 0, 0)
        assert ei.value.code == afd.AFD_ERR_INVALID
        s.pack(1)
        for q in s.peer_streams:
            q.synchronize()
        s.run()
        s.ffn_stream.synchronize()
        s.unpack_all()
        assert s.status().status == 0


def test_weight_pack_and_run_argument_errors():
    s, inp = _session()
    with s:
        n = s.layout.packed_weight_bytes
        ws = (s.w13.data_ptr(), s.w2.data_ptr(), s.ws13.data_ptr(), s.ws2.data_ptr())
        for args in [(*ws, 0, n),                              # no destination
                     (*ws, s.packed.data_ptr(), n - 16),        # too small
                     (*ws, s.packed.data_ptr() + 16, n),        # not 256-byte aligned
                     (0, *ws[1:], s.packed.data_ptr(), n),      # no routed gate/up weights
                     (*ws[:2], 0, ws[3], s.packed.data_ptr(), n)]:  # shared weights missing
            with pytest.raises(afd.AfdError) as ei:
                afd.afd_weights_pack(s.win, *args, s.ffn_stream.cuda_stream)
            assert ei.value.code == afd.AFD_ERR_INVALID
        for pw in (0, s.packed.data_ptr() + 16):
            with pytest.raises(afd.AfdError) as ei:
                afd.afd_ffn_run(s.win, 0, 0, pw, s.ffn_stream.cuda_stream)
            assert ei.value.code == afd.AFD_ERR_INVALID
        # the rejected calls left the window usable
        s.step()
        assert s.status().status == 0


def test_profile_modes():
    """Per-kernel event timing: mode 1 times every kernel, mode 2 the two
    GEMMs, mode 3 the gate/up GEMM only; other modes are rejected."""
    s, _ = _session()
    with s:
        names = [afd.lib().afd_profile_kernel_name(i).decode() for i in range(afd.AFD_PROFILE_SLOTS)]
        used = [n for n in names if n != "unused"]
        for mode, timed in ((1, set(used)), (2, {"gemm_gate_up_swiglu", "gemm_down"}), (3, {"gemm_gate_up_swiglu"})):
            afd.afd_profile_enable(s.win, mode)
            afd.afd_profile_read(s.win, reset=True)
            for _ in range(3):
                s.step()
            tot, runs = afd.afd_profile_read(s.win, reset=True)
            say(f"[protocol] profile mode {mode}: runs {runs} {tot}")
            assert runs >= 2
            for n in used:
                assert (tot[n] > 0.0) == (n in timed), (mode, n, tot[n])
        afd.afd_profile_enable(s.win, 0)
        for bad in (-1, 4):
            with pytest.raises(afd.AfdError) as ei:
                afd.afd_profile_enable(s.win, bad)
            assert ei.value.code == afd.AFD_ERR_INVALID
        s.step()
        assert s.status().status == 0


def test_repeated_execution_and_ring_depth_two(orc):
    wl = small_workload("ring2", seq_lens=(21, 0, 34), hidden=128, num_experts=8, top_k=2, intermediate=64,
                        shared_intermediate=64, token_cap=40, ring_depth=2)
    base = make_inputs(wl)
    with FfnSession(wl, base, poll_timeout_us=200_000) as s:
        for it in range(4):
            stage = it % 2
            wl_i = wl.with_(seed=100 + it)
            inp = make_inputs(wl_i, with_weights=False)
            inp.update({k: base[k] for k in ("W13", "W2", "Ws13", "Ws2")})
            s.set_inputs(inp)
            say(f"[protocol] repeated run {it} stage {stage}")
            s.step(stage=stage, layer=it)
            assert s.status(stage).status == 0
            r = _oracle_out(orc, wl, inp)
            for p, o in enumerate(s.outputs_f32()):
                assert row_rel_err(o, r["out_p"][p]) <= ROW_REL_TOL, (it, p)


def test_all_peers_empty():
    wl = small_workload("empty", seq_lens=(0, 0), hidden=64, num_experts=8, top_k=2, intermediate=32,
                        shared_intermediate=32, token_cap=8)
    inp = make_inputs(wl)
    with FfnSession(wl, inp, poll_timeout_us=200_000) as s:
        s.step()
        st = s.status()
        assert st.status == 0 and st.total_tokens == 0
        assert afd.afd_window_poll(s.win, 1, 2) == [0, 0]


@pytest.mark.parametrize("attention_routes", [0, 1])
def test_poison_mode(orc, monkeypatch, attention_routes):
    """AFD_POISON=1: every pack fills its slot's payload fields, and every run
    the return slots of the peers it serves, with 0xFFFFFFFF (NaN as bf16 and
    fp32) before writing, so a kernel that read a row the current message did
    not write would see NaN.  A full-length message followed by shorter ones
    (an empty peer among them) must give the oracle's rows and, bit for bit,
    the rows of a window without poisoning; the rows past each message read
    as the poison."""
    import dataclasses
    wl = small_workload("poison", seq_lens=(96, 0, 51), hidden=256, num_experts=12, top_k=3, intermediate=200,
                        shared_intermediate=136, token_cap=96, attention_routes=attention_routes)
    short = dataclasses.replace(wl, seq_lens=(37, 0, 12))
    full_inp, short_inp = make_inputs(wl), make_inputs(short.with_(seed=5))
    for k in ("W13", "W2", "Ws13", "Ws2"):
        short_inp[k] = full_inp[k]
    with FfnSession(wl, full_inp, poll_timeout_us=200_000) as s:
        s.step()
        s.wl = short
        s.set_inputs(short_inp)
        s.step()
        assert s.status().status == 0
        base = [o.copy() for o in s.outputs_f32()]
    monkeypatch.setenv("AFD_POISON", "1")
    with FfnSession(wl, full_inp, poll_timeout_us=200_000) as s:
        s.step()
        assert s.status().status == 0
        s.wl = short
        s.set_inputs(short_inp)
        s.step()
        st = s.status()
        assert st.status == 0 and st.total_tokens == short.total_tokens
        ref = _oracle_out(orc, short, short_inp)["out_p"]
        L, H = s.layout, wl.hidden
        for p, n in enumerate(short.seq_lens):
            o = s.outputs_f32()[p]
            assert np.isfinite(o).all()
            np.testing.assert_array_equal(o, base[p])
            assert row_rel_err(o, ref[p]) <= ROW_REL_TOL
            # rows past the message: inbound and return slots hold the poison
            rows = (wl.token_cap - n) if not attention_routes else 0
            if rows:
                for win in (L.in_off, L.ret_off):
                    off = _slot_off(s, win, p, 0) + L.field_off[2] + 2 * n * H
                    past = np.frombuffer(afd.afd_debug_read(s.win, off, 2 * rows * H), np.uint16)
                    assert (past == 0xFFFF).all(), (p, win)
