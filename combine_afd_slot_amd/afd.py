"""ctypes binding of libafd.so (include/afd.h).

Argument marshalling only: every step of the path runs in the library's HIP
kernels.  Function names match the C ABI.  Device buffers are passed as
integer addresses (e.g. ``tensor.data_ptr()``), streams as integer
hipStream_t handles (e.g. ``torch.cuda.Stream().cuda_stream``), so this module
has no dependency on torch.

The library must have been built (``python -m combine_afd_slot_amd.build``);
loading fails loudly otherwise -- there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libafd.so")

AFD_OK = 0
AFD_SHUTDOWN = 1
AFD_ERR_INVALID = -1
AFD_ERR_CAPACITY = -2
AFD_ERR_SHAPE = -3
AFD_ERR_RING = -4
AFD_ERR_TIMEOUT = -5
AFD_ERR_HEADER = -6
AFD_ERR_SEQ = -7
AFD_ERR_DEVICE = -8
AFD_FLAG_SHUTDOWN = 0x2
AFD_NUM_FIELDS = 5
AFD_PROFILE_SLOTS = 8
AFD_STATIC_WINDOW_BYTES = 32 << 20  # the static window of afd_window_create_static
FIELDS = ("header", "route_table", "routed_x", "shared_idx", "shared_x")
HDR_WORDS = 12

# Every symbol include/afd.h declares.
EXPORTS = (
    "afd_layout_compute", "afd_window_create", "afd_window_create_static", "afd_window_destroy", "afd_window_layout",
    "afd_slot_pack", "afd_weights_pack", "afd_ffn_run", "afd_ffn_run_ready", "afd_layer_table_set", "afd_ffn_run_table",
    "afd_ffn_loop_create", "afd_ffn_loop_launch", "afd_ffn_loop_destroy", "afd_ffn_serve", "afd_ffn_serve_result",
    "afd_slot_unpack", "afd_slot_unpack_ranks", "afd_window_status", "afd_peer_status",
    "afd_window_poll", "afd_debug_routing", "afd_debug_read", "afd_debug_write",
    "afd_profile_enable", "afd_profile_read", "afd_profile_kernel_name",
    "afd_header_encode", "afd_header_decode", "afd_last_error", "afd_status_string",
    "afd_abi_version",
)


class AfdError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"{status_string(code)} ({code}): {msg}")
        self.code = code


class WindowConfig(ctypes.Structure):
    _fields_ = [("struct_size", ctypes.c_uint32), ("num_peers", ctypes.c_int32),
                ("ring_depth", ctypes.c_int32), ("token_cap", ctypes.c_int32),
                ("hidden", ctypes.c_int32), ("num_experts", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("intermediate", ctypes.c_int32), ("shared_intermediate", ctypes.c_int32),
                ("routed_scaling_factor", ctypes.c_float), ("renormalize", ctypes.c_int32),
                ("poll_timeout_us", ctypes.c_int32), ("attention_routes", ctypes.c_int32),
                ("route_experts", ctypes.c_int32), ("expert_offset", ctypes.c_int32),
                ("w1_fp8", ctypes.c_int32), ("reserved", ctypes.c_int32 * 1)]


class Layout(ctypes.Structure):
    _fields_ = [("field_off", ctypes.c_int64 * AFD_NUM_FIELDS), ("field_bytes", ctypes.c_int64 * AFD_NUM_FIELDS),
                ("slot_bytes", ctypes.c_int64), ("window_bytes", ctypes.c_int64), ("in_off", ctypes.c_int64),
                ("in_slots_off", ctypes.c_int64), ("ret_off", ctypes.c_int64), ("ret_slots_off", ctypes.c_int64),
                ("workspace_off", ctypes.c_int64), ("workspace_bytes", ctypes.c_int64),
                ("total_bytes", ctypes.c_int64), ("packed_weight_bytes", ctypes.c_int64)]


class RunInfo(ctypes.Structure):
    _fields_ = [("status", ctypes.c_int32), ("failed_peer", ctypes.c_int32), ("last_seq", ctypes.c_int32),
                ("total_tokens", ctypes.c_int32), ("served_mask", ctypes.c_uint64)]


class MoeWeights(ctypes.Structure):
    _fields_ = [("w13", ctypes.c_void_p), ("w2", ctypes.c_void_p), ("ws13", ctypes.c_void_p),
                ("ws2", ctypes.c_void_p)]


class HeaderFields(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("flags", "seq", "echo_seq", "layer_idx", "stage_idx", "num_tokens",
                                             "routed_tokens", "shared_tokens", "src_peer", "n_counts")]


_lib = None


def lib():
    """Load libafd.so (raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with python -m combine_afd_slot_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        vp, i32, u32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_uint32, ctypes.c_int64
        P = ctypes.POINTER
        sig = {
            "afd_layout_compute": [P(WindowConfig), P(Layout)],
            "afd_window_create": [P(WindowConfig), P(vp)],
            "afd_window_create_static": [P(WindowConfig), P(vp)],
            "afd_window_destroy": [vp],
            "afd_window_layout": [vp, P(Layout)],
            "afd_slot_pack": [vp, i32, i32, i32, i32, vp, vp, u32, vp],
            "afd_weights_pack": [vp, P(MoeWeights), vp, i64, vp],
            "afd_ffn_run": [vp, i32, i32, vp, vp],
            "afd_ffn_run_ready": [vp, i32, i32, vp, i32, i32, vp],
            "afd_layer_table_set": [vp, i32, P(vp), vp],
            "afd_ffn_run_table": [vp, i32, vp],
            "afd_ffn_loop_create": [vp, i32, i32, vp, P(vp)],
            "afd_ffn_loop_launch": [vp, vp],
            "afd_ffn_loop_destroy": [vp],
            "afd_ffn_serve": [vp, i32, i32, i32, i32, vp],
            "afd_ffn_serve_result": [vp, vp, P(i32), P(i32), P(i32)],
            "afd_slot_unpack": [vp, i32, i32, i32, vp, vp],
            "afd_slot_unpack_ranks": [vp, i32, i32, i32, i32, vp, vp],
            "afd_window_status": [vp, i32, vp, P(RunInfo)],
            "afd_peer_status": [vp, i32, i32, vp, P(RunInfo)],
            "afd_window_poll": [vp, i32, vp],
            "afd_debug_routing": [vp, vp, vp, vp, vp, vp, vp, vp, vp],
            "afd_debug_read": [vp, i64, i64, vp],
            "afd_debug_write": [vp, i64, i64, vp],
            "afd_profile_enable": [vp, i32],
            "afd_profile_read": [vp, vp, i32, P(i32), i32],
            "afd_profile_kernel_name": [i32],
            "afd_header_encode": [P(HeaderFields), vp, vp],
            "afd_header_decode": [vp, i32, i32, P(HeaderFields)],
            "afd_last_error": [],
            "afd_status_string": [i32],
            "afd_abi_version": [],
        }
        for name, args in sig.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = i32
        for name in ("afd_last_error", "afd_status_string", "afd_profile_kernel_name"):
            getattr(L, name).restype = ctypes.c_char_p
        _lib = L
    return _lib


def status_string(code: int) -> str:
    return lib().afd_status_string(int(code)).decode()


def last_error() -> str:
    return lib().afd_last_error().decode()


def _check(rc: int) -> int:
    if rc < 0:
        raise AfdError(rc, last_error())
    return rc


def make_config(num_peers, token_cap, hidden, num_experts, top_k, intermediate, shared_intermediate,
                ring_depth=1, routed_scaling_factor=1.0, renormalize=1, poll_timeout_us=2_000_000,
                attention_routes=0, route_experts=0, expert_offset=0, w1_fp8=0) -> WindowConfig:
    c = WindowConfig()
    c.struct_size = ctypes.sizeof(WindowConfig)
    c.num_peers, c.ring_depth, c.token_cap = num_peers, ring_depth, token_cap
    c.hidden, c.num_experts, c.top_k = hidden, num_experts, top_k
    c.intermediate, c.shared_intermediate = intermediate, shared_intermediate
    c.routed_scaling_factor, c.renormalize, c.poll_timeout_us = routed_scaling_factor, renormalize, poll_timeout_us
    c.attention_routes = attention_routes
    c.route_experts, c.expert_offset = route_experts, expert_offset
    c.w1_fp8 = w1_fp8
    return c


def afd_layout_compute(cfg: WindowConfig) -> Layout:
    out = Layout()
    _check(lib().afd_layout_compute(ctypes.byref(cfg), ctypes.byref(out)))
    return out


def afd_window_create(cfg: WindowConfig) -> int:
    h = ctypes.c_void_p()
    _check(lib().afd_window_create(ctypes.byref(cfg), ctypes.byref(h)))
    return h.value


def afd_window_create_static(cfg: WindowConfig) -> int:
    """afd_window_create in the library's static device array (no allocation)."""
    h = ctypes.c_void_p()
    _check(lib().afd_window_create_static(ctypes.byref(cfg), ctypes.byref(h)))
    return h.value


def afd_window_destroy(win: int) -> None:
    _check(lib().afd_window_destroy(win))


def afd_window_layout(win: int) -> Layout:
    out = Layout()
    _check(lib().afd_window_layout(win, ctypes.byref(out)))
    return out


def afd_slot_pack(win, peer, stage, layer_idx, seq_len, hidden_ptr, logits_ptr, flags=0, stream=0) -> int:
    return _check(lib().afd_slot_pack(win, peer, stage, layer_idx, seq_len, hidden_ptr or None,
                                      logits_ptr or None, flags, stream or None))


def afd_weights_pack(win, w13, w2, ws13, ws2, dst, dst_bytes, stream=0) -> int:
    w = MoeWeights(w13, w2, ws13 or None, ws2 or None)
    return _check(lib().afd_weights_pack(win, ctypes.byref(w), dst or None, dst_bytes, stream or None))


def afd_ffn_run(win, stage, layer_idx, packed_weights, stream=0) -> int:
    return _check(lib().afd_ffn_run(win, stage, layer_idx, packed_weights or None, stream or None))


def afd_ffn_run_ready(win, stage, layer_idx, packed_weights, max_peers, gather_us=0, stream=0) -> int:
    """layer_idx < 0: layer from the headers, weights from the layer table."""
    return _check(lib().afd_ffn_run_ready(win, stage, layer_idx, packed_weights or None, max_peers, gather_us,
                                          stream or None))


def afd_layer_table_set(win, packed_ptrs, stream=0) -> int:
    """packed_ptrs: device pointers of each layer's packed weights (entry i = layer i)."""
    arr = (ctypes.c_void_p * len(packed_ptrs))(*[p or None for p in packed_ptrs])
    return _check(lib().afd_layer_table_set(win, len(packed_ptrs), arr, stream or None))


def afd_ffn_run_table(win, stage, stream=0) -> int:
    return _check(lib().afd_ffn_run_table(win, stage, stream or None))


def afd_ffn_loop_create(win, n_runs, first_stage, stream):
    h = ctypes.c_void_p()
    _check(lib().afd_ffn_loop_create(win, n_runs, first_stage, stream or None, ctypes.byref(h)))
    return h.value


def afd_ffn_loop_launch(loop, stream=0) -> int:
    return _check(lib().afd_ffn_loop_launch(loop, stream or None))


def afd_ffn_loop_destroy(loop) -> int:
    return _check(lib().afd_ffn_loop_destroy(loop or None))


def afd_slot_unpack(win, peer, stage, seq_len, out_ptr, stream=0) -> int:
    return _check(lib().afd_slot_unpack(win, peer, stage, seq_len, out_ptr or None, stream or None))


def afd_ffn_serve(win, first_stage, n_items, max_peers=0, gather_us=0, stream=0) -> int:
    return _check(lib().afd_ffn_serve(win, first_stage, n_items, max_peers, gather_us, stream or None))


def afd_ffn_serve_result(win, stream=0):
    """(stop status, items done, stop item) of the last afd_ffn_serve on `stream`."""
    st, done, item = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(lib().afd_ffn_serve_result(win, stream or None, ctypes.byref(st), ctypes.byref(done), ctypes.byref(item)))
    return st.value, done.value, item.value


def afd_slot_unpack_ranks(wins, peer, stage, seq_len, out_ptr, stream=0) -> int:
    arr = (ctypes.c_void_p * len(wins))(*wins)
    return _check(lib().afd_slot_unpack_ranks(arr, len(wins), peer, stage, seq_len, out_ptr or None,
                                              stream or None))


def afd_window_status(win, stage=0, stream=0) -> RunInfo:
    info = RunInfo()
    _check(lib().afd_window_status(win, stage, stream or None, ctypes.byref(info)))
    return info


def afd_peer_status(win, peer, stage=0, stream=0) -> RunInfo:
    info = RunInfo()
    _check(lib().afd_peer_status(win, peer, stage, stream or None, ctypes.byref(info)))
    return info


def afd_window_poll(win, which, n):
    arr = (ctypes.c_int32 * n)()
    _check(lib().afd_window_poll(win, which, arr))
    return list(arr)


def afd_debug_routing(win, stream, max_pairs, num_experts, num_peers):
    import numpy as np
    ids = np.zeros(max_pairs, np.int32)
    wts = np.zeros(max_pairs, np.float32)
    counts = np.zeros(num_experts, np.int32)
    eoff = np.zeros(num_experts + 1, np.int32)
    perm = np.zeros(max_pairs, np.int32)
    inv = np.zeros(max_pairs, np.int32)
    off = np.zeros(num_peers + 1, np.int32)
    p = lambda a: a.ctypes.data_as(ctypes.c_void_p)
    _check(lib().afd_debug_routing(win, stream or None, p(ids), p(wts), p(counts), p(eoff), p(perm), p(inv), p(off)))
    return {"ids": ids, "w": wts, "counts": counts, "expert_offsets": eoff, "perm": perm, "inv": inv, "off": off}


def afd_debug_read(win, offset, nbytes) -> bytes:
    buf = ctypes.create_string_buffer(nbytes)
    _check(lib().afd_debug_read(win, offset, nbytes, buf))
    return buf.raw


def afd_debug_write(win, offset, data: bytes) -> None:
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    _check(lib().afd_debug_write(win, offset, len(data), buf))


def afd_profile_enable(win, mode=1) -> None:
    """mode 0 off, 1 every kernel, 2 the two GEMM kernels only."""
    _check(lib().afd_profile_enable(win, int(mode)))


def afd_profile_read(win, reset=True):
    ms = (ctypes.c_float * AFD_PROFILE_SLOTS)()
    runs = ctypes.c_int32()
    _check(lib().afd_profile_read(win, ms, AFD_PROFILE_SLOTS, ctypes.byref(runs), 1 if reset else 0))
    names = [lib().afd_profile_kernel_name(i).decode() for i in range(AFD_PROFILE_SLOTS)]
    return {n: float(m) for n, m in zip(names, ms) if n != "unused"}, runs.value


def afd_header_encode(fields: dict, counts=None):
    import numpy as np
    f = HeaderFields(**{k: int(v) for k, v in fields.items()})
    out = np.zeros(HDR_WORDS + f.n_counts, np.int32)
    c = None if counts is None else np.ascontiguousarray(counts, np.int32)
    _check(lib().afd_header_encode(ctypes.byref(f), None if c is None else c.ctypes.data_as(ctypes.c_void_p),
                                   out.ctypes.data_as(ctypes.c_void_p)))
    return out


def afd_header_decode(words, expect_counts):
    import numpy as np
    w = np.ascontiguousarray(words, np.int32)
    f = HeaderFields()
    rc = lib().afd_header_decode(w.ctypes.data_as(ctypes.c_void_p), int(w.shape[0]), expect_counts, ctypes.byref(f))
    if rc != AFD_OK:
        return rc, None
    return rc, {n: getattr(f, n) for n, _ in HeaderFields._fields_}


def afd_abi_version() -> int:
    return lib().afd_abi_version()
