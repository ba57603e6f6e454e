"""CPU checks of the C ABI: the library loads, exports every declared symbol,
and its host-only pieces (configuration checks, window layout, header codec)
agree with the reference layout and codec written from "[RFC]: Async GPU
Connector", "Window and slot layout" (oracle/protocol.py).  No device call.
"""
import os
import re

import numpy as np
import pytest

from combine_afd_slot_amd import afd
from oracle import protocol as ref

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_symbols():
    text = open(os.path.join(ROOT, "include", "afd.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(afd_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    L = afd.lib()
    declared = _declared_symbols()
    assert declared, "no declarations parsed"
    missing = [s for s in declared if not hasattr(L, s)]
    assert not missing, missing
    assert sorted(afd.EXPORTS) == declared
    assert afd.afd_abi_version() == 9


CFGS = [
    dict(num_peers=2, token_cap=16, hidden=64, num_experts=8, top_k=2, intermediate=32, shared_intermediate=32),
    dict(num_peers=2, token_cap=4096, hidden=2048, num_experts=64, top_k=6, intermediate=1408,
         shared_intermediate=2816),
    dict(num_peers=4, token_cap=8192, hidden=2048, num_experts=64, top_k=6, intermediate=1408,
         shared_intermediate=2816, ring_depth=2),
    dict(num_peers=2, token_cap=4096, hidden=7168, num_experts=256, top_k=8, intermediate=2048,
         shared_intermediate=2048),
    dict(num_peers=8, token_cap=16, hidden=2048, num_experts=64, top_k=6, intermediate=1408,
         shared_intermediate=2816),
    dict(num_peers=3, token_cap=37, hidden=40, num_experts=5, top_k=5, intermediate=8, shared_intermediate=0),
    dict(num_peers=2, token_cap=16, hidden=64, num_experts=8, top_k=2, intermediate=32, shared_intermediate=32,
         attention_routes=1),
    dict(num_peers=4, token_cap=4096, hidden=2048, num_experts=64, top_k=6, intermediate=1408,
         shared_intermediate=0, attention_routes=1, ring_depth=2),
]


@pytest.mark.parametrize("kw", CFGS)
def test_layout_matches_reference(kw):
    cfg = afd.make_config(**kw)
    L = afd.afd_layout_compute(cfg)
    R = kw.get("ring_depth", 1)
    r = ref.window_layout(kw["num_peers"], R, kw["token_cap"], kw["hidden"], kw["num_experts"],
                          shared=kw["shared_intermediate"] > 0,
                          top_k=kw["top_k"] if kw.get("attention_routes") else 0)
    for i, name in enumerate(ref.FIELDS):
        assert L.field_off[i] == r["field_off"][name], name
        assert L.field_bytes[i] == r["field_bytes"][name], name
    assert L.slot_bytes == r["slot_bytes"]
    assert L.window_bytes == r["window_bytes"]
    assert L.in_slots_off - L.in_off == r["first_slot"]
    assert L.ret_slots_off - L.ret_off == r["first_slot"]
    # both windows share the slot layout; windows and workspace disjoint, aligned
    assert L.in_off == 0 and L.ret_off >= L.window_bytes and L.workspace_off >= L.ret_off + L.window_bytes
    assert L.total_bytes == L.workspace_off + L.workspace_bytes
    for off in (L.in_off, L.in_slots_off, L.ret_off, L.ret_slots_off, L.workspace_off):
        assert off % 256 == 0


@pytest.mark.parametrize("kw", CFGS)
def test_packed_weight_bytes(kw):
    # every weight once, in whole tiles of 256 rows x 32 depth values (16 KB):
    # gate/up tiles of 128 gate + 128 up rows, down tiles of 256 output rows
    cfg = afd.make_config(**kw)
    L = afd.afd_layout_compute(cfg)
    E, H, I, Is = kw["num_experts"], kw["hidden"], kw["intermediate"], kw["shared_intermediate"]
    cdiv = lambda a, b: -(-a // b)
    tiles = (E * cdiv(I, 128) * cdiv(H, 32) + cdiv(Is, 128) * cdiv(H, 32)
             + E * cdiv(H, 256) * cdiv(I, 32) + cdiv(H, 256) * cdiv(Is, 32))
    assert L.packed_weight_bytes == tiles * 16384
    # no padding when the widths are whole tiles
    if I % 128 == 0 and Is % 128 == 0 and H % 256 == 0:
        assert L.packed_weight_bytes == 2 * (E * 3 * I * H + 3 * Is * H)


@pytest.mark.parametrize("kw", CFGS)
def test_slot_fields_disjoint_aligned_viewable(kw):
    L = afd.afd_layout_compute(afd.make_config(**kw))
    itemsize = {"header": 4, "route_table": 4, "routed_x": 2, "shared_idx": 4, "shared_x": 2}
    spans = []
    for i, name in enumerate(afd.FIELDS):
        o, n = L.field_off[i], L.field_bytes[i]
        assert o % 256 == 0
        assert o % itemsize[name] == 0 and n % itemsize[name] == 0
        assert o + n <= L.slot_bytes
        spans.append((o, o + n))
    spans.sort()
    for (a0, a1), (b0, b1) in zip(spans, spans[1:]):
        assert a1 <= b0
    assert L.slot_bytes % 256 == 0


@pytest.mark.parametrize("bad", [
    dict(struct_size=3), dict(reserved=1), dict(num_peers=0), dict(num_peers=65), dict(ring_depth=0),
    dict(ring_depth=5), dict(token_cap=0), dict(hidden=60), dict(num_experts=0), dict(top_k=0),
    dict(top_k=9), dict(intermediate=12), dict(shared_intermediate=-8), dict(renormalize=2),
    dict(poll_timeout_us=0), dict(attention_routes=2), dict(attention_routes=-1),
    dict(route_experts=16), dict(expert_offset=1),
    dict(attention_routes=1, route_experts=1025), dict(attention_routes=1, route_experts=12, expert_offset=5),
    dict(attention_routes=1, route_experts=12, expert_offset=-1),
    dict(w1_fp8=2), dict(w1_fp8=1, hidden=96),
])

def test_config_rejected(bad):
    kw = dict(CFGS[0])
    cfg = afd.make_config(**kw)
    for k, v in bad.items():
        if k == "reserved":
            cfg.reserved[0] = v
        else:
            setattr(cfg, k, v)
    with pytest.raises(afd.AfdError) as ei:
        afd.afd_layout_compute(cfg)
    assert ei.value.code == afd.AFD_ERR_INVALID

def test_segment_config_accepted():
    # a window owning experts [8, 16) of 32 routed over; top_k may exceed its own experts
    cfg = afd.make_config(**dict(CFGS[0], top_k=10, attention_routes=1, route_experts=32, expert_offset=8))
    L = afd.afd_layout_compute(cfg)
    r = ref.window_layout(2, 1, 16, 64, 8, shared=True, top_k=10)
    assert L.slot_bytes == r["slot_bytes"] and L.field_bytes[2] == r["field_bytes"]["routed_x"]


def test_header_codec_round_trip_against_reference():
    E = 8
    counts = np.arange(E, dtype=np.int32) * 3
    f = dict(flags=afd.AFD_FLAG_SHUTDOWN, seq=41, echo_seq=17, layer_idx=5, stage_idx=1, num_tokens=13,
             routed_tokens=13, shared_tokens=13, src_peer=1, n_counts=E)
    words = afd.afd_header_encode(f, counts)
    d = ref.decode_header(words, E)
    assert d["magic"] == ref.MAGIC and d["version"] == ref.VERSION
    assert d["shutdown"] and d["seq"] == 41 and d["echo_seq"] == 17 and d["layer_idx"] == 5
    assert d["stage_idx"] == 1 and d["num_tokens"] == 13 and d["src_peer"] == 1
    assert (d["counts"] == counts).all()
    w2 = ref.encode_header(seq=7, layer_idx=3, stage_idx=0, num_tokens=4, src_peer=2, n_counts=E, counts=counts)
    rc, g = afd.afd_header_decode(w2, E)
    assert rc == afd.AFD_OK and g["seq"] == 7 and g["layer_idx"] == 3 and g["num_tokens"] == 4
    assert g["src_peer"] == 2 and g["flags"] == 0
    assert bytes(words[:1].tobytes()) == b"AFDG"


@pytest.mark.parametrize("word,value", [(0, 0x12345678), (1, 2), (11, 7)])
def test_header_self_check_rejects(word, value):
    w = ref.encode_header(seq=1, layer_idx=0, stage_idx=0, num_tokens=1, src_peer=0, n_counts=8)
    w[word] = value
    rc, _ = afd.afd_header_decode(w, 8)
    assert rc == afd.AFD_ERR_HEADER
    with pytest.raises(ValueError):
        ref.decode_header(w, 8)


def test_status_strings():
    assert afd.status_string(afd.AFD_ERR_TIMEOUT) == "AFD_ERR_TIMEOUT"
    assert afd.status_string(123) == "AFD_UNKNOWN"


@pytest.mark.parametrize("kw", [c for c in CFGS if c["hidden"] % 64 == 0 and not c.get("attention_routes")])
def test_packed_weight_bytes_fp8(kw):
    # e4m3 gate/up tiles (256 rows x 64 depth values of one byte), bf16 down
    # tiles, then one fp32 scale per W13 row and per Ws13 row (256-aligned)
    L = afd.afd_layout_compute(afd.make_config(**kw, w1_fp8=1))
    E, H, I, Is = kw["num_experts"], kw["hidden"], kw["intermediate"], kw["shared_intermediate"]
    cdiv = lambda a, b: -(-a // b)
    a256 = lambda n: cdiv(n, 256) * 256
    tiles = (E * cdiv(I, 128) * (H // 64) + cdiv(Is, 128) * (H // 64)
             + E * cdiv(H, 256) * cdiv(I, 32) + cdiv(H, 256) * cdiv(Is, 32))
    assert L.packed_weight_bytes == tiles * 16384 + a256(4 * E * 2 * I) + a256(4 * 2 * Is)
