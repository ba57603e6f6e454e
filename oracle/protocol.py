"""Reference window layout and header codec (TEST INFRASTRUCTURE ONLY).

Written from "[RFC]: Async GPU Connector" (vllm-project/afd-plugin #233),
section "Window and slot layout": the window is a flag array of
num_regions*ring_depth entries followed by the slots slot(0,0), slot(0,1), ...
(region-major), each slot holding header | route_table | routed_x |
shared_idx | shared_x with every field 256-byte aligned; the header is 12 int32
words followed by expert_counts, carries the magic "AFDG" and a version, and
flags bit 1 is the shutdown sentinel.  Section "Capacity and ring depth" gives
token_cap and ring_depth.

Readings where the page is silent (also listed in the design notes):
  * one FFN replica routes every token, so a slot is sized for token_cap
    tokens in every field: route_table fp32 [token_cap][E] (router logits),
    routed_x bf16 [token_cap][H], shared_idx int32 [token_cap],
    shared_x bf16 [token_cap][H];
  * a window without a shared expert on the FFN side follows the
    routed-only protocol of "[RFC]: Async AFD for Prefill on Ascend NPU",
    section "Shared-expert ownership" (no shared-expert data on the data
    plane): shared_idx and shared_x are 0 bytes and headers carry
    shared_tokens = 0;
  * when the attention side routes (the arrangement of section "Data flow":
    the sender sorts its flattened (token, expert) pairs stably and sends the
    routed rows grouped by expert, the group list in the header's
    expert_counts), no logits travel, so route_table is 0 bytes, and
    routed_x holds token_cap * top_k rows (section "Capacity and ring
    depth": routed_cap = token_cap * topk / ffn_size, with one FFN rank);
    routed_tokens is num_tokens * top_k;
  * flags are int32; the flag array also starts 256-byte aligned (offset 0)
    and the first slot starts at the next 256-byte boundary after it;
  * header word order: magic, version, flags, seq, echo_seq, layer_idx,
    stage_idx, num_tokens, routed_tokens, shared_tokens, src_peer, n_counts,
    then n_counts expert counts; magic is the bytes 'A','F','D','G'.

Used only to check the library's own layout and codec from the outside.
"""
from __future__ import annotations

import numpy as np

ALIGN = 256
HEADER_WORDS = 12
MAGIC = int.from_bytes(b"AFDG", "little")
VERSION = 1
FLAG_SHUTDOWN = 0x2

FIELDS = ("header", "route_table", "routed_x", "shared_idx", "shared_x")
WORD = {name: i for i, name in enumerate(
    ("magic", "version", "flags", "seq", "echo_seq", "layer_idx", "stage_idx", "num_tokens",
     "routed_tokens", "shared_tokens", "src_peer", "n_counts"))}


def align_up(n: int, a: int = ALIGN) -> int:
    return (n + a - 1) // a * a


def slot_fields(token_cap: int, hidden: int, num_experts: int, shared: bool = True,
                top_k: int = 0) -> dict:
    """Byte size of each slot field before alignment (shared=False: routed-only;
    top_k > 0: the attention side routes and sends top_k rows per token)."""
    return {
        "header": 4 * (HEADER_WORDS + num_experts),
        "route_table": 0 if top_k else 4 * token_cap * num_experts,
        "routed_x": 2 * token_cap * (top_k or 1) * hidden,
        "shared_idx": 4 * token_cap if shared else 0,
        "shared_x": 2 * token_cap * hidden if shared else 0,
    }


def window_layout(num_peers: int, ring_depth: int, token_cap: int, hidden: int,
                  num_experts: int, shared: bool = True, top_k: int = 0) -> dict:
    """Offsets of one window (flags, then slots), relative to its start
    (top_k > 0: an attention-routed window)."""
    sizes = slot_fields(token_cap, hidden, num_experts, shared, top_k)
    off, cur = {}, 0
    for name in FIELDS:
        off[name] = cur
        cur += align_up(sizes[name])
    slot_bytes = cur
    n_flags = num_peers * ring_depth
    first_slot = align_up(4 * n_flags)
    return {
        "field_off": off,
        "field_bytes": sizes,
        "slot_bytes": slot_bytes,
        "n_flags": n_flags,
        "first_slot": first_slot,
        "window_bytes": first_slot + n_flags * slot_bytes,
    }


def slot_offset(layout: dict, peer: int, stage: int, ring_depth: int) -> int:
    return layout["first_slot"] + (peer * ring_depth + stage) * layout["slot_bytes"]


def flag_index(peer: int, stage: int, ring_depth: int) -> int:
    return peer * ring_depth + stage


def encode_header(*, seq, layer_idx, stage_idx, num_tokens, src_peer, n_counts,
                  flags=0, echo_seq=0, routed_tokens=None, shared_tokens=None,
                  counts=None) -> np.ndarray:
    w = np.zeros(HEADER_WORDS + n_counts, dtype=np.int32)
    w[WORD["magic"]] = MAGIC
    w[WORD["version"]] = VERSION
    w[WORD["flags"]] = flags
    w[WORD["seq"]] = seq
    w[WORD["echo_seq"]] = echo_seq
    w[WORD["layer_idx"]] = layer_idx
    w[WORD["stage_idx"]] = stage_idx
    w[WORD["num_tokens"]] = num_tokens
    w[WORD["routed_tokens"]] = num_tokens if routed_tokens is None else routed_tokens
    w[WORD["shared_tokens"]] = num_tokens if shared_tokens is None else shared_tokens
    w[WORD["src_peer"]] = src_peer
    w[WORD["n_counts"]] = n_counts
    if counts is not None:
        w[HEADER_WORDS:] = counts
    return w


def decode_header(words, n_counts: int) -> dict:
    """Decode and self-check (magic, version, length); raises ValueError."""
    w = np.asarray(words, dtype=np.int32)
    if w.shape[0] < HEADER_WORDS:
        raise ValueError("header too short")
    if int(w[WORD["magic"]]) != MAGIC:
        raise ValueError("bad magic")
    if int(w[WORD["version"]]) != VERSION:
        raise ValueError("bad version")
    if int(w[WORD["n_counts"]]) != n_counts or w.shape[0] < HEADER_WORDS + n_counts:
        raise ValueError("bad length")
    d = {k: int(w[i]) for k, i in WORD.items()}
    d["shutdown"] = bool(d["flags"] & FLAG_SHUTDOWN)
    d["counts"] = w[HEADER_WORDS:HEADER_WORDS + n_counts].copy()
    return d
