// afd_proto.h -- window protocol pieces shared by host code and kernels:
// the window/slot layout and the header codec.
//
// Layout ("[RFC]: Async GPU Connector", "Window and slot layout"): a window
// is an int32 flag array with one entry per (peer, stage), then the slots in
// (peer, stage) order; a slot is header | route_table | routed_x |
// shared_idx | shared_x with every field 256-byte aligned.  The header is 12
// int32 words followed by per-expert counts, self-checked by a magic and a
// version; flags bit 1 marks shutdown.  Because this FFN replica routes every
// token itself (router logits travel with the hidden states, as with
// compute_gate_on_attention in "NCCL_P2P_CONNECTOR_USER_GUIDE.md",
// Configuration), the route_table field carries fp32 logits and every field
// is sized for token_cap tokens.
#pragma once

#include <stdint.h>

#include "../../include/afd.h"

#if defined(__HIPCC__)
#define AFD_HD __host__ __device__ inline
#else
#define AFD_HD inline
#endif

namespace afd {

constexpr int64_t kAlign = 256;

AFD_HD int64_t align_up(int64_t n, int64_t a = kAlign) { return (n + a - 1) / a * a; }

// Per-slot field sizes (unaligned bytes).  Without a shared expert on the
// FFN side the protocol is routed-only ("[RFC]: Async AFD for Prefill on
// Ascend NPU", "Shared-expert ownership": no shared-expert data crosses the
// data plane), so shared_idx and shared_x take no space.
// When the attention side routes ("[RFC]: Async GPU Connector", "Data flow":
// the sender sorts its (token, expert) pairs and sends the routed rows
// grouped by expert with the group list in the header; "Capacity and ring
// depth": routed_cap = token_cap * topk / ffn_size, here one FFN rank), no
// logits travel and routed_x holds token_cap * top_k rows.
AFD_HD void slot_field_bytes(int64_t token_cap, int64_t hidden, int64_t experts, int64_t top_k, bool shared,
                             bool attn_routes, int64_t out[AFD_NUM_FIELDS]) {
    out[AFD_FIELD_HEADER] = 4 * (AFD_HDR_WORDS + experts);
    out[AFD_FIELD_ROUTE_TABLE] = attn_routes ? 0 : 4 * token_cap * experts;
    out[AFD_FIELD_ROUTED_X] = 2 * token_cap * (attn_routes ? top_k : 1) * hidden;
    out[AFD_FIELD_SHARED_IDX] = shared ? 4 * token_cap : 0;
    out[AFD_FIELD_SHARED_X] = shared ? 2 * token_cap * hidden : 0;
}

// Header: encode into `w` (12 + n_counts words).
// The fixed words of a header (everything but the per-expert counts).
AFD_HD void header_encode_fixed(const afd_header_fields& f, int32_t* w) {
    w[AFD_HDR_MAGIC] = AFD_HDR_MAGIC_VALUE;
    w[AFD_HDR_VERSION] = AFD_HDR_VERSION_VALUE;
    w[AFD_HDR_FLAGS] = f.flags;
    w[AFD_HDR_SEQ] = f.seq;
    w[AFD_HDR_ECHO_SEQ] = f.echo_seq;
    w[AFD_HDR_LAYER] = f.layer_idx;
    w[AFD_HDR_STAGE] = f.stage_idx;
    w[AFD_HDR_NUM_TOKENS] = f.num_tokens;
    w[AFD_HDR_ROUTED_TOKENS] = f.routed_tokens;
    w[AFD_HDR_SHARED_TOKENS] = f.shared_tokens;
    w[AFD_HDR_SRC_PEER] = f.src_peer;
    w[AFD_HDR_N_COUNTS] = f.n_counts;
}

AFD_HD void header_encode(const afd_header_fields& f, const int32_t* counts, int32_t* w) {
    header_encode_fixed(f, w);
    for (int32_t i = 0; i < f.n_counts; ++i) w[AFD_HDR_WORDS + i] = counts ? counts[i] : 0;
}

// Header: decode the 12 fixed words and self-check magic, version and the
// counts length.  Returns AFD_OK or AFD_ERR_HEADER.
AFD_HD int32_t header_decode(const int32_t* w, int32_t expect_counts, afd_header_fields* f) {
    if (w[AFD_HDR_MAGIC] != AFD_HDR_MAGIC_VALUE) return AFD_ERR_HEADER;
    if (w[AFD_HDR_VERSION] != AFD_HDR_VERSION_VALUE) return AFD_ERR_HEADER;
    if (w[AFD_HDR_N_COUNTS] != expect_counts) return AFD_ERR_HEADER;
    f->flags = w[AFD_HDR_FLAGS];
    f->seq = w[AFD_HDR_SEQ];
    f->echo_seq = w[AFD_HDR_ECHO_SEQ];
    f->layer_idx = w[AFD_HDR_LAYER];
    f->stage_idx = w[AFD_HDR_STAGE];
    f->num_tokens = w[AFD_HDR_NUM_TOKENS];
    f->routed_tokens = w[AFD_HDR_ROUTED_TOKENS];
    f->shared_tokens = w[AFD_HDR_SHARED_TOKENS];
    f->src_peer = w[AFD_HDR_SRC_PEER];
    f->n_counts = w[AFD_HDR_N_COUNTS];
    return AFD_OK;
}

// Inbound message checks made by the FFN side on top of header_decode: the
// message must belong to this (peer, stage, layer), fit the slot, carry the
// seq of the flag that announced it, and (one FFN replica) route and share
// every token.
// shared: the window carries shared rows (every token has one); routed-only
// messages carry none (shared_tokens 0).  kmul: routed rows per token (1
// when the FFN routes, top_k when the attention side sends its routed rows).
// segmented: the window owns part of the experts, so a message carries only
// the pairs of those (at most num_tokens * kmul rows).
AFD_HD int32_t inbound_check(const afd_header_fields& f, int32_t peer, int32_t stage, int32_t layer,
                             int32_t token_cap, int32_t flag_seq, bool shared, int32_t kmul, bool segmented) {
    if (f.src_peer != peer || f.stage_idx != stage || f.layer_idx != layer) return AFD_ERR_HEADER;
    if (f.num_tokens < 0 || f.num_tokens > token_cap) return AFD_ERR_HEADER;
    const bool routed_ok = segmented ? f.routed_tokens >= 0 && f.routed_tokens <= f.num_tokens * kmul
                                     : f.routed_tokens == f.num_tokens * kmul;
    if (!routed_ok || f.shared_tokens != (shared ? f.num_tokens : 0)) return AFD_ERR_HEADER;
    if (f.seq != flag_seq) return AFD_ERR_HEADER;
    return AFD_OK;
}

}  // namespace afd
