// afd_host.cpp -- the C ABI of libafd.so (include/afd.h): configuration
// checks, the window layout, the per-(peer, stage) sequence and ring state
// kept by the host, and the launches.  Host-detectable errors return before
// anything is enqueued.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <new>
#include <string>
#include <vector>

#include "afd_internal.h"

namespace {

thread_local std::string g_err = "";

int32_t fail(int32_t code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_err = buf;
    return code;
}

int32_t hip_fail(hipError_t e, const char* what) {
    return fail(AFD_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

const char* kProfileNames[AFD_PROFILE_SLOTS] = {"wait_fanin", "route_topk", "scan_offsets", "permute",
                                                "gemm_gate_up_swiglu", "gemm_down", "combine_split_publish",
                                                "unused"};
constexpr int kProfileUsed = 7;
constexpr int kGemmFirst = 4;  // slots 4 and 5: the two GEMMs

int32_t validate(const afd_window_config* c) {
    if (!c) return fail(AFD_ERR_INVALID, "config is NULL");
    if (c->struct_size != sizeof(afd_window_config))
        return fail(AFD_ERR_INVALID, "struct_size %u != %zu", c->struct_size, sizeof(afd_window_config));
    for (int i = 0; i < 1; ++i)
        if (c->reserved[i] != 0) return fail(AFD_ERR_INVALID, "reserved[%d] must be 0", i);
    if (c->attention_routes != 0 && c->attention_routes != 1)
        return fail(AFD_ERR_INVALID, "attention_routes must be 0 or 1");
    if (c->w1_fp8 != 0 && c->w1_fp8 != 1) return fail(AFD_ERR_INVALID, "w1_fp8 must be 0 or 1");
    if (c->w1_fp8 && c->hidden % 64) return fail(AFD_ERR_INVALID, "w1_fp8 needs hidden a multiple of 64");
    // quantised rows: one per token, or (attention-routed) one per GEMM row
    if (c->w1_fp8 && (int64_t)c->num_peers * c->token_cap * (c->attention_routes ? c->top_k + 1 : 1) * c->hidden >=
                         ((int64_t)1 << 32))
        return fail(AFD_ERR_INVALID, "w1_fp8: the quantised rows must stay below 4 GiB");
    if (c->route_experts != 0) {
        if (!c->attention_routes) return fail(AFD_ERR_INVALID, "route_experts needs attention_routes = 1");
        if (c->route_experts > afd::kMaxExperts) return fail(AFD_ERR_INVALID, "route_experts above 1024");
        if (c->expert_offset < 0 || c->num_experts < 1 ||
            (int64_t)c->expert_offset + c->num_experts > c->route_experts)
            return fail(AFD_ERR_INVALID, "expert range [%d, %d+%d) not inside [0, route_experts %d)",
                        c->expert_offset, c->expert_offset, c->num_experts, c->route_experts);
    } else if (c->expert_offset != 0) {
        return fail(AFD_ERR_INVALID, "expert_offset needs route_experts > 0");
    }
    if (c->num_peers < 1 || c->num_peers > afd::kMaxPeers) return fail(AFD_ERR_INVALID, "num_peers out of [1,64]");
    if (c->ring_depth < 1 || c->ring_depth > 4) return fail(AFD_ERR_INVALID, "ring_depth out of [1,4]");
    if (c->token_cap < 1) return fail(AFD_ERR_INVALID, "token_cap must be >= 1");
    if (c->hidden < 8 || c->hidden % 8) return fail(AFD_ERR_INVALID, "hidden must be a positive multiple of 8");
    if (c->num_experts < 1 || c->num_experts > afd::kMaxExperts)
        return fail(AFD_ERR_INVALID, "num_experts out of [1,1024]");
    const int32_t routed_over = c->route_experts ? c->route_experts : c->num_experts;
    if (c->top_k < 1 || c->top_k > routed_over || c->top_k > afd::kMaxTopK)
        return fail(AFD_ERR_INVALID, "top_k out of [1, min(experts routed over,16)]");
    if (c->intermediate < 8 || c->intermediate % 8)
        return fail(AFD_ERR_INVALID, "intermediate must be a positive multiple of 8");
    if (c->shared_intermediate < 0 || c->shared_intermediate % 8)
        return fail(AFD_ERR_INVALID, "shared_intermediate must be a non-negative multiple of 8");
    if (c->renormalize != 0 && c->renormalize != 1) return fail(AFD_ERR_INVALID, "renormalize must be 0 or 1");
    if (c->poll_timeout_us < 1) return fail(AFD_ERR_INVALID, "poll_timeout_us must be >= 1");
    if (!(c->routed_scaling_factor == c->routed_scaling_factor)) return fail(AFD_ERR_INVALID, "rsf is NaN");
    const int64_t tmax = (int64_t)c->num_peers * c->token_cap;
    if (tmax * c->top_k > (int64_t)1 << 28) return fail(AFD_ERR_INVALID, "num_peers*token_cap*top_k too large");
    // the GEMM kernels address rows with 32-bit byte offsets from a base
    const int64_t lim = (int64_t)1 << 32;
    int64_t fb[AFD_NUM_FIELDS], slot = 0;
    afd::slot_field_bytes(c->token_cap, c->hidden, c->num_experts, c->top_k, c->shared_intermediate > 0,
                          c->attention_routes != 0, fb);
    for (int i = 0; i < AFD_NUM_FIELDS; ++i) slot += afd::align_up(fb[i]);
    const int64_t window = afd::align_up(4LL * c->num_peers * c->ring_depth) + slot * c->num_peers * c->ring_depth;
    if (window >= lim || 2 * tmax * c->top_k * c->intermediate >= lim || 2 * tmax * c->shared_intermediate >= lim ||
        4LL * c->intermediate * c->hidden >= lim || 4LL * c->shared_intermediate * c->hidden >= lim)
        return fail(AFD_ERR_INVALID, "window, activation buffers and per-expert weights must each stay below 4 GiB");
    return AFD_OK;
}

// Workspace carve-up, in bytes from the workspace start.
struct WsLayout {
    int64_t ctrl, peer_counts, blk_counts, blk_base, counts, eoff, tstart1, tstart2;
    int64_t tinfo1, tinfo2, seg1, seg2, tctr, psrc, max_tiles1, max_tiles2;
    int64_t ids, wts, perm, inv, tok_src, sh_src, h, hs, y, ys, ysp, shp, wtable, pid, pwt, ppos, pblk, pbase, pcnt, retoff, retoffs, xq, sx, sxp, bytes;
    int64_t ctrl_ints;
    // control-word offsets inside ctrl (in ints)
    int64_t c_seen_in, c_ret_seq, c_seen_ret, c_cur_seq, c_off, c_T, c_done, c_run_status, c_peer_status;
    int64_t c_layer_cur, c_nlayers, c_rr, c_prow, c_serve;
};

WsLayout ws_layout(const afd_window_config& c) {
    WsLayout w{};
    const int64_t P = c.num_peers, R = c.ring_depth, E = c.num_experts, K = c.top_k;
    const int64_t tmax = P * c.token_cap, np = tmax * K;
    const int64_t nb = (tmax + afd::kRouteChunk - 1) / afd::kRouteChunk + P;
    const int64_t G = E + (c.shared_intermediate > 0 ? 1 : 0);
    // depth parts of the shared expert's down GEMM (small windows only)
    const int64_t nks = (c.shared_intermediate + afd::kBK - 1) / afd::kBK;
    w.shp = c.shared_intermediate > 0 && tmax <= afd::kShSplitRows ? std::min<int64_t>(afd::kShParts, nks) : 1;
    int64_t ci = 0;
    w.c_seen_in = ci; ci += P * R;
    w.c_ret_seq = ci; ci += P * R;
    w.c_seen_ret = ci; ci += P * R;
    w.c_cur_seq = ci; ci += P;
    w.c_off = ci; ci += P + 1;
    w.c_T = ci; ci += 1;
    w.c_done = ci; ci += 1;
    w.c_run_status = ci; ci += R * afd::kStatusWords;
    w.c_peer_status = ci; ci += P * R * afd::kStatusWords;
    w.c_layer_cur = ci; ci += 1;
    w.c_nlayers = ci; ci += 1;
    w.c_rr = ci; ci += R;
    w.c_prow = ci; ci += P;
    w.c_serve = ci; ci += 3;
    w.ctrl_ints = ci;
    int64_t cur = 0;
    auto take = [&](int64_t bytes) {
        const int64_t o = cur;
        cur += afd::align_up(bytes > 0 ? bytes : 1);
        return o;
    };
    w.ctrl = take(4 * ci);
    w.peer_counts = take(4 * P * E);
    w.blk_counts = take(4 * nb * E);
    w.blk_base = take(4 * nb * E);
    w.counts = take(4 * E);
    w.eoff = take(4 * (E + 1));
    w.tstart1 = take(4 * (G + 1));
    w.tstart2 = take(4 * (G + 1));
    {
        // upper bounds of the tile counts: a group of M rows has
        // ceil(ceil(M/32) / kTileBlocks) <= (M + kBX - 1) / kBX row tiles, so
        // the sum over groups is <= (rows + groups*(kBX-1)) / kBX
        const int64_t mt_r = (np + E * (afd::kBX - 1)) / afd::kBX;
        const int64_t mt_s = c.shared_intermediate > 0 ? (tmax + afd::kBX - 1) / afd::kBX : 0;
        const int64_t nt1_r = (c.intermediate + afd::kBW / 2 - 1) / (afd::kBW / 2);
        const int64_t nt1_s = (c.shared_intermediate + afd::kBW / 2 - 1) / (afd::kBW / 2);
        const int64_t nt2 = (c.hidden + afd::kBW - 1) / afd::kBW;
        w.max_tiles1 = mt_r * nt1_r + mt_s * nt1_s;
        w.max_tiles2 = (mt_r + mt_s * w.shp) * nt2;
    }
    w.tinfo1 = take(16 * w.max_tiles1);
    w.tinfo2 = take(16 * w.max_tiles2);
    w.seg1 = take(4 * (afd::kSegs + 1));
    w.seg2 = take(4 * (afd::kSegs + 1));
    w.tctr = take(4 * 2 * afd::kSegs);
    w.psrc = take(8 * np);
    w.ids = take(4 * np);
    w.wts = take(4 * np);
    w.perm = take(4 * np);
    w.inv = take(4 * np);
    w.tok_src = take(8 * tmax);
    w.sh_src = take(8 * tmax);
    // h and hs depth-block major: ceil(I/32) blocks of rows x 64 bytes
    w.h = take(64 * np * ((c.intermediate + afd::kBK - 1) / afd::kBK));
    w.hs = take(64 * tmax * (c.shared_intermediate > 0 ? (c.shared_intermediate + afd::kBK - 1) / afd::kBK : 1));
    w.y = take(2 * np * c.hidden);
    w.ys = take(2 * tmax * c.hidden);
    w.ysp = take(w.shp > 1 ? 4 * w.shp * tmax * c.hidden : 0);
    w.wtable = take((int64_t)sizeof(afd::Weights) * afd::kMaxLayers);
    {
        // attention-side routing: per (peer, stage) message state on the peer side
        const int64_t ar = c.attention_routes ? 1 : 0;
        const int64_t msgs = P * R, pairs = (int64_t)c.token_cap * K;
        const int64_t nbp = (c.token_cap + afd::kRouteChunk - 1) / afd::kRouteChunk;
        w.pid = take(ar * 4 * msgs * pairs);
        w.pwt = take(ar * 4 * msgs * pairs);
        w.ppos = take(ar * 4 * msgs * pairs);
        w.pblk = take(ar * 4 * msgs * E * nbp);
        w.pbase = take(ar * 4 * msgs * E * nbp);
        w.pcnt = take(ar * 4 * msgs * E);
        w.retoff = take(ar * 4 * np);
        w.retoffs = take(ar * 4 * tmax);
    }
    {
        // fp8 W1: quantised token rows and their scales
        const int64_t q = c.w1_fp8 ? 1 : 0;
        w.xq = take(q * (c.attention_routes ? np + tmax : tmax) * c.hidden);
        w.sx = take(q * 4 * tmax);
        w.sxp = take(q * 4 * (np + tmax));
    }
    w.bytes = cur;
    return w;
}

void layout_from(const afd_window_config& c, afd_layout* L, WsLayout* wl) {
    std::memset(L, 0, sizeof *L);
    int64_t fb[AFD_NUM_FIELDS];
    afd::slot_field_bytes(c.token_cap, c.hidden, c.num_experts, c.top_k, c.shared_intermediate > 0,
                          c.attention_routes != 0, fb);
    int64_t cur = 0;
    for (int i = 0; i < AFD_NUM_FIELDS; ++i) {
        L->field_off[i] = cur;
        L->field_bytes[i] = fb[i];
        cur += afd::align_up(fb[i]);
    }
    L->slot_bytes = cur;
    const int64_t nflags = (int64_t)c.num_peers * c.ring_depth;
    const int64_t first_slot = afd::align_up(4 * nflags);
    L->window_bytes = first_slot + nflags * L->slot_bytes;
    L->in_off = 0;
    L->in_slots_off = first_slot;
    L->ret_off = afd::align_up(L->window_bytes);
    L->ret_slots_off = L->ret_off + first_slot;
    const WsLayout w = ws_layout(c);
    L->workspace_off = L->ret_off + afd::align_up(L->window_bytes);
    L->workspace_bytes = w.bytes;
    L->total_bytes = L->workspace_off + w.bytes;
    int64_t off[6];
    afd::packed_weight_layout(c, off, &L->packed_weight_bytes);
    if (wl) *wl = w;
}

}  // namespace

namespace afd {
void packed_weight_layout(const afd_window_config& c, int64_t off[6], int64_t* total) {
    const int64_t E = c.num_experts, H = c.hidden, I = c.intermediate, Is = c.shared_intermediate;
    // (fp8 W1: a gate/up tile row holds 64 depth values of one byte)
    const int64_t nk1 = c.w1_fp8 ? H / 64 : (H + kBK - 1) / kBK, nt2 = (H + kBW - 1) / kBW;
    const int64_t nt1 = (I + kBW / 2 - 1) / (kBW / 2), nk2 = (I + kBK - 1) / kBK;
    const int64_t nt1s = (Is + kBW / 2 - 1) / (kBW / 2), nk2s = (Is + kBK - 1) / kBK;
    int64_t cur = 0;
    off[0] = cur;  // w13
    cur += E * nt1 * nk1 * kWTileBytes;
    off[1] = cur;  // ws13
    cur += nt1s * nk1 * kWTileBytes;
    off[2] = cur;  // w2
    cur += E * nt2 * nk2 * kWTileBytes;
    off[3] = cur;  // ws2
    cur += nt2 * nk2s * kWTileBytes;
    off[4] = cur;  // sw13 (fp8 W1 only)
    cur += c.w1_fp8 ? align_up(4 * E * 2 * I) : 0;
    off[5] = cur;  // sws13
    cur += c.w1_fp8 ? align_up(4 * 2 * Is) : 0;
    *total = cur;
}
}  // namespace afd

struct afd_window {
    afd_window_config cfg;
    afd_layout lay;
    WsLayout wl;
    int device = 0;
    int num_cu = 0;
    long long ticks_per_us = 100;
    char* base = nullptr;
    afd::DevCtx ctx{};
    // per (peer, stage) = p * ring_depth + s; fixed arrays, so that a window
    // needs no host allocation beyond its handle
    int32_t pack_seq[afd::kMaxPeers * afd::kMaxRing] = {};    // last seq sent by the peer (host side of the peer)
    int32_t packed_len[afd::kMaxPeers * afd::kMaxRing] = {};
    uint8_t inflight[afd::kMaxPeers * afd::kMaxRing] = {};
    bool is_static = false;  // placed in the library's static device array (afd_window_create_static)
    bool poison = false;     // AFD_POISON=1 at creation: slots filled with NaN before each pack / reply
    int profile = 0;  // 0 off, 1 every kernel, 2 the two GEMMs, 3 the gate/up GEMM
    hipEvent_t ev[AFD_PROFILE_SLOTS + 1] = {};
    bool ev_pending = false;
    double prof_ms[AFD_PROFILE_SLOTS] = {};
    int prof_runs = 0;
    std::mutex prof_mu;
    int n_layers = 0;  // entries of the device layer table
};

// A captured sequence of layer-table runs (afd_ffn_loop_create).
struct afd_ffn_loop {
    afd_window* w = nullptr;
    hipGraph_t graph = nullptr;
    hipGraphExec_t exec = nullptr;
    int n_runs = 0;
};

namespace {

void fill_ctx(afd_window* w) {
    const afd_window_config& c = w->cfg;
    const WsLayout& L = w->wl;
    afd::DevCtx& d = w->ctx;
    d.P = c.num_peers;
    d.R = c.ring_depth;
    d.token_cap = c.token_cap;
    d.H = c.hidden;
    d.E = c.num_experts;
    d.K = c.top_k;
    d.I = c.intermediate;
    d.Is = c.shared_intermediate;
    d.renorm = c.renormalize;
    d.rsf = c.routed_scaling_factor;
    d.has_shared = c.shared_intermediate > 0 ? 1 : 0;
    d.G = c.num_experts + d.has_shared;
    const int64_t tmax = (int64_t)c.num_peers * c.token_cap;
    d.NB = (int)((tmax + afd::kRouteChunk - 1) / afd::kRouteChunk) + c.num_peers;  // peer-aligned chunks
    d.max_tiles1 = (int)L.max_tiles1;
    d.max_tiles2 = (int)L.max_tiles2;
    d.hrows = (int)(tmax * c.top_k);
    d.hsrows = (int)tmax;
    d.nt1 = (c.intermediate + afd::kBW / 2 - 1) / (afd::kBW / 2);
    d.nt2 = (c.hidden + afd::kBW - 1) / afd::kBW;
    d.slot_bytes = w->lay.slot_bytes;
    for (int i = 0; i < AFD_NUM_FIELDS; ++i) d.foff[i] = w->lay.field_off[i];
    d.in_win = w->base + w->lay.in_off;
    d.ret_win = w->base + w->lay.ret_off;
    d.slots_off = w->lay.in_slots_off - w->lay.in_off;
    char* ws = w->base + w->lay.workspace_off;
    int* ctrl = (int*)(ws + L.ctrl);
    d.seen_in = ctrl + L.c_seen_in;
    d.ret_seq = ctrl + L.c_ret_seq;
    d.seen_ret = ctrl + L.c_seen_ret;
    d.cur_seq = ctrl + L.c_cur_seq;
    d.off = ctrl + L.c_off;
    d.Tptr = ctrl + L.c_T;
    d.run_status = ctrl + L.c_run_status;
    d.layer_cur = ctrl + L.c_layer_cur;
    d.nlayers = ctrl + L.c_nlayers;
    d.rr = ctrl + L.c_rr;
    d.prow = ctrl + L.c_prow;
    d.serve = ctrl + L.c_serve;
    d.route_done = ctrl + L.c_done;
    d.poison = w->poison ? 1 : 0;
    d.attn_routes = c.attention_routes;
    d.Eg = c.route_experts ? c.route_experts : c.num_experts;
    d.w1_fp8 = c.w1_fp8;
    d.xq = (uint8_t*)(ws + L.xq);
    d.sx = (float*)(ws + L.sx);
    d.sxp = (float*)(ws + L.sxp);
    d.e0 = c.expert_offset;
    d.NBp = (c.token_cap + afd::kRouteChunk - 1) / afd::kRouteChunk;
    d.pid = (int*)(ws + L.pid);
    d.pwt = (float*)(ws + L.pwt);
    d.ppos = (int*)(ws + L.ppos);
    d.pblk = (int*)(ws + L.pblk);
    d.pbase = (int*)(ws + L.pbase);
    d.pcnt = (int*)(ws + L.pcnt);
    d.retoff = (uint32_t*)(ws + L.retoff);
    d.retoffs = (uint32_t*)(ws + L.retoffs);
    d.ret_bytes = (uint32_t)w->lay.window_bytes;  // (below 4 GiB: checked by validate)
    d.direct_ret = c.attention_routes && w->lay.window_bytes < ((int64_t)1 << 30);
    d.wtable = (const afd::Weights*)(ws + L.wtable);
    d.peer_status = ctrl + L.c_peer_status;
    d.peer_counts = (int*)(ws + L.peer_counts);
    d.blk_counts = (int*)(ws + L.blk_counts);
    d.blk_base = (int*)(ws + L.blk_base);
    d.counts = (int*)(ws + L.counts);
    d.eoff = (int*)(ws + L.eoff);
    d.tstart1 = (int*)(ws + L.tstart1);
    d.tstart2 = (int*)(ws + L.tstart2);
    d.tinfo1 = (int4*)(ws + L.tinfo1);
    d.tinfo2 = (int4*)(ws + L.tinfo2);
    d.seg1 = (int*)(ws + L.seg1);
    d.seg2 = (int*)(ws + L.seg2);
    d.tctr = (int*)(ws + L.tctr);
    d.psrc = (uint64_t*)(ws + L.psrc);
    d.ids = (int*)(ws + L.ids);
    d.wts = (float*)(ws + L.wts);
    d.perm = (int*)(ws + L.perm);
    d.inv = (int*)(ws + L.inv);
    d.tok_src = (uint64_t*)(ws + L.tok_src);
    d.sh_src = (uint64_t*)(ws + L.sh_src);
    d.h = (uint16_t*)(ws + L.h);
    d.hs = (uint16_t*)(ws + L.hs);
    d.y = (uint16_t*)(ws + L.y);
    d.ys = (uint16_t*)(ws + L.ys);
    d.ncu = w->num_cu;
    d.shp = (int)L.shp;
    d.ysp = (float*)(ws + L.ysp);
}

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Fold the previous run's events into the accumulated times.
void prof_collect(afd_window* w) {
    if (!w->ev_pending) return;
    const int lo = w->profile == 1 ? 0 : kGemmFirst;
    const int hi = w->profile == 1 ? kProfileUsed : w->profile == 2 ? kGemmFirst + 2 : kGemmFirst + 1;
    for (int i = lo; i <= hi; ++i) (void)hipEventSynchronize(w->ev[i]);
    for (int i = lo; i < hi; ++i) {
        float ms = 0.f;
        if (hipEventElapsedTime(&ms, w->ev[i], w->ev[i + 1]) == hipSuccess) w->prof_ms[i] += ms;
    }
    w->prof_runs += 1;
    w->ev_pending = false;
}

// The events a run records for the current profile mode (nullptr: none).
hipEvent_t* profile_events(afd_window* w, hipEvent_t (&evs)[AFD_PROFILE_SLOTS + 1]) {
    if (!w->profile) return nullptr;
    std::lock_guard<std::mutex> g(w->prof_mu);
    prof_collect(w);
    for (int i = 0; i <= kProfileUsed; ++i)
        if (w->profile == 1 || (i >= kGemmFirst && i <= kGemmFirst + (w->profile == 2 ? 2 : 1))) evs[i] = w->ev[i];
    w->ev_pending = true;
    return evs;
}

long long poll_ticks(const afd_window* w) { return (long long)w->cfg.poll_timeout_us * w->ticks_per_us; }

// The four packed regions of one layer's weights (afd_weights_pack layout).
afd::Weights packed_weights_of(const afd_window_config& c, const void* packed) {
    int64_t off[6], total = 0;
    afd::packed_weight_layout(c, off, &total);
    const char* pw = (const char*)packed;
    const bool sh = c.shared_intermediate > 0;
    return afd::Weights{pw + off[0], pw + off[2], sh ? pw + off[1] : nullptr, sh ? pw + off[3] : nullptr,
                        c.w1_fp8 ? (const float*)(pw + off[4]) : nullptr,
                        c.w1_fp8 && sh ? (const float*)(pw + off[5]) : nullptr};
}

}  // namespace

namespace {

// Device properties, the layout and the zeroed control words of a window
// whose memory (lay.total_bytes at base) is in place.
int32_t window_init(afd_window* w, const afd_window_config* cfg, char* base, hipStream_t zero_stream) {
    const afd_layout& L = w->lay;
    (void)hipDeviceGetAttribute(&w->num_cu, hipDeviceAttributeMultiprocessorCount, w->device);
    if (w->num_cu < 1) w->num_cu = 1;
    int khz = 0;
    if (hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, w->device) == hipSuccess && khz > 0)
        w->ticks_per_us = khz / 1000 > 0 ? khz / 1000 : 1;
    w->base = base;
    const char* pz = getenv("AFD_POISON");
    w->poison = pz && pz[0] == '1';
    // Flags, mirrors and status words start at zero; the slots are left as
    // they are (a slot is only read after its flag announces it).  A fill
    // kernel, not a memset, so that no memset node is ever recorded.
    hipError_t e = afd::launch_zero(base + L.in_off, L.in_slots_off - L.in_off, zero_stream);
    if (e == hipSuccess) e = afd::launch_zero(base + L.ret_off, L.ret_slots_off - L.ret_off, zero_stream);
    if (e == hipSuccess)
        e = afd::launch_zero(base + L.workspace_off + w->wl.ctrl, 4 * w->wl.ctrl_ints, zero_stream);
    if (e == hipSuccess) e = hipStreamSynchronize(zero_stream);
    if (e != hipSuccess) return hip_fail(e, "window init");
    fill_ctx(w);
    const char* lg = getenv("AFD_LOG");
    if (lg && lg[0] == '1')
        fprintf(stderr, "[afd] window%s: P=%d R=%d token_cap=%d slot=%lld B window=%lld B workspace=%lld B total=%lld B\n",
                w->is_static ? " (static)" : "", cfg->num_peers, cfg->ring_depth, cfg->token_cap,
                (long long)L.slot_bytes, (long long)L.window_bytes, (long long)L.workspace_bytes,
                (long long)L.total_bytes);
    return AFD_OK;
}

// ---------------------------------------------------------------------------
// The allocation-free window (afd_window_create_static).  One static device
// array per GPU the library runs on, held until the process ends; in host
// code `scratch` names a host-side stand-in, so its device address is looked
// up once per device (with that device current) and only that address is
// used: kernel arguments and fills take g_scratch[d].
constexpr int kMaxDevices = 64;
static __device__ __align__(256) char scratch[AFD_STATIC_WINDOW_BYTES];
std::mutex g_static_mu;
char* g_scratch[kMaxDevices] = {};                 // device address of `scratch`, per device
bool g_static_busy[kMaxDevices] = {};              // a static window of that device is open
alignas(afd_window) unsigned char g_static_handle[kMaxDevices][sizeof(afd_window)];

}  // namespace

extern "C" {

int32_t afd_abi_version(void) { return AFD_ABI_VERSION; }

const char* afd_last_error(void) { return g_err.c_str(); }

const char* afd_status_string(int32_t s) {
    switch (s) {
        case AFD_OK: return "AFD_OK";
        case AFD_SHUTDOWN: return "AFD_SHUTDOWN";
        case AFD_ERR_INVALID: return "AFD_ERR_INVALID";
        case AFD_ERR_CAPACITY: return "AFD_ERR_CAPACITY";
        case AFD_ERR_SHAPE: return "AFD_ERR_SHAPE";
        case AFD_ERR_RING: return "AFD_ERR_RING";
        case AFD_ERR_TIMEOUT: return "AFD_ERR_TIMEOUT";
        case AFD_ERR_HEADER: return "AFD_ERR_HEADER";
        case AFD_ERR_SEQ: return "AFD_ERR_SEQ";
        case AFD_ERR_DEVICE: return "AFD_ERR_DEVICE";
        default: return "AFD_UNKNOWN";
    }
}

int32_t afd_layout_compute(const afd_window_config* cfg, afd_layout* out) {
    const int32_t rc = validate(cfg);
    if (rc) return rc;
    if (!out) return fail(AFD_ERR_INVALID, "out is NULL");
    layout_from(*cfg, out, nullptr);
    return AFD_OK;
}

int32_t afd_header_encode(const afd_header_fields* f, const int32_t* counts, int32_t* words_out) {
    if (!f || !words_out || f->n_counts < 0) return fail(AFD_ERR_INVALID, "bad header arguments");
    afd::header_encode(*f, counts, words_out);
    return AFD_OK;
}

int32_t afd_header_decode(const int32_t* words, int32_t nwords, int32_t expect_counts, afd_header_fields* out) {
    if (!words || !out || nwords < AFD_HDR_WORDS) return fail(AFD_ERR_INVALID, "bad header arguments");
    if (nwords < AFD_HDR_WORDS + expect_counts) return fail(AFD_ERR_HEADER, "header shorter than its counts");
    const int32_t rc = afd::header_decode(words, expect_counts, out);
    if (rc) return fail(rc, "header failed its magic/version/length check");
    return AFD_OK;
}


int32_t afd_window_create(const afd_window_config* cfg, afd_window** out) {
    if (!out) return fail(AFD_ERR_INVALID, "out is NULL");
    *out = nullptr;
    int32_t rc = validate(cfg);
    if (rc) return rc;
    afd_window* w = new (std::nothrow) afd_window();
    if (!w) return fail(AFD_ERR_INVALID, "out of host memory");
    w->cfg = *cfg;
    layout_from(*cfg, &w->lay, &w->wl);
    hipError_t e = hipGetDevice(&w->device);
    if (e != hipSuccess) {
        delete w;
        return hip_fail(e, "hipGetDevice");
    }
    char* base = nullptr;
    e = hipMalloc((void**)&base, (size_t)w->lay.total_bytes);
    if (e != hipSuccess) {
        delete w;
        return hip_fail(e, "hipMalloc(window)");
    }
    rc = window_init(w, cfg, base, nullptr);
    if (rc) {
        (void)hipFree(base);
        delete w;
        return rc;
    }
    for (int i = 0; i <= AFD_PROFILE_SLOTS; ++i) (void)hipEventCreate(&w->ev[i]);
    *out = w;
    return AFD_OK;
}

int32_t afd_window_create_static(const afd_window_config* cfg, afd_window** out) {
    if (!out) return fail(AFD_ERR_INVALID, "out is NULL");
    *out = nullptr;
    int32_t rc = validate(cfg);
    if (rc) return rc;
    afd_layout lay;
    WsLayout wl;
    layout_from(*cfg, &lay, &wl);
    if (lay.total_bytes > (int64_t)AFD_STATIC_WINDOW_BYTES)
        return fail(AFD_ERR_CAPACITY, "window needs %lld bytes, more than the %lld of the static window",
                    (long long)lay.total_bytes, (long long)AFD_STATIC_WINDOW_BYTES);
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices) return fail(AFD_ERR_INVALID, "device %d out of range", dev);
    std::lock_guard<std::mutex> g(g_static_mu);
    if (g_static_busy[dev])
        return fail(AFD_ERR_INVALID, "the static window of device %d is open: destroy it first", dev);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
        g_scratch[dev] = (char*)p;
    }
    afd_window* w = new (g_static_handle[dev]) afd_window();
    w->cfg = *cfg;
    w->lay = lay;
    w->wl = wl;
    w->device = dev;
    w->is_static = true;
    rc = window_init(w, cfg, g_scratch[dev], nullptr);
    if (rc) {
        w->~afd_window();
        return rc;
    }
    g_static_busy[dev] = true;
    *out = w;
    return AFD_OK;
}

int32_t afd_window_destroy(afd_window* w) {
    if (!w) return AFD_OK;
    int32_t rc = AFD_OK;
    if (w->base) {
        hipError_t e = hipDeviceSynchronize();
        if (e != hipSuccess) rc = hip_fail(e, "hipDeviceSynchronize");
        if (!w->is_static) (void)hipFree(w->base);
    }
    for (int i = 0; i <= AFD_PROFILE_SLOTS; ++i)
        if (w->ev[i]) (void)hipEventDestroy(w->ev[i]);
    if (w->is_static) {
        std::lock_guard<std::mutex> g(g_static_mu);
        const int dev = w->device;
        w->~afd_window();
        g_static_busy[dev] = false;
    } else {
        delete w;
    }
    return rc;
}

int32_t afd_window_layout(const afd_window* w, afd_layout* out) {
    if (!w || !out) return fail(AFD_ERR_INVALID, "NULL argument");
    *out = w->lay;
    return AFD_OK;
}

int32_t afd_slot_pack(afd_window* w, int32_t peer, int32_t stage, int32_t layer_idx, int32_t seq_len,
                      const void* hidden, const float* logits, uint32_t flags, void* peer_stream) {
    if (!w) return fail(AFD_ERR_INVALID, "window is NULL");
    const afd_window_config& c = w->cfg;
    if (peer < 0 || peer >= c.num_peers) return fail(AFD_ERR_INVALID, "peer %d out of range", peer);
    if (stage < 0 || stage >= c.ring_depth) return fail(AFD_ERR_INVALID, "stage %d out of range", stage);
    if (seq_len < 0) return fail(AFD_ERR_INVALID, "seq_len < 0");
    if (seq_len > c.token_cap)
        return fail(AFD_ERR_CAPACITY, "seq_len %d exceeds token_cap %d", seq_len, c.token_cap);
    if (flags & ~AFD_FLAG_SHUTDOWN) return fail(AFD_ERR_INVALID, "unknown flag bits 0x%x", flags);
    if (seq_len > 0 && (!hidden || !logits)) return fail(AFD_ERR_INVALID, "hidden/logits NULL");
    if (seq_len > 0 && (!aligned(hidden, 16) || !aligned(logits, 4)))
        return fail(AFD_ERR_INVALID, "hidden must be 16-byte aligned, logits 4-byte aligned");
    const int idx = peer * c.ring_depth + stage;
    if (w->inflight[idx])
        return fail(AFD_ERR_RING, "(peer %d, stage %d) still in flight: unpack it before packing again", peer, stage);
    const int seq = w->pack_seq[idx] + 1;
    hipError_t e = afd::launch_pack(w->ctx, peer, stage, layer_idx, seq_len, hidden, logits, flags, seq,
                                    (hipStream_t)peer_stream);
    if (e != hipSuccess) return hip_fail(e, "pack launch");
    w->pack_seq[idx] = seq;
    w->packed_len[idx] = seq_len;
    // a shutdown message gets no reply; an empty one neither
    w->inflight[idx] = (seq_len > 0 && !(flags & AFD_FLAG_SHUTDOWN)) ? 1 : 0;
    return AFD_OK;
}

int32_t afd_weights_pack(afd_window* w, const afd_moe_weights* src, void* dst, int64_t dst_bytes, void* stream) {
    if (!w || !src || !dst) return fail(AFD_ERR_INVALID, "NULL argument");
    const afd_window_config& c = w->cfg;
    if (!src->w13 || !src->w2) return fail(AFD_ERR_INVALID, "routed weights are NULL");
    if (c.shared_intermediate > 0 && (!src->ws13 || !src->ws2))
        return fail(AFD_ERR_INVALID, "shared weights are NULL");
    if (!aligned(src->w13, 16) || !aligned(src->w2, 16) ||
        (c.shared_intermediate > 0 && (!aligned(src->ws13, 16) || !aligned(src->ws2, 16))))
        return fail(AFD_ERR_INVALID, "weights must be 16-byte aligned");
    if (!aligned(dst, 256)) return fail(AFD_ERR_INVALID, "packed weights must be 256-byte aligned");
    int64_t off[6], total = 0;
    afd::packed_weight_layout(c, off, &total);
    if (dst_bytes < total)
        return fail(AFD_ERR_INVALID, "packed weights need %lld bytes, got %lld", (long long)total, (long long)dst_bytes);
    hipError_t e = afd::launch_pack_weights(w->ctx, *src, (char*)dst, off, total, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "weight pack launch");
    return AFD_OK;
}

int32_t afd_ffn_run(afd_window* w, int32_t stage, int32_t layer_idx, const void* packed_weights,
                    void* ffn_stream) {
    if (!w || !packed_weights) return fail(AFD_ERR_INVALID, "NULL argument");
    const afd_window_config& c = w->cfg;
    if (stage < 0 || stage >= c.ring_depth) return fail(AFD_ERR_INVALID, "stage %d out of range", stage);
    if (!aligned(packed_weights, 256)) return fail(AFD_ERR_INVALID, "packed weights must be 256-byte aligned");
    const afd::Weights wt = packed_weights_of(c, packed_weights);
    hipEvent_t evs[AFD_PROFILE_SLOTS + 1] = {};
    hipError_t e = afd::launch_ffn(w->ctx, stage, layer_idx, wt, poll_ticks(w), w->num_cu, profile_events(w, evs),
                                   (hipStream_t)ffn_stream);
    if (e != hipSuccess) return hip_fail(e, "ffn launch");
    return AFD_OK;
}

int32_t afd_layer_table_set(afd_window* w, int32_t n_layers, const void* const* packed_weights, void* stream) {
    if (!w || !packed_weights) return fail(AFD_ERR_INVALID, "NULL argument");
    if (n_layers < 1 || n_layers > afd::kMaxLayers)
        return fail(AFD_ERR_INVALID, "n_layers %d outside 1..%d", n_layers, afd::kMaxLayers);
    std::vector<afd::Weights> tab((size_t)n_layers);
    for (int i = 0; i < n_layers; ++i) {
        if (!packed_weights[i] || !aligned(packed_weights[i], 256))
            return fail(AFD_ERR_INVALID, "layer %d: packed weights NULL or not 256-byte aligned", i);
        tab[(size_t)i] = packed_weights_of(w->cfg, packed_weights[i]);
    }
    hipStream_t st = (hipStream_t)stream;
    const int32_t n = n_layers;
    hipError_t e = hipMemcpyAsync((void*)w->ctx.wtable, tab.data(), tab.size() * sizeof(afd::Weights),
                                  hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipMemcpyAsync(w->ctx.nlayers, &n, sizeof n, hipMemcpyHostToDevice, st);
    if (e == hipSuccess) e = hipStreamSynchronize(st);  // the host copies are temporaries
    if (e != hipSuccess) return hip_fail(e, "layer table copy");
    w->n_layers = n_layers;
    return AFD_OK;
}

int32_t afd_ffn_run_ready(afd_window* w, int32_t stage, int32_t layer_idx, const void* packed_weights,
                          int32_t max_peers, int32_t gather_us, void* ffn_stream) {
    if (!w) return fail(AFD_ERR_INVALID, "window is NULL");
    const afd_window_config& c = w->cfg;
    if (stage < 0 || stage >= c.ring_depth) return fail(AFD_ERR_INVALID, "stage %d out of range", stage);
    if (max_peers < 1 || max_peers > c.num_peers)
        return fail(AFD_ERR_INVALID, "max_peers %d outside 1..%d", max_peers, c.num_peers);
    if (gather_us < 0 || gather_us > c.poll_timeout_us)
        return fail(AFD_ERR_INVALID, "gather_us %d outside 0..poll_timeout_us", gather_us);
    afd::Weights wt{};
    if (layer_idx < 0) {
        if (w->n_layers < 1) return fail(AFD_ERR_INVALID, "no layer table set (afd_layer_table_set)");
    } else {
        if (!packed_weights || !aligned(packed_weights, 256))
            return fail(AFD_ERR_INVALID, "packed weights NULL or not 256-byte aligned");
        wt = packed_weights_of(c, packed_weights);
    }
    hipEvent_t evs[AFD_PROFILE_SLOTS + 1] = {};
    hipError_t e = afd::launch_ffn(w->ctx, stage, layer_idx, wt, poll_ticks(w), w->num_cu, profile_events(w, evs),
                                   (hipStream_t)ffn_stream, max_peers, (long long)gather_us * w->ticks_per_us);
    if (e != hipSuccess) return hip_fail(e, "ffn launch");
    return AFD_OK;
}

int32_t afd_ffn_run_table(afd_window* w, int32_t stage, void* ffn_stream) {
    if (!w) return fail(AFD_ERR_INVALID, "window is NULL");
    if (stage < 0 || stage >= w->cfg.ring_depth) return fail(AFD_ERR_INVALID, "stage %d out of range", stage);
    if (w->n_layers < 1) return fail(AFD_ERR_INVALID, "no layer table set (afd_layer_table_set)");
    hipEvent_t evs[AFD_PROFILE_SLOTS + 1] = {};
    hipError_t e = afd::launch_ffn(w->ctx, stage, -1, afd::Weights{}, poll_ticks(w), w->num_cu,
                                   profile_events(w, evs), (hipStream_t)ffn_stream);
    if (e != hipSuccess) return hip_fail(e, "ffn launch");
    return AFD_OK;
}

int32_t afd_ffn_loop_create(afd_window* w, int32_t n_runs, int32_t first_stage, void* stream, afd_ffn_loop** out) {
    if (!w || !out) return fail(AFD_ERR_INVALID, "NULL argument");
    *out = nullptr;
    const afd_window_config& c = w->cfg;
    if (n_runs < 1) return fail(AFD_ERR_INVALID, "n_runs %d < 1", n_runs);
    if (first_stage < 0 || first_stage >= c.ring_depth)
        return fail(AFD_ERR_INVALID, "first_stage %d out of range", first_stage);
    if (w->n_layers < 1) return fail(AFD_ERR_INVALID, "no layer table set (afd_layer_table_set)");
    if (w->profile) return fail(AFD_ERR_INVALID, "per-kernel profiling must be off while capturing");
    if (!stream) return fail(AFD_ERR_INVALID, "capture needs a created stream, not the null stream");
    hipStream_t st = (hipStream_t)stream;
    hipError_t e = hipStreamBeginCapture(st, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail(e, "begin capture");
    for (int i = 0; i < n_runs && e == hipSuccess; ++i)
        e = afd::launch_ffn(w->ctx, (first_stage + i) % c.ring_depth, -1, afd::Weights{}, poll_ticks(w), w->num_cu,
                            nullptr, st);
    hipGraph_t g = nullptr;
    const hipError_t e2 = hipStreamEndCapture(st, &g);
    if (e == hipSuccess) e = e2;
    hipGraphExec_t x = nullptr;
    if (e == hipSuccess) e = hipGraphInstantiate(&x, g, nullptr, nullptr, 0);
    if (e != hipSuccess) {
        if (g) (void)hipGraphDestroy(g);
        return hip_fail(e, "capture of the FFN loop");
    }
    afd_ffn_loop* l = new (std::nothrow) afd_ffn_loop;
    if (!l) {
        (void)hipGraphExecDestroy(x);
        (void)hipGraphDestroy(g);
        return fail(AFD_ERR_DEVICE, "out of host memory");
    }
    l->w = w;
    l->graph = g;
    l->exec = x;
    l->n_runs = n_runs;
    *out = l;
    return AFD_OK;
}

int32_t afd_ffn_loop_launch(afd_ffn_loop* l, void* stream) {
    if (!l) return fail(AFD_ERR_INVALID, "loop is NULL");
    hipError_t e = hipGraphLaunch(l->exec, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "loop launch");
    return AFD_OK;
}

int32_t afd_ffn_serve(afd_window* w, int32_t first_stage, int32_t n_items, int32_t max_peers, int32_t gather_us,
                      void* stream) {
    if (!w) return fail(AFD_ERR_INVALID, "window is NULL");
    const afd_window_config& c = w->cfg;
    if (first_stage < 0 || first_stage >= c.ring_depth)
        return fail(AFD_ERR_INVALID, "first_stage %d out of range", first_stage);
    if (n_items < 1) return fail(AFD_ERR_INVALID, "n_items %d < 1", n_items);
    if (max_peers < 0 || max_peers > c.num_peers)
        return fail(AFD_ERR_INVALID, "max_peers %d outside 0..%d", max_peers, c.num_peers);
    if (gather_us < 0 || gather_us > c.poll_timeout_us)
        return fail(AFD_ERR_INVALID, "gather_us %d outside 0..poll_timeout_us", gather_us);
    if (w->n_layers < 1) return fail(AFD_ERR_INVALID, "no layer table set (afd_layer_table_set)");
    hipError_t e = afd::launch_serve_begin(w->ctx, (hipStream_t)stream);
    for (int i = 0; i < n_items && e == hipSuccess; ++i)
        e = afd::launch_ffn(w->ctx, (first_stage + i) % c.ring_depth, -1, afd::Weights{}, poll_ticks(w), w->num_cu,
                            nullptr, (hipStream_t)stream, max_peers, (long long)gather_us * w->ticks_per_us, i);
    if (e != hipSuccess) return hip_fail(e, "serve launch");
    return AFD_OK;
}

int32_t afd_ffn_serve_result(afd_window* w, void* stream, int32_t* status, int32_t* items_done, int32_t* stop_item) {
    if (!w || !status || !items_done || !stop_item) return fail(AFD_ERR_INVALID, "NULL argument");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    int32_t words[3];
    e = hipMemcpy(words, w->ctx.serve, sizeof words, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "hipMemcpy");
    *status = words[0];
    *items_done = words[1];
    *stop_item = words[2];
    return AFD_OK;
}

int32_t afd_ffn_loop_destroy(afd_ffn_loop* l) {
    if (!l) return AFD_OK;
    hipError_t e = hipSuccess;
    if (l->exec) e = hipGraphExecDestroy(l->exec);
    if (l->graph) {
        const hipError_t e2 = hipGraphDestroy(l->graph);
        if (e == hipSuccess) e = e2;
    }
    delete l;
    if (e != hipSuccess) return hip_fail(e, "loop destroy");
    return AFD_OK;
}

int32_t afd_slot_unpack(afd_window* w, int32_t peer, int32_t stage, int32_t seq_len, void* out,
                        void* peer_stream) {
    if (!w) return fail(AFD_ERR_INVALID, "window is NULL");
    const afd_window_config& c = w->cfg;
    if (peer < 0 || peer >= c.num_peers) return fail(AFD_ERR_INVALID, "peer %d out of range", peer);
    if (stage < 0 || stage >= c.ring_depth) return fail(AFD_ERR_INVALID, "stage %d out of range", stage);
    const int idx = peer * c.ring_depth + stage;
    if (seq_len != w->packed_len[idx])
        return fail(AFD_ERR_SHAPE, "seq_len %d differs from the packed length %d", seq_len, w->packed_len[idx]);
    if (w->ctx.Eg != c.num_experts)
        return fail(AFD_ERR_INVALID, "the window owns experts [%d, %d) of %d: combine with afd_slot_unpack_ranks",
                    c.expert_offset, c.expert_offset + c.num_experts, w->ctx.Eg);
    if (seq_len == 0) {
        w->inflight[idx] = 0;
        return AFD_OK;  // nothing was sent, nothing to wait for
    }
    if (!w->inflight[idx]) return fail(AFD_ERR_INVALID, "(peer %d, stage %d) has no message in flight", peer, stage);
    if (!out || !aligned(out, 16)) return fail(AFD_ERR_INVALID, "out must be a 16-byte aligned device pointer");
    const long long timeout = (long long)c.poll_timeout_us * w->ticks_per_us;
    hipError_t e = afd::launch_unpack(w->ctx, peer, stage, seq_len, w->pack_seq[idx], out, timeout,
                                      (hipStream_t)peer_stream);
    if (e != hipSuccess) return hip_fail(e, "unpack launch");
    w->inflight[idx] = 0;
    return AFD_OK;
}

int32_t afd_slot_unpack_ranks(afd_window* const* wins, int32_t n_wins, int32_t peer, int32_t stage, int32_t seq_len,
                              void* out, void* peer_stream) {
    if (!wins || n_wins < 1 || n_wins > afd::kMaxRanks)
        return fail(AFD_ERR_INVALID, "n_wins must be in [1, %d] with a window array", afd::kMaxRanks);
    for (int i = 0; i < n_wins; ++i)
        if (!wins[i]) return fail(AFD_ERR_INVALID, "window %d is NULL", i);
    const afd_window_config& c0 = wins[0]->cfg;
    const int Eg = wins[0]->ctx.Eg;
    if (!c0.attention_routes) return fail(AFD_ERR_INVALID, "windows must be attention-routed");
    if (peer < 0 || peer >= c0.num_peers) return fail(AFD_ERR_INVALID, "peer %d out of range", peer);
    if (stage < 0 || stage >= c0.ring_depth) return fail(AFD_ERR_INVALID, "stage %d out of range", stage);
    const int idx = peer * c0.ring_depth + stage;
    std::vector<std::pair<int, int>> ranges;
    int n_shared = 0;
    for (int i = 0; i < n_wins; ++i) {
        const afd_window* w = wins[i];
        const afd_window_config& c = w->cfg;
        if (!c.attention_routes || w->ctx.Eg != Eg || c.num_peers != c0.num_peers || c.ring_depth != c0.ring_depth ||
            c.token_cap != c0.token_cap || c.hidden != c0.hidden || c.top_k != c0.top_k ||
            c.renormalize != c0.renormalize || c.routed_scaling_factor != c0.routed_scaling_factor ||
            w->device != wins[0]->device)
            return fail(AFD_ERR_INVALID, "window %d does not fit window 0 (configuration or device)", i);
        for (int j = 0; j < i; ++j)
            if (wins[j] == w) return fail(AFD_ERR_INVALID, "window %d given twice", i);
        ranges.push_back({c.expert_offset, c.expert_offset + c.num_experts});
        n_shared += c.shared_intermediate > 0;
        if (seq_len != w->packed_len[idx])
            return fail(AFD_ERR_SHAPE, "seq_len %d differs from window %d's packed length %d", seq_len, i,
                        w->packed_len[idx]);
        if (seq_len > 0 && !w->inflight[idx])
            return fail(AFD_ERR_INVALID, "window %d has no message of (peer %d, stage %d) in flight", i, peer, stage);
    }
    std::sort(ranges.begin(), ranges.end());
    int next = 0;
    for (const auto& r : ranges) {
        if (r.first != next) return fail(AFD_ERR_INVALID, "the windows' expert ranges do not partition [0, %d)", Eg);
        next = r.second;
    }
    if (next != Eg) return fail(AFD_ERR_INVALID, "the windows' expert ranges do not partition [0, %d)", Eg);
    if (n_shared > 1) return fail(AFD_ERR_INVALID, "more than one window has a shared expert");
    if (seq_len == 0) {
        for (int i = 0; i < n_wins; ++i) wins[i]->inflight[idx] = 0;
        return AFD_OK;
    }
    if (!out || !aligned(out, 16)) return fail(AFD_ERR_INVALID, "out must be a 16-byte aligned device pointer");
    std::vector<const afd::DevCtx*> ctx(n_wins);
    std::vector<int> echo(n_wins);
    std::vector<long long> timeout(n_wins);
    for (int i = 0; i < n_wins; ++i) {
        ctx[i] = &wins[i]->ctx;
        echo[i] = wins[i]->pack_seq[idx];
        timeout[i] = (long long)wins[i]->cfg.poll_timeout_us * wins[i]->ticks_per_us;
    }
    hipError_t e = afd::launch_unpack_ranks(ctx.data(), n_wins, peer, stage, seq_len, echo.data(), out,
                                            timeout.data(), (hipStream_t)peer_stream);
    if (e != hipSuccess) return hip_fail(e, "unpack launch");
    for (int i = 0; i < n_wins; ++i) wins[i]->inflight[idx] = 0;
    return AFD_OK;
}

static int32_t read_status(afd_window* w, const int* dev_words, void* stream, afd_run_info* info) {
    if (!info) return fail(AFD_ERR_INVALID, "info is NULL");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    int32_t words[afd::kStatusWords];
    e = hipMemcpy(words, dev_words, sizeof words, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "status copy");
    info->status = words[0];
    info->failed_peer = words[1];
    info->last_seq = words[2];
    info->total_tokens = words[3];
    info->served_mask = (uint64_t)(uint32_t)words[4] | ((uint64_t)(uint32_t)words[5] << 32);
    (void)w;
    return AFD_OK;
}

int32_t afd_window_status(afd_window* w, int32_t stage, void* stream, afd_run_info* info) {
    if (!w) return fail(AFD_ERR_INVALID, "window is NULL");
    if (stage < 0 || stage >= w->cfg.ring_depth) return fail(AFD_ERR_INVALID, "stage out of range");
    return read_status(w, w->ctx.run_status + stage * afd::kStatusWords, stream, info);
}

int32_t afd_peer_status(afd_window* w, int32_t peer, int32_t stage, void* stream, afd_run_info* info) {
    if (!w) return fail(AFD_ERR_INVALID, "window is NULL");
    if (peer < 0 || peer >= w->cfg.num_peers || stage < 0 || stage >= w->cfg.ring_depth)
        return fail(AFD_ERR_INVALID, "peer/stage out of range");
    return read_status(w, w->ctx.peer_status + (peer * w->cfg.ring_depth + stage) * afd::kStatusWords, stream, info);
}

int32_t afd_window_poll(afd_window* w, int32_t which, int32_t* flags_out) {
    if (!w || !flags_out || (which != 0 && which != 1)) return fail(AFD_ERR_INVALID, "bad poll arguments");
    const char* src = which == 0 ? w->ctx.in_win : w->ctx.ret_win;
    hipError_t e = hipMemcpy(flags_out, src, sizeof(int32_t) * w->cfg.num_peers * w->cfg.ring_depth,
                             hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "poll copy");
    return AFD_OK;
}

int32_t afd_debug_routing(afd_window* w, void* stream, int32_t* ids, float* wts, int32_t* counts,
                          int32_t* expert_offsets, int32_t* perm, int32_t* inv, int32_t* split_offsets) {
    if (!w) return fail(AFD_ERR_INVALID, "window is NULL");
    hipError_t e = hipStreamSynchronize((hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "hipStreamSynchronize");
    const afd::DevCtx& d = w->ctx;
    const afd_window_config& c = w->cfg;
    int32_t T = 0;
    e = hipMemcpy(&T, d.Tptr, 4, hipMemcpyDeviceToHost);
    const size_t np = (size_t)T * c.top_k;
    auto cp = [&](void* dst, const void* src, size_t bytes) {
        if (e == hipSuccess && dst && bytes) e = hipMemcpy(dst, src, bytes, hipMemcpyDeviceToHost);
    };
    cp(ids, d.ids, 4 * np);
    cp(wts, d.wts, 4 * np);
    cp(counts, d.counts, 4 * (size_t)c.num_experts);
    cp(expert_offsets, d.eoff, 4 * ((size_t)c.num_experts + 1));
    cp(perm, d.perm, 4 * np);
    cp(inv, d.inv, 4 * np);
    cp(split_offsets, d.off, 4 * ((size_t)c.num_peers + 1));
    if (e != hipSuccess) return hip_fail(e, "debug copy");
    return AFD_OK;
}

int32_t afd_debug_read(afd_window* w, int64_t offset, int64_t bytes, void* host_dst) {
    if (!w || !host_dst || offset < 0 || bytes < 0 || offset + bytes > w->lay.total_bytes)
        return fail(AFD_ERR_INVALID, "debug read out of range");
    hipError_t e = hipMemcpy(host_dst, w->base + offset, (size_t)bytes, hipMemcpyDeviceToHost);
    if (e != hipSuccess) return hip_fail(e, "debug read");
    return AFD_OK;
}

int32_t afd_debug_write(afd_window* w, int64_t offset, int64_t bytes, const void* host_src) {
    if (!w || !host_src || offset < 0 || bytes < 0 || offset + bytes > w->lay.total_bytes)
        return fail(AFD_ERR_INVALID, "debug write out of range");
    hipError_t e = hipMemcpy(w->base + offset, host_src, (size_t)bytes, hipMemcpyHostToDevice);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) return hip_fail(e, "debug write");
    return AFD_OK;
}

int32_t afd_profile_enable(afd_window* w, int32_t on) {
    if (!w) return fail(AFD_ERR_INVALID, "window is NULL");
    if (on < 0 || on > 3) return fail(AFD_ERR_INVALID, "profile mode must be 0, 1, 2 or 3");
    if (on && w->is_static) return fail(AFD_ERR_INVALID, "a static window has no profiling events");
    std::lock_guard<std::mutex> g(w->prof_mu);
    prof_collect(w);
    w->profile = on;
    return AFD_OK;
}

int32_t afd_profile_read(afd_window* w, float* ms, int32_t n, int32_t* runs, int32_t reset) {
    if (!w) return fail(AFD_ERR_INVALID, "window is NULL");
    std::lock_guard<std::mutex> g(w->prof_mu);
    prof_collect(w);
    for (int i = 0; i < n && i < AFD_PROFILE_SLOTS; ++i) ms[i] = (float)w->prof_ms[i];
    if (runs) *runs = w->prof_runs;
    if (reset) {
        for (double& v : w->prof_ms) v = 0.0;
        w->prof_runs = 0;
    }
    return AFD_OK;
}

const char* afd_profile_kernel_name(int32_t i) {
    if (i < 0 || i >= AFD_PROFILE_SLOTS) return "";
    return kProfileNames[i];
}

}  // extern "C"
