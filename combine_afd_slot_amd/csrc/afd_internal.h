// afd_internal.h -- device context shared by the host launcher code and the
// kernels of libafd.so.  Not part of the ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "afd_proto.h"

namespace afd {

// Tokens handled by one routing / permutation workgroup.  The per-block
// expert histograms of the routing kernel and the stable ranks of the
// permutation kernel are both taken over these chunks, in token order.
constexpr int kRouteChunk = 16;
constexpr int kMaxTopK = 16;
constexpr int kMaxPeers = 64;
constexpr int kMaxRing = 4;      // ring_depth limit (stages in flight per peer)
constexpr int kMaxLayers = 1024;  // entries of the device layer table
constexpr int kMaxExperts = 1024;

// Grouped-GEMM tile: up to kBX token rows (8 blocks of 32) of one group x kBW
// weight rows, kBK deep per step, computed by kGemmThreads threads: 4 waves,
// one per SIMD, each owning a 128 x 128 block of the tile (4 x 4 MFMA
// outputs of 32 x 32), which keeps the LDS fragment traffic at half a KB per
// MFMA.  A group's 32-row blocks are split evenly over ceil(blocks/8) row
// tiles.  For the gate/up GEMM the kBW weight rows are kBW/2 gate rows and
// the same kBW/2 up rows.  kStages LDS stages of 32 KB form a ring whose
// loads run kStages-1 steps ahead of the MFMAs.
constexpr int kBX = 256;
constexpr int kBW = 256;
constexpr int kBK = 32;
constexpr int kStages = 4;
constexpr int kGemmThreads = 256;
constexpr int kTileBlocks = kBX / 32;
constexpr int kXcds = 8;

// Tile segments of a GEMM: the shared expert's tiles (the longest) cut into
// kXcds cost-balanced segments, then the heavy routed experts' tiles and the
// light routed experts' tiles (one token block) cut the same way; segment s
// covers tiles [seg[s], seg[s+1]).
constexpr int kSegs = 3 * kXcds;

// Windows of at most kShSplitRows tokens (Tmax = P * token_cap: one row tile
// of the shared expert) split the shared expert's down GEMM over its depth
// into up to kShParts tiles per column tile (decode-sized batches: the
// routed tiles fill whole rounds of the CUs, and the shared tiles, whose
// depth is the shared intermediate width, would add a round of their own).
// Each part writes an fp32 partial row; the consumers sum the parts in
// order and round the sum to bf16 once.
constexpr int kShSplitRows = 256;
constexpr int kShParts = 8;

// Per-stage run status words: [status, failed_peer, seq of peer 0, T].
// Run status words: [status, failed_peer, seq of peer 0, T, served peers
// (bits 0..31), served peers (bits 32..63)].
constexpr int kStatusWords = 6;

struct Weights;

// Everything a kernel needs, passed by value.
struct DevCtx {
    // configuration
    int P, R, token_cap, H, E, K, I, Is, renorm;
    float rsf;
    int has_shared;  // Is > 0
    int G;           // GEMM groups: shared first (when present), then experts
    int NB;          // routing chunks for P*token_cap tokens
    int max_tiles1, max_tiles2;  // upper bounds of the GEMM tile counts (sanity limits)
    int hrows, hsrows;           // row capacity of h (Tmax*K) and hs (Tmax)
    int nt1, nt2;                // column tiles of a routed expert: gate/up ceil(I/128), down ceil(H/256)
    int64_t slot_bytes;
    int64_t foff[AFD_NUM_FIELDS];
    // windows (flags at offset 0 of each window)
    char* in_win;
    char* ret_win;
    int64_t slots_off;  // first slot, relative to a window's start
    // control words
    int* seen_in;      // [P*R] FFN-side mirror of the inbound flags
    int* ret_seq;      // [P*R] FFN-side return sequence counters
    int* seen_ret;     // [P*R] peer-side mirror of the return flags
    int* cur_seq;      // [P]   inbound seq consumed by the current run
    int* off;          // [P+1] fan-in offsets
    int* Tptr;         // [1]   total tokens of the current run
    int* run_status;   // [R][kStatusWords]
    int* rr;           // [R]   first peer an any-ready run of the stage scans (rotates for fairness)
    int* prow;         // [P]   attention-routed runs: routed rows of each peer's message
    int* serve;        // [3]   serve loop: stop status (0: running), items done, stop item
    int* route_done;   // routing workgroups finished in this run (small work items; the last resets it)
    int poison;        // fill slots with 0xFFFFFFFF (NaN as fp32 and bf16) before each pack / reply
    int* layer_cur;    // [1]   layer of the current run (from the headers in layer-table runs)
    // attention-side routing (attn_routes): the routed rows arrive grouped by
    // expert, the peer keeps the top-k weights and combines on return
    int attn_routes;
    int w1_fp8;        // gate/up GEMMs on e4m3 operands
    uint8_t* xq;       // [Tmax][H] e4m3 codes of the token rows (fp8 W1); attention-routed:
                       //   [Tmax*K + Tmax][H], each GEMM row's (pairs, then shared rows)
    float* sx;         // [Tmax]   their dequantisation scales
    float* sxp;        // [Tmax*K + Tmax] the scale of each permuted pair's token row, then of
                       //   each shared row (token t at Tmax*K + t)
    int Eg;            // experts the peers route over (E unless the window owns a segment)
    int e0;            // first expert of the window's segment
    int NBp;           // routing chunks of one message: ceil(token_cap / kRouteChunk)
    int* pid;          // [P*R][token_cap*K] expert of pair (t, k) of the (peer, stage) message
    float* pwt;        // [P*R][token_cap*K] its weight
    int* ppos;         // [P*R][token_cap*K] its row among the message's grouped rows
    int* pblk;         // [P*R][E][NBp] chunk histograms of the message's pairs
    int* pbase;        // [P*R][E][NBp] pairs of the expert in earlier chunks
    int* pcnt;         // [P*R][E] the message's group list (pairs per expert)
    uint32_t* retoff;  // [Tmax*K] return-window byte offset of each grouped row's return row
    uint32_t* retoffs; // [Tmax]   return-window byte offset of each shared row's return row
    int direct_ret;    // the down GEMM stores straight into the return slots (window < 1 GiB)
    uint32_t ret_bytes;  // bytes of the return window
    int* nlayers;      // [1]   entries of the layer table (0: none set)
    const Weights* wtable;  // [kMaxLayers] packed weights of each layer (layer-table runs)
    int* peer_status;  // [P*R][kStatusWords]
    // routing / dispatch
    int* peer_counts;  // [P][E]
    int* blk_counts;   // [E][NB] per-chunk expert histograms (attention-routed runs, with NB >= P:
                       //   [P][E] first row of each group in the peer's slot)
    int* blk_base;     // [E][NB] stable base of each chunk inside its expert group (attention-
                       //   routed runs: [P][E] first row of the peer's share of each group)
    int* counts;       // [E]
    int* eoff;         // [E+1]
    int* tstart1;      // [G+1] gate/up GEMM tile prefix per group
    int* tstart2;      // [G+1] down GEMM tile prefix per group
    int4* tinfo1;      // [max_tiles1] (group, nt | tb << 16, first row, rows) of each gate/up tile
    int4* tinfo2;      // [max_tiles2]
    int* seg1;         // [kSegs+1] tile segments of the gate/up GEMM
    int* seg2;         // [kSegs+1]
    int* tctr;         // [2][kSegs] tiles taken from each segment (zeroed by the planner)
    uint64_t* psrc;    // [Tmax*K] address of the token row of each permuted pair
    int* ids;          // [Tmax*K]
    float* wts;        // [Tmax*K]
    int* perm;         // [Tmax*K]
    int* inv;          // [Tmax*K]
    uint64_t* tok_src; // [Tmax] address of token t's routed_x row
    uint64_t* sh_src;  // [Tmax] address of shared row t's shared_x row
    // expert activations
    // h and hs are stored depth-block major: element (row, j) at
    // ((j / 32) * rows + row) * 32 + j % 32, so the rows of one 32-deep
    // step of a down-GEMM tile are one contiguous run.
    uint16_t* h;       // [ceil(I/32)][Tmax*K][32]  bf16 SwiGLU activations, permuted order
    uint16_t* hs;      // [ceil(Is/32)][Tmax][32]   bf16 shared activations
    uint16_t* y;       // [Tmax*K][H]  bf16 routed expert outputs, permuted order
    uint16_t* ys;      // [Tmax][H]    bf16 shared expert output, token (= shared row) order
    int ncu;           // compute units: the GEMMs' grid, for which the planner reserves first tiles
    int shp;           // depth parts of the shared expert's down GEMM (1: not split)
    float* ysp;        // [shp][Tmax][H] fp32 partial shared outputs (shp > 1)
};

// One layer's packed weights (written by k_pack_weights): tiles of 256
// weight rows x 32 depth values, 16 KB each, a row's 64 bytes with chunk c
// of the row stored at chunk position c ^ swz4(row) (the LDS order of the
// GEMM stages).  Tile (column tile nt, depth step kt) of
//   w13  [E][nt1][nk1]: rows 0..127 gate rows nt*128 + r, rows 128..255 the
//        same up rows (rows past I zero); nk1 = ceil(H/32)
//   ws13 [ceil(Is/128)][nk1]: the same for the shared expert
//   w2   [E][nt2][nk2]: rows nt*256 + r of W2 (rows past H zero); nk2 = ceil(I/32)
//   ws2  [nt2][ceil(Is/32)]
// Depth past K is zero.
constexpr int kWTileBytes = kBW * kBK * 2;  // 16 KB
struct Weights {
    const char* w13;
    const char* w2;
    const char* ws13;
    const char* ws2;
    const float* sw13;   // fp8 W1: dequantisation scale of each W13 row ([E][2I])
    const float* sws13;  // and of each Ws13 row ([2Is])
};

// Byte offsets of the packed regions (w13, ws13, w2, ws2, then the fp8 row
// scales sw13, sws13) and the total (host).
void packed_weight_layout(const afd_window_config& c, int64_t off[6], int64_t* total);

// Launchers (afd_kernels.hip).  All return the launch's hipError_t.
hipError_t launch_pack_weights(const DevCtx& c, const afd_moe_weights& src, char* dst, const int64_t off[6],
                               int64_t total, hipStream_t st);
hipError_t launch_pack(const DevCtx& c, int peer, int stage, int layer, int seq_len, const void* hidden,
                       const float* logits, uint32_t flags, int seq, hipStream_t st);
constexpr int kMaxRanks = 16;  // windows combined by one afd_slot_unpack_ranks
hipError_t launch_unpack_ranks(const DevCtx* const* ctx, int n, int peer, int stage, int seq_len, const int* echo,
                               void* out, const long long* timeout_ticks, hipStream_t st);
hipError_t launch_unpack(const DevCtx& c, int peer, int stage, int seq_len, int expect_echo, void* out,
                         long long timeout_ticks, hipStream_t st);
// One FFN run; `ev` (may be null) holds kProfileSlots+1 events recorded
// between the launches.  max_take = 0: the work item is every peer of the
// stage; max_take > 0: at most max_take of the peers that are ready (an
// any-ready run), after waiting gather_ticks past the first one for more.
// serve_item >= 0: item serve_item of an afd_ffn_serve loop (skipped once
// the loop has stopped; its outcome recorded in the serve words).
hipError_t launch_ffn(const DevCtx& c, int stage, int layer, const Weights& w, long long timeout_ticks,
                      int num_cu, hipEvent_t* ev, hipStream_t st, int max_take = 0, long long gather_ticks = 0,
                      int serve_item = -1);
hipError_t launch_serve_begin(const DevCtx& c, hipStream_t st);
// Zero `bytes` bytes (a multiple of 4) at p on st with a fill kernel.
hipError_t launch_zero(void* p, int64_t bytes, hipStream_t st);

}  // namespace afd
