/*
 * afd.h -- C ABI of libafd.so, the MI355X (gfx950) FFN-rank hot path of
 * Attention-FFN Disaggregation (AFD).
 *
 * One FFN replica on one GPU serves P attention peers for one layer and
 * stage.  Each peer drops its bf16 hidden states and fp32 router logits into
 * a slot of a window in HBM and publishes a flag; the FFN side waits for all
 * P flags, fans the peers in along the token dimension, routes every token to
 * its top-k experts, groups the (token, expert) pairs per expert, runs the
 * routed SwiGLU experts and the shared expert, combines the expert outputs
 * with the router weights, and writes each peer's slice of the result into
 * that peer's return slot, publishing a return flag per peer.
 *
 * Beyond that single run: a device table of every layer's weights with the
 * layer taken from the headers (afd_layer_table_set, afd_ffn_run_table) and
 * runs captured into a replayable graph (afd_ffn_loop_*); runs that serve
 * whichever peers are ready (afd_ffn_run_ready) and a loop of runs stopped
 * on the device by a timeout or shutdown (afd_ffn_serve); windows without a
 * shared expert (routed-only protocol); and attention-routed windows, where
 * the peers route, send their rows grouped by expert and combine the
 * returned rows themselves, optionally with the experts split over several
 * FFN ranks' windows (attention_routes, route_experts, expert_offset,
 * afd_slot_unpack_ranks).
 *
 * Sources (page titles; sections):
 *   "[RFC]: Async GPU Connector" (vllm-project/afd-plugin issue 233):
 *     "Window and slot layout", "Capacity and ring depth", "Data flow",
 *     "Attention gate and FFN expert compute", "FFN main loop",
 *     "Risks and alternatives" (echo_seq, ring staging, host poll).
 *   "Data on the wire: tensors per layer and stage": Steps 1-4 (shape
 *     checks, transfer metadata, fan-in, split back by seq_lens).
 *   "NCCL_P2P_CONNECTOR_USER_GUIDE.md": Configuration
 *     (compute_gate_on_attention: logits travel to the FFN, which routes).
 *   "[RFC]: Async AFD for Prefill on Ascend NPU": "Asynchronous work-item
 *     contract" (write before ready; ready only when all participants
 *     published; layer and counts consumed on the device; completion) and
 *     "FFN execution modes" (fixed-shape buffers sized by the maximum
 *     reserved token count; device-side blocking receive; layer-select
 *     operators and graph mode), "Architecture", "Shared-expert ownership".
 *
 * Conventions for every entry point:
 *   - Return value: an afd_status (0 = AFD_OK).  Errors that the host can see
 *     (bad arguments, capacity, ring, shape) are returned before anything is
 *     enqueued; afd_last_error() then holds a message for the calling thread.
 *   - Errors that only the device can see (timeout, corrupt header, stale
 *     echo_seq, shutdown) are written to a device status word; every later
 *     kernel of that call exits early and no output flag is published, so a
 *     half-written result is never visible.  Read the word with
 *     afd_window_status / afd_peer_status (they synchronize the stream).
 *   - "stream" arguments are hipStream_t handles passed as void* (NULL = the
 *     null stream); they are borrowed, never destroyed.
 *   - Device pointers (hidden, logits, out, weights) are borrowed: the caller
 *     keeps them alive and unmodified until the enqueued work on that stream
 *     completes.  The window (flags, slots, workspace) is owned by the
 *     library and freed by afd_window_destroy.
 *   - Threading: calls for different peers may come from different host
 *     threads; calls for the same peer, and all afd_ffn_run calls of one
 *     window (they share one workspace and must be issued on one stream),
 *     must not race.
 */
#ifndef AFD_H_
#define AFD_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AFD_ABI_VERSION 9

/* Header flags bit 1: shutdown sentinel ("Window and slot layout"). */
#define AFD_FLAG_SHUTDOWN 0x2u

/* Slot fields in slot order ("Window and slot layout"). */
#define AFD_NUM_FIELDS 5
#define AFD_FIELD_HEADER 0      /* int32 [12 + num_experts]                    */
#define AFD_FIELD_ROUTE_TABLE 1 /* fp32 [token_cap][num_experts] router logits */
#define AFD_FIELD_ROUTED_X 2    /* bf16 [token_cap][hidden]; in: hidden states, return: output */
#define AFD_FIELD_SHARED_IDX 3  /* int32 [token_cap] shared-row token index     */
#define AFD_FIELD_SHARED_X 4    /* bf16 [token_cap][hidden] shared rows         */

/* Header word indices (12 words, then n_counts expert counts). */
#define AFD_HDR_MAGIC 0
#define AFD_HDR_VERSION 1
#define AFD_HDR_FLAGS 2
#define AFD_HDR_SEQ 3
#define AFD_HDR_ECHO_SEQ 4
#define AFD_HDR_LAYER 5
#define AFD_HDR_STAGE 6
#define AFD_HDR_NUM_TOKENS 7
#define AFD_HDR_ROUTED_TOKENS 8
#define AFD_HDR_SHARED_TOKENS 9
#define AFD_HDR_SRC_PEER 10
#define AFD_HDR_N_COUNTS 11
#define AFD_HDR_WORDS 12
#define AFD_HDR_MAGIC_VALUE 0x47444641 /* bytes 'A','F','D','G' little-endian */
#define AFD_HDR_VERSION_VALUE 1

typedef enum afd_status {
    AFD_OK = 0,
    AFD_SHUTDOWN = 1,        /* a peer's header carried the shutdown bit: normal exit ("FFN main loop") */
    AFD_ERR_INVALID = -1,    /* bad argument or config; unknown/nonzero reserved fields rejected */
    AFD_ERR_CAPACITY = -2,   /* seq_len > token_cap: raised before any write, never truncated
                                ("Capacity and ring depth") */
    AFD_ERR_SHAPE = -3,      /* seq_len disagrees with the header's num_tokens / the packed length
                                ("Data on the wire", shape checks) */
    AFD_ERR_RING = -4,       /* (peer, stage) still in flight: ring exhausted ("Capacity and ring depth") */
    AFD_ERR_TIMEOUT = -5,    /* flag not seen within poll_timeout_us ("FFN main loop"; bounded waits) */
    AFD_ERR_HEADER = -6,     /* magic / version / length / layer / stage / count check failed */
    AFD_ERR_SEQ = -7,        /* return header's echo_seq is not the seq this peer sent ("Risks") */
    AFD_ERR_DEVICE = -8      /* HIP runtime error; text in afd_last_error() */
} afd_status;

typedef struct afd_window afd_window; /* opaque, library-owned */

/* Window configuration.  struct_size must equal sizeof(afd_window_config)
 * and reserved[] must be zero (unknown fields are rejected, as the pages'
 * connector rejects unknown connector_extra_config fields).
 * Limits: 1 <= num_peers <= 64; 1 <= ring_depth <= 4; token_cap >= 1;
 * hidden, intermediate, shared_intermediate multiples of 8 (16-byte rows);
 * 1 <= top_k <= min(num_experts, 16); 1 <= num_experts <= 1024;
 * shared_intermediate 0 = no shared expert on the FFN side: the routed-only
 * protocol ("[RFC]: Async AFD for Prefill on Ascend NPU", "Shared-expert
 * ownership"), where the slots have no shared_idx / shared_x space (both
 * fields 0 bytes), nothing is copied into them, and headers carry
 * shared_tokens = 0 (the attention side adds its own shared branch to the
 * returned routed output); renormalize 0 or 1;
 * poll_timeout_us >= 1.
 *
 * attention_routes = 1: the attention side routes ("[RFC]: Async GPU
 * Connector", "Data flow"): afd_slot_pack takes the router logits, selects
 * and weighs the top_k experts with the same code as the FFN side, sorts the
 * message's (token, expert) pairs stably and writes the routed rows grouped
 * by expert, the group list (rows per expert) in the header's counts; no
 * logits travel (route_table 0 bytes, routed_x token_cap*top_k rows).  The
 * FFN runs send the expert outputs back in the order they came and
 * afd_slot_unpack combines them with the weights the pack kept.
 * Expert-parallel segmentation (same section; "Capacity and ring depth":
 * expert_per_rank): with route_experts > 0 the peers route over
 * route_experts experts and this window is the FFN rank that owns experts
 * [expert_offset, expert_offset + num_experts); a pack sends it only the
 * pairs of those experts (routed_tokens = their number, at most
 * num_tokens*top_k) and the outputs are combined over all ranks' windows
 * by afd_slot_unpack_ranks.  route_experts 0 means num_experts (one rank).
 * Limits: route_experts > 0 needs attention_routes = 1, top_k <=
 * route_experts <= 1024, 0 <= expert_offset, expert_offset + num_experts
 * <= route_experts; with route_experts 0, expert_offset must be 0.
 *
 * w1_fp8 = 1: the gate/up GEMMs (W13 and the shared Ws13) run on OCP FP8
 * E4M3 operands ("[RFC]: Async AFD for Prefill on Ascend NPU",
 * "Architecture": the routed W1 + SwiGLU grouped GEMM, quantised): each
 * token row is quantised when it is routed and each W13 / Ws13 row when the
 * weights are packed, one scale per row (r = 448 / max|x| and code =
 * e4m3(x * r) in fp32, round to nearest even, saturating; the row's value is
 * code * max|x| / 448); products accumulate in fp32 and both scales apply
 * before SwiGLU.  The down GEMM stays bf16.  Needs hidden a multiple of 64;
 * the packed weights then hold e4m3 gate/up tiles and their row scales
 * (layout.packed_weight_bytes).  In an attention-routed window the FFN side
 * quantises each arriving row (copies of a token row get that row's codes). */
typedef struct afd_window_config {
    uint32_t struct_size;
    int32_t num_peers;           /* P: attention peers fanned in by this FFN replica        */
    int32_t ring_depth;          /* stages in flight per peer (1 without micro-batching)     */
    int32_t token_cap;           /* max tokens per peer message (max_num_batched_tokens)     */
    int32_t hidden;              /* H                                                        */
    int32_t num_experts;         /* E routed experts                                         */
    int32_t top_k;               /* K                                                        */
    int32_t intermediate;        /* I: routed SwiGLU width                                   */
    int32_t shared_intermediate; /* Is: shared SwiGLU width (0 = none)                       */
    float routed_scaling_factor; /* scales the routed branch (1.0 = none)                    */
    int32_t renormalize;         /* 1: top-k weights renormalised to sum to 1                */
    int32_t poll_timeout_us;     /* bound of every device-side flag wait                     */
    int32_t attention_routes;    /* 0: the FFN routes (logits travel); 1: the attention side
                                    routes and sends rows grouped by expert (see above)      */
    int32_t route_experts;       /* experts the peers route over (0: num_experts)            */
    int32_t expert_offset;       /* first of the num_experts experts this window owns        */
    int32_t w1_fp8;              /* 1: gate/up GEMMs on e4m3 operands (see above)            */
    int32_t reserved[1];         /* must be 0                                                */
} afd_window_config;

/* Byte layout of the library's single device allocation.  The inbound
 * window (attention -> FFN) and the return window (FFN -> attention) share
 * one slot layout (both directions use the same layout: "Window and slot
 * layout").  Each window = int32 flags[num_peers*ring_depth] then the
 * slots slot(p, s) at index p*ring_depth + s; every field is 256-byte aligned. */
typedef struct afd_layout {
    int64_t field_off[AFD_NUM_FIELDS];   /* offset of each field inside a slot       */
    int64_t field_bytes[AFD_NUM_FIELDS]; /* unaligned size of each field             */
    int64_t slot_bytes;                  /* aligned slot stride                      */
    int64_t window_bytes;                /* flags + all slots of one window          */
    int64_t in_off;                      /* inbound window (its flags come first)    */
    int64_t in_slots_off;                /* first inbound slot                       */
    int64_t ret_off;                     /* return window                            */
    int64_t ret_slots_off;               /* first return slot                        */
    int64_t workspace_off;               /* FFN workspace                            */
    int64_t workspace_bytes;
    int64_t total_bytes;                 /* the whole allocation                     */
    int64_t packed_weight_bytes;         /* one layer's weights in GEMM tile order   */
} afd_layout;

/* Status of the last device-side operation of a stage (afd_window_status) or
 * of a peer's last unpack (afd_peer_status). */
typedef struct afd_run_info {
    int32_t status;       /* afd_status                                        */
    int32_t failed_peer;  /* first peer that failed, -1 if none                */
    int32_t last_seq;     /* FFN run: seq consumed from peer 0; unpack: return seq */
    int32_t total_tokens; /* FFN run: T = sum of the peers' num_tokens         */
    uint64_t served_mask; /* FFN run: bit p set = peer p's message was consumed (and answered
                             when non-empty); 0 when the run failed; unpack: 0          */
} afd_run_info;

/* Expert weights of one layer (device pointers, bf16, borrowed).
 *   w13  [E][2I][H]: rows [0, I) gate, rows [I, 2I) up
 *   w2   [E][H][I]
 *   ws13 [2Is][H] (NULL when shared_intermediate == 0), ws2 [H][Is]        */
typedef struct afd_moe_weights {
    const void* w13;
    const void* w2;
    const void* ws13;
    const void* ws2;
} afd_moe_weights;

/* Repack one layer's expert weights (the row-major afd_moe_weights layout
 * above) into the order the grouped GEMMs stream them, on `stream`.  A
 * one-time step when a layer's weights are loaded; afd_ffn_run reads only
 * the packed copy ("Attention gate and FFN expert compute": the expert FFN
 * weights of a layer stay resident on the FFN rank).  The packed format is
 * internal to this library version (it holds every weight once, padded to
 * whole GEMM tiles with zeros): dst must hold layout.packed_weight_bytes
 * bytes, 256-byte aligned, caller-owned, and must not overlap src.
 * Errors: AFD_ERR_INVALID (NULL or misaligned pointers, dst_bytes too small,
 * shared weights missing when shared_intermediate > 0). */
int32_t afd_weights_pack(afd_window* w, const afd_moe_weights* src, void* dst, int64_t dst_bytes,
                         void* stream);

/* Header fields for the host codec (tests; the device uses the same code). */
typedef struct afd_header_fields {
    int32_t flags, seq, echo_seq, layer_idx, stage_idx, num_tokens, routed_tokens,
        shared_tokens, src_peer, n_counts;
} afd_header_fields;

/* Layout for a configuration; host only, touches no device.  Validates cfg. */
int32_t afd_layout_compute(const afd_window_config* cfg, afd_layout* out);

/* Validate cfg, allocate the window + workspace on the current HIP device
 * (one hipMalloc), zero every flag and mirror, log the size when AFD_LOG=1.
 * The connector init of "Plugin boundary"/"Window and slot layout". */
int32_t afd_window_create(const afd_window_config* cfg, afd_window** out);

/* afd_window_create without any device allocation, for callers that cannot
 * call hipMalloc (code under HIP graph capture, tight serving loops,
 * harnesses that forbid allocation).  The window (flags, slots and FFN
 * workspace: layout.total_bytes, as afd_window_create would allocate) is
 * placed in a static device array of AFD_STATIC_WINDOW_BYTES that the
 * library holds on every GPU it runs on until the process ends.  The call
 * zeroes the flags, mirrors and status words with a fill kernel on the null
 * stream and synchronizes it; it calls no hipMalloc, hipFree or other
 * allocating routine, and profiling events are not available on such a
 * window.  One static window per device may be open at a time: every call on
 * a GPU shares that GPU's array, which keeps the last window's contents, so
 * a second afd_window_create_static on the device before the first is
 * destroyed is rejected, and work of two windows over the array must never
 * overlap.  All other entry points take the window as usual;
 * afd_window_destroy releases the array for the next static window (it
 * frees nothing).  Errors: AFD_ERR_INVALID (cfg, out, the device's static
 * window already open), AFD_ERR_CAPACITY (layout.total_bytes above
 * AFD_STATIC_WINDOW_BYTES; use afd_window_create), AFD_ERR_DEVICE. */
#define AFD_STATIC_WINDOW_BYTES (32ll << 20)
int32_t afd_window_create_static(const afd_window_config* cfg, afd_window** out);

/* Free everything.  NULL is accepted.  Waits for the device to go idle. */
int32_t afd_window_destroy(afd_window* w);

/* Offsets and sizes of the window (the pages log slot and total size at init). */
int32_t afd_window_layout(const afd_window* w, afd_layout* out);

/* Attention side, peer `peer`: write one message into inbound slot
 * (peer, stage) and publish it ("Data flow", send path; "Window and slot
 * layout": payload first, then the flag, ordered on one stream).
 *   hidden: device bf16 [seq_len][H] (row-major); logits: device fp32
 *   [seq_len][E]; seq_len may be 0 (header still published; unpack then
 *   returns without waiting).  flags: 0 or AFD_FLAG_SHUTDOWN (header only).
 * Writes routed_x = hidden, route_table = logits, shared_idx = 0..seq_len-1,
 * shared_x = hidden (one FFN replica owns every shared row), the header
 * (seq = this peer's next sequence number), then release-stores flag = seq.
 * Errors: AFD_ERR_INVALID (peer/stage/pointers), AFD_ERR_CAPACITY
 * (seq_len > token_cap), AFD_ERR_RING (the previous message of (peer,
 * stage) has not been unpacked yet). */
int32_t afd_slot_pack(afd_window* w, int32_t peer, int32_t stage, int32_t layer_idx,
                      int32_t seq_len, const void* hidden, const float* logits, uint32_t flags,
                      void* peer_stream);

/* FFN side: one work item = stage `stage` of all P peers for layer
 * `layer_idx`.  Enqueues on ffn_stream: a bounded device wait for all P
 * inbound flags (with header validation and the fan-in offsets), top-k
 * routing + per-expert histogram, the stable dispatch permutation, the routed
 * SwiGLU grouped GEMMs (gate/up + down), the shared expert, and the weighted
 * combine that writes each peer's rows into its return slot and publishes its
 * return flag.  The host reads nothing back: token counts, per-expert counts
 * and group sizes stay on the device.  Device-side failures land in the
 * stage's status word (afd_window_status).  Peers must have enqueued their
 * packs on other streams before this call can complete; keep the number of
 * concurrently waiting streams within the device's hardware queues.
 * packed_weights: the layer's weights as written by afd_weights_pack for
 * this window's configuration (borrowed; 256-byte aligned).
 * Errors: AFD_ERR_INVALID (NULL window or weights, misaligned weights, stage
 * out of range). */
int32_t afd_ffn_run(afd_window* w, int32_t stage, int32_t layer_idx, const void* packed_weights,
                    void* ffn_stream);

/* Layer-select weights ("[RFC]: Async AFD for Prefill on Ascend NPU",
 * "Architecture": layer-select operators take the address table of every
 * layer's weights and a layer index held on the device; "FFN execution
 * modes").  Copies a table of n_layers packed weight copies (each written by
 * afd_weights_pack for this window's configuration, 256-byte aligned,
 * borrowed: they must stay valid while runs that may select them are in
 * flight) into the window's device table; entry i serves layer_idx i.
 * packed_weights is a host array of n_layers device pointers.  Synchronizes
 * `stream` (the host array may be freed on return).  A later call replaces
 * the table; runs captured earlier read the new entries (the table and its
 * size live on the device).  Errors: AFD_ERR_INVALID (NULL arguments,
 * n_layers outside 1..1024, a NULL or misaligned entry), AFD_ERR_DEVICE. */
int32_t afd_layer_table_set(afd_window* w, int32_t n_layers, const void* const* packed_weights, void* stream);

/* afd_ffn_run with the layer identity kept on the device ("[RFC]: Async AFD
 * for Prefill on Ascend NPU", "FFN execution modes", eager mode): the layer is
 * the layer_idx that every peer's inbound header of the stage carries, and
 * the weights are that entry of the layer table.  Headers that disagree, or
 * a layer outside the table, fail the run with AFD_ERR_HEADER in the stage's
 * status word (nothing is consumed or published, as for any header error).
 * The return headers carry the selected layer.  The call reads nothing back
 * and allocates nothing, so it can be captured into a HIP graph.
 * Errors: AFD_ERR_INVALID (NULL window, stage out of range, no layer table
 * set). */
int32_t afd_ffn_run_table(afd_window* w, int32_t stage, void* ffn_stream);

/* Any-ready consumption ("[RFC]: Async AFD for Prefill on Ascend NPU",
 * "Asynchronous work-item contract": the FFN side may take any ready
 * replica without waiting for the others, and must not starve one;
 * "[RFC]: Async GPU Connector", "Risks and alternatives": a device-side wait
 * on the flag array, with a rotating scan start against starvation).  Like
 * afd_ffn_run, but the work item is not every peer of the stage: the device
 * waits (bounded by poll_timeout_us) until at least one peer's message of
 * the stage has arrived, then up to gather_us more microseconds for others
 * (0: none), and takes at most max_peers of the peers that are ready then,
 * scanning from a per-stage start that moves past the last peer taken
 * (round robin).  Only the taken peers are consumed and answered; the others
 * stay pending for a later run.  Each taken peer's rows are computed exactly
 * as in a run over all peers.  afd_window_status reports the taken peers in
 * served_mask.  layer_idx < 0 selects the layer from the headers and the
 * weights from the layer table (as afd_ffn_run_table; packed_weights is
 * ignored).  Nothing ready within the bound is AFD_ERR_TIMEOUT.  Errors:
 * AFD_ERR_INVALID (NULL window, stage out of range, max_peers outside
 * 1..num_peers, gather_us outside 0..poll_timeout_us, missing or misaligned
 * weights, layer_idx < 0 without a layer table). */
int32_t afd_ffn_run_ready(afd_window* w, int32_t stage, int32_t layer_idx, const void* packed_weights,
                          int32_t max_peers, int32_t gather_us, void* ffn_stream);

/* A fixed-length FFN loop captured once and replayed ("[RFC]: Async AFD for
 * Prefill on Ascend NPU", "FFN execution modes", graph mode: fixed-shape
 * buffers, a fixed number of iterations, receive steps that spin on the
 * device).  afd_ffn_loop_create captures n_runs consecutive
 * afd_ffn_run_table runs on stages first_stage, first_stage+1, ... (mod
 * ring_depth) from `stream` (a created stream, not the null stream) into a
 * HIP graph and instantiates it; nothing runs yet.  afd_ffn_loop_launch
 * enqueues one replay of all n_runs runs on `stream`: each run waits on the
 * device for its stage's inbound messages (peers pack on their own streams,
 * and may enqueue the packs of later runs once the return of the run that
 * last used the stage is unpacked on their stream), and takes its layer and
 * weights from the headers and the layer table at run time.  Sequence
 * numbers and mirrors live on the device, so replays continue where the
 * last run stopped.  The loop borrows the window: destroy the loop first.
 * Errors: AFD_ERR_INVALID (NULL arguments, n_runs < 1, first_stage out of
 * range, no layer table, per-kernel profiling on, null stream),
 * AFD_ERR_DEVICE (capture, instantiation or launch failed). */
typedef struct afd_ffn_loop afd_ffn_loop; /* opaque, library-owned */
int32_t afd_ffn_loop_create(afd_window* w, int32_t n_runs, int32_t first_stage, void* stream, afd_ffn_loop** out);
int32_t afd_ffn_loop_launch(afd_ffn_loop* loop, void* stream);
/* Frees the loop's graph; NULL is accepted. */
int32_t afd_ffn_loop_destroy(afd_ffn_loop* loop);

/* Connector-driven FFN loop ("[RFC]: Async AFD for Prefill on Ascend NPU",
 * "Asynchronous work-item contract" and "FFN execution modes": the FFN side
 * drains work items as they become ready, with bounded waits and a shutdown
 * sentinel, and no host round trip per item).  Enqueues n_items layer-table
 * runs on `stream` without any host synchronisation: item i on stage
 * (first_stage + i) % ring_depth, every peer of the stage (max_peers 0) or,
 * as afd_ffn_run_ready, at most max_peers ready peers after a gather window
 * of gather_us.  The first item that ends in shutdown, a timeout or an error
 * stops the loop on the device: the remaining items of the call consume
 * nothing and publish nothing (their stage status reads the stop status).
 * afd_ffn_serve_result synchronizes `stream` and reports the stop status
 * (AFD_OK: every item ran), the items that ran to completion, and the item
 * that stopped the loop (-1: none).  Peers may keep packing on their own
 * streams while the loop runs (each item waits on the device for its
 * stage's messages).  Errors: AFD_ERR_INVALID (NULL window, first_stage out
 * of range, n_items < 1, max_peers outside 0..num_peers, gather_us outside
 * 0..poll_timeout_us, no layer table), AFD_ERR_DEVICE. */
int32_t afd_ffn_serve(afd_window* w, int32_t first_stage, int32_t n_items, int32_t max_peers, int32_t gather_us,
                      void* stream);
int32_t afd_ffn_serve_result(afd_window* w, void* stream, int32_t* status, int32_t* items_done,
                             int32_t* stop_item);

/* Attention side, peer `peer`: wait (bounded, on the device) for the return
 * flag of (peer, stage), check its header (echo_seq must be the seq this
 * peer sent, num_tokens must equal seq_len), and copy the output rows
 * [seq_len][H] bf16 to `out` (device).  seq_len == 0: returns without waiting
 * (an empty message creates no wait; "Data flow").  Attention-routed
 * window: out[t] = rsf * sum over k, in k order, of w[t,k] * (returned row of
 * pair (t, k)) + the returned shared row, in fp32, rounded to bf16 (the FFN
 * side's combine).
 * Errors: AFD_ERR_SHAPE (seq_len differs from the packed length),
 * AFD_ERR_INVALID (also: a window that owns only part of the routed
 * experts, which afd_slot_unpack_ranks combines); device-side ones via
 * afd_peer_status. */
int32_t afd_slot_unpack(afd_window* w, int32_t peer, int32_t stage, int32_t seq_len, void* out,
                        void* peer_stream);

/* Attention side, expert-parallel segmentation ("[RFC]: Async GPU
 * Connector", "Data flow": the sender's combine takes every FFN rank's
 * returned rows): wins[0..n_wins) are the windows of all FFN ranks, whose
 * expert ranges [expert_offset, expert_offset + num_experts) must partition
 * [0, route_experts); at most one of them has a shared expert.  Waits for
 * the return of (peer, stage) in every window (bounded, on the device),
 * checks each header as afd_slot_unpack does, then writes
 * out[t] = rsf * sum over k, in k order, of w[t,k] * (the row of pair (t, k)
 * returned by the rank that owns its expert) + the shared row, in fp32,
 * rounded to bf16.  Every window must have the peer's message of seq_len
 * tokens in flight; the windows must agree on num_peers, ring_depth,
 * token_cap, hidden, top_k, route_experts, renormalize and
 * routed_scaling_factor.  1 <= n_wins <= 16.  Each window's afd_peer_status
 * reports its own wait; `out` is written only if every wait succeeded.
 * Errors: AFD_ERR_INVALID (arguments, windows that do not fit together),
 * AFD_ERR_SHAPE (seq_len differs from a window's packed length). */
int32_t afd_slot_unpack_ranks(afd_window* const* wins, int32_t n_wins, int32_t peer, int32_t stage,
                              int32_t seq_len, void* out, void* peer_stream);

/* Synchronize `stream` and read the status word of the last afd_ffn_run of
 * `stage`.  Off the hot path. */
int32_t afd_window_status(afd_window* w, int32_t stage, void* stream, afd_run_info* info);

/* Synchronize `stream` and read the status of the last unpack of (peer, stage). */
int32_t afd_peer_status(afd_window* w, int32_t peer, int32_t stage, void* stream, afd_run_info* info);

/* Host poll (debug path, "Risks": one D2H of all flags).  which = 0:
 * inbound flags, 1: return flags.  flags_out holds num_peers*ring_depth
 * int32.  Synchronous. */
int32_t afd_window_poll(afd_window* w, int32_t which, int32_t* flags_out);

/* Routing artefacts of the last afd_ffn_run (host copies, synchronizes
 * `stream`).  Any pointer may be NULL.  Sizes: ids/w/perm/inv
 * [T*top_k], counts [E], expert_offsets [E+1], split_offsets [P+1], where T
 * is split_offsets[P] (<= P*token_cap; pass buffers of that maximum size). */
int32_t afd_debug_routing(afd_window* w, void* stream, int32_t* ids, float* wts, int32_t* counts,
                          int32_t* expert_offsets, int32_t* perm, int32_t* inv,
                          int32_t* split_offsets);

/* Raw synchronous access to the allocation (tests inject corrupt headers or
 * stale flags from the host and inspect slots).  offset/bytes must lie in
 * [0, total_bytes). */
int32_t afd_debug_read(afd_window* w, int64_t offset, int64_t bytes, void* host_dst);
int32_t afd_debug_write(afd_window* w, int64_t offset, int64_t bytes, const void* host_src);

/* Per-kernel timing of afd_ffn_run with HIP events recorded on ffn_stream
 * between its launches.  mode: 0 off, 1 an event between every two kernels,
 * 2 events only around the two GEMM kernels (slots 4 and 5), 3 events only
 * around the gate/up GEMM (slot 4).  Each event record costs a few
 * microseconds between two launches; in modes 2 and 3 the other kernels run
 * back to back as without profiling.  afd_profile_read
 * returns the accumulated milliseconds per kernel slot and the number of
 * runs accumulated, then (reset != 0) clears them; it synchronizes the
 * pending events.  Kernel slot names: afd_profile_kernel_name(i),
 * i < AFD_PROFILE_SLOTS. */
#define AFD_PROFILE_SLOTS 8
int32_t afd_profile_enable(afd_window* w, int32_t mode);
int32_t afd_profile_read(afd_window* w, float* ms, int32_t n, int32_t* runs, int32_t reset);
const char* afd_profile_kernel_name(int32_t i);

/* Host header codec, the same code the kernels use.  encode writes
 * 12 + f->n_counts words (counts may be NULL: zeros).  decode checks magic,
 * version and that n_counts == expect_counts (AFD_ERR_HEADER otherwise). */
int32_t afd_header_encode(const afd_header_fields* f, const int32_t* counts, int32_t* words_out);
int32_t afd_header_decode(const int32_t* words, int32_t nwords, int32_t expect_counts,
                          afd_header_fields* out);

/* Thread-local text of the last error; never NULL. */
const char* afd_last_error(void);
const char* afd_status_string(int32_t status);
int32_t afd_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* AFD_H_ */
