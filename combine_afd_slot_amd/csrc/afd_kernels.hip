// afd_kernels.hip -- gfx950 kernels of the AFD FFN-rank hot path.
//
// One FFN run (afd_ffn_run) is seven launches on the FFN stream:
//   k_wait     bounded acquire-spin on the P inbound flags, header checks,
//              fan-in offsets (the fan-in itself is virtual: no copy)
//   k_route    one wavefront per token: top-k over the fp32 logits, weights,
//              per-chunk expert histogram, per-peer expert counts
//   k_scan     per-expert counts and offsets, stable per-chunk bases, the
//              GEMM group table and tile prefixes (all on the device)
//   k_permute  stable dispatch order: perm / inv
//   k_gemm<1>  grouped gate/up GEMM (MFMA bf16) with the SwiGLU epilogue
//   k_gemm<2>  grouped down GEMM (MFMA bf16)
//   k_combine  weighted combine + shared branch, bf16 rows written straight
//              into each peer's return slot, then the return flags
//
// Sources: "[RFC]: Async GPU Connector" (sections "Window and slot layout",
// "Data flow", "Attention gate and FFN expert compute"), "Data on the wire:
// tensors per layer and stage" (Steps 3-4), "[RFC]: Async AFD for Prefill on
// Ascend NPU" ("Asynchronous work-item contract", "FFN execution modes").
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "afd_internal.h"

namespace afd {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ inline float bf2f(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bf16, round to nearest even (NaN stays NaN).
__device__ inline uint32_t f2bf(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
    u += 0x7fffu + ((u >> 16) & 1u);
    return u >> 16;
}

__device__ inline char* slot_ptr(const DevCtx& c, char* win, int p, int s) {
    return win + c.slots_off + (int64_t)(p * c.R + s) * c.slot_bytes;
}

__device__ inline int peer_of(const DevCtx& c, int t) {
    int p = 0;
    while (p + 1 < c.P && c.off[p + 1] <= t) ++p;
    return p;
}

__device__ inline int ld_acquire(int* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void st_release(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Pack (attention side).  Payload first, then -- in a second launch on the
// same stream, so the whole payload is complete and written back -- the
// header and a release store of the flag ("Window and slot layout": payload
// and flag ordered on one stream; the flag value is the sender's seq).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_pack_payload(char* slot, int64_t o_rt, int64_t o_rx, int64_t o_si,
                                                      int64_t o_sx, const uint4* hidden, const float* logits,
                                                      int n, int H, int E) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nch = (int64_t)n * H / 8;
    uint4* rx = (uint4*)(slot + o_rx);
    uint4* sx = (uint4*)(slot + o_sx);
    for (int64_t i = gid; i < nch; i += stride) {
        uint4 v = hidden[i];
        rx[i] = v;
        sx[i] = v;
    }
    float* rt = (float*)(slot + o_rt);
    const int64_t nl = (int64_t)n * E;
    for (int64_t i = gid; i < nl; i += stride) rt[i] = logits[i];
    int* si = (int*)(slot + o_si);
    for (int64_t i = gid; i < n; i += stride) si[i] = (int)i;
}

__global__ void k_pack_publish(char* slot, int* flag, afd_header_fields f) {
    if (threadIdx.x == 0) {
        header_encode(f, nullptr, (int32_t*)slot);
        __threadfence();
        st_release(flag, f.seq);
    }
}

hipError_t launch_pack(const DevCtx& c, int peer, int stage, int layer, int seq_len, const void* hidden,
                       const float* logits, uint32_t flags, int seq, hipStream_t st) {
    char* slot = c.in_win + c.slots_off + (int64_t)(peer * c.R + stage) * c.slot_bytes;
    if (seq_len > 0) {
        int64_t work = (int64_t)seq_len * c.H / 8;
        int64_t lw = (int64_t)seq_len * c.E;
        if (lw > work) work = lw;
        int grid = (int)((work + 255) / 256);
        if (grid > 2048) grid = 2048;
        if (grid < 1) grid = 1;
        k_pack_payload<<<grid, 256, 0, st>>>(slot, c.foff[AFD_FIELD_ROUTE_TABLE], c.foff[AFD_FIELD_ROUTED_X],
                                             c.foff[AFD_FIELD_SHARED_IDX], c.foff[AFD_FIELD_SHARED_X],
                                             (const uint4*)hidden, logits, seq_len, c.H, c.E);
    }
    afd_header_fields f;
    f.flags = (int32_t)flags;
    f.seq = seq;
    f.echo_seq = 0;
    f.layer_idx = layer;
    f.stage_idx = stage;
    f.num_tokens = seq_len;
    f.routed_tokens = seq_len;
    f.shared_tokens = seq_len;
    f.src_peer = peer;
    f.n_counts = c.E;
    k_pack_publish<<<1, 64, 0, st>>>(slot + c.foff[AFD_FIELD_HEADER], (int*)c.in_win + peer * c.R + stage, f);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Unpack (attention side): bounded wait for the return flag, header checks
// (echo_seq is the seq this peer sent: "Risks and alternatives"), copy out.
// ---------------------------------------------------------------------------
__global__ void k_unpack_wait(DevCtx c, int p, int s, int expect_echo, int seq_len, long long timeout) {
    if (threadIdx.x != 0) return;
    const int idx = p * c.R + s;
    int* st = c.peer_status + idx * kStatusWords;
    int* flag = (int*)c.ret_win + idx;
    const int seen = c.seen_ret[idx];
    const long long t0 = wall_clock64();
    int f = seen;
    int err = AFD_OK;
    for (;;) {
        f = ld_acquire(flag);
        if (f != seen) break;
        if (wall_clock64() - t0 > timeout) {
            err = AFD_ERR_TIMEOUT;
            break;
        }
        __builtin_amdgcn_s_sleep(2);
    }
    if (err == AFD_OK) {
        afd_header_fields h;
        const int32_t* hw = (const int32_t*)(slot_ptr(c, c.ret_win, p, s) + c.foff[AFD_FIELD_HEADER]);
        err = header_decode(hw, c.E, &h);
        if (err == AFD_OK && (h.stage_idx != s || h.src_peer != p || h.seq != f)) err = AFD_ERR_HEADER;
        if (err == AFD_OK && h.echo_seq != expect_echo) err = AFD_ERR_SEQ;
        if (err == AFD_OK && h.num_tokens != seq_len) err = AFD_ERR_SHAPE;
        c.seen_ret[idx] = f;  // the message is consumed whatever it held
    }
    st[0] = err;
    st[1] = err == AFD_OK ? -1 : p;
    st[2] = f;
    st[3] = seq_len;
}

__global__ __launch_bounds__(256) void k_unpack_copy(const int* st, const uint4* src, uint4* out, int64_t nch) {
    if (*st != AFD_OK) return;
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nch; i += stride) out[i] = src[i];
}

hipError_t launch_unpack(const DevCtx& c, int peer, int stage, int seq_len, int expect_echo, void* out,
                         long long timeout_ticks, hipStream_t st) {
    k_unpack_wait<<<1, 64, 0, st>>>(c, peer, stage, expect_echo, seq_len, timeout_ticks);
    const int idx = peer * c.R + stage;
    const char* slot = c.ret_win + c.slots_off + (int64_t)idx * c.slot_bytes;
    int64_t nch = (int64_t)seq_len * c.H / 8;
    int grid = (int)((nch + 255) / 256);
    if (grid > 2048) grid = 2048;
    if (grid < 1) grid = 1;
    k_unpack_copy<<<grid, 256, 0, st>>>(c.peer_status + idx * kStatusWords,
                                        (const uint4*)(slot + c.foff[AFD_FIELD_ROUTED_X]), (uint4*)out, nch);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// a1: wait + fan-in.  Lane p spins (bounded) until inbound flag (p, s)
// differs from the FFN-side mirror -- the seq is monotonic per (peer, stage),
// so a change means a new message.  A work item is ready only when every
// peer has published ("Asynchronous work-item contract", items 1-2).  The
// headers are checked; the fan-in offsets are the exclusive scan of the
// peers' num_tokens ("Data on the wire", Steps 2-3).  Nothing is consumed
// unless every peer arrived with a valid header (or shutdown).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_wait(DevCtx c, int s, int layer, long long timeout) {
    __shared__ int s_flag[kMaxPeers], s_err[kMaxPeers], s_ntok[kMaxPeers], s_shut[kMaxPeers];
    const int p = threadIdx.x;
    int* st = c.run_status + s * kStatusWords;
    if (p < c.P) {
        const int idx = p * c.R + s;
        int* flag = (int*)c.in_win + idx;
        const int seen = c.seen_in[idx];
        const long long t0 = wall_clock64();
        int f = seen, err = AFD_OK, ntok = 0, shut = 0;
        for (;;) {
            f = ld_acquire(flag);
            if (f != seen) break;
            if (wall_clock64() - t0 > timeout) {
                err = AFD_ERR_TIMEOUT;
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        if (err == AFD_OK) {
            afd_header_fields h;
            const int32_t* hw = (const int32_t*)(slot_ptr(c, c.in_win, p, s) + c.foff[AFD_FIELD_HEADER]);
            err = header_decode(hw, c.E, &h);
            if (err == AFD_OK) err = inbound_check(h, p, s, layer, c.token_cap, f);
            if (err == AFD_OK) {
                ntok = h.num_tokens;
                shut = (h.flags & (int)AFD_FLAG_SHUTDOWN) != 0;
            }
        }
        s_flag[p] = f;
        s_err[p] = err;
        s_ntok[p] = ntok;
        s_shut[p] = shut;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        int status = AFD_OK, failed = -1, shut = 0;
        for (int q = 0; q < c.P; ++q) {
            if (s_err[q] != AFD_OK && status == AFD_OK) {
                status = s_err[q];
                failed = q;
            }
            shut |= s_shut[q];
        }
        if (status == AFD_OK && shut) status = AFD_SHUTDOWN;
        int T = 0;
        if (status == AFD_OK || status == AFD_SHUTDOWN) {
            c.off[0] = 0;
            for (int q = 0; q < c.P; ++q) {
                c.seen_in[q * c.R + s] = s_flag[q];
                c.cur_seq[q] = s_flag[q];
                c.off[q + 1] = c.off[q] + s_ntok[q];
            }
            T = c.off[c.P];
        }
        *c.Tptr = status == AFD_OK ? T : 0;
        *c.done_ctr = 0;
        st[0] = status;
        st[1] = failed;
        st[2] = s_flag[0];
        st[3] = status == AFD_OK ? T : 0;
    }
    for (int i = threadIdx.x; i < c.P * c.E; i += blockDim.x) c.peer_counts[i] = 0;
}

// ---------------------------------------------------------------------------
// a2: routing.  One wavefront per token; lane l holds logits e = l + 64*j.
// K rounds of a wavefront arg-max under the order (larger logit first, equal
// logits: lower expert index first; -0.0 equals +0.0 under float compare).
// Weights: w_k = exp(L_k - L_0) / sum_j exp(L_j - L_0) (softmax restricted to
// the top-k and renormalised); without renormalisation the denominator runs
// over all E experts.  ("[RFC]: Async GPU Connector", "Attention gate and FFN
// expert compute": grouped_topk with a single group.)
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void k_route(DevCtx c, int* status, int s) {
    if (*status != AFD_OK) return;
    const int T = *c.Tptr;
    const int t_begin = blockIdx.x * kRouteChunk;
    if (t_begin >= T) return;
    const int t_end = min(T, t_begin + kRouteChunk);
    __shared__ int hist[kMaxExperts];
    for (int e = threadIdx.x; e < c.E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = c.E, K = c.K;
    for (int t = t_begin + wave; t < t_end; t += 4) {
        const int p = peer_of(c, t);
        const int r = t - c.off[p];
        const char* slot = slot_ptr(c, c.in_win, p, s);
        const float* lg = (const float*)(slot + c.foff[AFD_FIELD_ROUTE_TABLE]) + (int64_t)r * E;
        float v[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            const float x = e < E ? lg[e] : -INFINITY;
            v[j] = x == x ? x : -INFINITY;  // NaN logits are out of contract; keep indices valid
        }
        unsigned selmask = 0;
        int my_id = 0;
        float my_val = 0.f;
        for (int k = 0; k < K; ++k) {
            float bv = -INFINITY;
            int bi = 0x7fffffff;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const int e = lane + 64 * j;
                if (e < E && !((selmask >> j) & 1u)) {
                    if (v[j] > bv || (v[j] == bv && e < bi)) {
                        bv = v[j];
                        bi = e;
                    }
                }
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) {
                const float ov = __shfl_xor(bv, o);
                const int oi = __shfl_xor(bi, o);
                if (ov > bv || (ov == bv && oi < bi)) {
                    bv = ov;
                    bi = oi;
                }
            }
            if (bi >= E) bi = 0;  // unreachable for K <= E; keeps every index in range
            if ((bi & 63) == lane) selmask |= 1u << (bi >> 6);
            if (lane == k) {
                my_id = bi;
                my_val = bv;
            }
        }
        const float m = __shfl(my_val, 0);
        const float ex = lane < K ? expf(my_val - m) : 0.f;
        float den = 0.f;
        if (c.renorm) {
            for (int k = 0; k < K; ++k) den += __shfl(ex, k);
        } else {
            float part = 0.f;
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const int e = lane + 64 * j;
                if (e < E) part += expf(v[j] - m);
            }
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
            den = part;
        }
        if (lane < K) {
            c.ids[(int64_t)t * K + lane] = my_id;
            c.wts[(int64_t)t * K + lane] = ex / den;
            atomicAdd(&hist[my_id], 1);
            atomicAdd(&c.peer_counts[p * E + my_id], 1);
        }
        if (lane == 0) {
            const int n_p = c.off[p + 1] - c.off[p];
            c.tok_src[t] = (uint64_t)(slot + c.foff[AFD_FIELD_ROUTED_X] + (int64_t)r * c.H * 2);
            c.sh_src[t] = (uint64_t)(slot + c.foff[AFD_FIELD_SHARED_X] + (int64_t)r * c.H * 2);
            int si = ((const int*)(slot + c.foff[AFD_FIELD_SHARED_IDX]))[r];
            if (si < 0 || si >= n_p) {
                atomicCAS(status, AFD_OK, AFD_ERR_HEADER);
                si = 0;
            }
            c.sh_dst[t] = c.off[p] + si;
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) c.blk_counts[blockIdx.x * E + e] = hist[e];
}

// ---------------------------------------------------------------------------
// a3 (first half): expert counts (bincount), expert offsets (exclusive
// cumsum), and for each chunk b and expert e the number of pairs of expert e
// in chunks before b -- the stable position base of that chunk.  Also the
// GEMM group table: group 0 is the shared expert (all T tokens), groups
// 1..E the routed experts in expert order; tile prefixes for both GEMMs.
// ---------------------------------------------------------------------------
__device__ int block_excl_scan_1024(int v, int* lds) {
    // 1024 threads; returns the exclusive prefix of v; lds holds 1024 ints.
    const int tid = threadIdx.x;
    lds[tid] = v;
    __syncthreads();
    for (int o = 1; o < 1024; o <<= 1) {
        const int add = tid >= o ? lds[tid - o] : 0;
        __syncthreads();
        lds[tid] += add;
        __syncthreads();
    }
    const int incl = lds[tid];
    __syncthreads();
    return incl - v;
}

__global__ __launch_bounds__(1024) void k_scan(DevCtx c, const int* status) {
    if (*status != AFD_OK) return;
    __shared__ int lds[1024];
    __shared__ int carry;
    const int T = *c.Tptr;
    const int nb = (T + kRouteChunk - 1) / kRouteChunk;
    const int E = c.E;
    const int tid = threadIdx.x;
    for (int e = tid; e < E; e += 1024) {
        int run = 0;
        for (int b = 0; b < nb; ++b) {
            const int v = c.blk_counts[b * E + e];
            c.blk_base[b * E + e] = run;
            run += v;
        }
        c.counts[e] = run;
    }
    __syncthreads();
    // expert offsets (E <= 1024)
    {
        const int v = tid < E ? c.counts[tid] : 0;
        const int ex = block_excl_scan_1024(v, lds);
        if (tid < E) c.eoff[tid] = ex;
        if (tid == E - 1) c.eoff[E] = ex + v;
    }
    __syncthreads();
    // group table and tile prefixes, in chunks of 1024 groups
    if (tid == 0) carry = 0;
    __syncthreads();
    const int nt1_r = (c.I + kBN / 2 - 1) / (kBN / 2);
    const int nt1_s = (c.Is + kBN / 2 - 1) / (kBN / 2);
    const int nt2 = (c.H + kBN - 1) / kBN;
    for (int pass = 0; pass < 2; ++pass) {
        int* tstart = pass == 0 ? c.tstart1 : c.tstart2;
        for (int base = 0; base < c.G; base += 1024) {
            const int j = base + tid;
            int tiles = 0;
            if (j < c.G) {
                const bool sh = c.has_shared && j == 0;
                const int e = j - c.has_shared;
                const int M = sh ? T : c.counts[e];
                const int mt = (M + kBM - 1) / kBM;
                tiles = mt * (pass == 0 ? (sh ? nt1_s : nt1_r) : nt2);
                if (pass == 0) {
                    c.grp_M[j] = M;
                    c.grp_row0[j] = sh ? 0 : c.eoff[e];
                }
            }
            const int ex = block_excl_scan_1024(tiles, lds);
            if (j < c.G) tstart[j] = carry + ex;
            __syncthreads();
            if (tid == 1023) carry += ex + tiles;
            __syncthreads();
        }
        if (tid == 0) {
            tstart[c.G] = carry;
            carry = 0;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// a3 (second half): the stable dispatch permutation ("[RFC]: Async GPU
// Connector", "Data flow": argsort(stable=True) over the flattened ids).
// Pair f = t*K + k goes to eoff[e] + #{f' < f : ids_f' = e}.  Chunk b holds
// its base per expert from k_scan; inside the chunk one thread per expert
// walks the chunk's pairs in flat order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_permute(DevCtx c, const int* status) {
    if (*status != AFD_OK) return;
    const int T = *c.Tptr;
    const int t0 = blockIdx.x * kRouteChunk;
    if (t0 >= T) return;
    const int t1 = min(T, t0 + kRouteChunk);
    const int K = c.K;
    const int np = (t1 - t0) * K;
    __shared__ int lids[kRouteChunk * kMaxTopK];
    for (int i = threadIdx.x; i < np; i += blockDim.x) lids[i] = c.ids[(int64_t)t0 * K + i];
    __syncthreads();
    for (int e = threadIdx.x; e < c.E; e += blockDim.x) {
        int pos = c.eoff[e] + c.blk_base[blockIdx.x * c.E + e];
        for (int i = 0; i < np; ++i) {
            if (lids[i] == e) {
                const int f = t0 * K + i;
                if (pos < T * K) c.perm[pos] = f;
                c.inv[f] = pos;
                ++pos;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// a4/a5/a6: grouped GEMMs on MFMA (v_mfma_f32_32x32x16_bf16).
//
// Tile = 128 rows x 128 columns, depth 64 per step, 256 threads = 4 waves in
// a 2x2 grid, each wave 64x64 = 2x2 MFMA blocks of 32x32.  A and B tiles are
// staged in LDS (double-buffered; 2 x 32 KB), K-contiguous, 16-byte chunks
// XOR-swizzled by row so that the 16-byte fragment reads of 8 or 16
// consecutive rows hit distinct banks.
//
// MODE 1 (gate/up + SwiGLU): A = token rows gathered straight from the
//   inbound slots (routed rows through perm and the per-token row address,
//   shared rows through the shared_x row address), B = 64 gate rows and the
//   same 64 up rows of W13, so each lane holds gate and up of the same
//   (row, column) and applies silu(g) * u in registers; h is stored bf16.
// MODE 2 (down): A = h rows of the group, B = 128 rows of W2; routed output
//   rows are stored bf16 in permuted order, shared rows fp32 in token order.
//
// Persistent: a grid of ~2 workgroups per CU walks the device-built tile
// list (group, row tile, column tile); groups are found by binary search in
// the tile prefix.  Rows past the group end and columns past the width load
// a valid row and are masked at the store.
// ---------------------------------------------------------------------------
__device__ inline int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <int MODE>
__global__ __launch_bounds__(256, 2) void k_gemm(DevCtx c, const int* status, Weights w) {
    if (*status != AFD_OK) return;
    __shared__ u32x4 lds[2][(kBM + kBN) * kBK / 8];
    const int* tstart = MODE == 1 ? c.tstart1 : c.tstart2;
    const int G = c.G;
    const int total = tstart[G];
    if (total < 0 || total > (MODE == 1 ? c.max_tiles1 : c.max_tiles2)) return;  // never with a sane plan
    const int T = *c.Tptr, npairs = T * c.K;
    const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
    const int wm = wid >> 1, wn = wid & 1;
    const int kc = tid & 7;
    const u32x4 zero4 = {0u, 0u, 0u, 0u};
    for (int tile = blockIdx.x; tile < total; tile += gridDim.x) {
        int lo = 0, hi = G;
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (tstart[mid] <= tile) lo = mid;
            else hi = mid;
        }
        const int j = lo;
        const bool sh = c.has_shared && j == 0;
        const int e = j - c.has_shared;
        const int M = c.grp_M[j], row0 = c.grp_row0[j];
        const int Ig = sh ? c.Is : c.I;
        const int local = tile - tstart[j];
        const int nt_per = MODE == 1 ? (Ig + kBN / 2 - 1) / (kBN / 2) : (c.H + kBN - 1) / kBN;
        const int mt = local / nt_per, nt = local - mt * nt_per;
        const int m0 = mt * kBM;
        const int Kdim = MODE == 1 ? c.H : Ig;

        const uint16_t* aptr[4];
        const uint16_t* bptr[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int r = (tid >> 3) + 32 * q;
            int m = m0 + r;
            if (m >= M) m = 0;
            if (MODE == 1) {
                if (sh) aptr[q] = (const uint16_t*)c.sh_src[m];
                else {
                    int tok = c.perm[min(row0 + m, npairs - 1)] / c.K;
                    tok = min(max(tok, 0), T - 1);
                    aptr[q] = (const uint16_t*)c.tok_src[tok];
                }
                int jj = nt * (kBN / 2) + (r & 63);
                if (jj >= Ig) jj = 0;
                const int wrow = (r >> 6) * Ig + jj;
                const uint16_t* base = sh ? w.ws13 : w.w13 + (int64_t)e * 2 * Ig * c.H;
                bptr[q] = base + (int64_t)wrow * c.H;
            } else {
                aptr[q] = sh ? c.hs + (int64_t)m * Ig : c.h + (int64_t)(row0 + m) * Ig;
                int n = nt * kBN + r;
                if (n >= c.H) n = 0;
                const uint16_t* base = sh ? w.ws2 : w.w2 + (int64_t)e * c.H * Ig;
                bptr[q] = base + (int64_t)n * Ig;
            }
        }

        f32x16 acc[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

        u32x4 ra[4], rb[4];
        const int nk = (Kdim + kBK - 1) / kBK;
        // global -> registers for depth step k0 (16-byte chunks; past Kdim: zeros)
#define AFD_GLOAD(k0)                                                      \
    {                                                                      \
        const int kx = (k0) + kc * 8;                                      \
        const bool ok = kx < Kdim;                                         \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) {                    \
            ra[q] = ok ? *(const u32x4*)(aptr[q] + kx) : zero4;            \
            rb[q] = ok ? *(const u32x4*)(bptr[q] + kx) : zero4;            \
        }                                                                  \
    }
        // registers -> LDS buffer `buf`, 16-byte chunks swizzled by row
#define AFD_SSTORE(buf)                                                    \
    {                                                                      \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) {                    \
            const int r = (tid >> 3) + 32 * q;                             \
            lds[buf][r * 8 + (kc ^ swz(r))] = ra[q];                       \
            lds[buf][(kBM + r) * 8 + (kc ^ swz(r))] = rb[q];               \
        }                                                                  \
    }
        AFD_GLOAD(0);
        AFD_SSTORE(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int buf = kt & 1;
            if (kt + 1 < nk) AFD_GLOAD((kt + 1) * kBK);
#pragma unroll
            for (int kk = 0; kk < kBK / 16; ++kk) {
                const int ch = kk * 2 + (lane >> 5);
                bf16x8 af[2], bfr[2];
#pragma unroll
                for (int mb = 0; mb < 2; ++mb) {
                    const int row = wm * 64 + mb * 32 + (lane & 31);
                    af[mb] = __builtin_bit_cast(bf16x8, lds[buf][row * 8 + (ch ^ swz(row))]);
                }
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const int brow = MODE == 1 ? nb * 64 + wn * 32 + (lane & 31) : wn * 64 + nb * 32 + (lane & 31);
                    bfr[nb] = __builtin_bit_cast(bf16x8, lds[buf][(kBM + brow) * 8 + (ch ^ swz(brow))]);
                }
#pragma unroll
                for (int mb = 0; mb < 2; ++mb)
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb)
                        acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[mb], bfr[nb], acc[mb][nb], 0, 0, 0);
            }
            if (kt + 1 < nk) AFD_SSTORE(buf ^ 1);
            __syncthreads();
        }
#undef AFD_GLOAD
#undef AFD_SSTORE

        // epilogue: lane holds column (lane & 31) of each 32x32 block, rows
        // (v/4)*8 + (lane/32)*4 + v%4
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
#pragma unroll
            for (int v = 0; v < 16; ++v) {
                const int row = wm * 64 + mb * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
                const int m = m0 + row;
                if (m >= M) continue;
                if (MODE == 1) {
                    const int jj = nt * (kBN / 2) + wn * 32 + (lane & 31);
                    if (jj < Ig) {
                        const float g = acc[mb][0][v], u = acc[mb][1][v];
                        const float hv = g / (1.f + expf(-g)) * u;
                        uint16_t* dst = sh ? c.hs + (int64_t)m * Ig : c.h + (int64_t)(row0 + m) * Ig;
                        dst[jj] = (uint16_t)f2bf(hv);
                    }
                } else {
#pragma unroll
                    for (int nb = 0; nb < 2; ++nb) {
                        const int n = nt * kBN + wn * 64 + nb * 32 + (lane & 31);
                        if (n < c.H) {
                            if (sh) c.ys[(int64_t)c.sh_dst[m] * c.H + n] = acc[mb][nb][v];
                            else c.y[(int64_t)(row0 + m) * c.H + n] = (uint16_t)f2bf(acc[mb][nb][v]);
                        }
                    }
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// a7: combine + split + publish.  out[t] = rsf * sum_k w[t,k] * y[inv[t*K+k]]
// + S[t] in fp32 (k in order), rounded to bf16 and written into row t - off[p]
// of peer p's return slot ("Data flow": weighted index_add_ combine with the
// shared branch added; "Data on the wire", Step 4: split back by seq_lens).
// The last workgroup to finish writes each non-empty peer's return header
// (num_tokens, echo_seq = the consumed seq, per-expert pair counts) and
// release-stores its return flag.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_combine(DevCtx c, const int* status, int s, int layer) {
    if (*status != AFD_OK) return;
    const int T = *c.Tptr;
    const int K = c.K, H = c.H, H8 = c.H / 8;
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        const int p = peer_of(c, t);
        const int r = t - c.off[p];
        uint4* dst = (uint4*)(slot_ptr(c, c.ret_win, p, s) + c.foff[AFD_FIELD_ROUTED_X] + (int64_t)r * H * 2);
        int pos[kMaxTopK];
        float wk[kMaxTopK];
#pragma unroll
        for (int k = 0; k < kMaxTopK; ++k) {
            pos[k] = k < K ? min(max(c.inv[(int64_t)t * K + k], 0), T * K - 1) : 0;
            wk[k] = k < K ? c.wts[(int64_t)t * K + k] : 0.f;
        }
        for (int ch = threadIdx.x; ch < H8; ch += blockDim.x) {
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
            for (int k = 0; k < kMaxTopK; ++k) {
                if (k < K) {
                    const uint4 v = *(const uint4*)(c.y + (int64_t)pos[k] * H + ch * 8);
                    const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int i = 0; i < 4; ++i) {
                        acc[2 * i] += wk[k] * bf2f(u[i] & 0xffffu);
                        acc[2 * i + 1] += wk[k] * bf2f(u[i] >> 16);
                    }
                }
            }
            float o[8];
            if (c.has_shared) {
                const float4* sp = (const float4*)(c.ys + (int64_t)t * H + ch * 8);
                const float4 s0 = sp[0], s1 = sp[1];
                const float sv[8] = {s0.x, s0.y, s0.z, s0.w, s1.x, s1.y, s1.z, s1.w};
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = c.rsf * acc[i] + sv[i];
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = c.rsf * acc[i];
            }
            uint4 out;
            out.x = f2bf(o[0]) | (f2bf(o[1]) << 16);
            out.y = f2bf(o[2]) | (f2bf(o[3]) << 16);
            out.z = f2bf(o[4]) | (f2bf(o[5]) << 16);
            out.w = f2bf(o[6]) | (f2bf(o[7]) << 16);
            dst[ch] = out;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        __threadfence();
        const int prev = atomicAdd(c.done_ctr, 1);
        if (prev == (int)gridDim.x - 1) {
            __threadfence();
            for (int p = 0; p < c.P; ++p) {
                const int n_p = c.off[p + 1] - c.off[p];
                if (n_p == 0) continue;  // an empty message gets no reply and creates no wait
                const int idx = p * c.R + s;
                const int rs = c.ret_seq[idx] + 1;
                c.ret_seq[idx] = rs;
                afd_header_fields f;
                f.flags = 0;
                f.seq = rs;
                f.echo_seq = c.cur_seq[p];
                f.layer_idx = layer;
                f.stage_idx = s;
                f.num_tokens = n_p;
                f.routed_tokens = n_p;
                f.shared_tokens = n_p;
                f.src_peer = p;
                f.n_counts = c.E;
                header_encode(f, c.peer_counts + p * c.E,
                              (int32_t*)(slot_ptr(c, c.ret_win, p, s) + c.foff[AFD_FIELD_HEADER]));
                __threadfence();
                st_release((int*)c.ret_win + idx, rs);
            }
            *c.done_ctr = 0;
        }
    }
}

// ---------------------------------------------------------------------------
hipError_t launch_ffn(const DevCtx& c, int stage, int layer, const Weights& w, long long timeout_ticks, int num_cu,
                      hipEvent_t* ev, hipStream_t st) {
    int* status = c.run_status + stage * kStatusWords;
    const int Tmax = c.P * c.token_cap;
    int slot = 0;
    auto mark = [&]() {
        if (ev) (void)hipEventRecord(ev[slot], st);
        ++slot;
    };
    mark();
    k_wait<<<1, 64, 0, st>>>(c, stage, layer, timeout_ticks);
    mark();
    if (c.E <= 64) k_route<1><<<c.NB, 256, 0, st>>>(c, status, stage);
    else if (c.E <= 128) k_route<2><<<c.NB, 256, 0, st>>>(c, status, stage);
    else if (c.E <= 256) k_route<4><<<c.NB, 256, 0, st>>>(c, status, stage);
    else if (c.E <= 512) k_route<8><<<c.NB, 256, 0, st>>>(c, status, stage);
    else k_route<16><<<c.NB, 256, 0, st>>>(c, status, stage);
    mark();
    k_scan<<<1, 1024, 0, st>>>(c, status);
    mark();
    k_permute<<<c.NB, 256, 0, st>>>(c, status);
    mark();
    k_gemm<1><<<num_cu * 2, 256, 0, st>>>(c, status, w);
    mark();
    k_gemm<2><<<num_cu * 2, 256, 0, st>>>(c, status, w);
    mark();
    int cgrid = Tmax < num_cu * 4 ? Tmax : num_cu * 4;
    if (cgrid < 1) cgrid = 1;
    k_combine<<<cgrid, 256, 0, st>>>(c, status, stage, layer);
    mark();
    return hipGetLastError();
}

}  // namespace afd
