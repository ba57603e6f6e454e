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
typedef float f32x4 __attribute__((ext_vector_type(4)));

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
        st[0] = status;
        st[1] = failed;
        st[2] = s_flag[0];
        st[3] = status == AFD_OK ? T : 0;
    }
}

// ---------------------------------------------------------------------------
// Block-wide exclusive prefix sum of one int per thread (blockDim a multiple
// of 64, at most 1024).  `sh` holds 16 ints.
// ---------------------------------------------------------------------------
__device__ int block_excl_scan(int v, int* sh) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) sh[wid] = x;
    __syncthreads();
    int wbase = 0;
    for (int w = 0; w < wid; ++w) wbase += sh[w];
    __syncthreads();
    return x + wbase - v;
}

// ---------------------------------------------------------------------------
// Routing chunks: kRouteChunk consecutive tokens of one peer (a peer's last
// chunk may be shorter).  Chunks are numbered in fan-in token order, so the
// flat pair order f = t*K + k runs through the chunks in order.
// ---------------------------------------------------------------------------
__device__ inline int num_chunks(const DevCtx& c) {
    int n = 0;
    for (int q = 0; q < c.P; ++q) n += (c.off[q + 1] - c.off[q] + kRouteChunk - 1) / kRouteChunk;
    return n;
}

__device__ inline bool chunk_range(const DevCtx& c, int b, int& t0, int& t1, int& p) {
    int cum = 0;
    for (int q = 0; q < c.P; ++q) {
        const int n = c.off[q + 1] - c.off[q];
        const int nc = (n + kRouteChunk - 1) / kRouteChunk;
        if (b < cum + nc) {
            p = q;
            t0 = c.off[q] + (b - cum) * kRouteChunk;
            t1 = min(c.off[q + 1], t0 + kRouteChunk);
            return true;
        }
        cum += nc;
    }
    return false;
}

// ---------------------------------------------------------------------------
// a2: routing.  One wavefront per token; each workgroup takes one chunk.
// The order is (larger logit first, equal logits: lower expert index first;
// -0.0 equals +0.0 under float compare).  The wave stages the token's E
// logits in LDS and every lane ranks its own logits against all E of them;
// the K experts of rank < K are the top-K, and rank k is the k-th selected.
// Weights: w_k = exp(L_k - L_max) / sum over the selected of exp(L - L_max)
// (the softmax restricted to the top-K and renormalised); without
// renormalisation the denominator runs over all E experts.  ("[RFC]: Async
// GPU Connector", "Attention gate and FFN expert compute": grouped_topk with
// a single group.)  The chunk's expert histogram goes to blk_counts[e][b].
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(256) void k_route(DevCtx c, int* status, int s) {
    if (*status != AFD_OK) return;
    int t_begin, t_end, p;
    if (!chunk_range(c, blockIdx.x, t_begin, t_end, p)) return;
    constexpr int TPW = kRouteChunk / 4;
    __shared__ int hist[kMaxExperts];
    __shared__ float lv[4][kMaxExperts];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int E = c.E, K = c.K;
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    const char* slot = slot_ptr(c, c.in_win, p, s);
    float v[TPW][EPL];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = t_begin + wave * TPW + i;
        const float* lg = (const float*)(slot + c.foff[AFD_FIELD_ROUTE_TABLE]) +
                          (int64_t)(min(t, t_end - 1) - c.off[p]) * E;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            const float x = e < E ? lg[e] : -INFINITY;
            v[i][j] = x == x ? x : -INFINITY;  // NaN logits are out of contract; keep the order total
        }
    }
    __syncthreads();  // hist zeroed
    float* L = lv[wave];
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
        const int t = t_begin + wave * TPW + i;
        if (t >= t_end) break;
#pragma unroll
        for (int j = 0; j < EPL; ++j)
            if (lane + 64 * j < E) L[lane + 64 * j] = v[i][j];
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        int rank[EPL];
#pragma unroll
        for (int j = 0; j < EPL; ++j) rank[j] = 0;
        for (int q = 0; q < E; ++q) {
            const float x = L[q];
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                const int e = lane + 64 * j;
                rank[j] += (x > v[i][j] || (x == v[i][j] && q < e)) ? 1 : 0;
            }
        }
        // the maximum is the value of rank 0
        float m = -INFINITY;
#pragma unroll
        for (int j = 0; j < EPL; ++j) m = fmaxf(m, (lane + 64 * j < E) ? v[i][j] : -INFINITY);
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
        float ex[EPL], part = 0.f;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            const bool sel = e < E && rank[j] < K;
            ex[j] = (e < E) ? expf(v[i][j] - m) : 0.f;
            if (c.renorm ? sel : (e < E)) part += ex[j];
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o);
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            if (e < E && rank[j] < K) {
                c.ids[(int64_t)t * K + rank[j]] = e;
                c.wts[(int64_t)t * K + rank[j]] = ex[j] / part;
                atomicAdd(&hist[e], 1);
            }
        }
        if (lane == 0) {
            const int r = t - c.off[p];
            c.tok_src[t] = (uint64_t)(slot + c.foff[AFD_FIELD_ROUTED_X] + (int64_t)r * c.H * 2);
            c.sh_src[t] = (uint64_t)(slot + c.foff[AFD_FIELD_SHARED_X] + (int64_t)r * c.H * 2);
            // one FFN replica owns every shared row: shared_idx must be 0..n_p-1
            const int si = ((const int*)(slot + c.foff[AFD_FIELD_SHARED_IDX]))[r];
            if (si != r) atomicCAS(status, AFD_OK, AFD_ERR_HEADER);
        }
        __builtin_amdgcn_wave_barrier();  // L is rewritten by the next token
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) c.blk_counts[(int64_t)e * c.NB + blockIdx.x] = hist[e];
}

// ---------------------------------------------------------------------------
// a3 (first half): one workgroup per expert e scans its column of chunk
// histograms: blk_base[e][b] = number of pairs of expert e in chunks before
// b (the stable position base of chunk b inside expert e's group),
// counts[e] = the column total (bincount), and peer_counts[p][e] = the
// column sum over peer p's chunks (the per-peer expert counts that return in
// each peer's header).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_scan(DevCtx c, const int* status) {
    if (*status != AFD_OK) return;
    __shared__ int sh[16];
    __shared__ int pc[kMaxPeers];
    __shared__ int pchunk[kMaxPeers + 1];
    const int e = blockIdx.x;
    if (threadIdx.x == 0) {
        pchunk[0] = 0;
        for (int q = 0; q < c.P; ++q)
            pchunk[q + 1] = pchunk[q] + (c.off[q + 1] - c.off[q] + kRouteChunk - 1) / kRouteChunk;
    }
    if (threadIdx.x < kMaxPeers) pc[threadIdx.x] = 0;
    __syncthreads();
    const int nb = pchunk[c.P];
    const int* col = c.blk_counts + (int64_t)e * c.NB;
    int* base = c.blk_base + (int64_t)e * c.NB;
    const int per = (nb + 255) / 256;
    const int b0 = threadIdx.x * per, b1 = min(nb, b0 + per);
    int sum = 0;
    for (int b = b0; b < b1; ++b) sum += col[b];
    int run = block_excl_scan(sum, sh);
    int q = 0;
    for (int b = b0; b < b1; ++b) {
        const int v = col[b];
        base[b] = run;
        run += v;
        while (q + 1 < c.P && pchunk[q + 1] <= b) ++q;
        if (v) atomicAdd(&pc[q], v);
    }
    if (threadIdx.x == 255) c.counts[e] = run;
    __syncthreads();
    for (int qq = threadIdx.x; qq < c.P; qq += 256) c.peer_counts[qq * c.E + e] = pc[qq];
}

// ---------------------------------------------------------------------------
// GEMM tile plan (run by one workgroup of 256 threads).  Group j: 0 is the
// shared expert over all T tokens, 1..E the routed experts.  A group of M
// rows has ceil(M/kBM) row tiles and, for the gate/up GEMM, ceil(Ig/(kBN/2))
// column tiles (kBN/2 gate + the same kBN/2 up rows of W13), for the down
// GEMM ceil(H/kBN).  Tiles are numbered group-major, column tile next, row
// tile fastest (row tiles of one column tile share their weight rows).  The
// cost of a tile is (32-row blocks it holds) x (depth steps); the tile list
// is cut into kXcds segments of equal cost, one per XCD.
// ---------------------------------------------------------------------------
struct PlanGroup {
    int M, mt, blocks, nt, nk;
};

__device__ inline PlanGroup plan_group(const DevCtx& c, int T, const int* s_eoff, int j, int mode) {
    PlanGroup g;
    const bool shd = c.has_shared && j == 0;
    const int e = j - c.has_shared;
    const int Ig = shd ? c.Is : c.I;
    g.M = shd ? T : s_eoff[e + 1] - s_eoff[e];
    g.mt = (g.M + kBM - 1) / kBM;
    g.blocks = (g.M + 31) / 32;
    g.nt = mode == 1 ? (Ig + kBN / 2 - 1) / (kBN / 2) : (c.H + kBN - 1) / kBN;
    g.nk = mode == 1 ? (c.H + kBK - 1) / kBK : (Ig + kBK - 1) / kBK;
    return g;
}

__device__ void plan_tiles(const DevCtx& c, int T, const int* s_eoff, int* sh) {
    if (threadIdx.x < 2 * kXcds) c.tctr[threadIdx.x] = 0;
    __shared__ int s_t[2][kMaxExperts + 2];
    __shared__ long long s_c[2][kMaxExperts + 2];
    const int tid = threadIdx.x, G = c.G;
    const int per = (G + 255) / 256;
    const int j0 = tid * per, j1 = min(G, j0 + per);
    for (int mode = 1; mode <= 2; ++mode) {
        int tiles = 0;
        long long cost = 0;
        for (int j = j0; j < j1; ++j) {
            const PlanGroup g = plan_group(c, T, s_eoff, j, mode);
            tiles += g.mt * g.nt;
            cost += (long long)g.nt * g.blocks * g.nk;
            if (mode == 1) {
                c.grp_M[j] = g.M;
                c.grp_row0[j] = (c.has_shared && j == 0) ? 0 : s_eoff[j - c.has_shared];
            }
        }
        // tile and cost prefixes over groups (costs fit in 31 bits for every
        // configuration the window accepts; scanned in two int halves anyway)
        int rt = block_excl_scan(tiles, sh);
        int rc_lo = block_excl_scan((int)(cost & 0xffff), sh);
        int rc_hi = block_excl_scan((int)(cost >> 16), sh);
        long long rc = ((long long)rc_hi << 16) + rc_lo;
        for (int j = j0; j < j1; ++j) {
            const PlanGroup g = plan_group(c, T, s_eoff, j, mode);
            s_t[mode - 1][j] = rt;
            s_c[mode - 1][j] = rc;
            rt += g.mt * g.nt;
            rc += (long long)g.nt * g.blocks * g.nk;
        }
        if (tid == 255) {
            s_t[mode - 1][G] = rt;
            s_c[mode - 1][G] = rc;
        }
        __syncthreads();
        int* tstart = mode == 1 ? c.tstart1 : c.tstart2;
        int2* tinfo = mode == 1 ? c.tinfo1 : c.tinfo2;
        const int maxt = mode == 1 ? c.max_tiles1 : c.max_tiles2;
        for (int j = tid; j <= G; j += 256) tstart[j] = s_t[mode - 1][j];
        const int total = s_t[mode - 1][G];
        // each group's tiles, column tile outer, row tile inner; the threads
        // of a wave split one group's tiles between them
        const int lane = tid & 63, wave = tid >> 6;
        for (int j = wave; j < G; j += 4) {
            const PlanGroup g = plan_group(c, T, s_eoff, j, mode);
            const int n = g.mt * g.nt, t0 = s_t[mode - 1][j];
            for (int i = lane; i < n; i += 64) {
                const int nt = i / g.mt, mt = i - nt * g.mt;
                if (t0 + i < maxt) tinfo[t0 + i] = make_int2(j, (mt << 16) | nt);
            }
        }
        // segment x starts at the first tile whose cost prefix is >= x*C/kXcds
        int* seg = mode == 1 ? c.seg1 : c.seg2;
        if (tid <= kXcds) {
            const long long C = s_c[mode - 1][G];
            const long long S = C * tid / kXcds;
            int res = total;
            if (tid < kXcds && S < C) {
                int lo = 0, hi = G;
                while (hi - lo > 1) {
                    const int mid = (lo + hi) >> 1;
                    if (s_c[mode - 1][mid] <= S) lo = mid;
                    else hi = mid;
                }
                // skip groups with no tiles that share the same cost start
                while (lo + 1 < G && s_c[mode - 1][lo + 1] <= S) ++lo;
                const PlanGroup g = plan_group(c, T, s_eoff, lo, mode);
                const long long u = (S - s_c[mode - 1][lo] + g.nk - 1) / g.nk;  // in 32-row blocks
                int nt = (int)(u / g.blocks);
                const int rem = (int)(u - (long long)nt * g.blocks);
                int mt = (rem + kBM / 32 - 1) / (kBM / 32);
                if (mt >= g.mt) {
                    ++nt;
                    mt = 0;
                }
                res = s_t[mode - 1][lo] + nt * g.mt + mt;
                if (res > total) res = total;
            }
            seg[tid] = res;
        }
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// a3 (second half): the stable dispatch permutation ("[RFC]: Async GPU
// Connector", "Data flow": argsort(stable=True) over the flattened ids,
// bincount, cumsum).  Each workgroup scans the expert counts into the expert
// offsets (workgroup 0 also publishes them, with the GEMM group table: group
// 0 is the shared expert over all T tokens, groups 1..E the routed experts,
// and the tile prefixes of both GEMMs).  Pair f = t*K + k goes to
// eoff[e] + #{f' < f : ids_f' = e}: the chunk's base per expert from k_scan,
// then, inside the chunk, one thread per expert walks the pairs in flat order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_permute(DevCtx c, const int* status) {
    if (*status != AFD_OK) return;
    const int T = *c.Tptr;
    int t0 = 0, t1 = 0, p = 0;
    const bool have = chunk_range(c, blockIdx.x, t0, t1, p);
    if (blockIdx.x != 0 && !have) return;
    __shared__ int sh[16];
    __shared__ int s_eoff[kMaxExperts + 1];
    __shared__ int lids[kRouteChunk * kMaxTopK];
    const int E = c.E, K = c.K, tid = threadIdx.x;
    {
        const int per = (E + 255) / 256;
        const int e0 = tid * per, e1 = min(E, e0 + per);
        int sum = 0;
        for (int e = e0; e < e1; ++e) sum += c.counts[e];
        int run = block_excl_scan(sum, sh);
        for (int e = e0; e < e1; ++e) {
            s_eoff[e] = run;
            run += c.counts[e];
        }
        if (tid == 255) s_eoff[E] = run;
    }
    __syncthreads();
    if (blockIdx.x == 0) {
        for (int e = tid; e <= E; e += 256) c.eoff[e] = s_eoff[e];
        plan_tiles(c, T, s_eoff, sh);
        if (!have) return;
    }
    __shared__ uint64_t ltok[kRouteChunk];
    const int np = (t1 - t0) * K;
    for (int i = tid; i < np; i += 256) lids[i] = c.ids[(int64_t)t0 * K + i];
    if (tid < t1 - t0) ltok[tid] = c.tok_src[t0 + tid];
    __syncthreads();
    const int npairs = T * K;
    for (int e = tid; e < E; e += 256) {
        int pos = s_eoff[e] + c.blk_base[(int64_t)e * c.NB + blockIdx.x];
        for (int i = 0; i < np; ++i) {
            if (lids[i] == e) {
                const int f = t0 * K + i;
                if (pos < npairs) {
                    c.perm[pos] = f;
                    c.psrc[pos] = ltok[i / K];
                }
                c.inv[f] = pos;
                ++pos;
            }
        }
    }
}

// ---------------------------------------------------------------------------
// a4/a5/a6: grouped GEMMs on MFMA (v_mfma_f32_32x32x16_bf16).
//
// A tile is up to 512 token rows of one group (16 blocks of 32) x 128
// weight rows, 64 deep per step.  1024 threads = 16 waves in 8 (token) x 2
// (weight) groups: wave (wm, wn) owns the token blocks wm and wm+8 (so a
// partly filled tile keeps the waves balanced; blocks past the group's end
// are skipped) and two 32-row weight blocks.  A group of at most 512 rows is
// one row tile, so every weight row is streamed from HBM once per group; the
// group's token rows are re-read from L2 by its column tiles.  Operands are K-contiguous rows
// (token rows of X or h, weight rows of W13 / W2), so every MFMA fragment is
// one 16-byte LDS read.  The weight fragment is the MFMA's first operand, so
// a lane's accumulators hold one token row (lane % 32) and 4 runs of 4
// consecutive output columns -- 8/16-byte stores in the epilogue.
//
// Global -> LDS: direct-to-LDS loads (global_load_lds_dwordx4), so staging
// costs no registers.  Two 80 KB stages (all 160 KB of LDS) are filled
// alternately, one step ahead: a wave waits on its own vector-memory counter
// for the stage it is about to read, then the workgroup barrier makes every
// wave's loads of that stage visible and frees the other stage for the next
// loads.  A 64-deep step covers each row's 128 bytes, one full L2 line.  One
// load instruction of a wave fills 1 KB = 8 rows x 128 B; lane i fetches row
// i/8, LDS chunk i%8 holding logical chunk (i%8) ^ swz(row), an XOR swizzle
// that keeps the 16-byte fragment reads of 8 or 16 consecutive rows on
// distinct banks.  Token-row load instructions whose 16 rows all lie past the group's
// end are not issued.
//
// MODE 1 (gate/up + SwiGLU): token rows are read straight from the inbound
//   slots (routed rows through the per-pair row address, shared rows through
//   the shared_x row address); the weight rows are 64 gate rows and the
//   same 64 up rows of W13, and wave wn takes gate block wn and up block wn,
//   so each lane holds gate and up of the same (row, column) and applies
//   silu(g) * u in registers; h is stored bf16.
// MODE 2 (down): token rows are the group's h rows, weight rows 128 rows of
//   W2; routed output rows are stored bf16 in permuted order, shared rows
//   fp32 in token order.
//
// Persistent: one workgroup per CU; the device-built tile list is cut into
// 8 segments of equal cost, one per XCD (workgroups are dispatched to the
// XCDs round-robin), whose workgroups take its tiles in turn.  Rows past the
// group end and columns past the width load a valid row and are masked at
// the store; depth past K loads zeros.
// ---------------------------------------------------------------------------
__device__ inline int swz8(int r) { return (r ^ (r >> 3)) & 7; }

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline void dma16(const void* g, lds_ptr_t l) { __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0); }

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
#define AFD_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))

__device__ inline void wait_vmcnt_upto(int n) {
    // n is wave-uniform; the instruction needs an immediate
    switch (n) {
        case 0: AFD_WAIT_VMCNT(0); break;
        case 1: AFD_WAIT_VMCNT(1); break;
        case 2: AFD_WAIT_VMCNT(2); break;
        case 3: AFD_WAIT_VMCNT(3); break;
        case 4: AFD_WAIT_VMCNT(4); break;
        case 5: AFD_WAIT_VMCNT(5); break;
        case 6: AFD_WAIT_VMCNT(6); break;
        case 7: AFD_WAIT_VMCNT(7); break;
        case 8: AFD_WAIT_VMCNT(8); break;
        default: AFD_WAIT_VMCNT(9); break;
    }
}

constexpr int kWaves = kGemmThreads / 64;                 // 16
constexpr int kRowBytes = kBK * 2;                        // 128
constexpr int kAStageBytes = kBM * kRowBytes;             // 64 KB
constexpr int kStageBytes = (kBM + kBN) * kRowBytes;      // 80 KB
constexpr int kRowsPerInstr = 1024 / kRowBytes;           // 8
constexpr int kAInstr = kBM / kRowsPerInstr / kWaves;     // 4 token-row instructions per wave
constexpr int kBTotal = kBN / kRowsPerInstr;              // 16 weight-row instructions per stage
constexpr int kChunks = kRowBytes / 16;                   // 8
constexpr int kWaveRows = kWaves / 2;                     // 8 token-block groups

template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm(DevCtx c, const int* status, Weights w) {
    if (*status != AFD_OK) return;
    __shared__ __attribute__((aligned(1024))) char smem[kStages * kStageBytes];
    const int2* tinfo = MODE == 1 ? c.tinfo1 : c.tinfo2;
    const int* seg = MODE == 1 ? c.seg1 : c.seg2;
    const int total = (MODE == 1 ? c.tstart1 : c.tstart2)[c.G];
    if (total <= 0 || total > (MODE == 1 ? c.max_tiles1 : c.max_tiles2)) return;  // nothing, or an insane plan
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wid >> 1, wn = wid & 1;

    // Tiles are taken dynamically: workgroup b starts on the segment of its
    // XCD (b % kXcds) and, when that is drained, continues with the next
    // segments.  Thread 0 owns the grabbing; each grab is issued a whole tile
    // before it is needed and the index is broadcast through LDS at the tile
    // boundary.
    int* ctr = c.tctr + (MODE - 1) * kXcds;
    int xi = (int)(blockIdx.x % kXcds), tries = 0, pend = 0;
    auto grab_slow = [&]() -> int {  // thread 0 only: next tile, or -1 when all are taken
        while (tries < kXcds) {
            const int lo = min(max(seg[xi], 0), total), hi = min(max(seg[xi + 1], lo), total);
            const int t = lo + atomicAdd(&ctr[xi], 1);
            if (t < hi) return t;
            xi = (xi + 1) % kXcds;
            ++tries;
        }
        return -1;
    };
    int* bcast = (int*)smem;  // free at tile boundaries
    if (tid == 0) {
        const int t = grab_slow();
        bcast[0] = t;
        if (t >= 0) pend = atomicAdd(&ctr[xi], 1);  // the following tile, resolved a tile later
    }
    __syncthreads();
    int tile = bcast[0];
    __syncthreads();

    const int lrow = lane >> 3;   // row inside a load instruction
    const int pc = lane & 7;      // LDS chunk of this lane
    // chunk fetched by this lane: (i%8) ^ swz8(row) for row = 8*instr + lrow,
    // which is (i%8) ^ lrow ^ (instr & 7)
    const int s_lane = pc ^ lrow;
    // weight fragment rows inside a stage (first MFMA operand)
    int wrl[2];
#pragma unroll
    for (int nb = 0; nb < 2; ++nb)
        wrl[nb] = MODE == 1 ? nb * (kBN / 2) + wn * 32 + (lane & 31) : (wn * 2 + nb) * 32 + (lane & 31);
    const bool has_b = wid < kBTotal;  // every wave loads one weight-row instruction

    while (tile >= 0) {
        const int2 ti = tinfo[tile];
        const int j = ti.x, mt = ti.y >> 16, nt = ti.y & 0xffff;
        const bool sh = c.has_shared && j == 0;
        const int e = j - c.has_shared;
        const int M = c.grp_M[j], row0 = c.grp_row0[j];
        const int Ig = sh ? c.Is : c.I;
        const int m0 = mt * kBM;
        const int rows = min(kBM, M - m0);         // valid token rows of this tile (>= 1)
        const int nblk = (rows + 31) >> 5;         // 32-row token blocks to compute
        const int Kdim = MODE == 1 ? c.H : Ig;
        const int nk = (Kdim + kBK - 1) / kBK;
        // token-row load instructions of this wave: rows (wid*kAInstr + q)*16 ..
        const int na = min(max((rows + kRowsPerInstr - 1) / kRowsPerInstr - wid * kAInstr, 0), kAInstr);
        const int nw = na + (has_b ? 1 : 0);

        // Row addresses as 32-bit byte offsets from a per-tile base (the
        // window and every buffer stay below 4 GiB: checked at create).
        const char* abase;
        if (MODE == 1) abase = c.in_win;
        else abase = (const char*)(sh ? c.hs : c.h);
        const char* bbase;
        if (MODE == 1) bbase = (const char*)(sh ? w.ws13 : w.w13 + (int64_t)e * 2 * Ig * c.H);
        else bbase = (const char*)(sh ? w.ws2 : w.w2 + (int64_t)e * c.H * Ig);
        uint32_t aoff[kAInstr], boff0 = 0;
#pragma unroll
        for (int q = 0; q < kAInstr; ++q) {
            const int r = (wid * kAInstr + q) * kRowsPerInstr + lrow;
            int m = m0 + r;
            if (m >= M) m = m0;
            if (MODE == 1) aoff[q] = (uint32_t)((sh ? c.sh_src[m] : c.psrc[row0 + m]) - (uint64_t)c.in_win);
            else aoff[q] = (uint32_t)(((int64_t)(sh ? m : row0 + m) * Ig) * 2);
        }
        {
            const int r = wid * kRowsPerInstr + lrow;  // weight row of this wave's instruction
            if (MODE == 1) {
                int jj = nt * (kBN / 2) + (r & (kBN / 2 - 1));
                if (jj >= Ig) jj = 0;
                boff0 = (uint32_t)((int64_t)(((r & (kBN - 1)) / (kBN / 2)) * Ig + jj) * c.H * 2);
            } else {
                int n = nt * kBN + (r & (kBN - 1));
                if (n >= c.H) n = 0;
                boff0 = (uint32_t)((int64_t)n * Ig * 2);
            }
        }
        const int kfull = Kdim / kBK;                // steps whose every chunk lies inside K
        const uint32_t row_lim = (uint32_t)Kdim * 2;  // bytes of a row

        // byte offset of this lane's chunk: (s_lane ^ (instr & 7)) * 16 =
        // (16 * s_lane) ^ (16 * (instr & 7)), the second term wave-uniform
        const uint32_t lco = (uint32_t)(s_lane * 16);

        // A depth step past the end of K (K not a multiple of 64) loads each
        // row's last 16 bytes in place of the missing chunks -- valid, finite
        // data -- and the token fragments of those chunks are zeroed before
        // the MFMA, so they contribute nothing.
        const uint32_t tail_clamp = row_lim - 16;
#define AFD_ISSUE(kt, st)                                                                            \
    {                                                                                                \
        char* sb_ = smem + (st) * kStageBytes;                                                       \
        const uint32_t kb_ = (uint32_t)(kt) * (kBK * 2);                                             \
        const bool full_ = (kt) < kfull;                                                             \
        _Pragma("unroll") for (int q = 0; q < kAInstr; ++q) if (q < na) {                            \
            uint32_t cc_ = kb_ + (lco ^ (uint32_t)(((wid * kAInstr + q) & 7) * 16));                 \
            if (!full_) cc_ = min(cc_, tail_clamp);                                                  \
            dma16(abase + (aoff[q] + cc_), (lds_ptr_t)(sb_ + (wid * kAInstr + q) * 1024));           \
        }                                                                                            \
        if (has_b) {                                                                                 \
            uint32_t cc_ = kb_ + (lco ^ (uint32_t)((wid & 7) * 16));                                 \
            if (!full_) cc_ = min(cc_, tail_clamp);                                                  \
            dma16(bbase + (boff0 + cc_), (lds_ptr_t)(sb_ + kAStageBytes + wid * 1024));              \
        }                                                                                            \
    }

        f32x16 acc[2][2];
#pragma unroll
        for (int a = 0; a < 2; ++a)
#pragma unroll
            for (int b = 0; b < 2; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

        // every wave is done with the previous tile's LDS, and this wave's
        // earlier memory operations have drained, before the ring is refilled
        AFD_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int p = 0; p < kStages - 1; ++p)
            if (p < nk) AFD_ISSUE(p, p);

        // this wave's valid token blocks: wm (if < nblk) and wm + 8 (if < nblk)
        const int nv = (wm < nblk ? 1 : 0) + (wm + kWaveRows < nblk ? 1 : 0);
        // fragment byte offsets inside a stage: chunk ch = 2*kk + lane/32 of
        // row r sits at r*128 + (ch ^ swz8(r))*16 = fbase(r) ^ (32*kk) with
        // fbase(r) = r*128 + ((lane/32) ^ swz8(r))*16
        constexpr int kKK = kBK / 16;
        uint32_t wfb[2], tfb[2];
#pragma unroll
        for (int nb = 0; nb < 2; ++nb)
            wfb[nb] = kAStageBytes + wrl[nb] * kRowBytes + (((lane >> 5) ^ swz8(wrl[nb])) * 16);
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int ar = (wm + kWaveRows * mb) * 32 + (lane & 31);
            tfb[mb] = ar * kRowBytes + (((lane >> 5) ^ swz8(ar)) * 16);
        }

        // One depth step: all fragment reads of the stage first, then the
        // MFMAs (NV = number of this wave's valid token blocks).
#define AFD_STEP(NV)                                                                                 \
    for (int kt = 0; kt < nk; ++kt) {                                                                \
        const int st = kt % kStages;                                                                 \
        const int later = min(nk - 1 - kt, kStages - 2);                                             \
        wait_vmcnt_upto(later * nw);                                                                 \
        __builtin_amdgcn_s_barrier();                                                                \
        const char* sb = smem + st * kStageBytes;                                                    \
        _Pragma("unroll") for (int kk = 0; kk < kKK; ++kk) {                                         \
            bf16x8 wf[2], tf[2];                                                                     \
            _Pragma("unroll") for (int nb = 0; nb < 2; ++nb)                                         \
                wf[nb] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sb + (wfb[nb] ^ (32u * kk))));   \
            _Pragma("unroll") for (int mb = 0; mb < NV; ++mb)                                        \
                tf[mb] = __builtin_bit_cast(bf16x8, *(const u32x4*)(sb + (tfb[mb] ^ (32u * kk))));   \
            /* refill the other stage while this stage's first reads are in flight */               \
            if (kk == 0 && kt + kStages - 1 < nk) AFD_ISSUE(kt + kStages - 1, (kt + kStages - 1) % kStages); \
            if (kt >= kfull && kt * kBK + (2 * kk + (lane >> 5)) * 8 >= Kdim) {                      \
                /* chunks at or past K contribute zero */                                            \
                _Pragma("unroll") for (int mb = 0; mb < NV; ++mb)                                    \
                    tf[mb] = __builtin_bit_cast(bf16x8, (u32x4){0u, 0u, 0u, 0u});                    \
            }                                                                                        \
            _Pragma("unroll") for (int mb = 0; mb < NV; ++mb)                                        \
                _Pragma("unroll") for (int nb = 0; nb < 2; ++nb)                                     \
                    acc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wf[nb], tf[mb], acc[mb][nb], 0, 0, 0); \
        }                                                                                            \
    }
        if (nv == 2) {
            AFD_STEP(2)
        } else if (nv == 1) {
            AFD_STEP(1)
        } else {
            AFD_STEP(0)
        }
#undef AFD_STEP
#undef AFD_ISSUE

        // epilogue: in block (mb, nb) lane holds token row (wm + 8*mb)*32 +
        // (lane & 31) and, for a = 0..3, the 4 output columns
        // 32*(weight block) + a*8 + (lane >> 5)*4 + 0..3 in registers 4a..4a+3
        const int cq = (lane >> 5) * 4;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
            const int tb = wm + kWaveRows * mb;
            if (tb >= nblk) continue;
            const int row = tb * 32 + (lane & 31);
            if (row >= rows) continue;
            const int m = m0 + row;
            if (MODE == 1) {
                uint16_t* dst = sh ? c.hs + (int64_t)m * Ig : c.h + (int64_t)(row0 + m) * Ig;
                const int jb = nt * (kBN / 2) + wn * 32 + cq;
#pragma unroll
                for (int a = 0; a < 4; ++a) {
                    const int jj = jb + a * 8;
                    if (jj < Ig) {
                        uint32_t hv[4];
#pragma unroll
                        for (int i = 0; i < 4; ++i) {
                            const float g = acc[mb][0][4 * a + i], u = acc[mb][1][4 * a + i];
                            hv[i] = f2bf(g * __builtin_amdgcn_rcpf(1.f + __expf(-g)) * u);
                        }
                        *(u32x2*)(dst + jj) = (u32x2){hv[0] | (hv[1] << 16), hv[2] | (hv[3] << 16)};
                    }
                }
            } else {
#pragma unroll
                for (int nb = 0; nb < 2; ++nb) {
                    const int nbase = nt * kBN + (wn * 2 + nb) * 32 + cq;
#pragma unroll
                    for (int a = 0; a < 4; ++a) {
                        const int n = nbase + a * 8;
                        if (n < c.H) {
                            if (sh) {
                                *(f32x4*)(c.ys + (int64_t)m * c.H + n) =
                                    (f32x4){acc[mb][nb][4 * a], acc[mb][nb][4 * a + 1], acc[mb][nb][4 * a + 2],
                                            acc[mb][nb][4 * a + 3]};
                            } else {
                                const uint32_t p0 = f2bf(acc[mb][nb][4 * a]) | (f2bf(acc[mb][nb][4 * a + 1]) << 16);
                                const uint32_t p1 = f2bf(acc[mb][nb][4 * a + 2]) | (f2bf(acc[mb][nb][4 * a + 3]) << 16);
                                *(u32x2*)(c.y + (int64_t)(row0 + m) * c.H + n) = (u32x2){p0, p1};
                            }
                        }
                    }
                }
            }
        }
        // next tile: resolve the grab issued a tile ago, broadcast it
        AFD_WAIT_VMCNT(0);
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
        __builtin_amdgcn_s_barrier();        // every wave is done with the LDS ring
        if (tid == 0) {
            const int lo = min(max(seg[xi], 0), total), hi = min(max(seg[xi + 1], lo), total);
            int t = lo + pend;
            if (t >= hi) {
                xi = (xi + 1) % kXcds;
                ++tries;
                t = grab_slow();
            }
            bcast[0] = t;
            if (t >= 0) pend = atomicAdd(&ctr[xi], 1);
        }
        __syncthreads();
        tile = bcast[0];
        __syncthreads();
    }
}

// ---------------------------------------------------------------------------
// a7: combine + split + publish.  out[t] = rsf * sum_k w[t,k] * y[inv[t*K+k]]
// + S[t] in fp32 (k in order), rounded to bf16 and written into row t - off[p]
// of peer p's return slot ("Data flow": weighted index_add_ combine with the
// shared branch added; "Data on the wire", Step 4: split back by seq_lens).
// ---------------------------------------------------------------------------
template <int KK>
__global__ __launch_bounds__(256) void k_combine(DevCtx c, const int* status, int s, int layer) {
    if (*status != AFD_OK) return;
    const int T = *c.Tptr;
    const int H = c.H, H8 = c.H / 8;
    const int npairs = T * KK;
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        const int p = peer_of(c, t);
        const int r = t - c.off[p];
        u32x4* dst = (u32x4*)(slot_ptr(c, c.ret_win, p, s) + c.foff[AFD_FIELD_ROUTED_X] + (int64_t)r * H * 2);
        int pos[KK];
        float wk[KK];
#pragma unroll
        for (int k = 0; k < KK; ++k) {
            pos[k] = min(max(c.inv[(int64_t)t * KK + k], 0), npairs - 1);
            wk[k] = c.wts[(int64_t)t * KK + k];
        }
        for (int ch = threadIdx.x; ch < H8; ch += blockDim.x) {
            u32x4 yv[KK];
#pragma unroll
            for (int k = 0; k < KK; ++k) yv[k] = *(const u32x4*)(c.y + (int64_t)pos[k] * H + ch * 8);
            float sv[8];
            if (c.has_shared) {
                const float4* sp = (const float4*)(c.ys + (int64_t)t * H + ch * 8);
                const float4 s0 = sp[0], s1 = sp[1];
                sv[0] = s0.x; sv[1] = s0.y; sv[2] = s0.z; sv[3] = s0.w;
                sv[4] = s1.x; sv[5] = s1.y; sv[6] = s1.z; sv[7] = s1.w;
            } else {
#pragma unroll
                for (int i = 0; i < 8; ++i) sv[i] = 0.f;
            }
            float acc[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = 0.f;
#pragma unroll
            for (int k = 0; k < KK; ++k) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    acc[2 * i] += wk[k] * bf2f(yv[k][i] & 0xffffu);
                    acc[2 * i + 1] += wk[k] * bf2f(yv[k][i] >> 16);
                }
            }
            u32x4 out;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                out[i] = f2bf(c.rsf * acc[2 * i] + sv[2 * i]) | (f2bf(c.rsf * acc[2 * i + 1] + sv[2 * i + 1]) << 16);
            __builtin_nontemporal_store(out, &dst[ch]);
        }
    }
}

// The return headers and flags, one thread per peer, launched after
// k_combine on the same stream: the kernel boundary makes every output row
// visible before any flag.  Each non-empty peer gets num_tokens, echo_seq =
// the inbound seq consumed, its per-expert pair counts, then a release store
// of its return flag = the FFN side's next return seq.  An empty message gets
// no reply and so creates no wait.
__global__ __launch_bounds__(64) void k_publish(DevCtx c, const int* status, int s, int layer) {
    if (*status != AFD_OK) return;
    const int p = threadIdx.x;
    if (p >= c.P) return;
    const int n_p = c.off[p + 1] - c.off[p];
    if (n_p == 0) return;
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
    header_encode(f, c.peer_counts + p * c.E, (int32_t*)(slot_ptr(c, c.ret_win, p, s) + c.foff[AFD_FIELD_HEADER]));
    __threadfence();
    st_release((int*)c.ret_win + idx, rs);
}

// ---------------------------------------------------------------------------
hipError_t launch_ffn(const DevCtx& c, int stage, int layer, const Weights& w, long long timeout_ticks, int num_cu,
                      hipEvent_t* ev, hipStream_t st) {
    int* status = c.run_status + stage * kStatusWords;
    const int Tmax = c.P * c.token_cap;
    // ev == nullptr: no events; otherwise ev[i] is recorded before kernel
    // slot i (and ev[7] after the last) unless it is null (only the slots
    // the caller asked for carry events)
    int slot = 0;
    auto mark = [&]() {
        if (ev && ev[slot]) (void)hipEventRecord(ev[slot], st);
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
    k_scan<<<c.E, 256, 0, st>>>(c, status);
    mark();
    k_permute<<<c.NB, 256, 0, st>>>(c, status);
    mark();
    k_gemm<1><<<num_cu, kGemmThreads, 0, st>>>(c, status, w);
    mark();
    k_gemm<2><<<num_cu, kGemmThreads, 0, st>>>(c, status, w);
    mark();
    int cgrid = Tmax < num_cu * 8 ? Tmax : num_cu * 8;
    if (cgrid < 1) cgrid = 1;
    switch (c.K) {
#define AFD_COMBINE_CASE(k) \
    case k: k_combine<k><<<cgrid, 256, 0, st>>>(c, status, stage, layer); break;
        AFD_COMBINE_CASE(1) AFD_COMBINE_CASE(2) AFD_COMBINE_CASE(3) AFD_COMBINE_CASE(4)
        AFD_COMBINE_CASE(5) AFD_COMBINE_CASE(6) AFD_COMBINE_CASE(7) AFD_COMBINE_CASE(8)
        AFD_COMBINE_CASE(9) AFD_COMBINE_CASE(10) AFD_COMBINE_CASE(11) AFD_COMBINE_CASE(12)
        AFD_COMBINE_CASE(13) AFD_COMBINE_CASE(14) AFD_COMBINE_CASE(15) AFD_COMBINE_CASE(16)
#undef AFD_COMBINE_CASE
        default: return hipErrorInvalidValue;
    }
    k_publish<<<1, 64, 0, st>>>(c, status, stage, layer);
    mark();
    return hipGetLastError();
}

}  // namespace afd
