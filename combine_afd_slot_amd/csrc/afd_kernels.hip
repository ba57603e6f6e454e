// afd_kernels.hip -- gfx950 kernels of the AFD FFN-rank hot path.
//
// One FFN run (afd_ffn_run) is eight launches on the FFN stream:
//   k_wait     bounded acquire-spin on the P inbound flags, header checks,
//              fan-in offsets (the fan-in itself is virtual: no copy)
//   k_route    one wavefront per token: top-k over the fp32 logits, weights,
//              per-chunk expert histogram
//   k_scan     per-expert counts, stable per-chunk bases, per-peer counts
//   k_permute  expert offsets, the GEMM tile plan, stable dispatch order
//              (perm / inv / token-row addresses)
//   k_gemm<1>  grouped gate/up GEMM (MFMA bf16) with the SwiGLU epilogue
//   k_gemm<2>  grouped down GEMM (MFMA bf16), routed and shared experts
//   k_combine  weighted combine + shared branch, bf16 rows written straight
//              into each peer's return slot
//   k_publish  return headers and flags, one wavefront per peer
// Weights are read from the tile-ordered copy written once per layer by
// k_pack_weights.
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

// Two floats -> two bf16 (round to nearest even) packed in a word: one
// v_cvt_pk_bf16_f32.
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ inline uint32_t pk_bf16(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// OCP FP8 E4M3 code of an fp32 value (bias 7, subnormals of 2^-9, largest
// finite 448 = code 0x7E, no infinities): round to nearest even, saturate to
// +-448; a zero result carries no sign.  Subnormal results: the value in
// units of 2^-9, rounded; normal results: the value scaled by a power of two
// to [8, 16), rounded, the exponent bumped when that reaches 16.
__device__ inline uint32_t e4m3_code(float v) {
    const float a = fabsf(v);
    uint32_t c;
    if (!(a < 448.0f)) {
        c = 0x7Eu;
    } else if (a < 0.015625f) {  // below 2^-6
        c = (uint32_t)__builtin_rintf(a * 512.0f);  // 0 .. 8 (8: the smallest normal, code 0x08)
    } else {
        int e = (int)((__float_as_uint(a) >> 23) & 0xFF) - 127;        // a in [2^e, 2^(e+1))
        float m = __builtin_rintf(a * __uint_as_float((uint32_t)(127 + 3 - e) << 23));  // 8 .. 16
        if (m == 16.0f) {
            m = 8.0f;
            ++e;
        }
        const int E = e + 7;
        c = E > 15 ? 0x7Eu : ((uint32_t)E << 3) | ((uint32_t)m - 8u);
        if (c == 0x7Fu) c = 0x7Eu;
    }
    return c == 0u ? 0u : c | (v < 0.0f ? 0x80u : 0u);
}

// Four e4m3 codes in a word (a in the low byte), by the hardware conversion
// (v_cvt_pk_fp8_f32, round to nearest even).  For inputs clamped to +-448 it
// gives e4m3_code's codes, but may give a sign to a zero; that changes no sum.
__device__ inline uint32_t pack4_e4m3(float a, float b, float c, float d) {
    const auto cl = [](float x) { return fminf(fmaxf(x, -448.0f), 448.0f); };
    int w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(a), cl(b), 0, false);
    w = __builtin_amdgcn_cvt_pk_fp8_f32(cl(c), cl(d), w, true);
    return (uint32_t)w;
}

__device__ inline char* slot_ptr(const DevCtx& c, char* win, int p, int s) {
    return win + c.slots_off + (int64_t)(p * c.R + s) * c.slot_bytes;
}

__device__ inline int ld_acquire(int* p) {
    return __hip_atomic_load(p, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ inline void st_release(int* p, int v) {
    __hip_atomic_store(p, v, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Wavefront inclusive prefix sums with DPP moves (register exchanges, no LDS
// traffic): within each row of 16 lanes add the value 1, 2, 4 and 8 lanes
// below (lanes past the row's start add 0), then carry row 0's total into
// row 1 and row 2's into row 3 (row_bcast:15), then rows 0-1's total into
// rows 2 and 3 (row_bcast:31).
// ---------------------------------------------------------------------------
__device__ __forceinline__ int wave_incl_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, true);  // row_shr:1
    x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, true);  // row_shr:2
    x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, true);  // row_shr:4
    x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, true);  // row_shr:8
    x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return x;
}
template <int CTRL, int ROWS, bool BOUND>
__device__ __forceinline__ long long dpp64(long long x) {
    const int lo = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)x, CTRL, ROWS, 0xF, BOUND);
    const int hi = __builtin_amdgcn_update_dpp(0, (int)(uint32_t)((uint64_t)x >> 32), CTRL, ROWS, 0xF, BOUND);
    return (long long)(((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo);
}
__device__ __forceinline__ long long wave_incl_scan64(long long x) {
    x += dpp64<0x111, 0xF, true>(x);
    x += dpp64<0x112, 0xF, true>(x);
    x += dpp64<0x114, 0xF, true>(x);
    x += dpp64<0x118, 0xF, true>(x);
    x += dpp64<0x142, 0xA, false>(x);
    x += dpp64<0x143, 0xC, false>(x);
    return x;
}

// ---------------------------------------------------------------------------
// Block-wide exclusive prefix sum of one int per thread (blockDim a multiple
// of 64, at most 1024).  `sh` holds 16 ints.
// ---------------------------------------------------------------------------
__device__ int block_excl_scan(int v, int* sh) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const int x = wave_incl_scan(v);
    if (lane == 63) sh[wid] = x;
    __syncthreads();
    // the totals of the waves below this one: one read per lane, summed
    // across the lanes (no chain of dependent reads)
    const int below = wave_incl_scan(lane < wid ? sh[lane] : 0);
    const int wbase = __builtin_amdgcn_readlane(below, 63);
    __syncthreads();
    return x + wbase - v;
}

// Sum over the 64 lanes of a wavefront with DPP moves (no LDS): butterflies
// inside each row of 16 lanes, then the row sums carried across rows with
// the row broadcasts; lane 63 ends up with the total.
__device__ inline float wave_sum(float x) {
    x += __builtin_amdgcn_update_dpp(0.f, x, 0xB1, 0xF, 0xF, false);   // quad_perm [1,0,3,2]
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x4E, 0xF, 0xF, false);   // quad_perm [2,3,0,1]
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x141, 0xF, 0xF, false);  // row_half_mirror
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x140, 0xF, 0xF, false);  // row_mirror
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x142, 0xA, 0xF, false);  // row_bcast:15 into rows 1, 3
    x += __builtin_amdgcn_update_dpp(0.f, x, 0x143, 0xC, 0xF, false);  // row_bcast:31 into rows 2, 3
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), 63));
}

// One token's top-K by a wavefront: lane l holds logits l, l+64, ... in v
// (-inf past E).  On return rank[j] is the rank of logit l + 64 j (rank < K:
// selected, rank k the k-th) and wt[j] its weight.  Shared by the FFN-side
// routing and the attention-side pack, so both select and weigh alike.
// The largest of the lanes' 64-bit keys (h high word, l low word, unsigned),
// in every lane: a running maximum over the row shifts and row broadcasts of
// wave_incl_scan (lanes shifted in from outside a row contribute 0, the
// smallest key), lane 63's result broadcast.  Each step is one 64-bit
// compare and two selects: vector instructions only (a compare combined
// with and/or becomes scalar mask logic, and a CU's waves share one scalar
// unit).
__device__ __forceinline__ uint64_t key64(uint32_t h, uint32_t l) { return ((uint64_t)h << 32) | l; }
__device__ __forceinline__ void wave_max_key(uint32_t& h, uint32_t& l) {
#define AFD_MAXKEY_STEP(CTRL, ROWS, BOUND)                                                   \
    {                                                                                        \
        const uint32_t nh = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)h, CTRL, ROWS, 0xF, BOUND); \
        const uint32_t nl = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)l, CTRL, ROWS, 0xF, BOUND); \
        const bool gt = key64(nh, nl) > key64(h, l);                                        \
        h = gt ? nh : h;                                                                     \
        l = gt ? nl : l;                                                                     \
    }
    AFD_MAXKEY_STEP(0x111, 0xF, true)
    AFD_MAXKEY_STEP(0x112, 0xF, true)
    AFD_MAXKEY_STEP(0x114, 0xF, true)
    AFD_MAXKEY_STEP(0x118, 0xF, true)
    AFD_MAXKEY_STEP(0x142, 0xA, false)
    AFD_MAXKEY_STEP(0x143, 0xC, false)
#undef AFD_MAXKEY_STEP
    h = (uint32_t)__builtin_amdgcn_readlane((int)h, 63);
    l = (uint32_t)__builtin_amdgcn_readlane((int)l, 63);
}

template <int EPL>
__device__ __forceinline__ void route_token(const float (&v)[EPL], int E, int K, int renorm, int lane,
                                            int (&rank)[EPL], float (&wt)[EPL]) {
    if constexpr (EPL == 1) {
        // Rank by broadcast: each lane counts the logits that precede its
        // own (larger, or equal with a smaller index).  A logit past E is
        // -inf with an index past every valid one, so it never raises a
        // valid logit's rank.  Compared as 64-bit keys: the value made
        // unsigned-orderable (-0 as +0) above the complement of the index,
        // so "precedes" is one unsigned compare (vector instructions only;
        // the or/and form becomes scalar mask logic, which the CU's waves
        // queue for on its one scalar unit).
        const uint32_t u = __float_as_uint(v[0] + 0.0f);
        const uint32_t kh = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
        const uint64_t mine = key64(kh, ~(uint32_t)lane);
        rank[0] = 0;
#pragma unroll
        for (int sl = 0; sl < 64; ++sl) {
            const uint32_t xh = (uint32_t)__builtin_amdgcn_readlane((int)kh, sl);
            rank[0] += key64(xh, ~(uint32_t)sl) > mine ? 1 : 0;
        }
    } else {
        // K rounds of a wave-wide maximum over the logits not yet taken, in
        // the same order (value descending, index ascending): the key of
        // logit e is its value made unsigned-orderable (-0 taken as +0)
        // above the complement of e.  Round k's winner gets rank k; the
        // rest keep rank K.
        uint32_t kh[EPL];
        uint32_t live = 0u;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const uint32_t u = __float_as_uint(v[j] + 0.0f);
            kh[j] = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
            rank[j] = K;
            if (lane + 64 * j < E) live |= 1u << j;
        }
        for (int k = 0; k < K; ++k) {
            uint32_t bh = 0u, bl = 0u;  // (a valid key is never (0, 0): finite values)
#pragma unroll
            for (int j = 0; j < EPL; ++j) {
                // (a taken or padding entry competes as key 0, which never wins)
                const uint32_t lo = ((live >> j) & 1u) ? ~(uint32_t)(lane + 64 * j) : 0u;
                const uint32_t hi = ((live >> j) & 1u) ? kh[j] : 0u;
                const bool better = key64(hi, lo) > key64(bh, bl);
                bh = better ? hi : bh;
                bl = better ? lo : bl;
            }
            wave_max_key(bh, bl);
            const int e = (int)~bl;
#pragma unroll
            for (int j = 0; j < EPL; ++j)
                if (e == lane + 64 * j) {
                    rank[j] = k;
                    live &= ~(1u << j);
                }
        }
    }
    // the maximum is the logit of rank 0 (exactly one lane holds it)
    float top = -INFINITY;
    bool has_top = false;
#pragma unroll
    for (int j = 0; j < EPL; ++j)
        if (lane + 64 * j < E && rank[j] == 0) {
            top = v[j];
            has_top = true;
        }
    const float m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(top), __builtin_ctzll(__ballot(has_top))));
    float ex[EPL], part = 0.f;
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        const bool sel = e < E && rank[j] < K;
        ex[j] = (e < E) ? expf(v[j] - m) : 0.f;
        if (renorm ? sel : (e < E)) part += ex[j];
    }
    part = wave_sum(part);
#pragma unroll
    for (int j = 0; j < EPL; ++j) wt[j] = ex[j] / part;
}

// ---------------------------------------------------------------------------
// Pack (attention side).  Payload first, then -- in a second launch on the
// same stream, so the whole payload is complete and written back -- the
// header and a release store of the flag ("Window and slot layout": payload
// and flag ordered on one stream; the flag value is the sender's seq).
// ---------------------------------------------------------------------------
// shared: the window carries shared rows (shared_x, shared_idx); a routed-
// only window does not.  grouped: the attention side routes, so no logits
// travel and the routed rows are written grouped by expert (k_pscatter).
// Fill n words at p with a pattern (poison mode).
__global__ __launch_bounds__(256) void k_fill(uint32_t* p, int64_t n, uint32_t v) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = v;
}

// Poison mode, FFN side: once the wait has consumed the work item, the
// return slot of every peer it serves (its payload fields, all rows) is
// filled with 0xFFFFFFFF before the run writes the reply, so a peer that
// reads a row the reply did not write sees NaN.  Peers not served keep
// their return slot (it may hold an earlier reply not yet unpacked).
__global__ __launch_bounds__(256) void k_poison_ret(DevCtx c, const int* status, int s) {
    if (status[0] != AFD_OK) return;
    const uint64_t served = (uint64_t)(uint32_t)status[4] | ((uint64_t)(uint32_t)status[5] << 32);
    const int p = blockIdx.y;
    if (!((served >> p) & 1)) return;
    char* slot = c.ret_win + c.slots_off + (int64_t)(p * c.R + s) * c.slot_bytes;
    const int64_t o = c.foff[AFD_FIELD_ROUTE_TABLE], n = (c.slot_bytes - o) / 4;
    uint32_t* q = (uint32_t*)(slot + o);
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) q[i] = 0xFFFFFFFFu;
}

__global__ __launch_bounds__(256) void k_pack_payload(char* slot, int64_t o_rt, int64_t o_rx, int64_t o_si,
                                                      int64_t o_sx, const uint4* hidden, const float* logits,
                                                      int n, int H, int E, int shared, int grouped) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    const int64_t gid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nch = (int64_t)n * H / 8;
    uint4* rx = (uint4*)(slot + o_rx);
    uint4* sx = (uint4*)(slot + o_sx);
    for (int64_t i = gid; i < nch; i += stride) {
        uint4 v = hidden[i];
        if (!grouped) rx[i] = v;
        if (shared) sx[i] = v;
    }
    float* rt = (float*)(slot + o_rt);
    const int64_t nl = grouped ? 0 : (int64_t)n * E;
    for (int64_t i = gid; i < nl; i += stride) rt[i] = logits[i];
    if (shared) {
        int* si = (int*)(slot + o_si);
        for (int64_t i = gid; i < n; i += stride) si[i] = (int)i;
    }
}

// counts != nullptr (attention-routed): the header's group list; routed_tokens
// is its sum (all pairs, or the pairs of the window's experts).
__global__ void k_pack_publish(char* slot, int* flag, afd_header_fields f, const int* counts) {
    if (counts) {
        int sum = 0;
        for (int e = threadIdx.x; e < f.n_counts; e += 64) sum += counts[e];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o);
        f.routed_tokens = sum;
    }
    if (threadIdx.x == 0) {
        header_encode(f, counts, (int32_t*)slot);
        __threadfence();
        st_release(flag, f.seq);
    }
}

// ---------------------------------------------------------------------------
// Attention-side routing of one message (attention-routed windows; "[RFC]:
// Async GPU Connector", "Data flow", step 1: the sender routes, flattens its
// top-k ids and sorts them stably, which groups the routed rows by expert;
// the counts are the group list; step 4: the top-k weights stay with the
// sender).  Message idx = peer * R + stage, its n tokens in chunks of
// kRouteChunk.  k_proute: one wavefront per token, the same top-K code as
// the FFN side (route_token); chunk histograms.  k_pscan: one workgroup per
// expert scans its column of chunk histograms.  k_pscatter: the row of pair
// f = t*K + k among the grouped rows is goff[e] + (pairs of e in earlier
// chunks) + (earlier tokens of the chunk that chose e); k_pcopy then copies
// token t's hidden row there, once per k.  A window that owns experts [e0, e0+E)
// of the Eg the peers route over keeps only the pairs of those (expert ids
// local, e - e0); the other pairs keep their weight with id -1 and no row.
// ---------------------------------------------------------------------------
template <int EPL>
__global__ __launch_bounds__(64 * kRouteChunk) void k_proute(DevCtx c, int idx, const float* logits, int n) {
    __shared__ int hist[kMaxExperts];
    const int lane = threadIdx.x & 63;
    const int E = c.E, K = c.K, Eg = c.Eg;
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    const int t = (int)blockIdx.x * kRouteChunk + (int)(threadIdx.x >> 6);
    const bool live = t < n;
    const int r = min(t, n - 1);
    float v[EPL];
#pragma unroll
    for (int j = 0; j < EPL; ++j) {
        const int e = lane + 64 * j;
        const float x = e < Eg ? logits[(int64_t)r * Eg + e] : -INFINITY;
        v[j] = x == x ? x : -INFINITY;  // (the same rule as the FFN side)
    }
    __syncthreads();  // hist zeroed
    if (live) {
        int rank[EPL];
        float wt[EPL];
        route_token<EPL>(v, Eg, K, c.renorm, lane, rank, wt);
        const int64_t base = (int64_t)idx * c.token_cap * K + (int64_t)t * K;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j - c.e0;  // local id
            if (lane + 64 * j < Eg && rank[j] < K) {
                const bool mine = e >= 0 && e < E;
                c.pid[base + rank[j]] = mine ? e : -1;
                c.pwt[base + rank[j]] = wt[j];
                if (mine) atomicAdd(&hist[e], 1);
            }
        }
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) c.pblk[((int64_t)idx * E + e) * c.NBp + blockIdx.x] = hist[e];
}

__global__ __launch_bounds__(256) void k_pscan(DevCtx c, int idx, int nb) {
    __shared__ int sh[16];
    const int e = blockIdx.x;
    const int* col = c.pblk + ((int64_t)idx * c.E + e) * c.NBp;
    int* base = c.pbase + ((int64_t)idx * c.E + e) * c.NBp;
    const int per = (nb + 255) / 256;
    const int b0 = threadIdx.x * per, b1 = min(nb, b0 + per);
    int sum = 0;
    for (int b = b0; b < b1; ++b) sum += col[b];
    int run = block_excl_scan(sum, sh);
    for (int b = b0; b < b1; ++b) {
        base[b] = run;
        run += col[b];
    }
    if (threadIdx.x == 255) c.pcnt[(int64_t)idx * c.E + e] = run;
}

__global__ __launch_bounds__(256) void k_pscatter(DevCtx c, int idx, char* slot, const uint4* hidden, int n) {
    static_assert(kRouteChunk <= 32 && kRouteChunk * kMaxTopK <= 256, "chunk masks and one pair per thread");
    __shared__ int sh[16];
    __shared__ int s_goff[kMaxExperts];
    __shared__ uint32_t emask[kMaxExperts];
    const int E = c.E, K = c.K, tid = threadIdx.x;
    const int b = blockIdx.x, t0 = b * kRouteChunk, nt = min(kRouteChunk, n - t0), np = nt * K;
    const int64_t pbase = (int64_t)idx * c.token_cap * K;
    int e = -1;  // (-1: a pair of another window's experts)
    if (tid < np) e = c.pid[pbase + (int64_t)t0 * K + tid];
    {
        const int per = (E + 255) / 256;
        const int e0 = tid * per, e1 = min(E, e0 + per);
        int cnt[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) cnt[j] = e0 + j < e1 ? c.pcnt[(int64_t)idx * E + e0 + j] : 0;
        int run = block_excl_scan(cnt[0] + cnt[1] + cnt[2] + cnt[3], sh);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e0 + j < e1) {
                s_goff[e0 + j] = run;
                run += cnt[j];
            }
    }
    for (int q = tid; q < E; q += 256) emask[q] = 0u;
    __syncthreads();
    if (e >= 0) atomicOr(&emask[e], 1u << (tid / K));
    __syncthreads();
    if (tid < np) {
        const int tl = tid / K;
        const int pos = e < 0 ? -1
                              : s_goff[e] + c.pbase[((int64_t)idx * E + e) * c.NBp + b] +
                                    __popc(emask[e] & ((1u << tl) - 1u));
        c.ppos[pbase + (int64_t)t0 * K + tid] = pos;
    }
}

// The grouped rows: pair f's token row to row ppos[f] (one workgroup per
// pair at a time, a grid wide enough to keep every CU's loads in flight).
__global__ __launch_bounds__(256) void k_pcopy(DevCtx c, int idx, char* slot, const uint4* hidden, int n) {
    const int K = c.K, H8 = c.H / 8, np = n * K;
    const int* ppos = c.ppos + (int64_t)idx * c.token_cap * K;
    uint4* rx = (uint4*)(slot + c.foff[AFD_FIELD_ROUTED_X]);
    for (int f = blockIdx.x; f < np; f += gridDim.x) {
        const int pos = ppos[f];
        if (pos < 0) continue;  // (a pair of another window's experts)
        const uint4* src = hidden + (int64_t)(f / K) * H8;
        uint4* dst = rx + (int64_t)pos * H8;
        for (int ch = threadIdx.x; ch < H8; ch += blockDim.x) dst[ch] = src[ch];
    }
}

hipError_t launch_pack(const DevCtx& c, int peer, int stage, int layer, int seq_len, const void* hidden,
                       const float* logits, uint32_t flags, int seq, hipStream_t st) {
    char* slot = c.in_win + c.slots_off + (int64_t)(peer * c.R + stage) * c.slot_bytes;
    if (c.poison) {
        // poison mode: every payload field of the slot (all token_cap rows)
        // reads 0xFFFFFFFF -- NaN as fp32 and bf16, -1 as a row index --
        // unless this message writes it, so a read of a stale row shows
        const int64_t o = c.foff[AFD_FIELD_ROUTE_TABLE], n = (c.slot_bytes - o) / 4;
        k_fill<<<(unsigned)std::min<int64_t>((n + 255) / 256, 1024), 256, 0, st>>>((uint32_t*)(slot + o), n, 0xFFFFFFFFu);
    }
    if (seq_len > 0) {
        int64_t work = (int64_t)seq_len * c.H / 8;
        int64_t lw = (int64_t)seq_len * c.E;
        if (lw > work) work = lw;
        int grid = (int)((work + 255) / 256);
        if (grid > 2048) grid = 2048;
        if (grid < 1) grid = 1;
        k_pack_payload<<<grid, 256, 0, st>>>(slot, c.foff[AFD_FIELD_ROUTE_TABLE], c.foff[AFD_FIELD_ROUTED_X],
                                             c.foff[AFD_FIELD_SHARED_IDX], c.foff[AFD_FIELD_SHARED_X],
                                             (const uint4*)hidden, logits, seq_len, c.H, c.E, c.has_shared,
                                             c.attn_routes);
        if (c.attn_routes && seq_len > 0) {
            const int idx = peer * c.R + stage;
            const int nb = (seq_len + kRouteChunk - 1) / kRouteChunk;
            if (c.Eg <= 64) k_proute<1><<<nb, 64 * kRouteChunk, 0, st>>>(c, idx, logits, seq_len);
            else if (c.Eg <= 128) k_proute<2><<<nb, 64 * kRouteChunk, 0, st>>>(c, idx, logits, seq_len);
            else if (c.Eg <= 256) k_proute<4><<<nb, 64 * kRouteChunk, 0, st>>>(c, idx, logits, seq_len);
            else if (c.Eg <= 512) k_proute<8><<<nb, 64 * kRouteChunk, 0, st>>>(c, idx, logits, seq_len);
            else k_proute<16><<<nb, 64 * kRouteChunk, 0, st>>>(c, idx, logits, seq_len);
            k_pscan<<<c.E, 256, 0, st>>>(c, idx, nb);
            k_pscatter<<<nb, 256, 0, st>>>(c, idx, slot, (const uint4*)hidden, seq_len);
            const int np = seq_len * c.K;
            k_pcopy<<<np < 4096 ? np : 4096, 256, 0, st>>>(c, idx, slot, (const uint4*)hidden, seq_len);
        }
    }
    afd_header_fields f;
    f.flags = (int32_t)flags;
    f.seq = seq;
    f.echo_seq = 0;
    f.layer_idx = layer;
    f.stage_idx = stage;
    f.num_tokens = seq_len;
    f.routed_tokens = seq_len * (c.attn_routes ? c.K : 1);
    f.shared_tokens = c.has_shared ? seq_len : 0;
    f.src_peer = peer;
    f.n_counts = c.E;
    // attention-routed: the header carries the group list
    const int* counts = c.attn_routes && seq_len > 0 ? c.pcnt + (int64_t)(peer * c.R + stage) * c.E : nullptr;
    k_pack_publish<<<1, 64, 0, st>>>(slot + c.foff[AFD_FIELD_HEADER], (int*)c.in_win + peer * c.R + stage, f, counts);
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

template <int KK>
__device__ __forceinline__ u32x4 combine_chunk(const u32x4 (&yv)[KK], const float (&wk)[KK], u32x4 sq, bool shared,
                                               float rsf);

// Attention-routed messages: the sender combines ("[RFC]: Async GPU
// Connector", "Data flow", step 4): out[t] = rsf * sum over k, in k order,
// of w[t,k] * (returned row ppos[t,k]) + the returned shared row t, with
// the weights and rows kept from the pack -- the arithmetic of k_combine.
template <int KK>
__global__ __launch_bounds__(256) void k_pcombine(DevCtx c, int idx, const int* st, const char* slot, u32x4* out,
                                                  int n) {
    if (*st != AFD_OK) return;
    const int H8 = c.H / 8;
    const int64_t pb = (int64_t)idx * c.token_cap * KK;
    const u32x4* rx = (const u32x4*)(slot + c.foff[AFD_FIELD_ROUTED_X]);
    const u32x4* sx = (const u32x4*)(slot + c.foff[AFD_FIELD_SHARED_X]);
    for (int t = blockIdx.x; t < n; t += gridDim.x) {
        int pos[KK];
        float wk[KK];
#pragma unroll
        for (int k = 0; k < KK; ++k) {
            pos[k] = min(max(c.ppos[pb + (int64_t)t * KK + k], 0), n * KK - 1);
            wk[k] = c.pwt[pb + (int64_t)t * KK + k];
        }
        for (int ch = threadIdx.x; ch < H8; ch += blockDim.x) {
            u32x4 yv[KK];
#pragma unroll
            for (int k = 0; k < KK; ++k) yv[k] = rx[(int64_t)pos[k] * H8 + ch];
            const u32x4 sq = c.has_shared ? sx[(int64_t)t * H8 + ch] : (u32x4)0u;
            out[(int64_t)t * H8 + ch] = combine_chunk<KK>(yv, wk, sq, c.has_shared, c.rsf);
        }
    }
}

// Expert-parallel segments: each pair's row comes back from the window of
// the FFN rank that owns its expert (the one whose pack gave the pair a
// row); the weights are the same in every window (same routing code), the
// shared row comes from the window with the shared expert.  The sum runs
// over k in order with the arithmetic of k_combine, so the result does not
// depend on how the experts are split.
struct RankView {
    const int* st;    // the window's status words of this unpack
    const int* ppos;  // its rows of the message's pairs (-1: another rank's)
    const float* pwt;
    const u32x4* rx;  // its returned routed rows
    const u32x4* sx;  // its returned shared rows
};
struct RankViews {
    RankView r[kMaxRanks];
    int n, shared;  // windows; the one with the shared expert (-1: none)
};

template <int KK>
__global__ __launch_bounds__(256) void k_rcombine(RankViews v, int64_t pb, u32x4* out, int n, int H8, float rsf) {
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i)
        if (i < v.n && *v.r[i].st != AFD_OK) return;
    const bool shared = v.shared >= 0;
    const u32x4* sx = nullptr;
#pragma unroll
    for (int i = 0; i < kMaxRanks; ++i)
        if (i == v.shared) sx = v.r[i].sx;
    for (int t = blockIdx.x; t < n; t += gridDim.x) {
        const u32x4* row[KK];
        float wk[KK];
#pragma unroll
        for (int k = 0; k < KK; ++k) {
            const int64_t f = pb + (int64_t)t * KK + k;
            row[k] = nullptr;
            wk[k] = v.r[0].pwt[f];
#pragma unroll
            for (int i = 0; i < kMaxRanks; ++i)
                if (i < v.n) {
                    const int pos = v.r[i].ppos[f];
                    if (pos >= 0 && pos < n * KK) row[k] = v.r[i].rx + (int64_t)pos * H8;
                }
        }
        for (int ch = threadIdx.x; ch < H8; ch += blockDim.x) {
            u32x4 yv[KK];
#pragma unroll
            for (int k = 0; k < KK; ++k) yv[k] = row[k] ? row[k][ch] : (u32x4)0u;
            const u32x4 sq = shared ? sx[(int64_t)t * H8 + ch] : (u32x4)0u;
            out[(int64_t)t * H8 + ch] = combine_chunk<KK>(yv, wk, sq, shared, rsf);
        }
    }
}

hipError_t launch_unpack_ranks(const DevCtx* const* ctx, int n, int peer, int stage, int seq_len, const int* echo,
                               void* out, const long long* timeout_ticks, hipStream_t st) {
    if (n < 1 || n > kMaxRanks) return hipErrorInvalidValue;
    RankViews v{};
    v.n = n;
    v.shared = -1;
    for (int i = 0; i < n; ++i) {
        const DevCtx& c = *ctx[i];
        k_unpack_wait<<<1, 64, 0, st>>>(c, peer, stage, echo[i], seq_len, timeout_ticks[i]);
        const int idx = peer * c.R + stage;
        const char* slot = c.ret_win + c.slots_off + (int64_t)idx * c.slot_bytes;
        v.r[i].st = c.peer_status + idx * kStatusWords;
        v.r[i].ppos = c.ppos;
        v.r[i].pwt = c.pwt;
        v.r[i].rx = (const u32x4*)(slot + c.foff[AFD_FIELD_ROUTED_X]);
        v.r[i].sx = (const u32x4*)(slot + c.foff[AFD_FIELD_SHARED_X]);
        if (c.has_shared) v.shared = i;
    }
    const DevCtx& c = *ctx[0];
    const int64_t pb = (int64_t)(peer * c.R + stage) * c.token_cap * c.K;
    int grid = seq_len < 2048 ? seq_len : 2048;
    if (grid < 1) grid = 1;
    switch (c.K) {
#define AFD_RCOMBINE_CASE(k) \
    case k: k_rcombine<k><<<grid, 256, 0, st>>>(v, pb, (u32x4*)out, seq_len, c.H / 8, c.rsf); break;
        AFD_RCOMBINE_CASE(1) AFD_RCOMBINE_CASE(2) AFD_RCOMBINE_CASE(3) AFD_RCOMBINE_CASE(4)
        AFD_RCOMBINE_CASE(5) AFD_RCOMBINE_CASE(6) AFD_RCOMBINE_CASE(7) AFD_RCOMBINE_CASE(8)
        AFD_RCOMBINE_CASE(9) AFD_RCOMBINE_CASE(10) AFD_RCOMBINE_CASE(11) AFD_RCOMBINE_CASE(12)
        AFD_RCOMBINE_CASE(13) AFD_RCOMBINE_CASE(14) AFD_RCOMBINE_CASE(15) AFD_RCOMBINE_CASE(16)
#undef AFD_RCOMBINE_CASE
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

hipError_t launch_unpack(const DevCtx& c, int peer, int stage, int seq_len, int expect_echo, void* out,
                         long long timeout_ticks, hipStream_t st) {
    k_unpack_wait<<<1, 64, 0, st>>>(c, peer, stage, expect_echo, seq_len, timeout_ticks);
    const int idx = peer * c.R + stage;
    const char* slot = c.ret_win + c.slots_off + (int64_t)idx * c.slot_bytes;
    if (c.attn_routes) {
        int grid = seq_len < 2048 ? seq_len : 2048;
        if (grid < 1) grid = 1;
        const int* sw = c.peer_status + idx * kStatusWords;
        switch (c.K) {
#define AFD_PCOMBINE_CASE(k) \
    case k: k_pcombine<k><<<grid, 256, 0, st>>>(c, idx, sw, slot, (u32x4*)out, seq_len); break;
            AFD_PCOMBINE_CASE(1) AFD_PCOMBINE_CASE(2) AFD_PCOMBINE_CASE(3) AFD_PCOMBINE_CASE(4)
            AFD_PCOMBINE_CASE(5) AFD_PCOMBINE_CASE(6) AFD_PCOMBINE_CASE(7) AFD_PCOMBINE_CASE(8)
            AFD_PCOMBINE_CASE(9) AFD_PCOMBINE_CASE(10) AFD_PCOMBINE_CASE(11) AFD_PCOMBINE_CASE(12)
            AFD_PCOMBINE_CASE(13) AFD_PCOMBINE_CASE(14) AFD_PCOMBINE_CASE(15) AFD_PCOMBINE_CASE(16)
#undef AFD_PCOMBINE_CASE
            default: return hipErrorInvalidValue;
        }
        return hipGetLastError();
    }
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
//
// layer < 0: a layer-table run; the layer is the one every peer's header
// carries, and it must have an entry in the table.
//
// max_take > 0: an any-ready run ("Asynchronous work-item contract", item
// 3; "Risks and alternatives": a device-side wait on the flag array with a
// rotating scan start).  The wavefront polls all P flags together until one
// has changed (bounded), then up to `gather` ticks more for others, and
// takes at most max_take of the changed ones, scanning from the stage's
// rotating start; only those are checked and consumed, the rest stay
// pending with no tokens in this run, and the start moves past the last one
// taken.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64) void k_wait(DevCtx c, int s, int layer, long long timeout, int max_take,
                                             long long gather, int serve_item) {
    __shared__ int s_flag[kMaxPeers], s_err[kMaxPeers], s_ntok[kMaxPeers], s_shut[kMaxPeers], s_layer[kMaxPeers];
    __shared__ int s_rt[kMaxPeers], s_gneg[kMaxPeers];
    __shared__ unsigned long long s_gsum[kMaxPeers];
    const int p = threadIdx.x;
    if (serve_item >= 0) {
        const int stop = c.serve[0];
        if (stop != AFD_OK) {
            // an earlier item of this serve loop stopped it: consume nothing,
            // and every later kernel of the run sees a non-OK status
            if (p == 0) {
                int* st = c.run_status + s * kStatusWords;
                st[0] = stop;
                st[1] = -1;
                st[3] = 0;
                st[4] = 0;
                st[5] = 0;
                *c.Tptr = 0;
            }
            return;
        }
    }
    int* st = c.run_status + s * kStatusWords;
    const bool in = p < c.P;
    const int idx = p * c.R + s;
    const int* flag = (const int*)c.in_win + idx;
    const int seen = in ? c.seen_in[idx] : 0;
    int f = seen, err = AFD_OK;
    uint64_t taken = c.P == 64 ? ~0ull : (1ull << c.P) - 1;  // peers of this work item
    int last = c.P - 1;                                     // the last one in scan order
    if (max_take == 0) {
        if (in) {
            const long long t0 = wall_clock64();
            for (;;) {
                f = ld_acquire((int*)flag);
                if (f != seen) break;
                if (wall_clock64() - t0 > timeout) {
                    err = AFD_ERR_TIMEOUT;
                    break;
                }
                __builtin_amdgcn_s_sleep(2);
            }
        }
    } else {
        // every decision below is wave-uniform (scalar clock, ballot)
        const long long t0 = wall_clock64();
        long long t1 = -1;
        uint64_t ready = 0;
        for (;;) {
            if (in) f = ld_acquire((int*)flag);
            ready = __ballot(in && f != seen);
            const long long now = wall_clock64();
            if (ready) {
                if (t1 < 0) t1 = now;
                if (__popcll(ready) == (unsigned)c.P || now - t1 >= gather) break;
            } else if (now - t0 > timeout) {
                break;
            }
            __builtin_amdgcn_s_sleep(2);
        }
        const int r0 = c.rr[s];
        taken = 0;
        for (int q = 0, n = 0; q < c.P && n < max_take; ++q) {
            const int pq = (r0 + q) % c.P;
            if ((ready >> pq) & 1) {
                taken |= 1ull << pq;
                last = pq;
                ++n;
            }
        }
        if (!((taken >> p) & 1)) f = seen;  // left pending for a later run
    }
    const bool take = in && ((taken >> p) & 1);
    if (in) {
        int ntok = 0, shut = 0, hl = -1;
        if (take && err == AFD_OK) {
            afd_header_fields h;
            // the fixed words in one batch of loads (the header is 256-byte aligned)
            static_assert(AFD_HDR_WORDS == 12, "three 16-byte loads");
            const u32x4* hq = (const u32x4*)(slot_ptr(c, c.in_win, p, s) + c.foff[AFD_FIELD_HEADER]);
            u32x4 hv[3];
#pragma unroll
            for (int i = 0; i < 3; ++i) hv[i] = hq[i];
            err = header_decode((const int32_t*)hv, c.E, &h);
            if (err == AFD_OK) {
                hl = h.layer_idx;
                err = inbound_check(h, p, s, layer < 0 ? hl : layer, c.token_cap, f, c.has_shared,
                                    c.attn_routes ? c.K : 1, c.Eg != c.E);
            }
            s_rt[p] = err == AFD_OK ? h.routed_tokens : -1;  // group list to check below
            if (err == AFD_OK) {
                ntok = h.num_tokens;
                shut = (h.flags & (int)AFD_FLAG_SHUTDOWN) != 0;
            }
        }
        s_flag[p] = f;
        s_err[p] = err;
        s_ntok[p] = ntok;
        s_shut[p] = shut;
        s_layer[p] = hl;
        if (!(take && err == AFD_OK)) s_rt[p] = -1;
        s_gsum[p] = 0;
        s_gneg[p] = 0;
    }
    __syncthreads();
    if (c.attn_routes) {
        // each group list non-negative and covering every routed row: the
        // P*E counts spread over the lanes, so their loads go out together
        const int E = c.E, n = c.P * E;
        for (int i = p; i < n; i += 64) {
            const int q = i / E;
            if (s_rt[q] < 0) continue;
            const int v = ((const int*)(slot_ptr(c, c.in_win, q, s) + c.foff[AFD_FIELD_HEADER]))[AFD_HDR_WORDS + i - q * E];
            if (v < 0) s_gneg[q] = 1;
            else atomicAdd(&s_gsum[q], (unsigned long long)v);
        }
        __syncthreads();
        if (in && s_rt[p] >= 0 && (s_gneg[p] || s_gsum[p] != (unsigned long long)s_rt[p])) {
            s_err[p] = AFD_ERR_HEADER;
            s_ntok[p] = 0;
            s_shut[p] = 0;
        }
        __syncthreads();
    }
    if (threadIdx.x == 0) {
        int status = taken ? AFD_OK : AFD_ERR_TIMEOUT, failed = -1, shut = 0;
        for (int q = 0; q < c.P; ++q) {
            if (s_err[q] != AFD_OK && status == AFD_OK) {
                status = s_err[q];
                failed = q;
            }
            shut |= s_shut[q];
        }
        if (status == AFD_OK && shut) status = AFD_SHUTDOWN;
        int L = layer;
        if (layer < 0 && status == AFD_OK) {
            const int q0 = __builtin_ctzll(taken);
            L = s_layer[q0];
            for (int q = q0 + 1; q < c.P && status == AFD_OK; ++q)
                if (((taken >> q) & 1) && s_layer[q] != L) {
                    status = AFD_ERR_HEADER;
                    failed = q;
                }
            if (status == AFD_OK && (L < 0 || L >= *c.nlayers)) {
                status = AFD_ERR_HEADER;
                failed = q0;
            }
        }
        *c.layer_cur = L;
        int T = 0;
        const bool consume = status == AFD_OK || status == AFD_SHUTDOWN;
        if (consume) {
            c.off[0] = 0;
            for (int q = 0; q < c.P; ++q) {
                c.seen_in[q * c.R + s] = s_flag[q];  // (unchanged for a peer not taken)
                c.cur_seq[q] = s_flag[q];
                T += s_ntok[q];
                c.off[q + 1] = T;
            }
            if (max_take) c.rr[s] = (last + 1) % c.P;
        }
        const uint64_t served = consume ? taken : 0;
        *c.Tptr = status == AFD_OK ? T : 0;
        st[0] = status;
        st[1] = failed;
        st[2] = s_flag[0];
        st[3] = status == AFD_OK ? T : 0;
        st[4] = (int)(uint32_t)served;
        st[5] = (int)(uint32_t)(served >> 32);
    }
}

// ---------------------------------------------------------------------------
// Routing chunks: kRouteChunk consecutive tokens of one peer (a peer's last
// chunk may be shorter).  Chunks are numbered in fan-in token order, so the
// flat pair order f = t*K + k runs through the chunks in order.
// ---------------------------------------------------------------------------
// Peer q's chunk count and the inclusive prefix over peers 0..q, in lane q
// of the calling wavefront (all 64 lanes active; P <= 64): one round of
// loads and a wave prefix sum.
__device__ inline void peer_chunks(const DevCtx& c, int& lo, int& n, int& nc, int& inc) {
    const int lane = threadIdx.x & 63;
    lo = 0;
    n = 0;
    if (lane < c.P) {
        lo = c.off[lane];
        n = c.off[lane + 1] - lo;
    }
    nc = (n + kRouteChunk - 1) / kRouteChunk;
    inc = wave_incl_scan(nc);
}

// Chunk b's token range [t0, t1) and its peer p (false: no such chunk).
__device__ inline bool chunk_range(const DevCtx& c, int b, int& t0, int& t1, int& p) {
    int lo, n, nc, inc;
    peer_chunks(c, lo, n, nc, inc);
    const uint64_t m = __ballot((int)(threadIdx.x & 63) < c.P && b >= inc - nc && b < inc);
    if (m == 0) return false;
    p = __builtin_ctzll(m);
    const int base = __shfl(lo, p), first = __shfl(inc - nc, p), np = __shfl(n, p);
    t0 = base + (b - first) * kRouteChunk;
    t1 = min(base + np, t0 + kRouteChunk);
    return true;
}

// ---------------------------------------------------------------------------
// a2: routing.  One workgroup per chunk, one wavefront per token.  The
// order is (larger logit first, equal logits: lower expert index first;
// -0.0 equals +0.0 under float compare).  Every lane ranks its own logits
// against all E of the token's logits, broadcast one at a time from the
// lane that holds them (a scalar read of a lane: no memory round trip); the
// K experts of rank < K are the top-K, and rank k is the k-th selected.
// Weights: w_k = exp(L_k - L_max) / sum over the selected of exp(L - L_max)
// (the softmax restricted to the top-K and renormalised); without
// renormalisation the denominator runs over all E experts.  ("[RFC]: Async
// GPU Connector", "Attention gate and FFN expert compute": grouped_topk with
// a single group.)  The chunk's expert histogram goes to blk_counts[e][b].
// ---------------------------------------------------------------------------
// One token's routing by one wavefront: token t of the fan-in, row r of its
// peer's slot.  Writes its expert ids and weights (rank order), its token-row
// (and shared-row) address, and for the fp8 W1 GEMMs its e4m3 codes and row
// scale; calls sel(e) in the lane that selected expert e.  Returns whether
// the token's shared_idx entry is wrong (one FFN replica owns every shared
// row: shared_idx must be 0..n_p-1).  Q: the fp8 token-row quantisation is
// compiled in (the bf16 kernels leave it out, and its registers with it).
template <int EPL, bool Q, typename Sel>
__device__ __forceinline__ bool route_one(const DevCtx& c, const char* slot, int t, int r, int lane, Sel sel) {
    const int E = c.E, K = c.K;
    float v[EPL];
    {
        const float* lg = (const float*)(slot + c.foff[AFD_FIELD_ROUTE_TABLE]) + (int64_t)r * E;
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            const float x = e < E ? lg[e] : -INFINITY;
            v[j] = x == x ? x : -INFINITY;  // NaN logits are out of contract; keep the order total
        }
    }
    bool si_bad = false;
    if (lane == 0) {
        c.tok_src[t] = (uint64_t)(slot + c.foff[AFD_FIELD_ROUTED_X] + (int64_t)r * c.H * 2);
        if (c.has_shared) {  // (a routed-only window carries no shared rows)
            c.sh_src[t] = (uint64_t)(slot + c.foff[AFD_FIELD_SHARED_X] + (int64_t)r * c.H * 2);
            si_bad = ((const int*)(slot + c.foff[AFD_FIELD_SHARED_IDX]))[r] != r;
        }
    }
    {
        int rank[EPL];
        float wt[EPL];
        route_token<EPL>(v, E, K, c.renorm, lane, rank, wt);
#pragma unroll
        for (int j = 0; j < EPL; ++j) {
            const int e = lane + 64 * j;
            if (e < E && rank[j] < K) {
                c.ids[(int64_t)t * K + rank[j]] = e;
                c.wts[(int64_t)t * K + rank[j]] = wt[j];
                sel(e);
            }
        }
    }
    if (Q && c.w1_fp8) {
        // fp8 W1: the token row's e4m3 codes and scale (r = 448 / max|x|,
        // code = e4m3(x * r), value = code * max|x| / 448)
        const u32x4* xr = (const u32x4*)(slot + c.foff[AFD_FIELD_ROUTED_X] + (int64_t)r * c.H * 2);
        const int n8 = c.H / 8;
        // the row's first 8 chunks a lane stay in registers for the encode
        // pass (all of a row up to hidden 4096), the rest are read again
        constexpr int kKeep = 8;
        u32x4 keep[kKeep];
        float amax = 0.0f;
#pragma unroll
        for (int j = 0; j < kKeep; ++j) keep[j] = lane + 64 * j < n8 ? xr[lane + 64 * j] : (u32x4)0u;
        for (int i = lane + 64 * kKeep; i < n8; i += 64) {
            const u32x4 v8 = xr[i];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                amax = fmaxf(amax, fmaxf(fabsf(bf2f(v8[j] & 0xffffu)), fabsf(bf2f(v8[j] >> 16))));
        }
#pragma unroll
        for (int k = 0; k < kKeep; ++k)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                amax = fmaxf(amax, fmaxf(fabsf(bf2f(keep[k][j] & 0xffffu)), fabsf(bf2f(keep[k][j] >> 16))));
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        const float rs = amax > 0.0f ? __fdiv_rn(448.0f, amax) : 0.0f;
        uint2* dst = (uint2*)(c.xq + (int64_t)t * c.H);
#pragma unroll
        for (int k = 0; k < kKeep; ++k) {
            const int i = lane + 64 * k;
            if (i < n8) {
                const u32x4 v8 = keep[k];
                dst[i] = make_uint2(pack4_e4m3(bf2f(v8[0] & 0xffffu) * rs, bf2f(v8[0] >> 16) * rs,
                                               bf2f(v8[1] & 0xffffu) * rs, bf2f(v8[1] >> 16) * rs),
                                    pack4_e4m3(bf2f(v8[2] & 0xffffu) * rs, bf2f(v8[2] >> 16) * rs,
                                               bf2f(v8[3] & 0xffffu) * rs, bf2f(v8[3] >> 16) * rs));
            }
        }
        for (int i = lane + 64 * kKeep; i < n8; i += 64) {
            const u32x4 v8 = xr[i];
            dst[i] = make_uint2(pack4_e4m3(bf2f(v8[0] & 0xffffu) * rs, bf2f(v8[0] >> 16) * rs,
                                           bf2f(v8[1] & 0xffffu) * rs, bf2f(v8[1] >> 16) * rs),
                                pack4_e4m3(bf2f(v8[2] & 0xffffu) * rs, bf2f(v8[2] >> 16) * rs,
                                           bf2f(v8[3] & 0xffffu) * rs, bf2f(v8[3] >> 16) * rs));
        }
        if (lane == 0) {
            const float d = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
            c.sx[t] = d;
            c.sxp[(int64_t)c.hrows + t] = d;  // (the shared row's scale, beside the pairs')
            c.tok_src[t] = (uint64_t)(c.xq + (int64_t)t * c.H);  // the GEMM reads the codes
            if (c.has_shared) c.sh_src[t] = (uint64_t)(c.xq + (int64_t)t * c.H);
        }
    }
    return si_bad;
}

template <int EPL, bool Q>
__global__ __launch_bounds__(64 * kRouteChunk) void k_route(DevCtx c, int* status, int s) {
    const int st = *status;  // loaded together with the peer offsets of chunk_range
    int t_begin, t_end, p;
    const bool have = chunk_range(c, blockIdx.x, t_begin, t_end, p);
    if (st != AFD_OK || !have) return;
    __shared__ int hist[kMaxExperts];
    const int lane = threadIdx.x & 63;
    const int E = c.E;
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    const char* slot = slot_ptr(c, c.in_win, p, s);
    const int t = t_begin + (int)(threadIdx.x >> 6);
    __syncthreads();  // hist zeroed
    bool si_bad = false;
    if (t < t_end) si_bad = route_one<EPL, Q>(c, slot, t, t - c.off[p], lane, [&](int e) { atomicAdd(&hist[e], 1); });
    if (si_bad) atomicCAS(status, AFD_OK, AFD_ERR_HEADER);
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
    if (threadIdx.x < 64) {
        int lo, n, nc, inc;
        peer_chunks(c, lo, n, nc, inc);
        if (threadIdx.x == 0) pchunk[0] = 0;
        if ((int)threadIdx.x < c.P) pchunk[threadIdx.x + 1] = inc;
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
// GEMM tile plan.  Group j: 0 is the shared expert over all T tokens (when
// present), then the routed experts.  A group of M rows has b = ceil(M/32)
// row blocks split evenly over ceil(b/kTileBlocks) row tiles and, for the
// gate/up GEMM, ceil(Ig/(kBW/2)) column tiles (kBW/2 gate + the same kBW/2
// up rows of W13), for the down GEMM ceil(H/kBW).  Tiles are numbered
// group-major (the order inside a group is below).  The cost of a tile is (32-row blocks it
// holds) x (depth steps).
//
// Plan order: the shared group, then the heavy routed groups, then the light
// routed groups (1 to 32 rows: tiles of a single token block, whose time is
// the streaming of their weight rows), each in expert order.  The shared
// tiles, the heavy routed tiles and the light routed tiles are each cut into
// kXcds segments of equal cost, one of each class per XCD.
//
// Inside a group the tiles run in panels of kPanel column tiles: panel by
// panel, and in a panel row tile by row tile with the panel's column tiles
// fastest.  The workgroups of one XCD take consecutive tiles of a segment at
// about the same time, so the tiles in flight on an XCD form a block of a
// few row tiles by up to kPanel column tiles that share both operands: each
// token-row block is fetched once per panel instead of once per column tile,
// and each weight tile once per row-tile pass of the panel.  (kPanel = 1 is
// plain column-tile order.)
// ---------------------------------------------------------------------------
#ifndef AFD_TILE_PANEL
#define AFD_TILE_PANEL 4
#endif
constexpr int kPanel = AFD_TILE_PANEL;
// One GEMM workgroup in kLightEvery (by its rank on its XCD) takes the light
// segments first (the tile scheduler below).
#ifndef AFD_LIGHT_EVERY
#define AFD_LIGHT_EVERY 5
#endif
constexpr int kLightEvery = AFD_LIGHT_EVERY;
struct PlanGroup {
    int M, mt, blocks, nt, nk;
};

__device__ inline PlanGroup plan_group(const DevCtx& c, int T, const int* s_eoff, int j, int mode) {
    PlanGroup g;
    const bool shd = c.has_shared && j == 0;
    const int e = j - c.has_shared;
    const int Ig = shd ? c.Is : c.I;
    g.M = shd ? T : s_eoff[e + 1] - s_eoff[e];
    g.blocks = (g.M + 31) / 32;
    g.mt = (g.blocks + kTileBlocks - 1) / kTileBlocks;
    g.nt = mode == 1 ? (Ig + kBW / 2 - 1) / (kBW / 2) : (c.H + kBW - 1) / kBW;
    g.nk = mode == 1 ? (c.H + kBK - 1) / kBK : (Ig + kBK - 1) / kBK;
    if (mode == 2 && shd && c.shp > 1) {
        // depth split: column index = part * (column tiles) + column tile,
        // each part ceil(depth / parts) steps deep at most
        g.nt *= c.shp;
        g.nk = (g.nk + c.shp - 1) / c.shp;
    }
    return g;
}

// Block-wide exclusive prefix sums of four int64 values per thread, over
// the first nw wavefronts (the values of the others are taken as zero and
// they do no scan work: on one CU every wavefront's VALU work counts).
// `sh` holds 4 values per wavefront (64 for 1024 threads).  Every thread
// of the block calls it.
__device__ void block_excl_scan4(long long (&v)[4], long long* sh, int nw) {
    const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
    const bool act = wid < nw;  // (wave-uniform)
    long long x[4];
    if (act) {
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = wave_incl_scan64(v[q]);
        if (lane == 63)
#pragma unroll
            for (int q = 0; q < 4; ++q) sh[wid * 4 + q] = x[q];
    }
    __syncthreads();
    if (act) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const long long below = wave_incl_scan64(lane < wid ? sh[lane * 4 + q] : 0ll);
            const uint32_t lo = __builtin_amdgcn_readlane((int)(uint32_t)below, 63);
            const uint32_t hi = __builtin_amdgcn_readlane((int)(uint32_t)((uint64_t)below >> 32), 63);
            v[q] = x[q] - v[q] + (long long)(((uint64_t)hi << 32) | lo);
        }
    }
    __syncthreads();
}

// floor(a / b) for 0 <= a < 2^53, b > 0: a double quotient corrected to
// the exact one (a 64-bit integer division is a long software sequence).
__device__ __forceinline__ long long div_floor(long long a, long long b) {
    long long q = (long long)((double)a / (double)b);
    while (q > 0 && q * b > a) --q;
    while ((q + 1) * b <= a) ++q;
    return q;
}

// floor(a / b) for 0 <= a and 0 < b: below 2^22 from a float quotient (the
// reciprocal's error keeps the estimate within one of the exact value,
// which the remainder then fixes), above it by the integer division.
__device__ __forceinline__ int div_small(int a, int b) {
    if ((a | b) >= (1 << 22)) return a / b;
    int q = (int)((float)a * __builtin_amdgcn_rcpf((float)b));
    const int r = a - q * b;
    q += r < 0 ? -1 : (r >= b ? 1 : 0);
    return q;
}

// A light group: a routed expert with 1 to 32 rows (one token block).
__device__ inline bool plan_light(const DevCtx& c, const int* s_eoff, int j) {
    if (c.has_shared && j == 0) return false;
    const int e = j - c.has_shared;
    const int M = s_eoff[e + 1] - s_eoff[e];
    return M >= 1 && M <= 32;
}

// The plan order of the groups and the tile and cost prefixes of both GEMMs
// over it, into LDS: s_ord[q] = the group at plan position q (heavy groups,
// the shared one first, then light ones, each in index order), *s_nh = the
// number of heavy groups (light positions start there), s_t[m][q] / s_c[m][q]
// = tiles / cost of GEMM m+1 before position q (q = G: the totals).
__device__ void plan_prefix(const DevCtx& c, int T, const int* s_eoff, int (*s_t)[kMaxExperts + 2],
                            long long (*s_c)[kMaxExperts + 2], int* s_ord, int* s_nh, long long* sh) {
    const int tid = threadIdx.x, G = c.G, NT = blockDim.x;
    const int per = (G + NT - 1) / NT;
    const int j0 = tid * per, j1 = min(G, j0 + per);
    const int last = (G + per - 1) / per - 1;  // the thread holding group G-1
    const int nw = last / 64 + 1;              // wavefronts holding groups
    {
        int nl = 0;
        for (int j = j0; j < j1; ++j) nl += plan_light(c, s_eoff, j) ? 1 : 0;
        long long v[4] = {nl, 0, 0, 0};
        block_excl_scan4(v, sh, nw);  // v[0]: light groups before j0
        if (tid == last) *s_nh = G - (int)(v[0] + nl);
        __syncthreads();
        const int nh = *s_nh;
        int lr = (int)v[0];
        for (int j = j0; j < j1; ++j) {
            const bool l = plan_light(c, s_eoff, j);
            s_ord[l ? nh + lr : j - lr] = j;
            lr += l ? 1 : 0;
        }
        __syncthreads();
    }
    long long v[4] = {0, 0, 0, 0};  // tiles of GEMM 1, 2; cost of GEMM 1, 2
    for (int q = j0; q < j1; ++q) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const PlanGroup g = plan_group(c, T, s_eoff, s_ord[q], m + 1);
            v[m] += g.mt * g.nt;
            v[2 + m] += (long long)g.nt * g.blocks * g.nk;
        }
    }
    block_excl_scan4(v, sh, nw);
    for (int q = j0; q < j1; ++q) {
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            const PlanGroup g = plan_group(c, T, s_eoff, s_ord[q], m + 1);
            s_t[m][q] = (int)v[m];
            s_c[m][q] = v[2 + m];
            v[m] += g.mt * g.nt;
            v[2 + m] += (long long)g.nt * g.blocks * g.nk;
        }
    }
    if (tid == last)
#pragma unroll
        for (int m = 0; m < 2; ++m) {
            s_t[m][G] = (int)v[m];
            s_c[m][G] = v[2 + m];
        }
    __syncthreads();
}

// The plan's global tables (one workgroup): tile prefixes, the zeroed tile
// counters and the segment boundaries.  Class k (0 shared, 1 heavy routed, 2
// light routed: plan positions [0, hs), [hs, nh), [nh, G)) with cost range
// [C0, C1) has boundaries k*kXcds + b, b < kXcds, at cost C0 + (C1-C0)*b/kXcds:
// the first tile whose cost prefix reaches it (boundary kSegs: the end).
__device__ void plan_publish(const DevCtx& c, int T, const int* s_eoff, int (*s_t)[kMaxExperts + 2],
                             long long (*s_c)[kMaxExperts + 2], const int* s_ord, int nh) {
    __shared__ int s_seg[2][kSegs + 1];
    const int tid = threadIdx.x, G = c.G;
    for (int i = tid; i < 2 * (G + 1); i += (int)blockDim.x) {
        const int m = i / (G + 1), j = i - m * (G + 1);
        (m == 0 ? c.tstart1 : c.tstart2)[j] = s_t[m][j];
    }
    // one thread per (GEMM, boundary): both GEMMs' searches run side by side
    if (tid < 2 * (kSegs + 1)) {
        const int m = tid / (kSegs + 1), sb = tid - m * (kSegs + 1);
        int* seg = m == 0 ? c.seg1 : c.seg2;
        const int hs = c.has_shared ? 1 : 0;
        const int cls = sb / kXcds, b = sb % kXcds;
        const int q0 = cls == 0 ? 0 : cls == 1 ? hs : cls == 2 ? nh : G;
        const int q1 = cls == 0 ? hs : cls == 1 ? nh : G;
        const int lo_t = s_t[m][q0], hi_t = s_t[m][q1];
        const long long C0 = s_c[m][q0], C1 = s_c[m][q1];
        const long long S = C0 + (C1 - C0) * b / kXcds;
        int res;
        if (b == 0 || cls == 3) res = lo_t;
        else if (S >= C1) res = hi_t;
        else {
            // the last plan position whose cost prefix is at most S (positions
            // of groups with no tiles share their successor's prefix)
            int lo = 0, hi = G;
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_c[m][mid] <= S) lo = mid;
                else hi = mid;
            }
            const PlanGroup g = plan_group(c, T, s_eoff, s_ord[lo], m + 1);
            const long long u = div_floor(S - s_c[m][lo] + g.nk - 1, g.nk);  // in 32-row blocks
            // the panel holding block-column u, then the first row tile
            // of that panel starting at or after its remaining blocks
            const int pw = min(kPanel, g.nt), np = (g.nt + pw - 1) / pw;
            int pp = min((int)div_floor(u, (long long)pw * g.blocks), np - 1);
            const int w = min(pw, g.nt - pp * pw);
            const long long rb = div_floor(u - (long long)pp * pw * g.blocks + w - 1, w);  // blocks into the panel
            int mt = (int)div_floor(rb * g.mt + g.blocks - 1, g.blocks);
            if (mt >= g.mt) {
                ++pp;
                mt = 0;
            }
            res = min(s_t[m][lo] + pp * pw * g.mt + mt * w, s_t[m][lo] + g.mt * g.nt);
        }
        seg[sb] = s_seg[m][sb] = min(max(res, lo_t), hi_t);
    }
    __syncthreads();
    // The tile counters start past the tiles that the GEMM workgroups take
    // without an atomic as their first (sched_first): on XCD x (workgroups b
    // = x, x + kXcds, ... of the ncu-workgroup grid) the light-first
    // workgroups, by rank, take the first tiles of the light segment x, the
    // normal ones the first tiles of the shared, then the heavy segment x,
    // then the light tiles after the light-first workgroups' share.
    if (tid < 2 * kSegs) {
        const int m = tid / kSegs, sidx = tid - m * kSegs;
        const int cls = sidx / kXcds, x = sidx % kXcds;
        const int nx = c.ncu > x ? (c.ncu - x + kXcds - 1) / kXcds : 0;
        const int nlf = (nx + kLightEvery - 1) / kLightEvery, nnorm = nx - nlf;
        const int size = s_seg[m][sidx + 1] - s_seg[m][sidx];
        int taken;
        const int sh = s_seg[m][x + 1] - s_seg[m][x], hv = s_seg[m][kXcds + x + 1] - s_seg[m][kXcds + x];
        if (cls == 0) taken = min(size, nnorm);
        else if (cls == 1) taken = min(size, max(0, nnorm - sh));
        else taken = min(size, nlf + max(0, nnorm - sh - hv));
        c.tctr[tid] = taken;
    }
}

// Share `part` of `nparts` of the tile descriptors of both GEMMs (the tile
// list split evenly): tile i belongs to the group at the plan position whose
// tile range holds i; row tile mt of a group holds its 32-row blocks
// [mt*b/mt_n, (mt+1)*b/mt_n).
__device__ void plan_fill(const DevCtx& c, int T, const int* s_eoff, int (*s_t)[kMaxExperts + 2], const int* s_ord,
                          int part, int nparts) {
    const int G = c.G;
    for (int m = 0; m < 2; ++m) {
        int4* tinfo = m == 0 ? c.tinfo1 : c.tinfo2;
        const int maxt = m == 0 ? c.max_tiles1 : c.max_tiles2;
        const int total = min(s_t[m][G], maxt);
        const int per = (total + nparts - 1) / nparts;
        const int i1 = min(total, (part + 1) * per);
        for (int i = part * per + (int)threadIdx.x; i < i1; i += blockDim.x) {
            int lo = 0, hi = G;  // s_t[m][lo] <= i < s_t[m][hi]
            while (hi - lo > 1) {
                const int mid = (lo + hi) >> 1;
                if (s_t[m][mid] <= i) lo = mid;
                else hi = mid;
            }
            const int j = s_ord[lo];
            const PlanGroup g = plan_group(c, T, s_eoff, j, m + 1);
            const int local = i - s_t[m][lo];
            // panel pp of width w, row tile mt, column tile nt (panel order)
            const int pw = min(kPanel, g.nt);
            const int pp = min(div_small(local, pw * g.mt), div_small(g.nt - 1, pw));
            const int w = min(pw, g.nt - pp * pw);
            const int within = local - pp * pw * g.mt;
            const int mt = div_small(within, w), nt = pp * pw + within - mt * w;
            const int b0 = div_small(mt * g.blocks, g.mt), b1 = div_small((mt + 1) * g.blocks, g.mt);
            const int row0 = (c.has_shared && j == 0) ? 0 : s_eoff[j - c.has_shared];
            tinfo[i] = make_int4(j, nt | ((b1 - b0) << 16), row0 + b0 * 32, min(b1 * 32, g.M) - b0 * 32);
        }
    }
}

// ---------------------------------------------------------------------------
// a3 (second half): the stable dispatch permutation ("[RFC]: Async GPU
// Connector", "Data flow": argsort(stable=True) over the flattened ids,
// bincount, cumsum).  Every workgroup scans the expert counts into the
// expert offsets and the GEMM plan prefixes and writes its share of the
// tile descriptors (workgroup 0 also publishes the offsets, the tile
// prefixes and the segments).  Pair f = t*K + k goes to eoff[e] + #{f' < f :
// ids_f' = e}: the chunk's base per expert from k_scan plus the number of
// earlier tokens of the chunk that chose e (a token's K experts are
// distinct, so that is the pair's rank inside the chunk): a bit mask of the
// chunk's tokens per expert and a population count.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_permute(DevCtx c, const int* status) {
    static_assert(kRouteChunk <= 32 && kRouteChunk * kMaxTopK <= 256, "chunk masks and one pair per thread");
    static_assert(kMaxExperts <= 4 * 256, "at most four expert counts per thread");
    __shared__ int sh[16];
    __shared__ long long sh4[64];
    __shared__ int s_eoff[kMaxExperts + 1];
    __shared__ int s_t[2][kMaxExperts + 2];
    __shared__ long long s_c[2][kMaxExperts + 2];
    __shared__ int s_ord[kMaxExperts + 1];
    __shared__ int s_nh;
    __shared__ uint32_t emask[kMaxExperts];
    __shared__ uint64_t ltok[kRouteChunk];
    const int E = c.E, K = c.K, tid = threadIdx.x;
    // Loads that do not depend on each other are issued together, so their
    // latencies overlap: the status word, the token count and the peer
    // offsets (chunk_range); then this chunk's expert ids and token-row
    // addresses with the expert counts; then the chunk's base in each of its
    // pairs' expert groups, which arrives while the plan is computed.
    const int st = *status;
    const int T = *c.Tptr;
    int t0 = 0, t1 = 0, p = 0;
    const bool have = chunk_range(c, blockIdx.x, t0, t1, p);
    if (st != AFD_OK) return;
    const int nt = have ? t1 - t0 : 0, np = nt * K;
    int e = 0;
    uint64_t trow = 0;
    if (tid < np) e = c.ids[(int64_t)t0 * K + tid];
    if (tid < nt) trow = c.tok_src[t0 + tid];
    const int per = (E + 255) / 256;
    const int e0 = tid * per, e1 = min(E, e0 + per);
    int cnt[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) cnt[j] = e0 + j < e1 ? c.counts[e0 + j] : 0;
    int base = 0;
    if (tid < np) base = c.blk_base[(int64_t)e * c.NB + blockIdx.x];
    {
        int run = block_excl_scan(cnt[0] + cnt[1] + cnt[2] + cnt[3], sh);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e0 + j < e1) {
                s_eoff[e0 + j] = run;
                run += cnt[j];
            }
        if (tid == 255) s_eoff[E] = run;
    }
    for (int q = tid; q < E; q += 256) emask[q] = 0u;
    if (tid < nt) ltok[tid] = trow;
    __syncthreads();
    plan_prefix(c, T, s_eoff, s_t, s_c, s_ord, &s_nh, sh4);
    if (blockIdx.x == 0) {
        for (int e = tid; e <= E; e += 256) c.eoff[e] = s_eoff[e];
        plan_publish(c, T, s_eoff, s_t, s_c, s_ord, s_nh);
    }
    plan_fill(c, T, s_eoff, s_t, s_ord, (int)blockIdx.x, (int)gridDim.x);
    if (!have) return;
    if (tid < np) atomicOr(&emask[e], 1u << (tid / K));
    __syncthreads();
    if (tid < np) {
        const int tl = tid / K;
        const int pos = s_eoff[e] + base + __popc(emask[e] & ((1u << tl) - 1u));
        const int f = t0 * K + tid;
        if (pos < T * K) {
            c.perm[pos] = f;
            c.psrc[pos] = ltok[tl];
            if (c.w1_fp8) c.sxp[pos] = c.sx[t0 + tl];
        }
        c.inv[f] = pos;
    }
}

// ---------------------------------------------------------------------------
// a2 + a3 in one launch, for work items of at most kSmallT tokens (decode-
// shaped batches): k_route's grid routes the chunks, and the last of its
// workgroups to finish (a device-scope counter: each releases its writes
// before counting itself, the last acquires them) builds the per-expert
// counts, the stable dispatch order and the GEMM plan of k_scan + k_permute,
// without their launches.  From the routed ids it sets bit t of each
// selected expert's token mask; pair f = t*K + k then goes to eoff[e] +
// (tokens before t that chose e), the stable position k_permute computes
// from its chunk bases.
// ---------------------------------------------------------------------------
#ifndef AFD_SMALL_T
#define AFD_SMALL_T 256
#endif
constexpr int kSmallT = AFD_SMALL_T;
constexpr int kSmallW = kSmallT / 32;  // mask words per expert
constexpr int kSmallIds = kSmallT * kMaxTopK / (64 * kRouteChunk);  // pair slots per thread

template <int EPL, bool Q>
__global__ __launch_bounds__(64 * kRouteChunk) void k_route_small(DevCtx c, int* status, int s) {
    __shared__ int sh[16];
    __shared__ long long sh4[64];
    __shared__ int s_eoff[kMaxExperts + 1];
    __shared__ int s_t[2][kMaxExperts + 2];
    __shared__ long long s_c[2][kMaxExperts + 2];
    __shared__ int s_ord[kMaxExperts + 1];
    __shared__ int s_nh;
    __shared__ uint32_t emask[kMaxExperts][kSmallW];
    __shared__ uint64_t s_src[kSmallT];
    __shared__ float s_sx[kSmallT];
    __shared__ int s_off[kMaxPeers + 1];
    __shared__ int s_last;
    const int tid = threadIdx.x, lane = tid & 63;
    {
        // every workgroup counts itself, whatever it had to do
        const int st = *status;
        int t_begin, t_end, p;
        const bool have = chunk_range(c, blockIdx.x, t_begin, t_end, p);
        const int t = t_begin + (tid >> 6);
        bool bad = false;
        if (st == AFD_OK && have && t < t_end)
            bad = route_one<EPL, Q>(c, slot_ptr(c, c.in_win, p, s), t, t - c.off[p], lane, [](int) {});
        if (bad) atomicCAS(status, AFD_OK, AFD_ERR_HEADER);
        __syncthreads();
        if (tid == 0) {
            // release the workgroup's routing (its stores completed at the barrier)
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
            s_last = atomicAdd(c.route_done, 1) == (int)gridDim.x - 1;
        }
        __syncthreads();
        if (!s_last) return;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");  // every workgroup's routing
    if (tid == 0) *c.route_done = 0;  // (the next run's launch starts after this one)
    // The tail's inputs, loaded together so that their latencies overlap: the
    // status, the token count, the fan-in offsets, the expert of every pair
    // slot of the window's Tmax = P * token_cap <= kSmallT tokens (slots past
    // the run's T * K pairs hold stale values and go unused) and every
    // token's row address (and fp8 scale).
    const int E = c.E, K = c.K, NT = blockDim.x, Tm = c.hsrows;
    const int st = __hip_atomic_load(status, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int T = *c.Tptr;
    int idv[kSmallIds];
#pragma unroll
    for (int i = 0; i < kSmallIds; ++i) {
        const int f = tid + i * NT;
        idv[i] = f < Tm * K ? c.ids[f] : 0;
    }
    const uint64_t tsrc = tid < Tm ? c.tok_src[tid] : 0;
    const float tsx = c.w1_fp8 && tid < Tm ? c.sx[tid] : 0.0f;
    const int toff = tid <= c.P ? c.off[tid] : 0;
    if (st != AFD_OK) return;
    if (T > kSmallT || Tm > kSmallT || Tm * K > kSmallIds * NT) {  // (the launcher picks this kernel only when Tmax <= kSmallT)
        if (tid == 0) atomicCAS(status, AFD_OK, AFD_ERR_INVALID);
        return;
    }
    for (int i = tid; i < E * kSmallW; i += NT) (&emask[0][0])[i] = 0u;
    if (tid < T) s_src[tid] = tsrc;
    if (tid < T) s_sx[tid] = tsx;
    if (tid <= c.P) s_off[tid] = toff;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kSmallIds; ++i) {
        const int f = tid + i * NT;
        if (f < T * K) atomicOr(&emask[idv[i]][(f / K) >> 5], 1u << ((f / K) & 31));
    }
    __syncthreads();
    // counts (bincount), expert offsets, per-peer counts
    {
        int cnt = 0;
        if (tid < E)
#pragma unroll
            for (int w = 0; w < kSmallW; ++w) cnt += __popc(emask[tid][w]);
        const int run = block_excl_scan(tid < E ? cnt : 0, sh);
        if (tid < E) {
            s_eoff[tid] = run;
            c.counts[tid] = cnt;
            c.eoff[tid] = run;
        }
        if (tid == E - 1) {
            s_eoff[E] = run + cnt;
            c.eoff[E] = run + cnt;
        }
    }
    for (int i = tid; i < c.P * E; i += NT) {
        const int q = i / E, e = i - q * E;
        const int a = s_off[q], b = s_off[q + 1];
        int n = 0;
        for (int w = a >> 5; a < b && w <= (b - 1) >> 5; ++w) {
            uint32_t m = emask[e][w];
            const int lo = w * 32;
            if (a > lo) m &= ~0u << (a - lo);
            if (b < lo + 32) m &= (1u << (b - lo)) - 1u;
            n += __popc(m);
        }
        c.peer_counts[q * E + e] = n;
    }
    __syncthreads();
    plan_prefix(c, T, s_eoff, s_t, s_c, s_ord, &s_nh, sh4);
    plan_publish(c, T, s_eoff, s_t, s_c, s_ord, s_nh);
    plan_fill(c, T, s_eoff, s_t, s_ord, 0, 1);  // (this one workgroup writes every tile)
    // the stable dispatch position of every pair
#pragma unroll
    for (int i = 0; i < kSmallIds; ++i) {
        const int f = tid + i * NT;
        if (f >= T * K) continue;
        const int t = f / K;
        const int e = idv[i];
        int below = 0;
        for (int w = 0; w < (t >> 5); ++w) below += __popc(emask[e][w]);
        below += __popc(emask[e][t >> 5] & ((1u << (t & 31)) - 1u));
        const int pos = s_eoff[e] + below;
        c.perm[pos] = f;
        c.psrc[pos] = s_src[t];
        if (c.w1_fp8) c.sxp[pos] = s_sx[t];
        c.inv[f] = pos;
    }
}

// ---------------------------------------------------------------------------
// Attention-routed runs, FFN side.  Each message's routed rows arrive
// grouped by expert, with the group list (rows per expert) in its header
// ("[RFC]: Async GPU Connector", "Data flow", steps 2-3), so the FFN side
// routes nothing and merges the P group lists.  The grouped GEMM takes its
// rows expert-major, then peer, then the peer's own order: the order the
// stable sort of an FFN-routed run gives, so in both modes every GEMM row
// has the same place and the tile plan is the same.
// k_gscan: workgroup p < P scans peer p's group list over the experts (the
// first row of each group in the peer's slot, kept in blk_counts[p][e])
// and keeps the list for the return header; every other workgroup takes
// one expert per thread and scans the lists over the peers (the peer's
// first row inside the expert's group, blk_base[p][e]) and sums them.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_gscan(DevCtx c, const int* status, int s) {
    if (*status != AFD_OK) return;
    __shared__ int sh[16];
    const int E = c.E, P = c.P, b = blockIdx.x, tid = threadIdx.x;
    if (b < P) {
        const bool live = c.off[b + 1] > c.off[b];  // (a peer not served has no tokens)
        const int* cnt = (const int*)(slot_ptr(c, c.in_win, b, s) + c.foff[AFD_FIELD_HEADER]) + AFD_HDR_WORDS;
        const int per = (E + 255) / 256;
        const int e0 = tid * per, e1 = min(E, e0 + per);
        int v[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) v[j] = live && e0 + j < e1 ? cnt[e0 + j] : 0;
        int run = block_excl_scan(v[0] + v[1] + v[2] + v[3], sh);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e0 + j < e1) {
                c.blk_counts[b * E + e0 + j] = run;
                c.peer_counts[b * E + e0 + j] = v[j];
                run += v[j];
            }
        if (tid == 255) c.prow[b] = run;  // the peer's routed rows
        return;
    }
    const int e = (b - P) * 256 + tid;
    if (e >= E) return;
    int run = 0;
    for (int q = 0; q < P; ++q) {
        const int* cnt = (const int*)(slot_ptr(c, c.in_win, q, s) + c.foff[AFD_FIELD_HEADER]) + AFD_HDR_WORDS;
        const int v = c.off[q + 1] > c.off[q] ? cnt[e] : 0;
        c.blk_base[q * E + e] = run;
        run += v;
    }
    c.counts[e] = run;
}

// k_gdispatch: the expert offsets and the GEMM plan as in k_permute, then
// for every GEMM row pos its expert (the group holding pos), its peer (the
// share holding it) and its row in that peer's slot: the token-row address
// for the gate/up GEMM and the return row (peer * token_cap*K + row) for
// k_retcopy.  Shared rows: addresses and the shared_idx check as in k_route.
__global__ __launch_bounds__(256) void k_gdispatch(DevCtx c, int* status, int s) {
    __shared__ int sh[16];
    __shared__ long long sh4[64];
    __shared__ int s_eoff[kMaxExperts + 1];
    __shared__ int s_t[2][kMaxExperts + 2];
    __shared__ long long s_c[2][kMaxExperts + 2];
    __shared__ int s_ord[kMaxExperts + 1];
    __shared__ int s_nh;
    __shared__ int s_off[kMaxPeers + 1];
    const int st = *status;
    const int T = *c.Tptr;
    const int toff = (int)threadIdx.x <= c.P ? c.off[threadIdx.x] : 0;
    if (st != AFD_OK) return;
    const int E = c.E, K = c.K, P = c.P, tid = threadIdx.x;
    if (tid <= P) s_off[tid] = toff;  // (read after the barriers of the scans below)
    {
        const int per = (E + 255) / 256;
        const int e0 = tid * per, e1 = min(E, e0 + per);
        int cnt[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) cnt[j] = e0 + j < e1 ? c.counts[e0 + j] : 0;
        int run = block_excl_scan(cnt[0] + cnt[1] + cnt[2] + cnt[3], sh);
#pragma unroll
        for (int j = 0; j < 4; ++j)
            if (e0 + j < e1) {
                s_eoff[e0 + j] = run;
                run += cnt[j];
            }
        if (tid == 255) s_eoff[E] = run;
    }
    __syncthreads();
    plan_prefix(c, T, s_eoff, s_t, s_c, s_ord, &s_nh, sh4);
    if (blockIdx.x == 0) {
        for (int e = tid; e <= E; e += 256) c.eoff[e] = s_eoff[e];
        plan_publish(c, T, s_eoff, s_t, s_c, s_ord, s_nh);
    }
    plan_fill(c, T, s_eoff, s_t, s_ord, (int)blockIdx.x, (int)gridDim.x);
    const int n = min(T * K, s_eoff[E]);  // (k_wait checked that every group list covers its rows)
    const int stride = (int)gridDim.x * 256;
    for (int pos = (int)blockIdx.x * 256 + tid; pos < n; pos += stride) {
        int lo = 0, hi = E;  // s_eoff[lo] <= pos < s_eoff[hi]
        while (hi - lo > 1) {
            const int mid = (lo + hi) >> 1;
            if (s_eoff[mid] <= pos) lo = mid;
            else hi = mid;
        }
        const int q = pos - s_eoff[lo];
        int pl = 0, ph = P;  // base(pl) <= q < base(ph), base(P) = the group's size
        while (ph - pl > 1) {
            const int mid = (pl + ph) >> 1;
            if (c.blk_base[mid * E + lo] <= q) pl = mid;
            else ph = mid;
        }
        const int local = c.blk_counts[pl * E + lo] + q - c.blk_base[pl * E + lo];
        const int64_t so = c.slots_off + (int64_t)(pl * c.R + s) * c.slot_bytes + c.foff[AFD_FIELD_ROUTED_X] +
                           (int64_t)local * c.H * 2;  // (same layout in both windows)
        c.psrc[pos] = (uint64_t)(c.in_win + so);
        c.retoff[pos] = (uint32_t)so;
    }
    if (c.has_shared) {
        bool bad = false;
        for (int t = (int)blockIdx.x * 256 + tid; t < T; t += stride) {
            // its peer: the last p with off[p] <= t (off[P] = T > t)
            int pl = 0, ph = P;
            while (ph - pl > 1) {
                const int mid = (pl + ph) >> 1;
                if (s_off[mid] <= t) pl = mid;
                else ph = mid;
            }
            const int p = pl, r = t - s_off[p];
            const char* slot = slot_ptr(c, c.in_win, p, s);
            c.sh_src[t] = (uint64_t)(slot + c.foff[AFD_FIELD_SHARED_X] + (int64_t)r * c.H * 2);
            c.retoffs[t] = (uint32_t)(slot - c.in_win + c.foff[AFD_FIELD_SHARED_X] + (int64_t)r * c.H * 2);
            bad |= ((const int*)(slot + c.foff[AFD_FIELD_SHARED_IDX]))[r] != r;
        }
        if (bad) atomicCAS(status, AFD_OK, AFD_ERR_HEADER);
    }
}

// fp8 W1 on an attention-routed window: every GEMM row (the grouped pair
// rows, then the shared rows) quantised like a token row in k_route, one
// wavefront a row: codes to its own xq row, scale beside it, and the row
// address pointed there.  Pair rows are copies of their token's row, so
// they get that row's codes and scale.
__global__ __launch_bounds__(256) void k_gquant(DevCtx c, const int* status) {
    const int st = *status;
    const int T = *c.Tptr;
    if (st != AFD_OK) return;
    const int lane = threadIdx.x & 63, n8 = c.H / 8;
    const int nr = min(T * c.K, c.eoff[c.E]), rows = nr + (c.has_shared ? T : 0);
    for (int g = (int)blockIdx.x * 4 + (int)(threadIdx.x >> 6); g < rows; g += (int)gridDim.x * 4) {
        const bool routed = g < nr;
        const int64_t q = routed ? g : (int64_t)c.hrows + (g - nr);  // its xq / sxp row
        uint64_t* src = routed ? &c.psrc[g] : &c.sh_src[g - nr];
        const u32x4* xr = (const u32x4*)*src;
        float amax = 0.0f;
        for (int i = lane; i < n8; i += 64) {
            const u32x4 v8 = xr[i];
#pragma unroll
            for (int j = 0; j < 4; ++j)
                amax = fmaxf(amax, fmaxf(fabsf(bf2f(v8[j] & 0xffffu)), fabsf(bf2f(v8[j] >> 16))));
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
        const float rs = amax > 0.0f ? __fdiv_rn(448.0f, amax) : 0.0f;
        uint2* dst = (uint2*)(c.xq + q * c.H);
        for (int i = lane; i < n8; i += 64) {
            const u32x4 v8 = xr[i];
            dst[i] = make_uint2(pack4_e4m3(bf2f(v8[0] & 0xffffu) * rs, bf2f(v8[0] >> 16) * rs,
                                           bf2f(v8[1] & 0xffffu) * rs, bf2f(v8[1] >> 16) * rs),
                                pack4_e4m3(bf2f(v8[2] & 0xffffu) * rs, bf2f(v8[2] >> 16) * rs,
                                           bf2f(v8[3] & 0xffffu) * rs, bf2f(v8[3] >> 16) * rs));
        }
        if (lane == 0) {
            c.sxp[q] = amax > 0.0f ? __fdiv_rn(amax, 448.0f) : 1.0f;
            *src = (uint64_t)(c.xq + q * c.H);
        }
    }
}

// ---------------------------------------------------------------------------
// a4/a5/a6: grouped GEMMs on MFMA (v_mfma_f32_32x32x16_bf16).
//
// A tile is up to 256 token rows of one group (8 blocks of 32) x 256 weight
// rows, 32 deep per step.  256 threads = 4 waves, one per SIMD, placed 2
// (token) x 2 (weight): wave (wx, ww) owns the token blocks wx, wx+2, wx+4,
// wx+6 of the tile (a partly filled tile keeps both token positions equally
// loaded; blocks past the tile's end are skipped) and four 32-row weight
// blocks: up to 16 accumulators of 32 x 32 in AGPRs.  Per 16-deep slice a
// wave reads 4 + 4 fragments of 1 KB from LDS and issues 16 MFMAs.  Operands
// are K-contiguous rows, so every fragment is one 16-byte LDS read per lane.
// The token fragment is the MFMA's first operand: a lane's accumulator holds
// one output column (lane % 32) of 16 token rows, and one store instruction
// writes 32 consecutive columns of two rows.
//
// Global -> LDS: direct-to-LDS 16-byte loads into a ring of 4 stages of
// 32 KB (16 KB token rows, 16 KB weight rows), issued 3 steps ahead; LDS
// rows of 64 bytes hold their four 16-byte chunks XOR-swizzled (swz4), which
// keeps the fragment reads of consecutive rows on distinct banks.  The
// weight rows come from the packed weight copy, already in that order: each
// load instruction copies one contiguous KB.  All LDS lives in one array
// (with a second __shared__ variable the compiler attaches alias scopes and
// makes every LDS read wait for the direct-to-LDS loads in flight).
//
// MODE 1 (gate/up + SwiGLU): token rows are read straight from the inbound
//   slots through the per-pair row address (shared rows through the
//   shared_x row address); the weight rows are 128 gate rows and the same
//   128 up rows of W13, and wave ww takes gate blocks 2ww, 2ww+1 and the
//   matching up blocks, so each lane holds gate and up of the same (row,
//   column) and applies silu(g) * u in registers; h is stored bf16,
//   depth-block major.
// MODE 2 (down): token rows are the group's h rows, weight rows 256 rows of
//   W2; output rows are stored bf16, routed rows in permuted order (y),
//   shared rows in token order (ys).
//
// Persistent: one workgroup per CU takes tiles from per-XCD segments of the
// device-built tile list (see the scheduler below).  Rows past the group end
// and columns past the width load valid rows and are dropped at the store;
// depth past K loads valid data whose token-row copies are zeroed before the
// MFMAs.
// ---------------------------------------------------------------------------

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ inline void dma16(const void* g, lds_ptr_t l) { __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0); }

// s_waitcnt with only the vector-memory counter limited (gfx9 encoding).
#define AFD_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 15) | (((n) >> 4) << 14))



// Workgroup barrier that the compiler may not move memory accesses across
// (a plain s_barrier: __syncthreads would also drain the load counters).
#define AFD_BARRIER()                        \
    do {                                     \
        asm volatile("" ::: "memory");       \
        __builtin_amdgcn_s_barrier();        \
        asm volatile("" ::: "memory");       \
    } while (0)

constexpr int kRowBytes = kBK * 2;                      // 64: one row segment of a depth step
constexpr int kRowsPerLoad = 1024 / kRowBytes;          // 16 rows per 1 KB load instruction
constexpr int kBlockBytes = 32 * kRowBytes;             // 2 KB per 32-row block
constexpr int kXStageBytes = kBX * kRowBytes;           // 16 KB of token rows
constexpr int kStageBytes = (kBX + kBW) * kRowBytes;    // 32 KB
constexpr int kGemmWaves = kGemmThreads / 64;           // 4
// Down GEMM of an attention-routed run storing straight into the return
// slots: two tables (the current tile's and the next one's) of the tile's
// 256 row offsets sit in LDS past the ring and the tile-index slot; rows past
// the tile get an offset past any such window (those windows are < 1 GiB).
constexpr int kRetTabOff = kStages * kStageBytes + 64;
constexpr int kSmemBytes = kRetTabOff + 2 * kBX * 4;
constexpr uint32_t kRetPast = 0x40000000u;
constexpr int kXInstr = kBX / kRowsPerLoad / kGemmWaves;  // 4 token-row loads per wave and step
constexpr int kWInstr = kBW / kRowsPerLoad / kGemmWaves;  // 4 weight-row loads per wave and step
static_assert(kGemmWaves == 4 && kTileBlocks == 8 && kBK == 32 && kStages == 4,
              "wave placement, swizzle and ring assume 4 waves, 8 token blocks, 32-deep steps, 4 stages");

// LDS swizzle of 64-byte row segments: logical chunk c of row r sits at
// chunk c ^ swz4(r).  The 16-byte fragment reads of 8 (or 16) consecutive
// rows at one logical chunk then hit distinct banks.  swz4(r) depends on r
// mod 8 only, so it is the same for every 32-row block and for every load
// instruction (16 rows each).
__device__ inline int swz4(int r) { return ((r >> 1) ^ (r >> 2)) & 3; }

// ---------------------------------------------------------------------------
// Weight packing (one-time per layer): one thread per 16-byte chunk of the
// packed tiles (the layout next to struct Weights).  Chunk position p of
// row r of a tile holds depth values kt*32 + 8*(p ^ swz4(r)) .. +7 of the
// tile's weight row r, or zeros past the matrix.
// ---------------------------------------------------------------------------
// fp8 W1: each W13 / Ws13 row's max |w|, one wavefront per row, into the
// row-scale arrays of the packed weights (rows e*2I + j, then 2I*E + j for
// the shared rows); k_wscale turns them into dequantisation scales once the
// tiles are written.
__global__ __launch_bounds__(256) void k_wamax(DevCtx c, afd_moe_weights src, float* sw13, float* sws13) {
    const int64_t nr = (int64_t)c.E * 2 * c.I, ns = c.has_shared ? 2 * (int64_t)c.Is : 0;
    const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    if (row >= nr + ns) return;
    const u32x4* x = (const u32x4*)((row < nr ? (const uint16_t*)src.w13 + row * c.H
                                               : (const uint16_t*)src.ws13 + (row - nr) * c.H));
    float amax = 0.0f;
    for (int i = lane; i < c.H / 8; i += 64) {
        const u32x4 v8 = x[i];
#pragma unroll
        for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf2f(v8[j] & 0xffffu)), fabsf(bf2f(v8[j] >> 16))));
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
    if (lane == 0) (row < nr ? sw13[row] : sws13[row - nr]) = amax;
}

__global__ __launch_bounds__(256) void k_wscale(float* s, int64_t n) {
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) s[i] = s[i] > 0.0f ? __fdiv_rn(s[i], 448.0f) : 1.0f;
}

__global__ __launch_bounds__(256) void k_pack_weights(DevCtx c, afd_moe_weights src, char* dst, int64_t off1,
                                                      int64_t off2, int64_t off3, int64_t total, const float* amax13,
                                                      const float* amaxs13) {
    const int64_t H = c.H, I = c.I, Is = c.Is;
    const bool f8 = c.w1_fp8;  // gate/up tiles of e4m3 codes: 64 depth values a row
    const int64_t nk1 = f8 ? H / 64 : (H + kBK - 1) / kBK, nk2 = (I + kBK - 1) / kBK, nk2s = (Is + kBK - 1) / kBK;
    const int64_t nt1 = c.nt1, nt1s = (Is + kBW / 2 - 1) / (kBW / 2), nt2 = c.nt2;
    const int64_t nchunks = total / 16;
    for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nchunks; q += (int64_t)gridDim.x * blockDim.x) {
        const int64_t byte = q * 16;
        const int region = byte < off1 ? 0 : byte < off2 ? 1 : byte < off3 ? 2 : 3;
        const int64_t local = byte - (region == 0 ? 0 : region == 1 ? off1 : region == 2 ? off2 : off3);
        const int64_t tile = local / kWTileBytes;
        const int within = (int)(local % kWTileBytes);
        const int r = within / kRowBytes, p = (within % kRowBytes) / 16;
        const int64_t ks = tile % (region < 2 ? nk1 : region == 2 ? nk2 : nk2s);
        const int64_t k0 = f8 && region < 2 ? ks * 64 + 16 * (p ^ swz4(r)) : ks * kBK + 8 * (p ^ swz4(r));
        const int64_t tt = tile / (region < 2 ? nk1 : region == 2 ? nk2 : nk2s);  // column tile (and expert)
        const uint16_t* row = nullptr;
        if (region == 0 || region == 1) {
            const int64_t Ig = region == 0 ? I : Is, nt = region == 0 ? tt % nt1 : tt % nt1s;
            const int64_t jj = nt * (kBW / 2) + (r & (kBW / 2 - 1));
            if (jj < Ig && k0 < H) {
                const int64_t srow = (r < kBW / 2 ? 0 : Ig) + jj;
                row = region == 0 ? (const uint16_t*)src.w13 + ((tt / nt1) * 2 * I + srow) * H
                                  : (const uint16_t*)src.ws13 + srow * H;
            }
        } else {
            const int64_t Ig = region == 2 ? I : Is, nt = tt % nt2;
            const int64_t n = nt * kBW + r;
            if (n < H && k0 < Ig)
                row = region == 2 ? (const uint16_t*)src.w2 + ((tt / nt2) * H + n) * I : (const uint16_t*)src.ws2 + n * Is;
        }
        u32x4 v = {0u, 0u, 0u, 0u};
        if (row && f8 && region < 2) {
            // 16 codes of the row: r = 448 / max|w|, code = e4m3(w * r)
            const int64_t srow = (row - (region == 0 ? (const uint16_t*)src.w13 : (const uint16_t*)src.ws13)) / H;
            const float am = region == 0 ? amax13[srow] : amaxs13[srow];
            const float rs = am > 0.0f ? __fdiv_rn(448.0f, am) : 0.0f;
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const u32x4 w8 = *(const u32x4*)(row + k0 + 8 * h);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const uint32_t lo = e4m3_code(bf2f(w8[j] & 0xffffu) * rs), hi = e4m3_code(bf2f(w8[j] >> 16) * rs);
                    v[2 * h + (j >> 1)] |= (lo | (hi << 8)) << (16 * (j & 1));
                }
            }
        } else if (row) {
            v = *(const u32x4*)(row + k0);
        }
        *(u32x4*)(dst + byte) = v;
    }
}

hipError_t launch_pack_weights(const DevCtx& c, const afd_moe_weights& src, char* dst, const int64_t off[6],
                               int64_t total, hipStream_t st) {
    // (the tiles end at off[4]; the fp8 row scales follow)
    const int64_t nchunks = off[4] / 16;
    const int64_t blocks = std::min<int64_t>((nchunks + 255) / 256, 65536);
    float* s13 = (float*)(dst + off[4]);
    float* ss13 = (float*)(dst + off[5]);
    const int64_t nr = (int64_t)c.E * 2 * c.I, ns = c.has_shared ? 2 * (int64_t)c.Is : 0;
    if (c.w1_fp8) hipLaunchKernelGGL(k_wamax, dim3((unsigned)((nr + ns + 3) / 4)), dim3(256), 0, st, c, src, s13, ss13);
    if (blocks > 0)
        hipLaunchKernelGGL(k_pack_weights, dim3((unsigned)blocks), dim3(256), 0, st, c, src, dst, off[1], off[2],
                           off[3], off[4], s13, ss13);
    if (c.w1_fp8) {
        hipLaunchKernelGGL(k_wscale, dim3((unsigned)((nr + 255) / 256)), dim3(256), 0, st, s13, nr);
        if (ns) hipLaunchKernelGGL(k_wscale, dim3((unsigned)((ns + 255) / 256)), dim3(256), 0, st, ss13, ns);
    }
    (void)total;
    return hipGetLastError();
}

// What one wave needs to know about the current tile.
struct GemmTile {
    const char* abase;  // token-row base (inbound window, h or hs)
    const char* bbase;  // weight-row base (this group's W13 / W2 slice)
    // Load instruction i of the wave covers stage rows 16*(wid + 4i) .. +15;
    // its lane offset (row offset + this lane's swizzled chunk) is fixed for
    // the tile, the depth step moves the wave-uniform base.
    uint32_t xo[kXInstr];
    uint32_t astep;        // token-side bytes per depth step (64 in slot rows, rows*64 in h / hs)
    uint32_t wlane;        // this lane's byte in a packed weight tile's first KB of the wave
    uint32_t cx;           // this lane's logical chunk, as a byte offset
    uint32_t tail_clamp;   // last 16-byte chunk of a slot row (K-tail loads of the gate/up GEMM)
    int tb;                // 32-row token blocks of the tile, 1..8
    int nk, kfull, Kdim;   // depth steps, steps fully inside K, K
    int r0;                // first token row of the tile (h / y / ys row; fan-in token for shared rows)
    int rows, Ig, nt;      // valid token rows, the group's intermediate width, column tile
    bool sh;
    int part;              // depth part of a split shared down-GEMM tile (-1: whole depth)
    int par;               // which of the two LDS row tables is this tile's
    uint32_t rofs;         // this thread's row's entry of the table: its return offset (down GEMM
                           // storing into the return slots) or its token scale (fp8 gate/up GEMM)
    float dw[4];           // fp8 gate/up GEMM: this lane's gate (0, 1) and up (2, 3) column scales
};


// Direct-to-LDS loads of depth step kt into `stage` (lane l of instruction
// i fills bytes 16 l of the instruction's 1 KB: row 16(wid + 4i) + l/4,
// LDS chunk l % 4, which holds the swizzled logical chunk the lane
// fetches).  NX of the 4 token-row loads are issued, enough for the tile's
// blocks: NX = ceil(tb / 2) covers rows below 64 NX >= 32 tb (rows past the
// tile's blocks are valid rows that land in LDS rows the MFMAs do not read).
// The weight rows come from the packed tile of the step, already in LDS
// order: each instruction copies one contiguous KB.  In the gate/up GEMM a
// step past the end of K (K not a multiple of 32) loads each token row's
// last 16 bytes in place of the missing chunks -- valid, finite data -- and
// the token-row copies of those chunks are zeroed in LDS before the MFMAs;
// h and hs rows are stored in whole 32-deep blocks.
template <int MODE, int NX>
__device__ __forceinline__ void gemm_issue_x(const GemmTile& t, char* stage, int wid, int kt) {
    const char* ab = t.abase + (int64_t)kt * t.astep;
    uint32_t fix = 0u;
    if (MODE == 1) {
        const uint32_t kb = (uint32_t)kt * kRowBytes;
        fix = kb + t.cx > t.tail_clamp ? t.tail_clamp - kb - t.cx : 0u;
    }
#pragma unroll
    for (int i = 0; i < NX; ++i)
        dma16(ab + (t.xo[i] + fix), (lds_ptr_t)(stage + (wid + kGemmWaves * i) * 1024));
}
__device__ __forceinline__ void gemm_issue_w(const GemmTile& t, char* stage, int wid, int kt) {
    const char* bb = t.bbase + (int64_t)kt * kWTileBytes;
#pragma unroll
    for (int i = 0; i < kWInstr; ++i)
        dma16(bb + (t.wlane + i * kGemmWaves * 1024), (lds_ptr_t)(stage + kXStageBytes + (wid + kGemmWaves * i) * 1024));
}
// Both halves of a step, weight rows first (the order every step keeps).
template <int MODE, int NX>
__device__ __forceinline__ void gemm_issue(const GemmTile& t, char* stage, int wid, int kt) {
    gemm_issue_w(t, stage, wid, kt);
    gemm_issue_x<MODE, NX>(t, stage, wid, kt);
}


// Fragments of one 16-deep slice: 4 weight fragments and NV token fragments.
template <int NV>
struct GemmFrags {
    bf16x8 w[4];
    bf16x8 x[NV > 0 ? NV : 1];
};

// Reads slice kk (0 or 1) of the stage at `rd`.  The wave's weight fragment
// jb sits at wl + (MODE 1) ((jb >> 1) * 4 + (jb & 1)) or (MODE 2) jb blocks
// of 2 KB, its token fragment ib at tl + ib * 4 KB; slice kk flips address
// bit 5 (the swizzled chunk).
template <int MODE, int NV>
__device__ __forceinline__ void gemm_frags(GemmFrags<NV>& f, const char* rd, int kk, uint32_t wl, uint32_t tl) {
    const char* w = rd + (wl ^ (32u * kk));
    const char* x = rd + (tl ^ (32u * kk));
#pragma unroll
    for (int jb = 0; jb < 4; ++jb)
        f.w[jb] = __builtin_bit_cast(bf16x8, *(const u32x4*)(w + (MODE == 1 ? (jb >> 1) * 4 + (jb & 1) : jb) * kBlockBytes));
#pragma unroll
    for (int ib = 0; ib < NV; ++ib) f.x[ib] = __builtin_bit_cast(bf16x8, *(const u32x4*)(x + ib * 2 * kBlockBytes));
}

// The fragment reads of slice kk alternating, in program order, with NL
// loads issued by `load(i)`: read 0, load 0, read 1, load 1, ... (then the
// remaining reads).  With the matching scheduling pattern each wave spreads
// its global-to-LDS loads over the whole phase instead of issuing them in
// one burst that the CU's load path (which moves about 64 bytes per clock)
// can only drain while the wave stalls.
template <int MODE, int NV, int NL, typename Load>
__device__ __forceinline__ void gemm_frags_loads(GemmFrags<NV>& f, const char* rd, int kk, uint32_t wl, uint32_t tl,
                                                 Load load) {
    const char* w = rd + (wl ^ (32u * kk));
    const char* x = rd + (tl ^ (32u * kk));
    constexpr int NR = 4 + NV;
#pragma unroll
    for (int i = 0; i < (NR > NL ? NR : NL); ++i) {
        if (i < 4)
            f.w[i] = __builtin_bit_cast(bf16x8, *(const u32x4*)(w + (MODE == 1 ? (i >> 1) * 4 + (i & 1) : i) * kBlockBytes));
        else if (i < NR)
            f.x[i - 4] = __builtin_bit_cast(bf16x8, *(const u32x4*)(x + (i - 4) * 2 * kBlockBytes));
        if (i < NL) load(i);
    }
}

// In a step that reaches past K: token-fragment lanes whose chunk (8 depth
// values at kt*32 + (2*kk + lane/32)*8) lies at or past K become zero, so
// the (finite) clamped copies loaded there contribute nothing.  A select,
// not a branch, so the step stays one basic block.
template <int NV>
__device__ __forceinline__ void gemm_tail(GemmFrags<NV>& f, const GemmTile& t, int kt, int kk, int lane) {
    const bool past = kt * kBK + (2 * kk + (lane >> 5)) * 8 >= t.Kdim;
#pragma unroll
    for (int ib = 0; ib < NV; ++ib) {
        u32x4 v = __builtin_bit_cast(u32x4, f.x[ib]);
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = past ? 0u : v[q];
        f.x[ib] = __builtin_bit_cast(bf16x8, v);
    }
}

template <int NV>
__device__ __forceinline__ void gemm_mfma(f32x16 (&acc)[NV > 0 ? NV : 1][4], const GemmFrags<NV>& f) {
#pragma unroll
    for (int ib = 0; ib < NV; ++ib)
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            acc[ib][jb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(f.x[ib], f.w[jb], acc[ib][jb], 0, 0, 0);
}

// Scheduling pattern matching gemm_frags_loads: each MFMA followed by the
// next memory instruction in program order (reads and loads alternate while
// both remain).
template <int NMFMA, int NREAD, int NLOAD>
__device__ __forceinline__ void gemm_interleave_alt() {
    constexpr int NPAIR = NREAD < NLOAD ? NREAD : NLOAD;
    constexpr int NOPS = NREAD + NLOAD;
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < NOPS) {
            const bool rd = i < 2 * NPAIR ? (i % 2 == 0) : (NREAD > NLOAD);
            if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
            else __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
        }
    }
#pragma unroll
    for (int i = NMFMA; i < NOPS; ++i) {
        const bool rd = i < 2 * NPAIR ? (i % 2 == 0) : (NREAD > NLOAD);
        if (rd) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        else __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
}

// Scheduling pattern: each MFMA of the group followed by one of the slice's
// other memory instructions -- first its LDS reads, then its vector-memory
// loads (the loads write LDS, so the scheduler keeps them after the reads)
// -- so that the MFMA pipe stays fed while the wave issues them.
template <int NMFMA, int NREAD, int NLOAD>
__device__ __forceinline__ void gemm_interleave() {
#pragma unroll
    for (int i = 0; i < NMFMA; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (i < NREAD) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        else if (i - NREAD < NLOAD) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
    }
    if (NMFMA - NREAD < NLOAD) __builtin_amdgcn_sched_group_barrier(0x010, NLOAD - (NMFMA - NREAD), 0);
}

// One depth step kt of a wave with NV valid token blocks, software-
// pipelined around a single barrier; TAIL: the step reaches past K.  On
// entry `a` holds slice 0 of step kt.  (1) Slice 0's MFMAs, interleaved with
// the reads of slice 1 into `b` and the weight-row loads of step kt+3 into
// the stage step kt-1 used (every wave finished reading it before the
// previous step's barrier).  (2) This wave's slice-1 reads done and its
// loads of step kt+1 landed, then the barrier: step kt+1 is complete in LDS
// and every wave is done reading step kt.  (3) Slice 1's MFMAs, interleaved
// with the reads of slice 0 of step kt+1 into `a` and the token-row loads
// of step kt+3.  Splitting a step's loads over both phases spreads the
// global-to-LDS traffic, which all four waves issue in the same phases,
// over the whole step.  Each phase is one basic block: past the last step
// the loads reload the last step into the idle stage and the reads read a
// stage nobody uses.
template <int MODE, int NV, int NX, bool TAIL>
__device__ __forceinline__ void gemm_step(f32x16 (&acc)[NV > 0 ? NV : 1][4], const GemmTile& t, char* smem,
                                          int kt, int wid, int lane, uint32_t wl, uint32_t tl, GemmFrags<NV>& a,
                                          GemmFrags<NV>& b) {
    char* const ld = smem + ((kt + kStages - 1) & (kStages - 1)) * kStageBytes;
    const int kl = min(kt + kStages - 1, t.nk - 1);
    if (TAIL) gemm_tail(a, t, kt, 0, lane);
    {
        const char* bb = t.bbase + (int64_t)kl * kWTileBytes;
        gemm_frags_loads<MODE, NV, kWInstr>(b, smem + (kt & (kStages - 1)) * kStageBytes, 1, wl, tl, [&](int i) {
            dma16(bb + (t.wlane + i * kGemmWaves * 1024), (lds_ptr_t)(ld + kXStageBytes + (wid + kGemmWaves * i) * 1024));
        });
    }
    gemm_mfma(acc, a);
    gemm_interleave_alt<4 * NV, 4 + NV, kWInstr>();
    __builtin_amdgcn_sched_barrier(0);

    // step kt+1 landed: in flight may be only the loads of step kt+2 and the
    // weight-row loads of step kt+3 just issued
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    AFD_WAIT_VMCNT(NX + 2 * kWInstr);
    AFD_BARRIER();

    if (TAIL) gemm_tail(b, t, kt, 1, lane);
    {
        const char* ab = t.abase + (int64_t)kl * t.astep;
        uint32_t fix = 0u;
        if (MODE == 1) {
            const uint32_t kb = (uint32_t)kl * kRowBytes;
            fix = kb + t.cx > t.tail_clamp ? t.tail_clamp - kb - t.cx : 0u;
        }
        gemm_frags_loads<MODE, NV, NX>(a, smem + ((kt + 1) & (kStages - 1)) * kStageBytes, 0, wl, tl, [&](int i) {
            dma16(ab + (t.xo[i] + fix), (lds_ptr_t)(ld + (wid + kGemmWaves * i) * 1024));
        });
    }
    gemm_mfma(acc, b);
    gemm_interleave_alt<4 * NV, 4 + NV, NX>();
    __builtin_amdgcn_sched_barrier(0);
}

// fp8 gate/up GEMM: a step is 64 depth values (each 64-byte row holds e4m3
// codes).  A lane's operand for the block-scaled MFMA is its slice-0 chunk
// followed by its slice-1 chunk (the two 16-byte reads of a bf16 step); any
// split of the 64 values over a lane pair works as long as both operands use
// the same one.  Unit E8M0 scales (127); the row scales apply in the epilogue.
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ i32x8 cat_frag(bf16x8 lo, bf16x8 hi) {
    return __builtin_shufflevector(__builtin_bit_cast(i32x4, lo), __builtin_bit_cast(i32x4, hi), 0, 1, 2, 3, 4, 5,
                                   6, 7);
}

template <int NV>
__device__ __forceinline__ void gemm_mfma_f8(f32x16 (&acc)[NV > 0 ? NV : 1][4], const GemmFrags<NV>& a,
                                             const GemmFrags<NV>& b) {
#pragma unroll
    for (int ib = 0; ib < NV; ++ib) {
        const i32x8 x = cat_frag(a.x[ib], b.x[ib]);
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
            acc[ib][jb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(x, cat_frag(a.w[jb], b.w[jb]), acc[ib][jb],
                                                                          0, 0, 0, 127, 0, 127);
    }
}

// One fp8 step: slice 1 of stage kt (with the weight loads of step kt+3),
// then every MFMA of the step, then -- once stage kt+1 has landed -- slice 0
// of stage kt+1 (with the token loads of step kt+3).  The load pattern and
// the waits are the bf16 step's.
template <int NV, int NX>
__device__ __forceinline__ void gemm_step_f8(f32x16 (&acc)[NV > 0 ? NV : 1][4], const GemmTile& t, char* smem, int kt,
                                             int wid, int lane, uint32_t wl, uint32_t tl, GemmFrags<NV>& a,
                                             GemmFrags<NV>& b) {
    char* const ld = smem + ((kt + kStages - 1) & (kStages - 1)) * kStageBytes;
    const int kl = min(kt + kStages - 1, t.nk - 1);
    {
        const char* bb = t.bbase + (int64_t)kl * kWTileBytes;
        gemm_frags_loads<1, NV, kWInstr>(b, smem + (kt & (kStages - 1)) * kStageBytes, 1, wl, tl, [&](int i) {
            dma16(bb + (t.wlane + i * kGemmWaves * 1024), (lds_ptr_t)(ld + kXStageBytes + (wid + kGemmWaves * i) * 1024));
        });
    }
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): slice 1 is in
    gemm_mfma_f8(acc, a, b);
    __builtin_amdgcn_sched_barrier(0);
    AFD_WAIT_VMCNT(NX + 2 * kWInstr);
    AFD_BARRIER();
    {
        const char* ab = t.abase + (int64_t)kl * t.astep;
        gemm_frags_loads<1, NV, NX>(a, smem + ((kt + 1) & (kStages - 1)) * kStageBytes, 0, wl, tl, [&](int i) {
            dma16(ab + t.xo[i], (lds_ptr_t)(ld + (wid + kGemmWaves * i) * 1024));
        });
    }
    __builtin_amdgcn_sched_barrier(0);
}

// Tile scheduler of a workgroup.  Tiles are taken dynamically: a workgroup
// on XCD x (x = b % kXcds: workgroups are dispatched to the XCDs round-
// robin) takes tiles from the shared-expert segment x, then from the heavy
// routed segment x, then from the segments of XCD x+1, x+2, ..., and last
// from the light segments x, x+1, ...: every XCD starts on its share of the
// longest tiles, and the tiles of one segment, which share weight rows, stay
// in one XCD's L2 until other XCDs run dry.  One workgroup in kLightEvery
// takes the light segments first instead: the light tiles' time is the
// streaming of their weight rows, which a few workgroups do next to the
// compute-bound tiles of the others, with HBM to spare, rather than all
// workgroups at once at the end.  Wave 0 owns the grabbing: the grab of the
// next tile is issued kGrabAhead depth steps before the current tile ends
// (late enough that a workgroup does not hold a tile that an idle one could
// run, early enough that the atomic has returned when the tile ends),
// resolved at the tile boundary and broadcast through LDS.  When the current
// segment is drained, one batch of loads (a lane per segment) finds the next
// segment with tiles left.
constexpr int kGrabAhead = 3;

struct GemmSched {
    const int* seg;
    int* ctr;
    int x;                // this workgroup's XCD
    bool lf;              // light segments first
    int tries, si, pend;  // wave 0 only: position in the visiting order, its segment, the pending grab
};

// k-th segment visited by a workgroup on XCD x: shared and heavy segments
// alternate (x, x+1, ...), the light ones (x, x+1, ...) come last, or first
// for a light-first workgroup.
__device__ __forceinline__ int sched_seg(int x, int k, bool lf) {
    const int kl = lf ? k : k - 2 * kXcds;  // index among the light segments
    if (kl >= 0 && kl < kXcds) return 2 * kXcds + (x + kl) % kXcds;
    const int kh = lf ? k - kXcds : k;      // index among the shared / heavy ones
    return (kh & 1) * kXcds + (x + (kh >> 1)) % kXcds;
}

// Next tile, or -1 when all are taken (wave 0, all lanes; uniform result).
// Tile counters only grow, so a segment seen drained stays drained.
__device__ __forceinline__ int sched_grab_slow(GemmSched& s, int lane) {
    while (s.tries < kSegs) {
        bool left = false;
        if (lane >= s.tries && lane < kSegs) {
            const int si = sched_seg(s.x, lane, s.lf);
            const int taken = __hip_atomic_load(&s.ctr[si], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            left = s.seg[si] + taken < s.seg[si + 1];
        }
        const uint64_t m = __ballot(left);
        if (m == 0) {
            s.tries = kSegs;
            break;
        }
        s.tries = __builtin_ctzll(m);
        s.si = sched_seg(s.x, s.tries, s.lf);
        int t = 0;
        if (lane == 0) t = s.seg[s.si] + atomicAdd(&s.ctr[s.si], 1);
        t = __builtin_amdgcn_readfirstlane(t);
        if (t < __builtin_amdgcn_readfirstlane(s.seg[s.si + 1])) return t;
        ++s.tries;  // lost the race for the segment's last tiles
    }
    return -1;
}

// First tile of a workgroup (wave 0, all lanes; uniform result).  Without
// an atomic where the planner reserved one (its tile counters start past
// these): a light-first workgroup of rank li among the light-first ones of
// its XCD takes tile li of its light segment; a normal one of rank ni among
// the normal ones takes tile ni of the concatenation of its shared segment,
// its heavy segment and the light segment past the light-first share.  The
// others grab.
__device__ __forceinline__ int sched_first(GemmSched& s, int lane) {
    const int i = (int)blockIdx.x / kXcds;
    int v = 0;
    if (lane < 6) v = s.seg[(lane >> 1) * kXcds + s.x + (lane & 1)];
    const int b0 = __builtin_amdgcn_readlane(v, 0), b1 = __builtin_amdgcn_readlane(v, 1);
    const int b2 = __builtin_amdgcn_readlane(v, 2), b3 = __builtin_amdgcn_readlane(v, 3);
    const int b4 = __builtin_amdgcn_readlane(v, 4), b5 = __builtin_amdgcn_readlane(v, 5);
    if (s.lf) {
        const int li = i / kLightEvery;
        if (li < b5 - b4) {
            s.si = 2 * kXcds + s.x;  // (visit 0 of a light-first workgroup)
            return b4 + li;
        }
    } else {
        const int ni = i - i / kLightEvery - 1;
        if (ni < b1 - b0) {
            s.si = s.x;  // (visit 0)
            return b0 + ni;
        }
        if (ni < (b1 - b0) + (b3 - b2)) {
            s.tries = 1;
            s.si = kXcds + s.x;  // (visit 1)
            return b2 + ni - (b1 - b0);
        }
        // past the light-first workgroups' share of the light segment (the
        // visiting order restarts at visit 0 once the segment is drained)
        const int nx = ((int)gridDim.x - s.x + kXcds - 1) / kXcds;
        const int li = (nx + kLightEvery - 1) / kLightEvery + ni - (b1 - b0) - (b3 - b2);
        if (li < b5 - b4) {
            s.si = 2 * kXcds + s.x;
            return b4 + li;
        }
    }
    return sched_grab_slow(s, lane);
}

__device__ __forceinline__ void sched_issue(GemmSched& s, int lane) {  // wave 0
    if (s.tries < kSegs && lane == 0) s.pend = atomicAdd(&s.ctr[s.si], 1);
}

// Resolve the grab issued near the end of the current tile (wave 0).
__device__ __forceinline__ int sched_next(GemmSched& s, int lane) {
    if (s.tries >= kSegs) return -1;
    const int t = __builtin_amdgcn_readfirstlane(s.seg[s.si] + s.pend);
    if (t < __builtin_amdgcn_readfirstlane(s.seg[s.si + 1])) return t;
    ++s.tries;
    return sched_grab_slow(s, lane);
}

// Per-tile state of the wave: group, rows, depth, and the row offsets of its
// load instructions.
template <int MODE, bool F8>
__device__ __forceinline__ void gemm_setup(const DevCtx& c, const Weights& w, int tile, int wid, int lrow, uint32_t lcx,
                                           GemmTile& t) {
    // (every value here is wave-uniform: keep them in scalar registers)
    const int4 ti = (MODE == 1 ? c.tinfo1 : c.tinfo2)[__builtin_amdgcn_readfirstlane(tile)];
    const int j = __builtin_amdgcn_readfirstlane(ti.x), ty = __builtin_amdgcn_readfirstlane(ti.y);
    t.nt = ty & 0xffff;
    t.tb = ty >> 16;
    t.r0 = __builtin_amdgcn_readfirstlane(ti.z);
    t.rows = __builtin_amdgcn_readfirstlane(ti.w);
    t.sh = c.has_shared && j == 0;
    const int e = j - c.has_shared;
    t.Ig = t.sh ? c.Is : c.I;
    t.Kdim = MODE == 1 ? c.H : t.Ig;
    // (fp8 gate/up: e4m3 rows, 64 depth values a step; hidden is a multiple of 64)
    constexpr bool f8 = F8;
    t.nk = f8 ? c.H / 64 : (t.Kdim + kBK - 1) / kBK;
    t.kfull = f8 ? t.nk : t.Kdim / kBK;
    t.tail_clamp = (uint32_t)t.Kdim * 2 - 16;
    // a split shared down-GEMM tile: part p of the column tile covers depth
    // steps [p*nk/parts, (p+1)*nk/parts); k0 moves both operand bases, and
    // the depth left from its start stands for K in the tile's K-tail test
    int k0 = 0;
    t.part = -1;
    if (MODE == 2 && t.sh && c.shp > 1) {
        t.part = t.nt / c.nt2;
        t.nt -= t.part * c.nt2;
        k0 = t.part * t.nk / c.shp;
        const int k1 = (t.part + 1) * t.nk / c.shp;
        t.Kdim -= k0 * kBK;
        t.kfull = min(k1 - k0, t.Kdim / kBK);
    }
    // Token rows: slot rows through their row addresses (gate/up; 32-bit
    // byte offsets from the window, which stays below 4 GiB: checked at
    // create) or rows of the depth-block-major h / hs (down).
    if (MODE == 1) {
        t.abase = F8 ? (const char*)c.xq : c.in_win;  // (fp8: the quantised token rows)
        t.astep = kRowBytes;
    } else {
        t.astep = (uint32_t)(t.sh ? c.hsrows : c.hrows) * kRowBytes;
        t.abase = (const char*)(t.sh ? c.hs : c.h) + (int64_t)k0 * t.astep;
    }
    // this group's packed weight tiles of column tile nt: nk consecutive tiles
    if (MODE == 1) t.bbase = t.sh ? w.ws13 + (int64_t)t.nt * t.nk * kWTileBytes
                                  : w.w13 + ((int64_t)e * c.nt1 + t.nt) * t.nk * kWTileBytes;
    else t.bbase = t.sh ? w.ws2 + ((int64_t)t.nt * t.nk + k0) * kWTileBytes
                        : w.w2 + ((int64_t)e * c.nt2 + t.nt) * t.nk * kWTileBytes;
    if (t.part >= 0) t.nk = (t.part + 1) * t.nk / c.shp - k0;
    t.wlane = (uint32_t)wid * 1024u + (uint32_t)(threadIdx.x & 63) * 16u;
    t.cx = lcx;
    if constexpr (F8) {
        t.tail_clamp = (uint32_t)c.H - 16;
        const int r = threadIdx.x;  // row r of the tile: its token scale, for the LDS table
        t.rofs = __float_as_uint(r < t.rows ? c.sxp[(t.sh ? (int64_t)c.hrows : 0) + t.r0 + r] : 0.0f);
        const float* sw = t.sh ? w.sws13 : w.sw13 + (int64_t)e * 2 * c.I;
        const int lj = threadIdx.x & 31;
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int col = t.nt * (kBW / 2) + (wid >> 1) * 64 + jb * 32 + lj;
            t.dw[jb] = col < t.Ig ? sw[col] : 0.0f;
            t.dw[2 + jb] = col < t.Ig ? sw[t.Ig + col] : 0.0f;
        }
    }
    if (MODE == 2 && c.direct_ret) {
        // row threadIdx.x of the tile: its return-window offset, or past the
        // window's end (the store's range check drops it)
        const int r = threadIdx.x;
        t.rofs = r < t.rows ? (t.sh ? c.retoffs : c.retoff)[t.r0 + r] : kRetPast;
    }
#pragma unroll
    for (int i = 0; i < kXInstr; ++i) {
        const int r = (wid + kGemmWaves * i) * kRowsPerLoad + lrow;
        const int m = t.r0 + (r < t.rows ? r : 0);
        uint32_t o;
        if (MODE == 1) o = (uint32_t)((t.sh ? c.sh_src[m] : c.psrc[m]) - (uint64_t)t.abase);
        else o = (uint32_t)m * kRowBytes;
        t.xo[i] = o + lcx;
    }
}

// The first kStages-1 steps of a tile go into stages 0 .. (the ring must be
// free; a tile shorter than the ring reloads its last step), one step per
// call so that the tile boundary can spread them over the epilogue of the
// previous tile.  All four token-row loads are issued whatever the tile's
// height (the extra ones load valid rows into LDS rows the MFMAs do not
// read): the first waits of the tile, sized for its own NX, then wait for at
// least as many loads as they need, and there is no branch on the tile's
// height among the loads.
template <int MODE>
__device__ __forceinline__ void gemm_prologue_step(const GemmTile& t, char* smem, int wid, int p) {
    gemm_issue<MODE, kXInstr>(t, smem + p * kStageBytes, wid, min(p, t.nk - 1));
}
template <int MODE>
__device__ __forceinline__ void gemm_prologue(const GemmTile& t, char* smem, int wid) {
#pragma unroll
    for (int p = 0; p < kStages - 1; ++p) gemm_prologue_step<MODE>(t, smem, wid, p);
}

// Tile boundary, between the last depth step of the current tile and its
// epilogue: once every wave is done with the ring, resolve the next tile and
// set it up (its first loads are issued during the epilogue).
template <int MODE, bool F8>
__device__ __forceinline__ void gemm_boundary(const DevCtx& c, const Weights& w, GemmSched& sc, char* smem, int tid,
                                              int wid, int lrow, uint32_t lcx, int nk, int& next, GemmTile& tn) {
    int* slot = (int*)(smem + kStages * kStageBytes);
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS reads are done
    // the loads past the last step may target the epilogue's staging stage
    // unless nk is a multiple of kStages: then they land first
    if (nk & (kStages - 1)) AFD_WAIT_VMCNT(0);
    AFD_BARRIER();
    if (wid == 0) {
        const int t = sched_next(sc, tid);
        if (tid == 0) *slot = t;
    }
    __syncthreads();
    next = __builtin_amdgcn_readfirstlane(*slot);
    if (next >= 0) gemm_setup<MODE, F8>(c, w, next, wid, lrow, lcx, tn);
}

// Word 3 of a raw buffer descriptor on gfx9-family GPUs (32-bit data
// format, stride 0: accesses are range-checked against the byte count).
constexpr int kBufferFlags = 0x00020000;

// Buffer descriptor over `bytes` bytes at `base` (wave-uniform values, made
// explicitly scalar: a descriptor in vector registers would cost a
// waterfall loop around every access).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t out_rsrc(const void* base, uint32_t bytes) {
    const uint64_t a = (uint64_t)base;
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc((void*)(((uint64_t)hi << 32) | lo), 0,
                                            (int)__builtin_amdgcn_readfirstlane(bytes), kBufferFlags);
}

// One accumulator element read out of its AGPR.  Reading the accumulators
// one at a time keeps them in AGPRs until they are needed (the compiler
// would otherwise copy all of them to VGPRs at the end of the depth loop and
// run out of registers).  The caller leaves at least 18 wait states between
// the last MFMA and the first read (the hardware does not interlock an MFMA
// result read by a VALU instruction).
__device__ __forceinline__ float agpr(float x) {
    float r;
    asm("v_accvgpr_read_b32 %0, %1" : "=v"(r) : "a"(x));
    return r;
}

// Accumulator elements converted between two scheduling barriers of the
// epilogue (the barriers keep the compiler from moving every accumulator out
// of its AGPR at once).
#ifndef AFD_EPI_GROUP
#define AFD_EPI_GROUP 2
#endif
constexpr int kEpiGroup = AFD_EPI_GROUP;

// The epilogue stages each 32-row block of a wave's outputs through LDS and
// writes it with 16-byte stores: a CU's vector-memory unit takes about as
// long for an instruction of 2-byte lane stores as for one of 16-byte lane
// stores, so 64 lanes x 16 bytes per instruction (8 KB of a block in 8
// stores instead of 64) keeps the epilogue's stores from serialising.  The
// staging area is ring stage kStages-1: the next tile's prologue loads go to
// stages 0 .. kStages-2, and its step 0, which loads stage kStages-1, starts
// after a barrier that every wave reaches only after its epilogue.  (Loads
// past a tile's last step go to stages nk, nk+1, nk+2 mod kStages: when nk is
// not a multiple of kStages, the boundary waits for them first.)
constexpr int kEpiStage = (kStages - 1) * kStageBytes;
constexpr int kEpiWaveBytes = 32 * 128 * 2;  // one wave's 32 rows x 128 bf16 columns
static_assert(kEpiWaveBytes * kGemmWaves <= kStageBytes, "the epilogue staging fits one ring stage");

// Rows v and v+1 (v even) of a lane's column, packed bf16 (row v low), are
// regrouped with the neighbouring lane's (lanes 2m and 2m+1 hold adjacent
// columns; the DPP move quad_perm [1,0,3,2] brings the neighbour's pair):
// the even lane keeps row v of both columns, the odd lane row v+1, each as
// one dword whose low half is the even column -- a byte permutation of the
// two pairs with the lane's selector pair_sel.
__device__ __forceinline__ uint32_t pair_sel(int lane) { return (lane & 1) ? 0x03020706u : 0x05040100u; }

// Epilogue of token block ib of a tile.  In accumulator (ib, jb) a lane
// holds output column 32*(weight block) + (lane & 31) and, in register v =
// 0..15, token row (wx + 2*ib)*32 + 8*(v/4) + 4*(lane/32) + v%4 of the
// tile.  Pairs of rows are regrouped between neighbouring lanes (pair_sel)
// and written to the wave's staging area in LDS, row-major; each lane then
// reads back 16 bytes (8 columns of one row) and stores them.  The stores go
// through a buffer descriptor that spans the tile's valid rows (rows past
// them fall outside and the hardware drops the stores); a column block past
// the output width adds 2^31 to its offsets.  Straight-line code (a
// divergent branch would keep every accumulator live across it).  The
// caller pads the wait states between the last MFMA and the first
// accumulator read.  Depth-split shared tiles store their fp32 partial rows
// directly.
template <int MODE, int NV, bool F8>
__device__ __forceinline__ void gemm_epilogue_ib(const f32x16 (&acc)[NV > 0 ? NV : 1][4], const DevCtx& c,
                                                 const GemmTile& t, char* smem, int lane, int ww, int wx,
                                                 int ib) {
    const int lj = lane & 31;
    const uint32_t rb = (uint32_t)((wx + 2 * ib) * 32 + 4 * (lane >> 5));  // this lane's first row of the block
    const uint32_t row0 = (uint32_t)((wx + 2 * ib) * 32);                   // the block's first row
    const uint32_t sel = pair_sel(lane);
    char* scr = smem + kEpiStage + (2 * ww + wx) * kEpiWaveBytes;
    // this lane's staging dword for (row 8q + v%4 (+1 for odd lanes), its column pair): row r of
    // the block at r * RB bytes, column pair at 4 * (lj/2)
    const uint32_t wq = (uint32_t)((4 * (lane >> 5) + (lane & 1)) * (MODE == 1 ? 64 : 256) + (lj & 30) * 2);
    if (MODE == 1) {
        // h = silu(gate) * up, bf16; gate in weight blocks jb, up in jb + 2.
        // Column block jb is one 32-deep block of h: 32 rows of 64 bytes,
        // contiguous (2 KB), staged at jb * 2 KB.
        const int64_t hrows = t.sh ? c.hsrows : c.hrows;
        char* hb = (char*)(t.sh ? c.hs : c.h);
        // fp8: the token scales of this lane's rows rb + 8q + i
        float dx[4][4];
        if constexpr (F8) {
            const u32x4* tab = (const u32x4*)(smem + kRetTabOff + t.par * (kBX * 4));
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const u32x4 o = tab[(rb >> 2) + 2 * q];
#pragma unroll
                for (int i = 0; i < 4; ++i) dx[q][i] = __uint_as_float(o[i]);
            }
        }
        // in stages over 8 elements at a time (independent instructions
        // back to back, not one dependent chain per element)
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
#pragma unroll
            for (int h8 = 0; h8 < 16; h8 += 8) {
                float g[8], u[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    g[i] = agpr(acc[ib][jb][h8 + i]);
                    u[i] = agpr(acc[ib][jb + 2][h8 + i]);
                }
                if constexpr (F8) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float sxr = dx[(h8 + i) >> 2][(h8 + i) & 3];
                        g[i] = g[i] * sxr * t.dw[jb];
                        u[i] = u[i] * sxr * t.dw[2 + jb];
                    }
                }
                float e[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] = __expf(-g[i]);
#pragma unroll
                for (int i = 0; i < 8; ++i) e[i] = __builtin_amdgcn_rcpf(1.f + e[i]);
                uint32_t pk[4], nb[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    pk[i] = pk_bf16(g[2 * i] * e[2 * i] * u[2 * i], g[2 * i + 1] * e[2 * i + 1] * u[2 * i + 1]);
#pragma unroll
                for (int i = 0; i < 4; ++i) nb[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)pk[i], 0xB1, 0xF, 0xF, false);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int v = h8 + 2 * i;
                    const uint32_t r = (uint32_t)(8 * (v >> 2) + (v & 3));
                    *(uint32_t*)(scr + jb * 2048 + r * 64 + wq) = __builtin_amdgcn_perm(nb[i], pk[i], sel);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }
#pragma unroll
        for (int jb = 0; jb < 2; ++jb) {
            const int col0 = t.nt * (kBW / 2) + ww * 64 + jb * 32;
            const __amdgpu_buffer_rsrc_t rs =
                out_rsrc(hb + ((int64_t)(col0 >> 5) * hrows + t.r0) * kRowBytes, (uint32_t)t.rows * kRowBytes);
            // (a block past the width has no place in h; a partial one stores into its padding
            // columns, which the down GEMM masks)
            const uint32_t cb = (col0 < t.Ig ? 0u : 0x80000000u) + row0 * kRowBytes + (uint32_t)lane * 16;
#pragma unroll
            for (int hh = 0; hh < 2; ++hh) {
                const u32x4 d = *(const u32x4*)(scr + jb * 2048 + hh * 1024 + lane * 16);
                __builtin_amdgcn_raw_buffer_store_b128(d, rs, (int)(cb + hh * 1024), 0, 0);
            }
        }
    } else if (t.part >= 0) {
        // a split shared tile: its fp32 partial rows, part p's rows of ysp
        // (token order), 32 consecutive columns of two rows per store
        const uint32_t ldb = (uint32_t)c.H * 4;
        const __amdgpu_buffer_rsrc_t rs =
            out_rsrc(c.ysp + ((int64_t)t.part * c.hsrows + t.r0) * c.H, (uint32_t)t.rows * ldb);
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            const int col = t.nt * kBW + (ww * 4 + jb) * 32 + lj;
            const uint32_t cb = (col < c.H ? 0u : 0x80000000u) + (uint32_t)col * 4 + rb * ldb;
#pragma unroll
            for (int v = 0; v < 16; v += 2) {
                const uint32_t r = (uint32_t)(8 * (v >> 2) + (v & 3));
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(agpr(acc[ib][jb][v])), rs, (int)(cb + r * ldb), 0, 0);
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(agpr(acc[ib][jb][v + 1])), rs,
                                                      (int)(cb + (r + 1) * ldb), 0, 0);
                if ((v + 2) % kEpiGroup == 0) __builtin_amdgcn_sched_barrier(0);
            }
        }
    } else {
        // bf16 rows: routed rows into y (permuted order), shared rows into ys
        // (token order), or -- attention-routed runs -- each row straight to
        // its return row (offsets from the tile's LDS table, the buffer over
        // the whole return window).  Staged as 32 rows of 256 bytes (the
        // wave's 128 columns).
        // in stages over one accumulator (16 elements) at a time
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
            float a[16];
#pragma unroll
            for (int v = 0; v < 16; ++v) a[v] = agpr(acc[ib][jb][v]);
            uint32_t pk[8], nb[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) pk[i] = pk_bf16(a[2 * i], a[2 * i + 1]);
#pragma unroll
            for (int i = 0; i < 8; ++i) nb[i] = (uint32_t)__builtin_amdgcn_mov_dpp((int)pk[i], 0xB1, 0xF, 0xF, false);
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const int v = 2 * i;
                const uint32_t r = (uint32_t)(8 * (v >> 2) + (v & 3));
                *(uint32_t*)(scr + r * 256 + jb * 64 + wq) = __builtin_amdgcn_perm(nb[i], pk[i], sel);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        const uint32_t ldb = (uint32_t)c.H * 2;
        const bool direct = c.direct_ret;
        const char* ob = direct ? c.ret_win : (const char*)((t.sh ? c.ys : c.y) + (int64_t)t.r0 * c.H);
        const __amdgpu_buffer_rsrc_t rs = out_rsrc(ob, direct ? c.ret_bytes : t.rows * ldb);
        // lane: row 4i + lane/16 of the block, columns 8 * (lane % 16) .. + 8 of the wave's 128
        const int col = t.nt * kBW + ww * 128 + (lane & 15) * 8;  // (H is a multiple of 8)
        const uint32_t cb = (col < c.H ? 0u : 0x80000000u) + (uint32_t)col * 2;
        const uint32_t* tab = (const uint32_t*)(smem + kRetTabOff + t.par * (kBX * 4));
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t row = row0 + 4 * i + (lane >> 4);
            const uint32_t ro = direct ? tab[row] : row * ldb;
            const u32x4 d = *(const u32x4*)(scr + i * 1024 + lane * 16);
            __builtin_amdgcn_raw_buffer_store_b128(d, rs, (int)(cb + ro), 0, 0);
        }
    }
}

// The depth loop, the tile boundary and the epilogue of one tile for a wave
// with NV valid token blocks (its blocks wx, wx+2, .. below tb).  Steps 0 ..
// kStages-2 have been issued into stages 0 ...; on return `next` and `tn`
// describe the next tile (next < 0: none), whose first steps are loading.
template <int MODE, int NV, int NX, bool F8>
__device__ __forceinline__ void gemm_run(const DevCtx& c, const Weights& w, GemmSched& sc, const GemmTile& t,
                                         char* smem, int tid, int wid, int lane, int ww, int wx, uint32_t wl,
                                         uint32_t tl, int lrow, uint32_t lcx, int& next, GemmTile& tn) {
    constexpr int NA = NV > 0 ? NV : 1;
    f32x16 acc[NA][4];
#pragma unroll
    for (int a = 0; a < NA; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

    // step 0 landed (this wave's loads, then everyone's), slice 0 read
    AFD_WAIT_VMCNT((NX + kWInstr) * (kStages - 2));
    AFD_BARRIER();
    GemmFrags<NV> fa, fb;
    gemm_frags<MODE, NV>(fa, smem, 0, wl, tl);
    int kt = 0;
    const int kg = min(t.kfull, max(t.nk - kGrabAhead, 0));
    if (F8) {
        for (; kt < kg; ++kt) gemm_step_f8<NV, NX>(acc, t, smem, kt, wid, lane, wl, tl, fa, fb);
        if (wid == 0) sched_issue(sc, tid);  // the next tile
        for (; kt < t.nk; ++kt) gemm_step_f8<NV, NX>(acc, t, smem, kt, wid, lane, wl, tl, fa, fb);
    } else {
        for (; kt < kg; ++kt) gemm_step<MODE, NV, NX, false>(acc, t, smem, kt, wid, lane, wl, tl, fa, fb);
        if (wid == 0) sched_issue(sc, tid);  // the next tile
        for (; kt < t.kfull; ++kt) gemm_step<MODE, NV, NX, false>(acc, t, smem, kt, wid, lane, wl, tl, fa, fb);
        for (; kt < t.nk; ++kt) gemm_step<MODE, NV, NX, true>(acc, t, smem, kt, wid, lane, wl, tl, fa, fb);
    }

    gemm_boundary<MODE, F8>(c, w, sc, smem, tid, wid, lrow, lcx, t.nk, next, tn);
    tn.par = t.par ^ 1;

    // Epilogue, token block by token block, with the next tile's first
    // steps issued in between: the global-to-LDS traffic of those loads
    // (which the CU moves at a fixed rate) overlaps the epilogue instead of
    // stalling the wave in one burst.
    asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7");  // MFMA results settle (>= 18 wait states)
#pragma unroll
    for (int ib = 0; ib < (NV > kStages - 1 ? NV : kStages - 1); ++ib) {
        if (ib < kStages - 1 && next >= 0) gemm_prologue_step<MODE>(tn, smem, wid, ib);
        // the next tile's return offsets into its table (its load was issued at set-up)
        if (ib == 0 && next >= 0 && ((MODE == 2 && c.direct_ret) || F8))
            ((uint32_t*)(smem + kRetTabOff + tn.par * (kBX * 4)))[threadIdx.x] = tn.rofs;
        if (ib < NV) gemm_epilogue_ib<MODE, NV, F8>(acc, c, t, smem, lane, ww, wx, ib);
    }
}

// The tile loop of one workgroup; F8: the gate/up GEMM on e4m3 operands
// (decided once per launch, so the bf16 loop carries none of it).
template <int MODE, bool F8>
__device__ __forceinline__ void gemm_tiles(const DevCtx& c, const Weights& w, char* smem) {
    int* slot = (int*)(smem + kStages * kStageBytes);
    GemmSched sc;
    sc.seg = MODE == 1 ? c.seg1 : c.seg2;
    sc.ctr = c.tctr + (MODE - 1) * kSegs;
    const int total = sc.seg[kSegs];
    if (total <= 0 || total > (MODE == 1 ? c.max_tiles1 : c.max_tiles2)) return;  // nothing, or an insane plan
    sc.x = (int)(blockIdx.x % kXcds);
    sc.lf = (blockIdx.x / kXcds) % kLightEvery == 0;
    sc.tries = 0;
    sc.si = 0;
    sc.pend = 0;
    const int tid = threadIdx.x, lane = tid & 63;
    const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wx = wid & 1, ww = wid >> 1;

    const int lrow = lane >> 2;  // row inside a load instruction
    // logical chunk fetched by this lane: (lane % 4) ^ swz4(16q + lrow) =
    // (lane % 4) ^ swz4(lrow) for every load instruction q
    const uint32_t lcx = (uint32_t)(((lane & 3) ^ swz4(lrow)) * 16);
    // fragment byte offsets inside a stage: chunk ch = 2*kk + lane/32 of row
    // r = 32*b + (lane & 31) sits at r*64 + (ch ^ swz4(r))*16 = b * 2 KB +
    // fb ^ (32*kk) with fb = (lane & 31)*64 + ((lane/32) ^ swz4(lane))*16,
    // the same lane part for every block.  The wave's weight blocks are
    // (MODE 1) 2ww, 2ww+1, 4+2ww, 5+2ww and (MODE 2) 4ww .. 4ww+3, its token
    // blocks wx, wx+2, wx+4, wx+6; the ww and wx terms go into the bases.
    const uint32_t fb = (uint32_t)((lane & 31) * kRowBytes + (((lane >> 5) ^ swz4(lane & 31)) * 16));
    const uint32_t wl = kXStageBytes + (uint32_t)ww * (MODE == 1 ? 2 : 4) * kBlockBytes + fb;
    const uint32_t tl = (uint32_t)wx * kBlockBytes + fb;

    // first tile (the planner reserved the first ones for a grid of c.ncu
    // workgroups, the grid of every launch)
    if (wid == 0) {
        const int t0 = sched_first(sc, tid);
        if (tid == 0) *slot = t0;
    }
    __syncthreads();
    int tile = __builtin_amdgcn_readfirstlane(*slot);
    GemmTile t;
    if (tile >= 0) {
        gemm_setup<MODE, F8>(c, w, tile, wid, lrow, lcx, t);
        gemm_prologue<MODE>(t, smem, wid);
        t.par = 0;
        if ((MODE == 2 && c.direct_ret) || F8) ((uint32_t*)(smem + kRetTabOff))[threadIdx.x] = t.rofs;
    }
    while (tile >= 0) {
        int next;
        GemmTile tn;
        // this wave's valid token blocks NV = ceil((tb - wx) / 2) and the
        // token-row loads per wave and step NX = ceil(tb / 2)
#define AFD_RUN(NV, NX) gemm_run<MODE, NV, NX, F8>(c, w, sc, t, smem, tid, wid, lane, ww, wx, wl, tl, lrow, lcx, next, tn)
        switch (t.tb * 2 + wx) {  // key 2 tb + wx -> (NV, NX)
            case 17: case 16: case 14: AFD_RUN(4, 4); break;  // tb 8, tb 7 wx 0
            case 15: AFD_RUN(3, 4); break;                    // tb 7 wx 1
            case 13: case 12: case 10: AFD_RUN(3, 3); break;  // tb 6, tb 5 wx 0
            case 11: AFD_RUN(2, 3); break;                    // tb 5 wx 1
            case 9: case 8: case 6: AFD_RUN(2, 2); break;     // tb 4, tb 3 wx 0
            case 7: AFD_RUN(1, 2); break;                     // tb 3 wx 1
            case 5: case 4: case 2: AFD_RUN(1, 1); break;     // tb 2, tb 1 wx 0
            default: AFD_RUN(0, 1); break;                    // tb 1 wx 1
        }
#undef AFD_RUN
        tile = next;
        t = tn;
    }
    // drain this wave's surplus loads before the workgroup ends
    AFD_WAIT_VMCNT(0);
}

template <int MODE>
__global__ __launch_bounds__(kGemmThreads, 1) void k_gemm(DevCtx c, const int* status, Weights w_arg, int layer) {
    if (*status != AFD_OK) return;
    // layer < 0: the layer-table entry of the run's layer (checked by k_wait)
    const Weights w = layer < 0 ? c.wtable[*c.layer_cur] : w_arg;
    // One LDS array: the operand ring and, past it, the tile-index slot and
    // the row tables.  (With a second __shared__ variable the compiler
    // attaches alias scopes to LDS accesses and then makes every LDS read
    // wait for the direct-to-LDS loads in flight; with one array it does not.)
    __shared__ __attribute__((aligned(1024))) char smem[kSmemBytes];
    if constexpr (MODE == 1) {
        if (c.w1_fp8) gemm_tiles<MODE, true>(c, w, smem);
        else gemm_tiles<MODE, false>(c, w, smem);
    } else {
        gemm_tiles<MODE, false>(c, w, smem);
    }
}

// ---------------------------------------------------------------------------
// a7: combine + split + publish.  out[t] = rsf * sum_k w[t,k] * y[inv[t*K+k]]
// + S[t] in fp32 (k in order; S the bf16 shared-expert row), rounded to bf16
// and written into row t - off[p]
// of peer p's return slot ("Data flow": weighted index_add_ combine with the
// shared branch added; "Data on the wire", Step 4: split back by seq_lens).
// ---------------------------------------------------------------------------
// One 16-byte chunk (8 columns) of an output row: rsf * (sum over k, in k
// order, of w[k] * y_k) + the shared row, from bf16 rows, summed in fp32,
// rounded to bf16 (RNE).  The FFN-side combine and the attention-side
// combine of attention-routed messages both use it.
template <int KK>
__device__ __forceinline__ u32x4 combine_chunk(const u32x4 (&yv)[KK], const float (&wk)[KK], u32x4 sq, bool shared,
                                               float rsf) {
    float sv[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sv[2 * i] = shared ? bf2f(sq[i] & 0xffffu) : 0.f;
        sv[2 * i + 1] = shared ? bf2f(sq[i] >> 16) : 0.f;
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
    for (int i = 0; i < 4; ++i) out[i] = pk_bf16(rsf * acc[2 * i] + sv[2 * i], rsf * acc[2 * i + 1] + sv[2 * i + 1]);
    return out;
}

// One 16-byte chunk (8 columns) of token t's shared-expert row: the bf16
// row of ys, or -- depth-split shared tiles -- the fp32 parts summed in part
// order and rounded to bf16 (RNE) once.
__device__ __forceinline__ u32x4 shared_chunk(const DevCtx& c, int t, int ch) {
    if (c.shp <= 1) return *(const u32x4*)(c.ys + (int64_t)t * c.H + ch * 8);
    float s[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) s[i] = 0.f;
    const int64_t pstride = (int64_t)c.hsrows * c.H;
    const float* p0 = c.ysp + (int64_t)t * c.H + ch * 8;
    // every part's loads first (their latencies overlap), then the sum in part order
    float4 a[kShParts], b[kShParts];
#pragma unroll
    for (int p = 0; p < kShParts; ++p) {
        const bool have = p < c.shp;
        a[p] = have ? *(const float4*)(p0 + p * pstride) : make_float4(0.f, 0.f, 0.f, 0.f);
        b[p] = have ? *(const float4*)(p0 + p * pstride + 4) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
#pragma unroll
    for (int p = 0; p < kShParts; ++p) {
        if (p >= c.shp) break;
        s[0] += a[p].x; s[1] += a[p].y; s[2] += a[p].z; s[3] += a[p].w;
        s[4] += b[p].x; s[5] += b[p].y; s[6] += b[p].z; s[7] += b[p].w;
    }
    u32x4 o;
#pragma unroll
    for (int i = 0; i < 4; ++i) o[i] = pk_bf16(s[2 * i], s[2 * i + 1]);
    return o;
}

// Attention-routed runs with depth-split shared tiles: every token's shared
// row summed from its parts (shared_chunk) into the return slot's shared
// row (where the down GEMM stores the other rows itself) or into ys (copied
// there by k_retcopy).
__global__ __launch_bounds__(256) void k_shsum(DevCtx c, const int* status) {
    const int st = *status;
    const int T = *c.Tptr;
    if (st != AFD_OK) return;
    const int H8 = c.H / 8;
    for (int t = blockIdx.x; t < T; t += gridDim.x) {
        u32x4* dst = c.direct_ret ? (u32x4*)(c.ret_win + c.retoffs[t]) : (u32x4*)(c.ys + (int64_t)t * c.H);
        for (int ch = threadIdx.x; ch < H8; ch += blockDim.x) dst[ch] = shared_chunk(c, t, ch);
    }
}

// Token t of a combine workgroup: its K pair positions and weights, then
// its rows (all K loads of a chunk go out together), summed in k order.
// offq: the fan-in offsets one per lane (see k_combine).
template <int KK>
__device__ __forceinline__ void combine_token(const DevCtx& c, int t, int offq, int s, int npairs) {
    const int H = c.H, H8 = c.H / 8;
    int pos[KK];
    float wk[KK];
#pragma unroll
    for (int k = 0; k < KK; ++k) {
        pos[k] = min(max(c.inv[(int64_t)t * KK + k], 0), npairs - 1);
        wk[k] = c.wts[(int64_t)t * KK + k];
    }
    // the token's peer: the peers after the first whose tokens start at or
    // before it (offsets are nondecreasing, empty peers included)
    const int p = __popcll(__ballot(offq <= t));
    const int r = t - (p > 0 ? __builtin_amdgcn_readlane(offq, p - 1) : 0);
    u32x4* dst = (u32x4*)(slot_ptr(c, c.ret_win, p, s) + c.foff[AFD_FIELD_ROUTED_X] + (int64_t)r * H * 2);
    for (int ch = threadIdx.x; ch < H8; ch += blockDim.x) {
        u32x4 yv[KK];
#pragma unroll
        for (int k = 0; k < KK; ++k) yv[k] = *(const u32x4*)(c.y + (int64_t)pos[k] * H + ch * 8);
        const u32x4 sq = c.has_shared ? shared_chunk(c, t, ch) : (u32x4)0u;
        __builtin_nontemporal_store(combine_chunk<KK>(yv, wk, sq, c.has_shared, c.rsf), &dst[ch]);
    }
}

template <int KK>
__global__ __launch_bounds__(256) void k_combine(DevCtx c, const int* status, int s, int layer) {
    const int st = *status;  // loaded together with the token count and the offsets
    const int T = *c.Tptr;
    // lane q: the first token of peer q + 1 (past the last peer: none)
    const int lane = threadIdx.x & 63;
    const int offq = lane + 1 < c.P ? c.off[lane + 1] : INT_MAX;
    if (st != AFD_OK) return;
    const int npairs = T * KK;
    for (int t = blockIdx.x; t < T; t += gridDim.x) combine_token<KK>(c, t, offq, s, npairs);
}

// Attention-routed runs: no combine on the FFN side ("[RFC]: Async GPU
// Connector", "Data flow", step 4: the expert outputs go back in the order
// they came, the sender combines).  GEMM row pos goes to return-window byte
// offset retoff[pos] (its row in its peer's return routed_x), shared row t to
// retoffs[t].  One workgroup per row.  Used when the down GEMM cannot store
// there itself (a return window of 1 GiB or more).
__global__ __launch_bounds__(256) void k_retcopy(DevCtx c, const int* status, int s) {
    const int st = *status;
    const int T = *c.Tptr;
    if (st != AFD_OK) return;
    const int H8 = c.H / 8;
    const int nr = min(T * c.K, c.eoff[c.E]), rows = nr + (c.has_shared ? T : 0);
    for (int row = blockIdx.x; row < rows; row += gridDim.x) {
        const bool routed = row < nr;
        const int m = routed ? row : row - nr;
        const u32x4* src = (const u32x4*)((routed ? c.y : c.ys) + (int64_t)m * c.H);
        u32x4* dst = (u32x4*)(c.ret_win + (routed ? c.retoff : c.retoffs)[m]);
        for (int ch = threadIdx.x; ch < H8; ch += blockDim.x) __builtin_nontemporal_store(src[ch], &dst[ch]);
    }
}

// The return headers and flags, one thread per peer, launched after
// k_combine on the same stream: the kernel boundary makes every output row
// visible before any flag.  Each non-empty peer gets num_tokens, echo_seq =
// the inbound seq consumed, its per-expert pair counts, then a release store
// of its return flag = the FFN side's next return seq.  An empty message gets
// no reply and so creates no wait.
__global__ __launch_bounds__(64) void k_publish(DevCtx c, const int* status, int s, int layer, int serve_item) {
    if (serve_item >= 0 && blockIdx.x == 0 && threadIdx.x == 0 && c.serve[0] == AFD_OK) {
        // the item's outcome: one more done, or the stop of the loop
        const int r = *status;
        if (r == AFD_OK) {
            c.serve[1] += 1;
        } else {
            c.serve[0] = r;
            c.serve[2] = serve_item;
        }
    }
    if (*status != AFD_OK) return;
    const int p = blockIdx.x, lane = threadIdx.x;  // one wavefront per peer
    const int n_p = c.off[p + 1] - c.off[p];
    if (n_p == 0) return;
    const int idx = p * c.R + s;
    int32_t* w = (int32_t*)(slot_ptr(c, c.ret_win, p, s) + c.foff[AFD_FIELD_HEADER]);
    const int rs = c.ret_seq[idx] + 1;
    for (int e = lane; e < c.E; e += 64) w[AFD_HDR_WORDS + e] = c.peer_counts[p * c.E + e];
    if (lane == 0) {
        c.ret_seq[idx] = rs;
        afd_header_fields f;
        f.flags = 0;
        f.seq = rs;
        f.echo_seq = c.cur_seq[p];
        f.layer_idx = layer < 0 ? *c.layer_cur : layer;
        f.stage_idx = s;
        f.num_tokens = n_p;
        f.routed_tokens = c.attn_routes ? c.prow[p] : n_p;
        f.shared_tokens = c.has_shared ? n_p : 0;
        f.src_peer = p;
        f.n_counts = c.E;
        header_encode_fixed(f, w);
    }
    __threadfence();  // the wave's header stores (every lane) before the flag
    if (lane == 0) st_release((int*)c.ret_win + idx, rs);
}

// ---------------------------------------------------------------------------
// layer < 0: a layer-table run (the layer from the headers, the weights from
// the device table; `w` is unused).
__global__ void k_serve_begin(DevCtx c) {
    if (threadIdx.x == 0) {
        c.serve[0] = AFD_OK;
        c.serve[1] = 0;
        c.serve[2] = -1;
    }
}

__global__ __launch_bounds__(256) void k_zero(uint32_t* p, int64_t n) {
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) p[i] = 0u;
}

hipError_t launch_zero(void* p, int64_t bytes, hipStream_t st) {
    const int64_t n = bytes / 4;
    if (n <= 0) return hipSuccess;
    int64_t grid = (n + 255) / 256;
    if (grid > 1024) grid = 1024;
    k_zero<<<(int)grid, 256, 0, st>>>((uint32_t*)p, n);
    return hipGetLastError();
}

hipError_t launch_serve_begin(const DevCtx& c, hipStream_t st) {
    k_serve_begin<<<1, 64, 0, st>>>(c);
    return hipGetLastError();
}

hipError_t launch_ffn(const DevCtx& c, int stage, int layer, const Weights& w, long long timeout_ticks, int num_cu,
                      hipEvent_t* ev, hipStream_t st, int max_take, long long gather_ticks, int serve_item) {
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
    k_wait<<<1, 64, 0, st>>>(c, stage, layer, timeout_ticks, max_take, gather_ticks, serve_item);
    if (c.poison) {
        const int64_t n = (c.slot_bytes - c.foff[AFD_FIELD_ROUTE_TABLE]) / 4;
        k_poison_ret<<<dim3((unsigned)std::min<int64_t>((n + 255) / 256, 256), (unsigned)c.P), 256, 0, st>>>(c, status,
                                                                                                          stage);
    }
    mark();
    if (c.attn_routes) {
        // (the routing slots: the merge of the group lists, then the dispatch)
        k_gscan<<<c.P + (c.E + 255) / 256, 256, 0, st>>>(c, status, stage);
        mark();
        mark();
        k_gdispatch<<<c.NB, 256, 0, st>>>(c, status, stage);
        if (c.w1_fp8) k_gquant<<<num_cu * 4, 256, 0, st>>>(c, status);
    } else if (Tmax <= kSmallT) {
        // small work items: routing, counts, dispatch order and plan in one launch
        // (its time lands in the routing slot)
#define AFD_ROUTE_SMALL(EPL)                                                                 \
    (c.w1_fp8 ? k_route_small<EPL, true><<<c.NB, 64 * kRouteChunk, 0, st>>>(c, status, stage) \
              : k_route_small<EPL, false><<<c.NB, 64 * kRouteChunk, 0, st>>>(c, status, stage))
        if (c.E <= 64) AFD_ROUTE_SMALL(1);
        else if (c.E <= 128) AFD_ROUTE_SMALL(2);
        else if (c.E <= 256) AFD_ROUTE_SMALL(4);
        else if (c.E <= 512) AFD_ROUTE_SMALL(8);
        else AFD_ROUTE_SMALL(16);
#undef AFD_ROUTE_SMALL
        mark();
        mark();
    } else {
#define AFD_ROUTE(EPL)                                                                 \
    (c.w1_fp8 ? k_route<EPL, true><<<c.NB, 64 * kRouteChunk, 0, st>>>(c, status, stage) \
              : k_route<EPL, false><<<c.NB, 64 * kRouteChunk, 0, st>>>(c, status, stage))
        if (c.E <= 64) AFD_ROUTE(1);
        else if (c.E <= 128) AFD_ROUTE(2);
        else if (c.E <= 256) AFD_ROUTE(4);
        else if (c.E <= 512) AFD_ROUTE(8);
        else AFD_ROUTE(16);
#undef AFD_ROUTE
        mark();
        k_scan<<<c.E, 256, 0, st>>>(c, status);
        mark();
        k_permute<<<c.NB, 256, 0, st>>>(c, status);
    }
    mark();
    k_gemm<1><<<num_cu, kGemmThreads, 0, st>>>(c, status, w, layer);
    mark();
    k_gemm<2><<<num_cu, kGemmThreads, 0, st>>>(c, status, w, layer);
    mark();
    int cgrid = Tmax < num_cu * 32 ? Tmax : num_cu * 32;  // (one token a workgroup pass)
    if (cgrid < 1) cgrid = 1;
    if (c.attn_routes) {
        // (the down GEMM stored every row into the return slots itself unless the window is too large;
        // the shared rows of depth-split tiles are summed from their parts first)
        if (c.shp > 1) k_shsum<<<cgrid, 256, 0, st>>>(c, status);
        if (!c.direct_ret) k_retcopy<<<num_cu * 8, 256, 0, st>>>(c, status, stage);
        k_publish<<<c.P, 64, 0, st>>>(c, status, stage, layer, serve_item);
        mark();
        return hipGetLastError();
    }
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
    k_publish<<<c.P, 64, 0, st>>>(c, status, stage, layer, serve_item);
    mark();
    return hipGetLastError();
}

}  // namespace afd
