/*
 * afd_oracle.c -- plain, slow CPU oracle for the FFN-rank hot path of
 * Attention-FFN Disaggregation (AFD).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file.  Only the test suite, the smoke check and the CPU-baseline
 * leg of the benchmark use it.  It shares no code, header, table or helper
 * with the HIP library: it is written from the pages, step by step, in their
 * order, with no blocking, fusion or reordering beyond what they state.
 *
 * Precision: every accumulation is in double.  Inputs are bf16 bit patterns
 * (hidden states, weights; upcast exactly) and fp32 router logits.
 *
 * Sources (titles of the pages, with the section used):
 *   [RFC-GPU]  "[RFC]: Async GPU Connector" (vllm-project/afd-plugin #233):
 *              "Data flow" (plan_dispatch: flatten topk_ids, stable argsort,
 *              bincount, cumsum; shared rows; weighted index_add_ combine),
 *              "Attention gate and FFN expert compute" (grouped_topk gate,
 *              fused_experts over expert-grouped rows, shared expert,
 *              routed_scaling_factor).
 *   [WIRE]     "Data on the wire: tensors per layer and stage": Step 2
 *              (total_tokens is the sum of seq_lens), Step 3 (fan-in: peers
 *              concatenated along tokens in subgroup order), Step 4 (split
 *              back by the recorded seq_lens).
 *   [NPU-RFC]  "[RFC]: Async AFD for Prefill on Ascend NPU", "Architecture"
 *              (the routed W1 + SwiGLU grouped GEMM, quantised).
 *   [P2P-UG]   "NCCL_P2P_CONNECTOR_USER_GUIDE.md", Configuration
 *              (compute_gate_on_attention=true: router logits travel to the
 *              FFN, which runs the expert path).
 *
 * Readings taken where the pages are silent (each also listed in the design
 * notes): softmax scoring renormalised over the top-K; selection by fp32 logit
 * value, larger first, equal values to the lower expert index; SwiGLU expert
 * with W13 = [gate rows; up rows] of shape [2I][H] and W2 of shape [H][I];
 * silu(z) = z / (1 + exp(-z)); the shared expert is unweighted and added after
 * the routed sum; with one FFN replica every token is a shared row.
 *
 * Parity status: every function below is pinned by the CPU tests (invariants,
 * library special cases, a float64 dense brute force with no permutation).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#define ORC_OK 0
#define ORC_ERR_ARG (-1)
#define ORC_ERR_NONFINITE (-2)
#define ORC_ERR_CAPACITY (-3)

/* bf16 bit pattern -> double.  bf16 is the top half of an IEEE binary32, so
 * the conversion is exact. */
static double bf16_to_double(uint16_t b) {
    uint32_t u = ((uint32_t)b) << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

void oracle_set_threads(int n) {
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ---------------------------------------------------------------------------
 * Step a1: fan-in offsets.  [WIRE] Step 2 / Step 3: peers are concatenated in
 * subgroup order; total_tokens = sum(seq_lens).  off[p] is where peer p's
 * first token lands in the concatenation, off[P] = total_tokens.
 * ------------------------------------------------------------------------- */
int oracle_fanin(int P, const int32_t* seq_lens, int32_t token_cap, int32_t* off) {
    if (P < 1 || !seq_lens || !off) return ORC_ERR_ARG;
    off[0] = 0;
    for (int p = 0; p < P; ++p) {
        if (seq_lens[p] < 0) return ORC_ERR_ARG;
        if (token_cap > 0 && seq_lens[p] > token_cap) return ORC_ERR_CAPACITY;
        off[p + 1] = off[p] + seq_lens[p];
    }
    return ORC_OK;
}

/* Fan-in of a row-major per-peer tensor: out = concat_p src_p along rows. */
int oracle_concat_rows(int P, const int32_t* seq_lens, const void* const* src,
                       int64_t row_bytes, void* out) {
    if (P < 1 || !seq_lens || !src || !out) return ORC_ERR_ARG;
    char* dst = (char*)out;
    for (int p = 0; p < P; ++p) {
        int64_t nb = (int64_t)seq_lens[p] * row_bytes;
        if (nb > 0) memcpy(dst, src[p], (size_t)nb);
        dst += nb;
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Step a2: top-k routing.  [RFC-GPU] "Attention gate and FFN expert compute"
 * names vLLM's grouped_topk as the gate; with one expert group that is a plain
 * softmax top-k.  For each token the experts are sorted by (logit descending,
 * expert index ascending) and the first K are kept in that order.  Weights:
 * the softmax over all E experts, restricted to the K kept experts and (when
 * renorm != 0) divided by their sum, which is
 *   w_k = exp(L[ids_k] - L[ids_0]) / sum_j exp(L[ids_j] - L[ids_0]).
 * ------------------------------------------------------------------------- */

/* true when expert a ranks before expert b for this token */
static int ranks_before(const float* l, int a, int b) {
    /* -0.0 == +0.0 under IEEE comparison, so both compare as equal values. */
    if (l[a] > l[b]) return 1;
    if (l[a] < l[b]) return 0;
    return a < b;
}

int oracle_route(int64_t T, int E, int K, int renorm, const float* logits,
                 int32_t* ids, double* w) {
    if (T < 0 || E < 1 || K < 1 || K > E || (T > 0 && (!logits || !ids || !w)))
        return ORC_ERR_ARG;
    for (int64_t i = 0; i < T * (int64_t)E; ++i)
        if (!isfinite(logits[i])) return ORC_ERR_NONFINITE;
    int bad = 0;
#pragma omp parallel
    {
        int* order = (int*)malloc(sizeof(int) * (size_t)E);
        if (!order) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t t = 0; t < T; ++t) {
                const float* l = logits + t * E;
                /* insertion sort of the expert indices by rank */
                for (int e = 0; e < E; ++e) {
                    int j = e;
                    while (j > 0 && ranks_before(l, e, order[j - 1])) {
                        order[j] = order[j - 1];
                        --j;
                    }
                    order[j] = e;
                }
                for (int k = 0; k < K; ++k) ids[t * K + k] = order[k];
                double m = (double)l[order[0]];
                if (renorm) {
                    double s = 0.0;
                    for (int k = 0; k < K; ++k) s += exp((double)l[order[k]] - m);
                    for (int k = 0; k < K; ++k) w[t * K + k] = exp((double)l[order[k]] - m) / s;
                } else {
                    double s = 0.0; /* full softmax denominator over all E */
                    for (int e = 0; e < E; ++e) s += exp((double)l[e] - m);
                    for (int k = 0; k < K; ++k) w[t * K + k] = exp((double)l[order[k]] - m) / s;
                }
            }
            free(order);
        }
    }
    return bad ? ORC_ERR_ARG : ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Step a3: dispatch plan.  [RFC-GPU] "Data flow", plan_dispatch: flatten the
 * [T,K] expert ids to pairs f = t*K + k, argsort them stably by expert id,
 * bincount for the per-expert group sizes, cumsum for the group offsets.
 * The stable argsort over a small integer key is written as a counting sort:
 * pairs are visited in increasing f and each goes to the next free position
 * of its expert's group, which is exactly the stable order.
 *   counts[e]          = #{f : ids_f == e}
 *   expert_offsets[e]  = sum_{e' < e} counts[e']      (E+1 entries)
 *   perm[pos] = f, inv[f] = pos.
 * ------------------------------------------------------------------------- */
int oracle_dispatch(int64_t T, int E, int K, const int32_t* ids, int32_t* counts,
                    int32_t* expert_offsets, int32_t* perm, int32_t* inv) {
    if (T < 0 || E < 1 || K < 1 || !counts || !expert_offsets) return ORC_ERR_ARG;
    int64_t n = T * (int64_t)K;
    for (int e = 0; e < E; ++e) counts[e] = 0;
    for (int64_t f = 0; f < n; ++f) {
        if (ids[f] < 0 || ids[f] >= E) return ORC_ERR_ARG;
        counts[ids[f]] += 1;
    }
    expert_offsets[0] = 0;
    for (int e = 0; e < E; ++e) expert_offsets[e + 1] = expert_offsets[e] + counts[e];
    int32_t* next = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    if (!next) return ORC_ERR_ARG;
    for (int e = 0; e < E; ++e) next[e] = expert_offsets[e];
    for (int64_t f = 0; f < n; ++f) {
        int32_t pos = next[ids[f]]++;
        perm[pos] = (int32_t)f;
        inv[f] = pos;
    }
    free(next);
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Steps a4/a5 for one row: a SwiGLU expert (the expert FFN that vLLM's
 * fused_experts applies, [RFC-GPU] "Attention gate and FFN expert compute").
 *   g_j = sum_h x_h W13[j][h],  u_j = sum_h x_h W13[I+j][h]      (j < I)
 *   a_j = silu(g_j) * u_j,      silu(z) = z / (1 + exp(-z))
 *   y_c = sum_j a_j W2[c][j]                                      (c < H)
 * x: H bf16; w13: [2I][H] bf16; w2: [H][I] bf16; y: H doubles.
 * scratch: I doubles.
 * ------------------------------------------------------------------------- */
static void swiglu_row(int64_t H, int64_t I, const uint16_t* x, const uint16_t* w13,
                       const uint16_t* w2, double* act, double* y) {
    for (int64_t j = 0; j < I; ++j) {
        const uint16_t* wg = w13 + j * H;
        const uint16_t* wu = w13 + (I + j) * H;
        double g = 0.0, u = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            double xv = bf16_to_double(x[h]);
            g += xv * bf16_to_double(wg[h]);
            u += xv * bf16_to_double(wu[h]);
        }
        act[j] = (g / (1.0 + exp(-g))) * u;
    }
    for (int64_t c = 0; c < H; ++c) {
        const uint16_t* wr = w2 + c * I;
        double s = 0.0;
        for (int64_t j = 0; j < I; ++j) s += act[j] * bf16_to_double(wr[j]);
        y[c] = s;
    }
}

/* One SwiGLU row, exposed so that tests can pin it against a textbook
 * formula. */
int oracle_swiglu_row(int64_t H, int64_t I, const uint16_t* x, const uint16_t* w13,
                      const uint16_t* w2, double* y) {
    if (H < 1 || I < 1 || !x || !w13 || !w2 || !y) return ORC_ERR_ARG;
    double* act = (double*)malloc(sizeof(double) * (size_t)I);
    if (!act) return ORC_ERR_ARG;
    swiglu_row(H, I, x, w13, w2, act, y);
    free(act);
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Step a4/a5 over the dispatch plan: every expert e runs over its group
 * [expert_offsets[e], expert_offsets[e+1]) of the permuted pairs; the row of
 * pair perm[i] is token perm[i] / K.  Y[i] is the expert output for permuted
 * position i.  (The rows inside a group are independent, so they may run in
 * parallel without changing any result.)
 * ------------------------------------------------------------------------- */
int oracle_experts(int64_t T, int64_t H, int E, int K, int64_t I, const uint16_t* X,
                   const int32_t* expert_offsets, const int32_t* perm,
                   const uint16_t* W13, const uint16_t* W2, double* Y) {
    if (T < 0 || H < 1 || E < 1 || K < 1 || I < 1) return ORC_ERR_ARG;
    int bad = 0;
    for (int e = 0; e < E; ++e) {
        const uint16_t* w13 = W13 + (int64_t)e * 2 * I * H;
        const uint16_t* w2 = W2 + (int64_t)e * H * I;
        int64_t lo = expert_offsets[e], hi = expert_offsets[e + 1];
#pragma omp parallel
        {
            double* act = (double*)malloc(sizeof(double) * (size_t)I);
            if (!act) {
#pragma omp atomic write
                bad = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int64_t i = lo; i < hi; ++i) {
                    int64_t t = perm[i] / K;
                    swiglu_row(H, I, X + t * H, w13, w2, act, Y + i * H);
                }
                free(act);
            }
        }
    }
    return bad ? ORC_ERR_ARG : ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Step a6: the shared expert over the shared rows.  [RFC-GPU] "Data flow":
 * the shared rows of FFN rank r are arange(r, num_tokens, ffn_size); with one
 * FFN replica that is every token, carried in the slot's shared_x field.
 * S[t] = SwiGLU_shared(Xs[t]), Ws13 [2Is][H], Ws2 [H][Is].
 * ------------------------------------------------------------------------- */
int oracle_shared(int64_t T, int64_t H, int64_t Is, const uint16_t* Xs,
                  const uint16_t* Ws13, const uint16_t* Ws2, double* S) {
    if (T < 0 || H < 1 || Is < 1) return ORC_ERR_ARG;
    int bad = 0;
#pragma omp parallel
    {
        double* act = (double*)malloc(sizeof(double) * (size_t)Is);
        if (!act) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t) swiglu_row(H, Is, Xs + t * H, Ws13, Ws2, act, S + t * H);
            free(act);
        }
    }
    return bad ? ORC_ERR_ARG : ORC_OK;
}

/* ---------------------------------------------------------------------------
 * Step a7: combine.  [RFC-GPU] "Data flow": each token's expert outputs are
 * accumulated with its router weights (a weighted index_add_), and the shared
 * branch is added by shared_idx.
 *   out[t] = rsf * sum_{k<K} w[t,k] * Y[inv[t*K+k]]  +  S[t]      (k in order)
 * S may be NULL (no shared expert).
 * ------------------------------------------------------------------------- */
int oracle_combine(int64_t T, int64_t H, int K, double rsf, const double* w,
                   const int32_t* inv, const double* Y, const double* S, double* out) {
    if (T < 0 || H < 1 || K < 1) return ORC_ERR_ARG;
#pragma omp parallel for schedule(static)
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t c = 0; c < H; ++c) {
            double r = 0.0;
            for (int k = 0; k < K; ++k) r += w[t * K + k] * Y[(int64_t)inv[t * K + k] * H + c];
            out[t * H + c] = rsf * r + (S ? S[t * H + c] : 0.0);
        }
    }
    return ORC_OK;
}

/* ---------------------------------------------------------------------------
 * The whole path, a1..a7, on per-peer inputs.  Outputs the concatenated
 * result out[T][H] (split back per peer by off[], [WIRE] Step 4) and the
 * routing/dispatch artefacts for bit-exact comparison.
 *   x[p]: [seq_lens[p]][H] bf16;  l[p]: [seq_lens[p]][E] fp32
 *   ids [T*K], w [T*K], counts [E], expert_offsets [E+1], perm/inv [T*K],
 *   off [P+1], out [T*H] (all caller-allocated; any may be NULL except out,
 *   which the computation needs).
 * ------------------------------------------------------------------------- */
int oracle_ffn(int P, const int32_t* seq_lens, const uint16_t* const* x, const float* const* l,
               int64_t H, int E, int K, int64_t I, int64_t Is, double rsf, int renorm,
               const uint16_t* W13, const uint16_t* W2, const uint16_t* Ws13, const uint16_t* Ws2,
               int32_t* ids_out, double* w_out, int32_t* counts_out, int32_t* eoff_out,
               int32_t* perm_out, int32_t* inv_out, int32_t* off_out, double* out) {
    if (P < 1 || !seq_lens || H < 1 || E < 1 || K < 1 || K > E || I < 1 || !out) return ORC_ERR_ARG;
    int rc;
    int32_t* off = (int32_t*)malloc(sizeof(int32_t) * (size_t)(P + 1));
    if (!off) return ORC_ERR_ARG;
    rc = oracle_fanin(P, seq_lens, 0, off);
    if (rc) { free(off); return rc; }
    int64_t T = off[P], n = T * K;
    uint16_t* X = (uint16_t*)malloc(sizeof(uint16_t) * (size_t)(T * H + 1));
    float* L = (float*)malloc(sizeof(float) * (size_t)(T * E + 1));
    int32_t* ids = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n + 1));
    double* w = (double*)malloc(sizeof(double) * (size_t)(n + 1));
    int32_t* counts = (int32_t*)malloc(sizeof(int32_t) * (size_t)E);
    int32_t* eoff = (int32_t*)malloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t* perm = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n + 1));
    int32_t* inv = (int32_t*)malloc(sizeof(int32_t) * (size_t)(n + 1));
    double* Y = (double*)malloc(sizeof(double) * (size_t)(n * H + 1));
    double* S = (Is > 0) ? (double*)malloc(sizeof(double) * (size_t)(T * H + 1)) : NULL;
    if (!X || !L || !ids || !w || !counts || !eoff || !perm || !inv || !Y || (Is > 0 && !S)) {
        rc = ORC_ERR_ARG;
        goto done;
    }
    /* a1: fan-in -- concatenate the peers along the token dimension */
    rc = oracle_concat_rows(P, seq_lens, (const void* const*)x, H * (int64_t)sizeof(uint16_t), X);
    if (rc) goto done;
    rc = oracle_concat_rows(P, seq_lens, (const void* const*)l, E * (int64_t)sizeof(float), L);
    if (rc) goto done;
    /* a2: route */
    rc = oracle_route(T, E, K, renorm, L, ids, w);
    if (rc) goto done;
    /* a3: dispatch */
    rc = oracle_dispatch(T, E, K, ids, counts, eoff, perm, inv);
    if (rc) goto done;
    /* a4/a5: routed experts over their groups */
    rc = oracle_experts(T, H, E, K, I, X, eoff, perm, W13, W2, Y);
    if (rc) goto done;
    /* a6: shared expert over the shared rows (all tokens with one replica) */
    if (Is > 0) {
        rc = oracle_shared(T, H, Is, X, Ws13, Ws2, S);
        if (rc) goto done;
    }
    /* a7: weighted combine (+ shared); the split is off[] */
    rc = oracle_combine(T, H, K, rsf, w, inv, Y, S, out);
    if (rc) goto done;
    if (ids_out) memcpy(ids_out, ids, sizeof(int32_t) * (size_t)n);
    if (w_out) memcpy(w_out, w, sizeof(double) * (size_t)n);
    if (counts_out) memcpy(counts_out, counts, sizeof(int32_t) * (size_t)E);
    if (eoff_out) memcpy(eoff_out, eoff, sizeof(int32_t) * (size_t)(E + 1));
    if (perm_out) memcpy(perm_out, perm, sizeof(int32_t) * (size_t)n);
    if (inv_out) memcpy(inv_out, inv, sizeof(int32_t) * (size_t)n);
    if (off_out) memcpy(off_out, off, sizeof(int32_t) * (size_t)(P + 1));
done:
    free(off); free(X); free(L); free(ids); free(w); free(counts); free(eoff);
    free(perm); free(inv); free(Y); free(S);
    return rc;
}

/* ---------------------------------------------------------------------------
 * Output rows for a chosen list of tokens, one token at a time, for sizes
 * where the whole path is too slow on the CPU.  For token t (an index into
 * the fan-in) it routes t alone (step a2 on one row), applies each selected
 * expert to x_t, and combines in k order with the shared row:
 *   out = rsf * sum_k w_k * SwiGLU_{ids_k}(x_t) + SwiGLU_shared(x_t)
 * which is the same value the grouped path gives for that token (the expert
 * output of pair t*K+k sits at inv[t*K+k]).
 *   X: [T][H] bf16 fan-in rows; L: [T][E]; tok: n token indices;
 *   out: [n][H]; ids: [n][K]; w: [n][K].
 * ------------------------------------------------------------------------- */
int oracle_token_rows(int64_t T, int64_t H, int E, int K, int64_t I, int64_t Is, double rsf,
                      int renorm, const uint16_t* X, const float* L, const uint16_t* W13,
                      const uint16_t* W2, const uint16_t* Ws13, const uint16_t* Ws2,
                      int64_t n, const int64_t* tok, double* out, int32_t* ids, double* w) {
    if (T < 0 || H < 1 || E < 1 || K < 1 || K > E || I < 1 || n < 0) return ORC_ERR_ARG;
    for (int64_t q = 0; q < n; ++q)
        if (tok[q] < 0 || tok[q] >= T) return ORC_ERR_ARG;
    int bad = 0;
#pragma omp parallel
    {
        int64_t amax = I > Is ? I : Is;
        double* act = (double*)malloc(sizeof(double) * (size_t)amax);
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        if (!act || !y) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t q = 0; q < n; ++q) {
                int64_t t = tok[q];
                int rc = oracle_route(1, E, K, renorm, L + t * E, ids + q * K, w + q * K);
                if (rc) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                double* o = out + q * H;
                for (int64_t c = 0; c < H; ++c) o[c] = 0.0;
                for (int k = 0; k < K; ++k) {
                    int e = ids[q * K + k];
                    swiglu_row(H, I, X + t * H, W13 + (int64_t)e * 2 * I * H,
                               W2 + (int64_t)e * H * I, act, y);
                    for (int64_t c = 0; c < H; ++c) o[c] += w[q * K + k] * y[c];
                }
                for (int64_t c = 0; c < H; ++c) o[c] = rsf * o[c];
                if (Is > 0) {
                    swiglu_row(H, Is, X + t * H, Ws13, Ws2, act, y);
                    for (int64_t c = 0; c < H; ++c) o[c] += y[c];
                }
            }
        }
        free(act);
        free(y);
    }
    return bad ? ORC_ERR_ARG : ORC_OK;
}

/* ---------------------------------------------------------------------------
 * FP8 for the quantised W1 (gate/up) GEMM ([NPU-RFC] "[RFC]: Async AFD for
 * Prefill on Ascend NPU", "Architecture": the routed W1 + SwiGLU grouped
 * GEMM with quantisation).  The pages name no format; the reading taken is
 * OCP FP8 E4M3 ("E4M3FN": 1 sign, 4 exponent bits with bias 7, 3 mantissa
 * bits, subnormals, largest finite 448, no infinities), round to nearest even
 * with saturation to +-448, one scale per row: a token's hidden row (dynamic)
 * and a W13 row (one output channel).
 *
 * e4m3 code of an fp32 value, from the format's definition.  Zero results
 * carry no sign.
 * ------------------------------------------------------------------------- */
uint8_t oracle_e4m3_encode(float v) {
    union { float f; uint32_t u; } b;
    b.f = v;
    const uint32_t sign = b.u >> 31, a = b.u & 0x7FFFFFFFu;
    uint32_t code;
    if (a >= 0x43E00000u) {               /* |v| >= 448 (and inf): saturate */
        code = 0x7E;
    } else if (a < 0x00800000u) {         /* fp32 zero or subnormal: below 2^-126 */
        code = 0;
    } else {
        const int e = (int)(a >> 23) - 127;   /* |v| = 1.m * 2^e */
        const uint32_t M = (a & 0x7FFFFFu) | 0x800000u;  /* 24-bit significand */
        if (e >= -6) {                    /* normal e4m3: keep 3 fraction bits */
            uint32_t q = M >> 20;         /* 1.xxx as 8..15 */
            const uint32_t rem = M & 0xFFFFFu, half = 0x80000u;
            if (rem > half || (rem == half && (q & 1u))) ++q;
            int E = e + 7;
            if (q == 16) { q = 8; ++E; }
            code = (E > 15 || (E == 15 && (q & 7u) == 7u)) ? 0x7Eu : ((uint32_t)E << 3) | (q & 7u);
        } else {                          /* subnormal e4m3: multiples of 2^-9 */
            const int s = 14 - e;         /* M * 2^(e-23) / 2^-9 = M >> s */
            if (s >= 32) {
                code = 0;
            } else {
                uint32_t q = M >> s;
                const uint32_t rem = M & ((1u << s) - 1u), half = 1u << (s - 1);
                if (rem > half || (rem == half && (q & 1u))) ++q;
                code = q;                 /* q == 8 is the smallest normal, code 0x08 */
            }
        }
    }
    return (uint8_t)(code == 0 ? 0 : (sign << 7) | code);
}

/* Value of an e4m3 code (0x7F / 0xFF, NaN, are never produced). */
double oracle_e4m3_decode(uint8_t c) {
    const int E = (c >> 3) & 15, q = c & 7;
    const double m = E == 0 ? ldexp((double)q, -9) : ldexp(1.0 + q / 8.0, E - 7);
    return (c & 0x80) ? -m : m;
}

/* Quantise n rows of H bf16 values, one scale per row: amax = max |x|;
 * r = 448 / amax (fp32, correctly rounded); code = e4m3(x * r) with the
 * product in fp32; the row's dequantisation scale is d = amax / 448 (fp32)
 * and x is taken as decode(code) * d (deq, in double).  A zero row has d = 1
 * and zero codes.  codes: [n][H]; d: [n]; deq: [n][H] (either may be NULL). */
int oracle_quant_rows(int64_t n, int64_t H, const uint16_t* x, uint8_t* codes, float* d, double* deq) {
    if (n < 0 || H < 1 || !x) return ORC_ERR_ARG;
    /* rows are independent: threads take whole rows */
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; ++i) {
        const uint16_t* row = x + i * H;
        float amax = 0.0f;
        for (int64_t h = 0; h < H; ++h) {
            const float v = fabsf((float)bf16_to_double(row[h]));
            if (v > amax) amax = v;
        }
        const float r = amax > 0.0f ? 448.0f / amax : 0.0f;
        const float di = amax > 0.0f ? amax / 448.0f : 1.0f;
        if (d) d[i] = di;
        for (int64_t h = 0; h < H; ++h) {
            const float v = (float)bf16_to_double(row[h]) * r;
            const uint8_t c = oracle_e4m3_encode(v);
            if (codes) codes[i * H + h] = c;
            if (deq) deq[i * H + h] = oracle_e4m3_decode(c) * (double)di;
        }
    }
    return ORC_OK;
}

/* One SwiGLU row on operands given in double (the dequantised fp8 token row
 * and gate/up rows); W2 stays bf16.  The same formula as swiglu_row. */
static void swiglu_row_d(int64_t H, int64_t I, const double* x, const double* w13, const uint16_t* w2,
                         double* act, double* y) {
    for (int64_t j = 0; j < I; ++j) {
        const double* wg = w13 + j * H;
        const double* wu = w13 + (I + j) * H;
        double g = 0.0, u = 0.0;
        for (int64_t h = 0; h < H; ++h) {
            g += x[h] * wg[h];
            u += x[h] * wu[h];
        }
        act[j] = (g / (1.0 + exp(-g))) * u;
    }
    for (int64_t c = 0; c < H; ++c) {
        const uint16_t* wr = w2 + c * I;
        double s = 0.0;
        for (int64_t j = 0; j < I; ++j) s += act[j] * bf16_to_double(wr[j]);
        y[c] = s;
    }
}

/* oracle_token_rows with the gate/up operands in double: Xd [T][H] and the
 * dequantised W13d [E][2I][H], Ws13d [2Is][H] (the fp8 W1 path); routing
 * and combine as there. */
int oracle_token_rows_d(int64_t T, int64_t H, int E, int K, int64_t I, int64_t Is, double rsf, int renorm,
                        const double* Xd, const float* L, const double* W13d, const uint16_t* W2,
                        const double* Ws13d, const uint16_t* Ws2, int64_t n, const int64_t* tok, double* out,
                        int32_t* ids, double* w) {
    if (T < 0 || H < 1 || E < 1 || K < 1 || K > E || I < 1 || n < 0) return ORC_ERR_ARG;
    for (int64_t q = 0; q < n; ++q)
        if (tok[q] < 0 || tok[q] >= T) return ORC_ERR_ARG;
    int bad = 0;
#pragma omp parallel
    {
        int64_t amax = I > Is ? I : Is;
        double* act = (double*)malloc(sizeof(double) * (size_t)amax);
        double* y = (double*)malloc(sizeof(double) * (size_t)H);
        if (!act || !y) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t q = 0; q < n; ++q) {
                int64_t t = tok[q];
                int rc = oracle_route(1, E, K, renorm, L + t * E, ids + q * K, w + q * K);
                if (rc) {
#pragma omp atomic write
                    bad = 1;
                    continue;
                }
                double* o = out + q * H;
                for (int64_t c = 0; c < H; ++c) o[c] = 0.0;
                for (int k = 0; k < K; ++k) {
                    int e = ids[q * K + k];
                    swiglu_row_d(H, I, Xd + t * H, W13d + (int64_t)e * 2 * I * H, W2 + (int64_t)e * H * I, act, y);
                    for (int64_t c = 0; c < H; ++c) o[c] += w[q * K + k] * y[c];
                }
                for (int64_t c = 0; c < H; ++c) o[c] = rsf * o[c];
                if (Is > 0) {
                    swiglu_row_d(H, Is, Xd + t * H, Ws13d, Ws2, act, y);
                    for (int64_t c = 0; c < H; ++c) o[c] += y[c];
                }
            }
        }
        free(act);
        free(y);
    }
    return bad ? ORC_ERR_ARG : ORC_OK;
}

/* ---------------------------------------------------------------------------
 * The fp8 W1 path grouped by expert, as oracle_experts / oracle_shared are
 * for bf16: expert e runs over its dispatch group [expert_offsets[e],
 * expert_offsets[e+1]) with the double gate/up operands (the dequantised
 * fp8 rows) and bf16 W2.  Each row is the swiglu_row_d of oracle_token_rows_d
 * on the same operands, so for the same routing the combined rows equal that
 * routine's rows; it exists because walking the experts one group at a time
 * keeps an expert's weights hot while its rows run, which the full-size
 * workloads need.
 *   Xd: [T][H]; W13d: [E][2I][H]; W2: [E][H][I] bf16; Y: [T*K][H].
 * ------------------------------------------------------------------------- */
int oracle_experts_d(int64_t T, int64_t H, int E, int K, int64_t I, const double* Xd,
                     const int32_t* expert_offsets, const int32_t* perm,
                     const double* W13d, const uint16_t* W2, double* Y) {
    if (T < 0 || H < 1 || E < 1 || K < 1 || I < 1 || !Xd || !expert_offsets || !perm || !W13d || !W2 || !Y)
        return ORC_ERR_ARG;
    int bad = 0;
    for (int e = 0; e < E; ++e) {
        const double* w13 = W13d + (int64_t)e * 2 * I * H;
        const uint16_t* w2 = W2 + (int64_t)e * H * I;
        int64_t lo = expert_offsets[e], hi = expert_offsets[e + 1];
#pragma omp parallel
        {
            double* act = (double*)malloc(sizeof(double) * (size_t)I);
            if (!act) {
#pragma omp atomic write
                bad = 1;
            } else {
#pragma omp for schedule(dynamic, 1)
                for (int64_t i = lo; i < hi; ++i) {
                    int64_t t = perm[i] / K;
                    swiglu_row_d(H, I, Xd + t * H, w13, w2, act, Y + i * H);
                }
                free(act);
            }
        }
    }
    return bad ? ORC_ERR_ARG : ORC_OK;
}

/* The shared expert on the double gate/up operands (Ws13d [2Is][H], bf16
 * Ws2 [H][Is]) over every row of Xd [T][H]; S: [T][H]. */
int oracle_shared_d(int64_t T, int64_t H, int64_t Is, const double* Xd, const double* Ws13d,
                    const uint16_t* Ws2, double* S) {
    if (T < 0 || H < 1 || Is < 1 || !Xd || !Ws13d || !Ws2 || !S) return ORC_ERR_ARG;
    int bad = 0;
#pragma omp parallel
    {
        double* act = (double*)malloc(sizeof(double) * (size_t)Is);
        if (!act) {
#pragma omp atomic write
            bad = 1;
        } else {
#pragma omp for schedule(dynamic, 1)
            for (int64_t t = 0; t < T; ++t) swiglu_row_d(H, Is, Xd + t * H, Ws13d, Ws2, act, S + t * H);
            free(act);
        }
    }
    return bad ? ORC_ERR_ARG : ORC_OK;
}
