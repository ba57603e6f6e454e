/* Host sanitizer run of the CPU oracle (test infrastructure): every entry
 * point of afd_oracle.c on small inputs, including the degenerate ones (an
 * empty peer, K = E, K = 1, all-equal logits, -0.0, a zero row, non-finite
 * logits and bad arguments, which must be refused without touching memory).
 * Built with -fsanitize=address,undefined by tests/test_sanitize_cpu.py;
 * exit 0 and no sanitizer report is a pass. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int oracle_fanin(int P, const int32_t* seq_lens, int32_t token_cap, int32_t* off);
int oracle_route(int64_t T, int E, int K, int renorm, const float* logits, int32_t* ids, double* w);
int oracle_dispatch(int64_t T, int E, int K, const int32_t* ids, int32_t* counts, int32_t* eoff, int32_t* perm,
                    int32_t* inv);
int oracle_ffn(int P, const int32_t* seq_lens, const uint16_t* const* x, const float* const* l, int64_t H, int E,
               int K, int64_t I, int64_t Is, double rsf, int renorm, const uint16_t* W13, const uint16_t* W2,
               const uint16_t* Ws13, const uint16_t* Ws2, int32_t* ids_out, double* w_out, int32_t* counts_out,
               int32_t* eoff_out, int32_t* perm_out, int32_t* inv_out, int32_t* off_out, double* out);
int oracle_token_rows(int64_t T, int64_t H, int E, int K, int64_t I, int64_t Is, double rsf, int renorm,
                      const uint16_t* X, const float* L, const uint16_t* W13, const uint16_t* W2, const uint16_t* Ws13,
                      const uint16_t* Ws2, int64_t n, const int64_t* tok, double* out, int32_t* ids, double* w);
uint8_t oracle_e4m3_encode(float v);
double oracle_e4m3_decode(uint8_t c);
int oracle_quant_rows(int64_t n, int64_t H, const uint16_t* x, uint8_t* codes, float* d, double* deq);
int oracle_experts_d(int64_t T, int64_t H, int E, int K, int64_t I, const double* Xd, const int32_t* eoff,
                     const int32_t* perm, const double* W13d, const uint16_t* W2, double* Y);
int oracle_shared_d(int64_t T, int64_t H, int64_t Is, const double* Xd, const double* Ws13d, const uint16_t* Ws2,
                    double* S);

static uint32_t rng = 12345u;
static float frand(void) {
    rng = rng * 1664525u + 1013904223u;
    return ((float)(rng >> 8) / 16777216.0f) * 2.0f - 1.0f;
}
static uint16_t bf(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}
static void* xalloc(size_t n) {
    void* p = calloc(n ? n : 1, 1);
    if (!p) exit(3);
    return p;
}

static int run_case(int P, const int32_t* seq, int64_t H, int E, int K, int64_t I, int64_t Is, int renorm) {
    int64_t T = 0;
    for (int p = 0; p < P; ++p) T += seq[p];
    uint16_t** x = xalloc(sizeof(uint16_t*) * P);
    float** l = xalloc(sizeof(float*) * P);
    for (int p = 0; p < P; ++p) {
        x[p] = xalloc(2 * (size_t)seq[p] * H);
        l[p] = xalloc(4 * (size_t)seq[p] * E);
        for (int64_t i = 0; i < seq[p] * H; ++i) x[p][i] = bf(frand());
        for (int64_t i = 0; i < seq[p] * E; ++i) l[p][i] = (i % 7 == 0) ? 0.5f : frand();
    }
    uint16_t* W13 = xalloc(2 * (size_t)E * 2 * I * H);
    uint16_t* W2 = xalloc(2 * (size_t)E * H * I);
    uint16_t* Ws13 = Is ? xalloc(2 * (size_t)2 * Is * H) : NULL;
    uint16_t* Ws2 = Is ? xalloc(2 * (size_t)H * Is) : NULL;
    for (int64_t i = 0; i < (int64_t)E * 2 * I * H; ++i) W13[i] = bf(0.02f * frand());
    for (int64_t i = 0; i < (int64_t)E * H * I; ++i) W2[i] = bf(0.02f * frand());
    for (int64_t i = 0; Is && i < 2 * Is * H; ++i) Ws13[i] = bf(0.02f * frand());
    for (int64_t i = 0; Is && i < H * Is; ++i) Ws2[i] = bf(0.02f * frand());
    int32_t* ids = xalloc(4 * (size_t)(T * K + 1));
    double* w = xalloc(8 * (size_t)(T * K + 1));
    int32_t* counts = xalloc(4 * (size_t)E);
    int32_t* eoff = xalloc(4 * (size_t)(E + 1));
    int32_t* perm = xalloc(4 * (size_t)(T * K + 1));
    int32_t* inv = xalloc(4 * (size_t)(T * K + 1));
    int32_t* off = xalloc(4 * (size_t)(P + 1));
    double* out = xalloc(8 * (size_t)(T * H + 1));
    int rc = oracle_ffn(P, seq, (const uint16_t* const*)x, (const float* const*)l, H, E, K, I, Is, 1.5, renorm, W13,
                        W2, Ws13, Ws2, ids, w, counts, eoff, perm, inv, off, out);
    if (rc) return rc;
    /* per-token path and the fp8 pieces on the same inputs */
    uint16_t* X = xalloc(2 * (size_t)(T * H + 1));
    float* L = xalloc(4 * (size_t)(T * E + 1));
    for (int p = 0, t = 0; p < P; t += seq[p], ++p) {
        memcpy(X + (int64_t)t * H, x[p], 2 * (size_t)seq[p] * H);
        memcpy(L + (int64_t)t * E, l[p], 4 * (size_t)seq[p] * E);
    }
    int64_t* tok = xalloc(8 * (size_t)(T + 1));
    for (int64_t t = 0; t < T; ++t) tok[t] = t;
    double* out2 = xalloc(8 * (size_t)(T * H + 1));
    int32_t* ids2 = xalloc(4 * (size_t)(T * K + 1));
    double* w2 = xalloc(8 * (size_t)(T * K + 1));
    rc = oracle_token_rows(T, H, E, K, I, Is, 1.5, renorm, X, L, W13, W2, Ws13, Ws2, T, tok, out2, ids2, w2);
    if (rc) return rc;
    for (int64_t i = 0; i < T * H; ++i)
        if (out2[i] != out[i]) return 10;
    uint8_t* codes = xalloc((size_t)(T * H + 1));
    float* d = xalloc(4 * (size_t)(T + 1));
    double* Xd = xalloc(8 * (size_t)(T * H + 1));
    if ((rc = oracle_quant_rows(T, H, X, codes, d, Xd))) return rc;
    double* W13d = xalloc(8 * (size_t)E * 2 * I * H);
    if ((rc = oracle_quant_rows((int64_t)E * 2 * I, H, W13, NULL, NULL, W13d))) return rc;
    double* Y = xalloc(8 * (size_t)(T * K * H + 1));
    if ((rc = oracle_experts_d(T, H, E, K, I, Xd, eoff, perm, W13d, W2, Y))) return rc;
    if (Is) {
        double* Ws13d = xalloc(8 * (size_t)2 * Is * H);
        double* S = xalloc(8 * (size_t)(T * H + 1));
        if ((rc = oracle_quant_rows(2 * Is, H, Ws13, NULL, NULL, Ws13d))) return rc;
        if ((rc = oracle_shared_d(T, H, Is, Xd, Ws13d, Ws2, S))) return rc;
        free(Ws13d);
        free(S);
    }
    for (int p = 0; p < P; ++p) {
        free(x[p]);
        free(l[p]);
    }
    free(x); free(l); free(W13); free(W2); free(Ws13); free(Ws2); free(ids); free(w); free(counts); free(eoff);
    free(perm); free(inv); free(off); free(out); free(X); free(L); free(tok); free(out2); free(ids2); free(w2);
    free(codes); free(d); free(Xd); free(W13d); free(Y);
    return 0;
}

int main(void) {
    int fails = 0;
    const int32_t s1[] = {7, 13}, s2[] = {5, 0, 9}, s3[] = {3};
    fails += run_case(2, s1, 64, 8, 2, 32, 32, 1) != 0;
    fails += run_case(3, s2, 40, 5, 5, 24, 0, 0) != 0;   /* empty peer, K = E, no shared expert */
    fails += run_case(1, s3, 24, 6, 1, 8, 16, 1) != 0;   /* K = 1 */
    /* ties and -0.0 */
    float lg[2 * 8] = {0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f, 0.5f, -0.0f, 0.0f, 1.0f, -1.0f, 0.0f, -0.0f, 2.0f, 2.0f};
    int32_t ids[2 * 3];
    double w[2 * 3];
    fails += oracle_route(2, 8, 3, 1, lg, ids, w) != 0;
    /* refusals: non-finite logits, bad sizes, capacity, NULLs */
    lg[3] = NAN;
    fails += oracle_route(2, 8, 3, 1, lg, ids, w) == 0;
    lg[3] = INFINITY;
    fails += oracle_route(2, 8, 3, 1, lg, ids, w) == 0;
    int32_t off[3];
    const int32_t big[] = {5, 9};
    fails += oracle_fanin(2, big, 8, off) == 0;
    fails += oracle_fanin(0, big, 8, off) == 0;
    fails += oracle_fanin(2, NULL, 8, off) == 0;
    fails += oracle_dispatch(-1, 8, 2, NULL, NULL, NULL, NULL, NULL) == 0;
    fails += oracle_quant_rows(-1, 4, NULL, NULL, NULL, NULL) == 0;
    /* every e4m3 code round-trips */
    for (int c = 0; c < 256; ++c) {
        if ((c & 0x7F) == 0x7F) continue;
        const double v = oracle_e4m3_decode((uint8_t)c);
        const uint8_t back = oracle_e4m3_encode((float)v);
        if (back != (uint8_t)c && !(v == 0.0 && back == 0)) ++fails;
    }
    /* a zero row quantises to zero codes with scale 1 */
    uint16_t zr[16] = {0};
    uint8_t zc[16];
    float zd;
    double zq[16];
    fails += oracle_quant_rows(1, 16, zr, zc, &zd, zq) != 0 || zd != 1.0f;
    printf("oracle sanitizer driver: %d failure(s)\n", fails);
    return fails ? 1 : 0;
}
