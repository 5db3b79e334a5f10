/*
 * Host harness of the C oracle (oracle/k3oracle.c), built together with it
 * under AddressSanitizer and UndefinedBehaviorSanitizer. It calls every
 * entry point on small seeded inputs that reach each branch (NaN and
 * infinite logits, E8M0 bytes 0 and 0xFF, every E2M1 code, dropped pairs,
 * T = 0, invalid sizes), with each buffer allocated to its exact size so an
 * access one element past it is reported. It also checks a few invariants
 * that need no reference: gates of finite logits sum to 1, grouping is a
 * permutation of the kept pairs.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

double k3o_e2m1(int code);
double k3o_e8m0(int b);
int k3o_dequant(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t K, double *W);
void k3o_bf16_to_f64(const uint16_t *bits, int64_t n, double *out);
int k3o_router_logits(const uint16_t *x, const float *wr, const float *bias, int64_t T, int64_t d,
                      int64_t E, float *logits);
int k3o_topk_gates(const float *logits, int64_t T, int64_t E, int64_t k, int32_t *idx,
                   double *gate);
double k3o_silu(double z);
void k3o_silu_array(const double *z, int64_t n, double *out);
int k3o_expert_ffn(const double *x, int64_t n, int64_t d, int64_t f, const uint8_t *gq,
                   const uint8_t *gs, const uint8_t *uq, const uint8_t *us, const uint8_t *dq,
                   const uint8_t *ds, double *hbuf, double *o, double *h);
int k3o_combine(const double *outs, const double *gate, const int32_t *idx, int64_t T, int64_t k,
                int64_t d, int64_t E, double *y);
int64_t k3o_group_pairs(const int32_t *idx, int64_t P, int64_t E, int32_t *counts,
                        int32_t *offsets, int32_t *perm);

static int g_fail = 0;
#define CHECK(c, msg)                                              \
    do {                                                           \
        if (!(c)) {                                                \
            fprintf(stderr, "FAIL %s:%d: %s\n", __FILE__, __LINE__, msg); \
            ++g_fail;                                              \
        }                                                          \
    } while (0)

static uint64_t g_rng = 0x9e3779b97f4a7c15ull;
static uint32_t rnd(void)
{
    g_rng ^= g_rng << 13;
    g_rng ^= g_rng >> 7;
    g_rng ^= g_rng << 17;
    return (uint32_t)(g_rng >> 32);
}
static double unif(void) { return (rnd() + 0.5) / 4294967296.0; }

static void *xalloc(size_t n)
{
    void *p = malloc(n ? n : 1);
    if (!p) {
        fprintf(stderr, "out of memory\n");
        exit(2);
    }
    return p;
}

static uint16_t bf16_of(float f)
{
    union { float f; uint32_t u; } v;
    v.f = f;
    return (uint16_t)(v.u >> 16);
}

static void formats(void)
{
    for (int c = -3; c < 20; ++c)
        (void)k3o_e2m1(c);
    for (int b = -2; b < 260; ++b)
        (void)k3o_e8m0(b);
    CHECK(isnan(k3o_e8m0(255)), "E8M0 0xFF is NaN");
    /* every code with scale bytes 0, 1, 127, 254, 255 */
    const int64_t rows = 3, K = 64;
    uint8_t *q = xalloc((size_t)(rows * K / 2));
    uint8_t *s = xalloc((size_t)(rows * K / 32));
    double *W = xalloc(sizeof(double) * (size_t)(rows * K));
    for (int64_t i = 0; i < rows * K / 2; ++i)
        q[i] = (uint8_t)(i * 17);
    const uint8_t sb[6] = {0, 1, 127, 254, 255, 131};
    for (int64_t i = 0; i < rows * K / 32; ++i)
        s[i] = sb[i % 6];
    CHECK(k3o_dequant(q, s, rows, K, W) == 0, "dequant");
    CHECK(k3o_dequant(q, s, rows, 40, W) < 0, "dequant rejects K % 32");
    CHECK(k3o_dequant(q, s, -1, K, W) < 0, "dequant rejects rows < 0");
    CHECK(k3o_dequant(q, s, 0, K, W) == 0, "dequant of no rows");
    uint16_t bits[5] = {0x0000, 0x8000, 0x7f80, 0x7fc1, 0x3f80};
    double out[5];
    k3o_bf16_to_f64(bits, 5, out);
    CHECK(out[4] == 1.0 && isinf(out[2]) && isnan(out[3]), "bf16 decode");
    free(q);
    free(s);
    free(W);
}

static void router(void)
{
    const int64_t T = 5, d = 96, E = 11;
    uint16_t *x = xalloc(sizeof(uint16_t) * (size_t)(T * d));
    float *wr = xalloc(sizeof(float) * (size_t)(E * d));
    float *bias = xalloc(sizeof(float) * (size_t)E);
    float *lg = xalloc(sizeof(float) * (size_t)(T * E));
    for (int64_t i = 0; i < T * d; ++i)
        x[i] = bf16_of((float)(unif() * 2.0 - 1.0));
    for (int64_t i = 0; i < E * d; ++i)
        wr[i] = (float)(0.02 * (unif() - 0.5));
    for (int64_t e = 0; e < E; ++e)
        bias[e] = (float)(unif() - 0.5);
    bias[2] = NAN;
    bias[7] = -INFINITY;
    CHECK(k3o_router_logits(x, wr, bias, T, d, E, lg) == 0, "router logits");
    CHECK(k3o_router_logits(x, wr, NULL, T, d, E, lg) == 0, "router logits, no bias");
    CHECK(k3o_router_logits(x, wr, NULL, 0, d, E, lg) == 0, "router logits, T = 0");
    CHECK(k3o_router_logits(x, wr, NULL, -1, d, E, lg) < 0, "router rejects T < 0");
    CHECK(k3o_router_logits(x, wr, bias, T, d, E, lg) == 0, "router logits again");
    for (int64_t k = 1; k <= E; ++k) {
        int32_t *idx = xalloc(sizeof(int32_t) * (size_t)(T * k));
        double *gate = xalloc(sizeof(double) * (size_t)(T * k));
        CHECK(k3o_topk_gates(lg, T, E, k, idx, gate) == 0, "topk");
        for (int64_t t = 0; t < T; ++t) {
            double sum = 0.0;
            for (int64_t j = 0; j < k; ++j) {
                CHECK(idx[t * k + j] >= 0 && idx[t * k + j] < E, "topk index in range");
                sum += gate[t * k + j];
            }
            CHECK(fabs(sum - 1.0) < 1e-12, "gates sum to 1");
        }
        free(idx);
        free(gate);
    }
    int32_t idx1[4];
    double g1[4];
    CHECK(k3o_topk_gates(lg, T, E, 0, idx1, g1) < 0, "topk rejects k = 0");
    CHECK(k3o_topk_gates(lg, T, E, E + 1, idx1, g1) < 0, "topk rejects k > E");
    float allnan[3] = {NAN, NAN, -INFINITY};
    CHECK(k3o_topk_gates(allnan, 1, 3, 2, idx1, g1) == 0 && isnan(g1[0]), "no finite logit");
    free(x);
    free(wr);
    free(bias);
    free(lg);
}

static void expert_and_combine(void)
{
    const int64_t d = 64, f = 96, n = 3, k = 4, E = 6;
    uint8_t *gq = xalloc((size_t)(f * d / 2)), *gs = xalloc((size_t)(f * d / 32));
    uint8_t *uq = xalloc((size_t)(f * d / 2)), *us = xalloc((size_t)(f * d / 32));
    uint8_t *dq = xalloc((size_t)(d * f / 2)), *ds = xalloc((size_t)(d * f / 32));
    for (int64_t i = 0; i < f * d / 2; ++i) {
        gq[i] = (uint8_t)rnd();
        uq[i] = (uint8_t)rnd();
        dq[i] = (uint8_t)rnd();
    }
    for (int64_t i = 0; i < f * d / 32; ++i) {
        gs[i] = (uint8_t)(120 + rnd() % 9);
        us[i] = (uint8_t)(120 + rnd() % 9);
        ds[i] = (uint8_t)(120 + rnd() % 9);
    }
    ds[5] = 0xFF; /* one NaN block */
    gs[3] = 0;    /* the smallest scale */
    double *x = xalloc(sizeof(double) * (size_t)(n * d));
    for (int64_t i = 0; i < n * d; ++i)
        x[i] = unif() * 4.0 - 2.0;
    double *hbuf = xalloc(sizeof(double) * (size_t)f);
    double *o = xalloc(sizeof(double) * (size_t)(n * d));
    double *h = xalloc(sizeof(double) * (size_t)(n * f));
    CHECK(k3o_expert_ffn(x, n, d, f, gq, gs, uq, us, dq, ds, hbuf, o, h) == 0, "expert ffn");
    CHECK(k3o_expert_ffn(x, n, d, f, gq, gs, uq, us, dq, ds, hbuf, o, NULL) == 0, "ffn, no h");
    CHECK(k3o_expert_ffn(x, 0, d, f, gq, gs, uq, us, dq, ds, hbuf, o, NULL) == 0, "ffn, n = 0");
    CHECK(k3o_expert_ffn(x, n, 48, f, gq, gs, uq, us, dq, ds, hbuf, o, NULL) < 0, "ffn rejects d");
    double z[5] = {-1000.0, -40.0, 0.0, 40.0, 1000.0}, zo[5];
    k3o_silu_array(z, 5, zo);
    CHECK(!isnan(zo[0]) && !isnan(zo[4]), "SiLU at +-1000");
    (void)k3o_silu(NAN);
    /* combine over T tokens, with dropped pairs */
    const int64_t T = 3;
    double *outs = xalloc(sizeof(double) * (size_t)(T * k * d));
    double *gate = xalloc(sizeof(double) * (size_t)(T * k));
    int32_t *idx = xalloc(sizeof(int32_t) * (size_t)(T * k));
    double *y = xalloc(sizeof(double) * (size_t)(T * d));
    for (int64_t i = 0; i < T * k * d; ++i)
        outs[i] = unif();
    for (int64_t i = 0; i < T * k; ++i) {
        gate[i] = unif();
        idx[i] = (int32_t)(rnd() % (uint32_t)E);
    }
    idx[1] = -1;
    idx[6] = (int32_t)E;
    CHECK(k3o_combine(outs, gate, idx, T, k, d, E, y) == 0, "combine");
    CHECK(k3o_combine(outs, gate, idx, 0, k, d, E, y) == 0, "combine, T = 0");
    CHECK(k3o_combine(outs, gate, idx, T, 0, d, E, y) < 0, "combine rejects k = 0");
    /* grouping: a permutation of the kept pairs, ordered by expert */
    const int64_t P = T * k;
    int32_t *counts = xalloc(sizeof(int32_t) * (size_t)E);
    int32_t *offsets = xalloc(sizeof(int32_t) * (size_t)(E + 1));
    int32_t *perm = xalloc(sizeof(int32_t) * (size_t)P);
    const int64_t kept = k3o_group_pairs(idx, P, E, counts, offsets, perm);
    CHECK(kept == P - 2, "grouping leaves out the two dropped pairs");
    for (int64_t i = 1; i < kept; ++i)
        CHECK(idx[perm[i - 1]] < idx[perm[i]] ||
                  (idx[perm[i - 1]] == idx[perm[i]] && perm[i - 1] < perm[i]),
              "grouping order");
    CHECK(k3o_group_pairs(idx, 0, E, counts, offsets, perm) == 0, "grouping, no pairs");
    CHECK(k3o_group_pairs(idx, P, 0, counts, offsets, perm) < 0, "grouping rejects E = 0");
    free(gq); free(gs); free(uq); free(us); free(dq); free(ds);
    free(x); free(hbuf); free(o); free(h);
    free(outs); free(gate); free(idx); free(y);
    free(counts); free(offsets); free(perm);
}

int main(void)
{
    formats();
    router();
    expert_and_combine();
    if (g_fail) {
        fprintf(stderr, "%d checks failed\n", g_fail);
        return 1;
    }
    printf("oracle harness: all checks passed\n");
    return 0;
}
