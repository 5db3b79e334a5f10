/*
 * k3oracle.c -- plain, single-threaded C99 reference of one sparse
 * Mixture-of-Experts layer whose expert weights are stored in MXFP4.
 *
 * TEST INFRASTRUCTURE ONLY. The tests, the package smoke check and the
 * benchmark's CPU-baseline leg may load this library (through oracle/); the
 * product path never does. It shares no code, table or helper with the HIP
 * kernels.
 *
 * What is computed, and where it comes from (pages on the kimi-k3-in-c C99
 * engine):
 *   - the layer is a routed MoE: each layer holds 896 experts and a token
 *     wakes 16 of them (pomoai.com overview, "architecture"; chenxutan.com
 *     article, section 01; qwbw.cn CHANGELOG walk-through, 0.1.0);
 *   - expert weights are MXFP4 nibbles, about half a byte per parameter,
 *     consumed as packed codes with no dequantised expert kept (overview,
 *     "first reduction"; CHANGELOG, 0.1.0);
 *   - the expert FFN is a gated linear unit (printed "SiTU-GLU" in the
 *     CHANGELOG's 0.1.0 section; read as SwiGLU);
 *   - chunk-union prefill equals the per-token path (CHANGELOG, 1.0.0
 *     "Added"), so the per-token definition below is the whole definition;
 *   - a failed expert contributes zero (CHANGELOG, "Unreleased": batched MoE
 *     prefill fix); an expert index outside [0, E) counts as failed.
 * Where the pages are silent, these readings are taken:
 *   - MXFP4 is OCP Microscaling v1.0: an E2M1 code per element, one E8M0
 *     scale per 32 consecutive elements along the reduction dimension;
 *     element 2i sits in the low nibble of byte i; matrices are [out][in]
 *     with the reduction dimension contiguous;
 *   - router logit l[t,e] = sum_i x[t,i] * Wr[e,i], accumulated in fp64 and
 *     rounded to fp32; an optional fp32 bias is then added in fp32, before
 *     both selection and softmax;
 *   - top-k by (logit descending, expert index ascending); +0 and -0 are
 *     equal; a NaN logit counts as -infinity, in the ranking (so it ties
 *     with -inf and the lower index goes first) and in the gates (gate 0);
 *   - gates: softmax over the k selected logits in fp64 (the same as a full
 *     softmax renormalised over the selection);
 *   - expert: g = Wg x, u = Wu x, h = SiLU(g) * u with SiLU(z) = z/(1+e^-z),
 *     o = Wd h; y[t] = sum_j gate[t,j] * o_j, j in selection order.
 * Everything is fp64 except the router logit and the bias add, which the
 * definition fixes in fp32. Sums run in index order with one accumulator.
 *
 * Parity pins: the "not gpu" tests check every entry point here against the
 * OCP MX value tables, closed forms, brute force on tiny inputs, exact sums
 * and an independent dense all-experts computation. Fidelity to the real
 * Kimi K3 checkpoint is parity unpinned (no checkpoint exists).
 *
 * Build: gcc -std=c99 -O2 -ffp-contract=off -fPIC -shared (no fast-math:
 * every operation is an IEEE operation in the order written).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#define K3O_OK 0
#define K3O_EINVAL (-1)

/* ------------------------------------------------------------ formats */

/* E2M1 (OCP MX v1.0 FP4): bit 3 sign, bits 2..1 exponent with bias 1,
 * bit 0 mantissa; exponent 0 is subnormal (0.5 * mantissa). Code 8 is -0. */
double k3o_e2m1(int code)
{
    int c = code & 15;
    int sign = (c >> 3) & 1;
    int e = (c >> 1) & 3;
    int m = c & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return sign ? -mag : mag;
}

/* E8M0 scale byte (OCP MX v1.0): 2^(b - 127); 0xFF is NaN. */
double k3o_e8m0(int b)
{
    if ((b & 255) == 255)
        return NAN;
    return ldexp(1.0, (b & 255) - 127);
}

/* Value tables evaluated once from the two closed forms above. */
static double g_e2m1[16];
static double g_e8m0[256];
static int g_tables_ready = 0;

static void tables_init(void)
{
    if (g_tables_ready)
        return;
    for (int c = 0; c < 16; ++c)
        g_e2m1[c] = k3o_e2m1(c);
    for (int b = 0; b < 256; ++b)
        g_e8m0[b] = k3o_e8m0(b);
    g_tables_ready = 1;
}

/* Element (r, i) of an MXFP4 matrix with K columns: codes q [rows][K/2],
 * scales s [rows][K/32]. */
static double mx_elem(const uint8_t *q, const uint8_t *s, int64_t K, int64_t r, int64_t i)
{
    uint8_t byte = q[r * (K / 2) + i / 2];
    int code = (i & 1) ? (byte >> 4) : (byte & 15);
    return g_e2m1[code] * g_e8m0[s[r * (K / 32) + i / 32]];
}

/* Dequantise a whole matrix into W [rows][K] (used by the pins only). */
int k3o_dequant(const uint8_t *q, const uint8_t *s, int64_t rows, int64_t K, double *W)
{
    if (rows < 0 || K <= 0 || K % 32 != 0)
        return K3O_EINVAL;
    tables_init();
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t i = 0; i < K; ++i)
            W[r * K + i] = mx_elem(q, s, K, r, i);
    return K3O_OK;
}

/* bf16 bit pattern -> fp64 (exact: bf16 is the top half of an fp32). */
static double bf16_value(uint16_t bits)
{
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)bits << 16;
    return (double)v.f;
}

void k3o_bf16_to_f64(const uint16_t *bits, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = bf16_value(bits[i]);
}

/* ------------------------------------------------------------ router */

/* logits [T][E] fp32: fp64 sum of x[t,i] * Wr[e,i] over i (each product is
 * exact in fp64), rounded to fp32; then + bias[e] in fp32 if bias != NULL. */
int k3o_router_logits(const uint16_t *x, const float *wr, const float *bias,
                      int64_t T, int64_t d, int64_t E, float *logits)
{
    if (T < 0 || d <= 0 || E <= 0)
        return K3O_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t e = 0; e < E; ++e) {
            double acc = 0.0;
            for (int64_t i = 0; i < d; ++i)
                acc += bf16_value(x[t * d + i]) * (double)wr[e * d + i];
            float l = (float)acc;
            if (bias != NULL) {
                float b = bias[e];
                l = l + b; /* fp32 add */
            }
            logits[t * E + e] = l;
        }
    }
    return K3O_OK;
}

/* A logit as the selection and the softmax see it: NaN is -infinity. */
static double logit_value(float l)
{
    return isnan(l) ? -INFINITY : (double)l;
}

/* Order of the selection: a before b when l_a > l_b, or l_a == l_b and
 * a < b. A NaN logit compares as -infinity. */
static int ranks_before(float la, int64_t a, float lb, int64_t b)
{
    double va = logit_value(la);
    double vb = logit_value(lb);
    if (va != vb)
        return va > vb;
    return a < b;
}

/* Per token: the k experts that rank first (repeated selection of the best
 * expert not yet taken), and gate_j = exp(l_j - l_first) / sum over the k
 * selected of exp(l - l_first), in fp64. A selected NaN logit counts as
 * -infinity here too, so its gate is 0 (when every selected logit is -inf or
 * NaN, l_j - l_first is NaN and so are all the gates). idx [T][k] int32,
 * gate [T][k]. */
int k3o_topk_gates(const float *logits, int64_t T, int64_t E, int64_t k,
                   int32_t *idx, double *gate)
{
    if (T < 0 || E <= 0 || k < 1 || k > E)
        return K3O_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        const float *row = logits + t * E;
        int32_t *sel = idx + t * k;
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int64_t p = 0; p < j; ++p)
                    if (sel[p] == e)
                        taken = 1;
                if (taken)
                    continue;
                if (best < 0 || ranks_before(row[e], e, row[best], best))
                    best = e;
            }
            sel[j] = (int32_t)best;
        }
        double l0 = logit_value(row[sel[0]]);
        double sum = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            gate[t * k + j] = exp(logit_value(row[sel[j]]) - l0);
            sum += gate[t * k + j];
        }
        for (int64_t j = 0; j < k; ++j)
            gate[t * k + j] /= sum;
    }
    return K3O_OK;
}

/* The selection-only bias reading of a router bias (the pages give the
 * skewed workload's per-expert bias without saying where it enters; the
 * plain reading adds it to the logits for both steps, the alternative uses
 * it only to choose the experts, as aux-loss-free balancing biases do):
 * per token, the k experts ranking first by sel_logits (order and NaN rule
 * as in k3o_topk_gates), and gate_j = exp(r_j - m) / sum over the selected
 * of exp(r - m), where r are the same experts' gate_logits (NaN counts as
 * -inf) and m the largest of them, in fp64. */
int k3o_topk_gates_split(const float *sel_logits, const float *gate_logits, int64_t T, int64_t E,
                         int64_t k, int32_t *idx, double *gate)
{
    if (T < 0 || E <= 0 || k < 1 || k > E)
        return K3O_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        const float *row = sel_logits + t * E;
        const float *raw = gate_logits + t * E;
        int32_t *sel = idx + t * k;
        for (int64_t j = 0; j < k; ++j) {
            int64_t best = -1;
            for (int64_t e = 0; e < E; ++e) {
                int taken = 0;
                for (int64_t p = 0; p < j; ++p)
                    if (sel[p] == e)
                        taken = 1;
                if (taken)
                    continue;
                if (best < 0 || ranks_before(row[e], e, row[best], best))
                    best = e;
            }
            sel[j] = (int32_t)best;
        }
        double m = -INFINITY;
        for (int64_t j = 0; j < k; ++j)
            if (logit_value(raw[sel[j]]) > m)
                m = logit_value(raw[sel[j]]);
        double sum = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            gate[t * k + j] = exp(logit_value(raw[sel[j]]) - m);
            sum += gate[t * k + j];
        }
        for (int64_t j = 0; j < k; ++j)
            gate[t * k + j] /= sum;
    }
    return K3O_OK;
}

/* ------------------------------------------------------------ expert */

/* SiLU(z) = z / (1 + e^-z); for very negative z, e^-z overflows to +inf and
 * the result is -0 (never NaN). */
double k3o_silu(double z)
{
    return z / (1.0 + exp(-z));
}

void k3o_silu_array(const double *z, int64_t n, double *out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = k3o_silu(z[i]);
}

/* One SwiGLU expert on n fp64 token rows x [n][d]:
 *   g[n] = sum_i x[i] Wg[n,i], u[n] = sum_i x[i] Wu[n,i]   (Wg, Wu: [f][d])
 *   h = SiLU(g) * u,   o[m] = sum_n h[n] Wd[m,n]           (Wd: [d][f])
 * o [n][d]; h [n][f] is written too when h != NULL. Each row is computed on
 * its own, element by element from the codes and scales. */
int k3o_expert_ffn(const double *x, int64_t n, int64_t d, int64_t f,
                   const uint8_t *gq, const uint8_t *gs,
                   const uint8_t *uq, const uint8_t *us,
                   const uint8_t *dq, const uint8_t *ds,
                   double *hbuf /* [f] scratch */, double *o, double *h)
{
    if (n < 0 || d <= 0 || f <= 0 || d % 32 != 0 || f % 32 != 0)
        return K3O_EINVAL;
    tables_init();
    for (int64_t t = 0; t < n; ++t) {
        const double *xt = x + t * d;
        for (int64_t r = 0; r < f; ++r) {
            double g = 0.0, u = 0.0;
            for (int64_t i = 0; i < d; ++i) {
                g += xt[i] * mx_elem(gq, gs, d, r, i);
                u += xt[i] * mx_elem(uq, us, d, r, i);
            }
            hbuf[r] = k3o_silu(g) * u;
            if (h != NULL)
                h[t * f + r] = hbuf[r];
        }
        for (int64_t m = 0; m < d; ++m) {
            double acc = 0.0;
            for (int64_t r = 0; r < f; ++r)
                acc += hbuf[r] * mx_elem(dq, ds, f, m, r);
            o[t * d + m] = acc;
        }
    }
    return K3O_OK;
}

/* ------------------------------------------------------------ combine */

/* y[t] = sum over j = 0..k-1, in order, of gate[t,j] * outs[t,j]; a slot
 * whose expert index lies outside [0, E) contributes zero.
 * outs [T][k][d], gate [T][k], idx [T][k], y [T][d]. */
int k3o_combine(const double *outs, const double *gate, const int32_t *idx,
                int64_t T, int64_t k, int64_t d, int64_t E, double *y)
{
    if (T < 0 || k < 1 || d <= 0 || E <= 0)
        return K3O_EINVAL;
    for (int64_t t = 0; t < T; ++t) {
        for (int64_t m = 0; m < d; ++m)
            y[t * d + m] = 0.0;
        for (int64_t j = 0; j < k; ++j) {
            int32_t e = idx[t * k + j];
            if (e < 0 || e >= E)
                continue;
            double g = gate[t * k + j];
            const double *oj = outs + (t * k + j) * d;
            for (int64_t m = 0; m < d; ++m)
                y[t * d + m] += g * oj[m];
        }
    }
    return K3O_OK;
}

/* ------------------------------------------------------------ grouping */

/* The chunk-union grouping: the (token, slot) pairs p = t*k + j bucketed by
 * expert with a stable counting sort. counts [E], offsets [E+1] (exclusive
 * prefix sum), perm [P]: pair ids ordered by (expert, t, j). Pairs whose
 * expert lies outside [0, E) are counted nowhere and left out of perm; the
 * return value is the number of pairs placed (or K3O_EINVAL). */
int64_t k3o_group_pairs(const int32_t *idx, int64_t P, int64_t E,
                        int32_t *counts, int32_t *offsets, int32_t *perm)
{
    if (P < 0 || E <= 0)
        return K3O_EINVAL;
    for (int64_t e = 0; e < E; ++e)
        counts[e] = 0;
    for (int64_t p = 0; p < P; ++p)
        if (idx[p] >= 0 && idx[p] < E)
            counts[idx[p]] += 1;
    offsets[0] = 0;
    for (int64_t e = 0; e < E; ++e)
        offsets[e + 1] = offsets[e] + counts[e];
    for (int64_t e = 0; e < E; ++e)
        counts[e] = 0; /* reused as the per-expert cursor, restored below */
    for (int64_t p = 0; p < P; ++p) {
        int32_t e = idx[p];
        if (e < 0 || e >= E)
            continue;
        perm[offsets[e] + counts[e]] = (int32_t)p;
        counts[e] += 1;
    }
    return offsets[E];
}
