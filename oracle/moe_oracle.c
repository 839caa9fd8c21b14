/*
 * moe_oracle.c -- plain fp64 CPU oracle of the Flint routed-expert MoE layer.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may load, call or
 * link this file: only the test suite, the smoke check and the benchmark's
 * CPU-baseline leg use it.  It shares no code, header, table or helper with
 * the HIP library; it is written from the pages and from the number-format
 * specifications, and is kept slow and literal on purpose.
 *
 * What the layer computes (sources):
 *  - An MoE feed-forward layer: a gating network scores the experts and each
 *    token runs only the few it selects  [kongchang.com, "Recursive
 *    Open-Sources Flint: A 40B MoE Local Coding Model with 2.5B Active
 *    Parameters", section "Architecture: The 40B Total vs. 2.5B Active
 *    Trade-off"].
 *  - 256 routed experts per MoE layer, 6 selected per token, plus one shared
 *    expert that every token always uses  [evermx.com, "Recursive Flint:
 *    Open-Weight MoE Coding Model, 2.5B Active", Feature Overview, paragraph
 *    "Sparse architecture"; swarmz.net, "Recursive Flint: 40B Open Model,
 *    2.5B Active", section "The architecture, in plain terms"; futurpulse.com,
 *    "Flint model: local coding with fewer active parameters", section "How
 *    does Flint use 39.8B parameters efficiently?"].
 *  - 4-bit weights are NVFP4  [evermx.com page above, paragraph
 *    "Quantization"]: E2M1 values with one E4M3 scale per 16 elements and an
 *    fp32 per-tensor scale (OCP Microscaling Formats v1.0 for E2M1, OCP 8-bit
 *    Floating Point Specification for E4M3).
 *
 * Where the pages are silent this oracle takes the stated readings:
 * SwiGLU experts without biases, h = SiLU(G x) * (U x), y = D h; a softmax
 * router whose weights are renormalised over the chosen k; selection on the
 * logits in descending order with ties to the lowest expert index; the
 * shared expert enters with weight exactly 1.
 *
 * Every accumulation is a left-to-right fp64 sum in index order.  Stored
 * inputs (fp32, bf16 bits, NVFP4 codes and scales) are converted exactly to
 * fp64 before use.  Nothing is rounded on the way to the output.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORACLE_F32 0
#define ORACLE_BF16 1
#define ORACLE_NVFP4 2

/* ---------------------------------------------------------------------- */
/* Exact decoders of the stored number formats.                             */
/* ---------------------------------------------------------------------- */

/* binary32 -> fp64 (exact). */
static double f32_value(const float* p) { return (double)*p; }

/* bfloat16 is the upper half of a binary32: 1 sign, 8 exponent, 7 fraction
 * bits.  Decoded field by field. */
double oracle_bf16_value(uint16_t bits) {
    int s = (bits >> 15) & 1;
    int e = (bits >> 7) & 0xFF;
    int m = bits & 0x7F;
    double v;
    if (e == 0xFF) {
        v = (m == 0) ? INFINITY : NAN;
    } else if (e == 0) {
        v = ldexp((double)m, -126 - 7); /* subnormal: 0.m * 2^-126 */
    } else {
        v = ldexp(1.0 + m / 128.0, e - 127);
    }
    return s ? -v : v;
}

/* FP4 E2M1 (OCP MX): 1 sign, 2 exponent bits (bias 1), 1 mantissa bit,
 * no infinities or NaN.  Exponent field 0 is subnormal: 0.m * 2^0. */
double oracle_e2m1_value(uint8_t code) {
    int s = (code >> 3) & 1;
    int e = (code >> 1) & 3;
    int m = code & 1;
    double v = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -v : v;
}

/* FP8 E4M3 (OCP "E4M3FN"): 1 sign, 4 exponent bits (bias 7), 3 mantissa
 * bits; exponent field 0 is subnormal (0.m * 2^-6); S.1111.111 is NaN; no
 * infinities. */
double oracle_e4m3_value(uint8_t code) {
    int s = (code >> 7) & 1;
    int e = (code >> 3) & 0xF;
    int m = code & 7;
    double v;
    if (e == 15 && m == 7) {
        v = NAN;
    } else if (e == 0) {
        v = ldexp((double)m / 8.0, -6);
    } else {
        v = ldexp(1.0 + m / 8.0, e - 7);
    }
    return s ? -v : v;
}

/* Round an fp64 value to the nearest bfloat16 (ties to even); returns the
 * bf16 bit pattern.  Used only where a configuration defines a bf16 tensor
 * as the rounding of an exact quantity (the stacked layers' normalised
 * input).  Finite normal range only; overflow saturates to infinity. */
uint16_t oracle_round_to_bf16(double v) {
    if (isnan(v)) return 0x7FC0;
    if (v == 0.0) return signbit(v) ? 0x8000 : 0x0000;
    double a = fabs(v);
    int ex;
    frexp(a, &ex);          /* a = g * 2^(ex-1), g in [1, 2) */
    int e = ex - 1;
    if (e < -126) e = -126; /* below the normal range the grid stays 2^-133 */
    /* bf16 keeps 8 significant bits: the grid step in this binade is 2^(e-7) */
    double r = nearbyint(ldexp(a, 7 - e)); /* default mode rounds ties to even */
    float back = (float)ldexp(r, e - 7);   /* exact (or +inf past the top) */
    uint32_t u;
    memcpy(&u, &back, 4);
    return (uint16_t)((u >> 16) | (v < 0 ? 0x8000u : 0u));
}

/* ---------------------------------------------------------------------- */
/* A read-only view of one stored weight matrix [rows][cols].               */
/* ---------------------------------------------------------------------- */
typedef struct {
    int dtype;
    const void* data;      /* fp32 / bf16 bits [rows][cols]; NVFP4 codes [rows][cols/2] */
    const uint8_t* scales; /* NVFP4 only: E4M3 codes [rows][cols/16] */
    double tensor_scale;   /* NVFP4 only */
    long cols;
} omat;

/* Element (r, c) of the matrix, exactly, in fp64.  NVFP4 keeps element c of
 * a row in byte c/2, even c in the low nibble; its block scale is scale
 * code c/16 of the row. */
static double omat_at(const omat* m, long r, long c) {
    switch (m->dtype) {
    case ORACLE_F32:
        return f32_value((const float*)m->data + r * m->cols + c);
    case ORACLE_BF16:
        return oracle_bf16_value(((const uint16_t*)m->data)[r * m->cols + c]);
    default: {
        uint8_t byte = ((const uint8_t*)m->data)[r * (m->cols / 2) + c / 2];
        uint8_t code = (c % 2 == 0) ? (byte & 0xF) : (byte >> 4);
        uint8_t sc = m->scales[r * (m->cols / 16) + c / 16];
        return oracle_e2m1_value(code) * oracle_e4m3_value(sc) * m->tensor_scale;
    }
    }
}

static double silu(double z) { return z / (1.0 + exp(-z)); }

/* One SwiGLU expert on one token: h_j = SiLU(G_j . x) * (U_j . x) for
 * j < f, then y_n = D_n . h for n < d. */
static void swiglu_expert(const omat* G, const omat* U, const omat* D, long d, long f,
                          const double* x, double* h, double* y) {
    for (long j = 0; j < f; ++j) {
        double g = 0.0, u = 0.0;
        for (long i = 0; i < d; ++i) g += omat_at(G, j, i) * x[i];
        for (long i = 0; i < d; ++i) u += omat_at(U, j, i) * x[i];
        h[j] = silu(g) * u;
    }
    for (long n = 0; n < d; ++n) {
        double acc = 0.0;
        for (long j = 0; j < f; ++j) acc += omat_at(D, n, j) * h[j];
        y[n] = acc;
    }
}

/* Views of expert e in a weight set laid out as gate_up [n][2f][d] (gate rows
 * first, then up rows) and down [n][d][f]; NVFP4 tensor scales [n][3] are
 * {gate, up, down}. */
static void expert_views(int wdtype, long d, long f, long e, const void* gate_up,
                         const void* down, const uint8_t* gu_scales,
                         const uint8_t* dn_scales, const float* tscales, omat* G,
                         omat* U, omat* D) {
    long gu_elems = 2 * f * d, dn_elems = d * f;
    G->dtype = U->dtype = D->dtype = wdtype;
    G->cols = U->cols = d;
    D->cols = f;
    G->scales = U->scales = D->scales = NULL;
    G->tensor_scale = U->tensor_scale = D->tensor_scale = 1.0;
    if (wdtype == ORACLE_F32) {
        const float* gu = (const float*)gate_up + e * gu_elems;
        G->data = gu;
        U->data = gu + f * d;
        D->data = (const float*)down + e * dn_elems;
    } else if (wdtype == ORACLE_BF16) {
        const uint16_t* gu = (const uint16_t*)gate_up + e * gu_elems;
        G->data = gu;
        U->data = gu + f * d;
        D->data = (const uint16_t*)down + e * dn_elems;
    } else {
        const uint8_t* gu = (const uint8_t*)gate_up + e * gu_elems / 2;
        G->data = gu;
        U->data = gu + f * d / 2;
        D->data = (const uint8_t*)down + e * dn_elems / 2;
        const uint8_t* gs = gu_scales + e * gu_elems / 16;
        G->scales = gs;
        U->scales = gs + f * d / 16;
        D->scales = dn_scales + e * dn_elems / 16;
        G->tensor_scale = (double)tscales[3 * e + 0];
        U->tensor_scale = (double)tscales[3 * e + 1];
        D->tensor_scale = (double)tscales[3 * e + 2];
    }
}

/* Router for one token: logits l_e = x . Wr_e + b_e; the k experts in order
 * of descending logit, ties to the lower index; weights are the softmax over
 * all E experts renormalised over the chosen k. */
static void route_token(long d, int E, int k, const double* x, const float* Wr,
                        const float* bias, int32_t* sel, double* w, double* logits,
                        unsigned char* taken, double* p) {
    for (int e = 0; e < E; ++e) {
        double acc = 0.0;
        for (long i = 0; i < d; ++i) acc += x[i] * (double)Wr[(long)e * d + i];
        logits[e] = acc + (bias ? (double)bias[e] : 0.0);
    }
    memset(taken, 0, (size_t)E);
    for (int j = 0; j < k; ++j) {
        int best = -1;
        for (int e = 0; e < E; ++e) {
            if (taken[e]) continue;
            /* strictly greater: on equal logits the earlier (lower) index stays */
            if (best < 0 || logits[e] > logits[best]) best = e;
        }
        sel[j] = best;
        taken[best] = 1;
    }
    double mx = logits[0];
    for (int e = 1; e < E; ++e)
        if (logits[e] > mx) mx = logits[e];
    double z = 0.0;
    for (int e = 0; e < E; ++e) {
        p[e] = exp(logits[e] - mx);
        z += p[e];
    }
    for (int e = 0; e < E; ++e) p[e] /= z;
    double s = 0.0;
    for (int j = 0; j < k; ++j) s += p[sel[j]];
    for (int j = 0; j < k; ++j) w[j] = p[sel[j]] / s;
}

static void load_row(int act_dtype, const void* x, long t, long d, double* out) {
    for (long i = 0; i < d; ++i) {
        if (act_dtype == ORACLE_F32)
            out[i] = (double)((const float*)x)[t * d + i];
        else
            out[i] = oracle_bf16_value(((const uint16_t*)x)[t * d + i]);
    }
}

/*
 * The whole layer on T tokens.
 *   x            [T][d], act_dtype (0 = fp32, 1 = bf16 bits)
 *   router_w     [E][d] fp32;  router_bias [E] fp32 or NULL
 *   gate_up/down routed weights of weight dtype wdtype (0, 1, 2 = NVFP4), see
 *                expert_views; the shared expert uses the same layout with
 *                one expert of width fs
 *   out          [T][d] fp64;  sel [T][k] int32;  w [T][k] fp64;
 *   logits       [T][E] fp64 (may be NULL)
 * Returns 0, or -1 on a malformed argument.
 */
int oracle_moe_forward(int T, int d, int E, int k, int f, int fs, int act_dtype,
                       int wdtype, const void* x, const float* router_w,
                       const float* router_bias, const void* gate_up, const void* down,
                       const uint8_t* gu_scales, const uint8_t* dn_scales,
                       const float* tscales, const void* s_gate_up, const void* s_down,
                       const uint8_t* s_gu_scales, const uint8_t* s_dn_scales,
                       const float* s_tscales, double* out, int32_t* sel, double* w,
                       double* logits) {
    if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E || f <= 0 || fs < 0) return -1;
    if (wdtype == ORACLE_NVFP4 && (d % 16 || f % 16 || (fs && fs % 16))) return -1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 1) reduction(| : fail)
    for (int t = 0; t < T; ++t) {
        long fm = f > fs ? f : fs;
        double* xr = malloc(sizeof(double) * d);
        double* lg = malloc(sizeof(double) * E);
        double* p = malloc(sizeof(double) * E);
        unsigned char* taken = malloc((size_t)E);
        double* h = malloc(sizeof(double) * (fm > 0 ? fm : 1));
        double* y = malloc(sizeof(double) * d);
        double* acc = malloc(sizeof(double) * d);
        if (!xr || !lg || !p || !taken || !h || !y || !acc) {
            fail = 1;
        } else {
            load_row(act_dtype, x, t, d, xr);
            route_token(d, E, k, xr, router_w, router_bias, sel + (long)t * k,
                        w + (long)t * k, lg, taken, p);
            if (logits) memcpy(logits + (long)t * E, lg, sizeof(double) * E);
            /* shared expert, weight 1 */
            for (long n = 0; n < d; ++n) acc[n] = 0.0;
            if (fs > 0) {
                omat G, U, D;
                expert_views(wdtype, d, fs, 0, s_gate_up, s_down, s_gu_scales,
                             s_dn_scales, s_tscales, &G, &U, &D);
                swiglu_expert(&G, &U, &D, d, fs, xr, h, y);
                for (long n = 0; n < d; ++n) acc[n] += y[n];
            }
            /* routed experts in selection order */
            for (int j = 0; j < k; ++j) {
                omat G, U, D;
                long e = sel[(long)t * k + j];
                expert_views(wdtype, d, f, e, gate_up, down, gu_scales, dn_scales,
                             tscales, &G, &U, &D);
                swiglu_expert(&G, &U, &D, d, f, xr, h, y);
                double wj = w[(long)t * k + j];
                for (long n = 0; n < d; ++n) acc[n] += wj * y[n];
            }
            memcpy(out + (long)t * d, acc, sizeof(double) * d);
        }
        free(xr); free(lg); free(p); free(taken); free(h); free(y); free(acc);
    }
    return fail ? -1 : 0;
}

/*
 * The router alone on T tokens: logits, the chosen k experts and their
 * weights, exactly as oracle_moe_forward computes them (route_token), without
 * the experts.  Arguments as in oracle_moe_forward.  Returns 0, or -1.
 */
int oracle_route(int T, int d, int E, int k, int act_dtype, const void* x,
                 const float* router_w, const float* router_bias, int32_t* sel,
                 double* w, double* logits) {
    if (T < 0 || d <= 0 || E <= 0 || k <= 0 || k > E) return -1;
    int fail = 0;
#pragma omp parallel for schedule(dynamic, 16) reduction(| : fail)
    for (int t = 0; t < T; ++t) {
        double* xr = malloc(sizeof(double) * d);
        double* lg = malloc(sizeof(double) * E);
        double* p = malloc(sizeof(double) * E);
        unsigned char* taken = malloc((size_t)E);
        if (!xr || !lg || !p || !taken) {
            fail = 1;
        } else {
            load_row(act_dtype, x, t, d, xr);
            route_token(d, E, k, xr, router_w, router_bias, sel + (long)t * k,
                        w + (long)t * k, lg, taken, p);
            if (logits) memcpy(logits + (long)t * E, lg, sizeof(double) * E);
        }
        free(xr); free(lg); free(p); free(taken);
    }
    return fail ? -1 : 0;
}

/* One expert applied to one fp64 vector (weights as above, expert e). */
int oracle_expert_forward(int d, int f, int wdtype, long e, const void* gate_up,
                          const void* down, const uint8_t* gu_scales,
                          const uint8_t* dn_scales, const float* tscales,
                          const double* x, double* y) {
    if (d <= 0 || f <= 0) return -1;
    double* h = malloc(sizeof(double) * f);
    if (!h) return -1;
    omat G, U, D;
    expert_views(wdtype, d, f, e, gate_up, down, gu_scales, dn_scales, tscales, &G, &U, &D);
    swiglu_expert(&G, &U, &D, d, f, x, h, y);
    free(h);
    return 0;
}

/* RMSNorm with unit gain: y = v / sqrt(mean(v^2) + eps), per row. */
void oracle_rmsnorm(int T, int d, const double* in, double eps, double* out) {
    for (long t = 0; t < T; ++t) {
        double ss = 0.0;
        for (long i = 0; i < d; ++i) ss += in[t * d + i] * in[t * d + i];
        double r = 1.0 / sqrt(ss / d + eps);
        for (long i = 0; i < d; ++i) out[t * d + i] = in[t * d + i] * r;
    }
}

double oracle_silu(double z) { return silu(z); }
