/*
 * CPU oracle for the gated delta rule recurrence with dynamic state fake-quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is a plain, slow, float64 statement of what the
 * GPU library computes.  Only the test suite, the smoke check and the bench's CPU
 * baseline may load it; the library never calls it and shares no code with it.
 *
 * Sources (the linear-attention state-QAT pages):
 *  - "Torch GDN/KDA decode QAT + INT8" (PR #2519), "What does this PR do?": GDN and KDA
 *    recurrent suffix, FP32 working values, straight-through state QDQ, INT8 groups of
 *    16/32/64 along the last (value) axis independent of tile width, INT8 + Hadamard.
 *  - "GDN state/W QAT foundation" (PR #2497, docs mirror page), "What does this PR do?":
 *    dynamic per-tile FP8 E4M3 state QDQ at 64-token boundaries over a full-key by
 *    64-value-column tile per sequence and head, scale = amax / 448 with a zero guard,
 *    identity straight-through gradients.
 *  - "Fused Triton GDN/KDA decode QAT" (PR #2562), "What does this PR do?": checkpointed
 *    backward, differentiable continuation carry (gradient of the initial state).
 *  The update equation itself is the gated delta rule:
 *      S~ = diag(a) S_{t-1},  a = exp(g_t)   (scalar for GDN, per key channel for KDA)
 *      u  = S~^T k_t,  delta = beta_t (v_t - u),  S' = S~ + k_t delta^T,  o_t = S'^T q_t
 *      S_t = Q(S') at quantization points, else S'.
 *  State layout: S[i][j], i = key index (d_k rows), j = value index (d_v columns, contiguous).
 *
 * Readings where the pages leave a step open (each is listed in the design notes):
 *  - The output o_t reads the state before it is rounded; only the carried state is
 *    rounded.
 *  - Quantization points: every token (interval 1) or after tokens n, 2n, ... and after the
 *    last token of the call (interval n).  The initial state is never rounded on entry.
 *  - The carried state is FP32 (the pages' working precision), so at a quantization point
 *    the float64 state is rounded to float32 and the codec decides in float32:
 *    s = fl32(amax / 127), y = fl32(x / s), code = clamp(rint(y), -127, 127),
 *    xhat = fl32(code * s).  amax == 0 gives s = 1 (zero guard, no epsilon floor).
 *  - E4M3 is OCP E4M3FN (bias 7, max 448, subnormal step 2^-9), round to nearest with ties
 *    to the even code, saturating at +-448; s = fl32(amax / 448).
 *  - Hadamard: Y = Hn S' with Hn the Sylvester Hadamard matrix of order d_k divided by
 *    sqrt(d_k); the INT8 codec acts on fl32(Y); the carried state is Hn Yhat.
 *  - Backward: identity straight-through gradient through Q (and through the rotations,
 *    since Hn Hn = I); the upstream gradient is dO and optionally dS_T.
 *  - Replay windows ("Torch GDN/KDA decode QAT + INT8", What does this PR do?: a window of
 *    one token checkpoints every token; longer windows keep BF16 key and update entries and
 *    refresh at the window boundary; "Fused Triton GDN/KDA decode QAT", What does this PR
 *    do?: replay with encode-once factors): the rounding points are those of qdq_interval =
 *    W (window ends, and the call's last token); at every other token the carried state takes
 *    the token's rank-1 update from its factors encoded once to BF16,
 *    S_t = S~ + bf16(k) bf16(delta)^T, each factor rounded from its FP32 value to nearest
 *    even; the output reads the token's own unencoded update (o_t = S'^T q_t, as always), and
 *    a window end rounds S' itself (the refresh absorbs its token without an entry).  The
 *    backward passes straight through the encoding as it does through Q.
 *
 * All functions are reentrant; none allocates beyond plain malloc scratch freed on return.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "oracle.h"

#ifdef _OPENMP
#include <omp.h>
#endif

/* Threads the parallel loops over units use (1 without OpenMP). */
int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of threads for later calls (no effect without OpenMP). */
void oracle_set_num_threads(int n) {
#ifdef _OPENMP
    if (n >= 1) omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------------------ */
/* FP8 E4M3FN value table                                                                */
/* ------------------------------------------------------------------------------------ */

/* Value of a non-negative E4M3FN code c in 0..126 (0x7F is NaN and never produced):
 * exponent field e = c >> 3, mantissa m = c & 7; e == 0 -> m * 2^-9, else (1 + m/8) 2^(e-7). */
double oracle_e4m3_value(int code) {
    int c = code & 0x7F;
    int e = c >> 3, m = c & 7;
    double mag = (e == 0) ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    return (code & 0x80) ? -mag : mag;
}

/* Nearest E4M3FN code to y: ties go to the even code, magnitudes beyond 448 saturate to 448.
 * Non-negative codes 0..126 are increasing in value, so a bisection finds the bracket. */
int oracle_e4m3_code(double y) {
    int neg = (y < 0) || (y == 0 && signbit(y));
    double a = fabs(y);
    if (a >= 448.0) return (neg ? 0x80 : 0) | 0x7E;
    int lo = 0, hi = 126; /* value(lo) <= a < value(hi) after the loop */
    while (hi - lo > 1) {
        int mid = (lo + hi) / 2;
        if (oracle_e4m3_value(mid) <= a) lo = mid; else hi = mid;
    }
    double dlo = a - oracle_e4m3_value(lo), dhi = oracle_e4m3_value(hi) - a;
    int c;
    if (dlo < dhi) c = lo;
    else if (dhi < dlo) c = hi;
    else c = (lo % 2 == 0) ? lo : hi;
    return (neg ? 0x80 : 0) | c;
}

/* Nearest BF16 value to fl32(x), ties to the even significand (x finite). */
double oracle_bf16(double x) {
    float f = (float)x;
    uint32_t b;
    memcpy(&b, &f, sizeof b);
    uint32_t lsb = (b >> 16) & 1u;
    b = (b + 0x7FFFu + lsb) & 0xFFFF0000u;
    memcpy(&f, &b, sizeof f);
    return (double)f;
}

/* ------------------------------------------------------------------------------------ */
/* Codecs on one d_k x d_v state matrix                                                  */
/* ------------------------------------------------------------------------------------ */

/* INT8 symmetric dynamic group QDQ along the value axis (groups of `group` columns).
 * X: input values (rounded to float32 here); Xhat: output; codes/scales/ypre optional:
 * codes [dk][dv] int32, scales [dk][dv/group] float, ypre [dk][dv] float (x/s before rint). */
static void int8_group_qdq(int dk, int dv, int group, const double* X, double* Xhat,
                           int32_t* codes, float* scales, float* ypre) {
    for (int i = 0; i < dk; i++) {
        for (int c0 = 0; c0 < dv; c0 += group) {
            float amax = 0.0f;
            for (int j = c0; j < c0 + group; j++) {
                float x = (float)X[i * dv + j];
                if (fabsf(x) > amax) amax = fabsf(x);
            }
            float s = (amax > 0.0f) ? amax / 127.0f : 1.0f;
            if (scales) scales[i * (dv / group) + c0 / group] = s;
            for (int j = c0; j < c0 + group; j++) {
                float x = (float)X[i * dv + j];
                float y = x / s;
                float r = rintf(y);
                if (r > 127.0f) r = 127.0f;
                if (r < -127.0f) r = -127.0f;
                float xh = r * s;
                Xhat[i * dv + j] = (double)xh;
                if (codes) codes[i * dv + j] = (int32_t)r;
                if (ypre) ypre[i * dv + j] = y;
            }
        }
    }
}

/* FP8 E4M3 dynamic per-tile QDQ: tile = all d_k rows x `tile` value columns. */
static void e4m3_tile_qdq(int dk, int dv, int tile, const double* X, double* Xhat,
                          int32_t* codes, float* scales, float* ypre) {
    for (int c0 = 0; c0 < dv; c0 += tile) {
        float amax = 0.0f;
        for (int i = 0; i < dk; i++)
            for (int j = c0; j < c0 + tile; j++) {
                float x = (float)X[i * dv + j];
                if (fabsf(x) > amax) amax = fabsf(x);
            }
        float s = (amax > 0.0f) ? amax / 448.0f : 1.0f;
        if (scales) scales[c0 / tile] = s;
        for (int i = 0; i < dk; i++)
            for (int j = c0; j < c0 + tile; j++) {
                float x = (float)X[i * dv + j];
                float y = x / s;
                int code = oracle_e4m3_code((double)y);
                float val = (float)oracle_e4m3_value(code);
                float xh = val * s;
                Xhat[i * dv + j] = (double)xh;
                if (codes) codes[i * dv + j] = code;
                if (ypre) ypre[i * dv + j] = y;
            }
    }
}

/* Normalized Sylvester Hadamard entry: (-1)^popcount(i & j) / sqrt(n). */
static double hadamard_entry(int n, int i, int j) {
    int p = __builtin_popcount((unsigned)(i & j));
    return ((p & 1) ? -1.0 : 1.0) / sqrt((double)n);
}

/* Y = Hn X on the key axis (plain matrix product). */
static void hadamard_rows(int dk, int dv, const double* X, double* Y) {
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int r = 0; r < dk; r++) acc += hadamard_entry(dk, i, r) * X[r * dv + j];
            Y[i * dv + j] = acc;
        }
}

void oracle_hadamard(int dk, int dv, const double* X, double* Y) { hadamard_rows(dk, dv, X, Y); }

int oracle_qdq(int qdq, int group, int hadamard, int dk, int dv, const double* X, double* Xhat,
               int32_t* codes, float* scales, float* ypre) {
    if (qdq == ORACLE_QDQ_NONE) {
        memcpy(Xhat, X, sizeof(double) * (size_t)dk * dv);
        return 0;
    }
    if (group <= 0 || dv % group != 0) return -1;
    if (qdq == ORACLE_QDQ_INT8) {
        if (!hadamard) {
            int8_group_qdq(dk, dv, group, X, Xhat, codes, scales, ypre);
            return 0;
        }
        if (dk & (dk - 1)) return -1;
        size_t n = (size_t)dk * dv;
        double* xs = (double*)malloc(sizeof(double) * n);
        double* y = (double*)malloc(sizeof(double) * n);
        double* yh = (double*)malloc(sizeof(double) * n);
        for (size_t e = 0; e < n; e++) xs[e] = (double)(float)X[e]; /* carried state is fp32 */
        hadamard_rows(dk, dv, xs, y);
        int8_group_qdq(dk, dv, group, y, yh, codes, scales, ypre);
        hadamard_rows(dk, dv, yh, Xhat);
        free(xs); free(y); free(yh);
        return 0;
    }
    if (qdq == ORACLE_QDQ_E4M3) {
        if (hadamard) return -1;
        e4m3_tile_qdq(dk, dv, group, X, Xhat, codes, scales, ypre);
        return 0;
    }
    return -1;
}

/* ------------------------------------------------------------------------------------ */
/* Forward recurrence                                                                    */
/* ------------------------------------------------------------------------------------ */

static int is_qdq_point(const oracle_cfg* c, int t /* 0-based token just processed */) {
    if (c->qdq == ORACLE_QDQ_NONE) return 0;
    int n = c->qdq_interval;
    return ((t + 1) % n == 0) || (t == c->T - 1);
}

static int check_cfg(const oracle_cfg* c) {
    if (c->B < 0 || c->T < 0 || c->H < 0 || c->dk <= 0 || c->dv <= 0) return -1;
    if (c->qdq != ORACLE_QDQ_NONE) {
        if (c->group <= 0 || c->dv % c->group) return -1;
        if (c->qdq_interval <= 0) return -1;
        if (c->hadamard && (c->qdq != ORACLE_QDQ_INT8 || (c->dk & (c->dk - 1)))) return -1;
    }
    if (c->ckpt_interval < 0) return -1;
    if (c->replay != 0 && c->replay != 1) return -1;
    if (c->replay && c->qdq == ORACLE_QDQ_NONE) return -1; /* replay windows end in a checkpoint codec */
    return 0;
}

/* One token of the recurrence on one (sequence, head) unit.
 * S (in): S_{t-1}; St, Sp: scratch d_k x d_v; u, delta: d_v; a: d_k gate factors.
 * Writes S' into Sp and o_t into o. */
static void token_step(int dk, int dv, const double* S, const double* a, const double* k,
                       const double* q, const double* v, double beta, double* St, double* Sp,
                       double* u, double* delta, double* o) {
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++) St[i * dv + j] = a[i] * S[i * dv + j];
    for (int j = 0; j < dv; j++) {
        double acc = 0.0;
        for (int i = 0; i < dk; i++) acc += St[i * dv + j] * k[i];
        u[j] = acc;
    }
    for (int j = 0; j < dv; j++) delta[j] = beta * (v[j] - u[j]);
    for (int i = 0; i < dk; i++)
        for (int j = 0; j < dv; j++) Sp[i * dv + j] = St[i * dv + j] + k[i] * delta[j];
    for (int j = 0; j < dv; j++) {
        double acc = 0.0;
        for (int i = 0; i < dk; i++) acc += Sp[i * dv + j] * q[i];
        o[j] = acc;
    }
}

static void gate_factors(const oracle_cfg* c, const double* g, int b, int t, int h, double* a) {
    if (c->gate == ORACLE_GATE_KEY) {
        const double* gp = g + (((size_t)b * c->T + t) * c->H + h) * c->dk;
        for (int i = 0; i < c->dk; i++) a[i] = exp(gp[i]);
    } else {
        double av = exp(g[((size_t)b * c->T + t) * c->H + h]);
        for (int i = 0; i < c->dk; i++) a[i] = av;
    }
}

/* The carried state after token t (0-based) from S~, S' = S~ + k delta^T and the token's
 * factors: Q(S') at a rounding point; in replay mode S~ + bf16(k) dhat^T elsewhere, with dhat
 * the given entry (dhat_t, when not NULL and not NaN) or bf16(delta); else S'. */
static void carry(const oracle_cfg* c, int t, const double* St, const double* Sp, const double* kt,
                  const double* delta, const double* dhat_t, double* S) {
    const int dk = c->dk, dv = c->dv;
    if (is_qdq_point(c, t)) {
        oracle_qdq(c->qdq, c->group, c->hadamard, dk, dv, Sp, S, NULL, NULL, NULL);
    } else if (c->replay) {
        for (int i = 0; i < dk; i++) {
            double kh = oracle_bf16(kt[i]);
            for (int j = 0; j < dv; j++) {
                double dh = (dhat_t && !isnan(dhat_t[j])) ? dhat_t[j] : oracle_bf16(delta[j]);
                S[i * dv + j] = St[i * dv + j] + kh * dh;
            }
        }
    } else {
        memcpy(S, Sp, sizeof(double) * (size_t)dk * dv);
    }
}

/* Forward pass of one (sequence, head) unit. */
static void unit_fwd(const oracle_cfg* c, int b, int h, const double* q, const double* k,
                     const double* v, const double* g, const double* beta, const double* S0,
                     double* o, double* ST, double* ckpts, const double* dhat_in, double* delta_out) {
    const int T = c->T, H = c->H, dk = c->dk, dv = c->dv;
    const size_t n = (size_t)dk * dv;
    const int nck = (c->ckpt_interval > 0) ? (T + c->ckpt_interval - 1) / c->ckpt_interval : 0;
    double* S = (double*)malloc(sizeof(double) * n);
    double* St = (double*)malloc(sizeof(double) * n);
    double* Sp = (double*)malloc(sizeof(double) * n);
    double* u = (double*)malloc(sizeof(double) * dv);
    double* delta = (double*)malloc(sizeof(double) * dv);
    double* a = (double*)malloc(sizeof(double) * dk);
    if (S0) memcpy(S, S0 + ((size_t)b * H + h) * n, sizeof(double) * n);
    else memset(S, 0, sizeof(double) * n);
    for (int t = 0; t < T; t++) {
        if (ckpts && c->ckpt_interval > 0 && t % c->ckpt_interval == 0)
            memcpy(ckpts + (((size_t)b * H + h) * nck + t / c->ckpt_interval) * n, S,
                   sizeof(double) * n);
        size_t tok = ((size_t)b * T + t) * H + h;
        gate_factors(c, g, b, t, h, a);
        token_step(dk, dv, S, a, k + tok * dk, q + tok * dk, v + tok * dv, beta[tok], St, Sp, u,
                   delta, o + tok * dv);
        if (delta_out) memcpy(delta_out + tok * dv, delta, sizeof(double) * dv);
        carry(c, t, St, Sp, k + tok * dk, delta, dhat_in ? dhat_in + tok * dv : NULL, S);
    }
    if (ST) memcpy(ST + ((size_t)b * H + h) * n, S, sizeof(double) * n);
    free(S); free(St); free(Sp); free(u); free(delta); free(a);
}

/* Units are independent, so they are spread over OpenMP threads (when built with it). */
int oracle_fwd_ex(const oracle_cfg* c, const double* q, const double* k, const double* v,
                  const double* g, const double* beta, const double* S0, double* o, double* ST,
                  double* ckpts, const double* dhat_in, double* delta_out) {
    if (check_cfg(c)) return -1;
    const int units = c->B * c->H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int unit = 0; unit < units; unit++)
        unit_fwd(c, unit / c->H, unit % c->H, q, k, v, g, beta, S0, o, ST, ckpts, dhat_in, delta_out);
    return 0;
}

int oracle_fwd(const oracle_cfg* c, const double* q, const double* k, const double* v,
               const double* g, const double* beta, const double* S0, double* o, double* ST,
               double* ckpts) {
    return oracle_fwd_ex(c, q, k, v, g, beta, S0, o, ST, ckpts, NULL, NULL);
}

/* ------------------------------------------------------------------------------------ */
/* Straight-through backward                                                             */
/* ------------------------------------------------------------------------------------ */

static void unit_bwd(const oracle_cfg* c, int b, int h, const double* q, const double* k,
                     const double* v, const double* g, const double* beta, const double* S0,
                     const double* states, const double* dout, const double* dST, double* dq,
                     double* dk_out, double* dv_out, double* dg, double* dbeta, double* dS0) {
    const int T = c->T, H = c->H, dk = c->dk, dv = c->dv;
    const size_t n = (size_t)dk * dv;
    double* traj = NULL; /* S_{t-1} for t = 0..T-1 when recomputed here */
    double* S = (double*)malloc(sizeof(double) * n);
    double* St = (double*)malloc(sizeof(double) * n);
    double* Sp = (double*)malloc(sizeof(double) * n);
    double* lam = (double*)malloc(sizeof(double) * n);
    double* dSt = (double*)malloc(sizeof(double) * n);
    double* u = (double*)malloc(sizeof(double) * dv);
    double* delta = (double*)malloc(sizeof(double) * dv);
    double* ddelta = (double*)malloc(sizeof(double) * dv);
    double* du = (double*)malloc(sizeof(double) * dv);
    double* otmp = (double*)malloc(sizeof(double) * dv);
    double* a = (double*)malloc(sizeof(double) * dk);
    const double* Sprev_base;
    if (states) {
        Sprev_base = states + ((size_t)b * H + h) * (size_t)T * n;
    } else {
        traj = (double*)malloc(sizeof(double) * n * (size_t)(T > 0 ? T : 1));
        if (S0) memcpy(S, S0 + ((size_t)b * H + h) * n, sizeof(double) * n);
        else memset(S, 0, sizeof(double) * n);
        for (int t = 0; t < T; t++) {
            memcpy(traj + (size_t)t * n, S, sizeof(double) * n);
            size_t tok = ((size_t)b * T + t) * H + h;
            gate_factors(c, g, b, t, h, a);
            token_step(dk, dv, S, a, k + tok * dk, q + tok * dk, v + tok * dv, beta[tok], St, Sp,
                       u, delta, otmp);
            carry(c, t, St, Sp, k + tok * dk, delta, NULL, S);
        }
        Sprev_base = traj;
    }
    if (dST) memcpy(lam, dST + ((size_t)b * H + h) * n, sizeof(double) * n);
    else memset(lam, 0, sizeof(double) * n);
    for (int t = T - 1; t >= 0; t--) {
        const double* Sprev = Sprev_base + (size_t)t * n;
        size_t tok = ((size_t)b * T + t) * H + h;
        const double* kt = k + tok * dk;
        const double* qt = q + tok * dk;
        const double* vt = v + tok * dv;
        const double* dot = dout + tok * dv;
        double bt = beta[tok];
        gate_factors(c, g, b, t, h, a);
        /* recompute S~, u, delta, S' from S_{t-1} */
        token_step(dk, dv, Sprev, a, kt, qt, vt, bt, St, Sp, u, delta, otmp);
        /* dS' = lambda (straight through Q) + q do^T */
        for (int i = 0; i < dk; i++)
            for (int j = 0; j < dv; j++) lam[i * dv + j] += qt[i] * dot[j];
        /* o = S'^T q: dq = S' do */
        for (int i = 0; i < dk; i++) {
            double acc = 0.0;
            for (int j = 0; j < dv; j++) acc += Sp[i * dv + j] * dot[j];
            dq[tok * dk + i] = acc;
        }
        /* S' = S~ + k delta^T: ddelta = dS'^T k, dk = dS' delta, dS~ = dS' */
        for (int j = 0; j < dv; j++) {
            double acc = 0.0;
            for (int i = 0; i < dk; i++) acc += lam[i * dv + j] * kt[i];
            ddelta[j] = acc;
        }
        /* delta = beta (v - u): dbeta, dv, du */
        double dbt = 0.0;
        for (int j = 0; j < dv; j++) {
            dbt += ddelta[j] * (vt[j] - u[j]);
            dv_out[tok * dv + j] = bt * ddelta[j];
            du[j] = -bt * ddelta[j];
        }
        dbeta[tok] = dbt;
        /* u = S~^T k: dS~ += k du^T, dk += S~ du */
        for (int i = 0; i < dk; i++) {
            double acc = 0.0;
            for (int j = 0; j < dv; j++) acc += lam[i * dv + j] * delta[j] + St[i * dv + j] * du[j];
            dk_out[tok * dk + i] = acc;
        }
        for (int i = 0; i < dk; i++)
            for (int j = 0; j < dv; j++) dSt[i * dv + j] = lam[i * dv + j] + kt[i] * du[j];
        /* S~ = diag(a) S_{t-1}, a = exp(g): da_i = sum_j S_{t-1,ij} dS~_ij, dg = a da */
        if (c->gate == ORACLE_GATE_KEY) {
            for (int i = 0; i < dk; i++) {
                double acc = 0.0;
                for (int j = 0; j < dv; j++) acc += Sprev[i * dv + j] * dSt[i * dv + j];
                dg[tok * dk + i] = a[i] * acc;
            }
        } else {
            double acc = 0.0;
            for (size_t e = 0; e < n; e++) acc += Sprev[e] * dSt[e];
            dg[tok] = a[0] * acc;
        }
        /* dS_{t-1} = diag(a) dS~ */
        for (int i = 0; i < dk; i++)
            for (int j = 0; j < dv; j++) lam[i * dv + j] = a[i] * dSt[i * dv + j];
    }
    memcpy(dS0 + ((size_t)b * H + h) * n, lam, sizeof(double) * n);
    free(traj); free(S); free(St); free(Sp); free(lam); free(dSt); free(u); free(delta);
    free(ddelta); free(du); free(otmp); free(a);
}

/* Reverse-mode derivative of oracle_fwd with Q replaced by the identity in the backward
 * pass.  The forward trajectory is either recomputed here (states == NULL) or taken from
 * `states` [B][H][T][dk][dv]: the carried state entering each token (as produced by a
 * forward pass with checkpoints after every token).  dST may be NULL (zero). */
int oracle_bwd(const oracle_cfg* c, const double* q, const double* k, const double* v,
               const double* g, const double* beta, const double* S0, const double* states,
               const double* dout, const double* dST, double* dq, double* dk_out, double* dv_out,
               double* dg, double* dbeta, double* dS0) {
    if (check_cfg(c)) return -1;
    const int units = c->B * c->H;
#pragma omp parallel for schedule(dynamic, 1)
    for (int unit = 0; unit < units; unit++)
        unit_bwd(c, unit / c->H, unit % c->H, q, k, v, g, beta, S0, states, dout, dST, dq, dk_out,
                 dv_out, dg, dbeta, dS0);
    return 0;
}
