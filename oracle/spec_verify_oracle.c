/*
 * spec_verify_oracle.c -- plain fp64 CPU oracle for batched draft-verify
 * rejection sampling.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may link, load or call
 * this file: only the test suite, the smoke check and the CPU-baseline leg of the
 * benchmark use it.  It shares no code, header, table or constant with the HIP
 * implementation.  It is deliberately slow and literal: every distribution is
 * materialised as a full vector of V doubles, every step follows the sources in
 * their order, and sorting is done with the C library's qsort.
 *
 * Sources (cited by page title and section):
 *   [SD]   zwjcode.cn, "生成 4 个 Token 为何不一定要跑 4 次大模型？Speculative
 *          Decoding 的提议、验证与接受" -- sections 02 (shapes), 03 (greedy),
 *          04 (acceptance ratio and residual), 05 (two-token worked example),
 *          06 (one-round pseudocode, identical transforms), 07 (verify_one),
 *          09 (advance S = A + 1), 13 (correctness checks).
 *   [VLLM] pinghaoyang.com.cn, "vLLM 源码完全拆解（十）：投机解码——草稿模型、
 *          批量验证与 token 接受流水线" -- sections "拒绝采样：RejectionSampler 的
 *          两个分支" (bonus token, temperature/top-k/top-p preprocessing, -1
 *          placeholder output), "Greedy kernel：逐 token 比较" and
 *          "Random kernel：无偏接受 + 重采样" (draft-free residual: the draft
 *          token's cell removed), "关于 synthetic / block 验证模式" (synthetic
 *          acceptance: draft j accepted iff u_j < rate_j, no target
 *          probabilities).
 *
 * Readings taken where the sources are silent or disagree (each is restated in
 * the design notes of the repository):
 *   - accept iff u * q'(y) < p'(y): the strict form of u < min(1, p/q) that three
 *     of four statements use; the product form needs no division and gives
 *     accept iff p'(y) > 0 when q'(y) = 0.
 *   - transforms in the order temperature -> top-k -> top-p -> renormalise,
 *     applied to p (from logits) and to q (given as probabilities, tempered as
 *     q^(1/T)) each with its own thresholds.
 *   - top-k keeps every value tied with the k-th largest; top-p keeps the
 *     smallest set of whole tie groups, taken from the largest value down,
 *     whose mass reaches top_p of the top-k mass.
 *   - the replacement / bonus token is drawn by inverse CDF over ascending token
 *     id with the injected uniform u_sample: z = min{x : C_x > u*S}.
 *   - zero residual mass falls back to drawing from p'.
 *   - greedy ties go to the lowest token id.
 *
 * Build: gcc -O2 -fPIC -shared -o liboracle.so spec_verify_oracle.c -lm
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* fault bits reported per request */
#define OF_DRAFT_ID      1   /* a draft id >= V before the first negative id  */
#define OF_TEMPERATURE   2   /* NaN, negative, infinite or subnormal T        */
#define OF_TOP_P         4   /* NaN or <= 0 top_p on a sampled request        */
#define OF_TARGET_ROW    8   /* NaN / +inf / no finite value in a read row    */
#define OF_DRAFT_ROW     16  /* NaN / inf / sign bit set in a read q row      */
#define OF_DRAFT_MASS    32  /* kept q mass is zero in a read q row           */

/* Tolerance of a comparison with another implementation: a decision whose
 * margin is below it may go either way (an accept ratio within OR_TOL of u, a
 * top-p cut within OR_TOL of top_p, u_sample within OR_TOL of a CDF boundary
 * C_x / S). */
#define OR_TOL 1e-6
#define AMB_ACCEPT 1
#define AMB_TOP_P  2
#define AMB_CDF    4

static double bf16_to_double(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

static double logit_at(const void *row, int dtype, long x) {
    if (dtype == 1) return bf16_to_double(((const uint16_t *)row)[x]);
    return (double)((const float *)row)[x];
}

static int cmp_double_desc(const void *a, const void *b) {
    double x = *(const double *)a, y = *(const double *)b;
    return (x < y) - (x > y);
}

typedef struct {
    double order;
    double mass;
} order_mass;

static int cmp_om_desc(const void *a, const void *b) {
    double x = ((const order_mass *)a)->order, y = ((const order_mass *)b)->order;
    return (x < y) - (x > y);
}

/*
 * Sampling filters [VLLM, "拒绝采样…两个分支", preprocessing step; SD §06 on
 * applying identical transforms to p and q].
 * order[x] ranks the tokens, mass[x] >= 0 is the unnormalised weight (a
 * non-decreasing function of order).  On return keep[x] marks the kept set and
 * the kept mass is returned.  *topp_margin receives the distance of top_p from
 * the two cumulative-mass fractions that bracket the chosen cut (+inf if top-p
 * is off).
 */
static double apply_filters(long V, const double *order, const double *mass, int top_k,
                            double top_p, unsigned char *keep, double *topp_margin) {
    long x;
    for (x = 0; x < V; x++) keep[x] = 1;

    /* top-k: keep every token whose value is >= the k-th largest value */
    if (top_k >= 1 && (long)top_k < V) {
        double *sorted = (double *)malloc(sizeof(double) * V);
        memcpy(sorted, order, sizeof(double) * V);
        qsort(sorted, V, sizeof(double), cmp_double_desc);
        double kth = sorted[top_k - 1];
        free(sorted);
        for (x = 0; x < V; x++) keep[x] = order[x] >= kth;
    }

    double zk = 0.0;
    for (x = 0; x < V; x++)
        if (keep[x]) zk += mass[x];

    *topp_margin = INFINITY;
    if (top_p < 1.0) {
        /* top-p over the top-k survivors: walk whole groups of equal value from
         * the largest down until the cumulative mass reaches top_p * zk */
        long n = 0;
        for (x = 0; x < V; x++) n += keep[x];
        order_mass *kept = (order_mass *)malloc(sizeof(order_mass) * (n ? n : 1));
        long t = 0;
        for (x = 0; x < V; x++)
            if (keep[x]) {
                kept[t].order = order[x];
                kept[t].mass = mass[x];
                t++;
            }
        qsort(kept, n, sizeof(order_mass), cmp_om_desc);
        double target = top_p * zk;
        double cum = 0.0;
        double cut = n ? kept[n - 1].order : -INFINITY; /* keep all if never reached */
        long g = 0;
        while (g < n) {
            double v = kept[g].order;
            double before = cum;
            while (g < n && kept[g].order == v) cum += kept[g++].mass;
            if (cum >= target) {
                cut = v;
                double m1 = top_p - before / zk, m2 = cum / zk - top_p;
                *topp_margin = m1 < m2 ? m1 : m2;
                break;
            }
        }
        free(kept);
        for (x = 0; x < V; x++) keep[x] = keep[x] && order[x] >= cut;
    }

    double z = 0.0;
    for (x = 0; x < V; x++)
        if (keep[x]) z += mass[x];
    return z;
}

/*
 * Target distribution p' of one row: s = l / T, softmax over the kept set of
 * the filters above [VLLM, "拒绝采样…两个分支"; SD §06].  Returns a fault bit
 * or 0.  p_out receives V probabilities.
 */
static int target_probs_row(long V, const void *row, int dtype, double T, int top_k,
                            double top_p, double *p_out, double *topp_margin, long *kept,
                            double *kept_frac) {
    double *s = (double *)malloc(sizeof(double) * V);
    double *e = (double *)malloc(sizeof(double) * V);
    unsigned char *keep = (unsigned char *)malloc(V);
    long x;
    int fault = 0;
    double m = -INFINITY;
    for (x = 0; x < V; x++) {
        double l = logit_at(row, dtype, x);
        if (isnan(l) || l == INFINITY) fault = OF_TARGET_ROW;
        s[x] = l / T;
        if (s[x] > m) m = s[x];
    }
    if (m == -INFINITY) fault = OF_TARGET_ROW; /* no finite logit */
    if (!fault) {
        double total = 0.0;
        for (x = 0; x < V; x++) {
            e[x] = exp(s[x] - m);
            total += e[x];
        }
        double z = apply_filters(V, s, e, top_k, top_p, keep, topp_margin);
        long n = 0;
        for (x = 0; x < V; x++) {
            p_out[x] = keep[x] ? e[x] / z : 0.0;
            n += keep[x];
        }
        *kept = n;
        *kept_frac = z / total;
    }
    free(s);
    free(e);
    free(keep);
    return fault;
}

/*
 * Draft distribution q' of one row: the given probabilities tempered as
 * q^(1/T), then the same filters with their own thresholds, renormalised
 * [SD §06: p and q must go through identical transforms].
 */
static int draft_probs_row(long V, const float *q, double T, int top_k, double top_p,
                           double *q_out, double *topp_margin, long *kept, double *kept_frac) {
    double *r = (double *)malloc(sizeof(double) * V);
    unsigned char *keep = (unsigned char *)malloc(V);
    long x;
    int fault = 0;
    for (x = 0; x < V; x++) {
        float f = q[x];
        if (isnan(f) || isinf(f) || signbit(f)) fault = OF_DRAFT_ROW;
        r[x] = (T == 1.0) ? (double)f : pow((double)f, 1.0 / T);
    }
    if (!fault) {
        double total = 0.0;
        for (x = 0; x < V; x++) total += r[x];
        double z = apply_filters(V, r, r, top_k, top_p, keep, topp_margin);
        if (z == 0.0) {
            fault = OF_DRAFT_MASS;
        } else {
            long n = 0;
            for (x = 0; x < V; x++) {
                q_out[x] = keep[x] ? r[x] / z : 0.0;
                n += keep[x];
            }
            *kept = n;
            *kept_frac = z / total;
        }
    }
    free(r);
    free(keep);
    return fault;
}

/* Greedy target token: argmax of the logits, lowest id on ties
 * [VLLM, "Greedy kernel：逐 token 比较"; SD §03]. */
static int greedy_row(long V, const void *row, int dtype, int32_t *arg) {
    double best = -INFINITY;
    long bi = -1, x;
    for (x = 0; x < V; x++) {
        double l = logit_at(row, dtype, x);
        if (isnan(l) || l == INFINITY) return OF_TARGET_ROW;
        if (l > best) {
            best = l;
            bi = x;
        }
    }
    if (bi < 0) return OF_TARGET_ROW;
    *arg = (int32_t)bi;
    return 0;
}

/*
 * Inverse-CDF draw over ascending token id: z = min{x : C_x > u * S}, with
 * C_x the running sum of w.  If rounding leaves no such x, the last token with
 * positive weight is returned.  *margin receives min over positive-weight x of
 * |u - C_x / S|.
 */
static int32_t inverse_cdf(long V, const double *w, double S, double u, double *margin) {
    double tau = u * S, c = 0.0, mg = INFINITY;
    long z = -1, last = -1, x;
    for (x = 0; x < V; x++) {
        if (w[x] > 0.0) {
            c += w[x];
            last = x;
            double d = fabs(u - c / S);
            if (d < mg) mg = d;
            if (z < 0 && c > tau) z = x;
        }
    }
    if (z < 0) z = last;
    *margin = mg;
    return (int32_t)z;
}

typedef struct {
    long V;
    int gmax;
    const int32_t *ids;      /* [gmax]          */
    const float *q;          /* [gmax, V] or NULL */
    const void *logits;      /* [gmax+1, V]     */
    int dtype;
    double T;
    int top_k;
    double top_p;
    const float *u_accept;   /* [gmax] */
    double u_sample;
    /* outputs */
    int32_t *tokens;         /* [gmax+1] */
    int32_t *num_accepted;
    double *p_y, *q_y;       /* [gmax] or NULL */
    double *resid_mass, *margin;
    int32_t *fault_out;
    /* per-row diagnostics [SD §14: record the filtered support and its mass],
     * each NULL or [gmax+1] (target rows) / [gmax] (draft rows): the top-p cut
     * margin of the row (the smaller of its target and draft margins), the
     * kept-set sizes, and the kept mass as a fraction of the tempered row's */
    double *row_margin;
    int32_t *kept_p, *kept_q;
    double *frac_p, *frac_q;
    /* per request, each NULL or one value: which decisions lie within OR_TOL of
     * their boundary (AMB_* bits), and the draw window: the tokens whose CDF
     * intervals meet [u - OR_TOL, u + OR_TOL] * S are those from z_lo to z_hi
     * (both drawn by inverse CDF, at u - OR_TOL and u + OR_TOL) */
    int32_t *amb_kind, *z_lo, *z_hi;
} request_t;

/* request i's slices of the batched per-row outputs ([N, gmax+1] / [N, gmax]) */
static void set_row_outputs(request_t *r, int i, double *row_margin, int32_t *kept_p, int32_t *kept_q,
                            double *frac_p, double *frac_q, int32_t *amb_kind, int32_t *z_lo, int32_t *z_hi) {
    size_t g = (size_t)r->gmax;
    r->amb_kind = amb_kind ? amb_kind + i : NULL;
    r->z_lo = z_lo ? z_lo + i : NULL;
    r->z_hi = z_hi ? z_hi + i : NULL;
    r->row_margin = row_margin ? row_margin + (size_t)i * (g + 1) : NULL;
    r->kept_p = kept_p ? kept_p + (size_t)i * (g + 1) : NULL;
    r->frac_p = frac_p ? frac_p + (size_t)i * (g + 1) : NULL;
    r->kept_q = kept_q ? kept_q + (size_t)i * g : NULL;
    r->frac_q = frac_q ? frac_q + (size_t)i * g : NULL;
}

/* the request's ambiguity kinds and draw window (see request_t) */
static void note_ambiguity(request_t *r, double mg_acc, double mg_topp, double mg_cdf, int32_t zlo, int32_t zhi) {
    if (r->amb_kind)
        *r->amb_kind = (mg_acc < OR_TOL ? AMB_ACCEPT : 0) | (mg_topp < OR_TOL ? AMB_TOP_P : 0) |
                       (mg_cdf < OR_TOL ? AMB_CDF : 0);
    if (r->z_lo) *r->z_lo = zlo;
    if (r->z_hi) *r->z_hi = zhi;
}

/* per-row diagnostics: unset rows read NaN (margins, fractions) and -1 (sizes) */
static void init_row_outputs(request_t *r) {
    int j;
    if (r->amb_kind) *r->amb_kind = 0;
    if (r->z_lo) *r->z_lo = -1;
    if (r->z_hi) *r->z_hi = -1;
    for (j = 0; j <= r->gmax; j++) {
        if (r->row_margin) r->row_margin[j] = NAN;
        if (r->kept_p) r->kept_p[j] = -1;
        if (r->frac_p) r->frac_p[j] = NAN;
        if (j < r->gmax) {
            if (r->kept_q) r->kept_q[j] = -1;
            if (r->frac_q) r->frac_q[j] = NAN;
        }
    }
}

/* row j's filter outcome: draft = 0 for the target row, 1 for the draft row */
static void note_row(request_t *r, int j, int draft, double topp_margin, long kept, double frac) {
    if (r->row_margin) {
        double m = r->row_margin[j];
        r->row_margin[j] = (isnan(m) || topp_margin < m) ? topp_margin : m;
    }
    if (!draft) {
        if (r->kept_p) r->kept_p[j] = (int32_t)kept;
        if (r->frac_p) r->frac_p[j] = frac;
    } else {
        if (r->kept_q) r->kept_q[j] = (int32_t)kept;
        if (r->frac_q) r->frac_q[j] = frac;
    }
}

static const void *logit_row(const request_t *r, int j) {
    size_t esz = r->dtype == 1 ? 2 : 4;
    return (const char *)r->logits + (size_t)j * (size_t)r->V * esz;
}

static void write_fault(request_t *r, int fault) {
    int j;
    for (j = 0; j <= r->gmax; j++) r->tokens[j] = -1;
    *r->num_accepted = -1;
    if (r->fault_out) *r->fault_out = fault;
}

/*
 * The token at the first rejection A (or the bonus position A = g): the
 * replacement weights max(0, p' - q') at a rejection [SD §04], with q' the
 * one-hot of the draft token when there are no draft probabilities [VLLM,
 * "Random kernel"], or p' of the bonus row when every draft was accepted
 * [SD §03, §06]; zero residual mass falls back to p'_A.  P[A] (and Q[A] with
 * draft probabilities, P[g] for the bonus) must be filled.
 */
static int32_t draw_token(const request_t *r, double *const *P, double *const *Q, int A, int g, double *S_out,
                          double *cmargin, int32_t *zlo, int32_t *zhi) {
    const long V = r->V;
    double *w = (double *)malloc(sizeof(double) * V);
    double S = 0.0;
    long x;
    if (A < g) {
        for (x = 0; x < V; x++) {
            double qx = r->q ? Q[A][x] : (x == r->ids[A] ? 1.0 : 0.0);
            double d = P[A][x] - qx;
            w[x] = d > 0.0 ? d : 0.0;
            S += w[x];
        }
        if (S == 0.0) {
            for (x = 0; x < V; x++) {
                w[x] = P[A][x];
                S += w[x];
            }
        }
    } else {
        for (x = 0; x < V; x++) {
            w[x] = P[g][x];
            S += w[x];
        }
    }
    int32_t z = inverse_cdf(V, w, S, r->u_sample, cmargin);
    double unused;
    *zlo = inverse_cdf(V, w, S, r->u_sample - OR_TOL, &unused);
    *zhi = inverse_cdf(V, w, S, r->u_sample + OR_TOL, &unused);
    *S_out = S;
    free(w);
    return z;
}

/* output row: accepted drafts, then the replacement or bonus, then -1
 * [VLLM, "拒绝采样…两个分支", output buffer of max_spec_len + 1] */
static void write_output(request_t *r, int A, int32_t z) {
    int j;
    for (j = 0; j <= r->gmax; j++) r->tokens[j] = -1;
    for (j = 0; j < A; j++) r->tokens[j] = r->ids[j];
    r->tokens[A] = z;
    *r->num_accepted = A;
}

/*
 * One request: the round of [SD §06] in the batched form of [VLLM,
 * "拒绝采样…两个分支"].
 */
static void verify_request(request_t *r) {
    const long V = r->V;
    int j, g = r->gmax, fault = 0;

    if (r->p_y)
        for (j = 0; j < r->gmax; j++) r->p_y[j] = NAN;
    if (r->q_y)
        for (j = 0; j < r->gmax; j++) r->q_y[j] = NAN;
    if (r->resid_mass) *r->resid_mass = NAN;
    if (r->margin) *r->margin = INFINITY;
    if (r->fault_out) *r->fault_out = 0;
    init_row_outputs(r);

    /* gamma_i: drafts run up to the first negative id (padding) */
    for (j = 0; j < r->gmax; j++)
        if (r->ids[j] < 0) {
            g = j;
            break;
        }
    for (j = 0; j < g; j++)
        if (r->ids[j] >= V) fault |= OF_DRAFT_ID;

    const double T = r->T;
    if (isnan(T) || T < 0.0 || isinf(T) || (T > 0.0 && T < (double)FLT_MIN)) fault |= OF_TEMPERATURE;
    const int greedy = (T == 0.0);
    if (!greedy && !(fault & OF_TEMPERATURE) && (isnan(r->top_p) || r->top_p <= 0.0)) fault |= OF_TOP_P;
    if (fault) {
        write_fault(r, fault);
        return;
    }

    int A;
    int32_t z;
    if (greedy) {
        /* [SD §03; VLLM "Greedy kernel"]: accept while the draft equals the
         * target argmax; the argmax of the first mismatching row (or of the
         * bonus row) completes the output. */
        int32_t *t = (int32_t *)malloc(sizeof(int32_t) * (g + 1));
        for (j = 0; j <= g; j++) fault |= greedy_row(V, logit_row(r, j), r->dtype, &t[j]);
        if (fault) {
            free(t);
            write_fault(r, fault);
            return;
        }
        A = g;
        for (j = 0; j < g; j++)
            if (r->ids[j] != t[j]) {
                A = j;
                break;
            }
        z = t[A];
        free(t);
        note_ambiguity(r, INFINITY, INFINITY, INFINITY, z, z);
    } else {
        /* full distributions p'_0..p'_g and q'_0..q'_{g-1} */
        double **P = (double **)malloc(sizeof(double *) * (g + 1));
        double **Q = (double **)malloc(sizeof(double *) * (g + 1));
        double mg = INFINITY, tm, mg_acc = INFINITY, mg_topp = INFINITY;
        for (j = 0; j <= g; j++) {
            P[j] = (double *)malloc(sizeof(double) * V);
            Q[j] = NULL;
        }
        double *topp_m = (double *)malloc(sizeof(double) * (2 * g + 2));
        for (j = 0; j <= g && !fault; j++) {
            long n = -1;
            double f = NAN;
            fault |= target_probs_row(V, logit_row(r, j), r->dtype, T, r->top_k, r->top_p, P[j], &tm, &n, &f);
            topp_m[2 * j] = tm;
            topp_m[2 * j + 1] = INFINITY;
            note_row(r, j, 0, tm, n, f);
        }
        if (r->q)
            for (j = 0; j < g && !fault; j++) {
                long n = -1;
                double f = NAN;
                Q[j] = (double *)malloc(sizeof(double) * V);
                fault |= draft_probs_row(V, r->q + (size_t)j * V, T, r->top_k, r->top_p, Q[j], &tm, &n, &f);
                topp_m[2 * j + 1] = tm;
                note_row(r, j, 1, tm, n, f);
            }
        if (fault) {
            for (j = 0; j <= g; j++) {
                free(P[j]);
                free(Q[j]);
            }
            free(P);
            free(Q);
            free(topp_m);
            write_fault(r, fault);
            return;
        }

        /* accept test per position until the first rejection [SD §04, §06, §07]:
         * accept iff u * q'(y) < p'(y); without draft probabilities q' is the
         * one-hot of the draft token [VLLM, "Random kernel"]. */
        A = g;
        for (j = 0; j < g; j++) {
            int32_t y = r->ids[j];
            double py = P[j][y];
            double qy = r->q ? Q[j][y] : 1.0;
            if (r->p_y) r->p_y[j] = py;
            if (r->q_y) r->q_y[j] = qy;
        }
        for (j = 0; j < g; j++) {
            int32_t y = r->ids[j];
            double py = P[j][y];
            double qy = r->q ? Q[j][y] : 1.0;
            double u = (double)r->u_accept[j];
            if (qy > 0.0) {
                double d = fabs(u - py / qy);
                if (d < mg_acc) mg_acc = d;
            }
            if (topp_m[2 * j] < mg_topp) mg_topp = topp_m[2 * j];
            if (topp_m[2 * j + 1] < mg_topp) mg_topp = topp_m[2 * j + 1];
            if (!(u * qy < py)) {
                A = j;
                break;
            }
        }
        if (A == g && topp_m[2 * g] < mg_topp) mg_topp = topp_m[2 * g];

        double cm, S;
        int32_t zlo, zhi;
        z = draw_token(r, P, Q, A, g, &S, &cm, &zlo, &zhi);
        mg = mg_acc < mg_topp ? mg_acc : mg_topp;
        if (cm < mg) mg = cm;
        if (r->resid_mass) *r->resid_mass = S;
        if (r->margin) *r->margin = mg;
        note_ambiguity(r, mg_acc, mg_topp, cm, zlo, zhi);
        for (j = 0; j <= g; j++) {
            free(P[j]);
            free(Q[j]);
        }
        free(P);
        free(Q);
        free(topp_m);
    }

    write_output(r, A, z);
}

/*
 * Batched entry.  All pointers are host pointers; draft_probs, temperature,
 * top_k, top_p and every diagnostic output may be NULL (temperature NULL means
 * 1.0, top_k NULL means off, top_p NULL means 1.0).  Layouts are row-major
 * with the vocabulary contiguous: draft_ids [N,gmax], draft_probs [N,gmax,V],
 * target_logits [N,gmax+1,V] (dtype 0 = fp32, 1 = bf16 bit patterns),
 * u_accept [N,gmax], u_sample [N], out_tokens [N,gmax+1], out_num_accepted [N],
 * p_y and q_y [N,gmax], resid_mass, margin [N], fault [N], and the per-row
 * diagnostics row_margin, kept_p, frac_p [N,gmax+1] and kept_q, frac_q [N,gmax],
 * and per request amb_kind, z_lo, z_hi [N] (see request_t).
 */
int oracle_spec_verify(int N, int gmax, int V, const int32_t *draft_ids, const float *draft_probs,
                       const void *target_logits, int dtype, const float *temperature,
                       const int32_t *top_k, const float *top_p, const float *u_accept,
                       const float *u_sample, int32_t *out_tokens, int32_t *out_num_accepted,
                       double *p_y, double *q_y, double *resid_mass, double *margin,
                       int32_t *fault, double *row_margin, int32_t *kept_p, int32_t *kept_q,
                       double *frac_p, double *frac_q, int32_t *amb_kind, int32_t *z_lo, int32_t *z_hi) {
    int i;
    if (N < 0 || gmax < 0 || V < 1 || (dtype != 0 && dtype != 1)) return 1;
    size_t esz = dtype == 1 ? 2 : 4;
    for (i = 0; i < N; i++) {
        request_t r;
        r.V = V;
        r.gmax = gmax;
        r.ids = draft_ids + (size_t)i * gmax;
        r.q = draft_probs ? draft_probs + (size_t)i * gmax * V : NULL;
        r.logits = (const char *)target_logits + (size_t)i * (gmax + 1) * (size_t)V * esz;
        r.dtype = dtype;
        r.T = temperature ? (double)temperature[i] : 1.0;
        r.top_k = top_k ? top_k[i] : 0;
        r.top_p = top_p ? (double)top_p[i] : 1.0;
        r.u_accept = u_accept + (size_t)i * gmax;
        r.u_sample = (double)u_sample[i];
        r.tokens = out_tokens + (size_t)i * (gmax + 1);
        r.num_accepted = out_num_accepted + i;
        r.p_y = p_y ? p_y + (size_t)i * gmax : NULL;
        r.q_y = q_y ? q_y + (size_t)i * gmax : NULL;
        r.resid_mass = resid_mass ? resid_mass + i : NULL;
        r.margin = margin ? margin + i : NULL;
        r.fault_out = fault ? fault + i : NULL;
        set_row_outputs(&r, i, row_margin, kept_p, kept_q, frac_p, frac_q, amb_kind, z_lo, z_hi);
        verify_request(&r);
    }
    return 0;
}

/*
 * One request in the synthetic acceptance mode [VLLM, "关于 synthetic / block
 * 验证模式"]: draft j is accepted iff u_j < rate_j, without the target
 * probabilities, so A (the first rejection, or gamma) is known before any row
 * is read.  Readings: only row A is read (faults come from it and from the
 * request's parameters), and its token is drawn as in the standard method:
 * the argmax of row A for a greedy request, else the replacement
 * max(0, p'_A - q'_A) (p'_A if that is zero) at a rejection, or p' of the
 * bonus row.  p_y and q_y are not computed (NaN).
 */
static void verify_request_synthetic(request_t *r, const float *rates) {
    const long V = r->V;
    int j, g = r->gmax, fault = 0;

    if (r->p_y)
        for (j = 0; j < r->gmax; j++) r->p_y[j] = NAN;
    if (r->q_y)
        for (j = 0; j < r->gmax; j++) r->q_y[j] = NAN;
    if (r->resid_mass) *r->resid_mass = NAN;
    if (r->margin) *r->margin = INFINITY;
    if (r->fault_out) *r->fault_out = 0;
    init_row_outputs(r);

    for (j = 0; j < r->gmax; j++)
        if (r->ids[j] < 0) {
            g = j;
            break;
        }
    for (j = 0; j < g; j++)
        if (r->ids[j] >= V) fault |= OF_DRAFT_ID;
    const double T = r->T;
    if (isnan(T) || T < 0.0 || isinf(T) || (T > 0.0 && T < (double)FLT_MIN)) fault |= OF_TEMPERATURE;
    const int greedy = (T == 0.0);
    if (!greedy && !(fault & OF_TEMPERATURE) && (isnan(r->top_p) || r->top_p <= 0.0)) fault |= OF_TOP_P;
    if (fault) {
        write_fault(r, fault);
        return;
    }

    /* the synthetic accept test, position by position until the first rejection */
    double mg = INFINITY, mg_acc = INFINITY, mg_topp = INFINITY, cm = INFINITY;
    int32_t zlo = -1, zhi = -1;
    int A = g;
    for (j = 0; j < g; j++) {
        double u = (double)r->u_accept[j], rate = (double)rates[j];
        double d = fabs(u - rate);
        if (d < mg) mg = d;
        if (d < mg_acc) mg_acc = d;
        if (!(u < rate)) {
            A = j;
            break;
        }
    }

    int32_t z = -1;
    if (greedy) {
        fault |= greedy_row(V, logit_row(r, A), r->dtype, &z);
        zlo = zhi = z;
    } else {
        /* only row A's distributions: P[A] (also P[g] when A = g), Q[A] */
        double **P = (double **)calloc((size_t)g + 1, sizeof(double *));
        double **Q = (double **)calloc((size_t)g + 1, sizeof(double *));
        double tm, f = NAN;
        long n = -1;
        P[A] = (double *)malloc(sizeof(double) * V);
        fault |= target_probs_row(V, logit_row(r, A), r->dtype, T, r->top_k, r->top_p, P[A], &tm, &n, &f);
        if (tm < mg) mg = tm;
        if (tm < mg_topp) mg_topp = tm;
        note_row(r, A, 0, tm, n, f);
        if (!fault && A < g && r->q) {
            Q[A] = (double *)malloc(sizeof(double) * V);
            fault |= draft_probs_row(V, r->q + (size_t)A * V, T, r->top_k, r->top_p, Q[A], &tm, &n, &f);
            if (tm < mg) mg = tm;
            if (tm < mg_topp) mg_topp = tm;
            note_row(r, A, 1, tm, n, f);
        }
        if (!fault) {
            double S;
            z = draw_token(r, P, Q, A, g, &S, &cm, &zlo, &zhi);
            if (cm < mg) mg = cm;
            if (r->resid_mass) *r->resid_mass = S;
        }
        free(P[A]);
        free(Q[A]);
        free(P);
        free(Q);
    }
    if (fault) {
        write_fault(r, fault);
        return;
    }
    if (r->margin) *r->margin = mg;
    note_ambiguity(r, mg_acc, mg_topp, cm, zlo, zhi);
    write_output(r, A, z);
}

/* The batched entry of the synthetic acceptance mode; rates [gmax]. */
int oracle_spec_verify_synthetic(int N, int gmax, int V, const int32_t *draft_ids, const float *draft_probs,
                                 const void *target_logits, int dtype, const float *temperature,
                                 const int32_t *top_k, const float *top_p, const float *rates,
                                 const float *u_accept, const float *u_sample, int32_t *out_tokens,
                                 int32_t *out_num_accepted, double *resid_mass, double *margin, int32_t *fault,
                                 double *row_margin, int32_t *kept_p, int32_t *kept_q, double *frac_p,
                                 double *frac_q, int32_t *amb_kind, int32_t *z_lo, int32_t *z_hi) {
    int i;
    if (N < 0 || gmax < 0 || V < 1 || (dtype != 0 && dtype != 1) || (gmax > 0 && !rates)) return 1;
    size_t esz = dtype == 1 ? 2 : 4;
    for (i = 0; i < N; i++) {
        request_t r;
        r.V = V;
        r.gmax = gmax;
        r.ids = draft_ids + (size_t)i * gmax;
        r.q = draft_probs ? draft_probs + (size_t)i * gmax * V : NULL;
        r.logits = (const char *)target_logits + (size_t)i * (gmax + 1) * (size_t)V * esz;
        r.dtype = dtype;
        r.T = temperature ? (double)temperature[i] : 1.0;
        r.top_k = top_k ? top_k[i] : 0;
        r.top_p = top_p ? (double)top_p[i] : 1.0;
        r.u_accept = u_accept + (size_t)i * gmax;
        r.u_sample = (double)u_sample[i];
        r.tokens = out_tokens + (size_t)i * (gmax + 1);
        r.num_accepted = out_num_accepted + i;
        r.p_y = NULL;
        r.q_y = NULL;
        r.resid_mass = resid_mass ? resid_mass + i : NULL;
        r.margin = margin ? margin + i : NULL;
        r.fault_out = fault ? fault + i : NULL;
        set_row_outputs(&r, i, row_margin, kept_p, kept_q, frac_p, frac_q, amb_kind, z_lo, z_hi);
        verify_request_synthetic(&r, rates);
    }
    return 0;
}

/* Single-row views of the two transforms, for checking them on their own. */
int oracle_target_probs(int V, const void *logits, int dtype, double T, int top_k, double top_p,
                        double *p_out, double *topp_margin) {
    double tm, frac;
    long n;
    int f = target_probs_row(V, logits, dtype, T, top_k, top_p, p_out, &tm, &n, &frac);
    if (topp_margin) *topp_margin = tm;
    return f;
}

int oracle_draft_probs(int V, const float *q, double T, int top_k, double top_p, double *q_out,
                       double *topp_margin) {
    double tm, frac;
    long n;
    int f = draft_probs_row(V, q, T, top_k, top_p, q_out, &tm, &n, &frac);
    if (topp_margin) *topp_margin = tm;
    return f;
}
