/*
 * spec_oracle.c -- plain CPU oracle for batched draft-token verification.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the reference that the GPU library
 * is compared against.  Only the test suite, the smoke check and the CPU
 * baseline of the benchmark load it; the GPU library never does, and the two
 * share no code, header or constant.
 *
 * Arithmetic: IEEE double throughout.  fp32 and bf16 logits are widened
 * exactly.  Every sum runs sequentially in token-id order.  No blocking, no
 * fusion, no reordering: each function follows the definition it cites.
 *
 * Sources (the pages are web summaries; none prints an equation or listing):
 *  [SD]   standard speculative sampling: the draft proposes a run of tokens and
 *         the target verifies them in parallel (MineDraft page, section 1;
 *         SpecTr-GBV page, section 1).  The per-token rule itself is the
 *         published one of Leviathan, Kalman & Matias (2023) and Chen et al.
 *         (2023), restated here from its mathematics.
 *  [GBV]  greedy block verification: verifies the whole drafted block jointly,
 *         optimal for a single draft (SpecTr-GBV page, section 1, second
 *         limitation).  Written from its published definition (Sun et al.,
 *         "Block Verification Accelerates Speculative Decoding", 2024).
 *  [KS]   SpecTr, the multi-draft baseline: verifies the drafts position by
 *         position and stops at the first rejection (SpecTr-GBV page, section 1),
 *         each selection step searching a scaling factor rho by bisection,
 *         O(V log K) (section 3).  Written from the published k-sequential
 *         selection of Sun et al., "SpecTr: Fast Speculative Decoding via
 *         Optimal Transport" (2023), restated from its mathematics.
 *  [DR]   drafting: K i.i.d. blocks sampled position by position from the
 *         draft rows (SpecTr-GBV page, section 2, step 1), by the same
 *         inverse CDF as every correction draw.
 *  [MD]   SpecTr-GBV, K i.i.d. drafts of length L (SpecTr-GBV page, section 2,
 *         "algorithmic procedure", steps 1-5): start from accepted length 0 and
 *         an empty rejected set H; walk the drafts; verify each one's sub-block
 *         from position tau+1; on acceptance advance tau and record the draft
 *         index; on rejection put the sub-block into H and skip it later; draw
 *         the correction from the target when tau = L, else from the residual.
 *
 * Readings taken where the pages are silent (each one is listed in the design
 * notes together with what pins it):
 *  - Node rows: drafts that share a prefix stand at the same node of the draft
 *    tree.  Every row is read from the lowest-index draft with that prefix.
 *  - Eq. (2) of the SpecTr-GBV paper is not printed: the acceptance
 *    probability of draft k is GBV's h on its sub-block, whose first position
 *    is tested against the node's current residual.
 *  - Eq. (4) / Algorithm 2 are not printed: the residual at the node is kept
 *    as omega(v) = [v not in H] * max(alpha*p(v) - beta*q(v), 0) with mass N.
 *    A rejection sets beta += N (the residual-of-residual step of recursive
 *    rejection sampling); a duplicate first token (in H) is rejected without a
 *    test but still updates the residual.
 *  - "Skip" keeps no state across calls: the ABI is stateless.
 *  - Tests are strict: accept iff u < h.  Among several successes the largest
 *    position wins (longest accepted prefix).
 *  - Sampling: inverse CDF in token-id order, y = min{v : C_v > u*Z}.
 *  - A residual with zero mass (reachable only by rounding) marks the request
 *    degenerate and falls back to the node's target distribution.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SVO_F32 0
#define SVO_BF16 1

#define SVO_TOKEN 0
#define SVO_BLOCK 1
#define SVO_MULTI 2
#define SVO_SPECTR 3

#define SVO_FLAG_DEGENERATE 1
#define SVO_FLAG_INVALID 2

#define SVO_KMAX 64
#define SVO_LMAX 16

typedef struct {
    int K, L, V, dtype;
    const void *tgt;        /* this request's target rows [K][L+1][V] */
    const void *drf;        /* this request's draft rows  [K][L][V]   */
    const int32_t *X;       /* draft tokens [K][L] */
    double T;
    const float *ua;        /* acceptance uniforms [K][L] (fp32 entry point) */
    const double *ua_d;     /* ... or as doubles (exact-law entry point); one is NULL */
    double uc;              /* correction uniform */
    double *law;            /* [V]: the distribution the correction is drawn from, or NULL */
    double *p, *q, *om;     /* scratch, V doubles each */
    double *h_out;          /* [K][L] evaluated acceptance probabilities, or NULL */
    double margin;          /* min |u - threshold| over every decision taken */
    int flags;
    int64_t tests;          /* acceptance tests evaluated */
    int64_t sweeps;         /* O(V) selection steps: residual masses, R_m, inverse CDFs */
    unsigned char *touched; /* [2L+1][K]: canonical rows whose logits were read */
} svo_req;

/* ---------------------------------------------------------------- inputs */

static double svo_logit(const svo_req *r, int target, int k, int j, int v)
{
    size_t row = target ? (size_t)k * (size_t)(r->L + 1) + (size_t)j
                        : (size_t)k * (size_t)r->L + (size_t)j;
    size_t idx = row * (size_t)r->V + (size_t)v;
    const void *base = target ? r->tgt : r->drf;
    if (r->dtype == SVO_F32)
        return (double)((const float *)base)[idx];
    uint32_t bits = (uint32_t)((const uint16_t *)base)[idx] << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return (double)f;
}

/* Node rows: the row of draft k at position j describes the node reached by
 * the prefix X[k][0..j-1].  It is read from the lowest-index draft that has the
 * same prefix, so every draft at one node sees one distribution. */
static int svo_canon(const svo_req *r, int k, int j)
{
    for (int c = 0; c < k; ++c) {
        int same = 1;
        for (int i = 0; i < j; ++i)
            if (r->X[c * r->L + i] != r->X[k * r->L + i]) { same = 0; break; }
        if (same)
            return c;
    }
    return k;
}

/* A row can be turned into a distribution iff it holds no NaN, no +inf and at
 * least one finite entry (-inf entries are tokens of probability zero). */
static int svo_row_valid(const svo_req *r, int target, int k, int j)
{
    int c = svo_canon(r, k, j);
    int finite = 0;
    for (int v = 0; v < r->V; ++v) {
        double l = svo_logit(r, target, c, j, v);
        if (isnan(l) || l == INFINITY)
            return 0;
        if (l != -INFINITY)
            finite = 1;
    }
    return finite;
}

/* ------------------------------------------------------------- softmax */

/* Temperature softmax of a node row:
 *   pi(v) = exp((l_v - max) / T) / sum_v' exp((l_v' - max) / T).
 * A row that is read but is not a distribution makes the request invalid. */
static void svo_softmax(svo_req *r, int target, int k, int j, double *out)
{
    int c = svo_canon(r, k, j);
    if (!svo_row_valid(r, target, k, j))
        r->flags |= SVO_FLAG_INVALID;
    r->touched[(target ? j : r->L + 1 + j) * r->K + c] = 1;
    double mx = -INFINITY;
    for (int v = 0; v < r->V; ++v) {
        double l = svo_logit(r, target, c, j, v);
        if (l > mx)
            mx = l;
    }
    double s = 0.0;
    for (int v = 0; v < r->V; ++v) {
        out[v] = exp((svo_logit(r, target, c, j, v) - mx) / r->T);
        s += out[v];
    }
    for (int v = 0; v < r->V; ++v)
        out[v] /= s;
}

/* Natural-log partition function of a node row at temperature T:
 * ln sum_v exp(l_v / T) = max/T + ln sum_v exp((l_v - max)/T). */
static double svo_row_lse(const svo_req *r, int target, int k, int j)
{
    int c = svo_canon(r, k, j);
    double mx = -INFINITY;
    for (int v = 0; v < r->V; ++v) {
        double l = svo_logit(r, target, c, j, v);
        if (l > mx)
            mx = l;
    }
    double s = 0.0;
    for (int v = 0; v < r->V; ++v)
        s += exp((svo_logit(r, target, c, j, v) - mx) / r->T);
    return mx / r->T + log(s);
}

/* ------------------------------------------------------- small helpers */

/* Likelihood ratio num/den of a drafted token.  A token the draft gives
 * probability zero cannot have been drafted; it is given ratio +inf when the
 * numerator is positive and 0 otherwise. */
static double svo_ratio(double num, double den)
{
    if (den > 0.0)
        return num / den;
    return num > 0.0 ? INFINITY : 0.0;
}

/* One step of GBV's weight chain: w' = min(w * num/den, 1); a zero weight
 * stays zero. */
static double svo_chain(double w, double num, double den)
{
    if (w == 0.0)
        return 0.0;
    double t = w * svo_ratio(num, den);
    return t < 1.0 ? t : 1.0;
}

/* Acceptance uniform i of the request, as a double. */
static double svo_ua(const svo_req *r, int i)
{
    return r->ua_d ? r->ua_d[i] : (double)r->ua[i];
}

static void svo_note_margin(svo_req *r, double m)
{
    if (m < r->margin)
        r->margin = m;
}

/* One acceptance test: accepted iff u < h. */
static int svo_test(svo_req *r, int k, int m, double h)
{
    double u = svo_ua(r, k * r->L + (m - 1));
    r->tests += 1;
    if (r->h_out)
        r->h_out[k * r->L + (m - 1)] = h;
    svo_note_margin(r, fabs(u - h));
    return u < h;
}

/* Inverse-CDF draw in token-id order from the unnormalised weights om[]:
 * Z = sum_v om(v), t = u*Z, y = min{v : C_v > t} with C_v the running sum.
 * If rounding leaves no such v, y is the last v with om(v) > 0.  Returns -1 if
 * Z is not positive (the caller then falls back). */
static int svo_icdf(svo_req *r, const double *om, double *Z_out)
{
    r->sweeps += 1;
    double Z = 0.0;
    for (int v = 0; v < r->V; ++v)
        Z += om[v];
    *Z_out = Z;
    if (!(Z > 0.0) || !isfinite(Z))
        return -1;
    if (r->law)   /* a uniform u gives v with probability om(v)/Z */
        for (int v = 0; v < r->V; ++v)
            r->law[v] = om[v] / Z;
    double t = r->uc * Z;
    double C = 0.0;
    for (int v = 0; v < r->V; ++v) {
        double prev = C;
        C += om[v];
        if (C > t) {
            double lo = (t - prev) / Z, hi = (C - t) / Z;
            svo_note_margin(r, lo < hi ? lo : hi);
            return v;
        }
    }
    svo_note_margin(r, 0.0);
    for (int v = r->V - 1; v >= 0; --v)
        if (om[v] > 0.0)
            return v;
    return -1;
}

/* Draw from the target row of node (k, j) itself (used at tau = L, and as the
 * fallback of a degenerate residual). */
static int svo_draw_target(svo_req *r, int k, int j, double *Z_out)
{
    svo_softmax(r, 1, k, j, r->p);
    return svo_icdf(r, r->p, Z_out);
}

/* ------------------------------------------------- token-level rule [SD] */

/* Standard speculative sampling, one draft: for j = 0..L-1 accept X[j] iff
 * u_j < min(1, p_j(x)/q_j(x)); at the first rejection tau = j and the
 * correction is drawn from norm(max(p_j - q_j, 0)); if all L are accepted the
 * correction is drawn from the target row after the block. */
static void svo_run_token(svo_req *r, int32_t *tau_o, int32_t *k_o, int32_t *y_o,
                          double *Z_o)
{
    const int L = r->L, V = r->V;
    for (int j = 0; j < L; ++j) {
        svo_softmax(r, 1, 0, j, r->p);
        svo_softmax(r, 0, 0, j, r->q);
        int x = r->X[j];
        double a = svo_ratio(r->p[x], r->q[x]);
        if (a > 1.0)
            a = 1.0;
        if (!svo_test(r, 0, j + 1, a)) {
            for (int v = 0; v < V; ++v)
                r->om[v] = fmax(r->p[v] - r->q[v], 0.0);
            int y = svo_icdf(r, r->om, Z_o);
            if (y < 0) {
                r->flags |= SVO_FLAG_DEGENERATE;
                y = svo_draw_target(r, 0, j, Z_o);
            }
            *tau_o = j;
            *k_o = j > 0 ? 0 : -1;
            *y_o = y;
            return;
        }
    }
    *tau_o = L;
    *k_o = 0;
    *y_o = svo_draw_target(r, 0, L, Z_o);
}

/* -------------------------------------------- block verification [GBV] */

/* GBV on the single draft X[0..L-1]:
 *   w_0 = 1,  w_i = min(w_{i-1} * p_{i-1}(X_i) / q_{i-1}(X_i), 1);
 *   for i < L: R_i = sum_v max(w_i p_i(v) - q_i(v), 0),  h_i = R_i / (R_i + 1 - w_i)
 *   (h_i = 1 when the denominator is 0);  h_L = w_L;
 *   tau = max{i >= 1 : u_i < h_i}, or 0 -- evaluated from i = L downward;
 *   correction ~ norm(max(w_tau p_tau - q_tau, 0)) if tau < L, else p_L. */
static void svo_run_block(svo_req *r, int32_t *tau_o, int32_t *k_o, int32_t *y_o,
                          double *Z_o)
{
    const int L = r->L, V = r->V;
    double w[SVO_LMAX + 1];
    w[0] = 1.0;
    for (int i = 1; i <= L; ++i) {
        svo_softmax(r, 1, 0, i - 1, r->p);
        svo_softmax(r, 0, 0, i - 1, r->q);
        int x = r->X[i - 1];
        w[i] = svo_chain(w[i - 1], r->p[x], r->q[x]);
    }
    int tau = 0;
    for (int m = L; m >= 1; --m) {
        double h;
        if (m == L) {
            h = w[L];
        } else {
            svo_softmax(r, 1, 0, m, r->p);
            svo_softmax(r, 0, 0, m, r->q);
            r->sweeps += 1;
            double R = 0.0;
            for (int v = 0; v < V; ++v)
                R += fmax(w[m] * r->p[v] - r->q[v], 0.0);
            double d = R + 1.0 - w[m];
            h = d > 0.0 ? R / d : 1.0;
        }
        if (svo_test(r, 0, m, h)) {
            tau = m;
            break;
        }
    }
    int y;
    if (tau == L) {
        y = svo_draw_target(r, 0, L, Z_o);
    } else {
        svo_softmax(r, 1, 0, tau, r->p);
        svo_softmax(r, 0, 0, tau, r->q);
        for (int v = 0; v < V; ++v)
            r->om[v] = fmax(w[tau] * r->p[v] - r->q[v], 0.0);
        y = svo_icdf(r, r->om, Z_o);
        if (y < 0) {
            r->flags |= SVO_FLAG_DEGENERATE;
            y = svo_draw_target(r, 0, tau, Z_o);
        }
    }
    *tau_o = tau;
    *k_o = tau > 0 ? 0 : -1;
    *y_o = y;
}

/* ------------------------------------------ K-draft block walk [MD] */

static int svo_in(const int *H, int nH, int x)
{
    for (int i = 0; i < nH; ++i)
        if (H[i] == x)
            return 1;
    return 0;
}

/* Residual weights at the current node s = (own, tau):
 *   omega(v) = [v not in H] * max(alpha * p_s(v) - beta * q_s(v), 0). */
static void svo_node_residual(svo_req *r, int own, int tau, double alpha, double beta,
                              const int *H, int nH)
{
    svo_softmax(r, 1, own, tau, r->p);
    svo_softmax(r, 0, own, tau, r->q);
    for (int v = 0; v < r->V; ++v)
        r->om[v] = svo_in(H, nH, v) ? 0.0 : fmax(alpha * r->p[v] - beta * r->q[v], 0.0);
}

static double svo_node_mass(svo_req *r, int own, int tau, double alpha, double beta,
                            const int *H, int nH)
{
    svo_node_residual(r, own, tau, alpha, beta, H, nH);
    r->sweeps += 1;
    double N = 0.0;
    for (int v = 0; v < r->V; ++v)
        N += r->om[v];
    return N;
}

static int svo_same_prefix(const svo_req *r, int a, int b, int n)
{
    for (int i = 0; i < n; ++i)
        if (r->X[a * r->L + i] != r->X[b * r->L + i])
            return 0;
    return 1;
}

/* K-draft block verification.  State: accepted node s (prefix of length tau of
 * draft `own`; the root when tau = 0), the last draft that advanced tau (kstar,
 * -1 at the root), the first tokens H rejected at s, and the residual
 * (alpha, beta, N); the start state (1, 0, 1) is the target itself.
 * Drafts are visited once, in index order:
 *  - a draft whose first tau tokens differ from s is skipped;
 *  - a draft whose token at s is in H is rejected without a test, then
 *    beta += N and N is recomputed;
 *  - otherwise GBV runs on its sub-block X[k][tau..L-1]: the first position is
 *    tested against omega/N with the node's draft row, deeper positions use the
 *    draft's own rows; positions m = L, L-1, ..., tau+1 are tested with
 *    u[k][m-1] < h_m and the first success wins;
 *  - success at m: tau = m, own = kstar = k, H = {} and, if m < L,
 *    (alpha, beta, N) = (w_m, 1, R_m); no success: H += {x}, beta += N, N anew;
 *  - the walk ends after the last draft or when tau = L.
 * The correction is drawn from the target row after the block of kstar when
 * tau = L, else from omega at the final node. */
static void svo_run_multi(svo_req *r, int32_t *tau_o, int32_t *k_o, int32_t *y_o,
                          double *Z_o)
{
    const int K = r->K, L = r->L, V = r->V;
    int tau = 0, own = 0, kstar = -1;
    double alpha = 1.0, beta = 0.0, N = 1.0;
    int H[SVO_KMAX];
    int nH = 0;
    double w[SVO_LMAX + 1], R[SVO_LMAX + 1];

    for (int k = 0; k < K && tau < L; ++k) {
        if (!svo_same_prefix(r, k, own, tau))
            continue;
        int x = r->X[k * L + tau];
        if (svo_in(H, nH, x)) {
            beta += N;
            N = svo_node_mass(r, own, tau, alpha, beta, H, nH);
        } else {
            /* first position: node residual omega/N against the node's draft row */
            svo_node_residual(r, own, tau, alpha, beta, H, nH);
            w[tau + 1] = svo_chain(1.0, r->om[x] / N, r->q[x]);
            /* deeper positions: the draft's own rows */
            for (int j = tau + 1; j < L; ++j) {
                svo_softmax(r, 1, k, j, r->p);
                svo_softmax(r, 0, k, j, r->q);
                int xj = r->X[k * L + j];
                w[j + 1] = svo_chain(w[j], r->p[xj], r->q[xj]);
            }
            int acc = 0;
            for (int m = L; m > tau; --m) {
                double h;
                if (m == L) {
                    h = w[L];
                } else {
                    svo_softmax(r, 1, k, m, r->p);
                    svo_softmax(r, 0, k, m, r->q);
                    r->sweeps += 1;
                    double Rm = 0.0;
                    for (int v = 0; v < V; ++v)
                        Rm += fmax(w[m] * r->p[v] - r->q[v], 0.0);
                    R[m] = Rm;
                    double d = Rm + 1.0 - w[m];
                    h = d > 0.0 ? Rm / d : 1.0;
                }
                if (svo_test(r, k, m, h)) {
                    acc = m;
                    break;
                }
            }
            if (acc > 0) {
                tau = acc;
                own = k;
                kstar = k;
                nH = 0;
                if (tau < L) {
                    alpha = w[tau];
                    beta = 1.0;
                    N = R[tau];
                }
            } else {
                H[nH++] = x;
                beta += N;
                N = svo_node_mass(r, own, tau, alpha, beta, H, nH);
            }
        }
        if (tau < L && !(N > 0.0)) {
            /* only rounding can empty the residual: restart from the node's target */
            r->flags |= SVO_FLAG_DEGENERATE;
            alpha = 1.0;
            beta = 0.0;
            N = 1.0;
            nH = 0;
        }
    }

    int y;
    if (tau == L) {
        y = svo_draw_target(r, own, L, Z_o);
    } else {
        svo_node_residual(r, own, tau, alpha, beta, H, nH);
        y = svo_icdf(r, r->om, Z_o);
        if (y < 0) {
            r->flags |= SVO_FLAG_DEGENERATE;
            y = svo_draw_target(r, own, tau, Z_o);
        }
    }
    *tau_o = tau;
    *k_o = kstar;
    *y_o = y;
}

/* --------------------------------------- k-sequential selection [KS] */

/* beta(rho) = sum_v min(q(v), p(v)/rho): the chance that one candidate drawn
 * from q is accepted with probability min(1, p/(rho q)). */
static double svo_ks_beta(const svo_req *r, double rho)
{
    double b = 0.0;
    for (int v = 0; v < r->V; ++v)
        b += fmin(r->q[v], r->p[v] / rho);
    return b;
}

/* c = sum_{i<n} (1 - beta)^i = (1 - (1 - beta)^n) / beta: the expected number
 * of tries when n candidates are tried in turn, each succeeding with
 * probability beta -- so the mass a token receives from acceptances is
 * c min(q, p/rho).  The sum form is exact at n = 1 and needs no limit at
 * beta = 0. */
static double svo_ks_c(double beta, int n)
{
    double c = 0.0, t = 1.0;
    for (int i = 0; i < n; ++i) {
        c += t;
        t *= 1.0 - beta;
    }
    return c;
}

/* D(rho) = sum_v max(p - rho q, 0): the p-mass that rho q does not cover. */
static double svo_ks_excess(const svo_req *r, double rho)
{
    double d = 0.0;
    for (int v = 0; v < r->V; ++v)
        d += fmax(r->p[v] - rho * r->q[v], 0.0);
    return d;
}

/* Whether rho is feasible, c(beta(rho)) <= rho.  Multiplied by beta this reads
 * 1 - rho beta <= (1 - beta)^n, and 1 - rho beta = sum_v p - sum_v min(p, rho q)
 * = D(rho).  The two forms decide the same thing; each is evaluated where the
 * rounding of its inputs cannot flip it.  The gap rho - c equals
 * rho ((1 - beta)^n - D) / (1 - D): once (1 - beta)^n is below double
 * rounding -- nearly identical rows, or many candidates -- the rounding of
 * beta alone moves c by more than that gap, while D and (1 - beta)^n are each
 * exact to rounding.  When beta is tiny (nearly disjoint supports) D and
 * (1 - beta)^n both lie within ~n beta of 1 and the product form cancels,
 * while rho - c does not.  The quotient form is taken for beta <= 2^-10
 * (there (1 - beta)^n >= 0.93 for n <= 64), the product form above. */
static int svo_ks_feasible(const svo_req *r, double rho, int n)
{
    double beta = svo_ks_beta(r, rho);
    if (beta <= 0x1p-10)
        return svo_ks_c(beta, n) <= rho;
    double x = 1.0 - beta, xn = 1.0;
    for (int i = 0; i < n; ++i)
        xn *= x;
    return svo_ks_excess(r, rho) <= xn;
}

/* The smallest rho in [1, n] with c(beta(rho)) <= rho -- exactly the rho for
 * which p - c min(q, p/rho) stays non-negative everywhere -- by bisection until
 * the bracket holds two adjacent doubles, one O(V) pass per step (about
 * 52 + log2 n passes).  A bracket this tight makes the oracle return the
 * definition's rho itself: rho can be badly conditioned (the slope below
 * tends to 0 as the p-mass of tokens with p/q < rho tends to 1), and the
 * residual mass (1 - beta)^n is small whenever rejection is rare.  The
 * condition is monotone in rho: wherever rho = c(beta(rho)), the slope of
 * rho - c(beta(rho)) is at least n x^(n-1) (1 - x) / (1 - x^n) > 0 with
 * x = 1 - beta, so the condition turns from false to true once. */
static double svo_ks_rho(svo_req *r, int n)
{
    if (n <= 1)
        return 1.0;
    r->sweeps += 1;
    if (svo_ks_feasible(r, 1.0, n))
        return 1.0;
    double lo = 1.0, hi = (double)n;
    for (;;) {
        double mid = 0.5 * (lo + hi);
        if (!(mid > lo && mid < hi))
            break;
        r->sweeps += 1;
        if (svo_ks_feasible(r, mid, n))
            hi = mid;
        else
            lo = mid;
    }
    return hi;
}

/* SpecTr over K drafts: at position j the candidates are the tokens X[k][j] of
 * the drafts whose first j tokens are the accepted prefix, tried in draft
 * order with u[k][j] < min(1, p(x)/(rho* q(x))); the first success extends the
 * prefix, no success stops the walk with tau = j and a correction from
 * norm(max(p - c(rho*) min(q, p/rho*), 0)); with all L accepted the correction
 * comes from the target row after the block.  The recorded draft is the one
 * whose candidate was accepted last. */
static void svo_run_spectr(svo_req *r, int32_t *tau_o, int32_t *k_o, int32_t *y_o,
                           double *Z_o)
{
    const int K = r->K, L = r->L, V = r->V;
    int own = 0, kacc = -1;
    for (int j = 0; j < L; ++j) {
        svo_softmax(r, 1, own, j, r->p);
        svo_softmax(r, 0, own, j, r->q);
        int n = 0;
        for (int k = 0; k < K; ++k)
            n += svo_same_prefix(r, k, own, j);
        double rho = svo_ks_rho(r, n);
        int acc = -1;
        for (int k = 0; k < K && acc < 0; ++k) {
            if (!svo_same_prefix(r, k, own, j))
                continue;
            int x = r->X[k * L + j];
            double a = svo_ratio(r->p[x], rho * r->q[x]);
            if (a > 1.0)
                a = 1.0;
            if (svo_test(r, k, j + 1, a))
                acc = k;
        }
        if (acc < 0) {
            double c = svo_ks_c(svo_ks_beta(r, rho), n);
            for (int v = 0; v < V; ++v)
                r->om[v] = fmax(r->p[v] - c * fmin(r->q[v], r->p[v] / rho), 0.0);
            int y = svo_icdf(r, r->om, Z_o);
            if (y < 0) {
                r->flags |= SVO_FLAG_DEGENERATE;
                y = svo_draw_target(r, own, j, Z_o);
            }
            *tau_o = j;
            *k_o = kacc;
            *y_o = y;
            return;
        }
        own = acc;
        kacc = acc;
    }
    *tau_o = L;
    *k_o = kacc;
    *y_o = svo_draw_target(r, own, L, Z_o);
}

/* ------------------------------------------------------------ validation */

/* Request data the rules cannot act on: T not a positive finite number, a
 * token outside [0, V) or a uniform outside [0, 1).  (A node row that is not a
 * distribution -- NaN, +inf or all -inf -- is detected when it is read.) */
static int svo_request_valid(const svo_req *r)
{
    if (!(r->T > 0.0) || !isfinite(r->T))
        return 0;
    for (int i = 0; i < r->K * r->L; ++i) {
        if (r->X[i] < 0 || r->X[i] >= r->V)
            return 0;
        double u = svo_ua(r, i);
        if (!(u >= 0.0 && u < 1.0))
            return 0;
    }
    if (!(r->uc >= 0.0 && r->uc < 1.0))
        return 0;
    return 1;
}

/* ------------------------------------------------------ drafting [DR] */

/*
 * Drafting K i.i.d. blocks of length L (SpecTr-GBV page, section 2, step 1),
 * the other half of the draft-then-verify loop (MineDraft page, section 1).
 * Position by position, draft k draws X[k][j] from the temperature softmax of
 * the node row of its prefix X[k][0..j-1] -- the row of the lowest-index draft
 * with that prefix, so drafts that meet at a node draw from one distribution --
 * by the inverse CDF of its own uniform u_draft[k][j] (token-id order, strict
 * ">", as every draw of this oracle).  Each draft's block is therefore an
 * independent draw from the draft model's sequence distribution.
 *
 * Requests [b_begin, b_end) of a batch: draft [B][K][L][V] (SVO_F32 or bf16
 * bits), temperature [B], u_draft [B][K][L] in, tokens [B][K][L] out.
 * flags [B]: SVO_FLAG_INVALID when T is not a positive finite number, a
 * uniform lies outside [0, 1), or a node row read is not a distribution; the
 * request's tokens are then all -1.  margin [B] (optional): the smallest
 * distance of a draw's threshold to a CDF boundary, in probability units.
 * rows [B] (optional): node rows read.  Returns 0, or -1 for bad arguments.
 */
int svo_draft(int B, int K, int L, int V, int dtype, const void *draft,
              const float *temperature, const float *u_draft, int b_begin, int b_end,
              int32_t *tokens, int32_t *flags, double *margin, int32_t *rows)
{
    if (B < 0 || K < 1 || K > SVO_KMAX || L < 1 || L > SVO_LMAX || V < 1 ||
        (dtype != SVO_F32 && dtype != SVO_BF16) || b_begin < 0 || b_end > B ||
        b_begin > b_end)
        return -1;
    size_t es = dtype == SVO_F32 ? 4 : 2;
    size_t drow = (size_t)K * (size_t)L * (size_t)V;
    double *q = (double *)malloc(sizeof(double) * (size_t)V);
    unsigned char *touched = (unsigned char *)malloc((size_t)(2 * L + 1) * (size_t)K);
    if (!q || !touched) {
        free(q);
        free(touched);
        return -2;
    }
    for (int b = b_begin; b < b_end; ++b) {
        int32_t *X = tokens + (size_t)b * (size_t)K * (size_t)L;
        const float *u = u_draft + (size_t)b * (size_t)K * (size_t)L;
        svo_req r;
        memset(&r, 0, sizeof r);
        r.K = K;
        r.L = L;
        r.V = V;
        r.dtype = dtype;
        r.drf = (const char *)draft + (size_t)b * drow * es;
        r.X = X;
        r.T = (double)temperature[b];
        r.q = q;
        r.margin = INFINITY;
        r.touched = touched;
        memset(touched, 0, (size_t)(2 * L + 1) * (size_t)K);
        int ok = r.T > 0.0 && isfinite(r.T);
        for (int i = 0; i < K * L; ++i) {
            X[i] = -1;
            ok &= u[i] >= 0.0f && u[i] < 1.0f;
        }
        for (int j = 0; j < L && ok; ++j) {
            for (int k = 0; k < K && ok; ++k) {
                svo_softmax(&r, 0, k, j, q);     /* node row of k's prefix */
                if (r.flags & SVO_FLAG_INVALID) {
                    ok = 0;
                    break;
                }
                r.uc = (double)u[k * L + j];     /* the draw's uniform */
                double Z;
                X[k * L + j] = svo_icdf(&r, q, &Z);
            }
        }
        int nrows = 0;
        for (int i = 0; i < (2 * L + 1) * K; ++i)
            nrows += touched[i];
        if (!ok) {
            for (int i = 0; i < K * L; ++i)
                X[i] = -1;
        }
        if (flags)
            flags[b] = ok ? 0 : SVO_FLAG_INVALID;
        if (margin)
            margin[b] = ok ? r.margin : INFINITY;
        if (rows)
            rows[b] = nrows;
    }
    free(q);
    free(touched);
    return 0;
}

/* --------------------------------------------------------------- entry */

/*
 * Verify requests [b_begin, b_end) of a batch.  Layouts (row-major, host memory):
 *   target [B][K][L+1][V], draft [B][K][L][V] (dtype SVO_F32 or SVO_BF16 bits),
 *   tokens [B][K][L], temperature [B], u_accept [B][K][L], u_correct [B].
 * Outputs [B]: accept_len (-1 for invalid request data), draft_index (-1 iff
 * accept_len <= 0), correction, flags (bit 0 degenerate residual, bit 1
 * invalid data: bad T, token or uniform, or a row read by the rules that is
 * not a distribution).  Optional (NULL to skip): row_lse [B][K][2L+1] (target rows
 * 0..L then draft rows 0..L-1, each the node row's ln-partition function at
 * T), accept_prob [B][K][L] (h of every evaluated test, NaN elsewhere),
 * resid_mass [B] (mass Z of the distribution the correction was drawn from,
 * in probability units), margin [B] (smallest |u - threshold| over the
 * request's decisions), counters [B][3] (tests, O(V) selection steps,
 * distinct logit rows read).
 * Returns 0, or -1 for arguments outside the supported ranges.
 */
static int svo_verify_any(int method, int B, int K, int L, int V, int dtype,
                          const void *target, const void *draft, const int32_t *tokens,
                          const float *temperature, const float *u_accept,
                          const double *u_accept_d, const float *u_correct,
                          const double *u_correct_d, int b_begin, int b_end,
                          int32_t *accept_len, int32_t *draft_index, int32_t *correction,
                          int32_t *flags, double *row_lse, double *accept_prob,
                          double *resid_mass, double *margin, int64_t *counters,
                          double *corr_law)
{
    if (method < SVO_TOKEN || method > SVO_SPECTR || B < 0 || K < 1 || K > SVO_KMAX ||
        L < 1 || L > SVO_LMAX || V < 1 || (dtype != SVO_F32 && dtype != SVO_BF16))
        return -1;
    if ((method == SVO_TOKEN || method == SVO_BLOCK) && K != 1)
        return -1;
    if (b_begin < 0 || b_end > B || b_begin > b_end)
        return -1;

    size_t es = dtype == SVO_F32 ? 4 : 2;
    size_t trow = (size_t)K * (size_t)(L + 1) * (size_t)V;
    size_t drow = (size_t)K * (size_t)L * (size_t)V;
    double *scratch = (double *)malloc(sizeof(double) * 3 * (size_t)V);
    unsigned char *touched = (unsigned char *)malloc((size_t)(2 * L + 1) * (size_t)K);
    if (!scratch || !touched) {
        free(scratch);
        free(touched);
        return -2;
    }

    for (int b = b_begin; b < b_end; ++b) {
        svo_req r;
        r.K = K;
        r.L = L;
        r.V = V;
        r.dtype = dtype;
        r.tgt = (const char *)target + (size_t)b * trow * es;
        r.drf = (const char *)draft + (size_t)b * drow * es;
        r.X = tokens + (size_t)b * (size_t)K * (size_t)L;
        r.T = (double)temperature[b];
        r.ua = u_accept ? u_accept + (size_t)b * (size_t)K * (size_t)L : NULL;
        r.ua_d = u_accept_d ? u_accept_d + (size_t)b * (size_t)K * (size_t)L : NULL;
        r.uc = u_correct_d ? u_correct_d[b] : (double)u_correct[b];
        r.law = corr_law ? corr_law + (size_t)b * (size_t)V : NULL;
        if (r.law)
            for (int v = 0; v < V; ++v)
                r.law[v] = NAN;
        r.p = scratch;
        r.q = scratch + V;
        r.om = scratch + 2 * (size_t)V;
        r.h_out = accept_prob ? accept_prob + (size_t)b * (size_t)K * (size_t)L : NULL;
        r.margin = INFINITY;
        r.flags = 0;
        r.tests = 0;
        r.sweeps = 0;
        r.touched = touched;
        memset(touched, 0, (size_t)(2 * L + 1) * (size_t)K);
        if (r.h_out)
            for (int i = 0; i < K * L; ++i)
                r.h_out[i] = NAN;

        int32_t tau = -1, ks = -1, y = -1;
        double Z = NAN;
        if (!svo_request_valid(&r)) {
            r.flags |= SVO_FLAG_INVALID;
            r.margin = INFINITY;
        } else if (method == SVO_TOKEN) {
            svo_run_token(&r, &tau, &ks, &y, &Z);
        } else if (method == SVO_BLOCK) {
            svo_run_block(&r, &tau, &ks, &y, &Z);
        } else if (method == SVO_MULTI) {
            svo_run_multi(&r, &tau, &ks, &y, &Z);
        } else {
            svo_run_spectr(&r, &tau, &ks, &y, &Z);
        }
        if (r.flags & SVO_FLAG_INVALID) {
            r.flags = SVO_FLAG_INVALID;
            r.margin = INFINITY;
            tau = -1;
            ks = -1;
            y = -1;
            Z = NAN;
        }
        accept_len[b] = tau;
        draft_index[b] = ks;
        correction[b] = y;
        if (flags)
            flags[b] = r.flags;
        if (resid_mass)
            resid_mass[b] = Z;
        if (margin)
            margin[b] = r.margin;
        if (row_lse) {
            double *o = row_lse + (size_t)b * (size_t)K * (size_t)(2 * L + 1);
            for (int k = 0; k < K; ++k) {
                for (int j = 0; j <= L; ++j)
                    o[k * (2 * L + 1) + j] = svo_row_lse(&r, 1, k, j);
                for (int j = 0; j < L; ++j)
                    o[k * (2 * L + 1) + L + 1 + j] = svo_row_lse(&r, 0, k, j);
            }
        }
        if (counters) {
            int64_t rows = 0;
            for (int i = 0; i < (2 * L + 1) * K; ++i)
                rows += touched[i];
            counters[3 * (size_t)b + 0] = r.tests;
            counters[3 * (size_t)b + 1] = r.sweeps;
            counters[3 * (size_t)b + 2] = rows;
        }
    }
    free(scratch);
    free(touched);
    return 0;
}

int svo_verify(int method, int B, int K, int L, int V, int dtype,
               const void *target, const void *draft, const int32_t *tokens,
               const float *temperature, const float *u_accept, const float *u_correct,
               int b_begin, int b_end,
               int32_t *accept_len, int32_t *draft_index, int32_t *correction,
               int32_t *flags, double *row_lse, double *accept_prob,
               double *resid_mass, double *margin, int64_t *counters)
{
    return svo_verify_any(method, B, K, L, V, dtype, target, draft, tokens, temperature,
                          u_accept, NULL, u_correct, NULL, b_begin, b_end, accept_len,
                          draft_index, correction, flags, row_lse, accept_prob, resid_mass,
                          margin, counters, NULL);
}

/* svo_verify with the uniforms as doubles, for enumerating the oracle's output
 * law exactly: a test is accepted iff u < h, so u = 0 takes the accepting branch
 * of any test with h > 0 and u = h the rejecting one, with no float32 rounding
 * in between.  corr_law [B][V] (optional) receives the distribution the
 * correction is drawn from (om/Z of the final draw; NaN for an invalid request):
 * the law of the correction token given everything else. */
int svo_verify_exact(int method, int B, int K, int L, int V, int dtype,
                     const void *target, const void *draft, const int32_t *tokens,
                     const float *temperature, const double *u_accept,
                     const double *u_correct, int b_begin, int b_end,
                     int32_t *accept_len, int32_t *draft_index, int32_t *correction,
                     int32_t *flags, double *accept_prob, double *resid_mass,
                     double *corr_law)
{
    return svo_verify_any(method, B, K, L, V, dtype, target, draft, tokens, temperature,
                          NULL, u_accept, NULL, u_correct, b_begin, b_end, accept_len,
                          draft_index, correction, flags, NULL, accept_prob, resid_mass,
                          NULL, NULL, corr_law);
}
