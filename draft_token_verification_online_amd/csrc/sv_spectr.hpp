// sv_spectr.hpp -- the scaling factor of SpecTr's k-sequential selection.
//
// SpecTr verifies K drafts position by position (SpecTr-GBV page, section 1)
// and spends a binary search over a scaling factor rho on every selection step
// (section 3 puts that step at O(V log K)).  With n candidates on the accepted
// prefix tried in turn, each accepted with probability min(1, p/(rho q)):
//   beta(rho) = sum_v min(q, p/rho),  c = sum_{i<n} (1 - beta)^i,
// and rho* is the smallest rho in [1, n] with c <= rho, the condition under
// which the residual p - c min(q, p/rho) is non-negative everywhere.
//
// Each sweep at rho returns sums of fp32 terms over the two sides of the
// breakpoint p = rho q: D = sum_{p > rho q} (p - rho q), and the p and q mass
// on either side.  Normalising by the sweep's own totals makes sum p = sum q = 1
// hold exactly for the values it summed; without that, the 1e-7 mismatch
// against the row statistics becomes a spurious root wherever (1 - beta)^n
// drops below 1e-7.  The normalised problem is the nominal one at
// rho_hat = kappa rho, kappa = 1 +- 1e-7, which the search carries along.
// With B1 = sum_{p > rho q} q and B2 = sum_{p <= rho q} p, beta = B1 + B2/rho
// and rho beta = 1 - D; c <= rho is tested in the form that rounding cannot
// flip (the same split as the CPU oracle):
//   beta <= 2^-10:  G = rho - c(x) >= 0, x = 1 - beta
//                   (G' = 1 - c'(x) B2/rho^2);
//   beta >  2^-10:  H = x^n - D >= 0,  x = (rho - 1 + D)/rho
//                   (H' = n x^(n-1) B2/rho^2 + B1).
// The quotient form loses its gap rho (1 - beta)^n below the rounding of c once
// (1 - beta)^n is tiny (nearly identical rows, many candidates); the product
// form compares two numbers within ~n beta of 1 when beta is tiny (nearly
// disjoint supports).  rho* = 1 exactly when D(1) = 0 (p = q).
//
// The search takes one histogram sweep and then Newton sweeps:
//   1. bin log2(p/q) over [0, log2 n) into kHistBins bins (fixed-point sums of
//      p and q per bin, so the result does not depend on the order of the
//      atomic adds); suffix and prefix sums give the condition at every bin
//      edge, and the first edge where it holds brackets rho* to a relative
//      width of about ln(n) / kHistBins;
//   2. from the regula-falsi point of that bin, Newton within [1, n],
//      safeguarded by bisection whenever a step leaves the bracket or fails to
//      halve the step before it; the search stops once the step is below
//      1e-7 rho -- the resolution of rho / S_q in fp32 -- taking that last step
//      without another sweep (the sums are constant between breakpoints).
// On the synthetic workloads this is 3 to 4.5 sweeps per step on average,
// against 50-odd for a bisection to double precision.
#pragma once

#include "sv_device.hpp"

namespace sv {

constexpr int kHistBins = 1024;
constexpr float kFixScale = 2147483648.0f;          // 2^31: p, q <= 1 per bin sum
constexpr double kFixUnit = 1.0 / 2147483648.0;
constexpr double kRhoTol = 1e-7;
constexpr double kQuotientFormBeta = 0x1p-10;

// Histogram of log2(p/q) over [0, log2 n): hist[b] and hist[kHistBins + b] hold
// the p and q mass (2^31 fixed point, p = 2^(l_p c - MPc) ap, MPc the shift term
// of the target row, likewise q) of tokens in
// bin b.  out[] receives, as sums of the unscaled exponentials e_p, e_q: e_p and
// e_q over tokens with p/q >= n, e_p over tokens with p/q < 1, then
// D(1) = sum max(p - q, 0), and e_p, e_q over all tokens.
template <int NT, typename RD>
__device__ void ratio_histogram(const RD &P, const RD &Q, int nch, float MPc, float MQc, float ap,
                                float aq, float off, float scale, const Scale &c, unsigned *hist,
                                double (&out)[6], double *red) {
    for (int i = threadIdx.x; i < 2 * kHistBins; i += NT) hist[i] = 0u;
    __syncthreads();
    double s[6] = {0.0, 0.0, 0.0, 0.0, 0.0, 0.0};
    auto chunk = [&](const float xp[8], const float xq[8]) {
        float cp = 0.0f, cq = 0.0f, cl = 0.0f, cd = 0.0f, ta = 0.0f, tb = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float yp = expo(xp[e], c, MPc), yq = expo(xq[e], c, MQc);
            const float ep = fast_exp2(yp), eq = fast_exp2(yq);
            ta += ep;
            tb += eq;
            cd += fmaxf(fmaf(ap, ep, -(aq * eq)), 0.0f);
            const float t = (yp - yq + off) * scale;   // NaN when p = q = 0: no bin
            if (t >= static_cast<float>(kHistBins)) {
                cp += ep;
                cq += eq;
            } else if (t >= 0.0f) {
                const int bin = static_cast<int>(t);
                atomicAdd(&hist[bin], __float2uint_rn(ep * ap * kFixScale));
                atomicAdd(&hist[kHistBins + bin], __float2uint_rn(eq * aq * kFixScale));
            } else if (t < 0.0f) {
                cl += ep;
            }
        }
        s[0] += static_cast<double>(cp);
        s[1] += static_cast<double>(cq);
        s[2] += static_cast<double>(cl);
        s[3] += static_cast<double>(cd);
        s[4] += static_cast<double>(ta);
        s[5] += static_cast<double>(tb);
    };
    stream_rows<NT, depth_for<RD, 32>(), true>(P, Q, nch,
                             [&](const float xp[8], const float xq[8], int) { chunk(xp, xq); });
    block_sum_n<NT, 6>(s, red);   // its barriers also publish hist[]
#pragma unroll
    for (int i = 0; i < 6; ++i) out[i] = s[i];
}

// Sums over a row pair split at p = rho q, with p = e_p ap, q = e_q aq and
// bq = rho aq in fp32: out = {sum_{p > rho q} (p - rho q), then e_q over
// p > rho q, e_q over p <= rho q, e_p over p > rho q, e_p over p <= rho q}.
template <int NT, typename RD>
__device__ void sweep_excess(const RD &P, const RD &Q, int nch, float MPc, float MQc, float ap,
                             float bq, const Scale &c, double (&out)[5], double *red) {
    double s[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
    auto chunk = [&](const float xp[8], const float xq[8]) {
        float cd = 0.0f, qa = 0.0f, qb = 0.0f, pa = 0.0f, pb = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float ep = fast_exp2(expo(xp[e], c, MPc));
            const float eq = fast_exp2(expo(xq[e], c, MQc));
            const float d = fmaf(ap, ep, -(bq * eq));
            const bool pos = d > 0.0f;
            cd += pos ? d : 0.0f;
            qa += pos ? eq : 0.0f;
            qb += pos ? 0.0f : eq;
            pa += pos ? ep : 0.0f;
            pb += pos ? 0.0f : ep;
        }
        s[0] += static_cast<double>(cd);
        s[1] += static_cast<double>(qa);
        s[2] += static_cast<double>(qb);
        s[3] += static_cast<double>(pa);
        s[4] += static_cast<double>(pb);
    };
    stream_rows<NT, depth_for<RD, 32>(), true>(P, Q, nch,
                             [&](const float xp[8], const float xq[8], int) { chunk(xp, xq); });
    block_sum_n<NT, 5>(s, red);
#pragma unroll
    for (int i = 0; i < 5; ++i) out[i] = s[i];
}

__device__ __forceinline__ double pow_int(double x, int n) {
    double r = 1.0;
    for (int i = 0; i < n; ++i) r *= x;
    return r;
}

// sum_{i<n} x^i, the expected number of tries.
__device__ __forceinline__ double tries(double x, int n) {
    double c = 0.0, t = 1.0;
    for (int i = 0; i < n; ++i) {
        c += t;
        t *= x;
    }
    return c;
}

// sum_{i=1}^{n-1} i x^(i-1), the derivative of tries().
__device__ __forceinline__ double tries_slope(double x, int n) {
    double d = 0.0, t = 1.0;
    for (int i = 1; i < n; ++i) {
        d += i * t;
        t *= x;
    }
    return d;
}

// The feasibility condition at rho (normalised problem) in the form rounding
// cannot flip (>= 0 iff feasible), its slope, and x = 1 - beta, from D, B1, B2.
__device__ __forceinline__ void feasibility(double rho, double D, double B1, double B2, int n,
                                            double *g, double *dg, double *x) {
    const double beta = B1 + B2 / rho;
    if (beta <= kQuotientFormBeta) {
        const double xx = 1.0 - beta;
        *g = rho - tries(xx, n);
        *dg = 1.0 - tries_slope(xx, n) * B2 / (rho * rho);
        *x = xx;
    } else {
        const double xx = (rho - 1.0 + D) / rho;
        const double xn1 = pow_int(xx, n - 1);
        *g = xn1 * xx - D;
        *dg = n * xn1 * B2 / (rho * rho) + B1;
        *x = xx;
    }
}

// The condition at a histogram edge e from the normalised mass of tokens with
// p/q >= e (Pge, Qge) and the p mass below it (A).
__device__ __forceinline__ double edge_gap(double e, double Pge, double Qge, double A, int n) {
    double g, dg, x;
    feasibility(e, fmax(Pge - e * Qge, 0.0), Qge, A, n, &g, &dg, &x);
    return g;
}

// rho* and c = sum_{i<n} x^i at rho* for the node rows P (target) and Q
// (draft) with shift terms MPc, MQc and sums SP, SQ under scale c2; n >= 2
// candidates.  Both are
// returned in the normalisation of (SP, SQ): acceptance min(1, p/(rho q)) and
// residual max(p - c q, (1 - c/rho) p) with p, q from those statistics.  Every
// thread of the block returns the same values.  hist[] holds 2 * kHistBins
// entries, red[] 6 * NT/64, br[] 4, ired[] NT/64.
template <int NT, typename RD>
__device__ void spectr_scale(const RD &P, const RD &Q, int nch, float MPc, double SP, float MQc,
                             double SQ, const Scale &c2, int n, double &rho_out,
                             double &c_out, unsigned *hist, double *red, double *br,
                             int *ired) {
    static_assert(2 * NT == kHistBins, "two histogram bins per thread");
    const int tid = threadIdx.x;
    const float ap = static_cast<float>(1.0 / SP), aq = static_cast<float>(1.0 / SQ);
    const double apd = ap, aqd = aq;
    const double scale = kHistBins / log2(static_cast<double>(n));
    const float off = static_cast<float>(log2(SQ) - log2(SP));
    double hs[6];
    ratio_histogram<NT, RD>(P, Q, nch, MPc, MQc, ap, aq, off, static_cast<float>(scale), c2, hist,
                            hs, red);
    if (!(hs[3] > 0.0)) {   // D(1) = 0: p = q, every token is accepted, rho* = 1
        rho_out = 1.0;
        c_out = 1.0;
        return;
    }
    // normalised masses: divide the e_p sums by their total, the bins (of e_p ap)
    // by ap times it
    const double hiP = hs[0] / hs[4], hiQ = hs[1] / hs[5], loP = hs[2] / hs[4];
    const double fP = kFixUnit / (apd * hs[4]), fQ = kFixUnit / (aqd * hs[5]);

    // thread t owns bins bh = kHistBins-1-2t and bl = bh-1 (descending in t): an
    // exclusive scan in thread order gives the mass above its bins.  The bin
    // sums are integers below 2^42, exact in doubles, so prefix = total - suffix
    // is exact too.
    const int bh = kHistBins - 1 - 2 * tid, bl = bh - 1;
    const double ph = hist[bh], pl = hist[bl];
    const double qh = hist[kHistBins + bh], ql = hist[kHistBins + bl];
    const double aboveP = block_exclusive_scan<NT>(ph + pl, red);
    const double aboveQ = block_exclusive_scan<NT>(qh + ql, red);
    const double totP = block_sum<NT>(ph + pl, red);
    const double sPh = aboveP + ph, sQh = aboveQ + qh;          // suffix sums at bh
    const double sPl = sPh + pl, sQl = sQh + ql;                // at bl
    const double eh = exp2(bh / scale), el = exp2(bl / scale);
    const double Gh = edge_gap(eh, hiP + sPh * fP, hiQ + sQh * fQ, loP + (totP - sPh) * fP, n);
    const double Gl = edge_gap(el, hiP + sPl * fP, hiQ + sQl * fQ, loP + (totP - sPl) * fP, n);
    // first edge >= 1 where the condition holds (rho = 1 is infeasible: D(1) > 0)
    int first = (bl >= 1 && Gl >= 0.0) ? bl : (Gh >= 0.0 ? bh : kHistBins);
    first = block_min_int<NT>(first, ired);
    // br: edge first-1 and edge first (edge kHistBins is rho = n), with their values
    if (bl == first - 1) { br[0] = el; br[1] = Gl; }
    if (bh == first - 1) { br[0] = eh; br[1] = Gh; }
    if (bl == first) { br[2] = el; br[3] = Gl; }
    if (bh == first) { br[2] = eh; br[3] = Gh; }
    if (tid == 0 && first == kHistBins) {
        br[2] = static_cast<double>(n);
        br[3] = edge_gap(static_cast<double>(n), hiP, hiQ, loP + totP * fP, n);
    }
    __syncthreads();
    const double ea = br[0], Ga = br[1], eb = br[2], Gb = br[3];
    double rho;
    if (first >= 2 && Ga < 0.0 && Gb >= 0.0) rho = ea + (eb - ea) * (-Ga / (Gb - Ga));
    else if (first == 1) rho = eb;
    else rho = 0.5 * (ea + eb);
    if (!(rho > 1.0 && rho <= static_cast<double>(n))) rho = 0.5 * (ea + eb);

    // Newton within [1, n], bisecting when a step leaves the bracket or does not
    // halve the one before it
    double lo = 1.0, hi = static_cast<double>(n);
    double dx_old = hi - lo, dx = dx_old;
    double rho_fin = hi, c_fin = static_cast<double>(n);
    for (int it = 0; it < 64; ++it) {
        double sw[5];
        sweep_excess<NT, RD>(P, Q, nch, MPc, MQc, ap, static_cast<float>(rho / SQ), c2, sw, red);
        const double EPt = sw[3] + sw[4], EQt = sw[1] + sw[2];
        const double kap = (aqd * EQt) / (apd * EPt);
        const double rh = rho * kap;
        const double B1 = sw[1] / EQt, B2 = sw[4] / EPt, D = sw[0] / (apd * EPt);
        double g, dg, x;
        feasibility(rh, D, B1, B2, n, &g, &dg, &x);
        dg *= kap;   // slope in nominal rho
        if (g < 0.0) lo = rho;
        else hi = rho;
        const double step = dg > 0.0 ? g / dg : INFINITY;
        if (fabs(step) <= kRhoTol * rho || hi - lo <= 2.0 * kRhoTol * hi) {
            double nr = isfinite(step) ? rho - step : hi;
            nr = fmin(fmax(nr, lo), hi);
            // the sums are constant and D linear in rho between breakpoints
            double gf, dgf, xf;
            feasibility(nr * kap, fmax(D - B1 * (nr * kap - rh), 0.0), B1, B2, n, &gf, &dgf, &xf);
            rho_fin = nr;
            c_fin = tries(xf, n) / kap;
            break;
        }
        double nr = rho - step;
        const bool newton = nr > lo && nr < hi && fabs(2.0 * g) <= fabs(dx_old * dg);
        dx_old = dx;
        if (newton) {
            dx = step;
        } else {
            nr = 0.5 * (lo + hi);
            dx = rho - nr;
        }
        rho = nr;
        rho_fin = hi;
        c_fin = tries(x, n) / kap;
    }
    rho_out = rho_fin;
    c_out = c_fin;
}

// rho* and c as spectr_scale returns them, found the way the SpecTr-GBV page
// costs SpecTr's selection step (section 3, O(|Omega| log K)): plain bisection
// of [1, n], one sweep per halving, until the bracket is below kRhoTol of rho --
// about 24 + log2(n) sweeps, each normalised like the Newton search's.
template <int NT, typename RD>
__device__ void spectr_scale_bisect(const RD &P, const RD &Q, int nch, float MPc, double SP,
                                    float MQc, double SQ, const Scale &c2, int n,
                                    double &rho_out, double &c_out, double *red) {
    const float ap = static_cast<float>(1.0 / SP), aq = static_cast<float>(1.0 / SQ);
    const double apd = ap, aqd = aq;
    // the condition at rho (>= 0 iff feasible) and c there, from one sweep
    auto probe = [&](double rho, double *c) {
        double sw[5];
        sweep_excess<NT, RD>(P, Q, nch, MPc, MQc, ap, static_cast<float>(rho / SQ), c2, sw, red);
        const double EPt = sw[3] + sw[4], EQt = sw[1] + sw[2];
        const double kap = (aqd * EQt) / (apd * EPt);
        const double B1 = sw[1] / EQt, B2 = sw[4] / EPt, D = sw[0] / (apd * EPt);
        double g, dg, x;
        feasibility(rho * kap, D, B1, B2, n, &g, &dg, &x);
        *c = tries(x, n) / kap;
        return (sw[0] > 0.0) ? g : 1.0;   // D(rho) = 0: nothing left uncovered
    };
    double c1;
    if (probe(1.0, &c1) >= 0.0) {   // p = q (or rho = 1 already feasible)
        rho_out = 1.0;
        c_out = 1.0;
        return;
    }
    double lo = 1.0, hi = static_cast<double>(n), c_hi = -1.0;
    while (hi - lo > kRhoTol * hi) {
        const double mid = 0.5 * (lo + hi);
        double cm;
        if (probe(mid, &cm) < 0.0) {
            lo = mid;
        } else {
            hi = mid;
            c_hi = cm;
        }
    }
    if (c_hi < 0.0) probe(hi, &c_hi);   // rho = n was never probed
    rho_out = hi;
    c_out = c_hi;
}

}  // namespace sv
