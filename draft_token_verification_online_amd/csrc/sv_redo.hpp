// sv_redo.hpp -- requests re-evaluated in fp64.
//
// The fast kernels form every exponential in fp32 (one v_exp_f32 per element),
// so an acceptance probability h or a residual mass carries a relative error
// of order 1e-7, amplified by the conditioning of the rule (GBV's
// h = R / (R + 1 - w) by ~1 / (R + 1 - w)).  A decision whose threshold lies
// within that error of its uniform could come out differently in exact
// arithmetic.  The fast walks therefore list every request with such a decision
// (the margin test of SV_FLAG_NEAR_TIE, widened by a first-order error estimate
// for ill-conditioned tests), and two launches take each listed request again
// from the start in fp64:
//
//   redo_stats_kernel  one workgroup per (listed request, node row), over the
//                      whole chip: M = max_v l_v and log2 S with
//                      S = sum_v exp((l_v - M) / T), in one pass (a running
//                      maximum, the sum rescaled when it grows);
//   redo_walk_kernel   one workgroup per listed request: every probability
//                      exp((l_v - M) / T) / S, residual mass, weight chain,
//                      scaling-factor search and inverse-CDF draw in double,
//                      with the rules stated in sv_walk.hpp (token level, GBV
//                      over K drafts, SpecTr).
//
// Double exponentials come from exp2_d (range reduction to |f| <= 1/2 and a
// degree-13 polynomial; within 1.4e-16).  The outputs differ from exact arithmetic
// only where a decision lies within double rounding (~1e-13, times the rule's
// conditioning) of its threshold.  Listed requests are rare -- about one in a
// hundred on flat residuals, where the correction draw lands within 1e-5 Z of a
// boundary of the cumulative weights -- and with none listed both launches
// return after reading the count.
#pragma once

#include "sv_device.hpp"
#include "sv_walk.hpp"

namespace sv {

constexpr int kFlagRedone = 8;
constexpr int kRedoThreads = 512;        // per listed request
constexpr int kRedoStatsThreads = 512;   // per (listed request, node row)
constexpr int kRedoDepth = 4;            // chunks per row in flight per thread


// 2^a in double precision: a = k + f with k = rint(a), |f| <= 1/2, and
// 2^f = exp(f ln2) by its Taylor polynomial of degree 13 (truncation below
// 5e-18 for |f ln2| <= 0.347), scaled by ldexp.  Within 1.4e-16 of 2^a over
// the double range (checked against a long-double exp2 on 2e7 arguments).
// No table: every exponential of a sweep is independent straight-line code.
// Branch-free: a is clamped to [-1080, 1030] (NaN to -1080), where ldexp gives
// 0 below the subnormal range and +inf above the double range.
__device__ __forceinline__ double exp2_d(double a) {
    a = fmin(fmax(a, -1080.0), 1030.0);
    const double k = rint(a);
    const double f = a - k;   // exact
    double p = 0x1.816193166d0f9p-40;
    p = fma(f, p, 0x1.c3bd650fc2986p-36);
    p = fma(f, p, 0x1.e8cac7351bb25p-32);
    p = fma(f, p, 0x1.e4cf5158b8ecap-28);
    p = fma(f, p, 0x1.b5253d395e7c4p-24);
    p = fma(f, p, 0x1.62c0223a5c824p-20);
    p = fma(f, p, 0x1.ffcbfc588b0c7p-17);
    p = fma(f, p, 0x1.430912f86c787p-13);
    p = fma(f, p, 0x1.5d87fe78a6731p-10);
    p = fma(f, p, 0x1.3b2ab6fba4e77p-7);
    p = fma(f, p, 0x1.c6b08d704a0c0p-5);
    p = fma(f, p, 0x1.ebfbdff82c58fp-3);
    p = fma(f, p, 0x1.62e42fefa39efp-1);
    p = fma(f, p, 1.0);
    return ldexp(p, static_cast<int>(k));
}

// fp64 statistics of one node row: pi(v) = 2^((l_v - M) cT - ls), cT = log2(e)/T,
// ls = log2 sum_v 2^((l_v - M) cT).  ok = 0 for a row that is not a distribution.
struct RedoStat {
    double ls;
    float M;
    int ok;
};

struct RedoArgs {
    const void *tgt;              // [B][K][L+1][V]
    const void *drf;              // [B][K][L][V]
    const int32_t *tok;           // [B][K][L]
    const float *temp, *ua, *uc;  // [B], [B][K][L], [B]
    const unsigned *count;        // listed requests
    const int32_t *list;          // [count]: their indices (| kListNoReplay)
    const unsigned char *dec;     // [B][K][L] the fast walk's test records, or null
    const double *rho_rec;        // [B][L] the fast SpecTr walk's rho per position, or null
    RedoStat *stats;              // [count][K][2L+1]: node rows of listed request i at i*K*(2L+1)
    int B, K, L, V;
    int method;                   // kMethodToken, kMethodBlockWalk or kMethodSpecTr
    int32_t *accept_len, *draft_index, *correction, *flags;
    float *accept_prob, *resid_mass;
};

// fp64 statistics of one row at temperature T, in one pass: each thread keeps
// a running maximum and rescales its sum when it grows; the block combines them
// (block-uniform call; every thread returns the result).
template <int NT, typename RD>
__device__ RedoStat redo_row_stat(const RD &R, int nch, float T, double *s_red, float *s_fred) {
    const int tid = threadIdx.x;
    const double cT = 1.4426950408889634 / static_cast<double>(T);
    float mx = -INFINITY;
    double sum = 0.0;
    int nan = !(T > 0.0f) || !isfinite(T);
    for (int q0 = tid; q0 < nch; q0 += kRedoDepth * NT) {   // loads issued ahead
        typename RD::Raw raw[kRedoDepth];
#pragma unroll
        for (int d = 0; d < kRedoDepth; ++d)
            if (q0 + d * NT < nch) raw[d] = R.raw(q0 + d * NT);
#pragma unroll
        for (int d = 0; d < kRedoDepth; ++d) {
            if (q0 + d * NT >= nch) break;
            float x[8];
            RD::unpack(raw[d], x);
            float cm = -INFINITY;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                nan |= isnan(x[e]) || x[e] == INFINITY;
                cm = fmaxf(cm, x[e]);
            }
            if (cm > mx) {   // rescale the sum to the new maximum
                if (mx > -INFINITY)
                    sum *= exp2_d((static_cast<double>(mx) - static_cast<double>(cm)) * cT);
                mx = cm;
            }
            if (mx > -INFINITY && !nan) {
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    sum += exp2_d((static_cast<double>(x[e]) - static_cast<double>(mx)) * cT);
            }
        }
    }
    nan = __syncthreads_or(nan);
    const float M = block_max<NT>(mx, s_fred);
    if (mx > -INFINITY && !nan)
        sum *= exp2_d((static_cast<double>(mx) - static_cast<double>(M)) * cT);
    else
        sum = 0.0;
    sum = block_sum<NT>(sum, s_red);
    RedoStat st;
    st.ok = !nan && M > -INFINITY && sum > 0.0 && isfinite(sum);
    st.M = M;
    st.ls = st.ok ? log2(sum) : 0.0;
    return st;
}

// One workgroup per (listed request, node row), grid-stride: the fp64
// statistics of the row when it is the node's own (no earlier draft shares its
// prefix; the walk reads only those).
template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void redo_stats_kernel(RedoArgs A) {
    __shared__ double s_red[NT / kWave];
    __shared__ float s_fred[NT / kWave];
    const unsigned n = *A.count;
    if (n == 0) return;
    const int tid = threadIdx.x;
    const int K = A.K, L = A.L, V = A.V, L1 = L + 1, RS = 2 * L + 1, per = K * RS;
    const int nch = (V + kChunk - 1) / kChunk;
    const long long items = static_cast<long long>(n) * per;
    for (long long it = blockIdx.x; it < items; it += gridDim.x) {
        const int i = static_cast<int>(it / per), r = static_cast<int>(it % per);
        const int k = r / RS, s = r % RS;
        const int b = A.list[i] & ~kListNoReplay;
        const bool target = s <= L;
        const int j = target ? s : s - L1;
        const int32_t *tk = A.tok + static_cast<long long>(b) * K * L;
        int dup = 0;
        for (int c = tid; c < k; c += NT) {
            int same = 1;
            for (int t = 0; t < j; ++t) same &= (tk[c * L + t] == tk[k * L + t]);
            dup |= same;
        }
        if (__syncthreads_or(dup)) continue;   // block-uniform
        const E *base = target
            ? static_cast<const E *>(A.tgt) + ((static_cast<long long>(b) * K + k) * L1 + j) * V
            : static_cast<const E *>(A.drf) + ((static_cast<long long>(b) * K + k) * L + j) * V;
        const RD R(base, V);
        const float T = A.temp[b];
        const RedoStat st = redo_row_stat<NT, RD>(R, nch, T, s_red, s_fred);
        if (tid == 0) A.stats[it] = st;
    }
}

// LDS of one re-evaluation.
struct RedoShared {
    int x[kMaxK * kMaxL];
    unsigned char can[kMaxK * (kMaxL + 1)];
    unsigned char ok[kMaxK * (2 * kMaxL + 1)];
    unsigned char have[kMaxK * (2 * kMaxL + 1)];
    float M[kMaxK * (2 * kMaxL + 1)];
    double ls[kMaxK * (2 * kMaxL + 1)];
    int H[kMaxK];
    unsigned char made[kMaxK * kMaxL];   // tests of the final path (accept_prob entries kept)
    double w[kMaxL + 1], R[kMaxL + 1];   // GBV's weight chain and residual sums
    double red[16];
    float fred[16];
    int ired[16];
    double pair[2];
};

// Re-evaluate request b in fp64 and overwrite its outputs (block-uniform call).
// entry: its list entry (kListNoReplay: no records to replay); st: its node
// rows' fp64 statistics [K][2L+1] from redo_stats_kernel, or null to compute
// each one in this workgroup when the walk first reads it.
template <int NT, typename RD, typename E>
__device__ __attribute__((noinline)) void redo_request(const RedoArgs &A, int b, int entry,
                                                       const RedoStat *st, RedoShared &sh) {
    int *s_x = sh.x;
    unsigned char *s_can = sh.can, *s_ok = sh.ok, *s_have = sh.have;
    float *s_fred = sh.fred;
    float *s_M = sh.M;
    double *s_ls = sh.ls;
    int *s_H = sh.H;
    double *s_red = sh.red, *s_pair = sh.pair;
    int *s_ired = sh.ired;
    const int tid = threadIdx.x;
    const int K = A.K, L = A.L, V = A.V, L1 = L + 1, RS = 2 * L + 1;
    const int nch = (V + kChunk - 1) / kChunk;
    {
        const long long bKL = static_cast<long long>(b) * K * L;
        // exp((l - M) / T) taken as 2^((l - M) log2(e) / T)
        const double cT = 1.4426950408889634 / static_cast<double>(A.temp[b]);
        const E *tgt = static_cast<const E *>(A.tgt);
        const E *drf = static_cast<const E *>(A.drf);
        for (int q = tid; q < K * L; q += NT) s_x[q] = A.tok[bKL + q];
        for (int q = tid; q < K * RS; q += NT) {
            if (st) {
                const RedoStat r = st[q];
                s_ok[q] = static_cast<unsigned char>(r.ok);
                s_M[q] = r.M;
                s_ls[q] = r.ls;
            }
            s_have[q] = st ? 1 : 0;
        }
        __syncthreads();
        // node of (k, j): the lowest-index draft with the same first j tokens
        for (int q = tid; q < K * L1; q += NT) {
            const int k = q / L1, j = q % L1;
            int c = k;
            for (int cc = 0; cc < k; ++cc) {
                int same = 1;
                for (int t = 0; t < j; ++t) same &= (s_x[cc * L + t] == s_x[k * L + t]);
                if (same) { c = cc; break; }
            }
            s_can[q] = static_cast<unsigned char>(c);
        }
        __syncthreads();
        auto row = [&](bool target, int c, int j) {
            return target ? RD(tgt + ((static_cast<long long>(b) * K + c) * L1 + j) * V, V)
                          : RD(drf + ((static_cast<long long>(b) * K + c) * L + j) * V, V);
        };
        auto slot = [&](bool target, int c, int j) { return c * RS + (target ? j : L1 + j); };
        int bad = 0;
        // node row (target?, node of (k, j)): its slot, its statistics computed
        // here when not given; an invalid row marks the request
        auto stats = [&](bool target, int k, int j) {
            const int c = s_can[k * L1 + j];
            const int sl = slot(target, c, j);
            if (!s_have[sl]) {
                const RedoStat r = redo_row_stat<NT, RD>(row(target, c, j), nch, A.temp[b], s_red,
                                                        s_fred);
                if (tid == 0) {
                    s_ok[sl] = static_cast<unsigned char>(r.ok);
                    s_M[sl] = r.M;
                    s_ls[sl] = r.ls;
                    s_have[sl] = 1;
                }
                __syncthreads();
            }
            bad |= !s_ok[sl];
            return sl;
        };
        auto prob = [&](int sl, float x) {
            return exp2_d(fma(static_cast<double>(x) - static_cast<double>(s_M[sl]), cT, -s_ls[sl]));
        };
        auto prob_at = [&](bool target, int k, int j, int x) {
            const int sl = stats(target, k, j);
            const int c = s_can[k * L1 + j];
            return prob(sl, row(target, c, j).at(x));
        };
        // block-wide sum of f(v, p(v), q(v)) over node (k, j)'s row pair
        auto sweep = [&](int k, int j, auto f) {
            const int c = s_can[k * L1 + j];
            const int sp = stats(true, k, j), sq = stats(false, k, j);
            const RD P = row(true, c, j), Q = row(false, c, j);
            double acc = 0.0;
            for (int q0 = tid; q0 < nch; q0 += 2 * NT) {   // loads issued ahead
                typename RD::Raw rp[2], rq[2];
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    if (q0 + d * NT < nch) {
                        rp[d] = P.raw(q0 + d * NT);
                        rq[d] = Q.raw(q0 + d * NT);
                    }
                }
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const int q = q0 + d * NT;
                    if (q >= nch) break;
                    float xp[8], xq[8];
                    RD::unpack(rp[d], xp);
                    RD::unpack(rq[d], xq);
                    // no test v < V: elements past the row read as -inf, so p = q = 0
                    // there and every weight below is 0
#pragma unroll
                    for (int e = 0; e < 8; ++e) acc += f(kChunk * q + e, prob(sp, xp[e]), prob(sq, xq[e]));
                }
            }
            return block_sum<NT>(acc, s_red);
        };
        // inverse-CDF draw in token-id order over weights w(v, p, q) of node (k, j)
        // (q = 0 when only the target row is involved): y = min{v : C_v > u Z};
        // the last v of positive weight when rounding leaves none.  Returns -1
        // when Z is not a positive finite number; *Z and *margin (distance of u Z
        // to the nearest boundary, over Z) are set.
        auto icdf = [&](int k, int j, bool with_q, auto w, double u, double *Z, double *margin) {
            const int c = s_can[k * L1 + j];
            const int sp = stats(true, k, j);
            const int sq = with_q ? stats(false, k, j) : sp;
            const RD P = row(true, c, j), Q = row(false, c, j);
            const int per = (nch + NT - 1) / NT;   // contiguous chunks per thread
            const int q0 = tid * per, q1 = min(q0 + per, nch);
            // (elements past the row read as -inf: weight 0)
            auto weight = [&](int q, int e, const float *xp, const float *xq) {
                return w(kChunk * q + e, prob(sp, xp[e]), with_q ? prob(sq, xq[e]) : 0.0);
            };
            double mine = 0.0;
            int lastpos = -1;
            for (int qb = q0; qb < q1; qb += 2) {   // loads issued ahead
                typename RD::Raw rp[2], rq[2];
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    if (qb + d < q1) {
                        rp[d] = P.raw(qb + d);
                        if (with_q) rq[d] = Q.raw(qb + d);
                    }
                }
#pragma unroll
                for (int d = 0; d < 2; ++d) {
                    const int q = qb + d;
                    if (q >= q1) break;
                    float xp[8], xq[8];
                    RD::unpack(rp[d], xp);
                    if (with_q) RD::unpack(rq[d], xq);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const double wv = weight(q, e, xp, xq);
                        mine += wv;
                        lastpos = wv > 0.0 ? kChunk * q + e : lastpos;
                    }
                }
            }
            const double pre = block_exclusive_scan<NT>(mine, s_red);
            const double z = block_sum<NT>(mine, s_red);
            *Z = z;
            *margin = 0.0;
            if (!(z > 0.0) || !isfinite(z)) return -1;
            const double thr = u * z;
            const int last = block_max_int<NT>(lastpos, s_ired);
            // the first thread whose range ends past u Z holds the crossing
            const int owner = block_min_int<NT>(pre + mine > thr ? tid : 0x7fffffff, s_ired);
            if (owner == 0x7fffffff) return last;   // rounding: no C_v exceeds u Z
            if (tid == owner) s_pair[1] = pre;
            __syncthreads();
            const double base = s_pair[1];
            // the owner's elements, recounted by the whole block in token order:
            // consecutive runs per thread, a block scan, then the run that
            // crosses u Z element by element
            const int e0 = kChunk * owner * per, e1 = min(e0 + kChunk * per, V);
            const int cnt = e1 > e0 ? (e1 - e0 + NT - 1) / NT : 0;
            const int a0 = min(e0 + tid * cnt, e1), a1 = min(a0 + cnt, e1);
            auto wat = [&](int v) {
                return w(v, prob(sp, P.at(v)), with_q ? prob(sq, Q.at(v)) : 0.0);
            };
            double part = 0.0;
            int lastrun = -1;
            for (int v = a0; v < a1; ++v) {
                const double wv = wat(v);
                part += wv;
                lastrun = wv > 0.0 ? v : lastrun;
            }
            const double pre2 = base + block_exclusive_scan<NT>(part, s_red);
            int cand = 0x7fffffff;
            double cm = 0.0;
            if (pre2 + part > thr) {
                double C = pre2;
                for (int v = a0; v < a1; ++v) {
                    const double before = C;
                    C += wat(v);
                    if (C > thr) {
                        cand = v;
                        cm = fmin(C - thr, thr - before);
                        break;
                    }
                }
            }
            const int got = cand;
            cand = block_min_int<NT>(cand, s_ired);
            if (cand != 0x7fffffff) {
                if (got == cand) s_pair[0] = cm;
                __syncthreads();
                *margin = s_pair[0] / z;
                __syncthreads();
                return cand;
            }
            // the recount's rounding left u Z past the owner's elements (a tie
            // at the level of double rounding): its last element of weight
            lastrun = block_max_int<NT>(lastrun, s_ired);
            return lastrun >= 0 ? lastrun : last;
        };
        auto same_prefix = [&](int a, int c, int n) {
            int same = 1;
            for (int t = 0; t < n; ++t) same &= (s_x[a * L + t] == s_x[c * L + t]);
            return same;
        };
        auto ratio = [](double num, double den) {   // a drafted token with q = 0
            return den > 0.0 ? num / den : (num > 0.0 ? INFINITY : 0.0);
        };
        auto chain = [&](double w, double num, double den) {
            if (w == 0.0) return 0.0;
            const double t = w * ratio(num, den);
            return t < 1.0 ? t : 1.0;
        };

        // accept_prob: every test of the final path is written (or, replayed
        // from the fast walk, kept); the others are set to NaN at the end
        float *hout = A.accept_prob ? A.accept_prob + bKL : nullptr;
        unsigned char *s_made = sh.made;
        for (int q = tid; q < K * L; q += NT) s_made[q] = 0;
        __syncthreads();
        const float *ub = A.ua + bKL;
        double tie = INFINITY;
        int flags = 0;
        auto test = [&](int k, int m, double h) {   // u < h for position m of draft k
            const double u = static_cast<double>(ub[k * L + m - 1]);
            if (tid == 0 && hout) hout[k * L + m - 1] = static_cast<float>(h);
            s_made[k * L + m - 1] = 1;
            tie = fmin(tie, fabs(u - h));
            return u < h;
        };
        const double uc = static_cast<double>(A.uc[b]);
        int tau = 0, kstar = -1, y = -1, own = 0;
        double Z = NAN, dm = INFINITY;
        auto draw_target = [&](int k, int j) {   // the node's target row itself
            return icdf(k, j, false, [](int, double p, double) { return p; }, uc, &Z, &dm);
        };

        if (A.method == kMethodToken) {
            tau = L;
            for (int j = 0; j < L && !bad; ++j) {
                const int x = s_x[j];
                const double p = prob_at(true, 0, j, x), q = prob_at(false, 0, j, x);
                double a = ratio(p, q);
                if (a > 1.0) a = 1.0;
                if (!test(0, j + 1, a)) { tau = j; break; }
            }
            kstar = tau > 0 ? 0 : -1;
            if (!bad) {
                if (tau == L) {
                    y = draw_target(0, L);
                } else {
                    y = icdf(0, tau, true, [](int, double p, double q) { return fmax(p - q, 0.0); },
                             uc, &Z, &dm);
                    if (y < 0) {
                        flags |= kFlagDegenerate;
                        y = draw_target(0, tau);
                    }
                }
            }
        } else if (A.method == kMethodSpecTr) {
            // SpecTr: rho* = the smallest rho in [1, n] with c(beta(rho)) <= rho; the
            // feasibility test is taken in the form rounding cannot flip (quotient
            // form for beta <= 2^-10).  While every decision agrees with the fast
            // walk's records, a position whose tests were all certain and where a
            // candidate was accepted needs no rho*; elsewhere rho* is bracketed
            // around the fast walk's rho (within 7.4e-7 of rho*) and narrowed by
            // safeguarded secant steps on rho - c(beta(rho)) to 2^-42 relative.
            const double *rrec = A.rho_rec ? A.rho_rec + static_cast<long long>(b) * L : nullptr;
            bool follow = A.dec != nullptr && rrec != nullptr && !(entry & kListNoReplay);
            int kacc = -1;
            bool done = false;
            for (int j = 0; j < L && !bad && !done; ++j) {
                stats(true, own, j);
                stats(false, own, j);
                if (bad) break;
                int n = 0;
                for (int k = 0; k < K; ++k) n += same_prefix(k, own, j);
                auto c_of = [&](double beta) {
                    double cc = 0.0, t = 1.0;
                    for (int i = 0; i < n; ++i) { cc += t; t *= 1.0 - beta; }
                    return cc;
                };
                // beta(rho) = sum min(q, p/rho) and D(rho) = sum max(p - rho q, 0), one sweep
                auto sums = [&](double rho, double &beta, double &D) {
                    const int c = s_can[own * L1 + j];
                    const int sp = stats(true, own, j), sq = stats(false, own, j);
                    const RD P = row(true, c, j), Q = row(false, c, j);
                    const double ir = 1.0 / rho;
                    double v[2] = {0.0, 0.0};
                    for (int q0 = tid; q0 < nch; q0 += 2 * NT) {
                        typename RD::Raw rp[2], rq[2];
#pragma unroll
                        for (int d = 0; d < 2; ++d) {
                            if (q0 + d * NT < nch) {
                                rp[d] = P.raw(q0 + d * NT);
                                rq[d] = Q.raw(q0 + d * NT);
                            }
                        }
#pragma unroll
                        for (int d = 0; d < 2; ++d) {
                            if (q0 + d * NT >= nch) break;
                            float xp[8], xq[8];
                            RD::unpack(rp[d], xp);
                            RD::unpack(rq[d], xq);
#pragma unroll
                            for (int e = 0; e < 8; ++e) {
                                const double pp = prob(sp, xp[e]), qq = prob(sq, xq[e]);
                                v[0] += fmin(qq, pp * ir);
                                v[1] += fmax(pp - rho * qq, 0.0);
                            }
                        }
                    }
                    block_sum_n<NT, 2>(v, s_red);
                    beta = v[0];
                    D = v[1];
                };
                auto feasible = [&](double rho, double *g, double *bt) {
                    double beta, D;
                    sums(rho, beta, D);
                    const double cc = c_of(beta);
                    *g = rho - cc;
                    *bt = beta;
                    if (beta <= kQuotientFormBeta) return cc <= rho;
                    double xn = 1.0;
                    for (int i = 0; i < n; ++i) xn *= 1.0 - beta;
                    return D <= xn;
                };
                // the fast walk's records at this position: all certain, and accepted?
                bool replay = follow && n > 1;
                int rec_acc = -1;
                if (replay) {
                    for (int k = 0; k < K && rec_acc < 0 && replay; ++k) {
                        if (!same_prefix(k, own, j)) continue;
                        const int dc = A.dec[bKL + k * L + j];
                        if (!(dc & kDecMade) || !(dc & kDecCertain)) replay = false;
                        else if (dc & kDecAccept) rec_acc = k;
                    }
                    if (rec_acc < 0) replay = false;   // the draw is here: it needs rho*
                }
                if (replay) {
                    for (int k = 0; k <= rec_acc; ++k)
                        if (same_prefix(k, own, j)) s_made[k * L + j] = 1;
                    own = rec_acc;
                    kacc = rec_acc;
                    continue;
                }
                // rho* and beta(rho*) (NAN: not swept at rho*)
                double rho = 1.0, beta_rho = NAN;
                double g, bt;
                // the fast rho is within 7.4e-7 of rho*: one this far above 1 puts rho*
                // above 1 without a sweep at 1
                const double rf = follow ? rrec[j] : 0.0;
                const bool above1 = rf > 1.0 + 8e-6;
                bool at1 = false;
                if (n > 1 && !above1) {
                    at1 = feasible(1.0, &g, &bt);
                    if (at1) beta_rho = bt;
                }
                if (n > 1 && !at1) {
                    double lo = 1.0, hi = static_cast<double>(n);   // c <= n: n is feasible
                    double glo = above1 ? NAN : g, ghi = NAN, bhi = NAN;
                    int keep = 0;   // Illinois: the end retained on the last steps
                    if (rf > lo && rf < hi) {
                        const double t0 = fmax(rf * (1.0 - 4e-6), lo), t1 = fmin(rf * (1.0 + 4e-6), hi);
                        if (t0 > lo) {
                            if (feasible(t0, &g, &bt)) { hi = t0; ghi = g; bhi = bt; }
                            else { lo = t0; glo = g; }
                        }
                        if (t1 < hi && t1 > lo) {
                            if (feasible(t1, &g, &bt)) { hi = t1; ghi = g; bhi = bt; }
                            else { lo = t1; glo = g; }
                        }
                    }
                    for (int it = 0; it < 200 && hi - lo > 0x1p-42 * hi; ++it) {
                        double t = 0.5 * (lo + hi);
                        if (isfinite(ghi) && isfinite(glo) && ghi > glo) {
                            const double sec = lo - glo * (hi - lo) / (ghi - glo);
                            const double w = hi - lo;
                            if (sec > lo + 1e-3 * w && sec < hi - 1e-3 * w) t = sec;
                        }
                        if (!(t > lo && t < hi)) break;
                        if (feasible(t, &g, &bt)) {
                            hi = t;
                            ghi = g;
                            bhi = bt;
                            if (keep == -1) glo *= 0.5;
                            keep = -1;
                        } else {
                            lo = t;
                            glo = g;
                            if (keep == 1) ghi *= 0.5;
                            keep = 1;
                        }
                    }
                    rho = hi;
                    beta_rho = bhi;
                }
                int acc = -1;
                for (int k = 0; k < K && acc < 0; ++k) {
                    if (!same_prefix(k, own, j)) continue;
                    const int x = s_x[k * L + j];
                    const double p = prob_at(true, own, j, x), q = prob_at(false, own, j, x);
                    double a = ratio(p, rho * q);
                    if (a > 1.0) a = 1.0;
                    const bool ak = test(k, j + 1, a);
                    if (follow && n > 1) {
                        const int dc = A.dec[bKL + k * L + j];
                        if (!(dc & kDecMade) || ak != ((dc & kDecAccept) != 0)) follow = false;
                    }
                    if (ak) acc = k;
                }
                if (acc < 0) {
                    double beta = beta_rho, D;
                    if (!isfinite(beta)) sums(rho, beta, D);
                    const double cc = c_of(beta);
                    y = icdf(own, j, true, [&](int, double p, double q) {
                        return fmax(p - cc * fmin(q, p / rho), 0.0);
                    }, uc, &Z, &dm);
                    if (y < 0) {
                        flags |= kFlagDegenerate;
                        y = draw_target(own, j);
                    }
                    tau = j;
                    kstar = kacc;
                    done = true;
                } else {
                    own = acc;
                    kacc = acc;
                }
            }
            if (!bad && !done) {
                tau = L;
                kstar = kacc;
                y = draw_target(own, L);
            }
        } else {
            // GBV over K drafts: residual omega(v) = [v not in H] max(alpha p_s - beta q_s, 0)
            double alpha = 1.0, beta = 0.0, N = 1.0;
            int nH = 0;
            double *w = sh.w, *R = sh.R;   // weight chain, residual sums (LDS: no scratch)
            auto in_H = [&](int v) {   // branch-free: nH is the same for every thread
                bool r = false;
                for (int i = 0; i < nH; ++i) r |= (s_H[i] == v);
                return r;
            };
            auto node_mass = [&]() {
                return sweep(own, tau, [&](int v, double p, double q) {
                    return in_H(v) ? 0.0 : fmax(alpha * p - beta * q, 0.0);
                });
            };
            // While every decision so far agrees with the fast walk's, the walks
            // are in the same state, and a test the fast walk recorded as certain
            // is taken from its record without R_m (R_m is still summed where the
            // test accepts: it is the next node's mass).
            bool follow = A.dec != nullptr && !(entry & kListNoReplay);
            for (int k = 0; k < K && tau < L && !bad; ++k) {
                if (!same_prefix(k, own, tau)) continue;
                const int x = s_x[k * L + tau];
                if (in_H(x)) {
                    beta += N;
                    N = node_mass();
                } else {
                    // first position: the node residual omega / N against q_s
                    const double ps = prob_at(true, own, tau, x), qs = prob_at(false, own, tau, x);
                    const double om = fmax(alpha * ps - beta * qs, 0.0);
                    w[tau + 1] = chain(1.0, om / N, qs);
                    for (int j = tau + 1; j < L; ++j) {
                        const int xj = s_x[k * L + j];
                        w[j + 1] = chain(w[j], prob_at(true, k, j, xj), prob_at(false, k, j, xj));
                    }
                    if (bad) break;
                    int acc = 0;
                    for (int m = L; m > tau; --m) {
                        const int dc = follow ? A.dec[bKL + k * L + m - 1] : 0;
                        if (follow && !(dc & kDecMade)) follow = false;
                        if (follow && (dc & kDecCertain)) {
                            s_made[k * L + m - 1] = 1;
                            if (!(dc & kDecAccept)) continue;
                            if (m < L) {
                                const double wm = w[m];
                                R[m] = sweep(k, m, [&](int, double p, double q) {
                                    return fmax(wm * p - q, 0.0);
                                });
                                if (bad) break;
                            }
                            acc = m;
                            break;
                        }
                        double h;
                        if (m == L) {
                            h = w[L];
                        } else {
                            const double wm = w[m];
                            const double u = static_cast<double>(ub[k * L + m - 1]);
                            // h_m <= w_m: a uniform that far above w_m rejects without
                            // R_m (its margin exceeds the near-tie band either way)
                            if (u >= wm + kNearTie) {
                                tie = fmin(tie, u - wm);
                                if (tid == 0 && hout) hout[k * L + m - 1] = NAN;
                                s_made[k * L + m - 1] = 1;
                                if (dc & kDecAccept) follow = false;
                                continue;
                            }
                            R[m] = sweep(k, m, [&](int, double p, double q) {
                                return fmax(wm * p - q, 0.0);
                            });
                            if (bad) break;
                            const double d = R[m] + 1.0 - wm;
                            h = d > 0.0 ? R[m] / d : 1.0;
                        }
                        const bool a_m = test(k, m, h);
                        if (a_m != ((dc & kDecAccept) != 0)) follow = false;
                        if (a_m) { acc = m; break; }
                    }
                    if (bad) break;
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
                        if (tid == 0) s_H[nH] = x;
                        __syncthreads();
                        ++nH;
                        beta += N;
                        N = node_mass();
                    }
                }
                if (tau < L && !(N > 0.0)) {   // only rounding empties a residual
                    flags |= kFlagDegenerate;
                    alpha = 1.0;
                    beta = 0.0;
                    N = 1.0;
                    nH = 0;
                    follow = false;
                }
            }
            if (!bad) {
                if (tau == L) {
                    y = draw_target(own, L);
                } else {
                    y = icdf(own, tau, true, [&](int v, double p, double q) {
                        return in_H(v) ? 0.0 : fmax(alpha * p - beta * q, 0.0);
                    }, uc, &Z, &dm);
                    if (y < 0) {
                        flags |= kFlagDegenerate;
                        y = draw_target(own, tau);
                    }
                }
            }
        }
        if (!bad && y < 0) bad = 1;
        tie = fmin(tie, dm);
        if (tie < kNearTie) flags |= kFlagNearTie;
        if (tid == 0) {
            if (bad) {
                tau = -1;
                kstar = -1;
                y = -1;
                flags = kFlagInvalid;
                Z = NAN;
            }
            A.accept_len[b] = tau;
            A.draft_index[b] = kstar;
            A.correction[b] = y;
            if (A.flags) A.flags[b] = flags | kFlagRedone;
            if (A.resid_mass) A.resid_mass[b] = static_cast<float>(Z);
        }
        __syncthreads();
        if (hout)
            for (int q = tid; q < K * L; q += NT)
                if (bad || !s_made[q]) hout[q] = NAN;
        __syncthreads();
    }
}

// One workgroup per listed request, grid-stride.
template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void redo_walk_kernel(RedoArgs A) {
    __shared__ RedoShared sh;
    const unsigned n = *A.count;
    if (n == 0) return;
    for (unsigned i = blockIdx.x; i < n; i += gridDim.x) {   // block-uniform
        const int entry = A.list[i];
        redo_request<NT, RD, E>(A, entry & ~kListNoReplay, entry,
                                A.stats + static_cast<long long>(i) * A.K * (2 * A.L + 1), sh);
    }
}

}  // namespace sv
