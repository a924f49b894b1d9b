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
// ls = log2 sum_v 2^((l_v - M) cT).  ok = 0 for a row that is not a distribution;
// kRedoStatAbsent for a row the statistics launch left out (computed by the
// re-walk if it reads the row).
struct RedoStat {
    double ls;
    float M;
    int ok;
};
constexpr int kRedoStatAbsent = 2;

// Teams.  When few requests are listed, each gets a team of workgroups that
// share its O(V) passes: the team's first workgroup runs the re-evaluation and,
// for each pass, publishes a command (the node, the weight, its parameters);
// every member sums the weights over its own contiguous range of the row's
// chunks and publishes the partial sums, which the first workgroup adds in
// member order (the same order whichever workgroup computed a range, so the
// result does not depend on timing).  No wait is unbounded: a member that has
// not answered within kTeamWaitTicks is computed by the first workgroup itself
// (the team then works alone), and a member that has seen no command for
// kTeamIdleTicks leaves.  Commands and partials go through device memory with
// agent-scope release and acquire (relaxed polls).
constexpr int kTeamMax = 32;                  // workgroups per team
constexpr int kTeamDepth = 4;                 // chunks per thread in flight in a member's range
constexpr int kTeamDone = 0x7fffffff;         // command number that ends a team
constexpr long long kTeamWaitTicks = 20000;   // 200 us of the 100 MHz real-time counter
                                              // (the default of RedoArgs::team_wait)
constexpr long long kTeamIdleTicks = 200000;  // 2 ms
constexpr int kTeamRes = 0;    // [v not in H] max(a p - bq q, 0)   (q = 0 without the draft row)
constexpr int kTeamSRes = 1;   // max(p - cc min(q, p / rho), 0)    (SpecTr residual)
constexpr int kTeamSSums = 2;  // min(q, p / rho) and max(p - rho q, 0), two sums

struct TeamBody {       // one pass: its node, weight and parameters
    int kind, c, j, with_q, nH;
    int H[kMaxK];
    float Mp, Mq;       // node rows' fp64 statistics (see RedoStat)
    double lsp, lsq;
    double a, bq, cc, rho;
};

struct TeamCmd {
    int seq;            // command number (0: none yet; kTeamDone: the team is finished)
    int acks;           // partials published by the members, over all commands
    TeamBody body;
};

struct TeamPart {
    double s[2];        // partial sums over the member's range
    int last;           // last token of positive weight in it (-1: none)
    int seq;            // the command they answer
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
    TeamCmd *team_cmd;            // [kRedoTeamSlots]: one per team
    TeamPart *team_part;          // [kRedoTeamSlots]: team t's members at t*T ..
    long long team_wait;          // ticks the first workgroup waits for its members'
                                  // answers to a command before summing their ranges itself
};

// Slots of the team areas (the re-evaluation launch's grid bound).
constexpr int kRedoTeamSlots = 256;

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
    // the team areas start clean for this call's re-evaluation launch
    for (int i = blockIdx.x * NT + tid; i < kRedoTeamSlots; i += gridDim.x * NT) {
        A.team_cmd[i].seq = 0;
        A.team_cmd[i].acks = 0;
        A.team_part[i].seq = 0;
    }
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
        // a row left out is marked absent, never left with another call's bytes
        auto absent = [&]() {
            if (tid == 0) {
                RedoStat st;
                st.ls = 0.0;
                st.M = 0.0f;
                st.ok = kRedoStatAbsent;
                A.stats[it] = st;
            }
        };
        if (__syncthreads_or(dup)) {   // block-uniform
            absent();
            continue;
        }
        // Only rows of drafts the fast walk tested (a draft sharing the row's
        // prefix [0, j) that has a test record): while the fp64 walk agrees with
        // the records those are the rows it reads; one it reaches after a
        // disagreement is marked absent and computed by the re-walk itself when
        // first read.
        if (A.dec && !(A.list[i] & kListNoReplay)) {
            const unsigned char *dk = A.dec + static_cast<long long>(b) * K * L;
            int used = 0;
            for (int c = k + tid; c < K; c += NT) {
                int same = 1;
                for (int t = 0; t < j; ++t) same &= (tk[c * L + t] == tk[k * L + t]);
                for (int m = 0; m < L && same; ++m) used |= (dk[c * L + m] & kDecMade) != 0;
            }
            if (!__syncthreads_or(used)) {   // block-uniform
                absent();
                continue;
            }
        }
        const E *base = target
            ? static_cast<const E *>(A.tgt) + ((static_cast<long long>(b) * K + k) * L1 + j) * V
            : static_cast<const E *>(A.drf) + ((static_cast<long long>(b) * K + k) * L + j) * V;
        const RD R(base, V);
        const float T = A.temp[b];
        const RedoStat st = redo_row_stat<NT, RD>(R, nch, T, s_red, s_fred);
        if (tid == 0) A.stats[it] = st;
    }
}

// Weight of token v (probabilities p, q) under a team command.
__device__ __forceinline__ double team_weight(const TeamBody &d, int v, double p, double q) {
    if (d.kind == kTeamSRes) return fmax(p - d.cc * fmin(q, p / d.rho), 0.0);
    bool inH = false;   // branch-free: nH is the same for every thread
    for (int i = 0; i < d.nH; ++i) inH |= (d.H[i] == v);
    return inH ? 0.0 : fmax(d.a * p - d.bq * q, 0.0);
}

// A team command's sums over chunks [q0, q1) of its node's rows (block-uniform;
// every thread returns them): out[0] (and for kTeamSSums out[1]); *last the last
// token of positive weight (-1: none).  Chunks are strided by the block, the
// order of the single-workgroup sweep, with up to kTeamDepth per thread in
// flight (a range of a 16th of a 151 936-token row, or less, in one round).
template <int NT, typename RD, typename E>
__device__ void team_slice(const RedoArgs &A, int b, const TeamBody &d, int q0, int q1,
                           double out[2], int *last, double *s_red, int *s_ired) {
    const int tid = threadIdx.x;
    const int K = A.K, L = A.L, V = A.V, L1 = L + 1;
    const double cT = 1.4426950408889634 / static_cast<double>(A.temp[b]);
    const RD P(static_cast<const E *>(A.tgt) + ((static_cast<long long>(b) * K + d.c) * L1 + d.j) * V,
               V);
    const RD Q(static_cast<const E *>(A.drf) +
                   ((static_cast<long long>(b) * K + d.c) * L + (d.with_q ? d.j : 0)) * V,
               V);
    const double Mp = d.Mp, Mq = d.Mq, lsp = d.lsp, lsq = d.lsq;
    const bool sums = d.kind == kTeamSSums;
    const double ir = sums ? 1.0 / d.rho : 0.0;
    double v0 = 0.0, v1 = 0.0;
    int lp = -1;
    for (int qa = q0 + tid; qa < q1; qa += kTeamDepth * NT) {   // loads issued ahead
        typename RD::Raw rp[kTeamDepth], rq[kTeamDepth];
#pragma unroll
        for (int e2 = 0; e2 < kTeamDepth; ++e2) {
            if (qa + e2 * NT < q1) {
                rp[e2] = P.raw(qa + e2 * NT);
                if (d.with_q) rq[e2] = Q.raw(qa + e2 * NT);
            }
        }
#pragma unroll
        for (int e2 = 0; e2 < kTeamDepth; ++e2) {
            const int q = qa + e2 * NT;
            if (q >= q1) break;
            float xp[8], xq[8];
            RD::unpack(rp[e2], xp);
            if (d.with_q) RD::unpack(rq[e2], xq);
            // elements past the row read as -inf: p = q = 0, weight 0
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const double p = exp2_d(fma(static_cast<double>(xp[e]) - static_cast<double>(Mp), cT, -lsp));
                const double qq =
                    d.with_q ? exp2_d(fma(static_cast<double>(xq[e]) - static_cast<double>(Mq), cT, -lsq))
                             : 0.0;
                if (sums) {
                    v0 += fmin(qq, p * ir);
                    v1 += fmax(p - d.rho * qq, 0.0);
                } else {
                    const double w = team_weight(d, kChunk * q + e, p, qq);
                    v0 += w;
                    lp = w > 0.0 ? kChunk * q + e : lp;
                }
            }
        }
    }
    out[0] = block_sum<NT>(v0, s_red);
    out[1] = sums ? block_sum<NT>(v1, s_red) : 0.0;
    *last = sums ? -1 : block_max_int<NT>(lp, s_ired);
}

// Chunk range of team member m of T over nch chunks.
__device__ __forceinline__ int team_lo(int m, int T, int nch) {
    return static_cast<int>(static_cast<long long>(nch) * m / T);
}

// A member (not the first) of request b's team: sums its range of every
// command until the team is finished or no command comes for kTeamIdleTicks.
template <int NT, typename RD, typename E>
__device__ void team_member(const RedoArgs &A, int b, int team, int m, int T, TeamBody &cmd,
                            double *s_red, int *s_ired, int *s_seq) {
    const int tid = threadIdx.x;
    const int nch = (A.V + kChunk - 1) / kChunk;
    TeamCmd *gc = A.team_cmd + team;
    TeamPart *gp = A.team_part + team * T + m;
    int seen = 0;
    while (true) {
        if (tid == 0) {
            const long long t0 = static_cast<long long>(__builtin_amdgcn_s_memrealtime());
            int got = -1;
            // relaxed polls (an acquire would drop this XCD's L2 at every poll), one
            // acquire fence once the number moved
            while (true) {
                const int sq = __hip_atomic_load(&gc->seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                if (sq != seen) { got = sq; break; }
                if (static_cast<long long>(__builtin_amdgcn_s_memrealtime()) - t0 > kTeamIdleTicks) break;
                __builtin_amdgcn_s_sleep(2);
            }
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
            if (got > 0 && got != kTeamDone) cmd = gc->body;
            *s_seq = got;
        }
        __syncthreads();
        const int sq = *s_seq;
        if (sq <= 0 || sq == kTeamDone) return;   // block-uniform
        double out[2];
        int last;
        team_slice<NT, RD, E>(A, b, cmd, team_lo(m, T, nch), team_lo(m + 1, T, nch), out, &last, s_red,
                              s_ired);
        if (tid == 0) {
            gp->s[0] = out[0];
            gp->s[1] = out[1];
            gp->last = last;
            __hip_atomic_store(&gp->seq, sq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_add(&gc->acks, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        seen = sq;
        __syncthreads();
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
    float gp[kMaxK * kMaxL], gq[kMaxK * kMaxL];   // drafted tokens' logits in their nodes' rows
    unsigned char dec[kMaxK * kMaxL];    // the fast walk's test records
    double w[kMaxL + 1], R[kMaxL + 1];   // GBV's weight chain and residual sums
    double red[16];
    float fred[16];
    int ired[16];
    double pair[2];
    TeamBody cmd;                         // the command being run (team of more than one)
    double tp[2][kTeamMax];               // members' partial sums, in member order
    int tlast[kTeamMax], tgot[kTeamMax];
    int tseq;
};

// Re-evaluate request b in fp64 and overwrite its outputs (block-uniform call).
// entry: its list entry (kListNoReplay: no records to replay); st: its node
// rows' fp64 statistics [K][2L+1] from redo_stats_kernel, or null to compute
// each one in this workgroup when the walk first reads it.  team, T: the
// request's team (T = 1: this workgroup alone); this workgroup is its first.
template <int NT, typename RD, typename E>
__device__ __attribute__((noinline)) void redo_request(const RedoArgs &A, int b, int entry,
                                                       const RedoStat *st, RedoShared &sh, int team,
                                                       int T) {
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
            int have = 0;
            if (st) {
                const RedoStat r = st[q];
                have = r.ok != kRedoStatAbsent;
                s_ok[q] = static_cast<unsigned char>(r.ok);
                s_M[q] = r.M;
                s_ls[q] = r.ls;
            }
            s_have[q] = static_cast<unsigned char>(have);
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
        // every drafted token's logit in its node's target and draft rows, and
        // the fast walk's test records, in one round of loads (the walk below
        // reads them one position at a time)
        for (int q = tid; q < K * L; q += NT) {
            const int k = q / L, j = q % L, x = s_x[q];
            float gp = NAN, gq = NAN;
            if (x >= 0 && x < V) {
                const int c = s_can[k * L1 + j];
                gp = row(true, c, j).at(x);
                gq = row(false, c, j).at(x);
            }
            sh.gp[q] = gp;
            sh.gq[q] = gq;
            sh.dec[q] = A.dec ? A.dec[bKL + q] : 0;
        }
        __syncthreads();
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
        // p or q of draft k's token at position j, in the row of its node (k, j)
        auto prob_tok = [&](bool target, int k, int j) {
            const int sl = stats(target, k, j);
            return prob(sl, target ? sh.gp[k * L + j] : sh.gq[k * L + j]);
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
        // ---- team passes (T > 1): the command in sh.cmd over the members' ranges
        int tseq = 0;        // commands published so far
        bool solo = false;   // a member failed to answer: every range is summed here
        auto team_run = [&]() {
            TeamCmd *gc = A.team_cmd + team;
            if (!solo) {
                ++tseq;
                if (tid == 0) {
                    gc->body = sh.cmd;
                    __hip_atomic_store(&gc->seq, tseq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
            double o[2];
            int lst;
            team_slice<NT, RD, E>(A, b, sh.cmd, team_lo(0, T, nch), team_lo(1, T, nch), o, &lst, s_red,
                                  s_ired);
            if (tid == 0) {
                sh.tp[0][0] = o[0];
                sh.tp[1][0] = o[1];
                sh.tlast[0] = lst;
                // every member's partial of this command counted (or the wait is over)
                if (!solo) {
                    const int want = tseq * (T - 1);
                    const long long t0 = static_cast<long long>(__builtin_amdgcn_s_memrealtime());
                    while (__hip_atomic_load(&gc->acks, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < want &&
                           static_cast<long long>(__builtin_amdgcn_s_memrealtime()) - t0 <= A.team_wait)
                        __builtin_amdgcn_s_sleep(1);
                }
            }
            __syncthreads();
            // the members' partials, one thread each: a partial counts only if it
            // answers this command (its number, published by a release after the
            // sums, read here before an acquire fence)
            if (tid > 0 && tid < T) {
                int got = 0;
                if (!solo) {
                    const TeamPart *gp = A.team_part + team * T + tid;
                    const int q = __hip_atomic_load(&gp->seq, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                    if (q == tseq) {
                        sh.tp[0][tid] = gp->s[0];
                        sh.tp[1][tid] = gp->s[1];
                        sh.tlast[tid] = gp->last;
                        got = 1;
                    }
                }
                sh.tgot[tid] = got;
            }
            __syncthreads();
            for (int m = 1; m < T; ++m) {   // block-uniform: ranges no member answered
                if (sh.tgot[m]) continue;
                team_slice<NT, RD, E>(A, b, sh.cmd, team_lo(m, T, nch), team_lo(m + 1, T, nch), o, &lst,
                                      s_red, s_ired);
                if (tid == 0) {
                    sh.tp[0][m] = o[0];
                    sh.tp[1][m] = o[1];
                    sh.tlast[m] = lst;
                }
                solo = true;
            }
            __syncthreads();
        };
        // the command for node (k, j): kind, parameters, the node rows' statistics
        auto team_cmd = [&](int k, int j, int kind, int with_q, double a, double bq, double cc,
                            double rho, int nh) {
            const int sp = stats(true, k, j);
            const int sq = with_q ? stats(false, k, j) : sp;
            if (tid == 0) {
                sh.cmd.kind = kind;
                sh.cmd.c = s_can[k * L1 + j];
                sh.cmd.j = j;
                sh.cmd.with_q = with_q;
                sh.cmd.nH = nh;
                for (int i = 0; i < nh; ++i) sh.cmd.H[i] = s_H[i];
                sh.cmd.Mp = s_M[sp];
                sh.cmd.lsp = s_ls[sp];
                sh.cmd.Mq = s_M[sq];
                sh.cmd.lsq = s_ls[sq];
                sh.cmd.a = a;
                sh.cmd.bq = bq;
                sh.cmd.cc = cc;
                sh.cmd.rho = rho;
            }
            __syncthreads();
        };
        // sum of the residual weight [v not in H] max(a p - bq q, 0) at node (k, j)
        auto team_sweep = [&](int k, int j, double a, double bq, int nh) {
            team_cmd(k, j, kTeamRes, 1, a, bq, 0.0, 1.0, nh);
            team_run();
            double z = 0.0;
            for (int m = 0; m < T; ++m) z += sh.tp[0][m];
            return z;
        };
        // the inverse-CDF draw of icdf over a team command set up by team_cmd
        auto team_icdf = [&](double u, double *Z, double *margin) {
            team_run();
            double z = 0.0;
            int last = -1;
            for (int m = 0; m < T; ++m) {
                z += sh.tp[0][m];
                last = max(last, sh.tlast[m]);
            }
            *Z = z;
            *margin = 0.0;
            if (!(z > 0.0) || !isfinite(z)) return -1;
            const double thr = u * z;
            // the first member range whose end passes u Z
            double base = 0.0;
            int ms = -1;
            for (int m = 0; m < T; ++m) {
                if (base + sh.tp[0][m] > thr) { ms = m; break; }
                base += sh.tp[0][m];
            }
            if (ms < 0) return last;   // rounding: no C_v exceeds u Z
            // that range's elements, recounted by the whole block in token order:
            // consecutive runs per thread, a block scan, then the run that crosses
            // u Z element by element
            const TeamBody &d = sh.cmd;
            const RD P(static_cast<const E *>(A.tgt) + ((static_cast<long long>(b) * K + d.c) * L1 + d.j) * V,
                       V);
            const RD Q(static_cast<const E *>(A.drf) +
                           ((static_cast<long long>(b) * K + d.c) * L + (d.with_q ? d.j : 0)) * V,
                       V);
            const double cT = 1.4426950408889634 / static_cast<double>(A.temp[b]);
            auto wat = [&](int v) {
                const double p = exp2_d(fma(static_cast<double>(P.at(v)) - static_cast<double>(d.Mp), cT, -d.lsp));
                const double q =
                    d.with_q ? exp2_d(fma(static_cast<double>(Q.at(v)) - static_cast<double>(d.Mq), cT, -d.lsq))
                             : 0.0;
                return team_weight(d, v, p, q);
            };
            const int e0 = kChunk * team_lo(ms, T, nch), e1 = min(kChunk * team_lo(ms + 1, T, nch), V);
            const int cnt = e1 > e0 ? (e1 - e0 + NT - 1) / NT : 0;
            const int a0 = min(e0 + tid * cnt, e1), a1 = min(a0 + cnt, e1);
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
            if (T > 1) {
                team_cmd(k, j, kTeamRes, 0, 1.0, 0.0, 0.0, 1.0, 0);
                return team_icdf(uc, &Z, &dm);
            }
            return icdf(k, j, false, [](int, double p, double) { return p; }, uc, &Z, &dm);
        };

        if (A.method == kMethodToken) {
            tau = L;
            for (int j = 0; j < L && !bad; ++j) {
                const double p = prob_tok(true, 0, j), q = prob_tok(false, 0, j);
                double a = ratio(p, q);
                if (a > 1.0) a = 1.0;
                if (!test(0, j + 1, a)) { tau = j; break; }
            }
            kstar = tau > 0 ? 0 : -1;
            if (!bad) {
                if (tau == L) {
                    y = draw_target(0, L);
                } else {
                    if (T > 1) {
                        team_cmd(0, tau, kTeamRes, 1, 1.0, 1.0, 0.0, 1.0, 0);
                        y = team_icdf(uc, &Z, &dm);
                    } else {
                        y = icdf(0, tau, true, [](int, double p, double q) { return fmax(p - q, 0.0); },
                                 uc, &Z, &dm);
                    }
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
                    if (T > 1) {
                        team_cmd(own, j, kTeamSSums, 1, 0.0, 0.0, 0.0, rho, 0);
                        team_run();
                        beta = 0.0;
                        D = 0.0;
                        for (int m = 0; m < T; ++m) {
                            beta += sh.tp[0][m];
                            D += sh.tp[1][m];
                        }
                        return;
                    }
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
                // Feasibility of rho, and g = rho - c(beta) for the secant steps.
                // Since rho beta + D = 1, (1 - beta)^n - D = beta (rho - c(beta)):
                // where beta is not small the difference ((1 - beta)^n - D) / beta
                // gives g without rho - c(beta)'s cancellation, whose noise near
                // rho* would turn the secant steps into bisection (~25 sweeps).
                auto feasible = [&](double rho, double *g, double *bt) {
                    double beta, D;
                    sums(rho, beta, D);
                    *bt = beta;
                    if (beta <= kQuotientFormBeta) {
                        const double cc = c_of(beta);
                        *g = rho - cc;
                        return cc <= rho;
                    }
                    double xn = 1.0;
                    for (int i = 0; i < n; ++i) xn *= 1.0 - beta;
                    *g = (xn - D) / beta;
                    return D <= xn;
                };
                // the fast walk's records at this position: all certain, and accepted?
                bool replay = follow && n > 1;
                int rec_acc = -1;
                if (replay) {
                    for (int k = 0; k < K && rec_acc < 0 && replay; ++k) {
                        if (!same_prefix(k, own, j)) continue;
                        const int dc = sh.dec[k * L + j];
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
                            // the secant point, kept 1e-3 of the width inside the
                            // bracket: where rho* lies that close to an end (an
                            // earlier step landed next to it) the bracket then
                            // shrinks a thousandfold a step instead of halving
                            const double sec = lo - glo * (hi - lo) / (ghi - glo);
                            const double w = hi - lo;
                            if (isfinite(sec)) t = fmin(fmax(sec, lo + 1e-3 * w), hi - 1e-3 * w);
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
                    // draft k shares node (own, j): its token's p and q there
                    const double p = prob_tok(true, k, j), q = prob_tok(false, k, j);
                    double a = ratio(p, rho * q);
                    if (a > 1.0) a = 1.0;
                    const bool ak = test(k, j + 1, a);
                    if (follow && n > 1) {
                        const int dc = sh.dec[k * L + j];
                        if (!(dc & kDecMade) || ak != ((dc & kDecAccept) != 0)) follow = false;
                    }
                    if (ak) acc = k;
                }
                if (acc < 0) {
                    double beta = beta_rho, D;
                    if (!isfinite(beta)) sums(rho, beta, D);
                    const double cc = c_of(beta);
                    if (T > 1) {
                        team_cmd(own, j, kTeamSRes, 1, 0.0, 0.0, cc, rho, 0);
                        y = team_icdf(uc, &Z, &dm);
                    } else {
                        y = icdf(own, j, true, [&](int, double p, double q) {
                            return fmax(p - cc * fmin(q, p / rho), 0.0);
                        }, uc, &Z, &dm);
                    }
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
                if (T > 1) return team_sweep(own, tau, alpha, beta, nH);
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
                    const double ps = prob_tok(true, k, tau), qs = prob_tok(false, k, tau);
                    const double om = fmax(alpha * ps - beta * qs, 0.0);
                    w[tau + 1] = chain(1.0, om / N, qs);
                    for (int j = tau + 1; j < L; ++j) {
                        w[j + 1] = chain(w[j], prob_tok(true, k, j), prob_tok(false, k, j));
                    }
                    if (bad) break;
                    int acc = 0;
                    for (int m = L; m > tau; --m) {
                        const int dc = follow ? sh.dec[k * L + m - 1] : 0;
                        if (follow && !(dc & kDecMade)) follow = false;
                        if (follow && (dc & kDecCertain)) {
                            s_made[k * L + m - 1] = 1;
                            if (!(dc & kDecAccept)) continue;
                            if (m < L) {
                                const double wm = w[m];
                                R[m] = T > 1 ? team_sweep(k, m, wm, 1.0, 0)
                                             : sweep(k, m, [&](int, double p, double q) {
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
                            R[m] = T > 1 ? team_sweep(k, m, wm, 1.0, 0)
                                         : sweep(k, m, [&](int, double p, double q) {
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
                    if (T > 1) {
                        team_cmd(own, tau, kTeamRes, 1, alpha, beta, 0.0, 1.0, nH);
                        y = team_icdf(uc, &Z, &dm);
                    } else {
                        y = icdf(own, tau, true, [&](int v, double p, double q) {
                            return in_H(v) ? 0.0 : fmax(alpha * p - beta * q, 0.0);
                        }, uc, &Z, &dm);
                    }
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

// The listed requests: with at least two workgroups per request, a team of
// T = min(grid / n, kTeamMax) per request (workgroup t*T runs it, the next T-1
// sum ranges of its passes); otherwise one workgroup per request, grid-stride.
// The grid is at most kRedoTeamSlots.
template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void redo_walk_kernel(RedoArgs A) {
    __shared__ RedoShared sh;
    const unsigned n = *A.count;
    if (n == 0) return;
    const int G = static_cast<int>(gridDim.x);
    const int T = static_cast<long long>(n) * 2 <= G ? min(G / static_cast<int>(n), kTeamMax) : 1;
    const long long per = static_cast<long long>(A.K) * (2 * A.L + 1);
    if (T == 1) {
        for (unsigned i = blockIdx.x; i < n; i += gridDim.x) {   // block-uniform
            const int entry = A.list[i];
            redo_request<NT, RD, E>(A, entry & ~kListNoReplay, entry, A.stats + i * per, sh, 0, 1);
        }
        return;
    }
    const int team = blockIdx.x / T, m = blockIdx.x % T;
    if (team >= static_cast<int>(n)) return;
    const int entry = A.list[team];
    const int b = entry & ~kListNoReplay;
    if (m == 0) {
        redo_request<NT, RD, E>(A, b, entry, A.stats + team * per, sh, team, T);
        if (threadIdx.x == 0)
            __hip_atomic_store(&A.team_cmd[team].seq, kTeamDone, __ATOMIC_RELEASE,
                               __HIP_MEMORY_SCOPE_AGENT);
    } else {
        team_member<NT, RD, E>(A, b, team, m, T, sh.cmd, sh.red, sh.ired, &sh.tseq);
    }
}

}  // namespace sv
