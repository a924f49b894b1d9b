// sv_walk.hpp -- per-request verification walk.
//
// One workgroup verifies one request.  Every thread runs the same scalar walk
// (fp64, identical inputs, hence identical decisions); the O(V) steps run
// block-wide over one node's row pair:
//   * residual mass   N = sum_v [v not in H] max(alpha p(v) - beta q(v), 0)
//   * GBV's R_m       = sum_v max(w_m p_m(v) - q_m(v), 0)
//   * inverse CDF     y = min{v : C_v > u Z} in token-id order.
// p and q are rebuilt per element from the row statistics: p(v) =
// 2^((l_v - M) c) / S.  Drafted-token probabilities come from one gathered
// logit per row and are kept in log2 form in fp64.  Repeated mass sweeps at
// one node, and the correction draw there, read a node list instead of the
// rows when one was built (NodeList below): the few thousand tokens whose
// residual weight can still matter, with a bound on the weight left out.
//
// Rules (see the header spec_verify.h for the full statement):
//  token level   -- standard speculative sampling: accept X_j iff
//                   u_j < min(1, p_j(X_j)/q_j(X_j)), stop at the first
//                   rejection, resample from norm(max(p - q, 0)), or from the
//                   target row after the block when all L are accepted.
//  block / K-draft -- GBV (SpecTr-GBV page, section 1) run draft after draft as
//                   the SpecTr-GBV page, section 2 ("algorithmic procedure",
//                   steps 1-5) describes: a draft off the accepted prefix is
//                   skipped; a draft whose token at the node is in H is rejected
//                   without a test; otherwise its sub-block is tested from
//                   position L down to tau+1 against w_m / h_m, where the first
//                   position's target is the node residual omega/N.
//                   Acceptance at m sets tau = m and, for m < L, the residual
//                   (alpha, beta, N) = (w_m, 1, R_m); rejection adds the first
//                   token to H and N to beta.  One O(V) sweep per selection
//                   step, no search over a scaling factor (section 3).
//  SpecTr        -- the position-by-position multi-draft baseline (SpecTr-GBV
//                   page, sections 1 and 3): at each position the n drafts on
//                   the accepted prefix are tried in draft order, each accepted
//                   with probability min(1, p(x)/(rho* q(x))) (rho* from
//                   sv_spectr.hpp); the first acceptance extends the prefix,
//                   none stops the walk with a correction from
//                   max(p - c q, (1 - c/rho*) p) = max(p - c min(q, p/rho*), 0).
// A test at m < L with u >= w_m is settled without its sweep: R_m <= w_m
// implies h_m = R_m / (R_m + 1 - w_m) <= w_m, so it rejects either way.
#pragma once

#include "sv_device.hpp"
#include "sv_rowstats.hpp"
#include "sv_spectr.hpp"

namespace sv {

constexpr int kMaxK = 64;
constexpr int kMaxL = 16;
constexpr int kMaxV = 1 << 22;
constexpr int kMethodToken = 0;
constexpr int kMethodBlockWalk = 1;
constexpr int kMethodSpecTr = 2;
constexpr int kMethodSpecTrBisect = 3;   // SpecTr with rho* found by plain bisection
constexpr int kFlagDegenerate = 1;
constexpr int kFlagInvalid = 2;
constexpr int kFlagNearTie = 4;
constexpr double kNearTie = 1e-5;   // decisions closer than this to their threshold are flagged
// Relative error of one probability formed from fp32 exponentials (v_exp_f32 and
// the rounding of its argument), the unit of the first-order error estimates
// that mark ill-conditioned GBV tests for re-evaluation in fp64.
constexpr double kExpEps = 0x1p-23;
// With diagnostics requested, a request whose estimated error of some h exceeds
// this (a quarter of the 1e-5 the acceptance probabilities are reported to) is
// taken again in fp64 too, so the reported h hold to fp64 however ill-conditioned.
constexpr double kDiagEh = 2.5e-6;
// A test's record for the fp64 re-evaluation (WalkArgs::dec).  Certain:
// its margin is at least SV_NEAR_TIE plus four times its error estimate, so
// the exact test agrees and its exact margin exceeds SV_NEAR_TIE.
constexpr unsigned char kDecMade = 1, kDecAccept = 2, kDecCertain = 4;
// A listed request whose walk met a degenerate residual, after which the fast
// and the fp64 walk can be in different states: re-evaluated without the records.
constexpr int kListNoReplay = 1 << 30;
// Node lists: entries per wave, and the cutoff 2^-kListCut below which a
// token's residual weight omega(v) / alpha leaves the list.
constexpr int kWaveList = 2048;
constexpr int kListCut = 50;

struct WalkArgs {
    const void *tgt;        // [B][K][L+1][V]
    const void *drf;        // [B][K][L][V]
    const int32_t *tok;     // [B][K][L]
    const float *temp;      // [B]
    const float *ua;        // [B][K][L]
    const float *uc;        // [B]
    const RowStat *stats;   // [B][K][2L+1]
    int B, K, L, V;
    int method;             // kMethodToken, kMethodBlockWalk or kMethodSpecTr
    int all_nodes;          // statistics of every node row are present (diagnostics, or given)
    int fv_depth;           // otherwise the first-visit rows are at positions j < fv_depth
    int stats_given;        // they came from the caller: no row was streamed here
    int round;              // 1, or 2 to resume the walks the first round suspended
    int two_round;          // a second round follows: the first may suspend
    int rho_bisect;         // SpecTr: find rho* by plain bisection instead of histogram + Newton
    struct WalkState *state;     // [B]
    unsigned char *need;    // [B][K][L]: node rows flagged for the second round
    RowRef *list;           // the same rows as a list for the statistics kernel
    unsigned *list_count;
    void *nodes;            // [B] node lists (node_list_bytes each), or null
    int32_t *accept_len, *draft_index, *correction, *flags, *rows_streamed;
    float *row_lse, *accept_prob, *resid_mass;
    unsigned *redo_count;   // requests with a decision within its error of its threshold,
    int32_t *redo_list;     // listed here for the fp64 re-evaluation
    unsigned char *dec;     // [B][K][L] tests made (kDecMade), accepted (kDecAccept) and
                            // certain in exact arithmetic (kDecCertain); entries of tests
                            // not made are left as they were
    double *rho_rec;        // [B][L] SpecTr's scaling factor at each position it reached
};

// Likelihood ratio from log2-probabilities, with the drafted-token convention:
// q = 0 gives +inf if p > 0 and 0 otherwise.
__device__ __forceinline__ double ratio_log2(double lp, double lq) {
    if (lq == -INFINITY) return lp > -INFINITY ? INFINITY : 0.0;
    return exp2(lp - lq);
}

__device__ __forceinline__ double chain_step(double w, double r) {
    if (w == 0.0) return 0.0;
    const double t = w * r;
    return t < 1.0 ? t : 1.0;
}

// Relative error estimate of a weight after min(t, 1), t carrying relative error
// rel: a value above 1 by more than four times its error clamps to exactly 1 in
// exact arithmetic too (error 0); otherwise the clamp may not hold exactly.
__device__ __forceinline__ double clamp_err(double t, double rel) {
    return (t >= 1.0 && t * (1.0 - 4.0 * rel) >= 1.0) ? 0.0 : rel;
}

// The chunks of the rejected-token set H that this thread reads (chunk c is
// read by thread c mod NT in every sweep): up to two are kept, and a third
// sets `many`, after which every chunk of the thread is checked.
struct HLanes {
    int c0, c1;
    bool many;
};
template <int NT>
__device__ __forceinline__ HLanes h_lanes(const int *H, int nH) {
    HLanes h{-1, -1, false};
    for (int i = 0; i < nH; ++i) {
        const int hc = H[i] / kChunk;
        if (hc % NT != static_cast<int>(threadIdx.x) || hc == h.c0 || hc == h.c1) continue;
        if (h.c0 < 0) h.c0 = hc;
        else if (h.c1 < 0) h.c1 = hc;
        else h.many = true;
    }
    return h;
}

// Zero the weights of chunk ch's tokens that are in H.
__device__ __forceinline__ void h_zero8(int ch, const int *H, int nH, const HLanes &hl, float w[8]) {
    if (ch == hl.c0 || ch == hl.c1 || hl.many) {
        for (int i = 0; i < nH; ++i) {
            const unsigned off = static_cast<unsigned>(H[i] - kChunk * ch);
            if (off < 8u) {
#pragma unroll
                for (int e = 0; e < 8; ++e) w[e] = (off == static_cast<unsigned>(e)) ? 0.0f : w[e];
            }
        }
    }
}

// omega(v) / a for the 8 elements of chunk ch, where omega(v) = [v not in H]
// max(a eP - bq eQ, 0), eP = 2^(x c - MPc) (MPc = shift_term of the row's
// shift): computed as max(eP - r eQ, 0) with r = bq / a, so one FMA and one
// max per element; the sweeps scale their sums by a once.  Without a Q row,
// omega / a = eP.  With FLOOR the lower bound is g eP (g >= 0) instead of 0.
template <bool HAS_Q, bool FLOOR = false>
__device__ __forceinline__ void omega8(const float xp[8], const float xq[8], float MPc, float MQc,
                                       float r, float g, const Scale &c, int ch, const int *H,
                                       int nH, const HLanes &hl, float w[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float ep = fast_exp2(expo(xp[e], c, MPc));
        if (HAS_Q) {
            const float eq = fast_exp2(expo(xq[e], c, MQc));
            w[e] = fmaxf(fmaf(-r, eq, ep), FLOOR ? g * ep : 0.0f);
        } else {
            w[e] = ep;
        }
    }
    h_zero8(ch, H, nH, hl, w);
}

// The residual a eP - bq eQ of a sweep, held as a (max(eP - r eQ, 0)) with
// r = bq / a.
struct SweepRows {
    float MPc, MQc;   // shift terms of the target and draft rows
    double a;         // > 0
    float r;          // bq / a, >= 0, finite
    float g = 0.0f;   // floor coefficient over a (FLOOR sweeps only)
    // a = alpha / S_P, bq = beta / S_Q (S = the rows' sums)
    __device__ void set(double alpha, double SP, double beta, double SQ) {
        a = alpha / SP;
        r = static_cast<float>(fmin(beta * SP / (alpha * SQ), 3.402823466e38));
    }
};

// Block-wide sum of omega over a row pair (or a single row when HAS_Q is false),
// 32 bytes per row in flight per lane (more costs the walk registers it
// spills elsewhere).
template <int NT, typename RD, bool HAS_Q, bool FLOOR = false>
__device__ double sweep_mass(const RD &P, const RD &Q, int nch, const SweepRows &s, const Scale &c,
                             const int *H, int nH, double *red) {
    const HLanes hl = h_lanes<NT>(H, nH);
    double acc = 0.0;
    stream_rows<NT, depth_for<RD, 32>(), HAS_Q>(P, Q, nch,
                                               [&](const float xp[8], const float xq[8], int ch) {
        float w[8];
        omega8<HAS_Q, FLOOR>(xp, xq, s.MPc, s.MQc, s.r, s.g, c, ch, H, nH, hl, w);
        acc += static_cast<double>(sum8(w));
    });
    return s.a * block_sum<NT>(acc, red);
}

// Node list: the tokens of one node whose residual weight can matter to a
// later mass sweep at that node.  While the walk stays at a node, alpha is
// fixed, beta only grows and H only gains tokens, so omega(v) = [v not in H]
// max(alpha p(v) - beta q(v), 0) never grows: a token whose weight is below
// alpha 2^-kListCut at the sweep that builds the list stays below it, and the
// weight the list leaves out (summed exactly by that sweep) bounds what any
// later sweep misses.  Each wave keeps its own list of up to kWaveList entries
// (token, eP, eQ: the sweep's own fp32 exponentials) in token order, compacted
// with wave ballots so the stores and the later loads are contiguous.
template <int NT>
struct NodeList {
    int *idx;
    float *ep, *eq;
    __device__ NodeList(void *base, long long b) {
        constexpr long long n = static_cast<long long>(NT / kWave) * kWaveList;
        char *p = static_cast<char *>(base) + b * (3 * n * 4);
        const long long w = static_cast<long long>(threadIdx.x / kWave) * kWaveList;
        idx = reinterpret_cast<int *>(p) + w;
        ep = reinterpret_cast<float *>(p + n * 4) + w;
        eq = reinterpret_cast<float *>(p + 2 * n * 4) + w;
    }
};

template <int NT>
constexpr long long node_list_bytes() {
    return 3LL * (NT / kWave) * kWaveList * 4;
}

// Rank of this lane among the lanes of the wave set in m.
__device__ __forceinline__ int lanes_below(unsigned long long m) {
    return static_cast<int>(__builtin_amdgcn_mbcnt_hi(
        static_cast<unsigned>(m >> 32), __builtin_amdgcn_mbcnt_lo(static_cast<unsigned>(m), 0u)));
}

// sweep_mass over a row pair that also writes the node list: a token enters
// it when omega / a > keep (keep = S_P 2^-kListCut, i.e. omega > alpha
// 2^-kListCut).  Returns the mass; *cnt is the entry count of this lane's wave,
// *out the weight left out (omega units), *overflow whether any wave ran out
// of room.  Every lane runs the same tiles of NT chunks (chunk t NT + tid,
// masked past the row), so the ballots see the whole wave and each wave's list
// is in token order; two tiles of each row stay in flight per lane.  A wave
// whose list is full stops compacting (flat rows keep most tokens) and sweeps
// on as sweep_mass does.
template <int NT, typename RD>
__device__ double sweep_mass_build(const RD &P, const RD &Q, int nch, const SweepRows &s,
                                   const Scale &c, const int *H, int nH, float keep,
                                   const NodeList<NT> &nl, int *cnt, double *out, bool *overflow,
                                   double *red2) {
    const HLanes hl = h_lanes<NT>(H, nH);
    const int tid = threadIdx.x;
    const int ntile = (nch + NT - 1) / NT;
    double acc = 0.0, exc = 0.0;
    int n = 0;   // entries of this wave so far (wave-uniform)
    typename RD::Raw rp[2], rq[2];
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int cl = min(i * NT + tid, nch - 1);
        rp[i] = P.raw(cl);
        rq[i] = Q.raw(cl);
        __builtin_amdgcn_sched_barrier(0);
    }
    for (int t0 = 0; t0 < ntile; t0 += 2) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (t0 + i >= ntile) break;                 // wave-uniform
            const int ch = (t0 + i) * NT + tid;
            const bool valid = ch < nch;
            float w[8];
            {
                float xp[8], xq[8];
                RD::unpack(rp[i], xp);
                RD::unpack(rq[i], xq);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float ep = fast_exp2(expo(xp[e], c, s.MPc));
                    const float eq = fast_exp2(expo(xq[e], c, s.MQc));
                    w[e] = valid ? fmaxf(fmaf(-s.r, eq, ep), 0.0f) : 0.0f;
                }
            }
            h_zero8(ch, H, nH, hl, w);
            acc += static_cast<double>(sum8(w));
            if (n <= kWaveList) {   // else this wave's list is full: a plain sweep from here
                float ex = 0.0f;
                unsigned long long any = 0;
                unsigned long long m[8];
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const bool k = w[e] > keep;
                    if (!k) ex += w[e];
                    m[e] = __ballot(k);
                    any |= m[e];
                }
                exc += static_cast<double>(ex);
                if (any) {
                    // slot of (lane, e): the wave's entries so far, the kept tokens
                    // of lower lanes in this tile, then this lane's kept tokens
                    // before e.  The exponentials are recomputed here from the
                    // chunk still held raw, so the sweep keeps none of them live.
                    int slot = n, tot = 0;
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        slot += lanes_below(m[e]);
                        tot += __popcll(m[e]);
                    }
                    float xp[8], xq[8];
                    RD::unpack(rp[i], xp);
                    RD::unpack(rq[i], xq);
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        if (w[e] > keep) {
                            if (slot < kWaveList) {
                                nl.idx[slot] = kChunk * ch + e;
                                nl.ep[slot] = fast_exp2(expo(xp[e], c, s.MPc));
                                nl.eq[slot] = fast_exp2(expo(xq[e], c, s.MQc));
                            }
                            ++slot;
                        }
                    }
                    n += tot;
                }
            }
            const int cl = min(ch + 2 * NT, nch - 1);   // refill with the tile two on
            rp[i] = P.raw(cl);
            rq[i] = Q.raw(cl);
        }
    }
    *cnt = n;
    *overflow = __syncthreads_or(n > kWaveList) != 0;
    double v[2] = {acc, exc};
    block_sum_n<NT, 2>(v, red2);
    *out = s.a * v[1];
    return s.a * v[0];
}

// The mass of the residual over a node list (cnt entries in this lane's wave;
// lane l takes entries l, l + 64, ...).  A lane's loads for eight entries go
// out before any is used: a typical list (a few hundred entries per wave) is
// then one round trip.
template <int NT>
__device__ double sweep_mass_list(const NodeList<NT> &nl, int cnt, const SweepRows &s,
                                  const int *H, int nH, double *red) {
    constexpr int U = 8;
    const int lane = threadIdx.x & (kWave - 1);
    double acc = 0.0;
    for (int i0 = 0; i0 < cnt; i0 += U * kWave) {
        float p[U], q[U];
        int x[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            const int i = i0 + j * kWave + lane;
            const int ic = i < cnt ? i : cnt - 1;
            p[j] = nl.ep[ic];
            q[j] = nl.eq[ic];
            x[j] = nl.idx[ic];
            if (i >= cnt) p[j] = q[j] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            float v = fmaxf(fmaf(-s.r, q[j], p[j]), 0.0f);
            for (int h = 0; h < nH; ++h) v = (H[h] == x[j]) ? 0.0f : v;
            acc += static_cast<double>(v);
        }
    }
    return s.a * block_sum<NT>(acc, red);
}

// Node-list draws cover rows of at most this many tiles of NT chunks.
constexpr int kListTiles = 64;

// Inverse-CDF draw over a node list, in token-id order: y = min{v : C_v > u Z}
// over the listed tokens, or the last listed token of positive weight when
// rounding leaves no crossing.  Token order across the lists is tile-major,
// then wave (wave w holds chunks 64 w .. 64 w + 63 of each tile), then the
// order inside a wave's list.  Each wave sums its entries per tile into
// seg[t NW + w] (runs of one tile are contiguous in its list, which also gives
// their first entry, segstart); wave 0 scans the segments for the crossing; the
// wave that owns it rescans that run.  Returns -1 when Z is not a positive
// finite number; Z (omega units) in *Z.
template <int NT>
__device__ int sweep_icdf_list(const NodeList<NT> &nl, int cnt, const SweepRows &s, const int *H,
                               int nH, double u, int ntile, double *Z, double *seg, int *segstart,
                               int *ired, double *red, double *margin) {
    *margin = 0.0;   // distance of u Z to the nearest boundary of the draw, over Z
    constexpr int NW = NT / kWave;
    constexpr int kTileTokens = kChunk * NT;
    const int lane = threadIdx.x & (kWave - 1);
    const int w = threadIdx.x / kWave;
    auto entry = [&](int i, int &x) {   // omega / a of entry i (0 for tokens in H)
        x = nl.idx[i];
        float f = fmaxf(fmaf(-s.r, nl.eq[i], nl.ep[i]), 0.0f);
        for (int h = 0; h < nH; ++h) f = (H[h] == x) ? 0.0f : f;
        return static_cast<double>(f);
    };
    for (int t = lane; t < ntile; t += kWave) {
        seg[t * NW + w] = 0.0;
        segstart[t * NW + w] = -1;
    }
    int tcarry = -1;   // tile of the previous batch's last entry
    for (int i0 = 0; i0 < cnt; i0 += kWave) {
        const int i = i0 + lane;
        const bool valid = i < cnt;
        int x = 0, t = 0x7fffffff;
        double v = 0.0;
        if (valid) {
            v = entry(i, x);
            t = x / kTileTokens;
        }
        int tp = __shfl_up(t, 1, kWave);
        if (lane == 0) tp = tcarry;
        if (valid && t != tp) segstart[t * NW + w] = i;   // first entry of tile t
        // first lane of this lane's run inside the batch
        int f = (valid && (lane == 0 || t != tp)) ? lane : -1;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
            const int g = __shfl_up(f, o, kWave);
            if (lane >= o) f = max(f, g);
        }
        const double inc = wave_exclusive_scan(v) + v;
        const double b0 = __shfl(inc, f > 0 ? f - 1 : 0, kWave);
        const double before = f > 0 ? b0 : 0.0;
        const int tn = __shfl_down(t, 1, kWave);
        if (valid && (lane == kWave - 1 || i + 1 >= cnt || tn != t)) seg[t * NW + w] += inc - before;
        tcarry = __shfl(t, kWave - 1, kWave);
    }
    __syncthreads();
    if (w == 0) {
        const int nq = ntile * NW;
        const int per = (nq + kWave - 1) / kWave;
        const int q0 = lane * per, q1 = min(q0 + per, nq);
        double ls = 0.0;
        for (int q = q0; q < q1; ++q) ls += seg[q];
        const double ex = wave_exclusive_scan(ls);
        const double z = __shfl(ex + ls, kWave - 1, kWave);
        const double thr = u * z;
        int qc = 0x7fffffff, ql = -1;
        double bc = 0.0, cum = ex;
        for (int q = q0; q < q1; ++q) {
            if (qc == 0x7fffffff && cum + seg[q] > thr) {
                qc = q;
                bc = cum;
            }
            cum += seg[q];
            if (seg[q] > 0.0) ql = q;
        }
        const int qmin = wave_min_int(qc);
        const double base = __shfl(bc, qmin == 0x7fffffff ? 0 : qmin / per, kWave);
        ql = wave_max_int(ql);
        if (lane == 0) {
            ired[0] = qmin;
            ired[1] = ql;
            red[0] = base;
            red[1] = z;
        }
    }
    __syncthreads();
    const int qs = ired[0], ql = ired[1];
    const double base = red[0], z = red[1];
    *Z = s.a * z;
    if (!(z > 0.0) || !isfinite(z) || ql < 0) {
        __syncthreads();
        return -1;
    }
    const double thr = u * z;
    const bool past = qs == 0x7fffffff;   // rounding left the threshold past every crossing
    const int q = past ? ql : qs;
    const int tq = q / NW;
    if (w == q % NW) {   // wave-uniform
        double carry = base;
        int found = -1, lastpos = -1;
        for (int i0 = segstart[q]; i0 >= 0; i0 += kWave) {
            const int i = i0 + lane;
            int x = 0;
            double v = 0.0;
            bool in = i < cnt;
            if (in) {
                v = entry(i, x);
                in = x / kTileTokens == tq;
                if (!in) v = 0.0;
            }
            const double inc = wave_exclusive_scan(v) + v + carry;
            const unsigned long long mc = __ballot(in && inc > thr);
            if (!past && mc) {
                const int fl = __ffsll(static_cast<long long>(mc)) - 1;
                found = __shfl(x, fl, kWave);
                const double hi = __shfl(inc, fl, kWave), lo = hi - __shfl(v, fl, kWave);
                if (lane == 0) red[2] = fmin(hi - thr, thr - lo);
                break;
            }
            const unsigned long long mp = __ballot(in && v > 0.0);
            if (mp) lastpos = __shfl(x, 63 - __clzll(static_cast<long long>(mp)), kWave);
            carry = __shfl(inc, kWave - 1, kWave);
            if (__ballot(in) != ~0ull) break;   // the run ends in this batch
        }
        if (lane == 0) {
            ired[2] = found >= 0 ? found : lastpos;
            if (found < 0) red[2] = 0.0;
        }
    }
    __syncthreads();
    const int y = ired[2];
    *margin = red[2] / z;
    __syncthreads();
    return y;
}

// Block-wide inverse-CDF draw over omega in token-id order.  Returns y, or -1
// when the mass Z is not a positive finite number.  Z is returned in *Z.
// Tiles of NT chunks are summed four at a time into tile[] (per-chunk sums in
// fp32, accumulated in fp64); the tile holding the threshold is rescanned with
// a block scan, element by element in fp64 inside the crossing chunk.  When
// rounding leaves the threshold past every crossing, the draw is the last
// token of positive weight, found from the last chunk with positive weight.
template <int NT, typename RD, bool HAS_Q, bool FLOOR = false>
__device__ int sweep_icdf(const RD &P, const RD &Q, int nch, const SweepRows &s, const Scale &c,
                          const int *H, int nH, double u, double *Z, double *tile, double *red,
                          double *red4, int *ired, double *margin) {
    *margin = 0.0;   // distance of u Z to the nearest boundary of the draw, over Z
    const HLanes hl = h_lanes<NT>(H, nH);
    const int ntile = (nch + NT - 1) / NT;
    int lastc = -1;
    // four tiles per group.  With 16-byte chunks each chunk's register slot is
    // refilled with the same lane's chunk of the next group (clamped into the
    // row) once it is unpacked, so the next group's loads overlap this group's
    // arithmetic and block sum; wider chunks are loaded group by group (the
    // rolling form would double their registers).
    constexpr bool kRoll = sizeof(typename RD::Raw) <= 16;
    typename RD::Raw rp[4], rq[4];
    auto load_group = [&](int t0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int cl = min((t0 + i) * NT + static_cast<int>(threadIdx.x), nch - 1);
            rp[i] = P.raw(cl);
            if (HAS_Q) rq[i] = Q.raw(cl);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    if (kRoll) load_group(0);
    for (int t0 = 0; t0 < ntile; t0 += 4) {
        if (!kRoll) load_group(t0);
        double cs[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int ch = (t0 + i) * NT + threadIdx.x;
            cs[i] = 0.0;
            float xp[8], xq[8], w[8];
            RD::unpack(rp[i], xp);
            if (HAS_Q) RD::unpack(rq[i], xq);
            if (kRoll) {
                const int cl = min(ch + 4 * NT, nch - 1);
                rp[i] = P.raw(cl);
                if (HAS_Q) rq[i] = Q.raw(cl);
            }
            if (ch < nch) {
                omega8<HAS_Q, FLOOR>(xp, xq, s.MPc, s.MQc, s.r, s.g, c, ch, H, nH, hl, w);
                const float t = sum8(w);
                cs[i] = static_cast<double>(t);
                if (t > 0.0f) lastc = ch;
            }
        }
        block_sum4<NT>(cs, red4);
        if (threadIdx.x == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (t0 + i < ntile) tile[t0 + i] = cs[i];
        }
    }
    lastc = block_max_int<NT>(lastc, ired);   // its barriers publish tile[]
    // the tiles hold omega / a: the threshold u z and every comparison with it
    // are taken at that scale
    double z = 0.0;
    for (int t = 0; t < ntile; ++t) z += tile[t];
    *Z = s.a * z;
    if (!(z > 0.0) || !isfinite(z)) return -1;
    // the last token of positive weight (block-uniform call)
    auto last_positive = [&]() {
        __syncthreads();   // readers of ired[] in the reductions above are done
        if (static_cast<int>(threadIdx.x) == lastc % NT) {
            float xp[8], xq[8], w[8];
            P.load(lastc, xp);
            if (HAS_Q) Q.load(lastc, xq);
            omega8<HAS_Q, FLOOR>(xp, xq, s.MPc, s.MQc, s.r, s.g, c, lastc, H, nH, hl, w);
            int last = kChunk * lastc;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (w[e] > 0.0f) last = kChunk * lastc + e;
            ired[0] = last;
        }
        __syncthreads();
        const int y = ired[0];
        __syncthreads();
        return y;
    };
    const double thr = u * z;
    double base = 0.0;
    int tc = -1;
    for (int t = 0; t < ntile; ++t) {
        if (base + tile[t] > thr) { tc = t; break; }
        base += tile[t];
    }
    if (tc < 0) return last_positive();

    const int ch = tc * NT + threadIdx.x;
    float w[8];
    double cs = 0.0;
    if (ch < nch) {
        float xp[8], xq[8];
        P.load(ch, xp);
        if (HAS_Q) Q.load(ch, xq);
        omega8<HAS_Q, FLOOR>(xp, xq, s.MPc, s.MQc, s.r, s.g, c, ch, H, nH, hl, w);
        cs = static_cast<double>(sum8(w));
    }
    const double pre = base + block_exclusive_scan<NT>(cs, red);
    int cand = 0x7fffffff;
    double cm = 0.0;
    if (ch < nch && pre <= thr && pre + cs > thr) {
        double C = pre;
        int last = -1;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (cand == 0x7fffffff) {
                if (w[e] > 0.0f) last = kChunk * ch + e;
                const double before = C;
                C += static_cast<double>(w[e]);
                if (C > thr) {
                    cand = kChunk * ch + e;
                    cm = fmin(C - thr, thr - before);
                }
            }
        }
        if (cand == 0x7fffffff && last >= 0) cand = last;
    }
    const int mine = cand;
    cand = block_min_int<NT>(cand, ired);
    if (cand == 0x7fffffff) return last_positive();
    // the margin from the lane that drew (the block reductions that read red[]
    // are done: block_min_int's barriers passed them)
    if (mine == cand) red[0] = cm;
    __syncthreads();
    *margin = red[0] / z;
    __syncthreads();
    return cand;
}

// Block-wide maximum of a row (NaN entries are ignored here; they surface as a
// NaN mass in the following sweep).
template <int NT, typename RD>
__device__ float sweep_rowmax(const RD &P, int nch, float *fred) {
    float m = -INFINITY;
    stream_rows<NT, depth_for<RD, 32>(), false>(
        P, P, nch, [&](const float x[8], const float *, int) { m = fmaxf(m, max8(x)); });
    return block_max<NT>(m, fred);
}

// Block-wide statistics of a node's target row and draft row; the walk's
// fallback for a row that no launch of the statistics kernel streamed.
template <int NT, typename RD>
__device__ void sweep_stats_pair(const RD &P, const RD &Q, int nch, const Scale &c, RowStat &sp,
                                 RowStat &sq, float *fred, double *red) {
    const int tid = threadIdx.x;
    float xp[8], xq[8];
    const bool have0 = tid < nch;
    if (have0) {
        P.load(tid, xp);
        Q.load(tid, xq);
    } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) xp[e] = xq[e] = -INFINITY;
    }
    LaneSoftmax lp, lq;
    lp.init(block_max<NT>(max8(xp), fred), c);
    lq.init(block_max<NT>(max8(xq), fred), c);
    if (have0) {
        lp.consume(xp, c);
        lq.consume(xq, c);
    }
    if (nch > NT) {
        const RD P1 = P.advanced(NT), Q1 = Q.advanced(NT);
        stream_rows<NT, depth_for<RD, 32>(), true>(P1, Q1, nch - NT,
                                 [&](const float (&ap)[8], const float (&aq)[8], int) {
                                     lp.consume(ap, c);
                                     lq.consume(aq, c);
                                 });
    }
    sp = finish_row<NT>(lp, c, fred, red);
    sq = finish_row<NT>(lq, c, fred, red);
}

// Walk state saved when the first round stops for rows below an accepted node.
struct WalkState {
    int status;             // kStateDone or kStateSuspended
    int k_next;             // draft to examine on resumption
    int tau, own, kstar, nH, flags, rows;
    int list_tries;         // node lists the request may still build
    double alpha, beta, N;
    double tie;             // smallest |u - threshold| over the decisions so far
    int H[kMaxK];
};
constexpr int kStateDone = 0;
constexpr int kStateSuspended = 1;

// Two 512-thread walks per CU (4 waves per SIMD) keep every request of a
// 512-request batch resident at once.  SPECTR selects SpecTr's forward walk;
// otherwise A.method chooses between the token-level rule and the block walk.
template <int NT, typename RD, typename E, bool SPECTR = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(4))) void walk_kernel(
    WalkArgs A) {
    constexpr int kMaxTiles = (kMaxV / kChunk + NT - 1) / NT;
    constexpr int kMaxRS = 2 * kMaxL + 1;
    constexpr int NW = NT / kWave;
    __shared__ int s_x[kMaxK * kMaxL];
    __shared__ unsigned char s_can[kMaxK * (kMaxL + 1)];
    __shared__ unsigned char s_have[kMaxK * (kMaxL + 1)];
    __shared__ float s_gp[kMaxK * kMaxL];
    __shared__ float s_gq[kMaxK * kMaxL];
    __shared__ float s_M[kMaxK * kMaxRS];
    __shared__ double s_S[kMaxK * kMaxRS];
    __shared__ double s_red[NW];
    __shared__ double s_red4[4 * NW];
    __shared__ float s_fred[NW];
    __shared__ int s_ired[NW];
    __shared__ double s_tile[kMaxTiles];
    __shared__ int s_H[kMaxK];
    __shared__ double s_w[kMaxL + 1];
    __shared__ double s_wrel[kMaxL + 1];   // relative error estimates of the weights
    __shared__ unsigned s_hist[SPECTR ? 2 * kHistBins : 1];
    __shared__ double s_red6[SPECTR ? 6 * NW : 1];
    __shared__ double s_br[4];
    __shared__ double s_lseg[SPECTR ? 1 : kListTiles * NW];   // node-list draw: tile x wave sums
    __shared__ int s_lstart[SPECTR ? 1 : kListTiles * NW];

    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int K = A.K, L = A.L, V = A.V, KL = K * L, RS = 2 * L + 1, L1 = L + 1;
    WalkState *ws = A.state + b;
    if (A.round == 2 && ws->status != kStateSuspended) return;   // finished in the first round

    const int nch = (V + kChunk - 1) / kChunk;
    const long long bKL = static_cast<long long>(b) * KL;
    const float T = A.temp[b];
    const Scale sc = temp_scale(T);           // exponent scale of this request
    const double scd = scale64(sc);
    const E *tgt = static_cast<const E *>(A.tgt);
    const E *drf = static_cast<const E *>(A.drf);
    const RowStat *st = A.stats + static_cast<long long>(b) * K * RS;
    unsigned char *need = A.need + bKL;
    auto trow = [&](int c, int j) {
        return tgt + ((static_cast<long long>(b) * K + c) * L1 + j) * V;
    };
    auto drow = [&](int c, int j) {
        return drf + ((static_cast<long long>(b) * K + c) * L + j) * V;
    };

    // 1. tokens, uniforms, temperature
    int bad = !(T > 0.0f) || !isfinite(T);
    for (int i = tid; i < KL; i += NT) {
        const int x = A.tok[bKL + i];
        s_x[i] = x;
        bad |= (x < 0 || x >= V);
        const float u = A.ua[bKL + i];
        bad |= !(u >= 0.0f && u < 1.0f);
        if (A.round == 1) {
            if (A.accept_prob) A.accept_prob[bKL + i] = NAN;
            if (A.dec) A.dec[bKL + i] = 0;   // this call's tests only
            need[i] = 0;
        }
    }
    const float ucf = A.uc[b];
    bad |= !(ucf >= 0.0f && ucf < 1.0f);
    bad = __syncthreads_or(bad);

    // 2. node (lowest-index draft with the same prefix) of every (k, j), j = 0..L,
    //    and the node rows whose statistics a launch of the statistics kernel made
    int streamed = 0;
    for (int i = tid; i < K * L1; i += NT) {
        const int k = i / L1, j = i % L1;
        int c = k;
        for (int cc = 0; cc < k; ++cc) {
            int same = 1;
            for (int t = 0; t < j; ++t) same &= (s_x[cc * L + t] == s_x[k * L + t]);
            if (same) { c = cc; break; }
        }
        s_can[i] = static_cast<unsigned char>(c);
        int first = 1;
        for (int cc = 0; cc < k; ++cc) first &= (s_x[cc * L] != s_x[k * L]);
        int have = 0;
        if (j < L && c == k) {
            const int fv = A.all_nodes || (j == 0 && k == 0) || (j > 0 && j < A.fv_depth && first);
            const int nd = A.round == 2 && need[k * L + j];
            have = fv || nd;
            streamed += fv ? (A.round == 1 ? 2 : 0) : (nd ? 2 : 0);
        }
        if (j == L && c == k && A.all_nodes) streamed += 1;
        s_have[i] = static_cast<unsigned char>(have);
    }
    __syncthreads();
    if (A.stats_given) streamed = 0;
    streamed = static_cast<int>(block_sum<NT>(static_cast<double>(streamed), s_red));

    // 3. statistics of those rows into LDS; logits at the drafted tokens
    if (!bad) {
        for (int i = tid; i < KL; i += NT) {
            const int k = i / L, j = i % L;
            const int c = s_can[k * L1 + j];
            const int x = s_x[i];
            s_gp[i] = RD(trow(c, j), V).at(x);
            s_gq[i] = RD(drow(c, j), V).at(x);
            if (c == k && s_have[k * L1 + j]) {
                const RowStat a = st[k * RS + j], q = st[k * RS + L1 + j];
                s_M[k * RS + j] = a.shift;
                s_S[k * RS + j] = a.sum;
                s_M[k * RS + L1 + j] = q.shift;
                s_S[k * RS + L1 + j] = q.sum;
            }
        }
    }
    __syncthreads();

    // statistics of node (c, j): 1 = present and valid, 0 = not a distribution,
    // -1 = not streamed yet and the walk may stop for it (first of two rounds);
    // otherwise they are computed here
    const bool may_suspend = A.round == 1 && A.two_round;
    auto ensure = [&](int c, int j) -> int {
        if (!s_have[c * L1 + j]) {
            if (may_suspend) return -1;
            RowStat sp, sq;
            sweep_stats_pair<NT, RD>(RD(trow(c, j), V), RD(drow(c, j), V), nch, sc, sp, sq, s_fred,
                                     s_red);
            if (tid == 0) {
                s_M[c * RS + j] = sp.shift;
                s_S[c * RS + j] = sp.sum;
                s_M[c * RS + L1 + j] = sq.shift;
                s_S[c * RS + L1 + j] = sq.sum;
                s_have[c * L1 + j] = 1;
            }
            __syncthreads();
        }
        RowStat a, q;
        a.shift = s_M[c * RS + j];
        a.sum = s_S[c * RS + j];
        q.shift = s_M[c * RS + L1 + j];
        q.sum = s_S[c * RS + L1 + j];
        return (stat_ok(a) && stat_ok(q)) ? 1 : 0;
    };
    // log2 p and log2 q of draft k's token at position j under its node rows
    // (the exponent x sc - shift_term(M, sc) in fp64, as the sweeps form it in fp32)
    auto lp2 = [&](int k, int j) {
        const int c = s_can[k * L1 + j];
        return static_cast<double>(s_gp[k * L + j]) * scd -
               static_cast<double>(shift_term(s_M[c * RS + j], sc)) - log2(s_S[c * RS + j]);
    };
    auto lq2 = [&](int k, int j) {
        const int c = s_can[k * L1 + j];
        return static_cast<double>(s_gq[k * L + j]) * scd -
               static_cast<double>(shift_term(s_M[c * RS + L1 + j], sc)) -
               log2(s_S[c * RS + L1 + j]);
    };
    // Whether node (c, j)'s list is likely to fit: of NT tokens spread evenly
    // over the target row, at most a tenth have p >= 2^-kListCut (a list keeps
    // a subset of those).  Flat rows (high temperature) keep most tokens and
    // would only fill their lists and overflow.
    auto sparse_row = [&](int c, int j) {
        const float lim = static_cast<float>(log2(s_S[c * RS + j]) - kListCut);
        const int v = static_cast<int>(static_cast<long long>(tid) * V / NT);
        const float y = expo(RD(trow(c, j), V).at(v), sc, shift_term(s_M[c * RS + j], sc));
        return __syncthreads_count(y >= lim) <= NT / 10;
    };
    auto node_sweep = [&](int c, int j, double alpha, double beta) {
        SweepRows sr;
        sr.MPc = shift_term(s_M[c * RS + j], sc);
        sr.MQc = shift_term(s_M[c * RS + L1 + j], sc);
        sr.set(alpha, s_S[c * RS + j], beta, s_S[c * RS + L1 + j]);
        return sr;
    };

    int tau = -1, kstar = -1, y = -1, flags = 0, rows = 0;
    double Zp = NAN;
    double rho = 1.0, cc = 1.0;   // SpecTr: scaling factor and tries at the last node
    bool suspend = false;
    int own = 0, nH = 0, k0 = 0, list_tries = 1;
    double alpha = 1.0, beta = 0.0, N = 1.0, tie = INFINITY;
    if (A.round == 2) {
        k0 = ws->k_next;
        tau = ws->tau;
        own = ws->own;
        kstar = ws->kstar;
        nH = ws->nH;
        flags = ws->flags;
        rows = ws->rows;
        list_tries = ws->list_tries;
        tie = ws->tie;
        alpha = ws->alpha;
        beta = ws->beta;
        N = ws->N;
        for (int i = tid; i < nH; i += NT) s_H[i] = ws->H[i];
        __syncthreads();
    }
    rows += streamed;

    // node list of the current node (list_node: the node it serves, -1 none);
    // list_built: the node a list was last built at; a request stops building
    // (list_tries, kept across rounds) once its sampled row looked flat or a
    // list overflowed: its rows share one temperature
    const NodeList<NT> nl(A.nodes, b);
    int lcnt = 0, list_node = -1, list_built = -1;
    double list_out = 0.0;
    if constexpr (SPECTR) {
        if (!bad) {
            if (A.round == 1) {
                tau = 0;
                own = 0;
                kstar = -1;
            }
            int j = tau;
            for (; j < L; ++j) {
                const int cn = s_can[own * L1 + j];
                const int ok = ensure(cn, j);
                if (ok < 0) { suspend = true; break; }
                if (ok == 0) { bad = 1; break; }
                // candidates: the drafts whose first j tokens are the accepted prefix
                int n = 0;
                for (int k = 0; k < K; ++k) {
                    int m2 = 1;
                    for (int t = 0; t < j; ++t) m2 &= (s_x[k * L + t] == s_x[own * L + t]);
                    n += m2;
                }
                rho = 1.0;
                cc = 1.0;
                if (n > 1 && A.rho_bisect)
                    spectr_scale_bisect<NT, RD>(RD(trow(cn, j), V), RD(drow(cn, j), V), nch,
                                                shift_term(s_M[cn * RS + j], sc), s_S[cn * RS + j],
                                                shift_term(s_M[cn * RS + L1 + j], sc),
                                                s_S[cn * RS + L1 + j], sc, n, rho, cc, s_red6);
                else if (n > 1)
                    spectr_scale<NT, RD>(RD(trow(cn, j), V), RD(drow(cn, j), V), nch,
                                         shift_term(s_M[cn * RS + j], sc), s_S[cn * RS + j],
                                         shift_term(s_M[cn * RS + L1 + j], sc),
                                         s_S[cn * RS + L1 + j], sc, n, rho, cc, s_hist, s_red6,
                                         s_br, s_ired);
                if (tid == 0 && A.rho_rec) A.rho_rec[static_cast<long long>(b) * L + j] = rho;
                int acc = -1;
                for (int k = 0; k < K && acc < 0; ++k) {
                    int m2 = 1;
                    for (int t = 0; t < j; ++t) m2 &= (s_x[k * L + t] == s_x[own * L + t]);
                    if (!m2) continue;
                    double h = ratio_log2(lp2(k, j), lq2(k, j)) / rho;
                    if (h > 1.0) h = 1.0;
                    const double u = static_cast<double>(A.ua[bKL + k * L + j]);
                    if (tid == 0 && A.accept_prob)
                        A.accept_prob[bKL + k * L + j] = static_cast<float>(h);
                    tie = fmin(tie, fabs(u - h));
                    // h's error: two row sums and rho (within 7.4e-7 relative of the
                    // fp64 search), four times over
                    if (tid == 0 && A.dec)
                        A.dec[bKL + k * L + j] =
                            kDecMade | (u < h ? kDecAccept : 0) |
                            (fabs(u - h) >= kNearTie + 4.0 * h * (4.0 * kExpEps + 1e-6) ? kDecCertain
                                                                                      : 0);
                    if (u < h) acc = k;
                }
                if (acc < 0) break;
                own = acc;
                kstar = acc;
            }
            tau = j;
        }
    } else if (!bad) {
        if (A.method == kMethodToken) {
            tau = L;
            for (int j = 0; j < L; ++j) {
                if (ensure(0, j) != 1) { bad = 1; break; }
                double a = ratio_log2(lp2(0, j), lq2(0, j));
                if (a > 1.0) a = 1.0;
                const double u = static_cast<double>(A.ua[bKL + j]);
                if (tid == 0 && A.accept_prob) A.accept_prob[bKL + j] = static_cast<float>(a);
                tie = fmin(tie, fabs(u - a));
                if (!(u < a)) { tau = j; break; }
            }
            kstar = tau > 0 ? 0 : -1;
            beta = 1.0;   // token-level residual max(p - q, 0)
        } else {
            if (A.round == 1) tau = 0;
            for (int k = k0; k < K && tau < L; ++k) {
                int match = 1;
                for (int t = 0; t < tau; ++t) match &= (s_x[k * L + t] == s_x[own * L + t]);
                if (!match) continue;
                const int x = s_x[k * L + tau];
                int dup = 0;
                for (int i = 0; i < nH; ++i) dup |= (s_H[i] == x);
                const int cn = s_can[own * L1 + tau];
                int ok = ensure(cn, tau);
                for (int j = tau + 1; j < L && ok == 1 && !dup; ++j) ok = ensure(s_can[k * L1 + j], j);
                if (ok < 0) { suspend = true; k0 = k; break; }
                if (ok == 0) { bad = 1; break; }
                bool rejected = true;
                if (!dup) {
                    // weight chain: first position against the node residual omega/N
                    const double ps = exp2(lp2(k, tau));
                    const double qs = exp2(lq2(k, tau));
                    const double om = fmax(alpha * ps - beta * qs, 0.0);
                    __syncthreads();   // previous readers of s_w are done
                    if (tid == 0) {
                        const double raw = (qs > 0.0) ? om / N / qs : (om > 0.0 ? INFINITY : 0.0);
                        double w = fmin(raw, 1.0);
                        s_w[tau + 1] = w;
                        // omega(x) cancels when alpha p ~ beta q; N and q add a sum's error
                        double rel = (om > 0.0 ? (alpha * ps + beta * qs) * 2.0 * kExpEps / om : 0.0) +
                                     6.0 * kExpEps;
                        rel = clamp_err(raw, rel);
                        s_wrel[tau + 1] = rel;
                        for (int j = tau + 1; j < L; ++j) {
                            const double r = ratio_log2(lp2(k, j), lq2(k, j));
                            rel = clamp_err(w * r, rel + 4.0 * kExpEps);   // two row sums per ratio
                            w = chain_step(w, r);
                            s_w[j + 1] = w;
                            s_wrel[j + 1] = rel;
                        }
                    }
                    __syncthreads();
                    int acc = 0;
                    double Racc = 0.0;
                    for (int m = L; m > tau; --m) {
                        const double u = static_cast<double>(A.ua[bKL + k * L + m - 1]);
                        const double wm = s_w[m];
                        // first-order error of w_m (exact where the chain clamped at 1
                        // with room to spare)
                        const double dw = wm * s_wrel[m];
                        double h, eh = dw;
                        if (m == L) {
                            h = wm;
                        } else {
                            if (!(u < wm)) {              // h_m <= w_m: rejects without a sweep
                                tie = fmin(tie, u - wm);
                                if (u - wm < 4.0 * dw) tie = 0.0;   // within its error
                                if (tid == 0 && A.dec)
                                    A.dec[bKL + k * L + m - 1] =
                                        kDecMade | (u - wm >= kNearTie + 4.0 * dw ? kDecCertain : 0);
                                continue;
                            }
                            const int cm = s_can[k * L1 + m];
                            const SweepRows sr = node_sweep(cm, m, wm, 1.0);
                            const RD P(trow(cm, m), V), Q(drow(cm, m), V);
                            const double R =
                                sweep_mass<NT, RD, true>(P, Q, nch, sr, sc, s_H, 0, s_red);
                            const double d = R + 1.0 - wm;
                            h = d > 0.0 ? R / d : 1.0;
                            Racc = R;
                            // h = R / (R + 1 - w): dh = ((1 - w) dR + R dw) / d^2
                            const double dR = dw + (wm + 1.0) * 2.0 * kExpEps;
                            eh = d > 0.0 ? ((1.0 - wm) * dR + R * dw) / (d * d) : INFINITY;
                        }
                        if (tid == 0 && A.accept_prob)
                            A.accept_prob[bKL + k * L + m - 1] = static_cast<float>(h);
                        tie = fmin(tie, fabs(u - h));
                        if (fabs(u - h) < 4.0 * eh) tie = 0.0;   // within its error estimate
                        if (A.accept_prob && eh > kDiagEh) tie = 0.0;   // h reported to 1e-5
                        if (tid == 0 && A.dec)
                            A.dec[bKL + k * L + m - 1] =
                                kDecMade | (u < h ? kDecAccept : 0) |
                                (fabs(u - h) >= kNearTie + 4.0 * eh &&
                                         !(A.accept_prob && eh > kDiagEh)
                                     ? kDecCertain
                                     : 0);
                        if (u < h) { acc = m; break; }
                    }
                    if (acc > 0) {
                        rejected = false;
                        tau = acc;
                        own = k;
                        kstar = k;
                        nH = 0;
                        if (tau < L) {
                            alpha = s_w[tau];
                            beta = 1.0;
                            N = Racc;
                        }
                    }
                }
                bool mass_known = true;
                if (rejected) {
                    if (!dup) {
                        if (tid == 0) s_H[nH] = x;
                        ++nH;
                        __syncthreads();
                    }
                    beta += N;
                    // The new mass is needed only if a later draft is examined at this
                    // node; otherwise the correction's inverse CDF sums the residual
                    // itself (and falls back to the node's target on zero mass, as the
                    // degenerate reset below would).
                    int later = 0;
                    for (int k2 = k + 1; k2 < K && later < 2; ++k2) {
                        int m2 = 1;
                        for (int t = 0; t < tau; ++t) m2 &= (s_x[k2 * L + t] == s_x[own * L + t]);
                        later += m2;
                    }
                    if (later) {
                        const SweepRows sr = node_sweep(cn, tau, alpha, beta);
                        const int node = cn * L1 + tau;
                        bool have = false;
                        if (list_node == node) {
                            // the list's left-out weight must stay below 2^-30 of the mass
                            const double Nl = sweep_mass_list<NT>(nl, lcnt, sr, s_H, nH, s_red);
                            have = list_out <= 0x1p-30 * Nl;
                            if (have) N = Nl;
                            else list_node = -1;
                        }
                        if (!have) {
                            const RD P(trow(cn, tau), V), Q(drow(cn, tau), V);
                            bool build = A.nodes && later > 1 && list_tries > 0 && node != list_built;
                            if (build && !sparse_row(cn, tau)) {
                                build = false;
                                list_tries = 0;   // the request's rows share a temperature
                            }
                            if (build) {
                                // two or more drafts still to come at this node: keep a list
                                // of the tokens that can still carry weight
                                const float keep =
                                    static_cast<float>(ldexp(s_S[cn * RS + tau], -kListCut));
                                bool ovf;
                                N = sweep_mass_build<NT, RD>(P, Q, nch, sr, sc, s_H, nH, keep, nl,
                                                             &lcnt, &list_out, &ovf, s_red4);
                                list_built = node;
                                if (ovf) --list_tries;
                                else list_node = node;
                            } else {
                                N = sweep_mass<NT, RD, true>(P, Q, nch, sr, sc, s_H, nH, s_red);
                            }
                        }
                    } else {
                        mass_known = false;
                    }
                }
                if (tau < L && mass_known && !(N > 0.0)) {
                    flags |= kFlagDegenerate;   // only rounding empties a residual
                    alpha = 1.0;
                    beta = 0.0;
                    N = 1.0;
                    nH = 0;
                    list_node = -1;   // beta fell: the list's bound no longer holds
                    list_built = -1;
                }
            }
        }
    }

    if (suspend) {
        // Flag every node row at positions tau..L-1 of the drafts that share the
        // accepted prefix; the next launch of the statistics kernel streams them.
        // Every draft examined after this point shares that prefix, so the walk
        // resumes with all the rows it can read.
        for (int i = tid; i < KL; i += NT) {
            const int c = i / L, j = i % L;
            if (j < tau || s_can[c * L1 + j] != c || s_have[c * L1 + j]) continue;
            int match = 1;
            for (int t = 0; t < tau; ++t) match &= (s_x[c * L + t] == s_x[own * L + t]);
            if (match) need[i] = 1;
        }
        __syncthreads();
        if (tid == 0) {
            int n = 0;
            for (int i = 0; i < KL; ++i) n += need[i];
            unsigned base = atomicAdd(A.list_count, static_cast<unsigned>(2 * n));
            for (int i = 0; i < KL; ++i) {
                if (!need[i]) continue;
                A.list[base].b = b;
                A.list[base].kjt = 2 * i + 1;
                A.list[base + 1].b = b;
                A.list[base + 1].kjt = 2 * i;
                base += 2;
            }
        }
        if (tid == 0) {
            ws->status = kStateSuspended;
            ws->k_next = k0;
            ws->tau = tau;
            ws->own = own;
            ws->kstar = kstar;
            ws->nH = nH;
            ws->flags = flags;
            ws->rows = rows;
            ws->list_tries = list_tries;
            ws->tie = tie;
            ws->alpha = alpha;
            ws->beta = beta;
            ws->N = N;
        }
        for (int i = tid; i < nH; i += NT) ws->H[i] = s_H[i];
        return;
    }

    // 5. correction token
    double dm = INFINITY;   // the draw's margin (distance of u Z to a boundary, over Z)
    if (!bad) {
        const double u = static_cast<double>(ucf);
        if (tau == L) {
            const int cb = s_can[(kstar < 0 ? 0 : kstar) * L1 + L];
            const RD P(trow(cb, L), V);
            const float M = sweep_rowmax<NT, RD>(P, nch, s_fred);
            SweepRows sr;
            sr.MPc = shift_term(M, sc);
            sr.MQc = 0.0f;
            sr.a = 1.0;
            sr.r = 0.0f;
            double Z;
            y = (M > -INFINITY && M < INFINITY)
                    ? sweep_icdf<NT, RD, false>(P, P, nch, sr, sc, s_H, 0, u, &Z, s_tile, s_red,
                                                s_red4, s_ired, &dm)
                    : -1;
            Zp = 1.0;
            if (y < 0) bad = 1;   // the target row after the block is not a distribution
        } else {
            const int cn = s_can[own * L1 + tau];
            SweepRows sr = node_sweep(cn, tau, alpha, beta);
            const RD P(trow(cn, tau), V), Q(drow(cn, tau), V);
            double Z;
            if constexpr (SPECTR) {
                // max(p - c q, (1 - c/rho) p): the residual after n tries
                sr = node_sweep(cn, tau, 1.0, cc);
                sr.g = static_cast<float>(fmax(1.0 - cc / rho, 0.0));   // over a = 1 / S_P
                y = sweep_icdf<NT, RD, true, true>(P, Q, nch, sr, sc, s_H, 0, u, &Z, s_tile, s_red,
                                                   s_red4, s_ired, &dm);
            } else {
                // from the node's list when it has one, its left-out weight is below
                // 2^-30 of the mass and the row fits the draw's segment table
                const int ntile = (nch + NT - 1) / NT;
                y = -1;
                if (list_node == cn * L1 + tau && ntile <= kListTiles) {
                    y = sweep_icdf_list<NT>(nl, lcnt, sr, s_H, nH, u, ntile, &Z, s_lseg,
                                            s_lstart, s_ired, s_red, &dm);
                    if (!(list_out <= 0x1p-30 * Z)) y = -1;
                }
                if (y < 0)
                    y = sweep_icdf<NT, RD, true>(P, Q, nch, sr, sc, s_H, nH, u, &Z, s_tile, s_red,
                                                 s_red4, s_ired, &dm);
            }
            Zp = Z;
            if (y < 0) {
                flags |= kFlagDegenerate;
                sr.a = 1.0 / s_S[cn * RS + tau];
                sr.r = 0.0f;
                y = sweep_icdf<NT, RD, false>(P, P, nch, sr, sc, s_H, 0, u, &Z, s_tile, s_red,
                                              s_red4, s_ired, &dm);
                Zp = Z;
            }
        }
    }

    tie = fmin(tie, dm);
    if (tie < kNearTie) flags |= kFlagNearTie;
    if (tid == 0) {
        if (bad) {
            tau = -1;
            kstar = -1;
            y = -1;
            flags = kFlagInvalid;
            Zp = NAN;
        }
        ws->status = kStateDone;
        if (!bad && (flags & kFlagNearTie))
            A.redo_list[atomicAdd(A.redo_count, 1u)] =
                b | ((flags & kFlagDegenerate) ? kListNoReplay : 0);
        A.accept_len[b] = tau;
        A.draft_index[b] = kstar;
        A.correction[b] = y;
        if (A.flags) A.flags[b] = flags;
        if (A.resid_mass) A.resid_mass[b] = static_cast<float>(Zp);
        if (A.rows_streamed) A.rows_streamed[b] = rows;
    }
    if (A.row_lse) {
        // diagnostics: the statistics kernel streamed every node row
        float *o = A.row_lse + static_cast<long long>(b) * K * RS;
        for (int i = tid; i < K * RS; i += NT) {
            const int k = i / RS, r = i % RS;
            const int j = r <= L ? r : r - L - 1;
            const int c = s_can[k * L1 + j];
            float v = NAN;
            if (!bad) {
                const RowStat a = st[c * RS + r];
                // ln sum_v exp(l_v / T): the shift in the exact scale plus the
                // rounding of its fp32 product, which the sum carries
                const double M = static_cast<double>(a.shift);
                const double off = static_cast<double>(shift_term(a.shift, sc)) - M * scd;
                v = static_cast<float>((M * (1.4426950408889634 / static_cast<double>(T)) + off +
                                        log2(a.sum)) *
                                       0.6931471805599453);
            }
            o[i] = v;
        }
    }
}

}  // namespace sv
