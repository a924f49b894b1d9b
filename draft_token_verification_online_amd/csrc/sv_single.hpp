// sv_single.hpp -- single-draft verification (K = 1) split across the vocabulary.
//
// With one draft every row a request can read is known in advance: target rows
// 0..L and draft rows 0..L-1.  The rule needs their softmax statistics, one
// gathered logit per row, and then O(V) residual sums only at the positions the
// decision can reach.  A small batch (B = 64 requests of V = 32 000) gives one
// workgroup per request far too little parallelism to fill 256 CUs, so here
// every O(V) pass is split into slices of kSliceChunks chunks and spread over
// the grid:
//
//   single_stats_kernel   one workgroup per (request, row, slice): the slice's
//                         maximum and sum of exponentials, from registers (one
//                         HBM read of every logit);
//   single_prep_kernel    one workgroup per request: combines the row statistics,
//                         gathers the drafted tokens' logits, runs the weight
//                         chain in fp64 and marks the positions the decision can
//                         reach (SinglePrep, ~1 KB per request);
//   single_partial_kernel one workgroup per (request, position m = 0..L, slice):
//                         if the decision can reach position m, sums the slice
//                         of the residual at m (or, at m = L, of the bonus row);
//   single_final_kernel   one workgroup per request: the decision from those
//                         sums, and the correction, found among the slice sums
//                         and rescanned in the one slice that holds the
//                         inverse-CDF crossing; a request with a decision within
//                         its fp32 error of its threshold is taken again in fp64
//                         (sv_redo.hpp) by the same workgroup.
// (The launch boundaries publish each step's sums to the next.  Handing them
// over inside one launch -- the last workgroup of a request to finish taking the
// decision -- needs a device-scope fence per workgroup, which on this chip
// writes back and invalidates the XCD's L2 and cost ~100 us per call here.)
//
// Rules (the same as the per-request walk, see sv_walk.hpp and the header):
//  token level  -- accept X_j iff u_j < min(1, p_j(X_j)/q_j(X_j)); stop at the
//                  first rejection j and draw from max(p_j - q_j, 0); with all L
//                  accepted draw from the target row L;
//  block (GBV)  -- w_0 = 1, w_i = min(w_{i-1} p/q, 1); test m = L (h = w_L), then
//                  m = L-1..1 with h_m = R_m / (R_m + 1 - w_m),
//                  R_m = sum_v max(w_m p_m - q_m, 0); the first success sets tau;
//                  draw from max(w_tau p_tau - q_tau, 0), or from row L at tau = L.
//                  A test with u_m >= w_m is settled without R_m (h_m <= w_m).
// Greedy block verification is the single-draft verifier of the SpecTr-GBV page
// (section 1); the token rule is standard speculative sampling.
#pragma once

#include "sv_device.hpp"
#include "sv_redo.hpp"
#include "sv_rowstats.hpp"
#include "sv_walk.hpp"

namespace sv {

constexpr int kSingleThreads = 256;
constexpr int kSliceChunksPerThread = 8;
constexpr int kSliceChunks = kSliceChunksPerThread * kSingleThreads;   // 16384 tokens

// Statistics of one slice of a row: its maximum and sum_v 2^(x c - K_s) with
// K_s = shift_term(maximum).
struct SliceStat {
    float shift;
    float pad;
    double sum;
};

struct SingleArgs {
    const void *tgt;        // [B][L+1][V]
    const void *drf;        // [B][L][V]
    const int32_t *tok;     // [B][L]
    const float *temp;      // [B]
    const float *ua;        // [B][L]
    const float *uc;        // [B]
    SliceStat *part;        // [B][2L+1][NS]: rows in the order target 0..L, draft 0..L-1
    double *rpart;          // [B][L+1][NS]: residual (m < L) or bonus-row (m = L) slice sums
    struct SinglePrep *prep;   // [B]: each request's combined statistics and chain
    int B, L, V, NS;
    int method;             // kMethodToken (token level) or anything else (block)
    int32_t *accept_len, *draft_index, *correction, *flags, *rows_streamed;
    float *row_lse, *accept_prob, *resid_mass;
};

// omega / a of 8 elements of a row pair: max(eP - r eQ, 0), eP = 2^(x c - KP);
// without Q (the bonus row, or a target row drawn from directly) just eP.
template <bool HAS_Q>
__device__ __forceinline__ void resid8(const float xp[8], const float xq[8], float KP, float KQ,
                                       float r, const Scale &c, float w[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float ep = fast_exp2(expo(xp[e], c, KP));
        if (HAS_Q) {
            const float eq = fast_exp2(expo(xq[e], c, KQ));
            w[e] = fmaxf(fmaf(-r, eq, ep), 0.0f);
        } else {
            w[e] = ep;
        }
    }
}

template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void single_stats_kernel(SingleArgs A) {
    __shared__ float s_fred[NT / kWave];
    __shared__ double s_red[NT / kWave];
    const int tid = threadIdx.x;
    const int L = A.L, V = A.V, NS = A.NS, RS = 2 * L + 1;
    const int nch = (V + kChunk - 1) / kChunk;
    const long long items = static_cast<long long>(A.B) * RS * NS;
    for (long long it = blockIdx.x; it < items; it += gridDim.x) {
        const int s = static_cast<int>(it % NS);
        const long long br = it / NS;
        const int r = static_cast<int>(br % RS);
        const int b = static_cast<int>(br / RS);
        const E *row = r <= L
            ? static_cast<const E *>(A.tgt) + (static_cast<long long>(b) * (L + 1) + r) * V
            : static_cast<const E *>(A.drf) + (static_cast<long long>(b) * L + (r - L - 1)) * V;
        const RD R(row, V);
        const Scale c = temp_scale(A.temp[b]);
        const int c0 = s * kSliceChunks;
        const int nc = min(kSliceChunks, nch - c0);
        typename RD::Raw raw[kSliceChunksPerThread];
#pragma unroll
        for (int i = 0; i < kSliceChunksPerThread; ++i)
            if (i * NT + tid < nc) raw[i] = R.raw_once(c0 + i * NT + tid);
        // the slice's maximum, then its exponentials (the chunks stay packed in
        // registers and are unpacked for each pass)
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < kSliceChunksPerThread; ++i) {
            if (i * NT + tid < nc) {
                float x[8];
                RD::unpack(raw[i], x);
                m = fmaxf(m, max8(x));
            }
        }
        const float M = block_max<NT>(m, s_fred);
        const float K = shift_term(fmaxf(M, -3.402823466e38f), c);
        double acc = 0.0;
#pragma unroll
        for (int i = 0; i < kSliceChunksPerThread; ++i) {
            if (i * NT + tid < nc) {
                float x[8], e[8];
                RD::unpack(raw[i], x);
#pragma unroll
                for (int k = 0; k < 8; ++k) e[k] = fast_exp2(expo(x[k], c, K));
                acc += static_cast<double>(sum8(e));
            }
        }
        const double S = block_sum<NT>(acc, s_red);
        if (tid == 0) {
            SliceStat st;
            st.shift = M;
            st.pad = 0.0f;
            st.sum = S;
            A.part[br * NS + s] = st;
        }
    }
}

// What every launch after the statistics needs of request b, in LDS: the rows'
// combined statistics, the drafted tokens' logits, the weight chain and which
// positions' residual sums the decision can reach.
struct SinglePrep {
    float M[2 * 16 + 1], K[2 * 16 + 1];
    double S[2 * 16 + 1];
    float gp[16], gq[16];
    double lr[16];      // log2 p - log2 q of the drafted token at position j
    double w[17];       // GBV's weights w_0..w_L
    double wrel[17];    // their relative error estimates (0 where clamped at 1 for certain)
    int need[17];       // positions whose slice sums the decision can use
    int tau;            // token level: the first rejected position (L: none)
    int bad;
    int pad[1];
};
static_assert(sizeof(SinglePrep) % 16 == 0, "whole words");

template <int NT, typename RD, typename E>
__device__ void single_prepare(const SingleArgs &A, int b, const Scale &c, double scd,
                               SinglePrep &P) {
    constexpr int NW = NT / kWave;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wv = tid / kWave;
    const int L = A.L, V = A.V, NS = A.NS, RS = 2 * L + 1, L1 = L + 1;
    const float T = A.temp[b];
    const E *tgt = static_cast<const E *>(A.tgt) + static_cast<long long>(b) * L1 * V;
    const E *drf = static_cast<const E *>(A.drf) + static_cast<long long>(b) * L * V;
    int bad = !(T > 0.0f) || !isfinite(T);
    for (int j = tid; j < L; j += NT) {
        const int x = A.tok[static_cast<long long>(b) * L + j];
        const float u = A.ua[static_cast<long long>(b) * L + j];
        bad |= (x < 0 || x >= V) || !(u >= 0.0f && u < 1.0f);
        if (x >= 0 && x < V) {
            P.gp[j] = RD(tgt + static_cast<long long>(j) * V, V).at(x);
            P.gq[j] = RD(drf + static_cast<long long>(j) * V, V).at(x);
        }
    }
    const float ucf = A.uc[b];
    bad |= !(ucf >= 0.0f && ucf < 1.0f);
    bad = __syncthreads_or(bad);
    for (int r = wv; r < RS; r += NW) {   // one wave per row, lanes over its slices
        const SliceStat *ps = A.part + (static_cast<long long>(b) * RS + r) * NS;
        float mx = -INFINITY;
        for (int q = lane; q < NS; q += kWave) mx = fmaxf(mx, ps[q].shift);
        mx = wave_max(mx);
        const float K = shift_term(fmaxf(mx, -3.402823466e38f), c);
        double sum = 0.0;
        for (int q = lane; q < NS; q += kWave) {
            const SliceStat st = ps[q];
            const float Ks = shift_term(fmaxf(st.shift, -3.402823466e38f), c);
            sum += st.sum * exp2(static_cast<double>(Ks) - static_cast<double>(K));
        }
        sum = wave_sum(sum);
        if (lane == 0) {
            P.M[r] = mx;
            P.K[r] = K;
            P.S[r] = sum;
        }
    }
    __syncthreads();
    // the drafted tokens' log-ratios, one lane per position (fp64, from the
    // exponents as the sweeps form them)
    if (!bad && tid < L) {
        const int j = tid;
        const double lp = static_cast<double>(P.gp[j]) * scd - static_cast<double>(P.K[j]) -
                          log2(P.S[j]);
        const double lq = static_cast<double>(P.gq[j]) * scd - static_cast<double>(P.K[L1 + j]) -
                          log2(P.S[L1 + j]);
        P.lr[j] = lq == -INFINITY ? (lp > -INFINITY ? INFINITY : -INFINITY) : lp - lq;
    }
    __syncthreads();
    if (tid == 0) {
        auto ok = [&](int r) { return isfinite(P.M[r]) && P.S[r] > 0.0 && isfinite(P.S[r]); };
        const float *u = A.ua + static_cast<long long>(b) * L;
        for (int j = 0; j <= L; ++j) P.need[j] = 0;
        P.tau = L;
        if (A.method == kMethodToken) {
            for (int j = 0; j < L && !bad; ++j) {
                if (!(ok(j) && ok(L1 + j))) { bad = 1; break; }
                double a = P.lr[j] == -INFINITY ? 0.0 : exp2(P.lr[j]);
                if (a > 1.0) a = 1.0;
                if (!(static_cast<double>(u[j]) < a)) { P.tau = j; break; }
            }
            if (!bad) P.need[P.tau] = 1;
        } else {
            for (int j = 0; j < L && !bad; ++j)
                if (!(ok(j) && ok(L1 + j))) bad = 1;
            if (!bad) {
                // first position: the target itself is the residual (alpha = 1,
                // beta = 0, N = 1); deeper ones the chain of likelihood ratios
                const double r0 = P.lr[0] == -INFINITY ? 0.0 : exp2(P.lr[0]);
                double w = fmin(r0, 1.0), rel = clamp_err(r0, 4.0 * kExpEps);
                P.w[0] = 1.0;
                P.w[1] = w;
                P.wrel[1] = rel;
                for (int j = 1; j < L; ++j) {
                    const double r = P.lr[j] == -INFINITY ? 0.0 : exp2(P.lr[j]);
                    rel = clamp_err(w * r, rel + 4.0 * kExpEps);   // two row sums per ratio
                    w = chain_step(w, r);
                    P.w[j + 1] = w;
                    P.wrel[j + 1] = rel;
                }
                if (static_cast<double>(u[L - 1]) < P.w[L]) {
                    P.need[L] = 1;
                } else {
                    P.need[0] = 1;   // tau = 0 is reachable: its residual
                    for (int j = 1; j < L; ++j)
                        P.need[j] = static_cast<double>(u[j - 1]) < P.w[j];
                }
            }
        }
        P.bad = bad;
    }
    __syncthreads();
}

// One workgroup per request: its SinglePrep, once, for the two launches after it.
template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void single_prep_kernel(SingleArgs A) {
    __shared__ SinglePrep P;
    for (int b = blockIdx.x; b < A.B; b += gridDim.x) {
        const Scale c = temp_scale(A.temp[b]);
        single_prepare<NT, RD, E>(A, b, c, scale64(c), P);
        const unsigned *src = reinterpret_cast<const unsigned *>(&P);
        unsigned *dst = reinterpret_cast<unsigned *>(A.prep + b);
        for (int i = threadIdx.x; i < static_cast<int>(sizeof(SinglePrep) / 4); i += NT)
            dst[i] = src[i];
        __syncthreads();
    }
}

// A request's SinglePrep into LDS (block-uniform call).
template <int NT>
__device__ __forceinline__ void load_prep(const SingleArgs &A, int b, SinglePrep &P) {
    const unsigned *src = reinterpret_cast<const unsigned *>(A.prep + b);
    unsigned *dst = reinterpret_cast<unsigned *>(&P);
    for (int i = threadIdx.x; i < static_cast<int>(sizeof(SinglePrep) / 4); i += NT)
        dst[i] = src[i];
    __syncthreads();
}

// One workgroup per (request, position m = 0..L, slice): the slice's sum of the
// residual at m (m < L: max(w_m p_m - q_m, 0) over w_m / S_P) or of the bonus
// row's exponentials (m = L), when the decision can reach it.
template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void single_partial_kernel(SingleArgs A) {
    constexpr int NW = NT / kWave;
    __shared__ SinglePrep P;
    __shared__ double s_red[NW];
    const int tid = threadIdx.x;
    const int L = A.L, V = A.V, NS = A.NS, L1 = L + 1;
    const int nch = (V + kChunk - 1) / kChunk;
    const bool token = A.method == kMethodToken;
    const long long items = static_cast<long long>(A.B) * L1 * NS;
    for (long long it = blockIdx.x; it < items; it += gridDim.x) {
        const int s = static_cast<int>(it % NS);
        const int m = static_cast<int>((it / NS) % L1);
        const int b = static_cast<int>(it / (static_cast<long long>(NS) * L1));
        // most items are not needed: check the request's flags before anything else
        const SinglePrep *G = A.prep + b;
        if (G->bad || !G->need[m]) continue;   // block-uniform
        const Scale c = temp_scale(A.temp[b]);
        load_prep<NT>(A, b, P);
        const E *tgt = static_cast<const E *>(A.tgt) + static_cast<long long>(b) * L1 * V;
        const E *drf = static_cast<const E *>(A.drf) + static_cast<long long>(b) * L * V;
        const int c0 = s * kSliceChunks;
        const int nc = min(kSliceChunks, nch - c0);
        double acc = 0.0;
        if (m == L) {
            const RD R(tgt + static_cast<long long>(L) * V, V);
            typename RD::Raw rp[kSliceChunksPerThread];
#pragma unroll
            for (int i = 0; i < kSliceChunksPerThread; ++i)
                if (i * NT + tid < nc) rp[i] = R.raw(c0 + i * NT + tid);
#pragma unroll
            for (int i = 0; i < kSliceChunksPerThread; ++i) {
                if (i * NT + tid < nc) {
                    float xp[8], w[8];
                    RD::unpack(rp[i], xp);
                    resid8<false>(xp, xp, P.K[L], 0.0f, 0.0f, c, w);
                    acc += static_cast<double>(sum8(w));
                }
            }
        } else {
            const double wm = token ? 1.0 : P.w[m];
            const float r = static_cast<float>(fmin(P.S[m] / (wm * P.S[L1 + m]), 3.402823466e38));
            const RD Rp(tgt + static_cast<long long>(m) * V, V), Rq(drf + static_cast<long long>(m) * V, V);
            typename RD::Raw rp[kSliceChunksPerThread], rq[kSliceChunksPerThread];
#pragma unroll
            for (int i = 0; i < kSliceChunksPerThread; ++i) {
                if (i * NT + tid < nc) {
                    rp[i] = Rp.raw(c0 + i * NT + tid);
                    rq[i] = Rq.raw(c0 + i * NT + tid);
                }
            }
#pragma unroll
            for (int i = 0; i < kSliceChunksPerThread; ++i) {
                if (i * NT + tid < nc) {
                    float xp[8], xq[8], w[8];
                    RD::unpack(rp[i], xp);
                    RD::unpack(rq[i], xq);
                    resid8<true>(xp, xq, P.K[m], P.K[L1 + m], r, c, w);
                    acc += static_cast<double>(sum8(w));
                }
            }
        }
        const double z = block_sum<NT>(acc, s_red);
        if (tid == 0) A.rpart[(static_cast<long long>(b) * L1 + m) * NS + s] = z;
    }
}

// One workgroup per request: the decision from the slice sums, then the
// correction, drawn by finding the slice that holds u Z and rescanning it.
template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void single_final_kernel(SingleArgs A) {
    constexpr int NW = NT / kWave;
    __shared__ SinglePrep P;
    __shared__ double s_zs[kMaxV / kSliceChunks / kChunk + 1];   // slice sums of the draw
    __shared__ double s_red[NW];
    __shared__ int s_ired[NW];
    __shared__ double s_z[2];
    __shared__ double s_zsum[kMaxL + 1];   // residual sum of each position
    __shared__ float s_u[kMaxL];
    __shared__ RedoShared s_redo;
    const int tid = threadIdx.x;
    const int L = A.L, V = A.V, NS = A.NS, RS = 2 * L + 1, L1 = L + 1;
    const int nch = (V + kChunk - 1) / kChunk;
    const bool token = A.method == kMethodToken;
    RedoArgs ra = {};
    ra.tgt = A.tgt;
    ra.drf = A.drf;
    ra.tok = A.tok;
    ra.temp = A.temp;
    ra.ua = A.ua;
    ra.uc = A.uc;
    ra.B = A.B;
    ra.K = 1;
    ra.L = L;
    ra.V = V;
    ra.method = A.method;
    ra.accept_len = A.accept_len;
    ra.draft_index = A.draft_index;
    ra.correction = A.correction;
    ra.flags = A.flags;
    ra.accept_prob = A.accept_prob;
    ra.resid_mass = A.resid_mass;
    for (int b = blockIdx.x; b < A.B; b += gridDim.x) {
        const float T = A.temp[b];
        const Scale c = temp_scale(T);
        const double scd = scale64(c);
        load_prep<NT>(A, b, P);
        const E *tgt = static_cast<const E *>(A.tgt) + static_cast<long long>(b) * L1 * V;
        const E *drf = static_cast<const E *>(A.drf) + static_cast<long long>(b) * L * V;
        auto trow = [&](int j) { return RD(tgt + static_cast<long long>(j) * V, V); };
        auto drow = [&](int j) { return RD(drf + static_cast<long long>(j) * V, V); };
        auto ok = [&](int r) { return isfinite(P.M[r]) && P.S[r] > 0.0 && isfinite(P.S[r]); };
        const double *rp = A.rpart + static_cast<long long>(b) * L1 * NS;
        // every position's uniform and residual sum (its slice sums in slice
        // order) into LDS at once, so the decision loop waits on no load
        if (tid < L1) {
            double z = 0.0;
            for (int q = 0; q < NS; ++q) z += rp[tid * NS + q];
            s_zsum[tid] = z;
        } else if (tid >= kWave && tid < kWave + L) {
            s_u[tid - kWave] = A.ua[static_cast<long long>(b) * L + (tid - kWave)];
        }
        const float *u = s_u;
        auto zsum = [&](int j) { return s_zsum[j]; };
        float *hout = A.accept_prob ? A.accept_prob + static_cast<long long>(b) * L : nullptr;
        if (hout)
            for (int j = tid; j < L; j += NT) hout[j] = NAN;
        __syncthreads();

        // 1. the decision (every thread takes the same one)
        int tau = -1, kstar = -1, y = -1, flags = 0;
        double tie = INFINITY, Zp = NAN;
        int bad = P.bad;
        if (!bad) {
            if (token) {
                tau = P.tau;
                for (int j = 0; j <= tau && j < L; ++j) {
                    double a = P.lr[j] == -INFINITY ? 0.0 : exp2(P.lr[j]);
                    if (a > 1.0) a = 1.0;
                    if (tid == 0 && hout) hout[j] = static_cast<float>(a);
                    tie = fmin(tie, fabs(static_cast<double>(u[j]) - a));
                }
            } else {
                tau = 0;
                for (int mm = L; mm >= 1; --mm) {
                    const double uu = static_cast<double>(u[mm - 1]);
                    const double wm = P.w[mm];
                    // first-order error of w_m (exact where the chain clamped at 1
                    // with room to spare) and of h_m = R / (R + 1 - w_m)
                    const double dw = wm * P.wrel[mm];
                    double h, eh = dw;
                    if (mm == L) {
                        h = wm;
                    } else {
                        if (!(uu < wm)) {   // h_m <= w_m: rejects without its sum
                            tie = fmin(tie, uu - wm);
                            if (uu - wm < 4.0 * dw) tie = 0.0;   // within its error
                            continue;
                        }
                        const double R = wm / P.S[mm] * zsum(mm);
                        const double d = R + 1.0 - wm;
                        h = d > 0.0 ? R / d : 1.0;
                        const double dR = dw + (wm + 1.0) * 2.0 * kExpEps;
                        eh = d > 0.0 ? ((1.0 - wm) * dR + R * dw) / (d * d) : INFINITY;
                    }
                    if (tid == 0 && hout) hout[mm - 1] = static_cast<float>(h);
                    tie = fmin(tie, fabs(uu - h));
                    if (fabs(uu - h) < 4.0 * eh) tie = 0.0;   // within its error estimate
                    if (hout && eh > kDiagEh) tie = 0.0;      // h reported to 1e-5
                    if (uu < h) { tau = mm; break; }
                }
            }
            kstar = tau > 0 ? 0 : -1;
            if (tau == L && !ok(L)) bad = 1;   // the bonus row is not a distribution
        }

        // 2. the correction: inverse CDF over the slices, then the crossing slice
        double dm = INFINITY;
        if (!bad) {
            const double u_c = static_cast<double>(A.uc[b]);
            const int jd = tau;
            bool has_q = tau < L;
            double a = 0.0;
            float r = 0.0f;
            if (has_q) {
                const double wm = token ? 1.0 : P.w[tau];
                a = wm / P.S[tau];
                r = static_cast<float>(fmin(P.S[tau] / (wm * P.S[L1 + tau]), 3.402823466e38));
            }
            double z = zsum(jd);
            bool fallback = false;
            if (has_q && (!(z > 0.0) || !isfinite(z))) {   // zero residual: rounding only
                flags |= kFlagDegenerate;
                fallback = true;
                has_q = false;
            }
            if (fallback) {
                // the node's target row, summed slice by slice here (rare)
                double zt = 0.0;
                const RD Pr = trow(jd);
                for (int q = 0; q < NS; ++q) {
                    double acc = 0.0;
                    const int q0 = q * kSliceChunks, qn = min(kSliceChunks, nch - q0);
                    for (int i = tid; i < qn; i += NT) {
                        float xp[8], w[8];
                        Pr.load(q0 + i, xp);
                        resid8<false>(xp, xp, P.K[jd], 0.0f, 0.0f, c, w);
                        acc += static_cast<double>(sum8(w));
                    }
                    acc = block_sum<NT>(acc, s_red);
                    if (tid == 0) s_zs[q] = acc;
                    zt += acc;
                }
                z = zt;
            } else {
                for (int q = tid; q < NS; q += NT) s_zs[q] = rp[jd * NS + q];
            }
            __syncthreads();
            const double thr = u_c * z;
            // the crossing slice
            double base = 0.0, cum = 0.0;
            int sc = -1, slast = -1;
            for (int q = 0; q < NS; ++q) {
                const double zq = s_zs[q];
                if (sc < 0 && cum + zq > thr) { sc = q; base = cum; }
                cum += zq;
                if (zq > 0.0) slast = q;
            }
            const bool past = sc < 0;
            if (past) sc = slast;
            if (sc < 0) {   // no slice of positive weight (cannot happen for a valid row)
                bad = 1;
            } else {
                // rescan slice sc: thread t takes its kSliceChunksPerThread
                // consecutive chunks, all loads issued at once, and keeps their
                // weights in registers for the recount
                const int q0 = sc * kSliceChunks, qn = min(kSliceChunks, nch - q0);
                const RD Pr = trow(jd), Qr = has_q ? drow(jd) : trow(jd);
                const float KP = P.K[jd], KQ = has_q ? P.K[L1 + jd] : 0.0f;
                float wv[kSliceChunksPerThread][8];   // omega / a (the sweeps' own arithmetic)
                {
                    typename RD::Raw rp[kSliceChunksPerThread], rq[kSliceChunksPerThread];
#pragma unroll
                    for (int i = 0; i < kSliceChunksPerThread; ++i) {
                        const int q = kSliceChunksPerThread * tid + i;
                        if (q < qn) {
                            rp[i] = Pr.raw(q0 + q);
                            if (has_q) rq[i] = Qr.raw(q0 + q);
                        }
                    }
#pragma unroll
                    for (int i = 0; i < kSliceChunksPerThread; ++i) {
                        const int q = kSliceChunksPerThread * tid + i;
                        if (q < qn) {
                            float xp[8], xq[8];
                            RD::unpack(rp[i], xp);
                            if (has_q) {
                                RD::unpack(rq[i], xq);
                                resid8<true>(xp, xq, KP, KQ, r, c, wv[i]);
                            } else {
                                resid8<false>(xp, xp, KP, 0.0f, 0.0f, c, wv[i]);
                            }
                        } else {
#pragma unroll
                            for (int e = 0; e < 8; ++e) wv[i][e] = 0.0f;
                        }
                    }
                }
                double tsum = 0.0;
                int lastpos = -1;
#pragma unroll
                for (int i = 0; i < kSliceChunksPerThread; ++i) {
                    const int q = kSliceChunksPerThread * tid + i;
                    tsum += static_cast<double>(sum8(wv[i]));
#pragma unroll
                    for (int e = 0; e < 8; ++e)
                        lastpos = (wv[i][e] > 0.0f && q < qn) ? kChunk * (q0 + q) + e : lastpos;
                }
                const double pre = base + block_exclusive_scan<NT>(tsum, s_red);
                int cand = 0x7fffffff;
                double cm = 0.0;
                if (!past && pre <= thr && pre + tsum > thr) {
                    // the crossing lies in this thread's chunks: recount them in order
                    double C = pre;
#pragma unroll
                    for (int i = 0; i < kSliceChunksPerThread; ++i) {
                        const int q = kSliceChunksPerThread * tid + i;
#pragma unroll
                        for (int e = 0; e < 8; ++e) {
                            if (cand == 0x7fffffff && q < qn) {
                                const double before = C;
                                C += static_cast<double>(wv[i][e]);
                                if (C > thr) {
                                    cand = kChunk * (q0 + q) + e;
                                    cm = fmin(C - thr, thr - before);
                                }
                            }
                        }
                    }
                }
                const int mine = cand;
                cand = block_min_int<NT>(cand, s_ired);
                if (cand != 0x7fffffff) {
                    if (mine == cand) s_z[0] = cm;
                    __syncthreads();
                    y = cand;
                    dm = s_z[0] / z;
                } else {   // rounding left the threshold past every crossing
                    y = block_max_int<NT>(lastpos, s_ired);
                    dm = 0.0;
                }
                __syncthreads();
                if (fallback || tau == L) Zp = fallback ? z / P.S[jd] : 1.0;
                else Zp = a * z;
                if (y < 0) bad = 1;
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
            A.accept_len[b] = tau;
            A.draft_index[b] = kstar;
            A.correction[b] = y;
            if (A.flags) A.flags[b] = flags;
            if (A.resid_mass) A.resid_mass[b] = static_cast<float>(Zp);
            if (A.rows_streamed) A.rows_streamed[b] = RS;
        }
        if (A.row_lse) {
            float *o = A.row_lse + static_cast<long long>(b) * RS;
            for (int q = tid; q < RS; q += NT) {
                float v = NAN;
                if (!bad) {
                    const double M = static_cast<double>(P.M[q]);
                    const double off = static_cast<double>(P.K[q]) - M * scd;
                    v = static_cast<float>((M * (1.4426950408889634 / static_cast<double>(T)) +
                                            off + log2(P.S[q])) *
                                           0.6931471805599453);
                }
                o[q] = v;
            }
        }
        if (bad && hout)
            for (int j = tid; j < L; j += NT) hout[j] = NAN;
        __syncthreads();
        // a decision within the fp32 error of its threshold: the request is taken
        // again in fp64 here, its 2L+1 rows' statistics computed by this
        // workgroup (sv_redo.hpp; block-uniform)
        if (!bad && (flags & kFlagNearTie)) redo_request<NT, RD, E>(ra, b, 0, nullptr, s_redo, 0, 1);
    }
}

}  // namespace sv
