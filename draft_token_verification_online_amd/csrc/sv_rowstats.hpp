// sv_rowstats.hpp -- temperature-softmax statistics of every node row.
//
// For each row l of logits and the request's temperature T this kernel finds a
// shift M and S = sum_v 2^((l_v - M) * c) with c = log2(e) / T, so that
//   p(v) = 2^((l_v - M) * c) / S   and   ln sum_v exp(l_v / T) = M / T + ln S.
// This is the temperature softmax the speculative-decoding verifiers apply to
// the target and draft distributions (SpecTr-GBV page, section 2: the
// acceptance probabilities and the residual are functions of those
// distributions).  Only node rows are streamed: the row of draft k at position
// j is skipped when a lower-index draft has the same prefix X[0..j-1].
//
// One workgroup streams one row once from HBM, 8 elements per thread per step
// (one 16-byte load for bf16).  The shift is the block maximum of the first
// tile; a lane only rescales (in fp64) when a later chunk exceeds its shift by
// more than 64 binary orders of magnitude, so the steady state costs one
// exp2 per element and no cross-lane traffic.  Per-chunk sums are formed in
// fp32 and accumulated in fp64.  NaN or +inf logits make S non-finite and an
// all -inf row makes S = 0; the walk treats both as invalid request data.
#pragma once

#include "sv_device.hpp"

namespace sv {

struct RowStat {
    float shift;   // M
    float pad;
    double sum;    // S
};

struct StatsArgs {
    const void *tgt;        // [B][K][L+1][V]
    const void *drf;        // [B][K][L][V]
    const int32_t *tok;     // [B][K][L]
    const float *temp;      // [B]
    RowStat *stats;         // [B][K][2L+1]: target rows 0..L, draft rows at L+1..2L
    int B, K, L, V;
    int rows_per_draft;     // 2L (positions 0..L-1 of both kinds) or 2L+1 (+ target row L)
};

template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void rowstats_kernel(StatsArgs A) {
    __shared__ float s_max[NT / kWave];
    __shared__ double s_sum[NT / kWave];

    const int tid = threadIdx.x;
    const int K = A.K, L = A.L, V = A.V, NR = A.rows_per_draft;
    const long long nrows = static_cast<long long>(A.B) * K * NR;
    const int nch = (V + kChunk - 1) / kChunk;

    for (long long r = blockIdx.x; r < nrows; r += gridDim.x) {
        const int slot = static_cast<int>(r % NR);
        const long long bk = r / NR;
        const int k = static_cast<int>(bk % K);
        const int b = static_cast<int>(bk / K);
        int j, is_target, row_index;
        if (slot < L) { is_target = 1; j = slot; row_index = j; }
        else if (slot < 2 * L) { is_target = 0; j = slot - L; row_index = L + 1 + j; }
        else { is_target = 1; j = L; row_index = L; }

        // node rows only: skip when a lower-index draft shares the prefix X[0..j-1]
        if (k > 0) {
            int dup = 0;
            if (j == 0) {
                dup = 1;
            } else {
                const int32_t *xk = A.tok + (static_cast<long long>(b) * K + k) * L;
                for (int c = tid; c < k; c += NT) {
                    const int32_t *xc = A.tok + (static_cast<long long>(b) * K + c) * L;
                    int same = 1;
                    for (int i = 0; i < j; ++i) same &= (xc[i] == xk[i]);
                    dup |= same;
                }
                dup = __syncthreads_or(dup);
            }
            if (dup) continue;
        }

        const E *base = static_cast<const E *>(is_target ? A.tgt : A.drf);
        const long long row_off = is_target
            ? ((static_cast<long long>(b) * K + k) * (L + 1) + j) * V
            : ((static_cast<long long>(b) * K + k) * L + j) * V;
        const RD row(base + row_off, V);

        const double c64 = 1.4426950408889634 / static_cast<double>(A.temp[b]);
        float chi, clo;
        split_scale(c64, chi, clo);
        const float headroom = 64.0f / chi;   // logit units kept below 2^64

        float x0[8];
        const bool have0 = tid < nch;
        if (have0) row.load(tid, x0);
        else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x0[e] = -INFINITY;
        }
        float m_l = fmaxf(block_max<NT>(max8(x0), s_max), -3.402823466e38f);
        double s = 0.0;

        auto consume = [&](const float (&x)[8]) {
            const float cm = max8(x);
            if (cm > m_l + headroom) {   // rare: move this lane's shift up, in fp64
                s *= exp2((static_cast<double>(m_l) - static_cast<double>(cm)) * c64);
                m_l = cm;
            }
            float e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float d = x[i] - m_l;
                e[i] = fast_exp2(fmaf(d, chi, d * clo));
            }
            s += static_cast<double>(sum8(e));
        };

        if (have0) consume(x0);
        int c = tid + NT;
        for (; c + NT < nch; c += 2 * NT) {
            float xa[8], xb[8];
            row.load(c, xa);
            row.load(c + NT, xb);
            consume(xa);
            consume(xb);
        }
        if (c < nch) {
            float xa[8];
            row.load(c, xa);
            consume(xa);
        }

        const float M = block_max<NT>(m_l, s_max);
        const double scaled =
            (m_l == M) ? s : s * exp2((static_cast<double>(m_l) - static_cast<double>(M)) * c64);
        const double S = block_sum<NT>(scaled, s_sum);
        if (tid == 0) {
            RowStat st;
            st.shift = M;
            st.pad = 0.0f;
            st.sum = S;
            A.stats[(static_cast<long long>(b) * K + k) * (2 * L + 1) + row_index] = st;
        }
    }
}

}  // namespace sv
