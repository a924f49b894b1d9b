// sv_rowstats.hpp -- temperature-softmax statistics of node rows.
//
// For a row l of logits and the request's temperature T the statistics are a
// shift M and S = sum_v 2^(l_v c - K) with c = log2(e) / T and the row
// constant K = shift_term(M) (sv_device.hpp), so that
//   p(v) = 2^(l_v c - K) / S   and   ln sum_v exp(l_v / T) = (K + log2 S) ln 2.
// This is the temperature softmax the speculative-decoding verifiers apply to
// the target and draft distributions (SpecTr-GBV page, section 2: the
// acceptance probabilities and the residual are functions of them).
//
// rowstats_kernel streams, once, the rows the walk reads first: the root pair
// of every request, and rows 1..L-1 of every draft whose first token no
// lower-index draft has (each such draft is examined at the root unless an
// earlier draft is accepted first).  Rows of drafts that repeat an earlier
// first token are read only after an acceptance: the walk then stops, lists the
// rows below the accepted node for every draft that shares it, and a second
// launch of this kernel streams the listed rows before the walk resumes.  With
// diagnostics requested the kernel covers every node row in one launch, the
// target rows at position L included.
//
// Each workgroup streams one row, 8 elements per thread per step (one 16-byte
// load for bf16).  The shift is the block maximum of the first tile; a lane
// only rescales (in fp64) when a later chunk exceeds its shift by more than 64
// binary orders of magnitude, so the steady state costs one exp2 per element
// and no cross-lane traffic.  Per-chunk sums are formed in fp32 and
// accumulated in fp64.  NaN or +inf logits make S non-finite and an all -inf
// row makes S = 0; the walk treats both as invalid data when it reads the row.
#pragma once

#include "sv_device.hpp"

namespace sv {

struct RowStat {
    float shift;   // M
    float pad;
    double sum;    // S
};

__device__ __forceinline__ bool stat_ok(const RowStat &s) {
    return isfinite(s.shift) && s.sum > 0.0 && isfinite(s.sum);
}

// Per-lane online accumulator of one row's statistics under scale c.
struct LaneSoftmax {
    float m;          // this lane's shift
    float mc;         // shift_term(m, c)
    double s;         // sum of 2^(x c - mc) over the lane's elements
    __device__ __forceinline__ void init(float block_first_max, const Scale &c) {
        m = fmaxf(block_first_max, -3.402823466e38f);
        mc = shift_term(m, c);
        s = 0.0;
    }
    // The chunk sum is checked instead of every exponent: it exceeds 2^64 (or is
    // +inf) whenever an element lies more than 64 binary orders above the lane's
    // shift, and then (rarely) the lane moves its shift up to the chunk maximum,
    // rescaling its sum in fp64, and sums the chunk again.  A NaN sum fails the
    // test and makes S NaN.
    __device__ __forceinline__ void consume(const float (&x)[8], const Scale &c) {
        float e[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) e[i] = fast_exp2(expo(x[i], c, mc));
        float t = sum8(e);
        if (t > 0x1p64f) {
            const float cm = max8(x);
            const float cmc = shift_term(cm, c);
            s *= exp2(static_cast<double>(mc) - static_cast<double>(cmc));
            m = cm;
            mc = cmc;
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = fast_exp2(expo(x[i], c, mc));
            t = sum8(e);
        }
        s += static_cast<double>(t);
    }
};

// Combine the lanes of a block into the row's (M, S); every thread gets it.
template <int NT>
__device__ __forceinline__ RowStat finish_row(const LaneSoftmax &ls, const Scale &c, float *fred,
                                              double *red) {
    const float M = block_max<NT>(ls.m, fred);
    const double scaled =
        (ls.m == M) ? ls.s
                    : ls.s * exp2(static_cast<double>(ls.mc) -
                                  static_cast<double>(shift_term(M, c)));
    RowStat st;
    st.shift = M;
    st.pad = 0.0f;
    st.sum = block_sum<NT>(scaled, red);
    return st;
}

// A row the walk asked for: request b, draft k, position j, target (1) or draft (0).
struct RowRef {
    int b;
    int kjt;                // (k * L + j) * 2 + is_target
};

struct StatsArgs {
    const void *tgt;        // [B][K][L+1][V]
    const void *drf;        // [B][K][L][V]
    const int32_t *tok;     // [B][K][L]
    const float *temp;      // [B]
    RowStat *stats;         // [B][K][2L+1]: target rows 0..L, draft rows at L+1..2L
    const RowRef *list;     // rows the walk asked for (mode kSelectListed)
    unsigned *list_count;   // their number; the first-visit launch resets it to 0
    unsigned *redo_count;   // requests listed for the fp64 re-evaluation; reset to 0 by
                            // every launch that is not of listed rows
    int B, K, L, V;
    int mode;               // kSelectAllNodes, kSelectFirstVisit or kSelectListed
    int depth;              // first-visit rows are at positions j < depth (1 <= depth <= L)
};

constexpr int kSelectFirstVisit = 0;   // root pair + rows 1..depth-1 of drafts with a new first token
constexpr int kSelectAllNodes = 1;     // every node row, target rows at position L included
constexpr int kSelectListed = 2;       // node rows the walk listed after an acceptance
constexpr int kStreamBytes = 128;      // bytes of a row in flight per lane (8 bf16 chunks)

template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void rowstats_kernel(StatsArgs A) {
    __shared__ float s_max[NT / kWave];
    __shared__ double s_sum[NT / kWave];

    const int tid = threadIdx.x;
    const int K = A.K, L = A.L, V = A.V;
    // row slots per (request, draft): target rows then draft rows at positions
    // 0..D-1, and with every node row the target row at position L
    const int D = A.mode == kSelectFirstVisit ? A.depth : L;
    const int NR = 2 * D + (A.mode == kSelectAllNodes ? 1 : 0);
    const long long nrows = A.mode == kSelectListed
                                ? static_cast<long long>(*A.list_count)
                                : static_cast<long long>(A.B) * K * NR;
    const int nch = (V + kChunk - 1) / kChunk;
    if (A.mode == kSelectFirstVisit && blockIdx.x == 0 && tid == 0) *A.list_count = 0u;
    if (A.mode != kSelectListed && blockIdx.x == 0 && tid == 0) *A.redo_count = 0u;

    for (long long r = blockIdx.x; r < nrows; r += gridDim.x) {
        int b, k, j, is_target, row_index;
        if (A.mode == kSelectListed) {
            const RowRef ref = A.list[r];
            b = ref.b;
            is_target = ref.kjt & 1;
            k = (ref.kjt >> 1) / L;
            j = (ref.kjt >> 1) % L;
            row_index = is_target ? j : L + 1 + j;
        } else {
            const int slot = static_cast<int>(r % NR);
            const long long bk = r / NR;
            k = static_cast<int>(bk % K);
            b = static_cast<int>(bk / K);
            if (slot < D) { is_target = 1; j = slot; row_index = j; }
            else if (slot < 2 * D) { is_target = 0; j = slot - D; row_index = L + 1 + j; }
            else { is_target = 1; j = L; row_index = L; }
        }

        // which rows: every node row (lowest-index draft per prefix X[0..j-1]);
        // first-visit rows (the root pair; rows 1 <= j < depth of drafts whose
        // first token is new among drafts 0..k); or the node rows the walk listed
        if (A.mode != kSelectListed && k > 0) {
            int skip = 0;
            if (j == 0) {
                skip = 1;
            } else {
                const int32_t *xk = A.tok + (static_cast<long long>(b) * K + k) * L;
                const int n = A.mode == kSelectAllNodes ? j : 1;
                for (int c = tid; c < k; c += NT) {
                    const int32_t *xc = A.tok + (static_cast<long long>(b) * K + c) * L;
                    int same = 1;
                    for (int i = 0; i < n; ++i) same &= (xc[i] == xk[i]);
                    skip |= same;
                }
                skip = __syncthreads_or(skip);
            }
            if (skip) continue;
        }

        const E *base = static_cast<const E *>(is_target ? A.tgt : A.drf);
        const long long row_off = is_target
            ? ((static_cast<long long>(b) * K + k) * (L + 1) + j) * V
            : ((static_cast<long long>(b) * K + k) * L + j) * V;
        const RD row(base + row_off, V);

        const Scale c = temp_scale(A.temp[b]);

        float x0[8];
        const bool have0 = tid < nch;
        if (have0) RD::unpack(row.raw_once(tid), x0);
        else {
#pragma unroll
            for (int e = 0; e < 8; ++e) x0[e] = -INFINITY;
        }
        LaneSoftmax ls;
        ls.init(block_max<NT>(max8(x0), s_max), c);
        if (have0) ls.consume(x0, c);
        // chunks NT.. of the row (the first tile is consumed above)
        const RD rest = row.advanced(NT);
        if (nch > NT)
            stream_rows<NT, depth_for<RD, kStreamBytes>(), false, true>(rest, rest, nch - NT,
                                           [&](const float (&x)[8], const float (&)[8], int) {
                                               ls.consume(x, c);
                                           });
        const RowStat st = finish_row<NT>(ls, c, s_max, s_sum);
        if (tid == 0)
            A.stats[(static_cast<long long>(b) * K + k) * (2 * L + 1) + row_index] = st;
    }
}

}  // namespace sv
