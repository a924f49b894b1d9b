// sv_draft.hpp -- drafting K i.i.d. blocks from given draft logits.
//
// The drafting half of the draft-then-verify loop (SpecTr-GBV page, section 2,
// step 1: K i.i.d. draft blocks of length L; MineDraft page, section 1).
// Position by position, draft k draws X[k][j] from the temperature softmax of
// the node row of its prefix X[k][0..j-1] -- the row of the lowest-index draft
// with that prefix, the same node rule the verifier reads -- by the inverse CDF
// of its own uniform u[k][j]: y = min{v : C_v > u Z} in token-id order, or the
// last token of positive weight if rounding leaves none.
//
// One launch per position (the node of a draft at position j depends on the
// tokens drawn before).  A workgroup per (request, draft) returns at once unless
// the draft is the lowest index at its node; otherwise it makes one pass over
// the node row, summing the weights 2^((l - M0) c) of each tile of NT chunks
// into LDS (M0: the maximum of the first tile; the pass is redone with the
// row maximum if any exponent exceeds 64), and then serves every draft at that
// node: the tile holding u Z is found from the tile sums and rescanned with a
// block scan.  The row is read once from HBM; the rescans touch one tile each.
#pragma once

#include "sv_device.hpp"

namespace sv {

struct DraftArgs {
    const void *drf;        // [B][K][L][V]
    const float *temp;      // [B]
    const float *ud;        // [B][K][L]
    int32_t *tok;           // [B][K][L]: drawn tokens (positions < j are read back)
    unsigned *bad;          // [B]: request data the rule cannot act on
    int32_t *rows;          // [B] or null: node rows read
    int B, K, L, V, j;
};

// Zero the per-request flags and row counts before the first position.
__global__ void draft_init_kernel(unsigned *bad, int32_t *rows, int B) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) {
        bad[b] = 0u;
        if (rows) rows[b] = 0;
    }
}

// After the last position: every token of an invalid request becomes -1.
__global__ void draft_fixup_kernel(const unsigned *bad, int32_t *tok, int32_t *flags, int B,
                                   int KL) {
    const long long i = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (i >= static_cast<long long>(B) * KL) return;
    const int b = static_cast<int>(i / KL);
    if (bad[b]) tok[i] = -1;
    if (flags && i % KL == 0) flags[b] = bad[b] ? 2 : 0;
}

// Tile sums of one row's weights 2^((x - M0) c) in fp64, one entry per tile of
// NT chunks, into tile[]; returns their total, sets *lastpos to the last token
// of positive weight and *ovf when an exponent exceeded 64 (the sums are then
// not usable).
template <int NT, typename RD>
__device__ double draft_tiles(const RD &P, int nch, float M0, float chi, float clo, double *tile,
                              int *lastpos, int *ovf, double *red, int *ired) {
    const int ntile = (nch + NT - 1) / NT;
    int last = -1, over = 0;
    for (int t0 = 0; t0 < ntile; t0 += 4) {
        typename RD::Raw r[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = (t0 + i) * NT + threadIdx.x;
            if (c < nch) r[i] = P.raw(c);
        }
        double v[5];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int c = (t0 + i) * NT + threadIdx.x;
            v[i] = 0.0;
            if (c < nch) {
                float x[8];
                RD::unpack(r[i], x);
                float e[8];
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const float d = x[k] - M0;
                    const float y = fmaf(d, chi, d * clo);
                    over |= y > 64.0f;
                    e[k] = fast_exp2(y);
                    if (e[k] > 0.0f) last = 8 * c + k;
                }
                v[i] = static_cast<double>(sum8(e));
            }
        }
        v[4] = static_cast<double>(over);
        block_sum_n<NT, 5>(v, red);   // also publishes the previous tile[] writes
        if (threadIdx.x == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                if (t0 + i < ntile) tile[t0 + i] = v[i];
        }
        if (v[4] > 0.0) break;        // block-uniform: redo with the row maximum
    }
    *ovf = block_max_int<NT>(over, ired);   // its barriers publish tile[]
    *lastpos = block_max_int<NT>(last, ired);
    double z = 0.0;
    for (int t = 0; t < ntile; ++t) z += tile[t];
    return z;
}

// The inverse-CDF pick for threshold thr = u Z from the tile sums; the tile
// holding it is rescanned with the same per-chunk arithmetic as draft_tiles.
template <int NT, typename RD>
__device__ int draft_pick(const RD &P, int nch, float M0, float chi, float clo,
                          const double *tile, double thr, int lastpos, double *red, int *ired) {
    const int ntile = (nch + NT - 1) / NT;
    double base = 0.0;
    int tc = -1;
    for (int t = 0; t < ntile; ++t) {
        if (base + tile[t] > thr) { tc = t; break; }
        base += tile[t];
    }
    if (tc < 0) return lastpos;
    const int c = tc * NT + threadIdx.x;
    float e[8];
    double cs = 0.0;
    if (c < nch) {
        float x[8];
        P.load(c, x);
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float d = x[k] - M0;
            e[k] = fast_exp2(fmaf(d, chi, d * clo));
        }
        cs = static_cast<double>(sum8(e));
    }
    const double pre = base + block_exclusive_scan<NT>(cs, red);
    int cand = 0x7fffffff;
    if (c < nch && pre <= thr && pre + cs > thr) {
        double C = pre;
        int lastp = -1;
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            if (cand == 0x7fffffff) {
                if (e[k] > 0.0f) lastp = 8 * c + k;
                C += static_cast<double>(e[k]);
                if (C > thr) cand = 8 * c + k;
            }
        }
        if (cand == 0x7fffffff && lastp >= 0) cand = lastp;
    }
    cand = block_min_int<NT>(cand, ired);
    return cand == 0x7fffffff ? lastpos : cand;
}

template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void draft_kernel(DraftArgs A) {
    constexpr int NW = NT / kWave;
    constexpr int kMaxTiles = ((1 << 22) / kChunk + NT - 1) / NT;
    __shared__ double s_tile[kMaxTiles];
    __shared__ double s_red[5 * NW];
    __shared__ float s_fred[NW];
    __shared__ int s_ired[NW];

    const int K = A.K, L = A.L, V = A.V, j = A.j;
    const int b = blockIdx.x / K, k = blockIdx.x % K;
    const int tid = threadIdx.x;
    const int32_t *X = A.tok + static_cast<long long>(b) * K * L;

    // the lowest-index draft at this node does the work for all of them
    int skip = 0;
    for (int c = tid; c < k; c += NT) {
        int same = 1;
        for (int t = 0; t < j; ++t) same &= (X[c * L + t] == X[k * L + t]);
        skip |= same;
    }
    if (__syncthreads_or(skip)) return;

    const float T = A.temp[b];
    if (!(T > 0.0f) || !isfinite(T)) {
        if (tid == 0) A.bad[b] = 1u;
        return;
    }
    const double c64 = 1.4426950408889634 / static_cast<double>(T);
    float chi, clo;
    split_scale(c64, chi, clo);
    const int nch = (V + kChunk - 1) / kChunk;
    const E *base = static_cast<const E *>(A.drf);
    const RD P(base + ((static_cast<long long>(b) * K + k) * L + j) * V, V);

    // pass over the row with the first tile's maximum as shift, again with the
    // row maximum if an exponent overflowed
    float x0[8];
    if (tid < nch) P.load(tid, x0);
    else {
#pragma unroll
        for (int e = 0; e < 8; ++e) x0[e] = -INFINITY;
    }
    float M0 = fmaxf(block_max<NT>(max8(x0), s_fred), -3.402823466e38f);
    int lastpos, ovf;
    double Z = draft_tiles<NT, RD>(P, nch, M0, chi, clo, s_tile, &lastpos, &ovf, s_red, s_ired);
    if (ovf) {
        float m = -INFINITY;
        for (int c = tid; c < nch; c += NT) {
            float x[8];
            P.load(c, x);
            m = fmaxf(m, max8(x));
        }
        M0 = fmaxf(block_max<NT>(m, s_fred), -3.402823466e38f);
        Z = draft_tiles<NT, RD>(P, nch, M0, chi, clo, s_tile, &lastpos, &ovf, s_red, s_ired);
    }
    if (tid == 0 && A.rows) atomicAdd(A.rows + b, 1);
    if (!(Z > 0.0) || !isfinite(Z) || ovf) {   // not a distribution
        if (tid == 0) A.bad[b] = 1u;
        return;
    }

    // every draft at this node: k itself and the higher drafts with its prefix
    for (int k2 = k; k2 < K; ++k2) {
        int same = 1;
        for (int t = 0; t < j; ++t) same &= (X[k2 * L + t] == X[k * L + t]);
        if (!same) continue;
        const long long at = (static_cast<long long>(b) * K + k2) * L + j;
        const float u = A.ud[at];
        int y = -1;
        if (u >= 0.0f && u < 1.0f)
            y = draft_pick<NT, RD>(P, nch, M0, chi, clo, s_tile, static_cast<double>(u) * Z,
                                   lastpos, s_red, s_ired);
        if (tid == 0) {
            A.tok[at] = y;
            if (y < 0) A.bad[b] = 1u;
        }
    }
}

}  // namespace sv
