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
// The node of a draft at position j depends on the tokens drawn before, so each
// position takes up to three launches:
//   1. draft_nodes_kernel -- one wave per request: the node of every draft, the
//      list of node rows to read (one per node, appended with one atomic per
//      wave) and, per draft, the list slot of its node's row.  The list has one
//      buffer per position parity, so position j+1 can be listed while
//      position j's draws still read theirs;
//   2. draft_tiles_kernel -- grid-stride over (listed row, tile of 512 chunks),
//      one 64-lane wave per tile (8 chunks per lane): the tile's maximum M_t and
//      the sum of 2^(l c - K_t) over it (K_t = shift_term(M_t), the exponent
//      convention of every kernel here), by wave reductions only (no barrier).
//      Every row is streamed once, by as many waves as it has tiles, so a
//      position with few nodes still fills the chip;
//   3. draft_pick_kernel  -- one wave per draft: rescale the tile sums of its
//      node's row to the row maximum, find the tile holding u Z and rescan it
//      with the tiles kernel's own per-chunk arithmetic (wave reductions only).
//      With K <= 16, draft_pick_next_kernel instead runs one workgroup per
//      request (wave k = draft k): the draws of position j, a barrier, then the
//      node rows of position j+1 -- one launch fewer per position.
#pragma once

#include "sv_device.hpp"

namespace sv {

constexpr int kDraftTileChunks = 512;                // chunks per tile (8 per lane of a wave)

struct DraftArgs {
    const void *drf;        // [B][K][L][V]
    const float *temp;      // [B]
    const float *ud;        // [B][K][L]
    int32_t *tok;           // [B][K][L]: drawn tokens (positions < j are read back)
    unsigned *bad;          // [B]: request data the rule cannot act on
    unsigned *count;        // [L]: node rows listed at each position
    int32_t *list;          // [2][B*K]: listed node rows, b*K + k (buffer j % 2)
    int32_t *slot;          // [B*K]: list slot of each draft's node row
    float *tmax;            // [B*K][ntiles]: shift of each tile (its maximum)
    double *tsum;           // [B*K][ntiles]: tile sums under their shift
    int32_t *rows;          // [B] or null: node rows read
    int B, K, L, V, j, ntiles;
};

// Zero the per-request flags, row counts and per-position list lengths.
__global__ void draft_init_kernel(unsigned *bad, int32_t *rows, unsigned *count, int B, int L) {
    const int b = blockIdx.x * blockDim.x + threadIdx.x;
    if (b < B) {
        bad[b] = 0u;
        if (rows) rows[b] = 0;
    }
    if (b < L) count[b] = 0u;
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

// The list buffer of position j.
__device__ __forceinline__ int32_t *draft_list(const DraftArgs &A, int j) {
    return A.list + static_cast<long long>(j & 1) * A.B * A.K;
}

// The node rows of request b at position j, given in lane k < K the lowest
// draft index whose prefix X[0..j-1] equals draft k's (the node's own draft):
// one list slot per node (one atomic per wave), and each draft's slot.
__device__ void draft_list_nodes(const DraftArgs &A, int b, int j, int canon) {
    const int lane = threadIdx.x & (kWave - 1);
    const int K = A.K;
    const bool head = lane < K && canon == lane;
    const unsigned long long heads = __ballot(head);
    unsigned base = 0;
    if (lane == 0) base = atomicAdd(A.count + j, static_cast<unsigned>(__popcll(heads)));
    base = __shfl(base, 0, kWave);
    const unsigned rank = __popcll(heads & ((1ull << lane) - 1ull));
    const int my_slot = static_cast<int>(base + rank);
    if (head) draft_list(A, j)[my_slot] = b * K + lane;
    const int node_slot = __shfl(my_slot, canon, kWave);
    if (lane < K) A.slot[b * K + lane] = node_slot;
    if (head && A.rows) atomicAdd(A.rows + b, 1);
}

// 1. One 64-lane wave per request, lane k = draft k (K <= 64): the node rows
// of request b at position j, from the drawn prefixes.
__device__ void draft_nodes_wave(const DraftArgs &A, int b, int j) {
    const int lane = threadIdx.x & (kWave - 1);
    const int K = A.K, L = A.L;
    const int32_t *X = A.tok + static_cast<long long>(b) * K * L;
    const float T = A.temp[b];
    if (!(T > 0.0f) || !isfinite(T)) {
        if (lane == 0) A.bad[b] = 1u;
        return;
    }
    int canon = lane;
    if (lane < K) {
        for (int c = 0; c < lane; ++c) {
            int same = 1;
            for (int t = 0; t < j; ++t) same &= (X[c * L + t] == X[lane * L + t]);
            if (same) { canon = c; break; }
        }
    }
    draft_list_nodes(A, b, j, canon);
}

__global__ __launch_bounds__(256) void draft_nodes_kernel(DraftArgs A) {
    const int b = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (b >= A.B) return;                      // whole waves only
    draft_nodes_wave(A, b, A.j);
}

// 2. Tile sums of the listed rows, one wave per tile.
template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void draft_tiles_kernel(DraftArgs A) {
    constexpr int kPerLane = kDraftTileChunks / kWave;
    constexpr int WPB = NT / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int K = A.K, L = A.L, V = A.V, j = A.j, ntiles = A.ntiles;
    const int nch = (V + kChunk - 1) / kChunk;
    const long long nitems = static_cast<long long>(A.count[j]) * ntiles;
    const E *base = static_cast<const E *>(A.drf);
    for (long long it = static_cast<long long>(blockIdx.x) * WPB + threadIdx.x / kWave;
         it < nitems; it += static_cast<long long>(gridDim.x) * WPB) {
        const int slot = static_cast<int>(it / ntiles);
        const int t = static_cast<int>(it % ntiles);
        const int bk = draft_list(A, j)[slot];
        const int b = bk / K, k = bk % K;
        const RD P(base + ((static_cast<long long>(b) * K + k) * L + j) * V, V);
        // all eight loads are issued before any is used (addresses clamped into
        // the row; chunks past its end are loaded but not counted), so they are
        // in flight together instead of one after another
        typename RD::Raw r[kPerLane];
#pragma unroll
        for (int i = 0; i < kPerLane; ++i)
            r[i] = P.raw_once(min(t * kDraftTileChunks + i * kWave + lane, nch - 1));
        float m = -INFINITY;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int c = t * kDraftTileChunks + i * kWave + lane;
            float x[8];
            RD::unpack(r[i], x);
            if (c < nch) m = fmaxf(m, max8(x));
        }
        const float M = fmaxf(wave_max(m), -3.402823466e38f);
        const Scale sc = temp_scale(A.temp[b]);
        const float Mc = shift_term(M, sc);
        double sum = 0.0;
#pragma unroll
        for (int i = 0; i < kPerLane; ++i) {
            const int c = t * kDraftTileChunks + i * kWave + lane;
            if (c < nch) {
                float x[8], e[8];
                RD::unpack(r[i], x);
#pragma unroll
                for (int q = 0; q < 8; ++q) e[q] = fast_exp2(expo(x[q], sc, Mc));
                sum += static_cast<double>(sum8(e));
            }
        }
        sum = wave_sum(sum);
        if (lane == 0) {
            A.tmax[static_cast<long long>(slot) * ntiles + t] = M;
            A.tsum[static_cast<long long>(slot) * ntiles + t] = sum;
        }
    }
}

// 3. One 64-lane wave per draft: the inverse-CDF draw from its node row's tiles.
// Returns, in every lane, the draft whose row is the node's and the token drawn
// (token -1 - k where the request is invalid and nothing was drawn).
template <typename RD, typename E>
__device__ int2 draft_pick_wave(const DraftArgs &A, int b, int k) {
    constexpr int kPerLane = kDraftTileChunks / kWave;   // rescanned chunks per lane
    const int lane = threadIdx.x & (kWave - 1);
    const int K = A.K, L = A.L, V = A.V, j = A.j;
    // the draft's uniform, the request's temperature and the draft's list slot
    // are loaded together with the request's flag; the slot (stale once a
    // request is invalid) is used only after the flag is checked
    const float u = A.ud[(static_cast<long long>(b) * K + k) * L + j];
    const Scale sc = temp_scale(A.temp[b]);
    const int slot = A.slot[b * K + k];
    const int2 none = make_int2(k, -1 - k);
    if (A.bad[b]) return none;   // one load for the wave; a flag set meanwhile changes nothing
    const int c0 = draft_list(A, j)[slot] % K;   // the draft whose row is the node's
    const int nch = (V + kChunk - 1) / kChunk;
    const int ntiles = A.ntiles;
    const float *tm = A.tmax + static_cast<long long>(slot) * ntiles;
    const double *ts = A.tsum + static_cast<long long>(slot) * ntiles;

    // row maximum over the tile shifts; each tile's weight in the row's scale
    float m = -INFINITY;
    for (int t = lane; t < ntiles; t += kWave) m = fmaxf(m, tm[t]);
    const float M = wave_max(m);
    const double Mcd = static_cast<double>(shift_term(M, sc));
    auto wt = [&](int t) {
        return ts[t] * exp2(static_cast<double>(shift_term(tm[t], sc)) - Mcd);
    };
    // lane l owns the contiguous tiles [l*per, (l+1)*per)
    const int per = (ntiles + kWave - 1) / kWave;
    const int t0 = min(lane * per, ntiles), t1 = min(t0 + per, ntiles);
    double own = 0.0;
    int last_tile = -1;
    for (int t = t0; t < t1; ++t) {
        const double w = wt(t);
        own += w;
        if (w > 0.0) last_tile = t;
    }
    const double pre = wave_exclusive_scan(own);
    const double Z = wave_sum(own);
    last_tile = wave_max_int(last_tile);
    if (!(Z > 0.0) || !isfinite(Z) || !(u >= 0.0f && u < 1.0f)) {
        if (lane == 0) A.bad[b] = 1u;
        return none;
    }
    const double thr = static_cast<double>(u) * Z;
    int tc = 0x7fffffff;
    if (pre <= thr && pre + own > thr) {
        double acc = pre;
        for (int t = t0; t < t1; ++t) {
            const double w = wt(t);
            if (acc + w > thr) { tc = t; break; }
            acc += w;
        }
    }
    tc = wave_min_int(tc);
    const bool fallback = tc == 0x7fffffff;    // rounding left no crossing: last positive token
    if (fallback) tc = last_tile;
    // the mass before tile tc, from the lane that owns it
    double tb = 0.0;
    if (tc >= t0 && tc < t1) {
        tb = pre;
        for (int t = t0; t < tc; ++t) tb += wt(t);
    }
    const double tbase = __shfl(tb, per > 0 ? tc / per : 0, kWave);

    // rescan tile tc with the tiles kernel's arithmetic; lane l takes chunks
    // [8l, 8l+8) of the tile, so the wave scan runs in token order
    const E *base = static_cast<const E *>(A.drf);
    const RD P(base + ((static_cast<long long>(b) * K + c0) * L + j) * V, V);
    const float Mgc = shift_term(tm[tc], sc);
    const double f = exp2(static_cast<double>(Mgc) - Mcd);
    const int c1 = tc * kDraftTileChunks + lane * kPerLane;
    // the lane's eight chunks are loaded before any is used (clamped addresses;
    // chunks past the row are not counted) and kept for the crossing lane's
    // in-order recount, so no chunk is read twice
    typename RD::Raw r[kPerLane];
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) r[i] = P.raw(min(c1 + i, nch - 1));
    double cs = 0.0;
    int lastp = -1;
#pragma unroll
    for (int i = 0; i < kPerLane; ++i) {
        const int c = c1 + i;
        if (c < nch) {
            float x[8], e[8];
            RD::unpack(r[i], x);
#pragma unroll
            for (int q = 0; q < 8; ++q) e[q] = fast_exp2(expo(x[q], sc, Mgc));
#pragma unroll
            for (int q = 0; q < 8; ++q)
                if (e[q] > 0.0f) lastp = 8 * c + q;
            cs += static_cast<double>(sum8(e));
        }
    }
    const double cpre = wave_exclusive_scan(cs);
    int cand = 0x7fffffff;
    if (!fallback && c1 < nch) {
        const double lo = tbase + f * cpre, hi = tbase + f * (cpre + cs);
        if (lo <= thr && hi > thr) {   // the crossing lane: its weights again, in order
            double C = cpre;
#pragma unroll
            for (int i = 0; i < kPerLane; ++i) {
                if (c1 + i < nch && cand == 0x7fffffff) {
                    float x[8], e[8];
                    RD::unpack(r[i], x);
#pragma unroll
                    for (int q = 0; q < 8; ++q) e[q] = fast_exp2(expo(x[q], sc, Mgc));
#pragma unroll
                    for (int q = 0; q < 8; ++q) {
                        if (cand == 0x7fffffff) {
                            C += static_cast<double>(e[q]);
                            if (tbase + f * C > thr) cand = 8 * (c1 + i) + q;
                        }
                    }
                }
            }
            if (cand == 0x7fffffff) cand = lastp;
        }
    }
    cand = wave_min_int(cand);
    const int lastrow = wave_max_int(lastp);
    const int y = cand == 0x7fffffff ? lastrow : cand;
    if (lane == 0) A.tok[(static_cast<long long>(b) * K + k) * L + j] = y;
    return make_int2(c0, y);
}

template <int NT, typename RD, typename E>
__global__ __launch_bounds__(NT) void draft_pick_kernel(DraftArgs A) {
    const long long d = static_cast<long long>(blockIdx.x) * (NT / kWave) + threadIdx.x / kWave;
    if (d >= static_cast<long long>(A.B) * A.K) return;        // whole waves
    (void)draft_pick_wave<RD, E>(A, static_cast<int>(d / A.K), static_cast<int>(d % A.K));
}

// 3'. One workgroup of K waves per request (K <= 16): the draws of position j,
// then (j + 1 < L) the node rows of position j + 1.  Drafts share a node at
// j + 1 exactly when they share one at j and drew the same token there, so
// wave 0 finds each draft's node from the K (node draft, token) pairs the waves
// leave in LDS, without reading the prefixes back.
constexpr int kDraftFusedMaxK = 16;
template <typename RD, typename E>
__global__ __launch_bounds__(kDraftFusedMaxK * kWave) void draft_pick_next_kernel(DraftArgs A) {
    __shared__ int s_node[kDraftFusedMaxK], s_tok[kDraftFusedMaxK];
    const int b = blockIdx.x, k = threadIdx.x / kWave, lane = threadIdx.x & (kWave - 1);
    const int2 r = draft_pick_wave<RD, E>(A, b, k);
    if (A.j + 1 < A.L) {
        if (lane == 0) { s_node[k] = r.x; s_tok[k] = r.y; }
        __syncthreads();
        if (k == 0 && !A.bad[b]) {   // an invalid request lists no more rows
            const int K = A.K;
            const int pn = lane < K ? s_node[lane] : -1, pt = lane < K ? s_tok[lane] : -1;
            int canon = lane;
            for (int c = K - 1; c >= 0; --c) {
                const int cn = __shfl(pn, c, kWave), ct = __shfl(pt, c, kWave);
                if (c < lane && cn == pn && ct == pt) canon = c;
            }
            draft_list_nodes(A, b, A.j + 1, canon);
        }
    }
}

}  // namespace sv
