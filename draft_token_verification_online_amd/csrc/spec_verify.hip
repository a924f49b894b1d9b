// spec_verify.hip -- C ABI of the verification library (see include/spec_verify.h).
//
// A call validates everything it can on the host before touching the device,
// then launches on the caller's stream:
//   1. rowstats_kernel  -- one workgroup per node row: softmax statistics of the
//                          rows the walk reads first (streams the logits);
//   2. walk_kernel      -- one workgroup per request: the verification walk (the
//                          block walk, the token rule, or SpecTr's forward walk); with
//                          K > 1 it may stop after an acceptance, flagging the rows
//                          below the accepted node;
//   3. rowstats_kernel  -- (K > 1) statistics of the flagged rows;
//   4. walk_kernel      -- (K > 1) resumes the stopped walks.
// spec_draft_sample draws the draft blocks instead: per position, the node rows
// are listed, streamed into tile sums and drawn from (three launches), between
// a clearing launch and a final pass over invalid requests.
// No allocation, no synchronisation.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <mutex>

#include "../../include/spec_verify.h"
#include "sv_draft.hpp"
#include "sv_lmhead.hpp"
#include "sv_redo.hpp"
#include "sv_rowstats.hpp"
#include "sv_single.hpp"
#include "sv_walk.hpp"

namespace {

constexpr int kStatsThreads = 256;
constexpr int kWalkThreads = 512;
constexpr long long kMaxStatsGrid = 1LL << 22;
constexpr long long kListGrid = 4096;
constexpr int kMaxB = 1 << 24;
// Re-evaluation launches: workgroups over (listed request, node row) and over
// listed requests, grid-stride.  With none listed every workgroup returns after
// one load, so the grids are kept small (one workgroup per CU at most): most
// calls list nothing.
constexpr long long kRedoStatsGrid = 1024;   // up to four 512-thread workgroups per CU

static_assert(SV_MAX_K == sv::kMaxK, "K limit");
static_assert(SV_MAX_L == sv::kMaxL, "L limit");
static_assert(SV_MAX_V == sv::kMaxV, "V limit");
static_assert(SV_FLAG_DEGENERATE == sv::kFlagDegenerate, "flag bits");
static_assert(SV_FLAG_INVALID == sv::kFlagInvalid, "flag bits");
static_assert(SV_FLAG_NEAR_TIE == sv::kFlagNearTie && SV_NEAR_TIE == sv::kNearTie, "flag bits");
static_assert(SV_FLAG_REDONE == sv::kFlagRedone, "flag bits");
static_assert(sizeof(sv::RowStat) == 16, "row statistics layout");
static_assert(sizeof(sv::RedoStat) == sizeof(sv::RowStat) && sizeof(sv::SliceStat) == sizeof(sv::RowStat),
              "the re-evaluation's fp64 statistics reuse the row-statistics region");
static_assert(sizeof(sv_row_stat) == sizeof(sv::RowStat) && offsetof(sv_row_stat, sum) == 8,
              "sv_row_stat is the library's row statistics layout");

size_t align_up(size_t n, size_t a) { return (n + a - 1) / a * a; }

bool sizes_ok(int32_t B, int32_t K, int32_t L, int32_t V, int32_t dtype) {
    return B >= 0 && B <= kMaxB && K >= 1 && K <= SV_MAX_K && L >= 1 && L <= SV_MAX_L &&
           V >= 1 && V <= SV_MAX_V && (dtype == SV_F32 || dtype == SV_BF16);
}

size_t stats_bytes(int32_t B, int32_t K, int32_t L) {
    return static_cast<size_t>(B) * static_cast<size_t>(K) * static_cast<size_t>(2 * L + 1) *
           sizeof(sv::RowStat);
}

// Workspace: row statistics (after the walk, the fp64 statistics of the requests
// listed for re-evaluation) | walk states | node rows flagged for the second
// round (bytes, then the same rows as a list) | list length | number of
// requests listed for re-evaluation in fp64 | their indices | the walk's test
// records (a byte per test) | SpecTr's scaling factor per position | node lists
// of the walk (K >= 3 only: a node sees a second mass sweep only with three or
// more drafts).
struct Layout {
    size_t stats, state, need, list, count, rcount, rlist, dec, rho, team, nodes, total;
    bool has_nodes;
};

// Single-draft workspace (K = 1 without given statistics): slice statistics of
// every row | residual slice sums per position | each request's combined
// statistics and weight chain.
struct SingleLayout {
    size_t part, rpart, prep, total;
    int NS;
};

SingleLayout single_layout(int32_t B, int32_t L, int32_t V) {
    SingleLayout l;
    const int nch = (V + sv::kChunk - 1) / sv::kChunk;
    l.NS = (nch + sv::kSliceChunks - 1) / sv::kSliceChunks;
    const size_t bs = static_cast<size_t>(B) * l.NS;
    l.part = 0;
    l.rpart = align_up(bs * (2 * L + 1) * sizeof(sv::SliceStat), 256);
    l.prep = l.rpart + align_up(bs * (L + 1) * sizeof(double), 256);
    l.total = l.prep + align_up(static_cast<size_t>(B) * sizeof(sv::SinglePrep), 256);
    return l;
}

Layout layout(int32_t B, int32_t K, int32_t L) {
    Layout l;
    const size_t bkl = static_cast<size_t>(B) * K * L;
    l.stats = 0;
    l.state = align_up(stats_bytes(B, K, L), 256);
    l.need = l.state + align_up(static_cast<size_t>(B) * sizeof(sv::WalkState), 256);
    l.list = l.need + align_up(bkl, 256);
    l.count = l.list + align_up(2 * bkl * sizeof(sv::RowRef), 256);
    l.rcount = l.count + 256;
    l.rlist = l.rcount + 256;
    l.dec = l.rlist + align_up(static_cast<size_t>(B) * sizeof(int32_t), 256);
    l.rho = l.dec + align_up(bkl, 256);
    l.team = l.rho + align_up(static_cast<size_t>(B) * L * sizeof(double), 256);
    l.nodes = l.team + align_up(sv::kRedoTeamSlots * (sizeof(sv::TeamCmd) + sizeof(sv::TeamPart)), 256);
    l.has_nodes = K >= 3;
    l.total = l.nodes + (l.has_nodes ? static_cast<size_t>(B) *
                                           static_cast<size_t>(sv::node_list_bytes<kWalkThreads>())
                                     : 0);
    return l;
}

hipError_t record(const sv_launch *ln, int i, hipStream_t stream) {
    return ln->phase_events[i] ? hipEventRecord(static_cast<hipEvent_t>(ln->phase_events[i]), stream)
                               : hipSuccess;
}

__global__ void reset_count_kernel(unsigned *count) {
    if (threadIdx.x == 0) *count = 0u;
}

// How long a team's first workgroup waits for its members' answers to a command
// (real-time counter ticks, 100 MHz) before it sums their ranges itself: 200 us,
// or SV_TEAM_WAIT_TICKS when that is set (tests set 0 to make every command take
// the fallback; the results do not depend on it).
long long team_wait_ticks() {
    const char *e = std::getenv("SV_TEAM_WAIT_TICKS");
    if (!e || !*e) return sv::kTeamWaitTicks;
    char *end = nullptr;
    const long long v = std::strtoll(e, &end, 10);
    return (end && *end == '\0' && v >= 0 && v <= sv::kTeamWaitTicks) ? v : sv::kTeamWaitTicks;
}

// Requests the fast path listed (a decision within the fp32 error of its
// threshold), taken again in fp64: their node rows' statistics over the whole
// chip, then one workgroup per request.  `stats` is a region of at least
// B * K * (2L + 1) * 16 bytes that the fast path no longer reads.
template <typename E, bool VEC>
hipError_t launch_redo(const sv_inputs *in, const sv_outputs *out, hipStream_t stream, int method,
                       const unsigned *count, const int32_t *list, void *stats,
                       const unsigned char *dec, const double *rho_rec, void *team) {
    using RD = typename sv::RowOf<E, VEC>::type;
    sv::RedoArgs ra;
    ra.tgt = in->target_logits;
    ra.drf = in->draft_logits;
    ra.tok = in->draft_tokens;
    ra.temp = in->temperature;
    ra.ua = in->u_accept;
    ra.uc = in->u_correct;
    ra.count = count;
    ra.list = list;
    ra.stats = static_cast<sv::RedoStat *>(stats);
    ra.dec = dec;
    ra.rho_rec = rho_rec;
    ra.B = in->B;
    ra.K = in->K;
    ra.L = in->L;
    ra.V = in->V;
    ra.method = method;
    ra.accept_len = out->accept_len;
    ra.draft_index = out->draft_index;
    ra.correction = out->correction;
    ra.flags = out->flags;
    ra.accept_prob = out->accept_prob;
    ra.resid_mass = out->resid_mass;
    ra.team_wait = team_wait_ticks();
    ra.team_cmd = static_cast<sv::TeamCmd *>(team);
    ra.team_part = reinterpret_cast<sv::TeamPart *>(static_cast<char *>(team) +
                                                    sv::kRedoTeamSlots * sizeof(sv::TeamCmd));
    const long long rows = static_cast<long long>(in->B) * in->K * (2 * in->L + 1);
    const unsigned g1 = static_cast<unsigned>(rows < kRedoStatsGrid ? rows : kRedoStatsGrid);
    hipLaunchKernelGGL((sv::redo_stats_kernel<sv::kRedoStatsThreads, RD, E>), dim3(g1),
                       dim3(sv::kRedoStatsThreads), 0, stream, ra);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // teams of up to kTeamMax workgroups per listed request (at most B of them)
    const long long want = static_cast<long long>(in->B) * sv::kTeamMax;
    const unsigned g2 = static_cast<unsigned>(want < sv::kRedoTeamSlots ? want : sv::kRedoTeamSlots);
    hipLaunchKernelGGL((sv::redo_walk_kernel<sv::kRedoThreads, RD, E>), dim3(g2),
                       dim3(sv::kRedoThreads), 0, stream, ra);
    return hipGetLastError();
}

template <typename E, bool VEC>
hipError_t launch(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln, int method) {
    using RD = typename sv::RowOf<E, VEC>::type;
    hipStream_t stream = static_cast<hipStream_t>(ln->stream);
    const bool diagnostics = out->row_lse != nullptr;
    const bool given = in->row_stats != nullptr;
    // a second round only pays when several drafts can share an accepted prefix
    const bool two_round = method != sv::kMethodToken && in->K > 1 && !diagnostics && !given;
    const bool spectr = method == sv::kMethodSpecTr || method == sv::kMethodSpecTrBisect;
    const Layout lay = layout(in->B, in->K, in->L);
    char *ws = static_cast<char *>(ln->workspace);

    sv::StatsArgs sa;
    sa.tgt = in->target_logits;
    sa.drf = in->draft_logits;
    sa.tok = in->draft_tokens;
    sa.temp = in->temperature;
    sa.stats = reinterpret_cast<sv::RowStat *>(ws + lay.stats);
    sa.list = reinterpret_cast<const sv::RowRef *>(ws + lay.list);
    sa.list_count = reinterpret_cast<unsigned *>(ws + lay.count);
    sa.redo_count = reinterpret_cast<unsigned *>(ws + lay.rcount);
    sa.B = in->B;
    sa.K = in->K;
    sa.L = in->L;
    sa.V = in->V;
    sa.mode = diagnostics ? sv::kSelectAllNodes : sv::kSelectFirstVisit;
    // First-visit depth.  The block walk examines a draft's whole sub-block at
    // once, so it streams the chains of every draft with a new first token.
    // SpecTr stops at its first rejected position and reaches position j only
    // through acceptances at every position before it: with several drafts it
    // streams the root pair and the position-1 node of every first token, and
    // a walk that gets further stops and lists the rest (the second round).
    sa.depth = (spectr && two_round) ? (in->L < 2 ? in->L : 2) : in->L;
    auto grid_for = [&](int rows_per_draft) {
        const long long n = static_cast<long long>(in->B) * in->K * rows_per_draft;
        return static_cast<unsigned>(n < kMaxStatsGrid ? n : kMaxStatsGrid);
    };

    sv::WalkArgs wa;
    wa.tgt = in->target_logits;
    wa.drf = in->draft_logits;
    wa.tok = in->draft_tokens;
    wa.temp = in->temperature;
    wa.ua = in->u_accept;
    wa.uc = in->u_correct;
    wa.stats = given ? static_cast<sv::RowStat *>(const_cast<void *>(in->row_stats)) : sa.stats;
    wa.B = in->B;
    wa.K = in->K;
    wa.L = in->L;
    wa.V = in->V;
    wa.method = spectr ? sv::kMethodSpecTr : method;
    wa.rho_bisect = method == sv::kMethodSpecTrBisect ? 1 : 0;
    wa.all_nodes = (diagnostics || given) ? 1 : 0;
    wa.fv_depth = sa.depth;
    wa.stats_given = given ? 1 : 0;
    wa.round = 1;
    wa.two_round = two_round ? 1 : 0;
    wa.state = reinterpret_cast<sv::WalkState *>(ws + lay.state);
    wa.need = reinterpret_cast<unsigned char *>(ws + lay.need);
    wa.list = reinterpret_cast<sv::RowRef *>(ws + lay.list);
    wa.list_count = sa.list_count;
    wa.nodes = (lay.has_nodes && method == sv::kMethodBlockWalk) ? ws + lay.nodes : nullptr;
    wa.accept_len = out->accept_len;
    wa.draft_index = out->draft_index;
    wa.correction = out->correction;
    wa.flags = out->flags;
    wa.rows_streamed = out->rows_streamed;
    wa.row_lse = out->row_lse;
    wa.accept_prob = out->accept_prob;
    wa.resid_mass = out->resid_mass;
    wa.redo_count = sa.redo_count;
    wa.redo_list = reinterpret_cast<int32_t *>(ws + lay.rlist);
    wa.dec = (method == sv::kMethodBlockWalk || spectr)
                 ? reinterpret_cast<unsigned char *>(ws + lay.dec)
                 : nullptr;
    wa.rho_rec = spectr ? reinterpret_cast<double *>(ws + lay.rho) : nullptr;

    hipError_t err;
    if ((err = record(ln, 0, stream)) != hipSuccess) return err;
    if (!given) {
        hipLaunchKernelGGL((sv::rowstats_kernel<kStatsThreads, RD, E>),
                           dim3(grid_for(diagnostics ? 2 * in->L + 1 : 2 * sa.depth)), dim3(kStatsThreads),
                           0, stream, sa);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    } else {
        hipLaunchKernelGGL(reset_count_kernel, dim3(1), dim3(64), 0, stream, sa.redo_count);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = record(ln, 1, stream)) != hipSuccess) return err;
    auto walk = [&]() {
        if (spectr)
            hipLaunchKernelGGL((sv::walk_kernel<kWalkThreads, RD, E, true>), dim3(in->B),
                               dim3(kWalkThreads), 0, stream, wa);
        else
            hipLaunchKernelGGL((sv::walk_kernel<kWalkThreads, RD, E>), dim3(in->B),
                               dim3(kWalkThreads), 0, stream, wa);
        return hipGetLastError();
    };
    if ((err = walk()) != hipSuccess) return err;
    if ((err = record(ln, 2, stream)) != hipSuccess) return err;
    if (two_round) {
        // the listed rows: at most 2*B*K*L, usually a few thousand; each block
        // takes rows grid-stride from the list
        sa.mode = sv::kSelectListed;
        const long long most = 2LL * in->B * in->K * in->L;
        const unsigned grid2 = static_cast<unsigned>(most < kListGrid ? most : kListGrid);
        hipLaunchKernelGGL((sv::rowstats_kernel<kStatsThreads, RD, E>), dim3(grid2),
                           dim3(kStatsThreads), 0, stream, sa);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    if ((err = record(ln, 3, stream)) != hipSuccess) return err;
    if (two_round) {
        wa.round = 2;   // only the stopped walks run
        if ((err = walk()) != hipSuccess) return err;
    }
    if ((err = launch_redo<E, VEC>(in, out, stream, wa.method, wa.redo_count, wa.redo_list,
                                   ws + lay.stats, wa.dec, wa.rho_rec, ws + lay.team)) != hipSuccess)
        return err;
    return record(ln, 4, stream);
}

// Bytes of workspace a call needs: the walk's layout, or for one draft the
// single-draft layout when it is larger (the two are never used together).
size_t workspace_total(int32_t B, int32_t K, int32_t L, int32_t V) {
    size_t n = layout(B, K, L).total;
    if (K == 1) {
        const size_t s = single_layout(B, L, V).total;
        if (s > n) n = s;
    }
    return n;
}

constexpr long long kMaxSingleGrid = 1LL << 20;

template <typename E, bool VEC>
hipError_t launch_single(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln,
                         int method) {
    using RD = typename sv::RowOf<E, VEC>::type;
    constexpr int NT = sv::kSingleThreads;
    hipStream_t stream = static_cast<hipStream_t>(ln->stream);
    const SingleLayout lay = single_layout(in->B, in->L, in->V);
    char *ws = static_cast<char *>(ln->workspace);
    sv::SingleArgs a;
    a.tgt = in->target_logits;
    a.drf = in->draft_logits;
    a.tok = in->draft_tokens;
    a.temp = in->temperature;
    a.ua = in->u_accept;
    a.uc = in->u_correct;
    a.part = reinterpret_cast<sv::SliceStat *>(ws + lay.part);
    a.rpart = reinterpret_cast<double *>(ws + lay.rpart);
    a.prep = reinterpret_cast<sv::SinglePrep *>(ws + lay.prep);
    a.B = in->B;
    a.L = in->L;
    a.V = in->V;
    a.NS = lay.NS;
    a.method = method;
    a.accept_len = out->accept_len;
    a.draft_index = out->draft_index;
    a.correction = out->correction;
    a.flags = out->flags;
    a.rows_streamed = out->rows_streamed;
    a.row_lse = out->row_lse;
    a.accept_prob = out->accept_prob;
    a.resid_mass = out->resid_mass;
    auto grid = [](long long n) {
        return static_cast<unsigned>(n < kMaxSingleGrid ? n : kMaxSingleGrid);
    };
    const long long n1 = static_cast<long long>(in->B) * (2 * in->L + 1) * lay.NS;
    const long long n2 = static_cast<long long>(in->B) * (in->L + 1) * lay.NS;
    hipError_t err;
    if ((err = record(ln, 0, stream)) != hipSuccess) return err;
    hipLaunchKernelGGL((sv::single_stats_kernel<NT, RD, E>), dim3(grid(n1)), dim3(NT), 0, stream, a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    if ((err = record(ln, 1, stream)) != hipSuccess) return err;
    hipLaunchKernelGGL((sv::single_prep_kernel<NT, RD, E>), dim3(grid(in->B)), dim3(NT), 0, stream,
                       a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((sv::single_partial_kernel<NT, RD, E>), dim3(grid(n2)), dim3(NT), 0, stream,
                       a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    hipLaunchKernelGGL((sv::single_final_kernel<NT, RD, E>), dim3(grid(in->B)), dim3(NT), 0, stream,
                       a);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    for (int i = 2; i < 5; ++i)
        if ((err = record(ln, i, stream)) != hipSuccess) return err;
    return hipSuccess;
}

int verify(int method, const sv_inputs *in, const sv_outputs *out, const sv_launch *ln,
           bool single_draft) {
    if (!in || !out || !ln) return SV_EINVAL;
    if (!sizes_ok(in->B, in->K, in->L, in->V, in->dtype)) return SV_EINVAL;
    if (single_draft && in->K != 1) return SV_EINVAL;
    if (in->B == 0) return SV_OK;
    if (!in->target_logits || !in->draft_logits || !in->draft_tokens || !in->temperature ||
        !in->u_accept || !in->u_correct)
        return SV_EINVAL;
    if (!out->accept_len || !out->draft_index || !out->correction) return SV_EINVAL;
    const size_t es = in->dtype == SV_F32 ? 4 : 2;
    const uintptr_t ta = reinterpret_cast<uintptr_t>(in->target_logits);
    const uintptr_t da = reinterpret_cast<uintptr_t>(in->draft_logits);
    if (ta % es || da % es) return SV_EINVAL;
    if (in->row_stats && reinterpret_cast<uintptr_t>(in->row_stats) % 16) return SV_EINVAL;
    if (!ln->workspace || reinterpret_cast<uintptr_t>(ln->workspace) % 256) return SV_EWORKSPACE;
    if (ln->workspace_bytes < workspace_total(in->B, in->K, in->L, in->V)) return SV_EWORKSPACE;

    const bool vec = (in->V % 8 == 0) && (ta % 16 == 0) && (da % 16 == 0);
    hipError_t err;
    if (in->K == 1 && !in->row_stats) {
        // one draft: split across the vocabulary (SpecTr with one candidate is the
        // token-level rule)
        const int m1 = (method == sv::kMethodSpecTr || method == sv::kMethodSpecTrBisect)
                           ? sv::kMethodToken : method;
        if (in->dtype == SV_BF16)
            err = vec ? launch_single<uint16_t, true>(in, out, ln, m1)
                      : launch_single<uint16_t, false>(in, out, ln, m1);
        else
            err = vec ? launch_single<float, true>(in, out, ln, m1)
                      : launch_single<float, false>(in, out, ln, m1);
        return err == hipSuccess ? SV_OK : SV_EHIP;
    }
    if (in->dtype == SV_BF16)
        err = vec ? launch<uint16_t, true>(in, out, ln, method)
                  : launch<uint16_t, false>(in, out, ln, method);
    else
        err = vec ? launch<float, true>(in, out, ln, method)
                  : launch<float, false>(in, out, ln, method);
    return err == hipSuccess ? SV_OK : SV_EHIP;
}

constexpr long long kDraftTileGrid = 16384;

// Drafting workspace: request flags | per-position list lengths | listed rows
// (two buffers, by position parity) | each draft's list slot | tile shifts |
// tile sums.
struct DraftLayout {
    size_t bad, count, list, slot, tmax, tsum, total;
    int ntiles;
};

DraftLayout draft_layout(int32_t B, int32_t K, int32_t V) {
    DraftLayout l;
    const int nch = (V + sv::kChunk - 1) / sv::kChunk;
    l.ntiles = (nch + sv::kDraftTileChunks - 1) / sv::kDraftTileChunks;
    const size_t bk = static_cast<size_t>(B) * K;
    l.bad = 0;
    l.count = align_up(static_cast<size_t>(B) * sizeof(unsigned), 256);
    l.list = l.count + 256;
    l.slot = l.list + align_up(2 * bk * sizeof(int32_t), 256);
    l.tmax = l.slot + align_up(bk * sizeof(int32_t), 256);
    l.tsum = l.tmax + align_up(bk * l.ntiles * sizeof(float), 256);
    l.total = l.tsum + align_up(bk * l.ntiles * sizeof(double), 256);
    return l;
}

template <typename E, bool VEC>
hipError_t launch_draft(const sv_draft_inputs *in, const sv_draft_outputs *out,
                        const sv_launch *ln) {
    using RD = typename sv::RowOf<E, VEC>::type;
    constexpr int NT = 256;
    hipStream_t stream = static_cast<hipStream_t>(ln->stream);
    const DraftLayout lay = draft_layout(in->B, in->K, in->V);
    char *ws = static_cast<char *>(ln->workspace);
    sv::DraftArgs a;
    a.drf = in->draft_logits;
    a.temp = in->temperature;
    a.ud = in->u_draft;
    a.tok = out->draft_tokens;
    a.bad = reinterpret_cast<unsigned *>(ws + lay.bad);
    a.count = reinterpret_cast<unsigned *>(ws + lay.count);
    a.list = reinterpret_cast<int32_t *>(ws + lay.list);
    a.slot = reinterpret_cast<int32_t *>(ws + lay.slot);
    a.tmax = reinterpret_cast<float *>(ws + lay.tmax);
    a.tsum = reinterpret_cast<double *>(ws + lay.tsum);
    a.rows = out->rows_streamed;
    a.B = in->B;
    a.K = in->K;
    a.L = in->L;
    a.V = in->V;
    a.ntiles = lay.ntiles;
    const unsigned bk = static_cast<unsigned>(in->B) * static_cast<unsigned>(in->K);
    const long long blocks = (static_cast<long long>(bk) * lay.ntiles + 3) / 4;   // 4 waves each
    const unsigned tile_grid = static_cast<unsigned>(blocks < kDraftTileGrid ? blocks : kDraftTileGrid);
    hipError_t err;
    if ((err = record(ln, 0, stream)) != hipSuccess) return err;
    const int n0 = in->B > in->L ? in->B : in->L;
    hipLaunchKernelGGL(sv::draft_init_kernel, dim3((n0 + 255) / 256), dim3(256), 0, stream, a.bad,
                       a.rows, a.count, in->B, in->L);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    // with K <= 16 the draws of position j and the node rows of position j + 1
    // share a launch (one workgroup per request)
    const bool fused = in->K <= sv::kDraftFusedMaxK;
    for (int j = 0; j < in->L; ++j) {
        a.j = j;
        if (j == 0 || !fused) {
            hipLaunchKernelGGL(sv::draft_nodes_kernel, dim3((in->B + 3) / 4), dim3(256), 0, stream,
                               a);
            if ((err = hipGetLastError()) != hipSuccess) return err;
        }
        hipLaunchKernelGGL((sv::draft_tiles_kernel<NT, RD, E>), dim3(tile_grid), dim3(NT), 0,
                           stream, a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
        if (fused)
            hipLaunchKernelGGL((sv::draft_pick_next_kernel<RD, E>), dim3(in->B),
                               dim3(in->K * sv::kWave), 0, stream, a);
        else
            hipLaunchKernelGGL((sv::draft_pick_kernel<NT, RD, E>), dim3((bk + 3) / 4), dim3(NT), 0,
                               stream, a);
        if ((err = hipGetLastError()) != hipSuccess) return err;
    }
    const long long n = static_cast<long long>(in->B) * in->K * in->L;
    hipLaunchKernelGGL(sv::draft_fixup_kernel, dim3(static_cast<unsigned>((n + 255) / 256)),
                       dim3(256), 0, stream, a.bad, out->draft_tokens, out->flags, in->B,
                       in->K * in->L);
    if ((err = hipGetLastError()) != hipSuccess) return err;
    return record(ln, 1, stream);
}

// LM-head workspace: per row and column block, the partial maximum and sum.
struct LmLayout {
    size_t pmax, psum, total;
    int nbm, nbn;
};

LmLayout lm_layout(int32_t R, int32_t V) {
    LmLayout l;
    l.nbm = (R + sv::kLmBM - 1) / sv::kLmBM;
    l.nbn = (V + sv::kLmBN - 1) / sv::kLmBN;
    const size_t n = static_cast<size_t>(R) * l.nbn;
    l.pmax = 0;
    l.psum = align_up(n * sizeof(float), 256);
    l.total = l.psum + align_up(n * sizeof(double), 256);
    if (l.total == 0) l.total = 256;
    return l;
}

bool lm_sizes_ok(int32_t R, int32_t d, int32_t V) {
    return R >= 0 && R <= (1 << 26) && d >= sv::kLmDMin && d <= 65536 && d % sv::kLmDStep == 0 &&
           V >= 1 && V <= SV_MAX_V;
}

size_t draft_workspace_bytes(int32_t B, int32_t K, int32_t V) {
    return draft_layout(B, K, V).total;
}

}  // namespace

// Scratch of spec_verify_multidraft_noalloc: the workspace of a multi-draft call,
// held by the library in device memory of its own (one copy on every device the
// library is used on, for the life of the process), for callers that cannot
// allocate.  In host code `scratch` names a host-side stand-in, not the device
// array: kernels receive the address hipGetSymbolAddress reports for the
// current device, kept per device below.
static_assert(SV_NOALLOC_SCRATCH_BYTES % 256 == 0, "scratch size");
static __device__ __align__(256) unsigned char scratch[SV_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on device `dev`, looked up once per device
// with that device current.  nullptr if the lookup fails.
void *scratch_on(int dev) {
    if (dev < 0 || dev >= kMaxDevices) return nullptr;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch_ptr[dev]) return g_scratch_ptr[dev];
    int cur = -1;
    if (hipGetDevice(&cur) != hipSuccess) return nullptr;
    if (cur != dev && hipSetDevice(dev) != hipSuccess) return nullptr;
    void *ptr = nullptr;
    const hipError_t err = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (cur != dev && hipSetDevice(cur) != hipSuccess) return nullptr;
    if (err != hipSuccess || !ptr || reinterpret_cast<uintptr_t>(ptr) % 256) return nullptr;
    g_scratch_ptr[dev] = ptr;
    return ptr;
}

}  // namespace

extern "C" {

size_t sv_lm_workspace_size(int32_t R, int32_t d, int32_t V) {
    if (!lm_sizes_ok(R, d, V)) return 0;
    return lm_layout(R, V).total;
}

int spec_lm_head(const sv_lm_inputs *in, const sv_lm_outputs *out, const sv_launch *ln) {
    if (!in || !out || !ln) return SV_EINVAL;
    if (!lm_sizes_ok(in->R, in->d, in->V)) return SV_EINVAL;
    if (in->R == 0) return SV_OK;
    if (!in->hidden || !in->weight || !in->temperature || !out->logits) return SV_EINVAL;
    if (out->logits_dtype != SV_F32 && out->logits_dtype != SV_BF16) return SV_EINVAL;
    if (reinterpret_cast<uintptr_t>(in->hidden) % 16 || reinterpret_cast<uintptr_t>(in->weight) % 16)
        return SV_EINVAL;
    if (out->row_stats && (out->stats_group < 1 || out->stats_stride < out->stats_group ||
                           out->stats_offset < 0 ||
                           reinterpret_cast<uintptr_t>(out->row_stats) % 16))
        return SV_EINVAL;
    const LmLayout lay = lm_layout(in->R, in->V);
    if (!ln->workspace || reinterpret_cast<uintptr_t>(ln->workspace) % 256) return SV_EWORKSPACE;
    if (ln->workspace_bytes < lay.total) return SV_EWORKSPACE;
    hipStream_t stream = static_cast<hipStream_t>(ln->stream);
    char *ws = static_cast<char *>(ln->workspace);
    sv::LmArgs a;
    a.h = static_cast<const uint16_t *>(in->hidden);
    a.w = static_cast<const uint16_t *>(in->weight);
    a.temp = in->temperature;
    a.logits = out->logits;
    a.bf16_out = out->logits_dtype == SV_BF16 ? 1 : 0;
    a.pmax = reinterpret_cast<float *>(ws + lay.pmax);
    a.psum = reinterpret_cast<double *>(ws + lay.psum);
    a.R = in->R;
    a.d = in->d;
    a.V = in->V;
    a.nbm = lay.nbm;
    a.nbn = lay.nbn;
    if (record(ln, 0, stream) != hipSuccess) return SV_EHIP;
    hipLaunchKernelGGL(sv::lm_head_kernel, dim3(static_cast<unsigned>(lay.nbm) * lay.nbn),
                       dim3(sv::kLmThreads), 0, stream, a);
    if (hipGetLastError() != hipSuccess) return SV_EHIP;
    if (out->row_stats) {
        sv::LmStatsArgs s;
        s.pmax = a.pmax;
        s.psum = a.psum;
        s.temp = in->temperature;
        s.stats = out->row_stats;
        s.R = in->R;
        s.nbn = lay.nbn;
        s.group = out->stats_group;
        s.stride = out->stats_stride;
        s.offset = out->stats_offset;
        hipLaunchKernelGGL(sv::lm_stats_kernel, dim3((in->R + 3) / 4), dim3(256), 0, stream, s);
        if (hipGetLastError() != hipSuccess) return SV_EHIP;
    }
    return record(ln, 1, stream) == hipSuccess ? SV_OK : SV_EHIP;
}

size_t sv_draft_workspace_size(int32_t B, int32_t K, int32_t L, int32_t V, int32_t dtype) {
    if (!sizes_ok(B, K, L, V, dtype)) return 0;
    return draft_workspace_bytes(B, K, V);
}

int spec_draft_sample(const sv_draft_inputs *in, const sv_draft_outputs *out,
                      const sv_launch *ln) {
    if (!in || !out || !ln) return SV_EINVAL;
    if (!sizes_ok(in->B, in->K, in->L, in->V, in->dtype)) return SV_EINVAL;
    if (in->B == 0) return SV_OK;
    if (!in->draft_logits || !in->temperature || !in->u_draft || !out->draft_tokens)
        return SV_EINVAL;
    const size_t es = in->dtype == SV_F32 ? 4 : 2;
    const uintptr_t da = reinterpret_cast<uintptr_t>(in->draft_logits);
    if (da % es) return SV_EINVAL;
    if (!ln->workspace || reinterpret_cast<uintptr_t>(ln->workspace) % 256) return SV_EWORKSPACE;
    if (ln->workspace_bytes < draft_workspace_bytes(in->B, in->K, in->V)) return SV_EWORKSPACE;
    const bool vec = (in->V % 8 == 0) && (da % 16 == 0);
    hipError_t err;
    if (in->dtype == SV_BF16)
        err = vec ? launch_draft<uint16_t, true>(in, out, ln)
                  : launch_draft<uint16_t, false>(in, out, ln);
    else
        err = vec ? launch_draft<float, true>(in, out, ln)
                  : launch_draft<float, false>(in, out, ln);
    return err == hipSuccess ? SV_OK : SV_EHIP;
}


size_t sv_workspace_size(int32_t B, int32_t K, int32_t L, int32_t V, int32_t dtype) {
    if (!sizes_ok(B, K, L, V, dtype)) return 0;
    const size_t n = workspace_total(B, K, L, V);
    return n ? n : 256;
}

int spec_verify_token(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln) {
    return verify(sv::kMethodToken, in, out, ln, true);
}

int spec_verify_block(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln) {
    return verify(sv::kMethodBlockWalk, in, out, ln, true);
}

int spec_verify_multidraft(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln) {
    return verify(sv::kMethodBlockWalk, in, out, ln, false);
}

int spec_verify_spectr(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln) {
    return verify(sv::kMethodSpecTr, in, out, ln, false);
}

int spec_verify_spectr_bisect(const sv_inputs *in, const sv_outputs *out, const sv_launch *ln) {
    return verify(sv::kMethodSpecTrBisect, in, out, ln, false);
}

int spec_verify_multidraft_noalloc(const sv_inputs *in, const sv_outputs *out, void *stream) {
    if (!in || !out) return SV_EINVAL;
    if (!sizes_ok(in->B, in->K, in->L, in->V, in->dtype)) return SV_EINVAL;
    if (workspace_total(in->B, in->K, in->L, in->V) > SV_NOALLOC_SCRATCH_BYTES)
        return SV_EUNSUPPORTED;
    if (in->B == 0) return SV_OK;
    int dev = -1;
    if (stream) {
        if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess)
            return SV_EHIP;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return SV_EHIP;
    }
    void *ws = scratch_on(dev);
    if (!ws) return SV_EHIP;
    sv_launch ln;
    std::memset(&ln, 0, sizeof ln);
    ln.stream = stream;
    ln.workspace = ws;
    ln.workspace_bytes = SV_NOALLOC_SCRATCH_BYTES;
    return verify(sv::kMethodBlockWalk, in, out, &ln, false);
}

const char *sv_status_string(int status) {
    switch (status) {
        case SV_OK: return "ok";
        case SV_EINVAL: return "invalid argument";
        case SV_EUNSUPPORTED: return "unsupported dtype or size";
        case SV_EHIP: return "HIP runtime error";
        case SV_EWORKSPACE: return "workspace missing, misaligned or too small";
        default: return "unknown status";
    }
}

const char *sv_version(void) { return "0.2.0"; }

}  // extern "C"
