// sv_lmhead.hpp -- the LM head with the verifier's row statistics in its epilogue.
//
// The verifier's inputs are logit rows, produced by the target and draft
// models' LM heads: logits = h W^T over hidden states h [R][d] and the
// vocabulary projection W [V][d] (bf16).  Verification is a large share of a
// speculative-decoding step (the performance study's page, section 1); here
// the first thing the verifier does with a row -- its temperature-softmax
// statistics (shift M, sum S = sum_v 2^(l_v c - K), c = log2(e)/T, K the row
// constant of the shift, in the exponent convention of every kernel here) -- is computed
// while the row is still in registers, so the statistics pass over the logits
// disappears.  The logits are still written, fp32 or rounded to bf16 (half the
// bytes; the statistics are then those of the rounded values): the walk's
// residual sweeps and correction draws read whole rows.
//
// lm_head_kernel: one 256-thread workgroup (one per CU: 128 KB of LDS, 256
// AGPRs per lane) per 256 x 256 output tile, four waves in a 2 x 2 arrangement
// each owning a 128 x 128 quarter (8 x 8 MFMA 16x16x32 bf16 tiles, 256 fp32
// accumulators per lane).  At that size a wave reads 16 KB of fragments from
// LDS per 64 MFMAs, half the LDS and L2 traffic per flop of a 64 x 64 wave
// tile.  The k dimension runs in regions of 32 columns between barriers; a
// wave computes region s from fragments it read during region s-1 while it
// reads those of region s+1, one read per four MFMAs.  Tiles reach LDS through
// buffer loads that write LDS directly (no registers, no LDS store
// instructions), 64 columns -- one 128-byte line per row -- at a time, into
// two stages: a stage's 16 loads per wave are issued one per four MFMAs of the
// region two regions before its first fragments are read (issued back to back
// they stall the wave behind the load queue: 0.94 against 1.1 PFLOP/s).  The MFMA operand A is the vocabulary tile and B the
// hidden-state tile, so a lane's four accumulators of a 16 x 16 tile are four
// consecutive vocabulary entries of one output row: the epilogue stores them
// as one 8- or 16-byte write and reduces a row with two cross-lane steps.
// Blocks are ordered in groups of row-blocks so a group reuses each vocabulary
// tile from L2, and remapped so that consecutive blocks of the order land on
// the same XCD.  The epilogue writes the tile and, per row, the partial
// (max, sum) over its 256 columns; a combine kernel folds the partials of a
// row into (M, S).
#pragma once

#include "sv_device.hpp"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kLmBM = 256, kLmBN = 256, kLmBK = 32;   // kLmBK: columns per region
constexpr int kLmThreads = 256;
constexpr int kLmStageK = 64;            // columns per LDS stage: one 128-byte line per row
constexpr int kLmStages = 2;             // 2 x (two 256 x 64 tiles) = 128 KB
constexpr int kLmTileElems = kLmBM * kLmStageK;
constexpr int kLmDStep = kLmStageK;      // d must be a multiple
constexpr int kLmDMin = 2 * kLmStageK;   // and at least the pipeline's last two stages
constexpr int kLmPastEnd = 0x3ff80000;   // a column offset whose byte offset no buffer range covers
constexpr int kLmGroupM = 8;             // row-blocks per group of the block order
constexpr int kXcds = 8;

typedef __attribute__((address_space(3))) void *lds_void_ptr;
__device__ __forceinline__ lds_void_ptr lds_ptr(uint16_t *p) { return (lds_void_ptr)p; }

// Buffer descriptor (as four words) over rows r0.. of a [rows][d] bf16 matrix:
// base, no stride, byte range clamped to 32 bits, raw 32-bit data format.
typedef int intx4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ intx4 lm_desc(const uint16_t *m, int r0, int rows, int d) {
    const long long bytes = static_cast<long long>(rows - r0) * d * 2;
    const uint64_t base = reinterpret_cast<uint64_t>(m + static_cast<long long>(r0) * d);
    return intx4{static_cast<int>(base & 0xffffffffu), static_cast<int>((base >> 32) & 0xffffu),
                 static_cast<int>(bytes < 0x7fffffffLL ? bytes : 0x7fffffffLL), 0x00020000};
}

// 16 bytes per lane from global memory (buffer range checked: zeros past the
// range) straight into LDS: lane l's bytes land at LDS address lds + 16 l.
// Issued as inline assembly so that the compiler, which cannot tell the stage
// a load writes from the stage a fragment read reads, does not wait for every
// such load before each LDS read; the kernel orders them itself with explicit
// vector-memory waits before its barriers.
// (m0 is reserved to the compiler, which warns that a clobber of it may not be
// honoured; nothing else in the LM-head kernel uses m0, each load sets it.)
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(uint32_t lds, int voff, intx4 desc, int soff) {
    asm volatile(
        "s_mov_b32 m0, %0\n\t"
        "s_nop 0\n\t"
        "buffer_load_dwordx4 %1, %2, %3 offen lds"
        :
        : "s"(lds), "v"(voff), "s"(desc), "s"(soff)
        : "memory", "m0");
}
#pragma clang diagnostic pop


// fp32 to bf16, round to nearest even (finite values; the LM head's logits are
// finite sums of finite products).
__device__ __forceinline__ uint16_t bf16_rne(float x) {
    const uint32_t u = __float_as_uint(x);
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

struct LmArgs {
    const uint16_t *h;      // [R][d] bf16 bits
    const uint16_t *w;      // [V][d] bf16 bits
    const float *temp;      // [R]: temperature of each row
    void *logits;           // [R][V] fp32, or bf16 bits when bf16_out
    int bf16_out;           // round the logits to bf16 (statistics from the rounded values)
    float *pmax;            // [R][nbn]: per column block, the row's maximum
    double *psum;           // [R][nbn]: and sum_v 2^((l_v - max) c) over the block
    int R, d, V, nbm, nbn;
};

__device__ __forceinline__ void lm_block_coords(int pid, int nbm, int nbn, int *bm, int *bn) {
    const int n = nbm * nbn;
    if (n % kXcds == 0) {                 // blocks go to XCDs round-robin: make runs local
        const int per = n / kXcds;
        pid = (pid % kXcds) * per + pid / kXcds;
    }
    const int in_group = kLmGroupM * nbn;
    const int g = pid / in_group;
    const int first = g * kLmGroupM;
    const int gsize = min(kLmGroupM, nbm - first);
    const int r = pid % in_group;
    *bm = first + r % gsize;
    *bn = r / gsize;
}

// acc += A B^T for one 16 x 16 x 32 step, the accumulator pinned to an AGPR
// quad.  (With 256 accumulators per lane and 128 fragment registers live, the
// compiler's own choice spreads accumulators over both register files and
// copies them between MFMAs.)  As volatile assembly the MFMAs keep the order
// they are written in, relative to each other and to the LDS reads between
// them, which is the interleave the kernel spells out.  The compiler still
// places the waits for the LDS reads an MFMA's operands come from; what it
// does not see: (a) an accumulator is read by ordinary instructions only after
// the wait states that follow the last MFMAs (below); (b) an LDS read may
// reuse the registers of a fragment whose last MFMA was issued a few
// instructions earlier -- the MFMA takes its A and B operands when it starts,
// and the read's data arrives tens of cycles after the read issues, by which
// time the earlier MFMA has finished.
__device__ __forceinline__ void mfma_acc(floatx4 &acc, const bf16x8 &a, const bf16x8 &b) {
    asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

template <int N> struct Par { static constexpr int value = N; };
template <bool B> struct Flag { static constexpr bool value = B; };

__global__ __launch_bounds__(kLmThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void lm_head_kernel(
    LmArgs A) {
    // [stage][0: hidden tile, 1: vocabulary tile][256 rows x 64 columns]; the
    // 16-byte chunk c (k = 8c .. 8c+7) of row r sits in slot c ^ (r % 8) of the
    // row's 128 bytes, so the 8 rows that 8 lanes of a fragment read touch at one
    // c fall in 8 distinct bank groups.
    __shared__ __attribute__((aligned(1024))) uint16_t sT[kLmStages][2][kLmTileElems];
    // the epilogue's per-row partials reuse stage 0 once the loop is done
    float(*s_m)[kLmBM] = reinterpret_cast<float(*)[kLmBM]>(&sT[0][0][0]);
    double(*s_s)[kLmBM] = reinterpret_cast<double(*)[kLmBM]>(&sT[0][1][0]);
    __shared__ float s_temp[kLmBM];   // the tile rows' temperatures, read before the loop

    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
    const int wv = wave & 1, wh = wave >> 1;   // vocabulary half, hidden-row half
    int bm, bn;
    lm_block_coords(blockIdx.x, A.nbm, A.nbn, &bm, &bn);
    const int row0 = bm * kLmBM, col0 = bn * kLmBN;
    const int R = A.R, d = A.d, V = A.V;

    // Tiles reach LDS by buffer loads that write LDS directly: one instruction
    // moves 64 lanes x 16 bytes to 1 KB of consecutive LDS, here 8 whole tile
    // rows (128-byte lines).  Wave w fills rows w*64 .. w*64+63 of both tiles,
    // 8 instructions each; lane l loads the chunk that belongs in slot l % 8 of
    // row l / 8.  Rows past the matrix read as zeros (hardware range check of
    // the buffer resource).
    // (loaded here so the epilogue waits on no global load: a load there would
    // also wait for every logits store before it)
    s_temp[tid] = row0 + tid < R ? A.temp[row0 + tid] : 1.0f;   // kLmThreads == kLmBM
    int voff[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int r = wave * 64 + i * 8 + (lane >> 3);
        voff[i] = (r * d + (((lane & 7) ^ (r & 7)) * 8)) * 2;
    }
    const intx4 dH = lm_desc(A.h, row0, R, d), dW = lm_desc(A.w, col0, V, d);
    const uint32_t lds0 = static_cast<uint32_t>(reinterpret_cast<uintptr_t>(lds_ptr(&sT[0][0][0]))) +
                          wave * 64 * kLmStageK * 2;
    // load j (0..15) of a stage: rows 8(j % 8) .. of the wave's share of the
    // hidden tile (j < 8) or of the vocabulary tile (j >= 8)
    auto load_one = [&](int k0, int buf, int j) __attribute__((always_inline)) {
        const uint32_t base = lds0 + buf * (2 * kLmTileElems * 2) + (j >> 3) * (kLmTileElems * 2);
        lds_dma16(base + (j & 7) * 8 * kLmStageK * 2, voff[j & 7], j < 8 ? dH : dW, k0 * 2);
    };
    auto load_stage = [&](int k0, int buf) __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < 16; ++j) load_one(k0, buf, j);
    };
    // fragment t of matrix m (0 hidden, 1 vocabulary) for the wave's half
    // `half`, of region step s: rows half*128 + t*16 + lane%16, k = 8*(lane/16)
    // within the step's 32 columns (chunk 4*(s%2) + lane/16 of the stage)
    const int fo0 = (lane & 15) * kLmStageK + ((((lane >> 4)) ^ (lane & 7)) * 8);
    const int fo1 = (lane & 15) * kLmStageK + (((4 + (lane >> 4)) ^ (lane & 7)) * 8);
    auto read_frag = [&](int buf, int h, int m, int half, int t) __attribute__((always_inline)) {
        return *reinterpret_cast<const bf16x8 *>(&sT[buf][m][(half * 128 + t * 16) * kLmStageK] +
                                                 (h ? fo1 : fo0));
    };

    floatx4 acc[8][8];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < 8; ++b) acc[a][b] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // Wait states after the MFMAs issued so far, before any accumulator is read
    // or copied.  The compiler does not know the MFMAs are MFMAs, so it could
    // place such a read (or a copy between registers, where it reshuffles them
    // between the loop and the code after it) right behind the MFMA that writes
    // it; every accumulator therefore passes through a volatile statement
    // ordered after the wait states, and its later uses depend on that.
    auto acc_fence = [&]() __attribute__((always_inline)) {
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7"
                     : "+a"(acc[7][0]), "+a"(acc[7][1]), "+a"(acc[7][2]), "+a"(acc[7][3]),
                       "+a"(acc[7][4]), "+a"(acc[7][5]), "+a"(acc[7][6]), "+a"(acc[7][7]));
#pragma unroll
        for (int a = 0; a < 7; ++a)
            asm volatile(""
                         : "+a"(acc[a][0]), "+a"(acc[a][1]), "+a"(acc[a][2]), "+a"(acc[a][3]),
                           "+a"(acc[a][4]), "+a"(acc[a][5]), "+a"(acc[a][6]), "+a"(acc[a][7]));
    };

    // Regions of 32 columns: region s computes step s from fragments read
    // during region s-1 (register set s % 2) and reads step s+1's.  Stage J % 2
    // holds columns 64J .. 64J+63 (steps 2J, 2J+1).  Odd region 2J+1 issues the
    // loads of stage-step J+2 into the stage stage-step J used (whose last
    // fragments were read during region 2J, before the barrier that ends it);
    // even region 2J+2 ends by waiting for them and a barrier, before step
    // 2J+4's fragments are read in region 2J+3.
    const int nk = d / kLmBK;     // even
    const int nj = d / kLmStageK; // >= 2
    bf16x8 wf[2][8], hf[2][8];
    load_stage(0, 0);
    load_stage(kLmStageK, 1);
    asm volatile("s_waitcnt vmcnt(16)" ::: "memory");   // stage-step 0
    __syncthreads();
    wf[0][0] = read_frag(0, 0, 1, wv, 0);
#pragma unroll
    for (int t = 0; t < 8; ++t) hf[0][t] = read_frag(0, 0, 0, wh, t);
#pragma unroll
    for (int t = 1; t < 8; ++t) wf[0][t] = read_frag(0, 0, 1, wv, t);
    auto region = [&](int r, auto par, auto load, auto read) __attribute__((always_inline)) {
        constexpr int P = decltype(par)::value, Q = P ^ 1;   // P = r % 2
        constexpr bool LOAD = decltype(load)::value, READ = decltype(read)::value;
        // loads of stage-step (r+3)/2; past the last one, an offset no buffer
        // reaches, so the loads return zeros without touching memory
        const int kl = ((r + 3) >> 1) < nj ? ((r + 3) >> 1) * kLmStageK : kLmPastEnd;
        const int sl = ((r + 3) >> 1) & 1;
        const int sn = ((r + 1) >> 1) & 1;   // stage of step r+1 (its half is Q)
#pragma unroll
        for (int a = 0; a < 8; ++a) {
#pragma unroll
            for (int b = 0; b < 8; ++b) {
                mfma_acc(acc[a][b], wf[P][a], hf[P][b]);
                // the stage's 16 loads spread over the region, one per four MFMAs
                if constexpr (LOAD) {
                    if ((b & 3) == 0) load_one(kl, sl, a * 2 + (b >> 2));
                }
                if constexpr (READ) {
                    if ((b & 3) == 3) {
                        // step r+1's reads in the order its MFMAs use them
                        const int t = a * 2 + (b >> 2);
                        if (t == 0)
                            wf[Q][0] = read_frag(sn, Q, 1, wv, 0);
                        else if (t <= 8)
                            hf[Q][t - 1] = read_frag(sn, Q, 0, wh, t - 1);
                        else
                            wf[Q][t - 8] = read_frag(sn, Q, 1, wv, t - 8);
                    }
                }
            }
        }
        // only even regions end in a barrier: it publishes stage-step (r+2)/2
        // (loaded during region r-1) and frees the stage region r+1 loads into
        // (its last fragments were read during region r)
        if constexpr (P == 0) {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
        }
    };
    using T = Flag<true>;
    using F = Flag<false>;
    // Every pair of regions is the same code, the last ones included: their loads
    // past the last stage-step return zeros from outside every buffer, and their
    // reads of fragments past the last step (into stages no MFMA then uses) read
    // whatever is there.  (Separate code for the last regions would hold the
    // accumulators in other registers, and the copies the compiler then makes
    // cannot be kept clear of the MFMAs.)
    for (int r = 0; r < nk; r += 2) {   // nk is even
        region(r, Par<0>{}, F{}, T{});
        region(r + 1, Par<1>{}, T{}, T{});
        // wait states inside the loop, so that any copy the compiler places after
        // it follows them (~1% of a pair of regions)
        asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
    }
    acc_fence();
    (void)nk;
    // epilogue: lane holds, of tile (a, b), the vocabulary entries
    // a*16 + 4*(lane/16) + i (i = 0..3) of hidden row b*16 + lane%16.  The
    // statistics describe the logits as stored (rounded to bf16 when they are).
    const bool vec = (V & 3) == 0;
    auto stored = [&](float x) __attribute__((always_inline)) {
        return A.bf16_out ? __uint_as_float(static_cast<uint32_t>(bf16_rne(x)) << 16) : x;
    };
    // (b is a template constant: a loop this large is not unrolled, and any
    // runtime index into acc would put it in scratch memory)
    // Column tests are selects, not branches (a branch per element costs more
    // than the element's arithmetic); the stores are guarded only in tiles that
    // reach past R or V (the test below is the same for the whole workgroup).
    const bool full = vec && row0 + kLmBM <= R && col0 + kLmBN <= V;
    auto epilogue_rows = [&](auto bc) __attribute__((always_inline)) {
        constexpr int b = decltype(bc)::value;
        const int rloc = wh * 128 + b * 16 + (lane & 15);
        const int row = row0 + rloc;
        const bool rok = row < R;
        float m = -INFINITY;
        float v[8][4];
        bool ok[8][4];
#pragma unroll
        for (int a = 0; a < 8; ++a) {
            const int col = col0 + wv * 128 + a * 16 + 4 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                ok[a][i] = col + i < V;
                v[a][i] = stored(acc[a][b][i]);
                m = fmaxf(m, ok[a][i] ? v[a][i] : -INFINITY);
            }
            const long long at = static_cast<long long>(row) * V + col;
            if (full) {
                if (A.bf16_out) {
                    *reinterpret_cast<uint2 *>(static_cast<uint16_t *>(A.logits) + at) =
                        make_uint2((__float_as_uint(v[a][0]) >> 16) | (__float_as_uint(v[a][1]) & 0xffff0000u),
                                   (__float_as_uint(v[a][2]) >> 16) | (__float_as_uint(v[a][3]) & 0xffff0000u));
                } else {
                    *reinterpret_cast<float4 *>(static_cast<float *>(A.logits) + at) =
                        make_float4(v[a][0], v[a][1], v[a][2], v[a][3]);
                }
            } else if (rok) {
                if (A.bf16_out) {
                    uint16_t *o = static_cast<uint16_t *>(A.logits) + at;
                    uint16_t hb[4];
#pragma unroll
                    for (int i = 0; i < 4; ++i) hb[i] = static_cast<uint16_t>(__float_as_uint(v[a][i]) >> 16);
                    if (vec && ok[a][3]) {
                        *reinterpret_cast<uint2 *>(o) =
                            make_uint2(hb[0] | (static_cast<uint32_t>(hb[1]) << 16),
                                       hb[2] | (static_cast<uint32_t>(hb[3]) << 16));
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (ok[a][i]) o[i] = hb[i];
                    }
                } else {
                    float *o = static_cast<float *>(A.logits) + at;
                    if (vec && ok[a][3]) {
                        *reinterpret_cast<float4 *>(o) = make_float4(v[a][0], v[a][1], v[a][2], v[a][3]);
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; ++i)
                            if (ok[a][i]) o[i] = v[a][i];
                    }
                }
            }
        }
        m = fmaxf(m, __shfl_xor(m, 16, kWave));
        m = fmaxf(m, __shfl_xor(m, 32, kWave));
        const Scale sc = temp_scale(s_temp[rloc]);
        const float msc = shift_term(m, sc);
        float e = 0.0f;
#pragma unroll
        for (int a = 0; a < 8; ++a)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float x = fast_exp2(expo(v[a][i], sc, msc));
                e += ok[a][i] ? x : 0.0f;
            }
        double s = static_cast<double>(e);
        s += __shfl_xor(s, 16, kWave);
        s += __shfl_xor(s, 32, kWave);
        if (lane < 16) {
            s_m[wv][rloc] = m;
            s_s[wv][rloc] = s;
        }
    };
    epilogue_rows(Par<0>{});
    epilogue_rows(Par<1>{});
    epilogue_rows(Par<2>{});
    epilogue_rows(Par<3>{});
    epilogue_rows(Par<4>{});
    epilogue_rows(Par<5>{});
    epilogue_rows(Par<6>{});
    epilogue_rows(Par<7>{});
    __syncthreads();
    {
        const int row = row0 + tid;   // kLmThreads == kLmBM
        if (row < R) {
            const Scale sc = temp_scale(s_temp[tid]);
            const float m0 = s_m[0][tid], m1 = s_m[1][tid];
            const float M = fmaxf(m0, m1);
            const double Mc = static_cast<double>(shift_term(M, sc));
            double S = 0.0;
            if (m0 > -INFINITY) S += s_s[0][tid] * exp2(static_cast<double>(shift_term(m0, sc)) - Mc);
            if (m1 > -INFINITY) S += s_s[1][tid] * exp2(static_cast<double>(shift_term(m1, sc)) - Mc);
            A.pmax[static_cast<long long>(row) * A.nbn + bn] = M;
            A.psum[static_cast<long long>(row) * A.nbn + bn] = S;
        }
    }
}
static_assert(kLmThreads == kLmBM, "one epilogue thread per tile row");

// The partials of row r folded into its statistics, written to slot
// (r / group) * stride + offset + r % group of a 16-byte {float M; float pad;
// double S} array (the verifier's node-row statistics layout).  One wave per row.
struct LmStatsArgs {
    const float *pmax;
    const double *psum;
    const float *temp;
    void *stats;
    int R, nbn, group, stride, offset;
};

__global__ __launch_bounds__(256) void lm_stats_kernel(LmStatsArgs A) {
    const int lane = threadIdx.x & (kWave - 1);
    const int r = blockIdx.x * (blockDim.x / kWave) + threadIdx.x / kWave;
    if (r >= A.R) return;
    const float *pm = A.pmax + static_cast<long long>(r) * A.nbn;
    const double *ps = A.psum + static_cast<long long>(r) * A.nbn;
    float m = -INFINITY;
    for (int i = lane; i < A.nbn; i += kWave) m = fmaxf(m, pm[i]);
    m = wave_max(m);
    const Scale sc = temp_scale(A.temp[r]);
    const double Mc = static_cast<double>(shift_term(m, sc));
    double s = 0.0;
    for (int i = lane; i < A.nbn; i += kWave)
        if (pm[i] > -INFINITY) s += ps[i] * exp2(static_cast<double>(shift_term(pm[i], sc)) - Mc);
    s = wave_sum(s);
    if (lane == 0) {
        const long long slot =
            static_cast<long long>(r / A.group) * A.stride + A.offset + r % A.group;
        char *p = static_cast<char *>(A.stats) + slot * 16;
        *reinterpret_cast<float *>(p) = fmaxf(m, -3.402823466e38f);
        *reinterpret_cast<float *>(p + 4) = 0.0f;
        *reinterpret_cast<double *>(p + 8) = s;
    }
}

}  // namespace sv
