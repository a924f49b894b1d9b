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
// lm_head_kernel: one 256-thread workgroup per 128 x 128 output tile, four waves
// in a 2 x 2 arrangement each owning 64 x 64 (4 x 4 MFMA 16x16x32 bf16 tiles),
// K stepped by 64 through double-buffered LDS (rows padded by 16 bytes against
// bank conflicts), with the global loads three steps ahead in registers.
// Blocks are ordered in groups of row-blocks so a group reuses each vocabulary
// tile from L2, and remapped so that consecutive blocks of the order land on
// the same XCD.  The epilogue writes the fp32
// tile and, per row, the partial (max, sum) over its 128 columns; a combine
// kernel folds the partials of a row into (M, S).
#pragma once

#include "sv_device.hpp"

namespace sv {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));

constexpr int kLmBM = 128, kLmBN = 128, kLmBK = 64;
constexpr int kLmThreads = 256;
constexpr int kLmStride = kLmBK + 8;     // LDS row stride in bf16 elements
constexpr int kLmGroupM = 16;            // row-blocks per group of the block order
constexpr int kXcds = 8;

template <int N> struct Stage { static constexpr int value = N; };

// Buffer resource over rows r0.. of a [rows][d] bf16 matrix (byte range clamped
// to 32 bits; the kernel's offsets within a tile stay below 128 rows).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t tile_rsrc(const uint16_t *m, int r0, int rows,
                                                            int d) {
    const long long bytes = static_cast<long long>(rows - r0) * d * 2;
    const int n = static_cast<int>(bytes < 0x7fffffffLL ? bytes : 0x7fffffffLL);
    return __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t *>(m + static_cast<long long>(r0) * d), 0, n, 0x00020000);
}

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

__global__ __launch_bounds__(kLmThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void lm_head_kernel(
    LmArgs A) {
    __shared__ __attribute__((aligned(16))) uint16_t sA[2][kLmBM * kLmStride];
    __shared__ __attribute__((aligned(16))) uint16_t sB[2][kLmBN * kLmStride];
    __shared__ float s_m[2][kLmBM];
    __shared__ double s_s[2][kLmBM];

    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
    const int wm = wave >> 1, wn = wave & 1;
    int bm, bn;
    lm_block_coords(blockIdx.x, A.nbm, A.nbn, &bm, &bn);
    const int row0 = bm * kLmBM, col0 = bn * kLmBN;
    const int R = A.R, d = A.d, V = A.V;

    // a 128 x 64 bf16 tile is 1024 chunks of 16 bytes: 4 per thread.  The loads
    // are buffer loads over the rows from the tile's first row to the end of the
    // matrix: the hardware range check returns zeros past the end, so partial
    // tiles need no branch in the loop.
    const __amdgpu_buffer_rsrc_t rsA = tile_rsrc(A.h, row0, R, d);
    const __amdgpu_buffer_rsrc_t rsB = tile_rsrc(A.w, col0, V, d);
    auto load_tile = [&](const __amdgpu_buffer_rsrc_t &rs, int k0, uint4 (&buf)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + kLmThreads * i;
            const int r = q >> 3, kc = q & 7;
            buf[i] = __builtin_bit_cast(
                uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, (r * d + k0 + kc * 8) * 2, 0, 0));
        }
    };
    auto store_tile = [&](uint16_t *s, const uint4 (&buf)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int q = tid + kLmThreads * i;
            const int r = q >> 3, kc = q & 7;
            *reinterpret_cast<uint4 *>(s + r * kLmStride + kc * 8) = buf[i];
        }
    };

    floatx4 acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = floatx4{0.0f, 0.0f, 0.0f, 0.0f};

    // three register stages: tile t lives in stage t % 3 from its load until it is
    // stored to LDS, two compute steps later, so each load has two steps to land
    // (stage indices are compile-time constants, so the stages stay in registers)
    const int nk = d / kLmBK;
    uint4 ra[3][4], rb[3][4];
    load_tile(rsA, 0, ra[0]);
    load_tile(rsB, 0, rb[0]);
    if (nk > 1) {
        load_tile(rsA, kLmBK, ra[1]);
        load_tile(rsB, kLmBK, rb[1]);
    }
    if (nk > 2) {
        load_tile(rsA, 2 * kLmBK, ra[2]);
        load_tile(rsB, 2 * kLmBK, rb[2]);
    }
    store_tile(sA[0], ra[0]);
    store_tile(sB[0], rb[0]);
    __syncthreads();

    auto compute = [&](int buf) {
#pragma unroll
        for (int kk = 0; kk < kLmBK; kk += 32) {
            bf16x8 af[4], bfr[4];
            const int ko = kk + (lane >> 4) * 8;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                const int r = wm * 64 + t * 16 + (lane & 15);
                af[t] = *reinterpret_cast<const bf16x8 *>(sA[buf] + r * kLmStride + ko);
                const int c = wn * 64 + t * 16 + (lane & 15);
                bfr[t] = *reinterpret_cast<const bf16x8 *>(sB[buf] + c * kLmStride + ko);
            }
#pragma unroll
            for (int a = 0; a < 4; ++a)
#pragma unroll
                for (int b = 0; b < 4; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[a], bfr[b], acc[a][b], 0,
                                                                       0, 0);
        }
    };
    // step t (stage S = t % 3): compute tile t, store tile t+1 (stage S+1), load
    // tile t+3 into stage S
    auto step = [&](int t, auto stage) {
        constexpr int S = decltype(stage)::value, S1 = (S + 1) % 3;
        compute(t & 1);
        if (t + 1 < nk) {
            store_tile(sA[(t + 1) & 1], ra[S1]);
            store_tile(sB[(t + 1) & 1], rb[S1]);
        }
        if (t + 3 < nk) {
            load_tile(rsA, (t + 3) * kLmBK, ra[S]);
            load_tile(rsB, (t + 3) * kLmBK, rb[S]);
        }
        __syncthreads();
    };
    // the same step where the next tile and the load three ahead both exist:
    // no condition, so the steps of the main loop form one scheduling region
    // apart from their barriers
    auto full_step = [&](int t, auto stage) {
        constexpr int S = decltype(stage)::value, S1 = (S + 1) % 3;
        compute(t & 1);
        store_tile(sA[(t + 1) & 1], ra[S1]);
        store_tile(sB[(t + 1) & 1], rb[S1]);
        load_tile(rsA, (t + 3) * kLmBK, ra[S]);
        load_tile(rsB, (t + 3) * kLmBK, rb[S]);
        __syncthreads();
    };
    int t = 0;
    for (; t + 5 < nk; t += 3) {
        full_step(t, Stage<0>{});
        full_step(t + 1, Stage<1>{});
        full_step(t + 2, Stage<2>{});
    }
    for (; t < nk; t += 3) {
        step(t, Stage<0>{});
        if (t + 1 < nk) step(t + 1, Stage<1>{});
        if (t + 2 < nk) step(t + 2, Stage<2>{});
    }

    // epilogue: lane holds C[4*(lane/16) + i][lane%16] of each 16 x 16 tile
#pragma unroll
    for (int a = 0; a < 4; ++a) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int rloc = wm * 64 + a * 16 + 4 * (lane >> 4) + i;
            const int row = row0 + rloc;
            const bool rok = row < R;
            float v[4];
            float m = -INFINITY;
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const int col = col0 + wn * 64 + b * 16 + (lane & 15);
                const long long at = static_cast<long long>(row) * V + col;
                if (A.bf16_out) {
                    // the statistics describe the logits as stored
                    const uint16_t hb = bf16_rne(acc[a][b][i]);
                    v[b] = col < V ? __uint_as_float(static_cast<uint32_t>(hb) << 16) : -INFINITY;
                    if (rok && col < V) static_cast<uint16_t *>(A.logits)[at] = hb;
                } else {
                    v[b] = col < V ? acc[a][b][i] : -INFINITY;
                    if (rok && col < V) static_cast<float *>(A.logits)[at] = v[b];
                }
                m = fmaxf(m, v[b]);
            }
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) m = fmaxf(m, __shfl_xor(m, o, kWave));
            const Scale sc = temp_scale(rok ? A.temp[row] : 1.0f);
            const float msc = shift_term(m, sc);
            float e = 0.0f;
#pragma unroll
            for (int b = 0; b < 4; ++b) e += fast_exp2(expo(v[b], sc, msc));
            double s = static_cast<double>(e);
#pragma unroll
            for (int o = 1; o < 16; o <<= 1) s += __shfl_xor(s, o, kWave);
            if ((lane & 15) == 0) {
                s_m[wn][rloc] = m;
                s_s[wn][rloc] = s;
            }
        }
    }
    __syncthreads();
    if (tid < kLmBM) {
        const int row = row0 + tid;
        if (row < R) {
            const Scale sc = temp_scale(A.temp[row]);
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
