// sv_device.hpp -- device-side building blocks for the verification kernels
// (gfx950 / CDNA4, wave64).
//
// Rows of logits are consumed in chunks of 8 consecutive elements: one 16-byte
// load for bf16, two for fp32, or 8 bounds-checked scalar loads when the row
// is not 16-byte aligned.  Elements past the end of a row read as -inf, which
// every consumer maps to probability zero.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sv {

constexpr int kChunk = 8;
constexpr int kWave = 64;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// 2^y on the transcendental unit (v_exp_f32).
__device__ __forceinline__ float fast_exp2(float y) { return __builtin_amdgcn_exp2f(y); }

// Base-2 exponents of temperature-scaled logits.  For a row with shift M and
// c = log2(e)/T, every kernel forms the exponent of logit x as
//   y = fmaf(x, c_lo, fmaf(x, c_hi, -K)),   K = shift_term(M) = M c_hi in fp32,
// where c = c_hi + c_lo holds c to ~2^-48 (c_hi rounded down, c_lo > 0, so a
// -inf logit still gives 2^-inf = 0).  Both products are exact inside their
// FMAs, so y is x c - K with two roundings at the scale of y itself.  K is a
// constant of the row (K clamped at -FLT_MAX): whatever its rounding, it
// cancels from every normalised probability, because every reader of a row's
// statistics forms K from the stored shift the same way.  In fp64 the same
// exponent is x (c_hi + c_lo) - K.
struct Scale {
    float hi, lo;
};
__device__ __forceinline__ Scale temp_scale(float T) {
    const double c = 1.4426950408889634 / static_cast<double>(T);
    float hi = static_cast<float>(c);
    if (static_cast<double>(hi) >= c) hi = nextafterf(hi, 0.0f);
    float lo = static_cast<float>(c - static_cast<double>(hi));
    if (!(lo > 0.0f)) {   // c within a rounding of a float: keep the sign of d * lo
        hi = nextafterf(hi, 0.0f);
        lo = static_cast<float>(c - static_cast<double>(hi));
    }
    return Scale{hi, lo};
}
__device__ __forceinline__ double scale64(const Scale &c) {
    return static_cast<double>(c.hi) + static_cast<double>(c.lo);
}
__device__ __forceinline__ float shift_term(float M, const Scale &c) {
    return fmaxf(M * c.hi, -3.402823466e38f);
}
__device__ __forceinline__ float expo(float x, const Scale &c, float K) {
    return fmaf(x, c.lo, fmaf(x, c.hi, -K));
}

// Row readers: load(c, x) fills x[0..7] with elements 8c..8c+7; raw(c) issues
// the same load into a compact register form that unpack() expands later, so
// several chunks can be in flight at 4 VGPRs each (bf16).  raw_once(c) is raw(c)
// as a non-temporal load, for a pass that reads each chunk once and never again
// (the statistics kernel): it streams faster than a cached load, where a pass
// that re-reads rows (the walk's sweeps) loses by it.
typedef unsigned int u32x4_nt __attribute__((ext_vector_type(4)));
typedef float f32x4_nt __attribute__((ext_vector_type(4)));
struct RowBf16Vec {
    using Raw = uint4;
    const uint4 *p;
    __device__ RowBf16Vec(const void *row, int) : p(static_cast<const uint4 *>(row)) {}
    __device__ RowBf16Vec(const uint4 *q) : p(q) {}
    // the same row from chunk n on
    __device__ __forceinline__ RowBf16Vec advanced(int n) const { return RowBf16Vec(p + n); }
    __device__ __forceinline__ Raw raw(int c) const { return p[c]; }
    __device__ __forceinline__ Raw raw_once(int c) const {
        const u32x4_nt v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_nt *>(p) + c);
        return Raw{v.x, v.y, v.z, v.w};
    }
    __device__ __forceinline__ static void unpack(const Raw &w, float x[8]) {
        x[0] = bf16_lo(w.x); x[1] = bf16_hi(w.x);
        x[2] = bf16_lo(w.y); x[3] = bf16_hi(w.y);
        x[4] = bf16_lo(w.z); x[5] = bf16_hi(w.z);
        x[6] = bf16_lo(w.w); x[7] = bf16_hi(w.w);
    }
    __device__ __forceinline__ void load(int c, float x[8]) const { unpack(raw(c), x); }
    __device__ __forceinline__ float at(int v) const {
        const uint16_t *s = reinterpret_cast<const uint16_t *>(p);
        return __uint_as_float(static_cast<uint32_t>(s[v]) << 16);
    }
};

struct RowF32Vec {
    struct Raw { float4 a, b; };
    const float4 *p;
    __device__ RowF32Vec(const void *row, int) : p(static_cast<const float4 *>(row)) {}
    __device__ __forceinline__ RowF32Vec advanced(int n) const { return RowF32Vec(p + 2 * n, 0); }
    __device__ __forceinline__ Raw raw(int c) const { return Raw{p[2 * c], p[2 * c + 1]}; }
    __device__ __forceinline__ Raw raw_once(int c) const {
        const f32x4_nt *q = reinterpret_cast<const f32x4_nt *>(p) + 2 * c;
        const f32x4_nt a = __builtin_nontemporal_load(q), b = __builtin_nontemporal_load(q + 1);
        return Raw{make_float4(a.x, a.y, a.z, a.w), make_float4(b.x, b.y, b.z, b.w)};
    }
    __device__ __forceinline__ static void unpack(const Raw &r, float x[8]) {
        x[0] = r.a.x; x[1] = r.a.y; x[2] = r.a.z; x[3] = r.a.w;
        x[4] = r.b.x; x[5] = r.b.y; x[6] = r.b.z; x[7] = r.b.w;
    }
    __device__ __forceinline__ void load(int c, float x[8]) const { unpack(raw(c), x); }
    __device__ __forceinline__ float at(int v) const {
        return reinterpret_cast<const float *>(p)[v];
    }
};

struct Raw8 {
    float v[8];
};

struct RowBf16Scalar {
    using Raw = Raw8;
    const uint16_t *p;
    int V;
    __device__ RowBf16Scalar(const void *row, int V_) : p(static_cast<const uint16_t *>(row)), V(V_) {}
    __device__ __forceinline__ RowBf16Scalar advanced(int n) const {
        return RowBf16Scalar(p + kChunk * n, V - kChunk * n);
    }
    __device__ __forceinline__ void load(int c, float x[8]) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            int v = 8 * c + e;
            x[e] = v < V ? __uint_as_float(static_cast<uint32_t>(p[v]) << 16) : -INFINITY;
        }
    }
    __device__ __forceinline__ Raw raw(int c) const { Raw r; load(c, r.v); return r; }
    __device__ __forceinline__ Raw raw_once(int c) const { return raw(c); }
    __device__ __forceinline__ static void unpack(const Raw &r, float x[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = r.v[e];
    }
    __device__ __forceinline__ float at(int v) const {
        return __uint_as_float(static_cast<uint32_t>(p[v]) << 16);
    }
};

struct RowF32Scalar {
    using Raw = Raw8;
    const float *p;
    int V;
    __device__ RowF32Scalar(const void *row, int V_) : p(static_cast<const float *>(row)), V(V_) {}
    __device__ __forceinline__ RowF32Scalar advanced(int n) const {
        return RowF32Scalar(p + kChunk * n, V - kChunk * n);
    }
    __device__ __forceinline__ void load(int c, float x[8]) const {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            int v = 8 * c + e;
            x[e] = v < V ? p[v] : -INFINITY;
        }
    }
    __device__ __forceinline__ Raw raw(int c) const { Raw r; load(c, r.v); return r; }
    __device__ __forceinline__ Raw raw_once(int c) const { return raw(c); }
    __device__ __forceinline__ static void unpack(const Raw &r, float x[8]) {
#pragma unroll
        for (int e = 0; e < 8; ++e) x[e] = r.v[e];
    }
    __device__ __forceinline__ float at(int v) const { return p[v]; }
};

template <typename E, bool VEC> struct RowOf;
template <> struct RowOf<uint16_t, true> { using type = RowBf16Vec; };
template <> struct RowOf<uint16_t, false> { using type = RowBf16Scalar; };
template <> struct RowOf<float, true> { using type = RowF32Vec; };
template <> struct RowOf<float, false> { using type = RowF32Scalar; };

// Chunks of a row kept in flight per lane for a given number of bytes: two
// 16-byte bf16 chunks or one 32-byte fp32 chunk in 32 bytes.
template <typename RD, int BYTES>
constexpr int depth_for() {
    return BYTES / static_cast<int>(sizeof(typename RD::Raw)) > 0
               ? BYTES / static_cast<int>(sizeof(typename RD::Raw))
               : 1;
}

// Stream the chunks c0, c0 + NT, ... (c0 = this thread's index, all < nch) of
// one row, or of a row pair when HAS_Q, through f(xp, xq, c).  D chunks per row
// stay in flight per lane: once a chunk is unpacked its register slot is
// refilled with the chunk D NT further on, so loads overlap the arithmetic of
// the chunks before them instead of being issued and drained group by group.
// Refill addresses are clamped into the row (nch >= 1); the refills issued in
// the last full group are discarded and the remainder is read one chunk at a
// time.  Without HAS_Q, xq is left unset and Q is not read.  ONCE: the pass
// reads these rows once (non-temporal loads).
template <int NT, int D, bool HAS_Q, bool ONCE = false, typename RD, typename F>
__device__ __forceinline__ void stream_rows(const RD &P, const RD &Q, int nch, F &&f) {
    auto rd = [](const RD &R, int c) { return ONCE ? R.raw_once(c) : R.raw(c); };
    int c = threadIdx.x;
    if (c + (D - 1) * NT < nch) {
        typename RD::Raw rp[D], rq[D];
        // issued in the order they are consumed (the scheduler would otherwise
        // be free to permute them, and the static waits in the loop then cover
        // the worst order)
#pragma unroll
        for (int i = 0; i < D; ++i) {
            rp[i] = rd(P, c + i * NT);
            if (HAS_Q) rq[i] = rd(Q, c + i * NT);
            __builtin_amdgcn_sched_barrier(0);
        }
        for (;;) {
            const int cn = c + D * NT;
#pragma unroll
            for (int i = 0; i < D; ++i) {
                float xp[8], xq[8];
                RD::unpack(rp[i], xp);
                if (HAS_Q) RD::unpack(rq[i], xq);
                const int cl = min(cn + i * NT, nch - 1);
                rp[i] = rd(P, cl);
                if (HAS_Q) rq[i] = rd(Q, cl);
                f(xp, xq, c + i * NT);
            }
            c = cn;
            if (c + (D - 1) * NT >= nch) break;
        }
    }
    for (; c < nch; c += NT) {
        float xp[8], xq[8];
        RD::unpack(rd(P, c), xp);
        if (HAS_Q) RD::unpack(rd(Q, c), xq);
        f(xp, xq, c);
    }
}

__device__ __forceinline__ float max8(const float x[8]) {
    return fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                 fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
}

__device__ __forceinline__ float sum8(const float e[8]) {
    return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
}

// ---------------------------------------------------------------- reductions
// Butterfly reductions give every lane the same bits (IEEE + is commutative),
// so every thread of a block leaves a block reduction with identical values.

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v += __shfl_xor(v, o, kWave);
    return v;
}

__device__ __forceinline__ int wave_max_int(int v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = max(v, __shfl_xor(v, o, kWave));
    return v;
}

__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
    for (int o = kWave / 2; o > 0; o >>= 1) v = min(v, __shfl_xor(v, o, kWave));
    return v;
}

// red[] must hold NT/64 entries; the leading barrier protects its previous use.
template <int NT>
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    float t = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) t = fmaxf(t, red[i]);
    return t;
}

template <int NT>
__device__ __forceinline__ double block_sum(double v, double *red) {
    v = wave_sum(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    double t = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) t += red[i];
    return t;
}

// N independent block sums at once; red[] must hold N * NT/64 entries.
template <int NT, int N>
__device__ __forceinline__ void block_sum_n(double (&v)[N], double *red) {
    constexpr int NW = NT / kWave;
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) red[i * NW + threadIdx.x / kWave] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        double t = red[i * NW];
#pragma unroll
        for (int w = 1; w < NW; ++w) t += red[i * NW + w];
        v[i] = t;
    }
}

// Four independent block sums at once; red[] must hold 4 * NT/64 entries.
template <int NT>
__device__ __forceinline__ void block_sum4(double v[4], double *red) {
    constexpr int NW = NT / kWave;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = wave_sum(v[i]);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) {
#pragma unroll
        for (int i = 0; i < 4; ++i) red[i * NW + threadIdx.x / kWave] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        double t = red[i * NW];
#pragma unroll
        for (int w = 1; w < NW; ++w) t += red[i * NW + w];
        v[i] = t;
    }
}

template <int NT>
__device__ __forceinline__ int block_max_int(int v, int *red) {
    v = wave_max_int(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    int t = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) t = max(t, red[i]);
    return t;
}

template <int NT>
__device__ __forceinline__ int block_min_int(int v, int *red) {
    v = wave_min_int(v);
    __syncthreads();
    if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = v;
    __syncthreads();
    int t = red[0];
#pragma unroll
    for (int i = 1; i < NT / kWave; ++i) t = min(t, red[i]);
    return t;
}

// Exclusive prefix sum over the 64 lanes of a wave, in lane order.
__device__ __forceinline__ double wave_exclusive_scan(double v) {
    const int lane = threadIdx.x & (kWave - 1);
    double s = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double n = __shfl_up(s, o, kWave);
        if (lane >= o) s += n;
    }
    const double excl = __shfl_up(s, 1, kWave);
    return lane == 0 ? 0.0 : excl;
}

// Exclusive prefix sum over the block in thread order.
template <int NT>
__device__ __forceinline__ double block_exclusive_scan(double v, double *red) {
    const int lane = threadIdx.x & (kWave - 1), w = threadIdx.x / kWave;
    double s = v;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        double n = __shfl_up(s, o, kWave);
        if (lane >= o) s += n;
    }
    double excl = __shfl_up(s, 1, kWave);
    if (lane == 0) excl = 0.0;
    __syncthreads();
    if (lane == kWave - 1) red[w] = s;
    __syncthreads();
    double base = 0.0;
    for (int i = 0; i < w; ++i) base += red[i];
    return base + excl;
}

}  // namespace sv
