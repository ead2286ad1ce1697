// Row kernels for gfx950 (CDNA4, wave64): fixed-width LayerNorm, residual add +
// LayerNorm, shifted-window index tables, window gather, fused norm-gather, and
// the steps around them (window reverse fused with add + LayerNorm, add +
// LayerNorm + gather, affine LayerNorm, float32 bias + tanh-GELU).
//
// What is computed follows the page "Pangu-Weather inference optimisation on
// Hygon BW1000 (gfx936)" (l189.com/news/2144533):
//   section 3 -- LayerNorm over rows of width 192 or 384 (and the model's
//                patch-merge width 768), FP16 in and out, no affine;
//   section 4 -- residual add whose FP16 rounding is kept, then LayerNorm of it;
//   section 5 -- INT32 window index tables (-1 = padding row = zeros), a gather
//                driven by them, and the norm-gather fusion;
// and the bias + GELU of the page "PyTorch + HIP custom fused operator".
// How it is computed is designed for CDNA4 rather than taken from that page
// (which used one wave per row and __half2 moves on gfx936):
//   * Every access is a 16-byte (8 x binary16) vector load or store. A row of C
//     values is split over LPR = C/(8K) consecutive lanes holding K chunks each;
//     chunk k of a lane sits at column chunk (lane % LPR) + k*LPR, so one wave
//     instruction reads 64/LPR rows x LPR*16 contiguous bytes (whole 128-byte
//     lines), and the K instructions of a wave cover 64/LPR full rows.
//   * Row statistics are reduced across the LPR lanes of a row with DPP
//     (quad_perm / row_half_mirror / row_mirror), no LDS and no barriers.
//   * Statistics and the normalisation run in binary64: CDNA4 issues FP64 vector
//     adds and FMAs at the same per-lane rate as plain FP32, and binary64 makes
//     each output the correctly rounded binary16 of the exact LayerNorm in
//     practice, where FP32 arithmetic flips about 1e-4 of outputs by one ulp.
//     The final binary64 -> binary16 rounding goes through a round-to-odd
//     binary32 intermediate, which makes the two-step conversion exact-once.
//   * All kernels are stateless and row-local: no atomics, no scratch memory.
//     Only the affine kernels use LDS, to hold gamma and beta for a workgroup;
//     the plain gathers reserve some, unread, to limit how many of their
//     workgroups share a compute unit.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <type_traits>

#include "lwg_launch.h"

namespace lwg {
namespace {

typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef uint32_t chunk_t __attribute__((ext_vector_type(4)));  // 16 bytes = 8 x binary16

constexpr int kBlock = 256;  // 4 waves per workgroup

// Memory hints of a kernel instance: non-temporal loads / stores (the `nt` bit
// on global_load/global_store: stream through the caches without keeping lines).
template <bool NTL, bool NTS>
struct Hints {
    static constexpr bool kNtLoad = NTL;
    static constexpr bool kNtStore = NTS;
};

template <class H>
__device__ __forceinline__ chunk_t load16(const chunk_t* p) {
    if constexpr (H::kNtLoad) return __builtin_nontemporal_load(p);
    else return *p;
}

template <class H>
__device__ __forceinline__ void store16(chunk_t* p, chunk_t v) {
    if constexpr (H::kNtStore) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// ---------------------------------------------------------------------------
// Lane geometry of a row tile

template <int C, int K>
struct Tile {
    static_assert(C % (8 * K) == 0, "a lane holds K whole 16-byte chunks");
    static constexpr int kChunks = C / 8;              // 16-byte chunks per row
    static constexpr int kLanes = kChunks / K;          // lanes sharing one row
    static constexpr int kRowsPerWave = 64 / kLanes;    // rows per wave instruction
    static constexpr int kValues = 8 * K;               // binary16 values per lane
    static_assert(kLanes == 2 || kLanes == 4 || kLanes == 8 || kLanes == 16,
                  "row groups must sit inside one 16-lane DPP row");
};


// ---------------------------------------------------------------------------
// Cross-lane sums inside a row group, with DPP

template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, false));
}

template <int CTRL>
__device__ __forceinline__ double dpp_f64(double v) {
    const uint64_t b = __builtin_bit_cast(uint64_t, v);
    const uint64_t lo = dpp_u32<CTRL>(static_cast<uint32_t>(b));
    const uint64_t hi = dpp_u32<CTRL>(static_cast<uint32_t>(b >> 32));
    return __builtin_bit_cast(double, (hi << 32) | lo);
}

// Sum over the LPR consecutive lanes of a row group; every lane of the group
// receives the same bits (each step adds a lane's value to its partner's, and
// IEEE addition commutes).
template <int LPR>
__device__ __forceinline__ double group_sum(double v) {
    v += dpp_f64<0xB1>(v);                          // quad_perm [1,0,3,2]: lane ^ 1
    if constexpr (LPR >= 4) v += dpp_f64<0x4E>(v);  // quad_perm [2,3,0,1]: lane ^ 2
    if constexpr (LPR >= 8) v += dpp_f64<0x141>(v); // row_half_mirror: quad <-> quad
    if constexpr (LPR >= 16) v += dpp_f64<0x140>(v);// row_mirror: 8 lanes <-> 8 lanes
    return v;
}

// ---------------------------------------------------------------------------
// Conversions

__device__ __forceinline__ void unpack8(const chunk_t& c, double* out) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2_t h = __builtin_bit_cast(half2_t, w[i]);
        out[2 * i] = static_cast<double>(static_cast<float>(h.x));
        out[2 * i + 1] = static_cast<double>(static_cast<float>(h.y));
    }
}

// binary64 -> binary16, rounded once to nearest-even. The binary64 value is
// first cut to binary32 with round-to-odd (truncate the 29 extra significand
// bits, set the binary32 last bit if any of them was set); binary32 keeps 13
// bits beyond binary16, so the following nearest-even conversion sees the same
// rounding decision as a direct one. NaN stays NaN, +-Inf and +-0 are kept.
// Magnitudes below the binary32 normal range are far below half the smallest
// binary16 subnormal and go to +-0 either way.
__device__ __forceinline__ _Float16 to_half_rn(double y) {
    const uint64_t b = __builtin_bit_cast(uint64_t, y);
    const uint32_t lo = static_cast<uint32_t>(b);
    const uint32_t sticky = ((lo & 0x1FFFFFFFu) + 0x1FFFFFFFu) & 0x20000000u;
    const uint64_t t = (b & 0xFFFFFFFFE0000000ull) | sticky;
    const float f = static_cast<float>(__builtin_bit_cast(double, t));  // exact
    return static_cast<_Float16>(f);
}

__device__ __forceinline__ uint32_t pack2(double a, double b) {
    half2_t h;
    h.x = to_half_rn(a);
    h.y = to_half_rn(b);
    return __builtin_bit_cast(uint32_t, h);
}

// ---------------------------------------------------------------------------
// Row math

// FP16 residual of section 4: residual + branch rounded once to binary16. The
// packed binary16 add computes the exact sum rounded to nearest-even.
template <int K>
__device__ __forceinline__ void residual_add(const chunk_t (&branch)[K], chunk_t (&res)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) {
        uint32_t r[4] = {res[k].x, res[k].y, res[k].z, res[k].w};
        const uint32_t b[4] = {branch[k].x, branch[k].y, branch[k].z, branch[k].w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const half2_t s = __builtin_bit_cast(half2_t, r[i]) + __builtin_bit_cast(half2_t, b[i]);
            r[i] = __builtin_bit_cast(uint32_t, s);
        }
        res[k] = chunk_t{r[0], r[1], r[2], r[3]};
    }
}

// 1/sqrt(a) for a > 0: the hardware reciprocal-square-root estimate refined by
// one Newton step, r' = r (3/2 - a r^2 / 2), which takes a relative error e to
// about 1.5 e^2: from the estimate's ~2^-24 to ~2^-47, far below the 2^-11 of a
// binary16 result. Inf and NaN give NaN.
__device__ __forceinline__ double rsqrt_refined(double a) {
    const double r = __builtin_amdgcn_rsq(a);
    const double h = 0.5 * a * r;
    return __builtin_fma(r, __builtin_fma(-h, r, 0.5), r);
}

// Row statistics of LayerNorm (section 3) for the row whose 1/LPR share this
// lane holds in v: the mean and the biased variance of the deviations, in two
// passes over registers. On return x holds this lane's deviations from the mean
// and the result is 1/sqrt(var + eps).
template <int C, int K>
__device__ __forceinline__ double row_stats(const chunk_t (&v)[K], double (&x)[8 * K], double eps) {
    using T = Tile<C, K>;
    constexpr double kInvC = 1.0 / C;
#pragma unroll
    for (int k = 0; k < K; ++k) unpack8(v[k], x + 8 * k);

    double s0 = 0.0, s1 = 0.0;
#pragma unroll
    for (int i = 0; i < T::kValues; i += 2) {
        s0 += x[i];
        s1 += x[i + 1];
    }
    const double mean = group_sum<T::kLanes>(s0 + s1) * kInvC;

    double q0 = 0.0, q1 = 0.0;
#pragma unroll
    for (int i = 0; i < T::kValues; i += 2) {
        x[i] -= mean;
        x[i + 1] -= mean;
        q0 = __builtin_fma(x[i], x[i], q0);
        q1 = __builtin_fma(x[i + 1], x[i + 1], q1);
    }
    return rsqrt_refined(group_sum<T::kLanes>(q0 + q1) * kInvC + eps);
}

// LayerNorm of the row whose 1/LPR share this lane holds in v: (x - mean) /
// sqrt(var + eps) rounded to binary16, written back into v. Every kernel that
// normalises a row calls this same function with the same (C, K), so their
// outputs agree bit for bit.
template <int C, int K>
__device__ __forceinline__ void layer_norm_lane(chunk_t (&v)[K], double eps) {
    double x[8 * K];
    const double rstd = row_stats<C, K>(v, x, eps);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        const double* xk = x + 8 * k;
        v[k] = chunk_t{pack2(xk[0] * rstd, xk[1] * rstd), pack2(xk[2] * rstd, xk[3] * rstd),
                       pack2(xk[4] * rstd, xk[5] * rstd), pack2(xk[6] * rstd, xk[7] * rstd)};
    }
}

// The 8 values of parameter chunk i, from LDS staged either as the binary16
// chunks themselves or already widened to binary64 (8 doubles per chunk).
__device__ __forceinline__ void param_chunk(const chunk_t* p, int i, double (&out)[8]) { unpack8(p[i], out); }
__device__ __forceinline__ void param_chunk(const double* p, int i, double (&out)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = p[8 * i + e];
}

// Affine LayerNorm: ((x - mean) / sqrt(var + eps)) * gamma + beta in binary64,
// rounded once to binary16. gamma and beta are binary16 [C], held in LDS by the
// affine kernels (as chunks, or widened: P); this lane reads its columns chunk
// by chunk as it writes them, so only one chunk of them is live next to the
// row's deviations.
template <int C, int K, class P>
__device__ __forceinline__ void layer_norm_affine_lane(chunk_t (&v)[K], const P* gamma,
                                                       const P* beta, int sub, double eps) {
    using T = Tile<C, K>;
    double x[8 * K];
    const double rstd = row_stats<C, K>(v, x, eps);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        double gk[8], bk[8];
        param_chunk(gamma, sub + k * T::kLanes, gk);
        param_chunk(beta, sub + k * T::kLanes, bk);
        const double* xk = x + 8 * k;
        v[k] = chunk_t{pack2(__builtin_fma(xk[0] * rstd, gk[0], bk[0]), __builtin_fma(xk[1] * rstd, gk[1], bk[1])),
                       pack2(__builtin_fma(xk[2] * rstd, gk[2], bk[2]), __builtin_fma(xk[3] * rstd, gk[3], bk[3])),
                       pack2(__builtin_fma(xk[4] * rstd, gk[4], bk[4]), __builtin_fma(xk[5] * rstd, gk[5], bk[5])),
                       pack2(__builtin_fma(xk[6] * rstd, gk[6], bk[6]), __builtin_fma(xk[7] * rstd, gk[7], bk[7]))};
    }
}

template <int K>
__device__ __forceinline__ void zero(chunk_t (&v)[K]) {
#pragma unroll
    for (int k = 0; k < K; ++k) v[k] = chunk_t{0u, 0u, 0u, 0u};
}

// ---------------------------------------------------------------------------
// Kernels
//
// Wave w of the grid handles row tiles w, w + (waves in the grid), ...; a tile
// is the kRowsPerWave rows one wave covers. The loop bound is the same for every
// lane of a wave, so the DPP reductions always run with the whole wave active.
// The launcher sizes the grid either to one tile per wave or to a fixed number
// of resident workgroups.

template <int kWaves>
__device__ __forceinline__ int64_t first_wave_in() {
    return static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
}

template <int kWaves>
__device__ __forceinline__ int64_t wave_stride_in() {
    return static_cast<int64_t>(gridDim.x) * kWaves;
}

// For kernels launched with kBlock threads per workgroup (all but the gathers,
// whose workgroup size is a launch-table choice).
__device__ __forceinline__ int64_t first_wave() { return first_wave_in<kBlock / 64>(); }
__device__ __forceinline__ int64_t wave_stride() { return wave_stride_in<kBlock / 64>(); }

// The K chunks this lane holds of row tile w (zeros past the last row). With
// kPrio > 0 the wave issues the loads at that scheduling priority (s_setprio)
// and drops back to 0 after them, so that a wave with loads to issue goes ahead
// of waves busy with row arithmetic on the same SIMD.
template <int C, int K, class H, int kPrio = 0>
__device__ __forceinline__ void load_tile(const chunk_t* x, int64_t w, int64_t rows, int lane,
                                          chunk_t (&v)[K]) {
    using T = Tile<C, K>;
    const int64_t row = w * T::kRowsPerWave + lane / T::kLanes;
    zero(v);
    if constexpr (kPrio > 0) __builtin_amdgcn_s_setprio(kPrio);
    if (row < rows) {
        const int64_t base = row * T::kChunks + lane % T::kLanes;
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = load16<H>(x + base + k * T::kLanes);
    }
    if constexpr (kPrio > 0) __builtin_amdgcn_s_setprio(0);
}

template <int C, int K, class H>
__device__ __forceinline__ void store_tile(chunk_t* y, int64_t w, int64_t rows, int lane,
                                           const chunk_t (&v)[K]) {
    using T = Tile<C, K>;
    const int64_t row = w * T::kRowsPerWave + lane / T::kLanes;
    if (row < rows) {
        const int64_t base = row * T::kChunks + lane % T::kLanes;
#pragma unroll
        for (int k = 0; k < K; ++k) store16<H>(y + base + k * T::kLanes, v[k]);
    }
}

// y may alias x: a lane reads all of its chunks before the row statistics
// exist, and writes only the chunks it read. With kPrefetch a wave issues the
// loads of its next tile before it normalises the current one, so on a grid
// smaller than the tile count the arithmetic of one tile overlaps the memory
// traffic of the next. (In place, the next tile's rows are other rows, read
// before this tile's stores: still no overlap between a lane's reads and
// another lane's writes.)
template <int C, int K, class H, bool kPrefetch>
__global__ __launch_bounds__(kBlock) void ln_fixed_kernel(const chunk_t* x, chunk_t* y,
                                                          int64_t rows, double eps) {
    using T = Tile<C, K>;
    const int lane = threadIdx.x & 63;
    if constexpr (kPrefetch) {
        const int64_t stride = wave_stride();
        int64_t w = first_wave();
        chunk_t v[K];
        load_tile<C, K, H>(x, w, rows, lane, v);
        for (; w * T::kRowsPerWave < rows; w += stride) {
            chunk_t next[K];
            load_tile<C, K, H>(x, w + stride, rows, lane, next);
            layer_norm_lane<C, K>(v, eps);
            store_tile<C, K, H>(y, w, rows, lane, v);
#pragma unroll
            for (int k = 0; k < K; ++k) v[k] = next[k];
        }
    } else {
        const int sub = lane % T::kLanes;
        for (int64_t w = first_wave(); w * T::kRowsPerWave < rows; w += wave_stride()) {
            const int64_t row = w * T::kRowsPerWave + lane / T::kLanes;
            const bool live = row < rows;
            const int64_t base = row * T::kChunks + sub;
            chunk_t v[K];
            zero(v);
            if (live) {
#pragma unroll
                for (int k = 0; k < K; ++k) v[k] = load16<H>(x + base + k * T::kLanes);
            }
            layer_norm_lane<C, K>(v, eps);
            if (live) {
#pragma unroll
                for (int k = 0; k < K; ++k) store16<H>(y + base + k * T::kLanes, v[k]);
            }
        }
    }
}

// residual_out and y may alias the inputs: each lane reads its chunks of a row
// before it writes any, and the prefetched tile is a different set of rows.
template <int C, int K, class H, bool kPrefetch, int kPrio>
__global__ __launch_bounds__(kBlock) void add_ln_kernel(const chunk_t* branch, const chunk_t* residual,
                                                        chunk_t* residual_out, chunk_t* y,
                                                        int64_t rows, double eps) {
    using T = Tile<C, K>;
    const int lane = threadIdx.x & 63;
    const int64_t stride = wave_stride();
    int64_t w = first_wave();
    chunk_t b[K], r[K];
    load_tile<C, K, H, kPrio>(branch, w, rows, lane, b);
    load_tile<C, K, H, kPrio>(residual, w, rows, lane, r);
    for (; w * T::kRowsPerWave < rows; w += stride) {
        chunk_t nb[K], nr[K];
        if constexpr (kPrefetch) {
            load_tile<C, K, H, kPrio>(branch, w + stride, rows, lane, nb);
            load_tile<C, K, H, kPrio>(residual, w + stride, rows, lane, nr);
        }
        residual_add<K>(b, r);
        store_tile<C, K, H>(residual_out, w, rows, lane, r);
        layer_norm_lane<C, K>(r, eps);
        store_tile<C, K, H>(y, w, rows, lane, r);
        if constexpr (kPrefetch) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                b[k] = nb[k];
                r[k] = nr[k];
            }
        } else {
            load_tile<C, K, H, kPrio>(branch, w + stride, rows, lane, b);
            load_tile<C, K, H, kPrio>(residual, w + stride, rows, lane, r);
        }
    }
}

// Affine LayerNorm and residual add + affine LayerNorm. gamma and beta are
// binary16 [C]; each workgroup copies them once into LDS and every lane reads
// its columns from there chunk by chunk, so the parameters neither occupy the
// vector-memory path nor sit widened in registers. kWide selects the LDS form:
// the binary16 chunks (2*C*2 bytes; each use converts 16 values to binary64),
// or values widened to binary64 as they are staged (2*C*8 bytes, at most
// 12 KB; each use is a plain LDS read). y may alias x, and residual_out / y may
// alias the inputs as in the plain kernels.
template <int C, bool kWide>
struct AffineStage {
    using P = std::conditional_t<kWide, double, chunk_t>;
    static constexpr int kHalf = kWide ? C : C / 8;     // entries of gamma (and of beta)
};

template <int C>
__device__ __forceinline__ void stage_params(chunk_t* params, const chunk_t* gamma, const chunk_t* beta) {
    constexpr int kChunks = C / 8;
    for (int i = threadIdx.x; i < 2 * kChunks; i += kBlock)
        params[i] = i < kChunks ? gamma[i] : beta[i - kChunks];
    __syncthreads();
}

template <int C>
__device__ __forceinline__ void stage_params(double* params, const chunk_t* gamma, const chunk_t* beta) {
    constexpr int kChunks = C / 8;
    for (int i = threadIdx.x; i < 2 * kChunks; i += kBlock) {
        double v[8];
        unpack8(i < kChunks ? gamma[i] : beta[i - kChunks], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) params[8 * i + e] = v[e];
    }
    __syncthreads();
}

template <int C, int K, class H, int kPrio, bool kWide>
__global__ __launch_bounds__(kBlock) void ln_affine_kernel(const chunk_t* x, const chunk_t* gamma,
                                                           const chunk_t* beta, chunk_t* y,
                                                           int64_t rows, double eps) {
    using T = Tile<C, K>;
    using S = AffineStage<C, kWide>;
    __shared__ typename S::P params[2 * S::kHalf];
    stage_params<C>(params, gamma, beta);
    const typename S::P* gamma_s = params;
    const typename S::P* beta_s = params + S::kHalf;
    const int lane = threadIdx.x & 63;
    const int sub = lane % T::kLanes;
    const int64_t stride = wave_stride();
    int64_t w = first_wave();
    chunk_t v[K];
    load_tile<C, K, H, kPrio>(x, w, rows, lane, v);
    for (; w * T::kRowsPerWave < rows; w += stride) {
        // re-read gamma/beta from LDS per row tile instead of letting the
        // compiler hoist 2*K widened chunks out of the loop into registers
        asm volatile("" ::: "memory");
        layer_norm_affine_lane<C, K>(v, gamma_s, beta_s, sub, eps);
        store_tile<C, K, H>(y, w, rows, lane, v);
        load_tile<C, K, H, kPrio>(x, w + stride, rows, lane, v);
    }
}

template <int C, int K, class H, bool kPrefetch, int kPrio, bool kWide>
__global__ __launch_bounds__(kBlock) void add_ln_affine_kernel(const chunk_t* branch, const chunk_t* residual,
                                                                 const chunk_t* gamma, const chunk_t* beta,
                                                                 chunk_t* residual_out, chunk_t* y,
                                                                 int64_t rows, double eps) {
    using T = Tile<C, K>;
    using S = AffineStage<C, kWide>;
    __shared__ typename S::P params[2 * S::kHalf];
    stage_params<C>(params, gamma, beta);
    const typename S::P* gamma_s = params;
    const typename S::P* beta_s = params + S::kHalf;
    const int lane = threadIdx.x & 63;
    const int sub = lane % T::kLanes;
    const int64_t stride = wave_stride();
    int64_t w = first_wave();
    chunk_t b[K], r[K];
    load_tile<C, K, H, kPrio>(branch, w, rows, lane, b);
    load_tile<C, K, H, kPrio>(residual, w, rows, lane, r);
    for (; w * T::kRowsPerWave < rows; w += stride) {
        chunk_t nb[K], nr[K];
        if constexpr (kPrefetch) {
            load_tile<C, K, H, kPrio>(branch, w + stride, rows, lane, nb);
            load_tile<C, K, H, kPrio>(residual, w + stride, rows, lane, nr);
        }
        asm volatile("" ::: "memory");  // as in ln_affine_kernel: no hoisting of gamma/beta
        residual_add<K>(b, r);
        store_tile<C, K, H>(residual_out, w, rows, lane, r);
        layer_norm_affine_lane<C, K>(r, gamma_s, beta_s, sub, eps);
        store_tile<C, K, H>(y, w, rows, lane, r);
        if constexpr (kPrefetch) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                b[k] = nb[k];
                r[k] = nr[k];
            }
        } else {
            load_tile<C, K, H, kPrio>(branch, w + stride, rows, lane, b);
            load_tile<C, K, H, kPrio>(residual, w + stride, rows, lane, r);
        }
    }
}

// Output-major gather: lane group j reads table[j] and, for a valid entry,
// the whole source row; padding and out-of-range entries read nothing and
// store +0.0 (LayerNorm of a zero row is exactly +0.0 as well).
// With kPrio > 0 the table read and the row loads are issued at that wave
// priority, as in load_tile.
template <int C, int K, class H, int kPrio = 0>
__device__ __forceinline__ void load_gathered(const chunk_t* x, int64_t n_src, const int32_t* table,
                                              int64_t n_out, int64_t w, int lane, chunk_t (&v)[K]) {
    using T = Tile<C, K>;
    if constexpr (kPrio > 0) __builtin_amdgcn_s_setprio(kPrio);
    const int64_t j = w * T::kRowsPerWave + lane / T::kLanes;
    const int32_t t = j < n_out ? table[j] : -1;
    zero(v);
    if (t >= 0 && static_cast<int64_t>(t) < n_src) {
        const int64_t src = static_cast<int64_t>(t) * T::kChunks + lane % T::kLanes;
#pragma unroll
        for (int k = 0; k < K; ++k) v[k] = load16<H>(x + src + k * T::kLanes);
    }
    if constexpr (kPrio > 0) __builtin_amdgcn_s_setprio(0);
}

template <int C, int K, bool kNorm, class H, bool kPrefetch, int kWaves, int kPrio>
__global__ __launch_bounds__(64 * kWaves) void gather_kernel(const chunk_t* __restrict__ x, int64_t n_src,
                                                             const int32_t* __restrict__ table,
                                                             int64_t n_out, chunk_t* __restrict__ out,
                                                             double eps) {
    using T = Tile<C, K>;
    const int lane = threadIdx.x & 63;
    if constexpr (kPrefetch) {
        const int64_t stride = wave_stride_in<kWaves>();
        int64_t w = first_wave_in<kWaves>();
        chunk_t v[K];
        load_gathered<C, K, H, kPrio>(x, n_src, table, n_out, w, lane, v);
        for (; w * T::kRowsPerWave < n_out; w += stride) {
            chunk_t next[K];
            load_gathered<C, K, H, kPrio>(x, n_src, table, n_out, w + stride, lane, next);
            if constexpr (kNorm) layer_norm_lane<C, K>(v, eps);
            store_tile<C, K, H>(out, w, n_out, lane, v);
#pragma unroll
            for (int k = 0; k < K; ++k) v[k] = next[k];
        }
    } else {
        const int sub = lane % T::kLanes;
        for (int64_t w = first_wave_in<kWaves>(); w * T::kRowsPerWave < n_out; w += wave_stride_in<kWaves>()) {
            const int64_t j = w * T::kRowsPerWave + lane / T::kLanes;
            const bool live = j < n_out;
            if constexpr (kPrio > 0) __builtin_amdgcn_s_setprio(kPrio);
            const int32_t t = live ? table[j] : -1;
            const bool valid = t >= 0 && static_cast<int64_t>(t) < n_src;
            const int64_t src = static_cast<int64_t>(t) * T::kChunks + sub;
            chunk_t v[K];
            zero(v);
            if (valid) {
#pragma unroll
                for (int k = 0; k < K; ++k) v[k] = load16<H>(x + src + k * T::kLanes);
            }
            if constexpr (kPrio > 0) __builtin_amdgcn_s_setprio(0);
            if constexpr (kNorm) layer_norm_lane<C, K>(v, eps);
            if (live) {
                const int64_t dst = j * T::kChunks + sub;
#pragma unroll
                for (int k = 0; k < K; ++k) store16<H>(out + dst + k * T::kLanes, v[k]);
            }
        }
    }
}

// Window reverse fused with the residual add + LayerNorm: token row i takes
// its branch from window row idx[i] (the inverse table), adds the residual,
// writes the rounded sum, and normalises it. An index outside [0, n_win) gives
// a zero branch. residual_out and y may alias residual (row i is read and
// written by the same lanes; a prefetched tile holds other rows); neither may
// overlap win, whose rows a prefetch may read after another row was written.
template <int C, int K, class H, bool kPrefetch, int kPrio>
__global__ __launch_bounds__(kBlock) void reverse_add_ln_kernel(
    const chunk_t* __restrict__ win, int64_t n_win, const int32_t* __restrict__ idx,
    const chunk_t* residual, chunk_t* residual_out, chunk_t* y, int64_t rows, double eps) {
    using T = Tile<C, K>;
    const int lane = threadIdx.x & 63;
    const int64_t stride = wave_stride();
    int64_t w = first_wave();
    chunk_t b[K], r[K];
    load_gathered<C, K, H>(win, n_win, idx, rows, w, lane, b);
    load_tile<C, K, H, kPrio>(residual, w, rows, lane, r);
    for (; w * T::kRowsPerWave < rows; w += stride) {
        chunk_t nb[K], nr[K];
        if constexpr (kPrefetch) {
            load_gathered<C, K, H>(win, n_win, idx, rows, w + stride, lane, nb);
            load_tile<C, K, H, kPrio>(residual, w + stride, rows, lane, nr);
        }
        residual_add<K>(b, r);
        store_tile<C, K, H>(residual_out, w, rows, lane, r);
        layer_norm_lane<C, K>(r, eps);
        store_tile<C, K, H>(y, w, rows, lane, r);
        if constexpr (kPrefetch) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                b[k] = nb[k];
                r[k] = nr[k];
            }
        } else {
            load_gathered<C, K, H>(win, n_win, idx, rows, w + stride, lane, b);
            load_tile<C, K, H, kPrio>(residual, w + stride, rows, lane, r);
        }
    }
}

// Branch and residual chunks of the source row of gathered row j (zeros and -1
// for padding or an out-of-range entry); returns the source row or -1.
template <int C, int K, class H>
__device__ __forceinline__ int32_t load_pair(const chunk_t* branch, const chunk_t* residual, int64_t n_src,
                                             const int32_t* table, int64_t n_out, int64_t w, int lane,
                                             chunk_t (&b)[K], chunk_t (&r)[K]) {
    using T = Tile<C, K>;
    const int64_t j = w * T::kRowsPerWave + lane / T::kLanes;
    int32_t t = j < n_out ? table[j] : -1;
    if (!(t >= 0 && static_cast<int64_t>(t) < n_src)) t = -1;
    zero(b);
    zero(r);
    if (t >= 0) {
        const int64_t src = static_cast<int64_t>(t) * T::kChunks + lane % T::kLanes;
#pragma unroll
        for (int k = 0; k < K; ++k) {
            b[k] = load16<H>(branch + src + k * T::kLanes);
            r[k] = load16<H>(residual + src + k * T::kLanes);
        }
    }
    return t;
}

// Residual add + LayerNorm + window gather, output-major: gathered row j reads
// token t = table[j] from branch and residual, writes the rounded sum to
// residual_out[t] and its LayerNorm to out[j]; padding rows store +0.0 and
// touch no token. With a table whose valid entries are distinct (as built by
// window_index_kernel) every token row is read and written by exactly one lane
// group, and a prefetched tile reads other tokens than the one being written,
// so residual_out may alias residual or branch.
template <int C, int K, class H, bool kPrefetch>
__global__ __launch_bounds__(kBlock) void add_norm_gather_kernel(
    const chunk_t* branch, const chunk_t* residual, chunk_t* residual_out, int64_t n_src,
    const int32_t* __restrict__ table, int64_t n_out, chunk_t* __restrict__ out, double eps) {
    using T = Tile<C, K>;
    const int lane = threadIdx.x & 63;
    const int sub = lane % T::kLanes;
    const int64_t stride = wave_stride();
    int64_t w = first_wave();
    chunk_t b[K], r[K];
    int32_t t = load_pair<C, K, H>(branch, residual, n_src, table, n_out, w, lane, b, r);
    for (; w * T::kRowsPerWave < n_out; w += stride) {
        chunk_t nb[K], nr[K];
        int32_t nt = -1;
        if constexpr (kPrefetch)
            nt = load_pair<C, K, H>(branch, residual, n_src, table, n_out, w + stride, lane, nb, nr);
        residual_add<K>(b, r);
        if (t >= 0) {
            const int64_t src = static_cast<int64_t>(t) * T::kChunks + sub;
#pragma unroll
            for (int k = 0; k < K; ++k) store16<H>(residual_out + src + k * T::kLanes, r[k]);
        }
        layer_norm_lane<C, K>(r, eps);
        store_tile<C, K, H>(out, w, n_out, lane, r);
        if constexpr (kPrefetch) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                b[k] = nb[k];
                r[k] = nr[k];
            }
            t = nt;
        } else {
            t = load_pair<C, K, H>(branch, residual, n_src, table, n_out, w + stride, lane, b, r);
        }
    }
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f) {
    return static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> f.s);
}

// One thread per table entry. Entry j = window * win_tokens + t; windows are
// row-major over (bz, bh, bw), tokens row-major over (dz, dh, dw). Gathered
// position p = (b*w + d) reads padded position (p + s) mod padded extent; a
// position past the real grid on any axis is padding (-1). The divisions by
// the window geometry use host-computed multiply-shift reciprocals.
__global__ __launch_bounds__(kBlock) void window_index_kernel(WindowGeometry g, int32_t* table) {
    const uint32_t j = blockIdx.x * kBlock + threadIdx.x;
    if (j >= static_cast<uint32_t>(g.rows)) return;
    const uint32_t wid = fdiv(j, g.div_win);
    const uint32_t t = j - wid * g.win_tokens;
    const uint32_t bzh = fdiv(wid, g.div_nbw);
    const uint32_t bw = wid - bzh * g.nbw;
    const uint32_t bz = fdiv(bzh, g.div_nbh);
    const uint32_t bh = bzh - bz * g.nbh;
    const uint32_t dzh = fdiv(t, g.div_ww);
    const uint32_t dw = t - dzh * g.ww;
    const uint32_t dz = fdiv(dzh, g.div_wh);
    const uint32_t dh = dzh - dz * g.wh;
    // b*w + d < padded extent and s < padded extent: the sum stays below 2^32
    int64_t qz = static_cast<int64_t>(bz) * g.wz + dz + g.sz;
    int64_t qh = static_cast<int64_t>(bh) * g.wh + dh + g.sh;
    int64_t qw = static_cast<int64_t>(bw) * g.ww + dw + g.sw;
    if (qz >= g.Zp) qz -= g.Zp;
    if (qh >= g.Hp) qh -= g.Hp;
    if (qw >= g.Wp) qw -= g.Wp;
    table[j] = (qz < g.Z && qh < g.H && qw < g.W)
                   ? static_cast<int32_t>((qz * g.H + qh) * g.W + qw)
                   : -1;
}

// One thread per source token i = (z*H + h)*W + w: its rolled position is
// g = (q - s) mod padded extent on each axis (the inverse of the forward
// table's q = (p + s) mod padded extent); the gathered row holding it is the
// window of g times the window volume plus g's offset inside the window.
__global__ __launch_bounds__(kBlock) void window_inverse_kernel(WindowGeometry g, int32_t* inverse) {
    const uint32_t i = blockIdx.x * kBlock + threadIdx.x;
    const uint32_t tokens = static_cast<uint32_t>(g.Z) * g.H * g.W;
    if (i >= tokens) return;
    const uint32_t zh = fdiv(i, g.div_W);
    const uint32_t w = i - zh * g.W;
    const uint32_t z = fdiv(zh, g.div_H);
    const uint32_t h = zh - z * g.H;
    // q < real extent <= padded extent and s < padded extent
    const uint32_t gz = z >= static_cast<uint32_t>(g.sz) ? z - g.sz : z + g.Zp - g.sz;
    const uint32_t gh = h >= static_cast<uint32_t>(g.sh) ? h - g.sh : h + g.Hp - g.sh;
    const uint32_t gw = w >= static_cast<uint32_t>(g.sw) ? w - g.sw : w + g.Wp - g.sw;
    const uint32_t bz = fdiv(gz, g.div_wz), bh = fdiv(gh, g.div_wh), bw = fdiv(gw, g.div_ww);
    const uint32_t dz = gz - bz * g.wz, dh = gh - bh * g.wh, dw = gw - bw * g.ww;
    const uint32_t window = (bz * g.nbh + bh) * g.nbw + bw;
    inverse[i] = static_cast<int32_t>(window * g.win_tokens + (dz * g.wh + dh) * g.ww + dw);
}

// ---------------------------------------------------------------------------
// Bias + tanh-GELU, float32 (the fused operator of the page "PyTorch + HIP
// custom fused operator", sections 3-6): y = g(x + bias) with
// g(t) = 0.5 t (1 + tanh z), z = sqrt(2/pi) (t + 0.044715 t^3).
// Since 0.5 (1 + tanh z) = 1 / (1 + exp(-2z)), g(t) = t / (1 + exp(-2z)); the
// exponential is the hardware base-2 one, exp(-2z) = 2^(-2 z log2 e), and the
// division the hardware reciprocal. In the negative tail exp(-2z) grows to
// +Inf and g goes to -0; for t = -Inf the product is NaN, as in the tanh form.

typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float gelu_tanh(float t) {
    constexpr float kMinus2ZLog2e = static_cast<float>(-2.0 * 0.79788456080286535588 * 1.44269504088896340736);
    const float u = t * __builtin_fmaf(0.044715f, t * t, 1.0f);     // t + 0.044715 t^3
    const float e = __builtin_amdgcn_exp2f(kMinus2ZLog2e * u);       // exp(-2z)
    return t * __builtin_amdgcn_rcpf(1.0f + e);
}

template <class H>
__global__ __launch_bounds__(kBlock) void bias_gelu_kernel(const f32x4_t* x, const f32x4_t* __restrict__ bias,
                                                           f32x4_t* y, int64_t n4, FastDiv cols4) {
    const int64_t stride = static_cast<int64_t>(gridDim.x) * kBlock;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kBlock + threadIdx.x; i < n4; i += stride) {
        const uint32_t i32 = static_cast<uint32_t>(i);             // n4 < 2^31
        const uint32_t col = i32 - fdiv(i32, cols4) * cols4.d;
        f32x4_t v;
        if constexpr (H::kNtLoad) v = __builtin_nontemporal_load(x + i);
        else v = x[i];
        const f32x4_t b = bias[col];
        v = f32x4_t{gelu_tanh(v.x + b.x), gelu_tanh(v.y + b.y), gelu_tanh(v.z + b.z), gelu_tanh(v.w + b.w)};
        if constexpr (H::kNtStore) __builtin_nontemporal_store(v, y + i);
        else y[i] = v;
    }
}

// ---------------------------------------------------------------------------
// Launch configuration

// Launch configuration, measured on MI355X with cache-cold buffers (every
// input re-read only after > 1 GiB of other traffic, so nothing is served from
// the 256 MB Infinity Cache).
//
// K (chunks per lane) is fixed per width, so that every LayerNorm kernel of one
// width reduces a row in the same order and their outputs agree bit for bit:
// K = 3 at C = 192 and K = 6 at C = 384, i.e. 8 lanes per row, each wave
// instruction reading whole 128-byte lines of 8 rows (4 lanes per row, 64-byte
// pieces of a line per instruction, measured 10-20% slower); K = 6 at C = 768,
// 16 lanes per row, 256 contiguous bytes of each of 4 rows per instruction.
// Every kernel streams its inputs once and never re-reads its outputs, so all
// loads and stores carry the non-temporal hint; on cold data that beat plain
// and store-only-hinted accesses for every kernel. The grid is one tile per
// wave unless the table of Launch entries below says otherwise. (K = 3 at
// C = 384, 16 lanes per row, measured -2% on the gathers and +5% / +16% on
// ln_fixed / ln_affine; the normalising kernels keep K = 6 so that all of them
// reduce a row alike, and only the plain gather takes K = 3.)
enum class Op { kLn, kAddLn, kGather, kNormGather, kReverseAddLn, kAddNormGather, kLnAffine, kAddLnAffine };

template <int C> struct Width;
// kWideParams: the affine kernels stage gamma and beta in LDS widened to
// binary64. Measured against binary16 staging: C = 384 ln_affine -2.8%,
// add_ln_affine -2.1%; C = 192 +1.2% / +1.0% and C = 768 ln_affine +4.3%, so
// only C = 384 takes it.
template <> struct Width<192> { static constexpr int K = 3; static constexpr bool kWideParams = false; };
template <> struct Width<384> { static constexpr int K = 6; static constexpr bool kWideParams = true; };
// the patch-merge width: 16 lanes per row, 6 chunks each (whole 256-byte pieces
// of 4 rows per wave instruction)
template <> struct Width<768> { static constexpr int K = 6; static constexpr bool kWideParams = false; };

using Streaming = Hints<true, true>;

// Per (width, op): kBlocksPerCu caps the grid at that many workgroups per
// compute unit (0 = one tile per wave); kPrefetch selects the software-pipelined
// row loop (the next tile's loads issued before the current tile is
// normalised); kPriority, kChunks and kWaves are described below. Each entry
// was measured against the alternatives on cold buffers, in interleaved runs on
// one MI355X:
//  * C = 384: with a cap each wave takes 1.3-2.3 tiles and, pipelined,
//    normalises one while the next loads: ln_fixed -11%, norm_gather -10%,
//    add_ln -4%, window_reverse_add_ln -4%, add_ln_affine -6%; ln_affine gains
//    from the cap alone (it loses with the pipeline): cap 3 at first (-9%),
//    cap 4 since its parameters are widened in LDS (128 VGPRs, 4 waves per
//    SIMD; -4% against cap 3, and cap 4 with priority -3%). Register counts
//    (the compiler's NumVgprs) set how many waves are resident, and these caps
//    fill exactly that: the single-input pipelined kernels hold 150-156 VGPRs
//    (3 waves per SIMD) and take cap 3; add_ln, window_reverse_add_ln and
//    add_ln_affine hold 180-194 (2 waves per SIMD) and take cap 2, caps 3 and
//    4 (a second generation of workgroups) measuring 3-16% slower.
//    add_norm_gather (188 VGPRs) is the exception: fastest pipelined at cap 4,
//    -3.4% against cap 2 without the pipeline. Halving the registers (each
//    pass re-widening the binary16 values instead of keeping the binary64
//    deviations) raised residency and made every LayerNorm kernel slower,
//    +3-7% at C = 192 and +13-23% at C = 384, with or without larger caps.
//  * C = 192, one tile per wave: the pipelined form of ln_fixed, add_ln and the
//    fused residual kernels issues the tile's loads ahead of the loop test and
//    measured 2-4% faster; the gathers and ln_affine are fastest as they are.
//    (ln_fixed, add_ln, window_reverse_add_ln and add_ln_affine carry caps
//    that apply only to inputs smaller than the model's; see kMaxTilesPerWave
//    below.)
//  * kPriority: the pipelined two-input kernels at C = 384 and ln_affine at
//    C = 192 issue their loads at wave priority 1 (s_setprio) and drop to 0
//    for the arithmetic: C = 384 add_ln -7%, add_ln_affine -5%,
//    window_reverse_add_ln -1%, C = 192 ln_affine -2.5%. On the one-tile-per-
//    wave kernels it cost up to 4% and is off. The C = 384 norm_gather took it
//    once it ran one-wave workgroups (-2.5 to -2.8%; with four-wave workgroups
//    it had been neutral).
//  * C = 384 norm_gather runs one wave per workgroup, 12 workgroups per
//    compute unit (the same 12 waves as 3 four-wave workgroups): -1.9%. Caps
//    of 8, 16 and 24 one-wave workgroups, the loop without the pipeline, and
//    one tile per wave measured 6-16% slower. (Numbering the waves across
//    workgroups, so that neighbouring tiles land on different XCDs, was 3-30%
//    slower on every kernel.)
//  * C = 384 plain gather: K = 3 (16 lanes per row, 4 rows per wave
//    instruction). Capped at 4 workgroups per compute unit it was -2 to -3%
//    against K = 6 at one tile per wave (caps 2, 3, 5 and 8 and the pipelined
//    loop equal or worse); one tile per wave with 3 resident workgroups per
//    compute unit (kResident, below) is faster again: -3.6% at 32,760 tokens,
//    -4.7% and -4.8% at 65,520 and 131,040 (4 resident -2.7%, K = 6 +1.7%).
//  * C = 768: ln_fixed (150 VGPRs) pipelined at cap 3, -3.4 to -4.5% (cap 2
//    +1%, cap 4 +10%, uncapped -2%); ln_affine at one tile per wave with load
//    priority, -1.1 to -1.4% (caps 2-4 +3 to +10%).
//  * kResident: the plain gather at every width (24-36 VGPRs, so 8 waves per
//    SIMD) reserves enough LDS per workgroup, unused, that at most 3 of its
//    workgroups are resident on a compute unit; the grid stays one tile per
//    wave and the dispatcher starts a workgroup as another ends. With fewer
//    rows in flight the permuted reads and the writes stream better: C = 192
//    -5.8 to -6.1% at 131,040 rows and -4.0% at 65,520 (-0.3% at 32,760),
//    C = 768 -2.3% at 131,040 rows; 4 per CU -4.8% / -1.3%, 5 per CU -4.2% at
//    C = 192, 2 per CU +3.2%. norm_gather at C = 192 (6 waves per SIMD) and
//    bias_gelu gained nothing this way (+0.4 to +0.9% and +3.5 to +24%), nor
//    did ln_affine at C = 192 (+8.3%); add_norm_gather at C = 192 was mixed
//    (-1.3% at 131,040 rows, +2.8% at 32,760).
//  * Everything else: the default.
template <int C, Op O> struct Launch {
    using H = Streaming;
    static constexpr int kBlocksPerCu = 0;
    static constexpr bool kPrefetch = false;
    static constexpr int kPriority = 0;
    static constexpr int kChunks = 0;
    static constexpr int kWaves = kBlock / 64;
    static constexpr int kResident = 0;
};
template <int Cap, bool Prefetch, int Priority = 0, int Chunks = 0, int Waves = kBlock / 64, int Resident = 0>
struct Tuned {
    using H = Streaming;
    static constexpr int kBlocksPerCu = Cap;
    static constexpr bool kPrefetch = Prefetch;
    static constexpr int kPriority = Priority;
    static constexpr int kChunks = Chunks;
    static constexpr int kWaves = Waves;       // waves per workgroup (gathers only)
    static constexpr int kResident = Resident; // resident workgroups per CU, by LDS (gathers only)
};
// Chunks per lane of (width, op): the width's K unless the entry sets kChunks.
// Only the plain gather may set it, as it copies bits and reduces nothing.
// Every normalising kernel of a width keeps Width<C>::K, so they all reduce a
// row in the same order.
template <int C, Op O> constexpr int kChunksOf = Launch<C, O>::kChunks > 0 ? Launch<C, O>::kChunks : Width<C>::K;
template <int C, Op O>
constexpr bool kChunksOk = O == Op::kGather || kChunksOf<C, O> == Width<C>::K;
//                                                  Tuned<cap, pipelined, priority, chunks, waves per workgroup, resident>
template <> struct Launch<192, Op::kLn> : Tuned<4, true> {};
template <> struct Launch<192, Op::kGather> : Tuned<0, false, 0, 0, 4, 3> {};
template <> struct Launch<192, Op::kAddLn> : Tuned<3, true> {};
template <> struct Launch<192, Op::kReverseAddLn> : Tuned<3, true> {};
template <> struct Launch<192, Op::kAddNormGather> : Tuned<0, true> {};
template <> struct Launch<192, Op::kAddLnAffine> : Tuned<2, true> {};
template <> struct Launch<192, Op::kLnAffine> : Tuned<0, false, 1> {};
template <> struct Launch<384, Op::kLn> : Tuned<3, true> {};
template <> struct Launch<384, Op::kNormGather> : Tuned<12, true, 1, 0, 1> {};
template <> struct Launch<384, Op::kGather> : Tuned<0, false, 0, 3, 4, 3> {};
template <> struct Launch<384, Op::kAddLn> : Tuned<2, true, 1> {};
template <> struct Launch<384, Op::kReverseAddLn> : Tuned<2, true, 1> {};
template <> struct Launch<384, Op::kAddLnAffine> : Tuned<2, true, 1> {};
template <> struct Launch<384, Op::kLnAffine> : Tuned<4, false> {};
template <> struct Launch<384, Op::kAddNormGather> : Tuned<4, true> {};
template <> struct Launch<768, Op::kLn> : Tuned<3, true> {};
template <> struct Launch<768, Op::kLnAffine> : Tuned<0, false, 1> {};
template <> struct Launch<768, Op::kGather> : Tuned<0, false, 0, 0, 4, 3> {};

// The caps above were chosen at the model's sizes, where each wave of a capped
// grid takes 1.1-2.3 row tiles. On larger inputs a capped grid makes every wave
// loop over many tiles, and one tile per wave streams better. A capped entry
// keeps its cap only while its waves would take at most kMaxTilesPerWave tiles
// each (0 = always). Measured at C = 384 on 65,520 and 131,040 tokens (grids
// 8 x 182 x 45 and 8 x 364 x 45), cap against one tile per wave: at 131,040 one
// tile per wave was 1-10% faster for every kernel; at 65,520 it was faster
// for norm_gather (-4.4%) and add_norm_gather (-6.0%) at 2.9 and 2.2 tiles per
// wave, and for add_ln, window_reverse_add_ln and add_ln_affine (-3 to -7%) at
// 4 tiles per wave, but slower for ln_fixed (+2.0%, 2.7 tiles per wave). (The
// plain gather, then capped, has since gone to one tile per wave at every
// size.) C = 768 ln_fixed on 131,040 rows: -10.4% with the same limit of 3
// (its 32,760-row size keeps the cap).
// The same rule gives C = 192 ln_fixed, add_ln, window_reverse_add_ln and
// add_ln_affine a cap (4, 3, 3 and 2 workgroups per compute unit) for inputs
// where their waves take at most 2 tiles: -13% (add_ln), -10%
// (window_reverse_add_ln, add_ln_affine) at 32,760 rows, -10% and -4%
// (ln_fixed) at 48,960 and 65,520 rows; at the model's 131,040 rows they run
// one tile per wave as before. The C = 192 gathers, add_norm_gather and
// ln_affine gained at most 2% or lost with caps at those sizes.
template <int C, Op O> constexpr int kMaxTilesPerWave = 0;
template <> constexpr int kMaxTilesPerWave<384, Op::kLn> = 3;
template <> constexpr int kMaxTilesPerWave<384, Op::kAddLn> = 3;
template <> constexpr int kMaxTilesPerWave<384, Op::kReverseAddLn> = 3;
template <> constexpr int kMaxTilesPerWave<384, Op::kAddLnAffine> = 3;
template <> constexpr int kMaxTilesPerWave<384, Op::kLnAffine> = 3;
template <> constexpr int kMaxTilesPerWave<384, Op::kNormGather> = 2;
template <> constexpr int kMaxTilesPerWave<384, Op::kAddNormGather> = 2;
template <> constexpr int kMaxTilesPerWave<768, Op::kLn> = 3;
template <> constexpr int kMaxTilesPerWave<192, Op::kLn> = 2;
template <> constexpr int kMaxTilesPerWave<192, Op::kAddLn> = 2;
template <> constexpr int kMaxTilesPerWave<192, Op::kReverseAddLn> = 2;
template <> constexpr int kMaxTilesPerWave<192, Op::kAddLnAffine> = 2;


// Compute units of the device, queried on first use (0 = not yet known). Only
// the launch shape of capped grids depends on it, never a result; a failed
// query falls back to the MI355X count and clears HIP's last-error state so the
// launch check that follows does not report it.
std::atomic<int> g_cus{0};

inline int compute_units() {
    int cus = g_cus.load(std::memory_order_relaxed);
    if (cus > 0) return cus;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    g_cus.store(cus, std::memory_order_relaxed);
    return cus;
}

template <int C, Op O>
unsigned grid_for(int64_t rows) {
    static_assert(kChunksOk<C, O>, "a normalising kernel must use its width's chunk count");
    static_assert(O == Op::kGather || O == Op::kNormGather || Launch<C, O>::kWaves == kBlock / 64,
                  "only the gathers take their workgroup size from the launch table");
    static_assert(O == Op::kGather || O == Op::kNormGather || Launch<C, O>::kResident == 0,
                  "only the gathers reserve LDS to limit their residency");
    using T = Tile<C, kChunksOf<C, O>>;
    constexpr int kWaves = Launch<C, O>::kWaves;
    const int64_t tiles = (rows + T::kRowsPerWave - 1) / T::kRowsPerWave;
    int64_t blocks = (tiles + kWaves - 1) / kWaves;
    if (Launch<C, O>::kBlocksPerCu > 0) {
        const int64_t cap = static_cast<int64_t>(compute_units()) * Launch<C, O>::kBlocksPerCu;
        constexpr int kMax = kMaxTilesPerWave<C, O>;
        if (blocks > cap && (kMax == 0 || tiles <= static_cast<int64_t>(kMax) * cap * kWaves)) blocks = cap;
    }
    // A dispatch counts its work-items in 32 bits: past 2^32 of them (C = 192
    // ln_fixed on more than 2^29 rows) the grid stops at the largest size below
    // that, and the waves loop over the remaining tiles with the grid stride,
    // as on a capped grid.
    constexpr int64_t kMaxBlocks = ((int64_t{1} << 32) - 1) / (64 * kWaves);
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    return static_cast<unsigned>(blocks);
}

// LDS per compute unit on gfx950 (CDNA4).
constexpr size_t kLdsPerCu = 160 * 1024;

// Dynamic LDS a workgroup of (C, O) reserves so that at most kResident of them
// fit on a compute unit (0 when the entry sets no limit). No kernel reads it.
template <int C, Op O>
constexpr size_t lds_reserve() {
    constexpr int k = Launch<C, O>::kResident;
    static_assert(k == 0 || kLdsPerCu / (k + 1) + 1024 <= 64 * 1024,
                  "a reservation stays within the 64 KB a workgroup may request at launch");
    return k == 0 ? 0 : kLdsPerCu / (k + 1) + 1024;
}

template <int C>
hipError_t ln_fixed_c(const void* x, void* y, int64_t rows, double eps, hipStream_t s) {
    using L = Launch<C, Op::kLn>;
    ln_fixed_kernel<C, Width<C>::K, typename L::H, L::kPrefetch><<<grid_for<C, Op::kLn>(rows), kBlock, 0, s>>>(
        static_cast<const chunk_t*>(x), static_cast<chunk_t*>(y), rows, eps);
    return hipGetLastError();
}

template <int C>
hipError_t add_ln_c(const void* b, const void* r, void* ro, void* y, int64_t rows, double eps,
                    hipStream_t s) {
    using L = Launch<C, Op::kAddLn>;
    add_ln_kernel<C, Width<C>::K, typename L::H, L::kPrefetch, L::kPriority><<<grid_for<C, Op::kAddLn>(rows), kBlock, 0, s>>>(
        static_cast<const chunk_t*>(b), static_cast<const chunk_t*>(r), static_cast<chunk_t*>(ro),
        static_cast<chunk_t*>(y), rows, eps);
    return hipGetLastError();
}

template <int C, bool kNorm>
hipError_t gather_c(const void* x, int64_t n_src, const int32_t* table, int64_t n_out, double eps,
                    void* out, hipStream_t s) {
    constexpr Op O = kNorm ? Op::kNormGather : Op::kGather;
    using L = Launch<C, O>;
    gather_kernel<C, kChunksOf<C, O>, kNorm, typename L::H, L::kPrefetch, L::kWaves, L::kPriority>
        <<<grid_for<C, O>(n_out), 64 * L::kWaves, lds_reserve<C, O>(), s>>>(
        static_cast<const chunk_t*>(x), n_src, table, n_out, static_cast<chunk_t*>(out), eps);
    return hipGetLastError();
}

}  // namespace

// Runs f(std::integral_constant<int, C>) for the served width C (192, 384 or
// 768; the C ABI has already refused any other).
template <class F>
hipError_t by_width(int32_t C, F&& f) {
    switch (C) {
        case 192: return f(std::integral_constant<int, 192>{});
        case 384: return f(std::integral_constant<int, 384>{});
        default: return f(std::integral_constant<int, 768>{});
    }
}

hipError_t launch_ln_fixed(const void* x, void* y, int64_t rows, int32_t C, double eps,
                           hipStream_t stream) {
    return by_width(C, [&](auto c) { return ln_fixed_c<decltype(c)::value>(x, y, rows, eps, stream); });
}

hipError_t launch_add_ln(const void* branch, const void* residual, void* residual_out, void* y,
                         int64_t rows, int32_t C, double eps, hipStream_t stream) {
    return by_width(C, [&](auto c) { return add_ln_c<decltype(c)::value>(branch, residual, residual_out, y, rows, eps, stream); });
}

hipError_t launch_window_index(const WindowGeometry& g, int32_t* table, hipStream_t stream) {
    const unsigned grid = static_cast<unsigned>((static_cast<int64_t>(g.rows) + kBlock - 1) / kBlock);
    window_index_kernel<<<grid, kBlock, 0, stream>>>(g, table);
    return hipGetLastError();
}

hipError_t launch_window_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table,
                                int64_t n_out, void* out, hipStream_t stream) {
    return by_width(C, [&](auto c) { return gather_c<decltype(c)::value, false>(x, n_src, table, n_out, 0.0, out, stream); });
}

hipError_t launch_norm_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table,
                              int64_t n_out, double eps, void* out, hipStream_t stream) {
    return by_width(C, [&](auto c) { return gather_c<decltype(c)::value, true>(x, n_src, table, n_out, eps, out, stream); });
}

hipError_t launch_window_inverse(const WindowGeometry& g, int32_t* inverse, hipStream_t stream) {
    const int64_t tokens = static_cast<int64_t>(g.Z) * g.H * g.W;
    const unsigned grid = static_cast<unsigned>((tokens + kBlock - 1) / kBlock);
    window_inverse_kernel<<<grid, kBlock, 0, stream>>>(g, inverse);
    return hipGetLastError();
}

template <int C>
hipError_t reverse_add_ln_c(const void* win, int64_t n_win, const int32_t* idx, const void* r, void* ro,
                            void* y, int64_t rows, double eps, hipStream_t s) {
    using L = Launch<C, Op::kReverseAddLn>;
    reverse_add_ln_kernel<C, Width<C>::K, typename L::H, L::kPrefetch, L::kPriority>
        <<<grid_for<C, Op::kReverseAddLn>(rows), kBlock, 0, s>>>(
            static_cast<const chunk_t*>(win), n_win, idx, static_cast<const chunk_t*>(r),
            static_cast<chunk_t*>(ro), static_cast<chunk_t*>(y), rows, eps);
    return hipGetLastError();
}

hipError_t launch_reverse_add_ln(const void* win, int64_t n_win, const int32_t* inverse,
                                 const void* residual, void* residual_out, void* y, int64_t rows,
                                 int32_t C, double eps, hipStream_t stream) {
    return by_width(C, [&](auto c) { return reverse_add_ln_c<decltype(c)::value>(win, n_win, inverse, residual, residual_out, y, rows, eps, stream); });
}

template <int C>
hipError_t add_norm_gather_c(const void* b, const void* r, void* ro, int64_t n_src, const int32_t* table,
                             int64_t n_out, double eps, void* out, hipStream_t s) {
    using L = Launch<C, Op::kAddNormGather>;
    add_norm_gather_kernel<C, Width<C>::K, typename L::H, L::kPrefetch>
        <<<grid_for<C, Op::kAddNormGather>(n_out), kBlock, 0, s>>>(
            static_cast<const chunk_t*>(b), static_cast<const chunk_t*>(r), static_cast<chunk_t*>(ro),
            n_src, table, n_out, static_cast<chunk_t*>(out), eps);
    return hipGetLastError();
}

hipError_t launch_add_norm_gather(const void* branch, const void* residual, void* residual_out,
                                  int64_t n_src, int32_t C, const int32_t* table, int64_t n_out,
                                  double eps, void* out, hipStream_t stream) {
    return by_width(C, [&](auto c) { return add_norm_gather_c<decltype(c)::value>(branch, residual, residual_out, n_src, table, n_out, eps, out, stream); });
}

template <int C>
hipError_t ln_affine_c(const void* x, const void* g, const void* b, void* y, int64_t rows, double eps,
                       hipStream_t s) {
    using L = Launch<C, Op::kLnAffine>;
    ln_affine_kernel<C, Width<C>::K, typename L::H, L::kPriority, Width<C>::kWideParams>
        <<<grid_for<C, Op::kLnAffine>(rows), kBlock, 0, s>>>(
        static_cast<const chunk_t*>(x), static_cast<const chunk_t*>(g), static_cast<const chunk_t*>(b),
        static_cast<chunk_t*>(y), rows, eps);
    return hipGetLastError();
}

hipError_t launch_ln_affine(const void* x, const void* gamma, const void* beta, void* y, int64_t rows,
                            int32_t C, double eps, hipStream_t stream) {
    return by_width(C, [&](auto c) { return ln_affine_c<decltype(c)::value>(x, gamma, beta, y, rows, eps, stream); });
}

template <int C>
hipError_t add_ln_affine_c(const void* br, const void* r, const void* g, const void* b, void* ro, void* y,
                           int64_t rows, double eps, hipStream_t s) {
    using L = Launch<C, Op::kAddLnAffine>;
    add_ln_affine_kernel<C, Width<C>::K, typename L::H, L::kPrefetch, L::kPriority, Width<C>::kWideParams>
        <<<grid_for<C, Op::kAddLnAffine>(rows), kBlock, 0, s>>>(
            static_cast<const chunk_t*>(br), static_cast<const chunk_t*>(r), static_cast<const chunk_t*>(g),
            static_cast<const chunk_t*>(b), static_cast<chunk_t*>(ro), static_cast<chunk_t*>(y), rows, eps);
    return hipGetLastError();
}

hipError_t launch_add_ln_affine(const void* branch, const void* residual, const void* gamma, const void* beta,
                                void* residual_out, void* y, int64_t rows, int32_t C, double eps,
                                hipStream_t stream) {
    return by_width(C, [&](auto c) {
        return add_ln_affine_c<decltype(c)::value>(branch, residual, gamma, beta, residual_out, y, rows, eps,
                                                   stream);
    });
}

hipError_t launch_bias_gelu(const void* x, const void* bias, void* y, int64_t rows, int32_t cols,
                            hipStream_t stream) {
    const int64_t n4 = rows * cols / 4;
    const unsigned grid = static_cast<unsigned>((n4 + kBlock - 1) / kBlock);
    bias_gelu_kernel<Streaming><<<grid, kBlock, 0, stream>>>(
        static_cast<const f32x4_t*>(x), static_cast<const f32x4_t*>(bias), static_cast<f32x4_t*>(y), n4,
        make_fastdiv(static_cast<uint32_t>(cols / 4)));
    return hipGetLastError();
}

}  // namespace lwg
