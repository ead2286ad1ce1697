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
//   * Statistics and the normalisation run in binary64 (CDNA4 issues FP64 vector
//     adds and FMAs at the per-lane rate of plain FP32). The sum of a row's
//     binary16 values is exact in binary64, so the mean is one rounding of the
//     exact mean. Where the row's mean is within about 3.9 standard deviations
//     of zero, the variance is taken in the same pass as the sum (mean of
//     squares minus squared mean, which is well conditioned there); other rows
//     (near-constant rows, rows far from zero mean) take a second pass over the
//     deviations. Every output is fma(x, rstd, -mean*rstd), with rstd = 0 for a
//     zero variance (a constant row), whose outputs are then exactly +0. Each
//     output is the correctly rounded binary16 of the exact LayerNorm unless the
//     exact value lies within about 2^-43 (relative) of a rounding midpoint, or
//     on a second-pass row within at most about 2^-38 (absolute); FP32
//     arithmetic would flip about 1e-4 of outputs by one ulp. The
//     final binary64 -> binary16 rounding goes through a round-to-odd binary32
//     intermediate, which makes the two-step conversion exact-once.
//   * All kernels are stateless and row-local: no atomics, no scratch memory.
//     Only the affine kernels use LDS, to hold gamma and beta for a workgroup
//     or a wave;
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

constexpr int kBlock = 256;  // 4 waves: the workgroup of the table builds and bias_gelu

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

// bound_ctrl is set: the row-local patterns used here (quad_perm, row_half_mirror,
// row_mirror) read a lane of the same 16-lane row, so no lane is out of range and
// the instruction needs no "old" operand.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u32(uint32_t v) {
    return static_cast<uint32_t>(
        __builtin_amdgcn_update_dpp(0, static_cast<int>(v), CTRL, 0xF, 0xF, true));
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

// The 8 binary16 values of a chunk widened to S (binary32 or binary64; both hold
// every binary16 value exactly).
template <class S>
__device__ __forceinline__ void unpack8(const chunk_t& c, S* out) {
    const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const half2_t h = __builtin_bit_cast(half2_t, w[i]);
        out[2 * i] = static_cast<S>(static_cast<float>(h.x));
        out[2 * i + 1] = static_cast<S>(static_cast<float>(h.y));
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

// 1/sqrt(a) for a > 0: the hardware reciprocal-square-root estimate (relative
// error below 2^-24, measured on MI355X) refined by two Newton steps,
// r' = r (3/2 - a r^2 / 2), each taking a relative error e to about 1.5 e^2:
// below 2^-47 after the first and at binary64's own rounding level (measured
// 2^-52.7) after the second. Inf and NaN give NaN.
__device__ __forceinline__ double newton_rsqrt(double a, double r) {
    const double h = a * (0.5 * r);    // 0.5 * r is exact; no underflow for subnormal a
    return __builtin_fma(r, __builtin_fma(-h, r, 0.5), r);
}

__device__ __forceinline__ double rsqrt_refined(double a) {
    return newton_rsqrt(a, newton_rsqrt(a, __builtin_amdgcn_rsq(a)));
}

// Row values kept in binary32 between the passes of the LayerNorm are widened
// to binary64 where each pass uses them. This empty register constraint tells
// the compiler the values may have changed, so it widens them again instead of
// keeping a binary64 copy live across the pass (which would double the
// registers the row takes). Binary64 row values need nothing.
template <int N>
__device__ __forceinline__ void rewiden_each_pass(float (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(x[i]));
}
template <int N>
__device__ __forceinline__ void rewiden_each_pass(double (&)[N]) {}

// Rows whose mean of squares is at most this multiple of their variance (|mean|
// up to sqrt(15) standard deviations) take the variance from the first pass.
// The mean of squares carries a relative error of at most ~2^-47 (a sum of at
// most 48 products per lane, 4 DPP steps and one scaling), so the first-pass
// variance is good to ~2^-43 there, far below the 2^-11 of a binary16 result.
constexpr double kOnePassLimit = 16.0;

// Scale of the LayerNorm of the row whose 1/LPR share this lane holds in x:
// every output is y = fma(x, rstd, shift) with shift = -mean * rstd.
//  * Rows whose mean is within about 3.9 standard deviations of zero (and
//    all-zero rows) take the variance from the first pass: the pre-rounding y
//    has a relative error below ~2^-43.
//  * Other rows take the variance over the deviations (a second pass). A
//    constant row has variance exactly 0 (its mean is exact) and gets rstd = 0,
//    so every output is exactly +0, as (x - mean) / sqrt(eps) is. Any other
//    binary16 row has |mean| below ~2^15 standard deviations, so rounding
//    mean * rstd costs at most ~2^-38 of absolute error in y.
//  * A row holding Inf or NaN gives NaN throughout.
struct RowScale {
    double rstd, shift;
};

template <int C, int K, class S>
__device__ __forceinline__ RowScale row_scale(S (&x)[8 * K], double eps) {
    using T = Tile<C, K>;
    constexpr double kInvC = 1.0 / C;
    double s0, s1, q0, q1;
    {
        const double a = x[0], b = x[1];
        s0 = a;
        s1 = b;
        q0 = a * a;
        q1 = b * b;
    }
#pragma unroll
    for (int i = 2; i < T::kValues; i += 2) {
        const double a = x[i], b = x[i + 1];
        s0 += a;
        s1 += b;
        q0 = __builtin_fma(a, a, q0);
        q1 = __builtin_fma(b, b, q1);
    }
    // the sum of binary16 values is a multiple of 2^-24 below 2^26: exact here
    const double mean = group_sum<T::kLanes>(s0 + s1) * kInvC;
    const double m2 = group_sum<T::kLanes>(q0 + q1) * kInvC;
    double var = __builtin_fma(-mean, mean, m2);
    // all-zero rows (padding) are one-pass too; NaN and Inf rows are not
    const bool one_pass = (var > 0.0 && m2 <= kOnePassLimit * var) || m2 == 0.0;
    rewiden_each_pass(x);
    if (__builtin_amdgcn_ballot_w64(!one_pass) != 0) {
        double p0 = 0.0, p1 = 0.0;
#pragma unroll
        for (int i = 0; i < T::kValues; i += 2) {
            const double d0 = static_cast<double>(x[i]) - mean;
            const double d1 = static_cast<double>(x[i + 1]) - mean;
            p0 = __builtin_fma(d0, d0, p0);
            p1 = __builtin_fma(d1, d1, p1);
        }
        const double var2 = group_sum<T::kLanes>(p0 + p1) * kInvC;
        if (!one_pass) var = var2;
        rewiden_each_pass(x);
    }
    RowScale rs;
    rs.rstd = var == 0.0 ? 0.0 : rsqrt_refined(var + eps);
    rs.shift = -mean * rs.rstd;
    return rs;
}

// LayerNorm of the row whose 1/LPR share this lane holds in v, rounded to
// binary16 and written back into v. S is the register type of the row values
// between passes (binary32 or binary64; the results do not depend on it). Every
// kernel that normalises a row calls this same function with its width's
// (C, K), so their outputs agree bit for bit.
template <int C, int K, class S>
__device__ __forceinline__ void layer_norm_lane(chunk_t (&v)[K], double eps) {
    S x[8 * K];
#pragma unroll
    for (int k = 0; k < K; ++k) unpack8(v[k], x + 8 * k);
    const RowScale rs = row_scale<C, K>(x, eps);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        double y[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) y[e] = __builtin_fma(static_cast<double>(x[8 * k + e]), rs.rstd, rs.shift);
        v[k] = chunk_t{pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7])};
    }
}

// The 8 values of parameter chunk i, from LDS staged either as the binary16
// chunks themselves or already widened to binary64 (8 doubles per chunk).
__device__ __forceinline__ void param_chunk(const chunk_t* p, int i, double (&out)[8]) { unpack8(p[i], out); }
__device__ __forceinline__ void param_chunk(const double* p, int i, double (&out)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) out[e] = p[8 * i + e];
}

// Affine LayerNorm: (normalised x) * gamma + beta in binary64, rounded once to
// binary16. gamma and beta are binary16 [C], held in LDS by the affine kernels
// (as chunks, or widened: P); this lane reads its columns chunk by chunk as it
// writes them, so only one chunk of them is live next to the row values.
template <int C, int K, class S, class P>
__device__ __forceinline__ void layer_norm_affine_lane(chunk_t (&v)[K], const P* gamma,
                                                       const P* beta, int sub, double eps) {
    using T = Tile<C, K>;
    S x[8 * K];
#pragma unroll
    for (int k = 0; k < K; ++k) unpack8(v[k], x + 8 * k);
    const RowScale rs = row_scale<C, K>(x, eps);
#pragma unroll
    for (int k = 0; k < K; ++k) {
        double gk[8], bk[8], y[8];
        param_chunk(gamma, sub + k * T::kLanes, gk);
        param_chunk(beta, sub + k * T::kLanes, bk);
#pragma unroll
        for (int e = 0; e < 8; ++e)
            y[e] = __builtin_fma(__builtin_fma(static_cast<double>(x[8 * k + e]), rs.rstd, rs.shift), gk[e], bk[e]);
        v[k] = chunk_t{pack2(y[0], y[1]), pack2(y[2], y[3]), pack2(y[4], y[5]), pack2(y[6], y[7])};
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
// of resident workgroups. kWaves is the number of waves in a workgroup.

template <int kWaves>
__device__ __forceinline__ int64_t first_wave_in() {
    return static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
}

template <int kWaves>
__device__ __forceinline__ int64_t wave_stride_in() {
    return static_cast<int64_t>(gridDim.x) * kWaves;
}

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
template <int C, int K, class H, bool kPrefetch, int kPrio, int kWaves, class S>
__global__ __launch_bounds__(64 * kWaves) void ln_fixed_kernel(const chunk_t* x, chunk_t* y,
                                                               int64_t rows, double eps) {
    using T = Tile<C, K>;
    const int lane = threadIdx.x & 63;
    const int64_t stride = wave_stride_in<kWaves>();
    int64_t w = first_wave_in<kWaves>();
    if constexpr (kPrefetch) {
        chunk_t v[K];
        load_tile<C, K, H, kPrio>(x, w, rows, lane, v);
        for (; w * T::kRowsPerWave < rows; w += stride) {
            chunk_t next[K];
            load_tile<C, K, H, kPrio>(x, w + stride, rows, lane, next);
            layer_norm_lane<C, K, S>(v, eps);
            store_tile<C, K, H>(y, w, rows, lane, v);
#pragma unroll
            for (int k = 0; k < K; ++k) v[k] = next[k];
        }
    } else {
        for (; w * T::kRowsPerWave < rows; w += stride) {
            chunk_t v[K];
            load_tile<C, K, H, kPrio>(x, w, rows, lane, v);
            layer_norm_lane<C, K, S>(v, eps);
            store_tile<C, K, H>(y, w, rows, lane, v);
        }
    }
}

// residual_out and y may alias the inputs: each lane reads its chunks of a row
// before it writes any, and the prefetched tile is a different set of rows.
template <int C, int K, class H, bool kPrefetch, int kPrio, int kWaves, class S>
__global__ __launch_bounds__(64 * kWaves) void add_ln_kernel(const chunk_t* branch, const chunk_t* residual,
                                                             chunk_t* residual_out, chunk_t* y,
                                                             int64_t rows, double eps) {
    using T = Tile<C, K>;
    const int lane = threadIdx.x & 63;
    const int64_t stride = wave_stride_in<kWaves>();
    int64_t w = first_wave_in<kWaves>();
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
        layer_norm_lane<C, K, S>(r, eps);
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
// binary16 [C]; each workgroup (or each wave, below) copies them into LDS and
// every lane reads its columns from there chunk by chunk, so the parameters
// neither occupy the vector-memory path nor sit widened in registers. kWide
// selects the LDS form:
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
    for (int i = threadIdx.x; i < 2 * kChunks; i += blockDim.x)
        params[i] = i < kChunks ? gamma[i] : beta[i - kChunks];
    __syncthreads();
}

template <int C>
__device__ __forceinline__ void stage_params(double* params, const chunk_t* gamma, const chunk_t* beta) {
    constexpr int kChunks = C / 8;
    for (int i = threadIdx.x; i < 2 * kChunks; i += blockDim.x) {
        double v[8];
        unpack8(i < kChunks ? gamma[i] : beta[i - kChunks], v);
#pragma unroll
        for (int e = 0; e < 8; ++e) params[8 * i + e] = v[e];
    }
    __syncthreads();
}

// Staging of gamma and beta, by the launch entry's kStage:
//  * kStageFirst: one copy per workgroup, staged (loaded, written, barrier)
//    before any row load;
//  * kWaveCopy: one copy per wave. The wave issues its parameter loads, then
//    its row loads, then waits for the parameter loads only (issued first, so
//    the rows stay in flight) and writes its copy. No workgroup barrier: LDS
//    operations of one wave complete in order, and the fences keep the
//    compiler from moving the wave's reads of its copy above its writes;
//  * kFetchFirst: one copy per workgroup, loaded ahead of the row loads and
//    written after them, behind a barrier: a slow parameter fetch then
//    delays only the arithmetic, not the row loads.
enum ParamStage : int { kStageFirst = 0, kWaveCopy = 1, kFetchFirst = 2 };

// The 2*C/8 parameter chunks (gamma, then beta) that the kThreads threads of
// one copy load, kPerThread per thread.
template <int C, int kThreads>
struct ParamChunks {
    static constexpr int kChunks = C / 8;
    static constexpr int kPerThread = (2 * kChunks + kThreads - 1) / kThreads;
    chunk_t v[kPerThread];
};

template <int C, int kThreads>
__device__ __forceinline__ ParamChunks<C, kThreads> fetch_params(const chunk_t* gamma, const chunk_t* beta, int t) {
    using PC = ParamChunks<C, kThreads>;
    PC p;
#pragma unroll
    for (int j = 0; j < PC::kPerThread; ++j) {
        const int i = t + kThreads * j;
        p.v[j] = i < PC::kChunks ? gamma[i] : i < 2 * PC::kChunks ? beta[i - PC::kChunks] : chunk_t{0u, 0u, 0u, 0u};
    }
    return p;
}

template <int C, int kThreads>
__device__ __forceinline__ void put_params(chunk_t* params, const ParamChunks<C, kThreads>& p, int t) {
    using PC = ParamChunks<C, kThreads>;
#pragma unroll
    for (int j = 0; j < PC::kPerThread; ++j) {
        const int i = t + kThreads * j;
        if (i < 2 * PC::kChunks) params[i] = p.v[j];
    }
}

template <int C, int kThreads>
__device__ __forceinline__ void put_params(double* params, const ParamChunks<C, kThreads>& p, int t) {
    using PC = ParamChunks<C, kThreads>;
#pragma unroll
    for (int j = 0; j < PC::kPerThread; ++j) {
        const int i = t + kThreads * j;
        if (i < 2 * PC::kChunks) {
            double v[8];
            unpack8(p.v[j], v);
#pragma unroll
            for (int e = 0; e < 8; ++e) params[8 * i + e] = v[e];
        }
    }
}

__device__ __forceinline__ void wave_params_written() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// An affine kernel's parameter staging around its first row loads: begin()
// before them, end() after; copy() is the copy this thread's wave reads.
template <int C, int kWaves, bool kWide, int kStage>
struct AffineParams {
    using A = AffineStage<C, kWide>;
    using P = typename A::P;
    static_assert(kStage == kStageFirst || kStage == kWaveCopy || kStage == kFetchFirst, "unknown parameter staging");
    static constexpr int kCopies = kStage == kWaveCopy ? kWaves : 1;
    static constexpr int kThreads = kStage == kWaveCopy ? 64 : 64 * kWaves;
    static constexpr int kEntries = kCopies * 2 * A::kHalf;
    P* base;
    ParamChunks<C, kThreads> fetched;
    __device__ __forceinline__ int thread() const {
        return kStage == kWaveCopy ? static_cast<int>(threadIdx.x & 63) : static_cast<int>(threadIdx.x);
    }
    __device__ __forceinline__ P* copy() const {
        return kStage == kWaveCopy ? base + (threadIdx.x >> 6) * 2 * A::kHalf : base;
    }
    __device__ __forceinline__ void begin(const chunk_t* gamma, const chunk_t* beta) {
        if constexpr (kStage == kStageFirst) stage_params<C>(base, gamma, beta);
        else fetched = fetch_params<C, kThreads>(gamma, beta, thread());
    }
    __device__ __forceinline__ void end() {
        if constexpr (kStage == kWaveCopy) {
            put_params<C, kThreads>(copy(), fetched, thread());
            wave_params_written();
        } else if constexpr (kStage == kFetchFirst) {
            put_params<C, kThreads>(copy(), fetched, thread());
            __syncthreads();
        }
    }
};

template <int C, int K, class H, bool kPrefetch, int kPrio, int kWaves, class S, bool kWide, int kStage>
__global__ __launch_bounds__(64 * kWaves) void ln_affine_kernel(const chunk_t* x, const chunk_t* gamma,
                                                                const chunk_t* beta, chunk_t* y,
                                                                int64_t rows, double eps) {
    using T = Tile<C, K>;
    using AP = AffineParams<C, kWaves, kWide, kStage>;
    __shared__ typename AP::P params[AP::kEntries];
    AP ap{params, {}};
    ap.begin(gamma, beta);
    const int lane = threadIdx.x & 63;
    const int sub = lane % T::kLanes;
    const int64_t stride = wave_stride_in<kWaves>();
    int64_t w = first_wave_in<kWaves>();
    chunk_t v[K];
    load_tile<C, K, H, kPrio>(x, w, rows, lane, v);
    ap.end();
    const typename AP::P* gamma_s = ap.copy();
    const typename AP::P* beta_s = gamma_s + AP::A::kHalf;
    for (; w * T::kRowsPerWave < rows; w += stride) {
        chunk_t next[K];
        if constexpr (kPrefetch) load_tile<C, K, H, kPrio>(x, w + stride, rows, lane, next);
        // re-read gamma/beta from LDS per row tile instead of letting the
        // compiler hoist 2*K widened chunks out of the loop into registers
        asm volatile("" ::: "memory");
        layer_norm_affine_lane<C, K, S>(v, gamma_s, beta_s, sub, eps);
        store_tile<C, K, H>(y, w, rows, lane, v);
        if constexpr (kPrefetch) {
#pragma unroll
            for (int k = 0; k < K; ++k) v[k] = next[k];
        } else {
            load_tile<C, K, H, kPrio>(x, w + stride, rows, lane, v);
        }
    }
}

template <int C, int K, class H, bool kPrefetch, int kPrio, int kWaves, class S, bool kWide, int kStage>
__global__ __launch_bounds__(64 * kWaves) void add_ln_affine_kernel(const chunk_t* branch, const chunk_t* residual,
                                                                    const chunk_t* gamma, const chunk_t* beta,
                                                                    chunk_t* residual_out, chunk_t* y,
                                                                    int64_t rows, double eps) {
    using T = Tile<C, K>;
    using AP = AffineParams<C, kWaves, kWide, kStage>;
    __shared__ typename AP::P params[AP::kEntries];
    AP ap{params, {}};
    ap.begin(gamma, beta);
    const int lane = threadIdx.x & 63;
    const int sub = lane % T::kLanes;
    const int64_t stride = wave_stride_in<kWaves>();
    int64_t w = first_wave_in<kWaves>();
    chunk_t b[K], r[K];
    load_tile<C, K, H, kPrio>(branch, w, rows, lane, b);
    load_tile<C, K, H, kPrio>(residual, w, rows, lane, r);
    ap.end();
    const typename AP::P* gamma_s = ap.copy();
    const typename AP::P* beta_s = gamma_s + AP::A::kHalf;
    for (; w * T::kRowsPerWave < rows; w += stride) {
        chunk_t nb[K], nr[K];
        if constexpr (kPrefetch) {
            load_tile<C, K, H, kPrio>(branch, w + stride, rows, lane, nb);
            load_tile<C, K, H, kPrio>(residual, w + stride, rows, lane, nr);
        }
        asm volatile("" ::: "memory");  // as in ln_affine_kernel: no hoisting of gamma/beta
        residual_add<K>(b, r);
        store_tile<C, K, H>(residual_out, w, rows, lane, r);
        layer_norm_affine_lane<C, K, S>(r, gamma_s, beta_s, sub, eps);
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

template <int C, int K, bool kNorm, class H, bool kPrefetch, int kWaves, int kPrio, class S>
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
            if constexpr (kNorm) layer_norm_lane<C, K, S>(v, eps);
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
            if constexpr (kNorm) layer_norm_lane<C, K, S>(v, eps);
            if (live) {
                const int64_t dst = j * T::kChunks + sub;
#pragma unroll
                for (int k = 0; k < K; ++k) store16<H>(out + dst + k * T::kLanes, v[k]);
            }
        }
    }
}

// Plain gather with kTiles row tiles per wave (tiles g + i * (waves in the
// grid)): the wave reads all of its table entries first, then the source rows
// of every tile, then stores them, so each wave has all of its loads in flight
// before the first store. The grid has ceil(tiles / kTiles) waves.
template <int C, int K, class H, int kTiles, int kWaves, int kPrio>
__global__ __launch_bounds__(64 * kWaves) void gather_tiles_kernel(const chunk_t* __restrict__ x, int64_t n_src,
                                                                   const int32_t* __restrict__ table,
                                                                   int64_t n_out, chunk_t* __restrict__ out) {
    using T = Tile<C, K>;
    const int lane = threadIdx.x & 63;
    const int sub = lane % T::kLanes;
    const int64_t g = first_wave_in<kWaves>();
    const int64_t waves = wave_stride_in<kWaves>();
    int64_t j[kTiles];
    int32_t t[kTiles];
    if constexpr (kPrio > 0) __builtin_amdgcn_s_setprio(kPrio);
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
        j[i] = (g + i * waves) * T::kRowsPerWave + lane / T::kLanes;
        t[i] = j[i] < n_out ? table[j[i]] : -1;
    }
    chunk_t v[kTiles][K];
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
        zero(v[i]);
        if (t[i] >= 0 && static_cast<int64_t>(t[i]) < n_src) {
            const int64_t src = static_cast<int64_t>(t[i]) * T::kChunks + sub;
#pragma unroll
            for (int k = 0; k < K; ++k) v[i][k] = load16<H>(x + src + k * T::kLanes);
        }
    }
    if constexpr (kPrio > 0) __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < kTiles; ++i) {
        if (j[i] < n_out) {
            const int64_t dst = j[i] * T::kChunks + sub;
#pragma unroll
            for (int k = 0; k < K; ++k) store16<H>(out + dst + k * T::kLanes, v[i][k]);
        }
    }
}

// Window reverse fused with the residual add + LayerNorm: token row i takes
// its branch from window row idx[i] (the inverse table), adds the residual,
// writes the rounded sum, and normalises it. An index outside [0, n_win) gives
// a zero branch. residual_out and y may alias residual (row i is read and
// written by the same lanes; a prefetched tile holds other rows); neither may
// overlap win, whose rows a prefetch may read after another row was written.
template <int C, int K, class H, bool kPrefetch, int kPrio, int kWaves, class S>
__global__ __launch_bounds__(64 * kWaves) void reverse_add_ln_kernel(
    const chunk_t* __restrict__ win, int64_t n_win, const int32_t* __restrict__ idx,
    const chunk_t* residual, chunk_t* residual_out, chunk_t* y, int64_t rows, double eps) {
    using T = Tile<C, K>;
    const int lane = threadIdx.x & 63;
    const int64_t stride = wave_stride_in<kWaves>();
    int64_t w = first_wave_in<kWaves>();
    chunk_t b[K], r[K];
    load_gathered<C, K, H, kPrio>(win, n_win, idx, rows, w, lane, b);
    load_tile<C, K, H, kPrio>(residual, w, rows, lane, r);
    for (; w * T::kRowsPerWave < rows; w += stride) {
        chunk_t nb[K], nr[K];
        if constexpr (kPrefetch) {
            load_gathered<C, K, H, kPrio>(win, n_win, idx, rows, w + stride, lane, nb);
            load_tile<C, K, H, kPrio>(residual, w + stride, rows, lane, nr);
        }
        residual_add<K>(b, r);
        store_tile<C, K, H>(residual_out, w, rows, lane, r);
        layer_norm_lane<C, K, S>(r, eps);
        store_tile<C, K, H>(y, w, rows, lane, r);
        if constexpr (kPrefetch) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                b[k] = nb[k];
                r[k] = nr[k];
            }
        } else {
            load_gathered<C, K, H, kPrio>(win, n_win, idx, rows, w + stride, lane, b);
            load_tile<C, K, H, kPrio>(residual, w + stride, rows, lane, r);
        }
    }
}

// Branch and residual chunks of the source row of gathered row j (zeros and -1
// for padding or an out-of-range entry); returns the source row or -1.
template <int C, int K, class H, int kPrio>
__device__ __forceinline__ int32_t load_pair(const chunk_t* branch, const chunk_t* residual, int64_t n_src,
                                             const int32_t* table, int64_t n_out, int64_t w, int lane,
                                             chunk_t (&b)[K], chunk_t (&r)[K]) {
    using T = Tile<C, K>;
    if constexpr (kPrio > 0) __builtin_amdgcn_s_setprio(kPrio);
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
    if constexpr (kPrio > 0) __builtin_amdgcn_s_setprio(0);
    return t;
}

// Residual add + LayerNorm + window gather, output-major: gathered row j reads
// token t = table[j] from branch and residual, writes the rounded sum to
// residual_out[t] and its LayerNorm to out[j]; padding rows store +0.0 and
// touch no token. With a table whose valid entries are distinct (as built by
// window_index_kernel) every token row is read and written by exactly one lane
// group, and a prefetched tile reads other tokens than the one being written,
// so residual_out may alias residual or branch.
template <int C, int K, class H, bool kPrefetch, int kPrio, int kWaves, class S>
__global__ __launch_bounds__(64 * kWaves) void add_norm_gather_kernel(
    const chunk_t* branch, const chunk_t* residual, chunk_t* residual_out, int64_t n_src,
    const int32_t* __restrict__ table, int64_t n_out, chunk_t* __restrict__ out, double eps) {
    using T = Tile<C, K>;
    const int lane = threadIdx.x & 63;
    const int sub = lane % T::kLanes;
    const int64_t stride = wave_stride_in<kWaves>();
    int64_t w = first_wave_in<kWaves>();
    chunk_t b[K], r[K];
    int32_t t = load_pair<C, K, H, kPrio>(branch, residual, n_src, table, n_out, w, lane, b, r);
    for (; w * T::kRowsPerWave < n_out; w += stride) {
        chunk_t nb[K], nr[K];
        int32_t nt = -1;
        if constexpr (kPrefetch)
            nt = load_pair<C, K, H, kPrio>(branch, residual, n_src, table, n_out, w + stride, lane, nb, nr);
        residual_add<K>(b, r);
        if (t >= 0) {
            const int64_t src = static_cast<int64_t>(t) * T::kChunks + sub;
#pragma unroll
            for (int k = 0; k < K; ++k) store16<H>(residual_out + src + k * T::kLanes, r[k]);
        }
        layer_norm_lane<C, K, S>(r, eps);
        store_tile<C, K, H>(out, w, n_out, lane, r);
        if constexpr (kPrefetch) {
#pragma unroll
            for (int k = 0; k < K; ++k) {
                b[k] = nb[k];
                r[k] = nr[k];
            }
            t = nt;
        } else {
            t = load_pair<C, K, H, kPrio>(branch, residual, n_src, table, n_out, w + stride, lane, b, r);
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
// and store-only-hinted accesses for every kernel.
enum class Op { kLn, kAddLn, kGather, kNormGather, kReverseAddLn, kAddNormGather, kLnAffine, kAddLnAffine };

template <int C> struct Width;
// kWideParams: the affine kernels stage gamma and beta in LDS widened to
// binary64 (C = 384), or as the binary16 chunks (C = 192 and 768).
template <> struct Width<192> { static constexpr int K = 3; static constexpr bool kWideParams = false; };
template <> struct Width<384> { static constexpr int K = 6; static constexpr bool kWideParams = true; };
// the patch-merge width: 16 lanes per row, 6 chunks each (whole 256-byte pieces
// of 4 rows per wave instruction)
template <> struct Width<768> { static constexpr int K = 6; static constexpr bool kWideParams = false; };

using Streaming = Hints<true, true>;

// Per (width, op):
//  * kBlocksPerCu caps the grid at that many workgroups per compute unit
//    (0 = one tile per wave, or kTiles tiles per wave);
//  * kPrefetch selects the software-pipelined row loop (the next tile's loads
//    issued before the current tile is normalised);
//  * kPriority > 0 issues the loads at that wave priority (s_setprio) and drops
//    to 0 for the arithmetic and the stores;
//  * kWaves is the workgroup size in waves;
//  * Row is the register type of a row between the passes of the LayerNorm:
//    double, or float (exact for binary16, widened again in each pass: one
//    conversion more per value and pass, half the registers);
//  * kResident reserves enough LDS per workgroup, unread, that at most that
//    many workgroups are resident on a compute unit;
//  * kChunks overrides K (plain gather only: it reduces nothing);
//  * kTiles > 1 gives each wave that many tiles, all loads first (plain gather
//    only);
//  * kStage (affine kernels) is how gamma and beta reach LDS (ParamStage): one
//    copy per workgroup staged before any row load; one copy per wave fetched
//    ahead of the row loads and written after them without a barrier; or one
//    copy per workgroup fetched ahead and written after them, behind a
//    barrier.
template <int C, Op O> struct Launch {
    using H = Streaming;
    using Row = double;
    static constexpr int kBlocksPerCu = 0;
    static constexpr bool kPrefetch = false;
    static constexpr int kPriority = 0;
    static constexpr int kWaves = 4;
    static constexpr int kResident = 0;
    static constexpr int kChunks = 0;
    static constexpr int kTiles = 1;
    static constexpr int kStage = 0;
};
template <int Cap, bool Prefetch, int Priority = 0, int Waves = 4, class R = double, int Resident = 0,
          int Chunks = 0, int Tiles = 1, int Stage = 0>
struct Tuned {
    using H = Streaming;
    using Row = R;
    static constexpr int kBlocksPerCu = Cap;
    static constexpr bool kPrefetch = Prefetch;
    static constexpr int kPriority = Priority;
    static constexpr int kWaves = Waves;
    static constexpr int kResident = Resident;
    static constexpr int kChunks = Chunks;
    static constexpr int kTiles = Tiles;
    static constexpr int kStage = Stage;
};
// Chunks per lane of a launch entry at width C: the width's K unless the entry
// sets kChunks.
template <int C, class L> constexpr int kChunksOf = L::kChunks > 0 ? L::kChunks : Width<C>::K;
template <int C, Op O, class L>
constexpr bool kChunksOk = O == Op::kGather || kChunksOf<C, L> == Width<C>::K;

// Level 1 (C = 192, 131,040 rows): every kernel holds its row in binary64.
//  * ln_fixed, add_ln and the fused residual kernels: the pipelined loop, which
//    issues a tile's loads ahead of the loop test (2-4% faster than the plain
//    loop at one tile per wave); their caps apply only below the model's size
//    (kMaxTilesPerWave).
//  * plain gather: one tile per wave with at most 3 resident workgroups per
//    compute unit (-6% against no limit: fewer rows in flight stream better).
//  * norm_gather: one tile per wave in 4-wave workgroups, at most 6 resident
//    per compute unit (its 70 registers would allow 7: -1.5%).
//  * ln_affine: one tile per wave with load priority.
//  * ln_affine and add_ln_affine: a per-wave copy of gamma and beta (-2.4% and
//    -1.1% against one copy per workgroup behind a barrier).
//                                                  Tuned<cap, pipelined, priority, waves, row, resident, chunks, tiles>
template <> struct Launch<192, Op::kLn> : Tuned<4, true> {};
template <> struct Launch<192, Op::kGather> : Tuned<0, false, 0, 4, double, 3> {};
template <> struct Launch<192, Op::kNormGather> : Tuned<0, false, 0, 4, double, 6> {};
template <> struct Launch<192, Op::kAddLn> : Tuned<3, true> {};
template <> struct Launch<192, Op::kReverseAddLn> : Tuned<3, true> {};
template <> struct Launch<192, Op::kAddNormGather> : Tuned<0, true> {};
template <> struct Launch<192, Op::kAddLnAffine> : Tuned<2, true, 0, 4, double, 0, 0, 1, kWaveCopy> {};
template <> struct Launch<192, Op::kLnAffine> : Tuned<0, false, 1, 4, double, 0, 0, 1, kWaveCopy> {};
// Level 2 (C = 384, 32,760 rows): one tile per wave with load priority and the
// row held in binary32, which leaves the single-input LayerNorm kernels and
// add_ln so few registers (68-88) that the whole grid is resident at once:
// each wave issues its loads as it starts and normalises as soon as they land.
// Against the pipelined loop on a capped grid (binary64 rows): ln_fixed -8%,
// norm_gather -5%, add_ln -2%, window_reverse_add_ln -1.4%.
//  * ln_fixed, norm_gather and window_reverse_add_ln: one-wave workgroups;
//    add_ln and ln_affine: 4-wave workgroups.
//  * ln_affine loads gamma and beta ahead of its rows and writes them to LDS
//    after (kFetchFirst). Staged before the row loads, the copy made every
//    wave wait on a cold parameter fetch first: on some MI355X devices its
//    timings then spread 6-13% (9.3-10.7 us); fetched first they stay within
//    1.5% at 9.6 us, the former mean.
//  * add_norm_gather and add_ln_affine stay on the pipelined loop over a capped
//    grid with binary64 rows (4 and 2 workgroups per compute unit; one tile per
//    wave measured 1-5% slower for them).
//  * plain gather: one-wave workgroups with 2 tiles per wave, all table
//    entries and rows loaded before the first store (-7.4% against one tile per
//    wave with 3 resident workgroups per compute unit).
template <> struct Launch<384, Op::kLn> : Tuned<0, false, 1, 1, float> {};
template <> struct Launch<384, Op::kNormGather> : Tuned<0, false, 1, 1, float> {};
template <> struct Launch<384, Op::kGather> : Tuned<0, false, 1, 1, double, 0, 6, 2> {};
template <> struct Launch<384, Op::kAddLn> : Tuned<0, false, 1, 4, float> {};
template <> struct Launch<384, Op::kReverseAddLn> : Tuned<0, false, 1, 1, float> {};
template <> struct Launch<384, Op::kAddLnAffine> : Tuned<2, true, 1, 4, double> {};
template <> struct Launch<384, Op::kLnAffine> : Tuned<0, false, 1, 4, float, 0, 0, 1, kFetchFirst> {};
template <> struct Launch<384, Op::kAddNormGather> : Tuned<4, true, 0, 4, double> {};
// Patch merge (C = 768, 32,760 rows): ln_fixed and ln_affine one tile per wave
// in one-wave workgroups with load priority and binary32 rows (-1.3% against
// the capped pipelined loop); ln_affine takes gamma and beta into its wave's
// own LDS copy behind its first row loads (-3.8% against 4-wave workgroups
// staging one copy before them). At C = 384 the per-wave copy, widened to
// binary64, measured +2.4 to +3.5% and is not used.
// add_ln and window_reverse_add_ln: the pipelined loop with binary64 rows
// (-2.8% and -5.2% against the plain loop at 32,760 rows, -4% and -7% at
// 131,040).
template <> struct Launch<768, Op::kLn> : Tuned<0, false, 1, 1, float> {};
template <> struct Launch<768, Op::kLnAffine> : Tuned<0, false, 1, 1, float, 0, 0, 1, kWaveCopy> {};
template <> struct Launch<768, Op::kGather> : Tuned<0, false, 0, 4, double, 3> {};
template <> struct Launch<768, Op::kAddLn> : Tuned<0, true> {};
template <> struct Launch<768, Op::kReverseAddLn> : Tuned<0, true> {};

// A capped entry keeps its cap only while its waves would take at most
// kMaxTilesPerWave tiles each (0 = always); on larger inputs a capped grid
// makes every wave loop over many tiles, and one tile per wave streams better.
// C = 192 ln_fixed, add_ln, window_reverse_add_ln and add_ln_affine take their
// caps (4, 3, 3 and 2 workgroups per compute unit) for inputs where their waves
// take at most 2 tiles: -13% (add_ln), -10% (window_reverse_add_ln,
// add_ln_affine) at 32,760 rows, -10% and -4% (ln_fixed) at 48,960 and 65,520
// rows; at the model's 131,040 rows they run one tile per wave.
template <int C, Op O> constexpr int kMaxTilesPerWave = 0;
template <> constexpr int kMaxTilesPerWave<192, Op::kLn> = 2;
template <> constexpr int kMaxTilesPerWave<192, Op::kAddLn> = 2;
template <> constexpr int kMaxTilesPerWave<192, Op::kReverseAddLn> = 2;
template <> constexpr int kMaxTilesPerWave<192, Op::kAddLnAffine> = 2;
template <> constexpr int kMaxTilesPerWave<384, Op::kAddLnAffine> = 3;
template <> constexpr int kMaxTilesPerWave<384, Op::kAddNormGather> = 2;

// Inputs well beyond the model's size. The level-2 entries above keep every
// wave of a 32,760-token grid resident at once; on inputs several times that,
// their one-tile-per-wave grids run in many generations, and other forms stream
// better. LaunchLarge<C, O> is the entry taken once the input has more than
// kLargeFromTilesPerCu<C, O> row tiles (of the width's K) per compute unit
// (0 = never). Measured at C = 384 on grids 8 x h x 45 against the entries
// above (the model's grid is 8 x 91 x 45, 16 tiles per compute unit):
//  * add_ln and window_reverse_add_ln: 4-wave workgroups, binary64 rows, the
//    pipelined loop; -6% / -10% at 65,520 tokens, -11% / -9% at 131,040, +7%
//    / +2% at 48,960 (24 tiles per compute unit), hence from 28 tiles;
//  * ln_fixed and norm_gather: the same form; -5% / -3% at 131,040, even at
//    65,520 (32 tiles per compute unit), hence from 48 tiles;
//  * the plain gather: K = 3 (4 rows per wave), one tile per wave, at most 3
//    resident 4-wave workgroups per compute unit; -8% at 131,040;
//  * ln_affine: one-wave workgroups, binary32 rows, load priority, the
//    pipelined loop; -9% at 131,040.
// At C = 768 (4 rows per tile; the patch merge's 32,760 rows are 32 tiles per
// compute unit) ln_fixed takes the 4-wave, binary64, pipelined form from 40
// tiles per compute unit: -5% at 48,960 rows and beyond, +4% at 32,760.
template <int C, Op O> struct LaunchLarge : Launch<C, O> {};
template <int C, Op O> constexpr int kLargeFromTilesPerCu = 0;
template <> struct LaunchLarge<384, Op::kAddLn> : Tuned<0, true> {};
template <> struct LaunchLarge<384, Op::kReverseAddLn> : Tuned<0, true> {};
template <> struct LaunchLarge<384, Op::kLn> : Tuned<0, true> {};
template <> struct LaunchLarge<384, Op::kNormGather> : Tuned<0, true> {};
template <> struct LaunchLarge<384, Op::kGather> : Tuned<0, false, 0, 4, double, 3, 3> {};
template <> struct LaunchLarge<384, Op::kLnAffine> : Tuned<0, true, 1, 1, float> {};
template <> constexpr int kLargeFromTilesPerCu<384, Op::kAddLn> = 28;
template <> constexpr int kLargeFromTilesPerCu<384, Op::kReverseAddLn> = 28;
template <> constexpr int kLargeFromTilesPerCu<384, Op::kLn> = 48;
template <> constexpr int kLargeFromTilesPerCu<384, Op::kNormGather> = 48;
template <> constexpr int kLargeFromTilesPerCu<384, Op::kGather> = 48;
template <> constexpr int kLargeFromTilesPerCu<384, Op::kLnAffine> = 48;
template <> struct LaunchLarge<768, Op::kLn> : Tuned<0, true> {};
template <> constexpr int kLargeFromTilesPerCu<768, Op::kLn> = 40;

// Compute units of the device, queried on first use (0 = not yet known). Only
// launch shapes depend on it (the size of a capped grid, the entry a large
// input takes), never a result: every entry of an op computes the same row
// function with the same arithmetic in the same order. A failed
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

template <int C, Op O, class L>
unsigned grid_for(int64_t rows) {
    static_assert(kChunksOk<C, O, L>, "a normalising kernel must use its width's chunk count");
    static_assert(O == Op::kGather || L::kTiles == 1, "only the plain gather takes several tiles per wave");
    static_assert(L::kTiles == 1 || L::kBlocksPerCu == 0, "a multi-tile grid is sized by its tiles, not capped");
    using T = Tile<C, kChunksOf<C, L>>;
    const int64_t tiles = (rows + T::kRowsPerWave - 1) / T::kRowsPerWave;
    const int64_t waves = (tiles + L::kTiles - 1) / L::kTiles;
    int64_t blocks = (waves + L::kWaves - 1) / L::kWaves;
    if (L::kBlocksPerCu > 0) {
        const int64_t cap = static_cast<int64_t>(compute_units()) * L::kBlocksPerCu;
        constexpr int kMax = kMaxTilesPerWave<C, O>;
        if (blocks > cap && (kMax == 0 || tiles <= static_cast<int64_t>(kMax) * cap * L::kWaves)) blocks = cap;
    }
    // A dispatch counts its work-items in 32 bits: past 2^32 of them (C = 192
    // ln_fixed on more than 2^29 rows) the grid stops at the largest size below
    // that, and the waves loop over the remaining tiles with the grid stride,
    // as on a capped grid. (A multi-tile gather has a table of fewer than 2^31
    // entries, far below that.)
    constexpr int64_t kMaxBlocks = ((int64_t{1} << 32) - 1) / (64 * L::kWaves);
    if (blocks > kMaxBlocks) blocks = kMaxBlocks;
    return static_cast<unsigned>(blocks);
}

// LDS per compute unit on gfx950 (CDNA4).
constexpr size_t kLdsPerCu = 160 * 1024;

// Dynamic LDS a workgroup of launch entry L reserves so that at most kResident
// of them fit on a compute unit (0 when the entry sets no limit). No kernel
// reads it.
template <class L>
constexpr size_t lds_reserve() {
    constexpr int k = L::kResident;
    static_assert(k == 0 || kLdsPerCu / (k + 1) + 1024 <= 64 * 1024,
                  "a reservation stays within the 64 KB a workgroup may request at launch");
    return k == 0 ? 0 : kLdsPerCu / (k + 1) + 1024;
}

template <class L>
dim3 block_of() { return dim3(64 * L::kWaves); }

template <class L> struct Use { using type = L; };

// Calls f(Use<entry>{}) with the launch entry of (C, O) for an input of `rows`
// rows (output rows for the gathers).
template <int C, Op O, class F>
hipError_t with_launch(int64_t rows, F&& f) {
    if constexpr (kLargeFromTilesPerCu<C, O> > 0) {
        constexpr int64_t kRows = Tile<C, Width<C>::K>::kRowsPerWave;
        const int64_t tiles = (rows + kRows - 1) / kRows;
        if (tiles > static_cast<int64_t>(kLargeFromTilesPerCu<C, O>) * compute_units())
            return f(Use<LaunchLarge<C, O>>{});
    }
    return f(Use<Launch<C, O>>{});
}

template <int C>
hipError_t ln_fixed_c(const void* x, void* y, int64_t rows, double eps, hipStream_t s) {
    constexpr Op O = Op::kLn;
    return with_launch<C, O>(rows, [&](auto use) {
        using L = typename decltype(use)::type;
        ln_fixed_kernel<C, Width<C>::K, typename L::H, L::kPrefetch, L::kPriority, L::kWaves, typename L::Row>
            <<<grid_for<C, O, L>(rows), block_of<L>(), lds_reserve<L>(), s>>>(
                static_cast<const chunk_t*>(x), static_cast<chunk_t*>(y), rows, eps);
        return hipGetLastError();
    });
}

template <int C>
hipError_t add_ln_c(const void* b, const void* r, void* ro, void* y, int64_t rows, double eps,
                    hipStream_t s) {
    constexpr Op O = Op::kAddLn;
    return with_launch<C, O>(rows, [&](auto use) {
        using L = typename decltype(use)::type;
        add_ln_kernel<C, Width<C>::K, typename L::H, L::kPrefetch, L::kPriority, L::kWaves, typename L::Row>
            <<<grid_for<C, O, L>(rows), block_of<L>(), lds_reserve<L>(), s>>>(
                static_cast<const chunk_t*>(b), static_cast<const chunk_t*>(r), static_cast<chunk_t*>(ro),
                static_cast<chunk_t*>(y), rows, eps);
        return hipGetLastError();
    });
}

template <int C>
hipError_t window_gather_c(const void* x, int64_t n_src, const int32_t* table, int64_t n_out, void* out,
                           hipStream_t s) {
    constexpr Op O = Op::kGather;
    return with_launch<C, O>(n_out, [&](auto use) {
        using L = typename decltype(use)::type;
        if constexpr (L::kTiles > 1) {
            gather_tiles_kernel<C, kChunksOf<C, L>, typename L::H, L::kTiles, L::kWaves, L::kPriority>
                <<<grid_for<C, O, L>(n_out), block_of<L>(), lds_reserve<L>(), s>>>(
                    static_cast<const chunk_t*>(x), n_src, table, n_out, static_cast<chunk_t*>(out));
        } else {
            gather_kernel<C, kChunksOf<C, L>, false, typename L::H, L::kPrefetch, L::kWaves, L::kPriority,
                          typename L::Row>
                <<<grid_for<C, O, L>(n_out), block_of<L>(), lds_reserve<L>(), s>>>(
                    static_cast<const chunk_t*>(x), n_src, table, n_out, static_cast<chunk_t*>(out), 0.0);
        }
        return hipGetLastError();
    });
}

template <int C>
hipError_t norm_gather_c(const void* x, int64_t n_src, const int32_t* table, int64_t n_out, double eps,
                         void* out, hipStream_t s) {
    constexpr Op O = Op::kNormGather;
    return with_launch<C, O>(n_out, [&](auto use) {
        using L = typename decltype(use)::type;
        gather_kernel<C, Width<C>::K, true, typename L::H, L::kPrefetch, L::kWaves, L::kPriority,
                      typename L::Row>
            <<<grid_for<C, O, L>(n_out), block_of<L>(), lds_reserve<L>(), s>>>(
                static_cast<const chunk_t*>(x), n_src, table, n_out, static_cast<chunk_t*>(out), eps);
        return hipGetLastError();
    });
}

template <int C>
hipError_t reverse_add_ln_c(const void* win, int64_t n_win, const int32_t* idx, const void* r, void* ro,
                            void* y, int64_t rows, double eps, hipStream_t s) {
    constexpr Op O = Op::kReverseAddLn;
    return with_launch<C, O>(rows, [&](auto use) {
        using L = typename decltype(use)::type;
        reverse_add_ln_kernel<C, Width<C>::K, typename L::H, L::kPrefetch, L::kPriority, L::kWaves,
                              typename L::Row>
            <<<grid_for<C, O, L>(rows), block_of<L>(), lds_reserve<L>(), s>>>(
                static_cast<const chunk_t*>(win), n_win, idx, static_cast<const chunk_t*>(r),
                static_cast<chunk_t*>(ro), static_cast<chunk_t*>(y), rows, eps);
        return hipGetLastError();
    });
}

template <int C>
hipError_t add_norm_gather_c(const void* b, const void* r, void* ro, int64_t n_src, const int32_t* table,
                             int64_t n_out, double eps, void* out, hipStream_t s) {
    constexpr Op O = Op::kAddNormGather;
    return with_launch<C, O>(n_out, [&](auto use) {
        using L = typename decltype(use)::type;
        add_norm_gather_kernel<C, Width<C>::K, typename L::H, L::kPrefetch, L::kPriority, L::kWaves,
                               typename L::Row>
            <<<grid_for<C, O, L>(n_out), block_of<L>(), lds_reserve<L>(), s>>>(
                static_cast<const chunk_t*>(b), static_cast<const chunk_t*>(r), static_cast<chunk_t*>(ro),
                n_src, table, n_out, static_cast<chunk_t*>(out), eps);
        return hipGetLastError();
    });
}

template <int C>
hipError_t ln_affine_c(const void* x, const void* g, const void* b, void* y, int64_t rows, double eps,
                       hipStream_t s) {
    constexpr Op O = Op::kLnAffine;
    return with_launch<C, O>(rows, [&](auto use) {
        using L = typename decltype(use)::type;
        ln_affine_kernel<C, Width<C>::K, typename L::H, L::kPrefetch, L::kPriority, L::kWaves, typename L::Row,
                         Width<C>::kWideParams, L::kStage>
            <<<grid_for<C, O, L>(rows), block_of<L>(), lds_reserve<L>(), s>>>(
                static_cast<const chunk_t*>(x), static_cast<const chunk_t*>(g), static_cast<const chunk_t*>(b),
                static_cast<chunk_t*>(y), rows, eps);
        return hipGetLastError();
    });
}

template <int C>
hipError_t add_ln_affine_c(const void* br, const void* r, const void* g, const void* b, void* ro, void* y,
                           int64_t rows, double eps, hipStream_t s) {
    constexpr Op O = Op::kAddLnAffine;
    return with_launch<C, O>(rows, [&](auto use) {
        using L = typename decltype(use)::type;
        add_ln_affine_kernel<C, Width<C>::K, typename L::H, L::kPrefetch, L::kPriority, L::kWaves,
                             typename L::Row, Width<C>::kWideParams, L::kStage>
            <<<grid_for<C, O, L>(rows), block_of<L>(), lds_reserve<L>(), s>>>(
                static_cast<const chunk_t*>(br), static_cast<const chunk_t*>(r), static_cast<const chunk_t*>(g),
                static_cast<const chunk_t*>(b), static_cast<chunk_t*>(ro), static_cast<chunk_t*>(y), rows, eps);
        return hipGetLastError();
    });
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
    return by_width(C, [&](auto c) { return window_gather_c<decltype(c)::value>(x, n_src, table, n_out, out, stream); });
}

hipError_t launch_norm_gather(const void* x, int64_t n_src, int32_t C, const int32_t* table,
                              int64_t n_out, double eps, void* out, hipStream_t stream) {
    return by_width(C, [&](auto c) { return norm_gather_c<decltype(c)::value>(x, n_src, table, n_out, eps, out, stream); });
}

hipError_t launch_window_inverse(const WindowGeometry& g, int32_t* inverse, hipStream_t stream) {
    const int64_t tokens = static_cast<int64_t>(g.Z) * g.H * g.W;
    const unsigned grid = static_cast<unsigned>((tokens + kBlock - 1) / kBlock);
    window_inverse_kernel<<<grid, kBlock, 0, stream>>>(g, inverse);
    return hipGetLastError();
}

hipError_t launch_reverse_add_ln(const void* win, int64_t n_win, const int32_t* inverse,
                                 const void* residual, void* residual_out, void* y, int64_t rows,
                                 int32_t C, double eps, hipStream_t stream) {
    return by_width(C, [&](auto c) { return reverse_add_ln_c<decltype(c)::value>(win, n_win, inverse, residual, residual_out, y, rows, eps, stream); });
}

hipError_t launch_add_norm_gather(const void* branch, const void* residual, void* residual_out,
                                  int64_t n_src, int32_t C, const int32_t* table, int64_t n_out,
                                  double eps, void* out, hipStream_t stream) {
    return by_width(C, [&](auto c) { return add_norm_gather_c<decltype(c)::value>(branch, residual, residual_out, n_src, table, n_out, eps, out, stream); });
}

hipError_t launch_ln_affine(const void* x, const void* gamma, const void* beta, void* y, int64_t rows,
                            int32_t C, double eps, hipStream_t stream) {
    return by_width(C, [&](auto c) { return ln_affine_c<decltype(c)::value>(x, gamma, beta, y, rows, eps, stream); });
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
        static_cast<const f32x4_t*>(x), static_cast<const f32x4_t*>(bias),
        static_cast<f32x4_t*>(y), n4, make_fastdiv(static_cast<uint32_t>(cols / 4)));
    return hipGetLastError();
}

}  // namespace lwg
