// rht.hip -- randomized Hadamard transform pre/post-processing for THC
// ("THC: Accelerating Distributed Deep Learning Using Tensor Homomorphic
// Compression", section 5): RHT(x) = H D x / sqrt(d), RHT^-1(y) = D H y /
// sqrt(d) on blocks of d = 2^k coordinates, the per-block norms, the
// norm-based range M = t_p max_i ||x_i|| / sqrt(d), m = -M, and truncation.
//
// The transform is the textbook radix-2 one: stage s = 0 .. k-1 turns every
// pair (i, i + 2^s), bit s of i clear, into (a + b, a - b) in binary32, and
// the result is scaled by fl32(1/sqrt(d)) at the end. Two passes keep every
// stage in LDS:
//  * tile pass: a workgroup loads 4096 consecutive coordinates (16 KiB;
//    several whole blocks when d < 4096) and runs stages 0 .. log2(T) - 1,
//    T = min(d, 4096);
//  * cross pass (d > T only): a workgroup loads a G x W sub-matrix of one
//    block (G = d / T rows spaced T apart, W = 4096 / G consecutive
//    columns) and runs the remaining stages along the rows.
// Each stage pairs the same elements in the same order as the plain loop,
// so the output is bit-for-bit that loop's.
//
// The Rademacher signs come from Philox4x32-10: key (seed), counter
// (q mod 2^32, q >> 32, 0x52485400, 0) with q = e / 128; coordinate e takes
// bit e mod 32 of output word (e / 32) mod 4, a set bit meaning -1. A
// workgroup first computes the Philox blocks it needs into LDS.
#include <cmath>

#include "common.hpp"
#include "philox.hpp"

namespace ga {
namespace {

constexpr int kTile = 4096;                 // coordinates per LDS tile
constexpr int kMaxRows = 1024;              // cross-pass rows: d <= kTile * kMaxRows = 2^22
constexpr uint32_t kSignDomain = 0x52485400u;

__device__ __forceinline__ float load_coord(const void* x, int64_t e, int64_t N, ga_dtype dt) {
    if (e >= N) return 0.0f;                 // zero padding to a whole block
    if (dt == GA_BF16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(x)[e] << 16);
    return static_cast<const float*>(x)[e];
}

// Butterflies on pairs (i, i + h), bit h of i clear, for h = h0, 2 h0, ...
// while h < h1, over the n coordinates in LDS; a barrier after each stage.
__device__ __forceinline__ void lds_stages(float* s, int n, int h0, int h1) {
    for (int h = h0; h < h1; h <<= 1) {
        for (int q = threadIdx.x; q < n / 2; q += kThreads) {
            const int i = ((q & ~(h - 1)) << 1) | (q & (h - 1));
            const float a = s[i], b = s[i + h];
            s[i] = a + b;
            s[i + h] = a - b;
        }
        __syncthreads();
    }
}

// Philox blocks q0 .. q0 + nq - 1 of the sign stream into LDS (nq <= 4 kThreads
// words handled: each thread computes at most one block).
__device__ __forceinline__ void sign_blocks(uint32_t* words, int64_t q0, int nq, uint32_t k0,
                                            uint32_t k1) {
    for (int t = threadIdx.x; t < nq; t += kThreads) {
        const uint64_t q = (uint64_t)(q0 + t);
        const Philox4 r = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), kSignDomain, 0u, k0, k1);
        words[4 * t + 0] = r.v[0];
        words[4 * t + 1] = r.v[1];
        words[4 * t + 2] = r.v[2];
        words[4 * t + 3] = r.v[3];
    }
}

__device__ __forceinline__ float sign_of(const uint32_t* words, int64_t q0, int64_t e) {
    const uint32_t w = words[4 * ((e >> 7) - q0) + ((e >> 5) & 3)];
    return ((w >> (e & 31)) & 1u) ? -1.0f : 1.0f;
}

__device__ __forceinline__ float clamp_to(float v, const float* mM, int64_t p) {
    const float m = mM[2 * p], M = mM[2 * p + 1];
    return v < m ? m : (v > M ? M : v);
}

// ---------------------------------------------------------------- forward

// Tile pass over n = min(kTile, Np - e0) consecutive coordinates (a whole
// number of blocks when d < kTile, one tile of a block otherwise): stages
// h = 1 .. T/2 with T = min(d, kTile). FINAL (d <= kTile): scale, clamp when
// mM is given, store; else store the partial transform for the cross pass.
template <ga_dtype DT, bool FINAL>
__global__ __launch_bounds__(kThreads) void rht_fwd_tile_kernel(PtrTable x, PtrTable y, int64_t N,
                                                                int64_t Np, int T, int64_t d,
                                                                uint32_t k0, uint32_t k1, float c,
                                                                const float* __restrict__ mM) {
    __shared__ float s[kTile];
    __shared__ uint32_t words[4 * (kTile / 128)];
    const int w = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * kTile;
    const int n = (int)min((int64_t)kTile, Np - e0);
    const int64_t q0 = e0 >> 7;
    sign_blocks(words, q0, (n + 127) / 128, k0, k1);
    __syncthreads();
    const void* xw = x.p[w];
    for (int i = threadIdx.x; i < n; i += kThreads)
        s[i] = sign_of(words, q0, e0 + i) * load_coord(xw, e0 + i, N, DT);
    __syncthreads();
    lds_stages(s, n, 1, T);
    float* yw = static_cast<float*>(y.p[w]);
    for (int i = threadIdx.x; i < n; i += kThreads) {
        float v = s[i];
        if (FINAL) {
            v = v * c;
            if (mM) v = clamp_to(v, mM, (e0 + i) / d);
        }
        yw[e0 + i] = v;
    }
}

// Cross pass: rows j = 0 .. G-1 of block b at stride T, columns c0 .. c0+W-1.
// FWD: scale and clamp; else (inverse): scale, apply the signs, write out.
template <bool FWD, ga_dtype OUT>
__global__ __launch_bounds__(kThreads) void rht_cross_kernel(PtrTable y, PtrTable out, int64_t N,
                                                             int T, int64_t d, int G, int W,
                                                             uint32_t k0, uint32_t k1, float c,
                                                             const float* __restrict__ mM) {
    __shared__ float s[kTile];
    // inverse only: the Philox blocks of every (row, 128-column group)
    __shared__ uint32_t words[FWD ? 1 : 4 * kMaxRows];
    const int w = blockIdx.y;
    const int64_t cols_per_block = T / W;
    const int64_t b = blockIdx.x / cols_per_block;
    const int64_t c0 = (blockIdx.x % cols_per_block) * W;
    const int64_t base = b * d + c0;           // a multiple of min(W, 128)
    float* yw = static_cast<float*>(y.p[w]);
    const int n = G * W;
    const int R = W >= 128 ? W / 128 : 1;      // sign blocks per row
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int j = i / W, col = i % W;
        s[i] = yw[base + (int64_t)j * T + col];
    }
    if (!FWD) {
        for (int t = threadIdx.x; t < G * R; t += kThreads) {
            const int j = t / R, gi = t % R;
            const uint64_t q = (uint64_t)(((base + (int64_t)j * T) >> 7) + gi);
            const Philox4 r = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), kSignDomain, 0u, k0, k1);
            words[4 * t + 0] = r.v[0];
            words[4 * t + 1] = r.v[1];
            words[4 * t + 2] = r.v[2];
            words[4 * t + 3] = r.v[3];
        }
    }
    __syncthreads();
    lds_stages(s, n, W, n);
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int j = i / W, col = i % W;
        const int64_t e = base + (int64_t)j * T + col;
        const float v = s[i] * c;
        if (FWD) {
            yw[e] = mM ? clamp_to(v, mM, b) : v;
        } else if (e < N) {
            const uint32_t wd = words[4 * (j * R + (col >> 7)) + ((e >> 5) & 3)];
            const float r = ((wd >> (e & 31)) & 1u) ? -v : v;
            if (OUT == GA_F32) static_cast<float*>(out.p[w])[e] = r;
            else static_cast<uint16_t*>(out.p[w])[e] = (uint16_t)f32_to_bf16_rne(r);
        }
    }
}

// ---------------------------------------------------------------- inverse

template <bool FINAL, ga_dtype OUT>
__global__ __launch_bounds__(kThreads) void rht_inv_tile_kernel(float* y, void* out, int64_t N,
                                                                int64_t Np, int T, uint32_t k0,
                                                                uint32_t k1, float c) {
    __shared__ float s[kTile];
    __shared__ uint32_t words[FINAL ? 4 * (kTile / 128) : 1];
    const int64_t e0 = (int64_t)blockIdx.x * kTile;
    const int n = (int)min((int64_t)kTile, Np - e0);
    const int64_t q0 = e0 >> 7;
    if (FINAL) sign_blocks(words, q0, (n + 127) / 128, k0, k1);
    for (int i = threadIdx.x; i < n; i += kThreads) s[i] = y[e0 + i];
    __syncthreads();
    lds_stages(s, n, 1, T);
    for (int i = threadIdx.x; i < n; i += kThreads) {
        const int64_t e = e0 + i;
        if (!FINAL) {
            y[e] = s[i];
        } else if (e < N) {
            const float r = sign_of(words, q0, e) * (s[i] * c);
            if (OUT == GA_F32) static_cast<float*>(out)[e] = r;
            else static_cast<uint16_t*>(out)[e] = (uint16_t)f32_to_bf16_rne(r);
        }
    }
}

// ---------------------------------------------------------------- norms and range

template <ga_dtype DT>
__global__ __launch_bounds__(kThreads) void rht_sumsq_kernel(PtrTable x, int64_t N, int64_t d,
                                                             int64_t nblk, double* sumsq) {
    const int w = blockIdx.y;
    const int64_t b = blockIdx.x;
    const int64_t lo = b * d, hi = min(lo + d, N);
    double acc = 0.0;
    for (int64_t e = lo + threadIdx.x; e < hi; e += kThreads) {
        const double v = (double)load_coord(x.p[w], e, N, DT);
        acc += v * v;
    }
    __shared__ double sh[kThreads / 64];
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
        for (int i = 0; i < kThreads / 64; i++) t += sh[i];
        sumsq[(int64_t)w * nblk + b] = t;
    }
}

__global__ __launch_bounds__(kThreads) void rht_range_kernel(const double* sumsq, int P, int64_t nblk,
                                                             double d, double t_p, float* mM) {
    const int64_t p = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (p >= nblk) return;
    double mx = 0.0;
    for (int i = 0; i < P; i++) mx = fmax(mx, sumsq[(int64_t)i * nblk + p]);
    const float M = (float)(t_p * sqrt(mx) / sqrt(d));
    mM[2 * p] = -M;
    mM[2 * p + 1] = M;
}

bool pow2_block(int64_t d) { return d >= 2 && d <= (int64_t)kTile * kMaxRows && (d & (d - 1)) == 0; }

// Tile size and cross-pass shape for a block length d.
struct Shape {
    int T, G, W;
};
Shape shape_of(int64_t d) {
    Shape s;
    s.T = (int)(d < kTile ? d : kTile);
    s.G = (int)(d / s.T);
    s.W = s.G > 1 ? kTile / s.G : 0;
    if (s.G > 1 && s.W > s.T) s.W = s.T;
    return s;
}

float inv_sqrt_d(int64_t d) { return (float)(1.0 / std::sqrt((double)d)); }

}  // namespace
}  // namespace ga

using namespace ga;

extern "C" ga_status thc_rht_sumsq(const void* const* bufs, int32_t P, int64_t N, ga_dtype dt,
                                   int64_t d, double* d_sumsq, void* stream) {
    const char* what = "thc_rht_sumsq";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (!pow2_block(d)) return fail(GA_EINVAL, "%s: d = %lld is not a power of two in [2, 2^22]", what, (long long)d);
    if (N < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(bufs, P, elem_size(dt), what);
    if (rc) return rc;
    if (!d_sumsq || !aligned(d_sumsq, 8)) return fail(GA_EINVAL, "%s: bad output pointer", what);
    const int64_t nblk = ceil_div(N, d);
    if (nblk > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: too many blocks", what);
    PtrTable t{};
    for (int i = 0; i < P; i++) t.p[i] = const_cast<void*>(bufs[i]);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (dt == GA_F32)
        hipLaunchKernelGGL(rht_sumsq_kernel<GA_F32>, dim3((unsigned)nblk, (unsigned)P), dim3(kThreads), 0, hs, t, N, d, nblk, d_sumsq);
    else
        hipLaunchKernelGGL(rht_sumsq_kernel<GA_BF16>, dim3((unsigned)nblk, (unsigned)P), dim3(kThreads), 0, hs, t, N, d, nblk, d_sumsq);
    return check_launch(what);
}

extern "C" ga_status thc_rht_range(const double* d_sumsq, int32_t P, int64_t nblk, int64_t d, double t_p,
                                   float* d_mM, void* stream) {
    const char* what = "thc_rht_range";
    if (!pow2_block(d)) return fail(GA_EINVAL, "%s: d = %lld is not a power of two in [2, 2^22]", what, (long long)d);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (nblk < 0 || !(t_p > 0.0) || !std::isfinite(t_p)) return fail(GA_EINVAL, "%s: bad nblk or t_p", what);
    if (nblk == 0) return GA_OK;
    if (!d_sumsq || !d_mM || !aligned(d_sumsq, 8) || !aligned(d_mM, 8))
        return fail(GA_EINVAL, "%s: bad pointer", what);
    hipLaunchKernelGGL(rht_range_kernel, dim3((unsigned)ceil_div(nblk, kThreads)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), d_sumsq, P, nblk, (double)d, t_p, d_mM);
    return check_launch(what);
}

extern "C" ga_status thc_rht_forward(const void* const* bufs, int32_t P, int64_t N, ga_dtype dt,
                                     int64_t d, uint64_t seed, const float* d_mM, float* const* y,
                                     void* stream) {
    const char* what = "thc_rht_forward";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (!pow2_block(d)) return fail(GA_EINVAL, "%s: d = %lld is not a power of two in [2, 2^22]", what, (long long)d);
    if (N < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(bufs, P, elem_size(dt), what);
    if (rc) return rc;
    if ((rc = check_workers(reinterpret_cast<const void* const*>(y), P, 4, what))) return rc;
    if (d_mM && !aligned(d_mM, 8)) return fail(GA_EINVAL, "%s: misaligned range", what);
    const int64_t Np = ceil_div(N, d) * d;
    const Shape sh = shape_of(d);
    const int64_t tiles = ceil_div(Np, kTile);
    if (tiles > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: too many tiles", what);
    PtrTable tx{}, ty{};
    for (int i = 0; i < P; i++) {
        tx.p[i] = const_cast<void*>(bufs[i]);
        ty.p[i] = y[i];
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const float c = inv_sqrt_d(d);
    const dim3 g1((unsigned)tiles, (unsigned)P);
    if (sh.G == 1) {
        if (dt == GA_F32)
            hipLaunchKernelGGL((rht_fwd_tile_kernel<GA_F32, true>), g1, dim3(kThreads), 0, hs, tx, ty, N, Np, sh.T, d, k0, k1, c, d_mM);
        else
            hipLaunchKernelGGL((rht_fwd_tile_kernel<GA_BF16, true>), g1, dim3(kThreads), 0, hs, tx, ty, N, Np, sh.T, d, k0, k1, c, d_mM);
        return check_launch(what);
    }
    if (dt == GA_F32)
        hipLaunchKernelGGL((rht_fwd_tile_kernel<GA_F32, false>), g1, dim3(kThreads), 0, hs, tx, ty, N, Np, sh.T, d, k0, k1, c, d_mM);
    else
        hipLaunchKernelGGL((rht_fwd_tile_kernel<GA_BF16, false>), g1, dim3(kThreads), 0, hs, tx, ty, N, Np, sh.T, d, k0, k1, c, d_mM);
    if ((rc = check_launch(what))) return rc;
    const dim3 g2((unsigned)((Np / d) * (sh.T / sh.W)), (unsigned)P);
    hipLaunchKernelGGL((rht_cross_kernel<true, GA_F32>), g2, dim3(kThreads), 0, hs, ty, ty, Np, sh.T, d, sh.G, sh.W, k0, k1, c, d_mM);
    return check_launch(what);
}

extern "C" ga_status thc_rht_inverse(float* y, int64_t N, int64_t d, uint64_t seed, void* out,
                                     ga_dtype out_dt, void* stream) {
    const char* what = "thc_rht_inverse";
    if (!valid_dtype(out_dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)out_dt);
    if (!pow2_block(d)) return fail(GA_EINVAL, "%s: d = %lld is not a power of two in [2, 2^22]", what, (long long)d);
    if (N < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (N == 0) return GA_OK;
    if (!y || !out || !aligned(y, 4) || !aligned(out, elem_size(out_dt)))
        return fail(GA_EINVAL, "%s: null or misaligned pointer", what);
    const int64_t Np = ceil_div(N, d) * d;
    const Shape sh = shape_of(d);
    const int64_t tiles = ceil_div(Np, kTile);
    if (tiles > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: too many tiles", what);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const float c = inv_sqrt_d(d);
    ga_status rc;
    if (sh.G == 1) {
        if (out_dt == GA_F32)
            hipLaunchKernelGGL((rht_inv_tile_kernel<true, GA_F32>), dim3((unsigned)tiles), dim3(kThreads), 0, hs, y, out, N, Np, sh.T, k0, k1, c);
        else
            hipLaunchKernelGGL((rht_inv_tile_kernel<true, GA_BF16>), dim3((unsigned)tiles), dim3(kThreads), 0, hs, y, out, N, Np, sh.T, k0, k1, c);
        return check_launch(what);
    }
    hipLaunchKernelGGL((rht_inv_tile_kernel<false, GA_F32>), dim3((unsigned)tiles), dim3(kThreads), 0, hs, y, out, N, Np, sh.T, k0, k1, c);
    if ((rc = check_launch(what))) return rc;
    PtrTable ty{}, to{};
    ty.p[0] = y;
    to.p[0] = out;
    const dim3 g2((unsigned)((Np / d) * (sh.T / sh.W)), 1u);
    if (out_dt == GA_F32)
        hipLaunchKernelGGL((rht_cross_kernel<false, GA_F32>), g2, dim3(kThreads), 0, hs, ty, to, N, sh.T, d, sh.G, sh.W, k0, k1, c, (const float*)nullptr);
    else
        hipLaunchKernelGGL((rht_cross_kernel<false, GA_BF16>), g2, dim3(kThreads), 0, hs, ty, to, N, sh.T, d, sh.G, sh.W, k0, k1, c, (const float*)nullptr);
    return check_launch(what);
}
