// thc.hip -- THC uniform homomorphic compression on the GPU ("THC:
// Accelerating Distributed Deep Learning Using Tensor Homomorphic
// Compression", sections 2-4, Algorithm 1): global extremes per partition,
// unbiased stochastic quantization to b-bit indices on the shared uniform
// grid, integer aggregation of the indices (the server's only work),
// dequantization of the average, and the NMSE of the estimate.
//
// Every kernel here streams HBM once: min/max reads P N elem_bytes;
// quantize reads P N elem_bytes and writes P N b / 8; aggregate reads
// P N b / 8 and writes 4 N; dequant reads 4 N and writes N out_bytes; NMSE
// reads 2 N elem_bytes. 128-bit loads and stores on aligned buffers.
#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "philox.hpp"

namespace ga {
namespace {

__device__ __forceinline__ float load_as_f32(const void* p, int64_t e, ga_dtype dt) {
    if (dt == GA_BF16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(p)[e] << 16);
    return static_cast<const float*>(p)[e];
}

// 8 consecutive elements starting at a 16-byte aligned address (bf16), or 4
// (fp32), widened to binary32.
template <ga_dtype DT> struct Vec16;
template <> struct Vec16<GA_F32> {
    static constexpr int kElems = 4;
    __device__ static __forceinline__ void load(const void* p, int64_t v, float* f) {
        const float4 x = static_cast<const float4*>(p)[v];
        f[0] = x.x; f[1] = x.y; f[2] = x.z; f[3] = x.w;
    }
};
template <> struct Vec16<GA_BF16> {
    static constexpr int kElems = 8;
    __device__ static __forceinline__ void load(const void* p, int64_t v, float* f) {
        const uint4 r = static_cast<const uint4*>(p)[v];
        f[0] = bf16_lo(r.x); f[1] = bf16_hi(r.x); f[2] = bf16_lo(r.y); f[3] = bf16_hi(r.y);
        f[4] = bf16_lo(r.z); f[5] = bf16_hi(r.z); f[6] = bf16_lo(r.w); f[7] = bf16_hi(r.w);
    }
};

// ------------------------------------------------------------------ min/max
// Float -> uint32 key whose unsigned order is the float order (finite
// values; -0 orders just below +0), and back.
__device__ __forceinline__ uint32_t order_key(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_value(uint32_t k) {
    return __uint_as_float((k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}

__global__ __launch_bounds__(kThreads) void minmax_init_kernel(uint32_t* keys, int64_t n_part) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n_part) {
        keys[2 * i] = 0xFFFFFFFFu;
        keys[2 * i + 1] = 0u;
    }
}

__global__ __launch_bounds__(kThreads) void minmax_final_kernel(uint32_t* keys, int64_t n_part) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < n_part) {
        // "+ 0.0f" turns a negative zero into +0
        const float m = key_value(keys[2 * i]) + 0.0f;
        const float M = key_value(keys[2 * i + 1]) + 0.0f;
        keys[2 * i] = __float_as_uint(m);
        keys[2 * i + 1] = __float_as_uint(M);
    }
}

__device__ __forceinline__ float wave_min(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fminf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}

// Workgroup (p, j) scans slice j of partition p in every worker's buffer.
template <ga_dtype DT>
__global__ __launch_bounds__(kThreads) void minmax_kernel(PtrTable bufs, int P, int64_t N,
                                                          int64_t plen, int slices,
                                                          int64_t slice_len, uint32_t* keys) {
    using V = Vec16<DT>;
    constexpr int E = V::kElems;
    const int64_t p = blockIdx.x / slices;
    const int64_t j = blockIdx.x % slices;
    const int64_t p0 = p * plen;
    const int64_t pend = min(p0 + plen, N);
    const int64_t lo = p0 + j * slice_len;
    const int64_t hi = min(lo + slice_len, pend);
    if (lo >= hi) return;
    float mn = INFINITY, mx = -INFINITY;
    constexpr int es = DT == GA_BF16 ? 2 : 4;
    for (int w = 0; w < P; w++) {
        const void* x = bufs.p[w];
        // head: elements before the first 16-byte boundary
        const char* xb = static_cast<const char*>(x);
        const int64_t mis = (int64_t)(((uintptr_t)xb + (uintptr_t)(lo * es)) & 15) / es;
        const int64_t vlo = min(mis ? lo + (E - mis) : lo, hi);
        const int64_t nv = (hi - vlo) / E;
        const int64_t vhi = vlo + nv * E;
        for (int64_t e = lo + threadIdx.x; e < vlo; e += kThreads) {
            const float a = load_as_f32(x, e, DT);
            mn = fminf(mn, a);
            mx = fmaxf(mx, a);
        }
        // body: 16-byte vectors from the first aligned element, four in flight
        const void* xa = xb + vlo * es;
        int64_t v = threadIdx.x;
        for (; v + 3 * kThreads < nv; v += 4 * kThreads) {
            float f[4][E];
#pragma unroll
            for (int u = 0; u < 4; u++) V::load(xa, v + u * kThreads, f[u]);
#pragma unroll
            for (int u = 0; u < 4; u++)
#pragma unroll
                for (int i = 0; i < E; i++) {
                    mn = fminf(mn, f[u][i]);
                    mx = fmaxf(mx, f[u][i]);
                }
        }
        for (; v < nv; v += kThreads) {
            float f[E];
            V::load(xa, v, f);
#pragma unroll
            for (int i = 0; i < E; i++) {
                mn = fminf(mn, f[i]);
                mx = fmaxf(mx, f[i]);
            }
        }
        // tail
        for (int64_t e = vhi + threadIdx.x; e < hi; e += kThreads) {
            const float a = load_as_f32(x, e, DT);
            mn = fminf(mn, a);
            mx = fmaxf(mx, a);
        }
    }
    __shared__ float smn[kThreads / 64], smx[kThreads / 64];
    mn = wave_min(mn);
    mx = wave_max(mx);
    if ((threadIdx.x & 63) == 0) {
        smn[threadIdx.x >> 6] = mn;
        smx[threadIdx.x >> 6] = mx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kThreads / 64; i++) {
            mn = fminf(mn, smn[i]);
            mx = fmaxf(mx, smx[i]);
        }
        atomicMin(&keys[2 * p], order_key(mn));
        atomicMax(&keys[2 * p + 1], order_key(mx));
    }
}

// ------------------------------------------------------------------ quantize
constexpr int kQElems = 16;   // elements per thread: two Philox calls of 8 uniforms

template <int B> struct Packed;               // 16 b-bit indices
template <> struct Packed<8> { using T = uint4; };
template <> struct Packed<4> { using T = uint2; };
template <> struct Packed<2> { using T = uint32_t; };
template <> struct Packed<1> { using T = uint16_t; };

struct Grid {                // one partition's grid
    float m;
    float s;                 // L / (M - m), or 0 when M == m
};

__device__ __forceinline__ Grid grid_of(const float* mM, int64_t p, int L) {
    const float m = mM[2 * p], M = mM[2 * p + 1];
    const float range = M - m;
    return {m, range == 0.0f ? 0.0f : (float)L / range};
}

// Stochastic rounding of one value to its grid index (binary32 throughout;
// with s = 0 the index is 0).
__device__ __forceinline__ uint32_t usq_index(float a, Grid g, int L, uint32_t r16) {
    const float u = (a - g.m) * g.s;
    const float z0 = fminf(floorf(u), (float)(L - 1));
    const float f = u - z0;
    const bool up = (float)(2u * r16 + 1u) < f * 131072.0f;
    return (uint32_t)z0 + (up ? 1u : 0u);
}

template <ga_dtype DT, int B>
__global__ __launch_bounds__(kThreads) void usq_quantize_kernel(PtrTable bufs, PtrTable packed,
                                                                int worker0, int64_t N, int64_t plen,
                                                                const float* __restrict__ mM,
                                                                uint32_t k0, uint32_t k1,
                                                                int vec_ok) {
    constexpr int L = (1 << B) - 1;
    const int slot = blockIdx.y;
    const int64_t e0 = thread_base(kQElems);
    if (e0 >= N) return;
    const void* x = bufs.p[slot];
    uint8_t* out = static_cast<uint8_t*>(packed.p[slot]);
    const bool full = e0 + kQElems <= N;

    float a[kQElems];
    if (full && vec_ok) {
        using V = Vec16<DT>;
#pragma unroll
        for (int i = 0; i < kQElems / V::kElems; i++) V::load(x, e0 / V::kElems + i, a + i * V::kElems);
    } else {
#pragma unroll
        for (int i = 0; i < kQElems; i++) a[i] = (e0 + i < N) ? load_as_f32(x, e0 + i, DT) : 0.0f;
    }

    // counter (g mod 2^32, g >> 32, worker, 0) for g = e / 8
    const uint64_t g = (uint64_t)e0 >> 3;
    const uint32_t wid = (uint32_t)(worker0 + slot);
    const Philox4 r0 = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), wid, 0u, k0, k1);
    const Philox4 r1 = philox4x32_10((uint32_t)(g + 1), (uint32_t)((g + 1) >> 32), wid, 0u, k0, k1);

    uint32_t z[kQElems];
    if (plen % kQElems == 0) {
        const Grid gr = grid_of(mM, e0 / plen, L);
#pragma unroll
        for (int i = 0; i < kQElems; i++) {
            const Philox4& r = i < 8 ? r0 : r1;
            const int j = i & 7;
            const uint32_t r16 = (r.v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            z[i] = usq_index(a[i], gr, L, r16);
        }
    } else {
#pragma unroll
        for (int i = 0; i < kQElems; i++) {
            const Grid gr = grid_of(mM, min(e0 + i, N - 1) / plen, L);
            const Philox4& r = i < 8 ? r0 : r1;
            const int j = i & 7;
            const uint32_t r16 = (r.v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
            z[i] = usq_index(a[i], gr, L, r16);
        }
    }
    if (!full) {
#pragma unroll
        for (int i = 0; i < kQElems; i++)
            if (e0 + i >= N) z[i] = 0;
    }

    // pack least significant bits first: 16 B bits = 2 B bytes
    uint32_t words[B / 2 > 0 ? B / 2 : 1];
    if (B == 1) {
        uint32_t acc = 0;
#pragma unroll
        for (int i = 0; i < 16; i++) acc |= z[i] << i;
        words[0] = acc;
    } else {
        constexpr int per_word = 32 / B;
#pragma unroll
        for (int q = 0; q < (B / 2 > 0 ? B / 2 : 1); q++) {
            uint32_t acc = 0;
#pragma unroll
            for (int i = 0; i < per_word; i++) acc |= z[q * per_word + i] << (i * B);
            words[q] = acc;
        }
    }
    const int64_t byte0 = e0 / 8 * B;          // e0 is a multiple of 16
    if (full && vec_ok) {
        typename Packed<B>::T v;
        __builtin_memcpy(&v, words, sizeof v);
        *reinterpret_cast<typename Packed<B>::T*>(out + byte0) = v;
    } else {
        const int64_t nbytes = (N * B + 7) / 8;
        const uint8_t* bytes = reinterpret_cast<const uint8_t*>(words);
        for (int i = 0; i < 2 * B; i++)
            if (byte0 + i < nbytes) out[byte0 + i] = bytes[i];
    }
}

// ------------------------------------------------------------------ aggregate
// Each thread sums WB bytes of every worker. Indices are summed as pairs in
// 16-bit lanes of 32-bit registers (at most 64 * 255 = 16320 per lane, no
// carry between lanes): lane pair g of a word collects elements g and
// g + 16 / B of that word.
template <int B>
__global__ __launch_bounds__(kThreads) void int_aggregate_kernel(PtrTable packed, int P, int64_t N,
                                                                 int64_t nbytes,
                                                                 int32_t* __restrict__ sum,
                                                                 int vec_ok) {
    constexpr int WB = B >= 4 ? 16 : (B == 2 ? 8 : 4);   // bytes per worker per thread
    constexpr int NW = WB / 4;                           // words per worker
    constexpr int EPW = 32 / B;                          // elements per word
    constexpr int G = 16 / B;                            // lane pairs per word
    constexpr uint32_t LM = (1u << B) - 1u;
    constexpr uint32_t MASK = LM | (LM << 16);
    const int64_t byte0 = ((int64_t)blockIdx.x * kThreads + threadIdx.x) * WB;
    if (byte0 >= nbytes) return;
    const int64_t e0 = byte0 * 8 / B;
    const bool full = vec_ok && byte0 + WB <= nbytes;

    uint32_t acc[NW][G];
#pragma unroll
    for (int q = 0; q < NW; q++)
#pragma unroll
        for (int g = 0; g < G; g++) acc[q][g] = 0;

    constexpr int kBatch = 8;
    for (int i0 = 0; i0 < P; i0 += kBatch) {
        uint32_t w[kBatch][NW];
#pragma unroll
        for (int k = 0; k < kBatch; k++) {
            if (i0 + k < P) {
                const uint8_t* src = static_cast<const uint8_t*>(packed.p[i0 + k]) + byte0;
                if (full) {
                    if constexpr (NW == 4) {
                        const uint4 t = *reinterpret_cast<const uint4*>(src);
                        w[k][0] = t.x; w[k][1] = t.y; w[k][2] = t.z; w[k][3] = t.w;
                    } else if constexpr (NW == 2) {
                        const uint2 t = *reinterpret_cast<const uint2*>(src);
                        w[k][0] = t.x; w[k][1] = t.y;
                    } else {
                        w[k][0] = *reinterpret_cast<const uint32_t*>(src);
                    }
                } else {
#pragma unroll
                    for (int q = 0; q < NW; q++) {
                        uint32_t v = 0;
#pragma unroll
                        for (int c = 0; c < 4; c++)
                            if (byte0 + q * 4 + c < nbytes) v |= (uint32_t)src[q * 4 + c] << (8 * c);
                        w[k][q] = v;
                    }
                }
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; k++) {
            if (i0 + k < P) {
#pragma unroll
                for (int q = 0; q < NW; q++)
#pragma unroll
                    for (int g = 0; g < G; g++) acc[q][g] += (w[k][q] >> (g * B)) & MASK;
            }
        }
    }

    // element e0 + q * EPW + t: t < G in the low lane of acc[q][t], else the
    // high lane of acc[q][t - G]
    int32_t outv[NW * EPW];
#pragma unroll
    for (int q = 0; q < NW; q++)
#pragma unroll
        for (int t = 0; t < EPW; t++)
            outv[q * EPW + t] = (int32_t)(t < G ? (acc[q][t] & 0xFFFFu) : (acc[q][t - G] >> 16));

    if (full && e0 + NW * EPW <= N) {
        int4* dst = reinterpret_cast<int4*>(sum + e0);
#pragma unroll
        for (int i = 0; i < NW * EPW / 4; i++)
            dst[i] = make_int4(outv[4 * i], outv[4 * i + 1], outv[4 * i + 2], outv[4 * i + 3]);
    } else {
#pragma unroll
        for (int i = 0; i < NW * EPW; i++)
            if (e0 + i < N) sum[e0 + i] = outv[i];
    }
}

// ------------------------------------------------------------------ dequant
constexpr int kDElems = 8;

template <ga_dtype OUT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const int32_t* __restrict__ S, int64_t N,
                                                           int64_t plen, const float* __restrict__ mM,
                                                           int L, int pow2, float pf, float recip,
                                                           void* out, int vec_ok) {
    const int64_t e0 = thread_base(kDElems);
    if (e0 >= N) return;
    const bool full = vec_ok && e0 + kDElems <= N;
    int32_t s[kDElems];
    if (full) {
        const int4 a = reinterpret_cast<const int4*>(S + e0)[0];
        const int4 b = reinterpret_cast<const int4*>(S + e0)[1];
        s[0] = a.x; s[1] = a.y; s[2] = a.z; s[3] = a.w;
        s[4] = b.x; s[5] = b.y; s[6] = b.z; s[7] = b.w;
    } else {
#pragma unroll
        for (int i = 0; i < kDElems; i++) s[i] = e0 + i < N ? S[e0 + i] : 0;
    }
    float v[kDElems];
#pragma unroll
    for (int i = 0; i < kDElems; i++) {
        const int64_t p = (plen % kDElems == 0 ? e0 : min(e0 + i, N - 1)) / plen;
        const float m = mM[2 * p], M = mM[2 * p + 1];
        const float range = M - m;
        const float delta = range / (float)L;
        const float avg_index = pow2 ? (float)s[i] * recip : (float)s[i] / pf;
        v[i] = range != 0.0f ? m + avg_index * delta : m;
    }
    if (OUT == GA_F32) {
        float* o = static_cast<float*>(out);
        if (full) {
            reinterpret_cast<float4*>(o + e0)[0] = make_float4(v[0], v[1], v[2], v[3]);
            reinterpret_cast<float4*>(o + e0)[1] = make_float4(v[4], v[5], v[6], v[7]);
        } else {
            for (int i = 0; i < kDElems; i++)
                if (e0 + i < N) o[e0 + i] = v[i];
        }
    } else {
        uint16_t* o = static_cast<uint16_t*>(out);
        if (full) {
            reinterpret_cast<uint4*>(o + e0)[0] =
                make_uint4(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]),
                           pack_bf16x2(v[4], v[5]), pack_bf16x2(v[6], v[7]));
        } else {
            for (int i = 0; i < kDElems; i++)
                if (e0 + i < N) o[e0 + i] = (uint16_t)f32_to_bf16_rne(v[i]);
        }
    }
}

// ------------------------------------------------------------------ NMSE
constexpr int kNmseBlocks = 1024;

__device__ __forceinline__ double block_sum(double v, double* sh) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = v;
    __syncthreads();
    double t = 0.0;
    if (threadIdx.x == 0)
        for (int i = 0; i < kThreads / 64; i++) t += sh[i];
    __syncthreads();
    return t;
}

template <ga_dtype DT>
__global__ __launch_bounds__(kThreads) void nmse_partial_kernel(const void* x, const void* xh,
                                                                int64_t N, double* ws, int vec_ok) {
    using V = Vec16<DT>;
    constexpr int E = V::kElems;
    double num = 0.0, den = 0.0;
    const int64_t nvec = vec_ok ? N / E : 0;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t v = (int64_t)blockIdx.x * kThreads + threadIdx.x; v < nvec; v += stride) {
        float a[E], h[E];
        V::load(x, v, a);
        V::load(xh, v, h);
#pragma unroll
        for (int i = 0; i < E; i++) {
            const double d = (double)a[i] - (double)h[i];
            num += d * d;
            den += (double)a[i] * (double)a[i];
        }
    }
    for (int64_t e = nvec * E + (int64_t)blockIdx.x * kThreads + threadIdx.x; e < N; e += stride) {
        const double a = load_as_f32(x, e, DT), h = load_as_f32(xh, e, DT);
        num += (a - h) * (a - h);
        den += a * a;
    }
    __shared__ double sh[kThreads / 64];
    num = block_sum(num, sh);
    den = block_sum(den, sh);
    if (threadIdx.x == 0) {
        ws[2 * blockIdx.x] = num;
        ws[2 * blockIdx.x + 1] = den;
    }
}

__global__ __launch_bounds__(kThreads) void nmse_final_kernel(const double* ws, int nblk,
                                                              double* out) {
    double num = 0.0, den = 0.0;
    for (int i = threadIdx.x; i < nblk; i += kThreads) {
        num += ws[2 * i];
        den += ws[2 * i + 1];
    }
    __shared__ double sh[kThreads / 64];
    num = block_sum(num, sh);
    den = block_sum(den, sh);
    if (threadIdx.x == 0) {
        out[0] = num;
        out[1] = den;
        out[2] = den != 0.0 ? num / den : (num == 0.0 ? 0.0 : INFINITY);
    }
}

unsigned blocks_for(int64_t items, int per_thread) {
    return (unsigned)ceil_div(items, (int64_t)kThreads * per_thread);
}

bool valid_bits(int b) { return b == 1 || b == 2 || b == 4 || b == 8; }

}  // namespace
}  // namespace ga

using namespace ga;

extern "C" ga_status thc_minmax(const void* const* bufs, int32_t P, int64_t N, ga_dtype dt,
                                int64_t part_elems, float* d_mM, void* stream) {
    const char* what = "thc_minmax";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (N < 0 || part_elems < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(bufs, P, elem_size(dt), what);
    if (rc) return rc;
    if (!d_mM || !aligned(d_mM, 8)) return fail(GA_EINVAL, "%s: bad output pointer", what);
    const int64_t plen = part_elems > 0 ? part_elems : N;
    const int64_t n_part = n_partitions(N, part_elems);
    // ~4096 workgroups in total, slices of at least 4096 elements, a
    // multiple of 64 elements so aligned partitions keep aligned slices
    int64_t slices = std::max<int64_t>(1, std::min<int64_t>(ceil_div(plen, 4096), ceil_div(4096, n_part)));
    int64_t slice_len = ceil_div(ceil_div(plen, slices), 64) * 64;
    slices = ceil_div(plen, slice_len);
    if (n_part * slices > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: too many partitions", what);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    uint32_t* keys = reinterpret_cast<uint32_t*>(d_mM);
    PtrTable t{};
    for (int i = 0; i < P; i++) t.p[i] = const_cast<void*>(bufs[i]);
    hipLaunchKernelGGL(minmax_init_kernel, dim3(blocks_for(n_part, 1)), dim3(kThreads), 0, hs, keys, n_part);
    if ((rc = check_launch(what))) return rc;
    const dim3 grid((unsigned)(n_part * slices));
    if (dt == GA_F32)
        hipLaunchKernelGGL(minmax_kernel<GA_F32>, grid, dim3(kThreads), 0, hs, t, P, N, plen, (int)slices, slice_len, keys);
    else
        hipLaunchKernelGGL(minmax_kernel<GA_BF16>, grid, dim3(kThreads), 0, hs, t, P, N, plen, (int)slices, slice_len, keys);
    if ((rc = check_launch(what))) return rc;
    hipLaunchKernelGGL(minmax_final_kernel, dim3(blocks_for(n_part, 1)), dim3(kThreads), 0, hs, keys, n_part);
    return check_launch(what);
}

extern "C" ga_status thc_usq_quantize(const void* const* bufs, int32_t P, int32_t worker0, int64_t N,
                                      ga_dtype dt, int64_t part_elems, const float* d_mM, int32_t b,
                                      uint64_t seed, uint8_t* const* packed, void* stream) {
    const char* what = "thc_usq_quantize";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (!valid_bits(b)) return fail(GA_EINVAL, "%s: b = %d is not 1, 2, 4 or 8", what, b);
    if (N < 0 || part_elems < 0 || worker0 < 0) return fail(GA_EINVAL, "%s: negative argument", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(bufs, P, elem_size(dt), what);
    if (rc) return rc;
    if ((rc = check_workers(reinterpret_cast<const void* const*>(packed), P, 1, what))) return rc;
    if (!d_mM || !aligned(d_mM, 4)) return fail(GA_EINVAL, "%s: bad grid pointer", what);
    const int64_t plen = part_elems > 0 ? part_elems : N;
    int vec_ok = 1;
    PtrTable tx{}, tp{};
    for (int i = 0; i < P; i++) {
        tx.p[i] = const_cast<void*>(bufs[i]);
        tp.p[i] = packed[i];
        vec_ok &= aligned(bufs[i], 16) && aligned(packed[i], 16);
    }
    const int64_t blocks = ceil_div(N, (int64_t)kThreads * kQElems);
    if (blocks > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: N too large", what);
    const dim3 grid((unsigned)blocks, (unsigned)P);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
#define GA_Q(DT, B)                                                                                  \
    hipLaunchKernelGGL((usq_quantize_kernel<DT, B>), grid, dim3(kThreads), 0, hs, tx, tp, worker0, N, \
                       plen, d_mM, k0, k1, vec_ok)
    if (dt == GA_F32) {
        switch (b) {
            case 1: GA_Q(GA_F32, 1); break;
            case 2: GA_Q(GA_F32, 2); break;
            case 4: GA_Q(GA_F32, 4); break;
            default: GA_Q(GA_F32, 8); break;
        }
    } else {
        switch (b) {
            case 1: GA_Q(GA_BF16, 1); break;
            case 2: GA_Q(GA_BF16, 2); break;
            case 4: GA_Q(GA_BF16, 4); break;
            default: GA_Q(GA_BF16, 8); break;
        }
    }
#undef GA_Q
    return check_launch(what);
}

extern "C" ga_status thc_int_aggregate(const uint8_t* const* packed, int32_t P, int64_t N, int32_t b,
                                       int32_t* d_sum, void* stream) {
    const char* what = "thc_int_aggregate";
    if (!valid_bits(b)) return fail(GA_EINVAL, "%s: b = %d is not 1, 2, 4 or 8", what, b);
    if (N < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(reinterpret_cast<const void* const*>(packed), P, 1, what);
    if (rc) return rc;
    if (!d_sum || !aligned(d_sum, 4)) return fail(GA_EINVAL, "%s: bad output pointer", what);
    const int64_t nbytes = (N * b + 7) / 8;
    int vec_ok = aligned(d_sum, 16);
    PtrTable t{};
    for (int i = 0; i < P; i++) {
        t.p[i] = const_cast<uint8_t*>(packed[i]);
        vec_ok &= aligned(packed[i], 16);
    }
    const int WB = b >= 4 ? 16 : (b == 2 ? 8 : 4);
    const int64_t blocks = ceil_div(nbytes, (int64_t)kThreads * WB);
    if (blocks > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: N too large", what);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const dim3 grid((unsigned)blocks);
    switch (b) {
        case 1: hipLaunchKernelGGL(int_aggregate_kernel<1>, grid, dim3(kThreads), 0, hs, t, P, N, nbytes, d_sum, vec_ok); break;
        case 2: hipLaunchKernelGGL(int_aggregate_kernel<2>, grid, dim3(kThreads), 0, hs, t, P, N, nbytes, d_sum, vec_ok); break;
        case 4: hipLaunchKernelGGL(int_aggregate_kernel<4>, grid, dim3(kThreads), 0, hs, t, P, N, nbytes, d_sum, vec_ok); break;
        default: hipLaunchKernelGGL(int_aggregate_kernel<8>, grid, dim3(kThreads), 0, hs, t, P, N, nbytes, d_sum, vec_ok); break;
    }
    return check_launch(what);
}

extern "C" ga_status thc_dequant(const int32_t* d_sum, int64_t N, int32_t P, int32_t b,
                                 int64_t part_elems, const float* d_mM, void* out, ga_dtype out_dt,
                                 void* stream) {
    const char* what = "thc_dequant";
    if (!valid_dtype(out_dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)out_dt);
    if (!valid_bits(b)) return fail(GA_EINVAL, "%s: b = %d is not 1, 2, 4 or 8", what, b);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N < 0 || part_elems < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (N == 0) return GA_OK;
    if (!d_sum || !d_mM || !out || !aligned(d_sum, 4) || !aligned(d_mM, 4) ||
        !aligned(out, elem_size(out_dt)))
        return fail(GA_EINVAL, "%s: null or misaligned pointer", what);
    const int64_t plen = part_elems > 0 ? part_elems : N;
    const int vec_ok = aligned(d_sum, 16) && aligned(out, 16);
    const int64_t blocks = ceil_div(N, (int64_t)kThreads * kDElems);
    if (blocks > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: N too large", what);
    const int L = (1 << b) - 1;
    const int pow2 = (P & (P - 1)) == 0;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (out_dt == GA_F32)
        hipLaunchKernelGGL(dequant_kernel<GA_F32>, dim3((unsigned)blocks), dim3(kThreads), 0, hs, d_sum, N, plen, d_mM, L, pow2, (float)P, 1.0f / (float)P, out, vec_ok);
    else
        hipLaunchKernelGGL(dequant_kernel<GA_BF16>, dim3((unsigned)blocks), dim3(kThreads), 0, hs, d_sum, N, plen, d_mM, L, pow2, (float)P, 1.0f / (float)P, out, vec_ok);
    return check_launch(what);
}

extern "C" size_t thc_nmse_ws_bytes(int64_t N) {
    (void)N;
    return (size_t)kNmseBlocks * 2 * sizeof(double);
}

extern "C" ga_status thc_nmse(const void* x, const void* xhat, int64_t N, ga_dtype dt, double* d_out,
                              void* d_ws, size_t ws_bytes, void* stream) {
    const char* what = "thc_nmse";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (N < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (!d_out || !aligned(d_out, 8) || !d_ws || !aligned(d_ws, 8))
        return fail(GA_EINVAL, "%s: null or misaligned output/workspace", what);
    if (ws_bytes < thc_nmse_ws_bytes(N))
        return fail(GA_EINVAL, "%s: workspace of %zu bytes, need %zu", what, ws_bytes, thc_nmse_ws_bytes(N));
    if (N > 0 && (!x || !xhat || !aligned(x, elem_size(dt)) || !aligned(xhat, elem_size(dt))))
        return fail(GA_EINVAL, "%s: null or misaligned input", what);
    const int E = dt == GA_F32 ? 4 : 8;
    const int vec_ok = N > 0 && aligned(x, 16) && aligned(xhat, 16);
    int64_t nblk = std::min<int64_t>(kNmseBlocks, std::max<int64_t>(1, ceil_div(N, (int64_t)kThreads * E * 4)));
    hipStream_t hs = static_cast<hipStream_t>(stream);
    double* ws = static_cast<double*>(d_ws);
    ga_status rc;
    if (dt == GA_F32)
        hipLaunchKernelGGL(nmse_partial_kernel<GA_F32>, dim3((unsigned)nblk), dim3(kThreads), 0, hs, x, xhat, N, ws, vec_ok);
    else
        hipLaunchKernelGGL(nmse_partial_kernel<GA_BF16>, dim3((unsigned)nblk), dim3(kThreads), 0, hs, x, xhat, N, ws, vec_ok);
    if ((rc = check_launch(what))) return rc;
    hipLaunchKernelGGL(nmse_final_kernel, dim3(1), dim3(kThreads), 0, hs, ws, (int)nblk, d_out);
    return check_launch(what);
}
