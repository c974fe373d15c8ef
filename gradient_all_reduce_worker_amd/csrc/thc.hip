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

#include <mutex>

#include "common.hpp"
#include "philox.hpp"
#include "quant.hpp"
#include "reduce.hpp"

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
        const uint4 x = load_stream(static_cast<const uint4*>(p) + v);
        f[0] = __uint_as_float(x.x); f[1] = __uint_as_float(x.y);
        f[2] = __uint_as_float(x.z); f[3] = __uint_as_float(x.w);
    }
};
template <> struct Vec16<GA_BF16> {
    static constexpr int kElems = 8;
    __device__ static __forceinline__ void load(const void* p, int64_t v, float* f) {
        const uint4 r = load_stream(static_cast<const uint4*>(p) + v);
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
    const int64_t i = flat_block() * kThreads + threadIdx.x;
    if (i < n_part) {
        keys[2 * i] = 0xFFFFFFFFu;
        keys[2 * i + 1] = 0u;
    }
}

__global__ __launch_bounds__(kThreads) void minmax_final_kernel(uint32_t* keys, int64_t n_part) {
    const int64_t i = flat_block() * kThreads + threadIdx.x;
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

// E binary32 error-feedback values of the elements of x vector v (x of
// type DT; the error buffer shares the element indexing).
template <ga_dtype DT>
__device__ __forceinline__ void load_err_vec(const float* err, int64_t v, float* f) {
    constexpr int E = Vec16<DT>::kElems;
#pragma unroll
    for (int q = 0; q < E / 4; q++) Vec16<GA_F32>::load(err, v * (E / 4) + q, f + 4 * q);
}

// Workgroup (p, j) scans slice j of partition p in every worker's buffer.
// EF: the values scanned are x + e (error feedback) in binary32; vec_ok
// says every x and e buffer is 16-byte aligned, else elements go one by one.
// BOTH (with EF): the extremes of x alone as well, into keys_x, from the
// same loads (the plain grid and the error-feedback grid in one read).
template <ga_dtype DT, bool EF, bool BOTH = false>
__global__ __launch_bounds__(kThreads) void minmax_kernel(PtrTable bufs, PtrTable errs, int vec_ok,
                                                          int P, int64_t N, int64_t plen, int slices,
                                                          int64_t slice_len, uint32_t* keys,
                                                          uint32_t* keys_x = nullptr) {
    static_assert(EF || !BOTH, "both grids need the residuals");
    using V = Vec16<DT>;
    constexpr int E = V::kElems;
    const int64_t blk = flat_block();                     // a folded grid's extra workgroups
    const int64_t p = blk / slices;                        // find lo >= hi below
    const int64_t j = blk % slices;
    const int64_t p0 = p * plen;
    const int64_t pend = min(p0 + plen, N);
    const int64_t lo = p0 + j * slice_len;
    const int64_t hi = min(lo + slice_len, pend);
    if (lo >= hi) return;
    float mn = INFINITY, mx = -INFINITY;
    float mn0 = INFINITY, mx0 = -INFINITY;                // BOTH: x alone
    constexpr int es = DT == GA_BF16 ? 2 : 4;
    if (EF && !vec_ok) {
        for (int w = 0; w < P; w++)
            for (int64_t e = lo + threadIdx.x; e < hi; e += kThreads) {
                const float x0 = load_as_f32(bufs.p[w], e, DT);
                if (BOTH) {
                    mn0 = fminf(mn0, x0);
                    mx0 = fmaxf(mx0, x0);
                }
                const float a = x0 + static_cast<const float*>(errs.p[w])[e];
                mn = fminf(mn, a);
                mx = fmaxf(mx, a);
            }
    } else
    for (int w = 0; w < P; w++) {
        const void* x = bufs.p[w];
        // head: elements before the first 16-byte boundary
        const char* xb = static_cast<const char*>(x);
        const int64_t mis = (int64_t)(((uintptr_t)xb + (uintptr_t)(lo * es)) & 15) / es;
        const int64_t vlo = min(mis ? lo + (E - mis) : lo, hi);
        const int64_t nv = (hi - vlo) / E;
        const int64_t vhi = vlo + nv * E;
        const float* ew = EF ? static_cast<const float*>(errs.p[w]) : nullptr;
        for (int64_t e = lo + threadIdx.x; e < vlo; e += kThreads) {
            const float x0 = load_as_f32(x, e, DT);
            if (BOTH) {
                mn0 = fminf(mn0, x0);
                mx0 = fmaxf(mx0, x0);
            }
            const float a = EF ? x0 + ew[e] : x0;
            mn = fminf(mn, a);
            mx = fmaxf(mx, a);
        }
        // body: 16-byte vectors from the first aligned element, four in flight
        // (with EF every buffer is aligned, so vlo is a multiple of E)
        const void* xa = xb + vlo * es;
        const float* ea = EF ? ew + vlo : nullptr;
        int64_t v = threadIdx.x;
        for (; v + 3 * kThreads < nv; v += 4 * kThreads) {
            float f[4][E];
#pragma unroll
            for (int u = 0; u < 4; u++) V::load(xa, v + u * kThreads, f[u]);
            if (EF) {
                float g[4][E];
#pragma unroll
                for (int u = 0; u < 4; u++) load_err_vec<DT>(ea, v + u * kThreads, g[u]);
#pragma unroll
                for (int u = 0; u < 4; u++)
#pragma unroll
                    for (int i = 0; i < E; i++) {
                        if (BOTH) {
                            mn0 = fminf(mn0, f[u][i]);
                            mx0 = fmaxf(mx0, f[u][i]);
                        }
                        f[u][i] = f[u][i] + g[u][i];
                    }
            }
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
            if (EF) {
                float g[E];
                load_err_vec<DT>(ea, v, g);
#pragma unroll
                for (int i = 0; i < E; i++) {
                    if (BOTH) {
                        mn0 = fminf(mn0, f[i]);
                        mx0 = fmaxf(mx0, f[i]);
                    }
                    f[i] = f[i] + g[i];
                }
            }
#pragma unroll
            for (int i = 0; i < E; i++) {
                mn = fminf(mn, f[i]);
                mx = fmaxf(mx, f[i]);
            }
        }
        // tail
        for (int64_t e = vhi + threadIdx.x; e < hi; e += kThreads) {
            const float x0 = load_as_f32(x, e, DT);
            if (BOTH) {
                mn0 = fminf(mn0, x0);
                mx0 = fmaxf(mx0, x0);
            }
            const float a = EF ? x0 + ew[e] : x0;
            mn = fminf(mn, a);
            mx = fmaxf(mx, a);
        }
    }
    __shared__ float smn[2][kThreads / 64], smx[2][kThreads / 64];
    mn = wave_min(mn);
    mx = wave_max(mx);
    if (BOTH) {
        mn0 = wave_min(mn0);
        mx0 = wave_max(mx0);
    }
    if ((threadIdx.x & 63) == 0) {
        smn[0][threadIdx.x >> 6] = mn;
        smx[0][threadIdx.x >> 6] = mx;
        if (BOTH) {
            smn[1][threadIdx.x >> 6] = mn0;
            smx[1][threadIdx.x >> 6] = mx0;
        }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kThreads / 64; i++) {
            mn = fminf(mn, smn[0][i]);
            mx = fmaxf(mx, smx[0][i]);
            if (BOTH) {
                mn0 = fminf(mn0, smn[1][i]);
                mx0 = fmaxf(mx0, smx[1][i]);
            }
        }
        atomicMin(&keys[2 * p], order_key(mn));
        atomicMax(&keys[2 * p + 1], order_key(mx));
        if (BOTH) {
            atomicMin(&keys_x[2 * p], order_key(mn0));
            atomicMax(&keys_x[2 * p + 1], order_key(mx0));
        }
    }
}

// ------------------------------------------------------------------ quantize
// One Philox call serves a group of 8 consecutive elements (g = e / 8). A
// thread takes kQGroups groups spaced one workgroup width apart, so every
// 16-byte load and every store instruction covers a contiguous span across
// the wave. When the partition length is a multiple of a workgroup's span
// of elements, all its groups share one grid, loaded once (scalar loads).
constexpr int kQGroups = 4;
constexpr size_t kLdsPerCu = 160 * 1024;      // LDS per CU (residency caps)
constexpr int64_t kQSpan = (int64_t)kThreads * kQGroups * 8;   // elements per workgroup
// The per-group fast kernel (bf16 input) is bound by the rounding
// arithmetic; eight groups per thread spread its fixed costs (grid, base
// addresses, counters) over twice as many elements.
constexpr int kFGroups = 8;
constexpr int64_t kFSpan = (int64_t)kThreads * kFGroups * 8;

template <ga_dtype DT>
__device__ __forceinline__ void load_group(const void* x, int64_t g, float* a) {
    if (DT == GA_BF16) {
        const uint4 r = load_stream(static_cast<const uint4*>(x) + g);
        a[0] = bf16_lo(r.x); a[1] = bf16_hi(r.x); a[2] = bf16_lo(r.y); a[3] = bf16_hi(r.y);
        a[4] = bf16_lo(r.z); a[5] = bf16_hi(r.z); a[6] = bf16_lo(r.w); a[7] = bf16_hi(r.w);
    } else {
        const uint4 r0 = load_stream(static_cast<const uint4*>(x) + 2 * g);
        const uint4 r1 = load_stream(static_cast<const uint4*>(x) + 2 * g + 1);
        a[0] = __uint_as_float(r0.x); a[1] = __uint_as_float(r0.y);
        a[2] = __uint_as_float(r0.z); a[3] = __uint_as_float(r0.w);
        a[4] = __uint_as_float(r1.x); a[5] = __uint_as_float(r1.y);
        a[6] = __uint_as_float(r1.z); a[7] = __uint_as_float(r1.w);
    }
}

// Error feedback (THC page, section 5): the value a worker's own level v
// stands for, m + v (M - m) / levels (m when M == m), the same binary32
// steps as the server's dequantization of a one-worker sum.
struct EfGrid {
    float m;
    float delta;             // (M - m) / levels
    bool flat;               // M == m
};

__device__ __forceinline__ EfGrid ef_grid_of(const float* mM, int64_t p, int levels) {
    const float m = mM[2 * p], M = mM[2 * p + 1];
    const float range = M - m;
    return {m, range / (float)levels, range == 0.0f};
}

__device__ __forceinline__ float ef_value(EfGrid q, float v) {
    return q.flat ? q.m : q.m + v * q.delta;
}

// The 8 residuals of group g, read and written through L2 (plain loads and
// stores): the lines just read are still cached when the two 16-byte
// halves of each group are written back, so no line is fetched twice.
__device__ __forceinline__ void load_err_group(const float* err, int64_t g, float* f) {
    const float4* q = reinterpret_cast<const float4*>(err) + 2 * g;
    const float4 a = q[0], b = q[1];
    f[0] = a.x; f[1] = a.y; f[2] = a.z; f[3] = a.w;
    f[4] = b.x; f[5] = b.y; f[6] = b.z; f[7] = b.w;
}
__device__ __forceinline__ void store_err_group(float* err, int64_t g, const float* f) {
    float4* q = reinterpret_cast<float4*>(err) + 2 * g;
    q[0] = make_float4(f[0], f[1], f[2], f[3]);
    q[1] = make_float4(f[4], f[5], f[6], f[7]);
}

// Fast kernel: every group of the workgroup is whole, the buffers are
// 16-byte aligned and the workgroup lies in one partition (the host only
// launches it over such workgroups). No bounds checks, grid loaded once.
// EF: the value quantized is x + e, and e is replaced by x + e minus the
// value of the index sent.
template <ga_dtype DT, int B, bool TABLE, bool EF>
__global__ __launch_bounds__(kThreads) void usq_quantize_fast_kernel(PtrTable bufs, PtrTable errs,
                                                                     PtrTable packed, int worker0,
                                                                     int64_t plen, int pshift,
                                                                     const float* __restrict__ mM,
                                                                     uint32_t k0, uint32_t k1,
                                                                     TableArg tab) {
    constexpr int L = (1 << B) - 1;
    constexpr bool NEG = !TABLE && L < 128;            // negated-index rounding
    extern __shared__ uint4 dyn_cells[];              // table cells (table_lds_bytes)
    const Rounder<TABLE> rd = make_rounder<TABLE>(tab, L, dyn_cells);
    const int slot = blockIdx.y;
    const void* x = bufs.p[slot];
    float* err = EF ? static_cast<float*>(errs.p[slot]) : nullptr;
    uint8_t* out = static_cast<uint8_t*>(packed.p[slot]);
    const uint32_t wid = (uint32_t)(worker0 + slot);
    const int64_t e_blk = (int64_t)blockIdx.x * kFSpan;
    const int64_t part = pshift >= 0 ? (int64_t)blockIdx.x >> pshift : e_blk / plen;
    const Grid gb = grid_of(mM, part, rd.levels);
    float a[kFGroups][8];
#pragma unroll
    for (int j = 0; j < kFGroups; j++)
        load_group<DT>(x, e_blk / 8 + (int64_t)j * kThreads + threadIdx.x, a[j]);
    if (EF) {
        float ev[kFGroups][8];
#pragma unroll
        for (int j = 0; j < kFGroups; j++)
            load_err_group(err, e_blk / 8 + (int64_t)j * kThreads + threadIdx.x, ev[j]);
#pragma unroll
        for (int j = 0; j < kFGroups; j++)
#pragma unroll
            for (int i = 0; i < 8; i++) a[j][i] = a[j][i] + ev[j][i];
    }
    const EfGrid q = EF ? ef_grid_of(mM, part, rd.levels) : EfGrid{};
#pragma unroll
    for (int j = 0; j < kFGroups; j++) {
        const int64_t g = e_blk / 8 + (int64_t)j * kThreads + threadIdx.x;
        const Philox4 r = philox4x32_10((uint32_t)g, (uint32_t)((uint64_t)g >> 32), wid, 0u, k0, k1);
        uint32_t z[8];                                  // NEG: -index mod 2^32
        float res[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            float v;
            if (NEG) {
                z[i] = usq_neg_index(a[j][i], gb, L, uniform16(r, i));
                v = -(float)(int)z[i];
            } else {
                z[i] = rd.index_v(a[j][i], gb, uniform16(r, i), &v);
            }
            if (EF) res[i] = a[j][i] - ef_value(q, v);
        }
        if constexpr (NEG) store_group<B>(out, g, pack_neg_group<B>(z));
        else store_group<B>(out, g, pack_group<B>(z));
        if (EF) store_err_group(err, g, res);
    }
}

// Fast kernel for binary32 inputs. A group of 8 fp32 is 32 bytes; loaded
// per thread it takes two 16-byte loads that each cover every other half
// of the lines a wave touches. Here every load and store instruction is
// contiguous across the wave instead: thread t takes 16-byte vectors t and
// t + 256 of a 2048-element span (elements 4t..4t+3 and 1024+4t..), i.e.
// one half of group t/2 and one half of group 128 + t/2. Each lane draws
// the Philox block of one of those groups and swaps two words with its
// neighbour (DPP), so a call still serves 8 elements and every element gets
// the uniform of the same counter and word as in the per-group kernels:
// identical bits. (MI355X, 32 workers x 138M fp32: b = 4 0.65 -> 0.75 of
// 8 TB/s, b = 8 0.68 -> 0.75.)
constexpr int64_t kLSpan = 2048;       // elements per workgroup of the lane kernel

__device__ __forceinline__ void widen_f32(const uint4& r, float* f) {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
}

// One span's 8 elements of this lane (a[h][i]: vector v0 + 256 h), rounded
// on grid gb and stored; EF: the residual x - value(index) replaces e.
template <int B, bool TABLE, bool EF>
__device__ __forceinline__ void lane_span(float (&a)[2][4], const Rounder<TABLE>& rd, Grid gb,
                                          EfGrid q, int64_t e_blk, int64_t v0, uint32_t wid,
                                          uint32_t k0, uint32_t k1, uint8_t* out, uint4* err) {
    const int t = threadIdx.x;
    const bool odd = t & 1;
    const int64_t g = e_blk / 8 + (odd ? 128 + (t >> 1) : (t >> 1));
    const Philox4 r = philox4x32_10((uint32_t)g, (uint32_t)((uint64_t)g >> 32), wid, 0u, k0, k1);
    const uint32_t ra = swap_pair(odd ? r.v[0] : r.v[2]);
    const uint32_t rb = swap_pair(odd ? r.v[1] : r.v[3]);
    // words of the uniforms of this lane's two half-groups
    const uint32_t u[2][2] = {{odd ? ra : r.v[0], odd ? rb : r.v[1]},
                              {odd ? r.v[2] : ra, odd ? r.v[3] : rb}};
    constexpr int L = (1 << B) - 1;
    constexpr bool NEG = !TABLE && L < 128;            // negated-index rounding
#pragma unroll
    for (int h = 0; h < 2; h++) {
        uint32_t bits = 0;
        float res[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t r16 = (u[h][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
            float v;
            if (NEG) {
                const uint32_t w = usq_neg_index(a[h][i], gb, L, r16);
                v = -(float)(int)w;
                bits += w << (i * B);
            } else {
                bits |= rd.index_v(a[h][i], gb, r16, &v) << (i * B);
            }
            if (EF) res[i] = a[h][i] - ef_value(q, v);
        }
        if (NEG) {
            asm("" : "+v"(bits));   // one negation, not one per term
            bits = 0u - bits;
        }
        const int64_t vv = v0 + h * 256;
        if (B == 8) {                               // written once: nontemporal
            __builtin_nontemporal_store(bits, reinterpret_cast<uint32_t*>(out) + vv);
        } else if (B == 4) {
            __builtin_nontemporal_store((uint16_t)bits, reinterpret_cast<uint16_t*>(out) + vv);
        } else if (B == 2) {
            __builtin_nontemporal_store((uint8_t)bits, out + vv);
        } else {                                    // two vectors per byte
            const uint32_t other = swap_pair(bits);
            if (!odd) out[vv >> 1] = (uint8_t)(bits | (other << 4));
        }
        if (EF)
            store_stream(err + vv, make_uint4(__float_as_uint(res[0]), __float_as_uint(res[1]),
                                              __float_as_uint(res[2]), __float_as_uint(res[3])));
    }
}

// A workgroup takes `spans` consecutive spans, two at a time: the loads of
// both are issued before either is rounded, and the grid (partition index
// and L / (M - m), both computed in vector registers) is worked out once
// per partition rather than per span. pshift >= 0: the partition of span
// s is s >> pshift (partitions of 2^pshift spans, or one partition);
// otherwise it is s kLSpan / plen.
template <int B, bool TABLE, bool EF>
__global__ __launch_bounds__(kThreads) void usq_quantize_lane_kernel(PtrTable bufs, PtrTable errs,
                                                                     PtrTable packed, int worker0,
                                                                     int64_t plen, int pshift,
                                                                     int64_t n_spans, int spans,
                                                                     const float* __restrict__ mM,
                                                                     uint32_t k0, uint32_t k1,
                                                                     TableArg tab) {
    constexpr int L = (1 << B) - 1;
    extern __shared__ uint4 dyn_cells[];              // table cells (table_lds_bytes)
    const Rounder<TABLE> rd = make_rounder<TABLE>(tab, L, dyn_cells);
    const int slot = blockIdx.y;
    const uint4* x = static_cast<const uint4*>(bufs.p[slot]);
    uint4* err = EF ? static_cast<uint4*>(errs.p[slot]) : nullptr;
    uint8_t* out = static_cast<uint8_t*>(packed.p[slot]);
    const uint32_t wid = (uint32_t)(worker0 + slot);
    const int t = threadIdx.x;
    int64_t p_have = -1;
    Grid gb{};
    EfGrid q{};
    for (int sp = 0; sp < spans; sp += 2) {               // spans of this workgroup
        const int64_t blk = flat_block() * spans + sp;
        if (blk >= n_spans) break;                       // also a folded grid's extras
        const bool two = sp + 1 < spans && blk + 1 < n_spans;
        float a[2][2][4];
#pragma unroll
        for (int k = 0; k < 2; k++) {
            const int64_t v0 = (blk + k) * (kLSpan / 4) + t;
            if (k == 0 || two) {
                widen_f32(load_stream(x + v0), a[k][0]);
                widen_f32(load_stream(x + v0 + 256), a[k][1]);
            }
        }
        if (EF) {
#pragma unroll
            for (int k = 0; k < 2; k++) {
                const int64_t v0 = (blk + k) * (kLSpan / 4) + t;
                if (k == 0 || two) {
                    float ev[2][4];
                    widen_f32(load_stream(err + v0), ev[0]);
                    widen_f32(load_stream(err + v0 + 256), ev[1]);
#pragma unroll
                    for (int h = 0; h < 2; h++)
#pragma unroll
                        for (int i = 0; i < 4; i++) a[k][h][i] = a[k][h][i] + ev[h][i];
                }
            }
        }
#pragma unroll
        for (int k = 0; k < 2; k++) {
            if (k == 1 && !two) break;
            const int64_t s = blk + k;
            const int64_t p = pshift >= 0 ? s >> pshift : s * kLSpan / plen;
            if (p != p_have) {                           // workgroup-uniform
                gb = grid_of(mM, p, rd.levels);
                if (EF) q = ef_grid_of(mM, p, rd.levels);
                p_have = p;
            }
            lane_span<B, TABLE, EF>(a[k], rd, gb, q, s * kLSpan, s * (kLSpan / 4) + t, wid, k0, k1,
                                    out, err);
        }
    }
}

// Generic kernel for what the fast kernels do not take (from element
// e_begin, a multiple of 8, on): partial groups, misaligned buffers,
// partitions that are not a multiple of a fast workgroup's span.
template <ga_dtype DT, int B, bool TABLE, bool EF>
__global__ __launch_bounds__(kThreads) void usq_quantize_kernel(PtrTable bufs, PtrTable errs,
                                                                PtrTable packed, int worker0,
                                                                int64_t N, int64_t plen,
                                                                const float* __restrict__ mM,
                                                                uint32_t k0, uint32_t k1,
                                                                int vec_ok, int64_t e_begin,
                                                                TableArg tab) {
    constexpr int L = (1 << B) - 1;
    extern __shared__ uint4 dyn_cells[];              // table cells (table_lds_bytes)
    const Rounder<TABLE> rd = make_rounder<TABLE>(tab, L, dyn_cells);
    const int slot = blockIdx.y;
    const void* x = bufs.p[slot];
    float* err = EF ? static_cast<float*>(errs.p[slot]) : nullptr;
    uint8_t* out = static_cast<uint8_t*>(packed.p[slot]);
    const uint32_t wid = (uint32_t)(worker0 + slot);
    const int64_t e_blk = e_begin + (int64_t)blockIdx.x * kQSpan;
    const int64_t n_full = N / 8;                      // groups of 8 elements
#pragma unroll 1
    for (int j = 0; j < kQGroups; j++) {
        const int64_t g = e_blk / 8 + (int64_t)j * kThreads + threadIdx.x;
        const int64_t e = g * 8;
        if (e >= N) break;
        const Philox4 r = philox4x32_10((uint32_t)g, (uint32_t)((uint64_t)g >> 32), wid, 0u, k0, k1);
        uint32_t z[8];
        const int n_in = g < n_full ? 8 : (int)(N - e);   // elements of this group inside N
        float a[8], res[8];
        if (g < n_full && vec_ok) {
            load_group<DT>(x, g, a);
            if (EF) {
                float ev[8];
                load_err_group(err, g, ev);
#pragma unroll
                for (int i = 0; i < 8; i++) a[i] = a[i] + ev[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < 8; i++) {
                a[i] = i < n_in ? load_as_f32(x, e + i, DT) : 0.0f;
                if (EF && i < n_in) a[i] = a[i] + err[e + i];
            }
        }
#pragma unroll
        for (int i = 0; i < 8; i++) {
            if (i < n_in) {
                const int64_t p = (e + i) / plen;
                float v;
                z[i] = rd.index_v(a[i], grid_of(mM, p, rd.levels), uniform16(r, i), &v);
                if (EF) res[i] = a[i] - ef_value(ef_grid_of(mM, p, rd.levels), v);
            } else {
                z[i] = 0u;                              // past N - 1: index 0
            }
        }
        const uint64_t bits = pack_group<B>(z);
        if (g < n_full && vec_ok) {
            store_group<B>(out, g, bits);
            if (EF) store_err_group(err, g, res);
        } else {
            const int64_t nbytes = (N * B + 7) / 8;
#pragma unroll
            for (int i = 0; i < B; i++)
                if (g * B + i < nbytes) out[g * B + i] = (uint8_t)(bits >> (8 * i));
            if (EF) {
#pragma unroll
                for (int i = 0; i < 8; i++)
                    if (i < n_in) err[e + i] = res[i];
            }
        }
    }
}

// ------------------------------------------------------------------ aggregate
// A unit is 4 consecutive elements: 4 b bits of every worker in, one
// 16-byte int4 out. A thread takes kAUnits units spaced one workgroup width
// apart, so both the narrow per-worker loads and the 16-byte stores are
// contiguous across the wave. b = 8 sums two elements per 32-bit register in
// 16-bit lanes (at most 64 * 255 = 16320 per lane); smaller widths extract
// each index with one bit-field extract.
constexpr int kAUnits = 4;

template <int B>
__device__ __forceinline__ uint32_t unit_bits(const uint8_t* src, int64_t u) {
    // read once: nontemporal (vgg16 b=4 fused pass 0.70 -> 0.67-0.68 ms)
    if (B == 8) return __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(src) + u);
    if (B == 4) return __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(src) + u);
    if (B == 2) return __builtin_nontemporal_load(src + u);
    return (uint32_t)(src[u >> 1] >> (4 * (u & 1))) & 0xFu;
}

template <int B>
__device__ __forceinline__ uint32_t unit_bits_bounded(const uint8_t* src, int64_t u, int64_t nbytes) {
    // bit offset of the unit: 4 u B; bytes past nbytes read as zero
    const int64_t bit0 = 4 * u * B;
    uint64_t v = 0;
    for (int k = 0; k < (4 * B + 7) / 8 + 1; k++) {   // at most 5 bytes
        const int64_t byte = bit0 / 8 + k;
        if (byte < nbytes) v |= (uint64_t)src[byte] << (8 * k);
    }
    return (uint32_t)((v >> (bit0 & 7)) & ((1ull << (4 * B)) - 1));
}

// The sums of kAUnits units u[j] (4 elements each) over the P workers:
// o[j][i] = sum of the indices (uniform) or of the table values tv[z]
// (TABLE) of element 4 u[j] + i. Units at or past n_units give 0.
template <int B, bool TABLE>
__device__ __forceinline__ void unit_sums(const PtrTable& packed, int P, const int64_t* u,
                                          const bool* full, int64_t n_units, int64_t nbytes,
                                          const uint32_t* tv, int32_t (&o)[kAUnits][4]) {
    constexpr uint32_t LM = (1u << B) - 1u;
    uint32_t acc[kAUnits][4];
#pragma unroll
    for (int j = 0; j < kAUnits; j++)
#pragma unroll
        for (int i = 0; i < 4; i++) acc[j][i] = 0;
    constexpr int kBatch = 8;
    for (int i0 = 0; i0 < P; i0 += kBatch) {
        uint32_t w[kBatch][kAUnits];
#pragma unroll
        for (int k = 0; k < kBatch; k++) {
            if (i0 + k < P) {
                const uint8_t* src = static_cast<const uint8_t*>(packed.p[i0 + k]);
#pragma unroll
                for (int j = 0; j < kAUnits; j++)
                    w[k][j] = u[j] < n_units ? (full[j] ? unit_bits<B>(src, u[j])
                                                        : unit_bits_bounded<B>(src, u[j], nbytes))
                                             : 0u;
            }
        }
#pragma unroll
        for (int k = 0; k < kBatch; k++) {
            if (i0 + k < P) {
#pragma unroll
                for (int j = 0; j < kAUnits; j++) {
                    if (TABLE) {
#pragma unroll
                        for (int i = 0; i < 4; i++) acc[j][i] += tv[(w[k][j] >> (i * B)) & LM];
                    } else if (B == 8) {
                        acc[j][0] += w[k][j] & 0x00FF00FFu;          // elements 0 and 2
                        acc[j][1] += (w[k][j] >> 8) & 0x00FF00FFu;   // elements 1 and 3
                    } else {
#pragma unroll
                        for (int i = 0; i < 4; i++) acc[j][i] += (w[k][j] >> (i * B)) & LM;
                    }
                }
            }
        }
    }
#pragma unroll
    for (int j = 0; j < kAUnits; j++) {
        if (B == 8 && !TABLE) {
            o[j][0] = (int32_t)(acc[j][0] & 0xFFFFu); o[j][2] = (int32_t)(acc[j][0] >> 16);
            o[j][1] = (int32_t)(acc[j][1] & 0xFFFFu); o[j][3] = (int32_t)(acc[j][1] >> 16);
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) o[j][i] = (int32_t)acc[j][i];
        }
    }
}

// TABLE: the server of non-uniform THC adds table values T[z] (from LDS)
// instead of the indices themselves (at most P g, plain int32 lanes).
template <int B, bool TABLE>
__global__ __launch_bounds__(kThreads) void int_aggregate_kernel(PtrTable packed, int P, int64_t N,
                                                                 int64_t nbytes,
                                                                 int32_t* __restrict__ sum,
                                                                 int vec_ok, int64_t u_begin,
                                                                 TableArg tab) {
    __shared__ uint32_t tv[TABLE ? 256 : 1];
    if (TABLE) {
        for (int z = threadIdx.x; z < tab.n; z += kThreads) tv[z] = tab.t[z];
        __syncthreads();
    }
    const int64_t n_units = (N + 3) / 4;
    const int64_t u_blk = u_begin + flat_block() * kThreads * kAUnits;
    if (u_blk >= n_units) return;                      // past the folded grid's end
    int64_t u[kAUnits];
    bool full[kAUnits];
#pragma unroll
    for (int j = 0; j < kAUnits; j++) {
        u[j] = u_blk + (int64_t)j * kThreads + threadIdx.x;
        // every byte the unit's bits touch lies below nbytes
        full[j] = vec_ok && (4 * (u[j] + 1) * B + 7) / 8 <= nbytes;
    }
    int32_t o[kAUnits][4];
    unit_sums<B, TABLE>(packed, P, u, full, n_units, nbytes, tv, o);
#pragma unroll
    for (int j = 0; j < kAUnits; j++) {
        if (u[j] >= n_units) continue;
        const int64_t e = 4 * u[j];
        if (vec_ok && e + 4 <= N) {
            store_stream(sum + e, make_uint4((uint32_t)o[j][0], (uint32_t)o[j][1], (uint32_t)o[j][2],
                                             (uint32_t)o[j][3]));
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++)
                if (e + i < N) sum[e + i] = o[j][i];
        }
    }
}

// Wide kernel: thread t loads 16 bytes of every worker (E = 128 / b
// indices), so every load instruction is contiguous across the wave, sums
// them in registers (uniform: two indices per register in 16-bit lanes, at
// most 64 * 255; table: one int32 per index), and writes the E sums through
// an LDS transpose, so every store instruction is contiguous too. Measured
// against the unit kernel on the same MI355X (32 workers x 138M): faster
// at b = 8 (0.92 -> 0.87 ms), slower at b = 4 (fewer resident waves), so
// the host uses it for b = 8; it covers the whole 16-byte vectors and the
// unit kernel above takes the rest.
template <int B, bool TABLE>
__global__ __launch_bounds__(kThreads) void int_aggregate_wide_kernel(PtrTable packed, int P,
                                                                      int32_t* __restrict__ sum,
                                                                      int64_t n_blocks, TableArg tab) {
    const int64_t blk = flat_block();
    if (blk >= n_blocks) return;                       // past the folded grid's end
    constexpr int E = 128 / B;                 // indices per 16 bytes
    constexpr int H = 16 / B;                  // index pairs (s, s + H) per 32-bit word
    constexpr uint32_t LM = (1u << B) - 1u;
    constexpr uint32_t M2 = LM | (LM << 16);
    __shared__ int32_t st[kThreads * E + kThreads * E / 32];
    __shared__ uint32_t tv[TABLE ? 256 : 1];
    if (TABLE) {
        for (int z = threadIdx.x; z < tab.n; z += kThreads) tv[z] = tab.t[z];
        __syncthreads();
    }
    const int64_t v = blk * kThreads + threadIdx.x;
    uint32_t acc[TABLE ? E : 4 * H];
#pragma unroll
    for (int i = 0; i < (TABLE ? E : 4 * H); i++) acc[i] = 0;
    constexpr int kBatch = 8;
    for (int i0 = 0; i0 < P; i0 += kBatch) {
        uint4 w[kBatch];
#pragma unroll
        for (int k = 0; k < kBatch; k++)
            if (i0 + k < P) w[k] = load_stream(static_cast<const uint4*>(packed.p[i0 + k]) + v);
#pragma unroll
        for (int k = 0; k < kBatch; k++) {
            if (i0 + k >= P) continue;
            const uint32_t ww[4] = {w[k].x, w[k].y, w[k].z, w[k].w};
#pragma unroll
            for (int q = 0; q < 4; q++) {
#pragma unroll
                for (int s2 = 0; s2 < 2 * H; s2++) {
                    if (TABLE) acc[q * 2 * H + s2] += tv[(ww[q] >> (B * s2)) & LM];
                    else if (s2 < H) acc[q * H + s2] += (ww[q] >> (B * s2)) & M2;
                }
            }
        }
    }
    // the sums in index order, into LDS (one pad word per 32)
    const int base = threadIdx.x * E;
#pragma unroll
    for (int q = 0; q < 4; q++) {
#pragma unroll
        for (int s2 = 0; s2 < 2 * H; s2++) {
            const int i = q * 2 * H + s2;                         // index within the 16 bytes
            const int32_t o = TABLE ? (int32_t)acc[i]
                                    : (int32_t)(s2 < H ? acc[q * H + s2] & 0xFFFFu
                                                       : acc[q * H + s2 - H] >> 16);
            const int idx = base + i;
            st[idx + idx / 32] = o;
        }
    }
    __syncthreads();
    int32_t* out = sum + blk * kThreads * E;
#pragma unroll
    for (int r = 0; r < E / 4; r++) {
        const int idx = (r * kThreads + threadIdx.x) * 4;
        store_stream(out + idx, make_uint4((uint32_t)st[idx + idx / 32], (uint32_t)st[idx + 1 + (idx + 1) / 32],
                                           (uint32_t)st[idx + 2 + (idx + 2) / 32],
                                           (uint32_t)st[idx + 3 + (idx + 3) / 32]));
    }
}

// ------------------------------------------------------------------ dequant
// A unit is 4 consecutive sums (one 16-byte load); a thread takes kDUnits
// units spaced one workgroup width apart.
constexpr int kDUnits = 4;
constexpr int64_t kDSpan = (int64_t)kThreads * kDUnits * 4;     // elements per workgroup

template <ga_dtype OUT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(const int32_t* __restrict__ S, int64_t N,
                                                           int64_t plen, const float* __restrict__ mM,
                                                           int L, int pow2, float pf, float recip,
                                                           void* out, int vec_ok) {
    const int64_t e_blk = (int64_t)blockIdx.x * kDSpan;
    const bool uniform = plen % kDSpan == 0 || plen >= N;    // one grid per workgroup
    float m0 = 0.0f, range0 = 0.0f, delta0 = 0.0f;
    if (uniform) {
        const int64_t p = e_blk / plen;
        m0 = mM[2 * p];
        range0 = mM[2 * p + 1] - m0;
        delta0 = range0 / (float)L;
    }
    int32_t s[kDUnits][4];
#pragma unroll
    for (int j = 0; j < kDUnits; j++) {
        const int64_t e = e_blk + 4 * ((int64_t)j * kThreads + threadIdx.x);
        if (vec_ok && e + 4 <= N) {
            const uint4 r = load_stream(S + e);
            s[j][0] = (int32_t)r.x; s[j][1] = (int32_t)r.y; s[j][2] = (int32_t)r.z; s[j][3] = (int32_t)r.w;
        } else {
#pragma unroll
            for (int i = 0; i < 4; i++) s[j][i] = e + i < N ? S[e + i] : 0;
        }
    }
#pragma unroll
    for (int j = 0; j < kDUnits; j++) {
        const int64_t e = e_blk + 4 * ((int64_t)j * kThreads + threadIdx.x);
        if (e >= N) break;
        float v[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            float m = m0, range = range0, delta = delta0;
            if (!uniform) {
                const int64_t p = min(e + i, N - 1) / plen;
                m = mM[2 * p];
                range = mM[2 * p + 1] - m;
                delta = range / (float)L;
            }
            const float avg_index = pow2 ? (float)s[j][i] * recip : (float)s[j][i] / pf;
            v[i] = range != 0.0f ? m + avg_index * delta : m;
        }
        const bool whole = vec_ok && e + 4 <= N;
        if (OUT == GA_F32) {
            float* o = static_cast<float*>(out);
            if (whole) {
                store_stream(o + e, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]),
                                               __float_as_uint(v[2]), __float_as_uint(v[3])));
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (e + i < N) o[e + i] = v[i];
            }
        } else {
            uint16_t* o = static_cast<uint16_t*>(out);
            if (whole) {
                *reinterpret_cast<uint2*>(o + e) = make_uint2(pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3]));
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (e + i < N) o[e + i] = (uint16_t)f32_to_bf16_rne(v[i]);
            }
        }
    }
}

// ------------------------------------------------------------------ NMSE
constexpr int kNmseVecs = 4;          // 16-byte vectors per thread and round of nmse_partial_kernel
constexpr int64_t kNmsePieces = 8192;  // about this many workgroups for large inputs

// rounds per workgroup for nvec vectors
__host__ __device__ __forceinline__ int64_t nmse_rounds(int64_t nvec) {
    const int64_t per_round = (int64_t)kNmseVecs * kThreads * kNmsePieces;
    return nvec > per_round ? (nvec + per_round - 1) / per_round : 1;
}

template <ga_dtype DT>
__global__ __launch_bounds__(kThreads) void nmse_partial_kernel(const void* x, const void* xh,
                                                                int64_t N, double* ws, int vec_ok) {
    using V = Vec16<DT>;
    constexpr int E = V::kElems;
    double num = 0.0, den = 0.0;
    const int64_t nvec = vec_ok ? N / E : 0;
    // one contiguous piece per workgroup, `it` rounds of kNmseVecs vectors
    // per thread (contiguous across the wave, loads in flight together);
    // about kNmsePieces pieces in all (2^31 bf16: 1.46 -> 1.27 ms against a
    // grid of 2,048 striding; one round per workgroup: 2.17 ms)
    const int64_t it = nmse_rounds(nvec);
    for (int64_t q = 0; q < it; q++) {
        const int64_t v0 = ((int64_t)blockIdx.x * it + q) * kNmseVecs * kThreads + threadIdx.x;
        float a[kNmseVecs][E], h[kNmseVecs][E];
#pragma unroll
        for (int k = 0; k < kNmseVecs; k++) {
            const int64_t v = v0 + (int64_t)k * kThreads;
            if (v < nvec) {
                V::load(x, v, a[k]);
                V::load(xh, v, h[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < kNmseVecs; k++) {
            if (v0 + (int64_t)k * kThreads < nvec) {
#pragma unroll
                for (int i = 0; i < E; i++) {
                    const double d = (double)a[k][i] - (double)h[k][i];
                    num += d * d;
                    den += (double)a[k][i] * (double)a[k][i];
                }
            }
        }
    }
    const int64_t stride = (int64_t)gridDim.x * kThreads;     // the rest, element by element
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

// ------------------------------------------------------------------ fused server and worker side
// One pass for THC's last three steps: the server's sum S of the P workers'
// indices (or table values), the workers' dequantized average x̂ and, given
// the exact average x, the NMSE partial sums. S and x̂ are computed with
// the same code and arithmetic as int_aggregate_kernel and dequant_kernel,
// so they are bit-identical; S need not be written (x̂ is computed from
// registers), and x̂ is not read back for the NMSE. One workgroup per span
// of kThreads * kAUnits units, launched in order, so the workgroups in
// flight read and write one narrow front of the buffers (a grid of 65,536
// workgroups striding over the spans: shard sum + dequant 3.49 -> 3.08 ms);
// each leaves one NMSE partial, summed in two levels.

template <int B, bool TABLE, ga_dtype OUT>
__global__ __launch_bounds__(kThreads) void agg_dequant_kernel(PtrTable packed, int P, int64_t N,
                                                               int64_t nbytes, int32_t* __restrict__ sum,
                                                               int64_t plen, const float* __restrict__ mM,
                                                               int L, int pow2, float pf, float recip,
                                                               void* out, const void* xref, double* ws,
                                                               int vec_ok, TableArg tab) {
    constexpr int64_t kSpanUnits = (int64_t)kThreads * kAUnits;
    const int64_t n_units = (N + 3) / 4;
    const int64_t blk = flat_block();
    if (blk > 0 && blk * kSpanUnits >= n_units) return; // past the folded grid's end (N = 0: one
                                                        // workgroup writes the zero NMSE partials)
    __shared__ uint32_t tv[TABLE ? 256 : 1];
    __shared__ double sh[kThreads / 64];
    if (TABLE) {
        for (int z = threadIdx.x; z < tab.n; z += kThreads) tv[z] = tab.t[z];
        __syncthreads();
    }
    const bool uniform = plen % (4 * kSpanUnits) == 0 || plen >= N;   // one grid per span
    double num = 0.0, den = 0.0;
    for (int64_t u_blk = blk * kSpanUnits; u_blk < n_units;
         u_blk += (int64_t)gridDim.x * gridDim.z * kSpanUnits) {
        int64_t u[kAUnits];
        bool full[kAUnits];
#pragma unroll
        for (int j = 0; j < kAUnits; j++) {
            u[j] = u_blk + (int64_t)j * kThreads + threadIdx.x;
            full[j] = vec_ok && (4 * (u[j] + 1) * B + 7) / 8 <= nbytes;
        }
        int32_t o[kAUnits][4];
        unit_sums<B, TABLE>(packed, P, u, full, n_units, nbytes, tv, o);
        float m0 = 0.0f, range0 = 0.0f, delta0 = 0.0f;
        if (uniform) {
            const int64_t p = 4 * u_blk / plen;
            m0 = mM[2 * p];
            range0 = mM[2 * p + 1] - m0;
            delta0 = range0 / (float)L;
        }
#pragma unroll
        for (int j = 0; j < kAUnits; j++) {
            if (u[j] >= n_units) continue;
            const int64_t e = 4 * u[j];
            const bool whole = vec_ok && e + 4 <= N;
            if (sum) {
                if (whole) {
                    store_stream(sum + e, make_uint4((uint32_t)o[j][0], (uint32_t)o[j][1],
                                                     (uint32_t)o[j][2], (uint32_t)o[j][3]));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (e + i < N) sum[e + i] = o[j][i];
                }
            }
            float v[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                float m = m0, range = range0, delta = delta0;
                if (!uniform) {
                    const int64_t p = min(e + i, N - 1) / plen;
                    m = mM[2 * p];
                    range = mM[2 * p + 1] - m;
                    delta = range / (float)L;
                }
                const float avg_index = pow2 ? (float)o[j][i] * recip : (float)o[j][i] / pf;
                v[i] = range != 0.0f ? m + avg_index * delta : m;
            }
            float h[4];                                   // x̂ as stored
            if (OUT == GA_F32) {
                float* oo = static_cast<float*>(out);
                if (whole) {
                    store_stream(oo + e, make_uint4(__float_as_uint(v[0]), __float_as_uint(v[1]),
                                                    __float_as_uint(v[2]), __float_as_uint(v[3])));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (e + i < N) oo[e + i] = v[i];
                }
#pragma unroll
                for (int i = 0; i < 4; i++) h[i] = v[i];
            } else {
                uint16_t* oo = static_cast<uint16_t*>(out);
                uint32_t hb[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    hb[i] = f32_to_bf16_rne(v[i]);
                    h[i] = __uint_as_float(hb[i] << 16);
                }
                if (whole) {
                    *reinterpret_cast<uint2*>(oo + e) = make_uint2(hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16));
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (e + i < N) oo[e + i] = (uint16_t)hb[i];
                }
            }
            if (xref) {
                float a[4];
                if (whole && OUT == GA_F32) {
                    widen_f32(load_stream(static_cast<const uint4*>(xref) + e / 4), a);
                } else if (whole) {
                    const uint2 q = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(xref) + e);
                    a[0] = __uint_as_float(q.x << 16); a[1] = __uint_as_float(q.x & 0xFFFF0000u);
                    a[2] = __uint_as_float(q.y << 16); a[3] = __uint_as_float(q.y & 0xFFFF0000u);
                } else {
#pragma unroll
                    for (int i = 0; i < 4; i++) a[i] = e + i < N ? load_as_f32(xref, e + i, OUT) : 0.0f;
                }
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    if (e + i < N) {
                        const double d = (double)a[i] - (double)h[i];
                        num += d * d;
                        den += (double)a[i] * (double)a[i];
                    }
                }
            }
        }
    }
    num = block_sum(num, sh);
    den = block_sum(den, sh);
    if (xref && threadIdx.x == 0) {
        ws[2 * blk] = num;
        ws[2 * blk + 1] = den;
    }
}

}  // namespace
}  // namespace ga

using namespace ga;

namespace ga {
namespace {

// d_mM_x (with errs): the grids of x alone as well, from the same read.
ga_status minmax_impl(const void* const* bufs, const float* const* errs, int32_t P, int64_t N,
                      ga_dtype dt, int64_t part_elems, float* d_mM, void* stream, const char* what,
                      float* d_mM_x = nullptr) {
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (N < 0 || part_elems < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(bufs, P, elem_size(dt), what);
    if (rc) return rc;
    if (errs && (rc = check_workers(reinterpret_cast<const void* const*>(errs), P, 4, what))) return rc;
    if (!d_mM || !aligned(d_mM, 8)) return fail(GA_EINVAL, "%s: bad output pointer", what);
    const int64_t plen = part_elems > 0 ? part_elems : N;
    const int64_t n_part = n_partitions(N, part_elems);
    if (d_mM_x) {
        const uintptr_t a = (uintptr_t)d_mM, b = (uintptr_t)d_mM_x, n = (uintptr_t)(8 * n_part);
        if (!errs || !aligned(d_mM_x, 8) || (a < b + n && b < a + n))
            return fail(GA_EINVAL, "%s: bad or overlapping output pointer", what);
    }
    // ~4096 workgroups in total, slices of at least 4096 elements, a
    // multiple of 64 elements so aligned partitions keep aligned slices
    int64_t slices = std::max<int64_t>(1, std::min<int64_t>(ceil_div(plen, 4096), ceil_div(4096, n_part)));
    int64_t slice_len = ceil_div(ceil_div(plen, slices), 64) * 64;
    slices = ceil_div(plen, slice_len);
    if (!flat_fits(n_part * slices)) return fail(GA_EINVAL, "%s: too many partitions", what);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    uint32_t* keys = reinterpret_cast<uint32_t*>(d_mM);
    uint32_t* keys_x = reinterpret_cast<uint32_t*>(d_mM_x);
    PtrTable t{}, te{};
    int vec_ok = 1;
    for (int i = 0; i < P; i++) {
        t.p[i] = const_cast<void*>(bufs[i]);
        if (errs) {
            te.p[i] = const_cast<float*>(errs[i]);
            vec_ok &= aligned(bufs[i], 16) && aligned(errs[i], 16);
        }
    }
    hipLaunchKernelGGL(minmax_init_kernel, flat_grid(ceil_div(n_part, kThreads)), dim3(kThreads), 0, hs, keys,
                       n_part);
    if ((rc = check_launch(what))) return rc;
    if (keys_x) {
        hipLaunchKernelGGL(minmax_init_kernel, flat_grid(ceil_div(n_part, kThreads)), dim3(kThreads), 0, hs,
                           keys_x, n_part);
        if ((rc = check_launch(what))) return rc;
    }
    const dim3 grid = flat_grid(n_part * slices);
    if (keys_x && dt == GA_F32)
        hipLaunchKernelGGL((minmax_kernel<GA_F32, true, true>), grid, dim3(kThreads), 0, hs, t, te, vec_ok, P, N, plen, (int)slices, slice_len, keys, keys_x);
    else if (keys_x)
        hipLaunchKernelGGL((minmax_kernel<GA_BF16, true, true>), grid, dim3(kThreads), 0, hs, t, te, vec_ok, P, N, plen, (int)slices, slice_len, keys, keys_x);
    else if (dt == GA_F32 && errs)
        hipLaunchKernelGGL((minmax_kernel<GA_F32, true>), grid, dim3(kThreads), 0, hs, t, te, vec_ok, P, N, plen, (int)slices, slice_len, keys);
    else if (dt == GA_F32)
        hipLaunchKernelGGL((minmax_kernel<GA_F32, false>), grid, dim3(kThreads), 0, hs, t, te, vec_ok, P, N, plen, (int)slices, slice_len, keys);
    else if (errs)
        hipLaunchKernelGGL((minmax_kernel<GA_BF16, true>), grid, dim3(kThreads), 0, hs, t, te, vec_ok, P, N, plen, (int)slices, slice_len, keys);
    else
        hipLaunchKernelGGL((minmax_kernel<GA_BF16, false>), grid, dim3(kThreads), 0, hs, t, te, vec_ok, P, N, plen, (int)slices, slice_len, keys);
    if ((rc = check_launch(what))) return rc;
    hipLaunchKernelGGL(minmax_final_kernel, flat_grid(ceil_div(n_part, kThreads)), dim3(kThreads), 0, hs, keys,
                       n_part);
    if (keys_x) {
        if ((rc = check_launch(what))) return rc;
        hipLaunchKernelGGL(minmax_final_kernel, flat_grid(ceil_div(n_part, kThreads)), dim3(kThreads), 0, hs,
                           keys_x, n_part);
    }
    return check_launch(what);
}

// Extremes of n partition grids: the smallest m and the largest M. min and
// max are exact, so this equals the extremes over the partitions' elements.
__global__ __launch_bounds__(kThreads) void minmax_combine_kernel(const float* __restrict__ parts,
                                                                  int64_t n, float* out) {
    float mn = INFINITY, mx = -INFINITY;
    for (int64_t i = threadIdx.x; i < n; i += kThreads) {
        mn = fminf(mn, parts[2 * i]);
        mx = fmaxf(mx, parts[2 * i + 1]);
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
        mn = fminf(mn, __shfl_xor(mn, o));
        mx = fmaxf(mx, __shfl_xor(mx, o));
    }
    __shared__ float sh[2][kThreads / 64];
    if ((threadIdx.x & 63) == 0) {
        sh[0][threadIdx.x >> 6] = mn;
        sh[1][threadIdx.x >> 6] = mx;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kThreads / 64; w++) {
            mn = fminf(mn, sh[0][w]);
            mx = fmaxf(mx, sh[1][w]);
        }
        out[0] = mn + 0.0f;                          // a negative zero as +0
        out[1] = mx + 0.0f;
    }
}

}  // namespace
}  // namespace ga

extern "C" ga_status thc_minmax_combine(const float* d_parts, int64_t n_part, float* d_mM, void* stream) {
    const char* what = "thc_minmax_combine";
    if (n_part < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (n_part == 0) return GA_OK;
    if (!d_parts || !d_mM || !aligned(d_parts, 8) || !aligned(d_mM, 8))
        return fail(GA_EINVAL, "%s: null or misaligned pointer", what);
    const uintptr_t a = (uintptr_t)d_parts, o = (uintptr_t)d_mM;
    if (o < a + (uintptr_t)(8 * n_part) && a < o + 8)
        return fail(GA_EINVAL, "%s: output overlaps the partition grids", what);
    hipLaunchKernelGGL(minmax_combine_kernel, dim3(1), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                       d_parts, n_part, d_mM);
    return check_launch(what);
}

extern "C" ga_status thc_minmax(const void* const* bufs, int32_t P, int64_t N, ga_dtype dt,
                                int64_t part_elems, float* d_mM, void* stream) {
    return minmax_impl(bufs, nullptr, P, N, dt, part_elems, d_mM, stream, "thc_minmax");
}

extern "C" ga_status thc_ef_minmax(const void* const* bufs, const float* const* errs, int32_t P,
                                   int64_t N, ga_dtype dt, int64_t part_elems, float* d_mM,
                                   void* stream) {
    if (!errs) return fail(GA_EINVAL, "thc_ef_minmax: null error buffers");
    return minmax_impl(bufs, errs, P, N, dt, part_elems, d_mM, stream, "thc_ef_minmax");
}

extern "C" ga_status thc_ef_minmax_pair(const void* const* bufs, const float* const* errs, int32_t P,
                                        int64_t N, ga_dtype dt, int64_t part_elems, float* d_mM_x,
                                        float* d_mM_ef, void* stream) {
    if (!errs) return fail(GA_EINVAL, "thc_ef_minmax_pair: null residuals");
    if (!d_mM_x) return fail(GA_EINVAL, "thc_ef_minmax_pair: bad output pointer");
    return minmax_impl(bufs, errs, P, N, dt, part_elems, d_mM_ef, stream, "thc_ef_minmax_pair", d_mM_x);
}

namespace ga {
namespace {

ga_status quantize_impl(const void* const* bufs, int32_t P, int32_t worker0, int64_t N, ga_dtype dt,
                        int64_t part_elems, const float* d_mM, int32_t b, uint64_t seed,
                        uint8_t* const* packed, void* stream, const TableArg* table,
                        const char* what, float* const* errs = nullptr) {
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (!valid_bits(b)) return fail(GA_EINVAL, "%s: b = %d is not 1, 2, 4 or 8", what, b);
    if (N < 0 || part_elems < 0 || worker0 < 0) return fail(GA_EINVAL, "%s: negative argument", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(bufs, P, elem_size(dt), what);
    if (rc) return rc;
    if ((rc = check_workers(reinterpret_cast<const void* const*>(packed), P, 1, what))) return rc;
    if (errs && (rc = check_workers(reinterpret_cast<const void* const*>(errs), P, 4, what))) return rc;
    if (!d_mM || !aligned(d_mM, 4)) return fail(GA_EINVAL, "%s: bad grid pointer", what);
    const int64_t plen = part_elems > 0 ? part_elems : N;
    int vec_ok = 1;
    PtrTable tx{}, tp{}, te{};
    for (int i = 0; i < P; i++) {
        tx.p[i] = const_cast<void*>(bufs[i]);
        tp.p[i] = packed[i];
        vec_ok &= aligned(bufs[i], 16) && aligned(packed[i], 16);
        if (errs) {
            te.p[i] = errs[i];
            vec_ok &= aligned(errs[i], 16);
        }
    }
    // workgroups wholly inside N and inside one partition take a fast kernel:
    // binary32 the lane kernel (2048 elements), bf16 the per-group one
    const int64_t span = dt == GA_F32 ? kLSpan : kFSpan;
    const int64_t fast = (vec_ok && (plen % span == 0 || plen >= N)) ? N / span : 0;
    const int64_t e_begin = fast * span;
    const int64_t blocks = ceil_div(N - e_begin, kQSpan);       // generic workgroups
    // the lane kernel streams best with at most six workgroups per CU (the
    // dynamic LDS also holds the table's cells); with a table each workgroup
    // builds its LDS cell map first, so it takes four spans to spread that over
    const size_t cells_lds = table ? table_lds_bytes(*table) : 0;
    const size_t lane_lds = std::max<size_t>(kLdsPerCu / 6 - 1024, cells_lds);
    const int lane_spans = table ? 4 : 1;
    // partitions of a power-of-two number of fast spans (or one partition):
    // the kernels find a span's partition by a shift
    int pshift = -1;
    if (plen >= N) {
        pshift = 62;
    } else if (plen % span == 0) {
        const int64_t sp = plen / span;
        if ((sp & (sp - 1)) == 0) pshift = __builtin_ctzll((unsigned long long)sp);
    }
    const int64_t lane_blocks = ceil_div(fast, lane_spans);
    if (!(dt == GA_F32 ? flat_fits(lane_blocks) : grid_fits(fast)) || !grid_fits(blocks))
        return fail(GA_EINVAL, "%s: N too large", what);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const TableArg tab = table ? *table : TableArg{};
#define GA_Q2(DT, B, TB, EF)                                                                          \
    do {                                                                                              \
        if (fast > 0 && DT == GA_F32)                                                                 \
            hipLaunchKernelGGL((usq_quantize_lane_kernel<B, TB, EF>),                                 \
                               flat_grid(lane_blocks, (unsigned)P), dim3(kThreads), lane_lds,         \
                               hs, tx, te, tp, worker0, plen, pshift, fast, lane_spans, d_mM, k0, k1,  \
                               tab);                                                                  \
        else if (fast > 0)                                                                            \
            hipLaunchKernelGGL((usq_quantize_fast_kernel<DT, B, TB, EF>),                             \
                               dim3((unsigned)fast, (unsigned)P), dim3(kThreads), cells_lds, hs, tx,  \
                               te, tp, worker0, plen, pshift, d_mM, k0, k1, tab);                     \
        if (blocks > 0)                                                                               \
            hipLaunchKernelGGL((usq_quantize_kernel<DT, B, TB, EF>),                                  \
                               dim3((unsigned)blocks, (unsigned)P), dim3(kThreads), cells_lds, hs,    \
                               tx, te, tp, worker0, N, plen, d_mM, k0, k1, vec_ok, e_begin, tab);     \
    } while (0)
#define GA_Q(DT, B, TB)                                \
    do {                                               \
        if (errs) GA_Q2(DT, B, TB, true);              \
        else GA_Q2(DT, B, TB, false);                  \
    } while (0)
#define GA_QB(DT, TB)                      \
    switch (b) {                           \
        case 1: GA_Q(DT, 1, TB); break;    \
        case 2: GA_Q(DT, 2, TB); break;    \
        case 4: GA_Q(DT, 4, TB); break;    \
        default: GA_Q(DT, 8, TB); break;   \
    }
    if (dt == GA_F32) {
        if (table) { GA_QB(GA_F32, true) } else { GA_QB(GA_F32, false) }
    } else {
        if (table) { GA_QB(GA_BF16, true) } else { GA_QB(GA_BF16, false) }
    }
#undef GA_QB
#undef GA_Q
#undef GA_Q2
    return check_launch(what);
}

ga_status aggregate_impl(const uint8_t* const* packed, int32_t P, int64_t N, int32_t b,
                         int32_t* d_sum, void* stream, const TableArg* table, const char* what) {
    if (!valid_bits(b)) return fail(GA_EINVAL, "%s: b = %d is not 1, 2, 4 or 8", what, b);
    if (N < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(reinterpret_cast<const void* const*>(packed), P, 1, what);
    if (rc) return rc;
    if (!d_sum || !aligned(d_sum, 4)) return fail(GA_EINVAL, "%s: bad output pointer", what);
    const int64_t nbytes = (N * b + 7) / 8;
    int vec_ok = aligned(d_sum, 16);
    bool wide_ok = aligned(d_sum, 16) && b == 8;
    PtrTable t{};
    for (int i = 0; i < P; i++) {
        t.p[i] = const_cast<uint8_t*>(packed[i]);
        vec_ok &= aligned(packed[i], 4);
        wide_ok = wide_ok && aligned(packed[i], 16);
    }
    // whole workgroups of the wide kernel (kThreads 16-byte vectors each),
    // then the unit kernel from the first element they leave
    const int64_t E = 128 / b;
    const int64_t wide_blocks = wide_ok ? (N / E) / kThreads : 0;
    const int64_t u_begin = wide_blocks * kThreads * E / 4;
    const int64_t blocks = ceil_div(ceil_div(N, 4) - u_begin, (int64_t)kThreads * kAUnits);
    if (!flat_fits(blocks) || !flat_fits(wide_blocks)) return fail(GA_EINVAL, "%s: N too large", what);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const dim3 grid = flat_grid(blocks), wide_grid = flat_grid(wide_blocks);
    const TableArg tab = table ? *table : TableArg{};
#define GA_A(B)                                                                                       \
    do {                                                                                              \
        if (wide_blocks > 0 && (B == 4 || B == 8)) {                                                  \
            if (table)                                                                                \
                hipLaunchKernelGGL((int_aggregate_wide_kernel<(B == 4 ? 4 : 8), true>), wide_grid,    \
                                   dim3(kThreads), 0, hs, t, P, d_sum, wide_blocks, tab);             \
            else                                                                                      \
                hipLaunchKernelGGL((int_aggregate_wide_kernel<(B == 4 ? 4 : 8), false>), wide_grid,   \
                                   dim3(kThreads), 0, hs, t, P, d_sum, wide_blocks, tab);             \
        }                                                                                             \
        if (blocks > 0) {                                                                             \
            if (table)                                                                                \
                hipLaunchKernelGGL((int_aggregate_kernel<B, true>), grid, dim3(kThreads), 0, hs, t, P, N, \
                                   nbytes, d_sum, vec_ok, u_begin, tab);                              \
            else                                                                                      \
                hipLaunchKernelGGL((int_aggregate_kernel<B, false>), grid, dim3(kThreads), 0, hs, t, P, N, \
                                   nbytes, d_sum, vec_ok, u_begin, tab);                              \
        }                                                                                             \
    } while (0)
    switch (b) {
        case 1: GA_A(1); break;
        case 2: GA_A(2); break;
        case 4: GA_A(4); break;
        default: GA_A(8); break;
    }
#undef GA_A
    return check_launch(what);
}

ga_status dequant_impl(const int32_t* d_sum, int64_t N, int32_t P, int32_t levels, int64_t part_elems,
                       const float* d_mM, void* out, ga_dtype out_dt, void* stream, const char* what) {
    if (!valid_dtype(out_dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)out_dt);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N < 0 || part_elems < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (N == 0) return GA_OK;
    if (!d_sum || !d_mM || !out || !aligned(d_sum, 4) || !aligned(d_mM, 4) ||
        !aligned(out, elem_size(out_dt)))
        return fail(GA_EINVAL, "%s: null or misaligned pointer", what);
    const int64_t plen = part_elems > 0 ? part_elems : N;
    const int vec_ok = aligned(d_sum, 16) && aligned(out, 16);
    const int64_t blocks = ceil_div(N, kDSpan);
    if (!grid_fits(blocks)) return fail(GA_EINVAL, "%s: N too large", what);
    const int pow2 = (P & (P - 1)) == 0;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (out_dt == GA_F32)
        hipLaunchKernelGGL(dequant_kernel<GA_F32>, dim3((unsigned)blocks), dim3(kThreads), 0, hs, d_sum, N, plen, d_mM, levels, pow2, (float)P, 1.0f / (float)P, out, vec_ok);
    else
        hipLaunchKernelGGL(dequant_kernel<GA_BF16>, dim3((unsigned)blocks), dim3(kThreads), 0, hs, d_sum, N, plen, d_mM, levels, pow2, (float)P, 1.0f / (float)P, out, vec_ok);
    return check_launch(what);
}

}  // namespace
}  // namespace ga

extern "C" ga_status thc_usq_quantize(const void* const* bufs, int32_t P, int32_t worker0, int64_t N,
                                      ga_dtype dt, int64_t part_elems, const float* d_mM, int32_t b,
                                      uint64_t seed, uint8_t* const* packed, void* stream) {
    return quantize_impl(bufs, P, worker0, N, dt, part_elems, d_mM, b, seed, packed, stream, nullptr,
                         "thc_usq_quantize");
}

extern "C" ga_status thc_int_aggregate(const uint8_t* const* packed, int32_t P, int64_t N, int32_t b,
                                       int32_t* d_sum, void* stream) {
    return aggregate_impl(packed, P, N, b, d_sum, stream, nullptr, "thc_int_aggregate");
}

extern "C" ga_status thc_dequant(const int32_t* d_sum, int64_t N, int32_t P, int32_t b,
                                 int64_t part_elems, const float* d_mM, void* out, ga_dtype out_dt,
                                 void* stream) {
    if (!valid_bits(b)) return fail(GA_EINVAL, "thc_dequant: b = %d is not 1, 2, 4 or 8", b);
    return dequant_impl(d_sum, N, P, (1 << b) - 1, part_elems, d_mM, out, out_dt, stream, "thc_dequant");
}

extern "C" ga_status thc_nuhc_quantize(const void* const* bufs, int32_t P, int32_t worker0, int64_t N,
                                       ga_dtype dt, int64_t part_elems, const float* d_mM, int32_t b,
                                       int32_t g, const int32_t* h_table, uint64_t seed,
                                       uint8_t* const* packed, void* stream) {
    TableArg tab;
    ga_status rc = load_table(b, g, h_table, &tab, "thc_nuhc_quantize");
    if (rc) return rc;
    return quantize_impl(bufs, P, worker0, N, dt, part_elems, d_mM, b, seed, packed, stream, &tab,
                         "thc_nuhc_quantize");
}

extern "C" ga_status thc_ef_quantize(const void* const* bufs, float* const* errs, int32_t P,
                                     int32_t worker0, int64_t N, ga_dtype dt, int64_t part_elems,
                                     const float* d_mM, int32_t b, int32_t g,
                                     const int32_t* h_table, uint64_t seed, uint8_t* const* packed,
                                     void* stream) {
    const char* what = "thc_ef_quantize";
    if (!errs) return fail(GA_EINVAL, "%s: null error buffers", what);
    if (!h_table)
        return quantize_impl(bufs, P, worker0, N, dt, part_elems, d_mM, b, seed, packed, stream,
                             nullptr, what, errs);
    TableArg tab;
    ga_status rc = load_table(b, g, h_table, &tab, what);
    if (rc) return rc;
    return quantize_impl(bufs, P, worker0, N, dt, part_elems, d_mM, b, seed, packed, stream, &tab,
                         what, errs);
}

extern "C" ga_status thc_nuhc_aggregate(const uint8_t* const* packed, int32_t P, int64_t N, int32_t b,
                                        int32_t g, const int32_t* h_table, int32_t* d_sum,
                                        void* stream) {
    TableArg tab;
    ga_status rc = load_table(b, g, h_table, &tab, "thc_nuhc_aggregate");
    if (rc) return rc;
    return aggregate_impl(packed, P, N, b, d_sum, stream, &tab, "thc_nuhc_aggregate");
}

extern "C" ga_status thc_nuhc_dequant(const int32_t* d_sum, int64_t N, int32_t P, int32_t g,
                                      int64_t part_elems, const float* d_mM, void* out,
                                      ga_dtype out_dt, void* stream) {
    if (g < 1 || g > kMaxGranularity)
        return fail(GA_EINVAL, "thc_nuhc_dequant: granularity %d outside [1, %d]", g, kMaxGranularity);
    return dequant_impl(d_sum, N, P, g, part_elems, d_mM, out, out_dt, stream, "thc_nuhc_dequant");
}

// One NMSE partial per span, plus one per group of kNmseGroup partials.
static int64_t ad_blocks(int64_t N) {
    return std::max<int64_t>(1, ceil_div(ceil_div(N, 4), (int64_t)kThreads * kAUnits));
}

extern "C" size_t thc_aggregate_dequant_ws_bytes(int64_t N) {
    const int64_t nblk = ad_blocks(std::max<int64_t>(N, 0));
    const int64_t ng = nblk > kNmseGroup ? ceil_div(nblk, kNmseGroup) : 0;
    return (size_t)(nblk + ng) * 2 * sizeof(double);
}

extern "C" ga_status thc_aggregate_dequant(const uint8_t* const* packed, int32_t P, int64_t N, int32_t b,
                                           int32_t g, const int32_t* h_table, int64_t part_elems,
                                           const float* d_mM, int32_t* d_sum, void* out, ga_dtype out_dt,
                                           const void* x_ref, double* d_nmse, void* d_ws, size_t ws_bytes,
                                           void* stream) {
    const char* what = "thc_aggregate_dequant";
    if (!valid_dtype(out_dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)out_dt);
    if (!valid_bits(b)) return fail(GA_EINVAL, "%s: b = %d is not 1, 2, 4 or 8", what, b);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N < 0 || part_elems < 0) return fail(GA_EINVAL, "%s: negative size", what);
    TableArg tab{};
    ga_status rc;
    if (h_table && (rc = load_table(b, g, h_table, &tab, what))) return rc;
    if (x_ref) {
        if (!d_nmse || !aligned(d_nmse, 8) || !d_ws || !aligned(d_ws, 8))
            return fail(GA_EINVAL, "%s: null or misaligned NMSE output/workspace", what);
        if (ws_bytes < thc_aggregate_dequant_ws_bytes(N))
            return fail(GA_EINVAL, "%s: workspace of %zu bytes, need %zu", what, ws_bytes,
                        thc_aggregate_dequant_ws_bytes(N));
        if (!aligned(x_ref, elem_size(out_dt))) return fail(GA_EINVAL, "%s: misaligned x_ref", what);
    }
    if (N > 0) {
        if ((rc = check_workers(reinterpret_cast<const void* const*>(packed), P, 1, what))) return rc;
        if (!d_mM || !out || !aligned(d_mM, 4) || !aligned(out, elem_size(out_dt)) || (d_sum && !aligned(d_sum, 4)))
            return fail(GA_EINVAL, "%s: null or misaligned pointer", what);
    } else if (!x_ref) {
        return GA_OK;
    }
    const int64_t plen = part_elems > 0 ? part_elems : std::max<int64_t>(N, 1);
    const int64_t nbytes = (N * b + 7) / 8;
    int vec_ok = aligned(out, 16) && (!d_sum || aligned(d_sum, 16)) && (!x_ref || aligned(x_ref, 16));
    PtrTable t{};
    for (int i = 0; i < P && N > 0; i++) {
        t.p[i] = const_cast<uint8_t*>(packed[i]);
        vec_ok &= aligned(packed[i], 4);
    }
    const int64_t nblk = ad_blocks(N);                  // one workgroup per span
    if (!flat_fits(nblk)) return fail(GA_EINVAL, "%s: N too large", what);
    const int levels = h_table ? g : (1 << b) - 1;
    const int pow2 = (P & (P - 1)) == 0;
    double* ws = static_cast<double*>(d_ws);
    hipStream_t hs = static_cast<hipStream_t>(stream);
#define GA_AD(B, TB)                                                                                  \
    do {                                                                                              \
        if (out_dt == GA_F32)                                                                         \
            hipLaunchKernelGGL((agg_dequant_kernel<B, TB, GA_F32>), flat_grid(nblk), dim3(kThreads), 0, hs, \
                               t, P, N, nbytes, d_sum, plen, d_mM, levels, pow2, (float)P, 1.0f / (float)P, \
                               out, x_ref, ws, vec_ok, tab);                                          \
        else                                                                                          \
            hipLaunchKernelGGL((agg_dequant_kernel<B, TB, GA_BF16>), flat_grid(nblk), dim3(kThreads), 0, hs, \
                               t, P, N, nbytes, d_sum, plen, d_mM, levels, pow2, (float)P, 1.0f / (float)P, \
                               out, x_ref, ws, vec_ok, tab);                                          \
    } while (0)
#define GA_ADB(TB)                           \
    switch (b) {                             \
        case 1: GA_AD(1, TB); break;         \
        case 2: GA_AD(2, TB); break;         \
        case 4: GA_AD(4, TB); break;         \
        default: GA_AD(8, TB); break;        \
    }
    if (h_table) { GA_ADB(true) } else { GA_ADB(false) }
#undef GA_ADB
#undef GA_AD
    if ((rc = check_launch(what))) return rc;
    if (x_ref) {
        if (nblk > kNmseGroup) {                         // two levels
            const int64_t ng = ceil_div(nblk, kNmseGroup);
            hipLaunchKernelGGL(nmse_group_kernel, dim3((unsigned)ng), dim3(kThreads), 0, hs, ws, nblk,
                               ws + 2 * nblk);
            if ((rc = check_launch(what))) return rc;
            hipLaunchKernelGGL(nmse_final_kernel, dim3(1), dim3(kThreads), 0, hs, ws + 2 * nblk, (int)ng,
                               d_nmse);
        } else {
            hipLaunchKernelGGL(nmse_final_kernel, dim3(1), dim3(kThreads), 0, hs, ws, (int)nblk, d_nmse);
        }
        return check_launch(what);
    }
    return GA_OK;
}

// One partial per workgroup piece, plus one per group of kNmseGroup
// partials.
static int64_t nmse_blocks(int64_t N, int E) {
    return std::max<int64_t>(1, ceil_div(N, (int64_t)kThreads * E * kNmseVecs * nmse_rounds(N / E)));
}

extern "C" size_t thc_nmse_ws_bytes(int64_t N) {
    const int64_t nblk = nmse_blocks(std::max<int64_t>(N, 0), 4);   // binary32: the most pieces
    const int64_t ng = nblk > kNmseGroup ? ceil_div(nblk, kNmseGroup) : 0;
    return (size_t)(nblk + ng) * 2 * sizeof(double);
}

namespace {

ga_status nmse_check(const void* x, const void* xhat, int64_t N, ga_dtype dt, double* d_out,
                     const char* what) {
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (N < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (!d_out || !aligned(d_out, 8)) return fail(GA_EINVAL, "%s: null or misaligned output", what);
    if (N > 0 && (!x || !xhat || !aligned(x, elem_size(dt)) || !aligned(xhat, elem_size(dt))))
        return fail(GA_EINVAL, "%s: null or misaligned input", what);
    if (!grid_fits(nmse_blocks(N, dt == GA_F32 ? 4 : 8))) return fail(GA_EINVAL, "%s: N too large", what);
    return GA_OK;
}

// The NMSE launches over the partials array ws (thc_nmse_ws_bytes(N)
// bytes): one partial per piece, summed in one or two levels.
ga_status nmse_launch(const void* x, const void* xhat, int64_t N, ga_dtype dt, double* d_out,
                      double* ws, hipStream_t hs, const char* what) {
    const int E = dt == GA_F32 ? 4 : 8;
    const int vec_ok = N > 0 && aligned(x, 16) && aligned(xhat, 16);
    const int64_t nblk = nmse_blocks(N, E);
    ga_status rc;
    if (dt == GA_F32)
        hipLaunchKernelGGL(nmse_partial_kernel<GA_F32>, dim3((unsigned)nblk), dim3(kThreads), 0, hs, x, xhat, N, ws, vec_ok);
    else
        hipLaunchKernelGGL(nmse_partial_kernel<GA_BF16>, dim3((unsigned)nblk), dim3(kThreads), 0, hs, x, xhat, N, ws, vec_ok);
    if ((rc = check_launch(what))) return rc;
    if (nblk > kNmseGroup) {                             // two levels
        const int64_t ng = ceil_div(nblk, kNmseGroup);
        hipLaunchKernelGGL(nmse_group_kernel, dim3((unsigned)ng), dim3(kThreads), 0, hs, ws, nblk,
                           ws + 2 * nblk);
        if ((rc = check_launch(what))) return rc;
        hipLaunchKernelGGL(nmse_final_kernel, dim3(1), dim3(kThreads), 0, hs, ws + 2 * nblk, (int)ng, d_out);
    } else {
        hipLaunchKernelGGL(nmse_final_kernel, dim3(1), dim3(kThreads), 0, hs, ws, (int)nblk, d_out);
    }
    return check_launch(what);
}

// Partials of thc_nmse_noalloc: a file-scope device array, one copy per GPU
// for the life of the process. Its name in host code is not a device
// address: each GPU's copy is found with hipGetSymbolAddress, once per
// device, and only that address is handed to kernels. Every slot a call
// reads is written earlier in the same call, so nothing needs clearing.
constexpr size_t kNmseScratchBytes = 160 << 10;
static __device__ __align__(256) double scratch[kNmseScratchBytes / sizeof(double)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// The device address of `scratch` on the GPU that owns stream hs.
ga_status scratch_of(hipStream_t hs, double** out, const char* what) {
    int dev = 0;
    if (hs) {
        hipDevice_t d;
        if (hipStreamGetDevice(hs, &d) != hipSuccess) return fail(GA_EHIP, "%s: unknown stream", what);
        dev = (int)d;
    } else if (hipGetDevice(&dev) != hipSuccess) {
        return fail(GA_EHIP, "%s: no current device", what);
    }
    if (dev < 0 || dev >= kMaxDevices) return fail(GA_EINVAL, "%s: device %d out of range", what, dev);
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        int cur = 0;
        if (hipGetDevice(&cur) != hipSuccess) return fail(GA_EHIP, "%s: no current device", what);
        if (cur != dev && hipSetDevice(dev) != hipSuccess)
            return fail(GA_EHIP, "%s: cannot select device %d", what, dev);
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (cur != dev) (void)hipSetDevice(cur);
        if (e != hipSuccess || !p)
            return fail(GA_EHIP, "%s: hipGetSymbolAddress of the scratch array: %s", what,
                        hipGetErrorString(e));
        g_scratch_ptr[dev] = p;
    }
    *out = static_cast<double*>(g_scratch_ptr[dev]);
    return GA_OK;
}

}  // namespace

extern "C" ga_status thc_nmse(const void* x, const void* xhat, int64_t N, ga_dtype dt, double* d_out,
                              void* d_ws, size_t ws_bytes, void* stream) {
    const char* what = "thc_nmse";
    ga_status rc = nmse_check(x, xhat, N, dt, d_out, what);
    if (rc) return rc;
    if (!d_ws || !aligned(d_ws, 8)) return fail(GA_EINVAL, "%s: null or misaligned workspace", what);
    if (ws_bytes < thc_nmse_ws_bytes(N))
        return fail(GA_EINVAL, "%s: workspace of %zu bytes, need %zu", what, ws_bytes, thc_nmse_ws_bytes(N));
    return nmse_launch(x, xhat, N, dt, d_out, static_cast<double*>(d_ws), static_cast<hipStream_t>(stream),
                       what);
}

extern "C" ga_status thc_nmse_noalloc(const void* x, const void* xhat, int64_t N, ga_dtype dt,
                                      double* d_out, void* stream) {
    const char* what = "thc_nmse_noalloc";
    ga_status rc = nmse_check(x, xhat, N, dt, d_out, what);
    if (rc) return rc;
    if (thc_nmse_ws_bytes(N) > kNmseScratchBytes)
        return fail(GA_EINVAL, "%s: N = %lld needs %zu bytes of partials, more than the %zu bytes of "
                    "the static scratch", what, (long long)N, thc_nmse_ws_bytes(N), kNmseScratchBytes);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    double* ws = nullptr;
    if ((rc = scratch_of(hs, &ws, what))) return rc;
    return nmse_launch(x, xhat, N, dt, d_out, ws, hs, what);
}
