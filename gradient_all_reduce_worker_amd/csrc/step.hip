// step.hip -- the ring average and one uniform THC pass in a single read of
// the workers' gradients.
//
// A step of the simulated data-parallel job computes, over P workers'
// buffers, THC's uniform quantization of every worker's gradient, the
// server's integer sum of the indices with the dequantized average and its
// NMSE ("THC: Accelerating Distributed Deep Learning Using Tensor
// Homomorphic Compression", sections 2-3, Algorithm 1), and the exact
// average by the ring all-reduce ("Horovod: Fast and Easy Distributed Deep
// Learning in TensorFlow", section 3.4; systemcraft lesson "Collective
// Communication: Ring All-Reduce", sections 4 and 7), which THC's estimate is
// measured against. Run one after another those stages read every gradient
// twice (quantizer, ring) and the indices and the average once more (sum,
// dequant, NMSE). Here one pass reads each gradient once and produces all of
// it: per group of 8 elements a thread loads each worker's 8 values,
// quantizes them with the worker's Philox stream and the partition's grid,
// adds the indices into the server's sum, and folds the values in the
// ring's order; then it writes the average to every worker, the
// dequantized average x̂, optionally the packed indices and the sums, and
// adds the NMSE terms. Every output is bit for bit what thc_usq_quantize,
// thc_aggregate_dequant and ga_ring_allreduce_sim (fused, op = avg) leave;
// the NMSE is summed in another order (within rounding of it).
//
// A workgroup takes 256 consecutive groups (2048 elements). When they lie
// in one chunk of one ring partition (every workgroup when chunks are
// multiples of 2048 elements), the workers are loaded in the chunk's fold
// order, so the fold is the load order and each value is quantized as it
// arrives; otherwise the indices are made in worker order and each element
// is folded in its own chunk's order from memory. bf16 buffers take
// thc_ring_kernel (a thread holds whole groups: 16 bytes per worker);
// binary32 buffers take thc_ring_lane_kernel (lane pairs share groups, so
// every load instruction is contiguous across the wave).
#include <algorithm>

#include "common.hpp"
#include "philox.hpp"
#include "quant.hpp"
#include "reduce.hpp"

namespace ga {
namespace {

constexpr int kBatch = 16;        // worker loads in flight per thread (P given at run time)

// x / P, or x * (1/P) when that is exact (P a power of two): the ring's
// average and the dequantizer's S / P.
struct Avg {
    int pow2;
    float pf;
    float recip;
    __device__ __forceinline__ float apply(float x) const { return pow2 ? x * recip : x / pf; }
};

// 8 consecutive elements (one group) of a worker as binary32 (bf16 buffers;
// binary32 ones take the lane-pair kernel below).
template <ga_dtype DT> struct Group8;

template <> struct Group8<GA_BF16> {
    static constexpr int kVecs = 1;       // 16-byte vectors per group
    __device__ static __forceinline__ void widen(const uint4* r, float* f) {
        f[0] = bf16_lo(r[0].x); f[1] = bf16_hi(r[0].x); f[2] = bf16_lo(r[0].y); f[3] = bf16_hi(r[0].y);
        f[4] = bf16_lo(r[0].z); f[5] = bf16_hi(r[0].z); f[6] = bf16_lo(r[0].w); f[7] = bf16_hi(r[0].w);
    }
    // stored value of f (round to nearest even) as bits, and as binary32.
    // gfx950 narrows two binary32 values to bf16 in one instruction
    // (v_cvt_pk_bf16_f32), rounding to nearest even like f32_to_bf16_rne
    // for every value but a NaN, which it quiets: one instruction per pair
    // instead of three per value.
    __device__ static __forceinline__ void narrow(const float* f, uint4* r, float* back) {
        typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
        typedef float f32x2 __attribute__((ext_vector_type(2)));
        uint32_t h[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const f32x2 v = {f[2 * j], f[2 * j + 1]};
            h[j] = __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2));
            back[2 * j] = __uint_as_float(h[j] << 16);
            back[2 * j + 1] = __uint_as_float(h[j] & 0xFFFF0000u);
        }
        r[0] = make_uint4(h[0], h[1], h[2], h[3]);
    }
    __device__ static __forceinline__ float load1(const void* p, int64_t e) {
        return __uint_as_float((uint32_t) static_cast<const uint16_t*>(p)[e] << 16);
    }
};

template <ga_dtype DT>
__device__ __forceinline__ void load8(const void* p, int64_t g, uint4* r) {
    constexpr int K = Group8<DT>::kVecs;
#pragma unroll
    for (int v = 0; v < K; v++) r[v] = load_stream(static_cast<const uint4*>(p) + K * g + v);
}

template <ga_dtype DT>
__device__ __forceinline__ void store8(void* p, int64_t g, const uint4* r) {
    constexpr int K = Group8<DT>::kVecs;
#pragma unroll
    for (int v = 0; v < K; v++) store_stream(static_cast<uint4*>(p) + K * g + v, r[v]);
}

// The ring chunk of element e: partition p of length plen (the last one
// short), chunk c = (e - p0) / ceil(n_p / P); the chunk's fold starts at
// worker c.
struct Chunk {
    int64_t part;
    int c;
};

__device__ __forceinline__ Chunk chunk_of(int64_t e, int64_t N, int64_t plen, int P) {
    const int64_t p = e / plen, p0 = p * plen;
    const int64_t n = min(N - p0, plen);
    const int64_t C = (n + P - 1) / P;
    return {p, (int)((e - p0) / C)};
}

// One worker's 8 values a of group g: quantized with the worker's Philox
// block of the group, indices added into zs (negated modulo 2^32 when the
// grid has fewer than 128 levels, as the quantizer's packer keeps them) and
// packed to the worker's index buffer.
template <int B>
__device__ __forceinline__ void quantize8(const float* a, Grid gq, int64_t g, uint32_t wid, uint32_t k0,
                                          uint32_t k1, uint32_t* zs, uint8_t* out) {
    constexpr int L = (1 << B) - 1;
    const Philox4 r = philox4x32_10((uint32_t)g, (uint32_t)((uint64_t)g >> 32), wid, 0u, k0, k1);
    uint32_t z[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        z[i] = L < 128 ? usq_neg_index(a[i], gq, L, uniform16(r, i)) : usq_index(a[i], gq, L, uniform16(r, i));
        zs[i] += z[i];
    }
    if (out) {
        if constexpr (L < 128) store_group<B>(out, g, pack_neg_group<B>(z));
        else store_group<B>(out, g, pack_group<B>(z));
    }
}

// PT > 0: P fixed at compile time (every worker loop unrolled, so the
// workers' Philox rounds and roundings interleave); WPE: waves per SIMD the
// register allocation aims for. Measured on 8 x 2^31 bf16, b = 2: P at run
// time (110 registers, 4 waves) 16.9-17.2 ms; P = 8 at compile time 14.5-15.5
// ms (96 registers); and held to 5 waves (92 registers, no spills) 14.2 ms;
// 6 waves spills and is slower.
template <ga_dtype DT, int B, int PT, int WPE>
__global__ __attribute__((amdgpu_waves_per_eu(WPE))) __launch_bounds__(kThreads) void thc_ring_kernel(
        PtrTable bufs, PtrTable packed, int has_packed, int P_, int worker0, int64_t N, int64_t rplen,
        int64_t qplen, const float* __restrict__ mM, uint32_t k0, uint32_t k1, Avg avg,
        int32_t* __restrict__ sum, void* xhat, double* ws, int64_t blk_base) {
    using G = Group8<DT>;
    constexpr int K = G::kVecs;
    constexpr int L = (1 << B) - 1;
    constexpr int kB = PT > 0 ? PT : kBatch;          // worker loads in flight
    const int P = PT > 0 ? PT : P_;
    __shared__ double sh[kThreads / 64];
    const int64_t n_groups = N / 8;
    const int64_t blk = blk_base + flat_block();       // this piece's first workgroup + ours
    const int64_t g0 = blk * kThreads;
    if (g0 >= n_groups) return;                        // past the folded grid's end
    const int64_t g = g0 + threadIdx.x;
    const bool live = g < n_groups;
    const int64_t gl = min(g0 + (int64_t)kThreads, n_groups) - 1;       // last group here
    const Chunk first = chunk_of(8 * g0, N, rplen, P), last = chunk_of(8 * gl + 7, N, rplen, P);
    const bool uniform = first.part == last.part && first.c == last.c;
    // the group's quantizer partition (qplen is a multiple of 8)
    const int64_t q = live ? 8 * g / qplen : 0;
    const Grid gq = grid_of(mM, q, L);
    float acc[8];
    uint32_t zs[8];
#pragma unroll
    for (int i = 0; i < 8; i++) zs[i] = 0u;
    if (uniform) {
        // workers in the chunk's fold order first.c, first.c + 1, ...
        for (int kb = 0; kb < P; kb += kB) {
            uint4 raw[kB][K];
#pragma unroll
            for (int kk = 0; kk < kB; kk++) {
                if (kb + kk < P && live) {
                    int w = first.c + kb + kk;
                    if (w >= P) w -= P;
                    load8<DT>(bufs.p[w], g, raw[kk]);
                }
            }
#pragma unroll
            for (int kk = 0; kk < kB; kk++) {
                if (kb + kk < P && live) {
                    int w = first.c + kb + kk;
                    if (w >= P) w -= P;
                    float a[8];
                    G::widen(raw[kk], a);
                    if (kb + kk == 0) {
#pragma unroll
                        for (int i = 0; i < 8; i++) acc[i] = a[i];
                    } else {
#pragma unroll
                        for (int i = 0; i < 8; i++) acc[i] = acc[i] + a[i];
                    }
                    quantize8<B>(a, gq, g, (uint32_t)(worker0 + w), k0, k1, zs,
                                 has_packed ? static_cast<uint8_t*>(packed.p[w]) : nullptr);
                }
            }
        }
    } else if (live) {
        // indices in worker order, then each element folded in its own
        // chunk's order, read again (a few workgroups per chunk boundary)
        for (int w = 0; w < P; w++) {
            uint4 raw[K];
            load8<DT>(bufs.p[w], g, raw);
            float a[8];
            G::widen(raw, a);
            quantize8<B>(a, gq, g, (uint32_t)(worker0 + w), k0, k1, zs,
                         has_packed ? static_cast<uint8_t*>(packed.p[w]) : nullptr);
        }
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const int64_t e = 8 * g + i;
            int w = chunk_of(e, N, rplen, P).c;
            float s = G::load1(bufs.p[w], e);
            for (int k = 1; k < P; k++) {
                w = w + 1 == P ? 0 : w + 1;
                s = s + G::load1(bufs.p[w], e);
            }
            acc[i] = s;
        }
    }
    double num = 0.0, den = 0.0;
    if (live) {
        // the ring's average, to every worker
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; i++) acc[i] = avg.apply(acc[i]);
        uint4 o[K];
        G::narrow(acc, o, x);
        for (int w = 0; w < P; w++) store8<DT>(bufs.p[w], g, o);
        // the server's sum and the dequantized average m + (S / P) delta
        const float m = mM[2 * q], range = mM[2 * q + 1] - m, delta = range / (float)L;
        int32_t S[8];
        float v[8], h[8];
#pragma unroll
        for (int i = 0; i < 8; i++) {
            S[i] = L < 128 ? (int32_t)(0u - zs[i]) : (int32_t)zs[i];
            v[i] = range != 0.0f ? m + avg.apply((float)S[i]) * delta : m;
        }
        if (sum) {
            store_stream(sum + 8 * g, make_uint4((uint32_t)S[0], (uint32_t)S[1], (uint32_t)S[2], (uint32_t)S[3]));
            store_stream(sum + 8 * g + 4, make_uint4((uint32_t)S[4], (uint32_t)S[5], (uint32_t)S[6], (uint32_t)S[7]));
        }
        uint4 ho[K];
        G::narrow(v, ho, h);
        store8<DT>(xhat, g, ho);
        // NMSE terms of the values as stored (each square added in one
        // fused binary64 operation)
#pragma unroll
        for (int i = 0; i < 8; i++) {
            const double xd = (double)x[i], d = xd - (double)h[i];
            num = fma(d, d, num);
            den = fma(xd, xd, den);
        }
    }
    if (ws) {
        num = block_sum(num, sh);
        den = block_sum(den, sh);
        if (threadIdx.x == 0) {
            ws[2 * blk] = num;
            ws[2 * blk + 1] = den;
        }
    }
}

// ---------------------------------------------------------------- binary32 in lane pairs

// A group of 8 binary32 is 32 bytes, so a thread holding whole groups makes
// each 16-byte load instruction cover every other half of the wave's lines.
// For binary32 the pass takes a workgroup's 2048 elements as the lane
// quantizer does: thread t holds 16-byte vectors t and t + 256 of the span
// (one half of group t/2 and one half of group 128 + t/2); per worker the
// even lane of a pair draws the Philox block of the first group and the odd
// lane that of the second, and they swap two words, so every element gets
// the uniform of the same counter and word as in the per-group pass.

// One worker's 8 values a[h][i] (vector v[h], element i) of this lane:
// indices on the grids gq[h] added into zs, packed into out.
template <int B>
__device__ __forceinline__ void lane_quantize(const float (&a)[2][4], const Grid (&gq)[2], int64_t g_lane,
                                              bool odd, uint32_t wid, uint32_t k0, uint32_t k1,
                                              uint32_t (&zs)[2][4], uint8_t* out, const int64_t (&v)[2],
                                              const bool (&live)[2]) {
    constexpr int L = (1 << B) - 1;
    constexpr bool NEG = L < 128;                  // negated indices, one negation per vector
    const Philox4 r = philox4x32_10((uint32_t)g_lane, (uint32_t)((uint64_t)g_lane >> 32), wid, 0u, k0, k1);
    const uint32_t ra = swap_pair(odd ? r.v[0] : r.v[2]);
    const uint32_t rb = swap_pair(odd ? r.v[1] : r.v[3]);
    const uint32_t u[2][2] = {{odd ? ra : r.v[0], odd ? rb : r.v[1]},
                              {odd ? r.v[2] : ra, odd ? r.v[3] : rb}};
#pragma unroll
    for (int h = 0; h < 2; h++) {
        uint32_t bits = 0;
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const uint32_t r16 = (u[h][i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
            if (NEG) {
                const uint32_t w = usq_neg_index(a[h][i], gq[h], L, r16);
                zs[h][i] += w;
                bits += w << (i * B);
            } else {
                const uint32_t z = usq_index(a[h][i], gq[h], L, r16);
                zs[h][i] += z;
                bits |= z << (i * B);
            }
        }
        if (NEG) {
            asm("" : "+v"(bits));
            bits = 0u - bits;
        }
        if (B == 1) {                              // two vectors per byte: every lane swaps
            const uint32_t other = swap_pair(bits);
            if (out && live[h] && !odd) out[v[h] >> 1] = (uint8_t)(bits | (other << 4));
        } else if (out && live[h]) {
            if (B == 8) __builtin_nontemporal_store(bits, reinterpret_cast<uint32_t*>(out) + v[h]);
            else if (B == 4) __builtin_nontemporal_store((uint16_t)bits, reinterpret_cast<uint16_t*>(out) + v[h]);
            else __builtin_nontemporal_store((uint8_t)bits, out + v[h]);
        }
    }
}

// As thc_ring_kernel for binary32 buffers, in lane pairs; KB worker loads in
// flight per vector.
template <int B, int PT, int KB, int WPE>
__global__ __attribute__((amdgpu_waves_per_eu(WPE))) __launch_bounds__(kThreads) void thc_ring_lane_kernel(
        PtrTable bufs, PtrTable packed, int has_packed, int P_, int worker0, int64_t N, int64_t rplen,
        int64_t qplen, const float* __restrict__ mM, uint32_t k0, uint32_t k1, Avg avg,
        int32_t* __restrict__ sum, void* xhat, double* ws, int64_t blk_base) {
    constexpr int L = (1 << B) - 1;
    const int P = PT > 0 ? PT : P_;
    __shared__ double sh[kThreads / 64];
    const int64_t n_vec = N / 4;
    const int64_t blk = blk_base + flat_block();
    const int64_t vb = blk * (2 * kThreads);         // the span's first vector
    if (vb >= n_vec) return;                         // past the folded grid's end
    const int t = threadIdx.x;
    const bool odd = t & 1;
    const int64_t v[2] = {vb + t, vb + t + kThreads};
    const bool live[2] = {v[0] < n_vec, v[1] < n_vec};
    const int64_t g_lane = (vb >> 1) + (odd ? kThreads / 2 + (t >> 1) : (t >> 1));
    const int64_t e_last = min(vb + 2 * kThreads, n_vec) * 4 - 1;
    const Chunk first = chunk_of(vb * 4, N, rplen, P), last = chunk_of(e_last, N, rplen, P);
    const bool uniform = first.part == last.part && first.c == last.c;
    int64_t q[2];
    Grid gq[2];
#pragma unroll
    for (int h = 0; h < 2; h++) {
        q[h] = live[h] ? 4 * v[h] / qplen : 0;     // qplen is a multiple of 8
        gq[h] = grid_of(mM, q[h], L);
    }
    float acc[2][4];
    uint32_t zs[2][4];
#pragma unroll
    for (int h = 0; h < 2; h++)
#pragma unroll
        for (int i = 0; i < 4; i++) zs[h][i] = 0u;
    const uint4 zero = make_uint4(0u, 0u, 0u, 0u);
    if (uniform) {
        // workers in the chunk's fold order first.c, first.c + 1, ...
        for (int kb = 0; kb < P; kb += KB) {
            uint4 raw[KB][2];
#pragma unroll
            for (int kk = 0; kk < KB; kk++) {
                if (kb + kk < P) {
                    int w = first.c + kb + kk;
                    if (w >= P) w -= P;
                    const uint4* src = static_cast<const uint4*>(bufs.p[w]);
#pragma unroll
                    for (int h = 0; h < 2; h++) raw[kk][h] = live[h] ? load_stream(src + v[h]) : zero;
                }
            }
#pragma unroll
            for (int kk = 0; kk < KB; kk++) {
                if (kb + kk < P) {
                    int w = first.c + kb + kk;
                    if (w >= P) w -= P;
                    float a[2][4];
#pragma unroll
                    for (int h = 0; h < 2; h++) {
                        a[h][0] = __uint_as_float(raw[kk][h].x); a[h][1] = __uint_as_float(raw[kk][h].y);
                        a[h][2] = __uint_as_float(raw[kk][h].z); a[h][3] = __uint_as_float(raw[kk][h].w);
#pragma unroll
                        for (int i = 0; i < 4; i++) acc[h][i] = kb + kk == 0 ? a[h][i] : acc[h][i] + a[h][i];
                    }
                    lane_quantize<B>(a, gq, g_lane, odd, (uint32_t)(worker0 + w), k0, k1, zs,
                                     has_packed ? static_cast<uint8_t*>(packed.p[w]) : nullptr, v, live);
                }
            }
        }
    } else {
        // indices in worker order, then each element folded in its own
        // chunk's order, read again (a few workgroups per chunk boundary)
        for (int w = 0; w < P; w++) {
            const uint4* src = static_cast<const uint4*>(bufs.p[w]);
            float a[2][4];
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const uint4 r4 = live[h] ? load_stream(src + v[h]) : zero;
                a[h][0] = __uint_as_float(r4.x); a[h][1] = __uint_as_float(r4.y);
                a[h][2] = __uint_as_float(r4.z); a[h][3] = __uint_as_float(r4.w);
            }
            lane_quantize<B>(a, gq, g_lane, odd, (uint32_t)(worker0 + w), k0, k1, zs,
                             has_packed ? static_cast<uint8_t*>(packed.p[w]) : nullptr, v, live);
        }
#pragma unroll
        for (int h = 0; h < 2; h++) {
#pragma unroll
            for (int i = 0; i < 4; i++) {
                if (!live[h]) continue;
                const int64_t e = 4 * v[h] + i;
                int w = chunk_of(e, N, rplen, P).c;
                float x = static_cast<const float*>(bufs.p[w])[e];
                for (int k = 1; k < P; k++) {
                    w = w + 1 == P ? 0 : w + 1;
                    x = x + static_cast<const float*>(bufs.p[w])[e];
                }
                acc[h][i] = x;
            }
        }
    }
    double num = 0.0, den = 0.0;
#pragma unroll
    for (int h = 0; h < 2; h++) {
        if (!live[h]) continue;
        // the ring's average, to every worker
        float x[4];
#pragma unroll
        for (int i = 0; i < 4; i++) x[i] = avg.apply(acc[h][i]);
        const uint4 o = make_uint4(__float_as_uint(x[0]), __float_as_uint(x[1]), __float_as_uint(x[2]),
                                   __float_as_uint(x[3]));
        for (int w = 0; w < P; w++) store_stream(static_cast<uint4*>(bufs.p[w]) + v[h], o);
        // the server's sum and the dequantized average m + (S / P) delta
        const float m = mM[2 * q[h]], range = mM[2 * q[h] + 1] - m, delta = range / (float)L;
        int32_t S[4];
        float hv[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            S[i] = L < 128 ? (int32_t)(0u - zs[h][i]) : (int32_t)zs[h][i];
            hv[i] = range != 0.0f ? m + avg.apply((float)S[i]) * delta : m;
        }
        if (sum) store_stream(sum + 4 * v[h], make_uint4((uint32_t)S[0], (uint32_t)S[1], (uint32_t)S[2], (uint32_t)S[3]));
        store_stream(static_cast<uint4*>(xhat) + v[h], make_uint4(__float_as_uint(hv[0]), __float_as_uint(hv[1]),
                                                                   __float_as_uint(hv[2]), __float_as_uint(hv[3])));
        // NMSE terms of the values as stored
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const double d = (double)x[i] - (double)hv[i];
            num += d * d;
            den += (double)x[i] * (double)x[i];
        }
    }
    if (ws) {
        num = block_sum(num, sh);
        den = block_sum(den, sh);
        if (threadIdx.x == 0) {
            ws[2 * blk] = num;
            ws[2 * blk + 1] = den;
        }
    }
}

// The pass is launched in pieces of at most kStepPiece workgroups (2^26
// elements); each piece's workgroups carry on the global numbering.
// Measured on 8 x 2^31 bf16, b = 2, builds loaded side by side and their
// calls interleaved (medians of 12): one launch 16.69 ms; pieces of 2^14 /
// 2^15 / 2^16 / 2^17 workgroups 16.16 / 16.00 / 16.19 / 16.45 ms.
constexpr int64_t kStepPiece = (int64_t)1 << 15;
// The lane-pair kernel with P at run time, 8 worker loads in flight per
// vector and 4 waves per SIMD (110-114 registers, no spills). Measured
// against the per-group layout with the same results, byte for byte:
// 32 x 138M binary32, b = 4: 14.50 -> 7.97 ms; 16 x 2^27, b = 4: 3.74 ->
// 3.63 ms; 8 x 2^28, b = 2: 3.88 -> 3.66 ms. P fixed at compile time spills
// at 4 waves; 16 loads in flight (168 registers, spills) 8.55 ms at 32 x 138M.
constexpr int kLaneWaves = 4;
constexpr int kLaneBatch = 8;

int64_t step_blocks(int64_t N) { return std::max<int64_t>(1, ceil_div(std::max<int64_t>(N, 0) / 8, kThreads)); }

// Workgroups resident per CU on large inputs. The ring alone streams best
// with few (its 2P open DRAM streams), but here the rounding arithmetic needs
// the waves to hide behind: 8 x 2^31 bf16, b = 2, 23.6 ms at two per CU,
// 16.9 at four, 16.9-17.3 uncapped. At 32 workers (fp32, 138M) two per CU
// measured best (14.0 ms; four 15.0, uncapped 15.1-15.7). Capped with unused
// dynamic LDS, as the ring does.
size_t step_lds(int P, int64_t bytes) {
    constexpr size_t kLdsPerCu = 160 * 1024;
    if (bytes < ((int64_t)1 << 28) || P <= 16) return 0;
    return kLdsPerCu / 2 - 1024;
}

}  // namespace
}  // namespace ga

using namespace ga;

extern "C" int64_t thc_ring_step_launches(int64_t N) {
    return N > 0 ? ceil_div(step_blocks(N), kStepPiece) : 0;
}

extern "C" size_t thc_ring_step_ws_bytes(int64_t N) {
    const int64_t nblk = step_blocks(N);
    const int64_t ng = nblk > kNmseGroup ? ceil_div(nblk, kNmseGroup) : 0;
    return (size_t)(nblk + ng) * 2 * sizeof(double);
}

extern "C" ga_status thc_ring_step(void* const* bufs, int32_t P, int64_t N, ga_dtype dt, int64_t ring_part,
                                   const float* d_mM, int64_t q_part, int32_t b, uint64_t seed,
                                   int32_t worker0, uint8_t* const* packed, int32_t* d_sum, void* xhat,
                                   double* d_nmse, void* d_ws, size_t ws_bytes, void* stream) {
    const char* what = "thc_ring_step";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    if (b != 1 && b != 2 && b != 4 && b != 8) return fail(GA_EINVAL, "%s: b = %d not in {1, 2, 4, 8}", what, b);
    if (N < 0 || ring_part < 0 || q_part < 0 || worker0 < 0)
        return fail(GA_EINVAL, "%s: negative size or worker", what);
    if (P < 1 || P > GA_MAX_WORKERS)
        return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if ((int64_t)P * ((1 << b) - 1) > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: sums overflow int32", what);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(bufs, P, 16, what);
    if (rc) return rc;
    const int64_t rplen = ring_part > 0 ? ring_part : N, qplen = q_part > 0 ? q_part : N;
    if (N % 8 || qplen % 8)
        return fail(GA_ENOTSUP, "%s: N and the quantizer partition must be multiples of 8 (groups of "
                    "8 elements); use the separate calls", what);
    const int64_t es = (int64_t)elem_size(dt);
    for (int i = 0; i < P; i++)
        for (int j = i + 1; j < P; j++) {
            const uintptr_t a = (uintptr_t)bufs[i], c = (uintptr_t)bufs[j];
            if (a < c + (uintptr_t)(N * es) && c < a + (uintptr_t)(N * es))
                return fail(GA_EINVAL, "%s: worker buffers overlap", what);
        }
    if (!d_mM || !aligned(d_mM, 8)) return fail(GA_EINVAL, "%s: null or misaligned grid", what);
    if (!xhat || !aligned(xhat, 16)) return fail(GA_EINVAL, "%s: null or misaligned estimate", what);
    if (d_sum && !aligned(d_sum, 16)) return fail(GA_EINVAL, "%s: misaligned sums", what);
    if (packed)
        for (int i = 0; i < P; i++)
            if (!packed[i] || !aligned(packed[i], 8))
                return fail(GA_EINVAL, "%s: worker %d: null or misaligned index buffer", what, i);
    if (d_nmse) {
        if (!aligned(d_nmse, 8) || !d_ws || !aligned(d_ws, 8))
            return fail(GA_EINVAL, "%s: null or misaligned NMSE output or workspace", what);
        if (ws_bytes < thc_ring_step_ws_bytes(N))
            return fail(GA_EINVAL, "%s: workspace of %zu bytes, need %zu", what, ws_bytes,
                        thc_ring_step_ws_bytes(N));
    }
    const int64_t nblk = step_blocks(N);
    if (!flat_fits(nblk)) return fail(GA_EINVAL, "%s: N too large", what);
    PtrTable tb{}, tp{};
    for (int i = 0; i < P; i++) {
        tb.p[i] = bufs[i];
        tp.p[i] = packed ? packed[i] : nullptr;
    }
    const Avg avg{(P & (P - 1)) == 0, (float)P, 1.0f / (float)P};
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    double* ws = d_nmse ? static_cast<double*>(d_ws) : nullptr;
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const size_t lds = step_lds(P, 2 * (int64_t)P * N * es);
    const int hp = packed != nullptr;
#define GA_STEP(DT, B, PT, W)                                                                   \
    hipLaunchKernelGGL((thc_ring_kernel<DT, B, PT, W>), flat_grid(nb), dim3(kThreads), lds, hs, tb, tp, hp, \
                       P, worker0, N, rplen, qplen, d_mM, k0, k1, avg, d_sum, xhat, ws, b0)
#define GA_STEP_P(DT, B)                                                                        \
    do {                                                                                        \
        if (P == 8) GA_STEP(DT, B, 8, 5);                                                       \
        else if (P == 16) GA_STEP(DT, B, 16, 3);                                                \
        else GA_STEP(DT, B, 0, 1);                                                              \
    } while (0)
#define GA_LANE(B, PT, KB, W)                                                                   \
    hipLaunchKernelGGL((thc_ring_lane_kernel<B, PT, KB, W>), flat_grid(nb), dim3(kThreads), lds, hs, tb, tp, \
                       hp, P, worker0, N, rplen, qplen, d_mM, k0, k1, avg, d_sum, xhat, ws, b0)
#define GA_LANE_P(B) GA_LANE(B, 0, kLaneBatch, kLaneWaves)
    for (int64_t b0 = 0; b0 < nblk; b0 += kStepPiece) {
        const int64_t nb = std::min(kStepPiece, nblk - b0);
        if (dt == GA_F32) {
            if (b == 1) GA_LANE_P(1); else if (b == 2) GA_LANE_P(2);
            else if (b == 4) GA_LANE_P(4); else GA_LANE_P(8);
        } else {
            if (b == 1) GA_STEP_P(GA_BF16, 1); else if (b == 2) GA_STEP_P(GA_BF16, 2);
            else if (b == 4) GA_STEP_P(GA_BF16, 4); else GA_STEP_P(GA_BF16, 8);
        }
        if ((rc = check_launch(what))) return rc;
    }
#undef GA_LANE_P
#undef GA_LANE
#undef GA_STEP_P
#undef GA_STEP
    if (!d_nmse) return GA_OK;
    if (nblk > kNmseGroup) {                             // two levels
        const int64_t ng = ceil_div(nblk, kNmseGroup);
        hipLaunchKernelGGL(nmse_group_kernel, dim3((unsigned)ng), dim3(kThreads), 0, hs, ws, nblk, ws + 2 * nblk);
        if ((rc = check_launch(what))) return rc;
        hipLaunchKernelGGL(nmse_final_kernel, dim3(1), dim3(kThreads), 0, hs, ws + 2 * nblk, (int)ng, d_nmse);
    } else {
        hipLaunchKernelGGL(nmse_final_kernel, dim3(1), dim3(kThreads), 0, hs, ws, (int)nblk, d_nmse);
    }
    return check_launch(what);
}
