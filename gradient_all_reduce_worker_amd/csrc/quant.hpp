// quant.hpp -- THC's rounding rules shared by the quantizer kernels (thc.hip)
// and the transform-and-quantize kernels (rht.hip): the grid of a
// partition, unbiased stochastic rounding to a uniform grid or to a lookup
// table's neighbouring values ("THC: Accelerating Distributed Deep Learning
// Using Tensor Homomorphic Compression", sections 3 and 4), the 16-bit
// uniforms cut from a Philox4x32-10 block, and LSB-first packing.
#pragma once
#include "common.hpp"
#include "philox.hpp"

namespace ga {
namespace {

struct Grid {                // one partition's grid
    float m;
    float s;                 // L / (M - m), or 0 when M == m
};

__device__ __forceinline__ Grid grid_of(const float* mM, int64_t p, int L) {
    const float m = mM[2 * p], M = mM[2 * p + 1];
    const float range = M - m;
    return {m, range == 0.0f ? 0.0f : (float)L / range};
}

// floor(x) as an int32 in one instruction (the compiler splits it in two
// when subnormals are kept; the arguments below are never subnormal).
__device__ __forceinline__ int floor_i32(float x) {
    int r;
    asm("v_cvt_flr_i32_f32 %0, %1" : "=v"(r) : "v"(x));
    return r;
}

// Stochastic rounding of one value to its grid index, binary32 throughout
// (a >= m, so the position u on the grid is >= 0; with s = 0 the index is
// 0). The rule is: z0 = min(floor(u), L - 1), f = u - z0, go up when
// 2 r + 1 < f 2^17 for the 16-bit uniform r. Computed here in fewer
// instructions with the same result for every finite input in [m, M]:
//  - u is first clamped to [0, L]; u >= L gives index L either way (f >= 1
//    and every r goes up, or f = 0 at z0 = L and none does), and inside the
//    range the clamp changes nothing;
//  - with t = (2 r + 1) 2^-17 (exact), going up is t < f, so
//    z = ceil(u - t) = -floor(t - u): if f > t, u - t lies in
//    (floor u, floor u + 1); if f <= t, in (floor u - 1, floor u].
//    t - u is exact when L < 128: for u >= 1 both are multiples of
//    ulp(u) <= 2^-17 and |t - u| < u; for u < 1 and u >= t likewise; for
//    u < t the rounded difference stays in (0, 1), whose floor is 0 as it
//    should be. It is never subnormal (0, or at least 2^-41 in magnitude).
//  - for L >= 128 (b = 8) t - u can round across an integer, so the
//    decision is made as r < f 2^16 - 1/2 (f 2^16 is exact and so is the
//    subtraction whenever the right side is >= 0), z = trunc(u) + up.
// usq_neg_index returns -z mod 2^32 (L < 128), for packers that add the
// negated indices and negate once per group.
__device__ __forceinline__ float usq_position(float a, Grid g, int L) {
    return __builtin_amdgcn_fmed3f((a - g.m) * g.s, 0.0f, (float)L);
}

__device__ __forceinline__ uint32_t usq_neg_index(float a, Grid g, int L, uint32_t r16) {
    const float u = usq_position(a, g, L);
    const float t = __builtin_fmaf((float)r16, 0x1p-16f, 0x1p-17f);
    return (uint32_t)floor_i32(t - u);
}

__device__ __forceinline__ uint32_t usq_index(float a, Grid g, int L, uint32_t r16) {
    if (L < 128) return 0u - usq_neg_index(a, g, L, r16);
    const float u = usq_position(a, g, L);
    const float f = __builtin_amdgcn_fractf(u);
    const bool up = (float)r16 < __builtin_fmaf(f, 65536.0f, -0.5f);
    return (uint32_t)u + (up ? 1u : 0u);
}

// Lanes 2k and 2k+1 exchange v (DPP quad permute [1, 0, 3, 2]); every lane
// of the wave must take part.
__device__ __forceinline__ uint32_t swap_pair(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, false);
}

__device__ __forceinline__ uint32_t uniform16(const Philox4& r, int i) {
    return (r.v[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
}

// The 8 b-bit indices of a group, least significant bits first (8 b bits).
template <int B>
__device__ __forceinline__ uint64_t pack_group(const uint32_t* z) {
    if (B == 8) {
        const uint32_t lo = z[0] | (z[1] << 8) | (z[2] << 16) | (z[3] << 24);
        const uint32_t hi = z[4] | (z[5] << 8) | (z[6] << 16) | (z[7] << 24);
        return (uint64_t)lo | ((uint64_t)hi << 32);
    }
    // one 32-bit shift-and-or per index (Horner order, most significant first)
    uint32_t acc = z[7];
#pragma unroll
    for (int i = 6; i >= 0; i--) acc = (acc << B) | z[i];
    return acc;
}

// The same from the negated indices w[i] = -z[i] mod 2^32 (B <= 4): the
// Horner sum of the w is -(the packed word) mod 2^32.
template <int B>
__device__ __forceinline__ uint32_t pack_neg_group(const uint32_t* w) {
    static_assert(B <= 4, "8 b-bit indices fit one word");
    uint32_t acc = w[7];
#pragma unroll
    for (int i = 6; i >= 0; i--) acc = (acc << B) + w[i];
    asm("" : "+v"(acc));        // keeps the one negation from being spread over the terms
    return 0u - acc;
}

// Packed indices are written once. Where a store instruction covers whole
// lines across the wave they go out nontemporal (32 x 138M fp32: b = 8
// quantize 3.85 -> 3.46 ms, b = 4 3.38 -> 3.16 ms); where it covers pieces
// of lines that other instructions or workgroups complete (NT = false),
// through L2, which merges them (nontemporal there: RHT second pass +2%).
template <int B, bool NT = true>
__device__ __forceinline__ void store_group(uint8_t* out, int64_t g, uint64_t bits) {
    if (!NT) {
        if (B == 8) *reinterpret_cast<uint2*>(out + 8 * g) = make_uint2((uint32_t)bits, (uint32_t)(bits >> 32));
        else if (B == 4) reinterpret_cast<uint32_t*>(out)[g] = (uint32_t)bits;
        else if (B == 2) reinterpret_cast<uint16_t*>(out)[g] = (uint16_t)bits;
        else out[g] = (uint8_t)bits;
    } else if (B == 8) {
        __builtin_nontemporal_store((unsigned long long)bits, reinterpret_cast<unsigned long long*>(out) + g);
    } else if (B == 4) {
        __builtin_nontemporal_store((uint32_t)bits, reinterpret_cast<uint32_t*>(out) + g);
    } else if (B == 2) {
        __builtin_nontemporal_store((uint16_t)bits, reinterpret_cast<uint16_t*>(out) + g);
    } else {
        __builtin_nontemporal_store((uint8_t)bits, out + g);
    }
}

// Rounding rules. Uniform THC: index k stands for m + k (M - m) / L. Non-
// uniform THC ("THC" page, section 4, Algorithm 2): index z stands for the
// table value T[z] on the finer grid m + t (M - m) / g, and a coordinate is
// rounded stochastically to one of its two neighbouring table values. A
// per-workgroup LDS map cell[k] for every integer cell k in [0, g) gives the
// neighbours of a position u in [k, k + 1): z0 = the largest z with
// T[z] <= k, lo = T[z0] and den = T[z0 + 1] - T[z0], stored as the binary32
// values lo, den (with z0 in its low 8 bits: an integer <= 4095 leaves at
// least 11 low mantissa bits zero) and 1 / den correctly rounded, so that
// one 16-byte LDS read and two masks decode it and no reciprocal is issued
// per coordinate. The cells live in dynamic LDS of table_lds_bytes(g) bytes.
constexpr int kMaxGranularity = 4095;

struct TableArg {
    uint16_t t[256];   // T[0 .. n-1], 0 = T[0] < ... < T[n-1] = g
    int g;
    int n;             // 2^b
};

inline size_t table_lds_bytes(const TableArg& tab) { return (size_t)tab.g * sizeof(uint4); }

template <bool TABLE>
struct Rounder {
    int levels;              // L for the uniform grid, g for a table
    const uint4* cell;       // LDS cells (table only)
    // The index of a; *v receives the grid level it stands for (the index
    // itself, or its table value).
    __device__ __forceinline__ uint32_t index_v(float a, Grid gr, uint32_t r16, float* v) const {
        if (!TABLE) {
            const uint32_t z = usq_index(a, gr, levels, r16);
            *v = (float)z;
            return z;
        }
        const float u = (a - gr.m) * gr.s;                      // position on <g+1>
        // cell min(floor(u), g - 1), u clamped to [0, g - 1] first (same cell
        // for every u >= 0; a value below m takes cell 0)
        const int k = floor_i32(__builtin_amdgcn_fmed3f(u, 0.0f, (float)(levels - 1)));
        const uint4 c = cell[k];
        const float lo = __uint_as_float(c.x), den = __uint_as_float(c.y & ~0xFFu);
        // up <=> r < fl((u - lo) / den) 2^16 - 1/2 (as in usq_index's b = 8
        // form), with a correctly rounded quotient. u - lo and den are exact
        // (integers <= 4095 and u < 2^12). num times the stored reciprocal
        // gives the quotient within 2^-23 relative, i.e. the threshold within
        // 0.01 of the exact one (|quotient| <= 1 + 2^-10); r is an integer, so
        // when it lies more than 1/8 from the estimate the decision is already
        // fixed. Only the rest (about one coordinate in 2.6 10^5) divides.
        const float num = u - lo;
        const float rf = (float)r16;
        const float yq = __builtin_fmaf(num * __uint_as_float(c.z), 65536.0f, -0.5f);
        bool up = rf < yq;
        if (!(fabsf(rf - yq) > 0.125f)) up = rf < __builtin_fmaf(num / den, 65536.0f, -0.5f);
        *v = up ? lo + den : lo;
        return (c.y & 0xFFu) + (up ? 1u : 0u);
    }
    __device__ __forceinline__ uint32_t index(float a, Grid gr, uint32_t r16) const {
        float v;
        return index_v(a, gr, r16, &v);
    }
};

// Called by every thread of the workgroup (NT threads) before any early exit;
// cells: the kernel's dynamic LDS (table_lds_bytes(g) bytes).
template <bool TABLE, int NT = kThreads>
__device__ __forceinline__ Rounder<TABLE> make_rounder(const TableArg& tab, int L, uint4* cells) {
    if (!TABLE) return {L, nullptr};
    for (int k = threadIdx.x; k < tab.g; k += NT) {
        int lo = 0, hi = tab.n - 1;             // the largest z with T[z] <= k
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (tab.t[mid] <= k) lo = mid; else hi = mid - 1;
        }
        const float tl = (float)tab.t[lo], den = (float)(tab.t[lo + 1] - tab.t[lo]);
        cells[k] = make_uint4(__float_as_uint(tl), __float_as_uint(den) | (uint32_t)lo,
                              __float_as_uint(1.0f / den), 0u);
    }
    __syncthreads();
    return {tab.g, cells};
}

inline bool valid_bits(int b) { return b == 1 || b == 2 || b == 4 || b == 8; }

// Host check of a non-uniform table: 0 = T[0] < ... < T[2^b - 1] = g,
// 2^b - 1 <= g <= kMaxGranularity.
inline ga_status load_table(int32_t b, int32_t g, const int32_t* h_table, TableArg* tab, const char* what) {
    if (!valid_bits(b)) return fail(GA_EINVAL, "%s: b = %d is not 1, 2, 4 or 8", what, b);
    if (!h_table) return fail(GA_EINVAL, "%s: null table", what);
    const int n = 1 << b;
    if (g < n - 1) return fail(GA_EINVAL, "%s: granularity %d < 2^b - 1", what, g);
    if (g > kMaxGranularity)
        return fail(GA_ENOTSUP, "%s: granularity %d above the supported %d", what, g, kMaxGranularity);
    if (h_table[0] != 0 || h_table[n - 1] != g)
        return fail(GA_EINVAL, "%s: table must start at 0 and end at g", what);
    *tab = TableArg{};
    for (int z = 0; z < n; z++) {
        if (z > 0 && h_table[z] <= h_table[z - 1])
            return fail(GA_EINVAL, "%s: table not strictly increasing at %d", what, z);
        tab->t[z] = (uint16_t)h_table[z];
    }
    tab->g = g;
    tab->n = n;
    return GA_OK;
}

}  // namespace
}  // namespace ga
