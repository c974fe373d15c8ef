// rht.hip -- randomized Hadamard transform pre/post-processing for THC
// ("THC: Accelerating Distributed Deep Learning Using Tensor Homomorphic
// Compression", section 5): RHT(x) = H D x / sqrt(d), RHT^-1(y) = D H y /
// sqrt(d) on blocks of d = 2^k coordinates, the per-block norms, the
// norm-based range M = t_p max_i ||x_i|| / sqrt(d), m = -M, and truncation.
//
// The transform is the textbook radix-2 one: stage s = 0 .. k-1 turns every
// pair (i, i + 2^s), bit s of i clear, into (a + b, a - b) in binary32, and
// the result is scaled by fl32(1/sqrt(d)) at the end. Stages on different
// bits do not commute in floating point, so they run strictly in that order.
//
// Layout of the work (512-thread workgroups, an 8192-coordinate tile of
// 32 KiB in LDS, padded against bank conflicts (pad() below); three or four
// workgroups fit a CU, so one loads while another computes):
//  * tile pass: a workgroup loads 8192 consecutive coordinates (several
//    whole blocks when d < 8192) and runs stages 0 .. log2(T) - 1 with
//    T = min(d, 8192);
//  * cross pass (d > 8192 only): a workgroup loads a G x W sub-matrix of
//    one block (G = d / 8192 rows spaced 8192 apart, W = 8192 / G >= 16
//    consecutive columns) and runs the remaining stages along the rows.
// Inside a pass, stages go four at a time through registers: every thread
// takes the 16 coordinates that differ only in four consecutive index bits,
// runs the stages on those bits, and writes them back (one LDS round trip
// per four stages; the passes of the blocks above 8192 coordinates run
// their first four stages on values loaded straight from memory and their
// tile pass's last stage on the way out). Each butterfly adds and
// subtracts the same two values as the plain loop, so the output is
// bit-for-bit that loop's.
//
// The Rademacher signs come from Philox4x32-10: key (seed), counter
// (q mod 2^32, q >> 32, 0x52485400, 0) with q = e / 128; coordinate e takes
// bit e mod 32 of output word (e / 32) mod 4, a set bit meaning -1. A
// workgroup first computes the Philox blocks it needs into LDS.
#include <cmath>

#include "common.hpp"
#include "philox.hpp"
#include "quant.hpp"

namespace ga {
namespace {

constexpr int kTileBits = 13;
constexpr int kTile = 1 << kTileBits;       // coordinates per LDS tile
constexpr int kTT = 512;                    // threads per transform workgroup
constexpr int kPer = kTile / kTT;           // coordinates per thread (16)
constexpr int kLds = kTile + kTile / 32 + 8 * (kTile / 256);   // padded tile, in words
constexpr int kMaxBits = 22;                // d <= 2^22: G <= 512, W >= 16
// blocks per chunk of the pipelined two-pass transform-and-quantize (32
// workers x 138M fp32, d = 2^20: 64 -> 12.5 ms, 128 -> 12.1, 256 -> 12.0,
// 512 -> 12.5; fewer launches against longer unpaired first and last ones).
// Chunks whose transformed vectors would fit the 256 MB Infinity Cache
// between the two passes (16 or 32 blocks: 64 or 128 MiB) take 13.8 ms:
// the second pass does not get its input from the cache, and the launches
// multiply.
constexpr int64_t kPipeUnits = 256;
constexpr int kSignWords = 4 * 512;         // Philox blocks a workgroup may need, x 4
static_assert(kPer == 16, "one set of 16 coordinates per thread and group");
constexpr uint32_t kSignDomain = 0x52485400u;

// LDS word of tile index i. The LDS serves a wave's 32-bit accesses one
// half-wave at a time over 32 banks (measured on gfx950: lanes 0-31 over
// words 0-15 and 32-47 take two passes, lanes 0-31 over words 0-31 and
// lanes 32-63 over 64-95 one). One word per 32 keeps 32 consecutive indices
// on 32 banks (the loads, stores and rounding reads); eight more per 256
// separate the half-wave's two rows in the 16-stride passes (indices
// 0-15 and 256-271). Of the transform's patterns only a thread's 16
// consecutive stores (first pass) still meet two to a bank. A sum of
// shifted copies of i splits over disjoint bits: pad(a + b) = pad(a) +
// pad(b) when a and b share no set bit, so a thread's 16 words are one
// register plus immediate offsets.
__host__ __device__ constexpr int pad(int i) { return i + (i >> 5) + 8 * (i >> 8); }
static_assert(pad(kTile - 1) < kLds, "the padded tile fits");

// pad(o + k kTT) for thread o < kTT, given po = pad(o): o and k kTT share
// no set bit (kTT a power of two), so the sum is split at compile time.
__device__ __forceinline__ int pad_at(int po, int k) { return po + pad(k * kTT); }

__device__ __forceinline__ float load_coord(const void* x, int64_t e, int64_t N, ga_dtype dt) {
    if (e >= N) return 0.0f;                 // zero padding to a whole block
    if (dt == GA_BF16) return __uint_as_float((uint32_t) static_cast<const uint16_t*>(x)[e] << 16);
    return static_cast<const float*>(x)[e];
}

// Stages on index bits LO .. HI-1 of the tile in LDS (WB <= LO < HI <= WB + 4,
// WB <= kTileBits - 4): thread o takes the 16 coordinates whose index bits
// WB .. WB+3 vary and whose other bits spell o. With WB fixed at compile
// time the 16 LDS addresses are one register plus immediate offsets; with
// LO and HI fixed too, every butterfly is straight-line code.
// The stages on bits LO .. HI-1 applied to 16 coordinates held in
// registers, v[r] being coordinate base + (r << WB): stage WB + q pairs
// v[r] with v[r | 2^q].
template <int WB, int LO, int HI>
__device__ __forceinline__ void butterflies(float* v) {
#pragma unroll
    for (int q = 0; q < 4; q++) {
        if (WB + q >= LO && WB + q < HI) {
            const int h = 1 << q;
#pragma unroll
            for (int r = 0; r < 16; r++) {
                if (!(r & h)) {
                    const float a = v[r], b = v[r | h];
                    v[r] = a + b;
                    v[r | h] = a - b;
                }
            }
        }
    }
}

// LDS index of thread o's first coordinate in a group16<WB> pass; bits
// WB .. WB+3 of it are clear, so coordinate r of the thread sits at
// pad(base) + pad(r << WB).
template <int WB>
__device__ __forceinline__ int group_base(int o) {
    return ((o >> WB) << (WB + 4)) | (o & ((1 << WB) - 1));
}

template <int WB, int LO, int HI>
__device__ __forceinline__ void group16(float* s) {
    float* p = s + pad(group_base<WB>(threadIdx.x));
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; r++) v[r] = p[pad(r << WB)];
    butterflies<WB, LO, HI>(v);
#pragma unroll
    for (int r = 0; r < 16; r++) p[pad(r << WB)] = v[r];
}

// Stages on index bits LO .. HI-1, four at a time, a barrier after each group.
template <int LO, int HI>
__device__ __forceinline__ void stages_ct(float* s) {
    if constexpr (LO < HI) {
        constexpr int WB = LO < kTileBits - 4 ? LO : kTileBits - 4;
        constexpr int H = LO + 4 < HI ? LO + 4 : HI;
        group16<WB, LO, H>(s);
        __syncthreads();
        stages_ct<LO + 4, HI>(s);
    }
}

// The two shapes in use: bits 0 .. hi-1 (a tile pass, 1 <= hi <= kTileBits)
// and bits lo .. kTileBits-1 (a cross pass, 4 <= lo < kTileBits).
__device__ __forceinline__ void stages(float* s, int lo, int hi) {
    if (lo == 0) {
        switch (hi) {
            case 1: stages_ct<0, 1>(s); break;
            case 2: stages_ct<0, 2>(s); break;
            case 3: stages_ct<0, 3>(s); break;
            case 4: stages_ct<0, 4>(s); break;
            case 5: stages_ct<0, 5>(s); break;
            case 6: stages_ct<0, 6>(s); break;
            case 7: stages_ct<0, 7>(s); break;
            case 8: stages_ct<0, 8>(s); break;
            case 9: stages_ct<0, 9>(s); break;
            case 10: stages_ct<0, 10>(s); break;
            case 11: stages_ct<0, 11>(s); break;
            case 12: stages_ct<0, 12>(s); break;
            default: stages_ct<0, kTileBits>(s); break;
        }
        return;
    }
    switch (lo) {
        case 4: stages_ct<4, kTileBits>(s); break;
        case 5: stages_ct<5, kTileBits>(s); break;
        case 6: stages_ct<6, kTileBits>(s); break;
        case 7: stages_ct<7, kTileBits>(s); break;
        case 8: stages_ct<8, kTileBits>(s); break;
        case 9: stages_ct<9, kTileBits>(s); break;
        case 10: stages_ct<10, kTileBits>(s); break;
        case 11: stages_ct<11, kTileBits>(s); break;
        default: stages_ct<12, kTileBits>(s); break;
    }
}

// Philox blocks q0 .. q0 + nq - 1 of the sign stream into LDS.
__device__ __forceinline__ void sign_blocks(uint32_t* words, int64_t q0, int nq, uint32_t k0,
                                            uint32_t k1) {
    for (int t = threadIdx.x; t < nq; t += kTT) {
        const uint64_t q = (uint64_t)(q0 + t);
        const Philox4 r = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), kSignDomain, 0u, k0, k1);
        words[4 * t + 0] = r.v[0];
        words[4 * t + 1] = r.v[1];
        words[4 * t + 2] = r.v[2];
        words[4 * t + 3] = r.v[3];
    }
}

// Sign bit of a coordinate from its Philox block (index blk in words) and
// any integer congruent to its index modulo 128.
__device__ __forceinline__ bool negated(const uint32_t* words, int blk, int e) {
    return (words[4 * blk + ((e >> 5) & 3)] >> (e & 31)) & 1u;
}

// v clamped to [m, M] (one median-of-three; the same value for every
// finite v, as m <= M)
__device__ __forceinline__ float clamp_to(float v, const float* mM, int64_t p) {
    return __builtin_amdgcn_fmed3f(v, mM[2 * p], mM[2 * p + 1]);
}


// ---------------------------------------------------------------- tile pass

// Coordinate e0 + i of a worker's input: x (fp32 or bf16) for the forward
// transform, the fp32 transformed vector for the inverse.
template <bool FWD, ga_dtype DT>
__device__ __forceinline__ float load_tile(const void* x, int64_t e0, int i) {
    if (FWD && DT == GA_BF16)
        return __uint_as_float((uint32_t)(static_cast<const uint16_t*>(x) + e0)[i] << 16);
    return (static_cast<const float*>(x) + e0)[i];
}

// Tile pass over n = min(kTile, Np - e0) consecutive coordinates (a whole
// number of blocks when d < kTile, one tile of a block otherwise): stages
// 0 .. kbits-1, kbits = log2(min(d, kTile)).
// FWD: apply the signs on load; else (inverse) on the final store.
// FINAL (d <= kTile): scale, then clamp (forward, mM given) or sign
// (inverse) and store; else store the partial transform for the cross pass.
template <bool FWD, bool FINAL, ga_dtype DT>
__global__ __launch_bounds__(kTT) void rht_tile_kernel(PtrTable x, PtrTable y, int64_t N, int64_t Np,
                                                       int kbits, uint32_t k0, uint32_t k1, float c,
                                                       const float* __restrict__ mM) {
    __shared__ float s[kLds];
    __shared__ uint32_t words[4 * (kTile / 128)];
    const int w = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * kTile;  // a multiple of 128
    const int n = (int)min((int64_t)kTile, Np - e0);  // coordinates of this tile
    const int nx = (int)max((int64_t)0, min((int64_t)kTile, N - e0));   // ... that exist in x
    if (FWD || FINAL) sign_blocks(words, e0 >> 7, (n + 127) >> 7, k0, k1);
    // all loads first, unconditionally on a full tile, so they are in flight together
    float v[kPer];
    const int lim = FWD ? nx : n;
    if (lim == kTile) {
#pragma unroll
        for (int k = 0; k < kPer; k++) v[k] = load_tile<FWD, DT>(x.p[w], e0, threadIdx.x + k * kTT);
    } else {
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            const int i = threadIdx.x + k * kTT;
            v[k] = i < lim ? load_tile<FWD, DT>(x.p[w], e0, i) : 0.0f;
        }
    }
    __syncthreads();                                  // the sign words
    const int po = pad(threadIdx.x);
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int i = threadIdx.x + k * kTT;
        s[pad_at(po, k)] = FWD && negated(words, i >> 7, i) ? -v[k] : v[k];
    }
    __syncthreads();
    stages(s, 0, kbits);
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int i = threadIdx.x + k * kTT;
        float r = s[pad_at(po, k)];
        if (!FINAL) {
            if (i < n) (static_cast<float*>(y.p[w]) + e0)[i] = r;
        } else if (FWD) {
            if (i < n) {
                r = r * c;
                if (mM) r = clamp_to(r, mM, (e0 + i) >> kbits);
                (static_cast<float*>(y.p[w]) + e0)[i] = r;
            }
        } else if (i < nx) {
            r = r * c;
            if (negated(words, i >> 7, i)) r = -r;
            if (DT == GA_F32) (static_cast<float*>(y.p[w]) + e0)[i] = r;
            else (static_cast<uint16_t*>(y.p[w]) + e0)[i] = (uint16_t)f32_to_bf16_rne(r);
        }
    }
}

// ---------------------------------------------------------------- cross pass

// Rows j = 0 .. G-1 of block b at stride kTile, columns c0 .. c0+W-1
// (W = 2^wbits >= 16): stages on the row bits, i.e. LDS index bits
// wbits .. kTileBits-1. FWD: scale and clamp; else scale, sign, write out.
template <bool FWD, ga_dtype OUT>
__global__ __launch_bounds__(kTT) void rht_cross_kernel(PtrTable y, PtrTable out, int64_t N, int dbits,
                                                        int wbits, uint32_t k0, uint32_t k1, float c,
                                                        const float* __restrict__ mM) {
    __shared__ float s[kLds];
    __shared__ uint32_t words[FWD ? 1 : kSignWords];
    const int w = blockIdx.y;
    const int W = 1 << wbits;
    const int gbits = dbits - kTileBits;             // G = 2^gbits rows
    const int G = 1 << gbits;
    const int64_t b = blockIdx.x >> gbits;
    const int64_t base = (b << dbits) + (int64_t)(blockIdx.x & (G - 1)) * W;   // a multiple of 16
    float* yb = static_cast<float*>(y.p[w]) + base;
    const int po = pad(threadIdx.x);
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int i = threadIdx.x + k * kTT;
        s[pad_at(po, k)] = yb[(i >> wbits) * kTile + (i & (W - 1))];
    }
    // inverse: the Philox blocks of every (row, 128-column group); R per row
    const int R = W >= 128 ? W >> 7 : 1;
    if (!FWD) {
        for (int t = threadIdx.x; t < G * R; t += kTT) {
            const int j = t / R, gi = t % R;
            const uint64_t q = (uint64_t)(((base + (int64_t)j * kTile) >> 7) + gi);
            const Philox4 r = philox4x32_10((uint32_t)q, (uint32_t)(q >> 32), kSignDomain, 0u, k0, k1);
            words[4 * t + 0] = r.v[0];
            words[4 * t + 1] = r.v[1];
            words[4 * t + 2] = r.v[2];
            words[4 * t + 3] = r.v[3];
        }
    }
    __syncthreads();
    stages(s, wbits, kTileBits);
    const int nb = (int)min(N - base, (int64_t)1 << 30);   // inverse: offsets below nb exist
    const int eb = (int)(base & 127);
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int i = threadIdx.x + k * kTT;
        const int j = i >> wbits, col = i & (W - 1);
        const int off = j * kTile + col;
        float v = s[pad_at(po, k)] * c;
        if (FWD) {
            yb[off] = mM ? clamp_to(v, mM, b) : v;
        } else if (off < nb) {
            if (negated(words, j * R + (col >> 7), eb + col)) v = -v;
            if (OUT == GA_F32) (static_cast<float*>(out.p[w]) + base)[off] = v;
            else (static_cast<uint16_t*>(out.p[w]) + base)[off] = (uint16_t)f32_to_bf16_rne(v);
        }
    }
}

// ---------------------------------------------------------------- transform and quantize

// THC's RHT variant quantizes the truncated transform (THC page, section 5,
// then section 3 or 4 on the result). These kernels take the transform's
// last pass and, instead of writing the binary32 coordinates, round them
// at once: the same clamp to [m_p, M_p], the same grid (the block is the
// quantizer's partition), the same Philox counters (coordinate index in the
// transformed vector, worker, seed) and packing as thc_rht_forward followed
// by thc_usq_quantize / thc_nuhc_quantize, so the indices are identical;
// the transformed vector is never written.

// Range and grid of one block, read once for the coordinates that share it.
struct BlockGrid {
    float m, M;
    Grid g;
};

__device__ __forceinline__ BlockGrid block_grid(const float* mM, int64_t p, int levels) {
    return {mM[2 * p], mM[2 * p + 1], grid_of(mM, p, levels)};
}

// 8 consecutive coordinates from LDS (index i0 on, coordinate e on),
// scaled, clamped and rounded on the grid of their block bg.
template <int B, bool TABLE>
__device__ __forceinline__ uint64_t round_group(const float* s, int i0, int64_t e, float c,
                                                const BlockGrid& bg, const Rounder<TABLE>& rd,
                                                uint32_t wid, uint32_t q0, uint32_t q1) {
    const uint64_t g = (uint64_t)e >> 3;
    const Philox4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), wid, 0u, q0, q1);
    const float* q = s + pad(i0);                    // i0 a multiple of 8: pad(i0 + i) = pad(i0) + i
    uint32_t z[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        const float v = __builtin_amdgcn_fmed3f(q[i] * c, bg.m, bg.M);   // clamp
        z[i] = rd.index(v, bg.g, uniform16(r, i));
    }
    return pack_group<B>(z);
}

// As round_group when the n_in <= 8 coordinates may lie in different
// blocks (d < 8): range and grid per coordinate; indices past n_in are 0.
template <int B, bool TABLE>
__device__ __forceinline__ uint64_t round_group_mixed(const float* s, int i0, int n_in, int64_t e,
                                                      int dbits, float c, const float* mM,
                                                      const Rounder<TABLE>& rd, uint32_t wid,
                                                      uint32_t q0, uint32_t q1) {
    const uint64_t g = (uint64_t)e >> 3;
    const Philox4 r = philox4x32_10((uint32_t)g, (uint32_t)(g >> 32), wid, 0u, q0, q1);
    const float* q = s + pad(i0);                    // i0 a multiple of 8
    uint32_t z[8];
#pragma unroll
    for (int i = 0; i < 8; i++) {
        if (i < n_in) {
            const int64_t blk = (e + i) >> dbits;
            const float v = clamp_to(q[i] * c, mM, blk);
            z[i] = rd.index(v, grid_of(mM, blk, rd.levels), uniform16(r, i));
        } else {
            z[i] = 0u;                               // past the vector's end: index 0
        }
    }
    return pack_group<B>(z);
}

// Single pass (d <= kTile): tile of n coordinates from e0, every stage in
// LDS, then groups of 8 rounded and packed (two groups per thread).
template <ga_dtype DT, int B, bool TABLE>
__global__ __launch_bounds__(kTT) void rht_tile_quant_kernel(PtrTable x, PtrTable packed, int worker0,
                                                             int64_t N, int64_t Np, int kbits,
                                                             uint32_t k0, uint32_t k1, float c,
                                                             const float* __restrict__ mM,
                                                             uint32_t q0, uint32_t q1, TableArg tab) {
    constexpr int L = (1 << B) - 1;
    __shared__ float s[kLds];
    __shared__ uint32_t words[4 * (kTile / 128)];
    extern __shared__ uint4 dyn_cells[];              // table cells (table_lds_bytes)
    const Rounder<TABLE> rd = make_rounder<TABLE, kTT>(tab, L, dyn_cells);
    const int w = blockIdx.y;
    const int64_t e0 = (int64_t)blockIdx.x * kTile;
    const int n = (int)min((int64_t)kTile, Np - e0);
    const int nx = (int)max((int64_t)0, min((int64_t)kTile, N - e0));
    sign_blocks(words, e0 >> 7, (n + 127) >> 7, k0, k1);
    float v[kPer];
    if (nx == kTile) {
#pragma unroll
        for (int k = 0; k < kPer; k++) v[k] = load_tile<true, DT>(x.p[w], e0, threadIdx.x + k * kTT);
    } else {
#pragma unroll
        for (int k = 0; k < kPer; k++) {
            const int i = threadIdx.x + k * kTT;
            v[k] = i < nx ? load_tile<true, DT>(x.p[w], e0, i) : 0.0f;
        }
    }
    __syncthreads();                                  // the sign words
    const int po = pad(threadIdx.x);
#pragma unroll
    for (int k = 0; k < kPer; k++) {
        const int i = threadIdx.x + k * kTT;
        s[pad_at(po, k)] = negated(words, i >> 7, i) ? -v[k] : v[k];
    }
    __syncthreads();
    stages(s, 0, kbits);
    uint8_t* out = static_cast<uint8_t*>(packed.p[w]);
    const int64_t nbytes = (Np * B + 7) / 8;
    const uint32_t wid = (uint32_t)(worker0 + w);
#pragma unroll
    for (int k = 0; k < kPer / 8; k++) {
        const int i0 = 8 * (threadIdx.x + k * kTT);
        if (i0 >= n) continue;
        const int n_in = min(8, n - i0);
        const int64_t e = e0 + i0;
        const uint64_t bits =
            kbits >= 3 ? round_group<B, TABLE>(s, i0, e, c, block_grid(mM, e >> kbits, rd.levels), rd, wid, q0, q1)
                       : round_group_mixed<B, TABLE>(s, i0, n_in, e, kbits, c, mM, rd, wid, q0, q1);
        if (n_in == 8) {
            store_group<B>(out, e >> 3, bits);
        } else {
#pragma unroll
            for (int q = 0; q < B; q++)
                if ((e >> 3) * B + q < nbytes) out[(e >> 3) * B + q] = (uint8_t)(bits >> (8 * q));
        }
    }
}

// First pass of the forward transform for one tile (d > kTile): the
// unscaled partial transform over index bits 0 .. kTileBits-1, stored to y
// (as rht_tile_kernel<true, false>). Thread o loads the 16 consecutive
// coordinates 16o .. 16o+15 (16-byte loads when vec), whose signs are 16
// bits of one Philox word, and runs stages 0-3 in registers before the
// first LDS store; stages 4-11 go through LDS and stage 12 is applied on
// the way out (a thread holds both coordinates of its last butterflies).
// wbits = 0: y in the vector's order. wbits > 0 (scratch for the second
// pass of blocks of G = 2^(kTileBits - wbits) tiles): column-blocked, so
// that each second-pass workgroup reads one contiguous run. Within a block,
// column i of tile (row) j sits at (i >> wbits) kTile + j W + (i mod W),
// W = 2^wbits: the G x W sub-matrix of column group i >> wbits is one
// kTile-long run. Written and read once, in whole lines, both nontemporal.
// Measured on 32 x 138M fp32, d = 2^20, table b = 4 (uniform b = 4), builds
// in alternating processes on one machine: the vector's order 12.1 (12.7) ms;
// column-blocked 11.8 (12.4); its stores nontemporal 11.0 (11.8); loads too
// 11.0 (11.2).
template <ga_dtype DT>
__device__ __forceinline__ void forward_tile_body(float* s, uint32_t* words, const void* x, float* y,
                                                  int64_t tile, int64_t N, bool vec, uint32_t k0,
                                                  uint32_t k1, double* norm = nullptr, int wbits = 0) {
    const int64_t e0 = tile * kTile;
    const int nx = (int)max((int64_t)0, min((int64_t)kTile, N - e0));
    const int i0 = 16 * threadIdx.x;
    sign_blocks(words, e0 >> 7, kTile >> 7, k0, k1);
    float v[16];
    if (vec && nx == kTile) {
        if (DT == GA_BF16) {
            const uint4* src = reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(x) + e0 + i0);
#pragma unroll
            for (int h = 0; h < 2; h++) {
                const uint4 q = src[h];
                const uint32_t w4[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
                for (int k = 0; k < 4; k++) {
                    v[8 * h + 2 * k] = __uint_as_float(w4[k] << 16);
                    v[8 * h + 2 * k + 1] = __uint_as_float(w4[k] & 0xFFFF0000u);
                }
            }
        } else {
            const float4* src = reinterpret_cast<const float4*>(static_cast<const float*>(x) + e0 + i0);
#pragma unroll
            for (int h = 0; h < 4; h++) {
                const float4 q = src[h];
                v[4 * h] = q.x;
                v[4 * h + 1] = q.y;
                v[4 * h + 2] = q.z;
                v[4 * h + 3] = q.w;
            }
        }
    } else {
#pragma unroll
        for (int r = 0; r < 16; r++) v[r] = i0 + r < nx ? load_tile<true, DT>(x, e0, i0 + r) : 0.0f;
    }
    if (norm) {
        // the tile's sum of squares of x (binary64, exact squares; a fixed
        // tree over the workgroup), for the block norms
        double acc = 0.0;
#pragma unroll
        for (int r = 0; r < 16; r++) acc += (double)v[r] * (double)v[r];
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
        __shared__ double sh[kTT / 64];
        if ((threadIdx.x & 63) == 0) sh[threadIdx.x >> 6] = acc;
        __syncthreads();
        if (threadIdx.x == 0) {
            double t = 0.0;
            for (int q = 0; q < kTT / 64; q++) t += sh[q];
            *norm = t;
        }
    }
    __syncthreads();                                  // the sign words
    const uint32_t sw = words[4 * (i0 >> 7) + ((i0 >> 5) & 3)] >> (i0 & 31);
#pragma unroll
    for (int r = 0; r < 16; r++)
        if ((sw >> r) & 1u) v[r] = -v[r];
    butterflies<0, 0, 4>(v);
    float* p = s + pad(i0);
#pragma unroll
    for (int r = 0; r < 16; r++) p[r] = v[r];
    __syncthreads();
    stages_ct<4, kTileBits - 1>(s);
    const int po = pad(threadIdx.x);
    if (wbits == 0) {
#pragma unroll
        for (int k = 0; k < kPer / 2; k++) {
            const int i = threadIdx.x + k * kTT;        // < kTile / 2
            const float a = s[pad_at(po, k)], b = s[pad_at(po, k) + pad(kTile / 2)];
            (y + e0)[i] = a + b;
            (y + e0)[i + kTile / 2] = a - b;
        }
    } else {
        const int W = 1 << wbits;
        const int j = (int)(tile & ((1 << (kTileBits - wbits)) - 1));      // row in the block
        float* yb = y + (e0 - (int64_t)j * kTile) + j * W;                 // the block, row j
        const int half = (kTile / 2) >> wbits;                             // column groups to i + kTile / 2
#pragma unroll
        for (int k = 0; k < kPer / 2; k++) {
            const int i = threadIdx.x + k * kTT;
            const float a = s[pad_at(po, k)], b = s[pad_at(po, k) + pad(kTile / 2)];
            const int off = (i >> wbits) * kTile + (i & (W - 1));
            __builtin_nontemporal_store(a + b, yb + off);      // read once, by the second pass
            __builtin_nontemporal_store(a - b, yb + off + half * kTile);
        }
    }
}

template <ga_dtype DT>
__global__ __launch_bounds__(kTT) void rht_forward_tile_kernel(PtrTable x, PtrTable y, int64_t N,
                                                               int vec, uint32_t k0, uint32_t k1) {
    __shared__ float s[kLds];
    __shared__ uint32_t words[4 * (kTile / 128)];
    const int w = blockIdx.y;
    forward_tile_body<DT>(s, words, x.p[w], static_cast<float*>(y.p[w]), blockIdx.x, N, vec != 0,
                          k0, k1);
}

// Second pass (d > kTile): as rht_cross_kernel on rows j = 0 .. G-1 of
// block b, columns cg W .. cg W + W - 1 (W = 2^WBITS >= 16), then the G x W
// sub-matrix rounded in groups of 8 consecutive columns of a row. The first
// four stages (row bits) run in registers on coordinates loaded straight
// from y, which the first pass left column-blocked: the sub-matrix is one
// contiguous run of kTile values, row after row; thread o takes 16 rows of
// one column, so each load instruction reads consecutive values across the
// wave.
template <int B, bool TABLE, int WBITS>
__device__ __forceinline__ void cross_quant_body(float* s, const Rounder<TABLE>& rd, const float* y,
                                                 uint8_t* out, uint32_t wid, int64_t b, int cg,
                                                 int dbits, float c, const float* mM, uint32_t q0,
                                                 uint32_t q1) {
    constexpr int W = 1 << WBITS;
    constexpr int WB = WBITS < kTileBits - 4 ? WBITS : kTileBits - 4;
    constexpr int H1 = WB + 4;                        // first pass: bits WBITS .. H1-1
    const int64_t base = (b << dbits) + (int64_t)cg * W;             // row 0, column cg W
    const float* yb = y + (b << dbits) + (int64_t)cg * kTile;         // the sub-matrix's run
    const int lb = group_base<WB>(threadIdx.x);
    float v[16];
#pragma unroll
    for (int r = 0; r < 16; r++) v[r] = __builtin_nontemporal_load(yb + lb + (r << WB));
    butterflies<WB, WBITS, H1>(v);
    float* p = s + pad(lb);
#pragma unroll
    for (int r = 0; r < 16; r++) p[pad(r << WB)] = v[r];
    __syncthreads();
    stages_ct<H1, kTileBits>(s);
    const BlockGrid bg = block_grid(mM, b, rd.levels);   // one block per workgroup
#pragma unroll
    for (int k = 0; k < kPer / 8; k++) {
        const int i0 = 8 * (threadIdx.x + k * kTT);
        const int64_t e = base + (int64_t)(i0 >> WBITS) * kTile + (i0 & (W - 1));
        store_group<B, false>(out, e >> 3, round_group<B, TABLE>(s, i0, e, c, bg, rd, wid, q0, q1));
    }
}

template <int B, bool TABLE>
__device__ __forceinline__ void cross_quant_dispatch(float* s, const Rounder<TABLE>& rd, const float* y,
                                                     uint8_t* out, uint32_t wid, int64_t b, int cg,
                                                     int dbits, float c, const float* mM, uint32_t q0,
                                                     uint32_t q1) {
    switch (2 * kTileBits - dbits) {                  // W = kTile / G
        case 4: cross_quant_body<B, TABLE, 4>(s, rd, y, out, wid, b, cg, dbits, c, mM, q0, q1); break;
        case 5: cross_quant_body<B, TABLE, 5>(s, rd, y, out, wid, b, cg, dbits, c, mM, q0, q1); break;
        case 6: cross_quant_body<B, TABLE, 6>(s, rd, y, out, wid, b, cg, dbits, c, mM, q0, q1); break;
        case 7: cross_quant_body<B, TABLE, 7>(s, rd, y, out, wid, b, cg, dbits, c, mM, q0, q1); break;
        case 8: cross_quant_body<B, TABLE, 8>(s, rd, y, out, wid, b, cg, dbits, c, mM, q0, q1); break;
        case 9: cross_quant_body<B, TABLE, 9>(s, rd, y, out, wid, b, cg, dbits, c, mM, q0, q1); break;
        case 10: cross_quant_body<B, TABLE, 10>(s, rd, y, out, wid, b, cg, dbits, c, mM, q0, q1); break;
        case 11: cross_quant_body<B, TABLE, 11>(s, rd, y, out, wid, b, cg, dbits, c, mM, q0, q1); break;
        default: cross_quant_body<B, TABLE, 12>(s, rd, y, out, wid, b, cg, dbits, c, mM, q0, q1); break;
    }
}

// Both passes of blocks above kTile, software-pipelined over launches: the
// blocks (units u = worker * nblk + block) are cut into consecutive chunks,
// and one launch runs the first pass of chunk k (units a0 .. a0+na-1) next
// to the second pass of chunk k - 1 (units b0 .. b0+nb-1), whose first pass
// the previous launch finished. The two roles touch disjoint parts of y.
// The first pass is bound by HBM and the second by the rounding arithmetic,
// so sharing the CUs overlaps them. Each unit has G = d / kTile
// workgroups per role; workgroups alternate roles while both have work.
template <ga_dtype DT, int B, bool TABLE>
__global__ __launch_bounds__(kTT) void rht_quant_pipe_kernel(PtrTable x, PtrTable y, PtrTable packed,
                                                             int worker0, int64_t N, int vec, int dbits,
                                                             int64_t nblk, int64_t a0, int64_t na,
                                                             int64_t b0, int64_t nb, uint32_t k0,
                                                             uint32_t k1, float c,
                                                             const float* __restrict__ mM,
                                                             uint32_t q0, uint32_t q1, TableArg tab,
                                                             int P, double* norms) {
    constexpr int L = (1 << B) - 1;
    constexpr int kAux = 4 * (kTile / 128);
    __shared__ float s[kLds];
    __shared__ uint32_t aux[kAux];                   // sign words (first pass)
    extern __shared__ uint4 dyn_cells[];              // table cells (second pass)
    const int gbits = dbits - kTileBits;
    const int64_t nA = na << gbits, nB = nb << gbits;
    const int64_t i = blockIdx.x, both = 2 * min(nA, nB);
    bool first;
    int64_t j;
    if (i < both) {
        first = (i & 1) == 0;
        j = i >> 1;
    } else {
        first = nA > nB;
        j = i - both + min(nA, nB);
    }
    const int64_t unit = (first ? a0 : b0) + (j >> gbits);
    // units worker-major (w nblk + b), or block-major (b P + w) when the
    // first pass also sums the squares of the tiles (norms: per unit, G
    // partial sums; a chunk then holds every worker of its blocks)
    int w;
    int64_t b;
    if (norms) {
        b = unit / P;
        w = (int)(unit - b * P);
    } else {
        w = (int)(unit / nblk);
        b = unit - (int64_t)w * nblk;
    }
    const int r = (int)(j & ((1 << gbits) - 1));
    if (first) {
        forward_tile_body<DT>(s, aux, x.p[w], static_cast<float*>(y.p[w]), (b << gbits) + r, N,
                              vec != 0, k0, k1, norms ? norms + (unit << gbits) + r : nullptr,
                              2 * kTileBits - dbits);
    } else {
        const Rounder<TABLE> rd = make_rounder<TABLE, kTT>(tab, L, dyn_cells);
        cross_quant_dispatch<B, TABLE>(s, rd, static_cast<const float*>(y.p[w]),
                                       static_cast<uint8_t*>(packed.p[w]), (uint32_t)(worker0 + w), b, r,
                                       dbits, c, mM, q0, q1);
    }
}

// ---------------------------------------------------------------- norms and range

// One workgroup per (block, worker): 16 coalesced loads in flight per thread,
// squares summed in binary64 (exact products), then a tree over the threads.
template <ga_dtype DT>
__global__ __launch_bounds__(kThreads) void rht_sumsq_kernel(PtrTable x, int64_t N, int dbits,
                                                             int64_t nblk, double* sumsq) {
    const int w = blockIdx.y;
    const int64_t b = flat_block();
    if (b >= nblk) return;                              // past the folded grid's end
    const int64_t lo = b << dbits, hi = min(lo + ((int64_t)1 << dbits), N);
    const void* xw = x.p[w];
    double acc = 0.0;
    for (int64_t c0 = lo; c0 < hi; c0 += 16 * kThreads) {
        float v[16];
        const int64_t e0 = c0 + threadIdx.x;
        if (c0 + 16 * kThreads <= hi) {               // a full chunk: loads in flight together
#pragma unroll
            for (int k = 0; k < 16; k++) v[k] = load_coord(xw, e0 + k * kThreads, hi, DT);
        } else {
#pragma unroll
            for (int k = 0; k < 16; k++) {
                const int64_t e = e0 + k * kThreads;
                v[k] = e < hi ? load_coord(xw, e, hi, DT) : 0.0f;
            }
        }
#pragma unroll
        for (int k = 0; k < 16; k++) acc += (double)v[k] * (double)v[k];
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
    const int64_t p = flat_block() * kThreads + threadIdx.x;
    if (p >= nblk) return;
    double mx = 0.0;
    for (int i = 0; i < P; i++) mx = fmax(mx, sumsq[(int64_t)i * nblk + p]);
    const float M = (float)(t_p * sqrt(mx) / sqrt(d));
    mM[2 * p] = -M;
    mM[2 * p + 1] = M;
}

// Blocks b0 .. b0+nb-1 of the block-major pipeline: every worker's sum of
// squares from its G tile partials (in tile order), then the block's range
// as rht_range_kernel. One workgroup per block, one thread per worker.
__global__ __launch_bounds__(64) void rht_norms_range_kernel(const double* norms, int P, int G,
                                                             int64_t b0, int64_t nblk, double d,
                                                             double t_p, double* sumsq, float* mM) {
    const int64_t b = b0 + blockIdx.x;
    __shared__ double nw[GA_MAX_WORKERS];
    for (int w = threadIdx.x; w < P; w += 64) {
        const double* pw = norms + ((b * P + w) * G);
        double t = 0.0;
        for (int q = 0; q < G; q++) t += pw[q];
        nw[w] = t;
        if (sumsq) sumsq[(int64_t)w * nblk + b] = t;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        double mx = 0.0;
        for (int i = 0; i < P; i++) mx = fmax(mx, nw[i]);
        const float M = (float)(t_p * sqrt(mx) / sqrt(d));
        mM[2 * b] = -M;
        mM[2 * b + 1] = M;
    }
}

int log2_block(int64_t d) {
    if (d < 2 || d > (1ll << kMaxBits) || (d & (d - 1))) return -1;
    int k = 0;
    while ((1ll << k) < d) k++;
    return k;
}
bool pow2_block(int64_t d) { return log2_block(d) > 0; }

float inv_sqrt_d(int64_t d) { return (float)(1.0 / std::sqrt((double)d)); }

}  // namespace
}  // namespace ga

using namespace ga;

extern "C" ga_status thc_rht_sumsq(const void* const* bufs, int32_t P, int64_t N, ga_dtype dt,
                                   int64_t d, double* d_sumsq, void* stream) {
    const char* what = "thc_rht_sumsq";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    const int dbits = log2_block(d);
    if (dbits < 0) return fail(GA_EINVAL, "%s: d = %lld is not a power of two in [2, 2^22]", what, (long long)d);
    if (N < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(bufs, P, elem_size(dt), what);
    if (rc) return rc;
    if (!d_sumsq || !aligned(d_sumsq, 8)) return fail(GA_EINVAL, "%s: bad output pointer", what);
    const int64_t nblk = ceil_div(N, d);
    if (!flat_fits(nblk)) return fail(GA_EINVAL, "%s: too many blocks", what);
    PtrTable t{};
    for (int i = 0; i < P; i++) t.p[i] = const_cast<void*>(bufs[i]);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    if (dt == GA_F32)
        hipLaunchKernelGGL(rht_sumsq_kernel<GA_F32>, flat_grid(nblk, (unsigned)P), dim3(kThreads), 0, hs, t, N, dbits, nblk, d_sumsq);
    else
        hipLaunchKernelGGL(rht_sumsq_kernel<GA_BF16>, flat_grid(nblk, (unsigned)P), dim3(kThreads), 0, hs, t, N, dbits, nblk, d_sumsq);
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
    if (!flat_fits(ceil_div(nblk, kThreads))) return fail(GA_EINVAL, "%s: too many blocks", what);
    hipLaunchKernelGGL(rht_range_kernel, flat_grid(ceil_div(nblk, kThreads)), dim3(kThreads), 0,
                       static_cast<hipStream_t>(stream), d_sumsq, P, nblk, (double)d, t_p, d_mM);
    return check_launch(what);
}

extern "C" ga_status thc_rht_forward(const void* const* bufs, int32_t P, int64_t N, ga_dtype dt,
                                     int64_t d, uint64_t seed, const float* d_mM, float* const* y,
                                     void* stream) {
    const char* what = "thc_rht_forward";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    const int dbits = log2_block(d);
    if (dbits < 0) return fail(GA_EINVAL, "%s: d = %lld is not a power of two in [2, 2^22]", what, (long long)d);
    if (N < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (N == 0) return GA_OK;
    ga_status rc = check_workers(bufs, P, elem_size(dt), what);
    if (rc) return rc;
    if ((rc = check_workers(reinterpret_cast<const void* const*>(y), P, 4, what))) return rc;
    if (d_mM && !aligned(d_mM, 8)) return fail(GA_EINVAL, "%s: misaligned range", what);
    const int64_t Np = ceil_div(N, d) * d;
    const int64_t tiles = ceil_div(Np, kTile);
    if (!grid_fits(tiles, kTT)) return fail(GA_EINVAL, "%s: too many tiles", what);
    PtrTable tx{}, ty{};
    int vec = 1;                                      // 16-byte loads of x in the first pass
    for (int i = 0; i < P; i++) {
        tx.p[i] = const_cast<void*>(bufs[i]);
        ty.p[i] = y[i];
        vec &= aligned(bufs[i], 16);
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const float c = inv_sqrt_d(d);
    const dim3 g1((unsigned)tiles, (unsigned)P);
    const bool one = dbits <= kTileBits;
    const int kbits = one ? dbits : kTileBits;
    if (one) {
        if (dt == GA_F32)
            hipLaunchKernelGGL((rht_tile_kernel<true, true, GA_F32>), g1, dim3(kTT), 0, hs, tx, ty, N, Np, kbits, k0, k1, c, d_mM);
        else
            hipLaunchKernelGGL((rht_tile_kernel<true, true, GA_BF16>), g1, dim3(kTT), 0, hs, tx, ty, N, Np, kbits, k0, k1, c, d_mM);
        return check_launch(what);
    }
    if (dt == GA_F32)
        hipLaunchKernelGGL((rht_forward_tile_kernel<GA_F32>), g1, dim3(kTT), 0, hs, tx, ty, N, vec, k0, k1);
    else
        hipLaunchKernelGGL((rht_forward_tile_kernel<GA_BF16>), g1, dim3(kTT), 0, hs, tx, ty, N, vec, k0, k1);
    if ((rc = check_launch(what))) return rc;
    const int wbits = 2 * kTileBits - dbits;         // W = kTile / G
    hipLaunchKernelGGL((rht_cross_kernel<true, GA_F32>), g1, dim3(kTT), 0, hs, ty, ty, Np, dbits, wbits, k0, k1, c, d_mM);
    return check_launch(what);
}

extern "C" ga_status thc_rht_inverse(float* y, int64_t N, int64_t d, uint64_t seed, void* out,
                                     ga_dtype out_dt, void* stream) {
    const char* what = "thc_rht_inverse";
    if (!valid_dtype(out_dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)out_dt);
    const int dbits = log2_block(d);
    if (dbits < 0) return fail(GA_EINVAL, "%s: d = %lld is not a power of two in [2, 2^22]", what, (long long)d);
    if (N < 0) return fail(GA_EINVAL, "%s: negative size", what);
    if (N == 0) return GA_OK;
    if (!y || !out || !aligned(y, 4) || !aligned(out, elem_size(out_dt)))
        return fail(GA_EINVAL, "%s: null or misaligned pointer", what);
    const int64_t Np = ceil_div(N, d) * d;
    const int64_t tiles = ceil_div(Np, kTile);
    if (!grid_fits(tiles, kTT)) return fail(GA_EINVAL, "%s: too many tiles", what);
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const float c = inv_sqrt_d(d);
    PtrTable ty{}, to{};
    ty.p[0] = y;
    to.p[0] = out;
    const dim3 g1((unsigned)tiles, 1u);
    const float* none = nullptr;
    if (dbits <= kTileBits) {
        if (out_dt == GA_F32)
            hipLaunchKernelGGL((rht_tile_kernel<false, true, GA_F32>), g1, dim3(kTT), 0, hs, ty, to, N, Np, dbits, k0, k1, c, none);
        else
            hipLaunchKernelGGL((rht_tile_kernel<false, true, GA_BF16>), g1, dim3(kTT), 0, hs, ty, to, N, Np, dbits, k0, k1, c, none);
        return check_launch(what);
    }
    hipLaunchKernelGGL((rht_tile_kernel<false, false, GA_F32>), g1, dim3(kTT), 0, hs, ty, ty, N, Np, (int)kTileBits, k0, k1, c, none);
    ga_status rc = check_launch(what);
    if (rc) return rc;
    const int wbits = 2 * kTileBits - dbits;
    if (out_dt == GA_F32)
        hipLaunchKernelGGL((rht_cross_kernel<false, GA_F32>), g1, dim3(kTT), 0, hs, ty, to, N, dbits, wbits, k0, k1, c, none);
    else
        hipLaunchKernelGGL((rht_cross_kernel<false, GA_BF16>), g1, dim3(kTT), 0, hs, ty, to, N, dbits, wbits, k0, k1, c, none);
    return check_launch(what);
}

extern "C" ga_status thc_rht_quantize(const void* const* bufs, int32_t P, int32_t worker0, int64_t N,
                                      ga_dtype dt, int64_t d, uint64_t rht_seed, const float* d_mM,
                                      int32_t b, int32_t g, const int32_t* h_table,
                                      uint64_t q_seed, float* const* y_scratch,
                                      uint8_t* const* packed, void* stream) {
    const char* what = "thc_rht_quantize";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    const int dbits = log2_block(d);
    if (dbits < 0) return fail(GA_EINVAL, "%s: d = %lld is not a power of two in [2, 2^22]", what, (long long)d);
    if (!valid_bits(b)) return fail(GA_EINVAL, "%s: b = %d is not 1, 2, 4 or 8", what, b);
    if (N < 0 || worker0 < 0) return fail(GA_EINVAL, "%s: negative argument", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    TableArg tab{};
    ga_status rc;
    if (h_table && (rc = load_table(b, g, h_table, &tab, what))) return rc;
    if (N == 0) return GA_OK;
    if ((rc = check_workers(bufs, P, elem_size(dt), what))) return rc;
    if ((rc = check_workers(reinterpret_cast<const void* const*>(packed), P, 16, what))) return rc;
    if (!d_mM || !aligned(d_mM, 8)) return fail(GA_EINVAL, "%s: bad range pointer", what);
    const bool two_pass = dbits > kTileBits;
    if (two_pass) {
        if (!y_scratch) return fail(GA_EINVAL, "%s: d > %d needs the scratch vectors", what, kTile);
        if ((rc = check_workers(reinterpret_cast<const void* const*>(y_scratch), P, 4, what))) return rc;
    }
    const int64_t Np = ceil_div(N, d) * d;
    const int64_t tiles = ceil_div(Np, kTile);
    if (!grid_fits(tiles, kTT)) return fail(GA_EINVAL, "%s: too many tiles", what);
    PtrTable tx{}, ty{}, tp{};
    int vec = 1;                                      // 16-byte loads of x in the first pass
    for (int i = 0; i < P; i++) {
        tx.p[i] = const_cast<void*>(bufs[i]);
        tp.p[i] = packed[i];
        if (two_pass) ty.p[i] = y_scratch[i];
        vec &= aligned(bufs[i], 16);
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint32_t k0 = (uint32_t)rht_seed, k1 = (uint32_t)(rht_seed >> 32);
    const uint32_t q0 = (uint32_t)q_seed, q1 = (uint32_t)(q_seed >> 32);
    const float c = inv_sqrt_d(d);
    const dim3 g1((unsigned)tiles, (unsigned)P);
    const bool tb = h_table != nullptr;
    if (!two_pass) {
#define GA_TQ(DT, B)                                                                                   \
        do {                                                                                           \
            if (tb) hipLaunchKernelGGL((rht_tile_quant_kernel<DT, B, true>), g1, dim3(kTT), table_lds_bytes(tab), hs, tx, tp, \
                                       worker0, N, Np, dbits, k0, k1, c, d_mM, q0, q1, tab);          \
            else hipLaunchKernelGGL((rht_tile_quant_kernel<DT, B, false>), g1, dim3(kTT), 0, hs, tx, tp, \
                                    worker0, N, Np, dbits, k0, k1, c, d_mM, q0, q1, tab);             \
        } while (0)
#define GA_TQB(DT)                               \
        switch (b) {                             \
            case 1: GA_TQ(DT, 1); break;         \
            case 2: GA_TQ(DT, 2); break;         \
            case 4: GA_TQ(DT, 4); break;         \
            default: GA_TQ(DT, 8); break;        \
        }
        if (dt == GA_F32) { GA_TQB(GA_F32) } else { GA_TQB(GA_BF16) }
#undef GA_TQB
#undef GA_TQ
        return check_launch(what);
    }
    // chunks of kPipeUnits blocks: launch k runs the first pass of chunk k
    // and the second of chunk k - 1
    double* const none_d = nullptr;
    const int64_t nblk = Np / d, units = (int64_t)P * nblk;
    const int64_t U = min(units, kPipeUnits);
    const int64_t nchunk = ceil_div(units, U);
    if ((units << (dbits - kTileBits)) > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: too many tiles", what);
    for (int64_t k = 0; k <= nchunk; k++) {
        const int64_t a0 = k * U, na = k < nchunk ? min(U, units - a0) : 0;
        const int64_t b0 = (k - 1) * U, nb = k > 0 ? min(U, units - b0) : 0;
        const dim3 grid((unsigned)((na + nb) << (dbits - kTileBits)));
#define GA_PQ(DT, B)                                                                                    \
        do {                                                                                            \
            if (tb) hipLaunchKernelGGL((rht_quant_pipe_kernel<DT, B, true>), grid, dim3(kTT), table_lds_bytes(tab), hs, tx, \
                                       ty, tp, worker0, N, vec, dbits, nblk, a0, na, b0, nb, k0, k1, c, d_mM, \
                                       q0, q1, tab, P, none_d);                                         \
            else hipLaunchKernelGGL((rht_quant_pipe_kernel<DT, B, false>), grid, dim3(kTT), 0, hs, tx,  \
                                    ty, tp, worker0, N, vec, dbits, nblk, a0, na, b0, nb, k0, k1, c, d_mM,   \
                                    q0, q1, tab, P, none_d);                                            \
        } while (0)
#define GA_PQB(DT)                               \
        switch (b) {                             \
            case 1: GA_PQ(DT, 1); break;         \
            case 2: GA_PQ(DT, 2); break;         \
            case 4: GA_PQ(DT, 4); break;         \
            default: GA_PQ(DT, 8); break;        \
        }
        if (dt == GA_F32) { GA_PQB(GA_F32) } else { GA_PQB(GA_BF16) }
#undef GA_PQB
#undef GA_PQ
        if ((rc = check_launch(what))) return rc;
    }
    return GA_OK;
}

extern "C" size_t thc_rht_norm_quantize_ws_bytes(int32_t P, int64_t N, int64_t d) {
    const int dbits = log2_block(d);
    if (dbits < 0 || P < 1 || N <= 0) return 0;
    const int64_t nblk = ceil_div(N, d);
    const int64_t per_block = dbits > kTileBits ? ((int64_t)1 << (dbits - kTileBits)) : 1;
    return (size_t)P * (size_t)nblk * (size_t)per_block * sizeof(double);
}

extern "C" ga_status thc_rht_norm_quantize(const void* const* bufs, int32_t P, int32_t worker0, int64_t N,
                                           ga_dtype dt, int64_t d, uint64_t rht_seed, double t_p,
                                           int32_t b, int32_t g, const int32_t* h_table, uint64_t q_seed,
                                           double* d_sumsq, float* d_mM, float* const* y_scratch,
                                           void* d_ws, size_t ws_bytes, uint8_t* const* packed,
                                           void* stream) {
    const char* what = "thc_rht_norm_quantize";
    if (!valid_dtype(dt)) return fail(GA_EINVAL, "%s: unknown dtype %d", what, (int)dt);
    const int dbits = log2_block(d);
    if (dbits < 0) return fail(GA_EINVAL, "%s: d = %lld is not a power of two in [2, 2^22]", what, (long long)d);
    if (!valid_bits(b)) return fail(GA_EINVAL, "%s: b = %d is not 1, 2, 4 or 8", what, b);
    if (N < 0 || worker0 < 0) return fail(GA_EINVAL, "%s: negative argument", what);
    if (P < 1 || P > GA_MAX_WORKERS) return fail(GA_EINVAL, "%s: P = %d outside [1, %d]", what, P, GA_MAX_WORKERS);
    if (!(t_p > 0.0) || !std::isfinite(t_p)) return fail(GA_EINVAL, "%s: bad t_p", what);
    TableArg tab{};
    ga_status rc;
    if (h_table && (rc = load_table(b, g, h_table, &tab, what))) return rc;
    if (N == 0) return GA_OK;
    if ((rc = check_workers(bufs, P, elem_size(dt), what))) return rc;
    if ((rc = check_workers(reinterpret_cast<const void* const*>(packed), P, 16, what))) return rc;
    if (!d_mM || !aligned(d_mM, 8)) return fail(GA_EINVAL, "%s: bad range pointer", what);
    if (d_sumsq && !aligned(d_sumsq, 8)) return fail(GA_EINVAL, "%s: misaligned sums", what);
    if (!d_ws || !aligned(d_ws, 8) || ws_bytes < thc_rht_norm_quantize_ws_bytes(P, N, d))
        return fail(GA_EINVAL, "%s: workspace missing or below %zu bytes", what,
                    thc_rht_norm_quantize_ws_bytes(P, N, d));
    const int64_t nblk = ceil_div(N, d);
    if (nblk > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: too many blocks", what);
    double* ws = static_cast<double*>(d_ws);
    if (dbits <= kTileBits) {
        // one pass quantizes as it transforms, so the norms come first
        double* sums = d_sumsq ? d_sumsq : ws;
        if ((rc = thc_rht_sumsq(bufs, P, N, dt, d, sums, stream))) return rc;
        if ((rc = thc_rht_range(sums, P, nblk, d, t_p, d_mM, stream))) return rc;
        return thc_rht_quantize(bufs, P, worker0, N, dt, d, rht_seed, d_mM, b, g, h_table, q_seed, nullptr,
                                packed, stream);
    }
    if (!y_scratch) return fail(GA_EINVAL, "%s: d > %d needs the scratch vectors", what, kTile);
    if ((rc = check_workers(reinterpret_cast<const void* const*>(y_scratch), P, 4, what))) return rc;
    const int64_t Np = nblk * d;
    PtrTable tx{}, ty{}, tp{};
    int vec = 1;
    for (int i = 0; i < P; i++) {
        tx.p[i] = const_cast<void*>(bufs[i]);
        tp.p[i] = packed[i];
        ty.p[i] = y_scratch[i];
        vec &= aligned(bufs[i], 16);
    }
    hipStream_t hs = static_cast<hipStream_t>(stream);
    const uint32_t k0 = (uint32_t)rht_seed, k1 = (uint32_t)(rht_seed >> 32);
    const uint32_t q0 = (uint32_t)q_seed, q1 = (uint32_t)(q_seed >> 32);
    const float c = inv_sqrt_d(d);
    const bool tb = h_table != nullptr;
    const int gbits = dbits - kTileBits;
    // block-major units (every worker of a block in one chunk): launch k
    // runs the first pass of chunk k (with the tiles' sums of squares) and
    // the second pass of chunk k - 1, whose ranges the kernel launched
    // after launch k - 1 derived from those sums
    const int64_t units = (int64_t)P * nblk;
    const int64_t bpc = std::max<int64_t>(1, kPipeUnits / P);          // blocks per chunk
    const int64_t U = std::min(units, bpc * P);
    const int64_t nchunk = ceil_div(units, U);
    if ((units << gbits) > 0x7FFFFFFF) return fail(GA_EINVAL, "%s: too many tiles", what);
    (void)Np;
    for (int64_t k = 0; k <= nchunk; k++) {
        const int64_t a0 = k * U, na = k < nchunk ? std::min(U, units - a0) : 0;
        const int64_t b0 = (k - 1) * U, nb = k > 0 ? std::min(U, units - b0) : 0;
        const dim3 grid((unsigned)((na + nb) << gbits));
#define GA_NQ(DT, B)                                                                                    \
        do {                                                                                            \
            if (tb) hipLaunchKernelGGL((rht_quant_pipe_kernel<DT, B, true>), grid, dim3(kTT), table_lds_bytes(tab), hs, tx, \
                                       ty, tp, worker0, N, vec, dbits, nblk, a0, na, b0, nb, k0, k1, c, d_mM, \
                                       q0, q1, tab, P, ws);                                             \
            else hipLaunchKernelGGL((rht_quant_pipe_kernel<DT, B, false>), grid, dim3(kTT), 0, hs, tx,  \
                                    ty, tp, worker0, N, vec, dbits, nblk, a0, na, b0, nb, k0, k1, c, d_mM, \
                                    q0, q1, tab, P, ws);                                                \
        } while (0)
#define GA_NQB(DT)                               \
        switch (b) {                             \
            case 1: GA_NQ(DT, 1); break;         \
            case 2: GA_NQ(DT, 2); break;         \
            case 4: GA_NQ(DT, 4); break;         \
            default: GA_NQ(DT, 8); break;        \
        }
        if (dt == GA_F32) { GA_NQB(GA_F32) } else { GA_NQB(GA_BF16) }
#undef GA_NQB
#undef GA_NQ
        if ((rc = check_launch(what))) return rc;
        if (na > 0) {                                   // the chunk's blocks: a0 / P .. (a0 + na) / P - 1
            hipLaunchKernelGGL(rht_norms_range_kernel, dim3((unsigned)(na / P)), dim3(64), 0, hs, ws, P,
                               1 << gbits, a0 / P, nblk, (double)d, t_p, d_sumsq, d_mM);
            if ((rc = check_launch(what))) return rc;
        }
    }
    return GA_OK;
}
