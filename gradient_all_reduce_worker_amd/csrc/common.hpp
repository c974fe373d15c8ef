// common.hpp -- internals shared by the libga.so translation units: error
// reporting across the C ABI, the worker pointer table passed by value in
// kernel arguments, bf16 widening/rounding, and small launch helpers.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "../../include/ga.h"

namespace ga {

constexpr int kThreads = 256;  // every kernel runs 256-thread workgroups (4 wave64)

// ------------------------------------------------------------------ errors
ga_status fail(ga_status code, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
ga_status check_launch(const char* what);

// ------------------------------------------------------------------ pointers
// Up to GA_MAX_WORKERS device pointers, passed by value (512 bytes of kernel
// arguments). Indexing with a wave-uniform index compiles to a scalar load.
struct PtrTable {
    void* p[GA_MAX_WORKERS];
};

inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

inline size_t elem_size(ga_dtype dt) { return dt == GA_BF16 ? 2 : 4; }

inline bool valid_dtype(int dt) { return dt == GA_F32 || dt == GA_BF16; }

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int64_t n_partitions(int64_t N, int64_t part) {
    if (N <= 0) return 0;
    int64_t plen = part > 0 ? part : N;
    return ceil_div(N, plen);
}

// Common argument checks for an array of P worker pointers.
ga_status check_workers(const void* const* bufs, int32_t P, size_t align, const char* what);

// ------------------------------------------------------------------ bf16
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// binary32 -> bf16 with round-to-nearest-even: add 0x7FFF plus the lowest
// kept bit, then drop the low 16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Streaming 16-byte accesses: the nontemporal hint keeps single-use
// gradient data from displacing other lines in the caches (measured ~8%
// faster than plain accesses for the multi-stream ring on MI355X).
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
// Device memory (global address space): pointers read from a table in
// memory are otherwise generic and would be accessed with flat instructions,
// whose completion counter also gates scalar loads.
typedef __attribute__((address_space(1))) u32x4_t g_u32x4_t;

__device__ __forceinline__ uint4 load_stream(const void* p) {
    const u32x4_t r = __builtin_nontemporal_load((const g_u32x4_t*)p);
    return make_uint4(r.x, r.y, r.z, r.w);
}
__device__ __forceinline__ void store_stream(void* p, uint4 v) {
    const u32x4_t r = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(r, (g_u32x4_t*)p);
}

// ------------------------------------------------------------------ launch geometry
// A dispatch packet carries each grid dimension as a 32-bit count of
// work-items: a launch of more than 2^32 - 1 work-items along x does not
// fail, the count wraps and fewer workgroups run. kMaxBlocksX is the most
// kThreads-thread workgroups one launch takes along x. Kernels whose
// workgroup count grows with N take a folded grid: flat_grid(n, y) spreads n
// workgroups over x and z (y stays free for the worker slot), and the kernel
// reads its linear index with flat_block() and returns when it is >= n
// (fewer than z such workgroups).
constexpr int64_t kMaxBlocksX = 0xFFFFFFFFll / kThreads;
constexpr int64_t kMaxFoldZ = 1024;

// A plain (unfolded) launch of `blocks` workgroups of `threads` threads fits.
inline bool grid_fits(int64_t blocks, int threads = kThreads) {
    return blocks >= 0 && blocks <= 0xFFFFFFFFll / threads;
}
// flat_grid can cover `blocks` workgroups.
inline bool flat_fits(int64_t blocks) { return blocks >= 0 && blocks <= kMaxBlocksX * kMaxFoldZ; }

inline dim3 flat_grid(int64_t blocks, unsigned y = 1) {
    const int64_t z = blocks > kMaxBlocksX ? ceil_div(blocks, kMaxBlocksX) : 1;
    return dim3((unsigned)ceil_div(blocks, z), y, (unsigned)z);
}

__device__ __forceinline__ int64_t flat_block() {
    return (int64_t)blockIdx.z * gridDim.x + blockIdx.x;
}

}  // namespace ga
