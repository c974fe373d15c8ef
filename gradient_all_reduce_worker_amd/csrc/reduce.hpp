// reduce.hpp -- the binary64 (numerator, denominator) partial sums of the
// NMSE ("THC: Accelerating Distributed Deep Learning Using Tensor
// Homomorphic Compression", section 2): a workgroup-wide sum, and the two
// kernels that fold per-workgroup partials in a fixed order, in one level or
// in groups of kNmseGroup first. Shared by the NMSE passes of thc.hip and
// the fused ring-and-THC pass of step.hip.
#pragma once
#include "common.hpp"

namespace ga {
namespace {

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

// Sum of the (num, den) partials lo .. hi-1 in a fixed order: four
// independent sums per thread (four loads in flight), then a tree over the
// workgroup.
__device__ __forceinline__ void sum_partials(const double* ws, int64_t lo, int64_t hi, double* num,
                                             double* den) {
    double n4[4] = {0.0, 0.0, 0.0, 0.0}, d4[4] = {0.0, 0.0, 0.0, 0.0};
    int64_t i = lo + threadIdx.x;
    for (; i + 3 * kThreads < hi; i += 4 * kThreads) {
#pragma unroll
        for (int k = 0; k < 4; k++) {
            n4[k] += ws[2 * (i + k * kThreads)];
            d4[k] += ws[2 * (i + k * kThreads) + 1];
        }
    }
    for (int k = 0; i < hi; i += kThreads, k = (k + 1) & 3) {
        n4[k] += ws[2 * i];
        d4[k] += ws[2 * i + 1];
    }
    __shared__ double sh[kThreads / 64];
    *num = block_sum((n4[0] + n4[1]) + (n4[2] + n4[3]), sh);
    *den = block_sum((d4[0] + d4[1]) + (d4[2] + d4[3]), sh);
}

__global__ __launch_bounds__(kThreads) void nmse_final_kernel(const double* ws, int nblk,
                                                              double* out) {
    double num, den;
    sum_partials(ws, 0, nblk, &num, &den);
    if (threadIdx.x == 0) {
        out[0] = num;
        out[1] = den;
        out[2] = den != 0.0 ? num / den : (num == 0.0 ? 0.0 : INFINITY);
    }
}

// First level for many partials: workgroup g sums partials
// g kNmseGroup .. (g + 1) kNmseGroup - 1 into out[2 g], out[2 g + 1].
constexpr int64_t kNmseGroup = 4096;

__global__ __launch_bounds__(kThreads) void nmse_group_kernel(const double* ws, int64_t nblk,
                                                              double* out) {
    const int64_t lo = (int64_t)blockIdx.x * kNmseGroup;
    double num, den;
    sum_partials(ws, lo, min(lo + kNmseGroup, nblk), &num, &den);
    if (threadIdx.x == 0) {
        out[2 * blockIdx.x] = num;
        out[2 * blockIdx.x + 1] = den;
    }
}

}  // namespace
}  // namespace ga
