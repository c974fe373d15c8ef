// philox.hpp -- Philox4x32-10 on the GPU, from its published definition:
// J. K. Salmon, M. A. Moraes, R. O. Dror, D. E. Shaw, "Parallel random
// numbers: as easy as 1, 2, 3", SC'11, section 3.2.
//
// State: a 128-bit counter (four 32-bit words) and a 64-bit key (two
// words). A round multiplies counter words 0 and 2 by the two Philox
// multipliers (full 32x32 -> 64-bit products), then the new counter is
// (hi(B x2) ^ x1 ^ k0, lo(B x2), hi(A x0) ^ x3 ^ k1, lo(A x0)). Before each
// round after the first, the key is advanced by the two Weyl increments
// (golden ratio and sqrt(3) - 1, scaled to 32 bits). Ten rounds.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace ga {

struct Philox4 {
    uint32_t v[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                                 uint32_t k0, uint32_t k1) {
    constexpr uint32_t kMulA = 0xD2511F53u, kMulB = 0xCD9E8D57u;
    constexpr uint32_t kWeylA = 0x9E3779B9u, kWeylB = 0xBB67AE85u;
#pragma unroll
    for (int r = 0; r < 10; r++) {
        if (r) {
            k0 += kWeylA;
            k1 += kWeylB;
        }
        const uint64_t pa = (uint64_t)kMulA * c0;
        const uint64_t pb = (uint64_t)kMulB * c2;
        // three-input exclusive or in one instruction (truth table 0x96)
        const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(pb >> 32), c1, k0, 0x96);
        const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(pa >> 32), c3, k1, 0x96);
        c1 = (uint32_t)pb;
        c3 = (uint32_t)pa;
        c0 = n0;
        c2 = n2;
    }
    return {{c0, c1, c2, c3}};
}

}  // namespace ga
