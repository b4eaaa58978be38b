// Counter-based uniforms for the verifier's draws.
//
// Philox4x32 with 10 rounds (Salmon, Moraes, Dror, Shaw, "Parallel Random
// Numbers: As Easy as 1, 2, 3", SC'11, section 3.2): each round multiplies
// counter words 0 and 2 by fixed 32-bit multipliers, keeps both halves of the
// products, and mixes the high halves with words 1 and 3 and the round key;
// the key advances by two Weyl increments between rounds.
//
// Streams (key = seed low word, seed high word):
//   accept draw of request b, position i  : counter (0, i, b, 0), word 0
//   level-1 draw of request b, row a, block c : (c, a, b, 1), word 0
//   level-2 draw of request b, row a, token j : (j >> 2, a, b, 2), word j & 3
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace sdv {

constexpr uint32_t kPhiloxM0 = 0xD2511F53u;  // SC'11, Table 2 (Philox4x32)
constexpr uint32_t kPhiloxM1 = 0xCD9E8D57u;
constexpr uint32_t kWeyl0 = 0x9E3779B9u;     // 2^32 * (golden ratio - 1)
constexpr uint32_t kWeyl1 = 0xBB67AE85u;     // 2^32 * (sqrt(3) - 1)

__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        const uint32_t lo0 = kPhiloxM0 * c.x;
        const uint32_t hi0 = __umulhi(kPhiloxM0, c.x);
        const uint32_t lo1 = kPhiloxM1 * c.z;
        const uint32_t hi1 = __umulhi(kPhiloxM1, c.z);
        c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
        k0 += kWeyl0;
        k1 += kWeyl1;
    }
    return c;
}

struct PhiloxKey {
    uint32_t k0, k1;
};

__device__ __forceinline__ PhiloxKey key_of(uint64_t seed) {
    return PhiloxKey{static_cast<uint32_t>(seed), static_cast<uint32_t>(seed >> 32)};
}

// [0, 1): the top 24 bits of a word, exact in float and double.
__device__ __forceinline__ double uniform_accept(uint32_t w) {
    return static_cast<double>(w >> 8) * 0x1p-24;
}

// (0, 1): odd multiples of 2^-24 from the top 23 bits.
__device__ __forceinline__ double uniform_open(uint32_t w) {
    return (static_cast<double>(w >> 9) * 2.0 + 1.0) * 0x1p-24;
}

__device__ __forceinline__ double gumbel_of(double u) { return -log(-log(u)); }

__device__ __forceinline__ double draw_accept(PhiloxKey key, uint32_t b, uint32_t i) {
    return uniform_accept(philox4x32_10(make_uint4(0u, i, b, 0u), key.k0, key.k1).x);
}

__device__ __forceinline__ double draw_block_gumbel(PhiloxKey key, uint32_t b, uint32_t a,
                                                    uint32_t c) {
    return gumbel_of(uniform_open(philox4x32_10(make_uint4(c, a, b, 1u), key.k0, key.k1).x));
}

// Gumbel variates of the 8 tokens j0 .. j0+7 (j0 a multiple of 8).
__device__ __forceinline__ void draw_token_gumbels8(PhiloxKey key, uint32_t b, uint32_t a,
                                                    uint32_t j0, double g[8]) {
    const uint4 w0 = philox4x32_10(make_uint4(j0 >> 2, a, b, 2u), key.k0, key.k1);
    const uint4 w1 = philox4x32_10(make_uint4((j0 >> 2) + 1u, a, b, 2u), key.k0, key.k1);
    g[0] = gumbel_of(uniform_open(w0.x));
    g[1] = gumbel_of(uniform_open(w0.y));
    g[2] = gumbel_of(uniform_open(w0.z));
    g[3] = gumbel_of(uniform_open(w0.w));
    g[4] = gumbel_of(uniform_open(w1.x));
    g[5] = gumbel_of(uniform_open(w1.y));
    g[6] = gumbel_of(uniform_open(w1.z));
    g[7] = gumbel_of(uniform_open(w1.w));
}

}  // namespace sdv
