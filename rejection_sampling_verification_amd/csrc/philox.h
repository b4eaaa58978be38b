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
//   level-1 draw of request b, row a, block c : (c >> 2, a, b, 1), word c & 3
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
        // both halves of each 32 x 32 product from one 64-bit multiply
        const uint64_t p0 = uint64_t(kPhiloxM0) * c.x;
        const uint64_t p1 = uint64_t(kPhiloxM1) * c.z;
        const uint32_t lo0 = uint32_t(p0), hi0 = uint32_t(p0 >> 32);
        const uint32_t lo1 = uint32_t(p1), hi1 = uint32_t(p1 >> 32);
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

// Standard Gumbel variate -ln(-ln u) in fp32 for u = (2n + 1) 2^-24, from the
// hardware base-2 logarithm: -ln 2 log2(ln 2 (-log2 u)).  Every u and every
// inner value is a normal fp32 number.  Compared with the exact value over all
// 2^23 possible u on gfx950, the result is within 1.7e-6 (the library
// logf/log1pf form is within 1.9e-6 and costs about eight times as much).
constexpr float kLn2f = 0.693147180559945309f;

__device__ __forceinline__ float gumbel_of(uint32_t w) {
    const float u = static_cast<float>((w >> 9) * 2u + 1u) * 0x1p-24f;
    return -kLn2f * __builtin_amdgcn_logf(kLn2f * -__builtin_amdgcn_logf(u));
}

// The same variate as a double, within 1.6e-7 of exact over all 2^23
// possible u on gfx950 (the fp32 form above loses up to 1.6e-6 where u is near
// 1, which is where the largest variates, the ones that win races, come
// from).  L = -ln u in fp32 to a few units of its last place: for u > 3/4
// from 1 - u = d (exact) as the series -ln(1 - d) = sum d^k / k to k = 13
// (truncation below 5e-9 relative); else from the exponent of u plus the
// hardware log2 of its mantissa.  Then G = -ln L = -ln 2 (e + log2 m) for
// L = m 2^e, with the sum formed in fp64, so that no log2 result larger than
// 1 in magnitude is rounded to fp32.
__device__ __forceinline__ double gumbel_wide(uint32_t w) {
    constexpr double kLn2d = 0.693147180559945309417;
    const uint32_t m = (w >> 9) * 2u + 1u;  // u = m 2^-24
    const uint32_t dm = (1u << 24) - m;      // 1 - u = dm 2^-24
    float L;
    if (dm < (1u << 22)) {
        const float d = static_cast<float>(dm) * 0x1p-24f;
        float s = 1.0f / 13.0f;
#pragma unroll
        for (int k = 12; k >= 1; --k) s = fmaf(s, d, 1.0f / static_cast<float>(k));
        L = d * s;
    } else {
        const float u = static_cast<float>(m) * 0x1p-24f;
        L = -kLn2f * (static_cast<float>(__builtin_amdgcn_frexp_expf(u)) +
                      __builtin_amdgcn_logf(__builtin_amdgcn_frexp_mantf(u)));
    }
    return -kLn2d * (static_cast<double>(__builtin_amdgcn_frexp_expf(L)) +
                     static_cast<double>(__builtin_amdgcn_logf(__builtin_amdgcn_frexp_mantf(L))));
}

__device__ __forceinline__ double draw_accept(PhiloxKey key, uint32_t b, uint32_t i) {
    return uniform_accept(philox4x32_10(make_uint4(0u, i, b, 0u), key.k0, key.k1).x);
}

// Level-2 Gumbel variates of tokens j0 .. j0 + 3 (j0 a multiple of 4).
__device__ __forceinline__ void draw_token_gumbels4(PhiloxKey key, uint32_t b, uint32_t a,
                                                    uint32_t j0, float g[4]) {
    const uint4 w = philox4x32_10(make_uint4(j0 >> 2, a, b, 2u), key.k0, key.k1);
    g[0] = gumbel_of(w.x);
    g[1] = gumbel_of(w.y);
    g[2] = gumbel_of(w.z);
    g[3] = gumbel_of(w.w);
}

}  // namespace sdv
