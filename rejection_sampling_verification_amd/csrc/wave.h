// Wave64 and workgroup reductions for gfx950.
//
// Wave reductions run the classic GFX9 DPP ladder: row_shr 1, 2, 4, 8 folds
// each row of 16 lanes into its lane 15, row_bcast:15 (rows 1 and 3) and
// row_bcast:31 (rows 2 and 3) fold the rows into lane 63, which is then read
// into a scalar.  Lanes whose DPP source is out of range keep the identity.
// Doubles move as two 32-bit halves.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <limits.h>

namespace sdv {

constexpr int kWave = 64;

// Index of the calling wave in its workgroup, as a scalar (wave-uniform)
// value, so that loops and branches over it stay on the scalar unit.
__device__ __forceinline__ int wave_id() {
    return __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ int dpp_i(int identity, int v) {
    return __builtin_amdgcn_update_dpp(identity, v, CTRL, ROW_MASK, 0xf, false);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f(float identity, float v) {
    return __int_as_float(dpp_i<CTRL, ROW_MASK>(__float_as_int(identity), __float_as_int(v)));
}

__device__ __forceinline__ float wave_max(float v) {
    const float id = -INFINITY;
    v = fmaxf(v, dpp_f<0x111, 0xf>(id, v));  // row_shr:1
    v = fmaxf(v, dpp_f<0x112, 0xf>(id, v));  // row_shr:2
    v = fmaxf(v, dpp_f<0x114, 0xf>(id, v));  // row_shr:4
    v = fmaxf(v, dpp_f<0x118, 0xf>(id, v));  // row_shr:8
    v = fmaxf(v, dpp_f<0x142, 0xa>(id, v));  // row_bcast:15
    v = fmaxf(v, dpp_f<0x143, 0xc>(id, v));  // row_bcast:31
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_sum(float v) {
    v += dpp_f<0x111, 0xf>(0.0f, v);
    v += dpp_f<0x112, 0xf>(0.0f, v);
    v += dpp_f<0x114, 0xf>(0.0f, v);
    v += dpp_f<0x118, 0xf>(0.0f, v);
    v += dpp_f<0x142, 0xa>(0.0f, v);
    v += dpp_f<0x143, 0xc>(0.0f, v);
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ int wave_min_i(int v) {
    v = min(v, dpp_i<0x111, 0xf>(INT_MAX, v));
    v = min(v, dpp_i<0x112, 0xf>(INT_MAX, v));
    v = min(v, dpp_i<0x114, 0xf>(INT_MAX, v));
    v = min(v, dpp_i<0x118, 0xf>(INT_MAX, v));
    v = min(v, dpp_i<0x142, 0xa>(INT_MAX, v));
    v = min(v, dpp_i<0x143, 0xc>(INT_MAX, v));
    return __builtin_amdgcn_readlane(v, 63);
}

__device__ __forceinline__ uint32_t wave_sum_u(uint32_t v) {
    int x = static_cast<int>(v);
    x += dpp_i<0x111, 0xf>(0, x);
    x += dpp_i<0x112, 0xf>(0, x);
    x += dpp_i<0x114, 0xf>(0, x);
    x += dpp_i<0x118, 0xf>(0, x);
    x += dpp_i<0x142, 0xa>(0, x);
    x += dpp_i<0x143, 0xc>(0, x);
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(x, 63));
}

// Inclusive prefix sum over the lanes: the same ladder leaves lane i holding
// the sum of lanes 0 .. i.
__device__ __forceinline__ uint32_t wave_prefix_u(uint32_t v) {
    int x = static_cast<int>(v);
    x += dpp_i<0x111, 0xf>(0, x);
    x += dpp_i<0x112, 0xf>(0, x);
    x += dpp_i<0x114, 0xf>(0, x);
    x += dpp_i<0x118, 0xf>(0, x);
    x += dpp_i<0x142, 0xa>(0, x);
    x += dpp_i<0x143, 0xc>(0, x);
    return static_cast<uint32_t>(x);
}

__device__ __forceinline__ uint32_t wave_max_u(uint32_t v) {
    v = max(v, static_cast<uint32_t>(dpp_i<0x111, 0xf>(0, static_cast<int>(v))));
    v = max(v, static_cast<uint32_t>(dpp_i<0x112, 0xf>(0, static_cast<int>(v))));
    v = max(v, static_cast<uint32_t>(dpp_i<0x114, 0xf>(0, static_cast<int>(v))));
    v = max(v, static_cast<uint32_t>(dpp_i<0x118, 0xf>(0, static_cast<int>(v))));
    v = max(v, static_cast<uint32_t>(dpp_i<0x142, 0xa>(0, static_cast<int>(v))));
    v = max(v, static_cast<uint32_t>(dpp_i<0x143, 0xc>(0, static_cast<int>(v))));
    return static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(v), 63));
}

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ double dpp_d(double identity, double v) {
    const long long iv = __double_as_longlong(v), ii = __double_as_longlong(identity);
    const int lo = dpp_i<CTRL, ROW_MASK>(static_cast<int>(ii), static_cast<int>(iv));
    const int hi = dpp_i<CTRL, ROW_MASK>(static_cast<int>(ii >> 32), static_cast<int>(iv >> 32));
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

__device__ __forceinline__ double readlane_d(double v, int lane) {
    const long long iv = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane(static_cast<int>(iv), lane);
    const int hi = __builtin_amdgcn_readlane(static_cast<int>(iv >> 32), lane);
    return __longlong_as_double((static_cast<long long>(hi) << 32) | static_cast<unsigned int>(lo));
}

__device__ __forceinline__ double wave_max_d(double v) {
    const double id = -INFINITY;
    v = fmax(v, dpp_d<0x111, 0xf>(id, v));
    v = fmax(v, dpp_d<0x112, 0xf>(id, v));
    v = fmax(v, dpp_d<0x114, 0xf>(id, v));
    v = fmax(v, dpp_d<0x118, 0xf>(id, v));
    v = fmax(v, dpp_d<0x142, 0xa>(id, v));
    v = fmax(v, dpp_d<0x143, 0xc>(id, v));
    return readlane_d(v, 63);
}

__device__ __forceinline__ double wave_sum_d(double v) {
    v += dpp_d<0x111, 0xf>(0.0, v);
    v += dpp_d<0x112, 0xf>(0.0, v);
    v += dpp_d<0x114, 0xf>(0.0, v);
    v += dpp_d<0x118, 0xf>(0.0, v);
    v += dpp_d<0x142, 0xa>(0.0, v);
    v += dpp_d<0x143, 0xc>(0.0, v);
    return readlane_d(v, 63);
}

// Order-preserving unsigned code of a float: for non-NaN a, b,
// a > b  <=>  code(a) > code(b).
__device__ __forceinline__ uint32_t ordered_code(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float float_of_code(uint32_t c) {
    return __uint_as_float((c & 0x80000000u) ? (c & 0x7fffffffu) : ~c);
}

// The largest of a wave's floats through their codes (a NaN lane wins): each
// step of the integer ladder is one DPP instruction, where the float ladder
// also needs moves that quiet signaling NaNs.
__device__ __forceinline__ float wave_max_coded(float v) { return float_of_code(wave_max_u(ordered_code(v))); }

// A key and its index in one word: the larger word holds the larger key, and
// the lower index among equal keys.  0 stands for "no candidate".
__device__ __forceinline__ uint64_t pack_key(float key, int idx) {
    return (static_cast<uint64_t>(ordered_code(key)) << 32) | (0xffffffffu - static_cast<uint32_t>(idx));
}

__device__ __forceinline__ float packed_key(uint64_t p) { return float_of_code(static_cast<uint32_t>(p >> 32)); }

__device__ __forceinline__ int packed_index(uint64_t p) {
    return static_cast<int>(0xffffffffu - static_cast<uint32_t>(p));
}

// A packed key built from an ordered code directly (code 0 = no candidate).
__device__ __forceinline__ uint64_t pack_code(uint32_t code, int idx) {
    return code ? (static_cast<uint64_t>(code) << 32) | (0xffffffffu - static_cast<uint32_t>(idx)) : 0ull;
}

// The largest of a wave's codes (0 = none) and the lowest index that holds
// it, as the packed word pack_code makes: a 32-bit max ladder, then a min
// ladder over the indices of the lanes holding the maximum.  Each lane
// passes its own largest code with the lowest index it has for that code.
// Cheaper than a 64-bit ladder, whose steps need two moves and a 64-bit
// compare each.
__device__ __forceinline__ uint64_t wave_argmax_code(uint32_t code, int idx) {
    const uint32_t m = wave_max_u(code);
    const int i = wave_min_i((m != 0u && code == m) ? idx : INT_MAX);
    return pack_code(m, i);
}

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_u64(uint64_t v) {  // out-of-range lanes read 0
    const int lo = dpp_i<CTRL, ROW_MASK>(0, static_cast<int>(static_cast<uint32_t>(v)));
    const int hi = dpp_i<CTRL, ROW_MASK>(0, static_cast<int>(static_cast<uint32_t>(v >> 32)));
    return (static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) | static_cast<uint32_t>(lo);
}

__device__ __forceinline__ uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = max_u64(v, dpp_u64<0x111, 0xf>(v));
    v = max_u64(v, dpp_u64<0x112, 0xf>(v));
    v = max_u64(v, dpp_u64<0x114, 0xf>(v));
    v = max_u64(v, dpp_u64<0x118, 0xf>(v));
    v = max_u64(v, dpp_u64<0x142, 0xa>(v));
    v = max_u64(v, dpp_u64<0x143, 0xc>(v));
    const uint32_t lo = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v)), 63);
    const uint32_t hi = __builtin_amdgcn_readlane(static_cast<int>(static_cast<uint32_t>(v >> 32)), 63);
    return (static_cast<uint64_t>(hi) << 32) | lo;
}

// Workgroup barrier that orders LDS traffic only: unlike __syncthreads it
// does not wait for the calling wave's outstanding global loads, stores and
// atomics.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Workgroup-wide reductions over NW waves through LDS; every thread gets the
// result.  `scratch` holds NW elements.  Each call starts with a barrier, so
// a scratch array may be reused by the next call.
template <int NW>
__device__ __forceinline__ double block_sum_d(double v, double *scratch) {
    v = wave_sum_d(v);
    lds_barrier();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    lds_barrier();
    double r = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) r += scratch[w];
    return r;
}

template <int NW>
__device__ __forceinline__ uint64_t block_max_u64(uint64_t v, uint64_t *scratch) {
    v = wave_max_u64(v);
    lds_barrier();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    lds_barrier();
    uint64_t r = scratch[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = max_u64(r, scratch[w]);
    return r;
}

template <int NW>
__device__ __forceinline__ uint32_t block_sum_u(uint32_t v, uint32_t *scratch) {
    v = wave_sum_u(v);
    lds_barrier();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    lds_barrier();
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) r += scratch[w];
    return r;
}

template <int NW>
__device__ __forceinline__ uint32_t block_max_u(uint32_t v, uint32_t *scratch) {
    v = wave_max_u(v);
    lds_barrier();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    lds_barrier();
    uint32_t r = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) r = max(r, scratch[w]);
    return r;
}

}  // namespace sdv
