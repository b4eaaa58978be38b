// Wave64 and workgroup reductions for gfx950.
//
// The float/int wave reductions run the classic GFX9 DPP ladder: row_shr 1, 2,
// 4, 8 folds each row of 16 lanes into its lane 15, row_bcast:15 (rows 1 and 3)
// and row_bcast:31 (rows 2 and 3) fold the rows into lane 63, which is then
// read into a scalar.  Lanes whose DPP source is out of range keep the
// identity.  Double-precision and pair reductions use cross-lane shuffles.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <math.h>
#include <limits.h>

namespace sdv {

constexpr int kWave = 64;

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

__device__ __forceinline__ bool wave_any(bool p) { return __ballot(p) != 0ull; }

__device__ __forceinline__ double wave_sum_d(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ double wave_max_d(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v = fmax(v, __shfl_xor(v, m, kWave));
    return v;
}

__device__ __forceinline__ unsigned long long wave_sum_u64(unsigned long long v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
    return v;
}

__device__ __forceinline__ uint32_t wave_or_u32(uint32_t v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v |= __shfl_xor(v, m, kWave);
    return v;
}

// Largest key with its index (lowest index on equal keys) and the runner-up key.
struct Top2 {
    double k1;
    int i1;
    double k2;
};

__device__ __forceinline__ Top2 top2_empty() { return Top2{-INFINITY, INT_MAX, -INFINITY}; }

__device__ __forceinline__ void top2_push(Top2 &t, double key, int idx) {
    if (key > t.k1 || (key == t.k1 && idx < t.i1)) {
        t.k2 = t.k1;
        t.k1 = key;
        t.i1 = idx;
    } else if (key > t.k2) {
        t.k2 = key;
    }
}

__device__ __forceinline__ Top2 top2_merge(Top2 a, Top2 b) {
    if (b.k1 > a.k1 || (b.k1 == a.k1 && b.i1 < a.i1))
        return Top2{b.k1, b.i1, fmax(a.k1, b.k2)};
    return Top2{a.k1, a.i1, fmax(b.k1, a.k2)};
}

__device__ __forceinline__ Top2 wave_top2(Top2 t) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) {
        Top2 o{__shfl_xor(t.k1, m, kWave), __shfl_xor(t.i1, m, kWave), __shfl_xor(t.k2, m, kWave)};
        t = top2_merge(t, o);
    }
    return t;
}

// Workgroup-wide reductions for 256-thread workgroups (4 waves).  Every thread
// gets the result.  `scratch` must hold 4 elements and is reused after return.
__device__ __forceinline__ double block_sum_d(double v, double *scratch) {
    v = wave_sum_d(v);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[w] = v;
    __syncthreads();
    return scratch[0] + scratch[1] + scratch[2] + scratch[3];
}

__device__ __forceinline__ Top2 block_top2(Top2 t, Top2 *scratch) {
    t = wave_top2(t);
    const int w = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[w] = t;
    __syncthreads();
    Top2 r = scratch[0];
    r = top2_merge(r, scratch[1]);
    r = top2_merge(r, scratch[2]);
    r = top2_merge(r, scratch[3]);
    return r;
}

}  // namespace sdv
