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

__device__ __forceinline__ double wave_sum_d(double v) {
    v += dpp_d<0x111, 0xf>(0.0, v);
    v += dpp_d<0x112, 0xf>(0.0, v);
    v += dpp_d<0x114, 0xf>(0.0, v);
    v += dpp_d<0x118, 0xf>(0.0, v);
    v += dpp_d<0x142, 0xa>(0.0, v);
    v += dpp_d<0x143, 0xc>(0.0, v);
    return readlane_d(v, 63);
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

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ Top2 top2_step(Top2 t) {
    const Top2 o{dpp_d<CTRL, ROW_MASK>(-INFINITY, t.k1), dpp_i<CTRL, ROW_MASK>(INT_MAX, t.i1),
                 dpp_d<CTRL, ROW_MASK>(-INFINITY, t.k2)};
    return top2_merge(t, o);
}

// The wave's Top2, broadcast from lane 63 after the DPP ladder.
__device__ __forceinline__ Top2 wave_top2(Top2 t) {
    t = top2_step<0x111, 0xf>(t);
    t = top2_step<0x112, 0xf>(t);
    t = top2_step<0x114, 0xf>(t);
    t = top2_step<0x118, 0xf>(t);
    t = top2_step<0x142, 0xa>(t);
    t = top2_step<0x143, 0xc>(t);
    return Top2{readlane_d(t.k1, 63), __builtin_amdgcn_readlane(t.i1, 63), readlane_d(t.k2, 63)};
}

// Workgroup-wide reductions over NW waves.  Every thread gets the result.
// `scratch` holds NW elements and may be reused once the call returns.
template <int NW>
__device__ __forceinline__ double block_sum_d(double v, double *scratch) {
    v = wave_sum_d(v);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) r += scratch[w];
    return r;
}

template <int NW>
__device__ __forceinline__ Top2 block_top2(Top2 t, Top2 *scratch) {
    t = wave_top2(t);
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[threadIdx.x >> 6] = t;
    __syncthreads();
    Top2 r = scratch[0];
#pragma unroll
    for (int w = 1; w < NW; ++w) r = top2_merge(r, scratch[w]);
    return r;
}

}  // namespace sdv
