// MI355X (gfx950) speculative-decoding verifier: kernels and C ABI.
//
// Two kernels per call, both on the caller's stream:
//
//   row_stats  One wave64 per (row, chunk of blocks).  It streams the row's
//              logits from HBM in 16-byte loads, applies the grammar bitmask,
//              and for every block of 2048 tokens writes 8 bytes:
//                sampling rows: (Mc, Sc) with Mc = fp32(max_j l_j * c),
//                  Sc = sum_j 2^(l_j * c - Mc), c = log2(e) / T
//                greedy rows:   (max_j l_j, lowest index of that max)
//              This is the only pass over the full logits and moves > 99% of
//              the bytes (pyshine "vLLM, part 2", "Verification": logits in
//              fp32, temperature applied before normalising; "Grammar gates":
//              one mask row per request and position).
//   finalize   One 256-thread workgroup per request.  It folds the block
//              statistics into each row's max and normaliser, gathers p(x)
//              and q(x) at the drafts, draws the accept uniforms from Philox,
//              scans for the first rejection (vllm-learning code walkthrough,
//              RejectionSampler), then samples the emitted token from the
//              residual max(p - q, 0), from p with the draft removed (one-hot
//              drafts, infra-guide 5.2 section 4.3) or from p at the bonus
//              position, by two-level Gumbel-max: level 1 over block masses,
//              level 2 over the winning block's 2048 tokens (re-read, 4 KB).
//              It writes the outputs and a per-request record; the last
//              workgroup to finish sums the records into R, I, D, A (fanout,
//              "Name the three counters").
#include <hip/hip_runtime.h>
#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>

#include "sd_verify.h"
#include "philox.h"
#include "wave.h"

#ifndef SDV_BLOCKS_PER_WAVE
#define SDV_BLOCKS_PER_WAVE 4   // element kernel: 2048-token blocks per wave task
#endif
#ifndef SDV_ROW_STATS_GRID
#define SDV_ROW_STATS_GRID 2048 // vector kernel: workgroups of the block sweep
#endif

namespace sdv {

constexpr int kBlock = SD_BLOCK_TOKENS;
constexpr int kThreads = 256;       // row statistics: 4 waves per workgroup
constexpr int kFinalThreads = 512;  // finalize: 8 waves per request
constexpr int kFinalWaves = kFinalThreads / 64;
constexpr int kMaxDraft = SD_MAX_DRAFT;
constexpr double kLog2e = 1.4426950408889634;
constexpr double kLn2 = 0.6931471805599453;
constexpr double kAcceptFlagEps = 1e-6;
constexpr double kGumbelFlagEps = 1e-5;
constexpr int kRecordWords = 8;

// ------------------------------------------------------------- element access

template <typename ET>
struct Logit;

template <>
struct Logit<uint16_t> {  // bfloat16 stored as its bit pattern
    static constexpr int kPer16 = 8;
    __device__ static float to_float(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }
    __device__ static void unpack(uint4 w, float *o) {
        o[0] = __uint_as_float(w.x << 16);
        o[1] = __uint_as_float(w.x & 0xffff0000u);
        o[2] = __uint_as_float(w.y << 16);
        o[3] = __uint_as_float(w.y & 0xffff0000u);
        o[4] = __uint_as_float(w.z << 16);
        o[5] = __uint_as_float(w.z & 0xffff0000u);
        o[6] = __uint_as_float(w.w << 16);
        o[7] = __uint_as_float(w.w & 0xffff0000u);
    }
};

template <>
struct Logit<float> {
    static constexpr int kPer16 = 4;
    __device__ static float to_float(float f) { return f; }
    __device__ static void unpack(uint4 w, float *o) {
        o[0] = __uint_as_float(w.x);
        o[1] = __uint_as_float(w.y);
        o[2] = __uint_as_float(w.z);
        o[3] = __uint_as_float(w.w);
    }
};

// One 16-byte group of a row starting at token `tok` (a multiple of the group
// width).  Tokens at or beyond V read as -inf.  ALIGNED: the row is 16-byte
// aligned and V is a multiple of the group width, so a group is either wholly
// inside the row or wholly outside.
template <typename ET, bool ALIGNED>
__device__ __forceinline__ void load_group(const ET *row, int64_t tok, int V, float *o) {
    constexpr int P = Logit<ET>::kPer16;
    if (ALIGNED) {
        if (tok < V) {
            Logit<ET>::unpack(*reinterpret_cast<const uint4 *>(row + tok), o);
        } else {
#pragma unroll
            for (int e = 0; e < P; ++e) o[e] = -INFINITY;
        }
    } else {
#pragma unroll
        for (int e = 0; e < P; ++e) o[e] = (tok + e < V) ? Logit<ET>::to_float(row[tok + e]) : -INFINITY;
    }
}

// Mask bits of the P tokens starting at `tok` (tok % P == 0, P = 4 or 8).
template <int P>
__device__ __forceinline__ uint32_t mask_bits(const uint8_t *mrow, int64_t tok, int V) {
    if (tok >= V) return 0u;
    const uint32_t byte = mrow[tok >> 3];
    return P == 8 ? byte : (byte >> (uint32_t(tok) & 4u)) & 0xfu;
}

// Eight consecutive tokens j0 .. j0+7 (j0 % 8 == 0) of a row, masked.
template <typename ET, bool ALIGNED>
__device__ __forceinline__ void load8_masked(const ET *row, const uint32_t *mrow, int64_t j0, int V,
                                             float *o) {
    constexpr int P = Logit<ET>::kPer16;
#pragma unroll
    for (int g = 0; g < 8 / P; ++g) load_group<ET, ALIGNED>(row, j0 + g * P, V, o + g * P);
    if (mrow != nullptr && j0 < V) {
        const uint32_t bits = reinterpret_cast<const uint8_t *>(mrow)[j0 >> 3];
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if (!((bits >> e) & 1u)) o[e] = -INFINITY;
    }
}

template <typename ET>
__device__ __forceinline__ float load_one(const void *base, int64_t idx) {
    return Logit<ET>::to_float(reinterpret_cast<const ET *>(base)[idx]);
}

__device__ __forceinline__ float scale_of(float T) {
    return static_cast<float>(kLog2e / static_cast<double>(T));
}

// A wave-uniform read of memory no kernel of the call writes, through the
// constant address space so that it becomes a scalar load (its own counter,
// no wait on outstanding vector loads).
template <typename T>
__device__ __forceinline__ T uniform_load(const T *p) {
    typedef const __attribute__((address_space(4))) T ConstT;
    return *(ConstT *)(reinterpret_cast<uintptr_t>(p));
}

// Raw buffer resource over `bytes` bytes at p (GFX9 word 3: raw 32-bit
// format).  Loads at offsets >= bytes return zero instead of faulting.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void *p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), 0, static_cast<int>(bytes),
                                             kBufferWord3);
}

// ------------------------------------------------------------ row statistics

struct RowStatsArgs {
    const void *logits;
    const uint32_t *mask;     // nullptr = no bitmask
    const float *temperature;
    const int32_t *draft;     // [B, k]; nullptr when k = 0
    float2 *bstats;           // [rows, C]
    float *sx;                // [rows]: Sc of the draft's own block without the draft
    uint64_t *out_counters;   // zeroed here, accumulated by finalize
    uint32_t *status;         // zeroed here when given
    uint32_t *dbg_flags;      // zeroed here when given
    int64_t ntasks;           // rows * nchunk (chunked element kernel)
    int64_t nblk;             // rows * C (vector kernel sweep)
    int k, kp1, V, W, C, cpw, nchunk;
};

// Per-block statistics of a sampling row from one lane's values v (masked
// tokens and tokens past V hold -inf): (Mc, Sc) with Mc = fp32(max l * c) and
// Sc = sum 2^(l c - Mc).
template <int NV>
__device__ __forceinline__ float2 softmax_block(const float *v, float c) {
    float m = v[0];
#pragma unroll
    for (int e = 1; e < NV; ++e) m = fmaxf(m, v[e]);
    m = wave_max(m);
    if (m == -INFINITY) return make_float2(-INFINITY, 0.0f);
    const float mc = m * c;
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < NV; ++e) s += __builtin_amdgcn_exp2f(fmaf(v[e], c, -mc));
    return make_float2(mc, wave_sum(s));
}

// Greedy rows: the block's largest logit and the lowest index holding it
// (NaN when the block holds an allowed NaN).  Element (g, e) of a lane is
// token blk_base + (g * 64 + lane) * P + e.
template <int G, int P>
__device__ __forceinline__ float2 greedy_block(const float *v, int64_t blk_base, int lane) {
    constexpr int NV = G * P;
    float m = -INFINITY;
    bool nan = false;
#pragma unroll
    for (int e = 0; e < NV; ++e) {
        nan |= (v[e] != v[e]);
        m = fmaxf(m, v[e]);
    }
    if (wave_any(nan)) return make_float2(NAN, __int_as_float(-1));
    m = wave_max(m);
    if (m == -INFINITY) return make_float2(-INFINITY, __int_as_float(-1));
    int idx = INT_MAX;
#pragma unroll
    for (int g = G - 1; g >= 0; --g)
#pragma unroll
        for (int e = P - 1; e >= 0; --e)
            if (v[g * P + e] == m) idx = static_cast<int>(blk_base + (g * kWave + lane) * P + e);
    return make_float2(m, __int_as_float(wave_min_i(idx)));
}

__device__ __forceinline__ void zero_call_outputs(const RowStatsArgs &a) {
    if (blockIdx.x != 0) return;
    if (threadIdx.x < 4) a.out_counters[threadIdx.x] = 0ull;
    if (threadIdx.x == 0 && a.status) *a.status = 0u;
    if (threadIdx.x < 2 && a.dbg_flags) a.dbg_flags[threadIdx.x] = 0u;
}

// Which row a wave works on, and its parameters (all wave-uniform).
struct RowTask {
    int row, c0, c1;
    bool greedy, skip;
    float c;
    int xblk, xrel;  // the draft's block and offset in it (-1: none)
};

__device__ __forceinline__ RowTask row_task(const RowStatsArgs &a, int64_t task) {
    RowTask t;
    t.row = static_cast<int>(task / a.nchunk);
    const int chunk = static_cast<int>(task - int64_t(t.row) * a.nchunk);
    t.c0 = chunk * a.cpw;
    t.c1 = min(a.C, t.c0 + a.cpw);
    const int b = t.row / a.kp1, i = t.row - b * a.kp1;
    const float T = a.temperature[b];
    t.greedy = (T == 0.0f);
    t.skip = !t.greedy && !(T > 0.0f && T <= FLT_MAX);  // reported by finalize
    t.c = t.greedy ? 0.0f : scale_of(T);
    t.xblk = t.xrel = -1;
    if (!t.greedy && i < a.k) {
        const int x = a.draft[int64_t(b) * a.k + i];
        if (x >= 0 && x < a.V) {
            t.xblk = x / kBlock;
            t.xrel = x - t.xblk * kBlock;
        }
    }
    return t;
}

// Raw 16-byte groups and mask bytes of one block wholly inside the row: lane
// l reads groups l, l + 64, ... (consecutive lanes, consecutive 16 bytes).
template <typename ET, bool MASKED>
__device__ __forceinline__ void load_full_block(const ET *rowp, const uint8_t *mrow, int blk,
                                                int lane, uint4 *r, uint32_t *m) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    const uint4 *bp = reinterpret_cast<const uint4 *>(rowp + int64_t(blk) * kBlock) + lane;
#pragma unroll
    for (int g = 0; g < G; ++g) r[g] = bp[g * kWave];
    if (MASKED) {
        // P tokens per group: the group's bits sit in byte (first token) / 8
        const uint8_t *mb = mrow + int64_t(blk) * (kBlock / 8);
#pragma unroll
        for (int g = 0; g < G; ++g) m[g] = mb[((g * kWave + lane) * P) >> 3];
    }
}

template <typename ET, bool MASKED>
__device__ __forceinline__ void unpack_full_block(const uint4 *r, const uint32_t *m, int lane,
                                                  float *v) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        Logit<ET>::unpack(r[g], v + g * P);
        if (MASKED) {
            const uint32_t bits = (P == 8) ? m[g] : (m[g] >> ((lane & 1) * 4));
#pragma unroll
            for (int e = 0; e < P; ++e)
                if (!((bits >> e) & 1u)) v[g * P + e] = -INFINITY;
        }
    }
}

// Values of one lane for any block (used for the row's partial last block and
// for re-reads): addresses clamped into the row, tokens past V and masked
// tokens become -inf.
template <typename ET, bool MASKED>
__device__ __forceinline__ void load_any_block(const ET *rowp, const uint8_t *mrow, int blk, int V,
                                               int lane, float *v) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    uint4 r[G];
    uint32_t m[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t tok = int64_t(blk) * kBlock + (g * kWave + lane) * P;
        const int64_t tc = tok < V ? tok : int64_t(V - P);
        r[g] = *reinterpret_cast<const uint4 *>(rowp + tc);
        m[g] = MASKED ? uint32_t(mrow[tc >> 3]) : 0xffu;
    }
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t tok = int64_t(blk) * kBlock + (g * kWave + lane) * P;
        Logit<ET>::unpack(r[g], v + g * P);
        uint32_t bits = tok < V ? 0xffu : 0u;
        if (MASKED) bits &= (P == 8) ? m[g] : (m[g] >> (uint32_t(tok) & 4u));
#pragma unroll
        for (int e = 0; e < P; ++e)
            if (!((bits >> e) & 1u)) v[g * P + e] = -INFINITY;
    }
}

template <bool GREEDY, int G, int P>
__device__ __forceinline__ void store_block(const RowStatsArgs &a, const RowTask &t, const float *v,
                                            int blk, int lane) {
    const float2 r = GREEDY ? greedy_block<G, P>(v, int64_t(blk) * kBlock, lane)
                            : softmax_block<G * P>(v, t.c);
    if (lane == 0) a.bstats[int64_t(t.row) * a.C + blk] = r;
}

// The sum of the draft's own block without the draft (the one-hot residual
// mass of that block), relative to the same Mc as the block statistics.
template <int G, int P>
__device__ __forceinline__ void store_excluded_sum(const RowStatsArgs &a, int row, float c, int xrel,
                                                   const float *v, int lane) {
    constexpr int NV = G * P;
    float m = v[0];
#pragma unroll
    for (int e = 1; e < NV; ++e) m = fmaxf(m, v[e]);
    m = wave_max(m);
    float s = 0.0f;
    if (m > -INFINITY) {
        const float mc = m * c;
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < P; ++e)
                if ((g * kWave + lane) * P + e != xrel)
                    s += __builtin_amdgcn_exp2f(fmaf(v[g * P + e], c, -mc));
    }
    s = wave_sum(s);
    if (lane == 0) a.sx[row] = s;
}

// One block's share of the sweep: where it lives and its row's parameters.
struct SweepBlock {
    int64_t gb;   // row * C + block
    int row, blk;
    bool full, greedy, skip;
    float c;
    int xrel;     // the draft's offset in this block, -1 if the draft is elsewhere
};

__device__ __forceinline__ SweepBlock sweep_block(const RowStatsArgs &a, int64_t gb) {
    SweepBlock s;
    s.gb = gb;
    s.row = static_cast<int>(gb / a.C);
    s.blk = static_cast<int>(gb - int64_t(s.row) * a.C);
    s.full = int64_t(s.blk + 1) * kBlock <= a.V;
    const int b = s.row / a.kp1, i = s.row - b * a.kp1;
    const float T = uniform_load(a.temperature + b);
    s.greedy = (T == 0.0f);
    s.skip = !s.greedy && !(T > 0.0f && T <= FLT_MAX);  // reported by finalize
    s.c = s.greedy ? 0.0f : scale_of(T);
    s.xrel = -1;
    if (!s.greedy && i < a.k) {
        const int x = uniform_load(a.draft + int64_t(b) * a.k + i);
        if (x >= 0 && x < a.V && x / kBlock == s.blk) s.xrel = x - s.blk * kBlock;
    }
    return s;
}

// Issue the loads of one block through buffer resources spanning its row (and
// its mask row): every block takes the same instructions, and the groups of a
// partial block that lie past the row read zeros (they are replaced by -inf
// when the block is reduced).
template <typename ET, bool MASKED>
__device__ __forceinline__ void issue_block(const RowStatsArgs &a, const SweepBlock &s, int lane,
                                            uint4 *r, uint32_t *m) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    const __amdgpu_buffer_rsrc_t rs = buffer_of(
        reinterpret_cast<const ET *>(a.logits) + int64_t(s.row) * a.V, uint32_t(a.V) * sizeof(ET));
    const int base = s.blk * kBlock * int(sizeof(ET)) + lane * 16;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, base + g * kWave * 16, 0, 0);
        r[g] = make_uint4(w.x, w.y, w.z, w.w);
    }
    if (MASKED) {
        const __amdgpu_buffer_rsrc_t rm = buffer_of(a.mask + int64_t(s.row) * a.W, uint32_t(a.W) * 4u);
        const int mbase = s.blk * (kBlock / 8) + ((lane * P) >> 3);
#pragma unroll
        for (int g = 0; g < G; ++g)
            m[g] = __builtin_amdgcn_raw_buffer_load_b8(rm, mbase + g * kWave * P / 8, 0, 0);
    }
}

template <typename ET, bool MASKED>
__device__ __forceinline__ void reduce_block(const RowStatsArgs &a, const SweepBlock &s, int lane,
                                             const uint4 *r, const uint32_t *m) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    if (s.skip) return;
    float v[G * P];
    if (s.full) {
        unpack_full_block<ET, MASKED>(r, m, lane, v);
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t tok = int64_t(s.blk) * kBlock + (g * kWave + lane) * P;
            Logit<ET>::unpack(r[g], v + g * P);
            uint32_t bits = tok < a.V ? 0xffu : 0u;
            if (MASKED) bits &= (P == 8) ? m[g] : (m[g] >> (uint32_t(tok) & 4u));
#pragma unroll
            for (int e = 0; e < P; ++e)
                if (!((bits >> e) & 1u)) v[g * P + e] = -INFINITY;
        }
    }
    float2 res;
    if (s.greedy) {
        res = greedy_block<G, P>(v, int64_t(s.blk) * kBlock, lane);
    } else {
        res = softmax_block<G * P>(v, s.c);
        if (s.xrel >= 0) store_excluded_sum<G, P>(a, s.row, s.c, s.xrel, v, lane);
    }
    if (lane == 0) a.bstats[s.gb] = res;
}

// Rows 16-byte aligned with V a multiple of the group width.  The grid sweeps
// the (row, block) pairs in memory order: wave w of the grid takes blocks
// w, w + Wt, w + 2 Wt, ... (Wt = waves in the grid), so the whole grid reads
// one contiguous window of the logits at a time.  Each wave keeps the loads of
// its next block in flight while it reduces the current one; the next index
// is clamped to the current block at the end of the sweep, so every path
// reaches a reduction with the same loads outstanding.
template <typename ET, bool MASKED>
__global__ __launch_bounds__(kThreads) void row_stats_vec_kernel(RowStatsArgs a) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    zero_call_outputs(a);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t stride = int64_t(gridDim.x) * (kThreads / kWave);
    int64_t g0 = int64_t(blockIdx.x) * (kThreads / kWave) + wave_id();
    if (g0 >= a.nblk) return;
    uint4 ra[G], rb[G];
    uint32_t ma[G], mb[G];
    SweepBlock sa = sweep_block(a, g0);
    issue_block<ET, MASKED>(a, sa, lane, ra, ma);
    for (;;) {
        const int64_t g1 = sa.gb + stride;
        const bool more1 = g1 < a.nblk;
        const SweepBlock sb = sweep_block(a, more1 ? g1 : sa.gb);
        issue_block<ET, MASKED>(a, sb, lane, rb, mb);
        reduce_block<ET, MASKED>(a, sa, lane, ra, ma);
        if (!more1) break;
        const int64_t g2 = sb.gb + stride;
        const bool more2 = g2 < a.nblk;
        sa = sweep_block(a, more2 ? g2 : sb.gb);
        issue_block<ET, MASKED>(a, sa, lane, ra, ma);
        reduce_block<ET, MASKED>(a, sb, lane, rb, mb);
        if (!more2) break;
    }
}

// Any alignment and any V: element loads clamped into the row.
template <typename ET, bool MASKED>
__device__ __forceinline__ void load_block_elem(const ET *rowp, const uint8_t *mrow, int blk, int V,
                                                int lane, float *v) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
#pragma unroll
    for (int g = 0; g < G; ++g)
#pragma unroll
        for (int e = 0; e < P; ++e) {
            const int64_t tok = int64_t(blk) * kBlock + (g * kWave + lane) * P + e;
            const int64_t tc = tok < V ? tok : int64_t(V - 1);
            const float x = Logit<ET>::to_float(rowp[tc]);
            bool live = tok < V;
            if (MASKED) live = live && ((mrow[tc >> 3] >> (tc & 7)) & 1u);
            v[g * P + e] = live ? x : -INFINITY;
        }
}

template <typename ET, bool MASKED>
__global__ __launch_bounds__(kThreads) void row_stats_elem_kernel(RowStatsArgs a) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    zero_call_outputs(a);
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t task = int64_t(blockIdx.x) * (kThreads / kWave) + wave_id();
    if (task >= a.ntasks) return;
    const RowTask t = row_task(a, task);
    if (t.skip) return;
    const ET *rowp = reinterpret_cast<const ET *>(a.logits) + int64_t(t.row) * a.V;
    const uint8_t *mrow =
        MASKED ? reinterpret_cast<const uint8_t *>(a.mask + int64_t(t.row) * a.W) : nullptr;
    float v[G * P];
    for (int blk = t.c0; blk < t.c1; ++blk) {
        load_block_elem<ET, MASKED>(rowp, mrow, blk, a.V, lane, v);
        if (t.greedy) {
            store_block<true, G, P>(a, t, v, blk, lane);
        } else {
            store_block<false, G, P>(a, t, v, blk, lane);
            if (blk == t.xblk) store_excluded_sum<G, P>(a, t.row, t.c, t.xrel, v, lane);
        }
    }
}

// ------------------------------------------------------------------ finalize

struct FinalArgs {
    const void *logits;
    const int32_t *draft;
    const float *q;        // nullptr = one-hot drafts
    const uint32_t *mask;  // nullptr = no bitmask
    const float *temperature;
    uint64_t seed;
    int32_t *out_tokens;
    int32_t *out_num_accepted;
    uint64_t *out_counters;
    double *dbg_lse;
    double *dbg_acc;
    uint32_t *dbg_req_flags;
    uint32_t *dbg_flags;
    uint32_t *status;
    const float2 *bstats;
    const float *sx;
    int B, k, V, W, C;
};

enum SampleMode { kModeP = 0, kModeOneHot = 1, kModeDense = 2 };

struct Level1 {
    int c;     // winning block, -1 when no block has mass
    int flag;  // 1 when the top-2 block keys are closer than the flag threshold
};

struct FinalShared {
    float M[kMaxDraft + 1];     // per row: fp32 max (log2 units), or greedy max logit
    double S[kMaxDraft + 1];    // per row: sum of 2^(t - M)
    int G[kMaxDraft + 1];       // greedy argmax
    Level1 l1p[kMaxDraft + 1];  // level-1 winner under p
    Level1 l1x[kMaxDraft + 1];  // level-1 winner under p without the row's draft
    int X[kMaxDraft];
    double acc[kMaxDraft];
    unsigned char ok[kMaxDraft], flag[kMaxDraft], invalid[kMaxDraft];
    uint32_t status;
    int nacc, flag_acc, ninvalid;
    int staged_c;               // block of the sampled row held in blockv (-1: none)
    double red_d[kFinalWaves];
    Top2 red_t[kFinalWaves];
    float blockv[kBlock];       // that block's logits, -inf where masked or past V
};

// Workgroup barrier that orders LDS only: global loads a wave has in flight
// stay in flight across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ Level1 level1_of(const Top2 &t) {
    if (t.k1 == -INFINITY) return Level1{-1, 0};
    return Level1{t.i1, (t.k2 > -INFINITY && t.k1 - t.k2 < kGumbelFlagEps) ? 1 : 0};
}

// Residual masses W_c = sum_j max(p_j - q_j, 0) of one row for dense q, with
// p_j = 2^(l_j c - M) / S in fp32.  One wave per block; clamped loads.
template <typename ET, bool ALIGNED>
__device__ void dense_block_masses(const ET *rowp, const uint32_t *mrow, const float *qrow, int V,
                                   int C, float c, float M, double S, double *Wout) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    const int lane = threadIdx.x & (kWave - 1);
    const float invS = static_cast<float>(1.0 / S);
    const uint8_t *mb = reinterpret_cast<const uint8_t *>(mrow);
    for (int blk = wave_id(); blk < C; blk += kFinalWaves) {
        float acc = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t tok = int64_t(blk) * kBlock + (g * kWave + lane) * P;
            float lv[P], qv[P];
            if (ALIGNED) {
                const int64_t tc = tok < V ? tok : int64_t(V - P);
                Logit<ET>::unpack(*reinterpret_cast<const uint4 *>(rowp + tc), lv);
#pragma unroll
                for (int h = 0; h < P / 4; ++h) {
                    const float4 f = *reinterpret_cast<const float4 *>(qrow + tc + 4 * h);
                    qv[4 * h] = f.x;
                    qv[4 * h + 1] = f.y;
                    qv[4 * h + 2] = f.z;
                    qv[4 * h + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < P; ++e) {
                    const int64_t tc = tok + e < V ? tok + e : int64_t(V - 1);
                    lv[e] = Logit<ET>::to_float(rowp[tc]);
                    qv[e] = qrow[tc];
                }
            }
#pragma unroll
            for (int e = 0; e < P; ++e) {
                const int64_t j = tok + e;
                const int64_t jc = j < V ? j : int64_t(V - 1);
                bool live = j < V && lv[e] > -INFINITY;
                if (mrow) live = live && ((mb[jc >> 3] >> (jc & 7)) & 1u);
                const float p = live ? __builtin_amdgcn_exp2f(fmaf(lv[e], c, -M)) * invS : 0.0f;
                acc += live ? fmaxf(p - qv[e], 0.0f) : 0.0f;
            }
        }
        const double w = wave_sum_d(static_cast<double>(acc));
        if (lane == 0) Wout[blk] = w;
    }
}

// Four consecutive tokens j0 .. j0+3 (j0 % 4 == 0) of a row, masked; tokens
// past V read as -inf.
template <typename ET, bool ALIGNED>
__device__ __forceinline__ void load4_masked(const ET *row, const uint32_t *mrow, int64_t j0, int V,
                                             float *o) {
    if (ALIGNED && j0 < V) {  // V is a multiple of 4 (fp32) or 8 (bf16): all four exist
        if (sizeof(ET) == 2) {
            const uint2 w = *reinterpret_cast<const uint2 *>(row + j0);
            o[0] = __uint_as_float(w.x << 16);
            o[1] = __uint_as_float(w.x & 0xffff0000u);
            o[2] = __uint_as_float(w.y << 16);
            o[3] = __uint_as_float(w.y & 0xffff0000u);
        } else {
            const float4 f = *reinterpret_cast<const float4 *>(row + j0);
            o[0] = f.x;
            o[1] = f.y;
            o[2] = f.z;
            o[3] = f.w;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) o[e] = (j0 + e < V) ? Logit<ET>::to_float(row[j0 + e]) : -INFINITY;
    }
    if (mrow != nullptr && j0 < V) {
        const uint32_t bits = reinterpret_cast<const uint8_t *>(mrow)[j0 >> 3] >> (uint32_t(j0) & 4u);
#pragma unroll
        for (int e = 0; e < 4; ++e)
            if (!((bits >> e) & 1u)) o[e] = -INFINITY;
    }
}

// Level 2: the token of block cb of row n drawn under the weights of `mode`
// (4 tokens per thread; values from the staged LDS copy when `staged`).  All
// threads call it; returns (token, near-tie flag), token -1 when the block
// holds no positive weight.
template <typename ET, bool ALIGNED>
__device__ int2 level2(const FinalArgs &a, FinalShared &sh, int b, int n, int cb, int mode, float c,
                       double invT, const float *qrow, bool staged) {
    const int k = a.k, V = a.V;
    const int64_t row = int64_t(b) * (k + 1) + n;
    const int x = (n < k) ? sh.X[n] : -1;
    const int64_t j0 = int64_t(cb) * kBlock + threadIdx.x * 4;
    float lv[4];
    if (staged) {
        const float4 f = *reinterpret_cast<const float4 *>(&sh.blockv[threadIdx.x * 4]);
        lv[0] = f.x;
        lv[1] = f.y;
        lv[2] = f.z;
        lv[3] = f.w;
    } else {
        load4_masked<ET, ALIGNED>(reinterpret_cast<const ET *>(a.logits) + row * V,
                                  a.mask ? a.mask + row * a.W : nullptr, j0, V, lv);
    }
    float g[4];
    draw_token_gumbels4(key_of(a.seed), b, n, static_cast<uint32_t>(j0), g);
    const float M = sh.M[n];
    const double S = sh.S[n];
    Top2 t = top2_empty();
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t j = j0 + e;
        if (!(lv[e] > -INFINITY)) continue;  // masked, -inf, or past V
        double key2;
        if (mode == kModeDense) {
            const double p = exp2(static_cast<double>(lv[e]) * c - static_cast<double>(M)) / S;
            const double r = p - static_cast<double>(qrow[j]);
            if (!(r > 0.0)) continue;
            key2 = log(r);
        } else {
            if (mode == kModeOneHot && j == x) continue;
            key2 = static_cast<double>(lv[e]) * invT;
        }
        top2_push(t, key2 + static_cast<double>(g[e]), static_cast<int>(j));
    }
    t = block_top2<kFinalWaves>(t, sh.red_t);
    if (t.k1 == -INFINITY) return make_int2(-1, 0);
    return make_int2(t.i1, (t.k2 > -INFINITY && t.k1 - t.k2 < kGumbelFlagEps) ? 1 : 0);
}

// Fold one greedy row's block statistics (one wave): max and lowest argmax.
__device__ __forceinline__ void fold_greedy_row(const float2 *st, int C, int i, FinalShared &sh) {
    const int lane = threadIdx.x & (kWave - 1);
    bool bad = false;
    float best = -INFINITY;
    int bidx = INT_MAX;
    for (int cb = lane; cb < C; cb += kWave) {
        const float2 e = st[cb];
        if (e.x != e.x || e.x == INFINITY) bad = true;
        if (e.x > best) {
            best = e.x;
            bidx = __float_as_int(e.y);
        }
    }
    bad = wave_any(bad);
    const float m = wave_max(best);
    const int gi = wave_min_i(best == m ? bidx : INT_MAX);
    if (lane == 0) {
        sh.M[i] = m;
        sh.G[i] = gi;
        sh.S[i] = 1.0;
        if (bad) atomicOr(&sh.status, SD_STATUS_BAD_LOGIT);
        else if (m == -INFINITY) atomicOr(&sh.status, SD_STATUS_EMPTY_ROW);
    }
}

// Fold one sampling row's block statistics (one wave) into its max and
// normaliser, and run the row's level-1 Gumbel race over block masses, both
// under p and under p without block cx's draft (mass sxi instead of Sc).
__device__ __forceinline__ void fold_sampling_row(const float2 *st, int C, int i, int b, int cx,
                                                  float sxi, PhiloxKey key, FinalShared &sh) {
    const int lane = threadIdx.x & (kWave - 1);
    bool bad = false;
    float mx = -INFINITY;
    for (int cb = lane; cb < C; cb += kWave) {
        const float2 e = st[cb];
        if (e.x != e.x || e.y != e.y || e.x == INFINITY) bad = true;
        mx = fmaxf(mx, e.x);
    }
    bad = wave_any(bad);
    const float m = wave_max(mx);
    double s = 0.0;
    Top2 tp = top2_empty(), tx = top2_empty();
    if (!bad && m > -INFINITY) {
        const int ngroups = (C + 3) >> 2;
        for (int g4 = lane; g4 < ngroups; g4 += kWave) {
            float gum[4];
            draw_block_gumbels4(key, b, i, g4, gum);
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int cb = 4 * g4 + q;
                if (cb >= C) break;
                const float2 e = st[cb];
                if (!(e.x > -INFINITY) || !(e.y > 0.0f)) continue;
                const double dm = static_cast<double>(e.x) - static_cast<double>(m);
                s += static_cast<double>(e.y) * exp2(dm);
                const double gq = static_cast<double>(gum[q]);
                const double kp = static_cast<double>(logf(e.y)) + dm * kLn2 + gq;
                top2_push(tp, kp, cb);
                if (cb != cx) {
                    top2_push(tx, kp, cb);
                } else if (sxi > 0.0f) {
                    top2_push(tx, static_cast<double>(logf(sxi)) + dm * kLn2 + gq, cb);
                }
            }
        }
    }
    s = wave_sum_d(s);
    tp = wave_top2(tp);
    tx = wave_top2(tx);
    if (lane == 0) {
        sh.M[i] = m;
        sh.S[i] = s;
        sh.G[i] = -1;
        sh.l1p[i] = level1_of(tp);
        sh.l1x[i] = level1_of(tx);
        if (bad) atomicOr(&sh.status, SD_STATUS_BAD_LOGIT);
        else if (m == -INFINITY) atomicOr(&sh.status, SD_STATUS_EMPTY_ROW);
    }
}

template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(kFinalThreads) void finalize_kernel(FinalArgs a) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    __shared__ FinalShared sh;
    extern __shared__ double sW[];  // dense q: per-block residual mass [C]
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    const int k = a.k, kp1 = a.k + 1, V = a.V, C = a.C;
    const float T = uniform_load(a.temperature + b);
    const bool greedy = (T == 0.0f);
    const bool bad_T = !greedy && !(T > 0.0f && T <= FLT_MAX);
    const PhiloxKey key = key_of(a.seed);
    const float c = greedy || bad_T ? 0.0f : scale_of(T);
    const bool one_hot = a.q == nullptr;

    // ---- drafts, and the gathers at the drafts
    int x = -1;
    if (tid < k) x = a.draft[int64_t(b) * k + tid];
    const bool xok = tid < k && x >= 0 && x < V;
    float lx = 0.0f, qx = 1.0f;
    uint32_t mw = 0xffffffffu;
    if (xok && !bad_T) {
        const int64_t rowi = int64_t(b) * kp1 + tid;
        if (!greedy) lx = load_one<ET>(a.logits, rowi * V + x);
        if (a.mask) mw = a.mask[rowi * a.W + (x >> 5)];
        if (!greedy && !one_hot) qx = a.q[(int64_t(b) * k + tid) * V + x];
    }
    if (tid == 0) {
        sh.status = bad_T ? SD_STATUS_TEMPERATURE : 0u;
        sh.nacc = 0;
        sh.flag_acc = 0;
        sh.ninvalid = 0;
        sh.staged_c = -1;
    }
    __syncthreads();
    if (tid < k) {
        sh.X[tid] = x;
        if (!xok) atomicOr(&sh.status, SD_STATUS_DRAFT_ID);
    }
    __syncthreads();

    // ---- one wave per row: fold the block statistics; sampling rows also run
    //      their level-1 race and start loading the block they would sample
    uint4 stage_r[G];
    uint32_t stage_m[G];
    int stage_row = -1, stage_c = -1;
    if (!bad_T) {
        for (int i = wave; i < kp1; i += kFinalWaves) {
            const int64_t row = int64_t(b) * kp1 + i;
            const float2 *st = a.bstats + row * C;
            if (greedy) {
                fold_greedy_row(st, C, i, sh);
                continue;
            }
            const int xi = (i < k) ? sh.X[i] : -1;
            const int cx = (one_hot && xi >= 0 && xi < V) ? xi / kBlock : -1;
            const float sxi = cx >= 0 ? uniform_load(a.sx + row) : 0.0f;
            fold_sampling_row(st, C, i, b, cx, sxi, key, sh);
            if (ALIGNED && kp1 <= kFinalWaves) {
                const Level1 l1 = (i < k) ? (one_hot ? sh.l1x[i] : Level1{-1, 0}) : sh.l1p[i];
                if (l1.c >= 0) {
                    RowStatsArgs ra;  // only the fields issue_block reads
                    ra.logits = a.logits;
                    ra.mask = a.mask;
                    ra.V = V;
                    ra.W = a.W;
                    SweepBlock sb;
                    sb.row = static_cast<int>(row);
                    sb.blk = l1.c;
                    if (a.mask) issue_block<ET, true>(ra, sb, lane, stage_r, stage_m);
                    else issue_block<ET, false>(ra, sb, lane, stage_r, stage_m);
                    stage_row = i;
                    stage_c = l1.c;
                }
            }
        }
    }
    lds_barrier();

    // ---- per-position accept probabilities and verdicts
    if (sh.status == 0 && tid < k) {
        const int i = tid;
        const bool allowed = (mw >> (x & 31)) & 1u;
        sh.invalid[i] = !allowed;
        double acc;
        bool ok, flag = false;
        if (greedy) {
            ok = (x == sh.G[i]);
            acc = ok ? 1.0 : 0.0;
        } else {
            double p = 0.0;
            if (allowed && lx > -INFINITY)
                p = exp2(static_cast<double>(lx) * c - static_cast<double>(sh.M[i])) / sh.S[i];
            if (!one_hot && !(qx >= 0.0f && qx <= FLT_MAX))
                atomicOr(&sh.status, SD_STATUS_BAD_DRAFT_PROB);
            const double q = qx;
            acc = (p == 0.0) ? 0.0 : (q == 0.0 ? 1.0 : fmin(1.0, p / q));
            const double u = draw_accept(key, b, i);
            ok = u < acc;
            flag = fabs(u - acc) < kAcceptFlagEps;
        }
        sh.acc[i] = acc;
        sh.ok[i] = ok;
        sh.flag[i] = flag;
    }
    lds_barrier();
    if (tid == 0 && sh.status == 0) {
        int n = 0, fa = 0, inv = 0;
        while (n < k && sh.ok[n]) fa += sh.flag[n++];
        if (n < k) fa += sh.flag[n];
        for (int i = 0; i < k; ++i) inv += sh.invalid[i];
        sh.nacc = n;
        sh.flag_acc = fa;
        sh.ninvalid = inv;
    }
    lds_barrier();

    // ---- the wave that loaded the sampled row's block puts it in LDS
    if (sh.status == 0 && stage_row >= 0 && stage_row == sh.nacc) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float v[P];
            Logit<ET>::unpack(stage_r[g], v);
            const int off = (g * kWave + lane) * P;  // token offset inside the block
            const int64_t tok = int64_t(stage_c) * kBlock + off;
            uint32_t bits = tok < V ? 0xffu : 0u;
            if (a.mask) bits &= (P == 8) ? stage_m[g] : (stage_m[g] >> (uint32_t(tok) & 4u));
#pragma unroll
            for (int e = 0; e < P; ++e)
                if (!((bits >> e) & 1u)) v[e] = -INFINITY;
#pragma unroll
            for (int h = 0; h < P / 4; ++h)
                *reinterpret_cast<float4 *>(&sh.blockv[off + 4 * h]) =
                    make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
        }
        if (lane == 0) sh.staged_c = stage_c;
    }
    __syncthreads();

    // ---- the emitted token
    const uint32_t st = sh.status;
    int y = -1, fg = 0;
    if (st == 0) {
        const int n = sh.nacc;
        if (greedy) {
            y = sh.G[n];
        } else {
            const double invT = 1.0 / static_cast<double>(T);
            const float *qrow = (n < k && !one_hot) ? a.q + (int64_t(b) * k + n) * V : nullptr;
            int mode = (n == k) ? kModeP : (one_hot ? kModeOneHot : kModeDense);
            Level1 l1 = (mode == kModeOneHot) ? sh.l1x[n] : sh.l1p[n];
            if (mode == kModeDense) {
                const int64_t row = int64_t(b) * kp1 + n;
                dense_block_masses<ET, ALIGNED>(
                    reinterpret_cast<const ET *>(a.logits) + row * V,
                    a.mask ? a.mask + row * a.W : nullptr, qrow, V, C, c, sh.M[n], sh.S[n], sW);
                __syncthreads();
                Top2 t = top2_empty();
                const int ngroups = (C + 3) >> 2;
                for (int g4 = tid; g4 < ngroups; g4 += kFinalThreads) {
                    float gum[4];
                    draw_block_gumbels4(key, b, n, g4, gum);
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int cb = 4 * g4 + q;
                        if (cb < C && sW[cb] > 0.0)
                            top2_push(t, log(sW[cb]) + static_cast<double>(gum[q]), cb);
                    }
                }
                l1 = level1_of(block_top2<kFinalWaves>(t, sh.red_t));
            }
            if (l1.c < 0) {  // no residual mass: draw from p instead
                mode = kModeP;
                l1 = sh.l1p[n];
            }
            int2 r2 = level2<ET, ALIGNED>(a, sh, b, n, l1.c, mode, c, invT, qrow, sh.staged_c == l1.c);
            if (r2.x < 0 && mode != kModeP) {  // the block lost its mass in double precision
                mode = kModeP;
                l1 = sh.l1p[n];
                r2 = level2<ET, ALIGNED>(a, sh, b, n, l1.c, mode, c, invT, qrow, sh.staged_c == l1.c);
            }
            y = r2.x;
            fg = l1.flag + r2.y;
        }
    }

    // ---- outputs, and this request's share of the counters
    const int n = st ? -1 : sh.nacc;
    if (tid < kp1) {
        int tok = -1;
        if (!st) tok = tid < n ? sh.X[tid] : (tid == n ? y : -1);
        a.out_tokens[int64_t(b) * kp1 + tid] = tok;
        if (a.dbg_lse) {
            double v = NAN;
            if (!st) v = greedy ? static_cast<double>(sh.M[tid])
                                : kLn2 * (static_cast<double>(sh.M[tid]) + log2(sh.S[tid]));
            a.dbg_lse[int64_t(b) * kp1 + tid] = v;
        }
    }
    if (tid < k && a.dbg_acc) a.dbg_acc[int64_t(b) * k + tid] = st ? NAN : sh.acc[tid];
    if (tid == 0) {
        a.out_num_accepted[b] = n;
        if (st) {
            if (a.status) atomicOr(a.status, st);
        } else {
            // integer atomics: the sums do not depend on the order of arrival
            atomicAdd(&a.out_counters[0], static_cast<unsigned long long>(k));
            if (sh.ninvalid) atomicAdd(&a.out_counters[1], static_cast<unsigned long long>(sh.ninvalid));
            atomicAdd(&a.out_counters[2], static_cast<unsigned long long>(k - sh.ninvalid));
            if (n) atomicAdd(&a.out_counters[3], static_cast<unsigned long long>(n));
            if (a.dbg_flags) {
                if (sh.flag_acc) atomicAdd(&a.dbg_flags[0], static_cast<uint32_t>(sh.flag_acc));
                if (fg) atomicAdd(&a.dbg_flags[1], static_cast<uint32_t>(fg));
            }
        }
        if (a.dbg_req_flags)
            a.dbg_req_flags[b] = st ? 0u : (uint32_t(min(sh.flag_acc, 0xffff)) | (uint32_t(fg) << 16));
    }
}

// Outputs of an empty batch: zero counters, status and flags.
__global__ void empty_batch_kernel(uint64_t *counters, uint32_t *status, uint32_t *flags) {
    if (threadIdx.x < 4) counters[threadIdx.x] = 0ull;
    if (threadIdx.x == 0 && status) *status = 0u;
    if (threadIdx.x < 2 && flags) flags[threadIdx.x] = 0u;
}

// ------------------------------------------------------------------ dispatch

using RowStatsFn = void (*)(RowStatsArgs);
using FinalFn = void (*)(FinalArgs);

template <typename ET>
RowStatsFn pick_row_stats(bool masked, bool aligned) {
    if (aligned) return masked ? row_stats_vec_kernel<ET, true> : row_stats_vec_kernel<ET, false>;
    return masked ? row_stats_elem_kernel<ET, true> : row_stats_elem_kernel<ET, false>;
}

template <typename ET>
FinalFn pick_final(bool aligned) {
    return aligned ? finalize_kernel<ET, true> : finalize_kernel<ET, false>;
}

struct Layout {
    int64_t rows;
    int C, W, nchunk;
    size_t off_bstats, off_sx, total;
};

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

inline bool sizes_ok(const sd_params *p) {
    return p && p->batch >= 0 && p->num_draft >= 0 && p->num_draft <= SD_MAX_DRAFT &&
           p->vocab >= 1 && p->vocab <= SD_MAX_VOCAB;
}

inline Layout layout_of(const sd_params *p) {
    Layout L{};
    L.rows = int64_t(p->batch) * (p->num_draft + 1);
    L.C = (p->vocab + kBlock - 1) / kBlock;
    L.W = (p->vocab + 31) / 32;
    L.nchunk = (L.C + SDV_BLOCKS_PER_WAVE - 1) / SDV_BLOCKS_PER_WAVE;
    L.off_bstats = 0;
    L.off_sx = align256(size_t(L.rows) * L.C * sizeof(float2));
    L.total = L.off_sx + align256(size_t(L.rows) * sizeof(float));
    return L;
}

}  // namespace sdv

// ---------------------------------------------------------------------- C ABI

extern "C" size_t sd_verify_workspace_size(const sd_params *p) {
    if (!sdv::sizes_ok(p) || p->batch == 0) return 0;
    return sdv::layout_of(p).total;
}

extern "C" const char *sd_status_string(int code) {
    switch (code) {
        case SD_OK: return "ok";
        case SD_ERR_INVALID_ARG: return "invalid argument";
        case SD_ERR_UNSUPPORTED: return "unsupported size";
        case SD_ERR_WORKSPACE: return "workspace missing or too small";
        case SD_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

extern "C" int sd_rates(const uint64_t *counters, uint64_t steps, double *out) {
    if (!counters || !out) return SD_ERR_INVALID_ARG;
    const uint64_t R = counters[0], I = counters[1], D = counters[2], A = counters[3];
    if (I > R || D != R - I || A > D) return SD_ERR_INVALID_ARG;
    out[0] = R ? double(D) / double(R) : NAN;           // grammar survival
    out[1] = D ? double(A) / double(D) : NAN;           // conditional acceptance
    out[2] = R ? double(A) / double(R) : NAN;           // end-to-end yield
    out[3] = steps ? 1.0 + double(A) / double(steps) : NAN;  // mean acceptance length
    return SD_OK;
}

extern "C" int sd_verify(const void *target_logits, const int32_t *draft_token_ids,
                         const float *draft_probs, const int32_t *bitmask,
                         const float *temperature, uint64_t seed, int32_t *out_tokens,
                         int32_t *out_num_accepted, uint64_t *out_counters, const sd_params *p,
                         void *workspace, size_t workspace_bytes, hipStream_t stream) {
    using namespace sdv;
    if (!p || !out_counters) return SD_ERR_INVALID_ARG;
    if (p->batch < 0 || p->num_draft < 0 || p->vocab < 1) return SD_ERR_INVALID_ARG;
    if (p->logits_dtype != SD_DTYPE_F32 && p->logits_dtype != SD_DTYPE_BF16) return SD_ERR_INVALID_ARG;
    if (!sizes_ok(p)) return SD_ERR_UNSUPPORTED;
    const int B = p->batch, k = p->num_draft, V = p->vocab;
    if (p->top_k) return SD_ERR_UNSUPPORTED;  // top-k path not built yet
    if (B == 0) {
        hipLaunchKernelGGL(empty_batch_kernel, dim3(1), dim3(64), 0, stream, out_counters, p->status,
                           p->dbg_flags);
        return hipGetLastError() == hipSuccess ? SD_OK : SD_ERR_HIP;
    }
    if (!target_logits || !temperature || !out_tokens || !out_num_accepted) return SD_ERR_INVALID_ARG;
    if (k > 0 && !draft_token_ids) return SD_ERR_INVALID_ARG;
    const Layout L = layout_of(p);
    if (!workspace || workspace_bytes < L.total || (reinterpret_cast<uintptr_t>(workspace) & 255u))
        return SD_ERR_WORKSPACE;

    const bool bf16 = p->logits_dtype == SD_DTYPE_BF16;
    const int per16 = bf16 ? 8 : 4;
    const bool aligned = (reinterpret_cast<uintptr_t>(target_logits) % 16 == 0) && (V % per16 == 0) &&
                         (!draft_probs || reinterpret_cast<uintptr_t>(draft_probs) % 16 == 0);
    const bool masked = bitmask != nullptr;
    char *ws = static_cast<char *>(workspace);

    RowStatsArgs ra;
    ra.logits = target_logits;
    ra.mask = reinterpret_cast<const uint32_t *>(bitmask);
    ra.temperature = temperature;
    ra.draft = draft_token_ids;
    ra.bstats = reinterpret_cast<float2 *>(ws + L.off_bstats);
    ra.sx = reinterpret_cast<float *>(ws + L.off_sx);
    ra.out_counters = out_counters;
    ra.status = p->status;
    ra.dbg_flags = p->dbg_flags;
    ra.ntasks = L.rows * L.nchunk;
    ra.nblk = L.rows * L.C;
    ra.k = k;
    ra.kp1 = k + 1;
    ra.V = V;
    ra.W = L.W;
    ra.C = L.C;
    ra.cpw = SDV_BLOCKS_PER_WAVE;
    ra.nchunk = L.nchunk;
    const int64_t waves_per_wg = kThreads / kWave;
    int64_t grid1 = aligned ? (ra.nblk + waves_per_wg - 1) / waves_per_wg
                            : (ra.ntasks + waves_per_wg - 1) / waves_per_wg;
    if (aligned) grid1 = std::min<int64_t>(grid1, SDV_ROW_STATS_GRID);
    if (grid1 > INT_MAX) return SD_ERR_UNSUPPORTED;

    FinalArgs fa;
    fa.logits = target_logits;
    fa.draft = draft_token_ids;
    fa.q = draft_probs;
    fa.mask = reinterpret_cast<const uint32_t *>(bitmask);
    fa.temperature = temperature;
    fa.seed = seed;
    fa.out_tokens = out_tokens;
    fa.out_num_accepted = out_num_accepted;
    fa.out_counters = out_counters;
    fa.dbg_lse = p->dbg_row_lse;
    fa.dbg_acc = p->dbg_accept_prob;
    fa.dbg_req_flags = p->dbg_request_flags;
    fa.dbg_flags = p->dbg_flags;
    fa.status = p->status;
    fa.bstats = ra.bstats;
    fa.sx = ra.sx;
    fa.B = B;
    fa.k = k;
    fa.V = V;
    fa.W = L.W;
    fa.C = L.C;
    const size_t dyn_lds = draft_probs ? size_t(L.C) * sizeof(double) : 0;

    RowStatsFn k1 = bf16 ? pick_row_stats<uint16_t>(masked, aligned) : pick_row_stats<float>(masked, aligned);
    FinalFn k2 = bf16 ? pick_final<uint16_t>(aligned) : pick_final<float>(aligned);

    if (p->row_stats_event_begin &&
        hipEventRecord(static_cast<hipEvent_t>(p->row_stats_event_begin), stream) != hipSuccess)
        return SD_ERR_HIP;
    hipLaunchKernelGGL(k1, dim3(static_cast<unsigned>(grid1)), dim3(kThreads), 0, stream, ra);
    if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    if (p->row_stats_event_end &&
        hipEventRecord(static_cast<hipEvent_t>(p->row_stats_event_end), stream) != hipSuccess)
        return SD_ERR_HIP;
    hipLaunchKernelGGL(k2, dim3(B), dim3(kFinalThreads), dyn_lds, stream, fa);
    if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    return SD_OK;
}
