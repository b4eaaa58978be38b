// MI355X (gfx950) speculative-decoding verifier: kernels and C ABI.
//
// One call runs these kernels in order on the caller's stream (those in
// brackets only when the call needs them):
//
//   [ragged_prep]  ragged calls with a pass before the sweep, or too large
//                  for its LDS: checks the draft offsets and maps every
//                  packed row to its request (otherwise the sweep's
//                  workgroups do both themselves).
//   [topk]         calls with top-p and no top-k, and top-k calls whose rows
//                  the single-pass selection cannot take (unaligned rows,
//                  very large V): each top-k / top-p row's threshold tau,
//                  from a pass over the row before the sweep (bf16 rows
//                  counted on their raw 16-bit codes).
//   row_stats      the sweep, the only full pass over the logits: waves claim
//                  2048-token blocks of all rows, stream them from HBM in
//                  16-byte loads, apply the grammar bitmask and temperature
//                  (pyshine "vLLM, part 2", "Verification": logits in fp32,
//                  temperature before normalising; "Grammar gates": one mask
//                  row per request and position), and write per block
//                    sampling rows: (Mc, Sc) with Mc = fp32(max_j l_j * c),
//                      Sc = sum_j 2^(l_j * c - Mc), c = log2(e) / T, and the
//                      block's level-1 Gumbel key;
//                    greedy rows:   (max_j l_j, lowest index of that max);
//                    sampling rows of a single-pass top-k / top-p call: the
//                      code of every 128-byte line's largest allowed logit
//                      instead;
//                  plus each draft row's record: l(x), the mask bit, q(x) and
//                  the draft block's mass without the draft.
//   [topk_lines]   single-pass top-k (and top-p after it): each row's tau
//                  from the line maxima and the few lines that can hold kept
//                  tokens, then the row's block statistics over the kept
//                  tokens and, with dense drafts, the list of the lines that
//                  hold a kept token (the only lines a residual draw from the
//                  row can weigh).
//   finalize       one 512-thread workgroup per request: folds the block
//                  statistics into each row's max and normaliser, forms p(x)
//                  and q(x), draws the accept uniforms from Philox, finds the
//                  first rejection (vllm-learning code walkthrough,
//                  RejectionSampler), then samples the emitted token from the
//                  residual max(p - q, 0), from p without the draft (one-hot
//                  drafts, infra-guide 5.2 section 4.3) or from p at the bonus
//                  position by two-level Gumbel-max: level 1 over block
//                  masses, level 2 over the chosen block's 2048 tokens.  A
//                  dense residual sums the listed lines after the single-pass
//                  selection (every line of a long row it did not list), and
//                  otherwise the rejected row of a short row here.  It
//                  writes the outputs and adds R, I, D, A (fanout, "Name the
//                  three counters") through a slot tally.
//   [dense_mass,   dense drafts over long rows, without the single-pass
//    dense_draw]   selection: the residual's block masses of every rejected
//                  row on a grid of (block, request) workgroups, then its
//                  draw.
//   [histogram]    requests per accepted length, when asked for.
#include <hip/hip_runtime.h>
#include <float.h>
#include <limits.h>
#include <math.h>
#include <stdint.h>

#include <algorithm>
#include <map>
#include <mutex>
#include <type_traits>
#include <utility>

#include "sd_verify.h"
#include "philox.h"
#include "wave.h"

#ifndef SDV_BLOCKS_PER_WAVE
#define SDV_BLOCKS_PER_WAVE 4   // element kernel: 2048-token blocks per wave task
#endif
#ifndef SDV_SWEEP_WAVES
#define SDV_SWEEP_WAVES 3072  // claimed sweep: waves in the grid when the occupancy query fails
#endif
#ifndef SDV_SWEEP_WAVES_PER_SIMD
#define SDV_SWEEP_WAVES_PER_SIMD 3  // claimed sweep: at most this many waves per SIMD
#endif
#ifndef SDV_LOGITS_CACHE_POLICY
#define SDV_LOGITS_CACHE_POLICY 2  // logits loads: non-temporal (read once, kept out of the caches)
#endif
#ifndef SDV_CACHED_LOGITS_BYTES
// Calls whose logits take at most this many bytes (a quarter of the 256 MB
// Infinity Cache) read them through the caches instead, so that the
// finalisation's second reads (the dense residual's rows, the sampled block)
// find them there.
#define SDV_CACHED_LOGITS_BYTES (64ll << 20)
#endif

namespace sdv {

constexpr int kBlock = SD_BLOCK_TOKENS;
constexpr int kThreads = 256;       // element path, dense residual grid: 4 waves per workgroup
#ifndef SDV_SWEEP_STATIC
#define SDV_SWEEP_STATIC 16  // claimed sweep without a mask: static blocks per wave before it claims
#endif
#ifndef SDV_MASKED_STATIC_PCT
#define SDV_MASKED_STATIC_PCT 75  // with a mask: percent of a wave's share taken statically
#endif
#ifndef SDV_SWEEP_THREADS
#define SDV_SWEEP_THREADS 768
#endif
// Claimed sweep: 12 waves per workgroup, one workgroup per CU.  The grid
// starts a third as many workgroups as with 4 waves each, and the
// dispatcher's ramp at the start of the kernel is that much shorter.
constexpr int kSweepThreads = SDV_SWEEP_THREADS;
constexpr int kSimdsPerCu = 4;
constexpr int kFinalThreads = 512;  // finalize: 8 waves per request
constexpr int kFinalWaves = kFinalThreads / 64;
// s_waitcnt operand (GFX9 layout: vmcnt in bits 3:0 and 15:14, expcnt in
// 6:4, lgkmcnt in 11:8) that waits for vmcnt = 0 only.
constexpr int kWaitVmcnt0 = 0x0F70;
constexpr int kTallyStride = 32;       // 64-bit words between tally words: one 256-byte line each
#ifndef SDV_DENSE_SPLIT_BLOCKS
#define SDV_DENSE_SPLIT_BLOCKS 32
#endif
constexpr int kDenseSplitBlocks = SDV_DENSE_SPLIT_BLOCKS;  // dense q rows of at least this many blocks use the grid
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
    // a 16-byte group whose eight tokens all unpack to -inf
    __device__ static uint4 neg_inf_group() { return make_uint4(0xff80ff80u, 0xff80ff80u, 0xff80ff80u, 0xff80ff80u); }
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
    __device__ static uint4 neg_inf_group() { return make_uint4(0xff800000u, 0xff800000u, 0xff800000u, 0xff800000u); }
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

// A wave-uniform read of memory that nothing writes while the kernel runs
// (an earlier kernel of the call may have written it), through the constant
// address space so that it becomes a scalar load (its own counter, no wait on
// outstanding vector loads).
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

// Wave-uniform words read with vector (buffer) loads at a uniform offset:
// they join the in-order vector memory counter of the loads issued next to
// them, so that one wait covers them all, where the wait for a scalar load
// also covers every scalar load issued after it.  The caller makes them
// uniform (`uniform_word`) where it first needs them.
__device__ __forceinline__ uint32_t uniform_word(uint32_t w) {
    return static_cast<uint32_t>(__builtin_amdgcn_readfirstlane(static_cast<int>(w)));
}

// ------------------------------------------------------------ request geometry

// Where request b's rows, drafts and output slots sit.  Uniform calls: k
// drafts per request, rows b (k + 1) ..; ragged calls (a cumulative draft
// offset table off[B + 1]): k_b = off[b+1] - off[b] drafts, rows off[b] + b ..
// and drafts off[b] ..  (infra-guide 5.2: drafters that propose a variable
// number of tokens).  `ok` is false for every request of a ragged call whose
// offsets the prep kernel found inconsistent; nothing is then read through
// them.
struct ReqGeom {
    int k;          // drafts of the request
    int64_t row0;   // its first row (and first output slot)
    int64_t draft0; // its first draft
    bool ok;
};

__device__ __forceinline__ ReqGeom req_geom(const int32_t *off, const uint32_t *off_ok, int b,
                                            int k_uniform) {
    ReqGeom g;
    if (off == nullptr) {
        g.k = k_uniform;
        g.row0 = int64_t(b) * (k_uniform + 1);
        g.draft0 = int64_t(b) * k_uniform;
        g.ok = true;
        return g;
    }
    g.ok = uniform_load(off_ok) != 0u;
    const int o0 = uniform_load(off + b), o1 = uniform_load(off + b + 1);
    g.k = g.ok ? o1 - o0 : 0;
    g.row0 = g.ok ? int64_t(o0) + b : 0;
    g.draft0 = g.ok ? o0 : 0;
    return g;
}

// The request and position of a row (ragged calls: through the row table the
// prep kernel wrote; only read when the offsets are consistent).
__device__ __forceinline__ void row_owner(const int32_t *off, const int32_t *row_req, int row,
                                          int kp1_uniform, int &b, int &i, int &k, int64_t &draft0) {
    if (off == nullptr) {
        b = row / kp1_uniform;
        i = row - b * kp1_uniform;
        k = kp1_uniform - 1;
        draft0 = int64_t(b) * k;
        return;
    }
    b = uniform_load(row_req + row);
    const int o0 = uniform_load(off + b);
    k = uniform_load(off + b + 1) - o0;
    i = row - o0 - b;
    draft0 = o0;
}

// ------------------------------------------------------------ row statistics

// Statistics of one 2048-token block of a row.  Sampling rows: m = Mc =
// fp32(max l * c), s = Sc = sum 2^(l c - Mc), key = ln Sc + Mc ln 2 + G_c, the
// block's level-1 Gumbel key up to a per-row constant.  Greedy rows: m = the
// largest logit, s = the lowest index holding it (int bits), key unused.
struct BlockStat {
    float m, s;
    double key;
};

// What the sweep learns about the draft of row i < k, in the draft's block.
struct DraftRec {
    float sx;        // Sc of the draft's block without the draft
    float lx;        // the draft's logit (-inf when masked)
    float qx;        // the draft probability q_i(x), 1 for one-hot drafts
    uint32_t allowed;  // the draft's mask bit
    double keyx;     // level-1 key of the draft's block without the draft
    double pad;
};

// Division of 0 <= n < 2^31 by a fixed 1 <= d < 2^31 as a multiply and a
// shift (Granlund and Montgomery, "Division by invariant integers using
// multiplication", the round-up method): with l = ceil(log2 d) and
// m = ceil(2^(31 + l) / d) <= 2^31 + ... < 2^32, n / d = (n m) >> (31 + l)
// for every such n.  Wave-uniform operands keep it on the scalar unit, and
// it has no branch.
struct DivMagic {
    uint32_t m;
    int shift;  // 31 + l
};

inline DivMagic div_magic(int d) {
    int l = 0;
    while ((int64_t(1) << l) < d) ++l;
    DivMagic r;
    r.shift = 31 + l;
    r.m = static_cast<uint32_t>(((uint64_t(1) << r.shift) + uint64_t(d) - 1) / uint64_t(d));
    return r;
}

__device__ __forceinline__ uint32_t div_fixed(uint32_t n, const DivMagic &f) {
    return static_cast<uint32_t>((static_cast<uint64_t>(n) * f.m) >> f.shift);
}

struct RowStatsArgs {
    const void *logits;
    const uint32_t *mask;     // nullptr = no bitmask
    const float *temperature;
    const int32_t *draft;     // [B, k]; nullptr when k = 0
    const float *q;           // [B, k, V] or nullptr
    uint64_t seed;
    const float *tau;         // [rows] top-k thresholds, or nullptr (no top-k)
    const int32_t *top_k;     // [B]: with linemax, the requests whose rows record line maxima
    const float *top_p;       // [B] or nullptr: with linemax, requests with top-p record them too
    void *linemax;            // [rows, C * lines per block] line maxima of top-k rows, or nullptr
    BlockStat *bstats;        // [rows, C]
    DraftRec *drec;           // [rows]
    unsigned long long *tally;  // counter tally, zeroed here, accumulated by finalize
    int ntally;                 // words of the tally
    uint64_t *out_counters;     // the call's R, I, D, A: zeroed here, added to by finalize
    uint32_t *status;         // zeroed here when given
    uint32_t *dbg_flags;      // zeroed here when given
    const int32_t *off;       // ragged: [B + 1] draft offsets, or nullptr
    const int32_t *row_req;   // ragged: [rows] request of each row
    const uint32_t *off_ok;   // ragged: 1 when the offsets are consistent
    // ragged calls the vector sweep maps itself (no prep launch): the check
    // and the row table it writes for the kernels after it
    int fold, B;
    int64_t total;            // the call's total drafts
    int32_t *row_req_out;
    uint32_t *off_ok_out;
    int64_t ntasks;           // rows * nchunk (chunked element kernel)
    int64_t nblk;             // rows * C (vector kernel sweep)
    int k, kp1, V, W, C, cpw, nchunk;
    uint32_t *sweep;          // claim counters of the vector sweep (zero on entry)
    int parts_log2;           // the sweep's partitions: 2^parts_log2 <= kSweepParts
    int sweep_static;         // claimed sweep with a mask: static blocks per wave (even, >= 2)
    DivMagic divC, divK;      // division by C and by kp1
};

// Per-block statistics of a sampling row from one lane's values v (masked
// tokens and tokens past V hold -inf): (Mc, Sc) with Mc = fp32(max l * c) and
// Sc = sum 2^(l c - Mc).
template <int NV>
__device__ __forceinline__ float2 softmax_block(const float *v, float c) {
    float m = v[0];
#pragma unroll
    for (int e = 1; e < NV; ++e) m = fmaxf(m, v[e]);
    m = wave_max_coded(m);  // a NaN logit makes the sum NaN either way
    if (m == -INFINITY) {
        // every value but a NaN is -inf here, so a NaN (of either sign) is a
        // nonzero mantissa among the values: the statistics then carry it
        uint32_t bits = 0u;
#pragma unroll
        for (int e = 0; e < NV; ++e) bits |= __float_as_uint(v[e]);
        return make_float2(-INFINITY, wave_any((bits & 0x7fffffu) != 0u) ? NAN : 0.0f);
    }
    const float mc = m * c;
    // four running sums of 8 terms each, combined pairwise: with the wave's
    // tree the fp32 sum of these positive terms is 15 additions deep, within
    // 15 units of 2^-24 of exact (relative)
    static_assert(NV == 32, "32 values per lane");
    float r[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        r[q] = __builtin_amdgcn_exp2f(fmaf(v[8 * q], c, -mc));
#pragma unroll
        for (int e = 1; e < 8; ++e) r[q] += __builtin_amdgcn_exp2f(fmaf(v[8 * q + e], c, -mc));
    }
    return make_float2(mc, wave_sum((r[0] + r[1]) + (r[2] + r[3])));
}

// The same sum without the token at offset xrel of the block (the one-hot
// residual mass of the draft's block), against the same Mc.
template <int G, int P>
__device__ __forceinline__ float excluded_sum(const float *v, float c, float mc, int xrel, int lane) {
    float s = 0.0f;
    if (mc > -INFINITY) {
        static_assert(G * P == 32, "32 values per lane");
        float r[4] = {0.0f, 0.0f, 0.0f, 0.0f};  // as in softmax_block
#pragma unroll
        for (int g = 0; g < G; ++g)
#pragma unroll
            for (int e = 0; e < P; ++e)
                if ((g * kWave + lane) * P + e != xrel)
                    r[(g * P + e) / 8] += __builtin_amdgcn_exp2f(fmaf(v[g * P + e], c, -mc));
        s = (r[0] + r[1]) + (r[2] + r[3]);
    }
    return wave_sum(s);
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

// Tokens below the row's top-k threshold leave the support like masked ones
// (NaN stays NaN, so that a bad logit is still reported).
template <int NV>
__device__ __forceinline__ void apply_tau(float *v, float tau) {
#pragma unroll
    for (int e = 0; e < NV; ++e)
        if (v[e] < tau) v[e] = -INFINITY;
}

// The level-1 Gumbel variate (fp64) of block blk of row i of request b.
__device__ __forceinline__ double block_gumbel(PhiloxKey key, int b, int i, int blk) {
    const uint4 w = philox4x32_10(make_uint4(uint32_t(blk) >> 2, uint32_t(i), uint32_t(b), 1u),
                                  key.k0, key.k1);
    const int q = blk & 3;
    return gumbel_wide(q == 0 ? w.x : (q == 1 ? w.y : (q == 2 ? w.z : w.w)));
}

// ln x of a positive fp32 value as (e + log2 m) ln 2 for x = m 2^e: the
// exponent exact and the hardware log2 of the mantissa (|log2 m| <= 1), the
// sum in fp64, so that the result is within about 5e-8 of ln x whatever its
// size.  -inf for x <= 0.
__device__ __forceinline__ double ln_f32(float x) {
    if (!(x > 0.0f)) return -INFINITY;
    return (static_cast<double>(__builtin_amdgcn_frexp_expf(x)) +
            static_cast<double>(__builtin_amdgcn_logf(__builtin_amdgcn_frexp_mantf(x)))) * kLn2;
}

// ln(mass) + Mc ln 2 + G in fp64: a level-1 key up to the row's constant
// (-inf when the mass is zero).
__device__ __forceinline__ double key_of_mass(float mass, float mc, double g) {
    if (!(mass > 0.0f) || !(mc > -INFINITY)) return -INFINITY;
    return ln_f32(mass) + static_cast<double>(mc) * kLn2 + g;
}

__device__ __forceinline__ void zero_call_outputs(const RowStatsArgs &a) {
    if (blockIdx.x != 0) return;
    for (int w = threadIdx.x; w < a.ntally; w += blockDim.x) a.tally[w * kTallyStride] = 0ull;
    if (threadIdx.x < 4) a.out_counters[threadIdx.x] = 0ull;
    if (threadIdx.x == 0 && a.status) *a.status = 0u;
    if (threadIdx.x < 3 && a.dbg_flags) a.dbg_flags[threadIdx.x] = 0u;
}

// Which rows a chunked wave works on, and their parameters (wave-uniform).
struct RowTask {
    int row, b, i, c0, c1;
    int64_t dpos;  // the row's draft index (draft rows)
    bool greedy, skip;
    float c, tau;
    int x, xblk, xrel;  // the draft, its block and offset in it (-1: none)
};

__device__ __forceinline__ RowTask row_task(const RowStatsArgs &a, int64_t task) {
    RowTask t;
    t.row = static_cast<int>(task / a.nchunk);
    const int chunk = static_cast<int>(task - int64_t(t.row) * a.nchunk);
    t.c0 = chunk * a.cpw;
    t.c1 = min(a.C, t.c0 + a.cpw);
    int kb;
    int64_t d0;
    row_owner(a.off, a.row_req, t.row, a.kp1, t.b, t.i, kb, d0);
    t.dpos = d0 + t.i;
    const float T = uniform_load(a.temperature + t.b);
    t.greedy = (T == 0.0f);
    t.skip = !t.greedy && !(T > 0.0f && T <= FLT_MAX);  // reported by finalize
    t.c = t.greedy ? 0.0f : scale_of(T);
    t.tau = a.tau ? uniform_load(a.tau + t.row) : -INFINITY;
    t.x = t.xblk = t.xrel = -1;
    if (t.i < kb) {
        const int x = uniform_load(a.draft + t.dpos);
        if (x >= 0 && x < a.V) {
            t.x = x;
            t.xblk = x / kBlock;
            t.xrel = x - t.xblk * kBlock;
        }
    }
    return t;
}

// The lane holding the draft writes its logit, its mask bit and q(x) into
// the row's draft record.  v: the block's masked values; bits(g): the lane's
// mask bits of group g.
template <int G, int P, bool MASKED>
__device__ __forceinline__ void record_draft(const RowStatsArgs &a, int row, int64_t dpos, int x,
                                             int xrel, const float *v, const uint32_t *m, int lane,
                                             float sx) {
    const int xg = xrel / (kWave * P), xl = (xrel / P) & (kWave - 1), xe = xrel % P;
    if (lane != xl) return;
    float lx = -INFINITY;
    uint32_t bits = 0xffu;
#pragma unroll
    for (int g = 0; g < G; ++g)
        if (g == xg) {
#pragma unroll
            for (int e = 0; e < P; ++e)
                if (e == xe) lx = v[g * P + e];
            if (MASKED) bits = (P == 8) ? m[g] : (m[g] >> ((lane & 1) * 4));
        }
    DraftRec &r = a.drec[row];
    r.sx = sx;
    r.lx = lx;
    r.allowed = (bits >> xe) & 1u;
    r.qx = a.q ? uniform_load(a.q + dpos * a.V + x) : 1.0f;
}

// The keep masks of a bf16 group for each of the 256 values of its mask
// byte: word i keeps its low half when bit 2i is set and its high half when
// bit 2i + 1 is, so a group masks in four bit-field inserts (forbidden tokens
// become the bf16 pattern of -inf) instead of a test and a select per token.
// Filled in LDS by every workgroup of a masked bf16 sweep.
__device__ __forceinline__ void fill_keep_table(uint4 *keep) {
    for (int t = threadIdx.x; t < 256 * 4; t += blockDim.x) {
        const uint32_t byte = uint32_t(t) >> 2, i = uint32_t(t) & 3u;
        const uint32_t lo = (byte >> (2 * i)) & 1u, hi = (byte >> (2 * i + 1)) & 1u;
        reinterpret_cast<uint32_t *>(keep)[t] = (lo ? 0x0000ffffu : 0u) | (hi ? 0xffff0000u : 0u);
    }
}

__device__ __forceinline__ uint32_t keep_or_neg_inf(uint32_t w, uint32_t k) {
    uint32_t r = (w & k) | (0xff80ff80u & ~k);
    asm("" : "+v"(r));  // one insert per word; the unpack then shifts and masks the result
    return r;
}

// Raw 16-byte groups and mask bytes of one block wholly inside the row: lane
// l reads groups l, l + 64, ... (consecutive lanes, consecutive 16 bytes).
// keep: the keep-mask table (masked bf16 rows).
template <typename ET, bool MASKED>
__device__ __forceinline__ void unpack_full_block(const uint4 *r, const uint32_t *m, int lane,
                                                  float *v, const uint4 *keep = nullptr) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    if constexpr (MASKED && P == 8) {
        uint4 k[G];  // all table reads in flight before the first is used
#pragma unroll
        for (int g = 0; g < G; ++g) k[g] = keep[m[g]];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const uint4 w = make_uint4(keep_or_neg_inf(r[g].x, k[g].x), keep_or_neg_inf(r[g].y, k[g].y),
                                       keep_or_neg_inf(r[g].z, k[g].z), keep_or_neg_inf(r[g].w, k[g].w));
            Logit<ET>::unpack(w, v + g * P);
        }
        return;
    }
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

// One block's share of the sweep: where it lives and its row's parameters.
struct SweepBlock {
    int64_t gb;   // row * C + block
    int row, blk, b, i;
    bool full, greedy, skip;
    bool lines;   // the block's line maxima are recorded (single-pass top-k)
    float c, tau;
    int x, xrel;  // the draft and its offset in this block (-1: elsewhere)
    int64_t dpos; // the row's draft index (draft rows)
};

// Where a block of the sweep lies: its (row, block) and, for calls with k
// drafts per request, the row's request and position.
struct SweepCursor {
    int64_t gb;
    int row, blk, b, i;
};

// A wave-uniform 64-bit value moved to scalar registers.
__device__ __forceinline__ int64_t uniform_i64(int64_t v) {
    const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint64_t>(v)));
    const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<int>(static_cast<uint64_t>(v) >> 32));
    return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

__device__ __forceinline__ SweepCursor cursor_at(const RowStatsArgs &a, int64_t gb) {
    // uniform by construction; said explicitly because the claim's lane-0
    // branch would otherwise let the compiler treat the index as per-lane
    gb = uniform_i64(gb);
    SweepCursor c;
    c.gb = gb;
    const uint32_t g = static_cast<uint32_t>(gb);  // < 2^31 (checked by the host)
    const uint32_t row = div_fixed(g, a.divC);
    c.row = static_cast<int>(row);
    c.blk = static_cast<int>(g - row * static_cast<uint32_t>(a.C));
    const uint32_t b = div_fixed(row, a.divK);  // uniform layout (ragged calls look their rows up)
    c.b = static_cast<int>(b);
    c.i = static_cast<int>(row - b * static_cast<uint32_t>(a.kp1));
    return c;
}

// The claimed sweep hands blocks out dynamically.  Per-wave throughput varies by
// tens of percent (which HBM channels a wave's blocks hit, which XCD it runs
// on), and workgroups that start late would otherwise carry a full share to
// the end of the kernel, so a static split ends with a long tail of few busy
// waves.  Instead the blocks form interleaved partitions (partition p:
// blocks p, p + P, p + 2P, ...), each with a claim counter that its home
// waves increment; P is kSweepParts, or a smaller power of two when the grid
// has fewer wave slots per XCD, so that every partition has home waves.  The
// grid is the resident capacity.  A wave takes its first SDV_SWEEP_STATIC
// blocks statically and claims the rest one at a time: a claim's result
// shares the in-order vector memory counter with the loads issued after it,
// so every claim can delay a block, and claims are kept for the part of the
// sweep where the imbalance builds up.  A claim's round trip under full HBM
// load is longer than one block's time, so two claims are kept in flight.  Home partitions mix workgroups of all eight XCDs (workgroups go to
// XCDs round-robin), so the XCDs' speeds average out within a partition.
// Each counter serves about 1/64 of the claims; the counters still contend
// (32 partitions measured 2.9 us slower per call, 16 partitions 16 us), and
// 128 measured 0.6 us slower.
constexpr int kSweepParts = 64;
constexpr int kSweepCtrStride = 64;  // 32-bit words between counters: one 256-byte line each

struct SweepPlan {  // 32-bit: block indices are below 2^31, and scalar compares are 32-bit
    int lg;     // log2 of the number of partitions
    int p;      // home partition
    int lim;    // blocks in the partition
    int k0, k1; // the wave's last two static blocks (partition indices)
    int kfirst, np;  // its first static block and the stride between its static blocks
    int kdyn;   // the partition index the counter's first claim stands for
    uint32_t *ctr;
};

// Needs gridDim.x to be a multiple of 8 and 2^parts_log2 <= 4 gridDim.x / 8.
__device__ __forceinline__ SweepPlan plan_of(const RowStatsArgs &a, int S) {
    constexpr int WPG = kSweepThreads / kWave;
    const int lg = a.parts_log2, P = 1 << lg;
    const int x = blockIdx.x & 7;
    const int u = static_cast<int>(blockIdx.x >> 3) * WPG + wave_id();
    const int U = static_cast<int>(gridDim.x >> 3) * WPG;
    SweepPlan pl;
    pl.lg = lg;
    pl.p = u & (P - 1);
    const int n_p = 8 * ((U - pl.p + P - 1) >> lg);  // waves at home in p
    pl.lim = a.nblk > pl.p ? static_cast<int>((a.nblk - pl.p + P - 1) >> lg) : 0;
    pl.kfirst = x + 8 * (u >> lg);
    pl.np = n_p;
    pl.k0 = pl.kfirst + (S - 2) * n_p;
    pl.k1 = pl.k0 + n_p;
    pl.kdyn = S * n_p;
    pl.ctr = a.sweep + pl.p * kSweepCtrStride;
    return pl;
}

__device__ __forceinline__ int64_t block_of(const SweepPlan &pl, int k) {
    return pl.p + (static_cast<int64_t>(k) << pl.lg);
}

// Waits for the last load of a block that is not reduced (skipped, or the
// dead look-ahead; loads complete in order), so that on every path the
// block's registers are settled when the loop comes round again and reusing
// them as temporaries waits for nothing.
__device__ __forceinline__ void settle(const uint4 &last) { asm volatile("" ::"v"(last.w)); }

// Issues a claim (lane 0's atomic); its result is read by `claimed`, as late
// as possible.
__device__ __forceinline__ uint32_t claim(const SweepPlan &pl, int lane) {
    uint32_t r = 0u;
    if (lane == 0) r = atomicAdd(pl.ctr, 1u);
    return r;
}

// The claimed partition index, saturated at lim (no more blocks).  kdyn may
// exceed lim (a partition with fewer blocks than two per home wave), and the
// counter's value is unbounded, so the sum is formed only below lim.
__device__ __forceinline__ int claimed(const SweepPlan &pl, uint32_t r) {
    const uint32_t c = static_cast<uint32_t>(__builtin_amdgcn_readlane(static_cast<int>(r), 0));
    if (pl.kdyn >= pl.lim) return pl.lim;
    return c < static_cast<uint32_t>(pl.lim - pl.kdyn) ? pl.kdyn + static_cast<int>(c) : pl.lim;
}

// Ragged calls whose offsets and rows fit in LDS: the vector sweep's
// workgroups check the draft offsets themselves, as the prep kernel does, and
// map rows to requests in LDS.
constexpr int kFoldRows = 8192;   // rows (total drafts + B) at most
constexpr int kFoldReqs = 2048;   // requests at most
struct FoldMap {
    int32_t off[kFoldReqs + 1];
    uint16_t req[kFoldRows];
};

__device__ __forceinline__ FoldMap &fold_map() {
    __shared__ FoldMap m;
    return m;
}

// Every workgroup: the offsets into LDS, the prep kernel's check, and the
// request of every row; workgroup 0 also writes the check and the row table
// for the kernels after the sweep.  Returns false in every thread when the
// offsets fail (the finalize kernel reports the call).
__device__ bool fold_ragged(const RowStatsArgs &a) {
    FoldMap &fm = fold_map();
    const int B = a.B;
    for (int j = threadIdx.x; j <= B; j += blockDim.x) fm.off[j] = a.off[j];
    __syncthreads();
    bool bad = threadIdx.x == 0 && (fm.off[0] != 0 || int64_t(fm.off[B]) != a.total);
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int64_t d = int64_t(fm.off[b + 1]) - int64_t(fm.off[b]);
        bad |= d < 0 || d > a.k;
    }
    const bool any_bad = __syncthreads_or(bad) != 0;
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.off_ok_out = any_bad ? 0u : 1u;
    if (any_bad) return false;
    // the offsets now partition rows [0, total + B): request b owns k_b + 1
    // rows from off[b] + b
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int r0 = fm.off[b] + b, kb = fm.off[b + 1] - fm.off[b];
        for (int i = 0; i <= kb; ++i) {
            fm.req[r0 + i] = static_cast<uint16_t>(b);
            if (blockIdx.x == 0) a.row_req_out[r0 + i] = b;
        }
    }
    __syncthreads();
    return true;
}

__device__ __forceinline__ SweepBlock sweep_block(const RowStatsArgs &a, const SweepCursor &c) {
    SweepBlock s;
    s.gb = c.gb;
    s.row = c.row;
    s.blk = c.blk;
    s.full = int64_t(s.blk + 1) * kBlock <= a.V;
    int kb;
    int64_t d0;
    if (a.fold) {
        const FoldMap &fm = fold_map();
        s.b = __builtin_amdgcn_readfirstlane(int(fm.req[s.row]));
        const int o0 = __builtin_amdgcn_readfirstlane(fm.off[s.b]);
        kb = __builtin_amdgcn_readfirstlane(fm.off[s.b + 1]) - o0;
        s.i = s.row - o0 - s.b;
        d0 = o0;
    } else if (a.off) {
        row_owner(a.off, a.row_req, s.row, a.kp1, s.b, s.i, kb, d0);
    } else {
        s.b = c.b;
        s.i = c.i;
        kb = a.kp1 - 1;
        d0 = int64_t(c.b) * kb;
    }
    s.dpos = d0 + s.i;
    const float T = uniform_load(a.temperature + s.b);
    s.greedy = (T == 0.0f);
    s.skip = !s.greedy && !(T > 0.0f && T <= FLT_MAX);  // reported by finalize
    s.c = s.greedy ? 0.0f : scale_of(T);
    s.tau = a.tau ? uniform_load(a.tau + s.row) : -INFINITY;
    if (a.linemax != nullptr && !s.greedy) {
        const float pp = a.top_p ? uniform_load(a.top_p + s.b) : 0.0f;
        s.lines = uniform_load(a.top_k + s.b) > 0 || (pp > 0.0f && pp < 1.0f);
    } else {
        s.lines = false;
    }
    s.x = s.xrel = -1;
    if (s.i < kb) {
        const int x = uniform_load(a.draft + s.dpos);
        if (x >= 0 && x < a.V && x / kBlock == s.blk) {
            s.x = x;
            s.xrel = x - s.blk * kBlock;
        }
    }
    return s;
}

// Byte offset beyond every row-based buffer range (rows are at most 16 MiB).
constexpr int kPastAnyBuffer = 0x40000000;

// Issue the loads of block blk of a row.  Without a mask the buffer resource
// starts at the block and ends with its row: every block takes the same
// instructions with the same per-lane offsets, and a dead issue (the sweep's
// look-ahead past its last block) gets an empty range.  With a mask the
// resources span the row and its mask row and the offsets carry the block (a
// dead issue points past the end); with masks that form measured faster (on
// the grid-stride sweep masked calls took before).  Either way the groups of a partial block that lie past the row
// read zeros (they are replaced by -inf when the block is reduced), and a
// dead issue's loads return zeros and touch no memory.
template <typename ET, bool MASKED, int POL = SDV_LOGITS_CACHE_POLICY>
__device__ __forceinline__ void issue_block(const RowStatsArgs &a, int row, int blk, int lane, uint4 *r,
                                            uint32_t *m, bool live = true) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    if constexpr (!MASKED) {
        const uint32_t boff = uint32_t(blk) * kBlock * uint32_t(sizeof(ET));
        const __amdgpu_buffer_rsrc_t rs =
            buffer_of(reinterpret_cast<const char *>(a.logits) + (int64_t(row) * a.V) * int64_t(sizeof(ET)) + boff,
                      live ? uint32_t(a.V) * uint32_t(sizeof(ET)) - boff : 0u);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, lane * 16 + g * kWave * 16, 0,
                                                                  POL);
            r[g] = make_uint4(w.x, w.y, w.z, w.w);
        }
    } else {
        const __amdgpu_buffer_rsrc_t rs = buffer_of(
            reinterpret_cast<const ET *>(a.logits) + int64_t(row) * a.V, uint32_t(a.V) * sizeof(ET));
        const int base = live ? blk * kBlock * int(sizeof(ET)) + lane * 16 : kPastAnyBuffer;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, base + g * kWave * 16, 0, POL);
            r[g] = make_uint4(w.x, w.y, w.z, w.w);
        }
        // the block's 256 mask bytes, one word per lane (spread to the lanes
        // that use them when the block is reduced)
        const __amdgpu_buffer_rsrc_t rm = buffer_of(a.mask + int64_t(row) * a.W, uint32_t(a.W) * 4u);
        m[0] = __builtin_amdgcn_raw_buffer_load_b32(rm, live ? blk * (kBlock / 8) + lane * 4 : kPastAnyBuffer, 0, 0);
    }
}

// The mask byte of each group of a lane, from the block's mask words held one
// per lane (lane l holds bytes 4l .. 4l + 3): group g's byte of the lane is
// byte (g * 64 + lane) * P / 8 of the block.
template <int G, int P>
__device__ __forceinline__ void spread_mask(uint32_t word, int lane, uint32_t *mm) {
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int byte = (g * kWave + lane) * P / 8;
        mm[g] = (static_cast<uint32_t>(__shfl(static_cast<int>(word), byte >> 2)) >> (8 * (byte & 3))) & 0xffu;
    }
}

// Per-lane record of one swept block, kept until the wave writes a batch of
// up to 64 blocks: each lane then draws its block's level-1 Gumbel variate,
// so one vector pass serves 64 blocks.
struct Stash {
    int64_t gb;
    int row, b, i, blk;
    float m, s, sx;
    int kind;  // 0 none, 1 greedy, 2 sampling, 3 sampling with the draft in it
};

__device__ __forceinline__ void flush_stash(const RowStatsArgs &a, const Stash &st, PhiloxKey key,
                                            int lane, int count) {
    if (lane >= count || st.kind == 0) return;
    BlockStat out;
    out.m = st.m;
    out.s = st.s;
    out.key = -INFINITY;
    if (st.kind >= 2 && st.m > -INFINITY) {
        const double g = block_gumbel(key, st.b, st.i, st.blk);
        out.key = key_of_mass(st.s, st.m, g);
        if (st.kind == 3) a.drec[st.row].keyx = key_of_mass(st.sx, st.m, g);
    } else if (st.kind == 3) {
        a.drec[st.row].keyx = -INFINITY;
    }
    a.bstats[st.gb] = out;
}

// Sampling rows of a top-k call: the line maxima of the block, for the
// single-pass top-k, which then computes the row's block statistics over the
// kept tokens; the sweep only marks a block holding an allowed NaN or +inf
// (statistics NaN, which report the row) and otherwise leaves (-inf, 0), the
// statistics of a row without an allowed finite value.  A line is a 128-byte
// line of the block (8 lanes of one group of loads); its code is the
// order-preserving code of its largest allowed finite value, 0 for none.
// 16-bit codes for bf16 rows (a bf16 value's code has an all-zero or all-one
// low half, so its top half orders the same), 32-bit codes for fp32 rows.
// Entry q * G + g of the block's codes is group g's line of lanes
// 8q .. 8q + 7, so that lane 8q + 7 stores its G codes with one write.
template <typename ET>
__device__ __forceinline__ float2 lines_block(const RowStatsArgs &a, int row, int blk, const float *v, int lane) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    constexpr int LPB = G * 8;  // lines per block
    bool bad = false;
    uint32_t code[G];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        float m = v[g * P];
        bad |= !(v[g * P] <= FLT_MAX);
#pragma unroll
        for (int e = 1; e < P; ++e) {
            m = fmaxf(m, v[g * P + e]);
            bad |= !(v[g * P + e] <= FLT_MAX);
        }
        m = fmaxf(m, dpp_f<0x111, 0xf>(-INFINITY, m));  // row_shr:1
        m = fmaxf(m, dpp_f<0x112, 0xf>(-INFINITY, m));  // row_shr:2
        m = fmaxf(m, dpp_f<0x114, 0xf>(-INFINITY, m));  // row_shr:4: lane 8q + 7 holds line q
        code[g] = (m > -INFINITY && m <= FLT_MAX) ? ordered_code(m) : 0u;
    }
    if ((lane & 7) == 7) {
        const int64_t idx = (int64_t(row) * a.C + blk) * LPB + (lane >> 3) * G;
        if constexpr (sizeof(ET) == 2) {
            *reinterpret_cast<uint2 *>(reinterpret_cast<uint16_t *>(a.linemax) + idx) =
                make_uint2((code[0] >> 16) | (code[1] & 0xffff0000u), (code[2] >> 16) | (code[3] & 0xffff0000u));
        } else {
            uint4 *dst = reinterpret_cast<uint4 *>(reinterpret_cast<uint32_t *>(a.linemax) + idx);
            dst[0] = make_uint4(code[0], code[1], code[2], code[3]);
            dst[1] = make_uint4(code[4], code[5], code[6], code[7]);
        }
    }
    return wave_any(bad) ? make_float2(NAN, NAN) : make_float2(-INFINITY, 0.0f);
}

// TOPK: 0 no top-k, 1 cut at the row's threshold tau (found before the
// sweep), 2 record line maxima of top-k rows (tau is found after it).
template <typename ET, bool MASKED, int TOPK>
__device__ __forceinline__ void reduce_block(const RowStatsArgs &a, const SweepBlock &s, int lane,
                                             const uint4 *r, const uint32_t *m, Stash &st, int slot,
                                             const uint4 *keep) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    // Without a mask every block is unpacked the same way and a partial one is
    // then cut at V in place (V is a multiple of the group width here): one
    // set of registers for both, where two unpacking paths end in copies.
    // With a mask the two paths measured faster.
    float v[G * P];
    uint32_t mm[G];
    if constexpr (MASKED) spread_mask<G, P>(m[0], lane, mm);
    if constexpr (!MASKED) {
        uint4 w[G];
#pragma unroll
        for (int g = 0; g < G; ++g) w[g] = r[g];
        if (!s.full) {
#pragma unroll
            for (int g = 0; g < G; ++g)
                if (s.blk * kBlock + (g * kWave + lane) * P >= a.V) w[g] = Logit<ET>::neg_inf_group();
        }
        unpack_full_block<ET, MASKED>(w, mm, lane, v);
    } else if (s.full) {
        unpack_full_block<ET, MASKED>(r, mm, lane, v, keep);
    } else {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t tok = int64_t(s.blk) * kBlock + (g * kWave + lane) * P;
            Logit<ET>::unpack(r[g], v + g * P);
            uint32_t bits = tok < a.V ? 0xffu : 0u;
            bits &= (P == 8) ? mm[g] : (mm[g] >> (uint32_t(tok) & 4u));
#pragma unroll
            for (int e = 0; e < P; ++e)
                if (!((bits >> e) & 1u)) v[g * P + e] = -INFINITY;
        }
    }
    if (TOPK == 1) apply_tau<G * P>(v, s.tau);
    float2 res;
    float sx = 0.0f;
    if (s.greedy) {
        res = greedy_block<G, P>(v, int64_t(s.blk) * kBlock, lane);
    } else if (TOPK == 2 && s.lines) {
        res = lines_block<ET>(a, s.row, s.blk, v, lane);
    } else {
        res = softmax_block<G * P>(v, s.c);
        if (s.xrel >= 0) sx = excluded_sum<G, P>(v, s.c, res.x, s.xrel, lane);
    }
    if (s.xrel >= 0) record_draft<G, P, MASKED>(a, s.row, s.dpos, s.x, s.xrel, v, mm, lane, sx);
    if (lane == slot) {
        st.gb = s.gb;
        st.row = s.row;
        st.b = s.b;
        st.i = s.i;
        st.blk = s.blk;
        st.m = res.x;
        st.s = res.y;
        st.sx = sx;
        st.kind = s.greedy ? 1 : (s.xrel >= 0 ? 3 : 2);
    }
}

// Rows 16-byte aligned with V a multiple of the group width.  Each wave takes
// a static prefix of its blocks (16 without a mask; three quarters of its
// share with one, where blocks take longer and claims would delay more of
// them) and claims the rest.  Each wave keeps the loads of its next block in
// flight while it reduces the current one.
template <typename ET, bool MASKED, int TOPK, int POL>
__device__ __forceinline__ void sweep_claimed(const RowStatsArgs &a, int lane, const uint4 *keep) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    // static blocks per wave: a build-time constant without a mask
    const int S = MASKED ? a.sweep_static : SDV_SWEEP_STATIC;
    const SweepPlan pl = plan_of(a, S);
    if (pl.kfirst >= pl.lim) return;
    const PhiloxKey key = key_of(a.seed);
    Stash st;
    st.kind = 0;
    int count = 0;
    uint4 ra[G], rb[G];
    uint32_t ma[G], mb[G];
    // The static blocks before the last two, two at a time, without claims.
    if (S > 2) {
        int ks = pl.kfirst;
        const SweepCursor s0 = cursor_at(a, block_of(pl, ks));
        issue_block<ET, MASKED, POL>(a, s0.row, s0.blk, lane, ra, ma);
        SweepBlock xa = sweep_block(a, s0);
        for (int j = 0; j < (S - 2) / 2; ++j) {
            const int kb = ks + pl.np, kc = ks + 2 * pl.np;  // kc is at most k0
            const bool lb = kb < pl.lim, lc = kc < pl.lim;
            const SweepCursor s1 = cursor_at(a, block_of(pl, lb ? kb : pl.kfirst));
            issue_block<ET, MASKED, POL>(a, s1.row, s1.blk, lane, rb, mb, lb);
            const SweepBlock xb = sweep_block(a, s1);
            if (!xa.skip) reduce_block<ET, MASKED, TOPK>(a, xa, lane, ra, ma, st, count++, keep);
            else settle(ra[G - 1]);
            if (count == kWave) {
                flush_stash(a, st, key, lane, count);
                st.kind = 0;
                count = 0;
            }
            const SweepCursor s2 = cursor_at(a, block_of(pl, lc ? kc : pl.kfirst));
            issue_block<ET, MASKED, POL>(a, s2.row, s2.blk, lane, ra, ma, lc);
            xa = sweep_block(a, s2);
            if (lb && !xb.skip) reduce_block<ET, MASKED, TOPK>(a, xb, lane, rb, mb, st, count++, keep);
            else settle(rb[G - 1]);
            if (count == kWave) {
                flush_stash(a, st, key, lane, count);
                st.kind = 0;
                count = 0;
            }
            if (!lc) {  // the partition ends within the static blocks
                settle(ra[G - 1]);
                flush_stash(a, st, key, lane, count);
                return;
            }
            ks = kc;
        }
    }
    // Blocks in flight: the current one's loads, the next one's index, and the
    // claims of the two after (issued before the loads of the blocks ahead of
    // them, so that waiting for a claim never waits for those loads).  A dead
    // look-ahead issue (no next block) names the wave's first block and reads
    // nothing.
    // Each block's loads are issued before the rest of its description is
    // worked out (the temperature scale is a double division): temporaries
    // placed after the issue cannot take the registers the loads fill, and a
    // temporary in a register with a load outstanding waits for every load.
    SweepBlock sa;
    if (S > 2) {
        sa = sweep_block(a, cursor_at(a, block_of(pl, pl.k0)));  // its loads are in flight
    } else {
        const SweepCursor c0 = cursor_at(a, block_of(pl, pl.k0));
        issue_block<ET, MASKED, POL>(a, c0.row, c0.blk, lane, ra, ma);
        sa = sweep_block(a, c0);
    }
    // Two claims are in flight, one for each half of the loop (claims of one
    // lane on one address return in the order issued, so once a claim finds
    // the partition exhausted, so does the other).  Claims are issued without
    // a condition: one past the end only returns "exhausted", and a claim kept
    // under a condition would have its register copied, which waits for it.
    int kn = pl.k1;
    uint32_t ca = claim(pl, lane);
    uint32_t cb = claim(pl, lane);
    // One exit, at the bottom: with breaks in both halves the compiler's
    // loop form has paths on which the look-ahead's loads look outstanding
    // at the top, and every temporary placed in those registers then waits
    // for all loads.
    bool more = true;
    do {
        const bool more1 = kn < pl.lim;
        const SweepCursor c1 = cursor_at(a, block_of(pl, more1 ? kn : pl.k0));
        issue_block<ET, MASKED, POL>(a, c1.row, c1.blk, lane, rb, mb, more1);
        const SweepBlock sb = sweep_block(a, c1);
        if (!sa.skip) reduce_block<ET, MASKED, TOPK>(a, sa, lane, ra, ma, st, count++, keep);
        else settle(ra[G - 1]);
        if (count == kWave) {
            flush_stash(a, st, key, lane, count);
            st.kind = 0;
            count = 0;
        }
        if (more1) {
            kn = claimed(pl, ca);
            const bool more2 = kn < pl.lim;
            ca = claim(pl, lane);
            const SweepCursor c2 = cursor_at(a, block_of(pl, more2 ? kn : pl.k0));
            issue_block<ET, MASKED, POL>(a, c2.row, c2.blk, lane, ra, ma, more2);
            sa = sweep_block(a, c2);
            if (!sb.skip) reduce_block<ET, MASKED, TOPK>(a, sb, lane, rb, mb, st, count++, keep);
            else settle(rb[G - 1]);
            if (count == kWave) {
                flush_stash(a, st, key, lane, count);
                st.kind = 0;
                count = 0;
            }
            if (more2) {
                kn = claimed(pl, cb);
                cb = claim(pl, lane);
            } else {
                settle(ra[G - 1]);  // the dead look-ahead (it reads nothing)
                more = false;
            }
        } else {
            settle(rb[G - 1]);
            more = false;
        }
    } while (more);
    flush_stash(a, st, key, lane, count);
}

// POL: the cache policy of the logits loads.
template <typename ET, bool MASKED, int TOPK, int POL>
__global__ __launch_bounds__(kSweepThreads) void row_stats_vec_kernel(RowStatsArgs a) {
    zero_call_outputs(a);
    if (a.fold) {
        if (!fold_ragged(a)) return;  // malformed ragged call: finalize reports it
    } else if (a.off && uniform_load(a.off_ok) == 0u) {
        return;
    }
    const int lane = threadIdx.x & (kWave - 1);
    if constexpr (MASKED && sizeof(ET) == 2) {
        __shared__ uint4 keep[256];
        fill_keep_table(keep);
        __syncthreads();
        sweep_claimed<ET, MASKED, TOPK, POL>(a, lane, keep);
    } else {
        sweep_claimed<ET, MASKED, TOPK, POL>(a, lane, nullptr);
    }
}

// Any alignment and any V: element loads clamped into the row, one chunk of
// blocks of one row per wave.
template <typename ET, bool MASKED>
__device__ __forceinline__ void load_block_elem(const ET *rowp, const uint8_t *mrow, int blk, int V,
                                                int lane, float *v, uint32_t *m) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
#pragma unroll
    for (int g = 0; g < G; ++g) {
        uint32_t bits = 0u;
#pragma unroll
        for (int e = 0; e < P; ++e) {
            const int64_t tok = int64_t(blk) * kBlock + (g * kWave + lane) * P + e;
            const int64_t tc = tok < V ? tok : int64_t(V - 1);
            const float x = Logit<ET>::to_float(rowp[tc]);
            bool live = tok < V;
            const bool mbit = MASKED ? ((mrow[tc >> 3] >> (tc & 7)) & 1u) : true;
            live = live && mbit;
            bits |= uint32_t(mbit) << e;
            v[g * P + e] = live ? x : -INFINITY;
        }
        // bits already aligned to the group, as record_draft reads them for P == 8
        m[g] = (P == 8) ? bits : (bits << ((lane & 1) * 4));
    }
}

template <typename ET, bool MASKED, int TOPK>
__global__ __launch_bounds__(kThreads) void row_stats_elem_kernel(RowStatsArgs a) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    zero_call_outputs(a);
    if (a.off && uniform_load(a.off_ok) == 0u) return;  // malformed ragged call: finalize reports it
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t task = int64_t(blockIdx.x) * (kThreads / kWave) + wave_id();
    if (task >= a.ntasks) return;
    const RowTask t = row_task(a, task);
    if (t.skip) return;
    const PhiloxKey key = key_of(a.seed);
    const ET *rowp = reinterpret_cast<const ET *>(a.logits) + int64_t(t.row) * a.V;
    const uint8_t *mrow =
        MASKED ? reinterpret_cast<const uint8_t *>(a.mask + int64_t(t.row) * a.W) : nullptr;
    float v[G * P];
    uint32_t m[G];
    for (int blk = t.c0; blk < t.c1; ++blk) {
        load_block_elem<ET, MASKED>(rowp, mrow, blk, a.V, lane, v, m);
        if (TOPK == 1) apply_tau<G * P>(v, t.tau);
        BlockStat out;
        out.key = -INFINITY;
        float sx = 0.0f;
        if (t.greedy) {
            const float2 r = greedy_block<G, P>(v, int64_t(blk) * kBlock, lane);
            out.m = r.x;
            out.s = r.y;
        } else {
            const float2 r = softmax_block<G * P>(v, t.c);
            out.m = r.x;
            out.s = r.y;
            const double g = block_gumbel(key, t.b, t.i, blk);
            out.key = key_of_mass(r.y, r.x, g);
            if (blk == t.xblk) {
                sx = excluded_sum<G, P>(v, t.c, r.x, t.xrel, lane);
                if (lane == 0) a.drec[t.row].keyx = key_of_mass(sx, r.x, g);
            }
        }
        if (blk == t.xblk) record_draft<G, P, true>(a, t.row, t.dpos, t.x, t.xrel, v, m, lane, sx);
        if (lane == 0) a.bstats[int64_t(t.row) * a.C + blk] = out;
    }
}

// ------------------------------------------------------------------ top-k

// Per row of a sampling request with top_k = K > 0: tau = the K-th largest
// allowed finite logit, counted with multiplicity, or -inf when the row holds
// at most K such logits (pyshine "vLLM, part 2", "Verification: rejection
// sampling on the GPU": top-k is applied to the logits before the accept
// test).  The kept set is {allowed, finite, l >= tau}: every tie at the K-th
// value stays.  Greedy rows, rows with top-k off and rows of requests with a
// bad temperature get -inf.  The row statistics and the sampler then treat
// l < tau like a masked token.
//
// Selection runs on order-preserving 32-bit codes of the values.  The top 16
// bits (the bf16 value itself) are counted in a histogram over a window of
// consecutive codes (256 for the first pass, 1024 after) placed around the
// largest code of the row's first 16 KB; elements above the window are only
// counted.  When the K-th largest
// lies outside the window, the window moves (another pass over the row) in the
// one direction that can hold it.  For fp32 rows two more passes pick the low
// two bytes among the elements that share the selected top half.
struct TopkArgs {
    const void *logits;
    const uint32_t *mask;
    const float *temperature;
    const int32_t *top_k;
    float *tau;  // [rows]
    uint32_t *tau_flag;      // [rows] 1: the top-p cut of the row is a boundary case
    const float *top_p;      // [B] or nullptr
    const int32_t *off;      // ragged: draft offsets, or nullptr
    const int32_t *row_req;  // ragged: request of each row
    const uint32_t *off_ok;  // ragged: 1 when the offsets are consistent
    int kp1, V, W;
};

constexpr int kTopkThreads = 256;
constexpr int kTopkWaves = kTopkThreads / kWave;
constexpr int kTopkWindow = 1024;
constexpr int kTopkUnroll = 4;
// The first window spans one binade of bf16 codes on either side of the
// anchor: for top-k of a few percent of the vocabulary or less it holds the
// K-th largest, and it draws few of the row's elements into the histogram.
constexpr uint32_t kTopkFirstSpan = 256;
constexpr double kTopPFlagEps = 1e-9;  // boundary threshold of a top-p cut, relative to the mass

// Bins ahead of the window, one per lane: the window pass over raw bf16 codes
// adds every element to some bin, those below the window to their lane's.
constexpr int kTopkLead = kWave;

struct TopkShared {
    // the lanes' bins, the window's bins, and one more: the raw bf16 pass
    // counts the elements above a window of n bins in bin n
    uint32_t bins[kTopkLead + kTopkWindow + 1];
    uint32_t part[kTopkThreads];  // per-thread sums of 4 bins, scanned in place
    uint32_t red[kTopkWaves];
    uint32_t found_digit, found_rank, lowest;
    __device__ __forceinline__ uint32_t *hist() { return bins + kTopkLead; }
};

// The top-p selection's per-bin masses beside the top-k histogram (only the
// kernels that apply top-p carry them).
struct ToppShared : TopkShared {
    double mass[kTopkWindow];     // kept mass per bin
    double dpart[kTopkThreads];
    double red_d[kTopkWaves];
    double found_mass;
};

// What the top-k selection leaves for a top-p cut after it.
struct TopkResult {
    float tau;         // the threshold; -inf when every supported token stays
    uint32_t lo;       // first code (top 16 bits) of the last histogram window
    uint32_t maxcode;  // the row's largest allowed finite code (0: none)
    bool window;       // bf16 rows: hist holds, per code from lo, the count of
                       // every kept element (nothing kept lies above the window)
};

// The bf16 value whose order-preserving code has top half d (a bf16 value's
// 32-bit code has an all-zero low half when positive, all-one when negative).
__device__ __forceinline__ float bf16_value_of_digit(uint32_t d) {
    return float_of_code((d << 16) | ((d & 0x8000u) ? 0u : 0xffffu));
}

// 2^t for t <= 0 in fp64, within about 3e-13 relative: t = n + f with
// n = rint(t) and |f| <= 1/2; e^(f ln 2) from its Taylor series to degree 10
// (the first omitted term, (ln 2 / 2)^11 / 11!, is below 2.2e-13), scaled by
// 2^n.  Arguments below -1100 give 0.  Top-p masses need far less than fp64
// rounding but far more than fp32 gives (the boundary band is 1e-9 of the
// mass), and this costs about half a general exp2.
__device__ __forceinline__ double exp2_precise_nonpos(double t) {
    t = fmax(t, -1100.0);
    const double n = rint(t);
    const double y = (t - n) * 0.6931471805599453;  // ln 2
    double p = 1.0 / 3628800.0;                     // 1/10!
    p = fma(p, y, 1.0 / 362880.0);
    p = fma(p, y, 1.0 / 40320.0);
    p = fma(p, y, 1.0 / 5040.0);
    p = fma(p, y, 1.0 / 720.0);
    p = fma(p, y, 1.0 / 120.0);
    p = fma(p, y, 1.0 / 24.0);
    p = fma(p, y, 1.0 / 6.0);
    p = fma(p, y, 0.5);
    p = fma(p, y, 1.0);
    p = fma(p, y, 1.0);
    return ldexp(p, static_cast<int>(n));
}

// The P values of one 16-byte group of the row at token `tok` with excluded
// tokens (masked, past V, NaN, +-inf) as NaN.
template <typename ET, bool ALIGNED>
__device__ __forceinline__ void topk_group(const ET *rowp, const uint8_t *mrow, int V, int64_t tok,
                                           float *v) {
    constexpr int P = Logit<ET>::kPer16;
    load_group<ET, ALIGNED>(rowp, tok, V, v);
    uint32_t bits = 0xffu;
    if (mrow != nullptr && tok < V) {
        if (ALIGNED) {
            const uint32_t byte = mrow[tok >> 3];
            bits = (P == 8) ? byte : (byte >> (uint32_t(tok) & 4u));
        } else {
            bits = 0u;
#pragma unroll
            for (int e = 0; e < P; ++e) {
                const int64_t j = tok + e < V ? tok + e : int64_t(V - 1);
                bits |= ((mrow[j >> 3] >> (j & 7)) & 1u) << e;
            }
        }
    }
#pragma unroll
    for (int e = 0; e < P; ++e) {
        const bool live = ((bits >> e) & 1u) && fabsf(v[e]) <= FLT_MAX;  // finite
        if (!live) v[e] = NAN;
    }
}

// The same for 16-byte aligned rows with V a multiple of P, through buffer
// loads: a group past V reads zeros (no memory access) and is excluded by
// its index, so no branch guards a load and the loads of several groups stay
// in flight together.
template <typename ET, bool MASKED>
__device__ __forceinline__ void topk_group_vec(__amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rm,
                                               int V, int64_t tok, float *v) {
    constexpr int P = Logit<ET>::kPer16;
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 w = __builtin_amdgcn_raw_buffer_load_b128(rs, static_cast<int>(tok * int64_t(sizeof(ET))), 0, 0);
    Logit<ET>::unpack(make_uint4(w.x, w.y, w.z, w.w), v);
    uint32_t bits = tok < V ? 0xffu : 0u;
    if (MASKED) {
        const uint32_t byte = __builtin_amdgcn_raw_buffer_load_b8(rm, static_cast<int>(tok >> 3), 0, 0);
        bits &= (P == 8) ? byte : (byte >> (uint32_t(tok) & 4u));
    }
#pragma unroll
    for (int e = 0; e < P; ++e) {
        const bool live = ((bits >> e) & 1u) && fabsf(v[e]) <= FLT_MAX;
        v[e] = live ? v[e] : NAN;
    }
}

// One group of the row for the top-k passes, through the path the row allows.
template <typename ET, bool ALIGNED, bool MASKED>
__device__ __forceinline__ void topk_load(const ET *rowp, const uint8_t *mrow,
                                          __amdgpu_buffer_rsrc_t rs, __amdgpu_buffer_rsrc_t rm, int V,
                                          int64_t tok, float *v) {
    if (ALIGNED) topk_group_vec<ET, MASKED>(rs, rm, V, tok, v);
    else topk_group<ET, false>(rowp, MASKED ? mrow : nullptr, V, tok, v);
}

// Finds, in a histogram of `nbins` bins (bin i = digit lo + i), the bin that
// holds the need-th largest element counted from the top.  Returns false
// when the histogram holds fewer than `need` elements.  All threads call it.
__device__ bool topk_pick(TopkShared &sh, int nbins, uint32_t lo, uint32_t need, uint32_t &digit,
                          uint32_t &rank) {
    const int tid = threadIdx.x;
    const int per = nbins / kTopkThreads;  // 4 or 1
    uint32_t own = 0;
    for (int i = 0; i < per; ++i) own += sh.hist()[tid * per + i];
    sh.part[tid] = own;
    // inclusive suffix sums: part[t] = sum of part[t'] for t' >= t
    for (int d = 1; d < kTopkThreads; d <<= 1) {
        lds_barrier();
        const uint32_t add = (tid + d < kTopkThreads) ? sh.part[tid + d] : 0u;
        lds_barrier();
        sh.part[tid] += add;
    }
    lds_barrier();
    const uint32_t incl = sh.part[tid];
    if (tid == 0) sh.found_digit = 0xffffffffu;
    lds_barrier();
    if (incl >= need && incl - own < need) {
        uint32_t acc = incl - own;
        for (int i = per - 1; i >= 0; --i) {
            const uint32_t h = sh.hist()[tid * per + i];
            if (acc + h >= need) {
                sh.found_digit = lo + uint32_t(tid * per + i);
                sh.found_rank = need - acc;
                break;
            }
            acc += h;
        }
    }
    lds_barrier();
    digit = sh.found_digit;
    rank = sh.found_rank;
    return digit != 0xffffffffu;
}

// One row of the threshold kernel: where its logits and mask lie.
template <typename ET, bool ALIGNED, bool MASKED>
struct TopkRow {
    const ET *rowp;
    const uint8_t *mrow;
    __amdgpu_buffer_rsrc_t rs, rm;
    int V;
    static constexpr int64_t kStep = int64_t(kTopkThreads) * Logit<ET>::kPer16;
    __device__ __forceinline__ void load(int64_t tok, float *v) const {
        topk_load<ET, ALIGNED, MASKED>(rowp, mrow, rs, rm, V, tok, v);
    }
    // Aligned rows: the raw 16-byte groups tok0 + u * kStep (u < kTopkUnroll)
    // and their mask bytes, with one offset register for all of them (the
    // groups' distance rides in the scalar offset).  Past V: zeros.
    __device__ __forceinline__ void raw(int64_t tok0, uint4 *w, uint32_t *m) const {
        typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
        const int off = static_cast<int>(tok0 * int64_t(sizeof(ET)));
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, u * int(kStep * sizeof(ET)), 0);
            w[u] = make_uint4(x.x, x.y, x.z, x.w);
        }
        if (MASKED) {
            const int moff = static_cast<int>(tok0 >> 3);
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u)
                m[u] = __builtin_amdgcn_raw_buffer_load_b8(rm, moff, u * int(kStep / 8), 0);
        }
    }
    // The values of such a batch, excluded tokens (masked, past V, NaN,
    // +-inf) as NaN, as load() gives them.
    __device__ __forceinline__ void values(int64_t tok0, const uint4 *w, const uint32_t *m,
                                           float (*v)[Logit<ET>::kPer16]) const {
        constexpr int P = Logit<ET>::kPer16;
#pragma unroll
        for (int u = 0; u < kTopkUnroll; ++u) {
            const int64_t tok = tok0 + u * kStep;
            Logit<ET>::unpack(w[u], v[u]);
            uint32_t bits = tok < V ? 0xffu : 0u;
            if (MASKED) bits &= (P == 8) ? m[u] : (m[u] >> (uint32_t(tok) & 4u));
#pragma unroll
            for (int e = 0; e < P; ++e) {
                const bool live = ((bits >> e) & 1u) && fabsf(v[u][e]) <= FLT_MAX;
                v[u][e] = live ? v[u][e] : NAN;
            }
        }
    }
};

// Per 16-bit half of a word of bf16 values: the half's order-preserving code
// (the top half of the 32-bit code of the value), and the larger of two codes.
__device__ __forceinline__ uint32_t bf16_codes(uint32_t x) {
    typedef short s16x2 __attribute__((ext_vector_type(2)));
    const uint32_t sgn = __builtin_bit_cast(uint32_t, __builtin_bit_cast(s16x2, x) >> (s16x2){15, 15});
    // per bit, (x ^ sgn) | (0x80008000 & ~x): a negative half has every bit
    // flipped, a positive one its sign bit set; one three-input bit op (the
    // compiler splits this form into three)
    uint32_t c;
    asm("v_bitop3_b32 %0, %1, %2, %3 bitop3:0x3e" : "=v"(c) : "v"(x), "v"(sgn), "s"(0x80008000u));
    return c;
}

// The middle of three signed integers (one instruction; the compiler's
// min-of-max form takes two).
__device__ __forceinline__ int med3_i32(int a, int lo, int hi) {
    int r;
    asm("v_med3_i32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(lo), "v"(hi));
    return r;
}

__device__ __forceinline__ uint32_t max_u16x2(uint32_t a, uint32_t b) {
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2, a),
                                                                  __builtin_bit_cast(u16x2, b)));
}

// The row's access for the selection passes.
template <typename ET, bool ALIGNED, bool MASKED>
__device__ __forceinline__ TopkRow<ET, ALIGNED, MASKED> topk_row(const void *logits, const uint32_t *mask,
                                                                 int64_t row, int V, int W) {
    TopkRow<ET, ALIGNED, MASKED> r;
    r.rowp = reinterpret_cast<const ET *>(logits) + row * V;
    r.mrow = MASKED ? reinterpret_cast<const uint8_t *>(mask + row * W) : nullptr;
    r.rs = buffer_of(r.rowp, uint32_t(V) * sizeof(ET));
    r.rm = buffer_of(MASKED ? static_cast<const void *>(r.mrow) : static_cast<const void *>(r.rowp),
                     MASKED ? uint32_t(W) * 4u : 0u);
    r.V = V;
    return r;
}

// The K-th largest allowed finite logit of the row, or -inf when the row
// holds at most K of them (see the comment above TopkArgs); also the row's
// largest code and, for bf16 rows, whether the last histogram holds every
// kept element (the largest code only when TRACK_MAX: a top-p cut follows).
template <typename ET, bool ALIGNED, bool MASKED, bool TRACK_MAX>
__device__ TopkResult select_top_k(const TopkRow<ET, ALIGNED, MASKED> &r, TopkShared &sh, int K,
                                   const uint4 *keep) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int64_t kStep = int64_t(kTopkThreads) * P;
    const int tid = threadIdx.x;
    const int64_t V = r.V;

    // anchor: the largest top-half code among the first 16 KB of the row
    uint32_t anchor = 0;
    for (int64_t tok = int64_t(tid) * P; tok < V && tok < 4 * kStep; tok += kStep) {
        float v[P];
        r.load(tok, v);
#pragma unroll
        for (int e = 0; e < P; ++e)
            if (v[e] == v[e]) anchor = max(anchor, ordered_code(v[e]) >> 16);
    }
    anchor = block_max_u<kTopkWaves>(anchor, sh.red);

    uint32_t hi = min(anchor + 128u, 0xffffu);
    uint32_t span = kTopkFirstSpan;  // the first window is narrow: fewer LDS atomics
    const uint32_t need = static_cast<uint32_t>(K);
    uint32_t digit = 0, rank = 0, maxcode = 0, lo_found = 0, above_found = 0;
    bool first = true, found = false;
    // The window only ever moves one way (up while the K-th largest lies above
    // it, down while it lies below), so at most 65536 / kTopkWindow + 1 passes
    // run; the bound below is never reached.
    for (int pass = 0; pass < 0x10000 / kTopkWindow + 2; ++pass) {
        const uint32_t lo = hi >= span - 1 ? hi - (span - 1) : 0u;
        for (int i = tid; i < kTopkLead + kTopkWindow + 1; i += kTopkThreads) sh.bins[i] = 0u;
        lds_barrier();
        uint32_t above = 0, support = 0, mx = 0;
        auto count = [&](const float (&v)[kTopkUnroll][P]) {
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u)
#pragma unroll
                for (int e = 0; e < P; ++e) {
                    if (v[u][e] != v[u][e]) continue;
                    ++support;
                    const uint32_t c = ordered_code(v[u][e]);
                    if (TRACK_MAX) mx = max(mx, c);
                    const uint32_t d = c >> 16;
                    if (d > hi) ++above;
                    else if (d >= lo) atomicAdd(&sh.hist()[d - lo], 1u);
                }
        };
        constexpr int64_t kBatch = kTopkUnroll * kStep;
        if constexpr (ALIGNED) {
            // bf16: each element's 16-bit code straight from the raw words,
            // and its bin without a branch: the offset from lo, clamped below
            // to a bin of the lane ahead of the window and above to the bin
            // past it, whose count is then the count above the window.  Valid
            // codes are 0x0080 .. 0xff7f (-inf and negative NaNs code below,
            // +inf and positive NaNs above); masked tokens get code 0.  A
            // batch that reaches past V, holds an allowed +inf or NaN, or
            // meets a window starting below 0x0080 is counted element by
            // element instead.  The wave's support count rides in a scalar.
            uint32_t support_w = 0, mx16 = 0;
            const int lane_bin = -1 - (tid & (kWave - 1));
            auto count_codes = [&](int64_t t0, const uint4 (&w)[kTopkUnroll], const uint32_t (&m)[kTopkUnroll]) {
                if (lo < 0x80u || __ballot(t0 + (kTopkUnroll - 1) * kStep >= V) != 0ull) return false;
                uint32_t c[kTopkUnroll][4];
                uint32_t bm = 0;
#pragma unroll
                for (int u = 0; u < kTopkUnroll; ++u) {
                    const uint32_t x[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
                    uint4 k = make_uint4(~0u, ~0u, ~0u, ~0u);
                    if (MASKED) k = keep[m[u]];
                    const uint32_t kk[4] = {k.x, k.y, k.z, k.w};
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        c[u][j] = MASKED ? bf16_codes(x[j]) & kk[j] : bf16_codes(x[j]);
                        bm = max_u16x2(bm, c[u][j]);
                    }
                }
                const uint32_t top = max(bm & 0xffffu, bm >> 16);
                if (__ballot(top >= 0xff80u) != 0ull) return false;
                if (TRACK_MAX) mx16 = max(mx16, top);
                if (first) {
#pragma unroll
                    for (int u = 0; u < kTopkUnroll; ++u)
#pragma unroll
                        for (int j = 0; j < 8; ++j) {
                            const uint32_t d = (j & 1) ? (c[u][j >> 1] >> 16) : (c[u][j >> 1] & 0xffffu);
                            support_w += __popcll(__ballot(d >= 0x80u));
                        }
                }
#pragma unroll
                for (int u = 0; u < kTopkUnroll; ++u)
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const uint32_t d = (j & 1) ? (c[u][j >> 1] >> 16) : (c[u][j >> 1] & 0xffffu);
                        const int t = int(d) - int(lo);
                        atomicAdd(&sh.hist()[med3_i32(t, lane_bin, int(span))], 1u);
                    }
                return true;
            };
            // kTopkUnroll groups per thread per batch, two batches in flight:
            // the next batch loads while this one is counted
            auto count_raw = [&](int64_t t0, const uint4 (&w)[kTopkUnroll], const uint32_t (&m)[kTopkUnroll]) {
                if constexpr (sizeof(ET) == 2)
                    if (count_codes(t0, w, m)) return;
                float v[kTopkUnroll][P];
                r.values(t0, w, m, v);
                count(v);
            };
            uint4 wa[kTopkUnroll], wb[kTopkUnroll];
            uint32_t ma[kTopkUnroll] = {}, mb[kTopkUnroll] = {};
            int64_t tok0 = int64_t(tid) * P;
            r.raw(tok0, wa, ma);
            for (; tok0 < V; tok0 += 2 * kBatch) {
                r.raw(tok0 + kBatch, wb, mb);
                count_raw(tok0, wa, ma);
                if (tok0 + kBatch >= V) break;
                r.raw(tok0 + 2 * kBatch, wa, ma);
                count_raw(tok0 + kBatch, wb, mb);
            }
            if (sizeof(ET) == 2) {
                if (TRACK_MAX && mx16 >= 0x80u) mx = max(mx, (mx16 << 16) | ((mx16 & 0x8000u) ? 0u : 0xffffu));
                if ((tid & (kWave - 1)) == 0) support += support_w;
            }
        } else {  // element loads: one batch at a time
            for (int64_t tok0 = int64_t(tid) * P; tok0 < V; tok0 += kBatch) {
                float v[kTopkUnroll][P];
#pragma unroll
                for (int u = 0; u < kTopkUnroll; ++u) r.load(tok0 + u * kStep, v[u]);
                count(v);
            }
        }
        above = block_sum_u<kTopkWaves>(above, sh.red);
        if (ALIGNED && sizeof(ET) == 2) above += sh.hist()[span];  // the raw pass's count above the window
        if (first) {
            support = block_sum_u<kTopkWaves>(support, sh.red);
            if (TRACK_MAX) maxcode = block_max_u<kTopkWaves>(mx, sh.red);
            if (support <= need) return TopkResult{-INFINITY, 0u, maxcode, false};  // every token stays
            first = false;
        }
        if (above >= need) {  // the K-th largest lies above the window
            hi = min(hi + span, 0xffffu);
            span = kTopkWindow;
            continue;
        }
        if (topk_pick(sh, int(span), lo, need - above, digit, rank)) {  // bins from span on: not the window's
            found = true;
            lo_found = lo;
            above_found = above;
            break;
        }
        if (lo == 0u) break;  // cannot happen: the row holds more than K
        hi = lo - 1u;         // the K-th largest lies below the window
        span = kTopkWindow;
    }
    if (!found) return TopkResult{-INFINITY, 0u, maxcode, false};

    uint32_t code;
    if (sizeof(ET) == 2) {
        // a bf16 value's code has all-zero (positive) or all-one (negative) low half
        code = (digit << 16) | ((digit & 0x8000u) ? 0u : 0xffffu);
    } else {
        uint32_t prefix = digit;  // selected high bits so far
        uint32_t want = rank;
        for (int shift = 8; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kTopkThreads) sh.hist()[i] = 0u;
            lds_barrier();
            for (int64_t tok = int64_t(tid) * P; tok < V; tok += kStep) {
                float v[P];
                r.load(tok, v);
#pragma unroll
                for (int e = 0; e < P; ++e) {
                    if (v[e] != v[e]) continue;
                    const uint32_t c = ordered_code(v[e]);
                    if ((c >> (shift + 8)) == prefix) atomicAdd(&sh.hist()[(c >> shift) & 0xffu], 1u);
                }
            }
            lds_barrier();
            uint32_t byte = 0, rk = 0;
            topk_pick(sh, 256, 0u, want, byte, rk);  // holds `want` elements by construction
            prefix = (prefix << 8) | byte;
            want = rk;
        }
        code = prefix;
    }
    return TopkResult{float_of_code(code), lo_found, maxcode, sizeof(ET) == 2 && above_found == 0u};
}

// Suffix sums of the per-bin masses (bin i = digit lo + i, nbins of them):
// finds the bin where the mass counted from the top first reaches `target`.
// Returns false when the histogram holds less; `before` receives the mass
// above the found bin.  All threads call it.
__device__ bool topp_pick(ToppShared &sh, int nbins, uint32_t lo, double target, uint32_t &digit,
                          double &before, bool clamp) {
    const int tid = threadIdx.x;
    const int per = nbins / kTopkThreads;  // 4 or 1
    double own = 0.0;
    for (int i = 0; i < per; ++i) own += sh.mass[tid * per + i];
    sh.dpart[tid] = own;
    if (tid == 0) sh.lowest = 0xffffffffu;
    for (int d = 1; d < kTopkThreads; d <<= 1) {
        lds_barrier();
        const double add = (tid + d < kTopkThreads) ? sh.dpart[tid + d] : 0.0;
        lds_barrier();
        sh.dpart[tid] += add;
    }
    lds_barrier();
    const double incl = sh.dpart[tid];
    if (tid == 0) sh.found_digit = 0xffffffffu;
    for (int i = 0; i < per; ++i)
        if (sh.mass[tid * per + i] > 0.0) atomicMin(&sh.lowest, uint32_t(tid * per + i));
    lds_barrier();
    if (incl >= target && incl - own < target) {
        double acc = incl - own;
        for (int i = per - 1; i >= 0; --i) {
            const double m = sh.mass[tid * per + i];
            if (acc + m >= target) {
                sh.found_digit = lo + uint32_t(tid * per + i);
                sh.found_mass = acc;
                break;
            }
            acc += m;
        }
    }
    lds_barrier();
    // A refinement pass sums the bin it refines in another order: a target
    // at the bin's very bottom may then sit a rounding error beyond its
    // sub-bins, and the lowest non-empty sub-bin is the cut.
    if (clamp && sh.found_digit == 0xffffffffu && sh.lowest != 0xffffffffu) {
        digit = lo + sh.lowest;
        before = sh.dpart[0] - sh.mass[sh.lowest];
        lds_barrier();
        return true;
    }
    digit = sh.found_digit;
    before = sh.found_mass;
    lds_barrier();  // the next histogram pass may clear the shared fields
    return digit != 0xffffffffu;
}

// The top-p cut of the row over the tokens with l >= tau_k: the largest
// logit value v whose tokens >= v hold top_p of the tempered mass left by
// top-k (pyshine "vLLM, part 2", "Verification": top-p among the sampling
// constraints applied before the accept test; ties at v stay).  Masses are
// 2^((l - M) log2(e) / T) with M the row's largest kept logit, in fp64 from
// the argument on (a cut deep in a long tail steps by masses far below fp32
// rounding).  *flag is set when the mass at the cut, or just above it, lies
// within the boundary threshold of top_p.  `known_max` (with have_max) is the
// row's largest allowed finite code when top-k already found it, which saves
// a pass over the row.
template <typename ET, bool ALIGNED, bool MASKED>
__device__ float select_top_p(const TopkRow<ET, ALIGNED, MASKED> &r, ToppShared &sh, float tau_k,
                              uint32_t known_max, bool have_max, float top_p, float T, uint32_t *flag) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int64_t kStep = int64_t(kTopkThreads) * P;
    constexpr bool kBf16 = sizeof(ET) == 2;
    constexpr int kPer = kTopkWindow / kTopkThreads;
    const int tid = threadIdx.x;
    const int64_t V = r.V;
    // the largest kept logit
    uint32_t mcode = known_max;
    if (!have_max) {
        for (int64_t tok0 = int64_t(tid) * P; tok0 < V; tok0 += kTopkUnroll * kStep) {
            float v[kTopkUnroll][P];
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) r.load(tok0 + u * kStep, v[u]);
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u)
#pragma unroll
                for (int e = 0; e < P; ++e)
                    if (v[u][e] == v[u][e] && !(v[u][e] < tau_k)) mcode = max(mcode, ordered_code(v[u][e]));
        }
        mcode = block_max_u<kTopkWaves>(mcode, sh.red);
    }
    *flag = 0u;
    if (mcode == 0u) return tau_k;  // nothing kept: the row is reported empty
    const float M = float_of_code(mcode);
    const double cd = kLog2e / static_cast<double>(T);
    const double mcd = static_cast<double>(M) * cd;

    const uint32_t top = mcode >> 16;
    uint32_t hi = top, span = kTopkFirstSpan;
    double total = 0.0, target = 0.0;
    uint32_t digit = 0;
    double before = 0.0, above_mass = 0.0;
    uint32_t lo_found = 0;
    bool found = false;
    // The first pass sums the whole kept mass; each further pass moves the
    // window down, so at most 65536 / kTopkWindow + 1 passes run.  bf16 bins
    // hold one value each: they are counted and priced once per bin.
    for (int pass = 0; pass < 0x10000 / kTopkWindow + 2; ++pass) {
        const uint32_t lo = hi >= span - 1 ? hi - (span - 1) : 0u;
        for (int i = tid; i < kTopkWindow; i += kTopkThreads) {
            if (kBf16) sh.hist()[i] = 0u;
            else sh.mass[i] = 0.0;
        }
        lds_barrier();
        double below = 0.0, in_window = 0.0;
        for (int64_t tok0 = int64_t(tid) * P; tok0 < V; tok0 += kTopkUnroll * kStep) {
            float v[kTopkUnroll][P];
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u) r.load(tok0 + u * kStep, v[u]);
#pragma unroll
            for (int u = 0; u < kTopkUnroll; ++u)
#pragma unroll
                for (int e = 0; e < P; ++e) {
                    const float x = v[u][e];
                    if (x != x || x < tau_k) continue;
                    const uint32_t d = ordered_code(x) >> 16;
                    if (d > hi) continue;  // counted in an earlier pass
                    if (d >= lo) {
                        if (kBf16) {
                            atomicAdd(&sh.hist()[d - lo], 1u);
                        } else {
                            const double w = exp2_precise_nonpos(fma(static_cast<double>(x), cd, -mcd));
                            atomicAdd(&sh.mass[d - lo], w);
                            in_window += w;
                        }
                    } else if (pass == 0) {  // below the window: only the total needs it
                        below += exp2_precise_nonpos(fma(static_cast<double>(x), cd, -mcd));
                    }
                }
        }
        if (kBf16) {
            lds_barrier();
#pragma unroll
            for (int i = 0; i < kPer; ++i) {
                const int bin = tid * kPer + i;
                const uint32_t n = sh.hist()[bin];
                const double m = n ? static_cast<double>(n) *
                                         exp2_precise_nonpos(fma(static_cast<double>(bf16_value_of_digit(lo + bin)), cd, -mcd))
                                   : 0.0;
                sh.mass[bin] = m;
                in_window += m;
            }
        }
        if (pass == 0) below = block_sum_d<kTopkWaves>(below, sh.red_d);
        in_window = block_sum_d<kTopkWaves>(in_window, sh.red_d);
        if (pass == 0) {
            total = below + in_window;
            target = static_cast<double>(top_p) * total;
        }
        if (topp_pick(sh, kTopkWindow, lo, target - above_mass, digit, before, false)) {
            before += above_mass;
            lo_found = lo;
            found = true;
            break;
        }
        if (lo == 0u) break;  // cannot happen: the window sums reach the total
        above_mass += in_window;
        hi = lo - 1u;
        span = kTopkWindow;
    }
    if (!found) return tau_k;

    uint32_t code;
    double at_cut, just_above;
    if (sizeof(ET) == 2) {
        code = (digit << 16) | ((digit & 0x8000u) ? 0u : 0xffffu);
        at_cut = before + sh.mass[digit - lo_found];  // a bf16 bin holds one value
        just_above = before;
    } else {
        // two byte passes over the elements sharing the selected top half
        uint32_t prefix = digit;
        double above_bin = before;
        for (int shift = 8; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kTopkThreads) sh.mass[i] = 0.0;
            lds_barrier();
            for (int64_t tok = int64_t(tid) * P; tok < V; tok += kStep) {
                float v[P];
                r.load(tok, v);
#pragma unroll
                for (int e = 0; e < P; ++e) {
                    const float x = v[e];
                    if (x != x || x < tau_k) continue;
                    const uint32_t cc = ordered_code(x);
                    if ((cc >> (shift + 8)) == prefix)
                        atomicAdd(&sh.mass[(cc >> shift) & 0xffu], exp2_precise_nonpos(fma(static_cast<double>(x), cd, -mcd)));
                }
            }
            lds_barrier();
            uint32_t byte = 0;
            double b2 = 0.0;
            topp_pick(sh, 256, 0u, target - above_bin, byte, b2, true);
            above_bin += b2;
            if (shift == 0) at_cut = above_bin + sh.mass[byte];
            prefix = (prefix << 8) | byte;
        }
        code = prefix;
        just_above = above_bin;
    }
    const double eps = kTopPFlagEps * total;
    *flag = (fabs(at_cut - target) < eps || fabs(target - just_above) < eps) ? 1u : 0u;
    return float_of_code(code);
}

// The top-p cut of a bf16 row straight from the top-k histogram, when that
// holds every kept element (TopkResult::window): bin masses are the counts
// times the bin value's mass, so no pass over the row is needed.
__device__ float top_p_in_window(ToppShared &sh, const TopkResult &tk, float top_p, float T, uint32_t *flag) {
    constexpr int kPer = kTopkWindow / kTopkThreads;
    const int tid = threadIdx.x;
    const uint32_t tau_digit = ordered_code(tk.tau) >> 16;
    const double cd = kLog2e / static_cast<double>(T);
    const double mcd = static_cast<double>(float_of_code(tk.maxcode)) * cd;
    double acc = 0.0;
#pragma unroll
    for (int i = 0; i < kPer; ++i) {
        const int bin = tid * kPer + i;
        const uint32_t d = tk.lo + uint32_t(bin);
        const uint32_t n = sh.hist()[bin];
        const double m = (n != 0u && d >= tau_digit)
                             ? static_cast<double>(n) *
                                   exp2_precise_nonpos(fma(static_cast<double>(bf16_value_of_digit(d)), cd, -mcd))
                             : 0.0;
        sh.mass[bin] = m;
        acc += m;
    }
    const double total = block_sum_d<kTopkWaves>(acc, sh.red_d);
    const double target = static_cast<double>(top_p) * total;
    uint32_t digit = 0;
    double before = 0.0;
    *flag = 0u;
    if (!topp_pick(sh, kTopkWindow, tk.lo, target, digit, before, false)) return tk.tau;  // cannot happen
    const double at_cut = before + sh.mass[digit - tk.lo];
    const double eps = kTopPFlagEps * total;
    *flag = (fabs(at_cut - target) < eps || fabs(target - before) < eps) ? 1u : 0u;
    return bf16_value_of_digit(digit);
}

template <typename ET, bool ALIGNED, bool MASKED, bool TOPP>
__global__ __launch_bounds__(kTopkThreads) void topk_kernel(TopkArgs a) {
    __shared__ typename std::conditional<TOPP, ToppShared, TopkShared>::type sh;
    const int row = blockIdx.x, tid = threadIdx.x;
    if (a.off && uniform_load(a.off_ok) == 0u) return;  // malformed ragged call
    int b, i, kb;
    int64_t d0;
    row_owner(a.off, a.row_req, row, a.kp1, b, i, kb, d0);
    const float T = uniform_load(a.temperature + b);
    const int K = a.top_k ? uniform_load(a.top_k + b) : 0;
    const float Pp = TOPP ? uniform_load(a.top_p + b) : 0.0f;
    const bool use_p = TOPP && Pp > 0.0f && Pp < 1.0f;
    if (!(T > 0.0f && T <= FLT_MAX) || (K <= 0 && !use_p)) {
        if (tid == 0) {
            a.tau[row] = -INFINITY;
            a.tau_flag[row] = 0u;
        }
        return;
    }
    // masked bf16 rows: the keep-mask table of the raw-code pass
    __shared__ uint4 keep[(MASKED && ALIGNED && sizeof(ET) == 2) ? 256 : 1];
    if constexpr (MASKED && ALIGNED && sizeof(ET) == 2) {
        fill_keep_table(keep);
        lds_barrier();
    }
    const TopkRow<ET, ALIGNED, MASKED> r = topk_row<ET, ALIGNED, MASKED>(a.logits, a.mask, row, a.V, a.W);
    TopkResult tk{-INFINITY, 0u, 0u, false};
    if (K > 0) tk = select_top_k<ET, ALIGNED, MASKED, TOPP>(r, sh, K, keep);
    float tau = tk.tau;
    uint32_t flag = 0u;
    if constexpr (TOPP) {
        if (use_p)
            tau = tk.window ? top_p_in_window(sh, tk, Pp, T, &flag)
                            : select_top_p(r, sh, tk.tau, tk.maxcode, K > 0, Pp, T, &flag);
    }
    if (tid == 0) {
        a.tau[row] = tau;
        a.tau_flag[row] = flag;
    }
}

// ------------------------------------------------------- single-pass top-k

// Calls with top-k and no top-p find each row's threshold after the sweep,
// without a second pass over the row (pyshine "vLLM, part 2",
// "Verification": top-k is applied before the accept test).  The sweep
// records the code of every 128-byte line's largest allowed value (line
// maxima).  L, the K-th largest line maximum, is at most tau, the K-th
// largest allowed finite logit: K distinct lines each hold a value >= L.  So
// every kept token (l >= tau) lies in a line whose maximum is >= L, and tau
// is the K-th largest of the tokens >= L in those lines, of which there are
// at least K.  Only the candidate lines are read again, about K of the row's
// lines (a few KB of a 300 KB row).  One workgroup per row:
//   1. the row's line codes into LDS (and registers), their largest;
//   2. L from a histogram of the 1024 keys at and below the largest (a key is
//      a bf16 code, or the top half of an fp32 code, refined by two 8-bit
//      digit passes); rows whose K-th key lies further down search the codes
//      in LDS instead;
//   3. the candidate lines numbered through an LDS counter, their codes
//      replaced by their numbers, their tokens' codes loaded into LDS and
//      counted in the same window;
//   4. tau the same way;
//   5. the row's block statistics over the kept tokens with the sweep's
//      arithmetic: each candidate line's mass by a wave over its tokens, then
//      each block's sum over its lines in stored order.
// The sweep computes no statistics for these rows (only marks for an allowed
// NaN or +inf): rows with at most K allowed finite tokens keep every one
// (tau = -inf) and get their statistics here too; rows with a NaN or +inf,
// or without an allowed finite token, keep the sweep's marks, which report
// them.  Rows with more than kCandLines candidate lines (K > 128, or ties)
// take tau from radix passes over global memory.
struct LinesArgs {
    const void *logits;
    const uint32_t *mask;
    const float *temperature;
    const int32_t *top_k;
    const float *top_p;      // [B] (the kernels that apply top-p)
    const int32_t *draft;
    const void *linemax;     // [rows, C * lines per block], per block in the sweep's lane order
    BlockStat *bstats;       // [rows, C]
    DraftRec *drec;          // [rows]
    float *tau;              // [rows], written for every row
    uint32_t *tau_flag;      // [rows], written for every row (0: no top-p here)
    uint16_t *klist;         // dense q: [rows, kCandLines] the lines holding a kept token, ascending
    uint32_t *kcount;        // dense q: [rows] their number, kNoLineList when not listed; or nullptr
    const int32_t *off;      // ragged: draft offsets, or nullptr
    const int32_t *row_req;  // ragged: request of each row
    const uint32_t *off_ok;  // ragged: 1 when the offsets are consistent
    uint64_t seed;
    int kp1, V, W, C;
};

constexpr int kLinesThreads = 256;
constexpr int kLinesMax = 4096;   // lines of a row, 16 per thread (bf16 V <= 262144, fp32 V <= 131072)
constexpr int kCandLines = 128;   // candidate lines whose tokens are staged in LDS
constexpr uint32_t kNoLineList = 0xffffffffu;  // a row whose kept tokens are not listed by line
constexpr int kResLines = kFinalThreads / 2;   // lines per residual chunk: four groups per finalize thread
constexpr int kWin = 1024;        // keys in the window histogram

struct LinesShared {
    uint32_t hist[2][256];  // 8-bit digit histograms, alternating
    uint32_t digit, above, total;
    uint32_t ncand;         // candidate lines numbered so far
};

// The digit holding the K-th largest of the codes counted in hist (the
// caller's pass, already complete behind a barrier), given `above` codes known
// to lie above the prefix they share: the largest digit d with
// above + #(digits >= d) >= K, the codes above it, and the histogram's total.
// Wave 0 scans (four bins per lane, a shuffle suffix-sum over the lanes); one
// barrier publishes the result, and the histogram is then cleared for the
// pass after next.
__device__ __forceinline__ uint3 pick_digit(LinesShared &sh, int hb, uint32_t K, uint32_t above) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    if (wave_id() == 0) {
        uint32_t c[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) c[j] = sh.hist[hb][4 * lane + j];
        const uint32_t tot = c[0] + c[1] + c[2] + c[3];
        uint32_t suf = tot;  // bins >= 4 lane
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint32_t t = __shfl_down(suf, d);
            if (lane + d < kWave) suf += t;
        }
        const uint64_t hits = __ballot(above + suf >= K);
        const int hl = hits ? 63 - static_cast<int>(__builtin_clzll(hits)) : 0;
        if (lane == hl) {
            int j = 3;
            uint32_t sj = suf - c[0] - c[1] - c[2];  // bins >= 4 lane + 3
            while (j > 0 && above + sj < K) {
                --j;
                sj += c[j];
            }
            sh.digit = static_cast<uint32_t>(4 * lane + j);
            sh.above = above + sj - c[j];
        }
        if (lane == 0) sh.total = suf;
    }
    __syncthreads();
    const uint3 r = make_uint3(sh.digit, sh.above, sh.total);
    sh.hist[hb][tid] = 0u;  // read by wave 0 before the barrier; used again two passes on
    return r;
}

// The K-th largest of the codes counted in a window histogram, whose bin d
// holds the codes with key top - d: the first d at which the count from the
// top reaches K, and the count above it; d = kWin when the window holds fewer
// than K.  Wave 0 scans 16 bins per lane with a shuffle prefix over the
// lanes; one barrier publishes the result, after which the bins are cleared
// (the next use comes after another barrier).
__device__ __forceinline__ uint2 window_pick(LinesShared &sh, uint32_t *hist, uint32_t K, bool clear = true) {
    const int tid = threadIdx.x, lane = tid & (kWave - 1);
    if (wave_id() == 0) {
        uint32_t c[16];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const uint4 q = reinterpret_cast<const uint4 *>(hist)[4 * lane + j];
            c[4 * j] = q.x;
            c[4 * j + 1] = q.y;
            c[4 * j + 2] = q.z;
            c[4 * j + 3] = q.w;
        }
        uint32_t tot = 0u;
#pragma unroll
        for (int j = 0; j < 16; ++j) tot += c[j];
        uint32_t pre = tot;  // bins < 16 (lane + 1)
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
            const uint32_t t = __shfl_up(pre, d);
            if (lane >= d) pre += t;
        }
        const uint64_t hits = __ballot(pre >= K);
        if (hits == 0ull) {
            if (lane == 0) sh.digit = kWin;
        } else if (lane == static_cast<int>(__builtin_ctzll(hits))) {
            uint32_t acc = pre - tot;
            int hit = 16;
#pragma unroll
            for (int j = 0; j < 16; ++j) {
                if (hit == 16) {
                    if (acc + c[j] >= K) hit = j;
                    else acc += c[j];
                }
            }
            sh.digit = static_cast<uint32_t>(16 * lane + hit);
            sh.above = acc;
        }
    }
    __syncthreads();
    const uint2 r = make_uint2(sh.digit, sh.above);
    if (clear) reinterpret_cast<uint4 *>(hist)[tid] = make_uint4(0u, 0u, 0u, 0u);
    return r;
}

// The K-th largest of the codes whose top half is hi16 (fp32 rows), given
// `above` codes above them: two 8-bit digit passes over the codes that
// `visit(f)` hands to f.
template <typename VISIT>
__device__ __forceinline__ uint32_t refine_low16(LinesShared &sh, uint32_t hi16, uint32_t K, uint32_t above,
                                                 VISIT visit) {
    uint32_t prefix = hi16 << 16;
#pragma unroll
    for (int pass = 0; pass < 2; ++pass) {
        const int shift = 8 - 8 * pass;
        const uint32_t match = 0xffffffffu << (shift + 8);
        visit([&](uint32_t c) {
            if ((c & match) == prefix) atomicAdd(&sh.hist[pass][(c >> shift) & 0xffu], 1u);
        });
        __syncthreads();
        const uint3 r = pick_digit(sh, pass, K, above);
        prefix |= r.x << shift;
        above = r.y;
    }
    return prefix;
}

// Sums over the workgroup of 16 per-thread counters: wave DPP ladders on
// pairs packed in 16-bit halves (a wave counts at most 64 * 64 codes here),
// then the waves' rows in LDS behind one barrier (red alternates by `round`).
__device__ __forceinline__ void block_count16(const uint32_t (&cnt)[16], uint32_t (*red)[kLinesThreads / 64][16],
                                              int round, uint32_t (&tot)[16]) {
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const uint32_t s = wave_sum_u(cnt[2 * j] | (cnt[2 * j + 1] << 16));
        if (lane == 0) {
            red[round & 1][wave][2 * j] = s & 0xffffu;
            red[round & 1][wave][2 * j + 1] = s >> 16;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        uint32_t t = 0u;
#pragma unroll
        for (int w = 0; w < kLinesThreads / 64; ++w) t += red[round & 1][w][j];
        tot[j] = t;
    }
}

// The K-th largest (with multiplicity) of the codes that `visit(f)` hands
// to f over the workgroup (at most 64 per thread), known to lie in [lo, hi]
// with at least K codes >= lo: a 16-way search of the code interval, each
// round counting the codes at or above 15 pivots.  For rows whose K-th key
// lies below the window.
template <typename VISIT>
__device__ __forceinline__ uint32_t kth_largest(VISIT visit, uint32_t K, uint32_t lo, uint32_t hi,
                                                uint32_t (*red)[kLinesThreads / 64][16], int &round) {
    while (lo < hi) {
        const uint32_t step = (hi - lo) / 16u + 1u;  // 16 parts cover [lo, hi]
        uint32_t cnt[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) cnt[j] = 0u;
        visit([&](uint32_t c) {
#pragma unroll
            for (int j = 1; j < 16; ++j) cnt[j] += (c >= lo + uint32_t(j) * step) ? 1u : 0u;
        });
        uint32_t tot[16];
        block_count16(cnt, red, round++, tot);
        // the part holding the K-th largest: the last pivot with K codes at or above it
        uint32_t nlo = lo, nhi = hi;
#pragma unroll
        for (int j = 1; j < 16; ++j) {
            const uint64_t pj = uint64_t(lo) + uint64_t(j) * step;
            if (pj > hi) break;
            if (tot[j] >= K) nlo = static_cast<uint32_t>(pj);
            else {
                nhi = static_cast<uint32_t>(pj - 1);
                break;
            }
        }
        lo = nlo;
        hi = nhi;
    }
    return lo;
}

// Line `line` of a row (entry q * G + g of block c in the stored order) is
// group g's line of lanes 8q .. 8q + 7: its first token.
template <typename ET>
__device__ __forceinline__ int64_t line_token(int line) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    constexpr int LPB = G * 8;
    const int c = line / LPB, j = line % LPB;
    return int64_t(c) * kBlock + ((j % G) * kWave + (j / G) * 8) * P;
}

template <typename ET>
__device__ __forceinline__ uint32_t line_code(const LinesArgs &a, int64_t row, int line) {
    constexpr int LPB = (kBlock / (kWave * Logit<ET>::kPer16)) * 8;
    const int64_t idx = row * int64_t(a.C) * LPB + line;
    return sizeof(ET) == 2 ? uint32_t(reinterpret_cast<const uint16_t *>(a.linemax)[idx])
                           : reinterpret_cast<const uint32_t *>(a.linemax)[idx];
}

// Group h (of 8) of line `line` of a row: its 16 bytes of logits and its
// mask byte (all ones without a mask), zeros past V.  Group h holds the
// line's tokens h * P .. h * P + P - 1.
struct LineGroup {
    uint4 w;
    uint32_t bits;
    int64_t tok;
};

template <typename ET, bool MASKED>
__device__ __forceinline__ LineGroup load_line_group(const LinesArgs &a, int64_t row, int line, int h) {
    constexpr int P = Logit<ET>::kPer16;
    LineGroup g;
    g.tok = line_token<ET>(line) + h * P;
    g.w = make_uint4(0u, 0u, 0u, 0u);
    g.bits = 0u;
    if (g.tok < a.V) {
        g.w = *reinterpret_cast<const uint4 *>(reinterpret_cast<const ET *>(a.logits) + row * a.V + g.tok);
        g.bits = 0xffu;
        if (MASKED) {
            const uint32_t byte = reinterpret_cast<const uint8_t *>(a.mask + row * a.W)[g.tok >> 3];
            g.bits = (P == 8) ? byte : (byte >> (uint32_t(g.tok) & 4u));
        }
    }
    return g;
}

// The group's codes: 0 for masked, infinite and past-V tokens (bf16: the top
// half of the code).
template <typename ET>
__device__ __forceinline__ void group_codes(const LineGroup &g, uint32_t *code) {
    constexpr int P = Logit<ET>::kPer16;
    float v[P];
    Logit<ET>::unpack(g.w, v);
#pragma unroll
    for (int e = 0; e < P; ++e) {
        const bool live = ((g.bits >> e) & 1u) && v[e] > -INFINITY && v[e] < INFINITY;
        const uint32_t c = ordered_code(v[e]);
        code[e] = live ? (sizeof(ET) == 2 ? (c >> 16) : c) : 0u;
    }
}

template <typename ET, bool MASKED>
__device__ __forceinline__ void line_group_codes(const LinesArgs &a, int64_t row, int line, int h,
                                                 uint32_t *code) {
    group_codes<ET>(load_line_group<ET, MASKED>(a, row, line, h), code);
}

template <typename ET>
__device__ __forceinline__ float value_of_code(uint32_t c) {
    return sizeof(ET) == 2 ? bf16_value_of_digit(c) : float_of_code(c);
}

// Element e of a 16-byte vector of codes (8 x 16 bits or 4 x 32 bits).
template <typename CT>
__device__ __forceinline__ uint32_t code_in(const uint4 &q, int e) {
    const uint32_t w = e * int(sizeof(CT)) < 4 ? q.x : (e * int(sizeof(CT)) < 8 ? q.y : (e * int(sizeof(CT)) < 12 ? q.z : q.w));
    return sizeof(CT) == 2 ? ((w >> (16 * (e & 1))) & 0xffffu) : w;
}

// What the block statistics need beside the codes: the row's coordinates.
struct LinesRow {
    int64_t row;
    int b, i, x;   // request, position, valid draft of a draft row (-1: none)
    float cT;      // log2(e) / T
};

// tau from global memory by radix selection, for rows with more candidate
// lines than LDS holds: passes over the line codes and the candidate lines.
// Returns 0 when at most K allowed finite tokens exist.
template <typename ET, bool MASKED>
__device__ __forceinline__ uint32_t tau_code_global(const LinesArgs &a, LinesShared &sh, int64_t row, uint32_t L, uint32_t Ku) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int LPB = (kBlock / (kWave * P)) * 8;
    constexpr int BITS = sizeof(ET) == 2 ? 16 : 32;
    const int tid = threadIdx.x;
    const int nlines = a.C * LPB;
    uint32_t prefix = 0u, above = 0u;
    int hb = 0;
    for (int shift = BITS - 8; shift >= 0; shift -= 8, hb ^= 1) {
        const uint32_t hi_mask = shift + 8 >= 32 ? 0u : (0xffffffffu << (shift + 8));
        for (int l = tid >> 3; l < nlines; l += kLinesThreads / 8) {  // 8 threads per line
            if (line_code<ET>(a, row, l) < L) continue;
            uint32_t code[P];
            line_group_codes<ET, MASKED>(a, row, l, tid & 7, code);
#pragma unroll
            for (int e = 0; e < P; ++e)
                if (code[e] >= L && (code[e] & hi_mask) == (prefix & hi_mask))
                    atomicAdd(&sh.hist[hb][(code[e] >> shift) & 0xffu], 1u);
        }
        __syncthreads();
        const uint3 r = pick_digit(sh, hb, Ku, above);
        if (shift == BITS - 8 && r.z < Ku) return 0u;
        prefix |= r.x << shift;
        above = r.y;
    }
    return prefix;
}

// Block statistics over the kept tokens read from global memory (rows with
// more candidate lines than LDS holds): one wave per block, lane t on token t
// of each candidate line.
template <typename ET, bool MASKED>
__device__ __forceinline__ void block_stats_global(const LinesArgs &a, const LinesRow &r, uint32_t L, uint32_t tcode) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    constexpr int LPB = G * 8;
    constexpr int TPL = 8 * P;
    constexpr int NW = kLinesThreads / kWave;
    const int lane = threadIdx.x & (kWave - 1), wave = wave_id();
    const PhiloxKey key = key_of(a.seed);
    for (int c = wave; c < a.C; c += NW) {
        const uint64_t cl = __ballot(lane < LPB && line_code<ET>(a, r.row, c * LPB + lane) >= L);
        const bool has_x = r.x >= 0 && r.x / kBlock == c;
        BlockStat out{-INFINITY, 0.0f, -INFINITY};
        float sx = 0.0f;
        uint32_t mcode = 0u;
        for (uint64_t ll = cl; ll; ll &= ll - 1) {
            uint32_t code[P];
            const int l = static_cast<int>(__builtin_ctzll(ll));
            line_group_codes<ET, MASKED>(a, r.row, c * LPB + l, (lane & (TPL - 1)) / P, code);
            uint32_t cd = 0u;
#pragma unroll
            for (int q = 0; q < P; ++q)
                if (lane < TPL && lane % P == q) cd = code[q];
            if (cd >= tcode) mcode = max(mcode, cd);
        }
        mcode = wave_max_u(mcode);
        if (mcode != 0u) {
            const float mc = value_of_code<ET>(mcode) * r.cT;
            float sl = 0.0f, sxl = 0.0f;
            for (uint64_t ll = cl; ll; ll &= ll - 1) {
                uint32_t code[P];
                const int l = static_cast<int>(__builtin_ctzll(ll));
                line_group_codes<ET, MASKED>(a, r.row, c * LPB + l, (lane & (TPL - 1)) / P, code);
                uint32_t cd = 0u;
#pragma unroll
            for (int q = 0; q < P; ++q)
                if (lane < TPL && lane % P == q) cd = code[q];
                if (cd >= tcode) {
                    const float term = __builtin_amdgcn_exp2f(fmaf(value_of_code<ET>(cd), r.cT, -mc));
                    sl += term;
                    if (line_token<ET>(c * LPB + l) + lane != r.x) sxl += term;
                }
            }
            const float sum = wave_sum(sl);
            sx = wave_sum(sxl);
            out.m = mc;
            out.s = sum;
            if (lane == 0) {
                const double g = block_gumbel(key, r.b, r.i, c);
                out.key = key_of_mass(sum, mc, g);
                if (has_x) a.drec[r.row].keyx = key_of_mass(sx, mc, g);
            }
        } else if (has_x && lane == 0) {
            a.drec[r.row].keyx = -INFINITY;
        }
        if (lane == 0) {
            a.bstats[r.row * a.C + c] = out;
            if (has_x) a.drec[r.row].sx = sx;
        }
    }
}

// The candidate lines' staged tokens of the single-pass selection.
template <typename CT, int TPL>
struct LinesStage {
    __align__(16) CT tcodes[kCandLines * TPL];  // the candidate lines' token codes
    uint16_t cand[kCandLines];                  // the candidate lines, ascending
    uint32_t cmax[kCandLines];                  // each candidate's largest code
    float lsum[kCandLines];                     // each candidate's kept mass
};

// Top-p over the staged tokens at or above tcode (what top-k keeps), with the
// selection passes' definition and arithmetic: the largest code c whose tokens
// at or above it hold top_p of their tempered mass, masses 2^((l - M)
// log2(e) / T) in fp64 with M the row's largest logit (code lmax); ties at c
// stay.  Radix passes of 8 bits over the codes sum the masses per digit into
// `bins` (256 doubles); wave 0 picks the digit where the mass from the top
// reaches the target (a rounding shortfall takes the lowest nonempty digit).
// Returns the cut value and sets *flag as the passes do.  All threads call it.
template <typename ET, typename CT>
__device__ float topp_staged(const CT *tcodes, int ntok, uint32_t tcode, uint32_t lmax, float T, float top_p,
                             double *bins, double *red, uint32_t *flag) {
    constexpr int W = sizeof(ET) == 2 ? 16 : 32;
    constexpr int NW = kLinesThreads / kWave;
    static_assert(kLinesThreads == 256, "one bin per thread");
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    const double cd = kLog2e / static_cast<double>(T);
    const double mcd = static_cast<double>(value_of_code<ET>(lmax)) * cd;
    auto mass = [&](uint32_t c) {
        return exp2_precise_nonpos(fma(static_cast<double>(value_of_code<ET>(c)), cd, -mcd));
    };
    double own = 0.0;
    for (int t = tid; t < ntok; t += kLinesThreads) {
        const uint32_t c = tcodes[t];
        if (c >= tcode) own += mass(c);
    }
    own = wave_sum_d(own);
    if (lane == 0) red[wave] = own;
    __syncthreads();
    double total = 0.0;
#pragma unroll
    for (int q = 0; q < NW; ++q) total += red[q];
    const double target = static_cast<double>(top_p) * total;
    uint32_t prefix = 0u;
    double above = 0.0, at = 0.0;
    for (int shift = W - 8; shift >= 0; shift -= 8) {
        bins[tid] = 0.0;
        __syncthreads();
        for (int t = tid; t < ntok; t += kLinesThreads) {
            const uint32_t c = tcodes[t];
            if (c >= tcode && (shift == W - 8 || (c >> (shift + 8)) == prefix))
                atomicAdd(&bins[(c >> shift) & 0xffu], mass(c));
        }
        __syncthreads();
        if (wave == 0) {
            double b4[4], sl = 0.0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                b4[j] = bins[4 * lane + j];
                sl += b4[j];
            }
            double suf = sl;  // mass of digits 4 * lane and up
#pragma unroll
            for (int d = 1; d < kWave; d <<= 1) {
                const double o = __shfl_down(suf, d);
                if (lane + d < kWave) suf += o;
            }
            const uint64_t hit = __ballot(above + suf >= target);
            const uint64_t nonempty = __ballot(sl > 0.0);
            // the lane of the crossing (suf falls with the lane), else the
            // lowest nonempty lane
            const int pick = hit ? 63 - __builtin_clzll(hit) : __builtin_ctzll(nonempty);
            if (lane == pick) {
                double acc = above + (suf - sl);  // mass of the digits above this lane's
                int d = -1;
                if (hit) {
                    for (int j = 3; j >= 0; --j) {
                        if (acc + b4[j] >= target) {
                            d = j;
                            break;
                        }
                        acc += b4[j];
                    }
                }
                if (d < 0) {  // a rounding shortfall: the lowest nonempty digit of the lane
                    acc = above + (suf - sl);
                    int lowest = 3;
                    for (int j = 0; j < 4; ++j)
                        if (b4[j] > 0.0) {
                            lowest = j;
                            break;
                        }
                    for (int j = 3; j > lowest; --j) acc += b4[j];
                    d = lowest;
                }
                red[NW] = acc;
                red[NW + 1] = static_cast<double>(4 * lane + d);
                red[NW + 2] = b4[d];
            }
        }
        __syncthreads();
        above = red[NW];
        prefix = (prefix << 8) | static_cast<uint32_t>(red[NW + 1]);
        at = red[NW + 2];
        __syncthreads();  // red and bins are reused by the next pass
    }
    const double eps = kTopPFlagEps * total;
    const double at_cut = above + at;
    *flag = (fabs(at_cut - target) < eps || fabs(target - above) < eps) ? 1u : 0u;
    return value_of_code<ET>(prefix);
}

// Top-p over what top-k keeps, read off the staged tokens' window histogram
// (bf16 rows whose K-th largest lies in the window): bin d counts the kept
// tokens of code top - d, and a bf16 bin holds one value, so its mass is its
// count times that value's mass 2^((l - M) log2(e) / T) (fp64, the selection
// passes' arithmetic); top-k keeps bins 0..dk.  The cut is the first bin from
// the top at which the mass reaches top_p of the kept total, the owning
// thread's last kept bin on a rounding shortfall.  Returns the cut's code and
// sets *flag as the passes do.  All threads call it; hist is only read.
__device__ uint32_t topp_window_bf16(const uint32_t *hist, uint32_t dk, uint32_t top, float T, float top_p,
                                     double *red, uint32_t *flag) {
    constexpr int NW = kLinesThreads / kWave;
    static_assert(kWin == 4 * kLinesThreads, "four bins per thread");
    __shared__ uint32_t first[NW];
    __shared__ uint32_t dsel;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    const double cd = kLog2e / static_cast<double>(T);
    const double mcd = static_cast<double>(bf16_value_of_digit(top)) * cd;
    const uint4 q = reinterpret_cast<const uint4 *>(hist)[tid];
    const uint32_t n[4] = {q.x, q.y, q.z, q.w};
    double m[4], s = 0.0;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const uint32_t d = 4u * uint32_t(tid) + uint32_t(j);
        m[j] = (n[j] != 0u && d <= dk)
                   ? static_cast<double>(n[j]) *
                         exp2_precise_nonpos(fma(static_cast<double>(bf16_value_of_digit(top - d)), cd, -mcd))
                   : 0.0;
        s += m[j];
    }
    double pre = s;  // inclusive prefix over the threads (bins by descending value)
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const double t = __shfl_up(pre, o);
        if (lane >= o) pre += t;
    }
    if (lane == kWave - 1) red[wave] = pre;
    __syncthreads();
    double before = 0.0, total = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        const double t = red[w];
        if (w < wave) before += t;
        total += t;
    }
    pre += before;
    const double target = static_cast<double>(top_p) * total;
    const uint64_t hit = __ballot(pre >= target);
    if (lane == 0) first[wave] = hit ? static_cast<uint32_t>(__builtin_ctzll(hit)) : uint32_t(kWave);
    __syncthreads();
    int owner = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w)
        if (owner < 0 && first[w] < uint32_t(kWave)) owner = w * kWave + static_cast<int>(first[w]);
    if (tid == (owner >= 0 ? owner : static_cast<int>(dk / 4u))) {
        double acc = pre - s, at = 0.0;
        int pick = -1;
        if (owner >= 0) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (pick < 0 && m[j] > 0.0) {
                    if (acc + m[j] >= target) {
                        pick = j;
                        at = m[j];
                    } else {
                        acc += m[j];
                    }
                }
            }
        }
        if (pick < 0) {  // a rounding shortfall: this thread's last kept bin
            acc = pre - s;
#pragma unroll
            for (int j = 0; j < 4; ++j)
                if (n[j] != 0u && 4u * uint32_t(tid) + uint32_t(j) <= dk) pick = j;
            if (pick < 0) pick = 0;
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                if (j < pick) acc += m[j];
                if (j == pick) at = m[j];
            }
        }
        red[NW] = acc;
        red[NW + 1] = at;
        dsel = 4u * uint32_t(tid) + uint32_t(pick);
    }
    __syncthreads();
    const double above = red[NW], at = red[NW + 1];
    const uint32_t d = dsel;
    const double eps = kTopPFlagEps * total;
    *flag = (fabs(above + at - target) < eps || fabs(target - above) < eps) ? 1u : 0u;
    __syncthreads();  // red, first and dsel are reused
    return top - d;
}

// A bf16 or fp32 value's code as the line maxima hold it, and the 32-bit
// order-preserving code of a line maximum.
template <typename ET>
__device__ __forceinline__ uint32_t line_code_of(float v) {
    return sizeof(ET) == 2 ? ordered_code(v) >> 16 : ordered_code(v);
}

template <typename ET>
__device__ __forceinline__ uint32_t code32_of_line(uint32_t c) {
    return sizeof(ET) == 2 ? ((c << 16) | ((c & 0x8000u) ? 0u : 0xffffu)) : c;
}

// TOPP: requests with top-p too (pyshine "vLLM, part 2", "Verification": the
// sampling constraints before the accept test): the cut over what top-k keeps,
// from the staged candidate tokens when every candidate line is staged, else
// by passes over the row; rows of requests with top-p alone (top-k 0) take the
// passes and their block statistics from global memory.
template <typename ET, bool MASKED, bool TOPP>
__global__ __launch_bounds__(kLinesThreads) __attribute__((amdgpu_waves_per_eu(6))) void topk_lines_kernel(LinesArgs a) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    constexpr int LPB = G * 8;            // lines per block
    constexpr int TPL = 8 * P;            // tokens per line
    constexpr int NW = kLinesThreads / kWave;
    constexpr bool BF = sizeof(ET) == 2;
    constexpr int KS = BF ? 0 : 16;       // key = code >> KS
    typedef typename std::conditional<BF, uint16_t, uint32_t>::type CT;
    constexpr int PER4 = 16 / int(sizeof(CT));                 // codes per 16-byte vector
    constexpr int NV4 = kLinesMax / kLinesThreads / PER4;      // vectors of line codes per thread
    constexpr int CPT = NV4 * PER4;                            // lines per thread, contiguous
    constexpr int NB = kLinesMax / 32;                         // blocks at most
    __shared__ LinesShared sh;
    __shared__ uint32_t red[2][NW][16];
    __shared__ __align__(16) uint32_t hist[kWin];
    // the staged candidates; calls with top-p lay the passes' bins over them
    // (the passes run only where nothing is staged)
    typedef LinesStage<CT, TPL> Stage;
    union StageOrPasses {
        Stage st;
        ToppShared tp;
    };
    __shared__ typename std::conditional<TOPP, StageOrPasses, Stage>::type staged;
    __shared__ double pred[NW + 3];                           // top-p's reductions
    CT *tcodes = reinterpret_cast<Stage &>(staged).tcodes;
    uint16_t *cand = reinterpret_cast<Stage &>(staged).cand;
    uint32_t *cmax = reinterpret_cast<Stage &>(staged).cmax;
    float *lsum = reinterpret_cast<Stage &>(staged).lsum;
    __shared__ uint32_t bmax[NB];                              // each block's largest kept code
    __shared__ uint8_t brun[NB][2];                            // each block's run of candidates
    __shared__ float xmass;                                    // the draft line's kept mass without it
    const int64_t row = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    if (a.off && uniform_load(a.off_ok) == 0u) return;  // malformed ragged call
    int b, i, kb;
    int64_t d0;
    row_owner(a.off, a.row_req, static_cast<int>(row), a.kp1, b, i, kb, d0);
    const int nlines = a.C * LPB;  // at most kLinesMax (the host checks)
    const int nv = nlines / PER4;
    // ---- 1. the row's line codes, lines tid * CPT .. + CPT - 1 per thread,
    // issued before the request's settings are known
    uint4 w[NV4];
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(static_cast<const CT *>(a.linemax) + row * nlines);
#pragma unroll
        for (int j = 0; j < NV4; ++j) {
            const int q = tid * NV4 + j;
            w[j] = q < nv ? src[q] : make_uint4(0u, 0u, 0u, 0u);
        }
    }
    const float T = uniform_load(a.temperature + b);
    const int K = uniform_load(a.top_k + b);
    const float Pp = TOPP ? uniform_load(a.top_p + b) : 0.0f;
    const bool use_p = TOPP && Pp > 0.0f && Pp < 1.0f;
    // the row is not cut unless a cut is found below, and its kept tokens are
    // not listed unless the staged path lists them
    if (tid == 0) {
        a.tau[row] = -INFINITY;
        a.tau_flag[row] = 0u;
        if (a.kcount) a.kcount[row] = kNoLineList;
    }
    if (!(T > 0.0f && T <= FLT_MAX) || (K <= 0 && !use_p)) return;
    const BlockStat *st = a.bstats + row * a.C;
    bool bad = false;
    if (tid < a.C) {  // C <= NB < kLinesThreads: thread c takes block c
        const BlockStat e = st[tid];
        bad = (e.m != e.m) | (e.s != e.s) | (e.m == INFINITY);
    }
    // block tid's level-1 Gumbel variate, drawn while the loads are in flight
    const double gum = tid < a.C ? block_gumbel(key_of(a.seed), b, i, tid) : 0.0;
    uint32_t mx = 0u, nz = 0u;
#pragma unroll
    for (int j = 0; j < NV4; ++j)
#pragma unroll
        for (int e = 0; e < PER4; ++e) {
            const uint32_t c = code_in<CT>(w[j], e);
            mx = max(mx, c);
            nz += c != 0u ? 1u : 0u;
        }
    reinterpret_cast<uint4 *>(hist)[tid] = make_uint4(0u, 0u, 0u, 0u);
    sh.hist[0][tid] = 0u;
    sh.hist[1][tid] = 0u;
    if (tid < NB) {
        bmax[tid] = 0u;
        brun[tid][0] = brun[tid][1] = 0;
    }
    mx = wave_max_u(mx);
    nz = wave_sum_u(nz);
    const bool wbad = wave_any(bad);
    if (lane == 0) {
        red[0][wave][0] = mx;
        red[0][wave][1] = nz;
        red[0][wave][2] = wbad ? 1u : 0u;
    }
    __syncthreads();
    uint32_t lmax = 0u, lnz = 0u, anybad = 0u;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
        lmax = max(lmax, red[0][q][0]);
        lnz += red[0][q][1];
        anybad |= red[0][q][2];
    }
    // bad rows keep the sweep's marks, which report them; rows without an
    // allowed finite token keep its (-inf, 0), which report them too
    if (anybad || lnz == 0u) return;
    LinesRow r;
    r.row = row;
    r.b = b;
    r.i = i;
    r.x = -1;
    if (i < kb) {
        const int xv = uniform_load(a.draft + d0 + i);
        if (xv >= 0 && xv < a.V) r.x = xv;
    }
    r.cT = scale_of(T);
    // the top-p cut over the tokens at or above tau_k (passes over the row)
    auto topp_passes = [&](float tauk, uint32_t *flag) -> float {
        if constexpr (TOPP) {
            const TopkRow<ET, true, MASKED> tr = topk_row<ET, true, MASKED>(a.logits, a.mask, row, a.V, a.W);
            return select_top_p<ET, true, MASKED>(tr, reinterpret_cast<ToppShared &>(staged), tauk,
                                                  code32_of_line<ET>(lmax), true, Pp, T, flag);
        } else {
            return tauk;
        }
    };
    if (TOPP && K <= 0) {
        // top-p alone: the cut from passes over the row, then the row's block
        // statistics over the tokens it keeps (the sweep recorded line maxima)
        uint32_t flag = 0u;
        const float tp = topp_passes(-INFINITY, &flag);
        const bool cutp = tp > -INFINITY;
        block_stats_global<ET, MASKED>(a, r, 1u, cutp ? line_code_of<ET>(tp) : 1u);
        if (tid == 0) {
            a.tau_flag[row] = flag;
            if (cutp) {
                a.tau[row] = tp;
                if (r.x >= 0 && !(a.drec[row].lx >= tp)) a.drec[row].lx = -INFINITY;
            }
        }
        return;
    }
    const uint32_t Ku = static_cast<uint32_t>(K);
    const uint32_t top = lmax >> KS;  // the window's first key
    int round = 1;
    auto visit_lines = [&](auto f) {
#pragma unroll
        for (int j = 0; j < NV4; ++j)
#pragma unroll
            for (int e = 0; e < PER4; ++e) f(code_in<CT>(w[j], e));
    };
    // ---- 2. L: the K-th largest line code (every nonempty line when fewer)
    uint32_t L = 1u;
    if (lnz >= Ku) {
        visit_lines([&](uint32_t c) {
            const uint32_t d = top - (c >> KS);
            if (c != 0u && d < uint32_t(kWin)) atomicAdd(&hist[d], 1u);
        });
        __syncthreads();
        const uint2 pk = window_pick(sh, hist, Ku);
        if (pk.x < uint32_t(kWin)) {
            if constexpr (BF) L = top - pk.x;
            else L = refine_low16(sh, top - pk.x, Ku, pk.y, visit_lines);
        } else {
            L = kth_largest(visit_lines, Ku, 1u, lmax, red, round);
        }
    }
    // ---- 3. the candidate lines (code >= L), listed in ascending order
    uint32_t mine = 0u;
    visit_lines([&](uint32_t c) { mine += c >= L ? 1u : 0u; });
    const uint32_t incl = wave_prefix_u(mine);
    if (lane == kWave - 1) red[round & 1][wave][0] = incl;
    __syncthreads();
    uint32_t pos = incl - mine, ncand = 0u;
#pragma unroll
    for (int q = 0; q < NW; ++q) {
        const uint32_t t = red[round & 1][q][0];
        pos += q < wave ? t : 0u;
        ncand += t;
    }
    ++round;
#pragma unroll
    for (int j = 0; j < NV4; ++j)
#pragma unroll
        for (int e = 0; e < PER4; ++e) {
            const uint32_t c = code_in<CT>(w[j], e);
            if (c >= L) {
                if (pos < uint32_t(kCandLines)) {
                    cand[pos] = static_cast<uint16_t>(tid * CPT + j * PER4 + e);
                    cmax[pos] = c;
                }
                ++pos;
            }
        }
    __syncthreads();
    uint32_t tcode;
    bool cut;
    if (ncand <= uint32_t(kCandLines)) {
        // ---- 4. the candidates' tokens into LDS, counted in the window
        uint32_t tn = 0u;
        auto take = [&](const LineGroup &lg, uint32_t e) {
            uint32_t code[P];
            group_codes<ET>(lg, code);
            uint4 ov;
            if constexpr (BF) {
                ov = make_uint4(code[0] | (code[1 % P] << 16), code[2 % P] | (code[3 % P] << 16),
                                code[4 % P] | (code[5 % P] << 16), code[6 % P] | (code[7 % P] << 16));
            } else {
                ov = make_uint4(code[0], code[1 % P], code[2 % P], code[3 % P]);
            }
            reinterpret_cast<uint4 *>(tcodes)[e] = ov;
#pragma unroll
            for (int q = 0; q < P; ++q) {
                if (code[q] >= L) {
                    ++tn;
                    const uint32_t d = top - (code[q] >> KS);
                    if (d < uint32_t(kWin)) atomicAdd(&hist[d], 1u);
                }
            }
        };
        // two groups in flight per thread
        const uint32_t ng = ncand * 8u;
        for (uint32_t e = tid; e < ng; e += 2 * kLinesThreads) {
            const uint32_t e2 = e + kLinesThreads;
            const LineGroup g1 = load_line_group<ET, MASKED>(a, row, cand[e >> 3], e & 7u);
            LineGroup g2;
            if (e2 < ng) g2 = load_line_group<ET, MASKED>(a, row, cand[e2 >> 3], e2 & 7u);
            take(g1, e);
            if (e2 < ng) take(g2, e2);
        }
        tn = wave_sum_u(tn);
        if (lane == 0) red[round & 1][wave][0] = tn;
        __syncthreads();
        uint32_t ttot = 0u;
#pragma unroll
        for (int q = 0; q < NW; ++q) ttot += red[round & 1][q][0];
        ++round;
        cut = ttot >= Ku;
        // ---- tau: the K-th largest candidate token at or above L.  With at
        // most K allowed finite tokens there is no cut: every candidate line
        // was taken (L = 1) and every allowed finite token is kept.
        const int ntok = static_cast<int>(ncand) * TPL;
        auto visit_tokens = [&](auto f) {
            for (int t = tid; t < ntok; t += kLinesThreads) {
                const uint32_t c = tcodes[t];
                if (c >= L) f(c);
            }
        };
        if (!cut) {
            tcode = 1u;
        } else {
            // with top-p on bf16 rows the counts stay for its cut
            const uint2 pk = window_pick(sh, hist, Ku, !(BF && use_p));
            if (pk.x < uint32_t(kWin)) {
                if constexpr (BF) tcode = top - pk.x;
                else tcode = refine_low16(sh, top - pk.x, Ku, pk.y, visit_tokens);
            } else {
                tcode = kth_largest(visit_tokens, Ku, L, lmax, red, round);
            }
        }
        if (use_p) {
            // ---- top-p over what top-k keeps: from the window histogram's
            // counts when the cut lies in it (bf16), else over the staged
            // tokens (the histogram's bins then hold their masses)
            const float tauk = cut ? value_of_code<ET>(tcode) : -INFINITY;
            uint32_t flag = 0u;
            float tp;
            if (BF && cut && top - tcode < uint32_t(kWin))
                tp = value_of_code<ET>(topp_window_bf16(hist, top - tcode, top, T, Pp, pred, &flag));
            else
                tp = topp_staged<ET, CT>(tcodes, ntok, tcode, lmax, T, Pp, reinterpret_cast<double *>(hist),
                                         pred, &flag);
            if (tid == 0) a.tau_flag[row] = flag;
            if (tp > tauk) {
                tcode = line_code_of<ET>(tp);
                cut = true;
            }
        }
        // ---- 5. the row's block statistics over the kept tokens: each
        // block's run of candidates and largest kept code, each candidate's
        // kept mass with a wave on its tokens, each block's sum over its run
        for (uint32_t s = tid; s < ncand; s += kLinesThreads) {
            const int c = cand[s] / LPB;
            if (s == 0u || cand[s - 1] / LPB != c) brun[c][0] = static_cast<uint8_t>(s);
            if (s + 1u == ncand || cand[s + 1] / LPB != c) brun[c][1] = static_cast<uint8_t>(s + 1u);
            if (cmax[s] >= tcode) atomicMax(&bmax[c], cmax[s]);
        }
        int xline = -1;  // the draft's line
        if (r.x >= 0) {
            const int o = r.x % kBlock;
            xline = (r.x / kBlock) * LPB + ((o % (kWave * P)) / P / 8) * G + o / (kWave * P);
        }
        __syncthreads();
        // four candidates per wave at a time (independent reductions)
        for (uint32_t s0 = wave; s0 < ncand; s0 += 4 * NW) {
            float term[4], ls[4];
            int line[4];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                const uint32_t s = s0 + u * NW;
                line[u] = s < ncand ? int(cand[s]) : -1;
                const uint32_t mk = line[u] >= 0 ? bmax[line[u] / LPB] : 0u;
                const float mc = value_of_code<ET>(mk) * r.cT;
                const uint32_t cd = (mk != 0u && lane < TPL) ? uint32_t(tcodes[s * TPL + lane]) : 0u;
                term[u] = cd >= tcode ? __builtin_amdgcn_exp2f(fmaf(value_of_code<ET>(cd), r.cT, -mc)) : 0.0f;
            }
#pragma unroll
            for (int u = 0; u < 4; ++u) ls[u] = wave_sum(term[u]);
#pragma unroll
            for (int u = 0; u < 4; ++u) {
                if (line[u] < 0) continue;
                if (lane == 0) lsum[s0 + u * NW] = ls[u];
                if (line[u] == xline) {
                    const float lx = wave_sum(line_token<ET>(line[u]) + lane != r.x ? term[u] : 0.0f);
                    if (lane == 0) xmass = lx;
                }
            }
        }
        __syncthreads();
        for (int c = tid; c < a.C; c += kLinesThreads) {
            const uint32_t mk = bmax[c];
            const bool has_x = r.x >= 0 && r.x / kBlock == c;
            BlockStat out{-INFINITY, 0.0f, -INFINITY};
            float sx = 0.0f;
            if (mk != 0u) {
                const float mc = value_of_code<ET>(mk) * r.cT;
                float sum = 0.0f;
                for (int s = brun[c][0]; s < brun[c][1]; ++s) {
                    const float ls = lsum[s];
                    sum += ls;
                    sx += cand[s] == xline ? xmass : ls;
                }
                out.m = mc;
                out.s = sum;
                out.key = key_of_mass(sum, mc, gum);  // c == tid
                if (has_x) a.drec[r.row].keyx = key_of_mass(sx, mc, gum);
            } else if (has_x) {
                a.drec[r.row].keyx = -INFINITY;
            }
            a.bstats[r.row * a.C + c] = out;
            if (has_x) a.drec[r.row].sx = sx;
        }
        // ---- 6. the lines holding a kept token, ascending (dense q): a
        // residual max(p - q, 0) drawn from this row is zero elsewhere
        if (a.kcount != nullptr && wave < 2) {  // ncand <= 128: two waves cover the candidates
            const auto kept = [&](int s) { return s < int(ncand) && cmax[s] >= tcode; };
            const uint64_t b0 = __ballot(kept(lane)), b1 = __ballot(kept(kWave + lane));
            const int s = wave * kWave + lane;
            const uint64_t bw = wave == 0 ? b0 : b1;
            const uint32_t pos = (wave == 0 ? 0u : uint32_t(__popcll(b0))) +
                                 uint32_t(__popcll(bw & ((1ull << lane) - 1ull)));
            if (kept(s)) a.klist[row * kCandLines + pos] = cand[s];
            if (tid == 0) a.kcount[row] = uint32_t(__popcll(b0) + __popcll(b1));
        }
    } else {
        tcode = tau_code_global<ET, MASKED>(a, sh, row, L, Ku);
        cut = tcode != 0u;
        if (!cut) tcode = 1u;  // no cut: every allowed finite token (then L = 1)
        if (use_p) {
            const float tauk = cut ? value_of_code<ET>(tcode) : -INFINITY;
            uint32_t flag = 0u;
            const float tp = topp_passes(tauk, &flag);
            if (tid == 0) a.tau_flag[row] = flag;
            if (tp > tauk) {
                tcode = line_code_of<ET>(tp);
                cut = true;
            }
        }
        block_stats_global<ET, MASKED>(a, r, L, tcode);
    }
    if (tid == 0 && cut) {
        const float tau = value_of_code<ET>(tcode);
        a.tau[row] = tau;
        if (r.x >= 0 && !(a.drec[row].lx >= tau)) a.drec[row].lx = -INFINITY;
    }
}

// ------------------------------------------------------------------ finalize

struct Level1 {
    int c;     // winning block, -1 when no block has mass
    int flag;  // 1 when the top-2 block keys are closer than the flag threshold
};

// A request whose draw comes from the dense residual max(p - q, 0): the
// finalize kernel leaves it to the residual-mass and residual-draw kernels.
struct DenseJob {
    double S;      // the row's sum of 2^(l c - M) over the support
    double invT;   // 1 / T in fp64
    float c, M;    // log2(e) / T and the row's fp32 max (log2 units)
    float tau;     // the row's top-k threshold (-inf: none)
    int64_t dpos;  // the rejected draft's index (its q row)
    int row;       // the rejected row (and output slot), or -1: no dense draw
    int n;         // the rejected position
    Level1 l1p;    // level-1 winner under p, for the fallback
};

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
    unsigned long long *tally;  // nslot slot words
    int nslot;
    double *dbg_lse;
    double *dbg_acc;
    uint32_t *dbg_req_flags;
    uint32_t *dbg_flags;
    uint32_t *status;
    const BlockStat *bstats;
    const DraftRec *drec;
    const float *tau;  // [rows] top-k / top-p thresholds, or nullptr
    const uint32_t *tau_flag;  // [rows] top-p boundary rows (with tau)
    DenseJob *jobs;    // [B] dense q only
    double *wmass;     // [B, C] dense q only: residual mass per block
    int split_dense;   // dense q: 1 = residual masses by the grid-wide kernels
    const uint16_t *klist;   // dense q after the single-pass selection: [rows, kCandLines], or nullptr
    const uint32_t *kcount;  // [rows]: listed lines, kNoLineList when a row's are not listed
    const int32_t *off;      // ragged: [B + 1] draft offsets, or nullptr
    const uint32_t *off_ok;  // ragged: 1 when the offsets are consistent
    uint32_t *sweep;         // the row-statistics sweep's claim counters, reset here
    int B, k, V, W, C;       // k: the uniform draft count, or the largest k_b
};

enum SampleMode { kModeP = 0, kModeOneHot = 1, kModeDense = 2 };

struct FinalShared {
    float M[kMaxDraft + 1];     // per row: fp32 max (log2 units), or greedy max logit
    double S[kMaxDraft + 1];    // per row: sum of 2^(t - M)
    int G[kMaxDraft + 1];       // greedy argmax
    Level1 l1p[kMaxDraft + 1];  // level-1 winner under p
    Level1 l1x[kMaxDraft + 1];  // level-1 winner under p without the row's draft
    int X[kMaxDraft];
    double acc[kMaxDraft];
    unsigned char ok[kMaxDraft], flag[kMaxDraft], invalid[kMaxDraft], badq[kMaxDraft];
    unsigned char rowst[kMaxDraft + 1];  // per row: SD_STATUS_* bits found by its wave
    int staged_c;               // block of the sampled row held in blockv (-1: none)
    uint4 race[2][kFinalWaves];  // per-wave level-2 results (best, index, runner-up), by attempt
    float blockv[kBlock];       // that block's logits, -inf where masked or past V
};

// Gumbel keys are compared in fp32 relative to a per-row constant, where
// they stay within 3e-6 of their exact values; as order-preserving codes
// (wave.h) a maximum finds the winner, lowest index on ties, and a second
// pass or the runner-up finds whether another key lies within the near-tie
// threshold.
constexpr float kTieEps = static_cast<float>(kGumbelFlagEps);

__device__ __forceinline__ bool near_tie(float key, int idx, uint64_t best) {
    return idx != packed_index(best) && key >= packed_key(best) - kTieEps;
}

// The level-1 winner in fp64.  The race runs on keys rounded to fp32
// (relative keys below 32 in magnitude round to within 2^-20), so its winner
// w is the fp64 winner unless another key lies within the two roundings of
// w's.  Lanes count their keys within kRaceSlack of w's fp32 key; when any
// key but w's is that close (rare), the race is run again on the fp64 keys
// kd (lowest block on ties), lane + 64 j for entry j, -inf where absent.
constexpr float kRaceSlack = 0x1p-18f;

template <int NJ>
__device__ __forceinline__ uint64_t race_in_fp64(uint64_t w, const double (&kd)[NJ]) {
    if (w == 0) return w;
    const int lane = threadIdx.x & (kWave - 1);
    const float wk = packed_key(w);
    int close = 0;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        close += (kd[j] > -INFINITY && static_cast<float>(kd[j]) >= wk - kRaceSlack) ? 1 : 0;
    if (!wave_any(close > 1) && __popcll(__ballot(close > 0)) <= 1) return w;
    double best = -INFINITY;
    int bi = INT_MAX;
#pragma unroll
    for (int j = 0; j < NJ; ++j)
        if (kd[j] > best) {  // j ascending: the lane's lowest block among equal keys
            best = kd[j];
            bi = lane + kWave * j;
        }
    const double m = wave_max_d(best);
    const int i = wave_min_i((m > -INFINITY && best == m) ? bi : INT_MAX);
    return pack_code(ordered_code(static_cast<float>(m)), i);
}

// Residual masses W_c = sum_j max(p_j - q_j, 0) of one row for dense q, with
// p_j = 2^(l_j c - M) / S in fp32.  One wave per block, two blocks of a wave
// in flight together; clamped loads.
template <typename ET, bool ALIGNED>
struct DenseSlab {  // one wave's share of a block: P logits and P q values per group
    static constexpr int P = Logit<ET>::kPer16;
    static constexpr int G = kBlock / (kWave * P);
    float lv[G][P], qv[G][P];

    __device__ __forceinline__ void load(const ET *rowp, const float *qrow, int V, int blk, int lane) {
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t tok = int64_t(blk) * kBlock + (g * kWave + lane) * P;
            if (ALIGNED) {
                const int64_t tc = tok < V ? tok : int64_t(V - P);
                Logit<ET>::unpack(*reinterpret_cast<const uint4 *>(rowp + tc), lv[g]);
#pragma unroll
                for (int h = 0; h < P / 4; ++h) {
                    const float4 f = *reinterpret_cast<const float4 *>(qrow + tc + 4 * h);
                    qv[g][4 * h] = f.x;
                    qv[g][4 * h + 1] = f.y;
                    qv[g][4 * h + 2] = f.z;
                    qv[g][4 * h + 3] = f.w;
                }
            } else {
#pragma unroll
                for (int e = 0; e < P; ++e) {
                    const int64_t tc = tok + e < V ? tok + e : int64_t(V - 1);
                    lv[g][e] = Logit<ET>::to_float(rowp[tc]);
                    qv[g][e] = qrow[tc];
                }
            }
        }
    }

    __device__ __forceinline__ double mass(const uint8_t *mb, int V, int blk, int lane, float c, float M,
                                           float invS, float tau) const {
        float acc = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t tok = int64_t(blk) * kBlock + (g * kWave + lane) * P;
#pragma unroll
            for (int e = 0; e < P; ++e) {
                const int64_t j = tok + e;
                const int64_t jc = j < V ? j : int64_t(V - 1);
                bool live = j < V && lv[g][e] > -INFINITY && !(lv[g][e] < tau);
                if (mb) live = live && ((mb[jc >> 3] >> (jc & 7)) & 1u);
                const float p = live ? __builtin_amdgcn_exp2f(fmaf(lv[g][e], c, -M)) * invS : 0.0f;
                acc += live ? fmaxf(p - qv[g][e], 0.0f) : 0.0f;
            }
        }
        return wave_sum_d(static_cast<double>(acc));
    }
};

// Residual masses W_c of a row from its lines (128-byte runs of the sweep's
// lane order, 8 groups of P tokens): with a list (the single-pass
// selection's lines holding a kept token, nl of them) only those lines, since
// max(p - q, 0) is zero wherever p is and every other block's W_c is zero;
// without one (nl = kNoLineList) every line of the row, kResLines at a time
// (a chunk covers whole blocks).  Eight threads take a line, P tokens each
// (a chunk's loads all in flight at once, four groups per thread); each sums
// its tokens in fp32 and the line's eight sums meet in fp64.  Each block adds
// its lines in order: a listed block's run by one thread, a whole block by a
// wave (its fixed reduction order).  lsum: kResLines doubles, lline:
// kResLines ints of LDS.  All threads call it; rows are 16-byte aligned (the
// single pass takes no others).
template <typename ET>
__device__ void line_block_masses(const FinalArgs &a, int64_t row, const float *qrow, uint32_t nl, float c,
                                  float M, double S, float tau, double *Wout, double *lsum, int *lline) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int LPB = (kBlock / (kWave * P)) * 8;
    constexpr int U = kResLines * 8 / kFinalThreads;  // line groups per thread
    static_assert(kCandLines <= kResLines, "a list fits one chunk");
    static_assert(kResLines % LPB == 0 && kResLines / LPB <= kFinalWaves, "a chunk is whole blocks, a wave each");
    const int tid = threadIdx.x, C = a.C, V = a.V;
    const float invS = static_cast<float>(1.0 / S);
    const ET *rowp = reinterpret_cast<const ET *>(a.logits) + row * V;
    const uint8_t *mb = a.mask ? reinterpret_cast<const uint8_t *>(a.mask + row * a.W) : nullptr;
    const bool listed = nl != kNoLineList;
    const uint16_t *list = a.klist + row * kCandLines;
    const int total = listed ? int(nl) : C * LPB;
    for (int cb = tid; cb < C; cb += kFinalThreads) Wout[cb] = 0.0;
    if (total == 0) lds_barrier();  // (each chunk ends with one)
    for (int base = 0; base < total; base += kResLines) {
        const int n = min(kResLines, total - base);  // lines of this chunk
        int line[U];
        bool has[U];
        uint4 lw[U];
        float qv[U][P];
        uint32_t bits[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int t = tid + u * kFinalThreads;
            has[u] = t < n * 8;
            line[u] = !has[u] ? 0 : (listed ? int(list[t >> 3]) : base + (t >> 3));
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int64_t tok = line_token<ET>(line[u]) + ((tid + u * kFinalThreads) & 7) * P;
            has[u] = has[u] && tok < V;
            lw[u] = make_uint4(0u, 0u, 0u, 0u);
            bits[u] = 0u;
#pragma unroll
            for (int e = 0; e < P; ++e) qv[u][e] = 0.0f;
            if (has[u]) {
                lw[u] = *reinterpret_cast<const uint4 *>(rowp + tok);
#pragma unroll
                for (int h = 0; h < P / 4; ++h) {
                    const float4 f = *reinterpret_cast<const float4 *>(qrow + tok + 4 * h);
                    qv[u][4 * h] = f.x;
                    qv[u][4 * h + 1] = f.y;
                    qv[u][4 * h + 2] = f.z;
                    qv[u][4 * h + 3] = f.w;
                }
                bits[u] = 0xffu;
                if (mb != nullptr) {
                    const uint32_t byte = mb[tok >> 3];
                    bits[u] = (P == 8) ? byte : (byte >> (uint32_t(tok) & 4u));
                }
            }
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            float lv[P];
            Logit<ET>::unpack(lw[u], lv);
            float acc = 0.0f;
#pragma unroll
            for (int e = 0; e < P; ++e) {
                const bool live = ((bits[u] >> e) & 1u) && lv[e] > -INFINITY && !(lv[e] < tau);
                const float p = live ? __builtin_amdgcn_exp2f(fmaf(lv[e], c, -M)) * invS : 0.0f;
                acc += live ? fmaxf(p - qv[u][e], 0.0f) : 0.0f;
            }
            double d = static_cast<double>(acc);  // the line's eight sums, lanes 8j .. 8j + 7
            d += __shfl_xor(d, 1);
            d += __shfl_xor(d, 2);
            d += __shfl_xor(d, 4);
            const int t = tid + u * kFinalThreads;
            if ((t & 7) == 0 && t < n * 8) {
                lsum[t >> 3] = d;
                lline[t >> 3] = line[u];
            }
        }
        lds_barrier();
        if (listed) {
            // each block's run of lines, summed in order by the thread at its start
            for (int i = tid; i < n; i += kFinalThreads) {
                const int cb = lline[i] / LPB;
                if (i == 0 || lline[i - 1] / LPB != cb) {
                    double w = 0.0;
                    for (int j = i; j < n && lline[j] / LPB == cb; ++j) w += lsum[j];
                    Wout[cb] = w;
                }
            }
        } else {
            // whole blocks (n is a multiple of LPB): block w of the chunk by wave w
            const int wave = wave_id(), lane = tid & (kWave - 1);
            if (wave * LPB < n) {
                const double w = wave_sum_d(lane < LPB ? lsum[wave * LPB + lane] : 0.0);
                if (lane == 0) Wout[(base + wave * LPB) / LPB] = w;
            }
        }
        lds_barrier();  // lsum and lline are reused by the next chunk
    }
}

template <typename ET, bool ALIGNED>
__device__ void dense_block_masses(const ET *rowp, const uint32_t *mrow, const float *qrow, int V,
                                   int C, float c, float M, double S, float tau, double *Wout) {
    const int lane = threadIdx.x & (kWave - 1);
    const float invS = static_cast<float>(1.0 / S);
    const uint8_t *mb = reinterpret_cast<const uint8_t *>(mrow);
    for (int blk = wave_id(); blk < C; blk += 2 * kFinalWaves) {
        const int blk2 = blk + kFinalWaves;
        const bool two = blk2 < C;
        DenseSlab<ET, ALIGNED> x, y;
        x.load(rowp, qrow, V, blk, lane);
        y.load(rowp, qrow, V, two ? blk2 : blk, lane);  // a repeat of blk is loaded but not summed
        const double wx = x.mass(mb, V, blk, lane, c, M, invS, tau);
        if (lane == 0) Wout[blk] = wx;
        if (two) {
            const double wy = y.mass(mb, V, blk2, lane, c, M, invS, tau);
            if (lane == 0) Wout[blk2] = wy;
        }
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

// ln x for positive x from the hardware base-2 logarithm of its fp32
// mantissa in [0.5, 1), where that logarithm is accurate to about 1e-7
// absolute: within about 1e-7 of ln x plus the rounding of x to fp32.
// Arguments below the fp32 range give -inf.
// The winner of a level-2 race over a workgroup of NW waves, and whether it
// is a near tie.  Thread t holds the codes (ordered_code of the key, 0 = no
// candidate) of indices base + 4t .. base + 4t + 3, so indices ascend with
// the thread and the slot.  Each wave finds its largest code (the lowest
// index on equal codes) and the largest code among its other candidates;
// the waves' triples meet in `scratch` after one barrier (consecutive races
// use different scratch, so none is needed between them).  Returns (index,
// near-tie flag), index -1 when no thread has a candidate.
template <int NW>
__device__ __forceinline__ int2 race_winner(const uint32_t (&code)[4], int base, uint4 *scratch) {
    uint32_t lm = code[0];
    int le = 0;
#pragma unroll
    for (int e = 1; e < 4; ++e)
        if (code[e] > lm) {
            lm = code[e];
            le = e;
        }
    uint32_t lrest = 0u;  // the lane's largest code besides its winner
#pragma unroll
    for (int e = 0; e < 4; ++e)
        if (e != le) lrest = max(lrest, code[e]);
    const int lane = threadIdx.x & (kWave - 1);
    const uint32_t wm = wave_max_u(lm);
    const uint64_t holders = __ballot(wm != 0u && lm == wm);
    const int wl = holders ? static_cast<int>(__builtin_ctzll(holders)) : 0;  // lowest lane, lowest index
    const uint32_t ws = wave_max_u(lane == wl ? lrest : lm);
    const int wi = __builtin_amdgcn_readlane(base + 4 * static_cast<int>(threadIdx.x) + le, wl);
    if (lane == 0) scratch[threadIdx.x >> 6] = make_uint4(wm, static_cast<uint32_t>(wi), ws, 0u);
    lds_barrier();
    uint32_t bm = 0u, sm = 0u;
    int bi = -1;
#pragma unroll
    for (int w = 0; w < NW; ++w) {  // waves hold ascending index ranges: strict > keeps the lowest
        const uint4 r = scratch[w];
        if (r.x > bm) {
            sm = max(sm, bm);
            bm = r.x;
            bi = static_cast<int>(r.y);
        } else {
            sm = max(sm, r.x);
        }
        sm = max(sm, r.z);
    }
    if (bm == 0u) return make_int2(-1, 0);
    const bool tie = sm != 0u && float_of_code(sm) >= float_of_code(bm) - kTieEps;
    return make_int2(bi, tie ? 1 : 0);
}

__device__ __forceinline__ double ln_of(double x) { return ln_f32(static_cast<float>(x)); }

// Level 1 of a residual draw: block c's key is ln W_c + G_c (G_c the level-1
// Gumbel variate of block c of position n of request b) rounded to fp32; the
// largest key wins, the lowest block on equal keys, flagged when another key
// lies within kTieEps.  w_of(r, c): the residual mass of block c = lane +
// 64 r.  Each wave runs the whole race, one block per lane and round, so all
// waves agree without a barrier.  *wwin receives the winner's mass.
template <typename GET>
__device__ __forceinline__ Level1 residual_level1(GET w_of, int C, PhiloxKey key, int b, int n, double *wwin) {
    const int lane = threadIdx.x & (kWave - 1);
    uint32_t lb = 0u, ls = 0u;  // the lane's largest code (at its lowest block) and the next
    int li = INT_MAX;
    double lw = 0.0;            // the mass of the lane's block li
    for (int r = 0, cb = lane; cb < C; ++r, cb += kWave) {
        const double w = w_of(r, cb);
        if (!(w > 0.0)) continue;
        const uint32_t code = ordered_code(static_cast<float>(ln_of(w) + block_gumbel(key, b, n, cb)));
        if (code > lb) {
            ls = lb;
            lb = code;
            li = cb;
            lw = w;
        } else {
            ls = max(ls, code);
        }
    }
    const uint32_t wm = wave_max_u(lb);
    if (wm == 0u) return Level1{-1, 0};
    const int wi = wave_min_i(lb == wm ? li : INT_MAX);
    const uint32_t ws = wave_max_u(li == wi ? ls : lb);
    const bool tie = ws != 0u && float_of_code(ws) >= float_of_code(wm) - kTieEps;
    *wwin = __shfl(lw, wi & (kWave - 1));  // block wi sits in lane wi mod 64
    return Level1{wi, tie ? 1 : 0};
}

// Level 2: the token of block cb of row n drawn under the weights of `mode`
// (4 tokens per thread; values from the staged LDS copy when `staged`).  All
// threads call it; returns (token, near-tie flag), token -1 when the block
// holds no positive weight.  wblk: the level-1 residual mass of block cb
// (dense mode; 1 otherwise).
template <typename ET, bool ALIGNED>
__device__ int2 level2(const FinalArgs &a, FinalShared &sh, int b, int n, int64_t row, int x, int cb,
                       int mode, float c, double invT, const float *qrow, bool staged, int attempt,
                       double wblk = 1.0) {
    const int V = a.V;
    const int64_t j0 = int64_t(cb) * kBlock + threadIdx.x * 4;
    float lv[4], qv[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (staged) {
        const float4 f = *reinterpret_cast<const float4 *>(&sh.blockv[threadIdx.x * 4]);
        lv[0] = f.x;
        lv[1] = f.y;
        lv[2] = f.z;
        lv[3] = f.w;
    } else {
        load4_masked<ET, ALIGNED>(reinterpret_cast<const ET *>(a.logits) + row * V,
                                  a.mask ? a.mask + row * a.W : nullptr, j0, V, lv);
        if (a.tau) apply_tau<4>(lv, a.tau[row]);
    }
    if (mode == kModeDense) {  // in flight with the logits; lanes past V read (and drop) the last four
        if (ALIGNED) {
            const int64_t jc = j0 + 4 <= V ? j0 : int64_t(V) - 4;
            const float4 f = *reinterpret_cast<const float4 *>(qrow + jc);
            qv[0] = f.x;
            qv[1] = f.y;
            qv[2] = f.z;
            qv[3] = f.w;
        } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) qv[e] = qrow[j0 + e < V ? j0 + e : int64_t(V - 1)];
        }
    }
    float g[4];
    draw_token_gumbels4(key_of(a.seed), b, n, static_cast<uint32_t>(j0), g);
    const float M = sh.M[n];
    const double S = sh.S[n];
    const double invS = 1.0 / S, invW = 1.0 / wblk;
    const double lref = static_cast<double>(M) / static_cast<double>(c);  // about the row's max logit
    uint32_t code[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int64_t j = j0 + e;
        code[e] = 0u;  // no candidate
        if (!(lv[e] > -INFINITY)) continue;  // masked, -inf, or past V
        if (mode == kModeDense) {
            const double p = exp2_precise_nonpos(static_cast<double>(lv[e]) * c - static_cast<double>(M)) * invS;
            const double r = p - static_cast<double>(qv[e]);
            if (!(r > 0.0)) continue;
            // Keys relative to the block's residual mass (one constant for the
            // whole draw): a token that can win has ln(r / W) >= ln(1/2048) -
            // 2.9 - 16.7 (W is at most 2048 times the largest r; Gumbel
            // variates lie in [-2.9, 16.7]), so its key stays small.
            code[e] = ordered_code(static_cast<float>(ln_of(r * invW) + static_cast<double>(g[e])));
        } else {
            if (mode == kModeOneHot && j == x) continue;
            code[e] = ordered_code(
                static_cast<float>((static_cast<double>(lv[e]) - lref) * invT + static_cast<double>(g[e])));
        }
    }
    return race_winner<kFinalWaves>(code, static_cast<int>(j0) - 4 * static_cast<int>(threadIdx.x),
                                    sh.race[attempt & 1]);
}

// A lane's share of one row's block statistics, blocks lane + 64 j for
// j < kFoldCache, loaded once (absent blocks are clamped to the last one and
// read as empty where the cached fold uses them, so that nothing waits for
// the loads here).  Rows of more
// than 64 kFoldCache blocks fold the rest straight from memory.
constexpr int kFoldCache = 2;

struct FoldCache {
    BlockStat e[kFoldCache];
};

__device__ __forceinline__ void load_fold_cache(const BlockStat *st, int C, int lane, FoldCache &fc) {
#pragma unroll
    for (int j = 0; j < kFoldCache; ++j) {
        const int cb = lane + kWave * j;
        const int cc = cb < C ? cb : C - 1;  // clamped: every lane loads, no branch
        fc.e[j] = st[cc];
    }
}

// Block cb's statistics for the fold: from the cache when it holds them.
__device__ __forceinline__ BlockStat fold_entry(const BlockStat *st, const FoldCache &fc, int j,
                                                int cb) {
    if (j < kFoldCache) {
        BlockStat r = fc.e[0];
#pragma unroll
        for (int q = 1; q < kFoldCache; ++q)
            if (j == q) r = fc.e[q];
        return r;
    }
    return st[cb];
}

// Fold one greedy row's block statistics (one wave): max and lowest argmax.
__device__ __forceinline__ void fold_greedy_row(const BlockStat *st, const FoldCache &fc, int C, int i,
                                                FinalShared &sh) {
    const int lane = threadIdx.x & (kWave - 1);
    bool bad = false;
    float best = -INFINITY;
    int bidx = INT_MAX;
    for (int j = 0, cb = lane; cb < C; ++j, cb += kWave) {
        const BlockStat e = fold_entry(st, fc, j, cb);
        if (e.m != e.m || e.m == INFINITY) bad = true;
        if (e.m > best) {
            best = e.m;
            bidx = __float_as_int(e.s);
        }
    }
    bad = wave_any(bad);
    const float m = wave_max(best);
    const int gi = wave_min_i(best == m ? bidx : INT_MAX);
    if (lane == 0) {
        sh.M[i] = m;
        sh.G[i] = gi;
        sh.S[i] = 1.0;
        if (bad) sh.rowst[i] |= SD_STATUS_BAD_LOGIT;
        else if (m == -INFINITY) sh.rowst[i] |= SD_STATUS_EMPTY_ROW;
    }
}

// 2^d for d <= 0 in double precision from an fp32 exp2 of the fractional
// part (relative error of a few 1e-8).
__device__ __forceinline__ double exp2_nonpos(double d) {
    const double n = floor(d);
    return ldexp(static_cast<double>(__builtin_amdgcn_exp2f(static_cast<float>(d - n))),
                 static_cast<int>(n));
}

// Fold one sampling row's block statistics (one wave) into its max and
// normaliser, and finish its level-1 races over the keys the sweep drew:
// under p, and under p with block cx's key replaced by the draft-excluded
// key keyx.
__device__ __forceinline__ void fold_sampling_row(const BlockStat *st, const FoldCache &fc, int C,
                                                  int i, int cx, double keyx, FinalShared &sh) {
    const int lane = threadIdx.x & (kWave - 1);
    bool bad = false;
    float mx = -INFINITY;
    for (int j = 0, cb = lane; cb < C; ++j, cb += kWave) {
        const BlockStat e = fold_entry(st, fc, j, cb);
        if (e.m != e.m || e.s != e.s || e.m == INFINITY) bad = true;
        mx = fmaxf(mx, e.m);
    }
    bad = wave_any(bad);
    const float m = wave_max(mx);
    const double ref = static_cast<double>(m) * kLn2;  // keys relative to the row
    double s = 0.0;
    uint32_t cp = 0u, cxm = 0u;  // the lane's largest codes (0 = none), at its lowest block
    int ip = INT_MAX, ix = INT_MAX;
    if (!bad && m > -INFINITY) {
        for (int j = 0, cb = lane; cb < C; ++j, cb += kWave) {
            const BlockStat e = fold_entry(st, fc, j, cb);
            if (!(e.m > -INFINITY) || !(e.s > 0.0f)) continue;
            s += static_cast<double>(e.s) * exp2_nonpos(static_cast<double>(e.m) - static_cast<double>(m));
            const uint32_t code = ordered_code(static_cast<float>(e.key - ref));
            const uint32_t codex = cb != cx ? code
                                   : (keyx > -INFINITY ? ordered_code(static_cast<float>(keyx - ref)) : 0u);
            if (code > cp) {
                cp = code;
                ip = cb;
            }
            if (codex > cxm) {
                cxm = codex;
                ix = cb;
            }
        }
    }
    s = wave_sum_d(s);
    uint64_t bp = wave_argmax_code(cp, ip);
    uint64_t bx = wave_argmax_code(cxm, ix);
    // the winners in fp64 (race_in_fp64 for rows of any length)
    for (int r = 0; r < 2; ++r) {
        uint64_t &w = r == 0 ? bp : bx;
        if (w == 0) continue;
        const float wk = packed_key(w);
        int close = 0;
        for (int j = 0, cb = lane; cb < C; ++j, cb += kWave) {
            const BlockStat e = fold_entry(st, fc, j, cb);
            if (!(e.m > -INFINITY) || !(e.s > 0.0f)) continue;
            const double kd = (r == 1 && cb == cx) ? keyx - ref : e.key - ref;
            close += (kd > -INFINITY && static_cast<float>(kd) >= wk - kRaceSlack) ? 1 : 0;
        }
        if (!wave_any(close > 1) && __popcll(__ballot(close > 0)) <= 1) continue;
        double best = -INFINITY;
        int bi = INT_MAX;
        for (int j = 0, cb = lane; cb < C; ++j, cb += kWave) {
            const BlockStat e = fold_entry(st, fc, j, cb);
            if (!(e.m > -INFINITY) || !(e.s > 0.0f)) continue;
            const double kd = (r == 1 && cb == cx) ? keyx - ref : e.key - ref;
            if (kd > best) {
                best = kd;
                bi = cb;
            }
        }
        const double m2 = wave_max_d(best);
        const int i2 = wave_min_i((m2 > -INFINITY && best == m2) ? bi : INT_MAX);
        w = pack_code(ordered_code(static_cast<float>(m2)), i2);
    }
    bool tp = false, tx = false;
    if (bp != 0) {
        for (int j = 0, cb = lane; cb < C; ++j, cb += kWave) {
            const BlockStat e = fold_entry(st, fc, j, cb);
            if (!(e.m > -INFINITY) || !(e.s > 0.0f)) continue;
            const float kp = static_cast<float>(e.key - ref);
            tp |= near_tie(kp, cb, bp);
            if (cb != cx) tx |= near_tie(kp, cb, bx);
            else if (keyx > -INFINITY) tx |= near_tie(static_cast<float>(keyx - ref), cb, bx);
        }
    }
    tp = wave_any(tp);
    tx = wave_any(tx);
    if (lane == 0) {
        sh.M[i] = m;
        sh.S[i] = s;
        sh.G[i] = -1;
        sh.l1p[i] = bp ? Level1{packed_index(bp), tp ? 1 : 0} : Level1{-1, 0};
        sh.l1x[i] = bx ? Level1{packed_index(bx), tx ? 1 : 0} : Level1{-1, 0};
        if (bad) sh.rowst[i] |= SD_STATUS_BAD_LOGIT;
        else if (m == -INFINITY) sh.rowst[i] |= SD_STATUS_EMPTY_ROW;
    }
}

// The same fold when the row has at most 64 kFoldCache blocks, so that the
// cache holds all of them (absent blocks read as empty): straight-line code
// over the cached entries instead of a loop whose trip count differs by lane.
// It runs in two parts so that the block the row would sample is known, and
// its loads issued, before the normaliser and the tie flags are worked out.
struct CachedFold {
    float m;                  // the row's max (log2 units)
    double ref;               // keys relative to m ln 2
    bool bad;                 // a NaN or +inf logit in the row
    uint64_t bp, bx;          // level-1 winners under p and without the draft (0: none)
    float kps[kFoldCache];    // the entries' keys relative to ref
    bool live[kFoldCache];    // entries with mass
};

__device__ __forceinline__ CachedFold fold_races(FoldCache &fc, int C, int cx, double keyx) {
    const int lane = threadIdx.x & (kWave - 1);
    CachedFold f;
    bool bad = false;
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < kFoldCache; ++j) {
        BlockStat &e = fc.e[j];
        if (lane + kWave * j >= C) {  // past the row: empty
            e.m = -INFINITY;
            e.s = 0.0f;
            e.key = -INFINITY;
        }
        bad |= (e.m != e.m) | (e.s != e.s) | (e.m == INFINITY);
        mx = fmaxf(mx, e.m);
    }
    f.bad = wave_any(bad);
    f.m = wave_max_coded(mx);
    f.ref = static_cast<double>(f.m) * kLn2;
    uint32_t cp = 0u, cxm = 0u;  // the lane's largest codes (0 = none), at its lowest block
    int ip = INT_MAX, ix = INT_MAX;
#pragma unroll
    for (int j = 0; j < kFoldCache; ++j) {
        const BlockStat &e = fc.e[j];
        const int cb = lane + kWave * j;
        f.live[j] = !f.bad && f.m > -INFINITY && e.m > -INFINITY && e.s > 0.0f;
        f.kps[j] = static_cast<float>(e.key - f.ref);
        if (!f.live[j]) continue;
        const uint32_t code = ordered_code(f.kps[j]);
        const uint32_t codex = cb != cx ? code
                               : (keyx > -INFINITY ? ordered_code(static_cast<float>(keyx - f.ref)) : 0u);
        if (code > cp) {
            cp = code;
            ip = cb;
        }
        if (codex > cxm) {
            cxm = codex;
            ix = cb;
        }
    }
    // Without a draft block to leave out (the bonus row, dense q, an invalid
    // draft) the second race is the first: it is not run.
    const bool xrace = cx >= 0;
    f.bp = wave_argmax_code(cp, ip);
    f.bx = xrace ? wave_argmax_code(cxm, ix) : f.bp;
    // The fp32 races stand unless another key lies within kRaceSlack of the
    // winner's (counted on the fp32 keys already at hand); only then are the
    // fp64 keys formed and raced (race_in_fp64).
    const float wkp = f.bp ? packed_key(f.bp) : INFINITY, wkx = f.bx ? packed_key(f.bx) : INFINITY;
    const float kpx = keyx > -INFINITY ? static_cast<float>(keyx - f.ref) : -INFINITY;
    int closep = 0, closex = 0;
#pragma unroll
    for (int j = 0; j < kFoldCache; ++j) {
        if (!f.live[j]) continue;
        const float kx = lane + kWave * j != cx ? f.kps[j] : kpx;
        closep += f.kps[j] >= wkp - kRaceSlack ? 1 : 0;
        closex += kx > -INFINITY && kx >= wkx - kRaceSlack ? 1 : 0;
    }
    const bool refine_p = __popcll(__ballot(closep > 0)) + __popcll(__ballot(closep > 1)) > 1;
    const bool refine_x = xrace && __popcll(__ballot(closex > 0)) + __popcll(__ballot(closex > 1)) > 1;
    if (refine_p || refine_x) {
        double kd[kFoldCache], kdx[kFoldCache];
#pragma unroll
        for (int j = 0; j < kFoldCache; ++j) {
            const int cb = lane + kWave * j;
            kd[j] = f.live[j] ? fc.e[j].key - f.ref : -INFINITY;
            kdx[j] = cb != cx ? kd[j] : (f.live[j] && keyx > -INFINITY ? keyx - f.ref : -INFINITY);
        }
        if (refine_p) f.bp = race_in_fp64(f.bp, kd);
        if (refine_x) f.bx = race_in_fp64(f.bx, kdx);
        if (!xrace) f.bx = f.bp;
    }
    return f;
}

__device__ __forceinline__ void fold_finish(const FoldCache &fc, const CachedFold &f, int i, int cx, double keyx,
                                            FinalShared &sh) {
    const int lane = threadIdx.x & (kWave - 1);
    double s = 0.0;
    bool tp = false, tx = false;
#pragma unroll
    for (int j = 0; j < kFoldCache; ++j) {
        const BlockStat &e = fc.e[j];
        const int cb = lane + kWave * j;
        if (!f.live[j]) continue;
        s += static_cast<double>(e.s) * exp2_nonpos(static_cast<double>(e.m) - static_cast<double>(f.m));
        tp |= near_tie(f.kps[j], cb, f.bp);
        if (cb != cx) tx |= near_tie(f.kps[j], cb, f.bx);
        else if (keyx > -INFINITY) tx |= near_tie(static_cast<float>(keyx - f.ref), cb, f.bx);
    }
    s = wave_sum_d(s);
    tp = f.bp != 0 && wave_any(tp);
    tx = f.bp != 0 && wave_any(tx);
    if (lane == 0) {
        sh.M[i] = f.m;
        sh.S[i] = s;
        sh.G[i] = -1;
        sh.l1p[i] = f.bp ? Level1{packed_index(f.bp), tp ? 1 : 0} : Level1{-1, 0};
        sh.l1x[i] = f.bx ? Level1{packed_index(f.bx), tx ? 1 : 0} : Level1{-1, 0};
        if (f.bad) sh.rowst[i] |= SD_STATUS_BAD_LOGIT;
        else if (f.m == -INFINITY) sh.rowst[i] |= SD_STATUS_EMPTY_ROW;
    }
}

// A draft row's draft token and what the row sweep recorded about it, read
// by the wave that folds the row, with the position's accept draw.
struct RowDraft {
    int x = -1;            // the draft token (unchecked)
    float lx = -INFINITY;  // its logit
    float qx = 1.0f;       // q_i(x)
    bool invalid = false;  // outside the mask
    double keyx = -INFINITY;  // level-1 key of its block without it
    double u = 0.0;        // the accept draw
};

// Row i's draft and record as issued loads (rows past the request's drafts
// read zeros); `settle_row_draft` takes the values once they are needed.
struct RowDraftLoads {
    uint32_t x;
    uint32_t lx, qx, allowed;
    uint32_t keyx_lo, keyx_hi;
};

__device__ __forceinline__ RowDraftLoads issue_row_draft(const FinalArgs &a, const ReqGeom &geo, int i) {
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    const __amdgpu_buffer_rsrc_t rd = buffer_of(a.draft + geo.draft0, uint32_t(geo.k) * 4u);
    const __amdgpu_buffer_rsrc_t rr =
        buffer_of(a.drec + geo.row0, uint32_t(geo.k + 1) * uint32_t(sizeof(DraftRec)));
    RowDraftLoads l;
    l.x = __builtin_amdgcn_raw_buffer_load_b32(rd, 0, i * 4, 0);
    const int ro = i * int(sizeof(DraftRec));
    const u32x4 r = __builtin_amdgcn_raw_buffer_load_b128(rr, 0, ro, 0);  // sx, lx, qx, allowed
    const u32x2 kx = __builtin_amdgcn_raw_buffer_load_b64(rr, 0, ro + 16, 0);
    l.lx = r.y;
    l.qx = r.z;
    l.allowed = r.w;
    l.keyx_lo = kx.x;
    l.keyx_hi = kx.y;
    return l;
}

__device__ __forceinline__ RowDraft settle_row_draft(const RowDraftLoads &l) {
    RowDraft d;  // the record is used only when x is valid
    d.x = static_cast<int>(uniform_word(l.x));
    d.lx = __uint_as_float(uniform_word(l.lx));
    d.qx = __uint_as_float(uniform_word(l.qx));
    d.invalid = !(uniform_word(l.allowed) & 1u);
    d.keyx = __hiloint2double(static_cast<int>(uniform_word(l.keyx_hi)), static_cast<int>(uniform_word(l.keyx_lo)));
    return d;
}

// Position i's verdict, taken by lane 0 of the wave that folded row i: the
// accept probability min(1, p/q) (pyshine "vLLM, part 2", "Verification"),
// the accept draw against it, its boundary flag, and whether the draft's q is
// unusable (reported only when nothing else is wrong).  Greedy rows accept a
// draft equal to the row's argmax.
__device__ __forceinline__ void judge_position(FinalShared &sh, int i, bool greedy, float c, bool one_hot,
                                               const RowDraft &d) {
    bool ok, flag = false, badq = false;
    double acc;
    if (greedy) {
        ok = (d.x == sh.G[i]);
        acc = ok ? 1.0 : 0.0;
    } else {
        double p = 0.0;
        if (!d.invalid && d.lx > -INFINITY)
            p = exp2(static_cast<double>(d.lx) * c - static_cast<double>(sh.M[i])) / sh.S[i];
        badq = !one_hot && !(d.qx >= 0.0f && d.qx <= FLT_MAX);
        const double q = d.qx;
        acc = (p == 0.0) ? 0.0 : (q == 0.0 ? 1.0 : fmin(1.0, p / q));
        const double u = d.u;
        ok = u < acc;
        flag = fabs(u - acc) < kAcceptFlagEps;
    }
    sh.acc[i] = acc;
    sh.ok[i] = ok;
    sh.flag[i] = flag;
    sh.badq[i] = badq;
}

// Counters of the call.  Every workgroup finishes at about the same time, so
// words hit by all of them would serialise their atomics; instead request b
// adds to slot word b % nslot, and the request that completes a slot adds the
// slot's sums to the four output counters (zeroed by the row-statistics
// kernel) with atomics whose results nobody waits for.  A slot word packs the
// arrival count with the sums, so the workgroup that completes a slot reads
// the slot's totals in its own atomic's return value: no fence and no
// ordering between different words is needed, and the integer sums do not
// depend on the order of arrival.  A request in error adds only its arrival.
//   slot word: arrivals [0,9)  accepted [9,24)  outside grammar [24,39)  drafts [39,54)
// Field widths hold at most 256 slots of at most 256 requests of at most 64
// drafts.
__device__ __forceinline__ unsigned long long tally_share(int accepted, int invalid, int drafts) {
    return 1ull | (static_cast<unsigned long long>(accepted) << 9) |
           (static_cast<unsigned long long>(invalid) << 24) |
           (static_cast<unsigned long long>(drafts) << 39);
}

// Adds request b's share to its slot word; returns the word's previous value.
// The caller reads the result as late as it can, so that the atomic's round
// trip overlaps other work.
__device__ __forceinline__ unsigned long long tally_slot(const FinalArgs &a, int b,
                                                         unsigned long long share) {
    return atomicAdd(&a.tally[(b % a.nslot) * kTallyStride], share);
}

// `before` is what tally_slot returned for request b with `share`.
__device__ __forceinline__ void tally_call(const FinalArgs &a, int b, unsigned long long before,
                                           unsigned long long share) {
    const unsigned long long slot = before + share;
    const int S = a.nslot, s = b % S;
    const int members = (a.B - s + S - 1) / S;  // requests b' < B with b' % S == s
    if (static_cast<int>(slot & 0x1ffull) != members) return;
    const unsigned long long acc = (slot >> 9) & 0x7fffull, inv = (slot >> 24) & 0x7fffull,
                             drafts = (slot >> 39) & 0x7fffull;
    unsigned long long *out = reinterpret_cast<unsigned long long *>(a.out_counters);
    atomicAdd(&out[0], drafts);        // R
    atomicAdd(&out[1], inv);           // I
    atomicAdd(&out[2], drafts - inv);  // D
    atomicAdd(&out[3], acc);           // A
}

// Issue the loads of block c of a row for the staging (c < 0: none); with a
// mask, m[0] receives the lane's word of the block's mask (spread_mask).
template <typename ET>
__device__ __forceinline__ void stage_block(const FinalArgs &a, int row, int c, int lane, uint4 *r, uint32_t *m) {
    if (c < 0) return;
    RowStatsArgs ra;  // only the fields issue_block reads
    ra.logits = a.logits;
    ra.mask = a.mask;
    ra.V = a.V;
    ra.W = a.W;
    if (a.mask) issue_block<ET, true>(ra, row, c, lane, r, m);
    else issue_block<ET, false>(ra, row, c, lane, r, m);
}

// DENSE: dense draft probabilities; SPLIT (with DENSE): the residual masses
// of rejected rows are left to the grid-wide kernels, so this instantiation
// carries no in-kernel residual pass and its registers.
template <typename ET, bool ALIGNED, bool DENSE, bool SPLIT>
__global__ __launch_bounds__(kFinalThreads) void finalize_kernel(FinalArgs a) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    __shared__ FinalShared sh;
    // dense q, short rows or listed lines: per-block residual mass [C]; with
    // listed lines also their sums [kCandLines] and indices [kCandLines]
    extern __shared__ double sW[];
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = wave_id();
    const ReqGeom geo = req_geom(a.off, a.off_ok, b, a.k);
    const int k = geo.k, kp1 = geo.k + 1, V = a.V, C = a.C;
    // ---- this wave's first row: its block statistics, draft and record are
    //      all in flight before anything waits for memory
    FoldCache fc;
    if (geo.ok && wave < kp1) load_fold_cache(a.bstats + (geo.row0 + wave) * C, C, lane, fc);
    const RowDraftLoads rl = issue_row_draft(a, geo, wave);
    const uint32_t Tw = __builtin_amdgcn_raw_buffer_load_b32(buffer_of(a.temperature, uint32_t(a.B) * 4u), 0, b * 4, 0);
    const PhiloxKey key = key_of(a.seed);
    // the accept draw depends on nothing loaded: drawn while the loads fly
    const double u0 = wave < k ? draw_accept(key, b, wave) : 0.0;
    // the row-statistics kernel has finished: its claim counters go back to
    // zero for the next call
    if (b == 0 && tid < kSweepParts) a.sweep[tid * kSweepCtrStride] = 0u;
    if (tid == 0) sh.staged_c = -1;  // read only after the fold's barrier
    const float T = __uint_as_float(uniform_word(Tw));
    const bool greedy = (T == 0.0f);
    const bool bad_T = !greedy && !(T > 0.0f && T <= FLT_MAX);
    const bool skip_rows = bad_T || !geo.ok;  // nothing of the request's rows is used
    const float c = greedy || bad_T ? 0.0f : scale_of(T);
    constexpr bool one_hot = !DENSE;
    RowDraft rd = settle_row_draft(rl);
    rd.u = u0;

    // ---- one wave per row: fold the block statistics; sampling rows also run
    //      their level-1 race and start loading the block they would sample;
    //      draft rows then take their position's verdict
    uint4 stage_r[G];
    uint32_t stage_m[G];
    int stage_row = -1, stage_c = -1;
    for (int i = wave; i < kp1; i += kFinalWaves) {
        const int64_t row = geo.row0 + i;
        const BlockStat *st = a.bstats + row * C;
        if (i != wave) {  // rows past the first wave of rows
            if (geo.ok) load_fold_cache(st, C, lane, fc);
            if (i < k) {
                rd = settle_row_draft(issue_row_draft(a, geo, i));
                rd.u = draw_accept(key, b, i);
            }
        }
        const int xi = (i < k) ? rd.x : -1;
        const bool xok = xi >= 0 && xi < V;
        if (lane == 0) {
            sh.rowst[i] = (i < k && !xok) ? SD_STATUS_DRAFT_ID : 0u;
            if (i < k) {
                sh.X[i] = xi;
                sh.invalid[i] = rd.invalid;
            }
        }
        if (skip_rows) continue;
        if (greedy) {
            fold_greedy_row(st, fc, C, i, sh);
            if (i < k && lane == 0) judge_position(sh, i, true, c, one_hot, rd);
            continue;
        }
        const int cx = (one_hot && xok) ? xi / kBlock : -1;
        const double keyx = cx >= 0 ? rd.keyx : -INFINITY;
        int pre = -1;  // the block this row samples from, if it is the one emitting
        if (C <= kWave * kFoldCache) {
            const CachedFold f = fold_races(fc, C, cx, keyx);
            const uint64_t w = (i < k) ? (one_hot ? f.bx : 0ull) : f.bp;
            pre = w ? packed_index(w) : -1;
            if (ALIGNED && kp1 <= kFinalWaves) stage_block<ET>(a, static_cast<int>(row), pre, lane, stage_r, stage_m);
            fold_finish(fc, f, i, cx, keyx, sh);
        } else {
            fold_sampling_row(st, fc, C, i, cx, keyx, sh);
            const Level1 l1 = (i < k) ? (one_hot ? sh.l1x[i] : Level1{-1, 0}) : sh.l1p[i];
            pre = l1.c;
            if (ALIGNED && kp1 <= kFinalWaves) stage_block<ET>(a, static_cast<int>(row), pre, lane, stage_r, stage_m);
        }
        if (ALIGNED && kp1 <= kFinalWaves && pre >= 0) {
            stage_row = i;
            stage_c = pre;
        }
        if (i < k && lane == 0) judge_position(sh, i, false, c, one_hot, rd);
    }
    lds_barrier();

    // ---- every wave reads the rows' status bits and the k <= 64 verdicts and
    //      finds the first rejection with ballots (all waves agree, so no
    //      barrier follows)
    uint32_t st = (bad_T ? SD_STATUS_TEMPERATURE : 0u) | (geo.ok ? 0u : SD_STATUS_BAD_OFFSETS);
    int nacc = 0, flag_acc = 0, ninv = 0;
    {
        uint32_t rs = lane < kp1 ? sh.rowst[lane] : 0u;
        if (kp1 > kWave) rs |= sh.rowst[kWave];
#pragma unroll
        for (uint32_t bit : {SD_STATUS_DRAFT_ID, SD_STATUS_EMPTY_ROW, SD_STATUS_BAD_LOGIT})
            if (__ballot((rs & bit) != 0u) != 0ull) st |= bit;
        bool okv = false, flv = false, inv = false, bq = false;
        if (lane < k) {
            okv = sh.ok[lane];
            flv = sh.flag[lane];
            inv = sh.invalid[lane];
            bq = sh.badq[lane];
        }
        if (st == 0 && __ballot(bq) != 0ull) st = SD_STATUS_BAD_DRAFT_PROB;
        const uint64_t okm = __ballot(okv), flm = __ballot(flv), invm = __ballot(inv);
        const uint64_t kmask = k >= 64 ? ~0ull : ((1ull << k) - 1ull);
        const uint64_t rejected = ~okm & kmask;
        nacc = rejected ? static_cast<int>(__builtin_ctzll(rejected)) : k;  // first rejection
        const uint64_t scanned = nacc < k ? ((2ull << nacc) - 1ull) : kmask;  // positions tested
        flag_acc = __popcll(flm & scanned);
        ninv = __popcll(invm);
    }

    // ---- the wave that loaded the sampled row's block puts it in LDS
    if (st == 0 && stage_row >= 0 && stage_row == nacc) {
        uint32_t smm[G];
        if (a.mask) spread_mask<G, P>(stage_m[0], lane, smm);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float v[P];
            Logit<ET>::unpack(stage_r[g], v);
            const int off = (g * kWave + lane) * P;  // token offset inside the block
            const int64_t tok = int64_t(stage_c) * kBlock + off;
            uint32_t bits = tok < V ? 0xffu : 0u;
            if (a.mask) bits &= (P == 8) ? smm[g] : (smm[g] >> (uint32_t(tok) & 4u));
#pragma unroll
            for (int e = 0; e < P; ++e)
                if (!((bits >> e) & 1u)) v[e] = -INFINITY;
            if (a.tau) apply_tau<P>(v, a.tau[geo.row0 + stage_row]);
#pragma unroll
            for (int h = 0; h < P / 4; ++h)
                *reinterpret_cast<float4 *>(&sh.blockv[off + 4 * h]) =
                    make_float4(v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]);
        }
        if (lane == 0) sh.staged_c = stage_c;
    }
    // The request's share of the counters is known now: its atomic is issued
    // here and completes while the emitted token is drawn (every barrier from
    // here on waits for LDS traffic only).
    unsigned long long share = 0, before = 0;
    // Loads still in flight finish first (they were issued long ago): the
    // memory counter retires in order, so a later wait for one of them would
    // also wait for the atomic.
    __builtin_amdgcn_s_waitcnt(kWaitVmcnt0);
    if (tid == 0) {
        const bool err = st != 0;
        share = tally_share(err ? 0 : nacc, err ? 0 : ninv, err ? 0 : k);
        before = tally_slot(a, b, share);
    }
    lds_barrier();

    // ---- the emitted token
    int y = -1, fg = 0;
    bool deferred = false;
    if (DENSE && tid == 0) a.jobs[b].row = -1;  // overwritten below for a dense draw
    if (st == 0) {
        const int n = nacc;
        if (greedy) {
            y = sh.G[n];
        } else {
            const double invT = 1.0 / static_cast<double>(T);
            const float *qrow = (DENSE && n < k) ? a.q + (geo.draft0 + n) * V : nullptr;
            int mode = (n == k) ? kModeP : (DENSE ? kModeDense : kModeOneHot);
            double wdense = 1.0;  // the winning block's residual mass
            Level1 l1 = (mode == kModeOneHot) ? sh.l1x[n] : sh.l1p[n];
            // after the single-pass selection (kcount given) the residual
            // masses come from the lines of the row, here: from the listed
            // lines that hold a kept token alone, or from every line of a
            // long row the selection did not list (no grid-wide residual
            // pass runs then); short unlisted rows stream their blocks below
            uint32_t nl = kNoLineList;
            if (DENSE && mode == kModeDense && a.kcount != nullptr) nl = uniform_load(a.kcount + geo.row0 + n);
            const bool listed = DENSE && mode == kModeDense && a.kcount != nullptr && (SPLIT || nl != kNoLineList);
            if (listed) {
                const int64_t row = geo.row0 + n;
                line_block_masses<ET>(a, row, qrow, nl, c, sh.M[n], sh.S[n], a.tau ? a.tau[row] : -INFINITY, sW,
                                      sW + C, reinterpret_cast<int *>(sW + C + kResLines));
                l1 = residual_level1([&](int, int cb) { return sW[cb]; }, C, key, b, n, &wdense);
            }
            if (DENSE && SPLIT && mode == kModeDense && !listed) {
                // left to the residual kernels; -1 stands in until they write y
                if (tid == 0) {
                    DenseJob j;
                    j.row = static_cast<int>(geo.row0 + n);
                    j.dpos = geo.draft0 + n;
                    j.n = n;
                    j.c = c;
                    j.M = sh.M[n];
                    j.S = sh.S[n];
                    j.tau = a.tau ? a.tau[geo.row0 + n] : -INFINITY;
                    j.l1p = sh.l1p[n];
                    j.invT = invT;
                    a.jobs[b] = j;
                }
                deferred = true;
            }
            if (DENSE && !SPLIT && mode == kModeDense && !listed) {
                const int64_t row = geo.row0 + n;
                dense_block_masses<ET, ALIGNED>(
                    reinterpret_cast<const ET *>(a.logits) + row * V,
                    a.mask ? a.mask + row * a.W : nullptr, qrow, V, C, c, sh.M[n], sh.S[n],
                    a.tau ? a.tau[row] : -INFINITY, sW);
                lds_barrier();
                // residual masses are <= 1, so their keys need no reference
                l1 = residual_level1([&](int, int cb) { return sW[cb]; }, C, key, b, n, &wdense);
            }
            // A zero residual mass, or a block that lost its mass in double
            // precision, falls back to drawing from p.
            for (int attempt = 0; attempt < 2 && !deferred; ++attempt) {
                if (l1.c < 0) {
                    mode = kModeP;
                    l1 = sh.l1p[n];
                }
                const int2 r2 =
                    level2<ET, ALIGNED>(a, sh, b, n, geo.row0 + n, n < k ? sh.X[n] : -1, l1.c, mode, c,
                                        invT, qrow, sh.staged_c == l1.c, attempt,
                                        (DENSE && (listed || !SPLIT) && mode == kModeDense) ? wdense : 1.0);
                if (r2.x >= 0) {
                    y = r2.x;
                    fg = l1.flag + r2.y;
                    break;
                }
                l1.c = -1;
            }
        }
    }

    // ---- outputs, and this request's share of the counters
    const int n = st ? -1 : nacc;
    if (tid < kp1 && geo.ok) {  // a malformed ragged call has no slots to write
        int tok = -1;
        if (!st) tok = tid < n ? sh.X[tid] : (tid == n ? y : -1);
        a.out_tokens[geo.row0 + tid] = tok;
        if (a.dbg_lse) {
            double v = NAN;
            if (!st) v = greedy ? static_cast<double>(sh.M[tid])
                                : kLn2 * (static_cast<double>(sh.M[tid]) + log2(sh.S[tid]));
            a.dbg_lse[geo.row0 + tid] = v;
        }
    }
    if (tid < k && a.dbg_acc) a.dbg_acc[geo.draft0 + tid] = st ? NAN : sh.acc[tid];
    if (tid == 0) {
        a.out_num_accepted[b] = n;
        // top-p boundary rows of this request (sampling requests only)
        uint32_t ftp = 0u;
        if (!st && a.tau && !greedy && (a.dbg_req_flags || a.dbg_flags))
            for (int r = 0; r < kp1; ++r) ftp += a.tau_flag[geo.row0 + r];
        if (a.dbg_req_flags)
            a.dbg_req_flags[b] = st ? 0u
                                    : (uint32_t(min(flag_acc, 0xfff)) | (uint32_t(min(fg, 0xfff)) << 12) |
                                       (min(ftp, 0xffu) << 24));
        if (st) {
            if (a.status) atomicOr(a.status, st);
        } else if (a.dbg_flags) {
            if (flag_acc) atomicAdd(&a.dbg_flags[0], static_cast<uint32_t>(flag_acc));
            if (fg) atomicAdd(&a.dbg_flags[1], static_cast<uint32_t>(fg));
            if (ftp) atomicAdd(&a.dbg_flags[2], ftp);
        }
        tally_call(a, b, before, share);
    }
}

// Residual masses W_c = sum_j max(p_j - q_j, 0) of the rejected rows of the
// deferred requests (pyshine "vLLM, part 2", "Verification": the rejected
// position is resampled from the clamped difference of the target and draft
// distributions).  Grid (ceil(C / 4), B); one wave per block, per-lane fp32
// partial sums added in fp64.
template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void dense_mass_kernel(FinalArgs a) {
    const int b = blockIdx.y;
    const int blk = blockIdx.x * (kThreads / kWave) + wave_id();
    const DenseJob j = a.jobs[b];
    if (j.row < 0 || blk >= a.C) return;
    const int V = a.V, lane = threadIdx.x & (kWave - 1);
    const ET *rowp = reinterpret_cast<const ET *>(a.logits) + int64_t(j.row) * V;
    const uint8_t *mb = a.mask ? reinterpret_cast<const uint8_t *>(a.mask + int64_t(j.row) * a.W) : nullptr;
    const float *qrow = a.q + j.dpos * V;
    const float invS = static_cast<float>(1.0 / j.S);
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    float lv[G][P], qv[G][P];
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t tok = int64_t(blk) * kBlock + (g * kWave + lane) * P;
        if (ALIGNED) {
            const int64_t tc = tok < V ? tok : int64_t(V - P);
            Logit<ET>::unpack(*reinterpret_cast<const uint4 *>(rowp + tc), lv[g]);
#pragma unroll
            for (int h = 0; h < P / 4; ++h) {
                const float4 f = *reinterpret_cast<const float4 *>(qrow + tc + 4 * h);
                qv[g][4 * h] = f.x;
                qv[g][4 * h + 1] = f.y;
                qv[g][4 * h + 2] = f.z;
                qv[g][4 * h + 3] = f.w;
            }
        } else {
#pragma unroll
            for (int e = 0; e < P; ++e) {
                const int64_t tc = tok + e < V ? tok + e : int64_t(V - 1);
                lv[g][e] = Logit<ET>::to_float(rowp[tc]);
                qv[g][e] = qrow[tc];
            }
        }
    }
    float acc = 0.0f;
#pragma unroll
    for (int g = 0; g < G; ++g) {
        const int64_t tok = int64_t(blk) * kBlock + (g * kWave + lane) * P;
        uint32_t bits = 0xffu;
        if (mb != nullptr) {
            const int64_t tc = tok < V ? tok : int64_t(V - 1);
            if (ALIGNED) {
                const uint32_t byte = mb[tc >> 3];
                bits = (P == 8) ? byte : (byte >> (uint32_t(tc) & 4u));
            } else {
                bits = 0u;
#pragma unroll
                for (int e = 0; e < P; ++e) {
                    const int64_t je = tok + e < V ? tok + e : int64_t(V - 1);
                    bits |= ((mb[je >> 3] >> (je & 7)) & 1u) << e;
                }
            }
        }
#pragma unroll
        for (int e = 0; e < P; ++e) {
            const bool live = tok + e < V && ((bits >> e) & 1u) && lv[g][e] > -INFINITY && !(lv[g][e] < j.tau);
            const float p = live ? __builtin_amdgcn_exp2f(fmaf(lv[g][e], j.c, -j.M)) * invS : 0.0f;
            acc += live ? fmaxf(p - qv[g][e], 0.0f) : 0.0f;
        }
    }
    const double w = wave_sum_d(static_cast<double>(acc));
    if (lane == 0) a.wmass[int64_t(b) * a.C + blk] = w;
}

// The token of each deferred request: level 1 over the residual masses, then
// level 2 inside the winning block (the same draws the finalize kernel makes
// for the other sampling modes); a zero residual falls back to p.
template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(kFinalThreads) void dense_draw_kernel(FinalArgs a) {
    __shared__ FinalShared sh;
    const int b = blockIdx.x, tid = threadIdx.x, lane = tid & (kWave - 1);
    const int C = a.C;
    // the residual masses of the first four rounds of blocks are read
    // together with the job (their place does not depend on it)
    const double *W = a.wmass + int64_t(b) * C;
    double w4[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) w4[r] = lane + kWave * r < C ? W[lane + kWave * r] : 0.0;
    const DenseJob j = a.jobs[b];
    if (j.row < 0) return;
    const int n = j.n;
    const PhiloxKey key = key_of(a.seed);
    if (tid == 0) {
        sh.M[n] = j.M;
        sh.S[n] = j.S;
    }
    lds_barrier();
    const float *qrow = a.q + j.dpos * a.V;
    // residual masses are <= 1, so their keys need no reference
    double wwin = 1.0;
    Level1 l1 = residual_level1(
        [&](int r, int cb) { return r == 0 ? w4[0] : r == 1 ? w4[1] : r == 2 ? w4[2] : r == 3 ? w4[3] : W[cb]; },
        C, key, b, n, &wwin);
    int mode = kModeDense, y = -1, fg = 0;
    const double invT = j.invT;
    for (int attempt = 0; attempt < 2; ++attempt) {
        if (l1.c < 0) {
            mode = kModeP;
            l1 = j.l1p;
        }
        // (no draft to exclude: dense q and its fallback to p keep every token)
        const int2 r2 = level2<ET, ALIGNED>(a, sh, b, n, j.row, -1, l1.c, mode, j.c, invT, qrow, false, attempt,
                                            mode == kModeDense ? wwin : 1.0);
        if (r2.x >= 0) {
            y = r2.x;
            fg = l1.flag + r2.y;
            break;
        }
        l1.c = -1;
    }
    if (tid == 0) {
        a.out_tokens[j.row] = y;
        if (a.dbg_req_flags) a.dbg_req_flags[b] += static_cast<uint32_t>(fg) << 12;
        if (a.dbg_flags && fg) atomicAdd(&a.dbg_flags[1], static_cast<uint32_t>(fg));
    }
}

// Outputs of an empty batch: zero counters, status, flags and histogram.
__global__ void empty_batch_kernel(uint64_t *counters, uint32_t *status, uint32_t *flags,
                                   uint32_t *hist, int kmax) {
    if (threadIdx.x < 4) counters[threadIdx.x] = 0ull;
    if (threadIdx.x == 0 && status) *status = 0u;
    if (threadIdx.x < 3 && flags) flags[threadIdx.x] = 0u;
    if (hist)
        for (int i = threadIdx.x; i <= kmax; i += blockDim.x) hist[i] = 0u;
}

// Ragged calls: checks the draft offsets (start at 0, never decrease, end at
// total, no request above kmax drafts) and, when they hold, writes the
// request of every row; one workgroup, so the check and the table need no
// ordering between workgroups.  Nothing is written through offsets that fail.
constexpr int kPrepThreads = 1024;

__global__ __launch_bounds__(kPrepThreads) void ragged_prep_kernel(const int32_t *off, int B, int kmax,
                                                                  int64_t total, int32_t *row_req,
                                                                  uint32_t *off_ok) {
    __shared__ uint32_t bad_any;
    if (threadIdx.x == 0) bad_any = 0u;
    __syncthreads();
    bool bad = threadIdx.x == 0 && (off[0] != 0 || int64_t(off[B]) != total);
    for (int b = threadIdx.x; b < B; b += kPrepThreads) {
        const int64_t d = int64_t(off[b + 1]) - int64_t(off[b]);
        bad |= d < 0 || d > kmax;
    }
    if (bad) atomicOr(&bad_any, 1u);
    __syncthreads();
    const bool ok = bad_any == 0u;
    if (threadIdx.x == 0) *off_ok = ok ? 1u : 0u;
    if (!ok) return;
    // the offsets now partition rows [0, total + B): request b owns k_b + 1
    // rows from off[b] + b
    for (int b = threadIdx.x; b < B; b += kPrepThreads) {
        const int64_t r0 = int64_t(off[b]) + b, kb = int64_t(off[b + 1]) - off[b];
        for (int64_t i = 0; i <= kb; ++i) row_req[r0 + i] = b;
    }
}

// Requests per accepted draft length 0 .. kmax (requests in error, with
// num_accepted = -1, left out); one workgroup, after the finalize kernels.
__global__ __launch_bounds__(1024) void histogram_kernel(const int32_t *num_accepted, int B, int kmax,
                                                         uint32_t *hist) {
    __shared__ uint32_t h[kMaxDraft + 1];
    for (int i = threadIdx.x; i <= kmax; i += blockDim.x) h[i] = 0u;
    __syncthreads();
    for (int b = threadIdx.x; b < B; b += blockDim.x) {
        const int n = num_accepted[b];
        if (n >= 0 && n <= kmax) atomicAdd(&h[n], 1u);
    }
    __syncthreads();
    for (int i = threadIdx.x; i <= kmax; i += blockDim.x) hist[i] = h[i];
}

// ------------------------------------------------------------------ dispatch

using RowStatsFn = void (*)(RowStatsArgs);
using FinalFn = void (*)(FinalArgs);

// topk: 0 none, 1 cut at tau, 2 line maxima (aligned rows only)
template <typename ET, int POL>
RowStatsFn pick_row_stats_vec(bool masked, int topk) {
    if (topk == 2) return masked ? row_stats_vec_kernel<ET, true, 2, POL> : row_stats_vec_kernel<ET, false, 2, POL>;
    if (topk == 1) return masked ? row_stats_vec_kernel<ET, true, 1, POL> : row_stats_vec_kernel<ET, false, 1, POL>;
    return masked ? row_stats_vec_kernel<ET, true, 0, POL> : row_stats_vec_kernel<ET, false, 0, POL>;
}

template <typename ET>
RowStatsFn pick_row_stats(bool masked, bool aligned, int topk, bool cached) {
    if (aligned) {
        return cached ? pick_row_stats_vec<ET, 0>(masked, topk)
                      : pick_row_stats_vec<ET, SDV_LOGITS_CACHE_POLICY>(masked, topk);
    }
    if (topk) return masked ? row_stats_elem_kernel<ET, true, 1> : row_stats_elem_kernel<ET, false, 1>;
    return masked ? row_stats_elem_kernel<ET, true, 0> : row_stats_elem_kernel<ET, false, 0>;
}

using TopkFn = void (*)(TopkArgs);
using LinesFn = void (*)(LinesArgs);

template <typename ET>
LinesFn pick_topk_lines(bool masked, bool topp) {
    if (topp) return masked ? topk_lines_kernel<ET, true, true> : topk_lines_kernel<ET, false, true>;
    return masked ? topk_lines_kernel<ET, true, false> : topk_lines_kernel<ET, false, false>;
}
using DenseFn = void (*)(FinalArgs);

template <typename ET>
DenseFn pick_dense_mass(bool aligned) {
    return aligned ? dense_mass_kernel<ET, true> : dense_mass_kernel<ET, false>;
}

template <typename ET>
DenseFn pick_dense_draw(bool aligned) {
    return aligned ? dense_draw_kernel<ET, true> : dense_draw_kernel<ET, false>;
}

template <typename ET, bool TOPP>
TopkFn pick_topk_p(bool aligned, bool masked) {
    if (aligned) return masked ? topk_kernel<ET, true, true, TOPP> : topk_kernel<ET, true, false, TOPP>;
    return masked ? topk_kernel<ET, false, true, TOPP> : topk_kernel<ET, false, false, TOPP>;
}

// Kernels without top-p leave its masses and fp64 registers out.
template <typename ET>
TopkFn pick_topk(bool aligned, bool masked, bool topp) {
    return topp ? pick_topk_p<ET, true>(aligned, masked) : pick_topk_p<ET, false>(aligned, masked);
}

template <typename ET>
FinalFn pick_final(bool aligned, bool dense, bool split) {
    if (dense && split)
        return aligned ? finalize_kernel<ET, true, true, true> : finalize_kernel<ET, false, true, true>;
    if (dense) return aligned ? finalize_kernel<ET, true, true, false> : finalize_kernel<ET, false, true, false>;
    return aligned ? finalize_kernel<ET, true, false, false> : finalize_kernel<ET, false, false, false>;
}

// Workgroups of kThreads threads of `kernel` that the current device holds
// at once, at most per_cu_max per CU (0 when the runtime cannot say); the
// runtime's answer is cached per device and kernel.
inline int64_t resident_workgroups(const void *kernel, int threads, int per_cu_max) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, std::pair<int, int>> cache;  // (CUs, per CU)
    std::lock_guard<std::mutex> lock(mu);
    const auto key = std::make_pair(dev, kernel);
    auto it = cache.find(key);
    if (it == cache.end()) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess)
            return 0;
        it = cache.emplace(key, std::make_pair(cus, per_cu)).first;
    }
    return int64_t(it->second.first) * std::min(it->second.second, per_cu_max);
}

// The single-pass top-k holds a row's line maxima in its threads' registers:
// top-k calls whose rows have at most kLinesMax lines (bf16 V <= 262144, fp32
// V <= 131072) take it, others the two-pass selection.
inline bool lines_fit(const sd_params *p) {
    const int64_t C = (int64_t(p->vocab) + kBlock - 1) / kBlock;
    return p->top_k != nullptr && C * (p->logits_dtype == SD_DTYPE_BF16 ? 32 : 64) <= kLinesMax;
}

struct Layout {
    int64_t rows;
    int C, W, nchunk;
    size_t off_sweep, off_bstats, off_drec, off_tau, off_tauflag, off_jobs, off_wmass, off_rowreq, off_offok, off_tally,
        off_linemax, off_klist, off_kcount, total;
    int nslot;
};

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

inline bool sizes_ok(const sd_params *p) {
    return p && p->batch >= 0 && p->batch <= SD_MAX_BATCH && p->num_draft >= 0 &&
           p->num_draft <= SD_MAX_DRAFT &&
           p->vocab >= 1 && p->vocab <= SD_MAX_VOCAB &&
           (!p->draft_offsets ||
            (p->total_drafts >= 0 && p->total_drafts <= int64_t(p->batch) * p->num_draft));
}

// Slots of the counter tally: about sqrt(B), at most 256.
inline int tally_slots(int B) {
    int s = 1;
    while (s < 256 && s * s < B) ++s;
    return s;
}

inline Layout layout_of(const sd_params *p) {
    Layout L{};
    L.rows = p->draft_offsets ? p->total_drafts + p->batch : int64_t(p->batch) * (p->num_draft + 1);
    L.C = (p->vocab + kBlock - 1) / kBlock;
    L.W = (p->vocab + 31) / 32;
    L.nchunk = (L.C + SDV_BLOCKS_PER_WAVE - 1) / SDV_BLOCKS_PER_WAVE;
    // the sweep's claim counters first, at the same place for every size
    L.off_sweep = 0;
    L.off_bstats = size_t(kSweepParts) * kSweepCtrStride * sizeof(uint32_t);
    L.off_drec = L.off_bstats + align256(size_t(L.rows) * L.C * sizeof(BlockStat));
    L.off_tau = L.off_drec + align256(size_t(L.rows) * sizeof(DraftRec));
    L.off_tauflag = L.off_tau + align256(size_t(L.rows) * sizeof(float));
    L.off_jobs = L.off_tauflag + align256(size_t(L.rows) * sizeof(uint32_t));
    L.off_wmass = L.off_jobs + align256(size_t(p->batch) * sizeof(DenseJob));
    L.off_rowreq = L.off_wmass + align256(size_t(p->batch) * L.C * sizeof(double));
    L.off_offok = L.off_rowreq + align256(p->draft_offsets ? size_t(L.rows) * sizeof(int32_t) : 0);
    L.off_tally = L.off_offok + 256;
    L.nslot = tally_slots(p->batch);
    L.off_linemax = L.off_tally + align256(size_t(L.nslot) * kTallyStride * sizeof(uint64_t));
    // line maxima of the single-pass top-k: one code per 128-byte line of
    // every row (2 bytes per 64 bf16 tokens, 4 per 32 fp32 tokens)
    const size_t line_bytes = lines_fit(p) ? size_t(L.rows) * L.C *
                                                 (p->logits_dtype == SD_DTYPE_BF16 ? kBlock / 64 * 2 : kBlock / 32 * 4)
                                           : 0;
    L.off_klist = L.off_linemax + align256(line_bytes);
    // with them, each row's list of the lines that hold a kept token
    const size_t nlist = lines_fit(p) ? size_t(L.rows) : 0;
    L.off_kcount = L.off_klist + align256(nlist * kCandLines * sizeof(uint16_t));
    L.total = L.off_kcount + align256(nlist * sizeof(uint32_t));
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
        case SD_ERR_SCRATCH_LIMIT: return "call needs more workspace than the static scratch holds";
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
    if (p->draft_offsets &&
        (p->total_drafts < 0 || p->total_drafts > int64_t(p->batch) * p->num_draft))
        return SD_ERR_INVALID_ARG;
    if (p->logits_dtype != SD_DTYPE_F32 && p->logits_dtype != SD_DTYPE_BF16) return SD_ERR_INVALID_ARG;
    if (!sizes_ok(p)) return SD_ERR_UNSUPPORTED;
    const int B = p->batch, k = p->num_draft, V = p->vocab;
    if (B == 0) {
        hipLaunchKernelGGL(empty_batch_kernel, dim3(1), dim3(64), 0, stream, out_counters, p->status,
                           p->dbg_flags, p->accept_histogram, k);
        return hipGetLastError() == hipSuccess ? SD_OK : SD_ERR_HIP;
    }
    if (!target_logits || !temperature || !out_tokens || !out_num_accepted) return SD_ERR_INVALID_ARG;
    const bool ragged = p->draft_offsets != nullptr;
    if ((ragged ? p->total_drafts > 0 : k > 0) && !draft_token_ids) return SD_ERR_INVALID_ARG;
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
    ra.q = draft_probs;
    ra.seed = seed;
    const bool thresholds = p->top_k != nullptr || p->top_p != nullptr;
    // top-k (with or without top-p) on aligned rows: the thresholds are found
    // after the sweep from its line maxima, with no second pass over the rows
    // that top-k cuts
    const bool single_pass = p->top_k != nullptr && aligned && lines_fit(p);
    float *tau_arr = reinterpret_cast<float *>(ws + L.off_tau);
    ra.tau = (thresholds && !single_pass) ? tau_arr : nullptr;
    ra.top_k = p->top_k;
    ra.top_p = single_pass ? p->top_p : nullptr;
    ra.linemax = single_pass ? static_cast<void *>(ws + L.off_linemax) : nullptr;
    uint32_t *tau_flag = reinterpret_cast<uint32_t *>(ws + L.off_tauflag);
    int32_t *row_req = reinterpret_cast<int32_t *>(ws + L.off_rowreq);
    uint32_t *off_ok = reinterpret_cast<uint32_t *>(ws + L.off_offok);
    ra.off = p->draft_offsets;
    ra.row_req = ragged ? row_req : nullptr;
    ra.off_ok = ragged ? off_ok : nullptr;
    // the vector sweep checks and maps a ragged call itself when nothing
    // before it needs the row table and the call fits its LDS
    ra.fold = ragged && aligned && !(thresholds && !single_pass) && L.rows <= kFoldRows && B <= kFoldReqs;
    ra.B = B;
    ra.total = ragged ? p->total_drafts : 0;
    ra.row_req_out = row_req;
    ra.off_ok_out = off_ok;
    ra.bstats = reinterpret_cast<BlockStat *>(ws + L.off_bstats);
    ra.drec = reinterpret_cast<DraftRec *>(ws + L.off_drec);
    ra.tally = reinterpret_cast<unsigned long long *>(ws + L.off_tally);
    ra.ntally = L.nslot;
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
    ra.sweep = reinterpret_cast<uint32_t *>(ws + L.off_sweep);
    ra.divC = div_magic(L.C);
    ra.divK = div_magic(k + 1);

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
    fa.tally = ra.tally;
    fa.nslot = L.nslot;
    fa.dbg_lse = p->dbg_row_lse;
    fa.dbg_acc = p->dbg_accept_prob;
    fa.dbg_req_flags = p->dbg_request_flags;
    fa.dbg_flags = p->dbg_flags;
    fa.status = p->status;
    fa.bstats = ra.bstats;
    fa.drec = ra.drec;
    fa.tau = thresholds ? tau_arr : nullptr;
    fa.tau_flag = tau_flag;
    fa.off = ra.off;
    fa.off_ok = ra.off_ok;
    fa.jobs = reinterpret_cast<DenseJob *>(ws + L.off_jobs);
    fa.wmass = reinterpret_cast<double *>(ws + L.off_wmass);
    // dense q after the single-pass selection: the rows' kept-line lists
    const bool listed = draft_probs != nullptr && single_pass;
    uint16_t *klist = listed ? reinterpret_cast<uint16_t *>(ws + L.off_klist) : nullptr;
    uint32_t *kcount = listed ? reinterpret_cast<uint32_t *>(ws + L.off_kcount) : nullptr;
    fa.klist = klist;
    fa.kcount = kcount;
    // Long rows: the residual masses of the rejected rows are summed by a
    // grid over (request, block); short rows are summed inside the finalize
    // kernel, which saves two launches.
    fa.split_dense = (draft_probs && L.C >= kDenseSplitBlocks) ? 1 : 0;
    fa.sweep = ra.sweep;
    fa.B = B;
    fa.k = k;
    fa.V = V;
    fa.W = L.W;
    fa.C = L.C;

    const int topk = single_pass ? 2 : (thresholds ? 1 : 0);
    const bool cached = L.rows * int64_t(V) * (bf16 ? 2 : 4) <= SDV_CACHED_LOGITS_BYTES;
    RowStatsFn k1 = bf16 ? pick_row_stats<uint16_t>(masked, aligned, topk, cached)
                         : pick_row_stats<float>(masked, aligned, topk, cached);
    const int k1_threads = aligned ? kSweepThreads : kThreads;
    const int64_t waves_per_wg = k1_threads / kWave;
    int64_t grid1;
    if (aligned && ra.nblk >= (int64_t(1) << 31)) return SD_ERR_UNSUPPORTED;  // block indices are 31-bit
    if (aligned) {
        // The resident capacity at three waves per SIMD (each with a block in
        // flight while it reduces another, they keep HBM busy; a fourth, where
        // the registers allow it, measured slower), a multiple of 8 (the
        // sweep's partition layout), and no more than two blocks per wave need.
        const int per_cu_max = std::max<int>(1, SDV_SWEEP_WAVES_PER_SIMD * kSimdsPerCu / int(waves_per_wg));
        int64_t cap = resident_workgroups(reinterpret_cast<const void *>(k1), k1_threads, per_cu_max);
        if (cap < 8) cap = SDV_SWEEP_WAVES / waves_per_wg;
        const int64_t need = (ra.nblk + 2 * waves_per_wg - 1) / (2 * waves_per_wg);
        grid1 = (std::min(cap, need) + 7) / 8 * 8;
        ra.parts_log2 = 0;  // partitions: a power of two, at most the wave slots per XCD
        while ((int64_t(2) << ra.parts_log2) <= std::min<int64_t>(kSweepParts, grid1 / 8 * waves_per_wg))
            ++ra.parts_log2;
        const int64_t per_wave = ra.nblk / (grid1 * waves_per_wg);
        int64_t S = masked ? per_wave * SDV_MASKED_STATIC_PCT / 100 : SDV_SWEEP_STATIC;
        S = std::max<int64_t>(2, std::min<int64_t>(S, 1 << 20)) & ~int64_t(1);
        ra.sweep_static = int(S);
    } else {
        grid1 = (ra.ntasks + waves_per_wg - 1) / waves_per_wg;
    }
    if (grid1 > INT_MAX) return SD_ERR_UNSUPPORTED;
    FinalFn k2 = bf16 ? pick_final<uint16_t>(aligned, draft_probs != nullptr, fa.split_dense != 0)
                      : pick_final<float>(aligned, draft_probs != nullptr, fa.split_dense != 0);

    if (ragged && !ra.fold) {
        hipLaunchKernelGGL(ragged_prep_kernel, dim3(1), dim3(kPrepThreads), 0, stream, p->draft_offsets, B, k,
                           p->total_drafts, row_req, off_ok);
        if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    }
    if (thresholds && !single_pass) {
        TopkArgs ta;
        ta.logits = target_logits;
        ta.mask = ra.mask;
        ta.temperature = temperature;
        ta.top_k = p->top_k;
        ta.tau = tau_arr;
        ta.tau_flag = tau_flag;
        ta.top_p = p->top_p;
        ta.off = ra.off;
        ta.row_req = ra.row_req;
        ta.off_ok = ra.off_ok;
        ta.kp1 = k + 1;
        ta.V = V;
        ta.W = L.W;
        const bool topp = p->top_p != nullptr;
        const TopkFn k0 = bf16 ? pick_topk<uint16_t>(aligned, masked, topp) : pick_topk<float>(aligned, masked, topp);
        hipLaunchKernelGGL(k0, dim3(static_cast<unsigned>(L.rows)), dim3(kTopkThreads), 0, stream, ta);
        if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    }
    const sd_debug_timing *dt = p->debug_timing;
    if (dt && dt->kernel_begin && hipEventRecord(static_cast<hipEvent_t>(dt->kernel_begin), stream) != hipSuccess)
        return SD_ERR_HIP;
    hipLaunchKernelGGL(k1, dim3(static_cast<unsigned>(grid1)), dim3(k1_threads), 0, stream, ra);
    if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    if (dt && dt->kernel_end && hipEventRecord(static_cast<hipEvent_t>(dt->kernel_end), stream) != hipSuccess)
        return SD_ERR_HIP;
    if (single_pass) {
        LinesArgs la;
        la.logits = target_logits;
        la.mask = ra.mask;
        la.temperature = temperature;
        la.top_k = p->top_k;
        la.top_p = p->top_p;
        la.draft = draft_token_ids;
        la.linemax = ra.linemax;
        la.bstats = ra.bstats;
        la.drec = ra.drec;
        la.tau = tau_arr;
        la.tau_flag = tau_flag;
        la.klist = klist;
        la.kcount = kcount;
        la.off = ra.off;
        la.row_req = ra.row_req;
        la.off_ok = ra.off_ok;
        la.seed = seed;
        la.kp1 = k + 1;
        la.V = V;
        la.W = L.W;
        la.C = L.C;
        const bool topp = p->top_p != nullptr;
        const LinesFn k5 = bf16 ? pick_topk_lines<uint16_t>(masked, topp) : pick_topk_lines<float>(masked, topp);
        hipLaunchKernelGGL(k5, dim3(static_cast<unsigned>(L.rows)), dim3(kLinesThreads), 0, stream, la);
        if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    }
    const size_t dyn_lds =
        (draft_probs && (!fa.split_dense || listed))
            ? size_t(L.C) * sizeof(double) + (listed ? size_t(kResLines) * (sizeof(double) + sizeof(int)) : 0)
            : 0;
    hipLaunchKernelGGL(k2, dim3(B), dim3(kFinalThreads), dyn_lds, stream, fa);
    if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    if (fa.split_dense && !listed) {
        const DenseFn k3 = bf16 ? pick_dense_mass<uint16_t>(aligned) : pick_dense_mass<float>(aligned);
        const DenseFn k4 = bf16 ? pick_dense_draw<uint16_t>(aligned) : pick_dense_draw<float>(aligned);
        const unsigned gx = static_cast<unsigned>((L.C + kThreads / kWave - 1) / (kThreads / kWave));
        hipLaunchKernelGGL(k3, dim3(gx, static_cast<unsigned>(B)), dim3(kThreads), 0, stream, fa);
        if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
        hipLaunchKernelGGL(k4, dim3(B), dim3(kFinalThreads), 0, stream, fa);
        if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    }
    if (p->accept_histogram) {
        hipLaunchKernelGGL(histogram_kernel, dim3(1), dim3(1024), 0, stream, out_num_accepted, B, k,
                           p->accept_histogram);
        if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    }
    return SD_OK;
}

// ------------------------------------------------------ allocation-free entry

namespace sdv {

// The workspace of sd_verify_noalloc, one copy on every device the library
// runs on.  In host code this name stands for a host-side shadow, not for a
// device address: the address of the copy on the current device comes from
// hipGetSymbolAddress, and only that address reaches a kernel.
static __device__ __align__(256) unsigned char scratch[SD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxScratchDevices = 64;
constexpr int kClaimWords = kSweepParts * kSweepCtrStride;  // the workspace's first 16 KB

struct ScratchSlot {
    void *ptr = nullptr;  // device address of `scratch` on this device
    bool clear = false;   // its block-claim counters are known to be zero
};

std::mutex scratch_mu;
ScratchSlot scratch_slots[kMaxScratchDevices];

__global__ __launch_bounds__(256) void clear_words_kernel(uint32_t *p, int n) {
    for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

}  // namespace sdv

extern "C" int sd_verify_noalloc(const void *target_logits, const int32_t *draft_token_ids,
                                 const float *draft_probs, const int32_t *bitmask,
                                 const float *temperature, uint64_t seed, int32_t *out_tokens,
                                 int32_t *out_num_accepted, uint64_t *out_counters, const sd_params *p,
                                 hipStream_t stream) {
    using namespace sdv;
    if (!p || !out_counters) return SD_ERR_INVALID_ARG;
    // 0 for B = 0 and for sizes sd_verify refuses itself
    if (sd_verify_workspace_size(p) > size_t(SD_NOALLOC_SCRATCH_BYTES)) return SD_ERR_SCRATCH_LIMIT;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxScratchDevices) return SD_ERR_HIP;
    void *ws = nullptr;
    bool clear = false;
    {
        std::lock_guard<std::mutex> lock(scratch_mu);
        ScratchSlot &slot = scratch_slots[dev];
        if (!slot.ptr) {  // set-up, once per device, with that device current
            void *ptr = nullptr;
            if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return SD_ERR_HIP;
            slot.ptr = ptr;
        }
        ws = slot.ptr;
        clear = slot.clear;
    }
    if (!clear) {  // a fill kernel, not a memset, so that a captured graph replays it correctly
        hipLaunchKernelGGL(clear_words_kernel, dim3(kClaimWords / 256), dim3(256), 0, stream,
                           static_cast<uint32_t *>(ws), kClaimWords);
        if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    }
    const int rc = sd_verify(target_logits, draft_token_ids, draft_probs, bitmask, temperature, seed,
                             out_tokens, out_num_accepted, out_counters, p, ws,
                             size_t(SD_NOALLOC_SCRATCH_BYTES), stream);
    {
        // every call that launched leaves the counters at zero; after a
        // launch failure the next call clears them again
        std::lock_guard<std::mutex> lock(scratch_mu);
        scratch_slots[dev].clear = (rc != SD_ERR_HIP);
    }
    return rc;
}
