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

#include "sd_verify.h"
#include "philox.h"
#include "wave.h"

#ifndef SDV_BLOCKS_PER_WAVE
#define SDV_BLOCKS_PER_WAVE 4
#endif

namespace sdv {

constexpr int kBlock = SD_BLOCK_TOKENS;
constexpr int kThreads = 256;
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

// ------------------------------------------------------------ row statistics

struct RowStatsArgs {
    const void *logits;
    const uint32_t *mask;  // nullptr = no bitmask
    const float *temperature;
    float2 *bstats;        // [rows, C]
    uint32_t *ticket;
    int64_t ntasks;        // rows * nchunk
    int kp1, V, W, C, cpw, nchunk;
};

template <int G, int P>
__device__ __forceinline__ float2 softmax_block(const float *v, float c) {
    constexpr int NV = G * P;
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

template <int G, int P>
__device__ __forceinline__ float2 greedy_block(const float *v, int64_t base) {
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
            if (v[g * P + e] == m) idx = static_cast<int>(base + g * kWave * P + e);
    return make_float2(m, __int_as_float(wave_min_i(idx)));
}

template <typename ET, bool MASKED, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void row_stats_kernel(RowStatsArgs a) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);  // 16-byte groups per lane per block
    if (blockIdx.x == 0 && threadIdx.x == 0) *a.ticket = 0u;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t task = int64_t(blockIdx.x) * (kThreads / kWave) + (threadIdx.x >> 6);
    if (task >= a.ntasks) return;
    const int row = static_cast<int>(task / a.nchunk);
    const int chunk = static_cast<int>(task - int64_t(row) * a.nchunk);
    const float T = a.temperature[row / a.kp1];
    const bool greedy = (T == 0.0f);
    if (!greedy && !(T > 0.0f && T <= FLT_MAX)) return;  // reported by finalize
    const float c = greedy ? 0.0f : scale_of(T);
    const ET *rowp = reinterpret_cast<const ET *>(a.logits) + int64_t(row) * a.V;
    const uint8_t *mrow =
        MASKED ? reinterpret_cast<const uint8_t *>(a.mask + int64_t(row) * a.W) : nullptr;
    float2 *out = a.bstats + int64_t(row) * a.C;
    const int c0 = chunk * a.cpw;
    const int c1 = min(a.C, c0 + a.cpw);
    for (int blk = c0; blk < c1; ++blk) {
        const int64_t base = int64_t(blk) * kBlock + lane * P;
        float v[G * P];
#pragma unroll
        for (int g = 0; g < G; ++g) load_group<ET, ALIGNED>(rowp, base + g * kWave * P, a.V, v + g * P);
        if (MASKED) {
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const uint32_t bits = mask_bits<P>(mrow, base + g * kWave * P, a.V);
#pragma unroll
                for (int e = 0; e < P; ++e)
                    if (!((bits >> e) & 1u)) v[g * P + e] = -INFINITY;
            }
        }
        const float2 r = greedy ? greedy_block<G, P>(v, base) : softmax_block<G, P>(v, c);
        if (lane == 0) out[blk] = r;
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
    int32_t *rec;  // [B, kRecordWords]
    uint32_t *ticket;
    int B, k, V, W, C;
};

enum SampleMode { kModeP = 0, kModeOneHot = 1, kModeDense = 2 };

struct FinalShared {
    float M[kMaxDraft + 1];   // per row: fp32 max (log2 units) or greedy max logit
    double S[kMaxDraft + 1];  // per row: sum of 2^(t - M)
    int G[kMaxDraft + 1];     // greedy argmax
    int X[kMaxDraft];
    double acc[kMaxDraft];
    unsigned char ok[kMaxDraft], flag[kMaxDraft], invalid[kMaxDraft];
    uint32_t status;
    int nacc, flag_acc, ninvalid, last;
    double red_d[4];
    Top2 red_t[4];
    unsigned long long red_u[4][4];
    uint32_t red_s[4];
};

// Per-block residual masses of row `row` for dense q: W_c = sum_j max(p_j - q_j, 0)
// with p_j = 2^(l_j c - M) / S, evaluated in fp32.  One wave per block.
template <typename ET, bool ALIGNED>
__device__ void dense_block_masses(const ET *rowp, const uint32_t *mrow, const float *qrow, int V,
                                   int C, float c, float M, double S, double *Wout) {
    constexpr int P = Logit<ET>::kPer16;
    constexpr int G = kBlock / (kWave * P);
    const int lane = threadIdx.x & (kWave - 1);
    const float invS = static_cast<float>(1.0 / S);
    for (int blk = threadIdx.x >> 6; blk < C; blk += kThreads / kWave) {
        const int64_t base = int64_t(blk) * kBlock + lane * P;
        float acc = 0.0f;
#pragma unroll
        for (int g = 0; g < G; ++g) {
            const int64_t tok = base + g * kWave * P;
            float lv[P];
            load_group<ET, ALIGNED>(rowp, tok, V, lv);
            float qv[P];
#pragma unroll
            for (int h = 0; h < P / 4; ++h) {
                if (ALIGNED) {
                    if (tok < V) {
                        const float4 f = *reinterpret_cast<const float4 *>(qrow + tok + 4 * h);
                        qv[4 * h] = f.x; qv[4 * h + 1] = f.y; qv[4 * h + 2] = f.z; qv[4 * h + 3] = f.w;
                    } else {
                        qv[4 * h] = qv[4 * h + 1] = qv[4 * h + 2] = qv[4 * h + 3] = 0.0f;
                    }
                } else {
#pragma unroll
                    for (int e = 0; e < 4; ++e)
                        qv[4 * h + e] = (tok + 4 * h + e < V) ? qrow[tok + 4 * h + e] : 0.0f;
                }
            }
            const uint32_t bits =
                mrow ? mask_bits<P>(reinterpret_cast<const uint8_t *>(mrow), tok, V) : 0xffu;
#pragma unroll
            for (int e = 0; e < P; ++e) {
                const bool live = ((bits >> e) & 1u) && lv[e] > -INFINITY;
                const float p = live ? __builtin_amdgcn_exp2f(fmaf(lv[e], c, -M)) * invS : 0.0f;
                acc += fmaxf(p - qv[e], 0.0f);
            }
        }
        const double w = wave_sum_d(static_cast<double>(acc));
        if (lane == 0) Wout[blk] = w;
    }
}

// Draw the emitted token of sampled row n of request b; all threads call it
// and all get the token.  Adds the number of near-tie flags to *flags.
template <typename ET, bool ALIGNED>
__device__ int sample_row(const FinalArgs &a, FinalShared &sh, double *sW, int b, int n, float c,
                          float T, int *flags) {
    const int k = a.k, V = a.V, C = a.C;
    const int64_t row = int64_t(b) * (k + 1) + n;
    const ET *rowp = reinterpret_cast<const ET *>(a.logits) + row * V;
    const uint32_t *mrow = a.mask ? a.mask + row * a.W : nullptr;
    const float2 *st = a.bstats + row * C;
    const PhiloxKey key = key_of(a.seed);
    const float M = sh.M[n];
    const double S = sh.S[n];
    const int x = (n < k) ? sh.X[n] : -1;
    const float *qrow = (n < k && a.q) ? a.q + (int64_t(b) * k + n) * V : nullptr;
    int mode = (n == k) ? kModeP : (qrow ? kModeDense : kModeOneHot);
    const int tid = threadIdx.x;

    for (int attempt = 0; attempt < 2; ++attempt) {
        // ---- level 1: block masses and their Gumbel keys
        int cx = -1;
        double wx = 0.0;
        if (mode == kModeOneHot) {  // the draft's own block, recomputed without the draft
            cx = x / kBlock;
            const int64_t j0 = int64_t(cx) * kBlock + tid * 8;
            float lv[8];
            load8_masked<ET, ALIGNED>(rowp, mrow, j0, V, lv);
            double s = 0.0;
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (lv[e] > -INFINITY && j0 + e != x)
                    s += exp2(static_cast<double>(lv[e]) * c - static_cast<double>(M));
            wx = block_sum_d(s, sh.red_d);
        } else if (mode == kModeDense) {
            dense_block_masses<ET, ALIGNED>(rowp, mrow, qrow, V, C, c, M, S, sW);
            __syncthreads();
        }
        Top2 t = top2_empty();
        for (int cb = tid; cb < C; cb += kThreads) {
            double w;
            if (mode == kModeDense) {
                w = sW[cb];
            } else if (cb == cx) {
                w = wx;
            } else {
                const float2 e = st[cb];
                w = e.x > -INFINITY ? static_cast<double>(e.y) *
                                          exp2(static_cast<double>(e.x) - static_cast<double>(M))
                                    : 0.0;
            }
            if (w > 0.0) top2_push(t, log(w) + draw_block_gumbel(key, b, n, cb), cb);
        }
        t = block_top2(t, sh.red_t);
        if (t.k1 == -INFINITY) {  // no residual mass: draw from p instead
            mode = kModeP;
            continue;
        }
        int nflag = (t.k2 > -INFINITY && t.k1 - t.k2 < kGumbelFlagEps) ? 1 : 0;

        // ---- level 2: tokens of the winning block
        const int64_t j0 = int64_t(t.i1) * kBlock + tid * 8;
        float lv[8];
        load8_masked<ET, ALIGNED>(rowp, mrow, j0, V, lv);
        double g[8];
        draw_token_gumbels8(key, b, n, static_cast<uint32_t>(j0), g);
        Top2 t2 = top2_empty();
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const int64_t j = j0 + e;
            if (!(lv[e] > -INFINITY)) continue;  // masked, -inf, or beyond V
            double kk;
            if (mode == kModeDense) {
                const double p = exp2(static_cast<double>(lv[e]) * c - static_cast<double>(M)) / S;
                const double r = p - static_cast<double>(qrow[j]);
                if (!(r > 0.0)) continue;
                kk = log(r) + g[e];
            } else {
                if (mode == kModeOneHot && j == x) continue;
                kk = static_cast<double>(lv[e]) / static_cast<double>(T) + g[e];
            }
            top2_push(t2, kk, static_cast<int>(j));
        }
        t2 = block_top2(t2, sh.red_t);
        if (t2.k1 == -INFINITY) {  // the block lost its mass in double precision
            mode = kModeP;
            continue;
        }
        nflag += (t2.k2 > -INFINITY && t2.k1 - t2.k2 < kGumbelFlagEps) ? 1 : 0;
        *flags += nflag;
        return t2.i1;
    }
    return -1;  // unreachable: a row that passed validation has mass under p
}

template <typename ET, bool ALIGNED>
__global__ __launch_bounds__(kThreads) void finalize_kernel(FinalArgs a) {
    __shared__ FinalShared sh;
    extern __shared__ double sW[];  // dense q: per-block residual mass [C]
    const int b = blockIdx.x;
    const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid >> 6;
    const int k = a.k, kp1 = a.k + 1, V = a.V, C = a.C;
    const float T = a.temperature[b];
    const bool greedy = (T == 0.0f);
    const PhiloxKey key = key_of(a.seed);

    if (tid == 0) {
        sh.status = (greedy || (T > 0.0f && T <= FLT_MAX)) ? 0u : SD_STATUS_TEMPERATURE;
        sh.nacc = 0;
        sh.flag_acc = 0;
        sh.ninvalid = 0;
    }
    __syncthreads();
    if (tid < k) {
        const int x = a.draft[int64_t(b) * k + tid];
        sh.X[tid] = x;
        if (x < 0 || x >= V) atomicOr(&sh.status, SD_STATUS_DRAFT_ID);
    }
    __syncthreads();
    const float c = greedy ? 0.0f : scale_of(T);

    // ---- fold block statistics into per-row max / normaliser / argmax
    if (!(sh.status & SD_STATUS_TEMPERATURE)) {
        for (int i = wave; i < kp1; i += kThreads / kWave) {
            const float2 *st = a.bstats + (int64_t(b) * kp1 + i) * C;
            bool bad = false;
            if (greedy) {
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
            } else {
                float mx = -INFINITY;
                for (int cb = lane; cb < C; cb += kWave) {
                    const float2 e = st[cb];
                    if (e.x != e.x || e.y != e.y || e.x == INFINITY) bad = true;
                    mx = fmaxf(mx, e.x);
                }
                bad = wave_any(bad);
                const float m = wave_max(mx);
                double s = 0.0;
                if (!bad && m > -INFINITY) {
                    for (int cb = lane; cb < C; cb += kWave) {
                        const float2 e = st[cb];
                        if (e.x > -INFINITY)
                            s += static_cast<double>(e.y) *
                                 exp2(static_cast<double>(e.x) - static_cast<double>(m));
                    }
                }
                s = wave_sum_d(s);
                if (lane == 0) {
                    sh.M[i] = m;
                    sh.S[i] = s;
                    sh.G[i] = -1;
                    if (bad) atomicOr(&sh.status, SD_STATUS_BAD_LOGIT);
                    else if (m == -INFINITY) atomicOr(&sh.status, SD_STATUS_EMPTY_ROW);
                }
            }
        }
    }
    __syncthreads();

    // ---- per-position accept probabilities and verdicts
    if (sh.status == 0 && tid < k) {
        const int i = tid, x = sh.X[i];
        const int64_t rowi = int64_t(b) * kp1 + i;
        bool allowed = true;
        if (a.mask) allowed = (a.mask[rowi * a.W + (x >> 5)] >> (x & 31)) & 1u;
        sh.invalid[i] = !allowed;
        double acc;
        bool ok, flag = false;
        if (greedy) {
            ok = (x == sh.G[i]);
            acc = ok ? 1.0 : 0.0;
        } else {
            const float lx = load_one<ET>(a.logits, rowi * V + x);
            double p = 0.0;
            if (allowed && lx > -INFINITY)
                p = exp2(static_cast<double>(lx) * c - static_cast<double>(sh.M[i])) / sh.S[i];
            double q = 1.0;
            if (a.q) {
                const float qf = a.q[(int64_t(b) * k + i) * V + x];
                if (!(qf >= 0.0f && qf <= FLT_MAX)) atomicOr(&sh.status, SD_STATUS_BAD_DRAFT_PROB);
                q = qf;
            }
            acc = (p == 0.0) ? 0.0 : (q == 0.0 ? 1.0 : fmin(1.0, p / q));
            const double u = draw_accept(key, b, i);
            ok = u < acc;
            flag = fabs(u - acc) < kAcceptFlagEps;
        }
        sh.acc[i] = acc;
        sh.ok[i] = ok;
        sh.flag[i] = flag;
    }
    __syncthreads();
    if (tid == 0 && sh.status == 0) {
        int n = 0, fa = 0, inv = 0;
        while (n < k && sh.ok[n]) fa += sh.flag[n++];
        if (n < k) fa += sh.flag[n];
        for (int i = 0; i < k; ++i) inv += sh.invalid[i];
        sh.nacc = n;
        sh.flag_acc = fa;
        sh.ninvalid = inv;
    }
    __syncthreads();

    // ---- the emitted token
    const uint32_t st = sh.status;
    int y = -1, fg = 0;
    if (st == 0) {
        const int n = sh.nacc;
        if (greedy)
            y = sh.G[n];
        else
            y = sample_row<ET, ALIGNED>(a, sh, sW, b, n, c, T, &fg);
    }

    // ---- outputs and the per-request record
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
        int32_t *r = a.rec + int64_t(b) * kRecordWords;
        r[0] = st ? 0 : k;
        r[1] = st ? 0 : sh.ninvalid;
        r[2] = st ? 0 : n;
        r[3] = static_cast<int32_t>(st);
        r[4] = st ? 0 : sh.flag_acc;
        r[5] = st ? 0 : fg;
        if (a.dbg_req_flags)
            a.dbg_req_flags[b] = st ? 0u : (uint32_t(min(sh.flag_acc, 0xffff)) | (uint32_t(fg) << 16));
    }

    // ---- the last workgroup to finish sums the records in request order
    __threadfence();
    __syncthreads();
    if (tid == 0) sh.last = (atomicAdd(a.ticket, 1u) == uint32_t(a.B - 1));
    __syncthreads();
    if (!sh.last) return;
    __threadfence();
    unsigned long long R = 0, I = 0, A = 0, FA = 0, FG = 0;
    uint32_t S = 0;
    for (int r = tid; r < a.B; r += kThreads) {
        const int32_t *rr = a.rec + int64_t(r) * kRecordWords;
        R += uint32_t(__hip_atomic_load(rr + 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        I += uint32_t(__hip_atomic_load(rr + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        A += uint32_t(__hip_atomic_load(rr + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        S |= uint32_t(__hip_atomic_load(rr + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        FA += uint32_t(__hip_atomic_load(rr + 4, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
        FG += uint32_t(__hip_atomic_load(rr + 5, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    }
    R = wave_sum_u64(R);
    I = wave_sum_u64(I);
    A = wave_sum_u64(A);
    FA = wave_sum_u64(FA);
    FG = wave_sum_u64(FG);
    S = wave_or_u32(S);
    if (lane == 0) {
        sh.red_u[wave][0] = R;
        sh.red_u[wave][1] = I;
        sh.red_u[wave][2] = A;
        sh.red_u[wave][3] = (FA & 0xffffffffull) | (FG << 32);
        sh.red_s[wave] = S;
    }
    __syncthreads();
    if (tid == 0) {
        unsigned long long tr = 0, ti = 0, ta = 0, tfa = 0, tfg = 0;
        uint32_t ts = 0;
        for (int w = 0; w < kThreads / kWave; ++w) {
            tr += sh.red_u[w][0];
            ti += sh.red_u[w][1];
            ta += sh.red_u[w][2];
            tfa += sh.red_u[w][3] & 0xffffffffull;
            tfg += sh.red_u[w][3] >> 32;
            ts |= sh.red_s[w];
        }
        a.out_counters[0] = tr;
        a.out_counters[1] = ti;
        a.out_counters[2] = tr - ti;
        a.out_counters[3] = ta;
        if (a.status) *a.status = ts;
        if (a.dbg_flags) {
            a.dbg_flags[0] = static_cast<uint32_t>(tfa);
            a.dbg_flags[1] = static_cast<uint32_t>(tfg);
        }
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
    if (masked) return aligned ? row_stats_kernel<ET, true, true> : row_stats_kernel<ET, true, false>;
    return aligned ? row_stats_kernel<ET, false, true> : row_stats_kernel<ET, false, false>;
}

template <typename ET>
FinalFn pick_final(bool aligned) {
    return aligned ? finalize_kernel<ET, true> : finalize_kernel<ET, false>;
}

struct Layout {
    int64_t rows;
    int C, W, nchunk;
    size_t off_bstats, off_rec, off_ticket, total;
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
    L.off_rec = align256(size_t(L.rows) * L.C * sizeof(float2));
    L.off_ticket = L.off_rec + align256(size_t(p->batch) * kRecordWords * sizeof(int32_t));
    L.total = L.off_ticket + 256;
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
    ra.bstats = reinterpret_cast<float2 *>(ws + L.off_bstats);
    ra.ticket = reinterpret_cast<uint32_t *>(ws + L.off_ticket);
    ra.ntasks = L.rows * L.nchunk;
    ra.kp1 = k + 1;
    ra.V = V;
    ra.W = L.W;
    ra.C = L.C;
    ra.cpw = SDV_BLOCKS_PER_WAVE;
    ra.nchunk = L.nchunk;
    const int64_t waves_per_wg = kThreads / kWave;
    const int64_t grid1 = (ra.ntasks + waves_per_wg - 1) / waves_per_wg;
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
    fa.rec = reinterpret_cast<int32_t *>(ws + L.off_rec);
    fa.ticket = ra.ticket;
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
    hipLaunchKernelGGL(k2, dim3(B), dim3(kThreads), dyn_lds, stream, fa);
    if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
    return SD_OK;
}
