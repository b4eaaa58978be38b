// n-gram (prompt lookup) draft proposer for gfx950.
//
// The rule (infra-guide 5.2 "Draft models and model-free methods", sections
// 4.1 and 6; pyshine "vLLM, part 2", "Choosing a drafter"): the history's last
// n tokens are looked up earlier in the same history, the longest window
// n <= max_n that occurs wins, then its earliest occurrence, and the tokens
// that followed it are proposed.
//
// The search is reorganised around the END of an occurrence.  For an end
// position e (the occurrence covers h[e - n, e), so e <= len - 1 keeps it off
// the tail itself) let c(e) be how many tokens before e agree with the tail,
// counted backwards: h[e - 1 - t] == h[len - 1 - t] for t = 0 .. c(e) - 1,
// capped at min(max_n, len - 1) and by e.  A window n occurs ending at e
// exactly when c(e) >= n, so the longest window is the largest capped c(e)
// of at least min_n, and for that window the earliest start is the smallest
// such e.  Every end position is independent: a workgroup takes a chunk of
// 2048 of them, stages the chunk (plus the max_n tokens before it) and the
// tail in LDS, and reduces the packed key (c << 32 | ~e) to its maximum, which
// orders by window length and then by earliest end.  A second one-workgroup
// kernel combines the chunks of each request, scans the draft counts into the
// ragged offsets the verifier takes and copies the drafts.
//
// Memory: each history token is read once by the chunk that holds it and at
// most once more as the halo of the next chunk; the work is a few integer
// compares per token, so the match kernel is bound by HBM and launch latency.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <limits.h>

#include "sd_ngram.h"
#include "wave.h"

namespace sdng {

using sdv::block_max_u64;
using sdv::lds_barrier;
using sdv::max_u64;

constexpr int kMatchThreads = 256;
constexpr int kMatchWaves = kMatchThreads / 64;
constexpr int kPerThread = 8;                          // end positions per thread
constexpr int kChunk = kMatchThreads * kPerThread;     // end positions per workgroup
constexpr int kStage = kChunk / kMatchThreads + 1;     // staged loads per thread: chunk + halo
static_assert(SD_NGRAM_MAX_N <= kMatchThreads, "the halo is one load per thread");

constexpr int kEmitThreads = 1024;
constexpr int kEmitWaves = kEmitThreads / 64;

__device__ __forceinline__ int uniform_i(int v) { return __builtin_amdgcn_readfirstlane(v); }

// A request takes part in the search when its length is valid, leaves room
// for its k drafts within the context length, and allows a window of min_n.
__device__ __forceinline__ bool searchable(int L, int64_t stride, int64_t max_model_len, int k, int min_n,
                                           int max_n, int &nmax) {
    nmax = min(max_n, L - 1);
    return L >= 0 && int64_t(L) <= stride && !(max_model_len > 0 && int64_t(L) + k > max_model_len) &&
           nmax >= min_n;
}

struct MatchArgs {
    const int32_t *tokens;
    const int32_t *lengths;
    unsigned long long *best;  // [B * nchunk] packed keys, 0 = no occurrence
    int64_t stride, max_model_len;
    int B, nchunk, min_n, max_n, k;
};

__global__ __launch_bounds__(kMatchThreads) void ngram_match_kernel(MatchArgs a) {
    __shared__ int32_t win[kChunk + SD_NGRAM_MAX_N];  // h[e0 - nmax + i]
    __shared__ int32_t tail[SD_NGRAM_MAX_N];          // tail[t] = h[L - 1 - t]
    __shared__ uint64_t red[kMatchWaves];
    const int task = blockIdx.x;
    const int b = task / a.nchunk;
    const int chunk = task - b * a.nchunk;
    const int tid = threadIdx.x;
    const int L = uniform_i(a.lengths[b]);
    const int64_t e0 = int64_t(chunk) * kChunk;
    int nmax = 0;
    if (!searchable(L, a.stride, a.max_model_len, a.k, a.min_n, a.max_n, nmax) || e0 >= L) {
        if (tid == 0) a.best[task] = 0ull;
        return;
    }
    const int32_t *h = a.tokens + int64_t(b) * a.stride;
    const int64_t base = e0 - nmax;
    // All loads first (indices clamped into [0, L), so none is guarded by a
    // branch and all stay in flight together), then the LDS stores.
    int32_t v[kStage];
#pragma unroll
    for (int s = 0; s < kStage; ++s) {
        int64_t j = base + s * kMatchThreads + tid;
        j = j < 0 ? 0 : (j >= L ? L - 1 : j);
        v[s] = h[j];
    }
    const int32_t tv = h[L - 1 - min(tid, nmax - 1)];
#pragma unroll
    for (int s = 0; s < kStage; ++s) {
        const int i = s * kMatchThreads + tid;
        if (i < kChunk + nmax) win[i] = v[s];
    }
    if (tid < nmax) tail[tid] = tv;
    lds_barrier();

    uint64_t key = 0;
#pragma unroll
    for (int j = 0; j < kPerThread; ++j) {
        const int64_t e = e0 + j * kMatchThreads + tid;
        if (e >= L || e < a.min_n) continue;
        const int lim = int(min(int64_t(nmax), e));
        const int32_t *w = win + (e - 1 - base);  // w[-t] = h[e - 1 - t]
        int c = 0;
        while (c < lim && w[-c] == tail[c]) ++c;
        if (c >= a.min_n) key = max_u64(key, (uint64_t(c) << 32) | (0xffffffffu - uint32_t(e)));
    }
    key = block_max_u64<kMatchWaves>(key, red);
    if (tid == 0) a.best[task] = key;
}

struct EmitArgs {
    const int32_t *tokens;
    const int32_t *lengths;
    const unsigned long long *best;
    int32_t *drafts, *num, *match, *offsets, *flat;
    uint32_t *status;
    int64_t stride;
    int B, nchunk, k;
};

// Request b's best chunk key; the keys are loaded eight at a time, all in
// flight together.
__device__ __forceinline__ uint64_t request_key(const EmitArgs &a, int b) {
    const unsigned long long *p = a.best + int64_t(b) * a.nchunk;
    uint64_t key = 0;
    int c = 0;
    for (; c + 8 <= a.nchunk; c += 8) {
        uint64_t v[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = p[c + j];
#pragma unroll
        for (int j = 0; j < 8; ++j) key = max_u64(key, v[j]);
    }
    for (; c < a.nchunk; ++c) key = max_u64(key, p[c]);
    return key;
}

// The winning window and the end of its earliest occurrence for request b,
// and how many drafts follow it.
__device__ __forceinline__ int request_result(const EmitArgs &a, int b, int L, int &n, int64_t &e) {
    const uint64_t key = request_key(a, b);
    n = int(key >> 32);
    e = int64_t(0xffffffffu - uint32_t(key));
    return n > 0 ? int(min(int64_t(a.k), int64_t(L) - e)) : 0;
}

// Threads own consecutive requests.  The draft counts are known from the
// chunk keys alone, so they are scanned into the ragged offsets first (a
// shuffle scan within each wave, then the wave totals); the history is then
// read once per draft, into the per-request slots and the packed list.
__global__ __launch_bounds__(kEmitThreads) void ngram_emit_kernel(EmitArgs a) {
    __shared__ uint32_t wtot[kEmitWaves];
    __shared__ uint32_t red[kEmitWaves];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int per = (a.B + kEmitThreads - 1) / kEmitThreads;
    const int b0 = min(tid * per, a.B), b1 = min(b0 + per, a.B);
    uint32_t total = 0, bad = 0;
    int n0 = 0, cnt0 = 0;  // the first owned request's result, kept for the copy
    int64_t e0 = 0;
    for (int b = b0; b < b1; ++b) {
        const int L = a.lengths[b];
        if (L < 0 || int64_t(L) > a.stride) bad = SD_NGRAM_STATUS_BAD_LENGTH;
        int n;
        int64_t e;
        const int cnt = request_result(a, b, L, n, e);
        if (b == b0) {
            n0 = n;
            e0 = e;
            cnt0 = cnt;
        }
        total += uint32_t(cnt);
    }
    uint32_t start = 0;
    if (a.offsets) {
        uint32_t incl = total;  // inclusive scan within the wave
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t t = static_cast<uint32_t>(__shfl_up(static_cast<int>(incl), d, 64));
            if (lane >= d) incl += t;
        }
        if (lane == 63) wtot[wave] = incl;
        lds_barrier();
        uint32_t before = 0;
        for (int w = 0; w < wave; ++w) before += wtot[w];
        start = before + incl - total;
        if (tid == kEmitThreads - 1) a.offsets[a.B] = int32_t(start + total);
    }
    for (int b = b0; b < b1; ++b) {
        int n = n0, cnt = cnt0;
        int64_t e = e0;
        if (b != b0) cnt = request_result(a, b, a.lengths[b], n, e);
        const int32_t *h = a.tokens + int64_t(b) * a.stride;
        int32_t *d = a.drafts + int64_t(b) * a.k;
        int32_t *f = (a.offsets && a.flat) ? a.flat + start : nullptr;
        for (int i = 0; i < a.k; ++i) {
            const int32_t t = i < cnt ? h[e + i] : -1;
            d[i] = t;
            if (f && i < cnt) f[i] = t;
        }
        a.num[b] = cnt;
        if (a.match) a.match[b] = n;
        if (a.offsets) a.offsets[b] = int32_t(start);
        start += uint32_t(cnt);
    }
    if (a.status) {
        bad = sdv::block_max_u<kEmitWaves>(bad, red);
        if (tid == 0) a.status[0] = bad;
    }
}

inline size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

inline int nchunk_of(int64_t stride) { return int((stride + kChunk - 1) / kChunk); }

// 0: fine; otherwise the sd_status to return.
inline int check_params(const sd_ngram_params *p) {
    if (!p) return SD_ERR_INVALID_ARG;
    if (p->batch < 0 || p->min_n < 1 || p->max_n < p->min_n || p->num_draft < 0 || p->stride < 1 ||
        p->max_model_len < 0 || (p->out_drafts_flat && !p->out_draft_offsets))
        return SD_ERR_INVALID_ARG;
    if (p->batch > SD_NGRAM_MAX_BATCH || p->max_n > SD_NGRAM_MAX_N || p->num_draft > SD_MAX_DRAFT ||
        p->stride > INT_MAX || int64_t(p->batch) * nchunk_of(p->stride) > INT_MAX)
        return SD_ERR_UNSUPPORTED;
    return 0;
}

}  // namespace sdng

extern "C" size_t sd_ngram_workspace_size(const sd_ngram_params *p) {
    using namespace sdng;
    if (check_params(p) != 0 || p->batch == 0) return 0;
    return align256(size_t(p->batch) * nchunk_of(p->stride) * sizeof(unsigned long long));
}

extern "C" int sd_ngram_propose(const int32_t *tokens, const int32_t *lengths, int32_t *out_drafts,
                                int32_t *out_num_drafts, const sd_ngram_params *p, void *workspace,
                                size_t workspace_bytes, hipStream_t stream) {
    using namespace sdng;
    const int rc = check_params(p);
    if (rc != 0) return rc;
    const int B = p->batch;
    if (B > 0 && (!tokens || !lengths || !out_num_drafts || (p->num_draft > 0 && !out_drafts)))
        return SD_ERR_INVALID_ARG;
    const int nchunk = nchunk_of(p->stride);
    const size_t need = B > 0 ? align256(size_t(B) * nchunk * sizeof(unsigned long long)) : 0;
    if (B > 0 && (!workspace || workspace_bytes < need || (reinterpret_cast<uintptr_t>(workspace) & 255u)))
        return SD_ERR_WORKSPACE;
    unsigned long long *best = static_cast<unsigned long long *>(workspace);
    if (B > 0) {
        MatchArgs m;
        m.tokens = tokens;
        m.lengths = lengths;
        m.best = best;
        m.stride = p->stride;
        m.max_model_len = p->max_model_len;
        m.B = B;
        m.nchunk = nchunk;
        m.min_n = p->min_n;
        m.max_n = p->max_n;
        m.k = p->num_draft;
        const sd_debug_timing *dt = p->debug_timing;
        if (dt && dt->kernel_begin &&
            hipEventRecord(static_cast<hipEvent_t>(dt->kernel_begin), stream) != hipSuccess)
            return SD_ERR_HIP;
        hipLaunchKernelGGL(ngram_match_kernel, dim3(unsigned(B) * unsigned(nchunk)), dim3(kMatchThreads), 0,
                           stream, m);
        if (hipGetLastError() != hipSuccess) return SD_ERR_HIP;
        if (dt && dt->kernel_end && hipEventRecord(static_cast<hipEvent_t>(dt->kernel_end), stream) != hipSuccess)
            return SD_ERR_HIP;
    }
    if (B == 0 && !p->out_draft_offsets && !p->status) return SD_OK;
    EmitArgs e;
    e.tokens = tokens;
    e.lengths = lengths;
    e.best = best;
    e.drafts = out_drafts;
    e.num = out_num_drafts;
    e.match = p->out_match_len;
    e.offsets = p->out_draft_offsets;
    e.flat = p->out_drafts_flat;
    e.status = p->status;
    e.stride = p->stride;
    e.B = B;
    e.nchunk = nchunk;
    e.k = p->num_draft;
    hipLaunchKernelGGL(ngram_emit_kernel, dim3(1), dim3(kEmitThreads), 0, stream, e);
    return hipGetLastError() == hipSuccess ? SD_OK : SD_ERR_HIP;
}
