// Calls the verifier through its C ABI alone, from C++ without Python: reads
// a workload from raw little-endian files in a directory, runs sd_verify on
// the current HIP device and writes the outputs into the same directory.
//
//   c_abi_check DIR
//
// DIR/meta.txt holds "B k V seed dense"; DIR/logits.f32 [B, k+1, V],
// DIR/drafts.i32 [B, k], DIR/temperature.f32 [B] and, when dense is 1,
// DIR/probs.f32 [B, k, V].  Written: out_tokens.i32 [B, k+1],
// num_accepted.i32 [B], counters.u64 [4], status.u32 [1], and host_checks.txt
// with the return codes of calls the host must refuse.  Exit status 0 on
// success.
#include <hip/hip_runtime_api.h>

#include <cstdint>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "sd_verify.h"

namespace {

bool read_file(const std::string &path, void *dst, size_t bytes) {
    FILE *f = std::fopen(path.c_str(), "rb");
    if (!f) return false;
    const size_t got = std::fread(dst, 1, bytes, f);
    std::fclose(f);
    return got == bytes;
}

bool write_file(const std::string &path, const void *src, size_t bytes) {
    FILE *f = std::fopen(path.c_str(), "wb");
    if (!f) return false;
    const size_t put = std::fwrite(src, 1, bytes, f);
    std::fclose(f);
    return put == bytes;
}

#define CHECK_HIP(x)                                                           \
    do {                                                                       \
        hipError_t e_ = (x);                                                   \
        if (e_ != hipSuccess) {                                                \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_)); \
            return 3;                                                          \
        }                                                                      \
    } while (0)

}  // namespace

int main(int argc, char **argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s DIR\n", argv[0]);
        return 1;
    }
    const std::string dir = argv[1];
    long long B = 0, k = 0, V = 0, dense = 0;
    unsigned long long seed = 0;
    {
        FILE *f = std::fopen((dir + "/meta.txt").c_str(), "r");
        if (!f || std::fscanf(f, "%lld %lld %lld %llu %lld", &B, &k, &V, &seed, &dense) != 5) {
            std::fprintf(stderr, "bad meta.txt\n");
            return 1;
        }
        std::fclose(f);
    }
    if (B < 1 || k < 0 || V < 1 || B * (k + 1) * V > (1ll << 28)) {
        std::fprintf(stderr, "sizes out of range for this check\n");
        return 1;
    }
    const size_t rows = size_t(B) * size_t(k + 1);
    std::vector<float> logits(rows * V), temperature(B), probs(dense ? size_t(B) * k * V : 0);
    std::vector<int32_t> drafts(size_t(B) * k);
    if (!read_file(dir + "/logits.f32", logits.data(), logits.size() * 4) ||
        !read_file(dir + "/drafts.i32", drafts.data(), drafts.size() * 4) ||
        !read_file(dir + "/temperature.f32", temperature.data(), temperature.size() * 4) ||
        (dense && !read_file(dir + "/probs.f32", probs.data(), probs.size() * 4))) {
        std::fprintf(stderr, "missing or short input file\n");
        return 1;
    }

    float *d_logits = nullptr, *d_T = nullptr, *d_probs = nullptr;
    int32_t *d_drafts = nullptr, *d_tokens = nullptr, *d_nacc = nullptr;
    uint64_t *d_counters = nullptr;
    uint32_t *d_status = nullptr;
    void *d_ws = nullptr;
    CHECK_HIP(hipMalloc(&d_logits, logits.size() * 4));
    CHECK_HIP(hipMalloc(&d_T, temperature.size() * 4));
    CHECK_HIP(hipMalloc(&d_drafts, (drafts.size() ? drafts.size() : 1) * 4));
    CHECK_HIP(hipMalloc(&d_tokens, rows * 4));
    CHECK_HIP(hipMalloc(&d_nacc, size_t(B) * 4));
    CHECK_HIP(hipMalloc(&d_counters, 4 * sizeof(uint64_t)));
    CHECK_HIP(hipMalloc(&d_status, sizeof(uint32_t)));
    if (dense) CHECK_HIP(hipMalloc(&d_probs, probs.size() * 4));
    CHECK_HIP(hipMemcpy(d_logits, logits.data(), logits.size() * 4, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(d_T, temperature.data(), temperature.size() * 4, hipMemcpyHostToDevice));
    if (!drafts.empty())
        CHECK_HIP(hipMemcpy(d_drafts, drafts.data(), drafts.size() * 4, hipMemcpyHostToDevice));
    if (dense) CHECK_HIP(hipMemcpy(d_probs, probs.data(), probs.size() * 4, hipMemcpyHostToDevice));

    sd_params p;
    std::memset(&p, 0, sizeof(p));
    p.batch = int32_t(B);
    p.num_draft = int32_t(k);
    p.vocab = int32_t(V);
    p.logits_dtype = SD_DTYPE_F32;
    p.status = d_status;
    const size_t ws = sd_verify_workspace_size(&p);
    CHECK_HIP(hipMalloc(&d_ws, ws ? ws : 256));
    CHECK_HIP(hipMemset(d_ws, 0, ws ? ws : 256));  // zero-filled before its first call

    // calls the host must refuse before launching anything
    int refused[4];
    {
        sd_params bad = p;
        bad.batch = -1;
        refused[0] = sd_verify(d_logits, d_drafts, d_probs, nullptr, d_T, seed, d_tokens, d_nacc,
                               d_counters, &bad, d_ws, ws, nullptr);
        bad = p;
        bad.num_draft = SD_MAX_DRAFT + 1;
        refused[1] = sd_verify(d_logits, d_drafts, d_probs, nullptr, d_T, seed, d_tokens, d_nacc,
                               d_counters, &bad, d_ws, ws, nullptr);
        refused[2] = sd_verify(d_logits, d_drafts, d_probs, nullptr, d_T, seed, d_tokens, d_nacc,
                               d_counters, &p, d_ws, ws ? ws - 1 : 0, nullptr);
        refused[3] = sd_verify(nullptr, d_drafts, d_probs, nullptr, d_T, seed, d_tokens, d_nacc,
                               d_counters, &p, d_ws, ws, nullptr);
    }

    hipStream_t stream;
    CHECK_HIP(hipStreamCreate(&stream));
    const int rc = sd_verify(d_logits, d_drafts, d_probs, nullptr, d_T, seed, d_tokens, d_nacc, d_counters,
                             &p, d_ws, ws, stream);
    if (rc != SD_OK) {
        std::fprintf(stderr, "sd_verify: %s (%d)\n", sd_status_string(rc), rc);
        return 2;
    }
    CHECK_HIP(hipStreamSynchronize(stream));

    std::vector<int32_t> tokens(rows), nacc(B);
    uint64_t counters[4];
    uint32_t status = 0;
    CHECK_HIP(hipMemcpy(tokens.data(), d_tokens, rows * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(nacc.data(), d_nacc, size_t(B) * 4, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(counters, d_counters, sizeof(counters), hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(&status, d_status, sizeof(status), hipMemcpyDeviceToHost));
    bool ok = write_file(dir + "/out_tokens.i32", tokens.data(), rows * 4) &&
              write_file(dir + "/num_accepted.i32", nacc.data(), size_t(B) * 4) &&
              write_file(dir + "/counters.u64", counters, sizeof(counters)) &&
              write_file(dir + "/status.u32", &status, sizeof(status));
    FILE *f = std::fopen((dir + "/host_checks.txt").c_str(), "w");
    if (f) {
        std::fprintf(f, "%d %d %d %d\n", refused[0], refused[1], refused[2], refused[3]);
        std::fclose(f);
    } else {
        ok = false;
    }
    hipStreamDestroy(stream);
    hipFree(d_ws);
    hipFree(d_logits);
    hipFree(d_T);
    hipFree(d_drafts);
    hipFree(d_tokens);
    hipFree(d_nacc);
    hipFree(d_counters);
    hipFree(d_status);
    if (d_probs) hipFree(d_probs);
    return ok ? 0 : 4;
}
