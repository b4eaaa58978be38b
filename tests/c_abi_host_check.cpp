// Host-side logic of the C ABI under AddressSanitizer, with no GPU: the
// argument checks of every entry point (each refused call returns before any
// HIP call), the workspace sizes over the whole range of supported shapes
// (the layout arithmetic and the division constants behind it), the rates
// helper and the status strings.  Built by tests/test_host_asan.py with
// AddressSanitizer on the host code only, linked with the library's sources.
// Prints "host checks ok" and exits 0, or names the first failed check and
// exits 1.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "sd_ngram.h"
#include "sd_verify.h"

namespace {

int failures = 0;

void check(bool ok, const char *what) {
    if (!ok) {
        std::fprintf(stderr, "FAILED: %s\n", what);
        ++failures;
    }
}

sd_params params(int B, int k, int V, sd_dtype dt) {
    sd_params p;
    std::memset(&p, 0, sizeof p);
    p.batch = B;
    p.num_draft = k;
    p.vocab = V;
    p.logits_dtype = dt;
    return p;
}

}  // namespace

int main() {
    // device-looking addresses, never dereferenced on the host
    void *fake = reinterpret_cast<void *>(uintptr_t(1) << 20);
    int32_t *fi = static_cast<int32_t *>(fake);
    float *ff = static_cast<float *>(fake);
    uint64_t counters[4];

    // workspace sizes: 0 for unsupported shapes, 256-byte multiples that grow
    // with the shape otherwise
    const int Bs[] = {1, 2, 63, 64, 65, 255, 256, 1000, 4096, SD_MAX_BATCH};
    const int ks[] = {0, 1, 4, 12, 63, SD_MAX_DRAFT};
    const int Vs[] = {1, 2, 7, 8, 2047, 2048, 2049, 32000, 131072, 151936, 262144, SD_MAX_VOCAB};
    for (int B : Bs)
        for (int k : ks)
            for (int V : Vs)
                for (sd_dtype dt : {SD_DTYPE_BF16, SD_DTYPE_F32}) {
                    sd_params p = params(B, k, V, dt);
                    const size_t ws = sd_verify_workspace_size(&p);
                    check(ws > 0 && ws % 256 == 0, "workspace size of a supported shape");
                    const int32_t one = 1;
                    p.top_k = &one;  // a host address is fine: never read on the host
                    const size_t wk = sd_verify_workspace_size(&p);
                    check(wk >= ws && wk % 256 == 0, "workspace size with top-k");
                    p.top_k = nullptr;
                    p.draft_offsets = reinterpret_cast<const int32_t *>(fake);
                    p.total_drafts = int64_t(B) * k;
                    check(sd_verify_workspace_size(&p) > 0, "ragged workspace size");
                    p.total_drafts = int64_t(B) * k + 1;
                    check(sd_verify_workspace_size(&p) == 0, "ragged total above B * k");
                }
    {
        sd_params p = params(0, 4, 100, SD_DTYPE_BF16);
        check(sd_verify_workspace_size(&p) == 0, "B = 0");
        p = params(4, SD_MAX_DRAFT + 1, 100, SD_DTYPE_BF16);
        check(sd_verify_workspace_size(&p) == 0, "k too large");
        p = params(4, 4, SD_MAX_VOCAB + 1, SD_DTYPE_BF16);
        check(sd_verify_workspace_size(&p) == 0, "V too large");
        p = params(SD_MAX_BATCH + 1, 4, 100, SD_DTYPE_BF16);
        check(sd_verify_workspace_size(&p) == 0, "B too large");
        check(sd_verify_workspace_size(nullptr) == 0, "null parameters");
    }

    // sd_verify refuses bad calls on the host
    {
        sd_params p = params(4, 3, 100, SD_DTYPE_BF16);
        check(sd_verify(nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr, counters, nullptr,
                        nullptr, 0, nullptr) == SD_ERR_INVALID_ARG, "null parameters");
        check(sd_verify(nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr, nullptr, &p, nullptr,
                        0, nullptr) == SD_ERR_INVALID_ARG, "null counters");
        check(sd_verify(nullptr, nullptr, nullptr, nullptr, nullptr, 0, nullptr, nullptr, counters, &p, nullptr,
                        0, nullptr) == SD_ERR_INVALID_ARG, "missing tensors");
        p.logits_dtype = static_cast<sd_dtype>(7);
        check(sd_verify(fake, fi, nullptr, nullptr, ff, 0, fi, fi, counters, &p, fake, 1 << 20,
                        nullptr) == SD_ERR_INVALID_ARG, "bad dtype");
        p = params(4, SD_MAX_DRAFT + 1, 100, SD_DTYPE_BF16);
        check(sd_verify(fake, fi, nullptr, nullptr, ff, 0, fi, fi, counters, &p, fake, 1 << 20,
                        nullptr) == SD_ERR_UNSUPPORTED, "k too large");
        p = params(4, 3, 100, SD_DTYPE_BF16);
        check(sd_verify(fake, fi, nullptr, nullptr, ff, 0, fi, fi, counters, &p, fake, 16, nullptr) ==
                  SD_ERR_WORKSPACE, "workspace too small");
        p.draft_offsets = reinterpret_cast<const int32_t *>(fake);
        p.total_drafts = 13;
        check(sd_verify(fake, fi, nullptr, nullptr, ff, 0, fi, fi, counters, &p, fake, 1 << 20,
                        nullptr) == SD_ERR_INVALID_ARG, "ragged total above B * k");
        p = params(8192, 12, 151936, SD_DTYPE_BF16);
        check(sd_verify_workspace_size(&p) > SD_NOALLOC_SCRATCH_BYTES, "a shape beyond the static scratch");
        check(sd_verify_noalloc(fake, fi, nullptr, nullptr, ff, 0, fi, fi, counters, &p, nullptr) ==
                  SD_ERR_SCRATCH_LIMIT, "noalloc refuses a shape beyond its scratch");
        check(sd_verify_noalloc(fake, fi, nullptr, nullptr, ff, 0, fi, fi, counters, nullptr, nullptr) ==
                  SD_ERR_INVALID_ARG, "noalloc without parameters");
    }

    // sd_ngram_propose refuses bad calls on the host
    {
        sd_ngram_params p;
        std::memset(&p, 0, sizeof p);
        p.batch = 4;
        p.min_n = 2;
        p.max_n = 5;
        p.num_draft = 4;
        p.stride = 5000;
        check(sd_ngram_workspace_size(&p) > 0, "n-gram workspace size");
        check(sd_ngram_propose(fi, fi, fi, fi, &p, nullptr, 0, nullptr) == SD_ERR_WORKSPACE,
              "n-gram without workspace");
        p.max_n = SD_NGRAM_MAX_N + 1;
        check(sd_ngram_workspace_size(&p) == 0, "n-gram max_n too large");
        check(sd_ngram_propose(fi, fi, fi, fi, &p, nullptr, 0, nullptr) == SD_ERR_UNSUPPORTED,
              "n-gram max_n too large");
        p.max_n = 1;
        check(sd_ngram_propose(fi, fi, fi, fi, &p, nullptr, 0, nullptr) == SD_ERR_INVALID_ARG,
              "n-gram max_n below min_n");
        check(sd_ngram_propose(fi, fi, fi, fi, nullptr, nullptr, 0, nullptr) == SD_ERR_INVALID_ARG,
              "n-gram null parameters");
    }

    // rates and status strings
    {
        const uint64_t c[4] = {1000, 200, 800, 600};
        double r[4] = {0, 0, 0, 0};
        check(sd_rates(c, 100, r) == SD_OK, "rates");
        check(r[0] == 0.8 && r[1] == 0.75 && r[2] == 0.6, "rates values");
        const uint64_t bad[4] = {10, 2, 9, 1};
        check(sd_rates(bad, 1, r) != SD_OK, "rates with D != R - I");
        check(sd_rates(nullptr, 1, r) == SD_ERR_INVALID_ARG, "rates without counters");
        for (int code = -10; code <= 1; ++code) check(sd_status_string(code) != nullptr, "status string");
    }

    if (failures) return 1;
    std::printf("host checks ok\n");
    return 0;
}
