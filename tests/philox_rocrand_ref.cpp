// Host-side reference outputs of rocRAND's Philox4x32-10 (header-only engine),
// used only to pin the oracle's Philox.  Reads lines "seed subsequence offset n"
// from stdin and prints n 32-bit outputs in hex per line.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>

int main() {
    unsigned long long seed, subseq, offset;
    int n;
    while (std::scanf("%llu %llu %llu %d", &seed, &subseq, &offset, &n) == 4) {
        rocrand_state_philox4x32_10 st;
        rocrand_init(seed, subseq, offset, &st);
        for (int i = 0; i < n; ++i) std::printf("%08x%c", rocrand(&st), i + 1 == n ? '\n' : ' ');
    }
    return 0;
}
