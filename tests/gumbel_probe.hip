// Writes the device Gumbel variates for every possible uniform: for
// n = 0 .. 2^23 - 1 (u = (2n + 1) 2^-24, the word w = n << 9), the fp32 form
// (gumbel_of) and the double form (gumbel_wide) of csrc/philox.h, as two
// little-endian float64 arrays in the file named on the command line.
// tests/test_gpu_gumbel.py compares them with -ln(-ln u) from NumPy.
#include <hip/hip_runtime.h>

#include <cstdio>
#include <vector>

#include "../rejection_sampling_verification_amd/csrc/philox.h"

namespace {
constexpr int kN = 1 << 23;

__global__ void variates(double *g32, double *gwide) {
    const int n = blockIdx.x * blockDim.x + threadIdx.x;
    if (n >= kN) return;
    const uint32_t w = static_cast<uint32_t>(n) << 9;
    g32[n] = static_cast<double>(sdv::gumbel_of(w));
    gwide[n] = sdv::gumbel_wide(w);
}
}  // namespace

int main(int argc, char **argv) {
    if (argc != 2) {
        std::fprintf(stderr, "usage: %s OUT\n", argv[0]);
        return 1;
    }
    double *d = nullptr;
    if (hipMalloc(&d, size_t(2) * kN * sizeof(double)) != hipSuccess) return 2;
    hipLaunchKernelGGL(variates, dim3(kN / 256), dim3(256), 0, 0, d, d + kN);
    std::vector<double> h(size_t(2) * kN);
    if (hipDeviceSynchronize() != hipSuccess ||
        hipMemcpy(h.data(), d, h.size() * sizeof(double), hipMemcpyDeviceToHost) != hipSuccess)
        return 3;
    hipFree(d);
    FILE *f = std::fopen(argv[1], "wb");
    if (!f) return 4;
    const size_t put = std::fwrite(h.data(), sizeof(double), h.size(), f);
    std::fclose(f);
    return put == h.size() ? 0 : 5;
}
