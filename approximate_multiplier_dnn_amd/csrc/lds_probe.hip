// lds_probe.hip -- measures the LDS rate of 16-bit table lookups on gfx950
// for the access patterns of the GEMM kernel: one 2^M-entry table column per
// instruction (the uniform operand's), rows chosen per lane (the lane
// operand's). Prints lookups per clock per CU at 2.4 GHz for: every lane on
// one entry (broadcast), consecutive entries, random rows of a 256-byte
// column (M = 7), random rows of a 512-byte column (M = 8), and M = 8 rows
// drawn with the density of normally distributed mantissas.
//
// Each workgroup stages a 132,096-byte table image (256 columns of 258
// entries) in LDS; every address read is inside it (row offset < 516 bytes,
// column offset <= 15 * 7 * 516 bytes).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

namespace {

constexpr int kImageU16 = 66048;
constexpr int kThreads = 1024;
constexpr int kOffsets = 16;

__global__ __launch_bounds__(kThreads) void probe(const uint16_t* img, const uint32_t* offs, int iters, uint32_t* out)
{
    __shared__ __align__(16) uint16_t lut[kImageU16];
    for (int i = threadIdx.x; i < kImageU16; i += kThreads) lut[i] = img[i];
    __syncthreads();
    uint32_t wa[kOffsets];
#pragma unroll
    for (int j = 0; j < kOffsets; ++j) wa[j] = offs[threadIdx.x * kOffsets + j] + (uint32_t)(uintptr_t)lut;
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
        uint32_t r[kOffsets];
#pragma unroll
        for (int j = 0; j < kOffsets; ++j)
            asm volatile("ds_read_u16 %0, %1 offset:%2" : "=v"(r[j]) : "v"(wa[j]), "i"(((j * 7) % 16) * 7 * 516) : "memory");
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int j = 0; j < kOffsets; j += 2) acc += r[j] ^ r[j + 1];
    }
    out[blockIdx.x * kThreads + threadIdx.x] = acc;
}

#define CHECK(x)                                                                              \
    do {                                                                                      \
        hipError_t e_ = (x);                                                                  \
        if (e_ != hipSuccess) {                                                               \
            std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));               \
            return 1;                                                                         \
        }                                                                                     \
    } while (0)

}  // namespace

int main()
{
    int cus = 0;
    CHECK(hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, 0));
    const int grid = cus, iters = 20000;
    std::vector<uint16_t> img(kImageU16);
    for (int i = 0; i < kImageU16; ++i) img[i] = (uint16_t)(i * 2654435761u >> 16);
    uint16_t* dimg = nullptr;
    uint32_t *doffs = nullptr, *dout = nullptr;
    CHECK(hipMalloc(&dimg, kImageU16 * 2));
    CHECK(hipMemcpy(dimg, img.data(), kImageU16 * 2, hipMemcpyHostToDevice));
    CHECK(hipMalloc(&doffs, kThreads * kOffsets * 4));
    CHECK(hipMalloc(&dout, (size_t)grid * kThreads * 4));
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    const char* names[] = {"broadcast", "consecutive", "random rows, 256-byte column (M=7)",
                           "random rows, 512-byte column (M=8)", "normal-mantissa rows, M=8"};
    std::printf("pattern | T lookups/s | lookups/clk/CU (2.4 GHz)\n");
    for (int mode = 0; mode < 5; ++mode) {
        std::vector<uint32_t> offs(kThreads * kOffsets);
        uint64_t s = 12345 + mode;
        for (int t = 0; t < kThreads; ++t)
            for (int j = 0; j < kOffsets; ++j) {
                s = s * 6364136223846793005ULL + 1442695040888963407ULL;
                const uint32_t r = (uint32_t)(s >> 33);
                uint32_t e;
                if (mode == 0) e = 5;
                else if (mode == 1) e = t & 63;
                else if (mode == 2) e = r % 128;
                else if (mode == 3) e = r % 256;
                else {
                    const double u = (r + 0.5) / 2147483648.0;   // mantissa density ~ 1 / (1 + x)
                    e = (uint32_t)((std::pow(2.0, u) - 1.0) * 256.0);
                    if (e > 255) e = 255;
                }
                offs[t * kOffsets + j] = e * 2;
            }
        CHECK(hipMemcpy(doffs, offs.data(), offs.size() * 4, hipMemcpyHostToDevice));
        hipLaunchKernelGGL(probe, dim3(grid), dim3(kThreads), 0, 0, dimg, doffs, 10, dout);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(a));
        hipLaunchKernelGGL(probe, dim3(grid), dim3(kThreads), 0, 0, dimg, doffs, iters, dout);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(b));
        CHECK(hipEventSynchronize(b));
        float ms = 0.0f;
        CHECK(hipEventElapsedTime(&ms, a, b));
        const double lookups = (double)grid * kThreads * iters * kOffsets;
        std::printf("%s | %.2f | %.1f\n", names[mode], lookups / ms / 1e9, lookups / (ms * 1e-3) / cus / 2.4e9);
    }
    return 0;
}
