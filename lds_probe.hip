// lds_probe.hip -- measures the LDS rate of 16-bit table lookups on gfx950
// for the access patterns of the GEMM kernel: one table column per
// instruction (the uniform operand's), rows chosen per lane (the lane
// operand's). Prints lookups per second and per clock per CU (2.4 GHz) for:
// every lane on one entry (broadcast), consecutive entries, random rows of a
// 256-byte column (M = 7), random rows of a 512-byte column (M = 8), M = 8
// rows drawn with the density of normally distributed mantissas, and the
// same rows read from the 640-byte M = 8 columns with second copies, the
// copy of each row chosen per half-wave as the library's decode pass does
// (replica.h).
//
// Each workgroup stages a table image in LDS (132,096 bytes: 256 columns of
// 258 entries; or 163,840 bytes: 256 columns of 320 entries); every address
// read is inside it (row offset < 640 bytes, column offset <= 90 columns).
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "approximate_multiplier_dnn_amd/csrc/replica.h"

namespace {

constexpr int kThreads = 1024;
constexpr int kOffsets = 16;
constexpr int kMaxImageBytes = 163840;

template <int IMAGE_BYTES, int COL_BYTES>
__global__ __launch_bounds__(kThreads) void probe(const uint32_t* img, const uint32_t* offs, int iters, uint32_t* out)
{
    __shared__ __align__(16) uint32_t lut[IMAGE_BYTES / 4];
    for (int i = threadIdx.x; i < IMAGE_BYTES / 4; i += kThreads) lut[i] = img[i];
    __syncthreads();
    uint32_t wa[kOffsets];
#pragma unroll
    for (int j = 0; j < kOffsets; ++j) wa[j] = offs[threadIdx.x * kOffsets + j] + (uint32_t)(uintptr_t)lut;
    uint32_t acc = 0;
    for (int it = 0; it < iters; ++it) {
        uint32_t r[kOffsets];
#pragma unroll
        for (int j = 0; j < kOffsets; ++j)
            asm volatile("ds_read_u16 %0, %1 offset:%2" : "=v"(r[j]) : "v"(wa[j]), "i"(((j * 7) % 16) * 6 * COL_BYTES) : "memory");
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
    std::vector<uint32_t> img(kMaxImageBytes / 4);
    for (size_t i = 0; i < img.size(); ++i) img[i] = (uint32_t)(i * 2654435761u);
    uint32_t *dimg = nullptr, *doffs = nullptr, *dout = nullptr;
    CHECK(hipMalloc(&dimg, kMaxImageBytes));
    CHECK(hipMemcpy(dimg, img.data(), kMaxImageBytes, hipMemcpyHostToDevice));
    CHECK(hipMalloc(&doffs, kThreads * kOffsets * 4));
    CHECK(hipMalloc(&dout, (size_t)grid * kThreads * 4));
    hipEvent_t a, b;
    CHECK(hipEventCreate(&a));
    CHECK(hipEventCreate(&b));
    const char* names[] = {"broadcast", "consecutive", "random rows, 256-byte column (M=7)",
                           "random rows, 512-byte column (M=8)", "normal-mantissa rows, M=8",
                           "normal-mantissa rows, M=8 with second copies (chosen per half-wave)"};
    std::printf("pattern | T lookups/s | lookups/clk/CU (2.4 GHz)\n");
    for (int mode = 0; mode < 6; ++mode) {
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
        if (mode == 5) {            // each half-wave's 32 rows of one instruction: choose the copies
            for (int h = 0; h < kThreads / 32; ++h)
                for (int j = 0; j < kOffsets; ++j) {
                    uint32_t w[32];
                    for (int l = 0; l < 32; ++l) w[l] = offs[(h * 32 + l) * kOffsets + j];
                    amx::rep8_assign_group(w, 32, 2u * 256u);
                    for (int l = 0; l < 32; ++l) offs[(h * 32 + l) * kOffsets + j] = w[l];
                }
        }
        CHECK(hipMemcpy(doffs, offs.data(), offs.size() * 4, hipMemcpyHostToDevice));
        auto launch = [&](int n) {
            if (mode == 5)
                hipLaunchKernelGGL((probe<163840, 640>), dim3(grid), dim3(kThreads), 0, 0, dimg, doffs, n, dout);
            else
                hipLaunchKernelGGL((probe<132096, 516>), dim3(grid), dim3(kThreads), 0, 0, dimg, doffs, n, dout);
        };
        launch(10);
        CHECK(hipGetLastError());
        CHECK(hipEventRecord(a));
        launch(iters);
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
