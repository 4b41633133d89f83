// Host driver run under AddressSanitizer and UndefinedBehaviorSanitizer by
// tests/test_sanitizers_host.py (built with the host compilers, no GPU): it
// exercises the oracle (oracle/oracle.c), the library's table builder
// (csrc/lut_build.cpp) and the M = 8 copy choice (csrc/replica.h) over every
// table width, odd shapes, padded leading dimensions, transposes, strides,
// paddings, sampled outputs and chunked FP32 sums, so that an out-of-bounds
// access or undefined behaviour on any of these paths stops the run. It also
// checks that the two table builders agree, and returns non-zero on any
// mismatch.
#include <algorithm>
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "../approximate_multiplier_dnn_amd/csrc/replica.h"
#include "../include/approx_mul.h"

extern "C" {
float orc_mul_exact(float a, float b);
float orc_mul_mitchell(float a, float b);
int orc_lut_generate(int M, float (*approx_mul)(float, float), uint16_t* lut);
void orc_lut_perturb(int M, uint16_t* lut, const int8_t* delta);
uint32_t orc_cast_bits(uint32_t x, int E);
uint32_t orc_amsim_bits_fmt(uint32_t a, uint32_t b, const uint16_t* lut, int M, int E);
void orc_amsim_many(int64_t count, const uint32_t* a, const uint32_t* b, const uint16_t* lut, int M, int E,
                    uint32_t* out);
double orc_mul_native(float a, float b);
void orc_gemm(int transA, int transB, int m, int n, int k, const float* A, int lda, const float* B, int ldb,
              const uint16_t* lut, int M, int E, double* R, double* S);
void orc_gemm_at(int transA, int transB, int m, int n, int k, const float* A, int lda, const float* B, int ldb,
                 const uint16_t* lut, int M, int E, int64_t count, const int32_t* rows, const int32_t* cols,
                 double* R, double* S);
void orc_gemm_f32_at(int transA, int transB, int m, int n, int k, const float* A, int lda, const float* B, int ldb,
                     const uint16_t* lut, int M, int E, int64_t count, const int32_t* rows, const int32_t* cols,
                     const int64_t* chunk, float* out);
void orc_conv2d_fwd(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                    const float* x, const float* w, const uint16_t* lut, int M, int E, int64_t count,
                    const int64_t* idx, double* Y, double* YS);
void orc_conv2d_dgrad(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                      const float* dy, const float* w, const uint16_t* lut, int M, int E, int64_t count,
                      const int64_t* idx, double* DX, double* DXS);
void orc_conv2d_wgrad(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                      const float* x, const float* dy, const uint16_t* lut, int M, int E, int64_t count,
                      const int64_t* idx, double* DW, double* DWS);
void orc_conv2d_f32(int pass, int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
                    const float* t1, const float* t2, const uint16_t* lut, int M, int E, int64_t count,
                    const int64_t* idx, const int64_t* chunk, float* out);
}

namespace {

uint64_t g_state = 0x9E3779B97F4A7C15ull;

// xorshift64* (Vigna): test data only
uint64_t next_u64()
{
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return g_state * 0x2545F4914F6CDD1Dull;
}

float next_float()
{
    // mostly moderate values, a few special or extreme ones
    const uint64_t r = next_u64();
    switch (r % 64) {
    case 0: return 0.0f;
    case 1: return -0.0f;
    case 2: return INFINITY;
    case 3: return -INFINITY;
    case 4: return NAN;
    case 5: return 1.0e-41f;              // subnormal
    case 6: return 3.0e38f;
    default: break;
    }
    const double u = (double)((r >> 11) & ((1ull << 40) - 1)) / (double)(1ull << 40);
    return (float)((u - 0.5) * 8.0);
}

std::vector<float> floats(size_t n)
{
    std::vector<float> v(n);
    for (auto& x : v) x = next_float();
    return v;
}

float my_model(float a, float b) { return a * b * 0.75f + 0.5f; }   // products in [1, 4): a valid model

int g_fail = 0;
#define CHECK(cond, ...)                     \
    do {                                     \
        if (!(cond)) {                       \
            std::fprintf(stderr, __VA_ARGS__); \
            std::fprintf(stderr, "\n");      \
            ++g_fail;                        \
        }                                    \
    } while (0)

void tables()
{
    for (int M = 1; M <= 11; ++M) {
        const size_t n = (size_t)1 << (2 * M);
        std::vector<uint16_t> a(n), b(n);
        CHECK(orc_lut_generate(M, orc_mul_exact, a.data()) == 0, "orc exact M=%d", M);
        CHECK(approx_lut_build(APPROX_MODEL_EXACT, M, nullptr, b.data()) == APPROX_OK, "lib exact M=%d", M);
        CHECK(a == b, "exact tables differ at M=%d", M);
        CHECK(orc_lut_generate(M, orc_mul_mitchell, a.data()) == 0, "orc mitchell M=%d", M);
        CHECK(approx_lut_build(APPROX_MODEL_MITCHELL, M, nullptr, b.data()) == APPROX_OK, "lib mitchell M=%d", M);
        CHECK(a == b, "mitchell tables differ at M=%d", M);
        std::vector<int8_t> d(n);
        for (auto& x : d) x = (next_u64() & 1) ? 1 : -1;
        orc_lut_perturb(M, a.data(), d.data());
        CHECK(approx_lut_build(APPROX_MODEL_MITCHELL, M, d.data(), b.data()) == APPROX_OK, "lib perturbed M=%d", M);
        CHECK(a == b, "perturbed tables differ at M=%d", M);
        if (M <= 8) {
            CHECK(approx_lut_build_from_model(M, my_model, b.data()) == APPROX_OK, "lib model M=%d", M);
            CHECK(orc_lut_generate(M, my_model, a.data()) == 0, "orc model M=%d", M);
            CHECK(a == b, "model tables differ at M=%d", M);
        }
    }
    uint16_t t[16];
    CHECK(approx_lut_build(APPROX_MODEL_EXACT, 0, nullptr, t) == APPROX_EUNSUPPORTED, "M=0 accepted");
    CHECK(approx_lut_build(APPROX_MODEL_EXACT, 12, nullptr, t) == APPROX_EUNSUPPORTED, "M=12 accepted");
    CHECK(approx_lut_build(7, 2, nullptr, t) == APPROX_EINVAL, "unknown model accepted");
}

void products()
{
    for (int M = 1; M <= 11; ++M) {
        std::vector<uint16_t> lut((size_t)1 << (2 * M));
        orc_lut_generate(M, orc_mul_mitchell, lut.data());
        const int count = 4000;
        std::vector<uint32_t> a(count), b(count), o(count);
        for (int i = 0; i < count; ++i) {
            a[i] = (uint32_t)next_u64();
            b[i] = (uint32_t)next_u64();
        }
        for (int E = 1; E <= 8; ++E) {
            orc_amsim_many(count, a.data(), b.data(), lut.data(), M, E, o.data());
            for (int i = 0; i < 64; ++i) (void)orc_cast_bits(a[i], E);
        }
    }
    for (int i = 0; i < 1000; ++i) (void)orc_mul_native(next_float(), next_float());
}

void gemms()
{
    std::vector<uint16_t> lut(1 << 14);
    orc_lut_generate(7, orc_mul_mitchell, lut.data());
    const int shapes[][3] = {{1, 1, 1}, {3, 5, 7}, {17, 4, 33}, {9, 13, 0}, {40, 2, 70}};
    for (const auto& sh : shapes) {
        const int m = sh[0], n = sh[1], k = sh[2];
        for (int tA = 0; tA < 2; ++tA)
            for (int tB = 0; tB < 2; ++tB)
                for (int native = 0; native < 2; ++native) {
                    const int lda = (tA ? m : k) + 3, ldb = (tB ? k : n) + 2;
                    const int arows = tA ? k : m, brows = tB ? n : k;
                    std::vector<float> A = floats((size_t)arows * lda + 1), B = floats((size_t)brows * ldb + 1);
                    const uint16_t* t = native ? nullptr : lut.data();
                    const int MM = native ? 0 : 7;
                    std::vector<double> R((size_t)m * n), S((size_t)m * n);
                    orc_gemm(tA, tB, m, n, k, A.data(), lda, B.data(), ldb, t, MM, 8, R.data(), S.data());
                    const int cnt = 7;
                    std::vector<int32_t> rows(cnt), cols(cnt);
                    std::vector<int64_t> ch(cnt);
                    for (int i = 0; i < cnt; ++i) {
                        rows[i] = (int32_t)(next_u64() % (uint64_t)m);
                        cols[i] = (int32_t)(next_u64() % (uint64_t)n);
                        ch[i] = 1 + (int64_t)(next_u64() % 9);
                    }
                    std::vector<double> r(cnt), s(cnt);
                    std::vector<float> f(cnt);
                    orc_gemm_at(tA, tB, m, n, k, A.data(), lda, B.data(), ldb, t, MM, 6, cnt, rows.data(),
                                cols.data(), r.data(), s.data());
                    orc_gemm_f32_at(tA, tB, m, n, k, A.data(), lda, B.data(), ldb, t, MM, 8, cnt, rows.data(),
                                    cols.data(), ch.data(), f.data());
                }
    }
}

void convs()
{
    std::vector<uint16_t> lut(1 << 6);
    orc_lut_generate(3, orc_mul_mitchell, lut.data());
    // N, H, W, C, K, R, S, sh, sw, ph, pw
    const int geoms[][11] = {{2, 5, 6, 3, 2, 3, 3, 1, 1, 1, 1}, {1, 7, 4, 2, 5, 3, 2, 2, 1, 0, 1},
                             {1, 3, 3, 1, 1, 3, 3, 1, 1, 2, 2}, {2, 8, 9, 4, 3, 4, 3, 3, 2, 1, 0}};
    for (const auto& g : geoms) {
        const int N = g[0], H = g[1], W = g[2], C = g[3], K = g[4], R = g[5], S = g[6];
        const int sh = g[7], sw = g[8], ph = g[9], pw = g[10];
        const int P = (H + 2 * ph - R) / sh + 1, Q = (W + 2 * pw - S) / sw + 1;
        std::vector<float> x = floats((size_t)N * H * W * C), w = floats((size_t)R * S * C * K),
                           dy = floats((size_t)N * P * Q * K);
        const int64_t ny = (int64_t)N * P * Q * K, nx = (int64_t)N * H * W * C, nw = (int64_t)R * S * C * K;
        std::vector<double> a(std::max({ny, nx, nw})), b(a.size());
        orc_conv2d_fwd(N, H, W, C, K, R, S, sh, sw, ph, pw, x.data(), w.data(), lut.data(), 3, 8, 0, nullptr,
                       a.data(), b.data());
        orc_conv2d_dgrad(N, H, W, C, K, R, S, sh, sw, ph, pw, dy.data(), w.data(), lut.data(), 3, 7, 0, nullptr,
                         a.data(), b.data());
        orc_conv2d_wgrad(N, H, W, C, K, R, S, sh, sw, ph, pw, x.data(), dy.data(), nullptr, 0, 8, 0, nullptr,
                         a.data(), b.data());
        const int64_t totals[3] = {ny, nx, nw};
        for (int pass = 0; pass < 3; ++pass) {
            const int64_t cnt = totals[pass];
            std::vector<int64_t> idx(cnt), ch(cnt);
            for (int64_t i = 0; i < cnt; ++i) {
                idx[i] = i;
                ch[i] = 4 * (1 + (int64_t)(next_u64() % 5));
            }
            std::vector<float> out(cnt);
            const float* t1 = pass == 1 ? dy.data() : x.data();
            const float* t2 = pass == 2 ? dy.data() : w.data();
            orc_conv2d_f32(pass, N, H, W, C, K, R, S, sh, sw, ph, pw, t1, t2, lut.data(), 3, 8, cnt, idx.data(),
                           ch.data(), out.data());
        }
    }
}

void copies()
{
    const uint32_t pad_w = 512;
    for (int it = 0; it < 20000; ++it) {
        uint32_t w[32];
        const int count = 1 + (int)(next_u64() % 32);
        for (int l = 0; l < 32; ++l) {
            const uint64_t r = next_u64();
            w[l] = (r % 10 == 0) ? pad_w : (uint32_t)(2 * (r % 256));
        }
        uint32_t before[32];
        std::memcpy(before, w, sizeof(w));
        const int top = amx::rep8_assign_group(w, count, pad_w);
        CHECK(top >= 1 && top <= 32, "busiest bank %d", top);
        for (int l = 0; l < 32; ++l) CHECK(w[l] < (uint32_t)amx::kRep8ColBytes, "offset %u out of a column", w[l]);
        for (int l = count; l < 32; ++l) CHECK(w[l] == before[l], "lane %d beyond the group was changed", l);
    }
}

}  // namespace

int main()
{
    tables();
    products();
    gemms();
    convs();
    copies();
    std::printf("sanitizer driver: %d failures\n", g_fail);
    return g_fail ? 1 : 0;
}
