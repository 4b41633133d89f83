// lut_build.cpp -- host-side mantissa-product table generation
// ("ApproxTrain", arXiv 2209.04161, Section V-A, Algorithm 1).
//
// For every pair of M-bit mantissas the multiplier's C model is run on the
// two operands 1.ia and 1.ib (sign +, unit exponent, so neither they nor the
// product is special). The carry is whether the product's binary exponent
// is above the un-normalised one (product in [2, 4) rather than [1, 2)); the
// entry keeps the carry in bit 15 and the first 15 bits of the product's
// fraction (chopped) in bits 14..0.
#include <cmath>
#include <cstdint>

#include "../../include/approx_mul.h"

namespace {

// The exact multiplier: the FP32 product, exact for M <= 11 because two
// (M+1)-bit significands multiply into at most 24 bits.
float model_exact(float a, float b) { return a * b; }

// Mitchell's logarithmic multiplier (J. N. Mitchell, 1962): with
// |a| = (1+x) 2^ea and |b| = (1+y) 2^eb, log2(1+x) is replaced by x, so the
// product is (1+x+y) 2^(ea+eb) if x+y < 1 and 2(x+y) 2^(ea+eb) otherwise.
float model_mitchell(float a, float b)
{
    int ea = 0, eb = 0;
    const float ma = std::frexp(std::fabs(a), &ea);   // |a| = ma * 2^ea, ma in [0.5, 1)
    const float mb = std::frexp(std::fabs(b), &eb);
    const float x = 2.0f * ma - 1.0f;                  // |a| = (1 + x) * 2^(ea - 1)
    const float y = 2.0f * mb - 1.0f;
    const float s = x + y;
    const float sig = s < 1.0f ? 1.0f + s : 2.0f * s;
    const float mag = std::ldexp(sig, (ea - 1) + (eb - 1));
    return (std::signbit(a) != std::signbit(b)) ? -mag : mag;
}

int build(int M, float (*mul)(float, float), uint16_t* out)
{
    const uint32_t side = 1u << M;
    const float step = std::ldexp(1.0f, -M);
    for (uint32_t ia = 0; ia < side; ++ia) {
        const float a = 1.0f + (float)ia * step;
        for (uint32_t ib = 0; ib < side; ++ib) {
            const float b = 1.0f + (float)ib * step;
            const float c = mul(a, b);
            if (!(c >= 1.0f && c < 4.0f)) return APPROX_EUNSUPPORTED;
            int e = 0;
            (void)std::frexp(c, &e);                  // c in [1,2): e = 1; [2,4): e = 2
            const uint32_t carry = (uint32_t)(e - 1);
            const float frac = std::ldexp(c, -(int)carry) - 1.0f;     // exact
            const uint32_t f15 = (uint32_t)std::ldexp(frac, 15);      // chop to 15 bits
            out[(ia << M) | ib] = (uint16_t)((carry << 15) | f15);
        }
    }
    return APPROX_OK;
}

}  // namespace

extern "C" int approx_lut_build(int model, int M, const int8_t* perturb, uint16_t* lut_out)
{
    if (lut_out == nullptr) return APPROX_EINVAL;
    if (M < 1 || M > 11) return APPROX_EUNSUPPORTED;
    float (*mul)(float, float) = nullptr;
    if (model == APPROX_MODEL_EXACT) mul = model_exact;
    else if (model == APPROX_MODEL_MITCHELL) mul = model_mitchell;
    else return APPROX_EINVAL;
    const int rc = build(M, mul, lut_out);
    if (rc != APPROX_OK) return rc;
    if (perturb != nullptr) {
        const uint32_t count = 1u << (2 * M);
        for (uint32_t i = 0; i < count; ++i) {
            int f = (lut_out[i] & 0x7FFF) + perturb[i];
            f = f < 0 ? 0 : (f > 0x7FFF ? 0x7FFF : f);
            lut_out[i] = (uint16_t)((lut_out[i] & 0x8000) | f);
        }
    }
    return APPROX_OK;
}

extern "C" int approx_lut_build_from_model(int M, float (*mul)(float, float), uint16_t* lut_out)
{
    if (lut_out == nullptr || mul == nullptr) return APPROX_EINVAL;
    if (M < 1 || M > 11) return APPROX_EUNSUPPORTED;
    return build(M, mul, lut_out);
}
