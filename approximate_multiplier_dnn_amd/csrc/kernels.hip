// kernels.hip -- gfx950 kernels of the LUT-based approximate GEMM.
//
// The product of every multiply-accumulate is the AMSim approximate product
// ("ApproxTrain", arXiv 2209.04161, Section V, Algorithm 2). One call queues:
//   1. decode  : one launch for both operands; each FP32 element is decoded
//                once into a Word (table offset + sign|exponent bits), laid
//                out for step 3. This is also where implicit-GEMM layouts for
//                Conv2D are produced (zero-padded images, the padded and
//                dilated errors and the transposed, reversed filter of
//                Section VI-B).
//   2. assign  : M = 8 only: the copy of each lane operand's table row
//                (replica.h), chosen per group of 32 operands.
//   3. main    : the table is staged in LDS once per persistent workgroup;
//                each lane owns 3 or 4 rows x 16 columns of the output; per
//                MAC it forms the LDS address, reads one 16-bit entry and
//                folds it into the FP32 accumulator.
//   4. reduce  : when reductions are split, sums the chunk partials in
//                ascending chunk order (all tiles, or only the tiles of the
//                last round).
//
// Fast path (3 VALU ops + 1 LDS read per MAC). When no product of the call
// can leave the normal range, the AMSim product equals exactly
//     fma(as_float(seA + (entry << 8)), as_float(seB), acc)
// where seA/seB are the operands' sign|exponent bits: seA + (entry << 8) is
// +-(1.f) * 2^(EA-127+carry) and seB is +-2^(EB-127), so the FMA's product is
// exact and its single rounding is the rounding of acc + product. Zero, Inf
// and NaN operands are encoded (zero pad entry, se = 0 / +-Inf / NaN) so the
// same FMA produces the rule's zero, infinity and NaN cases. The exponent
// range test is made from the per-operand min/max exponents gathered by the
// decode pass. When products may fall below the range but none above it, the
// fast path zeroes those products first; otherwise the checked path
// evaluates Algorithm 2 per product.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "internal.h"

namespace amx {

// The GEMM kernel is instantiated for each workgroup shape of internal.h:
// NW waves per workgroup, RPL output rows per lane; CPW output columns per wave.
constexpr int CPW = kColsPerWave;

// Global-memory views of pointers that may come from a device pointer array:
// loaded pointers are generic (flat), and flat loads count against the LDS
// wait counter too, which would serialise every table lookup behind them.
typedef const float __attribute__((address_space(1)))* gfloat_cptr;
typedef float __attribute__((address_space(1)))* gfloat_ptr;
typedef float v4f __attribute__((ext_vector_type(4)));
typedef v4f __attribute__((address_space(1)))* gv4f_ptr;

// Dword 3 of a raw buffer descriptor on this GPU family: data format field
// (bits 18:15) = 4, 32-bit elements; every other field zero (no swizzle, no
// index stride). Raw loads then address base + scalar offset + lane offset.
constexpr int kBufferConfig = 0x00020000;

// ------------------------------------------------------------------ decode

// Exponent cast of an FP32 operand to the multiplier's format (1, E, M)
// (ApproxTrain Section V: exponent widths below 8 with a casting function):
// a normal value whose biased exponent lies below elo becomes a signed zero,
// above ehi a signed infinity; zero, subnormal, Inf and NaN are kept. The
// identity for FP32's own range (elo = 1, ehi = 254).
__device__ __forceinline__ uint32_t cast_fmt(uint32_t bits, int elo, int ehi)
{
    const int e = (int)((bits >> 23) & 0xFFu);
    const uint32_t sign = bits & 0x80000000u;
    bits = (e != 0 && e != 255 && e < elo) ? sign : bits;
    bits = (e != 0 && e != 255 && e > ehi) ? (sign | 0x7F800000u) : bits;
    return bits;
}

// M = 0 selects the native multiplier: the Word carries the operand's own
// bits (se) and no table offset, and the exponent range is not gathered (nor
// is the operand cast: the native multiplier is FP32).
__device__ __forceinline__ Word decode_bits(uint32_t bits, int M, int lane_role, int& emin, int& emax, int elo,
                                            int ehi)
{
    if (M == 0) return Word{0u, bits};
    bits = cast_fmt(bits, elo, ehi);
    const uint32_t e = (bits >> 23) & 0xFFu;
    const uint32_t frac = bits & 0x7FFFFFu;
    const uint32_t idx = frac >> (23 - M);
    const uint32_t pad = (1u << M) * 2u;            // zero entry after the column's 2^M entries
    const uint32_t colb = (uint32_t)lut_col_bytes(M);   // column stride in bytes
    Word o;
    if (e == 0u) {                                  // zero or subnormal (counts as zero)
        o.se = 0u;
        o.w = lane_role ? pad : 0u;
    } else if (e == 255u) {                         // Inf or NaN
        o.se = frac ? 0x7FC00000u : (bits & 0xFF800000u);
        o.w = lane_role ? pad : 0u;
    } else {
        o.se = bits & 0xFF800000u;
        o.w = lane_role ? idx * 2u : idx * colb;
        emin = min(emin, (int)e);
        emax = max(emax, (int)e);
    }
    return o;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f)
{
    return (__umulhi(n, f.m) + n) >> f.l;
}

__device__ __forceinline__ Word zero_word(int M, int lane_role)
{
    Word w;
    w.se = 0u;
    w.w = (lane_role && M) ? (1u << M) * 2u : 0u;
    return w;
}

// Stores decoded words: 8-byte Words for a table; for the native multiplier
// (wbytes 4) only the operand's own bits, the se half of its Word.
__device__ __forceinline__ void put_word(void* dst, int64_t i, const Word& w, int wbytes)
{
    if (wbytes == 8) static_cast<Word*>(dst)[i] = w;
    else static_cast<uint32_t*>(dst)[i] = w.se;
}

// n (2 or 4) consecutive words from index i; `vec`: the destination is
// aligned for one 16- or 32-byte store (8 or 16 bytes for 4-byte words).
__device__ __forceinline__ void put_words(void* dst, int64_t i, const Word (&wd)[4], int n, bool vec, int wbytes)
{
    if (wbytes == 8) {
        Word* out = static_cast<Word*>(dst) + i;
        if (vec) {
            uint4* o = reinterpret_cast<uint4*>(out);
            o[0] = make_uint4(wd[0].w, wd[0].se, wd[1].w, wd[1].se);
            if (n == 4) o[1] = make_uint4(wd[2].w, wd[2].se, wd[3].w, wd[3].se);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)          // constant indices: wd stays in registers
                if (t < n) out[t] = wd[t];
        }
    } else {
        uint32_t* out = static_cast<uint32_t*>(dst) + i;
        if (vec && n == 4) *reinterpret_cast<uint4*>(out) = make_uint4(wd[0].se, wd[1].se, wd[2].se, wd[3].se);
        else if (vec && n == 2) *reinterpret_cast<uint2*>(out) = make_uint2(wd[0].se, wd[1].se);
        else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (t < n) out[t] = wd[t].se;
        }
    }
}

// Fold this thread's exponent range into the call's stats: wave reduction,
// then workgroup reduction through LDS, then one atomic pair per workgroup
// into slot (blk % STAT_SLOTS; blk: the workgroup's index in its decode), so
// no single address takes every atomic; and into a replica of the k-segment's
// range `seg` when the workgroup's elements lie in one segment (else null). Must be
// called by every thread of a 256-thread workgroup.
__device__ __forceinline__ void flush_stats(int* stats, int emin, int emax, uint32_t blk, int* seg = nullptr,
                                            uint32_t seg_gen = 0)
{
    __shared__ int red[2][4];
    for (int off = 32; off > 0; off >>= 1) {
        emin = min(emin, __shfl_xor(emin, off, 64));
        emax = max(emax, __shfl_xor(emax, off, 64));
    }
    const int wave = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) {
        red[0][wave] = emin;
        red[1][wave] = emax;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
        const int nw = blockDim.x >> 6;
        for (int w = 1; w < nw; ++w) {
            emin = min(emin, red[0][w]);
            emax = max(emax, red[1][w]);
        }
        if (emin <= emax) {
            int* slot = stats + (blk % STAT_SLOTS) * STAT_STRIDE;
            atomicMin(&slot[0], emin);
            atomicMax(&slot[1], emax);
            if (seg != nullptr) {
                unsigned int* r = reinterpret_cast<unsigned int*>(seg + 4 * (blk % SEG_REPL));
                atomicMax(&r[0], seg_gen | (uint32_t)(255 - emin));
                atomicMax(&r[1], seg_gen | (uint32_t)emax);
            }
        }
    }
}

// Source element (within one batch entry) of output word o, or -1 for a
// zero word (padding, dilation slot, or out-of-range tail). Used by the
// generic decode kernel; the image and tile kernels below cover the large
// layouts with coalesced accesses.
__device__ __forceinline__ int64_t decode_source(const DecodeParams& p, uint32_t o)
{
    switch (p.layout) {
    case L_DENSE_LANE: {        // [KB][Mp][4]: element (i, kb*4+t) of op(A)
        const uint32_t t = o & 3u, r = o >> 2;
        const uint32_t kb = fdiv(r, p.fd_Mp), i = r - kb * (uint32_t)p.Mp;
        const uint32_t kk = kb * 4u + t;
        if (i >= (uint32_t)p.m || kk >= (uint32_t)p.k) return -1;
        return p.trans ? (int64_t)kk * p.ld + i : (int64_t)i * p.ld + kk;
    }
    case L_DENSE_UNIFORM: {     // [Kp][Np]: element (kk, j) of op(B)
        const uint32_t kk = fdiv(o, p.fd_Np), j = o - kk * (uint32_t)p.Np;
        if (j >= (uint32_t)p.n || kk >= (uint32_t)p.k) return -1;
        return p.trans ? (int64_t)j * p.ld + kk : (int64_t)kk * p.ld + j;
    }
    case L_IMG_FWD: {           // [N][Hp][Cb][Wp][4]
        const uint32_t t = o & 3u;
        uint32_t r = o >> 2;
        uint32_t q = fdiv(r, p.fd_Wp);
        const int wq = (int)(r - q * (uint32_t)p.Wp);
        r = q; q = fdiv(r, p.fd_Cb);
        const int cb = (int)(r - q * (uint32_t)p.Cb);
        r = q; q = fdiv(r, p.fd_Hp);
        const int hq = (int)(r - q * (uint32_t)p.Hp), n = (int)q;
        const int c = cb * 4 + (int)t, h = hq - p.ph, w = wq - p.pw;
        if (c >= p.C || h < 0 || h >= p.H || w < 0 || w >= p.W) return -1;
        return (((int64_t)n * p.H + h) * p.W + w) * p.C + c;
    }
    case L_IMG_DGRAD: {         // padded, dilated errors [N][Hd][Kb][Wd][4]
        const uint32_t t = o & 3u;
        uint32_t r = o >> 2;
        uint32_t q = fdiv(r, p.fd_Wp);
        const int bq = (int)(r - q * (uint32_t)p.Wp);
        r = q; q = fdiv(r, p.fd_Kb);
        const int kb = (int)(r - q * (uint32_t)p.Kb);
        r = q; q = fdiv(r, p.fd_Hp);
        const int aq = (int)(r - q * (uint32_t)p.Hp), n = (int)q;
        const int ko = kb * 4 + (int)t;
        const int hh = aq - (p.R - 1 - p.ph), ww = bq - (p.S - 1 - p.pw);
        if (ko >= p.K || hh < 0 || ww < 0 || hh % p.sh != 0 || ww % p.sw != 0) return -1;
        const int pp = hh / p.sh, qq = ww / p.sw;
        if (pp >= p.P || qq >= p.Q) return -1;
        return (((int64_t)n * p.P + pp) * p.Q + qq) * p.K + ko;
    }
    case L_W_FWD: {             // [R*S*Cp][Np]: row (r, s, c), column k
        const uint32_t row = fdiv(o, p.fd_Np), j = o - row * (uint32_t)p.Np;
        const uint32_t rs = fdiv(row, p.fd_Cp), c = row - rs * (uint32_t)p.Cp;
        if (c >= (uint32_t)p.C || j >= (uint32_t)p.K) return -1;
        return ((int64_t)rs * p.C + c) * p.K + j;
    }
    case L_W_DGRAD: {           // [R*S*Kp][Np]: row (R-1-r, S-1-s, k), column c
        const uint32_t row = fdiv(o, p.fd_Np), j = o - row * (uint32_t)p.Np;
        const uint32_t rs = fdiv(row, p.fd_Kp), ko = row - rs * (uint32_t)p.Kp;
        if (ko >= (uint32_t)p.K || j >= (uint32_t)p.C) return -1;
        const uint32_t rq = fdiv(rs, p.fd_S);
        const int rr = p.R - 1 - (int)rq, ss = p.S - 1 - (int)(rs - rq * (uint32_t)p.S);
        return (((int64_t)rr * p.S + ss) * p.C + j) * p.K + ko;
    }
    case L_IMG_WGRAD: {         // [N][Hp][Wp][C], then a zero tail
        const uint32_t body = (uint32_t)p.N * p.Hp * p.Wp * p.C;
        if (o >= body) return -1;
        uint32_t r = o;
        uint32_t q = fdiv(r, p.fd_C);
        const int c = (int)(r - q * (uint32_t)p.C);
        r = q; q = fdiv(r, p.fd_Wp);
        const int wq = (int)(r - q * (uint32_t)p.Wp);
        r = q; q = fdiv(r, p.fd_Hp);
        const int hq = (int)(r - q * (uint32_t)p.Hp), n = (int)q;
        const int h = hq - p.ph, w = wq - p.pw;
        if (h < 0 || h >= p.H || w < 0 || w >= p.W) return -1;
        return (((int64_t)n * p.H + h) * p.W + w) * p.C + c;
    }
    case L_DY_WGRAD: {          // [Kp][Np]: row = output pixel, column = k
        const uint32_t kk = fdiv(o, p.fd_Np), j = o - kk * (uint32_t)p.Np;
        if (j >= (uint32_t)p.K || kk >= (uint32_t)(p.N * p.P * p.Q)) return -1;
        return (int64_t)kk * p.K + j;
    }
    }
    return -1;
}

// Each decode below runs as one part of decode_group_kernel: bid / gdim are
// the workgroup's index and the grid of its own part, blk its linear index.
__device__ __forceinline__ uint32_t linear_block(uint3 bid, uint3 gdim)
{
    return bid.x + bid.y * gdim.x + bid.z * gdim.x * gdim.y;
}

__device__ __forceinline__ void decode_generic_body(const DecodeParams& p, uint3 bid, uint3 gdim)
{
    int emin = 255, emax = 0;
    const int b = (int)bid.y;
    const float* src = p.src_ptrs ? p.src_ptrs[b] : p.src + b * p.src_batch_stride;
    const int64_t d0 = b * p.dst_batch_stride;
    const uint32_t stride = gdim.x * 256u;
    for (uint32_t o = bid.x * 256u + threadIdx.x; o < (uint32_t)p.count; o += stride) {
        const int64_t s = decode_source(p, o);
        const uint32_t row = fdiv(o, p.fd_rowlen);
        put_word(p.dst, d0 + (int64_t)row * p.ldw + (o - row * (uint32_t)p.rowlen),
                 s >= 0 ? decode_bits(__float_as_uint(src[s]), p.M, p.lane_role, emin, emax, p.elo, p.ehi)
                        : zero_word(p.M, p.lane_role), p.wbytes);
    }
    flush_stats(p.stats, emin, emax, linear_block(bid, gdim));
}

// Image layouts, one workgroup per output row: the source row (an NHWC row
// of x, or of dy for the padded, dilated errors) is staged in LDS with
// coalesced (16-byte where aligned) loads, then the output row is written
// contiguously, 2 or 4 Words (16 or 32 bytes) per thread and step.
constexpr int IMG_ROW_FLOATS_MAX = 8192;   // 32 KB of LDS per workgroup

__device__ __forceinline__ void decode_img_body(const DecodeParams& p, uint3 bid, uint3 gdim, float* row)
{
    int emin = 255, emax = 0;
    const int r = (int)bid.x;                      // output row
    if (r >= p.rows) {                             // zero tail of the weight-gradient image
        const int64_t body = (int64_t)p.rows * p.C * p.Wp;
        for (int64_t o = body + (int64_t)(r - p.rows) * 256 * 16 + threadIdx.x; o < p.count &&
             o < body + (int64_t)(r - p.rows + 1) * 256 * 16; o += 256)
            put_word(p.dst, o, zero_word(p.M, p.lane_role), p.wbytes);
        return;
    }
    // which source row feeds output row r (or none: a padding / dilation row)
    int n, srow = -1;
    if (p.layout == L_IMG_DGRAD) {
        n = r / p.Hp;
        const int hh = r - n * p.Hp - (p.R - 1 - p.ph);
        if (hh >= 0 && hh % p.sh == 0 && hh / p.sh < p.P) srow = hh / p.sh;
    } else {
        n = r / p.Hp;
        const int h = r - n * p.Hp - p.ph;
        if (h >= 0 && h < p.H) srow = h;
    }
    if (srow >= 0) {
        const int rows_per_image = p.layout == L_IMG_DGRAD ? p.P : p.H;
        const float* src = p.src + ((int64_t)n * rows_per_image + srow) * p.row_floats;
        if ((p.row_floats & 3) == 0 && (reinterpret_cast<uintptr_t>(src) & 15u) == 0) {
            const float4* s4 = reinterpret_cast<const float4*>(src);
            float4* r4 = reinterpret_cast<float4*>(row);
            for (int i = threadIdx.x; i < (p.row_floats >> 2); i += 256) r4[i] = s4[i];
        } else {
            for (int i = threadIdx.x; i < p.row_floats; i += 256) row[i] = src[i];
        }
    }
    __syncthreads();
    auto dec = [&](float v) { return decode_bits(__float_as_uint(v), p.M, p.lane_role, emin, emax, p.elo, p.ehi); };
    const Word z = zero_word(p.M, p.lane_role);
    if (p.layout == L_IMG_FWD || p.layout == L_IMG_DGRAD) {
        // [Cb][Wp][4] (fwd) or [Kb][Wd][4] (dgrad): item q = one (channel block, column), 4 Words
        const bool fwd = p.layout == L_IMG_FWD;
        const int CH = fwd ? p.C : p.K;            // channels of a source pixel
        const int items = (fwd ? p.Cb : p.Kb) * p.Wp;
        const int64_t out = (int64_t)r * items * 4;
        for (int q = threadIdx.x; q < items; q += 256) {
            const uint32_t blk = fdiv((uint32_t)q, p.fd_Wp);
            const int wq = q - (int)blk * p.Wp;
            int px = -1;                           // source pixel of this column
            if (srow >= 0) {
                if (fwd) {
                    const int w = wq - p.pw;
                    if (w >= 0 && w < p.W) px = w;
                } else {
                    const int ww = wq - (p.S - 1 - p.pw);
                    if (ww >= 0 && (p.sw == 1 || ww % p.sw == 0)) {
                        const int qq = p.sw == 1 ? ww : ww / p.sw;
                        if (qq < p.Q) px = qq;
                    }
                }
            }
            const int c0 = (int)blk * 4;
            Word wd[4];
            if (px >= 0 && (CH & 3) == 0) {        // 4 channels inside, 16 bytes of LDS
                const float4 v = *reinterpret_cast<const float4*>(row + px * CH + c0);
                wd[0] = dec(v.x); wd[1] = dec(v.y); wd[2] = dec(v.z); wd[3] = dec(v.w);
            } else {
#pragma unroll
                for (int t = 0; t < 4; ++t) wd[t] = (px >= 0 && c0 + t < CH) ? dec(row[px * CH + c0 + t]) : z;
            }
            put_words(p.dst, out + (int64_t)q * 4, wd, 4, true, p.wbytes);
        }
    } else {                                       // L_IMG_WGRAD: [Wp][C], 2 Words per item
        const int per_row = p.Wp * p.C;
        const int64_t out = (int64_t)r * per_row;
        const bool vec = (per_row & 1) == 0;       // rows (and so the pairs) 16-byte aligned
        for (int o = threadIdx.x * 2; o < per_row; o += 512) {
            Word wd[4];
            const int cnt = min(2, per_row - o);
#pragma unroll
            for (int t = 0; t < 2; ++t) {
                const uint32_t e = (uint32_t)(o + t);
                const uint32_t wq = fdiv(e, p.fd_C);
                const int c = (int)(e - wq * (uint32_t)p.C), w = (int)wq - p.pw;
                wd[t] = (t < cnt && srow >= 0 && w >= 0 && w < p.W) ? dec(row[w * p.C + c]) : z;
            }
            put_words(p.dst, out + o, wd, cnt, vec && cnt == 2, p.wbytes);
        }
    }
    flush_stats(p.stats, emin, emax, linear_block(bid, gdim));
}

// Dense layouts that transpose: 64 x 64 tiles through LDS, read along the
// source's contiguous dimension (16-byte loads where the source is aligned)
// and written along the output's.
//  lane (A not transposed):   out [KB][Mp][4], element (i, kk) = A[i*ld + kk];
//    a lane reads 4 consecutive kk of one tile row i (16 bytes of LDS, rows
//    kTileLaneLd floats apart) and writes their 4 Words (32 contiguous bytes)
//  uniform (B transposed):    out [Kp][Np],    element (kk, j) = B[j*ld + kk];
//    a lane reads tile rows j, j+1 at one kk (rows kTileUniLd floats apart:
//    the 32 lanes of a half-wave hit distinct banks) and writes 2 Words.
constexpr int kTileLaneLd = 68;
constexpr int kTileUniLd = 65;
constexpr int kTileLdsBytes = 64 * kTileLaneLd * 4;

__device__ __forceinline__ void decode_tile_body(const DecodeParams& p, uint3 bid, uint3 gdim, float* tile)
{
    int emin = 255, emax = 0;
    const int b = (int)bid.z;
    const float* src = p.src_ptrs ? p.src_ptrs[b] : p.src + b * p.src_batch_stride;
    const int64_t d0 = b * p.dst_batch_stride;
    const bool lane = p.layout == L_DENSE_LANE;
    const int tld = lane ? kTileLaneLd : kTileUniLd;
    const int outer0 = (int)bid.x * 64;            // i (lane) or j (uniform)
    const int k0 = (int)bid.y * 64;                // kk
    const int outer_n = lane ? p.m : p.n;
    const bool vec = (((uintptr_t)src & 15u) == 0) && (p.ld & 3) == 0;
    // load: source row = outer index, 4 consecutive kk per lane
    for (int e = threadIdx.x; e < 64 * 16; e += 256) {
        const int ro = e >> 4, c = (e & 15) * 4;
        const int oi = outer0 + ro, ki = k0 + c;
        float v[4];
        if (oi < outer_n && vec && ki + 3 < p.k) {
            const float4 q = *reinterpret_cast<const float4*>(src + (int64_t)oi * p.ld + ki);
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t)
                v[t] = (oi < outer_n && ki + t < p.k) ? src[(int64_t)oi * p.ld + ki + t] : 0.0f;
        }
        if (lane) {
            *reinterpret_cast<float4*>(tile + ro * kTileLaneLd + c) = make_float4(v[0], v[1], v[2], v[3]);
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) tile[ro * tld + c + t] = v[t];
        }
    }
    __syncthreads();
    if (lane) {
        // k-step kbl of the tile: rows outer0.. of [Mp][4] are contiguous
        for (int f = threadIdx.x; f < 16 * 64; f += 256) {
            const int kbl = f >> 6, i = f & 63;
            const int oi = outer0 + i, kb = (k0 >> 2) + kbl;
            if (kb >= p.KB || oi >= p.Mp) continue;
            const float4 q = *reinterpret_cast<const float4*>(tile + i * kTileLaneLd + kbl * 4);
            const float v[4] = {q.x, q.y, q.z, q.w};
            Word wd[4];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                wd[t] = (oi < p.m && k0 + kbl * 4 + t < p.k)
                    ? decode_bits(__float_as_uint(v[t]), p.M, 1, emin, emax, p.elo, p.ehi)
                    : zero_word(p.M, 1);
            put_words(p.dst, d0 + (int64_t)kb * p.ldw + (int64_t)oi * 4, wd, 4, true, p.wbytes);
        }
    } else {
        // output row kk holds 64 contiguous columns j: a lane takes j, j+1
        for (int f = threadIdx.x; f < 64 * 32; f += 256) {
            const int kk = ((f >> 6) << 1) | ((f >> 5) & 1), j = (f & 31) * 2;
            const int oj = outer0 + j, ki = k0 + kk;
            if (ki >= p.KB * 4) continue;
            Word wd[4];
#pragma unroll
            for (int t = 0; t < 2; ++t)
                wd[t] = (oj + t < p.n && ki < p.k)
                    ? decode_bits(__float_as_uint(tile[(j + t) * kTileUniLd + kk]), p.M, 0, emin, emax, p.elo, p.ehi)
                    : zero_word(p.M, 0);
            const int64_t out = d0 + (int64_t)ki * p.ldw + oj;
            if (oj + 1 < p.Np && (p.ldw & 1) == 0) {
                put_words(p.dst, out, wd, 2, true, p.wbytes);
            } else {
                if (oj < p.Np) put_word(p.dst, out, wd[0], p.wbytes);
                if (oj + 1 < p.Np) put_word(p.dst, out + 1, wd[1], p.wbytes);
            }
        }
    }
    // reduction indices [64 bid.y, 64 bid.y + 64): one k-segment
    flush_stats(p.stats, emin, emax, linear_block(bid, gdim), p.seg ? p.seg + 4 * SEG_REPL * bid.y : nullptr,
                p.seg_gen);
}

// The same two layouts without the trip through LDS, for small operands
// (panels of at most kDirectElems words over all batch entries): thread t of
// batch entry b takes k-step kb
// = t / outer of row (lane) or column (uniform) o = t % outer of the panel,
// reads its 4 source elements (16 bytes where aligned) and writes their 4
// Words: 32 contiguous bytes at (kb, o) of [KB][Mp][4] (lane), or one Word in
// each of the rows 4 kb .. 4 kb + 3 of [Kp][Np] (uniform; consecutive threads
// write consecutive columns). A workgroup's 256 threads lie in one k-segment
// (64 indices): outer is a multiple of 16, so 16 * outer is one of 256.
// One load, decode and store per thread: for such operands the transposing
// tile's LDS round trip and barrier were most of the launch's time.
constexpr int64_t kDirectElems = (int64_t)1 << 22;

__device__ __forceinline__ void decode_direct_body(const DecodeParams& p, uint3 bid, uint3 gdim)
{
    int emin = 255, emax = 0;
    const int b = (int)bid.y;
    const float* src = p.src_ptrs ? p.src_ptrs[b] : p.src + b * p.src_batch_stride;
    const int64_t d0 = b * p.dst_batch_stride;
    const bool lane = p.layout == L_DENSE_LANE;
    const int outer = lane ? p.Mp : p.Np;          // panel rows (lane) or columns (uniform)
    const int outer_n = lane ? p.m : p.n;          // of which hold source elements
    const uint32_t t0 = bid.x * 256u;
    const uint32_t t = t0 + threadIdx.x;
    const uint32_t kb = fdiv(t, lane ? p.fd_Mp : p.fd_Np), o = t - kb * (uint32_t)outer;
    if (kb < (uint32_t)p.KB) {
        const int k0 = (int)kb * 4;
        const bool in = (int)o < outer_n;
        const float* s = src + (int64_t)o * p.ld + k0;
        float v[4];
        if (in && k0 + 3 < p.k && ((reinterpret_cast<uintptr_t>(s) & 15u) == 0)) {
            const float4 q = *reinterpret_cast<const float4*>(s);
            v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] = (in && k0 + u < p.k) ? s[u] : 0.0f;
        }
        const int role = lane ? 1 : 0;
        Word wd[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            wd[u] = (in && k0 + u < p.k) ? decode_bits(__float_as_uint(v[u]), p.M, role, emin, emax, p.elo, p.ehi)
                                         : zero_word(p.M, role);
        if (lane) {
            put_words(p.dst, d0 + (int64_t)kb * p.ldw + (int64_t)o * 4, wd, 4, true, p.wbytes);
        } else {
#pragma unroll
            for (int u = 0; u < 4; ++u) put_word(p.dst, d0 + (int64_t)(k0 + u) * p.ldw + o, wd[u], p.wbytes);
        }
    }
    const uint32_t seg = fdiv(t0, lane ? p.fd_Mp : p.fd_Np) >> 4;   // the workgroup's k-segment
    flush_stats(p.stats, emin, emax, linear_block(bid, gdim), p.seg ? p.seg + 4 * SEG_REPL * seg : nullptr,
                p.seg_gen);
}

// Empty slots: min 255, max 0 (lane and uniform), and no readers yet.
__device__ __forceinline__ int stat_reset_value(int i) { return (i & 1) ? 0 : 255; }

// One workgroup per statistics block: slots, counts and k-segments.
__global__ __launch_bounds__(256) void init_stats_kernel(int* stats)
{
    int* blk = stats + (int64_t)blockIdx.x * STAT_BLOCK_INTS;
    for (int i = threadIdx.x; i < STAT_INTS; i += 256) blk[i] = stat_reset_value(i);
    for (int i = threadIdx.x; i < 4 * SEG_REPL * SEG_MAX; i += 256) blk[STAT_SEG + i] = 0;   // generation 0: no call's
    if (threadIdx.x == 0) blk[STAT_READERS] = 0;
}

// Plain row copies with decode: out[kk][j] (kk < rows_out, j < Np) from
// src[kk * ld + j] when kk < k and j < n (uniform panels of untransposed B
// and of the weight-gradient errors). Workgroup (x, ., z) takes rows
// [x * rb, x * rb + rb) of batch entry z as one run of 4-column quads (Np is
// a multiple of 16): a 16-byte load where the source allows it, 32 bytes of
// Words stored.
__device__ __forceinline__ void decode_rows_body(const DecodeParams& p, uint3 bid, uint3 gdim, int rb)
{
    int emin = 255, emax = 0;
    const int b = (int)bid.z;
    const float* src = p.src_ptrs ? p.src_ptrs[b] : p.src + b * p.src_batch_stride;
    const int64_t d0 = b * p.dst_batch_stride;
    const int r0 = (int)bid.x * rb;
    const uint32_t quads = (uint32_t)min(rb, p.KB * 4 - r0) * (uint32_t)(p.Np >> 2);
    const bool vsrc = ((reinterpret_cast<uintptr_t>(src) & 15u) == 0) && ((p.ld & 3) == 0);
    for (uint32_t q = threadIdx.x; q < quads; q += 256) {
        const uint32_t row = fdiv(q * 4u, p.fd_Np);
        const int col = (int)(q * 4u - row * (uint32_t)p.Np);
        const int kk = r0 + (int)row;
        const float* s = src + (int64_t)kk * p.ld + col;
        float v[4];
        if (kk < p.k && vsrc && col + 3 < p.n) {
            const float4 f = *reinterpret_cast<const float4*>(s);
            v[0] = f.x; v[1] = f.y; v[2] = f.z; v[3] = f.w;
        } else {
#pragma unroll
            for (int t = 0; t < 4; ++t) v[t] = (kk < p.k && col + t < p.n) ? s[t] : 0.0f;
        }
        Word wd[4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
            wd[t] = (kk < p.k && col + t < p.n)
                ? decode_bits(__float_as_uint(v[t]), p.M, p.lane_role, emin, emax, p.elo, p.ehi)
                : zero_word(p.M, p.lane_role);
        put_words(p.dst, d0 + (int64_t)kk * p.ldw + col, wd, 4, true, p.wbytes);
    }
    // rows [r0, r0 + rb) with rb dividing 64 (the host gives a segment pointer only then): one k-segment
    flush_stats(p.stats, emin, emax, linear_block(bid, gdim), p.seg ? p.seg + 4 * SEG_REPL * (r0 >> 6) : nullptr,
                p.seg_gen);
}

// The decodes of both operands of a call in one launch: workgroups [0, na)
// run job a's decode, the rest job b's. The dynamic LDS buffer holds the
// image row or the 64 x 65 transposing tile (sized by the host for the
// larger of the two jobs' needs).
__device__ __forceinline__ void decode_job(const DecodeJob& jb, uint32_t blk, float* smem)
{
    const uint3 gdim = make_uint3(jb.gx, jb.gy, jb.gz);
    const uint3 bid = make_uint3(blk % jb.gx, (blk / jb.gx) % jb.gy, blk / (jb.gx * jb.gy));
    switch (jb.variant) {
    case DV_IMG: decode_img_body(jb.p, bid, gdim, smem); break;
    case DV_ROWS: decode_rows_body(jb.p, bid, gdim, jb.rb); break;
    case DV_TILE: decode_tile_body(jb.p, bid, gdim, smem); break;
    case DV_DIRECT: decode_direct_body(jb.p, bid, gdim); break;
    default: decode_generic_body(jb.p, bid, gdim); break;
    }
}

// The decodes of up to 2 * kMaxGroup operands in one launch: job j takes
// workgroups [first[j], first[j + 1]).
struct DecodeGroup {
    int count;
    uint32_t first[2 * kMaxGroup + 1];
    DecodeJob job[2 * kMaxGroup];
};

__global__ __launch_bounds__(256) void decode_group_kernel(DecodeGroup g)
{
    extern __shared__ __align__(16) float smem[];
    int j = 0;
    while (j + 1 < g.count && blockIdx.x >= g.first[j + 1]) ++j;
    decode_job(g.job[j], blockIdx.x - g.first[j], smem);
}

// Copy choice for the M = 8 lane operands (replica.h): one thread per group
// of up to 32 Words that one half-wave of the GEMM kernel reads at one
// reduction index; moves some of their table offsets to the rows' second
// copies so that the group's lookups spread over the LDS banks.
constexpr int kAssignThreads = 256;

__global__ __launch_bounds__(kAssignThreads) void assign_kernel(AssignParams p)
{
    const int64_t groups = (int64_t)p.batch * p.G1 * p.G2 * p.G3;
    for (int64_t g = (int64_t)blockIdx.x * kAssignThreads + threadIdx.x; g < groups;
         g += (int64_t)gridDim.x * kAssignThreads) {
        int64_t r = g;
        const int g3 = (int)(r % p.G3);
        r /= p.G3;
        const int g2 = (int)(r % p.G2);
        r /= p.G2;
        const int64_t g1 = r % p.G1, b = r / p.G1;
        Word* base = p.panel + b * p.batch_stride + g1 * p.S1 + (int64_t)g2 * p.S2 + (int64_t)g3 * p.S3 + p.O;
        const int count = min(32, p.E - g2 * 32);
        uint32_t w[32], w0[32];
#pragma unroll
        for (int l = 0; l < 32; ++l) w0[l] = w[l] = l < count ? base[(int64_t)l * p.LS].w : p.pad_w;
        rep8_assign_group(w, count, p.pad_w);
#pragma unroll
        for (int l = 0; l < 32; ++l)
            if (l < count && w[l] != w0[l]) base[(int64_t)l * p.LS].w = w[l];
    }
}

// ------------------------------------------------------------------ products

// ------------------------------------------------------------------ GEMM

struct KCounter {
    int u1, u2, u3, off;
};

__device__ __forceinline__ KCounter kc_init(const MainParams& p, int u)
{
    KCounter c;
    c.u3 = u % p.U3;
    const int r = u / p.U3;
    c.u2 = r % p.U2;
    c.u1 = r / p.U2;
    c.off = c.u1 * p.K1 + c.u2 * p.K2 + c.u3 * p.K3;
    return c;
}

__device__ __forceinline__ void kc_next(const MainParams& p, KCounter& c)
{
    c.off += p.K3;
    if (++c.u3 == p.U3) {
        c.u3 = 0;
        c.off += p.K2 - p.U3 * p.K3;
        if (++c.u2 == p.U2) {
            c.u2 = 0;
            c.off += p.K1 - p.U2 * p.K2;
            ++c.u1;
        }
    }
}

// Offsets (in Words, relative to a lane's base) of the 4 reduction indices of
// k-step kb. Vector mode: 4 consecutive Words at one offset. Gather mode:
// one offset per reduction index, or the zero region past the last one.
template <bool GATHER>
__device__ __forceinline__ void step_offsets(const MainParams& p, KCounter& kc, int& ku, int (&off)[4])
{
    if (!GATHER) {
#pragma unroll
        for (int t = 0; t < 4; ++t) off[t] = kc.off + t;
        kc_next(p, kc);
    } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            off[t] = ku < p.nku ? kc.off : p.zoff;
            ++ku;
            kc_next(p, kc);
        }
    }
}

// Lane operand words (w, se) of the RPL rows of this lane at one offset.
template <int RPL>
__device__ __forceinline__ void load_lane(const Word* panel, const uint32_t (&base)[RPL], int off,
                                          uint32_t (&wa)[RPL], uint32_t (&sa)[RPL])
{
#pragma unroll
    for (int x = 0; x < RPL; ++x) {
        const uint2 q = *reinterpret_cast<const uint2*>(panel + base[x] + off);
        wa[x] = q.x;
        sa[x] = q.y;
    }
}

// Checked path: Algorithm 2 with every special case, as selects (no
// divergence), then acc + product. seA, seB: operands already cast to the
// format; elo..ehi: the format's normal range of biased exponents.
__device__ __forceinline__ float checked_product_acc(float acc, uint32_t e, uint32_t seA, uint32_t seB, int elo,
                                                     int ehi)
{
    const uint32_t ea = (seA >> 23) & 0xFFu, eb = (seB >> 23) & 0xFFu;
    const uint32_t sign = (seA ^ seB) & 0x80000000u;
    const int ex = (int)ea + (int)eb - 127 + (int)(e >> 15);
    uint32_t bits = sign | ((uint32_t)(ex & 0xFF) << 23) | ((e & 0x7FFFu) << 8);
    bits = ex > ehi ? (sign | 0x7F800000u) : bits;             // overflow -> signed Inf
    bits = ex < elo ? sign : bits;                             // underflow -> signed zero
    const bool zero = ea == 0u || eb == 0u;                    // zero or subnormal operand
    const bool a_inf = ea == 255u && (seA & 0x7FFFFFu) == 0u;
    const bool b_inf = eb == 255u && (seB & 0x7FFFFFu) == 0u;
    const bool nan = (ea == 255u && (seA & 0x7FFFFFu) != 0u) || (eb == 255u && (seB & 0x7FFFFFu) != 0u);
    bits = zero ? sign : bits;
    bits = (a_inf || b_inf) ? (zero ? 0x7FC00000u : (sign | 0x7F800000u)) : bits;
    bits = nan ? 0x7FC00000u : bits;
    return acc + __uint_as_float(bits);
}


// Uniform words of one reduction index for this wave's 16 columns, spread
// over the 4 lanes of each quad: lane i of a quad holds, in register
// 4j + t, dword 16j + 4i + t of the 32 dwords {w0, se0, w1, se1, ...}.
// 8 VGPRs per index instead of 32 (a quarter of the vector-memory return
// traffic of a full broadcast); a consumer reads column c's value with a
// quad_perm DPP broadcast of lane (c >> 1) & 3, folded into its own
// instruction (v_add_u32_dpp, v_fmac_f32_dpp).
constexpr int UQ = 8;

__device__ __forceinline__ void load_uniform(const Word* row, uint32_t quad, uint32_t (&q)[UQ])
{
    const uint4* src = reinterpret_cast<const uint4*>(row) + quad;
    const uint4 a = src[0], b = src[4];
    q[0] = a.x; q[1] = a.y; q[2] = a.z; q[3] = a.w;
    q[4] = b.x; q[5] = b.y; q[6] = b.z; q[7] = b.w;
}

// Lane i of every quad, broadcast to the quad (quad_perm:[i,i,i,i]). i is a
// constant once the callers' loops are unrolled.
__device__ __forceinline__ uint32_t quad_bcast(uint32_t v, int i)
{
    switch (i) {
    case 0: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x00, 0xF, 0xF, true);
    case 1: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x55, 0xF, 0xF, true);
    case 2: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xAA, 0xF, 0xF, true);
    default: return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xFF, 0xF, 0xF, true);
    }
}

// acc += (lane i of this lane's quad in q) * x, one v_fmac_f32 with a DPP
// broadcast operand (the compiler does not fold a DPP move into an FMA on
// this target). The asm statement also keeps each fold in place in the
// schedule. q comes straight from vector-memory loads, so no VALU write
// precedes its DPP read.
__device__ __forceinline__ void fmac_quad(float& acc, uint32_t q, float x, int i)
{
#define AMX_FMAC_DPP(I)                                                                                  \
    asm volatile("v_fmac_f32_dpp %0, %1, %2 quad_perm:[" #I "," #I "," #I "," #I "] row_mask:0xf bank_mask:0xf" \
                 : "+v"(acc) : "v"(q), "v"(x))
    switch (i) {
    case 0: AMX_FMAC_DPP(0); break;
    case 1: AMX_FMAC_DPP(1); break;
    case 2: AMX_FMAC_DPP(2); break;
    default: AMX_FMAC_DPP(3); break;
    }
#undef AMX_FMAC_DPP
}

// Column c's w (h = 0) or se (h = 1), in every lane.
__device__ __forceinline__ uint32_t col_word(const uint32_t (&q)[UQ], int c, int h)
{
    return quad_bcast(q[4 * (c >> 3) + 2 * (c & 1) + h], (c >> 1) & 3);
}

// Fast path over one reduction index, finer pipeline: a group is the RPL
// products of one column; the lookups of group g+LA are issued while group g
// is folded, so up to (LA+1)*RPL lookups per wave are in flight. LA = 3 for
// a table in LDS (the 4-bit LDS wait counter), 6 for a table in global
// memory (longer latency, 6-bit counter).
constexpr int LA_LDS = 3;
constexpr int LA_GLOBAL = 6;

template <int RPL, int LA>
__device__ __forceinline__ void fast_index(const uint32_t (&wa)[RPL], const uint32_t (&sa)[RPL], const uint32_t (&q)[UQ],
                                           const unsigned char* lut, float (&acc)[RPL][CPW])
{
    uint32_t e[LA + 1][RPL];
#define AMX_COLW(j) col_word(q, (j), 0)
#pragma unroll
    for (int g = 0; g < LA; ++g)
#pragma unroll
        for (int x = 0; x < RPL; ++x) e[g][x] = *reinterpret_cast<const uint16_t*>(lut + (wa[x] + AMX_COLW(g)));
#pragma unroll
    for (int g = 0; g < CPW; ++g) {
        if (g + LA < CPW) {
#pragma unroll
            for (int x = 0; x < RPL; ++x)
                e[(g + LA) % (LA + 1)][x] = *reinterpret_cast<const uint16_t*>(lut + (wa[x] + AMX_COLW(g + LA)));
        }
        // acc += as_float(seA + (entry << 8)) * as_float(seB): the fast-path product
#pragma unroll
        for (int x = 0; x < RPL; ++x)
            fmac_quad(acc[x][g], q[4 * (g >> 3) + 2 * (g & 1) + 1], __uint_as_float((e[g % (LA + 1)][x] << 8) + sa[x]),
                      (g >> 1) & 3);
        __builtin_amdgcn_sched_barrier(0);
    }
#undef AMX_COLW
}

// Columns of an index whose lookups go to the table image in global memory
// (L2-resident) instead of the LDS copy: GOFF of the 16, evenly spaced. The
// LDS then serves (16 - GOFF) / 16 of the lookups and the vector-memory path
// the rest, each at its own rate; both read the same image, so the entries
// are the same. Measured on MI355X (GEMM-kernel ms; 8192^3 at M = 8, the
// 3 x 3 conv passes at M = 7): GOFF 0: 70.07 / 0.598, 1: 67.86 / 0.587,
// 2: 73.74 / 0.598, 4: 103.4 / 1.295 (the gathers then saturate the
// texture path, which also carries the operand words).
#ifndef AMX_GOFF
#define AMX_GOFF 1
#endif
template <int GOFF>
__host__ __device__ constexpr bool gcol_is(int c)
{
    return GOFF > 0 && c % (CPW / GOFF) == CPW / GOFF - 1;
}
template <int GOFF>
__host__ __device__ constexpr int gcol(int s)
{
    return (s + 1) * (CPW / GOFF) - 1;
}
template <int GOFF>
__host__ __device__ constexpr int lcol(int i)          // i-th column served by the LDS
{
    int k = -1;
    for (int c = 0; c < CPW; ++c)
        if (!gcol_is<GOFF>(c) && ++k == i) return c;
    return 0;
}
typedef const unsigned char __attribute__((address_space(1)))* gbyte_ptr;

// The fast path with GOFF columns from global memory: their entries for this
// index (gcur) were requested during the previous index; those of the next
// index (wan, qn: its lane and uniform words) are requested here, before the
// LDS lookups, so they have a whole index to arrive.
template <int RPL, int LA, int GOFF>
__device__ __forceinline__ void fast_index_split(const uint32_t (&wa)[RPL], const uint32_t (&sa)[RPL],
                                                 const uint32_t (&q)[UQ], const unsigned char* lut,
                                                 float (&acc)[RPL][CPW], const uint32_t (&gcur)[GOFF][RPL], bool pre,
                                                 const uint32_t (&wan)[RPL], const uint32_t (&qn)[UQ], gbyte_ptr gtab,
                                                 uint32_t (&gnext)[GOFF][RPL])
{
    constexpr int NL = CPW - GOFF;
    uint32_t e[LA + 1][RPL];
#define AMX_COLW(j) col_word(q, (j), 0)
#pragma unroll
    for (int i = 0; i < LA; ++i)
#pragma unroll
        for (int x = 0; x < RPL; ++x) e[i][x] = *reinterpret_cast<const uint16_t*>(lut + (wa[x] + AMX_COLW(lcol<GOFF>(i))));
    if (pre) {
#pragma unroll
        for (int s2 = 0; s2 < GOFF; ++s2) {
            const uint32_t wb = col_word(qn, gcol<GOFF>(s2), 0);
#pragma unroll
            for (int x = 0; x < RPL; ++x)
                gnext[s2][x] = *reinterpret_cast<const uint16_t __attribute__((address_space(1)))*>(gtab + (wan[x] + wb));
        }
    }
#pragma unroll
    for (int i = 0; i < NL; ++i) {
        const int g = lcol<GOFF>(i);
        if (i + LA < NL) {
#pragma unroll
            for (int x = 0; x < RPL; ++x)
                e[(i + LA) % (LA + 1)][x] = *reinterpret_cast<const uint16_t*>(lut + (wa[x] + AMX_COLW(lcol<GOFF>(i + LA))));
        }
#pragma unroll
        for (int x = 0; x < RPL; ++x)
            fmac_quad(acc[x][g], q[4 * (g >> 3) + 2 * (g & 1) + 1], __uint_as_float((e[i % (LA + 1)][x] << 8) + sa[x]),
                      (g >> 1) & 3);
        __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int s2 = 0; s2 < GOFF; ++s2) {
        const int g = gcol<GOFF>(s2);
#pragma unroll
        for (int x = 0; x < RPL; ++x)
            fmac_quad(acc[x][g], q[4 * (g >> 3) + 2 * (g & 1) + 1], __uint_as_float((gcur[s2][x] << 8) + sa[x]),
                      (g >> 1) & 3);
    }
#undef AMX_COLW
}

// Fast path with underflow, over one reduction index: for calls where some
// products may fall below the format's range (tiny operands, or a format with
// fewer exponent bits) but none can exceed it. A product underflows exactly
// when |x| < 2^(elo - EB), where x = as_float(seA + (entry << 8)) is the
// lane operand's scaled significand and EB the uniform operand's biased
// exponent (|x| * 2^(EB - 127) is the product's magnitude; x is normal). Such
// an x is replaced by zero before the same FMA as the fast path, which gives
// the rule's signed zero (adding it never changes the +0-started sum). Each
// lane computes the bound 2^(elo - EB) for the 4 uniform operands it holds;
// it is 0 for EB >= elo + 127 (no product can underflow) and for Inf / NaN
// uniform operands, and 2^elo for a zero one, where any product is zero.
// Compares are unordered-true, so a NaN x is kept.
template <int RPL, int LA>
__device__ __forceinline__ void ranged_index(const uint32_t (&wa)[RPL], const uint32_t (&sa)[RPL], const uint32_t (&q)[UQ],
                                             const unsigned char* lut, float (&acc)[RPL][CPW], int elo)
{
    uint32_t tq[4];
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const int t = (int)((uint32_t)(elo + 127) << 23) - (int)(q[4 * j + 2 * c + 1] & 0x7F800000u);
            tq[2 * j + c] = (uint32_t)max(t, 0);
        }
    uint32_t e[LA + 1][RPL];
#define AMX_COLW(j) col_word(q, (j), 0)
#pragma unroll
    for (int g = 0; g < LA; ++g)
#pragma unroll
        for (int x = 0; x < RPL; ++x) e[g][x] = *reinterpret_cast<const uint16_t*>(lut + (wa[x] + AMX_COLW(g)));
#pragma unroll
    for (int g = 0; g < CPW; ++g) {
        if (g + LA < CPW) {
#pragma unroll
            for (int x = 0; x < RPL; ++x)
                e[(g + LA) % (LA + 1)][x] = *reinterpret_cast<const uint16_t*>(lut + (wa[x] + AMX_COLW(g + LA)));
        }
        const float tb = __uint_as_float(quad_bcast(tq[2 * (g >> 3) + (g & 1)], (g >> 1) & 3));
#pragma unroll
        for (int x = 0; x < RPL; ++x) {
            const float xv = __uint_as_float((e[g % (LA + 1)][x] << 8) + sa[x]);
            const float xk = !(__builtin_fabsf(xv) < tb) ? xv : 0.0f;
            fmac_quad(acc[x][g], q[4 * (g >> 3) + 2 * (g & 1) + 1], xk, (g >> 1) & 3);
        }
        __builtin_amdgcn_sched_barrier(0);
    }
#undef AMX_COLW
}

// Checked path over one reduction index: one product at a time (it only runs
// for operands that can leave the normal range, so it is kept small in
// registers rather than fast).
template <int RPL>
__device__ __forceinline__ void checked_index(const uint32_t (&wa)[RPL], const uint32_t (&sa)[RPL],
                                              const uint32_t (&q)[UQ], const unsigned char* lut,
                                              float (&acc)[RPL][CPW], int elo, int ehi)
{
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
        const uint32_t wb = col_word(q, j, 0);
        const uint32_t sb = col_word(q, j, 1);
#pragma unroll
        for (int x = 0; x < RPL; ++x) {
            const uint32_t e = *reinterpret_cast<const uint16_t*>(lut + (wa[x] + wb));
            acc[x][j] = checked_product_acc(acc[x][j], e, sa[x], sb, elo, ehi);
            asm volatile("" : "+v"(acc[x][j]));
        }
    }
}

// Fast k-loop over k-steps [kb0, kb1). The operand words of reduction index u
// are requested PD = R - 1 indices before use, into ring slot u % R; a loop
// body covers R indices, so every slot number is a compile-time constant.
// Vector mode: a k-step is 4 contiguous Words at offset so[q] + t, and the
// offsets of the NS k-steps a body touches are kept in so[]. Gather mode:
// every index has its own offset from the counter (the zero region past the
// last index). The steady-state body has no branch: the compiler's wait
// counts for the ring stay exact, so the prefetch is never drained early.
template <bool GATHER, bool RANGED, int R, int RPL, int LA, int GOFF = 0>
__device__ __forceinline__ void mainloop_fast(const MainParams& p, const Word* panel, const Word* bsrc,
                                              const uint32_t (&base)[RPL], int kb0, int kb1, uint32_t quad,
                                              const unsigned char* lut, float (&acc)[RPL][CPW])
{
    constexpr int NG = GOFF > 0 ? GOFF : 1;
    uint32_t gl[2][NG][RPL];                     // global-memory entries of the current / next index
    const gbyte_ptr gtab = (gbyte_ptr)p.lut;
    // index v's fold; v's words in slot s, the next index's in slot sn
    auto fold_at = [&](const uint32_t (&wa)[RPL], const uint32_t (&sa)[RPL], const uint32_t (&q)[UQ], int par,
                       bool pre, const uint32_t (&wan)[RPL], const uint32_t (&qn)[UQ]) {
        if constexpr (RANGED) ranged_index<RPL, LA>(wa, sa, q, lut, acc, p.elo);
        else if constexpr (GOFF > 0) {
            if (par == 0) fast_index_split<RPL, LA, NG>(wa, sa, q, lut, acc, gl[0], pre, wan, qn, gtab, gl[1]);
            else fast_index_split<RPL, LA, NG>(wa, sa, q, lut, acc, gl[1], pre, wan, qn, gtab, gl[0]);
        } else fast_index<RPL, LA>(wa, sa, q, lut, acc);
    };
    constexpr int PD = R - 1;
    constexpr int NS = R / 2;
    constexpr int SB = R / 4;                      // k-steps per loop body
    const int n = (kb1 - kb0) * 4;
    KCounter kc = kc_init(p, GATHER ? kb0 * 4 : kb0);
    int ku = kb0 * 4;
    int so[NS];
    if (!GATHER) {
#pragma unroll
        for (int q = 0; q < NS; ++q) {
            so[q] = kc.off;
            kc_next(p, kc);
        }
    }
    auto lane_off = [&](int v) -> int {          // offset of the v-th index a body loads
        if (!GATHER) return so[v >> 2] + (v & 3);
        const int off = ku < p.nku ? kc.off : p.zoff;
        ++ku;
        kc_next(p, kc);
        return off;
    };
    auto advance = [&]() {                       // the body moved SB k-steps on
        if (!GATHER) {
#pragma unroll
            for (int q = 0; q < NS; ++q) {
                if (q + SB < NS) {
                    so[q] = so[q + SB];
                } else {
                    so[q] = kc.off;
                    kc_next(p, kc);
                }
            }
        }
    };
    const Word* urow = bsrc + (int64_t)kb0 * 4 * p.bld;
    uint32_t wa[R][RPL], sa[R][RPL], qb[R][UQ];
    // the global-memory entries of the first index (its words are in slot 0)
    auto first_global = [&]() {
        if constexpr (GOFF > 0 && !RANGED) {
#pragma unroll
            for (int s2 = 0; s2 < GOFF; ++s2) {
                const uint32_t wb = col_word(qb[0], gcol<GOFF>(s2), 0);
#pragma unroll
                for (int x = 0; x < RPL; ++x)
                    gl[0][s2][x] = *reinterpret_cast<const uint16_t __attribute__((address_space(1)))*>(gtab + (wa[0][x] + wb));
            }
        }
    };
    int u0 = 0;
    if (n >= R + PD) {
        // unconditional prologue: the loop is entered with the same loads in
        // flight as at its back edge
#pragma unroll
        for (int v = 0; v < PD; ++v) {
            load_lane(panel, base, lane_off(v), wa[v], sa[v]);
            load_uniform(urow, quad, qb[v]);
            urow += p.bld;
            asm volatile("" ::: "memory");       // one load group per index, as in the loop
        }
        first_global();
        // The compiler drains the loads in flight at the loop head; folding
        // index u0 before requesting index u0 + PD means that drain only
        // waits for loads that were issued at least one index earlier.
        for (; u0 + R + PD <= n; u0 += R) {
#pragma unroll
            for (int j = 0; j < R; ++j) {
                if (j == 0) fold_at(wa[0], sa[0], qb[0], 0, true, wa[1], qb[1]);
                load_lane(panel, base, lane_off(j + PD), wa[(j + PD) % R], sa[(j + PD) % R]);
                load_uniform(urow, quad, qb[(j + PD) % R]);
                urow += p.bld;
                if (j > 0) fold_at(wa[j], sa[j], qb[j], j & 1, true, wa[(j + 1) % R], qb[(j + 1) % R]);
            }
            advance();
        }
    } else {
#pragma unroll
        for (int v = 0; v < PD; ++v) {
            if (v < n) {
                load_lane(panel, base, lane_off(v), wa[v], sa[v]);
                load_uniform(urow, quad, qb[v]);
                urow += p.bld;
            }
        }
        if (n > 0) first_global();
    }
    for (; u0 < n; u0 += R) {                    // tail: fewer than R + PD indices left
#pragma unroll
        for (int j = 0; j < R; ++j) {
            if (u0 + j >= n) break;
            if (u0 + j + PD < n) {
                load_lane(panel, base, lane_off(j + PD), wa[(j + PD) % R], sa[(j + PD) % R]);
                load_uniform(urow, quad, qb[(j + PD) % R]);
                urow += p.bld;
            }
            fold_at(wa[j], sa[j], qb[j], j & 1, u0 + j + 1 < n, wa[(j + 1) % R], qb[(j + 1) % R]);
        }
        advance();
    }
}

// Checked k-loop: operand words one index ahead, parity slots.
template <bool GATHER, int RPL>
__device__ __forceinline__ void mainloop_checked(const MainParams& p, const Word* panel, const Word* bsrc,
                                                 const uint32_t (&base)[RPL], int kb0, int kb1, uint32_t quad,
                                                 const unsigned char* lut, float (&acc)[RPL][CPW])
{
    KCounter kc = kc_init(p, GATHER ? kb0 * 4 : kb0);
    int ku = kb0 * 4;
    int off[4];
    step_offsets<GATHER>(p, kc, ku, off);
    uint32_t wa[2][RPL], sa[2][RPL];
    uint32_t qb[2][UQ];
    load_lane(panel, base, off[0], wa[0], sa[0]);
    load_uniform(bsrc + (int64_t)kb0 * 4 * p.bld, quad, qb[0]);
    for (int kb = kb0; kb < kb1; ++kb) {
        const bool more = kb + 1 < kb1;
        int noff[4];
        if (more) step_offsets<GATHER>(p, kc, ku, noff);
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            const int cur = t & 1, nxt = cur ^ 1;
            if (t < 3) {
                load_lane(panel, base, off[t + 1], wa[nxt], sa[nxt]);
                load_uniform(bsrc + ((int64_t)kb * 4 + t + 1) * p.bld, quad, qb[nxt]);
            } else if (more) {
                load_lane(panel, base, noff[0], wa[nxt], sa[nxt]);
                load_uniform(bsrc + ((int64_t)kb + 1) * 4 * p.bld, quad, qb[nxt]);
            }
            checked_index(wa[cur], sa[cur], qb[cur], lut, acc, p.elo, p.ehi);
        }
        if (more) {
#pragma unroll
            for (int t = 0; t < 4; ++t) off[t] = noff[t];
        }
    }
}


// Native multiplier (4-byte words: the operands' own bits). The words of one
// k-step (4 consecutive reduction indices) for this lane: its RPL
// lane-operand rows, and its quarter of the wave's 16 uniform columns. The
// uniform words of an index are spread over the 4 lanes of every quad: lane
// i of a quad holds the words of columns 4i .. 4i + 3, read by the FMA with a
// DPP quad_perm broadcast of lane c >> 2 (register c & 3).
template <int RPL>
struct StepWords {
    uint32_t a[RPL][4];      // lane operand: row x, index t
    uint32_t u[4][4];        // uniform operand: index t, column 4 * quad + c
};

// Loads one k-step. Vector mode: a row's 4 words are contiguous (one 16-byte
// load at the counter's offset). Gather mode: every index has its own
// offset (or the zero region past the last index). urow: the uniform row of
// the k-step's first index plus this lane's quad offset.
template <bool GATHER, int RPL>
__device__ __forceinline__ void load_step(const MainParams& p, const uint32_t* panel, const uint32_t (&base)[RPL],
                                          const uint32_t* urow, KCounter& kc, int& ku, StepWords<RPL>& s)
{
    if (!GATHER) {
#pragma unroll
        for (int x = 0; x < RPL; ++x) {
            const uint4 q = *reinterpret_cast<const uint4*>(panel + base[x] + kc.off);
            s.a[x][0] = q.x; s.a[x][1] = q.y; s.a[x][2] = q.z; s.a[x][3] = q.w;
        }
        kc_next(p, kc);
    } else {
        int off[4];
        step_offsets<true>(p, kc, ku, off);
#pragma unroll
        for (int x = 0; x < RPL; ++x)
#pragma unroll
            for (int t = 0; t < 4; ++t) s.a[x][t] = panel[base[x] + off[t]];
    }
#pragma unroll
    for (int t = 0; t < 4; ++t) {
        const uint4 q = *reinterpret_cast<const uint4*>(urow + (int64_t)t * p.bld);
        s.u[t][0] = q.x; s.u[t][1] = q.y; s.u[t][2] = q.z; s.u[t][3] = q.w;
    }
}

// Native multiplier over one reduction index: the IEEE single-precision
// product folded by the hardware FMA, acc = fma(a, b, acc) (the product is
// exact inside the FMA; one rounding per step). No table lookup: this is the
// reference point the approximate product is compared against. The words are
// the operands' own bits, straight from their loads.
template <int RPL>
__device__ __forceinline__ void native_step_index(const uint32_t (&a)[RPL], const uint32_t (&u)[4], float (&acc)[RPL][CPW])
{
#pragma unroll
    for (int g = 0; g < CPW; ++g)
#pragma unroll
        for (int x = 0; x < RPL; ++x) fmac_quad(acc[x][g], u[g & 3], __uint_as_float(a[x]), g >> 2);
}

// The native multiplier's k-loop over k-steps [kb0, kb1): the words of
// k-step v are requested NS - 1 k-steps before use, into ring slot v % NS; a
// loop body covers NS k-steps, so every slot number is a compile-time
// constant, and the steady-state body has no branch (the compiler's wait
// counts for the ring stay exact).
template <bool GATHER, int NS, int RPL>
__device__ __forceinline__ void mainloop_native(const MainParams& p, const uint32_t* panel, const uint32_t* bsrc,
                                                const uint32_t (&base)[RPL], int kb0, int kb1, uint32_t quad,
                                                float (&acc)[RPL][CPW])
{
    auto fold = [&](const StepWords<RPL>& s) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            uint32_t a[RPL];
#pragma unroll
            for (int x = 0; x < RPL; ++x) a[x] = s.a[x][t];
            native_step_index(a, s.u[t], acc);
        }
    };
    constexpr int PD = NS - 1;
    const int n = kb1 - kb0;
    KCounter kc = kc_init(p, GATHER ? kb0 * 4 : kb0);
    int ku = kb0 * 4;
    const uint32_t* urow = bsrc + quad * 4 + (int64_t)kb0 * 4 * p.bld;
    const int64_t ustep = (int64_t)4 * p.bld;
    StepWords<RPL> s[NS];
    int v0 = 0;
    if (n >= NS + PD) {
        // unconditional prologue: the loop is entered with the same loads in
        // flight as at its back edge
#pragma unroll
        for (int v = 0; v < PD; ++v) {
            load_step<GATHER, RPL>(p, panel, base, urow, kc, ku, s[v]);
            urow += ustep;
            asm volatile("" ::: "memory");
        }
        // The compiler drains the loads in flight at the loop head; folding
        // k-step v0 before requesting k-step v0 + PD means that drain only
        // waits for loads that were issued at least one k-step earlier.
        for (; v0 + NS + PD <= n; v0 += NS) {
#pragma unroll
            for (int j = 0; j < NS; ++j) {
                if (j == 0) fold(s[0]);
                load_step<GATHER, RPL>(p, panel, base, urow, kc, ku, s[(j + PD) % NS]);
                urow += ustep;
                if (j > 0) fold(s[j]);
            }
        }
    } else {
#pragma unroll
        for (int v = 0; v < PD; ++v) {
            if (v < n) {
                load_step<GATHER, RPL>(p, panel, base, urow, kc, ku, s[v]);
                urow += ustep;
            }
        }
    }
    for (; v0 < n; v0 += NS) {                   // tail: fewer than NS + PD k-steps left
#pragma unroll
        for (int j = 0; j < NS; ++j) {
            if (v0 + j >= n) break;
            if (v0 + j + PD < n) {
                load_step<GATHER, RPL>(p, panel, base, urow, kc, ku, s[(j + PD) % NS]);
                urow += ustep;
            }
            fold(s[j]);
        }
    }
}

// LDSB: bytes of the LDS table image (LDS_SMALL or LDS_LARGE), or NATIVE_LDS
// where no table is staged (native multiplier, table in global memory).
constexpr int NATIVE_LDS = 16;

// GEMM-kernel calls of one variant run by one launch: call g owns work items
// [first[g], first[g + 1]) and its own exponent stats (p[g].stats); they
// share the table.
struct MainGroup {
    int count;
    int first[kMaxGroup + 1];
    MainParams p[kMaxGroup];
};

// This lane's slot of a call's exponent stats (a wave holds all 64 slots).
__device__ __forceinline__ int4 stats_slot(const MainParams& p)
{
    const int* sl = p.stats + ((threadIdx.x & 63) % STAT_SLOTS) * STAT_STRIDE;
    return make_int4(sl[0], sl[1], sl[2], sl[3]);
}

// Exponent-range test of one call from its stats slots, as loaded by
// stats_slot (every wave folds them itself: the table takes all of the LDS at
// M = 8, so the range is not broadcast through it). fast: no product can
// leave the format's range; ranged: some may fall below it (none above);
// otherwise the checked path.
template <bool NATIVE>
__device__ __forceinline__ void fold_stats(const MainParams& p, const int4& slot, bool& fast, bool& ranged)
{
    int v0 = slot.x, v1 = slot.y, v2 = slot.z, v3 = slot.w;
    for (int off = 32; off > 0; off >>= 1) {
        v0 = min(v0, __shfl_xor(v0, off, 64));
        v1 = max(v1, __shfl_xor(v1, off, 64));
        v2 = min(v2, __shfl_xor(v2, off, 64));
        v3 = max(v3, __shfl_xor(v3, off, 64));
    }
    const int a_min = __builtin_amdgcn_readfirstlane(v0), a_max = __builtin_amdgcn_readfirstlane(v1);
    const int b_min = __builtin_amdgcn_readfirstlane(v2), b_max = __builtin_amdgcn_readfirstlane(v3);
    const bool none = (a_min > a_max) || (b_min > b_max);       // an operand without normal values
    const bool no_over = none || (a_max + b_max - 126 <= p.ehi && a_max <= 253);
    const bool no_under = none || a_min + b_min - 127 >= p.elo;
    fast = NATIVE || (!p.force_checked && no_over && no_under);
    ranged = !NATIVE && !p.force_checked && no_over && !no_under;
}

// Path of k-segment s of a call whose own range failed the fast test (as
// fold_stats, from the segment's ranges): 0 fast, 1 fast with underflow, 2
// checked; `call_mode` (1 or 2) where a range is unknown.
__device__ __forceinline__ int seg_mode(const MainParams& p, int s, int call_mode)
{
    const uint32_t* r = reinterpret_cast<const uint32_t*>(p.stats) + STAT_SEG + 4 * SEG_REPL * s;
    const uint32_t g = p.seg_gen;
    uint32_t la = 0, lb = 0, ua = 0, ub = 0;
#pragma unroll
    for (int q = 0; q < SEG_REPL; ++q) {
        la = max(la, r[4 * q]);
        lb = max(lb, r[4 * q + 1]);
        ua = max(ua, r[4 * q + 2]);
        ub = max(ub, r[4 * q + 3]);
    }
    // a tag below the call's: the call wrote nothing there (that operand has
    // no normal values in the segment, so no product can leave the range)
    if ((la & ~0xFFu) < g || (ua & ~0xFFu) < g) return 0;
    if ((la & ~0xFFu) != g || (lb & ~0xFFu) != g || (ua & ~0xFFu) != g || (ub & ~0xFFu) != g) return call_mode;
    const int a_min = 255 - (int)(la & 0xFFu), a_max = (int)(lb & 0xFFu);
    const int b_min = 255 - (int)(ua & 0xFFu), b_max = (int)(ub & 0xFFu);
    const bool no_over = a_max + b_max - 126 <= p.ehi && a_max <= 253;
    const bool no_under = a_min + b_min - 127 >= p.elo;
    return no_over ? (no_under ? 0 : 1) : 2;
}

// After every wave of the workgroup has read a call's stats (a barrier
// between): the last of the `readers` workgroups to do so resets them (and
// the count) for the stream's next call. Wave 0 only.
__device__ __forceinline__ void release_stats(const MainParams& p, int readers)
{
    static_assert(STAT_SLOTS == 64, "one slot per lane of a wave");
    int* stats = const_cast<int*>(p.stats);
    int ticket = 0;
    if (threadIdx.x == 0) ticket = atomicAdd(stats + STAT_READERS, 1);
    ticket = __shfl(ticket, 0, 64);
    if (ticket == readers - 1) {
        int* slot = stats + threadIdx.x * STAT_STRIDE;
        for (int t = 0; t < 4; ++t) slot[t] = stat_reset_value(t);
        if (threadIdx.x == 0) stats[STAT_READERS] = 0;
    }
}

// GTAB: the table (M = 9..11, too large for LDS) is read from global memory,
// where it stays resident in L2 / the last-level cache; LDSB is then unused.
// GROUP: the kernel argument is a MainGroup (calls chosen per work item);
// otherwise one call's MainParams, kept as the kernel's own argument so its
// fields stay in scalar registers through the main loop.
template <bool GROUP>
using MainArg = typename std::conditional<GROUP, MainGroup, MainParams>::type;

template <bool GROUP>
__device__ __forceinline__ const MainParams& call_params(const MainArg<GROUP>& a, int g)
{
    if constexpr (GROUP) return a.p[g];
    else return a;
}

template <int LDSB, bool GATHER, bool NATIVE, int NW, int RPL, bool GTAB, bool GROUP>
__global__ __launch_bounds__(NW * 64, 1) void main_kernel(MainArg<GROUP> grp)
{
    constexpr int NT = NW * 64;
    constexpr int LA = GTAB ? LA_GLOBAL : LA_LDS;
    __shared__ __align__(16) unsigned char lds_tab[LDSB];
    const MainParams& p0 = call_params<GROUP>(grp, 0);
    const int G = gridDim.x;
    // XCD-aware order: workgroups are dealt to the 8 XCDs round-robin (block
    // b runs on XCD b % 8, checked with HW_REG_XCC_ID), so give the workgroups
    // of one XCD consecutive work items: they share operand rows in its L2.
    // (A bijection of the block index: with the items of a call consecutive,
    // min(G, its items) workgroups read its stats.)
    const int v = (G & 7) == 0 ? (int)((blockIdx.x & 7u) * (unsigned)(G >> 3) + (blockIdx.x >> 3)) : (int)blockIdx.x;
    int items, cur = -1;                           // cur: the call whose stats this workgroup has folded
    if constexpr (GROUP) items = grp.first[grp.count];
    else items = (int)grp.items;
    // the stats of the first item's call, requested before the table copy so
    // that the two loads' latencies overlap
    int g0 = 0;
    if constexpr (GROUP)
        while (g0 + 1 < grp.count && v >= (int)grp.first[g0 + 1]) ++g0;
    const int4 slot0 = v < items ? stats_slot(call_params<GROUP>(grp, g0)) : make_int4(0, 0, 0, 0);
    if (!NATIVE && !GTAB) {
        const uint4* src = reinterpret_cast<const uint4*>(p0.lut);
        uint4* dst = reinterpret_cast<uint4*>(lds_tab);
        const int n16 = p0.lut_bytes >> 4;
        for (int t = threadIdx.x; t < n16; t += NT) dst[t] = src[t];
    }
    const unsigned char* lut;
    if constexpr (GTAB) lut = reinterpret_cast<const unsigned char*>(p0.lut);
    else lut = lds_tab;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const uint32_t quad = (uint32_t)lane & 3u;     // this lane's place in the uniform-word quads
    bool fast = false, ranged = false;
    uint32_t folded = 0;                           // the calls whose stats this workgroup has read

    for (int item = v; item < items; item += G) {
        int g = 0, first = 0, count = items;
        if constexpr (GROUP) {
            while (g + 1 < grp.count && item >= grp.first[g + 1]) ++g;
            first = grp.first[g];
            count = grp.first[g + 1] - first;
        }
        const MainParams& p = call_params<GROUP>(grp, g);
        if (g != cur) {                            // uniform: every wave of the workgroup enters together
            fold_stats<NATIVE>(p, cur < 0 ? slot0 : stats_slot(p), fast, ranged);
            __syncthreads();                       // the table is staged; every wave has read the stats
            folded |= 1u << g;
            cur = g;
        }
        const int wrow = wave / p.wc, wcol = wave - wrow * p.wc;
        const int TM = p.wr * 64 * RPL, TN = p.wc * CPW;
        const int tiles = p.tiles_m * p.tiles_n;
        const int li = item - first;               // the item within its call
        int tl, split;                             // (batch entry, tile) pair; split -1: whole
        if (li < p.full_items) {
            tl = li;
            split = -1;
        } else {
            const int t2 = li - p.full_items;
            split = t2 / p.tail_tiles;
            tl = p.full_items + (t2 - split * p.tail_tiles);
        }
        const int tile = tl % tiles;
        const int b = tl / tiles;
        int tm, tn;
        tile_coords(tile, p.tiles_m, p.tiles_n, tm, tn);
        const int row0 = tm * TM + wrow * 64 * RPL;
        const int col0 = tn * TN + wcol * CPW;
        if (row0 >= p.m_out || col0 >= p.n_out) continue;   // this wave has no output in the tile
        uint32_t base[RPL];
#pragma unroll
        for (int x = 0; x < RPL; ++x) {
            const int i = min(row0 + x * 64 + lane, p.m_rows - 1);
            const int i3 = i % p.E3, r2 = i / p.E3;
            const int i2 = r2 % p.E2, i1 = r2 / p.E2;
            base[x] = (uint32_t)(i1 * p.L1 + i2 * p.L2 + i3 * p.L3);
        }
        // table: 8-byte Words; native multiplier: 4-byte words (the operands' bits)
        const Word* panel = static_cast<const Word*>(p.panel) + (int64_t)b * p.panel_batch;
        const Word* bsrc = static_cast<const Word*>(p.bpanel) + (int64_t)b * p.bpanel_batch + col0;
        const uint32_t* npanel = static_cast<const uint32_t*>(p.panel) + (int64_t)b * p.panel_batch;
        const uint32_t* nbsrc = static_cast<const uint32_t*>(p.bpanel) + (int64_t)b * p.bpanel_batch + col0;
        const int kb0 = split < 0 ? 0 : split * p.chunk;
        const int kb1 = split < 0 ? p.KB : min(p.KB, kb0 + p.chunk);

        float acc[RPL][CPW];
#pragma unroll
        for (int x = 0; x < RPL; ++x)
#pragma unroll
            for (int j = 0; j < CPW; ++j) acc[x][j] = 0.0f;

        if (kb0 < kb1) {
            // a ring of 3 k-steps; 2 in the 12-wave shape, whose registers hold no third
            if constexpr (NATIVE) mainloop_native<GATHER, NW == 12 ? 2 : 3, RPL>(p, npanel, nbsrc, base, kb0, kb1, quad, acc);
            else if (fast) mainloop_fast<GATHER, false, 4, RPL, LA, GTAB ? 0 : AMX_GOFF>(p, panel, bsrc, base, kb0, kb1, quad, lut, acc);
            else if (p.segs > 0 && !p.force_checked) {
                // the call's range failed the fast test: each k-segment (16
                // k-steps) on the path its own ranges allow, in ascending order
                // (the paths give the same bits wherever more than one applies)
                for (int ka = kb0; ka < kb1;) {
                    const int sg = ka / SEG_KSTEPS, kz = min(kb1, (sg + 1) * SEG_KSTEPS);
                    const int mode = seg_mode(p, sg, ranged ? 1 : 2);
                    if (mode == 0)
                        mainloop_fast<GATHER, false, 4, RPL, LA, GTAB ? 0 : AMX_GOFF>(p, panel, bsrc, base, ka, kz, quad, lut, acc);
                    else if (mode == 1)
                        mainloop_fast<GATHER, true, 4, RPL, LA>(p, panel, bsrc, base, ka, kz, quad, lut, acc);
                    else
                        mainloop_checked<GATHER, RPL>(p, panel, bsrc, base, ka, kz, quad, lut, acc);
                    ka = kz;
                }
            } else {
                if (ranged) mainloop_fast<GATHER, true, 4, RPL, LA>(p, panel, bsrc, base, kb0, kb1, quad, lut, acc);
                else mainloop_checked<GATHER, RPL>(p, panel, bsrc, base, kb0, kb1, quad, lut, acc);
            }
        }

        gfloat_ptr out;
        int ld;
        if (split >= 0) {
            out = (gfloat_ptr)(p.ws + ((int64_t)b * p.splits + split) * (int64_t)p.m_out * p.n_out);
            ld = p.n_out;
        } else {
            out = (gfloat_ptr)(p.out_ptrs ? p.out_ptrs[b] : p.out + (int64_t)b * p.out_batch);
            ld = p.ldc;
        }
        // a lane's 16 columns of a row are contiguous: 16-byte stores when
        // the rows are 16-byte aligned and the wave's columns are all inside
        const bool vec = ((reinterpret_cast<uintptr_t>(out) & 15u) == 0) && ((ld & 3) == 0) && (col0 + CPW <= p.n_out);
#pragma unroll
        for (int x = 0; x < RPL; ++x) {
            const int i = row0 + x * 64 + lane;
            if (i < p.m_out) {
                gfloat_ptr o = out + (int64_t)i * ld + col0;
                if (vec) {
#pragma unroll
                    for (int j = 0; j < CPW; j += 4)
                        *reinterpret_cast<gv4f_ptr>(o + j) = v4f{acc[x][j], acc[x][j + 1], acc[x][j + 2], acc[x][j + 3]};
                } else {
#pragma unroll
                    for (int j = 0; j < CPW; ++j)
                        if (col0 + j < p.n_out) o[j] = acc[x][j];
                }
            }
        }
    }
    // Release the stats of the calls this workgroup read, after its last
    // item rather than at the first (the release's atomic round trip then
    // holds back no wave's k-loop); every wave read them before the barrier
    // that followed its fold.
    if (threadIdx.x < 64) {
        if constexpr (GROUP) {
            for (int g = 0; g < grp.count; ++g)
                if ((folded >> g) & 1u) release_stats(grp.p[g], min(G, (int)(grp.first[g + 1] - grp.first[g])));
        } else {
            if (folded & 1u) release_stats(grp, min(G, items));
        }
    }
}

// ------------------------------------------------------------------ row-vector GEMM


// sign | exponent of an operand for the checked product: 0 for zero and
// subnormal, +-Inf for Inf, 0x7FC00000 for NaN (as the decode pass writes).
__device__ __forceinline__ uint32_t se_of(uint32_t bits)
{
    const uint32_t e = (bits >> 23) & 0xFFu;
    const uint32_t se = e == 0u ? 0u : (bits & 0xFF800000u);
    return (e == 255u && (bits & 0x7FFFFFu)) ? 0x7FC00000u : se;
}

// C[r][j] = sum_kk approx(op(A)(r, kk), B[kk][j]) for few rows r < m.
// Work item (column block, block of up to kGemvMaxRows rows, split, batch
// entry): lane t owns columns
// block * NTG * kGemvColsPerLane + t + c * NTG (coalesced across the wave for
// every c) and sums reduction indices [split * chunk, (split + 1) * chunk) in
// ascending order. Columns past n read column n - 1 and are not stored, so
// the loop has no divergent branch. op(A) is the same for the whole wave at
// each index, so it is read with scalar loads and its sign, exponent and
// table row are worked out in scalar registers; a row of B is addressed as a
// wave-uniform base plus the lane's 32-bit column offset. PADROWS: the table
// is staged once per persistent workgroup in LDS as 2^M rows (one per op(A)
// mantissa index) of 2^M entries plus a pad (the pad entries are read by the
// checked path only). Otherwise (M = 9..11, and the checked path of the
// one-row kernel below) the table is read from global memory in index order.
//
// Fast path: with e the pair's table entry and seB the sign|exponent bits of
// B, y = as_float(0x3F800000 + (e << 8)) * as_float(seB) is
// +-(1.f) * 2^(EB-127+carry), the AMSim product of B with an op(A) operand of
// exponent 0, and fma(y, as_float(seA), acc) adds the product with one
// rounding: exact while every product stays inside the range (FP32), or no
// product exceeds it (a narrower format, whose products below it are zeroed
// first, as in the GEMM kernel's path with underflow). A zero or subnormal B
// has seB = +-0, so y is +-0 whatever entry is read. Per item the wave takes
// the exponent range of its op(A) chunk, which fixes the window [lo, hi] of
// B exponents that keeps every product inside; each lane keeps the largest
// |as_float(seB)|, which is below 2^(hi + 1 - 127) exactly when no exponent
// exceeds hi and no B is Inf or NaN (their seB is +-Inf), and the smallest
// (B bits << 1) - 2^24, which is at least (lo - 1) << 24 exactly when no
// normal exponent is below lo (zero and subnormal B wrap past every normal
// value). If any lane of the
// wave finds an element outside the window, the wave redoes its columns of
// the item with the checked path (Algorithm 2 as selects), which gives the
// same bits wherever both apply.
// Reduction indices whose operands are requested together in the row-vector kernels.
constexpr int GG = 8;

typedef const float __attribute__((address_space(4)))* cfloat_cptr;
typedef const uint32_t __attribute__((address_space(1)))* gu32_cptr;
typedef const uint16_t __attribute__((address_space(1)))* gu16_cptr;
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef const u32x4 __attribute__((address_space(1)))* gu4_cptr;

// Operand loads of the row-vector kernels for one work item over reduction
// indices [k0, k1). op(A) is read through the constant address space: it is
// not written while a kernel runs, and a wave-uniform index then gives a
// scalar load. A group of rows of B is read through a buffer descriptor
// (gemv_group_base: its rows and offsets): the lane's column offset plus a
// wave-uniform row offset, no 64-bit address arithmetic per load; the
// descriptor's extent ends with the group's last row. Rows of 2^26 floats or
// more (a group's row offsets would pass 2^32 bytes): one descriptor per row.
template <int MR, int NTG>
struct GemvOperands {
    const GemvParams& p;
    gfloat_cptr B;
    cfloat_cptr As;
    int k1;
    uint32_t ldb4;
    bool wide;
    uint32_t boff[kGemvColsPerLane];        // the lane's columns as byte offsets within a row of B (n < 2^30)

    __device__ __forceinline__ GemvOperands(const GemvParams& p_, gfloat_cptr A, gfloat_cptr B_, int j0, int k1_)
        : p(p_), B(B_), As((cfloat_cptr)(uintptr_t)A), k1(k1_), ldb4((uint32_t)p_.ldb * 4u), wide(p_.ldb >= (1 << 26))
    {
#pragma unroll
        for (int c = 0; c < kGemvColsPerLane; ++c) boff[c] = (uint32_t)min(j0 + c * NTG, p.n - 1) * 4u;
    }

    __device__ __forceinline__ uint32_t a_raw(int r, int kk) const
    {
        return __float_as_uint(p.transA ? As[(int64_t)kk * p.lda + r] : As[(int64_t)r * p.lda + kk]);
    }

    template <int NG>
    __device__ __forceinline__ void load(int kg, uint32_t (&bw)[NG][kGemvColsPerLane], uint32_t (&xa)[NG][MR]) const
    {
        const int base = gemv_group_base(kg, k1);
        if (!wide) {
            const uint32_t extent = (uint32_t)gemv_group_step(kg, k1, NG - 1) * ldb4 + (uint32_t)p.n * 4u;
            const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                (void*)(uintptr_t)((gbyte_ptr)B + (int64_t)base * p.ldb * 4), 0, (int)extent, kBufferConfig);
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const uint32_t so = (uint32_t)gemv_group_step(kg, k1, g) * ldb4;
#pragma unroll
                for (int c = 0; c < kGemvColsPerLane; ++c)
                    bw[g][c] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)boff[c], (int)so, 0);
            }
        } else {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const int64_t row = base + gemv_group_step(kg, k1, g);
                const __amdgpu_buffer_rsrc_t rsrc = __builtin_amdgcn_make_buffer_rsrc(
                    (void*)(uintptr_t)((gbyte_ptr)B + row * p.ldb * 4), 0, (int)((uint32_t)p.n * 4u), kBufferConfig);
#pragma unroll
                for (int c = 0; c < kGemvColsPerLane; ++c)
                    bw[g][c] = (uint32_t)__builtin_amdgcn_raw_buffer_load_b32(rsrc, (int)boff[c], 0, 0);
            }
        }
#pragma unroll
        for (int g = 0; g < NG; ++g)
#pragma unroll
            for (int r = 0; r < MR; ++r) xa[g][r] = a_raw(r, base + gemv_group_step(kg, k1, g));
    }
};

// Exponent range of the normal op(A) elements of rows [0, MR) over indices
// [k0, k1) (whole wave), and whether any is NaN; the window [lo, hi] of B
// exponents that keeps every product of them inside the format's range
// (lo > hi: none does).
//   B exponents eb (normal) that keep every product at or below the format's
// top ehi (and eb + carry below 255, so y stays finite). FP32 (FMT false):
// also at or above its bottom, else the checked path. A narrower format
// (FMT): products below the bottom elo are zeroed in the loop instead: y below
// 2^(elo - EA) (EA: op(A)'s biased exponent) means an underflow, the bound
// being 0 for Inf / NaN op(A) and 2^elo for a zero op(A).
template <int MR, bool FMT, typename Ops>
__device__ __forceinline__ void gemv_window(const GemvParams& p, const Ops& ops, int k0, int k1, int& lo, int& hi,
                                            bool& a_nan_any)
{
    const int lane = threadIdx.x & 63;
    int emin = 255, emax = 0;
    bool a_nan = false;
#pragma unroll
    for (int r = 0; r < MR; ++r)
        for (int kk = k0 + lane; kk < k1; kk += 64) {
            uint32_t bits = ops.a_raw(r, kk);
            if constexpr (FMT) bits = cast_fmt(bits, p.elo, p.ehi);
            const int e = (int)((bits >> 23) & 0xFFu);
            const bool normal = e != 0 && e != 255;
            emin = normal ? min(emin, e) : emin;
            emax = normal ? max(emax, e) : emax;
            a_nan |= (bits & 0x7FFFFFFFu) > 0x7F800000u;
        }
    for (int off = 32; off > 0; off >>= 1) {
        emin = min(emin, __shfl_xor(emin, off, 64));
        emax = max(emax, __shfl_xor(emax, off, 64));
    }
    lo = (FMT || emin > emax) ? 1 : max(1, p.elo + 127 - emin);
    hi = emin > emax ? 253 : min(253, p.ehi + 126 - emax);
    a_nan_any = __any(a_nan);
}

// One B element of the fast path: the table column index, the sign|exponent
// of B as a float (+-2^(EB-127), +-0 for zero and subnormal, +-Inf for Inf
// and NaN), and the lane's window accumulators: the largest |sign|exponent|
// and the smallest (B bits << 1) - 2^24.
__device__ __forceinline__ void gemv_fast_b(uint32_t bits, int sh, int M, float& smax, uint32_t& wmin, uint32_t& ix,
                                            float& sb)
{
    ix = __builtin_amdgcn_ubfe(bits, (uint32_t)sh, (uint32_t)M);
    sb = __uint_as_float(bits & 0xFF800000u);
    smax = __builtin_fmaxf(smax, __builtin_fabsf(sb));
    wmin = min(wmin, (bits << 1) - (1u << 24));
}

// One fast-path product added to acc: e the table entry, sb B's sign|exponent,
// seA op(A)'s sign|exponent bits (+-0 for a zero or subnormal op(A): the sign
// of a zero product never shows, as every sum starts from +0; +-Inf for Inf).
template <bool FMT>
__device__ __forceinline__ void gemv_fast_fma(float& acc, uint32_t e, float sb, uint32_t seA, int elo)
{
    const float y = __uint_as_float(0x3F800000u + (e << 8)) * sb;
    float yk = y;
    if constexpr (FMT) {
        const float tA = __int_as_float(max((int)((uint32_t)(elo + 127) << 23) - (int)(seA & 0x7F800000u), 0));
        yk = __builtin_fabsf(y) < tA ? 0.0f : y;
    }
    acc = __builtin_fmaf(yk, __uint_as_float(seA), acc);
}

// force: skip the fast path (the caller's fast path has failed its window).
template <int MR, bool NATIVE, int NTG, bool FMT, bool PADROWS>
__device__ __forceinline__ void gemv_item(const GemvParams& p, const uint16_t* lut, gfloat_cptr A, gfloat_cptr B,
                                          int j0, int k0, int k1, float (&acc)[kGemvMaxRows][kGemvColsPerLane],
                                          bool force = false)
{
    const int sh = 23 - p.M;
    const uint32_t mmask = (1u << p.M) - 1u;
    const uint32_t rs = (1u << p.M) + 8u;           // PADROWS: entries per row of the LDS image
    const GemvOperands<MR, NTG> ops(p, A, B, j0, k1);
    // operands are cast to the multiplier's format where they are used (the
    // native multiplier takes them as they are); a group's loads stay
    // together ahead of the casts
    auto cast = [&](uint32_t bits) -> uint32_t { return FMT ? cast_fmt(bits, p.elo, p.ehi) : bits; };
    // the item's indices in groups of GG, handed to use(count, B words, op(A)
    // words) in ascending order (a group past k1 - 1 reads row k1 - 1, unused)
    auto stream = [&](auto&& use) {
        for (int kg = k0; kg < k1; kg += GG) {
            uint32_t bw[GG][kGemvColsPerLane], xa[GG][MR];
            ops.load(kg, bw, xa);
            __builtin_amdgcn_sched_barrier(0);     // keep the group's loads issued together
            use(min(GG, k1 - kg), bw, xa);
        }
    };
#pragma unroll
    for (int r = 0; r < kGemvMaxRows; ++r)
#pragma unroll
        for (int c = 0; c < kGemvColsPerLane; ++c) acc[r][c] = 0.0f;

    bool checked = !NATIVE;
    if constexpr (!NATIVE) {
        int lo, hi;
        bool a_nan;
        gemv_window<MR, FMT>(p, ops, k0, k1, lo, hi, a_nan);
        // a NaN op(A) element sends the item to the checked path (the fast
        // product takes op(A)'s sign|exponent bits as they are)
        checked = force || lo > hi || p.force_checked || a_nan;
        if (!checked) {
            const float hi_s = __uint_as_float((uint32_t)(hi + 1) << 23);
            const uint32_t lo_w = (uint32_t)(lo - 1) << 24;
            float smax = 0.0f;
            uint32_t wmin = 0xFFFFFFFFu;
            stream([&](int cnt, const uint32_t (&bw)[GG][kGemvColsPerLane], const uint32_t (&xa)[GG][MR]) {
#pragma unroll
                for (int g = 0; g < GG; ++g) {
                    if (g >= cnt) break;
                    uint32_t ix[kGemvColsPerLane];
                    float sb[kGemvColsPerLane];
#pragma unroll
                    for (int c = 0; c < kGemvColsPerLane; ++c) gemv_fast_b(cast(bw[g][c]), sh, p.M, smax, wmin, ix[c], sb[c]);
                    // the index's lookups are issued together, then used
                    uint32_t e[MR][kGemvColsPerLane];
#pragma unroll
                    for (int r = 0; r < MR; ++r) {
                        const uint32_t ia = (cast(xa[g][r]) >> sh) & mmask;
                        if constexpr (PADROWS) {
                            const uint16_t* row = lut + ia * rs;
#pragma unroll
                            for (int c = 0; c < kGemvColsPerLane; ++c) e[r][c] = row[ix[c]];
                        } else {
                            const gbyte_ptr row = (gbyte_ptr)lut + (ia << (p.M + 1));
#pragma unroll
                            for (int c = 0; c < kGemvColsPerLane; ++c)
                                e[r][c] = *reinterpret_cast<gu16_cptr>(row + (ix[c] << 1));
                        }
                    }
#pragma unroll
                    for (int r = 0; r < MR; ++r) {
                        const uint32_t seA = cast(xa[g][r]) & 0xFF800000u;
#pragma unroll
                        for (int c = 0; c < kGemvColsPerLane; ++c) gemv_fast_fma<FMT>(acc[r][c], e[r][c], sb[c], seA, p.elo);
                    }
                }
            });
            checked = __any(!(smax < hi_s) || wmin < lo_w);
            if (checked) {
#pragma unroll
                for (int r = 0; r < kGemvMaxRows; ++r)
#pragma unroll
                    for (int c = 0; c < kGemvColsPerLane; ++c) acc[r][c] = 0.0f;
            }
        }
    }
    if (!checked && !NATIVE) return;
    stream([&](int cnt, const uint32_t (&bw)[GG][kGemvColsPerLane], const uint32_t (&xa)[GG][MR]) {
#pragma unroll
        for (int g = 0; g < GG; ++g) {
            if (g >= cnt) break;
#pragma unroll
            for (int r = 0; r < MR; ++r) {
                if constexpr (NATIVE) {
#pragma unroll
                    for (int c = 0; c < kGemvColsPerLane; ++c)
                        acc[r][c] = __builtin_fmaf(__uint_as_float(xa[g][r]), __uint_as_float(bw[g][c]), acc[r][c]);
                } else {
                    const uint32_t xr = cast(xa[g][r]);
                    const uint32_t seA = se_of(xr);
                    const uint32_t ia = (xr >> sh) & mmask;
                    const uint32_t row = PADROWS ? ia * rs : ia << p.M;
#pragma unroll
                    for (int c = 0; c < kGemvColsPerLane; ++c) {
                        const uint32_t bc = cast(bw[g][c]);
                        const uint32_t e = lut[row + ((bc >> sh) & mmask)];
                        acc[r][c] = checked_product_acc(acc[r][c], e, seA, se_of(bc), p.elo, p.ehi);
                    }
                }
            }
        }
    });
}

// Item order of the row-vector kernels: row blocks fastest, so the items of
// one (column block, chunk) read the same stretch of B. Workgroup b runs on
// XCD b % 8, so the workgroups of one XCD take consecutive items (as in the
// GEMM kernel): those row blocks then share B through that XCD's L2.
__device__ __forceinline__ int gemv_first_item()
{
    const int G = gridDim.x;
    return (G & 7) == 0 ? (int)((blockIdx.x & 7u) * (unsigned)(G >> 3) + (blockIdx.x >> 3)) : (int)blockIdx.x;
}

// The item's outputs: rows r0 .. r0 + mr - 1 of C, or of the item's split
// partials.
template <int NTG>
__device__ __forceinline__ void gemv_store(const GemvParams& p, int b, int split, int r0, int mr, int j0,
                                           const float (&acc)[kGemvMaxRows][kGemvColsPerLane])
{
    gfloat_ptr out;
    int64_t ld;
    if (p.splits > 1) {
        out = (gfloat_ptr)(p.out + ((int64_t)b * p.splits + split) * (int64_t)p.m * p.n);
        ld = p.n;
    } else {
        out = (gfloat_ptr)(p.out_ptrs ? p.out_ptrs[b] : p.out + b * p.out_batch);
        ld = p.ldc;
    }
#pragma unroll
    for (int r = 0; r < kGemvMaxRows; ++r) {
        if (r >= mr) break;
#pragma unroll
        for (int c = 0; c < kGemvColsPerLane; ++c)
            if (j0 + c * NTG < p.n) out[(int64_t)(r0 + r) * ld + j0 + c * NTG] = acc[r][c];
    }
}

// TABB > 0: bytes of the LDS table image, 2^M rows of 2^M + 8 entries (the
// op(A) element's row; entry 2^M of a row is 0, entry 2^M + 1 is 1).
template <bool NATIVE, int TABB, int NTG>
__global__ __launch_bounds__(NTG) void gemv_kernel(GemvParams p)
{
    constexpr bool PR = TABB > 0;
    __shared__ __align__(16) uint16_t tab[TABB > 0 ? TABB / 2 : 8];
    const uint16_t* lut = p.lut;
    if constexpr (TABB > 0) {
        const int rl = 1 << p.M, rs = rl + 8;
        if (p.M >= 3) {                            // 16-byte chunks: rows of 2 * rl bytes, 2 * rs apart
            const int cpr = rl >> 3;
            const uint4* src = reinterpret_cast<const uint4*>(p.lut);
            uint4* dst = reinterpret_cast<uint4*>(tab);
            for (int t = threadIdx.x; t < rl * cpr; t += NTG) {
                const int r = t / cpr, q = t - r * cpr;
                dst[r * (rs >> 3) + q] = src[t];
            }
        } else {
            for (int t = threadIdx.x; t < rl * rl; t += NTG) tab[(t >> p.M) * rs + (t & (rl - 1))] = p.lut[t];
        }
        for (int r = threadIdx.x; r < rl; r += NTG) {
            tab[r * rs + rl] = 0;
            tab[r * rs + rl + 1] = 1;
        }
        __syncthreads();
        lut = tab;
    }
    constexpr int COLS = NTG * kGemvColsPerLane;
    const int nblk = (p.n + COLS - 1) / COLS;
    const int rblk = (p.m + kGemvMaxRows - 1) / kGemvMaxRows;    // blocks of up to 4 rows of op(A)
    const int items = nblk * rblk * p.splits * p.batch;
    for (int item = gemv_first_item(); item < items; item += gridDim.x) {
        const int rb = item % rblk;
        int rest = item / rblk;
        const int blk = rest % nblk;
        rest /= nblk;
        const int split = rest % p.splits;
        const int b = rest / p.splits;
        const int r0 = rb * kGemvMaxRows, mr = min(kGemvMaxRows, p.m - r0);
        const gfloat_cptr A = (gfloat_cptr)(p.A_ptrs ? p.A_ptrs[b] : p.A + b * p.A_batch) +
                              (p.transA ? (int64_t)r0 : (int64_t)r0 * p.lda);
        const gfloat_cptr B = (gfloat_cptr)(p.B_ptrs ? p.B_ptrs[b] : p.B + b * p.B_batch);
        const int j0 = blk * COLS + threadIdx.x;
        const int k0 = split * p.chunk, k1 = min(p.k, k0 + p.chunk);
        float acc[kGemvMaxRows][kGemvColsPerLane];
        if (!NATIVE && (p.elo != 1 || p.ehi != 254)) {      // a format narrower than FP32
            switch (mr) {
            case 1: gemv_item<1, NATIVE, NTG, !NATIVE, PR>(p, lut, A, B, j0, k0, k1, acc); break;
            case 2: gemv_item<2, NATIVE, NTG, !NATIVE, PR>(p, lut, A, B, j0, k0, k1, acc); break;
            case 3: gemv_item<3, NATIVE, NTG, !NATIVE, PR>(p, lut, A, B, j0, k0, k1, acc); break;
            default: gemv_item<4, NATIVE, NTG, !NATIVE, PR>(p, lut, A, B, j0, k0, k1, acc); break;
            }
        } else {
            switch (mr) {
            case 1: gemv_item<1, NATIVE, NTG, false, PR>(p, lut, A, B, j0, k0, k1, acc); break;
            case 2: gemv_item<2, NATIVE, NTG, false, PR>(p, lut, A, B, j0, k0, k1, acc); break;
            case 3: gemv_item<3, NATIVE, NTG, false, PR>(p, lut, A, B, j0, k0, k1, acc); break;
            default: gemv_item<4, NATIVE, NTG, false, PR>(p, lut, A, B, j0, k0, k1, acc); break;
            }
        }
        gemv_store<NTG>(p, b, split, r0, mr, j0, acc);
    }
}

// One row of op(A) (m = 1) and a table of M <= 8: the lookups of index kk all
// read table row ia(kk), so instead of a whole-table copy per 1024-thread
// workgroup, a 256-thread workgroup stages, per window of kG1Window indices,
// just the window's rows (one per index, in index order) into LDS, double-
// buffered: the next window's rows are requested while the lookups of the
// current window read the other buffer, and stored after them. 32 KB of LDS
// per workgroup leaves room for several workgroups per CU. Same work items,
// window test and fast product as gemv_item; a wave that fails its window
// redoes its columns with gemv_item's checked path (table in global memory).
template <bool FMT>
__device__ __forceinline__ void gemv1_item(const GemvParams& p, unsigned char* rows, gfloat_cptr A, gfloat_cptr B,
                                           int j0, int k0, int k1, float (&acc)[kGemvMaxRows][kGemvColsPerLane])
{
    constexpr int NTG = kGemv1Threads, W = kGemv1Window;
    constexpr int G1 = 4;                               // indices per group load (8: 119 VGPRs, 3% slower)
    const int M = p.M, sh = 23 - M;
    const uint32_t mmask = (1u << M) - 1u;
    const GemvOperands<1, NTG> ops(p, A, B, j0, k1);
    auto cast = [&](uint32_t bits) -> uint32_t { return FMT ? cast_fmt(bits, p.elo, p.ehi) : bits; };
#pragma unroll
    for (int r = 0; r < kGemvMaxRows; ++r)
#pragma unroll
        for (int c = 0; c < kGemvColsPerLane; ++c) acc[r][c] = 0.0f;

    int lo, hi;
    bool a_nan;
    gemv_window<1, FMT>(p, ops, k0, k1, lo, hi, a_nan);
    // the same for every wave of the workgroup (one op(A) chunk), so all of
    // them run the windows and their barriers, or none
    bool checked = lo > hi || p.force_checked || a_nan;
    if (!checked) {
        // staging: a window's rows in pieces of 16 bytes (M >= 3) or 4 bytes
        // (M = 1, 2: rows of 4 and 8 bytes); at most W * 512 / 16 = 1024
        // pieces, kGemv1Stage per thread (a window past k1 - 1 loads rows it
        // does not store)
        const int rlog = M + 1;                             // log2 of the bytes per row
        const int ulog = M >= 3 ? 4 : 2;
        const int plog = rlog - ulog;                       // log2 of the pieces per row
        const int pieces = W << plog;
        const int tid = threadIdx.x;
        // piece q of a window: row t = q >> plog of the window (the table row
        // of op(A) at the window's index t, clamped to k1 - 1), stored at byte
        // q << ulog of the window's buffer. a_for reads that op(A) element
        // (one window ahead of fetch, so fetch waits on nothing recent); fetch
        // reads the piece from the table in global memory.
        auto a_for = [&](int q, int w0) -> uint32_t {
            return ops.a_raw(0, w0 >= k1 - 1 ? k1 - 1 : w0 + min(q >> plog, k1 - 1 - w0));
        };
        auto fetch = [&](int q, uint32_t abits) -> u32x4 {
            u32x4 v = {0u, 0u, 0u, 0u};
            if (q < pieces) {
                const uint32_t ia = (cast(abits) >> sh) & mmask;
                const gbyte_ptr src =
                    (gbyte_ptr)p.lut + ((size_t)ia << rlog) + ((size_t)(q & ((1 << plog) - 1)) << ulog);
                if (ulog == 4) v = *reinterpret_cast<gu4_cptr>(src);
                else v.x = *reinterpret_cast<gu32_cptr>(src);
            }
            return v;
        };
        auto put = [&](int buf, int q, u32x4 v) {
            if (q < pieces) {
                unsigned char* d = rows + ((size_t)buf << (rlog + 5)) + ((size_t)q << ulog);   // 32 rows a buffer
                if (ulog == 4) *reinterpret_cast<u32x4*>(d) = v;
                else *reinterpret_cast<uint32_t*>(d) = v.x;
            }
        };
        static_assert(kGemv1Stage == 4 && kGemv1Window == 32, "four pieces per thread, 32 rows per buffer");
        const float hi_s = __uint_as_float((uint32_t)(hi + 1) << 23);
        const uint32_t lo_w = (uint32_t)(lo - 1) << 24;
        float smax = 0.0f;
        uint32_t wmin = 0xFFFFFFFFu;
        const int q0 = tid, q1 = tid + NTG, q2 = tid + 2 * NTG, q3 = tid + 3 * NTG;
        uint32_t a0 = a_for(q0, k0), a1 = a_for(q1, k0), a2 = a_for(q2, k0), a3 = a_for(q3, k0);
        put(0, q0, fetch(q0, a0));
        put(0, q1, fetch(q1, a1));
        put(0, q2, fetch(q2, a2));
        put(0, q3, fetch(q3, a3));
        {
            const int wn = min(k0 + W, k1);                 // op(A) of the second window
            a0 = a_for(q0, wn), a1 = a_for(q1, wn), a2 = a_for(q2, wn), a3 = a_for(q3, wn);
        }
        __syncthreads();
        int buf = 0;
        for (int w0 = k0; w0 < k1; w0 += W) {
            const int w1 = min(w0 + W, k1);
            const bool more = w1 < k1;
            // the next window's rows, requested now and stored after this
            // window's lookups; then op(A) of the window after it
            const u32x4 s0 = fetch(q0, a0), s1 = fetch(q1, a1), s2 = fetch(q2, a2), s3 = fetch(q3, a3);
            {
                const int wn = min(w1 + W, k1);
                a0 = a_for(q0, wn), a1 = a_for(q1, wn), a2 = a_for(q2, wn), a3 = a_for(q3, wn);
            }
            const uint16_t* wrows = reinterpret_cast<const uint16_t*>(rows + ((size_t)buf << (rlog + 5)));
            for (int kg = w0; kg < w1; kg += G1) {
                uint32_t bw[G1][kGemvColsPerLane], xa[G1][1];
                ops.load(kg, bw, xa);
                __builtin_amdgcn_sched_barrier(0);         // keep the group's loads issued together
                const int cnt = min(G1, w1 - kg);
#pragma unroll
                for (int g = 0; g < G1; ++g) {
                    if (g >= cnt) break;
                    uint32_t ix[kGemvColsPerLane];
                    float sb[kGemvColsPerLane];
#pragma unroll
                    for (int c = 0; c < kGemvColsPerLane; ++c) gemv_fast_b(cast(bw[g][c]), sh, M, smax, wmin, ix[c], sb[c]);
                    const uint16_t* row = wrows + ((kg - w0 + g) << M);     // the index's staged row
                    uint32_t e[kGemvColsPerLane];
#pragma unroll
                    for (int c = 0; c < kGemvColsPerLane; ++c) e[c] = row[ix[c]];
                    const uint32_t seA = cast(xa[g][0]) & 0xFF800000u;
#pragma unroll
                    for (int c = 0; c < kGemvColsPerLane; ++c) gemv_fast_fma<FMT>(acc[0][c], e[c], sb[c], seA, p.elo);
                }
            }
            if (more) {
                put(buf ^ 1, q0, s0);
                put(buf ^ 1, q1, s1);
                put(buf ^ 1, q2, s2);
                put(buf ^ 1, q3, s3);
            }
            __syncthreads();
            buf ^= 1;
        }
        checked = __any(!(smax < hi_s) || wmin < lo_w);
        if (checked) {
#pragma unroll
            for (int c = 0; c < kGemvColsPerLane; ++c) acc[0][c] = 0.0f;
        }
    }
    if (checked) gemv_item<1, false, NTG, FMT, false>(p, p.lut, A, B, j0, k0, k1, acc, true);
}

__global__ __launch_bounds__(kGemv1Threads) void gemv1_kernel(GemvParams p)
{
    constexpr int NTG = kGemv1Threads;
    __shared__ __align__(16) unsigned char rows[2 * kGemv1Window * 512];
    constexpr int COLS = NTG * kGemvColsPerLane;
    const int nblk = (p.n + COLS - 1) / COLS;
    const int items = nblk * p.splits * p.batch;
    for (int item = gemv_first_item(); item < items; item += gridDim.x) {
        const int blk = item % nblk;
        const int rest = item / nblk;
        const int split = rest % p.splits;
        const int b = rest / p.splits;
        const gfloat_cptr A = (gfloat_cptr)(p.A_ptrs ? p.A_ptrs[b] : p.A + b * p.A_batch);
        const gfloat_cptr B = (gfloat_cptr)(p.B_ptrs ? p.B_ptrs[b] : p.B + b * p.B_batch);
        const int j0 = blk * COLS + threadIdx.x;
        const int k0 = split * p.chunk, k1 = min(p.k, k0 + p.chunk);
        float acc[kGemvMaxRows][kGemvColsPerLane];
        if (p.elo != 1 || p.ehi != 254) gemv1_item<true>(p, rows, A, B, j0, k0, k1, acc);
        else gemv1_item<false>(p, rows, A, B, j0, k0, k1, acc);
        gemv_store<NTG>(p, b, split, 0, 1, j0, acc);
    }
}

// ------------------------------------------------------------------ reduce / fill

// C = sum of the split partials in ascending split order, from +0. When the
// partials of one batch entry hold a multiple of 4 values, each thread sums 4
// consecutive outputs with 16-byte loads; the loads of 8 splits are issued
// ahead of their (ordered) adds.
// The bodies below take the workgroup's index and the number of workgroups
// of their own part of the grid (a reduction launch may hold several).
__device__ __forceinline__ void reduce_body(const ReduceParams& p, uint32_t blk, uint32_t nblk)
{
    const int64_t mn = (int64_t)p.m * p.n;
    const bool quad = (mn & 3) == 0;
    const int64_t units = quad ? mn / 4 : mn;
    const int64_t total = units * p.batch;
    for (int64_t g = blk * 256LL + threadIdx.x; g < total; g += (int64_t)nblk * 256) {
        const int64_t b = g / units, u = g - b * units;
        float* out = p.out_ptrs ? p.out_ptrs[b] : p.out + b * p.out_batch;
        if (quad) {
            const int64_t r = u * 4;
            const v4f* src = reinterpret_cast<const v4f*>(p.ws + b * p.splits * mn + r);
            const int64_t step = mn / 4;
            v4f s = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
            for (int sp = 0; sp < p.splits; ++sp) s += src[sp * step];
            int64_t i = r / p.n, j = r - i * p.n;
#pragma unroll
            for (int t = 0; t < 4; ++t) {
                out[i * p.ldc + j] = s[t];
                if (++j == p.n) {
                    j = 0;
                    ++i;
                }
            }
        } else {
            const float* src = p.ws + b * p.splits * mn + u;
            float s = 0.0f;
#pragma unroll 8
            for (int sp = 0; sp < p.splits; ++sp) s += src[sp * mn];
            const int64_t i = u / p.n, j = u - i * p.n;
            out[i * p.ldc + j] = s;
        }
    }
}

__global__ __launch_bounds__(256) void reduce_kernel(ReduceParams p) { reduce_body(p, blockIdx.x, gridDim.x); }

// Few outputs with many chunk partials each (the row-vector kernel's
// splits): 16 lanes (one DPP row) per 4 consecutive outputs. Lane l of a row
// requests partials l, l + 16, ... of its 4 outputs together; the row then
// adds them in ascending split order from +0, taking each partial from its
// lane with a row broadcast, so every lane of the row holds the same sums.
// Slots past the last split hold +0, which leaves such a sum unchanged (a sum
// started from +0 is never -0).
constexpr int kReduceRowLoads = 8;           // partials per lane per round (128 splits)

template <int T>
__device__ __forceinline__ float row_bcast(float v)
{
    // row_newbcast:T, lane T of each row of 16 to the whole row
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x150 + T, 0xF, 0xF, false));
}

template <int... T>
__device__ __forceinline__ void row_chain(v4f& s, const v4f& v, std::integer_sequence<int, T...>)
{
    ((s[0] += row_bcast<T>(v[0]), s[1] += row_bcast<T>(v[1]), s[2] += row_bcast<T>(v[2]),
      s[3] += row_bcast<T>(v[3])),
     ...);
}

__device__ __forceinline__ void reduce_rows_body(const ReduceParams& p, uint32_t blk)
{
    const int64_t mn = (int64_t)p.m * p.n;       // a multiple of 4
    const int64_t units = mn / 4;
    const int64_t unit = ((int64_t)blk * 256 + threadIdx.x) >> 4;
    if (unit >= units * p.batch) return;          // the 16 lanes of a row leave together
    const int l = threadIdx.x & 15;
    const int64_t b = unit / units, u = unit - b * units;
    const v4f* src = reinterpret_cast<const v4f*>(p.ws + b * p.splits * mn) + u;
    const int64_t step = mn / 4;
    v4f s = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int i0 = 0; i0 < p.splits; i0 += 16 * kReduceRowLoads) {
        v4f v[kReduceRowLoads];
#pragma unroll
        for (int j = 0; j < kReduceRowLoads; ++j) {
            const int sp = i0 + j * 16 + l;
            v[j] = sp < p.splits ? src[(int64_t)sp * step] : v4f{0.0f, 0.0f, 0.0f, 0.0f};
        }
#pragma unroll
        for (int j = 0; j < kReduceRowLoads; ++j) {
            if (i0 + j * 16 >= p.splits) break;
            row_chain(s, v[j], std::make_integer_sequence<int, 16>{});
        }
    }
    if (l < 4) {
        float* out = p.out_ptrs ? p.out_ptrs[b] : p.out + b * p.out_batch;
        const int64_t r = u * 4 + l;
        const int64_t i = r / p.n, j = r - i * p.n;
        out[i * p.ldc + j] = l == 0 ? s[0] : l == 1 ? s[1] : l == 2 ? s[2] : s[3];
    }
}

__global__ __launch_bounds__(256) void reduce_rows_kernel(ReduceParams p) { reduce_rows_body(p, blockIdx.x); }

// The split tiles' outputs: C = sum of their chunk partials in ascending
// split order, from +0. Thread unit = 4 consecutive columns of one tile row
// (16-byte loads when the rows are 4-float aligned and the 4 are inside).
__device__ __forceinline__ void reduce_tiles_body(const ReduceTilesParams& p, uint32_t blk, uint32_t nblk)
{
    const int quads = p.TN / 4;
    const int64_t per_tile = (int64_t)p.TM * quads;
    const int64_t total = per_tile * p.n_tiles;
    const int tiles = p.tiles_m * p.tiles_n;
    const int64_t mn = (int64_t)p.m * p.n;
    for (int64_t g = blk * 256LL + threadIdx.x; g < total; g += (int64_t)nblk * 256) {
        const int tt = (int)(g / per_tile);
        const int q = (int)(g - (int64_t)tt * per_tile);
        const int tl = p.first_tile + tt;
        const int b = tl / tiles;
        int tm, tn;
        tile_coords(tl - b * tiles, p.tiles_m, p.tiles_n, tm, tn);
        const int i = tm * p.TM + q / quads;
        const int j = tn * p.TN + (q % quads) * 4;
        if (i >= p.m || j >= p.n) continue;
        const float* src = p.ws + (int64_t)b * p.splits * mn + (int64_t)i * p.n + j;
        float* out = (p.out_ptrs ? p.out_ptrs[b] : p.out + b * p.out_batch) + (int64_t)i * p.ldc + j;
        if ((p.n & 3) == 0) {                      // j + 3 < n as well
            v4f sum = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
            for (int sp = 0; sp < p.splits; ++sp) sum += *reinterpret_cast<const v4f*>(src + sp * mn);
#pragma unroll
            for (int t = 0; t < 4; ++t) out[t] = sum[t];
        } else {
            const int nt = min(4, p.n - j);
            float sum[4] = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll 8
            for (int sp = 0; sp < p.splits; ++sp)
#pragma unroll
                for (int t = 0; t < 4; ++t)
                    if (t < nt) sum[t] += src[sp * mn + t];
#pragma unroll
            for (int t = 0; t < 4; ++t)
                if (t < nt) out[t] = sum[t];
        }
    }
}

__global__ __launch_bounds__(256) void reduce_tiles_kernel(ReduceTilesParams p)
{
    reduce_tiles_body(p, blockIdx.x, gridDim.x);
}

// The reductions of up to kMaxGroup calls in one launch (a grouped call's
// members): job j takes workgroups [first[j], first[j + 1]).
struct ReduceGroup {
    int count;
    uint32_t first[kMaxGroup + 1];
    ReduceJob job[kMaxGroup];
};

__global__ __launch_bounds__(256) void reduce_group_kernel(ReduceGroup g)
{
    int j = 0;
    while (j + 1 < g.count && blockIdx.x >= g.first[j + 1]) ++j;
    const ReduceJob& jb = g.job[j];
    const uint32_t blk = blockIdx.x - g.first[j], nblk = g.first[j + 1] - g.first[j];
    if (jb.variant == RV_ROWS) reduce_rows_body(jb.r, blk);
    else if (jb.variant == RV_TILES) reduce_tiles_body(jb.t, blk, nblk);
    else reduce_body(jb.r, blk, nblk);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(float* C, float* const* Cp, int m, int n, int ldc, int batch,
                                                        int64_t strideC)
{
    const int64_t mn = (int64_t)m * n, total = mn * batch;
    for (int64_t g = blockIdx.x * 256LL + threadIdx.x; g < total; g += (int64_t)gridDim.x * 256) {
        const int64_t b = g / mn, r = g - b * mn, i = r / n, j = r - i * n;
        float* out = Cp ? Cp[b] : C + b * strideC;
        out[i * ldc + j] = 0.0f;
    }
}

// ------------------------------------------------------------------ launchers

static int grid_for(int64_t work, int per_block, int cap)
{
    int64_t g = (work + per_block - 1) / per_block;
    if (g < 1) g = 1;
    if (g > cap) g = cap;
    return (int)g;
}

hipError_t launch_init_stats(int* stats, int blocks, hipStream_t s)
{
    hipLaunchKernelGGL(init_stats_kernel, dim3(blocks), dim3(256), 0, s, stats);
    return hipGetLastError();
}

hipError_t launch_assign(const AssignParams& p, hipStream_t s)
{
    const int64_t groups = (int64_t)p.batch * p.G1 * p.G2 * p.G3;
    if (groups <= 0) return hipSuccess;
    hipLaunchKernelGGL(assign_kernel, dim3(grid_for(groups, kAssignThreads, 65536)), dim3(kAssignThreads), 0, s, p);
    return hipGetLastError();
}

// The decode of one operand: its layout's variant and grid (the per-element
// divisors filled in).
static DecodeJob plan_decode(const DecodeParams& p0)
{
    constexpr int kRowsWgElems = 1024;   // elements per workgroup of a row copy (whole rows)
    DecodeJob jb;
    jb.rb = 0;
    DecodeParams& p = jb.p;
    p = p0;
    auto fd = [](int v) { return make_fastdiv((uint32_t)(v > 0 ? v : 1)); };
    p.fd_Mp = fd(p.Mp); p.fd_Np = fd(p.Np); p.fd_Cp = fd(p.Cp); p.fd_Kp = fd(p.Kp); p.fd_S = fd(p.S);
    p.fd_Wp = fd(p.Wp); p.fd_Cb = fd(p.Cb); p.fd_Kb = fd(p.Kb); p.fd_Hp = fd(p.Hp); p.fd_C = fd(p.C);
    if (p.rowlen <= 0) {                           // unpadded: one row of `count` Words
        p.rowlen = (int)p.count;
        p.ldw = (int)p.count;
    }
    p.fd_rowlen = fd(p.rowlen);
    auto grid = [&](int variant, uint32_t x, uint32_t y, uint32_t z) {
        jb.variant = variant;
        jb.gx = x;
        jb.gy = y;
        jb.gz = z;
        return jb;
    };
    const bool img = p.layout == L_IMG_FWD || p.layout == L_IMG_DGRAD || p.layout == L_IMG_WGRAD;
    if (img) {
        p.row_floats = p.layout == L_IMG_DGRAD ? p.Q * p.K : p.W * p.C;
        p.rows = p.N * p.Hp;
        if (p.row_floats <= IMG_ROW_FLOATS_MAX && p.batch == 1) {
            int extra = 0;
            if (p.layout == L_IMG_WGRAD) {
                const int64_t tail = p.count - (int64_t)p.rows * p.C * p.Wp;
                extra = (int)((tail + 256 * 16 - 1) / (256 * 16));
            }
            return grid(DV_IMG, (uint32_t)(p.rows + extra), 1, 1);
        }
    }
    const bool rows = (p.layout == L_DENSE_UNIFORM && !p.trans) || p.layout == L_DY_WGRAD;
    if (rows && p.batch <= 65535) {
        if (p.layout == L_DY_WGRAD) { p.k = p.N * p.P * p.Q; p.n = p.K; p.ld = p.K; }
        const int rows_out = p.KB * 4;
        // a power of two up to 64 rows, so that a workgroup's rows lie in one
        // k-segment (64 reduction indices) whatever the row length
        jb.rb = 1;
        while (jb.rb < 64 && 2 * jb.rb * std::max(p.Np, 1) <= kRowsWgElems) jb.rb *= 2;
        return grid(DV_ROWS, (uint32_t)((rows_out + jb.rb - 1) / jb.rb), 1, (uint32_t)p.batch);
    }
    const bool tile = (p.layout == L_DENSE_LANE && !p.trans) || (p.layout == L_DENSE_UNIFORM && p.trans);
    const int64_t outer = p.layout == L_DENSE_LANE ? p.Mp : p.Np;
    if (tile && p.batch <= 65535 && outer % 16 == 0 && outer * p.KB * 4 * p.batch <= kDirectElems)
        return grid(DV_DIRECT, (uint32_t)((outer * p.KB + 255) / 256), (uint32_t)p.batch, 1);
    if (tile && p.batch <= 65535) {
        const int outer = p.layout == L_DENSE_LANE ? p.Mp : p.Np;
        const int kext = p.KB * 4;
        const int gy = (kext + 63) / 64;
        if (gy <= 65535) return grid(DV_TILE, (uint32_t)((outer + 63) / 64), (uint32_t)gy, (uint32_t)p.batch);
    }
    return grid(DV_GENERIC, (uint32_t)grid_for(p.count, 256, 8192), (uint32_t)p.batch, 1);
}

hipError_t launch_decode_group(const DecodeParams* const* jobs, int count, hipStream_t s)
{
    if (count < 1 || count > 2 * kMaxGroup) return hipErrorInvalidValue;
    DecodeGroup g{};
    uint64_t blocks = 0;
    size_t bytes = 0;
    int n = 0;
    for (int i = 0; i < count; ++i) {
        const DecodeJob jb = plan_decode(*jobs[i]);
        const uint64_t nb = (uint64_t)jb.gx * jb.gy * jb.gz;
        if (nb == 0) continue;
        g.job[n] = jb;
        g.first[n] = (uint32_t)blocks;
        blocks += nb;
        if (jb.variant == DV_IMG) bytes = std::max(bytes, (size_t)jb.p.row_floats * sizeof(float));
        if (jb.variant == DV_TILE) bytes = std::max(bytes, (size_t)kTileLdsBytes);
        ++n;
        if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
    }
    if (n == 0) return hipSuccess;
    g.count = n;
    g.first[n] = (uint32_t)blocks;
    hipLaunchKernelGGL(decode_group_kernel, dim3((uint32_t)blocks), dim3(256), bytes, s, g);
    return hipGetLastError();
}

bool decode_covers_segments(const DecodeParams& p)
{
    const DecodeJob jb = plan_decode(p);
    if (jb.variant == DV_TILE) return true;              // 64 indices of k per workgroup, from a multiple of 64
    if (jb.variant == DV_DIRECT) return true;            // a workgroup's threads lie in one k-segment
    if (jb.variant == DV_ROWS) return p.layout == L_DENSE_UNIFORM && jb.rb > 0 && 64 % jb.rb == 0;
    return false;
}

hipError_t launch_decode_pair(const DecodeParams& a, const DecodeParams& b, hipStream_t s)
{
    const DecodeParams* jobs[2] = {&a, &b};
    return launch_decode_group(jobs, 2, s);
}

// The GEMM kernel variant of (lds_class, gather, shape): lds_class 0 = table
// of M <= 7 in LDS, 1 = M == 8 in LDS, 2 = native multiplier (no table),
// 3 = table of M = 9..11 in global memory; shape indexes kShapes.
template <int S>
static const void* main_variant_shape(int lds_class, int gather)
{
    constexpr int NW = kShapes[S].waves, R = kShapes[S].rows_per_lane;
    switch (lds_class) {
    case 0:
        return gather ? (const void*)main_kernel<LDS_SMALL, true, false, NW, R, false, false>
                      : (const void*)main_kernel<LDS_SMALL, false, false, NW, R, false, false>;
    case 1:
        return gather ? (const void*)main_kernel<LDS_LARGE, true, false, NW, R, false, false>
                      : (const void*)main_kernel<LDS_LARGE, false, false, NW, R, false, false>;
    case 2:
        return gather ? (const void*)main_kernel<NATIVE_LDS, true, true, NW, R, false, false>
                      : (const void*)main_kernel<NATIVE_LDS, false, true, NW, R, false, false>;
    default:
        return gather ? (const void*)main_kernel<NATIVE_LDS, true, false, NW, R, true, false>
                      : (const void*)main_kernel<NATIVE_LDS, false, false, NW, R, true, false>;
    }
}

// Dense calls (operands in vector mode) only: the variants of shape S.
template <int S, bool GROUP>
static const void* main_variant_dense(int lds_class)
{
    constexpr int NW = kShapes[S].waves, R = kShapes[S].rows_per_lane;
    switch (lds_class) {
    case 0: return (const void*)main_kernel<LDS_SMALL, false, false, NW, R, false, GROUP>;
    case 1: return (const void*)main_kernel<LDS_LARGE, false, false, NW, R, false, GROUP>;
    case 2: return (const void*)main_kernel<NATIVE_LDS, false, true, NW, R, false, GROUP>;
    default: return (const void*)main_kernel<NATIVE_LDS, false, false, NW, R, true, GROUP>;
    }
}

// (shape 2 is never planned for a gather-mode call)
static const void* main_variant(int lds_class, int gather, int shape)
{
    if (shape == 2) return gather ? nullptr : main_variant_dense<2, false>(lds_class);
    return shape == 0 ? main_variant_shape<0>(lds_class, gather) : main_variant_shape<1>(lds_class, gather);
}

// Grouped launches: operands in vector mode (dense GEMMs), shape 0 or 2, one
// shape per launch.
bool main_group_supported(int gather, int shape) { return gather == 0 && (shape == 0 || shape == 2); }

static const void* main_group_variant(int lds_class, int shape)
{
    return shape == 2 ? main_variant_dense<2, true>(lds_class) : main_variant_dense<0, true>(lds_class);
}

hipError_t launch_main(const MainParams& p, int lds_class, int gather, int shape, int grid, hipStream_t s)
{
    if (shape < 0 || shape >= kNumShapes || main_variant(lds_class, gather, shape) == nullptr) return hipErrorInvalidValue;
    MainParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(main_variant(lds_class, gather, shape), dim3(grid), dim3(kShapes[shape].waves * 64), args,
                           0, s);
}

hipError_t launch_main_group(const MainParams* const* ps, int count, int lds_class, int gather, int shape, int grid,
                             hipStream_t s)
{
    if (count < 1 || count > kMaxGroup) return hipErrorInvalidValue;
    if (count == 1) return launch_main(*ps[0], lds_class, gather, shape, grid, s);
    if (!main_group_supported(gather, shape)) return hipErrorInvalidValue;
    MainGroup arg{};
    int64_t total = 0;
    for (int g = 0; g < count; ++g) {
        arg.p[g] = *ps[g];
        arg.first[g] = (int)total;
        total += ps[g]->items;
    }
    if (total > INT32_MAX) return hipErrorInvalidValue;
    arg.count = count;
    arg.first[count] = (int)total;
    void* args[] = {&arg};
    return hipLaunchKernel(main_group_variant(lds_class, shape), dim3(grid), dim3(kShapes[shape].waves * 64), args, 0,
                           s);
}

int main_group_blocks_per_cu(int lds_class, int shape)
{
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, main_group_variant(lds_class, shape),
                                                                      kShapes[shape].waves * 64, 0);
    if (e != hipSuccess || n < 1) n = 1;
    return n;
}

int main_blocks_per_cu(int lds_class, int gather, int shape)
{
    int n = 0;
    const hipError_t e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, main_variant(lds_class, gather, shape),
                                                                      kShapes[shape].waves * 64, 0);
    if (e != hipSuccess || n < 1) n = 1;
    return n;
}

// Row-vector kernel variants: 0 = table of M <= 7 in LDS, 1 = M == 8 in LDS,
// 2 = table in global memory, 3 = native multiplier.
static const void* gemv_variant(int v)
{
    switch (v) {
    case 0: return (const void*)gemv_kernel<false, (1 << 7) * ((1 << 7) + 8) * 2, kGemvLdsThreads>;
    case 1: return (const void*)gemv_kernel<false, (1 << 8) * ((1 << 8) + 8) * 2, kGemvLdsThreads>;
    case 2: return (const void*)gemv_kernel<false, 0, kGemvThreads>;
    case 3: return (const void*)gemv_kernel<true, 0, kGemvThreads>;
    default: return (const void*)gemv1_kernel;
    }
}

int gemv_threads(int variant) { return variant <= 1 ? kGemvLdsThreads : variant == 4 ? kGemv1Threads : kGemvThreads; }

int gemv_blocks_per_cu(int variant)
{
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, gemv_variant(variant), gemv_threads(variant), 0) != hipSuccess ||
        n < 1)
        n = 1;
    return n;
}

hipError_t launch_gemv(const GemvParams& p, int variant, int grid, hipStream_t s)
{
    GemvParams arg = p;
    void* args[] = {&arg};
    return hipLaunchKernel(gemv_variant(variant), dim3(grid), dim3(gemv_threads(variant)), args, 0, s);
}

ReduceJob reduce_job(const ReduceParams& p)
{
    ReduceJob jb{};
    jb.r = p;
    const int64_t total = (int64_t)p.m * p.n * p.batch;
    // few outputs (fewer than 64 Ki threads' worth of 4) and many splits:
    // 16 lanes per 4 outputs; one workgroup of 256 lanes per 64 outputs
    if (reduce_by_rows(p.m, p.n, p.batch, p.splits)) {
        jb.variant = RV_ROWS;
        jb.blocks = (uint32_t)((total + 63) / 64);
    } else {
        jb.variant = RV_PLAIN;
        jb.blocks = (uint32_t)grid_for(total, 256, 16384);
    }
    return jb;
}

ReduceJob reduce_tiles_job(const ReduceTilesParams& p)
{
    ReduceJob jb{};
    jb.t = p;
    jb.variant = RV_TILES;
    jb.blocks = (uint32_t)grid_for((int64_t)p.TM * (p.TN / 4) * p.n_tiles, 256, 16384);
    return jb;
}

hipError_t launch_reduce(const ReduceParams& p, hipStream_t s)
{
    const ReduceJob jb = reduce_job(p);
    if (jb.variant == RV_ROWS) hipLaunchKernelGGL(reduce_rows_kernel, dim3(jb.blocks), dim3(256), 0, s, p);
    else hipLaunchKernelGGL(reduce_kernel, dim3(jb.blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_reduce_tiles(const ReduceTilesParams& p, hipStream_t s)
{
    hipLaunchKernelGGL(reduce_tiles_kernel, dim3(reduce_tiles_job(p).blocks), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_reduce_group(const ReduceJob* jobs, int count, hipStream_t s)
{
    if (count < 1 || count > kMaxGroup) return hipErrorInvalidValue;
    ReduceGroup g{};
    uint64_t blocks = 0;
    int n = 0;
    for (int i = 0; i < count; ++i) {
        if (jobs[i].blocks == 0) continue;
        g.job[n] = jobs[i];
        g.first[n] = (uint32_t)blocks;
        blocks += jobs[i].blocks;
        if (blocks > 0x7FFFFFFFull) return hipErrorInvalidValue;
        ++n;
    }
    if (n == 0) return hipSuccess;
    g.count = n;
    g.first[n] = (uint32_t)blocks;
    hipLaunchKernelGGL(reduce_group_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, g);
    return hipGetLastError();
}

hipError_t launch_fill_zero(float* C, float* const* Cp, int m, int n, int ldc, int batch, int64_t strideC,
                            hipStream_t s)
{
    const int64_t total = (int64_t)m * n * batch;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(total, 256, 16384)), dim3(256), 0, s,
                       C, Cp, m, n, ldc, batch, strideC);
    return hipGetLastError();
}

}  // namespace amx
