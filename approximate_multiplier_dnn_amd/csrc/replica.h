// replica.h -- the second copies that spread the M = 8 table lookups of a
// half-wave over the LDS banks, and the per-group choice of copy made by the
// decode pass.
//
// The LDS serves a wave64 read as two half-waves of 32 lanes; in each, the
// 32 four-byte banks deliver one dword per clock, so a half-wave costs as
// many clocks as the largest number of DISTINCT dwords any one bank is asked
// for (lanes reading the same dword share it). In a GEMM lookup every lane
// reads the same table column (the uniform operand's) at its own row (the
// lane operand's mantissa index). An M = 8 column of 16-bit entries is 128
// dwords, four per bank, so random rows leave some bank with about 2.8
// distinct dwords on average.
//
// Each 640-byte M = 8 column therefore holds, after its 128 dwords (dword d
// = entries 2d, 2d+1) and the pad dword (position 128: the two zero entries
// read by zero, Inf and NaN operands), a second copy of dwords d < 31 at
// position 129 + (d + 15) mod 31 (the 160 KB of LDS has room for no more).
// Copy 1 of dword d then lies in bank d + 16 for d < 16 and in bank d - 15
// for 16 <= d < 31, so the choice between the two copies of the dwords d < 31
// links the banks in one path
//     0 - 16 - 1 - 17 - 2 - ... - 14 - 30 - 15 - 31
// whose k-th link (k = 0..30) is dword d_k = k / 2 (k even) or 16 + k / 2
// (k odd): copy 0 of d_k lies in the link's left bank, copy 1 in its right.
//
// For each group of 32 lane operands that one half-wave reads together, the
// decode pass picks the copies that make the largest bank load smallest.
// Dwords >= 31 and the pad have one place; on a path, the smallest feasible
// load T is found by one left-to-right scan per T: a link is given to its
// left bank while that bank is below T, else to its right bank (a bank can
// only take its own two links, so taking the left one whenever possible is
// never worse). Any copy holds the same entry, so the choice changes only
// the speed, never a result.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace amx {

constexpr int kRep8Slots = 31;           // dwords with a second copy
constexpr int kRep8PadPos = 128;         // dword position of the pad
constexpr int kRep8ColBytes = 640;       // 128 + 1 + 31 dwords

// Dword position (within its column) of copy c of dword d (c = 1 only for d < 31).
__host__ __device__ inline int rep8_pos(int d, int c)
{
    return c ? 129 + (d + 15) % kRep8Slots : d;
}

// Byte offset, inside a column, of entry ia (0..255) read from copy c.
__host__ __device__ inline uint32_t rep8_offset(uint32_t ia, int c)
{
    return 4u * (uint32_t)rep8_pos((int)(ia >> 1), c) + 2u * (ia & 1u);
}

// Chooses the copies for one group. p0..p3: the dwords read (bit d & 31 of
// p[d >> 5]); pad: whether the pad is read. Returns the largest bank load and
// sets bit d of *second for each dword d < 31 to be read from copy 1.
__host__ __device__ inline int rep8_solve(uint32_t p0, uint32_t p1, uint32_t p2, uint32_t p3, bool pad,
                                          uint32_t* second)
{
    // dwords with one place, counted per bank in three bit planes (<= 5 each)
    const uint32_t fixed[5] = {p0 & 0x80000000u, p1, p2, p3, pad ? 1u : 0u};
    uint32_t c0 = 0, c1 = 0, c2 = 0;
    for (int i = 0; i < 5; ++i) {
        const uint32_t x = fixed[i], t0 = c0 & x;
        c0 ^= x;
        const uint32_t t1 = c1 & t0;
        c1 ^= t0;
        c2 |= t1;
    }
    const uint32_t links = p0 & 0x7FFFFFFFu;
    int T = c2 ? 4 : (c1 & c0) ? 3 : c1 ? 2 : 1;      // a lower bound: the fixed load
    for (;; ++T) {
        int carry = 0;
        bool ok = true;
        uint32_t push = 0;
        for (int k = 0; k < 32; ++k) {
            const int b = (k & 1) ? (k >> 1) + 16 : (k >> 1);       // k-th bank of the path
            const int load = (int)((c0 >> b) & 1u) + 2 * (int)((c1 >> b) & 1u) + 4 * (int)((c2 >> b) & 1u) + carry;
            if (load > T) {
                ok = false;
                break;
            }
            carry = 0;
            if (k < 31 && ((links >> b) & 1u)) {                     // link k is dword b (= d_k)
                if (load + 1 > T) {
                    carry = 1;
                    push |= 1u << b;
                }
            }
        }
        if (ok) {
            *second = push;
            return T;
        }
    }
}

// Rewrites the table offsets of one group of `count` (<= 32) lane-operand
// offsets `w` (2 * mantissa index in copy 0, or pad_w for an operand that
// reads the zero pad entry) with offsets into the chosen copies. Returns the
// largest bank load of the group. (The lane loops run to 32 so that w can
// live in registers once they are unrolled.)
__host__ __device__ inline int rep8_assign_group(uint32_t (&w)[32], int count, uint32_t pad_w)
{
    uint32_t p0 = 0, p1 = 0, p2 = 0, p3 = 0;
    bool pad = false;
#pragma unroll
    for (int l = 0; l < 32; ++l) {
        if (l >= count) continue;
        if (w[l] == pad_w) {
            pad = true;
            continue;
        }
        const uint32_t d = w[l] >> 2, bit = 1u << (d & 31u);
        const uint32_t q = d >> 5;
        p0 |= q == 0u ? bit : 0u;
        p1 |= q == 1u ? bit : 0u;
        p2 |= q == 2u ? bit : 0u;
        p3 |= q == 3u ? bit : 0u;
    }
    uint32_t second = 0;
    const int top = rep8_solve(p0, p1, p2, p3, pad, &second);
#pragma unroll
    for (int l = 0; l < 32; ++l) {
        if (l >= count || w[l] == pad_w) continue;
        const uint32_t d = w[l] >> 2;
        if (d < (uint32_t)kRep8Slots && ((second >> d) & 1u)) w[l] = rep8_offset(w[l] >> 1, 1);
    }
    return top;
}

}  // namespace amx
