/*
 * approx_mul.h -- C ABI of the LUT-based approximate FP32 multiplication
 * library for AMD Instinct MI355X (gfx950).
 *
 * Every product inside the GEMM and Conv2D passes below is the AMSim
 * approximate product of "ApproxTrain: Fast Simulation of Approximate
 * Multipliers for DNN Training and Inference" (arXiv 2209.04161), Section V,
 * Algorithm 2: sign = XOR of the signs; biased exponent = EA + EB - 127 plus
 * the carry read from the table; mantissa = the 15-bit mantissa read from the
 * table at index (top M fraction bits of the first operand << M) | (top M
 * fraction bits of the second operand). The resulting exponent decides the
 * special cases: e <= 0 gives a signed zero, e >= 255 a signed infinity.
 * Subnormal inputs count as zero; NaN inputs give NaN; infinity times zero
 * gives NaN; infinity times a non-zero gives a signed infinity.
 *
 * Products are accumulated in FP32 (round to nearest even), starting from
 * +0.0, in ascending order of the reduction sequence. When an output's
 * reduction is split, the sequence is cut into chunks of L consecutive
 * positions; each chunk is summed from +0.0 in ascending order and the chunk
 * sums are added from +0.0 in ascending chunk order. L depends only on the
 * call's shapes and the loaded table's width (approx_gemm_chunks and
 * approx_conv2d_chunks report it per output), so results are bitwise
 * reproducible for the same inputs. The sequences: GEMM, the index p of
 * op(A)(i,p) op(B)(p,j); Conv2D, see approx_conv2d_chunks. With the native
 * multiplier every step is a fused multiply-add (one rounding).
 *
 * Conventions shared by all calls:
 *  - Tensors are FP32, row-major (C order), in device memory owned by the
 *    caller. The library never frees or keeps them. Outputs are overwritten
 *    (there is no alpha / beta) and must not alias an input.
 *  - `stream` is a hipStream_t passed as void*; NULL means the null stream.
 *    The current HIP device is used. Compute calls are asynchronous: they
 *    return once the work is queued, and faults surface at the caller's next
 *    synchronisation with the stream.
 *  - The library keeps, per device, the loaded table and a scratch arena per
 *    stream (decoded operands, split-reduction partials). Calls queued on one
 *    stream reuse that stream's arena in order; calls on different streams
 *    use different arenas. An arena only grows, at least doubling; a
 *    superseded arena, like a superseded table, stays allocated until
 *    approx_release(), which frees them all.
 *  - Once a stream's arena is large enough (after a call of the same or
 *    larger sizes on that stream), a compute call queues kernel launches
 *    only: no allocation, copy, memset or synchronisation. Such calls can be
 *    captured into a HIP graph on that stream and replayed there; the graph
 *    stays valid when later calls grow the arena or load another table (it
 *    keeps using the memory it captured, including the table loaded at
 *    capture time), until approx_release().
 *  - Return value: APPROX_OK (0) or a negative status. Argument checks run
 *    before any work is queued; on an error nothing is written.
 */
#ifndef APPROX_MUL_H
#define APPROX_MUL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define APPROX_OK 0
#define APPROX_EINVAL (-1)       /* bad size, leading dimension, flag or NULL pointer */
#define APPROX_ENOLUT (-2)       /* no table loaded (and no native multiplier selected) on the current device */
#define APPROX_EUNSUPPORTED (-3) /* M outside the supported range, or a table the generator cannot express */
#define APPROX_EHIP (-4)         /* a HIP runtime call failed (allocation, copy, launch) */
#define APPROX_ESCRATCH (-5)     /* the call needs more scratch than approx_gemm_noalloc's fixed maximum */

#define APPROX_MAX_GROUP 4       /* GEMMs per approx_gemm_grouped call */

/* Built-in C models of multipliers for approx_lut_build. */
#define APPROX_MODEL_EXACT 0    /* the exact product of the M-bit mantissas */
#define APPROX_MODEL_MITCHELL 1 /* Mitchell's logarithmic multiplier: 1+x+y, or 2(x+y) when x+y >= 1 */

/*
 * Table generation, ApproxTrain Section V-A, Algorithm 1 (host only; makes no
 * HIP call and needs no GPU).
 *
 * Writes 4^M uint16 entries to lut_out (caller-owned host memory): entry
 * (ia << M) | ib is the product of the operands 1.ia and 1.ib (M fraction
 * bits each, sign + and exponent 2^0) under the chosen model, as
 * bit 15 = carry (the product's exponent exceeds the un-normalised exponent
 * by one) and bits 14..0 = the top 15 bits of the product's fraction.
 * `perturb` is NULL or 4^M int8 values added to each entry's 15-bit mantissa
 * field, saturating at 0 and 0x7FFF, carry unchanged (a synthetic model).
 * Errors: APPROX_EINVAL (NULL lut_out, unknown model),
 * APPROX_EUNSUPPORTED (M outside [1, 11]).
 */
int approx_lut_build(int model, int M, const int8_t *perturb, uint16_t *lut_out);

/*
 * The same generation for a caller-supplied C model `mul(a, b)` of the
 * multiplier (ApproxTrain Fig. 7: the user's functional model). mul is
 * called once per mantissa pair with two normal floats in [1, 2). Its
 * product must lie in [1, 4) (carry 0 or 1); otherwise
 * APPROX_EUNSUPPORTED is returned and lut_out is left partly written.
 */
int approx_lut_build_from_model(int M, float (*mul)(float a, float b), uint16_t *lut_out);

/*
 * Load a table for use by the compute calls on the current device
 * (ApproxTrain Section VI: tables are loaded into the run-time library at run
 * time). `lut` is caller-owned host memory of 4^M entries in the format
 * above; it is copied during the call (the copy is complete when it
 * returns). Calls queued after it returns use the new table; work queued
 * before keeps the previous one, which stays allocated until
 * approx_release(). Not thread-safe against compute calls queued by other
 * threads at the same time. Tables of M <= 8 (at most 128 KB of entries) are
 * staged in each workgroup's LDS (at M = 8 with second copies of part of each
 * column, 160 KB, which spread a wave's lookups over the LDS banks); tables of
 * M = 9..11 (512 KB to 8 MB, the top of the range Section V names) are read
 * from global memory, where they stay resident in the L2 and last-level
 * caches, at a lower lookup rate.
 * Errors: APPROX_EINVAL (NULL lut), APPROX_EUNSUPPORTED (M outside
 * [1, 11]), APPROX_EHIP.
 */
int approx_lut_load(const uint16_t *lut, int M);

/*
 * Select the native multiplier on the current device instead of a table
 * (ApproxTrain Section V: the simulator can invoke the hardware's native
 * multiplication, the reference point of its approximate-versus-native
 * timing, Fig. 6). Every product of the compute calls that follow is then
 * the exact product of the two FP32 operands, folded into the FP32
 * accumulator by a fused multiply-add: one rounding per step, in the same
 * order as above. Subnormal operands and sums are kept (IEEE-754), an
 * overflow of the accumulator gives a signed infinity, and the sign of a
 * zero result is not specified (the hardware FMA may return +0 where a tiny
 * negative sum rounds to zero). approx_lut_load
 * selects a table again. A previously loaded table is kept until
 * approx_release(), as by approx_lut_load. Errors: APPROX_EHIP.
 */
int approx_native_load(void);

/* M of the table loaded on the current device, 0 when the native multiplier
 * is selected, or APPROX_ENOLUT. */
int approx_lut_bits(void);

/*
 * Exponent width E of the approximate multiplier's format (1, E, M) on the
 * current device (ApproxTrain Section V: the exponent may have 1 to 8 bits
 * given an exponent casting function). The format's exponent has bias
 * b = 2^(E-1) - 1 and normal values 2^(1-b) <= |x| < 2^(b+1), without
 * subnormals. Before each product both FP32 operands are cast to it: a
 * normal operand below that range becomes a signed zero, above it a signed
 * infinity (zero, Inf and NaN operands are kept; the mantissa is chopped to
 * M bits as always). The product's exponent, with the table's carry, is then
 * tested against the same range: below gives a signed zero, above a signed
 * infinity. Accumulation stays FP32. E = 8 (the default) is FP32's own range,
 * where the cast changes nothing; E = 1 leaves no normal value, so every
 * finite operand becomes zero or infinity. The setting persists across table
 * loads; the native multiplier ignores it. Takes effect for calls queued
 * after it returns. Errors: APPROX_EUNSUPPORTED (E outside [1, 8]),
 * APPROX_EHIP.
 */
int approx_exponent_bits_set(int E);

/* E of the current device's format (8 unless set). */
int approx_exponent_bits(void);

/*
 * C[i*ldc + j] = sum_p approx(op(A)(i,p), op(B)(p,j)),  0 <= i < m, 0 <= j < n,
 * op(A)(i,p) = transA ? A[p*lda + i] : A[i*lda + p],
 * op(B)(p,j) = transB ? B[j*ldb + p] : B[p*ldb + j].
 * The first table operand of each product is the element of op(A).
 * (The GEMM kernel of ApproxTrain Section VI-D, behind Dense and, through
 * IM2COL, Conv2D.) m = 0 or n = 0 does nothing; k = 0 writes zeros. Calls
 * with transB = 0 and m <= 32 (or m <= 64 when k * n >= 2^22 or
 * k * n <= 2^16), i.e. batch-1 and few-row inference, run a row-vector
 * kernel (the section's separate matrix-vector kernel) in blocks of 4 rows
 * of op(A): the same products and order, with the reduction split into
 * chunks as described above.
 * Errors: APPROX_EINVAL (negative sizes, NULL pointers with non-empty
 * operands, lda/ldb/ldc smaller than the stored row length, flags not 0/1),
 * APPROX_ENOLUT, APPROX_EHIP.
 */
int approx_gemm(int transA, int transB, int m, int n, int k,
                const float *A, int lda, const float *B, int ldb,
                float *C, int ldc, void *stream);

/*
 * Several independent GEMMs in one call: `count` (1 .. APPROX_MAX_GROUP)
 * members, member g given by element g of each host array with the meaning
 * of approx_gemm's arguments (transA[g], transB[g], m[g], n[g], k[g], the
 * device pointers A[g], B[g], C[g], lda[g], ldb[g], ldc[g]). For callers that
 * run GEMMs that do not depend on each other back to back, such as the input
 * and weight gradients of a dense layer's backpropagation (ApproxTrain,
 * Section VI-D, AMDENSE): members that approx_gemm would run in its GEMM
 * kernel share one operand-decode launch and one GEMM-kernel launch, which
 * a small GEMM alone cannot fill. Each member is computed exactly as
 * approx_gemm computes it (same products and summation order, so the same
 * bits; approx_gemm_chunks describes each member's order); members that
 * approx_gemm runs otherwise (few rows, k = 0, or a kernel shape that cannot
 * be shared) run as approx_gemm runs them, on the same stream. The C of
 * different members must not overlap, nor alias any member's A or B. The
 * host arrays are read during the call only. Errors: APPROX_EINVAL (count
 * outside 1 .. APPROX_MAX_GROUP, a NULL array, or any member failing
 * approx_gemm's checks: nothing is queued then), APPROX_ENOLUT, APPROX_EHIP.
 */
int approx_gemm_grouped(int count, const int *transA, const int *transB, const int *m, const int *n,
                        const int *k, const float *const *A, const int *lda, const float *const *B,
                        const int *ldb, float *const *C, const int *ldc, void *stream);

/*
 * approx_gemm without any allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, hosts
 * that forbid allocation while they run): the same arguments, kernels,
 * products and summation order as approx_gemm, so the results are
 * bitwise identical. Its scratch (decoded operands, exponent statistics,
 * split partials) is one fixed array per device, reserved in the library's
 * code object for the life of the process: approx_gemm_noalloc_max_bytes()
 * bytes (64 MiB less the statistics). Its device address is looked up when
 * a table (or the native multiplier) is loaded on the device, so these calls
 * make no runtime lookups either. A call that needs more (about
 * 8 * (ceil(k/4)*4) * (m + n) bytes of decoded operands (4 * ... with the
 * native multiplier), rows and columns rounded up to the kernel's tiles,
 * plus split partials; row-vector calls
 * need only their partials) returns APPROX_ESCRATCH before queuing
 * anything. Every call on a device shares that device's array and
 * re-initialises what must start at zero, so calls that overlap in time on
 * one device (on different streams, or from different threads) race:
 * order them on one stream. The table must be loaded beforehand
 * (approx_lut_load allocates). Kernel timing (approx_profile_enable) skips
 * these calls. Errors: as approx_gemm, and APPROX_ESCRATCH.
 */
int approx_gemm_noalloc(int transA, int transB, int m, int n, int k,
                        const float *A, int lda, const float *B, int ldb,
                        float *C, int ldc, void *stream);

/* Bytes of scratch available to one approx_gemm_noalloc call. */
long long approx_gemm_noalloc_max_bytes(void);

/*
 * `batch` independent GEMMs: matrix b uses A + b*strideA, B + b*strideB and
 * C + b*strideC (strides in elements, >= 0), each as approx_gemm. Used for
 * the per-head products of attention (ApproxTrain Section III: attention is
 * matrix multiplication underneath). Output matrices must not overlap.
 */
int approx_gemm_strided_batched(int transA, int transB, int m, int n, int k,
                                const float *A, int lda, long long strideA,
                                const float *B, int ldb, long long strideB,
                                float *C, int ldc, long long strideC,
                                int batch, void *stream);

/*
 * `batch` independent GEMMs given by arrays of device pointers: A[b], B[b]
 * and C[b] (the arrays themselves in device memory, caller-owned, read by
 * the kernels while they run). Each entry is as approx_gemm with the shared
 * sizes and leading dimensions; output matrices must not overlap. Serves
 * batches that no single stride describes, such as the (sequence, head)
 * products of multi-head attention. Errors: as approx_gemm, and
 * APPROX_EINVAL for NULL arrays.
 */
int approx_gemm_batched(int transA, int transB, int m, int n, int k,
                        const float *const *A, int lda,
                        const float *const *B, int ldb,
                        float *const *C, int ldc,
                        int batch, void *stream);

/*
 * Conv2D as implicit GEMM (ApproxTrain Section VI-B, Algorithms 3 and 4).
 * Activations NHWC [N,H,W,C]; weights RSCK (HWIO) [R,S,C,K]; outputs NHWC
 * [N,P,Q,K] with P = (H + 2*pad_h - R)/stride_h + 1, Q likewise.
 * Cross-correlation (no filter flip in the forward pass), no dilation, no
 * groups. Padding positions are zero operands that are multiplied, exactly
 * as the zeros an explicit IM2COL buffer would hold.
 *
 * fwd:   y[n,p,q,k]  = sum_{r,s,c} approx(x[n, p*sh-ph+r, q*sw-pw+s, c], w[r,s,c,k])
 * dgrad: dx[n,h,w,c] = sum_{r,s,k} approx(D[n, h+ph-r, w+pw-s, k], w[r,s,c,k])
 *        where D holds dy[n, a/sh, b/sw, k] at offsets (a, b) that are
 *        multiples of the strides inside the output, and zero elsewhere (the
 *        padded, dilated errors, with the filter transposed and reversed).
 * wgrad: dw[r,s,c,k] = sum_{n,p,q} approx(x[n, p*sh-ph+r, q*sw-pw+s, c], dy[n,p,q,k])
 * Table operand order: (x, w), (dy, w) and (x, dy).
 * Errors: APPROX_EINVAL (non-positive sizes or strides, negative pads,
 * R > H + 2*pad_h or S > W + 2*pad_w, NULL pointers), APPROX_ENOLUT,
 * APPROX_EHIP.
 */
int approx_conv2d_fwd(int N, int H, int W, int C, int K, int R, int S,
                      int stride_h, int stride_w, int pad_h, int pad_w,
                      const float *x, const float *w, float *y, void *stream);

int approx_conv2d_dgrad(int N, int H, int W, int C, int K, int R, int S,
                        int stride_h, int stride_w, int pad_h, int pad_w,
                        const float *dy, const float *w, float *dx, void *stream);

int approx_conv2d_wgrad(int N, int H, int W, int C, int K, int R, int S,
                        int stride_h, int stride_w, int pad_h, int pad_w,
                        const float *x, const float *dy, float *dw, void *stream);

/*
 * The summation order of compute calls (see the top of this header), for
 * callers that reproduce results exactly. Host only: queues nothing, but
 * uses the current device's table width, which selects between kernels.
 *
 * approx_gemm_chunks: for a GEMM call with these arguments (batch = 1 for
 * approx_gemm), chunk[t] = the chunk length L of output (b[t], i[t], j[t]):
 * L = k when that output's reduction is one chunk, 0 when k = 0.
 *
 * approx_conv2d_chunks: pass APPROX_CONV_FWD, _DGRAD or _WGRAD, output at
 * flat index idx[t] of [N,P,Q,K], [N,H,W,C] or [R,S,C,K]. The reduction
 * sequences (C4, K4: C and K rounded up to a multiple of 4; positions past C
 * or K hold no product):
 *   fwd:   term (r, s, c) at position (r*S + s)*C4 + c;
 *   dgrad: term (r, s, k) at position ((R-1-r)*S + (S-1-s))*K4 + k (the
 *          transposed, reversed filter of Section VI-B);
 *   wgrad: term (n, p, q) at position (n*P + p)*Q + q.
 * chunk[t] >= the sequence's length means one chunk.
 * Errors: APPROX_EINVAL (bad sizes, flags, NULL arrays with count > 0,
 * indices out of range), APPROX_ENOLUT.
 */
#define APPROX_CONV_FWD 0
#define APPROX_CONV_DGRAD 1
#define APPROX_CONV_WGRAD 2
int approx_gemm_chunks(int transA, int transB, int m, int n, int k, int batch, long long count,
                       const int *b, const int *i, const int *j, long long *chunk);
int approx_conv2d_chunks(int pass, int N, int H, int W, int C, int K, int R, int S,
                         int stride_h, int stride_w, int pad_h, int pad_w,
                         long long count, const long long *idx, long long *chunk);

/*
 * Kernel timing for benchmarks. While enabled (on != 0), every compute call
 * records a HIP event pair around its GEMM kernel, on the call's stream.
 * approx_profile_read waits for the recorded events, returns the number of
 * GEMM-kernel launches and their summed duration in milliseconds, and clears
 * the record. Errors: APPROX_EINVAL (NULL outputs), APPROX_EHIP.
 */
int approx_profile_enable(int on);
int approx_profile_read(int *launches, double *total_ms);

/* Static text for a status code. */
const char *approx_status_string(int status);

/* Static text: the first 16 hex digits of a SHA-256 over the library's
 * source files at build time ("unstamped" when built without it), so that a
 * binary can be matched with the sources it came from. */
const char *approx_build_id(void);

/* Synchronise every device the library used, then free its tables and
 * arenas. A table must be loaded again before the next compute call. */
int approx_release(void);

#ifdef __cplusplus
}
#endif

#endif /* APPROX_MUL_H */
