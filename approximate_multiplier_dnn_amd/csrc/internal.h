// internal.h -- parameter blocks and launchers shared by the host API
// (api.cpp) and the gfx950 kernels (kernels.hip). Not part of the C ABI.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "replica.h"

namespace amx {

// Decoded operand word, one per FP32 element, written by the decode pass and
// read by the GEMM kernel (with the native multiplier, M = 0, the panels hold
// only the se half: 4 bytes per element, the operand's own bits). Two roles:
//  - lane operand (varies across the 64 lanes of a wave): w = byte offset,
//    relative to a table column, of its mantissa row (2 * index as the decode
//    writes it; at M = 8 the copy choice may move it to the row's second
//    copy, replica.h), or of the column's zero pad entry for zero /
//    subnormal / Inf / NaN;
//  - uniform operand (the same for every lane at a given step): w = byte
//    offset of its table column.
// se = sign | exponent bits for normals (the float +-2^(E-127) * 2^0 with the
//      exponent field kept), 0 for zero and subnormal, +-Inf for Inf and
//      0x7FC00000 for NaN.
struct Word {
    uint32_t w;
    uint32_t se;
};

// Workgroup shapes of the GEMM kernel: `waves` waves per workgroup, each lane
// accumulating `rows_per_lane` output rows x kColsPerWave columns, so a wave
// covers 64 * rows_per_lane rows and kColsPerWave columns. Shape 0: 8 waves
// (2 per SIMD) x 4 rows; shape 1: 12 waves (3 per SIMD) x 3 rows, which hides
// more lookup latency at the cost of coarser row tiles; shape 2: 8 waves x 2
// rows, tiles of half the area of shape 0's for small outputs, whose
// reductions then split into half as many chunks (vector mode only: GEMMs and
// the convolution's forward and input-gradient passes).
struct KernelShape {
    int waves, rows_per_lane;
};
constexpr int kNumShapes = 3;
constexpr KernelShape kShapes[kNumShapes] = {{8, 4}, {12, 3}, {8, 2}};
constexpr int kColsPerWave = 16;

// Table image in device memory, laid out as the LDS copy the kernels use.
// A column holds the 2^M entries of one uniform-operand mantissa (lane
// operand's mantissa = row) followed by two zero entries (the pad, read by
// zero, Inf and NaN lane operands). An M = 8 column is 640 bytes: its 256
// entries, the pad and second copies of its first 31 dwords (replica.h).
__host__ __device__ inline int lut_col_entries(int M) { return M == 8 ? kRep8ColBytes / 2 : (1 << M) + 2; }
__host__ __device__ inline int lut_col_bytes(int M) { return lut_col_entries(M) * 2; }
__host__ __device__ inline int lut_image_bytes(int M) { return (1 << M) * lut_col_bytes(M); }

// Row tiles per swizzle group: the 32 workgroups of one XCD (consecutive work
// items, see main_kernel) take 2 row tiles x 16 column tiles, which they
// share through that XCD's L2 (per reduction index 2 x 256 rows and 16 x 128
// columns of operand words at 8192^3, against 256 rows and 32 x 128 columns
// in plain row-major order). Measured on 8192^3 (FETCH_SIZE per launch): 1 ->
// 9.44 M KiB, 2 -> 6.38 M KiB, 4 -> 6.40 M KiB; the kernel time is unchanged
// because the LDS lookups bind.
constexpr int TILE_GROUP_M = 2;

// Tile order of the GEMM kernel's work items: groups of TILE_GROUP_M row
// tiles, column tiles outer, row tiles inner within a group.
__host__ __device__ inline void tile_coords(int tile, int tiles_m, int tiles_n, int& tm, int& tn)
{
    const int group = tile / (TILE_GROUP_M * tiles_n);
    const int first_m = group * TILE_GROUP_M;
    const int gm = (tiles_m - first_m < TILE_GROUP_M ? tiles_m - first_m : TILE_GROUP_M);
    const int in_group = tile - group * TILE_GROUP_M * tiles_n;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// The inverse: the position in that order of row tile tm, column tile tn.
__host__ __device__ inline int tile_index(int tm, int tn, int tiles_m, int tiles_n)
{
    const int group = tm / TILE_GROUP_M;
    const int first_m = group * TILE_GROUP_M;
    const int gm = tiles_m - first_m < TILE_GROUP_M ? tiles_m - first_m : TILE_GROUP_M;
    return group * TILE_GROUP_M * tiles_n + tn * gm + (tm - first_m);
}

// LDS footprint classes of the GEMM kernel (tables of M = 9..11 are read
// from global memory instead).
constexpr int LDS_SMALL = (1 << 7) * ((1 << 7) + 2) * 2;  // M <= 7: 33,280 bytes
constexpr int LDS_LARGE = (1 << 8) * kRep8ColBytes;       // M == 8: 163,840 bytes (all of the LDS)

enum Layout : int {
    L_DENSE_LANE = 0,    // A of a GEMM -> [batch][KB][Mp][4]
    L_DENSE_UNIFORM,     // B of a GEMM -> [batch][Kp][Np]
    L_IMG_FWD,           // conv x  -> [N][H+2ph][Cb][W+2pw][4]   (lane)
    L_IMG_DGRAD,         // conv dy -> padded dilated [N][H+R-1][Kb][W+S-1][4] (lane)
    L_W_FWD,             // conv w  -> [R*S*Cp][Np] (uniform)
    L_W_DGRAD,           // conv w  -> reversed, transposed [R*S*Kp][Np] (uniform)
    L_IMG_WGRAD,         // conv x  -> [N][H+2ph][W+2pw][C] + zero tail (lane)
    L_DY_WGRAD,          // conv dy -> [Kp = NPQ rounded up to 4][Np] (uniform)
};

// Division by a divisor fixed for the launch (Granlund & Montgomery,
// "Division by invariant integers using multiplication", 1994): for
// n < 2^31, n / d = (umulhi(n, m) + n) >> l with l = ceil(log2 d) and
// m = floor(2^32 (2^l - d) / d) + 1.
struct FastDiv {
    uint32_t d, m, l;
};

inline FastDiv make_fastdiv(uint32_t d)
{
    uint32_t l = 0;
    while (((uint64_t)1 << l) < d) ++l;
    const uint64_t m = (((uint64_t)1 << 32) * (((uint64_t)1 << l) - d)) / d + 1;
    return FastDiv{d, (uint32_t)m, l};
}

// Exponent statistics of one call: STAT_SLOTS slots, each on its own
// 128-byte line, holding {lane min, lane max, uniform min, uniform max}.
// Decode workgroups fold their range into slot (block % STAT_SLOTS); the GEMM
// kernel reduces the slots.
// The int after the slots counts the GEMM workgroups that have read them: the
// last one resets the slots (and the count) for the stream's next call, so a
// stream's stats need initialising only once. A grouped call keeps one such
// block per GEMM of the group, STAT_BLOCK_INTS apart.
constexpr int STAT_SLOTS = 64;
constexpr int STAT_STRIDE = 32;   // ints between slots
constexpr int STAT_INTS = STAT_SLOTS * STAT_STRIDE;
constexpr int STAT_READERS = STAT_INTS;   // index of the reader count
// Per k-segment ranges (dense GEMMs whose decodes write them): segment s
// covers reduction indices [64 s, 64 s + 64), that is k-steps [16 s, 16 s + 16),
// and holds SEG_REPL replicas of {lane min, lane max, uniform min, uniform max}
// at STAT_SEG + 4 (SEG_REPL s + r) (a decode workgroup folds into replica
// (its index mod SEG_REPL), so fewer workgroups meet at one address), each as
// (call generation << 8) | value, folded with atomicMax (a minimum e as
// 255 - e); a reader takes the maximum over the replicas. A call whose whole range fails the fast test still runs its
// fast path on every segment whose own ranges pass it. Nothing resets them:
// a tag older than the call's generation means the call wrote nothing there
// (no normal values), a newer one (a graph replayed after later calls) that
// the segment's ranges are unknown, so the call's own range decides it.
constexpr int STAT_SEG = STAT_INTS + 64;
constexpr uint32_t SEG_GEN_MAX = 1u << 24;   // generations run 1 .. 2^24 - 1, then the blocks are re-initialised
constexpr int SEG_KSTEPS = 16;
constexpr int SEG_MAX = 1024;             // segments per call (k up to 65,536)
constexpr int SEG_REPL = 4;
constexpr int STAT_BLOCK_INTS = STAT_SEG + 4 * SEG_REPL * SEG_MAX;   // one block: slots, counts, segments

// GEMMs of one grouped call (one decode launch, one GEMM-kernel launch).
constexpr int kMaxGroup = 4;

struct DecodeParams {
    int* seg;                       // this operand's k-segment ranges (segment s, replica r: min at seg[4 (SEG_REPL s + r)], max after it), or null
    uint32_t seg_gen;               // the call's generation, shifted left by 8
    const float* src;
    const float* const* src_ptrs;   // batched by pointer array (device), else src + b * stride
    void* dst;           // Words (wbytes 8) or, for the native multiplier, the operands' bits (wbytes 4)
    int wbytes;
    int* stats;          // slot base + role offset (0: lane, 2: uniform)
    int64_t count;       // words per batch entry
    int64_t src_batch_stride;  // elements
    int64_t dst_batch_stride;  // words
    int batch;
    int layout;
    int lane_role;       // 1: lane operand, 0: uniform operand
    int M;
    int elo, ehi;        // FP32 biased exponents of the format's normal range (1, 254 for FP32)
    // geometry (meaning depends on layout)
    int m, n, k, ld, trans;    // dense
    int Mp, Np, KB;            // padded extents
    int N, H, W, C, K, R, S, sh, sw, ph, pw, P, Q;
    int Hp, Wp, Cb, Cp, Kb, Kp;
    // divisors of the per-element index math (set by the host for the layout)
    FastDiv fd_Mp, fd_Np, fd_Cp, fd_Kp, fd_S, fd_Wp, fd_Cb, fd_Kb, fd_Hp, fd_C;
    int rows;            // image layouts: output rows (N * rows per image)
    int row_floats;      // image layouts: floats in one source row
    // dense and uniform panels: Words of one logical row (Mp*4 for the lane
    // panel, Np for uniform panels) and the padded stride between rows
    int rowlen, ldw;
    FastDiv fd_rowlen;
};

// One operand's decode in a combined launch: the variant for its layout and
// its own grid of 256-thread workgroups.
enum DecodeVariant : int { DV_IMG = 0, DV_ROWS, DV_TILE, DV_GENERIC, DV_DIRECT };
struct DecodeJob {
    DecodeParams p;
    int variant;
    uint32_t gx, gy, gz;
    int rb;              // row copies: rows per workgroup
};

// Row stride of a panel. Kept equal to the row length: padding the large
// power-of-two rows was measured to raise the GEMM kernel's L2 misses on
// MI355X (8192^3: FETCH_SIZE 10.3 -> 13.5 M KiB per launch).
inline int panel_ld(int rowlen)
{
    return rowlen;
}

// GEMM kernel parameters. The lane operand of row i and k-step u is read at
// panel + lane_base(i) + koff(u) (in Words); lane_base decomposes i into
// (i1, i2, i3) with extents (., E2, E3) and strides (L1, L2, L3); koff
// decomposes u into (u1, u2, u3) with extents (U1, U2, U3) and strides
// (K1, K2, K3), u3 fastest. In vector mode a k-step covers 4 consecutive
// reduction indices stored contiguously; in gather mode every reduction index
// is its own step and steps >= nku read the zero region at zoff.
struct MainParams {
    const void* panel;        // lane operand words (Words; 4-byte words for the native multiplier)
    const void* bpanel;       // uniform operand words [Kp][Np] (likewise)
    const uint16_t* lut;      // table image (lane-first layout)
    const int* stats;         // STAT_SLOTS slots of {lane min, lane max, uniform min, uniform max}
    float* out;               // C
    float* const* out_ptrs;   // batched by pointer array (device): C of entry b
    float* ws;                // chunk partials of the split tiles (splits > 1)
    int64_t panel_batch;      // Words between batch entries of the lane panel
    int64_t bpanel_batch;     // Words between batch entries of the uniform panel
    int64_t out_batch;        // floats between batch entries of C
    int lut_bytes;
    int m_rows;               // valid rows (lane rows are clamped below this)
    int m_out, n_out, ldc;    // output extent and leading dimension
    int Np;
    int bld;                  // Words between rows of the uniform panel (>= Np)
    int E2, E3, L1, L2, L3;
    int U1, U2, U3, K1, K2, K3;
    int nku, zoff;            // gather mode
    int KB;                   // k-steps of 4 reduction indices (vector) / 4-groups (gather)
    int wr, wc;               // waves per workgroup along rows / columns (wr*wc = the shape's waves)
    int tiles_m, tiles_n;
    // Work items: the first full_items (batch entry, tile) pairs whole, in
    // the order b * tiles + tile; then the remaining tail_tiles pairs in
    // `splits` reduction chunks of `chunk` k-steps (of 4) each, item
    // full_items + split * tail_tiles + t. Chunk partials go to
    // ws[(b * splits + split) * m_out * n_out + ...]; whole tiles to C.
    int full_items, tail_tiles, splits, chunk;
    int batch;
    int64_t items;
    int force_checked;        // 1: always use the per-product checked path
    int elo, ehi;             // FP32 biased exponents of the format's normal range (1, 254 for FP32)
    int segs;                 // k-segments with ranges in stats (0: the call's range only)
    uint32_t seg_gen;         // the call's generation, shifted left by 8
};

// Copy choice of the M = 8 lane-operand table offsets (replica.h), one group
// of up to 32 Words per thread: group (b, g1, g2, g3) holds the Words at
//   panel + b * batch_stride + g1 * S1 + g2 * S2 + g3 * S3 + O + l * LS
// for l < min(32, E - 32 * g2): the operands one half-wave of the GEMM
// kernel reads together at one reduction index.
struct AssignParams {
    Word* panel;
    int64_t batch_stride;
    int64_t S1;
    int batch, G1, G2, G3;
    int S2, S3, LS, O, E;
    uint32_t pad_w;        // offset of the zero pad entry
};

struct ReduceParams {
    const float* ws;
    float* out;
    float* const* out_ptrs;
    int m, n, ldc, splits, batch;
    int64_t out_batch;
};

// Sum of the chunk partials of the GEMM kernel's split tiles (the tail of
// its work items): tiles first_tile .. first_tile + n_tiles - 1 of the order
// b * tiles + tile, each TM x TN outputs of C.
struct ReduceTilesParams {
    const float* ws;
    float* out;
    float* const* out_ptrs;
    int m, n, ldc, splits;
    int64_t out_batch;
    int tiles_m, tiles_n, TM, TN;
    int first_tile, n_tiles;
};

// One call's reduction as a part of a combined launch: the variant (plain:
// a thread per 4 outputs; rows: 16 lanes per 4 outputs; tiles: the split
// tiles only), its parameters and its workgroups.
enum ReduceVariant : int { RV_PLAIN = 0, RV_ROWS, RV_TILES };
struct ReduceJob {
    int variant;
    uint32_t blocks;
    ReduceParams r;           // plain and rows
    ReduceTilesParams t;      // tiles
};

// Row-vector GEMM (few rows of op(A): up to 32, or 64 when k * n >= 2^22 or
// k * n <= 2^16; B not transposed), one launch of a persistent grid: a work
// item is a block of kGemvMaxRows rows x a column block x a reduction chunk
// of `chunk` indices; lanes run over output columns and each operand is
// decoded in registers as it is read. Tables of M <= 8 are staged in LDS
// once per workgroup, larger ones are read from global memory.
constexpr int kGemvMaxRows = 4;
constexpr int kGemvThreads = 256;            // table in global memory / native
constexpr int kGemvLdsThreads = 1024;        // table staged in LDS (one copy per workgroup)
constexpr int kGemvColsPerLane = 4;          // one workgroup's thread count apart
constexpr int kGemv1Threads = 256;           // one-row kernel (m = 1, M <= 8): table rows staged per window
constexpr int kGemv1Window = 32;             // reduction indices per staged window (one table row each)
constexpr int kGemv1Stage = 4;               // 16-byte pieces of a window (M = 8) per thread

// Group loads of the row-vector kernel. A work item sums reduction indices
// [k0, k1); a load of the group that starts at index kg >= k0 (kg may lie
// past k1 - 1: a request made ahead of the item's end) addresses B through a
// buffer descriptor based at row gemv_group_base(kg, k1), and its index g
// reads row base + gemv_group_step(kg, k1, g). Every row read lies in
// [k0, k1 - 1] and no offset from the base is negative; for kg + g < k1 the
// row is kg + g itself.
__host__ __device__ inline int gemv_group_base(int kg, int k1) { return kg < k1 - 1 ? kg : k1 - 1; }
__host__ __device__ inline int gemv_group_step(int kg, int k1, int g)
{
    const int last = k1 - 1 - gemv_group_base(kg, k1);
    return g < last ? g : last;
}

struct GemvParams {
    const float* A;
    const float* const* A_ptrs;   // batched by pointer array (device), else A + b * A_batch
    const float* B;
    const float* const* B_ptrs;
    const uint16_t* lut;          // table in index order (ia << M) | ib; unused by the native multiplier
    float* out;                   // C, or split partials when splits > 1
    float* const* out_ptrs;
    int64_t A_batch, B_batch, out_batch;   // elements
    int M, m, n, k, lda, ldb, ldc, transA;
    int splits, chunk, batch;
    int elo, ehi;                 // FP32 biased exponents of the format's normal range (1, 254 for FP32)
    int force_checked;            // 1: always use the per-product checked path
};

// variant: 0 = table of M <= 7 in LDS, 1 = M == 8 in LDS, 2 = table in global
// memory, 3 = native multiplier, 4 = one row of op(A) with M <= 8 (table rows
// staged per window). The kernel is persistent over `grid` workgroups of
// gemv_threads(variant) threads.
int gemv_threads(int variant);
int gemv_blocks_per_cu(int variant);
hipError_t launch_gemv(const GemvParams& p, int variant, int grid, hipStream_t s);
// Initialises `blocks` statistics blocks (STAT_BLOCK_INTS apart).
hipError_t launch_init_stats(int* stats, int blocks, hipStream_t s);
// The decodes of `count` operands (at most 2 * kMaxGroup) in one launch.
hipError_t launch_decode_group(const DecodeParams* const* jobs, int count, hipStream_t s);
// Whether this operand's decode runs in workgroups that each cover reduction
// indices of one k-segment only (and can so record the segment ranges).
bool decode_covers_segments(const DecodeParams& p);
hipError_t launch_decode_pair(const DecodeParams& a, const DecodeParams& b, hipStream_t s);
hipError_t launch_assign(const AssignParams& p, hipStream_t s);
hipError_t launch_main(const MainParams& p, int lds_class, int gather, int shape, int grid, hipStream_t s);
// `count` (at most kMaxGroup) GEMM-kernel calls of one variant in one launch:
// their work items in order, ps[g]->items each; each keeps its own stats.
hipError_t launch_main_group(const MainParams* const* ps, int count, int lds_class, int gather, int shape, int grid,
                             hipStream_t s);
// Whether several calls of this variant can share a launch (count > 1), and
// the resident workgroups per CU of that grouped kernel.
bool main_group_supported(int gather, int shape);
int main_group_blocks_per_cu(int lds_class, int shape);
hipError_t launch_reduce(const ReduceParams& p, hipStream_t s);

// The reduction runs 16 lanes per 4 outputs (reduce_rows_kernel) when the
// outputs are few (m * n * batch a multiple of 4, below 2^18) and the splits
// many (at least 32, or at least 16 for at most 2^16 outputs); otherwise a
// thread per 4 outputs (or one). Both sum each output's partials in
// ascending split order from +0. (256 x 784 outputs in 19 splits: 9.7 us by
// rows, where 16 lanes wait on 2 partials each, against 5 us for the
// thread-per-4 kernel on outputs of the same size.)
inline bool reduce_by_rows(int m, int n, int batch, int splits)
{
    const int64_t total = (int64_t)m * n * batch;
    return ((int64_t)m * n) % 4 == 0 && total < ((int64_t)1 << 18) &&
           (splits >= 32 || (splits >= 16 && total <= ((int64_t)1 << 16)));
}
hipError_t launch_reduce_tiles(const ReduceTilesParams& p, hipStream_t s);
// The reductions of several calls (their jobs, as reduce_job and
// reduce_tiles_job plan them) in one launch; count <= kMaxGroup.
ReduceJob reduce_job(const ReduceParams& p);
ReduceJob reduce_tiles_job(const ReduceTilesParams& p);
hipError_t launch_reduce_group(const ReduceJob* jobs, int count, hipStream_t s);
hipError_t launch_fill_zero(float* C, float* const* Cp, int m, int n, int ldc, int batch, int64_t strideC,
                            hipStream_t s);
int main_blocks_per_cu(int lds_class, int gather, int shape);

}  // namespace amx
