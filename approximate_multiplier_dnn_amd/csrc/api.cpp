// api.cpp -- the C ABI: argument checks, per-device table state, per-stream
// scratch arenas, and the plan (decode layouts, tiling, reduction split) of
// each GEMM / Conv2D call. Every arithmetic step runs in kernels.hip.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

#include "../../include/approx_mul.h"
#include "internal.h"

namespace {

using amx::DecodeParams;
using amx::MainParams;
using amx::ReduceParams;
using amx::Word;

constexpr int kMaxDevices = 64;
using amx::kColsPerWave;
using amx::kShapes;
// Reduction-split model (a function of the shapes only, so results never
// depend on the device): kSplitSlots resident workgroups (the MI355X's 256
// CUs, one GEMM workgroup each), kSplitMacRate approximate MAC/s over the
// GPU, kSplitBytesRate bytes/s for the reduction of the chunk partials.
constexpr int64_t kSplitSlots = 256;
constexpr double kSplitMacRate = 6.0e12;
constexpr double kSplitBytesRate = 4.0e12;
constexpr int kSplitMax = 1024;
constexpr int64_t kMaxPanelWords = (int64_t)1 << 31;
// Few-row GEMMs (B not transposed) run in the row-vector kernel, in blocks
// of 4 rows, instead of the GEMM kernel's 256-row tiles: always up to
// kRowVectorRows rows; up to kRowVectorRowsWide rows when k * n is large (B
// streams at full rate) or tiny (the launch dominates). Measured (M = 8,
// row-vector against GEMM kernel): 32 x 8192 x 8192 0.78 / 1.62 ms,
// 64 x 8192 x 8192 1.49 / 1.62 ms, 64 x 64 x 64 0.020 / 0.045 ms, but
// 64 x 1024 x 1024 0.103 / 0.093 ms.
constexpr int kRowVectorRows = 32;
constexpr int kRowVectorRowsWide = 64;
inline bool row_vector_fits(int m, int n, int k)
{
    const int64_t kn = (int64_t)k * n;
    if (n >= (1 << 30)) return false;          // the kernel's column offsets are 32-bit byte offsets
    return m <= kRowVectorRows || (m <= kRowVectorRowsWide && (kn >= ((int64_t)1 << 22) || kn <= ((int64_t)1 << 16)));
}

struct DeviceTable {
    uint16_t* image = nullptr;  // lane-first LDS image (the allocation; `flat` lies in it)
    uint16_t* flat = nullptr;   // the table in index order (ia << M) | ib, for the row-vector kernel
    int M = 0;
    bool native = false;        // the native FP32 multiplier is selected (no image)
};

// Per (device, stream) scratch: the exponent stats of the GEMM calls first
// (kStatsBytes), then decoded panels and split partials. The GEMM kernel
// leaves the stats reset for the next call on the stream, so they are
// initialised only when the arena is new or a call stopped between its decode
// and GEMM launches (stats_ready false).
struct Arena {
    void* ptr = nullptr;
    size_t bytes = 0;
    bool stats_ready = false;
    uint32_t gen = 0;           // generation of the last call's k-segment ranges (1 .. SEG_GEN_MAX - 1)
};

std::mutex g_mu;
DeviceTable g_tables[kMaxDevices];
int g_exp_bits[kMaxDevices];       // exponent width of the multiplier's format per device (0 = unset: 8)
bool g_profile = false;
std::vector<std::pair<hipEvent_t, hipEvent_t>> g_events;   // GEMM-kernel launches while profiling
std::map<std::pair<int, hipStream_t>, Arena> g_arenas;
// Device memory that a table load or an arena's growth superseded: kept until
// approx_release, so that work already queued and HIP graphs captured
// earlier never read freed memory.
std::vector<std::pair<int, void*>> g_retired;

int current_device(int* dev)
{
    if (hipGetDevice(dev) != hipSuccess) return APPROX_EHIP;
    if (*dev < 0 || *dev >= kMaxDevices) return APPROX_EHIP;
    return APPROX_OK;
}

size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

// One statistics block per GEMM of a grouped call (a single call uses the first).
const size_t kStatsBytes = align256((size_t)amx::STAT_BLOCK_INTS * amx::kMaxGroup * sizeof(int));

// Scratch memory for one call on (device, stream): `bytes` after the stats
// region (*out points past it; *stats at it). Grows only, at least doubling,
// so the superseded arenas (retired, not freed) hold less memory than the
// current one. *ready: whether the stats hold the reset values (the caller
// initialises them and sets it).
// Test hook for the allocation-failure path: with APPROX_TEST_ALLOC_LIMIT set
// to a byte count, a scratch allocation larger than it fails as a failed
// hipMalloc would (APPROX_EHIP, nothing queued).
bool alloc_refused(size_t bytes)
{
    const char* v = std::getenv("APPROX_TEST_ALLOC_LIMIT");
    return v != nullptr && v[0] != '\0' && bytes > (size_t)std::strtoull(v, nullptr, 10);
}

int arena_get(int dev, hipStream_t stream, size_t bytes, char** out, int** stats = nullptr, bool** ready = nullptr,
              uint32_t** gen = nullptr)
{
    std::lock_guard<std::mutex> lock(g_mu);
    Arena& a = g_arenas[{dev, stream}];
    bytes += kStatsBytes;
    if (a.bytes < bytes) {
        const size_t want = std::max(bytes + bytes / 8, 2 * a.bytes);
        void* p = nullptr;
        if (alloc_refused(want) || hipMalloc(&p, want) != hipSuccess) return APPROX_EHIP;
        if (a.ptr != nullptr) g_retired.emplace_back(dev, a.ptr);
        a.ptr = p;
        a.bytes = want;
        a.stats_ready = false;
    }
    *out = static_cast<char*>(a.ptr) + kStatsBytes;
    if (stats != nullptr) *stats = static_cast<int*>(a.ptr);
    if (ready != nullptr) *ready = &a.stats_ready;   // std::map nodes are stable
    if (gen != nullptr) *gen = &a.gen;
    return APPROX_OK;
}

// Fixed scratch of the allocation-free entry point: one array per device,
// in the code object's device memory, shared by every such call on that
// device. Its device address comes from hipGetSymbolAddress (the array's
// name in host code is a host-side stand-in, not a device address).
constexpr size_t kFixedScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kFixedScratchBytes];
char* g_scratch_ptr[kMaxDevices];

// The device address of this device's fixed scratch (the current device),
// looked up once per device: at its table load (the set-up call every
// device needs), or else on its first allocation-free call.
int fixed_scratch(int dev, char** out)
{
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch_ptr[dev] == nullptr) {
        void* p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return APPROX_EHIP;
        g_scratch_ptr[dev] = static_cast<char*>(p);
    }
    *out = g_scratch_ptr[dev];
    return APPROX_OK;
}

// Where a call's scratch comes from: the stream's arena, or (fixed != nullptr)
// the device's fixed scratch, whose stats region is initialised by every call
// (the previous call on the device may have left anything there).
struct ScratchSource {
    char* fixed = nullptr;
};

int scratch_get(const ScratchSource& src, int dev, hipStream_t stream, size_t bytes, char** out, int** stats,
                bool** ready, uint32_t** gen = nullptr)
{
    if (src.fixed == nullptr) return arena_get(dev, stream, bytes, out, stats, ready, gen);
    if (bytes > kFixedScratchBytes - kStatsBytes) return APPROX_ESCRATCH;
    *out = src.fixed + kStatsBytes;
    if (stats != nullptr) *stats = reinterpret_cast<int*>(src.fixed);
    if (ready != nullptr) *ready = nullptr;
    if (gen != nullptr) *gen = nullptr;
    return APPROX_OK;
}

// Resident GEMM workgroups per device (CUs x blocks per CU), per kernel
// variant; queried once per device and kept.
int64_t g_slots[kMaxDevices][4][2][amx::kNumShapes];

int64_t launch_slots(int dev, int lds_class, int gather, int shape)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int64_t& s = g_slots[dev][lds_class][gather][shape];
    if (s == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
        s = (int64_t)cus * amx::main_blocks_per_cu(lds_class, gather, shape);
    }
    return s;
}

// Resident workgroups of the grouped GEMM kernel (vector mode, shape 0 or 2).
int64_t g_group_slots[kMaxDevices][4][amx::kNumShapes];

int64_t group_slots(int dev, int lds_class, int shape)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int64_t& s = g_group_slots[dev][lds_class][shape];
    if (s == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
        s = (int64_t)cus * amx::main_group_blocks_per_cu(lds_class, shape);
    }
    return s;
}

int table_of(int dev, const uint16_t** image, int* M, const uint16_t** flat = nullptr)
{
    std::lock_guard<std::mutex> lock(g_mu);
    if (flat != nullptr) *flat = g_tables[dev].flat;
    if (g_tables[dev].native) {
        *image = nullptr;
        *M = 0;
        return APPROX_OK;
    }
    if (g_tables[dev].image == nullptr) return APPROX_ENOLUT;
    *image = g_tables[dev].image;
    *M = g_tables[dev].M;
    return APPROX_OK;
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// The format (1, E, M)'s normal range as FP32 biased exponents: bias
// b = 2^(E-1) - 1, unbiased exponents 1-b .. b. E = 8 gives 1 .. 254.
void format_range(int dev, int* elo, int* ehi)
{
    int E;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        E = g_exp_bits[dev] ? g_exp_bits[dev] : 8;
    }
    const int bias = (1 << (E - 1)) - 1;
    *elo = 128 - bias;
    *ehi = 127 + bias;
}

// Waves of a workgroup of the given shape are arranged wr x wc (wr * wc =
// waves): the arrangement whose tiles pad the m x n output least, the wider
// one on a tie (its waves share more lane-operand rows). Returns the padded
// output area.
int64_t pick_waves(int m, int n, int shape, int* wr, int* wc)
{
    const int waves = kShapes[shape].waves, rows = 64 * kShapes[shape].rows_per_lane;
    int64_t best = -1;
    for (int c = waves; c >= 1; --c) {
        if (waves % c) continue;
        const int r = waves / c;
        const int64_t tm = (int64_t)r * rows, tn = (int64_t)c * kColsPerWave;
        const int64_t area = cdiv(m, tm) * tm * (cdiv(n, tn) * tn);
        if (best < 0 || area < best) {
            best = area;
            *wr = r;
            *wc = c;
        }
    }
    return best;
}

// Reduction split. The work items run in rounds over the resident
// workgroups; a round costs its longest item. Two layouts are modelled:
//  - every tile split into the same number of chunks (a split trades the
//    idle workgroups of a partial last round against the partials it writes
//    and the reduction that reads them back);
//  - when the tiles fill at least one round: whole tiles for the full
//    rounds, and only the tiles of the partial last round split, so that
//    their chunks fill that round.
// Picks the layout and split count of least modelled time (returned); ties go
// to fewer splits and to the uniform layout.
double plan_split(int64_t tiles, int KB, double tile_macs_per_kstep, int64_t tile_outs, int64_t out_elems,
                  MainParams& mp)
{
    const int smax = std::max(1, std::min(kSplitMax, KB / 2));
    const double kstep_s = (double)tile_macs_per_kstep / (kSplitMacRate / (double)kSplitSlots);
    const double out_s = 4.0 / kSplitBytesRate;           // per output and pass over the partials
    double best = -1.0;
    int bs = 1;
    int64_t tail = tiles;
    for (int sc = 1; sc <= smax; ++sc) {
        const int c = (int)cdiv(KB, sc), sp = (int)cdiv(KB, c);
        const double gemm = (double)cdiv(tiles * sp, kSplitSlots) * c * kstep_s;
        const double red = sp > 1 ? (double)(sp + 1) * out_elems * out_s : 0.0;
        if (best < 0.0 || gemm + red < best * 0.999) {
            best = gemm + red;
            bs = sp;
            tail = tiles;
        }
    }
    const int64_t rem = tiles % kSplitSlots, full = tiles - rem;
    if (full > 0 && rem > 0) {
        for (int sc = 2; sc <= smax; ++sc) {
            const int c = (int)cdiv(KB, sc), sp = (int)cdiv(KB, c);
            const double gemm = (double)(full / kSplitSlots) * KB * kstep_s + (double)cdiv(rem * sp, kSplitSlots) * c * kstep_s;
            const double red = (double)(sp + 1) * std::min(out_elems, rem * tile_outs) * out_s;
            if (gemm + red < best * 0.999) {
                best = gemm + red;
                bs = sp;
                tail = rem;
            }
        }
    }
    if (bs == 1) tail = 0;
    mp.splits = bs;
    mp.chunk = (int)cdiv(KB, bs);
    mp.tail_tiles = (int)tail;
    mp.full_items = (int)(tiles - tail);
    mp.items = (int64_t)mp.full_items + (int64_t)tail * bs;
    return best;
}

// The split of a GEMM-kernel call (a function of its tiling, reduction
// length and batch only); returns its modelled time. Every shape is modelled
// at the same fold rate per workgroup: shape 2 measured at least shape 0's
// rate where both fill the GPU (M = 7: 2048^3 1.09 against 1.13 ms,
// 4096 x 4096 x 1024 2.12 ms each), although it loads its uniform words twice
// as often per MAC.
double split_of(int tiles_m, int tiles_n, int TM, int TN, int KB, int m, int n, int batch, MainParams& mp)
{
    const int64_t tiles = (int64_t)tiles_m * tiles_n * batch;
    return plan_split(tiles, KB, (double)TM * TN * 4, (int64_t)TM * TN, (int64_t)m * n * batch, mp);
}

// Workgroup shape of a call: the 8-wave shape, unless the 12-wave shape's
// row tiles (576 rows for 3 x 3 x 64 weight gradients, say) pad the output
// by at least 10% less; per MAC the 12-wave shape measured about 10% slower
// (3 x 3 conv forward: 0.720 against 0.653 ms; attention 1.019 against 0.938
// ms per GEMM launch on average), while its exact 576-row tiles cut the 3 x 3
// x 64 weight gradient from 1.065 to 0.622 ms. A call in vector mode
// (`dense`: a GEMM, or a convolution's forward or input-gradient pass; the
// weight gradient's gather mode has no shape-2 kernel) takes shape 2 instead
// of shape 0 when the split model
// gives it at least 3% less time: outputs whose 256 x 128 tiles do not fill
// the GPU, so that shape 0 splits their reductions into many chunks (the
// MLP's 256 x 1024 x 1024 GEMMs: 16 chunks of 128 x 128 tiles instead of 32
// of 256 x 128, 64-71 against 69-76 us per call).
// APPROX_KERNEL_SHAPE=0, 1 or 2 (2: vector mode only) forces a shape (for
// measurements).
int pick_shape(int m, int n, bool dense, int KB, int batch, int* wr, int* wc)
{
    int r[amx::kNumShapes], c[amx::kNumShapes];
    const int64_t a0 = pick_waves(m, n, 0, &r[0], &c[0]);
    const int64_t a1 = pick_waves(m, n, 1, &r[1], &c[1]);
    pick_waves(m, n, 2, &r[2], &c[2]);
    int shape = a1 * 10 <= a0 * 9 ? 1 : 0;
    if (dense && shape == 0 && KB > 0) {
        auto modelled = [&](int sh) {
            const int TM = r[sh] * 64 * kShapes[sh].rows_per_lane, TN = c[sh] * kColsPerWave;
            MainParams tmp{};
            return split_of((int)cdiv(m, TM), (int)cdiv(n, TN), TM, TN, KB, m, n, batch, tmp);
        };
        if (modelled(2) < 0.97 * modelled(0)) shape = 2;
    }
    const char* force = std::getenv("APPROX_KERNEL_SHAPE");
    if (force != nullptr && (force[0] == '0' || force[0] == '1' || (force[0] == '2' && dense))) shape = force[0] - '0';
    *wr = r[shape];
    *wc = c[shape];
    return shape;
}

// Tile geometry of a GEMM-kernel call with an m x n output per batch entry
// (KB k-steps; `dense`: see pick_shape).
struct Tiling {
    int shape, wr, wc, TM, TN, tiles_m, tiles_n;
};

Tiling tiling_of(int m, int n, bool dense, int KB, int batch)
{
    Tiling t;
    t.shape = pick_shape(m, n, dense, KB, batch, &t.wr, &t.wc);
    t.TM = t.wr * 64 * kShapes[t.shape].rows_per_lane;
    t.TN = t.wc * kColsPerWave;
    t.tiles_m = (int)cdiv(m, t.TM);
    t.tiles_n = (int)cdiv(n, t.TN);
    return t;
}

// Summation chunk, in positions of the reduction sequence (4 per k-step), of
// output (b, i, j) of a GEMM-kernel call; KB * 4 when the output is summed
// in one chunk.
struct KernelOrder {
    Tiling t;
    MainParams mp{};
    int KB = 0;

    KernelOrder(int m, int n, int KB_, int batch, bool dense) : t(tiling_of(m, n, dense, KB_, batch)), KB(KB_)
    {
        split_of(t.tiles_m, t.tiles_n, t.TM, t.TN, KB, m, n, batch, mp);
    }
    int64_t chunk(int b, int i, int j) const
    {
        if (mp.splits <= 1) return (int64_t)KB * 4;
        const int tile = amx::tile_index(i / t.TM, j / t.TN, t.tiles_m, t.tiles_n);
        const int64_t tl = (int64_t)b * t.tiles_m * t.tiles_n + tile;
        return tl < mp.full_items ? (int64_t)KB * 4 : (int64_t)mp.chunk * 4;
    }
};

bool force_checked()
{
    const char* v = std::getenv("APPROX_FORCE_CHECKED");
    return v != nullptr && v[0] == '1';
}

// One planned call: the decode of both operands, the GEMM kernel and the
// optional reduction, queued on `stream`.
struct Plan {
    DecodeParams lane{}, uni{};
    MainParams mp{};
    int64_t lane_words = 0, uni_words = 0;    // per batch entry, allocated (rows padded)
    int64_t lane_count = 0, uni_count = 0;    // per batch entry, logical words the decode writes
    int batch = 1;
    int gather = 0;
    int shape = 0;                // workgroup shape (index into kShapes)
    float* C = nullptr;
    float* const* Cp = nullptr;   // output pointer array (batched by pointers)
    int64_t strideC = 0;
    amx::AssignParams asg{};      // M = 8 copy choice of the lane operands (groups of one half-wave)
    // set by plan_finalize: word size, scratch bytes of each part, kernel variant
    int wbytes = 8;
    size_t lane_b = 0, uni_b = 0, part_b = 0;
    int lds_class = 0;
};

// The table-dependent part of a plan (a function of the shapes and M only):
// the reduction split, the word size, the scratch layout and the GEMM-kernel
// variant. APPROX_EUNSUPPORTED when a panel would exceed the word limit.
int plan_finalize(Plan& pl, int M)
{
    MainParams& mp = pl.mp;
    if (pl.lane_words * pl.batch >= kMaxPanelWords || pl.uni_words * pl.batch >= kMaxPanelWords)
        return APPROX_EUNSUPPORTED;
    // M = 0: native multiplier; M = 9..11: table in global memory
    pl.lds_class = M == 0 ? 2 : M <= 7 ? 0 : M == 8 ? 1 : 3;
    const int64_t TM = (int64_t)mp.wr * 64 * kShapes[pl.shape].rows_per_lane, TN = (int64_t)mp.wc * kColsPerWave;
    split_of(mp.tiles_m, mp.tiles_n, (int)TM, (int)TN, mp.KB, mp.m_out, mp.n_out, pl.batch, mp);
    pl.wbytes = M == 0 ? 4 : (int)sizeof(Word);     // the native multiplier keeps only the operands' bits
    pl.lane_b = align256((size_t)pl.lane_words * pl.batch * pl.wbytes);
    pl.uni_b = align256((size_t)pl.uni_words * pl.batch * pl.wbytes);
    pl.part_b = mp.splits > 1 ? align256((size_t)mp.splits * pl.batch * mp.m_out * mp.n_out * sizeof(float)) : 0;
    pl.lane.count = pl.lane_count ? pl.lane_count : pl.lane_words;
    pl.uni.count = pl.uni_count ? pl.uni_count : pl.uni_words;
    return APPROX_OK;
}

// Runs plans[0 .. count) as one call: one scratch request, one decode launch
// for all their operands, the M = 8 copy choices, one GEMM-kernel launch and
// each plan's reduction. count > 1 (at most kMaxGroup): plans of one grouped
// kernel variant (amx::main_group_supported), each with its own stats block.
int run_group(Plan* const* plans, int count, int dev, hipStream_t stream, const uint16_t* image, int M,
              const ScratchSource& src)
{
    if (count < 1 || count > amx::kMaxGroup) return APPROX_EINVAL;
    size_t total = 0;
    for (int g = 0; g < count; ++g) {
        const int rc = plan_finalize(*plans[g], M);
        if (rc != APPROX_OK) return rc;
        total += plans[g]->lane_b + plans[g]->uni_b + plans[g]->part_b;
    }
    const Plan& p0 = *plans[0];
    const int lds_class = p0.lds_class, gather = p0.gather, shape = p0.shape;
    char* base = nullptr;
    int* stats = nullptr;
    bool* stats_ready = nullptr;
    uint32_t* gen_ptr = nullptr;
    int rc = scratch_get(src, dev, stream, total, &base, &stats, &stats_ready, &gen_ptr);
    if (rc != APPROX_OK) return rc;
    // this call's generation for its k-segment ranges (the fixed scratch is
    // initialised by every call: generation 1 always)
    uint32_t gen = 1;
    bool wrapped = false;
    if (gen_ptr != nullptr) {
        std::lock_guard<std::mutex> lock(g_mu);
        if (++*gen_ptr >= amx::SEG_GEN_MAX) {
            *gen_ptr = 1;
            wrapped = true;
        }
        gen = *gen_ptr;
    }
    int elo, ehi;
    format_range(dev, &elo, &ehi);
    const bool forced = force_checked();
    const DecodeParams* jobs[2 * amx::kMaxGroup];
    const MainParams* mps[amx::kMaxGroup];
    int64_t items = 0;
    size_t off = 0;
    for (int g = 0; g < count; ++g) {
        Plan& pl = *plans[g];
        MainParams& mp = pl.mp;
        void* lane_panel = base + off;
        void* uni_panel = base + off + pl.lane_b;
        float* partials = reinterpret_cast<float*>(base + off + pl.lane_b + pl.uni_b);
        off += pl.lane_b + pl.uni_b + pl.part_b;
        int* sg = stats + (size_t)g * amx::STAT_BLOCK_INTS;

        pl.lane.dst = lane_panel;
        pl.lane.wbytes = pl.wbytes;
        pl.uni.wbytes = pl.wbytes;
        pl.lane.stats = sg;
        pl.lane.dst_batch_stride = pl.lane_words;
        pl.lane.batch = pl.batch;
        pl.lane.lane_role = 1;
        pl.lane.M = M;
        pl.lane.elo = pl.uni.elo = mp.elo = elo;
        pl.lane.ehi = pl.uni.ehi = mp.ehi = ehi;
        // k-segment ranges: dense operands decoded a segment per workgroup,
        // one batch entry (a batch's entries would meet in the same
        // segments) and more than one segment (else the call's range says
        // it all); the native multiplier is always on its fast path
        const bool segs = M != 0 && !pl.gather && pl.batch == 1 && mp.KB > amx::SEG_KSTEPS &&
                          mp.KB <= amx::SEG_MAX * amx::SEG_KSTEPS && amx::decode_covers_segments(pl.lane) &&
                          amx::decode_covers_segments(pl.uni);
        mp.segs = segs ? (int)cdiv(mp.KB, amx::SEG_KSTEPS) : 0;
        pl.lane.seg = segs ? sg + amx::STAT_SEG : nullptr;
        pl.uni.seg = segs ? sg + amx::STAT_SEG + 2 : nullptr;
        pl.lane.seg_gen = pl.uni.seg_gen = mp.seg_gen = gen << 8;
        pl.uni.dst = uni_panel;
        pl.uni.stats = sg + 2;
        pl.uni.dst_batch_stride = pl.uni_words;
        pl.uni.batch = pl.batch;
        pl.uni.lane_role = 0;
        pl.uni.M = M;

        mp.panel = lane_panel;
        mp.bpanel = uni_panel;
        mp.lut = image;
        mp.lut_bytes = M ? amx::lut_image_bytes(M) : 0;
        mp.stats = sg;
        mp.panel_batch = pl.lane_words;
        mp.bpanel_batch = pl.uni_words;
        mp.batch = pl.batch;
        mp.force_checked = forced ? 1 : 0;
        mp.out = pl.C;
        mp.out_ptrs = pl.Cp;
        mp.out_batch = pl.strideC;
        mp.ws = mp.splits > 1 ? partials : nullptr;
        jobs[2 * g] = &pl.lane;
        jobs[2 * g + 1] = &pl.uni;
        mps[g] = &mp;
        items += mp.items;
    }

    if (stats_ready == nullptr) {         // fixed scratch: initialised by every call
        if (amx::launch_init_stats(stats, count, stream) != hipSuccess) return APPROX_EHIP;
    } else {
        std::lock_guard<std::mutex> lock(g_mu);
        if (!*stats_ready || wrapped) {         // new arena, or the generations start again
            if (amx::launch_init_stats(stats, amx::kMaxGroup, stream) != hipSuccess) return APPROX_EHIP;
            *stats_ready = true;
        }
        // until the GEMM kernel is queued, the stats the decodes fill are not reset
        *stats_ready = false;
    }
    if (amx::launch_decode_group(jobs, 2 * count, stream) != hipSuccess) return APPROX_EHIP;
    if (M == 8) {                     // M = 8 columns carry second copies to choose from
        for (int g = 0; g < count; ++g) {
            Plan& pl = *plans[g];
            amx::AssignParams& ap = pl.asg;
            ap.panel = static_cast<Word*>(const_cast<void*>(pl.mp.panel));
            ap.batch_stride = pl.lane_words;
            ap.batch = pl.batch;
            ap.pad_w = (1u << M) * 2u;
            if (amx::launch_assign(ap, stream) != hipSuccess) return APPROX_EHIP;
        }
    }

    const int64_t slots = count == 1 ? launch_slots(dev, lds_class, gather, shape) : group_slots(dev, lds_class, shape);
    const int grid = (int)std::min<int64_t>(items, slots);
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    bool prof;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        prof = g_profile && src.fixed == nullptr;     // the allocation-free calls record no events
    }
    if (prof) {
        if (hipEventCreate(&ev0) != hipSuccess || hipEventCreate(&ev1) != hipSuccess) return APPROX_EHIP;
        if (hipEventRecord(ev0, stream) != hipSuccess) return APPROX_EHIP;
    }
    if (amx::launch_main_group(mps, count, lds_class, gather, shape, grid, stream) != hipSuccess) return APPROX_EHIP;
    if (stats_ready != nullptr) {
        std::lock_guard<std::mutex> lock(g_mu);
        *stats_ready = true;      // the GEMM kernel's last workgroups reset them
    }
    if (prof) {
        if (hipEventRecord(ev1, stream) != hipSuccess) return APPROX_EHIP;
        std::lock_guard<std::mutex> lock(g_mu);
        g_events.emplace_back(ev0, ev1);
    }

    // the members' reductions, in one launch
    amx::ReduceJob red[amx::kMaxGroup];
    int nred = 0;
    for (int g = 0; g < count; ++g) {
        const Plan& pl = *plans[g];
        const MainParams& mp = pl.mp;
        if (mp.splits <= 1) continue;
        if (mp.full_items == 0) {                  // every tile split: sum all of C
            ReduceParams rp{};
            rp.ws = mp.ws;
            rp.out = pl.C;
            rp.out_ptrs = pl.Cp;
            rp.m = mp.m_out;
            rp.n = mp.n_out;
            rp.ldc = mp.ldc;
            rp.splits = mp.splits;
            rp.batch = pl.batch;
            rp.out_batch = pl.strideC;
            red[nred++] = amx::reduce_job(rp);
        } else {                                   // only the tail tiles are split
            amx::ReduceTilesParams rp{};
            rp.ws = mp.ws;
            rp.out = pl.C;
            rp.out_ptrs = pl.Cp;
            rp.m = mp.m_out;
            rp.n = mp.n_out;
            rp.ldc = mp.ldc;
            rp.splits = mp.splits;
            rp.out_batch = pl.strideC;
            rp.tiles_m = mp.tiles_m;
            rp.tiles_n = mp.tiles_n;
            rp.TM = mp.wr * 64 * kShapes[pl.shape].rows_per_lane;
            rp.TN = mp.wc * kColsPerWave;
            rp.first_tile = mp.full_items;
            rp.n_tiles = mp.tail_tiles;
            red[nred++] = amx::reduce_tiles_job(rp);
        }
    }
    if (nred == 1 && red[0].variant != amx::RV_TILES) {
        if (amx::launch_reduce(red[0].r, stream) != hipSuccess) return APPROX_EHIP;
    } else if (nred == 1) {
        if (amx::launch_reduce_tiles(red[0].t, stream) != hipSuccess) return APPROX_EHIP;
    } else if (nred > 1) {
        if (amx::launch_reduce_group(red, nred, stream) != hipSuccess) return APPROX_EHIP;
    }
    return APPROX_OK;
}

int run_plan(Plan& pl, int dev, hipStream_t stream, const uint16_t* image, int M, const ScratchSource& src)
{
    Plan* plans[1] = {&pl};
    return run_group(plans, 1, dev, stream, image, M, src);
}

// Reduction split of the row-vector kernel (a function of the shapes and the
// table width only): about 256 x 1024 threads' worth of work items (column
// block x split), i.e. one 1024-thread workgroup per CU of the MI355X, so each
// item streams a long stretch of B; chunks of at least 8 indices.
constexpr int64_t kGemvTargetThreads = 256 * 1024;

int64_t g_gemv_slots[kMaxDevices][5];

// Row-vector kernel variant of a call: the native multiplier (3); one row at
// M <= 8 (4: table rows staged per window); at most 256 columns (2: the
// 256-thread kernel reading the table from global memory, since a 1024-thread
// workgroup that stages the whole table would leave 15 of 16 lanes without a
// column of their own); else the table in LDS (0: M <= 7, 1: M = 8) or in
// global memory (2: M = 9..11).
int gemv_variant_of(int M, int m, int n)
{
    if (M == 0) return 3;
    if (m == 1 && M <= 8) return 4;
    if (n <= 256) return 2;
    return M <= 7 ? 0 : M == 8 ? 1 : 2;
}

// The row-vector kernel's reduction split (sets g.chunk and g.splits); returns
// the work items (column blocks x row blocks x splits x batch).
int64_t gemv_split(amx::GemvParams& g, int batch)
{
    const int variant = gemv_variant_of(g.M, g.m, g.n);
    const int cols = amx::gemv_threads(variant) * amx::kGemvColsPerLane;
    const int64_t blocks = cdiv(g.n, cols) * cdiv(g.m, amx::kGemvMaxRows) * batch;
    const int64_t target = kGemvTargetThreads / amx::gemv_threads(variant);
    // as many splits as keep the items within one round of `target`
    // workgroups (a few more items than that would run in a second round)
    int s = (int)std::min<int64_t>(std::max<int64_t>(1, target / blocks), std::max(1, g.k / 8));
    g.chunk = (int)cdiv(g.k, s);
    g.splits = (int)cdiv(g.k, g.chunk);
    return blocks * g.splits;
}

int gemv_run(amx::GemvParams& g, int batch, float* C, int dev, hipStream_t stream, const ScratchSource& src)
{
    const int variant = gemv_variant_of(g.M, g.m, g.n);
    const int64_t items = gemv_split(g, batch);
    g.batch = batch;
    if (items > INT32_MAX) return APPROX_EUNSUPPORTED;
    int64_t slots;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        int64_t& sl = g_gemv_slots[dev][variant];
        if (sl == 0) {
            int cus = 0;
            if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus < 1) cus = 1;
            sl = (int64_t)cus * amx::gemv_blocks_per_cu(variant);
        }
        slots = sl;
    }
    const int grid = (int)std::min<int64_t>(items, slots);
    float* partials = nullptr;
    if (g.splits > 1) {
        char* base = nullptr;
        int rc = scratch_get(src, dev, stream, (size_t)g.splits * batch * g.m * g.n * sizeof(float), &base, nullptr,
                             nullptr);
        if (rc != APPROX_OK) return rc;
        partials = reinterpret_cast<float*>(base);
        g.out = partials;
    } else {
        g.out = C;
    }
    hipEvent_t ev0 = nullptr, ev1 = nullptr;
    bool prof;
    {
        std::lock_guard<std::mutex> lock(g_mu);
        prof = g_profile && src.fixed == nullptr;
    }
    if (prof) {
        if (hipEventCreate(&ev0) != hipSuccess || hipEventCreate(&ev1) != hipSuccess) return APPROX_EHIP;
        if (hipEventRecord(ev0, stream) != hipSuccess) return APPROX_EHIP;
    }
    if (amx::launch_gemv(g, variant, grid, stream) != hipSuccess) return APPROX_EHIP;
    if (prof) {
        if (hipEventRecord(ev1, stream) != hipSuccess) return APPROX_EHIP;
        std::lock_guard<std::mutex> lock(g_mu);
        g_events.emplace_back(ev0, ev1);
    }
    if (g.splits > 1) {
        ReduceParams rp{};
        rp.ws = partials;
        rp.out = C;
        rp.out_ptrs = g.out_ptrs;
        rp.m = g.m;
        rp.n = g.n;
        rp.ldc = g.ldc;
        rp.splits = g.splits;
        rp.batch = batch;
        rp.out_batch = g.out_batch;
        if (amx::launch_reduce(rp, stream) != hipSuccess) return APPROX_EHIP;
    }
    return APPROX_OK;
}

// The GEMM-kernel plan of a call's shapes (no pointers; leading dimensions
// default to the packed ones): decode layouts, tiling, k-step counters and
// the M = 8 copy-choice groups. A function of the arguments only.
void build_gemm_plan(int transA, int transB, int m, int n, int k, int batch, Plan& pl)
{
    pl.batch = batch;
    const int KB = (int)cdiv(k, 4);
    const Tiling tg = tiling_of(m, n, true, KB, batch);
    pl.shape = tg.shape;
    MainParams& mp = pl.mp;
    mp.wr = tg.wr;
    mp.wc = tg.wc;
    mp.tiles_m = tg.tiles_m;
    mp.tiles_n = tg.tiles_n;
    const int Mp = mp.tiles_m * tg.TM, Np = mp.tiles_n * tg.TN;

    DecodeParams& a = pl.lane;
    a.layout = amx::L_DENSE_LANE;
    a.m = m; a.n = n; a.k = k; a.ld = transA ? m : k; a.trans = transA;
    a.Mp = Mp; a.Np = Np; a.KB = KB;
    a.rowlen = Mp * 4;
    a.ldw = amx::panel_ld(Mp * 4);
    pl.lane_count = (int64_t)KB * Mp * 4;
    pl.lane_words = (int64_t)KB * a.ldw;

    DecodeParams& u = pl.uni;
    u.layout = amx::L_DENSE_UNIFORM;
    u.m = m; u.n = n; u.k = k; u.ld = transB ? k : n; u.trans = transB;
    u.Mp = Mp; u.Np = Np; u.KB = KB;
    u.rowlen = Np;
    u.ldw = amx::panel_ld(Np);
    pl.uni_count = (int64_t)KB * 4 * Np;
    pl.uni_words = (int64_t)KB * 4 * u.ldw;

    mp.m_rows = Mp;
    mp.m_out = m;
    mp.n_out = n;
    mp.ldc = n;
    mp.Np = Np;
    mp.bld = u.ldw;
    mp.E2 = 1; mp.E3 = Mp; mp.L1 = 0; mp.L2 = 0; mp.L3 = 4;
    mp.U1 = KB; mp.U2 = 1; mp.U3 = 1; mp.K1 = a.ldw; mp.K2 = 0; mp.K3 = 0;
    mp.KB = KB;
    pl.gather = 0;
    // a half-wave reads rows i0..i0+31 (i0 a multiple of 32) at one index
    pl.asg.G1 = KB; pl.asg.S1 = a.ldw;
    pl.asg.G2 = Mp / 32; pl.asg.S2 = 32 * 4;
    pl.asg.G3 = 4; pl.asg.S3 = 1;
    pl.asg.LS = 4; pl.asg.O = 0; pl.asg.E = Mp;
}

// Argument checks of one GEMM (row-major; pointer arrays: the matrices come
// from device pointer arrays, not A / B / C).
int gemm_check(int transA, int transB, int m, int n, int k, const float* A, int lda, const float* B, int ldb,
               const float* C, int ldc, bool arrays)
{
    if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1)) return APPROX_EINVAL;
    if (m < 0 || n < 0 || k < 0) return APPROX_EINVAL;
    if (lda < std::max(1, transA ? m : k)) return APPROX_EINVAL;
    if (ldb < std::max(1, transB ? k : n)) return APPROX_EINVAL;
    if (ldc < std::max(1, n)) return APPROX_EINVAL;
    if (m == 0 || n == 0) return APPROX_OK;
    if (!arrays && C == nullptr) return APPROX_EINVAL;
    if (!arrays && k > 0 && (A == nullptr || B == nullptr)) return APPROX_EINVAL;
    return APPROX_OK;
}

int gemm_impl(int transA, int transB, int m, int n, int k, const float* A, int lda, long long strideA,
              const float* B, int ldb, long long strideB, float* C, int ldc, long long strideC, int batch,
              void* stream_v, const float* const* Ap = nullptr, const float* const* Bp = nullptr,
              float* const* Cp = nullptr, bool noalloc = false)
{
    const bool arrays = Ap != nullptr || Bp != nullptr || Cp != nullptr;
    if (arrays && (Ap == nullptr || Bp == nullptr || Cp == nullptr)) return APPROX_EINVAL;
    if (strideA < 0 || strideB < 0 || strideC < 0 || batch < 0) return APPROX_EINVAL;
    int rc = gemm_check(transA, transB, m, n, k, A, lda, B, ldb, C, ldc, arrays);
    if (rc != APPROX_OK) return rc;
    if (batch > 65535) return APPROX_EUNSUPPORTED;
    if (m == 0 || n == 0 || batch == 0) return APPROX_OK;

    int dev = 0;
    rc = current_device(&dev);
    if (rc != APPROX_OK) return rc;
    const uint16_t* image = nullptr;
    const uint16_t* flat = nullptr;
    int M = 0;
    rc = table_of(dev, &image, &M, &flat);
    if (rc != APPROX_OK) return rc;
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    ScratchSource src;
    if (noalloc) {
        rc = fixed_scratch(dev, &src.fixed);
        if (rc != APPROX_OK) return rc;
    }

    if (k == 0) {
        return amx::launch_fill_zero(C, Cp, m, n, ldc, batch, strideC, stream) == hipSuccess ? APPROX_OK
                                                                                          : APPROX_EHIP;
    }
    // Few rows: the row-vector kernel, in blocks of 4 rows of op(A) within
    // one launch (the row blocks of one column block and chunk run on one
    // XCD, so B is streamed once into its L2 for all of them).
    if (!transB && row_vector_fits(m, n, k)) {
        amx::GemvParams g{};
        g.A = A; g.A_ptrs = Ap; g.A_batch = strideA;
        g.B = B; g.B_ptrs = Bp; g.B_batch = strideB;
        g.lut = flat;
        g.out_ptrs = Cp; g.out_batch = strideC;
        g.M = M; g.m = m; g.n = n; g.k = k; g.lda = lda; g.ldb = ldb; g.ldc = ldc; g.transA = transA;
        format_range(dev, &g.elo, &g.ehi);
        g.force_checked = force_checked() ? 1 : 0;
        return gemv_run(g, batch, C, dev, stream, src);
    }

    Plan pl;
    build_gemm_plan(transA, transB, m, n, k, batch, pl);
    pl.C = C;
    pl.strideC = strideC;
    pl.Cp = Cp;
    pl.lane.src = A;
    pl.lane.src_ptrs = Ap;
    pl.lane.src_batch_stride = strideA;
    pl.uni.src = B;
    pl.uni.src_ptrs = Bp;
    pl.uni.src_batch_stride = strideB;
    pl.mp.ldc = ldc;
    pl.lane.ld = lda;
    pl.uni.ld = ldb;
    return run_plan(pl, dev, stream, image, M, src);
}

struct ConvShape {
    int N, H, W, C, K, R, S, sh, sw, ph, pw, P, Q;
};

int conv_check(int N, int H, int W, int C, int K, int R, int S, int sh, int sw, int ph, int pw,
               const void* t1, const void* t2, const void* out, ConvShape* cs)
{
    if (N < 1 || H < 1 || W < 1 || C < 1 || K < 1 || R < 1 || S < 1) return APPROX_EINVAL;
    if (sh < 1 || sw < 1 || ph < 0 || pw < 0) return APPROX_EINVAL;
    if (R > H + 2 * ph || S > W + 2 * pw) return APPROX_EINVAL;
    if (t1 == nullptr || t2 == nullptr || out == nullptr) return APPROX_EINVAL;
    *cs = ConvShape{N, H, W, C, K, R, S, sh, sw, ph, pw, (H + 2 * ph - R) / sh + 1, (W + 2 * pw - S) / sw + 1};
    return APPROX_OK;
}

void fill_geom(DecodeParams& d, const ConvShape& s)
{
    d.N = s.N; d.H = s.H; d.W = s.W; d.C = s.C; d.K = s.K; d.R = s.R; d.S = s.S;
    d.sh = s.sh; d.sw = s.sw; d.ph = s.ph; d.pw = s.pw; d.P = s.P; d.Q = s.Q;
}

enum ConvKind { CONV_FWD, CONV_DGRAD, CONV_WGRAD };

// The implicit GEMM of a pass: rows = output pixels (fwd, dgrad) or filter
// taps x input channels (wgrad); columns = the output's channels.
void conv_gemm_extent(ConvKind kind, const ConvShape& s, int* m, int* n)
{
    if (kind == CONV_FWD) { *m = s.N * s.P * s.Q; *n = s.K; }
    else if (kind == CONV_DGRAD) { *m = s.N * s.H * s.W; *n = s.C; }
    else { *m = s.R * s.S * s.C; *n = s.K; }
}

// k-steps (4 reduction positions each) of a pass: the sequences of the
// header's Conv2D order, channels rounded up to a multiple of 4.
int conv_ksteps(ConvKind kind, const ConvShape& s)
{
    if (kind == CONV_FWD) return s.R * s.S * (int)cdiv(s.C, 4);
    if (kind == CONV_DGRAD) return s.R * s.S * (int)cdiv(s.K, 4);
    return (int)cdiv((int64_t)s.N * s.P * s.Q, 4);
}

// The GEMM-kernel plan of a Conv2D pass (no pointers): the implicit-GEMM
// layouts of both operands, tiling, k-step counters and the M = 8
// copy-choice groups. APPROX_EUNSUPPORTED when the image exceeds the word
// limit. A function of the shapes only.
int build_conv_plan(ConvKind kind, const ConvShape& s, Plan& pl)
{
    pl.batch = 1;
    MainParams& mp = pl.mp;
    DecodeParams& a = pl.lane;
    DecodeParams& u = pl.uni;
    fill_geom(a, s);
    fill_geom(u, s);

    int m, n;
    conv_gemm_extent(kind, s, &m, &n);
    // the forward and input-gradient passes run in vector mode: any shape
    const Tiling tg = tiling_of(m, n, kind != CONV_WGRAD, conv_ksteps(kind, s), 1);
    pl.shape = tg.shape;
    mp.wr = tg.wr;
    mp.wc = tg.wc;
    mp.tiles_m = tg.tiles_m;
    mp.tiles_n = tg.tiles_n;
    const int Np = mp.tiles_n * tg.TN;
    mp.m_rows = m;
    mp.m_out = m;
    mp.n_out = n;
    mp.ldc = n;
    mp.Np = Np;
    a.Np = u.Np = Np;
    u.rowlen = Np;
    u.ldw = amx::panel_ld(Np);
    mp.bld = u.ldw;

    if (kind == CONV_FWD) {
        const int Hp = s.H + 2 * s.ph, Wp = s.W + 2 * s.pw, Cb = (int)cdiv(s.C, 4), Cp = Cb * 4;
        a.layout = amx::L_IMG_FWD;
        a.Hp = Hp; a.Wp = Wp; a.Cb = Cb;
        pl.lane_words = (int64_t)s.N * Hp * Cb * Wp * 4;
        u.layout = amx::L_W_FWD;
        u.Cp = Cp;
        mp.KB = conv_ksteps(kind, s);
        pl.uni_count = (int64_t)mp.KB * 4 * Np;
        pl.uni_words = (int64_t)mp.KB * 4 * u.ldw;
        const int rowB = Cb * Wp * 4;                 // one padded image row, in words
        mp.E2 = s.P; mp.E3 = s.Q;
        mp.L1 = Hp * rowB; mp.L2 = s.sh * rowB; mp.L3 = s.sw * 4;
        mp.U1 = s.R; mp.U2 = s.S; mp.U3 = Cb;
        mp.K1 = rowB; mp.K2 = 4; mp.K3 = Wp * 4;
        pl.gather = 0;
        // groups: 32 image columns, sw apart, from the one the centre tap
        // reads for output column 0 (exact when Q = 32, close for the other taps)
        const int w0 = std::min(std::max((s.S - 1) / 2, 0), Wp - 1);
        pl.asg.G1 = s.N * Hp * Cb; pl.asg.S1 = (int64_t)Wp * 4;
        pl.asg.E = (Wp - 1 - w0) / s.sw + 1;
        pl.asg.G2 = (int)cdiv(pl.asg.E, 32); pl.asg.S2 = 32 * s.sw * 4;
        pl.asg.G3 = 4; pl.asg.S3 = 1;
        pl.asg.LS = s.sw * 4; pl.asg.O = w0 * 4;
    } else if (kind == CONV_DGRAD) {
        const int Hd = s.H + s.R - 1, Wd = s.W + s.S - 1, Kb = (int)cdiv(s.K, 4), Kp = Kb * 4;
        a.layout = amx::L_IMG_DGRAD;
        a.Hp = Hd; a.Wp = Wd; a.Kb = Kb;
        pl.lane_words = (int64_t)s.N * Hd * Kb * Wd * 4;
        u.layout = amx::L_W_DGRAD;
        u.Kp = Kp;
        mp.KB = conv_ksteps(kind, s);
        pl.uni_count = (int64_t)mp.KB * 4 * Np;
        pl.uni_words = (int64_t)mp.KB * 4 * u.ldw;
        const int rowB = Kb * Wd * 4;
        mp.E2 = s.H; mp.E3 = s.W;
        mp.L1 = Hd * rowB; mp.L2 = rowB; mp.L3 = 4;
        mp.U1 = s.R; mp.U2 = s.S; mp.U3 = Kb;
        mp.K1 = rowB; mp.K2 = 4; mp.K3 = Wd * 4;
        pl.gather = 0;
        const int w0 = std::min((s.S - 1) / 2, Wd - 1);
        pl.asg.G1 = s.N * Hd * Kb; pl.asg.S1 = (int64_t)Wd * 4;
        pl.asg.E = Wd - w0;
        pl.asg.G2 = (int)cdiv(pl.asg.E, 32); pl.asg.S2 = 32 * 4;
        pl.asg.G3 = 4; pl.asg.S3 = 1;
        pl.asg.LS = 4; pl.asg.O = w0 * 4;
    } else {
        const int Hp = s.H + 2 * s.ph, Wp = s.W + 2 * s.pw;
        const int64_t body = (int64_t)s.N * Hp * s.C * Wp;
        const int64_t npq = (int64_t)s.N * s.P * s.Q;
        if (body + (int64_t)s.R * s.C * Wp >= kMaxPanelWords || npq >= kMaxPanelWords) return APPROX_EUNSUPPORTED;
        a.layout = amx::L_IMG_WGRAD;
        a.Hp = Hp; a.Wp = Wp;
        pl.lane_words = body + (int64_t)s.R * s.C * Wp;
        u.layout = amx::L_DY_WGRAD;
        mp.KB = conv_ksteps(kind, s);
        u.Kp = mp.KB * 4;
        u.KB = mp.KB;
        pl.uni_count = (int64_t)mp.KB * 4 * Np;
        pl.uni_words = (int64_t)mp.KB * 4 * u.ldw;
        // lane row (r, s, c) of the padded NHWC image, reduction index (n, p, q)
        mp.E2 = s.S; mp.E3 = s.C;
        mp.L1 = Wp * s.C; mp.L2 = s.C; mp.L3 = 1;
        mp.U1 = s.N; mp.U2 = s.P; mp.U3 = s.Q;
        mp.K1 = Hp * Wp * s.C; mp.K2 = s.sh * Wp * s.C; mp.K3 = s.sw * s.C;
        mp.nku = (int)npq;
        mp.zoff = (int)body;
        pl.gather = 1;
        // a half-wave reads 32 consecutive channels of one image pixel
        pl.asg.G1 = s.N * Hp * Wp; pl.asg.S1 = s.C;
        pl.asg.E = s.C;
        pl.asg.G2 = (int)cdiv(s.C, 32); pl.asg.S2 = 32;
        pl.asg.G3 = 1; pl.asg.S3 = 0;
        pl.asg.LS = 1; pl.asg.O = 0;
    }
    return APPROX_OK;
}

int conv_impl(ConvKind kind, const ConvShape& s, const float* t1, const float* t2, float* out, void* stream_v)
{
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != APPROX_OK) return rc;
    const uint16_t* image = nullptr;
    int M = 0;
    rc = table_of(dev, &image, &M);
    if (rc != APPROX_OK) return rc;
    hipStream_t stream = static_cast<hipStream_t>(stream_v);

    Plan pl;
    rc = build_conv_plan(kind, s, pl);
    if (rc != APPROX_OK) return rc;
    pl.C = out;
    pl.lane.src = t1;
    pl.uni.src = t2;
    return run_plan(pl, dev, stream, image, M, ScratchSource{});
}

// ---------------------------------------------------------------- plan check
// Host-side bounds check of a planned call (a test hook, not part of the C
// ABI's header): the largest offset each kernel of the plan reads or writes,
// computed with the kernels' own index formulas (row bases, k-step counters,
// the zero region of gather mode, uniform rows and columns, split partials,
// copy-choice groups, table lookups), against what the plan allocates.
enum PlanSlot {
    PS_DECODE_LANE = 0,   // decode writes, lane panel (words)
    PS_DECODE_UNI,        // decode writes, uniform panel (words)
    PS_READ_LANE,         // GEMM-kernel reads, lane panel (words)
    PS_READ_UNI,          // GEMM-kernel reads, uniform panel (words)
    PS_PARTIALS,          // split partials written and summed (floats)
    PS_COPY_GROUPS,       // M = 8 copy choice, lane panel (words)
    PS_TABLE,             // table lookups (bytes of the table image)
    PS_SCRATCH,           // the three scratch parts together (bytes)
    PS_COUNT
};

void check_plan(const Plan& pl, int M, int64_t* need, int64_t* have)
{
    const MainParams& mp = pl.mp;
    for (int i = 0; i < PS_COUNT; ++i) need[i] = have[i] = 0;
    const int64_t lane_total = pl.lane_words * pl.batch, uni_total = pl.uni_words * pl.batch;
    // decode: word o < count of a batch entry goes to row o / rowlen, column
    // o % rowlen of rows ldw apart (every decode variant writes these places)
    auto decode_max = [&](const DecodeParams& d, int64_t batch_words) {
        const int64_t rowlen = d.rowlen > 0 ? d.rowlen : d.count, ldw = d.rowlen > 0 ? d.ldw : d.count;
        const int64_t o = d.count - 1, row = o / rowlen;
        return (pl.batch - 1) * batch_words + row * ldw + (o - row * rowlen) + 1;
    };
    need[PS_DECODE_LANE] = decode_max(pl.lane, pl.lane_words);
    have[PS_DECODE_LANE] = lane_total;
    need[PS_DECODE_UNI] = decode_max(pl.uni, pl.uni_words);
    have[PS_DECODE_UNI] = uni_total;
    // GEMM kernel, lane operand: row base of every row the kernel may read
    // (rows are clamped below m_rows), plus the largest k-step offset
    int64_t max_base = 0;
    for (int i = 0; i < mp.m_rows; ++i) {
        const int i3 = i % mp.E3, r2 = i / mp.E3, i2 = r2 % mp.E2, i1 = r2 / mp.E2;
        max_base = std::max<int64_t>(max_base, (int64_t)i1 * mp.L1 + (int64_t)i2 * mp.L2 + (int64_t)i3 * mp.L3);
    }
    int64_t max_off = 0;
    const int steps = pl.gather ? mp.nku : mp.KB;
    for (int u = 0; u < steps; ++u) {
        const int u3 = u % mp.U3, r = u / mp.U3, u2 = r % mp.U2, u1 = r / mp.U2;
        max_off = std::max<int64_t>(max_off, (int64_t)u1 * mp.K1 + (int64_t)u2 * mp.K2 + (int64_t)u3 * mp.K3);
    }
    if (!pl.gather) max_off += 3;                         // a k-step's 4 contiguous words
    else if ((int64_t)mp.KB * 4 > mp.nku) max_off = std::max<int64_t>(max_off, mp.zoff);   // the zero region
    need[PS_READ_LANE] = (pl.batch - 1) * pl.lane_words + max_base + max_off + 1;
    have[PS_READ_LANE] = lane_total;
    // uniform operand: rows 0 .. KB*4 - 1, a wave's 16 columns from its col0
    const int64_t TN = (int64_t)mp.wc * kColsPerWave;
    need[PS_READ_UNI] = (pl.batch - 1) * pl.uni_words + ((int64_t)mp.KB * 4 - 1) * mp.bld +
                        ((int64_t)mp.tiles_n * TN - kColsPerWave) + kColsPerWave;
    have[PS_READ_UNI] = uni_total;
    // partials: item (b, split, tile) writes ws[(b * splits + split) * m * n + i * n + j]
    if (mp.splits > 1) {
        need[PS_PARTIALS] = ((int64_t)pl.batch * mp.splits - 1) * mp.m_out * mp.n_out +
                            ((int64_t)mp.m_out - 1) * mp.n_out + mp.n_out;
        have[PS_PARTIALS] = (int64_t)(pl.part_b / sizeof(float));
    }
    // M = 8 copy choice: the last word of the last group
    if (M == 8) {
        const amx::AssignParams& a = pl.asg;
        const int count = std::min(32, a.E - (a.G2 - 1) * 32);
        need[PS_COPY_GROUPS] = (int64_t)(pl.batch - 1) * pl.lane_words + (int64_t)(a.G1 - 1) * a.S1 +
                               (int64_t)(a.G2 - 1) * a.S2 + (int64_t)(a.G3 - 1) * a.S3 + a.O +
                               (int64_t)(count - 1) * a.LS + 1;
        have[PS_COPY_GROUPS] = lane_total;
    }
    // table lookups: the last column's offset plus the largest row offset a
    // lane word can hold (the pad, or at M = 8 a second copy), 2 bytes read
    if (M >= 1) {
        const int64_t col = amx::lut_col_bytes(M);
        const int64_t row_max = M == 8 ? amx::kRep8ColBytes - 2 : (int64_t)2 << M;
        need[PS_TABLE] = ((int64_t)(1 << M) - 1) * col + row_max + 2;
        have[PS_TABLE] = amx::lut_image_bytes(M);
    }
    need[PS_SCRATCH] = (int64_t)pl.wbytes * (lane_total + uni_total) + 4 * need[PS_PARTIALS];
    have[PS_SCRATCH] = (int64_t)(pl.lane_b + pl.uni_b + pl.part_b);
}

}  // namespace

// Test hook (host only, no HIP call): the GEMM-kernel plan of a GEMM (kind 0)
// or Conv2D pass (kind 1..3), arguments as amx_plan_check. Writes out[0..11]:
// shape, wr, wc, TM, TN, tiles_m, tiles_n, KB, splits, chunk, full_items,
// tail_tiles; returns the work items (or a negative status).
extern "C" long long amx_plan_info(int kind, const int* args, int M, int* out)
{
    if (args == nullptr || out == nullptr || M < 0 || M > 11) return APPROX_EINVAL;
    Plan pl;
    if (kind == 0) {
        const int tA = args[0], tB = args[1], m = args[2], n = args[3], k = args[4], batch = args[5];
        if (m < 1 || n < 1 || k < 1 || batch < 1 || (tA & ~1) || (tB & ~1)) return APPROX_EINVAL;
        build_gemm_plan(tA, tB, m, n, k, batch, pl);
    } else if (kind >= 1 && kind <= 3) {
        ConvShape cs;
        int rc = conv_check(args[0], args[1], args[2], args[3], args[4], args[5], args[6], args[7], args[8], args[9],
                            args[10], &cs, &cs, &cs, &cs);
        if (rc != APPROX_OK) return rc;
        rc = build_conv_plan(kind == 1 ? CONV_FWD : kind == 2 ? CONV_DGRAD : CONV_WGRAD, cs, pl);
        if (rc != APPROX_OK) return rc;
    } else {
        return APPROX_EINVAL;
    }
    int rc = plan_finalize(pl, M);
    if (rc != APPROX_OK) return rc;
    const MainParams& mp = pl.mp;
    const int v[12] = {pl.shape, mp.wr, mp.wc, mp.wr * 64 * kShapes[pl.shape].rows_per_lane, mp.wc * kColsPerWave,
                       mp.tiles_m, mp.tiles_n, mp.KB, mp.splits, mp.chunk, mp.full_items, mp.tail_tiles};
    for (int i = 0; i < 12; ++i) out[i] = v[i];
    return (long long)mp.items;
}

// Test hook (host only, no HIP call): the rows of B that one group load of
// the row-vector kernel reads, for an item ending at index k1 (exclusive) and
// a group of ng indices starting at kg: writes them to rows[0 .. ng) and
// returns the descriptor's base row (-1 for invalid arguments).
extern "C" int amx_gemv_group_rows(int k1, int kg, int ng, int* rows)
{
    if (rows == nullptr || k1 < 1 || ng < 1 || kg < 0) return -1;
    const int base = amx::gemv_group_base(kg, k1);
    for (int g = 0; g < ng; ++g) rows[g] = base + amx::gemv_group_step(kg, k1, g);
    return base;
}

// Test hook (host only, no HIP call): plans a GEMM (kind 0: args transA,
// transB, m, n, k, batch) or a Conv2D pass (kind 1..3: fwd, dgrad, wgrad;
// args N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w) for a table of
// width M (0: the native multiplier) through the GEMM kernel and writes, per
// PlanSlot, the largest offset + 1 each kernel touches (need) and what the
// plan allocates (have). Returns the number of slots with need > have, or a
// negative status for invalid arguments.
extern "C" int amx_plan_check(int kind, const int* args, int M, long long* need, long long* have)
{
    if (args == nullptr || need == nullptr || have == nullptr || M < 0 || M > 11) return APPROX_EINVAL;
    Plan pl;
    if (kind == 0) {
        const int tA = args[0], tB = args[1], m = args[2], n = args[3], k = args[4], batch = args[5];
        if (m < 1 || n < 1 || k < 1 || batch < 1 || (tA & ~1) || (tB & ~1)) return APPROX_EINVAL;
        build_gemm_plan(tA, tB, m, n, k, batch, pl);
    } else if (kind >= 1 && kind <= 3) {
        ConvShape cs;
        int rc = conv_check(args[0], args[1], args[2], args[3], args[4], args[5], args[6], args[7], args[8], args[9],
                            args[10], &cs, &cs, &cs, &cs);
        if (rc != APPROX_OK) return rc;
        rc = build_conv_plan(kind == 1 ? CONV_FWD : kind == 2 ? CONV_DGRAD : CONV_WGRAD, cs, pl);
        if (rc != APPROX_OK) return rc;
    } else {
        return APPROX_EINVAL;
    }
    int rc = plan_finalize(pl, M);
    if (rc != APPROX_OK) return rc;
    int64_t nd[PS_COUNT], hv[PS_COUNT];
    check_plan(pl, M, nd, hv);
    int bad = 0;
    for (int i = 0; i < PS_COUNT; ++i) {
        need[i] = nd[i];
        have[i] = hv[i];
        bad += nd[i] > hv[i];
    }
    return bad;
}

// ====================================================================== C ABI

extern "C" int approx_lut_load(const uint16_t* lut, int M)
{
    if (lut == nullptr) return APPROX_EINVAL;
    if (M < 1 || M > 11) return APPROX_EUNSUPPORTED;
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != APPROX_OK) return rc;
    // lane-first image: column ib holds entries (ia, ib) for ia = 0..2^M-1 and
    // two zeros (at M = 8 also the second copies of replica.h); then (256-byte
    // aligned) the table in index order for the row-vector kernel
    const int side = 1 << M, cs = amx::lut_col_entries(M);
    const size_t img_entries = (size_t)amx::lut_image_bytes(M) / 2;
    const size_t flat_at = (img_entries + 127) & ~(size_t)127;   // entries
    const size_t entries = (size_t)1 << (2 * M);
    std::vector<uint16_t> img(flat_at + entries + 8, 0);   // + a zero entry (and padding) after the table
    for (int ib = 0; ib < side; ++ib)
        for (int ia = 0; ia < side; ++ia) {
            const uint16_t e = lut[((size_t)ia << M) | ib];
            if (M == 8) {                                  // and the second copy of dwords 0..30
                img[((size_t)ib * cs * 2 + amx::rep8_offset((uint32_t)ia, 0)) / 2] = e;
                if ((ia >> 1) < amx::kRep8Slots) img[((size_t)ib * cs * 2 + amx::rep8_offset((uint32_t)ia, 1)) / 2] = e;
            } else {
                img[(size_t)ib * cs + ia] = e;
            }
        }
    std::memcpy(img.data() + flat_at, lut, entries * sizeof(uint16_t));
    char* fixed = nullptr;
    rc = fixed_scratch(dev, &fixed);
    if (rc != APPROX_OK) return rc;
    uint16_t* d = nullptr;
    if (hipMalloc(&d, img.size() * sizeof(uint16_t)) != hipSuccess) return APPROX_EHIP;
    if (hipMemcpy(d, img.data(), img.size() * sizeof(uint16_t), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(d);
        return APPROX_EHIP;
    }
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_tables[dev].image != nullptr) g_retired.emplace_back(dev, g_tables[dev].image);
    g_tables[dev].image = d;
    g_tables[dev].flat = d + flat_at;
    g_tables[dev].M = M;
    g_tables[dev].native = false;
    return APPROX_OK;
}

extern "C" int approx_native_load(void)
{
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != APPROX_OK) return rc;
    char* fixed = nullptr;
    rc = fixed_scratch(dev, &fixed);
    if (rc != APPROX_OK) return rc;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_tables[dev].image != nullptr) g_retired.emplace_back(dev, g_tables[dev].image);
    g_tables[dev] = DeviceTable{};
    g_tables[dev].native = true;
    return APPROX_OK;
}

extern "C" int approx_exponent_bits_set(int E)
{
    if (E < 1 || E > 8) return APPROX_EUNSUPPORTED;
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != APPROX_OK) return rc;
    std::lock_guard<std::mutex> lock(g_mu);
    g_exp_bits[dev] = E;
    return APPROX_OK;
}

extern "C" int approx_exponent_bits(void)
{
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != APPROX_OK) return rc;
    std::lock_guard<std::mutex> lock(g_mu);
    return g_exp_bits[dev] ? g_exp_bits[dev] : 8;
}

extern "C" int approx_lut_bits(void)
{
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != APPROX_OK) return rc;
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_tables[dev].native) return 0;
    return g_tables[dev].image ? g_tables[dev].M : APPROX_ENOLUT;
}

extern "C" int approx_gemm(int transA, int transB, int m, int n, int k, const float* A, int lda, const float* B,
                           int ldb, float* C, int ldc, void* stream)
{
    return gemm_impl(transA, transB, m, n, k, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, stream);
}

extern "C" int approx_gemm_noalloc(int transA, int transB, int m, int n, int k, const float* A, int lda,
                                   const float* B, int ldb, float* C, int ldc, void* stream)
{
    return gemm_impl(transA, transB, m, n, k, A, lda, 0, B, ldb, 0, C, ldc, 0, 1, stream, nullptr, nullptr, nullptr,
                     true);
}

extern "C" int approx_gemm_grouped(int count, const int* transA, const int* transB, const int* m, const int* n,
                                   const int* k, const float* const* A, const int* lda, const float* const* B,
                                   const int* ldb, float* const* C, const int* ldc, void* stream_v)
{
    if (count < 1 || count > APPROX_MAX_GROUP) return APPROX_EINVAL;
    if (!transA || !transB || !m || !n || !k || !A || !lda || !B || !ldb || !C || !ldc) return APPROX_EINVAL;
    for (int g = 0; g < count; ++g) {         // every member checked before anything is queued
        const int rc = gemm_check(transA[g], transB[g], m[g], n[g], k[g], A[g], lda[g], B[g], ldb[g], C[g], ldc[g],
                                  false);
        if (rc != APPROX_OK) return rc;
    }
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != APPROX_OK) return rc;
    const uint16_t* image = nullptr;
    int M = 0;
    rc = table_of(dev, &image, &M);
    if (rc != APPROX_OK) return rc;
    hipStream_t stream = static_cast<hipStream_t>(stream_v);
    // members that approx_gemm runs in the GEMM kernel share launches when
    // their kernel variant allows it; the others run as approx_gemm would
    Plan plans[APPROX_MAX_GROUP];
    Plan* grouped[APPROX_MAX_GROUP];
    int ng = 0;
    for (int g = 0; g < count; ++g) {
        if (m[g] == 0 || n[g] == 0) continue;
        if (k[g] == 0 || (!transB[g] && row_vector_fits(m[g], n[g], k[g]))) {
            rc = gemm_impl(transA[g], transB[g], m[g], n[g], k[g], A[g], lda[g], 0, B[g], ldb[g], 0, C[g], ldc[g], 0, 1,
                           stream_v);
            if (rc != APPROX_OK) return rc;
            continue;
        }
        Plan& pl = plans[g];
        build_gemm_plan(transA[g], transB[g], m[g], n[g], k[g], 1, pl);
        pl.C = C[g];
        pl.lane.src = A[g];
        pl.uni.src = B[g];
        pl.mp.ldc = ldc[g];
        pl.lane.ld = lda[g];
        pl.uni.ld = ldb[g];
        // one launch holds calls of one shape: the first grouped member's
        if (!amx::main_group_supported(pl.gather, pl.shape) || (ng > 0 && pl.shape != grouped[0]->shape)) {
            rc = run_plan(pl, dev, stream, image, M, ScratchSource{});
            if (rc != APPROX_OK) return rc;
            continue;
        }
        grouped[ng++] = &pl;
    }
    if (ng == 0) return APPROX_OK;
    return run_group(grouped, ng, dev, stream, image, M, ScratchSource{});
}

extern "C" long long approx_gemm_noalloc_max_bytes(void)
{
    return (long long)(kFixedScratchBytes - kStatsBytes);
}

extern "C" int approx_gemm_strided_batched(int transA, int transB, int m, int n, int k, const float* A, int lda,
                                           long long strideA, const float* B, int ldb, long long strideB, float* C,
                                           int ldc, long long strideC, int batch, void* stream)
{
    return gemm_impl(transA, transB, m, n, k, A, lda, strideA, B, ldb, strideB, C, ldc, strideC, batch, stream);
}

extern "C" int approx_gemm_batched(int transA, int transB, int m, int n, int k, const float* const* A, int lda,
                                   const float* const* B, int ldb, float* const* C, int ldc, int batch, void* stream)
{
    if (batch > 0 && (A == nullptr || B == nullptr || C == nullptr)) return APPROX_EINVAL;
    return gemm_impl(transA, transB, m, n, k, nullptr, lda, 0, nullptr, ldb, 0, nullptr, ldc, 0, batch, stream,
                     A, B, C);
}

extern "C" int approx_conv2d_fwd(int N, int H, int W, int C, int K, int R, int S, int stride_h, int stride_w,
                                 int pad_h, int pad_w, const float* x, const float* w, float* y, void* stream)
{
    ConvShape s;
    int rc = conv_check(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, x, w, y, &s);
    if (rc != APPROX_OK) return rc;
    return conv_impl(CONV_FWD, s, x, w, y, stream);
}

extern "C" int approx_conv2d_dgrad(int N, int H, int W, int C, int K, int R, int S, int stride_h, int stride_w,
                                   int pad_h, int pad_w, const float* dy, const float* w, float* dx, void* stream)
{
    ConvShape s;
    int rc = conv_check(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, dy, w, dx, &s);
    if (rc != APPROX_OK) return rc;
    return conv_impl(CONV_DGRAD, s, dy, w, dx, stream);
}

extern "C" int approx_conv2d_wgrad(int N, int H, int W, int C, int K, int R, int S, int stride_h, int stride_w,
                                   int pad_h, int pad_w, const float* x, const float* dy, float* dw, void* stream)
{
    ConvShape s;
    int rc = conv_check(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, x, dy, dw, &s);
    if (rc != APPROX_OK) return rc;
    return conv_impl(CONV_WGRAD, s, x, dy, dw, stream);
}

extern "C" int approx_gemm_chunks(int transA, int transB, int m, int n, int k, int batch, long long count,
                                  const int* b, const int* i, const int* j, long long* chunk)
{
    if ((transA != 0 && transA != 1) || (transB != 0 && transB != 1)) return APPROX_EINVAL;
    if (m < 0 || n < 0 || k < 0 || batch < 0 || count < 0) return APPROX_EINVAL;
    if (count > 0 && (b == nullptr || i == nullptr || j == nullptr || chunk == nullptr)) return APPROX_EINVAL;
    for (long long t = 0; t < count; ++t)
        if (b[t] < 0 || b[t] >= batch || i[t] < 0 || i[t] >= m || j[t] < 0 || j[t] >= n) return APPROX_EINVAL;
    if (count == 0) return APPROX_OK;
    int dev = 0;
    int rc = current_device(&dev);
    if (rc != APPROX_OK) return rc;
    const uint16_t* image = nullptr;
    int M = 0;
    rc = table_of(dev, &image, &M);
    if (rc != APPROX_OK) return rc;
    if (k == 0) {
        for (long long t = 0; t < count; ++t) chunk[t] = 0;
        return APPROX_OK;
    }
    if (!transB && row_vector_fits(m, n, k)) {        // the row-vector kernel: one split for every output
        amx::GemvParams g{};
        g.M = M; g.m = m; g.n = n; g.k = k;
        gemv_split(g, batch);
        for (long long t = 0; t < count; ++t) chunk[t] = g.splits > 1 ? g.chunk : k;
        return APPROX_OK;
    }
    const KernelOrder ord(m, n, (int)cdiv(k, 4), batch, true);
    for (long long t = 0; t < count; ++t) chunk[t] = std::min<int64_t>(ord.chunk(b[t], i[t], j[t]), k);
    return APPROX_OK;
}

extern "C" int approx_conv2d_chunks(int pass, int N, int H, int W, int C, int K, int R, int S, int stride_h,
                                    int stride_w, int pad_h, int pad_w, long long count, const long long* idx,
                                    long long* chunk)
{
    if (pass < APPROX_CONV_FWD || pass > APPROX_CONV_WGRAD || count < 0) return APPROX_EINVAL;
    ConvShape s;
    // the shape checks of the compute calls (the tensor pointers are not used)
    int rc = conv_check(N, H, W, C, K, R, S, stride_h, stride_w, pad_h, pad_w, &s, &s, &s, &s);
    if (rc != APPROX_OK) return rc;
    if (count > 0 && (idx == nullptr || chunk == nullptr)) return APPROX_EINVAL;
    const ConvKind kind = pass == APPROX_CONV_FWD ? CONV_FWD : pass == APPROX_CONV_DGRAD ? CONV_DGRAD : CONV_WGRAD;
    int m, n;
    conv_gemm_extent(kind, s, &m, &n);
    for (long long t = 0; t < count; ++t)
        if (idx[t] < 0 || idx[t] >= (long long)m * n) return APPROX_EINVAL;
    const KernelOrder ord(m, n, conv_ksteps(kind, s), 1, kind != CONV_WGRAD);
    for (long long t = 0; t < count; ++t) chunk[t] = ord.chunk(0, (int)(idx[t] / n), (int)(idx[t] % n));
    return APPROX_OK;
}

extern "C" int approx_profile_enable(int on)
{
    std::lock_guard<std::mutex> lock(g_mu);
    g_profile = on != 0;
    return APPROX_OK;
}

extern "C" int approx_profile_read(int* launches, double* total_ms)
{
    if (launches == nullptr || total_ms == nullptr) return APPROX_EINVAL;
    std::lock_guard<std::mutex> lock(g_mu);
    int rc = APPROX_OK;
    double sum = 0.0;
    for (auto& ev : g_events) {
        float ms = 0.0f;
        if (hipEventSynchronize(ev.second) != hipSuccess || hipEventElapsedTime(&ms, ev.first, ev.second) != hipSuccess)
            rc = APPROX_EHIP;
        sum += ms;
        (void)hipEventDestroy(ev.first);
        (void)hipEventDestroy(ev.second);
    }
    *launches = (int)g_events.size();
    *total_ms = sum;
    g_events.clear();
    return rc;
}

extern "C" const char* approx_status_string(int status)
{
    switch (status) {
    case APPROX_OK: return "ok";
    case APPROX_EINVAL: return "invalid argument";
    case APPROX_ENOLUT: return "no table loaded on this device";
    case APPROX_EUNSUPPORTED: return "unsupported (table size or problem size)";
    case APPROX_EHIP: return "HIP runtime error";
    case APPROX_ESCRATCH: return "the call needs more scratch than the allocation-free entry point's fixed maximum";
    default: return "unknown status";
    }
}

#ifndef APPROX_BUILD_ID
#define APPROX_BUILD_ID "unstamped"
#endif

extern "C" const char* approx_build_id(void)
{
    return APPROX_BUILD_ID;
}

extern "C" int approx_release(void)
{
    std::lock_guard<std::mutex> lock(g_mu);
    int rc = APPROX_OK;
    int saved = -1;
    (void)hipGetDevice(&saved);
    for (auto& kv : g_arenas) {
        if (kv.second.ptr == nullptr) continue;
        if (hipSetDevice(kv.first.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess) rc = APPROX_EHIP;
        if (hipFree(kv.second.ptr) != hipSuccess) rc = APPROX_EHIP;
    }
    g_arenas.clear();
    for (auto& r : g_retired) {
        if (hipSetDevice(r.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess) rc = APPROX_EHIP;
        if (hipFree(r.second) != hipSuccess) rc = APPROX_EHIP;
    }
    g_retired.clear();
    for (int d = 0; d < kMaxDevices; ++d) {
        g_tables[d].native = false;
        if (g_tables[d].image == nullptr) continue;
        if (hipSetDevice(d) != hipSuccess || hipDeviceSynchronize() != hipSuccess) rc = APPROX_EHIP;
        if (hipFree(g_tables[d].image) != hipSuccess) rc = APPROX_EHIP;
        g_tables[d] = DeviceTable{};
    }
    if (saved >= 0) (void)hipSetDevice(saved);
    return rc;
}
