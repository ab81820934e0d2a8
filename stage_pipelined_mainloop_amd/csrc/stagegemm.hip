// C-ABI of the stage-pipelined fp16 TN GEMM: argument validation, the table
// of compiled variants, variant selection and the launch on the caller's
// stream.  The interface is documented in include/stagegemm.h.
#include "stagegemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "gemm_kernel.hpp"
#include "persistent_kernel.hpp"
#include "shortk_kernel.hpp"

// Scratch of the allocation-free split-K entry point: the partial tiles of
// one round of 256 split pieces (256 x 256 x 256 fp32 = 64 MiB), a fixed
// device array that each GPU the library runs on holds until the process
// ends.  Host code never uses this name as an address: the device address is
// looked up per device with hipGetSymbolAddress (scratch_address below).
static __device__ __align__(256) float scratch[256 * 256 * 256];

namespace {

typedef hipError_t (*launch_fn)(int M, int N, int K, float alpha, float beta, const void *A,
                                const void *B, const void *Cm, void *D, hipStream_t stream);

struct Variant {
    sg_config cfg;
    int threads;
    int ring_bytes;
    int lds_bytes;
    int loads;
    const void *kernel;
    launch_fn launch;
};

// The kernel's parameter list; the argument array below must match it.
typedef void (*gemm_kernel_fn)(const _Float16 *, const _Float16 *, const _Float16 *, _Float16 *,
                               int, int, int, float, float);

template <class C>
constexpr gemm_kernel_fn kernel_of()
{
    if constexpr (C::SCHED == 3)
        return &sg::gemm_tn_persistent_kernel<C>;
    else if constexpr (C::SCHED == 4)
        return &sg::gemm_tn_shortk_kernel<C>;
    else
        return &sg::gemm_tn_kernel<C>;
}

// Workgroups of kernel `k` that the device can keep resident at once (CUs x
// workgroups per CU), cached per device; 0 if the runtime cannot tell.  Calls
// from several host threads may fill the cache at once: each writes the same
// value, through an atomic.
int resident_capacity(const void *k, int threads, std::atomic<int> (&cache)[16])
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return 0;
    if (dev >= 0 && dev < 16) {
        const int hit = cache[dev].load(std::memory_order_relaxed);
        if (hit > 0) return hit;
    }
    int cus = 0, per_cu = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, k, threads, 0) != hipSuccess)
        return 0;
    const int cap = cus * per_cu;
    if (dev >= 0 && dev < 16) cache[dev].store(cap, std::memory_order_relaxed);
    return cap;
}

template <class C>
hipError_t launch(int M, int N, int K, float alpha, float beta, const void *A, const void *B,
                  const void *Cm, void *D, hipStream_t stream)
{
    const gemm_kernel_fn kernel = kernel_of<C>();  // fails to compile on drift
    const long long tiles = (long long)((M + C::BM - 1) / C::BM) * ((N + C::BN - 1) / C::BN);
    long long grid = tiles;
    if constexpr (C::SCHED == 3) {
        // one workgroup per resident slot; each loops over its output tiles
        static std::atomic<int> cache[16];
        const int cap = resident_capacity(reinterpret_cast<const void *>(kernel), C::T, cache);
        if (cap <= 0) return hipErrorInvalidConfiguration;
        if (grid > cap) grid = cap;
    }
    const _Float16 *a = static_cast<const _Float16 *>(A);
    const _Float16 *b = static_cast<const _Float16 *>(B);
    const _Float16 *c = static_cast<const _Float16 *>(Cm);
    _Float16 *d = static_cast<_Float16 *>(D);
    void *args[] = {&a, &b, &c, &d, &M, &N, &K, &alpha, &beta};
    static_assert(sizeof(args) / sizeof(args[0]) == 9, "one entry per kernel parameter");
    return hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)grid),
                           dim3(C::T), args, 0, stream);
}

template <class C>
constexpr Variant variant()
{
    return Variant{{C::BM, C::BN, C::BK, C::S, C::NW, C::SCHED}, C::T, C::RING_BYTES, C::LDS_BYTES,
                   C::L,
                   reinterpret_cast<const void *>(kernel_of<C>()), &launch<C>};
}

// Compiled variants.  256x256 tiles carry the large square shapes (half the
// global->LDS traffic of 128x128 per flop); 128x128 tiles fill the chip for
// M = N = 2048 (one workgroup per CU).  Stage counts 2..5 for the sweep.
const Variant kVariants[] = {
    // ping-pong wave groups (schedule 2)
    variant<sg::Cfg<256, 256, 64, 2, 2, 4, 2>>(),
    // cute-page order (schedule 1)
    variant<sg::Cfg<256, 256, 32, 2, 2, 4, 1>>(),
    variant<sg::Cfg<256, 256, 32, 3, 2, 4, 1>>(),
    variant<sg::Cfg<256, 256, 32, 4, 2, 4, 1>>(),
    variant<sg::Cfg<256, 256, 32, 5, 2, 4, 1>>(),
    variant<sg::Cfg<256, 256, 64, 2, 2, 4, 1>>(),
    variant<sg::Cfg<256, 256, 32, 4, 2, 2, 1>>(),
    variant<sg::Cfg<256, 256, 64, 2, 2, 2, 1>>(),
    variant<sg::Cfg<128, 128, 32, 2, 2, 2, 1>>(),
    variant<sg::Cfg<128, 128, 32, 3, 2, 2, 1>>(),
    variant<sg::Cfg<128, 128, 32, 4, 2, 2, 1>>(),
    variant<sg::Cfg<128, 128, 32, 5, 2, 2, 1>>(),
    variant<sg::Cfg<128, 128, 64, 2, 2, 2, 1>>(),
    variant<sg::Cfg<128, 128, 64, 3, 2, 2, 1>>(),
    // lesson's three-phase order (schedule 0)
    variant<sg::Cfg<256, 256, 32, 2, 2, 4, 0>>(),
    variant<sg::Cfg<256, 256, 32, 3, 2, 4, 0>>(),
    variant<sg::Cfg<256, 256, 32, 4, 2, 4, 0>>(),
    variant<sg::Cfg<256, 256, 32, 5, 2, 4, 0>>(),
    variant<sg::Cfg<256, 256, 64, 2, 2, 4, 0>>(),
    variant<sg::Cfg<128, 128, 32, 2, 2, 2, 0>>(),
    variant<sg::Cfg<128, 128, 32, 3, 2, 2, 0>>(),
    variant<sg::Cfg<128, 128, 32, 4, 2, 2, 0>>(),
    variant<sg::Cfg<128, 128, 32, 5, 2, 2, 0>>(),
    // cute-page order on 16x16x32 MFMAs (schedule 5)
    variant<sg::Cfg<256, 256, 64, 2, 2, 4, 5>>(),
    // ping-pong wave groups on 16x16x32 MFMAs (schedule 7), and with the
    // loads split between the groups (schedule 8: A ring of 2, B ring of 3)
    variant<sg::Cfg<256, 256, 64, 2, 2, 4, 7>>(),
    variant<sg::Cfg<256, 256, 64, 3, 2, 4, 8>>(),
    // one wave per SIMD, 128x128 each, the mainloop as scheduled assembly
    // (schedule 10: two 64 KiB slots)
    variant<sg::Cfg<256, 256, 64, 2, 2, 2, 10>>(),
    // (schedule 11: A in two slots, B in three, 160 KiB)
    variant<sg::Cfg<256, 256, 64, 3, 2, 2, 11>>(),
    // (schedule 12: as 11, the B loads in the first half of each tile)
    variant<sg::Cfg<256, 256, 64, 3, 2, 2, 12>>(),
    // (schedule 14: the same on 128x128 tiles, four 32 KiB slots)
    variant<sg::Cfg<128, 128, 64, 4, 2, 2, 14>>(),
    // whole K extent in the ring, epilogue per row block (schedule 4, K <= S * BK)
    variant<sg::Cfg<128, 128, 64, 2, 2, 2, 4>>(),
    // persistent workgroups, one ring across output tiles (schedule 3)
    variant<sg::Cfg<256, 256, 64, 2, 2, 4, 3>>(),
    variant<sg::Cfg<128, 128, 64, 2, 2, 2, 3>>(),
    variant<sg::Cfg<128, 128, 32, 2, 2, 2, 3>>(),
    variant<sg::Cfg<128, 128, 32, 3, 2, 2, 3>>(),
};
constexpr int kNumVariants = sizeof(kVariants) / sizeof(kVariants[0]);

const Variant *find_variant(const sg_config *c)
{
    for (int i = 0; i < kNumVariants; ++i) {
        const sg_config &v = kVariants[i].cfg;
        if (v.tile_m == c->tile_m && v.tile_n == c->tile_n && v.tile_k == c->tile_k &&
            v.stages == c->stages && v.waves == c->waves && v.schedule == c->schedule)
            return &kVariants[i];
    }
    return nullptr;
}

// Choice from the measured sweeps (MI355X, fp16 uniform[-1,1] inputs).
// First, K <= 128 with at least one wave of 128x128 workgroups and no C
// operand: where A and B fit in one XCD's L2 (4 MiB), the short-K schedule,
// whose row-block epilogue overlaps the write of D with the MFMAs; else the
// persistent 128x128 schedule, which streams a workgroup's tiles through
// one ring.  HIP-graph replays, short-K / persistent: 4096 x 4096 x 128 9.4
// / 9.8 us, x 64 8.0 / 9.1, 8192 x 4096 x 128 17.3 / 18.5, 2048 x 2048 x 128
// 3.9 / 4.5; 81920 x 256 x 128 12.6 / 11.6, 40960 x 512 x 128 12.5 / 11.7,
// 20480 x 1024 x 128 12.4 / 11.9 (8192 x 8192 x 64 and 16384 x 4096 x 64
// within 1.5 %).  Otherwise the cheapest of these, in units of
// one full round of 256 workgroups of the 256x256 kernel:
//   256x256x64, schedule 10 or 12 (one per CU)       1.00 per round of 256
//   128x128x64 S2, schedule 1 (two per CU)           0.66 per round of 512
//   128x128x64, one per CU: schedule 14 for a single round with K >= 1024
//     and rows on 128-byte lines, else S3 schedule 1  0.34 or 0.42 per round of 256
//   128x128x64 S2 persistent (K <= 1024, no C)       0.9 x the S2 figure
// A partial round costs 0.75 + 0.25 x its fill: its workgroups still run
// the whole K loop, only with less contention.  Each per-round figure is the
// family's flops per round relative to a 256x256 round over its MFMA busy
// relative to the 256x256 kernel's (about 0.90): 0.34 = 0.25 x 0.90 / 0.66,
// 0.66 being schedule 14's busy at M = N = 2048, K = 8192, where the
// LDS-DMA rate of about 45 bytes per cycle per CU caps a 128x128x64 tile at
// 0.71 (64 bytes per cycle needed at the full MFMA rate).  Fitted to interleaved
// timings at K = 4096 (2560^2 ... 6144^2, 16384 x 1024, 81920 x 256) and
// 8192 (2048^2, 2560^2); it picks the faster family at every one of them,
// and at K = 1024 and 512 it is within 2 % of the best choice.  The
// persistent factor comes from the tall shape 81920 x 256 x 256 (21.3 us
// against 23.7 tiled and 25.1 for 256x256 tiles).
// Within the 256x256 family, one wave per SIMD: schedule 10 when every row
// of A and B starts on a 128-byte line (K % 64 == 0 and 128-byte aligned
// operands), else schedule 12.  Schedule 10 was 1-4 % faster than the
// two-group ping-pong (schedule 8) at 8192^3, 4096^3, 12288^2 x 4096,
// 6144^2 x 4096, 5120^2 x 8192, 8000^2 x 8192 and 16384 x 1024 x 4096, and
// about 0.5 % faster than schedule 12 there.  Where rows straddle lines
// (K = 8200, 4104) a 16-byte load of a row slice touches two lines and the
// LDS-DMA issue holds the wave longer; schedule 12, which issues half as
// many loads in each half tile, was 2-3 % faster than schedule 8 there and
// schedule 10 1-4 % slower than schedule 8.

// Whether A and B start on 128-byte lines (with K % 64 == 0, every row does).
bool lines_aligned(const void *A, const void *B)
{
    return ((reinterpret_cast<uintptr_t>(A) | reinterpret_cast<uintptr_t>(B)) & 127) == 0;
}

// Whether the 256x256 grid reuses its panels so little that the operands
// stream from HBM: at most two tile rows or two tile columns, so each panel
// of the other operand is read by at most two tiles.  There schedule 12,
// which issues half as many loads in each half tile, beat schedule 10:
// 81920 x 256 x 4096 200.3 against 236.0 us, 65536 x 256 x 2048 56.6
// against 61.1, 32768 x 512 x 8192 215.2 against 221.6 (20480 x 512 x 4096
// equal).  A mirrored form with A in the third slot measured the same as
// schedule 12: the spread of the loads is what counts.
bool streams_from_hbm(int M, int N)
{
    return (M + 255) / 256 <= 2 || (N + 255) / 256 <= 2;
}

double rounds(long long tiles, long long per_round)
{
    const long long full = tiles / per_round;
    const long long rest = tiles % per_round;
    return (double)full + (rest ? 0.75 + 0.25 * (double)rest / (double)per_round : 0.0);
}

// Compute units of the current device, cached per device; 256 (MI355X)
// when the runtime cannot tell, so host-only queries keep one answer.
int device_cus()
{
    static std::atomic<int> cache[16];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return 256;
    int c = cache[dev].load(std::memory_order_relaxed);
    if (c > 0) return c;
    if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
        return 256;
    cache[dev].store(c, std::memory_order_relaxed);
    return c;
}

// The library's choice and its cost in rounds of the 256x256 kernel (0 for
// the short-K schedule, which the split form never competes with).  A round
// is `cus` workgroups of the one-per-CU families and 2 x cus of the
// two-per-CU one; the costs per round were measured on MI355X (256 CUs).
const Variant *select_variant(int M, int N, int K, bool with_c, double *cost = nullptr,
                              bool lines_aligned = true, int cus = 256)
{
    const long long t256 = (long long)((M + 255) / 256) * ((N + 255) / 256);
    const long long t128 = (long long)((M + 127) / 128) * ((N + 127) / 128);
    sg_config c;
    double best = 0.0;
    if (K <= 128 && t128 >= cus && !with_c) {
        // short-K where A and B fit in one XCD's L2, else persistent
        const bool fits = ((long long)M + N) * K * 2 <= (4ll << 20);
        c = fits ? sg_config{128, 128, 64, 2, 4, 4} : sg_config{128, 128, 64, 2, 4, 3};
    } else {
        const double c256 = rounds(t256, cus);
        const double c2 = 0.66 * rounds(t128, 2 * cus);
        // schedule 14 (one wave per SIMD, four slots) against schedule 1 S3,
        // interleaved at M = N = 2048: K = 2048 20.1 / 22.2 us, 8192 61.8 /
        // 75.1, 16384 119.3 / 145.8, 1024 10.7 / 11.9 (S2), but 8.5 / 7.6
        // at K = 512 (a longer prologue) and slower on rows that straddle
        // lines.  Over several rounds its tiles lose their L2 reuse: 4352^2
        // x 4096 189.6 against 159.4 us for 256x256 tiles (schedule 10).
        const bool c3_one_wave = lines_aligned && K % 64 == 0 && K >= 1024 && t128 <= cus;
        const double c3 = (c3_one_wave ? 0.34 : 0.42) * rounds(t128, cus);
        const bool persistent = K <= 1024 && !with_c && t128 > cus;
        const double cp = persistent ? 0.9 * c2 : 1e300;
        c = (lines_aligned && K % 64 == 0 && !streams_from_hbm(M, N)) ? sg_config{256, 256, 64, 2, 4, 10}
                                                                       : sg_config{256, 256, 64, 3, 4, 12};
        best = c256;
        if (c3 < best) {
            best = c3;
            c = c3_one_wave ? sg_config{128, 128, 64, 4, 4, 14} : sg_config{128, 128, 64, 3, 4, 1};
        }
        if (c2 < best) { best = c2; c = sg_config{128, 128, 64, 2, 4, 1}; }
        if (cp < best) { best = cp; c = sg_config{128, 128, 64, 2, 4, 3}; }
    }
    if (cost) *cost = best;
    return find_variant(&c);
}

// ---- remainder form of a plain call (adaptive tile size).  A grid of more
// than one round of 256x256 tiles whose last round is at most a quarter
// full runs its whole rounds as 256x256 tiles (schedule 10,
// gemm_tn_dp_kernel) and each remaining tile as four 128x128 quarters
// (schedule 14, gemm_tn_sub_kernel): one round of at most `capacity`
// quarters instead of a round of few 256x256 workgroups.  Only where
// schedule 14 runs well: rows on 128-byte lines and K >= 1024.  Estimated
// like a single-round schedule-14 grid (0.34 of a 256x256 round); measured
// in the comments of plain_rounds below.
using SubCfg = sg::Cfg<128, 128, 64, 4, 2, 2, 14>;
using DpCfg = sg::Cfg<256, 256, 64, 2, 2, 2, 10>;
using DpCfg12 = sg::Cfg<256, 256, 64, 3, 2, 2, 12>;   // the whole rounds of a streaming grid

struct SubPlan {
    int dp = 0;          // 256x256 tiles in whole rounds
    int quarters = 0;    // 128x128 quarters of the rest (0: no remainder form)
};

SubPlan plan_sub(int M, int N, int K, bool lines_aligned, int capacity)
{
    SubPlan p;
    const long long t256 = (long long)((M + 255) / 256) * ((N + 255) / 256);
    if (!lines_aligned || K % 64 != 0 || K < 1024 || capacity <= 0 || t256 <= capacity) return p;
    const long long left = t256 % capacity;
    if (left == 0 || 4 * left > capacity) return p;
    p.dp = (int)(t256 - left);
    p.quarters = (int)(4 * left);
    return p;
}

// Cost of the plain call in rounds of the 256x256 kernel, with the
// remainder form where it applies and the 256x256 family is chosen.
double plain_rounds(int M, int N, int K, bool with_c, bool lines_aligned, int capacity,
                    const Variant **chosen = nullptr, SubPlan *sub = nullptr)
{
    double cost = 0.0;
    const Variant *v = select_variant(M, N, K, with_c, &cost, lines_aligned,
                                      capacity > 0 ? capacity : 256);
    if (chosen) *chosen = v;
    if (!v || v->cfg.tile_m != 256) return cost;
    const SubPlan p = plan_sub(M, N, K, lines_aligned, capacity);
    if (p.quarters == 0) return cost;
    const double sub_cost = (double)p.dp / capacity + 0.34 * rounds(p.quarters, capacity);
    if (sub_cost >= cost) return cost;
    if (sub) *sub = p;
    return sub_cost;
}

// Largest M: tile counts (M + tile_m - 1) / tile_m stay within int.
constexpr int kMaxM = 0x7fffffff - 256;

// ---- split-K form of schedules 8 and 10 (gemm_fp16_tn_splitk).  Output
// tiles that fill whole rounds of resident workgroups run as in the tiled
// kernel; the rest -- every tile when there are fewer than one round -- are
// cut along K into `splits` runs computed by separate workgroups, whose fp32
// partials a second kernel adds up (sg::SplitWork, sg::split_reduce_kernel).
// The mainloop follows the tiled choice: schedule 10 when every row starts
// on a 128-byte line, else schedule 12.  The plan is made for the schedule-12
// kernel (SplitCfg, whose resident count the runtime reports: one per CU);
// the schedule-10 kernel has the same tiles, threads and residency.
using SplitCfg = sg::Cfg<256, 256, 64, 3, 2, 2, 12>;
using SplitCfg10 = sg::Cfg<256, 256, 64, 2, 2, 2, 10>;
static_assert(SplitCfg10::BM == SplitCfg::BM && SplitCfg10::BN == SplitCfg::BN &&
                  SplitCfg10::BK == SplitCfg::BK && SplitCfg10::T == SplitCfg::T,
              "one split plan serves both split kernels");
static_assert(2 * SplitCfg10::LDS_BYTES > 160 * 1024 && 2 * SplitCfg::LDS_BYTES > 160 * 1024,
              "one split workgroup per CU for both split kernels");
constexpr size_t kSplitTileBytes = (size_t)SplitCfg::BM * SplitCfg::BN * 4;
constexpr int kMaxSplits = 16;

struct SplitPlan {
    int tiles = 0;       // output tiles
    int dp_tiles = 0;    // computed whole
    int left = 0;        // cut along K
    int splits = 1;      // runs per cut tile (1: nothing is split)
    long long grid = 0;
    size_t bytes = 0;        // workspace: the partial tiles (0 when nothing is split)
};

// Resident workgroups of the split kernel on the current device (one per
// CU), cached per device; 0 if the runtime cannot tell.
int split_capacity()
{
    static std::atomic<int> cache[16];
    return resident_capacity(reinterpret_cast<const void *>(&sg::gemm_tn_split_kernel<SplitCfg>),
                             SplitCfg::T, cache);
}

SplitPlan plan_split(int M, int N, int K, int splits, int capacity)
{
    SplitPlan p;
    p.tiles = ((M + SplitCfg::BM - 1) / SplitCfg::BM) * ((N + SplitCfg::BN - 1) / SplitCfg::BN);
    const int ntile = (K + SplitCfg::BK - 1) / SplitCfg::BK;
    int s = splits < ntile ? splits : ntile;       // every run holds at least one K tile
    if (s > kMaxSplits) s = kMaxSplits;
    const int left = p.tiles >= capacity ? p.tiles % capacity : p.tiles;
    if (s <= 1 || left == 0 || capacity <= 0) {
        p.dp_tiles = p.tiles;
        p.grid = p.tiles;
        return p;
    }
    p.left = left;
    p.dp_tiles = p.tiles - left;
    p.splits = s;
    p.grid = (long long)p.dp_tiles + (long long)left * s;
    p.bytes = (size_t)left * s * kSplitTileBytes;
    return p;
}

// The split count the library uses (1: none), from a time model in
// microseconds fitted to interleaved timings of both forms on MI355X:
//   * a round of `capacity` 256x256 workgroups takes 1.55 us per 64-deep K
//     tile plus 3 us (prologue, epilogue and launch): 4096^3, 64 K tiles,
//     measures about 99 us;
//   * the plain call costs select_variant's rounds times that round time;
//   * the split call costs its whole-tile rounds, then ceil(pieces /
//     capacity) rounds of ceil(ntile / s) K tiles, then the reduction: about
//     2 us plus the partial tiles (L * s * 256 KiB) written and read back at
//     about 4.6 MB per us.
// Measured against it (us, plain / best split): 2048^2 x 16384 141.6 / 115.8
// (s = 4), 2048^2 x 8192 73.8 / 71.4, 4352^2 x 4096 164.3 / 134.9,
// 6144^2 x 4096 259.6 / 243.4, 1024^2 x 8192 55.4 / 34.6; plain stays
// faster at 2048^2 x 2048 (21.0 / 35.5), 2560^2 x 4096, 3072^2 x 4096,
// 4096 x 2048 x 4096 and 81920 x 256 x 256, where the model keeps it.
int choose_splits(int M, int N, int K, int capacity)
{
    const SplitPlan whole = plan_split(M, N, K, 1, capacity);
    const int left = whole.tiles >= capacity ? whole.tiles % capacity : whole.tiles;
    const int ntile = (K + SplitCfg::BK - 1) / SplitCfg::BK;
    if (left == 0 || ntile < 2 || capacity <= 0) return 1;
    const double k_tile_us = 1.55, round_us = 3.0, reduce_us = 2.0, partial_mb_per_us = 4.6;
    const double full_round = ntile * k_tile_us + round_us;
    // the plain call as the library would run it (remainder form included),
    // for 128-byte aligned operands
    const double plain_cost = plain_rounds(M, N, K, false, true, capacity);
    if (plain_cost <= 0.0) return 1;                   // short K: never split
    const double plain = plain_cost * full_round;
    const double dp = (double)(whole.tiles / capacity) * full_round;   // whole-tile rounds
    int best_s = 1;
    double best = plain;
    for (int s = 2; s <= kMaxSplits && s <= ntile; ++s) {
        const long long pieces = (long long)left * s;
        const double piece_rounds = (double)((pieces + capacity - 1) / capacity);
        const double run = ((ntile + s - 1) / s) * k_tile_us + round_us;
        const double mb = (double)pieces * (double)kSplitTileBytes / 1e6;
        const double t = dp + piece_rounds * run + reduce_us + mb / partial_mb_per_us;
        if (t < best) {
            best = t;
            best_s = s;
        }
    }
    return best_s;
}

bool overlaps(const void *p, size_t pbytes, const void *q, size_t qbytes)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uintptr_t b = reinterpret_cast<uintptr_t>(q);
    return pbytes && qbytes && a < b + qbytes && b < a + pbytes;
}

// Every check that does not need the runtime.  SG_OK means "launch".
sg_status validate(int M, int N, int K, const void *A, const void *B, const void *D)
{
    if (M < 0 || N < 0 || K < 0) return SG_ERR_SHAPE;
    if (M == 0 || N == 0) return SG_OK;
    if (!D) return SG_ERR_NULL;
    if (K > 0 && (!A || !B)) return SG_ERR_NULL;
    if (K > (1 << 21) || N > (1 << 21)) return SG_ERR_SHAPE;
    // tile counts and tile origins are computed in int: (M + 255) / 256
    // must not overflow
    if (M > kMaxM) return SG_ERR_SHAPE;
    const long long lim = 1LL << 40;
    if ((long long)M * K >= lim || (long long)M * N >= lim) return SG_ERR_SHAPE;
    if ((K & 7) || (N & 7)) return SG_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(D) & 15) ||
        (K > 0 && ((reinterpret_cast<uintptr_t>(A) & 15) || (reinterpret_cast<uintptr_t>(B) & 15))))
        return SG_ERR_ALIGN;
    const size_t dbytes = (size_t)M * N * 2;
    if (K > 0 && (overlaps(D, dbytes, A, (size_t)M * K * 2) ||
                  overlaps(D, dbytes, B, (size_t)N * K * 2)))
        return SG_ERR_ALIAS;
    return SG_OK;
}

// C operand of the beta variant: beta == 0 reads nothing; otherwise C must be
// 16-byte aligned and either be D itself (in place) or not overlap D.
sg_status validate_c(int M, int N, float beta, const void *Cm, const void *D)
{
    if (beta == 0.0f || M == 0 || N == 0) return SG_OK;
    if (!Cm) return SG_ERR_NULL;
    if (reinterpret_cast<uintptr_t>(Cm) & 15) return SG_ERR_ALIGN;
    const size_t bytes = (size_t)M * N * 2;
    if (Cm != D && overlaps(Cm, bytes, D, bytes)) return SG_ERR_ALIAS;
    return SG_OK;
}

sg_status run(const Variant *v, int M, int N, int K, float alpha, float beta, const void *A,
              const void *B, const void *Cm, void *D, void *stream)
{
    const long long tiles = (long long)((M + v->cfg.tile_m - 1) / v->cfg.tile_m) *
                            ((N + v->cfg.tile_n - 1) / v->cfg.tile_n);
    if (tiles * v->threads >= (1LL << 32)) return SG_ERR_SHAPE;
    // the persistent and short-K kernels have no C operand; the short-K
    // kernel holds the whole K extent in its ring
    if ((v->cfg.schedule == 3 || v->cfg.schedule == 4) && beta != 0.0f) return SG_ERR_UNSUPPORTED;
    if (v->cfg.schedule == 4 && (long long)(K + v->cfg.tile_k - 1) / v->cfg.tile_k > v->cfg.stages)
        return SG_ERR_UNSUPPORTED;
    const hipError_t e = v->launch(M, N, K, alpha, beta, A, B, beta == 0.0f ? nullptr : Cm, D,
                                   static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SG_OK : SG_ERR_HIP;
}

// Resident 256x256 workgroups of the remainder form's first kernel on the
// current device (one per CU), cached per device; 0 if the runtime cannot
// tell.
int sub_capacity()
{
    static std::atomic<int> cache[16];
    return resident_capacity(reinterpret_cast<const void *>(&sg::gemm_tn_dp_kernel<DpCfg>),
                             DpCfg::T, cache);
}

// The remainder form: the whole rounds, then the quarters of the rest.
sg_status launch_sub(const SubPlan &p, int M, int N, int K, float alpha, float beta,
                     const void *A, const void *B, const void *Cm, void *D, void *stream)
{
    const _Float16 *a = static_cast<const _Float16 *>(A);
    const _Float16 *b = static_cast<const _Float16 *>(B);
    const _Float16 *c = beta == 0.0f ? nullptr : static_cast<const _Float16 *>(Cm);
    _Float16 *d = static_cast<_Float16 *>(D);
    int dp = p.dp;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    void *args[] = {&a, &b, &c, &d, &M, &N, &K, &alpha, &beta, &dp};
    static_assert(DpCfg12::T == DpCfg::T, "one block size for the whole rounds");
    const void *dpk = streams_from_hbm(M, N)
                          ? reinterpret_cast<const void *>(&sg::gemm_tn_dp_kernel<DpCfg12>)
                          : reinterpret_cast<const void *>(&sg::gemm_tn_dp_kernel<DpCfg>);
    hipError_t e = hipLaunchKernel(dpk, dim3((unsigned)p.dp), dim3(DpCfg::T), args, 0, st);
    if (e != hipSuccess) return SG_ERR_HIP;
    e = hipLaunchKernel(reinterpret_cast<const void *>(&sg::gemm_tn_sub_kernel<SubCfg>),
                        dim3((unsigned)p.quarters), dim3(SubCfg::T), args, 0, st);
    return e == hipSuccess ? SG_OK : SG_ERR_HIP;
}

// The plain call: the chosen variant, or the remainder form where the plan
// takes it (the plan needs the device's resident count; without it, the
// chosen variant).
sg_status run_plain(int M, int N, int K, float alpha, float beta, const void *A, const void *B,
                    const void *Cm, void *D, void *stream)
{
    const bool lines = lines_aligned(A, B);
    const Variant *v = nullptr;
    SubPlan sub;
    // rounds of the device's CUs; the remainder form's resident count is a
    // cached runtime query, made only where that form can apply
    const int cap = lines && K % 64 == 0 && K >= 1024 && (M > 256 || N > 256) ? sub_capacity() : 0;
    plain_rounds(M, N, K, beta != 0.0f, lines, cap > 0 ? cap : device_cus(), &v, &sub);
    if (!v) return SG_ERR_UNSUPPORTED;
    if (sub.quarters > 0) return launch_sub(sub, M, N, K, alpha, beta, A, B, Cm, D, stream);
    return run(v, M, N, K, alpha, beta, A, B, Cm, D, stream);
}

sg_status launch_split(const SplitPlan &p, int M, int N, int K, float alpha, const void *A,
                       const void *B, void *D, void *workspace, void *stream)
{
    const _Float16 *a = static_cast<const _Float16 *>(A);
    const _Float16 *b = static_cast<const _Float16 *>(B);
    _Float16 *d = static_cast<_Float16 *>(D);
    float *part = static_cast<float *>(workspace);
    int dp = p.dp_tiles, splits = p.splits;
    const hipStream_t st = static_cast<hipStream_t>(stream);
    void *args[] = {&a, &b, &d, &M, &N, &K, &alpha, &part, &dp, &splits};
    const bool lines = K % 64 == 0 && lines_aligned(A, B) && !streams_from_hbm(M, N);
    const void *fn = lines ? reinterpret_cast<const void *>(&sg::gemm_tn_split_kernel<SplitCfg10>)
                           : reinterpret_cast<const void *>(&sg::gemm_tn_split_kernel<SplitCfg>);
    hipError_t e = hipLaunchKernel(fn, dim3((unsigned)p.grid), dim3(SplitCfg::T), args, 0, st);
    if (e != hipSuccess) return SG_ERR_HIP;
    const float *cpart = part;
    void *rargs[] = {&cpart, &d, &M, &N, &alpha, &dp, &splits};
    constexpr int per_tile = SplitCfg::BM * SplitCfg::BN / (256 * 8);
    e = hipLaunchKernel(
        reinterpret_cast<const void *>(&sg::split_reduce_kernel<SplitCfg::BM, SplitCfg::BN>),
        dim3((unsigned)(p.left * per_tile)), dim3(256), rargs, 0, st);
    return e == hipSuccess ? SG_OK : SG_ERR_HIP;
}

// Device address of `scratch` on the current device, looked up once per
// device (the array has its own address on every GPU); nullptr if the
// runtime cannot tell.  Threads may race to fill the cache: each stores the
// same value.
void *scratch_address()
{
    static std::atomic<void *> cache[16];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 16) return nullptr;
    void *p = cache[dev].load(std::memory_order_acquire);
    if (p) return p;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return nullptr;
    cache[dev].store(p, std::memory_order_release);
    return p;
}

}  // namespace

extern "C" {

sg_status gemm_fp16_tn_alpha(int M, int N, int K, float alpha, const void *A, const void *B,
                             void *D, void *stream)
{
    const sg_status st = validate(M, N, K, A, B, D);
    if (st != SG_OK || M == 0 || N == 0) return st;
    return run_plain(M, N, K, alpha, 0.0f, A, B, nullptr, D, stream);
}

sg_status gemm_fp16_tn_alpha_beta(int M, int N, int K, float alpha, float beta, const void *A,
                                  const void *B, const void *Cm, void *D, void *stream)
{
    sg_status st = validate(M, N, K, A, B, D);
    if (st != SG_OK) return st;
    st = validate_c(M, N, beta, Cm, D);
    if (st != SG_OK || M == 0 || N == 0) return st;
    return run_plain(M, N, K, alpha, beta, A, B, Cm, D, stream);
}

sg_status gemm_fp16_tn(int M, int N, int K, const void *A, const void *B, void *D, void *stream)
{
    return gemm_fp16_tn_alpha(M, N, K, 1.0f, A, B, D, stream);
}

sg_status gemm_fp16_tn_cfg(int M, int N, int K, float alpha, const void *A, const void *B,
                           void *D, const sg_config *cfg, void *stream)
{
    if (!cfg) return SG_ERR_NULL;
    const sg_status st = validate(M, N, K, A, B, D);
    if (st != SG_OK) return st;
    const Variant *v = find_variant(cfg);
    if (!v) return SG_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return SG_OK;
    return run(v, M, N, K, alpha, 0.0f, A, B, nullptr, D, stream);
}

sg_status sg_split_plan(int M, int N, int K, int splits, int capacity, sg_split_info *out)
{
    if (!out) return SG_ERR_NULL;
    if (M <= 0 || N <= 0 || K <= 0 || splits < 1 || capacity < 1 || M > kMaxM || K > (1 << 21) ||
        N > (1 << 21))
        return SG_ERR_SHAPE;
    const SplitPlan p = plan_split(M, N, K, splits, capacity);
    out->tiles = p.tiles;
    out->whole_tiles = p.dp_tiles;
    out->cut_tiles = p.left;
    out->splits = p.splits;
    out->workgroups = p.grid;
    out->workspace_bytes = p.bytes;
    out->chosen_splits = choose_splits(M, N, K, capacity);
    return SG_OK;
}

int gemm_fp16_tn_splitk_splits(int M, int N, int K)
{
    if (M <= 0 || N <= 0 || K < 0 || M > kMaxM || K > (1 << 21) || N > (1 << 21)) return -1;
    if (K == 0) return 1;
    const int cap = split_capacity();
    if (cap <= 0) return -1;
    return choose_splits(M, N, K, cap);
}

size_t gemm_fp16_tn_splitk_workspace_bytes(int M, int N, int K, int splits)
{
    if (M <= 0 || N <= 0 || K <= 0 || splits < 1 || M > kMaxM || K > (1 << 21) || N > (1 << 21))
        return 0;
    const int cap = split_capacity();
    if (cap <= 0) return 0;
    return plan_split(M, N, K, splits, cap).bytes;
}

sg_status gemm_fp16_tn_splitk(int M, int N, int K, float alpha, const void *A, const void *B,
                              void *D, int splits, void *workspace, size_t workspace_bytes,
                              void *stream)
{
    sg_status st = validate(M, N, K, A, B, D);
    if (st != SG_OK) return st;
    if (splits < 1) return SG_ERR_SHAPE;
    if (reinterpret_cast<uintptr_t>(workspace) & 15) return SG_ERR_ALIGN;
    if (M == 0 || N == 0) return SG_OK;
    if (splits == 1 || K == 0) return gemm_fp16_tn_alpha(M, N, K, alpha, A, B, D, stream);
    // the plan depends on the device's resident workgroup count (a runtime
    // query that changes nothing on the device)
    const int cap = split_capacity();
    if (cap <= 0) return SG_ERR_HIP;
    const SplitPlan p = plan_split(M, N, K, splits, cap);
    if (p.splits == 1) return gemm_fp16_tn_alpha(M, N, K, alpha, A, B, D, stream);
    if (p.grid * SplitCfg::T >= (1LL << 32)) return SG_ERR_SHAPE;
    if (!workspace) return SG_ERR_NULL;
    if (workspace_bytes < p.bytes) return SG_ERR_SHAPE;
    if (overlaps(workspace, p.bytes, A, (size_t)M * K * 2) ||
        overlaps(workspace, p.bytes, B, (size_t)N * K * 2) ||
        overlaps(workspace, p.bytes, D, (size_t)M * N * 2))
        return SG_ERR_ALIAS;
    return launch_split(p, M, N, K, alpha, A, B, D, workspace, stream);
}

sg_status gemm_fp16_tn_splitk_noalloc(int M, int N, int K, float alpha, const void *A,
                                      const void *B, void *D, int splits, void *stream)
{
    sg_status st = validate(M, N, K, A, B, D);
    if (st != SG_OK) return st;
    if (splits < 1) return SG_ERR_SHAPE;
    if (M == 0 || N == 0) return SG_OK;
    if (splits == 1 || K == 0) return gemm_fp16_tn_alpha(M, N, K, alpha, A, B, D, stream);
    const int cap = split_capacity();
    if (cap <= 0) return SG_ERR_HIP;
    const SplitPlan p = plan_split(M, N, K, splits, cap);
    if (p.splits == 1) return gemm_fp16_tn_alpha(M, N, K, alpha, A, B, D, stream);
    if (p.grid * SplitCfg::T >= (1LL << 32)) return SG_ERR_SHAPE;
    if (p.bytes > sizeof(scratch)) return SG_ERR_SHAPE;    // more partials than the array holds
    void *ws = scratch_address();
    if (!ws) return SG_ERR_HIP;
    return launch_split(p, M, N, K, alpha, A, B, D, ws, stream);
}

int gemm_fp16_tn_remainder_quarters(int M, int N, int K)
{
    if (M <= 0 || N <= 0 || K < 0 || M > kMaxM) return -1;
    const int cap = sub_capacity();
    if (cap <= 0) return -1;
    SubPlan sub;
    plain_rounds(M, N, K, false, true, cap, nullptr, &sub);
    return sub.quarters;
}

sg_status sg_select_config(int M, int N, int K, sg_config *out)
{
    if (!out) return SG_ERR_NULL;
    if (M < 0 || N < 0 || K < 0) return SG_ERR_SHAPE;
    const Variant *v = select_variant(M, N, K, false, nullptr, true, device_cus());
    if (!v) return SG_ERR_UNSUPPORTED;
    *out = v->cfg;
    return SG_OK;
}

int sg_num_configs(void) { return kNumVariants; }

sg_status sg_get_config(int index, sg_config *out)
{
    if (!out) return SG_ERR_NULL;
    if (index < 0 || index >= kNumVariants) return SG_ERR_UNSUPPORTED;
    *out = kVariants[index].cfg;
    return SG_OK;
}

sg_status sg_query_config(const sg_config *cfg, sg_config_info *info)
{
    if (!cfg || !info) return SG_ERR_NULL;
    const Variant *v = find_variant(cfg);
    if (!v) return SG_ERR_UNSUPPORTED;
    info->threads = v->threads;
    info->lds_bytes = v->ring_bytes;
    info->lds_total_bytes = v->lds_bytes;
    info->loads_per_stage = v->loads;
    info->wg_per_cu_lds = 163840 / v->lds_bytes;
    info->regs = -1;
    info->wg_per_cu_regs = -1;
    info->wg_per_cu = -1;
    hipFuncAttributes attr;
    if (hipFuncGetAttributes(&attr, v->kernel) != hipSuccess) return SG_ERR_HIP;
    info->regs = attr.numRegs;
    if (attr.numRegs > 0) {
        // 512 registers per lane per SIMD, allocated in granules of 8; four
        // SIMDs per CU, waves of a workgroup spread over them.
        const int alloc = (attr.numRegs + 7) / 8 * 8;
        int waves_per_simd = 512 / alloc;
        if (waves_per_simd > 8) waves_per_simd = 8;
        info->wg_per_cu_regs = (4 * waves_per_simd) / cfg->waves;
    }
    int blocks = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&blocks, v->kernel, v->threads, 0) ==
        hipSuccess)
        info->wg_per_cu = blocks;
    return SG_OK;
}

int sg_minimum_stages(long long copy_cycles, long long compute_cycles)
{
    if (copy_cycles <= 0 || compute_cycles <= 0) return -1;
    const long long in_flight = (copy_cycles + compute_cycles - 1) / compute_cycles;
    if (in_flight + 1 > 0x7fffffffLL) return -1;
    return (int)(in_flight + 1);
}

int sg_pipeline_wait_count(int stages, int loads_per_stage, int ntile, int k)
{
    if (stages < 2 || loads_per_stage < 1 || ntile < 1 || k < 0 || k >= ntile) return -1;
    return sg::pipeline_wait_count(stages, loads_per_stage, ntile, k);
}

int sg_persistent_wait_count(int stages, int loads_per_stage, int stores_per_tile, int ntile,
                             int total, int q)
{
    if (stages < 2 || stages > 3 || loads_per_stage < 1 || stores_per_tile < 0 || ntile < 1 ||
        total < 1 || total % ntile != 0 || q < 0 || q >= total)
        return -1;
    if (q == 0) return loads_per_stage * ((stages == 3 && total > 1) ? 1 : 0);
    const int g = q - 1;
    return sg::persistent_wait_count(stages, loads_per_stage, stores_per_tile, ntile, total,
                                     g / ntile, g % ntile);
}

const char *sg_status_string(sg_status status)
{
    switch (status) {
    case SG_OK: return "SG_OK";
    case SG_ERR_NULL: return "SG_ERR_NULL: a required pointer is NULL";
    case SG_ERR_SHAPE: return "SG_ERR_SHAPE: dimension negative or beyond the supported range";
    case SG_ERR_ALIGN: return "SG_ERR_ALIGN: K and N must be multiples of 8 and pointers 16-byte aligned";
    case SG_ERR_UNSUPPORTED: return "SG_ERR_UNSUPPORTED: no compiled kernel for this configuration";
    case SG_ERR_ALIAS: return "SG_ERR_ALIAS: D overlaps A or B";
    case SG_ERR_HIP: return "SG_ERR_HIP: the HIP runtime reported an error";
    }
    return "unknown sg_status";
}

}  // extern "C"
