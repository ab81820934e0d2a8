// C-ABI of the fused attention forward: argument validation and the launch
// on the caller's stream.  The interface is documented in include/stagegemm.h.
#include "stagegemm.h"

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

#include "attention_kernel.hpp"

namespace {

bool ranges_overlap(const void *p, size_t pbytes, const void *q, size_t qbytes)
{
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    const uintptr_t b = reinterpret_cast<uintptr_t>(q);
    return pbytes && qbytes && a < b + qbytes && b < a + pbytes;
}

// Checks shared by both entry points; SG_OK means "launch".
sg_status check_args(int H, int M, int N, int d, const void *Q, const void *K, const void *V,
                     const void *O)
{
    if (H < 0 || M < 0 || N < 0 || d < 0) return SG_ERR_SHAPE;
    if (d != sg::AttnCfg<4>::D) return SG_ERR_UNSUPPORTED;
    if (N == 0) return SG_ERR_SHAPE;                    // softmax over no keys
    if (!Q || !K || !V || !O) return SG_ERR_NULL;
    if (N > (1 << 21) || M > (1 << 21)) return SG_ERR_SHAPE;
    if ((long long)H * M * d >= (1LL << 40) || (long long)H * N * d >= (1LL << 40))
        return SG_ERR_SHAPE;
    const uintptr_t all = reinterpret_cast<uintptr_t>(Q) | reinterpret_cast<uintptr_t>(K) |
                          reinterpret_cast<uintptr_t>(V) | reinterpret_cast<uintptr_t>(O);
    if (all & 15) return SG_ERR_ALIGN;
    const size_t qbytes = (size_t)H * M * d * 2, kvbytes = (size_t)H * N * d * 2;
    if (ranges_overlap(O, qbytes, Q, qbytes) || ranges_overlap(O, qbytes, K, kvbytes) ||
        ranges_overlap(O, qbytes, V, kvbytes))
        return SG_ERR_ALIAS;
    return SG_OK;
}

int key_tiles(int N) { return (N + sg::AttnCfg<4>::BN - 1) / sg::AttnCfg<4>::BN; }

size_t workspace_bytes(int H, int M, int splits)
{
    return (size_t)H * splits * M * (sg::AttnCfg<4>::D + 2) * sizeof(float);
}

// Compute units of the current device (cached per device; 0 if the query
// fails).  Host threads that fill the cache at once write the same value,
// through an atomic.
int device_cus()
{
    static std::atomic<int> cache[64];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
    if (dev < 64) {
        const int hit = cache[dev].load(std::memory_order_relaxed);
        if (hit > 0) return hit;
    }
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return 0;
    if (dev < 64) cache[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

long long row_blocks(int M, int bm) { return (M + bm - 1) / bm; }

// splits == 1: O directly; otherwise the partials go to part_o / part_ml and
// a second kernel merges them.  Unsplit calls whose 256-row workgroups fill
// every CU take the 8-wave kernel, all others the 4-wave one.
sg_status launch(int H, int M, int N, float alpha, const void *Q, const void *K, const void *V,
                 void *O, int splits, void *workspace, hipStream_t stream)
{
    // the 4-wave grid is the larger one: bound it before any HIP call
    if ((long long)H * row_blocks(M, sg::AttnCfg<4>::BM) * splits >= (1LL << 31))
        return SG_ERR_SHAPE;
    const int cus = splits == 1 ? device_cus() : 0;
    const bool wide = cus > 0 && H * row_blocks(M, sg::AttnCfg<8>::BM) >= cus;
    const int bm = wide ? sg::AttnCfg<8>::BM : sg::AttnCfg<4>::BM;
    const long long blocks = (long long)H * row_blocks(M, bm) * splits;
    typedef void (*attn_fn)(const _Float16 *, const _Float16 *, const _Float16 *, _Float16 *,
                            float *, float *, int, int, float, int);
    const attn_fn kernel =
        wide ? (alpha < 0.0f ? &sg::attention_fwd_kernel<true, 8> : &sg::attention_fwd_kernel<false, 8>)
             : (alpha < 0.0f ? &sg::attention_fwd_kernel<true, 4> : &sg::attention_fwd_kernel<false, 4>);
    const _Float16 *q = static_cast<const _Float16 *>(Q);
    const _Float16 *k = static_cast<const _Float16 *>(K);
    const _Float16 *v = static_cast<const _Float16 *>(V);
    _Float16 *o = static_cast<_Float16 *>(O);
    float *part_o = splits > 1 ? static_cast<float *>(workspace) : nullptr;
    float *part_ml = splits > 1 ? part_o + (size_t)H * splits * M * sg::AttnCfg<4>::D : nullptr;
    void *args[] = {&q, &k, &v, &o, &part_o, &part_ml, &M, &N, &alpha, &splits};
    static_assert(sizeof(args) / sizeof(args[0]) == 10, "one entry per kernel parameter");
    hipError_t e = hipLaunchKernel(reinterpret_cast<const void *>(kernel), dim3((unsigned)blocks),
                                   dim3(64 * (wide ? 8 : 4)), args, 0, stream);
    if (e != hipSuccess || splits == 1) return e == hipSuccess ? SG_OK : SG_ERR_HIP;

    long long HM = (long long)H * M;
    const long long cblocks = (HM * 32 + 255) / 256;
    typedef void (*comb_fn)(const float *, const float *, _Float16 *, long long, int, int);
    const comb_fn comb = &sg::attention_combine_kernel;
    const float *cpo = part_o, *cpm = part_ml;
    void *cargs[] = {&cpo, &cpm, &o, &HM, &M, &splits};
    static_assert(sizeof(cargs) / sizeof(cargs[0]) == 6, "one entry per kernel parameter");
    e = hipLaunchKernel(reinterpret_cast<const void *>(comb), dim3((unsigned)cblocks), dim3(256),
                        cargs, 0, stream);
    return e == hipSuccess ? SG_OK : SG_ERR_HIP;
}

}  // namespace

extern "C" {

sg_status attention_fp16_fwd(int H, int M, int N, int d, float alpha, const void *Q,
                             const void *K, const void *V, void *O, void *stream)
{
    if (H < 0 || M < 0 || N < 0 || d < 0) return SG_ERR_SHAPE;
    if (H == 0 || M == 0) return SG_OK;
    const sg_status st = check_args(H, M, N, d, Q, K, V, O);
    if (st != SG_OK) return st;
    return launch(H, M, N, alpha, Q, K, V, O, 1, nullptr, static_cast<hipStream_t>(stream));
}

int attention_fp16_splits(int H, int M, int N, int d)
{
    if (H < 1 || M < 1 || N < 1 || d != sg::AttnCfg<4>::D) return -1;
    const int cus = device_cus();
    if (cus < 1) return -1;
    // A cost model fitted to one box's timings of 4-wave workgroups (128
    // rows, d = 128): a CU runs about one 64-key tile per microsecond, shared
    // by the workgroups it holds, so the forward takes
    //     max(tiles per workgroup, all tiles / CUs) microseconds,
    // and a split call adds the merge: about 4 us (its launch and the partial
    // epilogue) plus writing and reading the fp32 partials at about 5 TB/s.
    // The split count with the smallest estimate wins (ties: fewer splits).
    // It reproduces the fastest measured count on one head at 1024 to 4096
    // keys (8), four heads at 2048 (4) and sixteen heads at 512 to 4096 (1).
    constexpr double kTileUs = 1.0, kMergeUs = 4.0, kBytesPerUs = 5.0e6;
    const long long blocks = (long long)H * ((M + sg::AttnCfg<4>::BM - 1) / sg::AttnCfg<4>::BM);
    const int tiles = key_tiles(N);
    int best_s = 1;
    double best = 0.0;
    for (int s = 1; s <= tiles && s <= 64; ++s) {
        const long long per_wg = (tiles + s - 1) / s;
        const double work = (double)blocks * s * per_wg / cus;
        double t = kTileUs * (per_wg > work ? (double)per_wg : work);
        if (s > 1) t += kMergeUs + 2.0 * (double)workspace_bytes(H, M, s) / kBytesPerUs;
        if (s == 1 || t < best) { best = t; best_s = s; }
        if (blocks * s >= 4LL * cus) break;            // more splits only add partials
    }
    return best_s;
}

size_t attention_fp16_workspace_bytes(int H, int M, int N, int d, int splits)
{
    if (H < 1 || M < 1 || N < 1 || d != sg::AttnCfg<4>::D || splits <= 1) return 0;
    if (splits > key_tiles(N)) splits = key_tiles(N);
    return splits > 1 ? workspace_bytes(H, M, splits) : 0;
}

sg_status attention_fp16_fwd_split(int H, int M, int N, int d, float alpha, const void *Q,
                                   const void *K, const void *V, void *O, int splits,
                                   void *workspace, size_t workspace_bytes_given, void *stream)
{
    if (H < 0 || M < 0 || N < 0 || d < 0 || splits < 1) return SG_ERR_SHAPE;
    if (H == 0 || M == 0) return SG_OK;
    const sg_status st = check_args(H, M, N, d, Q, K, V, O);
    if (st != SG_OK) return st;
    if (splits > key_tiles(N)) splits = key_tiles(N);   // every split keeps a key tile
    if (splits > 1) {
        if (!workspace) return SG_ERR_NULL;
        const size_t need = workspace_bytes(H, M, splits);
        if (workspace_bytes_given < need) return SG_ERR_SHAPE;
        if (reinterpret_cast<uintptr_t>(workspace) & 15) return SG_ERR_ALIGN;
        const size_t qbytes = (size_t)H * M * d * 2, kvbytes = (size_t)H * N * d * 2;
        if (ranges_overlap(workspace, need, Q, qbytes) || ranges_overlap(workspace, need, K, kvbytes) ||
            ranges_overlap(workspace, need, V, kvbytes) || ranges_overlap(workspace, need, O, qbytes))
            return SG_ERR_ALIAS;
    }
    return launch(H, M, N, alpha, Q, K, V, O, splits, workspace, static_cast<hipStream_t>(stream));
}

}  // extern "C"
