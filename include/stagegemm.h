/*
 * stagegemm: stage-pipelined half-precision TN GEMM for MI355X (gfx950).
 *
 *     D = alpha * A * B^T
 *
 * A is M x K, B is N x K and D is M x N, all row-major and contiguous
 * (leading dimensions K, K and N), all IEEE binary16.  Products are
 * accumulated in fp32 and each output is rounded once to fp16
 * (round-to-nearest-even).
 *
 * Sources of the operation:
 *   - "cute(9) multistage_gemm", section 11.1: A(M,K), B(N,K) and D(M,N) are
 *     row-major and D = A @ B^T (the "TN" GEMM); sections 4-8 describe the
 *     kStage-deep shared-memory ring that the kernels behind this interface
 *     implement in LDS (prologue of S-1 tiles, a steady state that overlaps the
 *     load of tile k+S-1 with the math on tile k, a drain and an epilogue).
 *   - "CUDA operator notes 2", section "GEMM": fp16 matrices with an fp32
 *     scale factor alpha applied to the product before the cast to half.
 *   - "Lesson 6: Shared Memory layout and async pipeline", section 4: the
 *     stage-count model S_min = ceil(T_copy / T_compute) + 1 and the LDS
 *     footprint S * (tile_A + tile_B) * sizeof(T) behind sg_minimum_stages
 *     and sg_query_config.
 *
 * Ownership and threading.  Every matrix pointer is a caller-owned DEVICE
 * pointer.  The library allocates nothing, copies nothing and never
 * synchronises: a GEMM call validates its arguments on the host, enqueues one
 * kernel on `stream` (a hipStream_t; NULL = the default stream) and returns.
 * The result is ready when the stream reaches that point.  Calls may be made
 * from several host threads at once.
 *
 * Errors.  No function throws or aborts.  All argument checks happen before
 * any HIP call, so a rejected call has no effect on the device.
 *
 * Limits and layout rules (a reading: the pages assume tile multiples or pad):
 *   - M, N, K >= 0.  M == 0 or N == 0 is a no-op returning SG_OK; K == 0
 *     writes +0 to all of D (the empty sum).
 *   - K % 8 == 0 and N % 8 == 0 (rows are whole 16-byte chunks), and A, B, D
 *     16-byte aligned; otherwise SG_ERR_ALIGN.  M needs no multiple.  Tails
 *     in M, N and K that are not tile multiples are handled inside the
 *     kernel.
 *   - K <= 2^21, N <= 2^21, M <= 2^31 - 257, every matrix below 2^40
 *     elements and the launch below 2^32 threads; otherwise SG_ERR_SHAPE.
 *   - D must not overlap A or B (SG_ERR_ALIAS).
 */
#ifndef STAGEGEMM_H
#define STAGEGEMM_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sg_status {
    SG_OK = 0,
    SG_ERR_NULL = 1,        /* a required pointer is NULL */
    SG_ERR_SHAPE = 2,       /* negative or too large dimension */
    SG_ERR_ALIGN = 3,       /* K % 8, N % 8 or 16-byte pointer alignment */
    SG_ERR_UNSUPPORTED = 4, /* no compiled kernel for the requested config */
    SG_ERR_ALIAS = 5,       /* D overlaps A or B */
    SG_ERR_HIP = 6          /* the HIP runtime reported an error at launch */
} sg_status;

/* A compiled kernel variant: output tile tile_m x tile_n, K step tile_k,
 * `stages` LDS ring slots, `waves` 64-lane wavefronts per workgroup, and the
 * mainloop order `schedule`:
 *   0  "Lesson 6", section 2: per K step wait, barrier, refill the free slot,
 *      then read fragments and compute;
 *   1  "cute(9) multistage_gemm", sections 6 and 9: fragments double-buffered
 *      in registers, the next tile's first fragments read right after the
 *      barrier and before the current tile's last MFMAs;
 *   2  the same ring split over two wave groups that alternate between
 *      reading fragments and issuing MFMAs (two stages only);
 *   3  persistent: one workgroup per resident slot computes a sequence of
 *      output tiles whose K tiles stream through one ring (order 1 within
 *      each), so the next tile's loads overlap this tile's last MFMAs and
 *      epilogue; two or three stages, D = alpha * A * B^T only (the C
 *      operand of gemm_fp16_tn_alpha_beta selects another variant);
 *   4  short K: the whole K extent (K <= stages * tile_k) loaded into the
 *      ring at once, then each wave's row blocks computed and stored in
 *      turn; D = alpha * A * B^T only (SG_ERR_UNSUPPORTED for a longer K or
 *      with a C operand).  Schedules 3 and 4 take output tiles in row-major
 *      order where A and B together fit in one XCD's L2 (4 MiB), else with
 *      each XCD given a contiguous run of them; the library runs schedule 4
 *      for K <= 128 where they fit and schedule 3 where they do not;
 *   5  order 1 on 16x16x32 MFMAs instead of 32x32x16 (tile_k 64): the same
 *      LDS traffic per flop, a different balance between clock and MFMA
 *      occupancy under the power limit.  Compiled for comparison; the
 *      library's own choice never takes it;
 *   7  order 2 (ping-pong wave groups) on 16x16x32 MFMAs (tile_k 64, two
 *      stages).  Compiled for comparison;
 *   8  order 7 with the LDS-DMA loads split between the two wave groups:
 *      the first group loads A tiles, the second B tiles, each in its own
 *      fragment-read phase.  A keeps stages - 1 ring slots and B keeps
 *      `stages` (stages = 3: 64 + 96 KiB for 256 x 256 x 64 tiles), which
 *      gives the second group's loads two phases to land.  Compiled for
 *      comparison;
 *  10  one wave per SIMD ("cute(9) multistage_gemm", section 6, with the
 *      two-slot ring of "Lesson 6", section 4): 4 waves of 128 x 128 each,
 *      64-deep K tiles in two 64 KiB slots, one barrier per tile between
 *      its two 32-deep halves; the second half's fragment reads and the
 *      LDS-DMA of tile k + 2 into the slot just freed overlap its MFMAs.
 *      Only 256 x 256 x 64, stages 2, waves 4.  The library's choice for
 *      256 x 256 tiles when every row of A and B starts on a 128-byte line
 *      (K % 64 == 0 and 128-byte aligned A and B);
 *  11  order 10 with a third B slot (A: 2 slots, B: 3, 160 KiB), B loaded
 *      three tiles ahead.  Compiled for comparison;
 *  12  order 11 with the B loads moved to the first half of each tile (B two
 *      tiles ahead, into the slot the tile before last left), so each half
 *      tile issues 8 loads per wave instead of 16.  Only 256 x 256 x 64,
 *      stages 3, waves 4.  The library's choice for 256 x 256 tiles when
 *      rows of A or B straddle 128-byte lines (K % 64 != 0, or a base
 *      address not 128-byte aligned), where each load touches two lines
 *      and holds the issuing wave longer, and for grids of at most two
 *      tile rows or columns, whose operands stream from HBM;
 *  14  order 10 on 128 x 128 x 64 tiles: 4 waves of 64 x 64, a ring of four
 *      32 KiB slots, tile k + 3 loaded over the two halves of tile k.  Only
 *      stages 4, waves 4.  The library's choice for grids of at most one
 *      round of 128 x 128 tiles (one per compute unit) with K >= 1024 and
 *      rows on 128-byte lines. */
typedef struct sg_config {
    int tile_m;
    int tile_n;
    int tile_k;
    int stages;
    int waves;
    int schedule;
} sg_config;

/* Static facts about a compiled variant. */
typedef struct sg_config_info {
    int threads;            /* workgroup size */
    int lds_bytes;          /* LDS ring: stages * (tile_m + tile_n) * tile_k * 2 */
    int lds_total_bytes;    /* LDS allocated: the ring or the epilogue staging, if larger */
    int loads_per_stage;    /* 16-byte global->LDS loads per lane per stage */
    int wg_per_cu_lds;      /* floor(160 KiB / lds_total_bytes) */
    int regs;               /* VGPRs + AGPRs per lane (code object), -1 if unknown */
    int wg_per_cu_regs;     /* workgroups per CU allowed by the register file, -1 if unknown */
    int wg_per_cu;          /* resident workgroups per CU reported by the runtime, -1 if unknown */
} sg_config_info;

/* D = A * B^T.  See the rules above.  `stream` is a hipStream_t.
 *
 * The call runs the variant sg_select_config names, except where a grid of
 * more than one round of 256 x 256 tiles leaves its last round at most a
 * quarter full (rows on 128-byte lines, K % 64 == 0, K >= 1024): then the
 * whole rounds run as 256 x 256 tiles (schedule 10, or 12 for a grid of at
 * most two tile rows or columns) and each remaining tile
 * as four 128 x 128 quarters (schedule 14), two kernels on `stream`
 * ("cute(9) multistage_gemm", section 11.3, names adaptive tile sizes beside
 * split-K).  Every element is computed the same way either way: the same
 * MFMA in the same K order, so the results are bit for bit the same.  The
 * same holds for gemm_fp16_tn_alpha and gemm_fp16_tn_alpha_beta. */
sg_status gemm_fp16_tn(int M, int N, int K, const void *A, const void *B, void *D,
                       void *stream);

/* D = alpha * A * B^T: the fp32 accumulator is multiplied by the fp32 alpha
 * before the single rounding to fp16 ("CUDA operator notes 2", "GEMM"). */
sg_status gemm_fp16_tn_alpha(int M, int N, int K, float alpha, const void *A,
                             const void *B, void *D, void *stream);

/* D = alpha * A * B^T + beta * C, the full GEMM of "CUDA operator notes 2",
 * section "GEMM" (C = alpha A B + beta C with fp16 matrices and fp32 alpha,
 * beta).  C is M x N row-major fp16 (ldc = N), read only.  The fp32
 * accumulator is combined as fma(beta, c, alpha * acc) in fp32 and rounded
 * once to fp16.  beta == 0: C is not read (it may be NULL, and NaNs in it do
 * not propagate).  Otherwise C must be non-NULL (SG_ERR_NULL), 16-byte
 * aligned (SG_ERR_ALIGN), and either be D itself -- an in-place update, as
 * on the page -- or not overlap D at all (SG_ERR_ALIAS).  C may overlap A or
 * B.  Other rules as gemm_fp16_tn. */
sg_status gemm_fp16_tn_alpha_beta(int M, int N, int K, float alpha, float beta,
                                  const void *A, const void *B, const void *C, void *D,
                                  void *stream);

/* Split-K form of gemm_fp16_tn_alpha, for grids that leave compute units
 * idle: fewer 256 x 256 output tiles than one round of resident workgroups
 * (one per compute unit), or a last round that is only partly full
 * ("cute(9) multistage_gemm", section 11.3, names split-K as the remedy for
 * too few output tiles).  Output tiles that fill whole rounds are computed
 * as by the tiled schedule the library would pick (10 when every row of A
 * and B starts on a 128-byte line, else 12, and 12 for grids of at most two
 * tile rows or columns); each remaining tile is cut
 * along K into
 * `splits` contiguous runs of 64-deep K tiles (fewer if K has fewer tiles,
 * at most 16), each run computed by its own workgroup through the same
 * stage-pipelined mainloop, which writes the run's fp32 partial tile to the
 * workspace.  A second kernel then adds the runs of every cut tile in run
 * order (so the result does not depend on which run finished first),
 * multiplies by alpha and rounds once to fp16.
 *
 * Workspace: caller-owned device memory, 16-byte aligned (SG_ERR_ALIGN), of
 * at least gemm_fp16_tn_splitk_workspace_bytes(M, N, K, splits) bytes
 * (SG_ERR_SHAPE if smaller, SG_ERR_NULL if NULL when needed), not
 * overlapping A, B or D (SG_ERR_ALIAS).  Its contents on entry do not
 * matter and are scratch afterwards; calls that share a workspace must not
 * overlap in time.  splits == 1, or a shape with nothing to split, needs no
 * workspace and runs gemm_fp16_tn_alpha.  splits < 1: SG_ERR_SHAPE.  The
 * split plan depends on the current device's resident workgroup count, which
 * is read from the runtime (a query that changes nothing on the device):
 * errors that depend on the plan (workspace NULL, too small or overlapping)
 * are found after that query, all others before any HIP call.  Other rules
 * as gemm_fp16_tn.  Enqueues two kernels on `stream` (one when nothing is
 * split). */
sg_status gemm_fp16_tn_splitk(int M, int N, int K, float alpha, const void *A, const void *B,
                              void *D, int splits, void *workspace, size_t workspace_bytes,
                              void *stream);

/* Workspace bytes gemm_fp16_tn_splitk needs on the current device: one fp32
 * 256 x 256 partial tile per run of each cut tile.  0 when nothing is split,
 * for invalid sizes, or when the device cannot be queried. */
size_t gemm_fp16_tn_splitk_workspace_bytes(int M, int N, int K, int splits);

/* The split count the library would use for this shape on the current
 * device (1: the plain call is the better choice).  -1 for invalid sizes or
 * a failed device query. */
int gemm_fp16_tn_splitk_splits(int M, int N, int K);

/* The split plan gemm_fp16_tn_splitk makes for a device that keeps
 * `capacity` workgroups of the split kernel resident (one per compute unit:
 * 256 on MI355X), computed on the host without any HIP call: 256 x 256
 * tiles, the tiles computed whole (whole rounds of `capacity`), the tiles cut
 * along K, the split count after the caller's is lowered to the K tiles and
 * to 16, the workgroups launched by the first kernel, the workspace bytes,
 * and the split count the library's time model would choose for this shape
 * on such a device.  SG_ERR_SHAPE for non-positive or out-of-range sizes,
 * splits < 1 or capacity < 1; SG_ERR_NULL if out is NULL. */
typedef struct sg_split_info {
    int tiles;
    int whole_tiles;
    int cut_tiles;
    int splits;
    long long workgroups;
    size_t workspace_bytes;
    int chosen_splits;
} sg_split_info;

sg_status sg_split_plan(int M, int N, int K, int splits, int capacity, sg_split_info *out);

/* gemm_fp16_tn_splitk without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP-graph capture, tight serving loops,
 * harnesses that forbid allocation).  The partial tiles live in a fixed
 * 64 MiB device array of the library's own (256 fp32 partial tiles of
 * 256 x 256, one round of split pieces on a 256-CU device), which every GPU
 * the library runs on holds until the process ends; its address is looked
 * up once per device.  This call allocates and frees nothing and calls no
 * allocating library routine.  A plan whose partials exceed the array
 * (gemm_fp16_tn_splitk_workspace_bytes(M, N, K, splits) > 64 MiB) is
 * rejected with SG_ERR_SHAPE before any launch.  Every call on one GPU
 * shares the array: calls that overlap in time on one GPU (two streams, two
 * host threads) race and may return wrong results; serialise them.  Nothing
 * in the array needs to be zero.  Other arguments, rules and errors as
 * gemm_fp16_tn_splitk. */
sg_status gemm_fp16_tn_splitk_noalloc(int M, int N, int K, float alpha, const void *A,
                                      const void *B, void *D, int splits, void *stream);

/* As gemm_fp16_tn_alpha, but runs the named compiled variant instead of the
 * one the library would choose (used by the stage-count sweep).
 * SG_ERR_UNSUPPORTED if no such variant is compiled; SG_ERR_NULL if cfg is
 * NULL. */
sg_status gemm_fp16_tn_cfg(int M, int N, int K, float alpha, const void *A,
                           const void *B, void *D, const sg_config *cfg,
                           void *stream);

/* The number of 128 x 128 quarter tiles gemm_fp16_tn would run in the
 * remainder form for this shape with 128-byte aligned A and B on the current
 * device (0: it runs the variant sg_select_config names alone), or -1 for a
 * negative or empty shape or when the runtime cannot report the device's
 * resident workgroup count.  Reads only device attributes. */
int gemm_fp16_tn_remainder_quarters(int M, int N, int K);

/* The variant gemm_fp16_tn (and gemm_fp16_tn_alpha) would run for this
 * shape with 128-byte aligned A and B (a less aligned A or B turns
 * schedule 10 into schedule 12).  gemm_fp16_tn_alpha_beta with beta != 0 runs
 * the same variant unless it is persistent (schedule 3) or short-K
 * (schedule 4), which take no C operand: the choice is then made among the
 * tiled variants only, by the same cost model. */
sg_status sg_select_config(int M, int N, int K, sg_config *out);

/* Enumerate the compiled variants: index 0 .. sg_num_configs()-1. */
int sg_num_configs(void);
sg_status sg_get_config(int index, sg_config *out);

/* Footprint, register use and occupancy of a compiled variant.  Reads the
 * kernel's attributes through the HIP runtime (the only query that touches
 * HIP; SG_ERR_HIP without a device, with every LDS-derived field still
 * filled in). */
sg_status sg_query_config(const sg_config *cfg, sg_config_info *info);

/* S_min = ceil(copy_cycles / compute_cycles) + 1 ("Lesson 6", section 4, and
 * its exercise); -1 unless both arguments are positive. */
int sg_minimum_stages(long long copy_cycles, long long compute_cycles);

/* Number of this lane's 16-byte loads the kernel lets remain in flight when
 * it is about to consume K tile `k` of `ntile` (its s_waitcnt vmcnt value):
 * loads_per_stage * min(stages - 2, ntile - 1 - k).  -1 for bad arguments. */
int sg_pipeline_wait_count(int stages, int loads_per_stage, int ntile, int k);

/* The same for the persistent schedule (3): one workgroup streams the K tiles
 * of its output tiles (`total` = ntile x its output-tile count) through one
 * ring, and after each output tile issues the next load group early and then
 * `stores_per_tile` 16-byte stores per lane.  Count of this lane's loads and
 * stores the kernel lets remain in flight when it is about to consume stream
 * tile `q`: the later load group (three stages) and the stores issued after
 * tile q's loads.  Exact except with three stages and one K tile per output
 * tile, where the stores of the output tile two back are not counted (the
 * kernel then waits longer than it must).  -1 for bad arguments (stages
 * outside 2..3, non-positive sizes, q outside 0..total-1, total not a
 * multiple of ntile). */
int sg_persistent_wait_count(int stages, int loads_per_stage, int stores_per_tile, int ntile,
                             int total, int q);

/* Fused attention forward, "CUDA operator notes 2", section "Softmax
 * Attention": O = softmax(alpha * Q K^T) V with the softmax along each row,
 * for H independent heads.  Q is H x M x d, K and V are H x N x d, O is
 * H x M x d; every head is row-major fp16 and the heads are stored one after
 * another (head stride M * d or N * d elements).  The scores stay on chip:
 * one pass over the keys with a running reference exponent per row (raised
 * when the row's maximum passes it by more than 2^8; the quotient does not
 * depend on it) and a running row sum in fp32, P V accumulated in fp32 from
 * fp16 probabilities, O / l converted once to fp16.
 * alpha is fp32 (the page's 1/sqrt(d) is the caller's choice).
 * Only d == 128 is compiled (SG_ERR_UNSUPPORTED otherwise).  H == 0 or
 * M == 0: no work.  N == 0 with M > 0: SG_ERR_SHAPE (no keys to weight).
 * Pointers: caller-owned device memory, 16-byte aligned (SG_ERR_ALIGN), O
 * may not overlap Q, K or V (SG_ERR_ALIAS).  M, N <= 2^21.  Enqueues one
 * kernel on `stream`; allocates and synchronises nothing. */
sg_status attention_fp16_fwd(int H, int M, int N, int d, float alpha, const void *Q,
                             const void *K, const void *V, void *O, void *stream);

/* Split-key form of attention_fp16_fwd, for grids too small to fill the
 * device (one head of 4096 queries is 32 workgroups).  The keys of each head
 * are cut into `splits` contiguous runs of 64-key tiles (at most one run per
 * tile: a larger count is lowered to the number of key tiles); each run
 * yields an unnormalised partial of O with its own reference exponent and
 * row sum, written to `workspace` in fp32, and a second kernel merges the
 * runs of every row with the same online-softmax identity ("CUDA operator
 * notes 2", section "Softmax Attention"; the softmax does not depend on the
 * constant subtracted before the exponential).  Same arguments, layouts and
 * errors as attention_fp16_fwd, plus: splits >= 1 (SG_ERR_SHAPE otherwise);
 * splits == 1 needs no workspace and is attention_fp16_fwd.  For splits > 1,
 * `workspace` is caller-owned device memory of at least
 * attention_fp16_workspace_bytes(H, M, N, d, splits) bytes (SG_ERR_SHAPE if
 * smaller, SG_ERR_NULL if null), 16-byte aligned (SG_ERR_ALIGN), not
 * overlapping Q, K, V or O (SG_ERR_ALIAS); its contents on entry do not
 * matter and are scratch afterwards.  Enqueues two kernels on `stream`;
 * calls that share a workspace must not overlap in time. */
sg_status attention_fp16_fwd_split(int H, int M, int N, int d, float alpha, const void *Q,
                                   const void *K, const void *V, void *O, int splits,
                                   void *workspace, size_t workspace_bytes, void *stream);

/* Bytes of workspace attention_fp16_fwd_split needs: H * s * M * (d + 2) * 4
 * with s = min(splits, key tiles); 0 when s <= 1 or the sizes are invalid. */
size_t attention_fp16_workspace_bytes(int H, int M, int N, int d, int splits);

/* The split count this library would use on the current device: the count
 * (1 to min(64, key tiles)) that minimises a cost model of the forward (about
 * one 64-key tile per microsecond per compute unit, bounded below by one
 * workgroup's own tiles) plus the merge (a fixed cost and the fp32 partials'
 * traffic).  1 whenever the heads already fill the device.  -1 for invalid
 * sizes (d != 128 included) or a failed device query. */
int attention_fp16_splits(int H, int M, int N, int d);

/* Human-readable name of a status code (static storage). */
const char *sg_status_string(sg_status status);

#ifdef __cplusplus
}
#endif

#endif /* STAGEGEMM_H */
