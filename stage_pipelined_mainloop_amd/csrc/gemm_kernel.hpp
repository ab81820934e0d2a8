// Stage-pipelined fp16 TN GEMM kernel for gfx950 (CDNA4).
//
//   D[m][n] = RNE16( alpha * sum_k A[m][k] * B[n][k] ),   fp32 accumulation.
//
// Structure (the method of "cute(9) multistage_gemm", sections 4-7, and the
// three-phase order of "Lesson 6: Shared Memory layout and async pipeline",
// sections 2-3), redesigned for CDNA4:
//
//   * One workgroup per BM x BN output tile; NW = WM x WN wavefronts of 64
//     lanes, each owning a (BM/WM) x (BN/WN) sub-tile built from 32x32 MFMA
//     blocks (v_mfma_f32_32x32x16_f16, fp32 accumulators) or from 16x16 ones
//     (v_mfma_f32_16x16x32_f16, schedules 5, 7 and 8; see "MFMA shape"
//     below).
//   * An S-slot ring in LDS.  Each slot holds one K step: A rows [BM x BK] and
//     B rows [BN x BK], both K-contiguous (the TN layout needs no transpose).
//   * Global -> LDS copies are LDS-DMA buffer loads (buffer_load_dwordx4 ...
//     lds): 16 bytes per lane, written by the memory pipeline straight into
//     LDS without passing through VGPRs -- the CDNA counterpart of the async
//     copy the pages build on.  Each wave issues L of them per K step.  There
//     are no commit groups on this hardware, so a "batch" is those L loads and
//     the wait for tile k is `s_waitcnt vmcnt(L * min(S-2, ntile-1-k))`: the
//     loads issued after tile k's may stay in flight, tile k's may not.
//   * Per K step k (one barrier per step):
//        wait(own loads of tile k)  + lgkmcnt(0)      RAW on own part, and own
//                                                     LDS reads of step k-1 done
//        s_barrier                                    every wave: tile k landed,
//                                                     slot (k-1)%S no longer read
//        issue tile k+S-1 into slot (k+S-1)%S = (k-1)%S   (if it exists)  WAR-safe
//        ds_read_b128 fragments of slot k%S, MFMA      overlaps the loads in flight
//     The prologue issues tiles 0..S-2; the last S-2 steps issue nothing and
//     their waits shrink to 0 (drain).  Filling S-1 slots, not S, leaves the
//     slot the first refill needs ("cute(9) multistage_gemm", section 5.1).
//   * Bank conflicts: 16-byte chunk c of LDS row r is stored at chunk position
//     c ^ swz(r).  LDS-DMA writes 64 consecutive 16-byte chunks per wave load,
//     so the swizzle is applied by choosing which global chunk each lane
//     fetches; the fragment reads then hit distinct banks.
//   * Bounds: buffer resources per workgroup cover only the valid rows, so
//     rows past M (A) or N (B) read as zero and stores past M are dropped;
//     K-tail chunks and N-tail columns are sent to an offset past the
//     resource's range (reads 0 / store dropped).  Zero fill gives exactly the
//     plain sum (the padding reading of "CUDA operator notes 2", "GEMM").
//   * K order: every workgroup walks its K tiles from the first (a split
//     piece from the first of its run), so the workgroups of an XCD that
//     share an A or B panel fetch each of its K tiles at about the same time
//     and the XCD's L2 serves the others.  (Starting the tile rows of a group
//     at staggered K tiles, against channel conflicts of power-of-two row
//     strides, measured neutral to 1.5 % slower on the large grids and raised
//     the bytes leaving L2 at 8192^3 from 1.61 to 1.93 GB.)
//   * Epilogue: operands are fed to the MFMA swapped (B rows as the first
//     operand), so each lane's accumulators are four consecutive columns of
//     one row of D.  alpha * acc is converted to fp16 (one rounding), staged
//     through a per-wave LDS region and written back row-contiguously with
//     16-byte stores.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace sg {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4v __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// gfx9 buffer resource word 3 (raw 32-bit data format, no swizzle).
constexpr int kRsrcWord3 = 0x00020000;
// An offset no per-workgroup resource reaches (num_records < 2^31).
constexpr uint32_t kOutOfRange = 0x80000000u;
// Cache-policy bits of the D stores (gfx950 buffer instruction aux field):
// nt (2) marks the lines as streaming and sc1 (16) writes them through the
// XCD's L2 at device scope.  D is written once and never re-read by the
// kernel, so keeping it out of L2 leaves the capacity to the A and B panels
// that neighbouring workgroups re-read; measured +9 % at 8192^3 and -10 %
// time on the 4096x4096x128 shape against the default policy.
constexpr int kStoreStreaming = 2 | 16;

// s_waitcnt immediate for gfx9: vmcnt bits [3:0] and [15:14], expcnt [6:4],
// lgkmcnt [11:8].  expcnt is never waited on here.
constexpr int waitcnt_imm(int vm, int lgkm)
{
    return (vm & 15) | (7 << 4) | ((lgkm & 15) << 8) | (((vm >> 4) & 3) << 14);
}

// Loads of this lane allowed in flight when consuming K tile k.
__host__ __device__ constexpr int pipeline_wait_count(int stages, int loads, int ntile, int k)
{
    int after = ntile - 1 - k;
    if (after > stages - 2) after = stages - 2;
    if (after < 0) after = 0;
    return loads * after;
}

// Persistent schedule: one workgroup's K tiles of all its output tiles form
// one stream (stream tile g = u * ntile + k for output tile u, K step k; its
// loads, "group g", go to ring slot g mod S).  Every stream tile but the last
// issues L loads per lane at its first K step -- group g + S - 1, or, when
// that group does not exist or was issued early, L loads aimed out of range
// into the wave's epilogue staging area (they move no data and fill no ring
// slot, so every tile runs the same code) -- and waits for group g + 1 at its
// last K step.  When g ends an output tile, group g + S is issued at once
// (into the slot g's reads released) before the epilogue's stores, so that
// the stores stay out of the next wait.
__host__ __device__ constexpr bool persistent_real_issue(int stages, int ntile, int total, int u,
                                                         int k)
{
    return u * ntile + k + stages - 1 < total && !(k == 0 && u > 0);
}

// Counted operations (loads and stores, which leave vmcnt in issue order)
// allowed outstanding at the wait for group g + 1 inside stream tile
// g = u * ntile + k (g + 1 < total): the operations issued after that group.
// With two slots: none, except after an output-tile boundary (k == 0, u > 0)
// where group g + 1 was issued early and is followed by the stores and by
// this tile's out-of-range loads.  With three slots: this tile's loads, plus
// after a boundary the early group (if any) and the stores, or one tile later
// (k == 1) the stores and the previous tile's loads.  With three slots and one
// K tile per output tile the stores of the tile two back are left out (a
// smaller count only waits longer).
__host__ __device__ constexpr int persistent_wait_count(int stages, int loads, int stores,
                                                        int ntile, int total, int u, int k)
{
    const int g = u * ntile + k;
    const bool first = k == 0 && u > 0;
    if (stages == 2) return first ? loads + stores : 0;
    if (g == 0) return loads;
    if (first) return (g + 2 < total ? loads : 0) + stores + loads;
    if (k == 1 && u > 0) return stores + 2 * loads;
    return loads;
}

// XOR swizzle of 16-byte chunk positions within an LDS row, by row index.
// Rows of 4 chunks (BK = 32): bit0 = r2, bit1 = r1 ^ r3.
// Rows of 8 chunks (BK = 64): bit0 = r1, bit1 = r2, bit2 = r0 ^ r3.
// Both keep the 32-row ds_read_b128 fragment pattern on distinct banks for
// 8-lane / 128-byte and 16-lane / 256-byte bank groups, and depend only on
// r mod 16, so every 32-row MFMA block sees the same pattern.
template <int CPR>
__device__ __forceinline__ int swz(int r)
{
    if constexpr (CPR == 4) {
        return ((r >> 2) & 1) | ((((r >> 1) ^ (r >> 3)) & 1) << 1);
    } else {
        static_assert(CPR == 8, "rows of 4 or 8 chunks");
        return ((r >> 1) & 1) | (((r >> 2) & 1) << 1) | ((((r) ^ (r >> 3)) & 1) << 2);
    }
}

// SCHED selects the mainloop order: 0 = the three-phase order of "Lesson 6"
// (wait, barrier, refill, compute), 1 = the cute page's order with the next
// tile's first fragments prefetched across the barrier, 2 = ping-pong of two
// wave groups (one computes while the other reads and refills), 3 =
// persistent, 4 = short K, 5 = order 1 on 16x16x32 MFMAs, 7 = order 2 on
// 16x16x32 MFMAs, 8 = order 7 with the LDS-DMA loads split between the two
// wave groups (A ring of S - 1 slots, B ring of S; "order 8" below), 10 = one
// wave per SIMD with a 128x128 tile each, its whole mainloop one scheduled
// inline-assembly statement ("order 10" below), 11 = order 10 with a third B
// slot, B loaded three tiles ahead, 12 = order 11 with the B loads moved to
// the first half of each tile, 14 = order 10 on a 128x128 tile (64x64 per
// wave) with a ring of four slots.
//
// MFMA shape.  Schedules 0-4 use v_mfma_f32_32x32x16_f16 (32x32 blocks, K
// steps of 16); schedules 5, 7 and 8 use v_mfma_f32_16x16x32_f16 (16x16
// blocks, K steps of 32) in the mainloop order of schedule 1, 2 and the
// split-load form of 2 (order 8) respectively.  The
// LDS bytes read per flop are the same (a fragment is 1 KiB either way), but
// under the power limit the 16x16x32 form sustains more throughput on the
// same operands (measured 1867 against 1628 TFLOP/s in an MFMA-only loop on
// uniform [-1, 1] fp16 data).  With order 1 that gain is eaten by the
// fragment reads, which the waves of a workgroup issue all at once; with the
// ping-pong order one wave group reads while the other multiplies, and the
// 8192^3 GEMM runs about 7 % faster than order 1 on 32x32x16 blocks
// (clock 1.78 against 1.39 GHz under the counters, MFMA busy 74 against
// 85 %).  Order 8 then removes the ping-pong's remaining stall (the LDS-DMA
// issues of a whole tile in one read phase) and reaches MFMA busy 80 % at
// the same clock.
template <int BM_, int BN_, int BK_, int S_, int WM_, int WN_, int SCHED_ = 1>
struct Cfg {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, S = S_, WM = WM_, WN = WN_;
    static constexpr int SCHED = SCHED_;
    static constexpr bool MF16 = SCHED == 5 || SCHED == 7 || SCHED >= 8;   // 16x16x32 MFMAs
    static constexpr int ORDER = SCHED == 5 ? 1 : SCHED == 7 ? 2 : SCHED;   // mainloop order
    static constexpr int NW = WM * WN;              // wavefronts
    static constexpr int T = 64 * NW;               // threads
    static constexpr int WTM = BM / WM;             // wave sub-tile
    static constexpr int WTN = BN / WN;
    static constexpr int FM = WTM / 32;             // 32x32 MFMA blocks per wave
    static constexpr int FN = WTN / 32;
    static constexpr int RB = BK * 2;               // LDS row bytes
    static constexpr int CPR = BK / 8;              // 16-byte chunks per row
    static constexpr int KSTEP = MF16 ? 32 : 16;    // K depth of one MFMA
    static constexpr int NKS = BK / KSTEP;          // MFMA K steps per tile
    static constexpr int MB = MF16 ? 16 : 32;       // rows of one MFMA block
    static constexpr int AM = WTM / MB;             // MFMA blocks per wave
    static constexpr int AN = WTN / MB;
    static constexpr int A_BYTES = BM * RB;
    static constexpr int B_BYTES = BN * RB;
    static constexpr int STAGE_BYTES = A_BYTES + B_BYTES;
    // Orders 8, 11 and 12 keep S - 1 slots of A and S slots of B.
    static constexpr int RING_BYTES =
        ORDER == 8 || ORDER == 11 || ORDER == 12 ? (S - 1) * A_BYTES + S * B_BYTES : S * STAGE_BYTES;
    // Epilogue staging: one 32-row block of each wave's sub-tile at a time,
    // unpadded rows with the slot swizzle of staged_slot.
    static constexpr int EPI_ROW = WTN * 2;
    static constexpr int EPI_WAVE_BYTES = 32 * EPI_ROW;    // one 32-row block at a time
    static constexpr int EPI_BYTES = NW * EPI_WAVE_BYTES;
    // Persistent and short-K schedules: the ring stays live during the
    // epilogue, so the staging area is separate and holds one 32-row block
    // of every wave's sub-tile at a time (same layout).
    static constexpr int EPI_BLOCK_WAVE_BYTES = 32 * WTN * 2;
    static constexpr int EPI_BLOCK_BYTES = NW * EPI_BLOCK_WAVE_BYTES;
    static constexpr bool OWN_STAGING = SCHED == 3 || SCHED == 4;   // staging beside the ring
    static constexpr int LDS_BYTES = OWN_STAGING ? RING_BYTES + EPI_BLOCK_BYTES
                                   : (RING_BYTES > EPI_BYTES ? RING_BYTES : EPI_BYTES);
    // Epilogue stores per lane per output tile: 16 bytes each, WTN * 2 / 16
    // lanes per sub-tile row.
    static constexpr int EPI_CHUNKS_PER_ROW = WTN * 2 / 16;
    static constexpr int EPI_ROWS_PER_STORE = 64 / EPI_CHUNKS_PER_ROW;
    static constexpr int STORES = FM * (32 / EPI_ROWS_PER_STORE);
    static constexpr int NA = BM * CPR / (64 * NW); // LDS-DMA loads per wave per stage
    static constexpr int NB = BN * CPR / (64 * NW);
    static constexpr int L = NA + NB;
    static_assert(S >= 2, "a ring needs at least two slots");
    static_assert(SCHED >= 0 && SCHED <= 14 && SCHED != 6 && SCHED != 9 && SCHED != 13, "mainloop order");
    static_assert(!MF16 || BK == 64, "16x16x32 order: two K steps of 32 per tile");
    static_assert(SCHED != 3 || S == 2 || S == 3, "persistent ring: two or three slots");
    static_assert(!OWN_STAGING || WTN == 64, "unpadded staging rows are 128 bytes");
    static_assert(ORDER != 2 || (S == 2 && NW % 4 == 0 && (NW / 2) % 2 == 0 && BK == 64),
                  "ping-pong: two slots, two even wave groups, 128-byte rows");
    static_assert(ORDER != 8 || (S == 3 && NW % 4 == 0 && (NW / 2) % 2 == 0 && BK == 64 && BM == BN),
                  "split-load ping-pong: A ring of two slots, B ring of three, square tiles");
    static_assert(NKS % 2 == 0, "fragment double buffer alternates per K step");
    static_assert(ORDER != 10 || (BM == 256 && BN == 256 && BK == 64 && S == 2 && WM == 2 && WN == 2),
                  "one-wave form: 256x256x64 tiles, two slots, 2x2 waves of 128x128");
    static_assert((ORDER != 11 && ORDER != 12) ||
                      (BM == 256 && BN == 256 && BK == 64 && S == 3 && WM == 2 && WN == 2),
                  "one-wave form, third B slot: 256x256x64 tiles, 2x2 waves of 128x128");
    static_assert(ORDER != 14 || (BM == 128 && BN == 128 && BK == 64 && S == 4 && WM == 2 && WN == 2),
                  "one-wave form, 128x128x64 tiles, four slots, 2x2 waves of 64x64");
    static_assert(BK == 32 || BK == 64, "BK");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile is whole 32x32 blocks");
    static_assert(NA * 64 * NW == BM * CPR && NB * 64 * NW == BN * CPR, "even load split");
    static_assert(NA >= 1 && NB >= 1, "every wave loads both operands");
    static_assert(L * (S - 2) + (SCHED == 3 ? STORES + 2 * L : 0) <= 63, "vmcnt is a 6-bit counter");
    static_assert(32 % EPI_ROWS_PER_STORE == 0, "a 32-row block is whole store instructions");
    static_assert(LDS_BYTES <= 163840, "160 KiB of LDS per workgroup");
    static_assert((WTN * 2) % 16 == 0 && 64 % ((WTN * 2) / 16) == 0, "epilogue row chunks");
};

// Buffer resource for `bytes` bytes from `base` (stride 0): reads past the
// range return zero and stores past it are dropped.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                             kRsrcWord3);
}

// The same resource as plain words, for inline assembly (an SGPR quad).
__device__ __forceinline__ u32x4 rsrc_words(const void *base, uint32_t bytes)
{
    const uint64_t a = reinterpret_cast<uint64_t>(base);
    return u32x4{(uint32_t)a, (uint32_t)(a >> 32) & 0xffffu, bytes, (uint32_t)kRsrcWord3};
}

// LDS-DMA of 16 bytes per lane to the wave's 1 KiB at LDS address `lds`
// (lane l fills bytes 16 l .. 16 l + 15), issued through inline assembly.
// The compiler cannot tell later LDS reads apart from a pending DMA target
// and, for its own LDS-DMA builtin, waits for every VMEM operation in flight
// (the DMA and any earlier stores) before each of them; these loads it does
// not see at all, and the kernel's own vmcnt waits before its barriers order
// them.  (Loads the compiler does track are waited for with counts that
// ignore these: at worst it waits longer.)  m0 is written and consumed inside
// the statement, with the one wait state gfx9 needs between an SALU write of
// m0 and an LDS-DMA that reads it.  The compiler warns that a reserved
// register in a clobber list may not be preserved: no compiler-generated code
// in a kernel that calls this may use m0, which every build checks in the
// generated assembly (every m0 operand must sit inside an inline-assembly
// region).
__device__ __forceinline__ void dma16(const u32x4 &rsrc, uint32_t voff, uint32_t lds)
{
    asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
                 :
                 : "s"(lds), "v"(voff), "s"(rsrc)
                 : "memory", "m0");
}

// Compiler-level fence: no memory access moves across it (emits nothing).
__device__ __forceinline__ void compiler_fence() { asm volatile("" ::: "memory"); }

template <int N>
__device__ __forceinline__ void wait_vm_lgkm0()
{
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(N, 0));
}

// Wait until at most `n` (runtime, n = L * j for j in 0..S-2) of this lane's
// loads are outstanding and all its LDS reads have returned.
template <class C>
__device__ __forceinline__ void wait_tile(int j)
{
    if constexpr (C::S - 2 >= 3) { if (j == 3) { wait_vm_lgkm0<3 * C::L>(); return; } }
    if constexpr (C::S - 2 >= 2) { if (j == 2) { wait_vm_lgkm0<2 * C::L>(); return; } }
    if constexpr (C::S - 2 >= 1) { if (j == 1) { wait_vm_lgkm0<1 * C::L>(); return; } }
    wait_vm_lgkm0<0>();
}

// Grid position -> output tile.  Workgroups are dealt round-robin to the 8
// XCDs; renumber so each XCD receives a contiguous run of tiles, then walk
// the run in groups of GM tile-rows so concurrently resident workgroups of
// one XCD share A and B panels in that XCD's L2.  The renumbering applies to
// grid positions below `renumber` (the whole grid for the tiled kernels; the
// data-parallel part of a split-K grid) when that count is a multiple of 8.
__device__ __forceinline__ void tile_coords(int pid, int tiles_m, int tiles_n, int renumber,
                                            int &tm, int &tn)
{
    if ((renumber & 7) == 0 && pid < renumber) pid = (pid & 7) * (renumber >> 3) + (pid >> 3);
    constexpr int GM = 4;
    const int per_group = GM * tiles_n;
    const int group = pid / per_group;
    const int first_m = group * GM;
    int gm = tiles_m - first_m;
    if (gm > GM) gm = GM;
    const int in_group = pid - group * per_group;
    tm = first_m + in_group % gm;
    tn = in_group / gm;
}

// Grid position -> output tile for the kernels whose K loop is short (the
// short-K and persistent schedules), where writing D takes much of the time
// and the panels are read by few K steps.  When A and B together fit in one
// XCD's L2 (4 MiB), every XCD holds all of them after first touch and tiles
// go in plain row-major order: the workgroups resident together then write
// whole stretches of the same rows of D.  Otherwise the XCD renumbering of
// tile_coords comes first (each XCD a contiguous run of tiles, so both
// column tiles of a tall grid's row band share one L2), then row-major.  No
// groups of tile rows: they serve the panel reuse of long K loops and cost
// the write of D here.  Short-K kernel, HIP-graph replays: 4096 x 4096 x 128
// 11.2 us in tile_coords' order, 9.5-9.9 us row-major, 9.7 us renumbered;
// 81920 x 256 x 128 19.7 us row-major, 13.3 us renumbered.  Persistent
// kernel: 8192 x 8192 x 128 40.4 / 36.5 / 39.4 us (tile_coords, row-major,
// renumbered), 16384 x 4096 x 64 32.0 / 28.4 / 29.9, 81920 x 256 x 256
// 21.7 / 21.2 / 20.6, 40960 x 512 x 256 17.8 / 20.8 / 17.6.
__device__ __forceinline__ void short_k_coords(int pid, int tiles_m, int tiles_n, int M, int N,
                                               int K, int &tm, int &tn)
{
    const long long operand_bytes = ((long long)M + N) * K * 2;
    const int tiles = tiles_m * tiles_n;
    if (operand_bytes > (4ll << 20) && (tiles & 7) == 0 && pid < tiles)
        pid = (pid & 7) * (tiles >> 3) + (pid >> 3);
    tm = pid / tiles_n;
    tn = pid - tm * tiles_n;
}

// Epilogue staging layout (all kernels).  A wave stages a 32-row block of
// its sub-tile in unpadded rows of WTN fp16, in 8-byte slots (four
// consecutive columns, what one lane holds per accumulator piece); slot s of
// row r is stored at slot s ^ (r & 15).  On gfx950 (measured with the LDS
// bank-conflict counter on isolated access patterns) a 64-bit LDS write
// serves 16 consecutive lanes per cycle over 32 four-byte banks, and a
// 128-bit read 16 lanes per cycle over 64 banks.  A write instruction puts 16
// consecutive lanes on 16 rows (r & 15 all different) at one logical slot,
// so the XOR spreads them over 16 slot positions: all 32 banks.  A read
// lane takes the 16-byte chunk ec (slots 2 ec, 2 ec + 1) of its row, found at
// chunk ec ^ ((r & 15) >> 1) with its halves swapped when r is odd; 16
// lanes read two whole 128-byte rows (or one 256-byte row) in a permuted
// order: all 64 banks.  The earlier layouts (16-byte row padding, or a
// swizzle by (r >> 1)) put two rows of a write group on the same banks.
__device__ __forceinline__ int staged_slot(int r, int slot) { return slot ^ (r & 15); }

// alpha * acc as one fused operation with a +0 addend: the product is exact
// inside the fma and the +0 turns an exactly zero product (alpha < 0 times a
// zero sum) into +0, the value round-to-nearest gives the real sum 0; no other
// value changes.  The compiler folds it with the conversion to fp16 into
// v_fma_mixlo_f16.
__device__ __forceinline__ float scale_acc(float alpha, float acc)
{
    return __builtin_fmaf(alpha, acc, 0.0f);
}

// One 32-row block of a wave's sub-tile (its FN 32x32 accumulators, rows
// row0 .. row0+31 of the workgroup tile) to D = RNE16(alpha * acc), through
// the wave's unpadded staging area: 128-byte rows of sixteen 8-byte slots,
// slot c of row r at c ^ (r & 15) (staged_slot).  Wait for the LDS writes,
// read back 16 bytes per lane along rows (a logical 16-byte chunk is an
// aligned slot pair, halves swapped when the row's swizzle is odd) and store
// with the streaming policy.
// Lane holds D[m][n .. n+3] for m = row (lane & 31) of each block and
// n = 8 * g + 4 * (lane >> 5).  LDS runs one wave's accesses in order, so a
// later block's writes cannot overtake these reads.
template <class C>
__device__ __forceinline__ void store_block_staged(const f32x16 (&blk)[C::FN], float alpha,
                                                   char *epi, int lane,
                                                   __amdgpu_buffer_rsrc_t rd, int row0, int n,
                                                   bool n_ok, int N)
{
    static_assert(C::WTN == 64, "128-byte staging rows");
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    const int half = lane >> 5;
    const int wr = lane & 31;
    const int wsw = wr & 15;
#pragma unroll
    for (int j = 0; j < C::FN; ++j)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            const f32x16 &a = blk[j];
            u32x2 packed;
            packed[0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)scale_acc(alpha, a[4 * g + 0])) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)scale_acc(alpha, a[4 * g + 1])) << 16);
            packed[1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)scale_acc(alpha, a[4 * g + 2])) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)scale_acc(alpha, a[4 * g + 3])) << 16);
            const int slot8 = (8 * j + 2 * g + half) ^ wsw;
            *(u32x2 *)(epi + wr * 128 + slot8 * 8) = packed;
        }
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
    compiler_fence();
    const int ec = lane & 7;                           // 16-byte chunk of the row
#pragma unroll
    for (int it = 0; it < 4; ++it) {
        const int r = it * 8 + (lane >> 3);
        const int sw = r & 15;
        u32x4 v = *(const u32x4 *)(epi + r * 128 + ((ec ^ (sw >> 1)) << 4));
        if (sw & 1) v = u32x4{v[2], v[3], v[0], v[1]};
        const uint32_t off = n_ok ? (uint32_t)((row0 + r) * N + n) * 2u : kOutOfRange;
        __builtin_amdgcn_raw_buffer_store_b128(v, rd, off, 0, kStoreStreaming);
    }
    compiler_fence();
}

// Work of a split-K launch (the library runs it on schedules 10 and 12).  Grid positions below
// dp_tiles compute whole output tiles, as the tiled kernel does.  The
// remaining L = tiles - dp_tiles output tiles are each cut into `splits`
// contiguous runs of K tiles; run p of cut tile t is grid position
// dp_tiles + q, where the pieces are numbered q' = p * L + t (K run first)
// and q' is dealt to the 8 XCDs in contiguous blocks, so an XCD's pieces
// share one K run and neighbouring output tiles.  Each piece writes its fp32
// partial tile, row-major, to part[(t * splits + p) * BM * BN ...] and ends;
// split_reduce_kernel, launched after it on the same stream, adds the runs
// of every cut tile in run order and writes D.
struct SplitWork {
    float *part;          // L * splits partial tiles of BM * BN fp32
    int dp_tiles;
    int splits;
};

// The mainloop and epilogue of one workgroup (or, for a split piece, the
// mainloop and the write of its partial tile).  SUB: the workgroup computes
// one 128x128 quarter of a 256x256 output tile whose linear id in the
// grouped walk is sw.dp_tiles or later (the remainder of a grid whose whole
// rounds ran as 256x256 tiles; see gemm_tn_sub_kernel).
template <class C, bool SPLIT, bool SUB = false>
__device__ __forceinline__ void gemm_tn_body(const _Float16 *__restrict__ A,
                                             const _Float16 *__restrict__ B, const _Float16 *Cm,
                                             _Float16 *D, int M, int N, int K, float alpha,
                                             float beta, const SplitWork &sw)
{
    static_assert(C::SCHED <= 2 || C::SCHED >= 5, "schedules 3 and 4 have kernels of their own");
    static_assert(!SPLIT || C::ORDER == 8 || C::ORDER >= 10,
                  "split-K runs the split-load ping-pong or a one-wave schedule");
    // Cm and D may be the same buffer (in-place D = alpha A B^T + beta D): each
    // wave reads C only inside its own sub-tile and finishes those reads
    // before it stores, so they are not declared __restrict__.
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / C::WN;
    const int wn = wave % C::WN;

    const int tiles_m = (M + C::BM - 1) / C::BM;
    const int tiles_n = (N + C::BN - 1) / C::BN;
    const int ntile = (K + C::BK - 1) / C::BK;
    // This workgroup's output tile (linear id in the grouped walk) and its
    // run of K tiles [kfirst, kfirst + nk).
    int tile_id = blockIdx.x;
    // the XCD renumbering spans the whole grid, or (gemm_tn_dp_kernel) the
    // first sw.dp_tiles tiles that its grid covers
    int renumber = (!SPLIT && !SUB && sw.dp_tiles > 0) ? sw.dp_tiles : tiles_m * tiles_n;
    int kfirst = 0, nk = ntile;
    bool partial = false;
    int krun = 0, ltile = 0;
    if constexpr (SPLIT) {
        renumber = sw.dp_tiles;
        if ((int)blockIdx.x >= sw.dp_tiles) {
            const int L = tiles_m * tiles_n - sw.dp_tiles;
            const int G = L * sw.splits;
            int q = blockIdx.x - sw.dp_tiles;
            if ((G & 7) == 0) q = (q & 7) * (G >> 3) + (q >> 3);
            krun = q / L;
            ltile = q - krun * L;
            tile_id = sw.dp_tiles + ltile;
            renumber = 0;
            kfirst = (int)((long long)krun * ntile / sw.splits);
            nk = (int)((long long)(krun + 1) * ntile / sw.splits) - kfirst;
            partial = true;
        }
    }
    int tm, tn;
    tile_coords(tile_id, tiles_m, tiles_n, renumber, tm, tn);
    int m0v = tm * C::BM, n0v = tn * C::BN;
    if constexpr (SUB) {
        static_assert(!SPLIT && C::BM == 128 && C::BN == 128, "quarters of 256x256 tiles");
        // quarter q of remainder tile sw.dp_tiles + q / 4; the four quarters
        // of a tile go to one XCD (contiguous runs per XCD, as in tile_coords)
        const int G = gridDim.x;
        int q = blockIdx.x;
        if ((G & 7) == 0) q = (q & 7) * (G >> 3) + (q >> 3);
        int pm, pn;
        tile_coords(sw.dp_tiles + q / 4, (M + 255) / 256, (N + 255) / 256, 0, pm, pn);
        m0v = pm * 256 + 128 * ((q >> 1) & 1);
        n0v = pn * 256 + 128 * (q & 1);
        if (m0v >= M || n0v >= N) return;          // a quarter past the edge: nothing to do
    }
    const int m0 = m0v;
    const int n0 = n0v;
    const int rows_a = (M - m0 < C::BM) ? (M - m0) : C::BM;
    const int rows_b = (N - n0 < C::BN) ? (N - n0) : C::BN;

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)rows_a * K * 2u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (size_t)n0 * K, (uint32_t)rows_b * K * 2u);

    // K tiles run in order from kfirst (0 unless this is a split piece).
    const int kt0 = kfirst;

    // ---- per-lane LDS-DMA source offsets.  Wave load i of an operand fills
    // LDS chunks q = (i*NW + wave)*64 + lane: row r = q / CPR, position
    // q % CPR, holding logical chunk c = position ^ swz(r).  64/CPR rows per
    // load; r mod 16 (all swz depends on) is the same for every i when
    // 64/CPR >= 16 or NW is even, so c is fixed per lane and the source
    // offset of load i is base + i * (NW * 64/CPR) rows.
    constexpr int ROWS_PER_LOAD = 64 / C::CPR;
    static_assert(ROWS_PER_LOAD >= 16 || C::NW % 2 == 0, "swizzle fixed across a wave's loads");
    const int l_row0 = wave * ROWS_PER_LOAD + lane / C::CPR;
    const int l_chunk = (lane % C::CPR) ^ swz<C::CPR>(l_row0);
    const uint32_t l_base = (uint32_t)(l_row0 * K + l_chunk * 8) * 2u;
    const uint32_t l_step = (uint32_t)(C::NW * ROWS_PER_LOAD) * (uint32_t)K * 2u;

    // Issue the L loads of K tile `t` into ring slot `slot`.
    auto issue = [&](int t, int slot) {
        const int kbase = (t + kt0) * C::BK;
        // K-tail: this lane's chunk lies past K -> an offset past the range
        // (reads 0); its later loads keep that offset (step 0).
        const bool valid = l_chunk * 8 < K - kbase;
        const uint32_t v = valid ? l_base + (uint32_t)kbase * 2u : kOutOfRange;
        const uint32_t step = valid ? l_step : 0u;
        char *sa = smem + slot * C::STAGE_BYTES;
        char *sb = sa + C::A_BYTES;
#pragma unroll
        for (int i = 0; i < C::NA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void *)(sa + (i * C::NW + wave) * 1024),
                16, v + (uint32_t)i * step, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < C::NB; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (__attribute__((address_space(3))) void *)(sb + (i * C::NW + wave) * 1024),
                16, v + (uint32_t)i * step, 0, 0, 0);
    };

    // ---- per-lane fragment read offsets within a slot (bytes), per MFMA K step
    // 32x32x16: lane reads row lane % 32 of a block, 8-wide K group lane / 32;
    // 16x16x32: row lane % 16, K group lane / 16 (four per 32-deep step)
    const int half = lane >> 5;
    const int ra_row = wm * C::WTM + (lane & (C::MB - 1));
    const int rb_row = wn * C::WTN + (lane & (C::MB - 1));
    int fa[C::NKS], fb[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
        const int c = C::MF16 ? 4 * ks + (lane >> 4) : 2 * ks + half;
        fa[ks] = ra_row * C::RB + ((c ^ swz<C::CPR>(ra_row)) << 4);
        fb[ks] = C::A_BYTES + rb_row * C::RB + ((c ^ swz<C::CPR>(rb_row)) << 4);
    }

    using Acc = std::conditional_t<C::MF16, f32x4v, f32x16>;
    constexpr int ACC_N = C::MF16 ? 4 : 16;
    Acc acc[C::AM][C::AN];
#pragma unroll
    for (int i = 0; i < C::AM; ++i)
#pragma unroll
        for (int j = 0; j < C::AN; ++j)
#pragma unroll
            for (int e = 0; e < ACC_N; ++e) acc[i][j][e] = 0.0f;

    // LDS -> VGPR fragments of one MFMA K step, and the MFMAs of one K step.
    // Read order follows first use by mfma_step: A0, all of B, then A1...
    auto read_frags_ab = [&](f16x8 (&ra)[C::AM], f16x8 (&rb)[C::AN], const char *abase,
                             const char *bbase, int ks) {
        ra[0] = *(const f16x8 *)(abase + fa[ks]);
#pragma unroll
        for (int j = 0; j < C::AN; ++j)
            rb[j] = *(const f16x8 *)(bbase + fb[ks] + j * C::MB * C::RB);
#pragma unroll
        for (int i = 1; i < C::AM; ++i)
            ra[i] = *(const f16x8 *)(abase + fa[ks] + i * C::MB * C::RB);
    };
    auto read_frags = [&](f16x8 (&ra)[C::AM], f16x8 (&rb)[C::AN], const char *sbase, int ks) {
        read_frags_ab(ra, rb, sbase, sbase, ks);
    };
    auto mfma_step = [&](const f16x8 (&ra)[C::AM], const f16x8 (&rb)[C::AN]) {
#pragma unroll
        for (int i = 0; i < C::AM; ++i)
#pragma unroll
            for (int j = 0; j < C::AN; ++j) {
                if constexpr (C::MF16)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(rb[j], ra[i], acc[i][j], 0, 0, 0);
                else
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(rb[j], ra[i], acc[i][j], 0, 0, 0);
            }
    };
    // Wait for this lane's loads of tile `t` (and its own LDS reads), then a
    // workgroup barrier: tile t is visible to every wave and every read
    // issued before the barrier has completed.
    auto sync_tile = [&](int t) {
        int after = ntile - 1 - t;
        if (after > C::S - 2) after = C::S - 2;
        compiler_fence();
        __builtin_amdgcn_sched_barrier(0);
        wait_tile<C>(after);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        compiler_fence();
    };

    // The same with a compile-time count of later tiles in flight (steady
    // state: always S-2), so no branch splits the scheduling region.
    auto sync_tile_steady = [&]() {
        compiler_fence();
        __builtin_amdgcn_sched_barrier(0);
        wait_vm_lgkm0<(C::S - 2) * C::L>();
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        compiler_fence();
    };

    // ---- prologue: tiles 0 .. S-2 (order 8 has a prologue of its own)
    if constexpr (C::ORDER != 8 && C::ORDER < 10) {
#pragma unroll
        for (int t = 0; t < C::S - 1; ++t)
            if (t < ntile) issue(t, t);
    }

    int slot = 0;                                    // slot of tile k
    int wslot = C::S - 1;                            // slot of tile k+S-1
    if constexpr (C::ORDER == 0) {
        // ---- "Lesson 6" three-phase order: wait, barrier, refill, compute.
#pragma unroll 1
        for (int k = 0; k < ntile; ++k) {
            sync_tile(k);
            if (k + C::S - 1 < ntile) issue(k + C::S - 1, wslot);
            const char *sbase = smem + slot * C::STAGE_BYTES;
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
                f16x8 ra[C::AM], rb[C::AN];
                read_frags(ra, rb, sbase, ks);
                mfma_step(ra, rb);
            }
            slot = (slot + 1 == C::S) ? 0 : slot + 1;
            wslot = (wslot + 1 == C::S) ? 0 : wslot + 1;
        }
    } else if constexpr (C::ORDER == 2) {
        // ---- Ping-pong.  The two waves sharing a SIMD belong to different
        // groups (waves are dealt to SIMDs round-robin): G0 = waves 0..NG-1,
        // G1 = waves NG..NW-1.  Time is cut into phases, each ending in one
        // workgroup barrier.  In every phase one group issues all MFMAs of a
        // K tile from registers (C) while the other reads all fragments of
        // its next K tile from LDS (M), so each SIMD's matrix pipe is fed by
        // one wave while the other wave's LDS traffic is in flight:
        //     phase:  0      1      2      3    ...  2n-1    2n
        //     G0:    M(0)   C(0)   M(1)   C(1)  ...  C(n-1)  idle
        //     G1:    idle   M(0)   C(0)   M(1)  ...  M(n-1)  C(n-1)
        // Ring (two slots): tile j lives in slot j%2.  G0 refills at the start
        // of M(j) (phase 2j): tile j+1 into slot (j+1)%2, whose previous tile
        // j-1 was last read in phases 2j-2 (G0) and 2j-1 (G1), each closed by
        // lgkmcnt(0) + barrier (WAR).  G0 waits vmcnt(0) at the end of C(j),
        // so tile j+1 is complete before the barrier that opens phase 2j+2,
        // where it is first read (RAW).  Tile 0 is loaded by all waves before
        // the loop.  Every wave executes 2n+2 barriers.
        constexpr int NG = C::NW / 2;
        const int grp = wave / NG;                 // wave-uniform
        const int gw = wave - grp * NG;
        constexpr int NAG = C::BM * C::CPR / (64 * NG);
        constexpr int NBG = C::BN * C::CPR / (64 * NG);
        static_assert(NAG * 64 * NG == C::BM * C::CPR && NBG * 64 * NG == C::BN * C::CPR, "split");
        // Loader lane -> LDS chunk q = (i*NG + gw)*64 + lane: row
        // r = (i*NG + gw)*8 + lane/8, position lane%8.  NG is even, so r mod 16
        // and hence the swizzle do not depend on i: one base offset per
        // operand, advanced by NG*8 rows per load.
        const int pr0 = gw * 8 + (lane >> 3);
        const int pc = (lane & 7) ^ swz<C::CPR>(pr0);
        const uint32_t p_base = (uint32_t)(pr0 * K + pc * 8) * 2u;
        const uint32_t p_step = (uint32_t)(NG * 8) * (uint32_t)K * 2u;
        auto issue_g0 = [&](int t, int slot) {
            const int kbase = (t + kt0) * C::BK;
            const bool valid = pc * 8 < K - kbase;
            uint32_t v = valid ? p_base + (uint32_t)kbase * 2u : kOutOfRange;
            const uint32_t step = valid ? p_step : 0u;
            char *sa = smem + slot * C::STAGE_BYTES;
            char *sb = sa + C::A_BYTES;
#pragma unroll
            for (int i = 0; i < NAG; ++i) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ra, (__attribute__((address_space(3))) void *)(sa + (i * NG + gw) * 1024),
                    16, v + (uint32_t)i * step, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < NBG; ++i) {
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rb, (__attribute__((address_space(3))) void *)(sb + (i * NG + gw) * 1024),
                    16, v + (uint32_t)i * step, 0, 0, 0);
            }
        };
        auto barrier = [&]() {
            compiler_fence();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            compiler_fence();
        };
        f16x8 fra[C::NKS][C::AM], frb[C::NKS][C::AN];
        // tile 0 (already issued by the prologue) complete and visible
        compiler_fence();
        wait_vm_lgkm0<0>();
        barrier();
        if (grp == 1) barrier();                   // G1 idles in phase 0
#pragma unroll 1
        for (int j = 0; j < ntile; ++j) {
            // M(j)
            if (grp == 0 && j + 1 < ntile) issue_g0(j + 1, (j + 1) & 1);
            const char *sbase = smem + (j & 1) * C::STAGE_BYTES;
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) read_frags(fra[ks], frb[ks], sbase, ks);
            compiler_fence();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
            barrier();
            // C(j).  The computing wave runs at raised priority so that the
            // SIMD's issue arbiter prefers its MFMAs over the other wave's
            // LDS/VMEM traffic (measured: +15% at 8192^3).
            __builtin_amdgcn_s_setprio(1);
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) mfma_step(fra[ks], frb[ks]);
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_setprio(0);
            if (grp == 0) __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
            barrier();
        }
        if (grp == 0) barrier();                   // G0 idles in the last phase
    } else if constexpr (C::ORDER == 14) {
        // ---- Order 10 on a 128x128 tile: four waves of 64x64 (4x4 blocks of
        // 16x16x32 MFMAs, 16 per 32-deep half tile), 64-deep K tiles in a ring
        // of four 32 KiB slots, one barrier per tile between its halves.  Tile
        // k + 3 refills the slot tile k - 1 left, its A loads in the first half
        // of tile k and its B loads in the second (onewave128_mainloop.inc,
        // written by gen_onewave_mainloop.py).
        static_assert(C::AM == 4 && C::AN == 4 && C::NKS == 2 && C::NA == 4 && C::NB == 4,
                      "the assembly is written for 4x4 MFMA blocks and 4 + 4 loads per wave");
        static_assert(C::STAGE_BYTES == 32768 && C::A_BYTES == 16384, "slot layout of the assembly");
        const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) char *)smem);
        const u32x4 rwa = rsrc_words(A + (size_t)m0 * K, (uint32_t)rows_a * K * 2u);
        const u32x4 rwb = rsrc_words(B + (size_t)n0 * K, (uint32_t)rows_b * K * 2u);
        // this lane's first fragment of each slot and K step (fb holds + A_BYTES)
        constexpr uint32_t SB = C::STAGE_BYTES;
        const uint32_t rA00 = lds0 + fa[0], rA01 = lds0 + fa[1];
        const uint32_t rA10 = rA00 + SB, rA11 = rA01 + SB, rA20 = rA00 + 2 * SB, rA21 = rA01 + 2 * SB;
        const uint32_t rA30 = rA00 + 3 * SB, rA31 = rA01 + 3 * SB;
        const uint32_t rB00 = lds0 + fb[0], rB01 = lds0 + fb[1];
        const uint32_t rB10 = rB00 + SB, rB11 = rB01 + SB, rB20 = rB00 + 2 * SB, rB21 = rB01 + 2 * SB;
        const uint32_t rB30 = rB00 + 3 * SB, rB31 = rB01 + 3 * SB;
        const uint32_t lbase = l_base + (uint32_t)kt0 * (uint32_t)(C::BK * 2);
        const uint32_t lch8 = (uint32_t)(l_chunk * 8), lstep = l_step;
        const uint32_t oor = kOutOfRange;
        const uint32_t wb = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)wave * 1024u);
        const uint32_t ow_nk = __builtin_amdgcn_readfirstlane(nk);
        const uint32_t ow_kk = __builtin_amdgcn_readfirstlane(K - kt0 * C::BK);
        f16x8 xa[4], xb[4], ya[4], yb[4];
        uint32_t o0, o1, o2, o3, vs, sk, st, se;
#include "onewave128_mainloop.inc"
    } else if constexpr (C::ORDER >= 10) {
        // ---- One wave per SIMD, 128x128 of the tile each, 64-deep K tiles,
        // one barrier per K tile between its two 32-deep halves: the ring
        // protocol of "cute(9) multistage_gemm" (section 6) with the minimum
        // ring of "Lesson 6" (section 4, S = 2: a tile's copy takes about as
        // long as its MFMAs).  Order 10 keeps A and B in two slots; order 11
        // gives B a third slot and loads it three tiles ahead; order 12 loads
        // B two tiles ahead in the first half of each tile, so each half
        // issues 8 loads per wave instead of 16.  With a single wave per SIMD
        // nothing else hides an instruction that is not an MFMA, so the loop
        // is one inline-assembly statement in which every fragment read,
        // LDS-DMA load and address update sits between two MFMAs
        // (onewave_mainloop.inc, onewave_b3_mainloop.inc and
        // onewave_b3h_mainloop.inc, written by gen_onewave_mainloop.py, which
        // gives the schedule, the wait counts and the hazards it covers).
        // The accumulators stay in the 256 AGPRs,
        // which leaves the VGPRs to two fragment buffers of a 32-deep step
        // each.  Tile t's loads use the same lane-to-LDS mapping and K-tail
        // handling as `issue` above, computed in the loop.
        static_assert(C::AM == 8 && C::AN == 8 && C::NKS == 2 && C::NA == 8 && C::NB == 8,
                      "the assembly is written for 8x8 MFMA blocks and 8 + 8 loads per wave");
        static_assert(C::A_BYTES == 32768 && C::B_BYTES == 32768, "slot layout of the assembly");
        const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(
            (__attribute__((address_space(3))) char *)smem);
        const u32x4 rwa = rsrc_words(A + (size_t)m0 * K, (uint32_t)rows_a * K * 2u);
        const u32x4 rwb = rsrc_words(B + (size_t)n0 * K, (uint32_t)rows_b * K * 2u);
        // This lane's first fragment of each slot and K step.  fa / fb are
        // offsets within a stage of A rows then B rows (fb includes A_BYTES).
        // Order 10: slot s is the stage at s * STAGE_BYTES.  Orders 11 and 12:
        // two A slots of A_BYTES, then three B slots of B_BYTES.
        constexpr uint32_t A_SLOT = C::ORDER == 10 ? C::STAGE_BYTES : C::A_BYTES;
        constexpr uint32_t B_FIRST = C::ORDER == 10 ? 0u : (uint32_t)C::A_BYTES;
        constexpr uint32_t B_SLOT = C::ORDER == 10 ? C::STAGE_BYTES : C::B_BYTES;
        const uint32_t rA00 = lds0 + fa[0], rA01 = lds0 + fa[1];
        const uint32_t rA10 = rA00 + A_SLOT, rA11 = rA01 + A_SLOT;
        const uint32_t rB00 = lds0 + fb[0] + B_FIRST, rB01 = lds0 + fb[1] + B_FIRST;
        const uint32_t rB10 = rB00 + B_SLOT, rB11 = rB01 + B_SLOT;
        const uint32_t rB20 = rB10 + B_SLOT, rB21 = rB11 + B_SLOT;
        // The statement counts K tiles from 0: a split piece's first tile kt0
        // enters as a shifted source offset and a shorter K.
        const uint32_t lbase = l_base + (uint32_t)kt0 * (uint32_t)(C::BK * 2);
        const uint32_t lch8 = (uint32_t)(l_chunk * 8), lstep = l_step;
        const uint32_t oor = kOutOfRange;
        const uint32_t wb = __builtin_amdgcn_readfirstlane(lds0 + (uint32_t)wave * 1024u);
        const uint32_t ow_nk = __builtin_amdgcn_readfirstlane(nk);
        const uint32_t ow_kk = __builtin_amdgcn_readfirstlane(K - kt0 * C::BK);
        f16x8 xa[8], xb[8], ya[8], yb[8];
        uint32_t o0, o1, o2, o3, o4, o5, o6, o7, vs, sk, st, se;
        if constexpr (C::ORDER == 10) {
            (void)rB20;
            (void)rB21;
#include "onewave_mainloop.inc"
        } else if constexpr (C::ORDER == 11) {
            uint32_t p0, p1, p2, p3, p4, p5, p6, p7, ps;
#include "onewave_b3_mainloop.inc"
        } else {
            uint32_t p0, p1, p2, p3, p4, p5, p6, p7, ps;
#include "onewave_b3h_mainloop.inc"
        }
    } else if constexpr (C::ORDER == 8) {
        // ---- Ping-pong with the loads split between the groups.  The phases
        // are those of order 2, but G0 loads only A tiles and G1 only B
        // tiles, each group at the start of its own read phase, before its
        // fragment reads, so each read phase issues half of a tile's LDS-DMA
        // and the loads get the whole phase to travel (measured 1-1.5 %
        // faster at 4096^3 and 8192^3 than issuing them after the reads).
        // (In order 2, G0 issues the whole tile: the LDS-DMA path accepts an
        // instruction only as fast as it moves 16 bytes per lane, so those
        // issues held G0's read phase well past the other group's MFMAs.)
        // A ring: two slots, tile j in slot j % 2.  B ring: three slots,
        // tile j in slot j % 3.  Every slot a read phase refills was last
        // read before the barrier that opens the phase.
        //   G0, read phase of tile j (phase 2j): A(j+1) into slot (j+1) % 2,
        //     which held A(j-1), last read in phases 2j-2 and 2j-1 (WAR);
        //     complete by G0's vmcnt(0) at the end of phase 2j+1 (RAW:
        //     first read in phase 2j+2).
        //   G1, read phase of tile j (phase 2j+1): B(j+2) into slot
        //     (j+2) % 3, which held B(j-1), last read in phases 2j-2 and
        //     2j-1 (WAR); B(j+1), issued one read phase earlier, complete by
        //     the vmcnt at the end of this phase (RAW: first read in phase
        //     2j+2), B(j+2) may stay in flight.
        // The prologue loads A(0), B(0) and B(1).
        constexpr int NG = C::NW / 2;
        const int grp = wave / NG;                 // wave-uniform
        const int gw = wave - grp * NG;
        constexpr int NLG = C::BM * C::CPR / (64 * NG);   // loads per wave per operand tile
        static_assert(NLG * 64 * NG == C::BM * C::CPR, "split");
        const int pr0 = gw * 8 + (lane >> 3);
        const int pc = (lane & 7) ^ swz<C::CPR>(pr0);
        const uint32_t p_base = (uint32_t)(pr0 * K + pc * 8) * 2u;
        const uint32_t p_step = (uint32_t)(NG * 8) * (uint32_t)K * 2u;
        char *const b_ring = smem + 2 * C::A_BYTES;
        // Operand tile t (the t-th of this workgroup's nk K tiles) of `rs`
        // into `dst` by this group's waves.
        auto issue_op = [&](const __amdgpu_buffer_rsrc_t &rs, int t, char *dst) {
            const int kbase = (t + kt0) * C::BK;
            const bool valid = pc * 8 < K - kbase;
            const uint32_t v = valid ? p_base + (uint32_t)kbase * 2u : kOutOfRange;
            const uint32_t step = valid ? p_step : 0u;
#pragma unroll
            for (int i = 0; i < NLG; ++i)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (__attribute__((address_space(3))) void *)(dst + (i * NG + gw) * 1024),
                    16, v + (uint32_t)i * step, 0, 0, 0);
        };
        auto barrier = [&]() {
            compiler_fence();
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_barrier();
            __builtin_amdgcn_sched_barrier(0);
            compiler_fence();
        };
        if (nk > 0) {
            if (grp == 0) {
                issue_op(ra, 0, smem);
            } else {
                issue_op(rb, 0, b_ring);
                if (nk > 1) issue_op(rb, 1, b_ring + C::B_BYTES);
            }
        }
        f16x8 fra[C::NKS][C::AM], frb[C::NKS][C::AN];
        compiler_fence();
        wait_vm_lgkm0<0>();
        barrier();
        if (grp == 1) barrier();                   // G1 idles in phase 0
        int bslot = 0;                             // B slot of tile j
#pragma unroll 1
        for (int j = 0; j < nk; ++j) {
            // read phase of tile j: this group's loads, then its fragments
            const char *abase = smem + (j & 1) * C::A_BYTES;
            const char *bbase = b_ring - C::A_BYTES + bslot * C::B_BYTES;   // fb holds + A_BYTES
            const int b2 = bslot == 0 ? 2 : bslot - 1;   // (j + 2) % 3
            if (grp == 0 && j + 1 < nk) issue_op(ra, j + 1, smem + ((j + 1) & 1) * C::A_BYTES);
            if (grp == 1 && j + 2 < nk) issue_op(rb, j + 2, b_ring + b2 * C::B_BYTES);
            compiler_fence();
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) read_frags_ab(fra[ks], frb[ks], abase, bbase, ks);
            compiler_fence();
            __builtin_amdgcn_sched_barrier(0);
            // this wave's fragments; for G1 also B(j+1), while B(j+2) may
            // stay in flight
            if (grp == 0)
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));
            else if (j + 2 < nk)
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(NLG, 0));
            else
                __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
            barrier();
            // MFMA phase of tile j.  (No raised priority as in order 2: the
            // reading wave has finished its issues by the time it would
            // compete, and the priority switches measured 0.4-0.7 % slower.)
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) mfma_step(fra[ks], frb[ks]);
            __builtin_amdgcn_sched_barrier(0);
            if (grp == 0) __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
            barrier();
            bslot = bslot == 2 ? 0 : bslot + 1;
        }
        if (grp == 0) barrier();                   // G0 idles in the last phase
    } else {
        // ---- "cute(9) multistage_gemm" order (sections 6.2, 9): fragments are
        // double-buffered in VGPRs; step ks reads step ks+1 while its MFMAs
        // run.  At the last K step of tile k the wave waits for tile k+1,
        // barriers, and prefetches tile k+1's first step before issuing the
        // last MFMAs of tile k, so LDS latency hides under them.  The refill
        // of slot (k-1) mod S is issued at the first step of tile k: every
        // read of that slot was issued before the previous barrier.
        f16x8 ra0[C::AM], rb0[C::AN], ra1[C::AM], rb1[C::AN];
        // One K tile.  MODE: 2 = steady state (a next tile exists and tile
        // k+S-1 is issued), 1 = drain (a next tile exists, nothing issued),
        // 0 = the last tile.  The modes are separate loops so that every K
        // step is one branch-free scheduling region: a branch joining the
        // barrier path would make the compiler wait for the prefetched reads
        // before the remaining MFMAs.  Within a step the MFMAs are interleaved
        // one by one with the LDS reads and LDS-DMA issues.
        auto tile = [&](int k, auto mode) {
            constexpr int MODE = decltype(mode)::value;
            const char *sbase = smem + slot * C::STAGE_BYTES;
            const int nslot = (slot + 1 == C::S) ? 0 : slot + 1;
#pragma unroll
            for (int ks = 0; ks < C::NKS; ++ks) {
                // NKS is even, so step ks uses buffer ks & 1 in every tile
                f16x8(&cra)[C::AM] = (ks & 1) ? ra1 : ra0;
                f16x8(&crb)[C::AN] = (ks & 1) ? rb1 : rb0;
                f16x8(&nra)[C::AM] = (ks & 1) ? ra0 : ra1;
                f16x8(&nrb)[C::AN] = (ks & 1) ? rb0 : rb1;
                int nreads = C::AM + C::AN;
                if (ks == C::NKS - 1) {
                    if constexpr (MODE == 2) {
                        sync_tile_steady();
                    } else if constexpr (MODE == 1) {
                        sync_tile(k + 1);
                    } else {
                        nreads = 0;
                    }
                    if constexpr (MODE != 0)
                        read_frags(nra, nrb, smem + nslot * C::STAGE_BYTES, 0);
                } else {
                    read_frags(nra, nrb, sbase, ks + 1);
                }
                int nissue = 0;
                if constexpr (MODE == 2) {
                    if (ks == 0) {
                        issue(k + C::S - 1, wslot);
                        nissue = C::L;
                    }
                }
                mfma_step(cra, crb);
                // order: LDS read, MFMA, [LDS-DMA], LDS read, MFMA, ...
#pragma unroll
                for (int m = 0; m < C::AM * C::AN; ++m) {
                    if (m < nreads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    if (m < nissue) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
                }
                __builtin_amdgcn_sched_barrier(0);
            }
            slot = nslot;
            wslot = (wslot + 1 == C::S) ? 0 : wslot + 1;
        };
        if (ntile > 0) {
            sync_tile(0);
            read_frags(ra0, rb0, smem, 0);
            int k = 0;
#pragma unroll 1
            for (; k < ntile - (C::S - 1); ++k) tile(k, std::integral_constant<int, 2>{});
#pragma unroll 1
            for (; k < ntile - 1; ++k) tile(k, std::integral_constant<int, 1>{});
            tile(ntile - 1, std::integral_constant<int, 0>{});
        }
    }

    // ---- split-K piece: its fp32 partial tile, row-major, and done.  The
    // stores take the default cache policy: the reduction kernel reads the
    // partials right after this launch, and with the streaming policy of the
    // epilogue the call measured 1-2 % slower (2048^2 x 8192 and x 16384,
    // 6144^2 x 4096, four runs).
    // Block (i, j) of a wave holds rows 16 i + (lane % 16) and columns
    // 16 j + 4 (lane / 16) .. + 3 of the wave's sub-tile (operands swapped,
    // as in the epilogue): 64-byte row pieces of 16 rows per instruction.
    if constexpr (SPLIT) {
        if (partial) {
            const __amdgpu_buffer_rsrc_t rw = make_rsrc(
                sw.part + (size_t)(ltile * sw.splits + krun) * (C::BM * C::BN),
                (uint32_t)(C::BM * C::BN * 4));
            const int r0 = wm * C::WTM + (lane & 15);
            const int c0 = wn * C::WTN + 4 * (lane >> 4);
#pragma unroll
            for (int i = 0; i < C::AM; ++i)
#pragma unroll
                for (int j = 0; j < C::AN; ++j)
                    __builtin_amdgcn_raw_buffer_store_b128(
                        __builtin_bit_cast(u32x4, acc[i][j]), rw,
                        (uint32_t)(((r0 + 16 * i) * C::BN + c0 + 16 * j) * 4), 0, 0);
            return;
        }
    }

    // ---- epilogue ("cute(9) multistage_gemm", section 7.2: registers ->
    // shared memory -> global, so the global writes are row-contiguous).
    // Lane holds D[m][n .. n+3]: 4 consecutive columns of one row per
    // accumulator group (the pieces below).  Per 32-row block i of its sub-tile, each
    // wave converts alpha * acc (+ beta * C) to fp16 (one rounding), writes
    // the block into a private LDS region, waits for those writes, reads it
    // back row by row and stores 16 bytes per lane: every store instruction
    // covers whole row segments of WTN * 2 bytes, and block i's stores drain
    // while block i + 1 is converted (measured -8 % time on 4096x4096x128
    // against staging the whole sub-tile first).  LDS executes one wave's
    // accesses in order, so block i + 1's writes cannot overtake block i's
    // reads.
    compiler_fence();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();                 // every wave is done with the ring
    __builtin_amdgcn_sched_barrier(0);
    compiler_fence();
    char *epi = smem + wave * C::EPI_WAVE_BYTES;
    // four consecutive columns c .. c + 3 (c % 4 == 0) of block row r: one
    // 8-byte slot, at the swizzled position (staged_slot)
    auto stage4 = [&](int r, int c, float v0, float v1, float v2, float v3) {
        u32x2 packed;
        packed[0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v0) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v1) << 16);
        packed[1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v2) |
                    ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v3) << 16);
        *(u32x2 *)(epi + r * C::EPI_ROW + staged_slot(r, c >> 2) * 8) = packed;
    };
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    constexpr int CPRW = C::EPI_CHUNKS_PER_ROW;        // 16-byte chunks per sub-tile row
    constexpr int RPI = C::EPI_ROWS_PER_STORE;         // rows per wave instruction
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(D + (size_t)m0 * N, (uint32_t)rows_a * N * 2u);
    const int ec = lane % CPRW;
    const int n_st = n0 + wn * C::WTN + ec * 8;
    const bool n_ok = n_st < N;                        // N % 8 == 0: a chunk is all in or out
    const bool with_c = beta != 0.0f;
    const __amdgpu_buffer_rsrc_t rc =
        make_rsrc(with_c ? Cm + (size_t)m0 * N : D, with_c ? (uint32_t)rows_a * N * 2u : 0u);
    // Piece p (4 per 32-column group) of 32-row block i: this lane's row r of
    // the block, column c of the wave's sub-tile and its 4 accumulators.
    // 32x32 blocks: p = (j, g), r = lane % 32, c = 32 j + 8 g + 4 half.
    // 16x16 blocks: p = (h, jj) over the block's two 16-row halves and the
    // 16-column groups, r = 16 h + lane % 16, c = 16 jj + 4 (lane / 16).
    constexpr int PIECES = 4 * C::FN;
    auto piece = [&](int i, int p, int &r, int &c, float (&v)[4]) {
        if constexpr (C::MF16) {
            const int hh = p / C::AN, jj = p % C::AN;
            r = 16 * hh + (lane & 15);
            c = 16 * jj + 4 * (lane >> 4);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[2 * i + hh][jj][e];
        } else {
            const int j = p / 4, g = p % 4;
            r = lane & 31;
            c = 32 * j + 8 * g + 4 * half;
#pragma unroll
            for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * g + e];
        }
    };
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        if (!with_c) {
            // D = RNE16(alpha * acc): one rounding of the exact product (the
            // compiler emits v_fma_mixlo_f16); C is not read.
#pragma unroll
            for (int p = 0; p < PIECES; ++p) {
                int r, c;
                float v[4];
                piece(i, p, r, c, v);
                stage4(r, c, scale_acc(alpha, v[0]), scale_acc(alpha, v[1]), scale_acc(alpha, v[2]),
                       scale_acc(alpha, v[3]));
            }
        } else {
            // D = RNE16(alpha * acc + beta * C) ("CUDA operator notes 2",
            // "GEMM"): C is read in the accumulator layout (4 halves per lane
            // and piece), combined in fp32 and rounded once to fp16.  Each
            // wave reads only C elements of rows it stores itself, before it
            // stores them, so C may be D (in place).
            // four pieces at a time: their C loads, then their staging
#pragma unroll
            for (int p0 = 0; p0 < PIECES; p0 += 4) {
                u32x2 cv[4];
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    int r, c;
                    float v[4];
                    piece(i, p0 + q, r, c, v);
                    const int ml = wm * C::WTM + i * 32 + r;
                    const int n = n0 + wn * C::WTN + c;
                    const uint32_t off = (n < N) ? (uint32_t)(ml * N + n) * 2u : kOutOfRange;
                    cv[q] = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rc, off, 0, 0));
                }
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    int r, c;
                    float v[4];
                    piece(i, p0 + q, r, c, v);
                    const float c0 = (float)__builtin_bit_cast(_Float16, (uint16_t)(cv[q][0] & 0xffffu));
                    const float c1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(cv[q][0] >> 16));
                    const float c2 = (float)__builtin_bit_cast(_Float16, (uint16_t)(cv[q][1] & 0xffffu));
                    const float c3 = (float)__builtin_bit_cast(_Float16, (uint16_t)(cv[q][1] >> 16));
                    // a zero product is +0 here, so an exactly zero total is +0 too
                    stage4(r, c, __builtin_fmaf(beta, c0, scale_acc(alpha, v[0])),
                           __builtin_fmaf(beta, c1, scale_acc(alpha, v[1])),
                           __builtin_fmaf(beta, c2, scale_acc(alpha, v[2])),
                           __builtin_fmaf(beta, c3, scale_acc(alpha, v[3])));
                }
            }
        }
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(63, 0));   // this wave's LDS writes landed
        compiler_fence();
#pragma unroll
        for (int it = 0; it < 32 / RPI; ++it) {
            const int rr = it * RPI + lane / CPRW;     // row within block i
            u32x4 v = *(const u32x4 *)(epi + rr * C::EPI_ROW + ((ec ^ ((rr & 15) >> 1)) << 4));
            if (rr & 1) v = u32x4{v[2], v[3], v[0], v[1]};
            const int ml = wm * C::WTM + i * 32 + rr;  // row within the workgroup tile
            const uint32_t off = n_ok ? (uint32_t)(ml * N + n_st) * 2u : kOutOfRange;
            __builtin_amdgcn_raw_buffer_store_b128(v, rd, off, 0, kStoreStreaming);
        }
        compiler_fence();
    }
}

template <class C>
__global__ void __launch_bounds__(C::T)
gemm_tn_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B,
               const _Float16 *Cm, _Float16 *D, int M, int N, int K, float alpha, float beta)
{
    gemm_tn_body<C, false>(A, B, Cm, D, M, N, K, alpha, beta, SplitWork{nullptr, 0, 1});
}

// The remainder of a grid of 256x256 output tiles whose first dp_tiles (in
// the grouped walk) ran as whole rounds elsewhere: each of the remaining
// tiles as four 128x128 quarters, one workgroup each, so a part-full last
// round fills four times as many CUs ("cute(9) multistage_gemm", section
// 11.3, names adaptive tile sizes beside split-K).  Grid: 4 x the remaining
// tiles; quarters outside M x N end at once.
template <class C>
__global__ void __launch_bounds__(C::T)
gemm_tn_sub_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B,
                   const _Float16 *Cm, _Float16 *D, int M, int N, int K, float alpha, float beta,
                   int dp_tiles)
{
    gemm_tn_body<C, false, true>(A, B, Cm, D, M, N, K, alpha, beta, SplitWork{nullptr, dp_tiles, 1});
}

// The first dp_tiles output tiles (in the grouped walk) of a grid, as the
// tiled kernel computes them: the whole rounds of a call whose remainder
// runs in gemm_tn_sub_kernel.  Grid: dp_tiles.
template <class C>
__global__ void __launch_bounds__(C::T)
gemm_tn_dp_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B,
                  const _Float16 *Cm, _Float16 *D, int M, int N, int K, float alpha, float beta,
                  int dp_tiles)
{
    gemm_tn_body<C, false>(A, B, Cm, D, M, N, K, alpha, beta, SplitWork{nullptr, dp_tiles, 1});
}

// Split-K form of schedules 8, 10, 11 and 12 (see SplitWork): D = alpha * A * B^T, no C.
template <class C>
__global__ void __launch_bounds__(C::T)
gemm_tn_split_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B,
                     _Float16 *D, int M, int N, int K, float alpha, float *part, int dp_tiles,
                     int splits)
{
    gemm_tn_body<C, true>(A, B, nullptr, D, M, N, K, alpha, 0.0f, SplitWork{part, dp_tiles, splits});
}

// Second kernel of a split-K call: for every cut tile, the sum of its runs'
// partials in run order 0 .. splits-1 (so the result does not depend on
// which run finished first), scaled by alpha and rounded once to fp16, into
// D.  Each thread handles 8 consecutive columns of one row (two 16-byte
// loads per run, one 16-byte store); BM * BN / 2048 workgroups of 256
// threads per cut tile.  Rows past M and columns past N are not stored
// (N % 8 == 0: 8 columns are all in or all out).
template <int BM, int BN>
__global__ void __launch_bounds__(256)
split_reduce_kernel(const float *__restrict__ part, _Float16 *__restrict__ D, int M, int N,
                    float alpha, int dp_tiles, int splits)
{
    constexpr int PER_TILE = BM * BN / (256 * 8);
    const int lt = blockIdx.x / PER_TILE;
    const int e = ((blockIdx.x - lt * PER_TILE) * 256 + threadIdx.x) * 8;   // element in the tile
    const int tiles_m = (M + BM - 1) / BM;
    const int tiles_n = (N + BN - 1) / BN;
    int tm, tn;
    tile_coords(dp_tiles + lt, tiles_m, tiles_n, 0, tm, tn);
    const int m = tm * BM + e / BN;
    const int n = tn * BN + e % BN;
    if (m >= M || n >= N) return;
    const f32x4v *src = reinterpret_cast<const f32x4v *>(part + (size_t)lt * splits * (BM * BN) + e);
    f32x4v lo = src[0], hi = src[1];
#pragma unroll 1
    for (int p = 1; p < splits; ++p) {
        const f32x4v *q = src + (size_t)p * (BM * BN / 4);
        lo += q[0];
        hi += q[1];
    }
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    u32x4 out;
#pragma unroll
    for (int h = 0; h < 4; ++h) {
        const float a0 = scale_acc(alpha, h < 2 ? lo[2 * h] : hi[2 * h - 4]);
        const float a1 = scale_acc(alpha, h < 2 ? lo[2 * h + 1] : hi[2 * h - 3]);
        out[h] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a0) |
                 ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)a1) << 16);
    }
    __builtin_nontemporal_store(out, reinterpret_cast<u32x4 *>(D + (size_t)m * N + n));
}

}  // namespace sg
