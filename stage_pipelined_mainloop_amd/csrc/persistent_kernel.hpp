// Persistent variant of the stage-pipelined TN GEMM (schedule 3).
//
// The grid holds as many workgroups as the CUs keep resident; workgroup w
// computes output tiles w, w + G, w + 2G, ... (G = grid size).  Its K tiles
// form ONE stream through the LDS ring: the producer runs S - 1 tiles ahead
// of the consumer across output-tile boundaries, so the first loads of
// output tile u + 1 are in flight while tile u finishes its MFMAs and its
// epilogue, and tile u's stores drain while tile u + 1 computes.  This is
// the ring of "Lesson 6" (prologue, steady state that overlaps the load of
// tile k + S - 1 with compute on tile k, drain) and the mainloop order of
// "cute(9) multistage_gemm" section 9, with the prologue and drain paid once
// per workgroup instead of once per output tile.
//
// At an output-tile boundary the next group is issued before the epilogue's
// stores (into the slot the finished tile's reads just released), so the
// in-order vmcnt lets the stores stay in flight for the next S - 1 K tiles.
// Every K tile issues the same number of loads (out-of-range fillers where
// no group is due), so one loop body serves the whole stream; the wait
// counts are persistent_wait_count, which sg_persistent_wait_count exports.
//
// The epilogue ("cute(9) multistage_gemm", section 7.2: registers -> shared
// memory -> global) stages one 32-row block of a wave's sub-tile at a time in
// a per-wave LDS area beside the ring and stores it in row-contiguous 16-byte
// pieces.  Only D = alpha * A * B^T (no C operand).
#pragma once

#include "gemm_kernel.hpp"

namespace sg {

// Four-wave workgroups are compiled for two resident per CU (at most 256
// registers per lane), so one workgroup's epilogue overlaps another's MFMAs.
template <class C>
__global__ void __launch_bounds__(C::T, C::NW == 4 ? 2 : 1)
gemm_tn_persistent_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B,
                          const _Float16 *Cm, _Float16 *D, int M, int N, int K, float alpha,
                          float beta)
{
    static_assert(C::SCHED == 3, "persistent schedule");
    (void)Cm;
    (void)beta;                                    // the launcher passes beta == 0 only
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / C::WN;
    const int wn = wave % C::WN;
    const int half = lane >> 5;

    const int tiles_m = (M + C::BM - 1) / C::BM;
    const int tiles_n = (N + C::BN - 1) / C::BN;
    const int total_tiles = tiles_m * tiles_n;
    const int G = gridDim.x;                       // the launcher keeps G <= total_tiles
    const int nu = (total_tiles - 1 - (int)blockIdx.x) / G + 1;
    const int ntile = (K + C::BK - 1) / C::BK;
    const int total = nu * ntile;                  // K tiles in this workgroup's stream

    // Output tile u of this workgroup: origin and valid rows.
    auto geometry = [&](int u, int &m0, int &n0, int &rows_a,
                        int &rows_b) __attribute__((always_inline)) {
        int tm, tn;
        short_k_coords((int)blockIdx.x + u * G, tiles_m, tiles_n, M, N, K, tm, tn);
        m0 = tm * C::BM;
        n0 = tn * C::BN;
        rows_a = (M - m0 < C::BM) ? (M - m0) : C::BM;
        rows_b = (N - n0 < C::BN) ? (N - n0) : C::BN;
    };

    // ---- epilogue of one output tile: D = RNE16(alpha * acc), one rounding,
    // one 32-row block at a time through the wave's staging area beside the
    // ring (store_block_staged; no barrier, the area is private to the wave).
    char *epi = smem + C::RING_BYTES + wave * C::EPI_BLOCK_WAVE_BYTES;
    f32x16 acc[C::FM][C::FN];
    auto zero_acc = [&]() __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
#pragma unroll
                for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;
    };
    auto epilogue = [&](int m0, int n0, int rows_a) __attribute__((always_inline)) {
        const __amdgpu_buffer_rsrc_t rd = make_rsrc(D + (size_t)m0 * N, (uint32_t)rows_a * N * 2u);
        const int n = n0 + wn * C::WTN + (lane & 7) * 8;
        const bool n_ok = n < N;                   // N % 8 == 0: a chunk is all in or out
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
            store_block_staged<C>(acc[i], alpha, epi, lane, rd, wm * C::WTM + i * 32, n, n_ok, N);
    };

    zero_acc();
    if (ntile == 0) {                              // K == 0: every output is the empty sum
        for (int u = 0; u < nu; ++u) {
            int m0, n0, rows_a, rows_b;
            geometry(u, m0, n0, rows_a, rows_b);
            epilogue(m0, n0, rows_a);
        }
        return;
    }

    // ---- LDS-DMA loader (same lane mapping as the tiled kernel): wave load
    // i of an operand fills LDS chunks q = (i*NW + wave)*64 + lane, row
    // q / CPR, position q % CPR, holding logical chunk position ^ swz(row).
    constexpr int ROWS_PER_LOAD = 64 / C::CPR;
    static_assert(ROWS_PER_LOAD >= 16 || C::NW % 2 == 0, "swizzle fixed across a wave's loads");
    const int l_row0 = wave * ROWS_PER_LOAD + lane / C::CPR;
    const int l_chunk = (lane % C::CPR) ^ swz<C::CPR>(l_row0);
    const uint32_t l_base = (uint32_t)(l_row0 * K + l_chunk * 8) * 2u;
    const uint32_t l_step = (uint32_t)(C::NW * ROWS_PER_LOAD) * (uint32_t)K * 2u;

    // Producer cursor: output tile iu, K step ik of the next group to issue.
    int iu = 0, ik = 0;
    __amdgpu_buffer_rsrc_t ira, irb;
    auto set_issue_tile = [&](int u) __attribute__((always_inline)) {
        int m0, n0, rows_a, rows_b;
        geometry(u, m0, n0, rows_a, rows_b);
        ira = make_rsrc(A + (size_t)m0 * K, (uint32_t)rows_a * K * 2u);
        irb = make_rsrc(B + (size_t)n0 * K, (uint32_t)rows_b * K * 2u);
    };
    set_issue_tile(0);
    // Issue the cursor's group into ring slot `slot` when `real`; otherwise
    // the same L loads aimed out of range (they read nothing and write zeros
    // into the first 1 KiB of this wave's staging area).  The cursor is
    // advanced separately, outside the scheduling regions of the K steps.
    auto issue = [&](bool real, int slot) __attribute__((always_inline)) {
        const int kbase = ik * C::BK;
        const bool valid = real && l_chunk * 8 < K - kbase;
        const uint32_t v = valid ? l_base + (uint32_t)kbase * 2u : kOutOfRange;
        const uint32_t step = valid ? l_step : 0u;
        char *sa = real ? smem + slot * C::STAGE_BYTES + wave * 1024 : epi;
        char *sb = real ? smem + slot * C::STAGE_BYTES + C::A_BYTES + wave * 1024 : epi;
        const int lstride = real ? C::NW * 1024 : 0;
#pragma unroll
        for (int i = 0; i < C::NA; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ira, (__attribute__((address_space(3))) void *)(sa + i * lstride),
                16, v + (uint32_t)i * step, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < C::NB; ++i)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                irb, (__attribute__((address_space(3))) void *)(sb + i * lstride),
                16, v + (uint32_t)i * step, 0, 0, 0);
    };
    auto advance = [&]() __attribute__((always_inline)) {
        if (++ik == ntile) {
            ik = 0;
            if (++iu < nu) set_issue_tile(iu);
        }
    };

    // ---- fragment reads and MFMAs (as the tiled kernel)
    const int ra_row = wm * C::WTM + (lane & 31);
    const int rb_row = wn * C::WTN + (lane & 31);
    int fa[C::NKS], fb[C::NKS];
#pragma unroll
    for (int ks = 0; ks < C::NKS; ++ks) {
        const int c = 2 * ks + half;
        fa[ks] = ra_row * C::RB + ((c ^ swz<C::CPR>(ra_row)) << 4);
        fb[ks] = C::A_BYTES + rb_row * C::RB + ((c ^ swz<C::CPR>(rb_row)) << 4);
    }
    auto read_frags = [&](f16x8 (&fra)[C::FM], f16x8 (&frb)[C::FN], const char *sbase,
                          int ks) __attribute__((always_inline)) {
        fra[0] = *(const f16x8 *)(sbase + fa[ks]);
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            frb[j] = *(const f16x8 *)(sbase + fb[ks] + j * 32 * C::RB);
#pragma unroll
        for (int i = 1; i < C::FM; ++i)
            fra[i] = *(const f16x8 *)(sbase + fa[ks] + i * 32 * C::RB);
    };
    auto mfma_step = [&](const f16x8 (&fra)[C::FM],
                         const f16x8 (&frb)[C::FN]) __attribute__((always_inline)) {
#pragma unroll
        for (int i = 0; i < C::FM; ++i)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(frb[j], fra[i], acc[i][j], 0, 0, 0);
    };
    // Wait until at most `n` counted operations of this lane are outstanding
    // (and all its LDS reads), then a workgroup barrier.  s_waitcnt takes an
    // immediate, so `n` (from persistent_wait_count) is served by the largest
    // of the compiled counts 0, L, L + ST, 2L + ST not above it -- waiting
    // longer is safe -- through a uniform branch around the s_waitcnt alone:
    // every K tile runs the same code (several K-tile bodies in one loop
    // make the register allocator spill the accumulators).
    constexpr int N1 = C::L, N2 = C::L + C::STORES, N3 = 2 * C::L + C::STORES;
    static_assert(N3 <= 63, "vmcnt is a 6-bit counter");
    auto sync_n = [&](int n) __attribute__((always_inline)) {
        compiler_fence();
        __builtin_amdgcn_sched_barrier(0);
        if (n >= N3)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(N3, 0));
        else if (n >= N2)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(N2, 0));
        else if (n >= N1)
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(N1, 0));
        else
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        compiler_fence();
    };

    // ---- prologue: groups 0 .. S-2 of the stream; wait for group 0
#pragma unroll
    for (int t = 0; t < C::S - 1; ++t)
        if (t < total) {
            issue(true, t);
            advance();
        }
    sync_n((C::S == 3 && total > 1) ? C::L : 0);

    f16x8 ra0[C::FM], rb0[C::FN], ra1[C::FM], rb1[C::FN];
    read_frags(ra0, rb0, smem, 0);

    // One stream K tile in ring slot `slot`, fragments double-buffered in
    // VGPRs, MFMAs interleaved one by one with the LDS reads and, at the
    // first K step, the L loads (group into `wslot` if `real`).  Unless LAST:
    // at the last K step wait (`n` outstanding), barrier, and read the next
    // tile's first fragments from `nslot`.
    auto ktile = [&](auto last_c, bool real, int n, int slot, int nslot,
                     int wslot) __attribute__((always_inline)) {
        constexpr bool LAST = decltype(last_c)::value;
        const char *sbase = smem + slot * C::STAGE_BYTES;
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) {
            f16x8(&cra)[C::FM] = (ks & 1) ? ra1 : ra0;
            f16x8(&crb)[C::FN] = (ks & 1) ? rb1 : rb0;
            f16x8(&nra)[C::FM] = (ks & 1) ? ra0 : ra1;
            f16x8(&nrb)[C::FN] = (ks & 1) ? rb0 : rb1;
            int nreads = C::FM + C::FN;
            if (ks == C::NKS - 1) {
                if constexpr (!LAST) {
                    sync_n(n);
                    read_frags(nra, nrb, smem + nslot * C::STAGE_BYTES, 0);
                } else {
                    nreads = 0;
                }
            } else {
                read_frags(nra, nrb, sbase, ks + 1);
            }
            int nissue = 0;
            if constexpr (!LAST) {
                if (ks == 0) {
                    issue(real, wslot);
                    nissue = C::L;
                }
            }
            mfma_step(cra, crb);
#pragma unroll
            for (int m = 0; m < C::FM * C::FN; ++m) {
                if (m < nreads) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                if (m < nissue) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    };

    // Consumer side: output tile u's origin for its epilogue.
    int cm0, cn0, crows_a, crows_b;
    geometry(0, cm0, cn0, crows_a, crows_b);
    // After the last K tile g of output tile u: the early group g + S (into
    // slot g mod S) if it exists, then the epilogue.  The epilogue writes the
    // staging area, where out-of-range loads of this output tile's first K
    // tile may still be landing unless a later wait covered them, which the
    // wait for group g' + S in tile g' + S - 1 does when the output tile has
    // at least S K tiles and is not the stream's last: otherwise wait for all
    // of this lane's loads first.
    auto boundary = [&](int g, int u, int slot) __attribute__((always_inline)) {
        if (g + C::S < total) {
            issue(true, slot);
            advance();
        }
        if (ntile < C::S || u == nu - 1) {
            compiler_fence();
            __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
            compiler_fence();
        }
        epilogue(cm0, cn0, crows_a);
        zero_acc();
        if (u + 1 < nu) geometry(u + 1, cm0, cn0, crows_a, crows_b);
    };

    int u = 0, k = 0;                              // output tile and K step of stream tile g
    int slot = 0;                                  // g mod S
#pragma unroll 1
    for (int g = 0; g < total - 1; ++g) {
        const bool real = g + C::S - 1 < total && !(k == 0 && u > 0);
        const int nslot = (slot + 1 == C::S) ? 0 : slot + 1;
        const int wslot = (slot == 0) ? C::S - 1 : slot - 1;   // (g + S - 1) mod S
        ktile(std::false_type{}, real,
              persistent_wait_count(C::S, C::L, C::STORES, ntile, total, u, k), slot, nslot,
              wslot);
        if (real) advance();
        if (k == ntile - 1) {
            boundary(g, u, slot);
            k = 0;
            ++u;
        } else {
            ++k;
        }
        slot = nslot;
    }
    // the stream's last tile: no loads, no wait, then its output tile's epilogue
    ktile(std::true_type{}, false, 0, slot, 0, 0);
    boundary(total - 1, nu - 1, slot);
}

}  // namespace sg
