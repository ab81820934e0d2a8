// Short-K variant of the stage-pipelined TN GEMM (schedule 4), for
// K <= S * BK: the whole K extent of the tile fits in the LDS ring.
//
// The prologue of "Lesson 6" fills every K tile at once, and there is no
// steady state: one wait and one barrier, then each wave walks its sub-tile
// one 32-row block at a time -- all K steps of that block's MFMAs, then the
// block's epilogue ("cute(9) multistage_gemm", section 7.2: registers ->
// shared memory -> global) -- so the stores of block i drain while the
// MFMAs of block i + 1 run.  In the tiled kernels every block's MFMAs must
// end before the first store; with a short K loop (4096 x 4096 x 128) the
// loads, the MFMAs and the write of D then run one after another on each CU.
// A wave's B fragments for the whole K extent are read once and stay in
// registers; the A fragments of block i + 1 are read while block i's MFMAs
// and stores run.  Tiles go in the order of short_k_coords (row-major where
// the operands fit in an L2).  Only D = alpha * A * B^T (no C operand).
#pragma once

#include "gemm_kernel.hpp"

namespace sg {

// One output tile of the short-K schedule from a filled ring region `ring`
// (K tile t at ring + t * STAGE_BYTES, NT tiles): each wave reads its B
// fragments for the whole K extent once, then walks its sub-tile one 32-row
// block at a time -- all K steps of that block's MFMAs, then the block's
// staged store -- with the A fragments of the next block read ahead.  `rd`
// covers the tile's rows of D from its first row; n is this lane's first
// column of D and n_ok whether its 16-byte chunk lies inside N.
template <class C, int NT>
__device__ __forceinline__ void shortk_tile(const char *ring, char *epi, int lane, int wm, int wn,
                                            __amdgpu_buffer_rsrc_t rd, int n, bool n_ok, int N,
                                            float alpha)
{
    const int half = lane >> 5;
    constexpr int NQ = NT * C::NKS;                 // q = t * NKS + ks: every K step
    const int ra_row = wm * C::WTM + (lane & 31);
    const int rb_row = wn * C::WTN + (lane & 31);
    auto frag = [&](int t, int part, int row, int ks) {
        const int c = 2 * ks + half;
        return *(const f16x8 *)(ring + t * C::STAGE_BYTES + part + row * C::RB +
                                ((c ^ swz<C::CPR>(row)) << 4));
    };
    f16x8 fb[NQ][C::FN];                           // this wave's B columns, whole K
#pragma unroll
    for (int q = 0; q < NQ; ++q)
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
            fb[q][j] = frag(q / C::NKS, C::A_BYTES, rb_row + j * 32, q % C::NKS);
    f16x8 fa[2][NQ];                               // A rows of blocks i and i + 1
#pragma unroll
    for (int q = 0; q < NQ; ++q) fa[0][q] = frag(q / C::NKS, 0, ra_row, q % C::NKS);
#pragma unroll
    for (int i = 0; i < C::FM; ++i) {
        if (i + 1 < C::FM) {
#pragma unroll
            for (int q = 0; q < NQ; ++q)
                fa[(i + 1) & 1][q] = frag(q / C::NKS, 0, ra_row + (i + 1) * 32, q % C::NKS);
        }
        f32x16 acc[C::FN];
#pragma unroll
        for (int j = 0; j < C::FN; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
#pragma unroll
        for (int q = 0; q < NQ; ++q)
#pragma unroll
            for (int j = 0; j < C::FN; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fb[q][j], fa[i & 1][q], acc[j], 0, 0, 0);
        store_block_staged<C>(acc, alpha, epi, lane, rd, wm * C::WTM + i * 32, n, n_ok, N);
    }
}

template <class C>
__global__ void __launch_bounds__(C::T)
gemm_tn_shortk_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B,
                      const _Float16 *Cm, _Float16 *D, int M, int N, int K, float alpha,
                      float beta)
{
    static_assert(C::SCHED == 4, "short-K schedule");
    (void)Cm;
    (void)beta;                                    // the launcher passes beta == 0 only
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int wm = wave / C::WN;
    const int wn = wave % C::WN;

    const int tiles_m = (M + C::BM - 1) / C::BM;
    const int tiles_n = (N + C::BN - 1) / C::BN;
    int tm, tn;
    short_k_coords(blockIdx.x, tiles_m, tiles_n, M, N, K, tm, tn);
    const int m0 = tm * C::BM;
    const int n0 = tn * C::BN;
    const int rows_a = (M - m0 < C::BM) ? (M - m0) : C::BM;
    const int rows_b = (N - n0 < C::BN) ? (N - n0) : C::BN;
    const int ntile = (K + C::BK - 1) / C::BK;     // the launcher keeps ntile <= S

    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (size_t)m0 * K, (uint32_t)rows_a * K * 2u);
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(B + (size_t)n0 * K, (uint32_t)rows_b * K * 2u);

    // ---- prologue: every K tile t into ring slot t (loader lane mapping of
    // the tiled kernel; K-tail chunks get an out-of-range offset and read 0)
    constexpr int ROWS_PER_LOAD = 64 / C::CPR;
    static_assert(ROWS_PER_LOAD >= 16 || C::NW % 2 == 0, "swizzle fixed across a wave's loads");
    const int l_row0 = wave * ROWS_PER_LOAD + lane / C::CPR;
    const int l_chunk = (lane % C::CPR) ^ swz<C::CPR>(l_row0);
    const uint32_t l_base = (uint32_t)(l_row0 * K + l_chunk * 8) * 2u;
    const uint32_t l_step = (uint32_t)(C::NW * ROWS_PER_LOAD) * (uint32_t)K * 2u;
    // A one-K-tile extent (K <= BK, K = 0 included) fills slot 0 only and
    // runs one slot's K steps; otherwise slots past the last K tile are
    // filled with zeros by the same loads (their offsets lie past the buffer
    // range), so every block runs all S * NKS K steps without a branch.
    const bool one_tile = ntile <= 1;
#pragma unroll
    for (int t = 0; t < C::S; ++t) {
        if (t > 0 && one_tile) break;
        const int kbase = t * C::BK;
        const bool valid = l_chunk * 8 < K - kbase;
        const uint32_t v = valid ? l_base + (uint32_t)kbase * 2u : kOutOfRange;
        const uint32_t step = valid ? l_step : 0u;
        char *sa = smem + t * C::STAGE_BYTES;
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
    }
    // every K tile complete and visible (RAW); nothing is refilled (no WAR)
    compiler_fence();
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    compiler_fence();

    // ---- fragments, MFMAs and the row-block epilogue of the one tile
    char *epi = smem + C::RING_BYTES + wave * C::EPI_BLOCK_WAVE_BYTES;
    const __amdgpu_buffer_rsrc_t rd = make_rsrc(D + (size_t)m0 * N, (uint32_t)rows_a * N * 2u);
    const int n = n0 + wn * C::WTN + (lane & 7) * 8;
    if (one_tile)
        shortk_tile<C, 1>(smem, epi, lane, wm, wn, rd, n, n < N, N, alpha);
    else
        shortk_tile<C, C::S>(smem, epi, lane, wm, wn, rd, n, n < N, N, alpha);
}

}  // namespace sg
