// Fused attention forward O = softmax(alpha * Q K^T) V ("CUDA operator notes
// 2", section "Softmax Attention": scores Q K^T / sqrt(d), a row-wise softmax,
// then the product with V), for H independent heads with d = 128.
//
// The scores never leave the chip.  Each workgroup owns 128 or 256 query rows
// of one head (4 or 8 waves, 32 rows each) and streams the head's keys in
// tiles of 64 through two-slot LDS rings for K and V, filled by LDS-DMA one
// and two tiles ahead -- the stage-pipelined mainloop of "Lesson 6" -- and
// keeps a reference exponent m, a row sum l and an output accumulator O (the
// online form of the softmax):
//     S = Q K_j^T (MFMA, fp32), t = S * alpha * log2(e)
//     P = 2^(t - m), O += P V_j, l += sum P
// and writes O / l once at the end.  The quotient does not depend on m, so m
// only has to keep 2^(t - m) in range: it is raised (and O, l rescaled by
// 2^(m - m')) when a row's tile maximum exceeds m by more than TAU, not on
// every increase.  Probabilities then stay below 2^TAU, well inside fp16.
//
// The P V product contracts over keys, which are rows of V: a lane's MFMA
// operand needs one column of V over 8 keys.  V stays row-major in LDS and
// the operand is read with the transposing LDS load (ds_read_b64_tr_b16): in
// each group of 16 lanes, lane i receives element i % 4 of the 4-element
// pieces addressed by lanes i / 4, i / 4 + 4, i / 4 + 8 and i / 4 + 12.  The
// addresses are chosen so that the keys arrive in the order the score
// accumulators hold them (keys 0-3, 8-11, 4-7, 12-15 of every 16), so the
// fragment of probabilities a lane already holds is the other operand and
// the probabilities never move between lanes.
#pragma once

#include "gemm_kernel.hpp"

namespace sg {

typedef float f32x4 __attribute__((ext_vector_type(4)));

template <int NWAVES>
struct AttnCfg {
    static constexpr int D = 128;                  // head dimension
    static constexpr int BM = 32 * NWAVES;         // query rows per workgroup
    static constexpr int BN = 64;                  // keys per tile
    static constexpr int NW = NWAVES;              // waves, 32 query rows each
    static constexpr int T = 64 * NW;
    static constexpr int K_ROW = D * 2;            // 256-byte K rows
    static constexpr int K_BYTES = BN * K_ROW;     // 16 KiB
    static constexpr int V_ROW = D * 2;            // 256-byte V rows
    static constexpr int V_BYTES = BN * V_ROW;     // 16 KiB
    static constexpr int S = 2;                    // slots of each ring (K and V)
    static constexpr int V_OFFSET = S * K_BYTES;   // the V ring follows the K ring
    static constexpr int LDS_BYTES = S * (K_BYTES + V_BYTES);
    static constexpr int KL = K_BYTES / (16 * T);  // K LDS-DMA loads per lane per tile
    static_assert(KL * 16 * T == K_BYTES && K_BYTES == V_BYTES, "even K and V split");
    static constexpr float TAU = 8.0f;             // headroom of 2^(t - m), in exponent units
};

// 16-byte chunk position of logical chunk c in K row r (16 chunks per row).
__device__ __forceinline__ int k_chunk(int r, int c) { return c ^ (r & 15); }
// 16-byte chunk position of logical chunk c in V row r (16 chunks per row):
// the transposing reads of one half-wave touch 4 consecutive rows (a multiple
// of 4 apart) and 4 chunks 4 q .. 4 q + 3, which this places in 16 distinct
// 16-byte bank groups.
__device__ __forceinline__ int v_chunk(int r, int c) { return c ^ ((r & 3) << 2); }

// NEG: alpha < 0, so the largest scaled score comes from the smallest score.
//
// With splits > 1 the keys are divided too: workgroup (head, row block,
// split) takes a contiguous run of key tiles and, instead of O, writes its
// unnormalised accumulator to part_o and its reference exponent and row sum
// to part_ml; attention_combine_kernel then merges the splits of each row.
// This gives a single head enough workgroups to fill the device.  Layouts
// (fp32): part_o[(h * splits + sp) * M + row][D], part_ml[same index][2].
//
// NWAVES: 4 (128 query rows, two workgroups per CU) or 8 (256 rows, one per
// CU).  Both keep 8 waves on a CU; with 8 per workgroup every K and V tile
// is fetched into LDS once for twice the rows, which halves the DMA traffic
// per flop (measured -5 % time on 16 heads of 4096 x 4096).
template <bool NEG, int NWAVES>
__global__ void __launch_bounds__(64 * NWAVES, 8 / NWAVES)
attention_fwd_kernel(const _Float16 *__restrict__ Q, const _Float16 *__restrict__ Kg,
                     const _Float16 *__restrict__ V, _Float16 *__restrict__ O,
                     float *__restrict__ part_o, float *__restrict__ part_ml, int M, int N,
                     float alpha, int splits)
{
    using C = AttnCfg<NWAVES>;
    __shared__ __attribute__((aligned(1024))) char smem[C::LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int half = lane >> 5;
    const int r32 = lane & 31;

    // Workgroups are dealt round-robin to the 8 XCDs; renumber them so each
    // XCD takes a contiguous run (the same heads), whose K and V tiles its
    // L2 then holds for all the row blocks reading them.
    int pid = blockIdx.x;
    if ((gridDim.x & 7) == 0) pid = (pid & 7) * (gridDim.x >> 3) + (pid >> 3);
    const int row_blocks = (M + C::BM - 1) / C::BM;
    const int hb = pid / splits;                       // head-major row block
    const int sp = pid - hb * splits;
    const int h = hb / row_blocks;
    const int m0 = (hb - h * row_blocks) * C::BM;
    const int rows = (M - m0 < C::BM) ? (M - m0) : C::BM;
    const _Float16 *qh = Q + ((size_t)h * M + m0) * C::D;
    const _Float16 *kh = Kg + (size_t)h * N * C::D;
    const _Float16 *vh = V + (size_t)h * N * C::D;
    // buffer ranges cover only valid rows: rows past M or N read as zero
    const __amdgpu_buffer_rsrc_t rq = make_rsrc(qh, (uint32_t)rows * C::D * 2u);
    const u32x4 rk = rsrc_words(kh, (uint32_t)N * C::D * 2u);
    const u32x4 rv = rsrc_words(vh, (uint32_t)N * C::D * 2u);
    // LDS address of the ring (an LDS offset, not a generic address)
    const uint32_t lds0 = (uint32_t)reinterpret_cast<uintptr_t>(
        (__attribute__((address_space(3))) char *)smem);
    const int ntiles = (N + C::BN - 1) / C::BN;
    // this split's key tiles [t_lo, t_hi): never empty, as splits <= ntiles
    const int t_lo = (int)((long long)sp * ntiles / splits);
    const int t_hi = (int)((long long)(sp + 1) * ntiles / splits);

    // ---- Q fragments of this wave's 32 rows, all of d, kept in VGPRs:
    // step s holds Q[row][16 s + 8 half .. + 7]
    const int qrow = wave * 32 + r32;
    f16x8 qf[8];
#pragma unroll
    for (int s = 0; s < 8; ++s)
        qf[s] = __builtin_bit_cast(f16x8, __builtin_amdgcn_raw_buffer_load_b128(
                                              rq, (uint32_t)(qrow * C::D + 16 * s + 8 * half) * 2u, 0, 0));

    // ---- K tile j into slot: LDS-DMA, 1 KiB per wave instruction = 4 rows
    // of 256 bytes; lane -> row lane / 16, position lane % 16, which holds
    // logical chunk k_chunk(row, position) (the swizzle is its own inverse).
    auto issue_k = [&](int j, int slot) {
        const uint32_t base = lds0 + slot * C::K_BYTES;
#pragma unroll
        for (int i = 0; i < C::KL; ++i) {
            const int r = (i * C::NW + wave) * 4 + (lane >> 4);   // row within the tile
            const int c = k_chunk(r, lane & 15);
            const uint32_t off = (uint32_t)((j * C::BN + r) * C::D + c * 8) * 2u;
            dma16(rk, off, base + (i * C::NW + wave) * 1024);
        }
    };
    // ---- V tile j into slot: the same LDS-DMA pattern with V's swizzle
    auto issue_v = [&](int j, int slot) {
        const uint32_t base = lds0 + C::V_OFFSET + slot * C::V_BYTES;
#pragma unroll
        for (int i = 0; i < C::KL; ++i) {
            const int r = (i * C::NW + wave) * 4 + (lane >> 4);
            const int c = v_chunk(r, lane & 15);
            const uint32_t off = (uint32_t)((j * C::BN + r) * C::D + c * 8) * 2u;
            dma16(rv, off, base + (i * C::NW + wave) * 1024);
        }
    };
    // ---- per-lane byte offsets of the transposing V reads within a V tile:
    // as an address provider, lane l names key row 4 (l / 32) + (l % 16) / 4
    // (plus 16 G + 8 i for 16-key group G, half i) and columns
    // 32 c + 16 ((l / 16) % 2) + 4 (l % 4) .. + 3
    int vrd[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int row = 4 * half + ((lane & 15) >> 2);
        const int chunk = 4 * c + 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        vrd[c] = row * C::V_ROW + (v_chunk(row, chunk) << 4) + ((lane & 1) << 3);
    }

    auto barrier = [&]() {
        compiler_fence();
        __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 0));
        __builtin_amdgcn_s_barrier();
        compiler_fence();
    };

    const float c2 = alpha * 1.4426950408889634f;     // scores to base-2 exponents
    float mref = -__builtin_inff();                    // reference exponent m (row-wide)
    float lsum = 0.0f;                                 // running sum, this lane's keys
    // extreme of the raw scores that gives the largest t, and its identity
    auto ext = [](float a, float b) { return NEG ? __builtin_fminf(a, b) : __builtin_fmaxf(a, b); };
    const float none = NEG ? __builtin_inff() : -__builtin_inff();
    f32x16 oacc[4];                                    // O[row][32 c + 8 g + 4 half + e]
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int e = 0; e < 16; ++e) oacc[c][e] = 0.0f;

    // S = Q K^T of the tile in K slot `slot`: lane holds
    // S[row][32 b + 8 g + 4 half + e] in sa[b][4 g + e]
    auto scores = [&](int slot, f32x16 (&sa)[2]) {
        const char *kbase = smem + slot * C::K_BYTES;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e) sa[b][e] = 0.0f;
#pragma unroll
        for (int s = 0; s < 8; ++s) {
#pragma unroll
            for (int b = 0; b < 2; ++b) {
                const int key = 32 * b + r32;
                const f16x8 kf = *(const f16x8 *)(kbase + key * C::K_ROW +
                                                  (k_chunk(key, 2 * s + half) << 4));
                sa[b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(kf, qf[s], sa[b], 0, 0, 0);
            }
        }
    };

    // The online softmax in two halves, for this lane's row (its keys; the
    // partner lane lane ^ 32 holds the rest of the row).  Keys at or past
    // kvalid exist only in the last tile.
    auto key_of = [&](int b, int e) { return 32 * b + 8 * (e >> 2) + 4 * half + (e & 3); };
    // (1) Before a tile's probabilities: raise m where the row's maximum t in
    // the tile passed it by more than TAU and scale l to the new m; O is
    // scaled by the returned factor before the tile's P V, when the returned
    // flag says some row of the wave raised m (rarely, after the first tile).
    auto decide = [&](const f32x16 (&sa)[2], int kvalid, float &scale) -> bool {
        const bool ragged = kvalid < C::BN;            // uniform
        float sx = none;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int e = 0; e < 16; ++e)
                sx = ext(sx, (ragged && key_of(b, e) >= kvalid) ? none : sa[b][e]);
        sx = ext(sx, __builtin_bit_cast(float, __builtin_amdgcn_ds_bpermute(
                                                   (lane ^ 32) << 2, __builtin_bit_cast(int, sx))));
        // largest t of the row in this tile (finite: the tile has a key below
        // N); rounding is monotonic, so this is the largest rounded product
        const float tmax = sx * c2;
        const bool raise = tmax > mref + C::TAU;
        const float mnew = raise ? tmax : mref;
        scale = raise ? __builtin_amdgcn_exp2f(mref - mnew) : 1.0f;   // 0 on the first tile
        mref = mnew;
        lsum *= scale;
        return __builtin_amdgcn_ballot_w64(raise) != 0;   // uniform
    };
    auto rescale = [&](bool any, float scale) {
        if (any) {
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int e = 0; e < 16; ++e) oacc[c][e] *= scale;
        }
    };
    // (2) The probabilities 2^(t - m), added to l and returned as fp16 MFMA
    // fragments: fragment 2 b + t holds sa[b][8 t .. 8 t + 7].
    auto probs = [&](const f32x16 (&sa)[2], int kvalid, f16x8 (&pf)[4]) {
        const bool ragged = kvalid < C::BN;            // uniform
        const float negm = -mref;
        float psum = 0.0f;
#pragma unroll
        for (int b = 0; b < 2; ++b)
#pragma unroll
            for (int t = 0; t < 2; ++t)
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sa[b][8 * t + e], c2, negm));
                    if (ragged && key_of(b, 8 * t + e) >= kvalid) p = 0.0f;   // alpha = 0: t is NaN there
                    psum += p;
                    pf[2 * b + t][e] = (_Float16)p;
                }
        lsum += psum;
    };

    // O += P V for the tile in V slot `slot`: K step f covers keys
    // 16 f + {0..15}; this lane's probabilities pf[f] are keys
    // 16 f + 4 half + {0..3} and 16 f + 8 + 4 half + {0..3}, and the two
    // transposing reads bring V at the same keys, column 32 c + lane % 32
    auto pv = [&](int slot, const f16x8 (&pf)[4]) {
        const char *vbase = smem + C::V_OFFSET + slot * C::V_BYTES;
#pragma unroll
        for (int f = 0; f < 4; ++f)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                typedef short i16x4 __attribute__((ext_vector_type(4)));
                const char *p0 = vbase + vrd[c] + (16 * f) * C::V_ROW;
                const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4 *)(p0));
                const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                    (__attribute__((address_space(3))) i16x4 *)(p0 + 8 * C::V_ROW));
                const f16x8 vf = __builtin_bit_cast(f16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
                oacc[c] = __builtin_amdgcn_mfma_f32_32x32x16_f16(vf, pf[f], oacc[c], 0, 0, 0);
            }
    };
    // ---- prologue: K and V of the first tile, K of the second; scores of
    // the first tile
    issue_k(t_lo, 0);
    issue_v(t_lo, 0);
    if (t_lo + 1 < t_hi) issue_k(t_lo + 1, 1);
    compiler_fence();
    __builtin_amdgcn_s_waitcnt(waitcnt_imm(0, 15));
    compiler_fence();
    // the Q fragments count as produced here, after the wait: otherwise the
    // compiler sinks their loads towards the loop and waits for them (and,
    // vmcnt being in order, for the next tile's loads) inside every iteration
#pragma unroll
    for (int s = 0; s < 8; ++s) asm volatile("" : "+v"(qf[s]));
    barrier();
    f32x16 sacc[2];
    scores(0, sacc);
    float scale;
    bool any = decide(sacc, N - t_lo * C::BN, scale);
    barrier();                                         // K slot 0 is refilled next

    // ---- steady state, software-pipelined.  Step j: tile j's
    // probabilities, tile j + 1's scores (K runs one tile ahead of V), tile
    // j's P V, then m for tile j + 1 -- one branch-free stretch for the
    // scheduler to interleave; the rare rescale of O that m calls for comes
    // first in the next step.  K_{j+2}
    // goes to the K slot K_j held (read for S_j in the step before), V_{j+1}
    // to the V slot V_{j-1} held; both are waited for at the step's closing
    // barrier, which is also the WAR fence for the next refills.  The K
    // loads are issued after the probabilities and the V loads after the
    // scores, not together at the top of the step: the LDS-DMA path takes
    // each wave's 16-byte-per-lane load only as fast as it moves the bytes,
    // so a burst of all of them holds every wave at its issue point (4-wave
    // workgroups: -6.5 % time at 8 x 4096^2 x 128, -15 % at 2 heads).
    auto step = [&](int j, int kvalid_next) {
        const int cur = (j - t_lo) & 1;
        rescale(any, scale);
        f16x8 pf[4];
        probs(sacc, C::BN, pf);
        if (j + 2 < t_hi) issue_k(j + 2, cur);
        f32x16 snext[2];
        scores(cur ^ 1, snext);
        issue_v(j + 1, cur ^ 1);
        pv(cur, pf);
        any = decide(snext, kvalid_next, scale);
#pragma unroll
        for (int b = 0; b < 2; ++b) sacc[b] = snext[b];
        barrier();                                     // RAW for K_{j+2}, V_{j+1}; WAR for both slots
    };
#pragma unroll 1
    for (int j = t_lo; j < t_hi - 2; ++j) step(j, C::BN);
    if (t_hi - t_lo >= 2) step(t_hi - 2, N - (t_hi - 1) * C::BN);   // next is the last tile
    {   // ---- the last tile (the only one that can be ragged)
        const int j = t_hi - 1;
        rescale(any, scale);
        f16x8 pf[4];
        probs(sacc, N - j * C::BN, pf);
        pv((j - t_lo) & 1, pf);
    }

    const float lother = __builtin_bit_cast(
        float, __builtin_amdgcn_ds_bpermute((lane ^ 32) << 2, __builtin_bit_cast(int, lsum)));
    if (splits > 1) {
        // ---- partial of this split: O unnormalised, (m, l) of the row; rows
        // past M fall outside the buffer ranges and are dropped
        const size_t first = ((size_t)h * splits + sp) * M + m0;
        const __amdgpu_buffer_rsrc_t rpo = make_rsrc(part_o + first * C::D, (uint32_t)rows * C::D * 4u);
        const __amdgpu_buffer_rsrc_t rpm = make_rsrc(part_ml + first * 2, (uint32_t)rows * 8u);
#pragma unroll
        for (int c = 0; c < 4; ++c)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // whole-vector bit_cast: the same cast of a single vector
                // element yields element 0's bits whatever the index
                const f32x4 o4 = {oacc[c][4 * g], oacc[c][4 * g + 1], oacc[c][4 * g + 2],
                                  oacc[c][4 * g + 3]};
                const u32x4 v = __builtin_bit_cast(u32x4, o4);
                const uint32_t off = (uint32_t)(qrow * C::D + 32 * c + 8 * g + 4 * half) * 4u;
                __builtin_amdgcn_raw_buffer_store_b128(v, rpo, off, 0, 0);
            }
        if (__lane_id() < 32) {                        // recomputed: keeping `half` live spills
            u32x2 ml;
            ml[0] = __builtin_bit_cast(uint32_t, mref);
            ml[1] = __builtin_bit_cast(uint32_t, lsum + lother);
            __builtin_amdgcn_raw_buffer_store_b64(ml, rpm, (uint32_t)qrow * 8u, 0, 0);
        }
        return;
    }

    // ---- O / l, one conversion to fp16; lane stores 4 consecutive halves per
    // (c, g); rows past M fall outside the buffer range and are dropped
    const float inv = 1.0f / (lsum + lother);
    const __amdgpu_buffer_rsrc_t ro =
        make_rsrc(O + ((size_t)h * M + m0) * C::D, (uint32_t)rows * C::D * 2u);
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
        for (int g = 0; g < 4; ++g) {
            u32x2 packed;
            packed[0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(oacc[c][4 * g + 0] * inv)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(oacc[c][4 * g + 1] * inv)) << 16);
            packed[1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(oacc[c][4 * g + 2] * inv)) |
                        ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(oacc[c][4 * g + 3] * inv)) << 16);
            const uint32_t off = (uint32_t)(qrow * C::D + 32 * c + 8 * g + 4 * half) * 2u;
            __builtin_amdgcn_raw_buffer_store_b64(packed, ro, off, 0, 0);
        }
}

// Merge of the key splits of each row (the same online-softmax identity
// across splits): with m* the largest reference exponent of the row,
//     O = sum_s 2^(m_s - m*) O_s / sum_s 2^(m_s - m*) l_s,
// converted once to fp16.  32 threads per row, 4 columns (16 bytes) each;
// HM = H * M rows in all.
__global__ void __launch_bounds__(256)
attention_combine_kernel(const float *__restrict__ part_o, const float *__restrict__ part_ml,
                         _Float16 *__restrict__ O, long long HM, int M, int splits)
{
    using C = AttnCfg<4>;
    const long long t = (long long)blockIdx.x * 256 + threadIdx.x;
    const long long hr = t >> 5;                       // h * M + row
    if (hr >= HM) return;
    const int col = (int)(t & 31) * 4;
    const long long h = hr / M;
    const long long row = hr - h * M;
    const size_t first = (size_t)h * splits * M + row;   // index of split 0
    // one online pass, four runs per round so their loads are in flight together
    float mx = -__builtin_inff();
    float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    float l = 0.0f;
    for (int s0 = 0; s0 < splits; s0 += 4) {
        float ms[4], ls[4];
        f32x4 os[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const size_t i = first + (size_t)(s0 + u < splits ? s0 + u : s0) * M;
            typedef float f32x2 __attribute__((ext_vector_type(2)));
            const f32x2 ml = *(const f32x2 *)(part_ml + i * 2);
            ms[u] = s0 + u < splits ? ml[0] : -__builtin_inff();
            ls[u] = ml[1];
            os[u] = *(const f32x4 *)(part_o + i * C::D + col);
        }
        const float mr = __builtin_fmaxf(__builtin_fmaxf(ms[0], ms[1]), __builtin_fmaxf(ms[2], ms[3]));
        const float mnew = __builtin_fmaxf(mx, mr);
        const float keep = __builtin_amdgcn_exp2f(mx - mnew);   // 0 in the first round
        l *= keep;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] *= keep;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const float w = __builtin_amdgcn_exp2f(ms[u] - mnew);   // 0 for the padding runs
            l += w * ls[u];
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[e] += w * os[u][e];
        }
        mx = mnew;
    }
    const float inv = 1.0f / l;
    u32x2 packed;
    packed[0] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[0] * inv)) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[1] * inv)) << 16);
    packed[1] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[2] * inv)) |
                ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(acc[3] * inv)) << 16);
    *(u32x2 *)(O + hr * C::D + col) = packed;
}

}  // namespace sg
