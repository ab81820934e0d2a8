// Measurement probe (not part of the GEMM path): the fp16 MFMA throughput
// this GPU sustains on a given operand distribution when nothing but MFMAs
// runs.  MI355X is power-limited under dense fp16 MFMA: the clock, and so the
// throughput, depends on the operand bits.  The benchmark reports the GEMM
// next to this ceiling measured on fragments of the GEMM's own inputs.
//
// Each wave loads 16 A and 16 B fragments (8 halves per lane) from the input
// matrices once, then cycles 8 independent 32x32 accumulators through
// v_mfma_f32_32x32x16_f16 (or 16 independent 16x16 accumulators through
// v_mfma_f32_16x16x32_f16: the same flops per loop) with a different operand
// pair per MFMA; no memory traffic inside the timed loop.
//
// A second probe times the two quantities of the stage-count model of
// "Lesson 6: Shared Memory layout and async pipeline", section 4 --
// S_min = ceil(T_copy / T_compute) + 1 -- for the 256 x 256 x 64 tile of the
// large-shape GEMM kernel, in shader clock cycles (s_memtime), with one
// 512-thread workgroup per CU on every CU:
//   T_copy     from the issue of one K tile's LDS-DMA loads (A and B, 64 KiB
//              per workgroup, 16 bytes per lane per load as in the GEMM) to
//              their completion (vmcnt 0), with every CU copying at once and
//              nothing else in flight;
//   T_compute  the MFMAs of one K tile: each of the 8 waves issues the 64
//              v_mfma_f32_16x16x32_f16 of its 128 x 64 sub-tile from
//              registers, timed from a workgroup barrier to the last issue.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kFrags = 16;

__global__ void __launch_bounds__(256)
mfma_ceiling_kernel(const f16x8 *__restrict__ a, const f16x8 *__restrict__ b, long long a_vecs,
                    long long b_vecs, int iters, float *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    f16x8 fa[kFrags], fb[kFrags];
#pragma unroll
    for (int i = 0; i < kFrags; ++i) {
        fa[i] = a[((w * kFrags + i) * 64 + lane) % a_vecs];
        fb[i] = b[((w * kFrags + i) * 64 + lane + 4096) % b_vecs];
    }
    f32x16 acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) acc[j][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < kFrags; ++q)
#pragma unroll
            for (int j = 0; j < 8; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(fa[q], fb[(q + j) % kFrags], acc[j],
                                                                0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += acc[j][e];
    sink[blockIdx.x * 256 + threadIdx.x] = s;   // keeps the MFMAs live
}

__global__ void __launch_bounds__(256)
mfma_ceiling16_kernel(const f16x8 *__restrict__ a, const f16x8 *__restrict__ b, long long a_vecs,
                      long long b_vecs, int iters, float *__restrict__ sink)
{
    const int lane = threadIdx.x & 63;
    const long long w = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
    f16x8 fa[kFrags], fb[kFrags];
#pragma unroll
    for (int i = 0; i < kFrags; ++i) {
        fa[i] = a[((w * kFrags + i) * 64 + lane) % a_vecs];
        fb[i] = b[((w * kFrags + i) * 64 + lane + 4096) % b_vecs];
    }
    f32x4 acc[16];
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[j][e] = 0.0f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int q = 0; q < kFrags; ++q)
#pragma unroll
            for (int j = 0; j < 16; ++j)
                acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fa[q], fb[(q + j) % kFrags], acc[j],
                                                                0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int j = 0; j < 16; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) s += acc[j][e];
    sink[blockIdx.x * 256 + threadIdx.x] = s;
}

// Stage-model probe (see the file comment).  Workgroup w reads the A rows of
// tile row (w % tiles_m) and the B rows of tile column (w / tiles_m) of an
// M x K and N x K row-major fp16 pair (M, N >= 256 * those counts, K a
// multiple of 64, ntile <= K / 64).  out[w * 8 + wave] receives, per wave,
// {copy cycles summed over the ntile K tiles, compute cycles summed, ntile,
// a value that keeps the MFMA results live} as four 64-bit words.
__global__ void __launch_bounds__(512)
stage_timing_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B, int K,
                    int tiles_m, int ntile, unsigned long long *__restrict__ out)
{
    __shared__ __attribute__((aligned(1024))) char lds[65536];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tm = blockIdx.x % tiles_m;
    const int tn = blockIdx.x / tiles_m;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16 *>(A + (size_t)tm * 256 * K), (short)0, 256 * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16 *>(B + (size_t)tn * 256 * K), (short)0, 256 * K * 2, 0x00020000);
    // load j (0..3) of this wave fills LDS chunk q = (j * 8 + wave) * 64 + lane
    // of an operand: row q / 8, 16-byte column q % 8 of the 128-byte K slice
    f16x8 fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fa[i] = *(const f16x8 *)(A + (size_t)(tm * 256 + wave * 32 + i * 8 + (lane >> 3)) * K + (lane & 7) * 8);
        fb[i] = *(const f16x8 *)(B + (size_t)(tn * 256 + wave * 32 + i * 8 + (lane >> 3)) * K + (lane & 7) * 8);
    }
    f32x4 acc[8][4];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[i][j][e] = 0.0f;
    unsigned long long copy = 0, compute = 0;
    for (int t = 0; t < ntile; ++t) {
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const unsigned long long c0 = __builtin_amdgcn_s_memtime();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int q = (j * 8 + wave) * 64 + lane;
            const uint32_t off = (uint32_t)(((q >> 3) * K + t * 64 + (q & 7) * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void *)(lds + (j * 8 + wave) * 1024), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (__attribute__((address_space(3))) void *)(lds + 32768 + (j * 8 + wave) * 1024), 16, off, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
        __builtin_amdgcn_sched_barrier(0);
        const unsigned long long c1 = __builtin_amdgcn_s_memtime();
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        const unsigned long long m0 = __builtin_amdgcn_s_memtime();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
#pragma unroll
            for (int i = 0; i < 8; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(fb[j], fa[(i + ks) & 3], acc[i][j], 0, 0, 0);
        __builtin_amdgcn_sched_barrier(0);
        const unsigned long long m1 = __builtin_amdgcn_s_memtime();
        __builtin_amdgcn_sched_barrier(0);
        copy += c1 - c0;
        compute += m1 - m0;
    }
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) sum += acc[i][j][e];
    // one lane per wave records; the LDS contents feed the live value too
    sum += (float)*(const _Float16 *)(lds + lane * 16);
    if (lane == 0) {
        unsigned long long *o = out + ((size_t)blockIdx.x * 8 + wave) * 4;
        o[0] = copy;
        o[1] = compute;
        o[2] = (unsigned long long)ntile;
        o[3] = (unsigned long long)__builtin_bit_cast(uint32_t, sum);
    }
}

// LDS-DMA rate probe: the bytes per shader cycle one CU moves from global
// memory into LDS through the 16-byte-per-lane LDS-DMA loads of the tiled
// kernels, with every CU streaming at once and nothing else running -- the
// copy side of the stage-count model of "Lesson 6" (section 4) as a rate
// rather than a latency.  Workgroup w (4 waves, one per CU) streams the K
// tiles (64 deep: ROWS rows of 128 bytes per operand) of the A rows of tile
// row w % tiles_m and the B rows of tile column (w / tiles_m) % tiles_n of an
// M x K and N x K pair, in order, into a 128 KiB ring, keeping the loads of
// DEPTH tiles in flight; nothing reads the LDS, so no barrier is needed.
// out[w * 4 + wave] receives {cycles from the first issue to the last
// completion (s_memtime), K tiles, bytes per workgroup and K tile, 0}.
constexpr int vm_wait(int vm) { return (vm & 15) | (7 << 4) | (((vm >> 4) & 3) << 14); }

template <int ROWS, int DEPTH>
__global__ void __launch_bounds__(256, 1)
dma_rate_kernel(const _Float16 *__restrict__ A, const _Float16 *__restrict__ B, int K, int tiles_m,
                int tiles_n, int ntile, unsigned long long *__restrict__ out)
{
    constexpr int TILE = 2 * ROWS * 128;           // bytes of one K tile, A and B
    constexpr int SLOTS = 131072 / TILE;
    constexpr int NL = ROWS * 128 / (4 * 1024);    // loads per wave per operand and tile
    static_assert(2 * NL * (DEPTH - 1) <= 63, "vmcnt is a 6-bit counter");
    __shared__ __attribute__((aligned(1024))) char lds[131072];
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int tm = blockIdx.x % tiles_m;
    const int tn = (blockIdx.x / tiles_m) % tiles_n;
    const __amdgpu_buffer_rsrc_t ra = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16 *>(A + (size_t)tm * ROWS * K), (short)0, ROWS * K * 2, 0x00020000);
    const __amdgpu_buffer_rsrc_t rb = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<_Float16 *>(B + (size_t)tn * ROWS * K), (short)0, ROWS * K * 2, 0x00020000);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    __builtin_amdgcn_sched_barrier(0);
    for (int t = 0; t < ntile; ++t) {
        char *slot = lds + (t % SLOTS) * TILE;
#pragma unroll
        for (int j = 0; j < NL; ++j) {
            // load j of this wave: 1 KiB = 8 rows of the K tile's 128 bytes
            const int q = (j * 4 + wave) * 64 + lane;
            const uint32_t off = (uint32_t)(((q >> 3) * K + t * 64 + (q & 7) * 8) * 2);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                ra, (__attribute__((address_space(3))) void *)(slot + (j * 4 + wave) * 1024), 16, off, 0, 0, 0);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rb, (__attribute__((address_space(3))) void *)(slot + ROWS * 128 + (j * 4 + wave) * 1024), 16,
                off, 0, 0, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_waitcnt(vm_wait(2 * NL * (DEPTH - 1)));
        __builtin_amdgcn_sched_barrier(0);
    }
    __builtin_amdgcn_s_waitcnt(vm_wait(0));
    __builtin_amdgcn_sched_barrier(0);
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    __builtin_amdgcn_sched_barrier(0);
    if (lane == 0) {
        unsigned long long *o = out + ((size_t)blockIdx.x * 4 + wave) * 4;
        o[0] = c1 - c0;
        o[1] = (unsigned long long)ntile;
        o[2] = (unsigned long long)TILE;
        o[3] = 0;
    }
}

// LDS access-pattern probe: one wave per workgroup repeats one pattern of
// 64-bit writes or 128-bit reads over an epilogue staging block (32 rows of
// 64 fp16), `iters` times; run under the LDS bank-conflict counters, it
// shows how many cycles each pattern takes and how many of them are
// conflicts.  Pattern p, access v (0..7) of lane l, byte address in a
// 16 KiB block:
//   0 padded rows (144 B), 16x16 accumulator pieces, 64-bit write
//   1 padded rows, 16-byte read along rows
//   2 128-byte rows, slot swizzle by (r >> 1) & 15, 32x32 pieces, write
//   3 the same layout, read
//   4 128-byte rows, slot swizzle by r & 15, 32x32 pieces, write
//   5 the same layout, 16x16 pieces, write
//   6 the same layout, read
//   7 contiguous 64-bit write, 8 contiguous 128-bit read (no conflicts)
__device__ __forceinline__ int lds_pattern_addr(int p, int l, int v)
{
    switch (p) {
    case 0: { const int r = 16 * (v & 1) + (l & 15), c = 16 * ((v >> 1) & 3) + 4 * (l >> 4); return r * 144 + c * 2; }
    case 1: { const int r = (v & 3) * 8 + l / 8; return r * 144 + (l % 8) * 16; }
    case 2: { const int r = l & 31, s = (8 * (v & 1) + 2 * ((v >> 1) & 3) + (l >> 5)) ^ ((r >> 1) & 15); return r * 128 + s * 8; }
    case 3: { const int r = (v & 3) * 8 + (l >> 3); return r * 128 + (((l & 7) ^ (((r >> 1) & 15) >> 1)) << 4); }
    case 4: { const int r = l & 31, s = (8 * (v & 1) + 2 * ((v >> 1) & 3) + (l >> 5)) ^ (r & 15); return r * 128 + s * 8; }
    case 5: { const int r = 16 * (v & 1) + (l & 15), s = 4 * ((v >> 1) & 3) + (l >> 4); return r * 128 + (s ^ (r & 15)) * 8; }
    case 6: { const int r = (v & 3) * 8 + (l >> 3); return r * 128 + (((l & 7) ^ ((r & 15) >> 1)) << 4); }
    case 7: return l * 8;
    default: return l * 16;
    }
}

template <int P, bool WRITE>
__global__ void __launch_bounds__(64) lds_pattern_kernel(unsigned *__restrict__ sink, int iters)
{
    typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
    typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
    __shared__ __attribute__((aligned(1024))) char lds[16384];
    const int l = threadIdx.x;
    u32x4 acc = {0u, 0u, 0u, 0u};
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int v = 0; v < 8; ++v) {
            // volatile LDS accesses: every one is issued as written (none
            // merged or dropped, though nothing reads the written values)
            typedef __attribute__((address_space(3))) char lds_char;
            lds_char *at = (lds_char *)lds + lds_pattern_addr(P, l, v);
            if constexpr (WRITE)
                *(volatile __attribute__((address_space(3))) u32x2 *)at =
                    u32x2{(unsigned)(l + it), (unsigned)v};
            else
                acc += *(const volatile __attribute__((address_space(3))) u32x4 *)at;
        }
        __builtin_amdgcn_s_waitcnt(0xc07f);   // lgkmcnt(0)
    }
    sink[blockIdx.x * 64 + l] = acc[0] + acc[1] + acc[2] + acc[3];
}

}  // namespace

extern "C" {

// LDS pattern probe launch: pattern 0..8 (see lds_pattern_addr; 0, 2, 4,
// 5, 7 write, the others read), `blocks` one-wave workgroups, `iters`
// repetitions; sink: device buffer of blocks * 64 32-bit words.  Returns a
// hipError_t value.
int sg_probe_lds_pattern(int pattern, int blocks, int iters, void *sink, void *stream)
{
    if (!sink || blocks <= 0 || iters <= 0 || pattern < 0 || pattern > 8)
        return (int)hipErrorInvalidValue;
    static const void *const kernels[9] = {
        reinterpret_cast<const void *>(&lds_pattern_kernel<0, true>),
        reinterpret_cast<const void *>(&lds_pattern_kernel<1, false>),
        reinterpret_cast<const void *>(&lds_pattern_kernel<2, true>),
        reinterpret_cast<const void *>(&lds_pattern_kernel<3, false>),
        reinterpret_cast<const void *>(&lds_pattern_kernel<4, true>),
        reinterpret_cast<const void *>(&lds_pattern_kernel<5, true>),
        reinterpret_cast<const void *>(&lds_pattern_kernel<6, false>),
        reinterpret_cast<const void *>(&lds_pattern_kernel<7, true>),
        reinterpret_cast<const void *>(&lds_pattern_kernel<8, false>)};
    unsigned *s = static_cast<unsigned *>(sink);
    void *args[] = {&s, &iters};
    return (int)hipLaunchKernel(kernels[pattern], dim3(blocks), dim3(64), args, 0,
                                static_cast<hipStream_t>(stream));
}

// Stage-model probe launch: `blocks` workgroups (one per CU is the intended
// use) over an M x K (A) and N x K (B) fp16 pair with M >= 256 * tiles_m and
// N >= 256 * ceil(blocks / tiles_m); K a positive multiple of 64 below 2^21;
// 1 <= ntile <= K / 64; out: device buffer of blocks * 32 64-bit words.
// Returns a hipError_t value (hipErrorInvalidValue for arguments outside
// these bounds, checked here before the launch).
int sg_probe_stage_timing(const void *A, long long M, const void *B, long long N, int K,
                          int tiles_m, int blocks, int ntile, void *out, void *stream)
{
    if (!A || !B || !out || K <= 0 || (K & 63) || K > (1 << 21) || tiles_m <= 0 || blocks <= 0 ||
        ntile <= 0 || ntile > K / 64)
        return (int)hipErrorInvalidValue;
    const long long tiles_n = (blocks + tiles_m - 1) / tiles_m;
    if (M < 256LL * tiles_m || N < 256LL * tiles_n || 256LL * K * 2 >= (1LL << 31))
        return (int)hipErrorInvalidValue;
    const _Float16 *a = static_cast<const _Float16 *>(A);
    const _Float16 *b = static_cast<const _Float16 *>(B);
    unsigned long long *o = static_cast<unsigned long long *>(out);
    void *args[] = {&a, &b, &K, &tiles_m, &ntile, &o};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(&stage_timing_kernel), dim3(blocks),
                                dim3(512), args, 0, static_cast<hipStream_t>(stream));
}

// LDS-DMA rate probe launch: rows 128 or 256 per operand tile, depth 1..4
// tiles in flight, `blocks` workgroups (one per CU is the intended use) over
// an M x K (A) and N x K (B) fp16 pair with M >= rows * tiles_m and N >=
// rows * tiles_n (tiles_m, tiles_n >= 1); K a positive multiple of 8 below
// 2^21 (rows start on 16-byte boundaries; with K % 64 != 0 they straddle
// 128-byte lines, as in the GEMM); 1 <= ntile <= K / 64; out: device buffer
// of blocks * 16 64-bit words.
// Returns a hipError_t value (hipErrorInvalidValue for arguments outside
// these bounds, checked here before the launch).
int sg_probe_dma_rate(const void *A, long long M, const void *B, long long N, int K, int rows,
                      int depth, int tiles_m, int tiles_n, int blocks, int ntile, void *out,
                      void *stream)
{
    if (!A || !B || !out || K <= 0 || (K & 7) || K > (1 << 21) || tiles_m <= 0 || tiles_n <= 0 ||
        blocks <= 0 || ntile <= 0 || ntile > K / 64 || (rows != 128 && rows != 256) || depth < 1 ||
        depth > 4)
        return (int)hipErrorInvalidValue;
    if (M < (long long)rows * tiles_m || N < (long long)rows * tiles_n ||
        (long long)rows * K * 2 >= (1LL << 31))
        return (int)hipErrorInvalidValue;
    static const void *const kernels[2][4] = {
        {reinterpret_cast<const void *>(&dma_rate_kernel<128, 1>),
         reinterpret_cast<const void *>(&dma_rate_kernel<128, 2>),
         reinterpret_cast<const void *>(&dma_rate_kernel<128, 3>),
         reinterpret_cast<const void *>(&dma_rate_kernel<128, 4>)},
        {reinterpret_cast<const void *>(&dma_rate_kernel<256, 1>),
         reinterpret_cast<const void *>(&dma_rate_kernel<256, 2>),
         reinterpret_cast<const void *>(&dma_rate_kernel<256, 3>),
         reinterpret_cast<const void *>(&dma_rate_kernel<256, 4>)}};
    const _Float16 *a = static_cast<const _Float16 *>(A);
    const _Float16 *b = static_cast<const _Float16 *>(B);
    unsigned long long *o = static_cast<unsigned long long *>(out);
    void *args[] = {&a, &b, &K, &tiles_m, &tiles_n, &ntile, &o};
    return (int)hipLaunchKernel(kernels[rows == 256][depth - 1], dim3(blocks), dim3(256), args, 0,
                                static_cast<hipStream_t>(stream));
}

// Flops one launch performs: blocks x 4 waves x iters x 16 x 8 MFMAs of
// 2 * 32 * 32 * 16 flop.
double sg_probe_mfma_ceiling_flops(int blocks, int iters)
{
    return (double)blocks * 4.0 * iters * kFrags * 8.0 * 32768.0;
}

// a, b: device fp16 buffers of a_elems / b_elems elements (>= 8 each, 16-byte
// aligned); sink: device float buffer of blocks * 256 elements.  Enqueues on
// `stream`; returns a hipError_t value (0 = success).  shape16: the
// 16x16x32 form (same flops as sg_probe_mfma_ceiling_flops gives).
int sg_probe_mfma_ceiling_shape(int shape16, const void *a, long long a_elems, const void *b,
                                long long b_elems, int blocks, int iters, void *sink, void *stream)
{
    if (!a || !b || !sink || a_elems < 8 || b_elems < 8 || blocks <= 0 || iters <= 0)
        return (int)hipErrorInvalidValue;
    const f16x8 *pa = static_cast<const f16x8 *>(a);
    const f16x8 *pb = static_cast<const f16x8 *>(b);
    long long av = a_elems / 8, bv = b_elems / 8;
    float *ps = static_cast<float *>(sink);
    void *args[] = {&pa, &pb, &av, &bv, &iters, &ps};
    const void *k = shape16 ? reinterpret_cast<const void *>(&mfma_ceiling16_kernel)
                            : reinterpret_cast<const void *>(&mfma_ceiling_kernel);
    return (int)hipLaunchKernel(k, dim3(blocks), dim3(256), args, 0, static_cast<hipStream_t>(stream));
}

int sg_probe_mfma_ceiling(const void *a, long long a_elems, const void *b, long long b_elems,
                          int blocks, int iters, void *sink, void *stream)
{
    if (!a || !b || !sink || a_elems < 8 || b_elems < 8 || blocks <= 0 || iters <= 0)
        return (int)hipErrorInvalidValue;
    const f16x8 *pa = static_cast<const f16x8 *>(a);
    const f16x8 *pb = static_cast<const f16x8 *>(b);
    long long av = a_elems / 8, bv = b_elems / 8;
    float *ps = static_cast<float *>(sink);
    void *args[] = {&pa, &pb, &av, &bv, &iters, &ps};
    return (int)hipLaunchKernel(reinterpret_cast<const void *>(&mfma_ceiling_kernel), dim3(blocks),
                                dim3(256), args, 0, static_cast<hipStream_t>(stream));
}

}  // extern "C"
