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

}  // namespace

extern "C" {

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
