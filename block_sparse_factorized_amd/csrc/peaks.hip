// peaks.hip -- libsa_peaks: the sustained bf16 matrix-core rate and the HBM
// copy bandwidth of the machine at hand (include/sa_peaks.h).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/sa_peaks.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Eight independent accumulator chains per wave keep the matrix pipe busy
// while each product waits for the previous one of its chain.
__global__ __launch_bounds__(256) void mfma_bf16_kernel(float* out, int iters)
{
    bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(1.0f / (float)(1 + ((threadIdx.x + e) & 7)));
        b[e] = (__bf16)(1.0f / (float)(2 + ((threadIdx.x * 3 + e) & 7)));
    }
    f32x16 c[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = f32x16{};
    for (int i = 0; i < iters; ++i) {
#pragma unroll
        for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j)
#pragma unroll
        for (int e = 0; e < 16; ++e) s += c[j][e];
    out[blockIdx.x * 256 + threadIdx.x] = s;  // keeps the products live
}

// One 16-byte non-temporal load and store per lane and step, four
// workgroups per CU: the fastest of the shapes measured on MI355X
// (several loads in flight per lane and larger grids were slower).
__global__ __launch_bounds__(256) void copy_kernel(u32x4* __restrict__ dst, const u32x4* __restrict__ src, size_t n)
{
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride)
        __builtin_nontemporal_store(__builtin_nontemporal_load(&src[i]), &dst[i]);
}

double elapsed_ms(hipEvent_t a, hipEvent_t b)
{
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, a, b) != hipSuccess) return -1.0;
    return (double)ms;
}

}  // namespace

extern "C" double sap_mfma_bf16_tflops(int blocks, int iters, void* stream)
{
    if (blocks < 1 || iters < 1) return -1.0;
    hipStream_t s = (hipStream_t)stream;
    float* out = nullptr;
    if (hipMalloc(&out, (size_t)blocks * 256 * sizeof(float)) != hipSuccess) return -1.0;
    hipEvent_t e0, e1;
    double result = -1.0;
    if (hipEventCreate(&e0) == hipSuccess) {
        if (hipEventCreate(&e1) == hipSuccess) {
            // the best of three timed launches after an untimed one (clocks
            // settle under a sustained matrix load)
            hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(256), 0, s, out, iters);
            const double flops = (double)blocks * 4.0 * iters * 8.0 * (2.0 * 32 * 32 * 16);
            for (int rep = 0; rep < 3; ++rep) {
                hipEventRecord(e0, s);
                hipLaunchKernelGGL(mfma_bf16_kernel, dim3(blocks), dim3(256), 0, s, out, iters);
                hipEventRecord(e1, s);
                if (hipGetLastError() != hipSuccess || hipEventSynchronize(e1) != hipSuccess) {
                    result = -1.0;
                    break;
                }
                const double ms = elapsed_ms(e0, e1);
                if (ms > 0 && flops / (ms * 1e-3) / 1e12 > result) result = flops / (ms * 1e-3) / 1e12;
            }
            (void)hipEventDestroy(e1);
        }
        (void)hipEventDestroy(e0);
    }
    (void)hipFree(out);
    return result;
}

extern "C" double sap_copy_gbs(void* dst, const void* src, size_t bytes, int reps, void* stream)
{
    if (!dst || !src || bytes == 0 || bytes % 16 != 0 || reps < 1 || ((uintptr_t)dst & 15) || ((uintptr_t)src & 15))
        return -1.0;
    hipStream_t s = (hipStream_t)stream;
    const size_t n = bytes / 16;
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    const unsigned grid = (unsigned)(cus * 4);
    hipEvent_t e0, e1;
    double result = -1.0;
    if (hipEventCreate(&e0) != hipSuccess) return -1.0;
    if (hipEventCreate(&e1) == hipSuccess) {
        hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, s, (u32x4*)dst, (const u32x4*)src, n);
        hipEventRecord(e0, s);
        for (int r = 0; r < reps; ++r)
            hipLaunchKernelGGL(copy_kernel, dim3(grid), dim3(256), 0, s, (u32x4*)dst, (const u32x4*)src, n);
        hipEventRecord(e1, s);
        if (hipGetLastError() == hipSuccess && hipEventSynchronize(e1) == hipSuccess) {
            const double ms = elapsed_ms(e0, e1);
            if (ms > 0) result = 2.0 * (double)bytes * reps / (ms * 1e-3) / 1e9;
        }
        (void)hipEventDestroy(e1);
    }
    (void)hipEventDestroy(e0);
    return result;
}
