// Measurement aids: a matrix-core loop and a streaming copy, timed by the caller to give the
// device's achievable bf16 MFMA rate and HBM streaming rate next to the nominal figures.
#include <hip/hip_runtime.h>

#include "oal_calib.h"
#include "oal_device.h"

namespace {

constexpr int kChains = 8;   // independent accumulators per wavefront: covers the MFMA latency

__global__ __launch_bounds__(256) void oal_calib_mfma_kernel(int iters, float *out) {
    const int lane = threadIdx.x & 63;
    // operands depend on the lane so the loop cannot be folded; values stay small and finite
    oal_bf16x8 a, b;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        a[e] = (__bf16)(0.001f * (float)((lane + e) & 7));
        b[e] = (__bf16)(0.001f * (float)((lane * 3 + e) & 7));
    }
    oal_f32x4 acc[kChains];
#pragma unroll
    for (int j = 0; j < kChains; ++j) {   // distinct starting values: the chains are not common subexpressions
        const float x = (float)(j * 64 + lane);
        acc[j] = oal_f32x4{x, x + 1.f, x + 2.f, x + 3.f};
    }
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int j = 0; j < kChains; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < kChains; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
    out[(size_t)blockIdx.x * 256 + threadIdx.x] = s;
}

// one 16-byte load and store per thread and step (measured on MI355X: a flat grid of these
// streams faster than deeper per-thread unrolling or non-temporal hints)
__global__ __launch_bounds__(256) void oal_calib_copy_kernel(const uint4 *__restrict__ src,
                                                             uint4 *__restrict__ dst, size_t n) {
    const size_t stride = (size_t)gridDim.x * 256;
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" oal_status oal_calib_mfma_bf16(int blocks, int iters, float *out, double *flops,
                                          hipStream_t stream) {
    if (blocks < 1 || blocks > 65536 || iters < 1 || iters > (1 << 20) || !out) return OAL_E_ARG;
    if (flops) *flops = (double)blocks * 4.0 * iters * kChains * 2.0 * 16 * 16 * 32;
    hipLaunchKernelGGL(oal_calib_mfma_kernel, dim3(blocks), dim3(256), 0, stream, iters, out);
    return hipGetLastError() == hipSuccess ? OAL_OK : OAL_E_HIP;
}

extern "C" oal_status oal_calib_copy(const void *src, void *dst, size_t bytes, hipStream_t stream) {
    if (!src || !dst || bytes % 16) return OAL_E_ARG;
    if (((uintptr_t)src | (uintptr_t)dst) & 15) return OAL_E_ALIGN;
    if (bytes == 0) return OAL_OK;
    int dev = 0, cus = 0;   // grid: one element per thread, capped at 1024 workgroups per CU
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return OAL_E_HIP;
    const size_t n = bytes / 16;
    size_t grid = (n + 255) / 256;
    if (grid > (size_t)cus * 1024) grid = (size_t)cus * 1024;
    hipLaunchKernelGGL(oal_calib_copy_kernel, dim3((unsigned)grid), dim3(256), 0, stream,
                       static_cast<const uint4 *>(src), static_cast<uint4 *>(dst), n);
    return hipGetLastError() == hipSuccess ? OAL_OK : OAL_E_HIP;
}
