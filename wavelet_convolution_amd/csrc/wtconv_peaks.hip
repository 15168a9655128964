// Two measurement probes exported next to the layer's entry points. They are
// not part of the layer: they measure, on the device at hand, the two
// ceilings the layer's kernels are compared with - the rate of unpacked fp32
// fused multiply-adds on the vector ALU and the rate of a plain HBM copy.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "../../include/wtconv.h"

namespace {

constexpr int PROBE_THREADS = 256;
constexpr int CHAINS = 16;   // independent FMA chains per lane: hides the FMA latency

// Every lane runs CHAINS dependent chains of `iters` FMAs each and stores
// their sum, so nothing is dead code. 2 * CHAINS * iters flops per lane.
__global__ __launch_bounds__(PROBE_THREADS) void k_peak_fma(float* __restrict__ out, int iters, float m, float c) {
    const int gid = blockIdx.x * PROBE_THREADS + threadIdx.x;
    float a[CHAINS];
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) a[i] = (float)(gid + i) * 1e-7f;
#pragma unroll 4
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < CHAINS; ++i) a[i] = __builtin_fmaf(a[i], m, c);
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < CHAINS; ++i) s += a[i];
    out[gid] = s;
}

// Grid-stride copy of n 16-byte vectors, four loads in flight per lane
// before their stores.
constexpr int COPY_UNROLL = 4;
typedef float v4f __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(PROBE_THREADS) void k_peak_copy(const v4f* __restrict__ src, v4f* __restrict__ dst,
                                                             size_t n) {
    const size_t stride = (size_t)gridDim.x * PROBE_THREADS;
    size_t i = blockIdx.x * (size_t)PROBE_THREADS + threadIdx.x;
    for (; i + (COPY_UNROLL - 1) * stride < n; i += COPY_UNROLL * stride) {
        v4f v[COPY_UNROLL];
#pragma unroll
        for (int u = 0; u < COPY_UNROLL; ++u) v[u] = __builtin_nontemporal_load(&src[i + u * stride]);
#pragma unroll
        for (int u = 0; u < COPY_UNROLL; ++u) __builtin_nontemporal_store(v[u], &dst[i + u * stride]);
    }
    for (; i < n; i += stride) dst[i] = src[i];
}

}  // namespace

extern "C" {

wtconv_status_t wtconv_peak_fma(float* out, int32_t blocks, int32_t iters, void* stream) {
    if (!out || ((uintptr_t)out & 15u)) return WTCONV_ERR_INVALID_ARG;
    if (blocks < 1 || blocks > (1 << 20) || iters < 1 || iters > (1 << 20)) return WTCONV_ERR_INVALID_ARG;
    // m slightly below 1 keeps every chain bounded for any iteration count
    hipLaunchKernelGGL(k_peak_fma, dim3((unsigned)blocks), dim3(PROBE_THREADS), 0, (hipStream_t)stream, out, iters,
                       0.999999f, 1e-6f);
    return hipGetLastError() == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
}

wtconv_status_t wtconv_peak_copy(const void* src, void* dst, size_t bytes, void* stream) {
    if (!src || !dst || ((uintptr_t)src & 15u) || ((uintptr_t)dst & 15u) || bytes % 16 != 0)
        return WTCONV_ERR_INVALID_ARG;
    const uintptr_t a = (uintptr_t)src, b = (uintptr_t)dst;
    if (bytes > 0 && a < b + bytes && b < a + bytes) return WTCONV_ERR_INVALID_ARG;
    const size_t n = bytes / 16;
    if (n == 0) return WTCONV_OK;
    // enough workgroups to keep every CU's memory pipeline full; the loop covers the rest
    size_t g = (n + PROBE_THREADS - 1) / PROBE_THREADS;
    if (g > 256u * 32u) g = 256u * 32u;
    hipLaunchKernelGGL(k_peak_copy, dim3((unsigned)g), dim3(PROBE_THREADS), 0, (hipStream_t)stream,
                       (const v4f*)src, (v4f*)dst, n);
    return hipGetLastError() == hipSuccess ? WTCONV_OK : WTCONV_ERR_LAUNCH;
}

}  // extern "C"
