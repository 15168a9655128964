// Layout conversion between channels-last and planar activations. The fused
// kernels stream whole (b, c) planes, which in a channels-last tensor are
// strided by C; so a channels-last call converts its activations to planar
// order in the workspace, runs the planar kernels, and converts the result
// back. Each conversion is one read and one write of the tensor.
//
// Per batch image the conversion is the transpose of an R x S matrix
// (channels-last to planar: R = H*W rows of C channels; planar to
// channels-last: R = C rows of H*W pixels). 64 x 64 tiles go through LDS:
// reads coalesced along the source row, writes coalesced along the
// destination row.
#include "wtconv_device.h"
#include "wtconv_layout.h"

namespace wtc {
namespace {

constexpr int TT = 64;        // tile side
constexpr int TTHREADS = 256; // 64 columns x 4 row groups

// dst[b][s][r] = src[b][r][s] for r < R, s < S
template <typename T>
__global__ __launch_bounds__(TTHREADS) void k_transpose(const T* __restrict__ src, T* __restrict__ dst, int R,
                                                         int S) {
    __shared__ T tile[TT][TT + 1];
    const size_t base = (size_t)blockIdx.z * R * S;
    const int r0 = blockIdx.x * TT, s0 = blockIdx.y * TT;
    const int tx = threadIdx.x % TT, ty = threadIdx.x / TT;
#pragma unroll
    for (int i = ty; i < TT; i += TTHREADS / TT) {
        const int r = r0 + i, s = s0 + tx;
        if (r < R && s < S) tile[i][tx] = src[base + (size_t)r * S + s];
    }
    __syncthreads();
#pragma unroll
    for (int i = ty; i < TT; i += TTHREADS / TT) {
        const int s = s0 + i, r = r0 + tx;
        if (r < R && s < S) dst[base + (size_t)s * R + r] = tile[tx][i];
    }
}

// The same with 4-element vector accesses on both sides (R and S multiples
// of 4, so every vector lies inside one row and is aligned): 16 lanes cover
// a 64-element tile row.
constexpr int VE = 4;
template <typename T>
__global__ __launch_bounds__(TTHREADS) void k_transpose_v4(const T* __restrict__ src, T* __restrict__ dst, int R,
                                                            int S) {
    typedef T vec_t __attribute__((ext_vector_type(VE)));
    __shared__ T tile[TT][TT + 1];
    const size_t base = (size_t)blockIdx.z * R * S;
    const int r0 = blockIdx.x * TT, s0 = blockIdx.y * TT;
    const int g = threadIdx.x % (TT / VE), row = threadIdx.x / (TT / VE);
#pragma unroll
    for (int i = row; i < TT; i += TTHREADS / (TT / VE)) {
        const int r = r0 + i, s = s0 + g * VE;
        if (r < R && s < S) {
            const vec_t v = *(const vec_t*)(src + base + (size_t)r * S + s);
#pragma unroll
            for (int e = 0; e < VE; ++e) tile[i][g * VE + e] = v[e];
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = row; j < TT; j += TTHREADS / (TT / VE)) {
        const int s = s0 + j, r = r0 + g * VE;
        if (r < R && s < S) {
            vec_t v;
#pragma unroll
            for (int e = 0; e < VE; ++e) v[e] = tile[g * VE + e][j];
            *(vec_t*)(dst + base + (size_t)s * R + r) = v;
        }
    }
}

template <typename T>
hipError_t launch(const void* src, void* dst, int B, int R, int S, hipStream_t st) {
    const dim3 grid((unsigned)((R + TT - 1) / TT), (unsigned)((S + TT - 1) / TT), (unsigned)B);
    if (R % VE == 0 && S % VE == 0)
        hipLaunchKernelGGL(k_transpose_v4<T>, grid, dim3(TTHREADS), 0, st, (const T*)src, (T*)dst, R, S);
    else
        hipLaunchKernelGGL(k_transpose<T>, grid, dim3(TTHREADS), 0, st, (const T*)src, (T*)dst, R, S);
    return hipGetLastError();
}

}  // namespace

bool transpose_fits(int B, int C, int H, int W) {
    const long long hw = (long long)H * W;
    return B >= 1 && B <= 65535 && (C + TT - 1) / TT <= 65535 && (hw + TT - 1) / TT <= 65535;
}

hipError_t nhwc_to_nchw(const void* src, void* dst, int B, int C, int H, int W, bool bf16, hipStream_t st) {
    // per image: [H*W][C] -> [C][H*W]
    return bf16 ? launch<bf16_t>(src, dst, B, H * W, C, st) : launch<float>(src, dst, B, H * W, C, st);
}

hipError_t nchw_to_nhwc(const void* src, void* dst, int B, int C, int H, int W, bool bf16, hipStream_t st) {
    // per image: [C][H*W] -> [H*W][C]
    return bf16 ? launch<bf16_t>(src, dst, B, C, H * W, st) : launch<float>(src, dst, B, C, H * W, st);
}

}  // namespace wtc
