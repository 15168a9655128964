// Naive unfused WTConv: one kernel per step of the layer's definition, with
// every intermediate (each level's subbands, convolution outputs, scaled
// outputs, the synthesis carry and the base-convolution output) written to
// and read back from device memory. This is the shape of implementation the
// abstract of arXiv:2608.10805 describes as memory-bound (it moves too much
// data through HBM); it exists as the comparator for the fused kernels and as a
// second, independently written GPU implementation for parity checks. It
// uses the orthonormal Haar normalisation (1/2 per butterfly) literally.
//
// Band grids: level l holds ceil(h/2) x ceil(w/2) coefficients of the h x w
// image it analyses; an odd last row or column is paired with a zero one, and
// each synthesis writes back only the h x w image it came from. For planes
// that 2^L divides this is the plain halving.
#include "wtconv_device.h"
#include "wtconv_naive.h"

#include "../../include/wtconv.h"

namespace wtc {
namespace {

constexpr int NB = 256;

// Offset of element (plane p = b*nch + c, row i, column j) of an h x w
// activation: planar ([B][C][H][W], plane stride ps) or, with nhwc set,
// channels-last ([B][H][W][C]). Band buffers are always planar.
__device__ inline size_t act_at(size_t p, int i, int j, int h, int w, size_t ps, int nch, int nhwc) {
    if (!nhwc) return p * ps + (size_t)i * w + j;
    return (((p / nch) * h + i) * (size_t)w + j) * nch + p % nch;
}

inline unsigned grid_for(size_t n) {
    size_t g = (n + NB - 1) / NB;
    return (unsigned)(g > 65535u * 16u ? 65535u * 16u : (g ? g : 1));
}

// h x w image (row stride w, plane stride in_stride) -> four bands of
// ceil(h/2) x ceil(w/2); taps beyond the image read as zero.
template <typename TI>
__global__ void k_dwt(const TI* __restrict__ in, size_t in_stride, float* __restrict__ out,
                      int planes, int h, int w, int nch, int nhwc) {
    const int h2 = (h + 1) / 2, w2 = (w + 1) / 2;
    const size_t n = (size_t)planes * h2 * w2;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int j = (int)(e % w2);
        const int i = (int)((e / w2) % h2);
        const size_t p = e / ((size_t)h2 * w2);
        const bool r1 = 2 * i + 1 < h, c1 = 2 * j + 1 < w;
        const float a = widen(in[act_at(p, 2 * i, 2 * j, h, w, in_stride, nch, nhwc)]);
        const float b = c1 ? widen(in[act_at(p, 2 * i, 2 * j + 1, h, w, in_stride, nch, nhwc)]) : 0.f;
        const float c = r1 ? widen(in[act_at(p, 2 * i + 1, 2 * j, h, w, in_stride, nch, nhwc)]) : 0.f;
        const float d = (r1 && c1) ? widen(in[act_at(p, 2 * i + 1, 2 * j + 1, h, w, in_stride, nch, nhwc)]) : 0.f;
        float* o = out + p * 4 * h2 * w2 + (size_t)i * w2 + j;
        const size_t bs = (size_t)h2 * w2;
        o[0] = 0.5f * (a + b + c + d);
        o[bs] = 0.5f * (a + b - c - d);
        o[2 * bs] = 0.5f * (a - b + c - d);
        o[3 * bs] = 0.5f * (a - b - c + d);
    }
}

// 'same' depthwise cross-correlation, zero padded; plane p uses kernel
// p % nch; flip turns every kernel by 180 degrees.
template <typename TI>
__global__ void k_dwconv(const TI* __restrict__ in, float* __restrict__ out, int planes, int nch,
                         int h, int w, const float* __restrict__ wts, int k, int flip, int nhwc) {
    const size_t n = (size_t)planes * h * w;
    const int p2 = k / 2;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int j = (int)(e % w);
        const int i = (int)((e / w) % h);
        const size_t p = e / ((size_t)h * w);
        const float* wk = wts + (size_t)(p % nch) * k * k;
        float acc = 0.f;
        for (int m = 0; m < k; ++m) {
            const int ii = i + m - p2;
            if (ii < 0 || ii >= h) continue;
            for (int q = 0; q < k; ++q) {
                const int jj = j + q - p2;
                if (jj < 0 || jj >= w) continue;
                const float wv = flip ? wk[(k - 1 - m) * k + (k - 1 - q)] : wk[m * k + q];
                acc += wv * widen(in[act_at(p, ii, jj, h, w, (size_t)h * w, nch, nhwc)]);
            }
        }
        out[e] = acc;
    }
}

__global__ void k_scale(float* __restrict__ buf, const float* __restrict__ sc, int planes, int nch,
                        int hw) {
    const size_t n = (size_t)planes * hw;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x)
        buf[e] *= sc[(e / hw) % nch];
}

__global__ void k_lladd(float* __restrict__ bands, const float* __restrict__ r, int planes, int hw) {
    const size_t n = (size_t)planes * hw;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const size_t p = e / hw, t = e % hw;
        bands[p * 4 * hw + t] += r[e];
    }
}

// four bands of h2 x w2 -> the h x w image they were analysed from
// (h2 = ceil(h/2), w2 = ceil(w/2)); samples beyond it are dropped.
__global__ void k_iwt(const float* __restrict__ bands, float* __restrict__ out, int planes, int h2,
                      int w2, int h, int w) {
    const size_t n = (size_t)planes * h2 * w2;
    const size_t bs = (size_t)h2 * w2;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const int j = (int)(e % w2);
        const int i = (int)((e / w2) % h2);
        const size_t p = e / bs;
        const float* b = bands + p * 4 * bs + (size_t)i * w2 + j;
        const float b0 = b[0], b1 = b[bs], b2 = b[2 * bs], b3 = b[3 * bs];
        const bool r1 = 2 * i + 1 < h, c1 = 2 * j + 1 < w;
        float* o = out + p * h * w + (size_t)(2 * i) * w + 2 * j;
        o[0] = 0.5f * (b0 + b1 + b2 + b3);
        if (c1) o[1] = 0.5f * (b0 + b1 - b2 - b3);
        if (r1) o[w] = 0.5f * (b0 - b1 + b2 - b3);
        if (r1 && c1) o[w + 1] = 0.5f * (b0 - b1 - b2 + b3);
    }
}

// out = a + b (planar fp32 buffers) in the activation layout
template <typename T>
__global__ void k_final(const float* __restrict__ a, const float* __restrict__ b, T* __restrict__ out,
                        size_t n, int nch, int h, int w, int nhwc) {
    const size_t hw = (size_t)h * w;
    for (size_t e = blockIdx.x * (size_t)blockDim.x + threadIdx.x; e < n; e += (size_t)gridDim.x * blockDim.x) {
        const float v = a[e] + (b ? b[e] : 0.f);
        const size_t t = e % hw;
        const size_t o = act_at(e / hw, (int)(t / w), (int)(t % w), h, w, hw, nch, nhwc);
        if constexpr (sizeof(T) == 2) out[o] = narrow_bf16(v);
        else out[o] = v;
    }
}

// g[ch*k*k + tap] = sum over batch b and positions of v * u(shifted): one
// block per (channel, tap), fixed-order tree reduction.
template <typename TU, typename TV>
__global__ void k_wgrad(const TU* __restrict__ u, const TV* __restrict__ v, float* __restrict__ g,
                        int B, int nch, int h, int w, int k, int nhwc) {
    __shared__ float red[NB];
    const int ch = blockIdx.x / (k * k), tap = blockIdx.x % (k * k);
    const int m = tap / k, q = tap % k, p2 = k / 2;
    float acc = 0.f;
    const size_t per = (size_t)B * h * w;
    for (size_t e = threadIdx.x; e < per; e += blockDim.x) {
        const int j = (int)(e % w);
        const int i = (int)((e / w) % h);
        const size_t b = e / ((size_t)h * w);
        const int ii = i + m - p2, jj = j + q - p2;
        if (ii < 0 || ii >= h || jj < 0 || jj >= w) continue;
        const size_t plane = b * nch + ch;
        const size_t ps = (size_t)h * w;
        acc += widen(v[act_at(plane, i, j, h, w, ps, nch, nhwc)]) * widen(u[act_at(plane, ii, jj, h, w, ps, nch, nhwc)]);
    }
    red[threadIdx.x] = acc;
    __syncthreads();
    for (int s = NB / 2; s > 0; s >>= 1) {
        if ((int)threadIdx.x < s) red[threadIdx.x] += red[threadIdx.x + s];
        __syncthreads();
    }
    if (threadIdx.x == 0) g[blockIdx.x] = red[0];
}

__global__ void k_wfinal(const float* __restrict__ gb, const float* __restrict__ gl, int C, int L,
                         int kb, int k, const float* __restrict__ w_lvl, const float* __restrict__ scale,
                         float* __restrict__ dw_base, float* __restrict__ dw_lvl,
                         float* __restrict__ dscale) {
    const int c = blockIdx.x;
    for (int t = threadIdx.x; t < kb * kb; t += blockDim.x) dw_base[(size_t)c * kb * kb + t] = gb[(size_t)c * kb * kb + t];
    for (int ls = threadIdx.x; ls < 4 * L; ls += blockDim.x) {
        const int l = ls / 4, s = ls % 4;
        const size_t pi = ((size_t)l * C + c) * 4 + s;
        const float* G = gl + ((size_t)l * 4 * C + c * 4 + s) * k * k;
        float d = 0.f;
        for (int t = 0; t < k * k; ++t) {
            dw_lvl[pi * k * k + t] = scale[pi] * G[t];
            d += w_lvl[pi * k * k + t] * G[t];
        }
        dscale[pi] = d;
    }
}

// side of level l's band grid (level 0: the plane itself)
inline int side(int n, int l) {
    for (int i = 0; i < l; ++i) n = (n + 1) / 2;
    return n;
}

// floats of level l's four bands over all P planes
size_t level_floats(int P, int H, int W, int l) { return (size_t)P * 4 * side(H, l) * side(W, l); }

// floats of the synthesis output of level l (an image of level l-1's size)
size_t carry_floats(int P, int H, int W, int l) { return (size_t)P * side(H, l - 1) * side(W, l - 1); }

}  // namespace

size_t naive_workspace_bytes(int B, int C, int H, int W, int L, int KB, int K, int op) {
    (void)KB;
    const int P = B * C;
    size_t f = 0;
    if (op == WTCONV_OP_BWD_WEIGHT) {
        for (int l = 1; l <= L; ++l) f += 2 * level_floats(P, H, W, l);
        f += (size_t)C * KB * KB + (size_t)L * 4 * C * K * K;
    } else {
        for (int l = 1; l <= L; ++l) f += 2 * level_floats(P, H, W, l) + carry_floats(P, H, W, l);
        f += (size_t)P * H * W;   // base output
    }
    return f * sizeof(float) + 256 * (3 * L + 4);
}

static float* carve(char*& p, size_t floats) {
    float* r = (float*)p;
    p += ((floats * sizeof(float) + 255) / 256) * 256;
    return r;
}

template <typename T>
static hipError_t data_chain(int B, int C, int H, int W, int L, int KB, int K, bool flip, int nhwc,
                             const T* in, const float* w_base, const float* w_lvl, const float* scale,
                             T* out, void* ws, hipStream_t st) {
    const int P = B * C;
    char* cur = (char*)ws;
    float* bands[6] = {};
    float* conv[6] = {};
    float* carry[6] = {};   // carry[l] = R_{l} at level-l resolution, l = 0..L-1
    for (int l = 1; l <= L; ++l) {
        bands[l] = carve(cur, level_floats(P, H, W, l));
        conv[l] = carve(cur, level_floats(P, H, W, l));
        carry[l - 1] = carve(cur, carry_floats(P, H, W, l));
    }
    float* ybase = carve(cur, (size_t)P * H * W);

    for (int l = 1; l <= L; ++l) {
        const int h = side(H, l - 1), w = side(W, l - 1);
        const size_t n = (size_t)P * side(H, l) * side(W, l);
        if (l == 1)
            hipLaunchKernelGGL(k_dwt<T>, dim3(grid_for(n)), dim3(NB), 0, st, in, (size_t)H * W, bands[1], P, h, w,
                               C, nhwc);
        else
            hipLaunchKernelGGL(k_dwt<float>, dim3(grid_for(n)), dim3(NB), 0, st, (const float*)bands[l - 1],
                               (size_t)4 * h * w, bands[l], P, h, w, C, 0);
    }
    for (int l = 1; l <= L; ++l) {
        const int h = side(H, l), w = side(W, l);
        const size_t n = (size_t)P * 4 * h * w;
        hipLaunchKernelGGL(k_dwconv<float>, dim3(grid_for(n)), dim3(NB), 0, st, (const float*)bands[l], conv[l],
                           4 * P, 4 * C, h, w, w_lvl + (size_t)(l - 1) * C * 4 * K * K, K, (int)flip, 0);
        hipLaunchKernelGGL(k_scale, dim3(grid_for(n)), dim3(NB), 0, st, conv[l], scale + (size_t)(l - 1) * C * 4,
                           4 * P, 4 * C, h * w);
    }
    for (int l = L; l >= 1; --l) {
        const int h = side(H, l), w = side(W, l);
        const size_t n = (size_t)P * h * w;
        if (l < L)
            hipLaunchKernelGGL(k_lladd, dim3(grid_for(n)), dim3(NB), 0, st, conv[l], (const float*)carry[l], P, h * w);
        hipLaunchKernelGGL(k_iwt, dim3(grid_for(n)), dim3(NB), 0, st, (const float*)conv[l], carry[l - 1], P, h, w,
                           side(H, l - 1), side(W, l - 1));
    }
    const size_t n = (size_t)P * H * W;
    hipLaunchKernelGGL(k_dwconv<T>, dim3(grid_for(n)), dim3(NB), 0, st, in, ybase, P, C, H, W, w_base, KB,
                       (int)flip, nhwc);
    hipLaunchKernelGGL(k_final<T>, dim3(grid_for(n)), dim3(NB), 0, st, (const float*)ybase,
                       (const float*)(L > 0 ? carry[0] : nullptr), out, n, C, H, W, nhwc);
    return hipGetLastError();
}

hipError_t naive_data_launch(int B, int C, int H, int W, int L, int KB, int K, bool bf16, bool flip,
                             bool nhwc, const void* in, const float* w_base, const float* w_lvl,
                             const float* scale, void* out, void* ws, hipStream_t stream) {
    if (bf16)
        return data_chain<bf16_t>(B, C, H, W, L, KB, K, flip, (int)nhwc, (const bf16_t*)in, w_base, w_lvl,
                                  scale, (bf16_t*)out, ws, stream);
    return data_chain<float>(B, C, H, W, L, KB, K, flip, (int)nhwc, (const float*)in, w_base, w_lvl, scale,
                             (float*)out, ws, stream);
}

template <typename T>
static hipError_t wgrad_chain(int B, int C, int H, int W, int L, int KB, int K, int nhwc, const T* x,
                              const T* dy,
                              const float* w_lvl, const float* scale, float* dw_base, float* dw_lvl,
                              float* dscale, void* ws, hipStream_t st) {
    const int P = B * C;
    char* cur = (char*)ws;
    float* bx[6] = {};
    float* bd[6] = {};
    for (int l = 1; l <= L; ++l) {
        bx[l] = carve(cur, level_floats(P, H, W, l));
        bd[l] = carve(cur, level_floats(P, H, W, l));
    }
    float* gb = carve(cur, (size_t)C * KB * KB);
    float* gl = carve(cur, (size_t)L * 4 * C * K * K);
    for (int l = 1; l <= L; ++l) {
        const int h = side(H, l - 1), w = side(W, l - 1);
        const size_t n = (size_t)P * side(H, l) * side(W, l);
        if (l == 1) {
            hipLaunchKernelGGL(k_dwt<T>, dim3(grid_for(n)), dim3(NB), 0, st, x, (size_t)H * W, bx[1], P, h, w, C,
                               nhwc);
            hipLaunchKernelGGL(k_dwt<T>, dim3(grid_for(n)), dim3(NB), 0, st, dy, (size_t)H * W, bd[1], P, h, w, C,
                               nhwc);
        } else {
            hipLaunchKernelGGL(k_dwt<float>, dim3(grid_for(n)), dim3(NB), 0, st, (const float*)bx[l - 1],
                               (size_t)4 * h * w, bx[l], P, h, w, C, 0);
            hipLaunchKernelGGL(k_dwt<float>, dim3(grid_for(n)), dim3(NB), 0, st, (const float*)bd[l - 1],
                               (size_t)4 * h * w, bd[l], P, h, w, C, 0);
        }
    }
    hipLaunchKernelGGL((k_wgrad<T, T>), dim3((unsigned)(C * KB * KB)), dim3(NB), 0, st, x, dy, gb, B, C, H, W, KB,
                       nhwc);
    for (int l = 1; l <= L; ++l)
        hipLaunchKernelGGL((k_wgrad<float, float>), dim3((unsigned)(4 * C * K * K)), dim3(NB), 0, st,
                           (const float*)bx[l], (const float*)bd[l], gl + (size_t)(l - 1) * 4 * C * K * K, B,
                           4 * C, side(H, l), side(W, l), K, 0);
    hipLaunchKernelGGL(k_wfinal, dim3((unsigned)C), dim3(64), 0, st, (const float*)gb, (const float*)gl, C, L,
                       KB, K, w_lvl, scale, dw_base, dw_lvl, dscale);
    return hipGetLastError();
}

hipError_t naive_bwdw_launch(int B, int C, int H, int W, int L, int KB, int K, bool bf16, bool nhwc,
                             const void* x, const void* dy, const float* w_lvl, const float* scale,
                             float* dw_base, float* dw_lvl, float* dscale, void* ws, hipStream_t stream) {
    if (bf16)
        return wgrad_chain<bf16_t>(B, C, H, W, L, KB, K, (int)nhwc, (const bf16_t*)x, (const bf16_t*)dy, w_lvl,
                                   scale, dw_base, dw_lvl, dscale, ws, stream);
    return wgrad_chain<float>(B, C, H, W, L, KB, K, (int)nhwc, (const float*)x, (const float*)dy, w_lvl, scale,
                              dw_base, dw_lvl, dscale, ws, stream);
}

}  // namespace wtc
