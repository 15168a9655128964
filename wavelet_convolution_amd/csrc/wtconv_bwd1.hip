// Single-pass backward of a one-level whole plane (L = 1). One workgroup per
// channel and chunk of images reads x and dy from HBM once and produces both
// dx and the partial tap sums of every weight gradient:
//  - dx is the layer's transpose: the Haar analysis of dy, the base and
//    level taps turned by 180 degrees with the band scale and 1/4 folded in,
//    and the closed-form synthesis (the reformulations of the abstract of
//    arXiv:2608.10805, "I/O-aware reformulation of wavelet convolution");
//  - the weight gradients are correlations of the Haar pyramids of x and dy:
//    dy against the bordered x plane for the base taps, each dy band against
//    the same bordered band of x for the level taps.
//
// A step holds NPW planes of the chunk in LDS: bordered dy and its four
// bordered bands (the dx convolutions read their windows, the tap sums their
// values), bordered x and its four bordered bands (the tap sums' windows).
// Each of the four wavefronts takes one role, 350 multiply-adds per lane and
// step at 14x14: dx's base strips, dx's level-1 strips, the base tap sums,
// the level-1 tap sums. dx comes out exactly as the column kernel computes
// it (same layout, strips, staged taps and order of operations), so it
// equals the two-call dx bit for bit; the tap sums group the products
// differently from the weight-gradient kernel and agree with it to rounding.
// The fixed-order second stage (chunk sum, scale, normalisation) is the
// weight gradient's own.
#include "wtconv_bwd1.h"
#include "wtconv_bwdw_body.h"
#include "wtconv_plans.h"

namespace wtc {
namespace {

// P: the column plan whose layout and dx strips the kernel shares (L = 1,
// 256 threads, NPW planes per step).
template <class P>
struct Bwd1Plan {
    using CP = P;
    static constexpr int H = P::H, W = P::W, KB = P::KB, K = P::K, NT = P::NT, NPW = P::NPW;
    static_assert(P::L == 1 && NT == 256, "one level, four wavefronts");
    static constexpr int RB = P::RB, R1 = P::rl(1);
    // dx base strips: one per lane of one wavefront, the whole plane height
    static_assert(RB == H && P::LPB == 16 && NPW * P::NIB == 64, "dx base strips fill one wavefront");
    // dx level-1 strips: two per lane of one wavefront, the four bands of a
    // plane on each 32 lanes
    static_assert(R1 == H / 2 && P::lpl(1) == 8 && NPW * P::nil(1) == 128, "dx level-1 strips: two per lane");
    // tap sums: base strips of RT rows, two row blocks per lane
    static constexpr int RT = H / 2;
    static_assert(H % 2 == 0 && NPW == 4, "tap strips: one (plane, column) per lane");
    // per plane: bordered dy (A), its bands (B), bordered x (X), its bands (U)
    static constexpr int OA = 0, OB = P::ASIZE, OX = P::ASIZE + P::BSIZE, OU = OX + P::XSIZE;
    static constexpr int PLF = round_up(OU + P::BSIZE, 4);
    static constexpr int TOTAL = NPW * PLF + P::KB2P + 4 * P::K2P;
    static constexpr int KK = KB * KB > K * K ? KB * KB : K * K;
    static constexpr int TAPS = KB * KB + 4 * K * K;
    static_assert(4 * KB * KB + 64 * K * K <= NPW * PLF, "reduction scratch fits the planes");
    // stream-in cells: one Haar block (2 x 2 activations of x and of dy) per
    // thread on a power-of-two grid over the level-1 positions
    static constexpr int GC = strip_lanes(W / 2), NG = strip_lanes(H / 2) * GC;
    static_assert(NPW * NG == NT && P::VA == 2 && P::XO % 2 == 0 && P::SX % 2 == 0, "one cell per thread");
    static constexpr int WG_PER_CU = (160 * 1024) / (TOTAL * 4);
    static constexpr int WAVES_PER_EU = WG_PER_CU > 8 ? 8 : (WG_PER_CU < 1 ? 1 : WG_PER_CU);
};

template <class Q, typename T>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Q::WAVES_PER_EU)))
void bwd1_kernel(const T* __restrict__ x, const T* __restrict__ dy, const float* __restrict__ w_base,
                 const float* __restrict__ w_lvl, const float* __restrict__ scale, T* __restrict__ dx,
                 float* __restrict__ part, int B, int C, int bpc) {
    using P = typename Q::CP;
    constexpr int H = Q::H, W = Q::W, KB = Q::KB, K = Q::K, NPW = Q::NPW, RB = Q::RB, R1 = Q::R1, RT = Q::RT;
    constexpr int PB = P::PB, PK = P::PK, SX = P::SX, XO = P::XO, S1 = P::su(1), BS1 = P::bandsz(1);
    constexpr int KB2P = P::KB2P, K2P = P::K2P, PLF = Q::PLF, H1 = H / 2, W1 = W / 2;
    constexpr int OA = Q::OA, OB = Q::OB, OX = Q::OX, OU = Q::OU, GC = Q::GC, NG = Q::NG;
    __shared__ __attribute__((aligned(16))) float lds[Q::TOTAL];
    float* const WB = lds + NPW * PLF;   // base taps, turned
    float* const WL = WB + KB2P;         // level taps, turned, band scale and 1/4 folded in

    const int tid = threadIdx.x, lane = tid & 63;
    const int role = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int c = blockIdx.x % C, chunk = blockIdx.x / C;
    const int b0 = chunk * bpc, b1 = min(B, b0 + bpc);

    // this thread's stream-in cell: plane cp, level-1 position (ci, cj)
    const int cp = tid / NG, ci = (tid % NG) / GC, cj = tid % GC;
    const bool creal = ci < H1 && cj < W1;
    RawVec<T, 2> vx[2], vd[2];
    auto issue = [&](int b) {
        if (creal && b + cp < b1) {
            const size_t off = ((size_t)(b + cp) * C + c) * (H * W) + (size_t)(2 * ci) * W + 2 * cj;
            load_raw<T, 2>(x + off, vx[0]);
            load_raw<T, 2>(x + off + W, vx[1]);
            load_raw<T, 2>(dy + off, vd[0]);
            load_raw<T, 2>(dy + off + W, vd[1]);
        } else {   // a cell off the plane or a plane past the chunk: zeros
#pragma unroll
            for (int i = 0; i < RawVec<T, 2>::N; ++i) vx[0].w[i] = vx[1].w[i] = vd[0].w[i] = vd[1].w[i] = 0u;
        }
    };
    // The first step's loads go out first, the taps' right after them; the
    // taps are staged (as the column kernel stages them for the
    // backward-data pass) once both are in flight, so the two global round
    // trips overlap. Every plane region is cleared once in between: no step
    // writes a border cell.
    issue(b0);
    static_assert(KB * KB <= 256 && 4 * P::K2P <= 256, "one tap of each kind per thread");
    const float wb = w_base[(size_t)c * KB * KB + (KB * KB - 1 - min(tid, KB * KB - 1))];
    const int ts = min(tid, 4 * K2P - 1) / K2P, ttap = min(tid, 4 * K2P - 1) - ts * K2P;
    const float sc = scale[(size_t)c * 4 + ts];
    const float wl = w_lvl[((size_t)c * 4 + ts) * K * K + (K * K - 1 - min(ttap, K * K - 1))];
    {
        float4* const z = reinterpret_cast<float4*>(lds);
        for (int t = tid; t < NPW * PLF / 4; t += 256) z[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    if (tid < KB2P) WB[tid] = tid < KB * KB ? wb : 0.f;
    if (tid < 4 * K2P) WL[tid] = ttap < K * K ? wl * (sc * (1.0f / 4.0f)) : 0.f;

    // One register array serves the role of each wavefront (a wavefront's
    // role never changes): dx's base rows, its two level-1 strips, or the
    // tap sums that accumulate over the chunk. No two roles share a
    // wavefront, so they need no registers of their own (separate arrays
    // spilled at this occupancy).
    static_assert(RB <= Q::KK && 2 * R1 <= Q::KK, "role registers");
    float acc[Q::KK];
#pragma unroll
    for (int t = 0; t < Q::KK; ++t) acc[t] = 0.f;
    float(&yb)[RB] = *reinterpret_cast<float(*)[RB]>(&acc[0]);
    float(&z1a)[R1] = *reinterpret_cast<float(*)[R1]>(&acc[0]);
    float(&z1b)[R1] = *reinterpret_cast<float(*)[R1]>(&acc[R1]);

    // Stream-in of one step (all threads): the cell's x and dy rows into the
    // bordered planes, their four bands, then the next step's loads; the
    // barrier before it waits for the previous step's reads (or the zeros
    // and taps), the one after it for its stores.
    auto stream_in = [&](int b) {
        __syncthreads();
        float fx0[2], fx1[2], fd0[2], fd1[2];
        widen_raw<T, 2>(vx[0], fx0);
        widen_raw<T, 2>(vx[1], fx1);
        widen_raw<T, 2>(vd[0], fd0);
        widen_raw<T, 2>(vd[1], fd1);
        if (b + NPW < b1) issue(b + NPW);   // the next step's loads fly during this one
        if (creal) {
            float* const pl = lds + cp * PLF;
            const int xr = PB + 2 * ci, xc = XO + 2 * cj;
            store_vec<2>(pl + OA + xr * SX + xc, fd0);
            store_vec<2>(pl + OA + (xr + 1) * SX + xc, fd1);
            store_vec<2>(pl + OX + xr * SX + xc, fx0);
            store_vec<2>(pl + OX + (xr + 1) * SX + xc, fx1);
            float u[4], v[4];
            haar4(fx0[0], fx0[1], fx1[0], fx1[1], u[0], u[1], u[2], u[3]);
            haar4(fd0[0], fd0[1], fd1[0], fd1[1], v[0], v[1], v[2], v[3]);
            const int o = (PK + ci) * S1 + PK + cj;
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                pl[OB + s * BS1 + o] = v[s];
                pl[OU + s * BS1 + o] = u[s];
            }
        }
        __syncthreads();
    };

    // Each role runs its own loop over the chunk's steps (the role is
    // uniform over a wavefront, so these are scalar branches), so that only
    // its own addresses stay live; every wavefront passes the same four
    // barriers per step: two in the stream-in, one after the convolutions
    // and tap sums, one after the level-1 results are stored.
    if (role == 0) {
        // dx base strips: plane lane / 16, column lane % 16; then the
        // synthesis and the store of dx
        const int p = lane >> 4, w = lane & 15;
        const float* const src = lds + p * PLF + OA + XO - PB + w;
        // y[h][w] = base + A + sign(h & 1) B, A = Z0 + sign(w & 1) Z2,
        // B = Z1 + sign(w & 1) Z3 at (h / 2, w / 2)
        const float* const Z = lds + p * PLF + OB + PK * S1 + PK + (w >> 1);
        const float sw = (w & 1) ? -1.f : 1.f;
        for (int b = b0; b < b1; b += NPW) {
            stream_in(b);
            if (w < W) conv_col<KB, RB, SX>(src, WB, yb);
            __syncthreads();
            __syncthreads();
            if (w < W && b + p < b1) {
#pragma unroll
                for (int q = 0; q < H1; ++q) {
                    const float* z = Z + q * S1;
                    const float a = __builtin_fmaf(sw, z[2 * BS1], z[0]);
                    const float bb = __builtin_fmaf(sw, z[3 * BS1], z[BS1]);
                    const float plus = a + bb, minus = a - bb;
                    yb[2 * q] += plus;
                    yb[2 * q + 1] += minus;
                }
                T* __restrict__ dst = dx + ((size_t)(b + p) * C + c) * (H * W) + w;
                if constexpr (sizeof(T) == 2) {
#pragma unroll
                    for (int o = 0; o < RB; o += 2) {
                        const uint32_t pr = narrow_bf16x2(yb[o], yb[o + 1]);
                        dst[o * W] = (bf16_t)(pr & 0xffffu);
                        dst[(o + 1) * W] = (bf16_t)(pr >> 16);
                    }
                } else {
#pragma unroll
                    for (int o = 0; o < RB; ++o) dst[o * W] = yb[o];
                }
            }
        }
    } else if (role == 1) {
        // dx level-1 strips: item lane + 64 it is plane item / 32, band
        // (item / 8) % 4, column item % 8; the results go over their own
        // bands once every read of them is done
        const int s = (lane >> 3) & 3, j = lane & 7, p0 = lane >> 5;
        for (int b = b0; b < b1; b += NPW) {
            stream_in(b);
            if (j < W1) {
                conv_col<K, R1, S1>(lds + p0 * PLF + OB + s * BS1 + j, WL + s * K2P, z1a);
                conv_col<K, R1, S1>(lds + (p0 + 2) * PLF + OB + s * BS1 + j, WL + s * K2P, z1b);
            }
            __syncthreads();
            if (j < W1) {
#pragma unroll
                for (int o = 0; o < R1; ++o) {
                    lds[p0 * PLF + OB + s * BS1 + (PK + o) * S1 + PK + j] = z1a[o];
                    lds[(p0 + 2) * PLF + OB + s * BS1 + (PK + o) * S1 + PK + j] = z1b[o];
                }
            }
            __syncthreads();
        }
    } else if (role == 2) {
        // base tap sums: plane lane / 16, column lane % 16, both row blocks
        const int p = lane >> 4, w = lane & 15;
        for (int b = b0; b < b1; b += NPW) {
            stream_in(b);
            if (w < W) {
#pragma unroll
                for (int rb = 0; rb < 2; ++rb)
                    taps_col<KB, RT, SX, SX>(lds + p * PLF + OX + rb * RT * SX + XO - PB + w,
                                            lds + p * PLF + OA + (PB + rb * RT) * SX + XO + w, acc);
            }
            __syncthreads();
            __syncthreads();
        }
    } else {
        // level tap sums: band (lane / 8) % 4, column lane % 8, planes
        // lane / 32 and lane / 32 + 2
        const int s = (lane >> 3) & 3, j = lane & 7;
        for (int b = b0; b < b1; b += NPW) {
            stream_in(b);
            if (j < W1) {
#pragma unroll
                for (int it = 0; it < 2; ++it) {
                    const int p = (lane >> 5) + 2 * it;
                    taps_col<K, R1, S1, S1>(lds + p * PLF + OU + s * BS1 + j,
                                           lds + p * PLF + OB + s * BS1 + PK * S1 + PK + j, acc);
                }
            }
            __syncthreads();
            __syncthreads();
        }
    }

    // ------------------------------------------------ the chunk's tap sums
    // base: each 16-lane row's sum (DPP), then the four rows in order; level
    // band s: its 16 lanes (lane / 8 % 4 == s) in lane order
    __syncthreads();   // the planes become reduction scratch
    float* const red = lds;   // [4 rows][KB*KB] base, then [64 lanes][K*K] level
    if (role == 2) {
#pragma unroll
        for (int t = 0; t < KB * KB; ++t) acc[t] = row_sum(acc[t]);
        if ((lane & 15) == 0) {
#pragma unroll
            for (int t = 0; t < KB * KB; ++t) red[(lane >> 4) * KB * KB + t] = acc[t];
        }
    } else if (role == 3) {
#pragma unroll
        for (int t = 0; t < K * K; ++t) red[4 * KB * KB + lane * K * K + t] = acc[t];
    }
    __syncthreads();
    float* const dst = part + ((size_t)chunk * C + c) * Q::TAPS;
    for (int t = tid; t < Q::TAPS; t += 256) {
        float v = 0.f;
        if (t < KB * KB) {
#pragma unroll
            for (int q = 0; q < 4; ++q) v += red[q * KB * KB + t];
        } else {
            const int r = t - KB * KB, s = r / (K * K), tap = r - s * (K * K);
#pragma unroll
            for (int h = 0; h < 2; ++h)
#pragma unroll
                for (int i = 0; i < 8; ++i) v += red[4 * KB * KB + (32 * h + 8 * s + i) * K * K + tap];
        }
        dst[t] = v;   // base taps, then the level-1 taps ordered [4][K*K]
    }
}

// images per chunk: about one workgroup per resident slot of the chip
template <class Q>
int bwd1_bpc(int B, int C) {
    return chunk_units(B, C, cu_count() * Q::WG_PER_CU);
}

template <class Q>
size_t bwd1_ws(int B, int C) {
    return (size_t)cdiv(B, bwd1_bpc<Q>(B, C)) * C * Q::TAPS * sizeof(float);
}

template <class Q, typename T>
hipError_t bwd1_launch(const void* x, const void* dy, const float* w_base, const float* w_lvl, const float* scale,
                       void* dx, float* dw_base, float* dw_lvl, float* dscale, void* ws, int B, int C,
                       hipStream_t stream) {
    const int bpc = bwd1_bpc<Q>(B, C), nch = cdiv(B, bpc);
    float* const part = (float*)ws;
    hipLaunchKernelGGL((bwd1_kernel<Q, T>), dim3((unsigned)(nch * C)), dim3(256), 0, stream, (const T*)x,
                       (const T*)dy, w_base, w_lvl, scale, (T*)dx, part, B, C, bpc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // the weight gradient's second stage: the chunk sums in chunk order, the
    // level taps scaled and normalised, dscale from them
    return launch_bwdw_finalize(part, nch, 1, nullptr, 0, C, 1, Q::KB, Q::K, w_lvl, scale, dw_base, dw_lvl, dscale,
                                stream);
}

typedef hipError_t (*bwd1l_fn)(const void*, const void*, const float*, const float*, const float*, void*, float*,
                               float*, float*, void*, int, int, hipStream_t);
struct Bwd1LEntry {
    int H, W, L, KB, K;
    bwd1l_fn fn[2];   // [dtype: 0 fp32, 1 bf16]
    size_t (*ws)(int B, int C);
};

// the one-level stage plane of 14x14 with 5x5 kernels, four planes per step
typedef Bwd1Plan<ColPlan<14, 14, 1, 5, 5, 256, 14, 7, 8, 4>> B1_14_k55;

#define WTC_BWD1L(Q) {Q::H, Q::W, 1, Q::KB, Q::K, {bwd1_launch<Q, float>, bwd1_launch<Q, bf16_t>}, bwd1_ws<Q>}
const Bwd1LEntry kBwd1LEntries[] = {WTC_BWD1L(B1_14_k55)};

const Bwd1LEntry* find_bwd1l(int H, int W, int L, int KB, int K) {
    for (const Bwd1LEntry& e : kBwd1LEntries)
        if (e.H == H && e.W == W && e.L == L && e.KB == KB && e.K == K) return &e;
    return nullptr;
}

}  // namespace

size_t bwd1_level_workspace_bytes(int B, int C, int H, int W, int L, int KB, int K) {
    const Bwd1LEntry* e = find_bwd1l(H, W, L, KB, K);
    return e ? e->ws(B, C) : (size_t)-1;
}

hipError_t bwd1_level_launch(int B, int C, int H, int W, int L, int KB, int K, bool bf16, const void* x,
                             const void* dy, const float* w_base, const float* w_lvl, const float* scale, void* dx,
                             float* dw_base, float* dw_lvl, float* dscale, void* ws, hipStream_t stream) {
    const Bwd1LEntry* e = find_bwd1l(H, W, L, KB, K);
    if (!e) return hipErrorInvalidValue;
    return e->fn[bf16 ? 1 : 0](x, dy, w_base, w_lvl, scale, dx, dw_base, dw_lvl, dscale, ws, B, C, stream);
}

}  // namespace wtc
