// Fused WTConv backward-weight kernel for gfx950.
//
// For one channel c the gradients are correlations of the two Haar pyramids
// (the abstract of arXiv:2608.10805, reformulation (3): the learned scales
// fold out of the convolution, so one unscaled correlation G serves both the
// kernel and the scale gradient):
//   G_base[m][n] = sum_{b,h,w} dy[h][w] * x[h+m-kb/2][w+n-kb/2]
//   G_l^s[m][n]  = sum_{b,i,j} V_l^s[i][j] * U_l^s[i+m-k/2][j+n-k/2] * 4^-l
// with U_l, V_l the unnormalised level-l bands of x and dy (2^l times the
// orthonormal ones). Then dw_lvl = scale * G and dscale = sum(w_lvl * G).
//
// Stage 1: one workgroup per (channel, chunk of the batch), 8 wavefronts.
// Each plane of the chunk is streamed into LDS once (the next plane's loads
// are issued while the current one's level taps run); both Haar pyramids are
// built on chip; every wavefront owns one band of some levels (see BwPlan).
// Every lane keeps its tap sums in registers across the whole chunk; at the
// end they are reduced across the wavefront with shuffles, across
// wavefronts through LDS, and one partial per (chunk, channel, tap) goes to
// the workspace.
// Stage 2: one workgroup per channel sums the chunks in a fixed order and
// applies the scale and normalisation. No atomics: results are bitwise
// reproducible.
#include "wtconv_bwdw.h"
#include "wtconv_device.h"
#include "wtconv_plans.h"

namespace wtc {

// acc[m*K+n] += sum_{o,q} v[o*SV+q] * u[(o+m)*SU + q+n]: tap sums of an
// OR x OC tile of dy-side values v against the matching window of the
// bordered x-side plane u (u points at the window's top-left corner).
// Scheduling barriers keep each call's tile and window rows live only
// during the call.
template <int K, int OR, int OC, int SU, int SV, int NA>
__device__ __forceinline__ void taps_tile(const float* u, const float* v, float (&acc)[NA]) {
    static_assert(NA >= K * K, "accumulator slot too small");
    __builtin_amdgcn_sched_barrier(0);
    float vt[OR][OC];
#pragma unroll
    for (int o = 0; o < OR; ++o)
#pragma unroll
        for (int q = 0; q < OC; ++q) vt[o][q] = v[o * SV + q];
#pragma unroll
    for (int r = 0; r < OR + K - 1; ++r) {
        float win[OC + K - 1];
#pragma unroll
        for (int q = 0; q < OC + K - 1; ++q) win[q] = u[r * SU + q];
#pragma unroll
        for (int o = 0; o < OR; ++o) {
            const int m = r - o;
            if (m < 0 || m >= K) continue;
#pragma unroll
            for (int n = 0; n < K; ++n)
#pragma unroll
                for (int q = 0; q < OC; ++q) acc[m * K + n] = __builtin_fmaf(vt[o][q], win[q + n], acc[m * K + n]);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// H x W plane, L >= 1 levels; BR x BC dy positions per base work item.
// LDS: x (border KB/2), dy, the bordered x bands U_1..U_L (border K/2) and
// the unbordered dy bands V_1..V_L all stay resident.
//
// Work split, 8 wavefronts in two groups of four; wavefront w owns band
// s = w % 4 and keeps its tap sums for the whole chunk in registers:
//   group A (w < 4): a quarter of the base taps (slot 0), levels 3, 5 (slots 1, 2)
//   group B (w >= 4): level 1 (slot 0), levels 2, 4 (slots 1, 2)
// which balances the multiply-adds (level 1 alone equals the base work) and
// keeps every lane at about two or three slots of taps.
template <int H_, int W_, int L_, int KB_, int K_, int BR_, int BC_>
struct BwPlan {
    static constexpr int H = H_, W = W_, L = L_, KB = KB_, K = K_, BR = BR_, BC = BC_;
    static constexpr int NT = 512, NW = 8;
    static constexpr int PB = KB / 2, PK = K / 2;
    static_assert(L >= 1 && L <= 5 && H % (1 << L) == 0 && W % (1 << L) == 0, "plane must divide into 2^L blocks");
    static_assert(H % BR == 0 && W % BC == 0, "base tile must divide the plane");
    static constexpr int SX = odd_stride(W + 2 * PB);
    static constexpr int XSIZE = (H + 2 * PB) * SX;
    static constexpr int DSIZE = H * W;
    static constexpr int su(int l) { return odd_stride((W >> l) + 2 * PK); }
    static constexpr int bandsz(int l) { return ((H >> l) + 2 * PK) * su(l); }
    static constexpr int vsz(int l) { return (H >> l) * (W >> l); }
    static constexpr int uoff(int l) {
        int o = 0;
        for (int q = 1; q < l; ++q) o += 4 * bandsz(q);
        return o;
    }
    static constexpr int voff(int l) {
        int o = 0;
        for (int q = 1; q < l; ++q) o += 4 * vsz(q);
        return o;
    }
    static constexpr int UTOT = uoff(L + 1), VTOT = voff(L + 1);
    // role slots: group A = base, 3, 5; group B = 1, 2, 4
    static constexpr int NSLOT = 1 + (L >= 2 ? 1 : 0) + (L >= 4 ? 1 : 0);
    static constexpr int SLOT0 = KB * KB > K * K ? KB * KB : K * K;   // base or level-1 taps
    static constexpr int RED = NW * SLOT0 + NW * (NSLOT - 1) * K * K;   // reduction scratch
    static constexpr int DATA = XSIZE + DSIZE + UTOT + VTOT;
    static constexpr int LDS_FLOATS = DATA > RED ? DATA : RED;
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "plane does not fit in LDS");
    static constexpr int NI = (H / BR) * (W / BC);
    static constexpr int TAPS = KB * KB + 4 * L * K * K;
    static constexpr Tile band_tile(int l) { return pick_tile(H >> l, W >> l, 64); }
    static constexpr int WG_PER_CU = (160 * 1024) / (LDS_FLOATS * 4);
    static constexpr int WAVES_PER_EU_LDS = WG_PER_CU * NW / 4;
    // registers bound the occupancy too: each lane holds its tap slots plus
    // about 48 registers of tiles and addresses (512 VGPRs per SIMD lane)
    static constexpr int REGS = SLOT0 + (NSLOT - 1) * K * K + 48;
    static constexpr int WAVES_PER_EU_REG = 512 / (REGS <= 128 ? 128 : (REGS <= 168 ? 168 : 256));
    static constexpr int WAVES_PER_EU_MIN = WAVES_PER_EU_LDS < WAVES_PER_EU_REG ? WAVES_PER_EU_LDS : WAVES_PER_EU_REG;
    static constexpr int WAVES_PER_EU = WAVES_PER_EU_MIN < 1 ? 1 : WAVES_PER_EU_MIN;

    // group and slot of level l (1..5)
    static constexpr int group_of(int l) { return (l == 3 || l == 5) ? 0 : 1; }
    static constexpr int slot_of(int l) { return l == 1 ? 0 : (l == 2 || l == 3) ? 1 : 2; }

    template <class F>
    __device__ static __forceinline__ void for_levels(F&& f) {
        lv_impl(f, std::make_integer_sequence<int, L>{});
    }
    template <class F, int... I>
    __device__ static __forceinline__ void lv_impl(F& f, std::integer_sequence<int, I...>) {
        (f(std::integral_constant<int, I + 1>{}), ...);
    }
};

template <class P, typename T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(P::WAVES_PER_EU)))
void bwdw_kernel(const T* __restrict__ x, const T* __restrict__ dy, float* __restrict__ part, int B,
                 int C, int bpc) {
    constexpr int H = P::H, W = P::W, L = P::L, KB = P::KB, K = P::K, NT = P::NT;
    constexpr int PB = P::PB, PK = P::PK, SX = P::SX, H1 = H / 2, W1 = W / 2;
    constexpr int BR = P::BR, BC = P::BC, NI = P::NI, TPR = W / BC;
    constexpr int NSLOT = P::NSLOT, SLOT0 = P::SLOT0;
    constexpr int V = vec_elems<T>(W, H * W);
    constexpr int NV = H * W / V;
    constexpr int NL = cdiv(NV, NT);

    __shared__ __attribute__((aligned(16))) float lds[P::LDS_FLOATS];
    float* X = lds;
    float* DY = X + P::XSIZE;
    float* U = DY + P::DSIZE;
    float* Vb = U + P::UTOT;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int grp = wave >> 2, band = wave & 3, gtid = tid & 255;
    const int c = blockIdx.x % C, chunk = blockIdx.x / C;
    const int b0 = chunk * bpc, b1 = min(B, b0 + bpc);

    // borders stay zero for the whole chunk: nothing writes them
    zero_border<1, H, W, PB, SX>(X, tid, NT);
    P::for_levels([&](auto lc) {
        constexpr int l = decltype(lc)::value;
        zero_border<4, (H >> l), (W >> l), PK, P::su(l)>(U + P::uoff(l), tid, NT);
    });

    float acc0[SLOT0];
    float accl[NSLOT > 1 ? NSLOT - 1 : 1][K * K];
#pragma unroll
    for (int t = 0; t < SLOT0; ++t) acc0[t] = 0.f;
#pragma unroll
    for (int j = 0; j < (NSLOT > 1 ? NSLOT - 1 : 1); ++j)
#pragma unroll
        for (int t = 0; t < K * K; ++t) accl[j][t] = 0.f;

    // raw global loads of the next plane, issued ahead of the level taps
    float vx[NL][V], vd[NL][V];
    auto issue_loads = [&](int b) {
        const size_t plane = (size_t)b * C + c;
        const T* __restrict__ xs = x + plane * H * W;
        const T* __restrict__ ds = dy + plane * H * W;
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int q = tid + k * NT;
            if (NV % NT == 0 || q < NV) {
                load_vec<T, V>(xs + q * V, vx[k]);
                load_vec<T, V>(ds + q * V, vd[k]);
            }
        }
    };
    if (b0 < b1) issue_loads(b0);

    for (int b = b0; b < b1; ++b) {
        // ------------------------------------------------ P0: stream in
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int q = tid + k * NT;
            if (NV % NT == 0 || q < NV) {
                const int e = q * V, r = e / W, col = e - r * W;
#pragma unroll
                for (int i = 0; i < V; ++i) {
                    X[(r + PB) * SX + col + PB + i] = vx[k][i];
                    DY[e + i] = vd[k][i];
                }
            }
        }
        __syncthreads();
        // ------------------------------------- P1: base taps, level 1 bands
        if (grp == 0) {
            for (int item = gtid; item < NI; item += 256) {
                const int ti = item / TPR, tj = item - ti * TPR;
                const int h0 = BR * ti, w0 = BC * tj;
                taps_tile<KB, BR, BC, SX, W>(X + h0 * SX + w0, DY + h0 * W + w0, acc0);
            }
        }
        {
            constexpr int S1 = P::su(1), BS1 = P::bandsz(1), VS1 = P::vsz(1);
            for (int q = tid; q < H1 * W1; q += NT) {
                const int i = q / W1, j = q - i * W1;
                const float* x2 = X + (PB + 2 * i) * SX + PB + 2 * j;
                const float* d2 = DY + 2 * i * W + 2 * j;
                float u[4], v[4];
                haar4(x2[0], x2[1], x2[SX], x2[SX + 1], u[0], u[1], u[2], u[3]);
                haar4(d2[0], d2[1], d2[W], d2[W + 1], v[0], v[1], v[2], v[3]);
#pragma unroll
                for (int s = 0; s < 4; ++s) {
                    U[s * BS1 + (PK + i) * S1 + PK + j] = u[s];
                    Vb[s * VS1 + q] = v[s];
                }
            }
        }
        __syncthreads();
        // ----------------------------------------- P2: levels 2..L analysis
        P::for_levels([&](auto lc) {
            constexpr int l = decltype(lc)::value;
            if constexpr (l >= 2) {
                constexpr int hl = H >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), VSl = P::vsz(l);
                constexpr int Sp = P::su(l - 1), wp = W >> (l - 1);
                const float* LLu = U + P::uoff(l - 1) + PK * Sp + PK;
                const float* LLv = Vb + P::voff(l - 1);
                float* Ul = U + P::uoff(l);
                float* Vl = Vb + P::voff(l);
                for (int q = tid; q < hl * wl; q += NT) {
                    const int i = q / wl, j = q - i * wl;
                    const float* x2 = LLu + 2 * i * Sp + 2 * j;
                    const float* d2 = LLv + 2 * i * wp + 2 * j;
                    float u[4], v[4];
                    haar4(x2[0], x2[1], x2[Sp], x2[Sp + 1], u[0], u[1], u[2], u[3]);
                    haar4(d2[0], d2[1], d2[wp], d2[wp + 1], v[0], v[1], v[2], v[3]);
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        Ul[s * BSl + (PK + i) * Sl + PK + j] = u[s];
                        Vl[s * VSl + q] = v[s];
                    }
                }
                __syncthreads();
            }
        });
        // the next plane's loads fly while the level taps run; P0 of the
        // next plane writes only x and dy, which the level taps do not read
        if (b + 1 < b1) issue_loads(b + 1);
        // --------------------------- P3: level taps, one band per wavefront
        P::for_levels([&](auto lc) {
            constexpr int l = decltype(lc)::value;
            constexpr int hl = H >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), VSl = P::vsz(l);
            constexpr Tile tl = P::band_tile(l);
            constexpr int RR = tl.r, CC = tl.c, TPRl = wl / CC, NIl = (hl / RR) * TPRl;
            if (grp == P::group_of(l)) {
                const float* Us = U + P::uoff(l) + band * BSl;
                const float* Vs = Vb + P::voff(l) + band * VSl;
                for (int item = lane; item < NIl; item += 64) {
                    const int ti = item / TPRl, tj = item - ti * TPRl;
                    if constexpr (P::slot_of(l) == 0)
                        taps_tile<K, RR, CC, Sl, wl>(Us + RR * ti * Sl + CC * tj, Vs + RR * ti * wl + CC * tj, acc0);
                    else
                        taps_tile<K, RR, CC, Sl, wl>(Us + RR * ti * Sl + CC * tj, Vs + RR * ti * wl + CC * tj,
                                                     accl[P::slot_of(l) - 1]);
                }
            }
        });
    }

    // ------------------------------------------------------ reduction
#pragma unroll
    for (int t = 0; t < SLOT0; ++t) acc0[t] = wave_sum(acc0[t]);
#pragma unroll
    for (int j = 0; j < NSLOT - 1; ++j)
#pragma unroll
        for (int t = 0; t < K * K; ++t) accl[j][t] = wave_sum(accl[j][t]);
    __syncthreads();  // all of LDS becomes reduction scratch
    float* red0 = lds;                     // [NW][SLOT0]
    float* redl = lds + P::NW * SLOT0;     // [NW][NSLOT-1][K*K]
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < SLOT0; ++t) red0[wave * SLOT0 + t] = acc0[t];
#pragma unroll
        for (int j = 0; j < NSLOT - 1; ++j)
#pragma unroll
            for (int t = 0; t < K * K; ++t) redl[(wave * (NSLOT - 1) + j) * K * K + t] = accl[j][t];
    }
    __syncthreads();
    float* dst = part + ((size_t)chunk * C + c) * P::TAPS;
    for (int t = tid; t < P::TAPS; t += NT) {
        float v;
        if (t < KB * KB) {
            v = red0[t];   // group A, waves 0..3 in order
#pragma unroll
            for (int w = 1; w < 4; ++w) v += red0[w * SLOT0 + t];
        } else {
            const int r = t - KB * KB, ls = r / (K * K), tap = r - ls * (K * K);
            const int l = ls / 4 + 1, s = ls - (l - 1) * 4;   // taps are ordered [L][4][K*K]
            const int w = P::group_of(l) * 4 + s, slot = P::slot_of(l);
            v = slot == 0 ? red0[w * SLOT0 + tap] : redl[(w * (NSLOT - 1) + slot - 1) * K * K + tap];
        }
        dst[t] = v;
    }
}

// Stage 2: fixed-order sum over chunks, then scale and normalisation.
__global__ __launch_bounds__(256) void bwdw_finalize(const float* __restrict__ part, int nchunk, int C,
                                                     int L, int KB, int K,
                                                     const float* __restrict__ w_lvl,
                                                     const float* __restrict__ scale,
                                                     float* __restrict__ dw_base,
                                                     float* __restrict__ dw_lvl,
                                                     float* __restrict__ dscale) {
    __shared__ float G[49 + 4 * 5 * 49];
    const int c = blockIdx.x, tid = threadIdx.x;
    const int kb2 = KB * KB, k2 = K * K, taps = kb2 + 4 * L * k2;
    for (int t = tid; t < taps; t += blockDim.x) {
        float a = 0.f;
        for (int ch = 0; ch < nchunk; ++ch) a += part[((size_t)ch * C + c) * taps + t];
        if (t >= kb2) {
            const int l = (t - kb2) / (4 * k2);   // 0-based level
            a *= 1.0f / (float)(1 << (2 * (l + 1)));
        }
        G[t] = a;
    }
    __syncthreads();
    for (int t = tid; t < taps; t += blockDim.x) {
        if (t < kb2) {
            dw_base[(size_t)c * kb2 + t] = G[t];
        } else {
            const int r = t - kb2, ls = r / k2, tap = r - ls * k2, l = ls / 4, s = ls - 4 * l;
            const size_t pi = ((size_t)l * C + c) * 4 + s;
            dw_lvl[pi * k2 + tap] = scale[pi] * G[t];
        }
    }
    for (int ls = tid; ls < 4 * L; ls += blockDim.x) {
        const int l = ls / 4, s = ls - 4 * l;
        const size_t pi = ((size_t)l * C + c) * 4 + s;
        float a = 0.f;
        for (int tap = 0; tap < k2; ++tap) a += w_lvl[pi * k2 + tap] * G[kb2 + ls * k2 + tap];
        dscale[pi] = a;
    }
}

// ------------------------------------------------------------ registry

typedef hipError_t (*bwdw_fn)(const void*, const void*, float*, int, int, int, hipStream_t);

template <class P, typename T>
static hipError_t launch_bwdw(const void* x, const void* dy, float* part, int B, int C, int bpc,
                              hipStream_t stream) {
    const int nchunk = cdiv(B, bpc);
    hipLaunchKernelGGL((bwdw_kernel<P, T>), dim3((unsigned)(nchunk * C)), dim3(P::NT), 0, stream,
                       (const T*)x, (const T*)dy, part, B, C, bpc);
    return hipGetLastError();
}

struct BwEntry {
    int H, W, L, KB, K;
    bwdw_fn fn[2];
};

typedef BwPlan<32, 32, 2, 5, 5, 2, 2> BP_32_L2_k55;
typedef BwPlan<56, 56, 3, 5, 5, 4, 4> BP_56_L3_k55;
typedef BwPlan<28, 28, 2, 5, 5, 2, 2> BP_28_L2_k55;
typedef BwPlan<14, 14, 1, 5, 5, 1, 1> BP_14_L1_k55;
typedef BwPlan<32, 32, 3, 7, 5, 2, 2> BP_32_L3_k75;
typedef BwPlan<24, 40, 3, 3, 3, 2, 2> BP_24x40_L3_k33;
typedef BwPlan<16, 16, 4, 3, 7, 1, 1> BP_16_L4_k37;
typedef BwPlan<64, 64, 4, 7, 5, 4, 4> BP_64_L4_k75;

#define WTC_BW_ENTRY(PLAN) \
    { PLAN::H, PLAN::W, PLAN::L, PLAN::KB, PLAN::K, {launch_bwdw<PLAN, float>, launch_bwdw<PLAN, bf16_t>} }

static const BwEntry kBwEntries[] = {
    WTC_BW_ENTRY(BP_32_L2_k55), WTC_BW_ENTRY(BP_56_L3_k55),    WTC_BW_ENTRY(BP_28_L2_k55),
    WTC_BW_ENTRY(BP_14_L1_k55), WTC_BW_ENTRY(BP_32_L3_k75),    WTC_BW_ENTRY(BP_24x40_L3_k33),
    WTC_BW_ENTRY(BP_16_L4_k37), WTC_BW_ENTRY(BP_64_L4_k75),
};

static const BwEntry* find_bw(int H, int W, int L, int KB, int K) {
    for (const BwEntry& e : kBwEntries)
        if (e.H == H && e.W == W && e.L == L && e.KB == KB && e.K == K) return &e;
    return nullptr;
}

// batches per chunk: about three rounds of workgroups over the chip, so the
// per-chunk reduction is amortised over several planes
static int chunk_batches(int B, int C) {
    const int want_chunks = cdiv(1536, C);
    const int nchunk = want_chunks < B ? want_chunks : B;
    return cdiv(B, nchunk < 1 ? 1 : nchunk);
}

size_t bwdw_workspace_bytes(int B, int C, int H, int W, int L, int KB, int K) {
    if (!find_bw(H, W, L, KB, K)) return (size_t)-1;
    const int nchunk = cdiv(B, chunk_batches(B, C));
    return (size_t)nchunk * C * (KB * KB + 4 * L * K * K) * sizeof(float);
}

hipError_t bwdw_launch(int B, int C, int H, int W, int L, int KB, int K, bool bf16, const void* x,
                       const void* dy, const float* w_lvl, const float* scale, float* dw_base,
                       float* dw_lvl, float* dscale, void* ws, hipStream_t stream) {
    const BwEntry* e = find_bw(H, W, L, KB, K);
    if (!e) return hipErrorInvalidValue;
    const int bpc = chunk_batches(B, C), nchunk = cdiv(B, bpc);
    float* part = (float*)ws;
    hipError_t err = e->fn[bf16 ? 1 : 0](x, dy, part, B, C, bpc, stream);
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(bwdw_finalize, dim3((unsigned)C), dim3(256), 0, stream, (const float*)part,
                       nchunk, C, L, KB, K, w_lvl, scale, dw_base, dw_lvl, dscale);
    return hipGetLastError();
}

}  // namespace wtc
