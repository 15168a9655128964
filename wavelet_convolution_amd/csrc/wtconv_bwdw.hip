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
#include "wtconv_bwdw_body.h"
#include "wtconv_dw.h"
#include "wtconv_family.h"

namespace wtc {

// Stage 2 as its own kernel: one workgroup per channel.
__global__ __launch_bounds__(1024) void bwdw_finalize(FinalizeArgs f) {
    // w_lvl * G per level tap, sized for every shape the ABI accepts (the
    // host rejects L > 5 and kernels above 15 before any launch)
    constexpr int kMaxLevels = 5, kMaxK = 15;
    __shared__ float WG[4 * kMaxLevels * kMaxK * kMaxK];
    if (f.L > kMaxLevels || f.K > kMaxK) return;
    finalize_channel(f, blockIdx.x, threadIdx.x, blockDim.x, WG);
}

// Where the calling thread has asked for it (bwdw_launch_deferred), the
// second stage is not launched but handed back, for a later kernel of the
// same stream to run as extra workgroups.
static thread_local FinalizeArgs* g_defer = nullptr;

hipError_t launch_bwdw_finalize(const float* partA, int nA, int LA, const float* partB, int nB, int C, int L, int KB,
                                int K, const float* w_lvl, const float* scale, float* dw_base, float* dw_lvl,
                                float* dscale, hipStream_t stream) {
    const FinalizeArgs f{partA, nA, LA, partB, nB, C, L, KB, K, w_lvl, scale, dw_base, dw_lvl, dscale};
    if (g_defer) {
        *g_defer = f;
        return hipSuccess;
    }
    hipLaunchKernelGGL(bwdw_finalize, dim3((unsigned)C), dim3(finalize_threads(KB, K, L)), 0, stream, f);
    return hipGetLastError();
}

// ---------------------------------------------------- split fine pass

// Fine pass of the backward weight for planes too large for one workgroup:
// full-width tiles of TH rows of dy, the rows of x they reach plus a halo of
// G rows (as in the forward fine pass), base taps and the taps of levels
// 1..L0, and the tile's unnormalised level-L0 LL sums of x and dy, which the
// coarse pass (bwdw_kernel with BASE = false) correlates for levels L0+1..L.
// One workgroup per (channel, chunk of (b, tile) units); the units of a chunk
// follow each other down the plane, so the halo rows of consecutive tiles
// are read from L2.
//
// NT threads in two groups of NT/2: group A sums the base taps, group B the
// taps of the fine levels, each band of each level on NT/8 lanes (one or two
// wavefronts). A lane keeps one accumulator array for the whole chunk: the
// base taps (group A) or the taps of every fine level, level l at offset
// (l-1) K² (group B).
template <int H_, int W_, int L0_, int LT_, int KB_, int K_, int TH_, int NT_ = 512, bool MF_ = false>
struct TileBwPlan {
    static constexpr int H = H_, W = W_, L0 = L0_, LT = LT_, KB = KB_, K = K_, TH = TH_;
    static constexpr int L = L0;   // levels handled here (role helpers below)
    static constexpr int NT = NT_, NW = NT / 64, GW = NW / 2;   // waves per group
    static constexpr int GL = GW * 64, BL = GL / 4;              // lanes per group, per band
    static_assert(NT == 512 || NT == 1024, "two groups of four or eight wavefronts");
    static constexpr int RB = pick_rows(TH, W, GL, KB);
    static constexpr int PB = KB / 2, PK = K / 2, BLK = 1 << L0;
    static_assert(L0 >= 1 && L0 <= 2 && L0 <= LT, "fine levels: one or two (group B holds them all)");
    static_assert(H % (1 << LT) == 0 && W % (1 << LT) == 0, "plane must divide into 2^L blocks");
    static_assert(TH % BLK == 0 && H % TH == 0, "tile shapes");
    static constexpr int G0 = PB > (PK << L0) ? PB : (PK << L0);
    static constexpr int G = cdiv(G0, BLK) * BLK;
    static constexpr int RH0 = TH + 2 * G;
    // row layout as in BwPlan: aligned interiors for vector stores and reads
    static constexpr int VL = lds_vec(W);
    static constexpr int XO = round_up(PB, 4);
    static constexpr int SX = round_up(XO + W + PB, 4);
    static constexpr int XSIZE = RH0 * SX;
    static constexpr int SD = round_up(W, 4);
    static constexpr int DSIZE = TH * SD;
    static constexpr int rh(int l) { return RH0 >> l; }
    // band row strides: odd (scalar analysis stores of consecutive rows in
    // different banks), or even in the matrix-core form, whose analysis
    // stores cell pairs as 64-bit words
    static constexpr int su(int l) { return MF_ ? round_up((W >> l) + 2 * PK, 2) : odd_stride((W >> l) + 2 * PK); }
    static constexpr int bandsz(int l) { return rh(l) * su(l); }
    static constexpr int sv(int l) { return MF_ ? round_up(W >> l, 2) : odd_stride(W >> l); }
    static constexpr int vsz(int l) { return (TH >> l) * sv(l); }
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
    static constexpr int UTOT = uoff(L0 + 1), VTOT = voff(L0 + 1);
    // accumulators per lane: base taps, or the taps of all fine levels
    static constexpr int ACC = KB * KB > L0 * K * K ? KB * KB : L0 * K * K;
    static constexpr int boff(int l) { return (l - 1) * K * K; }
    static constexpr int RED = NW * ACC;
    static constexpr int DATA = XSIZE + DSIZE + UTOT + VTOT;
    static constexpr int LDS_FLOATS = DATA > RED ? DATA : RED;
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "tile does not fit in LDS");
    static constexpr int LPB = strip_lanes(W);
    static constexpr int NI = (TH / RB) * LPB;
    static constexpr int NTILE = H / TH;
    static constexpr int TAPS = KB * KB + 4 * L0 * K * K;
    static constexpr int band_rows(int l) { return pick_rows(TH >> l, W >> l, BL, K); }
    static constexpr int WG_PER_CU = (160 * 1024) / (LDS_FLOATS * 4);
    static constexpr int WAVES_PER_EU_LDS = WG_PER_CU * NW / 4;
    static constexpr int REGS = ACC + 64;
    static constexpr int WAVES_PER_EU_REG = 512 / (REGS <= 128 ? 128 : (REGS <= 168 ? 168 : 256));
    static constexpr int WAVES_PER_EU_MIN = WAVES_PER_EU_LDS < WAVES_PER_EU_REG ? WAVES_PER_EU_LDS : WAVES_PER_EU_REG;
    static constexpr int WAVES_PER_EU = WAVES_PER_EU_MIN < 1 ? 1 : WAVES_PER_EU_MIN;

    // Matrix-core form for bf16 activations (tile_bwdw_mf_kernel): the base
    // taps as 16x16x32 bf16 matrix products, every wavefront one pair of dy
    // rows; the level taps on all wavefronts (each band on NT/4 lanes). LDS:
    // the x rows the base taps read as bf16 (XRM rows, SXBM apart), dy as
    // words of overlapping bf16 pairs (word DOFF + c = dy[c], dy[c+1]; SDP
    // words a row; zero outside the plane), then the level bands U and V.
    static constexpr bool MF = MF_;
    // NTM threads; WPR wavefronts per dy row pair, each taking W / 32 / WPR
    // column chunks. The level-2 bands take the place of the x rows and dy
    // pair words once the matrix products are done (two workgroups per CU).
    static constexpr int NTM = 512, NWM = NTM / 64, WPR = NWM / (TH / 2);
    static constexpr int XRM = TH + 2 * PB, SXBM = W + 8, DOFF = 8, SDP = W + 48, BLM = NTM / 4;
    static constexpr int ACCM = L0 * K * K;
    static constexpr int XSM = (XRM * SXBM / 2 + 3) / 4 * 4, DPM = TH * SDP;
    static constexpr int U2M = 4 * bandsz(2), V2M = 4 * vsz(2), U1M = 4 * bandsz(1), V1M = 4 * vsz(1);
    static constexpr int AM = XSM + DPM > U2M + V2M ? XSM + DPM : U2M + V2M;   // x rows + dy words, then level 2
    static constexpr int DATAM = AM + U1M + V1M, REDM = NWM * (256 + ACCM);
    static constexpr int MF_FLOATS = DATAM > REDM ? DATAM : REDM;
    // (level 2 in four-row strips on half the lanes rather than two-row
    // strips on all: fewer LDS reads per multiply-add, and the waves wait on
    // LDS instruction issue more than on multiply-adds)
    static constexpr int band_rows_mf(int l) {
        return l == 2 && (TH >> 2) % 4 == 0 ? 4 : pick_rows(TH >> l, W >> l, BLM, K);
    }
    static_assert(!MF || (L0 == 2 && NWM % (TH / 2) == 0 && (W / 32) % WPR == 0 && KB <= 7 && PK % 2 == 0 && DOFF % 4 == 0 && SDP % 4 == 0 &&
                          7 - PB <= DOFF && DOFF + PB + W < SDP && SXBM % 8 == 0 &&
                          MF_FLOATS * 4 <= 160 * 1024),
                  "matrix-core weight gradient: one dy row pair per wavefront, 32-column chunks, taps up to 7x7");
    // occupancy the LDS allows, at most four waves per SIMD: the level-tap
    // accumulators and strips need up to 128 registers
    static constexpr int WPE_LDS = ((160 * 1024) / (MF_FLOATS * 4)) * NWM / 4;
    static constexpr int WAVES_PER_EU_MF = WPE_LDS < 1 ? 1 : (WPE_LDS > 4 ? 4 : WPE_LDS);

    template <class F>
    __device__ static __forceinline__ void for_levels(F&& f) {
        lv_impl(f, std::make_integer_sequence<int, L0>{});
    }
    template <class F, int... I>
    __device__ static __forceinline__ void lv_impl(F& f, std::integer_sequence<int, I...>) {
        (f(std::integral_constant<int, I + 1>{}), ...);
    }
};

template <class P, typename T>
__global__ __launch_bounds__(P::NT) __attribute__((amdgpu_waves_per_eu(P::WAVES_PER_EU)))
void tile_bwdw_kernel(const T* __restrict__ x, const T* __restrict__ dy, float* __restrict__ part,
                      float* __restrict__ px, float* __restrict__ pdy, int B, int C, int upc) {
    constexpr int H = P::H, W = P::W, L0 = P::L0, KB = P::KB, K = P::K, NT = P::NT, TH = P::TH;
    constexpr int PB = P::PB, PK = P::PK, SX = P::SX, G = P::G, RH0 = P::RH0, W1 = W / 2;
    constexpr int RB = P::RB, NI = P::NI, LPB = P::LPB, XO = P::XO, SD = P::SD;
    constexpr int ACC = P::ACC, GW = P::GW, GL = P::GL, BL = P::BL;
    constexpr int VL = P::VL;
    constexpr int NVX = RH0 * W / VL, NVD = TH * W / VL;
    constexpr int NLX = cdiv(NVX, NT), NLD = cdiv(NVD, NT);

    __shared__ __attribute__((aligned(16))) float lds[P::LDS_FLOATS];
    float* X = lds;
    const float* X0 = X + XO - PB;   // origin of the bordered x rows
    float* DY = X + P::XSIZE;
    float* U = DY + P::DSIZE;
    float* Vb = U + P::UTOT;

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    // group A (waves 0..GW-1): base taps; group B: band (wave - GW) & 3 of
    // every fine level, lanes blane of the band's BL
    const int grp = wave / GW, gtid = tid - grp * GL;
    const int band = (wave - GW) & 3, blane = (((wave - GW) >> 2) << 6) + lane;
    const int c = blockIdx.x % C, chunk = blockIdx.x / C;
    const int nunits = B * P::NTILE;
    const int u0 = chunk * upc, u1 = min(nunits, u0 + upc);

    // border columns stay zero: loads and analyses write interior columns only
    for (int i = tid; i < RH0 * (SX - W); i += NT) {
        const int r = i / (SX - W), q = i - r * (SX - W);
        X[r * SX + (q < XO ? q : q + W)] = 0.f;
    }
    P::for_levels([&](auto lc) {
        constexpr int l = decltype(lc)::value;
        constexpr int rl = P::rh(l), wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l);
        float* Ul = U + P::uoff(l);
        for (int i = tid; i < 4 * rl * (Sl - wl); i += NT) {
            const int b = i / (rl * (Sl - wl)), j = i - b * (rl * (Sl - wl));
            const int r = j / (Sl - wl), q = j - r * (Sl - wl);
            Ul[b * BSl + r * Sl + (q < PK ? q : q + wl)] = 0.f;
        }
    });

    float acc[ACC];
#pragma unroll
    for (int t = 0; t < ACC; ++t) acc[t] = 0.f;

    RawVec<T, VL> vx[NLX], vd[NLD];
    auto issue_loads = [&](int u) {
        const int b = u / P::NTILE, r0 = (u - b * P::NTILE) * TH;
        const size_t plane = (size_t)b * C + c;
        const T* __restrict__ xs = x + plane * H * W;
        const T* __restrict__ ds = dy + plane * H * W;
#pragma unroll
        for (int k = 0; k < NLX; ++k) {
            const int q = tid + k * NT;
            const int e = q * VL, rr = e / W, pr = r0 - G + rr;
            if ((NVX % NT == 0 || q < NVX) && pr >= 0 && pr < H)
                load_raw<T, VL>(xs + (size_t)pr * W + (e - rr * W), vx[k]);
            else
#pragma unroll
                for (int i = 0; i < RawVec<T, VL>::N; ++i) vx[k].w[i] = 0u;   // rows outside the plane: zeros
        }
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            const int q = tid + k * NT;
            if (NVD % NT == 0 || q < NVD) load_raw<T, VL>(ds + (size_t)r0 * W + q * VL, vd[k]);
        }
    };
    if (u0 < u1) issue_loads(u0);

    for (int u = u0; u < u1; ++u) {
        const int b = u / P::NTILE, r0 = (u - b * P::NTILE) * TH;
        const size_t plane = (size_t)b * C + c;
        // ------------------------------------------------ P0: stream in
#pragma unroll
        for (int k = 0; k < NLX; ++k) {
            const int q = tid + k * NT;
            if (NVX % NT == 0 || q < NVX) {
                const int e = q * VL, rr = e / W, col = e - rr * W;
                store_lds<T, VL>(X + rr * SX + XO + col, vx[k]);
            }
        }
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            const int q = tid + k * NT;
            if (NVD % NT == 0 || q < NVD) {
                const int e = q * VL, rr = e / W, col = e - rr * W;
                store_lds<T, VL>(DY + rr * SD + col, vd[k]);
            }
        }
        lds_barrier();
        if (u + 1 < u1) issue_loads(u + 1);
        // ----------------------------------------- P1: level 1 analysis
        {
            constexpr int S1 = P::su(1), BS1 = P::bandsz(1), VS1 = P::vsz(1);
            for (int q = tid; q < P::rh(1) * W1; q += NT) {
                const int i = q / W1, j = q - i * W1;
                const float2 a = *reinterpret_cast<const float2*>(X + (2 * i) * SX + XO + 2 * j);
                const float2 c2 = *reinterpret_cast<const float2*>(X + (2 * i + 1) * SX + XO + 2 * j);
                float uu[4];
                haar4(a.x, a.y, c2.x, c2.y, uu[0], uu[1], uu[2], uu[3]);
#pragma unroll
                for (int s = 0; s < 4; ++s) U[s * BS1 + i * S1 + PK + j] = uu[s];
            }
            constexpr int SV1 = P::sv(1);
            for (int q = tid; q < (TH / 2) * W1; q += NT) {
                const int i = q / W1, j = q - i * W1;
                const float2 a = *reinterpret_cast<const float2*>(DY + 2 * i * SD + 2 * j);
                const float2 c2 = *reinterpret_cast<const float2*>(DY + (2 * i + 1) * SD + 2 * j);
                float vv[4];
                haar4(a.x, a.y, c2.x, c2.y, vv[0], vv[1], vv[2], vv[3]);
#pragma unroll
                for (int s = 0; s < 4; ++s) Vb[s * VS1 + i * SV1 + j] = vv[s];
            }
        }
        lds_barrier();
        // ----------------------------------------- P2: levels 2..L0 analysis
        P::for_levels([&](auto lc) {
            constexpr int l = decltype(lc)::value;
            if constexpr (l >= 2) {
                constexpr int rl = P::rh(l), wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), VSl = P::vsz(l);
                constexpr int Sp = P::su(l - 1), SVp = P::sv(l - 1), SVl = P::sv(l);
                const float* LLu = U + P::uoff(l - 1) + PK;
                const float* LLv = Vb + P::voff(l - 1);
                float* Ul = U + P::uoff(l);
                float* Vl = Vb + P::voff(l);
                for (int q = tid; q < rl * wl; q += NT) {
                    const int i = q / wl, j = q - i * wl;
                    const float* x2 = LLu + 2 * i * Sp + 2 * j;
                    float uu[4];
                    haar4(x2[0], x2[1], x2[Sp], x2[Sp + 1], uu[0], uu[1], uu[2], uu[3]);
#pragma unroll
                    for (int s = 0; s < 4; ++s) Ul[s * BSl + i * Sl + PK + j] = uu[s];
                }
                for (int q = tid; q < (TH >> l) * wl; q += NT) {
                    const int i = q / wl, j = q - i * wl;
                    const float* d2 = LLv + 2 * i * SVp + 2 * j;
                    float vv[4];
                    haar4(d2[0], d2[1], d2[SVp], d2[SVp + 1], vv[0], vv[1], vv[2], vv[3]);
#pragma unroll
                    for (int s = 0; s < 4; ++s) Vl[s * VSl + i * SVl + j] = vv[s];
                }
                lds_barrier();
            }
        });
        // the coarse pass's inputs: the tile's level-L0 LL sums of x and dy
        if (P::LT > L0) {
            constexpr int hl = TH >> L0, wl = W >> L0, Sl = P::su(L0), GLv = G >> L0;
            const float* LLu = U + P::uoff(L0) + PK;
            const float* LLv = Vb + P::voff(L0);
            float* pxo = px + plane * (H >> L0) * wl + (size_t)(r0 >> L0) * wl;
            float* pdo = pdy + plane * (H >> L0) * wl + (size_t)(r0 >> L0) * wl;
            constexpr int SVL = P::sv(L0);
            for (int q = tid; q < hl * wl; q += NT) {
                const int i = q / wl, j = q - i * wl;
                pxo[q] = LLu[(GLv + i) * Sl + j];
                pdo[q] = LLv[i * SVL + j];
            }
        }
        // ------------------- P3: all taps at once: base taps (group A), one band per wavefront (group B)
        if (grp == 0) {
            for (int item = gtid; item < NI; item += GL) {
                const int rb = item / LPB, w = item - rb * LPB, h0 = rb * RB;
                if (LPB == W || w < W) taps_col<KB, RB, SX, SD>(X0 + (G + h0 - PB) * SX + w, DY + h0 * SD + w, acc);
            }
        } else {
            P::for_levels([&](auto lc) {
                constexpr int l = decltype(lc)::value;
                constexpr int hl = TH >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), VSl = P::vsz(l);
                constexpr int Gl = G >> l, SVl = P::sv(l), OFF = P::boff(l);
                constexpr int R = P::band_rows(l), LPl = strip_lanes(wl), NIl = (hl / R) * LPl;
                const float* Us = U + P::uoff(l) + band * BSl;
                const float* Vs = Vb + P::voff(l) + band * VSl;
                for (int item = blane; item < NIl; item += BL) {
                    const int rs = item / LPl, j = item - rs * LPl;
                    if (!(LPl == wl || j < wl)) continue;
                    taps_col<K, R, Sl, SVl, ACC, float, OFF>(Us + (Gl + R * rs - PK) * Sl + j,
                                                              Vs + R * rs * SVl + j, acc);
                }
            });
        }
        // the next unit's P0 overwrites x, dy, U and V: wait for every reader
        // (the loop's barriers order LDS only: the LL sums this unit wrote to
        // global memory are read by a later kernel, and the next unit's
        // loads stay in flight)
        lds_barrier();
    }

#pragma unroll
    for (int t = 0; t < ACC; ++t) acc[t] = wave_sum(acc[t]);
    __syncthreads();
    float* red = lds;   // [NW][ACC]
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < ACC; ++t) red[wave * ACC + t] = acc[t];
    }
    __syncthreads();
    float* dst = part + ((size_t)chunk * C + c) * P::TAPS;
    for (int t = tid; t < P::TAPS; t += NT) {
        float v = 0.f;
        if (t < KB * KB) {
            for (int w = 0; w < GW; ++w) v += red[w * ACC + t];   // group A, waves in order
        } else {
            const int r = t - KB * KB, ls = r / (K * K), tap = r - ls * (K * K);
            const int l = ls / 4 + 1, s = ls - (l - 1) * 4;
            for (int j = 0; j < GW / 4; ++j) v += red[(GW + 4 * j + s) * ACC + (l - 1) * K * K + tap];
        }
        dst[t] = v;
    }
}

// Matrix-core weight gradient of the fine tiles (bf16 activations): the same
// units, outputs and second stage as tile_bwdw_kernel, the base taps as
// bf16 matrix products (the products of bf16 values are exact in fp32).
// For the dy row pair (h, h+1) and a chunk of 32 x columns w0..w0+31:
//   D[m][n] += sum_k X[m][k] Y[k][n],  X[m][k] = x[h-PB+m][w0+k],
//   Y[k][n] = dy[h + n/8][w0 + k - n%8 + PB],
// so D[i][j] (n < 8) collects tap (i, j) from dy row h and D[i+1][8+j] tap
// (i, j) from dy row h+1: G[i][j] = sum over wavefronts of D[i][j] + D[i+1][8+j]
// (rows m >= 8 and columns n%8 >= KB are not taps; their lanes read valid
// LDS words whose products are discarded). Lane l holds X row l%16 (row 7 for
// l%16 > 7), columns 8(l/16)..+7, and Y column l%16, rows 8(l/16)..+7 (dy
// words at a lane-dependent column: the pair words make any start 4-byte
// aligned); D rows 4(l/16)..+3 of column l%16.
// The level taps run on every wavefront: band wave%4 of each fine level, on
// the lanes of waves band and band + 4.
template <class P>
__global__ __launch_bounds__(P::NTM) __attribute__((amdgpu_waves_per_eu(P::WAVES_PER_EU_MF)))
void tile_bwdw_mf_kernel(const bf16_t* __restrict__ x, const bf16_t* __restrict__ dy, float* __restrict__ part,
                         float* __restrict__ px, float* __restrict__ pdy, int B, int C, int upc) {
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    typedef float f32x4 __attribute__((ext_vector_type(4)));
    constexpr int H = P::H, W = P::W, L0 = P::L0, KB = P::KB, K = P::K, NT = P::NTM, TH = P::TH, NW = P::NWM;
    constexpr int PB = P::PB, PK = P::PK, G = P::G, RH0 = P::RH0, WPR = P::WPR;
    constexpr int XRM = P::XRM, SXBM = P::SXBM, DOFF = P::DOFF, SDP = P::SDP, BLM = P::BLM, ACCM = P::ACCM;
    constexpr int QW = W / 4;                       // 4-column items per row
    constexpr int NQX = (RH0 / 2) * QW, NQD = (TH / 2) * QW;
    constexpr int MQX = cdiv(NQX, NT), MQD = cdiv(NQD, NT);
    static_assert(W % 4 == 0 && (NQD % NT == 0 || NQD < NT), "whole dy items per thread");

    __shared__ __attribute__((aligned(16))) float lds[P::MF_FLOATS];
    uint16_t* const XS = reinterpret_cast<uint16_t*>(lds);
    uint32_t* const DP = reinterpret_cast<uint32_t*>(lds + P::XSM);
    float* const U2 = lds;              // level 2 over the x rows and dy words
    float* const V2 = lds + P::U2M;
    float* const U1 = lds + P::AM;
    float* const V1 = U1 + P::U1M;
    // band l of x (bordered) and of dy
    auto ub = [&](auto lc) -> float* {
        if constexpr (decltype(lc)::value == 1) return U1;
        else return U2;
    };
    auto vb = [&](auto lc) -> float* {
        if constexpr (decltype(lc)::value == 1) return V1;
        else return V2;
    };

    // (the wavefront index as a scalar: row indices derived from it stay uniform)
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
    const int band = wave & 3, blane = ((wave >> 2) << 6) + lane;
    const int c = blockIdx.x % C, chunk = blockIdx.x / C;
    const int nunits = B * P::NTILE;
    const int u0 = chunk * upc, u1 = min(nunits, u0 + upc);

    // once: the level-1 band border columns (nothing else writes them)
    {
        constexpr int rl = P::rh(1), wl = W >> 1, Sl = P::su(1), BSl = P::bandsz(1);
        for (int i = tid; i < 4 * rl * (Sl - wl); i += NT) {
            const int b = i / (rl * (Sl - wl)), j = i - b * (rl * (Sl - wl));
            const int r = j / (Sl - wl), q = j - r * (Sl - wl);
            U1[b * BSl + r * Sl + (q < PK ? q : q + wl)] = 0.f;
        }
    }

    float acc[ACCM];
#pragma unroll
    for (int t = 0; t < ACCM; ++t) acc[t] = 0.f;
    f32x4 dacc = {0.f, 0.f, 0.f, 0.f};

    // x: region rows 2ii, 2ii+1 (plane rows r0-G+2ii..), four columns from
    // 4uu; dy: tile rows 2ii, 2ii+1. Rows outside the plane load as zeros.
    // Held as 64-bit words until they are used: a 64-bit value keeps its
    // aligned register pair, where two 32-bit halves may be moved apart
    // right after the load, which waits for it and undoes the prefetch.
    uint64_t lx0[MQX], lx1[MQX], ld0[MQD], ld1[MQD];
    auto raw4 = [](uint64_t v) {
        RawVec<bf16_t, 4> r;
        r.w[0] = (uint32_t)v;
        r.w[1] = (uint32_t)(v >> 32);
        return r;
    };
    auto issue_loads = [&](int u) {
        const int b = u / P::NTILE, r0 = (u - b * P::NTILE) * TH;
        const size_t plane = (size_t)b * C + c;
        const bf16_t* __restrict__ xs = x + plane * H * W;
        const bf16_t* __restrict__ ds = dy + plane * H * W + (size_t)r0 * W;
#pragma unroll
        for (int k = 0; k < MQX; ++k) {
            const int q = tid + k * NT;
            const int ii = QW == 64 ? wave + k * (NT / 64) : udiv(q, QW), uu = QW == 64 ? lane : q - ii * QW, pr = r0 - G + 2 * ii;
            const bool inside = (NQX % NT == 0 || q < NQX) && pr >= 0 && pr < H;
            const bf16_t* s0 = xs + (inside ? (uint32_t)(pr * W + 4 * uu) : 0u);
            lx0[k] = *reinterpret_cast<const uint64_t*>(s0);
            lx1[k] = *reinterpret_cast<const uint64_t*>(s0 + (inside ? W : 0));
            // (the rows outside the plane are zeroed where they are used: a
            // select here would wait for the loads and undo the prefetch)
        }
#pragma unroll
        for (int k = 0; k < MQD; ++k) {
            const int q = tid + k * NT;
            if (!(NQD % NT == 0 || q < NQD)) continue;
            const int ii = QW == 64 ? wave + k * (NT / 64) : udiv(q, QW), uu = QW == 64 ? lane : q - ii * QW;
            ld0[k] = *reinterpret_cast<const uint64_t*>(ds + (uint32_t)(2 * ii * W + 4 * uu));
            ld1[k] = *reinterpret_cast<const uint64_t*>(ds + (uint32_t)((2 * ii + 1) * W + 4 * uu));
        }
    };
    if (u0 < u1) issue_loads(u0);

    for (int u = u0; u < u1; ++u) {
        const int b = u / P::NTILE, r0 = (u - b * P::NTILE) * TH;
        const size_t plane = (size_t)b * C + c;
        // ------------------------------------------------ P0: stream in
        {
            constexpr int S1 = P::su(1), BS1 = P::bandsz(1), VS1 = P::vsz(1), SV1 = P::sv(1);
            // dy pair words outside the plane (level 2 used this space)
            constexpr int ZW = SDP - W - 1;   // words 0..DOFF-2 and DOFF+W..SDP-1 of each row
            for (int i = tid; i < TH * ZW; i += NT) {
                const int r = udiv(i, ZW), q = i - r * ZW;
                DP[r * SDP + (q < DOFF - 1 ? q : q + W + 1)] = 0u;
            }
#pragma unroll
            for (int k = 0; k < MQX; ++k) {
                const int q = tid + k * NT;
                if (!(NQX % NT == 0 || q < NQX)) continue;
                const int ii = QW == 64 ? wave + k * (NT / 64) : udiv(q, QW), uu = QW == 64 ? lane : q - ii * QW, pr = r0 - G + 2 * ii;
                RawVec<bf16_t, 4> vx0 = raw4(lx0[k]), vx1 = raw4(lx1[k]);
                if (pr < 0 || pr >= H) {   // rows outside the plane: zeros
#pragma unroll
                    for (int e = 0; e < RawVec<bf16_t, 4>::N; ++e) {
                        vx0.w[e] = 0u;
                        vx1.w[e] = 0u;
                    }
                }
                // the x rows the base taps read, as loaded
                const int xr = 2 * ii - (G - PB);
                if (xr >= 0 && xr < XRM)
                    *reinterpret_cast<uint2*>(XS + xr * SXBM + 4 * uu) = make_uint2(vx0.w[0], vx0.w[1]);
                if (xr + 1 >= 0 && xr + 1 < XRM)
                    *reinterpret_cast<uint2*>(XS + (xr + 1) * SXBM + 4 * uu) = make_uint2(vx1.w[0], vx1.w[1]);
                float f0[4], f1[4];
                widen_raw<bf16_t, 4>(vx0, f0);
                widen_raw<bf16_t, 4>(vx1, f1);
                float bb[2][4];
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    haar4(f0[2 * m], f0[2 * m + 1], f1[2 * m], f1[2 * m + 1], bb[m][0], bb[m][1], bb[m][2], bb[m][3]);
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
                    *reinterpret_cast<float2*>(U1 + sb * BS1 + ii * S1 + PK + 2 * uu) = make_float2(bb[0][sb], bb[1][sb]);
            }
#pragma unroll
            for (int k = 0; k < MQD; ++k) {
                const int q = tid + k * NT;
                if (!(NQD % NT == 0 || q < NQD)) continue;
                const int ii = QW == 64 ? wave + k * (NT / 64) : udiv(q, QW), uu = QW == 64 ? lane : q - ii * QW;
                const RawVec<bf16_t, 4> vd0 = raw4(ld0[k]), vd1 = raw4(ld1[k]);
                // pair words c..c+3 as one 16-byte store; the last needs the
                // next item's first value (the next lane: a row's items are
                // one wavefront), zero past the plane; the word before
                // column 0 holds (0, dy[0])
                static_assert(64 % QW == 0, "a dy row's items on consecutive lanes of one wavefront");
#pragma unroll
                for (int rs = 0; rs < 2; ++rs) {
                    const uint32_t w0 = rs ? vd1.w[0] : vd0.w[0], w1 = rs ? vd1.w[1] : vd0.w[1];
                    const uint32_t nx = (uint32_t)__shfl_down((int)w0, 1, 64);
                    const uint32_t w3 = (w1 >> 16) | (uu + 1 < QW ? (nx << 16) : 0u);
                    const int wb = (2 * ii + rs) * SDP + DOFF + 4 * uu;
                    *reinterpret_cast<uint4*>(DP + wb) = make_uint4(w0, __builtin_amdgcn_alignbit(w1, w0, 16), w1, w3);
                    if (uu == 0) DP[wb - 1] = w0 << 16;
                }
                float f0[4], f1[4];
                widen_raw<bf16_t, 4>(vd0, f0);
                widen_raw<bf16_t, 4>(vd1, f1);
                float bb[2][4];
#pragma unroll
                for (int m = 0; m < 2; ++m)
                    haar4(f0[2 * m], f0[2 * m + 1], f1[2 * m], f1[2 * m + 1], bb[m][0], bb[m][1], bb[m][2], bb[m][3]);
#pragma unroll
                for (int sb = 0; sb < 4; ++sb)
                    *reinterpret_cast<float2*>(V1 + sb * VS1 + ii * SV1 + 2 * uu) = make_float2(bb[0][sb], bb[1][sb]);
            }
        }
        lds_barrier();
        if (u + 1 < u1) issue_loads(u + 1);

        // level taps of level l: band `band` on the lanes of its wavefronts
        auto level_taps = [&](auto lc) {
            constexpr int l = decltype(lc)::value;
            constexpr int hl = TH >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), VSl = P::vsz(l);
            constexpr int Gl = G >> l, SVl = P::sv(l), OFF = P::boff(l);
            constexpr int R = P::band_rows_mf(l), LPl = strip_lanes(wl), NIl = (hl / R) * LPl;
            const float* Us = ub(lc) + band * BSl;
            const float* Vs = vb(lc) + band * VSl;
            for (int item = blane; item < NIl; item += BLM) {
                const int rs = item / LPl, j = item - rs * LPl;
                if (!(LPl == wl || j < wl)) continue;
                taps_col<K, R, Sl, SVl, ACCM, float, OFF>(Us + (Gl + R * rs - PK) * Sl + j, Vs + R * rs * SVl + j,
                                                          acc);
            }
        };
        // ------------------- P1: base taps on the matrix cores, level-1 taps
        {
            const int m = lane & 15, qq = lane >> 4, rp = wave / WPR, c0 = (wave - rp * WPR) * (W / 32 / WPR);
            const uint16_t* xa = XS + (2 * rp + (m < 8 ? m : 7)) * SXBM + 8 * qq + 32 * c0;
            const uint32_t* ya = DP + (2 * rp + (m >> 3)) * SDP + DOFF + 8 * qq - (m & 7) + PB + 32 * c0;
#pragma unroll
            for (int ch = 0; ch < W / 32 / WPR; ++ch) {
                const bf16x8 a = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xa + 32 * ch));
                const uint32_t* yp = ya + 32 * ch;
                const bf16x8 bm = __builtin_bit_cast(bf16x8, make_uint4(yp[0], yp[2], yp[4], yp[6]));
                dacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, bm, dacc, 0, 0, 0);
            }
        }
        level_taps(std::integral_constant<int, 1>{});
        lds_barrier();   // the x rows and dy words are dead: level 2 goes over them
        // ----------------------------------------- P2: level 2 analysis
        {
            constexpr int rl = P::rh(2), wl = W >> 2, Sl = P::su(2), BSl = P::bandsz(2), VSl = P::vsz(2);
            constexpr int Sp = P::su(1), SVp = P::sv(1), SVl = P::sv(2), XB2 = Sl - wl;
            const float* LLu = U1 + PK;
            // border columns, then the interior cells
            for (int i = tid; i < 4 * rl * XB2; i += NT) {
                const int rb = udiv(i, XB2), q = i - rb * XB2;
                U2[rb * Sl + (q < PK ? q : q + wl)] = 0.f;
            }
            for (int q = tid; q < rl * wl; q += NT) {
                const int i = wl == 64 ? wave + (q - tid) / 64 : q / wl, j = wl == 64 ? lane : q - i * wl;
                const float2 t0 = *reinterpret_cast<const float2*>(LLu + 2 * i * Sp + 2 * j);
                const float2 t1 = *reinterpret_cast<const float2*>(LLu + (2 * i + 1) * Sp + 2 * j);
                float uu[4];
                haar4(t0.x, t0.y, t1.x, t1.y, uu[0], uu[1], uu[2], uu[3]);
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) U2[sb * BSl + i * Sl + PK + j] = uu[sb];
            }
            for (int q = tid; q < (TH >> 2) * wl; q += NT) {
                const int i = wl == 64 ? wave + (q - tid) / 64 : q / wl, j = wl == 64 ? lane : q - i * wl;
                const float2 t0 = *reinterpret_cast<const float2*>(V1 + 2 * i * SVp + 2 * j);
                const float2 t1 = *reinterpret_cast<const float2*>(V1 + (2 * i + 1) * SVp + 2 * j);
                float vv[4];
                haar4(t0.x, t0.y, t1.x, t1.y, vv[0], vv[1], vv[2], vv[3]);
#pragma unroll
                for (int sb = 0; sb < 4; ++sb) V2[sb * VSl + i * SVl + j] = vv[sb];
            }
        }
        lds_barrier();
        // the coarse pass's inputs: the tile's level-2 LL sums of x and dy
        if (P::LT > L0) {
            constexpr int hl = TH >> L0, wl = W >> L0, Sl = P::su(L0), GLv = G >> L0;
            const float* LLu = U2 + PK;
            float* pxo = px + plane * (H >> L0) * wl + (size_t)(r0 >> L0) * wl;
            float* pdo = pdy + plane * (H >> L0) * wl + (size_t)(r0 >> L0) * wl;
            constexpr int SVL = P::sv(L0);
            for (int q = tid; q < hl * wl; q += NT) {
                const int i = wl == 64 ? wave + (q - tid) / 64 : q / wl, j = wl == 64 ? lane : q - i * wl;
                pxo[q] = LLu[(GLv + i) * Sl + j];
                pdo[q] = V2[i * SVL + j];
            }
        }
        // ------------------------------------------------ P3: level-2 taps
        level_taps(std::integral_constant<int, 2>{});
        // the next unit's P0 overwrites every region: wait for every reader
        // (the loop's barriers order LDS only: the LL sums this unit wrote to
        // global memory are read by a later kernel, and the next unit's
        // loads stay in flight)
        lds_barrier();
    }

#pragma unroll
    for (int t = 0; t < ACCM; ++t) acc[t] = wave_sum(acc[t]);
    __syncthreads();
    float* red = lds;                // [NW][ACCM] level taps per wavefront
    float* redD = lds + NW * ACCM;   // [NW][16][16] matrix-core sums per wavefront
    if (lane == 0) {
#pragma unroll
        for (int t = 0; t < ACCM; ++t) red[wave * ACCM + t] = acc[t];
    }
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) redD[wave * 256 + (4 * (lane >> 4) + jj) * 16 + (lane & 15)] = dacc[jj];
    __syncthreads();
    float* dst = part + ((size_t)chunk * C + c) * P::TAPS;
    for (int t = tid; t < P::TAPS; t += NT) {
        float v = 0.f;
        if (t < KB * KB) {
            const int i = t / KB, j = t - i * KB;
            for (int w = 0; w < NW; ++w) {   // wavefronts in order, dy row h then h + 1
                v += redD[w * 256 + i * 16 + j];
                v += redD[w * 256 + (i + 1) * 16 + 8 + j];
            }
        } else {
            const int r = t - KB * KB, ls = r / (K * K), tap = r - ls * (K * K);
            const int l = ls / 4 + 1, sb = ls - (l - 1) * 4;
            for (int h = 0; h < NW / 4; ++h) v += red[(sb + 4 * h) * ACCM + (l - 1) * K * K + tap];
        }
        dst[t] = v;
    }
}

// ------------------------------------------------------------ registry

// Compute units of the current device (queried once per device).
int cu_count() {
    constexpr int MAXDEV = 64;
    static int cache[MAXDEV];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
    if (dev < MAXDEV && cache[dev] > 0) return cache[dev];
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n < 1) n = 256;
    if (dev < MAXDEV) cache[dev] = n;
    return n;
}

// split planes: the fine tiles (base and levels 1..L0, plus the LL sums),
// the coarse pass on the LL sums (levels L0+1..L), then the finalize
template <class FP, class CP>
static size_t split_bw_ws(int B, int C) {
    const int units = B * FP::NTILE;
    const int nA = cdiv(units, chunk_units(units, C));
    size_t n = bw_align256((size_t)nA * C * FP::TAPS * sizeof(float));
    if (FP::LT > FP::L0) {
        const int nB = cdiv(B, chunk_units(B, C));
        n += bw_align256((size_t)nB * C * 4 * (FP::LT - FP::L0) * FP::K * FP::K * sizeof(float));
        n += 2 * bw_align256((size_t)B * C * (FP::H >> FP::L0) * (FP::W >> FP::L0) * sizeof(float));
    }
    return n;
}

// byte offset of the dy sums (pdy) in the workspace split_bw_launch lays out
template <class FP, class CP>
static size_t split_bw_dy_sums_offset(int B, int C) {
    static_assert(FP::LT > FP::L0, "the LL planes exist only with a coarse pass");
    const int units = B * FP::NTILE;
    const int nA = cdiv(units, chunk_units(units, C)), nB = cdiv(B, chunk_units(B, C));
    return bw_align256((size_t)nA * C * FP::TAPS * sizeof(float)) +
           bw_align256((size_t)nB * C * 4 * (FP::LT - FP::L0) * FP::K * FP::K * sizeof(float)) +
           bw_align256((size_t)B * C * (FP::H >> FP::L0) * (FP::W >> FP::L0) * sizeof(float));
}

template <class FP, class CP, typename T>
static hipError_t split_bw_launch(const void* x, const void* dy, const float* w_lvl, const float* scale,
                                  float* dw_base, float* dw_lvl, float* dscale, void* ws, int B, int C,
                                  hipStream_t stream) {
    const int units = B * FP::NTILE;
    const int upc = chunk_units(units, C), nA = cdiv(units, upc);
    char* cur = (char*)ws;
    float* partA = (float*)cur;
    cur += bw_align256((size_t)nA * C * FP::TAPS * sizeof(float));
    float *partB = nullptr, *px = nullptr, *pdy = nullptr;
    int nB = 0;
    if constexpr (FP::LT > FP::L0) {
        nB = cdiv(B, chunk_units(B, C));
        partB = (float*)cur;
        cur += bw_align256((size_t)nB * C * 4 * (FP::LT - FP::L0) * FP::K * FP::K * sizeof(float));
        const size_t pl = (size_t)B * C * (FP::H >> FP::L0) * (FP::W >> FP::L0) * sizeof(float);
        px = (float*)cur;
        cur += bw_align256(pl);
        pdy = (float*)cur;
    }
    if constexpr (FP::MF && sizeof(T) == 2)
        hipLaunchKernelGGL((tile_bwdw_mf_kernel<FP>), dim3((unsigned)(nA * C)), dim3(FP::NTM), 0, stream,
                           (const bf16_t*)x, (const bf16_t*)dy, partA, px, pdy, B, C, upc);
    else
        hipLaunchKernelGGL((tile_bwdw_kernel<FP, T>), dim3((unsigned)(nA * C)), dim3(FP::NT), 0, stream,
                           (const T*)x, (const T*)dy, partA, px, pdy, B, C, upc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    if constexpr (FP::LT > FP::L0) {
        const int bpc = chunk_units(B, C);
        hipLaunchKernelGGL((bwdw_kernel<CP, float, false>), dim3((unsigned)(nB * C)), dim3(CP::NT), 0, stream,
                           (const float*)px, (const float*)pdy, partB, (float*)nullptr, (float*)nullptr, B, C,
                           bpc);
        err = hipGetLastError();
        if (err != hipSuccess) return err;
    }
    return launch_bwdw_finalize(partA, nA, FP::L0, partB, nB, C, FP::LT, FP::KB, FP::K, w_lvl, scale, dw_base, dw_lvl,
                                dscale, stream);
}

// L = 0: the base taps alone, G[m][n] = sum_{b,h,w} dy[h][w] x[h+m-kb/2][w+n-kb/2].
// One workgroup per (channel, chunk of the batch); NPW planes per step: their
// x interiors (bordered, zero borders written once) and dy stream into LDS,
// every lane correlates one RB-row column strip (taps_col) into kb*kb sums
// kept in registers across the chunk; the end of the chunk reduces them as
// the general kernel does (16-lane rows by DPP, rows and waves through LDS
// in a fixed order).
template <class P, typename T>
__global__ __launch_bounds__(P::NT) void dw_bwdw_kernel(const T* __restrict__ x, const T* __restrict__ dy,
                                                        float* __restrict__ part, int B, int C, int bpc) {
    constexpr int H = P::H, W = P::W, KB = P::KB, NT = P::NT, RB = P::RB, NPB = P::NPW, NW = NT / 64;
    constexpr int PB = P::PB, XO = P::XO, SX = P::SX, SD = P::SD, VA = P::VA, NQ = P::NQ, LPB = P::LPB;
    constexpr int NIB = P::NIB, KB2 = KB * KB;
    constexpr int PL = round_up(P::XSIZE + P::DSIZE, 4), RED = NW * 4 * KB2;
    __shared__ __attribute__((aligned(16))) float lds[NPB * PL > RED ? NPB * PL : RED];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c = blockIdx.x % C, chunk = blockIdx.x / C;
    const int b0 = chunk * bpc, b1 = min(B, b0 + bpc);
    {
        float4* const z = reinterpret_cast<float4*>(lds);
        for (int t = tid; t < NPB * PL / 4; t += NT) z[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float acc[KB2];
#pragma unroll
    for (int t = 0; t < KB2; ++t) acc[t] = 0.f;
    for (int b = b0; b < b1; b += NPB) {
        __syncthreads();   // the zeros, or the previous step's taps, are done
        for (int q = tid; q < NPB * NQ; q += NT) {
            const int p = udiv(q, NQ), r = q - p * NQ, row = udiv(r, W / VA), col = (r - row * (W / VA)) * VA;
            float* const X = lds + p * PL + (PB + row) * SX + XO + col;
            float* const D = lds + p * PL + P::XSIZE + row * SD + col;
            if (b + p < b1) {   // planes past the chunk's end hold zeros and add nothing
                const size_t off = ((size_t)(b + p) * C + c) * H * W + (size_t)row * W + col;
                RawVec<T, VA> vx, vd;
                load_raw<T, VA>(x + off, vx);
                load_raw<T, VA>(dy + off, vd);
                store_lds<T, VA>(X, vx);
                store_lds<T, VA>(D, vd);
            } else {
                float zero[VA] = {};
                store_vec<VA>(X, zero);
                store_vec<VA>(D, zero);
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < P::MB; ++it) {
            const int item = tid + it * NT;
            if (!((NPB * NIB) % NT == 0 || item < NPB * NIB)) continue;
            const int p = NPB == 1 ? 0 : udiv(item, NIB), r = item - p * NIB;
            const int rb = udiv(r, LPB), w = r - rb * LPB, h0 = rb * RB;
            if (LPB == W || w < W)
                taps_col<KB, RB, SX, SD>(lds + p * PL + XO - PB + h0 * SX + w, lds + p * PL + P::XSIZE + h0 * SD + w,
                                         acc);
        }
    }
#pragma unroll
    for (int t = 0; t < KB2; ++t) acc[t] = row_sum(acc[t]);
    __syncthreads();   // LDS becomes reduction scratch
    float* const red = lds;   // [NW * 4 rows][KB2]
    if ((lane & 15) == 0) {
        const int wr = wave * 4 + (lane >> 4);
#pragma unroll
        for (int t = 0; t < KB2; ++t) red[wr * KB2 + t] = acc[t];
    }
    __syncthreads();
    for (int t = tid; t < KB2; t += NT) {
        float v = 0.f;
        for (int wr = 0; wr < NW * 4; ++wr) v += red[wr * KB2 + t];
        part[((size_t)chunk * C + c) * KB2 + t] = v;
    }
}

// Single-pass backward for L = 0: each plane of x and dy is read once and
// gives both dx (the correlation of dy with the taps turned by 180 degrees)
// and the base-tap sums of the weight gradient. As dw_bwdw_kernel, with dy
// kept bordered in LDS (the dx windows read its zero border) and the turned
// taps staged once per workgroup.
template <class P, typename T>
__global__ __launch_bounds__(P::NT) void dw_bwd_kernel(const T* __restrict__ x, const T* __restrict__ dy,
                                                       const float* __restrict__ w_base, T* __restrict__ dx,
                                                       float* __restrict__ part, int B, int C, int bpc) {
    constexpr int H = P::H, W = P::W, KB = P::KB, NT = P::NT, RB = P::RB, NPB = P::NPW, NW = NT / 64;
    constexpr int PB = P::PB, XO = P::XO, SX = P::SX, VA = P::VA, NQ = P::NQ, LPB = P::LPB;
    constexpr int NIB = P::NIB, KB2 = KB * KB, KB2P = P::KB2P;
    constexpr int XS = round_up(P::XSIZE, 4), PL = 2 * XS, RED = NW * 4 * KB2;
    __shared__ __attribute__((aligned(16))) float lds[(NPB * PL > RED ? NPB * PL : RED) + KB2P];
    float* const WR = lds + (NPB * PL > RED ? NPB * PL : RED);   // turned taps
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int c = blockIdx.x % C, chunk = blockIdx.x / C;
    const int b0 = chunk * bpc, b1 = min(B, b0 + bpc);
    for (int t = tid; t < KB2P; t += NT) WR[t] = t < KB2 ? w_base[(size_t)c * KB2 + KB2 - 1 - t] : 0.f;
    {
        float4* const z = reinterpret_cast<float4*>(lds);
        for (int t = tid; t < NPB * PL / 4; t += NT) z[t] = make_float4(0.f, 0.f, 0.f, 0.f);
    }
    float acc[KB2];
#pragma unroll
    for (int t = 0; t < KB2; ++t) acc[t] = 0.f;
    for (int b = b0; b < b1; b += NPB) {
        __syncthreads();   // the zeros and taps, or the previous step's reads, are done
        for (int q = tid; q < NPB * NQ; q += NT) {
            const int p = udiv(q, NQ), r = q - p * NQ, row = udiv(r, W / VA), col = (r - row * (W / VA)) * VA;
            float* const X = lds + p * PL + (PB + row) * SX + XO + col;
            float* const D = X + XS;
            if (b + p < b1) {
                const size_t off = ((size_t)(b + p) * C + c) * H * W + (size_t)row * W + col;
                RawVec<T, VA> vx, vd;
                load_raw<T, VA>(x + off, vx);
                load_raw<T, VA>(dy + off, vd);
                store_lds<T, VA>(X, vx);
                store_lds<T, VA>(D, vd);
            } else {
                float zero[VA] = {};
                store_vec<VA>(X, zero);
                store_vec<VA>(D, zero);
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < P::MB; ++it) {
            const int item = tid + it * NT;
            if (!((NPB * NIB) % NT == 0 || item < NPB * NIB)) continue;
            const int p = NPB == 1 ? 0 : udiv(item, NIB), r = item - p * NIB;
            const int rb = udiv(r, LPB), w = r - rb * LPB, h0 = rb * RB;
            if (!(LPB == W || w < W)) continue;
            const float* const Xw = lds + p * PL + XO - PB + h0 * SX + w;   // window origin, x
            taps_col<KB, RB, SX, SX>(Xw, Xw + XS + PB * SX + PB, acc);      // dy interior rows h0..
            if (b + p < b1) {
                float y[RB];
                conv_col<KB, RB, SX>(Xw + XS, WR, y);   // the same window over bordered dy
                T* __restrict__ dst = dx + ((size_t)(b + p) * C + c) * H * W + (size_t)h0 * W + w;
#pragma unroll
                for (int o = 0; o < RB; ++o) {
                    if constexpr (sizeof(T) == 2) dst[o * W] = narrow_bf16(y[o]);
                    else dst[o * W] = y[o];
                }
            }
        }
    }
#pragma unroll
    for (int t = 0; t < KB2; ++t) acc[t] = row_sum(acc[t]);
    __syncthreads();   // LDS becomes reduction scratch
    float* const red = lds;   // [NW * 4 rows][KB2]
    if ((lane & 15) == 0) {
        const int wr = wave * 4 + (lane >> 4);
#pragma unroll
        for (int t = 0; t < KB2; ++t) red[wr * KB2 + t] = acc[t];
    }
    __syncthreads();
    for (int t = tid; t < KB2; t += NT) {
        float v = 0.f;
        for (int wr = 0; wr < NW * 4; ++wr) v += red[wr * KB2 + t];
        part[((size_t)chunk * C + c) * KB2 + t] = v;
    }
}

// planes per chunk: about four workgroups per CU in all
static int dw_bw_bpc(int B, int C) { return chunk_units(B, C, cu_count() * 4); }

template <class P>
static size_t dw_bw_ws(int B, int C) {
    return (size_t)cdiv(B, dw_bw_bpc(B, C)) * C * P::KB * P::KB * sizeof(float);
}

template <class P, typename T>
static hipError_t dw_bw_launch(const void* x, const void* dy, const float* w_lvl, const float* scale,
                               float* dw_base, float* dw_lvl, float* dscale, void* ws, int B, int C,
                               hipStream_t stream) {
    (void)w_lvl; (void)scale; (void)dw_lvl; (void)dscale;
    const int bpc = dw_bw_bpc(B, C), nch = cdiv(B, bpc);
    float* part = (float*)ws;
    hipLaunchKernelGGL((dw_bwdw_kernel<P, T>), dim3((unsigned)(nch * C)), dim3(P::NT), 0, stream, (const T*)x,
                       (const T*)dy, part, B, C, bpc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    // the finalize with no levels: the fixed-order chunk sum of the base taps
    return launch_bwdw_finalize(part, nch, 0, nullptr, 0, C, 0, P::KB, 1, nullptr, nullptr, dw_base, nullptr, nullptr,
                                stream);
}

template <class P, typename T>
static hipError_t dw_bwd_launch(const void* x, const void* dy, const float* w_base, void* dx, float* dw_base,
                                void* ws, int B, int C, hipStream_t stream) {
    const int bpc = dw_bw_bpc(B, C), nch = cdiv(B, bpc);
    float* part = (float*)ws;
    hipLaunchKernelGGL((dw_bwd_kernel<P, T>), dim3((unsigned)(nch * C)), dim3(P::NT), 0, stream, (const T*)x,
                       (const T*)dy, w_base, (T*)dx, part, B, C, bpc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_bwdw_finalize(part, nch, 0, nullptr, 0, C, 0, P::KB, 1, nullptr, nullptr, dw_base, nullptr, nullptr,
                                stream);
}

typedef hipError_t (*bwd1_fn)(const void* x, const void* dy, const float* w_base, void* dx, float* dw_base,
                              void* ws, int B, int C, hipStream_t stream);
struct Bwd1Entry {
    int H, W, KB;
    bwd1_fn fn[2];
    size_t (*ws)(int B, int C);
};

// whole-plane plans of the small test shapes
typedef BwPlan<32, 32, 2, 5, 5> BP_32_L2_k55;
typedef BwPlan<14, 14, 1, 5, 5, 1, 8> BP_14_L1_k55;
typedef BwPlan<32, 32, 3, 7, 5> BP_32_L3_k75;
typedef BwPlan<24, 40, 3, 3, 3> BP_24x40_L3_k33;
typedef BwPlan<16, 16, 4, 3, 7> BP_16_L4_k37;
typedef BwPlan<64, 64, 4, 7, 5> BP_64_L4_k75;

// split plans: fine tiles + coarse planes of LL_{L0} sums (no base taps)
// 32-row tiles where the halo is 4 rows (one fine level): 10 % faster than
// 16 at 128² L1; with two fine levels (8-row halo) 16 rows are 4-8 % faster
// (the matrix-core weight gradient measured slower at 128x128: 0.204 against
// about 0.18 ms per call at L = 2, 5x5 base taps being a smaller share)
typedef TileBwPlan<128, 128, 1, 1, 5, 5, 32> TB_128_L1_k55;
typedef TileBwPlan<128, 128, 2, 2, 5, 5, 16> TB_128_L2_k55;
typedef TileBwPlan<128, 128, 2, 3, 5, 5, 16> TB_128_L2of3_k55;
typedef TileBwPlan<128, 128, 2, 4, 5, 5, 16> TB_128_L2of4_k55;
typedef TileBwPlan<128, 128, 2, 5, 5, 5, 16> TB_128_L2of5_k55;
typedef BwPlan<32, 32, 1, 1, 5, 1, 4> CB_32_L1_k5;
typedef BwPlan<32, 32, 2, 1, 5, 2, 4> CB_32_L2_k5;
typedef BwPlan<32, 32, 3, 1, 5, 3, 4> CB_32_L3_k5;
// 16-row tiles: the 8-row halo on each side costs 1.5 tiles of rows instead
// of 3 with 8-row tiles (1.34 -> 1.06 ms at 16x256x256²). 1024 lanes (four
// waves per SIMD under the one workgroup per CU that 114 KB of LDS allow, 8-
// and 2-row strips) measured slower: 1.07 against 0.99 ms
typedef TileBwPlan<256, 256, 2, 4, 7, 5, 16, 512, true> TB_256_L2of4_k75;
typedef BwPlan<64, 64, 2, 1, 5> CB_64_L2_k5;
typedef TileBwPlan<64, 64, 2, 4, 3, 3, 8> TB_64_L2of4_k33;
typedef BwPlan<16, 16, 2, 1, 3, 2, 8> CB_16_L2_k3;
typedef TileBwPlan<64, 64, 1, 2, 5, 5, 16> TB_64_L1of2_k55;

// whole planes split by level (fine: base + level 1; coarse: the rest, on
// the level-1 LL planes, several planes per step)
typedef BwPlan<56, 56, 1, 5, 5, 3> WP_56_L1of3_k55;
typedef BwPlan<28, 28, 2, 1, 5, 2, 4> CB_28_L2_k5;
typedef BwPlan<28, 28, 1, 5, 5, 2, 2> WP_28_L1of2_k55;
typedef BwPlan<14, 14, 1, 1, 5, 1, 8> CB_14_L1_k5;

typedef DwPlan<56, 56, 5, 256, 14, 1> DB_56_k5;
typedef DwPlan<56, 56, 7, 256, 14, 1> DB_56_k7;
typedef DwPlan<28, 28, 5, 256, 7, 2> DB_28_k5;
typedef DwPlan<28, 28, 7, 256, 7, 2> DB_28_k7;
typedef DwPlan<14, 14, 5, 256, 14, 16> DB_14_k5;
typedef DwPlan<14, 14, 7, 256, 14, 16> DB_14_k7;
// L = 0 entries match any k_level (no level kernels)
#define WTC_BW_DW(PLAN) {PLAN::H, PLAN::W, 0, PLAN::KB, 0, {dw_bw_launch<PLAN, float>, dw_bw_launch<PLAN, bf16_t>}, dw_bw_ws<PLAN>}

#define WTC_BW_WHOLE(PLAN) \
    {PLAN::IH, PLAN::IW, PLAN::L, PLAN::KB, PLAN::K, {whole_launch<PLAN, float>, whole_launch<PLAN, bf16_t>}, whole_ws<PLAN>}
#define WTC_BW_PLANESPLIT(FPL, CPL)                                                               \
    {FPL::H, FPL::W, FPL::LT, FPL::KB, FPL::K,                                                   \
     {plane_split_launch<FPL, CPL, float>, plane_split_launch<FPL, CPL, bf16_t>}, plane_split_ws<FPL, CPL>}
#define WTC_BW_SPLIT(FPL, CPL)                                                                    \
    {FPL::H, FPL::W, FPL::LT, FPL::KB, FPL::K,                                                   \
     {split_bw_launch<FPL, CPL, float>, split_bw_launch<FPL, CPL, bf16_t>}, split_bw_ws<FPL, CPL>}
// ... and its dy sums, offered to the backward-data pass
#define WTC_BW_SPLIT_SUMS(FPL, CPL)                                                               \
    {FPL::H, FPL::W, FPL::LT, FPL::KB, FPL::K,                                                   \
     {split_bw_launch<FPL, CPL, float>, split_bw_launch<FPL, CPL, bf16_t>}, split_bw_ws<FPL, CPL>,  \
     FPL::L0, split_bw_dy_sums_offset<FPL, CPL>}

static const BwEntry kBwEntries[] = {
    WTC_BW_PLANESPLIT(WP_56_L1of3_k55, CB_28_L2_k5), WTC_BW_PLANESPLIT(WP_28_L1of2_k55, CB_14_L1_k5),
    WTC_BW_WHOLE(BP_32_L2_k55), WTC_BW_WHOLE(BP_14_L1_k55),    WTC_BW_WHOLE(BP_32_L3_k75),
    WTC_BW_WHOLE(BP_24x40_L3_k33), WTC_BW_WHOLE(BP_16_L4_k37), WTC_BW_WHOLE(BP_64_L4_k75),
    WTC_BW_SPLIT(TB_128_L1_k55, CB_32_L1_k5),      WTC_BW_SPLIT(TB_128_L2_k55, CB_32_L1_k5),
    WTC_BW_SPLIT(TB_128_L2of3_k55, CB_32_L1_k5),   WTC_BW_SPLIT(TB_128_L2of4_k55, CB_32_L2_k5),
    WTC_BW_SPLIT(TB_128_L2of5_k55, CB_32_L3_k5),   WTC_BW_SPLIT_SUMS(TB_256_L2of4_k75, CB_64_L2_k5),
    WTC_BW_SPLIT_SUMS(TB_64_L2of4_k33, CB_16_L2_k3),    WTC_BW_SPLIT_SUMS(TB_64_L1of2_k55, CB_32_L1_k5),
    WTC_BW_DW(DB_56_k5), WTC_BW_DW(DB_56_k7), WTC_BW_DW(DB_28_k5), WTC_BW_DW(DB_28_k7), WTC_BW_DW(DB_14_k5),
    WTC_BW_DW(DB_14_k7),
};

#define WTC_BWD1(PLAN) {PLAN::H, PLAN::W, PLAN::KB, {dw_bwd_launch<PLAN, float>, dw_bwd_launch<PLAN, bf16_t>}, dw_bw_ws<PLAN>}
static const Bwd1Entry kBwd1Entries[] = {
    WTC_BWD1(DB_56_k5), WTC_BWD1(DB_56_k7), WTC_BWD1(DB_28_k5),
    WTC_BWD1(DB_28_k7), WTC_BWD1(DB_14_k5), WTC_BWD1(DB_14_k7),
};

static const Bwd1Entry* find_bwd1(int H, int W, int KB) {
    for (const Bwd1Entry& e : kBwd1Entries)
        if (e.H == H && e.W == W && e.KB == KB) return &e;
    return nullptr;
}

size_t bwd_single_pass_workspace_bytes(int B, int C, int H, int W, int L, int KB) {
    const Bwd1Entry* e = L == 0 ? find_bwd1(H, W, KB) : nullptr;
    return e ? e->ws(B, C) : (size_t)-1;
}

hipError_t bwd_single_pass_launch(int B, int C, int H, int W, int KB, bool bf16, const void* x, const void* dy,
                                  const float* w_base, void* dx, float* dw_base, void* ws, hipStream_t stream) {
    const Bwd1Entry* e = find_bwd1(H, W, KB);
    if (!e) return hipErrorInvalidValue;
    return e->fn[bf16 ? 1 : 0](x, dy, w_base, dx, dw_base, ws, B, C, stream);
}

// the tuned plans first, then the stage-plane family
static const BwEntry* find_bw(int H, int W, int L, int KB, int K) {
    for (const BwEntry& e : kBwEntries)
        if (e.H == H && e.W == W && e.L == L && e.KB == KB && (L == 0 || e.K == K)) return &e;
    return L > 0 ? find_family_bw_entry(H, W, L, KB, K) : nullptr;
}

bool bwdw_dy_sums(int B, int C, int H, int W, int L, int KB, int K, int* l0, size_t* offset) {
    const BwEntry* e = find_bw(H, W, L, KB, K);
    if (!e || !e->dy_sums_offset) return false;
    *l0 = e->l0;
    *offset = e->dy_sums_offset(B, C);
    return true;
}

size_t bwdw_workspace_bytes(int B, int C, int H, int W, int L, int KB, int K) {
    const BwEntry* e = find_bw(H, W, L, KB, K);
    return e ? e->ws(B, C) : (size_t)-1;
}

hipError_t launch_finalize(const FinalizeArgs& f, hipStream_t stream) {
    hipLaunchKernelGGL(bwdw_finalize, dim3((unsigned)f.C), dim3(finalize_threads(f.KB, f.K, f.L)), 0, stream, f);
    return hipGetLastError();
}

hipError_t bwdw_launch_deferred(int B, int C, int H, int W, int L, int KB, int K, bool bf16, const void* x,
                                const void* dy, const float* w_lvl, const float* scale, float* dw_base,
                                float* dw_lvl, float* dscale, void* ws, hipStream_t stream, FinalizeArgs* fin) {
    fin->C = 0;
    g_defer = fin;
    const hipError_t err =
        bwdw_launch(B, C, H, W, L, KB, K, bf16, x, dy, w_lvl, scale, dw_base, dw_lvl, dscale, ws, stream);
    g_defer = nullptr;
    return err;
}

hipError_t bwdw_launch(int B, int C, int H, int W, int L, int KB, int K, bool bf16, const void* x,
                       const void* dy, const float* w_lvl, const float* scale, float* dw_base,
                       float* dw_lvl, float* dscale, void* ws, hipStream_t stream) {
    const BwEntry* e = find_bw(H, W, L, KB, K);
    if (!e) return hipErrorInvalidValue;
    return e->fn[bf16 ? 1 : 0](x, dy, w_lvl, scale, dw_base, dw_lvl, dscale, ws, B, C, stream);
}

}  // namespace wtc
