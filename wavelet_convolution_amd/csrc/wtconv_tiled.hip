// Fine pass of WTConv for planes too large for one workgroup's LDS.
//
// The layer splits at level L0 (the abstract of arXiv:2608.10805: the
// receptive field doubles per level, so a plane-sized tile would be needed
// for the coarse levels). Levels L0+1..L act on x only through the
// unnormalised LL band at level L0 (2^L0 x 2^L0 block sums), so a coarse
// pass (plane_kernel with SHIFT = L0) evaluates them once per plane on that
// small image and leaves C = 4^-L0 * branch(P), constant on 2^L0 blocks.
// This fine pass covers full-width tiles of TH rows: it streams the tile's
// rows of x plus a halo of G = max(kb/2, (k/2) 2^L0) rows (rounded to a
// whole 2^L0 block, so every level's band grid stays aligned), recomputes
// the Haar bands of levels 1..L0 on chip, and writes
//   y = base conv + sum_{l<=L0} closed-form synthesis + C[h >> L0][w >> L0].
// Rows of the halo outside the plane are zero, which is the zero padding of
// every level's band grid.
//
// Workgroups are numbered so that the tiles of one plane run on the same
// accelerator complex die (XCD): the hardware hands consecutive workgroups to
// consecutive XCDs, each with its own L2, and neighbouring tiles read the
// same halo rows.
#include "wtconv_plane.h"
#include "wtconv_tiled.h"

namespace wtc {

// logical workgroup index whose consecutive values land on one XCD
__device__ __forceinline__ int xcd_local_index() {
    const int n = gridDim.x, b = blockIdx.x;
    if (n % 8 != 0) return b;
    return (b % 8) * (n / 8) + b / 8;
}

template <int H_, int W_, int L0_, int LT_, int KB_, int K_, int TH_, int NT_, int TR_, int TC_>
struct TilePlan {
    static constexpr int H = H_, W = W_, L0 = L0_, LT = LT_, KB = KB_, K = K_, TH = TH_, NT = NT_;
    static constexpr int TR = TR_, TC = TC_;
    static constexpr int PB = KB / 2, PK = K / 2, BLK = 1 << L0;
    static_assert(L0 >= 1 && L0 <= LT, "fine levels 1..L0");
    static_assert(H % (1 << LT) == 0 && W % (1 << LT) == 0, "plane must divide into 2^L blocks");
    static_assert(TH % BLK == 0 && H % TH == 0, "tiles are whole 2^L0 blocks");
    static constexpr int G0 = PB > (PK << L0) ? PB : (PK << L0);
    static constexpr int G = cdiv(G0, BLK) * BLK;   // halo rows above and below
    static constexpr int RH0 = TH + 2 * G;
    static constexpr int SX = odd_stride(W + 2 * PB);
    static constexpr int XSIZE = RH0 * SX;
    static constexpr int rh(int l) { return RH0 >> l; }
    static constexpr int su(int l) { return odd_stride((W >> l) + 2 * PK); }
    static constexpr int bandsz(int l) { return rh(l) * su(l); }
    static constexpr int uoff(int l) {
        int o = 0;
        for (int q = 2; q < l; ++q) o += 4 * bandsz(q);
        return o;
    }
    static constexpr int UDEEP = uoff(L0 + 1);
    static constexpr int ASIZE = XSIZE > UDEEP ? XSIZE : UDEEP;
    static constexpr int BSIZE = 4 * bandsz(1);
    static constexpr int LDS_FLOATS = (ASIZE + BSIZE + 3) / 4 * 4;
    static constexpr int KB2P = kpad4(KB), K2P = kpad4(K);
    static constexpr int WFLOATS = KB2P + 4 * L0 * K2P;
    static_assert((LDS_FLOATS + WFLOATS) * 4 <= 160 * 1024, "tile does not fit in LDS");
    static_assert((TH / 2) % TR == 0 && (W / 2) % TC == 0, "main tile must divide the tile's level-1 grid");
    static constexpr int NI = ((TH / 2) / TR) * ((W / 2) / TC);
    static constexpr int MI = cdiv(NI, NT);
    static constexpr int NTILE = H / TH;
    static constexpr Tile deep_tile(int l) { return pick_tile(TH >> l, W >> l, NT); }
    static constexpr int WG_PER_CU = (160 * 1024) / ((LDS_FLOATS + WFLOATS) * 4);
    static constexpr int WAVES_PER_EU_LDS = (WG_PER_CU * (NT / 64)) / 4;
    static constexpr int WAVES_PER_EU =
        WAVES_PER_EU_LDS < 1 ? 1 : (WAVES_PER_EU_LDS > 4 ? 4 : WAVES_PER_EU_LDS);

    template <class F>
    __device__ static __forceinline__ void for_deep_levels(F&& f) {
        deep_impl(f, std::make_integer_sequence<int, (L0 >= 2 ? L0 - 1 : 0)>{});
    }
    template <class F, int... I>
    __device__ static __forceinline__ void deep_impl(F& f, std::integer_sequence<int, I...>) {
        (f(std::integral_constant<int, I + 2>{}), ...);
    }
};

template <class P, typename T, bool FLIP>
__global__ __launch_bounds__(P::NT) __attribute__((amdgpu_waves_per_eu(P::WAVES_PER_EU)))
void tile_kernel(const T* __restrict__ in, const float* __restrict__ w_base,
                 const float* __restrict__ w_lvl, const float* __restrict__ scale,
                 const float* __restrict__ coarse, T* __restrict__ out, int C) {
    constexpr int H = P::H, W = P::W, L0 = P::L0, KB = P::KB, K = P::K, NT = P::NT, TH = P::TH;
    constexpr int TR = P::TR, TC = P::TC, PB = P::PB, PK = P::PK, G = P::G, RH0 = P::RH0;
    constexpr int SX = P::SX, W1 = W / 2;
    constexpr int S1 = P::su(1), BS1 = P::bandsz(1);
    constexpr int NI = P::NI, MI = P::MI, TPR = W1 / TC;
    constexpr int KB2P = P::KB2P, K2P = P::K2P;

    __shared__ __attribute__((aligned(16))) float lds[P::LDS_FLOATS + P::WFLOATS];
    float* A = lds;               // x rows (bordered), later U_2..U_L0 and their results
    float* Bq = lds + P::ASIZE;   // U_1 rows (4 bands, bordered columns)
    float* WB = lds + P::LDS_FLOATS;
    float* WL = WB + KB2P;

    const int tid = threadIdx.x;
    const int lid = xcd_local_index();
    const int plane = lid / P::NTILE, tile = lid - plane * P::NTILE;
    const int c = plane % C;
    const int r0 = tile * TH;
    const T* __restrict__ src = in + (size_t)plane * H * W;
    T* __restrict__ dst = out + (size_t)plane * H * W;

    // ---------------------------------------------------------------- P0
    for (int t = tid; t < KB2P; t += NT)
        WB[t] = t < KB * KB ? w_base[(size_t)c * KB * KB + (FLIP ? KB * KB - 1 - t : t)] : 0.f;
    for (int t = tid; t < 4 * L0 * K2P; t += NT) {
        const int ls = t / K2P, tap = t - ls * K2P, l = ls >> 2, s = ls & 3;
        const size_t pi = ((size_t)l * C + c) * 4 + s;
        const float f = scale[pi] * (1.0f / (float)(1 << (2 * (l + 1))));
        WL[t] = tap < K * K ? w_lvl[pi * K * K + (FLIP ? K * K - 1 - tap : tap)] * f : 0.f;
    }
    // border columns of every x row; rows of the halo outside the plane are zero
    for (int i = tid; i < RH0 * (SX - W); i += NT) {
        const int r = i / (SX - W), q = i - r * (SX - W);
        A[r * SX + (q < PB ? q : q + W)] = 0.f;
    }
    for (int i = tid; i < 4 * P::rh(1) * (S1 - W1); i += NT) {
        const int b = i / (P::rh(1) * (S1 - W1)), j = i - b * (P::rh(1) * (S1 - W1));
        const int r = j / (S1 - W1), q = j - r * (S1 - W1);
        Bq[b * BS1 + r * S1 + (q < PK ? q : q + W1)] = 0.f;
    }
    {
        constexpr int V = vec_elems<T>(W, H * W);
        constexpr int NV = RH0 * W / V;
        constexpr int NL = cdiv(NV, NT);
        float v[NL][V];
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int q = tid + k * NT;
            const int e = q * V, rr = e / W, pr = r0 - G + rr;
            if ((NV % NT == 0 || q < NV) && pr >= 0 && pr < H)
                load_vec<T, V>(src + (size_t)pr * W + (e - rr * W), v[k]);
            else
#pragma unroll
                for (int i = 0; i < V; ++i) v[k][i] = 0.f;
        }
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int q = tid + k * NT;
            if (NV % NT == 0 || q < NV) {
                const int e = q * V, rr = e / W, col = e - rr * W;
#pragma unroll
                for (int i = 0; i < V; ++i) A[rr * SX + col + PB + i] = v[k][i];
            }
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- P1
    float yb[MI][2 * TR][2 * TC];
#pragma unroll
    for (int it = 0; it < MI; ++it) {
        const int item = tid + it * NT;
        if (NI % NT == 0 || item < NI) {
            const int ti = item / TPR, tj = item - ti * TPR;
            const int h0 = 2 * TR * ti, w0 = 2 * TC * tj;   // tile-relative output origin
            conv_tile<KB, 2 * TR, 2 * TC, SX>(A + (G + h0 - PB) * SX + w0, WB, yb[it]);
        }
    }
    // level-1 bands of every region row (the halo feeds the coarser levels)
    for (int q = tid; q < P::rh(1) * W1; q += NT) {
        const int i = q / W1, j = q - i * W1;
        const float* x2 = A + (2 * i) * SX + PB + 2 * j;
        float b[4];
        haar4(x2[0], x2[1], x2[SX], x2[SX + 1], b[0], b[1], b[2], b[3]);
#pragma unroll
        for (int s = 0; s < 4; ++s) Bq[s * BS1 + i * S1 + PK + j] = b[s];
    }
    __syncthreads();

    // ---------------------------------------------------------------- P2
    P::for_deep_levels([&](auto lc) {
        constexpr int l = decltype(lc)::value;
        constexpr int rl = P::rh(l), wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l);
        constexpr int Sp = P::su(l - 1);
        float* Ul = A + P::uoff(l);
        const float* LLp = (l == 2) ? (Bq + PK) : (A + P::uoff(l - 1) + PK);
        for (int i = tid; i < 4 * rl * (Sl - wl); i += NT) {
            const int b = i / (rl * (Sl - wl)), j = i - b * (rl * (Sl - wl));
            const int r = j / (Sl - wl), q = j - r * (Sl - wl);
            Ul[b * BSl + r * Sl + (q < PK ? q : q + wl)] = 0.f;
        }
        for (int q = tid; q < rl * wl; q += NT) {
            const int i = q / wl, j = q - i * wl;
            const float* x2 = LLp + 2 * i * Sp + 2 * j;
            float b[4];
            haar4(x2[0], x2[1], x2[Sp], x2[Sp + 1], b[0], b[1], b[2], b[3]);
#pragma unroll
            for (int s = 0; s < 4; ++s) Ul[s * BSl + i * Sl + PK + j] = b[s];
        }
        __syncthreads();
    });

    // ---------------------------------------------------------------- P3
    P::for_deep_levels([&](auto lc) {
        constexpr int l = decltype(lc)::value;
        constexpr int hl = TH >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), Gl = G >> l;
        constexpr Tile tl = P::deep_tile(l);
        constexpr int RR = tl.r, CC = tl.c, TPRl = wl / CC, NIl = (hl / RR) * TPRl;
        constexpr int MIl = cdiv(NIl, NT);
        float* Ul = A + P::uoff(l);
        float z[MIl][4][RR][CC];
#pragma unroll
        for (int it = 0; it < MIl; ++it) {
            const int item = tid + it * NT;
            const int ti = item / TPRl, tj = item - ti * TPRl;
#pragma unroll
            for (int s = 0; s < 4; ++s)
                if (NIl % NT == 0 || item < NIl)
                    conv_tile<K, RR, CC, Sl>(Ul + s * BSl + (Gl + RR * ti - PK) * Sl + CC * tj,
                                             WL + ((l - 1) * 4 + s) * K2P, z[it][s]);
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < MIl; ++it) {
            const int item = tid + it * NT;
            if (NIl % NT == 0 || item < NIl) {
                const int ti = item / TPRl, tj = item - ti * TPRl;
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int r = 0; r < RR; ++r)
#pragma unroll
                        for (int q = 0; q < CC; ++q)
                            Ul[s * BSl + (Gl + RR * ti + r) * Sl + PK + CC * tj + q] = z[it][s][r][q];
            }
        }
    });
    if constexpr (L0 >= 2) __syncthreads();

    // ---------------------------------------------------------------- P4
    constexpr int CW = W >> L0;   // coarse image row length
    const float* __restrict__ cpl = coarse ? coarse + (size_t)plane * (H >> L0) * CW : nullptr;
#pragma unroll
    for (int it = 0; it < MI; ++it) {
        const int item = tid + it * NT;
        if (!(NI % NT == 0 || item < NI)) continue;
        const int ti = item / TPR, tj = item - ti * TPR;
        const int i0 = TR * ti, j0 = TC * tj;   // tile-relative level-1 origin
        float z1[4][TR][TC];
#pragma unroll
        for (int s = 0; s < 4; ++s)
            conv_tile<K, TR, TC, S1>(Bq + s * BS1 + ((G >> 1) + i0 - PK) * S1 + j0, WL + s * K2P, z1[s]);
#pragma unroll
        for (int r = 0; r < TR; ++r) {
            float row0[2 * TC], row1[2 * TC];
#pragma unroll
            for (int q = 0; q < TC; ++q) {
                const int i = i0 + r, j = j0 + q;
                float e = 0.f;
                P::for_deep_levels([&](auto lc) {
                    constexpr int l = decltype(lc)::value;
                    constexpr int Sl = P::su(l), BSl = P::bandsz(l), Gl = G >> l;
                    const float* Zl = A + P::uoff(l) + (Gl + (i >> (l - 1))) * Sl + PK + (j >> (l - 1));
                    const bool bi = (i >> (l - 2)) & 1, bj = (j >> (l - 2)) & 1;
                    const float a0 = Zl[0], a1 = Zl[BSl], a2 = Zl[2 * BSl], a3 = Zl[3 * BSl];
                    e += a0 + (bi ? -a1 : a1) + (bj ? -a2 : a2) + ((bi != bj) ? -a3 : a3);
                });
                if (cpl) e += cpl[(size_t)(((r0 >> 1) + i) >> (L0 - 1)) * CW + (j >> (L0 - 1))];
                const float p0 = z1[0][r][q], p1 = z1[1][r][q], p2 = z1[2][r][q], p3 = z1[3][r][q];
                row0[2 * q] = yb[it][2 * r][2 * q] + (p0 + p1 + p2 + p3) + e;
                row0[2 * q + 1] = yb[it][2 * r][2 * q + 1] + (p0 + p1 - p2 - p3) + e;
                row1[2 * q] = yb[it][2 * r + 1][2 * q] + (p0 - p1 + p2 - p3) + e;
                row1[2 * q + 1] = yb[it][2 * r + 1][2 * q + 1] + (p0 - p1 - p2 + p3) + e;
            }
            const int h = r0 + 2 * (i0 + r), w0 = 2 * j0;
            store_row<2 * TC>(dst + (size_t)h * W + w0, row0);
            store_row<2 * TC>(dst + (size_t)(h + 1) * W + w0, row1);
        }
    }
}

// ------------------------------------------------------------ registry

template <class FP, class CP, typename T, bool FLIP>
static hipError_t launch_split(const void* in, const float* wb, const float* wl, const float* sc, void* out,
                               float* ws, int B, int C, hipStream_t stream) {
    constexpr int L0 = FP::L0, LT = FP::LT;
    const unsigned planes = (unsigned)B * (unsigned)C;
    float* coarse = nullptr;
    if constexpr (LT > L0) {
        coarse = ws;
        const size_t lvl = (size_t)C * 4 * FP::K * FP::K;
        hipError_t err = launch_coarse<CP, T, FLIP, L0>(in, wl + L0 * lvl, sc + (size_t)L0 * C * 4, coarse, B, C,
                                                        stream);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((tile_kernel<FP, T, FLIP>), dim3(planes * FP::NTILE), dim3(FP::NT), 0, stream,
                       (const T*)in, wb, wl, sc, (const float*)coarse, (T*)out, C);
    return hipGetLastError();
}

template <class FP>
static size_t split_ws(int B, int C) {
    if (FP::LT == FP::L0) return 0;
    return (size_t)B * C * (FP::H >> FP::L0) * (FP::W >> FP::L0) * sizeof(float);
}

// coarse-pass plans: the plane of LL_{L0} block sums, levels L0+1..L, no base
typedef PlanePlan<64, 64, 2, 1, 5, 256, 2, 2> CP_64_L2_k5;
typedef PlanePlan<16, 16, 2, 1, 3, 64, 1, 1> CP_16_L2_k3;
typedef PlanePlan<32, 32, 1, 1, 5, 256, 1, 1> CP_32_L1_k5;
// fine-pass plans
typedef TilePlan<256, 256, 2, 4, 7, 5, 16, 256, 1, 4> FP_256_L2of4_k75;
typedef TilePlan<64, 64, 2, 4, 3, 3, 8, 128, 1, 1> FP_64_L2of4_k33;
typedef TilePlan<64, 64, 1, 2, 5, 5, 16, 128, 1, 2> FP_64_L1of2_k55;

#define WTC_SPLIT_ENTRY(FPL, CPL)                                                              \
    {FPL::H, FPL::W, FPL::LT, FPL::KB, FPL::K, FPL::L0,                                       \
     {{launch_split<FPL, CPL, float, false>, launch_split<FPL, CPL, float, true>},            \
      {launch_split<FPL, CPL, bf16_t, false>, launch_split<FPL, CPL, bf16_t, true>}},         \
     split_ws<FPL>}

static const SplitEntry kSplitEntries[] = {
    WTC_SPLIT_ENTRY(FP_256_L2of4_k75, CP_64_L2_k5),
    WTC_SPLIT_ENTRY(FP_64_L2of4_k33, CP_16_L2_k3),
    WTC_SPLIT_ENTRY(FP_64_L1of2_k55, CP_32_L1_k5),
};

const SplitEntry* find_split_entry(int H, int W, int L, int KB, int K) {
    for (const SplitEntry& e : kSplitEntries)
        if (e.H == H && e.W == W && e.L == L && e.KB == KB && e.K == K) return &e;
    return nullptr;
}

}  // namespace wtc
