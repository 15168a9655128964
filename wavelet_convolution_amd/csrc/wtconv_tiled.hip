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

// Column-strip fine pass (the counterpart of tile_kernel with the work split
// of col_kernel): a workgroup owns TH output rows of a plane, full width, and
// the region of TH + 2G rows around them. Lanes take consecutive columns:
// a lane computes RB rows x 1 column of the base convolution and RL rows x 1
// column of one band of each fine level; the level results go through LDS
// and one closed-form pass synthesises every output, adding the coarse
// image. The region's rows are all plane rows (zeros outside the plane), so
// only the band columns carry a zero border.
template <int H_, int W_, int L0_, int LT_, int KB_, int K_, int TH_, int NT_, int RB_, int RL_, int WMAX_ = 4>
struct ColTilePlan {
    static constexpr int H = H_, W = W_, L0 = L0_, LT = LT_, KB = KB_, K = K_, TH = TH_, NT = NT_;
    static constexpr int RB = RB_, RL = RL_;
    static constexpr int PB = KB / 2, PK = K / 2, BLK = 1 << L0;
    static_assert(L0 >= 1 && L0 <= LT, "fine levels 1..L0");
    static_assert(H % (1 << LT) == 0 && W % (1 << LT) == 0, "plane must divide into 2^L blocks");
    static_assert(TH % BLK == 0 && H % TH == 0 && TH % RB == 0 && RB % BLK == 0,
                  "tiles and base strips are whole 2^L0 blocks");
    static constexpr int G0 = PB > (PK << L0) ? PB : (PK << L0);
    static constexpr int G = cdiv(G0, BLK) * BLK;   // halo rows above and below
    static constexpr int RH0 = TH + 2 * G;
    static constexpr int rh(int l) { return RH0 >> l; }
    static constexpr int VL = lds_vec(W);
    static constexpr int XO = round_up(PB, 4);
    static constexpr int SX = round_up(XO + W + PB, 4);
    // x rows kept in LDS: only those the base convolution reads (the level-1
    // analysis of the whole region runs on the loaded registers)
    static constexpr int XR0 = G - PB, XROWS = TH + 2 * PB;
    static constexpr int XSIZE = XROWS * SX;
    static constexpr int VA = VL >= 4 ? 4 : 2, CPI = VA / 2;
    static_assert(VL % 2 == 0 && PK % CPI == 0 && (XO - 2 * PK) % VA == 0 && XO + W + 2 * PK >= SX,
                  "analysis items cover the x rows in whole vectors");
    // output band rows of a tile, rows per level strip, band layout
    static constexpr int hout(int l) { return TH >> l; }
    static constexpr int rl(int l) { return RL < hout(l) ? RL : hout(l); }
    static_assert((W >> L0) >= 32, "level strips of whole half-wavefronts");
    static constexpr int su(int l) { return round_up((W >> l) + 2 * PK, 2); }
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
    static constexpr int LPB = strip_lanes(W);
    static constexpr int NIB = (TH / RB) * LPB;
    static constexpr int MB = cdiv(NIB, NT);
    static constexpr int lpl(int l) { return strip_lanes(W >> l); }
    static constexpr int nil(int l) { return 4 * (hout(l) / rl(l)) * lpl(l); }
    static constexpr int IPR = ((W >> 1) + 2 * PK) / CPI;
    static constexpr int NQ = rh(1) * IPR;
    static constexpr int NTILE = H / TH;
    static constexpr int WG_PER_CU = (160 * 1024) / ((LDS_FLOATS + WFLOATS) * 4);
    static constexpr int WAVES_PER_EU_LDS = (WG_PER_CU * (NT / 64)) / 4;
    static constexpr int WAVES_PER_EU =
        WAVES_PER_EU_LDS < 1 ? 1 : (WAVES_PER_EU_LDS > WMAX_ ? WMAX_ : WAVES_PER_EU_LDS);

    template <class F>
    __device__ static __forceinline__ void for_levels(F&& f) {
        lv_impl(f, std::make_integer_sequence<int, L0>{});
    }
    template <class F, int... I>
    __device__ static __forceinline__ void lv_impl(F& f, std::integer_sequence<int, I...>) {
        (f(std::integral_constant<int, I + 1>{}), ...);
    }
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
void coltile_kernel(const T* __restrict__ in, const float* __restrict__ w_base, const float* __restrict__ w_lvl,
                    const float* __restrict__ scale, const float* __restrict__ coarse, T* __restrict__ out, int C) {
    constexpr int H = P::H, W = P::W, L0 = P::L0, KB = P::KB, K = P::K, NT = P::NT, TH = P::TH, RB = P::RB;
    constexpr int PB = P::PB, PK = P::PK, G = P::G, SX = P::SX, XO = P::XO, W1 = W / 2;
    constexpr int S1 = P::su(1), BS1 = P::bandsz(1);
    constexpr int NIB = P::NIB, MB = P::MB, LPB = P::LPB;
    constexpr int KB2P = P::KB2P, K2P = P::K2P;

    __shared__ __attribute__((aligned(16))) float lds[P::LDS_FLOATS + P::WFLOATS];
    float* A = lds;               // x rows, later the bands of levels 2..L0
    float* Bq = lds + P::ASIZE;   // level-1 bands
    float* WB = lds + P::LDS_FLOATS;
    float* WL = WB + KB2P;

    const int tid = threadIdx.x;
    const int lid = xcd_local_index();
    const int plane = lid / P::NTILE, tile = lid - plane * P::NTILE;
    const int c = plane % C;
    const int r0 = tile * TH;
    const T* __restrict__ src = in + (size_t)plane * H * W;
    T* __restrict__ dst = out + (size_t)plane * H * W;
    auto ubase = [&](auto lc) -> float* {
        constexpr int l = decltype(lc)::value;
        constexpr int off = P::uoff(l);
        if constexpr (l == 1) return Bq;
        else return A + off;
    };

    // ---------------------------------------------------------------- P0
    for (int t = tid; t < KB2P; t += NT)
        WB[t] = t < KB * KB ? w_base[(size_t)c * KB * KB + (FLIP ? KB * KB - 1 - t : t)] : 0.f;
    for (int t = tid; t < 4 * L0 * K2P; t += NT) {
        const int ls = t / K2P, tap = t - ls * K2P, l = ls >> 2, s = ls & 3;
        const size_t pi = ((size_t)l * C + c) * 4 + s;
        const float f = scale[pi] * (1.0f / (float)(1 << (2 * (l + 1))));
        WL[t] = tap < K * K ? w_lvl[pi * K * K + (FLIP ? K * K - 1 - tap : tap)] * f : 0.f;
    }
    {
        // The region's x rows and their level-1 bands in one pass: an item
        // owns region rows 2i, 2i+1 and VA columns from 2*j0 (band cells
        // j0.. of band row i). Items on the column border, or on rows
        // outside the plane, store zeros.
        constexpr int NQ = P::NQ, IPR = P::IPR, CPI = P::CPI, VA = P::VA, MQ = cdiv(NQ, NT);
        RawVec<T, VA> v0[MQ], v1[MQ];
#pragma unroll
        for (int k = 0; k < MQ; ++k) {
            const int q = tid + k * NT;
            const int ii = q / IPR, uu = q - ii * IPR, j0 = uu * CPI - PK, pr = r0 - G + 2 * ii;
            if ((NQ % NT == 0 || q < NQ) && j0 >= 0 && j0 < W1 && pr >= 0 && pr < H) {
                const T* s0 = src + (size_t)pr * W + 2 * j0;
                load_raw<T, VA>(s0, v0[k]);
                load_raw<T, VA>(s0 + W, v1[k]);
            } else {
#pragma unroll
                for (int e = 0; e < RawVec<T, VA>::N; ++e) v0[k].w[e] = v1[k].w[e] = 0u;
            }
        }
#pragma unroll
        for (int k = 0; k < MQ; ++k) {
            const int q = tid + k * NT;
            if (!(NQ % NT == 0 || q < NQ)) continue;
            const int ii = q / IPR, uu = q - ii * IPR, j0 = uu * CPI - PK;
            float f0[VA], f1[VA];
            widen_raw<T, VA>(v0[k], f0);
            widen_raw<T, VA>(v1[k], f1);
            const int xc = XO + 2 * j0, xr = 2 * ii - P::XR0;
            if (xc >= 0 && xc + VA <= SX) {
                if (xr >= 0 && xr < P::XROWS) store_vec<VA>(A + xr * SX + xc, f0);
                if (xr + 1 >= 0 && xr + 1 < P::XROWS) store_vec<VA>(A + (xr + 1) * SX + xc, f1);
            }
            float b[4][CPI];
#pragma unroll
            for (int m = 0; m < CPI; ++m)
                haar4(f0[2 * m], f0[2 * m + 1], f1[2 * m], f1[2 * m + 1], b[0][m], b[1][m], b[2][m], b[3][m]);
            float* o = Bq + ii * S1 + uu * CPI;
#pragma unroll
            for (int s = 0; s < 4; ++s) store_vec<CPI>(o + s * BS1, b[s]);
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- P1
    float yb[MB][RB];
#pragma unroll
    for (int it = 0; it < MB; ++it) {
        const int item = tid + it * NT;
        if (NIB % NT == 0 || item < NIB) {
            const int rb = item / LPB, w = item - rb * LPB;
            if (LPB == W || w < W) conv_col<KB, RB, SX>(A + XO - PB + (rb * RB) * SX + w, WB, yb[it]);
        }
    }
    __syncthreads();   // x is dead: levels 2..L0 go over it

    // ---------------------------------------------------------------- P2
    P::for_deep_levels([&](auto lc) {
        constexpr int l = decltype(lc)::value;
        constexpr int wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), Sp = P::su(l - 1);
        constexpr int UO = P::uoff(l), UP = P::uoff(l - 1);
        float* Ul = A + UO;
        const float* LLp = (l == 2) ? (Bq + PK) : (A + UP + PK);
        constexpr int GW = wl + 2 * PK, GN = P::rh(l) * GW;
        for (int q = tid; q < GN; q += NT) {
            const int i = q / GW, jj = q - i * GW, j = jj - PK;
            float b[4] = {0.f, 0.f, 0.f, 0.f};
            if (j >= 0 && j < wl) {
                const float* x2 = LLp + 2 * i * Sp + 2 * j;
                haar4(x2[0], x2[1], x2[Sp], x2[Sp + 1], b[0], b[1], b[2], b[3]);
            }
            const int o = i * Sl + jj;
#pragma unroll
            for (int s = 0; s < 4; ++s) Ul[s * BSl + o] = b[s];
        }
        __syncthreads();
    });

    // ---------------------------------------------------------------- P3
    // every fine level: strips of rl(l) output rows x 1 column of one band
    auto level_items = [&](auto lc, auto&& f) {
        constexpr int l = decltype(lc)::value;
        constexpr int wl = W >> l, R = P::rl(l), NS = P::hout(l) / R, LP = P::lpl(l), NIl = P::nil(l);
#pragma unroll
        for (int it = 0; it < cdiv(NIl, NT); ++it) {
            const int item = tid + it * NT;
            if (NIl % NT == 0 || item < NIl) {
                const int s = item / (NS * LP), rem = item - s * (NS * LP);
                const int rs = rem / LP, j = rem - rs * LP;
                if (LP == wl || j < wl) f(it, s, (G >> l) + rs * R, j);
            }
        }
    };
    float z1[cdiv(P::nil(1), NT)][P::rl(1)];
    float z2[L0 >= 2 ? cdiv(P::nil(L0 >= 2 ? 2 : 1), NT) : 1][P::rl(L0 >= 2 ? 2 : 1)];
    static_assert(L0 <= 2, "fine levels: one or two");
    level_items(std::integral_constant<int, 1>{}, [&](int it, int s, int row, int j) {
        conv_col<K, P::rl(1), S1>(Bq + s * BS1 + (row - PK) * S1 + j, WL + s * K2P, z1[it]);
    });
    if constexpr (L0 >= 2) {
        constexpr int S2 = P::su(2), BS2 = P::bandsz(2), U2 = P::uoff(2);
        level_items(std::integral_constant<int, 2>{}, [&](int it, int s, int row, int j) {
            conv_col<K, P::rl(2), S2>(A + U2 + s * BS2 + (row - PK) * S2 + j, WL + (4 + s) * K2P, z2[it]);
        });
    }
    __syncthreads();
    level_items(std::integral_constant<int, 1>{}, [&](int it, int s, int row, int j) {
#pragma unroll
        for (int o = 0; o < P::rl(1); ++o) Bq[s * BS1 + (row + o) * S1 + PK + j] = z1[it][o];
    });
    if constexpr (L0 >= 2) {
        constexpr int S2 = P::su(2), BS2 = P::bandsz(2), U2 = P::uoff(2);
        level_items(std::integral_constant<int, 2>{}, [&](int it, int s, int row, int j) {
#pragma unroll
            for (int o = 0; o < P::rl(2); ++o) A[U2 + s * BS2 + (row + o) * S2 + PK + j] = z2[it][o];
        });
    }
    __syncthreads();

    // ---------------------------------------------------------------- P4
    // y = base + closed-form synthesis of the fine levels + the coarse image
    constexpr int CW = W >> L0;
    const float* __restrict__ cpl = coarse ? coarse + (size_t)plane * (H >> L0) * CW : nullptr;
#pragma unroll
    for (int it = 0; it < MB; ++it) {
        const int item = tid + it * NT;
        if (!(NIB % NT == 0 || item < NIB)) continue;
        const int rb = item / LPB, w = item - rb * LPB, h0 = rb * RB;
        if (!(LPB == W || w < W)) continue;
        // From the coarse image down to level 1, carry[p] is what the
        // coarser levels add to every row of level-l block p; level l splits
        // it into its two half-blocks as carry + a +- b.
        float carry[RB];
#pragma unroll
        for (int p = 0; p < (RB >> L0); ++p)
            carry[p] = cpl ? cpl[(size_t)(((r0 + h0) >> L0) + p) * CW + (w >> L0)] : 0.f;
        P::for_levels([&](auto lc) {
            constexpr int l = L0 + 1 - decltype(lc)::value;   // L0, ..., 1
            constexpr int Sl = P::su(l), BSl = P::bandsz(l);
            const float* Zl = ubase(std::integral_constant<int, l>{}) + ((G >> l) + (h0 >> l)) * Sl + PK + (w >> l);
            const float sw = ((w >> (l - 1)) & 1) ? -1.f : 1.f;
            float next[RB >> (l - 1)];
#pragma unroll
            for (int p = 0; p < (RB >> l); ++p) {
                const float* z = Zl + p * Sl;
                const float a = __builtin_fmaf(sw, z[2 * BSl], z[0]) + carry[p];
                const float b = __builtin_fmaf(sw, z[3 * BSl], z[BSl]);
                next[2 * p] = a + b;
                next[2 * p + 1] = a - b;
            }
#pragma unroll
            for (int q = 0; q < (RB >> (l - 1)); ++q) carry[q] = next[q];
        });
        float y[RB];
#pragma unroll
        for (int o = 0; o < RB; ++o) y[o] = yb[it][o] + carry[o];
        if constexpr (sizeof(T) == 2) {
            // two rows per conversion: the low half to row o, the high half to o + 1
#pragma unroll
            for (int o = 0; o < RB; o += 2) {
                const uint32_t pr = narrow_bf16x2(y[o], y[o + 1]);
                dst[(size_t)(r0 + h0 + o) * W + w] = (bf16_t)(pr & 0xffffu);
                dst[(size_t)(r0 + h0 + o + 1) * W + w] = (bf16_t)(pr >> 16);
            }
        } else {
#pragma unroll
            for (int o = 0; o < RB; ++o) dst[(size_t)(r0 + h0 + o) * W + w] = y[o];
        }
    }
}

template <class FP, class CP, typename T, bool FLIP>
static hipError_t launch_colsplit(const void* in, const float* wb, const float* wl, const float* sc, void* out,
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
    hipLaunchKernelGGL((coltile_kernel<FP, T, FLIP>), dim3(planes * FP::NTILE), dim3(FP::NT), 0, stream,
                       (const T*)in, wb, wl, sc, (const float*)coarse, (T*)out, C);
    return hipGetLastError();
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
#ifndef WTC_COLTILE
#define WTC_COLTILE 1
#endif
typedef TilePlan<256, 256, 2, 4, 7, 5, 16, 256, 1, 4> FP_256_L2of4_k75;
#ifndef WTC_CT256
#define WTC_CT256 16, 512, 8, 8
#endif
typedef ColTilePlan<256, 256, 2, 4, 7, 5, WTC_CT256> CT_256_L2of4_k75;
typedef TilePlan<64, 64, 2, 4, 3, 3, 8, 128, 1, 1> FP_64_L2of4_k33;
typedef TilePlan<64, 64, 1, 2, 5, 5, 16, 128, 1, 2> FP_64_L1of2_k55;

#define WTC_SPLIT_ENTRY(FPL, CPL)                                                              \
    {FPL::H, FPL::W, FPL::LT, FPL::KB, FPL::K, FPL::L0,                                       \
     {{launch_split<FPL, CPL, float, false>, launch_split<FPL, CPL, float, true>},            \
      {launch_split<FPL, CPL, bf16_t, false>, launch_split<FPL, CPL, bf16_t, true>}},         \
     split_ws<FPL>}

#define WTC_COLSPLIT_ENTRY(FPL, CPL)                                                           \
    {FPL::H, FPL::W, FPL::LT, FPL::KB, FPL::K, FPL::L0,                                       \
     {{launch_colsplit<FPL, CPL, float, false>, launch_colsplit<FPL, CPL, float, true>},      \
      {launch_colsplit<FPL, CPL, bf16_t, false>, launch_colsplit<FPL, CPL, bf16_t, true>}},   \
     split_ws<FPL>}

static const SplitEntry kSplitEntries[] = {
#if WTC_COLTILE
    WTC_COLSPLIT_ENTRY(CT_256_L2of4_k75, CP_64_L2_k5),
#else
    WTC_SPLIT_ENTRY(FP_256_L2of4_k75, CP_64_L2_k5),
#endif
    WTC_SPLIT_ENTRY(FP_64_L2of4_k33, CP_16_L2_k3),
    WTC_SPLIT_ENTRY(FP_64_L1of2_k55, CP_32_L1_k5),
};

const SplitEntry* find_split_entry(int H, int W, int L, int KB, int K) {
    for (const SplitEntry& e : kSplitEntries)
        if (e.H == H && e.W == W && e.L == L && e.KB == KB && e.K == K) return &e;
    return nullptr;
}

}  // namespace wtc
