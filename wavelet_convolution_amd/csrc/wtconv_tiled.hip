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
template <int H_, int W_, int L0_, int LT_, int KB_, int K_, int TH_, int NT_, int RB_, int RL_, int WMAX_ = 4,
          bool MF_ = false>
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
    // Base convolution on the matrix cores (bf16 activations; see P1 of
    // coltile_kernel). The x rows the base convolution reads stay in their
    // bf16 form, x column c at row position XOM + c, rows SXB apart (a
    // multiple of 8 elements: 16-byte operand reads; 4 dwords of stagger per
    // row spreads 8 consecutive rows over all banks), in region A, which is
    // then sized for them rather than for fp32 rows. The banded tap rows
    // follow the taps, as 32-bit words of overlapping entry pairs (word w =
    // entries w and w + 1; ZL words per row, three bf16 parts of each tap):
    // a lane's 8 entries from any e are the words e, e+2, e+4, e+6.
    // Half of the wavefronts run the matrix products while the other half
    // runs the level-1 convolution (MFW blocks per matrix wavefront).
    static constexpr bool MF = MF_;
    static constexpr int XOM = 4, SXB = W + 24, ZL = 48, ZOFF = 15 + (XOM - PB);
    static constexpr int ZFLOATS = 3 * KB * ZL;
    static constexpr int NW = NT / 64, MFW = MF ? (TH / 16) * (W / 16) / (NW / 2) : 1;
    template <typename T>
    static constexpr bool mf() { return MF && sizeof(T) == 2; }
    static constexpr int XSIZE_MF = (XROWS * SXB / 2 + 3) / 4 * 4;
    template <typename T>
    static constexpr int asize() { return mf<T>() ? (XSIZE_MF > UDEEP ? XSIZE_MF : UDEEP) : ASIZE; }
    // floats of LDS per workgroup: regions A and B, the taps, the banded taps
    // words of a channel's tap image: what the kernel keeps in LDS from its
    // base taps on (base taps, level taps, banded rows in the matrix-core form)
    template <typename T>
    static constexpr int tapw() { return WFLOATS + (mf<T>() ? ZFLOATS : 0); }
    template <typename T>
    static constexpr int lds_floats() {
        return (asize<T>() + BSIZE + 3) / 4 * 4 + tapw<T>();
    }
    static_assert(!MF || (TH % 16 == 0 && W % 16 == 0 && PB <= XOM && PB + XOM <= 16 && SXB % 8 == 0 &&
                          ZOFF + KB <= ZL && NW % 2 == 0 && ((TH / 16) * (W / 16)) % (NW / 2) == 0),
                  "matrix-core base convolution: 16 x 16 output blocks, whole blocks per wavefront");
    static_assert(lds_floats<float>() * 4 <= 160 * 1024 && lds_floats<bf16_t>() * 4 <= 160 * 1024,
                  "tile does not fit in LDS");
    static constexpr int LPB = strip_lanes(W);
    static constexpr int NIB = (TH / RB) * LPB;
    static constexpr int MB = cdiv(NIB, NT);
    static constexpr int lpl(int l) { return strip_lanes(W >> l); }
    static constexpr int nil(int l) { return 4 * (hout(l) / rl(l)) * lpl(l); }
    // threads of the level convolutions: all of them, or (matrix-core form)
    // the upper half for level 1 and the lower half for level 2
    static constexpr int lvl_t0(int l, bool mf) { return mf && l == 1 ? NT / 2 : 0; }
    static constexpr int lvl_nt(int l, bool mf) { return mf ? NT / 2 : NT; }
    static constexpr int IPR = ((W >> 1) + 2 * PK) / CPI;
    static constexpr int NQ = rh(1) * IPR;
    static constexpr int NTILE = H / TH;
    // occupancy the LDS footprint allows, at most WMAX waves per SIMD
    template <typename T>
    static constexpr int waves_per_eu() {
        const int wg = (160 * 1024) / (lds_floats<T>() * 4), w = (wg * (NT / 64)) / 4;
        return w < 1 ? 1 : (w > WMAX_ ? WMAX_ : w);
    }

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

// A channel's tap image for coltile_kernel, the words that kernel keeps in
// LDS from its base taps on: base taps (turned 180 degrees for the backward
// data pass), level taps with the band scale and 4^-l folded in, and in the
// matrix-core form the banded tap rows. Every tile of every plane of a
// channel reads the same image, so it is built once per call, a workgroup
// per channel, and the fine kernel copies it in with one 16-byte load per
// lane instead of rebuilding it per tile.
template <class P, typename T, bool FLIP>
__global__ __launch_bounds__(256) void coltile_taps_kernel(const float* __restrict__ w_base,
                                                           const float* __restrict__ w_lvl,
                                                           const float* __restrict__ scale, float* __restrict__ taps,
                                                           int C) {
    constexpr int KB = P::KB, K = P::K, L0 = P::L0, KB2P = P::KB2P, K2P = P::K2P, NT = 256;
    const int c = blockIdx.x, tid = threadIdx.x;
    float* const WB = taps + (size_t)c * P::template tapw<T>();
    float* const WL = WB + KB2P;
    for (int t = tid; t < KB2P; t += NT)
        WB[t] = t < KB * KB ? w_base[(size_t)c * KB * KB + (FLIP ? KB * KB - 1 - t : t)] : 0.f;
    for (int t = tid; t < 4 * L0 * K2P; t += NT) {
        const int ls = t / K2P, tap = t - ls * K2P, l = ls >> 2, s = ls & 3;
        const size_t pi = ((size_t)l * C + c) * 4 + s;
        const float f = scale[pi] * (1.0f / (float)(1 << (2 * (l + 1))));
        WL[t] = tap < K * K ? w_lvl[pi * K * K + (FLIP ? K * K - 1 - tap : tap)] * f : 0.f;
    }
    if constexpr (P::template mf<T>()) {
        // Banded tap rows: entry e of row (part p, tap row i) is part p of
        // tap (i, e - ZOFF), zero outside the row, stored as words of entry
        // pairs (e, e + 1). The three parts are the bf16 rounding of the tap,
        // of what that leaves, and of what remains then: their sum is the
        // fp32 tap exactly, and each product with a bf16 x is exact in fp32.
        constexpr int ZL = P::ZL;
        uint32_t* const zw = reinterpret_cast<uint32_t*>(WL + 4 * L0 * K2P);
        for (int t = tid; t < KB * ZL; t += NT) {
            const int i = t / ZL, w = t - i * ZL;
            bf16_t part[2][3];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int j = w + h - P::ZOFF;
                float v = 0.f;
                if (j >= 0 && j < KB) {
                    const int tap = i * KB + j;
                    v = w_base[(size_t)c * KB * KB + (FLIP ? KB * KB - 1 - tap : tap)];
                }
                part[h][0] = narrow_bf16(v);
                v -= widen(part[h][0]);
                part[h][1] = narrow_bf16(v);
                part[h][2] = narrow_bf16(v - widen(part[h][1]));
            }
#pragma unroll
            for (int pt = 0; pt < 3; ++pt) zw[(pt * KB + i) * ZL + w] = (uint32_t)part[0][pt] | ((uint32_t)part[1][pt] << 16);
        }
    }
}

template <class P, typename T, bool FLIP>
__global__ __launch_bounds__(P::NT) __attribute__((amdgpu_waves_per_eu(P::template waves_per_eu<T>())))
void coltile_kernel(const T* __restrict__ in, const float* __restrict__ taps, const float* __restrict__ coarse,
                    T* __restrict__ out, int C) {
    constexpr int H = P::H, W = P::W, L0 = P::L0, KB = P::KB, K = P::K, NT = P::NT, TH = P::TH, RB = P::RB;
    constexpr int PB = P::PB, PK = P::PK, G = P::G, SX = P::SX, XO = P::XO, W1 = W / 2;
    constexpr int S1 = P::su(1), BS1 = P::bandsz(1);
    constexpr int NIB = P::NIB, MB = P::MB, LPB = P::LPB;
    constexpr int KB2P = P::KB2P, K2P = P::K2P;

    // matrix-core base convolution: bf16 activations of a plan that asks for it
    constexpr bool MF = P::template mf<T>();
    constexpr int AS = P::template asize<T>();
    __shared__ __attribute__((aligned(16))) float lds[P::template lds_floats<T>()];
    float* A = lds;               // x rows, later the bands of levels 2..L0
    float* Bq = lds + AS;         // level-1 bands
    float* WB = lds + (AS + P::BSIZE + 3) / 4 * 4;
    float* WL = WB + KB2P;
    uint16_t* const XS = reinterpret_cast<uint16_t*>(A);                        // bf16 x rows (MF)
    uint16_t* const ZC = reinterpret_cast<uint16_t*>(WL + 4 * L0 * K2P);        // banded taps (MF)

    const int tid = threadIdx.x;
    // the wavefront index as a scalar: row indices derived from it (P0's
    // items are a wavefront per row pair on 256-wide planes) stay uniform
    const int wvu = __builtin_amdgcn_readfirstlane(tid >> 6), lane_ = tid & 63;
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
    // The channel's tap image (coltile_taps_kernel), loaded first and stored
    // to LDS once the x loads are in flight.
    constexpr int TW4 = P::template tapw<T>() / 4, MT = cdiv(TW4, NT);
    static_assert(P::template tapw<T>() % 4 == 0, "tap image of whole 16-byte words");
    const uint4* __restrict__ timg = reinterpret_cast<const uint4*>(taps) + (size_t)c * TW4;
    uint4 tv[MT];
#pragma unroll
    for (int k = 0; k < MT; ++k) tv[k] = timg[min(tid + k * NT, TW4 - 1)];
    // The coarse image's values under this thread's output strips (what the
    // levels above L0 add, constant on 2^L0 blocks): loaded with the x rows,
    // used by the synthesis at the end.
    constexpr int CW = W >> L0, NSTRIP = MF ? P::MFW : P::MB, RSTRIP = MF ? 4 : RB;
    // (a plan with no levels above L0 has no coarse image: zeros)
    const float* __restrict__ ctile = P::LT > L0 ? coarse + ((size_t)plane * (H >> L0) + (r0 >> L0)) * CW : nullptr;
    float cpre[NSTRIP][RSTRIP >> L0];
    {
        // Border columns, written once: the x rows' columns outside the
        // plane and the level-1 bands' zero border columns (nothing else
        // writes them). Then the interior: an item owns region rows 2i, 2i+1
        // and four columns from 4u (band cells 2u, 2u+1 of band row i); rows
        // outside the plane load nothing and store zeros (the zero padding of
        // every level's band grid).
        // (bf16 x rows: border columns written as 32-bit words, pairs of entries)
        constexpr int XB = MF ? (P::SXB - W) / 2 : SX - W, XB1 = S1 - W1;
        static_assert(XB > 0 && XB1 > 0 && XO + W <= SX, "border columns");
        static_assert(!MF || (P::XOM % 2 == 0 && (P::SXB - W) % 2 == 0), "bf16 border pairs");
        for (int i = tid; i < P::XROWS * XB + 4 * P::rh(1) * XB1; i += NT) {
            if (i < P::XROWS * XB) {
                const int r = udiv(i, XB), q = i - r * XB;
                if constexpr (MF)
                    reinterpret_cast<uint32_t*>(XS)[(r * P::SXB + (2 * q < P::XOM ? 2 * q : 2 * q + W)) / 2] = 0u;
                else
                    A[r * SX + (q < XO ? q : q + W)] = 0.f;
            } else {
                const int j = i - P::XROWS * XB, rb = udiv(j, XB1), q = j - rb * XB1;   // rb = band * rh(1) + row
                Bq[rb * S1 + (q < PK ? q : q + W1)] = 0.f;
            }
        }
        constexpr int QW = W / 4, NQI = P::rh(1) * QW, MQ = cdiv(NQI, NT);
        static_assert(W % 4 == 0 && PK % 2 == 0 && S1 % 2 == 0, "aligned 4-column items and band pairs");
        const int rtop = r0 - G;   // plane row of region row 0 (negative on the first tile)
        RawVec<T, 4> v0[MQ], v1[MQ];
#pragma unroll
        for (int k = 0; k < MQ; ++k) {
            const int q = tid + k * NT;
            const int ii = QW == 64 ? wvu + k * (NT / 64) : udiv(q, QW), uu = QW == 64 ? lane_ : q - ii * QW;
            const int pr = rtop + 2 * ii;
            // every lane loads (rows outside the plane: its first words) and
            // then selects zeros: no branch around the loads
            const bool inside = (NQI % NT == 0 || q < NQI) && pr >= 0 && pr < H;
            const T* s0 = src + (inside ? (uint32_t)(pr * W + 4 * uu) : 0u);
            load_raw<T, 4>(s0, v0[k]);
            load_raw<T, 4>(s0 + (inside ? W : 0), v1[k]);
#pragma unroll
            for (int e = 0; e < RawVec<T, 4>::N; ++e) {
                v0[k].w[e] = inside ? v0[k].w[e] : 0u;
                v1[k].w[e] = inside ? v1[k].w[e] : 0u;
            }
        }
        {
            const int lane = lane_, wv = wvu;
            auto cload = [&](int s, int h0, int w) {
#pragma unroll
                for (int p = 0; p < (RSTRIP >> L0); ++p)
                    cpre[s][p] = P::LT > L0 ? ctile[(uint32_t)(((h0 >> L0) + p) * CW + (w >> L0))] : 0.f;
            };
            if constexpr (MF) {
                if (wv < P::NW / 2) {
#pragma unroll
                    for (int bb = 0; bb < NSTRIP; ++bb) {
                        const int blk = wv + bb * (P::NW / 2), rbk = blk / (W / 16), cbk = blk - rbk * (W / 16);
                        cload(bb, 16 * rbk + 4 * (lane >> 4), 16 * cbk + (lane & 15));
                    }
                }
            } else {
#pragma unroll
                for (int it = 0; it < NSTRIP; ++it) {
                    const int item = min(tid + it * NT, NIB - 1), rb = item / LPB, w = min(item - rb * LPB, W - 1);
                    cload(it, rb * RB, w);
                }
            }
        }
#pragma unroll
        for (int k = 0; k < MT; ++k)
            if (TW4 % NT == 0 || tid + k * NT < TW4) reinterpret_cast<uint4*>(WB)[tid + k * NT] = tv[k];
#pragma unroll
        for (int k = 0; k < MQ; ++k) {
            const int q = tid + k * NT;
            if (!(NQI % NT == 0 || q < NQI)) continue;
            const int ii = QW == 64 ? wvu + k * (NT / 64) : udiv(q, QW), uu = QW == 64 ? lane_ : q - ii * QW;
            float f0[4], f1[4];
            widen_raw<T, 4>(v0[k], f0);
            widen_raw<T, 4>(v1[k], f1);
            const int xr = 2 * ii - P::XR0;   // kept x rows: those the base convolution reads
            if constexpr (MF) {
                // as loaded: four bf16 per row, one 64-bit store
                uint2* const xo = reinterpret_cast<uint2*>(XS + xr * P::SXB + P::XOM + 4 * uu);
                if (xr >= 0 && xr < P::XROWS) *xo = make_uint2(v0[k].w[0], v0[k].w[1]);
                if (xr + 1 >= 0 && xr + 1 < P::XROWS)
                    *reinterpret_cast<uint2*>(XS + (xr + 1) * P::SXB + P::XOM + 4 * uu) = make_uint2(v1[k].w[0], v1[k].w[1]);
            } else {
                float* const xo = A + xr * SX + XO + 4 * uu;
                if (xr >= 0 && xr < P::XROWS) store_vec<4>(xo, f0);
                if (xr + 1 >= 0 && xr + 1 < P::XROWS) store_vec<4>(xo + SX, f1);
            }
            float b[4][2];
#pragma unroll
            for (int m = 0; m < 2; ++m)
                haar4(f0[2 * m], f0[2 * m + 1], f1[2 * m], f1[2 * m + 1], b[0][m], b[1][m], b[2][m], b[3][m]);
            float* const o = Bq + ii * S1 + PK + 2 * uu;
#pragma unroll
            for (int s = 0; s < 4; ++s) store_vec<2>(o + s * BS1, b[s]);
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- P1
    // matrix-core form: 16 x 16 output blocks, MFW on each of the lower half
    // of the wavefronts; the upper half convolves level 1 meanwhile
    constexpr int NWV = NT / 64, NBC = W / 16, NBW = P::MFW;
    const int lane = lane_, wv = wvu, mn = lane & 15, mq = lane >> 4;
    float yb[MF ? NBW : MB][MF ? 4 : RB];
    // level convolutions: strips of rl(l) output rows x 1 column of one band,
    // on threads lvl_t0 .. lvl_t0 + lvl_nt
    auto level_items = [&](auto lc, auto&& f) {
        constexpr int l = decltype(lc)::value;
        constexpr int wl = W >> l, R = P::rl(l), NS = P::hout(l) / R, LP = P::lpl(l), NIl = P::nil(l);
        constexpr int T0 = P::lvl_t0(l, MF), TN = P::lvl_nt(l, MF);
        if constexpr (LP % 64 == 0 && TN % 64 == 0 && T0 % 64 == 0 && NIl % TN == 0) {
            // a wavefront's 64 items share band and strip row: those stay
            // scalar, the column is the lane's
            if (wvu < T0 / 64 || wvu >= (T0 + TN) / 64) return;
#pragma unroll
            for (int it = 0; it < NIl / TN; ++it) {
                const int wb = (wvu - T0 / 64) * 64 + it * TN;
                const int s = wb / (NS * LP), rem = wb - s * (NS * LP);
                const int rs = rem / LP, j = rem - rs * LP + lane_;
                if (LP == wl || j < wl) f(it, s, (G >> l) + rs * R, j);
            }
        } else {
            const int lt = tid - T0;
            if (lt < 0 || lt >= TN) return;
#pragma unroll
            for (int it = 0; it < cdiv(NIl, TN); ++it) {
                const int item = lt + it * TN;
                if (NIl % TN == 0 || item < NIl) {
                    const int s = item / (NS * LP), rem = item - s * (NS * LP);
                    const int rs = rem / LP, j = rem - rs * LP;
                    if (LP == wl || j < wl) f(it, s, (G >> l) + rs * R, j);
                }
            }
        }
    };
    // Matrix-core form on a band of whole 64-lane pairs of columns: a level-1
    // item is two adjacent output columns of one band (conv_tile with two
    // columns reads each window row once for both: half the LDS reads of two
    // one-column strips), one item per upper-half thread, the band scalar.
    constexpr bool L1P = MF && (W1 / 2) % 64 == 0 && 4 * (W1 / 2) == NT / 2 && P::hout(1) == P::rl(1);
    float z1[cdiv(P::nil(1), P::lvl_nt(1, MF))][P::rl(1)];   // (unused with L1P)
    float z1p[L1P ? P::rl(1) : 1][2];
    const int p_s = wvu - NT / 128, p_j = 2 * lane_;   // band, first column (upper half, L1P)
    auto level1_conv = [&]() {
        level_items(std::integral_constant<int, 1>{}, [&](int it, int s, int row, int j) {
            conv_col<K, P::rl(1), S1>(Bq + s * BS1 + (row - PK) * S1 + j, WL + s * K2P, z1[it]);
        });
    };
    if constexpr (MF) {
        if (wv < NWV / 2) {
            // Output block (h0, w0): y[h0+m][w0+n] = sum over tap rows i and
            // tap parts of sum_k X_i[m][k] T_i[k][n], with X_i[m][k] =
            // x[h0+m+i-PB][w0-XOM+k] (32 consecutive x columns of one row) and
            // T_i[k][n] = part of tap (i, k-n-(XOM-PB)) where that lies in the
            // row, else 0: one 16x16x32 bf16 matrix product each, fp32
            // accumulation. Lane l holds X row m = l%16, columns 8(l/16)..+7;
            // T column n = l%16, rows 8(l/16)..+7 (banded-table entries
            // 8(l/16)-n+15..+7); result rows 4(l/16)..+3 of column n.
            typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
            typedef float f32x4 __attribute__((ext_vector_type(4)));
            constexpr int ZL = P::ZL, SXB = P::SXB;
            const int e0 = 8 * mq - mn + 15;
            const uint32_t* const zw = reinterpret_cast<const uint32_t*>(ZC) + e0;
            f32x4 acc[NBW];
#pragma unroll
            for (int bb = 0; bb < NBW; ++bb) acc[bb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int i = 0; i < KB; ++i) {
                bf16x8 tb[3];
#pragma unroll
                for (int part = 0; part < 3; ++part) {
                    const uint32_t* zp = zw + (part * KB + i) * ZL;
                    tb[part] = __builtin_bit_cast(bf16x8, make_uint4(zp[0], zp[2], zp[4], zp[6]));
                }
#pragma unroll
                for (int bb = 0; bb < NBW; ++bb) {
                    const int blk = wv + bb * (NWV / 2), rbk = blk / NBC, cbk = blk - rbk * NBC;
                    const uint4 xv =
                        *reinterpret_cast<const uint4*>(XS + (16 * rbk + mn + i) * SXB + 16 * cbk + 8 * mq);
                    const bf16x8 xa = __builtin_bit_cast(bf16x8, xv);
#pragma unroll
                    for (int part = 0; part < 3; ++part)
                        acc[bb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(xa, tb[part], acc[bb], 0, 0, 0);
                }
            }
#pragma unroll
            for (int bb = 0; bb < NBW; ++bb)
#pragma unroll
                for (int o = 0; o < 4; ++o) yb[bb][o] = acc[bb][o];
        } else {
            if constexpr (L1P)
                conv_tile<K, P::rl(1), 2, S1>(Bq + p_s * BS1 + ((G >> 1) - PK) * S1 + p_j, WL + p_s * K2P, z1p);
            else
                level1_conv();
        }
    } else {
#pragma unroll
        for (int it = 0; it < MB; ++it) {
            const int item = tid + it * NT;
            if (NIB % NT == 0 || item < NIB) {
                const int rb = item / LPB, w = item - rb * LPB;
                if (LPB == W || w < W) conv_col<KB, RB, SX>(A + XO - PB + (rb * RB) * SX + w, WB, yb[it]);
            }
        }
    }
    __syncthreads();   // x is dead: levels 2..L0 go over it

    // ---------------------------------------------------------------- P2
    P::for_deep_levels([&](auto lc) {
        constexpr int l = decltype(lc)::value;
        constexpr int wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), Sp = P::su(l - 1);
        constexpr int UO = P::uoff(l), UP = P::uoff(l - 1), RL = P::rh(l), XBl = Sl - wl;
        static_assert(Sp % 2 == 0 && PK % 2 == 0, "LL pairs read as aligned 64-bit words");
        float* Ul = A + UO;
        const float* LLp = (l == 2) ? (Bq + PK) : (A + UP + PK);
        // border columns, then the interior cells
        for (int i = tid; i < 4 * RL * XBl; i += NT) {
            const int rb = udiv(i, XBl), q = i - rb * XBl;
            Ul[rb * Sl + (q < PK ? q : q + wl)] = 0.f;
        }
        for (int q = tid; q < RL * wl; q += NT) {
            // (64-wide bands: a wavefront per band row, the row a scalar)
            const int i = wl == 64 ? wvu + (q - tid) / 64 : udiv(q, wl), j = wl == 64 ? lane_ : q - i * wl;
            const float2 t = *reinterpret_cast<const float2*>(LLp + 2 * i * Sp + 2 * j);
            const float2 d = *reinterpret_cast<const float2*>(LLp + (2 * i + 1) * Sp + 2 * j);
            float b[4];
            haar4(t.x, t.y, d.x, d.y, b[0], b[1], b[2], b[3]);
            const int o = i * Sl + PK + j;
#pragma unroll
            for (int s = 0; s < 4; ++s) Ul[s * BSl + o] = b[s];
        }
        __syncthreads();
    });

    // ---------------------------------------------------------------- P3
    // every fine level into registers (level 1 already, in the matrix-core
    // form), then written over its own bands
    float z2[L0 >= 2 ? cdiv(P::nil(L0 >= 2 ? 2 : 1), P::lvl_nt(2, MF)) : 1][P::rl(L0 >= 2 ? 2 : 1)];
    static_assert(L0 <= 2, "fine levels: one or two");
    if constexpr (!MF) level1_conv();
    if constexpr (L0 >= 2) {
        constexpr int S2 = P::su(2), BS2 = P::bandsz(2), U2 = P::uoff(2);
        level_items(std::integral_constant<int, 2>{}, [&](int it, int s, int row, int j) {
            conv_col<K, P::rl(2), S2>(A + U2 + s * BS2 + (row - PK) * S2 + j, WL + (4 + s) * K2P, z2[it]);
        });
    }
    __syncthreads();
    if constexpr (L1P) {
        if (wvu >= NT / 128) {
#pragma unroll
            for (int o = 0; o < P::rl(1); ++o)
                *reinterpret_cast<float2*>(Bq + p_s * BS1 + ((G >> 1) + o) * S1 + PK + p_j) =
                    make_float2(z1p[o][0], z1p[o][1]);
        }
    } else {
        level_items(std::integral_constant<int, 1>{}, [&](int it, int s, int row, int j) {
#pragma unroll
            for (int o = 0; o < P::rl(1); ++o) Bq[s * BS1 + (row + o) * S1 + PK + j] = z1[it][o];
        });
    }
    if constexpr (L0 >= 2) {
        constexpr int S2 = P::su(2), BS2 = P::bandsz(2), U2 = P::uoff(2);
        level_items(std::integral_constant<int, 2>{}, [&](int it, int s, int row, int j) {
#pragma unroll
            for (int o = 0; o < P::rl(2); ++o) A[U2 + s * BS2 + (row + o) * S2 + PK + j] = z2[it][o];
        });
    }
    __syncthreads();

    // ---------------------------------------------------------------- P4
    // y = base + closed-form synthesis of the fine levels + the coarse image.
    // Stores and coarse reads use the tile's uniform bases plus 32-bit lane
    // offsets (rows at constant offsets from one address).
    static_assert(RB % 2 == 0, "bf16 rows are narrowed in pairs");
    T* __restrict__ dtile = dst + (size_t)r0 * W;
    // one strip of R output rows from h0 in column w + CO, base results yv,
    // the coarse image's values cv (loaded at the start); CO, a constant
    // multiple of 64, folds into the addresses' immediate offsets
    auto synth_store = [&](auto rc, auto co, const int h0, const int w, const float* yv, const float* cv) {
        constexpr int RS = decltype(rc)::value, CO = decltype(co)::value;
        static_assert(CO % 64 == 0 && L0 <= 6, "column offsets that leave every level's parity alone");
        static_assert(RS % (1 << L0) == 0 && RS % 2 == 0, "strips of whole 2^L0 blocks, rows in pairs");
        // From the coarse image down to level 1, carry[p] is what the
        // coarser levels add to every row of level-l block p; level l splits
        // it into its two half-blocks as carry + a +- b.
        float carry[RS];
#pragma unroll
        for (int p = 0; p < (RS >> L0); ++p) carry[p] = cv[p];
        P::for_levels([&](auto lc) {
            constexpr int l = L0 + 1 - decltype(lc)::value;   // L0, ..., 1
            constexpr int Sl = P::su(l), BSl = P::bandsz(l);
            const float* Zl = ubase(std::integral_constant<int, l>{}) + ((G >> l) + (h0 >> l)) * Sl + PK + (w >> l) + (CO >> l);
            const float sw = ((w >> (l - 1)) & 1) ? -1.f : 1.f;
            float next[RS >> (l - 1)];
#pragma unroll
            for (int p = 0; p < (RS >> l); ++p) {
                const float* z = Zl + p * Sl;
                const float a = __builtin_fmaf(sw, z[2 * BSl], z[0]) + carry[p];
                const float b = __builtin_fmaf(sw, z[3 * BSl], z[BSl]);
                next[2 * p] = a + b;
                next[2 * p + 1] = a - b;
            }
#pragma unroll
            for (int q = 0; q < (RS >> (l - 1)); ++q) carry[q] = next[q];
        });
        T* const out_col = dtile + (uint32_t)(h0 * W + w) + CO;
        if constexpr (sizeof(T) == 2) {
            // two rows per conversion: the low half to row o, the high half to o + 1
#pragma unroll
            for (int o = 0; o < RS; o += 2) {
                uint32_t pr = narrow_bf16x2(yv[o] + carry[o], yv[o + 1] + carry[o + 1]);
                // opaque to the compiler, which would otherwise convert the
                // high half again on its own instead of storing it directly
                asm volatile("" : "+v"(pr));
                out_col[o * W] = (bf16_t)(pr & 0xffffu);
                out_col[(o + 1) * W] = (bf16_t)(pr >> 16);
            }
        } else {
#pragma unroll
            for (int o = 0; o < RS; ++o) out_col[o * W] = yv[o] + carry[o];
        }
    };
    if constexpr (MF) {
        // the matrix-core blocks: rows 4(l/16)..+3 of column l%16 of each block
        if (wv < NWV / 2) {
            if constexpr (TH == 16 && (16 * (NWV / 2)) % 64 == 0) {
                // one row of blocks: block bb sits 16 (NWV / 2) bb columns on
                static_for<NBW>([&](auto bc) {
                    constexpr int bb = decltype(bc)::value;
                    synth_store(std::integral_constant<int, 4>{}, std::integral_constant<int, 16 * (NWV / 2) * bb>{},
                                4 * mq, 16 * wv + mn, yb[bb], cpre[bb]);
                });
            } else {
#pragma unroll
                for (int bb = 0; bb < NBW; ++bb) {
                    const int blk = wv + bb * (NWV / 2), rbk = blk / NBC, cbk = blk - rbk * NBC;
                    synth_store(std::integral_constant<int, 4>{}, std::integral_constant<int, 0>{}, 16 * rbk + 4 * mq,
                                16 * cbk + mn, yb[bb], cpre[bb]);
                }
            }
        }
    } else {
#pragma unroll
        for (int it = 0; it < MB; ++it) {
            const int item = tid + it * NT;
            if (!(NIB % NT == 0 || item < NIB)) continue;
            const int rb = item / LPB, w = item - rb * LPB;
            if (!(LPB == W || w < W)) continue;
            synth_store(std::integral_constant<int, RB>{}, std::integral_constant<int, 0>{}, rb * RB, w, yb[it], cpre[it]);
        }
    }
}

// Workspace of a column-tile plan: the coarse image (fp32 per plane at level
// L0, where levels above L0 exist), then the channels' tap images.
static size_t align_up256(size_t n) { return (n + 255) / 256 * 256; }
template <class FP>
static size_t coarse_bytes(int B, int C) {
    if (FP::LT == FP::L0) return 0;
    return (size_t)B * C * (FP::H >> FP::L0) * (FP::W >> FP::L0) * sizeof(float);
}
template <class FP>
static size_t colsplit_ws(int B, int C) {
    constexpr int TW = FP::template tapw<bf16_t>() > FP::template tapw<float>() ? FP::template tapw<bf16_t>()
                                                                                 : FP::template tapw<float>();
    return align_up256(coarse_bytes<FP>(B, C)) + (size_t)C * TW * sizeof(float);
}
template <class FP>
static float* colsplit_taps(float* ws, int B, int C) {
    return reinterpret_cast<float*>(reinterpret_cast<char*>(ws) + align_up256(coarse_bytes<FP>(B, C)));
}

template <class FP, class CP, typename T, bool FLIP>
static hipError_t launch_colsplit(const void* in, const float* wb, const float* wl, const float* sc, void* out,
                                  float* ws, int B, int C, hipStream_t stream) {
    constexpr int L0 = FP::L0, LT = FP::LT;
    const unsigned planes = (unsigned)B * (unsigned)C;
    float* const taps = colsplit_taps<FP>(ws, B, C);
    hipLaunchKernelGGL((coltile_taps_kernel<FP, T, FLIP>), dim3(C), dim3(256), 0, stream, wb, wl, sc, taps, C);
    float* coarse = nullptr;
    if constexpr (LT > L0) {
        coarse = ws;
        const size_t lvl = (size_t)C * 4 * FP::K * FP::K;
        hipError_t err = launch_coarse<CP, T, FLIP, L0>(in, wl + L0 * lvl, sc + (size_t)L0 * C * 4, coarse, B, C,
                                                        stream);
        if (err != hipSuccess) return err;
    }
    hipLaunchKernelGGL((coltile_kernel<FP, T, FLIP>), dim3(planes * FP::NTILE), dim3(FP::NT), 0, stream,
                       (const T*)in, (const float*)taps, (const float*)coarse, (T*)out, C);
    return hipGetLastError();
}

// Backward data with the coarse pass on given dy block sums (see
// split_sums_fn), then the fine pass as usual.
template <class FP, class CP, typename T, bool COLS>
static hipError_t launch_split_sums(const void* in, const float* sums, const float* wb, const float* wl,
                                    const float* sc, void* out, float* ws, int B, int C, hipStream_t stream,
                                    const FinalizeArgs* fin) {
    constexpr int L0 = FP::L0;
    static_assert(FP::LT > L0, "a coarse pass to feed");
    const unsigned planes = (unsigned)B * (unsigned)C;
    const size_t lvl = (size_t)C * 4 * FP::K * FP::K;
    float* taps = nullptr;
    if constexpr (COLS) {
        taps = colsplit_taps<FP>(ws, B, C);
        hipLaunchKernelGGL((coltile_taps_kernel<FP, T, true>), dim3(C), dim3(256), 0, stream, wb, wl, sc, taps, C);
    }
    hipError_t err = launch_coarse<CP, float, true, L0, true>(sums, wl + L0 * lvl, sc + (size_t)L0 * C * 4, ws, B, C,
                                                             stream, fin);
    if (err != hipSuccess) return err;
    if constexpr (COLS)
        hipLaunchKernelGGL((coltile_kernel<FP, T, true>), dim3(planes * FP::NTILE), dim3(FP::NT), 0, stream,
                           (const T*)in, (const float*)taps, (const float*)ws, (T*)out, C);
    else
        hipLaunchKernelGGL((tile_kernel<FP, T, true>), dim3(planes * FP::NTILE), dim3(FP::NT), 0, stream,
                           (const T*)in, wb, wl, sc, (const float*)ws, (T*)out, C);
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
// fine-pass plans: column-strip tiles of 16 rows on 512 lanes at 256x256
// (measured against 8- and 32-row tiles and 256 lanes); micro-tile fine
// passes for the 64x64 test shapes
typedef ColTilePlan<256, 256, 2, 4, 7, 5, 16, 512, 8, 8, 6, true> CT_256_L2of4_k75;
typedef TilePlan<64, 64, 2, 4, 3, 3, 8, 128, 1, 1> FP_64_L2of4_k33;
typedef TilePlan<64, 64, 1, 2, 5, 5, 16, 128, 1, 2> FP_64_L1of2_k55;

#define WTC_SPLIT_ENTRY(FPL, CPL)                                                              \
    {FPL::H, FPL::W, FPL::LT, FPL::KB, FPL::K, FPL::L0,                                       \
     {{launch_split<FPL, CPL, float, false>, launch_split<FPL, CPL, float, true>},            \
      {launch_split<FPL, CPL, bf16_t, false>, launch_split<FPL, CPL, bf16_t, true>}},         \
     split_ws<FPL>,                                                                           \
     {launch_split_sums<FPL, CPL, float, false>, launch_split_sums<FPL, CPL, bf16_t, false>},  \
     (CPL::LDS_FLOATS + CPL::WFLOATS) * sizeof(float)}

#define WTC_COLSPLIT_ENTRY(FPL, CPL)                                                           \
    {FPL::H, FPL::W, FPL::LT, FPL::KB, FPL::K, FPL::L0,                                       \
     {{launch_colsplit<FPL, CPL, float, false>, launch_colsplit<FPL, CPL, float, true>},      \
      {launch_colsplit<FPL, CPL, bf16_t, false>, launch_colsplit<FPL, CPL, bf16_t, true>}},   \
     colsplit_ws<FPL>,                                                                         \
     {launch_split_sums<FPL, CPL, float, true>, launch_split_sums<FPL, CPL, bf16_t, true>},    \
     (CPL::LDS_FLOATS + CPL::WFLOATS) * sizeof(float)}

static const SplitEntry kSplitEntries[] = {
    WTC_COLSPLIT_ENTRY(CT_256_L2of4_k75, CP_64_L2_k5),
    WTC_SPLIT_ENTRY(FP_64_L2of4_k33, CP_16_L2_k3),
    WTC_SPLIT_ENTRY(FP_64_L1of2_k55, CP_32_L1_k5),
};

const SplitEntry* find_split_entry(int H, int W, int L, int KB, int K) {
    for (const SplitEntry& e : kSplitEntries)
        if (e.H == H && e.W == W && e.L == L && e.KB == KB && e.K == K) return &e;
    return nullptr;
}

}  // namespace wtc
