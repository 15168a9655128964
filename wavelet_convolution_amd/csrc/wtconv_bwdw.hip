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
#include "wtconv_dw.h"
#include "wtconv_plans.h"

namespace wtc {

// acc[m*K+n] += sum_{o<R} v[o*SV] * u[(o+m)*SU + n]: tap sums of an R x 1
// column strip of dy-side values against its window of x-side values. Lanes
// of a wavefront take consecutive columns: every load is a run of
// consecutive LDS words across the wavefront, free of bank conflicts.
template <int K, int R, int SU, int SV, int NA, typename VT, int OFF = 0>
__device__ __forceinline__ void taps_col(const float* u, const VT* v, float (&acc)[NA]) {
    static_assert(OFF + K * K <= NA, "accumulator slot too small");
    constexpr int NR = R + K - 1;   // window rows
    __builtin_amdgcn_sched_barrier(0);
    float vt[R];
#pragma unroll
    for (int o = 0; o < R; ++o) vt[o] = widen(v[o * SV]);
    // window rows double-buffered: row r + 1 is requested before row r's
    // multiply-adds, so its LDS latency hides behind them (requesting two to
    // five rows ahead measured no faster)
    const RowAddr<SU, NR> rows(u);
    float win[2][K];
    {
        const lds_cfp r0 = rows.row(0);
#pragma unroll
        for (int n = 0; n < K; ++n) win[0][n] = r0[n];
    }
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (r + 1 < NR) {
            const lds_cfp rn = rows.row(r + 1);
#pragma unroll
            for (int n = 0; n < K; ++n) win[(r + 1) & 1][n] = rn[n];
        }
#pragma unroll
        for (int o = 0; o < R; ++o) {
            const int m = r - o;
            if (m < 0 || m >= K) continue;
#pragma unroll
            for (int n = 0; n < K; ++n)
                acc[OFF + m * K + n] = __builtin_fmaf(vt[o], win[r & 1][n], acc[OFF + m * K + n]);
        }
    }
    pin_regs(acc);
    __builtin_amdgcn_sched_barrier(0);
}

// Rows per column strip for an h x w grid on `lanes` lanes with k x k taps
// (strip_lanes(w) lanes per row block): the fewest cycles on the busiest lane, counting each strip's R*k*k
// multiply-adds plus its (R+k-1)*k + R LDS reads at two multiply-adds each
// (a CU issues one wavefront multiply-add per clock across its four SIMDs
// but moves only half a wavefront's worth of LDS words per clock).
constexpr int pick_rows(int h, int w, int lanes, int k, int npb = 1) {
    int best = 1, best_cost = 1 << 30;
    for (int r = 1; r <= 16 && r <= h; ++r) {
        if (h % r != 0) continue;
        const int cost = cdiv(npb * (h / r) * strip_lanes(w), lanes) * (r * k * k + 2 * ((r + k - 1) * k + r));
        if (cost < best_cost) {
            best = r;
            best_cost = cost;
        }
    }
    return best;
}

// Lane i takes lane i+1's value (the last lane takes 0): a DPP wave shift.
__device__ __forceinline__ float shl1(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), 0x130, 0xf, 0xf, true));
}

// Column-pair tap sums: acc[m*K+n] += sum_o v0[o] * u[o+m][n] + v1[o] * u[o+m][n+1]
// for a strip of R rows x 2 columns (the lane's dy pair v0, v1 per row).
// Each lane loads one aligned 64-bit pair per window row; the K-1 columns
// to its right come from the next (K-1)/2 lanes through DPP wave shifts, so
// a row block of w columns takes w/2 + (K-1)/2 lanes (the last ones only
// feed their neighbours: pass live = false and their dy counts as zero).
// Every lane of the wavefront must execute the call (no divergence): the
// shifts read the neighbours' registers.
template <int K, int R, int SU, int SV, int NA, typename VT>
__device__ __forceinline__ void taps_pair(const float* u, const VT* v, bool live, float (&acc)[NA]) {
    static_assert(NA >= K * K && K % 2 == 1, "accumulator slot too small / odd kernels only");
    constexpr int NR = R + K - 1, NS = (K - 1) / 2;
    __builtin_amdgcn_sched_barrier(0);
    float v0[R], v1[R];
#pragma unroll
    for (int o = 0; o < R; ++o) {
        float2 q;
        if constexpr (sizeof(VT) == 2) {   // a bf16 pair in one 32-bit word
            const uint32_t w2 = *reinterpret_cast<const uint32_t*>(v + o * SV);
            q = make_float2(__uint_as_float(w2 << 16), __uint_as_float(w2 & 0xffff0000u));
        } else {
            q = *reinterpret_cast<const float2*>(v + o * SV);
        }
        v0[o] = live ? q.x : 0.f;
        v1[o] = live ? q.y : 0.f;
    }
    float2 row[2];
    row[0] = *reinterpret_cast<const float2*>(u);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
        if (r + 1 < NR) row[(r + 1) & 1] = *reinterpret_cast<const float2*>(u + (r + 1) * SU);
        float w[K + 1];
        w[0] = row[r & 1].x;
        w[1] = row[r & 1].y;
#pragma unroll
        for (int q = 1; q <= NS; ++q) {
            w[2 * q] = shl1(w[2 * q - 2]);
            w[2 * q + 1] = shl1(w[2 * q - 1]);
        }
#pragma unroll
        for (int o = 0; o < R; ++o) {
            const int m = r - o;
            if (m < 0 || m >= K) continue;
#pragma unroll
            for (int n = 0; n < K; ++n) {
                acc[m * K + n] = __builtin_fmaf(v0[o], w[n], acc[m * K + n]);
                acc[m * K + n] = __builtin_fmaf(v1[o], w[n + 1], acc[m * K + n]);
            }
        }
    }
    pin_regs(acc);
    __builtin_amdgcn_sched_barrier(0);
}

// Lanes per row block of column-pair strips over w columns with k x k taps.
constexpr int pair_lanes(int w, int k) { return strip_lanes(w / 2 + (k - 1) / 2); }

// Rows per column-pair strip: as pick_rows, counting the DPP shifts and
// the pair loads.
constexpr int pick_rows2(int h, int w, int lanes, int k, int npb = 1) {
    int best = 1, best_cost = 1 << 30;
    for (int r = 1; r <= 16 && r <= h; ++r) {
        if (h % r != 0) continue;
        const int per = 2 * r * k * k + (r + k - 1) * (k - 1) + 2 * (2 * (r + k - 1) + 2 * r);
        const int cost = cdiv(npb * (h / r) * pair_lanes(w, k), lanes) * per;
        if (cost < best_cost) {
            best = r;
            best_cost = cost;
        }
    }
    return best;
}

// One butterfly stage across lanes: the pair (lane, lane ^ mask) holding
// (a, b) ends with a + b on the first lane and a - b on the second.
__device__ __forceinline__ float haar_pair(float own, int mask, bool second) {
    const float p = __shfl_xor(own, mask, 64);
    return second ? p - own : own + p;
}

// Sum over each 16-lane row of the wavefront, in a fixed order: DPP row
// rotations on the vector ALU (no LDS traffic); every lane of a row ends
// with its row's sum.
template <int N>
__device__ __forceinline__ float ror_row(float v) {
    return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + N, 0xf, 0xf, true));
}
__device__ __forceinline__ float row_sum(float v) {
    v += ror_row<8>(v);
    v += ror_row<4>(v);
    v += ror_row<2>(v);
    v += ror_row<1>(v);
    return v;
}

// Sum over the wavefront (row sums, then the four rows), valid in every lane.
__device__ __forceinline__ float wave_sum(float v) {
    v = row_sum(v);
    const int b = __builtin_bit_cast(int, v);
    const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 0));
    const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 16));
    const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 32));
    const float r3 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(b, 48));
    return (r0 + r1) + (r2 + r3);
}

// H x W plane, L >= 1 levels; base strips of RB rows.
// LDS: x (border KB/2), dy, the bordered x bands U_1..U_L (border K/2) and
// the unbordered dy bands V_1..V_L all stay resident.
//
// Work split, 8 wavefronts in two groups of four; wavefront w owns band
// s = w % 4 and keeps its tap sums for the whole chunk in registers:
//   group A (w < 4): a quarter of the base taps (slot 0), levels 3, 5 (slots 1, 2)
//   group B (w >= 4): level 1 (slot 0), levels 2, 4 (slots 1, 2)
// which balances the multiply-adds (level 1 alone equals the base work) and
// keeps every lane at about two or three slots of taps.
template <int H_, int W_, int L_, int KB_, int K_, int LT_ = L_, int NPB_ = 1>
struct BwPlan {
    static constexpr int H = H_, W = W_, L = L_, KB = KB_, K = K_;
    // LT > L: levels L+1..LT of the layer go to a coarse pass, which gets
    // the planes of level-L LL sums of x and dy from this one
    static constexpr int LT = LT_;
    // planes per step: NPB planes of the chunk share each barrier interval
    static constexpr int NPB = NPB_;
    // a coarse plan (1x1 "base", only level taps): no x or dy plane in LDS;
    // its input planes were just written (L2 hits), so a step's loads are
    // issued at the step's start rather than a step ahead (fewer registers)
    static constexpr bool COARSE = KB == 1;
    static constexpr bool PREFETCH = !COARSE;
    static constexpr int NT = 512, NW = 8;
    static constexpr int PB = KB / 2, PK = K / 2;
    static_assert(L >= 1 && L <= 5 && H % (1 << L) == 0 && W % (1 << L) == 0, "plane must divide into 2^L blocks");
    // Column-pair strips (windows shared through DPP shifts) pay where the
    // one-column strips read more than a third of an LDS word per
    // multiply-add, and the pair strips keep 3/4 of their lanes busy.
    static constexpr bool pair_worth(int h, int w, int k, int lanes) {
        const int r = pick_rows(h, w, lanes, k, NPB);
        return w % 2 == 0 && w / 2 + (k - 1) / 2 <= 64 && 4 * (w / 2) >= 3 * pair_lanes(w, k) &&
               3 * ((r + k - 1) * k + r) > r * k * k;
    }
    static constexpr bool BASE_PAIR = PB % 2 == 0 && pair_worth(H, W, KB, 256);
    static constexpr bool level_pair(int l) { return pair_worth(H >> l, W >> l, K, 64); }
    // x rows: interior from column XO (a multiple of 4, at least KB/2), row
    // stride a multiple of 4, so that streamed rows take aligned 128-bit
    // stores and 2x2 blocks aligned 64-bit reads; dy rows likewise
    static constexpr int VL = lds_vec(W);
    static constexpr int XO = round_up(PB, 4);
    static constexpr int SX = round_up(XO + W + PB, 4);
    static constexpr int XSIZE = COARSE ? 0 : (H + 2 * PB) * SX;
    static constexpr int SD = round_up(W, 4);
    static constexpr int DSIZE = COARSE ? 0 : H * SD;
    // band rows: even strides where column pairs are read (8-byte aligned
    // pairs), odd ones elsewhere (the analysis stores of lanes on
    // consecutive rows then fall into different banks)
    static constexpr int su(int l) {
        return level_pair(l) ? round_up((W >> l) + 2 * PK, 2) : odd_stride((W >> l) + 2 * PK);
    }
    static constexpr int bandsz(int l) { return ((H >> l) + 2 * PK) * su(l); }
    static constexpr int sv(int l) { return level_pair(l) ? round_up(W >> l, 2) : odd_stride(W >> l); }
    static constexpr int vsz(int l) { return (H >> l) * sv(l); }
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
    // Column-pair strips (DPP-shared windows) where a grid is wide and even:
    // the base when its window starts on an even column, and each level
    // whose pair strips keep at least 3/4 of a wavefront's lanes busy.
    // role slots: group A = base, 3, 5; group B = 1, 2, 4; in a coarse
    // plan group A = 2, 4 and group B = 1, 3, 5
    static constexpr int NSLOT = COARSE ? (L + 1) / 2 : 1 + (L >= 2 ? 1 : 0) + (L >= 4 ? 1 : 0);
    static constexpr int SLOT0 = KB * KB > K * K ? KB * KB : K * K;   // base or level-1 taps
    static constexpr int RED = 4 * (NW * SLOT0 + NW * (NSLOT - 1) * K * K);   // reduction scratch (4 rows)
    // dy stays in its 16-bit storage format in LDS when the activations are
    // bf16 (only the base taps read it): half the region
    template <typename T>
    static constexpr int dsize() { return sizeof(T) == 2 ? DSIZE / 2 : DSIZE; }
    static constexpr int band_rows(int l) {
        return level_pair(l) ? pick_rows2(H >> l, W >> l, 64, K, NPB) : pick_rows(H >> l, W >> l, 64, K, NPB);
    }
    // Bank conflicts of the level taps of a step at plane pitch ps: the
    // lanes of a pass may hold strips of several planes (narrow bands, NPB
    // planes per step). Cost: over the passes of U and V reads, the largest
    // number of lanes on one bank, summed.
    static constexpr int pitch_conflicts(int ps) {
        int cost = 0;
        for (int l = 1; l <= L; ++l) {
            const int hl = H >> l, wl = W >> l, R = band_rows(l), LP = strip_lanes(wl), NI = (hl / R) * LP;
            if (level_pair(l)) continue;
            for (int pass = 0; pass < 2; ++pass) {
                const int stride = pass == 0 ? su(l) : sv(l);
                for (int h0 = 0; h0 < NPB * NI; h0 += 32) {
                    int cnt[32] = {};
                    int worst = 0;
                    for (int t = h0; t < h0 + 32 && t < NPB * NI; ++t) {
                        const int pl = t / NI, r = t - pl * NI, rs = r / LP, j = r - rs * LP;
                        if (j >= wl) continue;
                        const int b = (pl * ps + rs * R * stride + j) % 32;
                        if (++cnt[b] > worst) worst = cnt[b];
                    }
                    cost += worst;
                }
            }
        }
        return cost;
    }
    // one plane's regions (x, dy, U, V); NPB of them side by side, at the
    // pitch within 32 floats above the minimum with the fewest conflicts (a
    // multiple of 4 where x and dy take 128-bit stores)
    static constexpr int best_pitch(int base) {
        if (NPB == 1) return base;
        const int step = COARSE ? 1 : 4;
        int best = base, best_cost = pitch_conflicts(base);
        for (int ps = base + step; ps < base + 32; ps += step)
            if (pitch_conflicts(ps) < best_cost) {
                best_cost = pitch_conflicts(ps);
                best = ps;
            }
        return best;
    }
    template <typename T>
    static constexpr int pstride() { return best_pitch(round_up(XSIZE + dsize<T>() + UTOT + VTOT, 4)); }
    template <typename T>
    static constexpr int lds_floats() { return NPB * pstride<T>() > RED ? NPB * pstride<T>() : RED; }
    static constexpr int LDS_FLOATS = lds_floats<float>();
    static_assert(LDS_FLOATS * 4 <= 160 * 1024, "plane does not fit in LDS");
    // base strips on group A's 256 lanes: rows, lanes per row block, slots
    static constexpr int RB = BASE_PAIR ? pick_rows2(H, W, 256, KB, NPB) : pick_rows(H, W, 256, KB, NPB);
    static constexpr int LPB = BASE_PAIR ? pair_lanes(W, KB) : strip_lanes(W);
    static constexpr int NI = (H / RB) * LPB;
    static constexpr int TAPS = KB * KB + 4 * L * K * K;
    // Analysis lanes: each owns 2 rows x CW columns of x and dy. The lanes
    // of one 2^L x 2^L block form a group of GS = BR x BC (BR row pairs,
    // BC column slices, row pair fastest) inside one wavefront.
    static constexpr int CW = W % 4 == 0 ? 4 : 2;
    static constexpr int NC = W / CW, NA = (H / 2) * NC;
    static constexpr int BR = L >= 2 ? 1 << (L - 1) : 1;
    static constexpr int BC = L >= 2 ? (CW == 4 ? 1 << (L - 2) : 1 << (L - 1)) : 1;
    static constexpr int GS = BR * BC, NBC = NC / BC;
    static_assert(NPB * NA <= NT, "one analysis lane per 2 x CW block of each plane of a step");
    static_assert(64 % GS == 0, "a block's analysis lanes share a wavefront");
    // Occupancy (waves per SIMD): what LDS allows, and what registers allow
    // at about 48 registers of strips and addresses beside the tap slots
    // (512 per SIMD lane, granted in blocks of 8).
    static constexpr int REGS = SLOT0 + (NSLOT - 1) * K * K + 48;
    static constexpr int waves_reg() {
        int w = 8;
        while (w > 1 && (512 / w) / 8 * 8 < REGS) --w;
        return w;
    }
    template <typename T>
    static constexpr int waves_per_eu() {
        const int lds = (160 * 1024) / (lds_floats<T>() * 4) * NW / 4;
        const int w = lds < waves_reg() ? lds : waves_reg();
        return w < 1 ? 1 : w;
    }

    // group and slot of level l (1..5)
    static constexpr int group_of(int l) { return COARSE ? (l % 2 == 0 ? 0 : 1) : ((l == 3 || l == 5) ? 0 : 1); }
    static constexpr int slot_of(int l) {
        return COARSE ? (l - 1) / 2 : (l == 1 ? 0 : (l == 2 || l == 3) ? 1 : 2);
    }

    template <class F>
    __device__ static __forceinline__ void for_levels(F&& f) {
        lv_impl(f, std::make_integer_sequence<int, L>{});
    }
    template <class F, int... I>
    __device__ static __forceinline__ void lv_impl(F& f, std::integer_sequence<int, I...>) {
        (f(std::integral_constant<int, I + 1>{}), ...);
    }
};

// BASE = false is the coarse pass of the split path: x and dy are the fp32
// planes P_x, P_dy of unnormalised level-L0 LL sums written by the fine pass,
// the kernel's levels are L0+1.. of the layer, and only level taps are
// produced (ordered [L][4][K*K], relative levels).
template <class P, typename T, bool BASE>
__device__ __forceinline__ void bwdw_body(const T* __restrict__ x, const T* __restrict__ dy, float* __restrict__ part,
                                          float* __restrict__ px, float* __restrict__ pdy, int B, int C, int bpc,
                                          float* __restrict__ lds) {
    constexpr int H = P::H, W = P::W, L = P::L, KB = P::KB, K = P::K, NT = P::NT;
    constexpr int PB = P::PB, PK = P::PK, SX = P::SX;
    constexpr int RB = P::RB, NI = P::NI, LPB = P::LPB, XO = P::XO, SD = P::SD;
    constexpr int NSLOT = P::NSLOT, SLOT0 = P::SLOT0;

    constexpr int NPB = P::NPB, PS = P::template pstride<T>();
    // plane p of a step: x (bordered), dy (storage format), U bands, V bands
    auto Xp = [&](int p) { return lds + p * PS; };
    auto DYp = [&](int p) { return reinterpret_cast<T*>(lds + p * PS + P::XSIZE); };
    auto Up = [&](int p) { return lds + p * PS + P::XSIZE + P::template dsize<T>(); };
    auto Vp = [&](int p) { return lds + p * PS + P::XSIZE + P::template dsize<T>() + P::UTOT; };

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int grp = wave >> 2, band = wave & 3, gtid = tid & 255;
    const int c = blockIdx.x % C, chunk = blockIdx.x / C;
    const int b0 = chunk * bpc, b1 = min(B, b0 + bpc);

    // borders stay zero for the whole chunk: nothing writes them
    for (int p = 0; p < NPB; ++p) {
        if constexpr (!P::COARSE) zero_border<1, H, W, PB, SX, XO>(Xp(p), tid, NT);
        P::for_levels([&](auto lc) {
            constexpr int l = decltype(lc)::value;
            zero_border<4, (H >> l), (W >> l), PK, P::su(l)>(Up(p) + P::uoff(l), tid, NT);
        });
    }

    float acc0[SLOT0];
    float accl[NSLOT > 1 ? NSLOT - 1 : 1][K * K];
#pragma unroll
    for (int t = 0; t < SLOT0; ++t) acc0[t] = 0.f;
#pragma unroll
    for (int j = 0; j < (NSLOT > 1 ? NSLOT - 1 : 1); ++j)
#pragma unroll
        for (int t = 0; t < K * K; ++t) accl[j][t] = 0.f;

    // Stream-in and the whole Haar analysis in registers: analysis lane
    // a < NA owns rows 2r, 2r+1 and columns CW q .. CW q + CW-1 of x and dy.
    // Level 1 comes from its own values; each deeper level combines the
    // 2x2 blocks of the level above across lanes with xor shuffles.
    // Analysis lane tid < NPB * NA belongs to plane a_p of the step.
    constexpr int CW = P::CW, NA = P::NA, BR = P::BR, BC = P::BC, GS = P::GS, NBC = P::NBC, NP = CW / 2;
    const int a_p = NPB == 1 ? 0 : tid / NA, a_i = tid - a_p * NA;
    const int a_lb = a_i % GS, a_blk = a_i / GS;
    const int a_rb = a_lb % BR, a_cb = a_lb / BR;
    const int a_r = (a_blk / NBC) * BR + a_rb, a_q = (a_blk % NBC) * BC + a_cb;
    float* const X = Xp(a_p < NPB ? a_p : 0);
    T* const DY = DYp(a_p < NPB ? a_p : 0);
    float* const U = Up(a_p < NPB ? a_p : 0);
    float* const Vb = Vp(a_p < NPB ? a_p : 0);

    // global loads of the next step's planes, in flight during the current
    // taps; a plane past the chunk's end reads as zeros (it adds nothing)
    RawVec<T, CW> vx[2], vd[2];
    auto issue_loads = [&](int b) {
        if (tid < NPB * NA) {
            if (b + a_p < b1) {
                const size_t off = ((size_t)(b + a_p) * C + c) * H * W + (size_t)(2 * a_r) * W + CW * a_q;
                load_raw<T, CW>(x + off, vx[0]);
                load_raw<T, CW>(x + off + W, vx[1]);
                load_raw<T, CW>(dy + off, vd[0]);
                load_raw<T, CW>(dy + off + W, vd[1]);
            } else {
#pragma unroll
                for (int i = 0; i < RawVec<T, CW>::N; ++i) vx[0].w[i] = vx[1].w[i] = vd[0].w[i] = vd[1].w[i] = 0u;
            }
        }
    };
    if (P::PREFETCH && b0 < b1) issue_loads(b0);

    for (int b = b0; b < b1; b += NPB) {
        if (!P::PREFETCH) issue_loads(b);
        // the previous step's taps read x, dy and the bands: all done first
        if (b > b0) __syncthreads();
        // ------------------------------------ P0: stream in and analyse
        if (tid < NPB * NA) {
            float xv[2][CW], dv[2][CW];
            widen_raw(vx[0], xv[0]);
            widen_raw(vx[1], xv[1]);
            widen_raw(vd[0], dv[0]);
            widen_raw(vd[1], dv[1]);
            if constexpr (BASE) {
                store_vec<CW>(X + (2 * a_r + PB) * SX + XO + CW * a_q, xv[0]);
                store_vec<CW>(X + (2 * a_r + 1 + PB) * SX + XO + CW * a_q, xv[1]);
                store_raw<T, CW>(DY + (2 * a_r) * SD + CW * a_q, vd[0]);
                store_raw<T, CW>(DY + (2 * a_r + 1) * SD + CW * a_q, vd[1]);
            }
            // the next step's loads fly during the analysis and the taps
            if (P::PREFETCH && b + NPB < b1) issue_loads(b + NPB);
            // level 1: NP horizontally adjacent positions per lane
            float u[NP][4], v[NP][4];
#pragma unroll
            for (int k = 0; k < NP; ++k) {
                haar4(xv[0][2 * k], xv[0][2 * k + 1], xv[1][2 * k], xv[1][2 * k + 1], u[k][0], u[k][1], u[k][2], u[k][3]);
                haar4(dv[0][2 * k], dv[0][2 * k + 1], dv[1][2 * k], dv[1][2 * k + 1], v[k][0], v[k][1], v[k][2], v[k][3]);
            }
            {
                constexpr int S1 = P::su(1), BS1 = P::bandsz(1), SV1 = P::sv(1), VS1 = P::vsz(1);
#pragma unroll
                for (int k = 0; k < NP; ++k)
#pragma unroll
                    for (int s = 0; s < 4; ++s) {
                        U[s * BS1 + (PK + a_r) * S1 + PK + NP * a_q + k] = u[k][s];
                        Vb[s * VS1 + a_r * SV1 + NP * a_q + k] = v[k][s];
                    }
            }
            // levels 2..L: the LL of the level above, where this lane holds one
            float llu = u[0][0], llv = v[0][0];
            if constexpr (L >= 2 && CW == 4) {
                // level 2: the lane's two level-1 positions are a horizontal
                // pair, its row-pair partner (lane ^ 1) holds the other row
                constexpr int S2 = P::su(2), BS2 = P::bandsz(2), SV2 = P::sv(2), VS2 = P::vsz(2);
                const bool lower = a_rb & 1;
                const float su0 = u[0][0] + u[1][0], du0 = u[0][0] - u[1][0];
                const float sv0 = v[0][0] + v[1][0], dv0 = v[0][0] - v[1][0];
                const float bu0 = haar_pair(su0, 1, lower), bu2 = haar_pair(du0, 1, lower);
                const float bv0 = haar_pair(sv0, 1, lower), bv2 = haar_pair(dv0, 1, lower);
                const int s0 = lower ? 1 : 0, r2 = a_r >> 1;
                U[P::uoff(2) + s0 * BS2 + (PK + r2) * S2 + PK + a_q] = bu0;
                U[P::uoff(2) + (s0 + 2) * BS2 + (PK + r2) * S2 + PK + a_q] = bu2;
                Vb[P::voff(2) + s0 * VS2 + r2 * SV2 + a_q] = bv0;
                Vb[P::voff(2) + (s0 + 2) * VS2 + r2 * SV2 + a_q] = bv2;
                llu = bu0;
                llv = bv0;
            }
            P::for_levels([&](auto lc) {
                constexpr int l = decltype(lc)::value;
                if constexpr (l >= (CW == 4 ? 3 : 2)) {
                    constexpr int Sl = P::su(l), BSl = P::bandsz(l), SVl = P::sv(l), VSl = P::vsz(l);
                    constexpr int MV = 1 << (l - 2), HB = CW == 4 ? 1 << (l - 3) : 1 << (l - 2), MH = BR * HB;
                    const bool right = a_lb & MH, lower = a_lb & MV;
                    // 2x2 butterfly: horizontal pairs, then vertical pairs
                    const float bu = haar_pair(haar_pair(llu, MH, right), MV, lower);
                    const float bv = haar_pair(haar_pair(llv, MH, right), MV, lower);
                    if ((a_rb & (MV - 1)) == 0 && (a_cb & (HB - 1)) == 0) {
                        const int s = (lower ? 1 : 0) + (right ? 2 : 0);
                        const int rl = a_r >> (l - 1), cl = (NP * a_q) >> (l - 1);
                        U[P::uoff(l) + s * BSl + (PK + rl) * Sl + PK + cl] = bu;
                        Vb[P::voff(l) + s * VSl + rl * SVl + cl] = bv;
                    }
                    llu = bu;
                    llv = bv;
                }
            });
            if (P::LT > L && b + a_p < b1) {
                // level-L LL sums for the coarse pass, from the lanes holding them
                constexpr int HL = H >> L, WL = W >> L;
                const size_t po = ((size_t)(b + a_p) * C + c) * HL * WL;
                if constexpr (L == 1) {
#pragma unroll
                    for (int k = 0; k < NP; ++k) {
                        px[po + a_r * WL + NP * a_q + k] = u[k][0];
                        pdy[po + a_r * WL + NP * a_q + k] = v[k][0];
                    }
                } else {
                    constexpr int MV = 1 << (L - 1), HB = CW == 4 ? 1 << (L - 2) : 1 << (L - 1);
                    if ((a_rb & (MV - 1)) == 0 && (a_cb & (HB - 1)) == 0) {
                        const int rl = a_r >> (L - 1), cl = (NP * a_q) >> (L - 1);
                        px[po + rl * WL + cl] = llu;
                        pdy[po + rl * WL + cl] = llv;
                    }
                }
            }
        }
        __syncthreads();
        // ------------------- P3: all taps at once, base taps and one band per wavefront
        if (BASE && grp == 0) {
            if constexpr (P::BASE_PAIR) {
                // column-pair strips; every lane of group A runs every pass
                constexpr int NB = H / RB, WP = (W + KB - 1) / 2;
#pragma unroll
                for (int it = 0; it < cdiv(NPB * NI, 256); ++it) {
                    const int item = gtid + 256 * it, pl = min(item / NI, NPB - 1), r = item - pl * NI;
                    const int rb = min(r / LPB, NB - 1), cq = r % LPB;
                    const bool live = item < NPB * NI && cq < W / 2;
                    const int cl = min(cq, WP - 1), cv = min(cq, W / 2 - 1);
                    taps_pair<KB, RB, SX, SD>(Xp(pl) + XO - PB + rb * RB * SX + 2 * cl, DYp(pl) + rb * RB * SD + 2 * cv,
                                              live, acc0);
                }
            } else {
                for (int item = gtid; item < NPB * NI; item += 256) {
                    const int pl = item / NI, r = item - pl * NI;
                    const int rb = r / LPB, w = r - rb * LPB, h0 = rb * RB;
                    if (LPB == W || w < W)
                        taps_col<KB, RB, SX, SD>(Xp(pl) + XO - PB + h0 * SX + w, DYp(pl) + h0 * SD + w, acc0);
                }
            }
        }
        P::for_levels([&](auto lc) {
            constexpr int l = decltype(lc)::value;
            constexpr int hl = H >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), VSl = P::vsz(l);
            constexpr int R = P::band_rows(l);
            if (grp == P::group_of(l)) {
                constexpr int SVl = P::sv(l);
                // band `band` of level l in plane pl of the step
                auto Us = [&](int pl) -> const float* { return Up(pl) + P::uoff(l) + band * BSl; };
                auto Vs = [&](int pl) -> const float* { return Vp(pl) + P::voff(l) + band * VSl; };
                auto& slot = [&]() -> auto& {
                    if constexpr (P::slot_of(l) == 0) return acc0;
                    else return accl[P::slot_of(l) - 1];
                }();
                if constexpr (P::level_pair(l)) {
                    // column-pair strips; every lane of the wavefront runs every pass
                    constexpr int LP = pair_lanes(wl, K), NS = hl / R, NIl = NS * LP, WP = (wl + K - 1) / 2;
#pragma unroll
                    for (int it = 0; it < cdiv(NPB * NIl, 64); ++it) {
                        const int item = lane + 64 * it, pl = min(item / NIl, NPB - 1), r = item - pl * NIl;
                        const int rs = min(r / LP, NS - 1), cq = r % LP;
                        const bool live = item < NPB * NIl && cq < wl / 2;
                        const int cl = min(cq, WP - 1), cv = min(cq, wl / 2 - 1);
                        taps_pair<K, R, Sl, SVl>(Us(pl) + R * rs * Sl + 2 * cl, Vs(pl) + R * rs * SVl + 2 * cv, live,
                                                 slot);
                    }
                } else {
                    constexpr int LPl = strip_lanes(wl), NIl = (hl / R) * LPl;
                    for (int item = lane; item < NPB * NIl; item += 64) {
                        const int pl = item / NIl, r = item - pl * NIl;
                        const int rs = r / LPl, j = r - rs * LPl;
                        if (!(LPl == wl || j < wl)) continue;
                        taps_col<K, R, Sl, SVl>(Us(pl) + R * rs * Sl + j, Vs(pl) + R * rs * SVl + j, slot);
                    }
                }
            }
        });
    }

    // ------------------------------------------------------ reduction
    // each 16-lane row's sum (DPP), the four rows of each wavefront through
    // LDS, then a fixed-order sum per tap
#pragma unroll
    for (int t = 0; t < SLOT0; ++t) acc0[t] = row_sum(acc0[t]);
#pragma unroll
    for (int j = 0; j < NSLOT - 1; ++j)
#pragma unroll
        for (int t = 0; t < K * K; ++t) accl[j][t] = row_sum(accl[j][t]);
    __syncthreads();  // all of LDS becomes reduction scratch
    float* red0 = lds;                         // [NW][4 rows][SLOT0]
    float* redl = lds + P::NW * 4 * SLOT0;     // [NW][4 rows][NSLOT-1][K*K]
    if ((lane & 15) == 0) {
        const int wr = wave * 4 + (lane >> 4);
#pragma unroll
        for (int t = 0; t < SLOT0; ++t) red0[wr * SLOT0 + t] = acc0[t];
#pragma unroll
        for (int j = 0; j < NSLOT - 1; ++j)
#pragma unroll
            for (int t = 0; t < K * K; ++t) redl[(wr * (NSLOT - 1) + j) * K * K + t] = accl[j][t];
    }
    __syncthreads();
    constexpr int NB = BASE ? KB * KB : 0;   // base taps written by this kernel
    constexpr int TOUT = NB + 4 * L * K * K;
    float* dst = part + ((size_t)chunk * C + c) * TOUT;
    for (int t = tid; t < TOUT; t += NT) {
        float v = 0.f;
        if (t < NB) {
#pragma unroll
            for (int wr = 0; wr < 16; ++wr) v += red0[wr * SLOT0 + t];   // group A: waves 0..3, rows in order
        } else {
            const int r = t - NB, ls = r / (K * K), tap = r - ls * (K * K);
            const int l = ls / 4 + 1, s = ls - (l - 1) * 4;   // taps are ordered [L][4][K*K]
            const int w = P::group_of(l) * 4 + s, slot = P::slot_of(l);
#pragma unroll
            for (int q = 0; q < 4; ++q)
                v += slot == 0 ? red0[(w * 4 + q) * SLOT0 + tap]
                               : redl[((w * 4 + q) * (NSLOT - 1) + slot - 1) * K * K + tap];
        }
        dst[t] = v;
    }
}

template <class P, typename T, bool BASE>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(P::template waves_per_eu<T>())))
void bwdw_kernel(const T* __restrict__ x, const T* __restrict__ dy, float* __restrict__ part,
                 float* __restrict__ px, float* __restrict__ pdy, int B, int C, int bpc) {
    __shared__ __attribute__((aligned(16))) float lds[P::template lds_floats<T>()];
    bwdw_body<P, T, BASE>(x, dy, part, px, pdy, B, C, bpc, lds);
}

// A level split in one workgroup: the fine pass over the chunk (base and
// levels 1..L, writing the chunk's level-L LL planes), then the coarse pass
// over the same planes (levels L+1..LT), read back from L2, with the same LDS.
template <class FP, class CP, typename T>
constexpr int split_waves() {
    const int a = FP::template waves_per_eu<T>(), b = CP::template waves_per_eu<float>();
    return a < b ? a : b;
}
template <class FP, class CP, typename T>
constexpr int split_lds() {
    const int a = FP::template lds_floats<T>(), b = CP::template lds_floats<float>();
    return a > b ? a : b;
}
template <class FP, class CP, typename T>
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(split_waves<FP, CP, T>())))
void bwdw_split_kernel(const T* __restrict__ x, const T* __restrict__ dy, float* __restrict__ partA,
                       float* __restrict__ partB, float* __restrict__ px, float* __restrict__ pdy, int B, int C,
                       int bpc) {
    __shared__ __attribute__((aligned(16))) float lds[split_lds<FP, CP, T>()];
    bwdw_body<FP, T, true>(x, dy, partA, px, pdy, B, C, bpc, lds);
    // the LL planes this workgroup wrote become visible to it; LDS is free
    __syncthreads();
    bwdw_body<CP, float, false>(px, pdy, partB, nullptr, nullptr, B, C, bpc, lds);
}

// Threads of the finalize kernel: one per tap, whole wavefronts.
static inline unsigned finalize_threads(int KB, int K, int L) {
    const int taps = KB * KB + 4 * L * K * K;
    return (unsigned)(((taps + 63) / 64) * 64 > 1024 ? 1024 : ((taps + 63) / 64) * 64);
}

// Stage 2: fixed-order sum over chunks, then scale and normalisation. Taps
// [0, TA) (base, levels 1..LA) come from partA, the rest (levels LA+1..L)
// from partB when the plane was split.
__global__ __launch_bounds__(1024) void bwdw_finalize(const float* __restrict__ partA, int nA, int LA,
                                                      const float* __restrict__ partB, int nB, int C,
                                                      int L, int KB, int K,
                                                      const float* __restrict__ w_lvl,
                                                      const float* __restrict__ scale,
                                                      float* __restrict__ dw_base,
                                                      float* __restrict__ dw_lvl,
                                                      float* __restrict__ dscale) {
    // w_lvl * G per level tap, sized for every shape the ABI accepts (the
    // host rejects L > 5 and kernels above 15 before any launch)
    constexpr int kMaxLevels = 5, kMaxK = 15;
    __shared__ float WG[4 * kMaxLevels * kMaxK * kMaxK];
    if (L > kMaxLevels || K > kMaxK) return;
    const int c = blockIdx.x, tid = threadIdx.x;
    const int kb2 = KB * KB, k2 = K * K, taps = kb2 + 4 * L * k2;
    const int TA = kb2 + 4 * LA * k2, TB = taps - TA;
    // one tap per thread (blockDim covers every tap): the partial sums, the
    // scale and the level tap are all requested before any is used
    for (int t = tid; t < taps; t += blockDim.x) {
        float sc = 1.f, wv = 0.f;
        size_t pi = 0;
        int tap = 0;
        if (t >= kb2) {
            const int r = t - kb2, ls = r / k2, l = ls / 4, s = ls - 4 * l;
            tap = r - ls * k2;
            pi = ((size_t)l * C + c) * 4 + s;
            sc = scale[pi];
            wv = w_lvl[pi * k2 + tap];
        }
        float a = 0.f;   // the sum stays in chunk order
        if (t < TA) {
#pragma unroll 8
            for (int ch = 0; ch < nA; ++ch) a += partA[((size_t)ch * C + c) * TA + t];
        } else {
#pragma unroll 8
            for (int ch = 0; ch < nB; ++ch) a += partB[((size_t)ch * C + c) * TB + (t - TA)];
        }
        if (t < kb2) {
            dw_base[(size_t)c * kb2 + t] = a;
        } else {
            const int l = (t - kb2) / (4 * k2);   // 0-based level
            a *= 1.0f / (float)(1 << (2 * (l + 1)));
            dw_lvl[pi * k2 + tap] = sc * a;
            WG[t - kb2] = wv * a;
        }
    }
    __syncthreads();
    for (int ls = tid; ls < 4 * L; ls += blockDim.x) {
        const int l = ls / 4, s = ls - 4 * l;
        float a = 0.f;
        for (int tap = 0; tap < k2; ++tap) a += WG[ls * k2 + tap];
        dscale[((size_t)l * C + c) * 4 + s] = a;
    }
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
template <int H_, int W_, int L0_, int LT_, int KB_, int K_, int TH_, int NT_ = 512>
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
    static constexpr int su(int l) { return odd_stride((W >> l) + 2 * PK); }
    static constexpr int bandsz(int l) { return rh(l) * su(l); }
    static constexpr int sv(int l) { return odd_stride(W >> l); }
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
        __syncthreads();
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
        __syncthreads();
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
                __syncthreads();
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
        __syncthreads();
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

// ------------------------------------------------------------ registry

// batches (or tile units) per chunk: about one workgroup per slot of the
// chip (256 CUs x 2 resident workgroups of 8 wavefronts), so the per-chunk
// reduction is amortised over as many planes as the parallelism allows
// (rounded down: a second, mostly empty round of workgroups would double
// the kernel's tail)
static int chunk_units(int units, int C, int slots = 512) {
    int nchunk = slots / C;
    if (nchunk > units) nchunk = units;
    if (nchunk < 1) nchunk = 1;
    return cdiv(units, nchunk);
}

// Compute units of the current device (queried once per device).
static int cu_count() {
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

// Resident workgroups of a whole-plane weight-gradient plan with activations
// of type T: CUs x the workgroups per CU its register and LDS budget allows.
template <class P, typename T>
static int bw_slots() {
    const int per_cu = P::template waves_per_eu<T>() * 4 / P::NW;
    return cu_count() * (per_cu < 1 ? 1 : per_cu);
}

static size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// whole planes: one kernel and the finalize
template <class P>
static size_t whole_ws(int B, int C) {
    const int slots = bw_slots<P, bf16_t>() > bw_slots<P, float>() ? bw_slots<P, bf16_t>() : bw_slots<P, float>();
    const int nchunk = cdiv(B, chunk_units(B, C, slots));
    return (size_t)nchunk * C * P::TAPS * sizeof(float);
}

template <class P, typename T>
static hipError_t whole_launch(const void* x, const void* dy, const float* w_lvl, const float* scale,
                               float* dw_base, float* dw_lvl, float* dscale, void* ws, int B, int C,
                               hipStream_t stream) {
    const int bpc = chunk_units(B, C, bw_slots<P, T>()), nchunk = cdiv(B, bpc);
    float* part = (float*)ws;
    hipLaunchKernelGGL((bwdw_kernel<P, T, true>), dim3((unsigned)(nchunk * C)), dim3(P::NT), 0, stream,
                       (const T*)x, (const T*)dy, part, (float*)nullptr, (float*)nullptr, B, C, bpc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(bwdw_finalize, dim3((unsigned)C), dim3(finalize_threads(P::KB, P::K, P::L)), 0, stream,
                       (const float*)part, nchunk,
                       P::L, (const float*)nullptr, 0, C, P::L, P::KB, P::K, w_lvl, scale, dw_base, dw_lvl,
                       dscale);
    return hipGetLastError();
}

// split planes: the fine tiles (base and levels 1..L0, plus the LL sums),
// the coarse pass on the LL sums (levels L0+1..L), then the finalize
template <class FP, class CP>
static size_t split_bw_ws(int B, int C) {
    const int units = B * FP::NTILE;
    const int nA = cdiv(units, chunk_units(units, C));
    size_t n = align256((size_t)nA * C * FP::TAPS * sizeof(float));
    if (FP::LT > FP::L0) {
        const int nB = cdiv(B, chunk_units(B, C));
        n += align256((size_t)nB * C * 4 * (FP::LT - FP::L0) * FP::K * FP::K * sizeof(float));
        n += 2 * align256((size_t)B * C * (FP::H >> FP::L0) * (FP::W >> FP::L0) * sizeof(float));
    }
    return n;
}

template <class FP, class CP, typename T>
static hipError_t split_bw_launch(const void* x, const void* dy, const float* w_lvl, const float* scale,
                                  float* dw_base, float* dw_lvl, float* dscale, void* ws, int B, int C,
                                  hipStream_t stream) {
    const int units = B * FP::NTILE;
    const int upc = chunk_units(units, C), nA = cdiv(units, upc);
    char* cur = (char*)ws;
    float* partA = (float*)cur;
    cur += align256((size_t)nA * C * FP::TAPS * sizeof(float));
    float *partB = nullptr, *px = nullptr, *pdy = nullptr;
    int nB = 0;
    if constexpr (FP::LT > FP::L0) {
        nB = cdiv(B, chunk_units(B, C));
        partB = (float*)cur;
        cur += align256((size_t)nB * C * 4 * (FP::LT - FP::L0) * FP::K * FP::K * sizeof(float));
        const size_t pl = (size_t)B * C * (FP::H >> FP::L0) * (FP::W >> FP::L0) * sizeof(float);
        px = (float*)cur;
        cur += align256(pl);
        pdy = (float*)cur;
    }
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
    hipLaunchKernelGGL(bwdw_finalize, dim3((unsigned)C), dim3(finalize_threads(FP::KB, FP::K, FP::LT)), 0,
                       stream, (const float*)partA, nA, FP::L0,
                       (const float*)partB, nB, C, FP::LT, FP::KB, FP::K, w_lvl, scale, dw_base, dw_lvl,
                       dscale);
    return hipGetLastError();
}

// whole planes split by level: the whole-plane kernel does the base and
// levels 1..L (one or two tap slots per lane, so more workgroups fit a CU)
// and writes the level-L LL sums; the coarse pass does levels L+1..LT
template <class FP, class CP>
static int plane_split_slots() {
    const int a = cu_count() * (split_waves<FP, CP, bf16_t>() * 4 / FP::NW);
    const int b = cu_count() * (split_waves<FP, CP, float>() * 4 / FP::NW);
    return (a > b ? a : b) < 1 ? 1 : (a > b ? a : b);
}

template <class FP, class CP>
static size_t plane_split_ws(int B, int C) {
    const int nch = cdiv(B, chunk_units(B, C, plane_split_slots<FP, CP>()));
    size_t n = align256((size_t)nch * C * FP::TAPS * sizeof(float));
    n += align256((size_t)nch * C * 4 * (FP::LT - FP::L) * FP::K * FP::K * sizeof(float));
    n += 2 * align256((size_t)B * C * (FP::H >> FP::L) * (FP::W >> FP::L) * sizeof(float));
    return n;
}

template <class FP, class CP, typename T>
static hipError_t plane_split_launch(const void* x, const void* dy, const float* w_lvl, const float* scale,
                                     float* dw_base, float* dw_lvl, float* dscale, void* ws, int B, int C,
                                     hipStream_t stream) {
    static_assert(FP::LT > FP::L && CP::LT == CP::L && CP::KB == 1 && CP::K == FP::K &&
                      CP::L == FP::LT - FP::L && CP::H == (FP::H >> FP::L) && CP::W == (FP::W >> FP::L) &&
                      FP::NT == CP::NT,
                  "coarse plan: levels L+1..LT of the fine plan on its LL planes");
    const int nch_ws = cdiv(B, chunk_units(B, C, plane_split_slots<FP, CP>()));
    const int slots = cu_count() * (split_waves<FP, CP, T>() * 4 / FP::NW);
    const int bpc = chunk_units(B, C, slots < 1 ? 1 : slots), nch = cdiv(B, bpc);
    char* cur = (char*)ws;
    float* partA = (float*)cur;
    cur += align256((size_t)nch_ws * C * FP::TAPS * sizeof(float));
    float* partB = (float*)cur;
    cur += align256((size_t)nch_ws * C * 4 * (FP::LT - FP::L) * FP::K * FP::K * sizeof(float));
    const size_t pl = (size_t)B * C * (FP::H >> FP::L) * (FP::W >> FP::L) * sizeof(float);
    float* px = (float*)cur;
    cur += align256(pl);
    float* pdy = (float*)cur;
    hipLaunchKernelGGL((bwdw_split_kernel<FP, CP, T>), dim3((unsigned)(nch * C)), dim3(FP::NT), 0, stream,
                       (const T*)x, (const T*)dy, partA, partB, px, pdy, B, C, bpc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    hipLaunchKernelGGL(bwdw_finalize, dim3((unsigned)C), dim3(finalize_threads(FP::KB, FP::K, FP::LT)), 0,
                       stream, (const float*)partA, nch, FP::L, (const float*)partB, nch, C, FP::LT, FP::KB, FP::K,
                       w_lvl, scale, dw_base, dw_lvl, dscale);
    return hipGetLastError();
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
    hipLaunchKernelGGL(bwdw_finalize, dim3((unsigned)C), dim3(finalize_threads(P::KB, 1, 0)), 0, stream,
                       (const float*)part, nch, 0, (const float*)nullptr, 0, C, 0, P::KB, 1, (const float*)nullptr,
                       (const float*)nullptr, dw_base, (float*)nullptr, (float*)nullptr);
    return hipGetLastError();
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
    hipLaunchKernelGGL(bwdw_finalize, dim3((unsigned)C), dim3(finalize_threads(P::KB, 1, 0)), 0, stream,
                       (const float*)part, nch, 0, (const float*)nullptr, 0, C, 0, P::KB, 1, (const float*)nullptr,
                       (const float*)nullptr, dw_base, (float*)nullptr, (float*)nullptr);
    return hipGetLastError();
}

typedef hipError_t (*bwd1_fn)(const void* x, const void* dy, const float* w_base, void* dx, float* dw_base,
                              void* ws, int B, int C, hipStream_t stream);
struct Bwd1Entry {
    int H, W, KB;
    bwd1_fn fn[2];
    size_t (*ws)(int B, int C);
};

typedef hipError_t (*bwdw_fn)(const void*, const void*, const float*, const float*, float*, float*, float*,
                              void*, int, int, hipStream_t);

struct BwEntry {
    int H, W, L, KB, K;
    bwdw_fn fn[2];
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
typedef TileBwPlan<256, 256, 2, 4, 7, 5, 16> TB_256_L2of4_k75;
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
    {PLAN::H, PLAN::W, PLAN::L, PLAN::KB, PLAN::K, {whole_launch<PLAN, float>, whole_launch<PLAN, bf16_t>}, whole_ws<PLAN>}
#define WTC_BW_PLANESPLIT(FPL, CPL)                                                               \
    {FPL::H, FPL::W, FPL::LT, FPL::KB, FPL::K,                                                   \
     {plane_split_launch<FPL, CPL, float>, plane_split_launch<FPL, CPL, bf16_t>}, plane_split_ws<FPL, CPL>}
#define WTC_BW_SPLIT(FPL, CPL)                                                                    \
    {FPL::H, FPL::W, FPL::LT, FPL::KB, FPL::K,                                                   \
     {split_bw_launch<FPL, CPL, float>, split_bw_launch<FPL, CPL, bf16_t>}, split_bw_ws<FPL, CPL>}

static const BwEntry kBwEntries[] = {
    WTC_BW_PLANESPLIT(WP_56_L1of3_k55, CB_28_L2_k5), WTC_BW_PLANESPLIT(WP_28_L1of2_k55, CB_14_L1_k5),
    WTC_BW_WHOLE(BP_32_L2_k55), WTC_BW_WHOLE(BP_14_L1_k55),    WTC_BW_WHOLE(BP_32_L3_k75),
    WTC_BW_WHOLE(BP_24x40_L3_k33), WTC_BW_WHOLE(BP_16_L4_k37), WTC_BW_WHOLE(BP_64_L4_k75),
    WTC_BW_SPLIT(TB_128_L1_k55, CB_32_L1_k5),      WTC_BW_SPLIT(TB_128_L2_k55, CB_32_L1_k5),
    WTC_BW_SPLIT(TB_128_L2of3_k55, CB_32_L1_k5),   WTC_BW_SPLIT(TB_128_L2of4_k55, CB_32_L2_k5),
    WTC_BW_SPLIT(TB_128_L2of5_k55, CB_32_L3_k5),   WTC_BW_SPLIT(TB_256_L2of4_k75, CB_64_L2_k5),
    WTC_BW_SPLIT(TB_64_L2of4_k33, CB_16_L2_k3),    WTC_BW_SPLIT(TB_64_L1of2_k55, CB_32_L1_k5),
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

static const BwEntry* find_bw(int H, int W, int L, int KB, int K) {
    for (const BwEntry& e : kBwEntries)
        if (e.H == H && e.W == W && e.L == L && e.KB == KB && (L == 0 || e.K == K)) return &e;
    return nullptr;
}

size_t bwdw_workspace_bytes(int B, int C, int H, int W, int L, int KB, int K) {
    const BwEntry* e = find_bw(H, W, L, KB, K);
    return e ? e->ws(B, C) : (size_t)-1;
}

hipError_t bwdw_launch(int B, int C, int H, int W, int L, int KB, int K, bool bf16, const void* x,
                       const void* dy, const float* w_lvl, const float* scale, float* dw_base,
                       float* dw_lvl, float* dscale, void* ws, hipStream_t stream) {
    const BwEntry* e = find_bw(H, W, L, KB, K);
    if (!e) return hipErrorInvalidValue;
    return e->fn[bf16 ? 1 : 0](x, dy, w_lvl, scale, dw_base, dw_lvl, dscale, ws, B, C, stream);
}

}  // namespace wtc
