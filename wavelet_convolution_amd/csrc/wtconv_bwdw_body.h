// Weight-gradient kernel templates shared by the translation units that
// instantiate plans: the tap-sum strips, the whole-plane plan and kernel, the
// level-split kernel, and the whole-plane launcher with its workspace size.
// The gradients are correlations of the two Haar pyramids (the abstract of
// arXiv:2608.10805, reformulation (3)); see wtconv_bwdw.hip.
#pragma once

#include "wtconv_bwdw.h"
#include "wtconv_device.h"
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
//
// IH x IW (at most H x W) is the plane in memory; a smaller one is zero-padded
// to H x W on chip, which for a plane that 2^L does not divide is exactly the
// layer's reading of odd band grids (the padded cells of x and dy are zero,
// so their bands are zero beyond each odd grid: no tap sum changes).
template <int H_, int W_, int L_, int KB_, int K_, int LT_ = L_, int NPB_ = 1, int IH_ = H_, int IW_ = W_,
          int REGX_ = 48>
struct BwPlan {
    static constexpr int H = H_, W = W_, L = L_, KB = KB_, K = K_;
    static constexpr int IH = IH_, IW = IW_;
    static constexpr bool PADDED = IH != H || IW != W;
    static_assert(IH <= H && IW <= W && IH > H - (1 << LT_) && IW > W - (1 << LT_), "padding below one 2^LT block");
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
    static constexpr int band_rows(int l) {
        return level_pair(l) ? pick_rows2(H >> l, W >> l, 64, K, NPB) : pick_rows(H >> l, W >> l, 64, K, NPB);
    }
    // band rows: even strides where column pairs are read (8-byte aligned
    // pairs), odd ones elsewhere (the analysis stores of lanes on
    // consecutive rows then fall into different banks). Where one 32-lane
    // pass of the one-column level strips holds several row strips of one
    // plane (28x28: level 1 in two 7-row strips), the stride is the first
    // from there with the fewest bank conflicts between them (28x28: 19
    // floats put the second strip 5 banks on, over 9 of the first strip's
    // 14; 25 put it 15 on, clear of them).
    static constexpr int row_conflicts(int l, int S) {
        const int hl = H >> l, wl = W >> l, R = band_rows(l), LP = strip_lanes(wl), NI = (hl / R) * LP;
        // lanes of one plane only (planes are placed apart by best_pitch)
        int cost = 0;
        for (int h0 = 0; h0 < NPB * NI; h0 += 32) {
            int worst = 0;
            for (int pl = 0; pl < NPB; ++pl) {
                int cnt[32] = {};
                for (int t = h0; t < h0 + 32 && t < NPB * NI; ++t) {
                    const int tp = t / NI, r = t - tp * NI, rs = r / LP, j = r - rs * LP;
                    if (tp != pl || j >= wl) continue;
                    const int b = (rs * R * S + j) % 32;
                    if (++cnt[b] > worst) worst = cnt[b];
                }
            }
            cost += worst;
        }
        return cost;
    }
    static constexpr int level_stride(int l, int base) {
        if (level_pair(l) || l > L) return base;
        int best = base, best_cost = row_conflicts(l, base);
        for (int S = base + 2; S < base + 32; S += 2)
            if (row_conflicts(l, S) < best_cost) {
                best_cost = row_conflicts(l, S);
                best = S;
            }
        return best;
    }
    static constexpr int su_calc(int l) {
        return l > L ? 1
                     : level_pair(l) ? round_up((W >> l) + 2 * PK, 2) : level_stride(l, odd_stride((W >> l) + 2 * PK));
    }
    static constexpr int sv_calc(int l) {
        return l > L ? 1 : level_pair(l) ? round_up(W >> l, 2) : level_stride(l, odd_stride(W >> l));
    }
    // computed once per plan (each is a search)
    static constexpr int SU[6] = {1, su_calc(1), su_calc(2), su_calc(3), su_calc(4), su_calc(5)};
    static constexpr int SV[6] = {1, sv_calc(1), sv_calc(2), sv_calc(3), sv_calc(4), sv_calc(5)};
    static constexpr int su(int l) { return SU[l]; }
    static constexpr int bandsz(int l) { return ((H >> l) + 2 * PK) * su(l); }
    static constexpr int sv(int l) { return SV[l]; }
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
    // Order of the one-column base strips over the lanes: plane-major
    // (strip s = plane s / (H/RB), row block s % (H/RB)), or row-block-major
    // with the planes of each group of four taken 0, 2, 1, 3, so that the
    // strips sharing a 32-lane LDS pass come from planes two apart rather
    // than from neighbouring row blocks of one plane (14x14: row blocks 7 x 20
    // floats apart share two banks, planes two pitches apart none). The
    // order with fewer bank conflicts on the x rows is taken.
    template <typename T>
    static constexpr int base_conflicts(bool rbmajor) {
        const int ps = pstride<T>(), n = NPB * NI;
        int cost = 0;
        for (int h0 = 0; h0 < n; h0 += 32) {
            int cnt[32] = {};
            int worst = 0;
            for (int t = h0; t < h0 + 32 && t < n; ++t) {
                int pl, rb;
                const int w = t % LPB;
                if (rbmajor) {
                    const int st = t / LPB, q = st % NPB;
                    rb = st / NPB;
                    pl = (q & ~3) | ((q & 1) << 1) | ((q >> 1) & 1);
                } else {
                    pl = t / NI;
                    rb = (t - pl * NI) / LPB;
                }
                if (w >= W) continue;
                const int b = (pl * ps + rb * RB * SX + w) % 32;
                if (++cnt[b] > worst) worst = cnt[b];
            }
            cost += worst;
        }
        return cost;
    }
    template <typename T>
    static constexpr bool base_rbmajor() {
        return !BASE_PAIR && !COARSE && NPB % 4 == 0 && base_conflicts<T>(true) < base_conflicts<T>(false);
    }
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
    // at about REGX registers of strips and addresses beside the tap slots
    // (512 per SIMD lane, granted in blocks of 8).
    static constexpr int REGS = SLOT0 + (NSLOT - 1) * K * K + REGX_;
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
    if constexpr (NPB > 1) {
        // several planes per step: their whole regions cleared with a few
        // 128-bit stores per thread (a border loop per plane and band costs
        // more: 14x14, eight planes, about a fifth of the multiply-adds);
        // the barrier keeps these stores ahead of the first stream-in
        constexpr int NZ = NPB * PS;
        float4* const z = reinterpret_cast<float4*>(lds);
        for (int t = tid; t < NZ / 4; t += NT) z[t] = make_float4(0.f, 0.f, 0.f, 0.f);
        if (tid < NZ % 4) lds[NZ / 4 * 4 + tid] = 0.f;
        __syncthreads();
    } else {
        if constexpr (!P::COARSE) zero_border<1, H, W, PB, SX, XO>(Xp(0), tid, NT);
        P::for_levels([&](auto lc) {
            constexpr int l = decltype(lc)::value;
            zero_border<4, (H >> l), (W >> l), PK, P::su(l)>(Up(0) + P::uoff(l), tid, NT);
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
    constexpr int IH = P::IH, IW = P::IW;
    auto issue_loads = [&](int b) {
        if (tid < NPB * NA) {
            if constexpr (P::PADDED) {
                // the padded plane: cells outside IH x IW read as zeros
                const size_t pl = ((size_t)(b + a_p) * C + c) * IH * IW;
                const bool live = b + a_p < b1;
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int r = 2 * a_r + h, c0 = CW * a_q;
                    load_raw_guarded<T, CW, IW>(x + pl + (size_t)r * IW, c0, live && r < IH, vx[h]);
                    load_raw_guarded<T, CW, IW>(dy + pl + (size_t)r * IW, c0, live && r < IH, vd[h]);
                }
            } else if (b + a_p < b1) {
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
        if (b > b0) lds_barrier();   // (LDS only: the next step's loads stay in flight)
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
        // (LDS only: the LL sums written to global memory above are read by
        // a later pass, and the next step's loads stay in flight)
        lds_barrier();
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
                    int pl, r;
                    if constexpr (P::template base_rbmajor<T>()) {
                        const int st = item / LPB, rbs = st / NPB, q = st - rbs * NPB;
                        pl = (q & ~3) | ((q & 1) << 1) | ((q >> 1) & 1);
                        r = rbs * LPB + (item - st * LPB);
                    } else {
                        pl = item / NI;
                        r = item - pl * NI;
                    }
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
inline unsigned finalize_threads(int KB, int K, int L) {
    const int taps = KB * KB + 4 * L * K * K;
    return (unsigned)(((taps + 63) / 64) * 64 > 1024 ? 1024 : ((taps + 63) / 64) * 64);
}

// Stage 2 (one workgroup per channel, the fixed-order chunk sum, scale and
// normalisation; wtconv_bwdw.hip), enqueued on `stream`.
hipError_t launch_bwdw_finalize(const float* partA, int nA, int LA, const float* partB, int nB, int C, int L, int KB,
                                int K, const float* w_lvl, const float* scale, float* dw_base, float* dw_lvl,
                                float* dscale, hipStream_t stream);


// batches (or tile units) per chunk: about one workgroup per slot of the
// chip (256 CUs x 2 resident workgroups of 8 wavefronts), so the per-chunk
// reduction is amortised over as many planes as the parallelism allows
// (rounded down: a second, mostly empty round of workgroups would double
// the kernel's tail)
inline int chunk_units(int units, int C, int slots = 512) {
    int nchunk = slots / C;
    if (nchunk > units) nchunk = units;
    if (nchunk < 1) nchunk = 1;
    return cdiv(units, nchunk);
}

// Compute units of the current device (queried once per device).
int cu_count();

// Resident workgroups of a whole-plane weight-gradient plan with activations
// of type T: CUs x the workgroups per CU its register and LDS budget allows.
template <class P, typename T>
int bw_slots() {
    const int per_cu = P::template waves_per_eu<T>() * 4 / P::NW;
    return cu_count() * (per_cu < 1 ? 1 : per_cu);
}

inline size_t bw_align256(size_t n) { return (n + 255) / 256 * 256; }

// whole planes: one kernel and the finalize
template <class P>
size_t whole_ws(int B, int C) {
    const int slots = bw_slots<P, bf16_t>() > bw_slots<P, float>() ? bw_slots<P, bf16_t>() : bw_slots<P, float>();
    const int nchunk = cdiv(B, chunk_units(B, C, slots));
    return (size_t)nchunk * C * P::TAPS * sizeof(float);
}

template <class P, typename T>
hipError_t whole_launch(const void* x, const void* dy, const float* w_lvl, const float* scale,
                               float* dw_base, float* dw_lvl, float* dscale, void* ws, int B, int C,
                               hipStream_t stream) {
    const int bpc = chunk_units(B, C, bw_slots<P, T>()), nchunk = cdiv(B, bpc);
    float* part = (float*)ws;
    hipLaunchKernelGGL((bwdw_kernel<P, T, true>), dim3((unsigned)(nchunk * C)), dim3(P::NT), 0, stream,
                       (const T*)x, (const T*)dy, part, (float*)nullptr, (float*)nullptr, B, C, bpc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_bwdw_finalize(part, nchunk, P::L, nullptr, 0, C, P::L, P::KB, P::K, w_lvl, scale, dw_base, dw_lvl,
                                dscale, stream);
}

// whole planes split by level: the whole-plane kernel does the base and
// levels 1..L (one or two tap slots per lane, so more workgroups fit a CU)
// and writes the level-L LL sums; the coarse pass does levels L+1..LT
template <class FP, class CP>
int plane_split_slots() {
    const int a = cu_count() * (split_waves<FP, CP, bf16_t>() * 4 / FP::NW);
    const int b = cu_count() * (split_waves<FP, CP, float>() * 4 / FP::NW);
    return (a > b ? a : b) < 1 ? 1 : (a > b ? a : b);
}

template <class FP, class CP>
size_t plane_split_ws(int B, int C) {
    const int nch = cdiv(B, chunk_units(B, C, plane_split_slots<FP, CP>()));
    size_t n = bw_align256((size_t)nch * C * FP::TAPS * sizeof(float));
    n += bw_align256((size_t)nch * C * 4 * (FP::LT - FP::L) * FP::K * FP::K * sizeof(float));
    n += 2 * bw_align256((size_t)B * C * (FP::H >> FP::L) * (FP::W >> FP::L) * sizeof(float));
    return n;
}

template <class FP, class CP, typename T>
hipError_t plane_split_launch(const void* x, const void* dy, const float* w_lvl, const float* scale,
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
    cur += bw_align256((size_t)nch_ws * C * FP::TAPS * sizeof(float));
    float* partB = (float*)cur;
    cur += bw_align256((size_t)nch_ws * C * 4 * (FP::LT - FP::L) * FP::K * FP::K * sizeof(float));
    const size_t pl = (size_t)B * C * (FP::H >> FP::L) * (FP::W >> FP::L) * sizeof(float);
    float* px = (float*)cur;
    cur += bw_align256(pl);
    float* pdy = (float*)cur;
    hipLaunchKernelGGL((bwdw_split_kernel<FP, CP, T>), dim3((unsigned)(nch * C)), dim3(FP::NT), 0, stream,
                       (const T*)x, (const T*)dy, partA, partB, px, pdy, B, C, bpc);
    hipError_t err = hipGetLastError();
    if (err != hipSuccess) return err;
    return launch_bwdw_finalize(partA, nch, FP::L, partB, nch, C, FP::LT, FP::KB, FP::K, w_lvl, scale, dw_base, dw_lvl,
                                dscale, stream);
}

typedef hipError_t (*bwdw_fn)(const void*, const void*, const float*, const float*, float*, float*, float*,
                              void*, int, int, hipStream_t);

struct BwEntry {
    int H, W, L, KB, K;
    bwdw_fn fn[2];
    size_t (*ws)(int B, int C);
    // plans that leave the fp32 planes [B][C][H >> l0][W >> l0] of level-l0
    // LL sums of dy in their workspace: l0 and the planes' byte offset
    int l0 = 0;
    size_t (*dy_sums_offset)(int B, int C) = nullptr;
};

}  // namespace wtc
