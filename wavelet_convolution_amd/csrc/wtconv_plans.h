// Compile-time plans of the whole-plane fused kernel: the LDS layout and the
// work split of one (b, c) plane over a workgroup.
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "wtconv_device.h"

namespace wtc {

// Compute units of the current device (queried once per device).
int cu_count();

struct Tile {
    int r, c;
};

// Tile (positions per work item) for a coarse level grid of h x w on nt
// threads: the shortest critical path (items per thread x tile size), ties
// going to the larger tile (fewer LDS reads per FMA).
constexpr Tile pick_tile(int h, int w, int nt) {
    const int cand[7][2] = {{4, 4}, {4, 2}, {2, 4}, {2, 2}, {2, 1}, {1, 2}, {1, 1}};
    Tile best{1, 1};
    int best_cost = 1 << 30, best_size = 0;
    for (int i = 0; i < 7; ++i) {
        const int r = cand[i][0], c = cand[i][1];
        if (h % r != 0 || w % c != 0) continue;
        const int items = (h / r) * (w / c);
        const int cost = cdiv(items, nt) * r * c;
        if (cost < best_cost || (cost == best_cost && r * c > best_size)) {
            best = Tile{r, c};
            best_cost = cost;
            best_size = r * c;
        }
    }
    return best;
}

// H x W plane, L levels, base kernel KB, level kernel K, NT threads; a main
// work item is a TR x TC tile of level-1 positions (a 2TR x 2TC output tile).
//
// LDS: region A holds x with a zero border of KB/2 (row stride SX); after the
// base convolution it is reused for the bordered subbands of levels 2..L.
// Region B holds the four bordered level-1 subbands. Bordered planes have a
// zero border of K/2 and an odd row stride.
//
// IH x IW (at most H x W) is the plane in memory. A smaller one is zero-padded
// to H x W on chip (H, W multiples of 2^L) and only its own pixels are
// written: for a plane that 2^L does not divide this is exactly the layer's
// reading of odd band grids (each odd grid analysed with one extra zero row
// or column, each synthesis cropped), since the padded rows and columns only
// ever meet zeros and only feed outputs outside the plane.
template <int H_, int W_, int L_, int KB_, int K_, int NT_, int TR_, int TC_, int IH_ = H_, int IW_ = W_>
struct PlanePlan {
    static constexpr int H = H_, W = W_, L = L_, KB = KB_, K = K_, NT = NT_, TR = TR_, TC = TC_;
    static constexpr int IH = IH_, IW = IW_;
    static constexpr bool PADDED = IH != H || IW != W;
    static_assert(IH <= H && IW <= W && IH > H - (1 << L) && IW > W - (1 << L), "padding below one 2^L block");
    static constexpr int PB = KB / 2, PK = K / 2;
    static_assert(L >= 1, "the whole-plane kernel needs at least one level");
    static_assert(H % (1 << L) == 0 && W % (1 << L) == 0, "plane must divide into 2^L blocks");
    static_assert((H / 2) % TR == 0 && (W / 2) % TC == 0, "main tile must divide the level-1 grid");
    static_assert(KB % 2 == 1 && K % 2 == 1, "odd kernels only");
    static_assert(NT % 64 == 0 && NT <= 1024, "whole wavefronts");

    static constexpr int SX = odd_stride(W + 2 * PB);
    static constexpr int XSIZE = (H + 2 * PB) * SX;
    static constexpr int su(int l) { return odd_stride((W >> l) + 2 * PK); }
    static constexpr int bandsz(int l) { return ((H >> l) + 2 * PK) * su(l); }
    static constexpr int uoff(int l) {
        int o = 0;
        for (int q = 2; q < l; ++q) o += 4 * bandsz(q);
        return o;
    }
    static constexpr int UDEEP = uoff(L + 1);
    static constexpr int ASIZE = XSIZE > UDEEP ? XSIZE : UDEEP;
    static constexpr int BSIZE = 4 * bandsz(1);
    static constexpr int LDS_FLOATS = (ASIZE + BSIZE + 3) / 4 * 4;   // taps start 16-byte aligned
    static constexpr int KB2P = kpad4(KB), K2P = kpad4(K);
    static constexpr int WFLOATS = KB2P + 4 * L * K2P;   // staged taps
    static_assert((LDS_FLOATS + WFLOATS) * 4 <= 160 * 1024, "plane does not fit in LDS");
    static constexpr int NI = ((H / 2) / TR) * ((W / 2) / TC);
    static constexpr int MI = cdiv(NI, NT);

    static constexpr Tile deep_tile(int l) { return pick_tile(H >> l, W >> l, NT); }

    // occupancy the LDS footprint allows (waves per SIMD, at most 8). With a
    // kernel above 5x5 it is also held to what the registers of one output
    // tile need (its staged taps, the tile, a window row and about 40 more),
    // so that the allocator is never asked for fewer registers than that
    static constexpr int WG_PER_CU = (160 * 1024) / ((LDS_FLOATS + WFLOATS) * 4);
    static constexpr int WAVES_PER_EU_LDS = (WG_PER_CU * (NT / 64)) / 4;
    static constexpr int KMAX = KB > K ? KB : K;
    static constexpr int REGS = kpad4(KMAX) + MI * 4 * TR * TC + 2 * TC + KMAX + 40;
    static constexpr int WAVES_PER_EU_REG = KMAX <= 5 ? 8 : 512 / round_up(REGS, 8);
    static constexpr int WAVES_PER_EU_MIN = WAVES_PER_EU_LDS < WAVES_PER_EU_REG ? WAVES_PER_EU_LDS : WAVES_PER_EU_REG;
    static constexpr int WAVES_PER_EU =
        WAVES_PER_EU_MIN < 1 ? 1 : (WAVES_PER_EU_MIN > 8 ? 8 : WAVES_PER_EU_MIN);

    // f(std::integral_constant<int, l>) for l = 2..L, unrolled at compile time
    template <class F>
    __device__ static __forceinline__ void for_deep_levels(F&& f) {
        deep_impl(f, std::make_integer_sequence<int, (L >= 2 ? L - 1 : 0)>{});
    }
    template <class F, int... I>
    __device__ static __forceinline__ void deep_impl(F& f, std::integer_sequence<int, I...>) {
        (f(std::integral_constant<int, I + 2>{}), ...);
    }
};

// fin: an optional deferred weight-gradient second stage run as extra
// workgroups of the same launch (null: none)
typedef hipError_t (*plane_launch_fn)(const void* in, const float* w_base, const float* w_lvl,
                                      const float* scale, void* out, int B, int C,
                                      hipStream_t stream, const FinalizeArgs* fin);

struct PlaneEntry {
    int H, W, L, KB, K;   // the plane in memory (a padded plan's IH, IW)
    plane_launch_fn fn[2][2];  // [dtype: 0 fp32, 1 bf16][flip: 0 fwd, 1 bwd_data]
    int lds_bytes;
    int nt;
    int npw;   // images per workgroup: the kernel needs npw*C*H*W < 2^32
};

const PlaneEntry* find_plane_entry(int H, int W, int L, int KB, int K);

// ------------------------------------------------------------ the plans
// Micro-tile plans of planes that no column-strip plan covers: small shapes
// with other kernel sizes, odd tile counts and non-square planes.
typedef PlanePlan<32, 32, 2, 5, 5, 64, 2, 2> PP_32_L2_k55;
typedef PlanePlan<32, 32, 3, 7, 5, 64, 2, 2> PP_32_L3_k75;
typedef PlanePlan<24, 40, 3, 3, 3, 64, 2, 2> PP_24x40_L3_k33;
typedef PlanePlan<16, 16, 4, 3, 7, 64, 1, 1> PP_16_L4_k37;
typedef PlanePlan<64, 64, 4, 7, 5, 64, 4, 4> PP_64_L4_k75;

#define WTC_PLANE_ENTRIES(X)                                                                 \
    X(PP_32_L2_k55), X(PP_32_L3_k75), X(PP_24x40_L3_k33), X(PP_16_L4_k37), X(PP_64_L4_k75)

}  // namespace wtc

namespace wtc {

// Bank conflicts of the column-strip level convolution over a bordered band
// grid (hl x wl, border pk, 4 bands `pitch` floats apart, rows `S` floats
// apart): strip slot t holds band s, strip rs (r rows) and column j, with lp
// slots per strip (the slots past wl idle). The lanes of one 32-lane LDS pass
// read one row of each strip they hold; the cost sums, over the passes, the
// largest number of lanes that read the same bank.
constexpr int strip_conflicts(int hl, int wl, int r, int lp, int S, int pitch) {
    const int ns = hl / r, items = 4 * ns * lp;
    int cost = 0;
    for (int h0 = 0; h0 < items; h0 += 32) {
        int cnt[32] = {};
        int worst = 0;
        for (int t = h0; t < h0 + 32 && t < items; ++t) {
            const int s = t / (ns * lp), rem = t - s * (ns * lp), rs = rem / lp, j = rem - rs * lp;
            if (j >= wl) continue;
            const int b = (s * pitch + rs * r * S + j) % 32;
            if (++cnt[b] > worst) worst = cnt[b];
        }
        cost += worst;
    }
    return cost;
}

// Layout of a level's bands for the column-strip convolution: row stride s
// (at least the bordered width, even when asked), band pitch, and strip
// slots per strip lp.
//  - Strips narrower than 32 columns normally get a power of two of lanes
//    (strip_lanes), the rest idle. If dropping that padding saves whole
//    wavefronts, strips are packed back to back instead, with a stride and
//    pitch that put slot t on bank t + const (mod 32): r * s = wl and
//    pitch = (hl / r) * wl (mod 32), so no pass has a conflict.
//  - Otherwise the stride is the smallest with the fewest conflicts.
struct BandLayout {
    int s, pitch, lp;
};
constexpr BandLayout band_layout(int hl, int wl, int pk, int r, bool even) {
    const int w0 = wl + 2 * pk, base = even ? round_up(w0, 2) : w0, rows = hl + 2 * pk;
    const int lpad = strip_lanes(wl), ns = hl / r;
    if (lpad > wl && cdiv(4 * ns * wl, 64) < cdiv(4 * ns * lpad, 64)) {
        for (int S = base; S < base + 64; S += (even ? 2 : 1)) {
            if ((r * S - wl) % 32 != 0) continue;
            int pitch = rows * S;
            while ((pitch - ns * wl) % 32 != 0) ++pitch;
            if (even && pitch % 2 != 0) break;
            return BandLayout{S, pitch, wl};
        }
    }
    if (lpad >= 32) return BandLayout{base, rows * base, lpad};
    BandLayout best{base, rows * base, lpad};
    int best_cost = 1 << 30;
    for (int S = base; S < base + 64; S += (even ? 2 : 1)) {
        const int cost = strip_conflicts(hl, wl, r, lpad, S, rows * S);
        if (cost < best_cost) {
            best_cost = cost;
            best = BandLayout{S, rows * S, lpad};
        }
    }
    return best;
}

// Column-strip variant of the whole-plane plan: a lane computes RB rows x 1
// column of the base convolution, and RL rows x 1 column of one band at each
// level, so the lanes of a wavefront read consecutive LDS words (no bank
// conflicts) and write consecutive output columns. The level results go
// through LDS and one closed-form pass synthesises every output. Strips of
// a row block get strip_lanes(width) lanes (whole half-wavefronts or
// aligned groups), the rest idle.
//
// Base strips start on RB-row boundaries. The synthesis needs, for each
// level l, either whole 2^l-row blocks per strip (RB a multiple of 2^l) or a
// strip inside one block whose row bit l-1 is constant (RB a power of two
// below 2^l): RB is a multiple of 2^L or a power of two.
template <int H_, int W_, int L_, int KB_, int K_, int NT_, int RB_, int RL_, int WMAX_ = 8, int NPW_ = 1,
          bool PERSIST_ = false>
struct ColPlan {
    static constexpr int H = H_, W = W_, L = L_, KB = KB_, K = K_, NT = NT_, RB = RB_, RL = RL_;
    // persistent workgroups: as many as fit the chip at once, each taking
    // every such-many-th plane with the next plane's x rows and taps loaded
    // during the current one (planes whose LDS admits one workgroup per CU
    // otherwise expose each plane's load latency). For bf16 activations
    // only: fp32 ones take twice the prefetch registers (128x128 L3: a
    // spill).
    static constexpr bool PERSIST = PERSIST_;
    template <typename T>
    static constexpr bool persist() { return PERSIST && sizeof(T) == 2; }
    // planes per workgroup: NPW planes of one channel (consecutive images)
    // share the staged taps, and every phase packs its strips of all of
    // them onto the lanes (small planes otherwise leave lanes idle)
    static constexpr int NPW = NPW_;
    static constexpr int PB = KB / 2, PK = K / 2;
    static_assert(L >= 1 && H % (1 << L) == 0 && W % (1 << L) == 0, "plane must divide into 2^L blocks");
    static_assert(H % RB == 0, "base strips must divide the plane");
    static_assert(RB % (1 << L) == 0 || (RB & (RB - 1)) == 0, "base strips: a multiple of 2^L rows or a power of two");
    static_assert(NT % 64 == 0 && NT <= 1024, "whole wavefronts");
    // level-1 analysis items: 2 x rows by VA columns (VA / 2 Haar blocks),
    // over the bordered level-1 grid; the items on the border write the
    // zeros of the band border and of the x border
    static constexpr int VL = lds_vec(W);
    static constexpr int VA = VL >= 4 ? 4 : 2;
    // x rows: interior from column XO (a multiple of VA, at least KB/2), row
    // stride a multiple of VA: streamed rows take aligned VA-wide stores
    // (128-bit, or 64-bit on planes whose rows take pairs: there the
    // narrower border saves LDS, 14x14: a sixth workgroup per CU)
    static constexpr int XO = round_up(PB, VA);
    static constexpr int SX = round_up(XO + W + PB, VA);
    static constexpr int XSIZE = (H + 2 * PB) * SX;
    static constexpr int CPI = VA / 2;
    static constexpr int rl(int l) { return RL < (H >> l) ? RL : (H >> l); }
    // band rows: level-1 cell pairs are stored as aligned 64-bit words
    // (an even stride); see band_layout for the rest
    static constexpr BandLayout lay_calc(int l) {
        return l <= L ? band_layout(H >> l, W >> l, PK, rl(l), l == 1 && CPI == 2) : BandLayout{1, 1, 1};
    }
    // computed once per plan (each is a search)
    static constexpr BandLayout LAYS[6] = {BandLayout{1, 1, 1}, lay_calc(1), lay_calc(2),
                                           lay_calc(3), lay_calc(4), lay_calc(5)};
    static constexpr BandLayout lay(int l) { return LAYS[l]; }
    static constexpr int su(int l) { return lay(l).s; }
    static constexpr int bandsz(int l) { return lay(l).pitch; }   // band pitch
    static constexpr int IPR = ((W >> 1) + 2 * PK) / CPI;
    static constexpr int NQ = ((H >> 1) + 2 * PK) * IPR;
    // Small planes, where border items are the majority (14²: 72 of 121):
    // zero the planes' x and level-1 regions with plain vector stores first,
    // then run items over the interior only, when that saves a round of
    // items per thread. Measured: 14² forward and backward data 10 % faster;
    // at 28² (border 40 %) no gain, at 128² (11 %) 4 % slower.
    static constexpr int IPRI = (W >> 1) / CPI;
    static constexpr int NQI = (H >> 1) * IPRI;
    static constexpr bool ZFILL = cdiv(NPW * NQI, NT) < cdiv(NPW * NQ, NT) && NQ >= 2 * NQI;
    // Interior items on a power-of-two grid (pow2(H/2) rows of pow2(IPRI)
    // items per plane, the extra cells idle) where that takes no more
    // rounds per thread: plane, row and item then come from shifts and
    // masks instead of divisions by constants (14x14: 8 x 8 cells for 7 x 7
    // items, 512 of them on 256 threads as 392 were)
    static constexpr int IPRP = strip_lanes(IPRI < 32 ? IPRI : 32), NQP = strip_lanes((H >> 1) < 32 ? H >> 1 : 32) * IPRP;
    static constexpr bool QPOW2 = ZFILL && IPRI <= 32 && (H >> 1) <= 32 && cdiv(NPW * NQP, NT) == cdiv(NPW * NQI, NT);
    static_assert((W >> 1) % CPI == 0, "interior items tile the level-1 rows");
    static_assert(VL % 2 == 0, "rows of whole Haar blocks");
    static_assert(PK % CPI == 0 && (XO - 2 * PK) % VA == 0 && PB <= 2 * PK && XO + W + 2 * PK >= SX,
                  "analysis items cover the bordered x plane in whole vectors");
    static constexpr int uoff(int l) {
        int o = 0;
        for (int q = 2; q < l; ++q) o += 4 * bandsz(q);
        return o;
    }
    static constexpr int UDEEP = uoff(L + 1);
    static constexpr int ASIZE = XSIZE > UDEEP ? XSIZE : UDEEP;
    static constexpr int BSIZE = 4 * bandsz(1);
    static constexpr int LDS_FLOATS = (ASIZE + BSIZE + 3) / 4 * 4;   // one plane
    static constexpr int KB2P = kpad4(KB), K2P = kpad4(K);
    static constexpr int WFLOATS = KB2P + 4 * L * K2P;
    static constexpr int LPB = strip_lanes(W);
    static constexpr int NIB = (H / RB) * LPB;   // base strip slots of one plane
    static constexpr int MB = cdiv(NPW * NIB, NT);
    // rows per strip at level l, lanes per row block, strip slots (4 bands)
    static constexpr int lpl(int l) { return lay(l).lp; }
    static constexpr int nil(int l) { return 4 * ((H >> l) / rl(l)) * lpl(l); }
    // levels 2..L share one register strip per thread when all their strip
    // slots fit the workgroup: level l takes threads [doff(l), doff(l) + nil(l)),
    // from the first whole wavefront after level 1's strips when one round
    // of those leaves room for them all (the deep strips then fall on
    // wavefronts that level 1 leaves idle), else from thread 0
    static constexpr int ddeep(int l) {
        int o = 0;
        for (int q = 2; q < l; ++q) o += NPW * nil(q);
        return o;
    }
    static constexpr int DBASE =
        (NPW * nil(1) <= NT && round_up(NPW * nil(1), 64) + ddeep(L + 1) <= NT) ? round_up(NPW * nil(1), 64) : 0;
    static constexpr int doff(int l) { return DBASE + ddeep(l); }
    static constexpr bool DSHARE = L >= 2 && doff(L + 1) <= NT;
    static constexpr int RLD = L >= 2 ? rl(2) : 1;
    // Level 1 beside the base convolution. With one level nothing overwrites
    // x before the synthesis, so when one round of base strips leaves whole
    // wavefronts idle (threads from NBL on), the level-1 strips run there in
    // the same phase, if that shortens the busiest wavefront's multiply-adds
    // (14x14: 350 on every wavefront instead of 525 on the base ones and 175
    // on the others).
    static constexpr int NBL = round_up(NPW * NIB, 64);
    static constexpr int conc1_cost() {
        const int base = RB * KB * KB, lv = cdiv(NPW * nil(1), NT - NBL) * rl(1) * K * K;
        return base > lv ? base : lv;
    }
    static constexpr bool CONC1 = L == 1 && MB == 1 && NT - NBL >= 64 &&
                                  conc1_cost() < RB * KB * KB + cdiv(NPW * nil(1), NT) * rl(1) * K * K;
    // occupancy the LDS footprint allows, at most WMAX waves per SIMD (a
    // plan whose registers need more than 512 / WMAX lowers WMAX)
    // planes of a workgroup lie PL floats apart: a multiple of 4 (128-bit
    // stores) at most 28 above one plane's size, placed so that the base and
    // level-1 strips of neighbouring planes sharing a 32-lane pass fall on
    // different banks
    static constexpr int pass_conflicts(int pl) {
        int cost = 0;
        for (int h0 = 0; h0 < NPW * NIB; h0 += 32) {   // base strips, first window row
            int cnt[32] = {};
            int worst = 0;
            for (int t = h0; t < h0 + 32 && t < NPW * NIB; ++t) {
                const int p = t / NIB, r = t - p * NIB, rb = r / LPB, w = r - rb * LPB;
                if (w >= W) continue;
                const int b = (p * pl + rb * RB * SX + w) % 32;
                if (++cnt[b] > worst) worst = cnt[b];
            }
            cost += worst;
        }
        const int n1 = nil(1), ns = (H >> 1) / rl(1), lp = lpl(1);
        for (int h0 = 0; h0 < NPW * n1; h0 += 32) {   // level-1 strips
            int cnt[32] = {};
            int worst = 0;
            for (int t = h0; t < h0 + 32 && t < NPW * n1; ++t) {
                const int p = t / n1, r = t - p * n1, s = r / (ns * lp), rem = r - s * (ns * lp);
                const int rs = rem / lp, j = rem - rs * lp;
                if (j >= (W >> 1)) continue;
                const int b = (p * pl + ASIZE + s * bandsz(1) + rs * rl(1) * su(1) + j) % 32;
                if (++cnt[b] > worst) worst = cnt[b];
            }
            cost += worst;
        }
        return cost;
    }
    static constexpr int plane_pitch() {
        if (NPW == 1) return LDS_FLOATS;
        int best = LDS_FLOATS, best_cost = pass_conflicts(LDS_FLOATS);
        for (int pl = LDS_FLOATS + 4; pl < LDS_FLOATS + 32; pl += 4)
            if (pass_conflicts(pl) < best_cost) {
                best_cost = pass_conflicts(pl);
                best = pl;
            }
        return best;
    }
    static constexpr int PL = plane_pitch();
    static constexpr int TOTAL_FLOATS = NPW * PL + WFLOATS;   // planes, then the taps
    static_assert(TOTAL_FLOATS * 4 <= 160 * 1024, "planes do not fit in LDS");
    static constexpr int WG_PER_CU = (160 * 1024) / (TOTAL_FLOATS * 4);
    static constexpr int WAVES_PER_EU_LDS = (WG_PER_CU * (NT / 64)) / 4;
    static constexpr int WAVES_PER_EU =
        WAVES_PER_EU_LDS < 1 ? 1 : (WAVES_PER_EU_LDS > WMAX_ ? WMAX_ : WAVES_PER_EU_LDS);

    template <class F>
    __device__ static __forceinline__ void for_levels(F&& f) {
        lv_impl(f, std::make_integer_sequence<int, L>{});
    }
    template <class F, int... I>
    __device__ static __forceinline__ void lv_impl(F& f, std::integer_sequence<int, I...>) {
        (f(std::integral_constant<int, I + 1>{}), ...);
    }
    template <class F>
    __device__ static __forceinline__ void for_deep_levels(F&& f) {
        deep_impl(f, std::make_integer_sequence<int, (L >= 2 ? L - 1 : 0)>{});
    }
    template <class F, int... I>
    __device__ static __forceinline__ void deep_impl(F& f, std::integer_sequence<int, I...>) {
        (f(std::integral_constant<int, I + 2>{}), ...);
    }
};

}  // namespace wtc

namespace wtc {
// Column-strip plans of the ConvNeXt stage planes and the 128x128 level
// sweep. Measured choices: the 56x56 plan runs 8 waves per SIMD (64 VGPRs);
// small planes put several images of one channel in a workgroup (28x28: two,
// 14x14: eight) with strips packed across them; 128x128 uses 16-row base
// and level strips on 1024 lanes.
typedef ColPlan<56, 56, 3, 5, 5, 512, 8, 7, 8> CP_56_L3_k55;
typedef ColPlan<28, 28, 2, 5, 5, 256, 4, 14, 8, 2> CP_28_L2_k55;
typedef ColPlan<14, 14, 1, 5, 5, 256, 14, 7, 8, 8> CP_14_L1_k55;
// Persistent (bf16 activations), against one workgroup per plane on one
// box: level-sweep step 0.488 -> 0.455, 0.536 -> 0.506 and 0.548 -> 0.539
// ms at L = 2, 4, 5 (L = 5 keeps a 12-byte spill and still gains); at L = 1
// and 3 0.398 -> 0.377 and 0.525 -> 0.505 ms with every stream-in item
// prefetched, a further 1 % with the interior items only.
typedef ColPlan<128, 128, 1, 5, 5, 1024, 16, 16, 8, 1, true> CP_128_L1_k55;
typedef ColPlan<128, 128, 2, 5, 5, 1024, 16, 16, 8, 1, true> CP_128_L2_k55;
typedef ColPlan<128, 128, 3, 5, 5, 1024, 16, 16, 8, 1, true> CP_128_L3_k55;
typedef ColPlan<128, 128, 4, 5, 5, 1024, 16, 16, 8, 1, true> CP_128_L4_k55;
typedef ColPlan<128, 128, 5, 5, 5, 1024, 16, 16, 8, 1, true> CP_128_L5_k55;
#define WTC_COL_ENTRIES(X)                                                                     \
    X(CP_56_L3_k55), X(CP_28_L2_k55), X(CP_14_L1_k55), X(CP_128_L1_k55), X(CP_128_L2_k55),     \
        X(CP_128_L3_k55), X(CP_128_L4_k55), X(CP_128_L5_k55)
}  // namespace wtc
