// Fused kernels for the ConvNeXt stage-plane family: planes of 56, 28, 14
// and 7 pixels square, L = 1 .. min(4, log2 H) levels, base kernels 5 and 7,
// level kernels 3, 5 and 7 (the WTConvNeXt setting the abstract evaluates,
// over decomposition levels and tensor shapes). Each member gets:
//  - forward / backward data: the column-strip kernel where its stream-in
//    layout admits the kernel sizes (level kernel 5 on 56x56 and 28x28, and
//    the 14x14 cases checked by col_fits), else the micro-tile whole-plane
//    kernel; a plane that 2^L does not divide runs zero-padded to the next
//    multiple of 2^L (exactly the odd-grid reading of the layer);
//  - backward weight: the whole-plane weight-gradient kernel, padded alike.
// The tuned plans of the benchmark shapes are listed first in the main
// registries and take precedence over these.
#pragma once

#include "wtconv_bwdw_body.h"
#include "wtconv_plane.h"

namespace wtc {

constexpr int fam_pad(int h, int L) { return round_up(h, 1 << L); }

// Column-strip plan parameters per plane size (the tuned values of the
// stage shapes): threads, base rows, level rows, waves cap, images per group.
// A 7x7 base kernel's staged taps take 24 registers more than a 5x5 one's:
// the 56x56 plan then runs at most 5 waves per SIMD instead of 8.
struct ColShape {
    int nt, rb, rl, wmax, npw;
};
constexpr ColShape col_shape(int h, int kb = 5) {
    return h == 56 ? ColShape{512, 8, 7, kb > 5 ? 5 : 8, 1}
                   : h == 28 ? ColShape{256, 4, 14, 8, 2} : ColShape{256, 14, 7, 8, 8};
}

// Whether the column-strip kernel's stream-in covers this member: its items
// cover the bordered level-1 grid in whole x vectors (the conditions the
// column plan asserts), the base strips fit the levels, and the plane divides.
constexpr bool col_fits(int h, int L, int kb, int k) {
    if (h != 56 && h != 28 && h != 14) return false;
    if (h % (1 << L) != 0) return false;
    const ColShape cs = col_shape(h);
    if (h % cs.rb != 0 || !(cs.rb % (1 << L) == 0 || (cs.rb & (cs.rb - 1)) == 0)) return false;
    const int pb = kb / 2, pk = k / 2, vl = lds_vec(h), va = vl >= 4 ? 4 : 2, cpi = va / 2;
    const int xo = round_up(pb, va), sx = round_up(xo + h + pb, va);
    return (h / 2) % cpi == 0 && pk % cpi == 0 && (xo - 2 * pk) % va == 0 && xo <= 2 * pk && pb <= 2 * pk &&
           xo + h + 2 * pk >= sx;
}

// Micro-tile whole-plane plan for a padded plane of h x h: the smallest
// output tile whose items fit 256 threads.
struct TileShape {
    int nt, tr, tc;
};
constexpr TileShape tile_shape(int h) {
    const int h1 = h / 2;
    const int cand[6][2] = {{1, 1}, {1, 2}, {2, 2}, {1, 4}, {2, 4}, {4, 4}};
    for (int i = 0; i < 6; ++i) {
        const int tr = cand[i][0], tc = cand[i][1];
        if (h1 % tr != 0 || h1 % tc != 0) continue;
        const int items = (h1 / tr) * (h1 / tc);
        if (items <= 256) return TileShape{round_up(items, 64), tr, tc};
    }
    return TileShape{256, 4, 4};
}

template <int IH, int L, int KB, int K>
struct FamCol {
    static constexpr ColShape cs = col_shape(IH, KB);
    using type = ColPlan<IH, IH, L, KB, K, cs.nt, cs.rb, cs.rl, cs.wmax, cs.npw>;
};
template <int IH, int L, int KB, int K>
struct FamTile {
    static constexpr int HP = fam_pad(IH, L);
    static constexpr TileShape ts = tile_shape(HP);
    using type = PlanePlan<HP, HP, L, KB, K, ts.nt, ts.tr, ts.tc, IH, IH>;
};

// planes per step of the weight-gradient plan: its analysis lanes
// ((h/2) x (h/cw) per plane) fill up to 512 threads, at most 8 planes
constexpr int bw_planes(int h) {
    const int cw = h % 4 == 0 ? 4 : 2, na = (h / 2) * (h / cw);
    int n = 512 / na;
    return n > 8 ? 8 : (n < 1 ? 1 : n);
}
// At L = 1 one whole-plane pass; at L >= 2 the level split of the stage-1
// plan: base and level 1 on the (padded) plane, which also writes its
// level-1 LL planes, then levels 2..L on those in the same workgroup. A
// lane then keeps one tap slot in the first pass and at most two in the
// second (three 7x7 slots in one pass do not fit the registers).
template <int IH, int L, int KB, int K>
struct FamBw {
    static constexpr int HP = fam_pad(IH, L), NPB = bw_planes(HP);
    // registers beside the tap slots: strips and addresses, more with
    // several planes per step
    using fine = BwPlan<HP, HP, 1, KB, K, L, NPB, IH, IH, 56 + 8 * NPB>;
    static constexpr int LC = L > 1 ? L - 1 : 1, NPBC = bw_planes(HP / 2);
    using coarse = BwPlan<HP / 2, HP / 2, LC, 1, K, LC, NPBC, HP / 2, HP / 2, 56 + 8 * NPBC>;
};

// The members of one plane size, as X(IH, L, KB, K).
#define WTC_FAM_KERNELS(X, IH, L) \
    X(IH, L, 5, 3), X(IH, L, 5, 5), X(IH, L, 5, 7), X(IH, L, 7, 3), X(IH, L, 7, 5), X(IH, L, 7, 7)
#define WTC_FAM_56(X) WTC_FAM_KERNELS(X, 56, 1), WTC_FAM_KERNELS(X, 56, 2), WTC_FAM_KERNELS(X, 56, 3), WTC_FAM_KERNELS(X, 56, 4)
#define WTC_FAM_28(X) WTC_FAM_KERNELS(X, 28, 1), WTC_FAM_KERNELS(X, 28, 2), WTC_FAM_KERNELS(X, 28, 3), WTC_FAM_KERNELS(X, 28, 4)
#define WTC_FAM_14(X) WTC_FAM_KERNELS(X, 14, 1), WTC_FAM_KERNELS(X, 14, 2), WTC_FAM_KERNELS(X, 14, 3)
#define WTC_FAM_7(X) WTC_FAM_KERNELS(X, 7, 1), WTC_FAM_KERNELS(X, 7, 2)

// Registry entries of one member (the launchers instantiate its kernels).
template <int IH, int L, int KB, int K>
constexpr PlaneEntry fam_data_entry() {
    if constexpr (col_fits(IH, L, KB, K)) {
        using P = typename FamCol<IH, L, KB, K>::type;
        return PlaneEntry{IH, IH, L, KB, K,
                          {{launch_col<P, float, false>, launch_col<P, float, true>},
                           {launch_col<P, bf16_t, false>, launch_col<P, bf16_t, true>}},
                          P::TOTAL_FLOATS * 4, P::NT, P::NPW};
    } else {
        using P = typename FamTile<IH, L, KB, K>::type;
        return PlaneEntry{IH, IH, L, KB, K,
                          {{launch_plane<P, float, false>, launch_plane<P, float, true>},
                           {launch_plane<P, bf16_t, false>, launch_plane<P, bf16_t, true>}},
                          (P::LDS_FLOATS + P::WFLOATS) * 4, P::NT, 1};
    }
}
template <int IH, int L, int KB, int K>
constexpr BwEntry fam_bw_entry() {
    using F = typename FamBw<IH, L, KB, K>::fine;
    using G = typename FamBw<IH, L, KB, K>::coarse;
    if constexpr (L == 1)
        return BwEntry{IH, IH, L, KB, K, {whole_launch<F, float>, whole_launch<F, bf16_t>}, whole_ws<F>};
    else
        return BwEntry{IH, IH, L, KB, K, {plane_split_launch<F, G, float>, plane_split_launch<F, G, bf16_t>},
                       plane_split_ws<F, G>};
}
#define WTC_FAM_DATA(IH, L, KB, K) fam_data_entry<IH, L, KB, K>()
#define WTC_FAM_BW(IH, L, KB, K) fam_bw_entry<IH, L, KB, K>()

// First entry of `table` (n entries) for this shape, or null.
template <class E>
const E* fam_find(const E* table, int n, int H, int W, int L, int KB, int K) {
    for (int i = 0; i < n; ++i) {
        const E& e = table[i];
        if (e.H == H && e.W == W && e.L == L && e.KB == KB && e.K == K) return &e;
    }
    return nullptr;
}

// the tables of each plane size (one translation unit each, so that they
// compile in parallel)
const PlaneEntry* find_fam56_data(int H, int W, int L, int KB, int K);
const PlaneEntry* find_fam28_data(int H, int W, int L, int KB, int K);
const PlaneEntry* find_fam14_data(int H, int W, int L, int KB, int K);
const PlaneEntry* find_fam7_data(int H, int W, int L, int KB, int K);
const BwEntry* find_fam56_bw(int H, int W, int L, int KB, int K);
const BwEntry* find_fam28_bw(int H, int W, int L, int KB, int K);
const BwEntry* find_fam14_bw(int H, int W, int L, int KB, int K);
const BwEntry* find_fam7_bw(int H, int W, int L, int KB, int K);

inline const PlaneEntry* find_family_plane_entry(int H, int W, int L, int KB, int K) {
    if (H != W) return nullptr;
    switch (H) {
    case 56: return find_fam56_data(H, W, L, KB, K);
    case 28: return find_fam28_data(H, W, L, KB, K);
    case 14: return find_fam14_data(H, W, L, KB, K);
    case 7: return find_fam7_data(H, W, L, KB, K);
    default: return nullptr;
    }
}
inline const BwEntry* find_family_bw_entry(int H, int W, int L, int KB, int K) {
    if (H != W) return nullptr;
    switch (H) {
    case 56: return find_fam56_bw(H, W, L, KB, K);
    case 28: return find_fam28_bw(H, W, L, KB, K);
    case 14: return find_fam14_bw(H, W, L, KB, K);
    case 7: return find_fam7_bw(H, W, L, KB, K);
    default: return nullptr;
    }
}

}  // namespace wtc
