// Whole-plane WTConv forward / backward-data kernel for gfx950: one workgroup owns
// one (b, c) plane, which lives in LDS together with its Haar pyramid.
//
// The abstract of arXiv:2608.10805 ("I/O-aware reformulation of wavelet
// convolution", Abstract) names three reformulations; all three are used:
//  (1) the Haar analysis butterfly is recomputed on chip from x: x is read
//      from HBM once and no subband ever leaves LDS;
//  (2) the synthesis cascade is one closed-form pass: level l adds
//        sum_s sign_s(bit_{l-1} h, bit_{l-1} w) * Z'_l^s[h >> l][w >> l]
//      to output pixel (h, w), where sign_s is the band's +-1 pattern;
//  (3) the per-(level, channel, band) scale and the Haar normalisation
//      4^-l are folded into each band's convolution result, so
//      Z'_l^s = 4^-l * scale * corr(U_l^s, w) with U_l the unnormalised band.
// y is written to HBM once. Backward data runs the same kernel with every
// kernel turned by 180 degrees (the layer's transpose).
//
// Phases (barriers between them):
//  P0  zero LDS borders, stream x into LDS (fp32, zero border k_base/2)
//  P1  per main item (a TR x TC tile of level-1 positions = a 2TR x 2TC
//      output tile): base convolution into registers, level-1 analysis into
//      LDS region B
//  P2  levels 2..L: analysis from the LL band below, into region A (x is dead)
//  P3  levels 2..L: per-band convolution into registers, then written over
//      their own subbands in LDS
//  P4  per main item: level-1 convolution of the four bands in registers,
//      closed-form synthesis of all levels, one store of y.
#pragma once

#include "wtconv_device.h"
#include "wtconv_plans.h"

namespace wtc {
// SUMS (with SHIFT > 0): `in` already holds the fp32 plane of 2^SHIFT x
// 2^SHIFT block sums (as the weight-gradient pass leaves them), so it is
// loaded as it is instead of being summed from the full-size activations.
//
// Workgroups from `nplanes` on run a deferred weight-gradient second stage
// (fin.C channels) instead: see FinalizeArgs.
template <class P, typename T, bool FLIP, int SHIFT, typename TO, bool SUMS = false>
__global__ __launch_bounds__(P::NT) __attribute__((amdgpu_waves_per_eu(P::WAVES_PER_EU))) void plane_kernel(const T* __restrict__ in,
                                                      const float* __restrict__ w_base,
                                                      const float* __restrict__ w_lvl,
                                                      const float* __restrict__ scale,
                                                      TO* __restrict__ out, int C,
                                                      unsigned nplanes, FinalizeArgs fin) {
    constexpr int H = P::H, W = P::W, L = P::L, KB = P::KB, K = P::K, NT = P::NT;
    constexpr int TR = P::TR, TC = P::TC, PB = P::PB, PK = P::PK;
    constexpr int SX = P::SX, H1 = H / 2, W1 = W / 2;
    constexpr int S1 = P::su(1), BS1 = P::bandsz(1);
    constexpr int NI = P::NI, MI = P::MI, TPR = W1 / TC;

    __shared__ __attribute__((aligned(16))) float lds[P::LDS_FLOATS + P::WFLOATS];
    if (blockIdx.x >= nplanes) {   // a deferred second stage of the weight gradient
        finalize_channel(fin, (int)(blockIdx.x - nplanes), threadIdx.x, P::NT, lds);
        return;
    }
    float* A = lds;               // x (bordered), later U_2..U_L and Z'_2..Z'_L
    float* Bq = lds + P::ASIZE;   // U_1 (4 bordered bands)
    float* WB = lds + P::LDS_FLOATS;   // base taps (turned for FLIP), padded to KB2P
    float* WL = WB + P::KB2P;          // level taps x scale x 4^-l, [L][4][K2P]

    constexpr bool BASE = SHIFT == 0;
    constexpr int IH = P::IH, IW = P::IW;   // the plane in memory (zero-padded to H x W here)
    static_assert(!P::PADDED || SHIFT == 0, "padded planes are whole planes");
    static_assert(!SUMS || (SHIFT > 0 && sizeof(T) == 4), "block sums are fp32 planes of a coarse pass");
    const int tid = threadIdx.x;
    const int plane = blockIdx.x;
    const int c = plane % C;
    const T* __restrict__ src = in + ((size_t)plane * IH * IW << (SUMS ? 0 : 2 * SHIFT));
    TO* __restrict__ dst = out + (size_t)plane * IH * IW;

    // ---------------------------------------------------------------- P0
    // stage the taps: turned by 180 degrees for the transpose, and the level
    // taps scaled by scale * 4^-l (reformulation (3)); padding taps are zero
    constexpr int KB2P = P::KB2P, K2P = P::K2P;
    if constexpr (BASE)
        for (int t = tid; t < KB2P; t += NT)
            WB[t] = t < KB * KB ? w_base[(size_t)c * KB * KB + (FLIP ? KB * KB - 1 - t : t)] : 0.f;
    for (int t = tid; t < 4 * L * K2P; t += NT) {
        const int ls = t / K2P, tap = t - ls * K2P, l = ls >> 2, s = ls & 3;
        const size_t pi = ((size_t)l * C + c) * 4 + s;
        const float f = scale[pi] * (1.0f / (float)(1 << (2 * (l + 1 + SHIFT))));
        WL[t] = tap < K * K ? w_lvl[pi * K * K + (FLIP ? K * K - 1 - tap : tap)] * f : 0.f;
    }
    zero_border<1, H, W, PB, SX>(A, tid, NT);
    zero_border<4, H1, W1, PK, S1>(Bq, tid, NT);
    if constexpr (P::PADDED) {
        // the padded rows and columns of x: zero (the plane's own pixels,
        // stored below, are other cells)
        for (int i = tid; i < H * W; i += NT) {
            const int r = i / W, col = i - r * W;
            if (r >= IH || col >= IW) A[(r + PB) * SX + col + PB] = 0.f;
        }
    }
    if constexpr (SHIFT == 0 || SUMS) {
        // every global load of the plane is issued before the first LDS
        // write, so the HBM latency is paid once per plane
        constexpr int V = vec_elems<T>(IW, IH * IW);
        constexpr int NV = IH * IW / V;
        constexpr int NL = cdiv(NV, NT);
        float v[NL][V];
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int q = tid + k * NT;
            if (NV % NT == 0 || q < NV) load_vec<T, V>(src + q * V, v[k]);
        }
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int q = tid + k * NT;
            if (NV % NT == 0 || q < NV) {
                const int e = q * V, r = e / IW, col = e - r * IW;
#pragma unroll
                for (int i = 0; i < V; ++i) A[(r + PB) * SX + col + PB + i] = v[k][i];
            }
        }
    } else {
        // P[i][j] = sum of the 2^SHIFT x 2^SHIFT block of x at (i, j): one
        // thread per block, 2^SHIFT-element row segments (lanes of a wave
        // read consecutive segments of the same rows). The sum runs in the
        // order of the Haar analysis's LL chain, (a + b) + (c + d) per 2x2
        // group, level by level: exactly the unnormalised LL band the
        // weight-gradient pass computes, so that its sums can stand in for
        // these bit for bit.
        constexpr int BS = 1 << SHIFT, WF = W << SHIFT;
        static_assert(BS * Act<T>::BYTES <= 16, "block row must fit one vector load");
        constexpr int NBLK = H * W, NL = cdiv(NBLK, NT);
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            const int q = tid + k * NT;
            if (NBLK % NT == 0 || q < NBLK) {
                const int i = q / W, j = q - i * W;
                float v[BS][BS];
#pragma unroll
                for (int u = 0; u < BS; ++u) load_vec<T, BS>(src + (size_t)(i * BS + u) * WF + j * BS, v[u]);
#pragma unroll
                for (int st = 1; st < BS; st *= 2)
#pragma unroll
                    for (int r = 0; r < BS; r += 2 * st)
#pragma unroll
                        for (int cc = 0; cc < BS; cc += 2 * st)
                            v[r][cc] = (v[r][cc] + v[r][cc + st]) + (v[r + st][cc] + v[r + st][cc + st]);
                A[(i + PB) * SX + j + PB] = v[0][0];
            }
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- P1
    float yb[MI][2 * TR][2 * TC];
#pragma unroll
    for (int it = 0; it < MI; ++it) {
        const int item = tid + it * NT;
#pragma unroll
        for (int r = 0; r < 2 * TR; ++r)
#pragma unroll
            for (int q = 0; q < 2 * TC; ++q) yb[it][r][q] = 0.f;
        if (item < NI) {
            const int ti = item / TPR, tj = item - ti * TPR;
            const int h0 = 2 * TR * ti, w0 = 2 * TC * tj;
            if constexpr (BASE) conv_tile<KB, 2 * TR, 2 * TC, SX>(A + h0 * SX + w0, WB, yb[it]);
            const int i0 = TR * ti, j0 = TC * tj;
#pragma unroll
            for (int r = 0; r < TR; ++r)
#pragma unroll
                for (int q = 0; q < TC; ++q) {
                    const float* x2 = A + (PB + 2 * (i0 + r)) * SX + PB + 2 * (j0 + q);
                    float b[4];
                    haar4(x2[0], x2[1], x2[SX], x2[SX + 1], b[0], b[1], b[2], b[3]);
                    const int o = (PK + i0 + r) * S1 + PK + j0 + q;
#pragma unroll
                    for (int s = 0; s < 4; ++s) Bq[s * BS1 + o] = b[s];
                }
        }
    }
    __syncthreads();

    // ---------------------------------------------------------------- P2
    P::for_deep_levels([&](auto lc) {
        constexpr int l = decltype(lc)::value;
        constexpr int hl = H >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l);
        constexpr int Sp = P::su(l - 1), BSp = P::bandsz(l - 1);
        float* Ul = A + P::uoff(l);
        const float* LLp = (l == 2) ? (Bq + PK * Sp + PK) : (A + P::uoff(l - 1) + PK * Sp + PK);
        (void)BSp;
        zero_border<4, hl, wl, PK, Sl>(Ul, tid, NT);
        for (int q = tid; q < hl * wl; q += NT) {
            const int i = q / wl, j = q - i * wl;
            const float* x2 = LLp + 2 * i * Sp + 2 * j;
            float b[4];
            haar4(x2[0], x2[1], x2[Sp], x2[Sp + 1], b[0], b[1], b[2], b[3]);
            const int o = (PK + i) * Sl + PK + j;
#pragma unroll
            for (int s = 0; s < 4; ++s) Ul[s * BSl + o] = b[s];
        }
        __syncthreads();
    });

    // ---------------------------------------------------------------- P3
    P::for_deep_levels([&](auto lc) {
        constexpr int l = decltype(lc)::value;
        constexpr int hl = H >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l);
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
            for (int s = 0; s < 4; ++s) {
#pragma unroll
                for (int r = 0; r < RR; ++r)
#pragma unroll
                    for (int q = 0; q < CC; ++q) z[it][s][r][q] = 0.f;
                if (item < NIl)
                    conv_tile<K, RR, CC, Sl>(Ul + s * BSl + RR * ti * Sl + CC * tj,
                                             WL + ((l - 1) * 4 + s) * K2P, z[it][s]);
            }
        }
        __syncthreads();
#pragma unroll
        for (int it = 0; it < MIl; ++it) {
            const int item = tid + it * NT;
            if (item < NIl) {
                const int ti = item / TPRl, tj = item - ti * TPRl;
#pragma unroll
                for (int s = 0; s < 4; ++s)
#pragma unroll
                    for (int r = 0; r < RR; ++r)
#pragma unroll
                        for (int q = 0; q < CC; ++q)
                            Ul[s * BSl + (PK + RR * ti + r) * Sl + PK + CC * tj + q] = z[it][s][r][q];
            }
        }
    });
    if constexpr (L >= 2) __syncthreads();

    // ---------------------------------------------------------------- P4
#pragma unroll
    for (int it = 0; it < MI; ++it) {
        const int item = tid + it * NT;
        if (item >= NI) continue;
        const int ti = item / TPR, tj = item - ti * TPR;
        const int i0 = TR * ti, j0 = TC * tj;
        float z1[4][TR][TC];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
            for (int r = 0; r < TR; ++r)
#pragma unroll
                for (int q = 0; q < TC; ++q) z1[s][r][q] = 0.f;
            conv_tile<K, TR, TC, S1>(Bq + s * BS1 + i0 * S1 + j0, WL + s * K2P, z1[s]);
        }
#pragma unroll
        for (int r = 0; r < TR; ++r) {
            float row0[2 * TC], row1[2 * TC];
#pragma unroll
            for (int q = 0; q < TC; ++q) {
                const int i = i0 + r, j = j0 + q;
                // coarser levels: constant over the 2x2 output block of (i, j)
                float e = 0.f;
                P::for_deep_levels([&](auto lc) {
                    constexpr int l = decltype(lc)::value;
                    constexpr int Sl = P::su(l), BSl = P::bandsz(l);
                    const float* Zl = A + P::uoff(l) + (PK + (i >> (l - 1))) * Sl + PK + (j >> (l - 1));
                    const bool bi = (i >> (l - 2)) & 1, bj = (j >> (l - 2)) & 1;
                    const float a0 = Zl[0], a1 = Zl[BSl], a2 = Zl[2 * BSl], a3 = Zl[3 * BSl];
                    e += a0 + (bi ? -a1 : a1) + (bj ? -a2 : a2) + ((bi != bj) ? -a3 : a3);
                });
                const float p0 = z1[0][r][q], p1 = z1[1][r][q], p2 = z1[2][r][q], p3 = z1[3][r][q];
                row0[2 * q] = yb[it][2 * r][2 * q] + (p0 + p1 + p2 + p3) + e;
                row0[2 * q + 1] = yb[it][2 * r][2 * q + 1] + (p0 + p1 - p2 - p3) + e;
                row1[2 * q] = yb[it][2 * r + 1][2 * q] + (p0 - p1 + p2 - p3) + e;
                row1[2 * q + 1] = yb[it][2 * r + 1][2 * q + 1] + (p0 - p1 - p2 + p3) + e;
            }
            const int h = 2 * (i0 + r), w0 = 2 * j0;
            if constexpr (!P::PADDED) {
                store_row<2 * TC>(dst + (size_t)h * W + w0, row0);
                store_row<2 * TC>(dst + (size_t)(h + 1) * W + w0, row1);
            } else {
                // the plane's own pixels only (the crop of the padded plane)
#pragma unroll
                for (int q = 0; q < 2 * TC; ++q) {
                    if (w0 + q >= IW) continue;
                    if (h < IH) store_one(dst + (size_t)h * IW + w0 + q, row0[q]);
                    if (h + 1 < IH) store_one(dst + (size_t)(h + 1) * IW + w0 + q, row1[q]);
                }
            }
        }
    }
}

// fin: a weight-gradient second stage to run as extra workgroups (its
// channels after the planes), or null
template <class P, typename T, bool FLIP, int SHIFT, bool SUMS = false>
hipError_t launch_coarse(const void* in, const float* wl, const float* sc, float* out, int B, int C,
                         hipStream_t stream, const FinalizeArgs* fin = nullptr) {
    const unsigned planes = (unsigned)B * (unsigned)C, extra = fin ? (unsigned)fin->C : 0u;
    hipLaunchKernelGGL((plane_kernel<P, T, FLIP, SHIFT, float, SUMS>), dim3(planes + extra), dim3(P::NT), 0, stream,
                       (const T*)in, (const float*)nullptr, wl, sc, out, C, planes, fin ? *fin : FinalizeArgs{});
    return hipGetLastError();
}

}  // namespace wtc

namespace wtc {

// Whole-plane forward / backward-data kernel, column-strip work split (see
// ColPlan). Same phases and LDS regions as plane_kernel; P3 convolves every
// level (level 1 included) into registers and writes the results over their
// own subbands, P4 synthesises each output column strip in closed form.
// Workgroups from cdiv(B, NPW) * C on run a deferred weight-gradient second
// stage (fin.C channels) instead: see FinalizeArgs.
template <class P, typename T, bool FLIP>
__global__ __launch_bounds__(P::NT) __attribute__((amdgpu_waves_per_eu(P::WAVES_PER_EU)))
void col_kernel(const T* __restrict__ in, const float* __restrict__ w_base, const float* __restrict__ w_lvl,
                const float* __restrict__ scale, T* __restrict__ out, int B, int C, FinalizeArgs fin) {
    constexpr int H = P::H, W = P::W, L = P::L, KB = P::KB, K = P::K, NT = P::NT, RB = P::RB;
    constexpr int PB = P::PB, PK = P::PK, SX = P::SX, H1 = H / 2, W1 = W / 2;
    constexpr int S1 = P::su(1), BS1 = P::bandsz(1);
    constexpr int NIB = P::NIB, MB = P::MB, LPB = P::LPB, XO = P::XO, VL = P::VL;
    constexpr int KB2P = P::KB2P, K2P = P::K2P, NPW = P::NPW, PL = P::PL;

    __shared__ __attribute__((aligned(16))) float lds[P::TOTAL_FLOATS];
    float* WB = lds + NPW * PL;
    float* WL = WB + KB2P;

    const int tid = threadIdx.x;
    constexpr bool PERS = P::template persist<T>();
    // Groups: channel c of images g*NPW .. g*NPW + NPW-1 (those < B), group
    // index g*C + c. One workgroup per group, or (PERSIST) the launch's
    // first ndata workgroups, each taking every ndata-th group from its own
    // index with the next group's loads in flight during the current one.
    const unsigned ngroups = (unsigned)cdiv(B, NPW) * (unsigned)C;
    const unsigned ndata = PERS ? gridDim.x - (unsigned)fin.C : ngroups;
    if (blockIdx.x >= ndata) {   // a deferred second stage of the weight gradient
        finalize_channel(fin, (int)(blockIdx.x - ndata), tid, NT, lds);
        return;
    }
    // A group's first plane is a uniform base; plane p lies p*C*H*W
    // elements further on. The host routes shapes whose NPW*C*H*W reaches
    // 2^32 elsewhere, so per-lane offsets stay 32-bit and the loads and
    // stores take the scalar-base, vector-offset form.
    auto plane_rel = [&](int p) -> uint32_t { return NPW == 1 ? 0u : (uint32_t)p * ((uint32_t)C * (H * W)); };
    // plane p of an item index over all NPW planes, and the index within it
    auto split = [&](int item, int n, int& r) {
        const int p = NPW == 1 ? 0 : udiv(item, n);
        r = item - p * n;
        return p;
    };

    // P0's loads. The taps' loads (of channel cc) go out first and the x
    // loads (of group gg, channel cc) right after them; the taps (level taps
    // with the band scale and 4^-l folded in) are staged once both are in
    // flight, so the two round trips overlap. Every lane loads (past the
    // end: the last tap again) and stores only its own.
    constexpr int MWB = cdiv(KB2P, NT), NWL = 4 * L * K2P, MWL = cdiv(NWL, NT);
    float wbv[MWB], wlv[MWL], scv[MWL];
    auto load_taps = [&](int cc) {
#pragma unroll
        for (int k = 0; k < MWB; ++k) {
            const int t = min(tid + k * NT, KB * KB - 1);
            wbv[k] = w_base[(size_t)cc * KB * KB + (FLIP ? KB * KB - 1 - t : t)];
        }
#pragma unroll
        for (int k = 0; k < MWL; ++k) {
            const int t = min(tid + k * NT, NWL - 1);
            const int ls = t / K2P, tap = min(t - ls * K2P, K * K - 1), l = ls >> 2, s = ls & 3;
            const size_t pi = ((size_t)l * C + cc) * 4 + s;
            scv[k] = scale[pi];
            wlv[k] = w_lvl[pi * K * K + (FLIP ? K * K - 1 - tap : tap)];
        }
    };
    // The whole bordered x plane and the bordered level-1 bands in one pass.
    // An item owns x rows 2i, 2i+1 and VA columns from 2*j0 (one or two Haar
    // blocks, band cells j0.. of row i): inside the plane it loads them,
    // stores them widened and stores their four bands; on the border it
    // stores zeros to both (the padding of the base convolution and of the
    // level-1 convolutions). With ZFILL the regions are zeroed first and the
    // items cover the interior cells only (row ii, item uu of the bordered
    // grid, offset by the border).
    constexpr bool ZF = P::ZFILL;
    constexpr int CPI = P::CPI, VA = P::VA;
    // QPOW2: items on the power-of-two grid, NQ cells per plane of IPR
    // per row, the cells past the plane's rows or items idle
    constexpr bool QP = P::QPOW2;
    constexpr int NQ = QP ? P::NQP : ZF ? P::NQI : P::NQ, IPR = QP ? P::IPRP : ZF ? P::IPRI : P::IPR;
    auto cell = [&](int q, int& ri, int& uq) {
        ri = udiv(q, IPR);
        uq = q - ri * IPR;
        return !QP || (ri < H1 && uq < P::IPRI);
    };
    constexpr int R0 = ZF ? PK : 0, U0 = ZF ? PK / CPI : 0;
    constexpr int NQA = NPW * NQ, MQ = cdiv(NQA, NT);
    static_assert(!PERS || (!ZF && NPW == 1), "persistent plans: one plane per group, bordered items");
    // Persistent plans load (and prefetch) the interior items only, on a
    // power-of-two grid of H/2 rows of IPN items, in MQN whole rounds; their
    // border items store zeros each plane (no registers held for them).
    constexpr int IPN = (W >> 1) / CPI, NQN = (H >> 1) * IPN, MQN = cdiv(NQN, NT);
    static_assert(!PERS || (NQN % NT == 0 && (IPN & (IPN - 1)) == 0), "whole rounds of interior items");
    constexpr int MQL = PERS ? MQN : MQ;   // rounds of loaded items
    RawVec<T, VA> r0[MQL], r1[MQL];
    auto load_x = [&](int gg, int cc) {
        const T* __restrict__ in_gg = in + ((size_t)gg * NPW * C + cc) * H * W;
        if constexpr (PERS) {
            const bool live_gg = NPW == 1 || gg * NPW < B;
#pragma unroll
            for (int k = 0; k < MQN; ++k) {
                const int q = tid + k * NT, i = q / IPN, j0 = (q - (q / IPN) * IPN) * CPI;
                const T* s0 = in_gg + (live_gg ? (uint32_t)((2 * i) * W + 2 * j0) : 0u);
                load_raw<T, VA>(s0, r0[k]);
                load_raw<T, VA>(s0 + W, r1[k]);
#pragma unroll
                for (int e = 0; e < RawVec<T, VA>::N; ++e) {
                    r0[k].w[e] = live_gg ? r0[k].w[e] : 0u;
                    r1[k].w[e] = live_gg ? r1[k].w[e] : 0u;
                }
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < MQ; ++k) {
            const int qa = tid + k * NT;
            int q;
            const int p = split(qa < NQA ? qa : 0, NQ, q);
            int ri, uq;
            const bool real = cell(q, ri, uq);
            const int ii = ri + R0, uu = uq + U0, i = ii - PK, j0 = uu * CPI - PK;
            const bool inside = (NQA % NT == 0 || qa < NQA) && (NPW == 1 || gg * NPW + p < B) && real &&
                                (ZF || (i >= 0 && i < H1 && j0 >= 0 && j0 < W1));
            // every lane loads (border items the plane's first words) and
            // then selects zeros: no branch, so the registers stay registers
            const T* s0 = in_gg + (inside ? plane_rel(p) + (uint32_t)((2 * i) * W + 2 * j0) : 0u);
            load_raw<T, VA>(s0, r0[k]);
            load_raw<T, VA>(s0 + (inside ? W : 0), r1[k]);
#pragma unroll
            for (int e = 0; e < RawVec<T, VA>::N; ++e) {
                r0[k].w[e] = inside ? r0[k].w[e] : 0u;
                r1[k].w[e] = inside ? r1[k].w[e] : 0u;
            }
        }
    };
    if constexpr (PERS) {
        load_taps((int)(blockIdx.x % C));
        load_x((int)(blockIdx.x / C), (int)(blockIdx.x % C));
    }

    for (unsigned grp = blockIdx.x;;) {
    // The thread index anew for each group: an empty asm makes it opaque, so
    // the compiler cannot hoist the group's address arithmetic out of the
    // loop, where it would stay live across every group and spill.
    int tid = (int)threadIdx.x;
    if constexpr (PERS) asm volatile("" : "+v"(tid));
    // this group: channel c of images g*NPW .. g*NPW + NPW-1 (those < B)
    const int c = grp % C, g = grp / C;
    auto live = [&](int p) { return NPW == 1 || g * NPW + p < B; };
    T* __restrict__ out_g = out + ((size_t)g * NPW * C + c) * H * W;
    // the previous group's reads of LDS are done before this one's stores
    if (PERS && grp != blockIdx.x) __syncthreads();
    // plane p's regions: x (A), level-1 bands (B); U_l (and then Z'_l) of
    // level l >= 2 in region A
    auto Ap = [&](int p) { return lds + p * PL; };
    auto ubase = [&](auto lc, int p) -> float* {
        constexpr int l = decltype(lc)::value;
        constexpr int off = P::uoff(l);   // evaluated at compile time
        if constexpr (l == 1) return lds + p * PL + P::ASIZE;
        else return lds + p * PL + off;
    };

    // ---------------------------------------------------------------- P0
    if constexpr (!PERS) load_taps(c);
    auto stage_taps = [&]() {
#pragma unroll
        for (int k = 0; k < MWB; ++k) {
            const int t = tid + k * NT;
            if (t < KB2P) WB[t] = t < KB * KB ? wbv[k] : 0.f;
        }
#pragma unroll
        for (int k = 0; k < MWL; ++k) {
            const int t = tid + k * NT;
            if (t < NWL) {
                const int ls = t / K2P, tap = t - ls * K2P, l = ls >> 2;
                const float f = scv[k] * (1.0f / (float)(1 << (2 * (l + 1))));
                WL[t] = tap < K * K ? wlv[k] * f : 0.f;
            }
        }
    };
    {
        if constexpr (ZF) {
            static_assert((NPW * PL) % 4 == 0, "planes span whole 128-bit words");
            float4* const z = reinterpret_cast<float4*>(lds);
            for (int t = tid; t < NPW * PL / 4; t += NT) z[t] = make_float4(0.f, 0.f, 0.f, 0.f);
            __syncthreads();
        }
        if constexpr (!PERS) load_x(g, c);
        stage_taps();
        // one item's stores: its two x rows, widened, and its four band cells
        auto store_item = [&](float* A, int ii, int uu, const float (&f0)[VA], const float (&f1)[VA]) {
            float* const Bq = A + P::ASIZE;
            const int i = ii - PK, j0 = uu * CPI - PK;
            const int xr = PB + 2 * i, xc = XO + 2 * j0;
            if (xc >= 0 && xc + VA <= SX) {
                if (xr >= 0 && xr < H + 2 * PB) store_vec<VA>(A + xr * SX + xc, f0);
                if (xr + 1 >= 0 && xr + 1 < H + 2 * PB) store_vec<VA>(A + (xr + 1) * SX + xc, f1);
            }
            float b[4][CPI];
#pragma unroll
            for (int m = 0; m < CPI; ++m)
                haar4(f0[2 * m], f0[2 * m + 1], f1[2 * m], f1[2 * m + 1], b[0][m], b[1][m], b[2][m], b[3][m]);
            float* o = Bq + ii * S1 + uu * CPI;
#pragma unroll
            for (int s = 0; s < 4; ++s) store_vec<CPI>(o + s * BS1, b[s]);
        };
        if constexpr (PERS) {
            // the interior items from the prefetched registers ...
#pragma unroll
            for (int k = 0; k < MQN; ++k) {
                const int q = tid + k * NT, ri = q / IPN, uq = q - ri * IPN;
                float f0[VA], f1[VA];
                widen_raw<T, VA>(r0[k], f0);
                widen_raw<T, VA>(r1[k], f1);
                store_item(Ap(0), ri + PK, uq + PK / CPI, f0, f1);
            }
            // ... and zeros for the border items: the PK top and bottom rows of
            // the bordered grid, then its PK / CPI items at each side of the
            // interior rows
            constexpr int UB = PK / CPI, NTB = 2 * PK * P::IPR, NBD = NTB + (H >> 1) * 2 * UB;
            for (int t = tid; t < NBD; t += NT) {
                int ii, uu;
                if (t < NTB) {
                    const int r = t / P::IPR;
                    ii = r < PK ? r : r + (H >> 1);
                    uu = t - r * P::IPR;
                } else {
                    const int t2 = t - NTB, r = t2 / (2 * UB), sd = t2 - r * (2 * UB);
                    ii = PK + r;
                    uu = sd < UB ? sd : sd + IPN;
                }
                float z[VA] = {};
                store_item(Ap(0), ii, uu, z, z);
            }
        } else {
#pragma unroll
        for (int k = 0; k < MQ; ++k) {
            const int qa = tid + k * NT;
            if (!(NQA % NT == 0 || qa < NQA)) continue;
            int q;
            const int p = split(qa, NQ, q);
            float* const A = Ap(p);
            float* const Bq = A + P::ASIZE;
            int ri, uq;
            if (!cell(q, ri, uq)) continue;
            const int ii = ri + R0, uu = uq + U0, i = ii - PK, j0 = uu * CPI - PK;
            float f0[VA], f1[VA];
            widen_raw<T, VA>(r0[k], f0);
            widen_raw<T, VA>(r1[k], f1);
            const int xr = PB + 2 * i, xc = XO + 2 * j0;
            if (xc >= 0 && xc + VA <= SX) {
                if (xr >= 0 && xr < H + 2 * PB) store_vec<VA>(A + xr * SX + xc, f0);
                if (xr + 1 >= 0 && xr + 1 < H + 2 * PB) store_vec<VA>(A + (xr + 1) * SX + xc, f1);
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
        if constexpr (PERS) {   // the next group's loads fly during this one
            const unsigned nx = grp + ndata;
            if (nx < ngroups) {
                load_taps((int)(nx % C));
                load_x((int)(nx / C), (int)(nx % C));
            }
        }
    }
    __syncthreads();

    // the level convolutions: strips of rl(l) rows x 1 column of one band,
    // into registers; level l's strips on threads T0.. (level 1 with CONC1:
    // the threads that the base strips leave idle, in P1), else all threads
    auto level_conv = [&](auto lc, auto& z) {
        constexpr int l = decltype(lc)::value;
        constexpr int hl = H >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), R = P::rl(l);
        constexpr int T0 = (l == 1 && P::CONC1) ? P::NBL : 0, NTH = NT - T0;
        constexpr int NS = hl / R, LP = P::lpl(l), NIl = P::nil(l), MIl = cdiv(NPW * NIl, NTH);
#pragma unroll
        for (int it = 0; it < MIl; ++it) {
            const int ia = tid - T0 + it * NTH;
            if ((T0 == 0 || tid >= T0) && ((NPW * NIl) % NTH == 0 || ia < NPW * NIl)) {
                int item;
                float* const Ul = ubase(lc, split(ia, NIl, item));
                const int s = udiv(item, NS * LP), rem = item - s * (NS * LP);
                const int rs = udiv(rem, LP), j = rem - rs * LP;
                if (LP == wl || j < wl)
                    conv_col<K, R, Sl>(Ul + s * BSl + (rs * R) * Sl + j, WL + ((l - 1) * 4 + s) * K2P, z[it]);
            }
        }
    };
    auto level_store = [&](auto lc, auto& z) {
        constexpr int l = decltype(lc)::value;
        constexpr int hl = H >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), R = P::rl(l);
        constexpr int T0 = (l == 1 && P::CONC1) ? P::NBL : 0, NTH = NT - T0;
        constexpr int NS = hl / R, LP = P::lpl(l), NIl = P::nil(l), MIl = cdiv(NPW * NIl, NTH);
#pragma unroll
        for (int it = 0; it < MIl; ++it) {
            const int ia = tid - T0 + it * NTH;
            if ((T0 == 0 || tid >= T0) && ((NPW * NIl) % NTH == 0 || ia < NPW * NIl)) {
                int item;
                float* const Ul = ubase(lc, split(ia, NIl, item));
                const int s = udiv(item, NS * LP), rem = item - s * (NS * LP);
                const int rs = udiv(rem, LP), j = rem - rs * LP;
                if (!(LP == wl || j < wl)) continue;
#pragma unroll
                for (int o = 0; o < R; ++o) Ul[s * BSl + (PK + rs * R + o) * Sl + PK + j] = z[it][o];
            }
        }
    };
    // ---------------------------------------------------------------- P1
    float yb[MB][RB];
    float z1[cdiv(NPW * P::nil(1), P::CONC1 ? NT - P::NBL : NT)][P::rl(1)];
#pragma unroll
    for (int it = 0; it < MB; ++it) {
        const int item = tid + it * NT;
        if ((NPW * NIB) % NT == 0 || item < NPW * NIB) {
            int r;
            const int p = split(item, NIB, r);
            const int rb = udiv(r, LPB), w = r - rb * LPB;
            const float* X0 = Ap(p) + XO - PB;   // origin of the bordered x plane
            if (LPB == W || w < W) conv_col<KB, RB, SX>(X0 + (rb * RB) * SX + w, WB, yb[it]);
        }
    }
    if constexpr (P::CONC1) level_conv(std::integral_constant<int, 1>{}, z1);
    __syncthreads();

    // ---------------------------------------------------------------- P2
    P::for_deep_levels([&](auto lc) {
        constexpr int l = decltype(lc)::value;
        constexpr int hl = H >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l);
        constexpr int Sp = P::su(l - 1);
        constexpr int UO = P::uoff(l), UP = P::uoff(l - 1);
        // over the bordered grid: zeros on the border
        constexpr int GW = wl + 2 * PK, GN = (hl + 2 * PK) * GW;
        for (int qa = tid; qa < NPW * GN; qa += NT) {
            int q;
            const int p = split(qa, GN, q);
            float* const Ul = Ap(p) + UO;
            const float* LLp = (l == 2) ? (Ap(p) + P::ASIZE + PK * Sp + PK) : (Ap(p) + UP + PK * Sp + PK);
            const int ii = udiv(q, GW), jj = q - ii * GW, i = ii - PK, j = jj - PK;
            float b[4] = {0.f, 0.f, 0.f, 0.f};
            if (i >= 0 && i < hl && j >= 0 && j < wl) {
                const float* x2 = LLp + 2 * i * Sp + 2 * j;
                haar4(x2[0], x2[1], x2[Sp], x2[Sp + 1], b[0], b[1], b[2], b[3]);
            }
            const int o = ii * Sl + jj;
#pragma unroll
            for (int s = 0; s < 4; ++s) Ul[s * BSl + o] = b[s];
        }
        __syncthreads();
    });

    // ---------------------------------------------------------------- P3
    // one level-2..L strip per thread when they all fit (fewer live registers)
    auto deep_conv = [&](auto lc, float (&zd)[P::RLD]) {
        constexpr int l = decltype(lc)::value;
        constexpr int hl = H >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), R = P::rl(l);
        constexpr int NS = hl / R, LP = P::lpl(l), NIl = P::nil(l), O = P::doff(l);
        const int ia = tid - O;
        if (ia >= 0 && ia < NPW * NIl) {
            int item;
            float* const Ul = ubase(lc, split(ia, NIl, item));
            const int s = udiv(item, NS * LP), rem = item - s * (NS * LP);
            const int rs = udiv(rem, LP), j = rem - rs * LP;
            if (LP == wl || j < wl) {
                float z[R];
                conv_col<K, R, Sl>(Ul + s * BSl + (rs * R) * Sl + j, WL + ((l - 1) * 4 + s) * K2P, z);
#pragma unroll
                for (int o = 0; o < R; ++o) zd[o] = z[o];
            }
        }
    };
    auto deep_store = [&](auto lc, const float (&zd)[P::RLD]) {
        constexpr int l = decltype(lc)::value;
        constexpr int hl = H >> l, wl = W >> l, Sl = P::su(l), BSl = P::bandsz(l), R = P::rl(l);
        constexpr int NS = hl / R, LP = P::lpl(l), NIl = P::nil(l), O = P::doff(l);
        const int ia = tid - O;
        if (ia >= 0 && ia < NPW * NIl) {
            int item;
            float* const Ul = ubase(lc, split(ia, NIl, item));
            const int s = udiv(item, NS * LP), rem = item - s * (NS * LP);
            const int rs = udiv(rem, LP), j = rem - rs * LP;
            if (LP == wl || j < wl) {
#pragma unroll
                for (int o = 0; o < R; ++o) Ul[s * BSl + (PK + rs * R + o) * Sl + PK + j] = zd[o];
            }
        }
    };
    // results of all levels stay in registers across one barrier (with
    // CONC1, level 1's were made in P1, and P1's barrier is that barrier)
    if constexpr (!P::CONC1) level_conv(std::integral_constant<int, 1>{}, z1);
    if constexpr (P::DSHARE) {
        float zd[P::RLD];
        P::for_deep_levels([&](auto lc) { deep_conv(lc, zd); });
        __syncthreads();
        level_store(std::integral_constant<int, 1>{}, z1);
        P::for_deep_levels([&](auto lc) { deep_store(lc, zd); });
    } else {
        float z2[L >= 2 ? cdiv(NPW * P::nil(L >= 2 ? 2 : 1), NT) : 1][P::rl(L >= 2 ? 2 : 1)];
        float z3[L >= 3 ? cdiv(NPW * P::nil(L >= 3 ? 3 : 1), NT) : 1][P::rl(L >= 3 ? 3 : 1)];
        float z4[L >= 4 ? cdiv(NPW * P::nil(L >= 4 ? 4 : 1), NT) : 1][P::rl(L >= 4 ? 4 : 1)];
        float z5[L >= 5 ? cdiv(NPW * P::nil(L >= 5 ? 5 : 1), NT) : 1][P::rl(L >= 5 ? 5 : 1)];
        if constexpr (L >= 2) level_conv(std::integral_constant<int, 2>{}, z2);
        if constexpr (L >= 3) level_conv(std::integral_constant<int, 3>{}, z3);
        if constexpr (L >= 4) level_conv(std::integral_constant<int, 4>{}, z4);
        if constexpr (L >= 5) level_conv(std::integral_constant<int, 5>{}, z5);
        if constexpr (!P::CONC1) __syncthreads();
        level_store(std::integral_constant<int, 1>{}, z1);
        if constexpr (L >= 2) level_store(std::integral_constant<int, 2>{}, z2);
        if constexpr (L >= 3) level_store(std::integral_constant<int, 3>{}, z3);
        if constexpr (L >= 4) level_store(std::integral_constant<int, 4>{}, z4);
        if constexpr (L >= 5) level_store(std::integral_constant<int, 5>{}, z5);
    }
    __syncthreads();

    // ---------------------------------------------------------------- P4
    // y[h][w] = base + sum_l A_l + sign(bit_{l-1} h) B_l with
    // A_l = Z0 + sign(bit_{l-1} w) Z2, B_l = Z1 + sign(bit_{l-1} w) Z3 at (h >> l, w >> l)
#pragma unroll
    for (int it = 0; it < MB; ++it) {
        const int item = tid + it * NT;
        if (!((NPW * NIB) % NT == 0 || item < NPW * NIB)) continue;
        int r;
        const int p = split(item, NIB, r);
        const int rb = udiv(r, LPB), w = r - rb * LPB, h0 = rb * RB;
        if (!(LPB == W || w < W) || !live(p)) continue;
        // this strip's column in its plane: rows at constant offsets from it
        T* __restrict__ dst = out_g + (plane_rel(p) + (uint32_t)(h0 * W + w));
        float y[RB];
#pragma unroll
        for (int o = 0; o < RB; ++o) y[o] = yb[it][o];
        if constexpr (RB % (1 << L) == 0) {
            // whole 2^L-row blocks. From the coarsest level down, carry[p] is
            // what the coarser levels add to every row of level-l block p
            // (constant over it: row bit l is); level l splits it into its
            // two half-blocks as carry + a +- b.
            float carry[RB];
            P::for_levels([&](auto lc) {
                constexpr int l = L + 1 - decltype(lc)::value;   // L, L-1, ..., 1
                constexpr int Sl = P::su(l), BSl = P::bandsz(l);
                const float* Zl = ubase(std::integral_constant<int, l>{}, p) + (PK + (h0 >> l)) * Sl + PK + (w >> l);
                const float sw = ((w >> (l - 1)) & 1) ? -1.f : 1.f;
                float next[RB >> (l - 1)];
#pragma unroll
                for (int p = 0; p < (RB >> l); ++p) {
                    const float* z = Zl + p * Sl;
                    float a = __builtin_fmaf(sw, z[2 * BSl], z[0]);
                    const float b = __builtin_fmaf(sw, z[3 * BSl], z[BSl]);
                    if constexpr (l < L) a += carry[p];
                    next[2 * p] = a + b;
                    next[2 * p + 1] = a - b;
                }
#pragma unroll
                for (int q = 0; q < (RB >> (l - 1)); ++q) carry[q] = next[q];
            });
#pragma unroll
            for (int o = 0; o < RB; ++o) y[o] += carry[o];
        } else {
        P::for_levels([&](auto lc) {
            constexpr int l = decltype(lc)::value;
            constexpr int Sl = P::su(l), BSl = P::bandsz(l);
            const float* Zl = ubase(lc, p) + (PK + (h0 >> l)) * Sl + PK + (w >> l);
            const float sw = ((w >> (l - 1)) & 1) ? -1.f : 1.f;
            if constexpr (RB % (1 << l) == 0) {
                // whole 2^l-row blocks: the row bits below l are strip-relative
                // and known at compile time
#pragma unroll
                for (int p = 0; p < (RB >> l); ++p) {
                    const float* z = Zl + p * Sl;
                    const float a = __builtin_fmaf(sw, z[2 * BSl], z[0]);
                    const float b = __builtin_fmaf(sw, z[3 * BSl], z[BSl]);
                    const float plus = a + b, minus = a - b;
#pragma unroll
                    for (int o = p << l; o < (p + 1) << l; ++o) y[o] += ((o >> (l - 1)) & 1) ? minus : plus;
                }
            } else {
                // the strip lies inside one 2^l-row block and shares its row
                // bit l-1 (RB is a power of two below 2^l)
                const float a = __builtin_fmaf(sw, Zl[2 * BSl], Zl[0]);
                const float b = __builtin_fmaf(sw, Zl[3 * BSl], Zl[BSl]);
                const float v = ((h0 >> (l - 1)) & 1) ? a - b : a + b;
#pragma unroll
                for (int o = 0; o < RB; ++o) y[o] += v;
            }
        });
        }
        if constexpr (sizeof(T) == 2 && RB % 2 == 0) {
            // two rows per conversion: the low half to row o, the high half
            // to row o + 1
#pragma unroll
            for (int o = 0; o < RB; o += 2) {
                const uint32_t pr = narrow_bf16x2(y[o], y[o + 1]);
                dst[o * W] = (bf16_t)(pr & 0xffffu);
                dst[(o + 1) * W] = (bf16_t)(pr >> 16);
            }
        } else {
#pragma unroll
            for (int o = 0; o < RB; ++o) {
                if constexpr (sizeof(T) == 2) dst[o * W] = narrow_bf16(y[o]);
                else dst[o * W] = y[o];
            }
        }
    }
    // one group per workgroup: no loop at all (the same code as a kernel
    // without one); persistent: the next of this workgroup's groups
    if constexpr (!PERS) break;
    grp += ndata;
    if (grp >= ngroups) break;
    }  // groups
}

// Launchers of the whole-plane kernels: one workgroup per plane
// (plane_kernel), or per channel and group of NPW images (col_kernel).
// A non-null `fin` with fin->C > 0 adds fin->C workgroups that run that
// deferred weight-gradient second stage (its scratch fits the kernel's LDS:
// the caller checks PlaneEntry::lds_bytes).
template <class P, typename T, bool FLIP>
hipError_t launch_plane(const void* in, const float* wb, const float* wl, const float* sc,
                               void* out, int B, int C, hipStream_t stream, const FinalizeArgs* fin) {
    const unsigned planes = (unsigned)B * (unsigned)C, extra = fin ? (unsigned)fin->C : 0u;
    hipLaunchKernelGGL((plane_kernel<P, T, FLIP, 0, T>), dim3(planes + extra), dim3(P::NT), 0, stream,
                       (const T*)in, wb, wl, sc, (T*)out, C, planes, fin ? *fin : FinalizeArgs{});
    return hipGetLastError();
}

template <class P, typename T, bool FLIP>
hipError_t launch_col(const void* in, const float* wb, const float* wl, const float* sc, void* out,
                             int B, int C, hipStream_t stream, const FinalizeArgs* fin) {
    // one workgroup per channel and group of NPW images, or (PERSIST) as
    // many as the chip holds at once, each looping over its share
    const unsigned groups = (unsigned)cdiv(B, P::NPW) * (unsigned)C, extra = fin ? (unsigned)fin->C : 0u;
    unsigned nwg = groups;
    if constexpr (P::template persist<T>()) {
        const unsigned slots = (unsigned)cu_count() * (unsigned)(P::WG_PER_CU > 0 ? P::WG_PER_CU : 1);
        nwg = groups < slots ? groups : slots;
    }
    hipLaunchKernelGGL((col_kernel<P, T, FLIP>), dim3(nwg + extra), dim3(P::NT), 0, stream, (const T*)in, wb, wl,
                       sc, (T*)out, B, C, fin ? *fin : FinalizeArgs{});
    return hipGetLastError();
}

}  // namespace wtc
