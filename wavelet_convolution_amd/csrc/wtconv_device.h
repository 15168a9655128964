// Device-side helpers shared by the WTConv HIP kernels (gfx950).
//
// Activation storage is fp32 or bf16; every product and sum is fp32. bf16 is
// widened exactly (a 16-bit shift) and narrowed with round-to-nearest-even.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <utility>

namespace wtc {

typedef uint16_t bf16_t;

constexpr int cdiv(int a, int b) { return (a + b - 1) / b; }

// Row strides of LDS planes are made odd so that lanes reading the same
// column of different rows fall into different banks.
constexpr int odd_stride(int w) { return (w % 2 == 0) ? w + 1 : w; }

// a / b for a >= 0 and b > 0, in unsigned arithmetic: no sign fix-up
__device__ __forceinline__ int udiv(int a, int b) { return (int)((unsigned)a / (unsigned)b); }

// A workgroup barrier that orders LDS only: each wavefront waits for its
// own LDS operations, not for its global loads and stores, so a prefetch
// in flight stays in flight across it (a full barrier waits for every
// outstanding vector memory operation, and loads and stores share one
// counter). For barriers where no wavefront reads what another wrote to
// global memory before it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// f(integral_constant<int, 0>), ..., f(integral_constant<int, N - 1>): an
// unrolled loop whose index is a compile-time constant in the body
template <class F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, class F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

__device__ __forceinline__ float widen(float v) { return v; }
__device__ __forceinline__ float widen(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even: gfx950's v_cvt_pk_bf16_f32 converts
// two values per instruction without branches (NaN stays NaN).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t narrow_bf16x2(float lo, float hi) {
    bf16x2_t v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ bf16_t narrow_bf16(float f) {
    return (bf16_t)(narrow_bf16x2(f, 0.f) & 0xffffu);
}

template <typename T> struct Act;
template <> struct Act<float> {
    static constexpr int BYTES = 4;
};
template <> struct Act<bf16_t> {
    static constexpr int BYTES = 2;
};

// Largest vector (elements) that divides a row and keeps every plane aligned.
template <typename T>
constexpr int vec_elems(int W, int HW) {
    const int cands[4] = {16 / Act<T>::BYTES, 8 / Act<T>::BYTES, 4 / Act<T>::BYTES, 1};
    for (int i = 0; i < 4; ++i) {
        int v = cands[i];
        if (v >= 1 && W % v == 0 && (HW * Act<T>::BYTES) % (v * Act<T>::BYTES) == 0) return v;
    }
    return 1;
}

// Load V consecutive activations (V * sizeof(T) bytes, naturally aligned)
// and widen them to fp32.
template <typename T, int V>
__device__ __forceinline__ void load_vec(const T* __restrict__ p, float (&out)[V]) {
    constexpr int BYTES = V * Act<T>::BYTES;
    if constexpr (BYTES == 16) {
        uint4 q = *reinterpret_cast<const uint4*>(p);
        uint32_t w[4] = {q.x, q.y, q.z, q.w};
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                out[2 * i] = __uint_as_float(w[i] << 16);
                out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) out[i] = __uint_as_float(w[i]);
        }
    } else if constexpr (BYTES == 8) {
        uint2 q = *reinterpret_cast<const uint2*>(p);
        uint32_t w[2] = {q.x, q.y};
        if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                out[2 * i] = __uint_as_float(w[i] << 16);
                out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
            }
        } else {
            out[0] = __uint_as_float(w[0]);
            out[1] = __uint_as_float(w[1]);
        }
    } else if constexpr (BYTES == 4 && sizeof(T) == 2) {
        uint32_t w = *reinterpret_cast<const uint32_t*>(p);
        out[0] = __uint_as_float(w << 16);
        out[1] = __uint_as_float(w & 0xffff0000u);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) out[i] = widen(p[i]);
    }
}

// Elements per lane when a plane is streamed into LDS: 4 when rows hold
// whole groups of four (one 128-bit LDS store per lane; consecutive lanes
// fill consecutive 16-byte words, which no two lanes of a pass share a bank
// in), else 2, else 1.
constexpr int lds_vec(int W) { return W % 4 == 0 ? 4 : (W % 2 == 0 ? 2 : 1); }

constexpr int round_up(int v, int m) { return (v + m - 1) / m * m; }

// V activations as loaded from HBM, still in their storage format (bf16
// pairs stay packed: half the registers while a load is in flight).
template <typename T, int V>
struct RawVec {
    static constexpr int N = (V * Act<T>::BYTES + 3) / 4;
    uint32_t w[N];
};

template <typename T, int V>
__device__ __forceinline__ void load_raw(const T* __restrict__ p, RawVec<T, V>& r) {
    constexpr int BYTES = V * Act<T>::BYTES;
    if constexpr (BYTES == 16) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        r.w[0] = q.x;
        r.w[1] = q.y;
        r.w[2] = q.z;
        r.w[3] = q.w;
    } else if constexpr (BYTES == 8) {
        const uint2 q = *reinterpret_cast<const uint2*>(p);
        r.w[0] = q.x;
        r.w[1] = q.y;
    } else if constexpr (BYTES == 4) {
        r.w[0] = *reinterpret_cast<const uint32_t*>(p);
    } else {
        r.w[0] = *reinterpret_cast<const uint16_t*>(p);
    }
}

// V activations of one row from column c0, in their storage format: the
// ones at columns >= IW, or all of them when !row_ok, are zero (the zero
// padding of a plane to whole 2^L blocks). A whole vector inside the row is
// one load when the row length keeps it aligned.
template <typename T, int V, int IW>
__device__ __forceinline__ void load_raw_guarded(const T* __restrict__ row, int c0, bool row_ok, RawVec<T, V>& r) {
#pragma unroll
    for (int i = 0; i < RawVec<T, V>::N; ++i) r.w[i] = 0u;
    if (!row_ok || c0 >= IW) return;
    if constexpr (IW % V == 0) {
        load_raw<T, V>(row + c0, r);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) {
            if (c0 + i >= IW) break;
            if constexpr (sizeof(T) == 2) {
                const uint32_t v = *reinterpret_cast<const uint16_t*>(row + c0 + i);
                r.w[i / 2] |= (i % 2 == 0) ? v : (v << 16);
            } else {
                r.w[i] = __float_as_uint(row[c0 + i]);
            }
        }
    }
}

// Widen to fp32 (exact for bf16).
template <typename T, int V>
__device__ __forceinline__ void widen_raw(const RawVec<T, V>& r, float (&f)[V]) {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int i = 0; i < V; ++i) f[i] = __uint_as_float(i % 2 == 0 ? r.w[i / 2] << 16 : r.w[i / 2] & 0xffff0000u);
    } else {
#pragma unroll
        for (int i = 0; i < V; ++i) f[i] = __uint_as_float(r.w[i]);
    }
}

// Store V floats at p (aligned to 4 * V bytes) with one vector store.
template <int V>
__device__ __forceinline__ void store_vec(float* p, const float (&f)[V]) {
    if constexpr (V == 4) *reinterpret_cast<float4*>(p) = make_float4(f[0], f[1], f[2], f[3]);
    else if constexpr (V == 2) *reinterpret_cast<float2*>(p) = make_float2(f[0], f[1]);
    else p[0] = f[0];
}

// Store V activations in their storage format at p (aligned to the vector).
template <typename T, int V>
__device__ __forceinline__ void store_raw(T* p, const RawVec<T, V>& r) {
    constexpr int N = RawVec<T, V>::N;
    static_assert(V * sizeof(T) == 4 * N, "whole 32-bit words");
    if constexpr (N == 4) *reinterpret_cast<uint4*>(p) = make_uint4(r.w[0], r.w[1], r.w[2], r.w[3]);
    else if constexpr (N == 2) *reinterpret_cast<uint2*>(p) = make_uint2(r.w[0], r.w[1]);
    else *reinterpret_cast<uint32_t*>(p) = r.w[0];
}

// Widen to fp32 and store at p (aligned to 4 * V bytes).
template <typename T, int V>
__device__ __forceinline__ void store_lds(float* p, const RawVec<T, V>& r) {
    float f[V];
    widen_raw(r, f);
    store_vec<V>(p, f);
}

// Lanes given to one row block of column strips over a row of w columns:
// whole wavefronts when w > 32, else the next power of two, so that the 32
// lanes of one LDS pass never straddle two row blocks (w >= 32) or cover
// whole aligned groups of them (w < 32). Lanes past w idle.
constexpr int strip_lanes(int w) {
    if (w > 32) return round_up(w, 64);
    int p = 1;
    while (p < w) p *= 2;
    return p;
}

// Store a row segment of N fp32 values (N even for bf16; the segment start
// is 4-byte aligned for bf16 and 8-byte aligned for fp32 pairs).
template <int N>
__device__ __forceinline__ void store_row(float* __restrict__ p, const float (&v)[N]) {
    if constexpr (N % 2 == 0) {
#pragma unroll
        for (int i = 0; i < N; i += 2) *reinterpret_cast<float2*>(p + i) = make_float2(v[i], v[i + 1]);
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i) p[i] = v[i];
    }
}
template <int N>
__device__ __forceinline__ void store_row(bf16_t* __restrict__ p, const float (&v)[N]) {
    static_assert(N % 2 == 0, "bf16 rows are stored as pairs");
#pragma unroll
    for (int i = 0; i < N; i += 2) {
        *reinterpret_cast<uint32_t*>(p + i) = narrow_bf16x2(v[i], v[i + 1]);
    }
}

// Store one value in the storage format (bf16: rounded to nearest even).
__device__ __forceinline__ void store_one(float* p, float v) { *p = v; }
__device__ __forceinline__ void store_one(bf16_t* p, float v) { *p = narrow_bf16(v); }

// Materialise values in registers at this point: an empty asm that reads and
// writes each one. Compiler passes may otherwise sink a convolution's FMAs
// down to the first use of its result, phases later, keeping every loaded
// window value live across the barriers in between (and spilling them).
template <int N>
__device__ __forceinline__ void pin_regs(float (&v)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}
template <int R, int N>
__device__ __forceinline__ void pin_regs(float (&v)[R][N]) {
#pragma unroll
    for (int r = 0; r < R; ++r) pin_regs(v[r]);
}

// LDS row addressing for window loads. The backend pairs dword loads that
// share a base into one two-address load whose offsets reach 1 KB; beyond
// that it makes a fresh base register for each pair (one VALU add per two
// loads). Window rows are therefore read from a base the compiler cannot see
// through (an empty asm), renewed every GROUP rows so that every pair's
// offsets stay in range: one add per GROUP rows.
typedef const float __attribute__((address_space(3)))* lds_cfp;
__device__ __forceinline__ lds_cfp opaque_lds(const float* p) {
    uint32_t a = (uint32_t)(uintptr_t)(lds_cfp)p;
    asm volatile("" : "+v"(a));
    return (lds_cfp)(uintptr_t)a;
}
template <int S>
struct RowBases {
    // rows per base: the farthest pair offset (GROUP-1 rows + 7 words) under
    // 1 KB. Rows longer than that get one base each (left to itself, the
    // compiler makes a base per pair of loads there: three adds per row)
    static constexpr int GROUP = (1020 / 4 - 8) / S + 1;
    static constexpr bool USE = GROUP >= 1;
};
template <int S, int NR>
struct RowAddr {
    static constexpr int GR = RowBases<S>::USE ? RowBases<S>::GROUP : NR;
    lds_cfp rb[cdiv(NR, GR)];
    const float* p;
    __device__ __forceinline__ explicit RowAddr(const float* base) : p(base) {
        if constexpr (RowBases<S>::USE) {
#pragma unroll
            for (int g = 0; g < cdiv(NR, GR); ++g) rb[g] = opaque_lds(base + g * GR * S);
        }
    }
    // the start of window row r (read its words with [n])
    __device__ __forceinline__ lds_cfp row(int r) const {
        if constexpr (RowBases<S>::USE) return rb[r / GR] + (r % GR) * S;
        else return (lds_cfp)(p + r * S);
    }
};

// acc[o][q] += sum_{m,n} w[m][n] * s[(o+m)*S + q+n]: an OR x OC tile of a
// 'same' cross-correlation read from a zero-bordered LDS plane (s points at
// the window's top-left corner, S is the plane's row stride). The K*K taps
// come from LDS too (every lane reads the same address: a broadcast). Window
// rows are streamed through registers; every loaded value feeds up to K*K
// FMAs. The first tap of each output initialises it (no separate zeroing).
//
// The taps block starts 16-byte aligned and is padded to a multiple of four
// floats (kpad4), so it is read with 128-bit broadcasts. Scheduling barriers
// on both ends and the pinned results keep one call's taps and window rows
// live only during that call: without them the taps of every band of a phase
// are hoisted at once, or the FMA chains sink to the results' use, and
// registers spill.
constexpr int kpad4(int k) { return (k * k + 3) / 4 * 4; }

template <int K, int OR, int OC, int S>
__device__ __forceinline__ void conv_tile(const float* s, const float* w, float (&acc)[OR][OC]) {
    __builtin_amdgcn_sched_barrier(0);
    float wr[kpad4(K)];
#pragma unroll
    for (int t = 0; t < kpad4(K); t += 4) {
        const float4 q = *reinterpret_cast<const float4*>(w + t);
        wr[t] = q.x;
        wr[t + 1] = q.y;
        wr[t + 2] = q.z;
        wr[t + 3] = q.w;
    }
#pragma unroll
    for (int r = 0; r < OR + K - 1; ++r) {
        float win[OC + K - 1];
#pragma unroll
        for (int q = 0; q < OC + K - 1; ++q) win[q] = s[r * S + q];
#pragma unroll
        for (int o = 0; o < OR; ++o) {
            const int m = r - o;
            if (m < 0 || m >= K) continue;
#pragma unroll
            for (int n = 0; n < K; ++n) {
#pragma unroll
                for (int q = 0; q < OC; ++q) {
                    if (m == 0 && n == 0) acc[o][q] = wr[0] * win[q];
                    else acc[o][q] = __builtin_fmaf(wr[m * K + n], win[q + n], acc[o][q]);
                }
            }
        }
    }
    pin_regs(acc);
    __builtin_amdgcn_sched_barrier(0);
}

// acc[o] += sum_{m,n} w[m][n] * s[(o+m)*S + n] for o < R: a column strip of R
// outputs of a 'same' cross-correlation from a zero-bordered LDS plane
// (s points at the window's top-left corner). Lanes of a wavefront take
// consecutive columns, so every window load is a run of consecutive words
// across the wavefront: no LDS bank conflicts. Each loaded value feeds up to
// K FMAs (the K taps of its column). Same pinning as conv_tile.
template <int K, int R, int S>
__device__ __forceinline__ void conv_col(const float* s, const float* w, float (&acc)[R]) {
    __builtin_amdgcn_sched_barrier(0);
    float wr[kpad4(K)];
#pragma unroll
    for (int t = 0; t < kpad4(K); t += 4) {
        const float4 q = *reinterpret_cast<const float4*>(w + t);
        wr[t] = q.x;
        wr[t + 1] = q.y;
        wr[t + 2] = q.z;
        wr[t + 3] = q.w;
    }
    // window rows double-buffered: row r+1 is requested before row r's
    // multiply-adds, so its LDS latency hides behind them
    constexpr int NR = R + K - 1;
    const RowAddr<S, NR> rows(s);
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
            for (int n = 0; n < K; ++n) {
                if (m == 0 && n == 0) acc[o] = wr[0] * win[r & 1][0];
                else acc[o] = __builtin_fmaf(wr[m * K + n], win[r & 1][n], acc[o]);
            }
        }
    }
    pin_regs(acc);
    __builtin_amdgcn_sched_barrier(0);
}

// Zero the border cells of NB bordered planes of interior h x w, border B,
// row stride S (everything outside rows [B, B+h) x cols [CO, CO+w); the
// interior starts at column CO, B by default).
template <int NB, int h, int w, int B, int S, int CO = B>
__device__ __forceinline__ void zero_border(float* base, int tid, int nt) {
    constexpr int ROWS = h + 2 * B;
    constexpr int TOPBOT = 2 * B * S;
    constexpr int SIDE = S - w;
    constexpr int PER = TOPBOT + h * SIDE;
    if constexpr (PER == 0 || SIDE == 0) {   // no border columns
        for (int i = tid; i < NB * TOPBOT; i += nt) {
            const int b = i / (TOPBOT > 0 ? TOPBOT : 1), j = i - b * TOPBOT, r0 = j / S;
            base[b * ROWS * S + (r0 >= B ? r0 + h : r0) * S + (j - r0 * S)] = 0.f;
        }
        return;
    }
    for (int i = tid; i < NB * PER; i += nt) {
        const int b = i / PER;
        int j = i - b * PER, r, c;
        if (j < TOPBOT) {
            r = j / S;
            c = j - r * S;
            if (r >= B) r += h;
        } else {
            j -= TOPBOT;
            r = B + j / SIDE;
            c = j % SIDE;
            if (c >= CO) c += w;
        }
        base[b * ROWS * S + r * S + c] = 0.f;
    }
}

// The weight gradient's second stage for one channel c: the fixed-order sum
// of the per-chunk partial tap sums, then scale and normalisation. Taps
// [0, TA) (base, levels 1..LA) come from partA, the rest (levels LA+1..L)
// from partB when the plane was split. WG holds 4 L K^2 floats. Run by one
// workgroup (nthreads lanes, tid its lane); c < C.
struct FinalizeArgs {
    const float* partA;
    int nA, LA;
    const float* partB;
    int nB, C, L, KB, K;
    const float* w_lvl;
    const float* scale;
    float* dw_base;
    float* dw_lvl;
    float* dscale;
};

__device__ __forceinline__ void finalize_channel(const FinalizeArgs& f, int c, int tid, int nthreads, float* WG) {
    const int kb2 = f.KB * f.KB, k2 = f.K * f.K, taps = kb2 + 4 * f.L * k2;
    const int TA = kb2 + 4 * f.LA * k2, TB = taps - TA, C = f.C;
    // one tap per lane: the partial sums, the scale and the level tap are
    // all requested before any is used
    for (int t = tid; t < taps; t += nthreads) {
        float sc = 1.f, wv = 0.f;
        size_t pi = 0;
        int tap = 0;
        if (t >= kb2) {
            const int r = t - kb2, ls = r / k2, l = ls / 4, s = ls - 4 * l;
            tap = r - ls * k2;
            pi = ((size_t)l * C + c) * 4 + s;
            sc = f.scale[pi];
            wv = f.w_lvl[pi * k2 + tap];
        }
        float a = 0.f;   // the sum stays in chunk order
        if (t < TA) {
#pragma unroll 8
            for (int ch = 0; ch < f.nA; ++ch) a += f.partA[((size_t)ch * C + c) * TA + t];
        } else {
#pragma unroll 8
            for (int ch = 0; ch < f.nB; ++ch) a += f.partB[((size_t)ch * C + c) * TB + (t - TA)];
        }
        if (t < kb2) {
            f.dw_base[(size_t)c * kb2 + t] = a;
        } else {
            const int l = (t - kb2) / (4 * k2);   // 0-based level
            a *= 1.0f / (float)(1 << (2 * (l + 1)));
            f.dw_lvl[pi * k2 + tap] = sc * a;
            WG[t - kb2] = wv * a;
        }
    }
    __syncthreads();
    for (int ls = tid; ls < 4 * f.L; ls += nthreads) {
        const int l = ls / 4, s = ls - 4 * l;
        float a = 0.f;
        for (int tap = 0; tap < k2; ++tap) a += WG[ls * k2 + tap];
        f.dscale[((size_t)l * C + c) * 4 + s] = a;
    }
}

// Butterfly of one 2x2 block (a b / c d), unnormalised: the four Haar bands
// times 2 (the 1/2 factors are folded into the convolution weights).
__device__ __forceinline__ void haar4(float a, float b, float c, float d, float& ll, float& b1,
                                      float& b2, float& b3) {
    const float s0 = a + b, d0 = a - b, s1 = c + d, d1 = c - d;
    ll = s0 + s1;
    b1 = s0 - s1;
    b2 = d0 + d1;
    b3 = d0 - d1;
}

}  // namespace wtc
