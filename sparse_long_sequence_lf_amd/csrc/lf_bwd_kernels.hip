// lf_bwd_kernels.hip -- gradients of the Longformer sparse self-attention
// forward (dq, dk, dv) for gfx950.
//
// The pages describe no backward pass (Longformer, ciallo.wiki, §5.2 only
// states that training cost grows linearly with the length).  These kernels
// compute the derivative of the forward map over the same allowed pairs:
// with P_ij the softmax weights of row i, dP_ij = dy_i . v_j,
// D_i = sum_j P_ij dP_ij and dS_ij = P_ij (dP_ij - D_i),
//     dq_i = sum_j dS_ij k_j / sqrt(d),  dk_j = sum_i dS_ij q_i / sqrt(d),
//     dv_j = sum_i P_ij dy_i .
// The allowed sets are those of the forward: the sliding window of radius
// r_h with stride delta_h (Longformer, eightmm.github.io, "Sliding-Window
// Attention"; ciallo.wiki §2.2.3), one- or two-sided ("Implementation
// Reading"), the global set G both ways ("Global Attention"), and padded
// keys and queries left out.
//
// Up to six launches on the call's stream; each output row is written by
// exactly one thread:
//   rows_kernel   non-global queries of one residue class: one pass with
//                 online-rescaled sums gives the row's log-sum-exp, D_i and
//                 dq_i; writes (lse_i, D_i) for the column kernels.
//   grows_stats_kernel, grows_dq_kernel
//                 global rows: every valid key, in splits of split_len keys
//                 (one workgroup each, reduced through LDS): the splits'
//                 (max, sum, sum of p dP), then their parts of dq.
//   cols_kernel   lane = a non-global key of one residue class: dk_j, dv_j
//                 from the queries whose window holds j, plus the global rows.
//   gcols_kernel  global keys: every valid query, in splits likewise.
//   combine_kernel  adds the splits' parts of dq, dk, dv of the global positions.
// In the band kernels four lanes share a row (16 channels each) and a wave
// holds 16 rows of one residue class; the other side's rows stream past,
// the next one loaded while the current one is used.  No atomics, so results
// are reproducible.  This is the plain vector-unit path; it does not use MFMA.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lf_bwd.h"

namespace lfb {

constexpr int D = LF_HEAD_DIM;
constexpr float LOG2E = 1.4426950408889634f;

__device__ __forceinline__ float ex2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float lg2(float x) { return __builtin_amdgcn_logf(x); }

// A row of D channels held as fp32 values.
struct RowF {
    float x[D];
};

template <typename ET>
__device__ __forceinline__ void load_row(const ET* __restrict__ p, RowF& r) {
    if constexpr (sizeof(ET) == 2) {
        const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int e = 0; e < D / 8; e++) {
            const uint4 w = p4[e];
            const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int t = 0; t < 4; t++) {
                r.x[8 * e + 2 * t] = __uint_as_float(u[t] << 16);
                r.x[8 * e + 2 * t + 1] = __uint_as_float(u[t] & 0xffff0000u);
            }
        }
    } else {
        const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
        for (int e = 0; e < D / 4; e++) {
            const float4 w = p4[e];
            r.x[4 * e] = w.x;
            r.x[4 * e + 1] = w.y;
            r.x[4 * e + 2] = w.z;
            r.x[4 * e + 3] = w.w;
        }
    }
}

__device__ __forceinline__ void zero_row(RowF& r) {
#pragma unroll
    for (int c = 0; c < D; c++) r.x[c] = 0.f;
}

__device__ __forceinline__ float dot(const RowF& a, const RowF& b) {
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int c = 0; c < D; c += 2) {
        s0 = __builtin_fmaf(a.x[c], b.x[c], s0);
        s1 = __builtin_fmaf(a.x[c + 1], b.x[c + 1], s1);
    }
    return s0 + s1;
}

__device__ __forceinline__ void axpy(RowF& acc, float a, const RowF& x) {
#pragma unroll
    for (int c = 0; c < D; c++) acc.x[c] = __builtin_fmaf(a, x.x[c], acc.x[c]);
}

template <typename ET>
__device__ __forceinline__ void store_row(ET* __restrict__ p, const RowF& r, float scale) {
    if constexpr (sizeof(ET) == 2) {
        uint4* p4 = reinterpret_cast<uint4*>(p);
#pragma unroll
        for (int e = 0; e < D / 8; e++) {
            uint32_t u[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const __bf16 lo = (__bf16)(r.x[8 * e + 2 * t] * scale);
                const __bf16 hi = (__bf16)(r.x[8 * e + 2 * t + 1] * scale);
                u[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            p4[e] = make_uint4(u[0], u[1], u[2], u[3]);
        }
    } else {
        float4* p4 = reinterpret_cast<float4*>(p);
#pragma unroll
        for (int e = 0; e < D / 4; e++)
            p4[e] = make_float4(r.x[4 * e] * scale, r.x[4 * e + 1] * scale, r.x[4 * e + 2] * scale,
                                r.x[4 * e + 3] * scale);
    }
}

__device__ __forceinline__ bool is_global(const uint32_t* __restrict__ gmap, int i) {
    return (gmap[i >> 5] >> (i & 31)) & 1u;
}

__device__ __forceinline__ bool padded(const uint8_t* __restrict__ pad, int i) { return pad && pad[i] != 0; }

// The band kernels give each query (or key) row four lanes, each owning 16
// of its 64 channels: a wave holds 16 rows, dot products end with a sum over
// the four lanes (two DPP steps), and a lane keeps 16-channel slices only.
constexpr int LPR = LFB_LANES_PER_ROW;  // lanes per row
constexpr int NQ = LFB_ROWS_PER_WAVE;   // rows per wave
constexpr int CS = D / LPR;             // channels per lane
static_assert(LPR == 4 || LPR == 8, "four or eight lanes per row");

struct Slice {
    float x[CS];
};

__device__ __forceinline__ void zero_slice(Slice& r) {
#pragma unroll
    for (int c = 0; c < CS; c++) r.x[c] = 0.f;
}

// A lane's 16-channel slice of an input row as loaded: bf16 rows stay packed
// two channels per word (dot products take them as they are, with
// v_dot2_f32_bf16; products of bf16 values are exact in fp32), fp32 rows are
// plain floats.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

template <typename ET>
struct In;
template <>
struct In<__bf16> {
    uint32_t w[CS / 2];
};
template <>
struct In<float> {
    float x[CS];
};

template <typename ET>
__device__ __forceinline__ void load_in(const ET* __restrict__ p, In<ET>& r) {
    if constexpr (sizeof(ET) == 2) {
        const uint4* p4 = reinterpret_cast<const uint4*>(p);
#pragma unroll
        for (int e = 0; e < CS / 8; e++) {
            const uint4 u = p4[e];
            r.w[4 * e] = u.x;
            r.w[4 * e + 1] = u.y;
            r.w[4 * e + 2] = u.z;
            r.w[4 * e + 3] = u.w;
        }
    } else {
        const float4* p4 = reinterpret_cast<const float4*>(p);
#pragma unroll
        for (int e = 0; e < CS / 4; e++) {
            const float4 u = p4[e];
            r.x[4 * e] = u.x;
            r.x[4 * e + 1] = u.y;
            r.x[4 * e + 2] = u.z;
            r.x[4 * e + 3] = u.w;
        }
    }
}

template <typename ET>
__device__ __forceinline__ void zero_in(In<ET>& r) {
    if constexpr (sizeof(ET) == 2) {
#pragma unroll
        for (int e = 0; e < CS / 2; e++) r.w[e] = 0u;
    } else {
#pragma unroll
        for (int c = 0; c < CS; c++) r.x[c] = 0.f;
    }
}

template <typename ET>
__device__ __forceinline__ float dot_in(const In<ET>& a, const In<ET>& b) {
    float s0 = 0.f, s1 = 0.f;
    if constexpr (sizeof(ET) == 2) {
#pragma unroll
        for (int e = 0; e < CS / 2; e += 2) {
            s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w[e]),
                                                 __builtin_bit_cast(bf16x2_t, b.w[e]), s0, false);
            s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a.w[e + 1]),
                                                 __builtin_bit_cast(bf16x2_t, b.w[e + 1]), s1, false);
        }
    } else {
#pragma unroll
        for (int c = 0; c < CS; c += 2) {
            s0 = __builtin_fmaf(a.x[c], b.x[c], s0);
            s1 = __builtin_fmaf(a.x[c + 1], b.x[c + 1], s1);
        }
    }
    return s0 + s1;
}

// acc += a * x (x widened to fp32)
template <typename ET>
__device__ __forceinline__ void axpy_in(Slice& acc, float a, const In<ET>& x) {
    if constexpr (sizeof(ET) == 2) {
#pragma unroll
        for (int e = 0; e < CS / 2; e++) {
            acc.x[2 * e] = __builtin_fmaf(a, __uint_as_float(x.w[e] << 16), acc.x[2 * e]);
            acc.x[2 * e + 1] = __builtin_fmaf(a, __uint_as_float(x.w[e] & 0xffff0000u), acc.x[2 * e + 1]);
        }
    } else {
#pragma unroll
        for (int c = 0; c < CS; c++) acc.x[c] = __builtin_fmaf(a, x.x[c], acc.x[c]);
    }
}

// acc += a * x for a bf16 row x without widening it: each channel pair takes
// two v_dot2_f32_bf16 against (a, 0) and (0, a), a rounded to bf16 (a
// relative error of at most 2^-9 per term; fp32 rows take plain FMAs).
template <typename ET>
__device__ __forceinline__ void axpy_w(Slice& acc, float a, const In<ET>& x) {
    if constexpr (sizeof(ET) == 2) {
        const uint32_t ab = (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)a);
        const bf16x2_t lo = __builtin_bit_cast(bf16x2_t, ab), hi = __builtin_bit_cast(bf16x2_t, ab << 16);
#pragma unroll
        for (int e = 0; e < CS / 2; e++) {
            const bf16x2_t xe = __builtin_bit_cast(bf16x2_t, x.w[e]);
            acc.x[2 * e] = __builtin_amdgcn_fdot2_f32_bf16(xe, lo, acc.x[2 * e], false);
            acc.x[2 * e + 1] = __builtin_amdgcn_fdot2_f32_bf16(xe, hi, acc.x[2 * e + 1], false);
        }
    } else {
        axpy_in(acc, a, x);
    }
}

// Sum over the LPR lanes of a row (an aligned group), in every lane of it.
__device__ __forceinline__ float quad_sum(float x) {
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));  // lane ^ 1
    x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));  // lane ^ 2
    if constexpr (LPR == 8)   // the other quad of the group of 8 (lane i reads lane 7 - i)
        x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
    return x;
}

template <typename ET>
__device__ __forceinline__ void store_slice(ET* __restrict__ p, const Slice& r, float scale) {
    if constexpr (sizeof(ET) == 2) {
        uint4* p4 = reinterpret_cast<uint4*>(p);
#pragma unroll
        for (int e = 0; e < CS / 8; e++) {
            uint32_t u[4];
#pragma unroll
            for (int t = 0; t < 4; t++) {
                const __bf16 lo = (__bf16)(r.x[8 * e + 2 * t] * scale);
                const __bf16 hi = (__bf16)(r.x[8 * e + 2 * t + 1] * scale);
                u[t] = (uint32_t)__builtin_bit_cast(uint16_t, lo) | ((uint32_t)__builtin_bit_cast(uint16_t, hi) << 16);
            }
            p4[e] = make_uint4(u[0], u[1], u[2], u[3]);
        }
    } else {
        float4* p4 = reinterpret_cast<float4*>(p);
#pragma unroll
        for (int e = 0; e < CS / 4; e++)
            p4[e] = make_float4(r.x[4 * e] * scale, r.x[4 * e + 1] * scale, r.x[4 * e + 2] * scale,
                                r.x[4 * e + 3] * scale);
    }
}

// One wave's share of the band kernels: batch b, head h, residue class c of
// stride delta, and class positions [t0, t0 + NQ) of the nc in the class.
struct Chunk {
    int b, h, c, t0, nc, delta, r, ra;
};

__device__ __forceinline__ bool decode(const lfk::BwdArgs& A, long long task, Chunk& k) {
    const long long per_b = A.head_chunk[A.H];
    if (task >= (long long)A.B * per_b) return false;
    k.b = (int)(task / per_b);
    int rem = (int)(task - (long long)k.b * per_b);
    int o = 0;
    while (o + 1 < A.H && A.head_chunk[o + 1] <= rem) o++;
    rem -= A.head_chunk[o];
    const int h = A.hord[o];
    k.h = h;
    const int delta = A.dil[h];
    const int T = A.T;
    const int q = T / delta, rm = T - q * delta;
    const int ch1 = (q + NQ) / NQ, ch0 = (q + NQ - 1) / NQ;   // chunks of a class with q+1 / q members
    if (rem < rm * ch1) {
        k.c = rem / ch1;
        k.t0 = (rem - k.c * ch1) * NQ;
        k.nc = q + 1;
    } else {
        rem -= rm * ch1;
        k.c = rm + rem / ch0;
        k.t0 = (rem % ch0) * NQ;
        k.nc = q;
    }
    k.delta = delta;
    k.r = A.rad[h];
    k.ra = A.one_sided ? 0 : k.r;
    return true;
}

// The class positions in [lo, hi] whose row is neither padded nor global, in
// ascending order: one ballot over 64 positions at a time (each lane tests
// one), then scalar bit scans.  Every value is wave-uniform.
struct ClassScan {
    const lfk::BwdArgs& A;
    const Chunk& ck;
    const uint8_t* pad;
    int hi, lane, base;
    uint64_t mask;
    __device__ ClassScan(const lfk::BwdArgs& A_, const Chunk& ck_, const uint8_t* pad_, int lo, int hi_, int lane_)
        : A(A_), ck(ck_), pad(pad_), hi(hi_), lane(lane_) {
        reset(lo);
    }
    __device__ void refill(int b) {
        base = b;
        const int x = b + lane;
        bool ok = false;
        if (x <= hi) {
            const int j = ck.c + x * ck.delta;
            ok = !padded(pad, j) && !(A.n_g > 0 && is_global(A.gmap, j));
        }
        mask = __ballot(ok);
    }
    __device__ void reset(int lo) { refill(lo); }
    // smallest listed position >= x (x never below the previous answer), or hi + 1
    __device__ int operator()(int x) {
        for (;;) {
            if (x > hi) return hi + 1;
            if (x >= base + 64) refill(x);
            const uint64_t m = mask >> (x - base);
            if (m) return x + __builtin_ctzll(m);
            x = base + 64;
        }
    }
};

// Visit the listed class positions from lo on in ascending order, with the
// rows of the next PF positions loaded ahead (a ring of PF register slots,
// unrolled so that every slot index is static).
template <int PF, typename Load, typename Use>
__device__ __forceinline__ void stream_rows(ClassScan& next, int lo, Load load, Use use) {
    using Item = decltype(load(0));
    const int hi = next.hi;
    Item buf[PF];
    int pos[PF];
    int tk = next(lo);
#pragma unroll
    for (int p = 0; p < PF; p++) {
        pos[p] = tk;
        if (tk <= hi) {
            buf[p] = load(tk);
            tk = next(tk + 1);
        }
    }
    bool done = false;
    while (!done) {
#pragma unroll
        for (int p = 0; p < PF; p++) {
            if (!done && pos[p] > hi) done = true;
            if (!done) {
                use(buf[p], pos[p]);
                pos[p] = tk;
                if (tk <= hi) {
                    buf[p] = load(tk);
                    tk = next(tk + 1);
                }
            }
        }
    }
}

template <typename ET>
struct KV {
    In<ET> k, v;
};
template <typename ET>
struct QY {
    In<ET> q, y;
    float2 st;
};

// rows loaded ahead: four for bf16 rows, two for the twice larger fp32 rows
template <typename ET>
constexpr int PREFETCH = sizeof(ET) == 2 ? 4 : 2;

// ---------------------------------------------------------------------------
// dq and the row statistics of the non-global queries.

template <typename ET>
__global__ __launch_bounds__(256) void rows_kernel(const lfk::BwdArgs A, const ET* __restrict__ Q,
                                                   const ET* __restrict__ K, const ET* __restrict__ V,
                                                   const ET* __restrict__ DY, ET* __restrict__ DQ,
                                                   float2* __restrict__ stats) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    Chunk ck;
    if (!decode(A, (long long)blockIdx.x * 4 + wave, ck)) return;
    const int T = A.T;
    const size_t bh = (size_t)ck.b * A.H + ck.h;
    const int part = lane & (LPR - 1);
    const ET* Kh = K + bh * T * D + CS * part;
    const ET* Vh = V + bh * T * D + CS * part;
    const uint8_t* pad = A.pad ? A.pad + (size_t)ck.b * T : nullptr;
    const int t = ck.t0 + lane / LPR;
    const bool in = t < ck.nc;
    const int i = ck.c + t * ck.delta;
    const bool glob_i = in && A.n_g > 0 && is_global(A.gmap, i);
    const bool live = in && !glob_i && !padded(pad, i);
    In<ET> q, dy;
    if (live) {
        load_in(Q + (bh * T + i) * D + CS * part, q);
        load_in(DY + (bh * T + i) * D + CS * part, dy);
    } else {
        zero_in(q);
        zero_in(dy);
    }
    const float sc = LOG2E / 8.0f;   // 1/sqrt(64), base 2
    const int k_lo = max(ck.t0 - ck.r, 0), k_hi = min(ck.t0 + NQ - 1 + ck.ra, ck.nc - 1);
    // next class position >= x whose key is neither padded nor global (the
    // globals take their own loop), or k_hi + 1
    ClassScan next_key(A, ck, pad, k_lo, k_hi, lane);
    auto in_window = [&](int tk) { return live && tk - t >= -ck.r && tk - t <= ck.ra; };

    // One pass with a running reference max m (base 2): l = sum e, dn = sum
    // e dP, A = sum e dP k, Bk = sum e k with e = 2^(s - m).  Then
    // lse = m + log2 l, D = dn / l and dq = (A - D Bk) / (8 l), the chain rule
    // sum_j P_ij (dP_ij - D_i) k_j / sqrt(d) regrouped.  m is moved (and the
    // sums rescaled) only when a score passes it by more than 8, so e stays
    // below 2^8.
    float m = -INFINITY, l = 0.f, dn = 0.f;
    Slice Aq, Bk;
    zero_slice(Aq);
    zero_slice(Bk);
    auto accum = [&](const In<ET>& kr, const In<ET>& vr, bool on) {
        const float s = quad_sum(dot_in(q, kr)) * sc;
        const float dp = quad_sum(dot_in(dy, vr));
        if (on && s > m + 8.f) {
            const float al = ex2(m - s);
            l *= al;
            dn *= al;
#pragma unroll
            for (int c = 0; c < CS; c++) {
                Aq.x[c] *= al;
                Bk.x[c] *= al;
            }
            m = s;
        }
        const float e = on ? ex2(s - m) : 0.f;
        l += e;
        dn += e * dp;
        axpy_in(Aq, e * dp, kr);
        axpy_in(Bk, e, kr);
    };
    auto load_kv = [&](int tk) {
        KV<ET> x;
        load_in(Kh + (size_t)(ck.c + tk * ck.delta) * D, x.k);
        load_in(Vh + (size_t)(ck.c + tk * ck.delta) * D, x.v);
        return x;
    };
    stream_rows<PREFETCH<ET>>(next_key, k_lo, load_kv,
                              [&](const KV<ET>& x, int tk) { accum(x.k, x.v, in_window(tk)); });
    for (int g = 0; g < A.n_g; g++) {
        const int j = A.glob[g];
        if (padded(pad, j)) continue;
        In<ET> kr, vr;
        load_in(Kh + (size_t)j * D, kr);
        load_in(Vh + (size_t)j * D, vr);
        accum(kr, vr, live);
    }
    if (A.n_rand > 0) {
        // the random key blocks of this wave's query block (undilated, so
        // class position = position and the 16 queries share one block);
        // keys already in a query's window count there
        const int32_t* rb = A.rtab + ((size_t)ck.h * ((T + 63) >> 6) + (ck.t0 >> 6)) * A.n_rand;
        for (int e = 0; e < A.n_rand; e++) {
            const int rho = rb[e];
            if (rho < 0) break;   // the list is ascending, -1 after the last
            ClassScan rnd(A, ck, pad, 64 * rho, min(64 * rho + 63, T - 1), lane);
            stream_rows<PREFETCH<ET>>(rnd, 64 * rho, load_kv, [&](const KV<ET>& x, int tk) {
                accum(x.k, x.v, live && !(tk - t >= -ck.r && tk - t <= ck.ra));
            });
        }
    }
    const float lse = live ? m + lg2(l) : 0.f;
    const float Dl = live ? dn / l : 0.f;
    const float inv = live ? 1.f / l : 0.f;
    Slice acc;
#pragma unroll
    for (int c = 0; c < CS; c++) acc.x[c] = (Aq.x[c] - Dl * Bk.x[c]) * inv;
    if (in && !glob_i) {
        store_slice(DQ + (bh * T + i) * D + CS * part, acc, 0.125f);
        if (part == 0) stats[bh * T + i] = make_float2(lse, Dl);
    }
}

// ---------------------------------------------------------------------------
// dk and dv of the non-global keys.

template <typename ET>
__global__ __launch_bounds__(256) void cols_kernel(const lfk::BwdArgs A, const ET* __restrict__ Q,
                                                   const ET* __restrict__ K, const ET* __restrict__ V,
                                                   const ET* __restrict__ DY, ET* __restrict__ DK,
                                                   ET* __restrict__ DV, const float2* __restrict__ stats) {
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    Chunk ck;
    if (!decode(A, (long long)blockIdx.x * 4 + wave, ck)) return;
    const int T = A.T;
    const size_t bh = (size_t)ck.b * A.H + ck.h;
    const int part = lane & (LPR - 1);
    const ET* Qh = Q + bh * T * D + CS * part;
    const ET* Yh = DY + bh * T * D + CS * part;
    const float2* Sh = stats + bh * T;
    const uint8_t* pad = A.pad ? A.pad + (size_t)ck.b * T : nullptr;
    const int t = ck.t0 + lane / LPR;
    const bool in = t < ck.nc;
    const int j = ck.c + t * ck.delta;
    const bool glob_j = in && A.n_g > 0 && is_global(A.gmap, j);
    const bool live = in && !glob_j && !padded(pad, j);
    In<ET> kr, vr;
    if (live) {
        load_in(K + (bh * T + j) * D + CS * part, kr);
        load_in(V + (bh * T + j) * D + CS * part, vr);
    } else {
        zero_in(kr);
        zero_in(vr);
    }
    const float sc = LOG2E / 8.0f;
    Slice dk, dv;
    zero_slice(dk);
    zero_slice(dv);
    auto acc = [&](const In<ET>& q, const In<ET>& dy, float2 st, bool on) {
        const float s = quad_sum(dot_in(q, kr)) * sc;
        const float dp = quad_sum(dot_in(dy, vr));
        const float p = on ? ex2(s - st.x) : 0.f;
        axpy_w(dv, p, dy);
        axpy_w(dk, p * (dp - st.y), q);
    };
    // query i (class position tq) holds key position t in its window iff
    // tq - t lies in [-ra, r]
    const int q_lo = max(ck.t0 - ck.ra, 0), q_hi = min(ck.t0 + NQ - 1 + ck.r, ck.nc - 1);
    ClassScan next_query(A, ck, pad, q_lo, q_hi, lane);
    auto load_qy = [&](int tq) {
        QY<ET> x;
        const size_t i = ck.c + (size_t)tq * ck.delta;
        load_in(Qh + i * D, x.q);
        load_in(Yh + i * D, x.y);
        x.st = Sh[i];
        return x;
    };
    stream_rows<PREFETCH<ET>>(next_query, q_lo, load_qy, [&](const QY<ET>& x, int tq) {
        acc(x.q, x.y, x.st, live && tq - t >= -ck.ra && tq - t <= ck.r);
    });
    for (int g = 0; g < A.n_g; g++) {
        const int i = A.glob[g];
        if (padded(pad, i)) continue;
        In<ET> q, dy;
        load_in(Qh + (size_t)i * D, q);
        load_in(Yh + (size_t)i * D, dy);
        acc(q, dy, Sh[i], live);
    }
    if (A.n_rand > 0) {
        // the query blocks that drew this wave's key block (undilated); a
        // query whose window already holds the key counts there
        const int kb = ck.t0 >> 6;
        const int32_t* off = A.inv_off + (size_t)ck.h * (((T + 63) >> 6) + 1);
        for (int e = off[kb]; e < off[kb + 1]; e++) {
            const int beta = A.inv_list[e];
            ClassScan rnd(A, ck, pad, 64 * beta, min(64 * beta + 63, T - 1), lane);
            stream_rows<PREFETCH<ET>>(rnd, 64 * beta, load_qy, [&](const QY<ET>& x, int tq) {
                acc(x.q, x.y, x.st, live && !(tq - t >= -ck.ra && tq - t <= ck.r));
            });
        }
    }
    if (in && !glob_j) {
        store_slice(DK + (bh * T + j) * D + CS * part, dk, 0.125f);
        store_slice(DV + (bh * T + j) * D + CS * part, dv, 1.0f);
    }
}

// ---------------------------------------------------------------------------
// Global rows and global keys.  Each (b, h, global position) is split into
// n_split ranges of split_len positions, one workgroup per range (256
// threads, split_len / 256 positions each); partial results go to gstat and
// gpart, and combine_kernel adds them up.

// Sum x[tid][c] over the 256 threads into thread c < 64; red holds 256 x 65
// floats.  Each thread first adds a quarter of one channel's column (64
// rows), then 64 threads add the four quarters.
__device__ __forceinline__ float block_sum_row(float* red, const RowF& x) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int c = 0; c < D; c++) red[tid * 65 + c] = x.x[c];
    __syncthreads();
    const int c = tid & 63, r0 = (tid >> 6) * 64;
    float s = 0.f;
    for (int e = 0; e < 64; e++) s += red[(r0 + e) * 65 + c];
    __syncthreads();
    red[tid] = s;
    __syncthreads();
    if (tid < D) s = red[tid] + red[64 + tid] + red[128 + tid] + red[192 + tid];
    __syncthreads();
    return s;
}

struct GTask {
    size_t bh, rec;   // (b*H + h), record index (b*H + h)*n_g + gi
    int b, g, sp, lo, hi;
};

__device__ __forceinline__ GTask gtask(const lfk::BwdArgs& A) {
    GTask t;
    t.sp = blockIdx.x % A.n_split;
    t.rec = blockIdx.x / A.n_split;
    const int gi = (int)(t.rec % A.n_g);
    t.bh = t.rec / A.n_g;
    t.b = (int)(t.bh / A.H);
    t.g = A.glob[gi];
    t.lo = t.sp * A.split_len;
    t.hi = min(t.lo + A.split_len, A.T);
    return t;
}

// pass 1 of a global row: (max, sum, sum of p dP) over the split's keys
template <typename ET>
__global__ __launch_bounds__(256) void grows_stats_kernel(const lfk::BwdArgs A, const ET* __restrict__ Q,
                                                          const ET* __restrict__ K, const ET* __restrict__ V,
                                                          const ET* __restrict__ DY) {
    __shared__ float red_m[256], red_l[256], red_d[256];
    const int tid = threadIdx.x;
    const GTask t = gtask(A);
    const int T = A.T;
    const uint8_t* pad = A.pad ? A.pad + (size_t)t.b * T : nullptr;
    float m = -INFINITY, l = 0.f, dn = 0.f;
    if (!padded(pad, t.g)) {
        const ET* Kh = K + t.bh * T * D;
        const ET* Vh = V + t.bh * T * D;
        RowF q, dy;
        load_row(Q + (t.bh * T + t.g) * D, q);
        load_row(DY + (t.bh * T + t.g) * D, dy);
        const float sc = LOG2E / 8.0f;
        for (int j = t.lo + tid; j < t.hi; j += 256) {
            if (padded(pad, j)) continue;
            RowF kr, vr;
            load_row(Kh + (size_t)j * D, kr);
            load_row(Vh + (size_t)j * D, vr);
            const float s = dot(q, kr) * sc;
            const float dp = dot(dy, vr);
            const float mn = fmaxf(m, s);
            const float al = ex2(m - mn), e = ex2(s - mn);
            l = l * al + e;
            dn = dn * al + e * dp;
            m = mn;
        }
    }
    red_m[tid] = m;
    red_l[tid] = l;
    red_d[tid] = dn;
    __syncthreads();
    if (tid == 0) {
        float M = -INFINITY;
        for (int e = 0; e < 256; e++) M = fmaxf(M, red_m[e]);
        float L = 0.f, DN = 0.f;
        for (int e = 0; e < 256; e++) {
            if (red_l[e] == 0.f) continue;   // a thread that met no valid key
            const float w = ex2(red_m[e] - M);
            L += red_l[e] * w;
            DN += red_d[e] * w;
        }
        A.gstat[t.rec * A.n_split + t.sp] = make_float4(M, L, DN, 0.f);
    }
}

// pass 2 of a global row: the split's part of dq; split 0 also writes the
// row's (lse, D) for the column kernels
template <typename ET>
__global__ __launch_bounds__(256) void grows_dq_kernel(const lfk::BwdArgs A, const ET* __restrict__ Q,
                                                       const ET* __restrict__ K, const ET* __restrict__ V,
                                                       const ET* __restrict__ DY, float2* __restrict__ stats) {
    __shared__ float red[256 * 65];
    const int tid = threadIdx.x;
    const GTask t = gtask(A);
    const int T = A.T;
    const uint8_t* pad = A.pad ? A.pad + (size_t)t.b * T : nullptr;
    RowF acc;
    zero_row(acc);
    if (!padded(pad, t.g)) {
        // the row's statistics from every split's record
        const float4* gs = A.gstat + t.rec * A.n_split;
        float M = -INFINITY;
        for (int e = 0; e < A.n_split; e++) M = fmaxf(M, gs[e].x);
        float L = 0.f, DN = 0.f;
        for (int e = 0; e < A.n_split; e++) {
            const float4 r = gs[e];
            if (r.y == 0.f) continue;
            const float w = ex2(r.x - M);
            L += r.y * w;
            DN += r.z * w;
        }
        const float lse = M + lg2(L), Dl = DN / L;   // key g itself is valid, so L >= 1
        if (t.sp == 0 && tid == 0) stats[t.bh * T + t.g] = make_float2(lse, Dl);
        const ET* Kh = K + t.bh * T * D;
        const ET* Vh = V + t.bh * T * D;
        RowF q, dy;
        load_row(Q + (t.bh * T + t.g) * D, q);
        load_row(DY + (t.bh * T + t.g) * D, dy);
        const float sc = LOG2E / 8.0f;
        for (int j = t.lo + tid; j < t.hi; j += 256) {
            if (padded(pad, j)) continue;
            RowF kr, vr;
            load_row(Kh + (size_t)j * D, kr);
            load_row(Vh + (size_t)j * D, vr);
            const float s = dot(q, kr) * sc;
            const float dp = dot(dy, vr);
            axpy(acc, ex2(s - lse) * (dp - Dl), kr);
        }
    }
    const float sum = block_sum_row(red, acc);
    if (tid < D) A.gpart[(t.rec * A.n_split + t.sp) * 192 + tid] = sum;
}

// a global key: the split's part of dk and dv (every valid query attends to it)
template <typename ET>
__global__ __launch_bounds__(256) void gcols_kernel(const lfk::BwdArgs A, const ET* __restrict__ Q,
                                                    const ET* __restrict__ K, const ET* __restrict__ V,
                                                    const ET* __restrict__ DY, const float2* __restrict__ stats) {
    __shared__ float red[256 * 65];
    const int tid = threadIdx.x;
    const GTask t = gtask(A);
    const int T = A.T;
    const uint8_t* pad = A.pad ? A.pad + (size_t)t.b * T : nullptr;
    RowF ak, av;
    zero_row(ak);
    zero_row(av);
    if (!padded(pad, t.g)) {
        const ET* Qh = Q + t.bh * T * D;
        const ET* Yh = DY + t.bh * T * D;
        RowF kr, vr;
        load_row(K + (t.bh * T + t.g) * D, kr);
        load_row(V + (t.bh * T + t.g) * D, vr);
        const float sc = LOG2E / 8.0f;
        for (int i = t.lo + tid; i < t.hi; i += 256) {
            if (padded(pad, i)) continue;
            RowF q, dy;
            load_row(Qh + (size_t)i * D, q);
            load_row(Yh + (size_t)i * D, dy);
            const float2 st = stats[t.bh * T + i];
            const float s = dot(q, kr) * sc;
            const float dp = dot(dy, vr);
            const float p = ex2(s - st.x);
            axpy(av, p, dy);
            axpy(ak, p * (dp - st.y), q);
        }
    }
    const float sk = block_sum_row(red, ak);
    const float sv = block_sum_row(red, av);
    float* rec = A.gpart + (t.rec * A.n_split + t.sp) * 192;
    if (tid < D) {
        rec[64 + tid] = sk;
        rec[128 + tid] = sv;
    }
}

// dq of each global row and dk, dv of each global key: the sum of the splits
// (zero at a padded position)
template <typename ET>
__global__ __launch_bounds__(64) void combine_kernel(const lfk::BwdArgs A, ET* __restrict__ DQ,
                                                     ET* __restrict__ DK, ET* __restrict__ DV) {
    const int c = threadIdx.x;
    const size_t rec = blockIdx.x;
    const int gi = (int)(rec % A.n_g);
    const size_t bh = rec / A.n_g;
    const int b = (int)(bh / A.H);
    const int g = A.glob[gi];
    const int T = A.T;
    float sq = 0.f, sk = 0.f, sv = 0.f;
    if (!padded(A.pad ? A.pad + (size_t)b * T : nullptr, g)) {
        const float* p = A.gpart + rec * A.n_split * 192;
        for (int e = 0; e < A.n_split; e++) {
            sq += p[e * 192 + c];
            sk += p[e * 192 + 64 + c];
            sv += p[e * 192 + 128 + c];
        }
    }
    const size_t o = (bh * T + g) * D + c;
    DQ[o] = (ET)(sq * 0.125f);
    DK[o] = (ET)(sk * 0.125f);
    DV[o] = (ET)sv;
}

template <typename ET>
hipError_t launch(const lfk::BwdArgs* A, const void* const* t, hipStream_t s) {
    const ET* q = (const ET*)t[0];
    const ET* k = (const ET*)t[1];
    const ET* v = (const ET*)t[2];
    const ET* dy = (const ET*)t[3];
    ET* dq = (ET*)t[4];
    ET* dk = (ET*)t[5];
    ET* dv = (ET*)t[6];
    float2* st = (float2*)A->stats;
    const long long waves = (long long)A->B * A->head_chunk[A->H];   // one wave per chunk of NQ rows
    const dim3 gl((unsigned)((waves + 3) / 4)), blk(256);
    const long long recs = (long long)A->B * A->H * A->n_g;
    const dim3 gs((unsigned)(recs * A->n_split)), gc((unsigned)recs);
    hipLaunchKernelGGL(rows_kernel<ET>, gl, blk, 0, s, *A, q, k, v, dy, dq, st);
    if (A->n_g > 0) {
        hipLaunchKernelGGL(grows_stats_kernel<ET>, gs, blk, 0, s, *A, q, k, v, dy);
        hipLaunchKernelGGL(grows_dq_kernel<ET>, gs, blk, 0, s, *A, q, k, v, dy, st);
    }
    hipLaunchKernelGGL(cols_kernel<ET>, gl, blk, 0, s, *A, q, k, v, dy, dk, dv, st);
    if (A->n_g > 0) {
        hipLaunchKernelGGL(gcols_kernel<ET>, gs, blk, 0, s, *A, q, k, v, dy, st);
        hipLaunchKernelGGL(combine_kernel<ET>, gc, dim3(64), 0, s, *A, dq, dk, dv);
    }
    return hipGetLastError();
}

}  // namespace lfb

// t = {q, k, v, dy, dq, dk, dv}
extern "C" hipError_t lfk_bwd_launch(const lfk::BwdArgs* A, const void* const* t, int dtype_bf16, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    return dtype_bf16 ? lfb::launch<__bf16>(A, t, s) : lfb::launch<float>(A, t, s);
}
