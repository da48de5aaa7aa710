// lf_fwd_kernels.hip -- gfx950 (CDNA4) kernels of the Longformer sparse
// self-attention forward pass.
//
// One tile kernel serves two task kinds that share a grid:
//
//  * band tasks: one tile of 64 consecutive queries of one dilation residue
//    class c of head (b, h), against the keys of that class inside the
//    window (Longformer, eightmm.github.io, "Sliding-Window Attention"),
//    then the global keys G (same page, "Global Attention": every ordinary
//    token also reads G; a global key already inside the window counts once)
//    and, when asked for, random key blocks (BigBird's random attention as
//    the mhpn.cn guide to long-text models sets it beside Longformer);
//  * global-row tasks: up to 64 global queries of head (b, h) against one
//    contiguous split of all T keys ("Global Attention": a global token
//    reads every position).  Each writes partial (max, sum, weighted-sum)
//    records; the last split of a head to finish rescales and adds them.
//
// Residue classes: with stride delta the positions c, c+delta, c+2*delta,
// ... form an undilated sequence of length n_c = ceil((T-c)/delta) on which
// the dilated window is an ordinary window of radius r (Longformer,
// ciallo.wiki §2.2.3; "Longformer长序列处理", 膨胀窗口设计).  Tiles are cut in
// class coordinates, so no MFMA work is spent on keys of other classes.
//
// Per wave: 32 queries.  S^T = K Q^T and O^T = V^T P^T are computed with
// v_mfma_f32_32x32x16_bf16, so every lane owns one query (column) in both
// accumulators and the softmax needs one cross-lane exchange (lanes l and
// l^32 hold the two halves of a query's keys).  The softmax is the running
// max/sum form (blockwise accumulation, "Longformer长序列处理", 显存优化技巧)
// kept in base 2 with the 1/sqrt(d) scale folded into one FMA; the running
// max only moves (and O is rescaled) when a block raises it by more than
// 2^8, which keeps every exponent <= 8 and leaves O / l exact.  Row sums are
// fp32 adds: v_dot2 shares the matrix cores' issue and stalls beside them.
//
// Key blocks (32 keys) reach LDS straight from memory (buffer_load ... lds)
// through a ring of stages of two blocks (one per key phase).  The band part
// of a tile runs a lean step: one barrier, this wave's fragment reads, the
// next stage's loads, the score MFMAs, softmax and PV; edge blocks take the
// window mask, interior blocks none.  Global-key and random blocks, and a
// stage that mixes them with band blocks, take the general step.
//
// fp32 inputs: a pre-pass splits K and V into three bf16 planes (hi, mid,
// lo: 24 significand bits in all) and Q and the weights are split the same
// way in registers; each product adds the six plane products whose weight
// is at least 2^-16 of the leading one, so scores and outputs carry fp32's
// own rounding error while the tiling, masking and softmax are the bf16
// path's code.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>
#include <type_traits>

#include "lf_kernels.h"
#include "lf_decode.h"
#include "lf_device.h"

namespace lfk {

constexpr int BM = LFK_BM;                // queries per band tile

template <typename T> struct Elem;
template <> struct Elem<__bf16> { static constexpr int NP = 1; };
template <> struct Elem<float> { static constexpr int NP = 3; };

// ---------------------------------------------------------------------------
// LDS layout.  A block holds, per bf16 plane (NP = 1 for bf16, 3 for the
// planes of fp32), 32 K rows then 32 V rows:
//
//   K: byte ks*1024 + row*32 + hs*16 holds channels 16ks + 8h .. +7 with
//      hs = h ^ ((row >> 3) & 1).  The 16 lanes of one ds_read_b128 (rows
//      t..t+15, one h) then touch 16 distinct 4-bank groups.
//   V: byte HALF + cb*2048 + row*64 + 16j holds channels 32cb + 8j .. +7.
//      Half a wave of ds_read_b64_tr_b16 reads rows t..t+3 x 64 B: 256
//      consecutive bytes, all 64 banks once.
//
// Each 1 KiB piece (a K slice of 16 channels, or 16 V rows of one cb) is
// what one buffer_load_dwordx4 ... lds of 64 lanes writes, lane p at byte
// 16p.  A stage is two blocks (one per key phase); the ring holds NBUF
// stages, two where LDS allows, else one (then each step waits for every
// wave's fragment reads before the next stage's loads).
template <int D, int NP>
struct Geo {
    static constexpr int KS = D / 16;          // k-steps of S^T = K Q^T
    static constexpr int CB = D / 32;          // 32-channel blocks of O^T
    static constexpr int HALF = 32 * D * 2;    // 32 rows of one plane of K (or V)
    static constexpr int PLANE = 2 * HALF;
    static constexpr int BLK = NP * PLANE;
    static constexpr int STAGE = 2 * BLK;
    static constexpr int NBUF = (2 * STAGE + 8192 <= 160 * 1024) ? 2 : 1;
    static constexpr int RING = NBUF * STAGE;
    static constexpr int ROWB = NP * D * 2;    // bytes per K/V row read by the loaders
    static constexpr int PPW = NP * KS;        // 1 KiB pieces one wave loads per stage (half a block)
    static constexpr int gposOff = RING;                         // global positions (sorted)
    static constexpr int gldOff = gposOff + 4 * LF_MAX_GLOBALS;  // position each slot loads (T: none)
    static constexpr int gclsOff = gldOff + 4 * LF_MAX_GLOBALS;  // class index, or kNotInClass
    static constexpr int gbadOff = gclsOff + 4 * LF_MAX_GLOBALS; // per global block: missing / padded slots
    static constexpr int bytes = gbadOff + 4 * (LF_MAX_GLOBALS / 32);
    static constexpr int REC = (D + 4) * 4;    // global-row partial record: O[D], m, l, 0, 0
    static_assert(2 * 64 * (16 * CB + 4) * 4 <= RING, "phase merge area inside the ring");
};

// waves per SIMD each instantiation is compiled for (registers: 512 / that).
// bf16 at d = 64 with both padding and random blocks takes three: at four it
// spilled 20 bytes a lane.
template <int D, int NP, bool PAD, bool RAND> struct Occupancy {
    static constexpr int v = NP == 1 ? (D == 128 ? 2 : (D == 64 && PAD && RAND ? 3 : 4)) : (D == 32 ? 2 : 1);
};

// the plane products of a split product a*b, smallest first: with three
// parts per operand the six (i, j) with i + j <= 2; with one part (bf16) the
// single product
template <int NP> struct Prods;
template <> struct Prods<1> { static constexpr int n = 1; static constexpr int a[1] = {0}; static constexpr int b[1] = {0}; };
template <> struct Prods<3> {
    static constexpr int n = 6;
    static constexpr int a[6] = {1, 2, 0, 1, 0, 0};
    static constexpr int b[6] = {1, 0, 2, 0, 1, 0};
};

// ---------------------------------------------------------------------------
// task description (all wave-uniform)

struct Task {
    int kind;        // 0 = band tile, 1 = global-row split
    int b, h, bh;
    int delta, c;    // residue class (band); delta = 1, c = 0 for global-row tasks
    int n;           // class length (band) / T (global rows)
    int m0;          // first query (class index) of the tile / first global slot
    int kb_lo;       // first key block (class block index)
    int nband;       // band (or dense) key blocks
    int key_end;     // keys >= key_end are out of range (class index)
    int split;       // global-row tasks: split index
    int r, ra;       // band: the window reaches r keys back and ra forward (ra = 0 one-sided)
};

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

// Task t from the kernel argument's decode fields (every head with the same
// stride and radius): the same Task as decode_task, with no memory access.
__device__ __forceinline__ Task decode_task_fast(const FastDecode& f, int t) {
    Task k;
    if (t < f.n_band) {
        k.kind = 0;
        k.bh = mdiv(t, f.mg_tph);
        const int x = t - k.bh * f.tph;
        k.b = mdiv(k.bh, f.mg_H);
        k.h = k.bh - k.b * f.H;
        k.delta = f.delta;
        int tile;
        if (f.delta == 1) {
            k.c = 0;
            tile = x;
            k.n = f.T;
        } else if (x < f.hrem * f.htb) {
            k.c = mdiv(x, f.mg_htb);
            tile = x - k.c * f.htb;
            k.n = f.hq + 1;
        } else {
            const int y = x - f.hrem * f.htb;
            const int cc = mdiv(y, f.mg_hts);
            k.c = f.hrem + cc;
            tile = y - cc * f.hts;
            k.n = f.hq;
        }
        k.m0 = tile * BM;
        k.r = f.r;
        k.ra = f.ra;
        int lo_k = k.m0 - k.r; if (lo_k < 0) lo_k = 0;
        int hi_k = k.m0 + BM - 1 + k.ra; if (hi_k > k.n - 1) hi_k = k.n - 1;
        k.kb_lo = lo_k / KBLK;
        k.nband = hi_k / KBLK - k.kb_lo + 1;
        k.key_end = k.n;
        k.split = 0;
    } else {
        const int g = t - f.n_band;
        k.kind = 1;
        k.r = 0;
        k.ra = 0;
        k.bh = mdiv(g, f.mg_per_bh);
        const int rem = g - k.bh * (f.n_split * f.n_ggroups);
        const int grp = mdiv(rem, f.mg_nsplit);
        k.split = rem - grp * f.n_split;
        k.b = mdiv(k.bh, f.mg_H);
        k.h = k.bh - k.b * f.H;
        k.delta = 1;
        k.c = 0;
        k.n = f.T;
        k.m0 = grp * BM;
        const int j0 = k.split * f.split_len;
        int j1 = j0 + f.split_len; if (j1 > f.T) j1 = f.T;
        k.kb_lo = j0 / KBLK;
        k.nband = cdiv(j1 - j0, KBLK);
        k.key_end = j1;
    }
    return k;
}

__device__ __forceinline__ Task decode_task(const Plan& P, int t) {
    Task k;
    if (t < P.n_band_tasks) {
        const BandTask bt = decode_band(P, t);
        k.kind = 0;
        k.b = bt.b;
        k.h = bt.h;
        k.bh = bt.b * P.H + bt.h;
        k.delta = P.dil[bt.h];
        k.c = bt.c;
        k.n = bt.n;
        k.m0 = bt.tile * BM;
        const int r = P.rad[bt.h];
        k.r = r;
        k.ra = P.one_sided ? 0 : r;
        int lo_k = k.m0 - r; if (lo_k < 0) lo_k = 0;
        int hi_k = k.m0 + BM - 1 + k.ra; if (hi_k > k.n - 1) hi_k = k.n - 1;
        k.kb_lo = lo_k / KBLK;
        k.nband = hi_k / KBLK - k.kb_lo + 1;
        k.key_end = k.n;
        k.split = 0;
    } else {
        const RowTask rt = decode_rows(P, t - P.n_band_tasks);
        k.kind = 1;
        k.r = 0;
        k.ra = 0;
        k.bh = rt.bh;
        k.split = rt.split;
        k.b = mdiv(k.bh, P.mg_H);
        k.h = k.bh - k.b * P.H;
        k.delta = 1;
        k.c = 0;
        k.n = P.T;
        k.m0 = rt.grp * BM;
        const int j0 = k.split * P.split_len;
        int j1 = j0 + P.split_len; if (j1 > P.T) j1 = P.T;
        k.kb_lo = j0 / KBLK;
        k.nband = cdiv(j1 - j0, KBLK);
        k.key_end = j1;
    }
    return k;
}

// ---------------------------------------------------------------------------
// Per-wave attention state and the work on one 32-key block.

template <int D, int NP>
struct WaveState {
    bf16x8 q[NP][D / 16];  // Q^T operands, one per bf16 part
    f32x16 o[D / 32];      // O^T: channels 32cb .. 32cb+31 of this lane's query
    float ms;              // running max in scaled base-2 units
    float nms;             // -ms, or 0 while ms is -inf (the exponent offset)
    float thr;             // raw score above which the max must move: (ms + 8) / scale
    float lp;              // this lane's part of the running sum
    int kbase;             // LDS offset of this lane's K operand bytes inside a stage
    int vbase;             // LDS offset of this lane's V^T operand bytes inside a stage
};

// K operands of one block for S^T = K Q^T (32 keys x this wave's 32
// queries): lane l supplies key row l%32, channels 16ks + 8(l/32) .. +7
template <int D, int NP>
struct KFrag { u32x4 k[D / 16][NP]; };

template <int D, int NP>
__device__ __forceinline__ KFrag<D, NP> load_k(const WaveState<D, NP>& W, const char* stage) {
    using G = Geo<D, NP>;
    KFrag<D, NP> f;
    const char* kb = stage + W.kbase;
#pragma unroll
    for (int ks = 0; ks < G::KS; ks++)
#pragma unroll
        for (int p = 0; p < NP; p++) f.k[ks][p] = *(const u32x4*)(kb + p * G::PLANE + 1024 * ks);
    return f;
}

template <int D, int NP>
__device__ __forceinline__ f32x16 block_scores(const WaveState<D, NP>& W, const KFrag<D, NP>& f) {
    using PR = Prods<NP>;
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < D / 16; ks++)
#pragma unroll
        for (int i = 0; i < PR::n; i++) s = mfma(as_bf16x8(f.k[ks][PR::a[i]]), W.q[PR::b[i]][ks], s);
    return s;
}

// Running max/sum update for one block's scores.  The raw-score max is taken
// to base 2 with the 1/sqrt(d) scale, and O is rescaled only when the max
// grows by more than 2^8.
template <int D, int NP>
__device__ __forceinline__ void update_max(WaveState<D, NP>& W, const f32x16& s) {
    constexpr float SC = ScaleLog2<D>::v;
    // maximum (not fmax): NaN-propagating, so no quieting of the MFMA results
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; i++) mx = __builtin_elementwise_maximum(mx, s[i]);
    // a row's maximum passes the threshold exactly when one of its halves
    // does, so the two halves meet only when some row moves
    if (__ballot(mx > W.thr)) {
        mx = halves_max(mx);
        const bool need = mx > W.thr;
        const float mxs = mx * SC;
        const float msn = need ? mxs : W.ms;
        const float alpha = need ? __builtin_amdgcn_exp2f(W.ms - msn) : 1.0f;
#pragma unroll
        for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
            for (int i = 0; i < 16; i++) W.o[cb][i] *= alpha;
        W.lp *= alpha;
        W.ms = msn;
        W.nms = msn == kNegInf ? 0.0f : -msn;
        W.thr = (msn + 8.0f) * (1.0f / SC);
    }
}

// V^T operands of one block, by transposing reads: lane (16G + L) supplies
// row 16st + 8hf + 4(G>>1) + (L>>2), channels 32cb + 16(G&1) + 4(L&3) .. +3
// (the lane-dependent part is W.vbase)
template <int D, int NP>
struct VFrag { bf16x8 v[2][D / 32][NP]; };   // [st][cb][plane]

template <int D, int NP>
__device__ __forceinline__ VFrag<D, NP> load_v(const WaveState<D, NP>& W, const char* stage) {
    using G = Geo<D, NP>;
    VFrag<D, NP> f;
    const char* vb = stage + G::HALF + W.vbase;
#pragma unroll
    for (int st = 0; st < 2; st++)
#pragma unroll
        for (int cb = 0; cb < G::CB; cb++)
#pragma unroll
            for (int p = 0; p < NP; p++) {
                const char* a = vb + p * G::PLANE + cb * 2048 + 16 * st * 64;
                f.v[st][cb][p] = cat_tr(ds_tr16(a), ds_tr16(a + 8 * 64));
            }
    return f;
}

// P^T operands of one block, one per bf16 part of the weights
template <int NP>
struct PFrag { bf16x8 p[NP][2]; };

// p = 2^(s*scale - m) for one block; returns this lane's part of the
// block's row sum (a tree of fp32 adds)
template <int D>
__device__ __forceinline__ float block_exp(float nms, const f32x16& s, float (&p)[16]) {
    constexpr float SC = ScaleLog2<D>::v;
#pragma unroll
    for (int i = 0; i < 16; i++) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], SC, nms));
    float t8[8];
#pragma unroll
    for (int i = 0; i < 8; i++) t8[i] = p[2 * i] + p[2 * i + 1];
#pragma unroll
    for (int i = 0; i < 4; i++) t8[i] += t8[i + 4];
    return (t8[0] + t8[2]) + (t8[1] + t8[3]);
}

// the weights as P^T operands (step st covers accumulator elements
// 8st .. 8st+7), one per bf16 part
template <int NP>
__device__ __forceinline__ void block_pack(const float (&p)[16], PFrag<NP>& pf) {
#pragma unroll
    for (int st = 0; st < 2; st++) {
        Raw32 x;
        x.a = __builtin_bit_cast(u32x4, (f32x4){p[8 * st], p[8 * st + 1], p[8 * st + 2], p[8 * st + 3]});
        x.b = __builtin_bit_cast(u32x4, (f32x4){p[8 * st + 4], p[8 * st + 5], p[8 * st + 6], p[8 * st + 7]});
        u32x4 parts[NP];
        split8<NP>(x, parts);
#pragma unroll
        for (int q = 0; q < NP; q++) pf.p[q][st] = as_bf16x8(parts[q]);
    }
}

// O^T += V^T P^T
template <int D, int NP>
__device__ __forceinline__ void block_product(WaveState<D, NP>& W, const PFrag<NP>& pf, const VFrag<D, NP>& f) {
    using PR = Prods<NP>;
#pragma unroll
    for (int st = 0; st < 2; st++)
#pragma unroll
        for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
            for (int i = 0; i < PR::n; i++) W.o[cb] = mfma(f.v[st][cb][PR::a[i]], pf.p[PR::b[i]][st], W.o[cb]);
}

// one block: the running maximum, the weights, their row sum and O^T += V^T P^T
template <int D, int NP>
__device__ __forceinline__ void block_pv(WaveState<D, NP>& W, const f32x16& s, const VFrag<D, NP>& f) {
    update_max<D, NP>(W, s);
    float p[16];
    W.lp += block_exp<D>(W.nms, s, p);
    PFrag<NP> pf;
    block_pack<NP>(p, pf);
    block_product<D, NP>(W, pf, f);
}

// A global key taken on the vector units: the K channels of this lane's half
// of the query (the Q operand layout, every bf16 part) and the V channels of
// its O^T rows (the input type).
template <int D, int NP>
struct GKey {
    u32x4 k[NP][D / 16];   // K parts: channels 16ks + 8lg .. +7
    u32x4 v[D / 8];        // V channels 32cb + 8j + 4lg .. +3 ([4cb + j]); bf16 inputs use .xy
};

// rk: K as bf16 rows of NP planes (NP * 2D bytes a row); rv: V rows in the
// input type.  pos past the end reads zeros.
template <int D, int NP>
__device__ __forceinline__ GKey<D, NP> load_gkey(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint32_t pos,
                                                  int lg) {
    GKey<D, NP> g;
    const uint32_t kro = pos * (uint32_t)(NP * 2 * D);
#pragma unroll
    for (int p = 0; p < NP; p++)
#pragma unroll
        for (int ks = 0; ks < D / 16; ks++) {
            const uint32_t o = kro + 2u * (p * D + 16 * ks + 8 * lg);
            g.k[p][ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
        }
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int ch = 32 * cb + 8 * j + 4 * lg;
            if constexpr (NP == 1) {
                const uint32_t vro = pos * (uint32_t)(2 * D);
                const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, vro + 2u * ch, 0, 0));
                g.v[4 * cb + j] = (u32x4){x[0], x[1], 0u, 0u};
            } else {
                const uint32_t vro = pos * (uint32_t)(4 * D);
                g.v[4 * cb + j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, vro + 4u * ch, 0, 0));
            }
        }
    return g;
}

// this lane's half of q . k over the split products.  Pairs are taken from
// whole bf16x8 vectors by shuffles: bit-casting single elements of an
// ext_vector miscompiles with this clang.
__device__ __forceinline__ bf16x2 pair(bf16x8 x, int e) {
    switch (e) {
        case 0: return __builtin_shufflevector(x, x, 0, 1);
        case 1: return __builtin_shufflevector(x, x, 2, 3);
        case 2: return __builtin_shufflevector(x, x, 4, 5);
        default: return __builtin_shufflevector(x, x, 6, 7);
    }
}

template <int D, int NP>
__device__ __forceinline__ float gkey_dot(const WaveState<D, NP>& W, const GKey<D, NP>& g) {
    using PR = Prods<NP>;
    float s = 0.f;
#pragma unroll
    for (int ks = 0; ks < D / 16; ks++)
#pragma unroll
        for (int i = 0; i < PR::n; i++) {
            const bf16x8 kk = as_bf16x8(g.k[PR::a[i]][ks]);
#pragma unroll
            for (int e = 0; e < 4; e++)
                s = __builtin_amdgcn_fdot2_f32_bf16(pair(W.q[PR::b[i]][ks], e), pair(kk, e), s, false);
        }
    return s;
}

// fold one key (scaled base-2 score sc, -inf when the key is not in the
// query's set) into the running (m, l, O): the running-max update of the
// blocks, for a single key.  lg == 0 lanes count its weight in l.
template <int D, int NP>
__device__ __forceinline__ void gkey_fold(WaveState<D, NP>& W, const GKey<D, NP>& g, float sc, int lg) {
    constexpr float SC = ScaleLog2<D>::v;
    const float mn = __builtin_fmaxf(W.ms, sc);
    const float alpha = W.ms == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(W.ms - mn);
    const float p = sc == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(sc - mn);
#pragma unroll
    for (int cb = 0; cb < D / 32; cb++) {
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const u32x4 x = g.v[4 * cb + j];
            f32x4 f;
            if constexpr (NP == 1) {
                // bf16 -> fp32 is the bf16 in the upper half: shift / mask whole vectors
                f = __builtin_bit_cast(f32x4, (u32x4){x[0] << 16, x[0] & 0xffff0000u, x[1] << 16, x[1] & 0xffff0000u});
            } else {
                f = __builtin_bit_cast(f32x4, x);
            }
#pragma unroll
            for (int e = 0; e < 4; e++) W.o[cb][4 * j + e] = __builtin_fmaf(W.o[cb][4 * j + e], alpha, p * f[e]);
        }
    }
    W.lp = __builtin_fmaf(W.lp, alpha, lg == 0 ? p : 0.0f);
    W.ms = mn;
    W.nms = mn == kNegInf ? 0.0f : -mn;
    W.thr = (mn + 8.0f) * (1.0f / SC);
}

// ---------------------------------------------------------------------------
// The tile kernel.

template <int D, typename ET, typename OT, bool PAD, bool RAND>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(Occupancy<D, Elem<ET>::NP, PAD, RAND>::v)))
void tile_kernel(const Args A) {
    constexpr int NP = Elem<ET>::NP;
    using G = Geo<D, NP>;
    constexpr int NT = 256;
    constexpr int ROWB = G::ROWB;
    constexpr int CB = G::CB;
    constexpr float SC = ScaleLog2<D>::v;
    __shared__ __attribute__((aligned(16))) char smem[G::bytes];
    const Plan& P = *A.plan;
    const int* gpos = (const int*)(smem + G::gposOff);
    const int* gcls = (const int*)(smem + G::gclsOff);
    const int* gld = (const int*)(smem + G::gldOff);
    const uint32_t* gbad = (const uint32_t*)(smem + G::gbadOff);

    // ---- which task.  Each of the 8 dies (blockIdx % 8) takes an eighth of
    // the global-row tasks first, then a contiguous eighth of the band tasks
    // (neighbouring tiles share keys in its L2), or the runs the plan cut by
    // cost when the heads' tiles differ in cost.
    const int xcd = blockIdx.x & 7, slot_in_xcd = blockIdx.x >> 3;
    const bool fast = A.fd.on != 0;
    int task_id;
    if (A.global_rows_only) {
        // an eighth of the global-row tasks per die, nothing else
        const int nb = fast ? A.fd.n_band : P.n_band_tasks, ng = (fast ? A.fd.n_tasks : P.n_tasks) - nb;
        const int ng_x = (ng >> 3) + (xcd < (ng & 7)), ng_o = xcd * (ng >> 3) + min(xcd, ng & 7);
        if (slot_in_xcd >= ng_x) return;
        task_id = nb + ng_o + slot_in_xcd;
    } else if (fast) {
        const int nb = A.fd.n_band, ng = A.fd.n_tasks - nb;
        const int nb_x = (nb >> 3) + (xcd < (nb & 7)), nb_o = xcd * (nb >> 3) + min(xcd, nb & 7);
        const int ng_x = (ng >> 3) + (xcd < (ng & 7)), ng_o = xcd * (ng >> 3) + min(xcd, ng & 7);
        if (slot_in_xcd < ng_x) task_id = nb + ng_o + slot_in_xcd;
        else if (slot_in_xcd - ng_x < nb_x) task_id = nb_o + (slot_in_xcd - ng_x);
        else return;
    } else {
        task_id = task_of_slot(P, xcd, slot_in_xcd, true);
        if (task_id < 0) return;
    }
    const Task tk = fast ? decode_task_fast(A.fd, task_id) : decode_task(P, task_id);
    const int T = fast ? A.fd.T : P.T;
    if constexpr (PAD) {
        // A band tile whose queries are all padded writes zero rows and ends
        // here: a padded query's output is zero whatever its keys.  Every
        // wave tests all of the tile's queries (lane l: query m0 + l), so the
        // decision is the same in each and no barrier is needed.
        if (tk.kind == 0) {
            const int l = threadIdx.x & 63;
            const int mq = tk.m0 + l;
            const int pos = tk.c + tk.delta * mq;
            const uint8_t* prow = A.pad + (size_t)tk.b * T;
            const bool live = mq < tk.n && prow[pos] == 0;
            if (__ballot(live) == 0) {
                constexpr int TPR = D * (int)sizeof(OT) / 16;   // threads per row, 16 bytes each
                for (int t = threadIdx.x; t < BM * TPR; t += NT) {
                    const int q = tk.m0 + t / TPR;
                    const int qp = tk.c + tk.delta * q;
                    bool global = false;
                    for (int g = 0; g < P.n_g; g++) global |= P.glob[g] == qp;
                    if (q < tk.n && !global) {
                        char* orow = (char*)A.out + ((size_t)tk.bh * T + qp) * D * sizeof(OT) + 16 * (t % TPR);
                        *(u32x4*)orow = (u32x4){0u, 0u, 0u, 0u};
                        if (A.lse && t % TPR == 0) A.lse[(size_t)tk.bh * T + qp] = kNegInf;
                    }
                }
                return;
            }
        }
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int qb = wave & 1;
    const int ph = wave >> 1;          // key phase of this wave: block ph of every stage
    const int lq = lane & 31;          // query column owned by this lane
    const int lg = lane >> 5;

    const size_t head_off = (size_t)tk.bh * T * D;
    const ET* __restrict__ Qg = (const ET*)A.q + head_off;
    const uint8_t* __restrict__ padrow = PAD ? A.pad + (size_t)tk.b * T : nullptr;
    // kernel-argument scalars used inside the loop live in registers (a value
    // select between an LDS table entry and a kernel argument would otherwise
    // become a flat load, which waits on every load in flight)
    const int n_g = fast ? A.fd.n_g : P.n_g, r = tk.r, ra = tk.ra;
    const uint32_t head_bytes = (uint32_t)T * ROWB;
    const void* kplanes = NP == 1 ? A.k : P.kp;   // bf16 input is its own plane
    const void* vplanes = NP == 1 ? A.v : P.vp;

    // ---- this wave's 32 queries
    const int mq0 = tk.m0 + 32 * qb;   // first query (class index, or global slot)
    bool wave_active;
    int my_pos = -1;                   // position of this lane's query
    if (tk.kind == 0) {
        wave_active = mq0 < tk.n;
        const int m = mq0 + lq;
        if (m < tk.n) my_pos = tk.c + tk.delta * m;
    } else {
        wave_active = mq0 < n_g;
        const int sl = mq0 + lq;
        if (sl < n_g) my_pos = P.glob[sl];
    }
    const int m_me = mq0 + lq;         // this lane's query (class index / global slot)

    // ---- block list: nb band (or dense) blocks, then the global-key blocks,
    // then the random blocks, in sequence positions q; stage s holds
    // positions 2s and 2s+1, and this wave works on position 2s + ph.
    const int nb = tk.nband;
    // A band task with a single global takes the key on the vector units
    // before the band (below): a global-key block would cost a whole step of
    // the loop for one key.  With more globals they follow the band blocks in
    // the ring: from two on, one step for up to 32 keys costs less than the
    // vector path run once per key (18.0 -> 17.2 us with globals {0, T-1} on
    // the headline shape).  Tiles with random blocks keep two globals on the
    // vector path: there a global-key step measured no faster and moved more
    // bytes (32.9 against 29.8 MB a launch).
    constexpr int kVecGlobals = RAND ? 2 : 1;
    const bool gvec = tk.kind == 0 && n_g > 0 && n_g <= kVecGlobals;
    const int ngb = (tk.kind == 0 && !gvec) ? cdiv(n_g, KBLK) : 0;
    // random key blocks of this query block (undilated heads): each block of
    // 64 keys is two 32-key blocks, after the band and the global-key blocks
    const int nrb = RAND && tk.kind == 0 ? 2 * P.n_rand : 0;   // RAND false: none, at compile time
    const int32_t* rrow = nrb > 0 ? P.rtab + ((size_t)tk.h * ((T + 63) >> 6) + (tk.m0 >> 6)) * P.n_rand : nullptr;
    // position of row 0 of random block position jr, or T for none (an empty
    // entry, or a position past this tile's list: a phase's last step can
    // fall past the end, and its entry must not be read)
    auto rand_p0 = [&](int jr) -> int {
        if (jr < 0 || jr >= nrb) return T;
        const int rho = rrow[jr >> 1];
        return rho >= 0 ? 64 * rho + 32 * (jr & 1) : T;
    };
    const int nblk = nb + nrb + ngb;
    // a global-row split whose keys are all padded contributes nothing: no
    // steps (its partial records get max -inf and sum 0)
    bool dead = false;
    if constexpr (PAD) {
        if (tk.kind == 1) {
            const uint8_t* prow = A.pad + (size_t)tk.b * T;
            bool any = false;
            for (int j = tk.kb_lo * KBLK + lane; j < tk.key_end; j += 64) any |= prow[j] == 0;
            dead = __ballot(any) == 0;
        }
    }
    const int NS = dead ? 0 : cdiv(nblk, 2);
    auto blk = [&](int s) -> int { return 2 * s + ph; };   // this phase's block of stage s
    // stages [0, s_fast) hold band blocks only and so does the stage after each
    const int s_fast = dead ? 0 : max((nb >> 1) - 1, 0);
    const int sb_end = (nb - ph + 1) >> 1;       // this wave's steps [0, sb_end) hold band (or dense) blocks
    int j_lo = 0, j_hi = -1;                     // band blocks with keys for this wave's queries
    int ji_lo = 0, ji_hi = -1;                   // band blocks that need no mask
    int sg_end = sb_end;                         // steps [sb_end, sg_end): global-key / random blocks
    if (wave_active) {
        j_hi = nb - 1;
        if (tk.kind == 0) {
            int a = mq0 - r; if (a < 0) a = 0;
            int z = mq0 + 31 + ra; if (z > tk.n - 1) z = tk.n - 1;
            j_lo = a / KBLK - tk.kb_lo;
            j_hi = z / KBLK - tk.kb_lo;
            // key0 = 32 (kb_lo + j) >= mq0 + 31 - r, key0 + 31 <= mq0 + ra, key0 + 32 <= key_end
            ji_lo = ((mq0 + 31 - r + 31) >> 5) - tk.kb_lo;
            ji_hi = min((mq0 + ra - 31) >> 5, (tk.key_end - 32) >> 5) - tk.kb_lo;
        } else {
            ji_hi = ((tk.key_end - 32) >> 5) - tk.kb_lo;
        }
        sg_end = (nblk - ph + 1) >> 1;
    }

    // ---- loads.  The two waves of a phase bring their own block of each
    // stage: query block 0 its K rows (lane p: row p/2), query block 1 its V
    // rows (lane p: rows p/4 and 16 + p/4).
    const int bw = ph;
    const bool kwave = qb == 0;
    const int rowA = kwave ? (lane >> 1) : (lane >> 2);
    const int rowB = kwave ? rowA : 16 + (lane >> 2);
    const uint32_t colA = kwave ? 16u * ((lane & 1) ^ ((rowA >> 3) & 1)) : 16u * (lane & 3);
    const uint32_t colB = kwave ? colA : 16u * (lane & 3);
    // piece i of this wave's load of a block: LDS offset and scalar byte
    // offset in the row; V pieces of odd index take the second row (voB)
    const char* kvhead = (const char*)(kwave ? kplanes : vplanes) + (size_t)tk.bh * head_bytes;
    auto pdst = [&](int i) -> int {
        if (kwave) return (i / G::KS) * G::PLANE + (i % G::KS) * 1024;
        const int p = i / G::KS, x = i % G::KS;    // V: x = 2 cb + half
        return p * G::PLANE + G::HALF + (x >> 1) * 2048 + (x & 1) * 1024;
    };
    auto psoff = [&](int i) -> uint32_t {
        const int p = i / G::KS, x = i % G::KS;
        return (uint32_t)(p * 2 * D + (kwave ? 32 * x : 64 * (x >> 1)));
    };
    // A band block is read through a window that starts at the block's row 0
    // and ends where the head ends, so that the lane offsets (rows delta
    // apart) stay fixed and rows past the end read zeros.
    auto row0_of = [&](int j) -> int { return tk.c + tk.delta * (tk.kb_lo + j) * KBLK; };   // position of row 0
    const uint32_t voA0 = (uint32_t)min((long long)tk.delta * rowA, (long long)T) * ROWB + colA;
    const uint32_t voB0 = (uint32_t)min((long long)tk.delta * rowB, (long long)T) * ROWB + colB;
    auto window_at = [&](int p0) -> __amdgpu_buffer_rsrc_t {
        return buffer_rsrc(kvhead + (uint64_t)p0 * ROWB, p0 < T ? (uint32_t)(T - p0) * ROWB : 0u);
    };
    auto global_pos = [&](int slot) -> uint32_t {   // position a loader lane reads for a global slot
        const int g = gld[min(slot, LF_MAX_GLOBALS - 1)];
        return (uint32_t)(slot < n_g ? g : T);
    };
    auto put = [&](__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t voA, uint32_t voB) {
#pragma unroll
        for (int i = 0; i < G::PPW; i++) {
            const bool second = !kwave && ((i % G::KS) & 1);
            load_lds16(rs, dst + pdst(i), second ? voB : voA, psoff(i));
        }
    };
    // band stage s into the ring slot at byte offset off (both blocks of the
    // stage are band blocks).  pm: padded rows of this wave's block, whose V
    // rows are loaded as zeros (so that NaN or Inf stored at padded positions
    // cannot reach the products).
    auto issue_band = [&](int s, int off, uint32_t pm) {
        const bool padA = PAD && !kwave && ((pm >> rowA) & 1u), padB = PAD && !kwave && ((pm >> rowB) & 1u);
        put(window_at(row0_of(blk(s))), smem + off + bw * G::BLK, padA ? kPastEnd : voA0, padB ? kPastEnd : voB0);
    };
    // any stage: band, global-key or random block, or nothing past the list;
    // padded global keys load as zeros through their table entry
    auto issue_stage = [&](int s, int off, uint32_t pm) {
        const bool padA = PAD && !kwave && ((pm >> rowA) & 1u), padB = PAD && !kwave && ((pm >> rowB) & 1u);
        const int jb = blk(s);
        if (jb >= nblk) return;
        char* dst = smem + off + bw * G::BLK;
        if (jb < nb) {
            put(window_at(row0_of(jb)), dst, padA ? kPastEnd : voA0, padB ? kPastEnd : voB0);
        } else if (jb >= nb + ngb) {
            put(window_at(rand_p0(jb - nb - ngb)), dst, padA ? kPastEnd : voA0, padB ? kPastEnd : voB0);
        } else {
            const int sl0 = (jb - nb) * KBLK;
            put(buffer_rsrc(kvhead, head_bytes), dst, global_pos(sl0 + rowA) * ROWB + colA,
                global_pos(sl0 + rowB) * ROWB + colB);
        }
    };

    // With padding, lane l < 32 reads the padding byte of row l of this
    // wave's block two stages ahead; one step ahead a ballot turns the bytes
    // into the block's padded-row word, which the step uses for the V rows it
    // loads and, one step later, for the scores.  Positions past the end read
    // zero (not padded; the range test covers them).
    const __amdgpu_buffer_rsrc_t rpad = buffer_rsrc(padrow, PAD ? (uint32_t)T : 0u);
    auto pad_at = [&](int s) -> uint32_t {
        const int q = blk(s);
        const int pos = q < nb ? row0_of(q) + tk.delta * lq
                               : (q >= nb + ngb && q < nblk ? rand_p0(q - nb - ngb) + lq : T);
        return __builtin_amdgcn_raw_buffer_load_b8(rpad, (uint32_t)min(pos, T), 0, 0);
    };
    auto pad_word = [&](uint32_t byte) -> uint32_t { return (uint32_t)__ballot(lane < 32 && byte != 0u); };

    WaveState<D, NP> W;
#pragma unroll
    for (int cb = 0; cb < CB; cb++) W.o[cb] = (f32x16){};
    W.ms = kNegInf;
    W.nms = 0.f;
    W.thr = kNegInf;
    W.lp = 0.f;
    W.kbase = ph * G::BLK + lq * 32 + ((lg ^ ((lq >> 3) & 1)) << 4);
    W.vbase = ph * G::BLK + (4 * (lane >> 5) + ((lane & 15) >> 2)) * 64 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

    // Q rows through a buffer resource: a lane with no query reads past its
    // end and gets zeros (a padded query keeps its row; the epilogues write
    // zeros for it)
    constexpr int QW = D / 16 * (NP == 1 ? 1 : 2);   // 16-byte loads per lane for its half of a Q row
    u32x4 qraw[QW];
    {
        constexpr uint32_t esz = sizeof(ET);
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(Qg, (uint32_t)T * D * esz);
        const uint32_t qoff = my_pos >= 0 ? (uint32_t)my_pos * D * esz : kPastEnd;
#pragma unroll
        for (int ks = 0; ks < D / 16; ks++)
#pragma unroll
            for (int h2 = 0; h2 < QW / (D / 16); h2++)
                qraw[(QW / (D / 16)) * ks + h2] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + (16 * ks + 8 * lg + 4 * h2) * esz, 0, 0));
    }
    // the first vector-path global key's K and V rows travel with Q
    const __amdgpu_buffer_rsrc_t rgk = buffer_rsrc((const char*)kplanes + (size_t)tk.bh * head_bytes, head_bytes);
    const __amdgpu_buffer_rsrc_t rgv = buffer_rsrc((const char*)A.v + tk.bh * (size_t)T * D * sizeof(ET),
                                                   (uint32_t)T * D * (uint32_t)sizeof(ET));
    GKey<D, NP> gk0;
    if (gvec && ph == 0) gk0 = load_gkey<D, NP>(rgk, rgv, (uint32_t)P.glob[0], lg);
    // ---- prologue: stage 0 and Q in flight, then the global-key tables (a
    // global-key block in stage 0, found only when the band has fewer than
    // two blocks, is loaded once its table is there).  Padded V rows of stage
    // 0 are cleared once it has landed.
    const bool early0 = blk(0) < nb;
    if (early0) issue_stage(0, 0, 0u);
    // padding: pm_cur = padded rows of this wave's block of stage s (in step
    // s), pbyte = the bytes of stage s+1 (in flight)
    uint32_t pm_cur = 0u, pbyte = 0u;
    if constexpr (PAD) {
        pm_cur = pad_at(0);
        pbyte = pad_at(1);
    }
    // global-key tables (band tasks): positions, load positions, class
    // indices, and per global block the slots that are no key (unused or
    // padded)
    if (ngb > 0) {
        for (int base = 64 * wave; base < ngb * KBLK; base += NT) {
            const int slot = base + lane;
            const bool inr = slot < n_g;
            const int pos = inr ? P.glob[slot] : T;
            const bool padded = PAD && inr && padrow[pos] != 0;
            int cls = kNotInClass;
            const int dpos = pos - tk.c;
            if (inr && dpos >= 0) {
                const int q = dpos / tk.delta;
                if (q * tk.delta == dpos) cls = q;
            }
            if (slot < LF_MAX_GLOBALS) {
                ((int*)gpos)[slot] = pos;
                ((int*)gld)[slot] = padded ? T : pos;
                ((int*)gcls)[slot] = cls;
            }
            const uint64_t badm = __ballot(!inr || padded);
            if (lane == 0 && base < LF_MAX_GLOBALS) {
                ((uint32_t*)gbad)[base >> 5] = (uint32_t)badm;
                if (base + 32 < LF_MAX_GLOBALS) ((uint32_t*)gbad)[(base >> 5) + 1] = (uint32_t)(badm >> 32);
            }
        }
        __syncthreads();
    }
    if (!early0) issue_stage(0, 0, 0u);
    // Without padding nothing reads stage 0 before the first step, whose own
    // barrier waits for it: the Q and global-key registers are waited for
    // where they are used, so the phase-0 waves fold the global key while
    // stage 0 is still landing.  (With no block at all nothing was issued.)
    // With padding, stage 0's padded V rows are cleared here first.
    if constexpr (PAD) {
        barrier_lds_loads();           // Q and stage 0 have landed
        pm_cur = pad_word(pm_cur);
        // the V loader clears the 16-byte pieces it brought for padded rows
        const bool padA = ((pm_cur >> rowA) & 1u) != 0u, padB = ((pm_cur >> rowB) & 1u) != 0u;
        if (!kwave && early0 && (padA || padB)) {
            char* dst = smem + bw * G::BLK + 16 * lane;
#pragma unroll
            for (int i = 0; i < G::PPW; i++) {
                const bool second = (i % G::KS) & 1;
                if (second ? padB : padA) *(u32x4*)(dst + pdst(i)) = (u32x4){0, 0, 0, 0};
            }
        }
        __syncthreads();
    }
#pragma unroll
    for (int ks = 0; ks < D / 16; ks++) {
        if constexpr (NP == 1) {
            W.q[0][ks] = as_bf16x8(qraw[ks]);
        } else {
            Raw32 x;
            x.a = qraw[2 * ks];
            x.b = qraw[2 * ks + 1];
            u32x4 parts[NP];
            split8<NP>(x, parts);
#pragma unroll
            for (int p = 0; p < NP; p++) W.q[p][ks] = as_bf16x8(parts[p]);
        }
    }
    // ---- vector-path global keys: the phase-0 waves (the phases are merged
    // at the end, so one of them takes the keys), every query, each key in
    // turn, unless the key is padded or already in the query's window (its
    // class, class distance in [-r, ra]: the band counts it)
    if (gvec && ph == 0) {
        const Magic md = P.mg_dil[tk.h];
        for (int g = 0; g < n_g; g++) {
            const int pos = P.glob[g];
            const GKey<D, NP> gk = g == 0 ? gk0 : load_gkey<D, NP>(rgk, rgv, (uint32_t)pos, lg);
            const float s = halves_sum(gkey_dot<D, NP>(W, gk));
            const int dpos = pos - tk.c;
            const int qd = dpos >= 0 ? mdiv(dpos, md) : -1;
            const bool in_class = dpos >= 0 && qd * tk.delta == dpos;
            const int dk = qd - m_me;
            const bool padded = PAD && padrow[pos] != 0;
            const bool ok = my_pos >= 0 && !padded && !(in_class && dk >= -r && dk <= ra);
            gkey_fold<D, NP>(W, gk, ok ? s * SC : kNegInf, lg);
        }
    }

    // ---- the lean band step: stage s holds two band blocks and stage s+1
    // does too.  Every LDS read of a step comes before that step's loads into
    // LDS are issued (the compiler makes any LDS read that follows such a
    // load wait for it); the score MFMAs wait for the K reads, the PV MFMAs
    // for the V reads, and the other waves of the SIMD run meanwhile.
    auto band_step = [&](int s, int oc, int on) {
        barrier_lds_loads();           // stage s landed; stage s-1 no longer read
        const int j = blk(s);
        const bool rel = j >= j_lo && j <= j_hi;
        KFrag<D, NP> kf;
        VFrag<D, NP> vf;
        if (rel) {
            kf = load_k<D, NP>(W, smem + oc);
            vf = load_v<D, NP>(W, smem + oc);
        }
        uint32_t pm_next = 0u;
        if constexpr (PAD) {
            pm_next = pad_word(pbyte);
            pbyte = pad_at(s + 2);
        }
        if constexpr (G::NBUF == 1) __syncthreads();   // every wave has its fragments: the slot is free
        issue_band(s + 1, on, pm_next);
        if (rel) {
            f32x16 sc = block_scores<D, NP>(W, kf);
            const bool clean = j >= ji_lo && j <= ji_hi && (!PAD || pm_cur == 0u);
            if (!clean) {
                if (tk.kind == 0) mask_window(sc, m_me - r - (tk.kb_lo + j) * KBLK - 4 * lg, r + ra);
                const int valid = tk.key_end - (tk.kb_lo + j) * KBLK;
                uint32_t bad = valid >= KBLK ? 0u : (0xffffffffu << valid);
                if constexpr (PAD) bad |= pm_cur;
                if (bad != 0u) mask_bits(sc, ~lane_bits(bad, lg));
            }
            block_pv<D, NP>(W, sc, vf);
        }
        pm_cur = pm_next;
    };

    // ---- the general step: band, global-key or random blocks, masks on
    // every block that needs one.  MODE 1: band or global-key blocks; MODE 2:
    // also random key blocks.
    auto step = [&](auto mode, int s, int oc, int on) {
        constexpr int MODE = decltype(mode)::value;
        barrier_lds_loads();           // stage s landed; stage s-1 no longer read
        const bool band = s < sb_end;
        const int jb = blk(s);         // sequence position
        const int j = min(jb, nb - 1); // its band block (band positions)
        const bool cur = band ? (j >= j_lo && j <= j_hi) : (s < sg_end);
        // The block's bad-row word, wave-uniform so that every test on it is
        // scalar: a global-key block's comes from LDS (read ahead of the
        // fragments), a band block's from its range and the padding ballot.
        uint32_t gword = 0u;
        const bool rnd = MODE == 2 && !band && jb >= nb + ngb;   // a random key block
        if (!band && !rnd) gword = gbad[min(max(jb - nb, 0), LF_MAX_GLOBALS / KBLK - 1)];
        KFrag<D, NP> kf;
        VFrag<D, NP> vf;
        if (cur) {
            kf = load_k<D, NP>(W, smem + oc);
            vf = load_v<D, NP>(W, smem + oc);
        }
        uint32_t bad;
        int p0r = T;
        if (band) {
            const int valid = tk.key_end - (tk.kb_lo + j) * KBLK;
            bad = valid <= 0 ? 0xffffffffu : (valid >= KBLK ? 0u : (0xffffffffu << valid));
            if constexpr (PAD) bad |= pm_cur;
        } else if (MODE == 2 && rnd) {
            // rows past the end, padded rows and global keys (the globals are
            // counted by their own path) are not keys of a random block
            p0r = rand_p0(jb - nb - ngb);
            const int valid = T - p0r;
            bad = valid <= 0 ? 0xffffffffu : (valid >= KBLK ? 0u : (0xffffffffu << valid));
            if constexpr (PAD) bad |= pm_cur;
            if (n_g > 0 && p0r < T) bad |= P.gmap[p0r >> 5];
        } else {
            bad = (uint32_t)uniform((int)gword);
        }
        if (!cur) bad = 0xffffffffu;
        uint32_t pm_next = 0u;
        if constexpr (PAD) {
            pm_next = pad_word(pbyte);
            pbyte = pad_at(s + 2);
        }
        if constexpr (G::NBUF == 1) __syncthreads();
        if (s + 1 < NS) issue_stage(s + 1, on, pm_next);
        // A block with no key for this wave's queries is skipped: its LDS may
        // hold anything (zero weights times NaN would still be NaN).
        if (bad != 0xffffffffu) {
            f32x16 sc = block_scores<D, NP>(W, kf);
            if (MODE == 2 && rnd) {
                if (p0r + 31 >= mq0 - r && p0r <= mq0 + 31 + ra)   // may meet this wave's windows
                    mask_window_out(sc, m_me - r - p0r - 4 * lg, r + ra);
                if (bad != 0u) mask_bits(sc, ~lane_bits(bad, lg));
            } else if (!band) {
                mask_global(sc, bad, gcls + (jb - nb) * KBLK, m_me, r, r + ra, lg);
            } else if (!(j >= ji_lo && j <= ji_hi && bad == 0u)) {
                if (tk.kind == 0) mask_window(sc, m_me - r - (tk.kb_lo + j) * KBLK - 4 * lg, r + ra);
                if (bad != 0u) mask_bits(sc, ~lane_bits(bad, lg));
            }
            block_pv<D, NP>(W, sc, vf);
        }
        pm_cur = pm_next;
    };

    // ---- main loop: stages [0, s_fast) hold band blocks only and so does the
    // stage each loads next; the rest (the last band stage, at most one mixed
    // stage, then global-key and random blocks) take the general step.
    using General = std::integral_constant<int, 1>;
    using WithRandom = std::integral_constant<int, 2>;
    constexpr int S1 = G::NBUF == 2 ? G::STAGE : 0;
    int s = 0;
    for (; s + 1 < s_fast; s += 2) {
        band_step(s, 0, S1);
        band_step(s + 1, S1, 0);
    }
    if (s < s_fast) {
        band_step(s, 0, S1);
        s++;
    }
    // stages from the first random block on take the step with random blocks
    const int s_rand = nrb > 0 ? (nb + ngb) >> 1 : NS;
    for (; s < min(NS, s_rand); s++) step(General{}, s, (s & 1) * S1, ((s + 1) & 1) * S1);
    if constexpr (RAND)
        for (; s < NS; s++) step(WithRandom{}, s, (s & 1) * S1, ((s + 1) & 1) * S1);
    __syncthreads();

    // ---- merge the two phases of each query block (LDS); phase 0 keeps the result
    {
        constexpr int RECF = 16 * CB + 4;   // floats per lane: O^T, then m, l
        float* mbuf = (float*)smem;
        if (ph > 0) {
            f32x4* dst = (f32x4*)(mbuf + (qb * 64 + lane) * RECF);
#pragma unroll
            for (int cb = 0; cb < CB; cb++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    dst[4 * cb + i] = (f32x4){W.o[cb][4 * i], W.o[cb][4 * i + 1], W.o[cb][4 * i + 2], W.o[cb][4 * i + 3]};
            dst[4 * CB] = (f32x4){W.ms, W.lp, 0.f, 0.f};
        }
        __syncthreads();
        if (ph == 0) {
            const f32x4* src = (const f32x4*)(mbuf + (qb * 64 + lane) * RECF);
            const f32x4 tail = src[4 * CB];
            const float ms2 = tail[0], lp2 = tail[1];
            const float mn = __builtin_fmaxf(W.ms, ms2);
            const float a1 = (W.ms == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(W.ms - mn);
            const float a2 = (ms2 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ms2 - mn);
#pragma unroll
            for (int cb = 0; cb < CB; cb++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const f32x4 x = src[4 * cb + i];
#pragma unroll
                    for (int e = 0; e < 4; e++) W.o[cb][4 * i + e] = W.o[cb][4 * i + e] * a1 + x[e] * a2;
                }
            W.lp = W.lp * a1 + lp2 * a2;
            W.ms = mn;
        }
    }

    const bool writer = ph == 0 && wave_active;
    const float l = halves_sum(W.lp);

    if (tk.kind == 0) {
        // ---- epilogue: y = O / l for the tile's valid queries; padded rows -> 0.
        // Rows of global queries are left to the global-row combine.
        if (!writer || my_pos < 0) return;
        if (gvec) {
            for (int g = 0; g < n_g; g++)
                if (P.glob[g] == my_pos) return;
        } else if (n_g > 0) {
            int lo = 0, hi = n_g - 1;
            while (lo < hi) {
                const int mid = (lo + hi) >> 1;
                if (gpos[mid] < my_pos) lo = mid + 1; else hi = mid;
            }
            if (gpos[lo] == my_pos) return;
        }
        const bool my_pad = padrow ? padrow[my_pos] != 0 : false;
        OT* orow = (OT*)A.out + head_off + (size_t)my_pos * D;
        // a padded query's row is written as zeros, whatever its Q held
        const bool zero = my_pad || l == 0.f;
        const float inv = zero ? 0.f : 1.0f / l;
        if (A.lse && lg == 0)
            A.lse[(size_t)tk.bh * T + my_pos] = zero ? kNegInf : (W.ms + __builtin_amdgcn_logf(l)) * kLn2;
#pragma unroll
        for (int cb = 0; cb < CB; cb++) {
            const f32x16& oc = W.o[cb];
            if constexpr (sizeof(OT) == 2) {
                // Channel groups 8j+4lg..+3 packed to bf16 (two dwords each). Lanes l
                // and l+32 trade groups with one v_permlane32_swap per dword so that
                // each ends up with 8 consecutive channels: the lower lane keeps group
                // 2m and takes its partner's, the upper lane keeps 2m+1 likewise.
                uint32_t g[4][2];
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const float y0 = zero ? 0.f : oc[4 * j + 0] * inv, y1 = zero ? 0.f : oc[4 * j + 1] * inv;
                    const float y2 = zero ? 0.f : oc[4 * j + 2] * inv, y3 = zero ? 0.f : oc[4 * j + 3] * inv;
                    g[j][0] = pack_bf16(y0, y1);
                    g[j][1] = pack_bf16(y2, y3);
                }
#pragma unroll
                for (int m = 0; m < 2; m++) {
                    const auto r0 = __builtin_amdgcn_permlane32_swap(g[2 * m][0], g[2 * m + 1][0], false, false);
                    const auto r1 = __builtin_amdgcn_permlane32_swap(g[2 * m][1], g[2 * m + 1][1], false, false);
                    const u32x4 w = {r0[0], r1[0], r0[1], r1[1]};
                    *(u32x4*)(orow + 32 * cb + 16 * m + 8 * lg) = w;
                }
            } else {
#pragma unroll
                for (int j = 0; j < 4; j++) {
                    const int c0 = 32 * cb + 8 * j + 4 * lg;
                    const f32x4 w = {zero ? 0.f : oc[4 * j + 0] * inv, zero ? 0.f : oc[4 * j + 1] * inv,
                                     zero ? 0.f : oc[4 * j + 2] * inv, zero ? 0.f : oc[4 * j + 3] * inv};
                    *(f32x4*)(orow + c0) = w;
                }
            }
        }
        return;
    }

    // ---- global rows: write this split's partial for each global slot, a
    // record [O[0..D-1], m, l, 0, 0].  Partials cross dies (each XCD has its
    // own L2), so they are written and read with the agent-coherent cache
    // policy (sc1) instead of fences, which would write back and invalidate
    // whole L2s.
    constexpr int REC = G::REC;
    const uint32_t stride = (uint32_t)P.g_pad * REC;          // bytes between splits of a slot
    const __amdgpu_buffer_rsrc_t rpart =
        buffer_rsrc((const char*)P.part + (size_t)tk.bh * P.n_split * stride, (uint32_t)P.n_split * stride);
    const int slot = mq0 + lq;
    if (writer && slot < n_g) {
        const uint32_t rec = (uint32_t)tk.split * stride + (uint32_t)slot * REC;
#pragma unroll
        for (int cb = 0; cb < CB; cb++) {
            const f32x16& oc = W.o[cb];
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const f32x4 o4 = {oc[4 * j], oc[4 * j + 1], oc[4 * j + 2], oc[4 * j + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o4), rpart,
                                                       rec + 4 * (32 * cb + 8 * j + 4 * lg), 0, kCoherent);
            }
        }
        if (lg == 0)
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, (f32x2){W.ms, l}), rpart, rec + 4 * D, 0,
                                                  kCoherent);
    }
    // The last of the n_split * n_ggroups workgroups of head (b, h) to finish
    // rescales and adds the partials of every global row of that head.  The
    // counter is returned to zero by that workgroup, ready for the next call.
    __builtin_amdgcn_s_waitcnt(0);   // this wave's partial stores have completed
    __syncthreads();
    int* flag = (int*)smem;
    if (tid == 0) {
        const int done = __hip_atomic_fetch_add(P.counter + tk.bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = done == P.n_split * P.n_ggroups - 1;
    }
    __syncthreads();
    if (*flag == 0) return;
    // Each thread combines 4 channels of one global row over all splits,
    // eight splits at a time with all of their loads in flight (splits past
    // n_split repeat the last one and get weight 0), folding each group into
    // a running (max, sum, weighted sum).
    constexpr int C4 = D / 4;
    for (int task = tid; task < n_g * C4; task += NT) {
        const int gi = task / C4, c4 = task % C4;
        float M = kNegInf, L = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int sp0 = 0; sp0 < P.n_split; sp0 += 8) {
            f32x2 ml[8];
            f32x4 o[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t rec = (uint32_t)min(sp0 + i, P.n_split - 1) * stride + (uint32_t)gi * REC;
                ml[i] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rpart, rec + 4 * D, 0, kCoherent));
                o[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rpart, rec + 16 * c4, 0, kCoherent));
            }
            float Mn = M;
#pragma unroll
            for (int i = 0; i < 8; i++) Mn = __builtin_fmaxf(Mn, ml[i][0]);
            const float a = (M == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(M - Mn);
            L *= a;
#pragma unroll
            for (int e = 0; e < 4; e++) acc[e] *= a;
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const float w = (sp0 + i < P.n_split && ml[i][0] != kNegInf) ? __builtin_amdgcn_exp2f(ml[i][0] - Mn) : 0.f;
                L += ml[i][1] * w;
#pragma unroll
                for (int e = 0; e < 4; e++) acc[e] += o[i][e] * w;
            }
            M = Mn;
        }
        const int pos = P.glob[gi];
        const bool padded = padrow && padrow[pos] != 0;
        const bool zero = padded || !(L > 0.f);
        if (zero) acc = (f32x4){0.f, 0.f, 0.f, 0.f};   // zeros even if the partials hold NaN
        const float inv = zero ? 0.f : 1.0f / L;
        OT* orow = (OT*)A.out + head_off + (size_t)pos * D + 4 * c4;
        if constexpr (sizeof(OT) == 2) {
            *(u32x2*)orow = (u32x2){pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
        } else {
            *(f32x4*)orow = (f32x4){acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
        }
        if (A.lse && c4 == 0) A.lse[(size_t)tk.bh * T + pos] = zero ? kNegInf : (M + __builtin_amdgcn_logf(L)) * kLn2;
    }
    if (tid == 0) __hip_atomic_store(P.counter + tk.bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fp32 K and V -> three bf16 planes per row [rows][3][D] (part 0 = RNE(x),
// each next part RNE of the remainder), one thread per 8 channels of a row;
// blockIdx.y picks K or V
template <int D>
__global__ __launch_bounds__(256) void split_planes_kernel(const float* __restrict__ k, const float* __restrict__ v,
                                                           uint16_t* __restrict__ kp, uint16_t* __restrict__ vp,
                                                           long long chunks) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= chunks) return;
    const float* src = blockIdx.y ? v : k;
    uint16_t* dst = blockIdx.y ? vp : kp;
    constexpr int CPR = D / 8;   // chunks per row
    const long long row = i / CPR;
    const int ch = (int)(i % CPR);
    Raw32 x;
    x.a = *(const u32x4*)(src + row * D + ch * 8);
    x.b = *(const u32x4*)(src + row * D + ch * 8 + 4);
    u32x4 parts[3];
    split8<3>(x, parts);
#pragma unroll
    for (int p = 0; p < 3; p++) *(u32x4*)(dst + row * 3 * D + p * D + ch * 8) = parts[p];
}

// ---------------------------------------------------------------------------
// The allocation-free entry point's workspace: one array per GPU, held until
// the process ends.  Host code never passes `scratch` itself to a kernel (on
// the host that name is a stand-in, not the device address): it passes the
// address hipGetSymbolAddress returns for the current device.

static __device__ __align__(256) char scratch[LF_NOALLOC_SCRATCH_BYTES];

// A piece of the plan passed by value (a kernel argument is captured with
// the launch, so the copy works inside graph capture): words [0, n) go to
// dst; the first piece also clears n_zero ints at zero (the global-row
// completion counters).  One workgroup of 256 threads.
struct PlanPiece {
    uint32_t* dst;
    int* zero;
    int n, n_zero;
    uint32_t w[880];
};
static_assert(sizeof(PlanPiece) <= 3584, "plan piece fits a kernel argument");

__global__ __launch_bounds__(256) void plan_piece_kernel(const PlanPiece c) {
    for (int i = threadIdx.x; i < c.n; i += 256) c.dst[i] = c.w[i];
    for (int i = threadIdx.x; i < c.n_zero; i += 256) c.zero[i] = 0;
}

}  // namespace lfk

// address of this device's scratch array, looked up once per device with
// that device current
extern "C" hipError_t lfk_noalloc_scratch(void** ptr) {
    static std::mutex mu;
    static void* addr[256] = {};
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= 256) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(lfk::scratch));
        if (e != hipSuccess) return e;
        addr[dev] = p;
    }
    *ptr = addr[dev];
    return hipSuccess;
}

// copy `bytes` of a plan (a multiple of 4) to dst in pieces passed by value,
// the first one also clearing n_zero ints at zero; all on `stream`
extern "C" hipError_t lfk_write_plan(const void* plan, size_t bytes, void* dst, int* zero, int n_zero, void* stream) {
    const uint32_t* src = (const uint32_t*)plan;
    const size_t words = bytes / 4;
    lfk::PlanPiece c;
    for (size_t w0 = 0; w0 < words || (w0 == 0 && n_zero > 0); w0 += 880) {
        const size_t n = words - w0 < 880 ? words - w0 : 880;
        c.dst = (uint32_t*)dst + w0;
        c.n = (int)n;
        for (size_t i = 0; i < n; i++) c.w[i] = src[w0 + i];
        c.zero = zero;
        c.n_zero = w0 == 0 ? n_zero : 0;
        hipLaunchKernelGGL(lfk::plan_piece_kernel, dim3(1), dim3(256), 0, (hipStream_t)stream, c);
        if (n == 0) break;
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// launchers (called from the host library)

// grid: the task slots of the 8 dies, each die holding ceil(n/8) band and
// ceil(n/8) global-row slots
extern "C" int lfk_grid(const lfk::Plan* P) {
    return 8 * lfk::slots_per_die(*P);
}

// A: kernel argument (A->plan is the device copy of *P); P: host copy of the plan.
// One instantiation per head dimension, input type, padding and random
// blocks (each present or not at compile time).
template <int D, typename ET, typename OT>
static void launch_tiles(const lfk::Args* A, const lfk::Plan* P, hipStream_t s) {
    const int grid = A->global_rows_only ? 8 * ((P->n_tasks - P->n_band_tasks + 7) / 8) : lfk_grid(P);
    const bool pad = A->pad != nullptr, rnd = P->n_rand > 0;
    const dim3 g(grid), b(256);
    if (pad && rnd) hipLaunchKernelGGL((lfk::tile_kernel<D, ET, OT, true, true>), g, b, 0, s, *A);
    else if (pad) hipLaunchKernelGGL((lfk::tile_kernel<D, ET, OT, true, false>), g, b, 0, s, *A);
    else if (rnd) hipLaunchKernelGGL((lfk::tile_kernel<D, ET, OT, false, true>), g, b, 0, s, *A);
    else hipLaunchKernelGGL((lfk::tile_kernel<D, ET, OT, false, false>), g, b, 0, s, *A);
}

template <int D>
static void launch_d(const lfk::Args* A, const lfk::Plan* P, int dtype_bf16, hipStream_t s) {
    if (dtype_bf16) {
        launch_tiles<D, __bf16, uint16_t>(A, P, s);
    } else {
        const long long chunks = (long long)P->B * P->H * P->T * (D / 8);
        hipLaunchKernelGGL(lfk::split_planes_kernel<D>, dim3((unsigned)((chunks + 255) / 256), 2), dim3(256), 0, s,
                           (const float*)A->k, (const float*)A->v, (uint16_t*)P->kp, (uint16_t*)P->vp, chunks);
        launch_tiles<D, float, float>(A, P, s);
    }
}

extern "C" hipError_t lfk_launch(const lfk::Args* A, const lfk::Plan* P, int dtype_bf16, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    switch (P->d) {
        case 32: launch_d<32>(A, P, dtype_bf16, s); break;
        case 64: launch_d<64>(A, P, dtype_bf16, s); break;
        case 128: launch_d<128>(A, P, dtype_bf16, s); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

// whether the library was built with head dimension d (the host checks this
// before any HIP call)
extern "C" int lfk_supports_d(int d) { return d == 32 || d == 64 || d == 128; }
