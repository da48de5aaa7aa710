// lf_attn_kernels.hip -- gfx950 (CDNA4) kernels of the Longformer sparse
// self-attention forward pass.
//
// One tile kernel serves two task kinds that share a grid:
//
//  * band tasks: one tile of BM = 32*QB consecutive queries of one dilation
//    residue class c of head (b, h), against the keys of that class inside
//    the window (Longformer, eightmm.github.io, "Sliding-Window
//    Attention"), followed by the global keys G (same page, "Global
//    Attention": every ordinary token also reads G; a global key already
//    inside the window is counted once);
//  * global-row tasks: up to 32*QB global queries of head (b, h) against
//    one contiguous split of all T keys ("Global Attention": a global token
//    reads every position), written as partial (max, sum, weighted-sum)
//    triples that the combine kernel rescales and adds.
//
// Residue classes: with stride delta the positions c, c+delta, c+2*delta,
// ... form an undilated sequence of length n_c = ceil((T-c)/delta) on which
// the dilated window is an ordinary window of radius r (Longformer,
// ciallo.wiki §2.2.3; "Longformer长序列处理", 膨胀窗口设计).  Tiles are cut in
// class coordinates, so no MFMA work is spent on keys of other classes.
//
// Per wave: 32 queries.  S^T = K Q^T and O^T = V^T P^T are computed with
// v_mfma_f32_32x32x16_bf16, so every lane owns one query (column) in both
// accumulators and the softmax needs only one cross-lane exchange (lanes l
// and l^32 hold the two halves of a query's keys).  K reaches the MFMA A
// operand by ds_read_b128 from a swizzled LDS tile; V reaches it through
// ds_read_b64_tr_b16 (transposing LDS read).  The softmax is the running
// max/sum form (blockwise accumulation, "Longformer长序列处理", 显存优化技巧)
// kept in base 2 with the 1/sqrt(d) scale folded into one FMA; the running
// max is only moved (and O rescaled) when a block raises it by more than
// 2^8, which keeps every exponent <= 8 and leaves the final O/l exact.
//
// KS waves share each query block: the key blocks of a tile are dealt out
// round-robin to KS "phases", and the KS partial states are merged in LDS
// at the end.  This gives the chip 4 waves per 64 queries instead of 2.
//
// fp32 inputs are split into bf16 hi + lo parts when staged; each product
// uses hi*hi + hi*lo + lo*hi (three MFMAs), which keeps the score and output
// error near 2^-16 relative while the tiling, masking and softmax code is
// the very code the bf16 path runs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lf_kernels.h"

namespace lfk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int D = 64;
constexpr int KBLK = 32;                  // keys per block (one S^T tile)
constexpr int BLK_BYTES = KBLK * D * 2;   // one bf16 plane of a block: 4 KiB
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kNotInClass = -(1 << 30);

// log2(e) / sqrt(64): scores are taken to base 2 with the 1/sqrt(d) scale.
constexpr float kScaleLog2 = 0.18033688011112042f;

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32); }

// ---------------------------------------------------------------------------
// LDS tile geometry.  A stage holds KS blocks of 32 keys; per block and
// plane, K and V are 32 rows x 128 B.  NP = 1 (bf16) or 2 (fp32: hi, lo).
template <int KS, int NP>
struct Stage {
    static constexpr int kOff(int p, int blk) { return (p * KS + blk) * BLK_BYTES; }
    static constexpr int vOff(int p, int blk) { return (NP * KS + p * KS + blk) * BLK_BYTES; }
    static constexpr int maskOff = 2 * NP * KS * BLK_BYTES;            // KS x 4 bytes
    static constexpr int gclsOff = maskOff + ((KS * 4 + 15) / 16) * 16;  // KS x 32 int32
    static constexpr int bytes = gclsOff + KS * KBLK * 4;
};

// K rows: 16-byte chunk ch of row t lives at chunk ch ^ ((t >> 1) & 7), so
// the 16 lanes that read one chunk column of 16 consecutive rows hit 16
// different bank groups.
__device__ __forceinline__ int swzK(int t, int ch) { return t * 128 + ((ch ^ ((t >> 1) & 7)) << 4); }
// V rows: chunk ch of row t lives at ch ^ (4 * ((t >> 1) & 1)); a transposing
// read touches 8 rows x 64 B and this spreads them over all 64 banks.
__device__ __forceinline__ int swzV(int t, int ch) { return t * 128 + ((ch ^ (((t >> 1) & 1) << 2)) << 4); }

// ---------------------------------------------------------------------------
// element-type traits

template <typename T> struct Elem;
template <> struct Elem<__bf16> {
    static constexpr int NP = 1;
    static constexpr int CHUNK_BYTES = 16;  // 8 channels
};
template <> struct Elem<float> {
    static constexpr int NP = 2;
    static constexpr int CHUNK_BYTES = 32;
};

struct Raw16 { u32x4 a; };
struct Raw32 { u32x4 a, b; };

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// two floats -> two bf16 (round to nearest even) in one dword; one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){lo, hi}, bf16x2));
}

// split 8 floats into hi/lo bf16 parts (hi = RNE(x), lo = RNE(x - hi)).
// Whole vectors are bit-cast: bit-casting single elements of an ext_vector
// miscompiles with this clang (every element reads as element 0).
__device__ __forceinline__ void split8(const Raw32& r, u32x4& hi, u32x4& lo) {
    const f32x4 fa = __builtin_bit_cast(f32x4, r.a);
    const f32x4 fb = __builtin_bit_cast(f32x4, r.b);
    const float f[8] = {fa[0], fa[1], fa[2], fa[3], fb[0], fb[1], fb[2], fb[3]};
#pragma unroll
    for (int i = 0; i < 4; i++) {
        const uint32_t hw = pack_bf16(f[2 * i], f[2 * i + 1]);
        const float h0 = __builtin_bit_cast(float, hw << 16);
        const float h1 = __builtin_bit_cast(float, hw & 0xffff0000u);
        hi[i] = hw;
        lo[i] = pack_bf16(f[2 * i] - h0, f[2 * i + 1] - h1);
    }
}

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 x) { return __builtin_bit_cast(bf16x8, x); }

__device__ __forceinline__ f32x16 mfma(bf16x8 a, bf16x8 b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ i16x4 ds_tr16(const char* lds_ptr) {
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4*)(lds_ptr));
}

__device__ __forceinline__ bf16x8 cat_tr(i16x4 a, i16x4 b) {
    typedef short i16x8 __attribute__((ext_vector_type(8)));
    i16x8 r;
    r[0] = a[0]; r[1] = a[1]; r[2] = a[2]; r[3] = a[3];
    r[4] = b[0]; r[5] = b[1]; r[6] = b[2]; r[7] = b[3];
    return __builtin_bit_cast(bf16x8, r);
}

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
};

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

template <int QB>
__device__ __forceinline__ Task decode_task(const Params& P, int t) {
    constexpr int BM = 32 * QB;
    Task k;
    if (t < P.n_band_tasks) {
        k.kind = 0;
        k.b = t / P.band_tasks_per_batch;
        int x = t - k.b * P.band_tasks_per_batch;
        // heads are few (<= LF_MAX_HEADS): binary search on the band-task prefix
        int lo = 0, hi = P.H - 1;
        while (lo < hi) {
            const int mid = (lo + hi + 1) >> 1;
            if (P.head_start[mid] <= x) lo = mid; else hi = mid - 1;
        }
        const int h = lo;
        x -= P.head_start[h];
        k.h = h;
        k.bh = k.b * P.H + h;
        const int delta = P.dil[h];
        int c, tile;
        if (delta == 1) {
            c = 0;
            tile = x;
            k.n = P.T;
        } else {
            const int q = P.T / delta, rem = P.T - q * delta;
            const int tb = cdiv(q + 1, BM), ts = cdiv(q, BM);
            if (x < rem * tb) { c = x / tb; tile = x - c * tb; }
            else { const int y = x - rem * tb; c = rem + y / ts; tile = y - (c - rem) * ts; }
            k.n = (P.T - c + delta - 1) / delta;
        }
        k.delta = delta;
        k.c = c;
        k.m0 = tile * BM;
        const int r = P.r;
        int lo_k = k.m0 - r; if (lo_k < 0) lo_k = 0;
        int hi_k = k.m0 + BM - 1 + r; if (hi_k > k.n - 1) hi_k = k.n - 1;
        k.kb_lo = lo_k / KBLK;
        k.nband = hi_k / KBLK - k.kb_lo + 1;
        k.key_end = k.n;
        k.split = 0;
    } else {
        k.kind = 1;
        const int g = t - P.n_band_tasks;
        const int per_bh = P.n_split * P.n_ggroups;
        k.bh = g / per_bh;
        const int rem = g - k.bh * per_bh;
        const int grp = rem / P.n_split;
        k.split = rem - grp * P.n_split;
        k.b = k.bh / P.H;
        k.h = k.bh - k.b * P.H;
        k.delta = 1;
        k.c = 0;
        k.n = P.T;
        k.m0 = grp * BM;
        const int j0 = k.split * P.split_len;
        int j1 = j0 + P.split_len; if (j1 > P.T) j1 = P.T;
        k.kb_lo = j0 / KBLK;
        k.nband = cdiv(j1 - j0, KBLK);
        k.key_end = j1;
    }
    return k;
}

// is position pos one of the (sorted) global positions?
__device__ __forceinline__ bool is_global(const Params& P, int pos) {
    int lo = 0, hi = P.n_g - 1;
    while (lo <= hi) {
        const int mid = (lo + hi) >> 1;
        const int g = P.glob[mid];
        if (g == pos) return true;
        if (g < pos) lo = mid + 1; else hi = mid - 1;
    }
    return false;
}

// max over the two 32-lane halves (lanes l and l^32 hold the two key halves of
// a query): one v_permlane32_swap, no LDS round trip
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const f32x2 f = __builtin_bit_cast(f32x2, r);
    return __builtin_fmaxf(f[0], f[1]);
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const f32x2 f = __builtin_bit_cast(f32x2, r);
    return f[0] + f[1];
}

// agent-scope relaxed atomic accesses (coherent across the XCDs' L2s)
__device__ __forceinline__ void store_coherent(uint32_t* p, float x) {
    __hip_atomic_store(p, __builtin_bit_cast(uint32_t, x), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_coherent(const uint32_t* p) {
    return __builtin_bit_cast(float, __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

// Block masks.  Bit t of a block's mask word is set when key row t of the
// block is not a real key (beyond the sequence/class/split, or padded).
enum BlockMode { kInterior = 0, kBandEdge = 1, kGlobalKeys = 2, kDense = 3 };

// ---------------------------------------------------------------------------
// Per-wave attention state and the work on one 32-key block.

template <int NP>
struct WaveState {
    bf16x8 qh[4], ql[4];  // Q^T operands (lo part only for fp32 inputs)
    f32x16 o0, o1;        // O^T: channels 0..31 and 32..63 of this lane's query
    float ms;             // running max in scaled base-2 units
    float lp;             // this lane's part of the running sum
};

// S^T = K Q^T for one block (32 keys x this wave's 32 queries), masked per MODE.
template <int MODE, int KS, int NP>
__device__ __forceinline__ f32x16 block_scores(const WaveState<NP>& W, const char* buf, int blk, int key0,
                                               uint32_t bad, int m, int r, int lane) {
    using SG = Stage<KS, NP>;
    const int lq = lane & 31, lg = lane >> 5;
    f32x16 s = {};
    const char* kb = buf + SG::kOff(0, blk);
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const bf16x8 kf = as_bf16x8(*(const u32x4*)(kb + swzK(lq, 2 * ks + lg)));
        s = mfma(kf, W.qh[ks], s);
        if constexpr (NP == 2) {
            const bf16x8 kfl = as_bf16x8(*(const u32x4*)(buf + SG::kOff(1, blk) + swzK(lq, 2 * ks + lg)));
            s = mfma(kf, W.ql[ks], s);
            s = mfma(kfl, W.qh[ks], s);
        }
    }
    if constexpr (MODE != kInterior) {
        const int* gcls = (const int*)(buf + SG::gclsOff) + blk * KBLK;
        // this lane's 16 keys are rows 8*(i>>2) + 4*lg + (i&3): shift the mask
        // word so that bit i of `badl` belongs to accumulator element i
        const uint32_t sh = bad >> (4 * lg);
        const uint32_t badl = (sh & 0xfu) | ((sh >> 4) & 0xf0u) | ((sh >> 8) & 0xf00u) | ((sh >> 12) & 0xf000u);
        int gc[16];
        if constexpr (MODE == kGlobalKeys) {
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                const u32x4 g4 = *(const u32x4*)(gcls + 8 * q4 + 4 * lg);
                gc[4 * q4 + 0] = (int)g4[0]; gc[4 * q4 + 1] = (int)g4[1];
                gc[4 * q4 + 2] = (int)g4[2]; gc[4 * q4 + 3] = (int)g4[3];
            }
        }
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int kl = 8 * (i >> 2) + 4 * lg + (i & 3);   // key row inside the block
            bool ok = ((badl >> i) & 1u) == 0u;
            if constexpr (MODE == kBandEdge) {
                const int dk = key0 + kl - m;
                ok &= (uint32_t)(dk + r) <= (uint32_t)(2 * r);
            } else if constexpr (MODE == kGlobalKeys) {
                const int dk = gc[i] - m;
                ok &= (uint32_t)(dk + r) > (uint32_t)(2 * r);   // not already in the window
            }
            s[i] = ok ? s[i] : kNegInf;
        }
    }
    return s;
}

// Running max/sum update for the scores of NB blocks at once: the raw-score
// max is taken to base 2 with the 1/sqrt(d) scale, and O is rescaled only when
// the max grows by more than 2^8 (so every exponent stays <= 8 and the final
// O / l is unaffected).
template <int NB, int NP>
__device__ __forceinline__ void update_max(WaveState<NP>& W, const f32x16 (&s)[NB]) {
    float mx = s[0][0];
#pragma unroll
    for (int b = 0; b < NB; b++)
#pragma unroll
        for (int i = 0; i < 16; i++) mx = __builtin_fmaxf(mx, s[b][i]);
    mx = halves_max(mx);
    const float mxs = mx * kScaleLog2;
    const bool need = mxs > W.ms + 8.0f;
    if (__ballot(need)) {
        const float msn = need ? mxs : W.ms;
        const float alpha = need ? __builtin_amdgcn_exp2f(W.ms - msn) : 1.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) { W.o0[i] *= alpha; W.o1[i] *= alpha; }
        W.lp *= alpha;
        W.ms = msn;
    }
}

// p = 2^(s*scale - m) for one block, its row-sum, and O^T += V^T P^T
template <int KS, int NP>
__device__ __forceinline__ void block_pv(WaveState<NP>& W, const f32x16& s, const char* buf, int blk, int lane) {
    using SG = Stage<KS, NP>;
    const float nms = (W.ms == kNegInf) ? 0.0f : -W.ms;
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; i++) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], kScaleLog2, nms));
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 16; i++) ps += p[i];
    W.lp += ps;
    // P^T operands: step st covers accumulator elements 8st .. 8st+7
    bf16x8 pb[2], pbl[2];
#pragma unroll
    for (int st = 0; st < 2; st++) {
        u32x4 w, wl;
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const float a = p[8 * st + 2 * e], b = p[8 * st + 2 * e + 1];
            const uint32_t hw = pack_bf16(a, b);
            w[e] = hw;
            if constexpr (NP == 2) {
                const float ah = __builtin_bit_cast(float, hw << 16);
                const float bh = __builtin_bit_cast(float, hw & 0xffff0000u);
                wl[e] = pack_bf16(a - ah, b - bh);
            }
        }
        pb[st] = as_bf16x8(w);
        if constexpr (NP == 2) pbl[st] = as_bf16x8(wl);
    }
    // V^T operands by transposing reads: lane (16G + L) supplies row
    // 16st + 8hf + 4(G>>1) + (L>>2), channels 32cb + 16(G&1) + 4(L&3)
    const int G = lane >> 4, L = lane & 15;
    const int t0 = 4 * (G >> 1) + (L >> 2);
#pragma unroll
    for (int st = 0; st < 2; st++) {
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            const int byte = 64 * cb + 32 * (G & 1) + 8 * (L & 3);
            const int ch = byte >> 4, inner = byte & 15;
            const int ta = 16 * st + t0, tb = ta + 8;
            const char* vb = buf + SG::vOff(0, blk);
            const bf16x8 va = cat_tr(ds_tr16(vb + swzV(ta, ch) + inner), ds_tr16(vb + swzV(tb, ch) + inner));
            f32x16& oc = cb ? W.o1 : W.o0;
            oc = mfma(va, pb[st], oc);
            if constexpr (NP == 2) {
                const char* vbl = buf + SG::vOff(1, blk);
                const bf16x8 val = cat_tr(ds_tr16(vbl + swzV(ta, ch) + inner), ds_tr16(vbl + swzV(tb, ch) + inner));
                oc = mfma(va, pbl[st], oc);
                oc = mfma(val, pb[st], oc);
            }
        }
    }
}

// One block: `bad` has bit t set when key row t of the block is not a real key.
template <int MODE, int KS, int NP>
__device__ __forceinline__ void attend_block(WaveState<NP>& W, const char* buf, int blk, int key0, uint32_t bad,
                                             int m, int r, int lane) {
    f32x16 s[1] = {block_scores<MODE, KS, NP>(W, buf, blk, key0, bad, m, r, lane)};
    update_max<1, NP>(W, s);
    block_pv<KS, NP>(W, s[0], buf, blk, lane);
}

// two blocks with one max update: the second block's score MFMAs are issued
// before the first block's softmax, so they overlap its VALU work
template <int MODE0, int MODE1, int KS, int NP>
__device__ __forceinline__ void attend_pair(WaveState<NP>& W, const char* buf, int blk0, int key0, uint32_t bad0,
                                            int blk1, int key1, uint32_t bad1, int m, int r, int lane) {
    f32x16 s[2];
    s[0] = block_scores<MODE0, KS, NP>(W, buf, blk0, key0, bad0, m, r, lane);
    s[1] = block_scores<MODE1, KS, NP>(W, buf, blk1, key1, bad1, m, r, lane);
    update_max<2, NP>(W, s);
    block_pv<KS, NP>(W, s[0], buf, blk0, lane);
    block_pv<KS, NP>(W, s[1], buf, blk1, lane);
}

// Masking chosen at run time (wave-uniform), so one code path serves every
// block kind and O stays in one set of registers.
enum MaskKind { kMaskNone = 0, kMaskBand = 1, kMaskGlobal = 2, kMaskBad = 3 };

__device__ __forceinline__ void apply_mask(f32x16& s, int kind, uint32_t bad, int key0, const int* gcls,
                                           int m, int r, int lg) {
    if (kind == kMaskNone) return;
    const uint32_t sh = bad >> (4 * lg);
    const uint32_t badl = (sh & 0xfu) | ((sh >> 4) & 0xf0u) | ((sh >> 8) & 0xf00u) | ((sh >> 12) & 0xf000u);
    if (kind == kMaskBand) {
        // keys key0 + kl with kl = 8*(i>>2) + 4*lg + (i&3) must lie in [m - r, m + r]
        const int lo = m - r - key0 - 4 * lg, hi = m + r - key0 - 4 * lg;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int kc = 8 * (i >> 2) + (i & 3);
            const bool ok = ((badl >> i) & 1u) == 0u && kc >= lo && kc <= hi;
            s[i] = ok ? s[i] : kNegInf;
        }
    } else if (kind == kMaskGlobal) {
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++) {
            const u32x4 g4 = *(const u32x4*)(gcls + 8 * q4 + 4 * lg);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const int i = 4 * q4 + e;
                const int dk = (int)g4[e] - m;
                const bool ok = ((badl >> i) & 1u) == 0u && (uint32_t)(dk + r) > (uint32_t)(2 * r);
                s[i] = ok ? s[i] : kNegInf;
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < 16; i++) s[i] = ((badl >> i) & 1u) ? kNegInf : s[i];
    }
}

// Up to two blocks of one stage for one wave.  live0/live1 say whether each
// block has work for this wave (a dead block costs no MFMA and adds nothing).
template <int KS, int NP>
__device__ __forceinline__ void attend_stage(WaveState<NP>& W, const char* buf, int blk0, bool live0, int kind0,
                                             uint32_t bad0, int key0, bool live1, int kind1, uint32_t bad1,
                                             int key1, int m, int r, int lane) {
    using SG = Stage<KS, NP>;
    const int lg = lane >> 5;
    const int* gcls = (const int*)(buf + SG::gclsOff);
    f32x16 s[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const bool live = u ? live1 : live0;
        if (live) {
            s[u] = block_scores<kInterior, KS, NP>(W, buf, blk0 + u, 0, 0u, m, r, lane);
            apply_mask(s[u], u ? kind1 : kind0, u ? bad1 : bad0, u ? key1 : key0, gcls + (blk0 + u) * KBLK,
                       m, r, lg);
        } else {
#pragma unroll
            for (int i = 0; i < 16; i++) s[u][i] = kNegInf;
        }
    }
    update_max<2, NP>(W, s);
    if (live0) block_pv<KS, NP>(W, s[0], buf, blk0, lane);
    if (live1) block_pv<KS, NP>(W, s[1], buf, blk0 + 1, lane);
}

// ---------------------------------------------------------------------------
// The tile kernel.

template <int QB, int KS, typename ET, typename OT>
__global__ __launch_bounds__(64 * QB * KS) __attribute__((amdgpu_waves_per_eu(LFK_WAVES_PER_EU)))
void tile_kernel(const Params P) {
    constexpr int NT = 64 * QB * KS;
    constexpr int NP = Elem<ET>::NP;
    constexpr int NBW = NP == 1 ? 2 : 1;       // blocks per wave per stage (processed as a pair)
    constexpr int NBLK = KS * NBW;             // blocks per stage
    static_assert(NBLK <= QB * KS, "one mask wave per block");
    using SG = Stage<NBLK, NP>;
    constexpr int R = NBLK * KBLK;             // key rows per stage
    constexpr int CHUNKS = R * 8;              // 8-channel chunks per tensor per stage
    static_assert(CHUNKS % NT == 0, "stage chunks must divide evenly over the workgroup");
    constexpr int CPT = CHUNKS / NT;           // chunks per thread per tensor
    constexpr int MERGE_BYTES = (KS - 1) * QB * 64 * 36 * 4;
    constexpr int SMEM = (SG::bytes > MERGE_BYTES) ? SG::bytes : MERGE_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];

    // ---- which task (XCD-aware: each of the 8 dies takes a contiguous task range)
    const int per_xcd = gridDim.x >> 3;
    const int task_id = (blockIdx.x & 7) * per_xcd + (blockIdx.x >> 3);
    if (task_id >= P.n_tasks) return;
    const Task tk = decode_task<QB>(P, task_id);

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int qb = wave % QB;
    const int ph = wave / QB;          // key phase of this wave
    const int lq = lane & 31;          // query column owned by this lane
    const int lg = lane >> 5;

    const size_t head_off = (size_t)tk.bh * P.T * D;
    const ET* __restrict__ Kg = (const ET*)P.k + head_off;
    const ET* __restrict__ Vg = (const ET*)P.v + head_off;
    const ET* __restrict__ Qg = (const ET*)P.q + head_off;
    const uint8_t* __restrict__ padrow = P.pad ? P.pad + (size_t)tk.b * P.T : nullptr;
    const int r = P.r;

    // ---- this wave's 32 queries
    const int mq0 = tk.m0 + 32 * qb;   // first query (class index, or global slot)
    bool wave_active;
    int my_pos = -1;                   // position of this lane's query
    if (tk.kind == 0) {
        wave_active = mq0 < tk.n;
        const int m = mq0 + lq;
        if (m < tk.n) my_pos = tk.c + tk.delta * m;
    } else {
        wave_active = mq0 < P.n_g;
        const int sl = mq0 + lq;
        if (sl < P.n_g) my_pos = P.glob[sl];
    }
    const bool my_pad = (my_pos >= 0 && padrow) ? padrow[my_pos] != 0 : false;

    WaveState<NP> W;
    {
        const bool ok = my_pos >= 0 && !my_pad;
        const ET* qrow = Qg + (size_t)(ok ? my_pos : 0) * D;
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const int c0 = 16 * ks + 8 * lg;
            if constexpr (NP == 1) {
                const u32x4 x = *(const u32x4*)(qrow + c0);
                W.qh[ks] = as_bf16x8(ok ? x : (u32x4){0, 0, 0, 0});
            } else {
                Raw32 x;
                x.a = *(const u32x4*)(qrow + c0);
                x.b = *(const u32x4*)(qrow + c0 + 4);
                if (!ok) { x.a = (u32x4){0, 0, 0, 0}; x.b = x.a; }
                u32x4 hi, lo;
                split8(x, hi, lo);
                W.qh[ks] = as_bf16x8(hi);
                W.ql[ks] = as_bf16x8(lo);
            }
        }
    }
    W.o0 = (f32x16){};
    W.o1 = (f32x16){};
    W.ms = kNegInf;
    W.lp = 0.f;

    // band blocks this wave's queries can reach
    int wb_lo = 0, wb_hi = -1;
    if (tk.kind == 0) {
        int a = mq0 - r; if (a < 0) a = 0;
        int z = mq0 + 31 + r; if (z > tk.n - 1) z = tk.n - 1;
        wb_lo = a / KBLK;
        wb_hi = z / KBLK;
    }

    // ---- stage plan: band (or dense) stages, then global-key stages
    const int ngb = tk.kind == 0 ? cdiv(P.n_g, KBLK) : 0;
    const int NSb = cdiv(tk.nband, NBLK);
    const int NS = NSb + cdiv(ngb, NBLK);
    // LDS mask words are only needed where the key range alone does not say
    // which rows are real: with padding, and for the global-key stages
    const bool lds_mask_band = padrow != nullptr;

    // loader geometry: chunk j of this thread is stage row lrow0 + j * NT/8,
    // channels 8*lch .. 8*lch+7; band rows advance by R keys per stage
    const int lch = tid & 7;
    const int lrow0 = tid >> 3;
    const int key_base = tk.kb_lo * KBLK;
    const int rowstep = tk.delta * D;                 // elements between consecutive class keys

    struct Regs {
        u32x4 k[CPT][NP];
        u32x4 v[CPT][NP];
        uint32_t inr;         // bit j: chunk j's row is a real position
        bool full;            // every row of the stage is a real, unpadded key
        uint8_t padb[CPT];    // that position's padding byte (0 without padding)
        bool minr;            // mask lanes: row is a real position
        uint8_t mpad;         // ... and its padding byte
        int gcls;
    };

    // Loads are issued unconditionally from clamped (always valid) addresses;
    // whether a row is real or padded is only applied when the registers are
    // written to LDS, so no branch waits on these loads before the compute.
    // Order inside a stage load: every position lookup and every small load
    // (padding bytes, global classes) first, the K/V loads last.  Nothing is
    // then written after the K/V loads into a register an earlier load could
    // still own, so the compiler places no wait on them before the compute.
    auto issue = [&](int st, Regs& Rg) {
        const bool band = st < NSb;
        const bool masklane = (!band || lds_mask_band) && wave < NBLK;
        int pos[CPT];
        int mpos = 0;
        bool minr = false;
        Rg.inr = 0;
        Rg.full = band && !padrow && key_base + (st + 1) * R <= tk.key_end;
        if (band) {
#pragma unroll
            for (int j = 0; j < CPT; j++) {
                const int kk = key_base + st * R + lrow0 + j * (NT / 8);
                const bool inr = kk < tk.key_end;
                pos[j] = inr ? tk.c + tk.delta * kk : 0;
                Rg.inr |= (uint32_t)inr << j;
            }
            if (masklane) {
                const int kk = key_base + st * R + 32 * wave + lq;
                minr = kk < tk.key_end;
                mpos = minr ? tk.c + tk.delta * kk : 0;
            }
        } else {
#pragma unroll
            for (int j = 0; j < CPT; j++) {
                const int slot = (st - NSb) * R + lrow0 + j * (NT / 8);
                const bool inr = slot < P.n_g;
                pos[j] = P.glob[inr ? slot : 0];
                Rg.inr |= (uint32_t)inr << j;
            }
            if (masklane) {
                const int slot = (st - NSb) * R + 32 * wave + lq;
                minr = slot < P.n_g;
                mpos = P.glob[minr ? slot : 0];
            }
        }
        if (masklane) {
            Rg.minr = minr && lg == 0;
            Rg.mpad = padrow ? padrow[mpos] : (uint8_t)0;
            const int dpos = mpos - tk.c;
            const int q = dpos / tk.delta;
            Rg.gcls = (!band && minr && dpos >= 0 && q * tk.delta == dpos) ? q : kNotInClass;
        }
        if (padrow) {
#pragma unroll
            for (int j = 0; j < CPT; j++) Rg.padb[j] = padrow[pos[j]];
        }
#pragma unroll
        for (int j = 0; j < CPT; j++) {
            const size_t off = (size_t)pos[j] * D + lch * 8;
#pragma unroll
            for (int p = 0; p < NP; p++) {
                Rg.k[j][p] = *(const u32x4*)(Kg + off + 4 * p);
                Rg.v[j][p] = *(const u32x4*)(Vg + off + 4 * p);
            }
        }
    };

    auto commit = [&](int st, const Regs& Rg) {
        const u32x4 z = {0, 0, 0, 0};
        char* buf = smem;
#pragma unroll
        for (int j = 0; j < CPT; j++) {
            const int row = lrow0 + j * (NT / 8);
            const int blk = row >> 5, t = row & 31;
            const bool ok = Rg.full || (((Rg.inr >> j) & 1u) != 0u && (!padrow || Rg.padb[j] == 0));
            if constexpr (NP == 1) {
                *(u32x4*)(buf + SG::kOff(0, blk) + swzK(t, lch)) = ok ? Rg.k[j][0] : z;
                *(u32x4*)(buf + SG::vOff(0, blk) + swzV(t, lch)) = ok ? Rg.v[j][0] : z;
            } else {
                u32x4 kh, kl, vh, vl;
                split8(Raw32{Rg.k[j][0], Rg.k[j][1]}, kh, kl);
                split8(Raw32{Rg.v[j][0], Rg.v[j][1]}, vh, vl);
                *(u32x4*)(buf + SG::kOff(0, blk) + swzK(t, lch)) = ok ? kh : z;
                *(u32x4*)(buf + SG::kOff(1, blk) + swzK(t, lch)) = ok ? kl : z;
                *(u32x4*)(buf + SG::vOff(0, blk) + swzV(t, lch)) = ok ? vh : z;
                *(u32x4*)(buf + SG::vOff(1, blk) + swzV(t, lch)) = ok ? vl : z;
            }
        }
        if ((st >= NSb || lds_mask_band) && wave < NBLK) {
            const uint32_t good = (uint32_t)__ballot(Rg.minr && Rg.mpad == 0);   // lanes 0..31 only
            if (lane == 0) *(uint32_t*)(buf + SG::maskOff + wave * 4) = ~good;
            if (lg == 0) ((int*)(buf + SG::gclsOff))[wave * KBLK + lq] = Rg.gcls;
        }
    };

    // mask word of stage block `blk`: from LDS, or from the key range alone
    auto block_bad = [&](int st, int blk) -> uint32_t {
        if (st >= NSb || lds_mask_band) return *(const uint32_t*)(smem + SG::maskOff + blk * 4);
        const int key0 = key_base + st * R + blk * KBLK;
        const int valid = tk.key_end - key0;
        return valid >= KBLK ? 0u : (valid <= 0 ? 0xffffffffu : (0xffffffffu << valid));
    };

    // ---- main loop: prefetch stage st+1 into registers while stage st is in LDS
    {
        Regs Rg;
        issue(0, Rg);
        commit(0, Rg);
        __syncthreads();
    }
    const int m_me = mq0 + lq;         // this lane's query (class index / global slot)
    // which of this wave's blocks of stage st have work, and how to mask them
    struct StagePlan {
        bool live[NBW];
        int kind[NBW], key0[NBW];
        uint32_t bad[NBW];
    };
    const int b0 = ph * NBW;           // this wave's blocks: NBW consecutive blocks of phase ph
    auto plan = [&](int st) {
        StagePlan sp;
#pragma unroll
        for (int u = 0; u < NBW; u++) {
            sp.bad[u] = block_bad(st, b0 + u);
            if (st < NSb) {
                const int jb = st * NBLK + b0 + u;
                const int kb = tk.kb_lo + jb;
                sp.key0[u] = kb * KBLK;
                sp.live[u] = wave_active && jb < tk.nband && sp.bad[u] != 0xffffffffu &&
                             (tk.kind == 1 || (kb >= wb_lo && kb <= wb_hi));
                const bool interior = tk.kind == 0 && sp.bad[u] == 0u && sp.key0[u] >= mq0 + 31 - r &&
                                      sp.key0[u] + 31 <= mq0 + r;
                sp.kind[u] = tk.kind == 1 ? kMaskBad : (interior ? kMaskNone : kMaskBand);
            } else {
                const int jg = (st - NSb) * NBLK + b0 + u;
                sp.key0[u] = 0;
                sp.live[u] = wave_active && jg < ngb && sp.bad[u] != 0xffffffffu;
                sp.kind[u] = kMaskGlobal;
            }
        }
        return sp;
    };
    // the score MFMAs of the stage's blocks
    auto scores = [&](const StagePlan& sp, f32x16 (&sc)[NBW]) {
#pragma unroll
        for (int u = 0; u < NBW; u++)
            if (sp.live[u]) sc[u] = block_scores<kInterior, NBLK, NP>(W, smem, b0 + u, 0, 0u, m_me, r, lane);
    };
    // masking, running max/sum and O += P V
    auto finish = [&](const StagePlan& sp, f32x16 (&sc)[NBW]) {
        bool any = false;
#pragma unroll
        for (int u = 0; u < NBW; u++) any = any || sp.live[u];
        if (!any) return;
        const int* gcls = (const int*)(smem + SG::gclsOff);
#pragma unroll
        for (int u = 0; u < NBW; u++) {
            if (sp.live[u]) {
                apply_mask(sc[u], sp.kind[u], sp.bad[u], sp.key0[u], gcls + (b0 + u) * KBLK, m_me, r, lg);
            } else {
#pragma unroll
                for (int i = 0; i < 16; i++) sc[u][i] = kNegInf;
            }
        }
        update_max<NBW, NP>(W, sc);
#pragma unroll
        for (int u = 0; u < NBW; u++)
            if (sp.live[u]) block_pv<NBLK, NP>(W, sc[u], smem, b0 + u, lane);
    };

    // Every stage but the last: score MFMAs, then the next stage's loads (they
    // queue while the matrix cores run), then the softmax and PV, then the LDS
    // hand-over.  Straight-line code, so the loads stay where they are.
    for (int st = 0; st + 1 < NS; st++) {
        const StagePlan sp = plan(st);
        f32x16 sc[NBW];
        scores(sp, sc);
        Regs Rg;
        issue(st + 1, Rg);
        finish(sp, sc);
        __syncthreads();               // every wave is done reading stage st
        commit(st + 1, Rg);
        __syncthreads();               // stage st+1 is in LDS
    }
    {
        const StagePlan sp = plan(NS - 1);
        f32x16 sc[NBW];
        scores(sp, sc);
        finish(sp, sc);
    }
    __syncthreads();

    // ---- merge the KS phases of each query block (LDS); phase 0 keeps the result
    if constexpr (KS > 1) {
        float* mbuf = (float*)smem;
        if (ph > 0) {
            float* dst = mbuf + (((ph - 1) * QB + qb) * 64 + lane) * 36;
            dst[0] = W.ms;
            dst[1] = W.lp;
#pragma unroll
            for (int i = 0; i < 16; i++) { dst[2 + i] = W.o0[i]; dst[18 + i] = W.o1[i]; }
        }
        __syncthreads();
        if (ph == 0) {
#pragma unroll
            for (int p2 = 1; p2 < KS; p2++) {
                const float* src = mbuf + (((p2 - 1) * QB + qb) * 64 + lane) * 36;
                const float ms2 = src[0], lp2 = src[1];
                const float mn = __builtin_fmaxf(W.ms, ms2);
                const float a1 = (W.ms == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(W.ms - mn);
                const float a2 = (ms2 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ms2 - mn);
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    W.o0[i] = W.o0[i] * a1 + src[2 + i] * a2;
                    W.o1[i] = W.o1[i] * a1 + src[18 + i] * a2;
                }
                W.lp = W.lp * a1 + lp2 * a2;
                W.ms = mn;
            }
        }
    }

    const bool writer = ph == 0 && wave_active;
    const float l = halves_sum(W.lp);

    if (tk.kind == 0) {
        // ---- epilogue: y = O / l for the tile's valid queries; padded rows -> 0.
        // Rows of global queries are left to the global-row combine.
        if (!writer || my_pos < 0) return;
        if (P.n_g > 0 && is_global(P, my_pos)) return;
        OT* orow = (OT*)P.out + head_off + (size_t)my_pos * D;
        const float inv = (my_pad || l == 0.f) ? 0.f : 1.0f / l;
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            const f32x16& oc = cb ? W.o1 : W.o0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int c0 = 32 * cb + 8 * j + 4 * lg;
                const float y0 = oc[4 * j + 0] * inv, y1 = oc[4 * j + 1] * inv;
                const float y2 = oc[4 * j + 2] * inv, y3 = oc[4 * j + 3] * inv;
                if constexpr (sizeof(OT) == 2) {
                    const u32x2 w = {pack_bf16(y0, y1), pack_bf16(y2, y3)};
                    *(u32x2*)(orow + c0) = w;
                } else {
                    const f32x4 w = {y0, y1, y2, y3};
                    *(f32x4*)(orow + c0) = w;
                }
            }
        }
        return;
    }

    // ---- global rows: write this split's (max, sum, O) for each global slot.
    // Partials cross dies (each XCD has its own L2), so they are written and
    // read as agent-scope relaxed atomics, which go to the coherent memory
    // side without writing back or invalidating whole L2s the way a
    // device-wide fence does.
    const int slot = mq0 + lq;
    if (writer && slot < P.n_g) {
        uint32_t* part = (uint32_t*)P.part + (((size_t)tk.bh * P.n_split + tk.split) * P.g_pad + slot) * (D + 2);
        if (lg == 0) {
            store_coherent(part + 0, W.ms);
            store_coherent(part + 1, l);
        }
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            const f32x16& oc = cb ? W.o1 : W.o0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int c0 = 32 * cb + 8 * j + 4 * lg;
#pragma unroll
                for (int e = 0; e < 4; e++) store_coherent(part + 2 + c0 + e, oc[4 * j + e]);
            }
        }
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
    // one wave per global row; lanes first span the splits (max and sum of the
    // rescaled partial sums), then the 64 channels (rescaled partial outputs,
    // loads issued back to back)
    constexpr int NW = NT / 64;
    const size_t stride = (size_t)P.g_pad * (D + 2);
    for (int gi = wave; gi < P.n_g; gi += NW) {
        const int pos = P.glob[gi];
        OT* orow = (OT*)P.out + head_off + (size_t)pos * D;
        const bool padded = padrow && padrow[pos] != 0;
        const uint32_t* base = (const uint32_t*)P.part + ((size_t)tk.bh * P.n_split * P.g_pad + gi) * (D + 2);
        const bool mine = lane < P.n_split;
        const float m_s = mine ? load_coherent(base + lane * stride) : kNegInf;
        const float l_s = mine ? load_coherent(base + lane * stride + 1) : 0.f;
        float M = m_s;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) M = __builtin_fmaxf(M, __shfl_xor(M, off));
        const float w_s = (m_s == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(m_s - M);
        float Lsum = l_s * w_s;
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) Lsum += __shfl_xor(Lsum, off);
        float O = 0.f;
        for (int s0 = 0; s0 < P.n_split; s0 += 16) {
            float ov[16];
#pragma unroll
            for (int j = 0; j < 16; j++) ov[j] = (s0 + j < P.n_split) ? load_coherent(base + (s0 + j) * stride + 2 + lane) : 0.f;
#pragma unroll
            for (int j = 0; j < 16; j++) O += ov[j] * __shfl(w_s, s0 + j);
        }
        const float y = (padded || !(Lsum > 0.f)) ? 0.f : O / Lsum;
        if constexpr (sizeof(OT) == 2) {
            orow[lane] = (OT)(pack_bf16(y, 0.f) & 0xffffu);
        } else {
            orow[lane] = y;
        }
    }
    if (tid == 0) __hip_atomic_store(P.counter + tk.bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

}  // namespace lfk

// ---------------------------------------------------------------------------
// launcher (called from the host library)

extern "C" hipError_t lfk_launch(const lfk::Params* P, int dtype_bf16, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    constexpr int QB = LFK_QB, KS = LFK_KS;
    const int grid = ((P->n_tasks + 7) / 8) * 8;
    if (dtype_bf16)
        hipLaunchKernelGGL((lfk::tile_kernel<QB, KS, __bf16, uint16_t>), dim3(grid), dim3(64 * QB * KS), 0, s, *P);
    else
        hipLaunchKernelGGL((lfk::tile_kernel<QB, KS, float, float>), dim3(grid), dim3(64 * QB * KS), 0, s, *P);
    return hipGetLastError();
}
