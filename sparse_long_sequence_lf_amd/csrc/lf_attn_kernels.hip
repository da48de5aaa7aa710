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
//    reads every position).  Each writes partial (max, sum, weighted-sum)
//    triples; the last split of a head to finish rescales and adds them.
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
// and l^32 hold the two halves of a query's keys).  The softmax is the
// running max/sum form (blockwise accumulation, "Longformer长序列处理",
// 显存优化技巧) kept in base 2 with the 1/sqrt(d) scale folded into one FMA;
// the running max only moves (and O is rescaled) when a block raises it by
// more than 2^8, which keeps every exponent <= 8 and leaves O / l exact.
//
// Key blocks (32 keys) reach LDS straight from memory (buffer_load ... lds,
// no register staging) through a ring of two stages of two blocks each.
// Step s of the loop: one barrier (stage s has landed, stage s-1 is free),
// this wave's fragment reads of its block of stage s, the loads of stage s+1
// into the free slot, then the score MFMAs, softmax and PV of the block.  The
// ring and tables take 38 KiB, so four workgroups share a compute unit (128
// VGPRs per lane for bf16) and the waves of the others run while one waits.
// Rows past the end of the head, and V rows of padded keys, read as zero.
// The two "phases" of a query block take the two blocks of each stage and
// are merged at the end.
//
// fp32 inputs: a pre-pass splits K and V into bf16 hi + lo planes and Q is
// split when loaded; each product uses hi*hi + hi*lo + lo*hi (three MFMAs),
// which keeps the score and output error near 2^-16 relative while the
// tiling, masking and softmax code is the very code the bf16 path runs.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "lf_kernels.h"

namespace lfk {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(p) ((__attribute__((address_space(3))) void*)(p))

constexpr int D = 64;
constexpr int KBLK = 32;                  // keys per block (one S^T tile)
constexpr float kNegInf = -__builtin_huge_valf();
constexpr int kNotInClass = -(1 << 30);
constexpr int kRawBufferWord3 = 0x00020000;   // raw buffer, 32-bit data format, no swizzle
constexpr uint32_t kPastEnd = 0xFFFFFF00u;     // buffer offset past any resource's end (reads zero)
constexpr int kCoherent = 16;                  // buffer cache policy sc1: coherent across the dies' L2s
constexpr int kRecBytes = 272;                 // global-row partial record: O[64], m, l, pad[2]
constexpr int kVecGlobals = 2;                 // band tasks take up to this many global keys on the VALU

// log2(e) / sqrt(64): scores are taken to base 2 with the 1/sqrt(d) scale.
constexpr float kScaleLog2 = 0.18033688011112042f;

// ---------------------------------------------------------------------------
// LDS layout.  A block holds, per bf16 plane (NP = 1 for bf16, 2 for the
// hi/lo planes of fp32), 32 K rows then 32 V rows:
//
//   K: byte ks*1024 + row*32 + hs*16 holds channels 16ks + 8h .. +7 with
//      hs = h ^ ((row >> 3) & 1).  The 16 lanes of one ds_read_b128 (rows
//      t..t+15, one h) then touch 16 distinct 4-bank groups.
//   V: byte 4096 + cb*2048 + row*64 + 16j holds channels 32cb + 8j .. +7.
//      Half a wave of ds_read_b64_tr_b16 reads rows t..t+3 x 64 B: 256
//      consecutive bytes, all 64 banks once.
//
// Each 1 KiB piece (a K slice, or 16 V rows of one cb) is what one
// buffer_load_dwordx4 ... lds of 64 lanes writes, lane p at byte 16p.
template <int NP>
struct Ring {
    static constexpr int PLANE = 8192;
    static constexpr int BLK = NP * PLANE;
    static constexpr int STAGE = 2 * BLK;                       // two blocks: one per phase
    static constexpr int NBUF = 2;
    static constexpr int gposOff = NBUF * STAGE;                // global positions (sorted)
    static constexpr int gldOff = gposOff + 4 * LF_MAX_GLOBALS;  // position each slot loads (T: none)
    static constexpr int gclsOff = gldOff + 4 * LF_MAX_GLOBALS;  // class index, or kNotInClass
    static constexpr int gbadOff = gclsOff + 4 * LF_MAX_GLOBALS; // per global block: missing / padded slots
    static constexpr int bytes = gbadOff + 4 * (LF_MAX_GLOBALS / 32);
};

template <typename T> struct Elem;
template <> struct Elem<__bf16> { static constexpr int NP = 1; };
template <> struct Elem<float> { static constexpr int NP = 2; };

struct Raw32 { u32x4 a, b; };

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
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) i16x4*)(lds_ptr));
}

__device__ __forceinline__ bf16x8 cat_tr(i16x4 a, i16x4 b) {
    return __builtin_bit_cast(bf16x8, __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7));
}

// raw buffer over [base, base + bytes): accesses at offsets >= bytes read zero
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRawBufferWord3);
}

// 16 bytes per lane from rsrc at voff + soff into LDS at dst + 16 * lane
__device__ __forceinline__ void load_lds16(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t voff, uint32_t soff) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, LDS_PTR(dst), 16, voff, soff, 0, 0);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Barrier after which every wave's loads into LDS have landed.  A plain
// __syncthreads() waits only for LDS instructions (lgkmcnt), not for
// buffer_load ... lds, which counts on vmcnt: each wave first waits for its
// own (s_waitcnt vmcnt(0): gfx9 encoding, expcnt and lgkmcnt left open).
__device__ __forceinline__ void barrier_lds_loads() {
    __builtin_amdgcn_s_waitcnt(0x0F70);
    __syncthreads();
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
    int r, ra;       // band: the window reaches r keys back and ra forward (ra = 0 one-sided)
};

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

template <int QB>
__device__ __forceinline__ Task decode_task(const Plan& P, int t) {
    constexpr int BM = 32 * QB;
    Task k;
    if (t < P.n_band_tasks) {
        k.kind = 0;
        k.b = t / P.band_tasks_per_batch;
        int x = t - k.b * P.band_tasks_per_batch;
        int h;
        if (P.uniform_head_tasks > 0) {
            h = x / P.uniform_head_tasks;
            x -= h * P.uniform_head_tasks;
        } else {
            // heads are few (<= LF_MAX_HEADS): binary search on the band-task prefix
            int lo = 0, hi = P.H - 1;
            while (lo < hi) {
                const int mid = (lo + hi + 1) >> 1;
                if (P.head_start[mid] <= x) lo = mid; else hi = mid - 1;
            }
            h = lo;
            x -= P.head_start[h];
        }
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
        const int r = P.rad[h];
        k.r = r;
        k.ra = P.one_sided ? 0 : r;
        int lo_k = k.m0 - r; if (lo_k < 0) lo_k = 0;
        int hi_k = k.m0 + BM - 1 + k.ra; if (hi_k > k.n - 1) hi_k = k.n - 1;
        k.kb_lo = lo_k / KBLK;
        k.nband = hi_k / KBLK - k.kb_lo + 1;
        k.key_end = k.n;
        k.split = 0;
    } else {
        k.kind = 1;
        k.r = 0;
        k.ra = 0;
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

// reductions over the two 32-lane halves (lanes l and l^32 hold the two key
// halves of a query): one v_permlane32_swap, no LDS round trip
__device__ __forceinline__ float halves_max(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const f32x2 f = __builtin_bit_cast(f32x2, r);
    return __builtin_elementwise_maximum(f[0], f[1]);
}
__device__ __forceinline__ float halves_sum(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__builtin_bit_cast(uint32_t, x),
                                                    __builtin_bit_cast(uint32_t, x), false, false);
    const f32x2 f = __builtin_bit_cast(f32x2, r);
    return f[0] + f[1];
}

// ---------------------------------------------------------------------------
// Per-wave attention state and the work on one 32-key block.

template <int NP>
struct WaveState {
    bf16x8 qh[4], ql[4];  // Q^T operands (lo part only for fp32 inputs)
    f32x16 o0, o1;        // O^T: channels 0..31 and 32..63 of this lane's query
    float ms;             // running max in scaled base-2 units
    float nms;            // -ms, or 0 while ms is -inf (the exponent offset)
    float thr;            // raw score above which the max must move: (ms + 8) / scale
    float lp;             // this lane's part of the running sum
    int kbase;            // LDS offset of this lane's K operand bytes inside a block
    int vbase;            // LDS offset of this lane's V^T operand bytes inside a block
};

// K operands of one block for S^T = K Q^T (32 keys x this wave's 32
// queries): lane l supplies key row l%32, channels 16ks + 8(l/32) .. +7
template <int NP>
struct KFrag { u32x4 k[4][NP]; };

template <int NP>
__device__ __forceinline__ KFrag<NP> load_k(const WaveState<NP>& W, const char* blk) {
    using RG = Ring<NP>;
    KFrag<NP> f;
    const char* kb = blk + W.kbase;
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
#pragma unroll
        for (int p = 0; p < NP; p++) f.k[ks][p] = *(const u32x4*)(kb + p * RG::PLANE + 1024 * ks);
    return f;
}

template <int NP>
__device__ __forceinline__ f32x16 block_scores(const WaveState<NP>& W, const KFrag<NP>& f) {
    f32x16 s = {};
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        s = mfma(as_bf16x8(f.k[ks][0]), W.qh[ks], s);
        if constexpr (NP == 2) {
            s = mfma(as_bf16x8(f.k[ks][0]), W.ql[ks], s);
            s = mfma(as_bf16x8(f.k[ks][1]), W.qh[ks], s);
        }
    }
    return s;
}

// Masking.  Lane l holds the scores of keys 8*(i>>2) + 4*(l/32) + (i&3) of
// the block in accumulator element i.  Bit t of a block's `bad` word is set
// when key row t is not a real key (past the sequence, class or split end,
// padded, or an unused global slot).

// keep bits of this lane's 16 elements from a 32-bit row word
__device__ __forceinline__ uint32_t lane_bits(uint32_t rows, int lg) {
    const uint32_t sh = rows >> (4 * lg);
    return (sh & 0xfu) | ((sh >> 4) & 0xf0u) | ((sh >> 8) & 0xf00u) | ((sh >> 12) & 0xf000u);
}

// band block whose rows are all real keys: keep kc in [lo, lo + width], where
// kc is the element's key row minus 4*lg and lo = m - r - key0 - 4*lg (the
// window reaches r keys back and width - r forward)
__device__ __forceinline__ void mask_window(f32x16& s, int lo, int width) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int kc = 8 * (i >> 2) + (i & 3);
        s[i] = (uint32_t)(kc - lo) <= (uint32_t)width ? s[i] : kNegInf;
    }
}

// random key block: drop the keys inside this query's window (the band
// counts those): kc in [lo, lo + width] as in mask_window
__device__ __forceinline__ void mask_window_out(f32x16& s, int lo, int width) {
#pragma unroll
    for (int i = 0; i < 16; i++) {
        const int kc = 8 * (i >> 2) + (i & 3);
        s[i] = (uint32_t)(kc - lo) <= (uint32_t)width ? kNegInf : s[i];
    }
}

// keep the elements whose bit is set in keep16
__device__ __forceinline__ void mask_bits(f32x16& s, uint32_t keep16) {
#pragma unroll
    for (int i = 0; i < 16; i++) s[i] = ((keep16 >> i) & 1u) ? s[i] : kNegInf;
}

// global-key block: drop unused / padded slots and keys already inside this
// query's window, class distance in [-r, width - r] (the band counts those)
__device__ __forceinline__ void mask_global(f32x16& s, uint32_t bad, const int* gcls, int m, int r, int width,
                                            int lg) {
    const uint32_t badl = lane_bits(bad, lg);
#pragma unroll
    for (int q4 = 0; q4 < 4; q4++) {
        const u32x4 g4 = *(const u32x4*)(gcls + 8 * q4 + 4 * lg);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            const int i = 4 * q4 + e;
            const int dk = (int)g4[e] - m;
            const bool ok = ((badl >> i) & 1u) == 0u && (uint32_t)(dk + r) > (uint32_t)width;
            s[i] = ok ? s[i] : kNegInf;
        }
    }
}

// Running max/sum update for one block's scores.  The raw-score max is taken
// to base 2 with the 1/sqrt(d) scale, and O is rescaled only when the max
// grows by more than 2^8.
template <int NP>
__device__ __forceinline__ void update_max(WaveState<NP>& W, const f32x16& s) {
    // maximum (not fmax): NaN-propagating, so no quieting of the MFMA results
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; i++) mx = __builtin_elementwise_maximum(mx, s[i]);
    // a row's maximum passes the threshold exactly when one of its halves
    // does, so the two halves meet only when some row moves
    if (__ballot(mx > W.thr)) {
        mx = halves_max(mx);
        const bool need = mx > W.thr;
        const float mxs = mx * kScaleLog2;
        const float msn = need ? mxs : W.ms;
        const float alpha = need ? __builtin_amdgcn_exp2f(W.ms - msn) : 1.0f;
#pragma unroll
        for (int i = 0; i < 16; i++) { W.o0[i] *= alpha; W.o1[i] *= alpha; }
        W.lp *= alpha;
        W.ms = msn;
        W.nms = msn == kNegInf ? 0.0f : -msn;
        W.thr = (msn + 8.0f) * (1.0f / kScaleLog2);
    }
}

// V^T operands of one block, by transposing reads: lane (16G + L) supplies
// row 16st + 8hf + 4(G>>1) + (L>>2), channels 32cb + 16(G&1) + 4(L&3) .. +3
// (the lane-dependent part is W.vbase)
template <int NP>
struct VFrag { bf16x8 v[2][2][NP]; };   // [st][cb][plane]

template <int NP>
__device__ __forceinline__ VFrag<NP> load_v(const WaveState<NP>& W, const char* blk) {
    using RG = Ring<NP>;
    VFrag<NP> f;
    const char* vb = blk + 4096 + W.vbase;
#pragma unroll
    for (int st = 0; st < 2; st++)
#pragma unroll
        for (int cb = 0; cb < 2; cb++)
#pragma unroll
            for (int p = 0; p < NP; p++) {
                const char* a = vb + p * RG::PLANE + cb * 2048 + 16 * st * 64;
                f.v[st][cb][p] = cat_tr(ds_tr16(a), ds_tr16(a + 8 * 64));
            }
    return f;
}

// P^T operands of one block (bf16; for fp32 inputs also the low parts)
template <int NP>
struct PFrag { bf16x8 h[2], l[2]; };

// p = 2^(s*scale - m) for one block as P^T operands; returns ps plus this
// lane's part of the block's row sum
template <int NP>
__device__ __forceinline__ float block_weights(const WaveState<NP>& W, const f32x16& s, PFrag<NP>& pf, float ps) {
    const float nms = W.nms;
    float p[16];
#pragma unroll
    for (int i = 0; i < 16; i++) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], kScaleLog2, nms));
    // P^T operands: step st covers accumulator elements 8st .. 8st+7
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
                ps += a + b;
            } else {
                // the row sum of the very bf16 weights that multiply V
                ps = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, hw),
                                                     (bf16x2){(__bf16)1.0f, (__bf16)1.0f}, ps, false);
            }
        }
        pf.h[st] = as_bf16x8(w);
        if constexpr (NP == 2) pf.l[st] = as_bf16x8(wl);
    }
    return ps;
}

// O^T += V^T P^T
template <int NP>
__device__ __forceinline__ void block_product(WaveState<NP>& W, const PFrag<NP>& pf, const VFrag<NP>& f) {
#pragma unroll
    for (int st = 0; st < 2; st++) {
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            f32x16& oc = cb ? W.o1 : W.o0;
            oc = mfma(f.v[st][cb][0], pf.h[st], oc);
            if constexpr (NP == 2) {
                oc = mfma(f.v[st][cb][0], pf.l[st], oc);
                oc = mfma(f.v[st][cb][1], pf.h[st], oc);
            }
        }
    }
}

template <int NP>
__device__ __forceinline__ void block_pv(WaveState<NP>& W, const f32x16& s, const VFrag<NP>& f) {
    PFrag<NP> pf;
    W.lp = block_weights<NP>(W, s, pf, W.lp);
    block_product<NP>(W, pf, f);
}

// A global key taken on the vector units: the K channels of this lane's half
// of the query (the Q operand layout) and the V channels of its O^T rows.
template <int NP>
struct GKey {
    u32x4 kh[4], kl[4];   // bf16 K (hi and, for fp32 inputs, lo part): channels 16ks + 8lg .. +7
    u32x4 v[8];           // V channels 32cb + 8j + 4lg .. +3 ([4cb + j]); bf16 inputs use .xy
};

// rk: K as bf16 rows of NP planes (NP * 128 bytes a row); rv: V rows in the
// input type.  pos past the end (or none) reads zeros.
template <int NP>
__device__ __forceinline__ GKey<NP> load_gkey(__amdgpu_buffer_rsrc_t rk, __amdgpu_buffer_rsrc_t rv, uint32_t pos,
                                               int lg) {
    GKey<NP> g;
    const uint32_t kro = pos * (uint32_t)(NP * 128u), vro = pos * (uint32_t)(NP * 128u);
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const uint32_t o = kro + 2u * (16 * ks + 8 * lg);
        g.kh[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o, 0, 0));
        if constexpr (NP == 2)
            g.kl[ks] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, o + 128u, 0, 0));
    }
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const int ch = 32 * cb + 8 * j + 4 * lg;
            if constexpr (NP == 1) {
                const u32x2 x = __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, vro + 2u * ch, 0, 0));
                g.v[4 * cb + j] = (u32x4){x[0], x[1], 0u, 0u};
            } else {
                g.v[4 * cb + j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rv, vro + 4u * ch, 0, 0));
            }
        }
    return g;
}

// this lane's half of q . k (fp32 inputs: qh kh + qh kl + ql kh, as the MFMA
// path).  Pairs are taken from whole bf16x8 vectors by shuffles: bit-casting
// single elements of an ext_vector miscompiles with this clang.
__device__ __forceinline__ bf16x2 pair(bf16x8 x, int e) {
    switch (e) {
        case 0: return __builtin_shufflevector(x, x, 0, 1);
        case 1: return __builtin_shufflevector(x, x, 2, 3);
        case 2: return __builtin_shufflevector(x, x, 4, 5);
        default: return __builtin_shufflevector(x, x, 6, 7);
    }
}

template <int NP>
__device__ __forceinline__ float gkey_dot(const WaveState<NP>& W, const GKey<NP>& g) {
    float s = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const bf16x8 kh = as_bf16x8(g.kh[ks]);
#pragma unroll
        for (int e = 0; e < 4; e++) {
            s = __builtin_amdgcn_fdot2_f32_bf16(pair(W.qh[ks], e), pair(kh, e), s, false);
            if constexpr (NP == 2) {
                const bf16x8 kl = as_bf16x8(g.kl[ks]);
                s = __builtin_amdgcn_fdot2_f32_bf16(pair(W.qh[ks], e), pair(kl, e), s, false);
                s = __builtin_amdgcn_fdot2_f32_bf16(pair(W.ql[ks], e), pair(kh, e), s, false);
            }
        }
    }
    return s;
}

// fold one key (scaled base-2 score sc, -inf when the key is not in the
// query's set) into the running (m, l, O): the running-max update of the
// blocks, for a single key.  lg == 0 lanes count its weight in l.
template <int NP>
__device__ __forceinline__ void gkey_fold(WaveState<NP>& W, const GKey<NP>& g, float sc, int lg) {
    const float mn = __builtin_fmaxf(W.ms, sc);
    const float alpha = W.ms == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(W.ms - mn);
    const float p = sc == kNegInf ? 0.0f : __builtin_amdgcn_exp2f(sc - mn);
#pragma unroll
    for (int cb = 0; cb < 2; cb++) {
        f32x16& oc = cb ? W.o1 : W.o0;
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const u32x4 x = g.v[4 * cb + j];
            float v4[4];
            if constexpr (NP == 1) {
                // bf16 -> fp32 is the bf16 in the upper half: shift / mask whole vectors
                const f32x4 f = __builtin_bit_cast(
                    f32x4, (u32x4){x[0] << 16, x[0] & 0xffff0000u, x[1] << 16, x[1] & 0xffff0000u});
                v4[0] = f[0]; v4[1] = f[1]; v4[2] = f[2]; v4[3] = f[3];
            } else {
                const f32x4 f = __builtin_bit_cast(f32x4, x);
                v4[0] = f[0]; v4[1] = f[1]; v4[2] = f[2]; v4[3] = f[3];
            }
#pragma unroll
            for (int e = 0; e < 4; e++) oc[4 * j + e] = __builtin_fmaf(oc[4 * j + e], alpha, p * v4[e]);
        }
    }
    W.lp = __builtin_fmaf(W.lp, alpha, lg == 0 ? p : 0.0f);
    W.ms = mn;
    W.nms = mn == kNegInf ? 0.0f : -mn;
    W.thr = (mn + 8.0f) * (1.0f / kScaleLog2);
}

// ---------------------------------------------------------------------------
// The tile kernel.

template <int QB, int KS, typename ET, typename OT, bool PAD, bool RAND>
__global__ __launch_bounds__(64 * QB * KS) __attribute__((amdgpu_waves_per_eu(Elem<ET>::NP == 1 ? LFK_WAVES_PER_EU_BF16 : LFK_WAVES_PER_EU_F32)))
void tile_kernel(const Args A) {
    static_assert(QB == 2 && KS == 2, "four waves: two phases of two query blocks");
    constexpr int NT = 64 * QB * KS;
    constexpr int NP = Elem<ET>::NP;
    constexpr int ROWB = NP * 128;             // bytes per K/V row in the bf16-plane layout
    using RG = Ring<NP>;
    constexpr int MERGE_BYTES = (KS - 1) * QB * 64 * 36 * 4;
    static_assert(MERGE_BYTES <= RG::NBUF * RG::STAGE, "merge area inside the ring");
    __shared__ __attribute__((aligned(16))) char smem[RG::bytes];
    const Plan& P = *A.plan;
    const int* gpos = (const int*)(smem + RG::gposOff);
    const int* gcls = (const int*)(smem + RG::gclsOff);
    const int* gld = (const int*)(smem + RG::gldOff);
    const uint32_t* gbad = (const uint32_t*)(smem + RG::gbadOff);

    // ---- which task.  Each of the 8 dies (blockIdx % 8) takes an eighth of
    // the global-row tasks first, then a contiguous eighth of the band tasks
    // (neighbouring tiles share keys in its L2).  Global-row tasks first was
    // measured faster than band tasks first, also where the tasks outnumber
    // the workgroup slots.
    const int xcd = blockIdx.x & 7, slot_in_xcd = blockIdx.x >> 3;
    int task_id;
    {
        const int nb = P.n_band_tasks, ng = P.n_tasks - P.n_band_tasks;
        const int nb_x = (nb >> 3) + (xcd < (nb & 7)), nb_o = xcd * (nb >> 3) + min(xcd, nb & 7);
        const int ng_x = (ng >> 3) + (xcd < (ng & 7)), ng_o = xcd * (ng >> 3) + min(xcd, ng & 7);
        if (slot_in_xcd < ng_x) {
            task_id = nb + ng_o + slot_in_xcd;
        } else if (P.band_chunk > 0) {
            // tiles of unequal cost (one radius per head): runs of C tiles go
            // to the dies in turn, so that every die gets a share of each head
            const int C = P.band_chunk, sb = slot_in_xcd - ng_x;
            const int t = ((sb / C) * 8 + xcd) * C + sb % C;
            if (t >= nb) return;
            task_id = t;
        } else if (slot_in_xcd - ng_x < nb_x) {
            task_id = nb_o + (slot_in_xcd - ng_x);
        } else {
            return;
        }
    }
    const Task tk = decode_task<QB>(P, task_id);
    if constexpr (PAD) {
        // A band tile whose queries are all padded writes zero rows and ends
        // here: a padded query's output is zero whatever its keys.  Every
        // wave tests all of the tile's queries (lane l: query m0 + l), so the
        // decision is the same in each and no barrier is needed.
        if (tk.kind == 0) {
            const int l = threadIdx.x & 63;
            const int mq = tk.m0 + l;
            const int pos = tk.c + tk.delta * mq;
            const uint8_t* prow = A.pad + (size_t)tk.b * P.T;
            const bool live = l < 32 * QB && mq < tk.n && prow[pos] == 0;
            if (__ballot(live) == 0) {
                const int t = threadIdx.x, q = tk.m0 + (t >> 2);
                const int qp = tk.c + tk.delta * q;
                bool global = false;
                for (int g = 0; g < P.n_g; g++) global |= P.glob[g] == qp;
                if ((t >> 2) < 32 * QB && q < tk.n && !global) {
                    OT* orow = (OT*)A.out + (size_t)tk.bh * P.T * D + (size_t)qp * D + 16 * (t & 3);
#pragma unroll
                    for (int i = 0; i < 16 * (int)sizeof(OT) / 16; i++) ((u32x4*)orow)[i] = (u32x4){0u, 0u, 0u, 0u};
                }
                return;
            }
        }
    }

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = uniform(tid >> 6);
    const int qb = wave % QB;
    const int ph = wave / QB;          // key phase of this wave: block ph of every stage
    const int lq = lane & 31;          // query column owned by this lane
    const int lg = lane >> 5;

    const size_t head_off = (size_t)tk.bh * P.T * D;
    const ET* __restrict__ Qg = (const ET*)A.q + head_off;
    const uint8_t* __restrict__ padrow = PAD ? A.pad + (size_t)tk.b * P.T : nullptr;
    // kernel-argument scalars used inside the loop live in registers (a value
    // select between an LDS table entry and a kernel argument would otherwise
    // become a flat load, which waits on every load in flight)
    const int T = P.T, n_g = P.n_g, r = tk.r, ra = tk.ra;
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
        wave_active = mq0 < P.n_g;
        const int sl = mq0 + lq;
        if (sl < P.n_g) my_pos = P.glob[sl];
    }
    const int m_me = mq0 + lq;         // this lane's query (class index / global slot)

    // band blocks this wave's queries can reach
    int wb_lo = 0, wb_hi = -1;
    if (tk.kind == 0) {
        int a = mq0 - r; if (a < 0) a = 0;
        int z = mq0 + 31 + ra; if (z > tk.n - 1) z = tk.n - 1;
        wb_lo = a / KBLK;
        wb_hi = z / KBLK;
    }

    // ---- block list: nb band (or dense) blocks, then the global-key blocks,
    // in sequence positions q; stage s holds positions 2s and 2s+1, and this
    // wave works on position 2s + ph.  Band blocks are visited in a rotated
    // order: position q < nb holds band block j = (q - kb_lo) mod nb (block
    // kb_lo + j of the class), so that the tiles around one another, whose
    // bands are the same class blocks shifted by two, load the same block in
    // the same step: the first step of every tile no longer needs its own
    // K/V from memory at once, and each block's first read is shared.
    const int nb = tk.nband;
    // A band task with at most kVecGlobals globals takes the global keys on
    // the vector units before the band (below): a global-key block would cost
    // a whole step of the loop for one or two keys.  With more globals they
    // follow the band blocks in the ring.
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
            const uint8_t* prow = A.pad + (size_t)tk.b * P.T;
            bool any = false;
            for (int j = tk.kb_lo * KBLK + lane; j < tk.key_end; j += 64) any |= prow[j] == 0;
            dead = __ballot(any) == 0;
        }
    }
    const int NS = dead ? 0 : cdiv(nblk, 2);
    const int rot = tk.kind == 0 ? tk.kb_lo % nb : 0;
    auto band_block = [&](int q) -> int { const int x = q - rot; return x < 0 ? x + nb : x; };
    const int sb_end = (nb - ph + 1) >> 1;       // steps [0, sb_end): band (or dense) blocks
    int j_lo = 0, j_hi = -1;                     // band blocks with keys for this wave's queries
    int ji_lo = 0, ji_hi = -1;                   // band blocks that need no mask
    int sg_end = sb_end;                         // steps [sb_end, sg_end): global-key blocks
    if (wave_active) {
        j_hi = nb - 1;
        if (tk.kind == 0) {
            j_lo = wb_lo - tk.kb_lo;
            j_hi = wb_hi - tk.kb_lo;
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
    // rows (lane p: rows p/4 and 16 + p/4).  Band rows of stage s sit
    // 64*delta positions after those of stage 0.
    const int bw = ph;
    const bool kwave = qb == 0;
    const int rowA = kwave ? (lane >> 1) : (lane >> 2);
    const int rowB = kwave ? rowA : 16 + (lane >> 2);
    const uint32_t colA = kwave ? 16u * ((lane & 1) ^ ((rowA >> 3) & 1)) : 16u * (lane & 3);
    const uint32_t colB = kwave ? colA : 16u * (lane & 3);
    // piece i of this wave's load of a block: LDS offset, scalar byte offset;
    // odd pieces of the V loaders take the second row (voB)
    const char* kvhead = (const char*)(kwave ? kplanes : vplanes) + (size_t)tk.bh * head_bytes;
    int pdst[4], psoff[4];
#pragma unroll
    for (int i = 0; i < 4; i++) {
        pdst[i] = kwave ? i * 1024 : 4096 + (i >> 1) * 2048 + (i & 1) * 1024;
        psoff[i] = kwave ? 32 * i : 64 * (i >> 1);
    }
    // A band block is read through a window that starts at the block's row 0
    // and ends where the head ends, so that the lane offsets (rows delta
    // apart) stay fixed and rows past the end read zeros: scalar work per
    // block, no vector work.
    auto row0_of = [&](int j) -> int { return tk.c + tk.delta * (tk.kb_lo + j) * KBLK; };   // position of row 0
    const uint32_t voA0 = (uint32_t)min((long long)tk.delta * rowA, (long long)T) * ROWB + colA;
    const uint32_t voB0 = (uint32_t)min((long long)tk.delta * rowB, (long long)T) * ROWB + colB;
    auto window = [&](int j) -> __amdgpu_buffer_rsrc_t {
        const int p0 = row0_of(j);
        return buffer_rsrc(kvhead + (uint64_t)p0 * ROWB, p0 < T ? (uint32_t)(T - p0) * ROWB : 0u);
    };
    auto global_pos = [&](int slot) -> uint32_t {   // position a loader lane reads for a global slot
        const int g = gld[min(slot, LF_MAX_GLOBALS - 1)];
        return (uint32_t)(slot < n_g ? g : T);
    };
    // stage s into the ring slot at byte offset off.
    // pm: padded rows of this wave's block of stage s, whose V rows are
    // loaded as zeros (so that NaN or Inf stored at padded positions cannot
    // reach the products); padded global keys load as zeros through their
    // table entry.
    auto issue_stage = [&](int s, int off, uint32_t pm) {
        const bool padA = !kwave && ((pm >> rowA) & 1u), padB = !kwave && ((pm >> rowB) & 1u);
        const int jb = 2 * s + bw;
        if (jb >= nblk) return;
        char* dst = smem + off + bw * RG::BLK;
        auto put = [&](__amdgpu_buffer_rsrc_t rs, uint32_t voA, uint32_t voB) {
#pragma unroll
            for (int p = 0; p < NP; p++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    load_lds16(rs, dst + p * RG::PLANE + pdst[i], (i & 1) ? voB : voA, psoff[i] + 128 * p);
        };
        // two copies of the loads: band offsets stay in their registers
        if (jb < nb) {
            put(window(band_block(jb)), padA ? kPastEnd : voA0, padB ? kPastEnd : voB0);
        } else if (jb >= nb + ngb) {
            const int p0 = rand_p0(jb - nb - ngb);
            put(buffer_rsrc(kvhead + (uint64_t)p0 * ROWB, p0 < T ? (uint32_t)(T - p0) * ROWB : 0u),
                padA ? kPastEnd : voA0, padB ? kPastEnd : voB0);
        } else {
            const int sl0 = (jb - nb) * KBLK;
            put(buffer_rsrc(kvhead, head_bytes), global_pos(sl0 + rowA) * ROWB + colA,
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
        const int q = 2 * s + ph;
        const int pos = q < nb ? row0_of(band_block(q)) + tk.delta * lq
                               : (q >= nb + ngb && q < nblk ? rand_p0(q - nb - ngb) + lq : T);
        return __builtin_amdgcn_raw_buffer_load_b8(rpad, (uint32_t)min(pos, T), 0, 0);
    };
    auto pad_word = [&](uint32_t byte) -> uint32_t { return (uint32_t)__ballot(lane < 32 && byte != 0u); };

    WaveState<NP> W;
    W.o0 = (f32x16){};
    W.o1 = (f32x16){};
    W.ms = kNegInf;
    W.nms = 0.f;
    W.thr = kNegInf;
    W.lp = 0.f;
    W.kbase = ph * RG::BLK + lq * 32 + ((lg ^ ((lq >> 3) & 1)) << 4);
    W.vbase = ph * RG::BLK + (4 * (lane >> 5) + ((lane & 15) >> 2)) * 64 + 32 * ((lane >> 4) & 1) + 8 * (lane & 3);

    // Q rows through a buffer resource: a lane with no query reads past its
    // end and gets zeros, so nothing consumes the loaded registers before the
    // barrier that waits for stage 0 (a padded query keeps its row; the
    // epilogues write zeros for it)
    u32x4 qraw[4 * NP];
    {
        constexpr uint32_t esz = sizeof(ET);
        const __amdgpu_buffer_rsrc_t rq = buffer_rsrc(Qg, (uint32_t)T * D * esz);
        const uint32_t qoff = my_pos >= 0 ? (uint32_t)my_pos * D * esz : kPastEnd;
#pragma unroll
        for (int ks = 0; ks < 4; ks++)
#pragma unroll
            for (int p = 0; p < NP; p++)
                qraw[NP * ks + p] = __builtin_bit_cast(
                    u32x4, __builtin_amdgcn_raw_buffer_load_b128(rq, qoff + (16 * ks + 8 * lg + 4 * p) * esz, 0, 0));
    }
    // the first vector-path global key's K and V rows travel with Q
    const __amdgpu_buffer_rsrc_t rgk = buffer_rsrc((const char*)kplanes + (size_t)tk.bh * head_bytes, head_bytes);
    const __amdgpu_buffer_rsrc_t rgv = buffer_rsrc((const char*)A.v + tk.bh * (size_t)T * D * sizeof(ET),
                                                   (uint32_t)T * D * (uint32_t)sizeof(ET));
    GKey<NP> gk0;
    if (gvec && ph == 0) gk0 = load_gkey<NP>(rgk, rgv, (uint32_t)P.glob[0], lg);
    // ---- prologue: stage 0 and Q in flight, then the global-key tables (a
    // global-key block in stage 0, found only when the band has fewer than
    // two blocks, is loaded once its table is there).  Padded V rows of stage
    // 0 are cleared once it has landed.
    const bool early0 = bw < nb;
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
    barrier_lds_loads();               // Q and stage 0 have landed
    if constexpr (PAD) {
        pm_cur = pad_word(pm_cur);
        // the V loader clears the 16-byte pieces it brought for padded rows
        const bool padA = ((pm_cur >> rowA) & 1u) != 0u, padB = ((pm_cur >> rowB) & 1u) != 0u;
        if (!kwave && early0 && (padA || padB)) {
            char* dst = smem + bw * RG::BLK + 16 * lane;
#pragma unroll
            for (int p = 0; p < NP; p++)
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if ((i & 1) ? padB : padA) *(u32x4*)(dst + p * RG::PLANE + pdst[i]) = (u32x4){0, 0, 0, 0};
        }
        __syncthreads();
    }
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        if constexpr (NP == 1) {
            W.qh[ks] = as_bf16x8(qraw[ks]);
        } else {
            Raw32 x;
            x.a = qraw[2 * ks];
            x.b = qraw[2 * ks + 1];
            u32x4 hi, lo;
            split8(x, hi, lo);
            W.qh[ks] = as_bf16x8(hi);
            W.ql[ks] = as_bf16x8(lo);
        }
    }
    // ---- vector-path global keys: the phase-0 waves (the phases are merged
    // at the end, so one of them takes the keys), every query, each key in
    // turn, unless the key is padded or already in the query's window (its
    // class, class distance in [-r, ra]: the band counts it)
    if (gvec && ph == 0) {
        for (int g = 0; g < n_g; g++) {
            const int pos = P.glob[g];
            const GKey<NP> gk = g == 0 ? gk0 : load_gkey<NP>(rgk, rgv, (uint32_t)pos, lg);
            const float s = halves_sum(gkey_dot<NP>(W, gk));
            const int dpos = pos - tk.c;
            const bool in_class = dpos >= 0 && dpos % tk.delta == 0;
            const int dk = dpos / tk.delta - m_me;
            const bool padded = PAD && padrow[pos] != 0;
            const bool ok = my_pos >= 0 && !padded && !(in_class && dk >= -r && dk <= ra);
            gkey_fold<NP>(W, gk, ok ? s * kScaleLog2 : kNegInf, lg);
        }
    }

    // One step: stage s is in the ring slot at byte offset oc, stage s+1 goes
    // to on.  Every LDS read of a step comes before that step's loads into
    // LDS are issued (the compiler makes any LDS read that follows such a load
    // wait for it); the score MFMAs wait for the K reads, the PV MFMAs for the
    // V reads, and the other waves of the SIMD run meanwhile.
    // (MODE 0: a stage whose blocks are band blocks for both phases, with no
    // global-key or random-block code at all; MODE 1: band or global-key
    // blocks; MODE 2: also random key blocks.)
    // (ANY_GLOBAL false: a stage whose blocks are band blocks for both
    // phases; such steps have no global-key code at all)
    auto step = [&](auto any_global, int s, int oc, int on) {
        constexpr int MODE = decltype(any_global)::value;
        constexpr bool ANY_GLOBAL = MODE > 0;
        barrier_lds_loads();           // stage s landed; stage s-1 no longer read
        const bool band = !ANY_GLOBAL || s < sb_end;
        const int jb = 2 * s + ph;     // sequence position
        const int j = band_block(min(jb, nb - 1));   // its band block (band positions)
        const bool cur = band ? (j >= j_lo && j <= j_hi) : (s < sg_end);
        // The block's bad-row word, wave-uniform so that every test on it is
        // scalar: a global-key block's comes from LDS (read ahead of the
        // fragments), a band block's from its range and the padding ballot.
        uint32_t gword = 0u;
        const bool rnd = MODE == 2 && !band && jb >= nb + ngb;   // a random key block
        if (ANY_GLOBAL && !band && !rnd) gword = gbad[min(max(jb - nb, 0), LF_MAX_GLOBALS / KBLK - 1)];
        const KFrag<NP> kf = load_k<NP>(W, smem + oc);
        const VFrag<NP> vf = load_v<NP>(W, smem + oc);
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
        if (s + 1 < NS) issue_stage(s + 1, on, pm_next);
        f32x16 sc = block_scores<NP>(W, kf);
        // one masking point (the global-key mask reads LDS; it waits for the
        // loads in flight only where the global keys fill two stages or more).
        // A block with no key for this wave's queries is skipped: its LDS may
        // hold anything (zero weights times NaN would still be NaN).
        if (bad != 0xffffffffu) {
            auto mask = [&](f32x16& x) {
                if (MODE == 2 && rnd) {
                    if (p0r + 31 >= mq0 - r && p0r <= mq0 + 31 + ra)   // may meet this wave's windows
                        mask_window_out(x, m_me - r - p0r - 4 * lg, r + ra);
                    if (bad != 0u) mask_bits(x, ~lane_bits(bad, lg));
                } else if (ANY_GLOBAL && !band) {
                    mask_global(x, bad, gcls + (jb - nb) * KBLK, m_me, r, r + ra, lg);
                } else if (!(j >= ji_lo && j <= ji_hi && bad == 0u)) {
                    if (tk.kind == 0) {
                        const int key0 = (tk.kb_lo + j) * KBLK;
                        mask_window(x, m_me - r - key0 - 4 * lg, r + ra);
                    }
                    if (bad != 0u) mask_bits(x, ~lane_bits(bad, lg));
                }
            };
            mask(sc);
            update_max<NP>(W, sc);
            block_pv<NP>(W, sc, vf);
        }
        pm_cur = pm_next;
    };

    // ---- main loop: one barrier per step; the two ring slots alternate.
    // Stages [0, nb/2) hold band blocks only; the rest (at most one mixed
    // stage, then global-key blocks) take the general step.
    using BandOnly = std::integral_constant<int, 0>;
    using General = std::integral_constant<int, 1>;
    using WithRandom = std::integral_constant<int, 2>;
    const int s_band = dead ? 0 : nb >> 1;
    int s = 0;
    for (; s + 1 < s_band; s += 2) {
        step(BandOnly{}, s, 0, RG::STAGE);
        step(BandOnly{}, s + 1, RG::STAGE, 0);
    }
    if (s < s_band) {
        step(BandOnly{}, s, 0, RG::STAGE);
        s++;
    }
    // stages from the first random block on take the step with random blocks
    const int s_rand = nrb > 0 ? (nb + ngb) >> 1 : NS;
    for (; s < min(NS, s_rand); s++) step(General{}, s, (s & 1) * RG::STAGE, ((s + 1) & 1) * RG::STAGE);
    if constexpr (RAND)
        for (; s < NS; s++) step(WithRandom{}, s, (s & 1) * RG::STAGE, ((s + 1) & 1) * RG::STAGE);
    __syncthreads();

    // ---- merge the KS phases of each query block (LDS); phase 0 keeps the result
    if constexpr (KS > 1) {
        float* mbuf = (float*)smem;
        if (ph > 0) {
            f32x4* dst = (f32x4*)(mbuf + (((ph - 1) * QB + qb) * 64 + lane) * 36);
#pragma unroll
            for (int i = 0; i < 4; i++) {
                dst[i] = (f32x4){W.o0[4 * i], W.o0[4 * i + 1], W.o0[4 * i + 2], W.o0[4 * i + 3]};
                dst[4 + i] = (f32x4){W.o1[4 * i], W.o1[4 * i + 1], W.o1[4 * i + 2], W.o1[4 * i + 3]};
            }
            dst[8] = (f32x4){W.ms, W.lp, 0.f, 0.f};
        }
        __syncthreads();
        if (ph == 0) {
#pragma unroll
            for (int p2 = 1; p2 < KS; p2++) {
                const f32x4* src = (const f32x4*)(mbuf + (((p2 - 1) * QB + qb) * 64 + lane) * 36);
                const f32x4 tail = src[8];
                const float ms2 = tail[0], lp2 = tail[1];
                const float mn = __builtin_fmaxf(W.ms, ms2);
                const float a1 = (W.ms == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(W.ms - mn);
                const float a2 = (ms2 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ms2 - mn);
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const f32x4 x0 = src[i], x1 = src[4 + i];
#pragma unroll
                    for (int e = 0; e < 4; e++) {
                        W.o0[4 * i + e] = W.o0[4 * i + e] * a1 + x0[e] * a2;
                        W.o1[4 * i + e] = W.o1[4 * i + e] * a1 + x1[e] * a2;
                    }
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
        if (gvec) {
            for (int g = 0; g < n_g; g++)
                if (P.glob[g] == my_pos) return;
        } else if (P.n_g > 0) {
            int lo = 0, hi = P.n_g - 1;
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
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            const f32x16& oc = cb ? W.o1 : W.o0;
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
    // 272-byte record [O[0..63], m, l, 0, 0].  Partials cross dies (each XCD
    // has its own L2), so they are written and read with the agent-coherent
    // cache policy (sc1) instead of fences, which would write back and
    // invalidate whole L2s.
    const uint32_t stride = (uint32_t)P.g_pad * kRecBytes;          // bytes between splits of a slot
    const __amdgpu_buffer_rsrc_t rpart =
        buffer_rsrc((const char*)P.part + (size_t)tk.bh * P.n_split * stride, (uint32_t)P.n_split * stride);
    const int slot = mq0 + lq;
    if (writer && slot < n_g) {
        const uint32_t rec = (uint32_t)tk.split * stride + (uint32_t)slot * kRecBytes;
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            const f32x16& oc = cb ? W.o1 : W.o0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const f32x4 o4 = {oc[4 * j], oc[4 * j + 1], oc[4 * j + 2], oc[4 * j + 3]};
                __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o4), rpart,
                                                       rec + 4 * (32 * cb + 8 * j + 4 * lg), 0, kCoherent);
            }
        }
        if (lg == 0)
            __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, (f32x2){W.ms, l}), rpart, rec + 256, 0,
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
    for (int task = tid; task < n_g * 16; task += NT) {
        const int gi = task >> 4, c4 = task & 15;
        float M = kNegInf, L = 0.f;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int sp0 = 0; sp0 < P.n_split; sp0 += 8) {
            f32x2 ml[8];
            f32x4 o[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t rec = (uint32_t)min(sp0 + i, P.n_split - 1) * stride + (uint32_t)gi * kRecBytes;
                ml[i] = __builtin_bit_cast(f32x2, __builtin_amdgcn_raw_buffer_load_b64(rpart, rec + 256, 0, kCoherent));
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
        if (padded || !(L > 0.f)) acc = (f32x4){0.f, 0.f, 0.f, 0.f};   // zeros even if the partials hold NaN
        const float inv = (padded || !(L > 0.f)) ? 0.f : 1.0f / L;
        OT* orow = (OT*)A.out + head_off + (size_t)pos * D + 4 * c4;
        if constexpr (sizeof(OT) == 2) {
            *(u32x2*)orow = (u32x2){pack_bf16(acc[0] * inv, acc[1] * inv), pack_bf16(acc[2] * inv, acc[3] * inv)};
        } else {
            *(f32x4*)orow = (f32x4){acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
        }
    }
    if (tid == 0) __hip_atomic_store(P.counter + tk.bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// fp32 K and V -> bf16 hi/lo planes [rows][2][64] (hi = RNE(x), lo = RNE(x - hi)),
// one thread per 8 channels of a row; blockIdx.y picks K or V
__global__ __launch_bounds__(256) void split_planes_kernel(const float* __restrict__ k, const float* __restrict__ v,
                                                           uint16_t* __restrict__ kp, uint16_t* __restrict__ vp,
                                                           long long chunks) {
    const long long i = (long long)blockIdx.x * 256 + threadIdx.x;
    if (i >= chunks) return;
    const float* src = blockIdx.y ? v : k;
    uint16_t* dst = blockIdx.y ? vp : kp;
    const long long row = i >> 3;
    const int ch = (int)(i & 7);
    Raw32 x;
    x.a = *(const u32x4*)(src + row * D + ch * 8);
    x.b = *(const u32x4*)(src + row * D + ch * 8 + 4);
    u32x4 hi, lo;
    split8(x, hi, lo);
    *(u32x4*)(dst + row * 2 * D + ch * 8) = hi;
    *(u32x4*)(dst + row * 2 * D + D + ch * 8) = lo;
}

}  // namespace lfk

// ---------------------------------------------------------------------------
// launchers (called from the host library)

// grid: the task slots of the 8 dies, each die holding ceil(n/8) band and
// ceil(n/8) global-row slots
extern "C" int lfk_grid(const lfk::Plan* P) {
    const int nb = P->n_band_tasks, ng = P->n_tasks - P->n_band_tasks;
    const int C = P->band_chunk;
    const int band_slots = C > 0 ? ((nb + C - 1) / C + 7) / 8 * C : (nb + 7) / 8;
    return 8 * (band_slots + (ng + 7) / 8);
}

// A: kernel argument (A->plan is the device copy of *P); P: host copy of the plan
// one instantiation per input type, padding and random blocks (each present
// or not at compile time)
template <typename ET, typename OT>
static void launch_tiles(const lfk::Args* A, const lfk::Plan* P, hipStream_t s) {
    constexpr int QB = LFK_QB, KS = LFK_KS;
    const int grid = lfk_grid(P);
    const bool pad = A->pad != nullptr, rnd = P->n_rand > 0;
    const dim3 g(grid), b(64 * QB * KS);
    if (pad && rnd) hipLaunchKernelGGL((lfk::tile_kernel<QB, KS, ET, OT, true, true>), g, b, 0, s, *A);
    else if (pad) hipLaunchKernelGGL((lfk::tile_kernel<QB, KS, ET, OT, true, false>), g, b, 0, s, *A);
    else if (rnd) hipLaunchKernelGGL((lfk::tile_kernel<QB, KS, ET, OT, false, true>), g, b, 0, s, *A);
    else hipLaunchKernelGGL((lfk::tile_kernel<QB, KS, ET, OT, false, false>), g, b, 0, s, *A);
}

extern "C" hipError_t lfk_launch(const lfk::Args* A, const lfk::Plan* P, int dtype_bf16, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (dtype_bf16) {
        launch_tiles<__bf16, uint16_t>(A, P, s);
    } else {
        const long long chunks = (long long)P->B * P->H * P->T * 8;
        hipLaunchKernelGGL(lfk::split_planes_kernel, dim3((unsigned)((chunks + 255) / 256), 2), dim3(256), 0, s,
                           (const float*)A->k, (const float*)A->v, (uint16_t*)P->kp, (uint16_t*)P->vp, chunks);
        launch_tiles<float, float>(A, P, s);
    }
    return hipGetLastError();
}
