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
        const int q = P.T / delta, rem = P.T - q * delta;
        const int tb = cdiv(q + 1, BM), ts = cdiv(q, BM);
        int c, tile;
        if (x < rem * tb) { c = x / tb; tile = x - c * tb; }
        else { const int y = x - rem * tb; c = rem + y / ts; tile = y - (c - rem) * ts; }
        k.delta = delta;
        k.c = c;
        k.n = (P.T - c + delta - 1) / delta;
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

template <int MODE, int KS, int NP>
__device__ __forceinline__ void attend_block(WaveState<NP>& W, const char* buf, int blk, int key0, int m,
                                             int r, int lane) {
    using SG = Stage<KS, NP>;
    const int lq = lane & 31, lg = lane >> 5;
    // S^T = K Q^T for this block: 32 keys x 32 queries
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
        const uint32_t bad = *(const uint32_t*)(buf + SG::maskOff + blk * 4);
        const int* gcls = (const int*)(buf + SG::gclsOff) + blk * KBLK;
#pragma unroll
        for (int i = 0; i < 16; i++) {
            const int kl = 8 * (i >> 2) + 4 * lg + (i & 3);   // key row inside the block
            bool ok = ((bad >> kl) & 1u) == 0u;
            if constexpr (MODE == kBandEdge) {
                const int dk = key0 + kl - m;
                ok = ok && (uint32_t)(dk + r) <= (uint32_t)(2 * r);
            } else if constexpr (MODE == kGlobalKeys) {
                const int dk = gcls[kl] - m;
                ok = ok && (uint32_t)(dk + r) > (uint32_t)(2 * r);   // not already in the window
            }
            s[i] = ok ? s[i] : kNegInf;
        }
    }
    // running max: raw-score max of the block, scaled; O is rescaled only when
    // the max grows by more than 2^8 (then every later p stays <= 2^8)
    float mx = s[0];
#pragma unroll
    for (int i = 1; i < 16; i++) mx = __builtin_fmaxf(mx, s[i]);
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
    // O^T += V^T P^T; V^T operands by transposing reads: lane (16G + L) supplies
    // row 16st + 8hf + 4(G>>1) + (L>>2), channels 32cb + 16(G&1) + 4(L&3)
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

// ---------------------------------------------------------------------------
// The tile kernel.

template <int QB, int KS, typename ET, typename OT>
__global__ __launch_bounds__(64 * QB * KS) __attribute__((amdgpu_waves_per_eu(LFK_WAVES_PER_EU))) void tile_kernel(const Params P) {
    constexpr int NT = 64 * QB * KS;
    constexpr int NP = Elem<ET>::NP;
    using SG = Stage<KS, NP>;
    constexpr int R = KS * KBLK;               // key rows per stage
    constexpr int CHUNKS = R * 8;              // 8-channel chunks per tensor per stage
    static_assert(CHUNKS % NT == 0, "stage chunks must divide evenly over the workgroup");
    constexpr int CPT = CHUNKS / NT;           // chunks per thread per tensor
    constexpr int MERGE_BYTES = (KS - 1) * QB * 64 * 36 * 4;
    constexpr int SMEM = (2 * SG::bytes > MERGE_BYTES) ? 2 * SG::bytes : MERGE_BYTES;
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
    const int NSb = cdiv(tk.nband, KS);
    const int NS = NSb + cdiv(ngb, KS);

    // loader geometry: chunk j of this thread is row (tid >> 3) + j * NT/8, channels 8*(tid & 7)..+7
    const int lch = tid & 7;
    const int lrow0 = tid >> 3;
    const int key_base = tk.kb_lo * KBLK;

    struct Regs {
        u32x4 k[CPT][NP];
        u32x4 v[CPT][NP];
        bool ok[CPT];
        uint32_t mword;   // mask lanes: this lane's row validity is folded in at commit
        bool mvalid;
        int gcls;
    };

    // position of stage row `row` of stage `st` (and whether it is a real key)
    auto row_pos = [&](int st, int row, int& pos, bool& inr) {
        if (st < NSb) {
            const int kk = key_base + st * R + row;
            inr = kk < tk.key_end;
            pos = inr ? tk.c + tk.delta * kk : 0;
        } else {
            const int slot = (st - NSb) * R + row;
            inr = slot < P.n_g;
            pos = inr ? P.glob[slot] : 0;
        }
    };

    auto issue = [&](int st, Regs& Rg) {
#pragma unroll
        for (int j = 0; j < CPT; j++) {
            int pos; bool inr;
            row_pos(st, lrow0 + j * (NT / 8), pos, inr);
            const size_t off = (size_t)pos * D + lch * 8;
#pragma unroll
            for (int p = 0; p < NP; p++) {
                Rg.k[j][p] = *(const u32x4*)(Kg + off + 4 * p);
                Rg.v[j][p] = *(const u32x4*)(Vg + off + 4 * p);
            }
            bool ok = inr;
            if (padrow) ok = ok && padrow[pos] == 0;
            Rg.ok[j] = ok;
        }
        // mask lanes: waves 0..KS-1, lanes 0..31 own stage row 32*wave + lane
        if (wave < KS) {
            int pos; bool inr;
            row_pos(st, 32 * wave + lq, pos, inr);
            bool ok = inr && lg == 0;
            if (padrow) ok = ok && padrow[pos] == 0;
            Rg.mvalid = ok;
            Rg.gcls = kNotInClass;
            if (st >= NSb && inr) {
                const int dpos = pos - tk.c;
                if (dpos >= 0 && dpos % tk.delta == 0) Rg.gcls = dpos / tk.delta;
            }
        }
    };

    auto commit = [&](const Regs& Rg, char* buf) {
        const u32x4 z = {0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < CPT; j++) {
            const int row = lrow0 + j * (NT / 8);
            const int blk = row >> 5, t = row & 31;
            if constexpr (NP == 1) {
                *(u32x4*)(buf + SG::kOff(0, blk) + swzK(t, lch)) = Rg.ok[j] ? Rg.k[j][0] : z;
                *(u32x4*)(buf + SG::vOff(0, blk) + swzV(t, lch)) = Rg.ok[j] ? Rg.v[j][0] : z;
            } else {
                u32x4 kh = z, kl = z, vh = z, vl = z;
                if (Rg.ok[j]) {
                    split8(Raw32{Rg.k[j][0], Rg.k[j][1]}, kh, kl);
                    split8(Raw32{Rg.v[j][0], Rg.v[j][1]}, vh, vl);
                }
                *(u32x4*)(buf + SG::kOff(0, blk) + swzK(t, lch)) = kh;
                *(u32x4*)(buf + SG::kOff(1, blk) + swzK(t, lch)) = kl;
                *(u32x4*)(buf + SG::vOff(0, blk) + swzV(t, lch)) = vh;
                *(u32x4*)(buf + SG::vOff(1, blk) + swzV(t, lch)) = vl;
            }
        }
        if (wave < KS) {
            const uint32_t good = (uint32_t)__ballot(Rg.mvalid);   // lanes 0..31 only
            if (lane == 0) *(uint32_t*)(buf + SG::maskOff + wave * 4) = ~good;
            if (lg == 0) ((int*)(buf + SG::gclsOff))[wave * KBLK + lq] = Rg.gcls;
        }
    };

    // ---- main loop over stages, double-buffered through LDS
    char* const buf0 = smem;
    char* const buf1 = smem + SG::bytes;
    {
        Regs Rg;
        issue(0, Rg);
        commit(Rg, buf0);
        __syncthreads();
    }
    const int m_me = mq0 + lq;         // this lane's query (class index / global slot)
    for (int st = 0; st < NS; st++) {
        Regs Rg;
        const bool more = st + 1 < NS;
        if (more) issue(st + 1, Rg);
        const char* cur = (st & 1) ? buf1 : buf0;
        if (wave_active) {
            if (st < NSb) {
                const int jb = st * KS + ph;
                if (jb < tk.nband) {
                    const uint32_t bad = *(const uint32_t*)(cur + SG::maskOff + ph * 4);
                    const int kb = tk.kb_lo + jb;
                    const int key0 = kb * KBLK;
                    if (bad != 0xffffffffu) {
                        if (tk.kind == 1) {
                            attend_block<kDense, KS, NP>(W, cur, ph, key0, m_me, r, lane);
                        } else if (kb >= wb_lo && kb <= wb_hi) {
                            const bool interior = bad == 0u && key0 >= mq0 + 31 - r && key0 + 31 <= mq0 + r;
                            if (interior) attend_block<kInterior, KS, NP>(W, cur, ph, key0, m_me, r, lane);
                            else attend_block<kBandEdge, KS, NP>(W, cur, ph, key0, m_me, r, lane);
                        }
                    }
                }
            } else {
                const int jg = (st - NSb) * KS + ph;
                if (jg < ngb) {
                    const uint32_t bad = *(const uint32_t*)(cur + SG::maskOff + ph * 4);
                    if (bad != 0xffffffffu) attend_block<kGlobalKeys, KS, NP>(W, cur, ph, 0, m_me, r, lane);
                }
            }
        }
        if (more) commit(Rg, (st & 1) ? buf0 : buf1);
        __syncthreads();
    }

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
