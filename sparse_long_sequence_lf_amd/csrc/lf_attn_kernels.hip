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
    int delta, c;    // residue class (band); delta = 1, c = 0 for global tasks
    int n;           // class length (band) / T (global)
    int m0;          // first query (class index) of the tile / first G-block slot
    int nband;       // band blocks
    int kb_lo;       // first band block (class block index)
    int nblk;        // total blocks incl. global blocks
    int key_end;     // keys >= key_end are out of range (class index)
    int split;       // global tasks: split index
};

__device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }

template <int QB>
__device__ Task decode_task(const Params& P, int t) {
    constexpr int BM = 32 * QB;
    Task k;
    if (t < P.n_band_tasks) {
        k.kind = 0;
        k.b = t / P.band_tasks_per_batch;
        int x = t - k.b * P.band_tasks_per_batch;
        int h = 0;
        // heads are few (<= LF_MAX_HEADS); binary search on the prefix
        int lo = 0, hi = P.H - 1;
        while (lo < hi) {
            int mid = (lo + hi + 1) >> 1;
            if (P.head_start[mid] <= x) lo = mid; else hi = mid - 1;
        }
        h = lo;
        x -= P.head_start[h];
        k.h = h;
        k.bh = k.b * P.H + h;
        int delta = P.dil[h];
        int q = P.T / delta, rem = P.T % delta;
        int tb = cdiv(q + 1, BM), ts = cdiv(q, BM);
        int c, tile;
        if (x < rem * tb) { c = x / tb; tile = x - c * tb; }
        else { int y = x - rem * tb; c = rem + y / ts; tile = y - (c - rem) * ts; }
        k.delta = delta;
        k.c = c;
        k.n = (P.T - c + delta - 1) / delta;
        k.m0 = tile * BM;
        int r = P.r;
        int lo_k = k.m0 - r; if (lo_k < 0) lo_k = 0;
        int hi_k = k.m0 + BM - 1 + r; if (hi_k > k.n - 1) hi_k = k.n - 1;
        k.kb_lo = lo_k / KBLK;
        k.nband = hi_k / KBLK - k.kb_lo + 1;
        k.nblk = k.nband + cdiv(P.n_g, KBLK);
        k.key_end = k.n;
        k.split = 0;
    } else {
        k.kind = 1;
        int g = t - P.n_band_tasks;
        int per_bh = P.n_split * P.n_ggroups;
        k.bh = g / per_bh;
        int rem = g - k.bh * per_bh;
        int grp = rem / P.n_split;
        k.split = rem - grp * P.n_split;
        k.b = k.bh / P.H;
        k.h = k.bh - k.b * P.H;
        k.delta = 1;
        k.c = 0;
        k.n = P.T;
        k.m0 = grp * BM;  // first global slot of this group
        int j0 = k.split * P.split_len;
        int j1 = j0 + P.split_len; if (j1 > P.T) j1 = P.T;
        k.kb_lo = j0 / KBLK;
        k.nband = cdiv(j1 - j0, KBLK);
        k.nblk = k.nband;
        k.key_end = j1;
    }
    return k;
}

// ---------------------------------------------------------------------------
// The tile kernel.

template <int QB, int KS, typename ET, typename OT>
__global__ __launch_bounds__(64 * QB * KS) void tile_kernel(const Params P) {
    constexpr int NT = 64 * QB * KS;
    constexpr int NP = Elem<ET>::NP;
    using SG = Stage<KS, NP>;
    constexpr int CHUNKS = KS * KBLK * 8;              // 16-byte (8-channel) chunks per tensor per stage
    constexpr int CPT = (CHUNKS + NT - 1) / NT;         // chunks per thread
    constexpr int MERGE_BYTES = (KS - 1) * QB * 64 * 36 * 4;
    constexpr int SMEM = (2 * SG::bytes > MERGE_BYTES) ? 2 * SG::bytes : MERGE_BYTES;
    __shared__ __attribute__((aligned(16))) char smem[SMEM];

    // ---- which task (XCD-aware: the 8 dies take contiguous task ranges)
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
    const int lg = lane >> 5;          // which half of the keys of a tile column

    const size_t head_off = (size_t)tk.bh * P.T * D;
    const ET* __restrict__ Kg = (const ET*)P.k + head_off;
    const ET* __restrict__ Vg = (const ET*)P.v + head_off;
    const ET* __restrict__ Qg = (const ET*)P.q + head_off;
    const uint8_t* __restrict__ padrow = P.pad ? P.pad + (size_t)tk.b * P.T : nullptr;
    const int r = P.r;

    // ---- this wave's queries
    const int mq0 = tk.m0 + 32 * qb;   // first query (class index or global slot)
    bool wave_active;
    int my_pos = -1;                   // position of this lane's query
    if (tk.kind == 0) {
        wave_active = mq0 < tk.n;
        int m = mq0 + lq;
        if (m < tk.n) my_pos = tk.c + tk.delta * m;
    } else {
        wave_active = mq0 < P.n_g;
        int s = mq0 + lq;
        if (s < P.n_g) my_pos = P.glob[s];
    }
    bool my_pad = (my_pos >= 0 && padrow) ? padrow[my_pos] != 0 : false;

    // Q^T fragments: lane (query lq, half lg) holds channels 16*ks + 8*lg .. +7
    bf16x8 qh[4], ql[4];
    {
        const bool ok = my_pos >= 0 && !my_pad;
        const ET* qrow = Qg + (size_t)(ok ? my_pos : 0) * D;
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const int c0 = 16 * ks + 8 * lg;
            if constexpr (NP == 1) {
                u32x4 x = ok ? *(const u32x4*)(qrow + c0) : (u32x4){0, 0, 0, 0};
                qh[ks] = as_bf16x8(x);
                ql[ks] = as_bf16x8((u32x4){0, 0, 0, 0});
            } else {
                Raw32 x;
                if (ok) { x.a = *(const u32x4*)(qrow + c0); x.b = *(const u32x4*)(qrow + c0 + 4); }
                else { x.a = (u32x4){0, 0, 0, 0}; x.b = x.a; }
                u32x4 hi, lo;
                split8(x, hi, lo);
                qh[ks] = as_bf16x8(hi);
                ql[ks] = as_bf16x8(lo);
            }
        }
    }

    // wave's own window, in band blocks (class block indices)
    int wb_lo = 0, wb_hi = -1;
    if (tk.kind == 0) {
        int a = mq0 - r; if (a < 0) a = 0;
        int z = mq0 + 31 + r; if (z > tk.n - 1) z = tk.n - 1;
        wb_lo = a / KBLK;
        wb_hi = z / KBLK;
    }

    // ---- running state
    f32x16 o0 = {}, o1 = {};
    float ms = kNegInf;  // running max, already in scaled base-2 units
    float lp = 0.f;      // this lane's part of the row sum

    const int NS = (tk.nblk + KS - 1) / KS;

    // ---- stage loader (global -> registers -> LDS)
    struct Regs {
        u32x4 k[CPT][NP == 1 ? 1 : 2];
        u32x4 v[CPT][NP == 1 ? 1 : 2];
        int pos[CPT];
        bool inr[CPT];
    };

    auto row_of = [&](int stage, int idx, int& pos, bool& inr, int& gcls) {
        const int blk = idx >> 8;
        const int t = (idx >> 3) & 31;
        const int jb = stage * KS + blk;
        pos = 0; inr = false; gcls = kNotInClass;
        if (jb >= tk.nblk) return;
        if (jb < tk.nband) {
            const int kk = (tk.kb_lo + jb) * KBLK + t;
            if (kk < tk.key_end) { inr = true; pos = tk.c + tk.delta * kk; }
        } else {
            const int s = (jb - tk.nband) * KBLK + t;
            if (s < P.n_g) {
                inr = true;
                pos = P.glob[s];
                const int dpos = pos - tk.c;
                if (dpos >= 0 && dpos % tk.delta == 0) gcls = dpos / tk.delta;
            }
        }
    };

    auto issue = [&](int stage, Regs& R) {
#pragma unroll
        for (int j = 0; j < CPT; j++) {
            const int idx = tid + j * NT;
            R.inr[j] = false;
            R.pos[j] = 0;
            if (idx < CHUNKS) {
                int pos, gcls; bool inr;
                row_of(stage, idx, pos, inr, gcls);
                R.inr[j] = inr;
                R.pos[j] = pos;
                const int ch = idx & 7;
                if (inr) {
                    const ET* kp = Kg + (size_t)pos * D + ch * 8;
                    const ET* vp = Vg + (size_t)pos * D + ch * 8;
                    R.k[j][0] = *(const u32x4*)kp;
                    R.v[j][0] = *(const u32x4*)vp;
                    if constexpr (NP == 2) {
                        R.k[j][1] = *(const u32x4*)(kp + 4);
                        R.v[j][1] = *(const u32x4*)(vp + 4);
                    }
                }
            }
        }
    };

    auto commit = [&](int stage, const Regs& R, char* buf) {
#pragma unroll
        for (int j = 0; j < CPT; j++) {
            const int idx = tid + j * NT;
            if (idx < CHUNKS) {  // wave-uniform: NT is a multiple of 64
                const int blk = idx >> 8;
                const int t = (idx >> 3) & 31;
                const int ch = idx & 7;
                bool valid = R.inr[j];
                if (valid && padrow) valid = padrow[R.pos[j]] == 0;
                u32x4 z = {0, 0, 0, 0};
                if constexpr (NP == 1) {
                    *(u32x4*)(buf + SG::kOff(0, blk) + swzK(t, ch)) = valid ? R.k[j][0] : z;
                    *(u32x4*)(buf + SG::vOff(0, blk) + swzV(t, ch)) = valid ? R.v[j][0] : z;
                } else {
                    u32x4 kh = z, kl = z, vh = z, vl = z;
                    if (valid) {
                        Raw32 rk{R.k[j][0], R.k[j][1]}, rv{R.v[j][0], R.v[j][1]};
                        split8(rk, kh, kl);
                        split8(rv, vh, vl);
                    }
                    *(u32x4*)(buf + SG::kOff(0, blk) + swzK(t, ch)) = kh;
                    *(u32x4*)(buf + SG::kOff(1, blk) + swzK(t, ch)) = kl;
                    *(u32x4*)(buf + SG::vOff(0, blk) + swzV(t, ch)) = vh;
                    *(u32x4*)(buf + SG::vOff(1, blk) + swzV(t, ch)) = vl;
                }
                // one mask bit per row: lanes 8u .. 8u+7 of a wave cover row u
                uint64_t bad = __ballot(!valid);
                if (lane == 0) {
                    uint64_t m8 = bad & 0x0101010101010101ull;
                    uint32_t bits = (uint32_t)((m8 * 0x0102040810204080ull) >> 56);
                    // bit u of the byte = row u of this wave's 8 rows
                    ((uint8_t*)(buf + SG::maskOff))[blk * 4 + (t >> 3)] = (uint8_t)bits;
                }
                if (ch == 0) {
                    int pos, gcls; bool inr;
                    row_of(stage, idx, pos, inr, gcls);
                    ((int*)(buf + SG::gclsOff))[blk * KBLK + t] = gcls;
                }
            }
        }
    };

    // ---- one block of 32 keys against this wave's 32 queries
    auto compute = [&](const char* buf, int blk, int mode, int key0) {
        // mode 0: interior band block (no masking)   1: masked band block
        //      2: global-key block                    3: dense block (global rows)
        const uint32_t mword = *(const uint32_t*)(buf + SG::maskOff + blk * 4);
        f32x16 s = {};
        const char* kb = buf + SG::kOff(0, blk);
#pragma unroll
        for (int ks = 0; ks < 4; ks++) {
            const bf16x8 kf = as_bf16x8(*(const u32x4*)(kb + swzK(lq, 2 * ks + lg)));
            s = mfma(kf, qh[ks], s);
            if constexpr (NP == 2) {
                const bf16x8 kfl = as_bf16x8(*(const u32x4*)(buf + SG::kOff(1, blk) + swzK(lq, 2 * ks + lg)));
                s = mfma(kf, ql[ks], s);
                s = mfma(kfl, qh[ks], s);
            }
        }
        if (mode != 0) {
            const int m = mq0 + lq;
            const int* gcls = (const int*)(buf + SG::gclsOff) + blk * KBLK;
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const int kl = 8 * (i >> 2) + 4 * lg + (i & 3);   // key row inside the block
                bool ok = ((mword >> kl) & 1u) == 0u;
                if (mode == 1) {
                    const int dk = key0 + kl - m;
                    ok = ok && dk <= r && dk >= -r;
                } else if (mode == 2) {
                    const int dk = gcls[kl] - m;
                    ok = ok && !(dk <= r && dk >= -r);   // already counted in the window
                }
                s[i] = ok ? s[i] : kNegInf;
            }
        }
        // row max over this block: 16 keys here, 16 in lane ^ 32
        float mx = s[0];
#pragma unroll
        for (int i = 1; i < 16; i++) mx = __builtin_fmaxf(mx, s[i]);
        mx = __builtin_fmaxf(mx, wave_xor32(mx));
        const float mxs = mx * kScaleLog2;
        const bool need = mxs > ms + 8.0f;
        if (__ballot(need)) {
            const float msn = need ? mxs : ms;
            const float alpha = need ? __builtin_amdgcn_exp2f(ms - msn) : 1.0f;
#pragma unroll
            for (int i = 0; i < 16; i++) { o0[i] *= alpha; o1[i] *= alpha; }
            lp *= alpha;
            ms = msn;
        }
        const float nms = (ms == kNegInf) ? 0.0f : -ms;
        float p[16];
#pragma unroll
        for (int i = 0; i < 16; i++) p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[i], kScaleLog2, nms));
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 16; i++) ps += p[i];
        lp += ps;
        // P^T operands: step st covers accumulator elements 8st .. 8st+7
        bf16x8 pb[2], pbl[2];
#pragma unroll
        for (int st = 0; st < 2; st++) {
            u32x4 w, wl;
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const float a = p[8 * st + 2 * e], b = p[8 * st + 2 * e + 1];
                w[e] = pack_bf16(a, b);
                if constexpr (NP == 2) {
                    const uint32_t hw = w[e];
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
#pragma unroll
        for (int st = 0; st < 2; st++) {
#pragma unroll
            for (int cb = 0; cb < 2; cb++) {
                const int t0 = 16 * st + 4 * (G >> 1) + (L >> 2);
                const int byte = 64 * cb + 32 * (G & 1) + 8 * (L & 3);
                const int ch = byte >> 4, inner = byte & 15;
                const char* vb = buf + SG::vOff(0, blk);
                const bf16x8 va = cat_tr(ds_tr16(vb + swzV(t0, ch) + inner), ds_tr16(vb + swzV(t0 + 8, ch) + inner));
                f32x16& oc = cb ? o1 : o0;
                oc = mfma(va, pb[st], oc);
                if constexpr (NP == 2) {
                    const char* vbl = buf + SG::vOff(1, blk);
                    const bf16x8 val = cat_tr(ds_tr16(vbl + swzV(t0, ch) + inner), ds_tr16(vbl + swzV(t0 + 8, ch) + inner));
                    oc = mfma(va, pbl[st], oc);
                    oc = mfma(val, pb[st], oc);
                }
            }
        }
    };

    // ---- main loop over stages, double-buffered
    char* buf0 = smem;
    char* buf1 = smem + SG::bytes;
    {
        Regs R;
        issue(0, R);
        commit(0, R, buf0);
        __syncthreads();
    }
    for (int st = 0; st < NS; st++) {
        Regs R;
        const bool more = st + 1 < NS;
        if (more) issue(st + 1, R);
        const char* cur = (st & 1) ? buf1 : buf0;
        const int jb = st * KS + ph;
        if (wave_active && jb < tk.nblk) {
            if (tk.kind == 1) {
                compute(cur, ph, 3, 0);
            } else if (jb < tk.nband) {
                const int kb = tk.kb_lo + jb;
                if (kb >= wb_lo && kb <= wb_hi) {
                    const int key0 = kb * KBLK;
                    const uint32_t mword = *(const uint32_t*)(cur + SG::maskOff + ph * 4);
                    const bool interior = mword == 0u && key0 >= mq0 + 31 - r && key0 + 31 <= mq0 + r;
                    if (mword != 0xffffffffu) compute(cur, ph, interior ? 0 : 1, key0);
                }
            } else {
                const uint32_t mword = *(const uint32_t*)(cur + SG::maskOff + ph * 4);
                if (mword != 0xffffffffu) compute(cur, ph, 2, 0);
            }
        }
        if (more) commit(st + 1, R, (st & 1) ? buf0 : buf1);
        __syncthreads();
    }

    // ---- merge the KS phases of each query block (LDS), phase 0 keeps the result
    if constexpr (KS > 1) {
        float* mbuf = (float*)smem;
        if (ph > 0) {
            float* dst = mbuf + (((ph - 1) * QB + qb) * 64 + lane) * 36;
            dst[0] = ms;
            dst[1] = lp;
#pragma unroll
            for (int i = 0; i < 16; i++) { dst[2 + i] = o0[i]; dst[18 + i] = o1[i]; }
        }
        __syncthreads();
        if (ph == 0) {
#pragma unroll
            for (int p2 = 1; p2 < KS; p2++) {
                const float* src = mbuf + (((p2 - 1) * QB + qb) * 64 + lane) * 36;
                const float ms2 = src[0], lp2 = src[1];
                const float mn = __builtin_fmaxf(ms, ms2);
                const float a1 = (ms == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ms - mn);
                const float a2 = (ms2 == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(ms2 - mn);
#pragma unroll
                for (int i = 0; i < 16; i++) {
                    o0[i] = o0[i] * a1 + src[2 + i] * a2;
                    o1[i] = o1[i] * a1 + src[18 + i] * a2;
                }
                lp = lp * a1 + lp2 * a2;
                ms = mn;
            }
        }
    }
    if (ph != 0 || !wave_active) return;

    const float l = lp + wave_xor32(lp);

    if (tk.kind == 0) {
        // ---- epilogue: y = O / l for the tile's valid queries; padded rows -> 0
        if (my_pos < 0) return;
        OT* orow = (OT*)P.out + head_off + (size_t)my_pos * D;
        const float inv = (my_pad || l == 0.f) ? 0.f : 1.0f / l;
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            const f32x16& oc = cb ? o1 : o0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int c0 = 32 * cb + 8 * j + 4 * lg;
                const float y0 = oc[4 * j + 0] * inv, y1 = oc[4 * j + 1] * inv;
                const float y2 = oc[4 * j + 2] * inv, y3 = oc[4 * j + 3] * inv;
                if constexpr (sizeof(OT) == 2) {
                    u32x2 w = {pack_bf16(y0, y1), pack_bf16(y2, y3)};
                    *(u32x2*)(orow + c0) = w;
                } else {
                    f32x4 w = {y0, y1, y2, y3};
                    *(f32x4*)(orow + c0) = w;
                }
            }
        }
    } else {
        // ---- global rows: write this split's (max, sum, O) for each global slot
        const int slot = mq0 + lq;
        if (slot >= P.n_g) return;
        float* part = P.part + (((size_t)tk.bh * P.n_split + tk.split) * P.g_pad + slot) * (D + 2);
        if (lg == 0) { part[0] = ms; part[1] = l; }
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            const f32x16& oc = cb ? o1 : o0;
#pragma unroll
            for (int j = 0; j < 4; j++) {
                const int c0 = 32 * cb + 8 * j + 4 * lg;
                part[2 + c0 + 0] = oc[4 * j + 0];
                part[2 + c0 + 1] = oc[4 * j + 1];
                part[2 + c0 + 2] = oc[4 * j + 2];
                part[2 + c0 + 3] = oc[4 * j + 3];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Combine the split partials of each global row (rescale to a common max,
// add, divide) and write the row.  One 64-lane workgroup per (b, h, global).

template <typename OT>
__global__ __launch_bounds__(64) void combine_kernel(const Params P) {
    const int gi = blockIdx.x % P.n_g;
    const int bh = blockIdx.x / P.n_g;
    const int b = bh / P.H;
    const int c = threadIdx.x;
    const int pos = P.glob[gi];
    OT* orow = (OT*)P.out + ((size_t)bh * P.T + pos) * D;
    const bool padded = P.pad && P.pad[(size_t)b * P.T + pos] != 0;
    float y = 0.f;
    if (!padded) {
        const float* base = P.part + ((size_t)bh * P.n_split * P.g_pad + gi) * (D + 2);
        const size_t stride = (size_t)P.g_pad * (D + 2);
        float M = kNegInf;
        for (int s = 0; s < P.n_split; s++) M = __builtin_fmaxf(M, base[s * stride]);
        float Lsum = 0.f, O = 0.f;
        if (M != kNegInf) {
            for (int s = 0; s < P.n_split; s++) {
                const float* p = base + s * stride;
                const float w = (p[0] == kNegInf) ? 0.f : __builtin_amdgcn_exp2f(p[0] - M);
                Lsum += p[1] * w;
                O += p[2 + c] * w;
            }
        }
        y = Lsum > 0.f ? O / Lsum : 0.f;
    }
    if constexpr (sizeof(OT) == 2) {
        __bf16 yb = (__bf16)y;
        orow[c] = __builtin_bit_cast(OT, yb);
    } else {
        orow[c] = y;
    }
}

}  // namespace lfk

// ---------------------------------------------------------------------------
// launchers (called from the host library)

namespace lfk {

template <int QB, int KS, typename ET, typename OT>
static hipError_t launch_tiles(const Params& P, int first_task, int n_tasks, hipStream_t s) {
    (void)first_task;
    const int grid = ((n_tasks + 7) / 8) * 8;
    hipLaunchKernelGGL((tile_kernel<QB, KS, ET, OT>), dim3(grid), dim3(64 * QB * KS), 0, s, P);
    return hipGetLastError();
}

}  // namespace lfk

extern "C" hipError_t lfk_launch(const lfk::Params* P, int dtype_bf16, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    hipError_t e;
    if (dtype_bf16)
        e = lfk::launch_tiles<LFK_QB, LFK_KS, __bf16, uint16_t>(*P, 0, P->n_tasks, s);
    else
        e = lfk::launch_tiles<LFK_QB, LFK_KS, float, float>(*P, 0, P->n_tasks, s);
    if (e != hipSuccess) return e;
    if (P->n_g > 0) {
        const int grid = P->B * P->H * P->n_g;
        if (dtype_bf16)
            hipLaunchKernelGGL(lfk::combine_kernel<uint16_t>, dim3(grid), dim3(64), 0, s, *P);
        else
            hipLaunchKernelGGL(lfk::combine_kernel<float>, dim3(grid), dim3(64), 0, s, *P);
        e = hipGetLastError();
    }
    return e;
}
