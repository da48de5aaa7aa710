// lf_bwd_mfma.hip -- the gradients of the Longformer sparse self-attention
// forward on the gfx950 matrix cores (bf16 inputs, d = 64), for every
// non-global query (dq) and every non-global key (dk, dv).
//
// The pages give no backward pass (Longformer, ciallo.wiki, §5.2 only says
// that training cost grows linearly with the length).  What is computed is
// the derivative of the forward map over its allowed pairs.  With the row
// statistics of the forward (lse_i, the log of row i's softmax denominator)
// the weights are P_ij = exp(s_ij - lse_i); with dP_ij = dy_i . v_j and
// D_i = sum_j P_ij dP_ij = dy_i . y_i (y the forward's output),
//     dS_ij = P_ij (dP_ij - D_i),
//     dq_i = sum_j dS_ij k_j / sqrt(d),  dk_j = sum_i dS_ij q_i / sqrt(d),
//     dv_j = sum_i P_ij dy_i.
//
// The tiles are the forward's: 64 consecutive positions of one dilation
// residue class (Longformer, ciallo.wiki §2.2.3), where query t and key u
// of the class are a band pair when u - t lies in [-r, ra] (ra = r
// two-sided, 0 one-sided; eightmm.github.io, "Sliding-Window Attention",
// "Implementation Reading").  Each pair of the allowed set is counted once:
//   * band blocks: the band pairs, global keys and rows among them;
//   * global blocks: a non-global query with the global keys outside its
//     band (dq), or a key with the global queries whose band misses it (dk,
//     dv) ("Global Attention": a global row reads every key, every row
//     reads the global keys);
//   * random blocks (undilated heads): a query block's drawn key blocks
//     without the keys of the window or of G, and for dk, dv the query
//     blocks that drew the key block, without global queries;
//   * global tasks (task kind 1): the global rows' dq over one split of the
//     keys, the global keys' dk, dv over one split of the queries; each
//     writes an fp32 partial record, and the last task of a head adds the
//     splits in order and writes the rows.
//
// Two launches:
//   dq_kernel    query-major: a tile of 64 class queries (two blocks of 32,
//                two key phases, four waves) streams its key blocks through
//                an LDS ring: S^T = K Q^T, dP^T = V dY^T,
//                dS^T = P^T (dP^T - D), dQ^T += K^T dS^T (12 MFMAs a block).
//                It also writes each row's statistics (lse_i log2 e,
//                D_i = dy_i . y_i; a padded row, lse = -inf, gets (+inf, 0),
//                so its weights vanish) for the dk/dv kernel.
//   dkdv_kernel  key-major: a tile of 64 class keys streams the blocks of
//                the queries that read them: S = Q K^T, dP = dY V^T,
//                dS = P (dP - D), dV^T += dY^T P, dK^T += Q^T dS (16 MFMAs).
// Every output row is written by one lane: no atomics, reproducible results.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "lf_kernels.h"
#include "lf_decode.h"
#include "lf_device.h"

namespace lfk {
namespace bwd {

constexpr int D = 64;
constexpr int BM = LFK_BM;
constexpr float SC = ScaleLog2<64>::v;   // log2(e) / 8
constexpr float kLog2e = 1.4426950408889634f;
constexpr int ROWB = 2 * D;              // bytes of a bf16 row
constexpr int GT = LF_MAX_GLOBALS;

// LDS form of a block of 32 rows x 64 channels (4 KiB): channel
// 32cb + 8j + e of row `row` at byte
//     cb*2048 + row*64 + 16*(j ^ ((row >> 2) & 3)) + 2e.
// One form serves both reads without bank conflicts: the row operand
// (ds_read_b128; lane l takes row l%32, channels 16ks + 8(l/32) .. +7) and
// the transposed operand of the products whose contraction runs over the
// block's rows (dQ^T = K^T dS^T; dV^T = dY^T P, dK^T = Q^T dS), read with
// ds_read_b64_tr_b16 in the row order in which a 32x32 accumulator packs
// into the other operand.  Each 1 KiB piece (cb, half: rows 16half ..
// +15) is written by one buffer_load_dwordx4 ... lds of a wave: lane p
// brings row 16half + p/4, channels 32cb + 8((p & 3) ^ ((p >> 4) & 3)) ..
// +7.

struct Tile {
    int kind;            // 0: band tile; 1: the global rows (dq) or global keys (dk, dv) of one split
    int b, h, bh, c, delta, n, m0, r, ra;
    int split, lo, hi;   // kind 1: the split and the rows it streams, [lo, hi)
};

__device__ __forceinline__ Tile decode_tile(const Plan& P, int t) {
    Tile k;
    if (t < P.n_band_tasks) {
        const BandTask bt = decode_band(P, t);
        k.kind = 0;
        k.b = bt.b;
        k.h = bt.h;
        k.bh = bt.b * P.H + bt.h;
        k.c = bt.c;
        k.delta = P.dil[bt.h];
        k.n = bt.n;
        k.m0 = bt.tile * BM;
        k.r = P.rad[bt.h];
        k.ra = P.one_sided ? 0 : k.r;
        k.split = 0;
        k.lo = 0;
        k.hi = k.n;
    } else {
        const RowTask rt = decode_rows(P, t - P.n_band_tasks);
        k.kind = 1;
        k.bh = rt.bh;
        k.b = mdiv(rt.bh, P.mg_H);
        k.h = rt.bh - k.b * P.H;
        k.c = 0;
        k.delta = 1;
        k.n = P.T;
        k.m0 = rt.grp * BM;
        k.r = 0;
        k.ra = 0;
        k.split = rt.split;
        k.lo = rt.split * P.split_len;
        k.hi = min(k.lo + P.split_len, P.T);
    }
    return k;
}

// Each of the 8 dies (blockIdx % 8) takes its band tiles (a contiguous
// eighth, or the run the plan cut by cost, so that neighbouring tiles, which
// read the same rows, share its L2) and its global tasks: after the tiles,
// where the short global tasks fill the tail of the tiles' last round, or
// before them when they are the longer kind; -1 for a slot past the end.
__device__ __forceinline__ int tile_of_block(const Plan& P) {
    return task_of_slot(P, blockIdx.x & 7, blockIdx.x >> 3, P.bwd_globals_first != 0);
}

// The last of the n_split * n_ggroups workgroups of head (b, h) to finish
// a global task returns true (and the counter to zero for the next call):
// every partial record of the head is then written.  The records cross
// dies, so they are written and read with the agent-coherent policy.
__device__ __forceinline__ bool last_arriver(const Plan& P, int* counter, int bh, char* smem) {
    __builtin_amdgcn_s_waitcnt(0);   // this wave's record stores have completed
    __syncthreads();
    int* flag = (int*)smem;
    if (threadIdx.x == 0) {
        const int done = __hip_atomic_fetch_add(counter + bh, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool last = done == P.n_split * P.n_ggroups - 1;
        if (last) __hip_atomic_store(counter + bh, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        *flag = last;
    }
    __syncthreads();
    return *flag != 0;
}

// write a partial record: this lane's channels 32cb + 8j + 4lg .. +3 of an
// O^T-form accumulator pair at float offset `rec` (+ 64 * part)
__device__ __forceinline__ void store_record(__amdgpu_buffer_rsrc_t rs, uint32_t rec, const f32x16 (&acc)[2],
                                             int lg) {
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const f32x4 o4 = {acc[cb][4 * j], acc[cb][4 * j + 1], acc[cb][4 * j + 2], acc[cb][4 * j + 3]};
            __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o4), rs,
                                                   4u * (rec + 32 * cb + 8 * j + 4 * lg), 0, kCoherent);
        }
}

// Sum of the splits' records of head bh: thread task (gi, part, c4) adds
// channels 4 c4 .. +3 of part `part` of global slot gi over the splits and
// writes them to the part's output row (bf16, times scale[part]); zeros at
// a padded position.  nparts: 1 (dq) or 2 (dk, dv); records hold 64 floats
// per part.
__device__ __forceinline__ void combine_records(const Plan& P, __amdgpu_buffer_rsrc_t rs, int nparts, int bh,
                                                const uint8_t* padrow, uint16_t* out0, uint16_t* out1,
                                                float scale0, float scale1) {
    const int n_g = P.n_g, T = P.T;
    const uint32_t rstride = 64u * nparts;                         // floats per record
    const uint32_t sstride = (uint32_t)P.g_pad * rstride;          // floats between splits of a slot
    for (int task = threadIdx.x; task < n_g * nparts * 16; task += 256) {
        const int gi = task / (nparts * 16), rem = task % (nparts * 16), part = rem / 16, c4 = rem % 16;
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        for (int sp0 = 0; sp0 < P.n_split; sp0 += 8) {
            f32x4 o[8];
#pragma unroll
            for (int i = 0; i < 8; i++) {
                const uint32_t rec = (uint32_t)min(sp0 + i, P.n_split - 1) * sstride + (uint32_t)gi * rstride +
                                     64u * part + 4u * c4;
                o[i] = __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, 4u * rec, 0, kCoherent));
            }
#pragma unroll
            for (int i = 0; i < 8; i++)
                if (sp0 + i < P.n_split) acc += o[i];
        }
        const int pos = P.glob[gi];
        const float sc = part == 0 ? scale0 : scale1;
        uint16_t* row = (part == 0 ? out0 : out1) + ((size_t)bh * T + pos) * D + 4 * c4;
        u32x2 w = {pack_bf16(acc[0] * sc, acc[1] * sc), pack_bf16(acc[2] * sc, acc[3] * sc)};
        if (padrow && padrow[pos] != 0) w = (u32x2){0u, 0u};   // zeros, whatever the records hold
        *(u32x2*)row = w;
    }
}

// One row as the MFMA operand of a 32x32x16 product, row per lane: lane l
// gets channels 16ks + 8(l/32) .. +7 of row pos (zeros for pos < 0).
__device__ __forceinline__ void load_operand(__amdgpu_buffer_rsrc_t rs, int pos, int lg, bf16x8 (&x)[4]) {
    const uint32_t off = pos >= 0 ? (uint32_t)pos * ROWB : kPastEnd;
#pragma unroll
    for (int ks = 0; ks < 4; ks++)
        x[ks] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off + 2u * (16 * ks + 8 * lg), 0, 0));
}

// Per-lane byte offsets of the two reads of a block (see the form above).
struct FormLane {
    int r0, r1;   // row operand: row l%32, channel groups 2(ks&1) + l/32 (ks even, odd)
    int t0, t1;   // transposed operand: rows 4(l/32) + (l&15)/4 and 8 more
    __device__ __forceinline__ FormLane(int lane) {
        const int lq = lane & 31, lg = lane >> 5, sw = (lq >> 2) & 3;
        r0 = lq * 64 + 16 * (lg ^ sw);
        r1 = lq * 64 + 16 * (lg ^ sw ^ 2);
        const int row = 4 * lg + ((lane & 15) >> 2), j = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);
        t0 = row * 64 + 16 * (j ^ lg) + 8 * (lane & 1);
        t1 = (row + 8) * 64 + 16 * (j ^ lg ^ 2) + 8 * (lane & 1);
    }
};

// row operand: lane l supplies row l%32, channels 16ks + 8(l/32) .. +7
__device__ __forceinline__ void read_rows(const char* blk, const FormLane& f, bf16x8 (&x)[4]) {
    x[0] = __builtin_bit_cast(bf16x8, *(const u32x4*)(blk + f.r0));
    x[1] = __builtin_bit_cast(bf16x8, *(const u32x4*)(blk + f.r1));
    x[2] = __builtin_bit_cast(bf16x8, *(const u32x4*)(blk + 2048 + f.r0));
    x[3] = __builtin_bit_cast(bf16x8, *(const u32x4*)(blk + 2048 + f.r1));
}

// transposed operand [st][cb]: rows 16st .. +15, channels 32cb .. +31
__device__ __forceinline__ void read_tr(const char* blk, const FormLane& f, bf16x8 (&x)[2][2]) {
#pragma unroll
    for (int st = 0; st < 2; st++)
#pragma unroll
        for (int cb = 0; cb < 2; cb++) {
            const char* a = blk + cb * 2048 + st * 1024;
            x[st][cb] = cat_tr(ds_tr16(a + f.t0), ds_tr16(a + f.t1));
        }
}

// the four pieces of a block into LDS at dst: o0, o1 the lane's row
// offsets for rows p/4 and 16 + p/4 (with the channel group of the form)
__device__ __forceinline__ void load_block(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t o0, uint32_t o1) {
#pragma unroll
    for (int x = 0; x < 4; x++) load_lds16(rs, dst + (x >> 1) * 2048 + (x & 1) * 1024, (x & 1) ? o1 : o0, 64 * (x >> 1));
}

// zeros over this lane's part of a block where its rows are padded
__device__ __forceinline__ void zero_block_rows(char* dst, int lane, bool pad0, bool pad1) {
    const u32x4 z = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int x = 0; x < 4; x++)
        if ((x & 1) ? pad1 : pad0) *(u32x4*)(dst + (x >> 1) * 2048 + (x & 1) * 1024 + 16 * lane) = z;
}

// accumulator elements 8st .. 8st+7 -> bf16 operand st
__device__ __forceinline__ void pack_operand(const float (&p)[16], bf16x8 (&x)[2]) {
#pragma unroll
    for (int st = 0; st < 2; st++) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; e++) w[e] = pack_bf16(p[8 * st + 2 * e], p[8 * st + 2 * e + 1]);
        x[st] = __builtin_bit_cast(bf16x8, w);
    }
}

// Write a transposed accumulator pair (this lane's row: channels
// 32cb + 8j + 4lg + e) as a bf16 row: lanes l and l^32 trade channel groups
// with v_permlane32_swap so that each writes 8 consecutive channels (the
// lower lane keeps group 2m and takes its partner's, the upper lane keeps
// 2m+1 likewise).  zero: write zeros.
__device__ __forceinline__ void store_row(uint16_t* row, const f32x16 (&acc)[2], float scale, bool zero, int lg) {
#pragma unroll
    for (int cb = 0; cb < 2; cb++) {
        uint32_t g[4][2];
#pragma unroll
        for (int j = 0; j < 4; j++) {
            const float y0 = zero ? 0.f : acc[cb][4 * j] * scale, y1 = zero ? 0.f : acc[cb][4 * j + 1] * scale;
            const float y2 = zero ? 0.f : acc[cb][4 * j + 2] * scale, y3 = zero ? 0.f : acc[cb][4 * j + 3] * scale;
            g[j][0] = pack_bf16(y0, y1);
            g[j][1] = pack_bf16(y2, y3);
        }
#pragma unroll
        for (int m = 0; m < 2; m++) {
            const auto r0 = __builtin_amdgcn_permlane32_swap(g[2 * m][0], g[2 * m + 1][0], false, false);
            const auto r1 = __builtin_amdgcn_permlane32_swap(g[2 * m][1], g[2 * m + 1][1], false, false);
            *(u32x4*)(row + 32 * cb + 16 * m + 8 * lg) = (u32x4){r0[0], r1[0], r0[1], r1[1]};
        }
    }
}

__device__ __forceinline__ bool is_global(const uint32_t* gmap, int pos) {
    return (gmap[pos >> 5] >> (pos & 31)) & 1u;
}

// rows of a block starting at position p0 (step 1) that lie at or past T
__device__ __forceinline__ uint32_t past_end(int p0, int T) {
    const int valid = T - p0;
    return valid >= 32 ? 0u : (valid <= 0 ? 0xffffffffu : 0xffffffffu << valid);
}

// The global tables of a tile, for slots [0, ngb * 32): the position a
// slot's rows load from (T: no global, or a padded one), its class index
// in the tile's class (kNotInClass: another class), and per 32 slots the
// ones that are no live global.
template <bool PAD>
__device__ void build_gtab(const Plan& P, const Tile& tk, const uint8_t* padrow, int ngb, int* gld, int* gcls,
                           uint32_t* gbad, int wave, int lane) {
    const int n_g = P.n_g, T = P.T;
    for (int base = 64 * wave; base < ngb * KBLK; base += 256) {
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
        if (slot < ngb * KBLK) {
            gld[slot] = padded ? T : pos;
            gcls[slot] = cls;
        }
        const uint64_t badm = __ballot(!inr || padded);
        if (lane == 0) {
            gbad[base >> 5] = (uint32_t)badm;
            if (base + 32 < ngb * KBLK) gbad[(base >> 5) + 1] = (uint32_t)(badm >> 32);
        }
    }
}

// ---------------------------------------------------------------------------

// ---------------------------------------------------------------------------
// Shared by both band kernels: the tile's block list.  Blocks 0 .. nb-1 are
// the band (class blocks kb_lo ..), then ngb global blocks (32 slots each),
// then nrb random blocks (32 rows each, two per drawn block of 64); stage s
// of the ring holds blocks 2s and 2s+1, and phase ph works on block 2s+ph.

enum { kBand = 0, kGlob = 1, kRand = 2, kNone = 3 };

struct Blocks {
    int nb, ngb, nrb, nblk, kb_lo;
    __device__ __forceinline__ int kind(int j) const {
        return j < nb ? kBand : (j < nb + ngb ? kGlob : (j < nblk ? kRand : kNone));
    }
};

// ---------------------------------------------------------------------------
// dq.  Per block in LDS: K at 0, V at 4096, both in the form above.
// Waves (qb, ph): qb = query block of the tile, ph = key phase.  A wave of
// query block 0 loads K of its phase's block, one of query block 1 V.

template <bool PAD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(3))) void dq_kernel(const BwdBandArgs A) {
    constexpr int BLK = 8192, STAGE = 2 * BLK, RING = 2 * STAGE;
    __shared__ __attribute__((aligned(16))) char smem[RING];
    __shared__ __attribute__((aligned(16))) int gld[GT];
    __shared__ __attribute__((aligned(16))) int gcls[GT];
    __shared__ uint32_t gbad[GT / 32];
    const Plan& P = *A.plan;
    const int task = tile_of_block(P);
    if (task < 0) return;
    const Tile tk = decode_tile(P, task);
    const int T = P.T;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int qb = wave & 1, ph = wave >> 1, lq = lane & 31, lg = lane >> 5;
    const int r = tk.r, ra = tk.ra;
    const size_t head = (size_t)tk.bh * T;
    const uint8_t* padrow = PAD ? A.pad + (size_t)tk.b * T : nullptr;

    // this wave's 32 queries (band: class positions; kind 1: global slots) and this lane's
    const int mq0 = tk.m0 + 32 * qb;
    const int m_me = mq0 + lq;
    const bool glob_task = tk.kind == 1;
    const bool wave_active = mq0 < (glob_task ? P.n_g : tk.n);
    int my_pos = -1;
    if (!glob_task && m_me < tk.n) my_pos = tk.c + tk.delta * m_me;
    if (glob_task && m_me < P.n_g) my_pos = P.glob[m_me];
    const int key_end = glob_task ? tk.hi : tk.n;   // keys at or past it (class index) are none

    Blocks bl;
    if (!glob_task) {
        int lo_k = tk.m0 - r; if (lo_k < 0) lo_k = 0;
        int hi_k = tk.m0 + BM - 1 + ra; if (hi_k > tk.n - 1) hi_k = tk.n - 1;
        bl.kb_lo = lo_k / KBLK;
        bl.nb = hi_k / KBLK - bl.kb_lo + 1;
        bl.ngb = P.n_g > 0 ? (P.n_g + KBLK - 1) / KBLK : 0;
        bl.nrb = P.n_rand > 0 ? 2 * P.n_rand : 0;
    } else {
        // a global row reads every key: the split's keys, no window
        bl.kb_lo = tk.lo / KBLK;
        bl.nb = (tk.hi - tk.lo + KBLK - 1) / KBLK;
        bl.ngb = 0;
        bl.nrb = 0;
    }
    bl.nblk = bl.nb + bl.ngb + bl.nrb;
    const int NS = (bl.nblk + 1) >> 1;
    // random key blocks of this query block (undilated: tile = query block)
    const int32_t* rrow = bl.nrb > 0 ? P.rtab + ((size_t)tk.h * ((T + 63) >> 6) + (tk.m0 >> 6)) * P.n_rand : nullptr;
    auto rand_p0 = [&](int jr) -> int {   // row 0 of random block jr, T for none
        if (jr < 0 || jr >= bl.nrb) return T;
        const int rho = rrow[jr >> 1];
        return rho >= 0 ? 64 * rho + 32 * (jr & 1) : T;
    };
    // band blocks with keys for this wave's queries, and those needing no mask
    int j_lo = 0, j_hi = -1, ji_lo = 0, ji_hi = -1;
    if (wave_active && !glob_task) {
        int a = mq0 - r; if (a < 0) a = 0;
        int z = mq0 + 31 + ra; if (z > tk.n - 1) z = tk.n - 1;
        j_lo = a / KBLK - bl.kb_lo;
        j_hi = z / KBLK - bl.kb_lo;
        ji_lo = ((mq0 + 31 - r + 31) >> 5) - bl.kb_lo;
        ji_hi = min((mq0 + ra - 31) >> 5, (tk.n - 32) >> 5) - bl.kb_lo;
    } else if (wave_active) {
        j_hi = bl.nb - 1;
        ji_hi = ((key_end - 32) >> 5) - bl.kb_lo;
    }

    // ---- loads
    const bool w0 = qb == 0;
    const int row0 = lane >> 2, row1 = 16 + (lane >> 2);
    const uint32_t colU = 16u * ((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t vo0 = (uint32_t)min((long long)tk.delta * row0, (long long)T) * ROWB + colU;
    const uint32_t vo1 = (uint32_t)min((long long)tk.delta * row1, (long long)T) * ROWB + colU;
    const char* khead = (const char*)A.k + head * ROWB;
    const char* vhead = (const char*)A.v + head * ROWB;
    auto row0_of = [&](int j) -> int { return tk.c + tk.delta * (bl.kb_lo + j) * KBLK; };
    auto win = [&](const char* base, int p0) -> __amdgpu_buffer_rsrc_t {
        return buffer_rsrc(base + (uint64_t)p0 * ROWB, p0 < T ? (uint32_t)(T - p0) * ROWB : 0u);
    };
    // block jb into the ring slot at off.  pm: padded rows of the block,
    // which load as zeros (NaN or Inf stored at a padded key must not reach
    // a product); global slots load through gld.
    auto issue = [&](int s, int off, uint32_t pm) {
        const int jb = 2 * s + ph;
        const int kd = bl.kind(jb);
        if (kd == kNone) return;
        char* dst = smem + off + ph * BLK + (w0 ? 0 : 4096);
        __amdgpu_buffer_rsrc_t rs;
        uint32_t o0, o1;
        if (kd == kGlob) {
            const int sl0 = (jb - bl.nb) * KBLK;
            rs = buffer_rsrc(w0 ? khead : vhead, (uint32_t)T * ROWB);
            o0 = (uint32_t)gld[sl0 + row0] * ROWB + colU;
            o1 = (uint32_t)gld[sl0 + row1] * ROWB + colU;
        } else {
            // p0 is the same in every lane; said so, the descriptor stays scalar
            const int p0 = uniform(kd == kBand ? row0_of(jb) : rand_p0(jb - bl.nb - bl.ngb));
            rs = win(w0 ? khead : vhead, p0);
            o0 = vo0;
            o1 = vo1;
        }
        if (PAD && ((pm >> row0) & 1u)) o0 = kPastEnd;
        if (PAD && ((pm >> row1) & 1u)) o1 = kPastEnd;
        load_block(rs, dst, o0, o1);
    };
    // padding: lane l < 32 reads the byte of row l of this phase's block two
    // stages ahead; a ballot one stage ahead makes the block's padded-row word
    const __amdgpu_buffer_rsrc_t rpad = buffer_rsrc(padrow, PAD ? (uint32_t)T : 0u);
    auto pad_at = [&](int s) -> uint32_t {
        const int q = 2 * s + ph;
        const int kd = bl.kind(q);
        const int pos = kd == kBand ? row0_of(q) + tk.delta * lq
                                    : (kd == kRand ? rand_p0(q - bl.nb - bl.ngb) + lq : T);
        return __builtin_amdgcn_raw_buffer_load_b8(rpad, (uint32_t)min(pos, T), 0, 0);
    };
    auto pad_word = [&](uint32_t byte) -> uint32_t { return (uint32_t)__ballot(lane < 32 && byte != 0u); };

    // this lane's query: Q and dY as operands, the forward's output row and
    // lse for its statistics
    const __amdgpu_buffer_rsrc_t rq = buffer_rsrc((const char*)A.q + head * ROWB, (uint32_t)T * ROWB);
    const __amdgpu_buffer_rsrc_t ry = buffer_rsrc((const char*)A.dy + head * ROWB, (uint32_t)T * ROWB);
    const __amdgpu_buffer_rsrc_t ro = buffer_rsrc((const char*)A.y + head * ROWB, (uint32_t)T * ROWB);
    bf16x8 qh[4], yh[4], oh[4];
    load_operand(rq, my_pos, lg, qh);
    load_operand(ry, my_pos, lg, yh);
    load_operand(ro, my_pos, lg, oh);
    const float lse_nat = my_pos >= 0 ? A.lse[head + my_pos] : kNegInf;
    f32x16 acc[2] = {(f32x16){}, (f32x16){}};
    const FormLane fl(lane);

    uint32_t pm_cur = 0u, pbyte = 0u;
    if constexpr (PAD) {
        pm_cur = pad_at(0);
        pbyte = pad_at(1);
    }
    const bool early0 = bl.kind(ph) != kGlob;
    if (early0) issue(0, 0, 0u);
    if (bl.ngb > 0) {
        build_gtab<PAD>(P, tk, padrow, bl.ngb, gld, gcls, gbad, wave, lane);
        __syncthreads();
    }
    if (!early0) issue(0, 0, 0u);
    barrier_lds_loads();
    // D = dy . y over this lane's 32 channels, then the other half's
    float dsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < 4; ks++) {
        const u32x4 a = __builtin_bit_cast(u32x4, yh[ks]), b = __builtin_bit_cast(u32x4, oh[ks]);
#pragma unroll
        for (int e = 0; e < 4; e++) dsum += bf_lo(a[e]) * bf_lo(b[e]) + bf_hi(a[e]) * bf_hi(b[e]);
    }
    dsum = halves_sum(dsum);
    const bool no_row = !(lse_nat > kNegInf);   // a padded row, or no row
    const float nl = no_row ? kNegInf : -lse_nat * kLog2e, Dq = no_row ? 0.f : dsum;
    // every row's statistics, for the dk/dv and global-row kernels (each row
    // is in one tile; the phase-0 waves write them)
    if (!glob_task && ph == 0 && lg == 0 && my_pos >= 0) ((float2*)A.stats)[head + my_pos] = make_float2(-nl, Dq);
    if constexpr (PAD) {
        pm_cur = pad_word(pm_cur);
        // stage 0 went out before its padding word was known: clear what this
        // wave brought for padded rows
        if (pm_cur != 0u)
            zero_block_rows(smem + ph * BLK + (w0 ? 0 : 4096), lane, (pm_cur >> row0) & 1u, (pm_cur >> row1) & 1u);
        __syncthreads();
    }

    for (int s = 0; s < NS; s++) {
        if (s > 0) barrier_lds_loads();   // stage s landed; stage s-1 no longer read
        const int oc = (s & 1) * STAGE, on = ((s + 1) & 1) * STAGE;
        const int j = 2 * s + ph;
        const int kd = bl.kind(j);
        const bool rel = kd == kBand ? (j >= j_lo && j <= j_hi) : (kd != kNone && wave_active);
        bf16x8 kf[4], vf[4];
        if (rel) {
            read_rows(smem + oc + ph * BLK, fl, kf);
            read_rows(smem + oc + ph * BLK + 4096, fl, vf);
        }
        uint32_t pm_next = 0u;
        if constexpr (PAD) {
            pm_next = pad_word(pbyte);
            pbyte = pad_at(s + 2);
        }
        if (s + 1 < NS) issue(s + 1, on, pm_next);
        if (rel) {
            f32x16 sc = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < 4; ks++) sc = mfma(kf[ks], qh[ks], sc);
#pragma unroll
            for (int ks = 0; ks < 4; ks++) dp = mfma(vf[ks], yh[ks], dp);
            if (kd == kBand) {
                if (!(j >= ji_lo && j <= ji_hi && (!PAD || pm_cur == 0u))) {
                    if (!glob_task) mask_window(sc, m_me - r - (bl.kb_lo + j) * KBLK - 4 * lg, r + ra);
                    const int valid = key_end - (bl.kb_lo + j) * KBLK;
                    uint32_t bad = valid >= KBLK ? 0u : (0xffffffffu << valid);
                    if constexpr (PAD) bad |= pm_cur;
                    if (bad != 0u) mask_bits(sc, ~lane_bits(bad, lg));
                }
            } else if (kd == kGlob) {
                const int sl0 = (j - bl.nb) * KBLK;
                mask_global(sc, gbad[sl0 >> 5], gcls + sl0, m_me, r, r + ra, lg);
            } else {
                // random keys: not in this query's window, not global, not padded
                const int p0 = rand_p0(j - bl.nb - bl.ngb);
                mask_window_out(sc, m_me - r - p0 - 4 * lg, r + ra);
                uint32_t bad = past_end(p0, T);
                if (p0 < T) bad |= A.gmap[p0 >> 5];
                if constexpr (PAD) bad |= pm_cur;
                if (bad != 0u) mask_bits(sc, ~lane_bits(bad, lg));
            }
            float ds[16];
#pragma unroll
            for (int i = 0; i < 16; i++) {
                const float p = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], SC, nl));
                ds[i] = p * (dp[i] - Dq);
            }
            bf16x8 dso[2];
            pack_operand(ds, dso);
            // K^T operands, read only now: the scheduling barrier keeps the
            // compiler from hoisting the reads above the products, where
            // their registers overflow the budget of three workgroups per
            // CU and spill
            __builtin_amdgcn_sched_barrier(0);
            bf16x8 tf[2][2];
            read_tr(smem + oc + ph * BLK, fl, tf);
#pragma unroll
            for (int st2 = 0; st2 < 2; st2++)
#pragma unroll
                for (int cb = 0; cb < 2; cb++) acc[cb] = mfma(tf[st2][cb], dso[st2], acc[cb]);
        }
        pm_cur = pm_next;
    }
    __syncthreads();

    // the two phases' sums meet through LDS
    f32x4* mbuf = (f32x4*)smem + (qb * 64 + lane) * 8;
    if (ph == 1) {
#pragma unroll
        for (int cb = 0; cb < 2; cb++)
#pragma unroll
            for (int i = 0; i < 4; i++)
                mbuf[4 * cb + i] = (f32x4){acc[cb][4 * i], acc[cb][4 * i + 1], acc[cb][4 * i + 2], acc[cb][4 * i + 3]};
    }
    __syncthreads();
    if (glob_task) {
        // this split's part of the global rows' dq, then the last of the
        // head's tasks adds the parts up
        const uint32_t rstride = (uint32_t)P.g_pad * 64u;
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(A.part_q + (size_t)tk.bh * P.n_split * rstride,
                                                      (uint32_t)P.n_split * rstride * 4u);
        if (ph == 0 && wave_active && m_me < P.n_g) {
#pragma unroll
            for (int cb = 0; cb < 2; cb++)
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const f32x4 x = mbuf[4 * cb + i];
#pragma unroll
                    for (int e = 0; e < 4; e++) acc[cb][4 * i + e] += x[e];
                }
            store_record(rs, (uint32_t)tk.split * rstride + (uint32_t)m_me * 64u, acc, lg);
        }
        if (last_arriver(P, A.count_q, tk.bh, smem))
            combine_records(P, rs, 1, tk.bh, padrow, (uint16_t*)A.dq, nullptr, 0.125f, 0.f);
        return;
    }
    if (ph == 1 || my_pos < 0) return;
#pragma unroll
    for (int cb = 0; cb < 2; cb++)
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const f32x4 x = mbuf[4 * cb + i];
#pragma unroll
            for (int e = 0; e < 4; e++) acc[cb][4 * i + e] += x[e];
        }
    if (is_global(A.gmap, my_pos)) return;   // the global-row tasks write it
    const bool zero = PAD && padrow[my_pos] != 0;
    store_row((uint16_t*)A.dq + (head + my_pos) * D, acc, 0.125f, zero, lg);
}

// ---------------------------------------------------------------------------
// dk, dv.  Per block in LDS: Q at 0, dY at 4096 (both in the form above),
// then the block's 32 values lse log2 e and 32 values D at 8192.  Waves
// (kb, ph): kb = key block of the tile, ph = query phase.  A wave of key
// block 0 loads Q of its phase's block, one of key block 1 dY and the
// statistics.

template <bool PAD>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void dkdv_kernel(const BwdBandArgs A) {
    constexpr int BLK = 8192 + 256, STAGE = 2 * BLK, RING = 2 * STAGE;
    __shared__ __attribute__((aligned(16))) char smem[RING];
    __shared__ __attribute__((aligned(16))) int gld[GT];
    __shared__ __attribute__((aligned(16))) int gcls[GT];
    __shared__ uint32_t gbad[GT / 32];
    const Plan& P = *A.plan;
    const int task = tile_of_block(P);
    if (task < 0) return;
    const Tile tk = decode_tile(P, task);
    const int T = P.T;
    const int tid = threadIdx.x, lane = tid & 63, wave = uniform(tid >> 6);
    const int kb = wave & 1, ph = wave >> 1, lq = lane & 31, lg = lane >> 5;
    const int r = tk.r, ra = tk.ra;
    const size_t head = (size_t)tk.bh * T;
    const uint8_t* padrow = PAD ? A.pad + (size_t)tk.b * T : nullptr;

    // this wave's 32 keys (band: class positions; kind 1: global slots) and this lane's
    const int mk0 = tk.m0 + 32 * kb;
    const int m_me = mk0 + lq;
    const bool glob_task = tk.kind == 1;
    const bool wave_active = mk0 < (glob_task ? P.n_g : tk.n);
    int my_pos = -1;
    if (!glob_task && m_me < tk.n) my_pos = tk.c + tk.delta * m_me;
    if (glob_task && m_me < P.n_g) my_pos = P.glob[m_me];
    const int q_end = glob_task ? tk.hi : tk.n;   // queries at or past it (class index) are none

    // query t reads key u when u - t is in [-r, ra]: key u is read by the
    // queries [u - ra, u + r]; every query reads a global key
    Blocks bl;
    if (!glob_task) {
        int lo_q = tk.m0 - ra; if (lo_q < 0) lo_q = 0;
        int hi_q = tk.m0 + BM - 1 + r; if (hi_q > tk.n - 1) hi_q = tk.n - 1;
        bl.kb_lo = lo_q / KBLK;
        bl.nb = hi_q / KBLK - bl.kb_lo + 1;
        bl.ngb = P.n_g > 0 ? (P.n_g + KBLK - 1) / KBLK : 0;
    } else {
        bl.kb_lo = tk.lo / KBLK;
        bl.nb = (tk.hi - tk.lo + KBLK - 1) / KBLK;
        bl.ngb = 0;
    }
    bl.nrb = 0;
    // random blocks: the query blocks that drew this key block (undilated)
    int ioff = 0;
    if (P.n_rand > 0 && !glob_task) {
        const int32_t* off = A.inv_off + (size_t)tk.h * (((T + 63) >> 6) + 1) + (tk.m0 >> 6);
        ioff = off[0];
        bl.nrb = 2 * (off[1] - off[0]);
    }
    bl.nblk = bl.nb + bl.ngb + bl.nrb;
    const int NS = (bl.nblk + 1) >> 1;
    auto rand_p0 = [&](int jr) -> int {
        if (jr < 0 || jr >= bl.nrb) return T;
        return 64 * A.inv_list[ioff + (jr >> 1)] + 32 * (jr & 1);
    };
    int j_lo = 0, j_hi = -1, ji_lo = 0, ji_hi = -1;
    if (wave_active && !glob_task) {
        int a = mk0 - ra; if (a < 0) a = 0;
        int z = mk0 + 31 + r; if (z > tk.n - 1) z = tk.n - 1;
        j_lo = a / KBLK - bl.kb_lo;
        j_hi = z / KBLK - bl.kb_lo;
        // every query q0 .. q0+31 of the block reads every key mk0 .. mk0+31
        ji_lo = ((mk0 + 31 - ra + 31) >> 5) - bl.kb_lo;
        ji_hi = min((mk0 + r - 31) >> 5, (tk.n - 32) >> 5) - bl.kb_lo;
    } else if (wave_active) {
        j_hi = bl.nb - 1;
        ji_hi = ((q_end - 32) >> 5) - bl.kb_lo;
    }

    // ---- loads
    const bool w0 = kb == 0;
    const int row0 = lane >> 2, row1 = 16 + (lane >> 2);
    const uint32_t colU = 16u * ((lane & 3) ^ ((lane >> 4) & 3));
    const uint32_t vo0 = (uint32_t)min((long long)tk.delta * row0, (long long)T) * ROWB + colU;
    const uint32_t vo1 = (uint32_t)min((long long)tk.delta * row1, (long long)T) * ROWB + colU;
    // statistics: lane l < 32 brings the lse of row l, lane l >= 32 the D of row l - 32
    const uint32_t voS = (uint32_t)min((long long)tk.delta * lq, (long long)T) * 8u + 4u * lg;
    const char* qhead = (const char*)A.q + head * ROWB;
    const char* yhead = (const char*)A.dy + head * ROWB;
    const char* shead = (const char*)(A.stats + 2 * head);
    auto row0_of = [&](int j) -> int { return tk.c + tk.delta * (bl.kb_lo + j) * KBLK; };
    auto win = [&](const char* base, int p0, int rb) -> __amdgpu_buffer_rsrc_t {
        return buffer_rsrc(base + (uint64_t)p0 * rb, p0 < T ? (uint32_t)(T - p0) * rb : 0u);
    };
    // block jb into the ring slot at off; pm: padded query rows, loaded as
    // zeros (their statistics give them zero weight)
    auto issue = [&](int s, int off, uint32_t pm) {
        const int jb = 2 * s + ph;
        const int kd = bl.kind(jb);
        if (kd == kNone) return;
        char* dst = smem + off + ph * BLK;
        __amdgpu_buffer_rsrc_t rs, rst;
        uint32_t o0, o1, oS;
        if (kd == kGlob) {
            const int sl0 = (jb - bl.nb) * KBLK;
            rs = buffer_rsrc(w0 ? qhead : yhead, (uint32_t)T * ROWB);
            rst = buffer_rsrc(shead, (uint32_t)T * 8u);
            o0 = (uint32_t)gld[sl0 + row0] * ROWB + colU;
            o1 = (uint32_t)gld[sl0 + row1] * ROWB + colU;
            oS = (uint32_t)gld[sl0 + lq] * 8u + 4u * lg;
        } else {
            const int p0 = uniform(kd == kBand ? row0_of(jb) : rand_p0(jb - bl.nb - bl.ngb));
            rs = win(w0 ? qhead : yhead, p0, ROWB);
            rst = win(shead, p0, 8);
            o0 = vo0;
            o1 = vo1;
            oS = voS;
        }
        if (PAD && ((pm >> row0) & 1u)) o0 = kPastEnd;
        if (PAD && ((pm >> row1) & 1u)) o1 = kPastEnd;
        load_block(rs, dst + (w0 ? 0 : 4096), o0, o1);
        if (!w0) __builtin_amdgcn_raw_ptr_buffer_load_lds(rst, LDS_PTR(dst + 8192), 4, oS, 0, 0, 0);
    };
    const __amdgpu_buffer_rsrc_t rpad = buffer_rsrc(padrow, PAD ? (uint32_t)T : 0u);
    auto pad_at = [&](int s) -> uint32_t {
        const int q = 2 * s + ph;
        const int kd = bl.kind(q);
        const int pos = kd == kBand ? row0_of(q) + tk.delta * lq
                                    : (kd == kRand ? rand_p0(q - bl.nb - bl.ngb) + lq : T);
        return __builtin_amdgcn_raw_buffer_load_b8(rpad, (uint32_t)min(pos, T), 0, 0);
    };
    auto pad_word = [&](uint32_t byte) -> uint32_t { return (uint32_t)__ballot(lane < 32 && byte != 0u); };

    // this lane's key: K and V as operands
    const __amdgpu_buffer_rsrc_t rk = buffer_rsrc((const char*)A.k + head * ROWB, (uint32_t)T * ROWB);
    const __amdgpu_buffer_rsrc_t rv = buffer_rsrc((const char*)A.v + head * ROWB, (uint32_t)T * ROWB);
    bf16x8 kh[4], vh[4];
    load_operand(rk, my_pos, lg, kh);
    load_operand(rv, my_pos, lg, vh);
    f32x16 ak[2] = {(f32x16){}, (f32x16){}}, av[2] = {(f32x16){}, (f32x16){}};
    const FormLane fl(lane);
    const int sbase = ph * BLK + 8192 + 16 * lg;   // lse of this lane's rows 8q4 + 4lg .. +3 at +32 q4

    uint32_t pm_cur = 0u, pbyte = 0u;
    if constexpr (PAD) {
        pm_cur = pad_at(0);
        pbyte = pad_at(1);
    }
    const bool early0 = bl.kind(ph) != kGlob;
    if (early0) issue(0, 0, 0u);
    if (bl.ngb > 0) {
        build_gtab<PAD>(P, tk, padrow, bl.ngb, gld, gcls, gbad, wave, lane);
        __syncthreads();
    }
    if (!early0) issue(0, 0, 0u);
    barrier_lds_loads();
    if constexpr (PAD) {
        pm_cur = pad_word(pm_cur);
        if (pm_cur != 0u)
            zero_block_rows(smem + ph * BLK + (w0 ? 0 : 4096), lane, (pm_cur >> row0) & 1u, (pm_cur >> row1) & 1u);
        __syncthreads();
    }

    for (int s = 0; s < NS; s++) {
        if (s > 0) barrier_lds_loads();
        const int oc = (s & 1) * STAGE, on = ((s + 1) & 1) * STAGE;
        const int j = 2 * s + ph;
        const int kd = bl.kind(j);
        const bool rel = kd == kBand ? (j >= j_lo && j <= j_hi) : (kd != kNone && wave_active);
        bf16x8 qf[4], yf[4];
        if (rel) {
            read_rows(smem + oc + ph * BLK, fl, qf);
            read_rows(smem + oc + ph * BLK + 4096, fl, yf);
        }
        uint32_t pm_next = 0u;
        if constexpr (PAD) {
            pm_next = pad_word(pbyte);
            pbyte = pad_at(s + 2);
        }
        if (s + 1 < NS) issue(s + 1, on, pm_next);
        if (rel) {
            f32x16 sc = {}, dp = {};
#pragma unroll
            for (int ks = 0; ks < 4; ks++) sc = mfma(qf[ks], kh[ks], sc);
#pragma unroll
            for (int ks = 0; ks < 4; ks++) dp = mfma(yf[ks], vh[ks], dp);
            // the statistics, read while the products run
            f32x4 l4[4], d4[4];
#pragma unroll
            for (int q4 = 0; q4 < 4; q4++) {
                l4[q4] = *(const f32x4*)(smem + oc + sbase + 32 * q4);
                d4[q4] = *(const f32x4*)(smem + oc + sbase + 128 + 32 * q4);
            }
            // element i: query row 8(i>>2) + 4lg + (i&3) of the block, this lane's key
            if (kd == kBand) {
                if (!(j >= ji_lo && j <= ji_hi)) {
                    if (!glob_task) mask_window(sc, m_me - ra - (bl.kb_lo + j) * KBLK - 4 * lg, r + ra);
                    const int valid = q_end - (bl.kb_lo + j) * KBLK;
                    if (valid < KBLK) mask_bits(sc, ~lane_bits(0xffffffffu << valid, lg));
                }
            } else if (kd == kGlob) {
                const int sl0 = (j - bl.nb) * KBLK;
                mask_global(sc, gbad[sl0 >> 5], gcls + sl0, m_me, ra, r + ra, lg);
            } else {
                // random queries: this key outside their window, not global
                const int p0 = rand_p0(j - bl.nb - bl.ngb);
                mask_window_out(sc, m_me - ra - p0 - 4 * lg, r + ra);
                uint32_t bad = past_end(p0, T);
                if (p0 < T) bad |= A.gmap[p0 >> 5];
                if (bad != 0u) mask_bits(sc, ~lane_bits(bad, lg));
            }
            float p[16], ds[16];
#pragma unroll
            for (int i = 0; i < 16; i++) {
                p[i] = __builtin_amdgcn_exp2f(__builtin_fmaf(sc[i], SC, -l4[i >> 2][i & 3]));
                ds[i] = p[i] * (dp[i] - d4[i >> 2][i & 3]);
            }
            bf16x8 po[2], dso[2];
            pack_operand(p, po);
            pack_operand(ds, dso);
            // Q^T and dY^T operands, read only now (as in the dq kernel: read
            // beside the products they made the kernel spill)
            __builtin_amdgcn_sched_barrier(0);
            bf16x8 qt[2][2], yt[2][2];
            read_tr(smem + oc + ph * BLK, fl, qt);
            read_tr(smem + oc + ph * BLK + 4096, fl, yt);
#pragma unroll
            for (int st2 = 0; st2 < 2; st2++)
#pragma unroll
                for (int cb = 0; cb < 2; cb++) {
                    av[cb] = mfma(yt[st2][cb], po[st2], av[cb]);
                    ak[cb] = mfma(qt[st2][cb], dso[st2], ak[cb]);
                }
        }
        pm_cur = pm_next;
    }
    __syncthreads();

    f32x4* mbuf = (f32x4*)smem + (kb * 64 + lane) * 16;
    if (ph == 1) {
#pragma unroll
        for (int cb = 0; cb < 2; cb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                mbuf[4 * cb + i] = (f32x4){ak[cb][4 * i], ak[cb][4 * i + 1], ak[cb][4 * i + 2], ak[cb][4 * i + 3]};
                mbuf[8 + 4 * cb + i] = (f32x4){av[cb][4 * i], av[cb][4 * i + 1], av[cb][4 * i + 2], av[cb][4 * i + 3]};
            }
    }
    __syncthreads();
    auto merge = [&]() {
#pragma unroll
        for (int cb = 0; cb < 2; cb++)
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const f32x4 x = mbuf[4 * cb + i], y = mbuf[8 + 4 * cb + i];
#pragma unroll
                for (int e = 0; e < 4; e++) {
                    ak[cb][4 * i + e] += x[e];
                    av[cb][4 * i + e] += y[e];
                }
            }
    };
    if (glob_task) {
        // this split's part of the global keys' dk and dv, then the last of
        // the head's tasks adds the parts up
        const uint32_t rstride = (uint32_t)P.g_pad * 128u;
        const __amdgpu_buffer_rsrc_t rs = buffer_rsrc(A.part_kv + (size_t)tk.bh * P.n_split * rstride,
                                                      (uint32_t)P.n_split * rstride * 4u);
        if (ph == 0 && wave_active && m_me < P.n_g) {
            merge();
            const uint32_t rec = (uint32_t)tk.split * rstride + (uint32_t)m_me * 128u;
            store_record(rs, rec, ak, lg);
            store_record(rs, rec + 64u, av, lg);
        }
        if (last_arriver(P, A.count_kv, tk.bh, smem))
            combine_records(P, rs, 2, tk.bh, padrow, (uint16_t*)A.dk, (uint16_t*)A.dv, 0.125f, 1.0f);
        return;
    }
    if (ph == 1 || my_pos < 0) return;
    merge();
    if (is_global(A.gmap, my_pos)) return;   // the global-key tasks write it
    const bool zero = PAD && padrow[my_pos] != 0;
    store_row((uint16_t*)A.dk + (head + my_pos) * D, ak, 0.125f, zero, lg);
    store_row((uint16_t*)A.dv + (head + my_pos) * D, av, 1.0f, zero, lg);
}

}  // namespace bwd
}  // namespace lfk

// grid of the band kernels: the slots of the 8 dies, each holding an eighth
// of the global tasks and of the band tiles
extern "C" int lfk_bwd_band_grid(const lfk::Plan* P) {
    return 8 * lfk::slots_per_die(*P);
}

// A: argument of the band kernels (A->plan: device copy of *P).  The dq
// kernel also writes every row's statistics, which the dk/dv kernel and
// the global-row kernels read: launch it first.
extern "C" hipError_t lfk_bwd_dq(const lfk::BwdBandArgs* A, const lfk::Plan* P, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const dim3 g(lfk_bwd_band_grid(P)), b(256);
    if (A->pad)
        hipLaunchKernelGGL(lfk::bwd::dq_kernel<true>, g, b, 0, s, *A);
    else
        hipLaunchKernelGGL(lfk::bwd::dq_kernel<false>, g, b, 0, s, *A);
    return hipGetLastError();
}

extern "C" hipError_t lfk_bwd_dkdv(const lfk::BwdBandArgs* A, const lfk::Plan* P, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const dim3 g(lfk_bwd_band_grid(P)), b(256);
    if (A->pad)
        hipLaunchKernelGGL(lfk::bwd::dkdv_kernel<true>, g, b, 0, s, *A);
    else
        hipLaunchKernelGGL(lfk::bwd::dkdv_kernel<false>, g, b, 0, s, *A);
    return hipGetLastError();
}
