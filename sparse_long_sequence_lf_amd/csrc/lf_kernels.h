// lf_kernels.h -- the launch records shared by the host planner
// (lf_host.cpp) and the gfx950 kernels (lf_fwd_kernels.hip).  Internal to
// liblfattn.so; the public interface is include/lf_attn.h.
#ifndef LF_KERNELS_H
#define LF_KERNELS_H

#include <stdint.h>

#include "lf_attn.h"

// Tile shape: two query blocks of 32 per workgroup and two key phases per
// query block (four waves), so a band tile holds 64 queries.
#define LFK_BM 64

namespace lfk {

// Division by a divisor d fixed for the call, for 0 <= n < 2^31:
//   s == 0:  n / 1 = n
//   s >= 1:  n / d = mulhi(n, m) >> (s - 1),  m = ceil(2^(31 + s) / d),  s = ceil(log2 d)
// (the error of the rounded-up reciprocal stays below 1/d for n < 2^31).
// Built on the host by magic_for(); one scalar multiply on the GPU.
struct Magic {
    uint32_t m;
    int32_t s;
};

// Everything about a call except the tensors: shape, per-head tables, the
// global set and workspace pointers.  Lives in device memory (one copy per
// (device, stream) workspace), re-uploaded only when it changes, so the
// kernel argument stays small (launch cost grows with argument size).
struct Plan {
    const void *kp, *vp;     // fp32 input: K and V as three bf16 planes per row [B*H][T][3][d]
    float *part;             // global-row partials [B*H][n_split][g_pad] records of d + 4 floats: O[d], m, l, 0, 0
    int *counter;            // [B*H] finished global-row workgroups; zero between calls
    int B, H, T, d;
    int r;                   // largest radius (clamped to T)
    int n_g;                 // distinct globals (sorted ascending in glob)
    int g_pad;               // n_ggroups * LFK_BM
    int n_ggroups;           // groups of LFK_BM global queries
    int n_split, split_len;  // global-row key splits (split_len multiple of 32)
    int n_band_tasks;        // B * band_tasks_per_batch
    int band_tasks_per_batch;
    int uniform_head_tasks;  // band tasks per head when every head has the same count, else 0
    int n_tasks;             // band + global-row tasks
    Magic mg_tpb;            // / band_tasks_per_batch
    Magic mg_uht;            // / uniform_head_tasks
    Magic mg_per_bh;         // / (n_split * n_ggroups)
    Magic mg_nsplit;         // / n_split
    Magic mg_H;              // / H
    int one_sided;           // 1: the window keeps the keys at or before the query
    const int32_t *rtab;     // random key blocks [H][ceil(T/64)][n_rand] (-1 = none), or null
    const uint32_t *gmap;    // bit j set iff position j is global ([ceil(T/32)] words), or null
    int n_rand;              // random key blocks (of 64 keys) per query block of 64
    int band_die[9];         // band_die[8] == 0: each die takes a contiguous eighth of the
                             // band tasks and of the global-row tasks; else die x takes band
                             // tasks [band_die[x], band_die[x+1]) and global-row tasks
                             // [glob_die[x], glob_die[x+1]) (numbered from 0)
    int glob_die[9];
    int bwd_globals_first;   // the backward kernels take a die's global tasks before its band tiles
    int head_start[LF_MAX_HEADS + 1];  // band-task prefix over heads
    int32_t dil[LF_MAX_HEADS];   // dilation delta_h
    int32_t rad[LF_MAX_HEADS];   // window radius per head (clamped to T)
    int32_t hq[LF_MAX_HEADS];    // T / delta_h: length of the shorter residue classes
    int32_t hrem[LF_MAX_HEADS];  // T % delta_h: classes 0 .. hrem-1 hold hq + 1 positions
    int32_t htb[LF_MAX_HEADS];   // tiles of a class of hq + 1 positions
    int32_t hts[LF_MAX_HEADS];   // tiles of a class of hq positions
    Magic mg_tb[LF_MAX_HEADS];   // / htb
    Magic mg_ts[LF_MAX_HEADS];   // / hts
    Magic mg_dil[LF_MAX_HEADS];  // / delta_h
    int32_t glob[LF_MAX_GLOBALS];
};

// Task decode for calls whose heads share one stride and one radius, carried
// in the kernel argument itself: a workgroup knows its tile after the one
// load of its arguments, instead of after a chain of dependent loads from
// the plan (its scalars, then the per-head tables).
struct FastDecode {
    int on;                  // 1: every head has stride delta and radius r (the fields below are set)
    int n_band, n_tasks;     // band tasks; band + global-row tasks
    int tph;                 // band tasks per (b, h)
    Magic mg_tph;            // / tph
    Magic mg_H;              // / H
    int H, T, delta, r, ra;
    int hq, hrem, htb, hts;  // class lengths and tiles per class (as in Plan)
    Magic mg_htb, mg_hts;
    int n_g, n_split, n_ggroups, split_len;
    Magic mg_per_bh, mg_nsplit;
};

// The kernel argument: the call's tensors and the device copy of its plan.
struct Args {
    const void *q, *k, *v;
    void *out;
    const uint8_t *pad;      // [B][T] or null
    const Plan *plan;
    float *lse;              // [B][H][T] natural log of each row's softmax denominator, or null
    int global_rows_only;    // 1: the grid holds the global-row tasks alone
    FastDecode fd;
};

// The argument of the matrix-core backward kernels (lf_bwd_mfma.hip): bf16
// tensors [B][H][T][64], the forward's output y and lse, the forward's plan
// (band tiles, radii, strides, global set, random key blocks) and the row
// statistics.
struct BwdBandArgs {
    const void *q, *k, *v, *dy;
    const void *y;           // the forward's output
    const float *lse;        // [B][H][T] its natural log-sum-exp (-inf for a padded row)
    void *dq, *dk, *dv;
    const uint8_t *pad;      // [B][T] or null
    const Plan *plan;
    float *stats;            // [B*H][T][2]: (lse * log2 e, D = dy . y); (+inf, 0) for a padded row,
                             // written by the dq kernel, read by the dk/dv and global-row kernels
    const uint32_t *gmap;    // bit j set iff position j is global ([ceil(T/32)] words)
    const int32_t *inv_off;  // random blocks: [H][ceil(T/64) + 1] offsets into inv_list per key block
    const int32_t *inv_list; // the query blocks that drew each key block, ascending
    // global tasks (the plan's global-row splits): partial records and
    // completion counters (zero between calls; the last task of a head
    // returns its counter to zero)
    float *part_q;           // [B*H][n_split][g_pad][64]: a split's part of a global row's dq
    float *part_kv;          // [B*H][n_split][g_pad][128]: a split's part of a global key's dk, dv
    int *count_q, *count_kv; // [B*H] each
};

}  // namespace lfk

#endif
