// lf_kernels.h -- the launch records shared by the host planner
// (lf_host.cpp) and the gfx950 kernels (lf_attn_kernels.hip).  Internal to
// liblfattn.so; the public interface is include/lf_attn.h.
#ifndef LF_KERNELS_H
#define LF_KERNELS_H

#include <stdint.h>

#include "lf_attn.h"

// Tile shape: LFK_QB query blocks of 32 per workgroup, LFK_KS key phases
// per query block (waves per workgroup = LFK_QB * LFK_KS = 4).
#define LFK_QB 2
#define LFK_KS 2
// Register budget: waves per SIMD the tile kernel is compiled for, one per
// workgroup of four waves resident on a compute unit (bf16: four workgroups,
// as many as its LDS allows; fp32 inputs double the LDS and the registers).
#ifndef LFK_WAVES_PER_EU_BF16
#define LFK_WAVES_PER_EU_BF16 4
#endif
#ifndef LFK_WAVES_PER_EU_F32
#define LFK_WAVES_PER_EU_F32 2
#endif

namespace lfk {

// Everything about a call except the tensors: shape, per-head tables, the
// global set and workspace pointers.  Lives in device memory (one copy per
// (device, stream) workspace), re-uploaded only when it changes, so the
// kernel argument stays small (launch cost grows with argument size).
struct Plan {
    const void *kp, *vp;     // K and V as bf16 planes [B*H][T][2][64] (fp32 input only)
    float *part;             // global-row partials [B*H][n_split][g_pad] x 272 B: O[64], m, l, 0, 0
    int *counter;            // [B*H] finished global-row workgroups; zero between calls
    int B, H, T, r;          // r already clamped to T
    int n_g;                 // distinct globals (sorted ascending in glob)
    int g_pad;               // n_ggroups * 32 * LFK_QB
    int n_ggroups;           // groups of 32*LFK_QB global queries
    int n_split, split_len;  // global-row key splits (split_len multiple of 32)
    int n_band_tasks;        // B * band_tasks_per_batch
    int band_tasks_per_batch;
    int uniform_head_tasks;  // band tasks per head when every head has the same count, else 0
    int n_tasks;             // band + global-row tasks
    int head_start[LF_MAX_HEADS + 1];  // band-task prefix over heads
    int32_t dil[LF_MAX_HEADS];      // 32-bit: a head's entry is one scalar load
    int32_t rad[LF_MAX_HEADS];      // window radius per head (clamped to T)
    int one_sided;                  // 1: the window keeps the keys at or before the query
    const int32_t *rtab;            // random key blocks [H][ceil(T/64)][n_rand] (-1 = none), or null
    const uint32_t *gmap;           // bit j set iff position j is global ([ceil(T/32)] words), or null
    int n_rand;                     // random key blocks (of 64 keys) per query block of 64
    int band_chunk;                 // 0: each die takes a contiguous eighth of the band tiles;
                                    // C > 0: runs of C tiles are dealt to the dies in turn
    int32_t glob[LF_MAX_GLOBALS];
};

// The kernel argument: the call's tensors and the device copy of its plan.
struct Args {
    const void *q, *k, *v;
    void *out;
    const uint8_t *pad;      // [B][T] or null
    const Plan *plan;
};

}  // namespace lfk

#endif
