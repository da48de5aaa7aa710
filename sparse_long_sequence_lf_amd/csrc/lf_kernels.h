// lf_kernels.h -- the launch record shared by the host planner
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
// Register budget: waves per SIMD the tile kernel is compiled for (three
// workgroups of four waves per compute unit).
#ifndef LFK_WAVES_PER_EU
#define LFK_WAVES_PER_EU 3
#endif

namespace lfk {

// Passed by value as the kernel argument (fits the 4 KiB kernarg limit).
struct Params {
    const void *q, *k, *v;
    const void *kp, *vp;     // K and V as bf16 planes: [B*H][T][NP][64] (bf16 input: k and v)
    void *out;
    const uint8_t *pad;      // [B][T] or null
    float *part;             // global-row partials [B*H][n_split][g_pad][66]
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
    uint16_t dil[LF_MAX_HEADS];
    int32_t glob[LF_MAX_GLOBALS];
};

}  // namespace lfk

#endif
