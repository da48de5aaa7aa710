// lf_bwd.h -- the launch record shared by the host code of lf_attn_bwd
// (lf_host.cpp) and the vector-unit backward kernels (lf_bwd_kernels.hip:
// fp32 input, and bf16 input at d = 32 and 128); bf16 input at d = 64 takes
// the matrix-core kernels of lf_bwd_mfma.hip, whose argument is in
// lf_kernels.h.  Internal to
// liblfattn.so; the public interface is include/lf_attn.h.
#ifndef LF_BWD_H
#define LF_BWD_H

#include <stdint.h>

#include <hip/hip_runtime.h>

#include "lf_attn.h"

// Lanes that share one row (query or key) in the backward's band kernels,
// 4, 8 or 16; a wave holds 64 / that many rows of one residue class, and
// head_chunk counts chunks of that many class positions.  These kernels
// serve fp32 inputs, the precision path, which is most used on small
// problems (and bf16 inputs at d = 32 and 128): there more lanes a row (more waves, fewer registers) measured
// faster (B = 1, H = 2, T = 1024, r = 64: 179 us at four, 140 at eight,
// 105 at sixteen, with the global-row statistics reduced across lanes),
// while on the T = 4096, r = 256 shape with 12 heads four were faster than
// eight (743 against 922 us).
#ifndef LFB_LANES_PER_ROW
#define LFB_LANES_PER_ROW 16
#endif
#define LFB_ROWS_PER_WAVE (64 / LFB_LANES_PER_ROW)

// The backward launches' argument (lf_bwd_kernels.hip).  The tables live in
// one device buffer of the workspace: radius, stride and wave-chunk prefix
// per head, the sorted global positions and their bitmap.
namespace lfk {

struct BwdArgs {
    const uint8_t *pad;          // [B][T] or null
    const uint32_t *gmap;        // bit i set iff position i is global ([ceil(T/32)] words)
    const int32_t *glob;         // [n_g] distinct globals, ascending
    const int32_t *rad;          // [H] window radius per head (clamped to T)
    const int32_t *dil;          // [H] stride per head
    const int32_t *head_chunk;   // [H+1] prefix of the class chunks (LFB_ROWS_PER_WAVE positions) over the heads
                                 // in the order hord lists them
    const int32_t *hord;         // [H] heads by decreasing radius: the longest waves are dealt out first
    void *stats;                 // float2 [B*H][T]: (log2-sum-exp of the scaled scores, D_i)
    float4 *gstat;               // [B*H*n_g][n_split]: a split's (max, sum, sum of p dP) of a global row
    float *gpart;                // [B*H*n_g][n_split][3 d]: a split's partial dq, dk, dv of a global position
    int B, H, T, n_g, one_sided;
    int n_chunks;                // head_chunk[H]: class chunks of one batch entry (the host's copy)
    int n_split, split_len;      // global rows and columns: splits of split_len positions (a multiple of 64)
    // random key blocks of 64 (undilated heads only), or n_rand = 0
    const int32_t *rtab;         // [H][ceil(T/64)][n_rand] key blocks per query block, ascending, -1 = none
    const int32_t *inv_off;      // [H][ceil(T/64) + 1] CSR offsets into inv_list per key block
    const int32_t *inv_list;     // query blocks that drew the key block, ascending
    int n_rand;
};

}  // namespace lfk

#endif
