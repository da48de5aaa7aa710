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
// 4, 8 or 16, chosen per call (BwdArgs::lpr); a wave holds 64 / that many
// rows of one residue class, and head_chunk counts chunks of that many class
// positions.  These kernels serve fp32 inputs, the precision path (and bf16
// inputs at d = 32 and 128).  Fewer lanes a row means fewer waves, each
// holding more channels in registers.  Measured on B = 1, H = 12, T = 4096,
// r = 256 (one global): fp32 d = 64 1042 us at eight, 1270 at sixteen,
// 1658 at four (176 registers); fp32 d = 128 1741 at sixteen, 2812 at eight; fp32 d = 32 536
// at four, 1220 at sixteen; bf16 d = 128 1312 at eight, 1577 at sixteen.
// So the host takes the fewest lanes that leave each lane 8 fp32 or 16 bf16
// channels (four at the least), and doubles them while that would make
// fewer than LFB_MIN_WAVES waves: small problems want more waves (B = 1,
// H = 2, T = 1024, r = 64, fp32: 179 us at four, 140 at eight, 105 at
// sixteen).
#define LFB_MIN_WAVES 2048

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
    const int32_t *head_chunk;   // [H+1] prefix of the class chunks (64 / lpr positions) over the heads
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
    int lpr;                     // lanes per row of the band kernels: 4, 8 or 16
};

}  // namespace lfk

#endif
