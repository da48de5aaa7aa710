/*
 * lf_attn.h -- C ABI of liblfattn.so: the Longformer sparse self-attention
 * forward pass (sliding window, optional per-head dilation, global tokens,
 * key padding) on AMD Instinct MI355X (gfx950).
 *
 * What is computed (Longformer, eightmm.github.io/papers/architectures/
 * longformer, sections "Sliding-Window Attention", "Global Attention" and
 * "Mask View"), with 0-based positions:
 *
 *   N_local(i) = { j : |i - j| <= r * delta_h  and  (i - j) mod delta_h == 0 }
 *   N(i)       = N_local(i) U G           for i not in G   (set union)
 *   N(i)       = { 0 .. T-1 }              for i in G
 *   keys j with key_padding_mask[b][j] != 0 are removed from every N(i);
 *   y_i = sum_{j in N(i)} softmax_j( q_i . k_j / sqrt(d) ) v_j ;
 *   a query row i with key_padding_mask[b][i] != 0 is written as zeros.
 *
 * The dilated window follows Longformer (ciallo.wiki) section 2.2.3 and
 * "Longformer长序列处理" (aiqz.cc), section 膨胀窗口设计: the window's keys
 * sit delta apart, the count stays 2r+1 and the reach grows delta-fold.
 * Positions that fall outside [0, T) are dropped ("Longformer长序列处理",
 * Python 演示, note 3).
 *
 * Thread safety: every call may come from any thread.  Calls on the same
 * stream are ordered by the stream; calls on different streams use separate
 * workspaces.  The same inputs give a bit-identical output (no atomics touch
 * data).
 */
#ifndef LF_ATTN_H
#define LF_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and out. */
typedef enum {
    LF_F32 = 0,  /* IEEE binary32.  Each product is taken on the bf16 matrix cores from
                    three bf16 parts per operand (hi + mid + lo carry all 24 significand
                    bits), adding the six part products down to 2^-16 of the leading
                    one, with fp32 accumulation: the error stays that of fp32 arithmetic
                    (scores of a few hundred included). */
    LF_BF16 = 1  /* bfloat16; fp32 accumulation; out rounded to nearest-even */
} lf_dtype_t;

typedef enum {
    LF_OK = 0,
    LF_E_INVALID = 1,     /* an argument breaks the contract below; nothing was enqueued */
    LF_E_UNSUPPORTED = 2, /* valid but outside what the library implements; nothing enqueued */
    LF_E_NOMEM = 3,       /* the workspace could not be allocated; nothing enqueued */
    LF_E_HIP = 4          /* a HIP runtime call or kernel launch failed */
} lf_status_t;

/* Limits of the library (LF_E_UNSUPPORTED beyond them). */
#define LF_HEAD_DIM 64        /* d of the matrix-core backward (bf16); every call takes any of LF_FWD_HEAD_DIMS */
#define LF_FWD_HEAD_DIMS {32, 64, 128}
#define LF_MAX_HEADS 128      /* H */
#define LF_MAX_GLOBALS 512    /* distinct global positions */
#define LF_MAX_SEQ ((1 << 24) - 1)  /* T: one head of fp32 K or V stays below 4 GiB */
#define LF_MAX_DILATION 65535 /* delta */
#define LF_MAX_RAND_BLOCKS 8  /* random key blocks per query block (lf_attn_fwd_ex) */
#define LF_NOALLOC_SCRATCH_BYTES (64 << 20) /* device workspace of lf_attn_fwd_noalloc, per GPU */

/*
 * lf_attn_fwd -- enqueue the forward pass on `stream`.
 *
 *   q, k, v   DEVICE pointers, each [B][H][T][d] contiguous row-major in
 *             `dtype`, 16-byte aligned.  Read only.
 *   B, H, T   batch, heads, sequence length; each >= 1 (T <= LF_MAX_SEQ,
 *             H <= LF_MAX_HEADS).
 *   d         head dimension: 32, 64 or 128 (the 1/sqrt(d) scale follows it).
 *             One head of q, k or v (T * d elements) must stay below 2 GiB,
 *             and below 2 GiB / 1.5 for fp32 (its three bf16 planes).
 *   r         one-sided window radius in window steps, r >= 0; the window
 *             holds 2r+1 keys away from the sequence ends.  r >= T means
 *             every key of the (dilated) class.
 *   dilation  HOST array [H] of per-head strides delta_h >= 1, or NULL for
 *             all 1.  Read during the call only.
 *   global_idx HOST array [n_global] of 0-based positions in [0, T); any
 *             order; duplicates are allowed and count once.  May be NULL
 *             when n_global == 0.  Read during the call only.
 *   n_global  >= 0; at most LF_MAX_GLOBALS distinct positions.
 *   key_padding_mask DEVICE array [B][T] of bytes, nonzero = padded, or
 *             NULL for no padding.  Any alignment.
 *   out       DEVICE pointer [B][H][T][d] in `dtype`, 16-byte aligned,
 *             must not overlap q, k or v.  Every element is written.
 *   dtype     LF_F32 or LF_BF16.
 *   stream    a hipStream_t (NULL = the null stream).  All work is enqueued
 *             there asynchronously; the call returns before it finishes.
 *
 * Ownership: the caller owns every buffer; the library keeps no pointer
 * after returning.  The library keeps one device workspace per (device,
 * stream) pair: global-row partials, the call's plan and tables (a few
 * configurations at once, so that calls alternating between them reuse
 * them).  A call never waits for the device: a plan or table it lacks is
 * written by a kernel on `stream`, and a buffer it outgrows is replaced
 * with hipMalloc, the old one freed once the stream has passed its last
 * use.  During stream capture nothing is allocated: a call that would
 * have to grow the workspace, or that needs a new plan slot after earlier
 * captures took every free one, is LF_E_UNSUPPORTED (make one identical
 * call on the stream outside capture first).  What a captured call uses
 * stays reserved for the graph until the process exits; later calls get
 * new slots and buffers instead.  A graph shares its stream's
 * workspace: do not replay it concurrently with calls on that stream or
 * with another replay of a graph captured on it (the global-row partials
 * and counters would race).
 *
 * Errors: all argument checks run before any HIP call; on LF_E_INVALID or
 * LF_E_UNSUPPORTED nothing is enqueued and `out` is untouched.  On any
 * non-OK status lf_last_error() describes the cause.
 */
lf_status_t lf_attn_fwd(const void *q, const void *k, const void *v,
                        int B, int H, int T, int d, int r,
                        const int32_t *dilation,
                        const int32_t *global_idx, int n_global,
                        const uint8_t *key_padding_mask,
                        void *out, lf_dtype_t dtype, void *stream);

/*
 * lf_attn_fwd_ex -- lf_attn_fwd with one window radius per head, a choice
 * of two-sided or one-sided windows, and random key blocks.
 *
 * The window list of "Longformer长序列处理" (section HF实践: one window per
 * layer, given as an int or a list) applied per head of one call; the one-
 * or two-sided question of Longformer (eightmm.github.io), section
 * "Implementation Reading"; and BigBird's random attention as the pages set
 * it beside Longformer (the mhpn.cn guide to long-text models, §2.2.1 and
 * §2.2.2: each token also attends to randomly chosen tokens, in blocks of
 * block_size, usually 64).
 *
 *   radius    HOST array [H] of radii r_h >= 0 (must not be NULL); head h
 *             uses r_h where lf_attn_fwd uses r.  Read during the call only.
 *   one_sided 0: the window of query i holds the class keys j with
 *             |i - j| <= r_h delta_h (as lf_attn_fwd).  1: only those with
 *             0 <= i - j <= r_h delta_h, the query and the keys before it.
 *             Global rows and global keys are the same in both cases (a
 *             global row sees every valid key; every row sees the globals).
 *   rand_blocks HOST array [H][ceil(T/64)][n_rand] of key-block indices in
 *             [0, ceil(T/64)), or NULL when n_rand == 0: a non-global query
 *             i of head h also attends to the valid keys of positions
 *             [64 b, 64 b + 64) for every b in rand_blocks[h][i / 64]
 *             (a set union with the window and the globals: each key counts
 *             once; a block listed twice counts once).  The caller draws
 *             them.  Read during the call only.
 *   n_rand    random key blocks per query block, 0 .. LF_MAX_RAND_BLOCKS;
 *             with n_rand > 0 every head must be undilated (delta = 1), else
 *             LF_E_UNSUPPORTED.
 *   lse       DEVICE float [B][H][T], 4-byte aligned, or NULL: when given,
 *             row i receives log(sum_{j in N(i)} exp(q_i . k_j / sqrt(d))),
 *             the natural log of its softmax denominator (the statistic a
 *             backward pass needs to rebuild the weights); -inf for a padded
 *             query row.  Must not overlap the other tensors.
 *   All other arguments, the ownership and the error behaviour are those
 *   of lf_attn_fwd; one_sided outside {0, 1}, a negative radius or n_rand,
 *   or a block index out of range is LF_E_INVALID.
 */
lf_status_t lf_attn_fwd_ex(const void *q, const void *k, const void *v,
                           int B, int H, int T, int d,
                           const int32_t *radius, int one_sided,
                           const int32_t *rand_blocks, int n_rand,
                           const int32_t *dilation,
                           const int32_t *global_idx, int n_global,
                           const uint8_t *key_padding_mask,
                           void *out, float *lse, lf_dtype_t dtype, void *stream);

/*
 * lf_attn_fwd_noalloc -- lf_attn_fwd for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc.  Same arguments, result and error behaviour as
 * lf_attn_fwd; the call itself performs no allocation (no hipMalloc, no
 * hipFree, no allocating library routine) and no host-to-device copy.
 *
 * Its workspace (the plan, the global-row completion counters and partial
 * records, and for fp32 inputs the three bf16 planes of K and V) is one
 * file-scope device array of LF_NOALLOC_SCRATCH_BYTES that every GPU the
 * library runs on holds until the process exits.  A call whose workspace
 * would exceed it returns LF_E_UNSUPPORTED before any HIP call (the needed
 * size grows with B*H*T*d for fp32 inputs and with B*H*n_global*T for
 * globals).  The plan reaches the GPU as kernel arguments of small copy
 * launches on `stream`, which also clear the counters, so the call can be
 * captured into a graph, also with a plan that differs from the last call.
 *
 * Every call on one GPU uses that GPU's single array: calls that overlap in
 * time on one GPU (on different streams, or concurrent graph replays) race
 * and may corrupt each other's results; order them on one stream.
 */
lf_status_t lf_attn_fwd_noalloc(const void *q, const void *k, const void *v,
                                int B, int H, int T, int d, int r,
                                const int32_t *dilation,
                                const int32_t *global_idx, int n_global,
                                const uint8_t *key_padding_mask,
                                void *out, lf_dtype_t dtype, void *stream);

/*
 * lf_attn_fwd_global_rows -- only the global rows of lf_attn_fwd: for every
 * (b, h) and every i in G, out[b][h][i] (and lse[b][h][i] when lse is not
 * NULL) as lf_attn_fwd and lf_attn_fwd_ex write them.  A global row attends
 * to every valid key (Longformer, eightmm.github.io, "Global Attention";
 * the N(i) = { 0 .. T-1 } case above), so no window, dilation, side or
 * random-block argument applies.  Every other row of out and lse is left as
 * it was.  For a caller that needs the global tokens' outputs alone, such as
 * a classification head reading the first token of the last layer.
 *
 *   q, k, v, B, H, T, d, global_idx, n_global, key_padding_mask, dtype,
 *   stream: as lf_attn_fwd.  n_global == 0 enqueues nothing.
 *   out       DEVICE pointer [B][H][T][d] in `dtype`; only the rows at the
 *             global positions are written.
 *   lse       DEVICE pointer [B][H][T] of floats, or NULL: as lf_attn_fwd_ex,
 *             at the global positions only.
 *   Ownership, workspace and errors: as lf_attn_fwd.
 */
lf_status_t lf_attn_fwd_global_rows(const void *q, const void *k, const void *v,
                                    int B, int H, int T, int d,
                                    const int32_t *global_idx, int n_global,
                                    const uint8_t *key_padding_mask,
                                    void *out, float *lse, lf_dtype_t dtype, void *stream);

/* Text describing the last non-OK status returned on the calling thread
 * (empty string if none).  The pointer stays valid until the next call on
 * this thread. */
const char *lf_last_error(void);

/* A hash of the sources this library was built from (16 hex digits), so
 * that a loader can refuse a build older than the sources beside it. */
const char *lf_build_hash(void);

/*
 * lf_attn_bwd -- enqueue the gradients of the forward pass on `stream`.
 *
 * The pages give no backward pass; Longformer (ciallo.wiki) §5.2 only says
 * that training cost grows linearly with the length.  This is the
 * derivative of the forward of lf_attn_fwd_ex over the same allowed pairs:
 * with P_ij the softmax weights of row i, dP_ij = dy_i . v_j,
 * D_i = sum_j P_ij dP_ij (= dy_i . y_i, y the forward's output) and
 * dS_ij = P_ij (dP_ij - D_i):
 *     dq_i = sum_j dS_ij k_j / sqrt(d),   dk_j = sum_i dS_ij q_i / sqrt(d),
 *     dv_j = sum_i P_ij dy_i.
 *
 *   q, k, v   DEVICE [B][H][T][d] of `dtype`, the forward's inputs; d one
 *             of LF_FWD_HEAD_DIMS (32, 64, 128).
 *   dy        DEVICE [B][H][T][d] of `dtype`: the gradient of the loss with
 *             respect to the forward's output.  Rows of padded queries are
 *             ignored (their output is zero whatever q holds).
 *   radius, one_sided, rand_blocks, n_rand, dilation, global_idx, n_global,
 *   key_padding_mask: as lf_attn_fwd_ex (radius, rand_blocks are HOST arrays).
 *   dq, dk, dv DEVICE [B][H][T][d] of `dtype`, written in full (zero rows
 *             at padded positions).  They must not overlap one another or
 *             the inputs.
 *
 * bf16 inputs at d = 64 run on the matrix cores: the weights come from the
 * forward's per-row log-sum-exp, which lf_attn_bwd obtains by running the
 * forward into its workspace first (lf_attn_bwd_ex takes the caller's
 * instead).  Products of bf16 values accumulate in fp32; the weights P and
 * the dS_ij enter the products over rows as bf16 (rounded to nearest even),
 * and D_i is taken from the bf16 output y.  fp32 inputs (every d) and bf16
 * inputs at d = 32 and 128 run on the vector units in fp32 arithmetic,
 * recomputing each row's statistics (bf16 products are exact in fp32; in
 * the sums over rows of dk and dv a bf16 row is scaled by its weight
 * rounded to bf16).  Results are rounded
 * to `dtype` (bf16 to nearest even).  Every result is written by exactly
 * one thread, without atomics: repeated calls give the same bits.
 * Ownership and errors as lf_attn_fwd: all checks run before any HIP
 * call; LF_E_INVALID / LF_E_UNSUPPORTED enqueue nothing.  The call keeps
 * a per-(device, stream) workspace (row statistics, 8 bytes per query
 * row, its tables, and for lf_attn_bwd on bf16 the forward's output and
 * lse); a change of shape, radii, dilation or globals or random key
 * blocks during stream capture is LF_E_UNSUPPORTED.
 */
lf_status_t lf_attn_bwd(const void *q, const void *k, const void *v, const void *dy,
                        int B, int H, int T, int d, const int32_t *radius, int one_sided,
                        const int32_t *rand_blocks, int n_rand, const int32_t *dilation,
                        const int32_t *global_idx, int n_global, const uint8_t *key_padding_mask,
                        void *dq, void *dk, void *dv, lf_dtype_t dtype, void *stream);

/*
 * lf_attn_bwd_ex -- lf_attn_bwd with the forward's results supplied.
 *
 *   out       DEVICE [B][H][T][d] of `dtype`, 16-byte aligned: the output of
 *             lf_attn_fwd_ex for the same inputs and arguments.
 *   lse       DEVICE [B][H][T] floats, 4-byte aligned: that call's lse.
 * Both given or both NULL (NULL: as lf_attn_bwd).  With bf16 inputs at
 * d = 64 they replace the forward pass lf_attn_bwd would run; the vector-unit
 * path (fp32, bf16 at d = 32 or 128) does not read them.  Neither may overlap dq, dk or dv.  Other arguments as lf_attn_bwd.
 */
lf_status_t lf_attn_bwd_ex(const void *q, const void *k, const void *v, const void *dy,
                           const void *out, const float *lse,
                           int B, int H, int T, int d, const int32_t *radius, int one_sided,
                           const int32_t *rand_blocks, int n_rand, const int32_t *dilation,
                           const int32_t *global_idx, int n_global, const uint8_t *key_padding_mask,
                           void *dq, void *dk, void *dv, lf_dtype_t dtype, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LF_ATTN_H */
