"""Dense brute-force reference used to pin the oracle on tiny T.

It takes the "Mask View" reading of the method (Longformer, eightmm.github.io,
section "Mask View"): build the full T x T boolean matrix of allowed pairs
straight from the set definitions, put -inf on the disallowed scores and
run an ordinary dense softmax(QK^T/sqrt(d) + M)V in float64.  It shares no
code with the oracle (which walks each query's neighbour list instead).
"""
import numpy as np


def allowed_matrix(T, r, delta, globals_, pad_row, one_sided=False, rand_blocks=None):
    """A[i, j] = True iff key j is in N(i) (no padding applied to rows here).
    One-sided: the window keeps only keys at or before the query.
    rand_blocks: [ceil(T/64)][n] key blocks of 64 that every query of block
    i // 64 also sees (global rows see everything anyway)."""
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    dist = i - j
    local = (np.abs(dist) <= r * delta) & (dist % delta == 0)
    if one_sided:
        local &= dist >= 0
    g = np.zeros(T, dtype=bool)
    for x in globals_:
        g[x] = True
    if rand_blocks is not None:
        rb = np.zeros((T, T), dtype=bool)
        for i_ in range(T):
            for blk in np.asarray(rand_blocks)[i_ // 64]:
                rb[i_, 64 * int(blk):64 * int(blk) + 64] = True
        local = local | rb
    A = local | g[None, :] | g[:, None]   # every row sees G; global rows see all
    if pad_row is not None:
        A &= ~pad_row.astype(bool)[None, :]
    return A


def dense_masked_attention(q, k, v, r, dilation=None, globals_=(), pad=None, one_sided=False,
                           rand_blocks=None):
    """r: one radius, or a list with one radius per head; rand_blocks:
    [H][ceil(T/64)][n] or None."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, T, d = q.shape
    out = np.zeros_like(q)
    for b in range(B):
        pad_row = None if pad is None else np.asarray(pad[b]).astype(bool)
        for h in range(H):
            delta = 1 if dilation is None else int(dilation[h])
            rh = int(r) if np.isscalar(r) else int(r[h])
            A = allowed_matrix(T, rh, delta, globals_, pad_row, one_sided,
                               None if rand_blocks is None else rand_blocks[h])
            S = q[b, h] @ k[b, h].T / np.sqrt(d)
            S = np.where(A, S, -np.inf)
            rows_ok = A.any(axis=1)
            if pad_row is not None:
                rows_ok &= ~pad_row
            m = np.max(np.where(A, S, -np.inf), axis=1, keepdims=True)
            m = np.where(np.isfinite(m), m, 0.0)
            P = np.where(A, np.exp(S - m), 0.0)
            l = P.sum(axis=1, keepdims=True)
            y = (P @ v[b, h]) / np.where(l > 0, l, 1.0)
            y[~rows_ok] = 0.0
            out[b, h] = y
    return out


def dense_masked_lse(q, k, r, dilation=None, globals_=(), pad=None, one_sided=False, rand_blocks=None):
    """log sum_{j allowed} exp(q_i . k_j / sqrt(d)) per row from the same
    T x T mask, by numpy's logaddexp reduction; -inf for a padded query and
    for a row with no allowed key."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    B, H, T, d = q.shape
    out = np.full((B, H, T), -np.inf)
    for b in range(B):
        pad_row = None if pad is None else np.asarray(pad[b]).astype(bool)
        for h in range(H):
            delta = 1 if dilation is None else int(dilation[h])
            rh = int(r) if np.isscalar(r) else int(r[h])
            A = allowed_matrix(T, rh, delta, globals_, pad_row, one_sided,
                               None if rand_blocks is None else rand_blocks[h])
            S = np.where(A, q[b, h] @ k[b, h].T / np.sqrt(d), -np.inf)
            lse = np.logaddexp.reduce(S, axis=1) if T else np.zeros(0)
            if pad_row is not None:
                lse[pad_row] = -np.inf
            out[b, h] = lse
    return out
