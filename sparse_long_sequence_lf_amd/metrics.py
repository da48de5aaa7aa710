"""Useful work of one forward call: the number of (query, key) pairs the
softmax runs over, and the FLOPs and bytes derived from it.

Useful FLOPs = 4 * d * sum_i |N(i)|: 2d for the q.k dot product and 2d for
the weighted sum of v, per allowed pair, following the O(T w d_k) cost
statement of Longformer (eightmm.github.io), "Sliding-Window Attention", and
its "Relation to Dense Attention" table (local O(Tw), global O(Tg)).  Masked
or padded pairs, tile padding and softmax arithmetic are not counted.

The count is closed-form per row (prefix sums over each dilation residue
class), vectorised with numpy; it never enumerates the pairs.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np


def pair_counts(B: int, H: int, T: int, r, dilation: Optional[Sequence[int]] = None,
                global_idx: Optional[Sequence[int]] = None, key_padding_mask=None,
                one_sided: bool = False, random_blocks=None) -> np.ndarray:
    """|N(i)| for every row, as an int64 array [B, H, T] (padded rows give 0).
    ``r`` is one radius or one per head; ``one_sided`` windows keep only the
    keys at or before the query; ``random_blocks`` [H][ceil(T/64)][n] adds
    to each query of block i // 64 the valid keys of those key blocks of 64
    (heads with random blocks are undilated)."""
    G = np.unique(np.asarray(list(global_idx) if global_idx is not None else [], dtype=np.int64))
    if key_padding_mask is None:
        valid = np.ones((B, T), dtype=bool)
    else:
        m = key_padding_mask
        if hasattr(m, "detach"):
            m = m.detach().cpu().numpy()
        valid = np.asarray(m) == 0
    out = np.zeros((B, H, T), dtype=np.int64)
    is_g = np.zeros(T, dtype=bool)
    is_g[G] = True
    for b in range(B):
        vb = valid[b]
        n_valid = int(vb.sum())
        Gv = G[vb[G]] if G.size else G          # globals that are real (unpadded) keys
        for h in range(H):
            delta = int(dilation[h]) if dilation is not None else 1
            rb = int(r) if np.isscalar(r) else int(r[h])   # reach back
            ra = 0 if one_sided else rb                    # reach forward
            cnt = np.zeros(T, dtype=np.int64)
            for c in range(min(delta, T)):
                pos = np.arange(c, T, delta)
                n = pos.size
                pre = np.concatenate([[0], np.cumsum(vb[pos].astype(np.int64))])
                m_ = np.arange(n)
                lo = np.maximum(0, m_ - rb)
                hi = np.minimum(n, m_ + ra + 1)
                win = pre[hi] - pre[lo]                  # valid keys of the window
                # valid globals not already inside the window: add |Gv| and take
                # back one for every window that contains a valid global of class c
                extra = np.full(n, Gv.size, dtype=np.int64)
                gc = Gv[(Gv - c) % delta == 0] if Gv.size else Gv
                if gc.size:
                    diff = np.zeros(n + 1, dtype=np.int64)
                    mg = (gc - c) // delta
                    # key mg is in the window of the queries m in [mg - ra, mg + rb]
                    np.add.at(diff, np.maximum(0, mg - ra), -1)
                    np.add.at(diff, np.minimum(n, mg + rb + 1), 1)
                    extra += np.cumsum(diff[:-1])
                cnt[pos] = win + extra
            if random_blocks is not None and np.asarray(random_blocks).shape[2] > 0:
                cnt += _random_extra(T, rb, ra, vb, is_g, np.asarray(random_blocks)[h])
            cnt[is_g] = n_valid                          # global rows read every valid key
            cnt[~vb] = 0                                 # padded rows are zero rows
            out[b, h] = cnt
    return out


def _random_extra(T, rb, ra, vb, is_g, blocks):
    """Per row: the valid keys of the row's random blocks that are neither in
    its window [i - rb, i + ra] nor global (those are counted already)."""
    pv = np.concatenate([[0], np.cumsum(vb.astype(np.int64))])            # valid keys
    pg = np.concatenate([[0], np.cumsum((vb & is_g).astype(np.int64))])   # valid globals
    i = np.arange(T)
    w_lo = np.maximum(0, i - rb)
    w_hi = np.minimum(T, i + ra + 1)
    extra = np.zeros(T, dtype=np.int64)
    qb = i // 64
    for e in range(blocks.shape[1]):
        blk = blocks[qb, e].astype(np.int64)
        # a block drawn twice for one query block counts once
        dup = np.zeros(T, dtype=bool)
        for e2 in range(e):
            dup |= blocks[qb, e2] == blocks[qb, e]
        lo = np.minimum(T, 64 * blk)
        hi = np.minimum(T, 64 * blk + 64)
        ilo = np.maximum(lo, w_lo)
        ihi = np.maximum(ilo, np.minimum(hi, w_hi))                       # block cut by the window
        add = (pv[hi] - pv[lo]) - (pv[ihi] - pv[ilo]) - ((pg[hi] - pg[lo]) - (pg[ihi] - pg[ilo]))
        extra += np.where(dup, 0, add)
    return extra


def useful_pairs(*args, **kw) -> int:
    return int(pair_counts(*args, **kw).sum())


def useful_flops(B, H, T, d, r, dilation=None, global_idx=None, key_padding_mask=None) -> int:
    return 4 * d * useful_pairs(B, H, T, r, dilation, global_idx, key_padding_mask)


def algorithmic_bytes(B, H, T, d, esize, key_padding_mask=None) -> int:
    """Compulsory HBM traffic of one call: q, k, v read once, out written once
    (plus the padding mask bytes)."""
    n = B * H * T * d * esize
    return 4 * n + (0 if key_padding_mask is None else B * T)
