"""ctypes front of the fp64 CPU oracle (oracle/lf_oracle.c).

TEST INFRASTRUCTURE: only the test suite, the smoke check and the CPU
baseline leg of the benchmark import this package.  The product path never
does.  Inputs may be torch tensors or numpy arrays; q/k/v are passed as
float32 (exact for bf16 and fp32 data) and results come back as float64.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "liblforacle.so")
_lib = None


def open_library(path):
    """Load an oracle build at ``path`` and declare its C signatures."""
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    I = ctypes.c_int
    LL = ctypes.c_longlong
    lib.lf_oracle_fwd.argtypes = [P, P, P, I, I, I, I, I, P, P, I, P, P, I]
    lib.lf_oracle_fwd.restype = I
    lib.lf_oracle_rows.argtypes = [P, P, P, I, I, I, I, I, P, P, I, P, P, LL, P, I]
    lib.lf_oracle_rows.restype = I
    lib.lf_oracle_neighbours.argtypes = [I, I, I, P, I, P, I, P]
    lib.lf_oracle_neighbours.restype = I
    lib.lf_oracle_count_pairs.argtypes = [I, I, I, I, P, P, I, P]
    lib.lf_oracle_count_pairs.restype = LL
    lib.lf_oracle_fwd2.argtypes = [P, P, P, I, I, I, I, I, P, I, P, I, P, P, I, P, P, I]
    lib.lf_oracle_fwd2.restype = I
    lib.lf_oracle_rows2.argtypes = [P, P, P, I, I, I, I, I, P, I, P, I, P, P, I, P, P, LL, P, I]
    lib.lf_oracle_rows2.restype = I
    lib.lf_oracle_neighbours2.argtypes = [I, I, I, I, P, I, P, I, P, I, P]
    lib.lf_oracle_neighbours2.restype = I
    lib.lf_oracle_count_pairs2.argtypes = [I, I, I, I, P, I, P, I, P, P, I, P]
    lib.lf_oracle_count_pairs2.restype = LL
    lib.lf_oracle_fwd_lse.argtypes = [P, P, P, I, I, I, I, I, P, I, P, I, P, P, I, P, P, P, I]
    lib.lf_oracle_fwd_lse.restype = I
    lib.lf_oracle_bwd.argtypes = [P, P, P, P, I, I, I, I, I, P, I, P, I, P, P, I, P, P, P, P, I]
    lib.lf_oracle_bwd.restype = I
    lib.lf_oracle_bwd_rows.argtypes = [P, P, P, P, I, I, I, I, I, P, I, P, I, P, P, I, P, P, LL, P, I]
    lib.lf_oracle_bwd_rows.restype = I
    lib.lf_oracle_bwd_keys.argtypes = [P, P, P, P, I, I, I, I, I, P, I, P, I, P, P, I, P, P, LL, P, P, I]
    lib.lf_oracle_bwd_keys.restype = I
    return lib


def _built_hash(path):
    """The source hash recorded beside an oracle build, or None."""
    try:
        with open(path + ".hash") as f:
            return f.read().strip()
    except OSError:
        return None


def _load():
    """The oracle library, (re)built with gcc when it is missing or was built
    from another version of lf_oracle.c."""
    global _lib
    if _lib is None:
        from . import build as _b
        if not os.path.exists(_LIB_PATH) or _built_hash(_LIB_PATH) != _b.source_hash():
            _b.build()
        _lib = open_library(_LIB_PATH)
    return _lib


def _f32(x):
    if hasattr(x, "detach"):
        x = x.detach().cpu().float().numpy()
    return np.ascontiguousarray(np.asarray(x, dtype=np.float32))


def _i32(x, n=None):
    if x is None:
        return None
    a = np.ascontiguousarray(np.asarray(list(x) if not isinstance(x, np.ndarray) else x, dtype=np.int32))
    return a


def _u8(x):
    if x is None:
        return None
    if hasattr(x, "detach"):
        x = x.detach().cpu().numpy()
    return np.ascontiguousarray((np.asarray(x) != 0).astype(np.uint8))


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


RAND_BLOCK = 64


def _rand_blocks(rb, H, T):
    """(array, n_rand): the random key blocks [H][ceil(T/64)][n_rand] or (None, 0)."""
    if rb is None:
        return None, 0
    a = np.ascontiguousarray(np.asarray(rb, dtype=np.int32))
    nqb = (T + RAND_BLOCK - 1) // RAND_BLOCK
    if a.ndim != 3 or a.shape[0] != H or a.shape[1] != nqb:
        raise ValueError("random blocks must be [H][ceil(T/64)][n_rand]")
    return a, int(a.shape[2])


def _radius(r, H):
    """(scalar r, per-head array or None): r is an int, or one radius per head."""
    if isinstance(r, (int, np.integer)):
        return int(r), None
    rad = _i32(r)
    if rad.size != H:
        raise ValueError("one radius per head")
    return int(rad.max()) if rad.size else 0, rad


def fwd(q, k, v, r, dilation=None, global_idx=None, key_padding_mask=None, n_threads=0,
        return_threads=False, lib=None, one_sided=False, random_blocks=None):
    """Full forward in fp64: returns out[B][H][T][d] (numpy float64).  ``r``
    is one radius or one per head; ``one_sided`` keeps only the keys at or
    before each query in its window; ``random_blocks`` [H][ceil(T/64)][n]
    lists the key blocks of 64 each query block of 64 also attends to."""
    lib = lib or _load()
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    B, H, T, d = qf.shape
    r0, rad = _radius(r, H)
    rb, nr = _rand_blocks(random_blocks, H, T)
    dil = _i32(dilation)
    g = _i32(global_idx if global_idx is not None else [])
    pad = _u8(key_padding_mask)
    out = np.zeros((B, H, T, d), dtype=np.float64)
    nt = lib.lf_oracle_fwd2(_ptr(qf), _ptr(kf), _ptr(vf), B, H, T, d, r0, _ptr(rad), int(bool(one_sided)),
                            _ptr(rb), nr, _ptr(dil), _ptr(g), int(g.size), _ptr(pad), _ptr(out), int(n_threads))
    if nt < 0:
        raise ValueError("oracle rejected its arguments")
    return (out, nt) if return_threads else out


def fwd_lse(q, k, v, r, dilation=None, global_idx=None, key_padding_mask=None, n_threads=0, lib=None,
            one_sided=False, random_blocks=None):
    """The forward and each row's log-sum-exp (natural log of its softmax
    denominator over N(i); -inf for a padded query): (out, lse), numpy
    float64 [B][H][T][d] and [B][H][T]."""
    lib = lib or _load()
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    B, H, T, d = qf.shape
    r0, rad = _radius(r, H)
    rb, nr = _rand_blocks(random_blocks, H, T)
    dil = _i32(dilation)
    g = _i32(global_idx if global_idx is not None else [])
    pad = _u8(key_padding_mask)
    out = np.zeros((B, H, T, d), dtype=np.float64)
    lse = np.zeros((B, H, T), dtype=np.float64)
    nt = lib.lf_oracle_fwd_lse(_ptr(qf), _ptr(kf), _ptr(vf), B, H, T, d, r0, _ptr(rad), int(bool(one_sided)),
                               _ptr(rb), nr, _ptr(dil), _ptr(g), int(g.size), _ptr(pad), _ptr(out), _ptr(lse),
                               int(n_threads))
    if nt < 0:
        raise ValueError("oracle rejected its arguments")
    return out, lse


def bwd(q, k, v, dy, r, dilation=None, global_idx=None, key_padding_mask=None, n_threads=0,
        lib=None, one_sided=False, random_blocks=None):
    """Gradients of the forward for the upstream gradient ``dy`` [B][H][T][d]:
    returns (dq, dk, dv), numpy float64, same arguments as ``fwd``."""
    lib = lib or _load()
    qf, kf, vf, dyf = _f32(q), _f32(k), _f32(v), _f32(dy)
    B, H, T, d = qf.shape
    if dyf.shape != qf.shape:
        raise ValueError("dy must have the shape of q")
    r0, rad = _radius(r, H)
    rb, nr = _rand_blocks(random_blocks, H, T)
    dil = _i32(dilation)
    g = _i32(global_idx if global_idx is not None else [])
    pad = _u8(key_padding_mask)
    dq, dk, dv = (np.zeros((B, H, T, d), dtype=np.float64) for _ in range(3))
    nt = lib.lf_oracle_bwd(_ptr(qf), _ptr(kf), _ptr(vf), _ptr(dyf), B, H, T, d, r0, _ptr(rad),
                           int(bool(one_sided)), _ptr(rb), nr, _ptr(dil), _ptr(g), int(g.size), _ptr(pad),
                           _ptr(dq), _ptr(dk), _ptr(dv), int(n_threads))
    if nt < 0:
        raise ValueError("oracle rejected its arguments")
    return dq, dk, dv


def _bwd_selected(q, k, v, dy, r, flat, dilation, global_idx, key_padding_mask, n_threads, lib, one_sided,
                  random_blocks, keys):
    lib = lib or _load()
    qf, kf, vf, dyf = _f32(q), _f32(k), _f32(v), _f32(dy)
    B, H, T, d = qf.shape
    if dyf.shape != qf.shape:
        raise ValueError("dy must have the shape of q")
    r0, rad = _radius(r, H)
    rb, nr = _rand_blocks(random_blocks, H, T)
    dil = _i32(dilation)
    g = _i32(global_idx if global_idx is not None else [])
    pad = _u8(key_padding_mask)
    sel = np.ascontiguousarray(np.asarray(flat, dtype=np.int64).reshape(-1))
    o1 = np.zeros((sel.size, d), dtype=np.float64)
    common = (_ptr(qf), _ptr(kf), _ptr(vf), _ptr(dyf), B, H, T, d, r0, _ptr(rad), int(bool(one_sided)),
              _ptr(rb), nr, _ptr(dil), _ptr(g), int(g.size), _ptr(pad), _ptr(sel), int(sel.size))
    if keys:
        o2 = np.zeros((sel.size, d), dtype=np.float64)
        nt = lib.lf_oracle_bwd_keys(*common, _ptr(o1), _ptr(o2), int(n_threads))
    else:
        o2 = None
        nt = lib.lf_oracle_bwd_rows(*common, _ptr(o1), int(n_threads))
    if nt < 0:
        raise ValueError("oracle rejected its arguments")
    return (o1, o2) if keys else o1


def bwd_rows(q, k, v, dy, r, rows_flat, dilation=None, global_idx=None, key_padding_mask=None, n_threads=0,
             lib=None, one_sided=False, random_blocks=None):
    """dq of chosen query rows: rows_flat[e] = (b*H + h)*T + i -> dq[e][d]
    (the rows of ``bwd``'s dq, bit for bit, without computing the rest)."""
    return _bwd_selected(q, k, v, dy, r, rows_flat, dilation, global_idx, key_padding_mask, n_threads, lib,
                         one_sided, random_blocks, keys=False)


def bwd_keys(q, k, v, dy, r, keys_flat, dilation=None, global_idx=None, key_padding_mask=None, n_threads=0,
             lib=None, one_sided=False, random_blocks=None):
    """dk and dv of chosen key positions: keys_flat[e] = (b*H + h)*T + j ->
    (dk[e][d], dv[e][d]); the sums run over every row that attends to j."""
    return _bwd_selected(q, k, v, dy, r, keys_flat, dilation, global_idx, key_padding_mask, n_threads, lib,
                         one_sided, random_blocks, keys=True)


def rows(q, k, v, r, rows_flat, dilation=None, global_idx=None, key_padding_mask=None,
         n_threads=0, return_threads=False, lib=None, one_sided=False, random_blocks=None):
    """Selected output rows: rows_flat[e] = (b*H + h)*T + i -> out[e][d]."""
    lib = lib or _load()
    qf, kf, vf = _f32(q), _f32(k), _f32(v)
    B, H, T, d = qf.shape
    r0, rad = _radius(r, H)
    rb, nr = _rand_blocks(random_blocks, H, T)
    dil = _i32(dilation)
    g = _i32(global_idx if global_idx is not None else [])
    pad = _u8(key_padding_mask)
    rr = np.ascontiguousarray(np.asarray(rows_flat, dtype=np.int64))
    out = np.zeros((rr.size, d), dtype=np.float64)
    nt = lib.lf_oracle_rows2(_ptr(qf), _ptr(kf), _ptr(vf), B, H, T, d, r0, _ptr(rad), int(bool(one_sided)),
                             _ptr(rb), nr, _ptr(dil), _ptr(g), int(g.size), _ptr(pad), _ptr(rr), int(rr.size),
                             _ptr(out), int(n_threads))
    if nt < 0:
        raise ValueError("oracle rejected its arguments")
    return (out, nt) if return_threads else out


def neighbours(T, r, delta, i, global_idx=None, pad_row=None, lib=None, one_sided=False,
               random_blocks=None):
    """Sorted list N(i) of one query (empty for a padded query).
    ``random_blocks``: this head's [ceil(T/64)][n] key blocks, or None."""
    lib = lib or _load()
    rb, nr = (None, 0) if random_blocks is None else _rand_blocks(np.asarray(random_blocks)[None], 1, T)
    g = _i32(global_idx if global_idx is not None else [])
    pad = _u8(pad_row)
    buf = np.zeros(T, dtype=np.int32)
    n = lib.lf_oracle_neighbours2(int(T), int(r), int(delta), int(bool(one_sided)), _ptr(rb), nr, _ptr(g),
                                  int(g.size), _ptr(pad), int(i), _ptr(buf))
    if n < 0:
        raise ValueError("oracle rejected its arguments")
    return [int(x) for x in buf[:n]]


def count_pairs(B, H, T, r, dilation=None, global_idx=None, key_padding_mask=None, lib=None,
                one_sided=False, random_blocks=None):
    """Sum of |N(i)| over all rows (padded rows count 0)."""
    lib = lib or _load()
    r0, rad = _radius(r, H)
    rb, nr = _rand_blocks(random_blocks, H, T)
    dil = _i32(dilation)
    g = _i32(global_idx if global_idx is not None else [])
    pad = _u8(key_padding_mask)
    n = lib.lf_oracle_count_pairs2(int(B), int(H), int(T), r0, _ptr(rad), int(bool(one_sided)), _ptr(rb), nr,
                                   _ptr(dil), _ptr(g), int(g.size), _ptr(pad))
    if n < 0:
        raise ValueError("oracle rejected its arguments")
    return int(n)
