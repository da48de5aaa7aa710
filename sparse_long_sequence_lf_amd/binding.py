"""Thin ctypes binding of liblfattn.so (include/lf_attn.h).

Argument marshalling only: torch supplies device memory and the stream;
every step of the forward pass runs in the library's HIP kernels.  If the
library is not built, calls raise -- there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "liblfattn.so")

LF_F32 = 0
LF_BF16 = 1
LF_OK = 0
LF_E_INVALID = 1
LF_E_UNSUPPORTED = 2
LF_E_NOMEM = 3
LF_E_HIP = 4
STATUS_NAMES = {0: "LF_OK", 1: "LF_E_INVALID", 2: "LF_E_UNSUPPORTED", 3: "LF_E_NOMEM", 4: "LF_E_HIP"}
HEAD_DIM = 64          # d of the matrix-core backward (bf16); the backward takes every d of FWD_HEAD_DIMS
FWD_HEAD_DIMS = (32, 64, 128)
MAX_HEADS = 128
MAX_GLOBALS = 512
MAX_RAND_BLOCKS = 8

_lib = None


class LfError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


def load():
    """Load liblfattn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m sparse_long_sequence_lf_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    _check_fresh(lib)
    P = ctypes.c_void_p
    I = ctypes.c_int
    lib.lf_attn_fwd.argtypes = [P, P, P, I, I, I, I, I, P, P, I, P, P, I, P]
    lib.lf_attn_fwd.restype = I
    lib.lf_attn_fwd_ex.argtypes = [P, P, P, I, I, I, I, P, I, P, I, P, P, I, P, P, P, I, P]
    lib.lf_attn_fwd_ex.restype = I
    lib.lf_attn_fwd_noalloc.argtypes = [P, P, P, I, I, I, I, I, P, P, I, P, P, I, P]
    lib.lf_attn_fwd_noalloc.restype = I
    lib.lf_attn_fwd_global_rows.argtypes = [P, P, P, I, I, I, I, P, I, P, P, P, I, P]
    lib.lf_attn_fwd_global_rows.restype = I
    lib.lf_attn_bwd.argtypes = [P, P, P, P, I, I, I, I, P, I, P, I, P, P, I, P, P, P, P, I, P]
    lib.lf_attn_bwd.restype = I
    lib.lf_attn_bwd_ex.argtypes = [P, P, P, P, P, P, I, I, I, I, P, I, P, I, P, P, I, P, P, P, P, I, P]
    lib.lf_attn_bwd_ex.restype = I
    lib.lf_last_error.argtypes = []
    lib.lf_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check_fresh(lib):
    """Refuse a library built from other sources than the ones beside it."""
    from . import build as _build

    lib.lf_build_hash.argtypes = []
    lib.lf_build_hash.restype = ctypes.c_char_p
    built, now = lib.lf_build_hash().decode(), _build.source_hash()
    if built != now:
        raise RuntimeError(f"{LIB_PATH} was built from other sources (hash {built}, sources {now}): "
                           "rebuild it with `python -m sparse_long_sequence_lf_amd.build`")


def last_error() -> str:
    return load().lf_last_error().decode()


def _per_head(r):
    """True when r is a list of per-head radii rather than one int."""
    return not isinstance(r, int) and hasattr(r, "__len__")


def _rand_table(random_blocks, H=None, T=None):
    """(ctypes int32 array, n_rand) of random key blocks [H][ceil(T/64)][n], or (None, 0).
    With H and T given, the table's first two extents must be H and ceil(T/64)."""
    if random_blocks is None:
        return None, 0
    import numpy as np
    a = np.ascontiguousarray(np.asarray(random_blocks, dtype=np.int32))
    if a.ndim != 3:
        raise ValueError("random_blocks must be [H][ceil(T/64)][n_rand]")
    if H is not None and T is not None and a.shape[:2] != (int(H), (int(T) + 63) // 64):
        raise ValueError(f"random_blocks has shape {a.shape}; expected [{int(H)}][{(int(T) + 63) // 64}][n_rand]")
    flat = a.reshape(-1)
    if flat.size == 0:
        return (ctypes.c_int32 * 1)(), int(a.shape[2])
    return (ctypes.c_int32 * flat.size).from_buffer_copy(flat.tobytes()), int(a.shape[2])


def _dilation_array(dilation, H):
    if dilation is None:
        return None
    if len(dilation) != int(H):
        raise ValueError(f"dilation has {len(dilation)} entries for {int(H)} heads")
    return (ctypes.c_int32 * len(dilation))(*[int(x) for x in dilation])


def raw_fwd(q_ptr, k_ptr, v_ptr, B, H, T, d, r, dilation, global_idx, n_global, kpm_ptr, out_ptr,
            dtype, stream_ptr, one_sided=False, random_blocks=None, lse_ptr=None) -> int:
    """Call the library with raw integer device pointers; returns the status.
    ``r`` is one radius (lf_attn_fwd) or a list of H radii; a list,
    ``one_sided``, ``random_blocks`` or ``lse_ptr`` goes to lf_attn_fwd_ex."""
    lib = load()
    dil = _dilation_array(dilation, H)
    g = None
    if global_idx is not None:
        g = (ctypes.c_int32 * max(1, len(global_idx)))(*[int(x) for x in global_idx])
    if _per_head(r) or one_sided or random_blocks is not None or lse_ptr is not None:
        rl = [int(x) for x in r] if _per_head(r) else [int(r)] * int(H)
        if len(rl) != int(H):
            raise ValueError(f"r has {len(rl)} radii for {int(H)} heads")
        rad = (ctypes.c_int32 * max(1, len(rl)))(*rl)
        rt, nr = _rand_table(random_blocks, H, T)
        return lib.lf_attn_fwd_ex(q_ptr, k_ptr, v_ptr, int(B), int(H), int(T), int(d), rad,
                                  int(one_sided) if not isinstance(one_sided, bool) else int(one_sided),
                                  rt, nr, dil, g, int(n_global), kpm_ptr, out_ptr, lse_ptr, int(dtype), stream_ptr)
    return lib.lf_attn_fwd(q_ptr, k_ptr, v_ptr, int(B), int(H), int(T), int(d), int(r), dil, g,
                           int(n_global), kpm_ptr, out_ptr, int(dtype), stream_ptr)


def _padding_arg(key_padding_mask, B, T, stream):
    """(pointer, tensor) of the [B, T] byte mask, or (None, None).  A mask that
    needs converting (bool, or not contiguous) becomes a temporary, which is
    recorded on the call's stream so that the caching allocator keeps it
    until the kernels have read it."""
    import torch
    if key_padding_mask is None:
        return None, None
    kpm = key_padding_mask
    if kpm.dtype == torch.bool:
        kpm = kpm.to(torch.uint8)
    if kpm.dtype != torch.uint8 or tuple(kpm.shape) != (B, T) or not kpm.is_cuda:
        raise ValueError("key_padding_mask must be a uint8/bool device tensor [B, T]")
    kpm = kpm.contiguous()
    if kpm is not key_padding_mask and stream is not None and hasattr(stream, "cuda_stream"):
        kpm.record_stream(stream)
    return kpm.data_ptr(), kpm


def attn_fwd(q, k, v, r, dilation: Optional[Sequence[int]] = None,
             global_idx: Optional[Sequence[int]] = None, global_attention_mask=None,
             key_padding_mask=None, out=None, stream=None, one_sided: bool = False, random_blocks=None,
             lse=None):
    """Longformer sparse attention forward on torch tensors [B, H, T, d], d in {32, 64, 128}.

    ``lse``: an fp32 device tensor [B, H, T] that receives each row's
    log-sum-exp of its scaled scores (natural log), or None.

    ``r`` is the window radius, or a list with one radius per head;
    ``one_sided`` keeps only the window keys at or before each query;
    ``random_blocks`` ([H][ceil(T/64)][n] key-block indices) adds BigBird-style
    random key blocks of 64 to every query block of 64.

    ``global_attention_mask`` (a 0/1 tensor of shape [T] or [B, T], 1 =
    global, as in the Hugging Face convention) is turned into the index list
    ``global_idx``; a [B, T] mask must mark the same positions in every
    sequence.  ``key_padding_mask`` is [B, T], nonzero = padded.
    """
    import torch

    if q.dtype == torch.bfloat16:
        dt = LF_BF16
    elif q.dtype == torch.float32:
        dt = LF_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype or t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{name} must match q in dtype, shape and device")
    if q.dim() != 4:
        raise ValueError("q, k, v must be [B, H, T, d]")
    if not (q.is_cuda and q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous device tensors")
    B, H, T, d = q.shape
    if global_attention_mask is not None:
        if global_idx is not None:
            raise ValueError("give global_idx or global_attention_mask, not both")
        gm = global_attention_mask.detach().to("cpu")
        if gm.dim() == 2:
            if not bool((gm == gm[0:1]).all()):
                raise ValueError("global_attention_mask must mark the same positions in every sequence")
            gm = gm[0]
        global_idx = torch.nonzero(gm != 0).flatten().tolist()
    gl = list(global_idx) if global_idx is not None else []
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    kpm_ptr, _kpm = _padding_arg(key_padding_mask, B, T, stream)
    if _per_head(r) and len(r) != H:
        raise ValueError(f"r has {len(r)} radii for {H} heads")
    lse_ptr = None
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, T) or not lse.is_contiguous() or \
                lse.device != q.device:
            raise ValueError("lse must be a contiguous float32 device tensor [B, H, T]")
        lse_ptr = lse.data_ptr()
    st = raw_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, T, d, r, dilation,
                 gl if gl else None, len(gl), kpm_ptr, out.data_ptr(), dt, sptr, one_sided, random_blocks,
                 lse_ptr)
    if st != LF_OK:
        raise LfError(st, last_error())
    return out


def attn_fwd_global_rows(q, k, v, global_idx: Sequence[int], key_padding_mask=None, out=None, stream=None,
                         lse=None):
    """lf_attn_fwd_global_rows: only the rows at the positions ``global_idx``
    of the forward's output (and of ``lse``, a float32 [B, H, T] tensor, when
    given) are written; a global row attends to every valid key, so no
    window argument applies.  Every other row of ``out`` keeps its value."""
    import torch

    if q.dtype == torch.bfloat16:
        dt = LF_BF16
    elif q.dtype == torch.float32:
        dt = LF_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype or t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{name} must match q in dtype, shape and device")
    if q.dim() != 4 or not (q.is_cuda and q.is_contiguous() and k.is_contiguous() and v.is_contiguous()):
        raise ValueError("q, k, v must be contiguous device tensors [B, H, T, d]")
    B, H, T, d = q.shape
    if out is None:
        out = torch.zeros_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    lse_ptr = None
    if lse is not None:
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, T) or not lse.is_contiguous() or \
                lse.device != q.device:
            raise ValueError("lse must be a contiguous float32 device tensor [B, H, T]")
        lse_ptr = lse.data_ptr()
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    kpm_ptr, _kpm = _padding_arg(key_padding_mask, B, T, stream)
    gl = [int(x) for x in global_idx]
    g = (ctypes.c_int32 * max(1, len(gl)))(*gl)
    st = load().lf_attn_fwd_global_rows(q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, T, d, g, len(gl), kpm_ptr,
                                        out.data_ptr(), lse_ptr, dt, sptr)
    if st != LF_OK:
        raise LfError(st, last_error())
    return out


def raw_bwd(q_ptr, k_ptr, v_ptr, dy_ptr, B, H, T, d, r, one_sided, dilation, global_idx, n_global, kpm_ptr,
            dq_ptr, dk_ptr, dv_ptr, dtype, stream_ptr, random_blocks=None, y_ptr=None, lse_ptr=None) -> int:
    """lf_attn_bwd (lf_attn_bwd_ex when the forward's output ``y_ptr`` and
    ``lse_ptr`` are given) with raw integer device pointers; ``r`` is one
    radius or a list of H radii.  Returns the status."""
    lib = load()
    rl = [int(x) for x in r] if _per_head(r) else [int(r)] * int(H)
    if len(rl) != int(H):
        raise ValueError(f"r has {len(rl)} radii for {int(H)} heads")
    rad = (ctypes.c_int32 * max(1, len(rl)))(*rl)
    dil = _dilation_array(dilation, H)
    g = None
    if global_idx is not None:
        g = (ctypes.c_int32 * max(1, len(global_idx)))(*[int(x) for x in global_idx])
    rt, nr = _rand_table(random_blocks, H, T)
    if y_ptr is not None or lse_ptr is not None:
        return lib.lf_attn_bwd_ex(q_ptr, k_ptr, v_ptr, dy_ptr, y_ptr, lse_ptr, int(B), int(H), int(T), int(d), rad,
                                  int(bool(one_sided)), rt, nr, dil, g, int(n_global), kpm_ptr, dq_ptr, dk_ptr,
                                  dv_ptr, int(dtype), stream_ptr)
    return lib.lf_attn_bwd(q_ptr, k_ptr, v_ptr, dy_ptr, int(B), int(H), int(T), int(d), rad, int(bool(one_sided)),
                           rt, nr, dil, g, int(n_global), kpm_ptr, dq_ptr, dk_ptr, dv_ptr, int(dtype), stream_ptr)


def attn_bwd(q, k, v, dy, r, dilation: Optional[Sequence[int]] = None,
             global_idx: Optional[Sequence[int]] = None, key_padding_mask=None, out=None, stream=None,
             one_sided: bool = False, random_blocks=None, y=None, lse=None):
    """Gradients (dq, dk, dv) of the forward for the upstream gradient ``dy``,
    torch tensors [B, H, T, d] like q (d in {32, 64, 128}); the same window, dilation, global,
    random-block and padding arguments as ``attn_fwd``.  ``out`` may be a
    tuple of three tensors like q to write into.  ``y`` and ``lse``: the
    forward's output (like q) and its lse (float32 [B, H, T]) from the same
    arguments, both or neither (then bf16 input at d = 64 runs the forward
    first; the vector-unit path, fp32 or bf16 at d = 32 and 128, reads
    neither)."""
    import torch

    if q.dtype == torch.bfloat16:
        dt = LF_BF16
    elif q.dtype == torch.float32:
        dt = LF_F32
    else:
        raise TypeError(f"unsupported dtype {q.dtype}")
    for name, t in (("k", k), ("v", v), ("dy", dy)):
        if t.dtype != q.dtype or t.shape != q.shape or t.device != q.device:
            raise ValueError(f"{name} must match q in dtype, shape and device")
    if q.dim() != 4:
        raise ValueError("q, k, v, dy must be [B, H, T, d]")
    if not (q.is_cuda and all(t.is_contiguous() for t in (q, k, v, dy))):
        raise ValueError("q, k, v, dy must be contiguous device tensors")
    B, H, T, d = q.shape
    if _per_head(r) and len(r) != H:
        raise ValueError(f"r has {len(r)} radii for {H} heads")
    gl = list(global_idx) if global_idx is not None else []
    if out is None:
        out = tuple(torch.empty_like(q) for _ in range(3))
    elif len(out) != 3 or any(o.shape != q.shape or o.dtype != q.dtype or not o.is_contiguous() for o in out):
        raise ValueError("out must be three contiguous tensors like q")
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    kpm_ptr, _kpm = _padding_arg(key_padding_mask, B, T, stream)
    if (y is None) != (lse is None):
        raise ValueError("y and lse are given together or not at all")
    y_ptr = lse_ptr = None
    if y is not None:
        if y.dtype != q.dtype or y.shape != q.shape or y.device != q.device or not y.is_contiguous():
            raise ValueError("y must be a contiguous tensor like q")
        if lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, T) or lse.device != q.device \
                or not lse.is_contiguous():
            raise ValueError("lse must be a contiguous float32 [B, H, T] tensor on q's device")
        y_ptr, lse_ptr = y.data_ptr(), lse.data_ptr()
    st = raw_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), dy.data_ptr(), B, H, T, d, r, one_sided, dilation,
                 gl if gl else None, len(gl), kpm_ptr, out[0].data_ptr(), out[1].data_ptr(), out[2].data_ptr(),
                 dt, sptr, random_blocks, y_ptr, lse_ptr)
    if st != LF_OK:
        raise LfError(st, last_error())
    return out


class Prepared:
    """lf_attn_fwd with every argument marshalled once, for tight loops.

    Holds references to the tensors it was built from; ``__call__`` is one
    ctypes call into the library on the given stream.
    """

    def __init__(self, q, k, v, r, dilation=None, global_idx=None, key_padding_mask=None, out=None,
                 stream=None, one_sided=False, random_blocks=None):
        import torch

        lib = load()
        self._keep = [q, k, v]
        B, H, T, d = q.shape
        dt = LF_BF16 if q.dtype == torch.bfloat16 else LF_F32
        self.out = torch.empty_like(q) if out is None else out
        gl = list(global_idx) if global_idx is not None else []
        self._dil = _dilation_array(dilation, H)
        self._g = (ctypes.c_int32 * max(1, len(gl)))(*gl) if gl else None
        kpm = None
        if key_padding_mask is not None:
            kpm = key_padding_mask.to(torch.uint8).contiguous()
            self._keep.append(kpm)
        if stream is None:
            stream = torch.cuda.current_stream(q.device)
        sptr = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
        kptr = None if kpm is None else kpm.data_ptr()
        if _per_head(r) or one_sided or random_blocks is not None:
            rl = [int(x) for x in r] if _per_head(r) else [int(r)] * H
            self._rad = (ctypes.c_int32 * H)(*rl)
            self._rt, nr = _rand_table(random_blocks, H, T)
            self._fn = lib.lf_attn_fwd_ex
            self._args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, T, d, self._rad, int(bool(one_sided)),
                          self._rt, nr, self._dil, self._g, len(gl), kptr, self.out.data_ptr(), None, dt, sptr)
        else:
            self._fn = lib.lf_attn_fwd
            self._args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), B, H, T, d, int(r), self._dil, self._g,
                          len(gl), kptr, self.out.data_ptr(), dt, sptr)

    def __call__(self):
        st = self._fn(*self._args)
        if st != LF_OK:
            raise LfError(st, last_error())
        return self.out
