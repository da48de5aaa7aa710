"""Helpers shared by the GPU parity tests: run the HIP path through the C ABI
and compare it with the fp64 oracle on the same seeded inputs."""
import numpy as np
import torch

import oracle
import sparse_long_sequence_lf_amd as lf

# Tolerances on max |gpu - oracle| (absolute): fp32 inputs 1e-4; bf16 inputs
# with fp32 accumulation 2e-2.
TOL = {"f32": 1e-4, "bf16": 2e-2}


def require_gpu():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    lf.load()  # raises if the HIP library is missing


def to_dev(inp):
    dev = torch.device("cuda:0")
    kpm = None if inp.key_padding_mask is None else inp.key_padding_mask.to(dev)
    return inp.q.to(dev), inp.k.to(dev), inp.v.to(dev), kpm


def gpu_fwd(inp, q=None, k=None, v=None):
    qd, kd, vd, kpm = to_dev(inp)
    if q is not None:
        qd = q.to("cuda:0")
    if k is not None:
        kd = k.to("cuda:0")
    if v is not None:
        vd = v.to("cuda:0")
    out = lf.attn_fwd(qd, kd, vd, inp.r, inp.dilation, inp.global_idx, key_padding_mask=kpm,
                      one_sided=inp.one_sided, random_blocks=inp.random_blocks)
    torch.cuda.synchronize()
    return out


def oracle_full(inp, q=None, k=None, v=None):
    return oracle.fwd(inp.q if q is None else q, inp.k if k is None else k,
                      inp.v if v is None else v, inp.r, inp.dilation, inp.global_idx,
                      inp.key_padding_mask, one_sided=inp.one_sided, random_blocks=inp.random_blocks)


def max_err(gpu_out, ref):
    g = gpu_out.detach().float().cpu().double().numpy()
    return float(np.max(np.abs(g - ref))) if ref.size else 0.0


def sample_rows(inp, n_random, seed=0):
    """Rows for sampled full-size parity: every global row, both ends of each
    class of each head, rows around each padding boundary, and random rows."""
    B, H, T, d = inp.q.shape
    rng = np.random.default_rng(seed)
    rows = set()
    for b in range(B):
        for h in range(H):
            base = (b * H + h) * T
            for g in inp.global_idx:
                rows.add(base + g)
            delta = inp.dilation[h] if inp.dilation else 1
            for c in range(min(delta, T)):
                for i in (c, c + delta, (T - 1 - c) - ((T - 1 - c) - c) % delta):
                    if 0 <= i < T:
                        rows.add(base + i)
            rh = inp.r if isinstance(inp.r, int) else inp.r[h]
            for x in (0, 1, rh, rh + 1, T - 1 - rh, T - 2, T - 1):
                if 0 <= x < T:
                    rows.add(base + x)
            if inp.lengths is not None:
                L = inp.lengths[b]
                for x in range(L - 3, L + 3):
                    if 0 <= x < T:
                        rows.add(base + x)
    rows |= set(int(x) for x in rng.choice(B * H * T, size=n_random, replace=False))
    return np.array(sorted(rows), dtype=np.int64)


def sample_keys(inp, n_heads, n_random, seed=0):
    """Key positions for sampled full-size gradient parity (a key's dk, dv sum
    over every row that attends to it, so a global key costs a whole head):
    in n_heads (b, h) pairs (the first, the last, the rest random) the
    positions sample_rows would take there; anywhere, n_random random keys."""
    B, H, T, d = inp.q.shape
    rng = np.random.default_rng(seed)
    heads = {0, B * H - 1}
    while len(heads) < min(n_heads, B * H):
        heads.add(int(rng.integers(0, B * H)))
    every = sample_rows(inp, n_random=0, seed=seed)
    keys = set(int(x) for x in every if int(x) // T in heads)
    keys |= set(int(x) for x in rng.choice(B * H * T, size=min(n_random, B * H * T), replace=False))
    return np.array(sorted(keys), dtype=np.int64)
