"""Checks that pin the fp64 oracle to something other than itself.

Each check takes an optional ``lib`` (an oracle build loaded with
``oracle.open_library``) so the same checks can be aimed at copies of the
oracle with a planted mistake; every planted mistake must trip at least
one of them.  The pins:

* brute force: dense masked attention with an explicit T x T mask
  (``dense_ref``), on tiny T, random r, dilation, globals and padding;
* closed forms of the neighbour counts (Longformer, eightmm.github.io,
  "Sliding-Window Attention": |N_local(i)| = 2r + 1 away from the ends;
  "Longformer长序列处理", 线性复杂度原理: cost grows 16x from 512 to 8192
  tokens at fixed window, 256x for dense attention);
* invariants and special cases: v == 1 gives 1; q == 0 gives the plain
  mean over N(i); r = 0 gives v; r >= T-1 gives textbook dense attention
  (torch's scaled_dot_product_attention in float64); a constant added to
  every key leaves the softmax unchanged; keys outside N(i) do not reach
  row i; a dilated head splits into delta undilated problems; global rows
  are dense rows; padded rows are zero;
* the set definitions N(i) = N_local(i) U G and N(i) = all for i in G;
* per-head radii and one-sided windows (the window list of "Longformer长序列
  处理", HF实践, and the one- or two-sided question of Longformer,
  eightmm.github.io, "Implementation Reading"): the brute force with the
  window taken per head and cut to keys at or before the query, the
  one-sided closed form sum_i (min(i, r) + 1) = T(r+1) - r(r+1)/2, and the
  one-sided dense limit equal to causal attention (torch's
  scaled_dot_product_attention with is_causal, float64);
* random key blocks (BigBird as the pages describe it: random attention in
  blocks of 64): the brute force with the blocks added to each row's mask,
  an exact count for r = 0, and every block drawn for every query block
  giving dense attention.
* the log-sum-exp of each row (the statistic a backward pass rebuilds the
  weights from): the brute force's logaddexp over the allowed scores of its
  mask, log |N(i)| for q = 0 (every score zero), and the dense limit equal to
  torch.logsumexp of the scaled scores; the forward written with it,
  sum_j exp(s_ij - lse_i) v_j, equals the forward itself;
* gradients (the derivative of the forward map; the pages give no backward
  pass): torch float64 autograd through the dense brute force, central
  finite differences of the oracle's own forward, and the sum rules
  sum_j dk_j = 0 (softmax weights sum to one, so the dS of a row sums to
  zero) and sum_j dv_j = sum of dy over the rows that attend to something;
  the gradient at chosen rows and keys (used where the whole gradient would
  take too long) against autograd and, bit for bit, the whole gradient.
"""
import numpy as np
import torch

import oracle
from dense_ref import allowed_matrix, dense_masked_attention, dense_masked_lse


def _rand(seed, B, H, T, d):
    g = torch.Generator("cpu").manual_seed(seed)
    return [torch.randn((B, H, T, d), generator=g, dtype=torch.float32) for _ in range(3)]


def random_cases(n, seed0=0, Ts=(1, 2, 7, 33, 64, 130, 257)):
    rng = np.random.default_rng(seed0)
    cases = []
    for c in range(n):
        T = int(Ts[c % len(Ts)])
        B = int(rng.integers(1, 3))
        H = int(rng.integers(1, 4))
        d = int(rng.choice([8, 16, 64]))
        r = int(rng.integers(0, T + 3))
        dil = [int(x) for x in rng.integers(1, 6, size=H)]
        kind = c % 4
        if kind == 0:
            G = []
        elif kind == 1:
            G = [int(x) for x in rng.integers(0, T, size=int(rng.integers(1, 5)))]  # dups ok
        elif kind == 2:
            G = list(range(T))
        else:
            G = [int(x) for x in rng.integers(0, T, size=2)]
        pk = int(rng.integers(0, 3))
        if pk == 0:
            pad = None
        elif pk == 1:
            lens = rng.integers(0, T + 1, size=B)
            pad = (np.arange(T)[None, :] >= lens[:, None]).astype(np.uint8)
        else:
            pad = (rng.random((B, T)) < 0.25).astype(np.uint8)
        q, k, v = _rand(1000 + c, B, H, T, d)
        # every third case one-sided, every other case one radius per head
        one = c % 3 == 2
        rr = [int(x) for x in rng.integers(0, T + 3, size=H)] if c % 2 else r
        # every fourth case (from the second on) with random key blocks, on undilated heads
        rb = None
        if c % 4 == 1:
            dil = [1] * H
            nqb = (T + 63) // 64
            rb = rng.integers(0, nqb, size=(H, nqb, int(rng.integers(1, 4)))).astype(np.int32)
        cases.append(dict(q=q, k=k, v=v, r=rr, dil=dil, G=G, pad=pad, one=one, rb=rb))
    return cases


# --------------------------------------------------------------------------
# brute force

def check_dense_bruteforce(lib=None, n=28, tol=1e-12):
    for c in random_cases(n):
        y = oracle.fwd(c["q"], c["k"], c["v"], c["r"], c["dil"], c["G"], c["pad"], lib=lib, one_sided=c["one"],
                       random_blocks=c["rb"])
        ref = dense_masked_attention(c["q"].numpy(), c["k"].numpy(), c["v"].numpy(), c["r"],
                                     c["dil"], c["G"], c["pad"], c["one"], c["rb"])
        err = np.max(np.abs(y - ref)) if y.size else 0.0
        assert err <= tol, f"oracle vs dense brute force: {err} (T={c['q'].shape[2]}, r={c['r']}, one={c['one']})"


# --------------------------------------------------------------------------
# closed-form counts

def local_count(T, r):
    """sum_i |{j in [0,T): |i-j| <= r}|, written out from min(i, r) terms."""
    if T <= 0:
        return 0
    rr = min(r, T - 1)
    # each row: 1 + min(i, rr) + min(T-1-i, rr); both sums equal S = sum_i min(i, rr)
    S = rr * (rr - 1) // 2 + (T - rr) * rr
    return T + 2 * S


def dilated_count(T, r, delta):
    return sum(local_count(len(range(c, T, delta)), r) for c in range(delta))


def check_closed_form_counts(lib=None):
    # T(2r+1) - r(r+1) for T >= r (the interior rows have w = 2r+1 keys)
    for T, r in [(1024, 64), (4096, 256), (4096, 128), (300, 7), (16384, 512), (10, 9), (10, 3)]:
        assert local_count(T, r) == T * (2 * r + 1) - r * (r + 1)
        assert oracle.count_pairs(1, 1, T, r, lib=lib) == local_count(T, r)
    # r beyond the sequence: dense
    for T in (1, 5, 64):
        assert oracle.count_pairs(1, 1, T, T + 3, lib=lib) == T * T
    # dilated heads: delta residue classes of length ceil((T - c)/delta)
    for T, r, dl in [(4096, 128, [1, 1, 2, 2, 2, 2, 3, 3, 3, 3, 4, 4]), (100, 5, [3, 7]), (37, 2, [5])]:
        want = sum(dilated_count(T, r, x) for x in dl)
        assert oracle.count_pairs(1, len(dl), T, r, dilation=dl, lib=lib) == want
    # one global at 0 (delta = 1): non-global rows gain key 0 when it is outside the window
    for T, r, H in [(1024, 64, 2), (4096, 256, 12)]:
        per_head = (local_count(T, r) - (r + 1)) + T + (T - (r + 1))
        assert oracle.count_pairs(1, H, T, r, global_idx=[0], lib=lib) == per_head * H
    # one-sided: row i keeps min(i, r) + 1 keys, T(r+1) - r(r+1)/2 in all for T >= r
    for T, r in [(1024, 64), (4096, 256), (300, 7), (10, 9), (10, 3), (1, 0)]:
        want = sum(min(i, r) + 1 for i in range(T))
        assert want == T * (r + 1) - r * (r + 1) // 2
        assert oracle.count_pairs(1, 1, T, r, lib=lib, one_sided=True) == want
    # one radius per head: the sum of the per-head closed forms
    rads = [0, 3, 64, 200]
    assert oracle.count_pairs(2, 4, 1000, rads, lib=lib) == 2 * sum(local_count(1000, x) for x in rads)
    assert oracle.count_pairs(1, 4, 1000, rads, lib=lib, one_sided=True) == sum(
        1000 * (x + 1) - x * (x + 1) // 2 for x in rads)
    # random key blocks with r = 0 and no globals: row i sees itself and the
    # keys of its block's random blocks (its own block counts once)
    rng = np.random.default_rng(17)
    for T in (64, 200, 1000):
        nqb = (T + 63) // 64
        rb = rng.integers(0, nqb, size=(1, nqb, 2)).astype(np.int32)
        want = 0
        for i in range(T):
            keys = {i}
            for blk in set(int(x) for x in rb[0, i // 64]):
                keys |= set(range(64 * blk, min(64 * blk + 64, T)))
            want += len(keys)
        assert oracle.count_pairs(1, 1, T, 0, lib=lib, random_blocks=rb) == want
    # 512 -> 8192 tokens: dense x256 exactly, fixed small window ~x16
    assert oracle.count_pairs(1, 1, 8192, 9000, lib=lib) == 256 * oracle.count_pairs(1, 1, 512, 9000, lib=lib)
    ratio = oracle.count_pairs(1, 1, 8192, 4, lib=lib) / oracle.count_pairs(1, 1, 512, 4, lib=lib)
    assert abs(ratio - 16.0) < 0.16


# --------------------------------------------------------------------------
# set definitions

def check_neighbour_sets(lib=None):
    rng = np.random.default_rng(7)
    for trial in range(60):
        T = int(rng.integers(1, 80))
        r = int(rng.integers(0, 12))
        delta = int(rng.integers(1, 5))
        G = [int(x) for x in rng.integers(0, T, size=int(rng.integers(0, 4)))]
        pad = (rng.random(T) < 0.2).astype(np.uint8) if trial % 2 else None
        for i in range(T):
            got = oracle.neighbours(T, r, delta, i, G, pad, lib=lib)
            valid = [j for j in range(T) if pad is None or not pad[j]]
            if pad is not None and pad[i]:
                want = []
            elif i in G:
                want = valid                                   # N(i) = all positions
            else:
                loc = {j for j in range(T) if abs(i - j) <= r * delta and (i - j) % delta == 0}
                want = sorted((loc | set(G)) & set(valid))     # N_local(i) U G
            assert got == want, (T, r, delta, G, i, got, want)
            # one-sided: the window part keeps the keys at or before i
            got1 = oracle.neighbours(T, r, delta, i, G, pad, lib=lib, one_sided=True)
            if (pad is not None and pad[i]) or i in G:
                want1 = want
            else:
                loc1 = {j for j in range(T) if 0 <= i - j <= r * delta and (i - j) % delta == 0}
                want1 = sorted((loc1 | set(G)) & set(valid))
            assert got1 == want1, (T, r, delta, G, i, got1, want1)


# --------------------------------------------------------------------------
# invariants and special cases

def check_invariants(lib=None):
    cases = random_cases(16, seed0=3)
    for c in cases:
        q, k, v = c["q"], c["k"], c["v"]
        B, H, T, d = q.shape
        pad = c["pad"]
        valid = np.ones((B, T), bool) if pad is None else ~pad.astype(bool)
        # v == 1 -> every valid row is exactly a convex combination of ones
        one = c["one"]
        y1 = oracle.fwd(q, k, torch.ones_like(v), c["r"], c["dil"], c["G"], pad, lib=lib, one_sided=one)
        for b in range(B):
            assert np.all(np.abs(y1[b][:, valid[b]] - 1.0) <= 1e-14)
            assert np.all(y1[b][:, ~valid[b]] == 0.0)
        # q == 0 -> uniform weights: the mean of v over N(i) (mask from dense_ref)
        y0 = oracle.fwd(torch.zeros_like(q), k, v, c["r"], c["dil"], c["G"], pad, lib=lib, one_sided=one)
        for b in range(B):
            for h in range(H):
                rh = c["r"] if np.isscalar(c["r"]) else c["r"][h]
                A = allowed_matrix(T, rh, c["dil"][h], c["G"],
                                   None if pad is None else pad[b], one)
                for i in range(T):
                    if not valid[b, i]:
                        continue
                    want = v[b, h].numpy().astype(np.float64)[A[i]].mean(axis=0)
                    assert np.max(np.abs(y0[b, h, i] - want)) <= 1e-13
        # shift invariance of the logits: k_j + c for every j
        base = oracle.fwd(q, k, v, c["r"], c["dil"], c["G"], pad, lib=lib, one_sided=one)
        shift = torch.randn(B, H, 1, d, generator=torch.Generator().manual_seed(5))
        ys = oracle.fwd(q, (k.double() + shift.double()).float(), v, c["r"], c["dil"], c["G"], pad, lib=lib,
                        one_sided=one)
        # k + shift is rounded to float32, so compare against the oracle on the rounded keys'
        # exact effect: scores change by q.shift up to float32 rounding of k (~1e-7 relative)
        assert np.max(np.abs(ys - base)) <= 5e-5
    # exact shift: keys and shift on a coarse grid so k + c is exact in float32
    g = torch.Generator().manual_seed(11)
    q = torch.randint(-4, 5, (1, 2, 40, 8), generator=g).float() / 4
    k = torch.randint(-4, 5, (1, 2, 40, 8), generator=g).float() / 4
    v = torch.randn(1, 2, 40, 8, generator=g)
    cvec = torch.randint(-8, 9, (1, 2, 1, 8), generator=g).float() / 8
    a = oracle.fwd(q, k, v, 3, [1, 2], [5], None, lib=lib)
    b2 = oracle.fwd(q, k + cvec, v, 3, [1, 2], [5], None, lib=lib)
    assert np.max(np.abs(a - b2)) <= 1e-12


def check_identity_and_dense_limits(lib=None):
    g = torch.Generator().manual_seed(21)
    for T in (1, 9, 64, 130):
        q, k, v = [torch.randn(2, 3, T, 16, generator=g) for _ in range(3)]
        # r = 0, no globals: each valid row attends only to itself
        y = oracle.fwd(q, k, v, 0, [1, 2, 3], [], None, lib=lib)
        assert np.array_equal(y, v.numpy().astype(np.float64))
        # r >= T - 1, delta = 1, no padding: textbook dense attention
        yd = oracle.fwd(q, k, v, T - 1, None, [], None, lib=lib)
        ref = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double()).numpy()
        assert np.max(np.abs(yd - ref)) <= 1e-12
        # globals do not change the dense limit
        yg = oracle.fwd(q, k, v, T + 5, None, [0, T - 1], None, lib=lib)
        assert np.max(np.abs(yg - ref)) <= 1e-12
        # one-sided, r >= T - 1, no globals: textbook causal attention
        yc = oracle.fwd(q, k, v, [T - 1, T + 2, 10 * T], None, [], None, lib=lib, one_sided=True)
        refc = torch.nn.functional.scaled_dot_product_attention(q.double(), k.double(), v.double(),
                                                                 is_causal=True).numpy()
        assert np.max(np.abs(yc - refc)) <= 1e-12
        # every key block drawn for every query block: dense attention
        nqb = (T + 63) // 64
        allb = np.tile(np.arange(nqb, dtype=np.int32), (3, nqb, 1))
        yr = oracle.fwd(q, k, v, 0, [1, 1, 1], [], None, lib=lib, random_blocks=allb)
        assert np.max(np.abs(yr - ref)) <= 1e-12
        # one-sided, r = 0: each row attends to itself only
        y1 = oracle.fwd(q, k, v, 0, [2, 1, 3], [], None, lib=lib, one_sided=True)
        assert np.array_equal(y1, v.numpy().astype(np.float64))
    # global rows: dense attention over the valid keys
    T = 50
    q, k, v = [torch.randn(1, 2, T, 16, generator=g) for _ in range(3)]
    pad = np.zeros((1, T), np.uint8)
    pad[0, 40:] = 1
    pad[0, 7] = 1
    G = [3, 7, 20]
    y = oracle.fwd(q, k, v, 2, [1, 3], G, pad, lib=lib)
    keep = ~pad[0].astype(bool)
    for h in range(2):
        for i in G:
            if pad[0, i]:
                assert np.all(y[0, h, i] == 0.0)
                continue
            s = (q[0, h, i].double() @ k[0, h].double().T / 4.0).numpy()
            s = s[keep]
            p = np.exp(s - s.max())
            want = (p[:, None] * v[0, h].double().numpy()[keep]).sum(0) / p.sum()
            assert np.max(np.abs(y[0, h, i] - want)) <= 1e-12
    assert np.all(y[0][:, 40:] == 0.0) and np.all(y[0][:, 7] == 0.0)


def check_window_exclusivity(lib=None):
    g = torch.Generator().manual_seed(31)
    T, d = 90, 16
    q, k, v = [torch.randn(1, 1, T, d, generator=g) for _ in range(3)]
    r, delta, G = 4, 3, [10, 70]
    base = oracle.fwd(q, k, v, r, [delta], G, None, lib=lib)
    for i in (0, 20, 45, 89):
        inside = set(j for j in range(T) if abs(i - j) <= r * delta and (i - j) % delta == 0) | set(G)
        outside = [j for j in range(T) if j not in inside]
        k2, v2 = k.clone(), v.clone()
        junk = torch.randn(len(outside), d, generator=g) * 10
        k2[0, 0, outside] = junk
        v2[0, 0, outside] = -junk
        y = oracle.fwd(q, k2, v2, r, [delta], G, None, lib=lib)
        assert np.array_equal(y[0, 0, i], base[0, 0, i])
        # permuting the keys that sit outside the window also changes nothing
        perm = np.random.default_rng(i).permutation(outside)
        k3, v3 = k.clone(), v.clone()
        k3[0, 0, outside] = k[0, 0, perm]
        v3[0, 0, outside] = v[0, 0, perm]
        y3 = oracle.fwd(q, k3, v3, r, [delta], G, None, lib=lib)
        assert np.array_equal(y3[0, 0, i], base[0, 0, i])


def check_dilation_split(lib=None):
    g = torch.Generator().manual_seed(41)
    T, d = 103, 8
    q, k, v = [torch.randn(1, 1, T, d, generator=g) for _ in range(3)]
    rng = np.random.default_rng(3)
    pad = (rng.random((1, T)) < 0.15).astype(np.uint8)
    for delta in (2, 3, 5):
        for r in (0, 1, 6):
            y = oracle.fwd(q, k, v, r, [delta], [], pad, lib=lib)
            for c in range(delta):
                idx = list(range(c, T, delta))
                ys = oracle.fwd(q[:, :, idx], k[:, :, idx], v[:, :, idx], r, [1], [], pad[:, idx], lib=lib)
                assert np.array_equal(y[0, 0, idx], ys[0, 0])


def check_rows_entry_point(lib=None):
    c = random_cases(3, seed0=9, Ts=(33, 64, 130))[2]
    B, H, T, d = c["q"].shape
    sel = np.random.default_rng(0).choice(B * H * T, size=min(50, B * H * T), replace=False)
    for one in (False, True):
        full = oracle.fwd(c["q"], c["k"], c["v"], c["r"], c["dil"], c["G"], c["pad"], lib=lib, one_sided=one)
        part = oracle.rows(c["q"], c["k"], c["v"], c["r"], sel, c["dil"], c["G"], c["pad"], lib=lib,
                           one_sided=one)
        assert np.array_equal(part, full.reshape(-1, d)[sel])


# --------------------------------------------------------------------------
# gradients

def dense_grads_autograd(c, dy):
    """dq, dk, dv of sum(y * dy) through the dense masked forward, by torch
    float64 autograd (an independent route to the same derivative)."""
    q = c["q"].double().clone().requires_grad_(True)
    k = c["k"].double().clone().requires_grad_(True)
    v = c["v"].double().clone().requires_grad_(True)
    B, H, T, d = q.shape
    outs = []
    for b in range(B):
        pad_row = None if c["pad"] is None else np.asarray(c["pad"][b]).astype(bool)
        per_h = []
        for h in range(H):
            rh = int(c["r"]) if np.isscalar(c["r"]) else int(c["r"][h])
            A = allowed_matrix(T, rh, int(c["dil"][h]), c["G"], pad_row, c["one"],
                               None if c["rb"] is None else c["rb"][h])
            if pad_row is not None:
                A = A & ~pad_row[:, None]
            At = torch.from_numpy(A)
            S = (q[b, h] @ k[b, h].T) / np.sqrt(d)
            S = S.masked_fill(~At, float("-inf"))
            live = At.any(dim=1, keepdim=True)
            S = torch.where(live, S, torch.zeros_like(S))       # rows with no key: no NaN
            P = torch.softmax(S, dim=1) * live
            per_h.append(P @ v[b, h])
        outs.append(torch.stack(per_h))
    y = torch.stack(outs)
    (y * torch.as_tensor(dy, dtype=torch.float64)).sum().backward()
    return q.grad.numpy(), k.grad.numpy(), v.grad.numpy()


def _dy(seed, shape):
    g = torch.Generator("cpu").manual_seed(seed)
    return torch.randn(shape, generator=g, dtype=torch.float32)


def check_grad_autograd(lib=None, n=16, tol=1e-11):
    for e, c in enumerate(random_cases(n, seed0=7, Ts=(1, 2, 7, 33, 64, 97))):
        dy = _dy(500 + e, c["q"].shape)
        got = oracle.bwd(c["q"], c["k"], c["v"], dy, c["r"], c["dil"], c["G"], c["pad"], lib=lib,
                         one_sided=c["one"], random_blocks=c["rb"])
        ref = dense_grads_autograd(c, dy.numpy())
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            err = np.max(np.abs(a - b)) if a.size else 0.0
            assert err <= tol * max(1.0, np.max(np.abs(b)) if b.size else 1.0), \
                f"{name} vs autograd: {err} (T={c['q'].shape[2]}, r={c['r']}, one={c['one']})"


def check_grad_finite_differences(lib=None):
    # f(x) = sum(y(x) * dy); central differences with a step exact in float32
    rng = np.random.default_rng(3)
    B, H, T, d = 1, 2, 11, 4
    q, k, v = _rand(77, B, H, T, d)
    dy = _dy(78, (B, H, T, d)).numpy().astype(np.float64)
    pad = np.zeros((B, T), dtype=np.uint8)
    pad[0, 9] = 1
    args = dict(r=[2, 1], dilation=[1, 2], global_idx=[4], key_padding_mask=pad)
    dq, dk, dv = oracle.bwd(q, k, v, dy, lib=lib, **args)
    h = 2.0 ** -10

    def f(qq, kk, vv):
        return float(np.sum(oracle.fwd(qq, kk, vv, lib=lib, **args) * dy))

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(12):
            idx = (0, int(rng.integers(0, H)), int(rng.integers(0, T)), int(rng.integers(0, d)))
            xs = [q.clone(), k.clone(), v.clone()]
            xs[which][idx] += h
            fp = f(*xs)
            xs[which][idx] -= 2 * h
            fm = f(*xs)
            fd = (fp - fm) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-5 * max(1.0, abs(fd)), (which, idx, fd, grad[idx])


def check_grad_sum_rules(lib=None):
    for e, c in enumerate(random_cases(12, seed0=11)):
        dy = _dy(900 + e, c["q"].shape)
        dq, dk, dv = oracle.bwd(c["q"], c["k"], c["v"], dy, c["r"], c["dil"], c["G"], c["pad"], lib=lib,
                                one_sided=c["one"], random_blocks=c["rb"])
        B, H, T, d = dq.shape
        assert np.max(np.abs(dk.sum(axis=2)), initial=0.0) <= 1e-9
        for b in range(B):
            for h in range(H):
                pad_row = None if c["pad"] is None else np.asarray(c["pad"][b])
                # a valid query always attends to itself, a padded one to nothing
                live = np.ones(T, dtype=bool) if pad_row is None else ~pad_row.astype(bool)
                want = dy.numpy()[b, h][live].astype(np.float64).sum(axis=0)
                assert np.max(np.abs(dv[b, h].sum(axis=0) - want), initial=0.0) <= 1e-9
                if pad_row is not None:
                    pr = pad_row.astype(bool)
                    assert not np.any(dq[b, h][pr]) and not np.any(dk[b, h][pr]) and not np.any(dv[b, h][pr])


def check_grad_selected_positions(lib=None):
    # dq of chosen rows and dk, dv of chosen keys (the entry points that make
    # full-size sampled checks possible): torch autograd of the dense brute
    # force, and the same bits as the whole gradient
    for e, c in enumerate(random_cases(12, seed0=13, Ts=(1, 7, 33, 64, 130))):
        dy = _dy(1300 + e, c["q"].shape)
        B, H, T, d = c["q"].shape
        n = B * H * T
        sel = np.random.default_rng(e).choice(n, size=min(n, 24), replace=False)
        sel[-1] = n - 1
        args = (c["q"], c["k"], c["v"], dy, c["r"])
        kw = dict(dilation=c["dil"], global_idx=c["G"], key_padding_mask=c["pad"], lib=lib, one_sided=c["one"],
                  random_blocks=c["rb"])
        dq_s = oracle.bwd_rows(*args, sel, **kw)
        dk_s, dv_s = oracle.bwd_keys(*args, sel, **kw)
        ref = dense_grads_autograd(c, dy.numpy())
        for name, got, want in (("dq", dq_s, ref[0]), ("dk", dk_s, ref[1]), ("dv", dv_s, ref[2])):
            want = want.reshape(-1, d)[sel]
            err = np.max(np.abs(got - want)) if got.size else 0.0
            assert err <= 1e-11 * max(1.0, np.max(np.abs(want)) if want.size else 1.0), \
                f"{name} at chosen positions vs autograd: {err} (T={T})"
        whole = oracle.bwd(*args, **kw)
        for got, w in zip((dq_s, dk_s, dv_s), whole):
            assert np.array_equal(got, w.reshape(-1, d)[sel])


# --------------------------------------------------------------------------
# log-sum-exp of each row

def check_lse(lib=None):
    # against the dense brute force, every kind of case
    for c in random_cases(20, seed0=5):
        y, lse = oracle.fwd_lse(c["q"], c["k"], c["v"], c["r"], c["dil"], c["G"], c["pad"], lib=lib,
                                one_sided=c["one"], random_blocks=c["rb"])
        ref = dense_masked_lse(c["q"].numpy(), c["k"].numpy(), c["r"], c["dil"], c["G"], c["pad"], c["one"],
                               c["rb"])
        fin = np.isfinite(ref)
        assert np.array_equal(fin, np.isfinite(lse)), "lse: -inf rows differ from the brute force"
        assert np.max(np.abs(lse[fin] - ref[fin]), initial=0.0) <= 1e-12
        y2 = oracle.fwd(c["q"], c["k"], c["v"], c["r"], c["dil"], c["G"], c["pad"], lib=lib, one_sided=c["one"],
                        random_blocks=c["rb"])
        assert np.array_equal(y, y2)
        # the forward rebuilt from lse: y_i = sum_j exp(s_ij - lse_i) v_j over the mask
        B, H, T, d = c["q"].shape
        for b in range(B):
            pad_row = None if c["pad"] is None else np.asarray(c["pad"][b]).astype(bool)
            for h in range(H):
                delta = 1 if c["dil"] is None else int(c["dil"][h])
                rh = int(c["r"]) if np.isscalar(c["r"]) else int(c["r"][h])
                A = allowed_matrix(T, rh, delta, c["G"], pad_row, c["one"],
                                   None if c["rb"] is None else c["rb"][h])
                S = c["q"][b, h].double().numpy() @ c["k"][b, h].double().numpy().T / np.sqrt(d)
                lrow = np.where(np.isfinite(lse[b, h]), lse[b, h], 0.0)[:, None]
                P = np.where(A, np.exp(S - lrow), 0.0)
                if pad_row is not None:
                    P[pad_row] = 0.0
                want = P @ c["v"][b, h].double().numpy()
                assert np.max(np.abs(want - y[b, h]), initial=0.0) <= 1e-12
    # q = 0: every score is zero, so lse_i = log |N(i)|
    g = torch.Generator().manual_seed(5)
    for T, r, dil, G in [(40, 3, [1, 2], [0, 17]), (100, 9, [3, 1], []), (7, 20, [1, 1], [6])]:
        k, v = [torch.randn(1, 2, T, 8, generator=g) for _ in range(2)]
        q0 = torch.zeros_like(k)
        _, lse = oracle.fwd_lse(q0, k, v, r, dil, G, None, lib=lib)
        for h in range(2):
            cnt = allowed_matrix(T, r, dil[h], G, None).sum(axis=1)
            assert np.max(np.abs(lse[0, h] - np.log(cnt))) <= 1e-12
    # r >= T - 1, no padding: the dense limit is torch.logsumexp of the scaled scores
    for T in (1, 9, 130):
        q, k, v = [torch.randn(2, 3, T, 16, generator=g) for _ in range(3)]
        _, lse = oracle.fwd_lse(q, k, v, T, None, [], None, lib=lib)
        ref = torch.logsumexp(q.double() @ k.double().transpose(-1, -2) / 4.0, dim=-1).numpy()
        assert np.max(np.abs(lse - ref)) <= 1e-12


ALL_CHECKS = [check_dense_bruteforce, check_lse, check_closed_form_counts, check_neighbour_sets,
              check_invariants, check_identity_and_dense_limits, check_window_exclusivity,
              check_dilation_split, check_rows_entry_point, check_grad_autograd,
              check_grad_finite_differences, check_grad_sum_rules, check_grad_selected_positions]
