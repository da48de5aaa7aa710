"""GPU parity: the HIP path (through the C ABI) against the fp64 oracle on
identical seeded inputs.

Bar: max |gpu - oracle| <= 1e-4 for fp32 inputs, <= 2e-2 for bf16 inputs
(fp32 accumulation).  Every workload shape also runs in fp32, where one
missing or doubled key is far above the bound.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_long_sequence_lf_amd as lf
from sparse_long_sequence_lf_amd import workloads as W
from parity_utils import TOL, gpu_fwd, max_err, oracle_full, require_gpu, sample_rows

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# ---- every workload at a size the oracle finishes in seconds (full compare)
REDUCED = {
    "fp32-b1h2t1024-r64-g1": dict(),
    "bf16-b1h12t4096-r256-g1": dict(T=1280),
    "bf16-b1h12t4096-r128-dil": dict(T=1100),
    "bf16-b2h12t4096-r256-g68": dict(T=1000, H=6),
    "bf16-b4h16t16384-r512-g8-pad": dict(T=2100, H=3),
    "bf16-b1h12t4096-r256-g1-onesided": dict(T=1300),
    "bf16-b1h12t4096-rhead-g1": dict(T=1400),
    "bf16-b1h12t4096-r96-g2-rand3": dict(T=1500),
}


@pytest.mark.parametrize("dtype", ["native", "f32"])
@pytest.mark.parametrize("name", list(REDUCED))
def test_workload_reduced_full_compare(name, dtype):
    w = W.workload(name)
    dt = w.dtype if dtype == "native" else "f32"
    inp = W.make_inputs(w, dtype=dt, **REDUCED[name])
    print(f"case {name} dtype={dt} shape={tuple(inp.q.shape)}", flush=True)
    out = gpu_fwd(inp)
    ref = oracle_full(inp)
    err = max_err(out, ref)
    print(f"  max abs err {err:.3e}", flush=True)
    assert err <= TOL[dt]


# ---- every workload at its full size (the size the benchmark times): sampled rows
@pytest.mark.parametrize("dtype", ["native", "f32"])
@pytest.mark.parametrize("name", [w.name for w in W.WORKLOADS])
def test_workload_full_size_sampled(name, dtype):
    w = W.workload(name)
    dt = w.dtype if dtype == "native" else "f32"
    inp = W.make_inputs(w, dtype=dt)
    print(f"case {name} dtype={dt} shape={tuple(inp.q.shape)} full size", flush=True)
    out = gpu_fwd(inp)
    rows = sample_rows(inp, n_random=1500, seed=w.seed)
    ref = oracle.rows(inp.q, inp.k, inp.v, inp.r, rows, inp.dilation, inp.global_idx,
                      inp.key_padding_mask, one_sided=inp.one_sided, random_blocks=inp.random_blocks)
    got = out.float().cpu().double().reshape(-1, w.d).numpy()[rows]
    err = float(np.max(np.abs(got - ref)))
    print(f"  {len(rows)} rows, max abs err {err:.3e}", flush=True)
    assert err <= TOL[dt]
    if inp.key_padding_mask is not None:
        # every padded query row is exactly zero
        pad = inp.key_padding_mask.bool()
        o = out.float().cpu()
        for b in range(w.B):
            assert torch.all(o[b][:, pad[b]] == 0)


# ---- random edge cases: ragged T, r around T, dilation, duplicates, padding patterns
EDGE_T = [1, 2, 3, 31, 32, 33, 63, 64, 65, 97, 130, 257, 300]


@pytest.mark.parametrize("pad", ["none", "right", "random"])
@pytest.mark.parametrize("T", EDGE_T)
def test_edge_cases(T, pad):
    for dt in ("f32", "bf16"):
        for seed in range(2):
            inp = W.random_case(seed * 1000 + T, B=2, H=3, T=T, dtype=dt, pad=pad)
            print(f"case T={T} pad={pad} dt={dt} seed={seed} r={inp.r} dil={inp.dilation} "
                  f"G={inp.global_idx}", flush=True)
            out = gpu_fwd(inp)
            err = max_err(out, oracle_full(inp))
            assert err <= TOL[dt], err


# ---- one radius per head and one-sided windows (lf_attn_fwd_ex): ragged T,
# radii around T, dilation, duplicated globals, every padding pattern
@pytest.mark.parametrize("one_sided", [True, False])
@pytest.mark.parametrize("T", [1, 2, 31, 33, 64, 65, 130, 257, 300])
def test_window_forms(T, one_sided):
    for dt in ("f32", "bf16"):
        for seed, pad in enumerate(("none", "right", "random")):
            base = W.random_case(seed * 7919 + T + 11, B=2, H=3, T=T, dtype=dt, pad=pad)
            rng = np.random.default_rng(seed * 31 + T)
            rads = [int(x) for x in rng.integers(0, T + 3, size=3)]
            inp = W.Inputs(base.q, base.k, base.v, rads, base.dilation, base.global_idx, base.lengths,
                           base.key_padding_mask, one_sided=one_sided)
            print(f"case T={T} one_sided={one_sided} dt={dt} pad={pad} radii={rads} dil={inp.dilation} "
                  f"G={inp.global_idx}", flush=True)
            out = gpu_fwd(inp)
            err = max_err(out, oracle_full(inp))
            assert err <= TOL[dt], err


# ---- random key blocks (lf_attn_fwd_ex): ragged T, blocks that repeat or
# overlap the window, globals inside random blocks, padding, both window forms
@pytest.mark.parametrize("n_rand", [1, 3])
@pytest.mark.parametrize("T", [1, 63, 64, 65, 200, 300, 700])
def test_random_blocks(T, n_rand):
    for dt in ("f32", "bf16"):
        for seed, pad in enumerate(("none", "right", "random")):
            base = W.random_case(seed * 104729 + T + n_rand, B=2, H=3, T=T, dtype=dt, pad=pad, n_rand=n_rand)
            rng = np.random.default_rng(seed * 17 + T)
            one = bool(seed % 2)
            r = [int(x) for x in rng.integers(0, 100, size=3)] if seed == 2 else int(rng.integers(0, 100))
            inp = W.Inputs(base.q, base.k, base.v, r, base.dilation, base.global_idx, base.lengths,
                           base.key_padding_mask, one_sided=one, random_blocks=base.random_blocks)
            print(f"case T={T} n_rand={n_rand} dt={dt} pad={pad} r={r} one_sided={one} G={inp.global_idx}",
                  flush=True)
            out = gpu_fwd(inp)
            err = max_err(out, oracle_full(inp))
            assert err <= TOL[dt], err


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_named_edge_cases(dt):
    base = W.random_case(5, B=2, H=2, T=200, dtype=dt, pad="none")
    cases = []
    # r = 0, no globals (identity); r >= T (dense); T < r; G = all positions
    for r, G, dil in [(0, [], [1, 1]), (300, [], [1, 1]), (250, [3], [1, 2]), (5, list(range(200)), [1, 3]),
                      (7, [10, 12, 100], [1, 1]),        # global inside and outside the window
                      (3, [0, 199], [4, 5]),             # delta not dividing T
                      (40, [50, 50, 50, 51], [3, 1])]:   # duplicated globals
        cases.append((r, G, dil, None))
    kpm = torch.zeros(2, 200, dtype=torch.uint8)
    kpm[0, 150:] = 1
    kpm[1, :] = 1                                         # a fully padded sequence
    cases.append((9, [20, 160], [1, 2], kpm))             # a global inside the padding
    kpm2 = torch.zeros(2, 200, dtype=torch.uint8)
    kpm2[1, 90:] = 1
    cases.append((30, [95], [2, 1], kpm2))
    for r, G, dil, m in cases:
        inp = W.Inputs(base.q, base.k, base.v, r, dil, G, None, m)
        print(f"case r={r} G={G[:6]} dil={dil} pad={'yes' if m is not None else 'no'}", flush=True)
        out = gpu_fwd(inp)
        err = max_err(out, oracle_full(inp))
        assert err <= TOL[dt], err
        if r == 0 and not G and dt == "bf16":
            assert torch.equal(out.cpu(), base.v)   # a single key: y_i = v_i exactly


# ---- the neighbour set itself, at bf16: q = 0 makes every weight exactly 1, and
# one-hot values count the keys of each residue mod 64 in N(i)
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_tracer_counts_exact_neighbour_sets(dt):
    for name in ["bf16-b1h12t4096-r256-g1", "bf16-b1h12t4096-r128-dil", "bf16-b2h12t4096-r256-g68",
                 "bf16-b4h16t16384-r512-g8-pad", "bf16-b1h12t4096-r256-g1-onesided",
                 "bf16-b1h12t4096-rhead-g1", "bf16-b1h12t4096-r96-g2-rand3"]:
        w = W.workload(name)
        inp = W.make_inputs(w, dtype=dt, T=min(w.T, 1500), H=min(w.H, 4))
        B, H, T, d = inp.q.shape
        q0 = torch.zeros_like(inp.q)
        onehot = (torch.arange(T)[:, None] % d == torch.arange(d)[None, :]).to(inp.q.dtype)
        v1 = onehot.expand(B, H, T, d).contiguous()
        print(f"case {name} dt={dt} tracer", flush=True)
        out = gpu_fwd(inp, q=q0, v=v1).float().cpu().double().numpy()
        ref = oracle_full(inp, q=q0, v=v1)
        rel = np.abs(out - ref) / np.maximum(np.abs(ref), 1e-30)
        # bf16 output rounding is the only error left: 2^-8 relative
        assert float(np.max(np.where(ref != 0, rel, np.abs(out)))) <= 2 ** -8


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_large_score_range(dt):
    """Scores up to a few hundred (in units of the softmax's exponent) and
    keys whose scores grow along the sequence, so that the running max of a
    query moves on many blocks and the weights span many binades."""
    base = W.random_case(77, B=1, H=2, T=700, dtype=dt, pad="none")
    ramp = torch.linspace(0.2, 3.0, 700).view(1, 1, 700, 1)
    q = (base.q.float() * 4.0).to(base.q.dtype)
    k = (base.k.float() * 4.0 * ramp).to(base.k.dtype)
    # the flat bar of each dtype: fp32 inputs are carried in three bf16 parts,
    # so large scores keep fp32's own rounding error
    tol = TOL[dt]
    for r, G, dil in [(200, [5, 650], [1, 2]), (700, [], [1, 1])]:
        inp = W.Inputs(q, k, base.v, r, dil, G, None, None)
        print(f"case dt={dt} r={r} G={G} dil={dil} tol={tol:.2e}", flush=True)
        out = gpu_fwd(inp)
        err = max_err(out, oracle_full(inp))
        print(f"  max abs err {err:.3e}", flush=True)
        assert err <= tol, err


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_fully_padded_tiles(dt):
    """Right padding that leaves whole 64-query tiles of every residue class
    padded (one sequence entirely): those rows come out exactly zero even
    over an output filled with NaN, the rest matches the oracle, and globals
    sit inside and outside the padding."""
    B, H, T = 3, 4, 900
    base = W.random_case(91, B=B, H=H, T=T, dtype=dt, pad="none")
    kpm = torch.zeros(B, T, dtype=torch.uint8)
    kpm[0, 130:] = 1
    kpm[1, 700:] = 1
    kpm[2, :] = 1
    inp = W.Inputs(base.q, base.k, base.v, 40, [1, 2, 3, 1], [5, 400, 800], None, kpm)
    print(f"case dt={dt} fully padded tiles", flush=True)
    q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    out = torch.full_like(q, float("nan"))
    lf.attn_fwd(q, k, v, inp.r, inp.dilation, inp.global_idx, key_padding_mask=kpm.cuda(), out=out)
    torch.cuda.synchronize()
    err = max_err(out, oracle_full(inp))
    assert err <= TOL[dt], err
    o = out.float().cpu()
    for b in range(B):
        assert torch.all(o[b][:, kpm[b].bool()] == 0)


def test_nan_in_padded_positions_is_ignored():
    w = W.workload("bf16-b4h16t16384-r512-g8-pad")
    inp = W.make_inputs(w, T=1500, H=2)
    clean = gpu_fwd(inp).cpu()
    pad = inp.key_padding_mask.bool()
    q, k, v = inp.q.clone(), inp.k.clone(), inp.v.clone()
    for b in range(w.B):
        q[b][:, pad[b]] = float("nan")
        k[b][:, pad[b]] = float("nan")
        v[b][:, pad[b]] = float("inf")
    dirty = gpu_fwd(inp, q=q, k=k, v=v).cpu()
    assert torch.equal(clean, dirty)


def test_bitwise_deterministic_and_stream():
    w = W.workload("bf16-b2h12t4096-r256-g68")
    inp = W.make_inputs(w, T=2048)
    a = gpu_fwd(inp)
    b = gpu_fwd(inp)
    assert torch.equal(a, b)
    s = torch.cuda.Stream()
    q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        c = lf.attn_fwd(q, k, v, inp.r, inp.dilation, inp.global_idx)
    s.synchronize()
    assert torch.equal(a, c)


def test_no_writes_outside_out():
    w = W.workload("bf16-b1h12t4096-r256-g1")
    inp = W.make_inputs(w, T=777, H=3)
    q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    n = q.numel()
    guard = 4096
    big = torch.full((n + 2 * guard,), 7.0, dtype=q.dtype, device="cuda")
    out = big[guard:guard + n].view_as(q)
    lf.attn_fwd(q, k, v, inp.r, inp.dilation, inp.global_idx, out=out)
    torch.cuda.synchronize()
    assert torch.all(big[:guard] == 7.0) and torch.all(big[guard + n:] == 7.0)
    ref = oracle_full(inp)
    assert max_err(out, ref) <= TOL["bf16"]


def test_hf_style_global_mask_matches_index_list():
    w = W.workload("bf16-b2h12t4096-r256-g68")
    inp = W.make_inputs(w, T=600, H=2)
    q, k, v = inp.q.cuda(), inp.k.cuda(), inp.v.cuda()
    gm = torch.zeros(w.B, 600, dtype=torch.long)
    gm[:, inp.global_idx] = 1
    a = lf.attn_fwd(q, k, v, inp.r, global_attention_mask=gm)
    b = lf.attn_fwd(q, k, v, inp.r, global_idx=inp.global_idx)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_rejected_call_leaves_out_untouched():
    q = torch.randn(1, 2, 64, 64, device="cuda", dtype=torch.bfloat16)
    out = torch.full_like(q, 3.0)
    with pytest.raises(lf.LfError) as e:
        lf.attn_fwd(q, q, q, 4, global_idx=[64], out=out)   # global index out of range
    assert e.value.status == lf.LF_E_INVALID
    torch.cuda.synchronize()
    assert torch.all(out == 3.0)


def test_workspace_reuse_across_dtypes_and_shapes():
    """Calls of different dtype and shape share one stream's workspace: an
    fp32 call without globals (K/V planes in scratch), then calls with
    globals whose B*H grows (completion counters must still read zero), each
    against the oracle, with `out` prefilled with NaN so a row the kernel
    never writes shows up."""
    cases = [
        dict(seed=71, B=1, H=2, T=700, dtype="f32", r=40, n_global=0, pad="none"),
        dict(seed=72, B=1, H=3, T=500, dtype="bf16", r=30, n_global=40, pad="none"),
        dict(seed=73, B=3, H=5, T=400, dtype="bf16", r=20, n_global=70, pad="right"),
        dict(seed=74, B=2, H=2, T=600, dtype="f32", r=50, n_global=5, pad="random"),
        dict(seed=75, B=4, H=7, T=300, dtype="bf16", r=10, n_global=3, pad="none"),
    ]
    for c in cases:
        inp = W.random_case(c.pop("seed"), **c, max_dil=3)
        q, k, v = (x.to("cuda:0") for x in (inp.q, inp.k, inp.v))
        kpm = None if inp.key_padding_mask is None else inp.key_padding_mask.to("cuda:0")
        out = torch.full_like(q, float("nan"))
        lf.attn_fwd(q, k, v, inp.r, inp.dilation, inp.global_idx, key_padding_mask=kpm, out=out)
        torch.cuda.synchronize()
        err = max_err(out, oracle_full(inp))
        dt = "f32" if inp.q.dtype == torch.float32 else "bf16"
        print(f"  {tuple(inp.q.shape)} {dt} n_g={len(set(inp.global_idx))}: max abs err {err:.3e}", flush=True)
        assert err <= TOL[dt]


def test_random_table_change_same_shape():
    # consecutive calls of one shape and plan whose random-block tables differ:
    # each call must see its own table
    base = W.random_case(77, B=1, H=2, T=200, dtype="f32", pad="none", n_rand=2)
    for s in range(3):
        rb = np.random.default_rng(s).integers(0, 4, size=base.random_blocks.shape).astype(np.int32)
        inp = W.Inputs(base.q, base.k, base.v, base.r, base.dilation, base.global_idx, base.lengths,
                       base.key_padding_mask, random_blocks=rb)
        print(f"case random table {s}", flush=True)
        err = max_err(gpu_fwd(inp), oracle_full(inp))
        assert err <= TOL["f32"], (s, err)


@pytest.mark.parametrize("case", [
    dict(seed=81, B=1, H=3, T=700, dtype="bf16", r=40, n_global=3, pad="none"),
    dict(seed=82, B=2, H=2, T=530, dtype="f32", r=5, n_global=70, pad="right"),
    dict(seed=83, B=3, H=4, T=300, dtype="bf16", r=0, n_global=130, pad="random"),
    dict(seed=84, B=1, H=2, T=97, dtype="f32", r=9, n_global=1, pad="random"),
], ids=["bf16-3g", "f32-70g-right", "bf16-130g-random", "f32-1g-ragged"])
def test_global_rows_only(case):
    # lf_attn_fwd_global_rows: the global rows (out and lse) equal the oracle's
    # and, bit for bit, those of the whole forward; every other row keeps the
    # value it held before the call
    c = dict(case)
    inp = W.random_case(c.pop("seed"), **c, max_dil=3)
    B, H, T, d = inp.q.shape
    q, k, v = (x.to("cuda:0") for x in (inp.q, inp.k, inp.v))
    kpm = None if inp.key_padding_mask is None else inp.key_padding_mask.to("cuda:0")
    out = torch.full_like(q, 7.0)
    lse = torch.full((B, H, T), 5.0, dtype=torch.float32, device="cuda:0")
    lf.attn_fwd_global_rows(q, k, v, inp.global_idx, key_padding_mask=kpm, out=out, lse=lse)
    full = torch.empty_like(q)
    full_lse = torch.empty_like(lse)
    lf.attn_fwd(q, k, v, inp.r, inp.dilation, inp.global_idx, key_padding_mask=kpm, out=full, lse=full_lse)
    torch.cuda.synchronize()
    G = sorted(set(inp.global_idx))
    is_g = torch.zeros(T, dtype=torch.bool)
    is_g[G] = True
    dt = "f32" if inp.q.dtype == torch.float32 else "bf16"
    ref = oracle_full(inp)
    err = max_err(out[:, :, G], ref[:, :, G])
    print(f"  {tuple(inp.q.shape)} {dt} n_g={len(G)}: global rows max abs err {err:.3e}", flush=True)
    assert err <= TOL[dt]
    assert torch.equal(out[:, :, G], full[:, :, G])
    assert torch.equal(lse[:, :, G], full_lse[:, :, G])
    rest = out[:, :, ~is_g.to("cuda:0")]
    assert bool((rest == 7.0).all()), "a row outside G was written"
    assert bool((lse[:, :, ~is_g.to("cuda:0")] == 5.0).all()), "an lse outside G was written"


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_unequal_radii_many_globals(dt):
    # heads of unequal radii cut into per-die runs of equal cost, with two and
    # three groups of global rows assigned to the dies of their heads' tiles
    for seed, (B, H, T, n_g, pad) in enumerate([(3, 5, 500, 70, "right"), (2, 7, 700, 140, "random"),
                                                (4, 3, 260, 65, "none")]):
        base = W.random_case(9100 + seed, B=B, H=H, T=T, dtype=dt, n_global=n_g, pad=pad, max_dil=3)
        rng = np.random.default_rng(9200 + seed)
        rads = [int(x) for x in rng.integers(0, T // 2, size=H)]
        inp = W.Inputs(base.q, base.k, base.v, rads, base.dilation, base.global_idx, base.lengths,
                       base.key_padding_mask, one_sided=bool(seed % 2))
        print(f"case B={B} H={H} T={T} n_g={len(set(inp.global_idx))} radii={rads} dil={inp.dilation}", flush=True)
        err = max_err(gpu_fwd(inp), oracle_full(inp))
        assert err <= TOL[dt], err


@pytest.mark.parametrize("case", [
    # one (b, h): 64 splits of 64 keys, the most a head takes (the combine
    # reads eight rounds of eight records)
    dict(seed=91, B=1, H=1, T=4096, dtype="f32", r=30, n_global=1, pad="none"),
    # two heads, a ragged length: 53 splits of 96 keys, the last one short
    dict(seed=92, B=1, H=2, T=5000, dtype="bf16", r=70, n_global=3, pad="none"),
    # twelve heads: 12 splits of 352 keys (the headline's split plan) with padding
    dict(seed=93, B=1, H=12, T=4096, dtype="f32", r=16, n_global=2, pad="right"),
], ids=["f32-64splits", "bf16-53splits-ragged", "f32-12splits-pad"])
def test_global_row_split_counts(case):
    # the global-row split plan at its extremes: every global row (and its
    # lse) against the oracle, and a sample of the other rows
    c = dict(case)
    inp = W.random_case(c.pop("seed"), **c, max_dil=1)
    B, H, T, d = inp.q.shape
    dt = "f32" if inp.q.dtype == torch.float32 else "bf16"
    print(f"case {tuple(inp.q.shape)} {dt} r={inp.r} G={sorted(set(inp.global_idx))}", flush=True)
    q, k, v = (x.to("cuda:0") for x in (inp.q, inp.k, inp.v))
    kpm = None if inp.key_padding_mask is None else inp.key_padding_mask.to("cuda:0")
    lse = torch.empty(B, H, T, dtype=torch.float32, device="cuda:0")
    out = lf.attn_fwd(q, k, v, inp.r, inp.dilation, inp.global_idx, key_padding_mask=kpm, lse=lse)
    torch.cuda.synchronize()
    G = sorted(set(inp.global_idx))
    rows = sorted(set(G) | set(range(0, T, 97)) | {T - 1})
    ref, ref_lse = oracle.fwd_lse(inp.q, inp.k, inp.v, inp.r, inp.dilation, inp.global_idx, inp.key_padding_mask)
    err = max_err(out[:, :, rows], ref[:, :, rows])
    print(f"  rows {len(rows)}: max abs err {err:.3e}", flush=True)
    assert err <= TOL[dt], err
    got_lse = lse[:, :, G].cpu().double().numpy()
    want_lse = ref_lse[:, :, G]
    fin = np.isfinite(want_lse)
    assert np.array_equal(np.isfinite(got_lse), fin)
    assert np.max(np.abs(got_lse[fin] - want_lse[fin]), initial=0.0) <= 1e-4 * max(1.0, np.max(np.abs(want_lse[fin]), initial=0.0))
