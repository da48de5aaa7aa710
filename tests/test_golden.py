"""The oracle against the figures the pages print (tests/golden/page_figures.txt,
each line with its source): window sizes and spans of plain and dilated
windows, and how the pair count grows with the sequence length."""
import os

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _rows():
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", "page_figures.txt"), encoding="utf-8") as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, args, want, src = [x.strip() for x in line.split("|")]
            kw = dict(a.split("=") for a in args.split())
            rows.append((name, {k: int(v) for k, v in kw.items()}, float(want), src))
    return rows


ROWS = _rows()


@pytest.mark.parametrize("name,kw,want,src", ROWS, ids=[f"{r[0]}-{i}" for i, r in enumerate(ROWS)])
def test_page_figure(name, kw, want, src):
    if name in ("dilated_window_keys", "dilated_window_span", "window_keys"):
        keys = oracle.neighbours(kw["T"], kw["r"], kw["delta"], kw["i"])
        got = len(keys) if name != "dilated_window_span" else max(keys) - min(keys)
        assert got == want, (src, got)
    elif name == "dense_pairs_ratio":
        T, base = kw["T"], kw["base"]
        got = oracle.count_pairs(1, 1, T, T) / oracle.count_pairs(1, 1, base, base)
        assert got == want, (src, got)
    elif name == "window_pairs_ratio":
        T, base, r = kw["T"], kw["base"], kw["r"]
        got = oracle.count_pairs(1, 1, T, r) / oracle.count_pairs(1, 1, base, r)
        assert abs(got - want) <= 0.01 * want, (src, got)
    else:
        raise AssertionError(f"unknown figure {name}")
