"""CPU tests that pin the fp64 oracle (oracle/lf_oracle.c) to the pages.

See tests/oracle_pins.py for what each pin is.  The last test plants
mistakes in copies of the oracle and checks that every one is caught.
"""
import os
import subprocess
import sys

import pytest

import oracle
import oracle_pins as P

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                          "oracle", "lf_oracle.c")


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check, oracle_mod):
    check()


# Planted mistakes: (name, text in lf_oracle.c, replacement).  Each must be
# caught by at least one pin.
MUTANTS = [
    ("no_scale", "s[t] = dot * inv_sqrt_d;", "s[t] = dot;"),
    ("dilation_ignored", "int j = (int)((long long)i + t * delta);", "int j = (int)((long long)i + t);"),
    ("global_counted_twice", "if (gi < G->n && G->pos[gi] == j) gi++;", ""),
    ("window_keeps_padded_keys", "if (!(pad && pad[j])) out[n++] = j;", "out[n++] = j;"),
    ("softmax_sign", "s[t] = exp(s[t] - m);", "s[t] = exp(m - s[t]);"),
    ("k_v_swapped", "jb->k + base, jb->v + base", "jb->v + base, jb->k + base"),
    ("no_normalisation", "for (int c = 0; c < d; c++) yi[c] /= l;", ""),
    ("window_one_short", "thi = (long long)r;", "thi = (long long)r - 1;"),
    ("global_rows_local", "if (gset_has(G, i)) {", "if (0) {"),
    ("padded_query_not_zero", "if (pad && pad[i]) return 0;", ""),
    ("globals_padded_kept", "if (!(pad && pad[g])) out[n++] = g;\n        }", "out[n++] = g;\n        }"),
    ("q_row_offset", "jb->q + base + (size_t)i * jb->d", "jb->q + base + (size_t)(i + 1 < jb->T ? i + 1 : i) * jb->d"),
    ("one_sided_ignored", "if (one_sided) thi = 0;", ""),
    ("one_sided_wrong_side", "if (one_sided) thi = 0;", "if (one_sided) tlo = 0;"),
    ("head_radius_ignored", "int rh = jb->rad ? jb->rad[h] : jb->r;", "int rh = jb->r;"),
    ("random_blocks_ignored", "if (rblk && n_rand > 0) {", "if (0) {"),
    ("random_block_shifted", "const int j0 = rb[e] * RAND_BLOCK;", "const int j0 = rb[e] * RAND_BLOCK + 1;"),
    ("random_padded_kept", "if (!(pad && pad[j])) mark[j] = 1;", "mark[j] = 1;"),
    ("random_block_of_wrong_query", "rblk + (size_t)(i / RAND_BLOCK) * n_rand", "rblk + (size_t)(i / RAND_BLOCK / 2) * n_rand"),
    ("lse_without_max", "if (lse) *lse = m + log(l);", "if (lse) *lse = log(l);"),
    ("lse_base_two", "if (lse) *lse = m + log(l);", "if (lse) *lse = m + log2(l);"),
    ("lse_of_padded_row_zero", "if (lse) *lse = -INFINITY;", "if (lse) *lse = 0.0;"),
    ("grad_no_D_term", "D += s[t] * dp;", ""),
    ("grad_dk_unscaled", "dK[(size_t)j * d + c] += ds * inv_sqrt_d * (double)qi[c];",
     "dK[(size_t)j * d + c] += ds * (double)qi[c];"),
    ("grad_weights_unnormalised", "s[t] /= l;", ""),
    ("grad_dq_from_v", "dqi[c] += ds * inv_sqrt_d * (double)kj[c];", "dqi[c] += ds * inv_sqrt_d * (double)V[(size_t)j * d + c];"),
    ("keys_dv_from_q", "dvj[c] += s[t] * (double)dyi[c];", "dvj[c] += s[t] * (double)qi[c];"),
    ("keys_search_off_by_one", "return lo < n && nb[lo] == j ? lo : -1;",
     "return lo + 1 < n && nb[lo] == j ? lo + 1 : -1;"),
    ("grad_dv_sign", "dV[(size_t)j * d + c] += s[t] * (double)dyi[c];", "dV[(size_t)j * d + c] -= s[t] * (double)dyi[c];"),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, tmp_path):
    src = open(ORACLE_SRC).read()
    assert old in src, f"mutation anchor for {name} not found"
    mut = tmp_path / "mut.c"
    mut.write_text(src.replace(old, new, 1))
    so = str(tmp_path / "libmut.so")
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                           "-pthread", str(mut), "-o", so, "-lm"])
    # run the pins against the copy in a child process: some planted mistakes
    # write past their buffers, and that must not take the test runner down
    here = os.path.dirname(os.path.abspath(__file__))
    code = (
        "import sys; sys.path[:0] = [%r, %r]\n"
        "import oracle, oracle_pins as P\n"
        "lib = oracle.open_library(%r)\n"
        "caught = []\n"
        "for check in P.ALL_CHECKS:\n"
        "    try:\n"
        "        check(lib=lib)\n"
        "    except (AssertionError, ValueError, IndexError):\n"
        "        caught.append(check.__name__)\n"
        "print('CAUGHT', ','.join(caught))\n"
    ) % (here, os.path.dirname(here), so)
    res = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=600)
    if res.returncode == 0:
        line = [l for l in res.stdout.splitlines() if l.startswith("CAUGHT")][-1]
        assert line.strip() != "CAUGHT", f"planted mistake {name} passed every pin"
    # a non-zero exit (crash inside the planted copy) also counts as caught
