"""The oracle's pins catch planted mistakes.

Each mutant is a copy of oracle.c with one plausible slip (a dropped term, a
transposed factor, a wrong sign, index or tie rule).  It is compiled on the
CPU into a scratch library and the pin suite is run against it; every mutant
must make at least one pin fail.  CPU only.
"""
import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "oracle.c")

MUTANTS = {
    "residual dropped from the page score":
        ("for (int x = 0; x < R + RK; ++x)", "for (int x = 0; x < R; ++x)"),
    "page score not divided by the token count":
        ("double sc = d->scale * dot / cnt;", "double sc = d->scale * dot;"),
    "basis used transposed in the writer":
        ("(double)B[((size_t)g * D + i) * R + j];\n    z[j]", "(double)B[((size_t)g * R + j) * D + i];\n    z[j]"),
    "Key remainder with the wrong sign":
        ("e[i] = ld(k, row * D + i, d->dtype) - khat;", "e[i] = ld(k, row * D + i, d->dtype) + khat;"),
    "ties go to the larger page":
        ("return (x->page > y->page) - (x->page < y->page);", "return (x->page < y->page) - (x->page > y->page);"),
    "softmax scale dropped":
        ("s[x] = d->scale * acc;", "s[x] = acc;"),
    "sum over heads instead of max":
        ("if (sc > best) best = sc;", "best = (best == -INFINITY ? 0 : best) + sc;"),
    "last page counted full":
        ("int cnt = n - j * ps < ps ? n - j * ps : ps;\n      double best", "int cnt = ps;\n      double best"),
    "fold without the basis":
        ("acc += (double)B[((size_t)g * D + i) * R + j] *", "acc += (double)(i == j) *"),
    "summary over one slot too many":
        ("int valid = end - page * ps;", "int valid = end - page * ps + 1;"),
    "per-head routing scores the group's first head":
        ("int h0 = d->head_select ? u : g * G;     /* its first query head */",
         "int h0 = g * G;     /* its first query head */"),
    "per-head decode attends with the group's first head":
        ("int h0 = d->head_select ? u : g * G;\n    int n = seq_lens[b];\n    int ns",
         "int h0 = g * G;\n    int n = seq_lens[b];\n    int ns"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor not unique: {name}"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    lib = oracle.compile_to(str(src), str(tmp_path / "libmutant.so"), werror=False)
    env = dict(os.environ, BASISKV_ORACLE_LIB=lib, OMP_NUM_THREADS="2")
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert r.returncode != 0, f"pins did not catch: {name}\n{r.stdout[-2000:]}"
