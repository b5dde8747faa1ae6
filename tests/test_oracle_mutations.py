"""Planted mistakes in the fp64 oracle must be caught by its pins.

Each case below plants one plausible error in a copy of oracle/gdn_oracle.c (a
dropped term, a wrong sign or index, a transposed operand, a missing
activation), builds the copy with gcc, points the oracle wrapper at it, and
runs every pin of tests/test_oracle_pins.py.  A case passes when at least one
pin fails on the mutant; a mutant that every pin accepts would mean the pins
do not fix that part of the oracle.  CPU only; the real oracle is restored
after each case.
"""
import inspect
import itertools
import os
import subprocess

import pytest

import oracle
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(os.path.abspath(oracle.__file__)), "gdn_oracle.c")

# (name, text in gdn_oracle.c, replacement): each text occurs exactly once.
MUTANTS = [
    ("alpha dropped from the erase term",
     "u[jj] = bt * (vv[jj] - a * u[jj]);", "u[jj] = bt * (vv[jj] - u[jj]);"),
    ("alpha dropped from the decay",
     "M[i * nj + jj] = a * M[i * nj + jj] + kv[i] * u[jj];", "M[i * nj + jj] = M[i * nj + jj] + kv[i] * u[jj];"),
    ("sign of the write flipped",
     "M[i * nj + jj] = a * M[i * nj + jj] + kv[i] * u[jj];", "M[i * nj + jj] = a * M[i * nj + jj] - kv[i] * u[jj];"),
    ("beta dropped",
     "u[jj] = bt * (vv[jj] - a * u[jj]);", "u[jj] = (vv[jj] - a * u[jj]);"),
    ("erase reads q instead of k",
     "for (int64_t jj = 0; jj < nj; ++jj) u[jj] += M[i * nj + jj] * kv[i];",
     "for (int64_t jj = 0; jj < nj; ++jj) u[jj] += M[i * nj + jj] * qv[i];"),
    ("key head h mod Hk instead of h / G",
     "hk = h / G;", "hk = h % d->Hk;"),
    ("state transposed on load",
     "M[i * nj + jj] = ld(state_in, d->state_dtype, ((b * Hv + h) * Dk + i) * Dv + j0 + jj);",
     "M[i * nj + jj] = ld(state_in, d->state_dtype, ((b * Hv + h) * Dk + (j0 + jj)) * Dv + i);"),
    ("output read before the update",
     "/* o = M^T q, read after the update */\n      if (o_out) {",
     "/* o = M^T q, read after the update */\n      if (o_out && t < 0) {"),
    ("q scale dropped", "for (int64_t i = 0; i < Dk; ++i) qv[i] *= d->q_scale;",
     "for (int64_t i = 0; i < Dk; ++i) qv[i] *= 1.0;"),
    ("L2 normalisation skipped", "if (d->l2norm) {", "if (0) {"),
    ("conv taps reversed", "acc += ld(w, w_dtype, c * K + j) * xv;", "acc += ld(w, w_dtype, c * K + (K - 1 - j)) * xv;"),
    ("conv window one token late", "const int64_t ts = t - (K - 1) + j;", "const int64_t ts = t - K + j;"),
    ("SiLU missing", "y_out[(t - t0) * nc + (c - c0)] = acc * sigmoid(acc);",
     "y_out[(t - t0) * nc + (c - c0)] = acc;"),
    ("norm epsilon outside the root", "const double inv = 1.0 / sqrt(ss / (double)D + eps);",
     "const double inv = 1.0 / (sqrt(ss / (double)D) + eps);"),
    ("norm over the sum instead of the mean", "const double inv = 1.0 / sqrt(ss / (double)D + eps);",
     "const double inv = 1.0 / sqrt(ss + eps);"),
    ("gate z without its sigmoid",
     "y_out[si * D + i] = ld(x, x_dtype, r * D + i) * inv * ld(w, w_dtype, i) * zv * sigmoid(zv);",
     "y_out[si * D + i] = ld(x, x_dtype, r * D + i) * inv * ld(w, w_dtype, i) * zv;"),
    ("beta and alpha outputs swapped",
     "const double b = ld(ba, ba_dtype, t * stride + h);\n      const double a = ld(ba, ba_dtype, t * stride + Hv + h);",
     "const double a = ld(ba, ba_dtype, t * stride + h);\n      const double b = ld(ba, ba_dtype, t * stride + Hv + h);"),
    ("softplus without its log", "log1p(exp(a + ld(dt_bias, p_dtype, h)))", "exp(a + ld(dt_bias, p_dtype, h))"),
    ("bf16 rounding ties away from zero", "nearbyint(xv / unit)", "round(xv / unit)"),
]


def _pin_calls():
    """Every pin of test_oracle_pins as (name, zero-argument callable), parametrizations expanded."""
    calls = []
    for name, fn in inspect.getmembers(pins, inspect.isfunction):
        if not name.startswith("test_"):
            continue
        marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            calls.append((name, fn))
            continue
        axes = []
        for m in marks:
            argnames = [a.strip() for a in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
            values = [v if len(argnames) > 1 else (v,) for v in m.args[1]]
            axes.append([dict(zip(argnames, v)) for v in values])
        for combo in itertools.product(*axes):
            kw = {}
            for d in combo:
                kw.update(d)
            calls.append((f"{name}{kw}", (lambda f, k: lambda: f(**k))(fn, kw)))
    return calls


@pytest.fixture(scope="module")
def mutant_dir(tmp_path_factory):
    return tmp_path_factory.mktemp("oracle_mutants")


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_is_caught(name, old, new, mutant_dir, monkeypatch):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site not found once in gdn_oracle.c: {old!r}"
    tag = "".join(c if c.isalnum() else "_" for c in name)
    c_path = os.path.join(mutant_dir, f"{tag}.c")
    so_path = os.path.join(mutant_dir, f"{tag}.so")
    open(c_path, "w").write(src.replace(old, new))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", c_path, "-o", so_path, "-lm"],
                   check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(so_path))
    caught = []
    for pin_name, call in _pin_calls():
        try:
            call()
        except Exception:       # an assertion, or an error the mutant provokes
            caught.append(pin_name)
    assert caught, f"no pin fails when the oracle has this mistake: {name}"
    print(f"{name}: caught by {len(caught)} pin runs, e.g. {caught[:3]}")


def test_unmutated_copy_passes_every_pin(mutant_dir, monkeypatch):
    """Control: the same build steps on the unchanged source give a library every pin accepts,
    so a failure above comes from the planted mistake alone."""
    c_path = os.path.join(mutant_dir, "control.c")
    so_path = os.path.join(mutant_dir, "control.so")
    open(c_path, "w").write(open(SRC).read())
    subprocess.run(["gcc", "-O1", "-std=c11", "-fopenmp", "-fPIC", "-shared", c_path, "-o", so_path, "-lm"],
                   check=True)
    monkeypatch.setattr(oracle, "_lib", oracle.load_library(so_path))
    failed = []
    for pin_name, call in _pin_calls():
        try:
            call()
        except Exception as e:
            failed.append((pin_name, repr(e)[:200]))
    assert not failed, failed
