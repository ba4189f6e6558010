"""Plant plausible mistakes in copies of the oracle and check that the pins
catch each one (CPU only; the planted copies live in a temporary directory).

A pin set that lets a dropped term, a swapped index or a reversed chain
through would not be worth trusting; every mutant below must fail at least
one pin.
"""
import os
import subprocess
import sys

import pytest

import oracle

SRC = os.path.join(os.path.dirname(oracle.__file__), "ks_oracle.c")

# (name, exact text in ks_oracle.c, replacement)
MUTANTS = [
    ("swap_beta_gamma_in_K",
     "* b + beta) * c + gamma];\n                    double v = x[", "* c + gamma) * b + beta];\n                    double v = x["),
    ("swap_alpha_delta_in_K",
     "double k = K[(((long long)alpha * d + delta) * b + beta) * c + gamma];\n                    double v = x[",
     "double k = K[(((long long)delta * a + alpha) * b + beta) * c + gamma];\n                    double v = x["),
    ("transpose_x_block",
     "double v = x[((long long)alpha * c + gamma) * d + delta];", "double v = x[((long long)alpha * d + delta) * c + gamma];"),
    ("transpose_y_block",
     " y[((long long)alpha * b + beta) * d + delta] = acc;", " y[((long long)alpha * d + delta) * b + beta] = acc;"),
    ("drop_last_gamma",
     "for (int gamma = 0; gamma < c; ++gamma) {\n                    double k",
     "for (int gamma = 0; gamma < c - 1; ++gamma) {\n                    double k"),
    ("skip_first_gamma",
     "for (int gamma = 0; gamma < c; ++gamma) {\n                    double k",
     "for (int gamma = 1; gamma < c; ++gamma) {\n                    double k"),
    ("wrong_sign",
     "acc += k * v;", "acc += (gamma == 1 ? -k : k) * v;"),
    ("dx_swap_beta_gamma_in_K",
     "double k = K[(((long long)alpha * d + delta) * b + beta) * c + gamma];\n                    double g = dy",
     "double k = K[(((long long)alpha * d + delta) * c + gamma) * b + beta];\n                    double g = dy"),
    ("dx_drop_last_beta",
     "for (int beta = 0; beta < b; ++beta) {\n                    double k", "for (int beta = 0; beta < b - 1; ++beta) {\n                    double k"),
    ("dx_transpose_dy_block",
     "double g = dy[((long long)alpha * b + beta) * d + delta];", "double g = dy[((long long)alpha * d + delta) * b + beta];"),
    ("dw_drop_first_row",
     "for (long long n = 0; n < batch; ++n) {\n                    double g = dY", "for (long long n = 1; n < batch; ++n) {\n                    double g = dY"),
    ("dw_swap_alpha_delta_in_dK",
     "dK[(((long long)alpha * d + delta) * b + beta) * c + gamma] = acc;", "dK[(((long long)delta * a + alpha) * b + beta) * c + gamma] = acc;"),
    ("dw_transpose_output_block",
     "dK[(((long long)alpha * d + delta) * b + beta) * c + gamma] = acc;", "dK[(((long long)alpha * d + delta) * c + gamma) * b + beta] = acc;"),
    ("dw_x_at_wrong_delta",
     "double v = X[n * n_in + ((long long)alpha * c + gamma) * d + delta];", "double v = X[n * n_in + ((long long)alpha * c + gamma) * d + (d - 1 - delta)];"),
    ("reverse_chain",
     "ks_factor_row(pat[4 * k], pat[4 * k + 1], pat[4 * k + 2], pat[4 * k + 3],\n                      Ks[k], cur, out);",
     "ks_factor_row(pat[4 * (nf - 1 - k)], pat[4 * (nf - 1 - k) + 1], pat[4 * (nf - 1 - k) + 2], pat[4 * (nf - 1 - k) + 3],\n                      Ks[nf - 1 - k], cur, out);"),
]


_RUNNER = r"""
import sys
sys.path[:0] = [%r, %r]
import oracle, oracle_pins
lib = oracle.load(sys.argv[1])
failed = []
for pin in oracle_pins.ALL_PINS:
    try:
        pin(lib)
    except (AssertionError, ValueError):
        failed.append(pin.__name__)
print("FAILED_PINS", ",".join(failed))
"""


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(tmp_path, name, old, new):
    with open(SRC) as f:
        text = f.read()
    assert text.count(old) == 1, "mutation site not found: %s" % name
    src = tmp_path / ("ks_oracle_%s.c" % name)
    src.write_text(text.replace(old, new))
    so = str(tmp_path / ("libks_oracle_%s.so" % name))
    oracle.build(force=True, out=so, src=str(src), extra_flags=["-w"])
    # A mutant may read or write out of bounds; run it in its own process so
    # that a corrupted heap cannot reach this one. A crash counts as caught,
    # and so does a hang (a corrupted heap can leave the process spinning):
    # the unmutated pins take about a second.
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    tests = os.path.dirname(os.path.abspath(__file__))
    try:
        proc = subprocess.run([sys.executable, "-c", _RUNNER % (root, tests), so],
                              capture_output=True, text=True, timeout=120)
    except subprocess.TimeoutExpired:
        return
    if proc.returncode != 0:
        return
    line = [l for l in proc.stdout.splitlines() if l.startswith("FAILED_PINS")][-1]
    failed = [x for x in line.split(" ", 1)[1].split(",") if x] if " " in line else []
    assert failed, "mutant %s passed every pin" % name
