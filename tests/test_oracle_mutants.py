"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant is a copy of oracle/lce_oracle.c with one plausible mistake (a
dropped term, a wrong sign or index, a transposed operand, a wrong
denominator...).  It is compiled into a temporary library and every pin in
oracle_pins.py is run against it; at least one pin must fail.  The real
oracle is never modified.
"""
import os
import subprocess

import pytest

import oracle
from oracle_pins import PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "lce_oracle.c")

MUTANTS = [
    ("drop smoothing term of the loss", "- (eps / (double)V) * zsum;", ";"),
    ("drop (1-eps) weight of the target logit", "- (1.0 - eps) * z[y]", "- z[y]"),
    ("target logit read before the cap", "- (1.0 - eps) * z[y]", "- (1.0 - eps) * x[y]"),
    ("lse without the max shift", "double lse = m + log(s);", "double lse = log(s);"),
    ("wrong sign of the target gradient", "dz = -(s_other / s) + eps - eps / (double)V;",
     "dz = (s_other / s) + eps - eps / (double)V;"),
    ("drop eps/V from the off-target gradient", "dz = exp(z[j] - lse) - eps / (double)V;",
     "dz = exp(z[j] - lse);"),
    ("drop the softcap chain factor", "chain = 1.0 / (c * c);", "chain = 1.0;"),
    ("chain factor sech instead of sech^2", "chain = 1.0 / (c * c);", "chain = 1.0 / c;"),
    ("softcap without the T multiplier", "T > 0.0 ? T * tanh(x[j] / T) : x[j]", "T > 0.0 ? tanh(x[j] / T) : x[j]"),
    ("argmax keeps the last tied index", "if (x[j] > x[am]) am = j;", "if (x[j] >= x[am]) am = j;"),
    ("mean forgets to divide by n_valid", "return n_valid > 0 ? g / (double)n_valid : 0.0;",
     "return n_valid > 0 ? g : 0.0;"),
    ("bad labels counted as valid", "if (label_is_valid(y, V, ignore_index)) ++nv;", "if (y != ignore_index) ++nv;"),
    ("row stride ignores ld", "x[j] = load_elem(logits, dtype, i * ld + j);", "x[j] = load_elem(logits, dtype, i * V + j);"),
    ("row subset ignored", "int64_t i = rows ? rows[r] : r;", "int64_t i = r;"),
    ("bf16 rounding ties away from zero", "double r = nearbyint(m);", "double r = round(m);"),
    ("transposed weight in grad_hidden", "acc += g[i * V + v] * w[v * H + k];", "acc += g[i * V + v] * w[k * H + v % H];"),
    ("grad_weight uses weight instead of hidden", "acc += g[i * V + v] * h[i * H + k];",
     "acc += g[i * V + v] * w[v * H + k];"),
    ("entropy with the wrong sign", "h -= exp(lp) * lp;", "h += exp(lp) * lp;"),
    ("entropy weighted by z instead of log p", "h -= exp(lp) * lp;", "h -= exp(lp) * z[j];"),
    ("target log-probability before the cap", "? z[y] - lse_r : 0.0;",
     "? load_elem(logits, dtype, row_i * ld + y) - lse_r : 0.0;"),
    ("row statistics without the max shift", "const double lse_r = m + log(s);", "const double lse_r = log(s);"),
    ("row statistics ignore the row subset", "const int64_t row_i = rows ? rows[r] : r;", "const int64_t row_i = r;"),
    ("fused-linear scale ignores the reduction",
     "double scale = token_scale(reduction, grad_out, i, n_valid);\n            int64_t am;\n            ce_row(zrow",
     "double scale = token_scale(OR_RED_SUM, grad_out, i, n_valid);\n            int64_t am;\n            ce_row(zrow"),
    ("ignored rows keep a loss", "        *loss = 0.0;\n        if (grad)", "        *loss = 1.0;\n        if (grad)"),
]


@pytest.mark.parametrize("desc,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(desc, old, new, tmp_path):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor not unique/present: {old!r}"
    mpath = tmp_path / "mutant.c"
    mpath.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                    "-o", str(lib), str(mpath), "-lm"], check=True)
    orc = oracle.Oracle(str(lib))
    caught = []
    for pin in PINS:
        try:
            pin(orc)
        except (AssertionError, ValueError) as e:
            caught.append(f"{pin.__name__}: {str(e)[:80]}")
            break
    assert caught, f"no pin caught the planted mistake: {desc}"
