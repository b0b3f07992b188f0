"""Plants plausible mistakes in copies of the gradient oracle's reverse pass (on the CPU)
and checks that the gradient pins catch every one."""
import ctypes
import os
import subprocess

import pytest

from grad_pins import all_grad_pins
from oracle import ssd_oracle as so

HERE = os.path.dirname(so.__file__)
SRC = os.path.join(HERE, "ssd_oracle.c")
SRC_GRAD = os.path.join(HERE, "ssd_oracle_grad.c")

# (name, text in the reverse pass, replacement)
MUTANTS = [
    ("dfinal-dropped", "if (J->dfinal) memcpy(Lam,", "if (0) memcpy(Lam,"),
    ("adjoint-not-decayed", "for (int64_t i = 0; i < PS; ++i) Lam[i] *= alpha;",
     "for (int64_t i = 0; i < PS; ++i) Lam[i] *= 1.0;"),
    ("dB-without-dt", "dBt[s] += dtv * db;", "dBt[s] += db;"),
    ("dC-from-previous-state", "dc += Ht[p * S + s] * dyt[p];", "dc += Hprev[p * S + s] * dyt[p];"),
    ("decay-gradient-from-current-state", "inner += Lam[i] * Hprev[i];",
     "inner += Lam[i] * Ht[i];"),
    ("ddt-sign", "= v + Ah * da;", "= v - Ah * da;"),
    ("dA-without-dt", "dA += dtv * da;", "dA += da;"),
    ("dx-without-skip", "dxt[p] = Dh * dyt[p] + dtv * acc;", "dxt[p] = dtv * acc;"),
    ("checkpoint-off-by-one", "if (t % CKPT == 0) memcpy(ckpt", "if (t % CKPT == 1) memcpy(ckpt"),
]


def _build(tmp_path, name, old, new):
    src = open(SRC_GRAD).read()
    assert src.count(old) == 1, f"mutation {name!r} does not apply"
    cpath = tmp_path / f"{name}_grad.c"
    cpath.write_text(src.replace(old, new))
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared",
                    "-std=c99", "-o", str(lib), SRC, str(cpath), "-lm", "-lpthread"], check=True)
    return str(lib)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_grad_pins_catch_mutant(tmp_path, monkeypatch, name, old, new):
    real = so._load()
    lib = ctypes.CDLL(_build(tmp_path, name, old, new))
    for fn in ("ssd_oracle_forward", "ssd_oracle_forward_f64", "ssd_oracle_backward"):
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
        getattr(lib, fn).restype = getattr(real, fn).restype
    monkeypatch.setattr(so, "_lib", lib)
    caught = []
    for pin_name, pin in all_grad_pins():
        try:
            pin(so)
        except AssertionError:
            caught.append(pin_name)
    assert caught, f"no gradient pin caught the planted mistake {name!r}"
