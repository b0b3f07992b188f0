"""Plants plausible mistakes in copies of the C oracle (on the CPU) and checks that the
pins catch every one: evidence that passing the pins means something."""
import ctypes
import os
import subprocess

import pytest

import oracle
from oracle import ssd_oracle as so
from pins import ALL_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

# (name, text in the oracle, replacement)
MUTANTS = [
    ("readout-before-update",
     "row[s] = alpha * row[s] + bs * xp;     /* state <- e^{a_t} state + b_t x_t^T */\n"
     "                acc += row[s] * (double)Ct[s];         /* c_t^T state (after the update) */",
     "acc += row[s] * (double)Ct[s];\n                row[s] = alpha * row[s] + bs * xp;"),
    ("b-without-dt", "const double bs = dtv * (double)Bt[s];", "const double bs = (double)Bt[s];"),
    ("decay-sign", "exp(Ah * dtv)", "exp(-Ah * dtv)"),
    ("decay-without-dt", "exp(Ah * dtv)", "exp(Ah)"),
    ("group-modulo", "g = h / hpg;", "g = h % G;"),
    ("no-skip-term", "yt[p] = acc + Dh * xp;", "yt[p] = acc;"),
    ("C-used-as-B", "const float* Bt = J->Bm", "const float* Bt = J->Cm"),
    ("state-not-decayed", "row[s] = alpha * row[s] + bs * xp;", "row[s] = row[s] + bs * xp;"),
    ("h0-ignored", "if (J->h0) {", "if (0) {"),
    ("emit-after-token", "if (J->hemit && J->emit_every > 0 && t % J->emit_every == 0) {",
     "if (J->hemit && J->emit_every > 0 && (t + 1) % J->emit_every == 0) {"),
]


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, f"mutation {name!r} does not apply"
    mut = src.replace(old, new, 1)
    cpath = tmp_path / f"{name}.c"
    cpath.write_text(mut)
    lib = tmp_path / f"lib{name}.so"
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fPIC", "-shared", "-std=c99", "-o", str(lib),
                    str(cpath), "-lm", "-lpthread"], check=True)
    return str(lib)


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(tmp_path, monkeypatch, name, old, new):
    so._load()  # make sure the real library's bindings exist, then swap in the mutant
    lib = ctypes.CDLL(_build_mutant(tmp_path, name, old, new))
    f = lib.ssd_oracle_forward
    f.argtypes = so._lib.ssd_oracle_forward.argtypes
    f.restype = ctypes.c_int
    monkeypatch.setattr(so, "_lib", lib)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(so.forward)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, f"no pin caught the planted mistake {name!r}"
