"""Planted mistakes for the pin-sensitivity test.

Each mutant is a copy of ``oracle/oracle.c`` with one plausible mistake
substituted into its text, compiled on its own into a temporary library.  The
oracle's source itself carries no switch for them: the pins must reject every
mutant, which shows that a mistake of that kind in the oracle would not go
unnoticed.  Only ``tests/test_oracle_pins.py`` uses this module.
"""
import os
import subprocess
import tempfile

import oracle

# name -> (text in oracle.c, replacement).  Each text must occur exactly once.
MUTANTS = {
    "nibble order swapped": (
        "int n = high ? (byte >> 4) & 15 : byte & 15;",
        "int n = high ? byte & 15 : (byte >> 4) & 15;"),
    "offset-binary decode": (
        "return n >= 8 ? n - 16 : n;",
        "return n - 8;"),
    "scale groups along rows": (
        "int g = c / GS;",
        "int g = (r / GS) % (cols / GS);"),
    "shared expert dropped": (
        "if (shared) {",
        "if (shared && 0) {"),
    "softmax over all experts": (
        "for (int j = 0; j < k; ++j) m = fmax(m, l[idx[j]]);\n"
        "  for (int j = 0; j < k; ++j) s += exp(l[idx[j]] - m);",
        "for (int e = 0; e < E; ++e) m = fmax(m, l[e]);\n"
        "  for (int e = 0; e < E; ++e) s += exp(l[e] - m);"),
    "ties to the higher index": (
        "return a < b;",
        "return a > b;"),
    "SiLU sign": (
        "return z / (1.0 + exp(-z));",
        "return z / (1.0 + exp(z));"),
    "router bias dropped": (
        "if (bias) acc += (double)bias[e];",
        "(void)bias;"),
    "top-p keeps the top-k weights of the kept experts": (
        "oracle_softmax_selected(l, E, idx, m, w);",
        "(void)l;"),
}

_built = {}


def build(name: str) -> str:
    """Path of the library built from oracle.c with mutant ``name`` applied."""
    if name in _built:
        return _built[name]
    src = open(oracle._SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, "mutant %r: its text occurs %d times in oracle.c" % (name, src.count(old))
    d = tempfile.mkdtemp(prefix="oracle_mutant_")
    c = os.path.join(d, "mutant.c")
    so = os.path.join(d, "libmutant.so")
    with open(c, "w") as fh:
        fh.write(src.replace(old, new))
    subprocess.check_call(["gcc", "-O2", "-fno-fast-math", "-ffp-contract=off", "-fopenmp", "-shared", "-fPIC",
                           "-o", so, c, "-lm"])
    _built[name] = so
    return so
