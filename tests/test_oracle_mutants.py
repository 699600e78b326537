"""The oracle's pins catch plausible slips in the oracle itself.

Each mutant plants one mistake in a copy of oracle/gdn_oracle.c (a dropped
decay, beta or scale, a sign, a transposed state, a wrong GQA map, a reversed
conv tap order, an output read before the update, ...), builds it with the
oracle's own gcc flags and runs every pin of tests/test_oracle_pins.py on it.
At least one pin other than the stored-value regression (whose values come
from the oracle) must fail, and for a slip on the prefill side one that checks
a closed form, a hand-worked example, a library routine or an invariant rather
than the oracle against itself.  All of this runs on the CPU; the product
library is not involved.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle_pins as pins

# (name, text in gdn_oracle.c (its first occurrence is replaced), replacement)
MUTANTS = [
    # sequential recurrence
    ("decay dropped", "for (int64_t e = 0; e < dv * dk; e++) S[e] *= decay;",
     "for (int64_t e = 0; e < dv * dk; e++) S[e] *= 1.0;"),
    ("decay of -g", "double decay = exp(g[t * Hv + h]);", "double decay = exp(-g[t * Hv + h]);"),
    ("prediction from the undecayed state", "                p[j] = s;\n",
     "                p[j] = s / decay;\n"),
    ("delta sign", "double dj = b * (vt[j] - p[j]);", "double dj = b * (vt[j] + p[j]);"),
    ("beta dropped", "double dj = b * (vt[j] - p[j]);", "double dj = (vt[j] - p[j]);"),
    ("output read before the update", "for (int64_t i = 0; i < dk; i++) s += S[j * dk + i] * qt[i];",
     "for (int64_t i = 0; i < dk; i++) s += (S[j * dk + i] - b * (vt[j] - p[j]) * kt[i]) * qt[i];"),
    ("output reads k", "for (int64_t i = 0; i < dk; i++) s += S[j * dk + i] * qt[i];",
     "for (int64_t i = 0; i < dk; i++) s += S[j * dk + i] * kt[i];"),
    ("scale dropped", "o[(t * Hv + h) * dv + j] = d->scale * s;", "o[(t * Hv + h) * dv + j] = s;"),
    ("initial state read untransposed",
     "S[j * dk + i] = initial_state ? initial_state[((n * Hv + h) * dk + i) * dv + j] : 0.0;",
     "S[j * dk + i] = initial_state ? initial_state[((n * Hv + h) * dv + j) * dk + i] : 0.0;"),
    ("GQA map h mod h_k", "int64_t n = u / Hv, h = u % Hv, hk = h / G;",
     "int64_t n = u / Hv, h = u % Hv, hk = h % Hk;"),
    # prologue
    ("conv taps reversed", "y += conv_w[c * W + j] *", "y += conv_w[c * W + (W - 1 - j)] *"),
    ("SiLU of -y", "a = y / (1.0 + exp(-y));", "a = y / (1.0 + exp(y));"),
    ("L2 norm without the square root",
     "double rq = 1.0 / sqrt(sq + d->l2_eps), rk = 1.0 / sqrt(sk + d->l2_eps);",
     "double rq = 1.0 / (sq + d->l2_eps), rk = 1.0 / (sk + d->l2_eps);"),
    ("conv state saved newest first", "conv_state_in, len - (W - 1) + j, c);", "conv_state_in, len - 1 - j, c);"),
    # chunked form
    ("chunk A decay reversed", "a = BETA(r) * exp(gam[r] - gam[s]) * kk;", "a = BETA(r) * exp(gam[s] - gam[r]) * kk;"),
    ("chunk output without the inter-chunk decay", "d->scale * (exp(gam[r]) * inter + intra);",
     "d->scale * (inter + intra);"),
    ("chunk state carried without decay", "H[i * dv + j] = exp(gl) * H[i * dv + j] + s_;",
     "H[i * dv + j] = H[i * dv + j] + s_;"),
    ("chunk forward substitution sign", "x -= A[r * C + s] * T[s * C + c];", "x += A[r * C + s] * T[s * C + c];"),
    # decode
    ("decode decay dropped", "for (int64_t e = 0; e < dk * dv; e++) Hs[e] *= decay;",
     "for (int64_t e = 0; e < dk * dv; e++) Hs[e] *= 1.0;"),
    ("decode newest tap on the oldest weight", "y += conv_w[c * W + W - 1] * x[c];", "y += conv_w[c * W] * x[c];"),
    ("decode conv history not shifted", "hist[j] = hist[j + 1];", "hist[j] = hist[j];"),
]


# Pins that compare the oracle with itself (two of its forms, or two calls);
# every other pin checks a closed form, a hand-worked example, a library
# routine or an invariant.  A slip in the prefill side (recurrence, prologue,
# chunked form) must fail at least one of the latter; the decode side is
# pinned through its equality with the (so pinned) prefill.
SELF_CONSISTENCY = ("test_chunked_equals_recurrent", "test_chunked_strong_decay", "test_packed_equals_per_sequence",
                    "test_split_and_resume_equals_one_shot", "test_decode_steps_equal_prefill",
                    "test_decode_multi_equals_prefill_prefixes")


def _pin_calls():
    """(name, function, kwargs) for every pin but the stored-value regression,
    one entry per parametrisation."""
    calls = []
    for name in sorted(dir(pins)):
        f = getattr(pins, name)
        if not name.startswith("test_") or name == "test_golden_regression" or not callable(f):
            continue
        marks = [m for m in getattr(f, "pytestmark", []) if m.name == "parametrize"]
        if not marks:
            calls.append((name, f, {}))
            continue
        argname, values = marks[0].args[0], marks[0].args[1]
        for val in values:
            calls.append((f"{name}[{val}]", f, {argname: val}))
    return calls


def _build(src: str, path: str) -> None:
    subprocess.run(["gcc", "-O2", "-ffp-contract=off", "-fno-fast-math", "-fopenmp", "-shared", "-fPIC",
                    "-o", path, "-x", "c", "-", "-lm"], input=src.encode(), check=True)


def test_every_mutant_site_exists():
    with open(os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")) as f:
        src = f.read()
    for name, old, _ in MUTANTS:
        assert old in src, name


def test_unmutated_oracle_passes_every_pin(tmp_path):
    """Control: the pins pass on a copy built the same way, unmutated."""
    with open(os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")) as f:
        src = f.read()
    lib_path = str(tmp_path / "liboracle_copy.so")
    _build(src, lib_path)
    saved = oracle._lib
    oracle._lib = ctypes.CDLL(lib_path)
    try:
        for _, f, kw in _pin_calls():
            f(oracle, **kw)
    finally:
        oracle._lib = saved


@pytest.mark.parametrize("mutant", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_catch_mutant(mutant, tmp_path):
    name, old, new = mutant
    with open(os.path.join(os.path.dirname(oracle.__file__), "gdn_oracle.c")) as f:
        src = f.read()
    assert old in src
    lib_path = str(tmp_path / "liboracle_mutant.so")
    _build(src.replace(old, new, 1), lib_path)
    saved = oracle._lib
    oracle._lib = ctypes.CDLL(lib_path)
    caught = []
    try:
        for pin, f, kw in _pin_calls():
            try:
                f(oracle, **kw)
            except Exception:
                caught.append(pin)
    finally:
        oracle._lib = saved
    print(f"  {name}: caught by {caught}", flush=True)
    assert caught, f"no pin catches the mutant '{name}'"
    if not name.startswith("decode"):
        external = [c for c in caught if not c.startswith(SELF_CONSISTENCY)]
        assert external, f"only self-consistency pins catch the mutant '{name}'"
