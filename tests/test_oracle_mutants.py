"""Mutation check of the oracle's pins (CPU only).

Each mutant is a copy of oracle/fmha_oracle.c with one plausible mistake
planted: a dropped term, a wrong sign, index or causal edge, or the wrong log
base. The copy is compiled with gcc into a temporary library and swapped in
for the real one. The pins of test_oracle.py are then run against it, and at
least one of them must fail. The real oracle source is never modified.
"""
import ctypes
import os
import subprocess

import pytest

import oracle
from tests import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "fmha_oracle.c")

MUTANTS = {
    "scale dropped": ("s[j] = jb->scale * dot;", "s[j] = dot;"),
    "exp sign flipped": ("exp(s[j] - m)", "exp(m - s[j])"),
    "max not subtracted in weights": ("exp(s[j] - m)", "exp(s[j])"),
    "strict causal edge": ("jb->causal ? i + 1 : N", "jb->causal ? (i > 0 ? i : 1) : N"),
    "lse in base 2": ("m + log(l)", "m + log2(l)"),
    "lse without max": ("jb->lse[r] = m + log(l);", "jb->lse[r] = log(l);"),
    "no normalisation": ("o[c] /= l;", "o[c] /= 1.0;"),
    "values in reverse key order": ("vh + j * d", "vh + (nvis - 1 - j) * d"),
    "batch and head swapped": ("(b * jb->H + h)", "(h * jb->B + b)"),
    "wrong query row": ("jb->q + head + i * d", "jb->q + head + (N - 1 - i) * d"),
    "half exponent bias": ("expo - 25", "expo - 24"),
    "subnormal scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "transposed score (k.q index)": ("qd[c] * g_half[kj[c]]", "qd[c] * g_half[kj[(c + 1) % d]]"),
}


def _pin_calls():
    calls = [
        pins.test_half_decode_exhaustive_matches_numpy,
        lambda: pins.test_identity_values_expose_softmax_matrix(False),
        lambda: pins.test_identity_values_expose_softmax_matrix(True),
        lambda: pins.test_multihead_rows_match_library_reference(False),
        lambda: pins.test_multihead_rows_match_library_reference(True),
        pins.test_large_scores_do_not_overflow,
        lambda: pins.test_brute_force_tiny(7, 5, True),
        lambda: pins.test_uniform_keys_give_mean_of_values(True),
        lambda: pins.test_one_hot_scores_select_one_value_row(64),
        pins.test_causal_first_row_is_first_value_row,
        pins.test_causal_row_sees_exactly_keys_up_to_itself,
        pins.test_key_shift_moves_lse_only,
        pins.test_lse_is_natural_log_of_scaled_scores,
    ]
    return calls


def _build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation site vanished: %s" % name
    mut = src.replace(old, new)
    cpath = tmp_path / "mut.c"
    cpath.write_text(mut)
    so = tmp_path / ("mut_%d.so" % abs(hash(name)))
    subprocess.run(["gcc", "-O1", "-std=c11", "-fPIC", "-shared", "-pthread",
                    str(cpath), "-o", str(so), "-lm"], check=True)
    return str(so)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = MUTANTS[name]
    so = _build_mutant(tmp_path, name, old, new)
    real = oracle._load()
    lib = ctypes.CDLL(so)
    for fn in ("oracle_fmha_rows", "oracle_half_to_double"):
        getattr(lib, fn).restype = getattr(real, fn).restype
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
    monkeypatch.setattr(oracle, "_lib", lib)
    failures = 0
    for call in _pin_calls():
        try:
            call()
        except (AssertionError, RuntimeError, FloatingPointError):
            failures += 1
    assert failures > 0, "no pin caught mutant %r" % name


def test_unmutated_copy_passes_every_pin(tmp_path, monkeypatch):
    """Control: the same build of the untouched source fails no pin."""
    so = _build_mutant(tmp_path, "identity", "exp(s[j] - m)", "exp(s[j] - m)")
    real = oracle._load()
    lib = ctypes.CDLL(so)
    for fn in ("oracle_fmha_rows", "oracle_half_to_double"):
        getattr(lib, fn).restype = getattr(real, fn).restype
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
    monkeypatch.setattr(oracle, "_lib", lib)
    for call in _pin_calls():
        call()
