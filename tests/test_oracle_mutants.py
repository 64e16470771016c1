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
    "sign of scale dropped": ("s[j] = jb->scale * dot;", "s[j] = fabs(jb->scale) * dot;"),
    "exp sign flipped": ("exp(s[j] - m)", "exp(m - s[j])"),
    "max not subtracted in weights": ("exp(s[j] - m)", "exp(s[j])"),
    "strict causal edge": ("jb->causal ? i + 1 : N", "jb->causal ? (i > 0 ? i : 1) : N"),
    "lse in base 2": ("m + log(l)", "m + log2(l)"),
    "lse without max": ("jb->lse[r] = m + log(l);", "jb->lse[r] = log(l);"),
    "no normalisation": ("o[c] /= l;", "o[c] /= 1.0;"),
    "values in reverse key order": ("vh + j * d", "vh + (nvis - 1 - j) * d"),
    "batch and head swapped": ("const int64_t head = (b * jb->H + h) * N * d;\n    const uint16_t *qi",
                               "const int64_t head = (h * jb->B + b) * N * d;\n    const uint16_t *qi"),
    "wrong query row": ("jb->q + head + i * d", "jb->q + head + (N - 1 - i) * d"),
    "half exponent bias": ("expo - 25", "expo - 24"),
    "subnormal scale": ("ldexp((double)frac, -24)", "ldexp((double)frac, -25)"),
    "transposed score (k.q index)": ("qd[c] * g_half[kj[c]]", "qd[c] * g_half[kj[(c + 1) % d]]"),
}


# Slips in the backward pass; each must fail a pin of test_oracle_bwd.py.
BWD_MUTANTS = {
    "bwd: dk scale dropped": ("        dk[c] *= a->scale;", "        dk[c] *= 1.0;"),
    "bwd: dq scale dropped": ("        dq[c] *= a->scale;", "        dq[c] *= 1.0;"),
    "bwd: D sign flipped in dq": ("const double dS = P * (dP - D);", "const double dS = P * (dP + D);"),
    "bwd: D sign flipped in dk": ("P * (dP - D[i])", "P * (dP + D[i])"),
    "bwd: dv weighted by dS": ("dv[c] += P * g_half[doi[c]];", "dv[c] += dS * g_half[doi[c]];"),
    "bwd: dk built from keys": ("dk[c] += dS * g_half[qi[c]];", "dk[c] += dS * g_half[kj[c]];"),
    "bwd: dP with keys": ("dP += g_half[doi[c]] * g_half[vj[c]];\n        const double dS",
                          "dP += g_half[doi[c]] * g_half[kj[c]];\n        const double dS"),
    "bwd: strict causal edge in dk/dv": ("a->causal ? j : 0", "a->causal ? j + 1 : 0"),
    "bwd: D from unnormalised output": ("(od[c] / l)", "od[c]"),
    "bwd: weights without lse": ("exp(a->scale * dot - lse[i])", "exp(a->scale * dot)"),
    "bwd: query gradient from values": ("dq[c] += dS * g_half[kj[c]];", "dq[c] += dS * g_half[vj[c]];"),
}


# Slips in the FP8 path; each must fail a pin of test_oracle_fp8.py.
FP8_MUTANTS = {
    "fp8: exponent bias 8": ("ldexp((double)(frac | 0x8), expo - 10)",
                             "ldexp((double)(frac | 0x8), expo - 11)"),
    "fp8: subnormal scale": ("ldexp((double)frac, -9)", "ldexp((double)frac, -10)"),
    "fp8: NaN rule dropped": ("if (expo == 0xf && frac == 0x7)", "if (0)"),
    "fp8: v descale dropped": ("o[c] += e * (jb->dv * g_e4m3[vj[c]]);", "o[c] += e * g_e4m3[vj[c]];"),
    "fp8: q descale squared": ("dot += (jb->dq * g_e4m3[qi[c]])", "dot += (jb->dq * jb->dq * g_e4m3[qi[c]])"),
}


def _fp8_pin_calls():
    from tests import test_oracle_fp8 as fp
    return [
        fp.test_e4m3_decode_matches_torch,
        lambda: fp.test_matches_fp16_oracle_on_exact_inputs(False, (0.25, 2.0, 0.5)),
        lambda: fp.test_matches_fp16_oracle_on_exact_inputs(True, (1.0, 1.0, 1.0)),
    ]


def _bwd_pin_calls():
    from tests import test_oracle_bwd as bp
    return [
        lambda: bp.test_matches_torch_autograd(False, 0.41),
        lambda: bp.test_matches_torch_autograd(True, 0.41),
        lambda: bp.test_matches_torch_autograd(True, -0.41),
        lambda: bp.test_key_gradients_sum_to_zero(True),
        lambda: bp.test_value_gradients_sum_to_output_gradients(True),
        lambda: bp.test_uniform_keys_give_zero_query_gradient(False),
        bp.test_single_key_closed_form,
        bp.test_last_causal_key_sees_only_last_query,
    ]


def _pin_calls():
    calls = [
        pins.test_half_decode_exhaustive_matches_numpy,
        lambda: pins.test_identity_values_expose_softmax_matrix(False, 0.37),
        lambda: pins.test_identity_values_expose_softmax_matrix(True, 0.37),
        lambda: pins.test_identity_values_expose_softmax_matrix(True, -0.37),
        lambda: pins.test_zero_scale_gives_mean_of_visible_values(True),
        lambda: pins.test_multihead_rows_match_library_reference(False),
        lambda: pins.test_multihead_rows_match_library_reference(True),
        pins.test_large_scores_do_not_overflow,
        lambda: pins.test_brute_force_tiny(7, 5, True, 0.5),
        lambda: pins.test_brute_force_tiny(7, 5, False, -0.5),
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


EXPORTS = ("oracle_fmha_rows", "oracle_fmha_bwd_rows", "oracle_half_to_double",
           "oracle_fmha_fp8_rows", "oracle_e4m3_to_double")


def _swap_in(so, monkeypatch):
    real = oracle._load()
    lib = ctypes.CDLL(so)
    for fn in EXPORTS:
        getattr(lib, fn).restype = getattr(real, fn).restype
        getattr(lib, fn).argtypes = getattr(real, fn).argtypes
    monkeypatch.setattr(oracle, "_lib", lib)


ALL_MUTANTS = {**MUTANTS, **BWD_MUTANTS, **FP8_MUTANTS}


def _calls_for(name):
    if name in MUTANTS:
        return _pin_calls()
    return _bwd_pin_calls() if name in BWD_MUTANTS else _fp8_pin_calls()


@pytest.mark.parametrize("name", sorted(ALL_MUTANTS))
def test_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = ALL_MUTANTS[name]
    so = _build_mutant(tmp_path, name, old, new)
    _swap_in(so, monkeypatch)
    failures = 0
    for call in _calls_for(name):
        try:
            call()
        except (AssertionError, RuntimeError, FloatingPointError):
            failures += 1
    assert failures > 0, "no pin caught mutant %r" % name


def test_unmutated_copy_passes_every_pin(tmp_path, monkeypatch):
    """Control: the same build of the untouched source fails no pin."""
    so = _build_mutant(tmp_path, "identity", "exp(s[j] - m)", "exp(s[j] - m)")
    _swap_in(so, monkeypatch)
    for call in _pin_calls() + _bwd_pin_calls() + _fp8_pin_calls():
        call()
