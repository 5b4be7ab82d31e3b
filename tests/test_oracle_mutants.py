"""The oracle's pins must reject plausible slips.

Each case copies oracle.c, plants one mistake in the copy (on the CPU, in a
temporary directory), builds it, and runs the pin tests of test_oracle.py
against the mutant; at least one pin has to fail.  The real oracle is never
modified.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import pytest

import oracle as oracle_pkg
from tests import test_oracle as pins

MUTANTS = {
    "gqa_head_map_modulo": ("const int g = hq / (J->Hq / J->Hkv);", "const int g = hq % J->Hkv;"),
    "causal_offset_top_left": ("int64_t lim = (int64_t)i + J->Sk - J->Sq + 1;",
                               "int64_t lim = (int64_t)i + 1;"),
    "causal_off_by_one": ("int64_t lim = (int64_t)i + J->Sk - J->Sq + 1;",
                          "int64_t lim = (int64_t)i + J->Sk - J->Sq;"),
    "scale_dropped": ("double s = J->scale * dot;", "double s = dot;"),
    "lse_base_two": ("*lse_out = m + log(l);", "*lse_out = m + log2(l);"),
    "lse_without_max": ("*lse_out = m + log(l);", "*lse_out = log(l);"),
    "v_indexed_by_query_head": (
        "const uint16_t *vrow = J->v + (((int64_t)b * J->Sk + j) * J->Hkv + g) * D;",
        "const uint16_t *vrow = J->v + (((int64_t)b * J->Sk + j) * J->Hkv + (hq % J->Hkv)) * D;"),
    "key_row_uses_query_index": (
        "const uint16_t *krow = J->k + (((int64_t)b * J->Sk + j) * J->Hkv + g) * D;",
        "const uint16_t *krow = J->k + (((int64_t)b * J->Sk + (j + i) % J->Sk) * J->Hkv + g) * D;"),
    "no_normalisation": ("        o_row[d] /= l;\n", "        o_row[d] /= 1.0;\n"),
    "empty_row_lse_zero": ("        *lse_out = -INFINITY;\n        return 0;", "        *lse_out = 0.0;\n        return 0;"),
}

PIN_TESTS = [
    lambda m: pins.test_oracle_matches_decimal_bruteforce(m, pins.BRUTE_CASES[2]),
    lambda m: pins.test_oracle_matches_decimal_bruteforce(m, pins.BRUTE_CASES[3]),
    lambda m: pins.test_two_keys_closed_form(m),
    lambda m: pins.test_uniform_scores_lse_is_log_count_and_o_is_prefix_mean(m, 3, 5),
    lambda m: pins.test_uniform_scores_lse_is_log_count_and_o_is_prefix_mean(m, 5, 3),
    lambda m: pins.test_causal_first_row_is_v0(m),
    lambda m: pins.test_gqa_equals_mha_with_repeated_kv_heads(m),
    lambda m: pins.test_layout_of_v_o_and_lse(m),
    lambda m: pins.test_layout_of_q_and_k(m),
    lambda m: pins.test_single_key_gives_that_value_row(m),
]


class _Mutant:
    """Quacks like the oracle package but calls the mutant library."""

    def __init__(self, lib):
        self._lib = lib

    def attn_fwd(self, *a, **kw):
        return oracle_pkg.attn_fwd(*a, _lib_override=self._lib, **kw)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, name):
    before, after = MUTANTS[name]
    src = open(os.path.join(os.path.dirname(oracle_pkg.__file__), "oracle.c")).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not found exactly once"
    path_c = tmp_path / "mutant.c"
    path_c.write_text(src.replace(before, after))
    path_so = tmp_path / "libmutant.so"
    subprocess.check_call(["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-pthread",
                           "-o", str(path_so), str(path_c), "-lm"])
    mutant = _Mutant(oracle_pkg._bind(ctypes.CDLL(str(path_so))))
    caught = 0
    for pin in PIN_TESTS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError):
            caught += 1
    assert caught > 0, f"no pin detects mutant {name}"


# slips in the paged gather (oracle/__init__.py), caught by the paged pins
PY_MUTANTS = {
    "page_and_slot_swapped": ("return cache[table_row[j // page_size], j % page_size]",
                              "return cache[table_row[j % page_size], j // page_size]"),
    "slots_reversed_in_page": ("return cache[table_row[j // page_size], j % page_size]",
                               "return cache[table_row[j // page_size], page_size - 1 - j % page_size]"),
    "next_sequence_table_row": ("kc = gather_pages(kb, table[b], n)[None]\n        vc = gather_pages(vb, table[b], n)[None]",
                                "kc = gather_pages(kb, table[(b + 1) % B], n)[None]\n        vc = gather_pages(vb, table[(b + 1) % B], n)[None]"),
    "length_off_by_one": ("n = int(lens[b])\n", "n = max(int(lens[b]) - 1, 1)\n"),
    "v_gathered_from_k": ("vc = gather_pages(vb, table[b], n)[None]", "vc = gather_pages(kb, table[b], n)[None]"),
}

PAGED_PIN_TESTS = [
    pins.test_paged_uniform_scores_average_the_sequences_own_rows,
    pins.test_paged_dominant_key_picks_its_slot,
    pins.test_paged_causal_offset_is_per_sequence,
    pins.test_paged_empty_sequence,
]


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_paged_pins_reject_mutant(name):
    import types
    before, after = PY_MUTANTS[name]
    src = open(oracle_pkg.__file__).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not found exactly once"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = oracle_pkg.__file__
    exec(compile(src.replace(before, after), "oracle_mutant", "exec"), mod.__dict__)
    caught = 0
    for pin in PAGED_PIN_TESTS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught > 0, f"no pin detects mutant {name}"


# slips in the FP8 decode and descale convention (oracle/__init__.py)
FP8_MUTANTS = {
    "exponent_bias_8": ("return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)",
                        "return sign * (1.0 + m / 8.0) * 2.0 ** (e - 8)"),
    "subnormal_as_normal": ("return sign * (m / 8.0) * 2.0 ** -6",
                            "return sign * (1.0 + m / 8.0) * 2.0 ** -7"),
    "no_nan_code": ("if e == 0xF and m == 0x7:\n        return float(\"nan\")",
                    "if False:\n        return float(\"nan\")"),
    "v_descale_dropped": ("return o * float(v_descale), lse", "return o, lse"),
    "k_descale_dropped": ("float(scale) * float(q_descale) * float(k_descale)",
                          "float(scale) * float(q_descale)"),
}

FP8_PIN_TESTS = [
    pins.test_fp8_decode_matches_the_format_and_torch,
    pins.test_fp8_uniform_scores_average_descaled_v,
    pins.test_fp8_descales_enter_scores_and_output,
]


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_pins_reject_mutant(name):
    import types
    before, after = FP8_MUTANTS[name]
    src = open(oracle_pkg.__file__).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not found exactly once"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = oracle_pkg.__file__
    exec(compile(src.replace(before, after), "oracle_mutant", "exec"), mod.__dict__)
    caught = 0
    for pin in FP8_PIN_TESTS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught > 0, f"no pin detects mutant {name}"


# slips in the backward oracle (oracle/__init__.py)
BWD_MUTANTS = {
    "softmax_jacobian_without_rowsum": ("ds = p * (dp - (dp * p).sum(axis=1, keepdims=True))",
                                        "ds = p * dp"),
    "dv_from_unnormalised_p": ("dV[b, :, g, :] += p.T @ dO[b, :, h, :]",
                               "dV[b, :, g, :] += e.T @ dO[b, :, h, :]"),
    "dq_scale_dropped": ("dQ[b, :, h, :] = scale * (ds @ K[b, :, g, :])",
                         "dQ[b, :, h, :] = ds @ K[b, :, g, :]"),
    "dk_overwritten_not_summed": ("dK[b, :, g, :] += scale * (ds.T @ Q[b, :, h, :])",
                                  "dK[b, :, g, :] = scale * (ds.T @ Q[b, :, h, :])"),
    "causal_offset_top_left": ("allowed = (j <= i + (Sk - Sq)) if causal",
                               "allowed = (j <= i) if causal"),
}

BWD_PIN_TESTS = [
    lambda m: pins.test_bwd_matches_torch_autograd(m, (1, 2, 2, 5, 7, 8, False)),
    lambda m: pins.test_bwd_matches_torch_autograd(m, (2, 4, 2, 6, 6, 4, True)),
    lambda m: pins.test_bwd_matches_torch_autograd(m, (1, 3, 1, 7, 4, 8, True)),
    pins.test_bwd_matches_finite_differences,
    pins.test_bwd_single_key_closed_form,
    pins.test_bwd_uniform_scores_dv_is_column_mean,
]


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_pins_reject_mutant(name):
    import types
    before, after = BWD_MUTANTS[name]
    src = open(oracle_pkg.__file__).read()
    assert src.count(before) == 1, f"mutation anchor for {name} not found exactly once"
    mod = types.ModuleType("oracle_mutant")
    mod.__file__ = oracle_pkg.__file__
    exec(compile(src.replace(before, after), "oracle_mutant", "exec"), mod.__dict__)
    caught = 0
    for pin in BWD_PIN_TESTS:
        try:
            pin(mod)
        except (AssertionError, IndexError, ValueError):
            caught += 1
    assert caught > 0, f"no pin detects mutant {name}"
