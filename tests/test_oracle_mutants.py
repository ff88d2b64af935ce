"""Plant plausible mistakes in a copy of the oracle's C source, build each
copy on the CPU, and check that the pins in test_oracle.py reject it.  This
shows the pins are strong enough: a dropped term, a wrong sign, a wrong
stride or index, or a wrong tie-break anywhere in the oracle fails at least
one of them."""
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

MUTANTS = {
    "residual_sign": ("r[i] = r[i] - c[i];", "r[i] = r[i] + c[i];"),
    "tie_to_highest": ("if (v[k] < v[best]) best = k;", "if (v[k] <= v[best]) best = k;"),
    "dropped_codeword_norm": ("double t = a[i] - b[i];\n        s += t * t;",
                              "s += a[i] * a[i] - 2.0 * a[i] * b[i];"),
    "level_stride": ("const double *C = cb + (int64_t)l * K * d;\n                    if (rn2)",
                     "const double *C = cb + (int64_t)l * d;\n                    if (rn2)"),
    "gap_sign": ("gap[row * L + l] = second - dist[id];", "gap[row * L + l] = dist[id] - second;"),
    "rn2_after_update": ("if (rn2) rn2[row * L + l] = sqnorm(r, d);",
                         "if (rn2) rn2[row * L + l] = sqnorm(x + row * d, d);"),
    "decode_transposed_ids": ("((int64_t)l * K + ids[row * L + l]) * d;\n            for (int32_t i = 0; i < d; ++i) o[i]",
                              "((int64_t)l * K + ids[l * n + row]) * d;\n            for (int32_t i = 0; i < d; ++i) o[i]"),
    "hist_transposed": ("hist[(int64_t)l * K + id] += 1;", "hist[(int64_t)id * L + l] += 1;"),
    "embed_text_from_level_table": ("const double *e = text + (int64_t)ids[t * L] * D;",
                                    "const double *e = vis + (int64_t)ids[t * L] * D;"),
    "embed_text_last_id": ("const double *e = text + (int64_t)ids[t * L] * D;",
                           "const double *e = text + (int64_t)ids[t * L + L - 1] * D;"),
    "embed_level_stride": ("const double *e = vis + ((int64_t)l * K + ids[t * L + l]) * D;",
                           "const double *e = vis + ((int64_t)l + ids[t * L + l]) * D;"),
    "embed_drops_first_level": ("            for (int32_t l = 0; l < L; ++l) {\n                const double *e = vis",
                                "            for (int32_t l = 1; l < L; ++l) {\n                const double *e = vis"),
    "msr_skips_level": ("for (int32_t i = 0; i < d; ++i) r[i] = r[i] - c[i];\n                    ms[row * L + l]",
                        "if (l) for (int32_t i = 0; i < d; ++i) r[i] = r[i] - c[i];\n                    ms[row * L + l]"),
}

PIN_FUNCS = [
    pins.test_hand_worked_example_encode,
    pins.test_hand_worked_example_decode_hist_msr,
    pins.test_duplicated_codewords_tie_to_lowest_index,
    pins.test_structured_rows_return_generating_ids,
    pins.test_greedy_equals_joint_search_on_separated_codebooks,
    pins.test_is_greedy_not_joint,
    pins.test_single_level_matches_scipy_vq,
    pins.test_decode_matches_torch_embedding_bag,
    pins.test_residual_equals_input_minus_reconstruction,
    pins.test_hist_matches_bincount,
    pins.test_msr_is_mean_squared_error_of_prefix_reconstruction,
    pins.test_teacher_forced_excess,
    pins.test_embed_hand_worked_example,
    pins.test_embed_visual_tokens_equal_decode,
    lambda: pins.test_embed_text_tokens_are_table_rows("f32"),
    lambda: pins.test_embed_text_tokens_are_table_rows("bf16"),
] + [(lambda c=c: pins.test_matches_exact_rational_greedy(c)) for c in pins._tiny_problems()]


def _build(tmp_path, name, old, new):
    src = oracle._SRC
    with open(src) as f:
        text = f.read()
    assert text.count(old) >= 1, f"mutation site for {name} not found"
    mutated = text.replace(old, new, 1)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
                    "-ffp-contract=off", "-o", str(so), str(c), "-lm"], check=True,
                   capture_output=True)
    return oracle.load_library(str(so))


def _caught(funcs):
    failures = 0
    for f in funcs:
        try:
            f()
        except (AssertionError, ValueError, IndexError):
            failures += 1
    return failures


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(name, tmp_path, monkeypatch, oracle_lib):
    old, new = MUTANTS[name]
    lib = _build(tmp_path, name, old, new)
    monkeypatch.setattr(oracle, "_lib", lib)
    assert _caught(PIN_FUNCS) > 0, f"no pin caught mutant {name}"


def test_unmutated_copy_passes_all_pins(tmp_path, monkeypatch, oracle_lib):
    lib = _build(tmp_path, "identity", "#include <math.h>", "#include <math.h>")
    monkeypatch.setattr(oracle, "_lib", lib)
    for f in PIN_FUNCS:
        f()
