"""Mutation tests for the oracle's pins (CPU only).

Each case copies the oracle's C source, plants one plausible mistake in the
copy (a dropped term, a wrong sign, index or mask, a decoder slip), builds it
with gcc in a temporary folder and requires that at least one pin rejects it.
The real oracle is never modified.
"""

import os
import shutil

import pytest

import oracle
from oracle_pins import CHECKS

SRC = os.path.join(os.path.dirname(oracle.__file__), "fa_oracle.c")

MUTANTS = {
    "dropped_scale": ("s[j] = scale * acc;", "s[j] = acc;"),
    "transposed_k_index": ("acc += qrow[d] * Kh[j * D + d];", "acc += qrow[d] * Kh[d * N + j];"),
    "reversed_v_rows": ("orow[d] += pj * Vh[j * D + d];", "orow[d] += pj * Vh[(N - 1 - j) * D + d];"),
    "mask_wrong_direction": ("if (causal && j > i) {", "if (causal && j < i) {"),
    "mask_drops_diagonal": ("if (causal && j > i) {", "if (causal && j >= i) {"),
    "no_normalisation": ("p[j] /= denom;", "p[j] /= 1.0;"),
    "softmax_sign": ("p[j] = exp(s[j] - m);", "p[j] = exp(m - s[j]);"),
    "no_max_subtraction": ("p[j] = exp(s[j] - m);", "p[j] = exp(s[j]);"),
    "f16_exponent_bias": ("val = ldexp((double)(f | 0x400), e - 25);",
                          "val = ldexp((double)(f | 0x400), e - 24);"),
    "f16_drops_sign": ("  return sign ? -val : val;\n}\n\n/* bfloat16",
                       "  return val;\n}\n\n/* bfloat16"),
    "bf16_hidden_bit": ("val = ldexp((double)(f | 0x80), e - 134);", "val = ldexp((double)f, e - 134);"),
    "f32_fraction_width": ("val = ldexp((double)(f | 0x800000), e - 150);",
                           "val = ldexp((double)(f | 0x800000), e - 149);"),
    "head_offset_ignores_batch": ("const int64_t base = bh * N * D;\n    decode_span(q",
                                  "const int64_t base = (bh % H) * N * D;\n    decode_span(q"),
    "accumulator_not_reset": ("for (int64_t d = 0; d < D; ++d) orow[d] = 0.0;", ""),
    "lse_drops_max": ("if (plse) *plse = m + log(denom);", "if (plse) *plse = log(denom);"),
    "lse_base_two": ("if (plse) *plse = m + log(denom);", "if (plse) *plse = m + log2(denom);"),
    "lse_of_normalised_sum": ("if (plse) *plse = m + log(denom);", "if (plse) *plse = m + log(total);"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation anchor for {name} not unique in the source"
    src = tmp_path / "fa_oracle.c"
    src.write_text(text.replace(old, new))
    lib = oracle.build(src=str(src), out=str(tmp_path / "libmutant.so"))
    mutant = oracle.Oracle(lib)
    caught = None
    for check in CHECKS:
        try:
            check(mutant)
        except Exception as e:  # any failure counts: assertion, NaN, exception
            caught = f"{check.__name__}: {str(e)[:120]}"
            break
    assert caught, f"mutant {name} passed every pin"
    print(f"{name} caught by {caught}")
