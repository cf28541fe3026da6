"""The oracle's pins must catch plausible mistakes (CPU only).

Each case copies ``oracle/sdpa_oracle.c``, plants one mistake in the copy (a
dropped term, a wrong sign, an off-by-one, a wrong index or operand), builds it
into a temporary library and runs the pin suite against that library in a
fresh process.  The suite must fail for every mutant.  The committed oracle is
never modified.
"""

import os
import subprocess
import sys

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "sdpa_oracle.c")

MUTANTS = {
    "causal_off_by_one": ("if (pr->causal && j > p) return 0;", "if (pr->causal && j >= p) return 0;"),
    "window_off_by_one": ("p - j >= pr->window", "p - j > pr->window"),
    "gqa_modulo_mapping": ("const long hk = hq / group;", "const long hk = hq % pr->Hkv;"),
    "scale_dropped": ("s[j] = pr->scale * dot;", "s[j] = dot;"),
    "exp_sign_flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(m - s[j]);"),
    "no_normalisation": ("for (long d = 0; d < Dv; ++d) o[d] /= l;", "(void)l;"),
    "q_offset_ignored": ("const long p = (long)pr->q_offset + i;", "const long p = i;"),
    "k_and_v_swapped_in_scores": ("dot += qd[d] * key_elem(pr, kvrow0 + j, d);",
                                  "dot += qd[d] * value_elem(pr, kvrow0 + j, d);"),
    "v_batch_offset_dropped": ("return widen(pr->v[row * pr->Dv + d], pr->dtype);",
                               "return widen(pr->v[(row % ((long)pr->Hkv * pr->kL)) * pr->Dv + d], pr->dtype);"),
    "fp16_exponent_bias": ("expo - 25", "expo - 24"),
    "bf16_widened_as_fp16": ("return dtype == ORACLE_BF16 ? widen_bf16(h) : widen_fp16(h);",
                             "return widen_fp16(h);"),
    "max_over_first_key_only": ("if (!any || s[j] > m) m = s[j];", "if (!any) m = s[j];"),
    "last_visible_key_skipped": ("    if (!key_visible(pr, p, j) || s[j] == -INFINITY) continue;\n    for (long d = 0; d < Dv; ++d) o[d] +=",
                                 "    if (!key_visible(pr, p, j) || s[j] == -INFINITY || !key_visible(pr, p, j + 1)) continue;\n    for (long d = 0; d < Dv; ++d) o[d] +="),
    "bias_ignored": ("if (brow) s[j] += widen(brow[j], pr->dtype);", "(void)brow;"),
    "bias_subtracted": ("if (brow) s[j] += widen(brow[j], pr->dtype);", "if (brow) s[j] -= widen(brow[j], pr->dtype);"),
    "bias_head_stride_dropped": ("hq * pr->bias_sh", "0 * pr->bias_sh"),
    "bias_row_stride_dropped": ("i * pr->bias_sq", "0 * pr->bias_sq"),
    "v_head_stride_uses_d": ("return widen(pr->v[row * pr->Dv + d], pr->dtype);",
                             "return widen(pr->v[(row / pr->kL) * pr->kL * pr->D + (row % pr->kL) * pr->Dv + d], pr->dtype);"),
    "v_row_stride_uses_d": ("return widen(pr->v[row * pr->Dv + d], pr->dtype);",
                            "return widen(pr->v[row * pr->D + d], pr->dtype);"),
    "value_columns_cut_at_d": ("for (long d = 0; d < Dv; ++d) o[d] += s[j]", "for (long d = 0; d < D; ++d) o[d] += s[j]"),
    "minus_inf_bias_not_excluded": ("    if (s[j] == -INFINITY) continue;\n    if (!any", "    if (!any"),
    "q4_nibble_order_reversed": ("(word >> (4 * (d % 8)))", "(word >> (4 * (7 - d % 8)))"),
    "q4_groups_of_32": ("const long g = row * (D / 64) + d / 64;", "const long g = row * (D / 64) + (d / 32) % (D / 64);"),
    "q4_scale_and_bias_swapped": ("return widen(scales[g], dtype) * (double)c + widen(biases[g], dtype);",
                                  "return widen(biases[g], dtype) * (double)c + widen(scales[g], dtype);"),
    "q4_signed_codes": ("widen(scales[g], dtype) * (double)c", "widen(scales[g], dtype) * ((double)c - 8.0)"),
    "q4_v_takes_k_scales": ("dequant4(pr->vq, pr->vs, pr->vb,", "dequant4(pr->vq, pr->ks, pr->kb,"),
    "q4_word_ignores_the_row": ("codes[row * (D / 8) + d / 8]", "codes[d / 8]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(tmp_path, name):
    before, after = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(before) == 1, f"mutation site for {name} not found exactly once"
    mutant_src = tmp_path / "mutant.c"
    mutant_src.write_text(src.replace(before, after))
    lib = str(tmp_path / "libmutant.so")
    oracle.build(out_path=lib, src_path=str(mutant_src))
    env = dict(os.environ, SDPA_ORACLE_LIB=lib)
    r = subprocess.run(
        [sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
         os.path.join(ROOT, "tests", "test_oracle_pins.py")],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=300,
    )
    assert r.returncode != 0, f"pins passed with planted mistake {name}:\n{r.stdout[-2000:]}"
    assert "failed" in r.stdout, r.stdout[-2000:]
