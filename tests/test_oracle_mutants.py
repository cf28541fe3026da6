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
    "k_and_v_swapped_in_scores": ("const uint16_t *krow = kbase + j * D;",
                                  "const uint16_t *krow = vbase + j * D;"),
    "v_batch_offset_dropped": ("const uint16_t *vbase = pr->v + (b * pr->Hkv + hk) * (long)pr->kL * Dv;",
                               "const uint16_t *vbase = pr->v + (hk) * (long)pr->kL * Dv;"),
    "fp16_exponent_bias": ("expo - 25", "expo - 24"),
    "bf16_widened_as_fp16": ("return dtype == ORACLE_BF16 ? widen_bf16(h) : widen_fp16(h);",
                             "return widen_fp16(h);"),
    "max_over_first_key_only": ("if (!any || s[j] > m) m = s[j];", "if (!any) m = s[j];"),
    "last_visible_key_skipped": ("    if (!key_visible(pr, p, j) || s[j] == -INFINITY) continue;\n    const uint16_t *vrow",
                                 "    if (!key_visible(pr, p, j) || s[j] == -INFINITY || !key_visible(pr, p, j + 1)) continue;\n    const uint16_t *vrow"),
    "bias_ignored": ("if (brow) s[j] += widen(brow[j], pr->dtype);", "(void)brow;"),
    "bias_subtracted": ("if (brow) s[j] += widen(brow[j], pr->dtype);", "if (brow) s[j] -= widen(brow[j], pr->dtype);"),
    "bias_head_stride_dropped": ("hq * pr->bias_sh", "0 * pr->bias_sh"),
    "bias_row_stride_dropped": ("i * pr->bias_sq", "0 * pr->bias_sq"),
    "v_head_stride_uses_d": ("(b * pr->Hkv + hk) * (long)pr->kL * Dv;", "(b * pr->Hkv + hk) * (long)pr->kL * D;"),
    "v_row_stride_uses_d": ("const uint16_t *vrow = vbase + j * Dv;", "const uint16_t *vrow = vbase + j * D;"),
    "value_columns_cut_at_d": ("for (long d = 0; d < Dv; ++d) o[d] += s[j]", "for (long d = 0; d < D; ++d) o[d] += s[j]"),
    "minus_inf_bias_not_excluded": ("    if (s[j] == -INFINITY) continue;\n    if (!any", "    if (!any"),
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
