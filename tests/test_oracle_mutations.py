"""Planted mistakes: each mutant of the C oracle must fail the pin suite.

Each case copies ``oracle/mla_oracle.c``, applies one plausible mistake, builds
it with gcc into a temporary library and runs ``test_oracle_pins.py`` against
it in a subprocess (``MLA_ORACLE_LIB``). The mutant must make at least one pin
fail; the unmodified source must pass.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "oracle", "mla_oracle.c")

MUTANTS = {
    "drop_rope_dims": ("for (d = 0; d < OR_DQK; ++d) acc +=", "for (d = 0; d < OR_DV; ++d) acc +="),
    "wrong_v_slice": ("out[d] += w * x[j * OR_DQK + d];", "out[d] += w * x[j * OR_DQK + d + 64];"),
    "nibble_order": ("(d & 1) ? (uint8_t)(byte >> 4) : (uint8_t)(byte & 0xF)",
                     "(d & 1) ? (uint8_t)(byte & 0xF) : (uint8_t)(byte >> 4)"),
    "mx_scale_column": ("row_scales[d / OR_MX_BLOCK]", "row_scales[(d / OR_MX_BLOCK) ^ 1]"),
    "lse_log2": ("*lse = M + log(Z);", "*lse = M + log2(Z);"),
    "e4m3_bias": ("ldexp(1.0 + (double)m / 8.0, e - 7)", "ldexp(1.0 + (double)m / 8.0, e - 8)"),
    "e2m1_exponent": ("(1.0 + 0.5 * m) * ldexp(1.0, e - 1)", "(1.0 + 0.5 * m) * ldexp(1.0, e)"),
    "fixed_sm_scale": ("return sm_scale * acc;", "return acc / 24.0;"),
    "gather_ignores_start": ("kv_indices[start + j]", "kv_indices[j]"),
    "combine_weight_sign": ("w = exp(plse[s] - M);", "w = exp(M - plse[s]);"),
    "fp8_scale_dropped": ("x[d] = c * s; /*", "x[d] = c; (void)s; /*"),
    "q8_scale_dropped": ("oracle_e4m3fn_value(p[d]) * q_scale;", "oracle_e4m3fn_value(p[d]); (void)q_scale;"),
    "encode_ties_odd": ("(c & 1) == 0 && (best & 1) == 1", "(c & 1) == 1 && (best & 1) == 0"),
    "encode_drops_sign": ("signbit(x) ? (best | 0x80) : best", "best"),
    "quant_scale_inverted": ("s = amax / 448.0f;", "s = 448.0f / amax;"),
    "quant_multiplies": ("oracle_bf16_value(q[i]) / s;", "oracle_bf16_value(q[i]) * s;"),
    "mtp_causal_off_by_one": ("L = L - n + 1 + t;", "L = L - n + t;"),
    "mtp_token_order": ("t = r - qo_indptr[b];", "t = n - 1 - (r - qo_indptr[b]);"),
    "paged_last_page_full": ("rows_in_page = last_page_len[b];", "rows_in_page = page_size; (void)last_page_len;"),
    "paged_row_of_page": ("int64_t row = (int64_t)page_ids[k] * page_size + i;",
                          "int64_t row = (int64_t)page_ids[k] + i;"),
    "paged_page_order": ("int64_t row = (int64_t)page_ids[k] * page_size + i;",
                         "int64_t row = (int64_t)page_ids[first + end - 1 - k] * page_size + i;"),
    "paged_rows_reversed": ("int64_t row = (int64_t)page_ids[k] * page_size + i;",
                            "int64_t row = (int64_t)page_ids[k] * page_size + (rows_in_page - 1 - i);"),
    "mtp_query_row": ("decode_query(0, q, 1.0f, (int64_t)r * OR_HEADS + h, qh);",
                      "decode_query(0, q, 1.0f, (int64_t)b * OR_HEADS + h, qh);"),
}


def _build(src_text, tmp_path, name):
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"lib{name}.so"
    c.write_text(src_text)
    subprocess.check_call(["gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp", "-o", str(so), str(c), "-lm"])
    return so


def _run_pins(so):
    env = dict(os.environ, MLA_ORACLE_LIB=str(so))
    r = subprocess.run([sys.executable, "-m", "pytest", "-x", "-q", "-p", "no:cacheprovider",
                        os.path.join(ROOT, "tests", "test_oracle_pins.py")],
                       cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    return r.returncode


def test_unmodified_oracle_passes(tmp_path):
    assert _run_pins(_build(open(SRC).read(), tmp_path, "orig")) == 0


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation site for {name} not found exactly once"
    assert _run_pins(_build(src.replace(old, new), tmp_path, name)) != 0
