"""Planted mistakes in a copy of the oracle must fail its pins.

Each case edits one line of oracle/oracle.c in a temporary copy of the
oracle, tests and input generators, then runs tests/test_oracle_pins.py
there; the pins must fail.  Nothing here touches a GPU.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTATIONS = {
    "mask_drops_diagonal": ("? P + E : P + i + 1;", "? P + E : P + i;"),
    "mask_sees_next_token": ("? P + E : P + i + 1;", "? P + E : P + i + 1 + (i + 1 < E);"),
    "kv_head_modulo": ("int32_t g = h / group;", "int32_t g = h % hkv;"),
    "default_scale_from_lv": ("1.0 / sqrt((double)lq)", "1.0 / sqrt((double)lv)"),
    "cap_without_division": ("x = logit_cap * tanh(x / logit_cap);", "x = tanh(x) * logit_cap;"),
    "extend_row_shift": ("koff = (qo_indptr[b] + (j - P)) * ke_st",
                         "koff = (qo_indptr[b] + (j - P) + (j > P)) * ke_st"),
    "index_copy_shift": ("unified_kv_indices[u + p_len + o]", "unified_kv_indices[u + p_len + o - (o > 0)]"),
    "first_weight_bias": ("double wgt = exp(s[j] - m);", "double wgt = exp(s[j] - m) * (j == 0 ? 1.0001 : 1.0);"),
    "unified_drops_diagonal": ("((j < P) || (j - P <= i)))", "((j < P) || (j - P < i)))"),
    "unified_causal_prefix": ("((j < P) || (j - P <= i)))", "((j - P <= i)))"),
    "window_one_key_short": ("? P + i - window : 0;", "? P + i - window + 1 : 0;"),
    "unified_window_open_end": ("j >= P + i - window);", "j > P + i - window);"),
    "mask_row_stride_e": ("custom_mask[mask_indptr[b] + i * (P + E) + j]", "custom_mask[mask_indptr[b] + i * E + j]"),
    "mask_ignored_past_diagonal": ("int64_t visible = custom_mask ? P + E : P + i + 1;",
                                   "int64_t visible = P + i + 1;"),
    "sink_without_max": ("if (sinks) den += exp((double)sinks[h] - m);", "if (sinks) den += exp((double)sinks[h]);"),
    "store_k_rows_by_token": ("memcpy((char*)k_pool + (slot * kp_ss", "memcpy((char*)k_pool + (t * kp_ss"),
    "gather_ignores_start": ("int64_t start = kv_start_idx ? kv_start_idx[b] : 0;", "int64_t start = 0;"),
    "gather_indptr_skips_first": ("kv_indptr[b + 1] = kv_indptr[b] + kv_lens[b];",
                                  "kv_indptr[b + 1] = kv_indptr[b] + kv_lens[b] + (b == 0);"),
    "decode_window_one_key_short": ("? n - 1 - window : 0;", "? n - window : 0;"),
    "decode_query_row_of_output": ("(int64_t)b * q_st + (int64_t)h * q_sh + d)",
                                   "(int64_t)r * q_st + (int64_t)h * q_sh + d)"),
    "decode_empty_request_nan": ("for (int32_t d = 0; d < lv; ++d) o[d] = 0.0;",
                                 "for (int32_t d = 0; d < lv; ++d) o[d] = NAN;"),
    "decode_kv_head_modulo": ("int32_t g = h / group;\n        int64_t n = kv_indptr",
                              "int32_t g = h % hkv;\n        int64_t n = kv_indptr"),
    "unified_batch_index_base": ("int64_t koff = kv_indices[kv_indptr[b] + j] * kp_ss",
                                 "int64_t koff = kv_indices[kv_indptr[0] + j] * kp_ss"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after = MUTATIONS[name]
    src = open(os.path.join(ROOT, "oracle", "oracle.c")).read()
    assert before in src
    ign = shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__")
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle", ignore=ign)
    os.makedirs(tmp_path / "tests")
    for f in ("conftest.py", "test_oracle_pins.py"):
        shutil.copy(os.path.join(ROOT, "tests", f), tmp_path / "tests" / f)
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    shutil.copy(os.path.join(ROOT, "workloads.py"), tmp_path / "workloads.py")
    (tmp_path / "oracle" / "oracle.c").write_text(src.replace(before, after, 1))
    r = subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                        "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode != 0, f"pins did not catch {name}:\n{r.stdout[-2000:]}"
