"""Planted mistakes in a copy of the oracle must fail its pins.

Each case edits one line of oracle/oracle.c in a temporary copy of the
oracle, its pins and the input generators, then runs
tests/test_oracle_pins.py there.  The unmutated copy must pass (exit 0) and
every mutated copy must fail with test failures (exit 1): a copy that cannot
be collected or run (exit 2..5) would say nothing about the pins.  Nothing
here touches a GPU or the HIP library: the copy gets a conftest of its own
that only puts the copy on the import path.
"""

import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CAP = "if (logit_cap > 0.0) x = logit_cap * tanh(x / logit_cap);"
CAP_BEFORE_SCALE = "if (logit_cap > 0.0) x = logit_cap * tanh(x / scale / logit_cap) * scale;"
CAP_HARD_CLIP = "if (logit_cap > 0.0) x = fmax(-logit_cap, fmin(logit_cap, x));"

# name: (text before, text after, which occurrence of the text is edited)
MUTATIONS = {
    "mask_drops_diagonal": ("? P + E : P + i + 1;", "? P + E : P + i;", 0),
    "mask_sees_next_token": ("? P + E : P + i + 1;", "? P + E : P + i + 1 + (i + 1 < E);", 0),
    "kv_head_modulo": ("int32_t g = h / group;", "int32_t g = h % hkv;", 0),
    "default_scale_from_lv": ("1.0 / sqrt((double)lq)", "1.0 / sqrt((double)lv)", 0),
    "cap_without_division": (CAP, "if (logit_cap > 0.0) x = tanh(x) * logit_cap;", 0),
    # the cap applied to the raw dot product and the scale after it, and a
    # hard clip in place of tanh, in each of the three attention functions
    # (two-part extend, unified extend, decode)
    "cap_before_scale": (CAP, CAP_BEFORE_SCALE, 0),
    "unified_cap_before_scale": (CAP, CAP_BEFORE_SCALE, 1),
    "decode_cap_before_scale": (CAP, CAP_BEFORE_SCALE, 2),
    "cap_is_hard_clip": (CAP, CAP_HARD_CLIP, 0),
    "unified_cap_is_hard_clip": (CAP, CAP_HARD_CLIP, 1),
    "decode_cap_is_hard_clip": (CAP, CAP_HARD_CLIP, 2),
    "extend_row_shift": ("koff = (qo_indptr[b] + (j - P)) * ke_st",
                         "koff = (qo_indptr[b] + (j - P) + (j > P)) * ke_st", 0),
    "index_copy_shift": ("unified_kv_indices[u + p_len + o]", "unified_kv_indices[u + p_len + o - (o > 0)]", 0),
    "first_weight_bias": ("double wgt = exp(s[j] - m);", "double wgt = exp(s[j] - m) * (j == 0 ? 1.0001 : 1.0);", 0),
    "unified_drops_diagonal": ("((j < P) || (j - P <= i)))", "((j < P) || (j - P < i)))", 0),
    # (a mutation of the j < P term alone is equivalent: for j < P, j - P <= i
    # holds for every query, so the prefix length itself is shifted instead)
    "unified_prefix_len_plus_one": ("int64_t P = prefix_lens[b];", "int64_t P = prefix_lens[b] + 1;", 0),
    "window_one_key_short": ("? P + i - window : 0;", "? P + i - window + 1 : 0;", 0),
    "unified_window_open_end": ("j >= P + i - window);", "j > P + i - window);", 0),
    "mask_row_stride_e": ("custom_mask[mask_indptr[b] + i * (P + E) + j]",
                          "custom_mask[mask_indptr[b] + i * E + j]", 0),
    "mask_ignored_past_diagonal": ("int64_t visible = custom_mask ? P + E : P + i + 1;",
                                   "int64_t visible = P + i + 1;", 0),
    "sink_without_max": ("if (sinks) den += exp((double)sinks[h] - m);", "if (sinks) den += exp((double)sinks[h]);", 0),
    "store_k_rows_by_token": ("memcpy((char*)k_pool + (slot * kp_ss", "memcpy((char*)k_pool + (t * kp_ss", 0),
    "gather_ignores_start": ("int64_t start = kv_start_idx ? kv_start_idx[b] : 0;", "int64_t start = 0;", 0),
    "gather_indptr_skips_first": ("kv_indptr[b + 1] = kv_indptr[b] + kv_lens[b];",
                                  "kv_indptr[b + 1] = kv_indptr[b] + kv_lens[b] + (b == 0);", 0),
    "decode_window_one_key_short": ("? n - 1 - window : 0;", "? n - window : 0;", 0),
    "decode_query_row_of_output": ("(int64_t)b * q_st + (int64_t)h * q_sh + d)",
                                   "(int64_t)r * q_st + (int64_t)h * q_sh + d)", 0),
    "decode_empty_request_nan": ("for (int32_t d = 0; d < lv; ++d) o[d] = 0.0;",
                                 "for (int32_t d = 0; d < lv; ++d) o[d] = NAN;", 0),
    "decode_kv_head_modulo": ("int32_t g = h / group;\n        int64_t n = kv_indptr",
                              "int32_t g = h % hkv;\n        int64_t n = kv_indptr", 0),
    "unified_batch_index_base": ("int64_t koff = kv_indices[kv_indptr[b] + j] * kp_ss",
                                 "int64_t koff = kv_indices[kv_indptr[0] + j] * kp_ss", 0),
}

# The copy's conftest: the copy on the import path, nothing else (the tree's
# own conftest also registers markers and builds the HIP library).
_CONFTEST = """import os, sys
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
"""


def _replace_nth(src, before, after, n):
    at = -1
    for _ in range(n + 1):
        at = src.find(before, at + 1)
        assert at >= 0, f"occurrence {n} of {before!r} not found"
    return src[:at] + after + src[at + len(before):]


def _run_pins(tmp_path, oracle_src):
    ign = shutil.ignore_patterns("*.so", "*.so.tmp*", "__pycache__")
    shutil.copytree(os.path.join(ROOT, "oracle"), tmp_path / "oracle", ignore=ign)
    os.makedirs(tmp_path / "tests")
    (tmp_path / "tests" / "conftest.py").write_text(_CONFTEST)
    shutil.copy(os.path.join(ROOT, "tests", "test_oracle_pins.py"), tmp_path / "tests" / "test_oracle_pins.py")
    shutil.copytree(os.path.join(ROOT, "tests", "golden"), tmp_path / "tests" / "golden")
    shutil.copy(os.path.join(ROOT, "workloads.py"), tmp_path / "workloads.py")
    (tmp_path / "oracle" / "oracle.c").write_text(oracle_src)
    return subprocess.run([sys.executable, "-m", "pytest", "-q", "-x", "-p", "no:cacheprovider",
                           "tests/test_oracle_pins.py"], cwd=tmp_path, capture_output=True, text=True,
                          timeout=600)


def _oracle_src():
    with open(os.path.join(ROOT, "oracle", "oracle.c")) as f:
        return f.read()


def test_unmutated_copy_passes(tmp_path):
    r = _run_pins(tmp_path, _oracle_src())
    assert r.returncode == 0, f"the unmutated copy fails its pins:\n{r.stdout[-3000:]}\n{r.stderr[-2000:]}"


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_pins_catch_planted_mistake(name, tmp_path):
    before, after, n = MUTATIONS[name]
    mutated = _replace_nth(_oracle_src(), before, after, n)
    r = _run_pins(tmp_path, mutated)
    # exit 1: tests ran and some failed; anything else is a harness problem
    assert r.returncode == 1, f"pins did not catch {name} (exit {r.returncode}):\n{r.stdout[-2000:]}\n{r.stderr[-1000:]}"
