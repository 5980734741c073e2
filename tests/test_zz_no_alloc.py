"""The no-allocation extend entry point against the workspace one.

extend_attention_fwd_noalloc keeps the plan and the split chunks' partial
states in the library's own scratch array (one per device); its output must
meet the parity bar against extend_attention_fwd's on the same inputs, on
two calls in a row, the second with a smaller batch (the array keeps the
first call's contents), and against the oracle.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import check, out_f64, run_gpu, say

pytestmark = pytest.mark.gpu


def _noalloc(w):
    dev = wl.to_torch(w)
    dev["o"].fill_(float("nan"))
    pkv.extend_attention_fwd_noalloc(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"],
                                     dev["qo_indptr"], dev["kv_indptr"], dev["kv_indices"], sm_scale=w.sm_scale,
                                     logit_cap=w.logit_cap)
    torch.cuda.synchronize()
    return out_f64(dev)


def test_noalloc_matches_workspace_entry_on_two_calls():
    big = wl.custom(dtype="bf16", prefix_lens=[20000, 300, 0, 77], extend_lens=[33, 200, 129, 1], hq=32, hkv=8,
                    lq=128, lv=128, seed=81)
    small = wl.custom(dtype="bf16", prefix_lens=[40, 5], extend_lens=[10, 3], hq=32, hkv=8, lq=128, lv=128,
                      seed=82)
    for what, w in (("first, long prefix (split chunks)", big), ("second, smaller", small)):
        say(f"noalloc {what}: bs={w.bs} T={w.total_q} P={w.num_prefix}")
        got = _noalloc(w)
        ref = out_f64(run_gpu(w))
        check(got, ref, "bf16", f"noalloc vs workspace entry, {what}")
        check(got, oracle.extend_attention_workload(w), "bf16", f"noalloc vs oracle, {what}")


def test_noalloc_other_shapes():
    cases = [
        dict(dtype="bf16", prefix_lens=[3000, 1], extend_lens=[4, 33], hq=16, hkv=1, lq=576, lv=512,
             v_aliases_k=True, std=0.5),
        dict(dtype="bf16", prefix_lens=[500, 0], extend_lens=[20, 90], hq=4, hkv=2, lq=256, lv=256, logit_cap=30.0),
        dict(dtype="fp32", prefix_lens=[16, 0], extend_lens=[8, 12], hq=4, hkv=2, lq=64, lv=64, sm_scale=1 / 8),
    ]
    for c in cases:
        w = wl.custom(**c)
        say(f"noalloc {w.cfg.dtype} {w.cfg.lq}/{w.cfg.lv}")
        got = _noalloc(w)
        check(got, out_f64(run_gpu(w)), w.cfg.dtype, "noalloc vs workspace entry")
        check(got, oracle.extend_attention_workload(w), w.cfg.dtype, "noalloc vs oracle")
