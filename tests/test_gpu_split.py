"""Split invariance on the GPU: one batch at several split granularities.

The planner cuts long key ranges into chunks whose partial softmax states a
merge launch combines (page "flashinfer_backend.py", forward_extend: the
ragged and paged parts merged with merge_state).  Any cut gives the same
softmax up to rounding, so every granularity must meet the oracle's bar and
agree with the others.  extend_attention_set_split forces the granularity;
the plan header at the start of the workspace shows how many items were
split.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import TOL, check, out_f64, say

pytestmark = pytest.mark.gpu

CASES = [
    dict(name="llama8b-shape", dtype="bf16", prefix_lens=[0, 300, 77, 1000, 5], extend_lens=[200, 1, 64, 33, 129],
         hq=32, hkv=8, lq=128, lv=128),
    dict(name="d64-long", dtype="bf16", prefix_lens=[9000, 40], extend_lens=[3, 70], hq=8, hkv=2, lq=64, lv=64),
    dict(name="d256-cap", dtype="bf16", prefix_lens=[5000, 0], extend_lens=[20, 90], hq=4, hkv=2, lq=256, lv=256,
         logit_cap=30.0),
    dict(name="mla", dtype="bf16", prefix_lens=[3000, 100], extend_lens=[4, 33], hq=16, hkv=1, lq=576, lv=512,
         v_aliases_k=True, std=0.5),
    dict(name="fp32-128", dtype="fp32", prefix_lens=[2500, 3], extend_lens=[5, 40], hq=4, hkv=2, lq=128, lv=128),
]


def _run(w, dev, rounds, min_chunk):
    desc = pkv.make_desc(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"], w.bs,
                         w.num_prefix)
    ws = torch.zeros(pkv.extend_attention_workspace_size(desc), dtype=torch.uint8, device=dev["q"].device)
    dev["o"].zero_()
    pkv.extend_attention_set_split(rounds, min_chunk)
    try:
        pkv.extend_attention_fwd(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"],
                                 dev["qo_indptr"], dev["kv_indptr"], dev["kv_indices"], sm_scale=w.sm_scale,
                                 logit_cap=w.logit_cap, workspace=ws)
    finally:
        pkv.extend_attention_set_split(0, 0)
    torch.cuda.synchronize()
    # plan header: num_work, num_merge, chunk_tiles, total_tiles, num_items, num_chunks
    hdr = ws[:24].view(torch.int32).cpu().numpy()
    return out_f64(dev), int(hdr[1]), int(hdr[5]), int(hdr[4])


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_split_granularities_agree(case):
    case = dict(case)
    name = case.pop("name")
    w = wl.custom(**case)
    dev = wl.to_torch(w)
    want = oracle.extend_attention_workload(w)
    outs = []
    for rounds, min_chunk in ((0, 0), (1, 1), (2, 1), (4, 1), (16, 1)):
        say(f"split {name}: rounds={rounds} min_chunk={min_chunk}")
        got, merges, chunks, items = _run(w, dev, rounds, min_chunk)
        say(f"  merges={merges} chunks={chunks} items={items}")
        check(got, want, w.cfg.dtype, f"{name}-r{rounds}")
        outs.append((rounds, merges, chunks, got))
    # the forced granularities really split, finer ones into more chunks
    assert outs[-1][1] > 0 and outs[-1][2] > outs[0][2]
    assert outs[-1][2] >= outs[2][2] >= outs[1][2]
    bar_max, bar_mean = TOL[w.cfg.dtype]
    for _, _, _, got in outs[1:]:
        d = np.abs(got - outs[0][3])
        assert d.max() <= bar_max and d.mean() <= bar_mean

