"""Sliding window and attention sinks on the GPU against the CPU oracle
(page "extend_attention.py", _fwd_kernel_unified: SLIDING_WINDOW_SIZE and
HAS_SINK), on both entry points, every kernel family and the split path."""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import check, out_f64, say

pytestmark = pytest.mark.gpu


def sinks_for(hq, seed=0):
    return np.random.default_rng(seed).uniform(-2.0, 3.0, size=hq).astype(np.float32)


def run(w, window, sinks, what):
    say(f"window/sinks {what}: bs={w.bs} T={w.total_q} P={w.num_prefix} dims={w.cfg.lq}/{w.cfg.lv} "
        f"window={window} sinks={'yes' if sinks is not None else 'no'}")
    dev = wl.to_torch(w)
    sk = torch.from_numpy(sinks).cuda() if sinks is not None else None
    pkv.extend_attention_fwd(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"],
                             dev["qo_indptr"], dev["kv_indptr"], dev["kv_indices"], sm_scale=w.sm_scale,
                             logit_cap=w.logit_cap, sliding_window=window, sinks=sk)
    torch.cuda.synchronize()
    check(out_f64(dev), oracle.extend_attention_workload(w, window=window, sinks=sinks), w.cfg.dtype, what)


REDUCED = {
    "tiny_fp32": dict(),
    "llama8b": dict(prefix_lens=[0, 300, 77, 1000, 5], extend_lens=[200, 1, 64, 33, 129]),
    "mla": dict(prefix_lens=[600, 1], extend_lens=[3, 20]),
    "skewed_cap": dict(prefix_lens=[0, 900, 13, 2], extend_lens=[300, 5, 64, 1]),
}
CASES = [(n, wdw, s) for n in REDUCED for wdw in (0, 5, 70, 400) for s in (False, True) if wdw or s]


@pytest.mark.parametrize("name,window,use_sinks", CASES, ids=[f"{n}-w{wd}-{'s' if s else 'n'}" for n, wd, s in CASES])
def test_window_sinks_reduced(name, window, use_sinks):
    w = wl.build(wl.CONFIGS[name], **{k: np.array(v) for k, v in REDUCED[name].items()})
    run(w, window, sinks_for(w.cfg.hq) if use_sinks else None, f"{name}-w{window}")


def test_window_sinks_split_chunks():
    # one long sequence: its items are split over KV ranges and merged, with
    # the sink added once in the merge
    w = wl.custom(dtype="bf16", prefix_lens=[20000], extend_lens=[300], hq=8, hkv=2, lq=128, lv=128)
    run(w, 3000, sinks_for(8, 1), "bs1-P20000-w3000")
    run(w, 0, sinks_for(8, 2), "bs1-P20000-sinks")


def test_unified_window_sinks():
    w = wl.build(wl.CONFIGS["llama8b"], prefix_lens=np.array([0, 300, 77]), extend_lens=np.array([200, 1, 64]))
    sinks = sinks_for(w.cfg.hq, 3)
    indptr, indices, plens = oracle.build_unified_kv_indices(
        w.kv_indptr, w.kv_indices, w.extend_start_loc, w.extend_lens, w.extend_kv_indices, w.bs)
    indices = indices[:int(indptr[-1])]
    dev = wl.to_torch(w)
    pkv.extend_attention_fwd_unified(dev["q"], dev["o"], dev["k_pool"], dev["v_pool"], dev["qo_indptr"],
                                     torch.from_numpy(indptr.astype(np.int32)).cuda(),
                                     torch.from_numpy(indices.astype(np.int64)).cuda(),
                                     torch.from_numpy(plens.astype(np.int32)).cuda(), sm_scale=w.sm_scale,
                                     sliding_window=100, sinks=torch.from_numpy(sinks).cuda())
    torch.cuda.synchronize()
    want = oracle.extend_attention_unified(w.q, w.k_pool, w.v_pool, w.qo_indptr, indptr, indices, plens,
                                           w.sm_scale, 0.0, "bf16", window=100, sinks=sinks)
    check(out_f64(dev), want, "bf16", "unified-w100-sinks")
