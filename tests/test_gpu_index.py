"""Unified index build on the GPU: bit-exact against the oracle."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def run_case(c, dev="cuda"):
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).to(dev) for k, v in c.items() if k != "bs"}
    indptr, indices, plens = pkv.build_unified_kv_indices(
        t["prefix_kv_indptr"], t["prefix_kv_indices"], t["extend_start_loc"], t["extend_seq_lens"],
        t["extend_kv_indices"], c["bs"])
    torch.cuda.synchronize()
    want_indptr, want_indices, want_plens = oracle.build_unified_kv_indices(
        c["prefix_kv_indptr"], c["prefix_kv_indices"], c["extend_start_loc"], c["extend_seq_lens"],
        c["extend_kv_indices"], c["bs"])
    n = int(want_indptr[-1])
    assert indptr.cpu().numpy().tolist() == want_indptr.tolist()
    assert np.array_equal(indices.cpu().numpy()[:n], want_indices[:n])
    assert plens.cpu().numpy().tolist() == want_plens.tolist()
    return n


@pytest.mark.parametrize("bs,max_p,max_e,extra,base", [
    (0, 10, 10, 0, 0), (1, 0, 5, 0, 0), (1, 70000, 3, 0, 0), (3, 300, 300, 4, 7),
    (16, 2048, 512, 0, 0), (64, 5000, 64, 2, 0), (300, 40, 40, 0, 3), (1000, 9, 9, 5, 0),
])
def test_index_build_bit_exact(bs, max_p, max_e, extra, base):
    say(f"index build bs={bs} max_p={max_p} max_e={max_e}")
    rng = np.random.default_rng(bs * 7 + max_p)
    run_case(wl.index_case(rng, bs, max_p=max_p, max_e=max_e, extra_tail=extra, indptr_base=base))


@pytest.mark.parametrize("name", ["tiny_fp32", "llama8b", "long_prefix", "mla", "skewed_cap"])
def test_index_build_workloads(name):
    say(f"index build workload {name}")
    cfg = wl.CONFIGS[name]
    rng = np.random.default_rng(cfg.seed)
    p = cfg.prefix_lens(rng, cfg.bs).astype(np.int64)
    e = cfg.extend_lens(rng, cfg.bs).astype(np.int64)
    perm = rng.permutation(cfg.pool_slots).astype(np.int64)
    indptr = np.concatenate([[0], np.cumsum(p)]).astype(np.int32)
    c = dict(prefix_kv_indptr=indptr, prefix_kv_indices=perm[:p.sum()],
             extend_start_loc=np.concatenate([[0], np.cumsum(e)[:-1]]).astype(np.int32),
             extend_seq_lens=e.astype(np.int32), extend_kv_indices=perm[p.sum():p.sum() + e.sum()],
             bs=cfg.bs)
    assert run_case(c) == int(p.sum() + e.sum())


def test_index_build_leaves_tail_untouched():
    rng = np.random.default_rng(5)
    c = wl.index_case(rng, 4, max_p=20, max_e=20, extra_tail=3)
    t = {k: torch.from_numpy(np.ascontiguousarray(v)).cuda() for k, v in c.items() if k != "bs"}
    cap = t["prefix_kv_indices"].numel() + t["extend_kv_indices"].numel()
    out = (torch.empty(5, dtype=torch.int32, device="cuda"),
           torch.full((cap,), -77, dtype=torch.int64, device="cuda"),
           torch.empty(4, dtype=torch.int32, device="cuda"))
    indptr, indices, _ = pkv.build_unified_kv_indices(
        t["prefix_kv_indptr"], t["prefix_kv_indices"], t["extend_start_loc"], t["extend_seq_lens"],
        t["extend_kv_indices"], 4, out=out)
    n = int(indptr[-1])
    assert (indices[n:] == -77).all()
