"""Unified one-stage extend attention on the GPU against the CPU oracle.

Every key of a sequence goes through one index array (page
"extend_attention.py", extend_attention_fwd_unified / _fwd_kernel_unified).
The unified arrays are built by the oracle's own index build on the CPU, so
no input comes from the HIP path; the workloads store every new token's K/V
in the pool at its extend slot, as the caller's cache store does.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import check, out_f64, run_gpu, say

pytestmark = pytest.mark.gpu


def unified_arrays(w, dev, prefix_lens=None):
    indptr, indices, plens = oracle.build_unified_kv_indices(
        w.kv_indptr, w.kv_indices, w.extend_start_loc, w.extend_lens, w.extend_kv_indices, w.bs)
    indices = indices[:int(indptr[-1])]
    if prefix_lens is not None:
        plens = np.asarray(prefix_lens, np.int32)
    dev["u_indptr"] = torch.from_numpy(indptr.astype(np.int32)).cuda()
    dev["u_indices"] = torch.from_numpy(indices.astype(np.int64)).cuda()
    dev["u_plens"] = torch.from_numpy(plens.astype(np.int32)).cuda()
    return indptr, indices, plens


def run_unified(w, dev):
    pkv.extend_attention_fwd_unified(dev["q"], dev["o"], dev["k_pool"], dev["v_pool"], dev["qo_indptr"],
                                     dev["u_indptr"], dev["u_indices"], dev["u_plens"],
                                     sm_scale=w.sm_scale, logit_cap=w.logit_cap)
    torch.cuda.synchronize()
    return dev


def oracle_unified(w, indptr, indices, plens, rows=None):
    return oracle.extend_attention_unified(w.q, w.k_pool, w.v_pool, w.qo_indptr, indptr, indices, plens,
                                           w.sm_scale, w.logit_cap, w.cfg.dtype, rows=rows)


def parity(w, what, prefix_lens=None):
    say(f"unified {what}: bs={w.bs} T={w.total_q} P={w.num_prefix} dims={w.cfg.lq}/{w.cfg.lv} "
        f"heads={w.cfg.hq}/{w.cfg.hkv} cap={w.logit_cap}")
    dev = wl.to_torch(w)
    arrays = unified_arrays(w, dev, prefix_lens)
    run_unified(w, dev)
    check(out_f64(dev), oracle_unified(w, *arrays), w.cfg.dtype, what)
    return dev


SMALL = {
    "tiny_fp32": dict(),
    "llama8b": dict(prefix_lens=[0, 300, 77, 1000, 5], extend_lens=[200, 1, 64, 33, 129]),
    "long_prefix": dict(prefix_lens=[3000, 1500], extend_lens=[70, 19]),
    "mla": dict(prefix_lens=[600, 1], extend_lens=[3, 20]),
    "skewed_cap": dict(prefix_lens=[0, 900, 13, 2], extend_lens=[300, 5, 64, 1]),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_unified_parity_reduced(name):
    w = wl.build(wl.CONFIGS[name], **{k: np.array(v) for k, v in SMALL[name].items()})
    parity(w, f"{name}-reduced")


EDGE = [
    dict(name="192x128", dtype="bf16", prefix_lens=[100, 33], extend_lens=[50, 7], hq=6, hkv=2, lq=192, lv=128),
    dict(name="288x256", dtype="bf16", prefix_lens=[65, 0], extend_lens=[30, 41], hq=4, hkv=1, lq=288, lv=256),
    dict(name="empty-seq", dtype="bf16", prefix_lens=[10, 40, 0, 7], extend_lens=[5, 0, 0, 9], hq=4, hkv=1,
         lq=64, lv=64),
    dict(name="fp32-128", dtype="fp32", prefix_lens=[40, 0, 100], extend_lens=[9, 50, 1], hq=4, hkv=2, lq=128,
         lv=128, sm_scale=0.05),
    dict(name="e1-decode", dtype="bf16", prefix_lens=[500, 0, 31], extend_lens=[1, 1, 1], hq=8, hkv=2, lq=128,
         lv=128),
    dict(name="d80", dtype="bf16", prefix_lens=[300, 0, 41], extend_lens=[70, 129, 3], hq=8, hkv=2, lq=80, lv=80),
    dict(name="d96", dtype="bf16", prefix_lens=[260, 7], extend_lens=[90, 200], hq=12, hkv=4, lq=96, lv=96),
    dict(name="d112", dtype="bf16", prefix_lens=[129, 400], extend_lens=[17, 60], hq=6, hkv=2, lq=112, lv=112),
    dict(name="d160-cap", dtype="bf16", prefix_lens=[200, 3], extend_lens=[45, 100], hq=8, hkv=4, lq=160, lv=160,
         logit_cap=10.0),
]


@pytest.mark.parametrize("case", EDGE, ids=[c["name"] for c in EDGE])
def test_unified_parity_edge(case):
    kw = {k: v for k, v in case.items() if k != "name"}
    parity(wl.custom(**kw), case["name"])


@pytest.mark.parametrize("name", ["llama8b", "mla"])
def test_unified_equals_two_part_bitwise(name):
    # with the new tokens' rows in the pool, both entries compute the same keys
    # in the same tiles and order: the results agree bit for bit
    w = wl.build(wl.CONFIGS[name], **{k: np.array(v) for k, v in SMALL[name].items()})
    two = run_gpu(w)["o"].clone()
    dev = wl.to_torch(w)
    unified_arrays(w, dev)
    uni = run_unified(w, dev)["o"]
    assert torch.equal(two.view(torch.int16), uni.view(torch.int16))


def test_unified_smaller_prefix_lens_move_the_causal_boundary():
    # prefix_lens below the true prefix: the keys between become causal keys
    w = wl.build(wl.CONFIGS["llama8b"], prefix_lens=np.array([300, 77, 1000]), extend_lens=np.array([40, 64, 9]))
    parity(w, "llama8b-short-prefix-lens", prefix_lens=[290, 0, 990])


@pytest.mark.parametrize("name", ["llama8b", "long_prefix"])
def test_unified_full_size(name):
    # every output element at the workload's full size
    w = wl.get(name)
    say(f"unified full-size {name}: T={w.total_q} P={w.num_prefix}")
    dev = wl.to_torch(w)
    arrays = unified_arrays(w, dev)
    run_unified(w, dev)
    check(out_f64(dev), oracle_unified(w, *arrays), w.cfg.dtype, f"{name}-unified-full")


def test_graph_replay_index_build_and_both_entries():
    # the index build, a two-part call with split chunks (one long prefix)
    # and a unified call over the built arrays, captured in one HIP graph:
    # their launches record no memset, so every replay equals the eager run
    w = wl.custom(dtype="bf16", prefix_lens=[20000, 300, 0, 77], extend_lens=[3, 200, 64, 1], hq=8, hkv=2,
                  lq=128, lv=128, seed=71)
    dev = wl.to_torch(w)
    n_u = dev["kv_indices"].numel() + dev["extend_kv_indices"].numel()
    uni = (torch.empty(w.bs + 1, dtype=torch.int32, device="cuda"),
           torch.empty(n_u, dtype=torch.int64, device="cuda"),
           torch.empty(w.bs, dtype=torch.int32, device="cuda"))
    o2 = torch.empty_like(dev["o"])
    d1 = pkv.make_desc(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"], w.bs,
                       dev["kv_indices"].numel())
    d2 = pkv.make_desc(dev["q"], None, None, o2, dev["k_pool"], dev["v_pool"], w.bs, n_u)
    nbytes = max(pkv.extend_attention_workspace_size(d1), pkv.extend_attention_workspace_size(d2))
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")

    def call():
        pkv.build_unified_kv_indices(dev["kv_indptr"], dev["kv_indices"], dev["extend_start_loc"],
                                     dev["extend_seq_lens"], dev["extend_kv_indices"], w.bs, out=uni)
        pkv.extend_attention_fwd(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"],
                                 dev["qo_indptr"], dev["kv_indptr"], dev["kv_indices"], sm_scale=w.sm_scale,
                                 workspace=ws)
        pkv.extend_attention_fwd_unified(dev["q"], o2, dev["k_pool"], dev["v_pool"], dev["qo_indptr"], uni[0],
                                         uni[1], uni[2], sm_scale=w.sm_scale, workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = (dev["o"].clone(), o2.clone(), uni[0].clone(), uni[1][:int(uni[0][-1])].clone(), uni[2].clone())
    check(eager[0].float().cpu().numpy().astype(np.float64), oracle.extend_attention_workload(w), "bf16",
          "graph batch, eager")
    assert torch.equal(eager[0], eager[1]), "unified and two-part calls differ"
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        call()
    for _ in range(3):
        dev["o"].fill_(float("nan"))
        o2.fill_(float("nan"))
        uni[0].fill_(-1)
        uni[1].fill_(-1)
        uni[2].fill_(-1)
        graph.replay()
        torch.cuda.synchronize()
        got = (dev["o"], o2, uni[0], uni[1][:int(eager[2][-1])], uni[2])
        for g, e in zip(got, eager):
            assert torch.equal(g, e), "a graph replay differs from the eager run"
        call()  # eager work between the replays
        torch.cuda.synchronize()
