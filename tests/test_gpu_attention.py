"""Extend attention on the GPU against the CPU oracle.

Full element-by-element comparison at sizes the oracle finishes in seconds
(several tiles and ragged tails) and at the workloads' full sizes in the
launch configuration the benchmark uses, edge cases, and bitwise invariants
(determinism, pool-slot permutation, batch order).
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import check, out_f64, run_gpu, say

pytestmark = pytest.mark.gpu


def parity_full(w, what):
    say(f"parity {what}: bs={w.bs} T={w.total_q} P={w.num_prefix} dims={w.cfg.lq}/{w.cfg.lv} "
        f"heads={w.cfg.hq}/{w.cfg.hkv} cap={w.logit_cap}")
    dev = run_gpu(w)
    want = oracle.extend_attention_workload(w)
    check(out_f64(dev), want, w.cfg.dtype, what)
    return dev


# ---- reduced sizes, every output compared

SMALL = {
    "tiny_fp32": dict(),  # the tiny workload itself
    "llama8b": dict(prefix_lens=[0, 300, 77, 1000, 5], extend_lens=[200, 1, 64, 33, 129]),
    "long_prefix": dict(prefix_lens=[3000, 1500], extend_lens=[70, 19]),
    "mla": dict(prefix_lens=[600, 1], extend_lens=[3, 20]),
    "skewed_cap": dict(prefix_lens=[0, 900, 13, 2], extend_lens=[300, 5, 64, 1]),
}


@pytest.mark.parametrize("name", list(SMALL))
def test_parity_reduced(name):
    w = wl.build(wl.CONFIGS[name], **{k: np.array(v) for k, v in SMALL[name].items()})
    parity_full(w, f"{name}-reduced")


EDGE = [
    dict(name="e1-decode", dtype="bf16", prefix_lens=[500, 0, 31], extend_lens=[1, 1, 1], hq=8, hkv=2, lq=128, lv=128),
    dict(name="p0-causal", dtype="bf16", prefix_lens=[0, 0], extend_lens=[257, 64], hq=4, hkv=4, lq=128, lv=128),
    dict(name="empty-seq", dtype="bf16", prefix_lens=[10, 40, 0, 7], extend_lens=[5, 0, 0, 9], hq=4, hkv=1, lq=64, lv=64),
    dict(name="cap1-d256", dtype="bf16", prefix_lens=[150, 3], extend_lens=[40, 70], hq=4, hkv=2, lq=256, lv=256, logit_cap=1.0),
    dict(name="192x128", dtype="bf16", prefix_lens=[100, 33], extend_lens=[50, 7], hq=6, hkv=2, lq=192, lv=128),
    dict(name="288x256", dtype="bf16", prefix_lens=[65, 0], extend_lens=[30, 41], hq=4, hkv=1, lq=288, lv=256),
    dict(name="mqa-64", dtype="bf16", prefix_lens=[129, 64, 1], extend_lens=[63, 65, 128], hq=16, hkv=1, lq=64, lv=64),
    dict(name="group7", dtype="bf16", prefix_lens=[200, 17], extend_lens=[37, 100], hq=28, hkv=4, lq=128, lv=128),
    dict(name="fp32-128", dtype="fp32", prefix_lens=[40, 0, 100], extend_lens=[9, 50, 1], hq=4, hkv=2, lq=128, lv=128, sm_scale=0.05),
    dict(name="neg-scale", dtype="bf16", prefix_lens=[20], extend_lens=[20], hq=2, hkv=1, lq=64, lv=64, sm_scale=-0.1),
    # head dim 128: soft-cap and a negative scale, ragged groups
    dict(name="cap-d128", dtype="bf16", prefix_lens=[90, 0, 300], extend_lens=[70, 130, 1], hq=12, hkv=4, lq=128,
         lv=128, logit_cap=20.0),
    dict(name="neg-d128", dtype="bf16", prefix_lens=[37, 64], extend_lens=[100, 3], hq=6, hkv=2, lq=128, lv=128,
         sm_scale=-0.07),
    # 576/512 with V the first 512 columns of K (split-wave kernel): ragged
    # groups of 3 rows, soft-cap, negative scale, and V stored apart from K
    dict(name="mla-g3-cap", dtype="bf16", prefix_lens=[70, 0, 200], extend_lens=[33, 65, 2], hq=3, hkv=1, lq=576,
         lv=512, v_aliases_k=True, std=0.5, logit_cap=30.0),
    dict(name="mla-g16-neg", dtype="bf16", prefix_lens=[45, 130], extend_lens=[19, 8], hq=16, hkv=1, lq=576, lv=512,
         v_aliases_k=True, std=0.5, sm_scale=-0.06),
    dict(name="mla-v-apart", dtype="bf16", prefix_lens=[33, 0], extend_lens=[10, 40], hq=8, hkv=1, lq=576, lv=512,
         std=0.5),
    # plain head dims between the tile widths (zero columns in the next wider
    # tile): several key tiles, ragged row tiles, a soft-cap and a negative scale
    dict(name="d80", dtype="bf16", prefix_lens=[300, 0, 41], extend_lens=[70, 129, 3], hq=8, hkv=2, lq=80, lv=80),
    dict(name="d96", dtype="bf16", prefix_lens=[260, 7], extend_lens=[90, 200], hq=12, hkv=4, lq=96, lv=96),
    dict(name="d96-cap", dtype="bf16", prefix_lens=[500, 0], extend_lens=[33, 64], hq=4, hkv=1, lq=96, lv=96,
         logit_cap=5.0),
    dict(name="d112-neg", dtype="bf16", prefix_lens=[129, 400], extend_lens=[17, 60], hq=6, hkv=2, lq=112, lv=112,
         sm_scale=-0.08),
    dict(name="d160", dtype="bf16", prefix_lens=[200, 3], extend_lens=[45, 100], hq=8, hkv=4, lq=160, lv=160),
    dict(name="d192-cap", dtype="bf16", prefix_lens=[90, 0], extend_lens=[30, 77], hq=4, hkv=2, lq=192, lv=192,
         logit_cap=20.0),
]


@pytest.mark.parametrize("case", EDGE, ids=[c["name"] for c in EDGE])
def test_parity_edge(case):
    case = dict(case)
    name = case.pop("name")
    parity_full(wl.custom(**case), name)


def test_long_prefix_single_sequence():
    w = wl.custom(dtype="bf16", prefix_lens=[65536], extend_lens=[3], hq=8, hkv=1, lq=128, lv=128)
    parity_full(w, "bs1-P65536")


def test_long_prefix_split_mla():
    # key ranges split into partials and merged, 64-row tiles of the split-wave kernel
    w = wl.custom(dtype="bf16", prefix_lens=[24000], extend_lens=[2], hq=16, hkv=1, lq=576, lv=512,
                  v_aliases_k=True, std=0.5)
    dev = wl.to_torch(w)
    desc = pkv.make_desc(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"], w.bs,
                         w.num_prefix)
    assert pkv.extend_attention_kernel_name(desc, dev["k_ext"], dev["v_ext"], dev["k_pool"],
                                            dev["v_pool"]) == "attn_dl_kernel"
    parity_full(w, "mla-bs1-P24000")


def test_planner_arrays_in_global_memory():
    # more sequences, or more row tiles, than the planner keeps in LDS
    w = wl.custom(dtype="bf16", prefix_lens=[3] * 4500, extend_lens=[1] * 4500, hq=4, hkv=2, lq=64, lv=64)
    parity_full(w, "bs4500")
    w = wl.custom(dtype="bf16", prefix_lens=[5] * 1100, extend_lens=[1] * 1100, hq=64, hkv=8, lq=64, lv=64)
    parity_full(w, "items9352")


def test_rows_beyond_descriptor_plan_nothing():
    # qo_indptr names far more rows than the descriptor's total_q_tokens (32 row
    # tiles against a bound of 4): no work, o untouched
    w = wl.custom(dtype="bf16", prefix_lens=[40], extend_lens=[2000], hq=4, hkv=2, lq=128, lv=128)
    dev = wl.to_torch(w)
    desc = pkv.make_desc(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"], w.bs,
                         w.num_prefix)
    desc.total_q_tokens = 10
    nbytes = pkv.extend_attention_workspace_size(desc)
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev["q"].device)
    lib = pkv.library()
    p = lambda t: t.data_ptr()
    rc = lib.extend_attention_fwd(p(dev["q"]), p(dev["k_ext"]), p(dev["v_ext"]), p(dev["o"]), p(dev["k_pool"]),
                                  p(dev["v_pool"]), p(dev["qo_indptr"]), p(dev["kv_indptr"]), p(dev["kv_indices"]),
                                  0.0, 0.0, ctypes.byref(desc), p(ws), nbytes,
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.isnan(dev["o"].float()).all(), "rows were written although the plan should be empty"


def test_empty_batch_is_noop():
    w = wl.custom(dtype="bf16", prefix_lens=[5, 0], extend_lens=[0, 0], hq=4, hkv=2, lq=64, lv=64)
    dev = wl.to_torch(w)
    pkv.extend_attention_fwd(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"],
                             dev["qo_indptr"], dev["kv_indptr"], dev["kv_indices"])
    torch.cuda.synchronize()
    assert dev["o"].numel() == 0


@pytest.mark.parametrize("kernel", ["dl", "attn"])
def test_every_kernel_on_one_batch(kernel):
    # each kernel that serves bf16 head dim 128, on the same ragged batch with split key ranges
    w = wl.build(wl.CONFIGS["llama8b"], prefix_lens=np.array([0, 300, 77, 9000, 5]),
                 extend_lens=np.array([200, 1, 64, 33, 129]))
    dev = wl.to_torch(w)
    desc = pkv.make_desc(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"], w.bs,
                         w.num_prefix)
    try:
        pkv.extend_attention_prefer_kernel(kernel)
        name = pkv.extend_attention_kernel_name(desc, dev["k_ext"], dev["v_ext"], dev["k_pool"], dev["v_pool"])
        assert name == {"dl": "attn_dl_kernel", "attn": "attn_kernel"}[kernel]
        parity_full(w, f"llama8b-shape-{kernel}")
    finally:
        pkv.extend_attention_prefer_kernel("auto")


# ---- full sizes, every output element, same launch path as the benchmark

@pytest.mark.parametrize("name", wl.CONFIG_ORDER + wl.AUX_CONFIGS)
def test_parity_full_size(name):
    w = wl.get(name)
    say(f"full-size {name}: T={w.total_q} P={w.num_prefix} ({w.causal_flops() / 1e9:.1f} GFLOP for the oracle)")
    dev = run_gpu(w)
    check(out_f64(dev), oracle.extend_attention_workload(w), w.cfg.dtype, f"{name}-full")


# ---- bitwise invariants

def test_deterministic_and_slot_permutation_invariant():
    w = wl.build(wl.CONFIGS["llama8b"], prefix_lens=np.array([700, 5, 1200]), extend_lens=np.array([100, 300, 17]))
    a = out_f64(run_gpu(w)).copy()
    b = out_f64(run_gpu(w))
    assert np.array_equal(a, b), "run-to-run results differ"
    perm = np.random.default_rng(1).permutation(w.cfg.pool_slots)
    k2 = np.empty_like(w.k_pool)
    v2 = np.empty_like(w.v_pool)
    k2[perm] = w.k_pool
    v2[perm] = w.v_pool
    w.k_pool, w.v_pool, w.kv_indices = k2, v2, perm[w.kv_indices]
    c = out_f64(run_gpu(w))
    assert np.array_equal(a, c), "pool-slot permutation changed the result"


def test_batch_order_invariant():
    w = wl.build(wl.CONFIGS["skewed_cap"], prefix_lens=np.array([0, 900, 13, 2, 40]),
                 extend_lens=np.array([300, 5, 64, 1, 8]))
    base = out_f64(run_gpu(w))
    order = [3, 1, 4, 0, 2]
    rows = np.concatenate([np.arange(w.qo_indptr[b], w.qo_indptr[b + 1]) for b in order])
    e = w.extend_lens[order]
    p = w.prefix_lens[order]
    w2 = wl.Workload(w.cfg, p, e, np.concatenate([[0], np.cumsum(e)]).astype(np.int32),
                     np.concatenate([[0], np.cumsum(p)]).astype(np.int32),
                     np.concatenate([w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]] for b in order]),
                     w.extend_kv_indices[rows], np.concatenate([[0], np.cumsum(e)[:-1]]).astype(np.int32),
                     np.ascontiguousarray(w.q[rows]), np.ascontiguousarray(w.k_ext[rows]),
                     np.ascontiguousarray(w.v_ext[rows]), w.k_pool, w.v_pool)
    got = out_f64(run_gpu(w2))
    assert np.array_equal(got, base[rows])


def test_two_streams_concurrently():
    # two batches issued on two streams at once (each stream has its own
    # workspace in the binding's cache) equal the same calls one after another
    wa = wl.build(wl.CONFIGS["llama8b"], **{k: np.array(v) for k, v in SMALL["llama8b"].items()})
    wb = wl.custom(dtype="bf16", prefix_lens=[20000, 5], extend_lens=[3, 70], hq=8, hkv=1, lq=128, lv=128, seed=73)
    da, db = run_gpu(wa), run_gpu(wb)
    want = (da["o"].clone(), db["o"].clone())
    da["o"].fill_(float("nan"))
    db["o"].fill_(float("nan"))
    sa, sb = torch.cuda.Stream(), torch.cuda.Stream()
    sa.wait_stream(torch.cuda.current_stream())
    sb.wait_stream(torch.cuda.current_stream())
    for _ in range(3):
        with torch.cuda.stream(sa):
            pkv.extend_attention_fwd(da["q"], da["k_ext"], da["v_ext"], da["o"], da["k_pool"], da["v_pool"],
                                     da["qo_indptr"], da["kv_indptr"], da["kv_indices"], sm_scale=wa.sm_scale,
                                     logit_cap=wa.logit_cap)
        with torch.cuda.stream(sb):
            pkv.extend_attention_fwd(db["q"], db["k_ext"], db["v_ext"], db["o"], db["k_pool"], db["v_pool"],
                                     db["qo_indptr"], db["kv_indptr"], db["kv_indices"], sm_scale=wb.sm_scale,
                                     logit_cap=wb.logit_cap)
    torch.cuda.synchronize()
    assert torch.equal(da["o"], want[0]) and torch.equal(db["o"], want[1])
