"""The steps before attention on the GPU against the CPU oracle, bit for bit:
the KV-cache store of the new tokens and the request-to-token index gather
(page "flashinfer_backend.py": set_kv_buffer in forward_extend,
create_flashinfer_kv_indices_triton)."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import say

pytestmark = pytest.mark.gpu


def _dev(x, dtype):
    t = torch.from_numpy(np.ascontiguousarray(x))
    return (t.view(torch.bfloat16) if dtype == "bf16" else t).cuda()


def _host(t, dtype):
    t = t.cpu()
    return (t.view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else t.numpy())


def _same_bits(a, b):
    # byte comparison: unused pool slots hold NaN, which never compares equal
    return a.shape == b.shape and np.array_equal(np.ascontiguousarray(a).view(np.uint8),
                                                 np.ascontiguousarray(b).view(np.uint8))


STORE_CASES = [
    dict(name="bf16-128-gqa", dtype="bf16", prefix_lens=[40, 0, 300], extend_lens=[17, 64, 1], hq=8, hkv=4,
         lq=128, lv=128),
    dict(name="fp32-64", dtype="fp32", prefix_lens=[16, 0], extend_lens=[8, 12], hq=4, hkv=2, lq=64, lv=64),
    dict(name="bf16-192x128", dtype="bf16", prefix_lens=[5], extend_lens=[33], hq=6, hkv=2, lq=192, lv=128),
    dict(name="mla-v-in-k", dtype="bf16", prefix_lens=[7, 21], extend_lens=[5, 40], hq=8, hkv=1, lq=576, lv=512,
         v_aliases_k=True, std=0.5),
]


@pytest.mark.parametrize("case", STORE_CASES, ids=[c["name"] for c in STORE_CASES])
def test_store_bit_exact(case):
    kw = {k: v for k, v in case.items() if k != "name"}
    w = wl.custom(**kw)
    dt = w.cfg.dtype
    say(f"store {case['name']}: T={w.total_q} slots={w.k_pool.shape[0]}")
    # clear the new tokens' rows first, then store them
    kp0 = w.k_pool.copy()
    kp0[w.extend_kv_indices] = 0
    if w.cfg.v_aliases_k:
        vp0 = kp0[..., :w.cfg.lv]
    else:
        vp0 = w.v_pool.copy()
        vp0[w.extend_kv_indices] = 0
    want_k, want_v = oracle.store_kv_cache(w.k_ext, w.v_ext if not w.cfg.v_aliases_k else w.k_ext[..., :w.cfg.lv],
                                           kp0, vp0, w.extend_kv_indices)
    kp = _dev(kp0, dt)
    ke = _dev(w.k_ext, dt)
    if w.cfg.v_aliases_k:
        vp, ve = kp[..., :w.cfg.lv], ke[..., :w.cfg.lv]
    else:
        vp, ve = _dev(vp0, dt), _dev(w.v_ext, dt)
    loc = torch.from_numpy(w.extend_kv_indices.astype(np.int64)).cuda()
    pkv.store_kv_cache(ke, ve, kp, vp, loc)
    torch.cuda.synchronize()
    assert _same_bits(_host(kp, dt), want_k)
    if not w.cfg.v_aliases_k:
        assert _same_bits(_host(vp, dt), want_v)


def test_store_full_size_llama8b():
    w = wl.get("llama8b")
    kp0 = w.k_pool.copy()
    vp0 = w.v_pool.copy()
    kp0[w.extend_kv_indices] = 0
    vp0[w.extend_kv_indices] = 0
    kp, vp = _dev(kp0, "bf16"), _dev(vp0, "bf16")
    loc = torch.from_numpy(w.extend_kv_indices.astype(np.int64)).cuda()
    pkv.store_kv_cache(_dev(w.k_ext, "bf16"), _dev(w.v_ext, "bf16"), kp, vp, loc)
    torch.cuda.synchronize()
    # the workload's pool already holds the new tokens at their slots
    assert _same_bits(_host(kp, "bf16"), w.k_pool) and _same_bits(_host(vp, "bf16"), w.v_pool)


def test_store_no_tokens_is_noop():
    kp = torch.zeros(8, 2, 64, dtype=torch.bfloat16, device="cuda")
    e = torch.zeros(0, 2, 64, dtype=torch.bfloat16, device="cuda")
    pkv.store_kv_cache(e, e, kp, kp.clone(), torch.zeros(0, dtype=torch.int64, device="cuda"))
    torch.cuda.synchronize()
    assert int(kp.view(torch.int16).abs().sum()) == 0


@pytest.mark.parametrize("bs,rows,stride,with_start", [(0, 4, 64, False), (1, 3, 5000, True), (7, 40, 300, False),
                                                       (33, 64, 2048, True), (1000, 1200, 96, True)])
def test_gather_bit_exact(bs, rows, stride, with_start):
    rng = np.random.default_rng(bs + stride)
    table = rng.integers(0, 1 << 30, size=(rows, stride)).astype(np.int32)
    rpi = rng.integers(0, rows, size=bs)
    start = rng.integers(0, stride // 2, size=bs).astype(np.int32)
    lens = rng.integers(0, stride // 2, size=bs).astype(np.int32)
    if bs:
        lens[0] = 0
    want_ptr, want_idx = oracle.gather_kv_indices(table, rpi, lens, start if with_start else None)
    say(f"gather bs={bs} total={int(want_ptr[-1])}")
    t = torch.from_numpy(table).cuda()
    ptr, idx = pkv.gather_kv_indices(t, torch.from_numpy(rpi.astype(np.int64)).cuda(),
                                     torch.from_numpy(lens).cuda(),
                                     torch.from_numpy(start).cuda() if with_start else None,
                                     capacity=int(want_ptr[-1]))
    torch.cuda.synchronize()
    assert np.array_equal(ptr.cpu().numpy(), want_ptr)
    assert np.array_equal(idx.cpu().numpy(), want_idx)


def test_gather_feeds_attention():
    # prefix indices from a request table, then attention, against the oracle on the workload
    w = wl.build(wl.CONFIGS["llama8b"], prefix_lens=np.array([300, 0, 77]), extend_lens=np.array([20, 9, 64]))
    table = np.zeros((5, 512), np.int32)
    rows = np.array([3, 0, 1])
    for b, r in enumerate(rows):
        p0, p1 = w.kv_indptr[b], w.kv_indptr[b + 1]
        table[r, 10:10 + (p1 - p0)] = w.kv_indices[p0:p1]
    dev = wl.to_torch(w)
    ptr, idx = pkv.gather_kv_indices(torch.from_numpy(table).cuda(), torch.from_numpy(rows).cuda(),
                                     torch.from_numpy(w.prefix_lens.astype(np.int32)).cuda(),
                                     torch.full((3,), 10, dtype=torch.int32, device="cuda"),
                                     capacity=w.num_prefix)
    pkv.extend_attention_fwd(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"],
                             dev["qo_indptr"], ptr, idx, sm_scale=w.sm_scale)
    torch.cuda.synchronize()
    from gpu_helpers import check, out_f64
    check(out_f64(dev), oracle.extend_attention_workload(w), "bf16", "gather-then-attend")
