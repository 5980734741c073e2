"""Attention on strided views against contiguous tensors and the oracle.

The entry points take (token, head) strides for q, o, the new tokens' K/V and
the pools, with only the last dimension contiguous.  Here q, k and v are
slices of one fused projection buffer [T, Hq + 2 Hkv, L], the output and the
pools are views with padded rows, and every pad holds NaN, so a read or write
outside a view shows up as a non-finite or changed value.  The kernels and
their tiling do not depend on the strides, so each result must equal the
contiguous call's bit for bit, and the oracle within the bf16 bounds.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import check, run_gpu, say

pytestmark = pytest.mark.gpu


def padded(t, pad):
    """A view of t's values whose rows are `pad` elements longer (NaN-filled)."""
    big = torch.full((t.shape[0], t.shape[1], t.shape[2] + pad), float("nan"), dtype=t.dtype, device=t.device)
    big[:, :, :t.shape[2]] = t
    return big, big[:, :, :t.shape[2]]


def fused_qkv(q, k, v):
    """q, k, v as head slices of one [T, Hq + 2 Hkv, L] buffer."""
    hq, hkv = q.shape[1], k.shape[1]
    buf = torch.empty((q.shape[0], hq + 2 * hkv, q.shape[2]), dtype=q.dtype, device=q.device)
    buf[:, :hq], buf[:, hq:hq + hkv], buf[:, hq + hkv:] = q, k, v
    return buf[:, :hq], buf[:, hq:hq + hkv], buf[:, hq + hkv:]


CASES = [
    dict(prefix_lens=[0, 300, 77, 1000], extend_lens=[200, 1, 64, 33], hq=32, hkv=8, lq=128, lv=128),
    dict(prefix_lens=[129, 64, 1], extend_lens=[63, 65, 128], hq=16, hkv=2, lq=64, lv=64, logit_cap=5.0),
    dict(prefix_lens=[150, 3], extend_lens=[40, 70], hq=4, hkv=2, lq=256, lv=256),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"d{c['lq']}-h{c['hq']}/{c['hkv']}")
@pytest.mark.parametrize("path", ["two-part", "unified"])
def test_extend_strided_views(case, path):
    w = wl.custom(dtype="bf16", seed=61, **case)
    say(f"strided extend {path}: dims={w.cfg.lq}/{w.cfg.lv} heads={w.cfg.hq}/{w.cfg.hkv} T={w.total_q}")
    dev = wl.to_torch(w)
    kw = dict(sm_scale=w.sm_scale, logit_cap=w.logit_cap)
    q, k_ext, v_ext = fused_qkv(dev["q"], dev["k_ext"], dev["v_ext"])
    _, k_pool = padded(dev["k_pool"], 8)
    _, v_pool = padded(dev["v_pool"], 24)
    o_big, o = padded(torch.empty_like(dev["q"][:, :, :w.cfg.lv]), 16)
    if path == "two-part":
        want = run_gpu(w, dev)["o"].clone()
        pkv.extend_attention_fwd(q, k_ext, v_ext, o, k_pool, v_pool, dev["qo_indptr"], dev["kv_indptr"],
                                 dev["kv_indices"], **kw)
    else:
        # every key through one index array (the oracle's index build; the
        # workload's pools already hold each new token's K/V at its extend slot)
        indptr, indices, plens = oracle.build_unified_kv_indices(
            w.kv_indptr, w.kv_indices, w.extend_start_loc, w.extend_lens, w.extend_kv_indices, w.bs)
        ind_ptr = torch.from_numpy(indptr.astype(np.int32)).cuda()
        ind = torch.from_numpy(indices[:int(indptr[-1])].astype(np.int64)).cuda()
        plens = torch.from_numpy(plens.astype(np.int32)).cuda()
        want = torch.empty_like(dev["o"])
        pkv.extend_attention_fwd_unified(dev["q"], want, dev["k_pool"], dev["v_pool"], dev["qo_indptr"], ind_ptr,
                                         ind, plens, **kw)
        pkv.extend_attention_fwd_unified(q, o, k_pool, v_pool, dev["qo_indptr"], ind_ptr, ind, plens, **kw)
    torch.cuda.synchronize()
    assert torch.equal(o, want), "strided views change the result"
    assert torch.isnan(o_big[:, :, w.cfg.lv:]).all(), "a write landed in the output's row padding"
    check(o.float().cpu().numpy().astype(np.float64), oracle.extend_attention_workload(w), "bf16",
          f"strided {path}")


def test_decode_strided_views():
    d = wl.decode_custom([0, 1, 300, 1000, 65, 2500], hq=32, hkv=8, lq=128, lv=128, seed=67)
    dev = wl.decode_to_torch(d)
    pkv.decode_attention_fwd(dev["q"], dev["o"], dev["k_pool"], dev["v_pool"], dev["kv_indptr"], dev["kv_indices"],
                             sm_scale=d.sm_scale)
    want = dev["o"].clone()
    _, q = padded(dev["q"], 64)
    _, k_pool = padded(dev["k_pool"], 8)
    _, v_pool = padded(dev["v_pool"], 40)
    o_big, o = padded(torch.empty_like(dev["o"]), 8)
    pkv.decode_attention_fwd(q, o, k_pool, v_pool, dev["kv_indptr"], dev["kv_indices"], sm_scale=d.sm_scale)
    torch.cuda.synchronize()
    assert torch.equal(o, want), "strided views change the result"
    assert torch.isnan(o_big[:, :, d.cfg.lv:]).all(), "a write landed in the output's row padding"
    got = o.float().cpu().numpy().astype(np.float64)
    check(got, oracle.decode_attention(d.q, d.k_pool, d.v_pool, d.kv_indptr, d.kv_indices, d.sm_scale,
                                       d.logit_cap, "bf16"), "bf16", "strided decode")
