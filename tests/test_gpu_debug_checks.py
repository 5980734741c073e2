"""The debug build (libpkv_debug.so): every index array is checked on the
device before any kernel reads it.

A valid batch gives the release library's result bit for bit (the same
kernels run); a pool slot outside [0, pool_slots), a decreasing indptr or a
negative prefix length returns PKV_ERR_RANGE (-6) and leaves the output
untouched -- the attention kernels never run, so the bad slot is never
dereferenced.
"""

import ctypes

import numpy as np
import pytest
import torch

import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import run_gpu, say

pytestmark = pytest.mark.gpu

PKV_ERR_RANGE = -6


def _ptr(t):
    return None if t is None else t.data_ptr()


def _extend_debug(w, dev, kv_indices=None, kv_indptr=None):
    lib = pkv.debug_library()
    kvi = dev["kv_indices"] if kv_indices is None else kv_indices
    kvp = dev["kv_indptr"] if kv_indptr is None else kv_indptr
    desc = pkv.make_desc(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"], w.bs,
                         kvi.numel())
    ws = torch.empty(pkv.extend_attention_workspace_size(desc), dtype=torch.uint8, device="cuda")
    rc = lib.extend_attention_fwd(_ptr(dev["q"]), _ptr(dev["k_ext"]), _ptr(dev["v_ext"]), _ptr(dev["o"]),
                                  _ptr(dev["k_pool"]), _ptr(dev["v_pool"]), _ptr(dev["qo_indptr"]), _ptr(kvp),
                                  _ptr(kvi), ctypes.c_float(w.sm_scale), ctypes.c_float(w.logit_cap),
                                  ctypes.byref(desc), _ptr(ws), ws.numel(),
                                  torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    return rc, lib.pkv_last_error().decode()


def _batch():
    return wl.custom(dtype="bf16", prefix_lens=[300, 0, 77], extend_lens=[40, 129, 5], hq=8, hkv=2, lq=128,
                     lv=128, seed=91)


def test_debug_build_matches_release_on_a_valid_batch():
    w = _batch()
    want = run_gpu(w)["o"].clone()
    dev = wl.to_torch(w)
    dev["o"].fill_(float("nan"))
    rc, msg = _extend_debug(w, dev)
    assert rc == 0, msg
    assert torch.equal(dev["o"].view(torch.int16), want.view(torch.int16))


@pytest.mark.parametrize("fault", ["slot-past-pool", "negative-slot", "decreasing-kv-indptr"])
def test_debug_build_rejects_bad_indices(fault):
    w = _batch()
    dev = wl.to_torch(w)
    dev["o"].fill_(float("nan"))
    kvi = dev["kv_indices"].clone()
    kvp = dev["kv_indptr"].clone()
    if fault == "slot-past-pool":
        kvi[17] = w.cfg.pool_slots
    elif fault == "negative-slot":
        kvi[-1] = -3
    else:
        kvp[2] = kvp[1] - 1  # sequence 1 would span -1 keys
    say(f"debug build, {fault}")
    rc, msg = _extend_debug(w, dev, kv_indices=kvi, kv_indptr=kvp)
    assert rc == PKV_ERR_RANGE, (rc, msg)
    assert "debug index check" in msg
    assert torch.isnan(dev["o"].float()).all(), "the output was written although the call failed"


def test_debug_build_checks_unified_prefix_lens_and_decode_slots():
    lib = pkv.debug_library()
    stream = torch.cuda.current_stream().cuda_stream
    # unified entry: a negative prefix length
    w = _batch()
    dev = wl.to_torch(w)
    import oracle
    indptr, indices, plens = oracle.build_unified_kv_indices(w.kv_indptr, w.kv_indices, w.extend_start_loc,
                                                             w.extend_lens, w.extend_kv_indices, w.bs)
    u_indptr = torch.from_numpy(indptr.astype(np.int32)).cuda()
    u_indices = torch.from_numpy(indices[:int(indptr[-1])].astype(np.int64)).cuda()
    u_plens = torch.from_numpy(plens.astype(np.int32)).cuda()
    u_plens[1] = -1
    desc = pkv.make_desc(dev["q"], None, None, dev["o"], dev["k_pool"], dev["v_pool"], w.bs, u_indices.numel())
    ws = torch.empty(pkv.extend_attention_workspace_size(desc), dtype=torch.uint8, device="cuda")
    rc = lib.extend_attention_fwd_unified(_ptr(dev["q"]), _ptr(dev["o"]), _ptr(dev["k_pool"]), _ptr(dev["v_pool"]),
                                          _ptr(dev["qo_indptr"]), _ptr(u_indptr), _ptr(u_indices), _ptr(u_plens),
                                          ctypes.c_float(0.0), ctypes.c_float(0.0), ctypes.byref(desc), _ptr(ws),
                                          ws.numel(), stream)
    torch.cuda.synchronize()
    assert rc == PKV_ERR_RANGE, lib.pkv_last_error().decode()
    # decode: a slot past the pool
    d = wl.decode_custom([5, 300, 0, 40], hq=8, hkv=2, lq=128, lv=128, seed=93)
    t = wl.decode_to_torch(d)
    t["kv_indices"][7] = d.k_pool.shape[0] + 5
    desc = pkv.make_desc(t["q"], None, None, t["o"], t["k_pool"], t["v_pool"], d.bs, d.num_keys)
    ws = torch.empty(pkv.decode_attention_workspace_size(desc), dtype=torch.uint8, device="cuda")
    rc = lib.decode_attention_fwd(_ptr(t["q"]), _ptr(t["o"]), _ptr(t["k_pool"]), _ptr(t["v_pool"]),
                                  _ptr(t["kv_indptr"]), _ptr(t["kv_indices"]), ctypes.c_float(0.0),
                                  ctypes.c_float(0.0), ctypes.byref(desc), _ptr(ws), ws.numel(), stream)
    torch.cuda.synchronize()
    assert rc == PKV_ERR_RANGE, lib.pkv_last_error().decode()
