"""Custom attention masks on the GPU against the CPU oracle (page
"extend_attention.py", _fwd_kernel_unified with USE_CUSTOM_MASK: a byte per
(query, key) replaces the causal rule), on every kernel family, with the
window and sinks, on the split path and through the unified entry."""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import check, out_f64, say

pytestmark = pytest.mark.gpu


def make_mask(w, kind, seed=0, span=None):
    """Byte matrices [E_b, L_b] (L_b = P_b + E_b, or span[b]) and int64 offsets.
    kind "tree": every prefix key, the row's own key and a random subset of the
    earlier new tokens; "random": any key, the own key always."""
    rng = np.random.default_rng(seed)
    parts, offs, off = [], [], 0
    for b in range(w.bs):
        E = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
        P = int(w.kv_indptr[b + 1] - w.kv_indptr[b])
        L = P + E if span is None else int(span[b])
        m = np.zeros((E, L), np.uint8)
        if kind == "tree":
            m[:, :P] = 1
            for i in range(E):
                m[i, P:P + i] = rng.random(i) < 0.4
        else:
            m[:] = rng.random((E, L)) < 0.3
        for i in range(E):
            if P + i < L:
                m[i, P + i] = 1
        offs.append(off)
        off += m.size
        parts.append(m.ravel())
    return (np.concatenate(parts) if parts else np.zeros(1, np.uint8)), np.array(offs, np.int64)


def run(w, kind, what, window=0, sinks=None, seed=0):
    m, mi = make_mask(w, kind, seed)
    say(f"mask {what}: bs={w.bs} T={w.total_q} P={w.num_prefix} dims={w.cfg.lq}/{w.cfg.lv} {kind} "
        f"window={window} sinks={'yes' if sinks is not None else 'no'} bytes={m.size}")
    dev = wl.to_torch(w)
    dm, dmi = torch.from_numpy(m).cuda(), torch.from_numpy(mi).cuda()
    desc = pkv.make_desc(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"], w.bs,
                         w.num_prefix)
    pkv.extend_attention_fwd(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"],
                             dev["qo_indptr"], dev["kv_indptr"], dev["kv_indices"], sm_scale=w.sm_scale,
                             logit_cap=w.logit_cap, sliding_window=window,
                             sinks=torch.from_numpy(sinks).cuda() if sinks is not None else None,
                             custom_mask=dm, mask_indptr=dmi)
    torch.cuda.synchronize()
    want = oracle.extend_attention_workload(w, window=window, sinks=sinks, custom_mask=m, mask_indptr=mi)
    check(out_f64(dev), want, w.cfg.dtype, what)


REDUCED = {
    "tiny_fp32": dict(),
    "llama8b": dict(prefix_lens=[0, 300, 77, 1000, 5], extend_lens=[200, 1, 64, 33, 129]),
    "mla": dict(prefix_lens=[600, 1], extend_lens=[3, 20]),
    "skewed_cap": dict(prefix_lens=[0, 900, 13, 2], extend_lens=[300, 5, 64, 1]),
}


@pytest.mark.parametrize("name", list(REDUCED))
@pytest.mark.parametrize("kind", ["tree", "random"])
def test_custom_mask_reduced(name, kind):
    w = wl.build(wl.CONFIGS[name], **{k: np.array(v) for k, v in REDUCED[name].items()})
    run(w, kind, f"{name}-{kind}")


def test_custom_mask_with_window_and_sinks():
    w = wl.build(wl.CONFIGS["llama8b"], prefix_lens=np.array([0, 300, 77]), extend_lens=np.array([200, 1, 64]))
    sinks = np.random.default_rng(4).uniform(-2, 3, size=w.cfg.hq).astype(np.float32)
    run(w, "random", "llama8b-random-w90-sinks", window=90, sinks=sinks, seed=5)


def test_custom_mask_192x128():
    w = wl.custom(dtype="bf16", prefix_lens=[100, 33], extend_lens=[50, 7], hq=6, hkv=2, lq=192, lv=128)
    run(w, "random", "192x128-random", seed=6)


def test_custom_mask_split_chunks():
    w = wl.custom(dtype="bf16", prefix_lens=[20000], extend_lens=[300], hq=8, hkv=2, lq=128, lv=128)
    run(w, "random", "bs1-P20000-random", seed=7)


def test_unified_custom_mask():
    w = wl.build(wl.CONFIGS["llama8b"], prefix_lens=np.array([0, 300, 77]), extend_lens=np.array([200, 1, 64]))
    indptr, indices, plens = oracle.build_unified_kv_indices(
        w.kv_indptr, w.kv_indices, w.extend_start_loc, w.extend_lens, w.extend_kv_indices, w.bs)
    indices = indices[:int(indptr[-1])]
    m, mi = make_mask(w, "random", 8, span=np.diff(indptr))
    dev = wl.to_torch(w)
    pkv.extend_attention_fwd_unified(dev["q"], dev["o"], dev["k_pool"], dev["v_pool"], dev["qo_indptr"],
                                     torch.from_numpy(indptr.astype(np.int32)).cuda(),
                                     torch.from_numpy(indices.astype(np.int64)).cuda(),
                                     torch.from_numpy(plens.astype(np.int32)).cuda(), sm_scale=w.sm_scale,
                                     custom_mask=torch.from_numpy(m).cuda(), mask_indptr=torch.from_numpy(mi).cuda())
    torch.cuda.synchronize()
    want = oracle.extend_attention_unified(w.q, w.k_pool, w.v_pool, w.qo_indptr, indptr, indices, plens,
                                           w.sm_scale, 0.0, "bf16", custom_mask=m, mask_indptr=mi)
    check(out_f64(dev), want, "bf16", "unified-random-mask")
