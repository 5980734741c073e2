"""Pins for the CPU oracle against facts fixed outside the oracle itself.

Index build: a hand-worked example and list concatenation of slices.
Attention: torch's scaled_dot_product_attention over an explicitly
concatenated prefix + extend K/V (the reference helper redundant_attention
on the SGLang page extend_attention.py does the same), closed forms (q = 0
gives the running mean of the visible values; saturated soft-cap logits give
weights e^{+-cap}), and exact invariants (pool-slot permutation, batch
permutation, KV-head expansion, cap -> infinity).
"""

import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ----------------------------------------------------------------------------- index build

def test_index_worked_example():
    with open(os.path.join(GOLDEN, "unified_indices_worked_example.json")) as f:
        ex = json.load(f)
    indptr, indices, plens = oracle.build_unified_kv_indices(
        ex["prefix_kv_indptr"], ex["prefix_kv_indices"], ex["extend_start_loc"],
        ex["extend_seq_lens"], ex["extend_kv_indices"], ex["bs"])
    n = ex["expected_unified_kv_indptr"][-1]
    assert indptr.tolist() == ex["expected_unified_kv_indptr"]
    assert indices[:n].tolist() == ex["expected_unified_kv_indices"]
    assert plens.tolist() == ex["expected_prefix_lens"]


def _concat_slices(c):
    out, indptr = [], [0]
    for b in range(c["bs"]):
        lo, hi = int(c["prefix_kv_indptr"][b]), int(c["prefix_kv_indptr"][b + 1])
        es, el = int(c["extend_start_loc"][b]), int(c["extend_seq_lens"][b])
        seg = list(c["prefix_kv_indices"][lo:hi]) + list(c["extend_kv_indices"][es:es + el])
        out += seg
        indptr.append(indptr[-1] + len(seg))
    return indptr, out


@pytest.mark.parametrize("bs,extra,base", [(0, 0, 0), (1, 0, 0), (5, 3, 0), (17, 0, 9), (64, 2, 1)])
def test_index_matches_slice_concatenation(bs, extra, base):
    rng = np.random.default_rng(100 + bs)
    c = wl.index_case(rng, bs, extra_tail=extra, indptr_base=base)
    indptr, indices, plens = oracle.build_unified_kv_indices(
        c["prefix_kv_indptr"], c["prefix_kv_indices"], c["extend_start_loc"],
        c["extend_seq_lens"], c["extend_kv_indices"], bs)
    want_indptr, want = _concat_slices(c)
    assert indptr.tolist() == want_indptr
    assert indices[:len(want)].tolist() == want
    assert plens.tolist() == np.diff(c["prefix_kv_indptr"]).tolist()
    # capacity is the two input lengths; the total fits
    assert len(indices) == len(c["prefix_kv_indices"]) + len(c["extend_kv_indices"])
    assert indptr[-1] <= len(indices)


# ----------------------------------------------------------------------------- attention

def _f64(x, dtype):
    return torch.from_numpy(wl.as_f32(np.ascontiguousarray(x), dtype).astype(np.float64))


def sdpa_reference(w, scale=None):
    """Library attention over the explicitly concatenated prefix + extend K/V."""
    c = w.cfg
    g = c.hq // c.hkv
    outs = []
    for b in range(w.bs):
        q0, q1 = int(w.qo_indptr[b]), int(w.qo_indptr[b + 1])
        k0, k1 = int(w.kv_indptr[b]), int(w.kv_indptr[b + 1])
        if q1 == q0:
            continue
        slots = w.kv_indices[k0:k1]
        k_full = torch.cat([_f64(w.k_pool[slots], c.dtype), _f64(w.k_ext[q0:q1], c.dtype)], 0)
        v_full = torch.cat([_f64(w.v_pool[slots], c.dtype), _f64(w.v_ext[q0:q1], c.dtype)], 0)
        q = _f64(w.q[q0:q1], c.dtype)
        E, P = q1 - q0, k1 - k0
        mask = torch.ones(E, P + E, dtype=torch.bool).tril(diagonal=P)
        k_h = k_full.transpose(0, 1).repeat_interleave(g, dim=0)  # [Hq, P+E, Lq]
        v_h = v_full.transpose(0, 1).repeat_interleave(g, dim=0)
        sc = scale if scale is not None else (c.sm_scale or 1.0 / math.sqrt(c.lq))
        o = torch.nn.functional.scaled_dot_product_attention(
            q.transpose(0, 1), k_h, v_h, attn_mask=mask, scale=sc)
        outs.append(o.transpose(0, 1))
    return torch.cat(outs, 0).numpy()


SDPA_CASES = [
    dict(dtype="fp32", prefix_lens=[16, 0], extend_lens=[8, 12], hq=4, hkv=2, lq=64, lv=64, sm_scale=1 / 8),
    dict(dtype="bf16", prefix_lens=[5, 0, 33, 1], extend_lens=[1, 7, 20, 3], hq=8, hkv=8, lq=32, lv=32),
    dict(dtype="bf16", prefix_lens=[40, 9], extend_lens=[17, 1], hq=6, hkv=2, lq=192, lv=128),
    dict(dtype="bf16", prefix_lens=[13], extend_lens=[6], hq=4, hkv=1, lq=288, lv=256),
    dict(dtype="bf16", prefix_lens=[7, 21], extend_lens=[5, 4], hq=8, hkv=1, lq=576, lv=512,
         v_aliases_k=True, std=0.5),
    dict(dtype="fp32", prefix_lens=[0, 0, 0], extend_lens=[9, 1, 15], hq=2, hkv=1, lq=16, lv=24,
         sm_scale=-0.3),
]


@pytest.mark.parametrize("case", SDPA_CASES, ids=lambda c: f"{c['dtype']}-{c['lq']}x{c['lv']}-h{c['hq']}/{c['hkv']}")
def test_oracle_matches_library_attention(case):
    w = wl.custom(**case)
    got = oracle.extend_attention_workload(w)
    want = sdpa_reference(w)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


def test_default_scale_uses_query_head_dim():
    # 192 / 128: the default scale is 1/sqrt(Lq), not 1/sqrt(Lv)
    w = wl.custom(dtype="bf16", prefix_lens=[11], extend_lens=[4], hq=2, hkv=1, lq=192, lv=128)
    got = oracle.extend_attention_workload(w)
    np.testing.assert_allclose(got, sdpa_reference(w, scale=1 / math.sqrt(192)), atol=1e-12)
    assert np.abs(got - sdpa_reference(w, scale=1 / math.sqrt(128))).max() > 1e-6


def test_zero_prefix_is_plain_causal_attention():
    w = wl.custom(dtype="bf16", prefix_lens=[0, 0], extend_lens=[23, 5], hq=4, hkv=2, lq=64, lv=64)
    got = oracle.extend_attention_workload(w)
    outs = []
    for b in range(2):
        q0, q1 = w.qo_indptr[b], w.qo_indptr[b + 1]
        q = _f64(w.q[q0:q1], "bf16").transpose(0, 1)
        k = _f64(w.k_ext[q0:q1], "bf16").transpose(0, 1).repeat_interleave(2, 0)
        v = _f64(w.v_ext[q0:q1], "bf16").transpose(0, 1).repeat_interleave(2, 0)
        outs.append(torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True).transpose(0, 1))
    np.testing.assert_allclose(got, torch.cat(outs).numpy(), atol=1e-12)


@pytest.mark.parametrize("cap", [0.0, 2.5])
def test_zero_query_gives_running_mean(cap):
    # q = 0 makes every logit 0 (also after the cap): row i averages V over keys 0..P+i.
    w = wl.custom(dtype="fp32", prefix_lens=[6, 0, 3], extend_lens=[4, 3, 1], hq=4, hkv=2,
                  lq=16, lv=8, logit_cap=cap)
    w.q[:] = 0
    got = oracle.extend_attention_workload(w)
    for b in range(w.bs):
        P = int(w.kv_indptr[b + 1] - w.kv_indptr[b])
        slots = w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]]
        q0 = int(w.qo_indptr[b])
        for i in range(int(w.extend_lens[b])):
            for h in range(4):
                g = h // 2
                vals = [w.v_pool[s, g].astype(np.float64) for s in slots]
                vals += [w.v_ext[q0 + j, g].astype(np.float64) for j in range(i + 1)]
                assert len(vals) == P + i + 1
                np.testing.assert_allclose(got[q0 + i, h], np.mean(vals, axis=0), atol=1e-13)


def test_kv_head_of_query_head_is_integer_division():
    # V constant per KV head g (value g + 1) makes every output equal to g(h) + 1.
    w = wl.custom(dtype="fp32", prefix_lens=[5, 2], extend_lens=[3, 4], hq=6, hkv=3, lq=8, lv=4)
    for g in range(3):
        w.v_pool[:, g] = g + 1
        w.v_ext[:, g] = g + 1
    got = oracle.extend_attention_workload(w)
    for h in range(6):
        np.testing.assert_allclose(got[:, h], h // 2 + 1, atol=1e-12)


def test_saturated_soft_cap_closed_form():
    # Logits +-1000 with cap 1: tanh saturates, the weights are exactly e and 1/e.
    lq = 4
    w = wl.custom(dtype="fp32", prefix_lens=[3], extend_lens=[1], hq=1, hkv=1, lq=lq, lv=2,
                  sm_scale=1.0, logit_cap=1.0)
    w.q[0, 0] = [1000.0, 0, 0, 0]
    signs = [1.0, -1.0, -1.0, 1.0]  # prefix keys 0..2, then the token's own key
    keys = [w.k_pool[s, 0] for s in w.kv_indices] + [w.k_ext[0, 0]]
    for k, sgn in zip(keys, signs):
        k[:] = [sgn, 0, 0, 0]
    vals = [w.v_pool[s, 0].astype(np.float64) for s in w.kv_indices] + [w.v_ext[0, 0].astype(np.float64)]
    wts = [math.e if s > 0 else 1 / math.e for s in signs]
    want = sum(wt * v for wt, v in zip(wts, vals)) / sum(wts)
    got = oracle.extend_attention_workload(w)
    np.testing.assert_allclose(got[0, 0], want, atol=1e-14)


def _softcap_example():
    with open(os.path.join(GOLDEN, "softcap_worked_example.json")) as f:
        ex = json.load(f)
    # pool slots 3 and 1 hold the two prefix keys, slot 4 the new token's key
    # (the unified and decode forms read it there); other slots hold NaN
    pool_k = np.full((6, 1, 2), np.nan, np.float32)
    pool_v = np.full((6, 1, 4), np.nan, np.float32)
    for slot, d, v in zip([3, 1, 4], ex["dots"], ex["v"]):
        pool_k[slot, 0] = [d, 0.0]
        pool_v[slot, 0] = v
    q = np.array(ex["q"], np.float32).reshape(1, 1, 2)
    return ex, q, pool_k, pool_v


def _check_softcap_output(ex, out):
    out = np.asarray(out).reshape(-1)
    np.testing.assert_allclose(out, ex["expected_output"], rtol=0, atol=1e-14)
    w = out[:3]
    np.testing.assert_allclose(w, ex["expected_weights"], rtol=0, atol=1e-14)
    # the logits themselves, up to the softmax's shift: log(w_j / w_0) = s_j - s_0
    cap = np.asarray(ex["expected_capped_logits"])
    np.testing.assert_allclose(np.log(w / w[0]), cap - cap[0], rtol=0, atol=1e-13)


def test_softcap_worked_example_two_part():
    ex, q, pool_k, pool_v = _softcap_example()
    k_ext = pool_k[4:5].copy()
    v_ext = pool_v[4:5].copy()
    out = oracle.extend_attention(q, k_ext, v_ext, pool_k, pool_v, [0, 1], [0, 2], [3, 1],
                                  sm_scale=ex["sm_scale"], logit_cap=ex["logit_cap"], dtype="fp32")
    _check_softcap_output(ex, out)


def test_softcap_worked_example_unified():
    ex, q, pool_k, pool_v = _softcap_example()
    out = oracle.extend_attention_unified(q, pool_k, pool_v, [0, 1], [0, 3], [3, 1, 4], [2],
                                          sm_scale=ex["sm_scale"], logit_cap=ex["logit_cap"], dtype="fp32")
    _check_softcap_output(ex, out)


def test_softcap_worked_example_decode():
    ex, q, pool_k, pool_v = _softcap_example()
    out = oracle.decode_attention(q, pool_k, pool_v, [0, 3], [3, 1, 4],
                                  sm_scale=ex["sm_scale"], logit_cap=ex["logit_cap"], dtype="fp32")
    _check_softcap_output(ex, out)


def test_huge_cap_is_no_cap():
    w = wl.custom(dtype="bf16", prefix_lens=[9, 30], extend_lens=[4, 11], hq=4, hkv=2, lq=64, lv=64)
    base = oracle.extend_attention_workload(w)
    object.__setattr__(w.cfg, "logit_cap", 1e30)
    np.testing.assert_allclose(oracle.extend_attention_workload(w), base, atol=1e-12)


def test_cap_bounds_weight_ratio():
    # With cap 1 every logit lies in [-1, 1]: weights differ by at most e^2, so each
    # output is within the values' range and no key dominates.
    w = wl.custom(dtype="fp32", prefix_lens=[3], extend_lens=[1], hq=1, hkv=1, lq=8, lv=3,
                  sm_scale=1.0, logit_cap=1.0, std=30.0)
    got = oracle.extend_attention_workload(w)
    vals = np.stack([w.v_pool[s, 0] for s in w.kv_indices] + [w.v_ext[0, 0]]).astype(np.float64)
    # o = sum a_j v_j with a_j >= e^-2 / (n e^0 ...) : each weight is at least 1/(1 + (n-1) e^2)
    n = len(vals)
    lo = 1.0 / (1 + (n - 1) * math.e ** 2)
    # recover weights from a second run where V is the identity basis
    w2 = wl.custom(dtype="fp32", prefix_lens=[3], extend_lens=[1], hq=1, hkv=1, lq=8, lv=4,
                   sm_scale=1.0, logit_cap=1.0, std=30.0)
    basis = np.eye(4, dtype=np.float32)
    for j, s in enumerate(w2.kv_indices):
        w2.v_pool[s, 0] = basis[j]
    w2.v_ext[0, 0] = basis[3]
    wts = oracle.extend_attention_workload(w2)[0, 0]
    assert wts.min() >= lo - 1e-12 and abs(wts.sum() - 1) < 1e-12
    assert np.isfinite(got).all()


def test_pool_slot_permutation_is_exact():
    w = wl.custom(dtype="bf16", prefix_lens=[12, 0, 25], extend_lens=[3, 9, 2], hq=4, hkv=2,
                  lq=64, lv=64, pool_slots=80)
    base = oracle.extend_attention_workload(w)
    perm = np.random.default_rng(3).permutation(80)  # new slot of old slot s is perm[s]
    k2 = np.empty_like(w.k_pool)
    v2 = np.empty_like(w.v_pool)
    k2[perm] = w.k_pool
    v2[perm] = w.v_pool
    got = oracle.extend_attention(w.q, w.k_ext, w.v_ext, k2, v2, w.qo_indptr, w.kv_indptr,
                                  perm[w.kv_indices], dtype="bf16")
    assert np.array_equal(got, base)


def test_batch_permutation_is_exact():
    w = wl.custom(dtype="bf16", prefix_lens=[12, 0, 25, 4], extend_lens=[3, 9, 2, 6], hq=4,
                  hkv=2, lq=32, lv=32)
    base = oracle.extend_attention_workload(w)
    order = [2, 0, 3, 1]
    q_rows, ke, ve, kvi, e_l, p_l = [], [], [], [], [], []
    for b in order:
        q0, q1 = w.qo_indptr[b], w.qo_indptr[b + 1]
        q_rows.append(np.arange(q0, q1))
        kvi.append(w.kv_indices[w.kv_indptr[b]:w.kv_indptr[b + 1]])
        e_l.append(q1 - q0)
        p_l.append(w.kv_indptr[b + 1] - w.kv_indptr[b])
    rows = np.concatenate(q_rows)
    qo = np.concatenate([[0], np.cumsum(e_l)]).astype(np.int32)
    kvp = np.concatenate([[0], np.cumsum(p_l)]).astype(np.int32)
    got = oracle.extend_attention(np.ascontiguousarray(w.q[rows]), np.ascontiguousarray(w.k_ext[rows]),
                                  np.ascontiguousarray(w.v_ext[rows]), w.k_pool, w.v_pool, qo, kvp,
                                  np.concatenate(kvi), dtype="bf16")
    assert np.array_equal(got, base[rows])


def test_kv_head_expansion_is_exact():
    w = wl.custom(dtype="bf16", prefix_lens=[10, 3], extend_lens=[5, 7], hq=6, hkv=2, lq=32, lv=32)
    base = oracle.extend_attention_workload(w)
    rep = lambda x: np.ascontiguousarray(np.repeat(x, 3, axis=1))
    got = oracle.extend_attention(w.q, rep(w.k_ext), rep(w.v_ext), rep(w.k_pool), rep(w.v_pool),
                                  w.qo_indptr, w.kv_indptr, w.kv_indices, dtype="bf16")
    assert np.array_equal(got, base)


def test_sampled_rows_equal_full_rows():
    w = wl.custom(dtype="bf16", prefix_lens=[10, 3, 0], extend_lens=[5, 7, 2], hq=4, hkv=2, lq=32, lv=32)
    base = oracle.extend_attention_workload(w)
    rows = np.array([13, 0, 6, 5])
    assert np.array_equal(oracle.extend_attention_workload(w, rows=rows), base[rows])


def test_out_of_range_slot_is_an_error():
    w = wl.custom(dtype="fp32", prefix_lens=[3], extend_lens=[1], hq=1, hkv=1, lq=8, lv=8, pool_slots=8)
    w.kv_indices[1] = 8
    with pytest.raises(ValueError):
        oracle.extend_attention_workload(w)


# ----------------------------------------------------------------------------- unified one-stage entry
# (page extend_attention.py, extend_attention_fwd_unified / _fwd_kernel_unified: every key through one
# index array, prefix_lens[b] of them prefix keys)

def _unified_arrays(w):
    """Unified indptr / indices / prefix_lens from the oracle's own index build."""
    indptr, indices, plens = oracle.build_unified_kv_indices(
        w.kv_indptr, w.kv_indices, w.extend_start_loc, w.extend_lens, w.extend_kv_indices, w.bs)
    return indptr, indices[:int(indptr[-1])], plens


def _unified(w, indptr, indices, plens, k_pool=None, v_pool=None):
    return oracle.extend_attention_unified(
        w.q, w.k_pool if k_pool is None else k_pool, w.v_pool if v_pool is None else v_pool,
        w.qo_indptr, indptr, indices, plens, w.sm_scale, w.logit_cap, w.cfg.dtype)


@pytest.mark.parametrize("case", SDPA_CASES, ids=lambda c: f"{c['dtype']}-{c['lq']}x{c['lv']}-h{c['hq']}/{c['hkv']}")
def test_unified_matches_library_attention(case):
    # the pool holds every new token's K/V at its extend slot (the caller's cache
    # store), so the one-index-array path must give the concatenated attention
    w = wl.custom(**case)
    got = _unified(w, *_unified_arrays(w))
    np.testing.assert_allclose(got, sdpa_reference(w), rtol=0, atol=1e-12)


def test_unified_all_prefix_is_full_attention():
    # prefix_lens equal to the whole span: no key is causal, every query sees
    # every key of its sequence (library attention without a mask)
    w = wl.custom(dtype="bf16", prefix_lens=[10, 3], extend_lens=[4, 6], hq=4, hkv=2, lq=64, lv=64)
    indptr, indices, _ = _unified_arrays(w)
    span = np.diff(indptr).astype(np.int32)
    got = _unified(w, indptr, indices, span)
    outs = []
    for b in range(w.bs):
        q0, q1 = w.qo_indptr[b], w.qo_indptr[b + 1]
        slots = indices[indptr[b]:indptr[b + 1]]
        q = _f64(w.q[q0:q1], "bf16").transpose(0, 1)
        k = _f64(w.k_pool[slots], "bf16").transpose(0, 1).repeat_interleave(2, 0)
        v = _f64(w.v_pool[slots], "bf16").transpose(0, 1).repeat_interleave(2, 0)
        outs.append(torch.nn.functional.scaled_dot_product_attention(q, k, v).transpose(0, 1))
    np.testing.assert_allclose(got, torch.cat(outs).numpy(), atol=1e-12)


def test_unified_pool_slot_permutation_is_exact():
    w = wl.custom(dtype="bf16", prefix_lens=[12, 0, 25], extend_lens=[3, 9, 2], hq=4, hkv=2,
                  lq=64, lv=64, pool_slots=80)
    indptr, indices, plens = _unified_arrays(w)
    base = _unified(w, indptr, indices, plens)
    perm = np.random.default_rng(5).permutation(80)
    k2 = np.empty_like(w.k_pool)
    v2 = np.empty_like(w.v_pool)
    k2[perm] = w.k_pool
    v2[perm] = w.v_pool
    assert np.array_equal(_unified(w, indptr, perm[indices], plens, k2, v2), base)


# ----------------------------------------------------------------------------- steps before attention
# (page flashinfer_backend.py: set_kv_buffer of the new tokens in forward_extend, and
# create_flashinfer_kv_indices_triton for the prefix indices)

def test_gather_worked_example():
    with open(os.path.join(GOLDEN, "req_to_token_gather_worked_example.json")) as f:
        ex = json.load(f)
    indptr, idx = oracle.gather_kv_indices(ex["req_to_token"], ex["req_pool_indices"], ex["kv_lens"],
                                           ex["kv_start_idx"])
    assert indptr.tolist() == ex["expected_kv_indptr"]
    assert idx.tolist() == ex["expected_kv_indices"]
    _, idx0 = oracle.gather_kv_indices(ex["req_to_token"], ex["req_pool_indices"], ex["kv_lens"])
    assert idx0.tolist() == ex["expected_kv_indices_without_start"]


@pytest.mark.parametrize("bs,with_start", [(0, False), (1, True), (7, False), (33, True)])
def test_gather_matches_slicing(bs, with_start):
    rng = np.random.default_rng(bs)
    table = rng.integers(0, 1 << 30, size=(40, 300)).astype(np.int32)
    rpi = rng.integers(0, 40, size=bs)
    start = rng.integers(0, 100, size=bs) if with_start else np.zeros(bs, np.int64)
    lens = rng.integers(0, 200, size=bs)
    indptr, idx = oracle.gather_kv_indices(table, rpi, lens, start if with_start else None)
    want = [table[r, s:s + n] for r, s, n in zip(rpi, start, lens)]
    want = np.concatenate(want).astype(np.int64) if bs else np.zeros(0, np.int64)
    assert np.array_equal(idx, want)
    assert indptr.tolist() == [0] + np.cumsum(lens).tolist()


def test_store_matches_fancy_index_assignment():
    rng = np.random.default_rng(7)
    k_ext = rng.integers(0, 1 << 16, size=(13, 3, 64)).astype(np.uint16)
    v_ext = rng.integers(0, 1 << 16, size=(13, 3, 32)).astype(np.uint16)
    k_pool = rng.integers(0, 1 << 16, size=(50, 3, 64)).astype(np.uint16)
    v_pool = rng.integers(0, 1 << 16, size=(50, 3, 32)).astype(np.uint16)
    loc = rng.permutation(50)[:13]
    kp, vp = oracle.store_kv_cache(k_ext, v_ext, k_pool, v_pool, loc)
    want_k, want_v = k_pool.copy(), v_pool.copy()
    want_k[loc] = k_ext
    want_v[loc] = v_ext
    assert np.array_equal(kp, want_k) and np.array_equal(vp, want_v)


def test_store_with_v_inside_k_writes_k_rows():
    rng = np.random.default_rng(8)
    k_ext = rng.standard_normal((5, 1, 48)).astype(np.float32)
    k_pool = rng.standard_normal((20, 1, 48)).astype(np.float32)
    loc = np.array([3, 19, 0, 7, 11])
    kp, vp = oracle.store_kv_cache(k_ext, k_ext[..., :32], k_pool, k_pool[..., :32], loc)
    want = k_pool.copy()
    want[loc] = k_ext
    assert np.array_equal(kp, want) and np.shares_memory(kp, vp) and np.array_equal(vp, want[..., :32])


@pytest.mark.parametrize("case", SDPA_CASES[:3], ids=lambda c: f"{c['dtype']}-{c['lq']}x{c['lv']}")
def test_store_then_unified_attention_is_library_attention(case):
    # overwrite the new tokens' pool rows, store them back, and attend through
    # the unified indices: the library attention over the concatenation
    w = wl.custom(**case)
    junk_k = np.full_like(w.k_pool, 0x7FC0 if w.cfg.dtype == "bf16" else 0)
    kp, vp = w.k_pool.copy(), w.v_pool.copy()
    kp[w.extend_kv_indices] = junk_k[w.extend_kv_indices]
    vp[w.extend_kv_indices] = 0
    kp, vp = oracle.store_kv_cache(w.k_ext, w.v_ext, kp, vp, w.extend_kv_indices)
    got = _unified(w, *_unified_arrays(w), k_pool=kp, v_pool=vp)
    np.testing.assert_allclose(got, sdpa_reference(w), rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- sliding window and sinks
# (page extend_attention.py, _fwd_kernel_unified: SLIDING_WINDOW_SIZE hides keys more than W
# positions before the query; HAS_SINK adds exp(sink - max) to the denominator)

WINDOW_CASE = dict(dtype="bf16", prefix_lens=[30, 0, 9], extend_lens=[12, 20, 5], hq=4, hkv=2, lq=64, lv=64)
BF16_NAN = 0x7FC0


def test_window_wider_than_any_sequence_is_no_window():
    w = wl.custom(**WINDOW_CASE)
    assert np.array_equal(oracle.extend_attention_workload(w, window=10_000), oracle.extend_attention_workload(w))


@pytest.mark.parametrize("window", [1, 3, 17])
def test_window_ignores_every_key_before_it(window):
    # for single rows: poisoning every key more than W positions before the
    # query leaves the row unchanged (and would spoil it without the window)
    w = wl.custom(**WINDOW_CASE)
    for t in (0, 11, 12 + 19, 12 + 20 + 4):
        b = int(np.searchsorted(w.qo_indptr, t, side="right") - 1)
        i = t - int(w.qo_indptr[b])
        P = int(w.kv_indptr[b + 1] - w.kv_indptr[b])
        kp, vp, ke, ve = w.k_pool.copy(), w.v_pool.copy(), w.k_ext.copy(), w.v_ext.copy()
        hidden = range(0, max(0, P + i - window))
        for j in hidden:
            if j < P:
                s = w.kv_indices[w.kv_indptr[b] + j]
                kp[s] = BF16_NAN
                vp[s] = BF16_NAN
            else:
                ke[w.qo_indptr[b] + j - P] = BF16_NAN
                ve[w.qo_indptr[b] + j - P] = BF16_NAN
        base = oracle.extend_attention_workload(w, rows=[t], window=window)
        got = oracle.extend_attention(w.q, ke, ve, kp, vp, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                      dtype="bf16", rows=[t], window=window)
        assert np.array_equal(got, base), t
        if len(hidden):
            plain = oracle.extend_attention(w.q, ke, ve, kp, vp, w.qo_indptr, w.kv_indptr, w.kv_indices,
                                            dtype="bf16", rows=[t])
            assert np.isnan(plain).all()


def _keys_f64(w, b, which):
    """K or V rows of sequence b's keys in order (prefix then new tokens), float64 [P+E, Hkv, L]."""
    pool, ext = (w.k_pool, w.k_ext) if which == "k" else (w.v_pool, w.v_ext)
    p0, p1 = w.kv_indptr[b], w.kv_indptr[b + 1]
    q0, q1 = w.qo_indptr[b], w.qo_indptr[b + 1]
    return np.concatenate([wl.as_f32(pool[w.kv_indices[p0:p1]], w.cfg.dtype),
                           wl.as_f32(ext[q0:q1], w.cfg.dtype)]).astype(np.float64)


@pytest.mark.parametrize("window", [1, 4, 25])
def test_zero_query_with_window_gives_window_mean(window):
    w = wl.custom(**WINDOW_CASE)
    w.q[:] = 0
    got = oracle.extend_attention_workload(w, window=window)
    g = w.cfg.hq // w.cfg.hkv
    for t in range(w.total_q):
        b = int(np.searchsorted(w.qo_indptr, t, side="right") - 1)
        i = t - int(w.qo_indptr[b])
        P = int(w.kv_indptr[b + 1] - w.kv_indptr[b])
        v = _keys_f64(w, b, "v")[max(0, P + i - window):P + i + 1]
        want = v.mean(axis=0).repeat(g, axis=0)  # [Hq, Lv]
        np.testing.assert_allclose(got[t], want, atol=1e-12)


def test_minus_infinite_sink_is_no_sink():
    w = wl.custom(**WINDOW_CASE)
    sinks = np.full(w.cfg.hq, -np.inf, np.float32)
    assert np.array_equal(oracle.extend_attention_workload(w, sinks=sinks), oracle.extend_attention_workload(w))


def test_sink_closed_form_with_zero_query():
    # all logits 0: out = sum_j V_j / (n + e^sink)
    w = wl.custom(**WINDOW_CASE)
    w.q[:] = 0
    sinks = np.array([-1.0, 0.0, 0.5, 3.0], np.float32)
    got = oracle.extend_attention_workload(w, sinks=sinks)
    g = w.cfg.hq // w.cfg.hkv
    for t in range(w.total_q):
        b = int(np.searchsorted(w.qo_indptr, t, side="right") - 1)
        i = t - int(w.qo_indptr[b])
        P = int(w.kv_indptr[b + 1] - w.kv_indptr[b])
        v = _keys_f64(w, b, "v")[:P + i + 1]
        n = P + i + 1
        for h in range(w.cfg.hq):
            want = v[:, h // g].sum(axis=0) / (n + math.exp(float(sinks[h])))
            np.testing.assert_allclose(got[t, h], want, atol=1e-12)


def test_unified_window_and_sinks_match_two_part():
    w = wl.custom(**WINDOW_CASE)
    sinks = np.array([0.3, -2.0, 1.0, 0.0], np.float32)
    for window in (2, 9):
        want = oracle.extend_attention_workload(w, window=window, sinks=sinks)
        indptr, indices, plens = _unified_arrays(w)
        got = oracle.extend_attention_unified(w.q, w.k_pool, w.v_pool, w.qo_indptr, indptr, indices, plens,
                                              dtype="bf16", window=window, sinks=sinks)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- custom mask
# (page extend_attention.py, _fwd_kernel_unified with USE_CUSTOM_MASK: a byte per (query, key)
# replaces the causal rule; sequence b's [E_b, L_b] matrix starts at mask_indptr[b])

def _mask_arrays(w, rule):
    """Byte matrices [E_b, P_b + E_b] from rule(b, i, j) -> bool, concatenated, and their offsets."""
    parts, offs, off = [], [], 0
    for b in range(w.bs):
        E = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
        P = int(w.kv_indptr[b + 1] - w.kv_indptr[b])
        m = np.array([[rule(b, i, j, P) for j in range(P + E)] for i in range(E)], np.uint8).reshape(E, P + E)
        offs.append(off)
        off += m.size
        parts.append(m.ravel())
    offs.append(off)
    return (np.concatenate(parts) if parts else np.zeros(0, np.uint8)), np.array(offs, np.int64)


MASK_CASE = dict(dtype="bf16", prefix_lens=[6, 0, 11], extend_lens=[5, 8, 3], hq=4, hkv=2, lq=32, lv=32)


def test_causal_pattern_mask_is_no_mask():
    w = wl.custom(**MASK_CASE)
    m, mi = _mask_arrays(w, lambda b, i, j, P: j <= P + i)
    assert np.array_equal(oracle.extend_attention_workload(w, custom_mask=m, mask_indptr=mi),
                          oracle.extend_attention_workload(w))


def test_all_ones_mask_is_full_attention():
    w = wl.custom(**MASK_CASE)
    m, mi = _mask_arrays(w, lambda b, i, j, P: True)
    got = oracle.extend_attention_workload(w, custom_mask=m, mask_indptr=mi)
    g = w.cfg.hq // w.cfg.hkv
    outs = []
    for b in range(w.bs):
        q0, q1 = w.qo_indptr[b], w.qo_indptr[b + 1]
        k = torch.from_numpy(_keys_f64(w, b, "k")).transpose(0, 1).repeat_interleave(g, 0)
        v = torch.from_numpy(_keys_f64(w, b, "v")).transpose(0, 1).repeat_interleave(g, 0)
        q = _f64(w.q[q0:q1], "bf16").transpose(0, 1)
        outs.append(torch.nn.functional.scaled_dot_product_attention(q, k, v).transpose(0, 1))
    np.testing.assert_allclose(got, torch.cat(outs).numpy(), atol=1e-12)


def test_zero_query_with_random_mask_gives_masked_mean():
    w = wl.custom(**MASK_CASE)
    w.q[:] = 0
    rng = np.random.default_rng(11)
    bits = {}

    def rule(b, i, j, P):  # a random pattern that keeps each row's own key
        return j == P + i or bits.setdefault((b, i, j), rng.random() < 0.4)
    m, mi = _mask_arrays(w, rule)
    got = oracle.extend_attention_workload(w, custom_mask=m, mask_indptr=mi)
    g = w.cfg.hq // w.cfg.hkv
    for t in range(w.total_q):
        b = int(np.searchsorted(w.qo_indptr, t, side="right") - 1)
        i = t - int(w.qo_indptr[b])
        P = int(w.kv_indptr[b + 1] - w.kv_indptr[b])
        E = int(w.qo_indptr[b + 1] - w.qo_indptr[b])
        row = m[mi[b] + i * (P + E):mi[b] + (i + 1) * (P + E)].astype(bool)
        v = _keys_f64(w, b, "v")[row]
        np.testing.assert_allclose(got[t], v.mean(axis=0).repeat(g, axis=0), atol=1e-12)


def test_unified_custom_mask_matches_two_part():
    w = wl.custom(**MASK_CASE)
    rng = np.random.default_rng(12)
    m, mi = _mask_arrays(w, lambda b, i, j, P: j == P + i or rng.random() < 0.5)
    want = oracle.extend_attention_workload(w, custom_mask=m, mask_indptr=mi, window=4)
    indptr, indices, plens = _unified_arrays(w)
    got = oracle.extend_attention_unified(w.q, w.k_pool, w.v_pool, w.qo_indptr, indptr, indices, plens,
                                          dtype="bf16", custom_mask=m, mask_indptr=mi, window=4)
    np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


# ----------------------------------------------------------------------------- decode
# (page flashinfer_backend.py, forward_decode: one query token per request over
# its pool keys; update_sliding_window keeps the last window + 1 keys)

def _decode(d, **kw):
    return oracle.decode_attention(d.q, d.k_pool, d.v_pool, d.kv_indptr, d.kv_indices, d.sm_scale,
                                   d.logit_cap, d.cfg.dtype, **kw)


def _decode_sdpa(d, keep=None, scale=None):
    """Library attention of each request's query over its gathered keys
    (the last `keep` of them when given)."""
    c = d.cfg
    g = c.hq // c.hkv
    out = np.zeros((d.bs, c.hq, c.lv))
    for b in range(d.bs):
        k0, k1 = int(d.kv_indptr[b]), int(d.kv_indptr[b + 1])
        if keep is not None:
            k0 = max(k0, k1 - keep)
        if k1 == k0:
            continue
        slots = d.kv_indices[k0:k1]
        k = _f64(d.k_pool[slots], c.dtype).transpose(0, 1).repeat_interleave(g, 0)  # [Hq, n, Lq]
        v = _f64(d.v_pool[slots], c.dtype).transpose(0, 1).repeat_interleave(g, 0)
        q = _f64(d.q[b:b + 1], c.dtype).transpose(0, 1)  # [Hq, 1, Lq]
        sc = scale if scale is not None else (c.sm_scale or 1.0 / math.sqrt(c.lq))
        out[b] = torch.nn.functional.scaled_dot_product_attention(q, k, v, scale=sc)[:, 0].numpy()
    return out


DECODE_CASES = [
    dict(key_lens=[37, 1, 200, 64], dtype="bf16", hq=32, hkv=8, lq=128, lv=128),
    dict(key_lens=[5, 90], dtype="fp32", hq=4, hkv=4, lq=64, lv=64, sm_scale=0.2),
    dict(key_lens=[33, 17, 3], dtype="bf16", hq=16, hkv=1, lq=576, lv=512, v_aliases_k=True, std=0.5),
    dict(key_lens=[12, 0, 40], dtype="bf16", hq=6, hkv=2, lq=192, lv=128),
    dict(key_lens=[70], dtype="bf16", hq=8, hkv=2, lq=256, lv=256, sm_scale=-0.05),
]


@pytest.mark.parametrize("case", DECODE_CASES, ids=lambda c: f"{c['dtype']}-{c['lq']}x{c['lv']}-h{c['hq']}/{c['hkv']}")
def test_decode_matches_library_attention(case):
    d = wl.decode_custom(**case)
    np.testing.assert_allclose(_decode(d), _decode_sdpa(d), rtol=0, atol=1e-12)


def test_decode_is_unified_extend_of_one_new_token():
    # a decode step is the unified extend of E = 1 whose prefix is every earlier key
    d = wl.decode_custom([25, 1, 60, 9], hq=8, hkv=2, lq=64, lv=64, logit_cap=3.0)
    sinks = np.array([0.5, -1.0, 2.0, 0.0, 1.5, -3.0, 0.25, 1.0], np.float32)
    qo = np.arange(d.bs + 1, dtype=np.int32)
    plens = (d.key_lens - 1).astype(np.int32)
    for window in (0, 4, 30):
        got = _decode(d, window=window, sinks=sinks)
        want = oracle.extend_attention_unified(d.q, d.k_pool, d.v_pool, qo, d.kv_indptr, d.kv_indices, plens,
                                               d.sm_scale, d.logit_cap, "bf16", window=window, sinks=sinks)
        np.testing.assert_allclose(got, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("window", [1, 7, 63, 500])
def test_decode_window_is_attention_over_the_last_keys(window):
    d = wl.decode_custom([1, 8, 64, 150], hq=4, hkv=2, lq=64, lv=64)
    np.testing.assert_allclose(_decode(d, window=window), _decode_sdpa(d, keep=window + 1), rtol=0, atol=1e-12)


def test_decode_single_key_returns_its_value():
    d = wl.decode_custom([1, 1], dtype="fp32", hq=4, hkv=2, lq=64, lv=48)
    got = _decode(d)
    for b in range(2):
        v = d.v_pool[d.kv_indices[b]].astype(np.float64)  # [Hkv, Lv]
        np.testing.assert_array_equal(got[b], v.repeat(2, axis=0))


def test_decode_request_without_keys_is_zero():
    d = wl.decode_custom([4, 0, 3], hq=4, hkv=2, lq=64, lv=64)
    sinks = np.array([1.0, 0.0, -1.0, 2.0], np.float32)
    for s in (None, sinks):
        got = _decode(d, sinks=s)
        assert np.array_equal(got[1], np.zeros_like(got[1]))
        assert np.isfinite(got).all()


def test_decode_sink_closed_form_with_zero_query():
    # all logits 0: out = sum_j V_j / (n + e^sink)
    d = wl.decode_custom([6, 31], hq=4, hkv=1, lq=64, lv=64)
    d.q[:] = 0
    sinks = np.array([-1.0, 0.0, 0.7, 4.0], np.float32)
    got = _decode(d, sinks=sinks)
    for b in range(d.bs):
        slots = d.kv_indices[d.kv_indptr[b]:d.kv_indptr[b + 1]]
        v = wl.as_f32(d.v_pool[slots], "bf16").astype(np.float64)[:, 0]  # [n, Lv]
        for h in range(4):
            want = v.sum(axis=0) / (len(slots) + math.exp(float(sinks[h])))
            np.testing.assert_allclose(got[b, h], want, atol=1e-12)


def test_decode_selected_requests_equal_full_batch():
    d = wl.decode_custom([9, 14, 2, 30, 5], hq=4, hkv=2, lq=64, lv=64)
    full = _decode(d)
    sel = [3, 0, 4]
    np.testing.assert_array_equal(_decode(d, seqs=sel), full[sel])
