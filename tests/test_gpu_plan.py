"""The device planner's output, read back from the workspace.

The plan (page "flashinfer_backend.py", forward_extend: key ranges cut into
pieces whose states merge_state combines) is checked against what any valid
plan must satisfy, without trusting the kernels that consume it: the chunks of
every item (sequence, KV head, row tile) tile its key range [first, end)
exactly once, in order; the item set is every row tile of every KV head of
every sequence with rows; an item's end tile is the last key its rows see;
split items own a dense, private run of partial slots and one merge record;
empty slots carry b = -1 (nothing else of them is read); no piece of a split item exceeds the chunk limit
or is empty.
Batches cover the planner's LDS arrays and its global-scratch path (more than
2048 sequences or 8192 items), sliding windows, and a forced granularity that
overflows the partial-state budget so that the limit doubles, and forced
one-tile granularity on a batch with fewer tiles than slots.
"""

import math

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import check, out_f64, say

pytestmark = pytest.mark.gpu

HEADER_BYTES = 256       # the plan header: 64 int32
WORK_OFFSET = 256 + 4096  # after the header and the zero row
WORK_INTS = 16           # b, g, t, kt_begin, kt_end, part, merge, pad, q0, E, kvs, P, n_idx, n_keys, pad, pad


def _plan(w, dev, window=0, split=None):
    desc = pkv.make_desc(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"], w.bs,
                         w.num_prefix)
    desc.sliding_window = window
    ws = torch.zeros(pkv.extend_attention_workspace_size(desc), dtype=torch.uint8, device="cuda")
    if split:
        pkv.extend_attention_set_split(*split)
    try:
        pkv.extend_attention_fwd(dev["q"], dev["k_ext"], dev["v_ext"], dev["o"], dev["k_pool"], dev["v_pool"],
                                 dev["qo_indptr"], dev["kv_indptr"], dev["kv_indices"], sm_scale=w.sm_scale,
                                 logit_cap=w.logit_cap, workspace=ws, sliding_window=window)
    finally:
        if split:
            pkv.extend_attention_set_split(0, 0)
    torch.cuda.synchronize()
    hdr = ws[:HEADER_BYTES].view(torch.int32).cpu().numpy()
    num_work = int(hdr[0])
    work = ws[WORK_OFFSET:WORK_OFFSET + 4 * WORK_INTS * num_work].view(torch.int32).cpu().numpy()
    return dict(num_work=num_work, num_merge=int(hdr[1]), chunk=int(hdr[2]), total=int(hdr[3]), items=int(hdr[4]),
                chunks=int(hdr[5]), xcds=int(hdr[6])), work.reshape(num_work, WORK_INTS)


def _expected_items(w, bm, bn, window):
    """(b, g, t) -> (first tile, end tile) for row tile BM and key tile BN."""
    g_ = w.cfg.hq // w.cfg.hkv
    out = {}
    for b in range(w.bs):
        e, p = int(w.extend_lens[b]), int(w.prefix_lens[b])
        for g in range(w.cfg.hkv):
            for t in range(math.ceil(e * g_ / bm)):
                row_hi = min((t + 1) * bm, e * g_) - 1
                first = max(0, p + (t * bm) // g_ - window) // bn if window > 0 else 0
                end = max(first + 1, math.ceil((p + row_hi // g_ + 1) / bn))
                out[(b, g, t)] = (first, end)
    return out


def _check_plan(w, hdr, work, window=0):
    live = work[work[:, 0] >= 0]
    assert len(live) == hdr["chunks"], (len(live), hdr)
    # each record carries its sequence's keys as the index pointers give them (two-part call)
    b = live[:, 0]
    assert (live[:, 8] == w.qo_indptr[b]).all() and (live[:, 9] == w.extend_lens[b]).all()
    assert (live[:, 10] == w.kv_indptr[b]).all() and (live[:, 11] == w.prefix_lens[b]).all()
    assert (live[:, 12] == w.prefix_lens[b]).all()
    assert (live[:, 13] == w.prefix_lens[b] + w.extend_lens[b]).all()
    assert (live[:, 4] > live[:, 3]).all(), "empty chunk"
    groups = {}
    for row in live:
        groups.setdefault((int(row[0]), int(row[1]), int(row[2])), []).append(row)
    assert len(groups) == hdr["items"]
    # the tiling the plan was made for: the one (BM, BN) that predicts every item
    fits = []
    for bm in (64, 128, 256):
        for bn in (16, 32, 64, 128):
            want = _expected_items(w, bm, bn, window)
            if set(want) == set(groups) and all(
                    min(int(r[3]) for r in rows) == want[k][0] and max(int(r[4]) for r in rows) == want[k][1]
                    for k, rows in groups.items()):
                fits.append((bm, bn))
    assert fits, "no row/key tiling explains the planned items"
    tiles = 0
    merges = set()
    parts = []
    for key, rows in groups.items():
        rows = sorted(rows, key=lambda r: int(r[3]))
        for a_, b_ in zip(rows, rows[1:]):
            assert int(a_[4]) == int(b_[3]), f"{key}: chunks do not tile the key range"
        tiles += int(rows[-1][4]) - int(rows[0][3])
        if len(rows) == 1:
            assert int(rows[0][5]) == -1 and int(rows[0][6]) == -1
            continue
        assert all(int(r[4]) - int(r[3]) <= hdr["chunk"] for r in rows), f"{key}: piece above the chunk limit"
        m = {int(r[6]) for r in rows}
        assert len(m) == 1 and m.isdisjoint(merges), f"{key}: merge records {m}"
        merges |= m
        p = [int(r[5]) for r in rows]
        assert p == list(range(p[0], p[0] + len(p))), f"{key}: partial slots {p}"
        parts += p
    assert tiles == hdr["total"] if window == 0 else True
    assert merges == set(range(hdr["num_merge"]))
    assert sorted(parts) == list(range(len(parts))), "partial slots not dense and private"
    return fits


CASES = [
    dict(name="long-prefix-e16", prefix_lens=[16384] * 4, extend_lens=[16] * 4, hq=28, hkv=4),
    dict(name="mixed", prefix_lens=[0, 300, 77, 1000, 5, 4000, 0, 9], extend_lens=[200, 1, 64, 33, 129, 7, 1000, 0],
         hq=32, hkv=8),
    dict(name="skewed", prefix_lens=[0] + [700] * 40, extend_lens=[4096] + [3] * 40, hq=16, hkv=8),
]


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_plan_tiles_every_item(case):
    kw = {k: v for k, v in case.items() if k != "name"}
    w = wl.custom(dtype="bf16", lq=128, lv=128, **kw)
    hdr, work = _plan(w, wl.to_torch(w))
    say(f"plan {case['name']}: {hdr}")
    _check_plan(w, hdr, work)


@pytest.mark.parametrize("n,hq,hkv", [(5000, 4, 2), (1500, 8, 8)], ids=["seqs-past-lds", "items-past-lds"])
def test_plan_global_scratch_path(n, hq, hkv):
    # more sequences (5000 > 2048) or more items (12 000 > 8192) than the
    # planner keeps in LDS: the same code on global arrays; the plan and the
    # attention output both checked
    rng = np.random.default_rng(3)
    lo = 0 if n == 5000 else 1
    w = wl.custom(dtype="bf16", prefix_lens=rng.integers(0, 50, n).tolist(),
                  extend_lens=rng.integers(lo, 4, n).tolist(), hq=hq, hkv=hkv, lq=64, lv=64, seed=29)
    dev = wl.to_torch(w)
    hdr, work = _plan(w, dev)
    say(f"plan bs={n}: {hdr}")
    assert hdr["items"] > (0 if n == 5000 else 8192)
    _check_plan(w, hdr, work)
    check(out_f64(dev), oracle.extend_attention_workload(w), "bf16", f"plan-global-{n}")


def test_plan_window():
    w = wl.custom(dtype="bf16", prefix_lens=[5000, 30, 900], extend_lens=[300, 20, 64], hq=16, hkv=4, lq=128, lv=128,
                  seed=31)
    hdr, work = _plan(w, wl.to_torch(w), window=700)
    say(f"plan window: {hdr}")
    _check_plan(w, hdr, work, window=700)


def test_plan_partial_budget_doubles_the_limit():
    # the forced granularity asks for more partial slots than the budget holds
    w = wl.custom(dtype="bf16", prefix_lens=[65536] * 4, extend_lens=[16] * 4, hq=16, hkv=4, lq=128, lv=128,
                  pool_slots=4 * 65552 + 64, seed=37)
    hdr, work = _plan(w, wl.to_torch(w), split=(16, 1))
    say(f"plan forced fine split: {hdr}")
    assert hdr["chunk"] > 1 and hdr["num_merge"] == 16
    _check_plan(w, hdr, work)


@pytest.mark.parametrize("split", [(1, 1), (2, 1), (16, 1)], ids=["r1", "r2", "r16"])
def test_plan_forced_split_of_a_small_batch(split):
    # fewer KV tiles in all than resident workgroups, with a forced minimum
    # chunk of one tile: items cut into one-tile pieces, none empty (an empty
    # piece has no size class and would corrupt the placement), and the
    # attention output still meets the oracle
    w = wl.custom(dtype="bf16", prefix_lens=[0, 300, 77, 1000, 5], extend_lens=[200, 1, 64, 33, 129], hq=32, hkv=8,
                  lq=128, lv=128)
    dev = wl.to_torch(w)
    hdr, work = _plan(w, dev, split=split)
    say(f"plan small forced {split}: {hdr}")
    assert hdr["total"] < torch.cuda.get_device_properties(0).multi_processor_count * split[0]
    _check_plan(w, hdr, work)
    check(out_f64(dev), oracle.extend_attention_workload(w), "bf16", f"plan-small-{split[0]}")
