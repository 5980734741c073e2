"""Decode attention on the GPU against the CPU oracle.

One query token per request over the request's pool keys (page
"flashinfer_backend.py", forward_decode; the sliding-window index updater
keeps the last window + 1 keys), through decode_attention_fwd.  Inputs are
the seeded decode batches of workloads.py; unused pool slots hold NaN, so a
read outside a request's keys shows up as a non-finite output.
"""

import numpy as np
import pytest
import torch

import oracle
import paged_kv_extend_amd as pkv
import workloads as wl
from gpu_helpers import check, say

pytestmark = pytest.mark.gpu


def run_decode(d, dev=None, window=0, sinks=None, sm_scale=None, logit_cap=None):
    dev = dev or wl.decode_to_torch(d)
    sk = None if sinks is None else torch.from_numpy(np.asarray(sinks, np.float32)).cuda()
    pkv.decode_attention_fwd(dev["q"], dev["o"], dev["k_pool"], dev["v_pool"], dev["kv_indptr"], dev["kv_indices"],
                             sm_scale=d.sm_scale if sm_scale is None else sm_scale,
                             logit_cap=d.logit_cap if logit_cap is None else logit_cap,
                             sliding_window=window, sinks=sk)
    torch.cuda.synchronize()
    return dev


def out_f64(dev):
    return dev["o"].float().cpu().numpy().astype(np.float64)


def oracle_decode(d, window=0, sinks=None, seqs=None):
    return oracle.decode_attention(d.q, d.k_pool, d.v_pool, d.kv_indptr, d.kv_indices, d.sm_scale, d.logit_cap,
                                   d.cfg.dtype, seqs=seqs, window=window, sinks=sinks)


def parity(d, what, window=0, sinks=None):
    c = d.cfg
    say(f"decode {what}: bs={d.bs} keys={d.num_keys} dims={c.lq}/{c.lv} heads={c.hq}/{c.hkv} "
        f"cap={c.logit_cap} window={window} sinks={sinks is not None} v_in_k={c.v_aliases_k}")
    dev = run_decode(d, window=window, sinks=sinks)
    got = out_f64(dev)
    check(got, oracle_decode(d, window=window, sinks=sinks), c.dtype, what)
    return dev, got


# key counts: empty, single key, tile edges, long requests over several chunks,
# many short requests in one chunk
LENS = [0, 1, 15, 16, 17, 63, 64, 65, 300, 1000, 2500] + [3, 9, 40] * 8
SHAPES = [
    dict(hq=4, hkv=2, lq=64, lv=64),
    dict(hq=32, hkv=8, lq=128, lv=128),
    dict(hq=8, hkv=4, lq=256, lv=256),
    dict(hq=6, hkv=2, lq=192, lv=128),
    dict(hq=16, hkv=2, lq=288, lv=256),
    dict(hq=16, hkv=1, lq=576, lv=512, v_aliases_k=True, std=0.5),
    dict(hq=16, hkv=1, lq=576, lv=512, std=0.5),
    dict(hq=32, hkv=1, lq=128, lv=128),   # 32 heads per KV head: two 16-row head blocks
    dict(hq=40, hkv=2, lq=128, lv=128),   # 20 per KV head: a partial second block
    dict(hq=8, hkv=8, lq=128, lv=128),    # MHA
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"{s['lq']}x{s['lv']}-h{s['hq']}/{s['hkv']}"
                         + ("-vk" if s.get("v_aliases_k") else ""))
def test_decode_shapes(shape):
    d = wl.decode_custom(LENS, seed=21, **shape)
    parity(d, "shapes")


@pytest.mark.parametrize("opt", ["cap1", "neg-scale", "window1", "window100", "sinks", "window+sinks+cap"])
def test_decode_options(opt):
    kw = dict(hq=8, hkv=2, lq=128, lv=128)
    window, sinks = 0, None
    if opt == "cap1":
        kw["logit_cap"] = 1.0
    elif opt == "neg-scale":
        kw["sm_scale"] = -0.07
    elif opt == "window1":
        window = 1
    elif opt == "window100":
        window = 100
    elif opt == "sinks":
        sinks = np.linspace(-2.0, 3.0, 8).astype(np.float32)
    else:
        window, kw["logit_cap"] = 37, 5.0
        sinks = np.linspace(1.0, -1.0, 8).astype(np.float32)
    d = wl.decode_custom(LENS, seed=23, **kw)
    parity(d, opt, window=window, sinks=sinks)


def test_decode_mla_window_and_sinks():
    d = wl.decode_custom([0, 700, 5, 2000], hq=16, hkv=1, lq=576, lv=512, v_aliases_k=True, std=0.5, seed=29)
    parity(d, "mla window+sinks", window=250, sinks=np.linspace(-1.0, 1.5, 16).astype(np.float32))


def test_decode_all_requests_empty():
    d = wl.decode_custom([0, 0, 0], hq=8, hkv=2, lq=128, lv=128, pool_slots=64)
    dev = wl.decode_to_torch(d)
    dev["o"].fill_(float("nan"))
    run_decode(d, dev)
    assert torch.count_nonzero(dev["o"]).item() == 0


def test_decode_is_deterministic_and_matches_unified_extend():
    d = wl.decode_custom([4000, 1, 900, 77, 3000], hq=32, hkv=8, lq=128, lv=128, seed=31)
    dev = run_decode(d)
    first = dev["o"].clone()
    run_decode(d, dev)
    assert torch.equal(first, dev["o"]), "decode is not bitwise reproducible"
    # the unified extend path with one new token per request (prefix = every earlier key)
    qo = torch.arange(d.bs + 1, dtype=torch.int32, device="cuda")
    plens = torch.from_numpy((d.key_lens - 1).astype(np.int32)).cuda()
    o2 = torch.empty_like(dev["o"])
    pkv.extend_attention_fwd_unified(dev["q"], o2, dev["k_pool"], dev["v_pool"], qo, dev["kv_indptr"],
                                     dev["kv_indices"], plens)
    torch.cuda.synchronize()
    check(first.float().cpu().numpy().astype(np.float64), o2.float().cpu().numpy().astype(np.float64), "bf16",
          "decode vs unified extend")


@pytest.mark.parametrize("name", list(wl.DECODE_CONFIGS))
def test_decode_full_size(name):
    d = wl.decode_get(name)
    dev = run_decode(d)
    got = out_f64(dev)
    assert np.isfinite(got).all()
    # every request at full size (the oracle finishes these in seconds)
    check(got, oracle_decode(d), "bf16", f"{name} full")


def test_decode_many_requests_and_offset_indptr():
    # more requests than one pass of the plan launch's scan (1024), and an
    # index array that starts past the first entry of kv_indices
    rng = np.random.default_rng(41)
    lens = rng.integers(0, 40, 2500)
    d = wl.decode_custom(lens.tolist(), hq=8, hkv=2, lq=64, lv=64, seed=41)
    want = oracle_decode(d)
    dev = wl.decode_to_torch(d)
    pad = 5
    dev["kv_indices"] = torch.cat([torch.zeros(pad, dtype=torch.int64, device="cuda"), dev["kv_indices"]])
    dev["kv_indptr"] = dev["kv_indptr"] + pad
    pkv.decode_attention_fwd(dev["q"], dev["o"], dev["k_pool"], dev["v_pool"], dev["kv_indptr"],
                             dev["kv_indices"][:].contiguous())
    torch.cuda.synchronize()
    check(out_f64(dev), want, "bf16", "2500 requests, offset indptr")


def test_decode_graph_replay():
    # the decode launches record no memset, so a captured call replays as run
    d = wl.decode_custom([300, 7, 1200, 0, 64], hq=16, hkv=4, lq=128, lv=128, seed=43)
    dev = wl.decode_to_torch(d)
    desc = pkv.make_desc(dev["q"], None, None, dev["o"], dev["k_pool"], dev["v_pool"], d.bs, d.num_keys)
    ws = torch.empty(pkv.decode_attention_workspace_size(desc), dtype=torch.uint8, device="cuda")

    def call():
        pkv.decode_attention_fwd(dev["q"], dev["o"], dev["k_pool"], dev["v_pool"], dev["kv_indptr"],
                                 dev["kv_indices"], workspace=ws)

    call()
    torch.cuda.synchronize()
    eager = dev["o"].clone()
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
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(dev["o"], eager)
        call()  # eager work between the replays
        torch.cuda.synchronize()


def test_decode_widest_window_is_no_window():
    d = wl.decode_custom([5, 300, 0, 2000], hq=8, hkv=2, lq=128, lv=128, seed=47)
    plain = run_decode(d)["o"].clone()
    widest = run_decode(d, window=2**31 - 1)["o"]
    assert torch.equal(plain, widest)


# fp32 batches run as the unified extend of one new token per request
@pytest.mark.parametrize("dims", [64, 128])
@pytest.mark.parametrize("opt", ["plain", "window+sinks+cap"])
def test_decode_fp32(dims, opt):
    kw = dict(hq=8, hkv=2, lq=dims, lv=dims, dtype="fp32")
    window, sinks = 0, None
    if opt != "plain":
        window, kw["logit_cap"] = 37, 5.0
        sinks = np.linspace(1.0, -1.0, 8).astype(np.float32)
    d = wl.decode_custom(LENS, seed=53, **kw)
    dev = wl.decode_to_torch(d)
    dev["o"].fill_(float("nan"))  # rows of keyless requests are written too
    run_decode(d, dev, window=window, sinks=sinks)
    check(out_f64(dev), oracle_decode(d, window=window, sinks=sinks), "fp32", f"fp32 {dims} {opt}")


# bf16 head dims without a decode kernel variant run through the extend route
# too (the plain dims the extend kernels pad to a wider tile)
@pytest.mark.parametrize("dims", [80, 96, 160])
def test_decode_plain_dims_through_extend(dims):
    d = wl.decode_custom(LENS, seed=59, hq=8, hkv=2, lq=dims, lv=dims)
    dev = wl.decode_to_torch(d)
    dev["o"].fill_(float("nan"))
    run_decode(d, dev)
    check(out_f64(dev), oracle_decode(d), "bf16", f"bf16 {dims} via extend")
