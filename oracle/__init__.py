"""CPU oracle for paged-KV extend attention -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP library
(``paged_kv_extend_amd``) and never imports it.

``liboracle.so`` (``oracle.c``) holds plain C loops with double accumulation
for the unified index build and for extend attention, parallel over output
rows with OpenMP; this module is its ctypes wrapper.

Definitions follow the SGLang page "extend_attention.py" (functions
build_unified_kv_indices, _copy_unified_indices_kernel, _fwd_kernel_unified,
redundant_attention) and the page "flashinfer_backend.py" (forward_extend,
call_begin_forward; forward_decode and the decode index updater).  Parity is pinned in tests/test_oracle_pins.py.
"""

from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def build_lib(force: bool = True) -> str:
    """Compile liboracle.so with gcc (OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + f".tmp{os.getpid()}"
        cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
            build_lib(force=True)
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        i32, i64, f64 = ctypes.c_int32, ctypes.c_int64, ctypes.c_double
        lib.oracle_build_unified_kv_indices.argtypes = [P, P, P, P, P, i32, P, P, P]
        lib.oracle_build_unified_kv_indices.restype = ctypes.c_int
        lib.oracle_extend_attention.argtypes = (
            [i32] + [P, i64, i64] * 5 + [i64, P, P, P, i32, i32, i32, i32, i32, f64, f64, P, i64, P, i32, i32, P, P, P])
        lib.oracle_extend_attention.restype = ctypes.c_int
        lib.oracle_extend_attention_unified.argtypes = (
            [i32] + [P, i64, i64] * 3 + [i64, P, P, P, P, i32, i32, i32, i32, i32, f64, f64, P, i64, P, i32, i32, P, P, P])
        lib.oracle_extend_attention_unified.restype = ctypes.c_int
        lib.oracle_decode_attention.argtypes = (
            [i32] + [P, i64, i64] * 3 + [i64, P, P, i32, i32, i32, i32, i32, f64, f64, P, i32, P, i32, i32, P])
        lib.oracle_decode_attention.restype = ctypes.c_int
        lib.oracle_store_kv_cache.argtypes = [i32, i64, i32, i32, i32] + [P, i64, i64] * 4 + [i64, P]
        lib.oracle_store_kv_cache.restype = ctypes.c_int
        lib.oracle_gather_kv_indices.argtypes = [P, i64, P, P, P, i32, P, P]
        lib.oracle_gather_kv_indices.restype = ctypes.c_int
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def _ptr(a: np.ndarray) -> int:
    return a.__array_interface__["data"][0]


def max_threads() -> int:
    return int(_load().oracle_max_threads())


def build_unified_kv_indices(prefix_kv_indptr, prefix_kv_indices, extend_start_loc,
                             extend_seq_lens, extend_kv_indices, bs):
    """Returns (unified_kv_indptr int32[bs+1], unified_kv_indices int64[n_p+n_e], prefix_lens)."""
    lib = _load()
    a = [np.ascontiguousarray(prefix_kv_indptr, np.int32),
         np.ascontiguousarray(prefix_kv_indices, np.int64),
         np.ascontiguousarray(extend_start_loc, np.int32),
         np.ascontiguousarray(extend_seq_lens, np.int32),
         np.ascontiguousarray(extend_kv_indices, np.int64)]
    indptr = np.zeros(bs + 1, np.int32)
    cap = len(a[1]) + len(a[4])
    indices = np.full(max(cap, 1), -1, np.int64)
    plens = np.zeros(max(bs, 1), np.int32)
    rc = lib.oracle_build_unified_kv_indices(*[_ptr(x) for x in a], int(bs), _ptr(indptr),
                                             _ptr(indices), _ptr(plens))
    if rc != 0:
        raise ValueError(f"oracle index build failed: {rc}")
    return indptr, indices[:cap], plens[:bs]


def _strides(a: np.ndarray):
    it = a.itemsize
    assert a.ndim == 3 and a.strides[2] == it, "last dim must be contiguous"
    return a.strides[0] // it, a.strides[1] // it


def _sinks(sinks, hq):
    if sinks is None:
        return None
    a = np.ascontiguousarray(sinks, np.float32)
    assert a.shape == (hq,), a.shape
    return a


def _mask(custom_mask, mask_indptr):
    if custom_mask is None:
        return None, None
    m = np.ascontiguousarray(custom_mask, np.uint8)
    mi = np.ascontiguousarray(mask_indptr, np.int64)
    return (m if m.size else np.zeros(1, np.uint8)), mi


def extend_attention(q, k_ext, v_ext, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices,
                     sm_scale=0.0, logit_cap=0.0, dtype="bf16", rows=None, num_threads=0, window=0, sinks=None,
                     custom_mask=None, mask_indptr=None):
    """Exact (double) extend attention for the given extend-token rows
    (window > 0: sliding window; sinks: float32 [Hq] sink logits or None;
    custom_mask: uint8 bytes, sequence b's [E_b, P_b + E_b] matrix at
    mask_indptr[b], replacing the causal rule).

    Arrays: bf16 tensors as uint16 bit patterns, fp32 tensors as float32,
    shapes [tokens|slots, heads, dim] with a contiguous last dim.  Returns
    float64 [len(rows) or T, Hq, Lv].
    """
    lib = _load()
    dt = 0 if dtype == "bf16" else 1
    want = np.uint16 if dt == 0 else np.float32
    for x in (q, k_ext, v_ext, k_pool, v_pool):
        assert x.dtype == want, (x.dtype, want)
    qo = np.ascontiguousarray(qo_indptr, np.int32)
    kvp = np.ascontiguousarray(kv_indptr, np.int32)
    kvi = np.ascontiguousarray(kv_indices, np.int64)
    if kvi.size == 0:
        kvi = np.zeros(1, np.int64)
    bs = len(qo) - 1
    hq, lq = q.shape[1], q.shape[2]
    hkv, lv = k_pool.shape[1], v_pool.shape[2]
    total = int(qo[-1]) if bs > 0 else 0
    if rows is None:
        rows_arr, n = None, total
    else:
        rows_arr = np.ascontiguousarray(rows, np.int64)
        n = len(rows_arr)
    out = np.zeros((max(n, 1), hq, lv), np.float64)
    args = [dt]
    for x in (q, k_ext, v_ext, k_pool, v_pool):
        s0, s1 = _strides(x)
        args += [_ptr(x) if x.size else 0, s0, s1]
    args += [k_pool.shape[0], _ptr(qo), _ptr(kvp), _ptr(kvi), bs, hq, hkv, lq, lv,
             float(sm_scale), float(logit_cap),
             _ptr(rows_arr) if rows_arr is not None else None, n, _ptr(out), int(num_threads)]
    sk = _sinks(sinks, hq)
    cm, mi = _mask(custom_mask, mask_indptr)
    args += [int(window), _ptr(sk) if sk is not None else None, _ptr(cm) if cm is not None else None,
             _ptr(mi) if mi is not None else None]
    rc = lib.oracle_extend_attention(*args)
    if rc != 0:
        raise ValueError(f"oracle attention failed: {rc}")
    return out[:n]


def extend_attention_unified(q, k_pool, v_pool, qo_indptr, kv_indptr, kv_indices, prefix_lens,
                             sm_scale=0.0, logit_cap=0.0, dtype="bf16", rows=None, num_threads=0, window=0,
                             sinks=None, custom_mask=None, mask_indptr=None):
    """Exact (double) unified one-stage extend attention: every key through
    kv_indices (the unified index array), prefix_lens[b] of them prefix keys.
    Same array conventions and return value as extend_attention."""
    lib = _load()
    dt = 0 if dtype == "bf16" else 1
    want = np.uint16 if dt == 0 else np.float32
    for x in (q, k_pool, v_pool):
        assert x.dtype == want, (x.dtype, want)
    qo = np.ascontiguousarray(qo_indptr, np.int32)
    kvp = np.ascontiguousarray(kv_indptr, np.int32)
    kvi = np.ascontiguousarray(kv_indices, np.int64)
    pl = np.ascontiguousarray(prefix_lens, np.int32)
    if kvi.size == 0:
        kvi = np.zeros(1, np.int64)
    if pl.size == 0:
        pl = np.zeros(1, np.int32)
    bs = len(qo) - 1
    hq, lq = q.shape[1], q.shape[2]
    hkv, lv = k_pool.shape[1], v_pool.shape[2]
    total = int(qo[-1]) if bs > 0 else 0
    if rows is None:
        rows_arr, n = None, total
    else:
        rows_arr = np.ascontiguousarray(rows, np.int64)
        n = len(rows_arr)
    out = np.zeros((max(n, 1), hq, lv), np.float64)
    args = [dt]
    for x in (q, k_pool, v_pool):
        s0, s1 = _strides(x)
        args += [_ptr(x) if x.size else 0, s0, s1]
    args += [k_pool.shape[0], _ptr(qo), _ptr(kvp), _ptr(kvi), _ptr(pl), bs, hq, hkv, lq, lv,
             float(sm_scale), float(logit_cap),
             _ptr(rows_arr) if rows_arr is not None else None, n, _ptr(out), int(num_threads)]
    sk = _sinks(sinks, hq)
    cm, mi = _mask(custom_mask, mask_indptr)
    args += [int(window), _ptr(sk) if sk is not None else None, _ptr(cm) if cm is not None else None,
             _ptr(mi) if mi is not None else None]
    rc = lib.oracle_extend_attention_unified(*args)
    if rc != 0:
        raise ValueError(f"oracle unified attention failed: {rc}")
    return out[:n]


def decode_attention(q, k_pool, v_pool, kv_indptr, kv_indices, sm_scale=0.0, logit_cap=0.0, dtype="bf16",
                     seqs=None, num_threads=0, window=0, sinks=None):
    """Exact (double) decode attention: row b of q ([bs, hq, lq]) attends to
    every key of request b through kv_indices (the last window + 1 of them
    with a sliding window).  Returns float64 [len(seqs) or bs, hq, lv]."""
    lib = _load()
    dt = 0 if dtype == "bf16" else 1
    want = np.uint16 if dt == 0 else np.float32
    for x in (q, k_pool, v_pool):
        assert x.dtype == want, (x.dtype, want)
    kvp = np.ascontiguousarray(kv_indptr, np.int32)
    kvi = np.ascontiguousarray(kv_indices, np.int64)
    if kvi.size == 0:
        kvi = np.zeros(1, np.int64)
    bs = len(kvp) - 1
    hq, lq = q.shape[1], q.shape[2]
    hkv, lv = k_pool.shape[1], v_pool.shape[2]
    seq_arr = None if seqs is None else np.ascontiguousarray(seqs, np.int32)
    n = bs if seq_arr is None else len(seq_arr)
    out = np.zeros((max(n, 1), hq, lv), np.float64)
    args = [dt]
    for x in (q, k_pool, v_pool):
        s0, s1 = _strides(x)
        args += [_ptr(x) if x.size else 0, s0, s1]
    sk = _sinks(sinks, hq)
    args += [k_pool.shape[0], _ptr(kvp), _ptr(kvi), bs, hq, hkv, lq, lv, float(sm_scale), float(logit_cap),
             _ptr(seq_arr) if seq_arr is not None and n else None, n, _ptr(out), int(num_threads), int(window),
             _ptr(sk) if sk is not None else None]
    rc = lib.oracle_decode_attention(*args)
    if rc != 0:
        raise ValueError(f"oracle decode attention failed: {rc}")
    return out[:n]


def store_kv_cache(k_ext, v_ext, k_pool, v_pool, out_cache_loc):
    """KV-cache store into copies of the pools: returns (k_pool', v_pool').

    Arrays [tokens|slots, heads, dim] with a contiguous last dim, bf16 as
    uint16 bit patterns or float32.  When v_pool is a view into k_pool (V the
    first lv columns of K), pass k_pool for both and v_ext a view of k_ext:
    the copies then alias the same way."""
    lib = _load()
    kp = np.array(k_pool, copy=True)
    alias = v_pool is k_pool or (isinstance(v_pool, np.ndarray) and np.shares_memory(v_pool, k_pool))
    vp = kp[..., :v_pool.shape[2]] if alias else np.array(v_pool, copy=True)
    loc = np.ascontiguousarray(out_cache_loc, np.int64)
    if loc.size == 0:
        loc = np.zeros(1, np.int64)
    n = len(np.asarray(out_cache_loc))
    args = [k_ext.itemsize, n, k_pool.shape[1], k_ext.shape[2], v_ext.shape[2]]
    for x in (k_ext, v_ext, kp, vp):
        s0, s1 = _strides(x)
        args += [_ptr(x) if x.size else 0, s0, s1]
    args += [kp.shape[0], _ptr(loc)]
    rc = lib.oracle_store_kv_cache(*args)
    if rc != 0:
        raise ValueError(f"oracle store failed: {rc}")
    return kp, vp


def gather_kv_indices(req_to_token, req_pool_indices, kv_lens, kv_start_idx=None):
    """Prefix index gather: returns (kv_indptr int32 [bs+1], kv_indices int64)."""
    lib = _load()
    r2t = np.ascontiguousarray(req_to_token, np.int32)
    rpi = np.ascontiguousarray(req_pool_indices, np.int64)
    lens = np.ascontiguousarray(kv_lens, np.int32)
    bs = len(lens)
    start = None if kv_start_idx is None else np.ascontiguousarray(kv_start_idx, np.int32)
    indptr = np.zeros(bs + 1, np.int32)
    out = np.zeros(max(1, int(lens.sum()) if bs else 0), np.int64)
    rc = lib.oracle_gather_kv_indices(_ptr(r2t), r2t.shape[1], _ptr(rpi) if bs else None, _ptr(lens) if bs else None,
                                      _ptr(start) if start is not None else None, bs, _ptr(indptr), _ptr(out))
    if rc != 0:
        raise ValueError(f"oracle gather failed: {rc}")
    return indptr, out[:int(indptr[-1])]


def extend_attention_workload(w, rows=None, num_threads=0, window=0, sinks=None, custom_mask=None,
                              mask_indptr=None):
    """Convenience: run the oracle on a workloads.Workload-like object."""
    return extend_attention(w.q, w.k_ext, w.v_ext, w.k_pool, w.v_pool, w.qo_indptr,
                            w.kv_indptr, w.kv_indices, w.sm_scale, w.logit_cap,
                            w.cfg.dtype, rows=rows, num_threads=num_threads, window=window, sinks=sinks,
                            custom_mask=custom_mask, mask_indptr=mask_indptr)
