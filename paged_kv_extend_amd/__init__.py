"""Python binding of libpkv.so: paged-KV extend attention for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/pkv.h.  PyTorch supplies device
memory and the current stream.  Importing works without a GPU; calling
requires the built library (``python -m paged_kv_extend_amd._build``) and
raises if it is missing -- there is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional, Tuple

import torch

__all__ = ["build_unified_kv_indices", "extend_attention_fwd", "extend_attention_fwd_unified",
           "extend_attention_workspace_size", "extend_attention_fwd_noalloc", "decode_attention_fwd", "decode_attention_workspace_size", "store_kv_cache", "gather_kv_indices",
           "extend_attention_kernel_name", "extend_attention_prefer_kernel", "extend_attention_set_split",
           "make_desc", "profile_enable", "profile_read", "last_error", "version", "library", "debug_library",
           "LIB_PATH", "LIB_DEBUG_PATH", "PkvError"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv.so")
# the same kernels with every index array checked on the device first (PKV_ERR_RANGE); one host sync per call
LIB_DEBUG_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpkv_debug.so")

PKV_BF16 = 0
PKV_FP32 = 1


class PkvError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"pkv error {code}: {msg}")
        self.code = code


class AttnDesc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in ("dtype", "bs", "num_q_heads", "num_kv_heads", "lq", "lv")] + \
               [(n, ctypes.c_int64) for n in (
                   "total_q_tokens", "num_prefix_indices", "pool_slots",
                   "q_stride_tok", "q_stride_head", "o_stride_tok", "o_stride_head",
                   "ke_stride_tok", "ke_stride_head", "ve_stride_tok", "ve_stride_head",
                   "kp_stride_slot", "kp_stride_head", "vp_stride_slot", "vp_stride_head")] + \
               [("sliding_window", ctypes.c_int32), ("pad0", ctypes.c_int32), ("sinks", ctypes.c_void_p),
                ("custom_mask", ctypes.c_void_p), ("mask_indptr", ctypes.c_void_p)]


_lib = None
_lib_debug = None


def library() -> ctypes.CDLL:
    """Load libpkv.so (raises if it has not been built)."""
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


def debug_library() -> ctypes.CDLL:
    """Load libpkv_debug.so: the same C ABI, which also checks every index array against
    the sizes passed (returning PKV_ERR_RANGE, -6) before any kernel reads it."""
    global _lib_debug
    if _lib_debug is None:
        _lib_debug = _load(LIB_DEBUG_PATH)
    return _lib_debug


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with `python -m paged_kv_extend_amd._build`")
    lib = ctypes.CDLL(path)
    P, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.build_unified_kv_indices.argtypes = [P, P, P, P, P, i32, i64, i64, P, P, i64, P, P]
    lib.build_unified_kv_indices.restype = ctypes.c_int
    lib.extend_attention_workspace_size.argtypes = [ctypes.POINTER(AttnDesc)]
    lib.extend_attention_workspace_size.restype = ctypes.c_size_t
    lib.extend_attention_fwd.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float,
                                         ctypes.POINTER(AttnDesc), P, ctypes.c_size_t, P]
    lib.extend_attention_fwd.restype = ctypes.c_int
    lib.extend_attention_fwd_unified.argtypes = [P, P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float,
                                                 ctypes.POINTER(AttnDesc), P, ctypes.c_size_t, P]
    lib.extend_attention_fwd_unified.restype = ctypes.c_int
    lib.extend_attention_fwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, ctypes.c_float, ctypes.c_float,
                                                 ctypes.POINTER(AttnDesc), P]
    lib.extend_attention_fwd_noalloc.restype = ctypes.c_int
    lib.extend_attention_noalloc_scratch_bytes.restype = ctypes.c_size_t
    lib.decode_attention_workspace_size.argtypes = [ctypes.POINTER(AttnDesc)]
    lib.decode_attention_workspace_size.restype = ctypes.c_size_t
    lib.decode_attention_fwd.argtypes = [P, P, P, P, P, P, ctypes.c_float, ctypes.c_float,
                                         ctypes.POINTER(AttnDesc), P, ctypes.c_size_t, P]
    lib.decode_attention_fwd.restype = ctypes.c_int
    lib.store_kv_cache.argtypes = [P, P, P, P, P, ctypes.POINTER(AttnDesc), P]
    lib.store_kv_cache.restype = ctypes.c_int
    lib.gather_kv_indices.argtypes = [P, i64, P, P, P, i32, P, P, i64, P]
    lib.gather_kv_indices.restype = ctypes.c_int
    lib.pkv_profile_enable.argtypes = [ctypes.c_int]
    lib.pkv_profile_enable.restype = ctypes.c_int
    lib.pkv_profile_read.argtypes = [ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]
    lib.pkv_profile_read.restype = ctypes.c_int
    lib.extend_attention_kernel_name.argtypes = [ctypes.POINTER(AttnDesc), P, P, P, P]
    lib.extend_attention_kernel_name.restype = ctypes.c_char_p
    lib.extend_attention_prefer_kernel.argtypes = [ctypes.c_char_p]
    lib.extend_attention_prefer_kernel.restype = ctypes.c_int
    lib.extend_attention_set_split.argtypes = [ctypes.c_int, ctypes.c_int]
    lib.extend_attention_set_split.restype = ctypes.c_int
    lib.pkv_last_error.restype = ctypes.c_char_p
    lib.pkv_version.restype = ctypes.c_char_p
    return lib


def profile_enable(on: bool = True) -> None:
    """Record HIP events around every later attention kernel (measurement only)."""
    _check(library().pkv_profile_enable(1 if on else 0))


def profile_read() -> Tuple[float, int]:
    """(summed attention-kernel milliseconds, number of calls) since profile_enable(True)."""
    ms, n = ctypes.c_double(), ctypes.c_int64()
    _check(library().pkv_profile_read(ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value


def last_error() -> str:
    return library().pkv_last_error().decode()


def version() -> str:
    return library().pkv_version().decode()


def _check(rc: int):
    if rc != 0:
        raise PkvError(rc, last_error())


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _want(t: torch.Tensor, name: str, dtype: torch.dtype):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")


def build_unified_kv_indices(prefix_kv_indptr: torch.Tensor, prefix_kv_indices: torch.Tensor,
                             extend_start_loc: torch.Tensor, extend_seq_lens: torch.Tensor,
                             extend_kv_indices: torch.Tensor, bs: int,
                             out: Optional[Tuple[torch.Tensor, torch.Tensor, torch.Tensor]] = None):
    """Unified KV indices: (unified_kv_indptr int32[bs+1], unified_kv_indices int64[n_p+n_e],
    prefix_lens int32[bs]).  Entries of unified_kv_indices past unified_kv_indptr[bs] are
    left unwritten (as torch.empty leaves them)."""
    for t, n, d in ((prefix_kv_indptr, "prefix_kv_indptr", torch.int32),
                    (prefix_kv_indices, "prefix_kv_indices", torch.int64),
                    (extend_start_loc, "extend_start_loc", torch.int32),
                    (extend_seq_lens, "extend_seq_lens", torch.int32),
                    (extend_kv_indices, "extend_kv_indices", torch.int64)):
        _want(t, n, d)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    dev = prefix_kv_indptr.device
    cap = prefix_kv_indices.numel() + extend_kv_indices.numel()
    if out is None:
        indptr = torch.empty(bs + 1, dtype=torch.int32, device=dev)
        indices = torch.empty(cap, dtype=torch.int64, device=dev)
        plens = torch.empty(bs, dtype=torch.int32, device=dev)
    else:
        indptr, indices, plens = out
    rc = library().build_unified_kv_indices(
        _ptr(prefix_kv_indptr), _ptr(prefix_kv_indices), _ptr(extend_start_loc), _ptr(extend_seq_lens),
        _ptr(extend_kv_indices), int(bs), prefix_kv_indices.numel(), extend_kv_indices.numel(),
        _ptr(indptr), _ptr(indices), indices.numel(), _ptr(plens) if plens is not None else None,
        _stream(dev))
    _check(rc)
    return indptr, indices, plens


def make_desc(q_extend, k_extend, v_extend, o, k_pool, v_pool, bs: int,
              num_prefix_indices: int) -> AttnDesc:
    """Descriptor of a call; k_extend / v_extend are None for a unified call."""
    if q_extend.dtype == torch.bfloat16:
        dt = PKV_BF16
    elif q_extend.dtype == torch.float32:
        dt = PKV_FP32
    else:
        raise ValueError(f"unsupported dtype {q_extend.dtype}")
    for t, n in ((q_extend, "q_extend"), (k_extend, "k_extend"), (v_extend, "v_extend"), (o, "o"),
                 (k_pool, "k_pool"), (v_pool, "v_pool")):
        if t is None and n in ("k_extend", "v_extend"):
            continue
        _want(t, n, q_extend.dtype)
        if t.dim() != 3 or (t.numel() > 0 and t.stride(2) != 1):
            raise ValueError(f"{n} must be 3-D with a contiguous last dimension")
    def st(t):  # strides of an empty tensor carry no meaning; report contiguous ones
        if t is None:
            return 0, 0
        return (t.stride(0), t.stride(1)) if t.numel() > 0 else (t.shape[1] * t.shape[2], t.shape[2])

    d = AttnDesc()
    d.dtype = dt
    d.bs = bs
    d.num_q_heads, d.lq = q_extend.shape[1], q_extend.shape[2]
    d.num_kv_heads, d.lv = k_pool.shape[1], v_pool.shape[2]
    d.total_q_tokens = q_extend.shape[0]
    d.num_prefix_indices = num_prefix_indices
    d.pool_slots = k_pool.shape[0]
    d.q_stride_tok, d.q_stride_head = st(q_extend)
    d.o_stride_tok, d.o_stride_head = st(o)
    d.ke_stride_tok, d.ke_stride_head = st(k_extend)
    d.ve_stride_tok, d.ve_stride_head = st(v_extend)
    d.kp_stride_slot, d.kp_stride_head = st(k_pool)
    d.vp_stride_slot, d.vp_stride_head = st(v_pool)
    return d


def _options(desc: AttnDesc, q_extend: torch.Tensor, sliding_window: int, sinks: Optional[torch.Tensor],
             custom_mask: Optional[torch.Tensor] = None, mask_indptr: Optional[torch.Tensor] = None) -> None:
    desc.sliding_window = int(sliding_window) if sliding_window and sliding_window > 0 else 0
    if sinks is not None:
        _want(sinks, "sinks", torch.float32)
        if sinks.shape != (q_extend.shape[1],) or not sinks.is_contiguous():
            raise ValueError("sinks must be a contiguous float32 [num_q_heads] tensor")
        desc.sinks = sinks.data_ptr()
    if custom_mask is not None:
        _want(custom_mask, "custom_mask", torch.uint8)
        if mask_indptr is None:
            raise ValueError("custom_mask needs mask_indptr")
        _want(mask_indptr, "mask_indptr", torch.int64)
        desc.custom_mask = custom_mask.data_ptr()
        desc.mask_indptr = mask_indptr.data_ptr()


def extend_attention_workspace_size(desc: AttnDesc) -> int:
    n = library().extend_attention_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise PkvError(-1, last_error())
    return int(n)


def extend_attention_kernel_name(desc: AttnDesc, k_extend=None, v_extend=None, k_pool=None,
                                 v_pool=None) -> str:
    """Symbol name of the attention kernel serving ``desc`` with these K/V tensors
    (for profiler output; V sharing K's storage selects a variant)."""
    n = library().extend_attention_kernel_name(ctypes.byref(desc), _ptr(k_extend), _ptr(v_extend), _ptr(k_pool),
                                               _ptr(v_pool))
    if n is None:
        raise PkvError(-1, last_error())
    return n.decode()


def extend_attention_prefer_kernel(name: str) -> None:
    """Process-wide kernel preference: "auto", "dl" or "attn" (tests, benchmarks)."""
    _check(library().extend_attention_prefer_kernel(name.encode()))


def extend_attention_set_split(rounds: int = 0, min_chunk_tiles: int = 0) -> None:
    """Process-wide split granularity (tests, benchmarks): items longer than 1/rounds of the
    average work per resident workgroup are cut into key chunks of at least min_chunk_tiles
    tiles, merged afterwards; 0 keeps a default."""
    _check(library().extend_attention_set_split(int(rounds), int(min_chunk_tiles)))


_ws_cache = {}


def _workspace(device: torch.device, stream: int, nbytes: int) -> torch.Tensor:
    key = (device.index, stream)
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _ws_cache[key] = ws
    return ws


def extend_attention_fwd(q_extend: torch.Tensor, k_extend: torch.Tensor, v_extend: torch.Tensor,
                         o: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                         qo_indptr: torch.Tensor, kv_indptr: torch.Tensor, kv_indices: torch.Tensor,
                         sm_scale: Optional[float] = None, logit_cap: float = 0.0,
                         workspace: Optional[torch.Tensor] = None, sliding_window: int = 0,
                         sinks: Optional[torch.Tensor] = None, custom_mask: Optional[torch.Tensor] = None,
                         mask_indptr: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Extend attention into ``o`` (see include/pkv.h for the exact semantics).

    kv_indptr / kv_indices describe the cached prefix only; the new tokens'
    K/V rows are addressed by qo_indptr.  sm_scale None or 0 means 1/sqrt(lq).
    sliding_window > 0, sinks (float32 [num_q_heads] logits) and custom_mask
    (uint8 bytes, sequence b's [E_b, P_b + E_b] matrix at the int64
    mask_indptr[b]) are the options of the unified kernel on the SGLang page.
    """
    _want(qo_indptr, "qo_indptr", torch.int32)
    _want(kv_indptr, "kv_indptr", torch.int32)
    _want(kv_indices, "kv_indices", torch.int64)
    bs = qo_indptr.numel() - 1
    desc = make_desc(q_extend, k_extend, v_extend, o, k_pool, v_pool, bs, kv_indices.numel())
    _options(desc, q_extend, sliding_window, sinks, custom_mask, mask_indptr)
    dev = q_extend.device
    stream = _stream(dev)
    nbytes = extend_attention_workspace_size(desc)
    if workspace is None:
        workspace = _workspace(dev, stream, nbytes)
    rc = library().extend_attention_fwd(
        _ptr(q_extend), _ptr(k_extend), _ptr(v_extend), _ptr(o), _ptr(k_pool), _ptr(v_pool),
        _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices),
        float(sm_scale or 0.0), float(logit_cap), ctypes.byref(desc),
        _ptr(workspace), workspace.numel() * workspace.element_size(), stream)
    _check(rc)
    return o


def extend_attention_fwd_noalloc(q_extend: torch.Tensor, k_extend: torch.Tensor, v_extend: torch.Tensor,
                                 o: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                                 qo_indptr: torch.Tensor, kv_indptr: torch.Tensor, kv_indices: torch.Tensor,
                                 sm_scale: Optional[float] = None, logit_cap: float = 0.0) -> torch.Tensor:
    """extend_attention_fwd without a workspace: the library keeps the plan and the
    partial states in a scratch array of its own per device (no allocation in the
    call; calls that overlap on one device race).  See include/pkv.h."""
    _want(qo_indptr, "qo_indptr", torch.int32)
    _want(kv_indptr, "kv_indptr", torch.int32)
    _want(kv_indices, "kv_indices", torch.int64)
    bs = qo_indptr.numel() - 1
    desc = make_desc(q_extend, k_extend, v_extend, o, k_pool, v_pool, bs, kv_indices.numel())
    rc = library().extend_attention_fwd_noalloc(
        _ptr(q_extend), _ptr(k_extend), _ptr(v_extend), _ptr(o), _ptr(k_pool), _ptr(v_pool),
        _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices), float(sm_scale or 0.0), float(logit_cap),
        ctypes.byref(desc), _stream(q_extend.device))
    _check(rc)
    return o


def store_kv_cache(k_extend: torch.Tensor, v_extend: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                   out_cache_loc: torch.Tensor) -> None:
    """Store the new tokens' K/V rows into the pool at out_cache_loc (int64)."""
    _want(out_cache_loc, "out_cache_loc", torch.int64)
    # the descriptor of the call, with the new tokens' K standing in for q / o (not read)
    desc = make_desc(k_extend, k_extend, v_extend, k_extend, k_pool, v_pool, 1, 0)
    desc.total_q_tokens = out_cache_loc.numel()
    _check(library().store_kv_cache(_ptr(k_extend), _ptr(v_extend), _ptr(k_pool), _ptr(v_pool),
                                    _ptr(out_cache_loc), ctypes.byref(desc), _stream(k_pool.device)))


def gather_kv_indices(req_to_token: torch.Tensor, req_pool_indices: torch.Tensor, kv_lens: torch.Tensor,
                      kv_start_idx: Optional[torch.Tensor] = None, capacity: Optional[int] = None,
                      out: Optional[Tuple[torch.Tensor, torch.Tensor]] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """Prefix indices of a batch from the request-to-token table: (kv_indptr int32, kv_indices int64).

    capacity (the length of kv_indices, at least the sum of kv_lens) comes from
    the caller, or from ``out`` when it is given: the binding never reads the
    device, so the call stays free of host syncs and can be captured."""
    _want(req_to_token, "req_to_token", torch.int32)
    _want(req_pool_indices, "req_pool_indices", torch.int64)
    _want(kv_lens, "kv_lens", torch.int32)
    if kv_start_idx is not None:
        _want(kv_start_idx, "kv_start_idx", torch.int32)
    if req_to_token.dim() != 2 or req_to_token.stride(1) != 1:
        raise ValueError("req_to_token must be 2-D with contiguous rows")
    bs = kv_lens.numel()
    dev = req_to_token.device
    if capacity is None:
        if out is None:
            raise ValueError("gather_kv_indices needs capacity (or out): the sum of kv_lens is not read "
                             "from the device")
        capacity = out[1].numel()
    if out is None:
        out = (torch.empty(bs + 1, dtype=torch.int32, device=dev),
               torch.empty(max(capacity, 1), dtype=torch.int64, device=dev))
    indptr, indices = out
    _check(library().gather_kv_indices(_ptr(req_to_token), req_to_token.stride(0), _ptr(req_pool_indices),
                                       _ptr(kv_lens), _ptr(kv_start_idx) if kv_start_idx is not None else None,
                                       bs, _ptr(indptr), _ptr(indices), capacity, _stream(dev)))
    return indptr, indices[:capacity]


def extend_attention_fwd_unified(q_extend: torch.Tensor, o: torch.Tensor, k_pool: torch.Tensor,
                                 v_pool: torch.Tensor, qo_indptr: torch.Tensor, kv_indptr: torch.Tensor,
                                 kv_indices: torch.Tensor, prefix_lens: torch.Tensor,
                                 sm_scale: Optional[float] = None, logit_cap: float = 0.0,
                                 workspace: Optional[torch.Tensor] = None, sliding_window: int = 0,
                                 sinks: Optional[torch.Tensor] = None, custom_mask: Optional[torch.Tensor] = None,
                                 mask_indptr: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Unified one-stage extend attention into ``o``: every key through the
    unified kv_indptr / kv_indices (as build_unified_kv_indices returns them),
    prefix_lens[b] of sequence b's keys prefix keys (see include/pkv.h)."""
    _want(qo_indptr, "qo_indptr", torch.int32)
    _want(kv_indptr, "kv_indptr", torch.int32)
    _want(kv_indices, "kv_indices", torch.int64)
    _want(prefix_lens, "prefix_lens", torch.int32)
    bs = qo_indptr.numel() - 1
    desc = make_desc(q_extend, None, None, o, k_pool, v_pool, bs, kv_indices.numel())
    _options(desc, q_extend, sliding_window, sinks, custom_mask, mask_indptr)
    dev = q_extend.device
    stream = _stream(dev)
    nbytes = extend_attention_workspace_size(desc)
    if workspace is None:
        workspace = _workspace(dev, stream, nbytes)
    rc = library().extend_attention_fwd_unified(
        _ptr(q_extend), _ptr(o), _ptr(k_pool), _ptr(v_pool), _ptr(qo_indptr), _ptr(kv_indptr),
        _ptr(kv_indices), _ptr(prefix_lens), float(sm_scale or 0.0), float(logit_cap), ctypes.byref(desc),
        _ptr(workspace), workspace.numel() * workspace.element_size(), stream)
    _check(rc)
    return o


def decode_attention_workspace_size(desc: AttnDesc) -> int:
    n = library().decode_attention_workspace_size(ctypes.byref(desc))
    if n == 0:
        raise PkvError(-1, last_error())
    return int(n)


def decode_attention_fwd(q: torch.Tensor, o: torch.Tensor, k_pool: torch.Tensor, v_pool: torch.Tensor,
                         kv_indptr: torch.Tensor, kv_indices: torch.Tensor, sm_scale: Optional[float] = None,
                         logit_cap: float = 0.0, workspace: Optional[torch.Tensor] = None, sliding_window: int = 0,
                         sinks: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode attention into ``o`` ([bs, num_q_heads, lv]): the query row q[b]
    attends to request b's keys kv_indices[kv_indptr[b]:kv_indptr[b+1]] (the
    last sliding_window + 1 of them with a window); see include/pkv.h."""
    _want(kv_indptr, "kv_indptr", torch.int32)
    _want(kv_indices, "kv_indices", torch.int64)
    bs = kv_indptr.numel() - 1
    if q.dim() != 3 or q.shape[0] != bs or o.dim() != 3 or o.shape[0] != bs:
        raise ValueError("q and o must be [bs, num_q_heads, dim] with bs = len(kv_indptr) - 1")
    desc = make_desc(q, None, None, o, k_pool, v_pool, bs, kv_indices.numel())
    _options(desc, q, sliding_window, sinks)
    dev = q.device
    stream = _stream(dev)
    nbytes = decode_attention_workspace_size(desc)
    if workspace is None:
        workspace = _workspace(dev, stream, nbytes)
    rc = library().decode_attention_fwd(
        _ptr(q), _ptr(o), _ptr(k_pool), _ptr(v_pool), _ptr(kv_indptr), _ptr(kv_indices),
        float(sm_scale or 0.0), float(logit_cap), ctypes.byref(desc),
        _ptr(workspace), workspace.numel() * workspace.element_size(), stream)
    _check(rc)
    return o
