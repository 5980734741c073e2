"""Seeded synthetic inputs for paged-KV extend attention.

This module only draws inputs: lengths, pool slots and tensor values.  It
holds none of the attention arithmetic, so both the CPU oracle (``oracle/``)
and the HIP path (``paged_kv_extend_amd``) consume its output without
sharing any computation.

Layout of one batch (all arrays are numpy; bf16 tensors are ``uint16`` bit
patterns, fp32 tensors are ``float32``):

* ``qo_indptr``  int32 [bs+1]   extend-token offsets (exclusive scan of E_b)
* ``kv_indptr``  int32 [bs+1]   prefix-index offsets (exclusive scan of P_b)
* ``kv_indices`` int64 [sum P]  pool slots of the cached prefix tokens
* ``extend_kv_indices`` int64 [sum E]  pool slots the new tokens are stored at
* ``extend_start_loc`` int32 [bs]  start of each sequence in extend_kv_indices
* ``q``      [T, Hq, Lq]        T = sum E
* ``k_ext``  [T, Hkv, Lq]
* ``v_ext``  [T, Hkv, Lv]       (a view of k_ext[..., :Lv] when V aliases K)
* ``k_pool`` [slots, Hkv, Lq]
* ``v_pool`` [slots, Hkv, Lv]   (a view of k_pool[..., :Lv] when V aliases K)

Pool rows that no sequence references hold NaN, so a stray gather shows up
as a NaN output.  The new tokens' K/V are also written into the pool at their
``extend_kv_indices`` slots, which is what the caller's KV-cache store does
before the unified (single index list) formulation reads them.

Draw recipe for a config with seed s: ``numpy.random.default_rng(s)``; draw
prefix lengths, then extend lengths, then one permutation of all pool slots
(prefix slots take its first sum(P) entries in batch order, extend slots the
next sum(E)), then q, k_ext, v_ext, prefix K, prefix V, each
``standard_normal(float32) * std``; bf16 configs round each value to the
nearest bf16 (ties to even).  Integer ranges U[a, b] include both ends.
"""

from __future__ import annotations

import dataclasses
import math
from typing import Callable, Optional, Sequence

import numpy as np

BF16_NAN = np.uint16(0x7FC0)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (round to nearest, ties to even)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    dtype: str  # "bf16" or "fp32"
    bs: int
    hq: int
    hkv: int
    lq: int
    lv: int
    pool_slots: int
    std: float
    sm_scale: float  # 0 means the default 1/sqrt(lq)
    logit_cap: float  # <= 0 disables the cap
    seed: int
    prefix_lens: Callable[[np.random.Generator, int], np.ndarray]
    extend_lens: Callable[[np.random.Generator, int], np.ndarray]
    v_aliases_k: bool = False
    description: str = ""


def _fixed(values: Sequence[int]):
    arr = np.asarray(values, dtype=np.int64)
    return lambda rng, bs: arr.copy()


def _uniform(lo: int, hi: int):
    return lambda rng, bs: rng.integers(lo, hi, size=bs, endpoint=True)


def _skewed_prefix(rng, bs):
    # one long causal sequence first, the rest with geometric prefixes (mean 1024)
    p = rng.geometric(1.0 / 1024.0, size=bs)
    p[0] = 0
    return p


def _skewed_extend(rng, bs):
    e = rng.integers(1, 64, size=bs, endpoint=True)
    e[0] = 8192
    return e


# The five benchmark workloads.  Seeds are 1000 + k for workload k.
CONFIGS = {
    "tiny_fp32": Config(
        "tiny_fp32", "fp32", bs=2, hq=4, hkv=2, lq=64, lv=64, pool_slots=64, std=1.0,
        sm_scale=1.0 / 8.0, logit_cap=0.0, seed=1001,
        prefix_lens=_fixed([16, 0]), extend_lens=_fixed([8, 12]),
        description="bs 2, 4/2 heads, D 64, P [16,0], E [8,12], 64-slot pool, fp32"),
    "llama8b": Config(
        "llama8b", "bf16", bs=16, hq=32, hkv=8, lq=128, lv=128, pool_slots=65536, std=1.0,
        sm_scale=1.0 / math.sqrt(128.0), logit_cap=0.0, seed=1002,
        prefix_lens=_uniform(0, 2048), extend_lens=_uniform(1, 512),
        description="Llama-3-8B-shaped: bs 16, 32/8 heads, D 128, P~U[0,2048], E~U[1,512]"),
    "long_prefix": Config(
        "long_prefix", "bf16", bs=4, hq=28, hkv=4, lq=128, lv=128, pool_slots=131072, std=1.0,
        sm_scale=0.0, logit_cap=0.0, seed=1003,
        prefix_lens=_fixed([16384] * 4), extend_lens=_fixed([1024] * 4),
        description="long prefix: bs 4, 28/4 heads, D 128, P 16384, E 1024"),
    "mla": Config(
        "mla", "bf16", bs=8, hq=128, hkv=1, lq=576, lv=512, pool_slots=65536, std=0.5,
        sm_scale=0.0, logit_cap=0.0, seed=1004,
        prefix_lens=_uniform(512, 4096), extend_lens=_fixed([256] * 8), v_aliases_k=True,
        description="MLA-shaped: bs 8, 128/1 heads, Lq 576 (512+64), Lv 512 = K[:, :512], P~U[512,4096], E 256"),
    "skewed_cap": Config(
        "skewed_cap", "bf16", bs=64, hq=16, hkv=8, lq=256, lv=256, pool_slots=262144, std=1.0,
        sm_scale=0.0, logit_cap=50.0, seed=1005,
        prefix_lens=_skewed_prefix, extend_lens=_skewed_extend,
        description="skewed: 64 seqs, 16/8 heads, D 256, seq0 P 0 E 8192, others P~Geom(mean 1024) E~U[1,64], cap 50"),
}

CONFIG_ORDER = ["tiny_fp32", "llama8b", "long_prefix", "mla", "skewed_cap"]

# Auxiliary: the long-prefix batch with 16 new tokens per sequence, the shape
# where extend attention is bound by HBM rather than by the products
# (~111 flop per algorithmic byte against the MI355X ridge of ~312).
CONFIGS["long_prefix_e16"] = Config(
    "long_prefix_e16", "bf16", bs=4, hq=28, hkv=4, lq=128, lv=128, pool_slots=131072, std=1.0,
    sm_scale=0.0, logit_cap=0.0, seed=1006,
    prefix_lens=_fixed([16384] * 4), extend_lens=_fixed([16] * 4),
    description="long prefix, short extend (HBM-bound): bs 4, 28/4 heads, D 128, P 16384, E 16")
AUX_CONFIGS = ["long_prefix_e16"]


@dataclasses.dataclass
class Workload:
    cfg: Config
    prefix_lens: np.ndarray
    extend_lens: np.ndarray
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    extend_kv_indices: np.ndarray
    extend_start_loc: np.ndarray
    q: np.ndarray
    k_ext: np.ndarray
    v_ext: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray

    @property
    def bs(self) -> int:
        return int(self.prefix_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.extend_lens.sum())

    @property
    def num_prefix(self) -> int:
        return int(self.prefix_lens.sum())

    @property
    def sm_scale(self) -> float:
        return self.cfg.sm_scale

    @property
    def logit_cap(self) -> float:
        return self.cfg.logit_cap

    def causal_flops(self) -> float:
        """Visible (query, key) pairs times 2*(Lq+Lv) per q head."""
        e = self.extend_lens.astype(np.float64)
        p = self.prefix_lens.astype(np.float64)
        pairs = float((e * p + e * (e + 1) / 2).sum())
        return pairs * self.cfg.hq * 2.0 * (self.cfg.lq + self.cfg.lv)

    def algorithmic_bytes(self) -> float:
        """Q read + O write + every K/V row read once + int64 prefix indices."""
        c = self.cfg
        s = 4 if c.dtype == "fp32" else 2
        t = float(self.total_q)
        rows = float(self.num_prefix + self.total_q)
        lv_kv = 0 if c.v_aliases_k else c.lv
        return (t * c.hq * (c.lq + c.lv) * s + rows * c.hkv * (c.lq + lv_kv) * s
                + 8.0 * self.num_prefix)


def _draw(rng, shape, std, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    return x


def build(cfg: Config, prefix_lens: Optional[np.ndarray] = None,
          extend_lens: Optional[np.ndarray] = None, rng: Optional[np.random.Generator] = None,
          poison_unused: bool = True) -> Workload:
    """Draw one batch for ``cfg`` (lengths may be overridden for test shapes)."""
    if rng is None:
        rng = np.random.default_rng(cfg.seed)
    p = cfg.prefix_lens(rng, cfg.bs) if prefix_lens is None else np.asarray(prefix_lens)
    e = cfg.extend_lens(rng, cfg.bs) if extend_lens is None else np.asarray(extend_lens)
    p = p.astype(np.int64)
    e = e.astype(np.int64)
    bs = p.shape[0]
    assert e.shape[0] == bs
    n_p, n_e = int(p.sum()), int(e.sum())
    if n_p + n_e > cfg.pool_slots:
        raise ValueError(f"{cfg.name}: {n_p}+{n_e} tokens do not fit {cfg.pool_slots} slots")
    perm = rng.permutation(cfg.pool_slots).astype(np.int64)
    kv_indices = perm[:n_p].copy()
    extend_kv_indices = perm[n_p:n_p + n_e].copy()

    qo_indptr = np.zeros(bs + 1, np.int32)
    qo_indptr[1:] = np.cumsum(e)
    kv_indptr = np.zeros(bs + 1, np.int32)
    kv_indptr[1:] = np.cumsum(p)
    extend_start_loc = qo_indptr[:-1].copy()

    dt = cfg.dtype
    q = _draw(rng, (n_e, cfg.hq, cfg.lq), cfg.std, dt)
    k_ext = _draw(rng, (n_e, cfg.hkv, cfg.lq), cfg.std, dt)
    v_ext = k_ext[..., :cfg.lv] if cfg.v_aliases_k else _draw(rng, (n_e, cfg.hkv, cfg.lv), cfg.std, dt)
    k_pref = _draw(rng, (n_p, cfg.hkv, cfg.lq), cfg.std, dt)
    v_pref = None if cfg.v_aliases_k else _draw(rng, (n_p, cfg.hkv, cfg.lv), cfg.std, dt)

    np_dtype = np.uint16 if dt == "bf16" else np.float32
    fill = BF16_NAN if dt == "bf16" else np.float32(np.nan)
    if not poison_unused:
        fill = np_dtype(0)
    k_pool = np.full((cfg.pool_slots, cfg.hkv, cfg.lq), fill, dtype=np_dtype)
    k_pool[kv_indices] = k_pref
    k_pool[extend_kv_indices] = k_ext
    if cfg.v_aliases_k:
        v_pool = k_pool[..., :cfg.lv]
    else:
        v_pool = np.full((cfg.pool_slots, cfg.hkv, cfg.lv), fill, dtype=np_dtype)
        v_pool[kv_indices] = v_pref
        v_pool[extend_kv_indices] = v_ext
    return Workload(cfg, p.astype(np.int32), e.astype(np.int32), qo_indptr, kv_indptr,
                    kv_indices, extend_kv_indices, extend_start_loc, q, k_ext, v_ext,
                    k_pool, v_pool)


def custom(name="custom", dtype="bf16", prefix_lens=(16,), extend_lens=(8,), hq=4, hkv=2,
           lq=64, lv=64, pool_slots=None, std=1.0, sm_scale=0.0, logit_cap=0.0, seed=7,
           v_aliases_k=False, poison_unused=True) -> Workload:
    """A test-shape batch with explicit lengths."""
    p = np.asarray(prefix_lens, np.int64)
    e = np.asarray(extend_lens, np.int64)
    if pool_slots is None:
        pool_slots = int(p.sum() + e.sum()) + 37
    cfg = Config(name, dtype, bs=len(p), hq=hq, hkv=hkv, lq=lq, lv=lv, pool_slots=pool_slots,
                 std=std, sm_scale=sm_scale, logit_cap=logit_cap, seed=seed,
                 prefix_lens=_fixed(p), extend_lens=_fixed(e), v_aliases_k=v_aliases_k)
    return build(cfg, poison_unused=poison_unused)


def get(name: str, **kw) -> Workload:
    return build(CONFIGS[name], **kw)


def as_f32(x: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float32 view of a workload tensor (bf16 bits are widened)."""
    return bf16_bits_to_f32(x) if dtype == "bf16" else np.asarray(x, np.float32)


def index_case(rng: np.random.Generator, bs: int, max_p: int = 300, max_e: int = 300,
               extra_tail: int = 0, indptr_base: int = 0):
    """Random inputs for the unified-index build (no pool or tensors)."""
    p = rng.integers(0, max_p, size=bs, endpoint=True) if bs else np.zeros(0, np.int64)
    e = rng.integers(0, max_e, size=bs, endpoint=True) if bs else np.zeros(0, np.int64)
    prefix_kv_indptr = np.zeros(bs + 1, np.int32)
    prefix_kv_indptr[1:] = np.cumsum(p)
    prefix_kv_indptr += indptr_base
    n_p = int(prefix_kv_indptr[-1]) + extra_tail
    prefix_kv_indices = rng.integers(0, 1 << 40, size=n_p).astype(np.int64)
    # extend starts: an exclusive scan, shuffled gaps allowed by placing sequences apart
    gaps = rng.integers(0, 3, size=bs) if bs else np.zeros(0, np.int64)
    extend_start_loc = np.zeros(bs + extra_tail, np.int32)
    pos = 0
    for b in range(bs):
        pos += int(gaps[b])
        extend_start_loc[b] = pos
        pos += int(e[b])
    n_e = pos + extra_tail
    extend_kv_indices = rng.integers(0, 1 << 40, size=n_e).astype(np.int64)
    extend_seq_lens = np.concatenate([e, rng.integers(0, 9, size=extra_tail)]).astype(np.int32)
    return dict(prefix_kv_indptr=prefix_kv_indptr, prefix_kv_indices=prefix_kv_indices,
                extend_start_loc=extend_start_loc, extend_seq_lens=extend_seq_lens,
                extend_kv_indices=extend_kv_indices, bs=bs)


# ----------------------------------------------------------------------------- decode batches
# One query token per request over its pool keys (the new token's K/V already
# stored).  Seeds are 1100 + k.

@dataclasses.dataclass
class DecodeConfig:
    name: str
    dtype: str
    bs: int
    hq: int
    hkv: int
    lq: int
    lv: int
    std: float
    sm_scale: float
    logit_cap: float
    seed: int
    key_lens: Callable[[np.random.Generator, int], np.ndarray]
    v_aliases_k: bool = False
    description: str = ""


DECODE_CONFIGS = {
    "decode_llama8b": DecodeConfig(
        "decode_llama8b", "bf16", bs=64, hq=32, hkv=8, lq=128, lv=128, std=1.0, sm_scale=0.0, logit_cap=0.0,
        seed=1101, key_lens=_uniform(2048, 6144),
        description="Llama-3-8B-shaped decode: bs 64, 32/8 heads, D 128, keys~U[2048,6144]"),
    "decode_long": DecodeConfig(
        "decode_long", "bf16", bs=8, hq=32, hkv=8, lq=128, lv=128, std=1.0, sm_scale=0.0, logit_cap=0.0,
        seed=1102, key_lens=_fixed([32768] * 8),
        description="long-context decode: bs 8, 32/8 heads, D 128, 32768 keys each"),
    "decode_mla": DecodeConfig(
        "decode_mla", "bf16", bs=32, hq=16, hkv=1, lq=576, lv=512, std=0.5, sm_scale=0.0, logit_cap=0.0,
        seed=1103, key_lens=_uniform(1024, 8192), v_aliases_k=True,
        description="MLA-shaped decode: bs 32, 16/1 heads, Lq 576, Lv 512 = K[:, :512], keys~U[1024,8192]"),
}


@dataclasses.dataclass
class DecodeBatch:
    cfg: DecodeConfig
    key_lens: np.ndarray   # int32 [bs]
    kv_indptr: np.ndarray  # int32 [bs + 1]
    kv_indices: np.ndarray  # int64, distinct pool slots
    q: np.ndarray          # [bs, hq, lq]
    k_pool: np.ndarray     # [pool_slots, hkv, lq]; unused slots hold NaN
    v_pool: np.ndarray     # [pool_slots, hkv, lv] (a view into k_pool when V lies inside K)

    @property
    def bs(self) -> int:
        return int(self.key_lens.shape[0])

    @property
    def num_keys(self) -> int:
        return int(self.kv_indptr[-1])

    @property
    def sm_scale(self) -> float:
        return self.cfg.sm_scale

    @property
    def logit_cap(self) -> float:
        return self.cfg.logit_cap

    def algorithmic_bytes(self) -> float:
        """Bytes a decode pass must move: every key's K (and V unless inside K)
        row per KV head, its slot index, the queries and the outputs."""
        c = self.cfg
        el = 2 if c.dtype == "bf16" else 4
        row = c.lq + (0 if c.v_aliases_k else c.lv)
        return float(self.num_keys * (c.hkv * row * el + 8) + self.bs * c.hq * (c.lq + c.lv) * el)


def decode_batch(cfg: DecodeConfig, key_lens: Optional[Sequence[int]] = None, pool_slots: Optional[int] = None,
                 rng: Optional[np.random.Generator] = None) -> DecodeBatch:
    """Draw one decode batch for cfg (key lengths may be overridden)."""
    if rng is None:
        rng = np.random.default_rng(cfg.seed)
    n = cfg.key_lens(rng, cfg.bs) if key_lens is None else np.asarray(key_lens, np.int64)
    n = n.astype(np.int64)
    bs = n.shape[0]
    total = int(n.sum())
    slots = pool_slots if pool_slots is not None else total + 37
    if total > slots:
        raise ValueError(f"{cfg.name}: {total} keys do not fit {slots} slots")
    kv_indices = rng.permutation(slots)[:total].astype(np.int64)
    kv_indptr = np.zeros(bs + 1, np.int32)
    kv_indptr[1:] = np.cumsum(n)
    dt = cfg.dtype
    q = _draw(rng, (bs, cfg.hq, cfg.lq), cfg.std, dt)
    np_dtype = np.uint16 if dt == "bf16" else np.float32
    fill = BF16_NAN if dt == "bf16" else np.float32(np.nan)
    k_pool = np.full((slots, cfg.hkv, cfg.lq), fill, dtype=np_dtype)
    k_pool[kv_indices] = _draw(rng, (total, cfg.hkv, cfg.lq), cfg.std, dt)
    if cfg.v_aliases_k:
        v_pool = k_pool[..., :cfg.lv]
    else:
        v_pool = np.full((slots, cfg.hkv, cfg.lv), fill, dtype=np_dtype)
        v_pool[kv_indices] = _draw(rng, (total, cfg.hkv, cfg.lv), cfg.std, dt)
    return DecodeBatch(cfg, n.astype(np.int32), kv_indptr, kv_indices, q, k_pool, v_pool)


def decode_custom(key_lens=(16,), dtype="bf16", hq=4, hkv=2, lq=64, lv=64, std=1.0, sm_scale=0.0, logit_cap=0.0,
                  seed=11, v_aliases_k=False, pool_slots=None) -> DecodeBatch:
    """A test-shape decode batch with explicit key counts."""
    n = np.asarray(key_lens, np.int64)
    cfg = DecodeConfig("decode_custom", dtype, bs=len(n), hq=hq, hkv=hkv, lq=lq, lv=lv, std=std,
                       sm_scale=sm_scale, logit_cap=logit_cap, seed=seed, key_lens=_fixed(n),
                       v_aliases_k=v_aliases_k)
    return decode_batch(cfg, pool_slots=pool_slots)


def decode_get(name: str, **kw) -> DecodeBatch:
    return decode_batch(DECODE_CONFIGS[name], **kw)


def decode_to_torch(d: DecodeBatch, device="cuda"):
    """Device tensors of a decode batch (bf16 bit patterns become torch.bfloat16)."""
    import torch

    def t(x):
        a = torch.from_numpy(np.ascontiguousarray(x))
        if d.cfg.dtype == "bf16":
            a = a.view(torch.bfloat16)
        return a.to(device)

    c = d.cfg
    out = dict(q=t(d.q), k_pool=t(d.k_pool))
    out["v_pool"] = out["k_pool"][..., :c.lv] if c.v_aliases_k else t(d.v_pool)
    out["kv_indptr"] = torch.from_numpy(d.kv_indptr.astype(np.int32)).to(device)
    out["kv_indices"] = torch.from_numpy(d.kv_indices.astype(np.int64)).to(device)
    out["o"] = torch.empty((d.bs, c.hq, c.lv), dtype=out["q"].dtype, device=device)
    return out


def to_torch(w: Workload, device="cuda"):
    """Device tensors of a workload (bf16 bit patterns become torch.bfloat16)."""
    import torch

    def t(x):
        a = torch.from_numpy(np.ascontiguousarray(x))
        if w.cfg.dtype == "bf16":
            a = a.view(torch.bfloat16)
        return a.to(device)

    def i(x, dt):
        return torch.from_numpy(np.ascontiguousarray(x).astype(dt)).to(device)

    c = w.cfg
    out = dict(q=t(w.q), k_ext=t(w.k_ext), k_pool=t(w.k_pool))
    if c.v_aliases_k:
        out["v_ext"] = out["k_ext"][..., :c.lv]
        out["v_pool"] = out["k_pool"][..., :c.lv]
    else:
        out["v_ext"] = t(w.v_ext)
        out["v_pool"] = t(w.v_pool)
    out["qo_indptr"] = i(w.qo_indptr, np.int32)
    out["kv_indptr"] = i(w.kv_indptr, np.int32)
    out["kv_indices"] = i(w.kv_indices, np.int64)
    out["extend_kv_indices"] = i(w.extend_kv_indices, np.int64)
    out["extend_start_loc"] = i(w.extend_start_loc, np.int32)
    out["extend_seq_lens"] = i(w.extend_lens, np.int32)
    tdt = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    out["o"] = torch.full((w.total_q, c.hq, c.lv), float("nan"), dtype=tdt, device=device)
    return out
