"""Host-side checks of the C ABI that need no GPU: the library loads, exports
every entry point include/pkv.h declares, sizes workspaces, and rejects bad
arguments before touching the device."""

import ctypes
import os
import re

import pytest

import paged_kv_extend_amd as pkv

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "pkv.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b([A-Za-z_]\w*)\s*\(", text, flags=re.M)))


def test_exports_every_declared_function():
    names = header_functions()
    assert {"build_unified_kv_indices", "extend_attention_fwd", "extend_attention_workspace_size",
            "pkv_last_error", "pkv_version"} <= set(names)
    lib = pkv.library()
    for n in names:
        assert hasattr(lib, n), n
    assert "gfx950" in pkv.version()


def test_debug_library_exports_the_same_functions():
    names = header_functions()
    lib = pkv.debug_library()
    for n in names:
        assert hasattr(lib, n), n
    assert "debug" in lib.pkv_version().decode() and "debug" not in pkv.version()
    # host-side checks are the same: a bad descriptor fails before any device work
    d = desc(num_kv_heads=7)
    assert lib.extend_attention_fwd(4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 0.0, 0.0,
                                    ctypes.byref(d), 4096, 1 << 30, None) == -1


def kernel_name(d, k_ext=4096, v_ext=8192, k_pool=12288, v_pool=16384):
    lib = pkv.library()
    n = lib.extend_attention_kernel_name(ctypes.byref(d), k_ext, v_ext, k_pool, v_pool)
    return None if n is None else n.decode()


def test_kernel_name_per_variant():
    assert kernel_name(desc()) == "attn_dl_kernel"
    assert kernel_name(desc(lq=64, lv=64)) == "attn_dl_kernel"
    mla = desc(lq=576, lv=512, num_kv_heads=1, q_stride_head=576, q_stride_tok=32 * 576, ke_stride_tok=576,
               ke_stride_head=576, kp_stride_slot=576, kp_stride_head=576, o_stride_tok=32 * 512,
               o_stride_head=512, ve_stride_tok=576, ve_stride_head=576, vp_stride_slot=576, vp_stride_head=576)
    # V stored apart from K: the register-staged kernel; V inside K: the direct-load kernel
    assert kernel_name(mla) == "attn_kernel"
    assert kernel_name(mla, 4096, 4096, 12288, 12288) == "attn_dl_kernel"
    assert kernel_name(desc(dtype=1, lq=64, lv=64)) == "attn_kernel"
    # plain head dims between the tile widths run in a wider tile of the direct-load kernel
    for dim in (80, 96, 112, 160, 192):
        assert kernel_name(desc(lq=dim, lv=dim)) == "attn_dl_kernel", dim
    assert kernel_name(desc(lq=72, lv=72)) is None
    assert kernel_name(desc(lq=80, lv=64)) is None
    assert kernel_name(desc(dtype=1, lq=96, lv=96)) is None


def test_kernel_preference():
    try:
        pkv.extend_attention_prefer_kernel("attn")
        assert kernel_name(desc()) == "attn_kernel"
        # a preferred kernel that does not serve the shape is passed over
        assert kernel_name(desc(lq=96, lv=96)) == "attn_dl_kernel"
        pkv.extend_attention_prefer_kernel("dl")
        assert kernel_name(desc(dtype=1, lq=64, lv=64)) == "attn_kernel"
        for gone in ("fastest", "r64"):
            with pytest.raises(pkv.PkvError):
                pkv.extend_attention_prefer_kernel(gone)
    finally:
        pkv.extend_attention_prefer_kernel("auto")
    assert kernel_name(desc()) == "attn_dl_kernel"


def test_split_setting_is_checked():
    for bad in ((-1, 0), (65, 0), (0, -2), (0, 1 << 21)):
        with pytest.raises(pkv.PkvError):
            pkv.extend_attention_set_split(*bad)
    pkv.extend_attention_set_split(4, 1)
    pkv.extend_attention_set_split(0, 0)


def test_workspace_covers_every_kernel():
    lib = pkv.library()
    d = desc()
    sizes = []
    try:
        for k in ("auto", "dl", "attn"):
            pkv.extend_attention_prefer_kernel(k)
            sizes.append(lib.extend_attention_workspace_size(ctypes.byref(d)))
    finally:
        pkv.extend_attention_prefer_kernel("auto")
    assert len(set(sizes)) == 1 and sizes[0] > 0


def desc(**kw):
    d = pkv.AttnDesc()
    base = dict(dtype=0, bs=2, num_q_heads=32, num_kv_heads=8, lq=128, lv=128, total_q_tokens=100,
                num_prefix_indices=50, pool_slots=1000, q_stride_tok=32 * 128, q_stride_head=128,
                o_stride_tok=32 * 128, o_stride_head=128, ke_stride_tok=8 * 128, ke_stride_head=128,
                ve_stride_tok=8 * 128, ve_stride_head=128, kp_stride_slot=8 * 128, kp_stride_head=128,
                vp_stride_slot=8 * 128, vp_stride_head=128)
    base.update(kw)
    for k, v in base.items():
        setattr(d, k, v)
    return d


def test_workspace_size_valid_and_grows():
    small = pkv.extend_attention_workspace_size(desc())
    big = pkv.extend_attention_workspace_size(desc(total_q_tokens=100000, bs=64))
    assert 0 < small < big
    assert small % 256 == 0


@pytest.mark.parametrize("kw,needle", [
    (dict(num_q_heads=30), "multiple"),
    (dict(lq=72, lv=72), "not supported"),
    (dict(lq=96, lv=80), "not supported"),
    (dict(dtype=1, lq=96, lv=96), "not supported"),
    (dict(dtype=5), "dtype"),
    (dict(bs=-1), "bs"),
    (dict(q_stride_head=100), "stride"),
    (dict(total_q_tokens=-3), "negative"),
    (dict(dtype=1, lq=576, lv=512), "not supported"),
])
def test_workspace_size_rejects(kw, needle):
    lib = pkv.library()
    assert lib.extend_attention_workspace_size(ctypes.byref(desc(**kw))) == 0
    assert needle in pkv.last_error()


def call_fwd(d, ws_bytes=1 << 30, ptr=4096, ws=4096):
    lib = pkv.library()
    return lib.extend_attention_fwd(ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, ptr, 0.0, 0.0,
                                    ctypes.byref(d) if d is not None else None, ws, ws_bytes, None)


def test_noalloc_rejects_batches_beyond_its_scratch_without_device():
    lib = pkv.library()
    assert lib.extend_attention_noalloc_scratch_bytes() == 32 << 20
    p = 4096

    def call(d):
        return lib.extend_attention_fwd_noalloc(p, p, p, p, p, p, p, p, p, 0.0, 0.0, ctypes.byref(d), None)

    assert call(desc(total_q_tokens=3_000_000, bs=64)) == -2
    assert "no-allocation" in pkv.last_error() and "scratch" in pkv.last_error()
    assert call(desc(lq=72, lv=72)) == -2
    assert call(desc(num_kv_heads=7)) == -1
    assert call(desc(bs=0)) == 0


def test_fwd_argument_errors_without_device():
    assert call_fwd(None) == pkv.PkvError(-1, "").code == -1
    assert call_fwd(desc(lq=72, lv=72)) == -2
    assert call_fwd(desc(num_kv_heads=7)) == -1
    assert call_fwd(desc(), ws_bytes=16) == -3
    assert "workspace" in pkv.last_error()
    assert call_fwd(desc(), ptr=4100) == -2  # misaligned base pointer
    assert call_fwd(desc(), ws=4096 + 16) == -3  # misaligned workspace
    assert call_fwd(desc(bs=0)) == 0  # nothing to do
    assert call_fwd(desc(total_q_tokens=0)) == 0
    lib = pkv.library()
    assert lib.extend_attention_fwd(4096, 4096, 4096, None, 4096, 4096, 4096, 4096, 4096, 0.0, 0.0,
                                    ctypes.byref(desc()), 4096, 1 << 30, None) == -1
    assert lib.extend_attention_fwd(4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096, 4096,
                                    float("nan"), 0.0, ctypes.byref(desc()), 4096, 1 << 30, None) == -1


def test_index_build_argument_errors_without_device():
    lib = pkv.library()
    p = 4096
    assert lib.build_unified_kv_indices(p, p, p, p, p, 3, 10, 5, p, p, 14, p, None) == -4
    assert "capacity" in pkv.last_error()
    assert lib.build_unified_kv_indices(p, p, p, p, p, -1, 10, 5, p, p, 15, p, None) == -1
    assert lib.build_unified_kv_indices(p, p, p, p, p, 3, 10, 5, None, p, 15, p, None) == -1
    assert lib.build_unified_kv_indices(p, None, p, p, p, 3, 10, 5, p, p, 15, p, None) == -1


def test_unified_argument_errors_without_device():
    lib = pkv.library()
    p = 4096
    d = desc()
    # no prefix_lens with rows to compute
    assert lib.extend_attention_fwd_unified(p, p, p, p, p, p, p, None, 0.0, 0.0, ctypes.byref(d), p,
                                            1 << 30, None) == -1
    assert "prefix_lens" in pkv.last_error()
    assert lib.extend_attention_fwd_unified(p, p, p, p, p, p, p, p, 0.0, 0.0, ctypes.byref(desc(bs=0)), p,
                                            1 << 30, None) == 0
    assert lib.extend_attention_fwd_unified(p, None, p, p, p, p, p, p, 0.0, 0.0, ctypes.byref(d), p,
                                            1 << 30, None) == -1
    assert lib.extend_attention_fwd_unified(p, p, p, p, p, p, p, p, 0.0, 0.0, ctypes.byref(d), p, 16,
                                            None) == -3


def test_unified_kernel_name_uses_the_pool_only():
    mla = desc(lq=576, lv=512, num_kv_heads=1, q_stride_head=576, q_stride_tok=32 * 576, ke_stride_tok=0,
               ke_stride_head=0, kp_stride_slot=576, kp_stride_head=576, o_stride_tok=32 * 512,
               o_stride_head=512, ve_stride_tok=0, ve_stride_head=0, vp_stride_slot=576, vp_stride_head=576)
    assert kernel_name(mla, None, None, 12288, 12288) == "attn_dl_kernel"
    assert kernel_name(mla, None, None, 12288, 16384) == "attn_kernel"


def test_store_and_gather_argument_errors_without_device():
    lib = pkv.library()
    p = 4096
    d = desc()
    assert lib.store_kv_cache(p, p, p, None, p, ctypes.byref(d), None) == -1
    assert lib.store_kv_cache(p, p, p, p, p, ctypes.byref(desc(total_q_tokens=0)), None) == 0
    assert lib.store_kv_cache(p + 4, p, p, p, p, ctypes.byref(d), None) == -2
    assert lib.store_kv_cache(p, p, p, p, p, ctypes.byref(desc(lq=72, lv=72)), None) == -2
    assert lib.gather_kv_indices(p, 64, p, p, None, -1, p, p, 10, None) == -1
    assert lib.gather_kv_indices(p, 64, p, p, None, 3, None, p, 10, None) == -1
    assert lib.gather_kv_indices(None, 64, p, p, None, 3, p, p, 10, None) == -1
    assert lib.gather_kv_indices(p, 64, p, p, None, 3, p, None, 10, None) == -1


def decode_desc(**kw):
    base = dict(bs=4, total_q_tokens=4, q_stride_tok=32 * 128, o_stride_tok=32 * 128, num_prefix_indices=5000)
    base.update(kw)
    return desc(**base)


def call_decode(d, ws_bytes=1 << 30, ptr=4096, ws=4096, k_pool=4096, v_pool=4096):
    lib = pkv.library()
    return lib.decode_attention_fwd(ptr, ptr, k_pool, v_pool, ptr, ptr, 0.0, 0.0,
                                    ctypes.byref(d) if d is not None else None, ws, ws_bytes, None)


def test_decode_workspace_size_grows_with_keys():
    small = pkv.decode_attention_workspace_size(decode_desc())
    big = pkv.decode_attention_workspace_size(decode_desc(num_prefix_indices=5_000_000, bs=64))
    assert 0 < small < big and small % 256 == 0
    # a sliding window bounds the keys a call can see, and with them the partial states
    windowed = pkv.decode_attention_workspace_size(decode_desc(num_prefix_indices=5_000_000, bs=64,
                                                               sliding_window=127))
    assert windowed < big


@pytest.mark.parametrize("kw,needle", [
    (dict(dtype=2), "dtype"),
    (dict(lq=72, lv=72), "not supported"),
    (dict(dtype=1, lq=256, lv=256), "not supported"),  # fp32 extend kernels serve 64 and 128 only
    (dict(dtype=1, kp_stride_slot=1002), "stride"),
    (dict(num_q_heads=30), "multiple"),
    (dict(bs=-1), "bs"),
    (dict(kp_stride_slot=1001), "stride"),
    (dict(num_prefix_indices=-1), "negative"),
    (dict(num_prefix_indices=1 << 31), "2^31"),
    (dict(custom_mask=4096, mask_indptr=4096), "custom mask"),
])
def test_decode_workspace_size_rejects(kw, needle):
    lib = pkv.library()
    assert lib.decode_attention_workspace_size(ctypes.byref(decode_desc(**kw))) == 0
    assert needle in pkv.last_error()


def test_decode_argument_errors_without_device():
    assert call_decode(None) == -1
    assert call_decode(decode_desc(dtype=1, lq=80, lv=80)) == -2
    # fp32 runs as a unified extend: its workspace is the extend workspace plus the row arrays
    f32 = decode_desc(dtype=1)
    ext = decode_desc(dtype=1, total_q_tokens=4)
    assert pkv.decode_attention_workspace_size(f32) >= pkv.extend_attention_workspace_size(ext) + 256
    assert call_decode(f32, ws_bytes=pkv.decode_attention_workspace_size(f32) - 256) == -3
    assert call_decode(f32, ws=4096 + 64) == -3
    assert call_decode(decode_desc(), ws_bytes=16) == -3
    assert call_decode(decode_desc(), ws=4096 + 64) == -3
    assert call_decode(decode_desc(), ptr=4100) == -2
    assert call_decode(decode_desc(bs=0)) == 0
    mla = decode_desc(lq=576, lv=512, num_kv_heads=1, q_stride_tok=32 * 576, q_stride_head=576,
                      o_stride_tok=32 * 512, o_stride_head=512, kp_stride_slot=576, kp_stride_head=576,
                      vp_stride_slot=512, vp_stride_head=512)
    # lq 576 / lv 512 with V in a pool of its own has a kernel; so does V inside K
    assert pkv.decode_attention_workspace_size(mla) > 0
    lib = pkv.library()
    assert lib.decode_attention_fwd(4096, None, 4096, 4096, 4096, 4096, 0.0, 0.0, ctypes.byref(decode_desc()),
                                    4096, 1 << 30, None) == -1
    assert lib.decode_attention_fwd(4096, 4096, 4096, 4096, 4096, 4096, float("inf"), 0.0,
                                    ctypes.byref(decode_desc()), 4096, 1 << 30, None) == -1
