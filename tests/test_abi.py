"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad descriptors before any HIP call (so nothing
is enqueued).  Data pointers here are fake and are never dereferenced."""
from __future__ import annotations

import ctypes
import os
import re

import pytest

from attention_kv_store_amd import _lib as L

HDR = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvstore.h")
FAKE = 0x10000  # 16-byte aligned, never touched


@pytest.fixture(scope="module")
def lib():
    return L.load()


def T(shape, dtype=L.KVS_BF16, data=FAKE, strides=None):
    return L.describe(data, dtype, shape, strides)


def ref(t):
    return ctypes.byref(t) if t is not None else None


def test_header_symbols_exported(lib):
    decl = re.findall(r"^\s*(?:kvs_status|size_t|const char\*)\s+(\w+)\s*\(", open(HDR).read(), re.M)
    assert set(decl) == set(L.EXPORTS)
    for name in decl:
        assert hasattr(lib, name), name


def test_debug_library_exports_the_same_symbols():
    """libkvstore_debug.so (the ABI built with KVS_DEBUG, same kernels) loads
    and exports every symbol the header declares, and its host-side checks
    behave as the release library's (no device call here)."""
    import os
    if not os.path.exists(L.DEBUG_LIB_PATH):
        pytest.skip("debug library not built")
    dbg = ctypes.CDLL(L.DEBUG_LIB_PATH)
    for name in L.EXPORTS:
        assert hasattr(dbg, name), name
    dbg.kvs_last_error.restype = ctypes.c_char_p
    dbg.attn_varlen_paged_ex.restype = ctypes.c_int
    a = _attn_args()
    a["q"] = T([8, 3, 64])                            # Hq % Hkv != 0: refused on the host
    st = dbg.attn_varlen_paged_ex(ref(a["q"]), ref(a["k"]), ref(a["v"]), ref(a["table"]), ref(a["cu"]), ref(a["lk"]),
                                  ctypes.c_float(0.125), 1, ref(a["out"]), ref(a.get("lse")), None, None,
                                  ctypes.c_size_t(0), None)
    assert st == L.KVS_ERR_INVALID, dbg.kvs_last_error()


def _attn_args(T_=8, Hq=4, Hkv=2, D=64, NB=8, B=2, MB=2, dtype=L.KVS_BF16):
    return dict(q=T([T_, Hq, D], dtype), k=T([NB, 16, Hkv, D], dtype), v=T([NB, 16, Hkv, D], dtype),
                table=T([B, MB], L.KVS_I32), cu=T([B + 1], L.KVS_I32), lk=T([B], L.KVS_I32),
                out=T([T_, Hq, D], dtype), lse=T([T_, Hq], L.KVS_F32))


def _call_ex(lib, a, hints=None, ws=None, ws_bytes=0, scale=0.125):
    return lib.attn_varlen_paged_ex(ref(a["q"]), ref(a["k"]), ref(a["v"]), ref(a["table"]), ref(a["cu"]),
                                    ref(a["lk"]), ctypes.c_float(scale), 1, ref(a["out"]), ref(a.get("lse")),
                                    ctypes.byref(hints) if hints else None, ws, ws_bytes, None)


@pytest.mark.parametrize("mutate,expect,msg", [
    (lambda a: a.update(q=T([8, 4, 96]), k=T([8, 16, 2, 96]), v=T([8, 16, 2, 96]), out=T([8, 4, 96])),
     L.KVS_ERR_UNSUPPORTED, "head dim"),
    (lambda a: a.update(q=T([8, 4, 128])), L.KVS_ERR_INVALID, "head dim 64 != q head dim 128"),
    (lambda a: a.update(k=T([8, 32, 2, 64]), v=T([8, 32, 2, 64])), L.KVS_ERR_UNSUPPORTED, "page size"),
    (lambda a: a.update(k=T([8, 16, 3, 64]), v=T([8, 16, 3, 64])), L.KVS_ERR_INVALID, "multiple of Hkv"),
    (lambda a: a.update(q=T([8, 4, 64], L.KVS_F32)), L.KVS_ERR_INVALID, "dtype"),
    (lambda a: a.update(out=T([8, 4, 64], L.KVS_F32)), L.KVS_ERR_INVALID, "out dtype"),
    (lambda a: a.update(out=T([8, 3, 64])), L.KVS_ERR_INVALID, "out shape"),
    (lambda a: a.update(lse=T([8, 4], L.KVS_BF16)), L.KVS_ERR_INVALID, "lse"),
    (lambda a: a.update(lse=T([8, 5], L.KVS_F32)), L.KVS_ERR_INVALID, "lse"),
    (lambda a: a.update(cu=T([2], L.KVS_I32)), L.KVS_ERR_INVALID, "cu_seqlens_q"),
    (lambda a: a.update(lk=T([3], L.KVS_I32)), L.KVS_ERR_INVALID, "seqlens_k"),
    (lambda a: a.update(table=T([2, 2], L.KVS_F32)), L.KVS_ERR_INVALID, "block_table"),
    (lambda a: a.update(q=T([1, 4, 64])), L.KVS_ERR_INVALID, "T=1 < batch"),
    (lambda a: a.update(q=T([8, 4, 64], data=FAKE + 8)), L.KVS_ERR_INVALID, "aligned"),
    (lambda a: a.update(q=T([8, 4, 64], data=0)), L.KVS_ERR_INVALID, "NULL"),
    (lambda a: a.update(q=T([8, 4, 64], strides=[512, 1, 4])), L.KVS_ERR_INVALID, "row-major"),
    (lambda a: a.update(v=T([9, 16, 2, 64])), L.KVS_ERR_INVALID, "v_cache shape"),
    (lambda a: a.update(v=None), L.KVS_ERR_INVALID, "v_cache"),
])
def test_attention_validation(lib, mutate, expect, msg):
    a = _attn_args()
    mutate(a)
    st = _call_ex(lib, a)
    assert st == expect
    assert msg in lib.kvs_last_error().decode()


def test_nonfinite_scale_rejected(lib):
    a = _attn_args()
    assert _call_ex(lib, a, scale=float("nan")) == L.KVS_ERR_INVALID


def test_decode_group_limit(lib):
    a = _attn_args(T_=2, Hq=34, Hkv=2, B=2)
    a["out"] = T([2, 34, 64])
    a["lse"] = None
    assert _call_ex(lib, a) == L.KVS_ERR_UNSUPPORTED
    assert "16 query heads" in lib.kvs_last_error().decode()


def test_workspace_sizing_and_check(lib):
    # decode shapes (T == B) with a long table need split scratch
    a = _attn_args(T_=4, Hq=8, Hkv=2, B=4, MB=128)
    a["out"] = T([4, 8, 64])
    a["lse"] = T([4, 8], L.KVS_F32)
    h = L.KvsHints()
    h.num_splits = 4
    need = lib.attn_varlen_paged_workspace_size(ref(a["q"]), ref(a["k"]), ref(a["table"]), ctypes.byref(h))
    # the fixed 4 MiB counter area, then (4 ranges + 4 sequences) slots x 8
    # heads x 64 floats and their lse, each part 256-byte aligned
    assert need == (1 << 22) + 8 * 8 * 64 * 4 + 256
    st = _call_ex(lib, a, hints=h, ws=FAKE, ws_bytes=need - 1)
    assert st == L.KVS_ERR_WORKSPACE
    h.num_splits = 1
    assert lib.attn_varlen_paged_workspace_size(ref(a["q"]), ref(a["k"]), ref(a["table"]), ctypes.byref(h)) == 0
    # prefill shapes need none
    p = _attn_args(T_=40, B=2)
    assert lib.attn_varlen_paged_workspace_size(ref(p["q"]), ref(p["k"]), ref(p["table"]), None) == 0
    # invalid shapes report (size_t)-1
    bad = T([4, 8, 96])
    assert lib.attn_varlen_paged_workspace_size(ref(bad), ref(a["k"]), ref(a["table"]), None) == ctypes.c_size_t(-1).value


def test_split_counter_limit(lib):
    # split decode keeps one counter per (sequence, KV head) in a fixed 4 MiB area
    a = _attn_args(T_=8192, Hq=256, Hkv=256, B=8192, MB=2, NB=8)
    a["out"] = T([8192, 256, 64])
    a["lse"] = None
    h = L.KvsHints()
    h.num_splits = 4
    assert _call_ex(lib, a, hints=h) == L.KVS_ERR_UNSUPPORTED
    assert "B * Hkv" in lib.kvs_last_error().decode()


def test_negative_hints_rejected(lib):
    a = _attn_args()
    h = L.KvsHints()
    h.num_splits = -1
    assert _call_ex(lib, a, hints=h) == L.KVS_ERR_INVALID


def _append_args(B=4, Hq=8, Hkv=2, D=64, NB=8, MB=2, dtype=L.KVS_BF16):
    return dict(q=T([B, Hq, D], dtype), kn=T([B, Hkv, D], dtype), vn=T([B, Hkv, D], dtype),
                k=T([NB, 16, Hkv, D], dtype), v=T([NB, 16, Hkv, D], dtype), table=T([B, MB], L.KVS_I32),
                lk=T([B], L.KVS_I32), out=T([B, Hq, D], dtype), lse=T([B, Hq], L.KVS_F32))


def _call_append(lib, a, hints=None, ws=None, ws_bytes=0, scale=0.125):
    return lib.attn_decode_append_paged(ref(a["q"]), ref(a["kn"]), ref(a["vn"]), ref(a["k"]), ref(a["v"]),
                                        ref(a["table"]), ref(a["lk"]), ctypes.c_float(scale), ref(a["out"]),
                                        ref(a.get("lse")), ctypes.byref(hints) if hints else None, ws, ws_bytes,
                                        None)


@pytest.mark.parametrize("mutate,expect,msg", [
    (lambda a: a.update(q=T([5, 8, 64]), out=T([5, 8, 64]), lse=T([5, 8], L.KVS_F32)), L.KVS_ERR_INVALID,
     "one query row per sequence"),
    (lambda a: a.update(kn=T([4, 2, 32]), vn=T([4, 2, 32])), L.KVS_ERR_INVALID, "k_new must be"),
    (lambda a: a.update(kn=T([4, 4, 64]), vn=T([4, 4, 64])), L.KVS_ERR_INVALID, "k_new must be"),
    (lambda a: a.update(kn=T([3, 2, 64]), vn=T([3, 2, 64])), L.KVS_ERR_INVALID, "k_new must be"),
    (lambda a: a.update(vn=T([4, 2, 32])), L.KVS_ERR_INVALID, "v_new shape"),
    (lambda a: a.update(kn=T([4, 2, 64], L.KVS_F32), vn=T([4, 2, 64], L.KVS_F32)), L.KVS_ERR_INVALID, "dtype"),
    (lambda a: a.update(kn=None), L.KVS_ERR_INVALID, "k_new"),
    (lambda a: a.update(vn=T([4, 2, 64], data=0)), L.KVS_ERR_INVALID, "NULL"),
    (lambda a: a.update(v=T([9, 16, 2, 64])), L.KVS_ERR_INVALID, "v_cache shape"),
    (lambda a: a.update(lk=T([3], L.KVS_I32)), L.KVS_ERR_INVALID, "seqlens_k"),
    (lambda a: a.update(lse=T([4, 7], L.KVS_F32)), L.KVS_ERR_INVALID, "lse"),
    (lambda a: a.update(q=T([4, 34, 64]), out=T([4, 34, 64]), lse=None), L.KVS_ERR_UNSUPPORTED, "16 query heads"),
])
def test_append_validation(lib, mutate, expect, msg):
    a = _append_args()
    mutate(a)
    assert _call_append(lib, a) == expect
    assert msg in lib.kvs_last_error().decode()


def test_append_workspace_check(lib):
    # the fused call takes the same workspace as the decode path of attn_varlen_paged_ex
    a = _append_args(B=4, MB=128)
    h = L.KvsHints()
    h.num_splits = 4
    need = lib.attn_varlen_paged_workspace_size(ref(a["q"]), ref(a["k"]), ref(a["table"]), ctypes.byref(h))
    assert need > 0
    assert _call_append(lib, a, hints=h, ws=FAKE, ws_bytes=need - 1) == L.KVS_ERR_WORKSPACE
    h.num_splits = -2
    assert _call_append(lib, a, hints=h) == L.KVS_ERR_INVALID


@pytest.mark.parametrize("mutate,expect,msg", [
    (lambda a: a.update(kn=T([4, 2, 32]), vn=T([4, 2, 32])), L.KVS_ERR_INVALID, "does not match"),
    (lambda a: a.update(kn=T([4, 2, 32])), L.KVS_ERR_INVALID, "v_new shape"),
    (lambda a: a.update(kn=T([4, 2, 64], L.KVS_F32), vn=T([4, 2, 64], L.KVS_F32)), L.KVS_ERR_INVALID, "one dtype"),
    (lambda a: a.update(slots=T([5], L.KVS_I32)), L.KVS_ERR_INVALID, "slot_mapping"),
    (lambda a: a.update(slots=T([4], L.KVS_F32)), L.KVS_ERR_INVALID, "slot_mapping"),
    (lambda a: a.update(kc=T([8, 8, 2, 64]), vc=T([8, 8, 2, 64])), L.KVS_ERR_UNSUPPORTED, "page size"),
    (lambda a: a.update(vc=T([7, 16, 2, 64])), L.KVS_ERR_INVALID, "v_cache shape"),
    (lambda a: a.update(kc=None), L.KVS_ERR_INVALID, "NULL"),
])
def test_store_validation(lib, mutate, expect, msg):
    a = dict(kn=T([4, 2, 64]), vn=T([4, 2, 64]), slots=T([4], L.KVS_I32), kc=T([8, 16, 2, 64]), vc=T([8, 16, 2, 64]))
    mutate(a)
    st = lib.kv_store_paged(ref(a["kn"]), ref(a["vn"]), ref(a["slots"]), ref(a["kc"]), ref(a["vc"]), None)
    assert st == expect
    assert msg in lib.kvs_last_error().decode()


def test_store_empty_is_noop(lib):
    st = lib.kv_store_paged(ref(T([0, 2, 64], data=0)), ref(T([0, 2, 64], data=0)), ref(T([0], L.KVS_I32, data=0)),
                            ref(T([8, 16, 2, 64])), ref(T([8, 16, 2, 64])), None)
    assert st == L.KVS_OK
    assert "empty" in lib.kvs_last_dispatch().decode()


def test_binding_fails_loudly_without_library(tmp_path):
    import importlib

    mod = importlib.import_module("attention_kv_store_amd._lib")
    saved = mod._lib
    try:
        mod._lib = None
        with pytest.raises(ImportError):
            mod.load(str(tmp_path / "missing.so"))
    finally:
        mod._lib = saved


# ---- sliding window entry points ----------------------------------------------
def _call_window(lib, a, window, hints=None):
    return lib.attn_varlen_paged_window_ex(ref(a["q"]), ref(a["k"]), ref(a["v"]), ref(a["table"]), ref(a["cu"]),
                                           ref(a["lk"]), ctypes.c_float(0.125), window, ref(a["out"]),
                                           ref(a.get("lse")), ctypes.byref(hints) if hints else None, None, 0, None)


def _call_append_window(lib, a, window):
    return lib.attn_decode_append_paged_window(ref(a["q"]), ref(a["kn"]), ref(a["vn"]), ref(a["k"]), ref(a["v"]),
                                               ref(a["table"]), ref(a["lk"]), ctypes.c_float(0.125), window,
                                               ref(a["out"]), ref(a.get("lse")), None, None, 0, None)


@pytest.mark.parametrize("window", [0, -1, -100])
def test_window_must_be_positive(lib, window):
    assert _call_window(lib, _attn_args(), window) == L.KVS_ERR_INVALID
    assert "window must be >= 1" in lib.kvs_last_error().decode()
    assert _call_append_window(lib, _append_args(), window) == L.KVS_ERR_INVALID
    assert "window must be >= 1" in lib.kvs_last_error().decode()


def test_window_entries_validate_like_the_others(lib):
    a = _attn_args()
    a.update(out=T([8, 3, 64]))
    assert _call_window(lib, a, 16) == L.KVS_ERR_INVALID
    assert "out shape" in lib.kvs_last_error().decode()
    h = L.KvsHints()
    h.num_splits = -1
    assert _call_window(lib, _attn_args(), 16, hints=h) == L.KVS_ERR_INVALID
    a = _append_args()
    a.update(kn=T([4, 2, 32]), vn=T([4, 2, 32]))
    assert _call_append_window(lib, a, 16) == L.KVS_ERR_INVALID
    assert "k_new must be" in lib.kvs_last_error().decode()


def test_binding_window_needs_causal():
    import attention_kv_store_amd as kvs
    with pytest.raises(ValueError):
        kvs.attn_varlen_paged(None, None, None, None, None, None, 0.125, False, window=4)


def test_window_context_limit(lib):
    # 16 * MB above 2^30 keys: the window arithmetic would leave 32 bits
    a = _attn_args(B=1, MB=(1 << 26) + 1, T_=8)
    a.update(cu=T([2], L.KVS_I32), lk=T([1], L.KVS_I32))
    assert _call_window(lib, a, 16) == L.KVS_ERR_UNSUPPORTED
    assert "16 * MB <= 2^30" in lib.kvs_last_error().decode()


# ---- RoPE + store ----------------------------------------------------------------
def _rope_args(T_=4, Hq=8, Hkv=2, D=64, NB=4, dtype=L.KVS_BF16):
    return dict(q=T([T_, Hq, D], dtype), kn=T([T_, Hkv, D], dtype), vn=T([T_, Hkv, D], dtype),
                pos=T([T_], L.KVS_I32), slots=T([T_], L.KVS_I32), k=T([NB, 16, Hkv, D], dtype),
                v=T([NB, 16, Hkv, D], dtype))


def _call_rope(lib, a, rotary_dim=0, style=0, base=10000.0, pos_scale=1.0, rope=True):
    r = L.KvsRope()
    r.rotary_dim, r.style, r.base, r.pos_scale = rotary_dim, style, base, pos_scale
    return lib.kv_store_rope_paged(ref(a["q"]), ref(a["kn"]), ref(a["vn"]), ref(a["pos"]), ref(a["slots"]),
                                   ref(a["k"]), ref(a["v"]), ctypes.byref(r) if rope else None, None)


@pytest.mark.parametrize("kw,mutate,expect,msg", [
    (dict(rotary_dim=8), None, L.KVS_ERR_INVALID, "rotary_dim"),
    (dict(rotary_dim=24), None, L.KVS_ERR_INVALID, "rotary_dim"),
    (dict(rotary_dim=80), None, L.KVS_ERR_INVALID, "rotary_dim"),
    (dict(style=2), None, L.KVS_ERR_INVALID, "style"),
    (dict(base=0.0), None, L.KVS_ERR_INVALID, "base and pos_scale"),
    (dict(base=float("inf")), None, L.KVS_ERR_INVALID, "base and pos_scale"),
    (dict(pos_scale=-1.0), None, L.KVS_ERR_INVALID, "base and pos_scale"),
    (dict(rope=False), None, L.KVS_ERR_INVALID, "NULL"),
    ({}, lambda a: a.update(q=T([4, 8, 64], L.KVS_F32)), L.KVS_ERR_INVALID, "one dtype"),
    ({}, lambda a: a.update(q=T([5, 8, 64])), L.KVS_ERR_INVALID, "q must be"),
    ({}, lambda a: a.update(pos=T([3], L.KVS_I32)), L.KVS_ERR_INVALID, "positions"),
    ({}, lambda a: a.update(slots=T([5], L.KVS_I32)), L.KVS_ERR_INVALID, "slot_mapping"),
    ({}, lambda a: a.update(kn=T([4, 2, 32]), vn=T([4, 2, 32])), L.KVS_ERR_INVALID, "k_new"),
    ({}, lambda a: a.update(k=T([4, 8, 2, 64]), v=T([4, 8, 2, 64])), L.KVS_ERR_UNSUPPORTED, "page size"),
    ({}, lambda a: a.update(q=T([4, 8, 40]), kn=T([4, 2, 40]), vn=T([4, 2, 40]), k=T([4, 16, 2, 40]),
                            v=T([4, 16, 2, 40])), L.KVS_ERR_UNSUPPORTED, "head dim"),
    ({}, lambda a: a.update(q=T([4, 8, 512]), kn=T([4, 2, 512]), vn=T([4, 2, 512]), k=T([4, 16, 2, 512]),
                            v=T([4, 16, 2, 512])), L.KVS_ERR_UNSUPPORTED, "head dim"),
])
def test_rope_validation(lib, kw, mutate, expect, msg):
    a = _rope_args()
    if mutate:
        mutate(a)
    assert _call_rope(lib, a, **kw) == expect
    assert msg in lib.kvs_last_error().decode()


def test_rope_empty_is_noop(lib):
    a = _rope_args(T_=0)
    assert _call_rope(lib, a) == L.KVS_OK
    assert "empty" in lib.kvs_last_dispatch().decode()


# ---- FP8 cache ---------------------------------------------------------------------
FP8 = L.KVS_FP8_E4M3


def _fp8_args(T_=2, B=2, Hq=4, Hkv=2, D=64, NB=8, MB=2):
    a = _attn_args(T_=T_, B=B, Hq=Hq, Hkv=Hkv, D=D, NB=NB, MB=MB)
    a.update(k=T([NB, 16, Hkv, D], FP8), v=T([NB, 16, Hkv, D], FP8),
             ks=T([NB, Hkv, 16], L.KVS_F32), vs=T([NB, Hkv, 16], L.KVS_F32))
    return a


def _call_fp8(lib, a, causal=1, window=0):
    return lib.attn_varlen_paged_fp8_ex(ref(a["q"]), ref(a["k"]), ref(a["v"]), ref(a["ks"]), ref(a["vs"]),
                                        ref(a["table"]), ref(a["cu"]), ref(a["lk"]), ctypes.c_float(0.125), causal,
                                        window, ref(a["out"]), ref(a.get("lse")), None, None, 0, None)


def test_fp8_cache_needs_the_fp8_entry(lib):
    a = _fp8_args()
    assert _call_ex(lib, a) == L.KVS_ERR_INVALID
    assert "attn_varlen_paged_fp8_ex" in lib.kvs_last_error().decode()


@pytest.mark.parametrize("mutate,expect,msg", [
    (lambda a: a.update(ks=T([8, 2, 8], L.KVS_F32)), L.KVS_ERR_INVALID, "scales must be"),
    (lambda a: a.update(vs=T([8, 3, 16], L.KVS_F32)), L.KVS_ERR_INVALID, "scales must be"),
    (lambda a: a.update(ks=T([8, 2, 16], L.KVS_BF16)), L.KVS_ERR_INVALID, "k_scale"),
    (lambda a: a.update(k=T([8, 16, 2, 64]), v=T([8, 16, 2, 64])), L.KVS_ERR_INVALID, "k_cache"),
    (lambda a: a.update(q=T([2, 4, 64], L.KVS_F32), out=T([2, 4, 64], L.KVS_F32)), L.KVS_ERR_INVALID, "does not go with"),
    (lambda a: a.update(v=T([8, 16, 2, 64])), L.KVS_ERR_INVALID, "v_cache"),
])
def test_fp8_attention_validation(lib, mutate, expect, msg):
    a = _fp8_args()
    mutate(a)
    assert _call_fp8(lib, a) == expect
    assert msg in lib.kvs_last_error().decode()


def test_fp8_window_needs_causal(lib):
    assert _call_fp8(lib, _fp8_args(), causal=0, window=4) == L.KVS_ERR_INVALID
    assert _call_fp8(lib, _fp8_args(), window=-2) == L.KVS_ERR_INVALID


def _call_store_fp8(lib, a):
    return lib.kv_store_paged_fp8(ref(a["kn"]), ref(a["vn"]), ref(a["slots"]), ref(a["k"]), ref(a["v"]),
                                  ref(a["ks"]), ref(a["vs"]), None)


def _store_fp8_args(Tn=4, Hkv=2, D=64, NB=4):
    return dict(kn=T([Tn, Hkv, D]), vn=T([Tn, Hkv, D]), slots=T([Tn], L.KVS_I32), k=T([NB, 16, Hkv, D], FP8),
                v=T([NB, 16, Hkv, D], FP8), ks=T([NB, Hkv, 16], L.KVS_F32), vs=T([NB, Hkv, 16], L.KVS_F32))


@pytest.mark.parametrize("mutate,expect,msg", [
    (lambda a: a.update(k=T([4, 16, 2, 64])), L.KVS_ERR_INVALID, "k_cache"),
    (lambda a: a.update(ks=T([4, 2, 15], L.KVS_F32)), L.KVS_ERR_INVALID, "scales must be"),
    (lambda a: a.update(vn=T([4, 2, 64], L.KVS_F32)), L.KVS_ERR_INVALID, "v_new dtype"),
    (lambda a: a.update(kn=T([4, 3, 64]), vn=T([4, 3, 64])), L.KVS_ERR_INVALID, "k_new"),
    (lambda a: a.update(slots=T([5], L.KVS_I32)), L.KVS_ERR_INVALID, "slot_mapping"),
    (lambda a: a.update(kn=T([4, 2, 96]), vn=T([4, 2, 96]), k=T([4, 16, 2, 96], FP8), v=T([4, 16, 2, 96], FP8)),
     L.KVS_ERR_UNSUPPORTED, "head dim"),
])
def test_fp8_store_validation(lib, mutate, expect, msg):
    a = _store_fp8_args()
    mutate(a)
    assert _call_store_fp8(lib, a) == expect
    assert msg in lib.kvs_last_error().decode()


def test_fp8_store_empty_is_noop(lib):
    assert _call_store_fp8(lib, _store_fp8_args(Tn=0)) == L.KVS_OK


# ---- INT8 cache ----------------------------------------------------------------------
I8 = L.KVS_INT8


def _int8_args():
    a = _fp8_args()
    a.update(k=T([8, 16, 2, 64], I8), v=T([8, 16, 2, 64], I8))
    return a


def _call_int8(lib, a, causal=1, window=0):
    return lib.attn_varlen_paged_int8_ex(ref(a["q"]), ref(a["k"]), ref(a["v"]), ref(a["ks"]), ref(a["vs"]),
                                         ref(a["table"]), ref(a["cu"]), ref(a["lk"]), ctypes.c_float(0.125), causal,
                                         window, ref(a["out"]), ref(a.get("lse")), None, None, 0, None)


def test_int8_cache_needs_a_scaled_entry(lib):
    a = _int8_args()
    assert _call_ex(lib, a) == L.KVS_ERR_INVALID
    assert "attn_varlen_paged_int8_ex" in lib.kvs_last_error().decode()


def test_int8_and_fp8_entries_take_only_their_codes(lib):
    assert _call_int8(lib, _fp8_args()) == L.KVS_ERR_INVALID      # E4M3 pool at the INT8 entry
    assert "k_cache" in lib.kvs_last_error().decode()
    assert _call_fp8(lib, _int8_args()) == L.KVS_ERR_INVALID      # INT8 pool at the FP8 entry
    assert "k_cache" in lib.kvs_last_error().decode()


@pytest.mark.parametrize("mutate,msg", [
    (lambda a: a.update(ks=T([8, 2, 8], L.KVS_F32)), "scales must be"),
    (lambda a: a.update(v=T([8, 16, 2, 64], FP8)), "v_cache"),
    (lambda a: a.update(q=T([2, 4, 64], L.KVS_F32), out=T([2, 4, 64], L.KVS_F32)), "does not go with"),
])
def test_int8_attention_validation(lib, mutate, msg):
    a = _int8_args()
    mutate(a)
    assert _call_int8(lib, a) == L.KVS_ERR_INVALID
    assert msg in lib.kvs_last_error().decode()


def _call_store_int8(lib, a):
    return lib.kv_store_paged_int8(ref(a["kn"]), ref(a["vn"]), ref(a["slots"]), ref(a["k"]), ref(a["v"]),
                                   ref(a["ks"]), ref(a["vs"]), None)


def test_int8_store_validation_and_empty(lib):
    a = _store_fp8_args()
    assert _call_store_int8(lib, a) == L.KVS_ERR_INVALID          # E4M3 pools at the INT8 store
    assert "k_cache" in lib.kvs_last_error().decode()
    a.update(k=T([4, 16, 2, 64], I8), v=T([4, 16, 2, 64], I8))
    assert _call_store_fp8(lib, a) == L.KVS_ERR_INVALID           # INT8 pools at the FP8 store
    a.update(kn=T([4, 2, 96]), vn=T([4, 2, 96]), k=T([4, 16, 2, 96], I8), v=T([4, 16, 2, 96], I8))
    assert _call_store_int8(lib, a) == L.KVS_ERR_UNSUPPORTED
    assert "head dim" in lib.kvs_last_error().decode()
    e = _store_fp8_args(Tn=0)
    e.update(k=T([4, 16, 2, 64], I8), v=T([4, 16, 2, 64], I8))
    assert _call_store_int8(lib, e) == L.KVS_OK
    assert "kv_store_paged_int8: empty" in lib.kvs_last_dispatch().decode()


# ---- decode_tail hint ----------------------------------------------------------------
def _hint(**kw):
    h = L.KvsHints()
    for k, v in kw.items():
        setattr(h, k, v)
    return h


@pytest.mark.parametrize("tail,msg", [(-1, "non-negative"), (3, "does not fit"), (2, "one query row per sequence")])
def test_decode_tail_validation(lib, tail, msg):
    a = _attn_args(T_=8, B=2)
    assert _call_ex(lib, a, hints=_hint(decode_tail=tail)) == L.KVS_ERR_INVALID
    assert msg in lib.kvs_last_error().decode()


def test_decode_tail_workspace_is_the_decode_parts():
    """With the hint, the workspace is sized for the last N sequences alone."""
    lib = L.load()
    B, MB, N, T_ = 40, 128, 30, 10 + 30 * 1 + 500
    q, k, table = T([T_, 32, 128]), T([4096, 16, 8, 128]), T([B, MB], L.KVS_I32)
    h = _hint(decode_tail=N, num_splits=64)
    got = lib.attn_varlen_paged_workspace_size(ref(q), ref(k), ref(table), ctypes.byref(h))
    qd, td = T([N, 32, 128]), T([N, MB], L.KVS_I32, data=FAKE + (B - N) * MB * 4)
    want = lib.attn_varlen_paged_workspace_size(ref(qd), ref(k), ref(td), ctypes.byref(_hint(num_splits=64)))
    assert got == want and got > 0


def _call_append_rope(lib, a, rope, window=0):
    return lib.attn_decode_append_paged_rope(ref(a["q"]), ref(a["kn"]), ref(a["vn"]), ref(a["k"]), ref(a["v"]),
                                             ref(a["table"]), ref(a["lk"]), ctypes.c_float(0.125), window,
                                             ctypes.byref(rope) if rope is not None else None, ref(a["out"]),
                                             ref(a.get("lse")), None, None, 0, None)


@pytest.mark.parametrize("dtype,D,kw,expect,msg", [
    (L.KVS_F32, 64, dict(), L.KVS_ERR_UNSUPPORTED, "bf16 only"),
    (L.KVS_BF16, 128, dict(rotary_dim=32), L.KVS_ERR_UNSUPPORTED, "multiple of 64"),
    (L.KVS_BF16, 64, dict(rotary_dim=8, style=1), L.KVS_ERR_UNSUPPORTED, "multiple of 16"),
    (L.KVS_BF16, 64, dict(style=3), L.KVS_ERR_INVALID, "style"),
    (L.KVS_BF16, 64, dict(base=-1.0), L.KVS_ERR_INVALID, "base and pos_scale"),
    (L.KVS_BF16, 64, None, L.KVS_ERR_INVALID, "NULL"),
])
def test_fused_rope_validation(lib, dtype, D, kw, expect, msg):
    a = _append_args(D=D, dtype=dtype)
    rope = None
    if kw is not None:
        rope = L.KvsRope()
        rope.rotary_dim, rope.style = kw.get("rotary_dim", 0), kw.get("style", 0)
        rope.base, rope.pos_scale = kw.get("base", 10000.0), 1.0
    assert _call_append_rope(lib, a, rope) == expect
    assert msg in lib.kvs_last_error().decode()


# ---------------------------------------------------------------- header ----
def _declarations(path):
    """(name, comment block right above it) of every function the header declares."""
    text = open(path).read()
    out = []
    for m in re.finditer(r"^\s*(?:kvs_status|size_t|const char\*)\s+(\w+)\s*\(", text, re.M):
        head = text[:m.start()]
        end = head.rfind("*/")
        start = head.rfind("/*", 0, end)
        between = head[end + 2:]
        # the comment must belong to this declaration: only blank lines or an
        # earlier declaration's closing text may not sit between them
        assert end >= 0 and ";" not in between, m.group(1)
        out.append((m.group(1), head[start:end]))
    return out


def test_every_declaration_cites_its_passage():
    """Each entry point's comment names the passage of the pages that defines
    the operation (a section sign, or one of the page titles); the
    no-allocation variant names the callers it exists for instead."""
    cites = ("§", "tiny-vLLM", "장부가 커널 인자로", "장부에서 텐서로")
    for hdr in (HDR, os.path.join(os.path.dirname(HDR), "kvstore_calib.h")):
        for name, comment in _declarations(hdr):
            if name == "attn_varlen_paged_noalloc":
                assert "cannot" in comment and "allocate" in comment, name
                continue
            assert any(c in comment for c in cites), f"{name} cites no passage"


def test_calibration_kernel_lives_outside_the_product_library(lib):
    """The benchmark's MFMA calibration kernel is exported by its own library,
    not by libkvstore.so."""
    assert not hasattr(lib, "kvs_mfma_peak_launch")
    path = os.path.join(os.path.dirname(L.LIB_PATH), "libkvstore_calib.so")
    if not os.path.exists(path):
        pytest.skip("calibration library not built")
    calib = ctypes.CDLL(path)
    assert hasattr(calib, "kvs_mfma_peak_launch")
    calib.kvs_mfma_peak_launch.restype = ctypes.c_int
    calib.kvs_mfma_peak_launch.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_void_p]
    # refused on the host (unaligned source), nothing launched
    assert calib.kvs_mfma_peak_launch(FAKE + 4, FAKE, 1, 1, None) == L.KVS_ERR_INVALID


# ------------------------------------------------- host sanitizer build ----
def test_abi_host_code_under_address_and_ub_sanitizers(tmp_path):
    """The C-ABI code (validation, planning, workspace handling) built for the
    host with AddressSanitizer and UndefinedBehaviorSanitizer, linked with
    host stand-ins for the kernels and the HIP runtime (tests/abi_sanitize),
    and driven through every entry point with valid and malformed
    descriptors.  Any memory error, undefined behaviour or unexpected status
    fails the test."""
    import shutil
    import subprocess

    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    clang = "/opt/rocm/llvm/bin/clang++"
    if not (os.path.exists(hipcc) and os.path.exists(clang)):
        pytest.skip("ROCm toolchain not found")
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    inc = os.path.join(root, "include")
    here = os.path.join(root, "tests", "abi_sanitize")
    san = ["-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer"]
    host_san = [x for f in san for x in ("-Xarch_host", f)]
    steps = [
        [hipcc, "--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fPIC", *host_san,
         "-Wno-unused-command-line-argument", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         f"-I{inc}", "-c", os.path.join(root, "attention_kv_store_amd", "csrc", "api.hip"),
         "-o", str(tmp_path / "api.o")],
        [clang, "-O1", "-g", "-std=c++17", *san, "-D__HIP_PLATFORM_AMD__", f"-I{inc}", "-I/opt/rocm/include",
         "-c", os.path.join(here, "stubs.cpp"), "-o", str(tmp_path / "stubs.o")],
        [clang, "-O1", "-g", "-std=c++17", *san, f"-I{inc}", "-c", os.path.join(here, "driver.cpp"),
         "-o", str(tmp_path / "driver.o")],
        [clang, *san, str(tmp_path / "api.o"), str(tmp_path / "stubs.o"), str(tmp_path / "driver.o"),
         "-o", str(tmp_path / "driver")],
    ]
    for cmd in steps:
        r = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
        assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0", UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([str(tmp_path / "driver")], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout + r.stderr)[-4000:]
    assert "abi sanitize driver: OK" in r.stdout
