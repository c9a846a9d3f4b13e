"""MI355X (gfx950) paged varlen attention and KV store.

Python names mirror the C ABI (include/kvstore.h):

* ``kv_store_paged(k_new, v_new, slot_mapping, k_cache, v_cache)``
* ``kv_store_rope_paged(q, k_new, v_new, positions, slot_mapping, k_cache,
  v_cache, rotary_dim=0, base=10000.0, style="neox", pos_scale=1.0)``
* ``kv_store_paged_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale,
  v_scale)`` and ``attn_varlen_paged_fp8(q, k_cache, v_cache, k_scale, v_scale,
  block_table, cu_seqlens_q, seqlens_k, scale, causal, ...)``: the FP8 (E4M3)
  cache with one scale per token row and KV head; ``kv_store_paged_int8``,
  ``attn_varlen_paged_int8`` and ``attn_decode_append_paged_int8``: the same
  for an INT8 cache (torch.int8 codes)
* ``attn_varlen_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k,
  scale, causal, out=None, lse=None, ...)`` (``window=W`` selects the
  sliding-window entry point ``attn_varlen_paged_window_ex``)
* ``attn_decode_append_paged(q, k_new, v_new, k_cache, v_cache, block_table,
  seqlens_k, scale, ...)`` (``window=W``: ``attn_decode_append_paged_window``)

They take torch tensors on the current HIP device (torch supplies memory and
the stream) and enqueue the library's kernels on torch's current stream.  The
binding marshals arguments only; every step runs in the HIP kernels, and a
missing library is an error, never a fallback.
"""
from __future__ import annotations

import ctypes
from typing import Optional

from . import _lib
from ._lib import KVS_BF16, KVS_F32, KVS_I32, KvsError, KvsHints, KvsRope, describe, last_dispatch  # noqa: F401

__all__ = ["kv_store_paged", "kv_store_rope_paged", "kv_store_paged_fp8", "attn_varlen_paged_fp8",
           "attn_decode_append_paged_fp8", "kv_store_paged_int8", "attn_varlen_paged_int8",
           "attn_decode_append_paged_int8", "attn_varlen_paged", "attn_decode_append_paged", "workspace_size", "last_dispatch", "KvsError", "release_workspace"]


def _dtype_code(t) -> int:
    import torch

    m = {torch.float32: KVS_F32, torch.bfloat16: KVS_BF16, torch.int32: KVS_I32,
         # FP8 caches: E4M3 codes, as torch's float8_e4m3fn or as raw bytes
         torch.float8_e4m3fn: _lib.KVS_FP8_E4M3, torch.uint8: _lib.KVS_FP8_E4M3,
         # INT8 caches: signed codes
         torch.int8: _lib.KVS_INT8}
    if t.dtype not in m:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return m[t.dtype]


def _desc(t):
    if t is None:
        return None
    return describe(t.data_ptr(), _dtype_code(t), list(t.shape), list(t.stride()))


def _ref(d):
    return ctypes.byref(d) if d is not None else None


def _stream(t) -> int:
    import torch

    return torch.cuda.current_stream(t.device).cuda_stream


def kv_store_paged(k_new, v_new, slot_mapping, k_cache, v_cache) -> None:
    """Write row t of k_new/v_new [T, Hkv, D] into slot slot_mapping[t] of the
    [NB, 16, Hkv, D] pools (negative slots are skipped), in place."""
    lib = _lib.load()
    d = [_desc(x) for x in (k_new, v_new, slot_mapping, k_cache, v_cache)]
    _lib.check(lib.kv_store_paged(*[_ref(x) for x in d], _stream(k_cache)))


def kv_store_rope_paged(q, k_new, v_new, positions, slot_mapping, k_cache, v_cache, *, rotary_dim: int = 0,
                        base: float = 10000.0, style: str = "neox", pos_scale: float = 1.0) -> None:
    """The RoPE + KV store step: rotate ``q`` [T, Hq, D] in place (may be None),
    write RoPE(``k_new``) and ``v_new`` [T, Hkv, D] into ``slot_mapping`` of the
    pools (negative slots skipped); token t sits at ``positions[t]``.  ``style``
    is "neox" (pairs i, i + rotary_dim/2) or "interleaved" (pairs 2i, 2i + 1);
    ``rotary_dim`` 0 means the whole head."""
    r = _rope(rotary_dim, base, style, pos_scale)
    lib = _lib.load()
    d = [_desc(x) for x in (q, k_new, v_new, positions, slot_mapping, k_cache, v_cache)]
    _lib.check(lib.kv_store_rope_paged(*[_ref(x) for x in d], ctypes.byref(r), _stream(k_cache)))


def kv_store_paged_fp8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale) -> None:
    """Quantize rows of ``k_new`` / ``v_new`` [T, Hkv, D] (f32 / bf16) into the E4M3
    pools [NB, 16, Hkv, D] (float8_e4m3fn or uint8 codes) at ``slot_mapping``,
    one fp32 scale per (row, head) into ``k_scale`` / ``v_scale`` [NB, Hkv, 16]."""
    lib = _lib.load()
    d = [_desc(x) for x in (k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale)]
    _lib.check(lib.kv_store_paged_fp8(*[_ref(x) for x in d], _stream(k_cache)))


def kv_store_paged_int8(k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale) -> None:
    """Quantize rows of ``k_new`` / ``v_new`` [T, Hkv, D] (f32 / bf16) into the INT8
    pools [NB, 16, Hkv, D] (torch.int8 codes, scale absmax / 127) at
    ``slot_mapping``, one fp32 scale per (row, head) into ``k_scale`` /
    ``v_scale`` [NB, Hkv, 16]."""
    lib = _lib.load()
    d = [_desc(x) for x in (k_new, v_new, slot_mapping, k_cache, v_cache, k_scale, v_scale)]
    _lib.check(lib.kv_store_paged_int8(*[_ref(x) for x in d], _stream(k_cache)))


def attn_varlen_paged_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, cu_seqlens_q, seqlens_k,
                          scale: float, causal: bool = True, out=None, lse=None, *, return_lse: bool = True,
                          num_splits: int = 0, workspace=None, window: int = 0, decode_tail: int = 0,
                          _entry: str = "attn_varlen_paged_fp8_ex"):
    """Attention over an FP8 cache (values = E4M3(code) * scale of the row and
    head); q / out bf16.  Returns ``(out, lse)``."""
    import torch

    if window and not causal:
        raise ValueError("a sliding window needs the causal mask")
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    h = _hints(0, 0, num_splits, decode_tail)
    ws_ptr, ws_bytes, workspace = _workspace(lib, q, k_cache, block_table, h, workspace)
    d = [_desc(x) for x in (q, k_cache, v_cache, k_scale, v_scale, block_table, cu_seqlens_q, seqlens_k)]
    st = getattr(lib, _entry)(*[_ref(x) for x in d], ctypes.c_float(scale), int(bool(causal)), int(window),
                              _ref(_desc(out)), _ref(_desc(lse)), ctypes.byref(h), ws_ptr, ws_bytes, _stream(q))
    _lib.check(st)
    return out, lse


def attn_varlen_paged_int8(q, k_cache, v_cache, k_scale, v_scale, block_table, cu_seqlens_q, seqlens_k,
                           scale: float, causal: bool = True, out=None, lse=None, **kw):
    """Attention over an INT8 cache (values = code * scale of the row and
    head); the arguments of ``attn_varlen_paged_fp8``.  Returns ``(out, lse)``."""
    return attn_varlen_paged_fp8(q, k_cache, v_cache, k_scale, v_scale, block_table, cu_seqlens_q, seqlens_k,
                                 scale, causal, out, lse, _entry="attn_varlen_paged_int8_ex", **kw)


def _rope(rotary_dim, base, style, pos_scale):
    styles = {"neox": _lib.KVS_ROPE_NEOX, "interleaved": _lib.KVS_ROPE_INTERLEAVED}
    if style not in styles:
        raise ValueError(f"style must be one of {sorted(styles)}")
    r = KvsRope()
    r.rotary_dim, r.style, r.base, r.pos_scale = int(rotary_dim), styles[style], float(base), float(pos_scale)
    return r


def _hints(max_seqlen_q=0, max_seqlen_k=0, num_splits=0, decode_tail=0):
    h = KvsHints()
    h.max_seqlen_q = int(max_seqlen_q or 0)
    h.max_seqlen_k = int(max_seqlen_k or 0)
    h.num_splits = int(num_splits or 0)
    h.decode_tail = int(decode_tail or 0)
    return h


def workspace_size(q, k_cache, block_table, *, max_seqlen_q=0, max_seqlen_k=0, num_splits=0, decode_tail=0) -> int:
    lib = _lib.load()
    h = _hints(max_seqlen_q, max_seqlen_k, num_splits, decode_tail)
    n = lib.attn_varlen_paged_workspace_size(_ref(_desc(q)), _ref(_desc(k_cache)), _ref(_desc(block_table)),
                                             ctypes.byref(h))
    if n == ctypes.c_size_t(-1).value:
        raise KvsError(_lib.KVS_ERR_INVALID, lib.kvs_last_error().decode())
    return int(n)


def attn_varlen_paged(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, scale: float,
                      causal: bool = True, out=None, lse=None, *, return_lse: bool = True,
                      max_seqlen_q: int = 0, max_seqlen_k: int = 0, num_splits: int = 0,
                      workspace=None, window: int = 0, decode_tail: int = 0):
    """Exact paged varlen attention.  Returns ``(out, lse)`` (lse is None when
    ``return_lse`` is False and no ``lse`` tensor was given).

    Uses the allocation-free ``attn_varlen_paged_ex`` entry point with the
    workspace passed in, which must have been zero-filled before its first use
    and be at least ``workspace_size`` bytes (the library checks), or else a
    torch-allocated one of the size needed.  ``window`` > 0 (needs ``causal``)
    calls ``attn_varlen_paged_window_ex``: the row at position p sees keys
    p - window + 1 .. p.  ``decode_tail`` = N states that the last N sequences
    have one query row each (they then run on the decode path)."""
    import torch

    if window and not causal:
        raise ValueError("a sliding window needs the causal mask")
    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    h = _hints(max_seqlen_q, max_seqlen_k, num_splits, decode_tail)
    ws_ptr, ws_bytes, workspace = _workspace(lib, q, k_cache, block_table, h, workspace)
    d = [_desc(q), _desc(k_cache), _desc(v_cache), _desc(block_table), _desc(cu_seqlens_q), _desc(seqlens_k)]
    if window:
        st = lib.attn_varlen_paged_window_ex(*[_ref(x) for x in d], ctypes.c_float(scale), int(window),
                                             _ref(_desc(out)), _ref(_desc(lse)), ctypes.byref(h), ws_ptr,
                                             ws_bytes, _stream(q))
    else:
        st = lib.attn_varlen_paged_ex(*[_ref(x) for x in d], ctypes.c_float(scale), int(bool(causal)),
                                      _ref(_desc(out)), _ref(_desc(lse)), ctypes.byref(h), ws_ptr, ws_bytes,
                                      _stream(q))
    _lib.check(st)
    return out, lse


def _workspace(lib, q, k_cache, block_table, h, workspace):
    """(pointer, bytes, tensor) of the decode workspace: the caller's as given (the
    library checks its size), else a new zero-filled one of the size needed.
    A workspace is zero-filled once: the decode counters in it must start at
    zero, and every call leaves them at zero, so it may be kept and reused."""
    if workspace is not None:
        return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace
    dq, dk, dt_ = _desc(q), _desc(k_cache), _desc(block_table)
    need = lib.attn_varlen_paged_workspace_size(_ref(dq), _ref(dk), _ref(dt_), ctypes.byref(h))
    if need == ctypes.c_size_t(-1).value:
        raise KvsError(_lib.KVS_ERR_INVALID, lib.kvs_last_error().decode())
    if not need:
        return None, 0, None
    import torch

    workspace = torch.zeros(int(need), dtype=torch.uint8, device=q.device)
    return workspace.data_ptr(), int(need), workspace


def attn_decode_append_paged(q, k_new, v_new, k_cache, v_cache, block_table, seqlens_k, scale: float,
                             out=None, lse=None, *, return_lse: bool = True, max_seqlen_k: int = 0,
                             num_splits: int = 0, workspace=None, window: int = 0, rope=None):
    """One decode step in one launch: writes row b of ``k_new`` / ``v_new`` as
    key ``seqlens_k[b] - 1`` of sequence b (its slot taken from the block
    table) and attends query row b over the sequence's ``seqlens_k[b]`` keys
    (the last ``window`` of them when ``window`` > 0).  Same result as
    ``kv_store_paged`` then ``attn_varlen_paged`` with ``cu_seqlens_q = 0..B``.
    ``rope`` (a dict of ``kv_store_rope_paged``'s rotary_dim / base / style /
    pos_scale) also rotates q and the new keys, sequence b's new token at
    position ``seqlens_k[b] - 1`` (``q`` itself is not modified).
    Returns ``(out, lse)``."""
    import torch

    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    h = _hints(1, max_seqlen_k, num_splits)
    ws_ptr, ws_bytes, workspace = _workspace(lib, q, k_cache, block_table, h, workspace)
    d = [_desc(q), _desc(k_new), _desc(v_new), _desc(k_cache), _desc(v_cache), _desc(block_table),
         _desc(seqlens_k)]
    if rope is not None:
        r = _rope(rope.get("rotary_dim", 0), rope.get("base", 10000.0), rope.get("style", "neox"),
                  rope.get("pos_scale", 1.0))
        st = lib.attn_decode_append_paged_rope(*[_ref(x) for x in d], ctypes.c_float(scale), int(window),
                                               ctypes.byref(r), _ref(_desc(out)), _ref(_desc(lse)), ctypes.byref(h),
                                               ws_ptr, ws_bytes, _stream(q))
    elif window:
        st = lib.attn_decode_append_paged_window(*[_ref(x) for x in d], ctypes.c_float(scale), int(window),
                                                 _ref(_desc(out)), _ref(_desc(lse)), ctypes.byref(h), ws_ptr,
                                                 ws_bytes, _stream(q))
    else:
        st = lib.attn_decode_append_paged(*[_ref(x) for x in d], ctypes.c_float(scale), _ref(_desc(out)),
                                          _ref(_desc(lse)), ctypes.byref(h), ws_ptr, ws_bytes, _stream(q))
    _lib.check(st)
    return out, lse


def attn_decode_append_paged_fp8(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, seqlens_k,
                                 scale: float, out=None, lse=None, *, return_lse: bool = True, num_splits: int = 0,
                                 workspace=None, window: int = 0, _entry: str = "attn_decode_append_paged_fp8"):
    """The fused decode step over an FP8 cache: row b of ``k_new`` / ``v_new``
    (bf16) is quantized as ``kv_store_paged_fp8`` does into key
    ``seqlens_k[b] - 1`` (codes and scales) and query row b attends over the
    dequantized keys.  Returns ``(out, lse)``."""
    import torch

    lib = _lib.load()
    if out is None:
        out = torch.empty_like(q)
    if lse is None and return_lse:
        lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    h = _hints(1, 0, num_splits)
    ws_ptr, ws_bytes, workspace = _workspace(lib, q, k_cache, block_table, h, workspace)
    d = [_desc(x) for x in (q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, seqlens_k)]
    st = getattr(lib, _entry)(*[_ref(x) for x in d], ctypes.c_float(scale), int(window),
                              _ref(_desc(out)), _ref(_desc(lse)), ctypes.byref(h), ws_ptr, ws_bytes, _stream(q))
    _lib.check(st)
    return out, lse


def attn_decode_append_paged_int8(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table, seqlens_k,
                                  scale: float, out=None, lse=None, **kw):
    """The fused decode step over an INT8 cache (the new rows quantized as
    ``kv_store_paged_int8`` does); the arguments of
    ``attn_decode_append_paged_fp8``.  Returns ``(out, lse)``."""
    return attn_decode_append_paged_fp8(q, k_new, v_new, k_cache, v_cache, k_scale, v_scale, block_table,
                                        seqlens_k, scale, out, lse, _entry="attn_decode_append_paged_int8", **kw)


def attn_varlen_paged_plain(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, scale: float,
                            causal: bool, out, lse=None) -> None:
    """The plain ``attn_varlen_paged`` entry point (library-owned scratch)."""
    lib = _lib.load()
    d = [_desc(x) for x in (q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k)]
    st = lib.attn_varlen_paged(*[_ref(x) for x in d], ctypes.c_float(scale), int(bool(causal)),
                               _ref(_desc(out)), _ref(_desc(lse)), _stream(q))
    _lib.check(st)


def attn_varlen_paged_noalloc(q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k, scale: float,
                              causal: bool, out, lse=None) -> None:
    """``attn_varlen_paged_noalloc``: the plain call with the library's static
    scratch (nothing allocated; shapes needing more scratch are refused)."""
    lib = _lib.load()
    d = [_desc(x) for x in (q, k_cache, v_cache, block_table, cu_seqlens_q, seqlens_k)]
    st = lib.attn_varlen_paged_noalloc(*[_ref(x) for x in d], ctypes.c_float(scale), int(bool(causal)),
                                       _ref(_desc(out)), _ref(_desc(lse)), _stream(q))
    _lib.check(st)


def release_workspace() -> None:
    _lib.check(_lib.load().kvs_release_workspace())
