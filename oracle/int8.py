"""INT8 quantized KV cache, numpy.  TEST INFRASTRUCTURE ONLY.

The pages name INT8 next to FP8 among the KV dtypes a kernel dispatch must
cover (Transformer 추론 커널 (3/10), §19) and list quantized KV in the
edge-case matrix (§24); they fix no encoding.  Reading (R19), the symmetric
per-row form that matches the FP8 reading's group and scale layout:

* Group: the D values of one token row of one KV head share one fp32 scale
  s = absmax / 127 (s = 0 for an all-zero row, whose codes are 0).
* Code: x / s taken in fp32, rounded to the nearest integer (ties to even)
  and clamped to [-127, 127]; stored as a two's-complement byte.
* Value: code * s.  Attention runs over these dequantized K and V.
"""
from __future__ import annotations

import numpy as np

I8_MAX = 127.0


def int8_encode(y) -> np.ndarray:
    """Nearest integer of each finite value (ties to even), clamped to +-127."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("int8_encode takes finite values")
    return np.clip(np.rint(y), -I8_MAX, I8_MAX).astype(np.int8)


def int8_decode(codes) -> np.ndarray:
    """float64 value of each code (a plain signed integer)."""
    return np.asarray(codes, dtype=np.int8).astype(np.float64)


def quantize_rows_int8(x):
    """Codes and scales of ``x [T, H, D]``: one fp32 scale per (t, h) row."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)                                  # exact
    scale = (amax / np.float32(I8_MAX)).astype(np.float32)               # fp32 division
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x32 / safe[..., None]).astype(np.float32)                       # fp32 division
    codes = int8_encode(y)
    codes = np.where(scale[..., None] > 0, codes, 0).astype(np.int8)
    return codes, scale


def kv_store_int8_oracle(k_new, v_new, slot_mapping, k_codes, v_codes, k_scales, v_scales, block_size: int = 16):
    """Quantize new rows and scatter them: returns updated copies of the code
    pools ``[NB, 16, Hkv, D]`` (int8) and scale pools ``[NB, Hkv, 16]`` (fp32).
    Negative slots are skipped."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    kq, ks = quantize_rows_int8(k_new)
    vq, vs = quantize_rows_int8(v_new)
    out = [np.array(a, copy=True) for a in (k_codes, v_codes, k_scales, v_scales)]
    live = slots >= 0
    s = slots[live]
    if np.unique(s).size != s.size:
        raise ValueError("duplicate slots")
    blk, row = s // block_size, s % block_size
    out[0][blk, row] = kq[live]
    out[1][blk, row] = vq[live]
    out[2][blk, :, row] = ks[live]
    out[3][blk, :, row] = vs[live]
    return tuple(out)


def dequantize_pool_int8(codes, scales) -> np.ndarray:
    """float64 values of a code pool ``[NB, 16, Hkv, D]`` with scales ``[NB, Hkv, 16]``."""
    sc = np.asarray(scales, dtype=np.float64).transpose(0, 2, 1)[..., None]   # [NB, 16, Hkv, 1]
    return int8_decode(codes) * sc
