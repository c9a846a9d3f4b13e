"""FP8 (E4M3) quantized KV cache, numpy.  TEST INFRASTRUCTURE ONLY.

The pages list FP8 and INT8 KV among the dtypes, and a quantized KV layout
among the layouts, that a kernel dispatch must cover (Transformer 추론 커널
(3/10), §19); quantized KV is an entry of the edge-case test matrix (§24); and
the quantization group and scale layout must be what the kernel expects (§7).
They fix no format, group or scale.  Reading (R18):

* Format: E4M3 of the OCP 8-bit floating point specification (OFP8, 2023):
  1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits.  Exponent field 0
  holds the subnormals m * 2^-9; the largest finite value is 448
  (S.1111.110); S.1111.111 is NaN; there are no infinities.
* Group: the D values of one token row of one KV head share one fp32 scale
  s = absmax / 448 (s = 0 for an all-zero row, whose codes are 0).
* Code: x / s taken in fp32, saturated at +-448, rounded to the nearest E4M3
  value, ties to even.
* Value: decode(code) * s.  Attention runs over these dequantized K and V.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """float64 value of each E4M3 code (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return sign * mag


def e4m3_encode(y) -> np.ndarray:
    """Nearest E4M3 code of each finite value (ties to even), saturating at
    +-448.  The sign of zero is kept (-0.0 -> 0x80)."""
    y = np.asarray(y, dtype=np.float64)
    if not np.all(np.isfinite(y)):
        raise ValueError("e4m3_encode takes finite values")
    a = np.minimum(np.abs(y), E4M3_MAX)
    sign = np.where(np.signbit(y), 0x80, 0)
    # subnormal range: a < 2^-6 is m * 2^-9 with m = round(a * 2^9) (8 -> 2^-6, the smallest normal)
    m_sub = np.rint(a * 512.0)
    # normal range: a = f * 2^e with f in [1, 2): mantissa = round((f - 1) * 8); 8 carries into e
    fr, ex = np.frexp(np.where(a > 0, a, 1.0))        # a = fr * 2^ex, fr in [0.5, 1)
    f, e = 2.0 * fr, ex - 1
    m_norm = np.rint((f - 1.0) * 8.0)
    code_norm = (e + 7) * 8 + m_norm
    code = np.where(a < 2.0 ** -6, m_sub, code_norm)   # a <= 448 keeps it <= 0x7E
    return (code.astype(np.int64) | sign).astype(np.uint8)


def quantize_rows(x):
    """Codes and scales of ``x [T, H, D]``: one fp32 scale per (t, h) row."""
    x32 = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(x32), axis=-1)                                  # exact
    scale = (amax / np.float32(E4M3_MAX)).astype(np.float32)             # fp32 division
    safe = np.where(scale > 0, scale, np.float32(1.0)).astype(np.float32)
    y = (x32 / safe[..., None]).astype(np.float32)                       # fp32 division
    codes = e4m3_encode(y)
    codes = np.where(scale[..., None] > 0, codes, 0).astype(np.uint8)
    return codes, scale


def kv_store_fp8_oracle(k_new, v_new, slot_mapping, k_codes, v_codes, k_scales, v_scales, block_size: int = 16):
    """Quantize new rows and scatter them: returns updated copies of the code
    pools ``[NB, 16, Hkv, D]`` (uint8) and scale pools ``[NB, Hkv, 16]`` (fp32).
    Negative slots are skipped."""
    slots = np.asarray(slot_mapping, dtype=np.int64)
    kq, ks = quantize_rows(k_new)
    vq, vs = quantize_rows(v_new)
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


def dequantize_pool(codes, scales) -> np.ndarray:
    """float64 values of a code pool ``[NB, 16, Hkv, D]`` with scales ``[NB, Hkv, 16]``."""
    sc = np.asarray(scales, dtype=np.float64).transpose(0, 2, 1)[..., None]   # [NB, 16, Hkv, 1]
    return e4m3_decode(codes) * sc
