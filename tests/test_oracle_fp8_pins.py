"""Pins of the FP8 (E4M3) oracle against facts that do not come from it.

* torch's own float8_e4m3fn conversion on the CPU (an independent
  implementation of the OCP E4M3 format): all 256 codes decoded, and encoding
  of values across the whole range, subnormals and exact midpoints included;
* codes written out by hand from the format definition;
* the format's error bound for the per-row quantization;
* planted mistakes that these pins must catch.
"""
from __future__ import annotations

import inspect
import types

import numpy as np
import pytest

import oracle.fp8 as of8
from oracle.fp8 import dequantize_pool, e4m3_decode, e4m3_encode, kv_store_fp8_oracle, quantize_rows

torch = pytest.importorskip("torch")


def _torch_decode_all():
    return torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(y):
    return torch.from_numpy(np.asarray(y, dtype=np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _range_values(seed=0, n=20000):
    """float32 values over the whole E4M3 range: random magnitudes, every
    representable value, and every midpoint between neighbours."""
    rng = np.random.default_rng(seed)
    mags = np.exp2(rng.uniform(-12, np.log2(448.0), size=n))
    reps = np.unique(np.abs(e4m3_decode(np.arange(0x7F))))
    mids = (reps[:-1] + reps[1:]) / 2
    v = np.concatenate([mags, reps, mids, [0.0, 448.0]])
    v = np.concatenate([v, -v]).astype(np.float32)
    return v[np.abs(v) <= 448.0]


# ---------------------------------------------------------------- F1 ------
def test_decode_table_matches_torch():
    mine = e4m3_decode(np.arange(256))
    ref = _torch_decode_all()
    assert np.array_equal(np.isnan(mine), np.isnan(ref))
    ok = ~np.isnan(ref)
    assert np.array_equal(mine[ok], ref[ok])
    assert np.isnan(mine[[0x7F, 0xFF]]).all() and int(np.isnan(mine).sum()) == 2


# ---------------------------------------------------------------- F2 ------
def test_encode_matches_torch_everywhere():
    """Nearest value, ties to even, over random values, all representable
    values and all midpoints (the tie cases) in [-448, 448]."""
    y = _range_values()
    mine = e4m3_encode(y)
    ref = _torch_encode(y)
    # zeros: both keep the sign
    assert np.array_equal(mine, ref)


# ---------------------------------------------------------------- F3 ------
HAND_CODES = [
    (0.0, 0x00), (-0.0, 0x80), (1.0, 0x38), (-2.5, 0xC2), (448.0, 0x7E), (-448.0, 0xFE),
    (2.0 ** -9, 0x01), (2.0 ** -6, 0x08), (7 * 2.0 ** -9, 0x07), (240.0, 0x77),
    (1.0625, 0x38),            # midpoint of 1 and 1.125: to the even mantissa 0
    (1.1875, 0x3A),            # midpoint of 1.125 and 1.25: to the even mantissa 2
    (1.5 * 2.0 ** -9, 0x02),   # subnormal midpoint of 1 and 2 (x 2^-9): to 2
    (0.5 * 2.0 ** -9, 0x00),   # half the smallest subnormal: to 0 (even)
    (500.0, 0x7E),             # beyond the largest finite value: saturates
]


@pytest.mark.parametrize("value,code", HAND_CODES)
def test_codes_by_hand(value, code):
    """Codes from the format: 1.0 = 2^0 is exponent field 7 (0x38); 2.5 = 1.25 x 2^1
    is field 8 mantissa 2 with the sign (0xC2); 448 = 1.75 x 2^8 is field 15
    mantissa 6 (0x7E); 2^-9 is the smallest subnormal (0x01); 240 = 1.875 x 2^7
    is field 14 mantissa 7 (0x77)."""
    assert int(e4m3_encode(np.array([value]))[0]) == code


def test_every_code_round_trips():
    c = np.array([i for i in range(256) if (i & 0x7F) != 0x7F])
    assert np.array_equal(e4m3_encode(e4m3_decode(c)), c.astype(np.uint8))


# ---------------------------------------------------------------- F4 ------
def test_row_quantization_error_bound():
    """Each row's largest magnitude maps to +-448; every value is within half a
    step of the E4M3 grid at its magnitude: |deq - x| <= 2^-4 |x| in the normal
    range (3 mantissa bits) and <= 2^-10 s in the subnormal range, plus the
    fp32 rounding of x / s (2^-24 relative)."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((50, 4, 64)) * np.exp2(rng.uniform(-8, 8, size=(50, 4, 1)))).astype(np.float32)
    x[3, 1] = 0.0                                  # an all-zero row
    codes, s = quantize_rows(x)
    assert s[3, 1] == 0 and not codes[3, 1].any()
    deq = e4m3_decode(codes) * s[..., None].astype(np.float64)
    xs = x.astype(np.float64)
    amax_code = np.max(np.abs(e4m3_decode(codes)), axis=-1)
    assert np.all(amax_code[s > 0] == 448.0)
    sub = np.abs(xs) < 2.0 ** -6 * s[..., None]
    bound = np.where(sub, 2.0 ** -10 * s[..., None], 2.0 ** -4 * np.abs(xs)) + 2.0 ** -22 * np.abs(xs)
    assert np.all(np.abs(deq - xs) <= bound)


def test_store_scatters_codes_and_scales():
    rng = np.random.default_rng(4)
    T, Hkv, D, NB = 6, 2, 16, 2
    k = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    slots = np.array([0, 17, -1, 31, 5, 16])
    kc = np.full((NB, 16, Hkv, D), 0x7F, np.uint8)
    sc = np.full((NB, Hkv, 16), np.nan, np.float32)
    kq, vq, ks, vs = kv_store_fp8_oracle(k, v, slots, kc, kc, sc, sc)
    rk, rks = quantize_rows(k)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        assert np.array_equal(kq[sl // 16, sl % 16], rk[t])
        assert np.array_equal(ks[sl // 16, :, sl % 16], rks[t])
    # slot 1 of block 0 was not written; dequantizing it gives NaN
    assert np.isnan(dequantize_pool(kq, ks)[0, 1]).all()
    full = dequantize_pool(kq, ks)
    assert np.array_equal(full[1, 1], e4m3_decode(rk[1]) * rks[1][:, None].astype(np.float64))


# ---------------------------------------------------------------- mutations -
MUTATIONS = {
    "ties away from zero": ("m_norm = np.rint((f - 1.0) * 8.0)", "m_norm = np.floor((f - 1.0) * 8.0 + 0.5)"),
    "exponent bias 8": ("code_norm = (e + 7) * 8 + m_norm", "code_norm = (e + 8) * 8 + m_norm"),
    "subnormal step 2^-10": ("m_sub = np.rint(a * 512.0)", "m_sub = np.rint(a * 1024.0)"),
    "no saturation": ("a = np.minimum(np.abs(y), E4M3_MAX)", "a = np.abs(y)"),
    "decode bias 8": ("np.exp2(e.astype(np.float64) - 7.0)", "np.exp2(e.astype(np.float64) - 8.0)"),
    "scale for 240": ("scale = (amax / np.float32(E4M3_MAX))", "scale = (amax / np.float32(240.0))"),
    "truncating mantissa": ("m_norm = np.rint((f - 1.0) * 8.0)", "m_norm = np.floor((f - 1.0) * 8.0)"),
}


def _mutant(a, b):
    src = inspect.getsource(of8)
    assert a in src, a
    mod = types.ModuleType("fp8_mutant")
    exec(compile(src.replace(a, b), "fp8_mutant", "exec"), mod.__dict__)
    return mod


def _battery(mod) -> bool:
    names = ("e4m3_decode", "e4m3_encode", "quantize_rows")
    saved = {n: globals()[n] for n in names}
    globals().update({n: getattr(mod, n) for n in names})
    try:
        for value, code in HAND_CODES:
            test_codes_by_hand(value, code)
        test_decode_table_matches_torch()
        test_encode_matches_torch_everywhere()
        test_every_code_round_trips()
        test_row_quantization_error_bound()
        return True
    except Exception:   # a wrong value or a crash: either way the mistake is caught
        return False
    finally:
        globals().update(saved)


def test_unmutated_fp8_passes_battery():
    assert _battery(of8)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_fp8_mutation_is_caught(name):
    assert not _battery(_mutant(*MUTATIONS[name])), f"planted mistake '{name}' went unnoticed"
