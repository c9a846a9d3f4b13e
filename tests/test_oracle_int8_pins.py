"""Pins of the INT8 oracle against facts that do not come from it.

* codes written out by hand from the definition (nearest integer, ties to
  even, clamp to +-127);
* an independent scalar definition (Python's built-in round, which rounds
  halves to even, and min/max) over random values and every half-integer;
* the error bound of the per-row quantization (half a step of s) and its
  invariants (each nonzero row's largest magnitude becomes +-127);
* planted mistakes that these pins must catch.
"""
from __future__ import annotations

import inspect
import types

import numpy as np
import pytest

import oracle.int8 as oi8
from oracle.int8 import dequantize_pool_int8, int8_decode, int8_encode, kv_store_int8_oracle, quantize_rows_int8

# ---------------------------------------------------------------- I1 ------
HAND_CODES = [
    (0.0, 0), (0.49, 0), (0.5, 0), (1.5, 2), (2.5, 2), (-2.5, -2), (-0.5, 0), (3.5, 4),
    (126.5, 126), (127.0, 127), (127.49, 127), (127.5, 127), (300.0, 127), (-300.0, -127),
    (-127.5, -127), (-126.5, -126), (64.25, 64), (-64.75, -65),
]


@pytest.mark.parametrize("value,code", HAND_CODES)
def test_codes_by_hand(value, code):
    """Nearest integer; an exact half goes to the even neighbour (0.5 -> 0,
    1.5 -> 2, 2.5 -> 2, 126.5 -> 126); beyond +-127 the code saturates."""
    assert int(int8_encode(np.array([value]))[0]) == code


# ---------------------------------------------------------------- I2 ------
def _scalar_code(y: float) -> int:
    return int(max(-127, min(127, round(y))))   # built-in round: halves to even


def test_encode_matches_scalar_definition():
    rng = np.random.default_rng(0)
    halves = np.arange(-140, 141) + 0.5
    vals = np.concatenate([rng.uniform(-160, 160, 20000), halves, np.arange(-140, 141, dtype=np.float64)])
    mine = int8_encode(vals)
    ref = np.array([_scalar_code(float(v)) for v in vals])
    assert np.array_equal(mine.astype(np.int64), ref)


def test_decode_is_the_signed_byte():
    c = np.arange(256, dtype=np.int64).astype(np.uint8).view(np.int8)
    d = int8_decode(c)
    assert d[0] == 0 and d[127] == 127 and d[128] == -128 and d[255] == -1
    assert np.array_equal(d, np.where(np.arange(256) < 128, np.arange(256), np.arange(256) - 256))


# ---------------------------------------------------------------- I3 ------
def test_row_quantization_error_bound():
    """|code s - x| <= s / 2 (plus the fp32 rounding of x / s, 2^-24
    relative); each nonzero row's largest magnitude maps to +-127 exactly;
    an all-zero row has s = 0 and codes 0."""
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((50, 4, 64)) * np.exp2(rng.uniform(-8, 8, size=(50, 4, 1)))).astype(np.float32)
    x[3, 1] = 0.0
    codes, s = quantize_rows_int8(x)
    assert codes.dtype == np.int8 and s.dtype == np.float32
    assert s[3, 1] == 0 and not codes[3, 1].any()
    deq = codes.astype(np.float64) * s[..., None].astype(np.float64)
    xs = x.astype(np.float64)
    bound = 0.5 * s[..., None].astype(np.float64) * (1 + 2.0 ** -20) + 2.0 ** -22 * np.abs(xs)
    assert np.all(np.abs(deq - xs) <= bound)
    amax_code = np.max(np.abs(codes.astype(np.int64)), axis=-1)
    assert np.all(amax_code[s > 0] == 127)
    assert np.all(np.abs(codes.astype(np.int64)) <= 127)


def test_integer_rows_round_trip():
    """A row of integers whose largest magnitude is 127 has s = 1 and codes
    equal to the row."""
    rng = np.random.default_rng(5)
    x = rng.integers(-127, 128, size=(8, 2, 64)).astype(np.float32)
    x[..., 0] = 127.0
    codes, s = quantize_rows_int8(x)
    assert np.all(s == 1.0)
    assert np.array_equal(codes.astype(np.float32), x)


def test_store_scatters_codes_and_scales():
    rng = np.random.default_rng(4)
    T, Hkv, D, NB = 6, 2, 16, 2
    k = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    v = rng.standard_normal((T, Hkv, D)).astype(np.float32)
    slots = np.array([0, 17, -1, 31, 5, 16])
    kc = np.full((NB, 16, Hkv, D), -128, np.int8)
    sc = np.full((NB, Hkv, 16), np.nan, np.float32)
    kq, vq, ks, vs = kv_store_int8_oracle(k, v, slots, kc, kc, sc, sc)
    rk, rks = quantize_rows_int8(k)
    rv, rvs = quantize_rows_int8(v)
    for t, sl in enumerate(slots):
        if sl < 0:
            continue
        assert np.array_equal(kq[sl // 16, sl % 16], rk[t]) and np.array_equal(vq[sl // 16, sl % 16], rv[t])
        assert np.array_equal(ks[sl // 16, :, sl % 16], rks[t]) and np.array_equal(vs[sl // 16, :, sl % 16], rvs[t])
    assert np.isnan(dequantize_pool_int8(kq, ks)[0, 1]).all()   # slot 1 never written
    assert np.array_equal(dequantize_pool_int8(kq, ks)[1, 1], rk[1].astype(np.float64) * rks[1][:, None])


# ---------------------------------------------------------------- mutations -
MUTATIONS = {
    "ties away from zero": ("np.clip(np.rint(y), -I8_MAX, I8_MAX)", "np.clip(np.floor(y + 0.5), -I8_MAX, I8_MAX)"),
    "truncation": ("np.clip(np.rint(y), -I8_MAX, I8_MAX)", "np.clip(np.trunc(y), -I8_MAX, I8_MAX)"),
    "clamp to -128": ("np.clip(np.rint(y), -I8_MAX, I8_MAX)", "np.clip(np.rint(y), -128.0, I8_MAX)"),
    "scale for 128": ("scale = (amax / np.float32(I8_MAX))", "scale = (amax / np.float32(128.0))"),
    "unsigned decode": ("np.asarray(codes, dtype=np.int8).astype(np.float64)",
                        "np.asarray(codes, dtype=np.int8).view(np.uint8).astype(np.float64)"),
}


def _mutant(a, b):
    src = inspect.getsource(oi8)
    assert a in src, a
    mod = types.ModuleType("int8_mutant")
    exec(compile(src.replace(a, b), "int8_mutant", "exec"), mod.__dict__)
    return mod


def _battery(mod) -> bool:
    names = ("int8_encode", "int8_decode", "quantize_rows_int8")
    saved = {n: globals()[n] for n in names}
    globals().update({n: getattr(mod, n) for n in names})
    try:
        for value, code in HAND_CODES:
            test_codes_by_hand(value, code)
        test_encode_matches_scalar_definition()
        test_decode_is_the_signed_byte()
        test_row_quantization_error_bound()
        test_integer_rows_round_trip()
        return True
    except Exception:   # a wrong value or a crash: either way the mistake is caught
        return False
    finally:
        globals().update(saved)


def test_unmutated_int8_passes_battery():
    assert _battery(oi8)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_int8_mutation_is_caught(name):
    assert not _battery(_mutant(*MUTATIONS[name])), f"planted mistake '{name}' went unnoticed"
