"""Pins of the RoPE oracle (oracle/rope.py) against facts that do not come from it.

Reading pinned (RoFormer, section 3.2): pair i of a token at position p turns by
a = (p / pos_scale) * base^(-2 i / rotary_dim), x1' = x1 cos a - x2 sin a,
x2' = x2 cos a + x1 sin a; pairs (2i, 2i+1) ("interleaved") or (i, i + rd/2)
("neox").  The pins are closed forms with the angles written out by hand,
invariants of rotations, and planted mistakes that each pin set must catch.
"""
from __future__ import annotations

import inspect
import math
import types

import numpy as np
import pytest

import oracle.rope as orope
from oracle.rope import INTERLEAVED, NEOX, apply_rope, kv_store_rope_oracle

TOL = 1e-13


def _x(seed, T=5, H=3, D=16):
    return np.random.default_rng(seed).standard_normal((T, H, D))


# ---------------------------------------------------------------- R1 ------
@pytest.mark.parametrize("style", [NEOX, INTERLEAVED])
def test_position_zero_is_identity(style):
    x = _x(1)
    y = apply_rope(x, np.zeros(5, np.int64), rotary_dim=16, base=10000.0, style=style)
    assert np.array_equal(x, y)


# ---------------------------------------------------------------- R2 ------
@pytest.mark.parametrize("p", [1, 2, 7, -3, 1000])
def test_two_dims_is_the_plane_rotation(p):
    """D = 2: theta_0 = 1, so e1 goes to (cos p, sin p) and e2 to (-sin p, cos p)
    -- a counter-clockwise turn by p radians (the paper's R matrix)."""
    x = np.array([[[1.0, 0.0], [0.0, 1.0], [3.0, -2.0]]])
    for style in (NEOX, INTERLEAVED):
        y = apply_rope(x, np.array([p]), rotary_dim=2, base=10000.0, style=style)[0]
        c, s = math.cos(p), math.sin(p)
        assert np.max(np.abs(y[0] - [c, s])) <= TOL
        assert np.max(np.abs(y[1] - [-s, c])) <= TOL
        assert np.max(np.abs(y[2] - [3 * c + 2 * s, -2 * c + 3 * s])) <= TOL


# ---------------------------------------------------------------- R3 ------
def test_frequency_schedule_by_hand():
    """D = rotary_dim = 4, base 100: theta = (1, 100^(-1/2) = 0.1).  At p = 10 the
    first pair turns by 10 rad and the second by 1 rad; neox pairs are (0, 2) and
    (1, 3), interleaved pairs (0, 1) and (2, 3)."""
    p = 10
    c0, s0, c1, s1 = math.cos(10.0), math.sin(10.0), math.cos(1.0), math.sin(1.0)
    eye = np.eye(4)[None]                      # [1, 4, 4]: head k holds e_k
    yn = apply_rope(eye, np.array([p]), rotary_dim=4, base=100.0, style=NEOX)[0]
    want_n = np.array([[c0, 0, s0, 0], [0, c1, 0, s1], [-s0, 0, c0, 0], [0, -s1, 0, c1]])
    assert np.max(np.abs(yn - want_n)) <= TOL
    yi = apply_rope(eye, np.array([p]), rotary_dim=4, base=100.0, style=INTERLEAVED)[0]
    want_i = np.array([[c0, s0, 0, 0], [-s0, c0, 0, 0], [0, 0, c1, s1], [0, 0, -s1, c1]])
    assert np.max(np.abs(yi - want_i)) <= TOL


def test_linear_scaling_by_hand():
    """pos_scale 4 at p = 8 is the angle of p = 2: D = 2 turns by exactly 2 rad."""
    y = apply_rope(np.array([[[1.0, 0.0]]]), np.array([8]), rotary_dim=2, base=10000.0, pos_scale=4.0)[0, 0]
    assert np.max(np.abs(y - [math.cos(2.0), math.sin(2.0)])) <= TOL


# ---------------------------------------------------------------- R4-R8 ---
@pytest.mark.parametrize("style", [NEOX, INTERLEAVED])
def test_rotation_invariants(style):
    """Each pair keeps its length; <R(m) q, R(n) k> depends on m - n only; R(-p)
    undoes R(p); R(n) R(m) = R(m + n)."""
    D, rd = 32, 24
    q, k = _x(2, T=6, H=2, D=D), _x(3, T=6, H=2, D=D)
    m = np.array([0, 5, 17, 100, 4095, 40000])
    n = np.array([3, 5, 2, 999, 7, 39990])
    kw = dict(rotary_dim=rd, base=10000.0, style=style)
    i1, i2 = orope.pair_index(D, rd, style)
    qm = apply_rope(q, m, **kw)
    assert np.max(np.abs(np.hypot(qm[..., i1], qm[..., i2]) - np.hypot(q[..., i1], q[..., i2]))) <= 1e-12
    for shift in (1, 77, 12345):
        a = np.einsum("thd,thd->th", apply_rope(q, m, **kw), apply_rope(k, n, **kw))
        b = np.einsum("thd,thd->th", apply_rope(q, m + shift, **kw), apply_rope(k, n + shift, **kw))
        assert np.max(np.abs(a - b)) <= 1e-9
    assert np.max(np.abs(apply_rope(apply_rope(q, m, **kw), -m, **kw) - q)) <= 1e-12
    assert np.max(np.abs(apply_rope(apply_rope(q, m, **kw), n, **kw) - apply_rope(q, m + n, **kw))) <= 1e-9


def test_interleaved_is_neox_after_a_permutation():
    """Moving element 2i to slot i and 2i + 1 to slot i + rd/2 turns the
    interleaved layout into the neox one."""
    D, rd = 16, 16
    x = _x(4, D=D)
    perm = np.concatenate([np.arange(0, rd, 2), np.arange(1, rd, 2)])
    pos = np.array([0, 1, 9, 300, 77777])
    yi = apply_rope(x, pos, rotary_dim=rd, base=500.0, style=INTERLEAVED)
    yn = apply_rope(x[..., perm], pos, rotary_dim=rd, base=500.0, style=NEOX)
    assert np.max(np.abs(yi[..., perm] - yn)) <= TOL


def test_partial_rotary_dim_keeps_the_tail():
    """rotary_dim < D: dims >= rotary_dim are copied bit for bit and the first
    rotary_dim dims are the rotation of a head of that width."""
    x = _x(5, D=32)
    pos = np.array([1, 2, 3, 400, 5000])
    for style in (NEOX, INTERLEAVED):
        y = apply_rope(x, pos, rotary_dim=16, base=10000.0, style=style)
        assert np.array_equal(y[..., 16:], x[..., 16:])
        assert np.array_equal(y[..., :16], apply_rope(x[..., :16], pos, rotary_dim=16, base=10000.0, style=style))


def test_complex_multiplication():
    """The interleaved pairs as complex numbers z = x1 + i x2 are multiplied by
    e^(i a) (the paper's complex form)."""
    x = _x(6, D=8)
    pos = np.array([0, 3, 50, 1000, 123456])
    y = apply_rope(x, pos, rotary_dim=8, base=10000.0, style=INTERLEAVED)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = np.array([1.0, 10000 ** -0.25, 10000 ** -0.5, 10000 ** -0.75])
    w = z * np.exp(1j * pos[:, None, None] * theta[None, None, :])
    assert np.max(np.abs(y[..., 0::2] - w.real)) <= 1e-10
    assert np.max(np.abs(y[..., 1::2] - w.imag)) <= 1e-10


def test_store_writes_rotated_k_and_plain_v():
    """The fused step stores RoPE(k) and v at their slots (negative slots
    skipped) and returns RoPE(q)."""
    T, Hq, Hkv, D = 4, 4, 2, 16
    rng = np.random.default_rng(7)
    q, k, v = rng.standard_normal((T, Hq, D)), rng.standard_normal((T, Hkv, D)), rng.standard_normal((T, Hkv, D))
    pos = np.array([5, 6, 7, 100])
    slots = np.array([3, -1, 40, 17])
    kc = np.full((4, 16, Hkv, D), np.nan)
    qr, kc2, vc2 = kv_store_rope_oracle(q, k, v, pos, slots, kc, kc.copy(), rotary_dim=16, base=10000.0)
    kw = dict(rotary_dim=16, base=10000.0)
    assert np.array_equal(qr, apply_rope(q, pos, **kw))
    kr = apply_rope(k, pos, **kw)
    for t, s in enumerate(slots):
        if s >= 0:
            assert np.array_equal(kc2[s // 16, s % 16], kr[t])
            assert np.array_equal(vc2[s // 16, s % 16], v[t])
    assert np.isnan(kc2[0, 1]).all()   # slot 1 was not written


# ---------------------------------------------------------------- mutations -
MUTATIONS = {
    "sign of the sine": ("y[:, :, i1] = x1 * c - x2 * s", "y[:, :, i1] = x1 * c + x2 * s"),
    "second output sign": ("y[:, :, i2] = x2 * c + x1 * s", "y[:, :, i2] = x2 * c - x1 * s"),
    "frequency exponent": ("(-2.0 * i / rotary_dim)", "(-1.0 * i / rotary_dim)"),
    "scaling multiplies": ("/ float(pos_scale)", "* float(pos_scale)"),
    "neox pairs swapped for interleaved": ("return np.arange(h), np.arange(h) + h", "return 2 * np.arange(h), 2 * np.arange(h) + 1"),
    "cos and sin swapped": ("c, s = np.cos(a)[:, None, :], np.sin(a)[:, None, :]", "s, c = np.cos(a)[:, None, :], np.sin(a)[:, None, :]"),
    "exponent from D not rotary_dim": ("rope_angles(positions, rotary_dim, base, pos_scale)", "rope_angles(positions, x.shape[2], base, pos_scale)"),
}


def _mutant(a, b):
    src = inspect.getsource(orope)
    assert a in src, a
    mod = types.ModuleType("rope_mutant")
    exec(compile(src.replace(a, b), "rope_mutant", "exec"), mod.__dict__)
    return mod


def _battery(mod) -> bool:
    saved = globals()["apply_rope"], globals()["orope"]
    globals()["apply_rope"], globals()["orope"] = mod.apply_rope, mod
    try:
        for fn, args in ((test_two_dims_is_the_plane_rotation, (7,)), (test_frequency_schedule_by_hand, ()),
                         (test_linear_scaling_by_hand, ()), (test_interleaved_is_neox_after_a_permutation, ()),
                         (test_partial_rotary_dim_keeps_the_tail, ())):
            fn(*args)
        return True
    except Exception:   # a wrong value or a crash: either way the mistake is caught
        return False
    finally:
        globals()["apply_rope"], globals()["orope"] = saved


def test_unmutated_rope_passes_battery():
    assert _battery(orope)


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_rope_mutation_is_caught(name):
    assert not _battery(_mutant(*MUTATIONS[name])), f"planted mistake '{name}' went unnoticed"
