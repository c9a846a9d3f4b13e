"""Rotary position embedding before the KV store, numpy float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages place a RoPE elementwise transform on Q and K right before attention
and fuse it with the KV-cache write in a layer's step list (Transformer 추론 커널
(3/10), §1 and §2: "RoPE + KV cache store"), and list the RoPE variant, its
scaling and a position offset among the dispatch axes and the edge-case matrix
(same page, §19 and §24).  They give no formula.  Reading (R17): the rotary
embedding of Su et al., "RoFormer: Enhanced Transformer with Rotary Position
Embedding" (2021), section 3.2: the first ``rotary_dim`` dims of each head are
cut into rotary_dim / 2 pairs, and pair i of a token at position p is turned
by the angle a = (p / pos_scale) * theta_i with theta_i = base^(-2 i / rotary_dim):

    x1' = x1 cos a - x2 sin a,     x2' = x2 cos a + x1 sin a.

Pairs are either (x[2i], x[2i + 1]) ("interleaved", the paper's layout) or
(x[i], x[i + rotary_dim / 2]) ("neox", the half-split layout); dims at or past
rotary_dim are left as they are.  pos_scale > 1 is linear position scaling
(positions divided by the factor); position offsets are carried by the
explicit per-token positions.
"""
from __future__ import annotations

import numpy as np

NEOX, INTERLEAVED = 0, 1


def rope_angles(positions, rotary_dim: int, base: float, pos_scale: float = 1.0) -> np.ndarray:
    """Angles a[t, i] = (positions[t] / pos_scale) * base^(-2 i / rotary_dim), float64."""
    if rotary_dim < 2 or rotary_dim % 2:
        raise ValueError("rotary_dim must be even and >= 2")
    if not (base > 0 and pos_scale > 0):
        raise ValueError("base and pos_scale must be positive")
    i = np.arange(rotary_dim // 2, dtype=np.float64)
    theta = float(base) ** (-2.0 * i / rotary_dim)
    p = np.asarray(positions, dtype=np.float64) / float(pos_scale)
    return p[:, None] * theta[None, :]


def pair_index(D: int, rotary_dim: int, style: int):
    """(first, second) element indices of the rotary pairs of one head."""
    if rotary_dim > D:
        raise ValueError("rotary_dim must not exceed the head dim")
    h = rotary_dim // 2
    if style == NEOX:
        return np.arange(h), np.arange(h) + h
    if style == INTERLEAVED:
        return 2 * np.arange(h), 2 * np.arange(h) + 1
    raise ValueError("style must be NEOX (0) or INTERLEAVED (1)")


def apply_rope(x, positions, *, rotary_dim: int, base: float, style: int = NEOX,
               pos_scale: float = 1.0) -> np.ndarray:
    """RoPE of ``x [T, H, D]`` with token t at ``positions[t]``; float64 result."""
    x = np.asarray(x, dtype=np.float64)
    if x.ndim != 3 or np.asarray(positions).shape != (x.shape[0],):
        raise ValueError("x must be [T, H, D] with one position per token")
    a = rope_angles(positions, rotary_dim, base, pos_scale)      # [T, rotary_dim / 2]
    c, s = np.cos(a)[:, None, :], np.sin(a)[:, None, :]          # broadcast over heads
    i1, i2 = pair_index(x.shape[2], rotary_dim, style)
    y = x.copy()
    x1, x2 = x[:, :, i1], x[:, :, i2]
    y[:, :, i1] = x1 * c - x2 * s
    y[:, :, i2] = x2 * c + x1 * s
    return y


def kv_store_rope_oracle(q, k_new, v_new, positions, slot_mapping, k_cache, v_cache, *, rotary_dim: int,
                         base: float, style: int = NEOX, pos_scale: float = 1.0, round_to=None):
    """The "RoPE + KV cache store" step: returns ``(q', k_cache', v_cache')``
    with q' = RoPE(q) and RoPE(k_new) / v_new scattered into the pools at
    ``slot_mapping`` (negative slots skipped), all float64.

    ``round_to`` (optional) maps the rotated q and k to the storage precision
    before they are returned / stored (e.g. bf16 round-to-nearest-even).
    """
    from .store import kv_store_oracle

    kw = dict(rotary_dim=rotary_dim, base=base, style=style, pos_scale=pos_scale)
    qr = apply_rope(q, positions, **kw)
    kr = apply_rope(k_new, positions, **kw)
    if round_to is not None:
        qr, kr = round_to(qr), round_to(kr)
    kc, vc = kv_store_oracle(kr, np.asarray(v_new, dtype=np.float64), slot_mapping,
                             np.asarray(k_cache, dtype=np.float64), np.asarray(v_cache, dtype=np.float64))
    return qr, kc, vc
