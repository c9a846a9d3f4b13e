"""Sliding-window attention on the HIP path against the CPU oracle.

Window W: the row at position p sees keys max(0, p - W + 1) .. p (a decode row
sits at position Lk - 1).  Same tolerances as the other parity tests: max-abs
1e-5 (fp32 inputs) and 2e-2 (bf16 inputs) on out and lse.  Windows are chosen
around the 16-key page and the 64-key (bf16) / 32-key (fp32) prefill tile:
1, 2, 15, 16, 17, 31, 33, 63, 64, 65, plus wider ones.
"""
from __future__ import annotations

import dataclasses

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

from tests.test_gpu_parity import _check, _mk, _pool_matches_oracle  # noqa: E402


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_kv_store_amd._lib as L
    L.load()


def _run(batch, **kw):
    from tests.gpu_side import run_attention, to_device
    db = to_device(batch)
    return run_attention(db, window=batch.window, **kw)


# prefill / extend rows: prompts, cached prefixes across several tiles, a
# one-row sequence inside a prefill batch, a ragged tail
PREFILL_Q = [1, 17, 64, 65, 100, 200, 30, 129]
PREFILL_K = [1, 17, 64, 65, 300, 200, 500, 129]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", [1, 2, 16, 17, 63, 64, 65, 130, 1000])
def test_window_prefill(dtype, D, W):
    b = _mk(700 + W, PREFILL_Q, PREFILL_K, Hq=8, Hkv=2, D=D, dtype=dtype, window=W,
            name=f"win-prefill-{dtype}-{D}-W{W}")
    out, lse = _run(b)
    _check(b, out, lse)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("heads", [(4, 4), (12, 4), (6, 2), (32, 8)])
@pytest.mark.parametrize("W", [15, 33])
def test_window_prefill_heads(dtype, heads, W):
    Hq, Hkv = heads
    b = _mk(720 + Hq + W, PREFILL_Q, PREFILL_K, Hq=Hq, Hkv=Hkv, D=128, dtype=dtype, window=W,
            name=f"win-heads-{dtype}-{Hq}/{Hkv}-W{W}")
    out, lse = _run(b)
    _check(b, out, lse)


DECODE_K = [1, 2, 15, 16, 17, 33, 100, 500, 2000, 64, 65, 31]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("W", [1, 16, 17, 100, 1000])
@pytest.mark.parametrize("splits", [0, 1, 7, 64])
def test_window_decode(dtype, D, W, splits):
    b = _mk(740 + W, [1] * len(DECODE_K), DECODE_K, Hq=8, Hkv=2, D=D, dtype=dtype, window=W,
            name=f"win-decode-{dtype}-{D}-W{W}-s{splits}")
    out, lse = _run(b, num_splits=splits)
    _check(b, out, lse)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("W", [1, 17, 100])
@pytest.mark.parametrize("splits", [0, 7])
def test_window_decode_append(dtype, W, splits):
    """The fused store + windowed decode equals the stored cache and the
    oracle's windowed attention."""
    from tests.gpu_side import run_append, to_device_before_append
    b = _mk(760 + W, [1] * len(DECODE_K), DECODE_K, Hq=8, Hkv=2, D=128, dtype=dtype, window=W,
            name=f"win-append-{dtype}-W{W}-s{splits}")
    db, kn, vn = to_device_before_append(b)
    out, lse = run_append(db, kn, vn, num_splits=splits, window=W)
    _check(b, out, lse)
    _pool_matches_oracle(b, db.k_cache, db.v_cache)


def _poison_below_window(batch):
    """Point every table entry whose block holds only keys below the first
    row's window start at the batch's poison block (NaN on the device)."""
    tbl = batch.block_table.copy()
    n = 0
    for s in range(batch.B):
        c = int(batch.k_lens[s]) - int(batch.q_lens[s])
        klo = max(0, c - batch.window + 1)
        for j in range(klo // 16):
            tbl[s, j] = batch.poison_block
            n += 1
    assert n > 0
    return dataclasses.replace(batch, block_table=tbl)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("W", [16, 40, 100])
def test_window_blocks_below_are_never_read(dtype, W):
    """Entries of blocks wholly below every row's window may name any block (a
    caller may have freed them): pointed at a NaN block, the result is finite
    and equals the oracle's, for the prefill and the decode path."""
    from tests.gpu_side import run_attention, to_device
    pre = _mk(780 + W, [40, 5, 70], [300, 200, 400], Hq=8, Hkv=2, D=128, dtype=dtype, window=W,
              name=f"win-poison-prefill-{dtype}-W{W}")
    dec = _mk(790 + W, [1] * 6, [300, 17, 33, 1000, 129, 64], Hq=8, Hkv=2, D=128, dtype=dtype, window=W,
              name=f"win-poison-decode-{dtype}-W{W}")
    for b in (pre, dec):
        db = to_device(b)   # the pool is filled through the real table first
        pb = _poison_below_window(b)
        db.block_table = torch.from_numpy(pb.block_table).cuda()
        for splits in ((0,) if b is pre else (0, 7)):
            out, lse = run_attention(db, window=W, num_splits=splits)
            _check(b, out, lse)


def test_window_wider_than_context_matches_causal():
    """A window at least as wide as every context reproduces the causal call
    (same kernels' results up to the masked path taken on more tiles)."""
    from tests.gpu_side import run_attention, to_device, to_f64
    b = _mk(799, PREFILL_Q, PREFILL_K, Hq=8, Hkv=2, D=128, dtype="fp32")
    db = to_device(b)
    o0, l0 = run_attention(db)
    o1, l1 = run_attention(db, window=max(PREFILL_K))
    assert np.max(np.abs(to_f64(o0) - to_f64(o1))) <= 1e-6
    assert np.max(np.abs(to_f64(l0) - to_f64(l1))) <= 1e-6


@pytest.mark.parametrize("name", ["sliding_window_decode_bf16", "sliding_window_prefill_bf16"])
def test_window_named_workload(name):
    from workloads import NAMED
    b = NAMED[name]()
    out, lse = _run(b)
    _check(b, out, lse)   # every row
