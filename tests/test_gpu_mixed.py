"""Mixed batches in one launch (no decode_tail hint): the sequences with one
query row run as split decode ranges and the others as prefill items, in the
same grid, the split formed in-kernel.  Every row against the oracle; the
dispatch string names the path taken."""
from __future__ import annotations

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu

TOL = {"fp32": 1e-5, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_kv_store_amd._lib as L
    L.load()


def _check(batch, out, lse, rows=None):
    from tests.gpu_side import to_f64
    from tests.oracle_side import oracle_attention

    ro, rl = oracle_attention(batch, rows=rows)
    go, gl = to_f64(out), to_f64(lse)
    if rows is not None:
        ro, rl, go, gl = ro[rows], rl[rows], go[rows], gl[rows]
    tol = TOL[batch.dtype]
    assert np.isfinite(go).all() and np.isfinite(gl).all(), "NaN/Inf in GPU output"
    eo = np.max(np.abs(go - ro))
    el = np.max(np.abs(gl - rl))
    print(f"[{batch.name or 'case'}] max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= tol, f"out max-abs {eo} > {tol}"
    assert el <= tol, f"lse max-abs {el} > {tol}"


def _mk(seed, q_lens, k_lens, **kw):
    from workloads import make_batch
    return make_batch(seed, q_lens, k_lens, **kw)


# decode rows first, last and in between; contexts of 1 key, exactly one
# block, one block + 1, and long ones that are cut into several pieces
MQ = [1, 40, 1, 1, 17, 1, 64, 1, 1, 2]
MK = [700, 40, 1, 2000, 100, 16, 300, 129, 17, 5]


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heads", [(32, 8), (8, 8), (128, 8), (32, 16), (16, 4)])
@pytest.mark.parametrize("wide", [False, True])
def test_mixed_one_launch_matches_oracle(D, heads, wide):
    """wide: a block table wide enough that the prefill part takes 8-wave
    workgroups (one KV head's K/V for a full table row exceeds 4 MiB); else
    4-wave ones, two per CU.  KV heads must come in whole groups of the
    workgroup's waves."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_attention, to_device
    Hq, Hkv = heads
    cols = (4 << 20) // (16 * D * 4) + 1 if wide else 0
    b = _mk(2100 + D + Hq + Hkv, MQ, MK, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", causal=True,
            extra_table_cols=cols, name=f"mixed-D{D}-{Hq}x{Hkv}-{'wide' if wide else 'narrow'}")
    print("case", b.name, flush=True)
    out, lse = run_attention(to_device(b))
    disp = kvs.last_dispatch()
    if wide and Hkv % 8:
        assert disp.startswith("prefill_bf16"), disp
    else:
        assert disp.startswith("mixed_bf16"), disp
        assert f"waves/wg={8 if wide else 4} " in disp, disp
    _check(b, out, lse)


@pytest.mark.parametrize("window", [1, 33, 512])
def test_mixed_sliding_window(window):
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_attention, to_device
    b = _mk(2200 + window, MQ, MK, Hq=32, Hkv=8, D=128, dtype="bf16", causal=True, window=window,
            name=f"mixed-window{window}")
    print("case", b.name, flush=True)
    out, lse = run_attention(to_device(b), window=window)
    assert kvs.last_dispatch().startswith("mixed_bf16"), kvs.last_dispatch()
    _check(b, out, lse)


def test_mixed_many_sequences():
    """300 sequences, 290 of them decode rows over contexts of 1..3000 keys and
    10 prompts of 2..150 rows, in shuffled order: every row."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_attention, to_device
    rng = np.random.default_rng(2300)
    q = np.ones(300, np.int64)
    pre = rng.choice(300, size=10, replace=False)
    q[pre] = rng.integers(2, 151, size=10)
    k = rng.integers(1, 3001, size=300)
    k = np.maximum(k, q)
    b = _mk(2300, list(q), list(k), Hq=32, Hkv=8, D=64, dtype="bf16", causal=True, name="mixed-300")
    print("case", b.name, flush=True)
    out, lse = run_attention(to_device(b))
    assert kvs.last_dispatch().startswith("mixed_bf16"), kvs.last_dispatch()
    _check(b, out, lse)


def test_mixed_long_decode_rows_need_many_ranges():
    """Two decode rows over 131072 and 50000 keys next to a short prompt: the
    decode part needs several ranges for its table window whatever the
    estimated costs say."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_attention, to_device
    b = _mk(2400, [1, 20, 1], [131072, 20, 50000], Hq=16, Hkv=8, D=64, dtype="bf16", causal=True,
            name="mixed-long-decode")
    print("case", b.name, flush=True)
    out, lse = run_attention(to_device(b))
    assert kvs.last_dispatch().startswith("mixed_bf16"), kvs.last_dispatch()
    _check(b, out, lse)


def test_mixed_without_workspace_runs_in_the_prefill_kernel():
    """A workspace smaller than the mixed plan needs: the prefill kernel serves
    every sequence (no error), with the same results to the tolerance."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_attention, to_device
    b = _mk(2500, MQ, MK, Hq=32, Hkv=8, D=128, dtype="bf16", causal=True, name="mixed-small-ws")
    print("case", b.name, flush=True)
    ws = torch.zeros(256, dtype=torch.uint8, device="cuda")
    out, lse = run_attention(to_device(b), workspace=ws)
    assert kvs.last_dispatch().startswith("prefill_bf16"), kvs.last_dispatch()
    _check(b, out, lse)


def test_mixed_repeated_calls_bitwise_and_noalloc():
    """Two calls in a row give the same bits (the merge order is fixed), and
    so does the no-allocation entry point, which runs the same kernel."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_attention, to_device
    from workloads import mixed_prefill_decode_bf16
    b = mixed_prefill_decode_bf16()
    print("case", b.name, flush=True)
    db = to_device(b)
    o1, l1 = run_attention(db)
    assert kvs.last_dispatch().startswith("mixed_bf16"), kvs.last_dispatch()
    o2, l2 = run_attention(db)
    o3 = torch.empty_like(o1)
    l3 = torch.empty_like(l1)
    kvs.attn_varlen_paged_noalloc(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q, db.seqlens_k,
                                  db.scale, True, out=o3, lse=l3)
    torch.cuda.synchronize()
    assert kvs.last_dispatch().startswith("mixed_bf16"), kvs.last_dispatch()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    assert torch.equal(o1, o3) and torch.equal(l1, l3)


def test_mixed_shapes_outside_the_mixed_kernel():
    """fp32, and KV heads not in whole groups of 4: the prefill kernel serves
    the mixed batch (correct, one launch)."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_attention, to_device
    for dtype, Hq, Hkv in (("fp32", 32, 8), ("bf16", 8, 2)):
        b = _mk(2600 + Hkv, MQ, MK, Hq=Hq, Hkv=Hkv, D=64, dtype=dtype, causal=True, name=f"mixed-{dtype}-{Hkv}")
        print("case", b.name, flush=True)
        out, lse = run_attention(to_device(b))
        assert kvs.last_dispatch().startswith("prefill_"), kvs.last_dispatch()
        _check(b, out, lse)
