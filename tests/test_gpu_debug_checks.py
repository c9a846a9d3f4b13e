"""The debug library (libkvstore_debug.so, the C ABI built with KVS_DEBUG).

Its calls check the device-resident preconditions on the GPU before enqueuing
their kernels: cu_seqlens_q[0] = 0 and cu_seqlens_q[B] = T, 1 <= Lq_b <=
Lk_b <= 16 MB, every block-table entry the call reads in [0, NB), store
slots below 16 NB.  A violation returns KVS_ERR_INVALID naming it, and no
kernel of the call runs (the outputs keep their sentinel values).  Valid
calls give the release library's results bit for bit (the same kernels).
Every invalid input here is caught by that check, which reads only inside
the arrays whose shapes the host has validated.
"""
from __future__ import annotations

import contextlib

import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import attention_kv_store_amd._lib as L
    L.load()


@contextlib.contextmanager
def debug_library():
    """Route the binding's calls to the debug library for the block."""
    import attention_kv_store_amd._lib as L
    saved = L.load()
    L._lib = None
    try:
        yield L.load(L.DEBUG_LIB_PATH)
    finally:
        L._lib = saved


def _batch(seed=1900, window=0):
    from workloads import make_batch
    return make_batch(seed, [1, 17, 70, 1], [40, 17, 200, 2000], Hq=8, Hkv=2, D=64, dtype="bf16", causal=True,
                      window=window, name="debug-checks")


def _dev(b, table=None, cu=None, lens=None):
    from tests.gpu_side import to_device
    d = to_device(b)
    if table is not None:
        d.block_table = torch.from_numpy(table).cuda()
    if cu is not None:
        d.cu_seqlens_q = torch.from_numpy(cu).cuda()
    if lens is not None:
        d.seqlens_k = torch.from_numpy(lens).cuda()
    return d


def _attn(d, b, out):
    import attention_kv_store_amd as kvs
    return kvs.attn_varlen_paged(d.q, d.k_cache, d.v_cache, d.block_table, d.cu_seqlens_q, d.seqlens_k, b.scale, True,
                                 out=out, window=b.window)


def test_valid_calls_match_the_release_library():
    b = _batch()
    d = _dev(b)
    ref = torch.empty_like(d.q)
    _attn(d, b, ref)
    out = torch.full_like(d.q, float("nan"))
    with debug_library():
        _attn(d, b, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


@pytest.mark.parametrize("case", ["table_entry", "seqlens_k", "cu_last", "cu_first", "empty_sequence"])
def test_violations_are_refused_before_any_kernel(case):
    import attention_kv_store_amd as kvs
    b = _batch()
    table, cu, lens = b.block_table.copy(), b.cu_seqlens_q.copy(), b.k_lens.copy()
    if case == "table_entry":
        table[2, 5] = b.num_blocks + 7            # a block the call reads (sequence 2 has 13 blocks)
        msg = "block_table[2][5]"
    elif case == "seqlens_k":
        lens[1] = 16 * table.shape[1] + 1          # more keys than the table row can name
        msg = "seqlens_k[1]"
    elif case == "cu_last":
        cu[-1] = cu[-1] - 1
        msg = "cu_seqlens_q[B]"
    elif case == "cu_first":
        cu[0] = 1
        msg = "cu_seqlens_q[0]"
    else:
        cu[2] = cu[1]                              # sequence 1 left with no query row
        msg = "query rows"
    d = _dev(b, table=table, cu=cu, lens=lens)
    out = torch.full_like(d.q, float("nan"))
    with debug_library():
        with pytest.raises(kvs.KvsError, match="KVS_DEBUG") as ei:
            _attn(d, b, out)
    torch.cuda.synchronize()
    assert msg in str(ei.value), str(ei.value)
    assert torch.isnan(out.float()).all()          # nothing was written


def test_entries_outside_what_a_call_reads_are_not_checked():
    """Entries past a sequence's last block, and (under a window) below its
    first row's window, may hold anything."""
    b = _batch(window=33)
    table = b.block_table.copy()
    nb = (b.k_lens + 15) // 16
    for i in range(b.B):
        table[i, nb[i]:] = -5                       # past the last block
    table[3, 0] = 10 ** 6                           # sequence 3: 2000 keys, one row, window 33 -> block 0 unread
    d = _dev(b, table=table)
    ref_d = _dev(b)
    ref = torch.empty_like(d.q)
    _attn(ref_d, b, ref)
    out = torch.empty_like(d.q)
    with debug_library():
        _attn(d, b, out)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), ref.view(torch.int16))


def test_decode_step_and_stores_are_checked():
    import attention_kv_store_amd as kvs
    from workloads import make_batch
    b = make_batch(1910, [1, 1, 1], [5, 40, 300], Hq=8, Hkv=2, D=64, dtype="bf16")
    d = _dev(b)
    new = b.new_token_rows()
    kn = torch.from_numpy(b.k_tokens[new]).to(torch.bfloat16).cuda()
    vn = torch.from_numpy(b.v_tokens[new]).to(torch.bfloat16).cuda()
    table = b.block_table.copy()
    table[2, (300 - 1) // 16] = -1                  # the new key's own block
    bad = torch.from_numpy(table).cuda()
    before = d.k_cache.clone()
    with debug_library():
        with pytest.raises(kvs.KvsError, match=r"block_table\[2\]\[18\]"):
            kvs.attn_decode_append_paged(d.q, kn, vn, d.k_cache, d.v_cache, bad, d.seqlens_k, b.scale)
        slots = torch.tensor([3, 16 * b.num_blocks, -1], dtype=torch.int32, device="cuda")
        with pytest.raises(kvs.KvsError, match=r"slot_mapping\[1\]"):
            kvs.kv_store_paged(kn, vn, slots, d.k_cache, d.v_cache)
        # a valid step still runs
        kvs.attn_decode_append_paged(d.q, kn, vn, d.k_cache, d.v_cache, d.block_table, d.seqlens_k, b.scale)
    torch.cuda.synchronize()
    # the refused calls wrote nothing; the valid step wrote exactly the new rows
    diff = d.k_cache.view(torch.int16) != before.view(torch.int16)   # bitwise (unowned slots hold NaN)
    changed = diff.reshape(d.k_cache.shape[0] * 16, -1).any(dim=1).nonzero().flatten().cpu().numpy()
    assert set(changed.tolist()) <= set(b.slots[new].tolist())
