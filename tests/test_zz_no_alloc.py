"""The no-allocation entry point (attn_varlen_paged_noalloc) against the plain
attn_varlen_paged, through the C ABI: the same kernels, so the same bits, on
two calls in a row whose second is smaller (the static scratch keeps the
first call's contents), for decode batches (which use the scratch) and a
prefill batch (which does not)."""
from __future__ import annotations

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


def _both(batch, **kw):
    import attention_kv_store_amd as kvs
    from workloads.device import to_device
    db = to_device(batch)
    outs = []
    for fn in (kvs.attn_varlen_paged_plain, kvs.attn_varlen_paged_noalloc):
        out = torch.full_like(db.q, float("nan"))
        lse = torch.full((db.q.shape[0], db.q.shape[1]), float("nan"), dtype=torch.float32, device="cuda")
        fn(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q, db.seqlens_k, db.scale, db.causal,
           out, lse)
        torch.cuda.synchronize()
        outs.append((out.cpu(), lse.cpu()))
    return outs


def _same(a, b):
    (o1, l1), (o2, l2) = a, b
    assert torch.equal(o1.view(torch.int16) if o1.dtype == torch.bfloat16 else o1.view(torch.int32),
                       o2.view(torch.int16) if o2.dtype == torch.bfloat16 else o2.view(torch.int32))
    assert torch.equal(l1.view(torch.int32), l2.view(torch.int32))
    assert torch.isfinite(o2.float()).all()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_noalloc_matches_plain_two_calls(dtype):
    from workloads import make_batch, paged_decode_bf16
    # 1: the decode workload (64 rows, 32 / 8 heads, contexts up to 2048): split, scratch used
    if dtype == "bf16":
        big = paged_decode_bf16()
    else:
        rng = np.random.default_rng(3)
        k = [int(x) for x in rng.integers(128, 2049, size=64)]
        big = make_batch(3, [1] * 64, k, Hq=32, Hkv=8, D=64, dtype="fp32", causal=True)
    a, b = _both(big)
    _same(a, b)
    # 2: a smaller decode batch right after (fewer sequences, fewer KV heads)
    small = make_batch(4, [1] * 5, [1, 17, 300, 64, 1999], Hq=8, Hkv=2, D=128, dtype=dtype, causal=True)
    a, b = _both(small)
    _same(a, b)


def test_noalloc_prefill_and_against_oracle():
    from tests.gpu_side import to_f64
    from tests.oracle_side import oracle_attention
    from workloads import make_batch
    b = make_batch(5, [33, 5, 1], [50, 5, 40], Hq=8, Hkv=2, D=128, dtype="bf16", causal=True)
    plain, noalloc = _both(b)
    _same(plain, noalloc)
    ro, rl = oracle_attention(b)
    assert np.max(np.abs(to_f64(noalloc[0]) - ro)) <= 2e-2
    assert np.max(np.abs(to_f64(noalloc[1]) - rl)) <= 2e-2


def test_noalloc_refuses_shapes_beyond_its_scratch():
    import attention_kv_store_amd as kvs
    from attention_kv_store_amd._lib import KvsError
    from workloads import make_batch
    # 2048 sequences x 32 heads x D 128: the split partials exceed 16 MiB
    b = make_batch(6, [1] * 2048, [40] * 2048, Hq=32, Hkv=8, D=128, dtype="bf16", causal=True)
    q = torch.zeros(b.T, 32, 128, dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros(b.num_blocks, 16, 8, 128, dtype=torch.bfloat16, device="cuda")
    meta = [torch.from_numpy(x).cuda() for x in (b.block_table, b.cu_seqlens_q, b.k_lens)]
    out = torch.empty_like(q)
    with pytest.raises(KvsError, match="KVS_ERR_WORKSPACE"):
        kvs.attn_varlen_paged_noalloc(q, kc, kc, *meta, b.scale, True, out)
