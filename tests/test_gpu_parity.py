"""HIP path vs the CPU oracle, element by element, through the C ABI.

Tolerances (max-abs, on both out and lse): 1e-5 for fp32 inputs, 2e-2 for
bf16 inputs (fp32 accumulation inside the kernels).  The store, the one-hot
probes and the indexing are bit-exact.
"""
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


def _mk(seed, q_lens, k_lens, **kw):
    from workloads import make_batch
    return make_batch(seed, q_lens, k_lens, **kw)


def _check(batch, out, lse, rows=None, tol=None):
    from tests.gpu_side import to_f64
    from tests.oracle_side import oracle_attention

    ro, rl = oracle_attention(batch, rows=rows)
    go, gl = to_f64(out), to_f64(lse)
    if rows is not None:
        ro, rl, go, gl = ro[rows], rl[rows], go[rows], gl[rows]
    tol = TOL[batch.dtype] if tol is None else tol
    assert np.isfinite(go).all() and np.isfinite(gl).all(), "NaN/Inf in GPU output"
    eo = np.max(np.abs(go - ro))
    el = np.max(np.abs(gl - rl))
    print(f"[{batch.name or 'case'}] max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= tol, f"out max-abs {eo} > {tol}"
    assert el <= tol, f"lse max-abs {el} > {tol}"


def _run(batch, **kw):
    from tests.gpu_side import run_attention, to_device
    db = to_device(batch)
    return run_attention(db, **kw)


# ------------------------------------------------------------------ store --
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_store_bitwise(dtype):
    from tests.gpu_side import to_device
    from tests.oracle_side import oracle_pool
    b = _mk(201, [17, 9, 40], [33, 9, 80], Hq=8, Hkv=2, D=64, dtype=dtype, extra_blocks=5)
    db = to_device(b)
    kc, vc = oracle_pool(b, dtype=np.float32)
    bits = np.uint32 if dtype == "fp32" else np.uint16
    for dev, ref in ((db.k_cache, kc), (db.v_cache, vc)):
        got = dev.cpu()
        if dtype == "bf16":
            got_bits = got.view(torch.int16).numpy().view(np.uint16)
            ref_bits = (ref.view(np.uint32) >> 16).astype(np.uint16)
        else:
            got_bits = got.numpy().view(np.uint32)
            ref_bits = ref.view(np.uint32)
        # NaN poison has one bit pattern on each side; compare owned rows bitwise
        owned = ~np.isnan(ref)
        assert np.array_equal(got_bits[owned], ref_bits[owned])
        assert np.isnan(got.float().numpy()[~owned]).all()


def test_store_negative_slots_skip():
    import attention_kv_store_amd as kvs
    kc = torch.zeros(4, 16, 2, 64, dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    kn = torch.randn(5, 2, 64, device="cuda").to(torch.bfloat16)
    vn = torch.randn(5, 2, 64, device="cuda").to(torch.bfloat16)
    slots = torch.tensor([3, -1, 63, -5, 17], dtype=torch.int32, device="cuda")
    kvs.kv_store_paged(kn, vn, slots, kc, vc)
    torch.cuda.synchronize()
    flat_k = kc.view(-1, 2, 64)
    for t, s in enumerate([3, -1, 63, -5, 17]):
        if s >= 0:
            assert torch.equal(flat_k[s], kn[t])
    touched = {3, 63, 17}
    for s in range(64):
        if s not in touched:
            assert flat_k[s].abs().sum().item() == 0


# ------------------------------------------------------------- tiny fp32 ---
def test_tiny_varlen_fp32():
    from workloads import tiny_varlen_fp32
    b = tiny_varlen_fp32()
    out, lse = _run(b)
    _check(b, out, lse)


# --------------------------------------------------------- edge matrix ----
EDGE_LENS = [1, 15, 16, 17, 31, 32, 33, 63, 64, 65, 100]


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("heads", [(4, 2), (8, 2), (4, 4), (12, 4), (6, 2)])
def test_prefill_edge_lengths(dtype, D, heads):
    Hq, Hkv = heads
    lens = [l for l in EDGE_LENS if l > 1]
    b = _mk(300 + D + Hq, lens, lens, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, causal=True, name=f"edge-{dtype}-{D}-{Hq}/{Hkv}")
    out, lse = _run(b)
    _check(b, out, lse)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("causal", [True, False])
def test_extend_with_cached_prefix(dtype, causal):
    q = [1, 5, 16, 17, 40, 64, 3, 130]
    c = [0, 11, 16, 15, 100, 3, 200, 60]
    b = _mk(411, q, [a + x for a, x in zip(q, c)], Hq=8, Hkv=2, D=128, dtype=dtype, causal=causal,
            name=f"extend-{dtype}-{causal}")
    out, lse = _run(b)
    _check(b, out, lse)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_batch_of_one_and_long_table(dtype):
    b = _mk(421, [200], [333], Hq=4, Hkv=1, D=64, dtype=dtype, causal=True, extra_table_cols=7, name="b1")
    out, lse = _run(b)
    _check(b, out, lse)


def test_shared_prefix_blocks():
    """Several table rows name the same physical blocks (a shared prefix)."""
    b = _mk(431, [20, 7, 33], [84, 71, 97], Hq=8, Hkv=2, D=128, dtype="bf16", causal=True,
            shared_prefix_blocks=3, name="shared-prefix")
    out, lse = _run(b)
    _check(b, out, lse)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("scale", [-0.11, 0.0, 0.9])
@pytest.mark.parametrize("decode", [False, True])
def test_scale_sign_and_size(dtype, scale, decode):
    """Negative, zero and large score scales.  A zero scale weighs the visible
    keys uniformly (masked keys must still get none); a large one makes row
    maxima jump by many powers of two between key tiles."""
    if decode:
        k = [1, 17, 300, 1000, 64]
        q = [1] * len(k)
    else:
        q = [1, 33, 70, 130, 64]
        k = [1, 38, 110, 130, 200]
    b = _mk(601, q, k, Hq=8, Hkv=2, D=64, dtype=dtype, causal=True, scale=scale,
            name=f"scale{scale}-{dtype}-{'dec' if decode else 'pre'}")
    out, lse = _run(b)
    # The fp32 bound is set for scale 1/sqrt(D), where scaled scores are O(1);
    # the rounding of the fp32 dot product q.k is multiplied by |scale|, so the
    # bound grows with |scale| * sqrt(D) beyond that.
    tol = TOL[dtype] * max(1.0, abs(scale) * 8.0) if dtype == "fp32" else None
    _check(b, out, lse, tol=tol)


@pytest.mark.parametrize("B", [65, 130, 300])
def test_prefill_many_sequences(B):
    """More than 64 sequences: the tile map searches the batch in several
    64-way levels."""
    rng = np.random.default_rng(700 + B)
    q = [int(x) for x in rng.integers(1, 41, size=B)]
    c = [int(x) for x in rng.integers(0, 25, size=B)]
    b = _mk(700 + B, q, [a + x for a, x in zip(q, c)], Hq=8, Hkv=2, D=64, dtype="bf16", causal=True,
            name=f"prefill-B{B}")
    out, lse = _run(b)
    _check(b, out, lse)


_ORDER_CASES = {
    # name: (B, rows range, cached range, Hq, Hkv, D, dtype, causal); rows drawn per sequence
    "b64_causal": (64, (1, 200), (0, 300), 8, 2, 64, "bf16", True),
    "b65_causal": (65, (1, 200), (0, 300), 8, 2, 64, "bf16", True),
    "b64_noncausal": (64, (1, 120), (0, 200), 8, 2, 64, "bf16", False),
    "b200_noncausal": (200, (1, 60), (0, 100), 8, 2, 64, "bf16", False),
    "b256_causal": (256, (1, 80), (0, 150), 8, 2, 64, "bf16", True),
    "b257_causal": (257, (1, 80), (0, 150), 8, 2, 64, "bf16", True),
    "fp32_one_head_group": (20, (1, 150), (0, 400), 4, 4, 128, "fp32", True),
    "six_head_groups": (24, (1, 160), (0, 250), 6, 2, 64, "bf16", True),
}


@pytest.mark.parametrize("case", sorted(_ORDER_CASES) + ["same_rows_other_prefixes", "one_long_prefix", "with_decode_rows",
                                  "window_37", "window_300_fp32", "window_huge"])
def test_prefill_heaviest_first_order(case):
    """Batches of up to 256 unequal sequences take their items heaviest
    first, ranked in-kernel from the staged lengths (each lane holding
    sequences l, l + 64, ...); 257 sequences, or sequences all of one shape,
    keep the plain order.  Head
    groups fewer than the XCDs, one-row sequences of a mixed launch and a
    long cached prefix (many key-tile levels) included, and windows (the
    cost capped at the most key tiles a window item spans); every row
    against the oracle."""
    window = 0
    if case in _ORDER_CASES:
        B, (qa, qb), (ca, cb), Hq, Hkv, D, dtype, causal = _ORDER_CASES[case]
        rng = np.random.default_rng(900 + B + Hq)
        q = [int(x) for x in rng.integers(qa, qb + 1, size=B)]
        k = [a + int(x) for a, x in zip(q, rng.integers(ca, cb + 1, size=B))]
    elif case == "same_rows_other_prefixes":
        q, k = [64] * 12, [64 + 37 * i for i in range(12)]
        Hq, Hkv, D, dtype, causal = 8, 2, 128, "bf16", True
    elif case == "one_long_prefix":
        q, k = [100, 17, 400, 2, 64], [8100, 17, 3400, 72, 64]
        Hq, Hkv, D, dtype, causal = 8, 2, 64, "bf16", True
    elif case.startswith("window"):
        rng = np.random.default_rng(960)
        q = [int(x) for x in rng.integers(1, 300, size=30)]
        k = [a + int(x) for a, x in zip(q, rng.integers(0, 700, size=30))]
        window = {"window_37": 37, "window_300_fp32": 300, "window_huge": 2**31 - 1}[case]
        Hq, Hkv, D, dtype, causal = 8, 2, 64, "fp32" if "fp32" in case else "bf16", True
    else:
        q = [1, 90, 1, 1, 33, 1, 250, 1, 7, 1]
        k = [300, 90, 17, 1000, 100, 64, 700, 5, 7, 2000]
        Hq, Hkv, D, dtype, causal = 8, 2, 64, "bf16", True
    b = _mk(950, q, k, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, causal=causal, window=window, name=f"order-{case}")
    out, lse = _run(b, window=window) if window else _run(b)
    _check(b, out, lse)


# --------------------------------------------------------------- decode ---
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("splits", [0, 1, 2, 7, 64])
def test_decode_forced_splits(dtype, D, splits):
    k = [1, 15, 16, 17, 64, 65, 300, 1000, 2048, 129]
    b = _mk(500 + D + splits, [1] * len(k), k, Hq=8, Hkv=2, D=D, dtype=dtype, causal=True,
            name=f"decode-{dtype}-{D}-s{splits}")
    out, lse = _run(b, num_splits=splits)
    _check(b, out, lse)


@pytest.mark.parametrize("heads", [(32, 8), (4, 4), (16, 1), (6, 3)])
def test_decode_group_sizes(heads):
    Hq, Hkv = heads
    k = [5, 77, 160, 1024, 513]
    b = _mk(551 + Hq, [1] * len(k), k, Hq=Hq, Hkv=Hkv, D=64, dtype="bf16", causal=True, name=f"decode-G{Hq}/{Hkv}")
    out, lse = _run(b)
    _check(b, out, lse)


@pytest.mark.parametrize("B", [65, 300, 1000])
def test_decode_many_sequences(B):
    """More than 64 sequences: the block prefix spans several waves."""
    rng = np.random.default_rng(800 + B)
    k = [int(x) for x in rng.integers(1, 400, size=B)]
    b = _mk(800 + B, [1] * B, k, Hq=8, Hkv=2, D=64, dtype="bf16", causal=True, name=f"decode-B{B}")
    out, lse = _run(b)
    _check(b, out, lse)


@pytest.mark.parametrize("splits", [0, 64, 300])
def test_decode_split_results_reproducible(splits):
    """Split sequences are merged by whichever workgroup finishes last; the
    merge groups a sequence's pieces the same way whoever merges it, so
    repeated calls give the same bits."""
    from tests.gpu_side import to_device
    rng = np.random.default_rng(571)
    k = [int(x) for x in rng.integers(1, 3000, size=40)]
    b = _mk(571 + splits, [1] * len(k), k, Hq=8, Hkv=2, D=64, dtype="bf16", causal=True)
    db = to_device(b)
    import attention_kv_store_amd as kvs
    first = None
    for _ in range(6):
        out, lse = kvs.attn_varlen_paged(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q,
                                         db.seqlens_k, db.scale, True, num_splits=splits)
        torch.cuda.synchronize()
        if first is None:
            first = (out.clone(), lse.clone())
            _check(b, out, lse)
        else:
            assert torch.equal(out, first[0]) and torch.equal(lse, first[1])


@pytest.mark.parametrize("fused", [False, True])
def test_decode_table_paths_agree(fused):
    """A small batch stages its whole block table; a table that is not 16-byte
    aligned, or too large, takes the per-range window instead.  The paths give
    the same bits, and both match the oracle."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_append, to_device, to_device_before_append
    k = [1, 15, 16, 17, 64, 65, 300, 1000, 2048, 129, 777, 31]
    b = _mk(611, [1] * len(k), k, Hq=8, Hkv=2, D=64, dtype="bf16", causal=True, name="table-paths")
    if fused:
        db, kn, vn = to_device_before_append(b)
    else:
        db = to_device(b)
    res = {}
    base = db.block_table
    shifted = torch.empty(base.numel() + 1, dtype=torch.int32, device="cuda")[1:].view(base.shape)
    shifted.copy_(base)
    wide = torch.zeros(base.shape[0], 2048, dtype=torch.int32, device="cuda")
    wide[:, :base.shape[1]] = base
    for name, tab, want in (("aligned", base, "table=whole"), ("shifted", shifted, "table=window"),
                            ("wide", wide, "table=window")):
        if fused:
            out, lse = kvs.attn_decode_append_paged(db.q, kn, vn, db.k_cache, db.v_cache, tab, db.seqlens_k,
                                                    db.scale, num_splits=64)
        else:
            out, lse = kvs.attn_varlen_paged(db.q, db.k_cache, db.v_cache, tab, db.cu_seqlens_q, db.seqlens_k,
                                             db.scale, True, num_splits=64)
        torch.cuda.synchronize()
        assert want in kvs.last_dispatch(), kvs.last_dispatch()
        _check(b, out, lse)
        res[name] = (out, lse)
    for name in ("shifted", "wide"):
        assert torch.equal(res[name][0], res["aligned"][0]) and torch.equal(res[name][1], res["aligned"][1])


def test_workspace_reused_across_shapes():
    """One workspace, zeroed once, serves decode calls of different batch sizes,
    head counts and split counts in any order (the split counters sit at a
    fixed place and every call leaves them at zero)."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_append, to_device, to_device_before_append
    rng = np.random.default_rng(591)
    cases = []
    for i, (B, Hq, Hkv) in enumerate([(10, 8, 2), (64, 32, 8), (3, 4, 1), (200, 8, 2)]):
        k = [int(x) for x in rng.integers(1, 1500, size=B)]
        cases.append(_mk(591 + i, [1] * B, k, Hq=Hq, Hkv=Hkv, D=64, dtype="bf16", causal=True, name=f"ws-{i}"))
    ws = torch.zeros(64 << 20, dtype=torch.uint8, device="cuda")
    order = [(0, 7), (1, 64), (0, 300), (2, 0), (3, 32), (1, 5), (0, 7), (3, 512), (2, 64), (1, 0)]
    for n, (ci, splits) in enumerate(order):
        b = cases[ci]
        if n % 3 == 2:
            db, kn, vn = to_device_before_append(b)
            out, lse = run_append(db, kn, vn, num_splits=splits, workspace=ws)
        else:
            db = to_device(b)
            out, lse = kvs.attn_varlen_paged(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q,
                                             db.seqlens_k, db.scale, True, num_splits=splits, workspace=ws)
            torch.cuda.synchronize()
        _check(b, out, lse)


def test_decode_plain_entry_point():
    """The plain call (library-owned scratch) gives the same bits as _ex."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import to_device
    k = [100, 900, 2000, 33]
    b = _mk(561, [1] * 4, k, Hq=8, Hkv=2, D=64, dtype="bf16", causal=True)
    db = to_device(b)
    out1, lse1 = kvs.attn_varlen_paged(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q,
                                       db.seqlens_k, db.scale, True)
    out2 = torch.empty_like(out1)
    lse2 = torch.empty_like(lse1)
    kvs.attn_varlen_paged_plain(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q,
                                db.seqlens_k, db.scale, True, out2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)
    kvs.release_workspace()


# ------------------------------------------------ fused decode append ----
def _pool_matches_oracle(batch, k_cache, v_cache):
    """Every slot the batch owns holds the oracle store's bits; the rest stay NaN."""
    from tests.gpu_side import cache_bits
    from tests.oracle_side import oracle_pool
    kc, vc = oracle_pool(batch, dtype=np.float32)
    for dev, ref in ((k_cache, kc), (v_cache, vc)):
        got = cache_bits(dev)
        ref_bits = (ref.view(np.uint32) >> 16).astype(np.uint16) if batch.dtype == "bf16" else ref.view(np.uint32)
        owned = ~np.isnan(ref)
        assert np.array_equal(got[owned], ref_bits[owned])
        assert np.isnan(dev.float().cpu().numpy()[~owned]).all()


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("splits", [0, 1, 7, 64])
def test_decode_append_matches_store_then_attention(dtype, D, splits):
    """The fused call equals kv_store_paged then attn_varlen_paged: out and lse
    against the oracle (whose pool holds the new rows), the written cache bit for
    bit, and the same bits as the two-call path."""
    from tests.gpu_side import run_append, to_device, to_device_before_append
    k = [1, 15, 16, 17, 64, 65, 300, 1000, 2048, 129]
    b = _mk(900 + D + splits, [1] * len(k), k, Hq=8, Hkv=2, D=D, dtype=dtype, causal=True,
            name=f"append-{dtype}-{D}-s{splits}")
    db, kn, vn = to_device_before_append(b)
    out, lse = run_append(db, kn, vn, num_splits=splits)
    _check(b, out, lse)
    _pool_matches_oracle(b, db.k_cache, db.v_cache)
    out2, lse2 = _run(b, num_splits=splits)
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    ref = to_device(b)
    assert torch.equal(db.k_cache.view(torch.uint8), ref.k_cache.view(torch.uint8))
    assert torch.equal(db.v_cache.view(torch.uint8), ref.v_cache.view(torch.uint8))


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_decode_append_steps(dtype):
    """Several decode steps in a row, each appending one token per sequence and
    crossing block boundaries; after every step out/lse match the oracle, and
    after the last the pool equals the oracle store of all tokens."""
    import dataclasses

    from tests.gpu_side import run_append, to_device_before_append
    from tests.oracle_side import oracle_attention, oracle_pool
    base = np.array([0, 14, 15, 16, 31, 47, 200])
    S = 5
    final = _mk(950, [1] * len(base), base + S, Hq=8, Hkv=2, D=64, dtype=dtype, causal=True,
                name=f"append-steps-{dtype}")
    # the device pool starts with tokens 0 .. base-1 of every sequence
    db, _, _ = to_device_before_append(_prefix_batch(final, base + 1))
    pool = oracle_pool(final)
    rng = np.random.default_rng(951)
    dt = db.q.dtype
    for s in range(S):
        lens = (base + s + 1).astype(np.int32)
        q = rng.standard_normal(final.q.shape, dtype=np.float32)
        if dtype == "bf16":
            q = torch.from_numpy(q).to(torch.bfloat16).float().numpy()
        rows = final.cu_seqlens_k[:-1] + lens - 1
        kn = torch.from_numpy(final.k_tokens[rows]).to(dt).cuda()
        vn = torch.from_numpy(final.v_tokens[rows]).to(dt).cuda()
        db.q = torch.from_numpy(q).to(dt).cuda()
        db.seqlens_k = torch.from_numpy(lens).cuda()
        out, lse = run_append(db, kn, vn)
        step = dataclasses.replace(final, q=q, k_lens=lens, name=f"append-steps-{dtype}-{s}")
        ro, rl = oracle_attention(step, pool=pool)
        go, gl = out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
        assert np.isfinite(go).all() and np.isfinite(gl).all()
        eo, el = np.max(np.abs(go - ro)), np.max(np.abs(gl - rl))
        print(f"[{step.name}] max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
        assert eo <= TOL[dtype] and el <= TOL[dtype]
    _pool_matches_oracle(final, db.k_cache, db.v_cache)


def _prefix_batch(batch, lens):
    """The same batch cut to ``lens`` keys per sequence (one new row each),
    drawn from the same token rows and slots."""
    import dataclasses
    lens = np.asarray(lens, np.int64)
    keep = np.concatenate([np.arange(int(batch.cu_seqlens_k[b]), int(batch.cu_seqlens_k[b]) + int(lens[b]))
                           for b in range(batch.B)])
    cu_k = np.zeros(batch.B + 1, np.int64)
    cu_k[1:] = np.cumsum(lens)
    return dataclasses.replace(batch, k_lens=lens.astype(np.int32), cu_seqlens_k=cu_k.astype(np.int32),
                               k_tokens=batch.k_tokens[keep], v_tokens=batch.v_tokens[keep],
                               slots=batch.slots[keep])


def test_decode_append_named_workload():
    """The 64-sequence bf16 decode workload through the fused call."""
    from tests.gpu_side import run_append, to_device_before_append
    from workloads import NAMED
    b = NAMED["paged_decode_bf16"]()
    db, kn, vn = to_device_before_append(b)
    out, lse = run_append(db, kn, vn)
    _check(b, out, lse)
    _pool_matches_oracle(b, db.k_cache, db.v_cache)


# ------------------------------------------------------- graph runner -----
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("window", [0, 37])
def test_decode_graph_runner_buckets(dtype, window):
    """Decode steps replayed from per-bucket graphs: a batch padded to the next
    bucket with dummy rows in a reserved block gives the oracle's out / lse
    for its real rows and writes exactly their new rows into the cache; then
    a smaller batch through another bucket, one token longer."""
    import dataclasses

    from attention_kv_store_amd.graph_runner import DecodeGraphRunner
    from tests.gpu_side import cache_bits, to_device_before_append
    from tests.oracle_side import oracle_attention, oracle_pool
    rng = np.random.default_rng(621)
    # step 2 appends key k + 1: keep it inside the sequence's last allocated
    # block (k + 1 not a multiple of 16), as a block manager would otherwise
    # hand out a new block first
    k = [int(x) - (1 if (int(x) + 1) % 16 == 0 else 0) for x in rng.integers(2, 900, size=37)]
    b = _mk(621, [1] * 37, [x + 1 for x in k], Hq=8, Hkv=2, D=64, dtype=dtype, causal=True,
            extra_table_cols=3, name=f"runner-{dtype}", window=window)
    # pool holding keys 0 .. k-1 of every sequence; step 1 appends key k
    db, _, _ = to_device_before_append(_prefix_batch(b, np.array(k) + 1))
    runner = DecodeGraphRunner(db.k_cache, db.v_cache, b.poison_block, [16, 32, 64], b.MB, Hq=8,
                               scale=b.scale, num_splits=7, window=window)
    before = cache_bits(db.k_cache).copy()
    rows = b.cu_seqlens_k[:-1] + np.array(k)
    dt = db.q.dtype
    kn = torch.from_numpy(b.k_tokens[rows]).to(dt).cuda()
    vn = torch.from_numpy(b.v_tokens[rows]).to(dt).cuda()
    out, lse = runner.step(db.q, kn, vn, db.block_table, torch.from_numpy((np.array(k) + 1).astype(np.int32)).cuda())
    torch.cuda.synchronize()
    step1 = dataclasses.replace(b, k_lens=(np.array(k) + 1).astype(np.int32))
    pool = oracle_pool(b)
    ro, rl = oracle_attention(step1, pool=pool)
    go, gl = out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)
    eo, el = np.max(np.abs(go - ro)), np.max(np.abs(gl - rl))
    print(f"[runner-{dtype} B=37 -> bucket 64] max|dout|={eo:.3e} max|dlse|={el:.3e}", flush=True)
    assert eo <= TOL[dtype] and el <= TOL[dtype]
    # the cache: the 37 new rows written, nothing else outside the reserved block changed
    after = cache_bits(db.k_cache)
    changed = np.argwhere((after != before).reshape(b.num_blocks * 16, -1).any(axis=1)).ravel()
    written = set(int(x) for x in b.slots[rows])
    assert set(int(x) for x in changed) - {b.poison_block * 16} <= written
    kc, _ = oracle_pool(_prefix_batch(b, np.array(k) + 1), dtype=np.float32)
    flat = after.reshape(b.num_blocks * 16, -1)
    ref = (kc.view(np.uint32) >> 16).astype(np.uint16) if dtype == "bf16" else kc.view(np.uint32)
    ref = ref.reshape(b.num_blocks * 16, -1)
    for sl in written:
        assert np.array_equal(flat[sl], ref[sl])
    # a second step: the first 10 sequences, one key longer, through bucket 16
    k2 = np.array(k[:10]) + 1
    b2 = _mk(622, [1] * 10, list(k2 + 1), Hq=8, Hkv=2, D=64, dtype=dtype, causal=True, window=window)
    q2 = torch.from_numpy(b2.q).to(dt).cuda()
    kn2 = torch.from_numpy(b2.k_tokens[b2.new_token_rows()]).to(dt).cuda()
    vn2 = torch.from_numpy(b2.v_tokens[b2.new_token_rows()]).to(dt).cuda()
    table2 = db.block_table[:10]
    # the new row of sequence s lands at key k2[s]; its block is in sequence s's table
    out2, lse2 = runner.step(q2, kn2, vn2, table2, torch.from_numpy((k2 + 1).astype(np.int32)).cuda())
    torch.cuda.synchronize()
    # oracle: the first 10 sequences' keys 0 .. k2 (key k2 = the new row)
    kt = np.concatenate([np.concatenate([b.k_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s] + k2[s]],
                                         b2.k_tokens[b2.new_token_rows()][s:s + 1]]) for s in range(10)])
    vt = np.concatenate([np.concatenate([b.v_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s] + k2[s]],
                                         b2.v_tokens[b2.new_token_rows()][s:s + 1]]) for s in range(10)])
    cu = np.zeros(11, np.int64)
    cu[1:] = np.cumsum(k2 + 1)
    slots = np.concatenate([b.block_table[s, np.arange(k2[s] + 1) // 16] * 16 + np.arange(k2[s] + 1) % 16
                            for s in range(10)])
    b3 = dataclasses.replace(b2, block_table=b.block_table[:10], num_blocks=b.num_blocks, poison_block=b.poison_block,
                             k_lens=(k2 + 1).astype(np.int32), cu_seqlens_k=cu.astype(np.int32), k_tokens=kt,
                             v_tokens=vt, slots=slots.astype(np.int32))
    ro2, rl2 = oracle_attention(b3)
    go2, gl2 = out2.float().cpu().numpy().astype(np.float64), lse2.cpu().numpy().astype(np.float64)
    eo2, el2 = np.max(np.abs(go2 - ro2)), np.max(np.abs(gl2 - rl2))
    print(f"[runner-{dtype} B=10 -> bucket 16] max|dout|={eo2:.3e} max|dlse|={el2:.3e}", flush=True)
    assert eo2 <= TOL[dtype] and el2 <= TOL[dtype]


# ------------------------------------------------------- graph capture ----
@pytest.mark.parametrize("mode", ["fused_decode", "decode", "prefill"])
def test_graph_replay_matches_eager(mode):
    """The calls captured into a HIP graph: every replay, with eager work and
    synchronisations between replays, gives the eager call's bits."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import to_device, to_device_before_append
    if mode == "prefill":
        b = _mk(981, [40, 17, 64], [40, 30, 100], Hq=8, Hkv=2, D=128, dtype="bf16", causal=True)
    else:
        k = [int(x) for x in np.random.default_rng(982).integers(1, 2000, size=24)]
        b = _mk(982, [1] * len(k), k, Hq=8, Hkv=2, D=64, dtype="bf16", causal=True)
    if mode == "fused_decode":
        db, kn, vn = to_device_before_append(b)
    else:
        db = to_device(b)
    need = kvs.workspace_size(db.q, db.k_cache, db.block_table, num_splits=32)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device="cuda")
    out = torch.empty_like(db.q)
    lse = torch.empty(db.q.shape[0], db.q.shape[1], dtype=torch.float32, device="cuda")

    def call(o, l):
        if mode == "fused_decode":
            kvs.attn_decode_append_paged(db.q, kn, vn, db.k_cache, db.v_cache, db.block_table, db.seqlens_k,
                                         db.scale, out=o, lse=l, num_splits=32, workspace=ws)
        else:
            kvs.attn_varlen_paged(db.q, db.k_cache, db.v_cache, db.block_table, db.cu_seqlens_q, db.seqlens_k,
                                  db.scale, True, out=o, lse=l, num_splits=32, workspace=ws)

    call(out, lse)
    torch.cuda.synchronize()
    _check(b, out, lse)
    ref_o, ref_l = out.clone(), lse.clone()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call(out, lse)
    o2, l2 = torch.empty_like(out), torch.empty_like(lse)
    for _ in range(4):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_o) and torch.equal(lse, ref_l)
        call(o2, l2)                  # eager work between replays
        torch.cuda.synchronize()
        assert torch.equal(o2, ref_o) and torch.equal(l2, ref_l)


# ------------------------------------------------------ one-hot probes ----
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("first", [False, True])
@pytest.mark.parametrize("decode", [False, True])
def test_one_hot_probes_bitwise(dtype, first, decode):
    """Scores scale*alpha*t with a huge slope make P exactly one-hot, so every
    output row must equal one V row bit for bit: the last visible key (causal
    boundary, cached prefix, block table, GQA map) or key 0 (alpha < 0)."""
    from tests.gpu_side import to_device, run_attention
    if decode:
        q_lens, k_lens = [1] * 5, [1, 17, 300, 64, 1999]
    else:
        q_lens, k_lens = [17, 1, 40, 9, 70], [17, 20, 40, 100, 333]
    D = 128 if dtype == "bf16" else 64
    b = _mk(600 + decode * 2 + first, q_lens, k_lens, Hq=8, Hkv=2, D=D, dtype=dtype, causal=True)
    for s in range(b.B):
        k0, k1 = int(b.cu_seqlens_k[s]), int(b.cu_seqlens_k[s + 1])
        t = np.arange(k1 - k0, dtype=np.float32)
        b.k_tokens[k0:k1] = 0.0
        b.k_tokens[k0:k1, :, 0] = (t // 256)[:, None]
        b.k_tokens[k0:k1, :, 1] = (t % 256)[:, None]
    alpha = -2048.0 if first else 2048.0
    b.q[:] = 0.0
    b.q[:, :, 0] = 256 * alpha
    b.q[:, :, 1] = alpha
    db = to_device(b)
    out, _ = run_attention(db)
    got = out.cpu()
    G = b.Hq // b.Hkv
    vt = torch.from_numpy(b.v_tokens).to(got.dtype)
    for s in range(b.B):
        lq, lk = int(b.q_lens[s]), int(b.k_lens[s])
        c = lk - lq
        for i in range(lq):
            j = 0 if first else ((c + i) if lq > 1 else lk - 1)
            r = int(b.cu_seqlens_q[s]) + i
            for h in range(b.Hq):
                assert torch.equal(got[r, h], vt[int(b.cu_seqlens_k[s]) + j, h // G]), (s, i, h)


# --------------------------------------------------- poison invariance ---
def test_poison_never_reaches_output():
    """Unowned blocks, tail rows and unused table entries hold NaN (the table
    entries point at a NaN block); the output has no NaN and matches the oracle."""
    b = _mk(701, [17, 9, 1, 33], [30, 9, 47, 33], Hq=8, Hkv=2, D=64, dtype="bf16", causal=True,
            extra_table_cols=4, name="poison")
    out, lse = _run(b)
    _check(b, out, lse)


# ------------------------------------------------------ named workloads --
@pytest.mark.parametrize("name", ["paged_decode_bf16", "causal_prefill_bf16", "extend_prefill_bf16",
                                  "mixed_prefill_decode_bf16"])
def test_named_workload_all_rows(name):
    """The named workloads at their full sizes, in the launch configuration the
    benchmark times: every output row and lse of every head against the
    oracle (so every (sequence, token tile, head group) item of the persistent
    grid, in its full-size order, is compared)."""
    from workloads import NAMED
    b = NAMED[name]()
    out, lse = _run(b)
    _check(b, out, lse)


def long_prefill_check_rows(T, tile=64, edge=2048):
    """Rows of a T-row prompt compared in full: the first and last row of every
    `tile`-row token tile, and every row of the first and last `edge`."""
    rows = set(range(min(edge, T))) | set(range(max(0, T - edge), T))
    for t0 in range(0, T, tile):
        rows |= {t0, min(T, t0 + tile) - 1}
    return sorted(rows)


def test_long_prefill_tile_rows():
    """The 32768-token prompt: the first and last row of each of its 512
    token tiles (all heads), plus every row of its first and last 2048."""
    from workloads import long_prefill_bf16
    b = long_prefill_bf16()
    out, lse = _run(b)
    rows = long_prefill_check_rows(b.T)
    assert len(rows) == 4992   # 2 x 2048 + 2 rows of each of the 448 tiles in between
    _check(b, out, lse, rows=rows)


# ------------------------------------------------ mixed batches: decode_tail --
MIXED_Q = [40, 17, 64, 1, 1, 1, 1, 1, 1]
MIXED_K = [40, 100, 300, 1, 16, 17, 700, 129, 2000]


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("splits", [0, 7])
@pytest.mark.parametrize("with_lse", [True, False])
def test_decode_tail_matches_oracle(dtype, D, splits, with_lse):
    """A mixed batch whose last 6 sequences are decode rows, run with
    decode_tail = 6 (prefill kernel on the first 3, decode kernel on the
    rest) and with smaller true statements (2, 1): every row matches the
    oracle."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_attention, to_device
    b = _mk(1500 + D + splits, MIXED_Q, MIXED_K, Hq=8, Hkv=2, D=D, dtype=dtype, causal=True,
            name=f"tail-{dtype}-{D}-s{splits}")
    db = to_device(b)
    for tail in (6, 2, 1):
        out, lse = run_attention(db, decode_tail=tail, num_splits=splits, return_lse=with_lse)
        assert kvs.last_dispatch().startswith(f"split (decode_tail {tail})"), kvs.last_dispatch()
        if with_lse:
            _check(b, out, lse)
        else:
            from tests.gpu_side import to_f64
            from tests.oracle_side import oracle_attention
            ro, _ = oracle_attention(b)
            assert lse is None and np.max(np.abs(to_f64(out) - ro)) <= TOL[dtype]


def test_decode_tail_whole_batch_and_window():
    """decode_tail = B on a decode batch (one launch), and the hint with a
    sliding window and with an FP8 cache."""
    import attention_kv_store_amd as kvs
    from tests.gpu_side import run_attention, to_device
    b = _mk(1510, [1] * 5, [1, 17, 200, 64, 33], Hq=8, Hkv=2, D=64, dtype="bf16", causal=True)
    out, lse = run_attention(to_device(b), decode_tail=5)
    assert not kvs.last_dispatch().startswith("split")
    _check(b, out, lse)
    w = _mk(1511, MIXED_Q, MIXED_K, Hq=8, Hkv=2, D=128, dtype="bf16", causal=True, window=33)
    out, lse = run_attention(to_device(w), decode_tail=6, window=33)
    assert kvs.last_dispatch().startswith("split")
    _check(w, out, lse)


def test_decode_tail_mixed_named_workload():
    """The 2 x 256 + 30 x 1 mixed batch with its 30 decode rows declared."""
    from tests.gpu_side import run_attention, to_device
    from workloads import mixed_prefill_decode_bf16
    b = mixed_prefill_decode_bf16()
    out, lse = run_attention(to_device(b), decode_tail=30)
    _check(b, out, lse)


# ------------------------------------------------------------ maximum sizes --
def test_decode_largest_batch():
    """8192 sequences (the decode path's limit), contexts 1..40, checked on
    sampled rows, with automatic and forced splits."""
    from workloads import make_batch
    rng = np.random.default_rng(1600)
    k = rng.integers(1, 41, size=8192)
    b = make_batch(1600, [1] * 8192, list(k), Hq=4, Hkv=2, D=64, dtype="bf16", causal=True, name="decode-8192")
    rows = sorted(set(rng.integers(0, 8192, size=400).tolist()) | {0, 1, 8190, 8191})
    for splits in (0, 3000):
        out, lse = _run(b, num_splits=splits)
        _check(b, out, lse, rows=rows)


@pytest.mark.parametrize("splits", [0, 7, 600])
def test_decode_very_long_contexts(splits):
    """Two decode rows over 262144 and 100001 keys: ranges are capped at 2048
    blocks (the splits are raised to at least 16384 / 2048), and the table
    window path is taken."""
    import attention_kv_store_amd as kvs
    b = _mk(1610, [1, 1], [262144, 100001], Hq=8, Hkv=2, D=64, dtype="bf16", causal=True, name="decode-262144")
    out, lse = _run(b, num_splits=splits)
    assert "table=window" in kvs.last_dispatch() or "table=whole" in kvs.last_dispatch()
    _check(b, out, lse)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("heads", [(16, 1), (32, 1), (32, 2)])
def test_prefill_largest_groups(dtype, heads):
    """Prefill and extend with 16 and 32 query heads per KV head."""
    Hq, Hkv = heads
    b = _mk(1620 + Hq + Hkv, [40, 1, 70], [40, 90, 200], Hq=Hq, Hkv=Hkv, D=128, dtype=dtype, causal=True,
            name=f"prefill-groups-{Hq}/{Hkv}")
    out, lse = _run(b)
    _check(b, out, lse)
