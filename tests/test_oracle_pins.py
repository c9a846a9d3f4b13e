"""Pins of the CPU oracle against facts that do not come from the oracle itself.

Each test names the fact it checks.  The pages print no attention values, so the
pins are closed forms, invariants, a multi-precision brute force written as
plain loops, and CPU torch SDPA in float64.  All run on the host.
"""
from __future__ import annotations

import math

import numpy as np
import pytest

from oracle import attention_oracle, gather_sequence, kv_store_oracle, lse_merge
from tests.oracle_side import gather_loop, oracle_attention, oracle_pool
from workloads import BLOCK_SIZE, make_batch, tiny_varlen_fp32

TOL = 1e-13


def _mk(seed, q_lens, k_lens, Hq=4, Hkv=2, D=8, causal=True, dtype="fp32", **kw):
    return make_batch(seed, q_lens, k_lens, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, causal=causal, **kw)


# ---------------------------------------------------------------- P1 ------
@pytest.mark.parametrize("causal", [True, False])
def test_rows_are_convex_weights(causal):
    """If every V row of a KV head equals one vector v, every output row equals v:
    the softmax weights of each row are non-negative and sum to 1."""
    b = _mk(11, [5, 17, 1], [5, 40, 33], Hq=6, Hkv=3, D=8, causal=causal)
    kc, vc = oracle_pool(b)
    v = np.random.default_rng(0).standard_normal((b.Hkv, b.D))
    vc = np.where(np.isnan(vc), np.nan, 0.0) + v[None, None]
    out, _ = attention_oracle(b.q, kc, vc, b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, causal)
    G = b.Hq // b.Hkv
    for h in range(b.Hq):
        assert np.max(np.abs(out[:, h, :] - v[h // G][None])) <= TOL


# ---------------------------------------------------------------- P2 ------
def test_single_key():
    """One key: the weight is exactly 1, so out = v0 bitwise and lse = scale q.k0."""
    b = _mk(12, [1, 1], [1, 1], Hq=4, Hkv=1, D=16)
    kc, vc = oracle_pool(b)
    out, lse = oracle_attention(b, pool=(kc, vc))
    for s in range(2):
        blk = b.block_table[s, 0]
        k0, v0 = kc[blk, 0, 0], vc[blk, 0, 0]
        for h in range(4):
            assert np.array_equal(out[s, h], v0)
            ref = b.scale * float(np.dot(b.q[s, h].astype(np.float64), k0))
            assert abs(lse[s, h] - ref) <= 1e-15 * max(1.0, abs(ref))


# ---------------------------------------------------------------- P3 ------
@pytest.mark.parametrize("causal", [True, False])
def test_zero_query_is_prefix_mean(causal):
    """Q = 0 makes every visible score 0: out_i is the plain mean of the visible V
    rows (keys 0..c+i when causal, all keys otherwise) and lse_i = ln(#visible)."""
    b = _mk(13, [9, 17, 3], [9, 40, 20], Hq=4, Hkv=2, D=8, causal=causal)
    b.q[:] = 0.0
    out, lse = oracle_attention(b)
    G = b.Hq // b.Hkv
    for s in range(b.B):
        lq, lk = int(b.q_lens[s]), int(b.k_lens[s])
        c = lk - lq
        V = b.v_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]].astype(np.float64)
        csum = np.cumsum(V, axis=0)
        for i in range(lq):
            n = (c + i + 1) if (causal and lq > 1) else lk
            r = int(b.cu_seqlens_q[s]) + i
            for h in range(b.Hq):
                mean = csum[n - 1, h // G] / n
                assert np.max(np.abs(out[r, h] - mean)) <= TOL
                assert abs(lse[r, h] - math.log(n)) <= TOL


# ---------------------------------------------------------------- G1/G2 ----
@pytest.mark.parametrize("causal", [True, False])
@pytest.mark.parametrize("first", [False, True])
def test_one_hot_probe(causal, first):
    """Scores proportional to the key position with a huge slope make the weights
    exactly one-hot: the row returns exactly one V row -- the last visible key
    (c+i when causal, the last key otherwise), or key 0 with the slope negated."""
    b = _mk(14, [17, 1, 33], [17, 20, 50], Hq=4, Hkv=2, D=4, causal=causal)
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
    out, _ = oracle_attention(b)
    G = b.Hq // b.Hkv
    for s in range(b.B):
        lq, lk = int(b.q_lens[s]), int(b.k_lens[s])
        c = lk - lq
        V = b.v_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]].astype(np.float64)
        for i in range(lq):
            j = 0 if first else ((c + i) if (causal and lq > 1) else lk - 1)
            r = int(b.cu_seqlens_q[s]) + i
            for h in range(b.Hq):
                assert np.array_equal(out[r, h], V[j, h // G])


# ---------------------------------------------------------------- P4/P5 ---
def test_paged_equals_contiguous():
    """The same sequences stored contiguously (identity table) and scattered
    through a permuted table give bitwise the same result."""
    b = _mk(15, [17, 9, 30], [40, 9, 47], Hq=4, Hkv=2, D=8)
    out_p, lse_p = oracle_attention(b)
    # contiguous layout: sequence s owns blocks base_s .. base_s + n_s - 1
    nblk = (b.k_lens + 15) // 16
    NB = int(nblk.sum()) + 1
    kc = np.full((NB, 16, b.Hkv, b.D), np.nan)
    vc = np.full_like(kc, np.nan)
    table = np.full_like(b.block_table, NB - 1)
    base = 0
    for s in range(b.B):
        table[s, :nblk[s]] = np.arange(base, base + nblk[s])
        ks = b.k_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
        vs = b.v_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
        for t in range(int(b.k_lens[s])):
            kc[base + t // 16, t % 16] = ks[t]
            vc[base + t // 16, t % 16] = vs[t]
        base += int(nblk[s])
    out_c, lse_c = attention_oracle(b.q, kc, vc, table, b.cu_seqlens_q, b.k_lens, b.scale, True)
    assert np.array_equal(out_p, out_c) and np.array_equal(lse_p, lse_c)


def test_block_table_permutation():
    """Relabelling physical blocks by a permutation (pool and table together)
    changes nothing, bitwise."""
    b = _mk(16, [17, 9], [33, 9], Hq=4, Hkv=2, D=8)
    kc, vc = oracle_pool(b)
    out1, lse1 = oracle_attention(b, pool=(kc, vc))
    pi = np.random.default_rng(1).permutation(b.num_blocks)
    kc2 = np.empty_like(kc)
    vc2 = np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    out2, lse2 = attention_oracle(b.q, kc2, vc2, pi[b.block_table], b.cu_seqlens_q, b.k_lens,
                                  b.scale, True)
    assert np.array_equal(out1, out2) and np.array_equal(lse1, lse2)


# ---------------------------------------------------------------- P6 ------
def _brute(q, k_rows, v_rows, lq, lk, scale, causal, G, dps=50, window=0):
    """mpmath loops: softmax(scale q.k + mask) V for one sequence, all heads.
    ``window`` > 0: the row at position p sees keys max(0, p - window + 1) .. p."""
    import mpmath as mp

    mp.mp.dps = dps
    Hq, D = q.shape[1], q.shape[2]
    c = lk - lq
    out = np.zeros((lq, Hq, D))
    lse = np.zeros((lq, Hq))
    for i in range(lq):
        last = (c + i) if (causal and lq > 1) else (lk - 1)
        first = max(0, c + i - window + 1) if window else 0
        keys = range(first, last + 1)
        for h in range(Hq):
            g = h // G
            sc = {}
            for j in keys:
                acc = mp.mpf(0)
                for d in range(D):
                    acc += mp.mpf(float(q[i, h, d])) * mp.mpf(float(k_rows[j, g, d]))
                sc[j] = mp.mpf(scale) * acc
            z = mp.fsum(mp.exp(sc[j]) for j in keys)
            for d in range(D):
                num = mp.fsum(mp.exp(sc[j]) * mp.mpf(float(v_rows[j, g, d])) for j in keys)
                out[i, h, d] = float(num / z)
            lse[i, h] = float(mp.log(z))
    return out, lse


@pytest.mark.parametrize("case", [
    dict(seed=21, q=[17, 9], k=[17, 9], Hq=4, Hkv=2, D=8, causal=True),
    dict(seed=22, q=[3, 1, 5], k=[20, 33, 5], Hq=3, Hkv=1, D=4, causal=True),
    dict(seed=23, q=[16, 2], k=[31, 2], Hq=2, Hkv=2, D=8, causal=False),
    dict(seed=24, q=[1, 1, 1], k=[1, 16, 17], Hq=4, Hkv=4, D=4, causal=True),
])
def test_bruteforce_mpmath(case):
    """The oracle equals a 50-digit brute force written as plain loops."""
    b = _mk(case["seed"], case["q"], case["k"], Hq=case["Hq"], Hkv=case["Hkv"], D=case["D"],
            causal=case["causal"])
    out, lse = oracle_attention(b)
    G = b.Hq // b.Hkv
    for s in range(b.B):
        r0, r1 = int(b.cu_seqlens_q[s]), int(b.cu_seqlens_q[s + 1])
        ks = b.k_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
        vs = b.v_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
        bo, bl = _brute(b.q[r0:r1], ks, vs, r1 - r0, int(b.k_lens[s]), b.scale, b.causal, G)
        assert np.max(np.abs(out[r0:r1] - bo)) <= TOL
        assert np.max(np.abs(lse[r0:r1] - bl)) <= TOL


def test_bruteforce_hypothesis():
    """Random small shapes (lengths across page edges, cached prefixes, GQA ratios,
    both mask modes) against the brute force."""
    hyp = pytest.importorskip("hypothesis")
    from hypothesis import given, settings, strategies as st

    @settings(max_examples=12, deadline=None, derandomize=True)
    @given(st.integers(1, 3), st.sampled_from([(1, 1), (2, 1), (4, 2), (3, 3)]),
           st.sampled_from([2, 4]), st.booleans(), st.integers(0, 2**31 - 1), st.data())
    def run(B, heads, D, causal, seed, data):
        Hq, Hkv = heads
        q_lens, k_lens = [], []
        for _ in range(B):
            lq = data.draw(st.integers(1, 18))
            lk = lq + data.draw(st.integers(0, 18))
            q_lens.append(lq)
            k_lens.append(lk)
        b = _mk(seed % 100000, q_lens, k_lens, Hq=Hq, Hkv=Hkv, D=D, causal=causal)
        out, lse = oracle_attention(b)
        for s in range(b.B):
            r0, r1 = int(b.cu_seqlens_q[s]), int(b.cu_seqlens_q[s + 1])
            ks = b.k_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
            vs = b.v_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
            bo, bl = _brute(b.q[r0:r1], ks, vs, r1 - r0, int(b.k_lens[s]), b.scale, causal,
                            Hq // Hkv, dps=30)
            assert np.max(np.abs(out[r0:r1] - bo)) <= TOL
            assert np.max(np.abs(lse[r0:r1] - bl)) <= TOL

    run()


# ---------------------------------------------------------------- P7 ------
def test_torch_sdpa_float64():
    """Independent library implementation: CPU torch SDPA in float64 per sequence,
    with an explicit bottom-right boolean mask and enable_gqa."""
    import torch
    import torch.nn.functional as F

    b = _mk(31, [17, 9, 40, 1], [17, 30, 64, 77], Hq=8, Hkv=2, D=16)
    kc, vc = oracle_pool(b)
    out, _ = oracle_attention(b, pool=(kc, vc))
    for s in range(b.B):
        lq, lk = int(b.q_lens[s]), int(b.k_lens[s])
        c = lk - lq
        r0 = int(b.cu_seqlens_q[s])
        K = torch.from_numpy(gather_loop(kc, b.block_table[s], lk)).permute(1, 0, 2)[None]
        V = torch.from_numpy(gather_loop(vc, b.block_table[s], lk)).permute(1, 0, 2)[None]
        Q = torch.from_numpy(b.q[r0:r0 + lq].astype(np.float64)).permute(1, 0, 2)[None]
        i = torch.arange(lq)[:, None]
        j = torch.arange(lk)[None, :]
        mask = j <= (c + i)
        ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=b.scale, enable_gqa=True)
        ref = ref[0].permute(1, 0, 2).numpy()
        assert np.max(np.abs(out[r0:r0 + lq] - ref)) <= 1e-12


# ---------------------------------------------------------------- P8 ------
def test_extend_is_suffix_of_full_prefill():
    """Extending c cached tokens by e new ones gives rows c..c+e-1 of the full causal
    prefill of c+e tokens; a one-row decode gives its last row."""
    L, c = 70, 45
    full = _mk(41, [L], [L], Hq=4, Hkv=2, D=8)
    pool = oracle_pool(full)
    out_f, lse_f = oracle_attention(full, pool=pool)
    for start in (c, L - 1):
        cu = np.array([0, L - start], np.int32)
        out_e, lse_e = attention_oracle(full.q[start:], pool[0], pool[1], full.block_table, cu,
                                        full.k_lens, full.scale, True)
        assert np.max(np.abs(out_e - out_f[start:])) <= TOL
        assert np.max(np.abs(lse_e - lse_f[start:])) <= TOL


# ---------------------------------------------------------------- P9 ------
def test_gqa_equals_repeated_kv():
    """GQA equals multi-head attention with each KV head repeated G times in a row
    (query head h reads KV head h // G)."""
    b = _mk(51, [17, 5], [30, 5], Hq=8, Hkv=2, D=8)
    kc, vc = oracle_pool(b)
    out, lse = oracle_attention(b, pool=(kc, vc))
    G = b.Hq // b.Hkv
    out2, lse2 = attention_oracle(b.q, np.repeat(kc, G, axis=2), np.repeat(vc, G, axis=2),
                                  b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, True)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# ---------------------------------------------------------------- P10 -----
@pytest.mark.parametrize("cuts", [[16], [32, 48], [16, 32, 64, 80]])
def test_split_merge_equals_unsplit(cuts):
    """Decode rows: the results over disjoint key ranges, merged with lse_merge,
    equal the result over all keys."""
    b = _mk(61, [1, 1, 1], [96, 97, 111], Hq=4, Hkv=2, D=8)
    kc, vc = oracle_pool(b)
    full_o, full_l = oracle_attention(b, pool=(kc, vc))
    parts = []
    edges = [0] + cuts + [None]
    for a, z in zip(edges[:-1], edges[1:]):
        lens = (b.k_lens if z is None else np.minimum(b.k_lens, z)) - a
        table = b.block_table[:, a // 16:]
        parts.append(attention_oracle(b.q, kc, vc, table, b.cu_seqlens_q, lens.astype(np.int32),
                                      b.scale, True))
    o, l = lse_merge(parts)
    assert np.max(np.abs(o - full_o)) <= TOL and np.max(np.abs(l - full_l)) <= TOL


def test_merge_skips_empty_parts():
    """A part with lse = -inf (no keys) carries no weight."""
    o = np.random.default_rng(2).standard_normal((3, 4))
    l = np.array([0.5, -1.0, 2.0])
    empty = (np.full((3, 4), np.nan), np.full(3, -np.inf))
    mo, ml = lse_merge([(o, l), empty])
    assert np.array_equal(mo, o) and np.array_equal(ml, l)


# ---------------------------------------------------------------- P11 -----
def test_batch_permutation():
    """Reordering the sequences of a batch reorders the output rows, bitwise."""
    b = _mk(71, [17, 9, 30], [40, 9, 47], Hq=4, Hkv=2, D=8)
    kc, vc = oracle_pool(b)
    out, lse = oracle_attention(b, pool=(kc, vc))
    perm = np.array([2, 0, 1])
    ql = b.q_lens[perm]
    cu = np.concatenate([[0], np.cumsum(ql)]).astype(np.int32)
    qp = np.concatenate([b.q[b.cu_seqlens_q[s]:b.cu_seqlens_q[s + 1]] for s in perm])
    out2, lse2 = attention_oracle(qp, kc, vc, b.block_table[perm], cu, b.k_lens[perm], b.scale, True)
    rows = np.concatenate([np.arange(b.cu_seqlens_q[s], b.cu_seqlens_q[s + 1]) for s in perm])
    assert np.array_equal(out2, out[rows]) and np.array_equal(lse2, lse[rows])


# ---------------------------------------------------------------- P12 -----
def test_poison_is_never_read():
    """NaN in unowned blocks and in tail rows past each sequence's length, and
    table entries past its last block set to ids that do not exist, leave the
    result unchanged and NaN-free (an out-of-range entry would raise if read)."""
    b = _mk(81, [17, 9, 3], [33, 9, 20], Hq=4, Hkv=2, D=8, extra_table_cols=3)
    kc, vc = oracle_pool(b)          # NaN everywhere no token was stored
    assert np.isnan(kc).any()
    out, lse = oracle_attention(b, pool=(kc, vc))
    assert not np.isnan(out).any() and not np.isnan(lse).any()
    table = b.block_table.copy()
    nblk = (b.k_lens + 15) // 16
    for s in range(b.B):
        table[s, nblk[s]:] = 10**9 + s
    out2, lse2 = attention_oracle(b.q, kc, vc, table, b.cu_seqlens_q, b.k_lens, b.scale, True)
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


# ---------------------------------------------------------------- P13 -----
def test_store_matches_loop_scatter():
    """kv_store_oracle equals an element-by-element loop; negative slots are skipped
    and leave the pool untouched."""
    rng = np.random.default_rng(3)
    NB, Hkv, D = 5, 2, 3
    kc0 = rng.standard_normal((NB, 16, Hkv, D))
    vc0 = rng.standard_normal((NB, 16, Hkv, D))
    kn = rng.standard_normal((7, Hkv, D))
    vn = rng.standard_normal((7, Hkv, D))
    slots = np.array([3, -1, 79, 16, 17, -7, 40])
    kc, vc = kv_store_oracle(kn, vn, slots, kc0, vc0)
    ek, ev = kc0.copy(), vc0.copy()
    for t, s in enumerate(slots):
        if s < 0:
            continue
        for h in range(Hkv):
            for d in range(D):
                ek[s // 16, s % 16, h, d] = kn[t, h, d]
                ev[s // 16, s % 16, h, d] = vn[t, h, d]
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)
    with pytest.raises(ValueError):
        kv_store_oracle(kn[:2], vn[:2], np.array([5, 5]), kc0, vc0)
    with pytest.raises(ValueError):
        kv_store_oracle(kn[:1], vn[:1], np.array([NB * 16]), kc0, vc0)


def test_store_then_gather_round_trip():
    """Storing every token at its slot and gathering through the block table gives
    the tokens back in position order."""
    b = tiny_varlen_fp32()
    kc, vc = oracle_pool(b)
    for s in range(b.B):
        ks = b.k_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
        got = gather_sequence(kc, b.block_table[s], int(b.k_lens[s]))
        assert np.array_equal(got, ks)


# ---------------------------------------------------------------- P14 -----
def test_token_table_equals_block_table():
    """A token-granular table (one slot per token) sliced every 16 entries and
    floor-divided by 16 gives the block table; gathering token by token through
    it gives the same rows as gathering through the block table."""
    b = _mk(91, [17, 9, 33], [33, 9, 70], Hq=2, Hkv=1, D=4)
    kc, vc = oracle_pool(b)
    maxk = int(b.k_lens.max())
    for s in range(b.B):
        lk = int(b.k_lens[s])
        tok_table = b.slots[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
        pages = tok_table[:maxk:16] // 16
        assert np.array_equal(pages, b.block_table[s, :len(pages)])
        by_tok = np.stack([kc[tok_table[t] // 16, tok_table[t] % 16] for t in range(lk)])
        assert np.array_equal(by_tok, gather_sequence(kc, b.block_table[s], lk))


# ---------------------------------------------------------------- P15 -----
def test_decode_ignores_causal_flag():
    """One query row per sequence sees every key with or without the causal flag."""
    b = _mk(101, [1, 1, 1], [5, 16, 49], Hq=4, Hkv=2, D=8)
    o1, l1 = oracle_attention(b, causal=True)
    o2, l2 = oracle_attention(b, causal=False)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ---------------------------------------------------------------- rows ----
def test_row_subset_matches_full():
    """Computing a subset of rows gives the same values as the full call."""
    b = _mk(111, [40, 33], [60, 33], Hq=4, Hkv=2, D=8)
    out, lse = oracle_attention(b)
    rows = [0, 5, 39, 40, 72]
    o2, l2 = oracle_attention(b, rows=rows)
    assert np.allclose(o2[rows], out[rows], atol=TOL, rtol=0) and np.allclose(l2[rows], lse[rows], atol=TOL)
    assert np.isnan(o2[1]).all()


def test_validation_errors():
    b = _mk(121, [3, 2], [3, 5], Hq=4, Hkv=2, D=8)
    kc, vc = oracle_pool(b)
    with pytest.raises(ValueError):
        attention_oracle(b.q, kc, vc, b.block_table, b.cu_seqlens_q, np.array([2, 5]), b.scale, True)
    with pytest.raises(ValueError):
        attention_oracle(b.q[:, :3], kc, vc, b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, True)
    with pytest.raises(ValueError):
        attention_oracle(b.q, kc, vc, b.block_table, np.array([0, 3, 4]), b.k_lens, b.scale, True)


# ---------------------------------------------------------------- W1-W6 ----
# Sliding window (reading: with window W the row at position p sees keys
# max(0, p - W + 1) .. p; a one-row decode sits at position Lk - 1).
def _rows_and_positions(b):
    for s in range(b.B):
        lq, lk = int(b.q_lens[s]), int(b.k_lens[s])
        for i in range(lq):
            yield s, int(b.cu_seqlens_q[s]) + i, lk - lq + i


def test_window_one_is_own_row():
    """W = 1: a row sees its own position only, so out = v_p bitwise and
    lse = scale q.k_p -- for prefill rows, extend rows and decode rows alike."""
    b = _mk(51, [17, 1, 5, 1], [17, 33, 40, 1], Hq=4, Hkv=2, D=8, window=1)
    out, lse = oracle_attention(b)
    G = b.Hq // b.Hkv
    for s, r, p in _rows_and_positions(b):
        kt = b.k_tokens[int(b.cu_seqlens_k[s]) + p].astype(np.float64)
        vt = b.v_tokens[int(b.cu_seqlens_k[s]) + p].astype(np.float64)
        for h in range(b.Hq):
            assert np.array_equal(out[r, h], vt[h // G])
            ref = b.scale * float(np.dot(b.q[r, h].astype(np.float64), kt[h // G]))
            assert abs(lse[r, h] - ref) <= 1e-15 * max(1.0, abs(ref))


def test_window_two_closed_form():
    """W = 2: a row at p >= 1 sees keys p - 1 and p.  With s = scale q.k the
    weight of key p is the logistic 1 / (1 + e^(s_{p-1} - s_p)) and
    lse = ln(e^(s_{p-1}) + e^(s_p)); the row at position 0 sees key 0 alone."""
    b = _mk(52, [18, 1, 3], [18, 50, 16], Hq=2, Hkv=1, D=8, window=2)
    out, lse = oracle_attention(b)
    for s, r, p in _rows_and_positions(b):
        base = int(b.cu_seqlens_k[s])
        for h in range(b.Hq):
            qv = b.q[r, h].astype(np.float64)
            sp = b.scale * float(np.dot(qv, b.k_tokens[base + p, 0].astype(np.float64)))
            vp = b.v_tokens[base + p, 0].astype(np.float64)
            if p == 0:
                ref_o, ref_l = vp, sp
            else:
                s1 = b.scale * float(np.dot(qv, b.k_tokens[base + p - 1, 0].astype(np.float64)))
                w = 1.0 / (1.0 + math.exp(s1 - sp))
                ref_o = w * vp + (1.0 - w) * b.v_tokens[base + p - 1, 0].astype(np.float64)
                ref_l = max(s1, sp) + math.log1p(math.exp(-abs(s1 - sp)))
            assert np.max(np.abs(out[r, h] - ref_o)) <= 1e-13
            assert abs(lse[r, h] - ref_l) <= 1e-13


@pytest.mark.parametrize("W", [3, 16, 17])
def test_window_zero_query_is_window_mean(W):
    """Q = 0 makes every visible score 0: out is the plain mean of the V rows of
    positions max(0, p - W + 1) .. p and lse = ln(min(p + 1, W))."""
    b = _mk(53, [9, 40, 1], [9, 60, 35], Hq=4, Hkv=2, D=8, window=W)
    b.q[:] = 0.0
    out, lse = oracle_attention(b)
    G = b.Hq // b.Hkv
    for s, r, p in _rows_and_positions(b):
        V = b.v_tokens[int(b.cu_seqlens_k[s]):int(b.cu_seqlens_k[s + 1])].astype(np.float64)
        lo = max(0, p - W + 1)
        for h in range(b.Hq):
            assert np.max(np.abs(out[r, h] - V[lo:p + 1, h // G].mean(axis=0))) <= TOL
            assert abs(lse[r, h] - math.log(p + 1 - lo)) <= TOL


@pytest.mark.parametrize("W", [1, 5, 16, 17, 33, 1000])
def test_window_torch_sdpa_float64(W):
    """CPU torch SDPA in float64 with an explicit band mask (j <= p and
    j >= p - W + 1) and enable_gqa."""
    import torch
    import torch.nn.functional as F

    b = _mk(54, [17, 9, 40, 1, 1], [17, 30, 64, 77, 5], Hq=8, Hkv=2, D=16, window=W)
    kc, vc = oracle_pool(b)
    out, lse = oracle_attention(b, pool=(kc, vc))
    for s in range(b.B):
        lq, lk = int(b.q_lens[s]), int(b.k_lens[s])
        r0 = int(b.cu_seqlens_q[s])
        K = torch.from_numpy(gather_loop(kc, b.block_table[s], lk)).permute(1, 0, 2)[None]
        V = torch.from_numpy(gather_loop(vc, b.block_table[s], lk)).permute(1, 0, 2)[None]
        Q = torch.from_numpy(b.q[r0:r0 + lq].astype(np.float64)).permute(1, 0, 2)[None]
        pos = (lk - lq + torch.arange(lq))[:, None]
        j = torch.arange(lk)[None, :]
        mask = (j <= pos) & (j >= pos - W + 1)
        ref = F.scaled_dot_product_attention(Q, K, V, attn_mask=mask, scale=b.scale, enable_gqa=True)
        assert np.max(np.abs(out[r0:r0 + lq] - ref[0].permute(1, 0, 2).numpy())) <= 1e-12


@pytest.mark.parametrize("case", [
    dict(seed=55, q=[17, 9], k=[17, 30], W=4),
    dict(seed=56, q=[1, 1, 20], k=[19, 3, 33], W=16),
    dict(seed=57, q=[5, 2], k=[40, 18], W=17),
])
def test_window_bruteforce_mpmath(case):
    """The windowed oracle equals the 50-digit brute force with the same band."""
    b = _mk(case["seed"], case["q"], case["k"], Hq=4, Hkv=2, D=4, window=case["W"])
    out, lse = oracle_attention(b)
    for s in range(b.B):
        r0, r1 = int(b.cu_seqlens_q[s]), int(b.cu_seqlens_q[s + 1])
        ks = b.k_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
        vs = b.v_tokens[b.cu_seqlens_k[s]:b.cu_seqlens_k[s + 1]]
        bo, bl = _brute(b.q[r0:r1], ks, vs, r1 - r0, int(b.k_lens[s]), b.scale, True, 2, window=case["W"])
        assert np.max(np.abs(out[r0:r1] - bo)) <= TOL
        assert np.max(np.abs(lse[r0:r1] - bl)) <= TOL


def test_window_wider_than_every_row_is_causal():
    """A window that covers every row's whole prefix (W >= Lk) changes nothing:
    the band is then the causal mask itself."""
    b = _mk(58, [17, 1, 9], [17, 40, 64], Hq=4, Hkv=2, D=8)
    kc, vc = oracle_pool(b)
    o0, l0 = oracle_attention(b, pool=(kc, vc), window=0)
    o1, l1 = oracle_attention(b, pool=(kc, vc), window=64)
    assert np.array_equal(o0, o1) and np.array_equal(l0, l1)


def test_window_keys_outside_the_band_are_never_read():
    """Poisoning (NaN) the K/V rows below every row's window start leaves the
    result finite and unchanged."""
    W = 8
    b = _mk(59, [5, 1], [40, 37], Hq=2, Hkv=1, D=8, window=W)
    kc, vc = oracle_pool(b)
    out0, lse0 = oracle_attention(b, pool=(kc, vc))
    kc2, vc2 = kc.copy(), vc.copy()
    for s in range(b.B):
        lq, lk = int(b.q_lens[s]), int(b.k_lens[s])
        for t in range(max(0, lk - lq - W + 1)):
            blk = int(b.block_table[s, t // BLOCK_SIZE])
            kc2[blk, t % BLOCK_SIZE] = np.nan
            vc2[blk, t % BLOCK_SIZE] = np.nan
    out1, lse1 = oracle_attention(b, pool=(kc2, vc2))
    assert np.array_equal(out0, out1) and np.array_equal(lse0, lse1)


def test_window_needs_causal():
    b = _mk(60, [3], [3], Hq=2, Hkv=1, D=8, causal=False)
    kc, vc = oracle_pool(b)
    with pytest.raises(ValueError):
        attention_oracle(b.q, kc, vc, b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, False, window=2)
    with pytest.raises(ValueError):
        attention_oracle(b.q, kc, vc, b.block_table, b.cu_seqlens_q, b.k_lens, b.scale, True, window=-1)
